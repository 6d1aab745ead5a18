"""fp64 CPU oracle: test infrastructure only (tests, the smoke check and the
benchmark's CPU-baseline leg).  The product path never imports it."""
from .fp8_head import (E4M3_MAX, e4m3_decode, e4m3_encode, oracle_dequant_fp8,
                       oracle_logits_fp8, oracle_project_argmax_fp8,
                       oracle_project_topk_fp8, oracle_quantize_fp8)
from .mxfp4_head import (MX_BLOCK, e2m1_decode, e2m1_encode, oracle_dequant_mxfp4,
                         oracle_logits_mxfp4, oracle_project_argmax_mxfp4,
                         oracle_project_topk_mxfp4, oracle_quantize_mxfp4)
from .nvfp4_head import (NV_BLOCK, oracle_dequant_nvfp4, oracle_logits_nvfp4,
                         oracle_project_argmax_nvfp4, oracle_project_topk_nvfp4,
                         oracle_quantize_nvfp4)
from .shortlist import oracle_overwrite_rows, oracle_union
from .lmhead_oracle import (OracleResult, TopkResult, argmax_of_logits, topk_of_logits,
                            bf16_bits_to_f64, oracle_logits,
                            oracle_project_argmax, oracle_project_argmax_indexed,
                            oracle_project_topk,
                            oracle_scatter_logits, oracle_trim)

__all__ = ["OracleResult", "TopkResult", "argmax_of_logits", "bf16_bits_to_f64",
           "oracle_logits", "oracle_project_argmax", "oracle_project_topk",
           "oracle_scatter_logits", "oracle_trim", "E4M3_MAX", "e4m3_decode",
           "e4m3_encode", "oracle_quantize_fp8", "oracle_dequant_fp8",
           "oracle_logits_fp8", "oracle_project_argmax_fp8", "oracle_overwrite_rows",
           "oracle_union", "oracle_project_argmax_indexed", "MX_BLOCK", "e2m1_decode",
           "e2m1_encode", "oracle_quantize_mxfp4", "oracle_dequant_mxfp4", "oracle_logits_mxfp4",
           "oracle_project_argmax_mxfp4", "topk_of_logits", "oracle_project_topk_fp8",
           "oracle_project_topk_mxfp4", "NV_BLOCK", "oracle_quantize_nvfp4", "oracle_dequant_nvfp4",
           "oracle_logits_nvfp4", "oracle_project_argmax_nvfp4", "oracle_project_topk_nvfp4"]
