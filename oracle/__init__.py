"""fp64 CPU oracle: test infrastructure only (tests, the smoke check and the
benchmark's CPU-baseline leg).  The product path never imports it."""
from .lmhead_oracle import (OracleResult, TopkResult, bf16_bits_to_f64,
                            oracle_logits, oracle_project_argmax,
                            oracle_project_topk, oracle_scatter_logits,
                            oracle_trim)

__all__ = ["OracleResult", "TopkResult", "bf16_bits_to_f64", "oracle_logits",
           "oracle_project_argmax", "oracle_project_topk",
           "oracle_scatter_logits", "oracle_trim"]
