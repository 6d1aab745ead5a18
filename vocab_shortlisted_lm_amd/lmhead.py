"""ctypes binding of liblmhead.so (include/lmhead.h).

Argument marshalling only: every step of the projection runs in the HIP
kernels of the library.  torch supplies device memory and streams.  The
functions keep the C names; they take torch tensors, pass their device
pointers, and raise LmheadError on a nonzero status.  If the library has
not been built, loading it raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "LmheadError", "lib", "LMH_OK", "LMH_EINVAL", "LMH_ERANGE", "LMH_EWORKSPACE",
    "LMH_EHIP", "LMH_MAX_M", "LMH_MIN_K", "LMH_MAX_K", "LMH_MAX_R", "LMH_NOALLOC_MAX_M", "LMH_PATH_AUTO", "LMH_PATH_VALU",
    "LMH_PATH_MFMA", "lmhead_trim", "draft_project_workspace_bytes", "draft_project_argmax",
    "draft_project_argmax_path", "draft_project_auto_path", "draft_project_auto_path_rows", "lmhead_status_str",
    "lmhead_last_error", "lmhead_bench_sink_words", "lmhead_bench_stream_read",
    "lmhead_bench_copy", "new_workspace", "read_id_list", "LMH_MAX_TOPK",
    "draft_project_topk_workspace_bytes", "draft_project_topk", "draft_project_logits",
    "lmhead_bench_time_argmax", "lmhead_quantize_fp8", "draft_project_argmax_fp8",
    "lmhead_bench_time_argmax_fp8", "lmhead_shortlist_overwrite", "lmhead_shortlist_union",
    "LMH_MAX_OVERWRITE", "LMH_MAX_UNION_VOCAB", "draft_project_argmax_indexed",
    "lmhead_bench_time_argmax_indexed", "lmhead_quantize_mxfp4", "draft_project_argmax_mxfp4",
    "lmhead_bench_time_argmax_mxfp4", "lmhead_mxfp4_scale_bytes", "lmhead_mxfp4_tile_scales",
    "mxfp4_scale_shape", "draft_project_topk_fp8", "draft_project_topk_mxfp4", "PreparedArgmax",
    "PreparedArgmaxFp8", "PreparedArgmaxMxfp4", "PreparedArgmaxNvfp4",
    "lmhead_quantize_nvfp4", "lmhead_nvfp4_scale_bytes", "lmhead_nvfp4_tile_scales", "nvfp4_scale_shape",
    "draft_project_argmax_nvfp4", "draft_project_topk_nvfp4", "lmhead_bench_time_argmax_nvfp4",
    "LMH_STATE_BYTES", "new_state", "draft_project_argmax_fused", "draft_project_argmax_fused_path",
    "draft_project_argmax_keys",
    "draft_project_argmax_noalloc",
]

# The in-tree build; LMHEAD_LIB names another build of the same source to load
# instead (the host-sanitizer build the CPU tests run under).
LIB_PATH = os.environ.get("LMHEAD_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblmhead.so")

LMH_OK, LMH_EINVAL, LMH_ERANGE, LMH_EWORKSPACE, LMH_EHIP = 0, 1, 2, 3, 4
LMH_MAX_M, LMH_MIN_K, LMH_MAX_K, LMH_MAX_TOPK = 32, 8, 8192, 16
LMH_MAX_R = (1 << 30) - 1
LMH_NOALLOC_MAX_M = LMH_MAX_M
LMH_STATE_BYTES = 8192
LMH_PATH_AUTO, LMH_PATH_VALU, LMH_PATH_MFMA = 0, 1, 2
LMH_MAX_OVERWRITE, LMH_MAX_UNION_VOCAB = 65536, 524288

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_INT = ctypes.c_int

# name -> (restype, argtypes); mirrors include/lmhead.h and include/lmhead_bench.h
SIGNATURES = {
    "lmhead_trim": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P]),
    "draft_project_workspace_bytes": (_SZ, [_I64]),
    "draft_project_argmax": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _SZ, _P]),
    "draft_project_argmax_path": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _SZ, _INT, _P]),
    "draft_project_auto_path": (_INT, [_I64, _I64]),
    "draft_project_auto_path_rows": (_INT, [_I64, _I64, _I64]),
    "draft_project_topk_workspace_bytes": (_SZ, [_I64, _I64]),
    "draft_project_topk": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _P, _SZ, _INT, _P]),
    "draft_project_logits": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _INT, _P]),
    "lmhead_status_str": (ctypes.c_char_p, [_INT]),
    "lmhead_last_error": (ctypes.c_char_p, []),
    "lmhead_bench_sink_words": (_INT, []),
    "lmhead_bench_stream_read": (_INT, [_P, _SZ, _P, _INT, _P]),
    "lmhead_bench_copy": (_INT, [_P, _P, _SZ, _INT, _P]),
    "lmhead_bench_time_argmax": (_INT, [_P, _I64, _I64, _P, _INT, _I64, _P, _P, _P, _P, _SZ, _INT, _INT,
                                        ctypes.POINTER(ctypes.c_double), _P]),
    "lmhead_quantize_fp8": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "lmhead_shortlist_overwrite": (_INT, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _P]),
    "lmhead_shortlist_union": (_INT, [_P, _I64, _P, _I64, _I64, _P, _I64, _P, _P]),
    "draft_project_argmax_fp8": (_INT, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P, _SZ, _INT, _P]),
    "lmhead_bench_time_argmax_fp8": (_INT, [_P, _I64, _I64, _P, _P, _INT, _I64, _P, _P, _P, _P, _SZ, _INT, _INT,
                                            ctypes.POINTER(ctypes.c_double), _P]),
    "draft_project_argmax_indexed": (_INT, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _P, _SZ, _INT, _P]),
    "lmhead_bench_time_argmax_indexed": (_INT, [_P, _I64, _I64, _P, _INT, _I64, _P, _I64, _P, _P, _P, _SZ, _INT,
                                                _INT, ctypes.POINTER(ctypes.c_double), _P]),
    "lmhead_quantize_mxfp4": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "lmhead_mxfp4_scale_bytes": (_I64, [_I64, _I64]),
    "lmhead_mxfp4_tile_scales": (_INT, [_P, _I64, _I64, _P, _P]),
    "draft_project_argmax_mxfp4": (_INT, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P, _SZ, _INT, _P]),
    "lmhead_bench_time_argmax_mxfp4": (_INT, [_P, _I64, _I64, _P, _P, _INT, _I64, _P, _P, _P, _P, _SZ, _INT, _INT,
                                              ctypes.POINTER(ctypes.c_double), _P]),
    "draft_project_topk_fp8": (_INT, [_P, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _P, _P, _SZ, _INT, _P]),
    "draft_project_topk_mxfp4": (_INT, [_P, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _P, _P, _SZ, _INT, _P]),
    "lmhead_quantize_nvfp4": (_INT, [_P, _I64, _I64, _P, _P, _P, _P]),
    "lmhead_nvfp4_scale_bytes": (_I64, [_I64, _I64]),
    "lmhead_nvfp4_tile_scales": (_INT, [_P, _I64, _I64, _P, _P]),
    "draft_project_argmax_nvfp4": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _P, _SZ, _INT, _P]),
    "draft_project_topk_nvfp4": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _I64, _P, _P, _P, _SZ, _INT, _P]),
    "lmhead_bench_time_argmax_nvfp4": (_INT, [_P, _I64, _I64, _P, _P, _P, _INT, _I64, _P, _P, _P, _P, _SZ, _INT,
                                              _INT, ctypes.POINTER(ctypes.c_double), _P]),
    "draft_project_argmax_keys": (_INT, [_P, _I64, _I64, _P, _I64, _I64, _P, _P, _SZ, _INT, _P]),
    "draft_project_argmax_noalloc": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P, _P, _P]),
    "draft_project_argmax_fused": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _SZ, _P]),
    "draft_project_argmax_fused_path": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _SZ, _INT, _P]),
}

_lib = None
_lock = threading.Lock()


class LmheadError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        text = lib().lmhead_status_str(code).decode()
        if code == LMH_EHIP:
            text += ": " + lib().lmhead_last_error().decode()
        super().__init__(f"{where}: status {code} ({text})")


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it was not built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m vocab_shortlisted_lm_amd.build` (hipcc, gfx950)")
                dll = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(dll, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = dll
    return _lib


def _check(code: int, where: str) -> None:
    if code != LMH_OK:
        raise LmheadError(code, where)


_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _index(device) -> int:
    """Ordinal of a GPU given as a torch.device, an int or a string."""
    if isinstance(device, int):
        return device
    if not isinstance(device, torch.device):
        device = torch.device(device)
    return device.index if device.index is not None else torch.cuda.current_device()


def _dev_tensor(t: torch.Tensor, name: str, dtypes, ndim: int, device=None) -> None:
    """A contiguous device tensor of one of `dtypes` with `ndim` dimensions
    (any dtype / rank if None), on `device` when given.  Every pointer the
    library receives goes through here: a host tensor's address in a
    kernel would fault the GPU."""
    # is_cuda and get_device() are the cheap forms of these checks (a
    # device object's type string costs more than the rest together); the
    # binding runs them on every tensor of every call
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.get_device() != _index(device):
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if (ndim is not None and t.dim() != ndim) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor" if ndim is not None
                         else f"{name} must be contiguous")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _outputs(m: int, out_id, out_logit, device):
    """(out_id int32, out_logit float32) of at least m entries on `device`,
    allocated when not given."""
    if out_id is None:
        out_id = torch.empty(m, dtype=torch.int32, device=device)
    if out_logit is None:
        out_logit = torch.empty(m, dtype=torch.float32, device=device)
    _dev_tensor(out_id, "out_id", (torch.int32,), 1, device)
    _dev_tensor(out_logit, "out_logit", (torch.float32,), 1, device)
    if out_id.shape[0] < m or out_logit.shape[0] < m:
        raise ValueError("outputs must hold M entries")
    return out_id, out_logit


def _workspace(workspace, device, stream_handle: int) -> torch.Tensor:
    """The caller's workspace (checked), or a cached one per device and stream."""
    if workspace is None:
        return _default_workspace(device, stream_handle)
    _dev_tensor(workspace, "workspace", None, None, device)
    return workspace


def _d2t(d2t, r: int, device, rows_of: str = "W"):
    if d2t is not None:
        _dev_tensor(d2t, "d2t", (torch.int32,), 1, device)
        if d2t.shape[0] != r:
            raise ValueError(f"d2t must have one entry per row of {rows_of}")


# The current stream's raw handle without building a torch Stream object
# (1.8 us per call through torch.cuda.current_stream, 0.07 us this way).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device) -> int:
    if stream is None:
        if _raw_stream is not None:
            return int(_raw_stream(_index(device)))
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def lmhead_trim(W: torch.Tensor, ids: torch.Tensor, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """W_trim[i] = W[ids[i]] (bf16 [S, K]).  Synchronizes `stream` once."""
    _dev_tensor(W, "W", _BF16_LIKE, 2)
    _dev_tensor(ids, "ids", (torch.int32,), 1, W.device)
    n, k = W.shape
    s = ids.shape[0]
    if out is None:
        out = torch.empty((s, k), dtype=W.dtype, device=W.device)
    _dev_tensor(out, "out", _BF16_LIKE, 2, W.device)
    if tuple(out.shape) != (s, k):
        raise ValueError("out must be [S, K]")
    _check(lib().lmhead_trim(W.data_ptr(), n, k, ids.data_ptr(), s, out.data_ptr(),
                             _stream(stream, W.device)), "lmhead_trim")
    return out


def draft_project_workspace_bytes(M: int) -> int:
    return int(lib().draft_project_workspace_bytes(M))


def draft_project_auto_path(M: int, K: int) -> int:
    return int(lib().draft_project_auto_path(M, K))


def draft_project_auto_path_rows(M: int, K: int, R: int) -> int:
    return int(lib().draft_project_auto_path_rows(M, K, R))


def new_workspace(device=None, M: int = LMH_MAX_M) -> torch.Tensor:
    """A workspace for calls with up to M hidden rows (contents irrelevant)."""
    nbytes = draft_project_workspace_bytes(M)
    return torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")


_ws_cache: dict = {}


def _default_workspace(device, stream_handle: int) -> torch.Tensor:
    key = (torch.device(device).index, stream_handle)
    ws = _ws_cache.get(key)
    if ws is None:
        ws = new_workspace(device)
        _ws_cache[key] = ws
    return ws


def draft_project_argmax_path(h: torch.Tensor, W: torch.Tensor, d2t: torch.Tensor | None,
                              path: int, out_id: torch.Tensor | None = None,
                              out_logit: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None, stream=None):
    """(out_id int32 [M], out_logit float32 [M]) for the best row of W per
    hidden row, mapped through d2t.  Queues one call; never synchronizes."""
    m, k, r = _check_hw(h, W, d2t)
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    code = lib().draft_project_argmax_path(
        h.data_ptr(), m, k, W.data_ptr(), r, d2t.data_ptr() if d2t is not None else None,
        out_id.data_ptr(), out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path, st)
    _check(code, "draft_project_argmax")
    return out_id, out_logit


class PreparedArgmax:
    """draft_project_argmax_path with its tensors checked once.

    A decode loop calls the draft head with the same buffers every step:
    the hidden rows are rewritten in place, the outputs and the workspace
    stay.  This object runs the binding's checks at construction and then
    makes one C call per step; the tensors must keep their storage
    (no resize or reallocation) while it is used, and it holds references so
    they stay alive.  Calling it queues the step on the stream given here
    and returns (out_id, out_logit).  Given a `state` (new_state), each step
    is the single-launch draft_project_argmax_fused_path instead, and no
    workspace is used."""

    def __init__(self, h: torch.Tensor, W: torch.Tensor, d2t: torch.Tensor | None = None,
                 path: int = LMH_PATH_AUTO, out_id: torch.Tensor | None = None,
                 out_logit: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
                 state: torch.Tensor | None = None):
        m, k, r = _check_hw(h, W, d2t)
        self.out_id, self.out_logit = _outputs(m, out_id, out_logit, h.device)
        st = _stream(stream, h.device)
        if state is not None:
            _check_state(state, h.device)
            self.workspace = state
            self._fn = lib().draft_project_argmax_fused_path
        else:
            self.workspace = _workspace(workspace, h.device, st)
            self._fn = lib().draft_project_argmax_path
        self._keep = (h, W, d2t)
        self._args = (h.data_ptr(), m, k, W.data_ptr(), r, d2t.data_ptr() if d2t is not None else None,
                      self.out_id.data_ptr(), self.out_logit.data_ptr(), self.workspace.data_ptr(),
                      _nbytes(self.workspace), path, st)

    def __call__(self):
        code = self._fn(*self._args)
        if code != LMH_OK:
            raise LmheadError(code, "draft_project_argmax")
        return self.out_id, self.out_logit


class _PreparedQuant:
    """One argmax C call over a quantized head, its arguments checked and
    fixed at construction (the contract of PreparedArgmax: the tensors keep
    their storage while it is used; calling it queues the step and returns
    (out_id, out_logit))."""

    def __init__(self, fn, name, args, keep, out_id, out_logit):
        self._fn, self._name, self._args, self._keep = fn, name, args, keep
        self.out_id, self.out_logit = out_id, out_logit

    def __call__(self):
        code = self._fn(*self._args)
        if code != LMH_OK:
            raise LmheadError(code, self._name)
        return self.out_id, self.out_logit


class PreparedArgmaxFp8(_PreparedQuant):
    """draft_project_argmax_fp8 with its tensors checked once."""

    def __init__(self, h: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor, d2t: torch.Tensor | None = None,
                 path: int = LMH_PATH_AUTO, out_id: torch.Tensor | None = None,
                 out_logit: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
        m, k, r = _check_fp8_head(h, Wq, scale, d2t)
        out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
        st = _stream(stream, h.device)
        ws = _workspace(workspace, h.device, st)
        super().__init__(lib().draft_project_argmax_fp8, "draft_project_argmax_fp8",
                         (h.data_ptr(), m, k, Wq.data_ptr(), scale.data_ptr(), r,
                          d2t.data_ptr() if d2t is not None else None, out_id.data_ptr(), out_logit.data_ptr(),
                          ws.data_ptr(), _nbytes(ws), path, st), (h, Wq, scale, d2t, ws), out_id, out_logit)


class PreparedArgmaxMxfp4(_PreparedQuant):
    """draft_project_argmax_mxfp4 with its tensors checked once."""

    def __init__(self, h: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, d2t: torch.Tensor | None = None,
                 path: int = LMH_PATH_AUTO, out_id: torch.Tensor | None = None,
                 out_logit: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
        m, k, r = _check_mx4_head(h, Wq, scales, d2t)
        out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
        st = _stream(stream, h.device)
        ws = _workspace(workspace, h.device, st)
        super().__init__(lib().draft_project_argmax_mxfp4, "draft_project_argmax_mxfp4",
                         (h.data_ptr(), m, k, Wq.data_ptr(), scales.data_ptr(), r,
                          d2t.data_ptr() if d2t is not None else None, out_id.data_ptr(), out_logit.data_ptr(),
                          ws.data_ptr(), _nbytes(ws), path, st), (h, Wq, scales, d2t, ws), out_id, out_logit)


class PreparedArgmaxNvfp4(_PreparedQuant):
    """draft_project_argmax_nvfp4 with its tensors checked once."""

    def __init__(self, h: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, gscale: torch.Tensor,
                 d2t: torch.Tensor | None = None, path: int = LMH_PATH_AUTO, out_id: torch.Tensor | None = None,
                 out_logit: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
        m, k, r = _check_nv4_head(h, Wq, scales, gscale, d2t)
        out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
        st = _stream(stream, h.device)
        ws = _workspace(workspace, h.device, st)
        super().__init__(lib().draft_project_argmax_nvfp4, "draft_project_argmax_nvfp4",
                         (h.data_ptr(), m, k, Wq.data_ptr(), scales.data_ptr(), gscale.data_ptr(), r,
                          d2t.data_ptr() if d2t is not None else None, out_id.data_ptr(), out_logit.data_ptr(),
                          ws.data_ptr(), _nbytes(ws), path, st), (h, Wq, scales, gscale, d2t, ws),
                         out_id, out_logit)


def draft_project_argmax(h, W, d2t=None, out_id=None, out_logit=None, workspace=None,
                         stream=None):
    """draft_project_argmax_path with the library's own kernel choice."""
    return draft_project_argmax_path(h, W, d2t, LMH_PATH_AUTO, out_id, out_logit, workspace,
                                     stream)


def draft_project_topk_workspace_bytes(M: int, topk: int) -> int:
    return int(lib().draft_project_topk_workspace_bytes(M, topk))


def _check_hw(h, W, d2t):
    _dev_tensor(h, "h", _BF16_LIKE, 2)
    _dev_tensor(W, "W", _BF16_LIKE, 2, h.device)
    m, k = h.shape
    r, k2 = W.shape
    if k != k2:
        raise ValueError("h and W must have the same K")
    _d2t(d2t, r, h.device)
    return m, k, r


def draft_project_topk(h: torch.Tensor, W: torch.Tensor, d2t: torch.Tensor | None, topk: int,
                       out_id: torch.Tensor | None = None, out_logit: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, path: int = LMH_PATH_AUTO,
                       stream=None):
    """(ids int32 [M, topk], logits float32 [M, topk]): the topk best rows of
    W per hidden row, best first, mapped through d2t.  Never synchronizes."""
    m, k, r = _check_hw(h, W, d2t)
    if out_id is None:
        out_id = torch.empty((m, topk), dtype=torch.int32, device=h.device)
    if out_logit is None:
        out_logit = torch.empty((m, topk), dtype=torch.float32, device=h.device)
    _dev_tensor(out_id, "out_id", (torch.int32,), 2, h.device)
    _dev_tensor(out_logit, "out_logit", (torch.float32,), 2, h.device)
    if tuple(out_id.shape) != (m, topk) or tuple(out_logit.shape) != (m, topk):
        raise ValueError("outputs must be [M, topk]")
    st = _stream(stream, h.device)
    if workspace is None:
        nbytes = draft_project_topk_workspace_bytes(m, topk)
        if nbytes == 0:
            raise LmheadError(LMH_EINVAL, "draft_project_topk")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=h.device)
    _dev_tensor(workspace, "workspace", None, None, h.device)
    code = lib().draft_project_topk(
        h.data_ptr(), m, k, W.data_ptr(), r, d2t.data_ptr() if d2t is not None else None, topk,
        out_id.data_ptr(), out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path, st)
    _check(code, "draft_project_topk")
    return out_id, out_logit


def draft_project_logits(h: torch.Tensor, W: torch.Tensor, d2t: torch.Tensor | None = None,
                         n: int | None = None, out: torch.Tensor | None = None,
                         path: int = LMH_PATH_AUTO, stream=None) -> torch.Tensor:
    """float32 logits: [M, R] without d2t; with d2t, [M, n] with the list's
    logits at their vocabulary ids and -inf elsewhere.  Never synchronizes."""
    m, k, r = _check_hw(h, W, d2t)
    cols = r if d2t is None else n
    if cols is None:
        raise ValueError("n (vocabulary size) is required with d2t")
    if out is None:
        out = torch.empty((m, cols), dtype=torch.float32, device=h.device)
    _dev_tensor(out, "out", (torch.float32,), 2, h.device)
    if tuple(out.shape) != (m, cols):
        raise ValueError(f"out must be [{m}, {cols}]")
    code = lib().draft_project_logits(
        h.data_ptr(), m, k, W.data_ptr(), r, d2t.data_ptr() if d2t is not None else None,
        cols if d2t is not None else 0, out.data_ptr(), path, _stream(stream, h.device))
    _check(code, "draft_project_logits")
    return out


def read_id_list(path: str):
    """Token ids of a shortlist file: one integer id per line (blank lines
    ignored), in file order -- the ranks / draft-vocabulary list format the
    head is trimmed from at load.  Returns an int32 numpy array."""
    import numpy as np
    with open(path) as f:
        vals = [int(tok) for tok in (line.strip() for line in f) if tok]
    return np.asarray(vals, dtype=np.int32)


def lmhead_status_str(code: int) -> str:
    return lib().lmhead_status_str(code).decode()


def lmhead_last_error() -> str:
    return lib().lmhead_last_error().decode()


def lmhead_bench_sink_words() -> int:
    return int(lib().lmhead_bench_sink_words())


def lmhead_bench_stream_read(buf: torch.Tensor, sink: torch.Tensor, grid: int = 0,
                             stream=None) -> None:
    _dev_tensor(buf, "buf", None, None)
    _dev_tensor(sink, "sink", (torch.int32,), 1, buf.device)
    if sink.numel() < lmhead_bench_sink_words():
        raise ValueError("sink must hold lmhead_bench_sink_words() int32 words")
    nbytes = _nbytes(buf)
    _check(lib().lmhead_bench_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid,
                                          _stream(stream, buf.device)),
           "lmhead_bench_stream_read")


def lmhead_bench_copy(src: torch.Tensor, dst: torch.Tensor, grid: int = 0, stream=None) -> None:
    _dev_tensor(src, "src", None, None)
    _dev_tensor(dst, "dst", None, None, src.device)
    nbytes = _nbytes(src)
    if _nbytes(dst) < nbytes:
        raise ValueError("dst too small")
    _check(lib().lmhead_bench_copy(src.data_ptr(), dst.data_ptr(), nbytes, grid,
                                   _stream(stream, src.device)), "lmhead_bench_copy")


def lmhead_bench_time_argmax(h: torch.Tensor, heads: list, d2t: torch.Tensor | None, path: int,
                             calls: int, out_id: torch.Tensor, out_logit: torch.Tensor,
                             workspace: torch.Tensor, stream=None) -> float:
    """Mean duration (ms) of the projection kernel over `calls` back-to-back
    argmax calls rotating through `heads`, from HIP events the library
    records around each projection launch.  Synchronizes."""
    _dev_tensor(h, "h", _BF16_LIKE, 2)
    m, k = h.shape
    if not heads:
        raise ValueError("at least one head")
    for w in heads:
        _dev_tensor(w, "W", _BF16_LIKE, 2, h.device)
        if w.shape != heads[0].shape or w.shape[1] != k:
            raise ValueError("every head must be [R, K] with the same R and K")
    r = heads[0].shape[0]
    _d2t(d2t, r, h.device)
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    ptrs = (ctypes.c_void_p * len(heads))(*[w.data_ptr() for w in heads])
    out = ctypes.c_double(0.0)
    _check(lib().lmhead_bench_time_argmax(
        h.data_ptr(), m, k, ptrs, len(heads), r, d2t.data_ptr() if d2t is not None else None,
        out_id.data_ptr(), out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path, calls,
        ctypes.byref(out), st), "lmhead_bench_time_argmax")
    return out.value


def lmhead_quantize_fp8(W: torch.Tensor, out: torch.Tensor | None = None,
                        scale: torch.Tensor | None = None, stream=None):
    """(Wq uint8 [R, K] E4M3 codes, scale float32 [R]) of a bf16 head, one
    scale per row.  Queues one kernel; never synchronizes."""
    _dev_tensor(W, "W", _BF16_LIKE, 2)
    r, k = W.shape
    if out is None:
        out = torch.empty((r, k), dtype=torch.uint8, device=W.device)
    if scale is None:
        scale = torch.empty(r, dtype=torch.float32, device=W.device)
    _dev_tensor(out, "Wq", (torch.uint8,), 2, W.device)
    _dev_tensor(scale, "scale", (torch.float32,), 1, W.device)
    if tuple(out.shape) != (r, k) or scale.shape[0] < r:
        raise ValueError("Wq must be [R, K] and scale hold R entries")
    _check(lib().lmhead_quantize_fp8(W.data_ptr(), r, k, out.data_ptr(), scale.data_ptr(),
                                     _stream(stream, W.device)), "lmhead_quantize_fp8")
    return out, scale


def _check_fp8_head(h, Wq, scale, d2t):
    _dev_tensor(h, "h", _BF16_LIKE, 2)
    _dev_tensor(Wq, "Wq", (torch.uint8,), 2, h.device)
    _dev_tensor(scale, "scale", (torch.float32,), 1, h.device)
    m, k = h.shape
    r, k2 = Wq.shape
    if k != k2:
        raise ValueError("h and Wq must have the same K")
    if scale.shape[0] != r:
        raise ValueError("scale must have one entry per row of Wq")
    _d2t(d2t, r, h.device, "Wq")
    return m, k, r


def draft_project_argmax_fp8(h: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor,
                             d2t: torch.Tensor | None = None, path: int = LMH_PATH_AUTO,
                             out_id: torch.Tensor | None = None, out_logit: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None, stream=None):
    """(out_id int32 [M], out_logit float32 [M]) for the best row of the
    dequantized FP8 head per hidden row, mapped through d2t.  Never
    synchronizes."""
    m, k, r = _check_fp8_head(h, Wq, scale, d2t)
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    _check(lib().draft_project_argmax_fp8(
        h.data_ptr(), m, k, Wq.data_ptr(), scale.data_ptr(), r,
        d2t.data_ptr() if d2t is not None else None, out_id.data_ptr(), out_logit.data_ptr(),
        workspace.data_ptr(), _nbytes(workspace), path, st),
        "draft_project_argmax_fp8")
    return out_id, out_logit


def lmhead_bench_time_argmax_fp8(h: torch.Tensor, heads: list, d2t: torch.Tensor | None, path: int,
                                 calls: int, out_id: torch.Tensor, out_logit: torch.Tensor,
                                 workspace: torch.Tensor, stream=None) -> float:
    """lmhead_bench_time_argmax over FP8 heads: `heads` is a list of
    (Wq, scale) pairs.  Synchronizes."""
    if not heads:
        raise ValueError("at least one head")
    m, k, r = _check_fp8_head(h, heads[0][0], heads[0][1], d2t)
    for wq, sc in heads:
        _check_fp8_head(h, wq, sc, None)
        if tuple(wq.shape) != (r, k):
            raise ValueError("every head must have the same shape")
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    qp = (ctypes.c_void_p * len(heads))(*[wq.data_ptr() for wq, _ in heads])
    sp = (ctypes.c_void_p * len(heads))(*[sc.data_ptr() for _, sc in heads])
    out = ctypes.c_double(0.0)
    _check(lib().lmhead_bench_time_argmax_fp8(
        h.data_ptr(), m, k, qp, sp, len(heads), r, d2t.data_ptr() if d2t is not None else None,
        out_id.data_ptr(), out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path, calls,
        ctypes.byref(out), st), "lmhead_bench_time_argmax_fp8")
    return out.value


def lmhead_shortlist_overwrite(W: torch.Tensor, W_trim: torch.Tensor, d2t: torch.Tensor,
                               rows: torch.Tensor, ids: torch.Tensor, stream=None) -> None:
    """W_trim[rows[i]] = W[ids[i]], d2t[rows[i]] = ids[i] in place (invalid
    entries skipped, the last entry for a row wins).  Never synchronizes."""
    _dev_tensor(W, "W", _BF16_LIKE, 2)
    _dev_tensor(W_trim, "W_trim", _BF16_LIKE, 2, W.device)
    _dev_tensor(d2t, "d2t", (torch.int32,), 1, W.device)
    _dev_tensor(rows, "rows", (torch.int32,), 1, W.device)
    _dev_tensor(ids, "ids", (torch.int32,), 1, W.device)
    n, k = W.shape
    cap, k2 = W_trim.shape
    if k != k2 or d2t.shape[0] != cap or rows.shape[0] != ids.shape[0]:
        raise ValueError("W [N, K], W_trim [cap, K], d2t [cap], rows and ids of one length")
    _check(lib().lmhead_shortlist_overwrite(W.data_ptr(), n, k, W_trim.data_ptr(), d2t.data_ptr(), cap,
                                            rows.data_ptr(), ids.data_ptr(), rows.shape[0],
                                            _stream(stream, W.device)), "lmhead_shortlist_overwrite")


def lmhead_shortlist_union(a: torch.Tensor, b: torch.Tensor, n_vocab: int, out: torch.Tensor | None = None,
                           counts: torch.Tensor | None = None, stream=None):
    """(out int32 [na + nb], counts int32 [4]): out[:counts[3]] is the
    ascending union of a and b; counts = (|set a|, |set b|, |b - a|, |a u b|).
    Never synchronizes."""
    _dev_tensor(a, "a", (torch.int32,), 1)
    _dev_tensor(b, "b", (torch.int32,), 1, a.device)
    na, nb = a.shape[0], b.shape[0]
    if out is None:
        out = torch.empty(max(1, na + nb), dtype=torch.int32, device=a.device)
    if counts is None:
        counts = torch.empty(4, dtype=torch.int32, device=a.device)
    _dev_tensor(out, "out", (torch.int32,), 1, a.device)
    _dev_tensor(counts, "counts", (torch.int32,), 1, a.device)
    if counts.shape[0] < 4:
        raise ValueError("counts must hold 4 entries")
    _check(lib().lmhead_shortlist_union(a.data_ptr(), na, b.data_ptr(), nb, n_vocab, out.data_ptr(),
                                        out.shape[0], counts.data_ptr(), _stream(stream, a.device)),
           "lmhead_shortlist_union")
    return out, counts


def draft_project_argmax_indexed(h: torch.Tensor, W: torch.Tensor, ids: torch.Tensor,
                                 path: int = LMH_PATH_AUTO, out_id: torch.Tensor | None = None,
                                 out_logit: torch.Tensor | None = None,
                                 workspace: torch.Tensor | None = None, stream=None):
    """(out_id int32 [M], out_logit float32 [M]): the best listed row per
    hidden row, reading rows W[ids[i]] of the full head in place (no trimmed
    copy); out_id is the winning entry's id.  Entries outside [0, N) are
    skipped.  Never synchronizes."""
    _dev_tensor(h, "h", _BF16_LIKE, 2)
    _dev_tensor(W, "W", _BF16_LIKE, 2, h.device)
    _dev_tensor(ids, "ids", (torch.int32,), 1, h.device)
    m, k = h.shape
    n, k2 = W.shape
    if k != k2:
        raise ValueError("h and W must have the same K")
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    _check(lib().draft_project_argmax_indexed(
        h.data_ptr(), m, k, W.data_ptr(), n, ids.data_ptr(), ids.shape[0], out_id.data_ptr(),
        out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path, st),
        "draft_project_argmax_indexed")
    return out_id, out_logit


def lmhead_bench_time_argmax_indexed(h: torch.Tensor, heads: list, ids: torch.Tensor, path: int,
                                     calls: int, out_id: torch.Tensor, out_logit: torch.Tensor,
                                     workspace: torch.Tensor, stream=None) -> float:
    """lmhead_bench_time_argmax for draft_project_argmax_indexed: `heads`
    are full heads [N, K] read through the same id list.  Synchronizes."""
    _dev_tensor(h, "h", _BF16_LIKE, 2)
    _dev_tensor(ids, "ids", (torch.int32,), 1, h.device)
    m, k = h.shape
    if not heads:
        raise ValueError("at least one head")
    for w in heads:
        _dev_tensor(w, "W", _BF16_LIKE, 2, h.device)
        if w.shape != heads[0].shape or w.shape[1] != k:
            raise ValueError("every head must be [N, K] with the same N and K")
    n = heads[0].shape[0]
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    ptrs = (ctypes.c_void_p * len(heads))(*[w.data_ptr() for w in heads])
    out = ctypes.c_double(0.0)
    _check(lib().lmhead_bench_time_argmax_indexed(
        h.data_ptr(), m, k, ptrs, len(heads), n, ids.data_ptr(), ids.shape[0], out_id.data_ptr(),
        out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path, calls,
        ctypes.byref(out), st), "lmhead_bench_time_argmax_indexed")
    return out.value


def lmhead_mxfp4_scale_bytes(R: int, K: int) -> int:
    """Bytes of the tiled scale array of an [R, K] MXFP4 head (-1: bad shape)."""
    return int(lib().lmhead_mxfp4_scale_bytes(R, K))


def mxfp4_scale_shape(r: int, k: int) -> tuple:
    """Shape of the tiled scale array of an [R, K] MXFP4 head:
    (ceil(R / 16), ceil(K / 512), 16, 16) bytes -- [tile][group of 16 blocks]
    [row in tile][block in group]."""
    if k % 32 or k <= 0 or r < 0:
        raise ValueError("K must be a positive multiple of 32")
    return ((r + 15) // 16, (k // 32 + 15) // 16, 16, 16)


def lmhead_quantize_mxfp4(W: torch.Tensor, out: torch.Tensor | None = None,
                          scales: torch.Tensor | None = None, stream=None):
    """(Wq uint8 [R, K / 2] packed E2M1 codes, scales uint8 in the tiled
    layout, shape mxfp4_scale_shape(R, K)) of a bf16 head, one E8M0 scale per
    32 elements.  Queues one kernel; never synchronizes."""
    _dev_tensor(W, "W", _BF16_LIKE, 2)
    r, k = W.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    if out is None:
        out = torch.empty((r, k // 2), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.zeros(mxfp4_scale_shape(r, k), dtype=torch.uint8, device=W.device)
    _dev_tensor(out, "Wq", (torch.uint8,), 2, W.device)
    _dev_tensor(scales, "scales", (torch.uint8,), 4, W.device)
    if tuple(out.shape) != (r, k // 2) or tuple(scales.shape) != mxfp4_scale_shape(r, k):
        raise ValueError("Wq must be [R, K / 2] and scales of shape mxfp4_scale_shape(R, K)")
    _check(lib().lmhead_quantize_mxfp4(W.data_ptr(), r, k, out.data_ptr(), scales.data_ptr(),
                                       _stream(stream, W.device)), "lmhead_quantize_mxfp4")
    return out, scales


def lmhead_mxfp4_tile_scales(src: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row-major E8M0 scales [R, K / 32] (a head quantized elsewhere) into
    the tiled layout.  Queues one kernel; never synchronizes."""
    _dev_tensor(src, "src", (torch.uint8,), 2)
    r, nblk = src.shape
    k = nblk * 32
    if out is None:
        out = torch.zeros(mxfp4_scale_shape(r, k), dtype=torch.uint8, device=src.device)
    _dev_tensor(out, "scales", (torch.uint8,), 4, src.device)
    if tuple(out.shape) != mxfp4_scale_shape(r, k):
        raise ValueError("scales must have shape mxfp4_scale_shape(R, K)")
    _check(lib().lmhead_mxfp4_tile_scales(src.data_ptr(), r, k, out.data_ptr(), _stream(stream, src.device)),
           "lmhead_mxfp4_tile_scales")
    return out


def _check_mx4_head(h, Wq, scales, d2t):
    _dev_tensor(h, "h", _BF16_LIKE, 2)
    _dev_tensor(Wq, "Wq", (torch.uint8,), 2, h.device)
    _dev_tensor(scales, "scales", (torch.uint8,), 4, h.device)
    m, k = h.shape
    r, half = Wq.shape
    if k != 2 * half:
        raise ValueError("Wq must be [R, K / 2] for h [M, K]")
    if tuple(scales.shape) != mxfp4_scale_shape(r, k):
        raise ValueError("scales must have shape mxfp4_scale_shape(R, K) (the tiled layout)")
    _d2t(d2t, r, h.device, "Wq")
    return m, k, r


def draft_project_argmax_mxfp4(h: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor,
                               d2t: torch.Tensor | None = None, path: int = LMH_PATH_AUTO,
                               out_id: torch.Tensor | None = None, out_logit: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None, stream=None):
    """(out_id int32 [M], out_logit float32 [M]) for the best row of the
    dequantized MXFP4 head per hidden row, mapped through d2t.  Never
    synchronizes."""
    m, k, r = _check_mx4_head(h, Wq, scales, d2t)
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    _check(lib().draft_project_argmax_mxfp4(
        h.data_ptr(), m, k, Wq.data_ptr(), scales.data_ptr(), r,
        d2t.data_ptr() if d2t is not None else None, out_id.data_ptr(), out_logit.data_ptr(),
        workspace.data_ptr(), _nbytes(workspace), path, st),
        "draft_project_argmax_mxfp4")
    return out_id, out_logit


def lmhead_bench_time_argmax_mxfp4(h: torch.Tensor, heads: list, d2t: torch.Tensor | None, path: int,
                                   calls: int, out_id: torch.Tensor, out_logit: torch.Tensor,
                                   workspace: torch.Tensor, stream=None) -> float:
    """lmhead_bench_time_argmax over MXFP4 heads: `heads` is a list of
    (Wq, scales) pairs.  Synchronizes."""
    if not heads:
        raise ValueError("at least one head")
    m, k, r = _check_mx4_head(h, heads[0][0], heads[0][1], d2t)
    for wq, sc in heads:
        _check_mx4_head(h, wq, sc, None)
        if wq.shape[0] != r:
            raise ValueError("every head must have the same shape")
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    qp = (ctypes.c_void_p * len(heads))(*[wq.data_ptr() for wq, _ in heads])
    sp = (ctypes.c_void_p * len(heads))(*[sc.data_ptr() for _, sc in heads])
    out = ctypes.c_double(0.0)
    _check(lib().lmhead_bench_time_argmax_mxfp4(
        h.data_ptr(), m, k, qp, sp, len(heads), r, d2t.data_ptr() if d2t is not None else None,
        out_id.data_ptr(), out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path, calls,
        ctypes.byref(out), st), "lmhead_bench_time_argmax_mxfp4")
    return out.value


def _topk_io(m, topk, out_id, out_logit, workspace, device):
    if out_id is None:
        out_id = torch.empty((m, topk), dtype=torch.int32, device=device)
    if out_logit is None:
        out_logit = torch.empty((m, topk), dtype=torch.float32, device=device)
    _dev_tensor(out_id, "out_id", (torch.int32,), 2, device)
    _dev_tensor(out_logit, "out_logit", (torch.float32,), 2, device)
    if tuple(out_id.shape) != (m, topk) or tuple(out_logit.shape) != (m, topk):
        raise ValueError("outputs must be [M, topk]")
    if workspace is None:
        nbytes = draft_project_topk_workspace_bytes(m, topk)
        if nbytes == 0:
            raise LmheadError(LMH_EINVAL, "top k")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _dev_tensor(workspace, "workspace", None, None, device)
    return out_id, out_logit, workspace


def draft_project_topk_fp8(h: torch.Tensor, Wq: torch.Tensor, scale: torch.Tensor, d2t: torch.Tensor | None,
                           topk: int, out_id: torch.Tensor | None = None, out_logit: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, path: int = LMH_PATH_AUTO, stream=None):
    """(ids int32 [M, topk], logits float32 [M, topk]): the topk best rows of
    the dequantized FP8 head per hidden row, best first, mapped through d2t.
    Never synchronizes."""
    m, k, r = _check_fp8_head(h, Wq, scale, d2t)
    out_id, out_logit, workspace = _topk_io(m, topk, out_id, out_logit, workspace, h.device)
    _check(lib().draft_project_topk_fp8(
        h.data_ptr(), m, k, Wq.data_ptr(), scale.data_ptr(), r, d2t.data_ptr() if d2t is not None else None,
        topk, out_id.data_ptr(), out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path,
        _stream(stream, h.device)), "draft_project_topk_fp8")
    return out_id, out_logit


def draft_project_topk_mxfp4(h: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, d2t: torch.Tensor | None,
                             topk: int, out_id: torch.Tensor | None = None, out_logit: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None, path: int = LMH_PATH_AUTO, stream=None):
    """(ids int32 [M, topk], logits float32 [M, topk]): the topk best rows of
    the dequantized MXFP4 head per hidden row, best first, mapped through
    d2t.  Never synchronizes."""
    m, k, r = _check_mx4_head(h, Wq, scales, d2t)
    out_id, out_logit, workspace = _topk_io(m, topk, out_id, out_logit, workspace, h.device)
    _check(lib().draft_project_topk_mxfp4(
        h.data_ptr(), m, k, Wq.data_ptr(), scales.data_ptr(), r, d2t.data_ptr() if d2t is not None else None,
        topk, out_id.data_ptr(), out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path,
        _stream(stream, h.device)), "draft_project_topk_mxfp4")
    return out_id, out_logit


# --------------------------------------------------------------------------
# NVFP4 heads
# --------------------------------------------------------------------------

def lmhead_nvfp4_scale_bytes(R: int, K: int) -> int:
    """Bytes of the tiled block-scale array of an [R, K] NVFP4 head (-1: bad shape)."""
    return int(lib().lmhead_nvfp4_scale_bytes(R, K))


def nvfp4_scale_shape(r: int, k: int) -> tuple:
    """Shape of the tiled block-scale array of an [R, K] NVFP4 head:
    (ceil(R / 16), ceil(K / 512), 16, 32) bytes -- [tile][group of 32 blocks]
    [row in tile][block in group]."""
    if k % 16 or k <= 0 or r < 0:
        raise ValueError("K must be a positive multiple of 16")
    return ((r + 15) // 16, (k // 16 + 31) // 32, 16, 32)


def lmhead_quantize_nvfp4(W: torch.Tensor, out: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                          gscale: torch.Tensor | None = None, stream=None):
    """(Wq uint8 [R, K / 2] packed E2M1 codes, scales uint8 E4M3 codes in the
    tiled layout (shape nvfp4_scale_shape(R, K)), gscale float32 [1]) of a
    bf16 head.  Queues four kernels; never synchronizes."""
    _dev_tensor(W, "W", _BF16_LIKE, 2)
    r, k = W.shape
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    if out is None:
        out = torch.empty((r, k // 2), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.zeros(nvfp4_scale_shape(r, k), dtype=torch.uint8, device=W.device)
    if gscale is None:
        gscale = torch.ones(1, dtype=torch.float32, device=W.device)
    _dev_tensor(out, "Wq", (torch.uint8,), 2, W.device)
    _dev_tensor(scales, "scales", (torch.uint8,), 4, W.device)
    _dev_tensor(gscale, "gscale", (torch.float32,), 1, W.device)
    if tuple(out.shape) != (r, k // 2) or tuple(scales.shape) != nvfp4_scale_shape(r, k):
        raise ValueError("Wq must be [R, K / 2] and scales of shape nvfp4_scale_shape(R, K)")
    _check(lib().lmhead_quantize_nvfp4(W.data_ptr(), r, k, out.data_ptr(), scales.data_ptr(), gscale.data_ptr(),
                                       _stream(stream, W.device)), "lmhead_quantize_nvfp4")
    return out, scales, gscale


def lmhead_nvfp4_tile_scales(src: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row-major E4M3 block scales [R, K / 16] (a head quantized elsewhere)
    into the tiled layout.  Queues one kernel; never synchronizes."""
    _dev_tensor(src, "src", (torch.uint8,), 2)
    r, nblk = src.shape
    k = nblk * 16
    if out is None:
        out = torch.zeros(nvfp4_scale_shape(r, k), dtype=torch.uint8, device=src.device)
    _dev_tensor(out, "scales", (torch.uint8,), 4, src.device)
    if tuple(out.shape) != nvfp4_scale_shape(r, k):
        raise ValueError("scales must have shape nvfp4_scale_shape(R, K)")
    _check(lib().lmhead_nvfp4_tile_scales(src.data_ptr(), r, k, out.data_ptr(), _stream(stream, src.device)),
           "lmhead_nvfp4_tile_scales")
    return out


def _check_nv4_head(h, Wq, scales, gscale, d2t):
    _dev_tensor(h, "h", _BF16_LIKE, 2)
    _dev_tensor(Wq, "Wq", (torch.uint8,), 2, h.device)
    _dev_tensor(scales, "scales", (torch.uint8,), 4, h.device)
    _dev_tensor(gscale, "gscale", (torch.float32,), 1, h.device)
    m, k = h.shape
    r, half = Wq.shape
    if k != 2 * half:
        raise ValueError("Wq must be [R, K / 2] for h [M, K]")
    if tuple(scales.shape) != nvfp4_scale_shape(r, k):
        raise ValueError("scales must have shape nvfp4_scale_shape(R, K) (the tiled layout)")
    _d2t(d2t, r, h.device, "Wq")
    return m, k, r


def draft_project_argmax_nvfp4(h: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, gscale: torch.Tensor,
                               d2t: torch.Tensor | None = None, path: int = LMH_PATH_AUTO,
                               out_id: torch.Tensor | None = None, out_logit: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None, stream=None):
    """(out_id int32 [M], out_logit float32 [M]) for the best row of the
    dequantized NVFP4 head per hidden row, mapped through d2t.  Never
    synchronizes."""
    m, k, r = _check_nv4_head(h, Wq, scales, gscale, d2t)
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    _check(lib().draft_project_argmax_nvfp4(
        h.data_ptr(), m, k, Wq.data_ptr(), scales.data_ptr(), gscale.data_ptr(), r,
        d2t.data_ptr() if d2t is not None else None, out_id.data_ptr(), out_logit.data_ptr(),
        workspace.data_ptr(), _nbytes(workspace), path, st), "draft_project_argmax_nvfp4")
    return out_id, out_logit


def draft_project_topk_nvfp4(h: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, gscale: torch.Tensor,
                             d2t: torch.Tensor | None, topk: int, out_id: torch.Tensor | None = None,
                             out_logit: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                             path: int = LMH_PATH_AUTO, stream=None):
    """(ids int32 [M, topk], logits float32 [M, topk]): the topk best rows of
    the dequantized NVFP4 head per hidden row, best first, mapped through
    d2t.  Never synchronizes."""
    m, k, r = _check_nv4_head(h, Wq, scales, gscale, d2t)
    out_id, out_logit, workspace = _topk_io(m, topk, out_id, out_logit, workspace, h.device)
    _check(lib().draft_project_topk_nvfp4(
        h.data_ptr(), m, k, Wq.data_ptr(), scales.data_ptr(), gscale.data_ptr(), r,
        d2t.data_ptr() if d2t is not None else None, topk, out_id.data_ptr(), out_logit.data_ptr(),
        workspace.data_ptr(), _nbytes(workspace), path, _stream(stream, h.device)), "draft_project_topk_nvfp4")
    return out_id, out_logit


def lmhead_bench_time_argmax_nvfp4(h: torch.Tensor, heads: list, d2t: torch.Tensor | None, path: int,
                                   calls: int, out_id: torch.Tensor, out_logit: torch.Tensor,
                                   workspace: torch.Tensor, stream=None) -> float:
    """lmhead_bench_time_argmax over NVFP4 heads: `heads` is a list of
    (Wq, scales, gscale) triples.  Synchronizes."""
    if not heads:
        raise ValueError("at least one head")
    m, k, r = _check_nv4_head(h, heads[0][0], heads[0][1], heads[0][2], d2t)
    for wq, sc, gs in heads:
        _check_nv4_head(h, wq, sc, gs, None)
        if wq.shape[0] != r:
            raise ValueError("every head must have the same shape")
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    qp = (ctypes.c_void_p * len(heads))(*[t[0].data_ptr() for t in heads])
    sp = (ctypes.c_void_p * len(heads))(*[t[1].data_ptr() for t in heads])
    gp = (ctypes.c_void_p * len(heads))(*[t[2].data_ptr() for t in heads])
    out = ctypes.c_double(0.0)
    _check(lib().lmhead_bench_time_argmax_nvfp4(
        h.data_ptr(), m, k, qp, sp, gp, len(heads), r, d2t.data_ptr() if d2t is not None else None,
        out_id.data_ptr(), out_logit.data_ptr(), workspace.data_ptr(), _nbytes(workspace), path, calls,
        ctypes.byref(out), st), "lmhead_bench_time_argmax_nvfp4")
    return out.value


# --------------------------------------------------------------------------
# single-launch argmax
# --------------------------------------------------------------------------

def new_state(device=None) -> torch.Tensor:
    """A zeroed state for draft_project_argmax_fused (it must start at zero;
    every call leaves it zero).  One per stream that calls concurrently."""
    return torch.zeros(LMH_STATE_BYTES, dtype=torch.uint8, device=device or "cuda")


def _check_state(state, device) -> None:
    _dev_tensor(state, "state", (torch.uint8,), 1, device)
    if state.numel() < LMH_STATE_BYTES:
        raise ValueError(f"state must hold {LMH_STATE_BYTES} bytes")


def draft_project_argmax_fused_path(h: torch.Tensor, W: torch.Tensor, d2t: torch.Tensor | None, path: int,
                                    state: torch.Tensor, out_id: torch.Tensor | None = None,
                                    out_logit: torch.Tensor | None = None, stream=None):
    """draft_project_argmax_path in one kernel launch per pass: the
    workgroups merge their keys into `state` (from new_state) with atomics
    and the last one writes the outputs.  Never synchronizes."""
    m, k, r = _check_hw(h, W, d2t)
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    _check_state(state, h.device)
    _check(lib().draft_project_argmax_fused_path(
        h.data_ptr(), m, k, W.data_ptr(), r, d2t.data_ptr() if d2t is not None else None, out_id.data_ptr(),
        out_logit.data_ptr(), state.data_ptr(), _nbytes(state), path, _stream(stream, h.device)),
        "draft_project_argmax_fused")
    return out_id, out_logit


def draft_project_argmax_fused(h, W, d2t=None, state=None, out_id=None, out_logit=None, stream=None):
    """draft_project_argmax_fused_path with the library's own kernel choice."""
    if state is None:
        raise ValueError("draft_project_argmax_fused needs a state (new_state) that persists across calls")
    return draft_project_argmax_fused_path(h, W, d2t, LMH_PATH_AUTO, state, out_id, out_logit, stream)


# --------------------------------------------------------------------------
# argmax keys of a head slice (vocabulary-parallel split)
# --------------------------------------------------------------------------

def draft_project_argmax_keys(h: torch.Tensor, W: torch.Tensor, row_base: int = 0, path: int = LMH_PATH_AUTO,
                              out_key: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                              stream=None) -> torch.Tensor:
    """int64 [M] packed keys (ordered logit << 32 | ~(row_base + row)) of
    the slice W's argmax per hidden row; the maximum over the slices' keys
    (compared as unsigned 64-bit) is the whole head's.  Never synchronizes."""
    m, k, r = _check_hw(h, W, None)
    if out_key is None:
        out_key = torch.empty(m, dtype=torch.int64, device=h.device)
    _dev_tensor(out_key, "out_key", (torch.int64,), 1, h.device)
    if out_key.shape[0] < m:
        raise ValueError("out_key must hold M entries")
    st = _stream(stream, h.device)
    workspace = _workspace(workspace, h.device, st)
    _check(lib().draft_project_argmax_keys(h.data_ptr(), m, k, W.data_ptr(), r, row_base, out_key.data_ptr(),
                                           workspace.data_ptr(), _nbytes(workspace), path, st),
           "draft_project_argmax_keys")
    return out_key



def draft_project_argmax_noalloc(h: torch.Tensor, W: torch.Tensor, d2t: torch.Tensor | None = None,
                                 out_id: torch.Tensor | None = None, out_logit: torch.Tensor | None = None,
                                 stream=None):
    """draft_project_argmax with no workspace: the library's own static
    device array holds the per-workgroup keys.  Calls that may overlap on one
    GPU race on that array.  Never synchronizes; the library allocates
    nothing (outputs are allocated here only when not given)."""
    m, k, r = _check_hw(h, W, d2t)
    out_id, out_logit = _outputs(m, out_id, out_logit, h.device)
    _check(lib().draft_project_argmax_noalloc(
        h.data_ptr(), m, k, W.data_ptr(), r, d2t.data_ptr() if d2t is not None else None, out_id.data_ptr(),
        out_logit.data_ptr(), _stream(stream, h.device)), "draft_project_argmax_noalloc")
    return out_id, out_logit
