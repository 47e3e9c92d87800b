"""ctypes binding over libsmqa.so — argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks dtype,
shape and contiguity, allocates outputs and workspace with torch when the
caller does not pass them, and calls the C entry point of the same name on
torch's current stream.  All computation happens in the library's HIP kernels.
If libsmqa.so has not been built, the first call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsmqa.so")
# the same library built with SMQA_DEBUG (device-side range checks, smqa_debug_flags)
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsmqa_debug.so")

SMQA_OK = 0
ERRORS = {-1: "SMQA_ERR_NULL", -2: "SMQA_ERR_SHAPE", -3: "SMQA_ERR_ALIGN",
          -4: "SMQA_ERR_UNSUPPORTED", -5: "SMQA_ERR_WORKSPACE", -6: "SMQA_ERR_HIP"}

_lib = None


class SmqaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class Layout(ctypes.Structure):
    """Mirror of smqa_layout (include/smqa.h)."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("seq_start", ctypes.c_void_p),
        ("num_q", ctypes.c_int32),
        ("q_start", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("max_ctx", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_L = ctypes.c_int64
_F = ctypes.c_float
_S = ctypes.c_size_t
_LP = ctypes.POINTER(Layout)

_SIGS = {
    "sparse_mqa_score": (_I, [_LP, _P, _P, _P, _P, _P, _I, _I, _I, _P, _L, _P]),
    "sparse_mqa_score_fp8mma": (_I, [_LP, _P, _P, _P, _P, _P, _I, _I, _I, _P, _L, _P]),
    "topk_select": (_I, [_LP, _P, _L, _P, _I, _I, _P, _P, _P, _S, _P]),
    "sparse_mqa_attend": (_I, [_LP, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _F,
                               _P, _P, _P, _S, _P]),
    "sparse_mqa_attend_fp8kv": (_I, [_LP, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _F,
                                     _P, _P, _P, _S, _P]),
    "sparse_mqa_attend_nvfp4": (_I, [_LP, _P, _P, _P, _P, _F, _P, _I, _P, _P, _P, _P, _I, _I, _I,
                                     _F, _P, _P, _P, _S, _P]),
    "sparse_mqa_attend_mxfp8q": (_I, [_LP, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _F,
                                      _P, _P, _P, _S, _P]),
    "sparse_mqa_attend_fused": (_I, [_LP, _P, _P, _P, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I,
                                     _I, _I, _F, _P, _P, _P, _P, _P, _S, _P]),
    "smqa_attend_fused_workspace_size": (_S, [_LP, _I, _I, _I, _I]),
    "decode_step": (_I, [_LP, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                         _I, _I, _I, _F, _I, _P, _P, _P, _P, _S, _P]),
    "decode_step_noalloc": (_I, [_LP, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _I, _I, _I, _F, _I, _P, _P, _P, _P]),
    "decode_step_fused": (_I, [_LP, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P,
                               _P, _P, _P, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _S, _P]),
    "smqa_topk_workspace_size": (_S, [_LP, _I, _I]),
    "smqa_attend_workspace_size": (_S, [_LP, _I, _I, _I, _I]),
    "smqa_decode_step_workspace_size": (_S, [_LP, _I, _I, _I, _I, _I]),
    "smqa_attend_plan": (_I, [_LP, _I, _I, _I, _I, _P, _P]),
    "smqa_last_error": (ctypes.c_char_p, []),
    "smqa_version": (ctypes.c_char_p, []),
    "smqa_debug_flags": (_I, [_P, _I]),
}


def load(path: Optional[str] = None):
    """Load libsmqa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m fp8_kv_cache_sparse_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


_debug_lib = None


@contextlib.contextmanager
def debug_build():
    """Inside the block every call of this binding goes to libsmqa_debug.so (the library built
    with SMQA_DEBUG: device-side range checks whose findings debug_flags() reads)."""
    global _lib, _debug_lib
    prev = load()
    if _debug_lib is None:
        _debug_lib = load(DEBUG_LIB_PATH)
    _lib = _debug_lib
    try:
        yield
    finally:
        _lib = prev


def debug_flags(clear: bool = True) -> int:
    """The debug word of the current device (SMQA_DEBUG_* bits; synchronises the device), then
    cleared unless clear is False.  Raises SmqaError outside a debug build."""
    v = ctypes.c_uint32(0)
    _check(load().smqa_debug_flags(ctypes.byref(v), 1 if clear else 0))
    return v.value


SMQA_DEBUG_POSITION = 1
SMQA_DEBUG_E8M0 = 2
SMQA_DEBUG_LAYOUT = 4
SMQA_DEBUG_CAND = 8


def _check(code: int):
    if code != SMQA_OK:
        raise SmqaError(code, load().smqa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, ndim=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


_U8 = (torch.uint8, torch.float8_e4m3fn)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class Batch:
    """Ragged layout (see smqa_layout).  Keeps the device tensors alive."""

    def __init__(self, seq_start: torch.Tensor, q_start: torch.Tensor, q_pos: torch.Tensor,
                 max_ctx: int):
        _dev(seq_start, "seq_start", torch.int64, 1)
        _dev(q_start, "q_start", torch.int32, 1)
        _dev(q_pos, "q_pos", torch.int32, 1)
        self.tensors = (seq_start, q_start, q_pos)
        self.B = seq_start.numel() - 1
        self.T = q_pos.numel()
        self.max_ctx = int(max_ctx)
        self.c = Layout(self.B, seq_start.data_ptr(), self.T, q_start.data_ptr(),
                        q_pos.data_ptr(), self.max_ctx)

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)


def _ws_ptr(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    p = ws.data_ptr()
    off = (-p) % 256
    return p + off, ws.numel() - off


def version() -> str:
    return load().smqa_version().decode()


def sparse_mqa_score(L: Batch, q_fp8, w, k_fp8, k_scale=None, cand=None, scores=None, stream=None):
    """Indexer scores -> float32 [T, ld] (dense: ld = max_ctx; candidate mode: ld = n_cand)."""
    return _score("sparse_mqa_score", L, q_fp8, w, k_fp8, k_scale, cand, scores, stream)


def sparse_mqa_score_fp8mma(L: Batch, q_fp8, w, k_fp8, k_scale=None, cand=None, scores=None, stream=None):
    """sparse_mqa_score with the contraction on the FP8 matrix cores (Di = 128)."""
    return _score("sparse_mqa_score_fp8mma", L, q_fp8, w, k_fp8, k_scale, cand, scores, stream)


def _score(entry, L, q_fp8, w, k_fp8, k_scale, cand, scores, stream):
    lib = load()
    _dev(q_fp8, "q_fp8", _U8, 3)
    _dev(w, "w", torch.float32, 2)
    _dev(k_fp8, "k_fp8", _U8, 2)
    _dev(k_scale, "k_scale", torch.float32, 1)
    _dev(cand, "cand", torch.int32, 2)
    T, Hi, Di = q_fp8.shape
    n_cand = 0 if cand is None else cand.shape[1]
    if scores is None:
        ld = n_cand if cand is not None else L.max_ctx
        scores = torch.empty((T, max(ld, 1)), dtype=torch.float32, device=q_fp8.device)
    _dev(scores, "scores", torch.float32, 2)
    _check(getattr(lib, entry)(L.ref, _ptr(q_fp8), _ptr(w), _ptr(k_fp8), _ptr(k_scale), _ptr(cand),
                               n_cand, Hi, Di, _ptr(scores), scores.shape[1], _stream(stream)))
    return scores


def topk_select(L: Batch, scores, k: int, cand=None, idx=None, workspace=None, stream=None,
                val=None, want_val=False):
    """Top-k positions -> int32 [T, k], ascending, -1 padded; with want_val (or val given)
    also their scores -> (idx, val float32 [T, k], -inf padded)."""
    lib = load()
    _dev(scores, "scores", torch.float32, 2)
    _dev(cand, "cand", torch.int32, 2)
    n_cand = 0 if cand is None else cand.shape[1]
    if idx is None:
        idx = torch.empty((L.T, k), dtype=torch.int32, device=scores.device)
    _dev(idx, "idx", torch.int32, 2)
    if want_val and val is None:
        val = torch.empty((L.T, k), dtype=torch.float32, device=scores.device)
    _dev(val, "val", torch.float32, 2)
    need = lib.smqa_topk_workspace_size(L.ref, k, n_cand)
    if workspace is None:
        workspace = _workspace(need, scores.device)
    wp, wb = _ws_ptr(workspace)
    _check(lib.topk_select(L.ref, _ptr(scores), scores.shape[1], _ptr(cand), n_cand, k, _ptr(idx),
                           _ptr(val), wp, wb, _stream(stream)))
    return (idx, val) if val is not None else idx


def sparse_mqa_attend(L: Batch, q, kv_codes, kv_e8m0, kv_rowscale, idx, swa, swa_scale, swa_pos0,
                      swa_clip, sm_scale: float, out=None, lse=None, workspace=None, stream=None):
    """Sparse MQA attention -> (out float32 [T, Hq, D], lse float32 [T, Hq])."""
    return _attend_mx("sparse_mqa_attend", L, q, kv_codes, kv_e8m0, kv_rowscale, idx, swa, swa_scale,
                      swa_pos0, swa_clip, sm_scale, out, lse, workspace, stream)


def sparse_mqa_attend_mxfp8q(L: Batch, q, kv_codes, kv_e8m0, kv_rowscale, idx, swa, swa_scale, swa_pos0,
                             swa_clip, sm_scale: float, out=None, lse=None, workspace=None, stream=None):
    """Sparse MQA attention on the scaled matrix cores with the query quantised to MXFP8
    -> (out float32 [T, Hq, D], lse float32 [T, Hq])."""
    return _attend_mx("sparse_mqa_attend_mxfp8q", L, q, kv_codes, kv_e8m0, kv_rowscale, idx, swa,
                      swa_scale, swa_pos0, swa_clip, sm_scale, out, lse, workspace, stream)


def _attend_mx(entry, L, q, kv_codes, kv_e8m0, kv_rowscale, idx, swa, swa_scale, swa_pos0, swa_clip,
               sm_scale, out, lse, workspace, stream):
    lib = load()
    _dev(q, "q", torch.bfloat16, 3)
    _dev(kv_codes, "kv_codes", torch.uint8, 2)
    _dev(kv_e8m0, "kv_e8m0", torch.uint8, 2)
    _dev(kv_rowscale, "kv_rowscale", torch.float32, 1)
    _dev(idx, "idx", torch.int32, 2)
    _dev(swa, "swa", _U8, 3)
    _dev(swa_scale, "swa_scale", torch.float32, 2)
    _dev(swa_pos0, "swa_pos0", torch.int32, 1)
    _dev(swa_clip, "swa_clip", torch.int32, 1)
    T, Hq, D = q.shape
    W = swa.shape[1]
    k = idx.shape[1]
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 3)
    _dev(lse, "lse", torch.float32, 2)
    need = lib.smqa_attend_workspace_size(L.ref, k, W, Hq, D)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wp, wb = _ws_ptr(workspace)
    _check(getattr(lib, entry)(L.ref, _ptr(q), _ptr(kv_codes), _ptr(kv_e8m0), _ptr(kv_rowscale),
                               _ptr(idx), k, _ptr(swa), _ptr(swa_scale), _ptr(swa_pos0),
                               _ptr(swa_clip), W, Hq, D, float(sm_scale), _ptr(out), _ptr(lse),
                               wp, wb, _stream(stream)))
    return out, lse


def sparse_mqa_attend_fp8kv(L: Batch, q, kv_fp8, kv_rowscale, idx, swa, swa_scale, swa_pos0,
                            swa_clip, sm_scale: float, out=None, lse=None, workspace=None,
                            stream=None):
    """Sparse MQA attention over an FP8 global cache -> (out float32 [T, Hq, D], lse)."""
    lib = load()
    _dev(q, "q", torch.bfloat16, 3)
    _dev(kv_fp8, "kv_fp8", torch.uint8, 2)
    _dev(kv_rowscale, "kv_rowscale", torch.float32, 1)
    _dev(idx, "idx", torch.int32, 2)
    _dev(swa, "swa", _U8, 3)
    _dev(swa_scale, "swa_scale", torch.float32, 2)
    _dev(swa_pos0, "swa_pos0", torch.int32, 1)
    _dev(swa_clip, "swa_clip", torch.int32, 1)
    T, Hq, D = q.shape
    W = swa.shape[1]
    k = idx.shape[1]
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 3)
    _dev(lse, "lse", torch.float32, 2)
    need = lib.smqa_attend_workspace_size(L.ref, k, W, Hq, D)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wp, wb = _ws_ptr(workspace)
    _check(lib.sparse_mqa_attend_fp8kv(L.ref, _ptr(q), _ptr(kv_fp8), _ptr(kv_rowscale), _ptr(idx),
                                       k, _ptr(swa), _ptr(swa_scale), _ptr(swa_pos0),
                                       _ptr(swa_clip), W, Hq, D, float(sm_scale), _ptr(out),
                                       _ptr(lse), wp, wb, _stream(stream)))
    return out, lse


def sparse_mqa_attend_nvfp4(L: Batch, q, kv_codes, kv_scales, kv_rowscale, kv_global_scale: float,
                            idx, swa, swa_scale, swa_pos0, swa_clip, sm_scale: float, out=None,
                            lse=None, workspace=None, stream=None):
    """Sparse MQA attention over an NVFP4 global cache -> (out float32 [T, Hq, D], lse)."""
    lib = load()
    _dev(q, "q", torch.bfloat16, 3)
    _dev(kv_codes, "kv_codes", torch.uint8, 2)
    _dev(kv_scales, "kv_scales", torch.uint8, 2)
    _dev(kv_rowscale, "kv_rowscale", torch.float32, 1)
    _dev(idx, "idx", torch.int32, 2)
    _dev(swa, "swa", _U8, 3)
    _dev(swa_scale, "swa_scale", torch.float32, 2)
    _dev(swa_pos0, "swa_pos0", torch.int32, 1)
    _dev(swa_clip, "swa_clip", torch.int32, 1)
    T, Hq, D = q.shape
    W = swa.shape[1]
    k = idx.shape[1]
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, 3)
    _dev(lse, "lse", torch.float32, 2)
    need = lib.smqa_attend_workspace_size(L.ref, k, W, Hq, D)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wp, wb = _ws_ptr(workspace)
    _check(lib.sparse_mqa_attend_nvfp4(L.ref, _ptr(q), _ptr(kv_codes), _ptr(kv_scales),
                                       _ptr(kv_rowscale), float(kv_global_scale), _ptr(idx), k,
                                       _ptr(swa), _ptr(swa_scale), _ptr(swa_pos0), _ptr(swa_clip),
                                       W, Hq, D, float(sm_scale), _ptr(out), _ptr(lse), wp, wb,
                                       _stream(stream)))
    return out, lse


def sparse_mqa_attend_fused(L: Batch, q, rope_cos, rope_sin, kv_codes, kv_e8m0, kv_rowscale, idx,
                            swa, swa_scale, swa_pos0, swa_clip, sm_scale: float, out_fp8=None,
                            out_scale=None, out=None, lse=None, want_out=True, workspace=None,
                            stream=None):
    """Query RoPE -> attention -> inverse RoPE -> FP8 in one call.
    -> (out_fp8 uint8 [T, Hq, D], out_scale float32 [T, Hq], out float32 or None, lse)."""
    lib = load()
    _dev(q, "q", torch.bfloat16, 3)
    _dev(rope_cos, "rope_cos", torch.float32, 2)
    _dev(rope_sin, "rope_sin", torch.float32, 2)
    _dev(kv_codes, "kv_codes", torch.uint8, 2)
    _dev(kv_e8m0, "kv_e8m0", torch.uint8, 2)
    _dev(kv_rowscale, "kv_rowscale", torch.float32, 1)
    _dev(idx, "idx", torch.int32, 2)
    _dev(swa, "swa", _U8, 3)
    _dev(swa_scale, "swa_scale", torch.float32, 2)
    _dev(swa_pos0, "swa_pos0", torch.int32, 1)
    _dev(swa_clip, "swa_clip", torch.int32, 1)
    T, Hq, D = q.shape
    W = swa.shape[1]
    k = idx.shape[1]
    R = 0 if rope_cos is None else rope_cos.shape[1]
    if out_fp8 is None:
        out_fp8 = torch.empty((T, Hq, D), dtype=torch.uint8, device=q.device)
    if out_scale is None:
        out_scale = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    if out is None and want_out:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _dev(out_fp8, "out_fp8", torch.uint8, 3)
    _dev(out_scale, "out_scale", torch.float32, 2)
    _dev(out, "out", torch.float32, 3)
    _dev(lse, "lse", torch.float32, 2)
    need = lib.smqa_attend_fused_workspace_size(L.ref, k, W, Hq, D)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wp, wb = _ws_ptr(workspace)
    _check(lib.sparse_mqa_attend_fused(L.ref, _ptr(q), _ptr(rope_cos), _ptr(rope_sin), R,
                                       _ptr(kv_codes), _ptr(kv_e8m0), _ptr(kv_rowscale), _ptr(idx), k,
                                       _ptr(swa), _ptr(swa_scale), _ptr(swa_pos0), _ptr(swa_clip), W,
                                       Hq, D, float(sm_scale), _ptr(out_fp8), _ptr(out_scale),
                                       _ptr(out), _ptr(lse), wp, wb, _stream(stream)))
    return out_fp8, out_scale, out, lse


def decode_step_workspace_size(L: Batch, k: int, n_cand: int, W: int, Hq: int, D: int) -> int:
    return load().smqa_decode_step_workspace_size(L.ref, k, n_cand, W, Hq, D)


def decode_step(L: Batch, q_fp8, w, k_fp8, k_scale, cand, q, kv_codes, kv_e8m0, kv_rowscale, swa,
                swa_scale, swa_pos0, swa_clip, k: int, sm_scale: float, out=None, lse=None,
                idx=None, workspace=None, stream=None, return_idx=True):
    """score -> top-k -> attend in one call -> (out, lse, idx or None)."""
    lib = load()
    for t_, n_, d_, nd in ((q_fp8, "q_fp8", _U8, 3), (w, "w", torch.float32, 2),
                           (k_fp8, "k_fp8", _U8, 2), (k_scale, "k_scale", torch.float32, 1),
                           (cand, "cand", torch.int32, 2), (q, "q", torch.bfloat16, 3),
                           (kv_codes, "kv_codes", torch.uint8, 2), (kv_e8m0, "kv_e8m0", torch.uint8, 2),
                           (kv_rowscale, "kv_rowscale", torch.float32, 1), (swa, "swa", _U8, 3),
                           (swa_scale, "swa_scale", torch.float32, 2),
                           (swa_pos0, "swa_pos0", torch.int32, 1), (swa_clip, "swa_clip", torch.int32, 1)):
        _dev(t_, n_, d_, nd)
    T, Hi, Di = q_fp8.shape
    _, Hq, D = q.shape
    W = swa.shape[1]
    n_cand = 0 if cand is None else cand.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if idx is None and return_idx:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    _dev(out, "out", torch.float32, 3)
    _dev(lse, "lse", torch.float32, 2)
    _dev(idx, "idx", torch.int32, 2)
    need = lib.smqa_decode_step_workspace_size(L.ref, k, n_cand, W, Hq, D)
    if workspace is None:
        workspace = _workspace(need, dev)
    wp, wb = _ws_ptr(workspace)
    _check(lib.decode_step(L.ref, _ptr(q_fp8), _ptr(w), _ptr(k_fp8), _ptr(k_scale), _ptr(cand), n_cand,
                           Hi, Di, _ptr(q), _ptr(kv_codes), _ptr(kv_e8m0), _ptr(kv_rowscale),
                           _ptr(swa), _ptr(swa_scale), _ptr(swa_pos0), _ptr(swa_clip), W, Hq, D,
                           float(sm_scale), k, _ptr(out), _ptr(lse), _ptr(idx), wp, wb,
                           _stream(stream)))
    return out, lse, idx


def decode_step_noalloc(L: Batch, q_fp8, w, k_fp8, k_scale, cand, q, kv_codes, kv_e8m0, kv_rowscale, swa,
                        swa_scale, swa_pos0, swa_clip, k: int, sm_scale: float, out, lse, idx=None,
                        stream=None):
    """decode_step on the library's device scratch buffer: the caller passes the outputs
    (out float32 [T, Hq, D], lse float32 [T, Hq], idx int32 [T, k] or None) and nothing is
    allocated, by this function or the library."""
    lib = load()
    for t_, n_, d_, nd in ((q_fp8, "q_fp8", _U8, 3), (w, "w", torch.float32, 2),
                           (k_fp8, "k_fp8", _U8, 2), (k_scale, "k_scale", torch.float32, 1),
                           (cand, "cand", torch.int32, 2), (q, "q", torch.bfloat16, 3),
                           (kv_codes, "kv_codes", torch.uint8, 2), (kv_e8m0, "kv_e8m0", torch.uint8, 2),
                           (kv_rowscale, "kv_rowscale", torch.float32, 1), (swa, "swa", _U8, 3),
                           (swa_scale, "swa_scale", torch.float32, 2),
                           (swa_pos0, "swa_pos0", torch.int32, 1), (swa_clip, "swa_clip", torch.int32, 1),
                           (out, "out", torch.float32, 3), (lse, "lse", torch.float32, 2),
                           (idx, "idx", torch.int32, 2)):
        _dev(t_, n_, d_, nd)
    T, Hi, Di = q_fp8.shape
    _, Hq, D = q.shape
    W = swa.shape[1]
    n_cand = 0 if cand is None else cand.shape[1]
    _check(lib.decode_step_noalloc(L.ref, _ptr(q_fp8), _ptr(w), _ptr(k_fp8), _ptr(k_scale), _ptr(cand),
                                   n_cand, Hi, Di, _ptr(q), _ptr(kv_codes), _ptr(kv_e8m0),
                                   _ptr(kv_rowscale), _ptr(swa), _ptr(swa_scale), _ptr(swa_pos0),
                                   _ptr(swa_clip), W, Hq, D, float(sm_scale), k, _ptr(out), _ptr(lse),
                                   _ptr(idx), _stream(stream)))
    return out, lse, idx


def decode_step_fused(L: Batch, q_fp8, w, k_fp8, k_scale, cand, q, rope_cos, rope_sin, kv_codes,
                      kv_e8m0, kv_rowscale, swa, swa_scale, swa_pos0, swa_clip, k: int,
                      sm_scale: float, out_fp8=None, out_scale=None, out=None, lse=None, idx=None,
                      want_out=True, workspace=None, stream=None):
    """score -> top-k -> fused attention (query RoPE, inverse RoPE, FP8 output) in one call
    -> (out_fp8, out_scale, out or None, lse, idx)."""
    lib = load()
    for t_, n_, dt, nd in ((q_fp8, "q_fp8", _U8, 3), (w, "w", torch.float32, 2), (k_fp8, "k_fp8", _U8, 2),
                           (k_scale, "k_scale", torch.float32, 1), (cand, "cand", torch.int32, 2),
                           (q, "q", torch.bfloat16, 3), (rope_cos, "rope_cos", torch.float32, 2),
                           (rope_sin, "rope_sin", torch.float32, 2), (kv_codes, "kv_codes", torch.uint8, 2),
                           (kv_e8m0, "kv_e8m0", torch.uint8, 2), (kv_rowscale, "kv_rowscale", torch.float32, 1),
                           (swa, "swa", _U8, 3), (swa_scale, "swa_scale", torch.float32, 2),
                           (swa_pos0, "swa_pos0", torch.int32, 1), (swa_clip, "swa_clip", torch.int32, 1)):
        _dev(t_, n_, dt, nd)
    T, Hi, Di = q_fp8.shape
    _, Hq, D = q.shape
    W = swa.shape[1]
    R = 0 if rope_cos is None else rope_cos.shape[1]
    n_cand = 0 if cand is None else cand.shape[1]
    dev = q.device
    if out_fp8 is None:
        out_fp8 = torch.empty((T, Hq, D), dtype=torch.uint8, device=dev)
    if out_scale is None:
        out_scale = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if out is None and want_out:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    for t_, n_, dt, nd in ((out_fp8, "out_fp8", torch.uint8, 3), (out_scale, "out_scale", torch.float32, 2),
                           (out, "out", torch.float32, 3), (lse, "lse", torch.float32, 2),
                           (idx, "idx", torch.int32, 2)):
        _dev(t_, n_, dt, nd)
    need = lib.smqa_decode_step_workspace_size(L.ref, k, n_cand, W, Hq, D)
    if workspace is None:
        workspace = _workspace(need, dev)
    wp, wb = _ws_ptr(workspace)
    _check(lib.decode_step_fused(L.ref, _ptr(q_fp8), _ptr(w), _ptr(k_fp8), _ptr(k_scale), _ptr(cand), n_cand,
                                 Hi, Di, _ptr(q), _ptr(rope_cos), _ptr(rope_sin), R, _ptr(kv_codes),
                                 _ptr(kv_e8m0), _ptr(kv_rowscale), _ptr(swa), _ptr(swa_scale),
                                 _ptr(swa_pos0), _ptr(swa_clip), W, Hq, D, float(sm_scale), k,
                                 _ptr(out_fp8), _ptr(out_scale), _ptr(out), _ptr(lse), _ptr(idx), wp, wb,
                                 _stream(stream)))
    return out_fp8, out_scale, out, lse, idx
