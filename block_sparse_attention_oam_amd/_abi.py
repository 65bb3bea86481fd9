"""ctypes binding of libstem.so (include/stem.h).  Argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module turns torch tensors into device
pointers, NumPy arrays into host pointers, and C status codes into exceptions.  If libstem.so is missing
the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# STEM_LIB names another build of the same library (the host-sanitized one the CPU tests load).
LIB_PATH = os.environ.get("STEM_LIB") or os.path.join(_PKG, "libstem.so")

STEM_OK = 0
STEM_E_INVALID_ARG = -1
STEM_E_UNSUPPORTED = -2
STEM_E_WORKSPACE = -3
STEM_E_HIP = -4

DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}
MAX_REQS = 256
SCRATCH_BYTES = 64 << 20  # STEM_SCRATCH_BYTES

EXPORTS = ["stem_block_counts", "stem_workspace_bytes", "stem_workspace_layout", "stem_tpd_budgets_host",
           "stem_status_string", "stem_last_error", "stem_score", "stem_tpd_topk", "bsa_prefill",
           "bsa_prefill_inloop", "stem_score_select", "stem_naive_workspace_bytes", "stem_naive_score",
           "stem_quantize_score", "stem_score_noalloc", "stem_quantize_fp8", "bsa_workspace_bytes", "bsa_prefill_ws"]


class StemError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class StemProblemC(ctypes.Structure):
    _fields_ = [
        ("num_reqs", ctypes.c_int32),
        ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("kv_paged", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("page_table_stride", ctypes.c_int32),
        ("q_scale", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libstem.so (built in-tree by block_sparse_attention_oam_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() (or "
                              f"python -m block_sparse_attention_oam_amd.build) first")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(StemProblemC)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.stem_block_counts.argtypes = [P, ctypes.POINTER(i64), ctypes.POINTER(i32)]
        L.stem_workspace_bytes.argtypes = [P]
        L.stem_workspace_bytes.restype = sz
        L.stem_workspace_layout.argtypes = [P, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.stem_tpd_budgets_host.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i32)]
        L.stem_status_string.argtypes = [ctypes.c_int]
        L.stem_status_string.restype = ctypes.c_char_p
        L.stem_last_error.argtypes = []
        L.stem_last_error.restype = ctypes.c_char_p
        L.stem_score.argtypes = [P, vp, vp, vp, ctypes.c_float, vp, i64, vp, sz, vp]
        L.stem_score_noalloc.argtypes = [P, vp, vp, vp, ctypes.c_float, vp, i64, vp]
        L.stem_tpd_topk.argtypes = [P, vp, i64, i32, i32, i32, i32, vp, i32, vp, vp]
        L.bsa_prefill.argtypes = [P, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp]
        L.bsa_prefill_inloop.argtypes = [P, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp]
        L.bsa_workspace_bytes.argtypes = [P]
        L.bsa_workspace_bytes.restype = sz
        L.bsa_prefill_ws.argtypes = [P, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp]
        L.stem_score_select.argtypes = [P, vp, vp, vp, ctypes.c_float, i32, i32, i32, i32, vp, i32, vp, vp, sz, vp]
        L.stem_quantize_score.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, i64, vp, sz, vp]
        L.stem_quantize_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.stem_naive_workspace_bytes.argtypes = [P, i32]
        L.stem_naive_workspace_bytes.restype = sz
        L.stem_naive_score.argtypes = [P, vp, vp, vp, ctypes.c_float, i32, vp, i64, vp, sz, vp, sz, vp]
        for name in ("stem_block_counts", "stem_workspace_layout", "stem_tpd_budgets_host", "stem_score",
                     "stem_tpd_topk", "bsa_prefill", "bsa_prefill_inloop", "stem_score_select", "stem_naive_score", "stem_quantize_score",
                     "stem_score_noalloc", "stem_quantize_fp8"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(status: int) -> str:
    try:
        return lib().stem_status_string(status).decode()
    except ImportError:
        return str(status)


def _check(status: int) -> None:
    if status != STEM_OK:
        raise StemError(status, lib().stem_last_error().decode())


def _ptr(t) -> int | None:
    """Device (torch tensor) or None -> address."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


@dataclass
class Problem:
    """Problem descriptor (stem_problem) plus the host arrays it points to."""

    c: StemProblemC
    cu_seqlens: np.ndarray  # host int32, kept alive for the descriptor
    _keep: tuple = ()

    @property
    def ref(self):
        return ctypes.byref(self.c)


def make_problem(cu_seqlens, hq: int, hkv: int, head_dim: int, block: int, dtype: str, *, page_table=None,
                 page_size: int = 0, num_pages: int = 0, q_scale=None, k_scale=None, v_scale=None) -> Problem:
    """Build a stem_problem.  cu_seqlens: host int32 [R+1]; page_table / scales: device tensors or None."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    c = StemProblemC()
    c.num_reqs = len(cu) - 1
    c.cu_seqlens = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    c.hq, c.hkv, c.head_dim, c.block = hq, hkv, head_dim, block
    c.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    c.kv_paged = 1 if page_table is not None else 0
    c.page_size = page_size
    c.num_pages = num_pages
    c.page_table = _ptr(page_table)
    c.page_table_stride = int(page_table.shape[-1]) if page_table is not None else 0
    c.q_scale, c.k_scale, c.v_scale = _ptr(q_scale), _ptr(k_scale), _ptr(v_scale)
    return Problem(c, cu, (page_table, q_scale, k_scale, v_scale))


def block_counts(p: Problem):
    nb, mx = ctypes.c_int64(), ctypes.c_int32()
    _check(lib().stem_block_counts(p.ref, ctypes.byref(nb), ctypes.byref(mx)))
    return nb.value, mx.value


def workspace_bytes(p: Problem) -> int:
    n = lib().stem_workspace_bytes(p.ref)
    if n == 0:
        _check(STEM_E_INVALID_ARG)
    return n


def workspace_layout(p: Problem):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().stem_workspace_layout(p.ref, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def stem_tpd_budgets_host(n: int, rho_num: int, rho_den: int, mu_num: int, mu_den: int) -> np.ndarray:
    out = np.zeros(max(n, 1), dtype=np.int32)
    _check(lib().stem_tpd_budgets_host(n, rho_num, rho_den, mu_num, mu_den,
                                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out[:n]


def stem_score(p: Problem, q, k, v, beta: float, scores, ws, stream=None) -> None:
    """scores: device float [hq][NB][stride]; ws: device uint8 workspace."""
    _check(lib().stem_score(p.ref, _ptr(q), _ptr(k), _ptr(v), float(beta), _ptr(scores),
                            int(scores.shape[-1]), _ptr(ws), int(ws.numel() * ws.element_size()),
                            _stream(stream)))


def stem_score_noalloc(p: Problem, q, k, v, beta: float, scores, stream=None) -> None:
    """stem_score with the pooled tensors in the library's static per-device scratch (no workspace)."""
    _check(lib().stem_score_noalloc(p.ref, _ptr(q), _ptr(k), _ptr(v), float(beta), _ptr(scores),
                                    int(scores.shape[-1]), _stream(stream)))


def stem_tpd_topk(p: Problem, scores, rho: tuple, mu: tuple, mask, counts, stream=None) -> None:
    """rho, mu: (num, den).  mask: device int32/uint32 [hq][NB][words]; counts: device int32 [hq][NB]."""
    _check(lib().stem_tpd_topk(p.ref, _ptr(scores), int(scores.shape[-1]), int(rho[0]), int(rho[1]),
                               int(mu[0]), int(mu[1]), _ptr(mask), int(mask.shape[-1]), _ptr(counts),
                               _stream(stream)))


def stem_score_select(p: Problem, q, k, v, beta: float, rho: tuple, mu: tuple, mask, counts, ws,
                      stream=None) -> None:
    """Pooling, scoring and selection in one call, without the score tensor (same mask and counts as
    stem_score followed by stem_tpd_topk)."""
    words = int(mask.shape[-1]) if mask is not None else 0
    ws_bytes = int(ws.numel() * ws.element_size()) if ws is not None else 0
    _check(lib().stem_score_select(p.ref, _ptr(q), _ptr(k), _ptr(v), float(beta), int(rho[0]), int(rho[1]),
                                   int(mu[0]), int(mu[1]), _ptr(mask), words, _ptr(counts), _ptr(ws), ws_bytes,
                                   _stream(stream)))


def stem_quantize_score(p: Problem, q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, beta: float, scores, ws,
                        stream=None) -> None:
    """bf16 q, k, v -> e4m3fn codes and per-head scales, pooled workspace and block scores (fp8 layer)."""
    _check(lib().stem_quantize_score(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale),
                                     _ptr(k_scale), _ptr(v_scale), float(beta), _ptr(scores),
                                     int(scores.shape[-1]) if scores is not None else 0, _ptr(ws),
                                     int(ws.numel() * ws.element_size()) if ws is not None else 0, _stream(stream)))


def stem_quantize_fp8(p: Problem, q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, stream=None) -> None:
    """bf16 q, k, v -> e4m3fn codes and per-head scales (no pooling)."""
    _check(lib().stem_quantize_fp8(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale),
                                   _ptr(k_scale), _ptr(v_scale), _stream(stream)))


def naive_workspace_bytes(p: Problem, samples: int) -> int:
    n = lib().stem_naive_workspace_bytes(p.ref, int(samples))
    if n == 0:
        raise StemError(STEM_E_INVALID_ARG, lib().stem_last_error().decode())
    return int(n)


def stem_naive_score(p: Problem, q, k, v, beta: float, samples: int, scores, ws, naive_ws, stream=None) -> None:
    """The naive token-level block scores (comparison path), in stem_score's layout."""
    _check(lib().stem_naive_score(p.ref, _ptr(q), _ptr(k), _ptr(v), float(beta), int(samples), _ptr(scores),
                                  int(scores.shape[-1]), _ptr(ws), int(ws.numel() * ws.element_size()),
                                  _ptr(naive_ws), int(naive_ws.numel() * naive_ws.element_size())
                                  if naive_ws is not None else 0, _stream(stream)))


def bsa_prefill(p: Problem, q, k, v, mask, out, lse=None, softmax_scale: float = 0.0, stream=None) -> None:
    """mask: device [hq][NB][words] or None (dense causal)."""
    words = int(mask.shape[-1]) if mask is not None else 0
    _check(lib().bsa_prefill(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(mask), words, float(softmax_scale),
                             _ptr(out), _ptr(lse), _stream(stream)))


def bsa_workspace_bytes(p: Problem) -> int:
    """Workspace of bsa_prefill_ws (0 for problems that need none); raises on an invalid problem."""
    block_counts(p)
    return int(lib().bsa_workspace_bytes(p.ref))


def bsa_prefill_ws(p: Problem, q, k, v, mask, out, lse=None, softmax_scale: float = 0.0, ws=None,
                   stream=None) -> None:
    """bsa_prefill with a workspace (fp8: V expanded to bf16 there first; same outputs)."""
    words = int(mask.shape[-1]) if mask is not None else 0
    nbytes = int(ws.numel() * ws.element_size()) if ws is not None else 0
    _check(lib().bsa_prefill_ws(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(mask), words, float(softmax_scale),
                                _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(stream)))


def bsa_prefill_inloop(p: Problem, q, k, v, mask, out, lse=None, softmax_scale: float = 0.0, stream=None) -> None:
    """The comparison variant with the skip test inside the loop (same outputs as bsa_prefill)."""
    words = int(mask.shape[-1]) if mask is not None else 0
    _check(lib().bsa_prefill_inloop(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(mask), words, float(softmax_scale),
                                    _ptr(out), _ptr(lse), _stream(stream)))
