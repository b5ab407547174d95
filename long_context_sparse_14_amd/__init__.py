"""Python binding of the MI355X (gfx950) DeepSeek Sparse Attention forward library.

Thin ctypes layer over the C ABI declared in ``include/dsa.h`` and built into
``libdsa.so`` next to this file.  It only checks and marshals arguments: every
step of the computation runs in the library's HIP kernels.  PyTorch provides
device memory and the stream (work is enqueued on the current stream unless
one is given).  There is no fallback: if the library is missing, importing
works but the first call raises.

Functions mirror the C entry points:
  index_scores(q_idx, k_idx, w, q_pos0=0)                 -> scores [B,Tq,N] float32
  topk(scores, K, q_pos0=0)                               -> idx [B,Tq,K] int32
  index_scores_presel(q_idx, k_idx, w, K, q_pos0=0)       -> (scores, top-k workspace with the pre-selection)
  topk_presel(scores, K, workspace, dtype, q_pos0=0)      -> idx (from the pre-selection)
  sparse_mla(q, kv, idx, scale, DV=512)                   -> (out [B,Tq,H,DV], lse [B,Tq,H])
  forward(q_idx, k_idx, w, q, kv, K, scale, q_pos0=0, DV=512, return_idx=False)
  forward_noalloc(q_idx, k_idx, w, q, kv, K, scale, ...) (no workspace: the library's per-GPU scratch)
  index_scores_varlen(q_idx, k_idx, w, seq_lens)          -> scores (per-sequence cache lengths)
  topk_varlen(scores, K, seq_lens)                        -> idx
  forward_varlen(q_idx, k_idx, w, q, kv, K, scale, seq_lens, ...)
  cache_append(k_idx, kv, new_k_idx, new_kv, pos)         (in place; either cache may be None)
  index_scores_compressed(q_idx, k_idx, w, m, q_pos0=0)   -> scores over m-compressed entries
  topk_compressed(scores, K, m, q_pos0=0)                 -> idx
  mla_absorb_q(q, w_uk)                                   -> q_lat [..., H, d_c + d_rope] (query absorption)
  mla_out_proj(o_lat, w_uv)                               -> o [..., H, d_v] (value up-projection)
  linear(x, w)                                            -> x w^T (indexer projections)
  indexer_quantize_fp8(x)                                 -> (codes uint8 [..., 128], scales float32 [...])
  index_scores_fp8(q8, q_scale, k8, k_scale, w, q_pos0=0) -> scores [B,Tq,N] float32
  forward_fp8(q8, q_scale, k8, k_scale, w, q, kv, K, scale, q_pos0=0, DV=512, return_idx=False)
  index_scores_paged(q_idx, k_pool, w, seq_lens, block_table)     -> scores over the logical axis
  index_scores_fp8_paged(q8, q_scale, k8_pool, k_scale_pool, w, seq_lens, block_table)
  sparse_mla_paged(q, kv_pool, idx, block_table, scale, DV=512)   -> (out, lse)
  forward_paged(q_idx, k_pool, w, q, kv_pool, K, scale, seq_lens, block_table, ...)
  cache_append_paged(k_pool, kv_pool, new_k_idx, new_kv, pos, block_table)
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree library; DSA_LIB names another build of the same sources (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("DSA_LIB") or os.path.join(_HERE, "libdsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dsa.h")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_BF16, DSA_F32 = 0, 1
DSA_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/dsa.h: the scratch of dsa_forward_noalloc

_lib = None


class DSAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


def _status_name(st: int) -> str:
    return ["DSA_OK", "DSA_ERR_INVALID_ARG", "DSA_ERR_UNSUPPORTED", "DSA_ERR_WORKSPACE",
            "DSA_ERR_HIP"][st] if 0 <= st <= 4 else f"status {st}"


_i64, _i32, _f32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "dsa_version": (ctypes.c_int, []),
    "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_index_scores": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "dsa_topk_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "dsa_topk": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _i64, _i32, _p, _sz, _p]),
    "dsa_index_scores_presel": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _p,
                                               _sz, _p]),
    "dsa_topk_presel": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _p, _sz, _p]),
    "dsa_sparse_mla_workspace_size": (_sz, [_i64, _i64, _i32, _i32, _i32, _i32]),
    "dsa_sparse_mla_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _f32,
                                          _i32, _p, _sz, _p]),
    "dsa_forward_workspace_size": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32, _i32]),
    "dsa_forward": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32,
                                   _i32, _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "dsa_forward_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32,
                                           _i32, _i32, _i32, _f32, _i32, _p]),
    "dsa_index_scores_varlen": (ctypes.c_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "dsa_topk_varlen": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _sz, _p]),
    "dsa_forward_varlen": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32,
                                          _i32, _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "dsa_cache_append": (ctypes.c_int, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "dsa_index_scores_compressed": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                                                   _p]),
    "dsa_topk_compressed": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _p, _sz, _p]),
    "dsa_index_scores_compressed_presel": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32,
                                                          _i32, _i32, _p, _sz, _p]),
    "dsa_topk_compressed_presel": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _p, _sz, _p]),
    "dsa_mla_absorb_q": (ctypes.c_int, [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _p]),
    "dsa_mla_out_proj": (ctypes.c_int, [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _p]),
    "dsa_linear": (ctypes.c_int, [_p, _p, _p, _i64, _i32, _i32, _i32, _p]),
    "dsa_calib_stream": (ctypes.c_int, [_p, _p, _sz, _p]),
    "dsa_indexer_quantize_fp8": (ctypes.c_int, [_p, _p, _p, _i64, _i32, _i32, _p]),
    "dsa_index_scores_fp8": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _p]),
    "dsa_index_scores_fp8_presel": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32,
                                                   _i32, _p, _sz, _p]),
    "dsa_topk_presel_fp8": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _i64, _i32, _p, _sz, _p]),
    "dsa_forward_fp8": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32,
                                       _i32, _i32, _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "dsa_paged_workspace_size": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32]),
    "dsa_index_scores_paged": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i64, _i32, _i32,
                                              _i32, _p]),
    "dsa_index_scores_fp8_paged": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i64,
                                                  _i32, _i32, _i32, _p]),
    "dsa_sparse_mla_fwd_paged": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i64, _i32, _i32,
                                                _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "dsa_forward_paged": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _i64,
                                         _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "dsa_cache_append_paged": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _i64, _i32, _i32, _i32,
                                              _p]),
}


def library() -> ctypes.CDLL:
    """The loaded libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with long_context_sparse_14_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_symbols() -> list:
    """Names of the functions include/dsa.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def _check(rc: int):
    if rc != DSA_OK:
        raise DSAError(rc, library().dsa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _dev(t: torch.Tensor, name: str, ndim: int, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace, workspace.numel() * workspace.element_size()


def index_scores(q_idx, k_idx, w, q_pos0: int = 0, scores=None, stream=None) -> torch.Tensor:
    B, Tq, H_I, D_I = q_idx.shape
    N = k_idx.shape[1]
    dt = q_idx.dtype
    pq = _dev(q_idx, "q_idx", 4)
    pk = _dev(k_idx, "k_idx", 3, dt)
    pw = _dev(w, "w", 3, dt)
    if tuple(k_idx.shape) != (B, N, D_I) or tuple(w.shape) != (B, Tq, H_I):
        raise ValueError("k_idx must be [B,N,D_I] and w [B,Tq,H_I]")
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q_idx.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    if tuple(scores.shape) != (B, Tq, N):
        raise ValueError("scores must be [B,Tq,N]")
    _check(library().dsa_index_scores(pq, pk, pw, ps, B, Tq, N, q_pos0, H_I, D_I, _dtype_code(q_idx),
                                      _stream(stream)))
    return scores


def topk(scores, K: int, q_pos0: int = 0, idx=None, workspace=None, stream=None) -> torch.Tensor:
    B, Tq, N = scores.shape
    ps = _dev(scores, "scores", 3, torch.float32)
    if idx is None:
        idx = torch.empty((B, Tq, K), dtype=torch.int32, device=scores.device)
    pi = _dev(idx, "idx", 3, torch.int32)
    if tuple(idx.shape) != (B, Tq, K):
        raise ValueError("idx must be [B,Tq,K]")
    lib = library()
    ws, nbytes = _workspace(lib.dsa_topk_workspace_size(B, Tq, N, K), scores.device, workspace)
    _check(lib.dsa_topk(ps, pi, B, Tq, N, q_pos0, K, ws.data_ptr() if ws is not None else None, nbytes,
                        _stream(stream)))
    return idx


def sparse_mla(q, kv, idx, scale: float, DV: int = 512, out=None, lse=True, workspace=None, stream=None):
    """Returns (out, lse); lse is None when lse=False."""
    B, Tq, H, D = q.shape
    N = kv.shape[1]
    K = idx.shape[2]
    pq = _dev(q, "q", 4)
    pkv = _dev(kv, "kv", 3, q.dtype)
    pi = _dev(idx, "idx", 3, torch.int32)
    if tuple(kv.shape) != (B, N, D) or tuple(idx.shape[:2]) != (B, Tq):
        raise ValueError("kv must be [B,N,D] and idx [B,Tq,K]")
    if out is None:
        out = torch.empty((B, Tq, H, DV), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", 4, q.dtype)
    lse_t = None
    if lse is True:
        lse_t = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device)
    elif isinstance(lse, torch.Tensor):
        lse_t = lse
    pl = _dev(lse_t, "lse", 3, torch.float32) if lse_t is not None else None
    lib = library()
    dt = _dtype_code(q)
    ws, nbytes = _workspace(lib.dsa_sparse_mla_workspace_size(B, Tq, H, DV, K, dt), q.device, workspace)
    _check(lib.dsa_sparse_mla_fwd(pq, pkv, pi, po, pl, B, Tq, N, H, D, DV, K, scale, dt,
                                  ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)))
    return out, lse_t


def forward_workspace_size(B, Tq, N, H, DV, K, dtype) -> int:
    dt = DSA_BF16 if dtype == torch.bfloat16 else DSA_F32
    return int(library().dsa_forward_workspace_size(B, Tq, N, H, DV, K, dt))


def _forward_args(q_idx, k_idx, w, q, kv, K, q_pos0, DV, out, lse, idx_out, return_idx):
    """Checks and marshals the arguments shared by the fused entry points."""
    B, Tq, H_I, D_I = q_idx.shape
    N = k_idx.shape[1]
    H, D = q.shape[2], q.shape[3]
    dt = q.dtype
    pqi = _dev(q_idx, "q_idx", 4, dt)
    pki = _dev(k_idx, "k_idx", 3, dt)
    pw = _dev(w, "w", 3, dt)
    pq = _dev(q, "q", 4, dt)
    pkv = _dev(kv, "kv", 3, dt)
    if tuple(q.shape[:2]) != (B, Tq) or tuple(kv.shape) != (B, N, D):
        raise ValueError("q must be [B,Tq,H,D] and kv [B,N,D]")
    if out is None:
        out = torch.empty((B, Tq, H, DV), dtype=dt, device=q.device)
    po = _dev(out, "out", 4, dt)
    lse_t = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if lse is True else (
        lse if isinstance(lse, torch.Tensor) else None)
    pl = _dev(lse_t, "lse", 3, torch.float32) if lse_t is not None else None
    if return_idx and idx_out is None:
        idx_out = torch.empty((B, Tq, K), dtype=torch.int32, device=q.device)
    pi = _dev(idx_out, "idx_out", 3, torch.int32) if idx_out is not None else None
    args = (pqi, pki, pw, pq, pkv, po, pl, pi, B, Tq, N, q_pos0, H_I, D_I, H, D, DV, K)
    return args, (B, Tq, N, H), out, lse_t, idx_out


def forward(q_idx, k_idx, w, q, kv, K: int, scale: float, q_pos0: int = 0, DV: int = 512, out=None, lse=True,
            idx_out=None, return_idx: bool = False, workspace=None, stream=None):
    """Indexer -> top-K -> sparse MLA in one call.  Returns (out, lse, idx or None)."""
    args, (B, Tq, N, H), out, lse_t, idx_out = _forward_args(q_idx, k_idx, w, q, kv, K, q_pos0, DV, out, lse,
                                                              idx_out, return_idx)
    lib = library()
    code = _dtype_code(q)
    ws, nbytes = _workspace(lib.dsa_forward_workspace_size(B, Tq, N, H, DV, K, code), q.device, workspace)
    _check(lib.dsa_forward(*args, scale, code, ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)))
    return out, lse_t, idx_out


def forward_noalloc(q_idx, k_idx, w, q, kv, K: int, scale: float, q_pos0: int = 0, DV: int = 512, out=None,
                    lse=True, idx_out=None, return_idx: bool = False, stream=None):
    """forward() through dsa_forward_noalloc: the library's static per-GPU scratch replaces the
    workspace (at most DSA_NOALLOC_SCRATCH_BYTES).  Pass out / lse / idx_out to allocate nothing
    on the Python side either."""
    args, _, out, lse_t, idx_out = _forward_args(q_idx, k_idx, w, q, kv, K, q_pos0, DV, out, lse, idx_out,
                                                 return_idx)
    _check(library().dsa_forward_noalloc(*args, scale, _dtype_code(q), _stream(stream)))
    return out, lse_t, idx_out


def index_scores_presel(q_idx, k_idx, w, K: int, q_pos0: int = 0, scores=None, workspace=None, stream=None):
    """index_scores plus the decode indexer's pre-selection lists, kept in a top-k workspace.
    Returns (scores, workspace): pass both to topk_presel."""
    B, Tq, H_I, D_I = q_idx.shape
    N = k_idx.shape[1]
    dt = q_idx.dtype
    pq, pk, pw = _dev(q_idx, "q_idx", 4, dt), _dev(k_idx, "k_idx", 3, dt), _dev(w, "w", 3, dt)
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q_idx.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    lib = library()
    ws, nbytes = _workspace(lib.dsa_topk_workspace_size(B, Tq, N, K), q_idx.device, workspace)
    _check(lib.dsa_index_scores_presel(pq, pk, pw, ps, B, Tq, N, q_pos0, H_I, D_I, K, _dtype_code(q_idx),
                                       ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)))
    return scores, ws


def topk_presel(scores, K: int, workspace, dtype, q_pos0: int = 0, idx=None, stream=None) -> torch.Tensor:
    """topk for scores and the workspace index_scores_presel filled (dtype: that call's torch dtype)."""
    B, Tq, N = scores.shape
    ps = _dev(scores, "scores", 3, torch.float32)
    if idx is None:
        idx = torch.empty((B, Tq, K), dtype=torch.int32, device=scores.device)
    pi = _dev(idx, "idx", 3, torch.int32)
    code = DSA_BF16 if dtype == torch.bfloat16 else DSA_F32
    nbytes = workspace.numel() if workspace is not None else 0
    _check(library().dsa_topk_presel(ps, pi, B, Tq, N, q_pos0, K, code,
                                     workspace.data_ptr() if workspace is not None else None, nbytes,
                                     _stream(stream)))
    return idx


def _seq_lens(seq_lens, B: int) -> int:
    p = _dev(seq_lens, "seq_lens", 1, torch.int64)
    if seq_lens.shape[0] != B:
        raise ValueError(f"seq_lens must have B={B} entries")
    return p


def index_scores_varlen(q_idx, k_idx, w, seq_lens, scores=None, stream=None) -> torch.Tensor:
    """Indexer scores with per-sequence cache lengths: sequence b's queries are
    its last Tq tokens (positions seq_lens[b] - Tq + t)."""
    B, Tq, H_I, D_I = q_idx.shape
    N = k_idx.shape[1]
    dt = q_idx.dtype
    pq = _dev(q_idx, "q_idx", 4)
    pk = _dev(k_idx, "k_idx", 3, dt)
    pw = _dev(w, "w", 3, dt)
    if tuple(k_idx.shape) != (B, N, D_I) or tuple(w.shape) != (B, Tq, H_I):
        raise ValueError("k_idx must be [B,N,D_I] and w [B,Tq,H_I]")
    pl = _seq_lens(seq_lens, B)
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q_idx.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    if tuple(scores.shape) != (B, Tq, N):
        raise ValueError("scores must be [B,Tq,N]")
    _check(library().dsa_index_scores_varlen(pq, pk, pw, ps, pl, B, Tq, N, H_I, D_I, _dtype_code(q_idx),
                                             _stream(stream)))
    return scores


def topk_varlen(scores, K: int, seq_lens, idx=None, workspace=None, stream=None) -> torch.Tensor:
    B, Tq, N = scores.shape
    ps = _dev(scores, "scores", 3, torch.float32)
    pl = _seq_lens(seq_lens, B)
    if idx is None:
        idx = torch.empty((B, Tq, K), dtype=torch.int32, device=scores.device)
    pi = _dev(idx, "idx", 3, torch.int32)
    if tuple(idx.shape) != (B, Tq, K):
        raise ValueError("idx must be [B,Tq,K]")
    lib = library()
    ws, nbytes = _workspace(lib.dsa_topk_workspace_size(B, Tq, N, K), scores.device, workspace)
    _check(lib.dsa_topk_varlen(ps, pi, pl, B, Tq, N, K, ws.data_ptr() if ws is not None else None, nbytes,
                               _stream(stream)))
    return idx


def forward_varlen(q_idx, k_idx, w, q, kv, K: int, scale: float, seq_lens, DV: int = 512, out=None, lse=True,
                   idx_out=None, return_idx: bool = False, workspace=None, stream=None):
    """forward() with per-sequence cache lengths.  Returns (out, lse, idx or None)."""
    B, Tq, H_I, D_I = q_idx.shape
    N = k_idx.shape[1]
    H, D = q.shape[2], q.shape[3]
    dt = q.dtype
    pqi = _dev(q_idx, "q_idx", 4, dt)
    pki = _dev(k_idx, "k_idx", 3, dt)
    pw = _dev(w, "w", 3, dt)
    pq = _dev(q, "q", 4, dt)
    pkv = _dev(kv, "kv", 3, dt)
    if tuple(q.shape[:2]) != (B, Tq) or tuple(kv.shape) != (B, N, D):
        raise ValueError("q must be [B,Tq,H,D] and kv [B,N,D]")
    pls = _seq_lens(seq_lens, B)
    if out is None:
        out = torch.empty((B, Tq, H, DV), dtype=dt, device=q.device)
    po = _dev(out, "out", 4, dt)
    lse_t = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if lse is True else (
        lse if isinstance(lse, torch.Tensor) else None)
    pl = _dev(lse_t, "lse", 3, torch.float32) if lse_t is not None else None
    if return_idx and idx_out is None:
        idx_out = torch.empty((B, Tq, K), dtype=torch.int32, device=q.device)
    pi = _dev(idx_out, "idx_out", 3, torch.int32) if idx_out is not None else None
    lib = library()
    code = _dtype_code(q)
    ws, nbytes = _workspace(lib.dsa_forward_workspace_size(B, Tq, N, H, DV, K, code), q.device, workspace)
    _check(lib.dsa_forward_varlen(pqi, pki, pw, pq, pkv, po, pl, pi, pls, B, Tq, N, H_I, D_I, H, D, DV, K, scale,
                                  code, ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)))
    return out, lse_t, idx_out


def cache_append(k_idx, kv, new_k_idx, new_kv, pos, stream=None):
    """Writes new_k_idx[b] to k_idx[b, pos[b]] and new_kv[b] to kv[b, pos[b]] in place
    (entries of pos outside [0, N) are skipped).  Either cache may be None."""
    ref = k_idx if k_idx is not None else kv
    if ref is None:
        raise ValueError("no cache to append to")
    B, N = ref.shape[0], ref.shape[1]
    dt = ref.dtype
    D_I = D = 0
    pk = pnk = pv = pnv = None
    if k_idx is not None:
        pk = _dev(k_idx, "k_idx", 3, dt)
        pnk = _dev(new_k_idx, "new_k_idx", 2, dt)
        D_I = k_idx.shape[2]
        if tuple(k_idx.shape[:2]) != (B, N) or tuple(new_k_idx.shape) != (B, D_I):
            raise ValueError("k_idx must be [B,N,D_I] and new_k_idx [B,D_I]")
    if kv is not None:
        pv = _dev(kv, "kv", 3, dt)
        pnv = _dev(new_kv, "new_kv", 2, dt)
        D = kv.shape[2]
        if tuple(kv.shape[:2]) != (B, N) or tuple(new_kv.shape) != (B, D):
            raise ValueError("kv must be [B,N,D] and new_kv [B,D]")
    pp = _dev(pos, "pos", 1, torch.int64)
    if pos.shape[0] != B:
        raise ValueError(f"pos must have B={B} entries")
    _check(library().dsa_cache_append(pk, pv, pnk, pnv, pp, B, N, D_I, D, _dtype_code(ref), _stream(stream)))


def index_scores_compressed(q_idx, k_idx, w, m: int, q_pos0: int = 0, scores=None, stream=None) -> torch.Tensor:
    """Indexer scores against N compressed entries (entry w visible to the query at
    position p when w < (p + 1) // m)."""
    B, Tq, H_I, D_I = q_idx.shape
    N = k_idx.shape[1]
    dt = q_idx.dtype
    pq = _dev(q_idx, "q_idx", 4)
    pk = _dev(k_idx, "k_idx", 3, dt)
    pw = _dev(w, "w", 3, dt)
    if tuple(k_idx.shape) != (B, N, D_I) or tuple(w.shape) != (B, Tq, H_I):
        raise ValueError("k_idx must be [B,N,D_I] and w [B,Tq,H_I]")
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q_idx.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    if tuple(scores.shape) != (B, Tq, N):
        raise ValueError("scores must be [B,Tq,N]")
    _check(library().dsa_index_scores_compressed(pq, pk, pw, ps, B, Tq, N, q_pos0, m, H_I, D_I,
                                                 _dtype_code(q_idx), _stream(stream)))
    return scores


def topk_compressed(scores, K: int, m: int, q_pos0: int = 0, idx=None, workspace=None, stream=None) -> torch.Tensor:
    """Top-K over N compressed entries; row t keeps only entries w < (q_pos0 + t + 1) // m."""
    B, Tq, N = scores.shape
    ps = _dev(scores, "scores", 3, torch.float32)
    if idx is None:
        idx = torch.empty((B, Tq, K), dtype=torch.int32, device=scores.device)
    pi = _dev(idx, "idx", 3, torch.int32)
    if tuple(idx.shape) != (B, Tq, K):
        raise ValueError("idx must be [B,Tq,K]")
    lib = library()
    ws, nbytes = _workspace(lib.dsa_topk_workspace_size(B, Tq, N, K), scores.device, workspace)
    _check(lib.dsa_topk_compressed(ps, pi, B, Tq, N, q_pos0, m, K, ws.data_ptr() if ws is not None else None, nbytes,
                                   _stream(stream)))
    return idx


def index_scores_compressed_presel(q_idx, k_idx, w, m: int, K: int, q_pos0: int = 0, scores=None, workspace=None,
                                   stream=None):
    """index_scores_compressed plus the decode pre-selection lists, kept in a top-k workspace.
    Returns (scores, workspace): pass both to topk_compressed_presel."""
    B, Tq, H_I, D_I = q_idx.shape
    N = k_idx.shape[1]
    dt = q_idx.dtype
    pq, pk, pw = _dev(q_idx, "q_idx", 4), _dev(k_idx, "k_idx", 3, dt), _dev(w, "w", 3, dt)
    if tuple(k_idx.shape) != (B, N, D_I) or tuple(w.shape) != (B, Tq, H_I):
        raise ValueError("k_idx must be [B,N,D_I] and w [B,Tq,H_I]")
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q_idx.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    if tuple(scores.shape) != (B, Tq, N):
        raise ValueError("scores must be [B,Tq,N]")
    lib = library()
    ws, nbytes = _workspace(lib.dsa_topk_workspace_size(B, Tq, N, K), q_idx.device, workspace)
    _check(lib.dsa_index_scores_compressed_presel(pq, pk, pw, ps, B, Tq, N, q_pos0, m, H_I, D_I, K, _dtype_code(q_idx),
                                                  ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)))
    return scores, ws


def topk_compressed_presel(scores, K: int, m: int, workspace, dtype, q_pos0: int = 0, idx=None,
                           stream=None) -> torch.Tensor:
    """topk_compressed for scores and the workspace index_scores_compressed_presel filled (dtype: that
    call's torch dtype)."""
    B, Tq, N = scores.shape
    ps = _dev(scores, "scores", 3, torch.float32)
    if idx is None:
        idx = torch.empty((B, Tq, K), dtype=torch.int32, device=scores.device)
    pi = _dev(idx, "idx", 3, torch.int32)
    code = DSA_BF16 if dtype == torch.bfloat16 else DSA_F32
    nbytes = workspace.numel() if workspace is not None else 0
    _check(library().dsa_topk_compressed_presel(ps, pi, B, Tq, N, q_pos0, m, K, code,
                                                workspace.data_ptr() if workspace is not None else None, nbytes,
                                                _stream(stream)))
    return idx


def mla_absorb_q(q, w_uk, q_lat=None, stream=None) -> torch.Tensor:
    """q [..., H, d_nope + d_rope], w_uk [H, d_nope, d_c] -> q_lat [..., H, d_c + d_rope]."""
    H, d_nope, d_c = w_uk.shape
    if q.dim() < 2 or q.shape[-2] != H or q.shape[-1] < d_nope:
        raise ValueError("q must be [..., H, d_nope + d_rope] with the H and d_nope of w_uk")
    d_rope = q.shape[-1] - d_nope
    M = q.numel() // (H * (d_nope + d_rope))
    pq = _dev(q, "q", q.dim())
    pw = _dev(w_uk, "w_uk", 3, q.dtype)
    if q_lat is None:
        q_lat = torch.empty(tuple(q.shape[:-1]) + (d_c + d_rope,), dtype=q.dtype, device=q.device)
    pl = _dev(q_lat, "q_lat", q.dim(), q.dtype)
    if tuple(q_lat.shape) != tuple(q.shape[:-1]) + (d_c + d_rope,):
        raise ValueError("q_lat must be [..., H, d_c + d_rope]")
    _check(library().dsa_mla_absorb_q(pq, pw, pl, M, H, d_nope, d_rope, d_c, _dtype_code(q), _stream(stream)))
    return q_lat


def mla_out_proj(o_lat, w_uv, o=None, stream=None) -> torch.Tensor:
    """o_lat [..., H, d_c], w_uv [H, d_v, d_c] -> o [..., H, d_v]."""
    H, d_v, d_c = w_uv.shape
    if o_lat.dim() < 2 or tuple(o_lat.shape[-2:]) != (H, d_c):
        raise ValueError("o_lat must be [..., H, d_c] with the H and d_c of w_uv")
    M = o_lat.numel() // (H * d_c)
    pi = _dev(o_lat, "o_lat", o_lat.dim())
    pw = _dev(w_uv, "w_uv", 3, o_lat.dtype)
    if o is None:
        o = torch.empty(tuple(o_lat.shape[:-1]) + (d_v,), dtype=o_lat.dtype, device=o_lat.device)
    po = _dev(o, "o", o_lat.dim(), o_lat.dtype)
    if tuple(o.shape) != tuple(o_lat.shape[:-1]) + (d_v,):
        raise ValueError("o must be [..., H, d_v]")
    _check(library().dsa_mla_out_proj(pi, pw, po, M, H, d_c, d_v, _dtype_code(o_lat), _stream(stream)))
    return o


def linear(x, w, y=None, stream=None) -> torch.Tensor:
    """x [..., K], w [N, K] -> y [..., N] = x w^T."""
    N, K = w.shape
    if x.shape[-1] != K:
        raise ValueError("x must be [..., K] with the K of w")
    M = x.numel() // K
    px = _dev(x, "x", x.dim())
    pw = _dev(w, "w", 2, x.dtype)
    if y is None:
        y = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=x.dtype, device=x.device)
    py = _dev(y, "y", x.dim(), x.dtype)
    if tuple(y.shape) != tuple(x.shape[:-1]) + (N,):
        raise ValueError("y must be [..., N]")
    _check(library().dsa_linear(px, pw, py, M, N, K, _dtype_code(x), _stream(stream)))
    return y


def calib_stream(src, dst=None, stream=None):
    """Stream src's bytes through the device once: a read (dst None) or a copy into dst (same size).
    The bandwidth yardstick for the HBM-bound kernels."""
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    pd = None
    if dst is not None:
        if not (dst.is_cuda and dst.is_contiguous()) or dst.numel() * dst.element_size() != nbytes:
            raise ValueError("dst must be a contiguous device tensor of src's size")
        pd = dst.data_ptr()
    _check(library().dsa_calib_stream(src.data_ptr(), pd, nbytes, _stream(stream)))


def indexer_quantize_fp8(x, codes=None, scales=None, stream=None):
    """bf16 rows [..., 128] -> (Hadamard-rotated E4M3 codes uint8 [..., 128], power-of-two scales float32 [...])."""
    D = x.shape[-1]
    R = x.numel() // D
    px = _dev(x, "x", x.dim(), torch.bfloat16)
    if codes is None:
        codes = torch.empty(tuple(x.shape), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(tuple(x.shape[:-1]), dtype=torch.float32, device=x.device)
    pc = _dev(codes, "codes", x.dim(), torch.uint8)
    ps = _dev(scales, "scales", x.dim() - 1, torch.float32)
    if tuple(codes.shape) != tuple(x.shape) or tuple(scales.shape) != tuple(x.shape[:-1]):
        raise ValueError("codes must be shaped like x and scales like x without its last axis")
    _check(library().dsa_indexer_quantize_fp8(px, pc, ps, R, D, DSA_BF16, _stream(stream)))
    return codes, scales


def _fp8_indexer_args(q8, q_scale, k8, k_scale, w):
    B, Tq, H_I, D_I = q8.shape
    N = k8.shape[1]
    ptrs = (_dev(q8, "q8", 4, torch.uint8), _dev(q_scale, "q_scale", 3, torch.float32),
            _dev(k8, "k8", 3, torch.uint8), _dev(k_scale, "k_scale", 2, torch.float32),
            _dev(w, "w", 3, torch.bfloat16))
    if (tuple(q_scale.shape) != (B, Tq, H_I) or tuple(k8.shape) != (B, N, D_I) or tuple(k_scale.shape) != (B, N)
            or tuple(w.shape) != (B, Tq, H_I)):
        raise ValueError("expected q8 [B,Tq,H_I,D_I], q_scale [B,Tq,H_I], k8 [B,N,D_I], k_scale [B,N], w [B,Tq,H_I]")
    return ptrs, (B, Tq, N, H_I, D_I)


def index_scores_fp8(q8, q_scale, k8, k_scale, w, q_pos0: int = 0, scores=None, stream=None) -> torch.Tensor:
    ptrs, (B, Tq, N, H_I, D_I) = _fp8_indexer_args(q8, q_scale, k8, k_scale, w)
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q8.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    if tuple(scores.shape) != (B, Tq, N):
        raise ValueError("scores must be [B,Tq,N]")
    _check(library().dsa_index_scores_fp8(*ptrs, ps, B, Tq, N, q_pos0, H_I, D_I, DSA_BF16, _stream(stream)))
    return scores


def index_scores_fp8_presel(q8, q_scale, k8, k_scale, w, K: int, q_pos0: int = 0, scores=None, workspace=None,
                            stream=None):
    """index_scores_fp8 plus the pre-selection lists over the FP8 kernel's segments, kept in a top-k
    workspace.  Returns (scores, workspace): pass both to topk_presel_fp8."""
    ptrs, (B, Tq, N, H_I, D_I) = _fp8_indexer_args(q8, q_scale, k8, k_scale, w)
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q8.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    if tuple(scores.shape) != (B, Tq, N):
        raise ValueError("scores must be [B,Tq,N]")
    lib = library()
    ws, nbytes = _workspace(lib.dsa_topk_workspace_size(B, Tq, N, K), q8.device, workspace)
    _check(lib.dsa_index_scores_fp8_presel(*ptrs, ps, B, Tq, N, q_pos0, H_I, D_I, K, DSA_BF16,
                                           ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)))
    return scores, ws


def topk_presel_fp8(scores, K: int, workspace, q_pos0: int = 0, idx=None, stream=None) -> torch.Tensor:
    """topk for scores and the workspace index_scores_fp8_presel filled."""
    B, Tq, N = scores.shape
    ps = _dev(scores, "scores", 3, torch.float32)
    if idx is None:
        idx = torch.empty((B, Tq, K), dtype=torch.int32, device=scores.device)
    pi = _dev(idx, "idx", 3, torch.int32)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(library().dsa_topk_presel_fp8(ps, pi, B, Tq, N, q_pos0, K,
                                         workspace.data_ptr() if workspace is not None else None, nbytes,
                                         _stream(stream)))
    return idx


def forward_fp8(q8, q_scale, k8, k_scale, w, q, kv, K: int, scale: float, q_pos0: int = 0, DV: int = 512,
                out=None, lse=True, workspace=None, return_idx=False, stream=None):
    """dsa_forward with the FP8 indexer: returns (out, lse) or (out, lse, idx)."""
    ptrs, (B, Tq, N, H_I, D_I) = _fp8_indexer_args(q8, q_scale, k8, k_scale, w)
    H, D = q.shape[2], q.shape[3]
    pq = _dev(q, "q", 4, torch.bfloat16)
    pkv = _dev(kv, "kv", 3, torch.bfloat16)
    if tuple(q.shape[:2]) != (B, Tq) or tuple(kv.shape) != (B, N, D):
        raise ValueError("q must be [B,Tq,H,D] and kv [B,N,D]")
    if out is None:
        out = torch.empty((B, Tq, H, DV), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", 4, q.dtype)
    lse_t = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if lse is True else (
        lse if isinstance(lse, torch.Tensor) else None)
    pl = _dev(lse_t, "lse", 3, torch.float32) if lse_t is not None else None
    idx = torch.empty((B, Tq, K), dtype=torch.int32, device=q.device) if return_idx else None
    lib = library()
    ws, nbytes = _workspace(lib.dsa_forward_workspace_size(B, Tq, N, H, DV, K, DSA_BF16), q.device, workspace)
    _check(lib.dsa_forward_fp8(*ptrs, pq, pkv, po, pl, idx.data_ptr() if idx is not None else None, B, Tq, N,
                               q_pos0, H_I, D_I, H, D, DV, K, scale, DSA_BF16,
                               ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)))
    return (out, lse_t, idx) if return_idx else (out, lse_t)


def _paged(block_table, pool_rows: int, B: int):
    """(table pointer, max_blocks, block_size, num_blocks) of a paged cache."""
    pt = _dev(block_table, "block_table", 2, torch.int32)
    if block_table.shape[0] != B:
        raise ValueError(f"block_table must have B={B} rows")
    return pt, block_table.shape[1]


def index_scores_paged(q_idx, k_pool, w, seq_lens, block_table, block_size: int, scores=None, stream=None):
    """Scores [B, Tq, max_blocks * block_size] over a paged indexer key pool [rows, D_I]."""
    B, Tq, H_I, D_I = q_idx.shape
    pt, max_blocks = _paged(block_table, k_pool.shape[0], B)
    num_blocks = k_pool.shape[0] // block_size
    N = max_blocks * block_size
    pq = _dev(q_idx, "q_idx", 4)
    pk = _dev(k_pool, "k_pool", 2, q_idx.dtype)
    pw = _dev(w, "w", 3, q_idx.dtype)
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q_idx.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    _check(library().dsa_index_scores_paged(pq, pk, pw, ps, _seq_lens(seq_lens, B), pt, B, Tq, max_blocks, block_size,
                                            num_blocks, H_I, D_I, _dtype_code(q_idx), _stream(stream)))
    return scores


def index_scores_fp8_paged(q8, q_scale, k8_pool, k_scale_pool, w, seq_lens, block_table, block_size: int,
                           scores=None, stream=None):
    B, Tq, H_I, D_I = q8.shape
    pt, max_blocks = _paged(block_table, k8_pool.shape[0], B)
    num_blocks = k8_pool.shape[0] // block_size
    N = max_blocks * block_size
    ptrs = (_dev(q8, "q8", 4, torch.uint8), _dev(q_scale, "q_scale", 3, torch.float32),
            _dev(k8_pool, "k8_pool", 2, torch.uint8), _dev(k_scale_pool, "k_scale_pool", 1, torch.float32),
            _dev(w, "w", 3, torch.bfloat16))
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q8.device)
    ps = _dev(scores, "scores", 3, torch.float32)
    _check(library().dsa_index_scores_fp8_paged(*ptrs, ps, _seq_lens(seq_lens, B), pt, B, Tq, max_blocks, block_size,
                                                num_blocks, H_I, D_I, DSA_BF16, _stream(stream)))
    return scores


def paged_workspace_size(B, Tq, max_blocks, block_size, H, DV, K, dtype=None) -> int:
    return library().dsa_paged_workspace_size(B, Tq, max_blocks, block_size, H, DV, K,
                                              DSA_BF16 if dtype is None else dtype)


def sparse_mla_paged(q, kv_pool, idx, block_table, block_size: int, scale: float, DV: int = 512, out=None, lse=True,
                     workspace=None, stream=None):
    B, Tq, H, D = q.shape
    K = idx.shape[2]
    pt, max_blocks = _paged(block_table, kv_pool.shape[0], B)
    num_blocks = kv_pool.shape[0] // block_size
    pq = _dev(q, "q", 4)
    pkv = _dev(kv_pool, "kv_pool", 2, q.dtype)
    pi = _dev(idx, "idx", 3, torch.int32)
    if out is None:
        out = torch.empty((B, Tq, H, DV), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", 4, q.dtype)
    lse_t = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if lse is True else (
        lse if isinstance(lse, torch.Tensor) else None)
    pl = _dev(lse_t, "lse", 3, torch.float32) if lse_t is not None else None
    lib = library()
    ws, nbytes = _workspace(paged_workspace_size(B, Tq, max_blocks, block_size, H, DV, K), q.device, workspace)
    _check(lib.dsa_sparse_mla_fwd_paged(pq, pkv, pi, pt, po, pl, B, Tq, max_blocks, block_size, num_blocks, H, D, DV,
                                        K, scale, _dtype_code(q), ws.data_ptr() if ws is not None else None, nbytes,
                                        _stream(stream)))
    return out, lse_t


def forward_paged(q_idx, k_pool, w, q, kv_pool, K: int, scale: float, seq_lens, block_table, block_size: int,
                  DV: int = 512, out=None, lse=True, workspace=None, return_idx=False, stream=None):
    B, Tq, H_I, D_I = q_idx.shape
    H, D = q.shape[2], q.shape[3]
    pt, max_blocks = _paged(block_table, kv_pool.shape[0], B)
    num_blocks = kv_pool.shape[0] // block_size
    if k_pool.shape[0] != kv_pool.shape[0]:
        raise ValueError("k_pool and kv_pool must hold the same number of rows")
    pq = _dev(q_idx, "q_idx", 4)
    pk = _dev(k_pool, "k_pool", 2, q_idx.dtype)
    pw = _dev(w, "w", 3, q_idx.dtype)
    pqq = _dev(q, "q", 4, q_idx.dtype)
    pkv = _dev(kv_pool, "kv_pool", 2, q_idx.dtype)
    if out is None:
        out = torch.empty((B, Tq, H, DV), dtype=q.dtype, device=q.device)
    po = _dev(out, "out", 4, q.dtype)
    lse_t = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if lse is True else (
        lse if isinstance(lse, torch.Tensor) else None)
    pl = _dev(lse_t, "lse", 3, torch.float32) if lse_t is not None else None
    idx = torch.empty((B, Tq, K), dtype=torch.int32, device=q.device) if return_idx else None
    lib = library()
    ws, nbytes = _workspace(paged_workspace_size(B, Tq, max_blocks, block_size, H, DV, K), q.device, workspace)
    _check(lib.dsa_forward_paged(pq, pk, pw, pqq, pkv, po, pl, idx.data_ptr() if idx is not None else None,
                                 _seq_lens(seq_lens, B), pt, B, Tq, max_blocks, block_size, num_blocks, H_I, D_I, H,
                                 D, DV, K, scale, _dtype_code(q), ws.data_ptr() if ws is not None else None, nbytes,
                                 _stream(stream)))
    return (out, lse_t, idx) if return_idx else (out, lse_t)


def cache_append_paged(k_pool, kv_pool, new_k_idx, new_kv, pos, block_table, block_size: int, stream=None):
    ref = k_pool if k_pool is not None else kv_pool
    B = (new_k_idx if new_k_idx is not None else new_kv).shape[0]
    pt, max_blocks = _paged(block_table, ref.shape[0], B)
    num_blocks = ref.shape[0] // block_size
    pk = _dev(k_pool, "k_pool", 2, ref.dtype) if k_pool is not None else None
    pv = _dev(kv_pool, "kv_pool", 2, ref.dtype) if kv_pool is not None else None
    pnk = _dev(new_k_idx, "new_k_idx", 2, ref.dtype) if new_k_idx is not None else None
    pnv = _dev(new_kv, "new_kv", 2, ref.dtype) if new_kv is not None else None
    D_I = k_pool.shape[1] if k_pool is not None else 0
    D = kv_pool.shape[1] if kv_pool is not None else 0
    pp = _dev(pos, "pos", 1, torch.int64)
    _check(library().dsa_cache_append_paged(pk, pv, pnk, pnv, pp, pt, B, max_blocks, block_size, num_blocks, D_I, D,
                                            _dtype_code(ref), _stream(stream)))
