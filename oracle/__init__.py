"""CPU oracle for the DeepSeek Sparse Attention (DSA) forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the CPU-baseline leg of the benchmark may import this module; the product
path (the HIP library and its Python binding) never does, and this module
never imports the product path.  The two share no code: the only thing both
sides consume is the seeded input generator in ``synth/``.

The arithmetic lives in ``dsa_oracle.cpp`` beside this file: plain C++17 in
double precision, one function per step of the method in the pages' order,
split by query rows over ``std::thread`` (a row is always computed by one
thread in one fixed order, so the thread count never changes a result).  It
is compiled with g++ into ``libdsa_oracle.so``.  This module only marshals
numpy arrays to that library through ctypes: it checks shapes, lays out row
lists and output buffers, and holds no step of the method.

Pages and sections followed (each function below names its own):
  DeepSeek-V3.2 model documentation, section "DeepSeek Sparse Attention
  (DSA)": the lightning indexer scores every query against the keys before
  it; it keeps its own single-head key cache; fine-grained token selection
  keeps the index_topk best keys per query and the main attention runs over
  those only, as an additive mask; FP8 after a Hadamard rotation computes the
  same scores.  Its "DeepseekV32Config" section: index_n_heads 64,
  index_head_dim 128, index_topk 2048, kv_lora_rank 512, qk_rope_head_dim 64.
  DeepSeek-V4 model documentation, attention mask layout: -1 means no
  selection; a compressed entry is visible once its window has closed.
  DeepSeek-V3 model documentation, "DeepseekV3Config" and its limitations
  note: LoRA ranks and head widths; the port computes attention per head.

Readings taken where the pages are silent (each listed with its reason in
the repository's design notes): the score is the head-weighted sum of
ReLU(per-head q.k), no further scale; a query sees its own position; top-k
ties go to the lower index, kept indices are listed ascending and padded with
-1; the MLA is in absorbed latent form (value = first DV entries of the
latent row); indices < 0 or >= N are masked; an empty row gives o = 0 and
lse = -inf; lse is a natural log.  FP8: OCP E4M3, the unnormalised Sylvester
rotation by the float32 fast Walsh-Hadamard transform (pair distance 1, 2,
4, ...), one power-of-two scale per rotated row, round to nearest even, the
factor D divided out of the score.

Storage dtypes accepted everywhere: numpy ``uint16`` arrays hold bf16 bit
patterns, ``float32`` and ``float64`` are themselves; every value is widened
exactly to double inside the library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "dsa_oracle.cpp")
LIB_PATH = os.path.join(_HERE, "libdsa_oracle.so")
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra"]

F64, F32, BF16 = 0, 1, 2

__all__ = [
    "Oracle", "build_library", "threads", "as_f64", "bf16_bits_to_f64", "n_valid_keys", "paged_gather",
    "index_scores_rows", "index_scores", "index_scores_batch", "topk_row", "topk", "topk_rows", "sparse_mla_rows",
    "sparse_mla", "sparse_mla_batch", "dense_masked_mla", "forward_rows", "forward_batch", "mla_naive_rows",
    "mla_absorb_query", "mla_output_projection", "linear", "fwht_f32", "e4m3_decode", "e4m3_encode_rne",
    "pow2_scale_exp", "quantize_fp8_rows", "index_scores_fp8_rows", "sylvester_hadamard",
]


def build_library(force: bool = False, source: str = SOURCE, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the C++ oracle with g++ into a shared library."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < max(
            os.path.getmtime(source), os.path.getmtime(os.path.join(_HERE, "dsa_oracle.h"))):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++"] + CXXFLAGS + list(extra_flags) + ["-I", _HERE, source, "-o", tmp])
        os.replace(tmp, out)
    return out


def threads() -> int:
    """Worker threads the oracle uses: DSA_ORACLE_THREADS, else OMP_NUM_THREADS
    (the CPU share of a shared host), else every core this process may run on."""
    for var in ("DSA_ORACLE_THREADS", "OMP_NUM_THREADS"):
        v = os.environ.get(var, "")
        if v.strip().isdigit() and int(v) > 0:
            return int(v)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


_i64, _i32, _int, _dbl, _p = ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_double, ctypes.c_void_p

_SIGNATURES = {
    "dsao_version": (_int, []),
    "dsao_widen": (_int, [_p, _int, _i64, _p]),
    "dsao_n_valid_keys": (_i64, [_i64, _i64, _i64, _i64]),
    "dsao_index_scores": (_int, [_p, _int, _p, _int, _p, _int, _i64, _i64, _i64, _i32, _i32, _p, _i64, _p, _i64,
                                 _p, _int]),
    "dsao_topk": (_int, [_p, _i64, _i64, _p, _i32, _p, _int]),
    "dsao_sparse_mla": (_int, [_p, _int, _p, _int, _p, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _dbl, _p, _i64,
                               _p, _p, _int]),
    "dsao_dense_masked_mla": (_int, [_p, _int, _p, _int, _p, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _dbl, _p,
                                     _p, _i64, _p, _p, _int]),
    "dsao_forward": (_int, [_p, _int, _p, _int, _p, _int, _p, _int, _p, _int, _i64, _i64, _i64, _p, _i32, _i32,
                            _i32, _i32, _i32, _i32, _dbl, _p, _i64, _p, _p, _p, _p, _int]),
    "dsao_sylvester_hadamard": (_int, [_i32, _p]),
    "dsao_fwht_f32": (_int, [_p, _i64, _i32]),
    "dsao_e4m3_decode": (_int, [_p, _i64, _p]),
    "dsao_e4m3_encode_rne": (_int, [_p, _i64, _p]),
    "dsao_pow2_scale_exp": (_int, [_dbl]),
    "dsao_quantize_fp8_rows": (_int, [_p, _int, _i64, _i32, _p, _p]),
    "dsao_index_scores_fp8": (_int, [_p, _p, _p, _p, _p, _int, _i64, _i64, _i64, _i32, _i32, _p, _p, _i64, _p,
                                     _int]),
    "dsao_linear": (_int, [_p, _int, _p, _int, _i64, _i64, _i64, _p, _int]),
    "dsao_mla_absorb_query": (_int, [_p, _int, _p, _int, _i64, _i32, _i32, _i32, _i32, _p, _int]),
    "dsao_mla_output_projection": (_int, [_p, _int, _p, _int, _i64, _i32, _i32, _i32, _p, _int]),
    "dsao_mla_naive_row": (_int, [_p, _int, _p, _int, _p, _int, _i64, _p, _i32, _p, _int, _p, _int, _i32, _i32,
                                  _i32, _i32, _i32, _dbl, _p, _p, _int]),
    "dsao_paged_gather": (_int, [_p, _i64, _i64, _p, _i64, _i64, _i64, _p]),
}


def _fp(a):
    """(contiguous array, dtype code) for a floating-point input tensor."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a), BF16
    if a.dtype == np.float32:
        return np.ascontiguousarray(a), F32
    return np.ascontiguousarray(a, dtype=np.float64), F64


def _ptr(a):
    return a.ctypes.data if a is not None else None


def _pos0(q_pos0, B):
    """Position of query 0 per sequence: a scalar for every sequence, or one per sequence."""
    return np.ascontiguousarray(np.broadcast_to(np.asarray(q_pos0, dtype=np.int64), (B,)))


def _row_list(rows):
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    return r, r.shape[0]


class Oracle:
    """The oracle library at one path (the default build, or a test's own build of a variant of the source)."""

    def __init__(self, path: str = LIB_PATH):
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        self.lib = lib
        self.path = path

    def _call(self, name, *args):
        rc = getattr(self.lib, name)(*args)
        if rc != 0:
            raise ValueError(f"{name} rejected its arguments (status {rc})")

    # ---------------------------------------------------------------- helpers

    def as_f64(self, x) -> np.ndarray:
        """Any accepted storage dtype -> float64 (bf16 bit patterns widened exactly)."""
        a, dt = _fp(x)
        out = np.empty(a.shape, dtype=np.float64)
        self._call("dsao_widen", _ptr(a), dt, a.size, _ptr(out))
        return out

    bf16_bits_to_f64 = as_f64

    def n_valid_keys(self, t: int, q_pos0: int, N: int, m: int = 1) -> int:
        """Keys the query at position q_pos0 + t sees: positions 0..q_pos0+t capped by N; with a key axis
        compressed at rate m, entry w is visible once w < (q_pos0 + t + 1) // m (DeepSeek-V4 documentation,
        attention mask layout)."""
        n = int(self.lib.dsao_n_valid_keys(int(t), int(q_pos0), int(N), int(m)))
        if n < 0:
            raise ValueError("n_valid_keys: m must be >= 1 and N >= 0")
        return n

    def paged_gather(self, pool, table_row, block_size: int, n_rows: int) -> np.ndarray:
        """Rows 0..n_rows-1 of one sequence of a paged cache: logical row r is pool row
        table_row[r // block_size] * block_size + r % block_size (reading of the static and growing cache
        layers of the DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)")."""
        pool = np.ascontiguousarray(pool)
        table = np.ascontiguousarray(np.asarray(table_row, dtype=np.int64).reshape(-1))
        out = np.empty((int(n_rows),) + pool.shape[1:], dtype=pool.dtype)
        row_bytes = pool.strides[0] if pool.ndim > 1 else pool.itemsize
        self._call("dsao_paged_gather", _ptr(pool), pool.shape[0], row_bytes, _ptr(table), table.size,
                   int(block_size), int(n_rows), _ptr(out))
        return out

    # ------------------------------------------------------------ O1 indexer

    def index_scores_batch(self, q_idx, k_idx, w, rows, q_pos0, m: int = 1) -> np.ndarray:
        """Index scores of the queries `rows` ((b, t) pairs) of a batch: q_idx [B,Tq,H_I,D_I],
        k_idx [B,N,D_I], w [B,Tq,H_I].  Returns float64 [n_rows, N]; entry s of row r is
            I[s] = sum_h w[b,t,h] * ReLU(sum_d q_idx[b,t,h,d] * k_idx[b,s,d])
        for the visible keys and NaN past them.  q_pos0: scalar or one per sequence."""
        qa, qd = _fp(q_idx)
        ka, kd = _fp(k_idx)
        wa, wd = _fp(w)
        B, Tq, H_I, D_I = qa.shape
        N = ka.shape[1]
        r, n = _row_list(rows)
        out = np.full((n, N), np.nan)
        self._call("dsao_index_scores", _ptr(qa), qd, _ptr(ka), kd, _ptr(wa), wd, B, Tq, N, H_I, D_I,
                   _ptr(_pos0(q_pos0, B)), int(m), _ptr(r), n, _ptr(out), threads())
        return out

    def index_scores_rows(self, q_idx_b, k_idx_b, w_b, ts, q_pos0: int, m: int = 1) -> list:
        """One sequence (q_idx_b [Tq,H_I,D_I], k_idx_b [N,D_I], w_b [Tq,H_I]): one float64 vector per query
        t in `ts`, of length n_valid_keys(t, q_pos0, N, m)."""
        ts = [int(t) for t in ts]
        N = np.asarray(k_idx_b).shape[0]
        full = self.index_scores_batch(np.asarray(q_idx_b)[None], np.asarray(k_idx_b)[None], np.asarray(w_b)[None],
                                       [(0, t) for t in ts], q_pos0, m)
        return [full[i, :self.n_valid_keys(t, q_pos0, N, m)].copy() for i, t in enumerate(ts)]

    def index_scores(self, q_idx, k_idx, w, q_pos0: int, m: int = 1) -> np.ndarray:
        """Full score tensor [B, Tq, N] (float64); entries a query may not see are NaN."""
        B, Tq = np.asarray(q_idx).shape[:2]
        N = np.asarray(k_idx).shape[1]
        full = self.index_scores_batch(q_idx, k_idx, w, [(b, t) for b in range(B) for t in range(Tq)], q_pos0, m)
        return full.reshape(B, Tq, N)

    # -------------------------------------------------------------- O2 top-k

    def topk_rows(self, scores, n_valid, K: int) -> np.ndarray:
        """scores [R, S] float32 with n_valid[r] visible entries per row -> idx [R, K] int32: the K best
        under (score desc, index asc), ascending, -1 padded (DeepSeek-V3.2 documentation, "DeepSeek Sparse
        Attention (DSA)", token selection; DeepSeek-V4 documentation: -1 is no selection)."""
        s = np.ascontiguousarray(np.asarray(scores, dtype=np.float32))
        if s.ndim == 1:
            s = s[None]
        nv = np.ascontiguousarray(np.asarray(n_valid, dtype=np.int64).reshape(-1))
        out = np.empty((s.shape[0], int(K)), dtype=np.int32)
        self._call("dsao_topk", _ptr(s), s.shape[0], s.shape[1], _ptr(nv), int(K), _ptr(out), threads())
        return out

    def topk_row(self, scores, K: int) -> np.ndarray:
        """One row of n visible scores (decided in float32, the precision scores are stored in)."""
        s = np.asarray(scores, dtype=np.float32).reshape(-1)
        return self.topk_rows(s[None], [s.shape[0]], K)[0]

    def topk(self, scores, K: int, q_pos0: int, m: int = 1) -> np.ndarray:
        """scores [B, Tq, N] -> idx [B, Tq, K] int32 (row t uses its visible keys only)."""
        s = np.asarray(scores, dtype=np.float32)
        B, Tq, N = s.shape
        nv = [self.n_valid_keys(t, q_pos0, N, m) for b in range(B) for t in range(Tq)]
        return self.topk_rows(s.reshape(B * Tq, N), nv, K).reshape(B, Tq, int(K))

    # --------------------------------------------------------- O3 sparse MLA

    def sparse_mla_batch(self, q, kv, idx, rows, scale: float, DV: int):
        """Queries `rows` of q [B,Tq,H,D] over kv [B,N,D] with idx [B,Tq,K] -> (o [R,H,DV], lse [R,H])."""
        qa, qd = _fp(q)
        ka, kd = _fp(kv)
        ia = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
        B, Tq, H, D = qa.shape
        N = ka.shape[1]
        K = ia.shape[-1]
        r, n = _row_list(rows)
        o = np.empty((n, H, int(DV)))
        lse = np.empty((n, H))
        self._call("dsao_sparse_mla", _ptr(qa), qd, _ptr(ka), kd, _ptr(ia), B, Tq, N, H, D, int(DV), K,
                   float(scale), _ptr(r), n, _ptr(o), _ptr(lse), threads())
        return o, lse

    def sparse_mla(self, q, kv, idx, scale: float, DV: int):
        """q [B,Tq,H,D], kv [B,N,D], idx [B,Tq,K] -> (o [B,Tq,H,DV], lse [B,Tq,H]) float64."""
        B, Tq, H, _ = np.asarray(q).shape
        o, lse = self.sparse_mla_batch(q, kv, idx, [(b, t) for b in range(B) for t in range(Tq)], scale, DV)
        return o.reshape(B, Tq, H, int(DV)), lse.reshape(B, Tq, H)

    def sparse_mla_rows(self, q_bt, kv_rows, idx_row, scale: float, DV: int):
        """One query: q_bt [H, D]; kv_rows is the sequence's cache [N, D] or a dict {index: row} of the rows
        the query selects.  Returns (o [H, DV], lse [H])."""
        idx_row = np.asarray(idx_row, dtype=np.int64).reshape(-1)
        if isinstance(kv_rows, dict):
            # the given rows, in a compact array, with the selection renumbered into it (masked stays masked)
            keys = [int(i) for i in idx_row if int(i) >= 0]
            pos = {k: j for j, k in enumerate(dict.fromkeys(keys))}
            D = np.asarray(q_bt).shape[-1]
            first = next(iter(kv_rows.values())) if kv_rows else np.zeros(D)
            kv = np.stack([np.asarray(kv_rows[k]) for k in pos]) if pos else np.zeros((0, D), np.asarray(first).dtype)
            idx_row = np.array([pos[int(i)] if int(i) >= 0 else -1 for i in idx_row], dtype=np.int64)
        else:
            kv = np.asarray(kv_rows)
        if kv.shape[0] == 0:
            kv = np.zeros((1, np.asarray(q_bt).shape[-1]), dtype=kv.dtype)
            idx_row = np.full_like(idx_row, -1)
        o, lse = self.sparse_mla_batch(np.asarray(q_bt)[None, None], kv[None], idx_row.astype(np.int32)[None, None],
                                       [(0, 0)], scale, DV)
        return o[0], lse[0]

    def dense_masked_mla(self, q, kv, idx, scale: float, DV: int, q_pos0):
        """The same attention as dense causal attention over all visible keys with an additive mask, 0 on
        selected keys and -inf elsewhere (the token-selection paragraph's mechanism)."""
        qa, qd = _fp(q)
        ka, kd = _fp(kv)
        ia = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
        B, Tq, H, D = qa.shape
        N = ka.shape[1]
        r, n = _row_list([(b, t) for b in range(B) for t in range(Tq)])
        o = np.empty((n, H, int(DV)))
        lse = np.empty((n, H))
        self._call("dsao_dense_masked_mla", _ptr(qa), qd, _ptr(ka), kd, _ptr(ia), B, Tq, N, H, D, int(DV),
                   ia.shape[-1], float(scale), _ptr(_pos0(q_pos0, B)), _ptr(r), n, _ptr(o), _ptr(lse), threads())
        return o.reshape(B, Tq, H, int(DV)), lse.reshape(B, Tq, H)

    # -------------------------------------------------------- O4 composition

    def forward_batch(self, q_idx, k_idx, w, q, kv, rows, q_pos0, K: int, scale: float, DV: int,
                      want_scores: bool = True) -> dict:
        """Indexer -> top-k -> sparse MLA for the queries `rows` of a batch.  Returns float64 scores
        [R, N] (NaN past the visible keys; None unless want_scores), int32 idx [R, K], o [R, H, DV] and
        lse [R, H]."""
        qia, qid = _fp(q_idx)
        kia, kid = _fp(k_idx)
        wa, wd = _fp(w)
        qa, qd = _fp(q)
        ka, kd = _fp(kv)
        B, Tq, H_I, D_I = qia.shape
        N = kia.shape[1]
        H, D = qa.shape[2], qa.shape[3]
        r, n = _row_list(rows)
        sc = np.full((n, N), np.nan) if want_scores else None
        idx = np.empty((n, int(K)), dtype=np.int32)
        o = np.empty((n, H, int(DV)))
        lse = np.empty((n, H))
        self._call("dsao_forward", _ptr(qia), qid, _ptr(kia), kid, _ptr(wa), wd, _ptr(qa), qd, _ptr(ka), kd, B, Tq,
                   N, _ptr(_pos0(q_pos0, B)), H_I, D_I, H, D, int(DV), int(K), float(scale), _ptr(r), n, _ptr(sc),
                   _ptr(idx), _ptr(o), _ptr(lse), threads())
        return {"scores": sc, "idx": idx, "o": o, "lse": lse}

    def forward_rows(self, q_idx_b, k_idx_b, w_b, q_b, kv_b, ts, q_pos0: int, K: int, scale: float, DV: int):
        """The three steps for queries `ts` of one sequence; a list of dicts with the query's float64
        scores (visible part), its int32 indices, and its (o, lse)."""
        ts = [int(t) for t in ts]
        N = np.asarray(k_idx_b).shape[0]
        res = self.forward_batch(np.asarray(q_idx_b)[None], np.asarray(k_idx_b)[None], np.asarray(w_b)[None],
                                 np.asarray(q_b)[None], np.asarray(kv_b)[None], [(0, t) for t in ts], q_pos0, K,
                                 scale, DV)
        return [{"t": t, "scores": res["scores"][i, :self.n_valid_keys(t, q_pos0, N)].copy(), "idx": res["idx"][i],
                 "o": res["o"][i], "lse": res["lse"][i]} for i, t in enumerate(ts)]

    # ------------------------------------------------------ MLA projections

    def mla_naive_rows(self, q_head, c_kv, k_rope, idx_row, W_UK, W_UV, scale: float):
        """Naive MLA for one query: head h's keys [W_UK[h] c_j | k_rope_j] and values W_UV[h] c_j over the
        selected tokens (DeepSeek-V3 documentation: the port's per-head attention).  q_head [H, d_nope +
        d_rope], c_kv [N, d_c], k_rope [N, d_rope], W_UK [H, d_nope, d_c], W_UV [H, d_v, d_c]."""
        qa, qd = _fp(q_head)
        ca, cd = _fp(c_kv)
        ra, rd = _fp(k_rope)
        ua, ud = _fp(W_UK)
        va, vd = _fp(W_UV)
        idx = np.ascontiguousarray(np.asarray(idx_row, dtype=np.int32).reshape(-1))
        H, d_nope, d_c = ua.shape
        d_v = va.shape[1]
        d_rope = ra.shape[1]
        o = np.empty((H, d_v))
        lse = np.empty(H)
        self._call("dsao_mla_naive_row", _ptr(qa), qd, _ptr(ca), cd, _ptr(ra), rd, ca.shape[0], _ptr(idx), idx.size,
                   _ptr(ua), ud, _ptr(va), vd, H, d_nope, d_rope, d_c, d_v, float(scale), _ptr(o), _ptr(lse), threads())
        return o, lse

    def mla_absorb_query(self, q_head, W_UK) -> np.ndarray:
        """Fold the key up-projection into the query: [..., H, d_nope + d_rope] -> [..., H, d_c + d_rope],
        q_lat[h] = [W_UK[h]^T q_nope[h], q_rope[h]]."""
        qa, qd = _fp(q_head)
        ua, ud = _fp(W_UK)
        H, d_nope, d_c = ua.shape
        d_rope = qa.shape[-1] - d_nope
        M = qa.size // (H * qa.shape[-1])
        out = np.empty(qa.shape[:-1] + (d_c + d_rope,))
        self._call("dsao_mla_absorb_query", _ptr(qa), qd, _ptr(ua), ud, M, H, d_nope, d_rope, d_c, _ptr(out), threads())
        return out

    def mla_output_projection(self, o_lat, W_UV) -> np.ndarray:
        """Value up-projection of the latent output: [..., H, d_c] -> [..., H, d_v], o[h] = W_UV[h] o_lat[h]."""
        oa, od = _fp(o_lat)
        va, vd = _fp(W_UV)
        H, d_v, d_c = va.shape
        M = oa.size // (H * d_c)
        out = np.empty(oa.shape[:-1] + (d_v,))
        self._call("dsao_mla_output_projection", _ptr(oa), od, _ptr(va), vd, M, H, d_c, d_v, _ptr(out), threads())
        return out

    def linear(self, x, W) -> np.ndarray:
        """y = x W^T with W [N, K] (out, in): the indexer's query projection wq_b and its head-weight
        projection (DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)")."""
        xa, xd = _fp(x)
        wa, wd = _fp(W)
        N, K = wa.shape
        M = xa.size // K
        out = np.empty(xa.shape[:-1] + (N,))
        self._call("dsao_linear", _ptr(xa), xd, _ptr(wa), wd, M, N, K, _ptr(out), threads())
        return out

    # ----------------------------------------------------------- FP8 indexer

    def fwht_f32(self, x) -> np.ndarray:
        """Unnormalised Walsh-Hadamard transform of the last axis (a power of two), in float32."""
        y = np.array(x, dtype=np.float32, copy=True, order="C")
        n = y.shape[-1]
        self._call("dsao_fwht_f32", _ptr(y), y.size // n, n)
        return y

    def e4m3_decode(self, codes) -> np.ndarray:
        """OCP E4M3 codes -> float64 (bias 7, subnormals M * 2^-9, S.1111.111 is NaN)."""
        c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
        out = np.empty(c.shape)
        self._call("dsao_e4m3_decode", _ptr(c), c.size, _ptr(out))
        return out

    def e4m3_encode_rne(self, v) -> np.ndarray:
        """float32 values with |v| <= 448 -> OCP E4M3 codes, rounded to nearest, ties to even."""
        a = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
        out = np.empty(a.shape, dtype=np.uint8)
        if self.lib.dsao_e4m3_encode_rne(_ptr(a), a.size, _ptr(out)) != 0:
            raise ValueError("e4m3_encode_rne: |v| must be <= 448")
        return out

    def pow2_scale_exp(self, amax: float) -> int:
        """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0)."""
        return int(self.lib.dsao_pow2_scale_exp(float(amax)))

    def quantize_fp8_rows(self, x):
        """Rows of the last axis -> (codes uint8 [..., D], scales float32 [...]): rotate, scale, round."""
        a, dt = _fp(x)
        D = a.shape[-1]
        codes = np.empty(a.shape, dtype=np.uint8)
        scales = np.empty(a.shape[:-1], dtype=np.float32)
        self._call("dsao_quantize_fp8_rows", _ptr(a), dt, a.size // D, D, _ptr(codes), _ptr(scales))
        return codes, scales

    def index_scores_fp8_rows(self, q8_b, qs_b, k8_b, ks_b, w_b, ts, q_pos0: int) -> list:
        """FP8 scores of queries `ts` of one sequence: q8_b [Tq,H_I,D], qs_b [Tq,H_I], k8_b [N,D], ks_b [N],
        w_b [Tq,H_I]; I[s] = sum_h w_h ReLU(qs_h ks_s / D sum_d dec(q8) dec(k8))."""
        q8 = np.ascontiguousarray(np.asarray(q8_b, dtype=np.uint8))
        qs = np.ascontiguousarray(np.asarray(qs_b, dtype=np.float32))
        k8 = np.ascontiguousarray(np.asarray(k8_b, dtype=np.uint8))
        ks = np.ascontiguousarray(np.asarray(ks_b, dtype=np.float32))
        wa, wd = _fp(w_b)
        Tq, H_I, D = q8.shape
        N = k8.shape[0]
        ts = [int(t) for t in ts]
        r, n = _row_list([(0, t) for t in ts])
        out = np.full((n, N), np.nan)
        self._call("dsao_index_scores_fp8", _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(wa), wd, 1, Tq, N, H_I, D,
                   _ptr(_pos0(q_pos0, 1)), _ptr(r), n, _ptr(out), threads())
        return [out[i, :self.n_valid_keys(t, q_pos0, N)].copy() for i, t in enumerate(ts)]

    # ----------------------------------------------------------- test helper

    def sylvester_hadamard(self, n: int) -> np.ndarray:
        """H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]; H H^T = n I (n a power of two)."""
        out = np.empty((int(n), int(n)))
        self._call("dsao_sylvester_hadamard", int(n), _ptr(out))
        return out


_default = None


def default() -> Oracle:
    """The oracle built from dsa_oracle.cpp (compiled on first use if missing).  DSA_ORACLE_LIB names
    another build of the same source to load instead (the sanitizer build the tests make)."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("DSA_ORACLE_LIB") or build_library())
    return _default


def _forward(name):
    def fn(*a, **k):
        return getattr(default(), name)(*a, **k)
    fn.__name__ = name
    fn.__doc__ = getattr(Oracle, name).__doc__
    return fn


for _name in __all__:
    if _name not in ("Oracle", "build_library", "threads"):
        globals()[_name] = _forward(_name)
del _name
