"""CPU oracle for the DeepSeek Sparse Attention (DSA) forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the CPU-baseline leg of the benchmark may import this module; the product
path (the HIP library and its Python binding) never does, and this module
never imports the product path.  The two share no code: the only thing both
sides consume is the seeded input generator in ``synth/``.

Plain numpy in float64, written from the method's definition so that a
reader can check it against the pages by eye:

  DeepSeek-V3.2 model documentation, section "DeepSeek Sparse Attention
  (DSA)":
    * the lightning indexer: a light scorer with few heads computes an index
      score between every query and all keys before it (the paragraph on the
      lightning indexer); the scores are the same whether computed in FP8
      after an orthogonal Hadamard rotation or directly in bf16/fp32;
    * the indexer keeps its own per-token key cache with a single head of
      width index_head_dim (the paragraph on the indexer cache);
    * fine-grained token selection: each query keeps the index_topk most
      relevant tokens and the main MLA attention runs over those tokens only,
      through an additive mask (the paragraph on token selection);
    * every layer runs its own indexer.
  DeepSeek-V3.2 model documentation, section "DeepseekV32Config": the shape
  defaults index_n_heads = 64, index_head_dim = 128, index_topk = 2048,
  kv_lora_rank = 512, qk_rope_head_dim = 64, qk_nope_head_dim = 128,
  num_attention_heads = 128.
  DeepSeek-V4 model documentation, section on the attention mask layout: an
  indexer entry of -1 means "no selection" and reaches the mask unchanged;
  a compressed entry w (positions m*w .. m*w + m - 1) becomes visible to the
  query at position p once its window has closed, w < (p + 1) // m, so
  queries before the first window closes (p < m - 1) select nothing.

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * score formula  I[t,s] = sum_h w[t,h] * ReLU(sum_d qI[t,h,d] * kI[s,d]),
    no extra scale (any scale is part of w);
  * "keys before the query" includes the query's own position: query t at
    absolute position p = q_pos0 + t sees keys s <= p (and s < N);
  * top-k ties go to the lower key index; the selection is emitted in
    ascending key order, then padded with -1 when fewer than K keys exist;
  * the MLA runs in absorbed latent form: each head's D-wide query meets one
    D-wide latent row shared by all heads; the value is the row's first DV
    entries; logits are scale * q.kv; negative indices are masked (additive
    -inf); a row with no valid index gives o = 0 and lse = -inf;
  * lse is the natural-log sum of exp(logits);
  * absorbed and naive MLA: head h's key up-projection W_UK[h] [d_nope, d_c]
    folds into its query (mla_absorb_query) and its value up-projection
    W_UV[h] [d_v, d_c] applies to the latent output (mla_output_projection);
    mla_naive_rows is the per-head form with explicit keys and values.

Every function works on float64 copies of its inputs.  bf16 inputs arrive as
uint16 bit patterns and are widened exactly by ``as_f64``.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "as_f64", "bf16_bits_to_f64", "n_valid_keys", "paged_gather", "index_scores", "index_scores_rows",
    "topk_row", "topk", "sparse_mla", "sparse_mla_rows", "dense_masked_mla", "forward_rows",
    "mla_naive_rows", "mla_absorb_query", "mla_output_projection", "linear", "fwht_f32", "e4m3_decode",
    "e4m3_encode_rne", "pow2_scale_exp", "quantize_fp8_rows", "index_scores_fp8_rows", "sylvester_hadamard",
]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: a bf16 is the top half of an fp32."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def n_valid_keys(t: int, q_pos0: int, N: int, m: int = 1) -> int:
    """Number of keys query t may see: positions 0..q_pos0+t, capped by the cache length.

    With a key axis compressed at rate m (entry w summarises positions
    m*w .. m*w+m-1), entry w is visible once its window has closed:
    w < (q_pos0 + t + 1) // m.  m = 1 is the plain causal rule.
    """
    p1 = q_pos0 + t + 1
    return 0 if p1 <= 0 else min(N, p1 // m)


def paged_gather(pool: np.ndarray, table_row, block_size: int, n_rows: int) -> np.ndarray:
    """Rows 0..n_rows-1 of one sequence of a paged cache as a contiguous array.

    A paged cache layer keeps its rows in a pool of blocks of block_size rows
    and one block table per sequence (reading of the cache layers named in
    the DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)"):
    logical row r is pool row table_row[r // block_size] * block_size +
    r % block_size.
    """
    table_row = np.asarray(table_row, dtype=np.int64)
    r = np.arange(n_rows)
    return np.asarray(pool)[table_row[r // block_size] * block_size + r % block_size]


# ----------------------------------------------------------------------------
# Lightning indexer
# ----------------------------------------------------------------------------

def index_scores_rows(q_idx_b: np.ndarray, k_idx_b: np.ndarray, w_b: np.ndarray,
                      ts, q_pos0: int, m: int = 1) -> list:
    """Index scores of queries `ts` of one sequence against their visible keys.

    q_idx_b [Tq, H_I, D_I], k_idx_b [N, D_I], w_b [Tq, H_I] (any storage dtype).
    Returns one float64 vector per query t, of length n_valid_keys(t, q_pos0, N, m):
        I[s] = sum_h w[t,h] * max(0, sum_d qI[t,h,d] * kI[s,d]).
    """
    kI = as_f64(k_idx_b)
    N = kI.shape[0]
    out = []
    for t in ts:
        n = n_valid_keys(int(t), q_pos0, N, m)
        qI = as_f64(q_idx_b[t])            # [H_I, D_I]
        w = as_f64(w_b[t])                 # [H_I]
        dots = kI[:n] @ qI.T               # [n, H_I]: per-head dot product q_h . k_s
        out.append(np.maximum(dots, 0.0) @ w)
    return out


def index_scores(q_idx: np.ndarray, k_idx: np.ndarray, w: np.ndarray, q_pos0: int, m: int = 1) -> np.ndarray:
    """Full score tensor [B, Tq, N] (float64); entries a query may not see are NaN."""
    B, Tq = q_idx.shape[:2]
    N = k_idx.shape[1]
    out = np.full((B, Tq, N), np.nan)
    for b in range(B):
        rows = index_scores_rows(q_idx[b], k_idx[b], w[b], range(Tq), q_pos0, m)
        for t, r in enumerate(rows):
            out[b, t, :len(r)] = r
    return out


# ----------------------------------------------------------------------------
# Top-k selection
# ----------------------------------------------------------------------------

def topk_row(scores: np.ndarray, K: int) -> np.ndarray:
    """Keep the K highest-scoring of the n = len(scores) visible keys.

    The decision is taken on float32 scores (the precision the GPU path stores
    them in).  Order: score descending, then key index ascending, so equal
    scores go to the lower index.  The kept indices are returned in ascending
    order; if n <= K every key is kept and the row is padded with -1.
    """
    v = np.asarray(scores, dtype=np.float32)
    n = v.shape[0]
    out = np.full(K, -1, dtype=np.int32)
    if n <= K:
        out[:n] = np.arange(n, dtype=np.int32)
        return out
    keys = np.arange(n)
    # np.lexsort sorts by the last key first: primary -v (i.e. v descending), secondary index
    order = np.lexsort((keys, -v.astype(np.float64)))
    out[:] = np.sort(order[:K]).astype(np.int32)
    return out


def topk(scores: np.ndarray, K: int, q_pos0: int, m: int = 1) -> np.ndarray:
    """scores [B, Tq, N] -> idx [B, Tq, K] int32 (row t uses its visible keys only)."""
    B, Tq, N = scores.shape
    out = np.empty((B, Tq, K), dtype=np.int32)
    for b in range(B):
        for t in range(Tq):
            n = n_valid_keys(t, q_pos0, N, m)
            out[b, t] = topk_row(scores[b, t, :n], K)
    return out


# ----------------------------------------------------------------------------
# Sparse MLA (absorbed latent form)
# ----------------------------------------------------------------------------

def _softmax_attend(logits: np.ndarray, values: np.ndarray):
    """Softmax over the last axis of logits [H, n] then weight values [n, DV].

    Returns (o [H, DV], lse [H]).  n == 0 gives o = 0 and lse = -inf.
    """
    H = logits.shape[0]
    if logits.shape[1] == 0:
        return np.zeros((H, values.shape[1])), np.full(H, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ values) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def sparse_mla_rows(q_bt: np.ndarray, kv_rows: np.ndarray, idx_row: np.ndarray, scale: float, DV: int):
    """One query: q_bt [H, D]; kv_rows maps a key index to its D-wide latent row.

    kv_rows is either the whole cache [N, D] or a dict {index: row}.  Entries of
    idx_row below zero are masked out.  Returns (o [H, DV], lse [H]) in float64.
    """
    sel = [int(i) for i in np.asarray(idx_row).reshape(-1) if int(i) >= 0]
    if isinstance(kv_rows, dict):
        rows = np.stack([as_f64(kv_rows[i]) for i in sel]) if sel else np.zeros((0, q_bt.shape[-1]))
    else:
        rows = as_f64(kv_rows[sel]) if sel else np.zeros((0, q_bt.shape[-1]))
    q = as_f64(q_bt)
    logits = scale * (q @ rows.T)             # [H, n]
    return _softmax_attend(logits, rows[:, :DV])


def sparse_mla(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, scale: float, DV: int):
    """q [B,Tq,H,D], kv [B,N,D], idx [B,Tq,K] -> (o [B,Tq,H,DV], lse [B,Tq,H]) float64."""
    B, Tq, H, _ = q.shape
    o = np.empty((B, Tq, H, DV))
    lse = np.empty((B, Tq, H))
    for b in range(B):
        kvb = as_f64(kv[b])
        for t in range(Tq):
            o[b, t], lse[b, t] = sparse_mla_rows(q[b, t], kvb, idx[b, t], scale, DV)
    return o, lse


def dense_masked_mla(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, scale: float, DV: int,
                     q_pos0: int):
    """The same attention written as dense causal attention plus an additive mask.

    For query t, every visible key s (s <= q_pos0 + t, s < N) gets the logit
    scale * q.kv[s] plus a mask term that is 0 when s is among the selected
    indices and -inf otherwise; the softmax then runs over all visible keys.
    """
    B, Tq, H, _ = q.shape
    N = kv.shape[1]
    o = np.empty((B, Tq, H, DV))
    lse = np.empty((B, Tq, H))
    for b in range(B):
        kvb = as_f64(kv[b])
        for t in range(Tq):
            n = n_valid_keys(t, q_pos0, N)
            mask = np.full(n, -np.inf)
            for i in np.asarray(idx[b, t]).reshape(-1):
                if 0 <= int(i) < n:
                    mask[int(i)] = 0.0
            logits = scale * (as_f64(q[b, t]) @ kvb[:n].T) + mask[None, :]
            keep = np.isfinite(mask)
            if not keep.any():
                o[b, t], lse[b, t] = 0.0, -np.inf
                continue
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)                # exp(-inf) = 0 for masked keys
            l = p.sum(axis=1, keepdims=True)
            o[b, t] = (p @ kvb[:n, :DV]) / l
            lse[b, t] = (m + np.log(l))[:, 0]
    return o, lse


# ----------------------------------------------------------------------------
# MLA projections around the absorbed form, and the naive per-head form
# ----------------------------------------------------------------------------
#
# DeepSeek-V3 documentation, "DeepseekV3Config": keys and values come from a
# kv_lora_rank-wide latent through low-rank (LoRA) projections; each head has
# a qk_nope_head_dim part without rotary embedding, a qk_rope_head_dim part
# with it, and a v_head_dim-wide value.  Its section on limitations notes
# that the port computes attention the "naive" way (per-head keys and values,
# not strictly MLA).  Reading: the key up-projection of head h is a matrix
# W_UK[h] [d_nope, d_c] and the value up-projection W_UV[h] [d_v, d_c], both
# applied to the latent c; the rope part of the key is one d_rope vector per
# token shared by all heads.  One latent cache row is [c (d_c) | k_rope
# (d_rope)].

def mla_naive_rows(q_head: np.ndarray, c_kv: np.ndarray, k_rope: np.ndarray, idx_row: np.ndarray,
                   W_UK: np.ndarray, W_UV: np.ndarray, scale: float):
    """Naive MLA for one query over its selected tokens, head by head.

    q_head [H, d_nope + d_rope]; c_kv [N, d_c]; k_rope [N, d_rope];
    W_UK [H, d_nope, d_c]; W_UV [H, d_v, d_c].  Head h builds explicit keys
    k_j = [W_UK[h] c_j, k_rope_j] and values v_j = W_UV[h] c_j for the selected
    tokens j (indices < 0 are masked), then runs softmax(scale * q.k) v.
    Returns (o [H, d_v], lse [H]).
    """
    q_head, c_kv, k_rope = as_f64(q_head), as_f64(c_kv), as_f64(k_rope)
    W_UK, W_UV = as_f64(W_UK), as_f64(W_UV)
    H = q_head.shape[0]
    sel = [int(i) for i in np.asarray(idx_row).reshape(-1) if int(i) >= 0]
    o = np.zeros((H, W_UV.shape[1]))
    lse = np.full(H, -np.inf)
    for h in range(H):
        keys = np.concatenate([c_kv[sel] @ W_UK[h].T, k_rope[sel]], axis=1)   # [n, d_nope + d_rope]
        values = c_kv[sel] @ W_UV[h].T                                         # [n, d_v]
        oh, lh = _softmax_attend(scale * (q_head[h][None, :] @ keys.T), values)
        o[h], lse[h] = oh[0], lh[0]
    return o, lse


def mla_absorb_query(q_head: np.ndarray, W_UK: np.ndarray) -> np.ndarray:
    """Fold the key up-projection into the query: [..., H, d_nope + d_rope] -> [..., H, d_c + d_rope].

    q_lat[h] = [W_UK[h]^T q_nope[h], q_rope[h]], so that q_lat[h] . [c | k_rope]
    equals the naive head's q[h] . [W_UK[h] c | k_rope].
    """
    q_head, W_UK = as_f64(q_head), as_f64(W_UK)
    d_nope = W_UK.shape[1]
    q_nope, q_rope = q_head[..., :d_nope], q_head[..., d_nope:]
    q_c = np.einsum("...hn,hnc->...hc", q_nope, W_UK)
    return np.concatenate([q_c, q_rope], axis=-1)


def mla_output_projection(o_lat: np.ndarray, W_UV: np.ndarray) -> np.ndarray:
    """Apply the value up-projection to the latent output: [..., H, d_c] -> [..., H, d_v], o[h] = W_UV[h] o_lat[h]."""
    return np.einsum("...hc,hvc->...hv", as_f64(o_lat), as_f64(W_UV))


def linear(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """A linear layer without bias, y = x W^T with W [N, K] (out, in): the
    indexer's query projection wq_b from the low-rank query latent (DeepSeek-V3.2
    documentation, "DeepSeek Sparse Attention (DSA)", note on the query LoRA
    path) and its per-head weight projection."""
    return as_f64(x) @ as_f64(W).T


# ----------------------------------------------------------------------------
# Composition: indexer -> top-k -> sparse MLA, for chosen query rows
# ----------------------------------------------------------------------------

def forward_rows(q_idx_b, k_idx_b, w_b, q_b, kv_b, ts, q_pos0: int, K: int, scale: float, DV: int):
    """The three steps for queries `ts` of one sequence.

    kv_b is the latent cache [N, D] of the sequence, or a callable that maps an
    array of row indices to those rows (for caches too large to widen whole).
    Returns a list of dicts with the query's float64 scores, its int32
    indices, and its (o, lse).
    """
    res = []
    scores = index_scores_rows(q_idx_b, k_idx_b, w_b, ts, q_pos0)
    for t, s in zip(ts, scores):
        idx = topk_row(s.astype(np.float32), K)
        sel = idx[idx >= 0]
        if callable(kv_b):
            rows = {int(i): r for i, r in zip(sel, kv_b(sel))}
        else:
            rows = kv_b
        o, lse = sparse_mla_rows(q_b[t], rows, idx, scale, DV)
        res.append({"t": int(t), "scores": s, "idx": idx, "o": o, "lse": lse})
    return res


# ----------------------------------------------------------------------------
# FP8 indexer: Hadamard rotation, e4m3 rows with power-of-two scales, scores
# ----------------------------------------------------------------------------
#
# DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)": the
# reference implementation runs the indexer in FP8 after a Hadamard rotation
# of queries and keys; the rotation is orthogonal (Hq . Hk = q . k) and FP8 is
# only a precision optimisation.  Readings (the pages give no format details):
#   * FP8 is OCP E4M3 (bias 7, largest finite 448, no infinities);
#   * the rotation is the unnormalised Sylvester matrix H (entries +-1, so
#     H H^T = D I), applied by the fast Walsh-Hadamard transform in float32
#     with pair distance 1, 2, 4, ... (a + b on the lower, a - b on the upper
#     element); the factor D is taken out of the score;
#   * each rotated row of D values (one key, or one head of one query) has
#     one scale 2^e, the smallest power of two with max|y| <= 448 * 2^e
#     (e = 0 for an all-zero row), and codes e4m3_rne(y / 2^e);
#   * the score is I[t,s] = sum_h w[t,h] * max(0, qs[t,h] * ks[s] / D *
#     sum_d dec(q8[t,h,d]) * dec(k8[s,d])), which is the bf16 score when
#     quantisation is exact.

def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of the last axis (a power of two), in float32."""
    y = np.array(x, dtype=np.float32)
    n = y.shape[-1]
    d = 1
    while d < n:
        blocks = y.reshape(y.shape[:-1] + (n // (2 * d), 2, d))
        a, b = blocks[..., 0, :], blocks[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(y.shape)
        d *= 2
    return y


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes -> float64 (S.EEEE.MMM, bias 7, subnormals M * 2^-9, S.1111.111 is NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 15
    M = (c & 7).astype(np.float64)
    mag = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode_rne(v: np.ndarray) -> np.ndarray:
    """float32 values with |v| <= 448 -> OCP E4M3 codes, rounded to nearest, ties to even."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)   # exact widening
    if np.any(np.abs(v) > 448.0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode_rne: |v| must be <= 448")
    a = np.abs(v)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: a multiple of 2^-9 (a code of 8 is the smallest normal, 0x08)
    out[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        e = np.floor(np.log2(a[nrm])).astype(np.int64)
        # log2 of a float can land one off at exact powers of two: fix up
        e = np.where(np.exp2(e.astype(np.float64)) > a[nrm], e - 1, e)
        e = np.where(np.exp2((e + 1).astype(np.float64)) <= a[nrm], e + 1, e)
        q = np.rint((a[nrm] / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
        e = np.where(q == 8, e + 1, e)
        q = np.where(q == 8, 0, q)
        out[nrm] = ((e + 7) << 3) | q
    out = np.where(np.signbit(v), out | 0x80, out)
    return out.astype(np.uint8)


def pow2_scale_exp(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    m, E = math.frexp(amax)          # amax = m * 2^E, 0.5 <= m < 1; 448 = 0.875 * 2^9
    return E - 9 if m <= 0.875 else E - 8


def quantize_fp8_rows(x: np.ndarray):
    """Rows of the last axis -> (codes uint8 [..., D], scales float32 [...]): rotate, scale, round."""
    y = fwht_f32(as_f64(x).astype(np.float32))
    amax = np.max(np.abs(y), axis=-1)
    flat_e = np.array([pow2_scale_exp(a) for a in amax.reshape(-1)], dtype=np.int64)
    e = flat_e.reshape(amax.shape)
    v = (y.astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None]).astype(np.float32)  # exact
    return e4m3_encode_rne(v), np.exp2(e.astype(np.float64)).astype(np.float32)


def index_scores_fp8_rows(q8_b, qs_b, k8_b, ks_b, w_b, ts, q_pos0: int) -> list:
    """FP8 index scores of queries `ts` of one sequence (float64 from the codes).

    q8_b [Tq, H_I, D] codes, qs_b [Tq, H_I] scales, k8_b [N, D] codes, ks_b [N]
    scales, w_b [Tq, H_I] head weights.  Query t sees keys s < n_valid_keys(t).
    """
    k = e4m3_decode(k8_b)
    ks = np.asarray(ks_b, dtype=np.float64)
    N, D = k.shape
    out = []
    for t in ts:
        n = n_valid_keys(int(t), q_pos0, N)
        q = e4m3_decode(q8_b[t])                                   # [H_I, D]
        qs = np.asarray(qs_b[t], dtype=np.float64)
        w = as_f64(w_b[t])
        dots = (k[:n] @ q.T) * ks[:n, None] * qs[None, :] / D      # [n, H_I]
        out.append(np.maximum(dots, 0.0) @ w)
    return out


# ----------------------------------------------------------------------------
# Test helper: the Sylvester Hadamard matrix (textbook construction)
# ----------------------------------------------------------------------------

def sylvester_hadamard(n: int) -> np.ndarray:
    """H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]; H H^T = n I (n a power of two)."""
    assert n >= 1 and (n & (n - 1)) == 0
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h
