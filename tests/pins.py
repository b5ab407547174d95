"""Pins for the CPU oracle: facts fixed by the pages or by mathematics.

Each check takes the oracle function it exercises as an argument and returns
True when the fact holds, so the same checks can be run on the real oracle
(they must all hold) and on deliberately broken copies of it (at least one
must fail), which shows that a plausible mistake cannot slip through.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- indexer ---

def pin_indexer_golden(index_scores_rows) -> bool:
    """Hand-derived 3-query example (derivation stored with the fixture)."""
    g = load_golden("indexer_topk_tiny.json")
    q = np.array(g["q_idx"], dtype=np.float64)
    k = np.array(g["k_idx"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    rows = index_scores_rows(q, k, w, range(q.shape[0]), g["q_pos0"])
    return all(len(r) == len(e) and np.array_equal(r, np.array(e, dtype=np.float64))
               for r, e in zip(rows, g["scores"]))


def pin_indexer_hadamard(index_scores_rows, hadamard) -> bool:
    """Hq.Hk = n q.k for the unnormalised Sylvester matrix (H H^T = n I); ReLU is
    positively homogeneous, so rotated scores are exactly n times the plain ones."""
    r = _rng(11)
    T, HI, DI = 9, 4, 32
    q = r.integers(-3, 4, size=(T, HI, DI)).astype(np.float64)
    k = r.integers(-3, 4, size=(T, DI)).astype(np.float64)
    w = r.choice([0.25, 0.5, 1.0, 2.0], size=(T, HI))
    h = hadamard(DI)
    if not np.array_equal(h @ h.T, DI * np.eye(DI)):
        return False
    a = index_scores_rows(q, k, w, range(T), 0)
    b = index_scores_rows(q @ h.T, k @ h.T, w, range(T), 0)
    return all(np.array_equal(DI * x, y) for x, y in zip(a, b))


def pin_indexer_unit_queries(index_scores_rows) -> bool:
    """Each head's query is a signed unit vector c_h * e_{i_h}: its dot product
    with key s is c_h * k[s, i_h], read off by indexing."""
    r = _rng(12)
    T, HI, DI, N = 6, 5, 8, 6
    k = r.integers(-4, 5, size=(N, DI)).astype(np.float64)
    w = r.choice([-1.0, 0.5, 2.0], size=(T, HI))
    pos = r.integers(0, DI, size=(T, HI))
    sgn = r.choice([-1.0, 1.0, 3.0], size=(T, HI))
    q = np.zeros((T, HI, DI))
    for t in range(T):
        for h in range(HI):
            q[t, h, pos[t, h]] = sgn[t, h]
    got = index_scores_rows(q, k, w, range(T), 0)
    for t in range(T):
        exp = np.zeros(t + 1)
        for s in range(t + 1):
            for h in range(HI):
                exp[s] += w[t, h] * max(0.0, sgn[t, h] * k[s, pos[t, h]])
        if not np.array_equal(got[t], exp):
            return False
    return True


def pin_indexer_causal(index_scores_rows) -> bool:
    """Query t at position q_pos0+t sees keys 0..q_pos0+t only (own key included):
    row lengths are fixed, and keys after the query cannot change its row."""
    r = _rng(13)
    T, HI, DI, N, p0 = 7, 3, 4, 12, 3
    q = r.integers(-3, 4, size=(T, HI, DI)).astype(np.float64)
    k = r.integers(-3, 4, size=(N, DI)).astype(np.float64)
    w = np.ones((T, HI))
    a = index_scores_rows(q, k, w, range(T), p0)
    if [len(x) for x in a] != [min(N, p0 + t + 1) for t in range(T)]:
        return False
    for t in range(T):
        k2 = k.copy()
        k2[p0 + t + 1:] = r.integers(-3, 4, size=k2[p0 + t + 1:].shape)
        if not np.array_equal(index_scores_rows(q, k2, w, [t], p0)[0], a[t]):
            return False
        # the own key does matter: flip it to a key that surely scores differently
        k3 = k.copy()
        k3[p0 + t] = q[t, 0] * 7.0 + 1.0
        if np.array_equal(index_scores_rows(q, k3, w, [t], p0)[0], a[t]):
            return False
    return True


def pin_indexer_heads(index_scores_rows) -> bool:
    """Heads are summed with their own weights: permuting heads together with
    their weights changes nothing, and the score is linear in the weights."""
    r = _rng(14)
    T, HI, DI = 5, 6, 8
    q = r.integers(-3, 4, size=(T, HI, DI)).astype(np.float64)
    k = r.integers(-3, 4, size=(T, DI)).astype(np.float64)
    w1 = r.choice([0.25, 0.5, 1.0, 2.0, -1.0], size=(T, HI))
    w2 = r.choice([0.25, 0.5, 1.0, 2.0], size=(T, HI))
    perm = r.permutation(HI)
    a = index_scores_rows(q, k, w1, range(T), 0)
    b = index_scores_rows(q[:, perm], k, w1[:, perm], range(T), 0)
    c = index_scores_rows(q, k, w2, range(T), 0)
    d = index_scores_rows(q, k, w1 + w2, range(T), 0)
    # a single head with weight one is ReLU of the dot product: all-negative dots give 0
    e = index_scores_rows(-np.abs(q[:, :1]) - 1, np.abs(k) , np.ones((T, 1)), range(T), 0)
    return (all(np.array_equal(x, y) for x, y in zip(a, b))
            and all(np.array_equal(x + y, z) for x, y, z in zip(a, c, d))
            and all(not np.any(x) for x in e))


def windows_closed(t, q_pos0, N, m):
    """Independent count: entry w of a key axis compressed at rate m summarises
    positions m*w .. m*w+m-1 and is visible to the query at position q_pos0+t
    once the last of them has arrived.  Counted entry by entry."""
    pos = q_pos0 + t
    return sum(1 for w in range(N) if m * w + m - 1 <= pos)


def pin_compressed_visibility(n_valid_keys) -> bool:
    """The visible-entry count follows the worked 16-token example and, on a
    grid of positions, rates and cache lengths, the closed-window count."""
    g = load_golden("compressed_visibility.json")
    hca = g["hca"]
    if [n_valid_keys(t, 0, g["tokens"], hca["m"]) for t in range(g["tokens"])] != hca["visible_entries_per_t"]:
        return False
    csa = g["csa"]
    for t in range(g["tokens"]):
        if (n_valid_keys(t, 0, g["tokens"], csa["m"]) == 0) != (t < csa["empty_rows_below_t"]):
            return False
    for m in (1, 2, 3, 4, 8, 128):
        for N in (0, 1, 5, 40):
            for p0 in (-3, 0, 5, 33):
                for t in range(12):
                    if n_valid_keys(t, p0, N, m) != windows_closed(t, p0, N, m):
                        return False
    return True


def pin_compressed_pipeline(index_scores, topk) -> bool:
    """Indexer and top-k over a compressed axis on the worked example: rows of
    queries whose first window is still open are all -1, and a row's scores are
    the prefix of the uncompressed row (compression only hides entries)."""
    g = load_golden("compressed_visibility.json")
    r = _rng(15)
    T, HI, DI, m, K = g["tokens"], 2, 4, g["csa"]["m"], g["csa"]["K"]
    nent = T // m
    q = r.integers(-3, 4, size=(1, T, HI, DI)).astype(np.float64)
    k = r.integers(-3, 4, size=(1, nent, DI)).astype(np.float64)
    w = r.choice([0.5, 1.0, 2.0], size=(1, T, HI))
    sc = index_scores(q, k, w, 0, m)
    sc1 = index_scores(q, k, w, 0, 1)
    idx = topk(np.nan_to_num(sc, nan=-np.inf).astype(np.float32), K, 0, m)
    for t in range(T):
        n = windows_closed(t, 0, nent, m)
        if not np.array_equal(sc[0, t, :n], sc1[0, t, :n]) or not np.all(np.isnan(sc[0, t, n:])):
            return False
        row = idx[0, t]
        if t < g["csa"]["empty_rows_below_t"] and not np.all(row == -1):
            return False
        kept = row[row >= 0]
        if len(kept) != min(n, K) or (len(kept) and kept.max() >= n):
            return False
    return True


# ------------------------------------------------------------------ top-k ---

def rank_count_topk(v, K):
    """Independent definition: key s is kept iff fewer than K keys precede it in
    the order (score desc, index asc); the result is listed in ascending order."""
    v = np.asarray(v, dtype=np.float32)
    n = len(v)
    keep = []
    for s in range(n):
        rank = sum(1 for s2 in range(n) if v[s2] > v[s] or (v[s2] == v[s] and s2 < s))
        if rank < K:
            keep.append(s)
    out = np.full(K, -1, dtype=np.int32)
    out[:len(keep)] = keep
    return out


def pin_topk_golden(topk_row) -> bool:
    g = load_golden("topk_ties.json")
    for c in g["cases"]:
        v = np.array([float(x) for x in c["scores"]], dtype=np.float32)
        if not np.array_equal(topk_row(v, c["K"]), np.array(c["idx"], dtype=np.int32)):
            return False
    g2 = load_golden("indexer_topk_tiny.json")
    for s, e in zip(g2["scores"], g2["idx"]):
        if not np.array_equal(topk_row(np.array(s, dtype=np.float32), g2["K"]), np.array(e)):
            return False
    return True


def pin_topk_bruteforce(topk_row) -> bool:
    """Agreement with the rank-count definition on many tiny rows with heavy ties."""
    r = _rng(21)
    for trial in range(300):
        n = int(r.integers(1, 40))
        K = int(r.integers(1, 45))
        if trial % 3 == 0:
            v = r.integers(0, 3, size=n).astype(np.float32)
        elif trial % 3 == 1:
            v = r.choice(np.array([-0.0, 0.0, -1.5, 2.0], dtype=np.float32), size=n)
        else:
            v = r.standard_normal(n).astype(np.float32)
        if not np.array_equal(topk_row(v, K), rank_count_topk(v, K)):
            return False
    return True


def pin_topk_short_rows(topk_row) -> bool:
    """A row with n <= K visible keys is exactly [0, 1, ..., n-1, -1, ...]."""
    r = _rng(22)
    for n in range(0, 20):
        K = 20
        got = topk_row(r.standard_normal(n).astype(np.float32), K)
        exp = np.array(list(range(n)) + [-1] * (K - n), dtype=np.int32)
        if not np.array_equal(got, exp):
            return False
    return True


# ------------------------------------------------------------- sparse MLA ---

def pin_mla_golden(sparse_mla_rows) -> bool:
    g = load_golden("sparse_mla_tiny.json")
    o, lse = sparse_mla_rows(np.array(g["q"]), np.array(g["kv"]), np.array(g["idx"]),
                             g["scale"], g["DV"])
    return (np.allclose(o, np.array(g["o"]), rtol=0, atol=1e-12)
            and np.allclose(lse, np.array(g["lse"]), rtol=0, atol=1e-12))


def pin_mla_single_key(sparse_mla_rows) -> bool:
    """One valid index: the output is that row's value part exactly, and the
    log-sum-exp is the single logit scale*q.kv."""
    r = _rng(31)
    H, D, DV, N = 3, 10, 6, 9
    q = r.standard_normal((H, D))
    kv = r.standard_normal((N, D))
    for j in range(N):
        idx = np.array([-1, j, -1, -1])
        o, lse = sparse_mla_rows(q, kv, idx, 0.3, DV)
        if not (np.array_equal(o, np.broadcast_to(kv[j, :DV], (H, DV)))
                and np.allclose(lse, 0.3 * (q @ kv[j]), rtol=1e-15, atol=1e-15)):
            return False
    return True


def pin_mla_uniform(sparse_mla_rows) -> bool:
    """q = 0 makes every logit 0: the output is the mean of the selected value rows
    and lse = ln(number selected)."""
    r = _rng(32)
    H, D, DV, N = 2, 7, 4, 20
    kv = r.standard_normal((N, D))
    idx = np.array([3, 17, -1, 5, 0, 11])
    sel = idx[idx >= 0]
    o, lse = sparse_mla_rows(np.zeros((H, D)), kv, idx, 1.7, DV)
    return (np.allclose(o, np.broadcast_to(kv[sel, :DV].mean(axis=0), (H, DV)), atol=1e-14)
            and np.allclose(lse, math.log(len(sel)), atol=1e-14))


def pin_mla_permutation_and_mask(sparse_mla_rows) -> bool:
    """The selection is a set: shuffling it or sprinkling -1 entries into it leaves
    the output unchanged up to rounding; an all-masked row gives o = 0, lse = -inf."""
    r = _rng(33)
    H, D, DV, N = 4, 12, 8, 50
    q = r.standard_normal((H, D))
    kv = r.standard_normal((N, D))
    idx = r.choice(N, size=10, replace=False)
    o1, l1 = sparse_mla_rows(q, kv, idx, 0.4, DV)
    idx2 = np.concatenate([r.permutation(idx), [-1, -1, -7]])
    idx2 = idx2[r.permutation(len(idx2))]
    o2, l2 = sparse_mla_rows(q, kv, idx2, 0.4, DV)
    o3, l3 = sparse_mla_rows(q, kv, np.array([-1, -1]), 0.4, DV)
    return (np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)
            and not np.any(o3) and np.all(np.isneginf(l3)))


def pin_mla_sdpa(sparse_mla, dense_masked_mla) -> bool:
    """With every visible key selected (K >= L), sparse attention is plain causal
    attention: compare against torch's scaled_dot_product_attention on the CPU in
    float64 (a library routine, with the latent row as key and its first DV
    entries as value).  The dense additive-mask form must agree as well."""
    import torch
    r = _rng(34)
    B, L, H, D, DV = 2, 13, 3, 10, 6
    q = r.standard_normal((B, L, H, D))
    kv = r.standard_normal((B, L, D))
    idx = np.full((B, L, L), -1, dtype=np.int32)
    for t in range(L):
        idx[:, t, :t + 1] = r.permutation(t + 1)
    scale = 0.37
    o, lse = sparse_mla(q, kv, idx, scale, DV)
    od, lsed = dense_masked_mla(q, kv, idx, scale, DV, 0)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)                   # [B,H,L,D]
    tk = torch.from_numpy(kv)[:, None].expand(B, H, L, D)
    tv = torch.from_numpy(kv[..., :DV])[:, None].expand(B, H, L, DV)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    logits = torch.einsum("bhld,bhsd->bhls", tq, tk) * scale
    causal = torch.ones(L, L, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(logits.masked_fill(~causal, float("-inf")), dim=-1).permute(0, 2, 1).numpy()
    return (np.allclose(o, ref, atol=1e-12) and np.allclose(od, ref, atol=1e-12)
            and np.allclose(lse, ref_lse, atol=1e-12) and np.allclose(lsed, ref_lse, atol=1e-12))


def pin_mla_sparse_equals_dense(sparse_mla, dense_masked_mla) -> bool:
    """Gathering the selected rows equals the dense causal form with an additive
    0/-inf mask (the selection mechanism named on the pages)."""
    r = _rng(35)
    B, L, H, D, DV, K = 1, 40, 3, 9, 5, 6
    q = r.standard_normal((B, L, H, D))
    kv = r.standard_normal((B, L, D))
    idx = np.full((B, L, K), -1, dtype=np.int32)
    for t in range(L):
        n = min(K, t + 1)
        idx[0, t, :n] = np.sort(r.choice(t + 1, size=n, replace=False))
    o, lse = sparse_mla(q, kv, idx, 0.5, DV)
    od, lsed = dense_masked_mla(q, kv, idx, 0.5, DV, 0)
    return np.allclose(o, od, atol=1e-13) and np.allclose(lse, lsed, atol=1e-13)


# ------------------------------------------------- MLA projections (absorbed) ---

def _mla_proj_case(seed, H=3, d_nope=4, d_rope=2, d_c=6, d_v=5, N=11):
    r = _rng(seed)
    return dict(q=r.standard_normal((H, d_nope + d_rope)), c=r.standard_normal((N, d_c)),
                kr=r.standard_normal((N, d_rope)), W_UK=r.standard_normal((H, d_nope, d_c)),
                W_UV=r.standard_normal((H, d_v, d_c)))


def _safe(fn, *a):
    try:
        return fn(*a)
    except Exception:
        return None


def pin_mla_naive_sdpa(mla_naive_rows) -> bool:
    """The naive per-head form is plain attention with per-head keys [W_UK c | k_rope]
    and values W_UV c: compare against torch's scaled_dot_product_attention (CPU,
    float64) over the selected tokens, and check lse against logsumexp."""
    import torch
    x = _mla_proj_case(41)
    H = x["q"].shape[0]
    idx = np.array([7, 2, -1, 9, 0, -1])
    sel = [int(i) for i in idx if i >= 0]
    out = _safe(mla_naive_rows, x["q"], x["c"], x["kr"], idx, x["W_UK"], x["W_UV"], 0.45)
    if out is None:
        return False
    o, lse = out
    c = torch.from_numpy(x["c"][sel])
    keys = torch.stack([torch.cat([c @ torch.from_numpy(x["W_UK"][h]).T, torch.from_numpy(x["kr"][sel])], 1)
                        for h in range(H)])                                  # [H, n, d_nope + d_rope]
    vals = torch.stack([c @ torch.from_numpy(x["W_UV"][h]).T for h in range(H)])  # [H, n, d_v]
    tq = torch.from_numpy(x["q"])[:, None, :]                                  # [H, 1, d]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, keys, vals, scale=0.45)[:, 0].numpy()
    ref_lse = torch.logsumexp((tq @ keys.transpose(1, 2))[:, 0] * 0.45, dim=-1).numpy()
    # no selected token: zero output, lse -inf
    o0, l0 = mla_naive_rows(x["q"], x["c"], x["kr"], np.array([-1, -1]), x["W_UK"], x["W_UV"], 0.45)
    return (o.shape == ref.shape and np.allclose(o, ref, atol=1e-12) and np.allclose(lse, ref_lse, atol=1e-12)
            and not np.any(o0) and np.all(np.isneginf(l0)))


def pin_mla_absorbed_equals_naive(mla_absorb_query, sparse_mla_rows, mla_output_projection, mla_naive_rows) -> bool:
    """Absorbed latent attention (query folded through W_UK, attention over the
    [c | k_rope] rows with value c, then W_UV) equals naive per-head attention
    with the same weights, on several index rows including masked and empty ones."""
    for seed, dims in ((42, {}), (43, dict(H=2, d_nope=3, d_rope=3, d_c=8, d_v=2, N=7))):
        x = _mla_proj_case(seed, **dims)
        d_c = x["c"].shape[1]
        rows = np.concatenate([x["c"], x["kr"]], axis=1)
        N = rows.shape[0]
        for idx in (np.arange(N), np.array([3, -1, 0, 5]), np.array([N - 1]), np.array([-1, -1])):
            q_lat = _safe(mla_absorb_query, x["q"], x["W_UK"])
            if q_lat is None or q_lat.shape != (x["q"].shape[0], rows.shape[1]):
                return False
            o_lat, lse = sparse_mla_rows(q_lat, rows, idx, 0.3, d_c)
            o = _safe(mla_output_projection, o_lat, x["W_UV"])
            on, ln = mla_naive_rows(x["q"], x["c"], x["kr"], idx, x["W_UK"], x["W_UV"], 0.3)
            if o is None or o.shape != on.shape or not np.allclose(o, on, atol=1e-12):
                return False
            if not np.allclose(lse, ln, atol=1e-12) and not (np.all(np.isneginf(lse)) and np.all(np.isneginf(ln))):
                return False
    return True


def pin_linear(linear) -> bool:
    """y = x W^T with W [out, in]: the identity weight returns x, a one-hot input
    row picks the matching column of W, and a one-hot weight row picks one input
    feature (fixes the orientation of W)."""
    r = _rng(44)
    x = r.standard_normal((3, 5))
    W = r.standard_normal((4, 5))
    e = np.zeros((1, 5))
    e[0, 2] = 1.0
    sel = np.zeros((1, 5))
    sel[0, 4] = 1.0
    y = _safe(linear, x, W)
    return (y is not None and y.shape == (3, 4) and np.array_equal(linear(x, np.eye(5)), x)
            and np.array_equal(linear(e, W)[0], W[:, 2]) and np.array_equal(linear(x, sel)[:, 0], x[:, 4]))


# ------------------------------------------------------------- FP8 indexer ---

def pin_e4m3(e4m3_decode, e4m3_encode_rne) -> bool:
    """The E4M3 table facts and rounding midpoints of tests/golden/e4m3_codes.json,
    the round trip of every finite code, and monotone encoding."""
    g = load_golden("e4m3_codes.json")
    for c in g["decode"]:
        v = _safe(e4m3_decode, np.array([int(c["code"], 16)], dtype=np.uint8))
        if v is None or v[0] != c["value"]:
            return False
    if not all(np.isnan(e4m3_decode(np.array([int(c, 16)], dtype=np.uint8))[0]) for c in g["nan_codes"]):
        return False
    for c in g["encode_rne"]:
        got = _safe(e4m3_encode_rne, np.array([c["value"]], dtype=np.float32))
        if got is None or int(got[0]) != int(c["code"], 16):
            return False
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    fin = ~np.isnan(vals)
    if not np.array_equal(e4m3_encode_rne(vals[fin].astype(np.float32)), codes[fin]):
        return False
    sweep = np.linspace(-448.0, 448.0, 20001).astype(np.float32)
    dec = e4m3_decode(e4m3_encode_rne(sweep))
    return bool(np.all(np.diff(dec) >= 0))


def pin_fwht(fwht_f32, hadamard) -> bool:
    """The transform is the Sylvester matrix product (exact on integer rows), and
    applying it twice multiplies by the length."""
    r = _rng(51)
    x = r.integers(-4, 5, size=(6, 128)).astype(np.float32)
    y = _safe(fwht_f32, x)
    if y is None:
        return False
    H = hadamard(128)
    if not (np.array_equal(y.astype(np.float64), x.astype(np.float64) @ H.T) and
            np.array_equal(fwht_f32(y).astype(np.float64), 128.0 * x)):
        return False
    # Real-valued rows: whatever order the float32 butterflies add in, each of
    # the log2(128) = 7 levels rounds a partial sum of at most sum|x| once, so
    # the result lies within 7 * 2^-24 * sum|x| of the exact product.
    g = r.standard_normal((16, 128)).astype(np.float32)
    yg = _safe(fwht_f32, g)
    if yg is None:
        return False
    exact = g.astype(np.float64) @ H.T
    bound = 7.0 * 2.0 ** -24 * np.abs(g.astype(np.float64)).sum(axis=1, keepdims=True)
    return bool(np.all(np.abs(yg.astype(np.float64) - exact) <= bound))


def pin_pow2_scale(pow2_scale_exp) -> bool:
    """e is the smallest integer with amax <= 448 * 2^e."""
    cases = [448.0, 448.0001, 224.0, 224.0001, 1.0, 3.5, 1e-3, 7e5, 2.0 ** -40]
    for a in cases:
        e = _safe(pow2_scale_exp, a)
        if e is None or not (a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)):
            return False
    return pow2_scale_exp(448.0) == 0 and pow2_scale_exp(224.0) == -1 and pow2_scale_exp(0.0) == 0


def pin_quantize_fp8(quantize_fp8_rows, fwht_f32, e4m3_decode) -> bool:
    """Dequantised rows equal the rotated rows within the e4m3 rounding bound
    (2^-4 relative in the normal range, half of 2^-9 * scale below it), and each
    row's largest value lands in [224, 448] after scaling."""
    r = _rng(52)
    x = np.concatenate([r.integers(-4, 5, size=(20, 128)).astype(np.float32),
                        r.standard_normal((20, 128)).astype(np.float32),
                        np.zeros((1, 128), dtype=np.float32)])
    out = _safe(quantize_fp8_rows, x)
    if out is None:
        return False
    codes, scales = out
    y = fwht_f32(x).astype(np.float64)
    deq = e4m3_decode(codes) * scales[:, None].astype(np.float64)
    v = np.abs(y) / scales[:, None]
    bound = np.where(v >= 2.0 ** -6, 2.0 ** -4 * np.abs(y), 2.0 ** -10 * scales[:, None])
    if not np.all(np.abs(deq - y) <= bound):
        return False
    top = np.max(np.abs(e4m3_decode(codes[:-1])), axis=-1)
    return bool(np.all((top >= 224.0) & (top <= 448.0)) and not np.any(codes[-1] & 0x7F))


def pin_fp8_scores_near_bf16(quantize_fp8_rows, index_scores_fp8_rows, index_scores_rows, fwht_f32,
                             e4m3_decode) -> bool:
    """Through the orthogonality H^T H = D I, the FP8 score equals the bf16 score
    up to the quantisation error of the rotated rows:
        |I_fp8 - I| <= sum_h |w_h| / D * sum_d (|dq||yk| + |yq||dk| + |dq||dk|)."""
    r = _rng(53)
    T, HI, D, N = 4, 3, 128, 40
    q = r.integers(-4, 5, size=(T, HI, D)).astype(np.float32)
    k = r.integers(-4, 5, size=(N, D)).astype(np.float32)
    w = r.choice([0.25, 0.5, 1.0, 2.0], size=(T, HI))
    q8, qs = quantize_fp8_rows(q)
    k8, ks = quantize_fp8_rows(k)
    got = _safe(index_scores_fp8_rows, q8, qs, k8, ks, w, range(T), 20)
    if got is None:
        return False
    ref = index_scores_rows(q, k, w, range(T), 20)
    yq, yk = fwht_f32(q).astype(np.float64), fwht_f32(k).astype(np.float64)
    dq = e4m3_decode(q8) * qs[..., None] - yq
    dk = e4m3_decode(k8) * ks[..., None] - yk
    for t in range(T):
        n = len(ref[t])
        if len(got[t]) != n:
            return False
        per_head = (np.abs(dq[t]) @ np.abs(yk[:n]).T + np.abs(yq[t]) @ np.abs(dk[:n]).T
                    + np.abs(dq[t]) @ np.abs(dk[:n]).T) / D                  # [H_I, n]
        bound = np.abs(w[t]) @ per_head
        if not np.all(np.abs(got[t] - ref[t]) <= bound + 1e-9):
            return False
    return True


# ------------------------------------------------------------------ paging ---

def pin_paged_gather(paged_gather) -> bool:
    """Scattering a contiguous cache into a pool by the table (written here row by
    row) and gathering it back returns the cache; an identity table reads the
    pool's prefix."""
    r = _rng(61)
    bs, n, width = 4, 13, 3
    blocks = -(-n // bs)
    table = r.permutation(10)[:blocks]
    x = r.standard_normal((n, width))
    pool = np.full((10 * bs, width), np.nan)
    for row in range(n):
        pool[table[row // bs] * bs + row % bs] = x[row]
    got = _safe(paged_gather, pool, table, bs, n)
    ident = _safe(paged_gather, pool, np.arange(10), bs, 10 * bs)
    return got is not None and np.array_equal(got, x) and ident is not None and \
        np.array_equal(ident, pool, equal_nan=True)


# ------------------------------------------------------------- composition ---

def pin_forward(forward_rows) -> bool:
    """Indexer -> top-k -> sparse MLA, composed: on the hand-derived indexer
    example the composition returns the fixture's scores and indices, and
    with K >= L (every visible key selected) its attention is plain causal
    attention, checked against torch's scaled_dot_product_attention (CPU,
    float64) and logsumexp."""
    import torch
    g = load_golden("indexer_topk_tiny.json")
    r = _rng(71)
    T, H, D, DV = len(g["q_idx"]), 2, 5, 3
    q = r.standard_normal((T, H, D))
    kv = r.standard_normal((T, D))
    res = _safe(forward_rows, np.array(g["q_idx"], dtype=np.float64), np.array(g["k_idx"], dtype=np.float64),
                np.array(g["w"], dtype=np.float64), q, kv, range(T), g["q_pos0"], g["K"], 0.6, DV)
    if res is None:
        return False
    for x, s, i in zip(res, g["scores"], g["idx"]):
        if not (np.array_equal(x["scores"], np.array(s, dtype=np.float64)) and np.array_equal(x["idx"], np.array(i))):
            return False
    L, HI, DI = 11, 3, 4
    qI = r.integers(-3, 4, size=(L, HI, DI)).astype(np.float64)
    kI = r.integers(-3, 4, size=(L, DI)).astype(np.float64)
    w = r.choice([0.5, 1.0, 2.0], size=(L, HI))
    q = r.standard_normal((L, H, D))
    kv = r.standard_normal((L, D))
    res = forward_rows(qI, kI, w, q, kv, range(L), 0, L, 0.45, DV)
    tq = torch.from_numpy(q).permute(1, 0, 2)                                   # [H, L, D]
    tk = torch.from_numpy(kv)[None].expand(H, L, D)
    tv = torch.from_numpy(kv[:, :DV])[None].expand(H, L, DV)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.45).permute(1, 0, 2)
    logits = (tq @ tk.transpose(1, 2)) * 0.45
    causal = torch.ones(L, L, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(logits.masked_fill(~causal, float("-inf")), dim=-1).permute(1, 0).numpy()
    for t, x in enumerate(res):
        exp_idx = np.array(list(range(t + 1)) + [-1] * (L - t - 1), dtype=np.int32)
        if not (np.array_equal(x["idx"], exp_idx) and np.allclose(x["o"], ref[t].numpy(), atol=1e-12)
                and np.allclose(x["lse"], ref_lse[t], atol=1e-12)):
            return False
    return True


def pin_topk_long_ties(topk_row) -> bool:
    """Rows of a few hundred keys drawn from three values: the rank-count
    definition fixes which of the tied keys are kept (the lower indices)."""
    r = _rng(23)
    for trial in range(20):
        n = int(r.integers(100, 400))
        K = int(r.integers(1, n))
        v = r.integers(0, 3, size=n).astype(np.float32)
        got = _safe(topk_row, v, K)
        if got is None:
            return False
        # rank-count definition, vectorised: rank(s) = #{s' : v[s'] > v[s] or (v[s'] == v[s] and s' < s)}
        i = np.arange(n)
        rank = ((v[None, :] > v[:, None]) | ((v[None, :] == v[:, None]) & (i[None, :] < i[:, None]))).sum(1)
        exp = np.flatnonzero(rank < K).astype(np.int32)
        if not np.array_equal(got, exp):
            return False
    return True
