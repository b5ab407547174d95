"""GPU parity for the projections on either side of the sparse MLA.

Query absorption, the value up-projection and the plain linear layer run
through the C-ABI and are compared with the oracle (float64) within the bf16
output tolerance; the copied rope part of an absorbed query is compared bit
for bit.  The last test runs absorption -> sparse MLA -> value projection on
the GPU and compares it with the oracle's naive per-head attention with the
same random weights, which is the absorbed reading of the attention checked
end to end.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, assert_lse_close, dev, host64

pytestmark = pytest.mark.gpu

PROJ_WID = 40  # generator stream family of these tests


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _dsa():
    import long_context_sparse_14_amd as dsa
    dsa.library()
    return dsa


def normal_bf16(shape, tensor_id, pow2=0, seed=0):
    """N(0,1) bf16 bit patterns from the seeded generator, scaled by 2^-pow2 (exact)."""
    n = int(np.prod(shape))
    bits = synth.fill(synth.stream_key(seed, PROJ_WID, tensor_id), 0, n, synth.NORMAL, "bf16")
    if pow2:
        f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** -pow2)
        bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    return bits.reshape(shape)


@pytest.mark.parametrize("M,H,d_nope,d_rope,d_c", [
    (37, 4, 128, 64, 512),     # ragged rows, the V3.2 head shape
    (32, 128, 128, 64, 512),   # the 128K decode batch, all 128 heads
    (130, 3, 32, 0, 40),       # no rope part, a column block cut at 40
    (200, 2, 128, 64, 512),    # 128-row blocks walking four column blocks, eight k-steps
    (300, 3, 64, 64, 264),     # short K, a last column block of 8
    (129, 2, 96, 32, 136),     # K = 96 (six k-steps), one row in the last row block
    (100, 2, 160, 0, 128),     # K above the column walk's 128: the tiled kernel
])
def test_absorb_q(M, H, d_nope, d_rope, d_c):
    dsa = _dsa()
    q = normal_bf16((M, H, d_nope + d_rope), 1)
    w = normal_bf16((H, d_nope, d_c), 2, pow2=4)
    got = dsa.mla_absorb_q(dev(q), dev(w))
    ref = oracle.mla_absorb_query(q, w)
    assert_close(host64(got[..., :d_c]), ref[..., :d_c], "bf16", "absorbed query")
    g16 = got[..., d_c:].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(g16, q[..., d_nope:]), "rope part not copied bit for bit"


@pytest.mark.parametrize("M,H,d_c,d_v", [
    (37, 4, 512, 128),
    (32, 128, 512, 128),
    (70, 2, 64, 40),
    (150, 2, 512, 128),        # eight 64-wide k steps, ragged rows
])
def test_out_proj(M, H, d_c, d_v):
    dsa = _dsa()
    o_lat = normal_bf16((M, H, d_c), 3)
    w = normal_bf16((H, d_v, d_c), 4, pow2=4)
    got = dsa.mla_out_proj(dev(o_lat), dev(w))
    assert_close(host64(got), oracle.mla_output_projection(o_lat, w), "bf16", "output projection")


@pytest.mark.parametrize("M,N,K", [
    (37, 8192, 1536),   # indexer query projection from the 1536-wide query latent, 64 heads x 128
    (5, 64, 7168),      # per-head weight projection from a 7168-wide hidden state
    (1, 200, 64),
    (300, 200, 96),     # 128-row tiles, ragged rows and columns, an odd number of k tiles
    (70, 64, 32),       # a single k tile
    (260, 136, 1536),   # 24 k tiles of 64, ragged rows and columns
    (140, 96, 320),     # an odd number (5) of 64-wide k tiles
])
def test_linear(M, N, K):
    dsa = _dsa()
    x = normal_bf16((M, K), 5)
    w = normal_bf16((N, K), 6, pow2=5)
    got = dsa.linear(dev(x), dev(w))
    assert_close(host64(got), oracle.linear(x, w), "bf16", "linear")


def test_absorbed_path_equals_naive():
    """absorb -> sparse MLA -> value projection (GPU) == naive per-head MLA (oracle)."""
    dsa = _dsa()
    B, Tq, N, H, d_nope, d_rope, d_c, d_v, K = 2, 3, 300, 128, 128, 64, 512, 128, 64
    scale = 1.0 / np.sqrt(192.0)
    q = normal_bf16((B, Tq, H, d_nope + d_rope), 7)
    kv = normal_bf16((B, N, d_c + d_rope), 8)
    w_uk = normal_bf16((H, d_nope, d_c), 9, pow2=4)
    w_uv = normal_bf16((H, d_v, d_c), 10, pow2=4)
    rng = np.random.default_rng(11)
    idx = np.full((B, Tq, K), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Tq):
            n = K - 7 * t                     # some rows end in -1 padding
            idx[b, t, :n] = np.sort(rng.choice(N, size=n, replace=False))
    q_lat = dsa.mla_absorb_q(dev(q), dev(w_uk))
    o_lat, lse = dsa.sparse_mla(q_lat, dev(kv), torch.from_numpy(idx).cuda(), scale, d_c)
    o = dsa.mla_out_proj(o_lat, dev(w_uv))
    torch.cuda.synchronize()
    o, lse = host64(o), host64(lse)
    for b in range(B):
        c, kr = kv[b, :, :d_c], kv[b, :, d_c:]
        for t in range(Tq):
            ref_o, ref_lse = oracle.mla_naive_rows(q[b, t], c, kr, idx[b, t], w_uk, w_uv, scale)
            assert_close(o[b, t], ref_o, "bf16", f"naive vs absorbed b={b} t={t}")
            assert_lse_close(lse[b, t], ref_lse, f"lse b={b} t={t}")
