"""CPU pins of the oracle's NVFP4 weight path (e2m1 codes, an e4m3 scale per
16 along K, an fp32 scale per expert matrix) and of the generator's NVFP4
quantiser.

The pages name NVFP4 beside MXFP4 without printing its layout; the oracle
takes the published two-level definition.  These pins tie the oracle to
PyTorch's own format casts (e4m3 through float8_e4m3fn, e2m1 through its
closed form), to exact scaling laws of the definition, and to brute force.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

from test_oracle_pins import _torch_quant_rows

NV = synth.WORKLOADS["decode_nvfp4"].with_shape(H=256, E=6, I=256, topk=3)
LUT = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _dequant_nvfp4(codes, scales, g):
    """Dense fp64 [N,K] from canonical NVFP4 with PyTorch ops only."""
    lo, hi = (codes & 15).to(torch.int64), (codes >> 4).to(torch.int64)
    nib = torch.stack([lo, hi], dim=-1).reshape(codes.shape[0], -1)
    v = LUT[nib & 7] * torch.where((nib & 8) > 0, -1.0, 1.0).to(torch.float64)
    s = scales.view(torch.float8_e4m3fn).to(torch.float64).repeat_interleave(16, 1)
    return v * s * float(g)


def _plain_mlp(wl, w, x):
    """E=1, k=1, weight 1: the plain quantised MLP with PyTorch ops only."""
    G = wl.act_group
    xq, xs = _torch_quant_rows(x.float(), G)
    xd = torch.from_numpy(xq).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(xs).to(torch.float64).repeat_interleave(G, 1)
    W1 = _dequant_nvfp4(w.w1[0], w.w1s[0], w.w1g[0])
    W2 = _dequant_nvfp4(w.w2[0], w.w2s[0], w.w2g[0])
    gu = xd @ W1.T
    h = (torch.nn.functional.silu(gu[:, : wl.I]) * gu[:, wl.I:]).to(torch.float32)
    hq, hs = _torch_quant_rows(h, G)
    hd = torch.from_numpy(hq).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(hs).to(torch.float64).repeat_interleave(G, 1)
    return (hd @ W2.T).numpy()


def test_single_expert_equals_plain_mlp():
    wl = NV.with_shape(E=1, topk=1)
    T = 9
    w = synth.gen_weights(wl, seed=7)
    x = synth.gen_x(T, wl.H, 7, wl.wid)
    ids = torch.zeros(T, 1, dtype=torch.int32)
    tw = torch.ones(T, 1)
    got = oracle.layer_for(wl, T, w).layer(x, ids, tw)
    ref = _plain_mlp(wl, w, x)
    assert np.abs(ref).max() > 0
    assert np.abs(got - ref).max() <= 1e-9 * np.abs(ref).max()


def test_layer_matches_bruteforce():
    T = 12
    w = synth.gen_weights(NV, seed=5)
    x, ids, tw = synth.gen_inputs(NV, T, seed=5)
    lay = oracle.layer_for(NV, T, w)
    a, b = lay.layer(x, ids, tw), lay.bruteforce(x, ids, tw)
    assert np.abs(b).max() > 0
    assert np.abs(a - b).max() <= 1e-9 * np.abs(b).max()


def test_matrix_scale_of_w2_scales_the_output_exactly():
    """Doubling every W2 matrix scale doubles every output exactly (h does
    not depend on W2, and a power-of-two factor is exact in fp64); doubling
    one expert's W2 scale changes only the tokens routed to it."""
    T = 8
    w = synth.gen_weights(NV, seed=3)
    x, ids, tw = synth.gen_inputs(NV, T, seed=3)
    base = oracle.layer_for(NV, T, w).layer(x, ids, tw)
    w2 = synth.Weights(w.w1, w.w1s, w.w2, w.w2s, w1g=w.w1g, w2g=w.w2g * 2)
    assert np.array_equal(oracle.layer_for(NV, T, w2).layer(x, ids, tw), 2 * base)
    e = int(ids[0, 0])
    g = w.w2g.clone()
    g[e] *= 2
    w3 = synth.Weights(w.w1, w.w1s, w.w2, w.w2s, w1g=w.w1g, w2g=g)
    out = oracle.layer_for(NV, T, w3).layer(x, ids, tw)
    hit = (ids == e).any(dim=1).numpy()
    assert np.array_equal(out[~hit], base[~hit])
    assert not np.array_equal(out[hit], base[hit])


def test_w1_matrix_scale_enters_the_gemm1_dot():
    """GEMM1's fp32 h of a row equals SwiGLU of the plain dot products with
    the W1 matrix scale applied (checked through the stage reference)."""
    wl = NV.with_shape(E=1, topk=1)
    T = 4
    w = synth.gen_weights(wl, seed=11)
    x = synth.gen_x(T, wl.H, 11, wl.wid)
    ids = torch.zeros(T, 1, dtype=torch.int32)
    xq, xs = oracle.quant_act(x, wl.act_group)
    counts, offsets, eidx, rtok = oracle.permute(ids, 1, False)
    h, _, _ = oracle.layer_for(wl, T, w).gemm1(xq, xs, rtok, offsets, range(T))
    xd = torch.from_numpy(xq).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(xs).to(torch.float64).repeat_interleave(wl.act_group, 1)
    W1 = _dequant_nvfp4(w.w1[0], w.w1s[0], w.w1g[0])
    gu = (xd[rtok.astype(np.int64)] @ W1.T)
    ref = (torch.nn.functional.silu(gu[:, : wl.I]) * gu[:, wl.I:]).to(torch.float32).numpy()
    assert np.abs(h - ref).max() <= 1e-6 * np.abs(ref).max()


def test_generator_quantiser_roundtrip_and_exact_values():
    """The generator's NVFP4 quantiser: a matrix built from representable
    values (codes x block scale x matrix scale with the block maximum 6) comes
    back exactly; random weights come back within half an e2m1 step of their
    block (saturation aside), and every block scale is a finite positive
    e4m3 code."""
    g = torch.Generator().manual_seed(1)
    N, K = 32, 64
    nib = torch.randint(0, 16, (N, K), generator=g)
    nib[:, ::16] = 7                                   # every block holds the maximum code 6
    bs_codes = torch.randint(0x20, 0x60, (N, K // 16), generator=g).to(torch.uint8)
    bs_codes[0, 0] = 0x7E                              # 448: this block's 6 is the matrix maximum
    S = 2.0 ** -9                                      # so the quantiser's matrix scale is S again
    bs = bs_codes.view(torch.float8_e4m3fn).to(torch.float64)
    v = LUT[nib & 7] * torch.where((nib & 8) > 0, -1.0, 1.0).to(torch.float64)
    w = (v * bs.repeat_interleave(16, 1) * S).to(torch.float32)
    codes, scales, Sg = synth._quant_nvfp4(w)
    assert float(Sg[0]) == S
    back = _dequant_nvfp4(codes, scales, Sg[0])
    assert torch.equal(back, w.to(torch.float64))
    w = torch.randn(N, K, generator=g) * 0.02
    codes, scales, Sg = synth._quant_nvfp4(w)
    sc = scales.view(torch.float8_e4m3fn).to(torch.float64)
    assert torch.isfinite(sc).all() and (sc > 0).all()
    back = _dequant_nvfp4(codes, scales, Sg[0])
    step = sc.repeat_interleave(16, 1) * float(Sg[0])    # scale of one e2m1 unit in the block
    err = (back - w.to(torch.float64)).abs() / step
    assert float(err.max()) <= 1.0 + 1e-9                # half the widest e2m1 gap (2) is 1 unit
