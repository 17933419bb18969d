"""Pins of the oracle's MXFP4-activation variant (CPU only): activations and
the SwiGLU output quantised to e2m1 with one e8m0 scale per 32 channels
(X = 2^(floor(log2 amax) - 2), round to nearest even, saturating at 6).

The oracle's C++ quantiser (brute-force nearest e2m1 code of v / X) is
checked against the input generator's independent PyTorch implementation of
the same Microscaling rule (threshold comparisons, torch.frexp) on random
rows, special values and every finite bf16 value; the layer against brute
force and against a single-expert MLP built only from PyTorch ops; a planted
scale-exponent mistake must fail.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.fixture(autouse=True)
def _clean(oracle_lib):
    oracle.set_mutation(0)
    yield
    oracle.set_mutation(0)


def _rows():
    g = torch.Generator().manual_seed(21)
    x = torch.randn(24, 256, generator=g)
    x[0] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = 1e-39                                    # subnormal group
    x[3] *= 1e30
    x[4, :32] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0] * 4)  # e2m1 midpoints, X = 1
    x[5, :32] = torch.linspace(-7.9, 7.9, 32)            # saturation at 6
    x[6, 32:64] = 2.0 ** -126
    x[7, ::3] *= 1e-20
    return x.to(torch.bfloat16)


def _agrees(x) -> bool:
    q, s = oracle.quant_act_mx(x)
    rq, rs = synth._quant_mxfp4(x.float())
    return np.array_equal(q, rq.numpy()) and np.array_equal(s, rs.numpy())


def test_mxfp4_activation_quant_matches_generator_rule():
    assert _agrees(_rows())


def test_mxfp4_activation_quant_every_bf16_value():
    """Every finite bf16 x in a group whose maximum is a sampled value >= |x|."""
    allb = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    allb = allb[torch.isfinite(allb)]
    g = torch.Generator().manual_seed(22)
    for _ in range(2):
        f = 1.0 + torch.rand(allb.shape, generator=g) * 7
        amax = torch.maximum((allb.abs() * f).clamp_max(3.3e38).to(torch.bfloat16).float(), allb.abs())
        grp = torch.zeros(allb.numel(), 32)
        grp[:, 0] = allb
        grp[:, 1] = amax
        assert _agrees(grp.to(torch.bfloat16))


def test_mxfp4_activation_spot_values():
    x = torch.zeros(1, 32)
    x[0, :4] = torch.tensor([6.0, -3.0, 0.5, -0.0])
    q, s = oracle.quant_act_mx(x.to(torch.bfloat16))
    assert s[0, 0] == 127                                # amax 6 -> X = 2^(2-2) = 1
    assert list(q[0, :2]) == [0x7 | (0xD << 4), 0x1 | (0x8 << 4)]
    q, s = oracle.quant_act_mx(torch.zeros(1, 32, dtype=torch.bfloat16))
    assert s[0, 0] == 0 and not q.any()


SMALL_A4 = synth.WORKLOADS["decode_mxfp4"].with_shape(H=256, E=6, I=256, topk=3, act_group=32, act_fmt=1)


def test_a4_layer_matches_bruteforce():
    wl = SMALL_A4
    T = 10
    w = synth.gen_weights(wl, seed=23)
    x, ids, tw = synth.gen_inputs(wl, T, seed=23)
    lay = oracle.layer_for(wl, T, w)
    a, b = lay.layer(x, ids, tw), lay.bruteforce(x, ids, tw)
    assert np.abs(a - b).max() <= 1e-9 * np.abs(b).max() and np.abs(b).max() > 0


def _mx_dequant(v: torch.Tensor) -> torch.Tensor:
    """Quantise fp32 rows with the generator's MXFP4 rule and dequantise with
    PyTorch ops (fp64)."""
    packed, code = synth._quant_mxfp4(v.float())
    lo, hi = (packed & 15).to(torch.int64), (packed >> 4).to(torch.int64)
    nib = torch.stack([lo, hi], dim=-1).reshape(v.shape[0], -1)
    lut = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)
    val = lut[nib & 7] * torch.where((nib & 8) > 0, -1.0, 1.0).to(torch.float64)
    return val * code.view(torch.float8_e8m0fnu).to(torch.float64).repeat_interleave(32, 1)


def test_a4_single_expert_equals_plain_mlp():
    """E = 1, k = 1, weight 1: the plain MXFP4 MLP written with PyTorch ops."""
    import test_oracle_pins as pins
    wl = SMALL_A4.with_shape(E=1, topk=1)
    T = 7
    w = synth.gen_weights(wl, seed=24)
    x = synth.gen_x(T, wl.H, 24, wl.wid)
    got = oracle.layer_for(wl, T, w).layer(x, torch.zeros(T, 1, dtype=torch.int32), torch.ones(T, 1))
    W1 = pins._dequant_torch(w.w1[0], w.w1s[0], wl.wfmt, wl.wblk)
    W2 = pins._dequant_torch(w.w2[0], w.w2s[0], wl.wfmt, wl.wblk)
    gu = _mx_dequant(x.float()) @ W1.T
    h = (torch.nn.functional.silu(gu[:, : wl.I]) * gu[:, wl.I:]).to(torch.float32)
    ref = (_mx_dequant(h) @ W2.T).numpy()
    assert np.abs(got - ref).max() <= 1e-9 * np.abs(ref).max()


def test_planted_mxfp4_scale_mistake_is_caught():
    assert _agrees(_rows())
    oracle.set_mutation(9)
    try:
        assert not _agrees(_rows())
    finally:
        oracle.set_mutation(0)
