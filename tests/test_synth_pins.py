"""Pins of the seeded input generator (CPU only).

The generator is not the oracle, but both sides consume its bytes, so its
quantised weights are checked against what the number formats fix: an FP8
block's largest value lands on the largest e4m3 code (448), and every MXFP4
nibble is the oracle's brute-force round-to-nearest-even e2m1 code of the
value divided by the block's power-of-two scale 2^(floor(log2 amax) - 2).
Planted generator mistakes (a wrong FP8 maximum, a moved e2m1 rounding
midpoint) must fail these pins.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.fixture(autouse=True)
def _lib(oracle_lib):
    yield


def _fp8_blocks_hit_448(wl, seed=0) -> bool:
    """Every b x b block of the generated e4m3 weights holds +-448 (code
    0x7E / 0xFE) and no larger magnitude; the dequantised weights keep the
    N(0, 0.02) spread."""
    w = synth.gen_weights(wl, seed=seed)
    for codes, scales in ((w.w1, w.w1s), (w.w2, w.w2s)):
        E, N, K = codes.shape
        b = wl.wblk
        v = codes.view(torch.float8_e4m3fn).to(torch.float64).abs()
        bmax = v.reshape(E, N // b, b, K // b, b).amax(dim=(2, 4))
        if not bool((bmax == 448.0).all()):
            return False
        deq = codes.view(torch.float8_e4m3fn).to(torch.float64) * \
            scales.to(torch.float64).repeat_interleave(b, 1).repeat_interleave(b, 2)
        if not 0.019 < float(deq.std()) < 0.021:
            return False
    return True


def _mxfp4_matches_oracle_encoder(seed=0) -> bool:
    """The MXFP4 quantiser on seeded N(0, 0.02) rows (plus an all-zero
    block, exact e2m1 midpoints and a saturating value) against the scale
    rule and the oracle's brute-force e2m1 encoder, element by element."""
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(48, 512, generator=g) * 0.02
    w[0, :32] = 0.0                                     # all-zero block: scale code 0, zero nibbles
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0])
    w[1, 32:64] = torch.cat([mids, -mids, mids / 2, -mids / 2])  # amax 5 -> X = 1: midpoints exact
    w[2, 64:96] = torch.linspace(-7.5, 7.9, 32)         # amax 7.9 -> X = 1: 6.x saturates at 6
    packed, sc = synth._quant_mxfp4(w)
    nib = torch.stack([packed & 15, packed >> 4], dim=-1).reshape(w.shape).numpy()
    sc = sc.numpy()
    wn = w.numpy()
    for r in range(w.shape[0]):
        for blk in range(w.shape[1] // 32):
            vals = wn[r, blk * 32:(blk + 1) * 32]
            amax = float(np.abs(vals).max())
            if amax == 0.0:
                if sc[r, blk] != 0 or np.any(nib[r, blk * 32:(blk + 1) * 32] != 0):
                    return False
                continue
            want = 127 + math.frexp(amax)[1] - 1 - 2      # floor(log2 amax) - 2, biased
            if sc[r, blk] != want:
                return False
            X = math.ldexp(1.0, want - 127)
            for i, v in enumerate(vals):
                if nib[r, blk * 32 + i] != oracle.enc_e2m1(float(np.float32(v / X))):
                    return False
    return True


def test_fp8_generator_block_max_is_448():
    assert _fp8_blocks_hit_448(synth.WORKLOADS["tiny_fp8"])
    assert _fp8_blocks_hit_448(synth.WORKLOADS["decode_fp8"].with_shape(H=256, I=128, E=2))


def test_mxfp4_generator_matches_oracle_encoder():
    assert _mxfp4_matches_oracle_encoder()


def test_mxfp4_generated_block_max_codes():
    """With X = 2^(floor(log2 amax) - 2), amax / X lies in [4, 8): each block's
    largest nibble magnitude is 4 (code 6) or 6 (code 7, saturated)."""
    wl = synth.WORKLOADS["decode_mxfp4"].with_shape(H=256, I=128, E=2)
    w = synth.gen_weights(wl, seed=2)
    for packed in (w.w1, w.w2):
        nib = torch.stack([packed & 15, packed >> 4], dim=-1).reshape(*packed.shape[:-1], -1)
        mag = (nib & 7).reshape(*nib.shape[:-1], -1, 32).amax(dim=-1)
        assert bool(((mag == 6) | (mag == 7)).all())


def test_planted_generator_mistakes_are_caught(monkeypatch):
    wl = synth.WORKLOADS["tiny_fp8"]
    assert _fp8_blocks_hit_448(wl) and _mxfp4_matches_oracle_encoder()
    with monkeypatch.context() as m:
        m.setattr(synth, "_FP8_MAX", 400.0)               # block maximum no longer on 448
        assert not _fp8_blocks_hit_448(wl)
    with monkeypatch.context() as m:
        m.setattr(synth, "_E2M1_MIDS", (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.5))  # 4|6 midpoint moved
        assert not _mxfp4_matches_oracle_encoder()
