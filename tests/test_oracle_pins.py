"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin checks the oracle against a library routine, a closed form, an
invariant the mathematics fixes, brute force, or a hand-derived worked
example, so that a plausible mistake (a dropped term, a wrong sign or index,
a transposed operand, an unstable order) fails at least one of them.  The
last group plants such mistakes in the oracle and shows the pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


@pytest.fixture(autouse=True)
def _clean_mutation(oracle_lib):
    oracle.set_mutation(0)
    yield
    oracle.set_mutation(0)


# ------------------------------------------------------------ number formats
def test_e4m3_decode_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.dec_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.isnan(got).sum() == 2  # S.1111.111 only
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x80] == 0.0 and math.copysign(1, got[0x80]) < 0


def test_e2m1_decode_all_codes_closed_form():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.dec_e2m1(c)
        assert abs(v) == mags[c & 7]
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)


def test_e8m0_decode_all_codes_match_torch_and_ldexp():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.dec_e8m0(c)
        if c == 255:
            assert math.isnan(v) and math.isnan(ref[c])
        else:
            assert v == math.ldexp(1.0, c - 127) == ref[c]


def test_e4m3_encode_roundtrip_and_ties_to_even():
    for c in range(256):
        v = oracle.dec_e4m3(c)
        if math.isnan(v):
            continue
        assert oracle.enc_e4m3(v) == c
    mags = [oracle.dec_e4m3(c) for c in range(0x7F)]
    for c in range(0x7E):
        mid = np.float32((mags[c] + mags[c + 1]) / 2)  # every midpoint is exact in fp32
        assert float(mid) == (mags[c] + mags[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.enc_e4m3(float(mid)) == even
        assert oracle.enc_e4m3(float(-mid)) == even | 0x80
        # one fp32 ulp either side of the midpoint goes to the nearer code
        lo = np.nextafter(mid, np.float32(-1))
        hi = np.nextafter(mid, np.float32(1000))
        assert oracle.enc_e4m3(float(lo)) == c and oracle.enc_e4m3(float(hi)) == c + 1


def test_e4m3_encode_saturation_and_signed_zero():
    assert oracle.enc_e4m3(448.0) == 0x7E
    assert oracle.enc_e4m3(1e30) == 0x7E and oracle.enc_e4m3(-1e30) == 0xFE
    assert oracle.enc_e4m3(0.0) == 0x00 and oracle.enc_e4m3(-0.0) == 0x80
    assert oracle.enc_e4m3(-1e-12) == 0x80  # rounds to zero, keeps the sign


def test_e4m3_encode_matches_torch_cast_in_range():
    g = torch.Generator().manual_seed(1)
    v = torch.cat([
        (torch.rand(200000, generator=g) * 2 - 1) * 448,
        torch.randn(200000, generator=g) * 2.0 ** torch.randint(-12, 8, (200000,), generator=g),
        torch.arange(-65536, 65536, dtype=torch.int32).to(torch.float32) * 2.0 ** -16,
    ]).to(torch.float32)
    v = v[v.abs() <= 448]
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.enc_e4m3_array(v.numpy())
    assert np.array_equal(ref, got)


def test_e2m1_encode_roundtrip_and_midpoints():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert oracle.enc_e2m1(mags[c]) == c
        assert oracle.enc_e2m1(-mags[c]) == c | 8
    for c in range(7):
        mid = (mags[c] + mags[c + 1]) / 2
        assert oracle.enc_e2m1(mid) == (c if c % 2 == 0 else c + 1)
    assert oracle.enc_e2m1(100.0) == 7


# ------------------------------------------------------------ activation quant
def _torch_quant_rows(v: torch.Tensor, G: int):
    """The quantisation rule written with PyTorch's fp32 ops and its fp32 ->
    float8_e4m3fn cast (saturating inputs never exceed 448 here)."""
    rows, cols = v.shape
    blk = v.reshape(rows, cols // G, G).to(torch.float32)
    a = blk.abs().amax(dim=2).clamp_min(2.0 ** -64)
    m = torch.full_like(a, 448.0) / a
    p = blk * m[:, :, None]
    p = torch.where(p.abs() > 448, torch.sign(p) * 448, p)
    q = p.to(torch.float8_e4m3fn).view(torch.uint8).reshape(rows, cols)
    s = torch.ones_like(m) / m
    return q.numpy(), s.numpy()


def test_quant_act_matches_torch_rule_random_rows():
    g = torch.Generator().manual_seed(2)
    x = torch.randn(64, 512, generator=g).to(torch.bfloat16)
    x[3] = 0                                         # all-zero token
    x[4, :128] = torch.tensor(1e-38).to(torch.bfloat16)  # denormal group
    x[5, 7] = -0.0
    x[6] *= 1e4
    for G in (32, 128):
        q, s = oracle.quant_act(x, G)
        rq, rs = _torch_quant_rows(x.float(), G)
        assert np.array_equal(q, rq)
        assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))


def test_quant_all_bf16_values_against_sampled_amax():
    """Every finite bf16 x paired with amax values >= |x| (groups of 2)."""
    allb = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    allb = allb[torch.isfinite(allb)]
    g = torch.Generator().manual_seed(3)
    for _ in range(3):
        f = 1.0 + torch.rand(allb.shape, generator=g) * 4
        amax = (allb.abs() * f).to(torch.bfloat16).float()
        amax = torch.maximum(amax.clamp_max(torch.finfo(torch.bfloat16).max), allb.abs())
        v = torch.stack([allb, amax], dim=1).contiguous()
        q, s = oracle.quant_rows_f32(v.numpy(), 2)
        rq, rs = _torch_quant_rows(v, 2)
        assert np.array_equal(q, rq)
        assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))


def test_quant_spot_values():
    q, s = oracle.quant_rows_f32(np.array([[3.5, -1.75, 0.0, -0.0]], np.float32), 4)
    assert list(q[0]) == [0x7E, 0xF6, 0x00, 0x80] and s[0, 0] == np.float32(1 / 128)
    q, s = oracle.quant_rows_f32(np.zeros((1, 4), np.float32), 4)
    assert list(q[0]) == [0, 0, 0, 0] and np.isfinite(s[0, 0]) and s[0, 0] > 0


# ------------------------------------------------------------ permute
def _ref_permute(ids: np.ndarray, E: int, has_shared: bool):
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    if has_shared:
        counts = np.append(counts, T)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    key = np.where(valid, flat, E + 1)
    order = np.argsort(key, kind="stable")          # library stable sort of (id, flat index)
    eidx = np.full(T * k, -1, np.int32)
    nv = int(valid.sum())
    eidx[order[:nv]] = np.arange(nv, dtype=np.int32)
    rtok = np.full(T * k + T * int(has_shared), -1, np.int32)
    rtok[:nv] = order[:nv] // k
    if has_shared:
        rtok[nv:nv + T] = np.arange(T)
    return counts.astype(np.int32), offsets, eidx, rtok


@pytest.mark.parametrize("T,k,E,shared,mask", [(16, 2, 8, False, False), (257, 8, 64, False, False),
                                                (100, 8, 256, True, False), (300, 4, 16, False, True),
                                                (0, 8, 64, False, False), (1, 8, 64, True, False),
                                                (33, 3, 5, False, True)])
def test_permute_matches_stable_sort(T, k, E, shared, mask):
    rng = np.random.default_rng(T * 31 + k)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)  # duplicates inside a token are legal
    if mask and T:
        ids[rng.random((T, k)) < 0.2] = -1
        ids[0, 0] = E + 3
    got = oracle.permute(ids, E, shared)
    ref = _ref_permute(ids, E, shared)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


def test_permute_invariants():
    wl = synth.WORKLOADS["decode_fp8_zipf_shared"]
    ids, _ = synth.gen_routing(256, wl.E, wl.topk, "zipf", 0, wl.wid)
    ids = ids.numpy()
    counts, offsets, eidx, rtok = oracle.permute(ids, wl.E, True)
    T, k = ids.shape
    assert counts[: wl.E].sum() == T * k and counts[wl.E] == T
    assert offsets[wl.E] == T * k and np.all(np.diff(offsets) >= 0)
    assert sorted(eidx.tolist()) == list(range(T * k))      # bijection
    flat = ids.reshape(-1)
    for i in range(T * k):
        r = eidx[i]
        assert rtok[r] == i // k
        assert offsets[flat[i]] <= r < offsets[flat[i] + 1]
    for e in range(wl.E):                                   # stable: rows increase with i
        rows = [eidx[i] for i in range(T * k) if flat[i] == e]
        assert rows == sorted(rows)
    assert (counts[: wl.E] == 0).sum() > 0                  # Zipf leaves experts empty


# ------------------------------------------------------------ layer pins
def _small(name, **kw):
    return synth.WORKLOADS[name].with_shape(**kw)


SMALL = {
    "tiny_fp8": synth.WORKLOADS["tiny_fp8"],
    "mxfp4": _small("decode_mxfp4", H=256, E=6, I=256, topk=3),
    "fp8_shared_zipf": _small("decode_fp8_zipf_shared", H=256, E=16, I=256, topk=4),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_matches_bruteforce(name):
    wl = SMALL[name]
    T = 12
    w = synth.gen_weights(wl, seed=5)
    x, ids, tw = synth.gen_inputs(wl, T, seed=5)
    lay = oracle.layer_for(wl, T, w)
    a = lay.layer(x, ids, tw)
    b = lay.bruteforce(x, ids, tw)
    assert np.abs(a - b).max() <= 1e-9 * np.abs(b).max()
    assert np.abs(b).max() > 0


def _dequant_torch(codes, scales, wfmt, wblk):
    """Dense fp64 weights from canonical codes with PyTorch's own format casts."""
    if wfmt == synth.FMT_FP8:
        v = codes.view(torch.float8_e4m3fn).to(torch.float64)
        s = scales.to(torch.float64).repeat_interleave(wblk, 0).repeat_interleave(wblk, 1)
        return v * s
    lo, hi = (codes & 15).to(torch.int64), (codes >> 4).to(torch.int64)
    nib = torch.stack([lo, hi], dim=-1).reshape(codes.shape[0], -1)
    lut = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)
    v = lut[nib & 7] * torch.where((nib & 8) > 0, -1.0, 1.0).to(torch.float64)
    s = scales.view(torch.float8_e8m0fnu).to(torch.float64).repeat_interleave(32, 1)
    return v * s


def _torch_plain_mlp(wl, w, x):
    """E=1, k=1, weight 1: the plain quantised MLP with PyTorch ops only."""
    G = wl.act_group
    xq, xs = _torch_quant_rows(x.float(), G)
    xd = torch.from_numpy(xq).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(xs).to(torch.float64).repeat_interleave(G, 1)
    W1 = _dequant_torch(w.w1[0], w.w1s[0], wl.wfmt, wl.wblk)
    W2 = _dequant_torch(w.w2[0], w.w2s[0], wl.wfmt, wl.wblk)
    gu = xd @ W1.T
    h = (torch.nn.functional.silu(gu[:, : wl.I]) * gu[:, wl.I:]).to(torch.float32)
    hq, hs = _torch_quant_rows(h, G)
    hd = torch.from_numpy(hq).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(hs).to(torch.float64).repeat_interleave(G, 1)
    return (hd @ W2.T).numpy()


def _torch_expert_mlp(wl, w1, w1s, w2, w2s, x):
    """One expert's quantised MLP over every token, PyTorch ops only (as
    _torch_plain_mlp, for the given expert matrices)."""
    G = wl.act_group
    xq, xs = _torch_quant_rows(x.float(), G)
    xd = torch.from_numpy(xq).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(xs).to(torch.float64).repeat_interleave(G, 1)
    gu = xd @ _dequant_torch(w1, w1s, wl.wfmt, wl.wblk).T
    h = (torch.nn.functional.silu(gu[:, : wl.I]) * gu[:, wl.I:]).to(torch.float32)
    hq, hs = _torch_quant_rows(h, G)
    hd = torch.from_numpy(hq).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(hs).to(torch.float64).repeat_interleave(G, 1)
    return (hd @ _dequant_torch(w2, w2s, wl.wfmt, wl.wblk).T).numpy()


def _mixture_agrees(name):
    """The oracle layer equals the layer written with PyTorch ops only: each
    token's output is the sum over its slots, in slot order, of the routing
    weight times that expert's quantised MLP (dense fp64 weights from
    PyTorch's own format casts), plus the shared expert with weight 1; a
    masked slot (id outside [0, E)) adds nothing.  It shares no decode table,
    quantiser, grouping or indexing with the oracle."""
    wl = SMALL[name]
    T = 10
    w = synth.gen_weights(wl, seed=13)
    x, ids, tw = synth.gen_inputs(wl, T, seed=13)
    ids = ids.clone()
    ids[3, 0] = -1
    ids[7, wl.topk - 1] = wl.E
    got = oracle.layer_for(wl, T, w).layer(x, ids, tw)
    mlp = [_torch_expert_mlp(wl, w.w1[e], w.w1s[e], w.w2[e], w.w2s[e], x) for e in range(wl.E)]
    ref = np.zeros((T, wl.H), np.float64)
    for t in range(T):
        for j in range(wl.topk):
            e = int(ids[t, j])
            if 0 <= e < wl.E:
                ref[t] += float(tw[t, j]) * mlp[e][t]
    if wl.shared:
        ref += _torch_expert_mlp(wl, w.sw1[0], w.sw1s[0], w.sw2[0], w.sw2s[0], x)
    assert np.abs(ref).max() > 0
    return np.abs(got - ref).max() <= 1e-9 * np.abs(ref).max()


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_equals_torch_mixture(name):
    assert _mixture_agrees(name)


def test_planted_expert_slice_mistake_is_caught_by_the_mixture():
    """Every routed expert reading its neighbour's matrices (planted in the
    weight decode, which the brute force shares) fails the PyTorch mixture."""
    oracle.set_mutation(10)
    try:
        assert not any(_mixture_agrees(n) for n in SMALL)
    finally:
        oracle.set_mutation(0)


@pytest.mark.parametrize("name", ["tiny_fp8", "mxfp4"])
def test_single_expert_equals_plain_mlp(name):
    wl = SMALL[name].with_shape(E=1, topk=1)
    T = 9
    w = synth.gen_weights(wl, seed=7)
    x = synth.gen_x(T, wl.H, 7, wl.wid)
    ids = torch.zeros(T, 1, dtype=torch.int32)
    tw = torch.ones(T, 1)
    got = oracle.layer_for(wl, T, w).layer(x, ids, tw)
    ref = _torch_plain_mlp(wl, w, x)
    assert np.abs(got - ref).max() <= 1e-9 * np.abs(ref).max()


def test_zero_weight_slot_contributes_nothing():
    wl = SMALL["tiny_fp8"]
    T = 6
    w = synth.gen_weights(wl, seed=9)
    x, ids, tw = synth.gen_inputs(wl, T, seed=9)
    tw[2, 1] = 0.0
    e = int(ids[2, 1])
    base = oracle.layer_for(wl, T, w).layer(x, ids, tw, toks=[2])
    w2 = synth.Weights(w.w1.clone(), w.w1s.clone(), w.w2.clone(), w.w2s.clone())
    g = torch.Generator().manual_seed(11)
    w2.w1[e] = torch.randint(0, 126, w2.w1[e].shape, generator=g, dtype=torch.uint8)
    w2.w2[e] = torch.randint(0, 126, w2.w2[e].shape, generator=g, dtype=torch.uint8)
    other = oracle.layer_for(wl, T, w2).layer(x, ids, tw, toks=[2])
    assert np.array_equal(base, other)


def test_doubling_routing_weights_doubles_output():
    wl = SMALL["mxfp4"]
    T = 5
    w = synth.gen_weights(wl, seed=4)
    x, ids, tw = synth.gen_inputs(wl, T, seed=4)
    lay = oracle.layer_for(wl, T, w)
    assert np.array_equal(lay.layer(x, ids, 2 * tw), 2 * lay.layer(x, ids, tw))


def test_relabelling_experts_is_invariant():
    wl = SMALL["tiny_fp8"]
    T = 8
    w = synth.gen_weights(wl, seed=12)
    x, ids, tw = synth.gen_inputs(wl, T, seed=12)
    perm = torch.randperm(wl.E, generator=torch.Generator().manual_seed(1))
    inv = torch.argsort(perm)
    ids2 = perm[ids.long()].to(torch.int32)             # expert e is now called perm[e]
    w2 = synth.Weights(w.w1[inv].contiguous(), w.w1s[inv].contiguous(), w.w2[inv].contiguous(),
                       w.w2s[inv].contiguous())
    a = oracle.layer_for(wl, T, w).layer(x, ids, tw)
    b = oracle.layer_for(wl, T, w2).layer(x, ids2, tw)
    assert np.array_equal(a, b)


def test_shared_expert_adds_with_weight_one():
    wl = SMALL["fp8_shared_zipf"]
    T = 4
    w = synth.gen_weights(wl, seed=13)
    x, ids, tw = synth.gen_inputs(wl, T, seed=13)
    with_shared = oracle.layer_for(wl, T, w).layer(x, ids, tw)
    routed = oracle.layer_for(wl.with_shape(shared=False), T, w).layer(x, ids, tw)
    # the shared expert alone: one expert holding the shared weights, every token, weight 1
    wl1 = wl.with_shape(E=1, topk=1, shared=False)
    ws = synth.Weights(w.sw1, w.sw1s, w.sw2, w.sw2s)
    alone = oracle.layer_for(wl1, T, ws).layer(x, torch.zeros(T, 1, dtype=torch.int32), torch.ones(T, 1))
    assert np.abs(with_shared - (routed + alone)).max() <= 1e-12 * np.abs(with_shared).max()


def test_masked_slots_are_ignored():
    wl = SMALL["tiny_fp8"]
    T = 6
    w = synth.gen_weights(wl, seed=14)
    x, ids, tw = synth.gen_inputs(wl, T, seed=14)
    ids_m = ids.clone()
    ids_m[1, 0] = -1
    ids_m[3, 1] = wl.E
    tw_z = tw.clone()
    tw_z[1, 0] = 0
    tw_z[3, 1] = 0
    lay = oracle.layer_for(wl, T, w)
    assert np.array_equal(lay.layer(x, ids_m, tw), lay.layer(x, ids, tw_z))


# ------------------------------------------------------------ stage combine
def _dense_routing_product(y, ids, tw, E, has_shared):
    """The combine as one matrix product: P [T, rows] holds each valid slot's
    routing weight in the column of the row its expert gave it (expert e's
    rows are offsets[e] .. offsets[e+1] - 1, taken by its slots in flat-index
    order; the shared group follows), so out = P @ y (numpy's matmul)."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    start = np.concatenate([[0], np.cumsum(counts)])
    P = np.zeros((T, y.shape[0]))
    seen = np.zeros(E, np.int64)
    for i in range(T * k):                    # slots in flat-index order
        e = flat[i]
        if 0 <= e < E:
            P[i // k, start[e] + seen[e]] += tw.reshape(-1)[i]
            seen[e] += 1
    if has_shared:
        for t in range(T):
            P[t, start[E] + t] += 1.0
    return P @ y.astype(np.float64)


COMBINE_CASES = [(37, 4, 9, False), (29, 8, 32, True), (1, 8, 64, True), (16, 2, 8, False)]


def _combine_case(T, k, E, has_shared, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if T > 3:
        ids[1, 0] = -1                         # masked slots: negative and past E
        ids[2, k - 1] = E + 2
        ids[3, :] = -1                         # a token with every slot masked
    tw = rng.random((T, k)).astype(np.float32) + 0.05
    counts, offsets, eidx, rtok = oracle.permute(ids, E, has_shared)
    y = rng.standard_normal((max(len(rtok), 1), 128)).astype(np.float32)
    wl = synth.Workload("combine", H=128, E=E, topk=k, I=128, wfmt=0, wblk=128, act_group=128,
                        routing="uniform", shared=has_shared, tokens=(T,), wid=0)
    lay = oracle.Layer.for_workload(wl, T, synth.Weights(*(torch.zeros(1, dtype=torch.uint8),) * 4))
    return lay, y, ids, tw, eidx, offsets


def _combine_agrees(T, k, E, has_shared, seed=0) -> bool:
    lay, y, ids, tw, eidx, offsets = _combine_case(T, k, E, has_shared, seed)
    got = lay.combine(y, eidx, offsets, tw)
    ref = _dense_routing_product(y, ids, tw, E, has_shared)
    return bool(np.all(np.abs(got - ref) <= 1e-12 * np.abs(ref).max()))


@pytest.mark.parametrize("T,k,E,has_shared", COMBINE_CASES)
def test_stage_combine_equals_routing_matrix_product(T, k, E, has_shared):
    """oracle_combine (the stage reference) against a dense routing matrix
    times y: masked slots add nothing, each slot's weight multiplies its own
    row, and every token adds its own shared row."""
    assert _combine_agrees(T, k, E, has_shared)
    lay, y, ids, tw, eidx, offsets = _combine_case(T, k, E, has_shared, 0)
    got = lay.combine(y, eidx, offsets, tw)
    if T > 3 and not has_shared:
        assert np.all(got[3] == 0)             # every slot masked, no shared expert


def test_stage_combine_of_layer_rows_equals_layer():
    """The stage combine over the layer's own GEMM2 rows (rounded to fp32)
    reproduces the layer's fp64 combine to fp32 rounding."""
    wl = SMALL["fp8_shared_zipf"]
    T = 7
    w = synth.gen_weights(wl, seed=15)
    x, ids, tw = synth.gen_inputs(wl, T, seed=15)
    lay = oracle.layer_for(wl, T, w)
    xq, xs = oracle.quant_act(x, wl.act_group)
    counts, offsets, eidx, rtok = oracle.permute(ids, wl.E, True)
    R = int(offsets[-1])
    _, hq, hs = lay.gemm1(xq, xs, rtok, offsets, range(R))
    y = lay.gemm2(hq, hs, offsets, range(R)).astype(np.float32)
    got = lay.combine(y, eidx, offsets, tw)
    ref = lay.layer(x, ids, tw)
    assert np.abs(got - ref).max() <= 1e-6 * np.abs(ref).max()


@pytest.mark.parametrize("mutation", [5, 6])
def test_planted_combine_mistakes_are_caught(mutation):
    assert all(_combine_agrees(*c) for c in COMBINE_CASES)
    oracle.set_mutation(mutation)
    try:
        assert not all(_combine_agrees(*c) for c in COMBINE_CASES), f"mutation {mutation} slipped through"
    finally:
        oracle.set_mutation(0)


# ------------------------------------------------------------ worked examples
def _golden_case(ex):
    c = ex["cfg"]
    T, H, I, E = c["T"], c["H"], c["I"], c["E"]
    x = torch.zeros(T, H)
    for t, i, v in ex["x_nonzero"]:
        x[t, i] = v
    x = x.to(torch.bfloat16)
    g = torch.Generator().manual_seed(99)
    if c["wfmt"] == 0:
        b = c["wblk"]
        w1 = torch.zeros(E, 2 * I, H, dtype=torch.uint8)
        w2 = torch.zeros(E, H, I, dtype=torch.uint8)
        w1s = torch.ones(E, 2 * I // b, H // b)
        w2s = torch.ones(E, H // b, I // b)
        w1[0] = torch.randint(0, 126, (2 * I, H), generator=g, dtype=torch.uint8)  # expert 0 noise
        w2[0] = torch.randint(0, 126, (H, I), generator=g, dtype=torch.uint8)
        for e, n, kk, code in ex["w1_codes"]:
            w1[e, n, kk] = code
        for e, nb, kb, s in ex["w1_scales"]:
            w1s[e, nb, kb] = s
        for e, n, kk, code in ex["w2_codes"]:
            w2[e, n, kk] = code
        for e, nb, kb, s in ex["w2_scales"]:
            w2s[e, nb, kb] = s
    else:
        def packed(N, K, ents):
            nib = torch.zeros(E, N, K, dtype=torch.uint8)
            nib[0] = torch.randint(0, 16, (N, K), generator=g, dtype=torch.uint8)
            for e, n, kk, v in ents:
                nib[e, n, kk] = v
            return nib[:, :, 0::2] | (nib[:, :, 1::2] << 4)

        def scales(N, K, ents):
            s = torch.full((E, N, K // 32), 127, dtype=torch.uint8)
            s[0] = torch.randint(120, 130, (N, K // 32), generator=g, dtype=torch.uint8)
            for e, n, kb, v in ents:
                s[e, n, kb] = v
            return s
        w1, w1s = packed(2 * I, H, ex["w1_nibbles"]), scales(2 * I, H, ex["w1_e8m0"])
        w2, w2s = packed(H, I, ex["w2_nibbles"]), scales(H, I, ex["w2_e8m0"])
    ids = torch.tensor(ex["topk_ids"], dtype=torch.int32)
    tw = torch.tensor(ex["topk_weights"], dtype=torch.float32)
    wl = synth.Workload(ex["name"], H=H, E=E, topk=c["k"], I=I, wfmt=c["wfmt"], wblk=c["wblk"],
                        act_group=c["G"], routing="uniform", shared=False, tokens=(T,), wid=0)
    return wl, synth.Weights(w1, w1s, w2, w2s), x, ids, tw


def golden_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", golden_examples(), ids=lambda e: e["name"])
def test_worked_example(ex):
    wl, w, x, ids, tw = _golden_case(ex)
    T = x.shape[0]
    lay = oracle.layer_for(wl, T, w)
    xq, xs = oracle.quant_act(x, wl.act_group)
    nz = [[i, int(v)] for i, v in enumerate(xq[0]) if v != 0]
    assert nz == ex["expect_xq_row0_nonzero"] and xs[0, 0] == ex["expect_xs_row0"]
    counts, offsets, eidx, rtok = oracle.permute(ids, wl.E, False)
    _, hq, hs = lay.gemm1(xq, xs, rtok, offsets, [eidx[0]])
    nz = [[i, int(v)] for i, v in enumerate(hq[0]) if v != 0]
    assert nz == ex["expect_hq_token0_nonzero"] and hs[0, 0] == ex["expect_hs_token0"]
    out = lay.layer(x, ids, tw)
    for t in range(T):
        want = np.zeros(wl.H)
        for i, v in ex["expect_out"][str(t)]:
            want[i] = v
        assert np.array_equal(out[t], want), (t, out[t][:4])
    assert np.array_equal(lay.bruteforce(x, ids, tw), out)


# ------------------------------------------------------------ planted mistakes
def _pins_pass() -> bool:
    """A compact run of the layer pins; False as soon as one fails."""
    try:
        for name in ("tiny_fp8",):
            test_single_expert_equals_plain_mlp(name)
            test_layer_matches_bruteforce(name)
        for ex in golden_examples():
            test_worked_example(ex)
        test_permute_matches_stable_sort(33, 3, 5, False, True)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutation", [1, 2, 3, 4])
def test_planted_mistakes_are_caught(mutation):
    assert _pins_pass()
    oracle.set_mutation(mutation)
    try:
        assert not _pins_pass(), f"mutation {mutation} slipped through every pin"
    finally:
        oracle.set_mutation(0)
