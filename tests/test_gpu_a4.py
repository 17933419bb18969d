"""GPU parity of the 4-bit-activation layer (MXFP4 activations and weights)
against the CPU oracle (needs an MI355X).

Activations are e2m1 codes with one e8m0 scale per 32 channels, so both
GEMMs are FP4 x FP4 on the scaled MFMA.  Index outputs and the activation
codes of the input quantisation are bit-exact.  The requantised SwiGLU codes
come from fp32 accumulation on the GPU and fp64 in the oracle, so they are
checked for agreement and, code by code, for lying within the quantiser's own
error of the oracle's unquantised h.  The layer output meets |gpu - ref| <=
1e-2 * max|ref| + 1e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_grouped_gemm_amd as moe
    moe.load()
    oracle.build(force=False)
    yield


def M():
    import bit_grouped_gemm_amd as moe
    return moe


A4 = synth.WORKLOADS["prefill_mxfp4_a4"]
CASES = {
    # 6 experts x top-2: ~T/3 rows per expert; the many-row kernels at every T
    "a4": A4.with_shape(H=512, I=384, E=6, topk=2),
    "a4_shared": A4.with_shape(H=768, I=256, E=4, topk=2, shared=True),
    # many sparse experts: most groups below 16 rows, padded token tiles
    "a4_sparse": A4.with_shape(H=256, I=128, E=64, topk=8),
}

_WCACHE = {}


def weights_for(wl, seed=0):
    key = (wl, seed)
    if key not in _WCACHE:
        if len(_WCACHE) > 3:
            _WCACHE.clear()
            torch.cuda.empty_cache()
        w = synth.gen_weights(wl, seed=seed, device=DEV)
        moe = M()
        wt = moe.moe_prepack_weights(moe.Cfg.for_workload(wl, 1), w)
        _WCACHE[key] = (wt, w.to("cpu"))
        del w
    return _WCACHE[key]


def tol_check(got, ref, what):
    err = np.abs(got - ref).max() if got.size else 0.0
    bound = 1e-2 * (np.abs(ref).max() if ref.size else 0.0) + 1e-3
    _note(f"  {what}: max|gpu-ref| = {err:.3e}  bound {bound:.3e}")
    assert err <= bound, f"{what}: {err} > {bound}"


def unpack(q):
    """[n, c/2] packed e2m1 bytes -> [n, c] codes (even channel from the low nibble)."""
    q = np.asarray(q, np.uint8)
    out = np.empty((q.shape[0], 2 * q.shape[1]), np.uint8)
    out[:, 0::2] = q & 15
    out[:, 1::2] = q >> 4
    return out


def dequant(q, s):
    codes = unpack(q)
    X = np.ldexp(1.0, np.asarray(s, np.int64) - 127)
    return E2M1[codes] * np.repeat(X, 32, axis=1)


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


# ------------------------------------------------------------ input quantisation
def _special_rows():
    """Rows of 256 channels covering every finite bf16 value: in bit order
    (groups of 32 neighbouring values, subnormal groups included) and in a
    seeded shuffle, plus hand-made groups (zeros, -0, rounding ties of every
    e2m1 boundary, values past 6 X)."""
    allb = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    allb = allb[torch.isfinite(allb)].numpy()
    rng = np.random.default_rng(9)
    parts = [allb, rng.permutation(allb)]
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.5, 0.0, -0.0, -0.25, -0.75, -1.25, -1.75,
                     -2.5, -3.5, -5.0, 4.0, 2.0, 1.0, 0.5, 0.125, 7.9375, 3.0, 6.0, -6.0, -7.9375, 1.5, 2.25,
                     0.3125, 5.5], np.float32)
    hand = [np.zeros(32, np.float32), -np.zeros(32, np.float32), ties, ties * 2.0 ** -100, ties * 2.0 ** 100,
            ties * 2.0 ** -130]
    parts.append(np.concatenate(hand))
    flat = np.concatenate(parts)
    n = (flat.size + 255) // 256 * 256
    flat = np.concatenate([flat, np.zeros(n - flat.size, np.float32)])
    return flat.reshape(-1, 256)


@pytest.mark.parametrize("case", ["random", "special"])
def test_a4_quant_bitexact(case):
    moe = M()
    if case == "random":
        g = torch.Generator().manual_seed(4)
        T, H = 97, 512
        x = torch.randn(T, H, generator=g) * torch.exp(4 * torch.randn(T, 1, generator=g))
        x = x.to(torch.bfloat16)
    else:
        x = _bf16(_special_rows())
        T, H = x.shape
    _note(f"a4 quant {case} T={T} H={H}")
    wl = A4.with_shape(H=H, I=128, E=4, topk=1)
    cfg = moe.Cfg.for_workload(wl, T)
    ids = torch.zeros(T, 1, dtype=torch.int32, device=DEV)
    out = moe.moe_permute(cfg, x.to(DEV), ids)
    torch.cuda.synchronize()
    qx, qs = oracle.quant_act_mx(x)
    got_q, got_s = out[4].cpu().numpy(), out[5].cpu().numpy()
    assert got_q.shape == qx.shape and got_s.shape == qs.shape
    bad = np.argwhere(got_q != qx)
    for r, c in bad[:8]:
        _note(f"  row {r} byte {c}: gpu {got_q[r, c]:#04x} oracle {qx[r, c]:#04x} scale {qs[r, c // 16]}")
    assert np.array_equal(got_s, qs)
    assert len(bad) == 0


# ------------------------------------------------------------ GEMM stages
def _half_step(u):
    """Largest rounding error of the e2m1 quantiser at |v| / X = u (in units
    of X): half the code spacing, or the clamp's error past 6."""
    return np.where(u < 2, 0.25, np.where(u < 4, 0.5, np.maximum(1.0, u - 6.0)))


@pytest.mark.parametrize("name,T", [("a4", 1), ("a4", 37), ("a4", 200), ("a4_shared", 700), ("a4_sparse", 300)])
def test_a4_gemm1_stage(name, T):
    moe = M()
    wl = CASES[name]
    _note(f"a4 gemm1 {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = synth.gen_inputs(wl, T, seed=2, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    ws = moe.workspace(cfg)
    hq, hs = moe.moe_grouped_gemm1_swiglu(cfg, xq, xs, rtok, offsets, w, ws)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    lay = oracle.layer_for(wl, T, wc)
    h_ref, hq_ref, hs_ref = lay.gemm1(xq.cpu(), xs.cpu(), rtok.cpu(), offsets.cpu(), range(R))
    hq_g, hs_g = hq.cpu().numpy()[:R], hs.cpu().numpy()[:R]
    # scale codes: equal, except where the group's maximum sits at a power of two
    # (fp32 against fp64 accumulation moves h by a few ulps)
    ds = hs_g.astype(np.int64) - hs_ref.astype(np.int64)
    amax = np.abs(h_ref.astype(np.float64)).reshape(R, -1, 32).max(axis=2)
    near = np.abs(np.log2(np.maximum(amax, 1e-300)) - np.round(np.log2(np.maximum(amax, 1e-300)))) < 1e-4
    _note(f"  scale codes differing {np.count_nonzero(ds)} of {ds.size}")
    assert np.all(np.abs(ds) <= 1) and np.all(near[ds != 0])
    agree = (hq_g == hq_ref).mean()
    _note(f"  h byte agreement {agree:.5f}")
    assert agree >= 0.99
    # every dequantised GPU value within the quantiser's error of the oracle's h
    dg = dequant(hq_g, hs_g)
    X = np.repeat(np.ldexp(1.0, hs_g.astype(np.int64) - 127), 32, axis=1)
    u = np.abs(h_ref) / X
    allow = _half_step(u * (1 + 1e-3)) * X * (1 + 1e-3) + 6e-5 * X
    err = np.abs(dg - h_ref)
    bad = np.argwhere(err > allow)
    for r, c in bad[:8]:
        _note(f"  row {r} col {c}: gpu {dg[r, c]:.6g} oracle h {h_ref[r, c]:.6g} X {X[r, c]:.3g}")
    assert len(bad) == 0


@pytest.mark.parametrize("name,T", [("a4", 37), ("a4", 200), ("a4_shared", 700)])
def test_a4_gemm2_stage(name, T):
    moe = M()
    wl = CASES[name]
    _note(f"a4 gemm2 {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = synth.gen_inputs(wl, T, seed=3, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    lay = oracle.layer_for(wl, T, wc)
    _, hq_r, hs_r = lay.gemm1(xq.cpu(), xs.cpu(), rtok.cpu(), offsets.cpu(), range(R))
    hq = torch.zeros(rtok.numel(), wl.I // 2, dtype=torch.uint8)
    hs = torch.full((rtok.numel(), wl.I // 32), 127, dtype=torch.uint8)
    hq[:R] = torch.from_numpy(hq_r)
    hs[:R] = torch.from_numpy(hs_r)
    y = moe.moe_grouped_gemm2(cfg, hq.to(DEV), hs.to(DEV), offsets, w)
    torch.cuda.synchronize()
    y_ref = lay.gemm2(hq, hs, offsets.cpu(), range(R))
    # the same codes on both sides: only the accumulation differs (fp4 products summed exactly
    # inside the MFMA per 128-K step, fp32 across steps)
    err = np.abs(y.cpu().numpy()[:R] - y_ref).max()
    _note(f"  gemm2 max|gpu-ref| / max|ref| = {err / np.abs(y_ref).max():.3e}")
    assert err <= 3e-4 * np.abs(y_ref).max(), err


# ------------------------------------------------------------ whole layer
@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("T", [1, 3, 37, 200, 700])
def test_a4_layer(name, T):
    moe = M()
    wl = CASES[name]
    _note(f"a4 layer {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = synth.gen_inputs(wl, T, seed=6, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(T + 5)
    toks = sorted(set([0, T - 1] + list(rng.choice(T, size=min(T, 48), replace=False))))
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu(), toks=toks)
    tol_check(out.float().cpu().numpy()[toks], ref, f"{name} T={T}")
    # the stage calls take the same path
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    ws = moe.workspace(cfg)
    hq, hs = moe.moe_grouped_gemm1_swiglu(cfg, xq, xs, rtok, offsets, w, ws)
    y = moe.moe_grouped_gemm2(cfg, hq, hs, offsets, w, ws)
    out2 = moe.moe_combine(cfg, y.to(torch.bfloat16).float().contiguous(), eidx, offsets, tw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_a4_layer_bitwise_deterministic():
    moe = M()
    wl = CASES["a4_shared"]
    T = 700
    w, _ = weights_for(wl)
    x, ids, tw = synth.gen_inputs(wl, T, seed=8, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    a = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
    ws.fill_(0x5A)
    b = moe.moe_layer(cfg, x, ids, tw, w, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_a4_layer_extreme_activation_ranges():
    """Tokens whose 32-groups mix all-zero, subnormal and very large values
    (the e8m0 scales then span the whole code range): finite output, each
    token within the bound taken over its own row."""
    moe = M()
    wl = CASES["a4_shared"]
    T = 200
    w, wc = weights_for(wl)
    x, ids, tw = synth.gen_inputs(wl, T, seed=21, device=DEV)
    x = x.float().cpu().clone()
    factors = [0.0, 1e16, 1e-39, 1.0, 3e17, 0.0, 1e-20, 1e16]
    for t in range(0, T, 3):
        for gi in range(wl.H // 32):
            f = factors[(gi + t) % len(factors)]
            if f != 1.0:
                x[t, gi * 32:(gi + 1) * 32] *= f
    x[1] = 0.0
    x = x.to(torch.bfloat16).to(DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    assert np.isfinite(ref).all() and np.abs(ref).max() > 1e20
    err = np.abs(got - ref).max(axis=1)
    bound = 1e-2 * np.abs(ref).max(axis=1) + 1e-3
    worst = int(np.argmax(err / bound))
    _note(f"  worst token {worst}: err {err[worst]:.3e} bound {bound[worst]:.3e}")
    assert np.all(err <= bound)
    assert np.all(got[1] == ref[1])


def test_a4_full_size_sampled():
    """The 4-bit-activation prefill workload at its full shape (T = 4096,
    H = 7168, E = 256, top-8, I = 2048), launched as the bench launches it:
    permute and quantisation bit-exact, the layer on 256 sampled tokens
    within the bound."""
    moe = M()
    wl = A4
    T = 4096
    _note(f"a4 full T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = synth.gen_inputs(wl, T, seed=0, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    out = moe.moe_layer(cfg, x, ids, tw, w, ws=ws)
    perm = moe.moe_permute(cfg, x, ids, ws=moe.workspace(cfg))
    torch.cuda.synchronize()
    counts, offsets, eidx, rtok, xq, xs = [t.cpu().numpy() for t in perm]
    rc, ro, re_, rr = oracle.permute(ids.cpu(), wl.E, wl.shared)
    assert np.array_equal(counts, rc) and np.array_equal(offsets, ro)
    assert np.array_equal(eidx, re_) and np.array_equal(rtok, rr)
    qx, qs = oracle.quant_act_mx(x.cpu())
    assert np.array_equal(xq, qx) and np.array_equal(xs, qs)
    rng = np.random.default_rng(T)
    toks = sorted(set([0, T - 1] + list(rng.choice(T, size=256, replace=False))))
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu(), toks=toks)
    tol_check(out.float().cpu().numpy()[toks], ref, f"a4 full T={T} sampled {len(toks)}")
    assert torch.isfinite(out.float()).all()
