"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Every call goes through the C ABI (bit_grouped_gemm_amd -> libmoe.so).
Index outputs and activation codes must be bit-exact; the layer output
must satisfy |gpu - ref| <= 1e-2 * max|ref| + 1e-3 with ref the oracle's
fp64 result.  Requantised SwiGLU codes cannot be bit-exact (fp32
accumulation order moves h by ulps), so they are checked for agreement and
for being at most one code step away from the oracle's.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


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


# ------------------------------------------------------------------ cases
def reduced(name, **kw):
    return synth.WORKLOADS[name].with_shape(**kw)


REDUCED = {
    # several 128-tiles and a ragged token count in every case
    "tiny_fp8": synth.WORKLOADS["tiny_fp8"],
    "fp8_b128": reduced("decode_fp8", H=512, I=384, E=16, topk=4),
    "fp8_b32": reduced("tiny_fp8", H=384, I=256, E=6, topk=3),
    "mxfp4": reduced("decode_mxfp4", H=512, I=384, E=16, topk=4),
    "fp8_zipf_shared": reduced("decode_fp8_zipf_shared", H=512, I=256, E=32, topk=8),
    "mxfp4_shared": reduced("decode_mxfp4", H=384, I=256, E=12, topk=2, shared=True),
    # long K with few experts: both GEMMs take the split-K path
    "fp8_split": reduced("decode_fp8", H=2048, I=1024, E=8, topk=2),
    "mxfp4_split_shared": reduced("decode_mxfp4", H=2048, I=1024, E=8, topk=2, shared=True),
}

BIG = {
    # many rows per expert select the 256-row x 160-token kernels; the shared group of
    # T rows needs two 160-token passes when T > 160
    "big_mxfp4_shared": reduced("decode_mxfp4", H=512, I=256, E=4, topk=2, shared=True),
    "big_fp8": reduced("decode_fp8", H=512, I=384, E=6, topk=2),
}

# stage-test cases: the decode-kernel cases at a few dozen tokens, and the
# many-row (prefill) kernels at enough tokens per expert to take that path
STAGE = [(n, None) for n in REDUCED] + [(n, 200) for n in BIG]


def stage_case(name):
    return REDUCED[name] if name in REDUCED else BIG[name]


_WCACHE = {}


def weights_for(wl, seed=0):
    """(weights tiled on the GPU for the library, row-major weights on the CPU
    for the oracle)."""
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


def inputs_for(wl, T, seed=0):
    x, ids, tw = synth.gen_inputs(wl, T, seed=seed, device=DEV)
    return x, ids, tw


def tol_check(got, ref, what):
    err = np.abs(got - ref).max() if got.size else 0.0
    bound = 1e-2 * (np.abs(ref).max() if ref.size else 0.0) + 1e-3
    _note(f"  {what}: max|gpu-ref| = {err:.3e}  bound {bound:.3e}")
    assert err <= bound, f"{what}: {err} > {bound}"
    return err


def run_permute(wl, T, x, ids):
    moe = M()
    cfg = moe.Cfg.for_workload(wl, T)
    outs = moe.moe_permute(cfg, x, ids)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


# ------------------------------------------------------------------ tiled weights
def _tile_ref(wfmt, w, s):
    """The tiled layout written out with numpy reshapes: tile (k step, row tile)
    holds lane l = 16 g + m's 16 bytes (row m, K group g) at l * 16; e4m3 tiles
    keep K 64..127 of the step in a second kilobyte; MXFP4 scale byte l is
    (row m, 32-block g)."""
    mats, N, KB = w.shape
    nrt = N // 16
    if wfmt == 0:
        nks = KB // 128
        wt = w.reshape(mats, nrt, 16, nks, 2, 4, 16).transpose(0, 3, 1, 4, 5, 2, 6)
        return wt.reshape(mats, N, KB), s
    nks = KB // 64
    wt = w.reshape(mats, nrt, 16, nks, 4, 16).transpose(0, 3, 1, 4, 2, 5).reshape(mats, N, KB)
    st = s.reshape(mats, nrt, 16, nks, 4).transpose(0, 3, 1, 4, 2).reshape(s.shape)
    return wt, st


@pytest.mark.parametrize("name", ["tiny_fp8", "fp8_b128", "mxfp4", "mxfp4_shared"])
def test_prepack_weights_bitexact(name):
    """Every tensor of moe_prepack_weights against numpy reshapes of the
    documented tiled layout (e4m3 block scales unchanged)."""
    moe = M()
    wl = synth.WORKLOADS.get(name) or REDUCED[name]
    _note(f"prepack {name}")
    w = synth.gen_weights(wl, seed=3, device=DEV)
    cfg = moe.Cfg.for_workload(wl, 1)
    wt = moe.moe_prepack_weights(cfg, w)
    torch.cuda.synchronize()
    pairs = [("w1", "w1s"), ("w2", "w2s")] + ([("sw1", "sw1s"), ("sw2", "sw2s")] if wl.shared else [])
    for wn, sn in pairs:
        ww, ss = getattr(w, wn).cpu().numpy(), getattr(w, sn).cpu().numpy()
        if ww.ndim == 2:
            ww, ss = ww[None], ss[None]
        rw, rs = _tile_ref(wl.wfmt, ww, ss)
        got_w, got_s = getattr(wt, wn).cpu().numpy(), getattr(wt, sn).cpu().numpy()
        assert np.array_equal(got_w.reshape(rw.shape), rw), wn
        assert np.array_equal(got_s.reshape(rs.shape), rs), sn


# ------------------------------------------------------------------ permute + quant
PERMUTE_CASES = [
    ("tiny_fp8", 16), ("decode_fp8", 1), ("decode_fp8", 8), ("decode_fp8", 256),
    ("decode_fp8_zipf_shared", 256), ("prefill_mxfp4", 4096), ("fp8_b32", 37), ("mxfp4_shared", 5),
    # more than 4096 slots: counted and placed in chunks (the last one ragged)
    ("mxfp4_shared", 3000), ("decode_fp8_zipf_shared", 700),
]


@pytest.mark.parametrize("name,T", PERMUTE_CASES)
def test_permute_and_quant_bitexact(name, T):
    wl = synth.WORKLOADS.get(name) or REDUCED[name]
    _note(f"permute {name} T={T}")
    x, ids, _ = inputs_for(wl, T, seed=1)
    counts, offsets, eidx, rtok, xq, xs = run_permute(wl, T, x, ids)
    rc, ro, re_, rr = oracle.permute(ids.cpu(), wl.E, wl.shared)
    assert np.array_equal(counts, rc) and np.array_equal(offsets, ro)
    assert np.array_equal(eidx, re_) and np.array_equal(rtok, rr)
    qx, qs = oracle.quant_act(x.cpu(), wl.act_group)
    assert np.array_equal(xq, qx)
    assert np.array_equal(xs.view(np.uint32), qs.view(np.uint32))


def test_permute_masked_duplicate_and_odd_expert_counts():
    moe = M()
    rng = np.random.default_rng(3)
    for E, k, T in ((5, 3, 300), (64, 8, 1000), (1000, 4, 700), (1, 1, 129), (9, 8, 1100), (1000, 16, 600)):
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)     # duplicates allowed
        ids[rng.random((T, k)) < 0.15] = -1
        ids[0, 0] = E + 7
        for shared in (0, 1):
            cfg = moe.Cfg(T, 128, 128, E, k, 0, 128, 128, shared)
            x = torch.randn(T, 128, device=DEV).to(torch.bfloat16)
            out = moe.moe_permute(cfg, x, torch.from_numpy(ids).to(DEV))
            torch.cuda.synchronize()
            ref = oracle.permute(ids, E, bool(shared))
            for a, b in zip(out[:4], ref):
                assert np.array_equal(a.cpu().numpy(), b), (E, k, T, shared)


def test_quant_special_values_bitexact():
    moe = M()
    T, H = 64, 256
    g = torch.Generator().manual_seed(5)
    x = torch.randn(T, H, generator=g)
    x[0] = 0.0
    x[1, :128] = 1e-38
    x[2, 5] = -0.0
    x[3] *= 1e30
    x[4] = torch.tensor(448.0)
    x[5, :] = torch.arange(H) * 2.0 ** -12
    x[6, ::2] = -x[6, 1::2]
    # every bf16 bit pattern that is finite, paired with a large group maximum
    allb = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    allb = allb[torch.isfinite(allb)]
    xb = x.to(torch.bfloat16)
    for G in (32, 128):
        cfg = moe.Cfg(T, H, 128, 4, 1, 0, G, G, 0)
        ids = torch.zeros(T, 1, dtype=torch.int32, device=DEV)
        got = moe.moe_permute(cfg, xb.to(DEV), ids)
        torch.cuda.synchronize()
        qx, qs = oracle.quant_act(xb, G)
        assert np.array_equal(got[4].cpu().numpy(), qx)
        assert np.array_equal(got[5].cpu().numpy().view(np.uint32), qs.view(np.uint32))
    n = allb.numel()
    Hb = 128
    rows = (n + Hb - 1) // Hb
    flat = torch.zeros(rows * Hb)
    flat[:n] = allb
    xb2 = flat.reshape(rows, Hb).to(torch.bfloat16)
    cfg = moe.Cfg(rows, Hb, 128, 4, 1, 0, 128, 128, 0)
    got = moe.moe_permute(cfg, xb2.to(DEV), torch.zeros(rows, 1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    qx, qs = oracle.quant_act(xb2, 128)
    assert np.array_equal(got[4].cpu().numpy(), qx)
    assert np.array_equal(got[5].cpu().numpy().view(np.uint32), qs.view(np.uint32))


def test_permute_T0():
    moe = M()
    wl = REDUCED["fp8_zipf_shared"]
    cfg = moe.Cfg.for_workload(wl, 0)
    x = torch.empty(0, wl.H, dtype=torch.bfloat16, device=DEV)
    ids = torch.empty(0, wl.topk, dtype=torch.int32, device=DEV)
    counts, offsets, *_ = moe.moe_permute(cfg, x, ids)
    torch.cuda.synchronize()
    assert counts.abs().sum().item() == 0 and offsets.abs().sum().item() == 0


# ------------------------------------------------------------------ stages
def dec_e4m3_np(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("name,T", STAGE)
def test_gemm1_stage(name, T):
    gemm1_stage_check(stage_case(name), T or (37 if name != "tiny_fp8" else 16), name)


def gemm1_stage_check(wl, T, name):
    """GEMM1's h codes and scales against the oracle's GEMM1 of the same
    permuted, quantised activations."""
    moe = M()
    _note(f"gemm1 {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=2)
    cfg = moe.Cfg.for_workload(wl, T)
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    ws = moe.workspace(cfg)
    hq, hs = moe.moe_grouped_gemm1_swiglu(cfg, xq, xs, rtok, offsets, w, ws)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    lay = oracle.layer_for(wl, T, wc)
    h_ref, hq_ref, hs_ref = lay.gemm1(xq.cpu(), xs.cpu(), rtok.cpu(), offsets.cpu(), range(R))
    hq_g, hs_g = hq.cpu().numpy()[:R], hs.cpu().numpy()[:R]
    # group maxima move with the fp32 / MFMA accumulation order, so the scales agree closely
    # but not bitwise
    rel = np.abs(hs_g - hs_ref) / np.abs(hs_ref)
    _note(f"  max rel scale difference {rel.max():.3e}")
    assert rel.max() <= 1e-3, rel.max()
    agree = (hq_g == hq_ref).mean()
    _note(f"  h code agreement {agree:.5f}")
    assert agree >= 0.99
    G = wl.act_group
    dg = dec_e4m3_np(hq_g) * np.repeat(hs_g, G, axis=1)
    dr = dec_e4m3_np(hq_ref) * np.repeat(hs_ref, G, axis=1)
    # a differing code is a neighbour: within one e4m3 step (1/8 relative, or 2^-9 * scale)
    # a differing code is a neighbour (one e4m3 step: 1/8 relative, 2^-9 of the scale when
    # subnormal), up to fp32 accumulation noise measured against the group's full scale 448*hs
    scale = np.repeat(hs_ref, G, axis=1)
    step = np.maximum(np.abs(dr) / 8, 2.0 ** -9 * scale) + 1e-4 * 448 * scale
    bad = np.argwhere(np.abs(dg - dr) > step * 1.0001)
    for r, c in bad[:8]:
        _note(f"  row {r} col {c}: gpu code {hq_g[r, c]:#x} ({dg[r, c]:.6g}) oracle {hq_ref[r, c]:#x} "
              f"({dr[r, c]:.6g}) h {h_ref[r, c]:.6g} scale g/o {hs_g[r, c // G]:.6g}/{hs_ref[r, c // G]:.6g}")
    assert len(bad) == 0
    # and every dequantised GPU value is within one code step of the oracle's unquantised h
    assert np.all(np.abs(dg - h_ref) <= step * 1.0001 + 1e-30)
    _note(f"  max |gpu deq h - oracle h| / group scale = {(np.abs(dg - h_ref) / (448 * scale)).max():.3e}")


@pytest.mark.parametrize("name,T", STAGE)
def test_gemm2_stage(name, T):
    gemm2_stage_check(stage_case(name), T or 29, name)


def gemm2_stage_check(wl, T, name):
    """GEMM2 on the oracle's own h codes against the oracle's GEMM2."""
    moe = M()
    _note(f"gemm2 {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=3)
    cfg = moe.Cfg.for_workload(wl, T)
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    lay = oracle.layer_for(wl, T, wc)
    _, hq_r, hs_r = lay.gemm1(xq.cpu(), xs.cpu(), rtok.cpu(), offsets.cpu(), range(R))
    hq = torch.zeros(rtok.numel(), wl.I, dtype=torch.uint8)
    hs = torch.ones(rtok.numel(), wl.I // wl.act_group)
    hq[:R] = torch.from_numpy(hq_r)
    hs[:R] = torch.from_numpy(hs_r)
    y = moe.moe_grouped_gemm2(cfg, hq.to(DEV), hs.to(DEV), offsets, w)
    torch.cuda.synchronize()
    y_ref = lay.gemm2(hq, hs, offsets.cpu(), range(R))
    # identical codes on both sides: the only difference is accumulation (fp8 products summed
    # inside the MFMA per 128-K block, then fp32 across blocks) against the oracle's fp64
    err = np.abs(y.cpu().numpy()[:R] - y_ref).max()
    _note(f"  gemm2 max|gpu-ref| / max|ref| = {err / np.abs(y_ref).max():.3e}")
    assert err <= 3e-4 * np.abs(y_ref).max(), err


def test_combine_stage():
    moe = M()
    wl = REDUCED["fp8_zipf_shared"]
    T = 41
    x, ids, tw = inputs_for(wl, T, seed=4)
    ids_c = ids.clone()
    ids_c[3, 2] = -1
    cfg = moe.Cfg.for_workload(wl, T)
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids_c)
    y = torch.randn(rtok.numel(), wl.H, device=DEV)
    out = moe.moe_combine(cfg, y, eidx, offsets, tw)
    torch.cuda.synchronize()
    lay = oracle.layer_for(wl, T, weights_for(wl)[1])
    ref = lay.combine(y.cpu(), eidx.cpu(), offsets.cpu(), tw.cpu())
    got = out.float().cpu().numpy()
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


# ------------------------------------------------------------------ whole layer
@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("T", [1, 3, 37])
def test_layer_reduced(name, T):
    moe = M()
    wl = REDUCED[name]
    _note(f"layer {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=6)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    torch.cuda.synchronize()
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    tol_check(out.float().cpu().numpy(), ref, f"{name} T={T}")


@pytest.mark.parametrize("T", [37, 64])
def test_layer_mxfp4_eight_tiles_per_wave(T):
    """MXFP4 decode GEMM2 with eight weight tiles per wave (512-row units):
    H = 2048 and 64 experts keep one unit per CU, and at T = 64 a pass holds
    two token tiles."""
    moe = M()
    wl = reduced("decode_mxfp4", H=2048, I=256, E=64, topk=8)
    _note(f"mxfp4 nj8 T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=31)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    ws = moe.workspace(cfg)
    hq, hs = moe.moe_grouped_gemm1_swiglu(cfg, xq, xs, rtok, offsets, w, ws)
    y = moe.moe_grouped_gemm2(cfg, hq, hs, offsets, w, ws)
    torch.cuda.synchronize()
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    tol_check(out.float().cpu().numpy(), ref, f"mxfp4 nj8 T={T}")
    # GEMM2 on the GPU's own h codes against the oracle's GEMM2 of the same codes
    R = int(offsets[-1].item())
    lay = oracle.layer_for(wl, T, wc)
    y_ref = lay.gemm2(hq.cpu(), hs.cpu(), offsets.cpu(), range(R))
    err = np.abs(y.cpu().numpy()[:R] - y_ref).max()
    assert err <= 3e-4 * np.abs(y_ref).max(), err


FULL = [(n, T) for n in ("decode_fp8", "decode_mxfp4") for T in synth.WORKLOADS[n].tokens] + \
       [("decode_fp8_zipf_shared", T) for T in synth.WORKLOADS["decode_fp8_zipf_shared"].tokens] + \
       [("prefill_mxfp4", 4096)]


def sample_tokens(T, seed):
    """Tokens whose layer output is checked at full size: every token up to
    T = 64, 64 of them up to T = 256 and 256 beyond (always the first and
    the last); tokens are independent once the permute is fixed."""
    n = T if T <= 64 else (64 if T <= 256 else 256)
    rng = np.random.default_rng(seed)
    return sorted(set([0, T - 1] + list(rng.choice(T, size=n, replace=False))))


@pytest.mark.parametrize("name,T", FULL)
def test_layer_full_size_sampled(name, T):
    """Full workload shapes, launched exactly as the bench launches them:
    the permute / quantisation outputs of the same shape and inputs checked
    bit-exact against the oracle, the layer output on sampled tokens (at
    least 64 of 256, 256 of 4096) against the oracle's within the bound."""
    moe = M()
    wl = synth.WORKLOADS[name]
    _note(f"full {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=0)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    out = moe.moe_layer(cfg, x, ids, tw, w, ws=ws)
    perm = moe.moe_permute(cfg, x, ids, ws=moe.workspace(cfg))
    torch.cuda.synchronize()
    counts, offsets, eidx, rtok, xq, xs = [t.cpu().numpy() for t in perm]
    rc, ro, re_, rr = oracle.permute(ids.cpu(), wl.E, wl.shared)
    assert np.array_equal(counts, rc) and np.array_equal(offsets, ro)
    assert np.array_equal(eidx, re_) and np.array_equal(rtok, rr)
    qx, qs = oracle.quant_act(x.cpu(), wl.act_group)
    assert np.array_equal(xq, qx) and np.array_equal(xs.view(np.uint32), qs.view(np.uint32))
    toks = sample_tokens(T, T)
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu(), toks=toks)
    tol_check(out.float().cpu().numpy()[toks], ref, f"{name} T={T} sampled {len(toks)}")
    assert torch.isfinite(out.float()).all()


# ------------------------------------------------------------------ big-tile (prefill) path


@pytest.mark.parametrize("name", list(BIG))
@pytest.mark.parametrize("T", [80, 200, 700])  # 80: 64-row passes (the shared group takes two)
def test_layer_big_tiles(name, T):
    moe = M()
    wl = BIG[name]
    _note(f"big {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=11)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(T + 1)
    toks = sorted(set([0, T - 1] + list(rng.choice(T, size=40, replace=False))))
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu(), toks=toks)
    tol_check(out.float().cpu().numpy()[toks], ref, f"{name} T={T}")
    # the stage calls take the same path
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    ws = moe.workspace(cfg)
    hq, hs = moe.moe_grouped_gemm1_swiglu(cfg, xq, xs, rtok, offsets, w, ws)
    y = moe.moe_grouped_gemm2(cfg, hq, hs, offsets, w, ws)
    out2 = moe.moe_combine(cfg, y.to(torch.bfloat16).float().contiguous(), eidx, offsets, tw)  # layer keeps y in bf16
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    # requantised codes of a sample of rows against the oracle's
    R = int(offsets[-1].item())
    rows = sorted(set(rng.choice(R, size=60, replace=False).tolist() + [R - 1]))
    lay = oracle.layer_for(wl, T, wc)
    _, hq_ref, hs_ref = lay.gemm1(xq.cpu(), xs.cpu(), rtok.cpu(), offsets.cpu(), rows)
    agree = (hq.cpu().numpy()[rows] == hq_ref).mean()
    _note(f"  h code agreement {agree:.5f}")
    assert agree >= 0.99
    assert np.abs(hs.cpu().numpy()[rows] / hs_ref - 1).max() <= 1e-3


# ------------------------------------------------------------------ edge cases
def test_layer_T0_is_a_no_op():
    moe = M()
    wl = REDUCED["fp8_zipf_shared"]
    w, _ = weights_for(wl)
    cfg = moe.Cfg.for_workload(wl, 0)
    out = moe.moe_layer(cfg, torch.empty(0, wl.H, dtype=torch.bfloat16, device=DEV),
                        torch.empty(0, wl.topk, dtype=torch.int32, device=DEV),
                        torch.empty(0, wl.topk, device=DEV), w)
    torch.cuda.synchronize()
    assert out.numel() == 0


def test_layer_masked_slots_and_zero_weights():
    moe = M()
    wl = REDUCED["mxfp4"]
    T = 20
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=8)
    ids[2, 0] = -1
    ids[5, :] = wl.E + 1          # a token with every slot masked: output is exactly zero
    tw[7, 1] = 0.0
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    torch.cuda.synchronize()
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    got = out.float().cpu().numpy()
    tol_check(got, ref, "masked")
    assert np.all(got[5] == 0)


HEAVY = {
    # 32-blocks (never the many-row kernels); long K and few units: split-K in
    # both GEMMs; 64-row passes, so expert 0's T rows are several work items
    "fp8_b32_split": reduced("tiny_fp8", H=2048, I=2048, E=6, topk=3),
    # H not a multiple of 256 keeps MXFP4 on the decode kernels; the shared
    # group's T rows add a second heavy group
    "mxfp4_h1152_shared": reduced("decode_mxfp4", H=1152, I=512, E=6, topk=3, shared=True),
}


@pytest.mark.parametrize("name", list(HEAVY))
def test_layer_one_hot_expert_many_passes(name):
    """Every token routes to expert 0 (its other slots to distinct experts):
    expert 0 holds all T rows, more than one pass of the decode GEMMs, so its
    passes run as separate work items with their own split-K counters."""
    moe = M()
    wl = HEAVY[name]
    T = 150
    _note(f"one-hot expert {name} T={T}")
    w, wc = weights_for(wl)
    x, _, tw = inputs_for(wl, T, seed=12)
    g = torch.Generator().manual_seed(12)
    others = torch.stack([torch.randperm(wl.E - 1, generator=g)[: wl.topk - 1] + 1 for _ in range(T)])
    ids = torch.cat([torch.zeros(T, 1, dtype=torch.int64), others], 1).to(torch.int32).to(DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    torch.cuda.synchronize()
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    tol_check(out.float().cpu().numpy(), ref, f"one-hot {name}")


@pytest.mark.parametrize("name,T", [("big_fp8", 200), ("big_fp8", 700), ("big_mxfp4_shared", 200)])
def test_big_tiles_bitwise_deterministic(name, T):
    """The many-row kernels share LDS tables and ring stages between waves:
    repeated calls (one from a poisoned workspace) must agree bit for bit, which
    the tolerance checks cannot show."""
    moe = M()
    wl = BIG[name]
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=14)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    ws.fill_(0xFF)
    outs = [moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone() for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))


def test_one_hot_expert_poisoned_workspace():
    """The per-item split-K counters of a heavy group are cleared inside every
    call: a workspace filled with 0xFF gives the same bits as a zeroed one."""
    moe = M()
    wl = HEAVY["fp8_b32_split"]
    T = 150
    w, _ = weights_for(wl)
    x, _, tw = inputs_for(wl, T, seed=13)
    g = torch.Generator().manual_seed(13)
    others = torch.stack([torch.randperm(wl.E - 1, generator=g)[: wl.topk - 1] + 1 for _ in range(T)])
    ids = torch.cat([torch.zeros(T, 1, dtype=torch.int64), others], 1).to(torch.int32).to(DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    ws.fill_(0xFF)
    a = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
    ws.fill_(0x00)
    b = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_poisoned_workspace_and_determinism():
    moe = M()
    for name, T in (("fp8_zipf_shared", 37), ("mxfp4", 1), ("fp8_b128", 2)):
        wl = REDUCED[name]
        w, _ = weights_for(wl)
        x, ids, tw = inputs_for(wl, T, seed=9)
        cfg = moe.Cfg.for_workload(wl, T)
        ws = moe.workspace(cfg)
        ws.fill_(0xFF)
        a = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
        ws.fill_(0x00)
        b = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
        c = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(b.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("name,T", [
    ("fp8_zipf_shared", 19),   # one token tile per pass: 128-row GEMM2 units
    ("fp8_b128", 37),          # two token tiles: 256-row GEMM2 units
    ("mxfp4_shared", 37),      # MXFP4 with the shared expert
])
def test_layer_matches_its_stages(name, T):
    """moe_layer equals the four stage calls chained through the C ABI, with
    the GEMM2 rows rounded to bf16 (RNE) before the combine, as the layer
    keeps them internally."""
    moe = M()
    wl = REDUCED[name]
    _note(f"layer == stages {name} T={T}")
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=10)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    ws = moe.workspace(cfg)
    hq, hs = moe.moe_grouped_gemm1_swiglu(cfg, xq, xs, rtok, offsets, w, ws)
    y = moe.moe_grouped_gemm2(cfg, hq, hs, offsets, w, ws)
    out2 = moe.moe_combine(cfg, y.to(torch.bfloat16).float().contiguous(), eidx, offsets, tw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_worked_examples_on_gpu():
    import test_oracle_pins as pins
    moe = M()
    for ex in pins.golden_examples():
        wl, wc, x, ids, tw = pins._golden_case(ex)
        T = x.shape[0]
        cfg = moe.Cfg.for_workload(wl, T)
        out = moe.moe_layer(cfg, x.to(DEV), ids.to(DEV), tw.to(DEV), moe.moe_prepack_weights(cfg, wc.to(DEV)))
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        for t in range(T):
            want = np.zeros(wl.H)
            for i, v in ex["expect_out"][str(t)]:
                want[i] = v
            assert np.array_equal(got[t], want), (ex["name"], t, got[t][:4])


# ------------------------------------------------------------ extreme activation ranges
# (case, T): the decode e4m3 kernels (128- and 32-blocks) and MXFP4 kernels,
# and the many-row e4m3 and MXFP4 kernels (enough rows per expert to select them)
EXTREME = [("fp8_b128", 37), ("fp8_b32", 37), ("mxfp4", 37), ("big_fp8", 200), ("big_mxfp4_shared", 200)]


def extreme_rows(x, G):
    """Overwrite some tokens' 128-groups with all-zero, subnormal and very
    large (1e16 .. 3e17) values, next to ordinary N(0,1) groups, in every
    order: the per-step token scales then differ by up to ~2^130 between
    neighbouring K steps.  h = silu(g) * up stays finite in fp32."""
    x = x.float().clone()
    T, H = x.shape
    ng = H // G
    factors = [0.0, 1e16, 1e-39, 1.0, 3e17, 0.0, 1e-20, 1e16]
    for t in range(0, T, 3):
        for gi in range(ng):
            f = factors[(gi + t) % len(factors)]
            if f != 1.0:
                x[t, gi * G:(gi + 1) * G] *= f
    x[1] = 0.0                                            # an all-zero token
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("name,T", EXTREME)
def test_layer_extreme_activation_ranges(name, T):
    """Rows whose 128-groups mix all-zero, subnormal and very large values,
    on each GEMM kernel path: the output is finite and each token's row
    matches the oracle within the bound taken over that row alone."""
    moe = M()
    wl = stage_case(name)
    _note(f"extreme {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=21)
    x = extreme_rows(x, wl.act_group).to(DEV)
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
    assert np.all(got[1] == ref[1])                       # all-zero token: shared expert / zero exactly


# ------------------------------------------------------------ weight layout flag
def test_canonical_weights_rejected_and_prepack_marks_tiled():
    """moe_layer refuses weights flagged canonical (it reads only the tiled
    layout); moe_prepack_weights flags its output as tiled."""
    moe = M()
    wl = REDUCED["fp8_b128"]
    T = 5
    w = synth.gen_weights(wl, seed=1, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    x, ids, tw = inputs_for(wl, T, seed=1)
    out = torch.full((T, wl.H), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer(cfg, x, ids, tw, w, out=out)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all())               # nothing was enqueued
    wt = moe.moe_prepack_weights(cfg, w)
    assert wt.prepacked == 1
    moe.moe_layer(cfg, x, ids, tw, wt, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


# ------------------------------------------------------------ fp32 -> e4m3 conversion
def test_e4m3_conversion_every_fp32_pattern():
    """The quantisers' hardware fp32 -> e4m3 conversion (saturating, round to
    nearest even, sign kept) against PyTorch's conversion of the value
    clamped to +-448, on every finite fp32 bit pattern (NaN and inf replaced
    by 0), and on a structured CPU sample against PyTorch's CPU conversion
    and the oracle's brute-force encoder."""
    moe = M()
    chunk = 1 << 28
    bad = 0
    for c in range(1 << 32 >> 28):
        _note(f"  e4m3 patterns chunk {c}")
        bits = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device=DEV).to(torch.int32)
        v = bits.view(torch.float32)
        v = torch.where(torch.isfinite(v), v, torch.zeros_like(v))
        got = moe.moe_encode_e4m3(v)
        want = v.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        bad += int((got != want).sum().item())
        del bits, v, got, want
    assert bad == 0, f"{bad} fp32 patterns encode differently"
    # every sign, exponent and top-8 mantissa bits, with four low-bit patterns
    # (round bit and sticky bits set or clear): the rounding boundaries
    hi = torch.arange(1 << 17, dtype=torch.int64) << 15
    pats = torch.cat([hi | lo for lo in (0, 1, 0x4000, 0x7FFF)]).to(torch.int32)
    vals = pats.view(torch.float32)
    vals = vals[torch.isfinite(vals)]
    got = moe.moe_encode_e4m3(vals.to(DEV)).cpu().numpy()
    want = vals.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(got, oracle.enc_e4m3_array(vals.numpy()))


# ------------------------------------------------------------ graph capture
@pytest.mark.parametrize("name,T", [("fp8_b128", 37), ("mxfp4_split_shared", 3), ("big_mxfp4_shared", 200)])
def test_layer_graph_capture_replays_bitexact(name, T):
    """moe_layer enqueues only kernels (no memsets, no host work), so it can
    be captured in a graph: every replay, with unrelated eager layer calls and
    synchronisations in between, equals the direct call bit for bit."""
    moe = M()
    wl = stage_case(name)
    _note(f"graph {name} T={T}")
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=17)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    ws.fill_(0xFF)
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device=DEV)
    ref = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_layer(cfg, x, ids, tw, w, ws=ws, out=out)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.moe_layer(cfg, x, ids, tw, w, ws=ws, out=out)
    x2, ids2, tw2 = inputs_for(wl, T, seed=18)
    for rep in range(4):
        out.zero_()
        ws.fill_(0xA5 if rep % 2 else 0x00)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        moe.moe_layer(cfg, x2, ids2, tw2, w)                # unrelated eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 24) + 16 * 37])
def test_stream_read_reads_every_word(nbytes):
    """The plain read stream folds every 32-bit word of the buffer exactly
    once: the XOR of its sink equals the XOR of the buffer (ragged sizes
    exercise the strided tail)."""
    moe = M()
    _note(f"stream_read nbytes={nbytes}")
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    sink = torch.zeros(8192, dtype=torch.int32, device=DEV)
    moe.moe_stream_read(host.to(DEV), sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("wfmt", [0, 1, 16])
@pytest.mark.parametrize("iters", [1, 777])
def test_mfma_rate_probe_result(wfmt, iters):
    """The MFMA rate probe computes what it claims: every workgroup's sum is
    exactly 4096 * iters (operands 1.0, unit scales, 8 accumulators of 4
    elements, 128 per MFMA), and the reported FLOP count matches the grid."""
    moe = M()
    _note(f"mfma_rate wfmt={wfmt} iters={iters}")
    sink = torch.full((1024,), -1.0, device=DEV)
    flops = moe.moe_mfma_rate(wfmt, iters, sink)
    torch.cuda.synchronize()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    grid = 4 * ncu
    assert flops == grid * 4 * iters * 8 * (16 * 16 * 128 * 2)
    got = sink.cpu().numpy()
    assert np.all(got[:grid] == 4096.0 * iters)
    assert np.all(got[grid:] == -1.0)
