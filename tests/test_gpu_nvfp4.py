"""GPU parity of the NVFP4-weight path (e2m1 codes, an e4m3 scale per 16 along
K, an fp32 scale per expert matrix) against the CPU oracle.

Both kernel families run it: e2m1 codes and activations are turned into fp16
in registers (exact: a code times a block scale has at most six significant
bits) and multiplied on the fp16 MFMA, the matrix scale applied once per
output.  Tolerances as for the other formats.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import (extreme_rows, gemm1_stage_check, gemm2_stage_check, inputs_for, sample_tokens,
                             tol_check, weights_for)

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


def nv(**kw):
    return synth.WORKLOADS["decode_nvfp4"].with_shape(**kw)


CASES = {
    # several 128-tiles, ragged token counts
    "nvfp4": nv(H=512, I=384, E=16, topk=4),
    "nvfp4_shared": nv(H=384, I=256, E=12, topk=2, shared=True),
    # long K with few experts: both GEMMs split K
    "nvfp4_split_shared": nv(H=2048, I=1024, E=8, topk=2, shared=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prepack_nvfp4_bitexact(name):
    """Codes tile as MXFP4's; scales: 128 bytes per tile, row m's eight
    16-blocks of the step at 8 m; matrix scales unchanged."""
    moe = M()
    wl = CASES[name]
    _note(f"prepack {name}")
    w = synth.gen_weights(wl, seed=3, device=DEV)
    wt = moe.moe_prepack_weights(moe.Cfg.for_workload(wl, 1), w)
    torch.cuda.synchronize()
    pairs = [("w1", "w1s", "w1g"), ("w2", "w2s", "w2g")] + \
        ([("sw1", "sw1s", "sw1g"), ("sw2", "sw2s", "sw2g")] if wl.shared else [])
    for wn, sn, gn in pairs:
        ww, ss = getattr(w, wn).cpu().numpy(), getattr(w, sn).cpu().numpy()
        mats, N, KB = ww.shape
        nrt, nks = N // 16, KB // 64
        rw = ww.reshape(mats, nrt, 16, nks, 4, 16).transpose(0, 3, 1, 4, 2, 5).reshape(mats, N, KB)
        rs = ss.reshape(mats, nrt, 16, nks, 8).transpose(0, 3, 1, 2, 4).reshape(ss.shape)
        assert np.array_equal(getattr(wt, wn).cpu().numpy().reshape(rw.shape), rw), wn
        assert np.array_equal(getattr(wt, sn).cpu().numpy().reshape(rs.shape), rs), sn
        assert torch.equal(getattr(wt, gn).cpu(), getattr(w, gn).cpu()), gn


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("T", [1, 3, 37, 200])
def test_layer_nvfp4_reduced(name, T):
    moe = M()
    wl = CASES[name]
    _note(f"layer {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=6)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    torch.cuda.synchronize()
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    tol_check(out.float().cpu().numpy(), ref, f"{name} T={T}")


# T = 200 on "nvfp4" and "nvfp4_split_shared" (50 rows per expert) takes the
# many-row kernels (128-token passes), the rest the decode kernels
@pytest.mark.parametrize("name,T", [("nvfp4", 37), ("nvfp4_shared", 64), ("nvfp4_split_shared", 5),
                                    ("nvfp4", 200), ("nvfp4_split_shared", 200)])
def test_gemm1_stage_nvfp4(name, T):
    gemm1_stage_check(CASES[name], T, name)


@pytest.mark.parametrize("name,T", [("nvfp4", 29), ("nvfp4_shared", 64), ("nvfp4_split_shared", 5),
                                    ("nvfp4", 200), ("nvfp4_split_shared", 200)])
def test_gemm2_stage_nvfp4(name, T):
    gemm2_stage_check(CASES[name], T, name)


@pytest.mark.parametrize("T", [1, 8, 64, 256])
def test_layer_nvfp4_full_size_sampled(T):
    """The decode NVFP4 workload (H=4096, E=64, top-8, I=1536) as the bench
    launches it: sampled tokens against the oracle."""
    moe = M()
    wl = synth.WORKLOADS["decode_nvfp4"]
    _note(f"full decode_nvfp4 T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=0)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w, ws=moe.workspace(cfg))
    torch.cuda.synchronize()
    toks = sample_tokens(T, T)
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu(), toks=toks)
    tol_check(out.float().cpu().numpy()[toks], ref, f"decode_nvfp4 T={T} sampled {len(toks)}")


def test_nvfp4_deterministic_and_layer_equals_stages():
    """Repeated calls with a poisoned workspace are bit-identical, and the
    layer equals its stage calls chained with y rounded to bf16."""
    moe = M()
    wl = CASES["nvfp4_shared"]
    T = 37
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=10)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    ws.fill_(0xFF)
    a = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
    b = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
    counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids)
    hq, hs = moe.moe_grouped_gemm1_swiglu(cfg, xq, xs, rtok, offsets, w, ws)
    y = moe.moe_grouped_gemm2(cfg, hq, hs, offsets, w, ws)
    c = moe.moe_combine(cfg, y.to(torch.bfloat16).float().contiguous(), eidx, offsets, tw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_nvfp4_persistent_is_refused():
    moe = M()
    wl = CASES["nvfp4"]
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, 3, seed=1)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_persistent(moe.Cfg.for_workload(wl, 3), x, ids, tw, w)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED


def test_nvfp4_extreme_activation_ranges():
    """Rows whose 128-groups mix all-zero, subnormal and very large values:
    the fp16 operands stay in range (codes, not values, are converted) and
    every token matches the oracle within the bound taken over its row."""
    moe = M()
    wl = CASES["nvfp4_shared"]
    T = 37
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=21)
    x = extreme_rows(x, wl.act_group).to(DEV)
    out = moe.moe_layer(moe.Cfg.for_workload(wl, T), x, ids, tw, w)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    assert np.isfinite(got).all() and np.abs(ref).max() > 1e20
    err = np.abs(got - ref).max(axis=1)
    assert np.all(err <= 1e-2 * np.abs(ref).max(axis=1) + 1e-3)


def test_nvfp4_one_hot_expert_many_passes_and_masked_slots():
    """Every token on expert 0 (its rows split into many work items, split K)
    plus masked slots; and the no-allocation entry point on the same call."""
    moe = M()
    wl = CASES["nvfp4_split_shared"]
    T = 150
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=33)
    ids = ids.clone()
    ids[:, 0] = 0
    ids[::4, 1] = -1
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w)
    out_s = moe.moe_layer_static(cfg, x, ids, tw, w)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_s.view(torch.int16))
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    tol_check(out.float().cpu().numpy(), ref, "nvfp4 one-hot")


def test_layer_nvfp4_prefill_size_sampled():
    """The prefill shape (T = 4096, H = 7168, E = 256, top-8, I = 2048) with
    NVFP4 weights, on the many-row kernels: 256 sampled tokens against the
    oracle."""
    moe = M()
    wl = synth.WORKLOADS["prefill_nvfp4"]
    T = 4096
    _note("full prefill_nvfp4 T=4096")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=0)
    cfg = moe.Cfg.for_workload(wl, T)
    out = moe.moe_layer(cfg, x, ids, tw, w, ws=moe.workspace(cfg))
    torch.cuda.synchronize()
    toks = sample_tokens(T, T)
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu(), toks=toks)
    tol_check(out.float().cpu().numpy()[toks], ref, f"prefill_nvfp4 sampled {len(toks)}")


@pytest.mark.parametrize("T", [200, 700])
def test_nvfp4_many_row_kernels_deterministic(T):
    """The many-row kernels' waves share LDS stages and tables: repeated
    calls with a poisoned workspace are bit-identical (a race would show as
    differing outputs), and the layer is within the bound of the oracle
    (T = 700: 175 rows per expert, so the larger groups take two passes)."""
    moe = M()
    wl = CASES["nvfp4"]
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=44)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    ws.fill_(0xFF)
    a = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
    ws.fill_(0x00)
    b = moe.moe_layer(cfg, x, ids, tw, w, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    tol_check(a.float().cpu().numpy(), ref, f"nvfp4 many-row T={T}")
