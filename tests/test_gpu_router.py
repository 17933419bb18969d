"""GPU parity of the router (moe_route) against the oracle's router (needs
an MI355X).  Every call goes through the C ABI.

The kernel sums logits in fp32 (bf16 products are exact), the oracle in
fp64.  For token t every logit's fp32 error is at most eps_t = H * 2^-24 *
max_e sum_h |x[t][h] w[e][h]| (any summation order), so: where the oracle's
sorted logits of ranks 0..k are more than 2 eps_t apart, the ids must be
bit-exact, order included; elsewhere the GPU's ids must be a valid top-k
within 2 eps_t.  Weights: within 1e-4 of the oracle's (they are in (0, 1]).
"""
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


def check_router(x, wg, k, ids, w):
    """Compare GPU (ids, w) with the oracle on the same bf16 inputs; returns
    (tokens past the rounding margin, tokens whose ids equal the oracle's)."""
    T, H = x.shape
    E = wg.shape[0]
    rid, rw, lg = oracle.router(x.cpu(), wg.cpu(), k)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    absdot = np.abs(x.cpu().float().double().numpy()) @ np.abs(wg.cpu().float().double().numpy()).T
    eps = H * 2.0 ** -24 * absdot.max(axis=1) * 1.01
    srt = -np.sort(-lg, axis=1)[:, : min(k + 1, E)]
    gap = np.abs(np.diff(srt, axis=1)).min(axis=1) if srt.shape[1] > 1 else np.full(T, np.inf)
    clear = gap > 2 * eps
    assert np.array_equal(ids[clear], rid[clear]), "ids differ on tokens with clear logit gaps"
    for t in np.nonzero(~clear)[0]:
        row = ids[t]
        assert len(set(row.tolist())) == k and row.min() >= 0 and row.max() < E
        chosen = lg[t, row]
        assert np.all(np.diff(chosen) <= 2 * eps[t])                     # descending within rounding
        rest = np.delete(lg[t], row)
        if rest.size:
            assert chosen.min() >= rest.max() - 2 * eps[t]                # a valid top-k
    same = np.all(ids == rid, axis=1)
    assert np.abs(w[same] - rw[same]).max(initial=0.0) <= 1e-4
    assert np.allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=1e-5)
    return int(clear.sum()), int(same.sum())


CASES = [
    # up to 512 tokens: partial logits of many workgroups, then the selection kernel
    ("decode_fp8", 1), ("decode_fp8", 37), ("decode_fp8", 256), ("decode_fp8", 512), ("prefill_mxfp4", 64),
    # above: 64-token tiles staged through LDS with K splits (E = 64: one expert tile per wave; E = 256:
    # four), then the same selection kernel
    ("decode_fp8", 600), ("prefill_mxfp4", 1000), ("prefill_mxfp4", 4096),
]


@pytest.mark.parametrize("name,T", CASES)
def test_route_matches_oracle(name, T):
    moe = M()
    wl = synth.WORKLOADS[name]
    _note(f"route {name} T={T}")
    wg = synth.gen_gate(wl, seed=1, device=DEV)
    x = synth.gen_x(T, wl.H, 1, wl.wid, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    ids, w = moe.moe_route(cfg, x, wg)
    torch.cuda.synchronize()
    n, same = check_router(x, wg, wl.topk, ids, w)
    _note(f"  {n} of {T} tokens past the rounding margin (bit-exact); {same} of {T} equal to the oracle's")
    # the margin is a worst-case bound; actual fp32 errors are ~1e-6, so
    # nearly every token's ids equal the oracle's
    assert same >= (T if T < 10 else 0.9 * T)


@pytest.mark.parametrize("H,E,k,T", [(512, 72, 16, 33), (256, 8, 2, 19), (256, 12, 12, 5), (128, 256, 32, 50),
                                     # above 512 tokens: one to four expert tiles per wave, ragged token
                                     # tiles, two 64-K stages (H = 128) up to many
                                     (512, 72, 16, 700), (384, 40, 6, 530), (256, 160, 8, 777), (128, 130, 4, 600),
                                     (1024, 256, 8, 1089)])
def test_route_odd_shapes(H, E, k, T):
    """E not a multiple of 16, k = E, k = 32, tiny E; both kernel paths."""
    moe = M()
    g = torch.Generator(device=DEV).manual_seed(H + E + k)
    x = torch.randn(T, H, generator=g, device=DEV).to(torch.bfloat16)
    wg = (torch.randn(E, H, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    cfg = moe.Cfg(T, H, 128, E, k, 0, 128, 128, 0)
    ids, w = moe.moe_route(cfg, x, wg)
    torch.cuda.synchronize()
    check_router(x, wg, k, ids, w)


@pytest.mark.parametrize("T,E,dup", [
    (40, 64, [(2, 50), (9, 10), (30, 31), (31, 63)]),
    # above 512 tokens (LDS-tiled GEMM, wave-per-token selection); with E = 256
    # the tied experts sit in different 64-id groups of the selection's ballots
    (700, 64, [(2, 50), (9, 10), (30, 31), (31, 63)]),
    (600, 256, [(2, 200), (70, 71), (130, 255), (64, 192)]),
])
def test_route_exact_ties_go_to_the_lower_id(T, E, dup):
    """Duplicated gate rows give equal logits on both sides: the lower expert
    id must come first, bit-exact."""
    moe = M()
    H, k = 512, 8
    g = torch.Generator(device=DEV).manual_seed(9)
    x = torch.randn(T, H, generator=g, device=DEV).to(torch.bfloat16)
    wg = (torch.randn(E, H, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    for a, b in dup:
        wg[b] = wg[a]
    x[0] = 0.0                                    # every logit 0: ids 0..k-1, weights 1/k
    cfg = moe.Cfg(T, H, 128, E, k, 0, 128, 128, 0)
    ids, w = moe.moe_route(cfg, x, wg)
    torch.cuda.synchronize()
    check_router(x, wg, k, ids, w)
    ids = ids.cpu().numpy()
    assert np.array_equal(ids[0], np.arange(k)) and np.all(w[0].cpu().numpy() == np.float32(1.0 / k))
    for t in range(T):
        row = ids[t].tolist()
        for a, b in dup:
            if a in row and b in row:
                assert row.index(a) < row.index(b), (t, row)


def test_route_feeds_the_layer():
    """moe_route's outputs drive moe_layer: equal to the oracle layer run on
    the oracle router's ids and weights, within the layer bound."""
    moe = M()
    wl = synth.WORKLOADS["decode_mxfp4"].with_shape(H=512, I=384, E=16, topk=4)
    T = 29
    wg = synth.gen_gate(wl, seed=2, device=DEV)
    x = synth.gen_x(T, wl.H, 2, wl.wid, device=DEV)
    w = synth.gen_weights(wl, seed=2, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    ids, tw = moe.moe_route(cfg, x, wg)
    out = moe.moe_layer(cfg, x, ids, tw, moe.moe_prepack_weights(cfg, w))
    torch.cuda.synchronize()
    rid, rw, _ = oracle.router(x.cpu(), wg.cpu(), wl.topk)
    assert np.array_equal(ids.cpu().numpy(), rid)
    ref = oracle.layer_for(wl, T, w.to("cpu")).layer(x.cpu(), rid, rw)
    got = out.float().cpu().numpy()
    assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max() + 1e-3


def test_route_T0_and_rejects_large_E():
    moe = M()
    cfg = moe.Cfg(0, 256, 128, 8, 2, 0, 128, 128, 0)
    ids, w = moe.moe_route(cfg, torch.empty(0, 256, dtype=torch.bfloat16, device=DEV),
                           torch.zeros(8, 256, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert ids.numel() == 0
    big = moe.Cfg(4, 256, 128, 300, 8, 0, 128, 128, 0)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(big, torch.zeros(4, 256, dtype=torch.bfloat16, device=DEV),
                      torch.zeros(300, 256, dtype=torch.bfloat16, device=DEV))
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("name,T", [("decode_fp8", 1), ("decode_fp8", 200), ("decode_fp8", 700),
                                    ("prefill_mxfp4", 1000)])
def test_route_deterministic_with_poisoned_workspace(name, T):
    """Repeated calls, the workspace refilled with garbage in between, give
    bit-identical ids and weights (the partial logits are summed in a fixed
    order, whatever the workspace held)."""
    moe = M()
    wl = synth.WORKLOADS[name]
    wg = synth.gen_gate(wl, seed=3, device=DEV)
    x = synth.gen_x(T, wl.H, 3, wl.wid, device=DEV)
    cfg = moe.Cfg.for_workload(wl, T)
    n = moe.moe_route_workspace_size(cfg)
    assert n > 0
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)
    ids0, w0 = moe.moe_route(cfg, x, wg, ws=ws)
    ids0, w0 = ids0.clone(), w0.clone()
    ws.fill_(0x7F)
    ids1, w1 = moe.moe_route(cfg, x, wg, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(ids0, ids1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))
