"""GPU checks of the persistent decode layer (moe_layer_persistent: the
routing launch, then GEMM1, GEMM2 and the combine in one launch whose units
are ordered by a ticket counter and chained by device-side counters).

It runs the same kernels' arithmetic as moe_layer, so its output must equal
moe_layer's bit for bit, and the oracle's within the layer bound.  Its
control block lives in the workspace and is zeroed by the routing launch:
repeated calls with changing shapes, poisoned workspaces, launches queued
back to back and graph replays check that.  Every call reports its expired
waits through `status`, which must be 0.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import REDUCED, inputs_for, reduced, sample_tokens, tol_check, weights_for

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


def persistent(cfg, x, ids, tw, w, ws=None, out=None):
    moe = M()
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    out = moe.moe_layer_persistent(cfg, x, ids, tw, w, ws=ws, out=out, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a wait expired"
    return out


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("T", [1, 3, 37])
def test_persistent_equals_layer_reduced(name, T):
    """Reduced shapes of every decode format (e4m3 128- and 32-blocks, MXFP4,
    the shared expert, split K in both GEMMs): bit-identical to moe_layer,
    within the bound of the oracle."""
    moe = M()
    wl = REDUCED[name]
    _note(f"persistent {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=6)
    cfg = moe.Cfg.for_workload(wl, T)
    ref_gpu = moe.moe_layer(cfg, x, ids, tw, w)
    out = persistent(cfg, x, ids, tw, w)
    assert same_bits(out, ref_gpu)
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    tol_check(out.float().cpu().numpy(), ref, f"persistent {name} T={T}")


FULL = [("decode_fp8", T) for T in (1, 8, 64)] + [("decode_mxfp4", T) for T in (1, 8, 64)] + \
       [("decode_fp8_zipf_shared", T) for T in (1, 16, 64)]


@pytest.mark.parametrize("name,T", FULL)
def test_persistent_full_size(name, T):
    """The full decode workloads: bit-identical to moe_layer; every token
    (T <= 64) within the bound of the oracle."""
    moe = M()
    wl = synth.WORKLOADS[name]
    _note(f"persistent full {name} T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=0)
    cfg = moe.Cfg.for_workload(wl, T)
    ref_gpu = moe.moe_layer(cfg, x, ids, tw, w)
    out = persistent(cfg, x, ids, tw, w)
    assert same_bits(out, ref_gpu)
    toks = sample_tokens(T, T)
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu(), toks=toks)
    tol_check(out.float().cpu().numpy()[toks], ref, f"persistent {name} T={T}")


@pytest.mark.parametrize("T", [37, 64])
def test_persistent_mxfp4_eight_tiles_per_wave(T):
    """MXFP4 with eight GEMM2 weight tiles per wave (the instantiation built
    for two workgroups per CU)."""
    moe = M()
    wl = reduced("decode_mxfp4", H=2048, I=256, E=64, topk=8)
    _note(f"persistent mxfp4 nj8 T={T}")
    w, wc = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=31)
    cfg = moe.Cfg.for_workload(wl, T)
    out = persistent(cfg, x, ids, tw, w)
    assert same_bits(out, moe.moe_layer(cfg, x, ids, tw, w))
    ref = oracle.layer_for(wl, T, wc).layer(x.cpu(), ids.cpu(), tw.cpu())
    tol_check(out.float().cpu().numpy(), ref, f"persistent mxfp4 nj8 T={T}")


def test_persistent_consecutive_calls_and_poisoned_workspaces():
    """Consecutive calls with changing token counts, formats and poisoned
    workspaces (the routing launch zeroes the control block): each equals
    moe_layer."""
    moe = M()
    seq = [("fp8_b128", 37), ("fp8_b128", 1), ("mxfp4_shared", 64), ("fp8_split", 5), ("fp8_b128", 37),
           ("fp8_zipf_shared", 2), ("mxfp4_split_shared", 3)]
    for i, (name, T) in enumerate(seq):
        wl = REDUCED[name]
        _note(f"persistent sequence {i}: {name} T={T}")
        w, _ = weights_for(wl)
        x, ids, tw = inputs_for(wl, T, seed=40 + i)
        cfg = moe.Cfg.for_workload(wl, T)
        ws = moe.workspace(cfg)
        ws.fill_(0xFF if i % 2 else 0xA5)
        out = persistent(cfg, x, ids, tw, w, ws=ws)
        assert same_bits(out, moe.moe_layer(cfg, x, ids, tw, w)), f"call {i}"


def test_persistent_back_to_back_without_sync():
    """Eight launches queued back to back on one stream (no host
    synchronisation between them), alternating two inputs: every output
    equals moe_layer's for its inputs."""
    moe = M()
    wl = REDUCED["fp8_zipf_shared"]
    T = 19
    w, _ = weights_for(wl)
    ins = [inputs_for(wl, T, seed=s) for s in (50, 51)]
    cfg = moe.Cfg.for_workload(wl, T)
    refs = [moe.moe_layer(cfg, *inp, w).clone() for inp in ins]
    status = torch.full((8,), -1, dtype=torch.int32, device=DEV)
    outs = []
    _note("persistent back-to-back x8")
    for i in range(8):
        outs.append(moe.moe_layer_persistent(cfg, *ins[i % 2], w, status=status[i:i + 1]))
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * 8
    for i, o in enumerate(outs):
        assert same_bits(o, refs[i % 2]), f"launch {i}"


@pytest.mark.parametrize("name,T", [("fp8_b128", 37), ("mxfp4_split_shared", 3)])
def test_persistent_graph_capture_replays_bitexact(name, T):
    """The launch can be captured in a graph: every replay, with eager calls of
    both layer entry points in between, equals moe_layer bit for bit."""
    moe = M()
    wl = REDUCED[name]
    _note(f"persistent graph {name} T={T}")
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=17)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg)
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device=DEV)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    ref = moe.moe_layer(cfg, x, ids, tw, w).clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_layer_persistent(cfg, x, ids, tw, w, ws=ws, out=out, status=status)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.moe_layer_persistent(cfg, x, ids, tw, w, ws=ws, out=out, status=status)
    x2, ids2, tw2 = inputs_for(wl, T, seed=18)
    for rep in range(4):
        out.zero_()
        status.fill_(-1)
        ws.fill_(0xA5 if rep % 2 else 0x00)
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert same_bits(out, ref), f"replay {rep}"
        persistent(cfg, x2, ids2, tw2, w)
        moe.moe_layer(cfg, x2, ids2, tw2, w)
        torch.cuda.synchronize()


def test_persistent_masked_slots_and_empty_experts():
    """Masked (-1) slots and most experts empty: the no-op work items of
    GEMM2 still count in, so the launch completes and equals moe_layer."""
    moe = M()
    wl = REDUCED["fp8_b128"]
    T = 9
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=22)
    ids = ids.clone()
    ids[:, 1:] = -1          # one slot per token
    ids[::2, 0] = 3          # half the tokens on expert 3
    cfg = moe.Cfg.for_workload(wl, T)
    out = persistent(cfg, x, ids, tw, w)
    assert same_bits(out, moe.moe_layer(cfg, x, ids, tw, w))


def test_persistent_chunked_permute():
    """More than 4096 slots (the permute places them in chunks) on the decode
    kernels: 1024 experts, top-8, T = 600 -- bit-identical to moe_layer."""
    moe = M()
    wl = reduced("decode_fp8", H=512, I=256, E=1024, topk=8)
    T = 600
    _note(f"persistent chunked permute T={T}")
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=23)
    cfg = moe.Cfg.for_workload(wl, T)
    out = persistent(cfg, x, ids, tw, w)
    assert same_bits(out, moe.moe_layer(cfg, x, ids, tw, w))


def test_persistent_expired_wait_is_reported_and_the_launch_ends():
    """Forced from the host: with a spin limit of 0 every wait that finds its
    producer unfinished expires at once.  The launch still ends (the stream
    synchronises), the status word reports the expiry, and the next call with
    the default limit is valid again (the routing launch zeroes the control
    block)."""
    moe = M()
    wl = REDUCED["fp8_b128"]
    T = 37
    w, _ = weights_for(wl)
    x, ids, tw = inputs_for(wl, T, seed=60)
    cfg = moe.Cfg.for_workload(wl, T)
    ref = moe.moe_layer(cfg, x, ids, tw, w).clone()
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    _note("persistent spin limit 0")
    moe.moe_layer_persistent_spin_limit(0)
    try:
        moe.moe_layer_persistent(cfg, x, ids, tw, w, status=status)
        torch.cuda.synchronize()
    finally:
        moe.moe_layer_persistent_spin_limit(moe.PERSIST_SPIN_LIMIT)
    assert int(status.item()) >= 1
    out = persistent(cfg, x, ids, tw, w)
    assert same_bits(out, ref)
