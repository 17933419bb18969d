"""The entry point that allocates nothing (moe_layer_static) against
moe_layer, through the C ABI (needs an MI355X).

moe_layer_static runs moe_layer's kernels over the library's static
per-GPU scratch array instead of a caller's workspace, so its output must
equal moe_layer's bit for bit.  Each case makes two calls in a row, the
second with fewer tokens: the array keeps the first call's contents, which
must not leak into the second.
"""
import sys

import pytest
import torch

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
    yield


def M():
    import bit_grouped_gemm_amd as moe
    return moe


CASES = {
    # decode kernels, several tiles and ragged token counts
    "decode_fp8_reduced": (synth.WORKLOADS["decode_fp8"].with_shape(H=512, I=384, E=16, topk=4), 64, 9),
    # long K, few experts: split-K with arrival counters in the scratch array
    "mxfp4_split_shared": (synth.WORKLOADS["decode_mxfp4"].with_shape(H=2048, I=1024, E=8, topk=2, shared=True),
                           3, 1),
    # many rows per expert: the many-row kernels
    "many_row_mxfp4_shared": (synth.WORKLOADS["decode_mxfp4"].with_shape(H=512, I=256, E=4, topk=2, shared=True),
                              300, 200),
    # the full decode FP8 shape
    "decode_fp8": (synth.WORKLOADS["decode_fp8"], 64, 8),
}


@pytest.mark.parametrize("name", list(CASES))
def test_static_scratch_layer_equals_workspace_layer(name):
    moe = M()
    wl, T1, T2 = CASES[name]
    w = moe.moe_prepack_weights(moe.Cfg.for_workload(wl, 1), synth.gen_weights(wl, seed=0, device=DEV))
    for T in (T1, T2):
        _note(f"static scratch {name} T={T}")
        x, ids, tw = synth.gen_inputs(wl, T, seed=T, device=DEV)
        cfg = moe.Cfg.for_workload(wl, T)
        ref = moe.moe_layer(cfg, x, ids, tw, w)
        got = moe.moe_layer_static(cfg, x, ids, tw, w)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (name, T)


def test_static_scratch_rejects_shapes_beyond_its_size():
    """A shape whose workspace exceeds the static array is refused on the
    host (MOE_ERR_WORKSPACE) and nothing is enqueued; T = 0 is a no-op."""
    moe = M()
    wl = synth.WORKLOADS["decode_fp8_zipf_shared"]
    T = 256
    cfg = moe.Cfg.for_workload(wl, T)
    assert moe.moe_workspace_size(cfg) > moe.STATIC_SCRATCH_BYTES
    w = moe.TiledWeights(*[torch.empty(16, dtype=torch.uint8, device=DEV) for _ in range(8)])
    x, ids, tw = synth.gen_inputs(wl, T, seed=1, device=DEV)
    out = torch.full((T, wl.H), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_static(cfg, x, ids, tw, w, out=out)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out.float() == 3.0).all())
    cfg0 = moe.Cfg.for_workload(wl, 0)
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    moe.moe_layer_static(cfg0, torch.empty(0, wl.H, dtype=torch.bfloat16, device=DEV), e.view(0, wl.topk),
                         torch.empty(0, wl.topk, device=DEV), w)
    torch.cuda.synchronize()
