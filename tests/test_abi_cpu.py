"""Host-side checks of the C-ABI library (no GPU work is enqueued).

The library must load, export every entry point include/moe.h declares, size
workspaces, and reject bad arguments with the documented codes before any
launch (all argument errors are host checks).
"""
import ctypes as C
import os
import re

import pytest

import bit_grouped_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from bit_grouped_gemm_amd import build
        build.build()
    return moe.load()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("moe_permute", "moe_grouped_gemm1_swiglu", "moe_grouped_gemm2", "moe_combine", "moe_layer"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(moe.EXPORTS)


def cfg(**kw):
    base = dict(T=4, H=256, I=128, E=8, topk=2, wfmt=0, wblk=32, act_group=32, has_shared=0)
    base.update(kw)
    return moe.Cfg(**base)


def ws_size(c):
    n = C.c_size_t(0)
    cc = c.c()
    return moe.raw_call("moe_workspace_size", C.byref(cc), C.byref(n)), n.value


def test_workspace_size_and_shape_errors(lib):
    rc, n = ws_size(cfg())
    assert rc == moe.MOE_OK and n > 0 and n % 256 == 0
    rc, n0 = ws_size(cfg(T=0))
    assert rc == moe.MOE_OK
    assert ws_size(cfg(topk=9))[0] == moe.MOE_ERR_BAD_SHAPE        # k > E
    assert ws_size(cfg(T=-1))[0] == moe.MOE_ERR_BAD_SHAPE
    assert ws_size(cfg(H=200))[0] == moe.MOE_ERR_BAD_SHAPE         # not a multiple of 128
    assert ws_size(cfg(E=2000, topk=2))[0] == moe.MOE_ERR_BAD_SHAPE
    # activation bytes beyond 32-bit offsets: T * H, and rows * I
    assert ws_size(cfg(T=1 << 18, H=8192))[0] == moe.MOE_ERR_BAD_SHAPE
    assert ws_size(cfg(T=(1 << 18) - 1, H=8192))[0] == moe.MOE_OK
    assert ws_size(cfg(T=1 << 16, topk=4, I=8192))[0] == moe.MOE_ERR_BAD_SHAPE
    assert ws_size(cfg(wblk=64, act_group=64))[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(cfg(act_group=128))[0] == moe.MOE_ERR_BAD_SHAPE  # FP8 group != block
    assert ws_size(cfg(wfmt=1, wblk=32, act_group=128))[0] == moe.MOE_OK
    assert ws_size(cfg(wfmt=1, wblk=32, act_group=32))[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(cfg(wfmt=7))[0] == moe.MOE_ERR_UNSUPPORTED
    assert moe.raw_call("moe_workspace_size", None, C.byref(C.c_size_t(0))) == moe.MOE_ERR_NULL_ARG
    cc = cfg().c()
    assert moe.raw_call("moe_workspace_size", C.byref(cc), None) == moe.MOE_ERR_NULL_ARG


def test_workspace_grows_with_tokens(lib):
    sizes = [ws_size(cfg(T=t, H=4096, I=1536, E=64, topk=8, wblk=128, act_group=128))[1] for t in (1, 64, 256)]
    assert sizes[0] < sizes[1] < sizes[2]


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails its host checks first


def _w(**kw):
    f = dict(w1=FAKE, w1s=FAKE, w2=FAKE, w2s=FAKE, sw1=None, sw1s=None, sw2=None, sw2s=None)
    f.update(kw)
    return moe.MoeWeights(**f)


def test_layer_argument_errors(lib):
    c = cfg()
    cc = c.c()
    _, n = ws_size(c)
    w = _w()
    call = lambda cfgp, x, ids, tw, wp, out, ws, nbytes: moe.raw_call(
        "moe_layer", cfgp, x, ids, tw, wp, out, ws, nbytes, None)
    assert call(None, FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE, n) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), None, FAKE, FAKE, C.byref(w), FAKE, FAKE, n) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), FAKE, FAKE, FAKE, None, FAKE, FAKE, n) == moe.MOE_ERR_NULL_ARG
    wnull = _w(w2s=None)
    assert call(C.byref(cc), FAKE, FAKE, FAKE, C.byref(wnull), FAKE, FAKE, n) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), FAKE + 4, FAKE, FAKE, C.byref(w), FAKE, FAKE, n) == moe.MOE_ERR_MISALIGNED
    wmis = _w(w1=FAKE + 8)
    assert call(C.byref(cc), FAKE, FAKE, FAKE, C.byref(wmis), FAKE, FAKE, n) == moe.MOE_ERR_MISALIGNED
    assert call(C.byref(cc), FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE, n - 1) == moe.MOE_ERR_WORKSPACE
    bad = cfg(topk=0).c()
    assert call(C.byref(bad), FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE, n) == moe.MOE_ERR_BAD_SHAPE
    # a shared expert needs its four tensors
    cs = cfg(has_shared=1)
    ccs = cs.c()
    _, ns = ws_size(cs)
    assert call(C.byref(ccs), FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE, ns) == moe.MOE_ERR_NULL_ARG


def test_stage_argument_errors(lib):
    c = cfg()
    cc = c.c()
    _, n = ws_size(c)
    w = _w()
    assert moe.raw_call("moe_permute", C.byref(cc), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        None, 0, None) == moe.MOE_ERR_NULL_ARG
    assert moe.raw_call("moe_permute", C.byref(cc), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                        None, 0, None) == moe.MOE_ERR_NULL_ARG
    assert moe.raw_call("moe_grouped_gemm1_swiglu", C.byref(cc), FAKE, FAKE, FAKE, FAKE, C.byref(w), FAKE,
                        FAKE, FAKE, n - 256, None) == moe.MOE_ERR_WORKSPACE
    assert moe.raw_call("moe_grouped_gemm1_swiglu", C.byref(cc), FAKE, FAKE, FAKE, FAKE, C.byref(w), FAKE,
                        FAKE, None, n, None) == moe.MOE_ERR_NULL_ARG
    assert moe.raw_call("moe_grouped_gemm2", C.byref(cc), FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE, 0,
                        None) == moe.MOE_ERR_WORKSPACE
    assert moe.raw_call("moe_combine", C.byref(cc), FAKE, FAKE, None, FAKE, FAKE, None) == moe.MOE_ERR_NULL_ARG
    assert moe.raw_call("moe_combine", C.byref(cc), FAKE, FAKE + 2, FAKE, FAKE, FAKE,
                        None) == moe.MOE_ERR_MISALIGNED


def test_status_strings(lib):
    for code in range(7):
        assert moe.status_str(code) != "unknown status"
    assert moe.status_str(99) == "unknown status"


def test_product_path_does_not_touch_the_oracle():
    """The HIP binding and the kernels never import or link the CPU oracle."""
    pkg = os.path.join(ROOT, "bit_grouped_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src, f


def test_prepack_argument_errors(lib):
    c = cfg()
    cc = c.c()
    src, dst = _w(), _w(w1=FAKE + 256, w1s=FAKE + 512, w2=FAKE + 768, w2s=FAKE + 1024)
    call = lambda cfgp, a, b: moe.raw_call("moe_prepack_weights", cfgp, a, b, None)
    assert call(None, C.byref(src), C.byref(dst)) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), None, C.byref(dst)) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), C.byref(src), None) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), C.byref(src), C.byref(_w(w2=None))) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), C.byref(src), C.byref(_w(w1=FAKE + 8))) == moe.MOE_ERR_MISALIGNED
    assert call(C.byref(cfg(topk=0).c()), C.byref(src), C.byref(dst)) == moe.MOE_ERR_BAD_SHAPE
    assert call(C.byref(cc), C.byref(src), C.byref(src)) == moe.MOE_ERR_UNSUPPORTED   # in place
    cs = cfg(has_shared=1).c()
    assert call(C.byref(cs), C.byref(src), C.byref(dst)) == moe.MOE_ERR_NULL_ARG       # shared tensors


def test_stream_read_argument_errors(lib):
    call = lambda buf, n, sink, sn: moe.raw_call("moe_stream_read", buf, C.c_size_t(n), sink, C.c_size_t(sn), None)
    assert call(None, 64, FAKE, 1 << 15) == moe.MOE_ERR_NULL_ARG
    assert call(FAKE, 64, None, 1 << 15) == moe.MOE_ERR_NULL_ARG
    assert call(FAKE + 4, 64, FAKE, 1 << 15) == moe.MOE_ERR_MISALIGNED
    assert call(FAKE, 64, FAKE + 8, 1 << 15) == moe.MOE_ERR_MISALIGNED
    assert call(FAKE, 65, FAKE, 1 << 15) == moe.MOE_ERR_BAD_SHAPE
    assert call(FAKE, 64, FAKE, 4) == moe.MOE_ERR_WORKSPACE


def test_mfma_rate_argument_errors(lib):
    fl = C.c_double(0.0)
    call = lambda wfmt, iters, sink, sn: moe.raw_call("moe_mfma_rate", wfmt, iters, sink, C.c_size_t(sn), C.byref(fl), None)
    assert call(0, 16, None, 1 << 12) == moe.MOE_ERR_NULL_ARG
    assert call(0, 16, FAKE + 4, 1 << 12) == moe.MOE_ERR_MISALIGNED
    assert call(2, 16, FAKE, 1 << 12) == moe.MOE_ERR_UNSUPPORTED
    assert call(0, 0, FAKE, 1 << 12) == moe.MOE_ERR_BAD_SHAPE
    assert call(1, 65537, FAKE, 1 << 12) == moe.MOE_ERR_BAD_SHAPE
    assert call(1, 16, FAKE, 16) == moe.MOE_ERR_WORKSPACE
