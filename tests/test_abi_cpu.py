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
    # 4-bit activations: MXFP4 weights, groups of 32, H a multiple of 256, H and I <= 8192
    a4 = dict(wfmt=1, wblk=32, act_group=32, act_fmt=1)
    assert ws_size(cfg(**a4))[0] == moe.MOE_OK
    assert ws_size(cfg(**dict(a4, T=0)))[0] == moe.MOE_OK
    assert ws_size(cfg(**dict(a4, wfmt=0)))[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(cfg(**dict(a4, act_group=128)))[0] == moe.MOE_ERR_BAD_SHAPE
    assert ws_size(cfg(**dict(a4, H=384)))[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(cfg(**dict(a4, H=8448)))[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(cfg(**dict(a4, I=8320)))[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(cfg(**dict(a4, act_fmt=2)))[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(cfg(act_fmt=-1))[0] == moe.MOE_ERR_UNSUPPORTED
    assert moe.raw_call("moe_workspace_size", None, C.byref(C.c_size_t(0))) == moe.MOE_ERR_NULL_ARG
    cc = cfg().c()
    assert moe.raw_call("moe_workspace_size", C.byref(cc), None) == moe.MOE_ERR_NULL_ARG


def test_workspace_grows_with_tokens(lib):
    sizes = [ws_size(cfg(T=t, H=4096, I=1536, E=64, topk=8, wblk=128, act_group=128))[1] for t in (1, 64, 256)]
    assert sizes[0] < sizes[1] < sizes[2]


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails its host checks first


def _w(**kw):
    """Tiled (prepacked) fake weights unless prepacked=0 is given."""
    f = dict(w1=FAKE, w1s=FAKE, w2=FAKE, w2s=FAKE, sw1=None, sw1s=None, sw2=None, sw2s=None, prepacked=1)
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


def test_canonical_weights_are_rejected_by_the_gemms(lib):
    """The GEMM entry points read only the tiled layout: weights flagged
    canonical (prepacked = 0), or with any flag other than 0 / 1, are
    rejected before anything is enqueued."""
    c = cfg()
    cc = c.c()
    _, n = ws_size(c)
    for flag in (0, 2, -1):
        w = _w(prepacked=flag)
        assert moe.raw_call("moe_layer", C.byref(cc), FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE, n,
                            None) == moe.MOE_ERR_UNSUPPORTED
        assert moe.raw_call("moe_grouped_gemm1_swiglu", C.byref(cc), FAKE, FAKE, FAKE, FAKE, C.byref(w), FAKE,
                            FAKE, FAKE, n, None) == moe.MOE_ERR_UNSUPPORTED
        assert moe.raw_call("moe_grouped_gemm2", C.byref(cc), FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE, n,
                            None) == moe.MOE_ERR_UNSUPPORTED
    # the binding marks canonical tensors (no prepacked attribute) as 0 and tiled ones as 1
    assert moe.weights_struct(object()).prepacked == 0


def test_null_pointers_are_rejected_before_shape_checks(lib):
    """A NULL required pointer wins over an invalid shape (NULL buffers are
    rejected before range validation)."""
    bad = cfg(topk=0, H=200).c()
    w = _w()
    assert moe.raw_call("moe_layer", C.byref(bad), None, FAKE, FAKE, C.byref(w), FAKE, FAKE, 1 << 20,
                        None) == moe.MOE_ERR_NULL_ARG
    assert moe.raw_call("moe_layer", C.byref(bad), FAKE, FAKE, FAKE, C.byref(_w(w2=None)), FAKE, FAKE, 1 << 20,
                        None) == moe.MOE_ERR_NULL_ARG
    assert moe.raw_call("moe_layer", C.byref(bad), FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE, 1 << 20,
                        None) == moe.MOE_ERR_BAD_SHAPE
    assert moe.raw_call("moe_combine", C.byref(bad), FAKE, None, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_NULL_ARG
    # alignment is checked after the shape
    assert moe.raw_call("moe_layer", C.byref(bad), FAKE + 4, FAKE, FAKE, C.byref(w), FAKE, FAKE, 1 << 20,
                        None) == moe.MOE_ERR_BAD_SHAPE


def test_encode_e4m3_argument_errors(lib):
    call = lambda v, n, q: moe.raw_call("moe_encode_e4m3", v, C.c_size_t(n), q, None)
    assert call(None, 4, FAKE) == moe.MOE_ERR_NULL_ARG
    assert call(FAKE, 4, None) == moe.MOE_ERR_NULL_ARG
    assert call(FAKE + 4, 4, FAKE) == moe.MOE_ERR_MISALIGNED
    assert call(FAKE, 1 << 40, FAKE) == moe.MOE_ERR_BAD_SHAPE
    assert call(None, 0, None) == moe.MOE_OK          # nothing to encode: nothing enqueued


def test_prepack_argument_errors(lib):
    c = cfg()
    cc = c.c()
    src, dst = _w(prepacked=0), _w(w1=FAKE + 256, w1s=FAKE + 512, w2=FAKE + 768, w2s=FAKE + 1024, prepacked=0)
    call = lambda cfgp, a, b: moe.raw_call("moe_prepack_weights", cfgp, a, b, None)
    assert call(None, C.byref(src), C.byref(dst)) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), None, C.byref(dst)) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), C.byref(src), None) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), C.byref(src), C.byref(_w(w2=None))) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), C.byref(src), C.byref(_w(w1=FAKE + 8))) == moe.MOE_ERR_MISALIGNED
    # the source must be canonical: already tiled tensors are not re-laid out
    assert call(C.byref(cc), C.byref(_w(prepacked=1)), C.byref(dst)) == moe.MOE_ERR_UNSUPPORTED
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
    assert call(3, 16, FAKE, 1 << 12) == moe.MOE_ERR_UNSUPPORTED
    assert call(2, 16, FAKE, 1 << 12) == moe.MOE_ERR_UNSUPPORTED   # NVFP4 is no probe pair
    assert call(0, 0, FAKE, 1 << 12) == moe.MOE_ERR_BAD_SHAPE
    assert call(1, 65537, FAKE, 1 << 12) == moe.MOE_ERR_BAD_SHAPE
    assert call(1, 16, FAKE, 16) == moe.MOE_ERR_WORKSPACE


def test_static_entry_point_host_checks(lib):
    """moe_layer_static takes moe_layer's arguments minus the workspace and
    refuses, on the host, shapes whose workspace exceeds its static array."""
    c = cfg()
    cc = c.c()
    w = _w()
    call = lambda cfgp, x, wp: moe.raw_call("moe_layer_static", cfgp, x, FAKE, FAKE, wp, FAKE, None)
    assert call(None, FAKE, C.byref(w)) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), None, C.byref(w)) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), FAKE, C.byref(_w(prepacked=0))) == moe.MOE_ERR_UNSUPPORTED
    big = cfg(T=256, H=7168, I=2048, E=256, topk=8, wblk=128, act_group=128, has_shared=1)
    assert ws_size(big)[1] > moe.STATIC_SCRATCH_BYTES
    bc = big.c()
    assert call(C.byref(bc), FAKE, C.byref(_w(sw1=FAKE, sw1s=FAKE, sw2=FAKE, sw2s=FAKE))) == moe.MOE_ERR_WORKSPACE


def test_route_argument_errors(lib):
    c = cfg()
    cc = c.c()
    call = lambda cfgp, x, wg, ids, w: moe.raw_call("moe_route", cfgp, x, wg, ids, w, FAKE, C.c_size_t(1 << 30), None)
    assert call(None, FAKE, FAKE, FAKE, FAKE) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), FAKE, None, FAKE, FAKE) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), FAKE, FAKE, FAKE, None) == moe.MOE_ERR_NULL_ARG
    assert call(C.byref(cc), FAKE + 2, FAKE, FAKE, FAKE) == moe.MOE_ERR_MISALIGNED
    assert call(C.byref(cfg(topk=0).c()), FAKE, FAKE, FAKE, FAKE) == moe.MOE_ERR_BAD_SHAPE
    assert call(C.byref(cfg(E=300, topk=8).c()), FAKE, FAKE, FAKE, FAKE) == moe.MOE_ERR_UNSUPPORTED


def test_route_workspace(lib):
    n = C.c_size_t(0)
    size = lambda c: (moe.raw_call("moe_route_workspace_size", C.byref(c.c()), C.byref(n)), n.value)
    # every T > 0 needs scratch for the K splits' partial logits: splits x T
    # (rounded up to 16, or 64 above 512 tokens) x E fp32 values, the splits
    # dividing H / 64
    rc, a = size(cfg(T=1, H=4096, E=64, topk=8))
    assert rc == moe.MOE_OK and a > 0 and a % (16 * 64 * 4) == 0 and (4096 // 64) % (a // (16 * 64 * 4)) == 0
    b = size(cfg(T=512, H=4096, E=64, topk=8))[1]
    assert b > 0 and b % (512 * 64 * 4) == 0
    c = size(cfg(T=513, H=4096, E=64, topk=8))[1]
    assert c > 0 and c % (576 * 64 * 4) == 0 and (4096 // 64) % (c // (576 * 64 * 4)) == 0
    d = size(cfg(T=4096, H=7168, E=256, topk=8))[1]
    assert d % (4096 * 256 * 4) == 0 and (7168 // 64) % (d // (4096 * 256 * 4)) == 0
    assert size(cfg(T=0)) == (moe.MOE_OK, 0)
    assert size(cfg(E=300, topk=8))[0] == moe.MOE_ERR_UNSUPPORTED
    assert size(cfg(topk=0))[0] == moe.MOE_ERR_BAD_SHAPE
    assert moe.raw_call("moe_route_workspace_size", None, C.byref(n)) == moe.MOE_ERR_NULL_ARG
    cc = cfg(T=4, H=256, E=8, topk=2).c()
    P = lambda v: None if v is None else C.c_void_p(v)
    call = lambda ws, nb: moe.raw_call("moe_route", C.byref(cc), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(ws),
                                       C.c_size_t(nb), None)
    assert call(None, 0) == moe.MOE_ERR_NULL_ARG              # needed but missing
    need = size(cfg(T=4, H=256, E=8, topk=2))[1]
    assert call(FAKE, need - 4) == moe.MOE_ERR_WORKSPACE
    assert call(FAKE + 4, need) == moe.MOE_ERR_MISALIGNED


def test_binding_declares_every_parameter(lib):
    """Each exported call's ctypes argtypes has exactly the header's parameter
    count: an undeclared trailing parameter would be passed as a 32-bit int
    (a truncated stream or size), which crashes the host inside the call."""
    import re
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    L = moe.load()
    for n in moe.EXPORTS:
        m = re.search(r"\b" + n + r"\(([^;]*?)\);", src, re.S)
        assert m, n
        nargs = len([a for a in m.group(1).split(",") if a.strip()])
        assert len(getattr(L, n).argtypes or []) == nargs, n


def test_persistent_layer_host_checks(lib):
    """moe_layer_persistent checks moe_layer's arguments, then refuses on the
    host the shapes it does not run (many-row kernels, MXFP4 activations)
    with MOE_ERR_UNSUPPORTED; T = 0 is a no-op."""
    P = lambda v: None if v is None else C.c_void_p(v)

    def call(c, x=FAKE, nbytes=None, w=None):
        cc = c.c()
        n = ws_size(c)[1] if nbytes is None else nbytes
        w = _w() if w is None else w
        return moe.raw_call("moe_layer_persistent", C.byref(cc), P(x), P(FAKE), P(FAKE), C.byref(w), P(FAKE),
                            P(FAKE), C.c_size_t(n), None, None)

    c = cfg(T=4, H=512, I=256, E=8, topk=2, wblk=128, act_group=128)
    assert call(c, x=None) == moe.MOE_ERR_NULL_ARG
    assert call(c, x=FAKE + 2) == moe.MOE_ERR_MISALIGNED
    assert call(c, nbytes=ws_size(c)[1] - 1) == moe.MOE_ERR_WORKSPACE
    assert call(c, w=_w(prepacked=0)) == moe.MOE_ERR_UNSUPPORTED
    assert call(cfg(T=0, H=512, I=256, E=8, topk=2, wblk=128, act_group=128), x=None) == moe.MOE_OK
    # many rows per expert: the many-row kernels, not this launch
    assert call(cfg(T=700, H=512, I=256, E=4, topk=2, wblk=128, act_group=128)) == moe.MOE_ERR_UNSUPPORTED
    # 4-bit activations run the many-row kernels at every T
    a4 = cfg(T=4, H=512, I=256, E=8, topk=2, wfmt=1, wblk=32, act_group=32, act_fmt=1)
    assert call(a4) == moe.MOE_ERR_UNSUPPORTED


def test_nvfp4_host_checks(lib):
    """NVFP4 (wfmt 2): wblk 16, FP8 activations in 128-groups; the matrix
    scales w1g / w2g (and the shared expert's) are required and 4-byte
    aligned; workspace sizing works like the other formats."""
    c = cfg(T=4, H=512, I=256, E=8, topk=2, wfmt=2, wblk=16, act_group=128)
    assert ws_size(c)[0] == moe.MOE_OK
    assert ws_size(cfg(T=4, H=512, I=256, E=8, topk=2, wfmt=2, wblk=32, act_group=128))[0] == moe.MOE_ERR_BAD_SHAPE
    assert ws_size(cfg(T=4, H=512, I=256, E=8, topk=2, wfmt=2, wblk=16, act_group=32))[0] == moe.MOE_ERR_UNSUPPORTED
    a4 = cfg(T=4, H=512, I=256, E=8, topk=2, wfmt=2, wblk=16, act_group=32, act_fmt=1)
    assert ws_size(a4)[0] == moe.MOE_ERR_UNSUPPORTED
    cc = c.c()
    _, n = ws_size(c)
    call = lambda w: moe.raw_call("moe_layer", C.byref(cc), FAKE, FAKE, FAKE, C.byref(w), FAKE, FAKE,
                                  C.c_size_t(n), None)
    assert call(_w(w1g=None, w2g=FAKE)) == moe.MOE_ERR_NULL_ARG
    assert call(_w(w1g=FAKE, w2g=None)) == moe.MOE_ERR_NULL_ARG
    assert call(_w(w1g=FAKE + 2, w2g=FAKE)) == moe.MOE_ERR_MISALIGNED
    # a shared expert needs its two matrix scales too
    cs = cfg(T=4, H=512, I=256, E=8, topk=2, wfmt=2, wblk=16, act_group=128, has_shared=1)
    ccs = cs.c()
    ws_ = _w(w1g=FAKE, w2g=FAKE, sw1=FAKE, sw1s=FAKE, sw2=FAKE, sw2s=FAKE)
    assert moe.raw_call("moe_layer", C.byref(ccs), FAKE, FAKE, FAKE, C.byref(ws_), FAKE, FAKE,
                        C.c_size_t(ws_size(cs)[1]), None) == moe.MOE_ERR_NULL_ARG
    # the other formats ignore the matrix-scale fields
    c8 = cfg(T=4, H=512, I=256, E=8, topk=2, wblk=128, act_group=128)
    cc8 = c8.c()
    assert moe.raw_call("moe_layer", C.byref(cc8), FAKE, FAKE, FAKE, C.byref(_w(w1g=FAKE + 2)), FAKE, FAKE,
                        C.c_size_t(0), None) == moe.MOE_ERR_WORKSPACE


def test_persistent_spin_limit_host_check(lib):
    assert moe.raw_call("moe_layer_persistent_spin_limit", -1) == moe.MOE_ERR_BAD_SHAPE
    assert moe.raw_call("moe_layer_persistent_spin_limit", 1 << 20) == moe.MOE_OK
