"""Python binding of the MI355X low-bit MoE expert layer (libmoe.so).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI in ``include/moe.h``.  PyTorch provides device memory and
the current stream.  There is no CPU or PyTorch fallback: if the library is
missing, importing the entry points raises.

Entry points (same names as the C ABI):
    moe_workspace_size(cfg) -> int
    moe_permute(cfg, x, topk_ids, ws=None) -> (counts, offsets, expand_idx, row_token, xq, xs)
    moe_grouped_gemm1_swiglu(cfg, xq, xs, row_token, offsets, weights, ws) -> (hq, hs)
    moe_grouped_gemm2(cfg, hq, hs, offsets, weights, ws) -> y
    moe_combine(cfg, y, expand_idx, offsets, topk_weights) -> out
    moe_layer(cfg, x, topk_ids, topk_weights, weights, ws=None, out=None) -> out
    moe_layer_static(cfg, x, topk_ids, topk_weights, weights, out=None) -> out   (no workspace)
    moe_layer_persistent(cfg, x, topk_ids, topk_weights, weights, ws=None, out=None, status=None) -> out
                                                                   (decode shapes: one launch)
    moe_prepack_weights(cfg, weights) -> TiledWeights
    moe_route(cfg, x, gate_w) -> (topk_ids, topk_weights)   (the router in front of the layer)
    moe_encode_e4m3(v) -> codes   (diagnostic: the quantisers' fp32 -> e4m3 conversion)

The GEMM entry points read expert weights in the tiled layout: convert the
canonical row-major tensors once with moe_prepack_weights(cfg, weights)
(a one-time step at weight load).
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libmoe.so")

MOE_OK = 0
MOE_ERR_NULL_ARG = 1
MOE_ERR_BAD_SHAPE = 2
MOE_ERR_UNSUPPORTED = 3
MOE_ERR_WORKSPACE = 4
MOE_ERR_MISALIGNED = 5
MOE_ERR_HIP = 6

WFMT_FP8_BLOCK = 0
WFMT_MXFP4 = 1
WFMT_NVFP4 = 2
RATE_E2M1_E2M1 = 16  # moe_mfma_rate's e2m1 x e2m1 operand pair

EXPORTS = ("moe_workspace_size", "moe_permute", "moe_grouped_gemm1_swiglu", "moe_grouped_gemm2",
           "moe_combine", "moe_layer", "moe_layer_static", "moe_layer_persistent", "moe_layer_persistent_spin_limit",
           "moe_prepack_weights",
           "moe_stream_read",
           "moe_mfma_rate", "moe_encode_e4m3", "moe_route", "moe_route_workspace_size", "moe_status_str")


class MoeCfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "H", "I", "E", "topk", "wfmt", "wblk", "act_group",
                                          "has_shared", "act_fmt")]


class MoeWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w1", "w1s", "w2", "w2s", "sw1", "sw1s", "sw2", "sw2s")] + \
        [("prepacked", C.c_int32)] + [(n, C.c_void_p) for n in ("w1g", "w2g", "sw1g", "sw2g")]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_str(status)})")


_lib: Optional[C.CDLL] = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with bit_grouped_gemm_amd.build.build() "
                          "(hipcc, gfx950); there is no fallback implementation")
    L = C.CDLL(path)
    vp, sz = C.c_void_p, C.c_size_t
    cfgp = C.POINTER(MoeCfg)
    wp = C.POINTER(MoeWeights)
    L.moe_workspace_size.argtypes = [cfgp, C.POINTER(sz)]
    L.moe_permute.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_grouped_gemm1_swiglu.argtypes = [cfgp, vp, vp, vp, vp, wp, vp, vp, vp, sz, vp]
    L.moe_grouped_gemm2.argtypes = [cfgp, vp, vp, vp, wp, vp, vp, sz, vp]
    L.moe_combine.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
    L.moe_layer.argtypes = [cfgp, vp, vp, vp, wp, vp, vp, sz, vp]
    L.moe_layer_static.argtypes = [cfgp, vp, vp, vp, wp, vp, vp]
    L.moe_layer_persistent.argtypes = [cfgp, vp, vp, vp, wp, vp, vp, sz, vp, vp]
    L.moe_layer_persistent_spin_limit.argtypes = [C.c_int]
    L.moe_prepack_weights.argtypes = [cfgp, wp, wp, vp]
    L.moe_stream_read.argtypes = [vp, sz, vp, sz, vp]
    L.moe_mfma_rate.argtypes = [C.c_int, C.c_int, vp, sz, C.POINTER(C.c_double), vp]
    L.moe_encode_e4m3.argtypes = [vp, sz, vp, vp]
    L.moe_route_workspace_size.argtypes = [cfgp, C.POINTER(sz)]
    L.moe_route.argtypes = [cfgp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_status_str.argtypes = [C.c_int]
    L.moe_status_str.restype = C.c_char_p
    for n in EXPORTS:
        if n != "moe_status_str":
            getattr(L, n).restype = C.c_int
    _lib = L
    return L


def status_str(status: int) -> str:
    return load().moe_status_str(int(status)).decode()


# ------------------------------------------------------------------ helpers
@dataclasses.dataclass(frozen=True)
class Cfg:
    T: int
    H: int
    I: int
    E: int
    topk: int
    wfmt: int
    wblk: int
    act_group: int
    has_shared: int = 0
    act_fmt: int = 0  # 0: e4m3 + fp32 scale per act_group; 1: MXFP4 (e2m1 + e8m0 per 32)

    def c(self) -> MoeCfg:
        return MoeCfg(self.T, self.H, self.I, self.E, self.topk, self.wfmt, self.wblk, self.act_group,
                      self.has_shared, self.act_fmt)

    @classmethod
    def for_workload(cls, wl, T: int) -> "Cfg":
        return cls(T, wl.H, wl.I, wl.E, wl.topk, wl.wfmt, wl.wblk, wl.act_group, int(wl.shared),
                   int(getattr(wl, "act_fmt", 0)))

    def act_tensors(self, rows: int, width: int, device) -> Tuple[torch.Tensor, torch.Tensor]:
        """Empty (codes, scales) of `rows` quantised activation rows of `width`
        channels: e4m3 [rows][width] + fp32 [rows][width / act_group], or for
        MXFP4 e2m1 pairs [rows][width / 2] + e8m0 [rows][width / 32]."""
        if self.act_fmt == 1:
            return (torch.empty(rows, width // 2, dtype=torch.uint8, device=device),
                    torch.empty(rows, width // 32, dtype=torch.uint8, device=device))
        return (torch.empty(rows, width, dtype=torch.uint8, device=device),
                torch.empty(rows, width // self.act_group, dtype=torch.float32, device=device))

    def with_T(self, T: int) -> "Cfg":
        return dataclasses.replace(self, T=T)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return t.data_ptr() or None


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def weights_struct(w) -> MoeWeights:
    """moe_weights from an object with w1, w1s, w2, w2s[, sw1, sw1s, sw2, sw2s] tensors,
    NVFP4's matrix scales w1g, w2g[, sw1g, sw2g] and an optional `prepacked` flag
    (absent: 0, the canonical row-major layout)."""
    g = lambda n: _ptr(getattr(w, n, None))
    return MoeWeights(g("w1"), g("w1s"), g("w2"), g("w2s"), g("sw1"), g("sw1s"), g("sw2"), g("sw2s"),
                      int(getattr(w, "prepacked", 0)), g("w1g"), g("w2g"), g("sw1g"), g("sw2g"))


def _u16(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


# ------------------------------------------------------------------ entry points
def moe_workspace_size(cfg: Cfg) -> int:
    n = C.c_size_t(0)
    c = cfg.c()
    _check("moe_workspace_size", load().moe_workspace_size(C.byref(c), C.byref(n)))
    return int(n.value)


def workspace(cfg: Cfg, device="cuda") -> torch.Tensor:
    return torch.empty(moe_workspace_size(cfg), dtype=torch.uint8, device=device)


def moe_permute(cfg: Cfg, x: torch.Tensor, topk_ids: torch.Tensor, ws: Optional[torch.Tensor] = None):
    dev = x.device
    T, k, E, sh = cfg.T, cfg.topk, cfg.E, cfg.has_shared
    counts = torch.empty(E + sh, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1 + sh, dtype=torch.int32, device=dev)
    eidx = torch.empty(T * k, dtype=torch.int32, device=dev)
    rtok = torch.empty(T * k + T * sh, dtype=torch.int32, device=dev)
    xq, xs = cfg.act_tensors(T, cfg.H, dev)
    c = cfg.c()
    ws = workspace(cfg, dev) if ws is None else ws  # per-chunk counts when T*topk > 4096
    _check("moe_permute", load().moe_permute(C.byref(c), _ptr(_u16(x)), _ptr(topk_ids), _ptr(counts),
                                             _ptr(offsets), _ptr(eidx), _ptr(rtok), _ptr(xq), _ptr(xs),
                                             _ptr(ws), ws.numel(), _stream()))
    return counts, offsets, eidx, rtok, xq, xs


def moe_grouped_gemm1_swiglu(cfg: Cfg, xq, xs, row_token, offsets, weights, ws: Optional[torch.Tensor] = None,
                             rows: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    dev = xq.device
    R = rows if rows is not None else cfg.T * cfg.topk + cfg.T * cfg.has_shared
    hq, hs = cfg.act_tensors(R, cfg.I, dev)
    ws = workspace(cfg, dev) if ws is None else ws
    c, w = cfg.c(), weights_struct(weights)
    _check("moe_grouped_gemm1_swiglu",
           load().moe_grouped_gemm1_swiglu(C.byref(c), _ptr(xq), _ptr(xs), _ptr(row_token), _ptr(offsets),
                                           C.byref(w), _ptr(hq), _ptr(hs), _ptr(ws), ws.numel(), _stream()))
    return hq, hs


def moe_grouped_gemm2(cfg: Cfg, hq, hs, offsets, weights, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    dev = hq.device
    y = torch.empty(hq.shape[0], cfg.H, dtype=torch.float32, device=dev)
    ws = workspace(cfg, dev) if ws is None else ws
    c, w = cfg.c(), weights_struct(weights)
    _check("moe_grouped_gemm2",
           load().moe_grouped_gemm2(C.byref(c), _ptr(hq), _ptr(hs), _ptr(offsets), C.byref(w), _ptr(y),
                                    _ptr(ws), ws.numel(), _stream()))
    return y


def moe_combine(cfg: Cfg, y, expand_idx, offsets, topk_weights) -> torch.Tensor:
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=y.device)
    c = cfg.c()
    _check("moe_combine", load().moe_combine(C.byref(c), _ptr(y), _ptr(expand_idx), _ptr(offsets),
                                             _ptr(topk_weights), _ptr(_u16(out)), _stream()))
    return out


def moe_layer(cfg: Cfg, x, topk_ids, topk_weights, weights, ws: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=x.device)
    ws = workspace(cfg, x.device) if ws is None else ws
    c, w = cfg.c(), weights_struct(weights)
    _check("moe_layer", load().moe_layer(C.byref(c), _ptr(_u16(x)), _ptr(topk_ids), _ptr(topk_weights), C.byref(w),
                                         _ptr(_u16(out)), _ptr(ws), ws.numel(), _stream()))
    return out


STATIC_SCRATCH_BYTES = 64 << 20  # MOE_STATIC_SCRATCH_BYTES


def moe_layer_static(cfg: Cfg, x, topk_ids, topk_weights, weights,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_layer with the library's static per-GPU scratch instead of a
    workspace (the call allocates nothing on the library side)."""
    if out is None:
        out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=x.device)
    c, w = cfg.c(), weights_struct(weights)
    _check("moe_layer_static", load().moe_layer_static(C.byref(c), _ptr(_u16(x)), _ptr(topk_ids), _ptr(topk_weights),
                                                       C.byref(w), _ptr(_u16(out)), _stream()))
    return out


def moe_layer_persistent(cfg: Cfg, x, topk_ids, topk_weights, weights, ws: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_layer as one persistent launch (decode shapes; raises with
    MOE_ERR_UNSUPPORTED otherwise).  `status`, an int32 device tensor of one
    element, receives the number of expired waits (0 in a correct run)."""
    if out is None:
        out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=x.device)
    ws = workspace(cfg, x.device) if ws is None else ws
    c, w = cfg.c(), weights_struct(weights)
    _check("moe_layer_persistent",
           load().moe_layer_persistent(C.byref(c), _ptr(_u16(x)), _ptr(topk_ids), _ptr(topk_weights), C.byref(w),
                                       _ptr(_u16(out)), _ptr(ws), ws.numel(), _ptr(status), _stream()))
    return out


PERSIST_SPIN_LIMIT = 1 << 20  # moe_layer_persistent's default polls per wait


def moe_layer_persistent_spin_limit(polls: int) -> None:
    """Polls per wait of moe_layer_persistent before it expires (process-wide;
    0 exercises the expiry path)."""
    _check("moe_layer_persistent_spin_limit", load().moe_layer_persistent_spin_limit(int(polls)))


@dataclasses.dataclass
class TiledWeights:
    """Expert weights in the layout the GEMM entry points read (prepacked = 1)."""
    w1: torch.Tensor
    w1s: torch.Tensor
    w2: torch.Tensor
    w2s: torch.Tensor
    sw1: Optional[torch.Tensor] = None
    sw1s: Optional[torch.Tensor] = None
    sw2: Optional[torch.Tensor] = None
    sw2s: Optional[torch.Tensor] = None
    prepacked: int = 1
    w1g: Optional[torch.Tensor] = None   # NVFP4: fp32 matrix scales (row-major, unchanged)
    w2g: Optional[torch.Tensor] = None
    sw1g: Optional[torch.Tensor] = None
    sw2g: Optional[torch.Tensor] = None


def moe_prepack_weights(cfg: Cfg, weights) -> TiledWeights:
    """Tiled copies of a layer's canonical row-major weights (w1, w1s, w2, w2s
    and, when cfg.has_shared, sw1..sw2s): the one-time step at weight load."""
    names = ["w1", "w1s", "w2", "w2s"] + (["sw1", "sw1s", "sw2", "sw2s"] if cfg.has_shared else [])
    if cfg.wfmt == WFMT_NVFP4:
        names += ["w1g", "w2g"] + (["sw1g", "sw2g"] if cfg.has_shared else [])
    out = TiledWeights(**{n: torch.empty_like(getattr(weights, n)) for n in names})
    c, src, dst = cfg.c(), weights_struct(weights), weights_struct(out)
    dst.prepacked = 0
    _check("moe_prepack_weights", load().moe_prepack_weights(C.byref(c), C.byref(src), C.byref(dst), _stream()))
    out.prepacked = int(dst.prepacked)
    return out





def moe_stream_read(buf: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read every byte of a device buffer once (a plain HBM read stream);
    returns the sink (one folded word per workgroup, one workgroup per CU)."""
    if sink is None:
        sink = torch.empty(8192, dtype=torch.int32, device=buf.device)
    _check("moe_stream_read", load().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                      sink.numel() * sink.element_size(), _stream()))
    return sink


def moe_mfma_rate(wfmt: int, iters: int, sink: torch.Tensor) -> float:
    """Enqueue the scaled-MFMA rate probe (all operands 1.0); returns the FLOP
    count enqueued.  `sink` (float32, device) receives 4096 * iters per
    workgroup."""
    flops = C.c_double(0.0)
    _check("moe_mfma_rate", load().moe_mfma_rate(int(wfmt), int(iters), _ptr(sink),
                                                  sink.numel() * sink.element_size(), C.byref(flops), _stream()))
    return flops.value


def moe_route_workspace_size(cfg: Cfg) -> int:
    n = C.c_size_t(0)
    c = cfg.c()
    _check("moe_route_workspace_size", load().moe_route_workspace_size(C.byref(c), C.byref(n)))
    return int(n.value)


def moe_route(cfg: Cfg, x: torch.Tensor, gate_w: torch.Tensor, ids: Optional[torch.Tensor] = None,
              weights: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Router: bf16 x [T,H] and gate rows [E,H] -> (topk_ids int32 [T,topk],
    topk_weights fp32 [T,topk]), the layer's routing inputs."""
    if ids is None:
        ids = torch.empty(cfg.T, cfg.topk, dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty(cfg.T, cfg.topk, dtype=torch.float32, device=x.device)
    if ws is None:
        n = moe_route_workspace_size(cfg)
        ws = torch.empty(n, dtype=torch.uint8, device=x.device) if n else None
    c = cfg.c()
    _check("moe_route", load().moe_route(C.byref(c), _ptr(_u16(x)), _ptr(_u16(gate_w)), _ptr(ids), _ptr(weights),
                                         _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return ids, weights


def moe_encode_e4m3(v: torch.Tensor, codes: Optional[torch.Tensor] = None) -> torch.Tensor:
    """e4m3 codes (uint8, same shape) of fp32 values by the quantisers' conversion."""
    if codes is None:
        codes = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check("moe_encode_e4m3", load().moe_encode_e4m3(_ptr(v), v.numel(), _ptr(codes), _stream()))
    return codes


def raw_call(name: str, *args) -> int:
    """Call a C entry point with raw ctypes arguments (for argument-check tests)."""
    return int(getattr(load(), name)(*args))
