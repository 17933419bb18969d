"""Seeded synthetic inputs for the MoE expert layer.

This module only *produces inputs*: bf16 activations, top-k routing and
quantised expert weights.  It holds none of the layer's own arithmetic
(activation quantisation, grouped GEMMs, SwiGLU, requantisation, combine);
both the CPU oracle and the HIP path consume the bytes it returns.

Workloads follow the shapes of the low-bit MoE decode / prefill regimes the
GC-MoE abstract describes (1-256 tokens per rank at decode, FP8 or FP4
block-scaled expert weights), at one GPU's share of the work.  No trained
weights or routing traces exist here: weights are drawn from N(0, 0.02) and
quantised, activations from N(0, 1).

Weight quantisation for the generator (inputs arrive already quantised):
  * FP8 e4m3 with one fp32 scale per b x b block: multiplier 448/amax, the
    code comes from PyTorch's own fp32 -> float8_e4m3fn cast (RNE), scale =
    1/multiplier.
  * MXFP4: e2m1 codes packed two per byte (even K index in the low nibble)
    with one e8m0 power-of-two scale per 32 elements along K, using the
    Microscaling rule X = 2^(floor(log2 amax) - 2) and round-to-nearest-even
    with saturation at +-6.
  * NVFP4: e2m1 codes packed the same way, one e4m3 scale per 16 elements
    along K and one fp32 scale per expert matrix: matrix scale S = amax /
    (448 * 6), block scale = e4m3(block amax / 6 / S) by PyTorch's cast,
    codes = e2m1 of w / (block scale * S), round-to-nearest-even with
    saturation at +-6 (a block whose scale is 0 gets zero codes).

Random streams: every tensor draws from its own torch.Generator on the
target device, seeded from (seed, workload, tensor id, expert).  A stream is
reproducible on one device type; CPU and GPU streams differ, so a parity
test always feeds both sides the very same generated tensors.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import torch

FMT_FP8 = 0
FMT_MXFP4 = 1
FMT_NVFP4 = 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one MoE expert layer on one GPU's share of the work."""
    name: str
    H: int
    E: int
    topk: int
    I: int
    wfmt: int            # FMT_FP8, FMT_MXFP4 or FMT_NVFP4
    wblk: int            # FP8: b x b scale block edge; MXFP4: 32 along K; NVFP4: 16 along K
    act_group: int       # activation / requantisation group along K
    routing: str         # "uniform" or "zipf"
    shared: bool         # one always-on shared expert with weight 1
    tokens: Tuple[int, ...]
    wid: int             # workload id mixed into the seeds
    act_fmt: int = 0     # 0: FP8 e4m3 activations (fp32 scale per act_group); 1: MXFP4 (e8m0 per 32)

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny FP8 layer, 32x32 weight blocks, activation groups of 32
    "tiny_fp8": Workload("tiny_fp8", H=256, E=8, topk=2, I=128, wfmt=FMT_FP8, wblk=32,
                         act_group=32, routing="uniform", shared=False, tokens=(16,), wid=0),
    # decode FP8: H=4096, E=64, top-8, I=1536, 128x128 blocks
    "decode_fp8": Workload("decode_fp8", H=4096, E=64, topk=8, I=1536, wfmt=FMT_FP8, wblk=128,
                           act_group=128, routing="uniform", shared=False,
                           tokens=(1, 8, 32, 64, 128, 256), wid=1),
    # decode MXFP4: same shapes and routing
    "decode_mxfp4": Workload("decode_mxfp4", H=4096, E=64, topk=8, I=1536, wfmt=FMT_MXFP4, wblk=32,
                             act_group=128, routing="uniform", shared=False,
                             tokens=(1, 8, 32, 64, 128, 256), wid=2),
    # decode NVFP4: same shapes and routing (e4m3 scale per 16, fp32 scale per matrix)
    "decode_nvfp4": Workload("decode_nvfp4", H=4096, E=64, topk=8, I=1536, wfmt=FMT_NVFP4, wblk=16,
                             act_group=128, routing="uniform", shared=False,
                             tokens=(1, 8, 32, 64, 128, 256), wid=6),
    # large decode FP8, Zipf(1.2) routing, one shared expert
    "decode_fp8_zipf_shared": Workload("decode_fp8_zipf_shared", H=7168, E=256, topk=8, I=2048,
                                       wfmt=FMT_FP8, wblk=128, act_group=128, routing="zipf",
                                       shared=True, tokens=(1, 16, 64, 256), wid=3),
    # prefill MXFP4, T=4096, uniform routing (~128 rows per expert)
    "prefill_mxfp4": Workload("prefill_mxfp4", H=7168, E=256, topk=8, I=2048, wfmt=FMT_MXFP4,
                              wblk=32, act_group=128, routing="uniform", shared=False,
                              tokens=(4096,), wid=4),
    # prefill NVFP4 weights against e4m3 activations, same shapes and routing
    "prefill_nvfp4": Workload("prefill_nvfp4", H=7168, E=256, topk=8, I=2048, wfmt=FMT_NVFP4,
                              wblk=16, act_group=128, routing="uniform", shared=False,
                              tokens=(4096,), wid=7),
    # the 4-bit-activation variant of the prefill layer: MXFP4 weights and MXFP4
    # activations (e2m1 with an e8m0 scale per 32 channels), same shapes and routing
    "prefill_mxfp4_a4": Workload("prefill_mxfp4_a4", H=7168, E=256, topk=8, I=2048, wfmt=FMT_MXFP4,
                                 wblk=32, act_group=32, routing="uniform", shared=False,
                                 tokens=(4096,), wid=5, act_fmt=1),
}

_MASK64 = (1 << 64) - 1


def _splitmix64(z: int) -> int:
    z = (z + 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_seed(seed: int, wid: int, tensor_id: int, sub: int = 0) -> int:
    """63-bit generator seed for one tensor (or one expert of it)."""
    key = (seed & 0xFFFFFFFF) ^ (wid << 48) ^ (tensor_id << 40) ^ (sub << 8)
    return _splitmix64(key & _MASK64) >> 1


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


# tensor ids for the seed derivation
_TID_X, _TID_ROUTE, _TID_LOGIT, _TID_W1, _TID_W2, _TID_SW1, _TID_SW2 = 1, 2, 3, 4, 5, 6, 7


def gen_x(T: int, H: int, seed: int, wid: int, device="cpu") -> torch.Tensor:
    """bf16 activations, N(0,1) rounded to bf16 (RNE)."""
    g = _gen(device, stream_seed(seed, wid, _TID_X, T))
    return torch.randn(T, H, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def gen_routing(T: int, E: int, k: int, routing: str, seed: int, wid: int,
                device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k expert ids (int32 [T,k], distinct per token, in draw order) and
    fp32 routing weights (softmax of N(0,1) logits over the k chosen slots,
    i.e. the full softmax renormalised over the top-k)."""
    g = _gen("cpu", stream_seed(seed, wid, _TID_ROUTE, T))
    if T == 0:
        ids = torch.empty(0, k, dtype=torch.int64)
    elif routing == "uniform":
        # the first k entries of a uniformly random permutation
        ids = torch.argsort(torch.rand(T, E, generator=g), dim=1)[:, :k]
    elif routing == "zipf":
        # p(e) ~ (e+1)^-1.2; k draws without replacement (draw, remove, renormalise)
        p = torch.arange(1, E + 1, dtype=torch.float64).pow(-1.2)
        ids = torch.multinomial((p / p.sum()).expand(T, E).contiguous(), k, replacement=False,
                                generator=g)
    else:
        raise ValueError(f"unknown routing {routing!r}")
    g2 = _gen("cpu", stream_seed(seed, wid, _TID_LOGIT, T))
    logits = torch.randn(T, k, generator=g2, dtype=torch.float32)
    w = torch.softmax(logits, dim=1)
    return ids.to(torch.int32).to(device), w.to(device)


_FP8_MAX = 448.0   # largest e4m3 magnitude: a block's maximum maps onto it


def _quant_fp8_blocks(w: torch.Tensor, b: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp32 [N,K] -> (e4m3 codes uint8 [N,K], fp32 scales [N/b, K/b])."""
    N, K = w.shape
    blk = w.reshape(N // b, b, K // b, b)
    amax = blk.abs().amax(dim=(1, 3)).clamp_min(2.0 ** -64)
    mult = torch.full_like(amax, _FP8_MAX) / amax
    q = (blk * mult[:, None, :, None]).to(torch.float8_e4m3fn)
    return q.reshape(N, K).view(torch.uint8), (1.0 / mult)


_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _quant_mxfp4(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp32 [N,K] -> (packed e2m1 uint8 [N,K/2], e8m0 scale codes uint8 [N,K/32])."""
    N, K = w.shape
    blk = w.reshape(N, K // 32, 32)
    amax = blk.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                    # amax = m * 2^ex, m in [0.5, 1)
    sexp = (ex - 1) - 2                          # floor(log2 amax) - 2
    zero = amax == 0
    code = torch.where(zero, torch.zeros_like(sexp), sexp + 127).clamp(0, 254)
    X = torch.ldexp(torch.ones_like(amax), code - 127)
    v = blk / X[:, :, None]
    a = v.abs()
    nib = torch.zeros_like(a, dtype=torch.int32)
    for i, mid in enumerate(_E2M1_MIDS):
        nib += (a > mid).to(torch.int32)
        if i % 2 == 1:                           # tie at an odd lower code goes up to the even one
            nib += (a == mid).to(torch.int32)
    nib = torch.where(zero[:, :, None], torch.zeros_like(nib), nib)
    nib = nib | (torch.signbit(v).to(torch.int32) << 3)
    nib = nib.reshape(N, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).to(torch.uint8)
    return packed, code.to(torch.uint8)


def _e2m1_rne(v: torch.Tensor) -> torch.Tensor:
    """e2m1 codes (int32, sign in bit 3) of v, round to nearest even, saturating at +-6."""
    a = v.abs()
    nib = torch.zeros_like(a, dtype=torch.int32)
    for i, mid in enumerate(_E2M1_MIDS):
        nib += (a > mid).to(torch.int32)
        if i % 2 == 1:                           # tie at an odd lower code goes up to the even one
            nib += (a == mid).to(torch.int32)
    return nib | (torch.signbit(v).to(torch.int32) << 3)


def _quant_nvfp4(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """fp32 [N,K] -> (packed e2m1 uint8 [N,K/2], e4m3 block scales uint8 [N,K/16],
    fp32 matrix scale [1])."""
    N, K = w.shape
    S = (w.abs().amax() / (_FP8_MAX * 6.0)).clamp_min(2.0 ** -100).reshape(1)
    blk = w.reshape(N, K // 16, 16)
    bs = (blk.abs().amax(dim=2) / 6.0 / S).clamp(max=_FP8_MAX).to(torch.float8_e4m3fn)
    den = bs.to(torch.float32) * S
    zero = den == 0
    v = blk / torch.where(zero, torch.ones_like(den), den)[:, :, None]
    nib = torch.where(zero[:, :, None], torch.zeros_like(v, dtype=torch.int32), _e2m1_rne(v)).reshape(N, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).to(torch.uint8)
    return packed, bs.view(torch.uint8), S


def _gen_matrix_set(n_exp: int, N: int, K: int, wfmt: int, wblk: int, seed: int, wid: int,
                    tid: int, device):
    """(codes, scales, matrix scales or None) of n_exp quantised [N,K] matrices."""
    gsc = None
    if wfmt == FMT_FP8:
        codes = torch.empty(n_exp, N, K, dtype=torch.uint8, device=device)
        scales = torch.empty(n_exp, N // wblk, K // wblk, dtype=torch.float32, device=device)
    elif wfmt == FMT_MXFP4:
        codes = torch.empty(n_exp, N, K // 2, dtype=torch.uint8, device=device)
        scales = torch.empty(n_exp, N, K // 32, dtype=torch.uint8, device=device)
    else:
        codes = torch.empty(n_exp, N, K // 2, dtype=torch.uint8, device=device)
        scales = torch.empty(n_exp, N, K // 16, dtype=torch.uint8, device=device)
        gsc = torch.empty(n_exp, dtype=torch.float32, device=device)
    for e in range(n_exp):
        g = _gen(device, stream_seed(seed, wid, tid, e))
        w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * 0.02
        if wfmt == FMT_FP8:
            q, s = _quant_fp8_blocks(w, wblk)
        elif wfmt == FMT_MXFP4:
            q, s = _quant_mxfp4(w)
        else:
            q, s, S = _quant_nvfp4(w)
            gsc[e:e + 1].copy_(S)
        codes[e].copy_(q)
        scales[e].copy_(s)
        del w, q, s
    return codes, scales, gsc


@dataclasses.dataclass
class Weights:
    """Canonical expert weights.

    FP8:   w1 uint8 [E,2I,H] (rows 0..I-1 gate, I..2I-1 up; K contiguous),
           w1s fp32 [E,2I/b,H/b]; w2 uint8 [E,H,I], w2s fp32 [E,H/b,I/b].
    MXFP4: w1 uint8 [E,2I,H/2], w1s uint8 e8m0 [E,2I,H/32];
           w2 uint8 [E,H,I/2],  w2s uint8 e8m0 [E,H,I/32].
    NVFP4: w1 uint8 [E,2I,H/2], w1s uint8 e4m3 [E,2I,H/16], w1g fp32 [E];
           w2 uint8 [E,H,I/2],  w2s uint8 e4m3 [E,H,I/16],  w2g fp32 [E].
    Shared expert (optional): the same with a leading dimension of 1.
    """
    w1: torch.Tensor
    w1s: torch.Tensor
    w2: torch.Tensor
    w2s: torch.Tensor
    sw1: Optional[torch.Tensor] = None
    sw1s: Optional[torch.Tensor] = None
    sw2: Optional[torch.Tensor] = None
    sw2s: Optional[torch.Tensor] = None
    w1g: Optional[torch.Tensor] = None
    w2g: Optional[torch.Tensor] = None
    sw1g: Optional[torch.Tensor] = None
    sw2g: Optional[torch.Tensor] = None

    def to(self, device) -> "Weights":
        f = lambda t: None if t is None else t.to(device)
        return Weights(*(f(getattr(self, fl.name)) for fl in dataclasses.fields(self)))

    def nbytes_expert(self) -> int:
        """Bytes of one routed expert (codes + scales, W1 and W2)."""
        ts = [self.w1, self.w1s, self.w2, self.w2s] + [t for t in (self.w1g, self.w2g) if t is not None]
        return sum(t[0].numel() * t.element_size() for t in ts)

    def nbytes_shared(self) -> int:
        if self.sw1 is None:
            return 0
        ts = [self.sw1, self.sw1s, self.sw2, self.sw2s] + [t for t in (self.sw1g, self.sw2g) if t is not None]
        return sum(t.numel() * t.element_size() for t in ts)


def gen_weights(wl: Workload, seed: int = 0, device="cpu") -> Weights:
    """Quantised expert weights for a workload (independent of T)."""
    w1, w1s, w1g = _gen_matrix_set(wl.E, 2 * wl.I, wl.H, wl.wfmt, wl.wblk, seed, wl.wid, _TID_W1, device)
    w2, w2s, w2g = _gen_matrix_set(wl.E, wl.H, wl.I, wl.wfmt, wl.wblk, seed, wl.wid, _TID_W2, device)
    out = Weights(w1, w1s, w2, w2s, w1g=w1g, w2g=w2g)
    if wl.shared:
        out.sw1, out.sw1s, out.sw1g = _gen_matrix_set(1, 2 * wl.I, wl.H, wl.wfmt, wl.wblk, seed, wl.wid,
                                                      _TID_SW1, device)
        out.sw2, out.sw2s, out.sw2g = _gen_matrix_set(1, wl.H, wl.I, wl.wfmt, wl.wblk, seed, wl.wid,
                                                      _TID_SW2, device)
    return out


_TID_GATE = 8


def gen_gate(wl: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """Router gate weights bf16 [E, H] (one row per expert), N(0, 0.02)
    rounded to bf16, so that gate logits of N(0,1) activations have a spread
    of 0.02 * sqrt(H)."""
    g = _gen(device, stream_seed(seed, wl.wid, _TID_GATE, 0))
    return (torch.randn(wl.E, wl.H, generator=g, device=device, dtype=torch.float32) * 0.02).to(torch.bfloat16)


def gen_inputs(wl: Workload, T: int, seed: int = 0, device="cpu"):
    """(x bf16 [T,H], topk_ids int32 [T,k], topk_weights fp32 [T,k])."""
    x = gen_x(T, wl.H, seed, wl.wid, device)
    ids, w = gen_routing(T, wl.E, wl.topk, wl.routing, seed, wl.wid, device)
    return x, ids, w


def touched_experts(ids: torch.Tensor, E: int) -> int:
    v = ids.flatten().to(torch.int64)
    v = v[(v >= 0) & (v < E)]
    return int(torch.unique(v).numel())


def weight_bytes_touched(wl: Workload, weights: Weights, ids: torch.Tensor) -> int:
    """Algorithmic weight bytes one layer call must read: every touched routed
    expert's W1, W2 and their scales, plus the shared expert."""
    return touched_experts(ids, wl.E) * weights.nbytes_expert() + weights.nbytes_shared()


def layer_flops(wl: Workload, T: int, ids: torch.Tensor) -> int:
    """2 * rows * (2I*H + H*I) over routed (valid) rows plus shared rows."""
    v = ids.flatten().to(torch.int64)
    R = int(((v >= 0) & (v < wl.E)).sum()) + (T if wl.shared else 0)
    return 2 * R * (2 * wl.I * wl.H + wl.H * wl.I)


def expected_touched_uniform(E: int, k: int, T: int) -> float:
    return E * (1.0 - (1.0 - k / E) ** T)

