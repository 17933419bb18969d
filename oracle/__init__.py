"""ctypes wrapper of the CPU oracle (``oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the product path.  All arrays are CPU
numpy arrays or CPU torch tensors; results come back as numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (plain C++17, no SIMD intrinsics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(_LIB), exist_ok=True)
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib: Optional[C.CDLL] = None


class Cfg(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("T", "H", "I", "E", "k", "wfmt", "wblk", "G", "has_shared", "act_fmt")]


class WSet(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w1", "w1s", "w2", "w2s", "sw1", "sw1s", "sw2", "sw2s",
                                          "w1g", "w2g", "sw1g", "sw2g")]


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        L.oracle_dec_e4m3.restype = C.c_double
        L.oracle_dec_e2m1.restype = C.c_double
        L.oracle_dec_e8m0.restype = C.c_double
        L.oracle_dec_e4m3.argtypes = [i32]
        L.oracle_dec_e2m1.argtypes = [i32]
        L.oracle_dec_e8m0.argtypes = [i32]
        L.oracle_enc_e4m3.argtypes = [C.c_float]
        L.oracle_enc_e2m1.argtypes = [C.c_float]
        L.oracle_enc_e4m3_array.argtypes = [vp, i64, vp]
        L.oracle_quant_rows_f32.argtypes = [vp, i64, i64, i32, vp, vp]
        L.oracle_quant_act.argtypes = [vp, i64, i64, i32, vp, vp]
        L.oracle_quant_act_cfg.argtypes = [vp, vp, i64, vp, vp]
        L.oracle_permute.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_gemm1.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp]
        L.oracle_gemm2.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp]
        L.oracle_combine.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp]
        L.oracle_layer.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp]
        L.oracle_bruteforce.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp]
        L.oracle_router.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, vp]
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_set_mutation.argtypes = [i32]
        _lib = L
    return _lib


# ------------------------------------------------------------------ helpers
def _np(a, dtype=None) -> np.ndarray:
    """torch CPU tensor or array-like -> C-contiguous numpy array (bf16 as uint16)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16).numpy().view(np.uint16)
            elif a.dtype in (torch.float8_e4m3fn, torch.float8_e8m0fnu):
                a = a.view(torch.uint8).numpy()
            else:
                a = a.numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        a = np.ascontiguousarray(a.astype(dtype))
    return a


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def threads() -> int:
    return int(lib().oracle_get_threads())


def set_mutation(m: int) -> None:
    lib().oracle_set_mutation(int(m))


def dec_e4m3(c: int) -> float:
    return lib().oracle_dec_e4m3(int(c))


def dec_e2m1(c: int) -> float:
    return lib().oracle_dec_e2m1(int(c))


def dec_e8m0(c: int) -> float:
    return lib().oracle_dec_e8m0(int(c))


def enc_e4m3(v: float) -> int:
    return int(lib().oracle_enc_e4m3(float(v)))


def enc_e2m1(v: float) -> int:
    return int(lib().oracle_enc_e2m1(float(v)))


def enc_e4m3_array(v) -> np.ndarray:
    v = _np(v, np.float32)
    q = np.empty(v.shape, np.uint8)
    lib().oracle_enc_e4m3_array(_p(v), v.size, _p(q))
    return q


def quant_rows_f32(v, G: int):
    v = _np(v, np.float32)
    rows, cols = v.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // G), np.float32)
    lib().oracle_quant_rows_f32(_p(v), rows, cols, G, _p(q), _p(s))
    return q, s


def quant_act(x, G: int):
    """bf16 [T,H] -> (xq uint8 [T,H], xs fp32 [T,H/G])."""
    x = _np(x)
    assert x.dtype == np.uint16
    T, H = x.shape
    xq = np.empty((T, H), np.uint8)
    xs = np.empty((T, H // G), np.float32)
    lib().oracle_quant_act(_p(x), T, H, G, _p(xq), _p(xs))
    return xq, xs


def quant_act_mx(x):
    """bf16 [T,H] -> MXFP4 activations: (xq uint8 [T,H/2] packed e2m1, even
    channel in the low nibble; xs uint8 [T,H/32] e8m0 scale codes)."""
    x = _np(x)
    assert x.dtype == np.uint16
    T, H = x.shape
    c = Cfg(T, H, 128, 1, 1, 1, 32, 32, 0, 1)
    xq = np.empty((T, H // 2), np.uint8)
    xs = np.empty((T, H // 32), np.uint8)
    lib().oracle_quant_act_cfg(C.byref(c), _p(x), T, _p(xq), _p(xs))
    return xq, xs


def permute(ids, E: int, has_shared: bool):
    """ids int32 [T,k] -> (counts, offsets, expand_idx [T*k], row_token)."""
    ids = _np(ids, np.int32)
    T, k = ids.shape
    ng = E + int(has_shared)
    counts = np.empty(ng, np.int32)
    offsets = np.empty(ng + 1, np.int32)
    eidx = np.empty(T * k, np.int32)
    rtok = np.empty(max(T * k + T * int(has_shared), 1), np.int32)
    lib().oracle_permute(_p(ids), T, k, E, int(has_shared), _p(counts), _p(offsets), _p(eidx), _p(rtok))
    return counts, offsets, eidx, rtok[: T * k + T * int(has_shared)]


def router(x, wg, k: int):
    """Router: x bf16 [T,H], wg bf16 [E,H] -> (ids int32 [T,k], weights fp32
    [T,k], logits fp64 [T,E])."""
    x, wg = _np(x), _np(wg)
    assert x.dtype == np.uint16 and wg.dtype == np.uint16
    T, H = x.shape
    E = wg.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lg = np.empty((T, E), np.float64)
    lib().oracle_router(_p(x), _p(wg), T, H, E, k, _p(ids), _p(w), _p(lg))
    return ids, w, lg


class Layer:
    """Binds a workload's shapes and one set of canonical weights."""

    def __init__(self, T: int, H: int, I: int, E: int, k: int, wfmt: int, wblk: int, G: int,
                 has_shared: bool, weights, act_fmt: int = 0):
        self.cfg = Cfg(T, H, I, E, k, wfmt, wblk, G, int(has_shared), int(act_fmt))
        self.T, self.H, self.I, self.E, self.k, self.G = T, H, I, E, k, G
        self.act_fmt = int(act_fmt)
        self.has_shared = bool(has_shared)
        f32 = np.float32 if wfmt == 0 else np.uint8
        self._keep = [
            _np(weights.w1, np.uint8), _np(weights.w1s, f32), _np(weights.w2, np.uint8), _np(weights.w2s, f32),
            _np(weights.sw1, np.uint8) if weights.sw1 is not None else None,
            _np(weights.sw1s, f32) if weights.sw1s is not None else None,
            _np(weights.sw2, np.uint8) if weights.sw2 is not None else None,
            _np(weights.sw2s, f32) if weights.sw2s is not None else None,
        ]
        # NVFP4: the fp32 scale of every expert matrix
        for n in ("w1g", "w2g", "sw1g", "sw2g"):
            g = getattr(weights, n, None)
            self._keep.append(None if g is None else _np(g, np.float32))
        self.wset = WSet(*[_p(a) for a in self._keep])

    @classmethod
    def for_workload(cls, wl, T: int, weights) -> "Layer":
        return cls(T, wl.H, wl.I, wl.E, wl.topk, wl.wfmt, wl.wblk, wl.act_group, wl.shared, weights,
                   getattr(wl, "act_fmt", 0))

    def _cb(self, n):   # code bytes of an n-channel quantised row
        return n // 2 if self.act_fmt == 1 else n

    def _sdt(self, n):  # (scale dtype, scales per n-channel row)
        return (np.uint8, n // 32) if self.act_fmt == 1 else (np.float32, n // self.G)

    def with_T(self, T: int) -> "Layer":
        other = object.__new__(Layer)
        other.__dict__.update(self.__dict__)
        c = self.cfg
        other.cfg = Cfg(T, c.H, c.I, c.E, c.k, c.wfmt, c.wblk, c.G, c.has_shared, c.act_fmt)
        other.T = T
        return other

    def _toks(self, toks: Optional[Sequence[int]]) -> np.ndarray:
        if toks is None:
            toks = range(self.T)
        return np.ascontiguousarray(np.asarray(list(toks), np.int64))

    def layer(self, x, ids, topk_w, toks: Optional[Sequence[int]] = None) -> np.ndarray:
        """fp64 output rows [len(toks), H] of the whole layer."""
        x, ids, w = _np(x), _np(ids, np.int32), _np(topk_w, np.float32)
        tk = self._toks(toks)
        out = np.empty((len(tk), self.H), np.float64)
        lib().oracle_layer(C.byref(self.cfg), C.byref(self.wset), _p(x), _p(ids), _p(w), len(tk),
                           _p(tk), _p(out))
        return out

    def bruteforce(self, x, ids, topk_w, toks: Optional[Sequence[int]] = None) -> np.ndarray:
        x, ids, w = _np(x), _np(ids, np.int32), _np(topk_w, np.float32)
        tk = self._toks(toks)
        out = np.empty((len(tk), self.H), np.float64)
        lib().oracle_bruteforce(C.byref(self.cfg), C.byref(self.wset), _p(x), _p(ids), _p(w), len(tk),
                                _p(tk), _p(out))
        return out

    def gemm1(self, xq, xs, row_token, offsets, rows: Sequence[int]):
        """(h fp32 [n,I], hq, hs) for the listed rows; hq / hs in the layer's
        activation format (FP8: uint8 [n,I], fp32 [n,I/G]; MXFP4: uint8
        [n,I/2], uint8 [n,I/32])."""
        sdt, _ = self._sdt(self.H)
        xq, xs = _np(xq, np.uint8), _np(xs, sdt)
        rt, off = _np(row_token, np.int32), _np(offsets, np.int32)
        rr = np.ascontiguousarray(np.asarray(list(rows), np.int64))
        n = len(rr)
        h = np.empty((n, self.I), np.float32)
        hq = np.empty((n, self._cb(self.I)), np.uint8)
        hs = np.empty((n, self._sdt(self.I)[1]), sdt)
        lib().oracle_gemm1(C.byref(self.cfg), C.byref(self.wset), _p(xq), _p(xs), _p(rt), _p(off), n,
                           _p(rr), _p(h), _p(hq), _p(hs))
        return h, hq, hs

    def gemm2(self, hq, hs, offsets, rows: Sequence[int]) -> np.ndarray:
        """fp64 y [n,H] for the listed rows (hq/hs indexed by row id)."""
        hq, hs, off = _np(hq, np.uint8), _np(hs, self._sdt(self.I)[0]), _np(offsets, np.int32)
        rr = np.ascontiguousarray(np.asarray(list(rows), np.int64))
        y = np.empty((len(rr), self.H), np.float64)
        lib().oracle_gemm2(C.byref(self.cfg), C.byref(self.wset), _p(hq), _p(hs), _p(off), len(rr),
                           _p(rr), _p(y))
        return y

    def combine(self, y, expand_idx, offsets, topk_w, toks: Optional[Sequence[int]] = None):
        y, ei = _np(y, np.float32), _np(expand_idx, np.int32)
        off, w = _np(offsets, np.int32), _np(topk_w, np.float32)
        tk = self._toks(toks)
        out = np.empty((len(tk), self.H), np.float64)
        lib().oracle_combine(C.byref(self.cfg), _p(y), _p(ei), _p(off), _p(w), len(tk), _p(tk), _p(out))
        return out


def layer_for(wl, T: int, weights) -> Layer:
    return Layer.for_workload(wl, T, weights)
