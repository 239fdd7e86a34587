"""CPU oracle for the fused MoE layer (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It wraps oracle/moe_oracle.c, a plain scalar C
implementation of the layer's definition, through ctypes.  It shares no code
with the GPU library (moe_layer_align_amd), and the GPU library never falls
back to it.

Functions:
  build()                      compile moe_oracle.c with gcc
  route(logits, k)             -> ids int32 [M,k], weights fp32 [M,k]
  align(ids, E, B, cap)        -> counts, offsets, sorted_ids, block_expert, num_padded
  layer(inputs, tokens, ...)   -> y_ref float64 [len(tokens), H] and intermediates
  bf16_encode / e4m3_encode / e4m3_decode   number-format helpers (numpy)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_BF16 = 0
DTYPE_E4M3 = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no contraction, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _LayerArgs(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64),
        ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("k", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p),
        ("logits", ctypes.c_void_p),
        ("w13", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("w13_scale", ctypes.c_float), ("w2_scale", ctypes.c_float),
        ("x_scale_static", ctypes.c_int32), ("x_scale", ctypes.c_float),
        ("h_scale_static", ctypes.c_int32), ("h_scale", ctypes.c_float),
        ("tokens", ctypes.c_void_p), ("n_tokens", ctypes.c_int64),
        ("y", ctypes.c_void_p),
        ("ids", ctypes.c_void_p),
        ("weights", ctypes.c_void_p),
        ("s_x_out", ctypes.c_void_p),
        ("s_h_out", ctypes.c_void_p),
        ("all_pairs_h", ctypes.c_int32),
        ("w13_scale_rows", ctypes.c_void_p),
        ("w2_scale_rows", ctypes.c_void_p),
        ("n_shared", ctypes.c_int32),
        ("block_scaled", ctypes.c_int32),
        ("w13_block", ctypes.c_void_p),
        ("w2_block", ctypes.c_void_p),
    ]


_ABI = 5  # oracle_abi_version() of moe_oracle.c that this binding matches


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_abi_version.restype = ctypes.c_int
    if lib.oracle_abi_version() != _ABI:
        raise RuntimeError("oracle/liboracle.so is a stale build (ABI %d, expected %d): run oracle.build()"
                           % (lib.oracle_abi_version(), _ABI))
    lib.oracle_bf16_decode.restype = ctypes.c_double
    lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_encode.restype = ctypes.c_uint16
    lib.oracle_bf16_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_scale_from_amax.restype = ctypes.c_float
    lib.oracle_scale_from_amax.argtypes = [ctypes.c_float]
    lib.oracle_e8m0_value.restype = ctypes.c_double
    lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_block_quant.restype = ctypes.c_uint8
    lib.oracle_block_quant.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_route.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_align.restype = ctypes.c_int
    lib.oracle_align.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_layer.restype = ctypes.c_int
    lib.oracle_layer.argtypes = [ctypes.POINTER(_LayerArgs)]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_router_logits.restype = ctypes.c_int
    lib.oracle_router_logits.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _np(t) -> np.ndarray:
    """torch tensor or array -> contiguous numpy view (host)."""
    if hasattr(t, "detach"):
        import torch
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.numpy()
    return np.ascontiguousarray(t)


# ---------------------------------------------------------------- formats
def bf16_encode(v: np.ndarray) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    return np.array([lib.oracle_bf16_encode(float(a)) for a in v], dtype=np.uint16)


def bf16_decode(c: np.ndarray) -> np.ndarray:
    lib = _load()
    return np.array([lib.oracle_bf16_decode(int(a)) for a in np.ravel(c)], dtype=np.float64)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    return np.array([lib.oracle_e4m3_encode(float(a)) for a in v], dtype=np.uint8)


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    lib = _load()
    return np.array([lib.oracle_e4m3_decode(int(a)) for a in np.ravel(c)], dtype=np.float64)


def e8m0_value(c: int) -> float:
    """Value of an E8M0 scale code: 2^(c-127) (NaN for 255)."""
    return float(_load().oracle_e8m0_value(int(c)))


def block_quant(v: np.ndarray):
    """Block quantisation of up to 128 fp32 values sharing one power-of-two
    scale (oracle_block_quant): returns (e4m3 codes uint8 [n], scale code)."""
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    if not 1 <= v.size <= 128:
        raise ValueError("a block holds 1..128 values")
    codes = np.zeros(v.size, dtype=np.uint8)
    c = lib.oracle_block_quant(_ptr(v), v.size, _ptr(codes))
    return codes, int(c)


def num_threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def scale_from_amax(amax: float) -> float:
    return float(_load().oracle_scale_from_amax(float(amax)))


# ---------------------------------------------------------------- routing
def route(logits, k: int):
    lib = _load()
    lg = np.ascontiguousarray(_np(logits), dtype=np.float32)
    M, E = lg.shape
    ids = np.zeros((M, k), dtype=np.int32)
    w = np.zeros((M, k), dtype=np.float32)
    rc = lib.oracle_route(_ptr(lg), M, E, k, _ptr(ids), _ptr(w))
    if rc:
        raise ValueError("oracle_route failed with code %d" % rc)
    return ids, w


def align_capacity(P: int, E: int, B: int) -> int:
    """Upper bound on the padded length: every expert that holds a pair can
    add at most B-1 sentinels, and at most min(E, P) experts hold one."""
    cap = P + min(E, P) * (B - 1)
    return ((cap + B - 1) // B) * B


def align(ids, E: int, B: int, capacity: Optional[int] = None):
    lib = _load()
    f = np.ascontiguousarray(_np(ids), dtype=np.int32).ravel()
    P = f.size
    cap = align_capacity(P, E, B) if capacity is None else capacity
    counts = np.zeros(E, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    sorted_ids = np.full(max(cap, 1), -7, dtype=np.int32)
    nblk = max(cap // B, 1)
    block_expert = np.full(nblk, -7, dtype=np.int32)
    num = np.zeros(1, dtype=np.int32)
    rc = lib.oracle_align(_ptr(f), P, E, B, _ptr(counts), _ptr(offsets), _ptr(sorted_ids), cap,
                          _ptr(block_expert), cap // B, _ptr(num))
    if rc:
        raise ValueError("oracle_align failed with code %d" % rc)
    return dict(counts=counts, offsets=offsets, sorted_ids=sorted_ids[:cap], block_expert=block_expert[:cap // B],
                num_padded=int(num[0]))


# ---------------------------------------------------------------- layer
def router_logits(x, w) -> np.ndarray:
    """Router logits x . w^T for bf16 x [M,H] and bf16 router weights w [E,H]:
    fp32 [M,E], each a double sum over t ascending rounded once."""
    lib = _load()
    xa, wa = _np(x), _np(w)
    if xa.dtype != np.uint16 or wa.dtype != np.uint16:
        raise TypeError("x and w must be bf16")
    M, H = xa.shape
    E = wa.shape[0]
    if wa.shape[1] != H:
        raise ValueError("w must be [E,H]")
    out = np.zeros((M, E), dtype=np.float32)
    rc = lib.oracle_router_logits(_ptr(xa) if xa.size else None, _ptr(wa), M, E, H, _ptr(out) if out.size else None)
    if rc:
        raise ValueError("oracle_router_logits failed with code %d" % rc)
    return out


def layer(x, logits, w13, w2, k: int, dtype: str, w13_scale: Optional[float] = None,
          w2_scale: Optional[float] = None, x_scale: Optional[float] = None, h_scale: Optional[float] = None,
          tokens: Optional[Sequence[int]] = None, experts: Optional[dict] = None, all_pairs_h: Optional[bool] = None,
          n_shared: int = 0, w13_block=None, w2_block=None):
    """Reference output of the layer.

    x: bf16 [M,H]; logits fp32 [M,E]; w13 [E,2I,H] / w2 [E,H,I] (bf16 or e4m3
    codes), or None together with `experts`, a dict e -> (w13_e, w2_e) holding
    only the experts that are needed.  w13_scale/w2_scale (fp8): one float per
    tensor, arrays [E,2I] / [E,H] with one scale per weight row, or arrays
    [E] with one per expert.  x_scale/h_scale: static fp8 activation
    scales, None = dynamic amax/448.  tokens: rows of y to produce (default all).
    n_shared: shared experts stacked after the E routed ones (w13 [E+n_shared,2I,H],
    per-row scales [E+n_shared,..]); every token passes through each with weight one.
    w13_block/w2_block (fp8, block-scaled mode, instead of w13_scale/w2_scale):
    uint8 E8M0 codes [E+n_shared, 2I/128, H/128] and [E+n_shared, H/128, I/128],
    one per 128 x 128 weight block; activations are then quantised per 128
    elements (block_quant) and s_x, s_h are reported as 0.
    Returns dict(y=float64 [T,H], ids, weights, s_x, s_h).
    """
    lib = _load()
    xa = _np(x)
    if xa.dtype != np.uint16:
        raise TypeError("x must be bf16")
    lg = np.ascontiguousarray(_np(logits), dtype=np.float32)
    M, H = xa.shape
    E = lg.shape[1]
    fp8 = dtype == "fp8"
    EW = E + n_shared  # expert weight sets: routed, then shared
    keep = []  # keep numpy buffers alive
    p13 = (ctypes.c_void_p * EW)()
    p2 = (ctypes.c_void_p * EW)()
    I = None
    if experts is None:
        a13, a2 = _np(w13), _np(w2)
        keep += [a13, a2]
        if a13.shape[0] != EW or a2.shape[0] != EW:
            raise ValueError("w13/w2 must hold E + n_shared = %d experts" % EW)
        I = a13.shape[1] // 2
        for e in range(EW):
            p13[e] = a13[e].ctypes.data
            p2[e] = a2[e].ctypes.data
    else:
        for e in range(EW):
            if e in experts:
                a13, a2 = _np(experts[e][0]), _np(experts[e][1])
                keep += [a13, a2]
                I = a13.shape[0] // 2
                p13[e] = a13.ctypes.data
                p2[e] = a2.ctypes.data
            else:
                p13[e] = None
                p2[e] = None
    if tokens is None:
        tokens = list(range(M))
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    y = np.zeros((len(tok), H), dtype=np.float64)
    ids = np.zeros((M, k), dtype=np.int32)
    w = np.zeros((M, k), dtype=np.float32)
    sx = np.zeros(1, dtype=np.float32)
    sh = np.zeros(1, dtype=np.float32)
    if all_pairs_h is None:
        all_pairs_h = fp8 and h_scale is None and w13_block is None

    def scale_rows(sc, rows):
        # one scale per weight row: E pointers to that expert's fp32 row scales;
        # one scale per expert ([E], E > 1) is every row of that expert at it
        if sc is None or np.ndim(_np(sc)) == 0 or np.size(_np(sc)) == 1:
            return None
        arr = np.ascontiguousarray(_np(sc), dtype=np.float32)
        if arr.shape == (EW,):
            arr = np.ascontiguousarray(np.repeat(arr[:, None], rows, axis=1))
        if arr.shape != (EW, rows):
            raise ValueError("per-row scales must have shape %s, got %s" % ((EW, rows), arr.shape))
        keep.append(arr)
        ptrs = (ctypes.c_void_p * EW)(*[arr[e].ctypes.data for e in range(EW)])
        keep.append(ptrs)
        return ctypes.cast(ptrs, ctypes.c_void_p)

    blk = w13_block is not None
    if blk != (w2_block is not None) or (blk and not fp8):
        raise ValueError("block scales need both w13_block and w2_block, in fp8 mode")
    rows13 = scale_rows(w13_scale, 2 * I) if fp8 and not blk else None
    rows2 = scale_rows(w2_scale, H) if fp8 and not blk else None

    def block_ptrs(b, shape):
        arr = np.ascontiguousarray(_np(b), dtype=np.uint8)
        if arr.shape != (EW,) + shape:
            raise ValueError("block scales must have shape %s, got %s" % ((EW,) + shape, arr.shape))
        keep.append(arr)
        ptrs = (ctypes.c_void_p * EW)(*[arr[e].ctypes.data for e in range(EW)])
        keep.append(ptrs)
        return ctypes.cast(ptrs, ctypes.c_void_p)

    b13 = block_ptrs(w13_block, (2 * I // 128, H // 128)) if blk else None
    b2 = block_ptrs(w2_block, (H // 128, I // 128)) if blk else None
    args = _LayerArgs(
        M=M, E=E, H=H, I=I, k=k, dtype=DTYPE_E4M3 if fp8 else DTYPE_BF16,
        x=_ptr(xa), logits=_ptr(lg),
        w13=ctypes.cast(p13, ctypes.c_void_p), w2=ctypes.cast(p2, ctypes.c_void_p),
        w13_scale=0.0 if rows13 else float(w13_scale or 0.0), w2_scale=0.0 if rows2 else float(w2_scale or 0.0),
        x_scale_static=int(x_scale is not None), x_scale=float(x_scale or 0.0),
        h_scale_static=int(h_scale is not None), h_scale=float(h_scale or 0.0),
        tokens=_ptr(tok) if tok.size else None, n_tokens=tok.size,
        y=_ptr(y) if y.size else None, ids=_ptr(ids) if ids.size else None, weights=_ptr(w) if w.size else None,
        s_x_out=_ptr(sx), s_h_out=_ptr(sh), all_pairs_h=int(bool(all_pairs_h)),
        w13_scale_rows=rows13, w2_scale_rows=rows2, n_shared=int(n_shared),
        block_scaled=int(blk), w13_block=b13, w2_block=b2,
    )
    rc = lib.oracle_layer(ctypes.byref(args))
    if rc:
        raise ValueError("oracle_layer failed with code %d" % rc)
    return dict(y=y, ids=ids, weights=w, s_x=float(sx[0]), s_h=float(sh[0]))
