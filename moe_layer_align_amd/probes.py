"""ctypes binding of the measurement probes (libmoe_probes.so, declared in
include/moe_probes.h): argument marshalling only, every probe runs in its
HIP kernel.  Not part of the layer; bench.py reports what they measure
beside the nameplate peaks."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import MoEError, _stream

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_probes.so")
_ABI = 4
_lib = None


def load():
    """Load libmoe_probes.so (built by moe_layer_align_amd.build); fails
    loudly when it is missing or stale."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("%s is missing: build it with moe_layer_align_amd.build.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_probes_abi_version.restype = ctypes.c_int32
    if lib.moe_probes_abi_version() != _ABI:
        raise RuntimeError("libmoe_probes.so is a stale build (ABI %d, expected %d)" % (lib.moe_probes_abi_version(), _ABI))
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.moe_probe_hbm_read.restype = ctypes.c_int
    lib.moe_probe_hbm_read.argtypes = [vp, sz, i32, vp, vp]
    lib.moe_probe_mfma_fp8_loop.restype = ctypes.c_int
    lib.moe_probe_mfma_fp8_loop.argtypes = [vp, i32, i32, i32, vp]
    lib.moe_probe_publish.restype = ctypes.c_int
    lib.moe_probe_publish.argtypes = [vp, vp, i32, i32, vp]
    lib.moe_probe_fp8_dot.restype = ctypes.c_int
    lib.moe_probe_fp8_dot.argtypes = [vp, vp, vp, i32, i32, ctypes.c_float, i32, vp]
    lib.moe_probe_ring_load.restype = ctypes.c_int
    lib.moe_probe_ring_load.argtypes = [vp, sz, i32, i32, i32, vp, vp]
    _lib = lib
    return lib


def _raise(rc: int, what: str):
    if rc != 0:
        raise MoEError(what, rc)


def hbm_read(buf: torch.Tensor, sink: torch.Tensor, grid: int, stream: Optional[torch.cuda.Stream] = None):
    """Streaming read of buf (contiguous GPU tensor, size a multiple of 16
    bytes) by `grid` workgroups; sink: uint32-sized int32 [grid] GPU tensor
    receiving each workgroup's XOR of the words it read."""
    if not (buf.is_cuda and buf.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32
            and sink.numel() >= grid):
        raise ValueError("buf: contiguous GPU tensor; sink: int32 GPU tensor of at least grid elements")
    s = _stream(stream)
    _raise(load().moe_probe_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(), grid, sink.data_ptr(), s),
           "moe_probe_hbm_read")


def mfma_fp8_loop(out: torch.Tensor, grid: int, iters: int, random_operands: bool = False,
                  stream: Optional[torch.cuda.Stream] = None):
    """fp8 MFMA issue loop (operands 1.0, or fixed pseudo-random bytes);
    out: float32 GPU tensor of at least grid*16 elements."""
    if not (out.is_cuda and out.dtype == torch.float32 and out.is_contiguous() and out.numel() >= grid * 16):
        raise ValueError("out: contiguous float32 GPU tensor of at least grid*16 elements")
    s = _stream(stream)
    _raise(load().moe_probe_mfma_fp8_loop(out.data_ptr(), grid, iters, int(bool(random_operands)), s),
           "moe_probe_mfma_fp8_loop")


def fp8_dot(A: torch.Tensor, B: torch.Tensor, sa: int = 127, sb: int = 127, c0: float = 0.0, form: int = 0,
            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """C [16,16] fp32 = c0 + 2^(sa-127) 2^(sb-127) A @ B.T for e4m3 codes A, B
    uint8 [16,128] on the GPU, as one fp8 matrix instruction (form 0) or four
    16x16x32 ones (form 1) compute it."""
    for t in (A, B):
        if not (t.is_cuda and t.dtype == torch.uint8 and t.shape == (16, 128) and t.is_contiguous()):
            raise ValueError("A and B: contiguous uint8 GPU tensors [16, 128]")
    C = torch.empty(16, 16, dtype=torch.float32, device=A.device)
    s = _stream(stream)
    _raise(load().moe_probe_fp8_dot(A.data_ptr(), B.data_ptr(), C.data_ptr(), sa, sb, float(c0), form, s),
           "moe_probe_fp8_dot")
    return C


def publish(buf: torch.Tensor, cnt: torch.Tensor, grid: int, mode: int, stream: Optional[torch.cuda.Stream] = None):
    """Every workgroup writes its 32 KB of buf (float32 GPU tensor of at least
    grid*8192 elements) and counts itself in at cnt[g % 1024] (int32 GPU
    tensor of 1024, caller-zeroed); mode 0 plain stores, 1 + an agent-scope
    release fence, 2 write-through stores."""
    if not (buf.is_cuda and buf.dtype == torch.float32 and buf.is_contiguous() and buf.numel() >= grid * 8192):
        raise ValueError("buf: contiguous float32 GPU tensor of at least grid*8192 elements")
    if not (cnt.is_cuda and cnt.dtype == torch.int32 and cnt.numel() >= 1024):
        raise ValueError("cnt: int32 GPU tensor of 1024 elements")
    _raise(load().moe_probe_publish(buf.data_ptr(), cnt.data_ptr(), grid, mode, _stream(stream)), "moe_probe_publish")


def ring_load(buf: torch.Tensor, sink: torch.Tensor, grid: int, steps: int, mode: int,
              stream: Optional[torch.cuda.Stream] = None):
    """The tiled prefill product's operand stream without its arithmetic
    (moe_probe_ring_load): `grid` workgroups walk `steps` 48 KB K-steps of buf
    (contiguous GPU tensor, size a multiple of 4096 bytes, 1.5 MiB..1 GiB)
    through a three-slot LDS ring; mode 0 direct-to-LDS loads, 1 register
    loads and LDS stores, 2 mode 0 plus the product's fragment reads, plus 4
    (K start rotated per workgroup), 8 (rows 4224 bytes apart) and 16 (a
    private 96 KB window per workgroup, re-read from L2), 32 (256 token rows, two
    slots) and 64 (256 token rows, 64-byte K-steps, four slots).  sink:
    int32 GPU tensor of at least grid*4 elements."""
    if not (buf.is_cuda and buf.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32
            and sink.numel() >= grid * 4):
        raise ValueError("buf: contiguous GPU tensor; sink: int32 GPU tensor of at least grid*4 elements")
    _raise(load().moe_probe_ring_load(buf.data_ptr(), buf.numel() * buf.element_size(), grid, steps, mode,
                                      sink.data_ptr(), _stream(stream)), "moe_probe_ring_load")
