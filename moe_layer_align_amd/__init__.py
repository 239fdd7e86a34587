"""MI355X (gfx950) fused Mixture-of-Experts layer.

Thin ctypes binding over libmoe_mi355x.so, the C ABI in include/moe.h.  The
functions here only check tensor shapes/dtypes/devices and marshal pointers;
every step of the layer runs in the library's HIP kernels.  PyTorch provides
device memory and the current stream.  There is no fallback: if the library
is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "MoEError", "load", "LIB_PATH", "route_topk", "router_logits", "align_capacity", "align", "quant_e4m3",
    "workspace_size", "fused_align_shape", "fused_forward", "Tuning", "STATUS", "NUM_STAGES", "STAGE_NAMES",
    "NOALLOC_SCRATCH_BYTES", "fused_path", "PATH_NAMES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE_TOO_SMALL",
          4: "MOE_ERR_DEVICE"}
DTYPE_BF16, DTYPE_FP8 = 0, 1
NUM_STAGES = 5
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
STAGE_NAMES = ("route", "align", "gate_up", "down", "finalize")
# moe_fused_path's MOE_PATH_* values, in order
PATH_NAMES = ("none", "prefill", "decode", "decode_token_down", "two_launches", "single_launch")


class MoEError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(code, "?"), code))
        self.code = code


class Tuning(ctypes.Structure):
    _fields_ = [("gemm1_ksplit", ctypes.c_int32), ("gemm2_ksplit", ctypes.c_int32),
                ("token_tiles", ctypes.c_int32), ("unroll", ctypes.c_int32),
                ("gemm2_wave_ksplit", ctypes.c_int32), ("gemm1_stream_tiles", ctypes.c_int32),
                ("gemm2_stream_tiles", ctypes.c_int32), ("reverse_order", ctypes.c_int32),
                ("single_launch", ctypes.c_int32), ("down_per_token", ctypes.c_int32),
                ("routing_in_gate_up", ctypes.c_int32), ("gemm1_feature_tiles", ctypes.c_int32),
                ("gemm2_row_tiles", ctypes.c_int32)]


class _FusedArgs(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int32), ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
        ("h_scale", ctypes.c_void_p), ("y", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p),
        ("topk_weights", ctypes.c_void_p), ("expert_counts", ctypes.c_void_p), ("scales_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("tuning", ctypes.POINTER(Tuning)),
        ("weight_scale_mode", ctypes.c_int32),
        ("router_w", ctypes.c_void_p), ("logits_out", ctypes.c_void_p),
        ("n_shared", ctypes.c_int32),
        ("expert_offsets", ctypes.c_void_p), ("sorted_ids", ctypes.c_void_p), ("block_expert", ctypes.c_void_p),
        ("num_padded", ctypes.c_void_p),
        ("deterministic", ctypes.c_int32),
    ]


_lib = None
_ABI = 15  # moe_abi_version() of the library whose moe_fused_args_t _FusedArgs mirrors


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoe_mi355x.so is not built (run `python -c 'import __graft_entry__ as g; g.build()'`)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_abi_version.restype = i32
    lib.moe_route_topk.restype = ctypes.c_int
    lib.moe_route_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.moe_align_capacity.restype = sz
    lib.moe_align_capacity.argtypes = [i32, i32, i32, i32]
    lib.moe_align.restype = ctypes.c_int
    lib.moe_align.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.moe_router_logits.restype = ctypes.c_int
    lib.moe_router_logits.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.moe_quant_e4m3.restype = ctypes.c_int
    lib.moe_quant_e4m3.argtypes = [vp, i64, vp, vp, vp]
    lib.moe_fused_workspace_size.restype = sz
    lib.moe_fused_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.moe_fused_align_shape.restype = ctypes.c_int
    lib.moe_fused_align_shape.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, i32, i32, vp, vp]
    lib.moe_fused_forward.restype = ctypes.c_int
    lib.moe_fused_forward.argtypes = [ctypes.POINTER(_FusedArgs), vp]
    lib.moe_fused_forward_profiled.restype = ctypes.c_int
    lib.moe_fused_forward_profiled.argtypes = [ctypes.POINTER(_FusedArgs), vp, vp]
    lib.moe_fused_forward_noalloc.restype = ctypes.c_int
    lib.moe_fused_path.restype = ctypes.c_int
    lib.moe_fused_path.argtypes = [ctypes.POINTER(_FusedArgs), ctypes.POINTER(i32)]
    lib.moe_fused_forward_noalloc.argtypes = [ctypes.POINTER(_FusedArgs), vp]
    if lib.moe_abi_version() != _ABI:
        raise RuntimeError("libmoe_mi355x.so has ABI version %d, this binding expects %d: rebuild it"
                           % (lib.moe_abi_version(), _ABI))
    _lib = lib
    return lib


def _check(fn: str, code: int):
    if code != 0:
        raise MoEError(fn, code)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _keep_for(t: torch.Tensor, stream) -> None:
    """For a tensor the binding allocates and drops while the call that uses
    it runs on another stream than the current one: tell torch's caching
    allocator, so that the memory is not handed out again before that
    stream's work is done."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream(stream))
    if s.cuda_stream != torch.cuda.current_stream(t.device).cuda_stream:
        t.record_stream(s)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, shape: Sequence[int]):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def route_topk(logits: torch.Tensor, top_k: int, ids: Optional[torch.Tensor] = None,
               weights: Optional[torch.Tensor] = None, stream=None):
    """Top-k experts per token and their softmax weights (moe_route_topk)."""
    M, E = logits.shape
    _need(logits, "logits", torch.float32, (M, E))
    if ids is None:
        ids = torch.empty(M, top_k, dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty(M, top_k, dtype=torch.float32, device=logits.device)
    _need(ids, "ids", torch.int32, (M, top_k))
    _need(weights, "weights", torch.float32, (M, top_k))
    _check("moe_route_topk", load().moe_route_topk(_ptr(logits), M, E, top_k, _ptr(ids), _ptr(weights),
                                                   _stream(stream)))
    return ids, weights


def router_logits(x: torch.Tensor, router_w: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """logits = x . router_w^T (moe_router_logits): x bf16 [M,H], router_w bf16
    [E,H] -> fp32 [M,E]."""
    M, H = x.shape
    E = router_w.shape[0]
    _need(x, "x", torch.bfloat16, (M, H))
    _need(router_w, "router_w", torch.bfloat16, (E, H))
    if out is None:
        out = torch.empty(M, E, dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (M, E))
    _check("moe_router_logits", load().moe_router_logits(_ptr(x), _ptr(router_w), M, E, H, _ptr(out), _stream(stream)))
    return out


def align_capacity(M: int, top_k: int, E: int, block: int) -> int:
    return int(load().moe_align_capacity(M, top_k, E, block))


def align(ids: torch.Tensor, E: int, block: int, stream=None):
    """Sort-and-pad of the (token, slot) pairs by expert (moe_align)."""
    M, k = ids.shape
    _need(ids, "ids", torch.int32, (M, k))
    cap = align_capacity(M, k, E, block)
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(cap // block, 1), dtype=torch.int32, device=dev)
    num = torch.empty(1, dtype=torch.int32, device=dev)
    _check("moe_align", load().moe_align(_ptr(ids), M, k, E, block, _ptr(counts), _ptr(offsets), _ptr(sorted_ids),
                                         _ptr(block_expert), _ptr(num), _stream(stream)))
    return dict(counts=counts, offsets=offsets, sorted_ids=sorted_ids[:cap], block_expert=block_expert[:cap // block],
                num_padded=num)


def quant_e4m3(x: torch.Tensor, scale: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """e4m3 codes of fp32 data with a per-tensor scale (moe_quant_e4m3)."""
    _need(x, "x", torch.float32, x.shape)
    _need(scale, "scale", torch.float32, (1,))
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, "out", torch.uint8, x.shape)
    _check("moe_quant_e4m3", load().moe_quant_e4m3(_ptr(x), x.numel(), _ptr(scale), _ptr(out), _stream(stream)))
    return out


def workspace_size(M: int, E: int, H: int, I: int, top_k: int, dtype: str) -> int:
    return int(load().moe_fused_workspace_size(M, E, H, I, top_k, DTYPE_FP8 if dtype == "fp8" else DTYPE_BF16))


def fused_align_shape(M: int, E: int, H: int, I: int, top_k: int, dtype: str, deterministic: bool = False,
                      weight_scale_mode: int = 0):
    """(block, capacity) of the fused call's sort-and-pad step
    (moe_fused_align_shape); E and top_k count the shared experts."""
    b, c = ctypes.c_int32(0), ctypes.c_int64(0)
    _check("moe_fused_align_shape", load().moe_fused_align_shape(
        M, E, H, I, top_k, DTYPE_FP8 if dtype == "fp8" else DTYPE_BF16, int(bool(deterministic)),
        int(weight_scale_mode), ctypes.byref(b), ctypes.byref(c)))
    return int(b.value), int(c.value)


def fused_path(M: int, E: int, H: int, I: int, top_k: int, dtype: str = "bf16", n_shared: int = 0,
               weight_scale_mode: int = 0, static_x_scale: bool = False, static_h_scale: bool = False,
               router_w: bool = False, deterministic: bool = False, tuning: Optional[Tuning] = None) -> str:
    """Name (PATH_NAMES) of the launch sequence fused_forward takes on a call
    of this shape (moe_fused_path; host only, no GPU needed).  E and top_k
    count the routed experts; static_x_scale/static_h_scale: fp8 scales given
    by the caller; router_w: logits computed in the layer."""
    fp8 = dtype == "fp8"
    fake = 1 << 20  # moe_fused_path reads no memory through the pointers
    args = _FusedArgs(
        M=M, E=E, H=H, I=I, top_k=top_k, dtype=DTYPE_FP8 if fp8 else DTYPE_BF16, x=fake, w13=fake, w2=fake,
        logits=None if router_w else fake, router_w=fake if router_w else None,
        w13_scale=fake if fp8 else None, w2_scale=fake if fp8 else None,
        x_scale=fake if static_x_scale else None, h_scale=fake if static_h_scale else None,
        tuning=ctypes.pointer(tuning) if tuning is not None else None, weight_scale_mode=int(weight_scale_mode),
        n_shared=int(n_shared), deterministic=int(bool(deterministic)))
    p = ctypes.c_int32(-1)
    _check("moe_fused_path", load().moe_fused_path(ctypes.byref(args), ctypes.byref(p)))
    return PATH_NAMES[p.value]


def fused_forward(x: torch.Tensor, logits: Optional[torch.Tensor], w13: torch.Tensor, w2: torch.Tensor, top_k: int,
                  dtype: str = "bf16", w13_scale: Optional[torch.Tensor] = None,
                  w2_scale: Optional[torch.Tensor] = None, x_scale: Optional[torch.Tensor] = None,
                  h_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, topk_ids: Optional[torch.Tensor] = None,
                  topk_weights: Optional[torch.Tensor] = None, expert_counts: Optional[torch.Tensor] = None,
                  scales_out: Optional[torch.Tensor] = None, tuning: Optional[Tuning] = None, stream=None,
                  events=None, router_w: Optional[torch.Tensor] = None,
                  logits_out: Optional[torch.Tensor] = None, n_shared: int = 0,
                  align_out: Optional[dict] = None, deterministic: bool = False,
                  noalloc: bool = False) -> torch.Tensor:
    """The fused layer (moe_fused_forward).

    x bf16 [M,H]; logits fp32 [M,E]; w13 [E,2I,H] and w2 [E,H,I] as bf16
    (dtype "bf16") or uint8 e4m3fn codes (dtype "fp8") with fp32 device
    scales, either one per tensor ([1] each), one per weight row (w13_scale
    [E,2I], w2_scale [E,H]) or one per expert ([E] each), or uint8 E8M0 codes
    one per 128 x 128 block (w13_scale [E,2I/128,H/128], w2_scale
    [E,H/128,I/128]: block-scaled mode, activations scaled per 128 elements);
    x_scale/h_scale: static fp8 activation scales or None (dynamic).  logits may be None when router_w (bf16 [E,H]) is given:
    the layer then computes them (into logits_out fp32 [M,E] when given).
    n_shared: S shared experts stacked after the E routed ones (w13 [E+S,2I,H],
    w2 [E+S,H,I], per-row scales [E+S,..]), each taken by every token with
    weight one; topk_ids/topk_weights are then [M,top_k+S], expert_counts [E+S].
    events: optional list of 2*NUM_STAGES hipEvent_t handles (ints) recorded
    around the stages on the stream.
    align_out: optional dict of int32 GPU tensors receiving the call's
    sort-and-pad outputs: "offsets" [E+S+1], "sorted_ids" [capacity],
    "block_expert" [capacity/block], "num_padded" [1] (block and capacity
    from fused_align_shape; any subset of the keys).
    deterministic: batch-invariant mode (fp8 needs x_scale and h_scale).
    noalloc: call moe_fused_forward_noalloc, whose workspace is the library's
    own scratch array (no workspace may be given; `out` must be given, so
    that the call allocates nothing here either).
    """
    M, H = x.shape
    if (logits is None) == (router_w is None):
        raise ValueError("give exactly one of logits and router_w")
    E = logits.shape[1] if logits is not None else router_w.shape[0]
    fp8 = dtype == "fp8"
    I = w2.shape[2]
    S = int(n_shared)
    ES, KS = E + S, top_k + S
    wdt = torch.uint8 if fp8 else torch.bfloat16
    _need(x, "x", torch.bfloat16, (M, H))
    if logits is not None:
        _need(logits, "logits", torch.float32, (M, E))
    else:
        _need(router_w, "router_w", torch.bfloat16, (E, H))
        if logits_out is not None:
            _need(logits_out, "logits_out", torch.float32, (M, E))
    _need(w13, "w13", wdt, (ES, 2 * I, H))
    _need(w2, "w2", wdt, (ES, H, I))
    # weight scale mode from the scale shapes: uint8 E8M0 codes
    # [E+S,2I/128,H/128] one per 128 x 128 block (3), [E+S,rows] one per row
    # (1), [E+S] with E+S > 1 one per expert (2), [1] one per tensor (0)
    mode = 0
    if w13_scale is not None and w13_scale.dtype == torch.uint8:
        mode = 3
        _need(w13_scale, "w13_scale", torch.uint8, (ES, 2 * I // 128, H // 128))
        _need(w2_scale, "w2_scale", torch.uint8, (ES, H // 128, I // 128))
    elif w13_scale is not None and w13_scale.dim() == 2:
        mode = 1
        _need(w13_scale, "w13_scale", torch.float32, (ES, 2 * I))
        _need(w2_scale, "w2_scale", torch.float32, (ES, H))
    elif w13_scale is not None and ES > 1 and w13_scale.numel() == ES:
        mode = 2
        _need(w13_scale, "w13_scale", torch.float32, (ES,))
        _need(w2_scale, "w2_scale", torch.float32, (ES,))
    for name, s in (("w13_scale", None if mode else w13_scale), ("w2_scale", None if mode else w2_scale),
                    ("x_scale", x_scale), ("h_scale", h_scale)):
        if s is not None:
            _need(s, name, torch.float32, (1,))
    if out is None:
        if noalloc:
            raise ValueError("the no-alloc call needs `out`")
        out = torch.empty(M, H, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (M, H))
    if topk_ids is not None:
        _need(topk_ids, "topk_ids", torch.int32, (M, KS))
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, (M, KS))
    if expert_counts is not None:
        _need(expert_counts, "expert_counts", torch.int32, (ES,))
    if scales_out is not None:
        _need(scales_out, "scales_out", torch.float32, (2,))
    al = dict(align_out or {})
    if set(al) - {"offsets", "sorted_ids", "block_expert", "num_padded"}:
        raise ValueError("unknown align_out keys: %s" % sorted(set(al) - {"offsets", "sorted_ids", "block_expert",
                                                                            "num_padded"}))
    if al:
        blk, cap = fused_align_shape(M, ES, H, I, KS, dtype, deterministic, mode)
        for key, shape in (("offsets", (ES + 1,)), ("sorted_ids", (cap,)), ("block_expert", (cap // blk,)),
                           ("num_padded", (1,))):
            if key in al:
                _need(al[key], "align_out[%s]" % key, torch.int32, shape)
    lib = load()
    if noalloc:
        if workspace is not None:
            raise ValueError("the no-alloc call takes no workspace")
    else:
        need = int(lib.moe_fused_workspace_size(M, ES, H, I, KS, DTYPE_FP8 if fp8 else DTYPE_BF16))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
            _keep_for(workspace, stream)
        if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    args = _FusedArgs(
        M=M, E=E, H=H, I=I, top_k=top_k, dtype=DTYPE_FP8 if fp8 else DTYPE_BF16,
        x=_ptr(x), logits=_ptr(logits), w13=_ptr(w13), w2=_ptr(w2),
        w13_scale=_ptr(w13_scale), w2_scale=_ptr(w2_scale), x_scale=_ptr(x_scale), h_scale=_ptr(h_scale),
        y=_ptr(out), topk_ids=_ptr(topk_ids), topk_weights=_ptr(topk_weights),
        expert_counts=_ptr(expert_counts), scales_out=_ptr(scales_out),
        workspace=_ptr(workspace), workspace_bytes=0 if workspace is None else workspace.numel(),
        tuning=ctypes.pointer(tuning) if tuning is not None else None,
        weight_scale_mode=mode,
        router_w=_ptr(router_w), logits_out=_ptr(logits_out), n_shared=S,
        expert_offsets=_ptr(al.get("offsets")), sorted_ids=_ptr(al.get("sorted_ids")),
        block_expert=_ptr(al.get("block_expert")), num_padded=_ptr(al.get("num_padded")),
        deterministic=int(bool(deterministic)),
    )
    if noalloc:
        if events is not None:
            raise ValueError("the no-alloc call records no stage events")
        _check("moe_fused_forward_noalloc", lib.moe_fused_forward_noalloc(ctypes.byref(args), _stream(stream)))
    elif events is None:
        _check("moe_fused_forward", lib.moe_fused_forward(ctypes.byref(args), _stream(stream)))
    else:
        if len(events) != 2 * NUM_STAGES:
            raise ValueError("events must hold %d hipEvent_t handles" % (2 * NUM_STAGES))
        arr = (ctypes.c_void_p * len(events))(*events)
        _check("moe_fused_forward_profiled",
               lib.moe_fused_forward_profiled(ctypes.byref(args), _stream(stream), ctypes.cast(arr, ctypes.c_void_p)))
    return out
