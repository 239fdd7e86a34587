"""Host-only checks of the C ABI (no GPU needed).

The library loads, exports every function include/moe.h declares, and its
host-only helpers and argument validation behave as documented: invalid
calls return their error code before anything is enqueued (so they never
touch a device).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    import moe_layer_align_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built; run __graft_entry__.build()")
    return m.load()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_route_topk", "moe_align", "moe_fused_forward", "moe_align_capacity",
              "moe_fused_workspace_size", "moe_status_string", "moe_quant_e4m3", "moe_router_logits",
              "moe_fused_align_shape"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_probe_library_exports_its_header():
    # the measurement probes' library (include/moe_probes.h): loads on the
    # CPU, exports every declared function, and rejects bad arguments before
    # any launch
    from moe_layer_align_amd import probes
    if not os.path.exists(probes.LIB_PATH):
        pytest.fail("libmoe_probes.so is not built; run __graft_entry__.build()")
    plib = probes.load()
    names = declared_functions(os.path.join(ROOT, "include", "moe_probes.h"))
    assert set(names) >= {"moe_probes_abi_version", "moe_probe_hbm_read", "moe_probe_mfma_fp8_loop",
                          "moe_probe_fp8_dot", "moe_probe_publish", "moe_probe_ring_load"}
    for n in names:
        assert hasattr(plib, n), n
    assert plib.moe_probe_hbm_read(None, 16, 1, 16, None) == 1
    assert plib.moe_probe_hbm_read(16, 15, 1, 16, None) == 1       # size not a multiple of 16
    assert plib.moe_probe_hbm_read(16, 16, 0, 16, None) == 1       # empty grid
    assert plib.moe_probe_mfma_fp8_loop(16, 1, 0, 0, None) == 1     # no iterations
    assert plib.moe_probe_mfma_fp8_loop(16, 1, 1, 2, None) == 1     # unknown operand mode
    assert plib.moe_probe_fp8_dot(16, 16, 16, 255, 127, 0.0, 0, None) == 1  # NaN scale code
    assert plib.moe_probe_fp8_dot(16, 16, 16, 120, 127, 0.0, 1, None) == 1  # form 1 has no scales
    assert plib.moe_probe_fp8_dot(16, 16, 16, 127, 127, 0.0, 2, None) == 1  # unknown form
    assert plib.moe_probe_publish(16, 16, 1, 3, None) == 1                    # unknown mode
    assert plib.moe_probe_publish(16, 16, 0, 0, None) == 1                    # empty grid
    rl, MB = plib.moe_probe_ring_load, 1 << 20
    assert rl(16, 4 * MB, 1, 3, 3, 16, None) == 1          # unknown mode
    assert rl(16, 4 * MB, 1, 3, 128, 16, None) == 1        # unknown flag
    assert rl(16, 4 * MB, 1, 3, 64 + 32, 16, None) == 1    # 64-byte steps with another flag
    assert rl(16, 4 * MB, 1, 3, 64 + 1, 16, None) == 1     # 64-byte steps of register loads
    assert rl(16, 4 * MB, 1, 3, 33, 16, None) == 1         # two-slot ring of register loads
    assert rl(16, 4 * MB, 1, 4, 0, 16, None) == 1          # steps not a multiple of 3
    assert rl(16, 4 * MB + 16, 1, 3, 0, 16, None) == 1     # size not a multiple of 4096
    assert rl(16, 512 * 4224 - 4096, 1, 3, 0, 16, None) == 1  # below 512 padded rows
    assert rl(16, 2048 * MB, 1, 3, 0, 16, None) == 1       # above 1 GiB
    assert rl(16, 4 * MB, 0, 3, 0, 16, None) == 1          # empty grid
    assert rl(None, 4 * MB, 1, 3, 0, 16, None) == 1


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"
    assert lib.moe_abi_version() == 15


def capacity_formula(M, k, E, B):
    P = M * k
    cap = P + min(E, P) * (B - 1)
    return -(-cap // B) * B


@pytest.mark.parametrize("M,k,E,B", [(0, 2, 8, 16), (1, 2, 8, 16), (63, 2, 8, 64), (4096, 8, 128, 64),
                                     (128, 8, 256, 16), (5, 16, 512, 256), (3, 1, 1, 1)])
def test_align_capacity(lib, M, k, E, B):
    assert lib.moe_align_capacity(M, k, E, B) == capacity_formula(M, k, E, B)


def test_align_capacity_invalid(lib):
    assert lib.moe_align_capacity(4, 3, 2, 16) == 0     # k > E
    assert lib.moe_align_capacity(4, 2, 8, 24) == 0     # not a power of two
    assert lib.moe_align_capacity(4, 2, 8, 512) == 0    # block too large
    assert lib.moe_align_capacity(-1, 2, 8, 16) == 0
    assert lib.moe_align_capacity(4, 2, 1024, 16) == 0  # E beyond the envelope


def test_workspace_size(lib):
    bf = lib.moe_fused_workspace_size(4, 8, 256, 512, 2, 0)
    f8 = lib.moe_fused_workspace_size(4, 8, 256, 512, 2, 1)
    assert bf > 0 and f8 > 0 and bf % 256 == 0
    # the fp32 partial outputs of the down product (at least one K slice) and the h buffer alone
    assert bf >= 8 * 256 * 4 + 8 * 512 * 2
    assert lib.moe_fused_workspace_size(4, 8, 200, 512, 2, 0) == 0  # H not a multiple of 128
    assert lib.moe_fused_workspace_size(4, 8, 256, 512, 2, 7) == 0  # unknown dtype


def align_shape(lib, M, E, H, I, k, dtype, det=0, mode=0):
    b, c = ctypes.c_int32(-1), ctypes.c_int64(-1)
    rc = lib.moe_fused_align_shape(M, E, H, I, k, dtype, det, mode, ctypes.byref(b), ctypes.byref(c))
    return rc, b.value, c.value


@pytest.mark.parametrize("M,E,H,I,k,dtype,det,mode,block", [
    (4, 8, 256, 512, 2, 0, 0, 0, 16),          # decode
    (4096, 128, 4096, 1536, 8, 1, 0, 0, 128),  # fp8 with 32768 pairs: prefill path
    (4096, 128, 4096, 1536, 8, 1, 1, 0, 16),   # deterministic mode: decode path at every M
    (4096, 128, 4096, 1536, 8, 1, 0, 3, 16),   # block-scaled: decode path at every M
    (4096, 128, 4096, 1536, 8, 1, 0, 1, 128),  # per-row scales: prefill path
    (4096, 128, 4096, 1536, 8, 0, 0, 0, 128),  # bf16 with 32768 pairs: prefill path too
    (4096, 128, 4096, 1536, 8, 0, 1, 0, 16),   # bf16, deterministic mode: decode path
    (1023, 8, 512, 512, 8, 1, 0, 0, 16),       # 8184 pairs: below the prefill threshold
    (1024, 8, 512, 512, 8, 1, 0, 0, 128),      # 8192 pairs
])
def test_fused_align_shape(lib, M, E, H, I, k, dtype, det, mode, block):
    rc, b, c = align_shape(lib, M, E, H, I, k, dtype, det, mode)
    assert rc == 0 and b == block and c == capacity_formula(M, k, E, block)
    # the workspace holds the sort-and-pad arrays of both modes
    assert lib.moe_fused_workspace_size(M, E, H, I, k, dtype) >= 4 * c + 4 * (c // b)


def test_fused_align_shape_invalid(lib):
    assert align_shape(lib, 4, 8, 256, 512, 9, 0)[0] == 1     # k > E
    assert align_shape(lib, 4, 8, 256, 512, 2, 3)[0] == 1     # unknown dtype
    assert align_shape(lib, 4, 8, 256, 512, 2, 0, 2)[0] == 1  # unknown mode
    assert align_shape(lib, 4, 8, 256, 512, 2, 1, 0, 4)[0] == 1  # unknown weight scale mode
    assert align_shape(lib, 4, 8, 256, 512, 2, 0, 0, 3)[0] == 1  # block-scaled bf16
    assert align_shape(lib, 4, 8, 200, 512, 2, 0)[0] == 2     # H not a multiple of 128
    b = ctypes.c_int32(0)
    assert lib.moe_fused_align_shape(4, 8, 256, 512, 2, 0, 0, 0, ctypes.byref(b), None) == 1


FAKE = 0x10000  # a 256-byte aligned non-null address; never dereferenced on these paths


def test_route_validation(lib):
    r = lib.moe_route_topk
    assert r(FAKE, 4, 8, 9, FAKE, FAKE, None) == 1      # k > E
    assert r(FAKE, 4, 8, 0, FAKE, FAKE, None) == 1      # k < 1
    assert r(FAKE, -1, 8, 2, FAKE, FAKE, None) == 1     # M < 0
    assert r(FAKE, 4, 600, 2, FAKE, FAKE, None) == 2    # E beyond 512
    assert r(FAKE, 4, 64, 17, FAKE, FAKE, None) == 2    # k beyond 16
    assert r(None, 4, 8, 2, FAKE, FAKE, None) == 1      # null logits
    assert r(FAKE + 2, 4, 8, 2, FAKE, FAKE, None) == 1  # misaligned
    assert r(None, 0, 8, 2, None, None, None) == 0      # M = 0: nothing to do


def test_align_validation(lib):
    a = lib.moe_align
    assert a(FAKE, 4, 2, 8, 24, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1   # block not a power of two
    assert a(FAKE, 4, 2, 8, 512, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2  # block too large
    assert a(FAKE, 4, 3, 2, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1   # k > E
    assert a(None, 4, 2, 8, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1   # null ids
    assert a(FAKE, 4, 2, 8, 16, None, FAKE, FAKE, FAKE, FAKE, None) == 1   # null counts
    assert a(FAKE, 4, 2, 8, 16, FAKE, FAKE, FAKE + 1, FAKE, FAKE, None) == 1  # misaligned


def test_quant_validation(lib):
    q = lib.moe_quant_e4m3
    assert q(FAKE, -1, FAKE, FAKE, None) == 1
    assert q(None, 10, FAKE, FAKE, None) == 1
    assert q(FAKE + 4, 10, FAKE, FAKE, None) == 1  # input needs 16-byte alignment
    assert q(None, 0, None, None, None) == 0


def fused_args(**kw):
    import moe_layer_align_amd as m
    base = dict(M=4, E=8, H=256, I=512, top_k=2, dtype=0, x=FAKE, logits=FAKE, w13=FAKE, w2=FAKE, y=FAKE,
                workspace=FAKE, workspace_bytes=1 << 30)
    base.update(kw)
    return m._FusedArgs(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=9), 1),
    (dict(M=-1), 1),
    (dict(dtype=5), 1),
    (dict(H=200), 2),
    (dict(I=64), 2),
    (dict(E=1024), 2),
    (dict(x=None), 1),
    (dict(w13=FAKE + 8), 1),
    (dict(workspace=FAKE + 16), 1),
    (dict(workspace_bytes=100), 3),
    (dict(w13_scale=FAKE), 1),           # a scale in bf16 mode
    (dict(dtype=1), 1),                  # fp8 without weight scales
    (dict(dtype=1, w13_scale=FAKE, w2_scale=FAKE + 1), 1),  # misaligned scale
    (dict(weight_scale_mode=1), 1),                   # per-channel weight scales in bf16 mode
    (dict(dtype=1, w13_scale=FAKE, w2_scale=FAKE, weight_scale_mode=4), 1),  # unknown scale mode
    (dict(dtype=1, w13_scale=FAKE, w2_scale=FAKE, weight_scale_mode=3, x_scale=FAKE), 1),  # block: static x scale
    (dict(dtype=1, w13_scale=FAKE, w2_scale=FAKE, weight_scale_mode=3, h_scale=FAKE), 1),  # block: static h scale
    (dict(weight_scale_mode=3), 1),                                           # block-scaled in bf16 mode
    (dict(dtype=1, w13_scale=FAKE, w2_scale=FAKE, weight_scale_mode=-1), 1),  # unknown scale mode
    (dict(weight_scale_mode=2), 1),                          # per-expert weight scales in bf16 mode
    (dict(dtype=1, w13_scale=FAKE + 4, w2_scale=FAKE, weight_scale_mode=1), 1),  # rows need 16-byte alignment
    (dict(router_w=FAKE), 1),                                # both logits and router weights
    (dict(logits=None), 1),                                  # neither
    (dict(logits_out=FAKE), 1),                              # logits out without router weights
    (dict(logits=None, router_w=FAKE + 8), 1),               # misaligned router weights
    (dict(n_shared=-1), 1),                                  # negative shared-expert count
    (dict(n_shared=15), 2),                                  # top_k + shared above 16
    (dict(E=500, n_shared=13), 2),                           # E + shared above 512
    (dict(sorted_ids=FAKE + 2), 1),                          # misaligned align output
    (dict(num_padded=FAKE + 1), 1),                          # misaligned align output
    (dict(deterministic=2), 1),                              # unknown mode
    (dict(deterministic=1, dtype=1, w13_scale=FAKE, w2_scale=FAKE), 1),                # fp8: dynamic scales
    (dict(deterministic=1, dtype=1, w13_scale=FAKE, w2_scale=FAKE, x_scale=FAKE), 1),  # fp8: dynamic h scale
])
def test_fused_validation(lib, kw, code):
    args = fused_args(**kw)
    assert lib.moe_fused_forward(ctypes.byref(args), None) == code
    # the path query validates the same way, bar the workspace size
    p = ctypes.c_int32(-1)
    assert lib.moe_fused_path(ctypes.byref(args), ctypes.byref(p)) == (0 if code == 3 else code)
    assert (p.value >= 0) == (code == 3)


# The launch sequence of each workload shape, and of the modes that change it
# (moe_fused_path plans on the host; no GPU).
@pytest.mark.parametrize("name,M,path", [
    ("mixtral", 1, "decode_token_down"),  # 2 x 896 gate/up items: above the two-launch default's 1024
    ("mixtral", 4, "decode"), ("mixtral", 63, "decode"),
    ("qwen3", 1, "two_launches"),
    ("qwen3", 8, "two_launches"),  # 3072 gate/up items, but of 64 KB each; x of 16384 elements
    ("qwen3", 16, "decode"), ("qwen3", 64, "decode"),
    ("deepseek", 1, "two_launches"),
    ("deepseek", 2, "decode_token_down"),  # 2048 items of 229 KB: above the two-launch default's 1024
    ("deepseek", 16, "decode"),
    ("prefill", 4096, "prefill"), ("prefill", 0, "none"),
])
def test_fused_path_of_the_workloads(name, M, path):
    import moe_layer_align_amd as m
    from synth import CONFIGS
    c = CONFIGS[name]
    assert m.fused_path(M, c.E, c.H, c.I, c.k, c.dtype) == path


def test_fused_path_modes():
    import moe_layer_align_amd as m
    T = m.Tuning
    q = (1, 128, 2048, 768, 8, "fp8")  # one Qwen3-shaped token
    assert m.fused_path(*q, tuning=T(single_launch=1)) == "single_launch"
    assert m.fused_path(*q, tuning=T(routing_in_gate_up=-1)) == "decode_token_down"
    assert m.fused_path(*q, tuning=T(gemm1_ksplit=2)) == "decode_token_down"  # pinned gate/up launch shape
    assert m.fused_path(*q, tuning=T(gemm1_ksplit=2, routing_in_gate_up=1)) == "two_launches"
    assert m.fused_path(*q, tuning=T(down_per_token=-1)) == "decode"
    assert m.fused_path(*q, static_x_scale=True, static_h_scale=True, deterministic=True) == "decode"
    assert m.fused_path(*q, weight_scale_mode=3) == "decode"  # block-scaled
    assert m.fused_path(*q, weight_scale_mode=1, n_shared=1) == "two_launches"
    assert m.fused_path(*q, router_w=True) == "two_launches"
    assert m.fused_path(2, 16, 256, 256, 2, "fp8") == "decode_token_down"  # H/4 not whole fp8 k-steps
    assert m.fused_path(2, 16, 512, 256, 2, "fp8") == "two_launches"
    assert m.fused_path(2, 16, 256, 256, 2, "bf16") == "two_launches"
    mix = (1, 8, 4096, 14336, 2, "bf16")
    assert m.fused_path(*mix) == "decode_token_down"
    assert m.fused_path(*mix, tuning=T(routing_in_gate_up=1)) == "two_launches"
    for bad in (dict(tuning=T(single_launch=1, routing_in_gate_up=1)),
                dict(tuning=T(routing_in_gate_up=1, down_per_token=-1)),
                dict(router_w=True, tuning=T(single_launch=1))):
        with pytest.raises(m.MoEError) as e:
            m.fused_path(*q, **bad)
        assert e.value.code == 2, bad
    with pytest.raises(m.MoEError) as e:
        m.fused_path(4096, 128, 4096, 1536, 8, "fp8", tuning=T(routing_in_gate_up=1))
    assert e.value.code == 2


def test_fused_path_needs_no_outputs_and_rejects_null(lib):
    args = fused_args(y=None, workspace=None, workspace_bytes=0)
    p = ctypes.c_int32(-1)
    assert lib.moe_fused_path(ctypes.byref(args), ctypes.byref(p)) == 0 and p.value >= 1
    assert lib.moe_fused_path(ctypes.byref(args), None) == 1
    assert lib.moe_fused_path(None, ctypes.byref(p)) == 1
    assert lib.moe_fused_forward(ctypes.byref(args), None) == 1  # the call itself needs them


def test_router_logits_validation(lib):
    r = lib.moe_router_logits
    assert r(FAKE, FAKE, -1, 8, 256, FAKE, None) == 1
    assert r(None, FAKE, 4, 8, 256, FAKE, None) == 1
    assert r(FAKE, FAKE + 8, 4, 8, 256, FAKE, None) == 1   # 16-byte alignment
    assert r(FAKE, FAKE, 4, 8, 200, FAKE, None) == 2       # H not a multiple of 128
    assert r(FAKE, FAKE, 4, 1024, 256, FAKE, None) == 2    # E above 512
    assert r(None, None, 0, 8, 256, None, None) == 0       # M = 0


def test_fused_tuning_validation(lib):
    import moe_layer_align_amd as m
    for t in (m.Tuning(gemm1_ksplit=3), m.Tuning(token_tiles=5), m.Tuning(unroll=3), m.Tuning(gemm2_ksplit=17),
              m.Tuning(gemm2_wave_ksplit=3), m.Tuning(reverse_order=2), m.Tuning(single_launch=2),
              m.Tuning(single_launch=-2), m.Tuning(down_per_token=2), m.Tuning(down_per_token=-2),
              m.Tuning(routing_in_gate_up=2), m.Tuning(routing_in_gate_up=-2), m.Tuning(gemm1_feature_tiles=3),
              m.Tuning(gemm1_feature_tiles=-1), m.Tuning(gemm2_row_tiles=3), m.Tuning(gemm2_row_tiles=-1)):
        args = fused_args(tuning=ctypes.pointer(t))
        assert lib.moe_fused_forward(ctypes.byref(args), None) == 2


def test_fused_deterministic_refuses_order_changing_tunings(lib):
    import moe_layer_align_amd as m
    for dt, t in ((0, m.Tuning(gemm1_ksplit=2)), (0, m.Tuning(gemm2_ksplit=2)), (0, m.Tuning(gemm2_wave_ksplit=1)),
                  (0, m.Tuning(gemm1_stream_tiles=2)), (0, m.Tuning(gemm2_stream_tiles=2)),
                  (1, m.Tuning(gemm2_ksplit=1))):
        kw = dict(dtype=1, w13_scale=FAKE, w2_scale=FAKE, x_scale=FAKE, h_scale=FAKE) if dt else {}
        args = fused_args(deterministic=1, tuning=ctypes.pointer(t), **kw)
        assert lib.moe_fused_forward(ctypes.byref(args), None) == 1, (dt, t)


def test_fused_noalloc_validation(lib):
    # a workspace given, and a layer beyond the scratch array (fp32 h of
    # 32768 pairs x 1024 features alone is 128 MB): refused before any launch
    args = fused_args()
    assert lib.moe_fused_forward_noalloc(ctypes.byref(args), None) == 1
    args = fused_args(workspace=None, workspace_bytes=0, M=4096, E=16, top_k=8, H=1024, I=1024, dtype=1,
                      w13_scale=FAKE, w2_scale=FAKE)
    assert lib.moe_fused_forward_noalloc(ctypes.byref(args), None) == 2
    args = fused_args(workspace=None, workspace_bytes=0, top_k=9)
    assert lib.moe_fused_forward_noalloc(ctypes.byref(args), None) == 1


def test_fused_single_launch_required_where_it_does_not_fit(lib):
    import moe_layer_align_amd as m
    t = m.Tuning(single_launch=1)
    for kw in (dict(M=17), dict(M=40, top_k=2), dict(M=8, top_k=9, E=16), dict(E=300, top_k=2, M=2)):
        args = fused_args(tuning=ctypes.pointer(t), **kw)
        assert lib.moe_fused_forward(ctypes.byref(args), None) == 2, kw
    # never with router weights or in the deterministic mode
    args = fused_args(tuning=ctypes.pointer(t), logits=None, router_w=FAKE)
    assert lib.moe_fused_forward(ctypes.byref(args), None) == 2
    args = fused_args(tuning=ctypes.pointer(t), deterministic=1)
    assert lib.moe_fused_forward(ctypes.byref(args), None) == 2


def test_fused_down_per_token_required_where_it_does_not_fit(lib):
    # more than 64 pairs, the deterministic and the block-scaled modes, and a
    # dynamic fp8 h scale whose token rows (top_k * I bytes) exceed 64 KB
    import moe_layer_align_amd as m
    t = m.Tuning(down_per_token=1)
    fp8 = dict(dtype=1, w13_scale=FAKE, w2_scale=FAKE)
    for kw in (dict(M=40, top_k=2), dict(deterministic=1), dict(weight_scale_mode=3, **fp8),
               dict(top_k=8, I=16384, **fp8)):
        args = fused_args(tuning=ctypes.pointer(t), **kw)
        assert lib.moe_fused_forward(ctypes.byref(args), None) == 2, kw


def test_fused_routing_in_gate_up_required_where_it_does_not_fit(lib):
    # more than 16 tokens or 64 pairs, the per-expert down product, E above
    # 256, fp8 x above 16384 elements, a gate/up K that four waves cannot split
    # into whole MFMA k-steps
    import moe_layer_align_amd as m
    fp8 = dict(dtype=1, w13_scale=FAKE, w2_scale=FAKE)
    for kw in (dict(M=17, top_k=2), dict(M=9, top_k=8), dict(E=300, top_k=2),
               dict(M=2, H=16384, **fp8), dict(M=2, H=256, **fp8), dict(M=2, H=384, **fp8)):
        t = m.Tuning(routing_in_gate_up=1)
        args = fused_args(tuning=ctypes.pointer(t), **kw)
        assert lib.moe_fused_forward(ctypes.byref(args), None) == 2, kw
    t = m.Tuning(routing_in_gate_up=1, down_per_token=-1)
    args = fused_args(tuning=ctypes.pointer(t))
    assert lib.moe_fused_forward(ctypes.byref(args), None) == 2


def test_fused_m0_is_noop(lib):
    args = fused_args(M=0, x=None, logits=None, y=None, workspace=None, workspace_bytes=0)
    assert lib.moe_fused_forward(ctypes.byref(args), None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    import moe_layer_align_amd as m
    with pytest.raises(ValueError):
        m.route_topk(torch.zeros(2, 8), 2)
