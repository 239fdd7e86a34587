"""Checks on the gfx950 assembly of every unit of both libraries (CPU only:
hipcc -S, no GPU): the spacing between the fp8 matrix instructions and the
first reads of their results, and that no kernel spills to scratch memory.

The hardware does not hold back an instruction that reads an MFMA's result
registers before the MFMA has written them: the compiler must put enough
independent instructions or s_nop wait states in between.  On gfx950 it
keeps at least 12 of them after a 16x16x128 scaled fp8 MFMA and at least 20
after a 32x32x64 one when the read follows in the same basic block; but a
probe whose store block was reached both from a 16x16x128 MFMA and from a
16x16x32 one got only 8 (the shorter instruction's wait) and stored a stale
accumulator element, which the GPU probe tests would catch as wrong sums.
This test follows every control-flow path from every scaled MFMA to the
first instruction that reads its destination registers and fails if any
path is shorter than those spacings, so that such a miss cannot reach a
product kernel unnoticed.

Scratch: every kernel keeps its state in registers and LDS (private segment
size 0).  A build of the prefill product whose registers spilled to scratch
faulted the GPU on its first run (its code was never kept, so the fault was
not traced); a kernel that spills is therefore not run before its scratch
accesses have been checked.
"""
import collections
import heapq
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_layer_align_amd", "csrc")
MIN_WAIT = {"16x16x128": 12, "32x32x64": 20}

_REG = re.compile(r"\b([av])(\d+)\b|\b([av])\[(\d+):(\d+)\]")
_WRITES_FIRST = ("global_store", "buffer_store", "flat_store", "scratch_store", "ds_write", "ds_store",
                 "global_atomic", "buffer_atomic", "ds_add", "ds_max", "ds_min")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def _operands(ins):
    parts = ins.split(None, 1)
    return parts[1].split(",") if len(parts) > 1 else []


def _reads(ins):
    """Registers an instruction reads: every operand but the first, which is
    the destination except for stores and atomics."""
    op = ins.split()[0]
    ops = _operands(ins)
    return set().union(*[_regs(o) for k, o in enumerate(ops) if k > 0 or op.startswith(_WRITES_FIRST)]) if ops \
        else set()


def _wait_states(ins):
    f = ins.split()
    return int(f[1]) + 1 if f[0] == "s_nop" else 1


def parse_functions(asm_text):
    """Kernels of a .s file as ordered basic blocks of instruction lines."""
    funcs, cur = [], None
    for raw in asm_text.split("\n"):
        t = raw.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":"):
            label = t[:-1]
            if not label.startswith((".", "$")):
                cur = {"name": label, "order": [label], "blocks": {label: []}}
                funcs.append(cur)
            elif cur is not None and label.startswith(".LBB"):
                cur["order"].append(label)
                cur["blocks"][label] = []
            continue
        if cur is not None and not t.startswith("."):
            cur["blocks"][cur["order"][-1]].append(t)
    return funcs


def _successors(func, bi):
    ins = func["blocks"][func["order"][bi]]
    last = ins[-1] if ins else ""
    op = last.split()[0] if last else ""
    if op == "s_branch":
        return [last.split()[1]]
    if op in ("s_endpgm", "s_setpc_b64"):
        return []
    out = [last.split()[1]] if op.startswith("s_cbranch") else []
    if bi + 1 < len(func["order"]):
        out.append(func["order"][bi + 1])
    return out


def min_read_distances(func):
    """(kind, fewest wait states on any path to a read, block) for every
    scaled MFMA of the function."""
    index = {label: i for i, label in enumerate(func["order"])}
    out = []
    for bi, label in enumerate(func["order"]):
        for ii, ins in enumerate(func["blocks"][label]):
            if not ins.startswith("v_mfma_scale"):
                continue
            kind = "16x16x128" if "16x16x128" in ins else "32x32x64"
            dst = _regs(_operands(ins)[0])
            best, seen, heap = 99, {}, [(0, bi, ii + 1)]
            while heap:
                d, b, p = heapq.heappop(heap)
                if d >= best or seen.get((b, p), 99) <= d:
                    continue
                seen[(b, p)] = d
                block = func["blocks"][func["order"][b]]
                ended = False
                while p < len(block):
                    t = block[p]
                    if t.startswith("v_mfma"):
                        if _regs(_operands(t)[0]) & dst:  # the accumulator chain goes on in the matrix unit
                            ended = True
                            break
                    elif _reads(t) & dst:
                        best = min(best, d)
                        ended = True
                        break
                    d += _wait_states(t)
                    p += 1
                    if d >= best or d > 40:
                        ended = True
                        break
                if not ended:
                    for s in _successors(func, b):
                        if s in index:
                            heapq.heappush(heap, (d, index[s], 0))
            out.append((kind, best, label))
    return out


def test_scanner_sees_a_short_cross_block_read():
    # a read in a block that one predecessor enters right after a 16x16x128
    # MFMA, with a wait long enough only for the other predecessor
    asm = "\n".join([
        "k:", "s_cbranch_scc1 .LBB0_2",
        "v_mfma_f32_16x16x32_fp8_fp8 a[0:3], v[0:1], v[2:3], a[0:3]", "s_branch .LBB0_3",
        ".LBB0_2:", "v_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[8:15], v[16:23], a[0:3], v1, v2",
        ".LBB0_3:", "s_nop 6", "v_accvgpr_read_b32 v5, a3", "global_store_dword v1, v5, s[2:3]", "s_endpgm"])
    (kind, dist, _), = min_read_distances(parse_functions(asm)[0])
    assert kind == "16x16x128" and dist == 7
    # and a chained MFMA followed by a long enough wait is not a read
    asm2 = "\n".join(["k:", "v_mfma_scale_f32_32x32x64_f8f6f4 a[0:15], v[0:7], v[8:15], a[0:15], v1, v2",
                      "s_nop 7", "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v0, a15", "s_endpgm"])
    assert min_read_distances(parse_functions(asm2)[0]) == [("32x32x64", 20, "k")]


def _units():
    import moe_layer_align_amd.build as b
    return list(b.UNITS) + list(b.PROBE_UNITS)


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not (os.path.exists(hipcc) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    import moe_layer_align_amd.build as b
    out_dir = tmp_path_factory.mktemp("asm")

    def gen(unit):
        dst = os.path.join(out_dir, unit.replace(".hip", ".s"))
        cmd = [hipcc, *b.FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
               os.path.join(CSRC, unit), "-o", dst]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return unit, open(dst).read()

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return dict(ex.map(gen, _units()))


def test_every_scaled_mfma_read_is_spaced(assembly):
    short, counts = [], collections.Counter()
    for unit, text in assembly.items():
        for func in parse_functions(text):
            for kind, dist, label in min_read_distances(func):
                counts[kind] += 1
                if dist < MIN_WAIT[kind]:
                    short.append((unit, func["name"][:80], label, kind, dist))
    assert counts["16x16x128"] > 0 and counts["32x32x64"] > 0  # the scan saw the fp8 products
    assert not short, short[:10]


def test_no_kernel_uses_scratch(assembly):
    spill = []
    for unit, text in assembly.items():
        names = re.findall(r"^\s*\.name:\s+(\S+)", text, flags=re.M)
        sizes = [int(v) for v in re.findall(r"^\s*\.private_segment_fixed_size:\s+(\d+)", text, flags=re.M)]
        assert len(sizes) >= 1 and len(names) >= len(sizes), unit
        spill += [(unit, n) for n, v in zip(names, sizes) if v != 0]
    assert not spill, spill[:10]
