"""The vector-memory waits of the scan kernels, checked on the CPU against
gfx950 code that hipcc generates.

The prefix scan stores a weight slot at the start of each chunk's first
k-tile, before that k-tile's MFMAs, and ends every k-tile with vmcnt(0) and
a barrier: no vector-memory operation is in flight when another wave reads
the LDS stage the direct-to-LDS loads filled.  (An earlier form left the slot
stores in flight with vmcnt(N), which is correct only if one counter retires
loads and stores in issue order; the code no longer relies on that.)

1. The counter model of the compiler's own wait insertion for gfx950, kept as
   the record of what vmcnt(N) means there: for a direct-to-LDS load, three
   stores and a workgroup barrier before the LDS is read, it emits vmcnt(3),
   not vmcnt(0); for a global load followed by three stores and a use of the
   loaded value, likewise vmcnt(3).
2. In the compiled scan kernels, no wait that guards a barrier leaves a load
   in flight on any path (a dataflow pass over the basic blocks).

No GPU is needed: both checks read the AMD assembly of code built here.
"""
import os
import re
import shutil
import subprocess

import pytest

from chunk_wise_weight_chunked_amd import build as hipbuild

HIPCC = next((c for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")) if c and os.path.exists(c)),
             None)
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")

DEVICE_FLAGS = [f"--offload-arch={hipbuild.ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-S",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

PROBE = r"""
#include <hip/hip_runtime.h>
__global__ void dma_stores_barrier(const float* a, float* o) {
  __shared__ float s[256];
  auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, 1 << 20, 0x00020000);
  auto ro = __builtin_amdgcn_make_buffer_rsrc((void*)o, (short)0, 1 << 20, 0x00020000);
  const int i = threadIdx.x;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)s, 4,
                                           i * 4, 0, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(1u, ro, i * 4, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(2u, ro, i * 4 + 256, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(3u, ro, i * 4 + 512, 0, 0);
  __syncthreads();
  const float v = s[i ^ 1];
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ro, i * 4 + 768, 0, 0);
}
__global__ void load_stores_use(const float* __restrict__ a, float* __restrict__ o1,
                                float* __restrict__ o2, float* __restrict__ o3) {
  const int i = threadIdx.x;
  const float x = a[i];
  o1[i] = 1.0f;
  o2[i] = 2.0f;
  o3[i] = 3.0f;
  o1[i + 64] = x * 2.0f;
}
"""

VMEM = re.compile(r"^\s*(buffer|global|flat|scratch)_(load|store|atomic)\w*")
WAIT_VM = re.compile(r"^\s*s_waitcnt\s.*vmcnt\((\d+)\)")


def _compile(src_path, out_path):
    r = subprocess.run([HIPCC, *DEVICE_FLAGS, src_path, "-o", out_path], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out_path) as fh:
        return fh.read()


def _functions(asm):
    """{mangled name: [instruction lines]} of the kernels in an assembly file."""
    funcs, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is not None:
            if line.startswith("\t.end_amdhsa_kernel") or re.match(r"^\.Lfunc_end", line):
                cur = None
                continue
            s = line.split(";")[0].rstrip()
            if s.strip():
                funcs[cur].append(s)
    return funcs


def _body(funcs, key):
    names = [n for n in funcs if key in n]
    assert len(names) == 1, (key, names)
    return funcs[names[0]]


def test_compiler_counts_loads_and_stores_in_issue_order(tmp_path):
    src = tmp_path / "probe.hip"
    src.write_text(PROBE)
    funcs = _functions(_compile(str(src), str(tmp_path / "probe.s")))

    body = _body(funcs, "dma_stores_barrier")
    i_dma = next(i for i, l in enumerate(body) if re.search(r"buffer_load_dword.*\blds\b", l))
    i_bar = next(i for i, l in enumerate(body) if "s_barrier" in l)
    i_read = next(i for i, l in enumerate(body) if "ds_read" in l)
    assert i_dma < i_bar < i_read
    stores = [l for l in body[i_dma:i_bar] if re.search(r"buffer_store", l)]
    waits = [int(m.group(1)) for l in body[i_dma:i_read] for m in [WAIT_VM.match(l)] if m]
    assert len(stores) == 3
    # the compiler covers the direct-to-LDS load with a wait that leaves the
    # three later stores in flight
    assert waits == [3], waits

    body = _body(funcs, "load_stores_use")
    waits = [int(m.group(1)) for l in body for m in [WAIT_VM.match(l)] if m]
    assert 3 in waits and 0 not in waits, waits


SCAN_KERNELS = ["scan_apply_kernelIt", "scan_apply_kernelIf", "scan_target_kernelIt",
                "scan_target_kernelIf", "dual_scan_kernelIt", "dual_scan_kernelIf"]

LABEL = re.compile(r"^(\.LBB\w+):")
BRANCH = re.compile(r"^\s*s_(branch|cbranch\w*)\s+(\.LBB\w+)")
END = re.compile(r"^\s*s_(endpgm|setpc_b64|trap)\b")
VMEM_ANY = re.compile(r"^\s*(buffer|global|flat|scratch)_(\w+)")


def _blocks(body):
    """Basic blocks of a kernel body: [line indices], successor block indices."""
    blocks, names = [[]], {}
    for at, line in enumerate(body):
        m = LABEL.match(line)
        if m:
            if blocks[-1]:
                blocks.append([])
            names[m.group(1)] = len(blocks) - 1
            continue
        blocks[-1].append(at)
        if BRANCH.match(line) or END.match(line):
            blocks.append([])
    succ = []
    for i, idx in enumerate(blocks):
        last = body[idx[-1]] if idx else ""
        m, out = BRANCH.match(last), []
        if m:
            out.append(names[m.group(2)])
        if not END.match(last) and not (m and m.group(1) == "branch") and i + 1 < len(blocks):
            out.append(i + 1)
        succ.append(out)
    return blocks, succ


def _vmem_kind(line):
    m = VMEM_ANY.match(line)
    if not m:
        return None
    op = m.group(2)
    return "L" if op.startswith(("load", "atomic")) else "S"


def _barrier_waits(body):
    """Every vmcnt(N > 0) wait that guards a barrier (no vector-memory
    instruction between it and the s_barrier), with the vector-memory
    operations that may still be in flight after it on some path: a dataflow
    pass over the basic blocks in which each state is the sequence of
    operations issued since the last full drain, and vmcnt(N) keeps the last
    N of them (one counter, retired in issue order)."""
    blocks, succ = _blocks(body)

    def guards(at):  # the text after a wait, through fall-through labels
        for nxt in body[at + 1:]:
            if _vmem_kind(nxt) or BRANCH.match(nxt) or END.match(nxt):
                return False
            if "s_barrier" in nxt:
                return True
        return False

    # each block as events: ("V", kind, run length) or ("W", n, line, guards)
    events = []
    for idx in blocks:
        ev = []
        for at in idx:
            kind = _vmem_kind(body[at])
            if kind:
                if ev and ev[-1][0] == "V" and ev[-1][1] == kind:
                    ev[-1] = ("V", kind, ev[-1][2] + 1)
                else:
                    ev.append(("V", kind, 1))
                continue
            m = WAIT_VM.match(body[at])
            if m:
                n = int(m.group(1))
                ev.append(("W", n, at, bool(n) and guards(at)))
        events.append(ev)

    found = {}
    seen = set()
    work = [(0, ())]
    while work:
        i, st = work.pop()
        if (i, st) in seen:
            continue
        seen.add((i, st))
        for e in events[i]:
            if e[0] == "V":
                st = (st + (e[1],) * e[2])[-64:]
            else:
                n = e[1]
                st = st[-n:] if n else ()
                if e[3]:
                    found.setdefault(e[2], set()).add(st)
        for j in succ[i]:
            if (j, st) not in seen:
                work.append((j, st))
    return found


def test_scan_kernels_leave_no_load_in_flight(tmp_path):
    src = os.path.join(hipbuild.CSRC, "kernels.hip")
    funcs = _functions(_compile(src, str(tmp_path / "kernels.s")))
    # the scan launches, and every instantiation of the scan-only kernel
    # (tile shapes, slot layouts, data types)
    prefix = [n for n in funcs if "prefix_update_kernel" in n]
    assert len(prefix) >= 4, prefix
    names = sorted({n for key in SCAN_KERNELS for n in funcs if key in n}) + prefix
    assert len(names) >= len(SCAN_KERNELS) + len(prefix), names
    for key in names:
        body = funcs[key]
        assert any("s_barrier" in l for l in body), key  # the k-loop's barrier is there
        for at, states in _barrier_waits(body).items():
            n = int(WAIT_VM.match(body[at]).group(1))
            # on every path of the control flow, what the wait leaves in
            # flight is stores only; or, where the pass cannot tell two tests
            # of one condition apart, the n vector-memory instructions right
            # before it in the text are all stores
            if any("L" in st for st in states):
                prev = [l for l in body[:at] if VMEM.match(l)][-n:]
                assert len(prev) == n and all(VMEM.match(l).group(2) == "store" for l in prev), (
                    key, at, n, [l.strip() for l in prev if VMEM.match(l).group(2) != "store"][:4])


def test_dataflow_sees_a_load_left_in_flight():
    """The check itself: a wait that leaves a direct-to-LDS load in flight
    across a barrier, on one of two paths, is found."""
    body = ["\tbuffer_store_dword v1, v2, s[0:3], 0 offen",
            "\ts_cbranch_scc1 .LBB0_2",
            "\tbuffer_load_dword v3, s[4:7], 0 offen lds",
            ".LBB0_2:",
            "\ts_waitcnt vmcnt(1)",
            "\ts_barrier",
            "\ts_endpgm"]
    waits = _barrier_waits(body)
    states = set().union(*waits.values())
    assert ("S",) in states and ("L",) in states
    # with the load waited for (vmcnt(0)) nothing is left
    body[4] = "\ts_waitcnt vmcnt(0)"
    assert _barrier_waits(body) == {}
