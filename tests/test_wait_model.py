"""The vector-memory wait model the scan kernels rely on, checked on the CPU
against gfx950 code that hipcc generates.

The prefix scan stores a weight slot between issuing the next k-tile's
direct-to-LDS loads and that k-tile's barrier, and then waits with
vmcnt(N) for N >= 1, leaving the last N vector-memory operations (the slot
stores) in flight.  That is correct only if one counter covers loads and
stores and they retire in issue order, so that vmcnt(N) implies that
everything issued before the last N operations has completed.

1. The compiler's own wait insertion for gfx950 assumes exactly that: for a
   direct-to-LDS load, three stores and a workgroup barrier before the LDS is
   read, it emits vmcnt(3), not vmcnt(0); for a global load followed by three
   stores and a use of the loaded value, likewise vmcnt(3).
2. In the compiled scan kernels, every vmcnt(N > 0) that guards a barrier has
   at least N stores, and no load, among the last N vector-memory
   instructions before it (in program text: the store block sits between the
   loads and the wait), so the loads it must cover are not among those left
   in flight.

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


def test_scan_kernels_leave_only_stores_in_flight(tmp_path):
    src = os.path.join(hipbuild.CSRC, "kernels.hip")
    funcs = _functions(_compile(src, str(tmp_path / "kernels.s")))
    checked = 0
    # the scan launches, and every instantiation of the scan-only kernel
    # (tile shapes, slot layouts, data types)
    prefix = [n for n in funcs if "prefix_update_kernel" in n]
    assert len(prefix) >= 4, prefix
    for key in SCAN_KERNELS + prefix:
        body = _body(funcs, key)
        for i, line in enumerate(body):
            m = WAIT_VM.match(line)
            if not m or int(m.group(1)) == 0:
                continue
            n = int(m.group(1))
            # does this wait guard a barrier (no vector-memory op in between)?
            guards = False
            for nxt in body[i + 1:]:
                if VMEM.match(nxt):
                    break
                if "s_barrier" in nxt:
                    guards = True
                    break
            if not guards:
                continue
            # the last n vector-memory instructions before it must all be stores
            prev = [l for l in body[:i] if VMEM.match(l)][-n:]
            assert len(prev) == n and all(VMEM.match(l).group(2) == "store" for l in prev), (
                key, i, n, [l.strip() for l in prev if VMEM.match(l).group(2) != "store"][:4])
            checked += 1
    # every scan kernel (two data types, three launch forms, the scan-only
    # instantiations) has its store wait
    assert checked >= len(SCAN_KERNELS) + len(prefix), checked
