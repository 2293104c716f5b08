"""The split-K rule of the weight-streaming GEMMs, checked on the CPU.

Every workgroup of a streaming launch and of its reduction launch evaluates
`stream_splits` (csrc/kernels.h) to find how many workgroups share one work
item's K steps, and the workspace holds the partial tiles of every split.  A
rule that returned more units than the workspace holds, a split without K
steps, or a split of a launch whose reduction grid is too small for it would
write or read outside its buffers on the GPU.  The rule is host+device code,
so it is compiled here for the host and swept over every item count a launch
can have.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_routed_softmax_amd", "csrc")

PROGRAM = r"""
#include "common.h"
#include "kernels.h"
#include <cstdio>
using namespace moe;
int main() {
  long checked = 0, bad = 0;
  const int slots_list[] = {256, 512, 768};   // resident workgroups of the streaming builds
  for (int slots : slots_list)
    for (int KT = 1; KT <= 1024; ++KT)
      for (int items = 0; items <= 2 * kStreamTarget + 8; ++items) {
        const int S = stream_splits(items, KT, slots);
        ++checked;
        bool ok = S >= 1 && S <= kStreamMaxSplit;
        if (S > 1) {
          // only launches below the slot count and the target split, so the
          // reduction grid min(item capacity, kStreamTarget) covers them
          ok = ok && items < slots && items < kStreamTarget;
          // units within the stated bound and the workspace's unit cap
          ok = ok && (long)items * S < kStreamTarget + 2L * items && (long)items * S <= 3L * kStreamTarget;
          // every split gets at least kStreamMinSteps K steps
          for (int sp = 0; sp < S; ++sp) {
            const int k0 = (int)((long)KT * sp / S), k1 = (int)((long)KT * (sp + 1) / S);
            ok = ok && k1 - k0 >= kStreamMinSteps;
          }
        }
        if (!ok) {
          if (bad < 5) printf("bad: slots=%d KT=%d items=%d S=%d\n", slots, KT, items, S);
          ++bad;
        }
      }
  printf("checked %ld bad %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_stream_split_rule(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    src = tmp_path / "split_rule.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "split_rule"
    subprocess.run([hipcc, "-O2", "-std=c++17", "--offload-arch=gfx950", "-I" + CSRC,
                    "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "bad 0" in r.stdout
