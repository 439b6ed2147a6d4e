"""Host-side checks of the index arithmetic the kernels share (CPU only).

The launch-order and packed-segment helpers of csrc/common.hpp are
__host__ __device__ or plain device code; the host versions are compiled with
hipcc into a small program here and checked exhaustively over small shapes:

* causal_order maps the logical work-groups of a causal launch one to one
  onto (tile rank, head slot), tile rank major, and pins every K/V stream to
  one XCD (work-group p runs on XCD p % 8) when the streams split evenly;
* find_segment_tile (a host copy of its body, checked against the source)
  finds, for
  every logical tile of a packed batch, the segment and rank a serial walk
  over the segments assigns, and every real tile of every segment once.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PROGRAM = r'''
#include "memory_efficient_exact_tiled_amd/csrc/common.hpp"
#include <cstdio>
#include <cstdlib>
#include <vector>
using namespace mea;

// Host copy of find_segment_tile's arithmetic (the test checks that its body
// is the device function's, token for token).
static int host_find(const int32_t* st, int B, int total, int bt, int t, int& rank, int& a0, int& a1, int& ntile) {
  auto base = [&](int s) { return min(max(st[s], 0), total) / bt + s; };
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base(mid) <= t) lo = mid; else hi = mid - 1;
  }
  const int b0 = base(lo);
  a0 = min(max(st[lo], 0), total);
  a1 = min(max(st[lo + 1], a0), total);
  ntile = (a1 - a0 + bt - 1) / bt;
  rank = t - b0;
  return (rank >= 0 && rank < ntile) ? lo : B;
}

int main() {
  long bad = 0, cases = 0;
  for (int nstreams : {1, 3, 8, 16, 24, 64, 128})
    for (int group : {1, 2, 4, 8})
      for (int ntiles : {1, 2, 7, 32}) {
        const int nbh = nstreams * group, total = nbh * ntiles;
        std::vector<int> seen(total, 0);
        for (int pid = 0; pid < total; ++pid) {
          int t, bh;
          causal_order(pid, nbh, group, t, bh);
          if (t < 0 || t >= ntiles || bh < 0 || bh >= nbh) { bad++; continue; }
          if (t != pid / nbh) bad++;
          seen[t * nbh + bh]++;
          if (nstreams % 8 == 0 && (bh / group) % 8 != pid % 8) bad++;
        }
        for (int i = 0; i < total; ++i) bad += seen[i] != 1;
        cases++;
      }
  srand(7);
  for (int trial = 0; trial < 400; ++trial) {
    const int B = 1 + rand() % 300, bt = (trial & 1) ? 128 : 256;
    const int maxlen = (trial % 3 == 0) ? 3 : (trial % 3 == 1) ? 70 : 700;
    std::vector<int32_t> st(B + 1, 0);
    for (int s = 0; s < B; ++s) st[s + 1] = st[s] + (rand() % (maxlen + 1));
    const int M = st[B];
    const int tiles = (M + bt - 1) / bt + B;      // the host's grid bound
    int expect_total = 0;
    for (int s = 0; s < B; ++s) expect_total += (st[s + 1] - st[s] + bt - 1) / bt;
    int found = 0;
    for (int t = 0; t < tiles; ++t) {
      int rank, a0, a1, nt;
      const int s = host_find(st.data(), B, M, bt, t, rank, a0, a1, nt);
      if (s == B) continue;
      if (a0 != st[s] || a1 != st[s + 1] || rank < 0 || rank >= nt) bad++;
      found++;
    }
    bad += found != expect_total;
    // every (segment, rank) appears once
    for (int s = 0; s < B; ++s) {
      const int nt = (st[s + 1] - st[s] + bt - 1) / bt;
      for (int r = 0; r < nt; ++r) {
        const int t = st[s] / bt + s + r;
        int rank, a0, a1, n2;
        if (t >= tiles || host_find(st.data(), B, M, bt, t, rank, a0, a1, n2) != s || rank != r) bad++;
      }
    }
    cases++;
  }
  printf("cases %ld bad %ld\n", cases, bad);
  return bad != 0;
}
'''


def test_launch_order_and_segment_search(tmp_path):
    src = open(os.path.join(ROOT, "memory_efficient_exact_tiled_amd", "csrc", "common.hpp")).read()
    # The host copy in PROGRAM must be the device function's own arithmetic.
    body = src[src.index("int find_segment_tile("):]
    body = body[body.index("{"):body.index("\n}\n") + 2]
    prog = PROGRAM
    host = prog[prog.index("static int host_find("):]
    host = host[host.index("{"):host.index("\n}\n") + 2]
    assert " ".join(body.split()) == " ".join(host.split()), "host copy of find_segment_tile is stale"
    (tmp_path / "check.hip").write_text(prog)
    exe = tmp_path / "check"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", ROOT, "-I",
                        os.path.join(ROOT, "include"), str(tmp_path / "check.hip"), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-3000:])
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "bad 0" in out.stdout
