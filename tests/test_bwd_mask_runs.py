"""The dK/dV kernels' split of query blocks into masked and mask-free runs (CPU).

The D = 64 dK/dV kernel runs the query blocks that need no entry mask through
a body without it (fa_mask_runs.h).  A block taken as mask-free
that does need the mask would give wrong gradients; a block taken as masked
that needs none only costs time.  This test compiles the header with the
host compiler and walks the kernels' loop over many tile shapes, checking
that every block is visited once, in order, and that the body chosen is
mask-free exactly when the kernels' per-block condition says so: no row past
the sequence end and, causal (bottom-right aligned), no row before the
diagonal of the wave's last key.
"""
import os
import shutil
import subprocess

import pytest

from exact_attention_forward_04_amd import build as fa_build

DRIVER = r"""
#define FA_HD
#include "fa_mask_runs.h"
#include <cstdio>
int main() {
  const int BN = 64;
  long long blocks = 0, free_blocks = 0;
  for (int causal = 0; causal < 2; ++causal)
  for (int L = 1; L <= 520; L += (L < 140 ? 1 : 37))
  for (int dk = -140; dk <= 140; dk += (dk >= -70 && dk < 70 ? 1 : 35)) {
    const int Lk = L + dk;
    if (Lk < 1) continue;
    const int koff = Lk - L;
    for (int G = 1; G <= 3; G += 2)
    for (int n0t = 0; n0t < Lk; n0t += 128)
    for (int wave = 0; wave < 4; ++wave) {
      const int key0 = n0t + 32 * wave;
      const int nqb = (L + BN - 1) / BN;
      const int qb0 = causal ? (n0t - koff > 0 ? n0t - koff : 0) / BN : 0;
      const int per = nqb > qb0 ? nqb - qb0 : 0;
      const int nblocks = G * per;
      if (nblocks == 0) continue;
      const fa::MaskRuns runs = fa::mask_runs(causal, L, qb0, per, key0, koff, BN);
      int expect = 0;
      for (int t = 0; t < nblocks;) {
        const int e = runs.run_end(t);
        const bool run = e > t;
        if (e < t || e > nblocks) { printf("bad run end %d at %d\n", e, t); return 1; }
        const int stop = run ? e : t + 1;
        for (; t < stop; ++t) {
          if (t != expect++) { printf("block %d out of order\n", t); return 1; }
          const int m0 = (qb0 + t % per) * BN;
          const bool need = (m0 + BN > L) || (causal && m0 < key0 - koff + 31);
          if (need == run) {
            printf("causal=%d L=%d Lk=%d G=%d n0t=%d wave=%d t=%d: need_mask=%d, body %s\n",
                   causal, L, Lk, G, n0t, wave, t, (int)need, run ? "mask-free" : "masked");
            return 1;
          }
          ++blocks;
          free_blocks += !need;
        }
      }
      if (expect != nblocks) { printf("visited %d of %d\n", expect, nblocks); return 1; }
    }
  }
  printf("%lld %lld\n", blocks, free_blocks);
  return 0;
}
"""


def test_mask_runs_match_the_kernels_mask_condition(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    src = tmp_path / "mask_runs.cpp"
    src.write_text(DRIVER)
    exe = str(tmp_path / "mask_runs")
    subprocess.run([cxx, "-O2", "-std=c++17", "-I" + fa_build.CSRC, str(src), "-o", exe],
                   check=True, capture_output=True, timeout=120)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    blocks, free_blocks = map(int, r.stdout.split())
    # both bodies are exercised, and most blocks of long tiles are mask-free
    assert blocks > 100000 and 0 < free_blocks < blocks
