// fa_mask_runs.h -- which query blocks of a dK/dV key tile need the entry
// mask (host and device).
//
// The dK/dV kernel visits, for each query head of a K/V group, the 64-row
// query blocks i = 0 .. per-1 (rows m0 = (qb0 + i) * bn ..), against one
// wave's 32 keys key0 .. key0+31.  A block needs the entry mask when one of
// its rows lies past the sequence end (m0 + bn > L) or, under the causal
// mask (bottom-right aligned: row r may use key j when j <= r + koff), when
// it starts before the diagonal of the wave's last key (m0 < key0 + 31 -
// koff).  Rows only grow with i, so the blocks i1 <= i < i2 of each head
// need no mask: at D = 64 the kernel runs those through a body without it.
#pragma once

#ifndef FA_HD
#define FA_HD __host__ __device__
#endif

namespace fa {

struct MaskRuns {
  int i1, i2, per;
  // The end of the run of mask-free blocks that starts at block t (block
  // index over all heads of the group, t = head * per + i); t itself when
  // block t needs the mask.  per > 0.
  FA_HD int run_end(int t) const {
    const int i = t % per;
    return (i >= i1 && i < i2) ? t - i + i2 : t;
  }
};

FA_HD inline int mask_runs_clamp(int v, int per) { return v < 0 ? 0 : (v > per ? per : v); }

FA_HD inline MaskRuns mask_runs(bool causal, int L, int qb0, int per, int key0, int koff,
                                int bn) {
  MaskRuns r;
  r.per = per;
  // m0 + bn <= L  <=>  qb0 + i + 1 <= floor(L / bn)
  r.i2 = mask_runs_clamp(L / bn - qb0, per);
  // m0 >= x  <=>  qb0 + i >= ceil(x / bn)  (every m0 >= 0 when x <= 0)
  const int x = key0 + 31 - koff;
  r.i1 = (causal && x > 0) ? mask_runs_clamp((x + bn - 1) / bn - qb0, per) : 0;
  return r;
}

}  // namespace fa
