// fa_fwd.hip -- exact attention forward for MI355X (gfx950): kernels and C ABI.
//
// O = softmax(scale * Q K^T + causal mask) V and LSE = ln sum exp, computed per
// tile of query rows with an online softmax so the score matrix stays on
// chip (FlashAttention-4 paper, sections 1 and 3.1; the engineering blog's
// "life of a tile").  The gfx950 design:
//
//   workgroup  NW wavefronts of 64 lanes; wave w owns 32 query rows, so a
//              tile is BM = 32*NW rows of one (sequence, head).
//   Q          loaded once per tile into VGPRs as the B operand of
//              v_mfma_f32_32x32x16_bf16 (lane l: row l%32, 8 consecutive d).
//   K, V       streamed in blocks of BN = 64 keys through LDS with
//              global_load_lds_dwordx4 (16 bytes per lane straight into LDS),
//              copied two blocks ahead of their use through a ring of four
//              buffers (D = 256: double-buffered).  Rows are stored with a
//              16-byte-chunk XOR swizzle so the MFMA operand reads do not
//              collide on LDS banks.
//   S^T = K Q^T  on MFMA (keys on the M side, query rows on N): every lane
//              then holds 16 keys of ONE query row per 32-key sub-block, so a
//              row maximum is an in-lane max plus one v_permlane32_swap with
//              the other half-wave, and the row statistics are per lane.
//   softmax    reference row max m_ref in log2 units.  p = exp2(c*s - m_ref)
//              with c = scale*log2(e) is computed against the stale m_ref,
//              by v_exp_f32 or, for a fixed share of column slots, by the
//              Cody-Waite degree-3 polynomial (paper section 3.1.3).  Only
//              when some lane's share of the block's row sum exceeds 2^tau
//              (or a row has no reference yet) does the whole wave take the
//              block maximum, move m_ref and rescale O and the row sums
//              (paper section 3.1.4: rescale only when the growth of the
//              maximum threatens the range); otherwise the final
//              normalisation absorbs the stale reference.  The row sum l = sum p is kept in fp32 from
//              the unrounded p (paper section 3.1.2 sums after the exp);
//              P is rounded to bf16 only as the operand of the PV product.
//   O^T += V^T P^T  on MFMA: the S accumulator registers, rounded to bf16,
//              are already the B operand (the contraction index runs over
//              the keys in the order the S layout holds them); V^T comes from
//              LDS with ds_read_b64_tr_b16, which transposes 16-bit elements
//              across each 16-lane group.
//   epilogue   O / l -> bf16, LSE = ln2 * (m_ref + log2 l).
//
// Scheduling: a persistent grid walks tiles in longest-processing-time-first
// order (fa_sched.h), or one workgroup per tile in natural order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>
#include <algorithm>
#include <array>

#include "fa.h"
#include "exp2_poly.h"
#include "fa_sched.h"
#include "fa_host.h"
#include "fa_tile.h"

namespace {

constexpr int kMatrixPrio = 2;    // wave priority (s_setprio) of a ping-pong matrix phase
constexpr float kMaxTau = 64.0f;  // largest accepted rescale threshold (log2 units)

// ---------------------------------------------------------------------------
// Polynomial exp2 (Cody-Waite split + degree-3 Horner, three FMAs).
// x is clamped to -127 so that n >= -127; with C0 == 1 a clamped input gives
// p = 1 and an exponent field of 0: exactly +0.  n = floor(x) is exact and
// f = x - n lies in [0, 1]: it rounds to exactly 1 only for tiny negative x,
// where p(1) ~ 2 with the same relative error.  (v_fract_f32 is not used:
// it clamps f below 1, after which x - f is no longer an integer.)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp2_poly(float x) {
  x = fmaxf(x, -127.0f);
  const float n = floorf(x);
  const float f = x - n;
  float p = __builtin_fmaf(FA_EXP2_C3, f, FA_EXP2_C2);
  p = __builtin_fmaf(p, f, FA_EXP2_C1);
  p = __builtin_fmaf(p, f, FA_EXP2_C0);
  const int bits = __float_as_int(p) + (static_cast<int>(n) << 23);
  return __int_as_float(bits);
}

template <int D>
struct Cfg {
  // D <= 192: eight waves (two per SIMD) in one workgroup per CU, run as two
  // halves that alternate matrix-product and softmax phases (run_tile).
  // D = 256 needs the whole register file (O alone is 128 VGPRs per lane):
  // four waves, one per SIMD, in the plain per-block sequence.
  static constexpr int DV = head_dim_v<D>();
  static constexpr int NW = (D == 256) ? 4 : 8;  // waves per workgroup
  static constexpr int OCC = 1;                  // workgroups per CU
  static constexpr bool PINGPONG = (NW == 8);    // two halves alternate MFMA and VALU phases
  static constexpr int WAVES_PER_SIMD = NW * OCC / 4;
  static constexpr int BM = 32 * NW;             // query rows per tile
  static constexpr int K_BYTES = kBN * D * 2;    // one K block in LDS
  static constexpr int V_BYTES = kBN * DV * 2;   // one V block in LDS
  static constexpr int THREADS = NW * kWave;
};

// Kernel arguments.
struct Args {
  const __bf16 *q, *k, *v;
  __bf16 *o;
  float *lse;
  const int *cu;            // varlen query offsets or nullptr
  const int *cu_k;          // varlen key offsets (cu for self-attention) or nullptr
  int B, H, S;              // S: (longest) query length
  int Sk;                   // (longest) key length
  int Hkv;                  // K/V heads (divides H); query head h reads K/V head h / (H / Hkv)
  float c;                  // scale * log2(e)
  float tau;                // rescale threshold (log2 units) of the max-first test
  float bound;              // 2^tau: largest lane share of a block's row sum kept without rescale
  unsigned long long *counters;
  int workers;              // persistent: number of workgroups
  // split-KV: each workgroup covers key blocks [split*kbps, (split+1)*kbps)
  // and writes a partial O (fp32) and LSE into the workspace, which a
  // combine kernel merges
  float *ws_o, *ws_lse;
  int kbps;
  // persistent dense causal with split levels: the nsplit costliest m-blocks
  // run as two parts (fa_sched.h); each part's partial rows go to ws_o /
  // ws_lse, and hs_cnt holds one arrival counter per (split tile, wave),
  // zero between launches
  int nsplit;
  int *hs_cnt;
};

// Per-wave state of one tile.
template <int D>
struct WaveState {
  bf16x8 qf[D / 16];                // Q rows of this wave (B operand of S^T = K Q^T)
  f32x16 o[head_dim_v<D>() / 32];   // O^T accumulators
  f32x16 s[2];        // S^T of the block between its product and its softmax
  bf16x8 p[4];        // bf16 P of the block between its softmax and its PV product
  float m_ref, l32;
};

// S^T = K Q^T for one 64-key block: two 32-key sub-blocks, D/16 k-steps each.
// The K operands are read kPrefK k-steps ahead of their products (the
// scheduling barriers keep that order), so LDS latency hides behind the
// matrix unit instead of stalling each product.
constexpr int kPrefK = 2;
template <int D>
__device__ __forceinline__ void qk_step(WaveState<D> &st, const LdsAddr<D> &la,
                                        const char LDS_AS *kbuf, const char LDS_AS *kbuf2) {
  constexpr int NS = D / 16;
  const unsigned ka = la.ky + lds_u32(kbuf);
  const unsigned ka2 = la.ky2 + lds_u32(kbuf2);
  bf16x8 kf[NS][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.s[kb][e] = 0.0f;
#pragma unroll
  for (int s = 0; s < kPrefK && s < NS; ++s) {
    kf[s][0] = read_k_step<D>(ka, ka2, 0, s);
    kf[s][1] = read_k_step<D>(ka, ka2, 1, s);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s + kPrefK < NS) {
      kf[s + kPrefK][0] = read_k_step<D>(ka, ka2, 0, s + kPrefK);
      kf[s + kPrefK][1] = read_k_step<D>(ka, ka2, 1, s + kPrefK);
    }
    __builtin_amdgcn_sched_barrier(0);
    st.s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s][0], st.qf[s], st.s[0], 0, 0, 0);
    st.s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s][1], st.qf[s], st.s[1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Softmax of one block, in pieces the pipelined D = 256 body interleaves with
// matrix products.  Scores are S^T accumulators s[kb] (kb: 32-key sub-block);
// the key index of s[kb][4i+j] is n0 + 32kb + 8i + 4h + j, h = lane / 32.
//
// mask_slice: mask scores e0 .. e0+7 of sub-block kb.  A key is kept iff
// key < L and (non-causal or key <= row), i.e. iff its in-block offset
// 32kb + 8(e>>2) + (e&3), a constant, is below the per-lane limit lim: one
// compare and one select per score.  max_slice folds the same scores into
// the running maximum mx.
template <bool CAUSAL>
__device__ __forceinline__ int mask_limit(int lane, int n0, int row, int L) {
  return (CAUSAL ? (row + 1 < L ? row + 1 : L) : L) - n0 - 4 * (lane >> 5);
}
__device__ __forceinline__ void mask_slice(f32x16 (&s)[2], int kb, int e0, int lim) {
#pragma unroll
  for (int e = e0; e < e0 + 8; ++e) {
    const int off = 32 * kb + 8 * (e >> 2) + (e & 3);
    s[kb][e] = off < lim ? s[kb][e] : -INFINITY;
  }
}
__device__ __forceinline__ void max_slice(const f32x16 (&s)[2], int kb, int e0, float &mx) {
#pragma unroll
  for (int e = e0; e < e0 + 8; ++e) mx = fmaxf(mx, s[kb][e]);
}

// Conditional rescale decided from the block's raw row maximum (both
// half-waves combined), for the pipelined single-wave body: the wave moves
// to max(m_ref, m_blk) when any row's block maximum exceeds m_ref by more
// than tau (paper section 3.1.4).  rescale_decide moves m_ref and the row
// sum; the caller scales O by alpha when `any`, after the products still in
// flight that use the old scale.
struct Rescale {
  bool any;
  float alpha;
};
template <int D, bool COUNT>
__device__ __forceinline__ Rescale rescale_decide(WaveState<D> &st, float mx, int lane,
                                                  const Args &a) {
  mx = max_halves(mx);
  const float m_blk = mx * a.c;  // -inf when the whole row of the block is masked
  const bool need = m_blk > st.m_ref + a.tau;
  Rescale r{__builtin_amdgcn_ballot_w64(need) != 0, 1.0f};
  if (r.any) {
    const float m_new = fmaxf(st.m_ref, m_blk);
    r.alpha = (st.m_ref == -INFINITY) ? 0.0f : exp2_hw(st.m_ref - m_new);
    st.m_ref = m_new;
    st.l32 *= r.alpha;
    if constexpr (COUNT) {
      if (lane == 0) atomicAdd(&a.counters[0], 1ull);
    }
  }
  if constexpr (COUNT) {
    if (lane == 0) atomicAdd(&a.counters[1], 1ull);
  }
  return r;
}
template <int D>
__device__ __forceinline__ void scale_o(WaveState<D> &st, float alpha) {
#pragma unroll
  for (int dt = 0; dt < head_dim_v<D>() / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[dt][e] *= alpha;
}
// The reference maximum the block's exponentials use.
template <int D>
__device__ __forceinline__ float m_use_of(const WaveState<D> &st) {
  return (st.m_ref == -INFINITY) ? 0.0f : st.m_ref;
}

// p = exp2(c*s - m) for scores e, e+1 of sub-block kb: row sum (one partial
// sum per sub-block, to halve the dependent chain) and bf16 pack into the PV
// operand layout.
template <int EMU>
__device__ __forceinline__ void exp_pair(bf16x8 (&p)[4], const f32x16 (&s)[2], int kb, int e,
                                         float m_use, bool last_block, const Args &a,
                                         float (&lsum)[2]) {
  const float x0 = __builtin_fmaf(s[kb][e], a.c, -m_use);
  const float x1 = __builtin_fmaf(s[kb][e + 1], a.c, -m_use);
  float p0, p1;
  if (EMU > 0 && !last_block && (e % EMU) == 0) p0 = exp2_poly(x0);
  else p0 = exp2_hw(x0);
  p1 = exp2_hw(x1);
  lsum[kb] += p0 + p1;
  const bf16x2 pb = {(__bf16)p0, (__bf16)p1};
  const int t = 2 * kb + (e >> 3);
  p[t][e & 7] = pb[0];
  p[t][(e & 7) + 1] = pb[1];
}

// Exponentials of one block against the reference m_use: p = exp2(c*s - m_use),
// this lane's share of the row sum, and the bf16 P operand.
template <int EMU>
__device__ __forceinline__ float exp_block(bf16x8 (&p)[4], const f32x16 (&s)[2], float m_use,
                                           bool last_block, const Args &a) {
  float lsum[2] = {0.0f, 0.0f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; e += 2) exp_pair<EMU>(p, s, kb, e, m_use, last_block, a, lsum);
  return lsum[0] + lsum[1];
}

// The rescale path of a block: row maximum of the block's scores (raw; c > 0
// so it commutes with scaling), new reference m_new = max(m_ref, m_blk) for
// every row of the wave, O and the row sum scaled by exp2(m_ref - m_new), and
// the block's exponentials against m_new.  Returns the lane's row-sum share.
template <int D, int EMU, bool COUNT>
__device__ __forceinline__ float rescale_block(WaveState<D> &st, int lane, bool last_block,
                                               const Args &a) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e0 = 0; e0 < 16; e0 += 8) max_slice(st.s, kb, e0, mx);
  const float m_blk = max_halves(mx) * a.c;  // -inf when the row's block is fully masked
  const float m_new = fmaxf(st.m_ref, m_blk);
  const float alpha = (st.m_ref == -INFINITY) ? 0.0f : exp2_hw(st.m_ref - m_new);
  st.m_ref = m_new;
  st.l32 *= alpha;
  scale_o<D>(st, alpha);
  if constexpr (COUNT) {
    if (lane == 0) atomicAdd(&a.counters[0], 1ull);
  }
  return exp_block<EMU>(st.p, st.s, m_use_of<D>(st), last_block, a);
}

// Mask, conditional rescale, exp2, row sums and bf16 packing of one block
// (scores in st.s, probabilities out to st.p).
//
// The rescale condition (paper section 3.1.4: correct O and the row sum only
// when the running maximum has grown enough to threaten the range of the
// exponentials) is tested on the exponentials themselves.  They are first
// computed against the stale reference m_ref; if every lane's share of the
// block's row sum stays within 2^tau, so does every p (all p >= 0), and the
// block is done without any row-maximum reduction.  Otherwise, and when some
// row of the wave has no reference yet (its first keys), the whole wave takes
// the rescale path: block row maximum, new reference max(m_ref, m_blk) for
// every row, O and the row sum scaled by exp2(m_ref - m_new), exponentials
// again.  The decision is a wave-wide ballot, so the wave never diverges.
// side(0) runs first and side(1) after the mask: the caller hangs its K/V
// copies and operand prefetches there.
template <int D, bool CAUSAL, int EMU, bool COUNT, typename Side>
__device__ __forceinline__ void softmax_step(WaveState<D> &st, int lane, int n0, int row, int L,
                                             bool need_mask, bool last_block, const Args &a,
                                             Side &&side) {
  side(0);
  if (need_mask) {
    const int lim = mask_limit<CAUSAL>(lane, n0, row, L);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e0 = 0; e0 < 16; e0 += 8) mask_slice(st.s, kb, e0, lim);
  }
  side(1);
  bool redo = __builtin_amdgcn_ballot_w64(st.m_ref == -INFINITY) != 0;
  float lsum = 0.0f;
  if (!redo) {
    lsum = exp_block<EMU>(st.p, st.s, st.m_ref, last_block, a);
    redo = __builtin_amdgcn_ballot_w64(!(lsum <= a.bound)) != 0;
  }
  if (redo) lsum = rescale_block<D, EMU, COUNT>(st, lane, last_block, a);
  if constexpr (COUNT) {
    if (lane == 0) atomicAdd(&a.counters[1], 1ull);
  }
  st.l32 += lsum;
}

// O^T += V^T P^T for one block: D/32 d-tiles, 4 steps of 16 keys.  The V^T
// operands of key step t+1 are read while the products of step t run.
template <int D>
__device__ __forceinline__ void pv_step(WaveState<D> &st, const LdsAddr<D> &la,
                                        const char LDS_AS *vbuf) {
  constexpr int DV = head_dim_v<D>();
  constexpr int NT = DV / 32;
  const unsigned va0 = la.vw0 + lds_u32(vbuf), va1 = la.vw1 + lds_u32(vbuf);
  bf16x8 vf[4][NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) vf[0][dt] = read_vt<DV>(va0, va1, 0, dt);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t + 1 < 4) {
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) vf[t + 1][dt] = read_vt<DV>(va0, va1, t + 1, dt);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t][dt], st.p[t], st.o[dt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// The pipelined single-wave body (D = 256; run_tile) runs the softmax of
// block j between the PV products of block j-1.  MFMAs run asynchronously to
// the instructions of their own wave, so VALU work placed between them runs
// in the matrix unit's shadow; the scheduling barriers keep that order.
// ---------------------------------------------------------------------------
// O^T += V^T P_prev^T (the previous block), with the exp pairs of the current
// block (scores s, probabilities out to p_cur) spread over its products.
// V^T of key step t+1, d tile dt, is read right after the product that
// consumed the step-t operand of the same tile.  (Placing the mask, row max
// and rescale decision beside the first products as well measured slower:
// the decision waits on the whole row maximum in the middle of the stream.)
template <int D, int EMU>
__device__ __forceinline__ void pv_with_exp(WaveState<D> &st, const LdsAddr<D> &la,
                                            const char LDS_AS *vbuf, const bf16x8 (&p_prev)[4],
                                            const f32x16 (&s)[2], bf16x8 (&p_cur)[4],
                                            float m_use, bool last_block, const Args &a,
                                            float (&lsum)[2]) {
  constexpr int DV = head_dim_v<D>();
  constexpr int NT = DV / 32;
  constexpr int PAIRS = 16;  // score pairs per lane and block
  static_assert((4 * NT) % PAIRS == 0, "exp pairs spread evenly over the products");
  const unsigned va0 = la.vw0 + lds_u32(vbuf), va1 = la.vw1 + lds_u32(vbuf);
  bf16x8 vf[4][NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) vf[0][dt] = read_vt<DV>(va0, va1, 0, dt);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      __builtin_amdgcn_sched_barrier(0);
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t][dt], p_prev[t], st.o[dt], 0, 0, 0);
      if (t + 1 < 4) vf[t + 1][dt] = read_vt<DV>(va0, va1, t + 1, dt);
      if ((t * NT + dt) % (4 * NT / PAIRS) == 0) {
        const int i = (t * NT + dt) / (4 * NT / PAIRS);
        exp_pair<EMU>(p_cur, s, i / 8, 2 * (i % 8), m_use, last_block, a, lsum);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// O^T += V^T P^T for a given P set (the pipelined body's last block).
template <int D>
__device__ __forceinline__ void pv_of(WaveState<D> &st, const LdsAddr<D> &la,
                                      const char LDS_AS *vbuf, const bf16x8 (&p)[4]) {
  constexpr int DV = head_dim_v<D>();
  constexpr int NT = DV / 32;
  const unsigned va0 = la.vw0 + lds_u32(vbuf), va1 = la.vw1 + lds_u32(vbuf);
  bf16x8 vf[4][NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) vf[0][dt] = read_vt<DV>(va0, va1, 0, dt);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      __builtin_amdgcn_sched_barrier(0);
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t][dt], p[t], st.o[dt], 0, 0, 0);
      if (t + 1 < 4) vf[t + 1][dt] = read_vt<DV>(va0, va1, t + 1, dt);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Which KV blocks a wave (32 rows from wrow0) needs, and which need masking.
// The causal mask is aligned to the bottom-right corner: query row i may use
// key j when j <= i + koff, koff = Lk - Lq (0 for self-attention).  krow0 and
// krow_last are the last usable keys of the wave's first and last row.
struct WaveRows {
  int wrow0, wrow_last;   // first and last valid row of the wave
  int krow0, krow_last;   // wrow0 + koff, wrow_last + koff
  bool active;
  int last_block;         // index of the wave's last useful block (-1: none)
  __device__ __forceinline__ bool useful(int j, bool causal) const {
    return active && (!causal || j * kBN <= krow_last);
  }
  __device__ __forceinline__ bool need_mask(int j, int Lk, bool causal) const {
    const int n0 = j * kBN;
    return (n0 + kBN > Lk) || (causal && n0 + kBN - 1 > krow0);
  }
};

// Process one tile (b, h, mb) with the whole workgroup.
//
// Eight-wave workgroups (D <= 128) run a two-phase "ping-pong" per KV block
// (the FlashAttention-4 paper, section 3.1.2: two output tiles per CTA, the
// matrix unit working on one while the other does its softmax).  Half 0
// (waves 0-3, one per SIMD) and half 1 (waves 4-7) hold different rows.
// After the barrier that opens interval j they run
//   half 0:  S_j = K_j Q^T, O += V_{j-1} P_{j-1}   then   softmax_j
//   half 1:  softmax_{j-1}                         then   S_j = K_j Q^T, O += V_{j-1} P_{j-1}
// so each SIMD has one wave on MFMA while the other is on VALU.  The matrix
// phase runs at raised wave priority, which keeps the matrix unit fed when
// both waves of a SIMD have an instruction ready; no barrier separates the
// two phases (the halves keep their offset on their own, and a barrier there
// only added the wait for the slower half).  K/V blocks rotate through four
// LDS buffers: block j+2 is copied while the workgroup still reads K_j and
// V_{j-1}.  (D = 192 keeps K in a ring of three, since K_{j-1} is no longer
// read in interval j, and V in a ring of four; see KvLayout.)  Four-wave
// workgroups (D = 256) run the plain sequence per block with two buffers.
// LDS placement of the K/V ring of a ping-pong instance.  Every part starts
// at a multiple of its 64-row block size, as the operand addressing needs.
//   D = 64, 128: four slots of [K block | V block], K_j and V_j in slot j%4.
//   D = 192:     V_j in slot j%4 (4 x 16 KiB at 0), K_j in slot j%3 with its
//                128-wide part (3 x 16 KiB at 64 KiB) and 64-wide part
//                (3 x 8 KiB at 112 KiB): 136 KiB in all.
template <int D>
struct KvLayout {
  using C = Cfg<D>;
  static constexpr int BYTES = (D == 192) ? 136 * 1024 : 4 * (C::K_BYTES + C::V_BYTES);
  static __device__ __forceinline__ char LDS_AS *k(char LDS_AS *lds, int j) {
    if constexpr (D == 192) return lds + 64 * 1024 + (j % 3) * 16 * 1024;
    else return lds + (j & 3) * (C::K_BYTES + C::V_BYTES);
  }
  static __device__ __forceinline__ char LDS_AS *k2(char LDS_AS *lds, int j) {
    if constexpr (D == 192) return lds + 112 * 1024 + (j % 3) * 8 * 1024;
    else return lds;  // unused
  }
  static __device__ __forceinline__ char LDS_AS *v(char LDS_AS *lds, int j) {
    if constexpr (D == 192) return lds + (j & 3) * 16 * 1024;
    else return lds + (j & 3) * (C::K_BYTES + C::V_BYTES) + C::K_BYTES;
  }
};

// PACK: h is a K/V head and the tile's rows are the (query index i, query
// head g of the group) pairs of that K/V head, row r = i*G + g, in one tile
// (the caller guarantees L*G <= BM): the group's K/V are streamed once for
// all G query heads instead of once per head (decode with grouped-query
// attention).  Otherwise row r is query index m0 + r of query head h.
template <int D, bool CAUSAL, bool VARLEN, int EMU, bool COUNT, bool SPLIT = false,
          bool PACK = false>
__device__ __forceinline__ void run_tile(const Args &a, int b, int h, int mb, char LDS_AS *lds,
                                         int split = 0, int part = 0) {
  using C = Cfg<D>;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  long long tok0, ktok0;  // first query token, first key token of the sequence
  int L, Lk;              // query length, key length
  if constexpr (VARLEN) {
    tok0 = a.cu[b];
    const int Lr = a.cu[b + 1] - a.cu[b];
    L = Lr < 0 ? 0 : (Lr > a.S ? a.S : Lr);
    ktok0 = a.cu_k[b];
    const int Lkr = a.cu_k[b + 1] - a.cu_k[b];
    Lk = Lkr < 0 ? 0 : (Lkr > a.Sk ? a.Sk : Lkr);
  } else {
    tok0 = (long long)b * a.S;
    L = a.S;
    ktok0 = (long long)b * a.Sk;
    Lk = a.Sk;
  }
  int koff = Lk - L;  // bottom-right causal alignment
  if constexpr (SPLIT) {
    // Keys [lo, hi) only: the tile sees a key sequence that starts at key
    // lo, with the causal alignment shifted to match.
    const int lo = split * a.kbps * kBN;
    const int hi = (Lk - lo > a.kbps * kBN) ? lo + a.kbps * kBN : Lk;
    ktok0 += lo;
    koff -= lo;
    Lk = hi > lo ? hi - lo : 0;
  }
  if (part != 0) {
    // One part of a split m-block (dense causal self-attention): of the
    // tile's n key blocks, part 1 takes the first floor(n/2) and part 2 the
    // rest, each as a key sequence of its own (as a split-KV slice).
    const int e = mb * C::BM + C::BM + koff;
    const int n_full = e < 0 ? 0 : (e < Lk ? e : Lk);
    const int half = fa::ceil_div(n_full, kBN) / 2 * kBN;
    const int lo = part == 1 ? 0 : half;
    const int hi = part == 1 ? half : n_full;
    ktok0 += lo;
    koff -= lo;
    Lk = hi - lo;
  }
  const int m0 = mb * C::BM;
  if (m0 >= L) return;  // workgroup-uniform
  const int H = a.H;
  const int Hk = a.Hkv;              // K/V row layout: [.., Hk, D]
  const int G = PACK ? H / Hk : 1;   // query heads per row index (packed)
  const int R = PACK ? L * G : L;    // rows of the tile's row space
  const int hk = PACK ? h : h / (H / Hk);  // the K/V head the rows read
  WaveRows wr;
  wr.wrow0 = m0 + wave * 32;
  wr.active = wr.wrow0 < R;
  wr.wrow_last = (wr.wrow0 + 31 < R - 1) ? wr.wrow0 + 31 : R - 1;
  wr.krow0 = (PACK ? wr.wrow0 / G : wr.wrow0) + koff;
  wr.krow_last = (PACK ? wr.wrow_last / G : wr.wrow_last) + koff;
  const int row = wr.wrow0 + (lane & 31);
  const int qi = PACK ? row / G : row;          // query index of the lane's row
  const int hq = PACK ? hk * G + row % G : h;   // query head of the lane's row

  // KV range shared by the workgroup (0 blocks: no row of the tile has a key)
  int n_end = Lk;
  if (CAUSAL) {
    const int e = (PACK ? L : m0 + C::BM) + koff;
    n_end = e < 0 ? 0 : (e < Lk ? e : Lk);
  }
  const int nblocks = fa::ceil_div(n_end, kBN);
  if (CAUSAL) {
    const int lb = wr.krow_last >= 0 ? wr.krow_last / kBN : -1;
    wr.last_block = lb < nblocks - 1 ? lb : nblocks - 1;
  } else {
    wr.last_block = nblocks - 1;
  }

  // Q fragments: lane l holds row (l%32), d = 16s + 8(l/32) .. +7
  WaveState<D> st;
  {
    const int rc = row < R ? row : R - 1;  // rows past the end read the last row (never stored)
    const int qrow = PACK ? rc / G : rc;
    const int qhead = PACK ? hk * G + rc % G : h;
    const bf16x8 *qp =
        (const bf16x8 *)(a.q + ((tok0 + qrow) * H + qhead) * (long long)D + 8 * (lane >> 5));
#pragma unroll
    for (int s = 0; s < D / 16; ++s) st.qf[s] = qp[2 * s];
    // Opaque to the compiler: Q stays in registers for the whole tile instead
    // of being re-fetched inside the KV loop (a re-fetch would share the
    // in-order vector-memory counter with the K/V prefetch and wait for it).
#pragma unroll
    for (int s = 0; s < D / 16; ++s) asm volatile("" : "+v"(st.qf[s]));
  }
  constexpr int DV = C::DV;
#pragma unroll
  for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[dt][e] = 0.0f;
  st.m_ref = -INFINITY;
  st.l32 = 0.0f;

  // K and V loaders (one object when both rows have the same width)
  BlockLoader<D, C::NW> ldk;
  ldk.init(Hk, wave, lane);
  BlockLoader<DV, C::NW> ldv_own;
  if constexpr (DV != D) ldv_own.init(Hk, wave, lane);
  const auto &ldv = [&]() -> const BlockLoader<DV, C::NW> & {
    if constexpr (DV != D) return ldv_own;
    else return ldk;
  }();
  constexpr int LOADS_BLOCK = BlockLoader<D, C::NW>::LOADS + BlockLoader<DV, C::NW>::LOADS;
  LdsAddr<D> la;
  la.init(lane);

  if constexpr (C::PINGPONG) {
    const int half = wave / 4;
    using KV = KvLayout<D>;
    auto kbuf = [&](int j) { return KV::k(lds, j); };
    auto kbuf2 = [&](int j) { return KV::k2(lds, j); };
    auto vbuf = [&](int j) { return KV::v(lds, j); };
    // Start of interval it: this wave's copies of block it have landed
    // (block it+1 may still be in flight), then the barrier makes everyone's
    // visible and ends interval it-1, so the buffer of block it-2 is free for
    // block it+2: copies run two intervals ahead of their use.
    auto interval_start = [&](int it) {
      if (it + 1 < nblocks) wait_vmcnt<LOADS_BLOCK>();
      else wait_vmcnt<0>();
      barrier_after_reads();
    };
    // This wave's copies of block it+2 (K on side 0, V on side 1), issued
    // from its softmax phase of interval it.  All eight waves issuing right
    // after the barrier would queue 32 KB on the CU's vector-memory path at
    // once and hold the waves that start matrix products behind it.
    // Part 0: this wave's K copies of block it+2; part 1: its V copies.
    const char *kseq = ldk.seq_base(a.k, ktok0, Hk, hk);
    const char *vseq = ldv.seq_base(a.v, ktok0, Hk, hk);
    auto copies = [&](int it) {
      return [&, it](int part) {
        if (it + 2 < nblocks) {
          if (part == 0) ldk.issue_at(kseq, (it + 2) * kBN, Lk, kbuf(it + 2), kbuf2(it + 2));
          else ldv.issue_at(vseq, (it + 2) * kBN, Lk, vbuf(it + 2));
        }
      };
    };
    auto softmax_phase = [&](bool run, int j, int it) {
      auto side = copies(it);
      if (run) {
        softmax_step<D, CAUSAL, EMU, COUNT>(st, lane, j * kBN, qi + koff, Lk,
                                            wr.need_mask(j, Lk, CAUSAL), j == wr.last_block, a,
                                            side);
      } else {
        side(0);
        side(1);
      }
    };
    // A persistent workgroup's waves leave a tile at different times (half
    // 1's last PV runs after half 0's): every wave is done reading the
    // previous tile's ring before this tile's first copies overwrite it.
    // (Placed after the Q load, whose latency covers the wait.)
    barrier_after_reads();
    if (nblocks > 0) {
      ldk.issue_at(kseq, 0, Lk, kbuf(0), kbuf2(0));
      ldv.issue_at(vseq, 0, Lk, vbuf(0));
    }
    if (nblocks > 1) {
      ldk.issue_at(kseq, kBN, Lk, kbuf(1), kbuf2(1));
      ldv.issue_at(vseq, kBN, Lk, vbuf(1));
    }
    // The two halves run separate loops that meet at the same barriers.
    if (half == 0) {
      for (int it = 0; it <= nblocks; ++it) {
        interval_start(it);
        const bool cur = it < nblocks && wr.useful(it, CAUSAL);
        __builtin_amdgcn_s_setprio(kMatrixPrio);
        if (cur) qk_step<D>(st, la, kbuf(it), kbuf2(it));
        __builtin_amdgcn_sched_barrier(0);
        if (it > 0 && wr.useful(it - 1, CAUSAL)) pv_step<D>(st, la, vbuf(it - 1));
        __builtin_amdgcn_s_setprio(0);
        debug_phase_barrier();
        softmax_phase(cur, it, it);
      }
    } else {
      for (int it = 0; it <= nblocks; ++it) {
        interval_start(it);
        const bool prev = it > 0 && wr.useful(it - 1, CAUSAL);
        softmax_phase(prev, it - 1, it);
        debug_phase_barrier();
        __builtin_amdgcn_s_setprio(kMatrixPrio);
        if (it < nblocks && wr.useful(it, CAUSAL)) qk_step<D>(st, la, kbuf(it), kbuf2(it));
        __builtin_amdgcn_sched_barrier(0);
        if (prev) pv_step<D>(st, la, vbuf(it - 1));
        __builtin_amdgcn_s_setprio(0);
      }
    }
  } else if constexpr (!VARLEN) {
    // One wave per SIMD (D = 256: O alone is 128 registers per lane), so
    // the matrix/softmax overlap comes from within the wave.  The iteration
    // of block j runs S_j = K_j Q^T and its mask, then the exp loop of block
    // j between the PV products of block j-1 (two P register sets), then
    // the rescale decision.  Every wave runs every block of the tile, so the
    // loop has one path: a wave whose rows lie past the sequence end works
    // on clamped rows and stores nothing, and under a causal mask the blocks
    // past a wave's diagonal are fully masked (their exponentials are zero;
    // at most the tile's last two blocks for some of its waves).  V_{j-1} is
    // read in the iteration of block j, so K sits in a ring of two 32 KiB
    // slots and V in a ring of three (160 KiB in all).  After the barrier
    // that opens iteration j, slot ((j+1)&1) of K (K_{j-1}) and slot
    // ((j+1)%3) of V (V_{j-2}) are free, and block j+1 is copied into them:
    // K one iteration ahead of its use, V two.
    static_assert(D == DV, "the pipelined single-wave body keeps K and V blocks of one size");
    constexpr int BLK = C::K_BYTES;
    auto kslot = [&](int j) { return lds + (j & 1) * BLK; };
    auto vslot = [&](int j) { return lds + 2 * BLK + (j % 3) * BLK; };
    constexpr int LK = BlockLoader<D, C::NW>::LOADS;
    const char *kseq = ldk.seq_base(a.k, ktok0, Hk, hk);
    const char *vseq = ldk.seq_base(a.v, ktok0, Hk, hk);
    auto issue_block = [&](int j) {
      if (j < nblocks) {
        ldk.issue_at(kseq, j * kBN, Lk, kslot(j));
        ldk.issue_at(vseq, j * kBN, Lk, vslot(j));
      }
    };
    // Opens iteration j: K_j and V_{j-1} have landed (V_j may still be in
    // flight), the barrier makes them visible and frees the slots of block j+1.
    auto open = [&](int j) {
      if (j < nblocks) wait_vmcnt<LK>();
      else wait_vmcnt<0>();
      barrier_after_reads();
      issue_block(j + 1);
    };
    // S_j and its mask.
    auto scores = [&](int j) {
      qk_step<D>(st, la, kslot(j), kslot(j));
      if (wr.need_mask(j, Lk, CAUSAL)) {
        const int lim = mask_limit<CAUSAL>(lane, j * kBN, qi + koff, Lk);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e0 = 0; e0 < 16; e0 += 8) mask_slice(st.s, kb, e0, lim);
      }
    };
    // The max-first form of the rescale test: the block's row maximum, then
    // the decision (rescale_decide).  The first block takes it (no row has a
    // reference yet); later blocks take the exponential-based form.
    auto decide = [&](float &m_use) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e0 = 0; e0 < 16; e0 += 8) max_slice(st.s, kb, e0, mx);
      const Rescale r = rescale_decide<D, COUNT>(st, mx, lane, a);
      m_use = m_use_of<D>(st);
      return r;
    };
    bf16x8 p_prev[4];
    // every wave is done reading the previous tile's rings (the last PV of a
    // persistent workgroup's previous tile) before this tile's first copies
    barrier_after_reads();
    if (nblocks > 0) {
      issue_block(0);
      open(0);
      scores(0);
      float m_use;
      const Rescale r = decide(m_use);  // O is still zero: nothing to scale
      (void)r;
      float lsum[2] = {0.0f, 0.0f};
      const bool last = wr.last_block == 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) exp_pair<EMU>(st.p, st.s, kb, e, m_use, last, a, lsum);
      st.l32 += lsum[0] + lsum[1];
    }
    for (int j = 1; j < nblocks; ++j) {
#pragma unroll
      for (int t = 0; t < 4; ++t) p_prev[t] = st.p[t];
      open(j);
      scores(j);
      const bool last = j == wr.last_block;  // the wave's last block with keys
      float lsum[2] = {0.0f, 0.0f};
      // The exponentials against the reference as it stands, between the PV
      // products of block j-1 (softmax_step's test): when every lane's share
      // of the block's row sum stays within 2^tau, so does every p, and the
      // block needs no row maximum.  Otherwise the wave takes the rescale
      // path, after those products: the block's row maximum, O and the row
      // sum scaled to the new reference, the exponentials again.  (A row has
      // a reference after block 0 unless the causal alignment leaves it no
      // key there; such a row's scores stay -inf until its first key, whose
      // exponentials then fail the test and take the rescale path.)
      pv_with_exp<D, EMU>(st, la, vslot(j - 1), p_prev, st.s, st.p, m_use_of<D>(st), last, a,
                          lsum);
      float ls = lsum[0] + lsum[1];
      if (__builtin_amdgcn_ballot_w64(!(ls <= a.bound)) != 0)
        ls = rescale_block<D, EMU, COUNT>(st, lane, last, a);
      if constexpr (COUNT) {
        if (lane == 0) atomicAdd(&a.counters[1], 1ull);
      }
      st.l32 += ls;
    }
    if (nblocks > 0) {
      open(nblocks);
      pv_of<D>(st, la, vslot(nblocks - 1), st.p);
    }
  } else {
    static_assert(D == DV, "the serial path keeps K and V blocks of one size");
    char LDS_AS *kb0 = lds;
    char LDS_AS *vb0 = lds + C::K_BYTES;
    char LDS_AS *kb1 = lds + 2 * C::K_BYTES;
    char LDS_AS *vb1 = lds + 3 * C::K_BYTES;
    if (nblocks > 0) {
      ldk.issue(a.k, ktok0, Hk, hk, 0, Lk, kb0);
      ldv.issue(a.v, ktok0, Hk, hk, 0, Lk, vb0);
    }
    for (int j = 0; j < nblocks; ++j) {
      const int n0 = j * kBN;
      char LDS_AS *kcur = (j & 1) ? kb1 : kb0;
      char LDS_AS *vcur = (j & 1) ? vb1 : vb0;
      if (j + 1 < nblocks) {
        char LDS_AS *knext = (j & 1) ? kb0 : kb1;
        char LDS_AS *vnext = (j & 1) ? vb0 : vb1;
        ldk.issue(a.k, ktok0, Hk, hk, n0 + kBN, Lk, knext);
        ldv.issue(a.v, ktok0, Hk, hk, n0 + kBN, Lk, vnext);
        wait_vmcnt<LOADS_BLOCK>();
      } else {
        wait_vmcnt<0>();
      }
      barrier_nofence();
      if (wr.useful(j, CAUSAL)) {
        qk_step<D>(st, la, kcur, kcur);
        softmax_step<D, CAUSAL, EMU, COUNT>(st, lane, n0, qi + koff, Lk,
                                            wr.need_mask(j, Lk, CAUSAL), j == wr.last_block, a,
                                            [](int) {});
        pv_step<D>(st, la, vcur);
      }
      barrier_after_reads();  // every wave is done reading this buffer
    }
  }

  if (!wr.active) return;
  // ---- epilogue: combine the two half-wave partial sums of each row
  const float l32 = sum_halves(st.l32);
  if constexpr (SPLIT) {
    // partial O (normalised over this split's keys) and LSE, fp32, into the
    // workspace slice of this split (rows of B*S query slots)
    if (row < R) {
      const float inv = l32 > 0.0f ? 1.0f / l32 : 0.0f;
      const int hh = lane >> 5;
      const long long slots = (long long)a.B * a.S * H;
      float *op = a.ws_o + (split * slots + (tok0 + qi) * H + hq) * (long long)DV + 4 * hh;
      typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 out = {st.o[dt][4 * i + 0] * inv, st.o[dt][4 * i + 1] * inv,
                       st.o[dt][4 * i + 2] * inv, st.o[dt][4 * i + 3] * inv};
          *(f32x4 *)(op + 32 * dt + 8 * i) = out;
        }
      if (hh == 0) {
        const float lse = (st.m_ref + log2f(l32)) * kLn2;
        float *lp = a.ws_lse + split * slots;
        if constexpr (VARLEN) lp[(long long)hq * a.cu[a.B] + tok0 + qi] = lse;
        else lp[((long long)b * H + hq) * a.S + qi] = lse;
      }
    }
    return;
  }
  if (part != 0) {
    // A part of a split m-block: the wave writes its partial rows (O
    // normalised over the part's keys, fp32, and the LSE) to the part's
    // slot and counts its arrival; the wave that arrives second for these
    // rows reads the other part's slot and writes the merged rows.  No wave
    // waits for another.
    //
    // The two parts may run on different XCDs, whose L2 caches are not
    // coherent with each other.  The slots are written and read with
    // device-coherent accesses (sc1: through to memory, and from it), so no
    // cache-wide write-back or invalidation is needed: the writer waits for
    // its stores to complete before it counts, and the reader reads after
    // the count it saw.  (Agent-scope fences would write back and invalidate
    // the whole L2 of the XCD, once per wave: measured 6x slower.)
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    constexpr int kCoherent = 16;  // cache policy sc1: coherent at device scope
    const int nmb = fa::ceil_div(a.S, C::BM);
    const int tix = (b * H + h) * a.nsplit + (mb - (nmb - a.nsplit));  // split tile
    const long long own = 2LL * tix + (part - 1), other = 2LL * tix + (2 - part);
    const int r = row - m0;  // row within the tile
    const int hh = lane >> 5;
    const float inv = l32 > 0.0f ? 1.0f / l32 : 0.0f;
    const float lse_own = (st.m_ref + log2f(l32)) * kLn2;  // -inf for a row without keys
    constexpr int SLOT = C::BM * DV * 4;                   // bytes of one part's rows
    const __amdgpu_buffer_rsrc_t own_o =
        __builtin_amdgcn_make_buffer_rsrc(a.ws_o + own * C::BM * DV, (short)0, SLOT, 0x00020000);
    const __amdgpu_buffer_rsrc_t other_o =
        __builtin_amdgcn_make_buffer_rsrc(a.ws_o + other * C::BM * DV, (short)0, SLOT, 0x00020000);
    const int lane_off = (r * DV + 4 * hh) * 4;  // byte offset of the lane's first value
    f32x4 mine[DV / 32][4];
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mine[dt][i] = f32x4{st.o[dt][4 * i + 0] * inv, st.o[dt][4 * i + 1] * inv,
                            st.o[dt][4 * i + 2] * inv, st.o[dt][4 * i + 3] * inv};
    if (row < R) {
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, mine[dt][i]), own_o,
                                                 lane_off + (32 * dt + 8 * i) * 4, 0, kCoherent);
      if (hh == 0)
        __hip_atomic_store(a.ws_lse + own * C::BM + r, lse_own, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmcnt<0>();  // this wave's partial rows are in memory before it counts
    int *cnt = a.hs_cnt + (long long)tix * C::NW + wave;
    int prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev == 0) return;  // the other part's wave merges these rows
    // both parts are in: zero for the next launch
    if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (row < R) {
      const float lse_x = __hip_atomic_load(a.ws_lse + other * C::BM + r, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
      // (part 1, part 2) order whichever arrived last: the merged rows do not
      // depend on the arrival order
      const float l1 = part == 1 ? lse_own : lse_x;
      const float l2 = part == 1 ? lse_x : lse_own;
      const float mx = fmaxf(l1, l2);
      const float w1 = mx == -INFINITY ? 0.0f : exp2_hw((l1 - mx) * kLog2e);
      const float w2 = mx == -INFINITY ? 0.0f : exp2_hw((l2 - mx) * kLog2e);
      const float sw = w1 + w2;
      const float winv = sw > 0.0f ? 1.0f / sw : 0.0f;
      __bf16 *op = a.o + ((tok0 + qi) * H + hq) * (long long)DV + 4 * hh;
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 x = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(other_o, lane_off + (32 * dt + 8 * i) * 4,
                                                           0, kCoherent));
          const f32x4 p1 = part == 1 ? mine[dt][i] : x;
          const f32x4 p2 = part == 1 ? x : mine[dt][i];
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = (__bf16)((w1 * p1[e] + w2 * p2[e]) * winv);
          *(bf16x4 *)(op + 32 * dt + 8 * i) = out;
        }
      if (a.lse != nullptr && hh == 0) {
        const float lse = sw > 0.0f ? mx + log2f(sw) * kLn2 : -INFINITY;
        a.lse[((long long)b * H + hq) * a.S + qi] = lse;
      }
    }
    return;
  }
  if (row < R) {
    const float inv = l32 > 0.0f ? 1.0f / l32 : 0.0f;  // a row without keys: O = 0, LSE = -inf
    const int hh = lane >> 5;
    __bf16 *op = a.o + ((tok0 + qi) * H + hq) * (long long)DV + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 out = {(__bf16)(st.o[dt][4 * i + 0] * inv), (__bf16)(st.o[dt][4 * i + 1] * inv),
                      (__bf16)(st.o[dt][4 * i + 2] * inv), (__bf16)(st.o[dt][4 * i + 3] * inv)};
        *(bf16x4 *)(op + 32 * dt + 8 * i) = out;
      }
    if (a.lse != nullptr && hh == 0) {
      const float lse = (st.m_ref + log2f(l32)) * kLn2;
      if constexpr (VARLEN) a.lse[(long long)hq * a.cu[a.B] + tok0 + qi] = lse;
      else a.lse[((long long)b * H + hq) * a.S + qi] = lse;
    }
  }
}

// Dynamic LDS of a kernel instance: the ping-pong K/V ring; for the
// single-wave body, rings of two K and three V blocks (the pipelined dense
// body) or the double buffer (varlen, whose tables need the rest).
template <int D, bool VARLEN, bool CAUSAL>
constexpr int lds_bytes() {
  return Cfg<D>::PINGPONG ? KvLayout<D>::BYTES : (VARLEN ? 4 : 5) * Cfg<D>::K_BYTES;
}

// Persistent kernel: each workgroup walks its static LPT list.
// One round of the greedy assignment (fa::greedy_round), with lane i of
// wave 0 standing for worker i of the group and for position r*W + i: the
// ranks of the positions' costs and of the workers' loads come from W
// broadcasts each; the position of each cost rank goes through LDS.  Writes
// this worker's (w) position, or -1, to *mine and updates the loads.
__device__ __forceinline__ void greedy_round_wave(const fa::Sched &s, const fa::SchedTables &t,
                                                  int x, int r, int W, int npos, int w,
                                                  int *gload, int *gpos, int *mine) {
  const int i = threadIdx.x;
  const int c = i < W ? fa::position_cost2(s, t, x, r * W + i, npos) : -2;
  const int ld = i < W ? gload[i] : 0x7fffffff;
  int rc = 0, rl = 0;
  for (int k = 0; k < W; ++k) {
    const int ck = __builtin_amdgcn_readlane(c, k);
    const int lk = __builtin_amdgcn_readlane(ld, k);
    rc += fa::cost_before(ck, k, c, i);
    rl += fa::load_before(lk, k, ld, i);
  }
  if (i < W) gpos[rc] = i;
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  const int gi = i < W ? gpos[rl] : 0;
  const int gc = __shfl(c, gi);
  if (i < W && gc > 0) gload[i] = ld + gc;
  if (i == w) *mine = gc > 0 ? r * W + gi : -1;
}

template <int D, bool CAUSAL, bool VARLEN, int EMU, bool COUNT>
__global__ __launch_bounds__(Cfg<D>::THREADS, Cfg<D>::WAVES_PER_SIMD) void fa_fwd_persistent(Args a) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  char LDS_AS *lds = (char LDS_AS *)lds_raw;
  using C = Cfg<D>;
  fa::Sched s = fa::make_sched(a.B, a.H, a.Hkv, a.S, C::BM, CAUSAL, VARLEN, a.workers,
                               a.cu_k == a.cu, a.nsplit);
  fa::SchedTables t{nullptr, nullptr, nullptr, nullptr, nullptr};
  int *gtab = nullptr;  // greedy rounds: loads [W], positions by cost rank [W], two slots
  if constexpr (VARLEN) {
    int *tab = (int *)(lds_raw + lds_bytes<D, VARLEN, CAUSAL>());
    t.len = tab;
    t.sorted = tab + fa::kMaxVarlenSeqs;
    t.off = tab + 2 * fa::kMaxVarlenSeqs;
    t.key = t.off + fa::kMaxVarlenLevels + 2;  // after the item count below
    fa::tables_phase1(s, a.cu, a.cu_k, t, threadIdx.x, blockDim.x);
    __syncthreads();
    fa::tables_phase2(s, t, threadIdx.x, blockDim.x);
    __syncthreads();
    fa::tables_phase3(s, t, threadIdx.x, blockDim.x);
    __syncthreads();
    int *n_items_sh = t.off + fa::kMaxVarlenLevels + 1;
    if (threadIdx.x == 0) *n_items_sh = fa::tables_phase4(s, t);
    __syncthreads();
    s.n_items = *n_items_sh;
    gtab = t.key + fa::kMaxVarlenSeqs;
  } else if constexpr (CAUSAL) {
    if (s.nsplit > 0) {
      // the virtual levels of the split schedule, by cost rank
      int *tab = (int *)(lds_raw + lds_bytes<D, VARLEN, CAUSAL>());
      t.vl = tab;
      gtab = tab + fa::kMaxSplitLevels;
      fa::split_levels(s, t.vl, threadIdx.x, blockDim.x);
      __syncthreads();
    }
  }
  int x, w, W;
  fa::worker_slot(s, blockIdx.x, a.workers, &x, &w, &W);
  const int npos = fa::group_positions(s);
  if constexpr (CAUSAL) {
    if (fa::greedy_rounds(s, W)) {
      // Greedy rounds: wave 0 works out each round's assignment for the
      // whole group (every worker of the group computes the same one) and
      // publishes this worker's position; two slots, so a round's slot is
      // rewritten only after every wave has passed the next round's barrier.
      int *gload = gtab;                          // [W] accumulated costs
      int *gpos = gload + fa::kGreedyMaxW;        // [W] position index by cost rank
      int *gmine = gpos + fa::kGreedyMaxW;        // [2] this worker's position
      if (threadIdx.x < W) gload[threadIdx.x] = 0;
      __syncthreads();
      for (int r = 0; r * W < npos; ++r) {
        if (threadIdx.x < kWave) greedy_round_wave(s, t, x, r, W, npos, w, gload, gpos, gmine + (r & 1));
        __syncthreads();
        const int p = gmine[r & 1];
        if (p < 0) continue;  // no tile for this worker in this round
        const fa::Tile tl = fa::decode_position(s, t, x, p);
        run_tile<D, CAUSAL, VARLEN, EMU, COUNT>(a, tl.b, tl.h, tl.mb, lds, 0, tl.part);
      }
      return;
    }
  }
  for (int r = 0;; ++r) {
    const int p = fa::snake_position(r, w, W);
    if (p >= npos) break;
    const fa::Tile tl = fa::decode_position(s, t, x, p);
    if (tl.b < 0) continue;  // a level this sequence does not reach
    run_tile<D, CAUSAL, VARLEN, EMU, COUNT>(a, tl.b, tl.h, tl.mb, lds);
  }
}

// One workgroup per tile, natural (b, h, mb) order.
template <int D, bool CAUSAL, bool VARLEN, int EMU, bool COUNT>
__global__ __launch_bounds__(Cfg<D>::THREADS, Cfg<D>::WAVES_PER_SIMD) void fa_fwd_grid(Args a) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  char LDS_AS *lds = (char LDS_AS *)lds_raw;
  using C = Cfg<D>;
  const int nmb = fa::ceil_div(a.S, C::BM);
  const int id = blockIdx.x;
  const int mb = id % nmb;
  const int h = (id / nmb) % a.H;
  const int b = id / (nmb * a.H);
  run_tile<D, CAUSAL, VARLEN, EMU, COUNT>(a, b, h, mb, lds);
}

// Split-KV: one workgroup per (tile, key split), natural order.  PACK: one
// tile per (sequence, K/V head) holding the rows of all its query heads.
template <int D, bool CAUSAL, bool VARLEN, bool PACK>
__global__ __launch_bounds__(Cfg<D>::THREADS, Cfg<D>::WAVES_PER_SIMD) void fa_fwd_split(Args a,
                                                                                        int splits) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  char LDS_AS *lds = (char LDS_AS *)lds_raw;
  using C = Cfg<D>;
  const int nmb = PACK ? 1 : fa::ceil_div(a.S, C::BM);
  const int nh = PACK ? a.Hkv : a.H;
  const int id = blockIdx.x;
  const int split = id % splits;
  const int rest = id / splits;
  const int mb = rest % nmb;
  const int h = (rest / nmb) % nh;
  const int b = rest / (nmb * nh);
  run_tile<D, CAUSAL, VARLEN, 0, false, true, PACK>(a, b, h, mb, lds, split);
}

// Merge the split partials of each (query row, head): with the splits'
// LSE_s and normalised O_s, LSE = ln sum_s e^{LSE_s} and
// O = sum_s e^{LSE_s - LSE} O_s (the merge of partial softmax results by
// their log-sum-exp).  One wavefront per row; a row whose every split was
// empty gets O = 0, LSE = -inf.
template <int DV, bool VARLEN>
__global__ __launch_bounds__(256) void fa_split_combine(Args a, int splits) {
  const long long rows = VARLEN ? (long long)a.cu[a.B] * a.H : (long long)a.B * a.S * a.H;
  const long long r = (long long)blockIdx.x * 4 + threadIdx.x / kWave;  // token*H + h
  const int lane = threadIdx.x % kWave;
  if (r >= rows) return;
  const int H = a.H;
  const long long t = r / H;  // query token
  const int h = (int)(r % H);
  long long li;               // index in the lse layout
  if constexpr (VARLEN) {
    li = (long long)h * a.cu[a.B] + t;
  } else {
    const long long b = t / a.S, i = t % a.S;
    li = (b * H + h) * a.S + i;
  }
  const long long slots = (long long)a.B * a.S * H;
  constexpr int PER = (DV + kWave - 1) / kWave;
  // The partial rows of the first PRE splits are loaded before the weights
  // are known, in flight together with the LSE loads: the merge of a short
  // batch (a decode step) is one memory round trip shorter.  32 covers the
  // split count of a long decode step (measured on one over 32768 keys with
  // 32 splits: 33.3 -> 29.4 us per step against 16).
  constexpr int PRE = 32;
  float pre[PRE][PER];
#pragma unroll
  for (int s = 0; s < PRE; ++s)
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + k * kWave;
      pre[s][k] = (s < splits && d < DV) ? a.ws_o[(s * slots + r) * (long long)DV + d] : 0.0f;
    }
  // Lane s holds the LSE of split s (splits <= 64): the row's maximum and
  // the split weights are wave reductions, not a serial walk over splits.
  const float ls = lane < splits ? a.ws_lse[lane * slots + li] : -INFINITY;
  float m = ls;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
  float lse = -INFINITY;
  if (m != -INFINITY) {
    const float wl = (ls == -INFINITY) ? 0.0f : exp2_hw((ls - m) * kLog2e);
    float wsum = wl;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o);
#pragma unroll
    for (int s = 0; s < PRE; ++s) {
      if (s < splits) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = __builtin_fmaf(w, pre[s][k], acc[k]);
      }
    }
    // the loads of several splits in flight at once
#pragma unroll 16
    for (int s = PRE; s < splits; ++s) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
      const float *op = a.ws_o + (s * slots + r) * (long long)DV;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int d = lane + k * kWave;
        if (d < DV) acc[k] = __builtin_fmaf(w, op[d], acc[k]);
      }
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] *= inv;
    lse = m + log2f(wsum) * kLn2;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = lane + k * kWave;
    if (d < DV) a.o[r * DV + d] = (__bf16)acc[k];
  }
  if (a.lse != nullptr && lane == 0) a.lse[li] = lse;
}

__global__ void exp2_emu_kernel(const float *x, float *y, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = exp2_poly(x[i]);
}

// ---------------------------------------------------------------------------
// The matrix-product ceiling of the D = 128 tile body (a measurement, not
// part of attention).  Every wave of a forward-shaped launch (one
// workgroup of 8 waves per CU) runs, per 64-key block, the forward's own QK
// and PV phases (qk_step, pv_step: 32 products of 32x32x16, with operands
// read from LDS exactly as the forward reads them), or the same product
// sequence with operands held in registers (REG), and nothing else: no
// softmax, copies or barriers.  The operands are pseudo-random (K, V and Q
// uniform on [-2, 2), P on [0, 1)) because the matrix unit's power, and so
// the clock the chip holds, depends on the data: constant operands run
// faster than attention's inputs ever could.  Lane 0 of each wave stamps the
// shader clock (s_memtime) and the constant-rate clock (s_memrealtime)
// around its loop.
// ---------------------------------------------------------------------------
constexpr int kCeilLds = 2 * 64 * 128 * 2;  // one K and one V block of 64 x 128 bf16

// A pseudo-random value in [0, 1) from an integer (a 32-bit integer hash).
__device__ __forceinline__ float hash_unit(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (float)(x >> 8) * (1.0f / 16777216.0f);
}

template <bool REG>
__global__ __launch_bounds__(512, 1) void mfma_ceiling_kernel(int blocks, long long *stamps,
                                                             float *sink) {
  __shared__ __attribute__((aligned(16))) char lds_raw[kCeilLds];
  char LDS_AS *lds = (char LDS_AS *)lds_raw;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const unsigned seed = (unsigned)blockIdx.x * 0x9e3779b9u;
  for (int i = tid; i < kCeilLds / 2; i += blockDim.x)
    ((__bf16 LDS_AS *)lds)[i] = (__bf16)(4.0f * hash_unit(seed + (unsigned)i) - 2.0f);
  LdsAddr<128> la;
  la.init(lane);
  WaveState<128> st;
  bf16x8 kops[8], vops[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const unsigned base = seed + 0x10000u + (unsigned)(tid * 64 + e);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      kops[r][e] = (__bf16)(4.0f * hash_unit(base + 8u * r) - 2.0f);
      vops[r][e] = (__bf16)(4.0f * hash_unit(base + 8u * r + 4096u) - 2.0f);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) st.p[t][e] = (__bf16)hash_unit(base + 8u * t + 8192u);
#pragma unroll
    for (int s = 0; s < 8; ++s) st.qf[s][e] = (__bf16)(4.0f * hash_unit(base + 8u * s + 12288u) - 2.0f);
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[dt][e] = 0.0f;
  __syncthreads();
  const long long t0 = (long long)__builtin_amdgcn_s_memtime();
  const long long r0 = (long long)__builtin_amdgcn_s_memrealtime();
  for (int j = 0; j < blocks; ++j) {
    if constexpr (REG) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.s[kb][e] = 0.0f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        st.s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kops[s], st.qf[s], st.s[0], 0, 0, 0);
        st.s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kops[7 - s], st.qf[s], st.s[1], 0, 0, 0);
      }
    } else {
      qk_step<128>(st, la, lds, lds);
    }
    // the scores are consumed (kept live) without any arithmetic
    asm volatile("" ::"v"(st.s[0]), "v"(st.s[1]));
    if constexpr (REG) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vops[(2 * t + dt) & 7], st.p[t],
                                                             st.o[dt], 0, 0, 0);
    } else {
      pv_step<128>(st, la, lds + kCeilLds / 2);
    }
  }
  const long long t1 = (long long)__builtin_amdgcn_s_memtime();
  const long long r1 = (long long)__builtin_amdgcn_s_memrealtime();
  float acc = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc += st.o[dt][e];
  sink[(size_t)blockIdx.x * blockDim.x + tid] = acc;
  if (lane == 0) {
    long long *w = stamps + ((size_t)blockIdx.x * (blockDim.x / kWave) + wave) * 4;
    w[0] = t0;
    w[1] = t1;
    w[2] = r0;
    w[3] = r1;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// Supported (q/k, v/o) head-dimension pairs; the kernel instance is named by
// the q/k dimension.
bool supported_dims(int D, int Dv) {
  return (D == Dv && (D == 64 || D == 128 || D == 256)) || (D == 192 && Dv == 128);
}

int validate(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
             int Hkv, int S, int Sk, int D, int Dv, float scale, int causal, const int *cu_q,
             const int *cu_k, const fa_tuning *t) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S <= 0 || Sk <= 0 || D <= 0 || Dv <= 0) return FA_ERR_INVALID_ARG;
  if ((cu_q == nullptr) != (cu_k == nullptr)) return FA_ERR_INVALID_ARG;
  if (Hkv <= 0 || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (t) {
    // p = exp2(c*s - m_ref) reaches 2^tau before a rescale: bounded so that
    // the fp32 row sums and O accumulators stay far from overflow.
    if (!(t->tau >= 0.0f && t->tau <= kMaxTau)) return FA_ERR_INVALID_ARG;
    if (t->exp2_emu != 0 && t->exp2_emu != 4 && t->exp2_emu != 8) return FA_ERR_INVALID_ARG;
    if (t->schedule != 0 && t->schedule != 1) return FA_ERR_INVALID_ARG;
    if (t->split_levels < -1) return FA_ERR_INVALID_ARG;
  }
  if (!supported_dims(D, Dv)) return FA_ERR_UNSUPPORTED;
  // sizes must fit the 32-bit index arithmetic used for rows and tiles
  const long long Smax = S > Sk ? S : Sk;
  if ((long long)B * Smax > (1LL << 31) - 1 || Smax * H > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

template <int D, bool CAUSAL, bool VARLEN, int EMU, bool COUNT>
int launch_variant(const Args &a0, int schedule, int cus, hipStream_t stream) {
  using C = Cfg<D>;
  Args a = a0;
  size_t lds = lds_bytes<D, VARLEN, CAUSAL>();
  const int nmb = fa::ceil_div(a.S, C::BM);
  bool persistent = (schedule == 0);
  if (VARLEN && (a.B > fa::kMaxVarlenSeqs || nmb > fa::kMaxVarlenLevels)) persistent = false;
  if (persistent) {
    a.workers = cus * C::OCC;
    // varlen tables, then the greedy rounds' loads, ranks and two slots
    if (VARLEN)
      lds += sizeof(int) * (3 * fa::kMaxVarlenSeqs + fa::kMaxVarlenLevels + 2 +
                            2 * fa::kGreedyMaxW + 2);
    // split levels: their table, then the greedy rounds' arrays
    if (!VARLEN && CAUSAL && a.nsplit > 0)
      lds += sizeof(int) * (fa::kMaxSplitLevels + 2 * fa::kGreedyMaxW + 2);
    auto kern = fa_fwd_persistent<D, CAUSAL, VARLEN, EMU, COUNT>;
    if (!allow_lds(kern, lds)) return FA_ERR_HIP;
    FA_LOG_LAUNCH("fa_fwd_persistent<D=%d causal=%d varlen=%d exp2_emu=%d counters=%d>: %d "
                  "workgroups x %d threads, %zu B LDS; B=%d H=%d H_kv=%d S_q=%d S_k=%d, "
                  "%d-row tiles, up to %lld tiles, %d split levels, tau=%g",
                  D, (int)CAUSAL, (int)VARLEN, EMU, (int)COUNT, a.workers, C::THREADS, lds, a.B,
                  a.H, a.Hkv, a.S, a.Sk, C::BM, (long long)a.B * a.H * nmb, a.nsplit,
                  (double)a.tau);
    hipLaunchKernelGGL(kern, dim3(a.workers), dim3(C::THREADS), lds, stream, a);
  } else {
    const long long grid = (long long)a.B * a.H * nmb;
    if (grid > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    auto kern = fa_fwd_grid<D, CAUSAL, VARLEN, EMU, COUNT>;
    if (!allow_lds(kern, lds)) return FA_ERR_HIP;
    FA_LOG_LAUNCH("fa_fwd_grid<D=%d causal=%d varlen=%d exp2_emu=%d counters=%d>: %lld "
                  "workgroups x %d threads, %zu B LDS; B=%d H=%d H_kv=%d S_q=%d S_k=%d, "
                  "%d-row tiles, tau=%g",
                  D, (int)CAUSAL, (int)VARLEN, EMU, (int)COUNT, grid, C::THREADS, lds, a.B, a.H,
                  a.Hkv, a.S, a.Sk, C::BM, (double)a.tau);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), lds, stream, a);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int bm_for(int D);
bool split_packs(int H, int Hkv, int S_q, int BM);

template <int D, bool CAUSAL, bool VARLEN>
int launch_split(const Args &a, int splits, hipStream_t stream) {
  using C = Cfg<D>;
  const bool pack = split_packs(a.H, a.Hkv, a.S, C::BM);
  const long long tiles =
      pack ? (long long)a.B * a.Hkv : (long long)a.B * a.H * fa::ceil_div(a.S, C::BM);
  const long long grid = tiles * splits;
  const long long rows = (long long)a.B * a.S * a.H;  // combine: 4 rows per workgroup
  if (grid > 0x7fffffffLL || (rows + 3) / 4 > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  auto kern = pack ? fa_fwd_split<D, CAUSAL, VARLEN, true> : fa_fwd_split<D, CAUSAL, VARLEN, false>;
  const size_t lds = lds_bytes<D, VARLEN, CAUSAL>();
  if (!allow_lds(kern, lds)) return FA_ERR_HIP;
  FA_LOG_LAUNCH("fa_fwd_split<D=%d causal=%d varlen=%d packed=%d>: %lld workgroups x %d threads, "
                "%zu B LDS; %lld tiles x %d splits of %d key blocks; B=%d H=%d H_kv=%d S_q=%d "
                "S_k=%d; then fa_split_combine: %lld workgroups x 256 threads",
                D, (int)CAUSAL, (int)VARLEN, (int)pack, grid, C::THREADS, lds, tiles, splits,
                a.kbps, a.B, a.H, a.Hkv, a.S, a.Sk, (rows + 3) / 4);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), lds, stream, a, splits);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  hipLaunchKernelGGL((fa_split_combine<C::DV, VARLEN>), dim3((unsigned)((rows + 3) / 4)), dim3(256),
                     0, stream, a, splits);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int D>
int dispatch_split(const Args &a, bool causal, bool varlen, int splits, hipStream_t st) {
  if (causal) return varlen ? launch_split<D, true, true>(a, splits, st) : launch_split<D, true, false>(a, splits, st);
  return varlen ? launch_split<D, false, true>(a, splits, st) : launch_split<D, false, false>(a, splits, st);
}

// Split count for a key range: enough (tile, split) pairs for one per CU
// (one workgroup fills a CU; measured on a one-row decode step over 32768
// keys, 32 query tiles: 8 splits run 7x faster than none, 16 or more lose
// again to the partial writes and the merge), at least two 64-key blocks per
// split, at most kMaxSplits.  Batches that already have a tile per CU get 1.
constexpr int kMaxSplits = 64;  // fa_split_combine holds one split per lane
static_assert(kMaxSplits <= kWave, "one split per lane in the merge");
// Split-KV packs the query heads of a K/V group into one tile when all their
// rows (S_q per head) fit one tile.
bool split_packs(int H, int Hkv, int S_q, int BM) {
  return H > Hkv && (long long)S_q * (H / Hkv) <= BM;
}

int auto_splits(int B, int H, int Hkv, int S_q, int S_k, int D, int cus) {
  const int BM = bm_for(D);
  const long long tiles = split_packs(H, Hkv, S_q, BM) ? (long long)B * Hkv
                                                       : (long long)B * H * fa::ceil_div(S_q, BM);
  const int kblocks = fa::ceil_div(S_k, kBN);
  long long want = ((long long)cus + tiles - 1) / tiles;
  if (want > kblocks / 2) want = kblocks / 2;
  if (want > kMaxSplits) want = kMaxSplits;
  return want < 1 ? 1 : (int)want;
}

// (splits, key blocks per split) actually used for a requested count.
void split_plan(int S_k, int requested, int *splits, int *kbps) {
  const int kblocks = fa::ceil_div(S_k, kBN);
  int n = requested < 1 ? 1 : (requested > kblocks ? kblocks : requested);
  const int per = fa::ceil_div(kblocks, n);
  *kbps = per;
  *splits = fa::ceil_div(kblocks, per);
}

template <int D, bool CAUSAL, bool VARLEN>
int dispatch_emu(const Args &a, const fa_tuning &t, int cus, hipStream_t st) {
  if (t.counters) return launch_variant<D, CAUSAL, VARLEN, 0, true>(a, t.schedule, cus, st);
  switch (t.exp2_emu) {
    case 8: return launch_variant<D, CAUSAL, VARLEN, 8, false>(a, t.schedule, cus, st);
    case 4: return launch_variant<D, CAUSAL, VARLEN, 4, false>(a, t.schedule, cus, st);
    default: return launch_variant<D, CAUSAL, VARLEN, 0, false>(a, t.schedule, cus, st);
  }
}

template <int D>
int dispatch_d(const Args &a, bool causal, bool varlen, const fa_tuning &t, int cus,
               hipStream_t st) {
  if (causal) {
    return varlen ? dispatch_emu<D, true, true>(a, t, cus, st) : dispatch_emu<D, true, false>(a, t, cus, st);
  }
  return varlen ? dispatch_emu<D, false, true>(a, t, cus, st) : dispatch_emu<D, false, false>(a, t, cus, st);
}

template <int D>
constexpr int bm_of() { return Cfg<D>::BM; }

int bm_for(int D) {
  switch (D) {
    case 64: return bm_of<64>();
    case 128: return bm_of<128>();
    case 192: return bm_of<192>();
    default: return bm_of<256>();
  }
}

// Waves per workgroup of the forward instance for D.
int nw_for(int D) {
  switch (D) {
    case 64: return Cfg<64>::NW;
    case 128: return Cfg<128>::NW;
    case 192: return Cfg<192>::NW;
    default: return Cfg<256>::NW;
  }
}

// ---- dense causal split levels: the plan and the workspace ----

// Makespan, in doubled cost units (fa::tile_cost2), of the busiest worker of
// group 0 under schedule s (every group of a dense batch holds the same
// costs): greedy rounds with split levels, the snake order without.
long long split_makespan(const fa::Sched &s, int workers) {
  int vl[fa::kMaxSplitLevels];
  fa::SchedTables t{nullptr, nullptr, nullptr, nullptr, vl};
  if (s.nsplit > 0) fa::split_levels(s, vl, 0, 1);
  int x0, w0, W;
  fa::worker_slot(s, 0, workers, &x0, &w0, &W);
  const int npos = fa::group_positions(s);
  if (fa::greedy_rounds(s, W)) {
    int load[fa::kGreedyMaxW] = {}, take[fa::kGreedyMaxW];
    for (int r = 0; r * W < npos; ++r) fa::greedy_round(s, t, 0, r, W, npos, load, take);
    return *std::max_element(load, load + W);
  }
  long long worst = 0;
  for (int w = 0; w < W; ++w) {
    long long load = 0;
    for (int r = 0;; ++r) {
      const int p = fa::snake_position(r, w, W);
      if (p >= npos) break;
      load += fa::tile_cost2(s, t, fa::decode_position(s, t, 0, p));
    }
    worst = load > worst ? load : worst;
  }
  return worst;
}

// Split levels for a dense causal self-attention launch of `workers`
// workgroups: `requested` clamped to what the schedule can hold, or, with
// requested < 0, the count the makespan model above finds best, when the
// unsplit batch leaves at least half of the workers without a tile and the
// model shortens the busiest worker's load by at least 5%.  Measured (D =
// 128, the best count against none): B=1, H=8, S=3000 -19%; B=1, H=16,
// S=2048 -10%.  Batches that fill the workers gain too little for the
// exchange of partial rows (B=2, H=16, S=2048: -5% with one level, slower
// with more), and are left whole.
int plan_nsplit(int B, int H, int S, int BM, int workers, int requested) {
  const fa::Sched s0 = fa::make_sched(B, H, H, S, BM, 1, 0, workers);
  int maxs = fa::kMaxSplitLevels - s0.nmb_max;
  if (maxs > s0.nmb_max) maxs = s0.nmb_max;
  if (maxs <= 0 || requested == 0) return 0;
  if (requested > 0) return requested < maxs ? requested : maxs;
  static std::mutex mu;
  static std::map<std::array<int, 4>, int> memo;
  const std::array<int, 4> key{B, H, S, BM * 4096 + workers};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = memo.find(key);
    if (it != memo.end()) return it->second;
  }
  if ((long long)B * H * s0.nmb_max * 2 > workers) return 0;
  int x0, w0, W;
  fa::worker_slot(s0, 0, workers, &x0, &w0, &W);
  long long total = 0;
  for (int mb = 0; mb < s0.nmb_max; ++mb) total += fa::split_cost2(s0, mb, 0);
  total *= (long long)B * s0.hpg;
  const long long base = split_makespan(s0, workers);
  int best_n = 0;
  if (base * 20 > total / W * 21) {  // the busiest worker is >5% above the mean
    long long best = base;
    for (int n = 1; n <= maxs; ++n) {
      const long long m = split_makespan(fa::make_sched(B, H, H, S, BM, 1, 0, workers, 1, n),
                                         workers);
      if (m < best) {
        best = m;
        best_n = n;
      }
    }
    if (best * 20 > base * 19) best_n = 0;
  }
  std::lock_guard<std::mutex> lock(mu);
  memo[key] = best_n;
  return best_n;
}

// Bytes of a split launch's arrival counters and of its partial rows (O and
// LSE of both parts of every split tile).
size_t split_counter_bytes(int B, int H, int nsplit, int NW) {
  return (size_t)B * H * nsplit * NW * sizeof(int);
}
size_t split_partial_bytes(int B, int H, int nsplit, int BM, int DV) {
  return (size_t)B * H * nsplit * 2 * BM * (DV + 1) * sizeof(float);
}
constexpr size_t kSplitPartialMax = (size_t)512 << 20;  // larger partials: no split

// Workspace of split launches, one per device and stream: launches on one
// stream run in order and so never share it, launches on different streams
// get their own.  The counters are zeroed when allocated (on the stream)
// and every launch leaves them zero.  A buffer grows by waiting for its
// stream and replacing it; it is kept until the process ends.  nullptr when
// it cannot be had (an allocation failure, or a stream being captured).
struct SplitBuf {
  void *ptr = nullptr;
  size_t bytes = 0;
};
bool split_buffer(std::map<std::pair<int, hipStream_t>, SplitBuf> &bufs, int dev, hipStream_t st,
                  size_t bytes, bool zero, void **out) {
  SplitBuf &b = bufs[{dev, st}];
  if (b.bytes >= bytes) {
    *out = b.ptr;
    return true;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
  if (b.ptr) {
    if (hipStreamSynchronize(st) != hipSuccess) return false;
    (void)hipFree(b.ptr);
    b.ptr = nullptr;
    b.bytes = 0;
  }
  void *p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) return false;
  if (zero && hipMemsetAsync(p, 0, bytes, st) != hipSuccess) {
    (void)hipFree(p);
    return false;
  }
  b.ptr = p;
  b.bytes = bytes;
  *out = p;
  return true;
}
bool split_workspace(hipStream_t st, size_t cnt_bytes, size_t part_bytes, int **cnt,
                     float **part) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, SplitBuf> counters, partials;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  void *c = nullptr, *p = nullptr;
  if (!split_buffer(counters, dev, st, cnt_bytes, true, &c)) return false;
  if (!split_buffer(partials, dev, st, part_bytes, false, &p)) return false;
  *cnt = (int *)c;
  *part = (float *)p;
  return true;
}

// The partial results of fa_fwd_splitkv_noalloc: a fixed array in each
// device's memory, so that the call allocates nothing.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// symbol); it uses the device address scratch_address() looks up once per
// device.
__device__ __align__(256) float scratch[FA_SPLITKV_SCRATCH_BYTES / sizeof(float)];

struct ScratchSlot {
  std::once_flag once;
  void *ptr = nullptr;
};
ScratchSlot g_scratch[64];

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept per device.
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FA_ERR_NO_DEVICE;
  ScratchSlot &slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) slot.ptr = p;
  });
  if (!slot.ptr) return FA_ERR_HIP;
  *out = slot.ptr;
  return FA_OK;
}

int splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
            int H_kv, int S_q, int S_k, int D, int D_v, float scale, int causal,
            const int *cu_seqlens_q, const int *cu_seqlens_k, int num_splits, void *workspace,
            size_t workspace_bytes, void *stream, bool fixed_scratch);

}  // namespace

extern "C" {

fa_tuning fa_tuning_default(void) {
  fa_tuning t;
  t.tau = 8.0f;
  t.exp2_emu = 0;
  t.schedule = 0;
  t.counters = nullptr;
  t.split_levels = -1;
  return t;
}

int fa_fwd_general(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                   int H, int H_kv, int S_q, int S_k, int D, int D_v, float scale, int causal,
                   const int *cu_seqlens_q, const int *cu_seqlens_k, void *stream,
                   const fa_tuning *tuning) {
  const fa_tuning t = tuning ? *tuning : fa_tuning_default();
  int rc = validate(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, D_v, scale, causal, cu_seqlens_q,
                    cu_seqlens_k, &t);
  if (rc != FA_OK) return rc;
  DeviceInfo *dev = nullptr;
  rc = current_device(&dev);
  if (rc != FA_OK) return rc;
  Args a;
  a.q = (const __bf16 *)q;
  a.k = (const __bf16 *)k;
  a.v = (const __bf16 *)v;
  a.o = (__bf16 *)o;
  a.lse = lse;
  a.cu = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.B = B;
  a.H = H;
  a.Hkv = H_kv;
  a.S = S_q;
  a.Sk = S_k;
  a.c = scale * kLog2e;
  a.tau = t.tau;
  a.bound = exp2f(t.tau);
  a.counters = t.counters;
  a.workers = 0;
  a.ws_o = a.ws_lse = nullptr;
  a.kbps = 0;
  a.nsplit = 0;
  a.hs_cnt = nullptr;
  hipStream_t st = (hipStream_t)stream;
  const bool varlen = cu_seqlens_q != nullptr;
  // (not for D = 256, whose pipelined body takes all 160 KiB of LDS: the split
  // schedule's tables would not fit beside it)
  if (causal && !varlen && S_q == S_k && t.schedule == 0 && t.split_levels != 0 && D != 256) {
    const int BM = bm_for(D), NW = nw_for(D);
    const int n = plan_nsplit(B, H, S_q, BM, dev->cus, t.split_levels);
    int *cnt = nullptr;
    float *part = nullptr;
    if (n > 0 && split_partial_bytes(B, H, n, BM, D_v) <= kSplitPartialMax &&
        split_workspace(st, split_counter_bytes(B, H, n, NW), split_partial_bytes(B, H, n, BM, D_v),
                        &cnt, &part)) {
      a.nsplit = n;
      a.hs_cnt = cnt;
      a.ws_o = part;
      a.ws_lse = part + (size_t)B * H * n * 2 * BM * D_v;
    }
  }
  switch (D) {
    case 64: return dispatch_d<64>(a, causal, varlen, t, dev->cus, st);
    case 128: return dispatch_d<128>(a, causal, varlen, t, dev->cus, st);
    case 192: return dispatch_d<192>(a, causal, varlen, t, dev->cus, st);
    default: return dispatch_d<256>(a, causal, varlen, t, dev->cus, st);
  }
}

size_t fa_splitkv_workspace_size(int B, int H, int S_q, int S_k, int D_v, int num_splits) {
  if (B <= 0 || H <= 0 || S_q <= 0 || S_k <= 0 || D_v <= 0 || num_splits < 0) return 0;
  int splits, kbps;
  split_plan(S_k, num_splits, &splits, &kbps);
  if (splits <= 1) return 0;
  return (size_t)splits * (size_t)B * (size_t)S_q * (size_t)H * ((size_t)D_v + 1) * sizeof(float);
}

int fa_splitkv_auto_splits(int B, int H, int S_q, int S_k, int D, int *splits_out) {
  return fa_splitkv_auto_splits_gqa(B, H, H, S_q, S_k, D, splits_out);
}

int fa_splitkv_auto_splits_gqa(int B, int H, int H_kv, int S_q, int S_k, int D, int *splits_out) {
  if (!splits_out || B <= 0 || H <= 0 || S_q <= 0 || S_k <= 0) return FA_ERR_INVALID_ARG;
  if (H_kv <= 0 || H % H_kv != 0) return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 192 && D != 256) return FA_ERR_UNSUPPORTED;
  DeviceInfo *dev = nullptr;
  const int rc = current_device(&dev);
  if (rc != FA_OK) return rc;
  int splits, kbps;
  split_plan(S_k, auto_splits(B, H, H_kv, S_q, S_k, D, dev->cus), &splits, &kbps);
  *splits_out = splits;
  return FA_OK;
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                   int H, int H_kv, int S_q, int S_k, int D, int D_v, float scale, int causal,
                   const int *cu_seqlens_q, const int *cu_seqlens_k, int num_splits,
                   void *workspace, size_t workspace_bytes, void *stream) {
  return splitkv(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, D_v, scale, causal, cu_seqlens_q,
                 cu_seqlens_k, num_splits, workspace, workspace_bytes, stream, false);
}

int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int H_kv, int S_q, int S_k, int D, int D_v,
                           float scale, int causal, const int *cu_seqlens_q,
                           const int *cu_seqlens_k, int num_splits, void *stream) {
  return splitkv(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, D_v, scale, causal, cu_seqlens_q,
                 cu_seqlens_k, num_splits, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {

int splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
            int H_kv, int S_q, int S_k, int D, int D_v, float scale, int causal,
            const int *cu_seqlens_q, const int *cu_seqlens_k, int num_splits, void *workspace,
            size_t workspace_bytes, void *stream, bool fixed_scratch) {
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  int rc = validate(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, D_v, scale, causal, cu_seqlens_q,
                    cu_seqlens_k, nullptr);
  if (rc != FA_OK) return rc;
  int splits, kbps;
  split_plan(S_k, num_splits, &splits, &kbps);
  if (splits <= 1)  // one split: the plain path, no workspace
    return fa_fwd_general(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, D_v, scale, causal,
                          cu_seqlens_q, cu_seqlens_k, stream, nullptr);
  const size_t need = fa_splitkv_workspace_size(B, H, S_q, S_k, D_v, num_splits);
  DeviceInfo *dev = nullptr;
  if (fixed_scratch) {
    if (need > FA_SPLITKV_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
    rc = current_device(&dev);
    if (rc != FA_OK) return rc;
    rc = scratch_address(&workspace);
    if (rc != FA_OK) return rc;
    workspace_bytes = FA_SPLITKV_SCRATCH_BYTES;
  } else {
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return FA_ERR_INVALID_ARG;
    rc = current_device(&dev);
    if (rc != FA_OK) return rc;
  }
  Args a;
  a.q = (const __bf16 *)q;
  a.k = (const __bf16 *)k;
  a.v = (const __bf16 *)v;
  a.o = (__bf16 *)o;
  a.lse = lse;
  a.cu = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.B = B;
  a.H = H;
  a.Hkv = H_kv;
  a.S = S_q;
  a.Sk = S_k;
  a.c = scale * kLog2e;
  a.tau = fa_tuning_default().tau;
  a.bound = exp2f(a.tau);
  a.counters = nullptr;
  a.workers = 0;
  const size_t slots = (size_t)B * S_q * H;
  a.ws_o = (float *)workspace;
  a.ws_lse = a.ws_o + (size_t)splits * slots * D_v;
  a.kbps = kbps;
  a.nsplit = 0;
  a.hs_cnt = nullptr;
  hipStream_t st = (hipStream_t)stream;
  const bool varlen = cu_seqlens_q != nullptr;
  switch (D) {
    case 64: return dispatch_split<64>(a, causal, varlen, splits, st);
    case 128: return dispatch_split<128>(a, causal, varlen, splits, st);
    case 192: return dispatch_split<192>(a, causal, varlen, splits, st);
    default: return dispatch_split<256>(a, causal, varlen, splits, st);
  }
}

}  // namespace

extern "C" {

int fa_fwd_hd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int H_kv, int S, int D, int D_v, float scale, int causal, const int *cu_seqlens,
              void *stream, const fa_tuning *tuning) {
  return fa_fwd_general(q, k, v, o, lse, B, H, H_kv, S, S, D, D_v, scale, causal, cu_seqlens,
                        cu_seqlens, stream, tuning);
}

int fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
               int H_kv, int S, int D, float scale, int causal, const int *cu_seqlens,
               void *stream, const fa_tuning *tuning) {
  return fa_fwd_hd(q, k, v, o, lse, B, H, H_kv, S, D, D, scale, causal, cu_seqlens, stream,
                   tuning);
}

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int S, int D, float scale, int causal, const int *cu_seqlens, void *stream,
              const fa_tuning *tuning) {
  return fa_fwd_gqa(q, k, v, o, lse, B, H, H, S, D, scale, causal, cu_seqlens, stream, tuning);
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int S,
           int D, float scale, int causal, const int *cu_seqlens, void *stream) {
  return fa_fwd_gqa(q, k, v, o, lse, B, H, H, S, D, scale, causal, cu_seqlens, stream, nullptr);
}

int fa_exp2_emu(const float *x, float *y, long long n, void *stream) {
  if (n < 0) return FA_ERR_INVALID_ARG;
  if (n == 0) return FA_OK;
  if (!x || !y) return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 3) || (reinterpret_cast<uintptr_t>(y) & 3)) return FA_ERR_INVALID_ARG;
  DeviceInfo *dev = nullptr;
  int rc = current_device(&dev);
  if (rc != FA_OK) return rc;
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(exp2_emu_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, x, y, n);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_mfma_ceiling(int mode, int blocks, int reps, fa_mfma_rate *out) {
  if ((mode != 0 && mode != 1) || blocks < 1 || blocks > (1 << 20) || reps < 1 || reps > 1000 ||
      !out)
    return FA_ERR_INVALID_ARG;
  DeviceInfo *dev = nullptr;
  int rc = current_device(&dev);
  if (rc != FA_OK) return rc;
  int dev_id = 0, wall_khz = 0;
  if (hipGetDevice(&dev_id) != hipSuccess ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev_id) != hipSuccess ||
      wall_khz <= 0)
    return FA_ERR_HIP;
  const int workers = dev->cus;
  const int waves = workers * 8;
  long long *stamps = nullptr;
  float *sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  std::vector<double> ms(reps), mhz(reps), cyc(reps);
  std::vector<long long> host((size_t)waves * 4);
  rc = FA_ERR_HIP;
  if (hipMalloc((void **)&stamps, host.size() * sizeof(long long)) != hipSuccess) goto done;
  if (hipMalloc((void **)&sink, (size_t)workers * 512 * sizeof(float)) != hipSuccess) goto done;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) goto done;
  for (int r = 0; r < reps; ++r) {
    (void)hipEventRecord(e0, nullptr);
    if (mode == 0)
      hipLaunchKernelGGL(mfma_ceiling_kernel<true>, dim3(workers), dim3(512), 0, nullptr, blocks,
                         stamps, sink);
    else
      hipLaunchKernelGGL(mfma_ceiling_kernel<false>, dim3(workers), dim3(512), 0, nullptr, blocks,
                         stamps, sink);
    if (hipGetLastError() != hipSuccess) goto done;
    (void)hipEventRecord(e1, nullptr);
    if (hipEventSynchronize(e1) != hipSuccess) goto done;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, e0, e1) != hipSuccess) goto done;
    if (hipMemcpy(host.data(), stamps, host.size() * sizeof(long long), hipMemcpyDeviceToHost) !=
        hipSuccess)
      goto done;
    double sclk = 0.0, real = 0.0;
    for (int w = 0; w < waves; ++w) {
      sclk += (double)(host[(size_t)w * 4 + 1] - host[(size_t)w * 4 + 0]);
      real += (double)(host[(size_t)w * 4 + 3] - host[(size_t)w * 4 + 2]);
    }
    ms[r] = t;
    // the shader clock over the waves' loops (s_memtime ticks per second of
    // the constant-rate clock), and the launch's cycles per product on one
    // SIMD's matrix unit at that clock (the two waves of a SIMD need not
    // overlap for their whole loops, so per-wave spans would undercount)
    mhz[r] = real > 0.0 ? sclk / (real / (wall_khz * 1e3)) / 1e6 : 0.0;
    cyc[r] = (double)t * 1e-3 * mhz[r] * 1e6 / ((double)waves * blocks * 32.0 / (workers * 4.0));
  }
  {
    // the median launch (by time) and its clock
    std::vector<int> order(reps);
    for (int r = 0; r < reps; ++r) order[r] = r;
    std::sort(order.begin(), order.end(), [&](int x, int y) { return ms[x] < ms[y]; });
    const int m = order[reps / 2];
    const double flops = (double)waves * blocks * 32.0 * (2.0 * 32 * 32 * 16);
    out->workers = workers;
    out->products = (long long)waves * blocks * 32;
    out->ms = ms[m];
    out->tflops = flops / (ms[m] * 1e-3) / 1e12;
    out->best_tflops = flops / (ms[order[0]] * 1e-3) / 1e12;
    out->clock_mhz = mhz[m];
    out->cycles_per_product = cyc[m];
  }
  rc = FA_OK;
done:
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (stamps) (void)hipFree(stamps);
  if (sink) (void)hipFree(sink);
  return rc;
}

int fa_schedule(int B, int H, int S, int D, int causal, const int *cu_seqlens, int workers,
                int *tiles, int max_rounds, int *rounds_out, int *bm_out) {
  return fa_schedule_gqa(B, H, H, S, D, causal, cu_seqlens, workers, tiles, max_rounds,
                         rounds_out, bm_out);
}

int fa_schedule_gqa(int B, int H, int H_kv, int S, int D, int causal, const int *cu_seqlens,
                    int workers, int *tiles, int max_rounds, int *rounds_out, int *bm_out) {
  return fa_schedule_general(B, H, H_kv, S, D, causal, cu_seqlens, cu_seqlens, workers, tiles,
                             max_rounds, rounds_out, bm_out);
}

int fa_schedule_general(int B, int H, int H_kv, int S, int D, int causal, const int *cu_seqlens,
                        const int *cu_seqlens_k, int workers, int *tiles, int max_rounds,
                        int *rounds_out, int *bm_out) {
  if (B <= 0 || H <= 0 || S <= 0 || workers <= 0 || !tiles || max_rounds <= 0) return FA_ERR_INVALID_ARG;
  if (H_kv <= 0 || H % H_kv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if ((cu_seqlens == nullptr) != (cu_seqlens_k == nullptr)) return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 192 && D != 256) return FA_ERR_UNSUPPORTED;
  const int BM = bm_for(D);
  const bool varlen = cu_seqlens != nullptr;
  fa::Sched s = fa::make_sched(B, H, H_kv, S, BM, causal, varlen, workers,
                               cu_seqlens_k == cu_seqlens);
  if (varlen && (B > fa::kMaxVarlenSeqs || s.nmb_max > fa::kMaxVarlenLevels)) return FA_ERR_UNSUPPORTED;
  static thread_local int len[fa::kMaxVarlenSeqs], sorted[fa::kMaxVarlenSeqs],
      off[fa::kMaxVarlenLevels + fa::kMaxVarlenSeqs + 1], key[fa::kMaxVarlenSeqs];
  fa::SchedTables t{len, sorted, off, key, nullptr};
  if (varlen) {
    fa::tables_phase1(s, cu_seqlens, cu_seqlens_k, t, 0, 1);
    fa::tables_phase2(s, t, 0, 1);
    fa::tables_phase3(s, t, 0, 1);
    s.n_items = fa::tables_phase4(s, t);
  }
  const int npos = fa::group_positions(s);
  int rounds = 0;
  int x0, w0, W;
  fa::worker_slot(s, 0, workers, &x0, &w0, &W);
  std::vector<int> count(workers, 0);
  auto put = [&](int wk, int p, int x) {
    const fa::Tile tl = fa::decode_position(s, t, x, p);
    if (tl.b < 0) return true;  // an idle position
    if (count[wk] == max_rounds) return false;  // the list must fit max_rounds
    tiles[(long long)wk * max_rounds + count[wk]++] = (tl.b * H + tl.h) * s.nmb_max + tl.mb;
    return true;
  };
  if (fa::greedy_rounds(s, W)) {
    // every group's rounds, in the order each worker runs them
    for (int x = 0; x < s.groups; ++x) {
      int load[fa::kGreedyMaxW] = {}, take[fa::kGreedyMaxW];
      for (int r = 0; r * W < npos; ++r) {
        fa::greedy_round(s, t, x, r, W, npos, load, take);
        for (int w = 0; w < W; ++w)
          if (take[w] >= 0 && !put(w * s.groups + x, take[w], x)) return FA_ERR_INVALID_ARG;
      }
    }
  } else {
    for (int wk = 0; wk < workers; ++wk) {
      int x, w;
      fa::worker_slot(s, wk, workers, &x, &w, &W);
      for (int r = 0;; ++r) {
        const int p = fa::snake_position(r, w, W);
        if (p >= npos) break;
        if (!put(wk, p, x)) return FA_ERR_INVALID_ARG;
      }
    }
  }
  for (int wk = 0; wk < workers; ++wk) {
    if (count[wk] > rounds) rounds = count[wk];
    for (int r = count[wk]; r < max_rounds; ++r) tiles[(long long)wk * max_rounds + r] = -1;
  }
  if (rounds_out) *rounds_out = rounds;
  if (bm_out) *bm_out = BM;
  return FA_OK;
}

int fa_device_info(int *cus_out, int *clock_khz_out) {
  if (!cus_out || !clock_khz_out) return FA_ERR_INVALID_ARG;
  DeviceInfo *dev = nullptr;
  const int rc = current_device(&dev);
  if (rc != FA_OK) return rc;
  *cus_out = dev->cus;
  *clock_khz_out = dev->clock_khz;
  return FA_OK;
}

int fa_num_workers(int D, int *workers_out) {
  if (!workers_out) return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 192 && D != 256) return FA_ERR_UNSUPPORTED;
  DeviceInfo *dev = nullptr;
  int rc = current_device(&dev);
  if (rc != FA_OK) return rc;
  *workers_out = dev->cus * (D == 256 ? Cfg<256>::OCC : Cfg<128>::OCC);  // OCC = 1 for every D
  return FA_OK;
}

const char *fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported configuration";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
    case FA_ERR_NO_DEVICE: return "FA_ERR_NO_DEVICE: no gfx950 device is current";
    case FA_ERR_TOO_LARGE: return "FA_ERR_TOO_LARGE: sizes exceed the fixed scratch buffer";
    default: return "unknown fa_status";
  }
}

int fa_split_plan(int B, int H, int S, int D, int workers, int requested, int *nsplit_out) {
  if (!nsplit_out || B <= 0 || H <= 0 || S <= 0 || workers <= 0 || requested < -1)
    return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 192 && D != 256) return FA_ERR_UNSUPPORTED;
  *nsplit_out = D == 256 ? 0 : plan_nsplit(B, H, S, bm_for(D), workers, requested);
  return FA_OK;
}

int fa_schedule_split(int B, int H, int S, int D, int nsplit, int workers, int *tiles,
                      int max_rounds, int *rounds_out, int *bm_out) {
  if (B <= 0 || H <= 0 || S <= 0 || workers <= 0 || !tiles || max_rounds <= 0 || nsplit < 0)
    return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 192 && D != 256) return FA_ERR_UNSUPPORTED;
  const int BM = bm_for(D);
  if ((D == 256 && nsplit > 0) || plan_nsplit(B, H, S, BM, workers, nsplit) != nsplit)
    return FA_ERR_INVALID_ARG;
  const fa::Sched s = fa::make_sched(B, H, H, S, BM, 1, 0, workers, 1, nsplit);
  int vl[fa::kMaxSplitLevels];
  fa::SchedTables t{nullptr, nullptr, nullptr, nullptr, vl};
  if (s.nsplit > 0) fa::split_levels(s, vl, 0, 1);
  const int npos = fa::group_positions(s);
  int x0, w0, W;
  fa::worker_slot(s, 0, workers, &x0, &w0, &W);
  std::vector<int> count(workers, 0);
  auto put = [&](int wk, int p, int x) {
    const fa::Tile tl = fa::decode_position(s, t, x, p);
    if (count[wk] == max_rounds) return false;
    tiles[(long long)wk * max_rounds + count[wk]++] =
        ((tl.b * H + tl.h) * s.nmb_max + tl.mb) * 3 + tl.part;
    return true;
  };
  if (fa::greedy_rounds(s, W)) {
    for (int x = 0; x < s.groups; ++x) {
      int load[fa::kGreedyMaxW] = {}, take[fa::kGreedyMaxW];
      for (int r = 0; r * W < npos; ++r) {
        fa::greedy_round(s, t, x, r, W, npos, load, take);
        for (int w = 0; w < W; ++w)
          if (take[w] >= 0 && !put(w * s.groups + x, take[w], x)) return FA_ERR_INVALID_ARG;
      }
    }
  } else {
    for (int wk = 0; wk < workers; ++wk) {
      int x, w;
      fa::worker_slot(s, wk, workers, &x, &w, &W);
      for (int r = 0;; ++r) {
        const int p = fa::snake_position(r, w, W);
        if (p >= npos) break;
        if (!put(wk, p, x)) return FA_ERR_INVALID_ARG;
      }
    }
  }
  int rounds = 0;
  for (int wk = 0; wk < workers; ++wk) {
    if (count[wk] > rounds) rounds = count[wk];
    for (int r = count[wk]; r < max_rounds; ++r) tiles[(long long)wk * max_rounds + r] = -1;
  }
  if (rounds_out) *rounds_out = rounds;
  if (bm_out) *bm_out = BM;
  return FA_OK;
}

int fa_version(void) { return 110; }

}  // extern "C"
