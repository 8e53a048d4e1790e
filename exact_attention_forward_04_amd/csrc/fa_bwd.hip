// fa_bwd.hip -- exact attention backward for MI355X (gfx950): kernels and C ABI.
//
// Given Q, K, V, the forward's O and LSE and the output gradient dO, this
// computes dQ, dK and dV, the gradients of sum <dO, O>.  Like the forward it
// never stores a score matrix: each block of S is recomputed from Q and K
// and consumed on chip (FlashAttention-4 paper, section 3.2: recompute S,
// then the products that give dP, dV, dQ and dK).
//
// The gfx950 design splits the work into two kernels so that every gradient
// row is owned by exactly one workgroup and reduced in its registers in a
// fixed order:
//
//   fa_bwd_dq    one tile of 32*NW query rows of one head per workgroup, as
//                in the forward; K and V stream through LDS in blocks of 64
//                keys.  In its prologue it forms Delta_i = <dO_i, O_i> for
//                its rows (stored for the second kernel).  Per block:
//                  S^T = K Q^T,  dP^T = V dO^T               (MFMA)
//                  P = exp2(c S - LSE log2 e),  dS = P (dP - Delta)
//                  dQ^T += K^T dS^T                          (MFMA)
//   fa_bwd_dkdv  one tile of 32*NW keys of one K/V head per workgroup; the
//                Q, dO, LSE and Delta blocks of every query head that reads
//                this K/V head stream through LDS in blocks of 64 rows.  Per
//                block:
//                  S = Q K^T,  dP = dO V^T                   (MFMA)
//                  P, dS as above
//                  dV^T += dO^T P,  dK^T += Q^T dS           (MFMA)
//
// In both kernels the wave's own 32 rows (query rows, or keys) sit in VGPRs
// as the B operand of v_mfma_f32_32x32x16_bf16, so the lane index is the
// row: S, dP, P and dS then hold 16 entries of the lane's row per 32-row
// sub-block, and the bf16 P and dS registers are directly the B operands of
// the products that contract over the streamed rows, whose A operands come
// from LDS through ds_read_b64_tr_b16 (the same layout the forward uses for
// V^T).
//
// The paper's kernel runs five products per block and adds dQ across
// workgroups with atomics in global memory, with a semaphore-ordered mode
// for reproducible results (section 3.2.4).  Here the dQ kernel recomputes S
// and dP instead (seven products per block pair in all): no atomics, no
// workspace beyond Delta, no ordering protocol, and bitwise reproducible
// results in every mode.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_host.h"
#include "fa_mask_runs.h"
#include "fa_sched.h"
#include "fa_tile.h"

namespace {

template <int D>
struct BwdCfg {
  // dQ: eight waves (two per SIMD), 32 query rows each.
  static constexpr int NW_DQ = 8;
  // dK/dV: one wave per SIMD, 32 keys each.  The two D-wide fp32
  // accumulators take 2*D/32*16 registers (128 at D = 128) and the software
  // pipeline of the block body holds two sub-blocks' S and dP at once, which
  // needs more than the 256 registers of two waves per SIMD.
  static constexpr int NW_KV = 4;
  static constexpr int BM = 32 * NW_DQ;  // query rows per dQ tile
  static constexpr int BN = 32 * NW_KV;  // keys per dK/dV tile
  static constexpr int BLK = kBN * D * 2;  // bytes of one 64-row block in LDS
  static constexpr int STATS = 2 * kBN * 4;  // LSE and Delta of one block
  // LDS: a ring of four [K | V] slots (dQ), or of four [Q | dO] slots
  // followed by four statistics slots (dK/dV); blocks are copied two ahead
  // of their use.  Blocks sit at multiples of BLK, as the operand addressing
  // needs.
  static constexpr int SLOTS = 4;
  static constexpr int LDS_DQ = SLOTS * 2 * BLK;
  static constexpr int LDS_KV = SLOTS * 2 * BLK + SLOTS * STATS;
};

struct BwdArgs {
  const __bf16 *q, *k, *v, *o, *dout;
  const float *lse;
  __bf16 *dq, *dk, *dv;
  float *delta;
  const int *cu;    // varlen query offsets or nullptr
  const int *cu_k;  // varlen key offsets (nullptr with cu)
  int B, H, Hkv, S, Sk;  // S: longest query length, Sk: longest key length
  float c;      // scale * log2(e)
  float scale;
};

struct Span {
  long long tok0;
  int L;
};

template <bool VARLEN>
__device__ __forceinline__ Span seq_of(const BwdArgs &a, int b) {
  if constexpr (VARLEN) {
    const int Lr = a.cu[b + 1] - a.cu[b];
    return {(long long)a.cu[b], Lr < 0 ? 0 : (Lr > a.S ? a.S : Lr)};
  } else {
    return {(long long)b * a.S, a.S};
  }
}

// Key span of sequence b (its own offsets and length when they differ from
// the queries').
template <bool VARLEN>
__device__ __forceinline__ Span kseq_of(const BwdArgs &a, int b) {
  if constexpr (VARLEN) {
    const int Lr = a.cu_k[b + 1] - a.cu_k[b];
    return {(long long)a.cu_k[b], Lr < 0 ? 0 : (Lr > a.Sk ? a.Sk : Lr)};
  } else {
    return {(long long)b * a.Sk, a.Sk};
  }
}

// Index of query row i of (b, h) in the LSE / Delta layout.
template <bool VARLEN>
__device__ __forceinline__ long long stat_index(const BwdArgs &a, int b, int h, long long tok0,
                                                int i) {
  if constexpr (VARLEN) return (long long)h * a.cu[a.B] + tok0 + i;
  else return ((long long)b * a.H + h) * a.S + i;
}

// One 4-byte-per-lane copy: global (64-bit lane address) -> LDS at m0 + 4*lane.
__device__ __forceinline__ void dma4(const float *gaddr, unsigned lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off"
      :
      : "s"(lds_addr), "v"(gaddr)
      : "memory", "m0");
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product with the register files chosen explicitly (the dK/dV
// kernel needs more than 256 registers per lane; left to itself the
// compiler shuttles S and dP between AGPRs and VGPRs on every block):
//   mfma_v0 / mfma_v: accumulator in VGPRs (read by the softmax VALU code),
//                     B operand in AGPRs; mfma_v0 starts from zero;
//   mfma_a:           accumulator in AGPRs (only MFMAs touch it).
// The compiler does not look inside these statements for hazards, so the
// caller keeps dependent products of one accumulator apart (two chains
// alternate, as the compiler itself schedules them) and waits with
// mfma_result_wait() before VALU code reads a result.
__device__ __forceinline__ void mfma_v0(f32x16 &c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_v(f32x16 &c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_a(f32x16 &c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// 32 wait states: more than an XDL product's result latency before VALU
// code (or v_accvgpr_read) may read its destination.
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

// The products of the dK/dV kernel: the explicit-register forms above when
// ASM (only safe while the compiler never copies their accumulators between
// register files inside the loop, which a test checks on the generated
// code), else the intrinsic, whose hazards the compiler tracks itself.
template <bool ASM>
__device__ __forceinline__ void prod_first(f32x16 &c, bf16x8 a, bf16x8 b) {
  if constexpr (ASM) {
    mfma_v0(c, a, b);
  } else {
    f32x16 z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.0f;
    c = mfma(a, b, z);
  }
}
template <bool ASM>
__device__ __forceinline__ void prod_next(f32x16 &c, bf16x8 a, bf16x8 b) {
  if constexpr (ASM) mfma_v(c, a, b);
  else c = mfma(a, b, c);
}
template <bool ASM>
__device__ __forceinline__ void prod_acc(f32x16 &c, bf16x8 a, bf16x8 b) {
  if constexpr (ASM) mfma_a(c, a, b);
  else c = mfma(a, b, c);
}
// Waits tied to the data they protect: every read of x (and y) comes after
// the wait because the wait is a use and a new definition of them, which no
// earlier code motion can reorder.
template <bool ASM>
__device__ __forceinline__ void result_wait_v(f32x16 &x, f32x16 &y) {
  if constexpr (ASM) asm volatile("s_nop 15\n\ts_nop 15" : "+v"(x), "+v"(y));
}
template <bool ASM>
__device__ __forceinline__ void result_wait_a(f32x16 &x, f32x16 &y) {
  if constexpr (ASM) asm volatile("s_nop 15\n\ts_nop 15" : "+a"(x), "+a"(y));
}

// Store the transposed accumulators acc[dt] (row d = 32dt + 8i + 4(l/32) + j,
// column = the lane's row) times f as bf16 into the lane's output row.
template <int D>
__device__ __forceinline__ void store_rows(__bf16 *row_ptr, const f32x16 *acc, float f, int hh) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  __bf16 *op = row_ptr + 4 * hh;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 out = {(__bf16)(acc[dt][4 * i + 0] * f), (__bf16)(acc[dt][4 * i + 1] * f),
                    (__bf16)(acc[dt][4 * i + 2] * f), (__bf16)(acc[dt][4 * i + 3] * f)};
      *(bf16x4 *)(op + 32 * dt + 8 * i) = out;
    }
}

// ---------------------------------------------------------------------------
// dQ (and Delta): one tile of BM query rows of head h.
// ---------------------------------------------------------------------------
// Launch slot -> (head slot hs of n_hs, level r; level 0 is the longest tile
// for causal masking).  Dense batches: tiles of one head are n_hs slots
// apart (the same XCD when n_hs is a multiple of 8).  Varlen batches have
// many more (sequence, head) pairs than CUs, and that order ran every
// concurrent tile on a pair of its own, each streaming its own operands past
// the L2.  There, XCD x = slot % 8 owns the head slots x, x+8, ... and its
// stream runs kBwdChunk consecutive levels of one head slot together, so
// those tiles share their K/V (or Q/dO) in the XCD's L2; chunks go longest
// first.  The grid is padded to whole chunks; slots past the last level exit.
constexpr int kBwdChunk = 8;
__device__ __forceinline__ void bwd_slot(int id, int n_hs, bool chunked, int *hs, int *r) {
  if (!chunked) {
    *hs = id % n_hs;
    *r = id / n_hs;
    return;
  }
  const int x = id % 8, q = id / 8;
  const int per = n_hs / 8;  // head slots per XCD
  const int chunk = q / (per * kBwdChunk);
  const int rem = q - chunk * per * kBwdChunk;
  const int k = rem / kBwdChunk, j = rem - k * kBwdChunk;
  *hs = x + 8 * k;
  *r = chunk * kBwdChunk + j;
}
__host__ __device__ inline bool bwd_chunked(bool varlen, int n_hs) { return varlen && n_hs % 8 == 0; }

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(BwdCfg<D>::NW_DQ * kWave, BwdCfg<D>::NW_DQ / 4) void fa_bwd_dq(
    BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int NW = C::NW_DQ;
  constexpr int NS = D / 16;
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  char LDS_AS *lds = (char LDS_AS *)lds_raw;

  // Launch order (bwd_slot): causal, the last (longest) m-blocks start first.
  const int nmb = fa::ceil_div(a.S, C::BM);
  const int BH = a.B * a.H;
  int bh, r;
  bwd_slot(blockIdx.x, BH, bwd_chunked(VARLEN, BH), &bh, &r);
  if (r >= nmb) return;  // grid padding
  const int mb = CAUSAL ? nmb - 1 - r : r;
  const int b = bh / a.H, h = bh % a.H;
  const Span sp = seq_of<VARLEN>(a, b);
  const int L = sp.L;
  const int m0 = mb * C::BM;
  if (m0 >= L) return;  // workgroup-uniform
  // Keys of the sequence; causal masks align to the bottom-right corner:
  // row i may use key j when j <= i + koff.
  const Span spk = kseq_of<VARLEN>(a, b);
  const int Lk = spk.L;
  const int koff = Lk - L;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int hh = lane >> 5;
  const int hk = h / (a.H / a.Hkv);
  const int wrow0 = m0 + 32 * wave;
  const bool active = wrow0 < L;
  const int wrow_last = (wrow0 + 31 < L - 1) ? wrow0 + 31 : L - 1;
  const int row = wrow0 + (lane & 31);
  const int rowc = row < L ? row : L - 1;  // rows past L read row L-1 (never stored)

  // Q and dO rows as B operands (lane: row l%32, d = 16s + 8(l/32) + 0..7);
  // Delta = <dO, O> of the row (two half-rows, then one permlane swap).
  bf16x8 qf[NS], gf[NS];
  float delta, lse2;
  {
    const long long si = stat_index<VARLEN>(a, b, h, sp.tok0, rowc);
    lse2 = a.lse[si] * kLog2e;
    const long long base = ((sp.tok0 + rowc) * a.H + h) * (long long)D + 8 * hh;
    const bf16x8 *qp = (const bf16x8 *)(a.q + base);
    const bf16x8 *gp = (const bf16x8 *)(a.dout + base);
    const bf16x8 *op = (const bf16x8 *)(a.o + base);
    float dsum = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = qp[2 * s];
      gf[s] = gp[2 * s];
      const bf16x8 of = op[2 * s];
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)gf[s][e], (float)of[e], dsum);
    }
    delta = sum_halves(dsum);
    if (hh == 0 && row < L) a.delta[si] = delta;
    // Keep the operands in registers for the whole tile (a re-fetch inside
    // the loop would wait behind the K/V copies on the vector-memory counter).
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(qf[s]), "+v"(gf[s]));
    asm volatile("" : "+v"(lse2), "+v"(delta));
  }

  int n_end = Lk;
  if (CAUSAL) n_end = (m0 + C::BM + koff < Lk) ? m0 + C::BM + koff : Lk;
  if (n_end < 0) n_end = 0;  // no row of the tile may use a key
  const int nblocks = fa::ceil_div(n_end, kBN);

  BlockLoader<D, NW> ld;
  ld.init(a.Hkv, wave, lane);
  constexpr int LOADS_BLOCK = 2 * BlockLoader<D, NW>::LOADS;
  LdsAddr<D> la;
  la.init(lane);
  auto kbuf = [&](int j) { return lds + (j % C::SLOTS) * 2 * C::BLK; };
  auto vbuf = [&](int j) { return lds + (j % C::SLOTS) * 2 * C::BLK + C::BLK; };
  auto issue = [&](int j) {
    ld.issue(a.k, spk.tok0, a.Hkv, hk, j * kBN, Lk, kbuf(j));
    ld.issue(a.v, spk.tok0, a.Hkv, hk, j * kBN, Lk, vbuf(j));
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;

  // Ring of four slots, copies two blocks ahead: block j+2 goes to the slot
  // of block j-2, whose reads every wave finished before the barrier that
  // opened block j-1.  One barrier per block.
  if (nblocks > 0) issue(0);
  if (nblocks > 1) issue(1);
  for (int j = 0; j < nblocks; ++j) {
    if (j + 2 < nblocks) {
      issue(j + 2);
      wait_vmcnt<2 * LOADS_BLOCK>();
    } else if (j + 1 < nblocks) {
      wait_vmcnt<LOADS_BLOCK>();
    } else {
      wait_vmcnt<0>();
    }
    barrier_nofence();
    const int n0 = j * kBN;
    if (active && (!CAUSAL || n0 <= wrow_last + koff)) {
      // ---- S^T = K Q^T and dP^T = V dO^T (keys on the M side)
      const unsigned ka = la.ky + lds_u32(kbuf(j));
      const unsigned va = la.ky + lds_u32(vbuf(j));
      f32x16 s[2], dp[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[i][e] = 0.0f;
          dp[i][e] = 0.0f;
        }
      // (S first, then dP: the scheduling barriers bound how many operand
      // reads the compiler hoists, which keeps two waves per SIMD in VGPRs.)
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 k0 = read_k<D>(ka, 0, st), k1 = read_k<D>(ka, 1, st);
        s[0] = mfma(k0, qf[st], s[0]);
        s[1] = mfma(k1, qf[st], s[1]);
        if (st % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 v0 = read_k<D>(va, 0, st), v1 = read_k<D>(va, 1, st);
        dp[0] = mfma(v0, gf[st], dp[0]);
        dp[1] = mfma(v1, gf[st], dp[1]);
        if (st % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
      // ---- P and dS.  Entry e of sub-block i is key n0 + 32i + 8(e>>2) +
      // 4h + (e&3) of the lane's row; it is kept iff its in-block offset is
      // below lim (key < Lk, and key <= row + koff when causal).
      const bool need_mask = (n0 + kBN > Lk) || (CAUSAL && n0 + kBN - 1 > wrow0 + koff);
      const int lim = (CAUSAL ? (row + koff + 1 < Lk ? row + koff + 1 : Lk) : Lk) - n0 - 4 * hh;
      bf16x8 ds8[4];
      // (two instances: blocks off the diagonal and inside the sequence,
      // the common case, skip the per-entry select)
      auto p_ds = [&](auto masked) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int off = 32 * i + 8 * (e >> 2) + (e & 3);
            float p = exp2_hw(__builtin_fmaf(s[i][e], a.c, -lse2));
            if constexpr (decltype(masked)::value) p = off < lim ? p : 0.0f;
            ds8[2 * i + (e >> 3)][e & 7] = (__bf16)(p * (dp[i][e] - delta));
          }
      };
      if (need_mask) p_ds(std::true_type{});
      else p_ds(std::false_type{});
      // ---- dQ^T += K^T dS^T (K^T by transposed reads of the K block)
      const unsigned kt0 = la.vw0 + lds_u32(kbuf(j)), kt1 = la.vw1 + lds_u32(kbuf(j));
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] = mfma(read_vt<D>(kt0, kt1, t, dt), ds8[t], acc[dt]);
    }
  }

  if (active && row < L)
    store_rows<D>(a.dq + ((sp.tok0 + row) * a.H + h) * (long long)D, acc, a.scale, hh);
}

// ---------------------------------------------------------------------------
// dK and dV: one tile of BN keys of K/V head hk.
// ---------------------------------------------------------------------------
// FULL: the launch guarantees that no block needs the entry mask (dense,
// non-causal, the query length a multiple of 64), so every block runs the
// body without it.
template <int D, bool CAUSAL, bool VARLEN, bool FULL = false>
__global__ __launch_bounds__(BwdCfg<D>::NW_KV * kWave, BwdCfg<D>::NW_KV / 4) void fa_bwd_dkdv(
    BwdArgs a) {
  static_assert(!FULL || (!CAUSAL && !VARLEN), "mask-free launches are dense and non-causal");
  using C = BwdCfg<D>;
  constexpr int NW = C::NW_KV;
  constexpr int NS = D / 16;
  // D = 128 needs more than 256 registers per lane and places them itself
  // (K, V and the dK/dV accumulators in AGPRs); D = 64 fits in VGPRs.
  constexpr bool ASM = (D == 128);
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  char LDS_AS *lds = (char LDS_AS *)lds_raw;

  // Launch order (bwd_slot): causal, the first key tiles, which every later
  // query row reads, are the longest and start first.
  const int BK = a.B * a.Hkv;
  int bhk, nb;
  bwd_slot(blockIdx.x, BK, bwd_chunked(VARLEN, BK), &bhk, &nb);
  if (nb >= fa::ceil_div(a.Sk, C::BN)) return;  // grid padding
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const Span spk = kseq_of<VARLEN>(a, b);  // keys of the sequence
  const int Lk = spk.L;
  const int n0t = nb * C::BN;
  if (n0t >= Lk) return;  // workgroup-uniform
  // Query rows of the sequence; causal: row i may use key j when
  // j <= i + koff (bottom-right alignment), i.e. i >= j - koff.
  const Span sp = seq_of<VARLEN>(a, b);
  const int L = sp.L;
  const int koff = Lk - L;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int hh = lane >> 5;
  const int G = a.H / a.Hkv;
  const int key0 = n0t + 32 * wave;  // first key of this wave
  const bool active = key0 < Lk;
  const int key = key0 + (lane & 31);
  const int keyc = key < Lk ? key : Lk - 1;  // keys past Lk read key Lk-1 (never stored)

  // K and V rows as B operands (lane: key l%32, d = 16s + 8(l/32) + 0..7).
  bf16x8 kf[NS], vf[NS];
  {
    const long long base = ((spk.tok0 + keyc) * a.Hkv + hk) * (long long)D + 8 * hh;
    const bf16x8 *kp = (const bf16x8 *)(a.k + base);
    const bf16x8 *vp = (const bf16x8 *)(a.v + base);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = kp[2 * s];
      vf[s] = vp[2 * s];
    }
    // K and V stay in registers for the whole tile (D = 128: in AGPRs, as
    // B operands of mfma_v).
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (ASM) asm volatile("" : "+a"(kf[s]), "+a"(vf[s]));
      else asm volatile("" : "+v"(kf[s]), "+v"(vf[s]));
    }
  }

  // Query blocks: for each query head of the group, the 64-row blocks from
  // the one holding the first row that may use the tile's first key (causal)
  // to the end.
  const int nqb = fa::ceil_div(L, kBN);
  const int qb0 = CAUSAL ? (n0t - koff > 0 ? n0t - koff : 0) / kBN : 0;
  const int per = nqb > qb0 ? nqb - qb0 : 0;
  const int nblocks = G * per;

  BlockLoader<D, NW> ld;
  ld.init(a.H, wave, lane);
  constexpr int LOADS_BLOCK = 2 * BlockLoader<D, NW>::LOADS;
  LdsAddr<D> la;
  la.init(lane);
  auto qbuf = [&](int t) { return lds + (t % C::SLOTS) * 2 * C::BLK; };
  auto gbuf = [&](int t) { return lds + (t % C::SLOTS) * 2 * C::BLK + C::BLK; };
  auto sbuf = [&](int t) { return lds + C::SLOTS * 2 * C::BLK + (t % C::SLOTS) * C::STATS; };
  // Block t: Q and dO rows (every wave), LSE (wave 0) and Delta (wave 1) of
  // its 64 rows, one row per lane, rows past L reading row L-1.
  auto issue = [&](int t) {
    const int h = hk * G + t / per;
    const int m0 = (qb0 + t % per) * kBN;
    ld.issue(a.q, sp.tok0, a.H, h, m0, L, qbuf(t));
    ld.issue(a.dout, sp.tok0, a.H, h, m0, L, gbuf(t));
    if (wave < 2) {
      const int rr = m0 + lane < L ? m0 + lane : L - 1;
      const float *src = (wave == 0 ? a.lse : a.delta) + stat_index<VARLEN>(a, b, h, sp.tok0, rr);
      dma4(src, lds_u32(sbuf(t)) + (unsigned)wave * (kBN * 4));
    }
  };
  // Wait for block t while the n_after later blocks (0, 1 or 2) may still be
  // in flight (waves 0 and 1 issue one statistics copy per block on top of
  // the row copies).
  auto wait_block = [&](int n_after) {
    if (wave < 2) {
      if (n_after >= 2) wait_vmcnt<2 * (LOADS_BLOCK + 1)>();
      else if (n_after == 1) wait_vmcnt<LOADS_BLOCK + 1>();
      else wait_vmcnt<0>();
    } else {
      if (n_after >= 2) wait_vmcnt<2 * LOADS_BLOCK>();
      else if (n_after == 1) wait_vmcnt<LOADS_BLOCK>();
      else wait_vmcnt<0>();
    }
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[dt][e] = 0.0f;
      dv[dt][e] = 0.0f;
    }
  if constexpr (ASM) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) asm volatile("" : "+a"(dk[dt]), "+a"(dv[dt]));
    mfma_result_wait();  // the AGPR writes above land before the first product reads them
  }

  // Ring of four slots, copies two blocks ahead (as in fa_bwd_dq).
  if (nblocks > 0) issue(0);
  if (nblocks > 1) issue(1);
  // Block t (masked: with the entry mask).
  auto step = [&](int t, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    if (t + 2 < nblocks) issue(t + 2);
    wait_block(t + 2 < nblocks ? 2 : (t + 1 < nblocks ? 1 : 0));
    const int m0 = (qb0 + t % per) * kBN;
    if constexpr (ASM && CAUSAL) {
      // A row without keys (r + koff < 0: more query rows than keys) has
      // LSE = -inf, and every entry of it is masked.  The D = 128 body masks
      // scores to -inf before the exponential, where -inf - (-inf) would give
      // NaN, so wave 0, whose copy of the block's LSE has landed, sets such
      // rows' LSE to +inf (P = exp2(-inf) = 0 either way) before the barrier.
      if (wave == 0 && m0 < -koff) {
        if (m0 + lane < -koff) ((float LDS_AS *)sbuf(t))[lane] = INFINITY;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
    barrier_nofence();
    if (active && (!CAUSAL || m0 + kBN - 1 >= key0 - koff)) {
      const unsigned qa = la.ky + lds_u32(qbuf(t));
      const unsigned ga = la.ky + lds_u32(gbuf(t));
      const unsigned gt0 = la.vw0 + lds_u32(gbuf(t)), gt1 = la.vw1 + lds_u32(gbuf(t));
      const unsigned qt0 = la.vw0 + lds_u32(qbuf(t)), qt1 = la.vw1 + lds_u32(qbuf(t));
      const float LDS_AS *lse_l = (const float LDS_AS *)sbuf(t);
      const float LDS_AS *del_l = lse_l + kBN;
      // Mask bounds for this wave's keys (a block that needs no mask gets
      // bounds that keep every entry; D = 64 runs such blocks through a body
      // without the mask, and D = 128 skips its score mask on them).
      const bool need_mask = (m0 + kBN > L) || (CAUSAL && m0 < key0 - koff + 31);
      const int hi = need_mask ? L - m0 - 4 * hh : INT_MAX;
      const int lo = (need_mask && CAUSAL) ? key - koff - m0 - 4 * hh : INT_MIN;
      // Entry offsets lie in [0, 64): kept iff lo <= off < hi, i.e. iff
      // off - lo_c < span as unsigned, with lo and hi clamped to [0, 64]:
      // one subtract, one compare and one select per entry.  (The two-sided
      // test written out was compiled into a branch per entry, with its
      // exec-mask bookkeeping.)
      const int lo_c = lo < 0 ? 0 : (lo > 64 ? 64 : lo);
      const int hi_c = hi < 0 ? 0 : (hi > 64 ? 64 : hi);
      const unsigned span = hi_c > lo_c ? (unsigned)(hi_c - lo_c) : 0u;
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      f32x16 s[2], dp[2];
      bf16x8 p8[4], ds8[4];
      // The block is done in four phases of NST steps, two matrix products
      // per step, with the operand reads of step k+2 issued before the
      // products of step k, across phase boundaries too (LDS latency hides
      // behind the matrix unit):
      //   A: S_0 = Q_0 K^T, dP_0 = dO_0 V^T         (query rows 0-31)
      //   B: S_1, dP_1                    + VALU: P_0, dS_0
      //   C: dV^T, dK^T over rows 0-31    + VALU: P_1, dS_1
      //   D: dV^T, dK^T over rows 32-63
      // One wave per SIMD: the VALU work of one sub-block runs between the
      // matrix products of the other, so the matrix unit keeps running
      // (software pipelining inside the wave).
      constexpr int NST = NS;  // steps per phase
      constexpr int NT = D / 32;
      static_assert(NST == 2 * NT, "phases C and D have 2*D/32 steps");
      // Entry e of S_i/dP_i is query row m0 + 32i + 8(e>>2) + 4h + (e&3)
      // against the lane's key; it is kept iff its in-block offset off
      // satisfies lo <= off < hi (row < L, and row >= key - koff when causal).
      f32x4 l4[2][4], d4[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int r0 = 32 * i + 8 * g4 + 4 * hh;
          l4[i][g4] = *(const f32x4 LDS_AS *)(lse_l + r0);
          d4[i][g4] = *(const f32x4 LDS_AS *)(del_l + r0);
        }
      // P and dS of the n entries e0 .. e0+n-1 of sub-block i (the 16
      // entries of a sub-block spread over the NST steps of a phase, EPS
      // per step).
      constexpr int EPS = 16 / NST;
      static_assert(EPS * NST == 16, "entries split evenly over the steps");
      auto softmax_grad_part = [&](int i, int e0, int n) {
#pragma unroll
        for (int e = e0; e < e0 + n; ++e) {
          const int g4 = e >> 2, jj = e & 3;
          const int off = 32 * i + 8 * g4 + jj;
          float p = exp2_hw(__builtin_fmaf(s[i][e], a.c, -(l4[i][g4][jj] * kLog2e)));
          if constexpr (MASKED && !ASM) p = ((unsigned)(off - lo_c) < span) ? p : 0.0f;
          const int tt = 2 * i + (e >> 3);
          p8[tt][e & 7] = (__bf16)p;
          ds8[tt][e & 7] = (__bf16)(p * (dp[i][e] - d4[i][g4][jj]));
          // An operand is complete here: pin it, so no part of its
          // arithmetic can be moved down to the product that reads it
          // (which comes at least one step later).
          if ((e & 7) == 7) asm volatile("" : "+v"(p8[tt]), "+v"(ds8[tt]));
        }
      };
      // Scores of sub-block i that the mask drops set to -inf (D = 128), so
      // that P = exp2(c*s - log2(e)*LSE) = 0 (the LSE of a row without keys
      // reads +inf here: see the block's start).
      auto mask_scores = [&](int i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = 32 * i + 8 * (e >> 2) + (e & 3);
          s[i][e] = ((unsigned)(off - lo_c) < span) ? s[i][e] : -INFINITY;
        }
      };
      // Operands of step k: rows of Q and dO (phases A, B) or transposed
      // reads of dO and Q (phases C, D: 16-row step tt, d tile dt).
      auto read_step = [&](int k, bf16x8 &x, bf16x8 &y) {
        const int ph = k / NST, st = k % NST;
        if (ph < 2) {
          x = read_k<D>(qa, ph, st);
          y = read_k<D>(ga, ph, st);
        } else {
          const int tt = 2 * (ph - 2) + st / NT, dt = st % NT;
          x = read_vt<D>(gt0, gt1, tt, dt);
          y = read_vt<D>(qt0, qt1, tt, dt);
        }
      };
      constexpr int NK = 4 * NST;
      bf16x8 ox[NK], oy[NK];
      read_step(0, ox[0], oy[0]);
      read_step(1, ox[1], oy[1]);
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        if (k + 2 < NK) read_step(k + 2, ox[k + 2], oy[k + 2]);
        __builtin_amdgcn_sched_barrier(0);
        const int ph = k / NST, st = k % NST;
        const bool valu = (ph == 1 || ph == 2);
        // The first product of the step, then half of the step's VALU share
        // while it runs, the second product, the other half: with one wave
        // per SIMD the second product would otherwise hold the wave until
        // the matrix unit is free, and the VALU work would start only then.
        if (ph < 2) {
          if (st == 0) prod_first<ASM>(s[ph], ox[k], kf[st]);
          else prod_next<ASM>(s[ph], ox[k], kf[st]);
        } else {
          const int tt = 2 * (ph - 2) + st / NT, dt = st % NT;
          prod_acc<ASM>(dv[dt], ox[k], p8[tt]);
        }
        if (valu) {
          // S/dP of sub-block ph-1 were produced by the products just before
          if (st == 0) {
            result_wait_v<ASM>(s[ph - 1], dp[ph - 1]);
            // D = 128 masks the scores instead (-inf before the exponential
            // gives the same P = 0), and only on blocks that need it: a
            // wave-uniform branch around the sub-block's selects keeps one
            // copy of the body, and with it the fixed register plan.
            if constexpr (ASM && MASKED) {
              if (need_mask) mask_scores(ph - 1);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          softmax_grad_part(ph - 1, EPS * st, EPS / 2);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (ph < 2) {
          if (st == 0) prod_first<ASM>(dp[ph], oy[k], vf[st]);
          else prod_next<ASM>(dp[ph], oy[k], vf[st]);
        } else {
          const int tt = 2 * (ph - 2) + st / NT, dt = st % NT;
          prod_acc<ASM>(dk[dt], oy[k], ds8[tt]);
        }
        if (valu) {
          __builtin_amdgcn_sched_barrier(0);
          softmax_grad_part(ph - 1, EPS * st + EPS / 2, EPS / 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // The mask costs a subtract, a compare and a select per entry, and only
  // the diagonal and tail blocks need it.  D = 64 runs the blocks that need
  // none (one run per query head, fa_mask_runs.h) through a second copy of
  // the body without it; every wave still passes one barrier per block,
  // whichever body it runs.  D = 128 keeps one body (with two, the compiler
  // no longer holds its fixed register plan: the accumulators and K/V move
  // between register files inside the products' stream); it masks scores
  // behind a wave-uniform branch instead (mask_scores).
  if (nblocks > 0) {
    if constexpr (FULL) {
      for (int t = 0; t < nblocks; ++t) step(t, std::false_type{});
    } else if constexpr (!ASM) {
      const fa::MaskRuns runs = fa::mask_runs(CAUSAL, L, qb0, per, key0, koff, kBN);
      for (int t = 0; t < nblocks;) {
        const int e = runs.run_end(t);
        if (e > t) {
          for (; t < e; ++t) step(t, std::false_type{});
        } else {
          step(t, std::true_type{});
          ++t;
        }
      }
    } else {
      for (int t = 0; t < nblocks; ++t) step(t, std::true_type{});
    }
  }

  // the last products into dK/dV have landed
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) result_wait_a<ASM>(dk[dt], dv[dt]);
  if (active && key < Lk) {
    const long long rowoff = ((spk.tok0 + key) * a.Hkv + hk) * (long long)D;
    store_rows<D>(a.dk + rowoff, dk, a.scale, hh);
    store_rows<D>(a.dv + rowoff, dv, 1.0f, hh);
  }
}

// ---------------------------------------------------------------------------
// Wide heads: D = 256, and D = 192 with D_v = 128 (the pair of DeepSeek V3
// the FlashAttention-4 paper benchmarks, section 5.1).  A wave's operands
// and accumulators need more than the 256 registers of two waves per SIMD,
// so both kernels run one wave per SIMD (4 waves, 128-row tiles) and the
// compiler places what does not fit in VGPRs in AGPRs.  The streamed blocks
// use a two-slot LDS ring copied one block ahead: the copy of block j+1
// starts right after the barrier that opens block j, into the slot of block
// j-1, which every wave finished reading before that barrier.  The dK/dV
// kernel for D = 256 splits dK's and dV's columns over two workgroups per
// key tile (each recomputes S and dP); that keeps its accumulators in the
// register file.
// ---------------------------------------------------------------------------
template <int D>
struct WideCfg {
  static constexpr int DV = head_dim_v<D>();
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;  // query rows per dQ tile
  static constexpr int BN = 32 * NW;  // keys per dK/dV tile
  static constexpr int DSPLIT = (D == 256) ? 2 : 1;  // dK/dV column parts per key tile
  // One slot holds a D-wide block (K or Q; D = 192 in two parts, 128 and 64
  // wide) and a DV-wide block (V or dO).  Every part starts at a multiple of
  // its own size, as the operand addressing needs.
  static constexpr int W1 = (D == 192) ? 128 : D;
  static constexpr int P1 = W1 * kBN * 2;
  static constexpr int P2 = (D == 192) ? 64 * kBN * 2 : 0;
  static constexpr int PV = DV * kBN * 2;
  static constexpr int OFF2 = P1;
  static constexpr int OFFV = ((P1 + P2 + PV - 1) / PV) * PV;
  static constexpr int SLOT = ((OFFV + PV + P1 - 1) / P1) * P1;
  static constexpr int STATS = 2 * kBN * 4;  // LSE and Delta of one block
  static constexpr int LDS_DQ = 2 * SLOT;
  static constexpr int LDS_KV = 2 * SLOT + 2 * STATS;
  static_assert(SLOT % P1 == 0 && SLOT % PV == 0 && OFFV % PV == 0, "part alignment");
  static_assert(LDS_KV <= 160 * 1024, "LDS");
};

// Operand reads of one slot: rows (A operands over a 32-row sub-block kb
// and a 16-wide k-step s) and transposed reads (A operands over a 16-row
// step t and a 32-wide d tile dt) of its D-wide and DV-wide blocks.
template <int D>
struct WideOps {
  static constexpr int DV = head_dim_v<D>();
  static constexpr int W1 = WideCfg<D>::W1;
  unsigned r1, r2, rv, t1a, t1b, t2a, t2b, tva, tvb;
  __device__ __forceinline__ void init(int lane) {
    r1 = k_lane_const<W1>(lane);
    r2 = (D == 192) ? k_lane_const<64>(lane) : 0u;
    rv = k_lane_const<DV>(lane);
    LdsAddr<W1> l1;
    l1.init(lane);
    t1a = l1.vw0;
    t1b = l1.vw1;
    LdsAddr<64> l2;
    l2.init(lane);
    t2a = l2.vw0;
    t2b = l2.vw1;
    LdsAddr<DV> lv;
    lv.init(lane);
    tva = lv.vw0;
    tvb = lv.vw1;
  }
  // b1, b2: the D-wide block's parts; bv: the DV-wide block (LDS byte addresses)
  __device__ __forceinline__ bf16x8 row_d(unsigned b1, unsigned b2, int kb, int s) const {
    if constexpr (D == 192) {
      if (s >= 8) return read_k<64>(r2 + b2, kb, s - 8);
    }
    return read_k<W1>(r1 + b1, kb, s);
  }
  __device__ __forceinline__ bf16x8 row_v(unsigned bv, int kb, int s) const {
    return read_k<DV>(rv + bv, kb, s);
  }
  __device__ __forceinline__ bf16x8 tr_d(unsigned b1, unsigned b2, int t, int dt) const {
    if constexpr (D == 192) {
      if (dt >= 4) return read_vt<64>(t2a + b2, t2b + b2, t, dt - 4);
    }
    return read_vt<W1>(t1a + b1, t1b + b1, t, dt);
  }
  __device__ __forceinline__ bf16x8 tr_v(unsigned bv, int t, int dt) const {
    return read_vt<DV>(tva + bv, tvb + bv, t, dt);
  }
};

// Store NT transposed accumulator tiles (as store_rows) times f as bf16
// into the lane's output row from column 0 of row_ptr.
template <int NT>
__device__ __forceinline__ void store_tiles(__bf16 *row_ptr, const f32x16 *acc, float f, int hh) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  __bf16 *op = row_ptr + 4 * hh;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 out = {(__bf16)(acc[dt][4 * i + 0] * f), (__bf16)(acc[dt][4 * i + 1] * f),
                    (__bf16)(acc[dt][4 * i + 2] * f), (__bf16)(acc[dt][4 * i + 3] * f)};
      *(bf16x4 *)(op + 32 * dt + 8 * i) = out;
    }
}

// dQ (and Delta) for wide heads: as fa_bwd_dq, one wave per SIMD.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(WideCfg<D>::NW * kWave, 1) void fa_bwd_dq_wide(BwdArgs a) {
  using C = WideCfg<D>;
  constexpr int DV = C::DV;
  constexpr int NW = C::NW;
  constexpr int NS = D / 16, NSV = DV / 16, NT = D / 32;
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  char LDS_AS *lds = (char LDS_AS *)lds_raw;

  const int nmb = fa::ceil_div(a.S, C::BM);
  const int BH = a.B * a.H;
  int bh, r;
  bwd_slot(blockIdx.x, BH, bwd_chunked(VARLEN, BH), &bh, &r);
  if (r >= nmb) return;  // grid padding
  const int mb = CAUSAL ? nmb - 1 - r : r;
  const int b = bh / a.H, h = bh % a.H;
  const Span sp = seq_of<VARLEN>(a, b);
  const int L = sp.L;
  const int m0 = mb * C::BM;
  if (m0 >= L) return;  // workgroup-uniform
  const Span spk = kseq_of<VARLEN>(a, b);
  const int Lk = spk.L;
  const int koff = Lk - L;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int hh = lane >> 5;
  const int hk = h / (a.H / a.Hkv);
  const int wrow0 = m0 + 32 * wave;
  const bool active = wrow0 < L;
  const int wrow_last = (wrow0 + 31 < L - 1) ? wrow0 + 31 : L - 1;
  const int row = wrow0 + (lane & 31);
  const int rowc = row < L ? row : L - 1;

  // Q (D wide) and dO (DV wide) rows as B operands; Delta = <dO, O>.
  bf16x8 qf[NS], gf[NSV];
  float delta, lse2;
  {
    const long long si = stat_index<VARLEN>(a, b, h, sp.tok0, rowc);
    lse2 = a.lse[si] * kLog2e;
    const long long tok = (sp.tok0 + rowc) * a.H + h;
    const bf16x8 *qp = (const bf16x8 *)(a.q + tok * D + 8 * hh);
    const bf16x8 *gp = (const bf16x8 *)(a.dout + tok * DV + 8 * hh);
    const bf16x8 *op = (const bf16x8 *)(a.o + tok * DV + 8 * hh);
    float dsum = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = qp[2 * s];
#pragma unroll
    for (int s = 0; s < NSV; ++s) {
      gf[s] = gp[2 * s];
      const bf16x8 of = op[2 * s];
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)gf[s][e], (float)of[e], dsum);
    }
    delta = sum_halves(dsum);
    if (hh == 0 && row < L) a.delta[si] = delta;
  }

  int n_end = Lk;
  if (CAUSAL) n_end = (m0 + C::BM + koff < Lk) ? m0 + C::BM + koff : Lk;
  if (n_end < 0) n_end = 0;
  const int nblocks = fa::ceil_div(n_end, kBN);

  BlockLoader<D, NW> ldk;
  ldk.init(a.Hkv, wave, lane);
  BlockLoader<DV, NW> ldv;
  ldv.init(a.Hkv, wave, lane);
  WideOps<D> ops;
  ops.init(lane);
  auto slot = [&](int j) { return lds + (j & 1) * C::SLOT; };
  auto issue = [&](int j) {
    ldk.issue(a.k, spk.tok0, a.Hkv, hk, j * kBN, Lk, slot(j), slot(j) + C::OFF2);
    ldv.issue(a.v, spk.tok0, a.Hkv, hk, j * kBN, Lk, slot(j) + C::OFFV);
  };

  f32x16 acc[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;

  if (nblocks > 0) issue(0);
  for (int j = 0; j < nblocks; ++j) {
    wait_vmcnt<0>();        // this wave's copies of block j have landed
    barrier_after_reads();  // everyone's have, and block j-1 is read
    if (j + 1 < nblocks) issue(j + 1);
    const int n0 = j * kBN;
    if (active && (!CAUSAL || n0 <= wrow_last + koff)) {
      const unsigned b1 = lds_u32(slot(j)), b2 = b1 + C::OFF2, bv = b1 + C::OFFV;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[i][e] = 0.0f;
          dp[i][e] = 0.0f;
        }
      // S^T = K Q^T, dP^T = V dO^T
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s[0] = mfma(ops.row_d(b1, b2, 0, st), qf[st], s[0]);
        s[1] = mfma(ops.row_d(b1, b2, 1, st), qf[st], s[1]);
      }
#pragma unroll
      for (int st = 0; st < NSV; ++st) {
        dp[0] = mfma(ops.row_v(bv, 0, st), gf[st], dp[0]);
        dp[1] = mfma(ops.row_v(bv, 1, st), gf[st], dp[1]);
      }
      // P and dS (entry layout and mask as in fa_bwd_dq)
      const bool need_mask = (n0 + kBN > Lk) || (CAUSAL && n0 + kBN - 1 > wrow0 + koff);
      const int lim = (CAUSAL ? (row + koff + 1 < Lk ? row + koff + 1 : Lk) : Lk) - n0 - 4 * hh;
      bf16x8 ds8[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = 32 * i + 8 * (e >> 2) + (e & 3);
          float p = exp2_hw(__builtin_fmaf(s[i][e], a.c, -lse2));
          if (need_mask) p = off < lim ? p : 0.0f;
          ds8[2 * i + (e >> 3)][e & 7] = (__bf16)(p * (dp[i][e] - delta));
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) acc[dt] = mfma(ops.tr_d(b1, b2, t, dt), ds8[t], acc[dt]);
    }
  }

  if (active && row < L)
    store_tiles<NT>(a.dq + ((sp.tok0 + row) * a.H + h) * (long long)D, acc, a.scale, hh);
}

// dK and dV for wide heads: as fa_bwd_dkdv, with column part `part` of
// DSPLIT of dK and dV per workgroup.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(WideCfg<D>::NW * kWave, 1) void fa_bwd_dkdv_wide(BwdArgs a) {
  using C = WideCfg<D>;
  constexpr int DV = C::DV;
  constexpr int NW = C::NW;
  constexpr int DS = C::DSPLIT;
  constexpr int NS = D / 16, NSV = DV / 16;
  constexpr int NTK = D / 32 / DS, NTV = DV / 32 / DS;
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  char LDS_AS *lds = (char LDS_AS *)lds_raw;

  // Launch slot -> (tile slot, column part): the DS parts of one key tile
  // are 8 slots apart, on the same XCD, so they share their Q/dO in its L2.
  int part = 0, tslot = blockIdx.x;
  if constexpr (DS > 1) {
    const int x = blockIdx.x % 8, q = blockIdx.x / 8;
    part = q % DS;
    tslot = (q / DS) * 8 + x;
  }
  const int BK = a.B * a.Hkv;
  int bhk, nb;
  bwd_slot(tslot, BK, bwd_chunked(VARLEN, BK), &bhk, &nb);
  if (bhk >= BK || nb >= fa::ceil_div(a.Sk, C::BN)) return;  // grid padding
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const Span spk = kseq_of<VARLEN>(a, b);
  const int Lk = spk.L;
  const int n0t = nb * C::BN;
  if (n0t >= Lk) return;
  const Span sp = seq_of<VARLEN>(a, b);
  const int L = sp.L;
  const int koff = Lk - L;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int hh = lane >> 5;
  const int G = a.H / a.Hkv;
  const int key0 = n0t + 32 * wave;
  const bool active = key0 < Lk;
  const int key = key0 + (lane & 31);
  const int keyc = key < Lk ? key : Lk - 1;

  // K (D wide) and V (DV wide) rows of the lane's key as B operands.
  bf16x8 kf[NS], vf[NSV];
  {
    const long long tok = (spk.tok0 + keyc) * a.Hkv + hk;
    const bf16x8 *kp = (const bf16x8 *)(a.k + tok * D + 8 * hh);
    const bf16x8 *vp = (const bf16x8 *)(a.v + tok * DV + 8 * hh);
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[s] = kp[2 * s];
#pragma unroll
    for (int s = 0; s < NSV; ++s) vf[s] = vp[2 * s];
  }

  const int nqb = fa::ceil_div(L, kBN);
  const int qb0 = CAUSAL ? (n0t - koff > 0 ? n0t - koff : 0) / kBN : 0;
  const int per = nqb > qb0 ? nqb - qb0 : 0;
  const int nblocks = G * per;

  BlockLoader<D, NW> ldq;
  ldq.init(a.H, wave, lane);
  BlockLoader<DV, NW> ldg;
  ldg.init(a.H, wave, lane);
  WideOps<D> ops;
  ops.init(lane);
  auto slot = [&](int t) { return lds + (t & 1) * C::SLOT; };
  auto sbuf = [&](int t) { return lds + 2 * C::SLOT + (t & 1) * C::STATS; };
  auto issue = [&](int t) {
    const int h = hk * G + t / per;
    const int m0 = (qb0 + t % per) * kBN;
    ldq.issue(a.q, sp.tok0, a.H, h, m0, L, slot(t), slot(t) + C::OFF2);
    ldg.issue(a.dout, sp.tok0, a.H, h, m0, L, slot(t) + C::OFFV);
    if (wave < 2) {
      const int rr = m0 + lane < L ? m0 + lane : L - 1;
      const float *src = (wave == 0 ? a.lse : a.delta) + stat_index<VARLEN>(a, b, h, sp.tok0, rr);
      dma4(src, lds_u32(sbuf(t)) + (unsigned)wave * (kBN * 4));
    }
  };

  f32x16 dk[NTK], dv[NTV];
#pragma unroll
  for (int dt = 0; dt < NTK; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[dt][e] = 0.0f;
#pragma unroll
  for (int dt = 0; dt < NTV; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dv[dt][e] = 0.0f;

  if (nblocks > 0) issue(0);
  for (int t = 0; t < nblocks; ++t) {
    wait_vmcnt<0>();
    barrier_after_reads();
    if (t + 1 < nblocks) issue(t + 1);
    const int m0 = (qb0 + t % per) * kBN;
    if (active && (!CAUSAL || m0 + kBN - 1 >= key0 - koff)) {
      const unsigned b1 = lds_u32(slot(t)), b2 = b1 + C::OFF2, bv = b1 + C::OFFV;
      const float LDS_AS *lse_l = (const float LDS_AS *)sbuf(t);
      const float LDS_AS *del_l = lse_l + kBN;
      const bool need_mask = (m0 + kBN > L) || (CAUSAL && m0 < key0 - koff + 31);
      const int hi = need_mask ? L - m0 - 4 * hh : INT_MAX;
      const int lo = (need_mask && CAUSAL) ? key - koff - m0 - 4 * hh : INT_MIN;
      // Entry offsets lie in [0, 64): kept iff lo <= off < hi, i.e. iff
      // off - lo_c < span as unsigned, with lo and hi clamped to [0, 64]:
      // one subtract, one compare and one select per entry.  (The two-sided
      // test written out was compiled into a branch per entry, with its
      // exec-mask bookkeeping.)
      const int lo_c = lo < 0 ? 0 : (lo > 64 ? 64 : lo);
      const int hi_c = hi < 0 ? 0 : (hi > 64 ? 64 : hi);
      const unsigned span = hi_c > lo_c ? (unsigned)(hi_c - lo_c) : 0u;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[i][e] = 0.0f;
          dp[i][e] = 0.0f;
        }
      // S = Q K^T, dP = dO V^T for query sub-blocks 0 and 1
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s[0] = mfma(ops.row_d(b1, b2, 0, st), kf[st], s[0]);
        s[1] = mfma(ops.row_d(b1, b2, 1, st), kf[st], s[1]);
      }
#pragma unroll
      for (int st = 0; st < NSV; ++st) {
        dp[0] = mfma(ops.row_v(bv, 0, st), vf[st], dp[0]);
        dp[1] = mfma(ops.row_v(bv, 1, st), vf[st], dp[1]);
      }
      // P and dS (entry layout and mask as in fa_bwd_dkdv)
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      bf16x8 p8[4], ds8[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int r0 = 32 * i + 8 * g4 + 4 * hh;
          const f32x4 l4 = *(const f32x4 LDS_AS *)(lse_l + r0);
          const f32x4 d4 = *(const f32x4 LDS_AS *)(del_l + r0);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int e = 4 * g4 + jj;
            const int off = 32 * i + 8 * g4 + jj;
            float p = exp2_hw(__builtin_fmaf(s[i][e], a.c, -(l4[jj] * kLog2e)));
            p = ((unsigned)(off - lo_c) < span) ? p : 0.0f;
            const int tt = 2 * i + (e >> 3);
            p8[tt][e & 7] = (__bf16)p;
            ds8[tt][e & 7] = (__bf16)(p * (dp[i][e] - d4[jj]));
          }
        }
      // dV^T += dO^T P and dK^T += Q^T dS over this part's d tiles
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int dt = 0; dt < NTV; ++dt)
          dv[dt] = mfma(ops.tr_v(bv, tt, part * NTV + dt), p8[tt], dv[dt]);
#pragma unroll
        for (int dt = 0; dt < NTK; ++dt)
          dk[dt] = mfma(ops.tr_d(b1, b2, tt, part * NTK + dt), ds8[tt], dk[dt]);
      }
    }
  }

  if (active && key < Lk) {
    const long long tok = (spk.tok0 + key) * a.Hkv + hk;
    store_tiles<NTK>(a.dk + tok * D + 32 * NTK * part, dk, a.scale, hh);
    store_tiles<NTV>(a.dv + tok * DV + 32 * NTV * part, dv, 1.0f, hh);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int validate_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H,
                 int Hkv, int S, int Sk, int D, int Dv, float scale, int causal, const int *cu_q,
                 const int *cu_k) {
  const void *bufs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void *p : bufs)
    if (!p || !aligned16(p)) return FA_ERR_INVALID_ARG;
  if (!lse || !delta) return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(lse) & 3) || (reinterpret_cast<uintptr_t>(delta) & 3))
    return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S <= 0 || Sk <= 0 || D <= 0 || Dv <= 0) return FA_ERR_INVALID_ARG;
  if ((cu_q == nullptr) != (cu_k == nullptr)) return FA_ERR_INVALID_ARG;
  if (Hkv <= 0 || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  const bool pair_ok = (D == Dv && (D == 64 || D == 128 || D == 256)) || (D == 192 && Dv == 128);
  if (!pair_ok) return FA_ERR_UNSUPPORTED;
  const long long Smax = S > Sk ? S : Sk;
  if ((long long)B * Smax > (1LL << 31) - 1 || Smax * H > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

template <int D, bool CAUSAL, bool VARLEN>
int launch_bwd(const BwdArgs &a, hipStream_t st) {
  using C = BwdCfg<D>;
  // levels per head slot, padded to whole chunks where bwd_slot chunks them
  auto levels = [](int n, bool chunked) {
    return chunked ? fa::ceil_div(n, kBwdChunk) * kBwdChunk : n;
  };
  const long long g1 = (long long)a.B * a.H *
                       levels(fa::ceil_div(a.S, C::BM), bwd_chunked(VARLEN, a.B * a.H));
  const long long g2 = (long long)a.B * a.Hkv *
                       levels(fa::ceil_div(a.Sk, C::BN), bwd_chunked(VARLEN, a.B * a.Hkv));
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  auto k1 = fa_bwd_dq<D, CAUSAL, VARLEN>;
  auto k2 = fa_bwd_dkdv<D, CAUSAL, VARLEN>;
  // D = 128 keeps one block body; a launch in which no block needs the mask
  // takes the instance without it (D = 64 runs its mask-free blocks through a
  // second body, which measured faster than this instance).
  const bool full = D == 128 && !CAUSAL && !VARLEN && a.S % kBN == 0;
  if constexpr (D == 128 && !CAUSAL && !VARLEN) {
    if (full) k2 = fa_bwd_dkdv<D, false, false, true>;
  }
  if (!allow_lds(k1, C::LDS_DQ) || !allow_lds(k2, C::LDS_KV)) return FA_ERR_HIP;
  FA_LOG_LAUNCH("fa_bwd_dq<D=%d causal=%d varlen=%d>: %lld workgroups x %d threads, %d B LDS; "
                "fa_bwd_dkdv%s: %lld workgroups x %d threads, %d B LDS; B=%d H=%d H_kv=%d "
                "S_q=%d S_k=%d",
                D, (int)CAUSAL, (int)VARLEN, g1, C::NW_DQ * kWave, C::LDS_DQ,
                full ? " (no block masked)" : "", g2,
                C::NW_KV * kWave, C::LDS_KV, a.B, a.H, a.Hkv, a.S, a.Sk);
  // dQ first: it also writes Delta, which the dK/dV kernel reads.
  hipLaunchKernelGGL(k1, dim3((unsigned)g1), dim3(C::NW_DQ * kWave), C::LDS_DQ, st, a);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  hipLaunchKernelGGL(k2, dim3((unsigned)g2), dim3(C::NW_KV * kWave), C::LDS_KV, st, a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int D, bool CAUSAL, bool VARLEN>
int launch_bwd_wide(const BwdArgs &a, hipStream_t st) {
  using C = WideCfg<D>;
  auto levels = [](int n, bool chunked) {
    return chunked ? fa::ceil_div(n, kBwdChunk) * kBwdChunk : n;
  };
  const long long g1 = (long long)a.B * a.H *
                       levels(fa::ceil_div(a.S, C::BM), bwd_chunked(VARLEN, a.B * a.H));
  long long g2 = (long long)a.B * a.Hkv *
                 levels(fa::ceil_div(a.Sk, C::BN), bwd_chunked(VARLEN, a.B * a.Hkv));
  if (C::DSPLIT > 1) g2 = ((g2 + 7) / 8) * 8 * C::DSPLIT;  // whole groups of 8 tile slots
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  auto k1 = fa_bwd_dq_wide<D, CAUSAL, VARLEN>;
  auto k2 = fa_bwd_dkdv_wide<D, CAUSAL, VARLEN>;

  if (!allow_lds(k1, C::LDS_DQ) || !allow_lds(k2, C::LDS_KV)) return FA_ERR_HIP;
  FA_LOG_LAUNCH("fa_bwd_dq_wide<D=%d D_v=%d causal=%d varlen=%d>: %lld workgroups x %d threads, "
                "%d B LDS; fa_bwd_dkdv_wide: %lld workgroups x %d threads, %d B LDS, %d column "
                "parts; B=%d H=%d H_kv=%d S_q=%d S_k=%d",
                D, C::DV, (int)CAUSAL, (int)VARLEN, g1, C::NW * kWave, C::LDS_DQ, g2,
                C::NW * kWave, C::LDS_KV, C::DSPLIT, a.B, a.H, a.Hkv, a.S, a.Sk);
  hipLaunchKernelGGL(k1, dim3((unsigned)g1), dim3(C::NW * kWave), C::LDS_DQ, st, a);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  hipLaunchKernelGGL(k2, dim3((unsigned)g2), dim3(C::NW * kWave), C::LDS_KV, st, a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int D>
int dispatch_bwd_wide(const BwdArgs &a, bool causal, bool varlen, hipStream_t st) {
  if (causal)
    return varlen ? launch_bwd_wide<D, true, true>(a, st) : launch_bwd_wide<D, true, false>(a, st);
  return varlen ? launch_bwd_wide<D, false, true>(a, st) : launch_bwd_wide<D, false, false>(a, st);
}

template <int D>
int dispatch_bwd(const BwdArgs &a, bool causal, bool varlen, hipStream_t st) {
  if (causal) return varlen ? launch_bwd<D, true, true>(a, st) : launch_bwd<D, true, false>(a, st);
  return varlen ? launch_bwd<D, false, true>(a, st) : launch_bwd<D, false, false>(a, st);
}

}  // namespace

extern "C" {

int fa_bwd_hd(const void *q, const void *k, const void *v, const void *o, const void *dout,
              const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H,
              int H_kv, int S_q, int S_k, int D, int D_v, float scale, int causal,
              const int *cu_seqlens_q, const int *cu_seqlens_k, void *stream) {
  int rc = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H_kv, S_q, S_k, D, D_v,
                        scale, causal, cu_seqlens_q, cu_seqlens_k);
  if (rc != FA_OK) return rc;
  DeviceInfo *dev = nullptr;
  rc = current_device(&dev);
  if (rc != FA_OK) return rc;
  BwdArgs a;
  a.q = (const __bf16 *)q;
  a.k = (const __bf16 *)k;
  a.v = (const __bf16 *)v;
  a.o = (const __bf16 *)o;
  a.dout = (const __bf16 *)dout;
  a.lse = lse;
  a.dq = (__bf16 *)dq;
  a.dk = (__bf16 *)dk;
  a.dv = (__bf16 *)dv;
  a.delta = delta;
  a.cu = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.B = B;
  a.H = H;
  a.Hkv = H_kv;
  a.S = S_q;
  a.Sk = S_k;
  a.c = scale * kLog2e;
  a.scale = scale;
  hipStream_t st = (hipStream_t)stream;
  const bool varlen = cu_seqlens_q != nullptr;
  switch (D) {
    case 64: return dispatch_bwd<64>(a, causal, varlen, st);
    case 128: return dispatch_bwd<128>(a, causal, varlen, st);
    case 192: return dispatch_bwd_wide<192>(a, causal, varlen, st);
    default: return dispatch_bwd_wide<256>(a, causal, varlen, st);
  }
}

int fa_bwd_general(const void *q, const void *k, const void *v, const void *o, const void *dout,
                   const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H,
                   int H_kv, int S_q, int S_k, int D, float scale, int causal,
                   const int *cu_seqlens_q, const int *cu_seqlens_k, void *stream) {
  return fa_bwd_hd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H_kv, S_q, S_k, D, D, scale,
                   causal, cu_seqlens_q, cu_seqlens_k, stream);
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H, int H_kv,
           int S, int D, float scale, int causal, const int *cu_seqlens, void *stream) {
  return fa_bwd_general(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H_kv, S, S, D, scale,
                        causal, cu_seqlens, cu_seqlens, stream);
}

}  // extern "C"
