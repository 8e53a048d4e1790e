// fa_tile.h -- device-side building blocks shared by the attention kernels
// for gfx950: operand types, the 16-byte-chunk LDS swizzle, the
// global->LDS block loader, the MFMA operand reads from LDS and a few wave
// primitives.  Everything here is header-only and internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kBN = 64;           // keys per KV block
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;


__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one held 32 lanes away (the other half-wave).
// v_permlane32_swap(v, v) exchanges the upper half of its first operand with
// the lower half of its second: lanes 0-31 get {own, partner} and lanes
// 32-63 get {partner, own}, so the symmetric combination of both results is
// the same on the two lanes of a pair.
__device__ __forceinline__ float max_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Race-check builds (compiled with FA_SYNC_DEBUG; a second library used only
// to test this one): every wait below drains every counter, every barrier
// drains them first, each wave waits for its global->LDS copies right after
// issuing them, and the ping-pong body adds a barrier between its two
// phases.  Such a build computes the same values in the same order, so its
// results must equal the pipelined build's bit for bit; a copy that is read
// before it lands or overwritten while still being read would show as a
// difference.
#ifdef FA_SYNC_DEBUG
constexpr bool kSyncDebug = true;
#else
constexpr bool kSyncDebug = false;
#endif

__device__ __forceinline__ void drain_all() {
  asm volatile("s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)" ::: "memory");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (kSyncDebug) {
    drain_all();
  } else {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  }
}

// Workgroup barrier without a memory fence.  __syncthreads() would also wait
// for every outstanding global->LDS copy (vmcnt(0)), including the next
// block's prefetch; the copies this barrier must cover are waited for
// explicitly with wait_vmcnt<>() first.  The "memory" clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  if constexpr (kSyncDebug) drain_all();
  asm volatile("s_barrier" ::: "memory");
}

// Barrier after this wave's LDS reads of a buffer have all returned, so no
// read is still queued when another wave's copy starts overwriting it.
__device__ __forceinline__ void barrier_after_reads() {
  if constexpr (kSyncDebug) drain_all();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A barrier that only race-check builds have (between the ping-pong phases;
// every wave passes the same number of them).
__device__ __forceinline__ void debug_phase_barrier() {
  if constexpr (kSyncDebug) {
    drain_all();
    asm volatile("s_barrier" ::: "memory");
  }
}

// 16-byte chunk swizzle of an LDS row: chunk c of row r lives at c ^ swz(r).
// For D >= 128 (rows of 16+ chunks) rows r..r+15 get distinct values (bank
// spread for the K operand reads, 16 rows x one chunk) and rows 4a..4a+3
// differ in bits 2-3 (spread for the transposed V reads, 4 rows x 4 chunks).
// For D = 64 (8 chunks, two rows per 256 bytes) the same two properties hold
// on the row-pair level.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Kernel instances are named by the q/k head dimension D; the v/o head
// dimension DV equals D except for D = 192, which is the (192, 128) pair the
// FlashAttention-4 paper benchmarks for DeepSeek V3 (section 5.1).
template <int D>
constexpr int head_dim_v() { return D == 192 ? 128 : D; }

// Issue the global->LDS copies of one K or V block (this wave's share).
// LDS slot p (16 bytes) of the block holds row p / CPR, physical chunk
// p % CPR, i.e. logical chunk (p % CPR) ^ swz(row).  The copies are issued
// from inline assembly so that the compiler does not track them: it would
// otherwise wait for every outstanding copy (including the prefetch of the
// next block) before any LDS read it cannot prove disjoint.  Completion is
// waited for explicitly with wait_vmcnt<>(), which is exact because the
// vector-memory counter retires loads in issue order.
template <int W, int NW>
struct BlockLoader {
  // Rows are W bf16 wide; W = 192 rows are stored as two LDS parts: chunks
  // 0-15 of every row in a 128-wide layout (16 KiB, slots 0..1023) and
  // chunks 16-23 in a 64-wide layout (8 KiB, slots 1024..1535), so that each
  // part keeps the power-of-two row pitch the operand addressing relies on.
  static constexpr int CPR = W / 8;                           // 16-byte chunks per row
  static constexpr int LOADS = (kBN * CPR) / (NW * kWave);    // per wave
  static_assert(LOADS * NW * kWave == kBN * CPR, "block must split evenly over waves");
  static_assert(W != 192 || (1024 % (NW * kWave)) == 0, "no copy may straddle the two parts");
  unsigned voff[LOADS];  // byte offset of this lane's 16-byte chunk from the block's first row
  unsigned row_bytes;    // Hk*W*2: distance between consecutive tokens of a head
  int wave, lane;

  __device__ __forceinline__ int slot0(int i) const { return (i * NW + wave) * kWave; }
  // Slot p of the block -> (row, logical chunk).
  static __device__ __forceinline__ void row_chunk(int p, int &row, int &c) {
    if constexpr (W == 192) {
      if (p < 1024) {
        row = p / 16;
        c = (p % 16) ^ swz<128>(row);
      } else {
        const int q = p - 1024;
        row = q / 8;
        c = 16 + ((q % 8) ^ swz<64>(row));
      }
    } else {
      row = p / CPR;
      c = (p % CPR) ^ swz<W>(row);
    }
  }
  __device__ __forceinline__ int row_of(int i) const {
    int row, c;
    row_chunk(slot0(i) + lane, row, c);
    return row;
  }
  // Copy i goes to the second part of a W = 192 block (compile-time: the
  // copies of one index i cover slots i*NW*64 .. (i+1)*NW*64-1 over the waves).
  static constexpr bool second_part(int i) { return W == 192 && i * NW * kWave >= 1024; }

  __device__ __forceinline__ void init(int Hk, int wave_, int lane_) {
    wave = __builtin_amdgcn_readfirstlane(wave_);
    lane = lane_;
    row_bytes = (unsigned)Hk * (unsigned)W * 2u;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int row, c;
      row_chunk(slot0(i) + lane, row, c);
      voff[i] = (unsigned)row * row_bytes + (unsigned)c * 16u;
    }
  }

  // One 16-byte-per-lane copy: global (SGPR base + 32-bit lane offset) -> LDS
  // at m0 + 16*lane.
  static __device__ __forceinline__ void dma16(const char *blk, unsigned voff_, unsigned lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds_addr), "v"(voff_), "s"(blk)
        : "memory", "m0");
  }

  // LDS byte address of this wave's copy I in the block at dst (dst2: the
  // second part of a W = 192 block).
  template <int I>
  __device__ __forceinline__ unsigned lds_slot(unsigned dst, unsigned dst2) const {
    return second_part(I) ? dst2 + (unsigned)(slot0(I) - 1024) * 16u
                          : dst + (unsigned)slot0(I) * 16u;
  }

  // Row 0 of one (sequence, K/V head): the per-tile base of issue_at.
  static __device__ __forceinline__ const char *seq_base(const __bf16 *base, long long tok0,
                                                         int Hk, int hk) {
    return (const char *)(base + (tok0 * Hk + hk) * (long long)W);
  }

  // Copy this wave's chunks of rows n0 .. n0+BN-1 of the (sequence, head)
  // whose row 0 is at seq into the LDS block dst (dst2: its second part,
  // W = 192).  Rows at or past L read row L-1 instead (in bounds; masked
  // later).  The block address and the full-block test are computed once per
  // block on scalars, so a copy costs one m0 write and the load: the scalar
  // unit is shared by every wave of the CU, and per-copy address arithmetic
  // and branches used to hold the issuing wave for hundreds of cycles.
  __device__ __forceinline__ void issue_at(const char *seq, int n0, int L, char LDS_AS *dst,
                                           char LDS_AS *dst2 = nullptr) const {
    const char *blk = seq + (long long)n0 * row_bytes;
    const unsigned d0 = (unsigned)(uintptr_t)dst, d1 = (unsigned)(uintptr_t)dst2;
    if (n0 + kBN <= L) {
      issue_full(blk, d0, d1, std::make_integer_sequence<int, LOADS>{});
    } else {
      issue_tail(blk, d0, d1, L - 1 - n0, std::make_integer_sequence<int, LOADS>{});
    }
    if constexpr (kSyncDebug) drain_all();
  }
  template <int... I>
  __device__ __forceinline__ void issue_full(const char *blk, unsigned d0, unsigned d1,
                                             std::integer_sequence<int, I...>) const {
    (dma16(blk, voff[I], lds_slot<I>(d0, d1)), ...);
  }
  // last = L-1-n0 >= 0 (blocks start below L): rows past it read row last.
  template <int... I>
  __device__ __forceinline__ void issue_tail(const char *blk, unsigned d0, unsigned d1, int last,
                                             std::integer_sequence<int, I...>) const {
    (dma16(blk, voff[I] - (unsigned)(row_of(I) - (row_of(I) < last ? row_of(I) : last)) * row_bytes,
           lds_slot<I>(d0, d1)),
     ...);
  }
  // All of this wave's chunks of rows n0 .. n0+BN-1 of one (sequence, head).
  __device__ __forceinline__ void issue(const __bf16 *base, long long tok0, int Hk, int hk, int n0,
                                        int L, char LDS_AS *dst,
                                        char LDS_AS *dst2 = nullptr) const {
    issue_at(seq_base(base, tok0, Hk, hk), n0, L, dst, dst2);
  }
};

// LDS operand addressing.  With the swizzle above, the byte offset of the
// K operand of lane l for sub-block kb and k-step s is
//   row*2D + ((2s + h) ^ swz(row)) * 16,   row = 32kb + l%32, h = l/32,
// and since 2s occupies other bits than h and swz(row) = swz(l%32), this is
//   ((KY + buf) ^ 32s) + kb*32*2D   with the per-lane constant
//   KY = (l%32)*2D | (16h ^ 16 swz(l%32)).
// (This needs the K/V buffers to start at multiples of 2D*64 bytes of LDS:
// the kernels declare no static LDS, so the dynamic allocation starts at 0.)
// Likewise the transposed V read r (r = 0, 1) for 16-key step t and d tile
// dt is ((VW_r + buf) ^ 64dt) + t*16*2D.  Buffers start at multiples of
// 2D*64 bytes, so adding the buffer base commutes with the XOR.  Each read
// is then one v_xor plus an instruction offset, with three base registers.
// For D = 192 the K layout has two parts (128- and 64-wide, see
// BlockLoader): k-steps 0-7 read the first with KY, k-steps 8-11 the second
// with KY2 (each part's own pitch and swizzle).  V uses the DV-wide layout.
template <int W>
__device__ __forceinline__ unsigned k_lane_const(int lane) {
  const int row = lane & 31, h = lane >> 5;
  return (unsigned)(row * (2 * W)) | (unsigned)((16 * h) ^ (swz<W>(row) << 4));
}

template <int D>
struct LdsAddr {
  static constexpr int KW = (D == 192) ? 128 : D;  // pitch of the (first) K part
  static constexpr int DV = head_dim_v<D>();
  unsigned ky, ky2, vw0, vw1;
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5;
    ky = k_lane_const<KW>(lane);
    ky2 = (D == 192) ? k_lane_const<64>(lane) : 0u;
    const int j = lane & 15, g = lane >> 4;
    const int cl = 2 * (g & 1) + ((j & 3) >> 1);
    unsigned w[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int kk = 4 * h + (j >> 2) + 8 * r;
      const int sw = swz<DV>(kk);
      const int z = ((sw & ~3) << 4) | ((cl ^ (sw & 3)) << 4);
      w[r] = (unsigned)(kk * (2 * DV)) | (unsigned)z | (unsigned)((j & 1) * 8);
    }
    vw0 = w[0];
    vw1 = w[1];
  }
};

__device__ __forceinline__ unsigned lds_u32(const char LDS_AS *p) { return (unsigned)(uintptr_t)p; }

// K operand (A of S^T = K Q^T) for key sub-block kb, k-step s of a W-wide
// layout; ka = KY + buffer.
template <int W>
__device__ __forceinline__ bf16x8 read_k(unsigned ka, int kb, int s) {
  const unsigned addr = (ka ^ (unsigned)(32 * s)) + (unsigned)(kb * 32 * 2 * W);
  return *(const bf16x8 LDS_AS *)(uintptr_t)addr;
}
// k-step s of a D-instance K block: ka addresses the first part, ka2 the
// second part of a D = 192 block.
template <int D>
__device__ __forceinline__ bf16x8 read_k_step(unsigned ka, unsigned ka2, int kb, int s) {
  if constexpr (D == 192) {
    if (s >= 8) return read_k<64>(ka2, kb, s - 8);
    return read_k<128>(ka, kb, s);
  } else {
    return read_k<D>(ka, kb, s);
  }
}

// V^T operand (A of O^T += V^T P^T) for 16-key step t and 32-wide d tile dt:
// lane l gets d = 32*dt + l%32 and keys 16t + 4h + {0..3}, 16t + 8 + 4h + {0..3}
// (h = l/32), matching the key order of the P operand taken from the S
// accumulator layout.  Within a 16-lane group the transposed read hands lane
// i element i%4 of the rows supplied by lanes 4e + i/4, so lane j supplies
// key (j/4) and d-quad (j%4) of its group's 16 d values.  va_r = VW_r + buffer.
template <int D>
__device__ __forceinline__ bf16x8 read_vt(unsigned va0, unsigned va1, int t, int dt) {
  const unsigned off = (unsigned)(t * 16 * 2 * D);
  const unsigned p0 = (va0 ^ (unsigned)(64 * dt)) + off;
  const unsigned p1 = (va1 ^ (unsigned)(64 * dt)) + off;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(uintptr_t)p0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(uintptr_t)p1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace
