// fa_sched.h -- tile order for the persistent attention kernel (host and device).
//
// A tile is (sequence b, head h, m-block mb): BM query rows of one head.  The
// persistent kernel launches a fixed number of workgroups ("workers"); each
// walks a static list of tiles.  The order follows the FlashAttention-4
// paper, section 3.3 (scheduling):
//   - longest-processing-time first: for causal masking the m-blocks are
//     visited in reverse, so the tiles with the most KV blocks start first;
//     for variable-length batches the sequences are sorted by length
//     (a virtual -> actual sequence map), longest first;
//   - heads innermost within an m-block level, so the tiles running at the
//     same time on one L2 share the same K/V;
//   - heads are split across the 8 XCDs (each with its own L2) when H is a
//     multiple of 8: XCD x owns heads x, x+8, ...; workgroup w runs on XCD
//     w % 8 because the dispatcher deals workgroups to XCDs round-robin.
//     With grouped-query attention (G = H / Hkv query heads per K/V head)
//     and Hkv a multiple of 8, XCD x owns the K/V heads x, x+8, ... and all
//     G query heads of each, visited one K/V head at a time (every query
//     head of one K/V head before the next, as the paper's section 3.3
//     orders grouped-query tiles), so a K/V head is read into one L2 only.
// Within an XCD, workers take positions W at a time (one round).  Dense
// batches, whose rounds hold tiles of equal cost, pair them in "snake"
// order: round r gives worker w position r*W + w on even rounds and
// r*W + W-1-w on odd rounds.  Varlen causal batches (and dense causal
// batches with split levels), whose rounds mix costs
// (chunks of levels, idle positions), pair them greedily: the round's
// costliest position goes to the worker with the least accumulated cost
// (greedy_round; host model on the 16-sequence batch: the busiest worker
// 1.064x the mean with the snake, 1.00x greedily).
//
// Item order (an item is (b, mb); heads are expanded innermost):
//   causal   : level l = 0..nmb_max-1 is m-block nmb_max-1-l; a level holds
//              the sequences with more than that many m-blocks, in sorted
//              order (for dense inputs: every sequence).
//   noncausal: sequences in sorted order, each with its m-blocks ascending.
//   varlen causal self-attention: the levels are taken in chunks of `sub`
//              consecutive levels, and an item is (sequence, chunk): the
//              sequence's m-blocks of those levels, then heads innermost.
//              Ordering one level at a time makes the tiles that run
//              together on an XCD belong to different sequences, each
//              streaming its own K/V past the L2 (measured on a 16-sequence
//              batch: a 23% L2 hit rate, every K/V block fetched from HBM;
//              with chunks of 8: 41%, 25% less traffic).  With chunks, the
//              sub m-blocks x hpg heads of one sequence run together and
//              share their K/V stream, as the m-blocks of a dense batch do.
//              LPT holds from chunk to chunk; inside a chunk the tile costs
//              differ by at most sub-1 m-blocks.  A level that a sequence
//              does not reach is an idle position, which the worker skips.
//   varlen causal with key lengths of their own (bottom-right aligned): a
//              query tile sees nearly all of its sequence's keys, so its
//              cost follows the key length, not the m-block.  Sequences are
//              sorted by key length, each with its m-blocks descending
//              (host model on a 16-sequence mixed batch: makespan 1.08x the
//              ideal, against 1.43x for the level order).
//
//   dense causal with split levels: when a batch has few tiles, its
//              costliest m-blocks outlast the mean worker load (B=2, H=16,
//              S=2048: 32 key blocks against a mean of 18).  The nsplit
//              costliest m-blocks then run as two parts, each over one half
//              of the tile's key blocks (part 1 the first floor(n/2), part 2
//              the rest with the diagonal), on workers of their own; the part
//              that finishes second merges the two partial results.  A
//              "virtual level" is an (m-block, part) pair; the levels are
//              ordered by cost (descending) and paired with the workers in
//              greedy rounds.
//
// The same code builds the tables on the host (tid = 0, nth = 1) for
// fa_schedule() and in LDS on the device (tid = thread, nth = block size,
// with a barrier between phases).
#pragma once

#ifndef FA_HD
#define FA_HD __host__ __device__
#endif

namespace fa {

constexpr int kXcds = 8;
constexpr int kMaxVarlenSeqs = 1024;     // persistent varlen table limit (B)
constexpr int kMaxVarlenLevels = 2048;   // persistent varlen table limit (nmb_max)
constexpr int kMaxSplitLevels = 64;      // virtual levels (m-blocks + split parts) of a dense split schedule

struct SchedTables {
  int *len;        // [B] clamped (query) sequence lengths
  int *sorted;     // [B] sequence index by rank (sort key descending, index ascending)
  int *off;        // [nlev + 1] (causal: level-chunk offsets) or [B + 1] (rank offsets)
  int *key;        // [B] sort key: key lengths (by_klen), else the same as len
  int *vl;         // [nvl] dense split schedule: virtual level by rank, mb | part << 16
};

struct Sched {
  int B, H, S, BM;
  int G;           // query heads per K/V head (1: multi-head attention)
  int kv_grouped;  // XCD groups follow K/V heads (Hkv a multiple of the group count)
  int causal, varlen;
  int by_klen;     // varlen causal with key lengths of their own: rank order by key length
  int nmb_max;     // ceil(S / BM)
  int sub;         // levels per item (varlen causal chunks; 1 otherwise)
  int nlev;        // level chunks: ceil(nmb_max / sub)
  int groups;      // kXcds or 1
  int hpg;         // heads per group
  int n_items;     // number of (b, mb) items
  int nsplit;      // dense causal: the nsplit costliest m-blocks run as two parts (0: none)
  int nvl;         // dense causal: virtual levels, nmb_max + nsplit
};

FA_HD inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// self_attn: the query and key lengths of every sequence are equal (the
// level chunks of varlen causal batches apply only then: with key lengths of
// their own a tile's cost follows its key length rather than its m-block).
FA_HD inline Sched make_sched(int B, int H, int Hkv, int S, int BM, int causal, int varlen,
                              int workers, int self_attn = 1, int nsplit = 0) {
  Sched s;
  s.B = B; s.H = H; s.S = S; s.BM = BM; s.causal = causal; s.varlen = varlen;
  s.G = H / Hkv;
  s.nmb_max = ceil_div(S, BM);
  s.groups = (H % kXcds == 0 && workers % kXcds == 0) ? kXcds : 1;
  s.kv_grouped = (Hkv % s.groups == 0);
  s.hpg = H / s.groups;
  s.sub = 1;
  s.by_klen = varlen && causal && !self_attn;
  if (varlen && causal && self_attn) {
    // enough m-blocks of one sequence to fill an XCD's workers with its heads,
    // at most 8 (the cost spread inside a chunk)
    const int per_group = workers / s.groups;
    int k = per_group / s.hpg;
    s.sub = k < 1 ? 1 : (k > 8 ? 8 : k);
  }
  s.nlev = ceil_div(s.nmb_max, s.sub);
  s.nsplit = 0;
  s.nvl = s.nmb_max;
  if (!varlen && causal && nsplit > 0) {
    s.nsplit = nsplit < s.nmb_max ? nsplit : s.nmb_max;
    s.nvl = s.nmb_max + s.nsplit;
    if (s.nvl > kMaxSplitLevels) {  // not representable: no split
      s.nsplit = 0;
      s.nvl = s.nmb_max;
    }
  }
  s.n_items = B * s.nvl;  // dense; varlen fills it from the tables
  return s;
}

// ---- dense causal split levels ----

// Key blocks (of 64) of part `part` of m-block mb in a dense causal
// self-attention batch: part 0 is the whole key range of the tile, part 1
// its first floor(n/2) blocks, part 2 the other ceil(n/2).
FA_HD inline int split_blocks(const Sched &s, int mb, int part) {
  const int e = (mb + 1) * s.BM;
  const int n = ceil_div(e < s.S ? e : s.S, 64);
  return part == 0 ? n : (part == 1 ? n / 2 : n - n / 2);
}
// Doubled cost (as tile_cost2) of a part; a split part adds the exchange
// of its partial rows (written through to memory, counted, and for one of
// the two parts read back and merged), measured at about nine key blocks'
// time on B=1, H=16, S=2048.
constexpr int kSplitMergeCost2 = 18;
FA_HD inline int split_cost2(const Sched &s, int mb, int part) {
  return 2 * split_blocks(s, mb, part) + 5 + (part ? kSplitMergeCost2 : 0);
}
// Virtual level i in natural order: the unsplit m-blocks 0 .. nmb-nsplit-1,
// then both parts of each split m-block.  Code: mb | part << 16.
FA_HD inline int split_natural(const Sched &s, int i) {
  const int nfull = s.nmb_max - s.nsplit;
  if (i < nfull) return i;
  const int j = i - nfull;
  return (nfull + j / 2) | ((1 + (j & 1)) << 16);
}
// vl[rank] = the virtual level of that cost rank (cost descending, ties:
// natural order).
FA_HD inline void split_levels(const Sched &s, int *vl, int tid, int nth) {
  for (int i = tid; i < s.nvl; i += nth) {
    const int ci = split_natural(s, i);
    const int cost_i = split_cost2(s, ci & 0xffff, ci >> 16);
    int rank = 0;
    for (int k = 0; k < s.nvl; ++k) {
      const int ck = split_natural(s, k);
      const int cost_k = split_cost2(s, ck & 0xffff, ck >> 16);
      rank += (cost_k > cost_i) || (cost_k == cost_i && k < i);
    }
    vl[rank] = ci;
  }
}

// ---- varlen table construction, in phases (barrier between phases) ----

// Phase 1: clamped lengths and sort keys (cu_k: key offsets, read when by_klen).
FA_HD inline void tables_phase1(const Sched &s, const int *cu, const int *cu_k, SchedTables t,
                                int tid, int nth) {
  for (int b = tid; b < s.B; b += nth) {
    int L = cu[b + 1] - cu[b];
    L = L < 0 ? 0 : (L > s.S ? s.S : L);
    t.len[b] = L;
    if (s.by_klen) {
      const int Lk = cu_k[b + 1] - cu_k[b];
      t.key[b] = Lk < 0 ? 0 : Lk;
    }
  }
}

// Phase 2: rank of each sequence (sort key descending, index ascending).
FA_HD inline void tables_phase2(const Sched &s, SchedTables t, int tid, int nth) {
  const int *key = s.by_klen ? t.key : t.len;
  for (int b = tid; b < s.B; b += nth) {
    const int Lb = key[b];
    int rank = 0;
    for (int c = 0; c < s.B; ++c) {
      const int Lc = key[c];
      rank += (Lc > Lb) || (Lc == Lb && c < b);
    }
    t.sorted[rank] = b;
  }
}

// Phase 3: per-chunk of levels (causal) or per-rank (noncausal) item counts
// into off[i+1].  A sequence has an item in chunk c when it reaches the
// chunk's last level, i.e. has more m-blocks than that level's m-block.
FA_HD inline void tables_phase3(const Sched &s, SchedTables t, int tid, int nth) {
  if (s.causal && !s.by_klen) {
    for (int c = tid; c < s.nlev; c += nth) {
      const int last = (c + 1) * s.sub < s.nmb_max ? (c + 1) * s.sub - 1 : s.nmb_max - 1;
      const int mb = s.nmb_max - 1 - last;
      int cnt = 0;
      for (int r = 0; r < s.B; ++r) cnt += ceil_div(t.len[t.sorted[r]], s.BM) > mb;
      t.off[c + 1] = cnt;
    }
  } else {
    for (int r = tid; r < s.B; r += nth) t.off[r + 1] = ceil_div(t.len[t.sorted[r]], s.BM);
  }
  if (tid == 0) t.off[0] = 0;
}

// Phase 4 (one thread): inclusive prefix sum; returns the item count.
FA_HD inline int tables_phase4(const Sched &s, SchedTables t) {
  const int n = (s.causal && !s.by_klen) ? s.nlev : s.B;
  for (int i = 0; i < n; ++i) t.off[i + 1] += t.off[i];
  return t.off[n];
}

// ---- decode ----

struct Tile {
  int b, h, mb;
  int part;  // 0: the whole tile; 1, 2: a part of a split m-block
};

// Item index and level j within it (0 <= j < sub) -> (b, mb); b = -1 for a
// level the sequence does not reach (an idle position).
FA_HD inline void decode_item(const Sched &s, const SchedTables &t, int it, int j, int *b,
                              int *mb, int *part) {
  *part = 0;
  if (!s.varlen) {
    if (s.causal) {
      const int l = it / s.B;
      *b = it - l * s.B;
      if (s.nsplit > 0) {
        const int c = t.vl[l];
        *mb = c & 0xffff;
        *part = c >> 16;
      } else {
        *mb = s.nmb_max - 1 - l;
      }
    } else {
      *b = it / s.nmb_max;
      *mb = it - *b * s.nmb_max;
    }
    return;
  }
  const int n = (s.causal && !s.by_klen) ? s.nlev : s.B;
  int lo = 0, hi = n;  // find the last i with off[i] <= it
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (t.off[mid] <= it) lo = mid; else hi = mid;
  }
  const int r = it - t.off[lo];
  if (s.causal && !s.by_klen) {
    const int lev = lo * s.sub + j;
    const int m = s.nmb_max - 1 - lev;
    const int bb = t.sorted[r];
    const bool has = lev < s.nmb_max && m < ceil_div(t.len[bb], s.BM);
    *b = has ? bb : -1;
    *mb = m;
  } else {
    *b = t.sorted[lo];
    // causal (by key length): m-blocks descending; noncausal: ascending
    *mb = s.by_klen ? t.off[lo + 1] - t.off[lo] - 1 - r : r;
  }
}

// Position p (within group x's list) -> tile; tl.b = -1: idle position.
FA_HD inline Tile decode_position(const Sched &s, const SchedTables &t, int x, int p) {
  Tile tl;
  const int per = s.sub * s.hpg;
  const int it = p / per;
  const int rem = p - it * per;
  const int j = rem / s.hpg;
  const int hi = rem - j * s.hpg;
  decode_item(s, t, it, j, &tl.b, &tl.mb, &tl.part);
  if (s.kv_grouped) {
    // hi -> (K/V head x + groups*kvl, query head g of it); g innermost
    const int kvl = hi / s.G;
    tl.h = (x + s.groups * kvl) * s.G + (hi - kvl * s.G);
  } else {
    tl.h = x + s.groups * hi;
  }
  return tl;
}

// Number of positions in each group's list.
FA_HD inline int group_positions(const Sched &s) { return s.n_items * s.sub * s.hpg; }

// Worker -> (group, index within group, workers in group).
FA_HD inline void worker_slot(const Sched &s, int worker, int workers, int *x, int *w, int *W) {
  *x = worker % s.groups;
  *w = worker / s.groups;
  *W = workers / s.groups;
}

// Snake position of worker w (of W) in round r.
FA_HD inline int snake_position(int r, int w, int W) {
  return r * W + ((r & 1) ? (W - 1 - w) : w);
}

// ---- greedy rounds (varlen causal batches, dense causal split levels) ----
constexpr int kGreedyMaxW = 64;  // one lane per worker of a group on the device
FA_HD inline bool greedy_rounds(const Sched &s, int W) {
  return s.causal && (s.varlen || s.nsplit > 0) && W <= kGreedyMaxW;
}

// Doubled cost of a tile: two per 64-key block it reads, plus 5 for its
// fixed part (about 2.5 blocks: the pipeline's fill and drain and the
// epilogue).  The key range follows the kernel's causal bound.
FA_HD inline int tile_cost2(const Sched &s, const SchedTables &t, const Tile &tl) {
  if (!s.varlen) return split_cost2(s, tl.mb, tl.part);
  const int L = t.len[tl.b];
  const int Lk = s.by_klen ? t.key[tl.b] : L;
  const int e = tl.mb * s.BM + s.BM + (Lk - L);
  const int n_end = e < 0 ? 0 : (e < Lk ? e : Lk);
  return 2 * ceil_div(n_end, 64) + 5;
}

// Cost of position p of group x: > 0 for a tile, 0 for an idle position,
// -1 past the end of the list.
FA_HD inline int position_cost2(const Sched &s, const SchedTables &t, int x, int p, int npos) {
  if (p >= npos) return -1;
  const Tile tl = decode_position(s, t, x, p);
  return tl.b < 0 ? 0 : tile_cost2(s, t, tl);
}

// Whether position i of a round goes before position k (cost descending,
// ties: lower index), and whether worker i's load ranks before worker k's
// (ascending, ties: lower index).
FA_HD inline bool cost_before(int ci, int i, int ck, int k) { return ci > ck || (ci == ck && i < k); }
FA_HD inline bool load_before(int li, int i, int lk, int k) { return li < lk || (li == lk && i < k); }

// One greedy round on the host: take[w] = the position worker w takes in
// round r (-1: none), load[] updated.  The device computes the same
// assignment with one lane per worker (fa_fwd_persistent).
inline void greedy_round(const Sched &s, const SchedTables &t, int x, int r, int W, int npos,
                         int *load, int *take) {
  int cost[kGreedyMaxW], by_cost[kGreedyMaxW], by_load[kGreedyMaxW];
  for (int i = 0; i < W; ++i) cost[i] = position_cost2(s, t, x, r * W + i, npos);
  for (int i = 0; i < W; ++i) {
    int rc = 0, rl = 0;
    for (int k = 0; k < W; ++k) {
      rc += cost_before(cost[k], k, cost[i], i);
      rl += load_before(load[k], k, load[i], i);
    }
    by_cost[rc] = i;
    by_load[rl] = i;
  }
  for (int q = 0; q < W; ++q) {
    const int w = by_load[q], i = by_cost[q];
    take[w] = cost[i] > 0 ? r * W + i : -1;
    if (cost[i] > 0) load[w] += cost[i];
  }
}

}  // namespace fa
