/*
 * fa.h -- C ABI of the MI355X (gfx950) exact attention forward library
 * (libfa_mi355x.so).
 *
 * The operation is the one the FlashAttention-4 pages centre on: exact
 * multi-head attention forward, O = softmax(scale * Q K^T + causal mask) V,
 * computed in tiles with an online softmax so the S x S score matrix never
 * reaches device memory (FlashAttention-4 paper, sections 1, 2.1 and 3.1;
 * the usage guide's "what it is" section).  Each row's natural-log
 * logsumexp is returned as well.
 *
 * Conventions shared by every entry point:
 *   - Device pointers are allocated, owned and freed by the caller.  The
 *     library keeps no pointer after a call returns, apart from work it has
 *     enqueued on the caller's stream, and allocates no device memory.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Every call is asynchronous: it enqueues kernels and returns without
 *     synchronising.  Results are valid once the stream has reached them.
 *   - Arguments are validated on the host before any HIP call, so a bad
 *     argument is reported without touching the GPU.  No call aborts or
 *     throws; each returns an fa_status.
 *   - Calls are thread-safe; concurrent calls on different streams are
 *     independent.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Diagnostics: with the environment variable FA_LOG set to a value other
 * than "" or "0" when the library first launches a kernel, every launch
 * writes one line to stderr: "[fa] " followed by the kernel variant, its
 * grid and LDS bytes, and the sizes it covers.
 */

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size, bad scale, ... */
    FA_ERR_UNSUPPORTED = -2,   /* valid request this build does not implement (e.g. D) */
    FA_ERR_HIP = -3,           /* a HIP runtime call or kernel launch failed */
    FA_ERR_NO_DEVICE = -4,     /* no gfx950 device is current */
    FA_ERR_TOO_LARGE = -5      /* the sizes need more than a fixed scratch buffer holds */
} fa_status;

/*
 * fa_fwd -- exact attention forward.
 *
 * Computes, for every sequence b, head h and query row i,
 *   s_ij   = scale * <q_i, k_j>  for the allowed keys j
 *            (all j < L_b; with causal=1 only j <= i, i.e. scores above the
 *            diagonal are masked as in the FlashAttention-4 paper,
 *            section 3.3, LPT scheduling for causal masking)
 *   o_i    = sum_j softmax_j(s_ij) v_j                        (bf16 output)
 *   lse_i  = ln sum_j exp(s_ij)                                (fp32 output)
 *
 * Layouts (row-major, contiguous, 16-byte aligned base pointers):
 *   dense  (cu_seqlens == NULL): q, k, v, o are bf16 [B, S, H, D];
 *                                lse is fp32 [B, H, S]
 *   varlen (cu_seqlens != NULL): q, k, v, o are bf16 [T, H, D] with
 *                                T = cu_seqlens[B]; lse is fp32 [H, T].
 *          Sequence b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 and
 *          attends within itself (query and key lengths are equal).  S is
 *          the maximum sequence length.  cu_seqlens is an int32 device array
 *          of B+1 entries; its contents are not read on the host, so the
 *          caller guarantees cu_seqlens[0] == 0, non-decreasing entries,
 *          every length <= S, and T matching the tensors.  (The kernel clamps
 *          each length to [0, S] to keep its own tables in bounds.)
 *
 * Arguments:
 *   q, k, v   read-only inputs; o, lse write-only outputs that must not alias
 *             the inputs.  lse may be NULL (not written).
 *   B, H, S   >= 1.  D in {64, 128, 256} (FA_ERR_UNSUPPORTED otherwise; the
 *             usage guide's interface limit is D <= 256).
 *   scale     finite and > 0 (1/sqrt(D) is the usual choice).
 *   causal    0 or 1.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_NO_DEVICE or
 * FA_ERR_HIP.  On an error nothing has been enqueued unless the error is
 * FA_ERR_HIP from the launch itself.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int S, int D, float scale, int causal,
           const int *cu_seqlens, void *stream);

/*
 * Experiment knobs for fa_fwd_ex.  fa_fwd uses fa_tuning_default().
 *
 *   tau        Rescale threshold in log2 units, 0 <= tau <= 64 (other
 *              values, NaN included, are FA_ERR_INVALID_ARG).  Each block's
 *              exponentials are computed against the running reference
 *              maximum as it stands; the reference is moved to the block
 *              maximum, and the output and row sums rescaled, only when
 *              some lane's share of the block's row sum exceeds 2^tau (so
 *              every exponential stays within 2^tau) or a row has no
 *              reference yet.  The decision is taken for the whole
 *              wavefront, so it never diverges (FlashAttention-4 paper,
 *              section 3.1.4, skipping online-softmax rescaling: the final
 *              normalisation corrects the skipped steps).  The result does
 *              not depend on tau; tau = 0 rescales whenever an exponential
 *              could exceed 1, i.e. on every growth of the maximum, as the
 *              textbook online softmax does.  Default 8 (factor 256).
 *   exp2_emu   Share of exponentials evaluated by the degree-3 polynomial
 *              instead of v_exp_f32 (paper section 3.1.3, partial emulation):
 *              0 = none, 8 = one column slot in 8 (12.5 %), 4 = one in 4
 *              (25 %).  Other values are FA_ERR_INVALID_ARG.
 *   schedule   0 = persistent workgroups walking the tiles in
 *              longest-processing-time-first order (paper section 3.3);
 *              1 = one workgroup per tile in natural (batch, head, m-block)
 *              order.  Both give bitwise identical results when no level is
 *              split (split_levels below).
 *   counters   NULL, or a device array of 2 uint64 that the call adds to:
 *              [0] wavefront-level rescale events, [1] wavefront-block steps
 *              (their ratio is the rescale rate).  Slower; for measurement.
 *   split_levels  Dense causal self-attention (no cu_seqlens, S_q = S_k)
 *              with D < 256 under schedule 0: the number of costliest
 *              m-block levels run
 *              as two parts, each over half of the tile's key blocks on a
 *              workgroup of its own, the second part to finish merging both
 *              partial results (O normalised per part and its LSE, combined
 *              by their LSE weights).  When a batch has few tiles, its
 *              last m-blocks, which read every key, otherwise outlast the
 *              mean worker load (B=2, H=16, S=2048: 32 key blocks against a
 *              mean of 18).  Each split tile exchanges its two parts'
 *              partial rows through memory, which costs about nine key
 *              blocks' time, so splitting pays only where workers would
 *              otherwise idle.  -1 = chosen by the library: only batches
 *              whose tiles leave at least half of the workers idle, and
 *              only as many levels as its makespan model finds shorten the
 *              busiest worker by 5% (B=1, H=8, S=3000: 19% faster; B=2,
 *              H=16, S=2048 stays whole), 0 = never,
 *              n > 0 = the n costliest (clamped to what the schedule holds:
 *              at most ceil(S/BM) levels and 64 levels in all); other
 *              values are FA_ERR_INVALID_ARG.  A split launch keeps a
 *              workspace per device and stream (counters and partial rows,
 *              up to 512 MiB), allocated on first need and kept until the
 *              process ends; when it cannot be allocated (or the stream is
 *              being captured into a graph and it would have to grow) the
 *              launch runs unsplit.  Results of split and unsplit launches
 *              differ by the fp32 rounding of the merge.  Default -1.
 */
typedef struct fa_tuning {
    float tau;
    int exp2_emu;
    int schedule;
    unsigned long long *counters;
    int split_levels;
} fa_tuning;

fa_tuning fa_tuning_default(void);

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int S, int D, float scale, int causal,
              const int *cu_seqlens, void *stream, const fa_tuning *tuning);

/*
 * fa_fwd_gqa -- grouped-query attention forward (the FlashAttention-4 paper,
 * section 3.3, reports its LPT scheduling results for MQA as well as MHA).
 *
 * Same operation, layouts, arguments and errors as fa_fwd_ex, except that k
 * and v carry H_kv heads:
 *   dense  k, v bf16 [B, S, H_kv, D];   varlen  k, v bf16 [T, H_kv, D]
 * while q, o and lse keep H heads.  H_kv >= 1 must divide H
 * (FA_ERR_INVALID_ARG otherwise); query head h reads K/V head
 * h / (H / H_kv), so each run of H/H_kv consecutive query heads shares one
 * K/V head.  H_kv = H is fa_fwd_ex itself, H_kv = 1 is multi-query attention.
 * tuning may be NULL (fa_tuning_default()).
 */
int fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int H, int H_kv, int S, int D, float scale, int causal,
               const int *cu_seqlens, void *stream, const fa_tuning *tuning);

/*
 * fa_fwd_hd -- fa_fwd_gqa with separate q/k and v/o head dimensions.
 *
 * q and k rows have D entries, v and o rows D_v entries:
 *   dense  q [B,S,H,D], k [B,S,H_kv,D], v [B,S,H_kv,D_v], o [B,S,H,D_v]
 *   varlen q [T,H,D],   k [T,H_kv,D],   v [T,H_kv,D_v],   o [T,H,D_v]
 * The scores use D (scale is typically 1/sqrt(D)); the output has D_v
 * columns.  Supported pairs: D = D_v in {64, 128, 256}, and (D, D_v) =
 * (192, 128), the DeepSeek V3 shape the FlashAttention-4 paper benchmarks
 * (section 5.1); anything else is FA_ERR_UNSUPPORTED.  fa_fwd_gqa is the
 * D_v = D case.
 */
int fa_fwd_hd(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int H_kv, int S, int D, int D_v, float scale, int causal,
              const int *cu_seqlens, void *stream, const fa_tuning *tuning);

/*
 * fa_fwd_general -- the complete parameter set: fa_fwd_hd with query and key
 * lengths that may differ (decode and mixed prefill/decode batches; the
 * FlashAttention-4 paper's section 3.3 motivates its varlen scheduling with
 * such batches).
 *
 *   dense  (both offsets NULL): q, o [B, S_q, H, .]; k, v [B, S_k, H_kv, .];
 *                               lse fp32 [B, H, S_q]
 *   varlen (both non-NULL):     q, o [T_q, H, .]; k, v [T_k, H_kv, .] with
 *          T_q = cu_seqlens_q[B], T_k = cu_seqlens_k[B]; lse fp32 [H, T_q].
 *          Sequence b has query tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *          and key tokens cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1; S_q and S_k
 *          are the longest lengths (the same trust rules as fa_fwd apply to
 *          both offset arrays).
 * With causal = 1 the mask is aligned to the bottom-right corner: with
 * lengths L_q and L_k, query i may use key j when j <= i + L_k - L_q, so the
 * last query sees every key (for L_q = L_k this is fa_fwd's j <= i).  A row
 * that may use no key (L_q > L_k and i < L_q - L_k, or L_k = 0) gets O = 0
 * and LSE = -inf.  One offset array NULL and the other not is
 * FA_ERR_INVALID_ARG.  fa_fwd_hd is the S_q = S_k, cu_seqlens_q =
 * cu_seqlens_k case.
 */
int fa_fwd_general(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int H_kv, int S_q, int S_k, int D, int D_v, float scale,
                   int causal, const int *cu_seqlens_q, const int *cu_seqlens_k, void *stream,
                   const fa_tuning *tuning);

/*
 * fa_fwd_splitkv -- fa_fwd_general with each key range split over
 * num_splits workgroups ("split-KV"), for batches with few query rows per
 * (sequence, head), such as decode steps, where one workgroup per query tile
 * would leave most of the GPU idle while it streams a long K/V range (the
 * FlashAttention-4 paper motivates its varlen scheduling with such mixed
 * prefill/decode batches, section 3.3).
 *
 * Each (query tile, split) covers consecutive blocks of 64 keys and writes
 * the softmax over its own keys, O_s (normalised) and LSE_s, into the
 * workspace; a second kernel merges them per row:
 *   LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * The result is the same attention as fa_fwd_general (up to rounding).
 *
 * Arguments are those of fa_fwd_general, plus:
 *   num_splits       1 .. 64; fewer are used when the longest key range has
 *                    fewer 64-key blocks (1 = fa_fwd_general, no workspace);
 *                    fa_splitkv_auto_splits suggests a count.
 *   workspace        caller-owned device scratch, 16-byte aligned, of at
 *                    least fa_splitkv_workspace_size(...) bytes; its
 *                    contents on entry do not matter, and it must not be
 *                    used by another call until this one has completed on
 *                    the stream.
 * Errors: as fa_fwd_general, plus FA_ERR_INVALID_ARG for num_splits out of
 * range or a missing, misaligned or too small workspace.
 */
int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int H_kv, int S_q, int S_k, int D, int D_v, float scale,
                   int causal, const int *cu_seqlens_q, const int *cu_seqlens_k,
                   int num_splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the partial results live in a fixed scratch array
 * that the library holds in each device's memory (FA_SPLITKV_SCRATCH_BYTES,
 * from the first call on a device until the process ends) instead of a
 * workspace argument.  The call allocates nothing; the caller passes inputs
 * and outputs as for fa_fwd_splitkv.
 *
 * Arguments and results are those of fa_fwd_splitkv without workspace and
 * workspace_bytes.  Errors: as fa_fwd_splitkv, plus FA_ERR_TOO_LARGE when
 * fa_splitkv_workspace_size(B, H, S_q, S_k, D_v, num_splits) exceeds
 * FA_SPLITKV_SCRATCH_BYTES (nothing is enqueued then), and FA_ERR_HIP when
 * the scratch address cannot be obtained.
 *
 * All calls on one device share its scratch array: calls whose work can
 * overlap on that device (different streams, or host threads without
 * ordering) race and give wrong results.  Calls on one stream are ordered
 * and safe.  The scratch contents on entry do not matter.
 */
#define FA_SPLITKV_SCRATCH_BYTES ((size_t)16 << 20)
int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int H_kv, int S_q, int S_k, int D, int D_v,
                           float scale, int causal, const int *cu_seqlens_q,
                           const int *cu_seqlens_k, int num_splits, void *stream);

/* Workspace bytes fa_fwd_splitkv needs for these sizes (B, H, the longest
 * query and key lengths S_q and S_k, D_v) and num_splits: partial O and LSE,
 * fp32, for splits x B x S_q x H rows.  0 when no workspace is needed (one
 * split) or for invalid sizes. */
size_t fa_splitkv_workspace_size(int B, int H, int S_q, int S_k, int D_v, int num_splits);

/* A split count for these sizes on the current device: enough (tile,
 * split) pairs for one per CU (1 when the batch already has a query tile per
 * CU), at least two 64-key blocks per split.
 * Writes it to *splits_out; returns an fa_status. */
int fa_splitkv_auto_splits(int B, int H, int S_q, int S_k, int D, int *splits_out);

/* fa_splitkv_auto_splits for H_kv K/V heads (H_kv divides H).  When the rows
 * of a K/V group's query heads fit one tile (S_q * H/H_kv <= the row-tile
 * height), fa_fwd_splitkv packs them into one tile per (sequence, K/V head),
 * so the group's K/V are streamed once per split, and the count is sized for
 * those B*H_kv tiles. */
int fa_splitkv_auto_splits_gqa(int B, int H, int H_kv, int S_q, int S_k, int D, int *splits_out);

/*
 * fa_bwd -- exact attention backward (FlashAttention-4 paper, section 3.2,
 * "attention backward pass": S is recomputed block by block from Q and K,
 * then dP, dV, dQ and dK follow from it).
 *
 * With P_ij = exp(scale * <q_i, k_j> - lse_i) over the allowed keys (the
 * forward's probabilities) and dO the gradient of a loss with respect to o,
 * computes the gradients of that loss:
 *   delta_i = <dO_i, o_i>                                      (fp32 output)
 *   dS_ij   = P_ij (<dO_i, v_j> - delta_i)
 *   dq_i    = scale * sum_j dS_ij k_j                          (bf16 output)
 *   dk_j    = scale * sum_(h, i) dS_ij q_i                     (bf16 output)
 *   dv_j    = sum_(h, i) P_ij dO_i                             (bf16 output)
 * where (h, i) runs over the rows of every query head that reads K/V head
 * j's head (grouped-query attention sums the group's contributions).
 *
 * q, k, v, cu_seqlens, B, H, H_kv, S, D, scale and causal are those of the
 * forward call that produced o and lse (query and key lengths are equal).
 * Layouts (16-byte aligned base pointers; lse and delta 4-byte aligned):
 *   q, o, dout, dq: bf16 [B, S, H, D]    (varlen [T, H, D])
 *   k, v, dk, dv:   bf16 [B, S, H_kv, D] (varlen [T, H_kv, D])
 *   lse, delta:     fp32 [B, H, S]       (varlen [H, T])
 * o and lse are read as the forward wrote them (lse in natural-log units).
 * delta is caller-owned scratch that this call fills; dq, dk, dv and delta
 * must not alias any input.  Every gradient row is accumulated by one
 * workgroup in a fixed order, so results are bitwise reproducible, without
 * atomics.  Supported D: 64, 128 and 256 (fa_bwd_hd adds the (192, 128)
 * pair).
 *
 * Errors (nothing is launched): FA_ERR_INVALID_ARG for a null or misaligned
 * pointer, a size <= 0, H not a multiple of H_kv, a non-finite or
 * non-positive scale or causal not 0/1; FA_ERR_UNSUPPORTED for another D or
 * sizes beyond 32-bit row indexing; FA_ERR_NO_DEVICE when no gfx950 is
 * current; FA_ERR_HIP for a failed launch.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H,
           int H_kv, int S, int D, float scale, int causal, const int *cu_seqlens,
           void *stream);

/*
 * fa_bwd_general -- fa_bwd for query and key lengths that may differ, the
 * backward of fa_fwd_general (D_v = D).  The same gradients, over the keys
 * each row may use under fa_fwd_general's rules: with causal = 1 the mask is
 * aligned to the bottom-right corner, row i of a sequence with lengths L_q,
 * L_k using key j when j <= i + L_k - L_q.
 *
 *   dense  (both offsets NULL): q, o, dout, dq [B, S_q, H, D];
 *          k, v, dk, dv [B, S_k, H_kv, D]; lse, delta fp32 [B, H, S_q]
 *   varlen (both non-NULL):     q, o, dout, dq [T_q, H, D];
 *          k, v, dk, dv [T_k, H_kv, D]; lse, delta fp32 [H, T_q]; device
 *          int32 offsets cu_seqlens_q, cu_seqlens_k of B+1 entries as in
 *          fa_fwd_general, S_q and S_k the longest lengths.
 * A row that may use no key (the forward gave it O = 0 and LSE = -inf) gets
 * dq = 0; a key that no row may use gets dk = dv = 0.  One offset array NULL
 * and the other not, or S_k <= 0, is FA_ERR_INVALID_ARG; otherwise the
 * errors, alignment, ownership and determinism of fa_bwd apply.  fa_bwd is
 * the S_q = S_k, cu_seqlens_q = cu_seqlens_k case.
 */
int fa_bwd_general(const void *q, const void *k, const void *v, const void *o, const void *dout,
                   const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H,
                   int H_kv, int S_q, int S_k, int D, float scale, int causal,
                   const int *cu_seqlens_q, const int *cu_seqlens_k, void *stream);

/*
 * fa_bwd_hd -- fa_bwd_general with a value head dimension D_v of its own,
 * the backward of fa_fwd_general for every head-dimension pair it serves:
 * (D, D_v) in {(64, 64), (128, 128), (256, 256), (192, 128)} (the last is
 * the DeepSeek V3 pair the FlashAttention-4 paper benchmarks, section 5.1).
 * q, dq [.., H, D]; k, dk [.., H_kv, D]; v, dv [.., H_kv, D_v];
 * o, dout [.., H, D_v]; otherwise as fa_bwd_general, which is the D_v = D
 * case.  Another pair is FA_ERR_UNSUPPORTED.
 */
int fa_bwd_hd(const void *q, const void *k, const void *v, const void *o, const void *dout,
              const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H,
              int H_kv, int S_q, int S_k, int D, int D_v, float scale, int causal,
              const int *cu_seqlens_q, const int *cu_seqlens_k, void *stream);

/*
 * fa_exp2_emu -- test hook: y[i] = the device's polynomial 2^x[i] for n
 * floats (device pointers, 4-byte aligned).  The function is the one the
 * attention kernel uses for its emulated exponentials: Cody-Waite
 * reduction x = n + f with n = floor(x), f in [0, 1), then a degree-3 Horner
 * polynomial for 2^f (three FMAs) and an exponent add (paper section 3.1.3;
 * the engineering blog's approximate-exponent section).  Inputs below -127
 * are clamped to -127, which yields exactly +0; for x in (-127, -126) the
 * result is a subnormal below 2^-126.  n >= 0.
 */
int fa_exp2_emu(const float *x, float *y, long long n, void *stream);

/*
 * fa_schedule -- host-only view of the persistent tile order (no GPU use).
 *
 * Fills tiles[w * max_rounds + r] with the r-th tile that persistent
 * workgroup w processes, or -1 when it has no more work, for a launch of
 * `workers` workgroups (positions of the order that hold no tile, such as a
 * level a short sequence does not reach, are skipped as the kernel skips
 * them).  A tile is encoded as
 *   ((seq * H + head) * n_mblocks_max + mblock)
 * with n_mblocks_max = ceil(S / BM) and BM the row-tile height chosen for D
 * (the q/k head dimension: 64, 128, 192 or 256).
 * cu_seqlens, if not NULL, is a HOST int32 array of B+1 entries.  *rounds_out
 * receives the length of the longest list and *bm_out the BM used.  Returns
 * FA_ERR_INVALID_ARG when max_rounds is too small or an argument is invalid.
 */
int fa_schedule(int B, int H, int S, int D, int causal, const int *cu_seqlens,
                int workers, int *tiles, int max_rounds, int *rounds_out, int *bm_out);

/*
 * fa_schedule_gqa -- fa_schedule for grouped-query attention with H_kv K/V
 * heads (H_kv divides H; FA_ERR_INVALID_ARG otherwise).  Tiles are still
 * (sequence, query head, m-block).  When H_kv is a multiple of 8, the heads
 * are split across the 8 XCDs by K/V head, so all query heads sharing a K/V
 * head run on one XCD, one K/V head at a time.  fa_schedule is the
 * H_kv = H case.
 */
int fa_schedule_gqa(int B, int H, int H_kv, int S, int D, int causal, const int *cu_seqlens,
                    int workers, int *tiles, int max_rounds, int *rounds_out, int *bm_out);

/*
 * fa_schedule_general -- fa_schedule_gqa for query and key lengths of their
 * own, as fa_fwd_general takes them: cu_seqlens_q and cu_seqlens_k are both
 * NULL (dense) or both HOST int32 arrays of B+1 entries; S_q is the longest
 * query length.  For causal batches whose key lengths differ from their query
 * lengths, the order ranks the sequences by key length (a query tile's cost
 * follows its key length under bottom-right alignment).  Tile codes use
 * n_mblocks_max = ceil(S_q / BM).
 */
int fa_schedule_general(int B, int H, int H_kv, int S_q, int D, int causal,
                        const int *cu_seqlens_q, const int *cu_seqlens_k, int workers, int *tiles,
                        int max_rounds, int *rounds_out, int *bm_out);

/*
 * fa_split_plan -- host-only: the split_levels count (fa_tuning) a dense
 * causal self-attention launch of B x H heads of S tokens with head
 * dimension D uses on `workers` persistent workgroups, for a requested
 * count (-1: the makespan model's choice; always 0 for D = 256).  No GPU
 * use.
 */
int fa_split_plan(int B, int H, int S, int D, int workers, int requested, int *nsplit_out);

/*
 * fa_schedule_split -- fa_schedule for a dense causal batch with the nsplit
 * costliest m-block levels split in two parts (0 <= nsplit <= what
 * fa_split_plan allows, 0 for D = 256; FA_ERR_INVALID_ARG otherwise).  A work item is
 * encoded as ((seq * H + head) * n_mblocks_max + mblock) * 3 + part, part 0
 * being a whole tile and parts 1 and 2 the first and second half of a split
 * tile's key blocks.  No GPU use.
 */
int fa_schedule_split(int B, int H, int S, int D, int nsplit, int workers, int *tiles,
                      int max_rounds, int *rounds_out, int *bm_out);

/*
 * fa_device_info -- the current device as the library sees it: its compute
 * unit count and peak shader clock in kHz (the figures a dense MFMA peak is
 * computed from: CUs x 4096 bf16 flop per clock x clock).  FA_ERR_NO_DEVICE
 * when the current device is not a gfx950.
 */
int fa_device_info(int *cus_out, int *clock_khz_out);

/* Number of persistent workgroups fa_fwd launches on the current device. */
int fa_num_workers(int D, int *workers_out);

/*
 * fa_mfma_ceiling -- a measurement, not attention: the rate the matrix unit
 * sustains on the forward's own product sequence, against which the
 * forward's rate is judged (the FlashAttention-4 paper's rate analysis,
 * section 3.1.1, compares a tile's matrix time with its other work; this
 * measures the matrix time's floor on the device).
 *
 * Launches the D = 128 forward's shape (one workgroup of 8 waves per CU);
 * every wave runs `blocks` 64-key blocks of its matrix phases only: 32
 * products of v_mfma_f32_32x32x16_bf16 per block (QK for two 32-key
 * sub-blocks over 8 k-steps, PV over 4 key steps and 4 d-tiles), with no
 * softmax, copies or barriers.
 *   mode 0: operands held in registers (the matrix unit alone);
 *   mode 1: K and V^T operands read from LDS exactly as the forward reads
 *           them (the matrix phases as the forward runs them).
 * Operands are pseudo-random (K, V, Q uniform on [-2, 2), P on [0, 1)): the
 * matrix unit's power, and so the clock the device sustains, depends on the
 * data, and constant operands would overstate the ceiling.
 * Runs `reps` launches on the null stream and waits for them (it allocates
 * and frees small device buffers; not for use inside a captured stream).
 * *out receives the median launch (by time): its duration, TFLOP/s
 * (2*32*32*16 flop per product), the fastest launch's TFLOP/s, the shader
 * clock over the loop (s_memtime ticks per s_memrealtime second, averaged
 * over waves) and the cycles per product on one SIMD's matrix unit (launch
 * duration times that clock over the products per SIMD; 32 is the unit's
 * issue rate for this instruction).
 * Returns FA_ERR_INVALID_ARG for mode not 0/1, blocks outside 1..2^20,
 * reps outside 1..1000 or out == NULL; FA_ERR_NO_DEVICE or FA_ERR_HIP.
 */
typedef struct fa_mfma_rate {
    int workers;                  /* workgroups launched (one per CU) */
    long long products;           /* matrix products per launch */
    double ms;                    /* median launch duration */
    double tflops;                /* rate of the median launch */
    double best_tflops;           /* rate of the fastest launch */
    double clock_mhz;             /* shader clock during the median launch */
    double cycles_per_product;    /* per SIMD, median launch */
} fa_mfma_rate;
int fa_mfma_ceiling(int mode, int blocks, int reps, fa_mfma_rate *out);

/* Human-readable name of an fa_status value (static string, never NULL). */
const char *fa_status_string(int status);

/* Library ABI version: 100 * major + minor (101: fa_fwd_gqa; 102: fa_fwd_hd;
 * 103: fa_fwd_general; 104: fa_bwd; 105: fa_fwd_splitkv; 106: fa_bwd_general;
 * 107: fa_fwd_splitkv_noalloc; 108: fa_mfma_ceiling; 109: fa_bwd_hd;
 * 110: fa_tuning.split_levels, fa_split_plan, fa_schedule_split, fa_device_info). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
