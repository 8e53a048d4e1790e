/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU implementation of exact attention
 * forward, O = softmax(scale * Q K^T + causal mask) V, plus the natural-log
 * logsumexp of each row.  It exists to check the GPU library against; it is
 * not part of the product.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load it.  It shares no source, header,
 * table or constant with the HIP library.
 *
 * What it follows (FlashAttention-4 paper as translated on 171host.com):
 *   - section 2.1 "Multi-head attention" names the operation; its formula was
 *     lost from the page, so the textbook definition is written out here:
 *     s_ij = scale * <q_i, k_j>, P = softmax over the allowed keys, O = P V;
 *   - section 3.1.2: per row, take the maximum, subtract it, exponentiate,
 *     then sum;  section 3.1.4: the output is normalised by that sum at the
 *     end;
 *   - section 3.3 (LPT for causal masking): scores above the diagonal are
 *     masked, i.e. query i may use key j only when j <= i.
 * The row is processed in two plain passes (max, then exp/sum/weighted sum);
 * no blocking, no online rescaling, no reordering beyond that.
 *
 * Layouts (row-major, contiguous):
 *   dense : q, o are [B, Sq, H, D]; k, v are [B, Sk, Hkv, D]; lse is [B, H, Sq]
 *   varlen: q, o are [Tq, H, D] with Tq = cu_q[B]; k, v are [Tk, Hkv, D] with
 *           Tk = cu_k[B]; lse is [H, Tq].  Sequence b owns query tokens
 *           cu_q[b] .. cu_q[b+1]-1 and key tokens cu_k[b] .. cu_k[b+1]-1 and
 *           attends only within itself.
 * Query and key lengths may differ (Lq, Lk).  The causal mask is aligned to
 * the bottom-right corner: query i may use key j when j <= i + Lk - Lq, so
 * the last query sees every key (for Lq = Lk this is the plain j <= i).  A
 * row that may use no key (Lq > Lk, i < Lq - Lk) has output 0 and LSE -inf
 * (the empty sum).
 * Grouped-query attention (the paper's section 3.3 reports LPT results for
 * MQA): Hkv divides H and query head h reads K/V head h / (H / Hkv), i.e.
 * each run of H/Hkv consecutive query heads shares one K/V head.  Hkv = H is
 * plain multi-head attention, Hkv = 1 is multi-query attention.
 * Head dimensions: q and k rows have D entries, v and o rows Dv entries
 * (the paper's section 5.1 also benchmarks the (192, 128) pair of
 * DeepSeek V3); Dv = D is the usual case.
 * Inputs come either as double or as bfloat16 bit patterns (uint16), which
 * are widened exactly to double (bf16 is the top half of an IEEE float).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of one bfloat16 bit pattern. */
double oracle_bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* A read-only tensor that is either double or bf16 bits. */
typedef struct {
    const void *p;
    int is_bf16;
} tensor_in;

static inline double at(tensor_in t, int64_t i)
{
    if (t.is_bf16)
        return oracle_bf16_to_f64(((const uint16_t *)t.p)[i]);
    return ((const double *)t.p)[i];
}

/* Where a sequence lives: first token index and length. */
typedef struct {
    int64_t tok0;
    int len;
} seq_span;

/* Sizes of one call.  cu_q / cu_k are NULL for dense inputs. */
typedef struct {
    int B, H, Hkv, Sq, Sk, D, Dv;
    const int *cu_q, *cu_k;
} attn_shape;

/*
 * One query row i of one (sequence, head): two passes over the allowed keys.
 * s must hold at least spk.len doubles.  Writes Dv outputs to o_row and the
 * row's logsumexp to *lse_out.
 */
static void attend_one_row(tensor_in q, tensor_in k, tensor_in v,
                           double *o_row, double *lse_out,
                           seq_span spq, seq_span spk, int i, int h, const attn_shape *sh,
                           double scale, int causal, double *s)
{
    const int H = sh->H, Hkv = sh->Hkv, D = sh->D, Dv = sh->Dv;
    int nkeys = spk.len;
    if (causal) {
        const int last = i + spk.len - spq.len;  /* bottom-right alignment */
        nkeys = last + 1 < 0 ? 0 : (last + 1 < spk.len ? last + 1 : spk.len);
    }
    const int64_t qbase = ((spq.tok0 + i) * H + h) * (int64_t)D;
    const int hk = h / (H / Hkv);  /* the K/V head of query head h */
    if (nkeys == 0) {
        for (int d = 0; d < Dv; ++d)
            o_row[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }

    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        const int64_t kbase = ((spk.tok0 + j) * Hkv + hk) * (int64_t)D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += at(q, qbase + d) * at(k, kbase + d);
        s[j] = scale * dot;
        if (s[j] > m)
            m = s[j];
    }

    /* pass 2: exponentiate against the maximum, sum, weight V */
    double l = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int d = 0; d < Dv; ++d) {
        double acc = 0.0;
        for (int j = 0; j < nkeys; ++j)
            acc += s[j] * at(v, ((spk.tok0 + j) * Hkv + hk) * (int64_t)Dv + d);
        o_row[d] = acc / l;
    }
    *lse_out = m + log(l);
}

/* Span of sequence b: dense uses b*S .. b*S+S-1, varlen reads cu. */
static seq_span span_of(int b, int S, const int *cu)
{
    seq_span sp;
    if (cu) {
        sp.tok0 = cu[b];
        sp.len = cu[b + 1] - cu[b];
    } else {
        sp.tok0 = (int64_t)b * S;
        sp.len = S;
    }
    return sp;
}

/*
 * Map a row id, numbered like the lse layout, to (b, h, i).
 *   dense : row = (b*H + h)*Sq + i
 *   varlen: row = h*Tq + t, t a global query token index; b the sequence holding t
 */
static void decode_row(int64_t row, const attn_shape *sh, int *b, int *h, int *i)
{
    const int B = sh->B, H = sh->H, S = sh->Sq;
    const int *cu = sh->cu_q;
    if (!cu) {
        *i = (int)(row % S);
        *h = (int)((row / S) % H);
        *b = (int)(row / ((int64_t)S * H));
        return;
    }
    const int64_t T = cu[B];
    const int64_t t = row % T;
    *h = (int)(row / T);
    int bb = 0;
    while (bb + 1 < B && cu[bb + 1] <= t)
        ++bb;
    *b = bb;
    *i = (int)(t - cu[bb]);
}

static int max_len(int B, int S, const int *cu)
{
    if (!cu)
        return S;
    int mx = 0;
    for (int b = 0; b < B; ++b) {
        int L = cu[b + 1] - cu[b];
        if (L > mx)
            mx = L;
    }
    return mx;
}

static int shape_ok(const attn_shape *sh)
{
    if (sh->B <= 0 || sh->H <= 0 || sh->Hkv <= 0 || sh->H % sh->Hkv != 0 || sh->D <= 0 ||
        sh->Dv <= 0)
        return 0;
    if ((sh->cu_q == NULL) != (sh->cu_k == NULL))
        return 0;
    if (!sh->cu_q && (sh->Sq <= 0 || sh->Sk <= 0))
        return 0;
    return 1;
}

/*
 * Attention for an explicit list of rows.  o_rows is [n_rows, Dv] and
 * lse_rows is [n_rows]; either may be NULL.  Returns 0, or -1 on bad input.
 */
static int attend_rows(tensor_in q, tensor_in k, tensor_in v,
                       const int64_t *rows, int64_t n_rows,
                       double *o_rows, double *lse_rows,
                       const attn_shape *sh, double scale, int causal)
{
    if (!shape_ok(sh))
        return -1;
    const int Lmax = max_len(sh->B, sh->Sk, sh->cu_k);
    const int Dv = sh->Dv;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
        double *o_tmp = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (!s || !o_tmp) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t r = 0; r < n_rows; ++r) {
                int b, h, i;
                decode_row(rows[r], sh, &b, &h, &i);
                seq_span spq = span_of(b, sh->Sq, sh->cu_q);
                seq_span spk = span_of(b, sh->Sk, sh->cu_k);
                double lse;
                attend_one_row(q, k, v, o_tmp, &lse, spq, spk, i, h, sh, scale, causal, s);
                if (o_rows)
                    memcpy(o_rows + r * (int64_t)Dv, o_tmp, sizeof(double) * (size_t)Dv);
                if (lse_rows)
                    lse_rows[r] = lse;
            }
        }
        free(s);
        free(o_tmp);
    }
    return bad ? -1 : 0;
}

/*
 * Full attention: o in the q layout (with Dv columns), lse in the lse layout
 * (either may be NULL).  Every row of every (sequence, head) is computed.
 */
static int attend_all(tensor_in q, tensor_in k, tensor_in v, double *o, double *lse,
                      const attn_shape *sh, double scale, int causal)
{
    if (!shape_ok(sh))
        return -1;
    const int H = sh->H, Dv = sh->Dv;
    const int64_t T = sh->cu_q ? sh->cu_q[sh->B] : (int64_t)sh->B * sh->Sq;
    const int64_t n_rows = T * H;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_rows > 0 ? n_rows : 1));
    double *o_rows = (double *)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1) * Dv);
    double *l_rows = (double *)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1));
    if (!rows || !o_rows || !l_rows) {
        free(rows);
        free(o_rows);
        free(l_rows);
        return -1;
    }
    for (int64_t r = 0; r < n_rows; ++r)
        rows[r] = r;
    int rc = attend_rows(q, k, v, rows, n_rows, o_rows, l_rows, sh, scale, causal);
    if (rc == 0) {
        for (int64_t r = 0; r < n_rows; ++r) {
            int b, h, i;
            decode_row(r, sh, &b, &h, &i);
            seq_span spq = span_of(b, sh->Sq, sh->cu_q);
            if (o)
                memcpy(o + ((spq.tok0 + i) * H + h) * (int64_t)Dv, o_rows + r * (int64_t)Dv,
                       sizeof(double) * (size_t)Dv);
            if (lse)
                lse[r] = l_rows[r];
        }
    }
    free(rows);
    free(o_rows);
    free(l_rows);
    return rc;
}

/* ---- exported entry points (C ABI, loaded by ctypes from Python) ----
 * Hkv is the number of K/V heads (Hkv = H for multi-head attention); D is the
 * q/k head dimension and Dv the v/o head dimension; Sq and Sk are the dense
 * query and key lengths; cu_q and cu_k (both NULL for dense inputs) the
 * varlen query and key offsets. */

int oracle_attn_fwd_f64(const double *q, const double *k, const double *v,
                        double *o, double *lse, int B, int H, int Hkv, int Sq, int Sk,
                        int D, int Dv, double scale, int causal, const int *cu_q,
                        const int *cu_k)
{
    tensor_in tq = {q, 0}, tk = {k, 0}, tv = {v, 0};
    attn_shape sh = {B, H, Hkv, Sq, Sk, D, Dv, cu_q, cu_k};
    return attend_all(tq, tk, tv, o, lse, &sh, scale, causal);
}

int oracle_attn_fwd_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         double *o, double *lse, int B, int H, int Hkv, int Sq, int Sk,
                         int D, int Dv, double scale, int causal, const int *cu_q,
                         const int *cu_k)
{
    tensor_in tq = {q, 1}, tk = {k, 1}, tv = {v, 1};
    attn_shape sh = {B, H, Hkv, Sq, Sk, D, Dv, cu_q, cu_k};
    return attend_all(tq, tk, tv, o, lse, &sh, scale, causal);
}

int oracle_attn_rows_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const int64_t *rows, int64_t n_rows,
                          double *o_rows, double *lse_rows,
                          int B, int H, int Hkv, int Sq, int Sk, int D, int Dv,
                          double scale, int causal, const int *cu_q, const int *cu_k)
{
    tensor_in tq = {q, 1}, tk = {k, 1}, tv = {v, 1};
    attn_shape sh = {B, H, Hkv, Sq, Sk, D, Dv, cu_q, cu_k};
    return attend_rows(tq, tk, tv, rows, n_rows, o_rows, lse_rows, &sh, scale, causal);
}

/*
 * 2^x in double precision for float inputs: the definition that the
 * device-side polynomial exp2 approximates (FlashAttention-4 paper,
 * section 3.1.3, "Emulation of the exponential").
 */
void oracle_exp2(const float *x, double *y, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        y[i] = exp2((double)x[i]);
}

/* Number of threads a parallel region of this library will use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
