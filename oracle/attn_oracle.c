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

/* ------------------------------------------------------------------------
 * Backward pass (FlashAttention-4 paper, section 3.2 "Attention backward
 * pass": recompute S, then the products that give dP, dV, dQ and dK).
 * Given the output gradient dO, these are the gradients of
 * F(Q, K, V) = sum_i <dO_i, O_i>, written out by the chain rule through the
 * row softmax:
 *   P_ij     = exp(s_ij - LSE_i)            (the forward's probabilities)
 *   dP_ij    = <dO_i, v_j>
 *   Delta_i  = sum_j P_ij dP_ij
 *   dS_ij    = P_ij (dP_ij - Delta_i)
 *   dQ_i     = scale * sum_j dS_ij k_j
 *   dK_j     = scale * sum_(h, i) dS_ij q_i   over the query heads h that
 *   dV_j     =         sum_(h, i) P_ij dO_i   read K/V head hk, and their rows
 * Masked pairs (i, j) have P_ij = 0 and take no part.  A row without keys
 * contributes nothing and has dQ_i = 0.
 * Pass 1 takes one query row at a time (its probabilities, Delta, dQ);
 * pass 2 one key row at a time (dK, dV), reading the LSE and Delta of the
 * query rows from pass 1.  Both are plain loops over the definition.
 *
 * Next to each gradient it can return the sum of the absolute values of
 * the terms that make it up, with dS_ij widened by P_ij * E_i where
 * E_i = sum_d |dO_id| |O_id|:
 *   |dQ|_id = scale * sum_j (|dS_ij| + P_ij E_i) |k_jd|
 *   |dK|_jd = scale * sum_(h, i) (|dS_ij| + P_ij E_i) |q_id|
 *   |dV|_jd = sum_(h, i) P_ij |dO_id|
 * These are the scales against which a rounding error in P, in dS or in
 * O (through Delta = <dO, O>) shows up; the tests derive tolerances from
 * them.
 * ---------------------------------------------------------------------- */

/* Row statistics of one query row. */
typedef struct {
    double lse, delta, e;
    int nkeys;
} row_stats;

/* Probabilities p[0..nkeys) of query row i of head h over its allowed keys,
 * the row's logsumexp and its key count. */
static int row_probs(tensor_in q, tensor_in k, seq_span spq, seq_span spk, int i, int h,
                     const attn_shape *sh, double scale, int causal, double *p, double *lse)
{
    const int H = sh->H, Hkv = sh->Hkv, D = sh->D;
    int nkeys = spk.len;
    if (causal) {
        const int last = i + spk.len - spq.len;
        nkeys = last + 1 < 0 ? 0 : (last + 1 < spk.len ? last + 1 : spk.len);
    }
    const int hk = h / (H / Hkv);
    const int64_t qbase = ((spq.tok0 + i) * H + h) * (int64_t)D;
    double m = -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        const int64_t kbase = ((spk.tok0 + j) * Hkv + hk) * (int64_t)D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += at(q, qbase + d) * at(k, kbase + d);
        p[j] = scale * dot;
        if (p[j] > m)
            m = p[j];
    }
    double l = 0.0;
    for (int j = 0; j < nkeys; ++j)
        l += exp(p[j] - m);
    *lse = nkeys > 0 ? m + log(l) : -INFINITY;
    for (int j = 0; j < nkeys; ++j)
        p[j] = exp(p[j] - *lse);
    return nkeys;
}

/* Pass 1 for query row i of head h: statistics, and (if dq_row is given)
 * dQ_i with its magnitude.  p and dp hold at least spk.len doubles. */
static void bwd_query_row(tensor_in q, tensor_in k, tensor_in v, tensor_in dout,
                          seq_span spq, seq_span spk, int i, int h, const attn_shape *sh,
                          double scale, int causal, double *p, double *dp, row_stats *st,
                          double *dq_row, double *dq_mag)
{
    const int H = sh->H, Hkv = sh->Hkv, D = sh->D, Dv = sh->Dv;
    const int hk = h / (H / Hkv);
    const int n = row_probs(q, k, spq, spk, i, h, sh, scale, causal, p, &st->lse);
    const int64_t obase = ((spq.tok0 + i) * H + h) * (int64_t)Dv;
    double delta = 0.0, e = 0.0;
    for (int j = 0; j < n; ++j) {
        const int64_t vbase = ((spk.tok0 + j) * Hkv + hk) * (int64_t)Dv;
        double acc = 0.0;
        for (int d = 0; d < Dv; ++d)
            acc += at(dout, obase + d) * at(v, vbase + d);
        dp[j] = acc;
        delta += p[j] * acc;
    }
    for (int d = 0; d < Dv; ++d) {
        double od = 0.0;
        for (int j = 0; j < n; ++j)
            od += p[j] * at(v, ((spk.tok0 + j) * Hkv + hk) * (int64_t)Dv + d);
        e += fabs(at(dout, obase + d)) * fabs(od);
    }
    st->delta = delta;
    st->e = e;
    st->nkeys = n;
    if (!dq_row)
        return;
    for (int d = 0; d < D; ++d) {
        double g = 0.0, mag = 0.0;
        for (int j = 0; j < n; ++j) {
            const double kd = at(k, ((spk.tok0 + j) * Hkv + hk) * (int64_t)D + d);
            const double ds = p[j] * (dp[j] - delta);
            g += ds * kd;
            mag += (fabs(ds) + p[j] * e) * fabs(kd);
        }
        dq_row[d] = scale * g;
        if (dq_mag)
            dq_mag[d] = scale * mag;
    }
}

/* Row id of query row i of head h in sequence b (the lse layout). */
static int64_t query_row_id(int b, int h, int i, const attn_shape *sh)
{
    if (sh->cu_q)
        return (int64_t)h * sh->cu_q[sh->B] + sh->cu_q[b] + i;
    return ((int64_t)b * sh->H + h) * sh->Sq + i;
}

/* Pass 2 for key row j of K/V head hk in sequence b: dK_j and dV_j (and
 * magnitudes when the pointers are given), from the row statistics of
 * every query row (indexed by query_row_id). */
static void bwd_key_row(tensor_in q, tensor_in k, tensor_in v, tensor_in dout,
                        const row_stats *stats, int b, int j, int hk, const attn_shape *sh,
                        double scale, int causal, double *dk_row, double *dv_row,
                        double *dk_mag, double *dv_mag)
{
    const int H = sh->H, Hkv = sh->Hkv, D = sh->D, Dv = sh->Dv, G = H / Hkv;
    const seq_span spq = span_of(b, sh->Sq, sh->cu_q);
    const seq_span spk = span_of(b, sh->Sk, sh->cu_k);
    const int64_t kbase = ((spk.tok0 + j) * Hkv + hk) * (int64_t)D;
    const int64_t vbase = ((spk.tok0 + j) * Hkv + hk) * (int64_t)Dv;
    for (int d = 0; d < D; ++d) {
        dk_row[d] = 0.0;
        if (dk_mag)
            dk_mag[d] = 0.0;
    }
    for (int d = 0; d < Dv; ++d) {
        dv_row[d] = 0.0;
        if (dv_mag)
            dv_mag[d] = 0.0;
    }
    /* with the bottom-right causal alignment, key j is used by rows
     * i >= j - (Lk - Lq) */
    int i0 = 0;
    if (causal) {
        i0 = j - (spk.len - spq.len);
        if (i0 < 0)
            i0 = 0;
    }
    for (int g = 0; g < G; ++g) {
        const int h = hk * G + g;
        for (int i = i0; i < spq.len; ++i) {
            const row_stats *st = &stats[query_row_id(b, h, i, sh)];
            const int64_t qbase = ((spq.tok0 + i) * H + h) * (int64_t)D;
            const int64_t obase = ((spq.tok0 + i) * H + h) * (int64_t)Dv;
            double s = 0.0, dp = 0.0;
            for (int d = 0; d < D; ++d)
                s += at(q, qbase + d) * at(k, kbase + d);
            for (int d = 0; d < Dv; ++d)
                dp += at(dout, obase + d) * at(v, vbase + d);
            const double p = exp(scale * s - st->lse);
            const double ds = p * (dp - st->delta);
            for (int d = 0; d < D; ++d) {
                const double qd = at(q, qbase + d);
                dk_row[d] += scale * ds * qd;
                if (dk_mag)
                    dk_mag[d] += scale * (fabs(ds) + p * st->e) * fabs(qd);
            }
            for (int d = 0; d < Dv; ++d) {
                const double gd = at(dout, obase + d);
                dv_row[d] += p * gd;
                if (dv_mag)
                    dv_mag[d] += p * fabs(gd);
            }
        }
    }
}

/* Map a key row id ((b*Hkv + hk)*Sk + j dense, hk*Tk + t varlen) to (b, hk, j). */
static void decode_key_row(int64_t row, const attn_shape *sh, int *b, int *hk, int *j)
{
    const int B = sh->B, Hkv = sh->Hkv, S = sh->Sk;
    const int *cu = sh->cu_k;
    if (!cu) {
        *j = (int)(row % S);
        *hk = (int)((row / S) % Hkv);
        *b = (int)(row / ((int64_t)S * Hkv));
        return;
    }
    const int64_t T = cu[B];
    const int64_t t = row % T;
    *hk = (int)(row / T);
    int bb = 0;
    while (bb + 1 < B && cu[bb + 1] <= t)
        ++bb;
    *b = bb;
    *j = (int)(t - cu[bb]);
}

/*
 * Backward for explicit row lists.  q_rows (lse-layout ids) get dQ rows
 * ([n_q, D]) and their magnitudes; k_rows (key row ids) get dK ([n_k, D]),
 * dV ([n_k, Dv]) rows and magnitudes.  Magnitude pointers may be NULL.
 * The statistics pass runs over every query row of each (sequence, head)
 * that a requested key row needs.  Returns 0, or -1 on bad input.
 */
static int bwd_rows(tensor_in q, tensor_in k, tensor_in v, tensor_in dout,
                    const int64_t *q_rows, int64_t n_q, double *dq_rows, double *dq_mag,
                    const int64_t *k_rows, int64_t n_k, double *dk_rows, double *dv_rows,
                    double *dk_mag, double *dv_mag, const attn_shape *sh, double scale,
                    int causal)
{
    if (!shape_ok(sh))
        return -1;
    const int B = sh->B, H = sh->H, G = sh->H / sh->Hkv, D = sh->D, Dv = sh->Dv;
    const int64_t Tq = sh->cu_q ? sh->cu_q[B] : (int64_t)B * sh->Sq;
    const int64_t n_rows = Tq * H;
    const int Lmax = max_len(B, sh->Sk, sh->cu_k);
    row_stats *stats = NULL;
    unsigned char *need = NULL;
    int bad = 0;
    if (n_k > 0) {
        stats = (row_stats *)calloc((size_t)(n_rows > 0 ? n_rows : 1), sizeof(row_stats));
        need = (unsigned char *)calloc((size_t)B * H, 1);
        if (!stats || !need) {
            free(stats);
            free(need);
            return -1;
        }
        for (int64_t r = 0; r < n_k; ++r) {
            int b, hk, j;
            decode_key_row(k_rows[r], sh, &b, &hk, &j);
            for (int g = 0; g < G; ++g)
                need[b * H + hk * G + g] = 1;
        }
    }
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
        if (!p || !dp) {
#pragma omp atomic write
            bad = 1;
        } else {
            if (n_k > 0) {
#pragma omp for schedule(dynamic, 16)
                for (int64_t r = 0; r < n_rows; ++r) {
                    int b, h, i;
                    decode_row(r, sh, &b, &h, &i);
                    if (!need[b * H + h])
                        continue;
                    bwd_query_row(q, k, v, dout, span_of(b, sh->Sq, sh->cu_q),
                                  span_of(b, sh->Sk, sh->cu_k), i, h, sh, scale, causal, p, dp,
                                  &stats[r], NULL, NULL);
                }
            }
#pragma omp for schedule(dynamic, 8)
            for (int64_t r = 0; r < n_q; ++r) {
                int b, h, i;
                decode_row(q_rows[r], sh, &b, &h, &i);
                row_stats st;
                bwd_query_row(q, k, v, dout, span_of(b, sh->Sq, sh->cu_q),
                              span_of(b, sh->Sk, sh->cu_k), i, h, sh, scale, causal, p, dp, &st,
                              dq_rows + r * (int64_t)D, dq_mag ? dq_mag + r * (int64_t)D : NULL);
            }
#pragma omp for schedule(dynamic, 8)
            for (int64_t r = 0; r < n_k; ++r) {
                int b, hk, j;
                decode_key_row(k_rows[r], sh, &b, &hk, &j);
                bwd_key_row(q, k, v, dout, stats, b, j, hk, sh, scale, causal,
                            dk_rows + r * (int64_t)D, dv_rows + r * (int64_t)Dv,
                            dk_mag ? dk_mag + r * (int64_t)D : NULL,
                            dv_mag ? dv_mag + r * (int64_t)Dv : NULL);
            }
        }
        free(p);
        free(dp);
    }
    free(stats);
    free(need);
    return bad ? -1 : 0;
}

/* Key row id of token t (global key token index) of K/V head hk. */
static int64_t key_row_id_of_token(int64_t t, int hk, const attn_shape *sh)
{
    if (sh->cu_k)
        return (int64_t)hk * sh->cu_k[sh->B] + t;
    const int64_t b = t / sh->Sk, j = t % sh->Sk;
    return (b * sh->Hkv + hk) * sh->Sk + j;
}

/*
 * Full backward: dq in the q layout, dk in the k layout, dv in the v layout;
 * the magnitude arrays (each may be NULL) in the layout of their gradient.
 */
static int bwd_all(tensor_in q, tensor_in k, tensor_in v, tensor_in dout, double *dq,
                   double *dk, double *dv, double *dq_mag, double *dk_mag, double *dv_mag,
                   const attn_shape *sh, double scale, int causal)
{
    if (!shape_ok(sh))
        return -1;
    const int B = sh->B, H = sh->H, Hkv = sh->Hkv, D = sh->D, Dv = sh->Dv;
    const int64_t Tq = sh->cu_q ? sh->cu_q[B] : (int64_t)B * sh->Sq;
    const int64_t Tk = sh->cu_k ? sh->cu_k[B] : (int64_t)B * sh->Sk;
    const int64_t nq = Tq * H, nk = Tk * Hkv;
    int64_t *qr = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nq > 0 ? nq : 1));
    int64_t *kr = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nk > 0 ? nk : 1));
    double *bq = (double *)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1) * D);
    double *bqm = (double *)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1) * D);
    double *bk = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * D);
    double *bv = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * Dv);
    double *bkm = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * D);
    double *bvm = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * Dv);
    int rc = -1;
    if (qr && kr && bq && bqm && bk && bv && bkm && bvm) {
        /* query rows in q-layout order: token-major, then head */
        for (int64_t t = 0; t < Tq; ++t)
            for (int h = 0; h < H; ++h) {
                int b = 0;
                int64_t i = t;
                if (sh->cu_q) {
                    while (b + 1 < B && sh->cu_q[b + 1] <= t)
                        ++b;
                    i = t - sh->cu_q[b];
                } else {
                    b = (int)(t / sh->Sq);
                    i = t % sh->Sq;
                }
                qr[t * H + h] = query_row_id(b, h, (int)i, sh);
            }
        for (int64_t t = 0; t < Tk; ++t)
            for (int hk = 0; hk < Hkv; ++hk)
                kr[t * Hkv + hk] = key_row_id_of_token(t, hk, sh);
        rc = bwd_rows(q, k, v, dout, qr, nq, bq, bqm, kr, nk, bk, bv, bkm, bvm, sh, scale,
                      causal);
        if (rc == 0) {
            if (dq)
                memcpy(dq, bq, sizeof(double) * (size_t)nq * D);
            if (dq_mag)
                memcpy(dq_mag, bqm, sizeof(double) * (size_t)nq * D);
            if (dk)
                memcpy(dk, bk, sizeof(double) * (size_t)nk * D);
            if (dv)
                memcpy(dv, bv, sizeof(double) * (size_t)nk * Dv);
            if (dk_mag)
                memcpy(dk_mag, bkm, sizeof(double) * (size_t)nk * D);
            if (dv_mag)
                memcpy(dv_mag, bvm, sizeof(double) * (size_t)nk * Dv);
        }
    }
    free(qr);
    free(kr);
    free(bq);
    free(bqm);
    free(bk);
    free(bv);
    free(bkm);
    free(bvm);
    return rc;
}

/* ---- backward entry points: dout is [.., H, Dv] in the o layout; the
 * output and magnitude arrays are double, any of them may be NULL. */

int oracle_attn_bwd_f64(const double *q, const double *k, const double *v, const double *dout,
                        double *dq, double *dk, double *dv, double *dq_mag, double *dk_mag,
                        double *dv_mag, int B, int H, int Hkv, int Sq, int Sk, int D, int Dv,
                        double scale, int causal, const int *cu_q, const int *cu_k)
{
    tensor_in tq = {q, 0}, tk = {k, 0}, tv = {v, 0}, tg = {dout, 0};
    attn_shape sh = {B, H, Hkv, Sq, Sk, D, Dv, cu_q, cu_k};
    return bwd_all(tq, tk, tv, tg, dq, dk, dv, dq_mag, dk_mag, dv_mag, &sh, scale, causal);
}

int oracle_attn_bwd_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *dout, double *dq, double *dk, double *dv,
                         double *dq_mag, double *dk_mag, double *dv_mag, int B, int H, int Hkv,
                         int Sq, int Sk, int D, int Dv, double scale, int causal,
                         const int *cu_q, const int *cu_k)
{
    tensor_in tq = {q, 1}, tk = {k, 1}, tv = {v, 1}, tg = {dout, 1};
    attn_shape sh = {B, H, Hkv, Sq, Sk, D, Dv, cu_q, cu_k};
    return bwd_all(tq, tk, tv, tg, dq, dk, dv, dq_mag, dk_mag, dv_mag, &sh, scale, causal);
}

int oracle_attn_bwd_rows_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const uint16_t *dout, const int64_t *q_rows, int64_t n_q,
                              double *dq_rows, double *dq_mag, const int64_t *k_rows,
                              int64_t n_k, double *dk_rows, double *dv_rows, double *dk_mag,
                              double *dv_mag, int B, int H, int Hkv, int Sq, int Sk, int D,
                              int Dv, double scale, int causal, const int *cu_q,
                              const int *cu_k)
{
    tensor_in tq = {q, 1}, tk = {k, 1}, tv = {v, 1}, tg = {dout, 1};
    attn_shape sh = {B, H, Hkv, Sq, Sk, D, Dv, cu_q, cu_k};
    return bwd_rows(tq, tk, tv, tg, q_rows, n_q, dq_rows, dq_mag, k_rows, n_k, dk_rows, dv_rows,
                    dk_mag, dv_mag, &sh, scale, causal);
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
