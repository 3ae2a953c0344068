/*
 * mfa_oracle.c -- plain fp64 CPU reference for the fused attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code with the HIP library.
 *
 * What it computes (the plain definition, not a tiled algorithm):
 *
 *     O[b,i,hq,:] = sum_j P_ij V[b,j,kvh,:],   P_ij = exp(s_ij - LSE_i)
 *     LSE_i       = log sum_{j visible} exp(s_ij)
 *     s_ij        = T(scale * <Q[b,i,hq,:], K[b,j,kvh,:]>)
 *
 * with T the optional tanh soft-cap and the sum over the keys visible to row
 * i.  The pages present the tiled online softmax as an exact re-association
 * of this sum (vision_rs flash_attn2.rs, module doc: the full score matrix is
 * never formed; brotensor flash_attention.h, flash_attention_decode_len:
 * different split points agree up to rounding), so the definition itself is
 * the oracle.  Each row's probability vector is formed in full, as the forge
 * attention.metal forward kernel does for its CPU-parity path.
 *
 * Layouts (row-major, contiguous): Q and O [B, Lq, Hq, D]; K and V
 * [B, Lk, Hkv, D]; key_mask [B, Lk] or NULL.  Inputs are float32 arrays that
 * hold the already-rounded input tensors exactly; all arithmetic is double.
 *
 * Every function here has pins in tests/ (closed forms, invariants, library
 * special cases and brute force); none is "parity unpinned".
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -pthread (no fast-math).
 * Defining ORACLE_MUTANT=n plants deliberate mistake n; the test suite builds
 * those variants only to show that its pins catch them.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

typedef struct {
    int64_t B, Lq, Lk, Hq, Hkv, D;
    double scale;
    int causal;
    int64_t window;
    int64_t q_offset;
    double softcap;
    /* additive score bias, element (b, hq, i, j) at b*bs[0] + hq*bs[1] +
     * i*bs[2] + j*bs[3] (stride 0 broadcasts a size-1 dimension), or NULL */
    const float* bias;
    int64_t bs[4];
    /* attention dropout: drop probability p and the seed of its pattern */
    double dropout_p;
    uint64_t seed;
} oracle_dims;

/*
 * Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011): ten rounds over a 256-bit counter with a
 * 128-bit key.  Each round multiplies counter words 0 and 2 by the two
 * round constants into 128-bit products, rebuilds the counter from the
 * products' halves XOR-ed with words 1 and 3 and the key, and the key is
 * bumped by the two Weyl constants between rounds.
 */
void mfa_oracle_philox4x64(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        const unsigned __int128 p0 = (unsigned __int128)M0 * c0;
        const unsigned __int128 p1 = (unsigned __int128)M1 * c2;
        const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += W0;
        k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * Dropout decision of score (b, hq, i, j).  The pages fix only that a seed
 * drives the pattern, of which only the low 32 bits are used (ferrotensor
 * attention.rs, AttentionOptions, `seed`); the oracle reads the rest as: one
 * Philox4x64-10 block per sixteen consecutive keys, counter
 * (floor(j / 16), i, hq, b) and key (seed mod 2^32, 0); its four 64-bit
 * output words hold sixteen 16-bit fields, field f being bits 16 (f mod 4) ..
 * 16 (f mod 4) + 15 of word floor(f / 4), and key j reads field j mod 16; the
 * weight is kept iff that field is >= round(p * 2^16).
 */
int mfa_oracle_dropout_keep(uint64_t seed, double p, int64_t b, int64_t hq, int64_t i, int64_t j)
{
    const uint64_t ctr[4] = {(uint64_t)(j / 16), (uint64_t)i, (uint64_t)hq, (uint64_t)b};
    const uint64_t key[2] = {seed & 0xffffffffull, 0};
    uint64_t out[4];
    mfa_oracle_philox4x64(ctr, key, out);
    const uint64_t threshold = (uint64_t)llround(p * 65536.0);
    const int64_t f = j % 16;
#if ORACLE_MUTANT == 18
    (void)f;
    return (out[0] & 0xffffu) >= threshold;  /* every key of the block reads field 0 */
#else
    return ((out[f / 4] >> (16 * (f % 4))) & 0xffffu) >= threshold;
#endif
}

/*
 * Key range [lo, hi] (inclusive) visible to a query at absolute position aq,
 * before the key mask is applied.  brotensor flash_attention.h,
 * flash_attention_windowed_forward: the causal form keeps keys from
 * aq-window+1 up to aq (clipped at 0); the bidirectional form keeps keys within
 * window/2 (integer division) on either side of aq, clipped to [0, Lk-1]; a
 * window <= 0 removes the window in both forms.  The causal upper bound is
 * also clipped to Lk-1 so a range never leaves the key axis.
 * Returns lo > hi when nothing is in range.
 */
void mfa_oracle_key_range(int64_t aq, int64_t Lk, int causal, int64_t window,
                          int64_t* lo_out, int64_t* hi_out)
{
    int64_t lo, hi;
    if (causal) {
        hi = aq;
#if ORACLE_MUTANT == 2
        hi = aq - 1;                         /* off by one: excludes the diagonal */
#endif
        lo = 0;
        if (window > 0) {
            lo = aq - window + 1;
#if ORACLE_MUTANT == 3
            lo = aq - window;                /* off by one: one key too many */
#endif
        }
    } else if (window > 0) {
        int64_t half = window / 2;
#if ORACLE_MUTANT == 9
        half = window;                       /* full width on each side */
#endif
        lo = aq - half;
        hi = aq + half;
    } else {
        lo = 0;
        hi = Lk - 1;
    }
    if (lo < 0) lo = 0;
    if (hi > Lk - 1) hi = Lk - 1;
    *lo_out = lo;
    *hi_out = hi;
}

/* Key j of batch b passes the key mask: brotensor flash_attention.h describes
 * the mask as 1 for a valid key and 0 for an invalid one, combined
 * multiplicatively; its bare-core backward drops keys whose mask is at most
 * one half.  Both readings agree on a 0/1 mask: keep iff mask > 0.5. */
static int key_mask_keeps(const float* key_mask, int64_t Lk, int64_t b, int64_t j)
{
    if (key_mask == NULL) return 1;
#if ORACLE_MUTANT == 8
    return 1;                                /* mask ignored */
#elif ORACLE_MUTANT == 13
    (void)b;
    return key_mask[j] > 0.5f;               /* batch 0's mask for every batch */
#else
    return key_mask[b * Lk + j] > 0.5f;
#endif
}

/* Absolute position of query row i: the queries are the last Lq positions of
 * the key sequence shifted by q_offset (brotensor flash_attention.h,
 * flash_attention_windowed_forward; ferrotensor attention.rs,
 * AttentionOptions::causal_offset). */
static int64_t query_position(const oracle_dims* d, int64_t i)
{
#if ORACLE_MUTANT == 10
    (void)d;
    return i;                                /* offset ignored */
#else
    return i + d->q_offset;
#endif
}

/* kv head that serves q head hq: consecutive groups of Hq/Hkv query heads
 * share one kv head (brotensor flash_attention.h, flash_attention_decode GQA
 * note; forge attention.metal forward kernel). */
static int64_t kv_head_of(const oracle_dims* d, int64_t hq)
{
#if ORACLE_MUTANT == 4
    return hq % d->Hkv;                      /* interleaved instead of grouped */
#else
    return hq / (d->Hq / d->Hkv);
#endif
}

/* Visible-key count of query row i of batch b, by testing every key. */
int64_t mfa_oracle_row_count(const float* key_mask, const oracle_dims* d,
                             int64_t b, int64_t i)
{
    int64_t lo, hi, n = 0;
    mfa_oracle_key_range(query_position(d, i), d->Lk, d->causal, d->window, &lo, &hi);
    for (int64_t j = 0; j < d->Lk; ++j)
        if (j >= lo && j <= hi && key_mask_keeps(key_mask, d->Lk, b, j)) ++n;
    return n;
}

/*
 * One output row.  scores must hold Lk doubles of scratch.
 * Writes out[0..D), *lse and *nvis.  A row with no visible key writes zeros
 * and lse = -inf (the pages leave this open; brotensor's decode_len writes
 * zeros for an empty cache, which this follows).
 */
static void oracle_row(const float* q, const float* k, const float* v, const float* key_mask,
                       const oracle_dims* d, int64_t b, int64_t hq, int64_t i,
                       double* out, double* lse, int64_t* nvis, double* scores)
{
    const int64_t D = d->D;
    const int64_t kvh = kv_head_of(d, hq);
    const float* qrow = q + ((b * d->Lq + i) * d->Hq + hq) * D;
#if ORACLE_MUTANT == 12
    qrow = q + ((b * d->Hq + hq) * d->Lq + i) * D;   /* [B,H,L,D] indexing */
#endif
    int64_t lo, hi;
    mfa_oracle_key_range(query_position(d, i), d->Lk, d->causal, d->window, &lo, &hi);

    /* scores of the visible keys; invisible keys never enter the sums */
    int64_t n = 0;
    double m = -INFINITY;
    for (int64_t j = 0; j < d->Lk; ++j) {
        if (!(j >= lo && j <= hi && key_mask_keeps(key_mask, d->Lk, b, j))) {
            scores[j] = NAN;                 /* marks an invisible key */
            continue;
        }
        const float* krow = k + ((b * d->Lk + j) * d->Hkv + kvh) * D;
        double dot = 0.0;
        for (int64_t e = 0; e < D; ++e) dot += (double)qrow[e] * (double)krow[e];
        double s = d->scale * dot;
#if ORACLE_MUTANT == 1
        s = dot;                             /* scale dropped */
#endif
        if (d->softcap > 0.0) {
            /* soft-cap after the scale, before masking and the softmax
             * (brotensor flash_attention.h, flash_attention_decode;
             * forge attention.metal AttnParams) */
#if ORACLE_MUTANT == 7
            s = d->softcap * tanh(s);        /* missing division by the cap */
#elif ORACLE_MUTANT == 14
            s = d->softcap * tanh(dot / d->softcap) * d->scale;  /* cap before scale */
#else
            s = d->softcap * tanh(s / d->softcap);
#endif
        }
        if (d->bias) {
            /* additive mask with size-1 dimensions broadcast (ferrotensor
             * attention.rs, flash_attention_v2 and mask_strides), added to
             * the scaled (and capped) score */
#if ORACLE_MUTANT == 15
            s += d->bias[b * d->bs[0] + hq * d->bs[1] + j * d->bs[2] + i * d->bs[3]];  /* i, j swapped */
#else
            s += d->bias[b * d->bs[0] + hq * d->bs[1] + i * d->bs[2] + j * d->bs[3]];
#endif
        }
        scores[j] = s;
        if (s > m) m = s;
        ++n;
    }
    *nvis = n;
    for (int64_t e = 0; e < D; ++e) out[e] = 0.0;
    if (n == 0 || m == -INFINITY) {          /* no key, or a bias of -inf on every one */
        *lse = -INFINITY;
        return;
    }
    /* softmax row: P_j = exp(s_j - m) / sum_j exp(s_j - m) */
    double sum = 0.0;
    for (int64_t j = 0; j < d->Lk; ++j) {
        if (isnan(scores[j])) continue;
        scores[j] = exp(scores[j] - m);
        sum += scores[j];
    }
    for (int64_t j = 0; j < d->Lk; ++j) {
        if (isnan(scores[j])) continue;
#if ORACLE_MUTANT == 11
        (void)0;                             /* normalisation dropped */
#else
        scores[j] /= sum;
#endif
    }
    /* attention dropout on the normalised weights: a dropped weight becomes
     * 0 and a kept one is divided by 1 - p (ferrotensor attention.rs,
     * flash_attention_v2: dropout_prob and seed); the LSE is not affected */
    if (d->dropout_p > 0.0) {
        for (int64_t j = 0; j < d->Lk; ++j) {
            if (isnan(scores[j])) continue;
#if ORACLE_MUTANT == 16
            scores[j] = mfa_oracle_dropout_keep(d->seed, d->dropout_p, b, hq, j, i) ? scores[j] / (1.0 - d->dropout_p) : 0.0;
#else
            scores[j] = mfa_oracle_dropout_keep(d->seed, d->dropout_p, b, hq, i, j) ? scores[j] / (1.0 - d->dropout_p) : 0.0;
#endif
        }
    }
    /* O = P V */
    for (int64_t j = 0; j < d->Lk; ++j) {
        if (isnan(scores[j])) continue;
#if ORACLE_MUTANT == 5
        const float* vrow = k + ((b * d->Lk + j) * d->Hkv + kvh) * D;  /* K in place of V */
#else
        const float* vrow = v + ((b * d->Lk + j) * d->Hkv + kvh) * D;
#endif
        for (int64_t e = 0; e < D; ++e) out[e] += scores[j] * (double)vrow[e];
    }
    /* natural-log LSE of the scaled (and capped) scores, as the vision_rs
     * flash_attn2.rs forward stores it (running max plus log of the sum) */
#if ORACLE_MUTANT == 6
    *lse = log(sum);                         /* max shift dropped */
#else
    *lse = m + log(sum);
#endif
}

typedef struct {
    const float *q, *k, *v, *key_mask;
    const oracle_dims* d;
    const int64_t* rows;
    int64_t n_rows;
    double *out, *lse;
    int64_t* nvis;
    int64_t first, step;
    int failed;
} row_job;

static void* row_worker(void* arg)
{
    row_job* job = (row_job*)arg;
    double* scores = (double*)malloc(sizeof(double) * (size_t)(job->d->Lk > 0 ? job->d->Lk : 1));
    if (!scores) { job->failed = 1; return NULL; }
    for (int64_t r = job->first; r < job->n_rows; r += job->step) {
        const int64_t* t = job->rows + 3 * r;
        oracle_row(job->q, job->k, job->v, job->key_mask, job->d, t[0], t[1], t[2],
                   job->out + r * job->d->D, job->lse + r, job->nvis + r, scores);
    }
    free(scores);
    return NULL;
}

/*
 * Evaluate n_rows rows given as (b, hq, i) triples.  out is n_rows x D,
 * lse and nvis have n_rows entries.  Rows are dealt round-robin to nthreads
 * POSIX threads; the arithmetic of each row is independent of the threading.
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int mfa_oracle_rows_ext(const float* q, const float* k, const float* v, const float* key_mask,
                        int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D,
                        double scale, int causal, int64_t window, int64_t q_offset, double softcap,
                        const float* bias, const int64_t* bias_strides, double dropout_p, uint64_t seed,
                        const int64_t* rows, int64_t n_rows,
                        double* out, double* lse, int64_t* nvis, int nthreads)
{
    if (!q || !k || !v || !rows || !out || !lse || !nvis) return -1;
    if (B <= 0 || Lq <= 0 || Lk <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return -1;
    if (bias && !bias_strides) return -1;
    if (!(dropout_p >= 0.0 && dropout_p < 1.0)) return -1;
    oracle_dims d = {B, Lq, Lk, Hq, Hkv, D, scale, causal, window, q_offset, softcap,
                     bias, {0, 0, 0, 0}, dropout_p, seed};
    if (bias)
        for (int e = 0; e < 4; ++e) d.bs[e] = bias_strides[e];
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t* t = rows + 3 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= Hq || t[2] < 0 || t[2] >= Lq) return -1;
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    row_job jobs[256];
    pthread_t tids[256];
    int created[256];
    int failed = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (row_job){q, k, v, key_mask, &d, rows, n_rows, out, lse, nvis, t, nthreads, 0};
        created[t] = nthreads > 1 && pthread_create(&tids[t], NULL, row_worker, &jobs[t]) == 0;
        if (!created[t]) row_worker(&jobs[t]);   /* inline when no thread is available */
    }
    for (int t = 0; t < nthreads; ++t) {
        if (created[t]) pthread_join(tids[t], NULL);
        failed |= jobs[t].failed;
    }
    return failed ? -1 : 0;
}

/* mfa_oracle_rows_ext without bias and dropout. */
int mfa_oracle_rows(const float* q, const float* k, const float* v, const float* key_mask,
                    int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D,
                    double scale, int causal, int64_t window, int64_t q_offset, double softcap,
                    const int64_t* rows, int64_t n_rows,
                    double* out, double* lse, int64_t* nvis, int nthreads)
{
    return mfa_oracle_rows_ext(q, k, v, key_mask, B, Lq, Lk, Hq, Hkv, D, scale, causal, window, q_offset,
                               softcap, NULL, NULL, 0.0, 0, rows, n_rows, out, lse, nvis, nthreads);
}

/*
 * Visible-key count of every query row: counts[b*Lq + i] for all b < B and
 * i < Lq (the count does not depend on the head).  Returns the total number of
 * visible (query row, key) pairs over all batches and rows, for one head.
 */
int64_t mfa_oracle_visible_counts(const float* key_mask, int64_t B, int64_t Lq, int64_t Lk,
                                  int causal, int64_t window, int64_t q_offset,
                                  int64_t* counts)
{
    oracle_dims d = {B, Lq, Lk, 1, 1, 1, 1.0, causal, window, q_offset, 0.0, NULL, {0, 0, 0, 0}, 0.0, 0};
    int64_t total = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < Lq; ++i) {
            int64_t n = mfa_oracle_row_count(key_mask, &d, b, i);
            if (counts) counts[b * Lq + i] = n;
            total += n;
        }
    return total;
}

/*
 * Gradients of the forward with respect to Q, K and V for an upstream
 * gradient dO, from the definition: with P the row's softmax weights, Z the
 * dropout factors (keep / (1 - p), or 1) and O = sum_j P_j Z_j V_j,
 *     dV_j += P_j Z_j dO,      dP_j = Z_j <dO, V_j>,
 *     dS_j  = P_j (dP_j - sum_l P_l dP_l)            (softmax derivative),
 *     g_j   = dS_j * d s_j / d <Q, K_j>  = dS_j * scale * (1 - tanh^2) or scale,
 *     dQ   += g_j K_j,         dK_j += g_j Q.
 * (vision_rs flash_attn2.rs, backward kernels: D = rowsum(O * dO) and
 * dS = P (dO . V - D); the additive mask takes no gradient, ferrotensor
 * attention.rs backward.)  Masked keys contribute nothing.  Each (batch, kv
 * head) is one job, so dK/dV sums run in a fixed order.
 */
typedef struct {
    const float *q, *k, *v, *dout, *key_mask;
    const oracle_dims* d;
    double *dq, *dk, *dv;
    int64_t first, step;
    int failed;
} bwd_job;

static void bwd_group(const bwd_job* job, int64_t b, int64_t kvh, double* P, double* Z, double* dP, double* dl)
{
    const oracle_dims* d = job->d;
    const int64_t D = d->D, g = d->Hq / d->Hkv, Lk = d->Lk;
    for (int64_t hq = kvh * g; hq < (kvh + 1) * g; ++hq) {
        for (int64_t i = 0; i < d->Lq; ++i) {
            const float* qrow = job->q + ((b * d->Lq + i) * d->Hq + hq) * D;
            const float* grow = job->dout + ((b * d->Lq + i) * d->Hq + hq) * D;
            double* dqrow = job->dq + ((b * d->Lq + i) * d->Hq + hq) * D;
            int64_t lo, hi;
            mfa_oracle_key_range(query_position(d, i), Lk, d->causal, d->window, &lo, &hi);
            /* scores of the visible keys (NaN marks the others) and d s / d <Q, K> */
            double m = -INFINITY;
            for (int64_t j = 0; j < Lk; ++j) {
                P[j] = NAN;
                if (!(j >= lo && j <= hi && key_mask_keeps(job->key_mask, Lk, b, j))) continue;
                const float* krow = job->k + ((b * Lk + j) * d->Hkv + kvh) * D;
                double dot = 0.0;
                for (int64_t e = 0; e < D; ++e) dot += (double)qrow[e] * (double)krow[e];
                const double t = d->scale * dot;
                double x = t;
                dl[j] = d->scale;
                if (d->softcap > 0.0) {
                    const double th = tanh(t / d->softcap);
                    x = d->softcap * th;
                    dl[j] = d->scale * (1.0 - th * th);
                }
                if (d->bias) x += d->bias[b * d->bs[0] + hq * d->bs[1] + i * d->bs[2] + j * d->bs[3]];
                P[j] = x;
                if (x > m) m = x;
            }
            if (m == -INFINITY) continue;            /* no weight: no gradient */
            /* softmax weights P, dropout factors Z, dP = Z <dO, V_j>, and sum P dP */
            double sum = 0.0;
            for (int64_t j = 0; j < Lk; ++j)
                if (!isnan(P[j])) { P[j] = exp(P[j] - m); sum += P[j]; }
            double pdp = 0.0;
            for (int64_t j = 0; j < Lk; ++j) {
                if (isnan(P[j])) continue;
                P[j] /= sum;
                Z[j] = 1.0;
                if (d->dropout_p > 0.0)
                    Z[j] = mfa_oracle_dropout_keep(d->seed, d->dropout_p, b, hq, i, j) ? 1.0 / (1.0 - d->dropout_p) : 0.0;
                const float* vrow = job->v + ((b * Lk + j) * d->Hkv + kvh) * D;
                double dov = 0.0;
                for (int64_t e = 0; e < D; ++e) dov += (double)grow[e] * (double)vrow[e];
                dP[j] = Z[j] * dov;
                pdp += P[j] * dP[j];
            }
            for (int64_t j = 0; j < Lk; ++j) {
                if (isnan(P[j])) continue;
#if ORACLE_MUTANT == 17
                const double gj = P[j] * (dP[j] - pdp);                 /* logit derivative dropped */
#else
                const double gj = P[j] * (dP[j] - pdp) * dl[j];
#endif
                const float* krow = job->k + ((b * Lk + j) * d->Hkv + kvh) * D;
                double* dkrow = job->dk + ((b * Lk + j) * d->Hkv + kvh) * D;
                double* dvrow = job->dv + ((b * Lk + j) * d->Hkv + kvh) * D;
                for (int64_t e = 0; e < D; ++e) {
                    dqrow[e] += gj * (double)krow[e];
                    dkrow[e] += gj * (double)qrow[e];
                    dvrow[e] += P[j] * Z[j] * (double)grow[e];
                }
            }
        }
    }
}

static void* bwd_worker(void* arg)
{
    bwd_job* job = (bwd_job*)arg;
    const oracle_dims* d = job->d;
    const size_t n = (size_t)(d->Lk > 0 ? d->Lk : 1);
    double* buf = (double*)malloc(sizeof(double) * 4 * n);
    if (!buf) { job->failed = 1; return NULL; }
    for (int64_t t = job->first; t < d->B * d->Hkv; t += job->step)
        bwd_group(job, t / d->Hkv, t % d->Hkv, buf, buf + n, buf + 2 * n, buf + 3 * n);
    free(buf);
    return NULL;
}

/*
 * dQ [B, Lq, Hq, D] and dK, dV [B, Lk, Hkv, D] (fp64, overwritten) for the
 * upstream gradient dout [B, Lq, Hq, D]; other arguments as for
 * mfa_oracle_rows_ext.  Returns 0, or -1 on bad arguments.
 */
int mfa_oracle_bwd(const float* q, const float* k, const float* v, const float* dout, const float* key_mask,
                   int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t D,
                   double scale, int causal, int64_t window, int64_t q_offset, double softcap,
                   const float* bias, const int64_t* bias_strides, double dropout_p, uint64_t seed,
                   double* dq, double* dk, double* dv, int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if (B <= 0 || Lq <= 0 || Lk <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return -1;
    if (bias && !bias_strides) return -1;
    if (!(dropout_p >= 0.0 && dropout_p < 1.0)) return -1;
    oracle_dims d = {B, Lq, Lk, Hq, Hkv, D, scale, causal, window, q_offset, softcap,
                     bias, {0, 0, 0, 0}, dropout_p, seed};
    if (bias)
        for (int e = 0; e < 4; ++e) d.bs[e] = bias_strides[e];
    memset(dq, 0, sizeof(double) * (size_t)(B * Lq * Hq * D));
    memset(dk, 0, sizeof(double) * (size_t)(B * Lk * Hkv * D));
    memset(dv, 0, sizeof(double) * (size_t)(B * Lk * Hkv * D));
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    bwd_job jobs[256];
    pthread_t tids[256];
    int created[256];
    int failed = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (bwd_job){q, k, v, dout, key_mask, &d, dq, dk, dv, t, nthreads, 0};
        created[t] = nthreads > 1 && pthread_create(&tids[t], NULL, bwd_worker, &jobs[t]) == 0;
        if (!created[t]) bwd_worker(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) {
        if (created[t]) pthread_join(tids[t], NULL);
        failed |= jobs[t].failed;
    }
    return failed ? -1 : 0;
}

/* Which mistake (0 = none) this compiled oracle carries; the mutation test reads it. */
int mfa_oracle_mutant(void) { return ORACLE_MUTANT; }
