/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for MoE token
 * routing followed by moe_align_block_size.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library; it has its own bf16 decoding and rounding.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math), so
 * every double operation below is a single IEEE-754 operation in program
 * order.
 *
 * Sources (web pages; cited by title and section):
 *   [R]  "[AMD] One-launch small-M MoE router ... on gfx950" (sglang),
 *        sections Motivation, Modifications, Accuracy Tests.
 *   [A]  "W4A16 MoE prefill: M-aware moe_align block size" (ROCm vLLM),
 *        sections Purpose, Scope and safety.
 *   [N]  "Open-Source ROCm Kernels for AMD MI350X" (Netra Kernel blog),
 *        section "Sampling: make small batches large enough".
 *
 * What each function computes, in the order the route takes:
 *   or_gate            z[m][e] = sum_h x[m][h] * W[e][h] in double, summed
 *                      sequentially over h; the shared logit likewise  ([R]
 *                      Modifications: every gate row, routed and shared, is a
 *                      dot product over the hidden size; [R] Accuracy Tests:
 *                      the reference accumulates in double and
 *                      only then rounds to bf16).
 *   or_round_bf16      double -> bf16, round to nearest, ties to even, in ONE
 *                      step from double ([R] Modifications: the routed logits
 *                      are rounded to bf16 before top-k).
 *   or_select          top-k on the rounded logits, ties to the lowest expert
 *                      id, then softmax over all routed experts and
 *                      renormalisation over the chosen k, then the shared slot
 *                      k = (E, sigmoid(s) * scale) ([R] Modifications).
 *   or_select_alignment  A = 128 when M*k >= 128*E, else 64 ([A] Purpose,
 *                      second commit: tier on routed rows per expert).
 *   or_align           stable counting sort of the (token, slot) pairs by
 *                      expert, each touched expert padded to a multiple of A;
 *                      npp = sum over touched experts of ceil(c_e/A)*A ([A]
 *                      Purpose).
 *   or_align_local     the align of one expert-parallel rank: each pair's
 *                      global expert id goes through the rank's expert map
 *                      (its local id, or -1 for an expert another rank
 *                      owns) and the pairs of local experts are aligned by
 *                      local id as or_align does; non-local pairs are
 *                      skipped.  (The design the scope table's EP row
 *                      describes; the pages themselves run the router
 *                      replicated, [R] Motivation.)
 *   or_grouped_gemm    the consumer of the align output that [A] Purpose
 *                      describes: block b of A slots (launched while
 *                      b*A < npp) multiplies its rows by the weights of
 *                      expert expert_ids[b]; a slot holding pair p < M*S
 *                      produces y[p][n] = sum_h x[p / S][h] * W[e][n][h]
 *                      (double, sequential in h); padding produces nothing.
 *   or_argmax_rows     row-wise argmax of an fp32 matrix with PyTorch's
 *                      semantics as [N] Sampling states them: a NaN beats
 *                      every number and the first NaN beats later ones; among
 *                      equal numbers the lowest index wins; -0 equals +0.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - rounding mode of the logit rounding: nearest, ties to even;
 *   - slot order inside a row: (rounded logit descending, id ascending), the
 *     order k successive lowest-id-wins argmax passes produce; shared last;
 *   - -0 and +0 compare equal (double comparison does this by itself);
 *   - the shared logit is NOT rounded to bf16 (the page rounds the routed
 *     logits only);
 *     round_shared=1 selects the other reading for diagnostics;
 *   - align sees the shared expert as id E among E' = E+1 experts;
 *   - inside one expert, pairs keep ascending flat index i = m*S + slot;
 *   - padding entries hold the sentinel M*S; ids outside [0, E') are skipped;
 *   - untouched experts get no block.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ECAPACITY (-3)

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 bit pattern -> double.  A bf16 value is the upper half of an IEEE
 * binary32 word, so placing the 16 bits on top of 16 zero bits gives the
 * float exactly, and float -> double is exact. */
double or_bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* double -> bf16 bits, round to nearest, ties to even, directly from the
 * double (no intermediate binary32 rounding, which could round twice).
 *
 * bf16 keeps 8 significant bits and binary32's exponent range.  For
 * z = f * 2^ex with 0.5 <= |f| < 1 the representable neighbours are spaced
 * q = 2^(ex-8); below the smallest normal 2^-126 the spacing is fixed at
 * 2^-133 (subnormals).  nearbyint() under FE_TONEAREST rounds half to even.
 * A result of magnitude 2^128 or more is beyond the largest finite bf16 and
 * becomes infinity. */
uint16_t or_round_bf16(double z)
{
    if (isnan(z))
        return 0x7FC0;
    if (isinf(z))
        return z > 0 ? 0x7F80 : 0xFF80;
    int ex;
    (void)frexp(z, &ex);
    int qexp = ex - 8;
    if (qexp < -133)
        qexp = -133;
    int saved = fegetround();
    fesetround(FE_TONEAREST);
    double r = ldexp(nearbyint(ldexp(z, -qexp)), qexp);
    fesetround(saved);
    if (fabs(r) >= ldexp(1.0, 128))
        return signbit(r) ? 0xFF80 : 0x7F80;
    /* r is a bf16 value, hence also exactly a binary32 value. */
    float f = (float)r;
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return (uint16_t)(w >> 16);
}

/* ---------------------------------------------------------------- gate -- */

/* z[m*E + e] = sum_{h=0}^{H-1} x[m][h] * W[e][h], sequential in h, double.
 * If ws != NULL, s[m] = sum_h x[m][h] * ws[h] likewise.
 * x is [M, H] row-major, W is [E, H] row-major (nn.Linear [out, in] layout,
 * read in place), ws is [H].  All three hold bf16 bit patterns.
 * [R] Modifications (gate rows, routed and shared, with fp32-or-better
 * accumulation); [R] Accuracy Tests (reference accumulates in fp64). */
void or_gate(const uint16_t *x, const uint16_t *W, const uint16_t *ws,
             int M, int H, int E, double *z, double *s, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for collapse(2) schedule(static)
#endif
    for (int m = 0; m < M; ++m)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += or_bf16_value(x[(size_t)m * H + h]) *
                       or_bf16_value(W[(size_t)e * H + h]);
            z[(size_t)m * E + e] = acc;
        }
    if (ws && s) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += or_bf16_value(x[(size_t)m * H + h]) * or_bf16_value(ws[h]);
            s[m] = acc;
        }
    }
}

/* -------------------------------------------------------------- select -- */

typedef struct {
    double r; /* rounded logit, as a double */
    int e;    /* expert id */
} or_cand;

/* Larger rounded logit first; equal logits (including -0 == +0): lower id
 * first.  This is a strict total order on distinct ids, so the sort result
 * does not depend on the sort algorithm's stability.
 * [R] Modifications: on equal logits the lower expert id is chosen. */
static int or_cand_cmp(const void *pa, const void *pb)
{
    const or_cand *a = (const or_cand *)pa, *b = (const or_cand *)pb;
    if (a->r > b->r)
        return -1;
    if (a->r < b->r)
        return 1;
    return (a->e < b->e) ? -1 : (a->e > b->e);
}

/* Steps after the gate, for M rows of routed logits z [M, E] (double) and
 * optional shared logits s [M]:
 *   1. r = bf16_RNE(z)                           ([R] Modifications)
 *   2. sort experts by (r desc, id asc); ids[m][0..k-1] = the first k
 *                                                ([R] Modifications)
 *   3. p_e = softmax over all E rounded logits; w_j = p_{id_j} / sum over the
 *      chosen k of p (softmax, then renormalisation over the chosen
 *      experts: [R] Motivation and Modifications).  Shifting by the row maximum changes no value
 *      mathematically and keeps exp() in range.
 *   4. if has_shared: ids[m][k] = E, w[m][k] = scale * sigmoid(s[m])
 *                                                ([R] Modifications, slot k)
 *      The shared logit is used unrounded unless round_shared != 0.
 * ids and weights are [M, S] with S = k + has_shared. */
int or_select(const double *z, const double *s, int M, int E, int k,
              int has_shared, double scale, int round_shared,
              int32_t *ids, float *weights, uint16_t *r_bits_out, int nthreads)
{
    if (M < 0 || E < 1 || k < 1 || k > E || (has_shared && !s))
        return OR_EINVAL;
    const int S = k + (has_shared ? 1 : 0);
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        or_cand *c = (or_cand *)malloc(sizeof(or_cand) * (size_t)E);
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
        if (!c || !p) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int m = 0; m < M; ++m) {
            if (!c || !p)
                continue;
            const double *zr = z + (size_t)m * E;
            /* 1. round */
            for (int e = 0; e < E; ++e) {
                uint16_t b = or_round_bf16(zr[e]);
                if (r_bits_out)
                    r_bits_out[(size_t)m * E + e] = b;
                c[e].r = or_bf16_value(b);
                c[e].e = e;
            }
            /* 3a. full softmax over the E rounded logits (before sorting, in
             * id order) */
            double rmax = c[0].r;
            for (int e = 1; e < E; ++e)
                if (c[e].r > rmax)
                    rmax = c[e].r;
            double denom = 0.0;
            for (int e = 0; e < E; ++e) {
                p[e] = exp(c[e].r - rmax);
                denom += p[e];
            }
            for (int e = 0; e < E; ++e)
                p[e] /= denom;
            /* 2. select */
            qsort(c, (size_t)E, sizeof(or_cand), or_cand_cmp);
            /* 3b. renormalise over the chosen k */
            double sel = 0.0;
            for (int j = 0; j < k; ++j)
                sel += p[c[j].e];
            for (int j = 0; j < k; ++j) {
                ids[(size_t)m * S + j] = c[j].e;
                weights[(size_t)m * S + j] = (float)(p[c[j].e] / sel);
            }
            /* 4. shared slot */
            if (has_shared) {
                double sm = s[m];
                if (round_shared)
                    sm = or_bf16_value(or_round_bf16(sm));
                ids[(size_t)m * S + k] = E;
                weights[(size_t)m * S + k] = (float)(scale / (1.0 + exp(-sm)));
            }
        }
        free(c);
        free(p);
    }
    return err ? OR_EINVAL : OR_OK;
}

/* Whole route: gate (double) then select.  z_out [M, E] and s_out [M] are
 * optional copies of the double logits (the tests use them to measure each
 * row's rank-k / rank-k+1 margin). */
int or_route(const uint16_t *x, const uint16_t *W, const uint16_t *ws, int M,
             int H, int E, int k, double scale, int round_shared,
             int32_t *ids, float *weights, double *z_out, double *s_out,
             int nthreads)
{
    if (M < 0 || H < 1 || E < 1 || k < 1 || k > E)
        return OR_EINVAL;
    double *z = z_out ? z_out : (double *)malloc(sizeof(double) * (size_t)M * E + 1);
    double *s = NULL;
    if (ws)
        s = s_out ? s_out : (double *)malloc(sizeof(double) * (size_t)M + 1);
    if (!z || (ws && !s))
        return OR_EINVAL;
    or_gate(x, W, ws, M, H, E, z, s, nthreads);
    int rc = or_select(z, s, M, E, k, ws != NULL, scale, round_shared, ids,
                       weights, NULL, nthreads);
    if (!z_out)
        free(z);
    if (ws && !s_out)
        free(s);
    return rc;
}

/* --------------------------------------------------------------- align -- */

/* [A] Purpose: the crossover is one full padding block of routed rows per
 * expert, and the tier is chosen on tokens * top-k / E.  Reaching one block
 * per expert already selects 128, so the comparison is >=.  The routed k and
 * E are used (not the shared slot). */
int or_select_alignment(int M, int k, int E)
{
    return ((int64_t)M * k >= (int64_t)128 * E) ? 128 : 64;
}

/* Largest npp any routing of n = M*S pairs over E' experts can produce:
 * every pair, plus at most A-1 padding entries for each touched expert, and
 * at most min(E', n) experts are touched.  With loose != 0, the form that
 * pads every expert: n + E'*(A-1) ([A] Scope and safety gives that number
 * for the workspace at 128 and 1024 tokens). */
int64_t or_align_capacity(int M, int S, int Eprime, int A, int loose)
{
    int64_t n = (int64_t)M * S;
    int64_t touched = loose ? Eprime : (Eprime < n ? Eprime : n);
    return n + touched * (int64_t)(A - 1);
}

/* moe_align_block_size, by stable counting sort ([A] Purpose):
 *   c_e  = number of pairs i in [0, n) with ids[i] == e, for e in [0, E')
 *   P_e  = ceil(c_e / A) * A          (0 for an untouched expert)
 *   off_e = sum_{e' < e} P_e'          npp = sum_e P_e
 *   sorted[off_e + j] = j-th (ascending) flat index whose id is e, for
 *   j < c_e; sorted[off_e + c_e .. off_e + P_e) = n (sentinel);
 *   expert_ids[b] = e for b in [off_e / A, (off_e + P_e) / A).
 * Entries at or past npp (and expert_ids past npp/A) are left untouched. */
int or_align(const int32_t *ids, int M, int S, int Eprime, int A,
             int32_t *sorted, int64_t sorted_cap, int32_t *expert_ids,
             int64_t expert_cap, int32_t *npp_out)
{
    if (M < 0 || S < 1 || Eprime < 1 || A < 1)
        return OR_EINVAL;
    const int64_t n = (int64_t)M * S;
    int64_t *cnt = (int64_t *)calloc((size_t)Eprime, sizeof(int64_t));
    int64_t *off = (int64_t *)calloc((size_t)Eprime, sizeof(int64_t));
    if (!cnt || !off) {
        free(cnt);
        free(off);
        return OR_EINVAL;
    }
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = ids[i];
        if (e >= 0 && e < Eprime)
            cnt[e] += 1;
    }
    int64_t total = 0;
    for (int e = 0; e < Eprime; ++e) {
        off[e] = total;
        total += (cnt[e] + A - 1) / A * A;
    }
    if (total > sorted_cap || total / A > expert_cap) {
        free(cnt);
        free(off);
        return OR_ECAPACITY;
    }
    for (int64_t p = 0; p < total; ++p)
        sorted[p] = (int32_t)n;
    for (int e = 0; e < Eprime; ++e) {
        int64_t padded = (cnt[e] + A - 1) / A * A;
        for (int64_t b = off[e] / A; b < (off[e] + padded) / A; ++b)
            expert_ids[b] = e;
    }
    /* scatter in ascending flat index: off[] becomes each expert's fill
     * cursor */
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = ids[i];
        if (e >= 0 && e < Eprime)
            sorted[off[e]++] = (int32_t)i;
    }
    *npp_out = (int32_t)total;
    free(cnt);
    free(off);
    return OR_OK;
}

/* Align of one expert-parallel rank (see the header): map, then or_align
 * over the local experts.  Global ids outside [0, Eglobal) and map entries
 * outside [0, Elocal) are not local. */
int or_align_local(const int32_t *ids, int M, int S, int Eglobal, const int32_t *map, int Elocal,
                   int A, int32_t *sorted, int64_t sorted_cap, int32_t *expert_ids,
                   int64_t expert_cap, int32_t *npp_out)
{
    if (M < 0 || S < 1 || Eglobal < 1 || Elocal < 1)
        return OR_EINVAL;
    const int64_t n = (int64_t)M * S;
    int32_t *loc = (int32_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    if (!loc)
        return OR_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t e = ids[i];
        const int32_t l = (e >= 0 && e < Eglobal) ? map[e] : -1;
        loc[i] = (l >= 0 && l < Elocal) ? l : -1;
    }
    const int rc = or_align(loc, M, S, Elocal, A, sorted, sorted_cap, expert_ids, expert_cap, npp_out);
    free(loc);
    return rc;
}

/* Grouped expert GEMM over the align output (see the header).  y [M*S, N]
 * is written only for the pairs that appear in sorted[0, npp). */
int or_grouped_gemm(const uint16_t *x, int M, int H, const uint16_t *W, int Ep, int N, int S,
                    const int32_t *sorted, const int32_t *expert_ids, int64_t npp, int A, double *y,
                    int nthreads)
{
    if (M < 0 || H < 1 || Ep < 1 || N < 1 || S < 1 || A < 1 || npp < 0 || npp % A != 0)
        return OR_EINVAL;
    const int64_t n = (int64_t)M * S;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16) if (nthreads != 1)
#endif
    for (int64_t j = 0; j < npp; ++j) {
        const int32_t p = sorted[j];
        const int32_t e = expert_ids[j / A];
        if (p < 0 || p >= n || e < 0 || e >= Ep)
            continue; /* padding slot */
        const uint16_t *xr = x + (size_t)(p / S) * H;
        for (int c = 0; c < N; ++c) {
            const uint16_t *wr = W + ((size_t)e * N + c) * H;
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += or_bf16_value(xr[h]) * or_bf16_value(wr[h]);
            y[(size_t)p * N + c] = acc;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------- array helpers -- */

/* Element-wise or_round_bf16 / or_bf16_value over arrays (for the tests). */
void or_round_bf16_array(const double *z, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_round_bf16(z[i]);
}

void or_bf16_value_array(const uint16_t *bits, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_bf16_value(bits[i]);
}

/* -------------------------------------------------------------- argmax -- */

/* out[r] = index of the winner of row r of x [R, N] (row stride ld floats),
 * scanning the row left to right and replacing the current winner only when
 * the new value beats it ([N] Sampling): a NaN beats any number, a NaN never
 * loses its place to a later NaN, and a number beats another only when it is
 * strictly greater (so equal numbers, including -0 and +0, keep the lowest
 * index).  Returns OR_EINVAL for R < 0, N < 1 or ld < N. */
int or_argmax_rows(const float *x, int64_t R, int64_t N, int64_t ld, int64_t *out, int nthreads)
{
    if (R < 0 || N < 1 || ld < N)
        return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) if (nthreads != 1)
#endif
    for (int64_t r = 0; r < R; ++r) {
        const float *row = x + r * ld;
        int64_t best = 0;
        for (int64_t j = 1; j < N; ++j) {
            const float b = row[best], v = row[j];
            if (isnan(b))
                break; /* the first NaN has won the row */
            if (isnan(v) || v > b)
                best = j;
        }
        out[r] = best;
    }
    return OR_OK;
}

