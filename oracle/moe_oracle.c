/*
 * moe_oracle.c — plain CPU oracle of the MoE expert-FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code with the HIP library.
 *
 * What it computes (HyperMegaMoE issue page, sections 2.1 "forward fusion",
 * 2.2 "backward fusion", 3.1 "Python API" parameter table and 4.1 "routing and
 * expert parallelism"; the correctness-protocol section 6 of the Comet-style
 * overlap explainer page):
 *
 *   slot s = t*K + k expands token t into its K chosen experts e_s with gate g_s
 *   h_s   = x_t · W1[e_s]                (W1 = up_proj_weight [E, H, 2I])
 *   act_s = silu(h_s[0:I]) ⊙ h_s[I:2I]   (SwiGLU, silu(a) = a·sigmoid(a))
 *   o_s   = act_s · W2[e_s]              (W2 = down_proj_weight [E, I, H])
 *   y_t   = Σ_k g_{t,k} · o_{t*K+k}      (top-k gate-weighted combine)
 *
 * The routing step ("dispatch": per-expert counts, offsets and the token
 * permutation into expert-contiguous order) is a counting sort that is stable
 * in the slot index s.  Every floating-point sum is accumulated in double, in
 * ascending index order; bf16 inputs are widened exactly.
 *
 * Readings where the pages leave a step open (the gate half of up_proj is the
 * first I columns; gates are applied at the combine as given, without
 * renormalisation; no biases; gradients overwrite) are the plainest ones and
 * are listed with the rest of the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_I32 = 0, OR_I64 = 1 };
enum {
    OR_OK = 0,
    OR_ERR_ID = 1,      /* an expert id outside [0, E) */
    OR_ERR_ARG = 2,     /* bad sizes or pointers */
    OR_ERR_NOMEM = 3,
    OR_ERR_INVARIANT = 4 /* a self-check of the combine protocol failed */
};

static double widen(const void *p, int dt, int64_t i)
{
    if (dt == OR_F32)
        return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int64_t load_id(const void *ids, int id_dt, int64_t i)
{
    return id_dt == OR_I64 ? ((const int64_t *)ids)[i] : (int64_t)((const int32_t *)ids)[i];
}

static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }
static double silu(double a) { return a * sigmoid(a); }

/* ------------------------------------------------------------------------ */
/* Routing: counting sort of the T*K slots by expert, stable in slot index.  */
/* counts[e], offsets[0..E] (offsets[E] = T*K), sorted_slot[p] = s and its   */
/* inverse slot_pos[s] = p.  Returns OR_ERR_ID on an id outside [0, E).      */
/* ------------------------------------------------------------------------ */
int moe_oracle_route(int64_t T, int64_t K, int64_t E, const void *ids, int id_dt,
                     int32_t *counts, int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos)
{
    if (T < 0 || K <= 0 || E <= 0)
        return OR_ERR_ARG;
    const int64_t TK = T * K;
    for (int64_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t s = 0; s < TK; ++s) {
        int64_t e = load_id(ids, id_dt, s);
        if (e < 0 || e >= E)
            return OR_ERR_ID;
        counts[e] += 1;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor)
        return OR_ERR_NOMEM;
    for (int64_t e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int64_t s = 0; s < TK; ++s) {
        int64_t e = load_id(ids, id_dt, s);
        int32_t p = cursor[e]++;
        sorted_slot[p] = (int32_t)s;
        slot_pos[s] = p;
    }
    free(cursor);
    return OR_OK;
}

/* One expert FFN on one row: h = x·W1e, act = silu(h[:I]) ⊙ h[I:], o = act·W2e.
 * x is given in double; W1e, W2e point at expert e's matrices in storage dtype. */
static void expert_row(int64_t H, int64_t I, const double *x, const void *W1, const void *W2,
                       int dt, int64_t e, double *h, double *act, double *o)
{
    const int64_t w1_base = e * H * 2 * I;
    const int64_t w2_base = e * I * H;
    for (int64_t j = 0; j < 2 * I; ++j)
        h[j] = 0.0;
    for (int64_t c = 0; c < H; ++c) {
        const double xc = x[c];
        const int64_t row = w1_base + c * 2 * I;
        for (int64_t j = 0; j < 2 * I; ++j)
            h[j] += xc * widen(W1, dt, row + j);
    }
    for (int64_t i = 0; i < I; ++i)
        act[i] = silu(h[i]) * h[I + i];
    for (int64_t c = 0; c < H; ++c)
        o[c] = 0.0;
    for (int64_t i = 0; i < I; ++i) {
        const double ai = act[i];
        const int64_t row = w2_base + i * H;
        for (int64_t c = 0; c < H; ++c)
            o[c] += ai * widen(W2, dt, row + c);
    }
}

static void load_row(int64_t H, const void *x, int dt, int64_t t, double *dst)
{
    for (int64_t c = 0; c < H; ++c)
        dst[c] = widen(x, dt, t * H + c);
}

/* The combine protocol of the overlap explainer's section 6: every returned
 * branch bumps done[token]; a token is complete when done == K.  Checked over
 * the permuted order together with the bijection and the count total. */
static int check_route(int64_t T, int64_t K, int64_t E, const int32_t *counts,
                       const int32_t *sorted_slot, const int32_t *slot_pos)
{
    const int64_t TK = T * K;
    int64_t total = 0;
    for (int64_t e = 0; e < E; ++e)
        total += counts[e];
    if (total != TK)
        return OR_ERR_INVARIANT;
    int32_t *done = (int32_t *)calloc((size_t)(T > 0 ? T : 1), sizeof(int32_t));
    if (!done)
        return OR_ERR_NOMEM;
    int rc = OR_OK;
    for (int64_t p = 0; p < TK && rc == OR_OK; ++p) {
        int32_t s = sorted_slot[p];
        if (s < 0 || s >= TK || slot_pos[s] != p)
            rc = OR_ERR_INVARIANT;
        else
            done[s / K] += 1;
    }
    for (int64_t t = 0; t < T && rc == OR_OK; ++t)
        if (done[t] != K)
            rc = OR_ERR_INVARIANT;
    free(done);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Forward over the whole batch, organised as the method's stages:           */
/* route → per-row GMM1 → SwiGLU → GMM2 in expert order → k-ordered combine. */
/* y is [T, H] double.  act_out [TK, I] and o_out [TK, H] (permuted order)   */
/* and the four route arrays are optional outputs (NULL to skip).            */
/* ------------------------------------------------------------------------ */
int moe_oracle_fwd(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, int dt,
                   const void *x, const void *ids, int id_dt, const float *gates,
                   const void *W1, const void *W2, double *y,
                   int32_t *counts_out, int32_t *offsets_out, int32_t *sorted_out,
                   int32_t *slotpos_out, double *act_out, double *o_out)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || !y)
        return OR_ERR_ARG;
    const int64_t TK = T * K;
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sorted_slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)(TK + 1));
    int32_t *slot_pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(TK + 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)((TK > 0 ? TK : 1) * H));
    if (!counts || !offsets || !sorted_slot || !slot_pos || !o) {
        free(counts); free(offsets); free(sorted_slot); free(slot_pos); free(o);
        return OR_ERR_NOMEM;
    }
    int rc = moe_oracle_route(T, K, E, ids, id_dt, counts, offsets, sorted_slot, slot_pos);
    if (rc == OR_OK)
        rc = check_route(T, K, E, counts, sorted_slot, slot_pos);
    if (rc != OR_OK)
        goto done;

    /* Dispatch + GMM1 + SwiGLU + GMM2: each permuted row p is independent. */
#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *h = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *act = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 4)
        for (int64_t p = 0; p < TK; ++p) {
            const int64_t s = sorted_slot[p];
            const int64_t t = s / K;
            const int64_t e = load_id(ids, id_dt, s);
            load_row(H, x, dt, t, xr);
            expert_row(H, I, xr, W1, W2, dt, e, h, act, o + p * H);
            if (act_out)
                memcpy(act_out + p * I, act, sizeof(double) * (size_t)I);
        }
        free(xr); free(h); free(act);
    }

    /* Combine: y_t = Σ_k g_{t,k} o[slot_pos[tK+k]], k ascending. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double *yt = y + t * H;
        for (int64_t c = 0; c < H; ++c)
            yt[c] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double g = (double)gates[t * K + k];
            const double *op = o + (int64_t)slot_pos[t * K + k] * H;
            for (int64_t c = 0; c < H; ++c)
                yt[c] += g * op[c];
        }
    }
    if (o_out)
        memcpy(o_out, o, sizeof(double) * (size_t)(TK * H));
    if (counts_out) memcpy(counts_out, counts, sizeof(int32_t) * (size_t)E);
    if (offsets_out) memcpy(offsets_out, offsets, sizeof(int32_t) * (size_t)(E + 1));
    if (sorted_out) memcpy(sorted_out, sorted_slot, sizeof(int32_t) * (size_t)TK);
    if (slotpos_out) memcpy(slotpos_out, slot_pos, sizeof(int32_t) * (size_t)TK);
done:
    free(counts); free(offsets); free(sorted_slot); free(slot_pos); free(o);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Forward for a list of tokens only, straight from the per-token definition */
/* y_t = Σ_k g_{t,k} · FFN_{e_{t,k}}(x_t).  y_rows is [ntok, H] double.      */
/* Used to check full-size runs on sampled rows.                             */
/* ------------------------------------------------------------------------ */
int moe_oracle_fwd_tokens(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, int dt,
                          const void *x, const void *ids, int id_dt, const float *gates,
                          const void *W1, const void *W2, const int64_t *toks, int64_t ntok,
                          double *y_rows)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0)
        return OR_ERR_ARG;
    for (int64_t n = 0; n < ntok; ++n) {
        if (toks[n] < 0 || toks[n] >= T)
            return OR_ERR_ARG;
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = load_id(ids, id_dt, toks[n] * K + k);
            if (e < 0 || e >= E)
                return OR_ERR_ID;
        }
    }
    const int64_t work = ntok * K;
    double *o = (double *)malloc(sizeof(double) * (size_t)((work > 0 ? work : 1) * H));
    if (!o)
        return OR_ERR_NOMEM;
#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *h = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *act = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < work; ++w) {
            const int64_t t = toks[w / K], k = w % K;
            load_row(H, x, dt, t, xr);
            expert_row(H, I, xr, W1, W2, dt, load_id(ids, id_dt, t * K + k), h, act, o + w * H);
        }
        free(xr); free(h); free(act);
    }
    for (int64_t n = 0; n < ntok; ++n) {
        const int64_t t = toks[n];
        for (int64_t c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)gates[t * K + k] * o[(n * K + k) * H + c];
            y_rows[n * H + c] = acc;
        }
    }
    free(o);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward (HyperMegaMoEGrad, section 2.2 of the issue page), given dY:     */
/*   d_g[t,k] = dY_t · o_s                 dO_s  = g_s · dY_t                */
/*   dact_s   = dO_s · W2[e]^T             db_s  = dact_s ⊙ silu(a_s)        */
/*   da_s     = dact_s ⊙ b_s ⊙ σ(a_s)(1 + a_s(1 − σ(a_s)))   dh_s = [da, db] */
/*   dx_t     = Σ_k dh_s · W1[e]^T                                           */
/*   dW1[e]   = Σ_{s: e_s=e} x_t^T dh_s    dW2[e] = Σ_{s: e_s=e} act_s^T dO_s */
/* with (a_s, b_s) = (h_s[:I], h_s[I:]).  Every output is overwritten; an    */
/* expert that receives no slot gets dW1[e] = dW2[e] = 0.  Outputs double.   */
/* ------------------------------------------------------------------------ */
int moe_oracle_bwd(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, int dt,
                   const void *dy, const void *x, const void *ids, int id_dt, const float *gates,
                   const void *W1, const void *W2, double *dx, double *dW1, double *dW2,
                   double *dg)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0)
        return OR_ERR_ARG;
    const int64_t TK = T * K;
    const size_t tk1 = (size_t)(TK > 0 ? TK : 1);
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sorted_slot = (int32_t *)malloc(sizeof(int32_t) * tk1);
    int32_t *slot_pos = (int32_t *)malloc(sizeof(int32_t) * tk1);
    double *act = (double *)malloc(sizeof(double) * tk1 * (size_t)I);
    double *dh = (double *)malloc(sizeof(double) * tk1 * (size_t)(2 * I));
    double *dO = (double *)malloc(sizeof(double) * tk1 * (size_t)H);
    double *dxp = (double *)malloc(sizeof(double) * tk1 * (size_t)H);
    int rc = OR_OK;
    if (!counts || !offsets || !sorted_slot || !slot_pos || !act || !dh || !dO || !dxp) {
        rc = OR_ERR_NOMEM;
        goto done;
    }
    rc = moe_oracle_route(T, K, E, ids, id_dt, counts, offsets, sorted_slot, slot_pos);
    if (rc == OR_OK)
        rc = check_route(T, K, E, counts, sorted_slot, slot_pos);
    if (rc != OR_OK)
        goto done;

#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *dyr = (double *)malloc(sizeof(double) * (size_t)H);
        double *h = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        double *dact = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 4)
        for (int64_t p = 0; p < TK; ++p) {
            const int64_t s = sorted_slot[p];
            const int64_t t = s / K;
            const int64_t e = load_id(ids, id_dt, s);
            const double g = (double)gates[s];
            load_row(H, x, dt, t, xr);
            load_row(H, dy, dt, t, dyr);
            double *ap = act + p * I;
            expert_row(H, I, xr, W1, W2, dt, e, h, ap, o);
            double d = 0.0;
            for (int64_t c = 0; c < H; ++c)
                d += dyr[c] * o[c];
            dg[s] = d;
            double *dOp = dO + p * H;
            for (int64_t c = 0; c < H; ++c)
                dOp[c] = g * dyr[c];
            const int64_t w2_base = e * I * H;
            for (int64_t i = 0; i < I; ++i) {
                double acc = 0.0;
                for (int64_t c = 0; c < H; ++c)
                    acc += dOp[c] * widen(W2, dt, w2_base + i * H + c);
                dact[i] = acc;
            }
            double *dhp = dh + p * 2 * I;
            for (int64_t i = 0; i < I; ++i) {
                const double a = h[i], b = h[I + i], sg = sigmoid(a);
                dhp[i] = dact[i] * b * sg * (1.0 + a * (1.0 - sg));
                dhp[I + i] = dact[i] * silu(a);
            }
            const int64_t w1_base = e * H * 2 * I;
            double *dxr = dxp + p * H;
            for (int64_t c = 0; c < H; ++c) {
                double acc = 0.0;
                const int64_t row = w1_base + c * 2 * I;
                for (int64_t j = 0; j < 2 * I; ++j)
                    acc += dhp[j] * widen(W1, dt, row + j);
                dxr[c] = acc;
            }
        }
        free(xr); free(dyr); free(h); free(o); free(dact);
    }

    /* Combine(dX): dx_t = Σ_k dx_perm[slot_pos[tK+k]], k ascending. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += dxp[(int64_t)slot_pos[t * K + k] * H + c];
            dx[t * H + c] = acc;
        }
    }

    /* Weight gradients, reduced over each expert's segment in ascending p. */
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t e = 0; e < E; ++e) {
        for (int64_t c = 0; c < H; ++c) {
            double *row = dW1 + (e * H + c) * 2 * I;
            for (int64_t j = 0; j < 2 * I; ++j)
                row[j] = 0.0;
            for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) {
                const double xv = widen(x, dt, (int64_t)(sorted_slot[p] / K) * H + c);
                const double *dhp = dh + p * 2 * I;
                for (int64_t j = 0; j < 2 * I; ++j)
                    row[j] += xv * dhp[j];
            }
        }
    }
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t e = 0; e < E; ++e) {
        for (int64_t i = 0; i < I; ++i) {
            double *row = dW2 + (e * I + i) * H;
            for (int64_t c = 0; c < H; ++c)
                row[c] = 0.0;
            for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) {
                const double av = act[p * I + i];
                const double *dOp = dO + p * H;
                for (int64_t c = 0; c < H; ++c)
                    row[c] += av * dOp[c];
            }
        }
    }
done:
    free(counts); free(offsets); free(sorted_slot); free(slot_pos);
    free(act); free(dh); free(dO); free(dxp);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Sampled backward for full-size checks, from the same formulas:            */
/*   dx and d_g for the tokens in toks[ntok]   → dx_rows [ntok,H], dg_rows   */
/*   dW1[e][:, j] for the (e, j) pairs in w1c  → dW1_cols [n1, H]            */
/*   dW2[e][i, :] for the (e, i) pairs in w2r  → dW2_rows [n2, H]            */
/* ------------------------------------------------------------------------ */
int moe_oracle_bwd_sampled(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, int dt,
                           const void *dy, const void *x, const void *ids, int id_dt,
                           const float *gates, const void *W1, const void *W2,
                           const int64_t *toks, int64_t ntok, double *dx_rows, double *dg_rows,
                           const int64_t *w1c, int64_t n1, double *dW1_cols,
                           const int64_t *w2r, int64_t n2, double *dW2_rows)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0)
        return OR_ERR_ARG;
    const int64_t TK = T * K;
    for (int64_t s = 0; s < TK; ++s) {
        int64_t e = load_id(ids, id_dt, s);
        if (e < 0 || e >= E)
            return OR_ERR_ID;
    }
    for (int64_t n = 0; n < ntok; ++n)
        if (toks[n] < 0 || toks[n] >= T)
            return OR_ERR_ARG;
    for (int64_t n = 0; n < n1; ++n)
        if (w1c[2 * n] < 0 || w1c[2 * n] >= E || w1c[2 * n + 1] < 0 || w1c[2 * n + 1] >= 2 * I)
            return OR_ERR_ARG;
    for (int64_t n = 0; n < n2; ++n)
        if (w2r[2 * n] < 0 || w2r[2 * n] >= E || w2r[2 * n + 1] < 0 || w2r[2 * n + 1] >= I)
            return OR_ERR_ARG;

    /* token rows: dx_t and d_g[t, :] */
#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *dyr = (double *)malloc(sizeof(double) * (size_t)H);
        double *h = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *act = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        double *dh = (double *)malloc(sizeof(double) * (size_t)(2 * I));
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < ntok; ++n) {
            const int64_t t = toks[n];
            load_row(H, x, dt, t, xr);
            load_row(H, dy, dt, t, dyr);
            double *dxr = dx_rows + n * H;
            for (int64_t c = 0; c < H; ++c)
                dxr[c] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t s = t * K + k, e = load_id(ids, id_dt, s);
                const double g = (double)gates[s];
                expert_row(H, I, xr, W1, W2, dt, e, h, act, o);
                double d = 0.0;
                for (int64_t c = 0; c < H; ++c)
                    d += dyr[c] * o[c];
                dg_rows[n * K + k] = d;
                const int64_t w2_base = e * I * H;
                for (int64_t i = 0; i < I; ++i) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < H; ++c)
                        acc += g * dyr[c] * widen(W2, dt, w2_base + i * H + c);
                    const double a = h[i], b = h[I + i], sg = sigmoid(a);
                    dh[i] = acc * b * sg * (1.0 + a * (1.0 - sg));
                    dh[I + i] = acc * silu(a);
                }
                const int64_t w1_base = e * H * 2 * I;
                for (int64_t c = 0; c < H; ++c) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < 2 * I; ++j)
                        acc += dh[j] * widen(W1, dt, w1_base + c * 2 * I + j);
                    dxr[c] += acc;
                }
            }
        }
        free(xr); free(dyr); free(h); free(act); free(o); free(dh);
    }

    /* dW1 columns: dW1[e][c][j] = Σ_{s: e_s=e, s ascending} x[t_s][c] · dh_s[j] */
#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *dyr = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n1; ++n) {
            const int64_t e = w1c[2 * n], j = w1c[2 * n + 1], i = j % I;
            double *col = dW1_cols + n * H;
            for (int64_t c = 0; c < H; ++c)
                col[c] = 0.0;
            for (int64_t s = 0; s < TK; ++s) {
                if (load_id(ids, id_dt, s) != e)
                    continue;
                const int64_t t = s / K;
                load_row(H, x, dt, t, xr);
                load_row(H, dy, dt, t, dyr);
                double a = 0.0, b = 0.0, dact = 0.0;
                for (int64_t c = 0; c < H; ++c) {
                    a += xr[c] * widen(W1, dt, (e * H + c) * 2 * I + i);
                    b += xr[c] * widen(W1, dt, (e * H + c) * 2 * I + I + i);
                }
                for (int64_t c = 0; c < H; ++c)
                    dact += (double)gates[s] * dyr[c] * widen(W2, dt, (e * I + i) * H + c);
                const double sg = sigmoid(a);
                const double dhj = (j < I) ? dact * b * sg * (1.0 + a * (1.0 - sg)) : dact * silu(a);
                for (int64_t c = 0; c < H; ++c)
                    col[c] += xr[c] * dhj;
            }
        }
        free(xr); free(dyr);
    }

    /* dW2 rows: dW2[e][i][c] = Σ_{s: e_s=e, s ascending} act_s[i] · g_s · dY[t_s][c] */
#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n2; ++n) {
            const int64_t e = w2r[2 * n], i = w2r[2 * n + 1];
            double *row = dW2_rows + n * H;
            for (int64_t c = 0; c < H; ++c)
                row[c] = 0.0;
            for (int64_t s = 0; s < TK; ++s) {
                if (load_id(ids, id_dt, s) != e)
                    continue;
                const int64_t t = s / K;
                load_row(H, x, dt, t, xr);
                double a = 0.0, b = 0.0;
                for (int64_t c = 0; c < H; ++c) {
                    a += xr[c] * widen(W1, dt, (e * H + c) * 2 * I + i);
                    b += xr[c] * widen(W1, dt, (e * H + c) * 2 * I + I + i);
                }
                const double actv = silu(a) * b * (double)gates[s];
                for (int64_t c = 0; c < H; ++c)
                    row[c] += actv * widen(dy, dt, t * H + c);
            }
        }
        free(xr);
    }
    return OR_OK;
}

int moe_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
