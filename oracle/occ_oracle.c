/*
 * occ_oracle.c -- plain, slow CPU oracle for Occult's MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This code is loaded by the tests, by the smoke
 * check and by the benchmark's CPU-baseline leg, and by nothing else; the
 * product path never calls it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * Source: "Occult: Optimizing Collaborative Communication across Experts for
 * Accelerated Parallel MoE Training and Inference" (Luo et al., ICML 2025,
 * arXiv 2505.13345).  Each function names the passage it follows.  Floating
 * point is fp64 unless the passage (or a stated reading) fixes the precision.
 *
 * Readings taken where the paper is silent or garbled (each one is listed in
 * the design notes of the repository):
 *   - top-k order is (logit descending, expert index ascending), on the fp32
 *     logits; the k weights are the full softmax probabilities, not
 *     renormalised (Eq. 2 only zeroes the entries outside the top k);
 *   - the expert FFN is SwiGLU: E(x) = W_down (silu(W_gate x) * (W_up x));
 *   - shared experts are dense, ungated, weight 1;
 *   - BRIM entries equal to -1 are skipped;
 *   - the co-activation graph C keeps its diagonal (the expert loads); P uses
 *     the largest off-diagonal entry as its maximum and has a zero diagonal;
 *   - CT is the mean number of distinct groups per token;
 *   - Algorithm 1 runs on the integer counts C (the 1/|L| and 1/max factors
 *     do not change any argmax or argmin), ties go to the lowest index, and
 *     a group grows while it holds fewer than Ne/Nd experts.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_PRUNE_OFF = 0, ORC_PRUNE_TRAVERSE = 1, ORC_PRUNE_GROUPSUM = 2 };
enum { ORC_OK = 0, ORC_BAD = 1 };

/* One element of an fp32 or bf16 array, exactly, as a double.  A bf16 value
 * is the upper half of an fp32 bit pattern. */
static double elem(const void *p, int dtype, size_t i)
{
    if (dtype == ORC_F32)
        return (double)((const float *)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Group (device) and position inside the group of every expert, from the
 * placement L: Nd lists of n = Ne/Nd experts (section 3.2).  Returns ORC_BAD
 * unless L is a permutation of 0..Ne-1. */
static int group_table(int Ne, int Nd, const int32_t *L, int *grp, int *slot)
{
    if (Nd <= 0 || Ne % Nd != 0)
        return ORC_BAD;
    int n = Ne / Nd;
    for (int e = 0; e < Ne; e++)
        grp[e] = -1;
    for (int g = 0; g < Nd; g++)
        for (int j = 0; j < n; j++) {
            int e = L[g * n + j];
            if (e < 0 || e >= Ne || grp[e] != -1)
                return ORC_BAD;
            grp[e] = g;
            if (slot)
                slot[e] = j;
        }
    return ORC_OK;
}

/* Does expert a come before expert b in routing-score order? */
static int ranks_before(const float *l, int a, int b)
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

/* All Ne experts in routing-score order (a plain insertion sort). */
static void score_order(const float *l, int Ne, int *ord)
{
    for (int i = 0; i < Ne; i++) {
        int e = i, q = i;
        while (q > 0 && ranks_before(l, e, ord[q - 1])) {
            ord[q] = ord[q - 1];
            q--;
        }
        ord[q] = e;
    }
}

/*
 * Router, Eq. 2 (section 2.1): R(x) = Top-K(Softmax(g(x)), k).  The logits
 * g(x) are given.  Softmax is monotone, so the top k of the probabilities are
 * the top k of the logits.
 *
 * Collaboration pruning (section 3.3, routing-score-based): the token's
 * experts are restricted to G groups, then the top k experts inside those
 * groups are taken in descending score order.  The groups are found
 *   TRAVERSE: by walking the token's k routed experts in descending score
 *             and collecting their groups until G are reached;
 *   GROUPSUM: by ranking the groups that hold at least one of the k routed
 *             experts by the fp32 sum (taken in top-k order) of those
 *             experts' logits, ties to the lower group, and keeping G.
 * Weights stay the full-softmax probabilities.
 *
 * ids[t*k + j] is the j-th chosen expert, w the matching probability.
 */
int orc_route(int T, int Ne, int k, const float *logits, int Nd, const int32_t *L,
              int prune_rule, int G, int32_t *ids, double *w)
{
    if (T < 0 || k < 1 || k > Ne)
        return ORC_BAD;
    int *grp = malloc(sizeof(int) * Ne), *ord = malloc(sizeof(int) * Ne);
    int *chosen = malloc(sizeof(int) * Nd), *elig = malloc(sizeof(int) * Nd);
    float *score = malloc(sizeof(float) * Nd);
    int rc = group_table(Ne, Nd, L, grp, NULL);
    int prune = prune_rule != ORC_PRUNE_OFF && G < Nd;
    if (prune && (G < 1 || G * (Ne / Nd) < k))
        rc = ORC_BAD;
    for (int t = 0; t < T && rc == ORC_OK; t++) {
        const float *l = logits + (size_t)t * Ne;
        score_order(l, Ne, ord);

        double m = l[ord[0]], s = 0.0;
        for (int e = 0; e < Ne; e++)
            s += exp((double)l[e] - m);

        for (int g = 0; g < Nd; g++)
            chosen[g] = !prune;
        if (prune && prune_rule == ORC_PRUNE_TRAVERSE) {
            int have = 0;
            for (int j = 0; j < k && have < G; j++) {
                int g = grp[ord[j]];
                if (!chosen[g]) {
                    chosen[g] = 1;
                    have++;
                }
            }
        } else if (prune && prune_rule == ORC_PRUNE_GROUPSUM) {
            for (int g = 0; g < Nd; g++) {
                score[g] = 0.0f;
                elig[g] = 0;
            }
            for (int j = 0; j < k; j++) {
                int g = grp[ord[j]];
                score[g] = score[g] + l[ord[j]];
                elig[g] = 1;
            }
            for (int r = 0; r < G; r++) {
                int best = -1;
                for (int g = 0; g < Nd; g++)
                    if (elig[g] && !chosen[g] && (best < 0 || score[g] > score[best]))
                        best = g;
                if (best < 0)
                    break;
                chosen[best] = 1;
            }
        } else if (prune) {
            rc = ORC_BAD;
        }

        int j = 0;
        for (int q = 0; q < Ne && j < k; q++) {
            int e = ord[q];
            if (!chosen[grp[e]])
                continue;
            ids[(size_t)t * k + j] = e;
            w[(size_t)t * k + j] = exp((double)l[e] - m) / s;
            j++;
        }
        if (j != k)
            rc = ORC_BAD;
    }
    free(grp); free(ord); free(chosen); free(elig); free(score);
    return rc;
}

/*
 * Expert similarity table, appendix A.3, Eq. 6-8.  H is the profiled
 * router-logit matrix (tokens x Ne).  Eq. 8's numerator and denominator are
 * built from the Gram matrix of H's columns, gram[i][j] = sum_t H[t][i] H[t][j],
 * which is accumulated batch by batch: this call adds one batch, tokens in
 * ascending order, in fp64 (the products of two fp32 logits are exact).
 */
int orc_sim_accumulate(int T, int Ne, const float *logits, double *gram)
{
    if (T < 0 || Ne < 1)
        return ORC_BAD;
    for (int i = 0; i < Ne; i++)
        for (int j = 0; j < Ne; j++) {
            double acc = gram[(size_t)i * Ne + j];
            for (int t = 0; t < T; t++)
                acc += (double)logits[(size_t)t * Ne + i] * (double)logits[(size_t)t * Ne + j];
            gram[(size_t)i * Ne + j] = acc;
        }
    return ORC_OK;
}

/*
 * The table itself.  Eq. 7 (equal to Eq. 8, whose 1/N factors cancel): the
 * squared cosine similarity of columns i and j,
 *   T2[i][j] = gram[i][j]^2 / (gram[i][i] * gram[j][j]),
 * 0 when either column is all zero.  The table the pruning rule consults is
 * declared integer (section 3.3), read as each row's ranking: rank[i][q] is
 * the q-th most similar expert to i, by T2 descending, ties to the lower
 * index (a plain insertion sort per row).  t2 may be NULL.
 */
int orc_sim_rank(int Ne, const double *gram, double *t2, int32_t *rank)
{
    if (Ne < 1)
        return ORC_BAD;
    double *row = malloc(sizeof(double) * Ne);
    for (int i = 0; i < Ne; i++) {
        double gii = gram[(size_t)i * Ne + i];
        for (int j = 0; j < Ne; j++) {
            double gij = gram[(size_t)i * Ne + j], gjj = gram[(size_t)j * Ne + j];
            double den = gii * gjj;
            row[j] = den > 0.0 ? (gij * gij) / den : 0.0;
            if (t2)
                t2[(size_t)i * Ne + j] = row[j];
        }
        int32_t *r = rank + (size_t)i * Ne;
        for (int j = 0; j < Ne; j++) {
            int q = j;
            while (q > 0 && (row[j] > row[r[q - 1]] || (row[j] == row[r[q - 1]] && j < r[q - 1]))) {
                r[q] = r[q - 1];
                q--;
            }
            r[q] = j;
        }
    }
    free(row);
    return ORC_OK;
}

/*
 * Collaboration pruning, expert-similarity-based (section 3.3): the allowed
 * groups are the first G met walking the token's top-k list in descending
 * score (as in TRAVERSE).  The list is walked again in the same order; an
 * expert in an allowed group stays, any other is replaced by the first
 * expert of its row of the ranked table that sits in an allowed group and is
 * not yet selected.  "Selected" holds the experts of the list that stay plus
 * the replacements made so far, so the k results are distinct.  A
 * replacement takes the replaced expert's place and routing weight (its
 * full-softmax probability).  rank must hold a permutation of 0..Ne-1 in
 * every row.
 */
int orc_route_similarity(int T, int Ne, int k, const float *logits, int Nd, const int32_t *L,
                         int G, const int32_t *rank, int32_t *ids, double *w)
{
    if (T < 0 || k < 1 || k > Ne)
        return ORC_BAD;
    int *grp = malloc(sizeof(int) * Ne), *ord = malloc(sizeof(int) * Ne);
    int *chosen = malloc(sizeof(int) * Nd), *picked = malloc(sizeof(int) * Ne);
    int rc = group_table(Ne, Nd, L, grp, NULL);
    if (G < 1 || G * (Ne / Nd) < k)
        rc = ORC_BAD;
    for (int t = 0; t < T && rc == ORC_OK; t++) {
        const float *l = logits + (size_t)t * Ne;
        score_order(l, Ne, ord);
        double m = l[ord[0]], s = 0.0;
        for (int e = 0; e < Ne; e++)
            s += exp((double)l[e] - m);

        for (int g = 0; g < Nd; g++)
            chosen[g] = 0;
        int have = 0;
        for (int j = 0; j < k && have < G; j++)
            if (!chosen[grp[ord[j]]]) {
                chosen[grp[ord[j]]] = 1;
                have++;
            }
        for (int e = 0; e < Ne; e++)
            picked[e] = 0;
        for (int j = 0; j < k; j++)
            if (chosen[grp[ord[j]]])
                picked[ord[j]] = 1;
        for (int j = 0; j < k; j++) {
            int e = ord[j];
            if (!chosen[grp[e]]) {
                const int32_t *row = rank + (size_t)e * Ne;
                int q = 0;
                while (q < Ne && !(chosen[grp[row[q]]] && !picked[row[q]]))
                    q++;
                if (q == Ne) {
                    rc = ORC_BAD;
                    break;
                }
                picked[row[q]] = 1;
                ids[(size_t)t * k + j] = row[q];
            } else {
                ids[(size_t)t * k + j] = e;
            }
            w[(size_t)t * k + j] = exp((double)l[ord[j]] - m) / s;
        }
    }
    free(grp); free(ord); free(chosen); free(picked);
    return rc;
}

/* Does token t route to an expert kept on group g? */
static int token_uses_group(const int32_t *ids_t, int k, const int *grp, int g)
{
    for (int j = 0; j < k; j++)
        if (grp[ids_t[j]] == g)
            return 1;
    return 0;
}

/*
 * BRIM_0, Algorithm 3 (appendix A.2): one counter, devices outer, tokens
 * inner; entry [g, t] is the SFD row holding token t's replica for group g,
 * or -1.  sfd_off[g] is the counter when row g starts; sfd_off[Nd] = N_sfd.
 */
int orc_brim0(int T, int k, const int32_t *ids, int Ne, int Nd, const int32_t *L,
              int32_t *brim0, int64_t *sfd_off)
{
    int *grp = malloc(sizeof(int) * Ne);
    int rc = group_table(Ne, Nd, L, grp, NULL);
    int64_t ctr = 0;
    for (int g = 0; g < Nd && rc == ORC_OK; g++) {
        sfd_off[g] = ctr;
        for (int t = 0; t < T; t++)
            brim0[(size_t)g * T + t] =
                token_uses_group(ids + (size_t)t * k, k, grp, g) ? (int32_t)ctr++ : -1;
    }
    sfd_off[Nd] = ctr;
    free(grp);
    return rc;
}

/*
 * BRIM_1, Algorithm 5 (appendix A.2), built per group g (each device builds
 * its own): the group's SFD tokens are t' = 0..N_g-1 in SFD order; a counter
 * that restarts for each group runs over local experts outer (placement
 * order) and SFD tokens inner; entry [j, t'] is the local EPD row of
 * (t', L[g][j]), or -1.
 *
 * brim1 holds group g's N_g-wide block at offset n * sfd_off[g].  Also
 * written, as a condensed form of the same matrix: epd_off (Ne+1, in
 * placement order) where the global EPD rows of position g*n+j start (the
 * groups' EPD blocks laid end to end), and for each EPD row its SFD row
 * (epd_src) and routing weight (epd_w).
 */
int orc_brim1(int T, int k, const int32_t *ids, const double *w, int Ne, int Nd,
              const int32_t *L, const int32_t *brim0, const int64_t *sfd_off,
              int32_t *brim1, int64_t *epd_off, int64_t *epd_src, double *epd_w)
{
    int *grp = malloc(sizeof(int) * Ne);
    int rc = group_table(Ne, Nd, L, grp, NULL);
    int n = Ne / Nd;
    int64_t glob = 0;
    for (int g = 0; g < Nd && rc == ORC_OK; g++) {
        int64_t Ng = sfd_off[g + 1] - sfd_off[g];
        int64_t *tok = malloc(sizeof(int64_t) * (Ng > 0 ? Ng : 1));
        for (int t = 0; t < T; t++) {
            int32_t r = brim0[(size_t)g * T + t];
            if (r >= 0)
                tok[r - sfd_off[g]] = t;
        }
        int32_t *B = brim1 + (size_t)n * sfd_off[g];
        int64_t ctr = 0;
        for (int j = 0; j < n; j++) {
            int e = L[g * n + j];
            epd_off[g * n + j] = glob + ctr;
            for (int64_t tp = 0; tp < Ng; tp++) {
                const int32_t *ids_t = ids + (size_t)tok[tp] * k;
                int jj = -1;
                for (int q = 0; q < k; q++)
                    if (ids_t[q] == e)
                        jj = q;
                if (jj < 0) {
                    B[(size_t)j * Ng + tp] = -1;
                    continue;
                }
                B[(size_t)j * Ng + tp] = (int32_t)ctr;
                epd_src[glob + ctr] = sfd_off[g] + tp;
                epd_w[glob + ctr] = w[(size_t)tok[tp] * k + jj];
                ctr++;
            }
        }
        glob += ctr;
        free(tok);
    }
    epd_off[Ne] = glob;
    free(grp);
    return rc;
}

/* SwiGLU hidden state of one expert for one token, in fp64:
 * h[f] = silu(W_gate[f,:] . x) * (W_up[f,:] . x), silu(z) = z / (1 + e^-z).
 * base indexes the expert's (F x d) matrices inside Wg and Wu. */
static void swiglu_hidden(const double *x, const void *Wg, const void *Wu, int dtype,
                          size_t base, int F, int d, double *h)
{
    for (int f = 0; f < F; f++) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < d; c++) {
            g += elem(Wg, dtype, base + (size_t)f * d + c) * x[c];
            u += elem(Wu, dtype, base + (size_t)f * d + c) * x[c];
        }
        h[f] = g / (1.0 + exp(-g)) * u;
    }
}

/* out += scale * (W_down h); base indexes the expert's (d x F) matrix. */
static void down_add(const double *h, const void *Wd, int dtype, size_t base, int F, int d,
                     double scale, double *out)
{
    for (int c = 0; c < d; c++) {
        double s = 0.0;
        for (int f = 0; f < F; f++)
            s += elem(Wd, dtype, base + (size_t)c * F + f) * h[f];
        out[c] += scale * s;
    }
}

/* Shared experts, added with weight 1 (a reading: the paper names them only
 * in section 5, for DeepSeek-MoE). */
static void shared_add(const double *x, int n_sh, int F_sh, int d, int dtype, const void *Wsg,
                       const void *Wsu, const void *Wsd, double *h, double *out)
{
    for (int s = 0; s < n_sh; s++) {
        swiglu_hidden(x, Wsg, Wsu, dtype, (size_t)s * F_sh * d, F_sh, d, h);
        down_add(h, Wsd, dtype, (size_t)s * d * F_sh, F_sh, d, 1.0, out);
    }
}

/*
 * Gate projection g(x) (section 2.1: the router logits come from a single
 * linear layer): logits[t][e] = sum_i x[t][i] * W_r[e][i], fp64, for the
 * listed rows.  W_r is Ne x d (nn.Linear layout), x and W_r fp32 or bf16.
 */
int orc_gate(int nrows, const int64_t *rows, int d, int Ne, int dtype, const void *x,
             const void *Wr, double *logits)
{
    if (nrows < 0 || d < 1 || Ne < 1)
        return ORC_BAD;
    for (int i = 0; i < nrows; i++)
        for (int e = 0; e < Ne; e++) {
            double s = 0.0;
            for (int c = 0; c < d; c++)
                s += elem(x, dtype, (size_t)rows[i] * d + c) * elem(Wr, dtype, (size_t)e * d + c);
            logits[(size_t)i * Ne + e] = s;
        }
    return ORC_OK;
}

/*
 * Layer output, Eq. 1 (section 2.1): MoE(x) = sum_i R(x)_i E_i(x), the sum
 * running over the k routed experts of the token (the other entries of R are
 * zero), plus the shared experts.  One row per requested token, in fp64.
 */
int orc_moe_rows(int nrows, const int64_t *rows, int d, int k, int F, int n_sh, int F_sh,
                 int dtype, const void *x, const int32_t *ids, const double *w, const void *Wg,
                 const void *Wu, const void *Wd, const void *Wsg, const void *Wsu,
                 const void *Wsd, int nthreads, double *y)
{
    int Fmax = F > F_sh ? F : F_sh;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *xt = malloc(sizeof(double) * d), *h = malloc(sizeof(double) * Fmax);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int i = 0; i < nrows; i++) {
            int64_t t = rows[i];
            double *yt = y + (size_t)i * d;
            for (int c = 0; c < d; c++) {
                xt[c] = elem(x, dtype, (size_t)t * d + c);
                yt[c] = 0.0;
            }
            for (int j = 0; j < k; j++) {
                int e = ids[(size_t)t * k + j];
                swiglu_hidden(xt, Wg, Wu, dtype, (size_t)e * F * d, F, d, h);
                down_add(h, Wd, dtype, (size_t)e * d * F, F, d, w[(size_t)t * k + j], yt);
            }
            shared_add(xt, n_sh, F_sh, d, dtype, Wsg, Wsu, Wsd, h, yt);
        }
        free(xt);
        free(h);
    }
    return ORC_OK;
}

/*
 * One token's backward through one expert (see orc_moe_backward below for
 * the formulas): from x_t and dy_t, the expert's activation a (F), the
 * gradients dg, du of its pre-activations (F, already scaled by the
 * routing weight wt) and the routing-weight gradient <dh, a>.
 */
static double expert_backward(const double *xt, const double *dyt, const void *Wg,
                              const void *Wu, const void *Wd, int dtype, size_t wb, size_t db,
                              int F, int d, double wt, double *a_out, double *dg, double *du)
{
    double dwt = 0.0;
    for (int f = 0; f < F; f++) {
        double gf = 0.0, uf = 0.0, dh = 0.0;
        for (int c = 0; c < d; c++) {
            gf += elem(Wg, dtype, wb + (size_t)f * d + c) * xt[c];
            uf += elem(Wu, dtype, wb + (size_t)f * d + c) * xt[c];
            dh += elem(Wd, dtype, db + (size_t)c * F + f) * dyt[c];
        }
        double sg = 1.0 / (1.0 + exp(-gf)), a = gf * sg * uf;
        dwt += dh * a;
        double da = wt * dh;
        dg[f] = da * uf * sg * (1.0 + gf * (1.0 - sg));
        du[f] = da * gf * sg;
        if (a_out)
            a_out[f] = a;
    }
    return dwt;
}

/* dx contribution W_g^T dg + W_u^T du of one expert. */
static void expert_dx(const void *Wg, const void *Wu, int dtype, size_t wb, int F, int d,
                      const double *dg, const double *du, double *out)
{
    for (int c = 0; c < d; c++) {
        double s = 0.0;
        for (int f = 0; f < F; f++)
            s += elem(Wg, dtype, wb + (size_t)f * d + c) * dg[f] +
                 elem(Wu, dtype, wb + (size_t)f * d + c) * du[f];
        out[c] = s;
    }
}

/* Full softmax of one token's logits into p. */
static void softmax_row(const float *l, int Ne, double *p)
{
    double m = l[0], s = 0.0;
    for (int e = 1; e < Ne; e++)
        if (l[e] > m)
            m = l[e];
    for (int e = 0; e < Ne; e++)
        s += exp((double)l[e] - m);
    for (int e = 0; e < Ne; e++)
        p[e] = exp((double)l[e] - m) / s;
}

/*
 * Backward pass of the layer (the gradients the paper's training runs need,
 * sections 1 and 4.3; the pages give no formulas, these are the derivatives
 * of Eq. 1 with the routing ids held fixed).  For token t and its j-th
 * expert e with weight w = R(x)_e and SwiGLU pre-activations g = W_g x,
 * u = W_u x, activation a = silu(g) u and upstream gradient dy:
 *   dh = W_d^T dy                   (gradient of the modulated state w a)
 *   dw = <dh, a>                    (gradient of the routing weight)
 *   da = w dh,  dg = da u silu'(g),  du = da silu(g),
 *   silu'(g) = s (1 + g (1 - s)), s = 1 / (1 + e^-g)
 *   dW_d[e] += dy (w a)^T,  dW_g[e] += dg x^T,  dW_u[e] += du x^T,
 *   dx += W_g^T dg + W_u^T du.
 * Shared experts are the same with w = 1 and no dw.  The logits' gradient
 * goes through Eq. 2's full softmax p (the k weights are p at the chosen
 * experts, not renormalised):
 *   dlogits[i] = p_i ([i chosen] dw_i - sum_j dw_j p_(e_j)).
 * All in fp64; dlogits is skipped when logits is NULL.  The weight
 * gradients are accumulated expert by expert, the input gradient token by
 * token over j in order, then the shared experts.
 */
int orc_moe_backward(int T, int d, int Ne, int k, int F, int n_sh, int F_sh, int dtype,
                     const void *x, const int32_t *ids, const double *w, const float *logits,
                     const void *Wg, const void *Wu, const void *Wd, const void *Wsg,
                     const void *Wsu, const void *Wsd, const double *dy, double *dx,
                     double *dWg, double *dWu, double *dWd, double *dWsg, double *dWsu,
                     double *dWsd, double *dw, double *dlogits)
{
    if (T < 1 || d < 1 || Ne < 1 || k < 1 || F < 1 || n_sh < 0)
        return ORC_BAD;
    for (size_t i = 0; i < (size_t)T * k; i++)
        if (ids[i] < 0 || ids[i] >= Ne)
            return ORC_BAD;
    /* per (t, j) input-gradient contributions, summed per token afterwards */
    double *dxp = calloc((size_t)T * k * d, sizeof(double));
    memset(dWg, 0, sizeof(double) * (size_t)Ne * F * d);
    memset(dWu, 0, sizeof(double) * (size_t)Ne * F * d);
    memset(dWd, 0, sizeof(double) * (size_t)Ne * d * F);
#ifdef _OPENMP
#pragma omp parallel
#endif
    {
        double *xt = malloc(sizeof(double) * d), *g = malloc(sizeof(double) * F);
        double *u = malloc(sizeof(double) * F), *dg = malloc(sizeof(double) * F);
        double *du = malloc(sizeof(double) * F);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int e = 0; e < Ne; e++) {
            size_t wb = (size_t)e * F * d, db = (size_t)e * d * F;
            for (int t = 0; t < T; t++)
                for (int j = 0; j < k; j++) {
                    if (ids[(size_t)t * k + j] != e)
                        continue;
                    double wt = w[(size_t)t * k + j];
                    const double *dyt = dy + (size_t)t * d;
                    for (int c = 0; c < d; c++)
                        xt[c] = elem(x, dtype, (size_t)t * d + c);
                    double dwt = expert_backward(xt, dyt, Wg, Wu, Wd, dtype, wb, db, F, d, wt, g,
                                                 dg, du);
                    for (int f = 0; f < F; f++)
                        for (int c = 0; c < d; c++) {
                            dWd[db + (size_t)c * F + f] += dyt[c] * (wt * g[f]);
                            dWg[wb + (size_t)f * d + c] += dg[f] * xt[c];
                            dWu[wb + (size_t)f * d + c] += du[f] * xt[c];
                        }
                    expert_dx(Wg, Wu, dtype, wb, F, d, dg, du, dxp + ((size_t)t * k + j) * d);
                    dw[(size_t)t * k + j] = dwt;
                }
        }
        free(xt); free(g); free(u); free(dg); free(du);
    }
    for (int t = 0; t < T; t++)
        for (int c = 0; c < d; c++) {
            double s = 0.0;
            for (int j = 0; j < k; j++)
                s += dxp[((size_t)t * k + j) * d + c];
            dx[(size_t)t * d + c] = s;
        }
    free(dxp);

    if (n_sh > 0) {
        memset(dWsg, 0, sizeof(double) * (size_t)n_sh * F_sh * d);
        memset(dWsu, 0, sizeof(double) * (size_t)n_sh * F_sh * d);
        memset(dWsd, 0, sizeof(double) * (size_t)n_sh * d * F_sh);
        double *xt = malloc(sizeof(double) * d), *dg = malloc(sizeof(double) * F_sh);
        double *du = malloc(sizeof(double) * F_sh), *a = malloc(sizeof(double) * F_sh);
        double *dxs = malloc(sizeof(double) * d);
        for (int sx = 0; sx < n_sh; sx++) {
            size_t wb = (size_t)sx * F_sh * d, db = (size_t)sx * d * F_sh;
            for (int t = 0; t < T; t++) {
                const double *dyt = dy + (size_t)t * d;
                for (int c = 0; c < d; c++)
                    xt[c] = elem(x, dtype, (size_t)t * d + c);
                expert_backward(xt, dyt, Wsg, Wsu, Wsd, dtype, wb, db, F_sh, d, 1.0, a, dg, du);
                for (int f = 0; f < F_sh; f++)
                    for (int c = 0; c < d; c++) {
                        dWsd[db + (size_t)c * F_sh + f] += dyt[c] * a[f];
                        dWsg[wb + (size_t)f * d + c] += dg[f] * xt[c];
                        dWsu[wb + (size_t)f * d + c] += du[f] * xt[c];
                    }
                expert_dx(Wsg, Wsu, dtype, wb, F_sh, d, dg, du, dxs);
                for (int c = 0; c < d; c++)
                    dx[(size_t)t * d + c] += dxs[c];
            }
        }
        free(xt); free(dg); free(du); free(a); free(dxs);
    }

    if (logits) {
        double *p = malloc(sizeof(double) * Ne);
        for (int t = 0; t < T; t++) {
            double acc = 0.0;
            softmax_row(logits + (size_t)t * Ne, Ne, p);
            for (int j = 0; j < k; j++)
                acc += dw[(size_t)t * k + j] * p[ids[(size_t)t * k + j]];
            for (int e = 0; e < Ne; e++)
                dlogits[(size_t)t * Ne + e] = -p[e] * acc;
            for (int j = 0; j < k; j++) {
                int e = ids[(size_t)t * k + j];
                dlogits[(size_t)t * Ne + e] += p[e] * dw[(size_t)t * k + j];
            }
        }
        free(p);
    }
    return ORC_OK;
}

/*
 * The per-token parts of orc_moe_backward for the listed token rows only
 * (dy is the full T x d gradient): dx rows (nrows x d), routing-weight
 * gradient rows (nrows x k) and, when logits is non-NULL, dlogits rows
 * (nrows x Ne).  Same arithmetic and order as the full pass.
 */
int orc_moe_backward_rows(int nrows, const int64_t *rows, int d, int Ne, int k, int F, int n_sh,
                          int F_sh, int dtype, const void *x, const int32_t *ids, const double *w,
                          const float *logits, const void *Wg, const void *Wu, const void *Wd,
                          const void *Wsg, const void *Wsu, const void *Wsd, const double *dy,
                          double *dx, double *dw, double *dlogits)
{
    int Fmax = F > F_sh ? F : F_sh;
    int rc = ORC_OK;
#ifdef _OPENMP
#pragma omp parallel
#endif
    {
        double *xt = malloc(sizeof(double) * d), *dg = malloc(sizeof(double) * Fmax);
        double *du = malloc(sizeof(double) * Fmax), *part = malloc(sizeof(double) * d);
        double *p = malloc(sizeof(double) * Ne);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int i = 0; i < nrows; i++) {
            int64_t t = rows[i];
            const double *dyt = dy + (size_t)t * d;
            double *dxt = dx + (size_t)i * d;
            for (int c = 0; c < d; c++) {
                xt[c] = elem(x, dtype, (size_t)t * d + c);
                dxt[c] = 0.0;
            }
            for (int j = 0; j < k; j++) {
                int e = ids[(size_t)t * k + j];
                if (e < 0 || e >= Ne) {
                    rc = ORC_BAD;
                    continue;
                }
                dw[(size_t)i * k + j] =
                    expert_backward(xt, dyt, Wg, Wu, Wd, dtype, (size_t)e * F * d,
                                    (size_t)e * d * F, F, d, w[(size_t)t * k + j], NULL, dg, du);
                expert_dx(Wg, Wu, dtype, (size_t)e * F * d, F, d, dg, du, part);
                for (int c = 0; c < d; c++)
                    dxt[c] += part[c];
            }
            for (int sx = 0; sx < n_sh; sx++) {
                expert_backward(xt, dyt, Wsg, Wsu, Wsd, dtype, (size_t)sx * F_sh * d,
                                (size_t)sx * d * F_sh, F_sh, d, 1.0, NULL, dg, du);
                expert_dx(Wsg, Wsu, dtype, (size_t)sx * F_sh * d, F_sh, d, dg, du, part);
                for (int c = 0; c < d; c++)
                    dxt[c] += part[c];
            }
            if (logits) {
                double acc = 0.0;
                softmax_row(logits + (size_t)t * Ne, Ne, p);
                for (int j = 0; j < k; j++)
                    acc += dw[(size_t)i * k + j] * p[ids[(size_t)t * k + j]];
                for (int e = 0; e < Ne; e++)
                    dlogits[(size_t)i * Ne + e] = -p[e] * acc;
                for (int j = 0; j < k; j++) {
                    int e = ids[(size_t)t * k + j];
                    dlogits[(size_t)i * Ne + e] += p[e] * dw[(size_t)i * k + j];
                }
            }
        }
        free(xt); free(dg); free(du); free(part); free(p);
    }
    return rc;
}

/*
 * Rows of one routed expert's weight gradients, summed over every token
 * routed to it (t ascending, as in orc_moe_backward): rows fs[0..nf) of
 * dW_g[e] and dW_u[e] (d values each) and rows ns[0..nn) of dW_d[e] (F
 * values each).
 */
int orc_moe_wgrad_rows(int T, int d, int k, int F, int dtype, const void *x, const int32_t *ids,
                       const double *w, const void *Wg, const void *Wu, const void *Wd,
                       const double *dy, int e, int nf, const int32_t *fs, int nn,
                       const int32_t *ns, double *dWg, double *dWu, double *dWd)
{
    int cnt = 0;
    for (size_t i = 0; i < (size_t)T * k; i++)
        cnt += ids[i] == e;
    int64_t *tok = malloc(sizeof(int64_t) * (cnt + 1));
    double *wts = malloc(sizeof(double) * (cnt + 1));
    int q = 0;
    for (int t = 0; t < T; t++)
        for (int j = 0; j < k; j++)
            if (ids[(size_t)t * k + j] == e) {
                tok[q] = t;
                wts[q++] = w[(size_t)t * k + j];
            }
    /* per token: dg, du at the sampled f and the modulated activation */
    double *sdg = malloc(sizeof(double) * ((size_t)cnt * nf + 1));
    double *sdu = malloc(sizeof(double) * ((size_t)cnt * nf + 1));
    double *sh = malloc(sizeof(double) * ((size_t)cnt * F + 1));
#ifdef _OPENMP
#pragma omp parallel
#endif
    {
        double *xt = malloc(sizeof(double) * d), *dg = malloc(sizeof(double) * F);
        double *du = malloc(sizeof(double) * F), *a = malloc(sizeof(double) * F);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
        for (int i = 0; i < cnt; i++) {
            for (int c = 0; c < d; c++)
                xt[c] = elem(x, dtype, (size_t)tok[i] * d + c);
            expert_backward(xt, dy + (size_t)tok[i] * d, Wg, Wu, Wd, dtype, (size_t)e * F * d,
                            (size_t)e * d * F, F, d, wts[i], a, dg, du);
            for (int r = 0; r < nf; r++) {
                sdg[(size_t)i * nf + r] = dg[fs[r]];
                sdu[(size_t)i * nf + r] = du[fs[r]];
            }
            for (int f = 0; f < F; f++)
                sh[(size_t)i * F + f] = wts[i] * a[f];
        }
        free(xt); free(dg); free(du); free(a);
    }
    for (int r = 0; r < nf; r++)
        for (int c = 0; c < d; c++) {
            double sg = 0.0, su = 0.0;
            for (int i = 0; i < cnt; i++) {
                double xv = elem(x, dtype, (size_t)tok[i] * d + c);
                sg += sdg[(size_t)i * nf + r] * xv;
                su += sdu[(size_t)i * nf + r] * xv;
            }
            dWg[(size_t)r * d + c] = sg;
            dWu[(size_t)r * d + c] = su;
        }
    for (int r = 0; r < nn; r++)
        for (int f = 0; f < F; f++) {
            double s = 0.0;
            for (int i = 0; i < cnt; i++)
                s += dy[(size_t)tok[i] * d + ns[r]] * sh[(size_t)i * F + f];
            dWd[(size_t)r * F + f] = s;
        }
    free(tok); free(wts); free(sdg); free(sdu); free(sh);
    return ORC_OK;
}

/* Number of threads orc_moe_rows runs with when asked for nthreads. */
int orc_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    int used = 1;
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
    return used;
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * The Occult pipeline of Algorithm 2 (appendix A.1) in fp64, on one host,
 * the Nd groups standing in for the devices and the two all-to-alls being
 * identities:
 *   Dispatch (Alg. 4): x_sfd[BRIM_0[g, t]] = x[t];
 *   SMM scattering (Alg. 6) and weight modulation (Alg. 7): for every
 *     BRIM_1 entry v >= 0 of group g at (j, t'), x_epd[v] = w * h where h is
 *     the SwiGLU hidden state of x_sfd row t' for expert L[g][j] -- the
 *     routing weight scales the hidden state after the activation;
 *   SMM merging (Alg. 8): sfd_out[t'] += W_down x_epd[v], zero-initialised;
 *   Combine (Alg. 9): y[t] = sum over g of sfd_out[BRIM_0[g, t]].
 * Shared experts are added at the end.  Used on small inputs to check that
 * the two-stage split reproduces Eq. 1.
 */
int orc_occult_replay(int T, int d, int Ne, int k, int Nd, int F, int n_sh, int F_sh, int dtype,
                      const void *x, const int32_t *ids, const double *w, const int32_t *L,
                      const void *Wg, const void *Wu, const void *Wd, const void *Wsg,
                      const void *Wsu, const void *Wsd, double *y)
{
    int n = Ne / Nd;
    int32_t *brim0 = malloc(sizeof(int32_t) * (size_t)Nd * T);
    int64_t *sfd_off = malloc(sizeof(int64_t) * (Nd + 1));
    int rc = orc_brim0(T, k, ids, Ne, Nd, L, brim0, sfd_off);
    if (rc != ORC_OK) {
        free(brim0); free(sfd_off);
        return rc;
    }
    int64_t N_sfd = sfd_off[Nd], N_epd = (int64_t)T * k;
    int32_t *brim1 = malloc(sizeof(int32_t) * (size_t)(n * N_sfd + 1));
    int64_t *epd_off = malloc(sizeof(int64_t) * (Ne + 1));
    int64_t *epd_src = malloc(sizeof(int64_t) * (N_epd + 1));
    double *epd_w = malloc(sizeof(double) * (N_epd + 1));
    rc = orc_brim1(T, k, ids, w, Ne, Nd, L, brim0, sfd_off, brim1, epd_off, epd_src, epd_w);

    double *x_sfd = calloc((size_t)(N_sfd + 1) * d, sizeof(double));
    double *sfd_out = calloc((size_t)(N_sfd + 1) * d, sizeof(double));
    double *xt = malloc(sizeof(double) * d);
    int Fmax = F > F_sh ? F : F_sh;
    double *h = malloc(sizeof(double) * Fmax);

    for (int g = 0; g < Nd; g++)
        for (int t = 0; t < T; t++) {
            int32_t r = brim0[(size_t)g * T + t];
            if (r >= 0)
                for (int c = 0; c < d; c++)
                    x_sfd[(size_t)r * d + c] = elem(x, dtype, (size_t)t * d + c);
        }

    for (int g = 0; g < Nd && rc == ORC_OK; g++) {
        int64_t Ng = sfd_off[g + 1] - sfd_off[g];
        int64_t *tok = malloc(sizeof(int64_t) * (Ng > 0 ? Ng : 1));
        for (int t = 0; t < T; t++) {
            int32_t r = brim0[(size_t)g * T + t];
            if (r >= 0)
                tok[r - sfd_off[g]] = t;
        }
        const int32_t *B = brim1 + (size_t)n * sfd_off[g];
        int64_t n_loc = 0;
        for (int j = 0; j < n; j++)
            for (int64_t tp = 0; tp < Ng; tp++)
                n_loc += B[(size_t)j * Ng + tp] >= 0;
        double *x_epd = malloc(sizeof(double) * (size_t)(n_loc + 1) * F);
        for (int j = 0; j < n; j++) {
            int e = L[g * n + j];
            for (int64_t tp = 0; tp < Ng; tp++) {
                int32_t v = B[(size_t)j * Ng + tp];
                if (v < 0)
                    continue;
                const int32_t *ids_t = ids + (size_t)tok[tp] * k;
                double wt = 0.0;
                for (int q = 0; q < k; q++)
                    if (ids_t[q] == e)
                        wt = w[(size_t)tok[tp] * k + q];
                swiglu_hidden(x_sfd + (size_t)(sfd_off[g] + tp) * d, Wg, Wu, dtype,
                              (size_t)e * F * d, F, d, h);
                for (int f = 0; f < F; f++)
                    x_epd[(size_t)v * F + f] = wt * h[f];
            }
        }
        for (int j = 0; j < n; j++) {
            int e = L[g * n + j];
            for (int64_t tp = 0; tp < Ng; tp++) {
                int32_t v = B[(size_t)j * Ng + tp];
                if (v >= 0)
                    down_add(x_epd + (size_t)v * F, Wd, dtype, (size_t)e * d * F, F, d, 1.0,
                             sfd_out + (size_t)(sfd_off[g] + tp) * d);
            }
        }
        free(x_epd);
        free(tok);
    }

    for (int t = 0; t < T && rc == ORC_OK; t++) {
        double *yt = y + (size_t)t * d;
        for (int c = 0; c < d; c++)
            yt[c] = 0.0;
        for (int g = 0; g < Nd; g++) {
            int32_t r = brim0[(size_t)g * T + t];
            if (r >= 0)
                for (int c = 0; c < d; c++)
                    yt[c] += sfd_out[(size_t)r * d + c];
        }
        for (int c = 0; c < d; c++)
            xt[c] = elem(x, dtype, (size_t)t * d + c);
        shared_add(xt, n_sh, F_sh, d, dtype, Wsg, Wsu, Wsd, h, yt);
    }
    free(brim0); free(sfd_off); free(brim1); free(epd_off); free(epd_src); free(epd_w);
    free(x_sfd); free(sfd_out); free(xt); free(h);
    return rc;
}

/*
 * Co-activation statistics.  Eq. 3 (section 2.1): C[i][j] counts the tokens
 * of the batch that activate both i and j, over every ordered pair of the
 * token's k experts (so C[i][i] is expert i's load).  Eq. 4: P = C / max C,
 * the max taken over i != j, P[i][i] = 0, one fp32 division per entry
 * (P = 0 when no pair exists).  Section 2.2: CT is the mean number of
 * replicas per token, i.e. distinct groups among the token's experts; n_sfd
 * is their sum.  intra is the share of off-diagonal co-activations whose two
 * experts sit in one group (the Intra / Inter row of Table 1).
 */
int orc_coact(int T, int k, const int32_t *ids, int Ne, int Nd, const int32_t *L, int64_t *C,
              float *P, int64_t *n_sfd, double *ct, double *intra)
{
    int *grp = malloc(sizeof(int) * Ne);
    int rc = group_table(Ne, Nd, L, grp, NULL);
    memset(C, 0, sizeof(int64_t) * (size_t)Ne * Ne);
    int64_t nsfd = 0;
    for (int t = 0; t < T && rc == ORC_OK; t++) {
        const int32_t *ids_t = ids + (size_t)t * k;
        for (int a = 0; a < k; a++)
            for (int b = 0; b < k; b++)
                C[(size_t)ids_t[a] * Ne + ids_t[b]] += 1;
        for (int g = 0; g < Nd; g++)
            nsfd += token_uses_group(ids_t, k, grp, g);
    }
    int64_t mx = 0, same = 0, all = 0;
    for (int i = 0; i < Ne; i++)
        for (int j = 0; j < Ne; j++)
            if (i != j) {
                int64_t c = C[(size_t)i * Ne + j];
                if (c > mx)
                    mx = c;
                all += c;
                if (grp[i] == grp[j])
                    same += c;
            }
    for (int i = 0; i < Ne; i++)
        for (int j = 0; j < Ne; j++)
            P[(size_t)i * Ne + j] =
                (i == j || mx == 0) ? 0.0f : (float)C[(size_t)i * Ne + j] / (float)mx;
    *n_sfd = nsfd;
    *ct = T > 0 ? (double)nsfd / (double)T : 0.0;
    *intra = all > 0 ? (double)same / (double)all : 0.0;
    free(grp);
    return rc;
}

/*
 * Expert placement rescheduling, Algorithm 1 (section 3.2), a greedy
 * clustering in the manner of farthest point sampling.  Group 0 is seeded
 * with the most collaborative pair (i < j); every later group with the
 * unused expert least collaborative with all placed experts; each group then
 * grows, while it holds fewer than n experts, by the unused expert most
 * collaborative with the group's members.  With n = 1 there is no pair and
 * group 0 starts empty (its first pick, over all-zero scores, is expert 0).
 * L receives Nd lists of n experts in push order.
 */
int orc_placement(int Ne, int Nd, const int64_t *C, int32_t *L)
{
    if (Nd <= 0 || Ne % Nd != 0)
        return ORC_BAD;
    int n = Ne / Nd;
    int *used = calloc(Ne, sizeof(int));
    for (int g = 0; g < Nd; g++) {
        int len = 0;
        int32_t *Lg = L + g * n;
        if (g == 0 && n >= 2) {
            int bi = -1, bj = -1;
            for (int i = 0; i < Ne; i++)
                for (int j = i + 1; j < Ne; j++)
                    if (bi < 0 || C[(size_t)i * Ne + j] > C[(size_t)bi * Ne + bj]) {
                        bi = i;
                        bj = j;
                    }
            Lg[len++] = bi;
            Lg[len++] = bj;
            used[bi] = used[bj] = 1;

        } else if (g > 0) {
            int best = -1;
            int64_t bsum = 0;
            for (int e = 0; e < Ne; e++) {
                if (used[e])
                    continue;
                int64_t s = 0;
                for (int gg = 0; gg < g; gg++)
                    for (int q = 0; q < n; q++)
                        s += C[(size_t)L[gg * n + q] * Ne + e];
                if (best < 0 || s < bsum) {
                    best = e;
                    bsum = s;
                }
            }
            Lg[len++] = best;
            used[best] = 1;

        }
        while (len < n) {
            int best = -1;
            int64_t bsum = 0;
            for (int e = 0; e < Ne; e++) {
                if (used[e])
                    continue;
                int64_t s = 0;
                for (int q = 0; q < len; q++)
                    s += C[(size_t)Lg[q] * Ne + e];
                if (best < 0 || s > bsum) {
                    best = e;
                    bsum = s;
                }
            }
            Lg[len++] = best;
            used[best] = 1;

        }
    }
    free(used);
    return ORC_OK;
}
