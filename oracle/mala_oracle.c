/*
 * Plain fp64 CPU oracle of MassAlloc Attention (MALA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load this library.  The GPU operator never calls
 * it, and it shares no code, header or constant with the GPU path.
 *
 * Everything is fp64, loops are written in the order the method states them,
 * and nothing is blocked, fused or reordered beyond the tile order the method
 * itself prescribes.  OpenMP only runs independent units side by side (one
 * query block in forward; one query block or one key tile in backward; one
 * KV group in decode); each unit's arithmetic is sequential.
 *
 * Source: "MassAlloc Attention: Let Attention Allocate Its Own Compute",
 * digest page at agihunt.info (paper 2609.32712).  Paragraphs are cited by
 * topic:
 *   [threshold]  the paragraph introducing the per-tile test against tau/Lq
 *   [forward]    the paragraph on the forward test, visit order, first tile
 *   [backward]   the paragraph on the backward test against the final lse
 *   [savings]    the paragraph on what is skipped and the tau -> 0 limit
 *   [limits]     the paragraph with the omitted-mass bound tau/(1+tau)
 *   [motivation] the paragraph listing the dense post-score path
 *
 * Readings of points the pages leave open (each one also listed in the
 * design notes):
 *   - The contribution ratio of key j for row i is exp(s_ij)/Z_i with Z_i the
 *     running normalizer BEFORE the tile is merged ([threshold], [forward]).
 *     In the running (m, l) form: exp(s_ij - m_i) / l_i.  A row with l_i = 0
 *     has ratio +inf, which is how the first tile visited is always kept.
 *   - A row skips iff its largest ratio in the tile is < tau/Lq_i (strict);
 *     equality keeps.  The tile is kept iff any row with a visible key in the
 *     tile keeps; rows with no visible key in the tile abstain.
 *   - A kept tile updates every row of the block with all of that row's
 *     visible keys in the tile; a skipped tile changes nothing.
 *   - Lq_i = i + 1 for prefill (keys and queries aligned at 0); Lk for decode.
 *   - tau = 0 bypasses the test (every legal tile kept: full attention).
 *   - Backward: P = exp(s - lse) with the forward lse, D_i = sum_c dO_ic O_ic
 *     with the forward O; no forced keep; same tiles and vote as forward.
 *     Row 0's only key is key 0, which the forward always keeps, so its P_00
 *     is 1 by definition (taken as such, not from a rounded lse).
 *
 * The test statistic of a tile is T = max over voting rows of
 * (largest ratio of the row) / (tau / Lq_i); the tile is kept iff T >= 1.
 * In replay mode a tile whose |T - 1| <= band takes the decision given by
 * the caller instead (used to follow another implementation through
 * near-threshold tiles, where either decision is correct).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_MEM (-2)

static double dot(const double* a, const double* b, int d) {
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

static long ceil_div(long a, long b) { return (a + b - 1) / b; }

/* ------------------------------------------------------------------------ */
/* Forward, one query block.  [forward], [threshold], [savings]              */
/* ------------------------------------------------------------------------ */
/* Rows are the L query rows of a chunk whose first row sits at key position
 * p0 (p0 = 0 for a whole sequence): row i is position p0 + i, sees keys
 * 0 .. p0 + i, and has Lq_i = p0 + i + 1 visible keys.  Keys come from k, v
 * ([p0 + L][d]); query blocks are counted from the chunk start, key tiles
 * from key 0. */
static double sq_norm(const double* a, int d) { return dot(a, a, d); }

static int fwd_block(const double* q, const double* k, const double* v, long L, long p0, int d,
                     double scale, double tau, int bq, int bk, long qb, long ntiles,
                     const uint8_t* replay, double band,
                     double* o, double* lse, uint8_t* keep, double* T, double* rs)
{
    const long r0 = qb * (long)bq;
    const long r1 = (r0 + bq < L) ? r0 + bq : L;
    const long Lk = p0 + L;
    const int nr = (int)(r1 - r0);
    double* m = malloc(sizeof(double) * nr);
    double* l = malloc(sizeof(double) * nr);
    double* acc = calloc((size_t)nr * d, sizeof(double));
    double* s = malloc(sizeof(double) * (size_t)nr * bk);
    double* r2 = calloc((size_t)nr, sizeof(double)); /* error scale: sum of (exp(s - m) |v_j|)^2 */
    if (!m || !l || !acc || !s || !r2) { free(m); free(l); free(acc); free(s); free(r2); return ORACLE_ERR_MEM; }
    for (int r = 0; r < nr; ++r) { m[r] = -INFINITY; l[r] = 0.0; }

    /* legal tiles of this block: 0 .. jmax, visited jmax down to 0 */
    const long jmax = (p0 + r1 - 1) / bk;
    for (long t = jmax; t >= 0; --t) {
        const long c0 = t * (long)bk;
        const long c1 = (c0 + bk < Lk) ? c0 + bk : Lk;
        /* scores of every visible (i, j) in the tile */
        for (int r = 0; r < nr; ++r) {
            const long i = r0 + r;
            for (long j = c0; j < c1; ++j)
                s[(size_t)r * bk + (j - c0)] = (j <= p0 + i) ? scale * dot(q + i * d, k + j * d, d) : -INFINITY;
        }
        int kp;
        double Tt;
        if (tau == 0.0) {
            kp = 1;
            Tt = NAN;
        } else {
            Tt = 0.0;
            for (int r = 0; r < nr; ++r) {
                const long i = p0 + r0 + r;            /* key position of the row */
                if (c0 > i) continue;                  /* no visible key: abstain */
                const long jl = (i < c1 - 1) ? i : c1 - 1;
                double smax = -INFINITY;
                for (long j = c0; j <= jl; ++j) {
                    const double x = s[(size_t)r * bk + (j - c0)];
                    if (x > smax) smax = x;
                }
                double Tr;
                if (l[r] == 0.0) Tr = INFINITY;          /* empty running state */
                else Tr = (exp(smax - m[r]) / l[r]) / (tau / (double)(i + 1));
                if (Tr > Tt) Tt = Tr;
            }
            kp = (Tt >= 1.0);
            if (replay && fabs(Tt - 1.0) <= band) kp = replay[qb * ntiles + t] ? 1 : 0;
        }
        if (kp) {
            for (int r = 0; r < nr; ++r) {
                const long i = p0 + r0 + r;            /* key position of the row */
                if (c0 > i) continue;
                const long jl = (i < c1 - 1) ? i : c1 - 1;
                double smax = -INFINITY;
                for (long j = c0; j <= jl; ++j) {
                    const double x = s[(size_t)r * bk + (j - c0)];
                    if (x > smax) smax = x;
                }
                const double mn = (smax > m[r]) ? smax : m[r];
                const double a = exp(m[r] - mn);       /* m = -inf gives 0 */
                double* ar = acc + (size_t)r * d;
                l[r] *= a;
                for (int c = 0; c < d; ++c) ar[c] *= a;
                if (rs) r2[r] *= a * a;
                for (long j = c0; j <= jl; ++j) {
                    const double p = exp(s[(size_t)r * bk + (j - c0)] - mn);
                    l[r] += p;
                    const double* vj = v + j * d;
                    for (int c = 0; c < d; ++c) ar[c] += p * vj[c];
                    if (rs) r2[r] += p * p * sq_norm(vj, d);
                }
                m[r] = mn;
            }
        }
        if (keep) keep[qb * ntiles + t] = (uint8_t)kp;
        if (T) T[qb * ntiles + t] = Tt;
    }
    for (int r = 0; r < nr; ++r) {
        const long i = r0 + r;
        for (int c = 0; c < d; ++c) o[i * d + c] = acc[(size_t)r * d + c] / l[r];
        lse[i] = m[r] + log(l[r]);
        if (rs) rs[i] = sqrt(r2[r]) / l[r];
    }
    free(m); free(l); free(acc); free(s); free(r2);
    return ORACLE_OK;
}

/*
 * Forward of one (batch, head): q, k, v are [L][d].  qblocks lists the query
 * blocks to compute (NULL: all).  o [L][d] and lse [L] are written for the
 * rows of computed blocks; keep and T ([nqb][ntiles], ntiles = ceil(L/bk))
 * for their legal tiles.  replay (same layout) may be NULL.
 *
 * rs [L] (may be NULL) receives an error scale of every computed row for the
 * parity tests' per-row bound; it is not part of the method:
 *   rs[i] = sqrt(sum over the row's kept keys j of (p_ij |v_j|)^2),
 * p_ij = exp(s_ij - lse_i), |.| the Euclidean norm.  A kernel that rounds each
 * p_ij to bf16 (relative error at most u = 2^-8, independent across keys)
 * before the PV product moves O_i by about u * rs[i] / sqrt(3).
 */
int oracle_fwd_head(const double* q, const double* k, const double* v, long L, int d,
                    double scale, double tau, int bq, int bk,
                    const long* qblocks, long nqblocks,
                    const uint8_t* replay, double band,
                    double* o, double* lse, uint8_t* keep, double* T, double* rs)
{
    if (!q || !k || !v || !o || !lse || L <= 0 || d <= 0 || bq <= 0 || bk <= 0) return ORACLE_ERR_ARG;
    if (!(tau >= 0.0)) return ORACLE_ERR_ARG;           /* rejects NaN and tau < 0 */
    const long nqb = ceil_div(L, bq), ntiles = ceil_div(L, bk);
    const long n = qblocks ? nqblocks : nqb;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < n; ++u) {
        const long qb = qblocks ? qblocks[u] : u;
        if (qb < 0 || qb >= nqb) { err = ORACLE_ERR_ARG; continue; }
        int e = fwd_block(q, k, v, L, 0, d, scale, tau, bq, bk, qb, ntiles, replay, band, o, lse, keep, T, rs);
        if (e) err = e;
    }
    return err;
}

/*
 * Forward of a query chunk against a key cache, one (batch, head): q is
 * [L][d] (the chunk's rows, at key positions p0 .. p0 + L - 1), k and v are
 * [p0 + L][d] (every key the chunk can see, its own included).  Same test,
 * visit order and update as the whole-sequence forward; Lq_i = p0 + i + 1
 * ([threshold]: the row's count of visible keys).  keep and T are
 * [nqb][ntiles] with nqb = ceil(L/bq), ntiles = ceil((p0 + L)/bk).
 */
int oracle_fwd_chunk_head(const double* q, const double* k, const double* v, long L, long p0, int d,
                          double scale, double tau, int bq, int bk,
                          const long* qblocks, long nqblocks,
                          const uint8_t* replay, double band,
                          double* o, double* lse, uint8_t* keep, double* T, double* rs)
{
    if (!q || !k || !v || !o || !lse || L <= 0 || p0 < 0 || d <= 0 || bq <= 0 || bk <= 0) return ORACLE_ERR_ARG;
    if (!(tau >= 0.0)) return ORACLE_ERR_ARG;
    const long nqb = ceil_div(L, bq), ntiles = ceil_div(p0 + L, bk);
    const long n = qblocks ? nqblocks : nqb;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < n; ++u) {
        const long qb = qblocks ? qblocks[u] : u;
        if (qb < 0 || qb >= nqb) { err = ORACLE_ERR_ARG; continue; }
        int e = fwd_block(q, k, v, L, p0, d, scale, tau, bq, bk, qb, ntiles, replay, band, o, lse, keep, T, rs);
        if (e) err = e;
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Backward.  [backward], [motivation]                                        */
/* ------------------------------------------------------------------------ */

/* Backward probability of key j for row i against the final normalizer:
 * P_ij = exp(s_ij - lse_i).  Row 0 sees only key 0, and the forward always
 * keeps the first tile it visits, so row 0's final normalizer is exp(s_00)
 * and P_00 = 1 exactly; it is taken from that definition, because an lse
 * rounded to fp32 cannot represent it, and at tau = 1 its test 1 >= tau/1 is
 * an exact tie that equality keeps ([forward], [backward], ties keep). */
static double bwd_prob(double s, double lse_i, long i)
{
    return (i == 0) ? 1.0 : exp(s - lse_i);
}

/* Scores of tile (qb, t) into s [bq][bk] (-inf where j > i) and the tile's
 * backward decision against the final lse. */
static int bwd_decide(const double* q, const double* k, long L, int d, double scale, double tau,
                      int bq, int bk, long qb, long t, long ntiles, const double* lse,
                      const uint8_t* replay, double band, double* s, double* Tout)
{
    const long r0 = qb * (long)bq;
    const long r1 = (r0 + bq < L) ? r0 + bq : L;
    const long c0 = t * (long)bk;
    const long c1 = (c0 + bk < L) ? c0 + bk : L;
    for (long i = r0; i < r1; ++i)
        for (long j = c0; j < c1; ++j)
            s[(i - r0) * bk + (j - c0)] = (j <= i) ? scale * dot(q + i * d, k + j * d, d) : -INFINITY;
    if (tau == 0.0) { *Tout = NAN; return 1; }
    double Tt = 0.0;
    for (long i = r0; i < r1; ++i) {
        if (c0 > i) continue;                          /* abstain */
        const long jl = (i < c1 - 1) ? i : c1 - 1;
        for (long j = c0; j <= jl; ++j) {
            const double Tr = bwd_prob(s[(i - r0) * bk + (j - c0)], lse[i], i) / (tau / (double)(i + 1));
            if (Tr > Tt) Tt = Tr;
        }
    }
    *Tout = Tt;
    int kp = (Tt >= 1.0);
    if (replay && fabs(Tt - 1.0) <= band) kp = replay[qb * ntiles + t] ? 1 : 0;
    return kp;
}

/* sum_c |a_c b_c| */
static double abs_dot(const double* a, const double* b, int d) {
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += fabs(a[c] * b[c]);
    return s;
}

/*
 * Backward of one (batch, head).  Inputs [L][d] (lse [L]) as produced by a
 * forward pass.  dq rows of the listed query blocks and dk/dv rows of the
 * listed key tiles are written (NULL list: all).  keep/T [nqb][ntiles] get
 * the decision of every tile visited.
 *
 * es (may be NULL) receives five [L] arrays of error scales for the parity
 * tests' per-row bound (not part of the method), over the kept tiles, with
 * a_ij = sum_c |dO_ic v_jc| and b_i = sum_c |dO_ic O_ic| (the magnitudes
 * behind the dot products dP_ij and D_i):
 *   es[0][i] = scale sqrt(sum_j (dS_ij |k_j|)^2)            (dQ row i)
 *   es[1][i] = scale sqrt(sum_j (P_ij (a_ij + b_i) |k_j|)^2)  (dQ row i)
 *   es[2][j] = scale sqrt(sum_i (dS_ij |q_i|)^2)            (dK row j)
 *   es[3][j] = scale sqrt(sum_i (P_ij (a_ij + b_i) |q_i|)^2)  (dK row j)
 *   es[4][j] = sqrt(sum_i (P_ij |dO_i|)^2)                  (dV row j)
 * The first of each pair sizes the effect of rounding P and dS to bf16
 * (relative u each, independent across terms); the second the effect of fp32
 * rounding in the dot products that form dP - D, which cancel where a row's
 * probability sits on one key.
 */
int oracle_bwd_head(const double* q, const double* k, const double* v, const double* o,
                    const double* lse, const double* dout, long L, int d,
                    double scale, double tau, int bq, int bk,
                    const long* qblocks, long nq, const long* ktiles, long nk,
                    const uint8_t* replay, double band,
                    double* dq, double* dk, double* dv, uint8_t* keep, double* T, double* es)
{
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || L <= 0 || d <= 0 || bq <= 0 || bk <= 0)
        return ORACLE_ERR_ARG;
    if (!(tau >= 0.0)) return ORACLE_ERR_ARG;
    const long nqb = ceil_div(L, bq), ntiles = ceil_div(L, bk);
    double* D = malloc(sizeof(double) * L);
    double* Dabs = malloc(sizeof(double) * L);
    if (!D || !Dabs) { free(D); free(Dabs); return ORACLE_ERR_MEM; }
    for (long i = 0; i < L; ++i) {
        D[i] = dot(dout + i * d, o + i * d, d);
        Dabs[i] = abs_dot(dout + i * d, o + i * d, d);
    }
    double *erq = es ? es : NULL, *ecq = es ? es + L : NULL, *erk = es ? es + 2 * L : NULL;
    double *eck = es ? es + 3 * L : NULL, *erv = es ? es + 4 * L : NULL;
    int err = ORACLE_OK;

    /* dQ: one query block at a time, over its legal tiles */
    const long n1 = qblocks ? nq : nqb;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < n1; ++u) {
        const long qb = qblocks ? qblocks[u] : u;
        if (qb < 0 || qb >= nqb) { err = ORACLE_ERR_ARG; continue; }
        double* s = malloc(sizeof(double) * (size_t)bq * bk);
        if (!s) { err = ORACLE_ERR_MEM; continue; }
        const long r0 = qb * (long)bq;
        const long r1 = (r0 + bq < L) ? r0 + bq : L;
        for (long i = r0; i < r1; ++i) {
            memset(dq + i * d, 0, sizeof(double) * d);
            if (es) { erq[i] = 0.0; ecq[i] = 0.0; }
        }
        const long jmax = (r1 - 1) / bk;
        for (long t = 0; t <= jmax; ++t) {
            double Tt;
            const int kp = bwd_decide(q, k, L, d, scale, tau, bq, bk, qb, t, ntiles, lse, replay, band, s, &Tt);
            if (keep) keep[qb * ntiles + t] = (uint8_t)kp;
            if (T) T[qb * ntiles + t] = Tt;
            if (!kp) continue;
            const long c0 = t * (long)bk;
            const long c1 = (c0 + bk < L) ? c0 + bk : L;
            for (long i = r0; i < r1; ++i) {
                for (long j = c0; j < c1 && j <= i; ++j) {
                    const double P = bwd_prob(s[(i - r0) * bk + (j - c0)], lse[i], i);
                    const double dP = dot(dout + i * d, v + j * d, d);
                    const double dS = P * (dP - D[i]);
                    for (int c = 0; c < d; ++c) dq[i * d + c] += scale * dS * k[j * d + c];
                    if (es) {
                        const double kn2 = sq_norm(k + j * d, d);
                        const double g = P * (abs_dot(dout + i * d, v + j * d, d) + Dabs[i]);
                        erq[i] += dS * dS * kn2;
                        ecq[i] += g * g * kn2;
                    }
                }
            }
        }
        if (es)
            for (long i = r0; i < r1; ++i) { erq[i] = scale * sqrt(erq[i]); ecq[i] = scale * sqrt(ecq[i]); }
        free(s);
    }

    /* dK, dV: one key tile at a time, over the query blocks that see it */
    const long n2 = ktiles ? nk : ntiles;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < n2; ++u) {
        const long t = ktiles ? ktiles[u] : u;
        if (t < 0 || t >= ntiles) { err = ORACLE_ERR_ARG; continue; }
        double* s = malloc(sizeof(double) * (size_t)bq * bk);
        if (!s) { err = ORACLE_ERR_MEM; continue; }
        const long c0 = t * (long)bk;
        const long c1 = (c0 + bk < L) ? c0 + bk : L;
        for (long j = c0; j < c1; ++j) {
            memset(dk + j * d, 0, sizeof(double) * d);
            memset(dv + j * d, 0, sizeof(double) * d);
            if (es) { erk[j] = 0.0; eck[j] = 0.0; erv[j] = 0.0; }
        }
        for (long qb = c0 / bq; qb < nqb; ++qb) {
            double Tt;
            const int kp = bwd_decide(q, k, L, d, scale, tau, bq, bk, qb, t, ntiles, lse, replay, band, s, &Tt);
            if (keep) keep[qb * ntiles + t] = (uint8_t)kp;
            if (T) T[qb * ntiles + t] = Tt;
            if (!kp) continue;
            const long r0 = qb * (long)bq;
            const long r1 = (r0 + bq < L) ? r0 + bq : L;
            for (long i = r0; i < r1; ++i) {
                for (long j = c0; j < c1 && j <= i; ++j) {
                    const double P = bwd_prob(s[(i - r0) * bk + (j - c0)], lse[i], i);
                    const double dP = dot(dout + i * d, v + j * d, d);
                    const double dS = P * (dP - D[i]);
                    for (int c = 0; c < d; ++c) {
                        dk[j * d + c] += scale * dS * q[i * d + c];
                        dv[j * d + c] += P * dout[i * d + c];
                    }
                    if (es) {
                        const double qn2 = sq_norm(q + i * d, d);
                        const double g = P * (abs_dot(dout + i * d, v + j * d, d) + Dabs[i]);
                        erk[j] += dS * dS * qn2;
                        eck[j] += g * g * qn2;
                        erv[j] += P * P * sq_norm(dout + i * d, d);
                    }
                }
            }
        }
        if (es)
            for (long j = c0; j < c1; ++j) {
                erk[j] = scale * sqrt(erk[j]);
                eck[j] = scale * sqrt(eck[j]);
                erv[j] = sqrt(erv[j]);
            }
        free(s);
    }
    free(D);
    free(Dabs);
    return err;
}

/* ------------------------------------------------------------------------ */
/* Decode (split-KV), one (batch, KV group).  [threshold], [forward]          */
/* ------------------------------------------------------------------------ */
/*
 * q: [G][d] rows of the G query heads that share this KV head, all at
 * position Lk-1, so every key 0..Lk-1 is visible and Lq = Lk.  k, v: [Lk][d].
 * Keys are cut into partitions [p*S, min((p+1)*S, Lk)); each partition is cut
 * into bk-key tiles aligned to its start and visited last to first, starting
 * from an empty state (so its first visited tile is kept).  The vote runs
 * over rows_per_vote consecutive rows (1 or G).  Partial states are merged
 * exactly at the end.
 * keep/T: [G/rows_per_vote][nsplit][tps], tps = ceil(S/bk).
 * part_m, part_l: [G][nsplit]; part_acc: [G][nsplit][d] (unnormalized), may be NULL.
 */
int oracle_decode_group(const double* q, int G, const double* k, const double* v, long Lk, int d,
                        double scale, double tau, long split_keys, int bk, int rows_per_vote,
                        const uint8_t* replay, double band,
                        double* o, double* lse, uint8_t* keep, double* T,
                        double* part_m, double* part_l, double* part_acc)
{
    if (!q || !k || !v || !o || G <= 0 || Lk <= 0 || d <= 0 || split_keys <= 0 || bk <= 0) return ORACLE_ERR_ARG;
    if (rows_per_vote <= 0 || G % rows_per_vote) return ORACLE_ERR_ARG;
    if (!(tau >= 0.0)) return ORACLE_ERR_ARG;
    const long nsplit = ceil_div(Lk, split_keys), tps = ceil_div(split_keys, bk);
    const int R = rows_per_vote, nvg = G / R;
    double* pm = malloc(sizeof(double) * G * nsplit);
    double* pl = malloc(sizeof(double) * G * nsplit);
    double* pa = calloc((size_t)G * nsplit * d, sizeof(double));
    double* s = malloc(sizeof(double) * (size_t)R * bk);
    if (!pm || !pl || !pa || !s) { free(pm); free(pl); free(pa); free(s); return ORACLE_ERR_MEM; }

    for (int vg = 0; vg < nvg; ++vg) {
        for (long p = 0; p < nsplit; ++p) {
            const long k0 = p * split_keys;
            const long k1 = (k0 + split_keys < Lk) ? k0 + split_keys : Lk;
            /* per-row state of this partition lives in pm/pl/pa at [row][p] */
            for (int r = 0; r < R; ++r) { pm[(vg * R + r) * nsplit + p] = -INFINITY; pl[(vg * R + r) * nsplit + p] = 0.0; }
            const long nt = ceil_div(k1 - k0, bk);
            for (long t = nt - 1; t >= 0; --t) {
                const long c0 = k0 + t * bk;
                const long c1 = (c0 + bk < k1) ? c0 + bk : k1;
                for (int r = 0; r < R; ++r)
                    for (long j = c0; j < c1; ++j)
                        s[(size_t)r * bk + (j - c0)] = scale * dot(q + (size_t)(vg * R + r) * d, k + j * d, d);
                const long idx = ((long)vg * nsplit + p) * tps + t;
                int kp;
                double Tt;
                if (tau == 0.0) { kp = 1; Tt = NAN; }
                else {
                    Tt = 0.0;
                    for (int r = 0; r < R; ++r) {
                        const double mr = pm[(vg * R + r) * nsplit + p], lr = pl[(vg * R + r) * nsplit + p];
                        double smax = -INFINITY;
                        for (long j = c0; j < c1; ++j) if (s[(size_t)r * bk + (j - c0)] > smax) smax = s[(size_t)r * bk + (j - c0)];
                        const double Tr = (lr == 0.0) ? INFINITY : (exp(smax - mr) / lr) / (tau / (double)Lk);
                        if (Tr > Tt) Tt = Tr;
                    }
                    kp = (Tt >= 1.0);
                    if (replay && fabs(Tt - 1.0) <= band) kp = replay[idx] ? 1 : 0;
                }
                if (keep) keep[idx] = (uint8_t)kp;
                if (T) T[idx] = Tt;
                if (!kp) continue;
                for (int r = 0; r < R; ++r) {
                    const int row = vg * R + r;
                    double* mr = pm + row * nsplit + p;
                    double* lr = pl + row * nsplit + p;
                    double* ar = pa + ((size_t)row * nsplit + p) * d;
                    double smax = -INFINITY;
                    for (long j = c0; j < c1; ++j) if (s[(size_t)r * bk + (j - c0)] > smax) smax = s[(size_t)r * bk + (j - c0)];
                    const double mn = (smax > *mr) ? smax : *mr;
                    const double a = exp(*mr - mn);
                    *lr *= a;
                    for (int c = 0; c < d; ++c) ar[c] *= a;
                    for (long j = c0; j < c1; ++j) {
                        const double pr = exp(s[(size_t)r * bk + (j - c0)] - mn);
                        *lr += pr;
                        for (int c = 0; c < d; ++c) ar[c] += pr * v[j * d + c];
                    }
                    *mr = mn;
                }
            }
        }
    }
    /* exact merge of the partitions' states */
    for (int row = 0; row < G; ++row) {
        double M = -INFINITY;
        for (long p = 0; p < nsplit; ++p) if (pm[row * nsplit + p] > M) M = pm[row * nsplit + p];
        double Lam = 0.0;
        for (int c = 0; c < d; ++c) o[(size_t)row * d + c] = 0.0;
        for (long p = 0; p < nsplit; ++p) {
            const double w = exp(pm[row * nsplit + p] - M);
            Lam += pl[row * nsplit + p] * w;
            for (int c = 0; c < d; ++c) o[(size_t)row * d + c] += pa[((size_t)row * nsplit + p) * d + c] * w;
        }
        for (int c = 0; c < d; ++c) o[(size_t)row * d + c] /= Lam;
        if (lse) lse[row] = M + log(Lam);
    }
    if (part_m) memcpy(part_m, pm, sizeof(double) * G * nsplit);
    if (part_l) memcpy(part_l, pl, sizeof(double) * G * nsplit);
    if (part_acc) memcpy(part_acc, pa, sizeof(double) * (size_t)G * nsplit * d);
    free(pm); free(pl); free(pa); free(s);
    return ORACLE_OK;
}

/* Many (batch, KV group) units in parallel: q [n][G][d], k/v [n][kstride] rows of [Lk][d]. */
int oracle_decode_groups(long n, const double* q, int G, const double* k, const double* v, long kstride,
                         long Lk, int d, double scale, double tau, long split_keys, int bk, int rows_per_vote,
                         const uint8_t* replay, double band,
                         double* o, double* lse, uint8_t* keep, double* T)
{
    if (n <= 0 || rows_per_vote <= 0) return ORACLE_ERR_ARG;
    const long nsplit = ceil_div(Lk, split_keys), tps = ceil_div(split_keys, bk);
    const long kb = (long)(G / rows_per_vote) * nsplit * tps;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < n; ++u) {
        int e = oracle_decode_group(q + u * G * d, G, k + u * kstride, v + u * kstride, Lk, d, scale, tau,
                                    split_keys, bk, rows_per_vote, replay ? replay + u * kb : NULL, band,
                                    o + u * G * d, lse ? lse + u * G : NULL,
                                    keep ? keep + u * kb : NULL, T ? T + u * kb : NULL, NULL, NULL, NULL);
        if (e) err = e;
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Decode with seeded partitions, one (batch, KV group).                      */
/* [threshold], [forward]: the test of a tile uses a normalizer established  */
/* on the more recent keys; here every older partition starts from the       */
/* state of the partition that holds the newest keys.                        */
/* ------------------------------------------------------------------------ */
/*
 * Tiles are the bk-key tiles counted from key 0 (tile j = keys
 * [j*bk, min((j+1)*bk, Lk))); jd = (Lk-1)/bk is the tile holding the newest
 * key.  With tps = split_keys/bk (split_keys must be a multiple of bk),
 * partition p holds tiles lo_p .. hi_p, hi_p = jd - p*tps,
 * lo_p = max(0, hi_p - tps + 1): partition 0 is the newest.  Every partition
 * visits its tiles from hi_p down to lo_p.
 *   - Partition 0 starts from an empty state (its first visited tile is kept)
 *     and is tested against its own running normalizer, as in plain decode.
 *   - Partition p >= 1 is tested against the normalizer of partition 0's
 *     final state plus the keys it has itself kept so far; nothing is kept
 *     by force.  Its output state holds only its own kept keys.
 * The output is the exact merge of the partitions' own states.
 * keep/T: [G/rows_per_vote][nsplit][tps], bit t of partition p = tile lo_p + t.
 * part_m, part_l: [G][nsplit]; part_acc: [G][nsplit][d] (own states), may be NULL.
 */
int oracle_decode_seeded_group(const double* q, int G, const double* k, const double* v, long Lk, int d,
                               double scale, double tau, long split_keys, int bk, int rows_per_vote,
                               const uint8_t* replay, double band,
                               double* o, double* lse, uint8_t* keep, double* T,
                               double* part_m, double* part_l, double* part_acc)
{
    if (!q || !k || !v || !o || G <= 0 || Lk <= 0 || d <= 0 || split_keys <= 0 || bk <= 0) return ORACLE_ERR_ARG;
    if (split_keys % bk || rows_per_vote <= 0 || G % rows_per_vote) return ORACLE_ERR_ARG;
    if (!(tau >= 0.0)) return ORACLE_ERR_ARG;
    const long tps = split_keys / bk, jd = (Lk - 1) / bk, nsplit = ceil_div(jd + 1, tps);
    const int R = rows_per_vote, nvg = G / R;
    double* om = malloc(sizeof(double) * G * nsplit);  /* own state per (row, partition) */
    double* ol = malloc(sizeof(double) * G * nsplit);
    double* oa = calloc((size_t)G * nsplit * d, sizeof(double));
    double* tm = malloc(sizeof(double) * R);             /* test state of the current partition */
    double* tl = malloc(sizeof(double) * R);
    double* s = malloc(sizeof(double) * (size_t)R * bk);
    if (!om || !ol || !oa || !tm || !tl || !s) {
        free(om); free(ol); free(oa); free(tm); free(tl); free(s);
        return ORACLE_ERR_MEM;
    }

    for (int vg = 0; vg < nvg; ++vg) {
        for (long p = 0; p < nsplit; ++p) {
            const long hi = jd - p * tps;
            const long lo = (hi - tps + 1 > 0) ? hi - tps + 1 : 0;
            for (int r = 0; r < R; ++r) {
                const int row = vg * R + r;
                om[row * nsplit + p] = -INFINITY;
                ol[row * nsplit + p] = 0.0;
                /* partition 0: empty test state; later ones: partition 0's final state */
                tm[r] = (p == 0) ? -INFINITY : om[row * nsplit + 0];
                tl[r] = (p == 0) ? 0.0 : ol[row * nsplit + 0];
            }
            for (long j = hi; j >= lo; --j) {
                const long c0 = j * bk;
                const long c1 = (c0 + bk < Lk) ? c0 + bk : Lk;
                for (int r = 0; r < R; ++r)
                    for (long c = c0; c < c1; ++c)
                        s[(size_t)r * bk + (c - c0)] = scale * dot(q + (size_t)(vg * R + r) * d, k + c * d, d);
                const long idx = ((long)vg * nsplit + p) * tps + (j - lo);
                int kp;
                double Tt;
                if (tau == 0.0) { kp = 1; Tt = NAN; }
                else {
                    Tt = 0.0;
                    for (int r = 0; r < R; ++r) {
                        double smax = -INFINITY;
                        for (long c = c0; c < c1; ++c) if (s[(size_t)r * bk + (c - c0)] > smax) smax = s[(size_t)r * bk + (c - c0)];
                        const double Tr = (tl[r] == 0.0) ? INFINITY : (exp(smax - tm[r]) / tl[r]) / (tau / (double)Lk);
                        if (Tr > Tt) Tt = Tr;
                    }
                    kp = (Tt >= 1.0);
                    if (replay && fabs(Tt - 1.0) <= band) kp = replay[idx] ? 1 : 0;
                }
                if (keep) keep[idx] = (uint8_t)kp;
                if (T) T[idx] = Tt;
                if (!kp) continue;
                for (int r = 0; r < R; ++r) {
                    const int row = vg * R + r;
                    double smax = -INFINITY;
                    for (long c = c0; c < c1; ++c) if (s[(size_t)r * bk + (c - c0)] > smax) smax = s[(size_t)r * bk + (c - c0)];
                    /* the test normalizer absorbs the tile */
                    const double mt = (smax > tm[r]) ? smax : tm[r];
                    double lt = tl[r] * exp(tm[r] - mt);
                    for (long c = c0; c < c1; ++c) lt += exp(s[(size_t)r * bk + (c - c0)] - mt);
                    tm[r] = mt;
                    tl[r] = lt;
                    /* and so does the partition's own state */
                    double* mr = om + row * nsplit + p;
                    double* lr = ol + row * nsplit + p;
                    double* ar = oa + ((size_t)row * nsplit + p) * d;
                    const double mn = (smax > *mr) ? smax : *mr;
                    const double a = exp(*mr - mn);
                    *lr *= a;
                    for (int c = 0; c < d; ++c) ar[c] *= a;
                    for (long c = c0; c < c1; ++c) {
                        const double pr = exp(s[(size_t)r * bk + (c - c0)] - mn);
                        *lr += pr;
                        for (int e = 0; e < d; ++e) ar[e] += pr * v[c * d + e];
                    }
                    *mr = mn;
                }
            }
        }
    }
    /* exact merge of the partitions' own states (an empty state weighs 0) */
    for (int row = 0; row < G; ++row) {
        double M = -INFINITY;
        for (long p = 0; p < nsplit; ++p) if (om[row * nsplit + p] > M) M = om[row * nsplit + p];
        double Lam = 0.0;
        for (int c = 0; c < d; ++c) o[(size_t)row * d + c] = 0.0;
        for (long p = 0; p < nsplit; ++p) {
            if (ol[row * nsplit + p] == 0.0) continue;
            const double w = exp(om[row * nsplit + p] - M);
            Lam += ol[row * nsplit + p] * w;
            for (int c = 0; c < d; ++c) o[(size_t)row * d + c] += oa[((size_t)row * nsplit + p) * d + c] * w;
        }
        for (int c = 0; c < d; ++c) o[(size_t)row * d + c] /= Lam;
        if (lse) lse[row] = M + log(Lam);
    }
    if (part_m) memcpy(part_m, om, sizeof(double) * G * nsplit);
    if (part_l) memcpy(part_l, ol, sizeof(double) * G * nsplit);
    if (part_acc) memcpy(part_acc, oa, sizeof(double) * (size_t)G * nsplit * d);
    free(om); free(ol); free(oa); free(tm); free(tl); free(s);
    return ORACLE_OK;
}

/* Many (batch, KV group) units of the seeded decode in parallel (layout as oracle_decode_groups). */
int oracle_decode_seeded_groups(long n, const double* q, int G, const double* k, const double* v, long kstride,
                                long Lk, int d, double scale, double tau, long split_keys, int bk,
                                int rows_per_vote, const uint8_t* replay, double band,
                                double* o, double* lse, uint8_t* keep, double* T)
{
    if (n <= 0 || rows_per_vote <= 0 || bk <= 0 || split_keys <= 0) return ORACLE_ERR_ARG;
    const long tps = split_keys / bk, nsplit = ceil_div((Lk - 1) / bk + 1, tps > 0 ? tps : 1);
    const long kb = (long)(G / rows_per_vote) * nsplit * tps;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < n; ++u) {
        int e = oracle_decode_seeded_group(q + u * G * d, G, k + u * kstride, v + u * kstride, Lk, d, scale, tau,
                                           split_keys, bk, rows_per_vote, replay ? replay + u * kb : NULL, band,
                                           o + u * G * d, lse ? lse + u * G : NULL,
                                           keep ? keep + u * kb : NULL, T ? T + u * kb : NULL, NULL, NULL, NULL);
        if (e) err = e;
    }
    return err;
}
