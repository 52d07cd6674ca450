/*
 * oracle.c -- plain, slow fp64 CPU reference of the skip-masked tiled
 * attention forward (LiteAttention).  TEST INFRASTRUCTURE ONLY: the tests,
 * the smoke check and the benchmark's CPU-baseline leg call it; the product
 * path never does.  It shares no code with the HIP library.
 *
 * What it computes, per (batch b, head h, query tile qt) -- a "row":
 *
 *  1. Output (a plain definition).  Attention restricted to the live tiles:
 *       out[r] = sum_{c live} exp(s[r,c] - M[r]) v[c] / sum_{c live} exp(s[r,c] - M[r])
 *       s[r,c] = scale * q[r].k[c],  M[r] = max_{c live} s[r,c],
 *       lse[r] = M[r] + ln(sum_{c live} exp(s[r,c] - M[r])).
 *     "Live" = key tiles not set in mask_in.  Marked tiles drop out of the
 *     whole iteration: no QK^T, no softmax, no PV ([README] "Full-Stage
 *     Elimination").  This is the flash-style online softmax's result
 *     ([ABSTRACT]: the kernel is built on FlashAttention; the online
 *     normaliser of Milakov & Gimelshein), written here as its definition.
 *
 *  2. QK-Skip decisions (a heuristic, so its steps are followed in order).
 *     Key tiles are visited from the last to the first ([README] Python API,
 *     must-do list: the kernel iterates in reverse order).  A running row max
 *     m_run[r] starts at -inf and takes in each visited tile.  For each
 *     visited tile, with m_loc[r] its local row max:
 *       margin = max over the tile's valid rows r of (m_loc[r] - m_run[r])
 *     (m_run taken before the tile), and the tile is newly marked when
 *       margin < tau      (natural-log units, strict).
 *     Readings adopted where the pages are silent:
 *       - every valid row must pass (max over rows), so a marked tile's
 *         local probabilities are all below e^tau;
 *       - skipped tiles are never visited and do not move m_run;
 *       - a newly marked tile still counts in this step's output and is
 *         skipped from the next step on ([README] "QK-Skip Algorithm": the
 *         mask is refreshed every denoising step, and a tile marked at one
 *         step drops out from the following steps);
 *       - mask_out = mask_in OR newly-marked: marks are never removed;
 *       - keys >= Nk do not exist (excluded from every max and sum);
 *         query rows >= Nq do not vote and are not written;
 *       - tau = -inf never marks.
 *
 *  3. Token ranges ([README] must_do_list / must_skip_list).  Each list holds
 *     pairs (start_i, end_i) with start_i > end_i, start inclusive and end
 *     exclusive, in descending order; read literally, pair i covers the key
 *     tokens t with end_i < t <= start_i.  A key tile
 *       - is "must-do" when any of its keys lies in a must-do range: it is
 *         visited whatever mask_in says, and it is never newly marked;
 *       - is "must-skip" when every one of its keys lies in must-skip ranges
 *         (and it is not must-do): it is never visited.
 *     mask_out is still mask_in OR newly-marked.
 *
 * Inputs are exact upcasts to fp64 of bf16 (raw 16-bit patterns), fp32 or
 * fp64 storage.  q is BSHD [B][Nq][H][D] and k, v are [B][Nk][H][D]: element
 * (b, n, h, e) of q at ((b*Nq + n)*H + h)*D + e, of k and v with Nk.
 * Mask rows: W = ceil(Tk/32) uint32 words per row, row id (b*H + h)*Tq + qt,
 * tile kt at word kt/32, bit kt%32; 1 = skip.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_FP32 = 1, ORACLE_FP64 = 2 };

static double elem(const void *p, int dtype, size_t i)
{
    if (dtype == ORACLE_BF16) {
        /* a bf16 value is the top 16 bits of the fp32 with the same pattern */
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_FP32)
        return (double)((const float *)p)[i];
    return ((const double *)p)[i];
}

/* s[r][c] = scale * sum_e q[row r][e] * k[key c][e], for one tile */
static void tile_logits(const void *q, const void *k, int dtype, int Nq, int Nk, int H, int D,
                        int b, int h, int r0, int nr, int c0, int nc, double scale,
                        double *s /* [nr][nc] */)
{
    for (int r = 0; r < nr; ++r) {
        size_t qo = ((size_t)(b * (size_t)Nq + r0 + r) * H + h) * D;
        for (int c = 0; c < nc; ++c) {
            size_t ko = ((size_t)(b * (size_t)Nk + c0 + c) * H + h) * D;
            double dot = 0.0;
            for (int e = 0; e < D; ++e)
                dot += elem(q, dtype, qo + e) * elem(k, dtype, ko + e);
            s[r * nc + c] = scale * dot;
        }
    }
}

static int is_skipped(const uint32_t *mrow, int kt)
{
    return mrow ? (int)((mrow[kt >> 5] >> (kt & 31)) & 1u) : 0;
}

/* key token t lies in one of the n ranges (start_i, end_i): end_i < t <= start_i */
static int in_ranges(const int32_t *rg, int n, int t)
{
    for (int i = 0; i < n; ++i)
        if (rg[2 * i + 1] < t && t <= rg[2 * i])
            return 1;
    return 0;
}

/* some key of [c0, c0 + nc) is in a must-do range */
static int tile_must_do(const int32_t *rg, int n, int c0, int nc)
{
    for (int t = c0; t < c0 + nc; ++t)
        if (in_ranges(rg, n, t))
            return 1;
    return 0;
}

/* every key of [c0, c0 + nc) is in a must-skip range */
static int tile_must_skip(const int32_t *rg, int n, int c0, int nc)
{
    if (n <= 0)
        return 0;
    for (int t = c0; t < c0 + nc; ++t)
        if (!in_ranges(rg, n, t))
            return 0;
    return 1;
}

/*
 * oracle_fwd: compute the rows listed in `rows` (row ids as above; NULL = all
 * rows in order).  must_do / must_skip: n_do / n_skip (start, end) pairs, or
 * NULL.  Outputs are packed per listed row i:
 *   out      [i][BM][D]   (rows >= Nq left 0)
 *   lse      [i][BM]      (natural log; -inf for a row with no live key)
 *   margin   [i][Tk]      (NaN where the tile was not visited)
 *   mask_out [i][W]       (only when want_mask_out; bits >= Tk are 0)
 * Any output pointer may be NULL.  Returns 0, or -1 on bad arguments.
 */
int oracle_fwd(int B, int Nq, int Nk, int H, int D, int BM, int BN, int dtype,
               const void *q, const void *k, const void *v,
               const uint32_t *mask_in, int want_mask_out, double tau, double scale,
               const int32_t *must_do, int n_do, const int32_t *must_skip, int n_skip,
               const int64_t *rows, int64_t nrows,
               double *out, double *lse, double *margin, uint32_t *mask_out, int nthreads)
{
    if (B <= 0 || Nq <= 0 || Nk < 0 || H <= 0 || D <= 0 || BM <= 0 || BN <= 0 || isnan(tau) || !(scale > 0.0))
        return -1;
    if (n_do < 0 || n_skip < 0 || (n_do > 0 && !must_do) || (n_skip > 0 && !must_skip))
        return -1;
    const int Tq = (Nq + BM - 1) / BM, Tk = (Nk + BN - 1) / BN, W = (Tk + 31) / 32;
    const int64_t total = (int64_t)B * H * Tq;
    if (!rows)
        nrows = total;
    if (nrows < 0)
        return -1;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= total)
            return -1;
    if (nthreads <= 0)
        nthreads = 1;

    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)BM * BN);
        double *m_run = (double *)malloc(sizeof(double) * BM);
        double *m_loc = (double *)malloc(sizeof(double) * BM);
        double *l = (double *)malloc(sizeof(double) * BM);
        double *acc = (double *)malloc(sizeof(double) * (size_t)BM * D);
        uint32_t *newly = (uint32_t *)malloc(sizeof(uint32_t) * W);
        if (!s || !m_run || !m_loc || !l || !acc || !newly) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            if (bad)
                continue;
            const int64_t row = rows ? rows[i] : i;
            const int qt = (int)(row % Tq), h = (int)((row / Tq) % H), b = (int)(row / ((int64_t)Tq * H));
            const int r0 = qt * BM, nr = (Nq - r0 < BM) ? Nq - r0 : BM;
            const uint32_t *mrow = mask_in ? mask_in + row * W : NULL;

            /* ---- pass 1: reverse traversal, running max, QK-Skip decisions ---- */
            for (int r = 0; r < nr; ++r)
                m_run[r] = -INFINITY;
            memset(newly, 0, sizeof(uint32_t) * W);
            for (int kt = Tk - 1; kt >= 0; --kt) {
                if (margin)
                    margin[i * Tk + kt] = NAN;
                const int c0 = kt * BN, nc = (Nk - c0 < BN) ? Nk - c0 : BN;
                const int must_do_t = tile_must_do(must_do, n_do, c0, nc);
                if (!must_do_t && (is_skipped(mrow, kt) || tile_must_skip(must_skip, n_skip, c0, nc)))
                    continue; /* bypassed: no logits, m_run untouched */
                tile_logits(q, k, dtype, Nq, Nk, H, D, b, h, r0, nr, c0, nc, scale, s);
                double mg = -INFINITY;
                for (int r = 0; r < nr; ++r) {
                    double mx = -INFINITY;
                    for (int c = 0; c < nc; ++c)
                        if (s[r * nc + c] > mx)
                            mx = s[r * nc + c];
                    m_loc[r] = mx;
                    double d = mx - m_run[r]; /* +inf while m_run is -inf */
                    if (d > mg)
                        mg = d;
                }
                if (margin)
                    margin[i * Tk + kt] = mg;
                if (mg < tau && !must_do_t)
                    newly[kt >> 5] |= 1u << (kt & 31);
                for (int r = 0; r < nr; ++r)
                    if (m_loc[r] > m_run[r])
                        m_run[r] = m_loc[r];
            }

            /* ---- pass 2: softmax over live keys with the final max, times V ---- */
            for (int r = 0; r < nr; ++r)
                l[r] = 0.0;
            memset(acc, 0, sizeof(double) * (size_t)BM * D);
            for (int kt = Tk - 1; kt >= 0; --kt) {
                const int c0 = kt * BN, nc = (Nk - c0 < BN) ? Nk - c0 : BN;
                if (!tile_must_do(must_do, n_do, c0, nc) &&
                    (is_skipped(mrow, kt) || tile_must_skip(must_skip, n_skip, c0, nc)))
                    continue;
                tile_logits(q, k, dtype, Nq, Nk, H, D, b, h, r0, nr, c0, nc, scale, s);
                for (int r = 0; r < nr; ++r) {
                    for (int c = 0; c < nc; ++c) {
                        double p = exp(s[r * nc + c] - m_run[r]);
                        l[r] += p;
                        size_t vo = ((size_t)(b * (size_t)Nk + c0 + c) * H + h) * D;
                        for (int e = 0; e < D; ++e)
                            acc[r * D + e] += p * elem(v, dtype, vo + e);
                    }
                }
            }
            for (int r = 0; r < BM; ++r) {
                const int valid = r < nr && l[r] > 0.0;
                if (out)
                    for (int e = 0; e < D; ++e)
                        out[(i * BM + r) * D + e] = valid ? acc[r * D + e] / l[r] : 0.0;
                if (lse)
                    lse[i * BM + r] = valid ? m_run[r] + log(l[r]) : -INFINITY;
            }
            if (mask_out)
                for (int w = 0; w < W; ++w) {
                    uint32_t in = mrow ? mrow[w] : 0u;
                    uint32_t nw = want_mask_out ? newly[w] : 0u;
                    uint32_t keep_bits = (w == W - 1 && (Tk & 31)) ? ((1u << (Tk & 31)) - 1u) : 0xffffffffu;
                    mask_out[i * W + w] = (in | nw) & keep_bits;
                }
        }
        free(s);
        free(m_run);
        free(m_loc);
        free(l);
        free(acc);
        free(newly);
    }
    return bad ? -1 : 0;
}

/* Number of hardware threads OpenMP would use by default. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
