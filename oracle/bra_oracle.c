/*
 * bra_oracle.c -- plain, slow, fp64 CPU oracle of the BRA forward pass.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).
 * Page keys [P1]..[P5] are listed in bra_oracle.h.
 *
 * The method is its own definition here (a sparse attention whose result is
 * this algorithm, not an approximation of something simpler), so the code
 * takes the steps in the order the pages give them:
 *   1. split the map into n_win x n_win square windows      [P3 §1; P4 §1.1]
 *   2. mean of Q and of K over each window, per head         [P4 §1.2; P5 §五 ③]
 *   3. region affinity Qbar . Kbar                           [P4 §1.2; P5 §五 ③]
 *   4. keep the k largest per row (torch.topk semantics,
 *      exact ties to the lower region id)                    [P1 §2.1; P5 §五 ④]
 *   5. softmax attention of each token over the tokens of
 *      its k routed windows, scale head_dim^-0.5             [P3 §2.2; P5 §五 ⑤-⑦]
 *   6. + depthwise 5x5 convolution of V (LePE), zero pad 2   [P5 §五 lepe, ⑧; P2 §2.2]
 * Built with -O2 -fopenmp -ffp-contract=off and no fast-math.
 */
#include "bra_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- shape helpers ------------------------------------------------------ */

static int cfg_ok(const oracle_cfg_t* c) {
    if (!c) return 0;
    if (c->batch <= 0 || c->height <= 0 || c->width <= 0 || c->channels <= 0 ||
        c->num_heads <= 0 || c->n_win <= 0)
        return 0;
    if (c->height % c->n_win != 0 || c->width % c->n_win != 0) return 0;
    if (c->channels % c->num_heads != 0) return 0;
    return 1;
}

int32_t oracle_topk_effective(const oracle_cfg_t* c) {
    int32_t R = c->n_win * c->n_win;
    if (c->topk <= 0 || c->topk > R) return R;
    return c->topk;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Index of element (b, y, x, ch) of a [B, H, W, C] map. */
static size_t at(const oracle_cfg_t* c, int b, int y, int x, int ch) {
    return (((size_t)b * c->height + y) * c->width + x) * c->channels + ch;
}

/* Map coordinates of slot `slot` of region `r` (window row-major inside). */
static void region_slot_yx(const oracle_cfg_t* c, int r, int slot, int* y, int* x) {
    int hs = c->height / c->n_win, ws = c->width / c->n_win;
    int ri = r / c->n_win, rj = r % c->n_win;
    *y = ri * hs + slot / ws;
    *x = rj * ws + slot % ws;
}

/* ---- step 2: region means ----------------------------------------------- */

int oracle_region_means(const oracle_cfg_t* c, const double* x, double* xbar) {
    if (!cfg_ok(c) || !x || !xbar) return -1;
    const int hd = c->channels / c->num_heads;
    const int R = c->n_win * c->n_win;
    const int t = (c->height / c->n_win) * (c->width / c->n_win);
    const int nitems = c->batch * c->num_heads * R;
#pragma omp parallel for schedule(static)
    for (int item = 0; item < nitems; ++item) {
        int r = item % R;
        int h = (item / R) % c->num_heads;
        int b = item / (R * c->num_heads);
        for (int d = 0; d < hd; ++d) {
            double s = 0.0;
            for (int slot = 0; slot < t; ++slot) {
                int y, xx;
                region_slot_yx(c, r, slot, &y, &xx);
                s += x[at(c, b, y, xx, h * hd + d)];
            }
            xbar[(size_t)item * hd + d] = s / (double)t;
        }
    }
    return 0;
}

/* ---- steps 3-4: affinity and top-k -------------------------------------- */

/* Top-k of one affinity row: k passes, each keeping the largest entry not yet
 * taken.  Strict '>' while scanning upward leaves an exact tie with the lower
 * id.  `taken` is R bytes of scratch. */
static void topk_row(const double* row, int R, int k, unsigned char* taken, int32_t* out) {
    for (int s = 0; s < R; ++s) taken[s] = 0;
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int s = 0; s < R; ++s) {
            if (taken[s]) continue;
            if (best < 0 || row[s] > row[best]) best = s;
        }
        taken[best] = 1;
        out[j] = best;
    }
}

int oracle_route(const oracle_cfg_t* c, const double* qbar, const double* kbar,
                 double* aff, int32_t* idx) {
    if (!cfg_ok(c) || !qbar || !kbar || !idx) return -1;
    const int hd = c->channels / c->num_heads;
    const int R = c->n_win * c->n_win;
    const int k = oracle_topk_effective(c);
    const int nrows = c->batch * c->num_heads * R;
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * (size_t)R);
        unsigned char* taken = (unsigned char*)malloc((size_t)R);
#pragma omp for schedule(static)
        for (int rowid = 0; rowid < nrows; ++rowid) {
            int bh = rowid / R; /* (b, h) pair */
            const double* qr = qbar + (size_t)rowid * hd;
            for (int s = 0; s < R; ++s) {
                const double* ks = kbar + ((size_t)bh * R + s) * hd;
                double a = 0.0;
                for (int d = 0; d < hd; ++d) a += qr[d] * ks[d];
                row[s] = a;
                if (aff) aff[(size_t)rowid * R + s] = a;
            }
            topk_row(row, R, k, taken, idx + (size_t)rowid * k);
        }
        free(row);
        free(taken);
    }
    return 0;
}

int oracle_route_shared(const oracle_cfg_t* c, const double* qbar, const double* kbar,
                        double* aff, int32_t* idx) {
    if (!cfg_ok(c) || !qbar || !kbar || !idx) return -1;
    const int H = c->num_heads, hd = c->channels / H;
    const int R = c->n_win * c->n_win;
    const int k = oracle_topk_effective(c);
    const int nrows = c->batch * R;
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * (size_t)R);
        unsigned char* taken = (unsigned char*)malloc((size_t)R);
#pragma omp for schedule(static)
        for (int rowid = 0; rowid < nrows; ++rowid) {
            const int b = rowid / R, r = rowid % R;
            for (int s = 0; s < R; ++s) {
                /* one sum over the C channels, c = h * hd + d in order */
                double a = 0.0;
                for (int h = 0; h < H; ++h) {
                    const double* qh = qbar + (((size_t)b * H + h) * R + r) * hd;
                    const double* kh = kbar + (((size_t)b * H + h) * R + s) * hd;
                    for (int d = 0; d < hd; ++d) a += qh[d] * kh[d];
                }
                row[s] = a;
                if (aff) aff[(size_t)rowid * R + s] = a;
            }
            topk_row(row, R, k, taken, idx + (size_t)rowid * k);
        }
        free(row);
        free(taken);
    }
    return 0;
}

/* ---- step 5: token attention over the routed windows -------------------- */

/* Attention of the queries of map `c` over keys and values of map `ckv`:
 * the same map, or its K/V downsampled (same batch, channels, heads and
 * region grid, smaller windows). */
static int attend_impl(const oracle_cfg_t* c, const oracle_cfg_t* ckv, const double* q,
                       const double* kk, const double* v, const int32_t* idx, double* o) {
    if (!cfg_ok(c) || !cfg_ok(ckv) || !q || !kk || !v || !idx || !o) return -1;
    const int hd = c->channels / c->num_heads;
    const int R = c->n_win * c->n_win;
    const int tq = (c->height / c->n_win) * (c->width / c->n_win);
    const int t = (ckv->height / ckv->n_win) * (ckv->width / ckv->n_win);
    const int k = oracle_topk_effective(c);
    const int nkeys = k * t;
    const double scale = c->scale > 0.0 ? c->scale : 1.0 / sqrt((double)hd);
    const int nitems = c->batch * c->num_heads * R;
#pragma omp parallel
    {
        double* logit = (double*)malloc(sizeof(double) * (size_t)nkeys);
        size_t* key_at = (size_t*)malloc(sizeof(size_t) * (size_t)nkeys);
        double* acc = (double*)malloc(sizeof(double) * (size_t)hd);
#pragma omp for schedule(static)
        for (int item = 0; item < nitems; ++item) {
            int r = item % R;
            int h = (item / R) % c->num_heads;
            int b = item / (R * c->num_heads);
            const int32_t* routed = idx + (size_t)item * k;
            /* The gathered key list: routed window j, then its slots in order. */
            for (int j = 0; j < k; ++j)
                for (int slot = 0; slot < t; ++slot) {
                    int y, x;
                    region_slot_yx(ckv, routed[j], slot, &y, &x);
                    key_at[j * t + slot] = at(ckv, b, y, x, h * hd);
                }
            for (int qslot = 0; qslot < tq; ++qslot) {
                int qy, qx;
                region_slot_yx(c, r, qslot, &qy, &qx);
                const double* qv = q + at(c, b, qy, qx, h * hd);
                double mx = -INFINITY;
                for (int m = 0; m < nkeys; ++m) {
                    const double* kv = kk + key_at[m];
                    double dot = 0.0;
                    for (int d = 0; d < hd; ++d) dot += qv[d] * kv[d];
                    logit[m] = scale * dot;
                    if (logit[m] > mx) mx = logit[m];
                }
                double denom = 0.0;
                for (int d = 0; d < hd; ++d) acc[d] = 0.0;
                for (int m = 0; m < nkeys; ++m) {
                    double w = exp(logit[m] - mx);
                    denom += w;
                    const double* vv = v + key_at[m];
                    for (int d = 0; d < hd; ++d) acc[d] += w * vv[d];
                }
                double* ov = o + at(c, b, qy, qx, h * hd);
                for (int d = 0; d < hd; ++d) ov[d] = acc[d] / denom;
            }
        }
        free(logit);
        free(key_at);
        free(acc);
    }
    return 0;
}

int oracle_attend(const oracle_cfg_t* c, const double* q, const double* kk,
                  const double* v, const int32_t* idx, double* o) {
    return attend_impl(c, c, q, kk, v, idx, o);
}

/* The map of K/V after a ratio x ratio average pool (same everything else). */
static oracle_cfg_t kv_cfg(const oracle_cfg_t* c, int ratio) {
    oracle_cfg_t d = *c;
    d.height = c->height / ratio;
    d.width = c->width / ratio;
    return d;
}

static int ratio_ok(const oracle_cfg_t* c, int ratio) {
    return cfg_ok(c) && ratio >= 1 && (c->height / c->n_win) % ratio == 0 &&
           (c->width / c->n_win) % ratio == 0;
}

int oracle_kv_downsample(const oracle_cfg_t* c, int ratio, const double* x, double* xd) {
    if (!ratio_ok(c, ratio) || !x || !xd) return -1;
    const oracle_cfg_t d = kv_cfg(c, ratio);
    const int n = c->batch * d.height * d.width;
#pragma omp parallel for schedule(static)
    for (int cell = 0; cell < n; ++cell) {
        const int b = cell / (d.height * d.width);
        const int yd = (cell / d.width) % d.height, xq = cell % d.width;
        for (int ch = 0; ch < c->channels; ++ch) {
            /* the ratio x ratio block, row-major, one plain sum, then / ratio^2 */
            double s = 0.0;
            for (int u = 0; u < ratio; ++u)
                for (int w = 0; w < ratio; ++w)
                    s += x[at(c, b, yd * ratio + u, xq * ratio + w, ch)];
            xd[at(&d, b, yd, xq, ch)] = s / (double)(ratio * ratio);
        }
    }
    return 0;
}

int oracle_attend_kvds(const oracle_cfg_t* c, int ratio, const double* q, const double* k,
                       const double* v, const int32_t* idx, double* o) {
    if (!ratio_ok(c, ratio) || !q || !k || !v || !idx || !o) return -1;
    const oracle_cfg_t d = kv_cfg(c, ratio);
    const size_t nd = (size_t)c->batch * d.height * d.width * c->channels;
    double* kd = (double*)malloc(sizeof(double) * nd);
    double* vd = (double*)malloc(sizeof(double) * nd);
    int rc = -1;
    if (kd && vd && oracle_kv_downsample(c, ratio, k, kd) == 0 &&
        oracle_kv_downsample(c, ratio, v, vd) == 0)
        rc = attend_impl(c, &d, q, kd, vd, idx, o);
    free(kd);
    free(vd);
    return rc;
}

int oracle_bra_forward_kvds(const oracle_cfg_t* c, int ratio, const double* q,
                            const double* k, const double* v, const double* w,
                            const double* bias, double* out, int32_t* idx) {
    if (!ratio_ok(c, ratio) || !q || !k || !v || !out || !idx) return -1;
    const int hd = c->channels / c->num_heads;
    const size_t nbar = (size_t)c->batch * c->num_heads * c->n_win * c->n_win * hd;
    const oracle_cfg_t d = kv_cfg(c, ratio);
    const size_t nd = (size_t)c->batch * d.height * d.width * c->channels;
    double* qb = (double*)malloc(sizeof(double) * nbar);
    double* kb = (double*)malloc(sizeof(double) * nbar);
    double* kd = (double*)malloc(sizeof(double) * nd);
    double* vd = (double*)malloc(sizeof(double) * nd);
    double* L = w ? (double*)malloc(sizeof(double) * (size_t)c->batch * c->height * c->width *
                                    c->channels)
                  : NULL;
    int rc = -1;
    /* routing on the full-resolution region means; attention over the
     * downsampled keys and values; LePE on the full-resolution V */
    if (qb && kb && kd && vd && (!w || L) && oracle_region_means(c, q, qb) == 0 &&
        oracle_region_means(c, k, kb) == 0 && oracle_route(c, qb, kb, NULL, idx) == 0 &&
        oracle_kv_downsample(c, ratio, k, kd) == 0 &&
        oracle_kv_downsample(c, ratio, v, vd) == 0 &&
        attend_impl(c, &d, q, kd, vd, idx, out) == 0 &&
        (!w || oracle_lepe(c, v, w, bias, L) == 0)) {
        if (w) {
            const size_t n = (size_t)c->batch * c->height * c->width * c->channels;
            for (size_t i = 0; i < n; ++i) out[i] += L[i];
        }
        rc = 0;
    }
    free(qb);
    free(kb);
    free(kd);
    free(vd);
    free(L);
    return rc;
}

/* ---- step 6: LePE -------------------------------------------------------- */

int oracle_lepe(const oracle_cfg_t* c, const double* v, const double* w,
                const double* bias, double* L) {
    if (!cfg_ok(c) || !v || !w || !L) return -1;
    const int H = c->height, W = c->width, C = c->channels;
    const int nrows = c->batch * H;
#pragma omp parallel for schedule(static)
    for (int row = 0; row < nrows; ++row) {
        int b = row / H, y = row % H;
        for (int x = 0; x < W; ++x)
            for (int ch = 0; ch < C; ++ch) {
                double s = bias ? bias[ch] : 0.0;
                for (int i = 0; i < 5; ++i)
                    for (int j = 0; j < 5; ++j) {
                        int yy = y + i - 2, xx = x + j - 2;
                        if (yy < 0 || yy >= H || xx < 0 || xx >= W) continue; /* zero pad */
                        s += w[(size_t)ch * 25 + i * 5 + j] * v[at(c, b, yy, xx, ch)];
                    }
                L[at(c, b, y, x, ch)] = s;
            }
    }
    return 0;
}

/* ---- composition ---------------------------------------------------------- */

int oracle_attend_with_routing(const oracle_cfg_t* c, const double* q, const double* k,
                               const double* v, const double* w, const double* bias,
                               const int32_t* idx, double* out) {
    if (!cfg_ok(c) || !out) return -1;
    if (oracle_attend(c, q, k, v, idx, out) != 0) return -1;
    if (!w) return 0;
    size_t n = (size_t)c->batch * c->height * c->width * c->channels;
    double* L = (double*)malloc(sizeof(double) * n);
    if (!L) return -1;
    int rc = oracle_lepe(c, v, w, bias, L);
    if (rc == 0)
        for (size_t i = 0; i < n; ++i) out[i] = out[i] + L[i];
    free(L);
    return rc;
}

int oracle_bra_forward_shared(const oracle_cfg_t* c, const double* q, const double* k,
                              const double* v, const double* w, const double* bias,
                              double* out, int32_t* idx, double* aff) {
    if (!cfg_ok(c) || !q || !k || !v || !out || !idx) return -1;
    const int H = c->num_heads, hd = c->channels / H;
    const int R = c->n_win * c->n_win;
    const int kk = oracle_topk_effective(c);
    const size_t nbar = (size_t)c->batch * H * R * hd;
    double* qb = (double*)malloc(sizeof(double) * nbar);
    double* kb = (double*)malloc(sizeof(double) * nbar);
    int32_t* full = (int32_t*)malloc(sizeof(int32_t) * (size_t)c->batch * H * R * kk);
    int rc = -1;
    if (qb && kb && full && oracle_region_means(c, q, qb) == 0 &&
        oracle_region_means(c, k, kb) == 0 && oracle_route_shared(c, qb, kb, aff, idx) == 0) {
        /* every head of region r attends over the same routed regions */
        for (int b = 0; b < c->batch; ++b)
            for (int h = 0; h < H; ++h)
                for (int r = 0; r < R; ++r)
                    for (int j = 0; j < kk; ++j)
                        full[(((size_t)b * H + h) * R + r) * kk + j] =
                            idx[((size_t)b * R + r) * kk + j];
        rc = oracle_attend_with_routing(c, q, k, v, w, bias, full, out);
    }
    free(qb);
    free(kb);
    free(full);
    return rc;
}

int oracle_bra_forward(const oracle_cfg_t* c, const double* q, const double* k,
                       const double* v, const double* w, const double* bias, double* out,
                       int32_t* idx, double* aff, double* qbar, double* kbar) {
    if (!cfg_ok(c) || !q || !k || !v || !out || !idx) return -1;
    const int hd = c->channels / c->num_heads;
    const size_t nbar = (size_t)c->batch * c->num_heads * c->n_win * c->n_win * hd;
    double* qb = qbar ? qbar : (double*)malloc(sizeof(double) * nbar);
    double* kb = kbar ? kbar : (double*)malloc(sizeof(double) * nbar);
    int rc = -1;
    if (qb && kb && oracle_region_means(c, q, qb) == 0 && oracle_region_means(c, k, kb) == 0 &&
        oracle_route(c, qb, kb, aff, idx) == 0)
        rc = oracle_attend_with_routing(c, q, k, v, w, bias, idx, out);
    if (!qbar) free(qb);
    if (!kbar) free(kb);
    return rc;
}

/* ---- the projections either side of the path ------------------------------
 * [P5 §五 ① qkv = Linear(dim, 3*dim) of the input, ⑧ proj = Linear(dim, dim) of
 * the attention output; P4 §1.1 the 1x1 projections around the attention] */

/* Nearest bf16 value of x (ties to even), as a double.  bf16 keeps 8
 * significant bits: within the binade [2^(e-1), 2^e) its spacing is
 * 2^(e-8), and below the smallest normal (2^-126) it is 2^-133; rint rounds
 * to nearest even in the default rounding mode.  Beyond the largest finite
 * bf16 ((2 - 2^-7) * 2^127) the result is +-inf. */
static double round_bf16(double x) {
    if (!isfinite(x) || x == 0.0) return x;
    int e;
    frexp(x, &e); /* x = m * 2^e with 0.5 <= |m| < 1 */
    if (e < -125) e = -125;
    const double r = ldexp(rint(ldexp(x, 8 - e)), e - 8);
    return fabs(r) > 3.3895313892515355e38 ? copysign(INFINITY, x) : r;
}

static double round_to(double x, int round) {
    if (round == 1) return round_bf16(x);
    if (round == 2) return (double)(float)x;
    return x;
}

int oracle_round(int round, int64_t n, const double* x, double* y) {
    if (round < 0 || round > 2 || n < 0 || (n > 0 && (!x || !y))) return -1;
    for (int64_t i = 0; i < n; ++i) y[i] = round_to(x[i], round);
    return 0;
}

int oracle_linear(int64_t rows, int in_f, int out_f, const double* x, const double* w,
                  const double* b, int round, double* y) {
    if (rows < 0 || in_f <= 0 || out_f <= 0 || round < 0 || round > 2 || !x || !w || !y)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int o = 0; o < out_f; ++o) {
            double s = 0.0;
            for (int ci = 0; ci < in_f; ++ci) s += x[i * in_f + ci] * w[(size_t)o * in_f + ci];
            if (b) s += b[o];
            y[i * out_f + o] = round_to(s, round);
        }
    return 0;
}

int oracle_bra_forward_proj(const oracle_cfg_t* c, int round, const double* x,
                            const double* w_qkv, const double* b_qkv, const double* lepe_w,
                            const double* lepe_b, const double* w_o, const double* b_o,
                            double* out, int32_t* idx, double* qkv) {
    if (!cfg_ok(c) || round < 0 || round > 2 || !x || !w_qkv || !w_o || !out || !idx) return -1;
    const int C = c->channels;
    const int64_t N = (int64_t)c->batch * c->height * c->width;
    double* P = qkv ? qkv : (double*)malloc(sizeof(double) * (size_t)N * 3 * C);
    double* q = (double*)malloc(sizeof(double) * (size_t)N * C);
    double* k = (double*)malloc(sizeof(double) * (size_t)N * C);
    double* v = (double*)malloc(sizeof(double) * (size_t)N * C);
    double* y = (double*)malloc(sizeof(double) * (size_t)N * C);
    int rc = -1;
    if (P && q && k && v && y && oracle_linear(N, C, 3 * C, x, w_qkv, b_qkv, round, P) == 0) {
        /* q, k, v are the three C-channel blocks of each token's 3C outputs */
        for (int64_t i = 0; i < N; ++i)
            for (int ci = 0; ci < C; ++ci) {
                q[i * C + ci] = P[i * 3 * C + ci];
                k[i * C + ci] = P[i * 3 * C + C + ci];
                v[i * C + ci] = P[i * 3 * C + 2 * C + ci];
            }
        if (oracle_bra_forward(c, q, k, v, lepe_w, lepe_b, y, idx, NULL, NULL, NULL) == 0 &&
            oracle_linear(N, C, C, y, w_o, b_o, 0, out) == 0)
            rc = 0;
    }
    if (!qkv) free(P);
    free(q);
    free(k);
    free(v);
    free(y);
    return rc;
}
