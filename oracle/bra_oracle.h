/*
 * bra_oracle.h -- plain CPU oracle for the Bi-Level Routing Attention (BRA)
 * forward pass.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark call it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Sources (web pages; cited below by key and section):
 *   [P1] "从静态到动态：Bi-Level Routing Attention如何重塑视觉Transformer的注意力机制",
 *        www.mhpn.cn/news/199372
 *   [P2] "BiFormer用双层路由注意力重塑视觉Transformer效率极限", www.mooersco.com/news/894234
 *   [P3] "从零构建BiFormer：PyTorch实战双层路由注意力机制与调试全攻略",
 *        www.mhpn.cn/news/564882
 *   [P4] "手把手解析BiFormer：双水平路由注意力机制与PyTorch实战指南", www.jsqmd.com/news/719213
 *   [P5] "【医学图像分割模块】BiFormer / 双层路由注意力（CVPR 2023）", www.mhpn.cn/news/2512273
 *
 * Every floating-point value is an IEEE double; every sum is a plain
 * left-to-right loop (the library is compiled with -ffp-contract=off, so a
 * product is rounded before it is added).
 *
 * Tensor layouts (all row-major, host memory, owned by the caller):
 *   q, k, v, out, o, lepe_out : [B, H, W, C]      C = heads * head_dim,
 *                                                 channel of (head h, dim d) = h*head_dim + d
 *   qbar, kbar                : [B, heads, R, head_dim]   R = n_win^2
 *   aff                       : [B, heads, R, R]
 *   idx                       : [B, heads, R, k_eff]      int32 region ids
 *   lepe_w                    : [C, 5, 5]  (a depthwise Conv2d weight [C,1,5,5])
 *   lepe_b                    : [C]
 * Region r = i*n_win + j covers rows i*hs .. i*hs+hs-1 and columns
 * j*ws .. j*ws+ws-1 (hs = H/n_win, ws = W/n_win); its t = hs*ws tokens are
 * numbered in row-major order inside the window ("slot" u*ws + w).
 *
 * Every function returns 0 on success and -1 on an invalid configuration
 * (non-positive sizes, H or W not divisible by n_win, C not divisible by
 * heads).  Nothing is allocated that outlives a call.
 *
 * parity: every function is pinned by the CPU tests (dense-attention special
 * case, constant inputs, brute-force argsort routing, forced ties, LePE versus
 * a library convolution and its impulse response, an independent PyTorch
 * formulation); see the tests for the list.
 */
#ifndef BRA_ORACLE_H
#define BRA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t batch, height, width, channels, num_heads;
    int32_t n_win; /* regions per side */
    int32_t topk;  /* <= 0 or > n_win^2 means all regions */
    double scale;  /* <= 0 means head_dim^-0.5 */
} oracle_cfg_t;

/* k actually used: min(topk, R), with topk <= 0 meaning R.
 * [P5 §五 step ④ clamps with min(topk, n*n); P2 §3.1 uses -1 for "all"] */
int32_t oracle_topk_effective(const oracle_cfg_t* cfg);

/* Region mean of one projected tensor, per head.  [P4 §1.2 step 1; P2 §2.1] */
int oracle_region_means(const oracle_cfg_t* cfg, const double* x, double* xbar);

/* Region affinity A = Qbar Kbar^T per (batch, head) and the top-k selection,
 * descending affinity, exact ties to the lower region id.  aff may be NULL.
 * [P4 §1.2 steps 2-3; P1 §2.1 TopkRouting; P5 §五 steps ③-④] */
int oracle_route(const oracle_cfg_t* cfg, const double* qbar, const double* kbar,
                 double* aff, int32_t* idx);

/* Head-shared routing: the affinity of a region pair is one sum over all C
 * channels (c = h*head_dim + d in order) of Qbar . Kbar -- the region means
 * over the full channel dimension -- and one top-k per (batch, region)
 * serves every head.  idx: [B, R, k_eff]; aff: [B, R, R] or NULL.
 * [P1 §2.2 index without a head axis; P2 §2.1; P3 §2.1; P4 §1.2] */
int oracle_route_shared(const oracle_cfg_t* cfg, const double* qbar, const double* kbar,
                        double* aff, int32_t* idx);

/* Token-to-token attention of every token over the tokens of its k routed
 * regions (idx as produced by oracle_route, any order).  o excludes LePE.
 * [P3 §2.2 TokenAttention; P5 §五 steps ⑤-⑦] */
int oracle_attend(const oracle_cfg_t* cfg, const double* q, const double* k,
                  const double* v, const int32_t* idx, double* o);

/* LePE: 5x5 depthwise convolution of V, zero padding 2, plus bias.
 * lepe_b may be NULL (zero bias).  [P5 §五 self.lepe and step ⑧; P2 §2.2] */
int oracle_lepe(const oracle_cfg_t* cfg, const double* v, const double* lepe_w,
                const double* lepe_b, double* lepe_out);

/* attend + LePE with a given routing (lepe_w NULL: no LePE term at all). */
int oracle_attend_with_routing(const oracle_cfg_t* cfg, const double* q, const double* k,
                               const double* v, const double* lepe_w, const double* lepe_b,
                               const int32_t* idx, double* out);

/* Whole forward: means -> route -> attend -> + LePE.  aff, qbar, kbar may be
 * NULL; idx and out are required. */
int oracle_bra_forward(const oracle_cfg_t* cfg, const double* q, const double* k,
                       const double* v, const double* lepe_w, const double* lepe_b,
                       double* out, int32_t* idx, double* aff, double* qbar, double* kbar);

/* Whole forward with head-shared routing: means -> oracle_route_shared ->
 * attend (every head over the same routed regions) -> + LePE.
 * idx: [B, R, k_eff]; aff: [B, R, R] or NULL. */
int oracle_bra_forward_shared(const oracle_cfg_t* cfg, const double* q, const double* k,
                              const double* v, const double* lepe_w, const double* lepe_b,
                              double* out, int32_t* idx, double* aff);

/* KV downsampling [P1 §4.1 kv_downsample_ratio, avgpool; §3.1]: K or V
 * averaged over ratio x ratio blocks (row-major block, one plain sum, divided
 * by ratio^2), x [B,H,W,C] -> xd [B,H/ratio,W/ratio,C].  The ratio must
 * divide the window sides.  -1 on a bad configuration or ratio. */
int oracle_kv_downsample(const oracle_cfg_t* cfg, int ratio, const double* x, double* xd);

/* Attention (no LePE) of every query over the downsampled K/V tokens of the
 * regions idx names ([B, heads, R, k_eff], any order). */
int oracle_attend_kvds(const oracle_cfg_t* cfg, int ratio, const double* q, const double* k,
                       const double* v, const int32_t* idx, double* o);

/* Whole forward with KV downsampling: routing on the full-resolution region
 * means (as oracle_bra_forward), attention of every query over the
 * downsampled K/V tokens of its routed regions ((hs/ratio)*(ws/ratio) per
 * region, in window row-major order), + LePE of the full-resolution V.
 * idx: [B, heads, R, k_eff]. */
int oracle_bra_forward_kvds(const oracle_cfg_t* cfg, int ratio, const double* q,
                            const double* k, const double* v, const double* lepe_w,
                            const double* lepe_b, double* out, int32_t* idx);

/* The projections either side of the path [P5 §五 ① qkv Linear(dim, 3*dim),
 * ⑧ proj Linear(dim, dim); P4 §1.1].
 *
 * oracle_round: y[i] = x[i] rounded to the I/O type: round 0 = none (fp64),
 * 1 = bf16 (nearest, ties to even), 2 = fp32.
 *
 * oracle_linear: y[i][o] = (sum_c x[i][c] * w[o][c]) + b[o], then rounded as
 * oracle_round; x [rows, in_f], w [out_f, in_f] (a PyTorch Linear weight),
 * b [out_f] or NULL, y [rows, out_f].
 *
 * oracle_bra_forward_proj: qkv = linear(x, w_qkv [3C, C], b_qkv [3C] or NULL)
 * rounded to the I/O type (`round`), q, k, v = its channel blocks [0, C),
 * [C, 2C), [2C, 3C); y = oracle_bra_forward(q, k, v, lepe) kept in fp64;
 * out = linear(y, w_o [C, C], b_o [C] or NULL) in fp64.  qkv ([B*H*W, 3C],
 * the rounded projections) may be NULL. */
int oracle_round(int round, int64_t n, const double* x, double* y);
int oracle_linear(int64_t rows, int in_f, int out_f, const double* x, const double* w,
                  const double* b, int round, double* y);
int oracle_bra_forward_proj(const oracle_cfg_t* cfg, int round, const double* x,
                            const double* w_qkv, const double* b_qkv, const double* lepe_w,
                            const double* lepe_b, const double* w_o, const double* b_o,
                            double* out, int32_t* idx, double* qkv);

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
