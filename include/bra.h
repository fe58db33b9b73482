/*
 * bra.h -- C ABI of libbra.so: the Bi-Level Routing Attention (BRA) forward
 * pass on AMD Instinct MI355X (gfx950), as hand-written HIP kernels.
 *
 * What is computed (pages cited by key):
 *   [P1] "从静态到动态：Bi-Level Routing Attention如何重塑视觉Transformer的注意力机制",
 *        www.mhpn.cn/news/199372
 *   [P2] "BiFormer用双层路由注意力重塑视觉Transformer效率极限", www.mooersco.com/news/894234
 *   [P3] "从零构建BiFormer：PyTorch实战双层路由注意力机制与调试全攻略",
 *        www.mhpn.cn/news/564882
 *   [P4] "手把手解析BiFormer：双水平路由注意力机制与PyTorch实战指南", www.jsqmd.com/news/719213
 *   [P5] "【医学图像分割模块】BiFormer / 双层路由注意力（CVPR 2023）", www.mhpn.cn/news/2512273
 *
 *   1. The H x W map is cut into n_win x n_win square windows ("regions"),
 *      R = n_win^2 of them, each hs x ws = (H/n_win) x (W/n_win) tokens
 *      [P3 §1 region_partition; P4 §1.1].  Region r = i*n_win + j holds rows
 *      i*hs.. and columns j*ws..; its tokens are numbered row-major.
 *   2. Per head, Q and K are averaged over each region [P4 §1.2; P5 §五 ③].
 *   3. Per head (or, with shared_routing, once over all C channels in the
 *      order c = h*head_dim + d, one routing for every head),
 *      A[r][s] = Qbar_r . Kbar_s (the head_dim^-0.5 factor of
 *      [P5 §五 ③] does not change the order and is not applied) and each row
 *      keeps its k largest entries, in descending order, exact ties to the
 *      lower region id [P1 §2.1 TopkRouting; P5 §五 ④].  k = min(topk, R),
 *      topk <= 0 meaning every region [P5 §五 ④; P2 §3.1].
 *   4. Every token of region r attends, per head, to the k*t tokens of its
 *      routed regions: softmax(scale * q K^T) V [P3 §2.2; P5 §五 ⑤-⑦].
 *      With kv_downsample_ratio r > 1 the keys and values are those of K and
 *      V average-pooled over r x r blocks (k*t/r^2 keys) [P1 §4.1].
 *   5. out = attention + LePE, LePE = depthwise 5x5 convolution of V with
 *      zero padding 2 over the whole map, plus a per-channel bias
 *      [P5 §五 self.lepe and ⑧; P2 §2.2].
 *   Routing is computed in fp64, so routing_idx equals a float64 evaluation
 *   of steps 2-3 with the region sums taken in slot order.  fp32 I/O sums in
 *   that order.  bf16 I/O sums in other orders (trees over lanes), which
 *   give the same sums because a sum of bf16 values is exact in fp64 while
 *   the nonzero values of one (region, channel) span at most
 *   2^(45 - ceil(log2 t)) in magnitude (2^39 for 64-token regions); inputs
 *   beyond that span may route differently where two affinities differ by
 *   less than the rounding of those sums.  (Where a faster fp32 pass is
 *   taken first, an error bound decides whether its order is the fp64 one;
 *   otherwise the fp64 values decide.)  Attention runs on bf16 MFMA with
 *   fp32 accumulation and an fp32 online softmax (bf16 I/O) or in fp32 VALU
 *   arithmetic (fp32 I/O).  LePE accumulates in fp32; for bf16 windows that
 *   tile by 4 x 4 (the benchmark shapes) it runs on MFMA, which first rounds
 *   lepe_w once to bf16 (the bias stays fp32).
 *
 * Layouts (device memory, C-contiguous, owned by the caller):
 *   q, k, v, out   [B, H, W, C] (NHWC), C = heads * head_dim, the channel of
 *                  (head h, dim d) is h*head_dim + d; element type = dtype
 *   lepe_w         [C, 5, 5] fp32 (a PyTorch depthwise weight [C, 1, 5, 5])
 *   lepe_b         [C] fp32
 *   routing_idx    [B, heads, R, k] int32 ([B, 1, R, k] with shared_routing)
 *
 * Errors: every call returns a bra_status_t; nothing throws or aborts across
 * the ABI.  bra_last_error() gives a thread-local message for the last
 * failing call.  A kernel fault is asynchronous and surfaces at the caller's
 * next synchronisation.
 *
 * Threads and streams: a handle may be used from any host thread but by one
 * stream at a time (its workspace is shared by the calls made with it).
 */
#ifndef BRA_H
#define BRA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bra_handle_s* bra_handle_t; /* opaque */

typedef enum {
    BRA_OK = 0,
    BRA_ERR_NULL = 1,        /* a required pointer is NULL */
    BRA_ERR_SHAPE = 2,       /* sizes not positive, H or W not divisible by n_win,
                                C not divisible by num_heads, too large for int32 indexing,
                                shared_routing or projections not 0/1, or
                                kv_downsample_ratio not dividing the window sides */
    BRA_ERR_UNSUPPORTED = 3, /* head_dim != 32, unknown dtype, n_win > 16, H*W >= 2^23,
                                a region whose on-chip tiles (with its LePE halo) need
                                more than a CU's 160 KB of LDS, or projections with
                                fp32 (or on a handle without them) */
    BRA_ERR_HIP = 4,         /* a HIP runtime call failed (see bra_last_error) */
    BRA_ERR_NOMEM = 5,       /* device memory for the workspace could not be allocated */
    BRA_ERR_BAD_HANDLE = 6,  /* not a live handle (never created, or destroyed) */
    BRA_ERR_ALIGN = 7,       /* q, k, v or out not 16-byte aligned, or lepe_w, lepe_b,
                                routing_idx not 4-byte aligned */
    BRA_ERR_ALIAS = 8,       /* out overlaps q, k or v */
    BRA_ERR_DEVICE = 9       /* the current HIP device is not the handle's device */
} bra_status_t;

typedef enum { BRA_F32 = 0, BRA_BF16 = 1 } bra_dtype_t;

typedef struct {
    int32_t batch, height, width, channels, num_heads;
    int32_t n_win;     /* regions per side: H % n_win == 0 and W % n_win == 0 */
    int32_t topk;      /* routed regions per region; <= 0 or > n_win^2 means all */
    int32_t dtype;     /* element type of q, k, v and out: a bra_dtype_t (BRA_F32 or
                          BRA_BF16; other values are rejected) */
    float scale;       /* attention logit scale; <= 0 means head_dim^-0.5 */
    int32_t shared_routing; /* 0: routing per head (the default, [P5 §五 ③-④]);
                               1: one routing per region shared by every head,
                               from the region means over all C channels
                               [P1 §2.2; P2 §2.1; P3 §2.1; P4 §1.2] */
    int32_t kv_downsample_ratio; /* <= 1: none.  r > 1: the attention gathers K and V
                               average-pooled over r x r blocks (windows of
                               (H/n_win/r) x (W/n_win/r) tokens), routing and LePE
                               stay at full resolution [P1 §4.1]; r must divide
                               H/n_win and W/n_win */
    int32_t projections;    /* 1: the handle also runs bra_forward_proj (the
                               module's qkv and output projections around the
                               path, [P5 §五 ① and ⑧]); its workspace then holds
                               the projected q, k, v.  bf16, C <= 512, per-head
                               routing and no KV downsampling only
                               (BRA_ERR_UNSUPPORTED otherwise).  0: none */
} bra_config_t;

/* Validate cfg and allocate the handle and its device workspace on the
 * current HIP device: the region means of Q and K (2*B*C*R*8 bytes in fp64,
 * B*C*R*4 more for an fp32 copy of the K means), a
 * routing buffer (B*heads*R*k*4 bytes), for window shapes whose LePE runs on
 * MFMA a C*320-byte operand table, with KV downsampling the pooled K and V
 * (2*B*H*W*C*sizeof(dtype)/r^2 bytes), and with projections the projected
 * q, k, v (3*B*H*W*C*2 bytes).  On success *out is a live handle; on failure
 * *out is left NULL. */
bra_status_t bra_create(const bra_config_t* cfg, bra_handle_t* out);

/* Enqueue the forward pass on `stream` (a hipStream_t; NULL = the null
 * stream) and return without synchronising.  The kernels are the region
 * means, then (with KV downsampling) the pooled K/V, then the routing, then
 * attention + LePE: two to four launches.  The attention kernel routes by
 * itself for at most 64 regions and at most 4 heads (per-head routing); the
 * region-mean kernel routes too for at most 64 regions, more heads, regions
 * of at most 16 tokens and R * t <= 256 (bf16, per head).  No allocation
 * happens here; the calls may be captured in a HIP graph.
 *   q, k, v       device, [B,H,W,C], dtype, 16-byte aligned
 *   lepe_w        device [C,5,5] fp32, or NULL for no LePE term (lepe_b is then ignored)
 *   lepe_b        device [C] fp32, or NULL for a zero bias
 *   out           device, [B,H,W,C], dtype, 16-byte aligned, must not overlap q/k/v
 *   routing_idx   device [B,heads,R,k] int32 to receive the routing, or NULL
 * The current device must be the handle's device. */
bra_status_t bra_forward(bra_handle_t h, const void* q, const void* k, const void* v,
                         const float* lepe_w, const float* lepe_b, void* out,
                         int32_t* routing_idx, void* stream);

/* Attention and LePE with a routing the caller supplies: steps 4-5 above on
 * the regions routing_idx names, without computing the region means or the
 * routing (for reusing one routing across several calls, the reuse the pages
 * suggest for consecutive slices [P2 §4.2]).
 *   routing_idx   device [B,rheads,R,k] int32, required (rheads = 1 on a
 *                 handle with shared_routing, else heads); row (b,h,r) lists
 *                 the k regions whose tokens the queries of region r attend
 *                 to, for head h (every head, with shared_routing) -- any
 *                 order; a region listed twice counts twice.  Ids are
 *                 clamped into [0, R) before use.
 *   the other arguments and the checks are those of bra_forward.
 * Enqueued on `stream` without synchronising or allocating. */
bra_status_t bra_forward_routed(bra_handle_t h, const void* q, const void* k, const void* v,
                                const float* lepe_w, const float* lepe_b,
                                const int32_t* routing_idx, void* out, void* stream);

/* The path with the module's projections on either side [P5 §五 ① qkv =
 * Linear(dim, 3*dim), ⑧ proj = Linear(dim, dim); P4 §1.1], for handles created
 * with projections = 1:
 *   q|k|v = x w_qkv^T + b_qkv, each rounded once to bf16 (channel blocks
 *           [0,C), [C,2C), [2C,3C) of the 3C outputs)
 *   y     = the bra_forward result of (q, k, v, lepe_w, lepe_b), rounded
 *           once to bf16 (as bra_forward's out is)
 *   out   = y w_o^T + b_o, accumulated in fp32, rounded once to bf16
 *   x             device [B,H,W,C] bf16, 16-byte aligned
 *   w_qkv         device [3C, C] bf16 (a PyTorch Linear weight), 16-byte aligned
 *   b_qkv         device [3C] fp32, or NULL for none
 *   w_o           device [C, C] bf16 (Linear weight), 16-byte aligned
 *   b_o           device [C] fp32, or NULL for none
 *   lepe_w, lepe_b, routing_idx, stream: as bra_forward; out: [B,H,W,C] bf16,
 *   must not overlap x.
 * The qkv projection runs on MFMA with the region means of the projected q
 * and k computed in the same pass, writing q, k, v to the handle's
 * workspace.  For C <= 4t the output projection runs in the attention
 * kernel's epilogue on the y tile in LDS, so y never goes to memory; for
 * larger C, y goes to the workspace and a kernel of its own applies the
 * projection.  Enqueued without synchronising or allocating.
 * BRA_ERR_UNSUPPORTED for a handle created without projections. */
bra_status_t bra_forward_proj(bra_handle_t h, const void* x, const void* w_qkv,
                              const float* b_qkv, const float* lepe_w, const float* lepe_b,
                              const void* w_o, const float* b_o, void* out,
                              int32_t* routing_idx, void* stream);

/* bra_forward without a handle and without allocating, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc.  Same computation, kernels, arguments and
 * checks as bra_forward on a handle created with *cfg; the workspace (the
 * sizes bra_create lists) comes from a device array of 16 MiB that the
 * library holds on each device it runs on until the process ends.  A
 * configuration whose workspace exceeds 16 MiB gives BRA_ERR_UNSUPPORTED,
 * as do projections (bra_forward_proj only).  Every call on a device uses
 * that device's one array and leaves it in use until its kernels finish:
 * calls that overlap on one device (another stream, another thread) race,
 * so serialise them.  Calls no hipMalloc, hipFree or memset; enqueued on
 * `stream` (the current device's) without synchronising. */
bra_status_t bra_forward_noalloc(const bra_config_t* cfg, const void* q, const void* k,
                                const void* v, const float* lepe_w, const float* lepe_b,
                                void* out, int32_t* routing_idx, void* stream);

/* Release the workspace and the handle.  NULL is a no-op (BRA_OK); a handle
 * that is not live gives BRA_ERR_BAD_HANDLE. */
bra_status_t bra_destroy(bra_handle_t h);

/* k actually used by the handle (min(topk, R), or R); -1 for a bad handle. */
int32_t bra_topk_effective(bra_handle_t h);

/* Static description of a status code ("unknown status" for any other
 * value; taken as an int32_t so that any value can be passed). */
const char* bra_status_string(int32_t s);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* bra_last_error(void);

/* Per-kernel timing for profiling.  bra_timing_enable(h, n) makes the next n
 * calls of bra_forward record HIP events around each of its steps on the
 * call's stream (n = 0 turns recording off).  bra_timing_read waits for the
 * recorded events and writes, for each recorded call i < *count,
 * ms[3*i] = region means (and KV downsampling), ms[3*i+1] = routing kernel and
 * ms[3*i+2] = attention/LePE kernel time (milliseconds), then clears the
 * record.  When the attention or the region-mean kernel routes, ms[3*i+1]
 * measures only the gap between two back-to-back events.  With projections
 * the first slot is the qkv projection and the last includes the output
 * projection.  `ms` holds at least 3*n floats. */
bra_status_t bra_timing_enable(bra_handle_t h, int32_t n);
bra_status_t bra_timing_read(bra_handle_t h, float* ms, int32_t* count);

/* Testing hooks (failure handling without exhausting a device).
 * bra_debug_inject_alloc_failure(which, n): the next n allocations of kind
 * `which` made by bra_create fail as if memory were exhausted -- the handle
 * itself (BRA_ALLOC_HOST) or its device workspace (BRA_ALLOC_DEVICE) --, so
 * bra_create returns BRA_ERR_NOMEM, leaves *out NULL and frees whatever it
 * had allocated; n = 0 disarms.  Both failures are injected before any HIP
 * call, so they are testable without a GPU.  BRA_ERR_SHAPE for n < 0 or an
 * unknown kind.  bra_debug_live_handles() is the number of handles created
 * and not yet destroyed, in this process. */
enum { BRA_ALLOC_HOST = 1, BRA_ALLOC_DEVICE = 2 };
bra_status_t bra_debug_inject_alloc_failure(int32_t which, int32_t count);
int32_t bra_debug_live_handles(void);

/* Testing hook: the q, k, v of the last bra_forward_proj on h (the bf16
 * outputs of its qkv projection, kept in the handle's workspace until the
 * next call on h), copied into q, k, v (device [B,H,W,C] bf16 each, owned by
 * the caller) on `stream`, enqueued after that call when on its stream.
 * BRA_ERR_BAD_HANDLE, BRA_ERR_UNSUPPORTED for a handle without projections,
 * BRA_ERR_NULL for a missing pointer, BRA_ERR_HIP if a copy fails. */
bra_status_t bra_debug_projected_qkv(bra_handle_t h, void* q, void* k, void* v, void* stream);

#ifdef __cplusplus
}
#endif
#endif
