// bra_route.hip -- region-level routing [P4 §1.2; P1 §2.1 TopkRouting;
// P5 §五 ③-④] (page keys in bra_device.h).
//
// For each (image, head) -- each image with head-shared routing [P1 §2.2;
// P2 §2.1; P3 §2.1] -- and each query region r: the fp64 affinity
// A[r][s] = Qbar_r . Kbar_s against every region s (over one head's 32 dims,
// or all C channels when shared), then the k largest entries of the row, in
// descending order with exact ties to the lower region id.  The
// head_dim^-0.5 factor the pages apply to the affinity does not change the
// order and is left out.
//
// Every entry is the sequential fp64 sum of dot32_seq_from (with shared
// routing the heads follow one another in one running sum, c = h * 32 + d).
// A lane holds the K mean of one region s in registers, the query rows are
// wave-uniform (scalar loads), and kRouteChains rows run as independent
// chains.
//   R <= 64: a wave owns kRouteChains rows from the affinity to the routed
//            ids, in registers: the arg-max (k = 1), or a bitonic sort of
//            each row over the wave's lanes (k > 1).  No LDS, no barrier.
//   R > 64:  the lanes of a row span SPAN/64 waves; the rows go through LDS
//            to one wave each, which keeps the k best by a bitonic sort whose
//            cross-lane partners come from DPP and permlane swaps.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_shapes.h"

namespace bra {
namespace {

constexpr int kRouteChains = 4;  // query rows whose dots run interleaved

// Region-span of the large-map kernel: threads tid % SPAN own region tid % SPAN,
// SPAN = the power of two >= R (128 or 256 = kMaxRegions).
__host__ __device__ constexpr int route_span(int R) { return R <= 64 ? 64 : R <= 128 ? 128 : 256; }
// Query rows a workgroup routes: kRouteChains per wave for R <= 64, 2 per
// wave for R <= 128, 1 per wave above (more workgroups: the selection over
// 256 entries is long, and 4 rows per workgroup measured 2.3 us faster than 8
// on 8 x 2 x 256 rows, despite the K means being read twice as often).
__host__ __device__ constexpr int route_rows(int span) {
    return span == 64 ? kWaves * kRouteChains : span == 256 ? kWaves : kWaves * 2;
}
// fp64 row stride of the affinity tile (even, so pairs of entries are 16-byte aligned).
__host__ __device__ constexpr int route_row_stride(int R) { return (R + 1) & ~1; }

// acc[j] += q[j] . k over the 32 dims of one head, left to right, each
// product rounded before it is added (dot32_seq_from, N rows at once).
template <int N>
__device__ __forceinline__ void dots_seq(double (&acc)[N], const double* const (&q)[N],
                                         const double (&k)[kHeadDim]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d)
#pragma unroll
        for (int j = 0; j < N; ++j) acc[j] = acc[j] + q[j][d] * k[d];
}

// Writes the first k ids of row r to dst[r] (rows with live[r]).
template <int E, int NRW>
__device__ __forceinline__ void wave_topk_bitonic(const double* const (&rows)[NRW], int R, int k,
                                                  int32_t* const (&dst)[NRW],
                                                  const bool (&live)[NRW]) {
    const int lane = threadIdx.x & 63;
    double v[NRW][E];
    int ix[NRW][E];
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = lane * E + e;
            v[r][e] = i < R ? rows[r][i] : -INFINITY;
            ix[r][e] = i;
        }
    }
    route_topk<E, NRW>(v, ix, lane, k);
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = lane * E + e;
            if (live[r] && i < k) dst[r][i] = ix[r][e];
        }
    }
}

// ---------------------------------------------------------------------------
// R <= 64.  Wave w of workgroup (routing group rg, chunk) routes rows
// r0 .. r0 + kRouteChains - 1, r0 = (chunk * kWaves + w) * kRouteChains.
template <int NW, int KTOP>
__global__ __launch_bounds__(kThreads) void route_small_kernel(const double* __restrict__ means,
                                                               int32_t* __restrict__ idx_out,
                                                               Params p_in) {
    Params p = p_in;
    if constexpr (NW > 0) {
        p.n = NW;
        p.R = NW * NW;
    }
    if constexpr (KTOP > 0) p.k = KTOP;
    constexpr int ROWS = route_rows(64);
    const int R = p.R, lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunk = (R + ROWS - 1) / ROWS;
    // rg: the routing's (image, head) pair, or the image with shared routing
    const int rg = blockIdx.x / nchunk, chunk = blockIdx.x - rg * nchunk;
    const int r0 = chunk * ROWS + w * kRouteChains;
    if (r0 >= R) return;  // wave-uniform; nothing below synchronises waves
    const int h0 = p.shared ? rg * p.heads : rg;  // first (image, head) summed
    const int nh = p.shared ? p.heads : 1;        // heads summed into one affinity

    double acc[kRouteChains];
#pragma unroll
    for (int j = 0; j < kRouteChains; ++j) acc[j] = 0.0;
    for (int hh = 0; hh < nh; ++hh) {
        const int bh = h0 + hh;
        double kreg[kHeadDim];
        load_kmean(p, means, bh, min(lane, R - 1), kreg);
        // rows past the map repeat the last one (never written)
        const double* q[kRouteChains];
#pragma unroll
        for (int j = 0; j < kRouteChains; ++j) q[j] = means + qmean_index(p, bh, min(r0 + j, R - 1), 0);
        dots_seq<kRouteChains>(acc, q, kreg);
    }

    int32_t* const base = idx_out + (static_cast<size_t>(rg) * R + r0) * p.k;
    const int nrows = min(kRouteChains, R - r0);
    if (p.k == 1) {
        // (a NaN row leaves the arg-max undefined; the id is clamped into range)
#pragma unroll
        for (int j = 0; j < kRouteChains; ++j) {
            double best = lane < R ? acc[j] : -INFINITY;
            int bs = lane < R ? lane : 0x7fffffff;
            wave_argmax(best, bs);
            if (lane == 0 && j < nrows) base[j] = min(max(bs, 0), R - 1);
        }
    } else {
        // one bitonic sort per row, lane s holding entry s
        double v[kRouteChains][1];
        int ix[kRouteChains][1];
#pragma unroll
        for (int j = 0; j < kRouteChains; ++j) {
            v[j][0] = lane < R ? acc[j] : -INFINITY;
            ix[j][0] = lane;
        }
        route_topk<1, kRouteChains>(v, ix, lane, p.k);
#pragma unroll
        for (int j = 0; j < kRouteChains; ++j)
            if (j < nrows && lane < p.k) base[j * p.k + lane] = ix[j][0];
    }
}

// ---------------------------------------------------------------------------
// R > 64 (SPAN = 128 or 256).  Affinity: thread (s, g) = (tid % SPAN,
// tid / SPAN) keeps K mean s in registers and takes its dots with query rows
// g, g + G, ... of the chunk (G = kThreads / SPAN row groups; g is
// wave-uniform), kRouteChains at a time; the entries go to LDS.  Top-k: wave
// w takes rows w and w + kWaves.
template <int NW, int KTOP, int SPAN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void
route_large_kernel(const double* __restrict__ means, int32_t* __restrict__ idx_out, Params p_in) {
    Params p = p_in;
    if constexpr (NW > 0) {
        p.n = NW;
        p.R = NW * NW;
    }
    if constexpr (KTOP > 0) p.k = KTOP;
    constexpr int ROWS = route_rows(SPAN);
    constexpr int RPW = ROWS / kWaves;  // top-k rows per wave
    constexpr int G = kThreads / SPAN;
    constexpr int NR = ROWS / G;        // rows per thread in the affinity phase
    static_assert(NR % kRouteChains == 0, "rows per thread come in whole chain groups");
    extern __shared__ __align__(16) unsigned char smem[];
    double* sA = reinterpret_cast<double*>(smem);  // [ROWS][RS]

    const int R = p.R, RS = route_row_stride(R);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunk = (R + ROWS - 1) / ROWS;
    const int rg = blockIdx.x / nchunk, chunk = blockIdx.x - rg * nchunk;
    const int r0 = chunk * ROWS, nrows = min(ROWS, R - r0);
    const int h0 = p.shared ? rg * p.heads : rg;
    const int nh = p.shared ? p.heads : 1;

    const int s = tid % SPAN;
    const int g = __builtin_amdgcn_readfirstlane(tid / SPAN);
    double acc[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[j] = 0.0;
    for (int hh = 0; hh < nh; ++hh) {
        const int bh = h0 + hh;
        double kreg[kHeadDim];
        load_kmean(p, means, bh, min(s, R - 1), kreg);
#pragma unroll
        for (int c = 0; c < NR / kRouteChains; ++c) {
            const double* q[kRouteChains];
            double part[kRouteChains];
#pragma unroll
            for (int j = 0; j < kRouteChains; ++j) {
                const int row = g + G * (c * kRouteChains + j);
                q[j] = means + qmean_index(p, bh, min(r0 + row, R - 1), 0);
                part[j] = acc[c * kRouteChains + j];
            }
            dots_seq<kRouteChains>(part, q, kreg);
#pragma unroll
            for (int j = 0; j < kRouteChains; ++j) acc[c * kRouteChains + j] = part[j];
        }
    }
    if (s < R) {
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const int row = g + G * j;
            if (row < nrows) sA[row * RS + s] = acc[j];
        }
    }
    __syncthreads();

    int32_t* const base = idx_out + (static_cast<size_t>(rg) * R + r0) * p.k;
    if (p.k == 1) {
        double best[RPW];
        int bs[RPW];
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const double* row = sA + min(w + kWaves * j, nrows - 1) * RS;
            best[j] = -INFINITY;
            bs[j] = 0x7fffffff;
            for (int x = lane; x < R; x += 64) {
                const double a = row[x];
                if (a > best[j] || bs[j] == 0x7fffffff) {
                    best[j] = a;
                    bs[j] = x;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < RPW; ++j) wave_argmax(best[j], bs[j]);
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int row = w + kWaves * j;
            if (lane == 0 && row < nrows) base[row] = min(max(bs[j], 0), R - 1);
        }
    } else {
        constexpr int E = SPAN / 64;
        const double* rows[RPW];
        int32_t* dst[RPW];
        bool live[RPW];
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int row = w + kWaves * j;
            rows[j] = sA + min(row, nrows - 1) * RS;
            dst[j] = base + row * p.k;
            live[j] = row < nrows;
        }
        wave_topk_bitonic<E, RPW>(rows, R, p.k, dst, live);
    }
}

// ---------------------------------------------------------------------------
// Region means and routing in one kernel, for small region grids routed
// outside the attention kernel (R <= 64 with more than kWaves heads, bf16,
// per head) whose K for one head fits LDS.  Workgroup (image b, head h,
// chunk of route_rows(64) query rows):
//   1. K of head h for all R regions (R * t tokens, 64 bytes each) and Q of
//      the chunk's regions reach LDS by LDS DMA (global_load_lds_dwordx4: a
//      wave instruction fills 64 consecutive 16-byte slots, lane L slot L).
//   2. Threads take (region, dim) items: the fp64 sum of the t bf16 values
//      (exact within the span condition of row16_sum_exact in bra_device.h)
//      divided by t -- bit for bit the pool kernel's mean -- into
//      K-bar [32][R] (lane s reads region s) and Q-bar [rows][32], which
//      overlay the staged K and Q once every sum is taken.
//   3. Each wave routes kRouteChains rows as route_small_kernel does, from
//      the LDS means.
// The means never go to HBM, and the routing needs no second launch.
constexpr int kPoolRouteRows = kWaves * kRouteChains;

// 16-byte slots of one head's K (R * t tokens, 4 slots each) and of the
// chunk's Q, in whole DMA rounds of kThreads slots.
__host__ __device__ constexpr int pr_k_rounds(int R, int t) {
    return (R * t * 4 + kThreads - 1) / kThreads;
}
__host__ __device__ constexpr int pr_q_rounds(int t) {
    return (kPoolRouteRows * t * 4 + kThreads - 1) / kThreads;
}
// LDS: staged K, then K-bar over it; staged Q, then Q-bar over it.
__host__ __device__ constexpr int pr_k_bytes(int R, int t) {
    return pr_k_rounds(R, t) * kThreads * 16 > kHeadDim * R * 8 ? pr_k_rounds(R, t) * kThreads * 16
                                                                 : kHeadDim * R * 8;
}
__host__ __device__ constexpr int pr_q_bytes(int t) {
    return pr_q_rounds(t) * kThreads * 16 > kPoolRouteRows * kHeadDim * 8
               ? pr_q_rounds(t) * kThreads * 16
               : kPoolRouteRows * kHeadDim * 8;
}
__host__ __device__ constexpr int pool_route_lds_bytes(int R, int t) {
    return pr_k_bytes(R, t) + pr_q_bytes(t);
}
// (region, dim) mean items per thread: at most 64 regions of 32 dims, and
// the chunk's 16 query rows.
constexpr int kKMeanItems = 64 * kHeadDim / kThreads;
constexpr int kQMeanItems = kPoolRouteRows * kHeadDim / kThreads;

template <int HS, int WS, int NW, int HEADS, int KTOP>
__global__ __launch_bounds__(kThreads) void pool_route_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int32_t* __restrict__ idx_out,
    const float* __restrict__ lepe_w, uint2* __restrict__ lepe_table, Params p_in) {
    const Params p = fold_geometry<HS, WS, NW, HEADS, KTOP, 8>(p_in);
    extern __shared__ __align__(16) unsigned char smem[];
    const int R = p.R, t = p.t, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunk = (R + kPoolRouteRows - 1) / kPoolRouteRows;
    const int tasks = p.B * p.heads * nchunk;
    if (static_cast<int>(blockIdx.x) >= tasks) {
        // trailing workgroups: the Toeplitz operands of the MFMA LePE
        const int it = (blockIdx.x - tasks) * kThreads + tid;
        if (it < p.table_items) lepe_table[it] = lepe_table_entry(lepe_w, it);
        return;
    }
    const int krounds = pr_k_rounds(R, t), qrounds = pr_q_rounds(t);
    uint16_t* sK = reinterpret_cast<uint16_t*>(smem);                    // [R * t][32]
    uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + pr_k_bytes(R, t));  // [rows * t][32]
    double* sKbar = reinterpret_cast<double*>(sK);  // [32][R], over sK
    double* sQbar = reinterpret_cast<double*>(sQ);  // [rows][32], over sQ
    const int blk = xcd_logical_block(blockIdx.x, tasks);
    const int bh = blk / nchunk, chunk = blk - bh * nchunk;
    const int b = bh / p.heads, h = bh - b * p.heads;
    const int r0 = chunk * kPoolRouteRows;
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C + h * kHeadDim;
    const int wave_slot0 = __builtin_amdgcn_readfirstlane(tid & ~63);
    // 1. DMA: slot i holds 16-byte piece i % 4 of token i / 4 (region
    //    token / t, slot token % t); slots past the end copy the last piece
    {
        const int last = R * t * 4 - 1;
        for (int j = 0; j < krounds; ++j) {
            const int i = min(j * kThreads + tid, last);
            const int tok = i >> 2, s = tok / t, u = tok - s * t;
            __builtin_amdgcn_global_load_lds(
                k + img + token_offset(p, s, u) + 8 * (i & 3),
                (__attribute__((address_space(3))) void*)(sK + 8 * (j * kThreads + wave_slot0)),
                16, 0, 0);
        }
        const int qlast = kPoolRouteRows * t * 4 - 1;
        for (int j = 0; j < qrounds; ++j) {
            const int i = min(j * kThreads + tid, qlast);
            const int tok = i >> 2, row = tok / t, u = tok - row * t;
            __builtin_amdgcn_global_load_lds(
                q + img + token_offset(p, min(r0 + row, R - 1), u) + 8 * (i & 3),
                (__attribute__((address_space(3))) void*)(sQ + 8 * (j * kThreads + wave_slot0)),
                16, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA has landed
    __syncthreads();
    // 2. the means: fp64 sums of bf16 values (any order: exact within the
    //    span condition of row16_sum_exact), then / t,
    //    held in registers until every staged value is read
    double km[kKMeanItems], qm[kQMeanItems];
#pragma unroll
    for (int j = 0; j < kKMeanItems; ++j) {
        const int item = tid + j * kThreads, s = item / kHeadDim, d = item - s * kHeadDim;
        double sum = 0.0;
        if (s < R)
            for (int u = 0; u < t; ++u)
                sum += static_cast<double>(bf16_to_f32(sK[(s * t + u) * kHeadDim + d]));
        km[j] = mean_of(sum, t);
    }
#pragma unroll
    for (int j = 0; j < kQMeanItems; ++j) {
        const int item = tid + j * kThreads, row = item / kHeadDim, d = item - row * kHeadDim;
        double sum = 0.0;
        for (int u = 0; u < t; ++u)
            sum += static_cast<double>(bf16_to_f32(sQ[(row * t + u) * kHeadDim + d]));
        qm[j] = mean_of(sum, t);
    }
    __syncthreads();  // the staged K and Q are read: the means overlay them
#pragma unroll
    for (int j = 0; j < kKMeanItems; ++j) {
        const int item = tid + j * kThreads, s = item / kHeadDim, d = item - s * kHeadDim;
        if (s < R) sKbar[d * R + s] = km[j];
    }
#pragma unroll
    for (int j = 0; j < kQMeanItems; ++j) sQbar[tid + j * kThreads] = qm[j];
    __syncthreads();
    // 3. routing of rows r0 + w * kRouteChains ..: lane s holds K-bar s
    const int rw = r0 + w * kRouteChains;
    if (rw >= R) return;  // wave-uniform; no barrier follows
    double kreg[kHeadDim];
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) kreg[d] = sKbar[d * R + min(lane, R - 1)];
    double acc[kRouteChains];
    const double* qr[kRouteChains];
#pragma unroll
    for (int j = 0; j < kRouteChains; ++j) {
        acc[j] = 0.0;
        qr[j] = sQbar + (w * kRouteChains + j) * kHeadDim;
    }
    dots_seq<kRouteChains>(acc, qr, kreg);
    int32_t* const base = idx_out + (static_cast<size_t>(bh) * R + rw) * p.k;
    const int nrows = min(kRouteChains, R - rw);
    if (p.k == 1) {
#pragma unroll
        for (int j = 0; j < kRouteChains; ++j) {
            double best = lane < R ? acc[j] : -INFINITY;
            int bs = lane < R ? lane : 0x7fffffff;
            wave_argmax(best, bs);
            if (lane == 0 && j < nrows) base[j] = min(max(bs, 0), R - 1);
        }
    } else {
        double v[kRouteChains][1];
        int ix[kRouteChains][1];
#pragma unroll
        for (int j = 0; j < kRouteChains; ++j) {
            v[j][0] = lane < R ? acc[j] : -INFINITY;
            ix[j][0] = lane;
        }
        route_topk<1, kRouteChains>(v, ix, lane, p.k);
#pragma unroll
        for (int j = 0; j < kRouteChains; ++j)
            if (j < nrows && lane < p.k) base[j * p.k + lane] = ix[j][0];
    }
}

template <int NW, int KTOP>
void launch_route_shape(const Params& p, const double* means, int32_t* idx, hipStream_t stream) {
    const int span = route_span(p.R);
    const int rows = route_rows(span);
    const int nchunk = (p.R + rows - 1) / rows;
    const dim3 grid(p.B * p.rheads * nchunk), block(kThreads);
    const int lds = rows * route_row_stride(p.R) * 8;
    // a fixed shape instantiates only its own span
    constexpr int kSpan = NW > 0 ? route_span(NW * NW) : 0;
    if constexpr (kSpan == 0 || kSpan == 64)
        if (span == 64) {
            hipLaunchKernelGGL((route_small_kernel<NW, KTOP>), grid, block, 0, stream, means,
                               idx, p);
            return;
        }
    if constexpr (kSpan == 0 || kSpan == 128)
        if (span == 128) {
            hipLaunchKernelGGL((route_large_kernel<NW, KTOP, 128>), grid, block, lds, stream,
                               means, idx, p);
            return;
        }
    if constexpr (kSpan == 0 || kSpan == 256)
        if (span == 256)
            hipLaunchKernelGGL((route_large_kernel<NW, KTOP, 256>), grid, block, lds, stream,
                               means, idx, p);
}

}  // namespace

int pool_route_lds(const Params& p) { return pool_route_lds_bytes(p.R, p.t); }

hipError_t launch_pool_route(const Params& p, const void* q, const void* k,
                             const float* lepe_w, uint2* lepe_table, int32_t* idx,
                             hipStream_t stream) {
    Params pp = p;
    if (!lepe_w) pp.table_items = 0;
    const int nchunk = (p.R + kPoolRouteRows - 1) / kPoolRouteRows;
    const int table_blocks = (pp.table_items + kThreads - 1) / kThreads;
    const dim3 grid(p.B * p.heads * nchunk + table_blocks), block(kThreads);
    const int lds = pool_route_lds_bytes(p.R, p.t);
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
#define BRA_POOL_ROUTE(T, HS, WS, NW, HEADS, KTOP)                                              \
    if constexpr (sizeof(T) == 2 && NW * NW <= 64 && HEADS > kWaves) {                         \
        if (matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, true, true)) {                   \
            hipLaunchKernelGGL((pool_route_kernel<HS, WS, NW, HEADS, KTOP>), grid, block, lds,  \
                               stream, qq, kk, idx, lepe_w, lepe_table, pp);                    \
            return hipGetLastError();                                                          \
        }                                                                                      \
    }
    BRA_FOR_EACH_SHAPE(BRA_POOL_ROUTE)
#undef BRA_POOL_ROUTE
    hipLaunchKernelGGL((pool_route_kernel<0, 0, 0, 0, 0>), grid, block, lds, stream, qq, kk, idx,
                       lepe_w, lepe_table, pp);
    return hipGetLastError();
}

hipError_t launch_route(const Params& p, bool bf16, const double* means, int32_t* idx,
                        hipStream_t stream) {
#define BRA_ROUTE(T, HS, WS, NW, HEADS, KTOP)                             \
    if (matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, true)) { \
        launch_route_shape<NW, KTOP>(p, means, idx, stream);             \
        return hipGetLastError();                                        \
    }
    BRA_FOR_EACH_SHAPE(BRA_ROUTE)
#undef BRA_ROUTE
    launch_route_shape<0, 0>(p, means, idx, stream);
    return hipGetLastError();
}

}  // namespace bra
