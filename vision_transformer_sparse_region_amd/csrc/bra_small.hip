// bra_small.hip -- the whole fp32 forward of a small problem in one launch:
// one workgroup per (image, head, query region), for problems with at most
// 256 of them (one workgroup per CU at most), where a second launch and the
// memory round trips between kernels cost more than recomputing every
// region mean of the head in each workgroup.  (page keys in bra_device.h)
//
// A workgroup (image b, head h, region r):
//   1. stages by LDS DMA the K map of head h (every token, in map order),
//      the Q rows of region r and the V window of r with its 2-cell halo;
//      the LePE weights and bias of the head's channels go to LDS by plain
//      loads (they need only be 4-byte aligned)               [P5 §五 ③, ⑤]
//   2. the K mean of every region and the Q mean of r: fp64 sums of the fp32
//      values in slot order, as the oracle takes them   [P4 §1.2; P5 §五 ③]
//   3. routes row r on one wave (route_row_wave, exact fp64 pass: the
//      oracle-order dot, affinity descending, ties to the lower id)
//                                          [P1 §2.1 TopkRouting; P5 §五 ④]
//   4. gathers the routed regions' V rows by LDS DMA -- their K rows are
//      already staged -- and, while they land, forms the scores and the
//      softmax (fp32, one query per group of L lanes, L a compile-time
//      8, 16 or 32)                                   [P3 §2.2; P5 §五 ⑤-⑥]
//   5. out = P V + dwconv5x5(V) + bias, in fp32, stored as the map's rows
//                                             [P5 §五 ⑦-⑧, lepe; P2 §2.2]
// Staged rows are 8 pieces of 16 bytes (32 fp32 dims); piece c of row i sits
// at slot c ^ (i & 7), so that the rows the lanes of one LDS instruction
// read fall on different banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_launch.h"
#include "bra_small.h"

namespace bra {
namespace small {

constexpr int kST = kSmallThreads;

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dma16(const float* src, float* lds_slot0) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_slot0, 16,
                                     0, 0);
}

// Piece c (4 dims) of staged row i.
__device__ __forceinline__ f32x4v piece(const float* base, int i, int c) {
    return *reinterpret_cast<const f32x4v*>(base + 32 * i + 4 * (c ^ (i & 7)));
}

__device__ __forceinline__ float elem(const float* base, int i, int d) {
    return base[32 * i + 4 * ((d >> 2) ^ (i & 7)) + (d & 3)];
}

// Dims d0 .. d0 + N - 1 of staged row i (d0 a multiple of N, N = 1, 2, 4, 8).
template <int N>
__device__ __forceinline__ void dims(const float* base, int i, int d0, float (&x)[N]) {
    if constexpr (N >= 4) {
#pragma unroll
        for (int c = 0; c < N / 4; ++c) {
            const f32x4v v4 = piece(base, i, (d0 >> 2) + c);
            x[4 * c] = v4[0];
            x[4 * c + 1] = v4[1];
            x[4 * c + 2] = v4[2];
            x[4 * c + 3] = v4[3];
        }
    } else if constexpr (N == 2) {
        const float2 v2 = *reinterpret_cast<const float2*>(
            base + 32 * i + 4 * ((d0 >> 2) ^ (i & 7)) + (d0 & 3));
        x[0] = v2.x;
        x[1] = v2.y;
    } else {
        x[0] = elem(base, i, d0);
    }
}

// Max and sum over the L consecutive lanes of one query (L = 8, 16 or 32):
// DPP within rows of 16 (lane ^ 1, ^ 2, the half-row and row mirrors), the
// row swap for lanes 16 apart.  Each step pairs lanes symmetrically, so every
// lane of the group ends with the same value; no step goes through the LDS
// crossbar.
template <int L>
__device__ __forceinline__ float group_max(float x) {
    static_assert(L == 8 || L == 16 || L == 32, "8, 16 or 32 lanes a query");
    x = fmaxf(x, dpp_f32<0xB1>(x));
    x = fmaxf(x, dpp_f32<0x4E>(x));
    x = fmaxf(x, dpp_f32<0x141>(x));
    if constexpr (L >= 16) x = fmaxf(x, dpp_f32<0x140>(x));
    if constexpr (L == 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    }
    return x;
}
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(L == 8 || L == 16 || L == 32, "8, 16 or 32 lanes a query");
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0x141>(x);
    if constexpr (L >= 16) x += dpp_f32<0x140>(x);
    if constexpr (L == 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    return x;
}

// floor(a / b) for 0 <= a < 2^12, 1 <= b <= 64: a + 1/2 stays at least
// 1/128 of b away from a multiple of b, far beyond the product's rounding
__device__ __forceinline__ int small_div(int a, float inv_b) {
    return __float2int_rz((static_cast<float>(a) + 0.5f) * inv_b);
}

template <int L>
__device__ __forceinline__ void small_body(const float* __restrict__ q,
                                           const float* __restrict__ k,
                                           const float* __restrict__ v,
                                           const float* __restrict__ lepe_w,
                                           const float* __restrict__ lepe_b,
                                           int32_t* __restrict__ routing, float* __restrict__ out,
                                           Params p) {
    constexpr int DPL = kHeadDim / L;  // output dims of a lane
    extern __shared__ __align__(16) unsigned char smem[];
    const SmallGeo G = small_geo(p);
    float* sK = reinterpret_cast<float*>(smem + G.off_k);
    double* sKbar = reinterpret_cast<double*>(smem + G.off_kbar);
    float* sV = reinterpret_cast<float*>(smem + G.off_v);
    float* sP = reinterpret_cast<float*>(smem + G.off_p);
    float* sH = reinterpret_cast<float*>(smem + G.off_h);
    float* sQ = reinterpret_cast<float*>(smem + G.off_q);
    float* sW = reinterpret_cast<float*>(smem + G.off_w);  // [25 taps][32 dims], then the bias
    int* sIds = reinterpret_cast<int*>(smem + G.off_ids);
    int* sSlot = reinterpret_cast<int*>(smem + G.off_tab);  // slot -> token offset in a window
    int* sRegTok = sSlot + 64;                              // region -> its first token

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot0 = __builtin_amdgcn_readfirstlane(tid & ~63);
    // consecutive logical blocks -- the regions of one (image, head) -- on one
    // XCD, whose L2 then serves the repeated K map reads
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int r = blk % p.R, bh = blk / p.R, h = bh % p.heads, b = bh / p.heads;
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C + h * kHeadDim;
    const int t = p.t, R = p.R, nk = p.nkeys, HW = p.H * p.W, C = p.C;
    const bool has_lepe = p.has_lepe != 0;
    const int y0 = (r / p.n) * p.hs, x0 = (r % p.n) * p.ws;
    const int hw4 = p.ws + 4, ncell = (p.hs + 4) * hw4;
    const int rtok = y0 * p.W + x0;

    // the LePE weights and bias of the head's channels, loaded first (into
    // registers: their rows need only be 4-byte aligned, which LDS DMA does
    // not take) and stored to LDS once the DMA below is issued
    constexpr int kWPer = (kHeadDim * 25 + kST - 1) / kST;
    float wv[kWPer];
    float bv = 0.f;
    if (has_lepe) {
#pragma unroll
        for (int j = 0; j < kWPer; ++j) {
            const int i = tid + j * kST;
            wv[j] = i < kHeadDim * 25 ? lepe_w[h * kHeadDim * 25 + i] : 0.f;
        }
        if (tid < kHeadDim && lepe_b) bv = lepe_b[h * kHeadDim + tid];
    }

    // 1. DMA.  Slot s of a staged array holds piece (s & 7) ^ (row & 7) of
    //    row s >> 3; slots past the last (up to a whole number of rounds)
    //    repeat the last piece.  K rows are map tokens, Q rows the window's
    //    slots, halo rows the window's cells with their 2-cell border.
    for (int j = 0; j < G.rk; ++j) {
        const int s = min(j * kST + tid, 8 * HW - 1);
        const int tok = s >> 3, c = (s & 7) ^ (tok & 7);
        dma16(k + img + static_cast<size_t>(tok) * C + 4 * c, sK + 4 * (j * kST + slot0));
    }
    for (int j = 0; j < G.rq; ++j) {
        const int s = min(j * kST + tid, 8 * t - 1);
        const int u = s >> 3, uy = u / p.ws, c = (s & 7) ^ (u & 7);
        dma16(q + img + static_cast<size_t>(rtok + uy * p.W + u - uy * p.ws) * C + 4 * c,
              sQ + 4 * (j * kST + slot0));
    }
    if (has_lepe) {
        // cells outside the map load a clamped cell; their taps weigh zero
        for (int j = 0; j < G.rh; ++j) {
            const int s = min(j * kST + tid, 8 * ncell - 1);
            const int cell = s >> 3, hy = cell / hw4, hx = cell - hy * hw4;
            const int y = min(max(y0 + hy - 2, 0), p.H - 1), x = min(max(x0 + hx - 2, 0), p.W - 1);
            const int c = (s & 7) ^ (cell & 7);
            dma16(v + img + (static_cast<size_t>(y) * p.W + x) * C + 4 * c,
                  sH + 4 * (j * kST + slot0));
        }
#pragma unroll
        for (int j = 0; j < kWPer; ++j) {
            const int i = tid + j * kST;
            if (i < kHeadDim * 25) {
                const int d = i / 25, tap = i - d * 25;
                sW[tap * kHeadDim + d] = wv[j];
            }
        }
        if (tid < kHeadDim) sW[25 * kHeadDim + tid] = bv;
    }
    if (tid < t) sSlot[tid] = (tid / p.ws) * p.W + tid % p.ws;
    if (tid < R) sRegTok[tid] = (tid / p.n) * p.hs * p.W + (tid % p.n) * p.ws;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA has landed
    __syncthreads();

    // 2. the means: item (region s, dims 4c .. 4c + 3) sums its slots in order
    for (int it = tid; it < R * 8; it += kST) {
        const int s = it >> 3, c = it & 7, tb = sRegTok[s];
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        // (unrolled so that the LDS reads go out together; the additions
        // stay in slot order)
#pragma unroll 8
        for (int u = 0; u < t; ++u) {
            const f32x4v x = piece(sK, tb + sSlot[u], c);
            a0 += static_cast<double>(x[0]);
            a1 += static_cast<double>(x[1]);
            a2 += static_cast<double>(x[2]);
            a3 += static_cast<double>(x[3]);
        }
        double* dst = sKbar + s * kHeadDim + 4 * c;
        dst[0] = mean_of(a0, t);
        dst[1] = mean_of(a1, t);
        dst[2] = mean_of(a2, t);
        dst[3] = mean_of(a3, t);
    }
    // the Q mean of region r, in the routing wave's lane layout (lane d and
    // d + 32 hold dim d)
    double qmean = 0.0;
    if (w == 0) {
        const int d = lane & 31;
#pragma unroll 8
        for (int u = 0; u < t; ++u) qmean += static_cast<double>(elem(sQ, u, d));
        qmean = mean_of(qmean, t);
    }
    __syncthreads();

    // 3. the routing of row r (wave 0; ids to LDS, then to the caller)
    if (w == 0) {
        double kreg[kHeadDim];
        const double* km = sKbar + min(lane, R - 1) * kHeadDim;
#pragma unroll
        for (int d = 0; d < kHeadDim; ++d) kreg[d] = km[d];
        route_row_wave(p, qmean, false, kreg, nullptr, bh, sIds + kMaxSmallK, sIds);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < p.k) {
            const int id = sIds[lane];
            // the routed region's first token (over its base offset, which
            // the gathers here do not use)
            sIds[kMaxSmallK + lane] = sRegTok[id];
            if (routing) routing[(static_cast<size_t>(bh) * R + r) * p.k + lane] = id;
        }
    }
    __syncthreads();

    // 4. the routed V rows by DMA (key kk = rank * t + slot); meanwhile the
    //    scores from the staged K rows and the softmax
    const float inv_t = 1.f / static_cast<float>(t), inv_ws = 1.f / static_cast<float>(p.ws);
    const int* sRankTok = sIds + kMaxSmallK;
    // the map token of key kk: rank kk / t, slot kk % t of that region
    auto key_token = [&](int kk) {
        const int rank = small_div(kk, inv_t), u = kk - rank * t;
        const int uy = small_div(u, inv_ws);
        return sRankTok[rank] + uy * p.W + (u - uy * p.ws);
    };
    for (int j = 0; j < G.rv; ++j) {
        const int s = min(j * kST + tid, 8 * nk - 1);
        const int kk = s >> 3;
        const int tok = key_token(kk);
        const int c = (s & 7) ^ (kk & 7);
        dma16(v + img + static_cast<size_t>(tok) * C + 4 * c, sV + 4 * (j * kST + slot0));
    }
    const int qi = tid / L, li = tid - qi * L;
    const bool active = qi < t;
    float* prow = sP + qi * G.pstride;
    float inv = 0.f;
    if (active) {
        float qv[kHeadDim];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const f32x4v x = piece(sQ, qi, c);
            qv[4 * c] = x[0];
            qv[4 * c + 1] = x[1];
            qv[4 * c + 2] = x[2];
            qv[4 * c + 3] = x[3];
        }
        // raw scaled scores into the row, then the exponentials in place
        float mx = -INFINITY;
#pragma unroll 4
        for (int kk = li; kk < nk; kk += L) {
            const int tok = key_token(kk);
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const f32x4v x = piece(sK, tok, c);
                a = fmaf(qv[4 * c], x[0], a);
                a = fmaf(qv[4 * c + 1], x[1], a);
                a = fmaf(qv[4 * c + 2], x[2], a);
                a = fmaf(qv[4 * c + 3], x[3], a);
            }
            const float sc = a * p.scale_log2e;
            prow[kk] = sc;
            mx = fmaxf(mx, sc);
        }
        mx = group_max<L>(mx);
        float sum = 0.f;
#pragma unroll 4
        for (int kk = li; kk < nk; kk += L) {
            const float e = exp2f(prow[kk] - mx);
            prow[kk] = e;
            sum += e;
        }
        sum = group_sum<L>(sum);
        inv = 1.f / sum;
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's V DMA has landed
    __syncthreads();

    // 5. P V, LePE, store: lane li of query qi takes dims li * DPL ..
    if (active) {
        const int d0 = li * DPL;
        float o[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = 0.f;
#pragma unroll 16
        for (int kk = 0; kk < nk; ++kk) {
            const float pk = prow[kk];
            float x[DPL];
            dims<DPL>(sV, kk, d0, x);
#pragma unroll
            for (int e = 0; e < DPL; ++e) o[e] = fmaf(pk, x[e], o[e]);
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] *= inv;
        if (has_lepe) {
            const int yy = qi / p.ws, xx = qi - yy * p.ws;
            float acc[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[e] = sW[25 * kHeadDim + d0 + e];
            // every tap reads its (clamped) halo cell; a tap outside the map
            // weighs zero
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int y = y0 + yy + i - 2;
                const bool yin = y >= 0 && y < p.H;
#pragma unroll
                for (int jx = 0; jx < 5; ++jx) {
                    const int x = x0 + xx + jx - 2;
                    const bool in = yin && x >= 0 && x < p.W;
                    float hv[DPL], wt[DPL];
                    dims<DPL>(sH, (yy + i) * hw4 + xx + jx, d0, hv);
                    const float* wrow = sW + (i * 5 + jx) * kHeadDim + d0;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) {
                        wt[e] = in ? wrow[e] : 0.f;
                        acc[e] = fmaf(wt[e], hv[e], acc[e]);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < DPL; ++e) o[e] += acc[e];
        }
        float* dst = out + img + static_cast<size_t>(rtok + sSlot[qi]) * C + d0;
#pragma unroll
        for (int e = 0; e < DPL; ++e) dst[e] = o[e];
    }
}

// (__global__ wrappers around the body: a kernel whose body the host pass
// cannot instantiate would lose its launch stub)
template <int L>
__global__ __launch_bounds__(kST) void small_kernel(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    const float* __restrict__ v,
                                                    const float* __restrict__ lepe_w,
                                                    const float* __restrict__ lepe_b,
                                                    int32_t* __restrict__ routing,
                                                    float* __restrict__ out, Params p) {
    small_body<L>(q, k, v, lepe_w, lepe_b, routing, out, p);
}

template <int L>
const void* kernel_of() {
    return reinterpret_cast<const void*>(&small_kernel<L>);
}

}  // namespace small

bool small_applies(const Params& p, bool bf16) {
    if (bf16 || p.shared || p.kv_ratio != 1) return false;
    if (static_cast<long>(p.B) * p.heads * p.R > kSmallMaxBlocks) return false;
    if (p.R > 64 || p.t > 64 || p.k > kMaxSmallK) return false;
    const SmallGeo G = small_geo(p);
    return G.lds <= kMaxLdsBytes;
}

int small_lds_bytes(const Params& p) { return small_geo(p).lds; }

hipError_t prepare_small(const Params& p) {
    if (small_geo(p).lds <= kDefaultLdsBytes) return hipSuccess;
    for (const void* f : {small::kernel_of<8>(), small::kernel_of<16>(), small::kernel_of<32>()}) {
        const hipError_t e =
            hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_small(const Params& p, const float* q, const float* k, const float* v,
                        const float* lepe_w, const float* lepe_b, int32_t* routing, float* out,
                        hipStream_t stream) {
    Params pp = p;
    pp.has_lepe = lepe_w != nullptr;
    const SmallGeo G = small_geo(p);
    const dim3 grid(p.B * p.heads * p.R), block(kSmallThreads);
#define BRA_SMALL_L(LL)                                                                        \
    case LL:                                                                                   \
        hipLaunchKernelGGL(small::small_kernel<LL>, grid, block, G.lds, stream, q, k, v,       \
                           lepe_w, lepe_b, routing, out, pp);                                  \
        break;
    switch (G.L) {
        BRA_SMALL_L(8)
        BRA_SMALL_L(16)
        BRA_SMALL_L(32)
        default:
            return hipErrorInvalidValue;
    }
#undef BRA_SMALL_L
    return hipGetLastError();
}

}  // namespace bra
