// bra_route.hip -- region-level routing [P4 §1.2; P1 §2.1 TopkRouting;
// P5 §五 ③-④] (page keys in bra_device.h).
//
// One workgroup per (image, head, chunk of query regions): the fp64 affinity
// A[r][s] = Qbar_r . Kbar_s of each row r of the chunk against every region
// s, then the k largest entries of each row, in descending order with exact
// ties to the lower region id.  The head_dim^-0.5 factor the pages apply to
// the affinity does not change the order and is left out.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_shapes.h"

namespace bra {
namespace {

__device__ __forceinline__ bool beats(double a, int ia, double b, int ib) {
    return a > b || (a == b && ia < ib);
}

// Top-k of one row by a wave-wide bitonic sort, best first (affinity
// descending, region id ascending).  Lane `lane` holds elements
// lane * E .. lane * E + E - 1; partners within a lane swap in registers,
// across lanes through shuffles.  Padding elements (ids >= R) carry -inf and
// sort last.  Writes the first k ids.
template <int E>
__device__ __forceinline__ void wave_topk_bitonic(const double* row, int R, int k,
                                                  int32_t* __restrict__ dst) {
    const int lane = threadIdx.x & 63;
    double v[E];
    int ix[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = lane * E + e;
        v[e] = i < R ? row[i] : -INFINITY;
        ix[e] = i;
    }
#pragma unroll
    for (int size = 2; size <= 64 * E; size <<= 1) {
#pragma unroll
        for (int j = size >> 1; j > 0; j >>= 1) {
            if (j < E) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int pe = e ^ j;
                    if (pe > e) {
                        const bool dir = ((lane * E + e) & size) == 0;
                        if (beats(v[e], ix[e], v[pe], ix[pe]) != dir) {
                            const double tv = v[e];
                            v[e] = v[pe];
                            v[pe] = tv;
                            const int ti = ix[e];
                            ix[e] = ix[pe];
                            ix[pe] = ti;
                        }
                    }
                }
            } else {
                const int lj = j / E;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const double ov = __shfl_xor(v[e], lj);
                    const int oi = __shfl_xor(ix[e], lj);
                    const int i = lane * E + e;
                    const bool lower = (i & j) == 0;
                    const bool dir = (i & size) == 0;
                    const bool mine = beats(v[e], ix[e], ov, oi);
                    if ((lower == dir) != mine) {
                        v[e] = ov;
                        ix[e] = oi;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = lane * E + e;
        if (i < k) dst[i] = ix[e];
    }
}

template <int NW, int KTOP>
__global__ __launch_bounds__(kThreads) void route_kernel(const double* __restrict__ means,
                                                         int32_t* __restrict__ idx_out,
                                                         Params p_in) {
    Params p = p_in;
    if constexpr (NW > 0) {
        p.n = NW;
        p.R = NW * NW;
    }
    if constexpr (KTOP > 0) p.k = KTOP;
    __shared__ double sQ[kRouteMaxRows * kHeadDim];
    extern __shared__ __align__(16) unsigned char smem[];
    double* sA = reinterpret_cast<double*>(smem);  // [rows][R]

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rows = p.route_rows;
    const int nchunk = (p.R + rows - 1) / rows;
    const int bh = blockIdx.x / nchunk, chunk = blockIdx.x - bh * nchunk;
    const int r0 = chunk * rows, nrows = min(rows, p.R - r0);
    const size_t mstride = static_cast<size_t>(p.B) * p.heads * p.R * kHeadDim;
    const double* qbar = means + static_cast<size_t>(bh) * p.R * kHeadDim;  // [R][32]
    const double* kbar = qbar + mstride;

    for (int i = tid; i < nrows * kHeadDim / 2; i += kThreads)
        reinterpret_cast<double2*>(sQ)[i] = reinterpret_cast<const double2*>(qbar + r0 * kHeadDim)[i];
    __syncthreads();

    // Affinity: a thread keeps one K mean in registers and takes the dot with
    // several query rows (exact sequential order, see dot32_seq).
    const int L = p.R <= 64 ? 64 : (p.R <= 128 ? 128 : 256);
    const int G = kThreads / L;
    const int s0 = tid % L, g = tid / L;
    for (int s = s0; s < p.R; s += L) {
        double kreg[kHeadDim];
        const double2* src = reinterpret_cast<const double2*>(kbar + s * kHeadDim);
#pragma unroll
        for (int d = 0; d < kHeadDim / 2; ++d) {
            const double2 x = src[d];
            kreg[2 * d] = x.x;
            kreg[2 * d + 1] = x.y;
        }
        for (int rr = g; rr < nrows; rr += G) sA[rr * p.R + s] = dot32_seq(sQ + rr * kHeadDim, kreg);
    }
    __syncthreads();

    // Top-k, one wave per row.
    for (int rr = w; rr < nrows; rr += kWaves) {
        const double* row = sA + rr * p.R;
        int32_t* dst = idx_out + (static_cast<size_t>(bh) * p.R + r0 + rr) * p.k;
        if (p.k == 1) {
            double best = -INFINITY;
            int bs = 0x7fffffff;
            for (int s = lane; s < p.R; s += 64) {
                const double a = row[s];
                if (a > best || bs == 0x7fffffff) {
                    best = a;
                    bs = s;
                }
            }
            wave_argmax(best, bs);
            if (lane == 0) dst[0] = bs;
        } else {
            const int e = (p.R + 63) / 64;
            if constexpr (NW > 0) {
                constexpr int RR = NW * NW;
                constexpr int EE = RR <= 64 ? 1 : RR <= 128 ? 2 : 4;
                wave_topk_bitonic<EE>(row, p.R, p.k, dst);
            } else if (e <= 1) {
                wave_topk_bitonic<1>(row, p.R, p.k, dst);
            } else if (e <= 2) {
                wave_topk_bitonic<2>(row, p.R, p.k, dst);
            } else {
                wave_topk_bitonic<4>(row, p.R, p.k, dst);  // R <= kMaxRegions = 256
            }
        }
    }
}

}  // namespace

hipError_t launch_route(const Params& p, bool bf16, const double* means, int32_t* idx,
                        hipStream_t stream) {
    const int nchunk = (p.R + p.route_rows - 1) / p.route_rows;
    const dim3 grid(p.B * p.heads * nchunk), block(kThreads);
    const int lds = p.route_rows * p.R * 8;
#define BRA_ROUTE(T, HS, WS, NW, HEADS, KTOP)                                                   \
    if (matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, true)) {                       \
        hipLaunchKernelGGL((route_kernel<NW, KTOP>), grid, block, lds, stream, means, idx, p); \
        return hipGetLastError();                                                              \
    }
    BRA_FOR_EACH_SHAPE(BRA_ROUTE)
#undef BRA_ROUTE
    hipLaunchKernelGGL((route_kernel<0, 0>), grid, block, lds, stream, means, idx, p);
    return hipGetLastError();
}

}  // namespace bra
