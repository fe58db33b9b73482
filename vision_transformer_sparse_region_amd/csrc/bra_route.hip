// bra_route.hip -- region-level routing [P4 §1.2; P1 §2.1 TopkRouting;
// P5 §五 ③-④] (page keys in bra_device.h).
//
// One workgroup per (image, head, chunk of query regions) -- per image with
// head-shared routing [P1 §2.2; P2 §2.1; P3 §2.1] -- : the fp64 affinity
// A[r][s] = Qbar_r . Kbar_s of each row r of the chunk against every region
// s (over one head's 32 dims, or all C channels when shared), then the k
// largest entries of each row, in descending order with exact ties to the
// lower region id.  The head_dim^-0.5 factor the pages apply to
// the affinity does not change the order and is left out.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_shapes.h"

namespace bra {
namespace {

// Region-span of the affinity phase: threads tid % SPAN own region tid % SPAN,
// SPAN = the power of two >= R (64, 128 or 256 = kMaxRegions).
__host__ __device__ constexpr int route_span(int R) { return R <= 64 ? 64 : R <= 128 ? 128 : 256; }
// Query rows a workgroup routes: 4 per wave for R <= 64, else 2 per wave.
__host__ __device__ constexpr int route_rows_per_wave(int span) { return span == 64 ? 4 : 2; }
// fp64 row stride of the affinity tile (even, so pairs of entries are 16-byte aligned).
__host__ __device__ constexpr int route_row_stride(int R) { return (R + 1) & ~1; }

__device__ __forceinline__ bool beats(double a, int ia, double b, int ib) {
    return a > b || (a == b && ia < ib);
}

// Top-k of NRW rows at once by wave-wide bitonic sorts, best first (affinity
// descending, region id ascending).  Lane `lane` holds elements
// lane * E .. lane * E + E - 1 of every row; partners within a lane swap in
// registers, across lanes through shuffles.  Padding elements (ids >= R)
// carry -inf and sort last.  Writes the first k ids of row j to dst[j].
template <int E, int NRW>
__device__ __forceinline__ void wave_topk_bitonic(const double* const (&rows)[NRW], int R, int k,
                                                  int32_t* const (&dst)[NRW], const bool (&live)[NRW]) {
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
#pragma unroll
    for (int size = 2; size <= 64 * E; size <<= 1) {
#pragma unroll
        for (int j = size >> 1; j > 0; j >>= 1) {
            if (j < E) {
#pragma unroll
                for (int r = 0; r < NRW; ++r) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int pe = e ^ j;
                        if (pe > e) {
                            const bool dir = ((lane * E + e) & size) == 0;
                            if (beats(v[r][e], ix[r][e], v[r][pe], ix[r][pe]) != dir) {
                                const double tv = v[r][e];
                                v[r][e] = v[r][pe];
                                v[r][pe] = tv;
                                const int ti = ix[r][e];
                                ix[r][e] = ix[r][pe];
                                ix[r][pe] = ti;
                            }
                        }
                    }
                }
            } else {
                const int lj = j / E;
#pragma unroll
                for (int r = 0; r < NRW; ++r) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const double ov = __shfl_xor(v[r][e], lj);
                        const int oi = __shfl_xor(ix[r][e], lj);
                        const int i = lane * E + e;
                        const bool lower = (i & j) == 0;
                        const bool dir = (i & size) == 0;
                        const bool mine = beats(v[r][e], ix[r][e], ov, oi);
                        if ((lower == dir) != mine) {
                            v[r][e] = ov;
                            ix[r][e] = oi;
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = lane * E + e;
            if (live[r] && i < k) dst[r][i] = ix[r][e];
        }
    }
}

// NW > 0 / KTOP > 0 fold the region count / k at compile time.  SPAN is
// route_span(R).  Rows of a chunk go to waves round-robin (row = w + 4j).
template <int NW, int KTOP, int SPAN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void route_kernel(const double* __restrict__ means,
                                                         int32_t* __restrict__ idx_out,
                                                         Params p_in) {
    Params p = p_in;
    if constexpr (NW > 0) {
        p.n = NW;
        p.R = NW * NW;
    }
    if constexpr (KTOP > 0) p.k = KTOP;
    constexpr int RPW = route_rows_per_wave(SPAN);
    constexpr int ROWS = kWaves * RPW;
    constexpr int G = kThreads / SPAN;  // row groups of the affinity phase
    constexpr int NR = ROWS / G;        // rows per thread in the affinity phase
    __shared__ double sQ[ROWS * kHeadDim];
    extern __shared__ __align__(16) unsigned char smem[];
    double* sA = reinterpret_cast<double*>(smem);  // [ROWS][RS]

    const int R = p.R, RS = route_row_stride(R);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nchunk = (R + ROWS - 1) / ROWS;
    // rg: the routing's (image, head) pair, or the image with shared routing
    const int rg = blockIdx.x / nchunk, chunk = blockIdx.x - rg * nchunk;
    const int r0 = chunk * ROWS, nrows = min(ROWS, R - r0);
    const int h0 = p.shared ? rg * p.heads : rg;          // first (image, head) summed
    const int nh = p.shared ? p.heads : 1;                // heads summed into one affinity

    // Affinity.  Thread (s, g) keeps K mean s in registers and takes its dot
    // with query rows g, g + G, ...; rows past the chunk read zeros.  With
    // shared routing the heads follow one another in one running sum per
    // entry (kept in sA), so every entry is the sequential sum over all C
    // channels in the order c = h * 32 + d.
    const int s = tid % SPAN, g = tid / SPAN;
    for (int hh = 0; hh < nh; ++hh) {
        const int bh = h0 + hh;
        const double* qbar = means + qmean_index(p, bh, 0, 0);  // [R][32]
        double kreg[kHeadDim];
        load_kmean(p, means, bh, min(s, R - 1), kreg);
        for (int i = tid; i < ROWS * kHeadDim / 2; i += kThreads) {
            const bool in = i < nrows * kHeadDim / 2;
            reinterpret_cast<double2*>(sQ)[i] =
                in ? reinterpret_cast<const double2*>(qbar + r0 * kHeadDim)[i]
                   : double2{0.0, 0.0};
        }
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < NR; ++j) {
            const int row = g + G * j;
            if (s < R && row < nrows) {
                const double a0 = hh == 0 ? 0.0 : sA[row * RS + s];
                sA[row * RS + s] = dot32_seq_from(a0, sQ + row * kHeadDim, kreg);
            }
        }
        __syncthreads();
    }

    // Top-k, rows w, w + 4, ... of the chunk on wave w.
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
            if (lane == 0 && row < nrows) base[row] = bs[j];
        }
    } else if constexpr (SPAN == 64) {
        // R <= 64: lane i ranks element i of each row against the whole row
        // (broadcast reads); ranks are distinct, and rank < k places the id.
        double mine[RPW];
        int rank[RPW];
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const double* row = sA + min(w + kWaves * j, nrows - 1) * RS;
            mine[j] = lane < R ? row[lane] : -INFINITY;
            rank[j] = 0;
        }
        for (int x = 0; x < R; ++x) {
#pragma unroll
            for (int j = 0; j < RPW; ++j) {
                const double a = sA[min(w + kWaves * j, nrows - 1) * RS + x];
                rank[j] += (a > mine[j] || (a == mine[j] && x < lane)) ? 1 : 0;
            }
        }
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int row = w + kWaves * j;
            if (row < nrows && lane < R && rank[j] < p.k) base[row * p.k + rank[j]] = lane;
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

}  // namespace

hipError_t launch_route(const Params& p, bool bf16, const double* means, int32_t* idx,
                        hipStream_t stream) {
    const int span = route_span(p.R);
    const int rows = kWaves * route_rows_per_wave(span);
    const int nchunk = (p.R + rows - 1) / rows;
    const dim3 grid(p.B * p.rheads * nchunk), block(kThreads);
    const int lds = rows * route_row_stride(p.R) * 8;
#define BRA_ROUTE(T, HS, WS, NW, HEADS, KTOP)                                                \
    if (matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, true)) {                    \
        hipLaunchKernelGGL((route_kernel<NW, KTOP, route_span(NW * NW)>), grid, block, lds, \
                           stream, means, idx, p);                                          \
        return hipGetLastError();                                                           \
    }
    BRA_FOR_EACH_SHAPE(BRA_ROUTE)
#undef BRA_ROUTE
    if (span == 64)
        hipLaunchKernelGGL((route_kernel<0, 0, 64>), grid, block, lds, stream, means, idx, p);
    else if (span == 128)
        hipLaunchKernelGGL((route_kernel<0, 0, 128>), grid, block, lds, stream, means, idx, p);
    else
        hipLaunchKernelGGL((route_kernel<0, 0, 256>), grid, block, lds, stream, means, idx, p);
    return hipGetLastError();
}

}  // namespace bra
