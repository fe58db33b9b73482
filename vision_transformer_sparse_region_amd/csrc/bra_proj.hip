// bra_proj.hip -- the qkv projection before the path [P5 §五 ① qkv =
// Linear(dim, 3*dim); P4 §1.1], on MFMA, with the region means of the
// projected Q and K in its epilogue (page keys in bra_device.h).
//
// A workgroup takes up to proj_slice(C) tokens (64; 32 or 16 for wide maps)
// at a time: the tokens of `group` whole regions of one image when a region
// is smaller than that, or slices of one larger region.  The slice of x goes
// to LDS once; then for each of q, k and v and each 16-channel output tile,
//   D^T = W[o0 .. o0+15, :] . X^T          (v_mfma_f32_16x16x32_bf16, fp32 sums)
// with operand A row m the PyTorch Linear weight row o0 + m (16 contiguous
// bytes per lane and 32-channel step, from L2) and operand B column n token
// n of a 16-token tile (from LDS).  Lane (n, g) receives output channels
// o0 + 4g .. o0 + 4g + 3 of token n; adding the bias and rounding once to
// bf16 gives q, k or v as the module's Linear layer would produce them.  The
// rounded tile goes through LDS to 16-byte row stores, and for q and k each
// (region, channel) sums its tokens' rounded values in fp64 -- every partial
// sum of bf16 values is exact, so the region means equal those of the pool
// kernel over the stored maps, bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_shapes.h"

namespace bra {
namespace {

// LDS row stride (bf16 elements) of the x and output tiles: C plus 8, so
// consecutive rows start 16 bytes apart in the banks.
__host__ __device__ constexpr int proj_row(int C) { return C + 8; }

// Tokens a workgroup takes at a time: 64, fewer for wide maps, so that the
// two LDS tiles stay within 64 KB (C <= 512).
__host__ __device__ constexpr int proj_slice(int C) { return C <= 224 ? 64 : C <= 480 ? 32 : 16; }

// 32-channel steps of the contraction (C / 32), at most 16.
constexpr int kMaxProjSteps = 16;

// Regions per workgroup: the whole regions that fit one slice, else one.
__host__ __device__ constexpr int proj_group(int C, int t) {
    return t >= proj_slice(C) ? 1 : proj_slice(C) / t;
}

template <int HS, int WS, int NW, int HEADS>
__global__ __launch_bounds__(kThreads) void proj_qkv_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_qkv,
    const float* __restrict__ b_qkv, uint16_t* __restrict__ qs, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ vs, double* __restrict__ means, const float* __restrict__ lepe_w,
    uint2* __restrict__ lepe_table, Params p_in) {
    const Params p = fold_geometry<HS, WS, NW, HEADS, 1, 8>(p_in);
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int C = p.C, RS = proj_row(C), ST = proj_slice(C);
    const int group = proj_group(C, p.t);
    const int gpi = (p.R + group - 1) / group;  // workgroups per image
    if (static_cast<int>(blockIdx.x) >= p.B * gpi) {
        // trailing workgroups: the Toeplitz operands of the MFMA LePE
        const int it = (blockIdx.x - p.B * gpi) * kThreads + tid;
        if (it < p.table_items) lepe_table[it] = lepe_toeplitz_entry(lepe_w, it);
        return;
    }
    uint16_t* sX = reinterpret_cast<uint16_t*>(smem);  // [ST][RS]
    uint16_t* sO = sX + ST * RS;                         // [ST][RS]
    const int blk = xcd_logical_block(blockIdx.x, p.B * gpi);
    const int b = blk / gpi, r0 = (blk - b * gpi) * group;
    const int nreg = min(group, p.R - r0);
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C;
    const int nvec = C / 8, ksteps = C / 32, otiles = C / 16;
    const int n = lane & 15, g = lane >> 4;
    // token u of the workgroup: region r0 + u / t, slot u % t with several
    // regions; slot u of region r0, one slice of ST tokens at a time, with one
    const int span = group > 1 ? nreg * p.t : p.t;
    auto tok_offset = [&](int u) {
        return group > 1 ? token_offset(p, r0 + u / p.t, u - (u / p.t) * p.t)
                         : token_offset(p, r0, u);
    };
    // one region: the (channel) sums of q and k across slices, C <= 512
    // channels over the workgroup's threads
    constexpr int kCh = (512 + kThreads - 1) / kThreads;
    double qsum[kCh], ksum[kCh];
#pragma unroll
    for (int j = 0; j < kCh; ++j) qsum[j] = ksum[j] = 0.0;

    for (int u0 = 0; u0 < span; u0 += ST) {
        const int nt = min(ST, span - u0);
        __syncthreads();  // the previous slice's LDS reads are done
        for (int i = tid; i < nt * nvec; i += kThreads) {
            const int u = i / nvec, pv = i - u * nvec;
            *reinterpret_cast<uint4*>(sX + u * RS + 8 * pv) =
                *reinterpret_cast<const uint4*>(x + img + tok_offset(u0 + u) + 8 * pv);
        }
        __syncthreads();
        const int ttiles = (nt + 15) / 16;
        for (int which = 0; which < 3; ++which) {
            uint16_t* dst = which == 0 ? qs : which == 1 ? ks : vs;
            // wave wu takes output tiles wu, wu + kWaves, ...: the tile's weight
            // operands are loaded once and serve every token tile of the slice
            for (int ot = wu; ot < otiles; ot += kWaves) {
                const int o0 = ot * 16, ow = which * C + o0;  // row of w_qkv
                uint4 a[kMaxProjSteps];
#pragma unroll
                for (int s = 0; s < kMaxProjSteps; ++s)
                    if (s < ksteps)
                        a[s] = *reinterpret_cast<const uint4*>(
                            w_qkv + static_cast<size_t>(ow + n) * C + 32 * s + 8 * g);
                float bias[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) bias[i] = b_qkv ? b_qkv[ow + 4 * g + i] : 0.f;
                for (int tt = 0; tt < ttiles; ++tt) {
                    const int row = min(tt * 16 + n, nt - 1);
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < kMaxProjSteps; ++s)
                        if (s < ksteps) {
                            const uint4 xb = *reinterpret_cast<const uint4*>(sX + row * RS +
                                                                             32 * s + 8 * g);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, a[s]),
                                __builtin_bit_cast(bf16x8_t, xb), acc, 0, 0, 0);
                        }
                    uint32_t h[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) h[i] = f32_to_bf16(acc[i] + bias[i]);
                    if (tt * 16 + n < nt)
                        *reinterpret_cast<uint2*>(sO + (tt * 16 + n) * RS + o0 + 4 * g) =
                            uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                }
            }
            __syncthreads();
            // 16-byte row stores, then the q / k sums
            for (int i = tid; i < nt * nvec; i += kThreads) {
                const int u = i / nvec, pv = i - u * nvec;
                *reinterpret_cast<uint4*>(dst + img + tok_offset(u0 + u) + 8 * pv) =
                    *reinterpret_cast<const uint4*>(sO + u * RS + 8 * pv);
            }
            if (which < 2 && group > 1) {
                // whole regions in this (only) slice: the means directly
                for (int item = tid; item < nreg * C; item += kThreads) {
                    const int rr = item / C, c = item - rr * C;
                    double sum = 0.0;
                    for (int u = rr * p.t; u < (rr + 1) * p.t; ++u)
                        sum += static_cast<double>(bf16_to_f32(sO[u * RS + c]));
                    const int h = c / kHeadDim, d = c - h * kHeadDim, bh = b * p.heads + h;
                    means[which == 0 ? qmean_index(p, bh, r0 + rr, d)
                                     : kmean_index(p, bh, d, r0 + rr)] = mean_of(sum, p.t);
                }
            } else if (which < 2) {
                // one region in slices: thread (part, c) sums tokens part,
                // part + P, ... of the slice (P = kThreads / C parts, or 1);
                // the parts meet in LDS and thread c adds them to its total
                const int P = C >= kThreads ? 1 : kThreads / C;
                double* sP = reinterpret_cast<double*>(sX + ST * RS * 2);  // [P][C]
                for (int item = tid; item < P * C; item += kThreads) {
                    const int part = item / C, c = item - part * C;
                    double sum = 0.0;
                    for (int u = part; u < nt; u += P)
                        sum += static_cast<double>(bf16_to_f32(sO[u * RS + c]));
                    sP[part * C + c] = sum;
                }
                __syncthreads();
#pragma unroll
                for (int j = 0; j < kCh; ++j) {
                    const int c = tid + j * kThreads;
                    if (c < C) {
                        double sum = 0.0;
                        for (int part = 0; part < P; ++part) sum += sP[part * C + c];
                        if (which == 0)
                            qsum[j] += sum;
                        else
                            ksum[j] += sum;
                    }
                }
            }
            __syncthreads();  // sO is rewritten by the next of q, k, v
        }
    }
    if (group == 1) {
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int c = tid + j * kThreads;
            if (c < C) {
                const int h = c / kHeadDim, d = c - h * kHeadDim, bh = b * p.heads + h;
                means[qmean_index(p, bh, r0, d)] = mean_of(qsum[j], p.t);
                means[kmean_index(p, bh, d, r0)] = mean_of(ksum[j], p.t);
            }
        }
    }
}

}  // namespace

int proj_qkv_lds_bytes(const Params& p) {
    // two bf16 tiles, then the fp64 partial sums of one region's channels
    const int P = p.C >= kThreads ? 1 : kThreads / p.C;
    return 2 * proj_slice(p.C) * proj_row(p.C) * 2 + P * p.C * 8;
}

hipError_t launch_proj_qkv(const Params& p, const void* x, const void* w_qkv,
                           const float* b_qkv, void* qs, void* ks, void* vs, double* means,
                           const float* lepe_w, uint2* lepe_table, hipStream_t stream) {
    Params pp = p;
    if (!lepe_w) pp.table_items = 0;
    const int group = proj_group(p.C, p.t);
    const int gpi = (p.R + group - 1) / group;
    const int table_blocks = (pp.table_items + kThreads - 1) / kThreads;
    const dim3 grid(p.B * gpi + table_blocks), block(kThreads);
    const int lds = proj_qkv_lds_bytes(p);
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    const uint16_t* ww = static_cast<const uint16_t*>(w_qkv);
    uint16_t* q = static_cast<uint16_t*>(qs);
    uint16_t* k = static_cast<uint16_t*>(ks);
    uint16_t* v = static_cast<uint16_t*>(vs);
#define BRA_PROJ(T, HS, WS, NW, HEADS, KTOP)                                                    \
    if constexpr (sizeof(T) == 2) {                                                            \
        if (matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, true, false)) {                  \
            hipLaunchKernelGGL((proj_qkv_kernel<HS, WS, NW, HEADS>), grid, block, lds, stream, \
                               xx, ww, b_qkv, q, k, v, means, lepe_w, lepe_table, pp);         \
            return hipGetLastError();                                                          \
        }                                                                                      \
    }
    BRA_FOR_EACH_SHAPE(BRA_PROJ)
#undef BRA_PROJ
    hipLaunchKernelGGL((proj_qkv_kernel<0, 0, 0, 0>), grid, block, lds, stream, xx, ww, b_qkv, q,
                       k, v, means, lepe_w, lepe_table, pp);
    return hipGetLastError();
}

}  // namespace bra
