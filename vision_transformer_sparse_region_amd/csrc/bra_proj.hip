// bra_proj.hip -- the qkv projection before the path [P5 §五 ① qkv =
// Linear(dim, 3*dim); P4 §1.1], on MFMA, with the region means of the
// projected Q and K in its epilogue (page keys in bra_device.h).
//
// One workgroup per (image, region).  For each 16-token tile of the region
// and each 16-channel tile of the 3C outputs,
//   D^T = W[o0 .. o0+15, :] . X^T          (v_mfma_f32_16x16x32_bf16, fp32 sums)
// where operand A row m is output channel o0 + m (16 contiguous bytes of the
// PyTorch Linear weight [3C, C] per lane and 32-channel step) and operand B
// column n is token n of the tile (16 contiguous bytes of x per lane).  Lane
// (n, g) receives output channels o0 + 4g .. o0 + 4g + 3 of token n; adding
// the bias and rounding once to bf16 gives q, k or v as the module's Linear
// layer would produce them.  The rounded q and k values are also summed in
// fp64 over the region's tokens: every partial sum of bf16 values is exact,
// so these region means equal those of the pool kernel over the stored q and
// k, bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_shapes.h"

namespace bra {
namespace {

template <int HS, int WS, int NW, int HEADS>
__global__ __launch_bounds__(kThreads) void proj_qkv_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_qkv,
    const float* __restrict__ b_qkv, uint16_t* __restrict__ qs, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ vs, double* __restrict__ means, const float* __restrict__ lepe_w,
    uint2* __restrict__ lepe_table, Params p_in) {
    const Params p = fold_geometry<HS, WS, NW, HEADS, 1, 8>(p_in);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (static_cast<int>(blockIdx.x) >= p.B * p.R) {
        // trailing workgroups: the Toeplitz operands of the MFMA LePE
        const int it = (blockIdx.x - p.B * p.R) * kThreads + tid;
        if (it < p.table_items) lepe_table[it] = lepe_toeplitz_entry(lepe_w, it);
        return;
    }
    const int blk = xcd_logical_block(blockIdx.x, p.B * p.R);
    const int b = blk / p.R, r = blk - b * p.R;
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C;
    const int C = p.C, ksteps = C / 32, otiles = 3 * C / 16, ttiles = (p.t + 15) / 16;
    const int n = lane & 15, g = lane >> 4;

    // wave wu owns output tiles wu, wu + 4, ... (a tile never straddles q,
    // k and v: C is a multiple of 32); per tile, fp64 sums of its 4 channels
    // over the region's tokens (q and k tiles only)
    for (int ot = wu; ot < otiles; ot += kWaves) {
        const int o0 = ot * 16;
        const int which = o0 / C, c0 = o0 - which * C;  // 0 q, 1 k, 2 v; channel in C
        uint16_t* dst = which == 0 ? qs : which == 1 ? ks : vs;
        float bias[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bias[i] = b_qkv ? b_qkv[o0 + 4 * g + i] : 0.f;
        double sum[4] = {0.0, 0.0, 0.0, 0.0};
        for (int tt = 0; tt < ttiles; ++tt) {
            const int tok = tt * 16 + n;
            const bool live = tok < p.t;
            const int toff = token_offset(p, r, min(tok, p.t - 1));
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < ksteps; ++s) {
                const uint4 a = *reinterpret_cast<const uint4*>(
                    w_qkv + static_cast<size_t>(o0 + n) * C + 32 * s + 8 * g);
                const uint4 xb =
                    *reinterpret_cast<const uint4*>(x + img + toff + 32 * s + 8 * g);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, xb), acc, 0, 0,
                    0);
            }
            // lane (n, g): channels c0 + 4g + i of token tok
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[i] = f32_to_bf16(acc[i] + bias[i]);
                if (live && which < 2) sum[i] += static_cast<double>(bf16_to_f32(h[i]));
            }
            if (live)
                *reinterpret_cast<uint2*>(dst + img + toff + c0 + 4 * g) =
                    uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        }
        if (which < 2) {
            // sum over the 16 token lanes of each row: exact, any pairing
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[i] = row16_sum_exact(sum[i]);
            if (n == 0) {
                const int c = c0 + 4 * g, h = c / kHeadDim, d = c - h * kHeadDim;
                const int bh = b * p.heads + h;
                if (which == 0) {
                    double* qd = means + qmean_index(p, bh, r, d);
                    *reinterpret_cast<double2*>(qd) =
                        double2{mean_of(sum[0], p.t), mean_of(sum[1], p.t)};
                    *reinterpret_cast<double2*>(qd + 2) =
                        double2{mean_of(sum[2], p.t), mean_of(sum[3], p.t)};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        means[kmean_index(p, bh, d + i, r)] = mean_of(sum[i], p.t);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_proj_qkv(const Params& p, const void* x, const void* w_qkv,
                           const float* b_qkv, void* qs, void* ks, void* vs, double* means,
                           const float* lepe_w, uint2* lepe_table, hipStream_t stream) {
    Params pp = p;
    if (!lepe_w) pp.table_items = 0;
    const int table_blocks = (pp.table_items + kThreads - 1) / kThreads;
    const dim3 grid(p.B * p.R + table_blocks), block(kThreads);
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    const uint16_t* ww = static_cast<const uint16_t*>(w_qkv);
    uint16_t* q = static_cast<uint16_t*>(qs);
    uint16_t* k = static_cast<uint16_t*>(ks);
    uint16_t* v = static_cast<uint16_t*>(vs);
#define BRA_PROJ(T, HS, WS, NW, HEADS, KTOP)                                                  \
    if constexpr (sizeof(T) == 2) {                                                          \
        if (matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, true, false)) {                \
            hipLaunchKernelGGL((proj_qkv_kernel<HS, WS, NW, HEADS>), grid, block, 0, stream, \
                               xx, ww, b_qkv, q, k, v, means, lepe_w, lepe_table, pp);       \
            return hipGetLastError();                                                        \
        }                                                                                    \
    }
    BRA_FOR_EACH_SHAPE(BRA_PROJ)
#undef BRA_PROJ
    hipLaunchKernelGGL((proj_qkv_kernel<0, 0, 0, 0>), grid, block, 0, stream, xx, ww, b_qkv, q,
                       k, v, means, lepe_w, lepe_table, pp);
    return hipGetLastError();
}

}  // namespace bra
