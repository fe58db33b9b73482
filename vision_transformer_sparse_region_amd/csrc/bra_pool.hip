// bra_pool.hip -- region means of Q and K (fp64) for the routing, and the
// Toeplitz operand table of the MFMA LePE.  [P4 §1.2; P2 §2.1; P5 §五 ③]
// (page keys in bra_device.h)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_shapes.h"

namespace bra {
namespace {

// x plus the x of lane l ^ M, in VALU registers: DPP row permutations for
// M = 4 and 8, v_permlane16/32_swap for M = 16 and 32.  (The pool sums are
// exact, so the order of the two terms is immaterial.)
template <int M>
__device__ __forceinline__ double xor_sum(double x) {
    const u32x2_t u = __builtin_bit_cast(u32x2_t, x);
    if constexpr (M == 16 || M == 32) {
        const auto a = M == 16 ? __builtin_amdgcn_permlane16_swap(u.x, u.x, false, false)
                               : __builtin_amdgcn_permlane32_swap(u.x, u.x, false, false);
        const auto b = M == 16 ? __builtin_amdgcn_permlane16_swap(u.y, u.y, false, false)
                               : __builtin_amdgcn_permlane32_swap(u.y, u.y, false, false);
        return __builtin_bit_cast(double, u32x2_t{a[0], b[0]}) +
               __builtin_bit_cast(double, u32x2_t{a[1], b[1]});
    } else {
        const int lo = lane_xor_dpp<M>(static_cast<int>(u.x));
        const int hi = lane_xor_dpp<M>(static_cast<int>(u.y));
        return x + __builtin_bit_cast(double, u32x2_t{static_cast<unsigned>(lo),
                                                       static_cast<unsigned>(hi)});
    }
}

// Sum over the lanes that share l % nvec (nvec = 4, 8, 16, 32 or 64).
__device__ __forceinline__ void token_group_sum(double (&acc)[8], int nvec) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (nvec <= 4) acc[e] = xor_sum<4>(acc[e]);
        if (nvec <= 8) acc[e] = xor_sum<8>(acc[e]);
        if (nvec <= 16) acc[e] = xor_sum<16>(acc[e]);
        if (nvec <= 32) acc[e] = xor_sum<32>(acc[e]);
    }
}

// ---------------------------------------------------------------------------
// Region means of Q and K (fp64); of K alone when the attention kernel sums
// the Q means itself (p.qmean_attend).
//  bf16, C/8 dividing 64: one wave per (region, tensor).  Lane (pv, tg) holds
//        fp64 sums of channels 8pv..8pv+7 over every (64/(C/8))-th token of the
//        window; the lanes of one pv are then combined with shuffles.  Within
//        the span condition of row16_sum_exact (bra_device.h) every partial
//        sum is an exact fp64 number: the order of the additions cannot
//        change the result, and the mean is the slot-order mean.
//  otherwise (fp32, or other channel counts): one thread per channel sums
//        the tokens in slot order -- the order of a plain loop -- staged
//        through LDS in chunks.
template <typename T, int HS, int WS, int NW, int HEADS>
__global__ __launch_bounds__(kThreads) void pool_qk_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           double* __restrict__ means,
                                                           const float* __restrict__ lepe_w,
                                                           uint2* __restrict__ lepe_table,
                                                           Params p_in) {
    constexpr int VEC = Elem<T>::kVec;
    const Params p = fold_geometry<HS, WS, NW, HEADS, 1, VEC>(p_in);
    const int tid = threadIdx.x;
    if (static_cast<int>(blockIdx.x) >= p.pool_blocks) {
        // Trailing workgroups: the Toeplitz LePE operands of the MFMA LePE.
        const int it = (blockIdx.x - p.pool_blocks) * kThreads + tid;
        if (it < p.table_items) lepe_table[it] = lepe_table_entry(lepe_w, it);
        return;
    }
    const int nvec = p.C / VEC;

    if (VEC == 8 && 64 % nvec == 0) {
        // Q and K: two regions per workgroup, wave w -> region 2*blk + (w >> 1),
        // tensor w & 1; K alone: four regions, wave w -> region 4*blk + w
        const int lane = tid & 63, w = tid >> 6;
        const int blk = xcd_logical_block(blockIdx.x, p.pool_blocks);
        const int region = p.qmean_attend ? kWaves * blk + w : 2 * blk + (w >> 1);
        if (region >= p.B * p.R) return;
        const int b = region / p.R, r = region - b * p.R;
        const int tensor = p.qmean_attend ? 1 : w & 1;
        const T* src = (tensor == 0 ? q : k) + static_cast<size_t>(b) * p.H * p.W * p.C;
        const int pv = lane % nvec, tg = lane / nvec, TG = 64 / nvec;
        double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
        for (int slot = tg; slot < p.t; slot += TG) {
            const uint4 u =
                *reinterpret_cast<const uint4*>(src + token_offset(p, r, slot) + pv * VEC);
            acc[0] += bf16lo(u.x); acc[1] += bf16hi(u.x);
            acc[2] += bf16lo(u.y); acc[3] += bf16hi(u.y);
            acc[4] += bf16lo(u.z); acc[5] += bf16hi(u.z);
            acc[6] += bf16lo(u.w); acc[7] += bf16hi(u.w);
        }
        token_group_sum(acc, nvec);
        // every lane of a channel piece now holds the piece's sums
        const int c = pv * 8, h = c / kHeadDim, d = c - h * kHeadDim;
        const int bh = b * p.heads + h;
        if (tensor == 0) {
            if (tg == 0) {
                double* dst = means + qmean_index(p, bh, r, d);
#pragma unroll
                for (int e = 0; e < 8; e += 2)
                    *reinterpret_cast<double2*>(dst + e) =
                        double2{mean_of(acc[e], p.t), mean_of(acc[e + 1], p.t)};
            }
        } else {
            // K: lane tg of the piece stores dim pair tg (pairs tg, tg + TG,
            // .. when fewer than 4 lanes share the piece), the pair picked by
            // selects rather than a dynamic register index
            for (int j = tg; j < 4; j += TG) {
                double m0 = acc[0], m1 = acc[1];
#pragma unroll
                for (int e = 2; e < 8; e += 2)
                    if (j == e / 2) {
                        m0 = acc[e];
                        m1 = acc[e + 1];
                    }
                store_kmean_pair(p, means, bh, d + 2 * j, r, mean_of(m0, p.t), mean_of(m1, p.t));
            }
        }
        return;
    }

    extern __shared__ __align__(16) unsigned char smem[];
    T* tile = reinterpret_cast<T*>(smem);
    const int blk = xcd_logical_block(blockIdx.x, p.pool_blocks);
    const int b = blk / p.R, r = blk - b * p.R;
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C;
    for (int tensor = p.qmean_attend ? 1 : 0; tensor < 2; ++tensor) {
        const T* src = (tensor == 0 ? q : k) + img;
        double acc[kMaxChannels / kThreads] = {};
        for (int t0 = 0; t0 < p.t; t0 += p.pool_chunk) {
            const int nt = min(p.pool_chunk, p.t - t0);
            for (int i = tid; i < nt * nvec; i += kThreads) {
                const int tt = i / nvec, pv = i - tt * nvec;
                *reinterpret_cast<uint4*>(tile + tt * p.C + pv * VEC) =
                    *reinterpret_cast<const uint4*>(src + token_offset(p, r, t0 + tt) + pv * VEC);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kMaxChannels / kThreads; ++j) {
                const int c = tid + j * kThreads;
                if (c < p.C) {
                    double s = acc[j];
                    for (int tt = 0; tt < nt; ++tt)
                        s += static_cast<double>(Elem<T>::f32(tile[tt * p.C + c]));
                    acc[j] = s;
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < kMaxChannels / kThreads; ++j) {
            const int c = tid + j * kThreads;
            if (c < p.C) {
                const int h = c / kHeadDim, d = c - h * kHeadDim;
                const int bh = b * p.heads + h;
                if (tensor == 0)
                    means[qmean_index(p, bh, r, d)] = mean_of(acc[j], p.t);
                else
                    store_kmean(p, means, bh, d, r, mean_of(acc[j], p.t));
            }
        }
    }
}

}  // namespace

namespace {
__global__ __launch_bounds__(kThreads) void lepe_table_kernel(const float* __restrict__ lepe_w,
                                                              uint2* __restrict__ lepe_table,
                                                              int items) {
    const int it = blockIdx.x * kThreads + threadIdx.x;
    if (it < items) lepe_table[it] = lepe_table_entry(lepe_w, it);
}
}  // namespace

// ---------------------------------------------------------------------------
// KV downsampling [P1 §4.1 kv_downsample_ratio, avgpool]: one thread per
// (tensor, image, pooled token, VEC-channel piece) sums the kv_ratio^2 input
// tokens of its block in fp32 (block row-major), scales by 1/kv_ratio^2 and
// rounds once to the I/O type.  Reads K and V once, writes 2/kv_ratio^2 of
// them.
namespace {
template <typename T>
__global__ __launch_bounds__(kThreads) void kv_pool_kernel(const T* __restrict__ k,
                                                           const T* __restrict__ v,
                                                           T* __restrict__ kd,
                                                           T* __restrict__ vd, Params p) {
    constexpr int VEC = Elem<T>::kVec;
    const int nvec = p.C / VEC;
    const long per = static_cast<long>(p.B) * p.kH * p.kW * nvec;  // pieces per tensor
    const long it = static_cast<long>(blockIdx.x) * kThreads + threadIdx.x;
    if (it >= 2 * per) return;
    const int tensor = it >= per;
    const long i = it - tensor * per;
    const int pv = static_cast<int>(i % nvec);
    const long cell = i / nvec;
    const int xd = static_cast<int>(cell % p.kW);
    const long rest = cell / p.kW;
    const int yd = static_cast<int>(rest % p.kH), b = static_cast<int>(rest / p.kH);
    const T* src = (tensor ? v : k) + static_cast<size_t>(b) * p.H * p.W * p.C + pv * VEC;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    for (int u = 0; u < p.kv_ratio; ++u)
        for (int w = 0; w < p.kv_ratio; ++w) {
            const size_t tok = static_cast<size_t>(yd * p.kv_ratio + u) * p.W +
                               (xd * p.kv_ratio + w);
            const uint4 x = *reinterpret_cast<const uint4*>(src + tok * p.C);
            if constexpr (VEC == 8) {
                acc[0] += bf16lo(x.x); acc[1] += bf16hi(x.x);
                acc[2] += bf16lo(x.y); acc[3] += bf16hi(x.y);
                acc[4] += bf16lo(x.z); acc[5] += bf16hi(x.z);
                acc[6] += bf16lo(x.w); acc[7] += bf16hi(x.w);
            } else {
                acc[0] += __uint_as_float(x.x); acc[1] += __uint_as_float(x.y);
                acc[2] += __uint_as_float(x.z); acc[3] += __uint_as_float(x.w);
            }
        }
    const float inv = 1.0f / static_cast<float>(p.kv_ratio * p.kv_ratio);
    T* dst = (tensor ? vd : kd) + static_cast<size_t>(cell) * p.C + pv * VEC;
    uint4 o;
    if constexpr (VEC == 8) {
        o.x = f32_to_bf16(acc[0] * inv) | (f32_to_bf16(acc[1] * inv) << 16);
        o.y = f32_to_bf16(acc[2] * inv) | (f32_to_bf16(acc[3] * inv) << 16);
        o.z = f32_to_bf16(acc[4] * inv) | (f32_to_bf16(acc[5] * inv) << 16);
        o.w = f32_to_bf16(acc[6] * inv) | (f32_to_bf16(acc[7] * inv) << 16);
    } else {
        o = uint4{__float_as_uint(acc[0] * inv), __float_as_uint(acc[1] * inv),
                  __float_as_uint(acc[2] * inv), __float_as_uint(acc[3] * inv)};
    }
    *reinterpret_cast<uint4*>(dst) = o;
}
}  // namespace

hipError_t launch_kv_pool(const Params& p, bool bf16, const void* k, const void* v, void* kd,
                          void* vd, hipStream_t stream) {
    const long per = static_cast<long>(p.B) * p.kH * p.kW * (p.C / (bf16 ? 8 : 4));
    const dim3 grid(static_cast<unsigned>((2 * per + kThreads - 1) / kThreads)), block(kThreads);
    if (bf16)
        hipLaunchKernelGGL(kv_pool_kernel<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                           static_cast<uint16_t*>(kd), static_cast<uint16_t*>(vd), p);
    else
        hipLaunchKernelGGL(kv_pool_kernel<float>, grid, block, 0, stream,
                           static_cast<const float*>(k), static_cast<const float*>(v),
                           static_cast<float*>(kd), static_cast<float*>(vd), p);
    return hipGetLastError();
}

hipError_t launch_lepe_table(const Params& p, const float* lepe_w, uint2* lepe_table,
                             hipStream_t stream) {
    if (p.table_items <= 0) return hipSuccess;
    const dim3 grid((p.table_items + kThreads - 1) / kThreads), block(kThreads);
    hipLaunchKernelGGL(lepe_table_kernel, grid, block, 0, stream, lepe_w, lepe_table,
                       p.table_items);
    return hipGetLastError();
}

hipError_t launch_pool_qk(const Params& p, bool bf16, const void* q, const void* k,
                          const float* lepe_w, double* means, uint2* lepe_table,
                          hipStream_t stream) {
    const int nvec = p.C / (bf16 ? 8 : 4);
    const bool wave_path = bf16 && 64 % nvec == 0;
    Params pp = p;
    if (!lepe_w) pp.table_items = 0;
    const int table_blocks = (pp.table_items + kThreads - 1) / kThreads;
    const dim3 grid(p.pool_blocks + table_blocks), block(kThreads);
    const int lds = wave_path ? 0 : p.pool_lds_bytes;
#define BRA_POOL(T, HS, WS, NW, HEADS, KTOP)                                                    \
    if (matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, false)) {                      \
        hipLaunchKernelGGL((pool_qk_kernel<T, HS, WS, NW, HEADS>), grid, block, lds, stream,   \
                           static_cast<const T*>(q), static_cast<const T*>(k), means, lepe_w,  \
                           lepe_table, pp);                                                    \
        return hipGetLastError();                                                              \
    }
    BRA_FOR_EACH_SHAPE(BRA_POOL)
#undef BRA_POOL
    if (bf16)
        hipLaunchKernelGGL((pool_qk_kernel<uint16_t, 0, 0, 0, 0>), grid, block, lds, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           means, lepe_w, lepe_table, pp);
    else
        hipLaunchKernelGGL((pool_qk_kernel<float, 0, 0, 0, 0>), grid, block, lds, stream,
                           static_cast<const float*>(q), static_cast<const float*>(k), means,
                           lepe_w, lepe_table, pp);
    return hipGetLastError();
}

}  // namespace bra
