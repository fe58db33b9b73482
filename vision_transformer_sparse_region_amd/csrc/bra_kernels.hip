// bra_kernels.hip -- HIP kernels (gfx950) of the Bi-Level Routing Attention
// forward pass.
//
// Pages cited by key:
//   [P1] "从静态到动态：Bi-Level Routing Attention如何重塑视觉Transformer的注意力机制",
//        www.mhpn.cn/news/199372
//   [P2] "BiFormer用双层路由注意力重塑视觉Transformer效率极限", www.mooersco.com/news/894234
//   [P3] "从零构建BiFormer：PyTorch实战双层路由注意力机制与调试全攻略",
//        www.mhpn.cn/news/564882
//   [P4] "手把手解析BiFormer：双水平路由注意力机制与PyTorch实战指南", www.jsqmd.com/news/719213
//   [P5] "【医学图像分割模块】BiFormer / 双层路由注意力（CVPR 2023）", www.mhpn.cn/news/2512273
//
// Two launches per forward:
//   pool_k_kernel        one workgroup per (image, region): fp64 mean of K over
//                        the region's window, per channel            [P4 §1.2; P5 §五 ③]
//   route_attend_kernel  one workgroup per (image, region), all heads:
//     1    stage the Q window and the V window + 2-token halo in LDS
//     2-4  fp64 Q mean, fp64 affinity against every K mean, rank-based
//          top-k with ties to the lower id                     [P1 §2.1; P5 §五 ③-④]
//     5    each wave issues the gather of its first routed K/V chunk ...
//     6    ... and computes the 5x5 depthwise LePE of V from the LDS halo
//          while those loads are in flight                    [P5 §五 lepe, ⑧; P2 §2.2]
//     7    token attention over the routed tokens: S^T = K Q^T and
//          O^T += V^T P^T on bf16 MFMA, fp32 online softmax, the next chunk's
//          gather in flight during each chunk                 [P3 §2.2; P5 §五 ⑤-⑦]
//     8    out = LePE + O, one rounding, 16-byte NHWC stores
// The routed K/V tokens are never copied to HBM: [P3 §4.2] and [P1 §2.2]
// build a dense k-fold gathered tensor with torch.gather; here the routing
// index drives the loads straight into MFMA operands.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bra_launch.h"

namespace bra {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int kVec = 4;  // elements per 16-byte piece
    __device__ static float f32(float x) { return x; }
    // two consecutive channels
    __device__ static float2 pair(const float* p) { return *reinterpret_cast<const float2*>(p); }
};
template <>
struct Elem<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static float f32(uint16_t x) { return bf16_to_f32(x); }
    __device__ static float2 pair(const uint16_t* p) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
        return float2{bf16lo(u), bf16hi(u)};
    }
};

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap so that consecutive logical ids -- the regions of one image --
// run on one XCD and share its L2 for the routed K/V and halo reads.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
    const int full = nblocks & ~7;
    if (bid >= full) return bid;
    return (bid & 7) * (full >> 3) + (bid >> 3);
}

// Max and sum over the four lanes l, l^16, l^32, l^48 -- in the MFMA
// attention these hold the four key groups of one query.  v_permlane16_swap
// and v_permlane32_swap exchange rows of 16 and halves of 32 lanes in VALU
// registers, without a trip through the LDS crossbar; every lane of the four
// ends with the same value.
__device__ __forceinline__ float group4_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// mean = sum / t, as a multiplication when t is a power of two (exact then).
__device__ __forceinline__ double mean_of(double sum, int t) {
    return (t & (t - 1)) == 0 ? sum * (1.0 / static_cast<double>(t)) : sum / static_cast<double>(t);
}

// Token offset (elements) of slot `slot` of region `reg` inside one image.
__device__ __forceinline__ int token_offset(const Params& p, int reg, int slot) {
    const int ri = reg / p.n, rj = reg - ri * p.n;
    const int u = slot / p.ws, w = slot - u * p.ws;
    return ((ri * p.hs + u) * p.W + rj * p.ws + w) * p.C;
}

// Window geometry as compile-time constants.  A kernel instantiated with
// nonzero HS, WS, NW, HEADS, KTOP replaces the matching runtime fields (the
// host launches such an instance only for exactly that shape), so divisions
// and loop bounds fold; zeros keep the runtime values.
template <int HS, int WS, int NW, int HEADS, int KTOP, int VEC>
__device__ __forceinline__ Params fold_geometry(const Params& in) {
    Params p = in;
    if constexpr (HS > 0) p.hs = HS;
    if constexpr (WS > 0) p.ws = WS;
    if constexpr (NW > 0) {
        p.n = NW;
        p.R = NW * NW;
    }
    if constexpr (HEADS > 0) {
        p.heads = HEADS;
        p.C = HEADS * kHeadDim;
        p.lstride = HEADS * kHeadDim + 4;
    }
    if constexpr (HS > 0 && WS > 0 && NW > 0 && HEADS > 0 && KTOP > 0) {
        p.H = NW * HS;
        p.W = NW * WS;
        p.t = HS * WS;
        p.k = KTOP;
        p.nkeys = KTOP * HS * WS;
        p.lepe_items = (HEADS * kHeadDim / 2) * HS * ((WS + kLepeCols - 1) / kLepeCols);
        p.lepe_alias = p.lepe_items <= kThreads;
        p.halo_pieces = (HS + 4) * (WS + 4) * (HEADS * kHeadDim / VEC);
    }
    return p;
}

// One entry of the Toeplitz operand table of the MFMA LePE (see
// lepe_mfma_compute): entry it = ((cg * 64 + lane) * 5 + i) * 2 + ks holds the
// B operand of lane `lane` for channel group cg, tap row i and column step ks:
// four bf16 w[c][i][4ks + kk - n] (zero outside 0..4), c = 16cg + lane/4,
// n = lane % 4.
__device__ __forceinline__ uint2 lepe_toeplitz_entry(const float* __restrict__ lepe_w, int it) {
    const int ks = it & 1, i = (it >> 1) % 5, lane_cg = it / 10;
    const int lane = lane_cg & 63, cg = lane_cg >> 6;
    const int c = 16 * cg + (lane >> 2), n = lane & 3;
    uint32_t h[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int j = 4 * ks + kk - n;
        h[kk] = (j >= 0 && j <= 4) ? f32_to_bf16(lepe_w[c * 25 + i * 5 + j]) : 0u;
    }
    return uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// ---------------------------------------------------------------------------
// Region means of Q and K (fp64).
//  bf16, C/8 dividing 64: one wave per (region, tensor).  Lane (pv, tg) holds
//        fp64 sums of channels 8pv..8pv+7 over every (64/(C/8))-th token of the
//        window; the lanes of one pv are then combined with shuffles.  A bf16
//        value has an 8-bit significand, so every partial sum of a window is an
//        exact fp64 number: the order of the additions cannot change the
//        result, and the mean is the correctly rounded exact mean.
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
        if (it < p.table_items) lepe_table[it] = lepe_toeplitz_entry(lepe_w, it);
        return;
    }
    const size_t mstride = static_cast<size_t>(p.B) * p.heads * p.R * kHeadDim;
    const int nvec = p.C / VEC;

    if (VEC == 8 && 64 % nvec == 0) {
        // two regions per workgroup: wave w -> region 2*blk + (w >> 1), tensor w & 1
        const int lane = tid & 63, w = tid >> 6;
        const int blk = xcd_logical_block(blockIdx.x, p.pool_blocks);
        const int region = 2 * blk + (w >> 1);
        if (region >= p.B * p.R) return;
        const int b = region / p.R, r = region - b * p.R;
        const int tensor = w & 1;
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
        for (int m = nvec; m < 64; m *= 2)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], m);
        if (tg == 0) {
            const int c = pv * 8, h = c / kHeadDim, d = c - h * kHeadDim;
            double* dst = means + tensor * mstride +
                          ((static_cast<size_t>(b) * p.heads + h) * p.R + r) * kHeadDim + d;
#pragma unroll
            for (int e = 0; e < 8; e += 2)
                *reinterpret_cast<double2*>(dst + e) =
                    double2{mean_of(acc[e], p.t), mean_of(acc[e + 1], p.t)};
        }
        return;
    }

    extern __shared__ __align__(16) unsigned char smem[];
    T* tile = reinterpret_cast<T*>(smem);
    const int blk = xcd_logical_block(blockIdx.x, p.pool_blocks);
    const int b = blk / p.R, r = blk - b * p.R;
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C;
    double* mimg = means + static_cast<size_t>(b) * p.heads * p.R * kHeadDim;
    for (int tensor = 0; tensor < 2; ++tensor) {
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
                mimg[tensor * mstride + (static_cast<size_t>(h) * p.R + r) * kHeadDim + d] =
                    mean_of(acc[j], p.t);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA token attention.
//
// A wave owns "jobs": one head and up to kMaxQTiles tiles of 16 query tokens.
// Keys stream in chunks of 32; the wave's (job, chunk) steps are flattened so
// that the gather of step s+1 is in flight while step s computes.  For a
// chunk, two v_mfma_f32_16x16x32_bf16 give S^T (keys x queries): operand A
// row i (lane & 15) is the key 32c + 8*(i/4) + 4*blk + i%4, so that output
// lane (query li, group g = lane/16) holds the scores of the 8 consecutive
// keys 32c + 8g .. 32c + 8g + 7.  Those 8 probabilities are exactly that
// lane's B operand of O^T += V^T P^T (k-slot 8g + e = key 32c + 8g + e), so P
// never leaves registers; V^T is read transposed from a per-wave LDS buffer.
// O^T lands with the query on lane & 15 like the scores, so the online-softmax
// rescale is lane-local.
struct WaveJobs {
    int QT, G, tpg, njobs, nchunks, nsteps;
    __device__ __forceinline__ WaveJobs(const Params& p, int w) {
        QT = (p.t + 15) / 16;
        const int wph = max(1, kWaves / p.heads);
        const int g0 = max(min(wph, QT), (QT + kMaxQTiles - 1) / kMaxQTiles);
        tpg = (QT + g0 - 1) / g0;
        G = (QT + tpg - 1) / tpg;  // every group non-empty
        njobs = p.heads * G;
        nchunks = (p.nkeys + 31) / 32;
        const int mine = w < njobs ? (njobs - 1 - w) / kWaves + 1 : 0;
        nsteps = mine * nchunks;
    }
};

// Registers of one (job, chunk) step: the two K^T operands (16 B per lane)
// and this lane's two 16-byte pieces of the 32-key x 32-dim V chunk.
struct StepRegs {
    bf16x8_t ka[2];
    uint4 vv[2];
};

// Q^T operands of a job: lane (query li, group g) holds dims 8g..8g+7 of
// query (qt0 + jq) * 16 + li of head h (zero past the window).
__device__ __forceinline__ void load_q_operands(const Params& p, const WaveJobs& J, int job,
                                                const uint16_t* __restrict__ qimg, int r,
                                                bf16x8_t (&qb)[kMaxQTiles]) {
    const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
    const int h = job / J.G, grp = job - h * J.G;
    const int qt0 = grp * J.tpg;
    const int nq = min(J.tpg, J.QT - qt0);
#pragma unroll
    for (int jq = 0; jq < kMaxQTiles; ++jq) {
        const int qi = (qt0 + jq) * 16 + li;
        uint4 u = {0u, 0u, 0u, 0u};
        if (jq < nq && qi < p.t)
            u = *reinterpret_cast<const uint4*>(qimg + token_offset(p, r, qi) + h * kHeadDim +
                                                8 * g);
        qb[jq] = __builtin_bit_cast(bf16x8_t, u);
    }
}

__device__ __forceinline__ void gather_step(const Params& p, const WaveJobs& J, int w, int step,
                                            const uint16_t* __restrict__ kimg,
                                            const uint16_t* __restrict__ vimg, const int* sIdx,
                                            StepRegs& g8) {
    const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
    const int jl = step / J.nchunks, c = step - jl * J.nchunks;
    const int job = w + kWaves * jl;
    const int h = job / J.G;
    const int hoff = h * kHeadDim;
    const int* idx = sIdx + h * p.k;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int key = 32 * c + 8 * (li >> 2) + 4 * blk + (li & 3);
        uint4 u = {0u, 0u, 0u, 0u};
        if (key < p.nkeys) {
            const int j = key / p.t, slot = key - j * p.t;
            u = *reinterpret_cast<const uint4*>(kimg + token_offset(p, idx[j], slot) + hoff +
                                                8 * g);
        }
        g8.ka[blk] = __builtin_bit_cast(bf16x8_t, u);
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        const int pc = lane + 64 * pp;
        const int key = 32 * c + (pc >> 2);
        uint4 u = {0u, 0u, 0u, 0u};
        if (key < p.nkeys) {
            const int j = key / p.t, slot = key - j * p.t;
            u = *reinterpret_cast<const uint4*>(vimg + token_offset(p, idx[j], slot) + hoff +
                                                8 * (pc & 3));
        }
        g8.vv[pp] = u;
    }
}

__device__ __forceinline__ void attend_mfma(const Params& p, const WaveJobs& J, const uint16_t* __restrict__ qimg,
                            const uint16_t* __restrict__ kimg, const uint16_t* __restrict__ vimg,
                            int r, uint16_t* sVt_all, float* sL, const int* sIdx, StepRegs& cur,
                            bf16x8_t (&qb)[kMaxQTiles]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    uint16_t* sVt = sVt_all + w * 32 * kVtStride;

    float m[kMaxQTiles], l[kMaxQTiles];
    f32x4_t o0[kMaxQTiles], o1[kMaxQTiles];
    for (int s = 0; s < J.nsteps; ++s) {
        const int jl = s / J.nchunks, c = s - jl * J.nchunks;
        const int job = w + kWaves * jl;
        const int h = job / J.G, grp = job - h * J.G;
        const int qt0 = grp * J.tpg;
        const int nq = min(J.tpg, J.QT - qt0);
        const int hoff = h * kHeadDim;
        if (c == 0) {
            // the first job's operands were loaded with its first gather
            if (s > 0) load_q_operands(p, J, job, qimg, r, qb);
#pragma unroll
            for (int jq = 0; jq < kMaxQTiles; ++jq) {
                m[jq] = -INFINITY;
                l[jq] = 0.f;
                o0[jq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                o1[jq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        StepRegs nxt;
        if (s + 1 < J.nsteps) gather_step(p, J, w, s + 1, kimg, vimg, sIdx, nxt);

        // This step's V chunk into the wave's LDS buffer, read back transposed.
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const int pc = lane + 64 * pp;
            uint2* dst = reinterpret_cast<uint2*>(sVt + (pc >> 2) * kVtStride + 8 * (pc & 3));
            dst[0] = uint2{cur.vv[pp].x, cur.vv[pp].y};
            dst[1] = uint2{cur.vv[pp].z, cur.vv[pp].w};
        }
        // A wave's LDS operations complete in order; the fences keep the
        // compiler from moving the transposed reads above the writes.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        bf16x8_t va[2];
#pragma unroll
        for (int db = 0; db < 2; ++db) {
            u16x8_t t8;
#pragma unroll
            for (int e = 0; e < 8; ++e) t8[e] = sVt[(8 * g + e) * kVtStride + li + 16 * db];
            va[db] = __builtin_bit_cast(bf16x8_t, t8);
        }

        const int kbase = 32 * c + 8 * g;
#pragma unroll
        for (int jq = 0; jq < kMaxQTiles; ++jq) {
            if (jq >= nq) break;
            const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t s0 =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.ka[0], qb[jq], z4, 0, 0, 0);
            const f32x4_t s1 =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.ka[1], qb[jq], z4, 0, 0, 0);
            // raw scores; the running max m is kept in raw units and the
            // scale * log2(e) factor enters each exponent through one FMA
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = s0[e];
                x[4 + e] = s1[e];
            }
            if (kbase + 8 > p.nkeys) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (kbase + e >= p.nkeys) x[e] = -INFINITY;
            }
            const float mx = group4_max(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                              fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
            const float mnew = fmaxf(m[jq], mx);
            const float alpha = __builtin_amdgcn_exp2f((m[jq] - mnew) * p.scale_log2e);
            const float mb = mnew * p.scale_log2e;
            float psum = 0.f;
            bf16x8_t pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(x[e], p.scale_log2e, -mb));
                psum += pe;
                pb[e] = static_cast<__bf16>(pe);
            }
            l[jq] = l[jq] * alpha + psum;
            m[jq] = mnew;
            o0[jq] *= alpha;
            o1[jq] *= alpha;
            o0[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[0], pb, o0[jq], 0, 0, 0);
            o1[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[1], pb, o1[jq], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();

        if (c == J.nchunks - 1) {
#pragma unroll
            for (int jq = 0; jq < kMaxQTiles; ++jq) {
                if (jq >= nq) break;
                const float inv = 1.f / group4_sum(l[jq]);
                const int qi = (qt0 + jq) * 16 + li;
                if (qi < p.t) {
                    float* dst = sL + qi * p.lstride + hoff + 4 * g;
                    const f32x4_t a = *reinterpret_cast<f32x4_t*>(dst);
                    const f32x4_t bq = *reinterpret_cast<f32x4_t*>(dst + 16);
                    *reinterpret_cast<f32x4_t*>(dst) = a + o0[jq] * inv;
                    *reinterpret_cast<f32x4_t*>(dst + 16) = bq + o1[jq] * inv;
                }
            }
        }
        if (s + 1 < J.nsteps) cur = nxt;
    }
}

// fp32 VALU token attention: 8 lanes per (query token, head), 4 dims each;
// keys in routed order with an online softmax, the next key's loads in
// flight while the current one is processed; fp32 throughout.
__device__ __forceinline__ void attend_valu(const Params& p, const float* __restrict__ qimg,
                            const float* __restrict__ kimg, const float* __restrict__ vimg, int r,
                            float* sL, const int* sIdx) {
    const int sub = threadIdx.x & 7;
    for (int item = threadIdx.x >> 3; item < p.t * p.heads; item += kThreads / 8) {
        const int h = item / p.t, slot = item - h * p.t;
        const int hoff = h * kHeadDim + 4 * sub;
        const float4 qv = *reinterpret_cast<const float4*>(qimg + token_offset(p, r, slot) + hoff);
        const int* idx = sIdx + h * p.k;
        float m = -INFINITY, l = 0.f;
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        int off = token_offset(p, idx[0], 0) + hoff;
        float4 kv = *reinterpret_cast<const float4*>(kimg + off);
        float4 vv = *reinterpret_cast<const float4*>(vimg + off);
        for (int key = 0; key < p.nkeys; ++key) {
            float4 kn = kv, vn = vv;
            if (key + 1 < p.nkeys) {
                const int j = (key + 1) / p.t, ks = key + 1 - j * p.t;
                const int o2 = token_offset(p, idx[j], ks) + hoff;
                kn = *reinterpret_cast<const float4*>(kimg + o2);
                vn = *reinterpret_cast<const float4*>(vimg + o2);
            }
            float d = qv.x * kv.x + qv.y * kv.y + qv.z * kv.z + qv.w * kv.w;
            d += __shfl_xor(d, 1);
            d += __shfl_xor(d, 2);
            d += __shfl_xor(d, 4);
            const float x = d * p.scale_log2e;
            const float mnew = fmaxf(m, x);
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            const float pe = __builtin_amdgcn_exp2f(x - mnew);
            l = l * alpha + pe;
            m = mnew;
            acc.x = fmaf(pe, vv.x, acc.x * alpha);
            acc.y = fmaf(pe, vv.y, acc.y * alpha);
            acc.z = fmaf(pe, vv.z, acc.z * alpha);
            acc.w = fmaf(pe, vv.w, acc.w * alpha);
            kv = kn;
            vv = vn;
        }
        const float inv = 1.f / l;
        float4* dst = reinterpret_cast<float4*>(sL + slot * p.lstride + hoff);
        const float4 a = *dst;
        *dst = float4{a.x + acc.x * inv, a.y + acc.y * inv, a.z + acc.z * inv, a.w + acc.w * inv};
    }
}

// One LePE work item: channels c0, c0+1 of window row y, columns xs..xs+7
// (fewer at the window's right edge), bias + 25 taps from the LDS halo.
// Weights come from LDS (sW, [C][25] then the bias [C]) or from global memory.
template <typename T>
__device__ __forceinline__ void lepe_item(const Params& p, const T* sVh, const float* wsrc,
                                          const float* bsrc, int c0, int y, int xs, int nx,
                                          float (&acc)[2][kLepeCols]) {
    float b0 = 0.f, b1 = 0.f;
    if (p.has_lepe && bsrc) {
        b0 = bsrc[c0];
        b1 = bsrc[c0 + 1];
    }
#pragma unroll
    for (int x = 0; x < kLepeCols; ++x) {
        acc[0][x] = b0;
        acc[1][x] = b1;
    }
    if (!p.has_lepe) return;
    const int hw = p.ws + 4;
#pragma unroll 1
    for (int i = 0; i < 5; ++i) {
        float w0[5], w1[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            w0[j] = wsrc[c0 * 25 + i * 5 + j];
            w1[j] = wsrc[(c0 + 1) * 25 + i * 5 + j];
        }
        const T* row = sVh + ((y + i) * hw + xs) * p.C + c0;
        float in0[kLepeCols + 4], in1[kLepeCols + 4];
#pragma unroll
        for (int xx = 0; xx < kLepeCols + 4; ++xx) {
            float2 v2 = {0.f, 0.f};
            if (xx < nx + 4) v2 = Elem<T>::pair(row + xx * p.C);
            in0[xx] = v2.x;
            in1[xx] = v2.y;
        }
#pragma unroll
        for (int x = 0; x < kLepeCols; ++x)
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                acc[0][x] = fmaf(w0[j], in0[x + j], acc[0][x]);
                acc[1][x] = fmaf(w1[j], in1[x + j], acc[1][x]);
            }
    }
}

__device__ __forceinline__ void store_lepe(const Params& p, float* sL, int c0, int y, int xs,
                                           int nx, const float (&acc)[2][kLepeCols]) {
#pragma unroll
    for (int x = 0; x < kLepeCols; ++x)
        if (x < nx)
            *reinterpret_cast<float2*>(sL + (y * p.ws + xs + x) * p.lstride + c0) =
                float2{acc[0][x], acc[1][x]};
}

// The whole LePE step: every (channel pair, row, column block) item, written
// to sL.  In alias mode sL overlays the halo, so the items (at most one per
// thread) are computed first and stored after a barrier.  Ends with a barrier.
template <typename T>
__device__ __forceinline__ void lepe_phase(const Params& p, const T* sVh, float* sL, const float* wsrc,
                           const float* bsrc) {
    const int npairs = p.C / 2;
    const int nxb = (p.ws + kLepeCols - 1) / kLepeCols;
    float acc[2][kLepeCols];
    int mine = -1;
    for (int it = threadIdx.x; it < p.lepe_items; it += kThreads) {
        const int cp = it % npairs, rest = it / npairs;
        const int xb = rest % nxb, y = rest / nxb;
        const int xs = xb * kLepeCols, nx = min(kLepeCols, p.ws - xs);
        lepe_item<T>(p, sVh, wsrc, bsrc, 2 * cp, y, xs, nx, acc);
        if (p.lepe_alias)
            mine = it;
        else
            store_lepe(p, sL, 2 * cp, y, xs, nx, acc);
    }
    if (p.lepe_alias) {
        __syncthreads();  // every halo read is done before sL overwrites it
        if (mine >= 0) {
            const int cp = mine % npairs, rest = mine / npairs;
            const int xb = rest % nxb, y = rest / nxb;
            const int xs = xb * kLepeCols;
            store_lepe(p, sL, 2 * cp, y, xs, min(kLepeCols, p.ws - xs), acc);
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// LePE on the 4x4x4 MFMA with 16 independent blocks (bf16, fixed windows whose
// sides are multiples of 4).  The depthwise 5x5 convolution has no channel
// contraction, but v_mfma_f32_4x4x4_16b_bf16 runs 16 separate 4x4x4 products:
// block b is one channel.  For a 4x4 output tile and tap row i,
//   D[m][n] += sum_{k<4} A[m][k] B[k][n],  A[m][k] = V[y0+m+i][x0+4ks+k],
//   B[k][n] = w[i][4ks+k-n] (zero outside 0..4),
// over ks = 0, 1 covers the 8 halo columns a 4-wide tile reads, so ten
// products give all 25 taps.  Lane l is block l/4; it holds A row l%4 (four
// consecutive halo columns of one channel: the halo is staged channel-planar)
// and B / D column l%4.  The Toeplitz B operands depend only on the channel
// and the lane's column: the pool kernel writes them once per forward to a
// small table (lepe_toeplitz_entry).  Weights enter the product as bf16 (the
// accumulation is fp32).
__host__ __device__ constexpr bool lepe_mfma_fits(int hs, int ws, int heads) {
    return hs > 0 && ws > 0 && heads > 0 && hs % 4 == 0 && ws % 4 == 0 &&
           (hs / 4) * (ws / 4) * ((heads * kHeadDim / 16 + kWaves - 1) / kWaves) <= 8;
}

template <int HS, int WS, int HEADS>
struct LepeMfmaShape {
    static constexpr int C = HEADS * kHeadDim;
    static constexpr int TY = HS / 4, TX = WS / 4;
    static constexpr int HWP = WS + 4;                    // halo row pitch (elements)
    static constexpr int PS = (HS + 4) * (WS + 4) + 4;    // channel plane stride (elements)
    static constexpr int NG = C / 16;                     // groups of 16 channels
    static constexpr int GPW = (NG + kWaves - 1) / kWaves;  // groups per wave
    static constexpr bool ok = lepe_mfma_fits(HS, WS, HEADS);
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// The Toeplitz B operands and the bias of this lane's channel in each of the
// wave's channel groups, loaded from the table the pool kernel built.
template <int HS, int WS, int HEADS>
struct LepeOperands {
    uint4 tb[LepeMfmaShape<HS, WS, HEADS>::GPW][5];  // 10 x 8 bytes per group
    float bias[LepeMfmaShape<HS, WS, HEADS>::GPW];
};

template <int HS, int WS, int HEADS>
__device__ __forceinline__ void lepe_mfma_load(const uint2* __restrict__ table,
                                               const float* __restrict__ lepe_b,
                                               LepeOperands<HS, WS, HEADS>& o) {
    using S = LepeMfmaShape<HS, WS, HEADS>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int g = 0; g < S::GPW; ++g) {
        const int cg = w + kWaves * g;
        o.bias[g] = 0.f;
        if (cg < S::NG) {
            const uint4* src = reinterpret_cast<const uint4*>(table + (cg * 64 + lane) * 10);
#pragma unroll
            for (int e = 0; e < 5; ++e) o.tb[g][e] = src[e];
            if (lepe_b) o.bias[g] = lepe_b[16 * cg + (lane >> 2)];
        }
    }
}

template <int HS, int WS, int HEADS>
__device__ __forceinline__ void lepe_mfma_compute(const Params& p, const uint16_t* sVp, float* sL,
                                                  const LepeOperands<HS, WS, HEADS>& o) {
    using S = LepeMfmaShape<HS, WS, HEADS>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int blk = lane >> 2, n = lane & 3;
    f32x4_t dacc[S::GPW][S::TY * S::TX];
#pragma unroll
    for (int g = 0; g < S::GPW; ++g) {
        const int cg = w + kWaves * g;
        if (cg < S::NG) {
            const int c = 16 * cg + blk;
            const uint16_t* plane = sVp + c * S::PS;
#pragma unroll
            for (int ty = 0; ty < S::TY; ++ty)
#pragma unroll
                for (int tx = 0; tx < S::TX; ++tx) {
                    f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 5; ++i)
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            const s16x4_t a = *reinterpret_cast<const s16x4_t*>(
                                plane + (4 * ty + n + i) * S::HWP + 4 * tx + 4 * ks);
                            const uint4 t4 = o.tb[g][i];
                            const uint2 bw = ks == 0 ? uint2{t4.x, t4.y} : uint2{t4.z, t4.w};
                            d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                                a, __builtin_bit_cast(s16x4_t, bw), d, 0, 0, 0);
                        }
                    dacc[g][ty * S::TX + tx] = d;
                }
        }
    }
    __syncthreads();  // every halo read is done; sL overlays the halo
#pragma unroll
    for (int g = 0; g < S::GPW; ++g) {
        const int cg = w + kWaves * g;
        if (cg < S::NG) {
            const int c = 16 * cg + blk;
#pragma unroll
            for (int ty = 0; ty < S::TY; ++ty)
#pragma unroll
                for (int tx = 0; tx < S::TX; ++tx)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sL[((4 * ty + e) * WS + 4 * tx + n) * p.lstride + c] =
                            dacc[g][ty * S::TX + tx][e] + o.bias[g];
        }
    }
    __syncthreads();
}

// Wave-wide arg-max of (value, index) pairs: the larger value wins, an exact
// tie goes to the lower index.  Partners: lane^1 and lane^2 by DPP quad
// permutation, the other quad of 8 lanes by row_half_mirror, the other half of
// 16 by row_mirror (every lane of a group holds the group's winner by then,
// so any cross pairing works), then rows of 16 and halves of 32 by
// v_permlane16_swap / v_permlane32_swap.  Every lane ends with the winner.
__device__ __forceinline__ void argmax_take(double& best, int& bs, double ob, int os) {
    if (ob > best || (ob == best && os < bs)) {
        best = ob;
        bs = os;
    }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(double& best, int& bs) {
    const int2 u = __builtin_bit_cast(int2, best);
    int2 o;
    o.x = __builtin_amdgcn_mov_dpp(u.x, CTRL, 0xf, 0xf, false);
    o.y = __builtin_amdgcn_mov_dpp(u.y, CTRL, 0xf, 0xf, false);
    const int os = __builtin_amdgcn_mov_dpp(bs, CTRL, 0xf, 0xf, false);
    argmax_take(best, bs, __builtin_bit_cast(double, o), os);
}
// The two elements a swap returns are this lane's and its partner's values
// (in some order); both lanes keep the better of the two.
template <bool ROWS16>
__device__ __forceinline__ void argmax_swap(double& best, int& bs) {
    const int2 u = __builtin_bit_cast(int2, best);
    const auto lo = ROWS16 ? __builtin_amdgcn_permlane16_swap(u.x, u.x, false, false)
                           : __builtin_amdgcn_permlane32_swap(u.x, u.x, false, false);
    const auto hi = ROWS16 ? __builtin_amdgcn_permlane16_swap(u.y, u.y, false, false)
                           : __builtin_amdgcn_permlane32_swap(u.y, u.y, false, false);
    const auto ix = ROWS16 ? __builtin_amdgcn_permlane16_swap(bs, bs, false, false)
                           : __builtin_amdgcn_permlane32_swap(bs, bs, false, false);
    double a = __builtin_bit_cast(double, int2{static_cast<int>(lo[0]), static_cast<int>(hi[0])});
    int ia = static_cast<int>(ix[0]);
    argmax_take(a, ia,
                __builtin_bit_cast(double, int2{static_cast<int>(lo[1]), static_cast<int>(hi[1])}),
                static_cast<int>(ix[1]));
    best = a;
    bs = ia;
}
__device__ __forceinline__ void wave_argmax(double& best, int& bs) {
    argmax_dpp<0xB1>(best, bs);   // quad_perm [1,0,3,2]: lane ^ 1
    argmax_dpp<0x4E>(best, bs);   // quad_perm [2,3,0,1]: lane ^ 2
    argmax_dpp<0x141>(best, bs);  // row_half_mirror: the other quad of 8
    argmax_dpp<0x140>(best, bs);  // row_mirror: the other 8 of 16
    argmax_swap<true>(best, bs);
    argmax_swap<false>(best, bs);
}

// One stage of the affinity relay: quad lane J adds its 8 products to the
// running sums (products rounded before each addition), then lane J's sums
// are broadcast to its quad with a DPP quad permutation.
template <int J>
__device__ __forceinline__ double quad_bcast(double x) {
    const int2 u = __builtin_bit_cast(int2, x);
    int2 o;
    o.x = __builtin_amdgcn_mov_dpp(u.x, J * 0x55, 0xf, 0xf, false);
    o.y = __builtin_amdgcn_mov_dpp(u.y, J * 0x55, 0xf, 0xf, false);
    return __builtin_bit_cast(double, o);
}

template <int J>
__device__ __forceinline__ void relay_stage(int sub, const double (&q0)[8], const double (&k0)[8],
                                            const double (&q1)[8], const double (&k1)[8],
                                            double& r0, double& r1) {
    if (sub == J) {
#pragma clang fp contract(off)
        double a = r0, b = r1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a = a + q0[e] * k0[e];
            b = b + q1[e] * k1[e];
        }
        r0 = a;
        r1 = b;
    }
    r0 = quad_bcast<J>(r0);
    r1 = quad_bcast<J>(r1);
}

// ---------------------------------------------------------------------------
// Routing + attention + LePE, one workgroup per (image, region), all heads.
// Fixed shapes with the MFMA LePE need little enough LDS for five workgroups
// per CU, so they are compiled for five waves per SIMD.
#define KWAVES_PER_EU (VEC_OF(T) == 8 && LepeMfmaShape<HS, WS, HEADS>::ok ? 4 : 4)
#define VEC_OF(T) (sizeof(T) == 2 ? 8 : 4)
template <typename T, int HS, int WS, int NW, int HEADS, int KTOP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KWAVES_PER_EU, 8))) void
route_attend_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                    const double* __restrict__ means, const float* __restrict__ lepe_w,
                    const float* __restrict__ lepe_b, const uint2* __restrict__ lepe_table,
                    T* __restrict__ out, int32_t* __restrict__ routing_idx, Params p_in) {
    const Params p = fold_geometry<HS, WS, NW, HEADS, KTOP, Elem<T>::kVec>(p_in);
    extern __shared__ __align__(16) unsigned char smem[];
    double* sAff = reinterpret_cast<double*>(smem + p.off_aff);
    T* sVh = reinterpret_cast<T*>(smem + p.off_vh);
    float* sL = reinterpret_cast<float*>(smem + p.off_l);
    float* sW = reinterpret_cast<float*>(smem + p.off_w);
    int* sIdx = reinterpret_cast<int*>(smem + p.off_idx);
    const bool w_in_lds = p.off_w >= 0;

    constexpr int VEC = Elem<T>::kVec;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int b = blk / p.R, r = blk - b * p.R;
    const int y0 = (r / p.n) * p.hs, x0 = (r % p.n) * p.ws;
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C;
    const int nvec = p.C / VEC;
    const int hw = p.ws + 4;
    const int naff = p.heads * p.R;
    const size_t mstride = static_cast<size_t>(p.B) * p.heads * p.R * kHeadDim;
    const double* qbar_img = means + static_cast<size_t>(b) * naff * kHeadDim;
    const double* kbar_img = qbar_img + mstride;

    // 1. Issue every load that does not depend on the routing, oldest first:
    //    the LePE weights (to LDS; the barrier after step 2 publishes them),
    //    this lane's slices of the Q mean and of two K means (affinity items),
    //    then the V window with its halo (HBM, the slowest) into registers.
    // LePE weights and bias (nw + nb 16-byte pieces): the first kWRegs pieces
    // of each thread ride in registers and are stored after the affinity, so
    // no LDS store waits on its load here; any further pieces go directly.
    const int nw = p.C * 25 / 4, nb = lepe_b ? p.C / 4 : 0;
    const bool stage_w = w_in_lds && p.has_lepe;
    float4 wreg[kWRegs];
#pragma unroll
    for (int u = 0; u < kWRegs; ++u) {
        const int i = tid + u * kThreads;
        wreg[u] = float4{0.f, 0.f, 0.f, 0.f};
        if (stage_w && i < nw + nb)
            wreg[u] = i < nw ? reinterpret_cast<const float4*>(lepe_w)[i]
                             : reinterpret_cast<const float4*>(lepe_b)[i - nw];
    }
    // Affinity item `it` = h * R + s is computed by the four lanes of a quad;
    // lane `sub` of the quad owns dims 8*sub .. 8*sub+7.
    const int sub = tid & 3;
    auto load_slices = [&](int it, double (&qs)[8], double (&ks)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[e] = ks[e] = 0.0;
        if (it < naff) {
            const int h = it / p.R;
            const double2* qsrc =
                reinterpret_cast<const double2*>(qbar_img + (h * p.R + r) * kHeadDim + sub * 8);
            const double2* ksrc =
                reinterpret_cast<const double2*>(kbar_img + it * kHeadDim + sub * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double2 x = qsrc[e], y = ksrc[e];
                qs[2 * e] = x.x;
                qs[2 * e + 1] = x.y;
                ks[2 * e] = y.x;
                ks[2 * e + 1] = y.y;
            }
        }
    };
    double q0[8], k0[8], q1[8], k1[8];
    load_slices(tid >> 2, q0, k0);
    load_slices(64 + (tid >> 2), q1, k1);
    // halo pieces kept in registers: all of them for a fixed shape (when they
    // fit kHaloRegs per thread), kHaloRegs otherwise
    constexpr int kHaloFixed =
        (HS > 0 && WS > 0 && HEADS > 0) ? ((HS + 4) * (WS + 4) * (HEADS * kHeadDim / VEC) +
                                           kThreads - 1) / kThreads
                                        : kHaloRegs;
    constexpr int kHR = kHaloFixed < kHaloRegs ? kHaloFixed : kHaloRegs;
    uint4 hreg[kHR];
#pragma unroll
    for (int u = 0; u < kHR; ++u) {
        const int i = tid + u * kThreads;
        hreg[u] = uint4{0u, 0u, 0u, 0u};
        if (p.has_lepe && i < p.halo_pieces) {
            const int cell = i / nvec, pv = i - cell * nvec;
            const int hy = cell / hw, hx = cell - hy * hw;
            const int y = y0 + hy - 2, x = x0 + hx - 2;
            if (y >= 0 && y < p.H && x >= 0 && x < p.W)
                hreg[u] = *reinterpret_cast<const uint4*>(v + img + (y * p.W + x) * p.C + pv * VEC);
        }
    }
    // the routed-region list starts as valid ids, so even non-finite
    // affinities cannot send the gather outside the image
    for (int i = tid; i < p.heads * p.k; i += kThreads) sIdx[i] = 0;

    // 2. Affinity Qbar . Kbar per (head, region), fp64, two items per quad at
    //    a time.  Quad lane `sub` continues the running sum of lane sub-1
    //    (broadcast inside the quad with DPP), so the additions happen in the
    //    order d = 0, 1, ..., 31 -- the same IEEE operations as a plain
    //    sequential loop.
    for (int base = 0; base < naff; base += 128) {
        if (base > 0) {
            load_slices(base + (tid >> 2), q0, k0);
            load_slices(base + 64 + (tid >> 2), q1, k1);
        }
        double r0 = 0.0, r1 = 0.0;
        relay_stage<0>(sub, q0, k0, q1, k1, r0, r1);
        relay_stage<1>(sub, q0, k0, q1, k1, r0, r1);
        relay_stage<2>(sub, q0, k0, q1, k1, r0, r1);
        relay_stage<3>(sub, q0, k0, q1, k1, r0, r1);
        if (sub == 0) {
            const int i0 = base + (tid >> 2), i1 = base + 64 + (tid >> 2);
            if (i0 < naff) sAff[i0] = r0;
            if (i1 < naff) sAff[i1] = r1;
        }
    }
    if (stage_w) {
#pragma unroll
        for (int u = 0; u < kWRegs; ++u) {
            const int i = tid + u * kThreads;
            if (i < nw + nb) reinterpret_cast<float4*>(sW)[i] = wreg[u];
        }
        for (int i = tid + kWRegs * kThreads; i < nw + nb; i += kThreads)
            reinterpret_cast<float4*>(sW)[i] = i < nw
                                                   ? reinterpret_cast<const float4*>(lepe_w)[i]
                                                   : reinterpret_cast<const float4*>(lepe_b)[i - nw];
    }
    __syncthreads();

    // 3. Top-k.  k = 1: wave argmax per head (exact ties to the lower id).
    //    Otherwise by rank: position of region s in the order (affinity
    //    descending, region id ascending); the k first positions are kept.
    if constexpr (KTOP == 1) {
        for (int h = w; h < p.heads; h += kWaves) {
            double best = -INFINITY;
            int bs = 0x7fffffff;
            for (int s = lane; s < p.R; s += 64) {
                const double a = sAff[h * p.R + s];
                if (a > best || bs == 0x7fffffff) {
                    best = a;
                    bs = s;
                }
            }
            wave_argmax(best, bs);
            if (lane == 0) {
                const int sel = bs < p.R ? bs : 0;
                sIdx[h] = sel;
                if (routing_idx)
                    routing_idx[(static_cast<size_t>(b) * p.heads + h) * p.R + r] = sel;
            }
        }
    } else {
        for (int it = tid; it < naff; it += kThreads) {
            const int h = it / p.R, s = it - h * p.R;
            const double a = sAff[it];
            const double* row = sAff + h * p.R;
            int rank = 0;
            int s2 = 0;
            for (; s2 + 8 <= p.R; s2 += 8) {
                double a2[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) a2[e] = row[s2 + e];
#pragma unroll
                for (int e = 0; e < 8; ++e) rank += (a2[e] > a) || (a2[e] == a && s2 + e < s);
            }
            for (; s2 < p.R; ++s2) {
                const double a2 = row[s2];
                rank += (a2 > a) || (a2 == a && s2 < s);
            }
            if (rank < p.k) {
                sIdx[h * p.k + rank] = s;
                if (routing_idx)
                    routing_idx[((static_cast<size_t>(b) * p.heads + h) * p.R + r) * p.k + rank] =
                        s;
            }
        }
    }
    __syncthreads();

    // 4. The V halo into LDS (pieces beyond the register batch load here):
    //    channel-planar for the MFMA LePE, NHWC otherwise.  The MFMA LePE
    //    operands are loaded first, so that they are not queued behind the
    //    gather issued in step 6.
    constexpr bool kLepeMfma = VEC == 8 && LepeMfmaShape<HS, WS, HEADS>::ok;
    LepeOperands<kLepeMfma ? HS : 4, kLepeMfma ? WS : 4, kLepeMfma ? HEADS : 1> lop;
    if constexpr (kLepeMfma) {
        if (p.has_lepe) lepe_mfma_load<HS, WS, HEADS>(lepe_table, lepe_b, lop);
    }
    auto halo_store = [&](int i, uint4 val) {
        const int cell = i / nvec, pv = i - cell * nvec;
        if constexpr (kLepeMfma) {
            using S = LepeMfmaShape<HS, WS, HEADS>;
            uint16_t* dst = reinterpret_cast<uint16_t*>(sVh) + pv * 8 * S::PS + cell;
            const uint32_t wd[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dst[(2 * e) * S::PS] = static_cast<uint16_t>(wd[e] & 0xffffu);
                dst[(2 * e + 1) * S::PS] = static_cast<uint16_t>(wd[e] >> 16);
            }
        } else {
            *reinterpret_cast<uint4*>(sVh + cell * p.C + pv * VEC) = val;
        }
    };
    if (p.has_lepe) {
#pragma unroll
        for (int u = 0; u < kHR; ++u) {
            const int i = tid + u * kThreads;
            if (i < p.halo_pieces) halo_store(i, hreg[u]);
        }
        for (int i = tid + kHR * kThreads; i < p.halo_pieces; i += kThreads) {
            const int cell = i / nvec, pv = i - cell * nvec;
            const int hy = cell / hw, hx = cell - hy * hw;
            const int y = y0 + hy - 2, x = x0 + hx - 2;
            uint4 val = {0u, 0u, 0u, 0u};
            if (y >= 0 && y < p.H && x >= 0 && x < p.W)
                val = *reinterpret_cast<const uint4*>(v + img + (y * p.W + x) * p.C + pv * VEC);
            halo_store(i, val);
        }
    }
    __syncthreads();

    // 5. LePE with weights from global memory happens before the gather is
    //    issued (a load queued behind the gather would wait for it) ...
    const float* wsrc = w_in_lds ? sW : lepe_w;
    const float* bsrc = w_in_lds ? (lepe_b ? sW + p.C * 25 : nullptr) : lepe_b;
    if (!kLepeMfma && !w_in_lds) lepe_phase<T>(p, sVh, sL, wsrc, bsrc);

    // 6. ... each wave issues the gather of its first (job, chunk) step ...
    WaveJobs J(p, w);
    StepRegs cur;
    bf16x8_t qb[kMaxQTiles];
    if constexpr (VEC == 8) {
        if (J.nsteps > 0) {
            load_q_operands(p, J, w, reinterpret_cast<const uint16_t*>(q) + img, r, qb);
            gather_step(p, J, w, 0, reinterpret_cast<const uint16_t*>(k) + img,
                        reinterpret_cast<const uint16_t*>(v) + img, sIdx, cur);
        }
    }
    // ... and LePE with weights staged in LDS runs while it is in flight.
    if constexpr (kLepeMfma) {
        if (p.has_lepe) {
            lepe_mfma_compute<HS, WS, HEADS>(p, reinterpret_cast<const uint16_t*>(sVh), sL, lop);
        } else {
            for (int i = tid; i < p.t * p.lstride; i += kThreads) sL[i] = 0.f;
            __syncthreads();
        }
    } else {
        if (w_in_lds) lepe_phase<T>(p, sVh, sL, wsrc, bsrc);
    }

    // 7. Token attention over the routed tokens, added into sL.
    if constexpr (VEC == 8) {
        attend_mfma(p, J, reinterpret_cast<const uint16_t*>(q) + img,
                    reinterpret_cast<const uint16_t*>(k) + img,
                    reinterpret_cast<const uint16_t*>(v) + img, r,
                    reinterpret_cast<uint16_t*>(smem + p.off_vt), sL, sIdx, cur, qb);
    } else {
        attend_valu(p, reinterpret_cast<const float*>(q) + img,
                    reinterpret_cast<const float*>(k) + img,
                    reinterpret_cast<const float*>(v) + img, r, sL, sIdx);
    }
    __syncthreads();

    // 8. out = LePE + O, one rounding, 16-byte NHWC stores.
    for (int i = tid; i < p.t * nvec; i += kThreads) {
        const int slot = i / nvec, pv = i - slot * nvec;
        const float* src = sL + slot * p.lstride + pv * VEC;
        T* dst = out + img + token_offset(p, r, slot) + pv * VEC;
        if constexpr (VEC == 8) {
            const float4 a = *reinterpret_cast<const float4*>(src);
            const float4 c = *reinterpret_cast<const float4*>(src + 4);
            uint4 u;
            u.x = f32_to_bf16(a.x) | (f32_to_bf16(a.y) << 16);
            u.y = f32_to_bf16(a.z) | (f32_to_bf16(a.w) << 16);
            u.z = f32_to_bf16(c.x) | (f32_to_bf16(c.y) << 16);
            u.w = f32_to_bf16(c.z) | (f32_to_bf16(c.w) << 16);
            *reinterpret_cast<uint4*>(dst) = u;
        } else {
            *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
        }
    }
}

}  // namespace

// Shapes with a compiled instance whose geometry is folded at compile time;
// every other shape runs the generic instance.
struct GeoKey {
    bool bf16;
    int hs, ws, n, heads, k;
};

template <typename T, int HS, int WS, int NW, int HEADS, int KTOP>
struct Inst {
    static constexpr GeoKey key{sizeof(T) == 2, HS, WS, NW, HEADS, KTOP};
};

static bool matches(const GeoKey& g, const Params& p, bool bf16, bool with_k) {
    return g.bf16 == bf16 && g.hs == p.hs && g.ws == p.ws && g.n == p.n && g.heads == p.heads &&
           (!with_k || g.k == p.k);
}

// The fixed shapes: BiFormer-S stages 1-3 (7x7 regions of 8x8, 4x4 and 2x2
// tokens), the 512x512 segmentation map at stride 4 (16x16 regions of 8x8),
// and the small fp32 map (7x7 regions of 4x4).
#define BRA_FOR_EACH_SHAPE(X)            \
    X(uint16_t, 8, 8, 7, 2, 1)           \
    X(uint16_t, 4, 4, 7, 4, 4)           \
    X(uint16_t, 2, 2, 7, 8, 16)          \
    X(uint16_t, 8, 8, 16, 2, 16)         \
    X(float, 4, 4, 7, 2, 4)

// ---------------------------------------------------------------------------
static long align16(long x) { return (x + 15) & ~15L; }

bool plan(Params& p, int B, int H, int W, int C, int heads, int n_win, int k, float scale,
          bool bf16) {
    p.B = B;
    p.H = H;
    p.W = W;
    p.C = C;
    p.heads = heads;
    p.n = n_win;
    p.R = n_win * n_win;
    p.hs = H / n_win;
    p.ws = W / n_win;
    p.t = p.hs * p.ws;
    p.k = k;
    p.nkeys = k * p.t;
    p.scale_log2e = scale * 1.4426950408889634f;
    p.has_lepe = 0;
    const long es = bf16 ? 2 : 4;
    const int vec = bf16 ? 8 : 4;
    p.lstride = C + 4;
    p.lepe_items = (C / 2) * p.hs * ((p.ws + kLepeCols - 1) / kLepeCols);
    p.halo_pieces = (p.hs + 4) * (p.ws + 4) * (C / vec);

    long off = 0;
    auto take = [&](long bytes) {
        const long o = off;
        off = align16(off + bytes);
        return static_cast<int>(o);
    };
    const long t = p.t;
    // The routing scratch (affinities) shares its bytes with the per-wave V
    // staging of the attention, which starts after routing ends.
    const long vt_bytes = bf16 ? static_cast<long>(kWaves) * 32 * kVtStride * 2 : 0;
    const long aff_bytes = align16(static_cast<long>(heads) * p.R * 8);
    const int base = take(std::max(vt_bytes, aff_bytes));
    p.off_vt = base;
    p.off_aff = base;
    // The fixed bf16 shapes whose windows tile by 4x4 run LePE on MFMA with a
    // channel-planar halo; the others on VALU with an NHWC halo.
    bool specialized = false;
#define BRA_IS_FIXED(T, HS, WS, NW, HEADS, KTOP) \
    specialized = specialized || matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, true);
    BRA_FOR_EACH_SHAPE(BRA_IS_FIXED)
#undef BRA_IS_FIXED
    p.lepe_mfma = bf16 && specialized && lepe_mfma_fits(p.hs, p.ws, heads);
    const long vh_bytes =
        p.lepe_mfma ? static_cast<long>(C) * ((p.hs + 4) * (p.ws + 4) + 4) * 2
                    : static_cast<long>(p.hs + 4) * (p.ws + 4) * C * es;
    const long l_bytes = t * p.lstride * 4;
    p.lepe_alias = p.lepe_mfma || p.lepe_items <= kThreads;
    if (p.lepe_alias) {
        p.off_vh = take(std::max(vh_bytes, l_bytes));
        p.off_l = p.off_vh;
    } else {
        p.off_vh = take(vh_bytes);
        p.off_l = take(l_bytes);
    }
    p.off_idx = take(static_cast<long>(heads) * k * 4);
    // LePE weights and bias go to LDS while four workgroups still fit a CU.
    const long w_bytes = static_cast<long>(C) * 26 * 4;
    if (!p.lepe_mfma && off + w_bytes <= 40 * 1024) {
        p.off_w = take(w_bytes);
    } else {
        p.off_w = -1;
    }
    p.lds_bytes = static_cast<int>(off);
    p.table_items = p.lepe_mfma ? C * 40 : 0;
    {
        const int nvec = C / vec;
        const bool wave_path = bf16 && 64 % nvec == 0;
        p.pool_blocks = wave_path ? (B * p.R + 1) / 2 : B * p.R;
    }
    p.pool_chunk = std::max(1, std::min(p.t, kPoolChunkBytes / (C * static_cast<int>(es))));
    // LDS of the pool kernel's staged path (fp32, or C/8 not dividing 64)
    p.pool_lds_bytes = p.pool_chunk * C * static_cast<int>(es);
    return off <= kMaxLdsBytes && C <= kMaxChannels && C % 32 == 0;
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

hipError_t launch_route_attend(const Params& p, bool bf16, const void* q, const void* k,
                               const void* v, const double* means, const float* lepe_w,
                               const float* lepe_b, const uint2* lepe_table, void* out,
                               int32_t* routing_idx, hipStream_t stream) {
    Params pp = p;
    pp.has_lepe = lepe_w != nullptr;
    if (!pp.has_lepe) lepe_b = nullptr;
    const dim3 grid(p.B * p.R), block(kThreads);
#define BRA_ATTEND(T, HS, WS, NW, HEADS, KTOP)                                                 \
    if (matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, true)) {                       \
        hipLaunchKernelGGL((route_attend_kernel<T, HS, WS, NW, HEADS, KTOP>), grid, block,     \
                           p.lds_bytes, stream, static_cast<const T*>(q),                      \
                           static_cast<const T*>(k), static_cast<const T*>(v), means, lepe_w,  \
                           lepe_b, lepe_table, static_cast<T*>(out), routing_idx, pp);         \
        return hipGetLastError();                                                              \
    }
    BRA_FOR_EACH_SHAPE(BRA_ATTEND)
#undef BRA_ATTEND
    if (bf16)
        hipLaunchKernelGGL((route_attend_kernel<uint16_t, 0, 0, 0, 0, 0>), grid, block,
                           p.lds_bytes, stream, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), means,
                           lepe_w, lepe_b, lepe_table, static_cast<uint16_t*>(out), routing_idx,
                           pp);
    else
        hipLaunchKernelGGL((route_attend_kernel<float, 0, 0, 0, 0, 0>), grid, block, p.lds_bytes,
                           stream, static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), means, lepe_w, lepe_b, lepe_table,
                           static_cast<float*>(out), routing_idx, pp);
    return hipGetLastError();
}

}  // namespace bra
