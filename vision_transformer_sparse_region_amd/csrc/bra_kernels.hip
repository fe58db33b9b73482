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
//                        stage the Q window and the V window + 2-token halo in LDS,
//                        fp64 Q mean, fp64 affinity against every K mean, rank-based
//                        top-k (ties to the lower id)                 [P1 §2.1; P5 §五 ③-④]
//                        gather the routed K/V tokens by index straight into MFMA
//                        operands / LDS, S^T = K Q^T and O^T += V^T P^T on bf16 MFMA
//                        with an fp32 online softmax                  [P3 §2.2; P5 §五 ⑤-⑦]
//                        epilogue: 5x5 depthwise LePE of V from the LDS halo, + O,
//                        one rounding to the output type, NHWC store  [P5 §五 lepe, ⑧]
// The gathered K/V tiles are never materialised in HBM ([P3 §4.2] and [P1 §2.2]
// build a dense k-fold copy with torch.gather; here the index drives the loads).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_launch.h"

namespace bra {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bf16 bits.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int kVec = 4;  // elements per 16-byte piece
    __device__ static float f32(float x) { return x; }
};
template <>
struct Elem<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static float f32(uint16_t x) { return bf16_to_f32(x); }
};

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap so that consecutive logical ids -- the regions of one image --
// run on one XCD and share its L2 for the routed K/V and halo reads.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
    const int full = nblocks & ~7;
    if (bid >= full) return bid;
    return (bid & 7) * (full >> 3) + (bid >> 3);
}

// Token offset (elements) of slot `slot` of region `reg` inside one image.
__device__ __forceinline__ int token_offset(const Params& p, int reg, int slot) {
    const int ri = reg / p.n, rj = reg - ri * p.n;
    const int u = slot / p.ws, w = slot - u * p.ws;
    return ((ri * p.hs + u) * p.W + rj * p.ws + w) * p.C;
}

// Q_r . K_s over the 32 dims of one head, left to right, each product rounded
// before it is added -- the same IEEE operations as a plain fp64 loop.
__device__ __forceinline__ double dot32_seq(const double* a, const double* __restrict__ b) {
#pragma clang fp contract(off)
    double s = 0.0;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) s = s + a[d] * b[d];
    return s;
}

// ---------------------------------------------------------------------------
// Region means of K (fp64).  Summation runs over the window's tokens in
// row-major slot order per channel; for bf16 (8-bit significand) and fp32
// inputs of ordinary range every partial sum is exact in fp64, so the mean is
// the correctly rounded quotient of the exact sum.
template <typename T>
__global__ __launch_bounds__(kThreads) void pool_k_kernel(const T* __restrict__ kin,
                                                          double* __restrict__ kbar, Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    T* tile = reinterpret_cast<T*>(smem);
    constexpr int VEC = Elem<T>::kVec;
    const int tid = threadIdx.x;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int b = blk / p.R, r = blk - b * p.R;
    const T* kimg = kin + static_cast<size_t>(b) * p.H * p.W * p.C;
    const int nvec = p.C / VEC;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};  // channels tid + 256*j (C <= 1024)
    for (int t0 = 0; t0 < p.t; t0 += p.pool_chunk) {
        const int nt = min(p.pool_chunk, p.t - t0);
        for (int i = tid; i < nt * nvec; i += kThreads) {
            const int tt = i / nvec, pv = i - tt * nvec;
            const uint4 val =
                *reinterpret_cast<const uint4*>(kimg + token_offset(p, r, t0 + tt) + pv * VEC);
            *reinterpret_cast<uint4*>(tile + tt * p.C + pv * VEC) = val;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
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
    for (int j = 0; j < 4; ++j) {
        const int c = tid + j * kThreads;
        if (c < p.C) {
            const int h = c / kHeadDim, d = c - h * kHeadDim;
            kbar[((static_cast<size_t>(b) * p.heads + h) * p.R + r) * kHeadDim + d] =
                acc[j] / static_cast<double>(p.t);
        }
    }
}

// ---------------------------------------------------------------------------
// Token attention, bf16 MFMA path.
//
// A wave owns a "job": one head and up to kMaxQTiles tiles of 16 query tokens.
// Keys stream in chunks of 32.  For a chunk, two v_mfma_f32_16x16x32_bf16
// give S^T (keys x queries): operand A row i (lane & 15) is the key
//   32c + 8*(i/4) + 4*blk + i%4,
// so that output lane (query li, group g = lane/16) holds the scores of the
// 8 consecutive keys 32c + 8g .. 32c + 8g + 7.  Those 8 probabilities are
// exactly that lane's B operand of O^T += V^T P^T (k-slot 8g + e = key
// 32c + 8g + e), so P never leaves registers; V^T is read transposed from a
// per-wave LDS staging buffer.  O^T lands with the query on lane & 15, like
// the scores, so the online-softmax rescale is lane-local.
__device__ void attend_mfma(const Params& p, const uint16_t* __restrict__ kimg,
                            const uint16_t* __restrict__ vimg, const uint16_t* sQ,
                            uint16_t* sVt_all, float* sO, const int* sIdx) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    uint16_t* sVt = sVt_all + w * 32 * kVtStride;
    const int QT = (p.t + 15) / 16;
    const int wph = max(1, kWaves / p.heads);
    int G = min(wph, QT);
    G = max(G, (QT + kMaxQTiles - 1) / kMaxQTiles);
    const int tpg = (QT + G - 1) / G;
    const int njobs = p.heads * G;
    const int nchunks = (p.nkeys + 31) / 32;
    const bf16x8_t zero8 = __builtin_bit_cast(bf16x8_t, u16x8_t{0, 0, 0, 0, 0, 0, 0, 0});

    for (int job = w; job < njobs; job += kWaves) {
        const int h = job / G, grp = job - h * G;
        const int qt0 = grp * tpg;
        const int nq = min(tpg, QT - qt0);
        if (nq <= 0) continue;
        const int* idx = sIdx + h * p.k;
        const int hoff = h * kHeadDim;

        bf16x8_t qb[kMaxQTiles];
        float m[kMaxQTiles], l[kMaxQTiles];
        f32x4_t o0[kMaxQTiles], o1[kMaxQTiles];
#pragma unroll
        for (int jq = 0; jq < kMaxQTiles; ++jq) {
            const int qi = (qt0 + jq) * 16 + li;
            qb[jq] = (jq < nq && qi < p.t)
                         ? *reinterpret_cast<const bf16x8_t*>(sQ + qi * p.qstride + hoff + 8 * g)
                         : zero8;
            m[jq] = -INFINITY;
            l[jq] = 0.f;
            o0[jq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            o1[jq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        for (int c = 0; c < nchunks; ++c) {
            // K^T operands straight from global memory (16 B per lane).
            bf16x8_t ka[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int key = 32 * c + 8 * (li >> 2) + 4 * blk + (li & 3);
                ka[blk] = zero8;
                if (key < p.nkeys) {
                    const int j = key / p.t, slot = key - j * p.t;
                    ka[blk] = *reinterpret_cast<const bf16x8_t*>(
                        kimg + token_offset(p, idx[j], slot) + hoff + 8 * g);
                }
            }
            // V chunk (32 keys x 32 dims) into this wave's LDS buffer.
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int pc = lane + 64 * pp;
                const int kl = pc >> 2, d0 = 8 * (pc & 3);
                const int key = 32 * c + kl;
                uint4 val = {0u, 0u, 0u, 0u};
                if (key < p.nkeys) {
                    const int j = key / p.t, slot = key - j * p.t;
                    val = *reinterpret_cast<const uint4*>(vimg + token_offset(p, idx[j], slot) +
                                                         hoff + d0);
                }
                uint2* dst = reinterpret_cast<uint2*>(sVt + kl * kVtStride + d0);
                dst[0] = uint2{val.x, val.y};
                dst[1] = uint2{val.z, val.w};
            }
            // A wave's LDS operations complete in order; the fence keeps the
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

#pragma unroll
            for (int jq = 0; jq < kMaxQTiles; ++jq) {
                if (jq >= nq) break;
                const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
                const f32x4_t s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0], qb[jq], z4, 0, 0, 0);
                const f32x4_t s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1], qb[jq], z4, 0, 0, 0);
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = s0[e] * p.scale_log2e;
                    x[4 + e] = s1[e] * p.scale_log2e;
                }
                const int kbase = 32 * c + 8 * g;
                if (kbase + 8 > p.nkeys) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (kbase + e >= p.nkeys) x[e] = -INFINITY;
                }
                float mx = x[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mnew = fmaxf(m[jq], mx);
                const float alpha = __builtin_amdgcn_exp2f(m[jq] - mnew);
                float psum = 0.f;
                bf16x8_t pb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pe = __builtin_amdgcn_exp2f(x[e] - mnew);
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
        }

#pragma unroll
        for (int jq = 0; jq < kMaxQTiles; ++jq) {
            if (jq >= nq) break;
            float lt = l[jq];
            lt += __shfl_xor(lt, 16);
            lt += __shfl_xor(lt, 32);
            const float inv = 1.f / lt;
            const int qi = (qt0 + jq) * 16 + li;
            if (qi < p.t) {
                float* dst = sO + qi * p.C + hoff + 4 * g;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dst[e] = o0[jq][e] * inv;
                    dst[16 + e] = o1[jq][e] * inv;
                }
            }
        }
    }
}

// Token attention, fp32 VALU path: one thread per (query token, head), keys
// in routed order with an online softmax; fp32 throughout.
__device__ void attend_valu(const Params& p, const float* __restrict__ kimg,
                            const float* __restrict__ vimg, const float* sQ, float* sO,
                            const int* sIdx) {
    for (int it = threadIdx.x; it < p.t * p.heads; it += kThreads) {
        const int h = it / p.t, slot = it - h * p.t;
        const int hoff = h * kHeadDim;
        float qv[kHeadDim], acc[kHeadDim];
#pragma unroll
        for (int d = 0; d < kHeadDim; ++d) {
            qv[d] = sQ[slot * p.qstride + hoff + d];
            acc[d] = 0.f;
        }
        float m = -INFINITY, l = 0.f;
        const int* idx = sIdx + h * p.k;
        for (int key = 0; key < p.nkeys; ++key) {
            const int j = key / p.t, ks = key - j * p.t;
            const int off = token_offset(p, idx[j], ks) + hoff;
            const float4* kp = reinterpret_cast<const float4*>(kimg + off);
            float dot = 0.f;
#pragma unroll
            for (int d4 = 0; d4 < kHeadDim / 4; ++d4) {
                const float4 kv = kp[d4];
                dot = fmaf(qv[4 * d4 + 0], kv.x, dot);
                dot = fmaf(qv[4 * d4 + 1], kv.y, dot);
                dot = fmaf(qv[4 * d4 + 2], kv.z, dot);
                dot = fmaf(qv[4 * d4 + 3], kv.w, dot);
            }
            const float x = dot * p.scale_log2e;
            const float mnew = fmaxf(m, x);
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            const float pe = __builtin_amdgcn_exp2f(x - mnew);
            l = l * alpha + pe;
            m = mnew;
            const float4* vp = reinterpret_cast<const float4*>(vimg + off);
#pragma unroll
            for (int d4 = 0; d4 < kHeadDim / 4; ++d4) {
                const float4 vv = vp[d4];
                acc[4 * d4 + 0] = fmaf(pe, vv.x, acc[4 * d4 + 0] * alpha);
                acc[4 * d4 + 1] = fmaf(pe, vv.y, acc[4 * d4 + 1] * alpha);
                acc[4 * d4 + 2] = fmaf(pe, vv.z, acc[4 * d4 + 2] * alpha);
                acc[4 * d4 + 3] = fmaf(pe, vv.w, acc[4 * d4 + 3] * alpha);
            }
        }
        const float inv = 1.f / l;
#pragma unroll
        for (int d = 0; d < kHeadDim; ++d) sO[slot * p.C + hoff + d] = acc[d] * inv;
    }
}

__device__ __forceinline__ void store2(float* dst, float a, float b) {
    *reinterpret_cast<float2*>(dst) = float2{a, b};
}
__device__ __forceinline__ void store2(uint16_t* dst, float a, float b) {
    const uint32_t packed =
        static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
    *reinterpret_cast<uint32_t*>(dst) = packed;
}

// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void route_attend_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const double* __restrict__ kbar, const float* __restrict__ lepe_w,
    const float* __restrict__ lepe_b, T* __restrict__ out, int32_t* __restrict__ routing_idx,
    Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    T* sQ = reinterpret_cast<T*>(smem + p.off_q);
    float* sO = reinterpret_cast<float*>(smem + p.off_o);
    T* sVh = reinterpret_cast<T*>(smem + p.off_vh);
    double* sAff = reinterpret_cast<double*>(smem + p.off_aff);
    double* sQbar = reinterpret_cast<double*>(smem + p.off_qbar);
    int* sIdx = reinterpret_cast<int*>(smem + p.off_idx);

    constexpr int VEC = Elem<T>::kVec;
    const int tid = threadIdx.x;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int b = blk / p.R, r = blk - b * p.R;
    const int y0 = (r / p.n) * p.hs, x0 = (r % p.n) * p.ws;
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C;
    const int nvec = p.C / VEC;
    const int hw = p.ws + 4;

    // 1. Stage the Q window and the V window with a 2-token halo (zero off-map).
    for (int i = tid; i < p.t * nvec; i += kThreads) {
        const int slot = i / nvec, pv = i - slot * nvec;
        *reinterpret_cast<uint4*>(sQ + slot * p.qstride + pv * VEC) =
            *reinterpret_cast<const uint4*>(q + img + token_offset(p, r, slot) + pv * VEC);
    }
    if (p.has_lepe) {
        for (int i = tid; i < (p.hs + 4) * hw * nvec; i += kThreads) {
            const int cell = i / nvec, pv = i - cell * nvec;
            const int hy = cell / hw, hx = cell - hy * hw;
            const int y = y0 + hy - 2, x = x0 + hx - 2;
            uint4 val = {0u, 0u, 0u, 0u};
            if (y >= 0 && y < p.H && x >= 0 && x < p.W)
                val = *reinterpret_cast<const uint4*>(v + img + (y * p.W + x) * p.C + pv * VEC);
            *reinterpret_cast<uint4*>(sVh + cell * p.C + pv * VEC) = val;
        }
    }
    __syncthreads();

    // 2. Q region mean per channel, fp64, slot order.  (The routed-region
    //    list starts as valid ids, so even non-finite affinities cannot send
    //    the gather out of the image.)
    for (int i = tid; i < p.heads * p.k; i += kThreads) sIdx[i] = 0;
    for (int c = tid; c < p.C; c += kThreads) {
        double s = 0.0;
        for (int slot = 0; slot < p.t; ++slot)
            s += static_cast<double>(Elem<T>::f32(sQ[slot * p.qstride + c]));
        sQbar[c] = s / static_cast<double>(p.t);
    }
    __syncthreads();

    // 3. Region affinity of this region against every region, per head.
    const double* kb_img = kbar + static_cast<size_t>(b) * p.heads * p.R * kHeadDim;
    for (int it = tid; it < p.heads * p.R; it += kThreads) {
        const int h = it / p.R;
        sAff[it] = dot32_seq(sQbar + h * kHeadDim, kb_img + static_cast<size_t>(it) * kHeadDim);
    }
    __syncthreads();

    // 4. Top-k by rank: position of region s in the order (affinity
    //    descending, region id ascending); the k lowest positions are kept.
    for (int it = tid; it < p.heads * p.R; it += kThreads) {
        const int h = it / p.R, s = it - h * p.R;
        const double a = sAff[it];
        const double* row = sAff + h * p.R;
        int rank = 0;
        for (int s2 = 0; s2 < p.R; ++s2) {
            const double a2 = row[s2];
            rank += (a2 > a) || (a2 == a && s2 < s);
        }
        if (rank < p.k) {
            sIdx[h * p.k + rank] = s;
            if (routing_idx)
                routing_idx[((static_cast<size_t>(b) * p.heads + h) * p.R + r) * p.k + rank] = s;
        }
    }
    __syncthreads();

    // 5. Attention over the routed tokens -> normalised O in sO (fp32).
    if constexpr (VEC == 8) {
        attend_mfma(p, reinterpret_cast<const uint16_t*>(k) + img,
                    reinterpret_cast<const uint16_t*>(v) + img,
                    reinterpret_cast<const uint16_t*>(sQ),
                    reinterpret_cast<uint16_t*>(smem + p.off_vt), sO, sIdx);
    } else {
        attend_valu(p, reinterpret_cast<const float*>(k) + img,
                    reinterpret_cast<const float*>(v) + img, reinterpret_cast<const float*>(sQ),
                    sO, sIdx);
    }
    __syncthreads();

    // 6. LePE from the staged halo, + O, one rounding, NHWC store.  A thread
    //    owns a channel pair and one window row.
    const int npairs = p.C / 2;
    for (int it = tid; it < npairs * p.hs; it += kThreads) {
        const int y = it / npairs, cp = it - y * npairs;
        const int c0 = 2 * cp;
        float w0[25], w1[25];
        float b0 = 0.f, b1 = 0.f;
        if (p.has_lepe) {
#pragma unroll
            for (int i = 0; i < 25; ++i) {
                w0[i] = lepe_w[c0 * 25 + i];
                w1[i] = lepe_w[(c0 + 1) * 25 + i];
            }
            if (lepe_b) {
                b0 = lepe_b[c0];
                b1 = lepe_b[c0 + 1];
            }
        }
        for (int x = 0; x < p.ws; ++x) {
            float a0 = b0, a1 = b1;
            if (p.has_lepe) {
#pragma unroll
                for (int i = 0; i < 5; ++i)
#pragma unroll
                    for (int j = 0; j < 5; ++j) {
                        const T* pv = sVh + ((y + i) * hw + x + j) * p.C + c0;
                        a0 += w0[i * 5 + j] * Elem<T>::f32(pv[0]);
                        a1 += w1[i * 5 + j] * Elem<T>::f32(pv[1]);
                    }
            }
            const float* po = sO + (y * p.ws + x) * p.C + c0;
            store2(out + img + ((y0 + y) * p.W + x0 + x) * p.C + c0, po[0] + a0, po[1] + a1);
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
static int align16(int x) { return (x + 15) & ~15; }

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
    const int es = bf16 ? 2 : 4;
    p.qstride = C + (bf16 ? 8 : 0);
    int off = 0;
    auto take = [&](long bytes) {
        const int o = off;
        off = align16(static_cast<int>(off + bytes));
        return o;
    };
    p.off_q = take(static_cast<long>(p.t) * p.qstride * es);
    p.off_vt = take(bf16 ? kWaves * 32 * kVtStride * 2 : 0);
    p.off_o = take(static_cast<long>(p.t) * C * 4);
    p.off_vh = take(static_cast<long>(p.hs + 4) * (p.ws + 4) * C * es);
    p.off_aff = take(static_cast<long>(heads) * p.R * 8);
    p.off_qbar = take(static_cast<long>(C) * 8);
    p.off_idx = take(static_cast<long>(heads) * k * 4);
    p.lds_bytes = off;
    p.pool_chunk = max(1, min(p.t, kPoolChunkBytes / (C * es)));
    p.pool_lds_bytes = p.pool_chunk * C * es;
    return p.lds_bytes <= kMaxLdsBytes && C <= 4 * kThreads && C % 8 == 0;
}

hipError_t launch_pool_k(const Params& p, bool bf16, const void* k, double* kbar,
                         hipStream_t stream) {
    const dim3 grid(p.B * p.R), block(kThreads);
    if (bf16)
        hipLaunchKernelGGL(pool_k_kernel<uint16_t>, grid, block, p.pool_lds_bytes, stream,
                           static_cast<const uint16_t*>(k), kbar, p);
    else
        hipLaunchKernelGGL(pool_k_kernel<float>, grid, block, p.pool_lds_bytes, stream,
                           static_cast<const float*>(k), kbar, p);
    return hipGetLastError();
}

hipError_t launch_route_attend(const Params& p, bool bf16, const void* q, const void* k,
                               const void* v, const double* kbar, const float* lepe_w,
                               const float* lepe_b, void* out, int32_t* routing_idx,
                               hipStream_t stream) {
    Params pp = p;
    pp.has_lepe = lepe_w != nullptr;
    const dim3 grid(p.B * p.R), block(kThreads);
    if (bf16)
        hipLaunchKernelGGL(route_attend_kernel<uint16_t>, grid, block, p.lds_bytes, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), kbar, lepe_w, lepe_b,
                           static_cast<uint16_t*>(out), routing_idx, pp);
    else
        hipLaunchKernelGGL(route_attend_kernel<float>, grid, block, p.lds_bytes, stream,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), kbar, lepe_w, lepe_b,
                           static_cast<float*>(out), routing_idx, pp);
    return hipGetLastError();
}

}  // namespace bra
