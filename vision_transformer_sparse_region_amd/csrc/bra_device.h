// bra_device.h -- device helpers shared by the BRA kernels (gfx950).
//
// Pages cited by key in the kernels:
//   [P1] "从静态到动态：Bi-Level Routing Attention如何重塑视觉Transformer的注意力机制",
//        www.mhpn.cn/news/199372
//   [P2] "BiFormer用双层路由注意力重塑视觉Transformer效率极限", www.mooersco.com/news/894234
//   [P3] "从零构建BiFormer：PyTorch实战双层路由注意力机制与调试全攻略",
//        www.mhpn.cn/news/564882
//   [P4] "手把手解析BiFormer：双水平路由注意力机制与PyTorch实战指南", www.jsqmd.com/news/719213
//   [P5] "【医学图像分割模块】BiFormer / 双层路由注意力（CVPR 2023）", www.mhpn.cn/news/2512273
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_launch.h"

namespace bra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

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

// max(a, b) for non-NaN operands.  IEEE 754-2019 maximum (NaN-propagating)
// lowers to gfx950's v_maximum3_f32 with its operands as they are; fmaxf and
// a median with +inf both become maxNum, for which the compiler first quiets
// every operand it cannot prove canonical (an MFMA result, a lane exchange):
// an extra instruction per operand.
__device__ __forceinline__ float max_f(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}
// Max and sum over the four lanes l, l^16, l^32, l^48 -- in the MFMA
// attention these hold the four key groups of one query.  v_permlane16_swap
// and v_permlane32_swap exchange rows of 16 and halves of 32 lanes in VALU
// registers, without a trip through the LDS crossbar; every lane of the four
// ends with the same value.
__device__ __forceinline__ float group4_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = max_f(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return max_f(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Layout of the fp64 region means in the workspace: Q means row-major
// [B][heads][R][32] (a row is read whole, as wave-uniform scalar loads), then
// K means in dim pairs, [B][heads][16][R][2]: lane s of a wave reads dims
// 2j, 2j + 1 of region s as one 16-byte load, and the lanes' loads of a pair
// are one contiguous run.
__device__ __forceinline__ size_t qmean_index(const Params& p, int bh, int r, int d) {
    return (static_cast<size_t>(bh) * p.R + r) * kHeadDim + d;
}
__device__ __forceinline__ size_t kmean_index(const Params& p, int bh, int d, int s) {
    return static_cast<size_t>(p.B) * p.heads * p.R * kHeadDim +
           ((static_cast<size_t>(bh) * (kHeadDim / 2) + (d >> 1)) * p.R + s) * 2 + (d & 1);
}
// The K mean of region s, head bh, into registers (16 coalesced 16-byte loads).
__device__ __forceinline__ void load_kmean(const Params& p, const double* __restrict__ means,
                                           int bh, int s, double (&kreg)[kHeadDim]) {
#pragma unroll
    for (int j = 0; j < kHeadDim / 2; ++j) {
        const double2 v = *reinterpret_cast<const double2*>(means + kmean_index(p, bh, 2 * j, s));
        kreg[2 * j] = v.x;
        kreg[2 * j + 1] = v.y;
    }
}

// The fp32 copy of the K means (each rounded to nearest), after the fp64 Q
// and K means, in dim quads: [B][heads][8][R][4], so that lane s reads dims
// 4j .. 4j + 3 of region s as one 16-byte load; written when p.kmean32 is
// set.  The routing inside the attention kernel screens with it (half the
// bytes of the fp64 means) and reads the fp64 means only where the screen
// cannot decide.
__device__ __forceinline__ size_t kmean32_offset(const Params& p, int bh, int d, int s) {
    return ((static_cast<size_t>(bh) * (kHeadDim / 4) + (d >> 2)) * p.R + s) * 4 + (d & 3);
}
__device__ __forceinline__ const float* kmean32_base(const Params& p, const double* means) {
    return reinterpret_cast<const float*>(means +
                                          2 * static_cast<size_t>(p.B) * p.heads * p.R * kHeadDim);
}
__device__ __forceinline__ float* kmean32_base(const Params& p, double* means) {
    return reinterpret_cast<float*>(means + 2 * static_cast<size_t>(p.B) * p.heads * p.R * kHeadDim);
}
__device__ __forceinline__ void store_kmean(const Params& p, double* __restrict__ means, int bh,
                                            int d, int s, double m) {
    means[kmean_index(p, bh, d, s)] = m;
    if (p.kmean32)
        kmean32_base(p, means)[kmean32_offset(p, bh, d, s)] = static_cast<float>(m);
}
// Dims d and d + 1 (d even) of one K mean: one 16-byte and one 8-byte store.
__device__ __forceinline__ void store_kmean_pair(const Params& p, double* __restrict__ means,
                                                 int bh, int d, int s, double m0, double m1) {
    *reinterpret_cast<double2*>(means + kmean_index(p, bh, d, s)) = double2{m0, m1};
    if (p.kmean32)
        *reinterpret_cast<float2*>(kmean32_base(p, means) + kmean32_offset(p, bh, d, s)) =
            float2{static_cast<float>(m0), static_cast<float>(m1)};
}
// The fp32 K mean of region s, head bh: dims 2j, 2j + 1 as the two halves
// of kb[j], j < 16 (8 coalesced 16-byte loads; kb[16..31] untouched, so the
// same registers can hold the fp64 mean instead).
__device__ __forceinline__ void load_kmean32(const Params& p, const double* __restrict__ means,
                                             int bh, int s, double (&kb)[kHeadDim]) {
    const float* base = kmean32_base(p, means);
#pragma unroll
    for (int j = 0; j < kHeadDim / 4; ++j) {
        const u32x4_t v =
            *reinterpret_cast<const u32x4_t*>(base + kmean32_offset(p, bh, 4 * j, s));
        kb[2 * j] = __builtin_bit_cast(double, u32x2_t{v[0], v[1]});
        kb[2 * j + 1] = __builtin_bit_cast(double, u32x2_t{v[2], v[3]});
    }
}

// mean = sum / t, as a multiplication when t is a power of two (exact then).
__device__ __forceinline__ double mean_of(double sum, int t) {
    return (t & (t - 1)) == 0 ? sum * (1.0 / static_cast<double>(t)) : sum / static_cast<double>(t);
}

// Element offset, inside one image, of the first token of region `reg`, and
// of slot `slot` relative to it; a token's offset is their sum.  Every factor
// is below 2^24 (an image has fewer than 2^31 elements), so the products are
// 24-bit multiplies.
__device__ __forceinline__ int region_base(const Params& p, int reg) {
    const int ri = reg / p.n, rj = reg - ri * p.n;
    return __mul24(__mul24(__mul24(ri, p.hs), p.W) + __mul24(rj, p.ws), p.C);
}
__device__ __forceinline__ int slot_offset(const Params& p, int slot) {
    const int u = slot / p.ws, w = slot - u * p.ws;
    return __mul24(__mul24(u, p.W) + w, p.C);
}
__device__ __forceinline__ int token_offset(const Params& p, int reg, int slot) {
    return region_base(p, reg) + slot_offset(p, slot);
}
// The same in the K/V map the attention gathers from (downsampled or not).
__device__ __forceinline__ int region_base_kv(const Params& p, int reg) {
    const int ri = reg / p.n, rj = reg - ri * p.n;
    return __mul24(__mul24(__mul24(ri, p.khs), p.kW) + __mul24(rj, p.kws), p.C);
}
__device__ __forceinline__ int slot_offset_kv(const Params& p, int slot) {
    const int u = slot / p.kws, w = slot - u * p.kws;
    return __mul24(__mul24(u, p.kW) + w, p.C);
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
        // fixed shapes run without KV downsampling
        p.kv_ratio = 1;
        p.kH = p.H;
        p.kW = p.W;
        p.khs = HS;
        p.kws = WS;
        p.kt = HS * WS;
        p.lepe_items = (HEADS * kHeadDim / 2) * HS * ((WS + kLepeCols - 1) / kLepeCols);
        p.lepe_alias = p.lepe_items <= kThreads;
        p.halo_pieces = (HS + 4) * (WS + 4) * (HEADS * kHeadDim / VEC);
    }
    return p;
}

// One entry of the weight table of the MFMA LePE (see lepe_mfma_load): row c
// of the table is channel c's 25 weights w[c][i][j] in tap order (5i + j) as
// bf16, then 7 zeros -- 64 bytes, eight 8-byte entries.  Entry it = 8c + q
// holds taps 4q .. 4q + 3 of channel c.
__device__ __forceinline__ uint2 lepe_table_entry(const float* __restrict__ lepe_w, int it) {
    const int c = it >> 3, q = it & 7;
    // the four loads go out together (clamped tap, always in the row), the
    // taps past the 25th are zeroed afterwards
    float wv[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) wv[kk] = lepe_w[c * 25 + min(4 * q + kk, 24)];
    uint32_t h[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) h[kk] = 4 * q + kk < 25 ? f32_to_bf16(wv[kk]) : 0u;
    return uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// Q_r . K_s over the 32 dims of one head, left to right, each product rounded
// before it is added -- the same IEEE operations as a plain fp64 loop --
// appended to a running sum s0 (s0 = 0 for one head; a longer sequential dot
// over several heads otherwise).
__device__ __forceinline__ double dot32_seq_from(double s0, const double* a, const double* b) {
#pragma clang fp contract(off)
    double s = s0;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) s = s + a[d] * b[d];
    return s;
}

// LePE on the 4x4x4 MFMA applies to windows whose sides are multiples of 4
// when the per-wave accumulators (tiles x channel groups) stay small.
__host__ __device__ constexpr bool lepe_mfma_fits(int hs, int ws, int heads) {
    return hs > 0 && ws > 0 && heads > 0 && hs % 4 == 0 && ws % 4 == 0 &&
           (hs / 4) * (ws / 4) * ((heads * kHeadDim / 16 + kWaves - 1) / kWaves) <= 8;
}

// The channel-planar halo of the MFMA LePE: channel c's (hs + 4) x (ws + 4)
// plane starts at element lepe_plane_offset(c, ps).  The stride and the
// 4-element step per 8 channels spread over the LDS banks both the halo
// writes (the 8 lanes of one cell write channels 8 apart: 2-byte stores for
// 8 x 8 windows, 8-byte stores of 4 cells for 4 x 4) and the 4x4x4 operand
// reads (16 channels x 4 rows per instruction).  The strides come from a
// bank model of those two patterns (32 banks serving 16 lanes, or 64
// serving 32): 8 x 8 windows conflict-free (the unpadded 148 took 4- and
// 2-way conflicts), 4 x 4 writes conflict-free and reads 2-way (68: 8-way
// and 2-way).
__host__ __device__ constexpr int lepe_plane_stride(int hs, int ws) {
    return hs == 8 && ws == 8 ? 176 : hs == 4 && ws == 4 ? 76 : (hs + 4) * (ws + 4) + 4;
}
__host__ __device__ constexpr int lepe_plane_offset(int c, int ps) { return c * ps + 4 * (c >> 3); }

template <int HS, int WS, int HEADS>
struct LepeMfmaShape {
    static constexpr int C = HEADS * kHeadDim;
    static constexpr int TY = HS / 4, TX = WS / 4;
    static constexpr int HWP = WS + 4;                    // halo row pitch (elements)
    static constexpr int PS = lepe_plane_stride(HS, WS);  // channel plane stride (elements)
    static constexpr int NG = C / 16;                     // groups of 16 channels
    static constexpr int GPW = (NG + kWaves - 1) / kWaves;  // groups per wave
    static constexpr bool ok = lepe_mfma_fits(HS, WS, HEADS);
};

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
// Sum of x over the 16 lanes of each DPP row (partners lane ^ 1, lane ^ 2,
// the other quad, the other half); every lane of the row ends with the same
// value.  For exact sums only, where the pairing cannot change the result:
// fp64 sums of the t bf16 values of one (region, channel).  Those are
// multiples of the smallest nonzero value's last significand bit, so while
// the nonzero values span at most 2^(45 - ceil(log2 t)) in magnitude every
// partial sum is an integer number of those units below 2^53, exact in
// fp64, and every order of the additions gives the slot-order sum.  Wider
// spans may round differently (include/bra.h states the condition).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const int2 u = __builtin_bit_cast(int2, x);
    int2 o;
    o.x = __builtin_amdgcn_mov_dpp(u.x, CTRL, 0xf, 0xf, false);
    o.y = __builtin_amdgcn_mov_dpp(u.y, CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, o);
}
__device__ __forceinline__ double row16_sum_exact(double x) {
    x += dpp_f64<0xB1>(x);
    x += dpp_f64<0x4E>(x);
    x += dpp_f64<0x141>(x);
    x += dpp_f64<0x140>(x);
    return x;
}
// x of lane ^ J (J = 1, 2, 4, 8) by DPP row permutations: quad_perm for 1
// and 2; for 4, the quad reversal (lane ^ 3) after row_half_mirror (lane ^ 7);
// for 8, row_mirror (lane ^ 15) after row_half_mirror.
template <int J>
__device__ __forceinline__ int lane_xor_dpp(int x) {
    static_assert(J == 1 || J == 2 || J == 4 || J == 8, "DPP partners within a row of 16");
    if constexpr (J == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false);
    if constexpr (J == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false);
    const int m7 = __builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false);
    if constexpr (J == 4) return __builtin_amdgcn_mov_dpp(m7, 0x1B, 0xf, 0xf, false);
    return __builtin_amdgcn_mov_dpp(m7, 0x140, 0xf, 0xf, false);
}
// Maximum over the wave (every lane ends with it), non-NaN values: DPP
// within rows of 16, then the row swaps of group4_max.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max_f32(float x) {
    x = max_f(x, dpp_f32<0xB1>(x));   // lane ^ 1
    x = max_f(x, dpp_f32<0x4E>(x));   // lane ^ 2
    x = max_f(x, dpp_f32<0x141>(x));  // the other quad of 8
    x = max_f(x, dpp_f32<0x140>(x));  // the other 8 of 16
    return group4_max(x);
}
// Lane `src`'s x, wave-uniform.
__device__ __forceinline__ double readlane_f64(double x, int src) {
    const int2 u = __builtin_bit_cast(int2, x);
    return __builtin_bit_cast(double, int2{__builtin_amdgcn_readlane(u.x, src),
                                           __builtin_amdgcn_readlane(u.y, src)});
}
// dot32_seq_from(0, a, b) with a spread over lanes: lane d holds a[d].
__device__ __forceinline__ double dot32_seq_lanes(double a_lane, const double (&b)[kHeadDim]) {
#pragma clang fp contract(off)
    double s = 0.0;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) s = s + readlane_f64(a_lane, d) * b[d];
    return s;
}

__device__ __forceinline__ void wave_argmax(double& best, int& bs) {
    argmax_dpp<0xB1>(best, bs);   // quad_perm [1,0,3,2]: lane ^ 1
    argmax_dpp<0x4E>(best, bs);   // quad_perm [2,3,0,1]: lane ^ 2
    argmax_dpp<0x141>(best, bs);  // row_half_mirror: the other quad of 8
    argmax_dpp<0x140>(best, bs);  // row_mirror: the other 8 of 16
    argmax_swap<true>(best, bs);
    argmax_swap<false>(best, bs);
}

// (a, ia) ranks before (b, ib): a larger value, or an equal one with a lower
// id.  Bitwise, not short-circuit: no branch per comparison.
__device__ __forceinline__ bool beats(double a, int ia, double b, int ib) {
    return (a > b) | ((a == b) & (ia < ib));
}

// ---------------------------------------------------------------------------
// Bitonic sort of NRW rows at once, best first (affinity descending, region
// id ascending), for the top-k selections of the routing.  Lane `lane` holds elements lane * E .. lane * E + E - 1 of
// every row; partners within a lane swap in registers, partners across lanes
// come from DPP (lane ^ 1 .. lane ^ 8) or a permlane swap (lane ^ 16, ^ 32).
// Padding elements (ids >= R) carry -inf and sort last.

// This lane's pair {own, partner at lane ^ LJ} as (a, ia), (b, ib); the
// permlane swaps return the two in an order that depends on the lane, which
// a compare-exchange does not need.
template <int LJ>
__device__ __forceinline__ void lane_pair(double v, int ix, double& a, int& ia, double& b,
                                          int& ib) {
    const int2 u = __builtin_bit_cast(int2, v);
    if constexpr (LJ < 16) {
        a = v;
        ia = ix;
        b = __builtin_bit_cast(double, int2{lane_xor_dpp<LJ>(u.x), lane_xor_dpp<LJ>(u.y)});
        ib = lane_xor_dpp<LJ>(ix);
    } else {
        const auto lo = LJ == 16 ? __builtin_amdgcn_permlane16_swap(u.x, u.x, false, false)
                                 : __builtin_amdgcn_permlane32_swap(u.x, u.x, false, false);
        const auto hi = LJ == 16 ? __builtin_amdgcn_permlane16_swap(u.y, u.y, false, false)
                                 : __builtin_amdgcn_permlane32_swap(u.y, u.y, false, false);
        const auto ii = LJ == 16 ? __builtin_amdgcn_permlane16_swap(ix, ix, false, false)
                                 : __builtin_amdgcn_permlane32_swap(ix, ix, false, false);
        a = __builtin_bit_cast(double, int2{static_cast<int>(lo[0]), static_cast<int>(hi[0])});
        ia = static_cast<int>(ii[0]);
        b = __builtin_bit_cast(double, int2{static_cast<int>(lo[1]), static_cast<int>(hi[1])});
        ib = static_cast<int>(ii[1]);
    }
}

// One half-cleaner step of distance J inside bitonic blocks of SIZE
// elements, then the steps J/2 .. 1.  Position i keeps the better of the
// pair when (i & J) == 0 and (i & SIZE) == 0 agree, else the worse.
template <int E, int NRW, int SIZE, int J>
__device__ __forceinline__ void bitonic_steps(double (&v)[NRW][E], int (&ix)[NRW][E], int lane) {
    if constexpr (J < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int pe = e ^ J;
            if (pe > e) {
                const bool dir = ((lane * E + e) & SIZE) == 0;
#pragma unroll
                for (int r = 0; r < NRW; ++r) {
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
        constexpr int LJ = J / E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = lane * E + e;
            const bool keep_better = ((i & J) == 0) == ((i & SIZE) == 0);
#pragma unroll
            for (int r = 0; r < NRW; ++r) {
                double a, b;
                int ia, ib;
                lane_pair<LJ>(v[r][e], ix[r][e], a, ia, b, ib);
                const bool take_a = beats(a, ia, b, ib) == keep_better;
                v[r][e] = take_a ? a : b;
                ix[r][e] = take_a ? ia : ib;
            }
        }
    }
    if constexpr (J > 1) bitonic_steps<E, NRW, SIZE, J / 2>(v, ix, lane);
}

template <int E, int NRW, int SIZE>
__device__ __forceinline__ void bitonic_sort(double (&v)[NRW][E], int (&ix)[NRW][E], int lane) {
    bitonic_steps<E, NRW, SIZE, SIZE / 2>(v, ix, lane);
    if constexpr (SIZE < 64 * E) bitonic_sort<E, NRW, SIZE * 2>(v, ix, lane);
}

// ---------------------------------------------------------------------------
// The same network on fp32 keys alone (equal keys in any order): a lane
// moves two dwords per partner instead of three, and a compare-exchange is
// one compare and two selects instead of three compares and three selects.
template <int LJ>
__device__ __forceinline__ void lane_pair_f32(float v, int ix, float& a, int& ia, float& b,
                                              int& ib) {
    if constexpr (LJ < 16) {
        a = v;
        ia = ix;
        b = __int_as_float(lane_xor_dpp<LJ>(__float_as_int(v)));
        ib = lane_xor_dpp<LJ>(ix);
    } else {
        const auto vv = LJ == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v),
                                                                    __float_as_uint(v), false,
                                                                    false)
                                 : __builtin_amdgcn_permlane32_swap(__float_as_uint(v),
                                                                    __float_as_uint(v), false,
                                                                    false);
        const auto ii = LJ == 16 ? __builtin_amdgcn_permlane16_swap(ix, ix, false, false)
                                 : __builtin_amdgcn_permlane32_swap(ix, ix, false, false);
        a = __uint_as_float(vv[0]);
        ia = static_cast<int>(ii[0]);
        b = __uint_as_float(vv[1]);
        ib = static_cast<int>(ii[1]);
    }
}

template <int E, int NRW, int SIZE, int J>
__device__ __forceinline__ void bitonic_steps_f32(float (&v)[NRW][E], int (&ix)[NRW][E],
                                                  int lane) {
    if constexpr (J < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int pe = e ^ J;
            if (pe > e) {
                const bool dir = ((lane * E + e) & SIZE) == 0;
#pragma unroll
                for (int r = 0; r < NRW; ++r) {
                    if ((v[r][e] > v[r][pe]) != dir) {
                        const float tv = v[r][e];
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
        constexpr int LJ = J / E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = lane * E + e;
            const bool keep_better = ((i & J) == 0) == ((i & SIZE) == 0);
#pragma unroll
            for (int r = 0; r < NRW; ++r) {
                float a, b;
                int ia, ib;
                lane_pair_f32<LJ>(v[r][e], ix[r][e], a, ia, b, ib);
                const bool take_a = (a > b) == keep_better;
                v[r][e] = take_a ? a : b;
                ix[r][e] = take_a ? ia : ib;
            }
        }
    }
    if constexpr (J > 1) bitonic_steps_f32<E, NRW, SIZE, J / 2>(v, ix, lane);
}

template <int E, int NRW, int SIZE>
__device__ __forceinline__ void bitonic_sort_f32(float (&v)[NRW][E], int (&ix)[NRW][E],
                                                 int lane) {
    bitonic_steps_f32<E, NRW, SIZE, SIZE / 2>(v, ix, lane);
    if constexpr (SIZE < 64 * E) bitonic_sort_f32<E, NRW, SIZE * 2>(v, ix, lane);
}

// The k best entries of NRW rows, best first, exactly as bitonic_sort would
// order them (fp64 value descending, exact ties to the lower id): ix[r][e]
// holds the id at position lane * E + e.  The rows are first sorted on fp32
// keys (round-to-nearest is monotone).  If in every row the fp32 keys of
// positions 0 .. k are strictly decreasing (position k when it exists), the
// fp64 values are too, and every entry past position k - 1 has a smaller
// fp32 key -- hence a smaller fp64 value -- than every entry before: that
// order is the exact one.  Otherwise (fp64 values that round to one fp32
// key, exact ties) the rows are sorted again on the fp64 values and ids.
template <int E, int NRW>
__device__ __forceinline__ void route_topk(double (&v)[NRW][E], int (&ix)[NRW][E], int lane,
                                           int k) {
    float f[NRW][E];
    int fx[NRW][E];
#pragma unroll
    for (int r = 0; r < NRW; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            f[r][e] = static_cast<float>(v[r][e]);
            fx[r][e] = ix[r][e];
        }
    bitonic_sort_f32<E, NRW, 2>(f, fx, lane);
    bool bad = false;
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
        // position lane * E + E is lane + 1's first entry
        const float after = __shfl_down(f[r][0], 1);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = lane * E + e;
            const float next = e + 1 < E ? f[r][e + 1] : after;
            if (j < k && j + 1 < 64 * E && !(f[r][e] > next)) bad = true;
        }
    }
    if (__ballot(bad) != 0ull) {  // wave-uniform
        bitonic_sort<E, NRW, 2>(v, ix, lane);
    } else {
#pragma unroll
        for (int r = 0; r < NRW; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) ix[r][e] = fx[r][e];
    }
}

// ---------------------------------------------------------------------------
// Routing of one (image, head, query region) row on one wave, R <= 64
// [P4 §1.2; P1 §2.1 TopkRouting; P5 §五 ③-④].  Lane d (and d + 32) holds dim
// d of the row's Q mean, read back wave-uniform; lane s routes region s.  The
// result is the one of the fp64 affinities A[s] (sequential 32-term fp64 sum
// of dot32_seq_lanes): affinity descending, exact ties to the lower id.
//  1. Screen: lane s holds the fp32 K mean of region s (kf) and forms
//     a[s] = sum of fp32 products, with a bound on |a[s] - A[s]|.  Rounding
//     the means to fp32 moves each product by at most 2u of its size
//     (u = 2^-24), the 32 fused multiply-adds add at most 32u of the sum of
//     |products| S, and the fp64 sum is within 2^-47 S of the exact one: 35u
//     of S in the normal range.  With S <= Q K1 (Q = max |q_d|, K1 = sum
//     |k_d|), the bound taken is e = 2^-18 Q K1 (64u) plus 2^-120 (K1 + 32 Q
//     + 64), which also covers the fp32 subnormal range (at most 2^-150 per
//     rounding there); E is e at the row's largest K1.  Two fp32 values more
//     than 2E apart order the fp64 affinities the same way.
//     k = 1: if one region alone lies within 2E of the fp32 maximum, it is
//     the fp64 arg-max.  k > 1: the fp32 values are sorted (bitonic, in
//     registers); if each of ranks 0 .. k-1 exceeds the next rank by more
//     than 2E, the fp64 order of the first k and the set below them agree.
//  2. Otherwise (near or exact ties, or a non-finite value or bound): the
//     fp64 K means are read and the exact pass decides -- a wave arg-max, or
//     route_topk.
// Writes each routed region's base offset to off[rank] (LDS) and its id to
// out[rank] (a global or an LDS array).
// kreg holds the fp32 K mean as load_kmean32 leaves it when screening;
// without the fp32 means (p.kmean32 = 0) it holds the fp64 K mean and only
// the exact pass runs.
__device__ __forceinline__ void route_row_wave(const Params& p, double qmean_lane, bool screen,
                                               double (&kreg)[kHeadDim],
                                               const double* __restrict__ means, int bh,
                                               int* off, int32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const bool in = lane < p.R;
    if (screen) {
        float a = 0.f, k1 = 0.f;
        const float ql = static_cast<float>(qmean_lane);
#pragma unroll
        for (int d = 0; d < kHeadDim; ++d) {
            const float qd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ql), d));
            const float kd = __uint_as_float(__builtin_bit_cast(u32x2_t, kreg[d >> 1])[d & 1]);
            a = fmaf(qd, kd, a);
            k1 += fabsf(kd);
        }
        const bool finite = __builtin_isfinite(a) && __builtin_isfinite(k1);
        const bool screened = __ballot(in && !finite) == 0ull;
        const float qinf = wave_max_f32(fabsf(ql));  // lanes d and d + 32 hold dim d
        const float k1max = wave_max_f32(in ? k1 : 0.f);
        // e = (2^-18 Q + 2^-120) K1 + (32 Q + 64) 2^-120, increasing in K1
        const float band =
            2.f * ((qinf * 0x1p-18f + 0x1p-120f) * k1max + (32.f * qinf + 64.f) * 0x1p-120f);
        if (p.k == 1) {
            const float mx = wave_max_f32(in ? a : -INFINITY);
            const unsigned long long near = __ballot(in && !(a < mx - band));
            if (screened && __popcll(near) == 1) {
                if (lane == 0) {
                    const int bs = __ffsll(static_cast<long long>(near)) - 1;
                    off[0] = region_base_kv(p, bs);
                    out[0] = bs;
                }
                return;
            }
        } else {
            float f[1][1] = {{in ? a : -INFINITY}};
            int fx[1][1] = {{lane}};
            bitonic_sort_f32<1, 1, 2>(f, fx, lane);
            const float next = __shfl_down(f[0][0], 1);
            const bool bad = lane < p.k && lane + 1 < p.R && !(f[0][0] - next > band);
            if (screened && __ballot(bad) == 0ull) {
                if (lane < p.k) {
                    const int id = min(max(fx[0][0], 0), p.R - 1);
                    off[lane] = region_base_kv(p, id);
                    out[lane] = id;
                }
                return;
            }
        }
        // the exact pass needs the fp64 means (wave-uniform branch)
        load_kmean(p, means, bh, min(lane, p.R - 1), kreg);
    }
    const double ad = dot32_seq_lanes(qmean_lane, kreg);
    // (Non-finite affinities leave the routing undefined, but every offset
    // the gather uses stays inside the map: the ids are clamped.)
    if (p.k == 1) {
        double best = in ? ad : -INFINITY;
        int bs = in ? lane : 0x7fffffff;
        wave_argmax(best, bs);
        if (lane == 0) {
            bs = min(max(bs, 0), p.R - 1);
            off[0] = region_base_kv(p, bs);
            out[0] = bs;
        }
    } else {
        double v[1][1] = {{in ? ad : -INFINITY}};
        int ix[1][1] = {{lane}};
        route_topk<1, 1>(v, ix, lane, p.k);
        if (lane < p.k) {
            const int id = min(max(ix[0][0], 0), p.R - 1);
            off[lane] = region_base_kv(p, id);
            out[lane] = id;
        }
    }
}

}  // namespace bra
