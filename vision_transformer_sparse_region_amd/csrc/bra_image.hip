// bra_image.hip -- the whole BRA forward of one (image, head group) in one
// workgroup, for maps whose group K and V fit the 160 KB of LDS of a gfx950
// CU (BiFormer stages 2 and 3: 28 x 28 and 14 x 14 maps of 7 x 7 regions)
// (page keys in bra_device.h).
//
// A workgroup of 16 waves owns image b and heads hg*HG .. hg*HG + HG - 1:
//   1  the group's K slice of the whole map and the Q operands of the
//      wave's jobs, all at once into registers, then to LDS token-major as
//      they arrive; the V slice loads once they are in     [P5 §五 ⑤]
//   2  the K and Q region means: slot-order fp64 sums of the staged K and Q
//      (the oracle's operations)            [P4 §1.2; P2 §2.1; P5 §五 ③]
//   3  routing, four lanes per query row: the fp64 MFMA forms the affinities
//      of 16 rows with 16 regions at a time (lane j of each row of 16 lanes
//      then holds 16 regions of row j), each affinity becomes a 32-bit key
//      (26-bit fixed point over the row's range, region id in the low 6
//      bits), a lane sorts its 16 keys and the row's four lanes merge their
//      lists to the top 16.  Keys whose fixed-point parts are at least G
//      apart order the exact sequential fp64 affinities the same way (G
//      covers the fixed point and the gap between the MFMA's sums and the
//      sequential ones); rows whose k + 1 leading keys are not that far
//      apart are routed again exactly, a wave per row, on the sequential
//      fp64 affinities                       [P1 §2.1 TopkRouting; P5 §五 ④]
//   3b V goes to LDS channel-planar with a 2-cell zero border in x (the
//      LePE halo of the whole map is that border), written by the waves
//      that do not route while the others route
//   4  each job -- one 4 x 4 token tile of one head: one region of 4 x 4
//      tokens, or four regions of 2 x 2 -- runs the 5 x 5 depthwise LePE of
//      the tile on the 4x4x4 MFMA from the planar V, the token attention
//      over the routed K/V gathered from LDS on the 16x16x32 bf16 MFMA, and
//      stores LePE + O through a wave-private LDS tile as 16-byte rows
//                                       [P3 §2.2; P5 §五 ⑤-⑧; P2 §2.2]
// Nothing but q, k, v, the weights and the output crosses HBM: every gather
// and the halo come from LDS, so each byte of q, k and v is read once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_image.h"

namespace bra {
namespace img {

constexpr int kImgThreads = kImgWaves * 64;

template <int HS_, int NW_, int HG_, int HEADS_, int KTOP_>
struct ImgShape {
    static constexpr int HS = HS_, NW = NW_, HG = HG_, HEADS = HEADS_, KTOP = KTOP_;
    static constexpr ImgGeo geo = img_geo(HS, NW, HG, HEADS, KTOP);
    static constexpr int H = NW * HS, W = H, N = H * W, R = NW * NW, T = HS * HS;
    static constexpr int C = HEADS * kHeadDim, CG = HG * kHeadDim, NGRP = HEADS / HG;
    static constexpr int PCT = CG / 8;            // 16-byte pieces of a token in the group
    static constexpr int TS = geo.ts;             // 4 x 4 tiles per map side
    static constexpr int TPH = TS * TS;           // jobs per head
    static constexpr int JOBS = HG * TPH;
    static constexpr int JPW = (JOBS + kImgWaves - 1) / kImgWaves;
    static constexpr int RPS = 4 / HS;            // regions per tile side
    static constexpr int RPT = RPS * RPS;         // regions per tile
    static constexpr int NKEYS = KTOP * T;
    static constexpr int NPAIR = (NKEYS + 63) / 64;
    static constexpr int PW = geo.pw;             // plane row pitch (elements)
    static constexpr int PS = geo.ps;             // plane stride (elements)
    static constexpr int RS = geo.rs;             // K map row stride (elements)
    static constexpr int QS = geo.qs;             // region-mean row stride (doubles)
    static constexpr int NPK = N * PCT;           // 16-byte pieces of the K slice
    static constexpr int KR = (NPK + kImgThreads - 1) / kImgThreads;
    static constexpr int PPH = (R + 15) / 16;     // routing passes per head (16 rows each)
    static constexpr int PASSES = HG * PPH;
    static constexpr int NT = (R + 15) / 16;      // 16-region tiles of the affinity
    static constexpr int ROWS = HG * R;
    static constexpr int RI = (HG * R * KTOP + kImgThreads - 1) / kImgThreads;
    static constexpr int NCH = 2 * NPAIR;         // 32-key chunks (pairs of)
    static constexpr int GXN = PW / 4;            // 4-cell column groups of a plane row
    static constexpr int NVT = PCT * H * GXN;     // V staging tasks
    static constexpr int NTE = CG * 40;           // Toeplitz entries
    static_assert(HS == 2 || HS == 4, "4 x 4 tiles of whole regions");
    static_assert(R <= 64 && KTOP <= 16 && KTOP >= 1, "quad routing: R <= 64, k <= 16");
    static_assert(NT <= 4, "16 keys per lane");
    static_assert(HEADS % HG == 0, "whole head groups");
    static_assert(RS % 8 == 0, "16-byte rows");
    static_assert(PASSES < kImgWaves, "waves left to stage V while the others route");
};

// 26-bit fixed point keys: region id in the low 6 bits (63 - id, so that the
// larger key wins an exact tie of the fixed-point part for the lower id).
constexpr double kKeySpan = 67108861.0;  // 2^26 - 3: values 1 .. 2^26 - 2

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Bitonic sort of 16 keys held by one lane, largest first.
__device__ __forceinline__ void sort16_desc(uint32_t (&x)[16]) {
#pragma unroll
    for (int size = 2; size <= 16; size *= 2)
#pragma unroll
        for (int j = size / 2; j > 0; j /= 2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    const uint32_t a = x[i], b = x[l];
                    if ((i & size) == 0) {
                        x[i] = umax32(a, b);
                        x[l] = umin32(a, b);
                    } else {
                        x[i] = umin32(a, b);
                        x[l] = umax32(a, b);
                    }
                }
            }
}

// The 16 largest of this lane's sorted list and that of lane ^ XOR, sorted;
// `drop` becomes the largest key left out (with its own earlier value and
// the partner's).  Both lanes end with the same list.
template <int XOR>
__device__ __forceinline__ void merge16(uint32_t (&x)[16], uint32_t& drop) {
    uint32_t p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        p[i] = static_cast<uint32_t>(__shfl_xor(static_cast<int>(x[15 - i]), XOR));
    uint32_t d = umax32(drop, static_cast<uint32_t>(__shfl_xor(static_cast<int>(drop), XOR)));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        d = umax32(d, umin32(x[i], p[i]));
        x[i] = umax32(x[i], p[i]);
    }
    drop = d;
    // x is bitonic: the merge half of a bitonic sort
#pragma unroll
    for (int j = 8; j > 0; j /= 2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int l = i ^ j;
            if (l > i) {
                const uint32_t a = x[i], b = x[l];
                x[i] = umax32(a, b);
                x[l] = umin32(a, b);
            }
        }
}

__device__ __forceinline__ uint32_t pick4(const uint32_t (&x)[16], int q, int m) {
    // x[4m + q] with q lane-dependent (0..3)
    const uint32_t a = x[4 * m], b = x[4 * m + 1], c = x[4 * m + 2], d = x[4 * m + 3];
    return q == 0 ? a : q == 1 ? b : q == 2 ? c : d;
}

// Workgroup barrier that orders LDS only: the fences carry the "local"
// address-space tag, so the compiler does not make the waves wait for their
// outstanding global loads (the V slice, which is consumed later) here.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename S>
struct ImgLds {
    uint16_t* sK;       // [H][RS] K of the group, token-major, a padded row per map row
    double* sKbar;      // [HG][R][QS] K region means
    double* sQbar;      // [HG][R][QS] Q region means
    float* sStage;      // [kImgWaves][16][36] output tiles (over the means)
    uint16_t* sVp;      // [CG][PS] channel-planar V, rows of PW with a 2-cell border
    uint16_t* sQs;      // [H][RS] staged Q, over the V planes (until the means)
    uint2* sTab;        // [CG / 16][64][10] Toeplitz B operands of the MFMA LePE
    float* sBias;       // [CG]
    int* sOffK;         // [HG][R][KTOP] routed regions: K element offset of the first token
    int* sOffV;         // [HG][R][KTOP] routed regions: V plane offset of the first cell
    int* sRegK;         // [R] K element offset of each region's first token
    int* sRegV;         // [R] V plane offset of each region's first cell
    uint16_t* sZero;    // 8 zero elements
    unsigned* sKinf;    // [HG] max |K mean| (float bits)
    int* sNFail;        // rows to route exactly, and their list
    int* sFail;
    __device__ ImgLds(unsigned char* smem) {
        constexpr ImgGeo g = S::geo;
        sK = reinterpret_cast<uint16_t*>(smem + g.off_k);
        sKbar = reinterpret_cast<double*>(smem + g.off_over);
        sQbar = sKbar + S::HG * S::R * S::QS;
        sStage = reinterpret_cast<float*>(smem + g.off_over);
        sVp = reinterpret_cast<uint16_t*>(smem + g.off_vp);
        sQs = sVp;
        sTab = reinterpret_cast<uint2*>(smem + g.off_tab);
        sBias = reinterpret_cast<float*>(smem + g.off_bias);
        sOffK = reinterpret_cast<int*>(smem + g.off_offk);
        sOffV = reinterpret_cast<int*>(smem + g.off_offv);
        sRegK = reinterpret_cast<int*>(smem + g.off_regk);
        sRegV = reinterpret_cast<int*>(smem + g.off_regv);
        sZero = reinterpret_cast<uint16_t*>(smem + g.off_misc);
        sKinf = reinterpret_cast<unsigned*>(smem + g.off_misc + 16);
        sNFail = reinterpret_cast<int*>(smem + g.off_misc + 16 + 4 * S::HG);
        sFail = sNFail + 1;
    }
};

// Element offset in sK (or sQs) of token (y, x).
template <typename S>
__device__ __forceinline__ int kofs(int y, int x) {
    return y * S::RS + x * S::CG;
}
// ... of slot u of region s.
template <typename S>
__device__ __forceinline__ int region_kofs(int s, int u) {
    return kofs<S>((s / S::NW) * S::HS + u / S::HS, (s % S::NW) * S::HS + u % S::HS);
}

// Records region id `id` as rank j of row (hl, r): its K and V offsets for
// the gathers.
template <typename S>
__device__ __forceinline__ void put_route(const ImgLds<S>& L, int hl, int r, int j, int id) {
    const int e = (hl * S::R + r) * S::KTOP + j;
    L.sOffK[e] = L.sRegK[id];
    L.sOffV[e] = L.sRegV[id];
}

// Region means of the staged K and Q maps ([H][RS] each), both in one pass:
// item (tensor, head hl, region s, dims DPI o .. DPI o + DPI - 1) reads the
// region's slots as 16- or 8-byte pieces and adds each dim's values in slot
// order, as the oracle does.  DPI is 4 where the items of 4 dims still fit
// one a thread (16-token regions: half the chain of 8-dim items), else 8.
// Returns the max |K mean| of the thread's items.
template <typename S>
__device__ __forceinline__ float region_means_kq(const uint16_t* sK, const uint16_t* sQ,
                                                 double* sKbar, double* sQbar) {
    constexpr int NHR = S::HG * S::R;
    constexpr int DPI = 2 * NHR * (kHeadDim / 4) <= kImgThreads ? 4 : 8;
    constexpr int IPR = kHeadDim / DPI, NI = 2 * NHR * IPR;
    float mx = 0.f;
#pragma unroll
    for (int u = 0; u < (NI + kImgThreads - 1) / kImgThreads; ++u) {
        const int item = threadIdx.x + u * kImgThreads;
        if (item < NI) {
            const int o = item % IPR, rest = item / IPR;
            const int tensor = rest >= NHR ? 1 : 0, hs = rest - tensor * NHR;
            const int hl = hs / S::R, s = hs - hl * S::R;
            const uint16_t* src = (tensor ? sQ : sK) + hl * kHeadDim + DPI * o;
            double acc[DPI];
#pragma unroll
            for (int e = 0; e < DPI; ++e) acc[e] = 0.0;
#pragma unroll
            for (int uu = 0; uu < S::T; ++uu) {
                uint32_t x[DPI / 2];
                if constexpr (DPI == 8) {
                    const uint4 v4 = *reinterpret_cast<const uint4*>(src + region_kofs<S>(s, uu));
                    x[0] = v4.x;
                    x[1] = v4.y;
                    x[2] = v4.z;
                    x[3] = v4.w;
                } else {
                    const uint2 v2 = *reinterpret_cast<const uint2*>(src + region_kofs<S>(s, uu));
                    x[0] = v2.x;
                    x[1] = v2.y;
                }
#pragma unroll
                for (int e = 0; e < DPI / 2; ++e) {
                    acc[2 * e] += bf16lo(x[e]);
                    acc[2 * e + 1] += bf16hi(x[e]);
                }
            }
            double* dst = (tensor ? sQbar : sKbar) + (hl * S::R + s) * S::QS + DPI * o;
#pragma unroll
            for (int e = 0; e < DPI; ++e) {
                const double m = mean_of(acc[e], S::T);
                dst[e] = m;
                if (!tensor) mx = fmaxf(mx, static_cast<float>(fabs(m)));
            }
        }
    }
    return mx;
}

// Routing of the group's rows (see the file header).  Pass p covers rows
// r0 .. r0 + 15 of head hl; lane (j = lane % 16, grp = lane / 16) holds the
// affinities of row r0 + j with regions 16t + grp + 4e (the fp64 MFMA's
// output layout).  Rows the keys cannot decide are left to route_exact.
template <typename S>
__device__ __forceinline__ void route_rows(const ImgLds<S>& L, int b, int hg,
                                           int32_t* __restrict__ routing) {
    typedef double d4_t __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int j = lane & 15, grp = lane >> 4;
    for (int pass = w; pass < S::PASSES; pass += kImgWaves) {
        const int hl = pass / S::PPH, r0 = (pass - hl * S::PPH) * 16;
        const int r = r0 + j;
        const bool row_ok = r < S::R;
        const double* qrow = L.sQbar + (hl * S::R + min(r, S::R - 1)) * S::QS + grp;
        const double* kbase = L.sKbar + hl * S::R * S::QS + grp;
        d4_t acc[S::NT];
#pragma unroll
        for (int t = 0; t < S::NT; ++t) acc[t] = d4_t{0.0, 0.0, 0.0, 0.0};
        double q1 = 0.0;
#pragma unroll
        for (int k = 0; k < kHeadDim / 4; ++k) {
            const double bq = qrow[4 * k];
            q1 += fabs(bq);
#pragma unroll
            for (int t = 0; t < S::NT; ++t) {
                const double ka = kbase[min(16 * t + j, S::R - 1) * S::QS + 4 * k];
                acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(ka, bq, acc[t], 0, 0, 0);
            }
        }
        q1 += __shfl_xor(q1, 16);
        q1 += __shfl_xor(q1, 32);
        // row range over the valid regions
        double amax = -INFINITY, amin = INFINITY;
#pragma unroll
        for (int t = 0; t < S::NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (16 * t + grp + 4 * e < S::R) {
                    amax = fmax(amax, acc[t][e]);
                    amin = fmin(amin, acc[t][e]);
                }
        amax = fmax(amax, __shfl_xor(amax, 16));
        amax = fmax(amax, __shfl_xor(amax, 32));
        amin = fmin(amin, __shfl_xor(amin, 16));
        amin = fmin(amin, __shfl_xor(amin, 32));
        const double range = amax - amin;
        // |MFMA sum - sequential sum| <= 65 u sum_d |q_d k_d| <= 2^-47 Q1 Kinf
        // (each within 33 u of the exact dot); beta = 2^-45 Q1 Kinf, plus an
        // allowance for the subnormal range
        const double kinf = static_cast<double>(__uint_as_float(L.sKinf[hl]));
        const double beta = 0x1p-45 * q1 * kinf + 0x1p-1000;
        const double scale = kKeySpan / range;
        const double quantum = range / kKeySpan;
        const double gq = 2.0 * beta / quantum;
        // keys differing by at least G in their fixed-point parts are more
        // than 2 beta apart in the MFMA affinities (2 units cover the
        // truncation and the rounding of (a - amin) * scale)
        const bool range_ok = range > 0.0 && range < INFINITY && gq < 1.0e6;
        const uint32_t G = range_ok ? 3u + static_cast<uint32_t>(ceil(gq)) : 0xffffffffu;
        uint32_t x[16];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * t + grp + 4 * e;
                if (t < S::NT && s < S::R) {
                    const double f = range_ok ? (acc[t < S::NT ? t : 0][e] - amin) * scale : 0.0;
                    const uint32_t u = 1u + static_cast<uint32_t>(f);
                    x[4 * t + e] = (u << 6) | static_cast<uint32_t>(63 - s);
                } else {
                    x[4 * t + e] = 0u;
                }
            }
        sort16_desc(x);
        uint32_t drop = 0u;
        merge16<16>(x, drop);
        merge16<32>(x, drop);
        // ranks 0 .. k (or all R) must be G apart
        constexpr int NCHK = S::KTOP < S::R ? S::KTOP : S::R - 1;
        bool ok = range_ok;
#pragma unroll
        for (int jj = 0; jj < NCHK; ++jj) {
            const uint32_t nx = jj + 1 < 16 ? x[jj + 1] : drop;
            ok = ok && (x[jj] >> 6) >= (nx >> 6) + G;
        }
        if (row_ok) {
            if (ok) {
                int32_t* gout = routing +
                                ((static_cast<size_t>(b) * S::HEADS + hg * S::HG + hl) * S::R + r) *
                                    S::KTOP;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int rank = 4 * m + grp;
                    if (rank < S::KTOP) {
                        const uint32_t key = pick4(x, grp, m);
                        const int id = min(max(63 - static_cast<int>(key & 63u), 0), S::R - 1);
                        put_route<S>(L, hl, r, rank, id);
                        gout[rank] = id;
                    }
                }
            } else if (grp == 0) {
                const int slot = atomicAdd(L.sNFail, 1);
                L.sFail[slot] = hl * S::R + r;
            }
        }
    }
}

// Exact routing of the rows route_rows could not decide, a wave per row:
// lane s forms the sequential fp64 affinity (the oracle's operations), then
// the exact bitonic sort (value descending, ties to the lower id).
template <typename S>
__device__ __forceinline__ void route_exact(const ImgLds<S>& L, int b, int hg,
                                            int32_t* __restrict__ routing) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nf = *L.sNFail;
    for (int i = w; i < nf; i += kImgWaves) {
        const int row = L.sFail[i];
        const int hl = row / S::R, r = row - hl * S::R;
        const int s = min(lane, S::R - 1);
        const double* qrow = L.sQbar + (hl * S::R + r) * S::QS;
        const double* kb = L.sKbar + (hl * S::R + s) * S::QS;
        double acc;
        {
#pragma clang fp contract(off)
            acc = 0.0;
#pragma unroll
            for (int d = 0; d < kHeadDim; ++d) acc = acc + qrow[d] * kb[d];
        }
        double v[1][1] = {{lane < S::R ? acc : -INFINITY}};
        int ix[1][1] = {{lane}};
        bitonic_sort<1, 1, 2>(v, ix, lane);
        if (lane < S::KTOP) {
            const int id = min(max(ix[0][0], 0), S::R - 1);
            put_route<S>(L, hl, r, lane, id);
            routing[((static_cast<size_t>(b) * S::HEADS + hg * S::HG + hl) * S::R + r) * S::KTOP +
                    lane] = id;
        }
    }
}

// V staging task `task` = (piece pv, map row y, column group gx): the four
// map cells 4gx - 2 .. 4gx + 1 of row y (clamped into the map; bit jj of
// the returned mask says cell jj is inside it).
template <typename S>
__device__ __forceinline__ unsigned load_vtask(const uint16_t* __restrict__ v, size_t img, int task,
                                               uint4 (&vr)[4]) {
    const int t = min(task, S::NVT - 1);
    const int pv = t % S::PCT, rest = t / S::PCT;
    const int gx = rest % S::GXN, y = rest / S::GXN;
    unsigned valid = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int x = 4 * gx + jj - 2, xc = min(max(x, 0), S::W - 1);
        vr[jj] = *reinterpret_cast<const uint4*>(v + img + static_cast<size_t>(y * S::W + xc) * S::C +
                                                 8 * pv);
        if (x == xc) valid |= 1u << jj;
    }
    return task < S::NVT ? valid : 0u;
}

// ... writes it to plane columns 4gx .. 4gx + 3 of the 8 channel planes of
// piece pv (the cells outside the map as zeros).
template <typename S>
__device__ __forceinline__ void store_vtask(const ImgLds<S>& L, int task, const uint4 (&vr)[4],
                                            unsigned valid) {
    if (task >= S::NVT) return;
    const int pv = task % S::PCT, rest = task / S::PCT;
    const int gx = rest % S::GXN, y = rest / S::GXN;
    uint32_t wd[4][4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const unsigned mk = 0u - ((valid >> jj) & 1u);
        wd[jj][0] = vr[jj].x & mk;
        wd[jj][1] = vr[jj].y & mk;
        wd[jj][2] = vr[jj].z & mk;
        wd[jj][3] = vr[jj].w & mk;
    }
    uint16_t* base = L.sVp + (8 * pv) * S::PS + y * S::PW + 4 * gx;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const uint32_t c0 = (wd[0][e >> 1] >> sh) & 0xffffu;
        const uint32_t c1 = (wd[1][e >> 1] >> sh) & 0xffffu;
        const uint32_t c2 = (wd[2][e >> 1] >> sh) & 0xffffu;
        const uint32_t c3 = (wd[3][e >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(base + e * S::PS) = uint2{c0 | (c1 << 16), c2 | (c3 << 16)};
    }
}

// The V planes, the LePE operand table and the bias, by NST threads (st =
// 0 .. NST - 1 of them).  Task st of the V staging came in with the
// prologue's loads (vr0, valid0); the later tasks and the LePE taps are
// loaded here, their loads in flight while the first task is written.
template <typename S, int NST>
__device__ __forceinline__ void stage_planes(const ImgLds<S>& L, const uint16_t* __restrict__ v,
                                             size_t img, const float* __restrict__ lepe_w,
                                             const float* __restrict__ lepe_b, int hg,
                                             int has_lepe, int st, const uint4 (&vr0)[4],
                                             unsigned valid0) {
    constexpr int VR = (S::NVT + NST - 1) / NST;  // V tasks per thread
    constexpr int TR = (S::NTE + NST - 1) / NST;  // Toeplitz entries per thread
    uint4 vr[VR > 1 ? VR - 1 : 1][4];
    unsigned valid[VR > 1 ? VR - 1 : 1];
#pragma unroll
    for (int u = 1; u < VR; ++u) valid[u - 1] = load_vtask<S>(v, img, st + u * NST, vr[u - 1]);
    // the four taps of each Toeplitz entry (w[c][i][4ks + kk - n]), clamped
    // into the row; the taps outside the kernel are zeroed below
    float wv[TR][4];
    float bias = 0.f;
    if (has_lepe) {
#pragma unroll
        for (int u = 0; u < TR; ++u) {
            const int it = min(st + u * NST, S::NTE - 1);
            const int ks = it & 1, i = (it >> 1) % 5, lane_cg = it / 10;
            const int c = 16 * (lane_cg >> 6) + ((lane_cg & 63) >> 2), n = lane_cg & 3;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                wv[u][kk] = lepe_w[(hg * S::CG + c) * 25 + i * 5 + min(max(4 * ks + kk - n, 0), 4)];
        }
        if (lepe_b) bias = lepe_b[hg * S::CG + min(st, S::CG - 1)];
    }
    store_vtask<S>(L, st, vr0, valid0);
#pragma unroll
    for (int u = 1; u < VR; ++u) store_vtask<S>(L, st + u * NST, vr[u - 1], valid[u - 1]);
    if (has_lepe) {
#pragma unroll
        for (int u = 0; u < TR; ++u) {
            const int it = st + u * NST;
            if (it < S::NTE) {
                const int ks = it & 1, lane_cg = it / 10, n = lane_cg & 3;
                uint32_t hh[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int jj = 4 * ks + kk - n;
                    hh[kk] = (jj >= 0 && jj <= 4) ? f32_to_bf16(wv[u][kk]) : 0u;
                }
                L.sTab[it] = uint2{hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16)};
            }
        }
        if (st < S::CG) L.sBias[st] = bias;
    }
}

template <int HS, int NW, int HG, int HEADS, int KTOP, bool ROUTED>
__device__ __forceinline__ void image_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lepe_w,
    const float* __restrict__ lepe_b, int32_t* __restrict__ routing, uint16_t* __restrict__ out,
    int has_lepe, float scale_log2e) {
    using S = ImgShape<HS, NW, HG, HEADS, KTOP>;
    extern __shared__ __align__(16) unsigned char smem[];
    const ImgLds<S> L(smem);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, g = lane >> 4;
    // the head groups of one image run on one XCD: their 64-byte slices of
    // each token row share that XCD's L2 lines
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int b = blk / S::NGRP, hg = blk - b * S::NGRP;
    const size_t img = static_cast<size_t>(b) * S::N * S::C + hg * S::CG;

    // 1. loads, all at once and in the order they are needed: K (piece
    //    i % PCT of token i / PCT), the Q operands of the wave's jobs, the V
    //    staging tasks, the LePE weights (and the caller's routing).  The
    //    compiler waits for each register set where it is first used.
    uint4 kreg[S::KR];
#pragma unroll
    for (int u = 0; u < S::KR; ++u) {
        const int i = min(tid + u * kImgThreads, S::NPK - 1);
        const int tok = i / S::PCT, pc = i - tok * S::PCT;
        kreg[u] = *reinterpret_cast<const uint4*>(k + img + static_cast<size_t>(tok) * S::C +
                                                  8 * pc);
    }
    // Q operands: lane (query slot li of the 4 x 4 tile, group g) holds dims
    // 8g .. 8g + 7; slots outside the map load the nearest in-map token
    // (never stored)
    bf16x8_t qb[S::JPW];
#pragma unroll
    for (int jl = 0; jl < S::JPW; ++jl) {
        const int job = min(w + kImgWaves * jl, S::JOBS - 1);
        const int hl = job / S::TPH, tile = job - hl * S::TPH;
        const int y = min(4 * (tile / S::TS) + (li >> 2), S::H - 1);
        const int x = min(4 * (tile % S::TS) + (li & 3), S::W - 1);
        qb[jl] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(q + img + static_cast<size_t>(y * S::W + x) *
                                                                    S::C +
                                                      hl * kHeadDim + 8 * g));
    }
    // the first V staging task of each thread that stages the V planes:
    // every thread when the routing is the caller's, else the threads of
    // the waves that do not route (they stage while the others route)
    constexpr int NST = ROUTED ? kImgThreads : kImgThreads - 64 * S::PASSES;
    const int st = ROUTED ? tid : tid - 64 * S::PASSES;
    uint4 vreg[4];
    unsigned vvalid = 0;
    if constexpr (ROUTED) vvalid = load_vtask<S>(v, img, st, vreg);
    int rid[ROUTED ? S::RI : 1];
    if constexpr (ROUTED) {
#pragma unroll
        for (int u = 0; u < S::RI; ++u) {
            const int i = min(tid + u * kImgThreads, S::ROWS * S::KTOP - 1);
            const int hl = i / (S::R * S::KTOP), rest = i - hl * S::R * S::KTOP;
            rid[u] = routing[(static_cast<size_t>(b) * S::HEADS + hg * S::HG + hl) * S::R *
                                 S::KTOP +
                             rest];
        }
    }
    // offsets of every region's first token / cell; zero row; counters
    if (tid < S::R) {
        const int ry = tid / S::NW, rx = tid - ry * S::NW;
        L.sRegK[tid] = kofs<S>(ry * S::HS, rx * S::HS);
        L.sRegV[tid] = ry * S::HS * S::PW + rx * S::HS + 2;
    }
    if (tid < 4) reinterpret_cast<uint32_t*>(L.sZero)[tid] = 0u;
    if constexpr (!ROUTED) {
        if (tid < S::HG) L.sKinf[tid] = 0u;
        if (tid == 0) *L.sNFail = 0;
    }
    // K to LDS as it arrives, then Q
#pragma unroll
    for (int u = 0; u < S::KR; ++u) {
        const int i = tid + u * kImgThreads;
        if (i < S::NPK) {
            const int tok = i / S::PCT, pc = i - tok * S::PCT;
            const int y = tok / S::W, x = tok - y * S::W;
            *reinterpret_cast<uint4*>(L.sK + kofs<S>(y, x) + 8 * pc) = kreg[u];
        }
    }
    if constexpr (!ROUTED) {
#pragma unroll
        for (int jl = 0; jl < S::JPW; ++jl) {
            const int job = w + kImgWaves * jl;
            if (job < S::JOBS) {
                const int hl = job / S::TPH, tile = job - hl * S::TPH;
                const int y = 4 * (tile / S::TS) + (li >> 2), x = 4 * (tile % S::TS) + (li & 3);
                if (y < S::H && x < S::W)
                    *reinterpret_cast<bf16x8_t*>(L.sQs + kofs<S>(y, x) + hl * kHeadDim + 8 * g) =
                        qb[jl];
            }
        }
    }
    lds_barrier();

    // Where this kernel routes, the V loads go out now, once K and Q are in:
    // issued with them, they shared the HBM bandwidth that the means and the
    // routing wait on; from here they arrive during the means
    if constexpr (!ROUTED) {
        if (w >= S::PASSES) vvalid = load_vtask<S>(v, img, st, vreg);
    }

    // 2. the region means (or the caller's routing)
    if constexpr (!ROUTED) {
        const float kmx = region_means_kq<S>(L.sK, L.sQs, L.sKbar, L.sQbar);
        // the float bits of a nonnegative value order like the value
        // (rounded to nearest, plus one ulp; the bound it feeds carries a
        // factor 4); one max over all items of the wave, for every head
        const float m0 = wave_max_f32(kmx);
        if (lane == 0) {
#pragma unroll
            for (int hl = 0; hl < S::HG; ++hl) atomicMax(L.sKinf + hl, __float_as_uint(m0) + 1u);
        }
    } else {
        // the caller's routing, ids clamped into range
#pragma unroll
        for (int u = 0; u < S::RI; ++u) {
            const int i = tid + u * kImgThreads;
            if (i < S::ROWS * S::KTOP) {
                const int id = min(max(rid[u], 0), S::R - 1);
                L.sOffK[i] = L.sRegK[id];
                L.sOffV[i] = L.sRegV[id];
            }
        }
    }
    lds_barrier();

    // 3. routing; the waves that do not route stage the V planes (over the
    //    staged Q, read only by the means), the LePE operand table and the
    //    bias meanwhile
    if constexpr (!ROUTED) {
        if (w < S::PASSES)
            route_rows<S>(L, b, hg, routing);
        else
            stage_planes<S, NST>(L, v, img, lepe_w, lepe_b, hg, has_lepe, st, vreg,
                                 vvalid);
        lds_barrier();
        if (*L.sNFail > 0) {  // workgroup-uniform
            route_exact<S>(L, b, hg, routing);
            lds_barrier();
        }
    } else {
        stage_planes<S, NST>(L, v, img, lepe_w, lepe_b, hg, has_lepe, st, vreg, vvalid);
        lds_barrier();
    }

    // 4. jobs: LePE, attention, store.  Per-lane gather constants: the K
    //    operand rows (key 32c + 8(li/4) + 4blk + li%4: routed rank and the
    //    slot's offset inside its region) and the V operand keys (32c + 8g ..)
    int jrk[S::NCH][2], slk[S::NCH][2], jrv[S::NCH], rov[S::NCH];
#pragma unroll
    for (int c = 0; c < S::NCH; ++c) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int key = min(32 * c + 8 * (li >> 2) + 4 * blk + (li & 3), S::NKEYS - 1);
            const int jr = key / S::T, su = key - jr * S::T;
            jrk[c][blk] = jr;
            slk[c][blk] = (su / S::HS) * S::RS + (su % S::HS) * S::CG + 8 * g;
        }
        const int k0 = 32 * c + 8 * g;
        if constexpr (S::HS == 4) {
            jrv[c] = min(k0 >> 4, S::KTOP - 1);
            rov[c] = ((k0 & 15) >> 2) * S::PW;
        } else {
            jrv[c] = min(k0 >> 2, S::KTOP - 2);
            rov[c] = 0;
        }
    }
    const float sl2e = scale_log2e;
    float* stg = L.sStage + w * (16 * 36);
    const int zoff = static_cast<int>(L.sZero - L.sVp);  // the zero row, from any plane base
#pragma unroll 1
    for (int jl = 0; jl < S::JPW; ++jl) {
        const int job = w + kImgWaves * jl;
        if (job >= S::JOBS) break;
        const int hl = job / S::TPH, tile = job - hl * S::TPH;
        const int ty0 = 4 * (tile / S::TS), tx0 = 4 * (tile % S::TS);
        // this job's Q operand (a select chain: a register array indexed by
        // the loop counter would go to scratch)
        bf16x8_t qj = qb[0];
#pragma unroll
        for (int jj = 1; jj < S::JPW; ++jj)
            if (jj == jl) qj = qb[jj];
        // LePE of the tile: lane (channel b4 = lane / 4 of the group, output
        // row n of the 4 x 4 tile); rows outside the map read the zero row
        f32x4_t lep[2];
        {
            const int b4 = lane >> 2, n = lane & 3;
            int rowoff[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int y = ty0 + n + i - 2;
                rowoff[i] = (y >= 0 && y < S::H) ? y * S::PW + tx0 : -1;
            }
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) {
                const int cl = hl * kHeadDim + 16 * cg + b4;
                f32x4_t d = {0.f, 0.f, 0.f, 0.f};
                if (has_lepe) {
                    const float bs = L.sBias[cl];
                    d = f32x4_t{bs, bs, bs, bs};
                    const uint4* tb = reinterpret_cast<const uint4*>(
                        L.sTab + ((hl * 2 + cg) * 64 + lane) * 10);
                    const int pbase = cl * S::PS;
#pragma unroll
                    for (int i = 0; i < 5; ++i) {
                        const uint4 t4 = tb[i];
                        const uint16_t* row =
                            L.sVp + (rowoff[i] >= 0 ? pbase + rowoff[i] : zoff);
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            const s16x4_t a = *reinterpret_cast<const s16x4_t*>(row + 4 * ks);
                            const uint2 bw = ks == 0 ? uint2{t4.x, t4.y} : uint2{t4.z, t4.w};
                            d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                                a, __builtin_bit_cast(s16x4_t, bw), d, 0, 0, 0);
                        }
                    }
                }
                lep[cg] = d;
            }
        }

        // attention over the routed keys of each region of the tile
        const int my_m = S::RPT == 1 ? 0 : ((li >> 3) << 1) | ((li & 3) >> 1);
        // the Q operand for each region of the tile: this lane's query where
        // the query lies in that region, else zero (bit masks, no branches)
        bf16x8_t qm[S::RPT];
#pragma unroll
        for (int m = 0; m < S::RPT; ++m) {
            const uint32_t mk = (S::RPT == 1 || my_m == m) ? 0xffffffffu : 0u;
            const u32x4_t qw = __builtin_bit_cast(u32x4_t, qj);
            qm[m] = __builtin_bit_cast(bf16x8_t, u32x4_t{qw[0] & mk, qw[1] & mk, qw[2] & mk, qw[3] & mk});
        }
        int rb[S::RPT];  // row base of (hl, region m) in the routing tables
#pragma unroll
        for (int m = 0; m < S::RPT; ++m) {
            const int ry = min(ty0 / S::HS + m / S::RPS, S::NW - 1);
            const int rx = min(tx0 / S::HS + m % S::RPS, S::NW - 1);
            rb[m] = (hl * S::R + ry * S::NW + rx) * S::KTOP;
        }
        const uint16_t* kh = L.sK + hl * kHeadDim;
        const uint16_t* vp0 = L.sVp + (hl * kHeadDim + li) * S::PS;
        const uint16_t* vp1 = vp0 + 16 * S::PS;
        float mrun = -INFINITY, lsum = 0.f;
        f32x4_t o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < S::NPAIR; ++u) {
            // S^T of each 32-key chunk, one accumulator per key block: the
            // regions' products are summed with their own queries' Q (the
            // other query slots zeroed), so a query's sum holds its own
            // region's scores plus exact zeros (K is finite)
            float x[2][8];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                const int c = 2 * u + ch;
                if (32 * c >= S::NKEYS) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[ch][e] = -INFINITY;
                    continue;
                }
                f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int m = 0; m < S::RPT; ++m) {
#pragma unroll
                    for (int blk = 0; blk < 2; ++blk) {
                        const int off = L.sOffK[rb[m] + jrk[c][blk]] + slk[c][blk];
                        const bf16x8_t ka =
                            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kh + off));
                        sc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qm[m], sc[blk], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[ch][e] = sc[0][e];
                    x[ch][4 + e] = sc[1][e];
                }
            }
            // keys past the routed set (a ragged last chunk) weigh nothing
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (64 * u + 32 * ch + 8 * g + e >= S::NKEYS) x[ch][e] = -INFINITY;
            float mx = x[0][0];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (ch | e) mx = max_f(mx, x[ch][e]);
            mx = group4_max(mx);
            const float mnew = u == 0 ? mx : max_f(mrun, mx);
            const float mb = mnew * sl2e;
            bf16x8_t pb[2];
            float psum = 0.f;
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pe = __builtin_amdgcn_exp2f(fmaf(x[ch][e], sl2e, -mb));
                    psum += pe;
                    pb[ch][e] = static_cast<__bf16>(pe);
                }
            if (u == 0) {
                lsum = psum;
            } else {
                const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * sl2e);
                lsum = fmaf(lsum, alpha, psum);
                o0 *= alpha;
                o1 *= alpha;
            }
            mrun = mnew;
#pragma unroll
            for (int m = 0; m < S::RPT; ++m) {
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    const int c = 2 * u + ch;
                    if (32 * c >= S::NKEYS) break;
                    bf16x8_t pm = pb[ch];
                    if constexpr (S::RPT > 1) {
                        if (my_m != m) pm = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
                    }
                    // V^T operands: dims li and 16 + li of keys 32c + 8g .. + 7
                    uint32_t w0[4], w1[4];
                    if constexpr (S::HS == 4) {
                        // rows rov, rov + 1 of one region, 4 columns each
                        const int o = L.sOffV[rb[m] + jrv[c]] + rov[c];
                        w0[0] = *reinterpret_cast<const uint32_t*>(vp0 + o);
                        w0[1] = *reinterpret_cast<const uint32_t*>(vp0 + o + 2);
                        w0[2] = *reinterpret_cast<const uint32_t*>(vp0 + o + S::PW);
                        w0[3] = *reinterpret_cast<const uint32_t*>(vp0 + o + S::PW + 2);
                        w1[0] = *reinterpret_cast<const uint32_t*>(vp1 + o);
                        w1[1] = *reinterpret_cast<const uint32_t*>(vp1 + o + 2);
                        w1[2] = *reinterpret_cast<const uint32_t*>(vp1 + o + S::PW);
                        w1[3] = *reinterpret_cast<const uint32_t*>(vp1 + o + S::PW + 2);
                    } else {
                        // two regions, rows 0 and 1, 2 columns each
                        const int oa = L.sOffV[rb[m] + jrv[c]];
                        const int ob = L.sOffV[rb[m] + jrv[c] + 1];
                        w0[0] = *reinterpret_cast<const uint32_t*>(vp0 + oa);
                        w0[1] = *reinterpret_cast<const uint32_t*>(vp0 + oa + S::PW);
                        w0[2] = *reinterpret_cast<const uint32_t*>(vp0 + ob);
                        w0[3] = *reinterpret_cast<const uint32_t*>(vp0 + ob + S::PW);
                        w1[0] = *reinterpret_cast<const uint32_t*>(vp1 + oa);
                        w1[1] = *reinterpret_cast<const uint32_t*>(vp1 + oa + S::PW);
                        w1[2] = *reinterpret_cast<const uint32_t*>(vp1 + ob);
                        w1[3] = *reinterpret_cast<const uint32_t*>(vp1 + ob + S::PW);
                    }
                    const bf16x8_t va0 =
                        __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w0[2], w0[3]});
                    const bf16x8_t va1 =
                        __builtin_bit_cast(bf16x8_t, u32x4_t{w1[0], w1[1], w1[2], w1[3]});
                    o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va0, pm, o0, 0, 0, 0);
                    o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va1, pm, o1, 0, 0, 0);
                }
            }
        }
        const float inv = __builtin_amdgcn_rcpf(group4_sum(lsum));

        // LePE + O through the wave's LDS tile, then 16-byte rows
        {
            const int b4 = lane >> 2, n = lane & 3;
#pragma unroll
            for (int cg = 0; cg < 2; ++cg)
#pragma unroll
                for (int e = 0; e < 4; ++e) stg[(4 * e + n) * 36 + 16 * cg + b4] = lep[cg][e];
        }
        wave_sync_lds();
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(stg + li * 36 + 4 * g);
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(stg + li * 36 + 16 + 4 * g);
        const f32x4_t r0 = a0 + o0 * inv, r1 = a1 + o1 * inv;
        wave_sync_lds();
        {
            uint16_t* row = reinterpret_cast<uint16_t*>(stg + li * 36);
            *reinterpret_cast<uint2*>(row + 4 * g) =
                uint2{f32_to_bf16(r0[0]) | (f32_to_bf16(r0[1]) << 16),
                      f32_to_bf16(r0[2]) | (f32_to_bf16(r0[3]) << 16)};
            *reinterpret_cast<uint2*>(row + 16 + 4 * g) =
                uint2{f32_to_bf16(r1[0]) | (f32_to_bf16(r1[1]) << 16),
                      f32_to_bf16(r1[2]) | (f32_to_bf16(r1[3]) << 16)};
        }
        wave_sync_lds();
        {
            const int slot = lane >> 2, pc = lane & 3;
            const int y = ty0 + (slot >> 2), x = tx0 + (slot & 3);
            const uint4 val = *reinterpret_cast<const uint4*>(
                reinterpret_cast<const uint16_t*>(stg + slot * 36) + 8 * pc);
            if (y < S::H && x < S::W)
                __builtin_nontemporal_store(
                    u32x4_t{val.x, val.y, val.z, val.w},
                    reinterpret_cast<u32x4_t*>(out + img + static_cast<size_t>(y * S::W + x) *
                                                              S::C +
                                               hl * kHeadDim + 8 * pc));
        }
        wave_sync_lds();
    }
}

template <int HS, int NW, int HG, int HEADS, int KTOP, bool ROUTED>
__global__ __launch_bounds__(kImgThreads) void image_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lepe_w,
    const float* __restrict__ lepe_b, int32_t* __restrict__ routing, uint16_t* __restrict__ out,
    int has_lepe, float scale_log2e) {
    image_body<HS, NW, HG, HEADS, KTOP, ROUTED>(q, k, v, lepe_w, lepe_b, routing, out, has_lepe,
                                                 scale_log2e);
}

template <int HS, int NW, int HG, int HEADS, int KTOP>
bool image_matches(const Params& p) {
    return p.hs == HS && p.ws == HS && p.n == NW && p.heads == HEADS && p.k == KTOP &&
           p.kv_ratio == 1 && !p.shared;
}

}  // namespace img

using img::image_kernel;
using img::image_matches;
using img::kImgThreads;

#define BRA_FOR_EACH_IMAGE_SHAPE(X) \
    X(4, 7, 1, 4, 4)                \
    X(2, 7, 2, 8, 16)

bool image_applies(const Params& p, bool bf16) {
    if (!bf16) return false;
#define BRA_IMG_MATCH(HS, NW, HG, HEADS, KTOP) \
    if (image_matches<HS, NW, HG, HEADS, KTOP>(p)) return true;
    BRA_FOR_EACH_IMAGE_SHAPE(BRA_IMG_MATCH)
#undef BRA_IMG_MATCH
    return false;
}

int image_lds_bytes(const Params& p) {
#define BRA_IMG_LDS(HS, NW, HG, HEADS, KTOP) \
    if (image_matches<HS, NW, HG, HEADS, KTOP>(p)) return img_geo(HS, NW, HG, HEADS, KTOP).lds;
    BRA_FOR_EACH_IMAGE_SHAPE(BRA_IMG_LDS)
#undef BRA_IMG_LDS
    return 0;
}

hipError_t prepare_image(const Params& p) {
#define BRA_IMG_PREP(HS, NW, HG, HEADS, KTOP)                                                      \
    if (image_matches<HS, NW, HG, HEADS, KTOP>(p)) {                                             \
        const int lds = img_geo(HS, NW, HG, HEADS, KTOP).lds;                                    \
        hipError_t e = hipFuncSetAttribute(                                                       \
            reinterpret_cast<const void*>(&image_kernel<HS, NW, HG, HEADS, KTOP, false>),         \
            hipFuncAttributeMaxDynamicSharedMemorySize, lds);                                     \
        if (e != hipSuccess) return e;                                                            \
        return hipFuncSetAttribute(                                                               \
            reinterpret_cast<const void*>(&image_kernel<HS, NW, HG, HEADS, KTOP, true>),          \
            hipFuncAttributeMaxDynamicSharedMemorySize, lds);                                     \
    }
    BRA_FOR_EACH_IMAGE_SHAPE(BRA_IMG_PREP)
#undef BRA_IMG_PREP
    return hipErrorInvalidValue;
}

hipError_t launch_image(const Params& p, const void* q, const void* k, const void* v,
                        const float* lepe_w, const float* lepe_b, int32_t* routing, bool routed,
                        void* out, hipStream_t stream) {
    const uint16_t* q16 = static_cast<const uint16_t*>(q);
    const uint16_t* k16 = static_cast<const uint16_t*>(k);
    const uint16_t* v16 = static_cast<const uint16_t*>(v);
    uint16_t* o16 = static_cast<uint16_t*>(out);
    const int has_lepe = lepe_w != nullptr;
#define BRA_IMG_LAUNCH(HS, NW, HG, HEADS, KTOP)                                                    \
    if (image_matches<HS, NW, HG, HEADS, KTOP>(p)) {                                             \
        const ImgGeo geo = img_geo(HS, NW, HG, HEADS, KTOP);                                     \
        const dim3 grid(p.B * (HEADS / HG)), block(kImgThreads);                                  \
        if (routed)                                                                               \
            hipLaunchKernelGGL((image_kernel<HS, NW, HG, HEADS, KTOP, true>), grid, block,        \
                               geo.lds, stream, q16, k16, v16, lepe_w, lepe_b, routing, o16,      \
                               has_lepe, p.scale_log2e);                                                         \
        else                                                                                      \
            hipLaunchKernelGGL((image_kernel<HS, NW, HG, HEADS, KTOP, false>), grid, block,       \
                               geo.lds, stream, q16, k16, v16, lepe_w, lepe_b, routing, o16,      \
                               has_lepe, p.scale_log2e);                                                         \
        return hipGetLastError();                                                                 \
    }
    BRA_FOR_EACH_IMAGE_SHAPE(BRA_IMG_LAUNCH)
#undef BRA_IMG_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace bra
