// bra_small.h -- interface of the one-launch fp32 kernel for small problems
// (bra_small.hip): one workgroup per (image, head, region), at most 256 of
// them.  Not installed; the public ABI is include/bra.h.
#pragma once

#include "bra_launch.h"

namespace bra {

constexpr int kSmallThreads = 512;    // 8 waves: the phases after the DMA are latency-bound
constexpr int kSmallMaxBlocks = 256;  // (image, head, region) triples: one workgroup per CU
constexpr int kMaxSmallK = 16;        // routed regions per row

// LDS layout (byte offsets, 16-byte aligned) and the lane split of a small
// problem.  A query takes L lanes (L = kSmallThreads / the power of two >= t,
// 8 to 32): lane li scores keys li, li + L, .. and outputs dims li * 32 / L ..
// Staged arrays are whole rounds of kSmallThreads 16-byte DMA slots.
struct SmallGeo {
    int L, pstride;
    int rk, rq, rh, rv;  // DMA rounds: K map, Q rows, V halo, routed V rows
    int off_k, off_kbar, off_v, off_p, off_h, off_q, off_w, off_ids, off_tab, lds;
};

__host__ __device__ constexpr int small_align16(int x) { return (x + 15) & ~15; }

__host__ __device__ constexpr SmallGeo small_geo(const Params& p) {
    SmallGeo g{};
    int tp = 1;
    while (tp < p.t) tp <<= 1;
    g.L = kSmallThreads / tp > 32 ? 32 : kSmallThreads / tp;
    g.pstride = p.nkeys + 4;
    const int round = kSmallThreads * 16;
    const int ncell = (p.hs + 4) * (p.ws + 4);
    g.rk = (p.H * p.W * 8 + kSmallThreads - 1) / kSmallThreads;
    g.rq = (p.t * 8 + kSmallThreads - 1) / kSmallThreads;
    g.rh = (ncell * 8 + kSmallThreads - 1) / kSmallThreads;
    g.rv = (p.nkeys * 8 + kSmallThreads - 1) / kSmallThreads;
    int off = 0;
    g.off_k = off;
    off += g.rk * round;
    g.off_kbar = off;
    off = small_align16(off + p.R * kHeadDim * 8);
    g.off_v = off;
    off += g.rv * round;
    g.off_p = off;
    off = small_align16(off + p.t * g.pstride * 4);
    g.off_h = off;
    off += g.rh * round;
    g.off_q = off;
    off += g.rq * round;
    g.off_w = off;
    off = small_align16(off + (kHeadDim * 25 + kHeadDim) * 4);
    g.off_ids = off;
    off = small_align16(off + 2 * kMaxSmallK * 4);
    g.off_tab = off;  // slot offsets [64], region first tokens [64]
    off = small_align16(off + 2 * 64 * 4);
    g.lds = off;
    return g;
}

// The small kernel takes the forward: fp32, per-head routing, no KV
// downsampling, at most kSmallMaxBlocks (image, head, region) triples,
// R <= 64, t <= 64, k <= 16, and its tiles (the head's whole K map among
// them) within a CU's LDS.
bool small_applies(const Params& p, bool bf16);
int small_lds_bytes(const Params& p);
// Raises the kernel's dynamic LDS limit when its tiles need more than 64 KB.
hipError_t prepare_small(const Params& p);
hipError_t launch_small(const Params& p, const float* q, const float* k, const float* v,
                        const float* lepe_w, const float* lepe_b, int32_t* routing, float* out,
                        hipStream_t stream);

}  // namespace bra
