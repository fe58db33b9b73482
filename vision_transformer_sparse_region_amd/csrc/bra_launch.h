// bra_launch.h -- internal interface between the C ABI (bra_api.cpp) and the
// HIP kernels (bra_pool.hip, bra_route.hip, bra_attend.hip).  Not installed; the public ABI is include/bra.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace bra {

constexpr int kHeadDim = 32;     // the only head_dim the kernels implement
constexpr int kThreads = 256;    // threads per workgroup (4 wave64s)
constexpr int kWaves = kThreads / 64;
// LDS one workgroup may take: a gfx950 CU's whole 160 KB.  A kernel whose
// tiles need more than the default 64 KB has its dynamic-LDS limit raised
// first (prepare_attend).
constexpr int kMaxLdsBytes = 160 * 1024;
constexpr int kDefaultLdsBytes = 64 * 1024;
constexpr int kPoolChunkBytes = 16 * 1024;
constexpr int kVtRow = 32;       // bf16 elements per staged V row (32 dims; swizzled, no pad)
constexpr int kMaxQTiles = 2;    // 16-query tiles one wave carries at once
constexpr int kLepeCols = 8;     // output columns one LePE work item covers
constexpr int kHaloRegs = 8;     // 16-byte halo pieces a thread keeps in flight
constexpr int kWRegs = 2;        // 16-byte LePE weight pieces a thread keeps in flight
constexpr int kMaxChannels = 1024;
constexpr int kMaxRegions = 256;    // n_win <= 16

// Problem geometry plus the on-chip layout of the routing/attention kernel.
struct Params {
    int B, H, W, C, heads;
    int n, R;        // regions per side, regions per map
    int hs, ws, t;   // region height, width, tokens per region
    int k;           // routed regions per region (already clamped)
    int shared;      // 1: one routing per region for every head (full-C affinity)
    int rheads;      // heads of the routing buffer: 1 when shared, else heads
    int nkeys;       // k * kt keys per query
    // the K/V map the attention gathers from: the input map, or its K/V
    // average-pooled over kv_ratio x kv_ratio blocks (KV downsampling)
    int kv_ratio, kH, kW, khs, kws, kt;
    float scale_log2e;
    int has_lepe;
    int lstride;     // floats per staged output row (C plus 16 bytes)
    int lepe_items;  // (channel pair, window row, 8-column block) work items
    int lepe_alias;  // 1: outputs overwrite the V halo after a single LePE round
    int lepe_mfma;   // 1: LePE on the 4x4x4 MFMA with a channel-planar halo
    int out_proj;    // 1: the attention kernel applies the output projection (bf16)
    int halo_pieces; // 16-byte pieces of the V window with its 2-token halo
    // LDS byte offsets of the routing/attention kernel
    int off_vt, off_vh, off_l, off_w, off_idx, lds_bytes;
    int table_items; // 8-byte entries of the MFMA LePE Toeplitz operand table (0: none)
    // region-pool kernel
    int pool_blocks; // workgroups computing means (the table follows them)
    int qmean_attend; // 1: the attention kernel sums the Q means itself; the
                      // pool kernel then computes only the K means
    int kmean32;     // 1: the K means are also written in fp32 (the in-kernel
                     // routing's first pass reads them)
    int pool_chunk;  // staged path: tokens staged per step
    int pool_lds_bytes;
};

// Fills the geometry and layout; returns false when a tile does not fit.
bool plan(Params& p, int B, int H, int W, int C, int heads, int n_win, int k, float scale,
          bool bf16, bool shared, int kv_ratio);

// Kernel launches on `stream`; return the launch status.
//   means: fp64 region means, Q as [B][heads][R][32], then K as [B][heads][16][R][2]
//   (kmean_index: dims in pairs), then K again in fp32 as [B][heads][8][R][4]
//   (kmean32_offset: dims in quads; written when p.kmean32).
//   lepe_table: p.table_items 8-byte entries (written by the pool kernel when
//   lepe_w is given and the shape runs LePE on MFMA).
//   routing: [B][rheads][R][k] int32 region ids.
hipError_t launch_pool_qk(const Params& p, bool bf16, const void* q, const void* k,
                          const float* lepe_w, double* means, uint2* lepe_table,
                          hipStream_t stream);
hipError_t launch_route(const Params& p, bool bf16, const double* means, int32_t* routing,
                        hipStream_t stream);
// Maps of at most 64 regions and at most one head per wave are routed inside
// the attention kernel (one region per lane, one head per wave); others by
// the routing kernel.
constexpr bool route_fused(int R, int heads) {
    return R <= 64 && heads <= kWaves;
}
inline bool route_in_attend(const Params& p) { return !p.shared && route_fused(p.R, p.heads); }
// The in-kernel routing screens with fp32 K means where a mean sums at least
// 32 tokens: the fp32 copy then adds at most 1/16 to the bytes the pool
// kernel moves (measured: stage-1 windows of 64 tokens gain 1 us per forward,
// 16-token windows lose 0.4).
__host__ __device__ constexpr bool kmean32_pays(int t) { return t >= 32; }

// Small region grids routed outside the attention kernel (per head, bf16)
// with small regions: one kernel computes the region means and routes
// (pool_route_kernel), staging one head's K of every region (R * t * 64
// bytes, at most 16 KB) and Q of 16 regions (at most 16 KB) in LDS; no mean
// array goes to HBM.
constexpr bool route_in_pool(bool bf16, bool shared, int R, int heads, int t) {
    return bf16 && !shared && R <= 64 && !route_fused(R, heads) && t <= 16 && R * t <= 256;
}
int pool_route_lds(const Params& p);
hipError_t launch_pool_route(const Params& p, const void* q, const void* k,
                             const float* lepe_w, uint2* lepe_table, int32_t* idx,
                             hipStream_t stream);

// How the attention kernel splits a region's queries into wave jobs: QT tiles
// of 16 queries per head, in G groups of tpg tiles (at most kMaxQTiles); a
// job is one (head, group), heads * G jobs in all, dealt to the waves
// round-robin.  Heads with fewer than kWaves waves between them split their
// tiles over the spare waves.
struct JobShape {
    int QT, tpg, G, njobs;
};
constexpr JobShape job_shape(int t, int heads) {
    const int QT = (t + 15) / 16;
    const int wph = kWaves / heads > 1 ? kWaves / heads : 1;
    const int g_spread = wph < QT ? wph : QT;
    const int g_fit = (QT + kMaxQTiles - 1) / kMaxQTiles;
    const int g0 = g_spread > g_fit ? g_spread : g_fit;
    const int tpg = (QT + g0 - 1) / g0;
    const int G = (QT + tpg - 1) / tpg;  // every group non-empty
    return JobShape{QT, tpg, G, heads * G};
}
// 64-token windows with two heads (four query tiles per head, two per wave):
// the two waves of a head split each routed pair of 32-key V chunks, one
// chunk each, and share them through an LDS buffer per head, double-buffered
// over pairs: 2 parities x 2 heads x 2 chunks x 32 keys x 32 dims of bf16.
constexpr bool share_v(int hs, int ws, int heads) {
    return hs * ws == 64 && heads == 2 && job_shape(64, 2).njobs == kWaves &&
           job_shape(64, 2).G == 2;
}
constexpr int kVtSharedBytes = 2 * 2 * 2 * 32 * kVtRow * 2;
// bf16 maps routed inside the attention kernel whose jobs are each some
// wave's first job hold every query of the region in the waves' first Q
// operands, so the kernel sums the Q means from them (exactly, in fp64) and
// the pool kernel reads only K.
constexpr bool qmean_in_attend(bool bf16, bool fused, int t, int heads) {
    return bf16 && fused && job_shape(t, heads).njobs <= kWaves;
}

// Raises the dynamic-LDS limit of the attention kernel instance that
// launch_attend picks for p to kMaxLdsBytes when its tiles need more than
// kDefaultLdsBytes (a no-op otherwise).  Every handle raises it to the same
// value, so no handle lowers it under another.
hipError_t prepare_attend(const Params& p, bool bf16);

//   kg, vg: the K and V the attention gathers from -- k and v, or their
//   downsampled copies ([B, kH, kW, C]) when kv_ratio > 1; v still feeds LePE.
//   use_routing: read the routing from `routing` (written by the routing
//   kernel or given by the caller); otherwise route in the kernel (needs
//   route_in_attend) and write the ids to `routing`.
//   zero_bias: C zero floats (device), used when lepe_b is NULL.
//   w_o, b_o: the output projection (bf16 [C, C] Linear weight, fp32 [C] bias
//   or NULL), applied in the kernel's epilogue; NULL w_o: none.
hipError_t launch_attend(const Params& p, bool bf16, const void* q, const void* v,
                         const void* kg, const void* vg, const double* means, int32_t* routing,
                         bool use_routing, const float* lepe_w, const float* lepe_b,
                         const uint2* lepe_table, const float* zero_bias, const void* w_o,
                         const float* b_o, void* out, hipStream_t stream);
// The qkv projection [P5 §五 ①] of x (bf16 [B,H,W,C]) by w_qkv (bf16 [3C, C]
// Linear weight) + b_qkv (fp32 [3C] or NULL) into qs, ks, vs (bf16
// [B,H,W,C]), with the region means of the projected Q and K written to
// `means` as launch_pool_qk does, and the MFMA LePE table when lepe_w is given.
// (C <= 512; its dynamic LDS is proj_qkv_lds_bytes, at most 45 KB)
int proj_qkv_lds_bytes(const Params& p);
hipError_t launch_proj_qkv(const Params& p, const void* x, const void* w_qkv,
                           const float* b_qkv, void* qs, void* ks, void* vs, double* means,
                           const float* lepe_w, uint2* lepe_table, hipStream_t stream);
// The output projection [P5 §五 ⑧] runs in the attention kernel's epilogue
// when a region has enough tokens to amortise the C x C weight that each
// attention workgroup reads (C <= 4 t; measured, the epilogue saves 11 us
// per forward at C = t, 64 x 64 tokens, and the separate kernel saves 4 us
// at C = 8 t and 30 us at C = 64 t); otherwise the attention kernel stores y
// (bf16) and launch_proj_out applies the projection over slices of the
// token rows.  Both give the same bits: y rounded to bf16, the same MFMA
// sums in the same order, one rounding.
constexpr bool out_proj_in_attend(int t, int C) { return C <= 4 * t; }
// out = y w_o^T + b_o over the B*H*W token rows of y (bf16 [B,H,W,C]).
hipError_t launch_proj_out(const Params& p, const void* y, const void* w_o, const float* b_o,
                           void* out, hipStream_t stream);
// KV downsampling: k and v averaged over kv_ratio x kv_ratio blocks into
// kd, vd ([B, kH, kW, C], the input dtype; fp32 sums, one rounding).
hipError_t launch_kv_pool(const Params& p, bool bf16, const void* k, const void* v, void* kd,
                          void* vd, hipStream_t stream);
// The MFMA LePE operand table alone (the region-pool kernel's trailing
// workgroups), for the entry point that skips the region means.
hipError_t launch_lepe_table(const Params& p, const float* lepe_w, uint2* lepe_table,
                             hipStream_t stream);

// The allocation-free forward's device scratch array (bra_noalloc.hip):
// its size, its device address on the current device `device`, and a
// graph-safe clear of n floats.
size_t scratch_bytes();
hipError_t scratch_pointer(int device, void** ptr);
hipError_t launch_zero_fill(float* p, int n, hipStream_t stream);

}  // namespace bra
