// bra_launch.h -- internal interface between the C ABI (bra_api.cpp) and the
// HIP kernels (bra_kernels.hip).  Not installed; the public ABI is include/bra.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace bra {

constexpr int kHeadDim = 32;   // the only head_dim the kernels implement
constexpr int kThreads = 256;  // threads per workgroup (4 wave64s)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxLdsBytes = 64 * 1024;
constexpr int kPoolChunkBytes = 16 * 1024;
constexpr int kVtStride = 36;   // bf16 elements per staged V row (32 dims + pad)
constexpr int kMaxQTiles = 4;   // 16-query tiles one wave carries at once

// Problem geometry plus the on-chip layout of the routing/attention kernel.
struct Params {
    int B, H, W, C, heads;
    int n, R;        // regions per side, regions per map
    int hs, ws, t;   // region height, width, tokens per region
    int k;           // routed regions per region (already clamped)
    int nkeys;       // k * t keys per query
    float scale_log2e;
    int has_lepe;
    // LDS byte offsets (routing/attention kernel)
    int qstride;     // elements per staged Q row (C plus padding)
    int off_q, off_vt, off_o, off_vh, off_aff, off_qbar, off_idx, lds_bytes;
    int pool_chunk;  // tokens staged per step by the pool kernel
    int pool_lds_bytes;
};

// Fills the geometry and layout; returns false when a tile does not fit.
bool plan(Params& p, int B, int H, int W, int C, int heads, int n_win, int k, float scale,
          bool bf16);

// Kernel launches on `stream`; return the launch status.
hipError_t launch_pool_k(const Params& p, bool bf16, const void* k, double* kbar,
                         hipStream_t stream);
hipError_t launch_route_attend(const Params& p, bool bf16, const void* q, const void* k,
                               const void* v, const double* kbar, const float* lepe_w,
                               const float* lepe_b, void* out, int32_t* routing_idx,
                               hipStream_t stream);

}  // namespace bra
