// bra_proj.hip -- the module's Linear layers either side of the path, on
// MFMA: the qkv projection before it [P5 §五 ① qkv = Linear(dim, 3*dim);
// P4 §1.1], with the region means of the projected Q and K in its epilogue,
// and the output projection after it [P5 §五 ⑧ proj] for shapes whose
// regions are too small to carry it in the attention kernel's epilogue
// (page keys in bra_device.h).
//
// Both kernels compute, for a slice of up to proj_slice(C) tokens staged in
// LDS and one chunk of 64 output channels (16 per wave),
//   D^T = W[o0 .. o0+15, :] . X^T          (v_mfma_f32_16x16x32_bf16, fp32 sums)
// with operand A row m the PyTorch Linear weight row o0 + m (16 contiguous
// bytes per lane and 32-channel step, loaded once per workgroup) and operand
// B column n token n of a 16-token tile (from LDS).  Lane (n, g) receives
// output channels o0 + 4g .. o0 + 4g + 3 of token n; adding the bias and
// rounding once to bf16 gives the Linear layer's bf16 output.  The rounded
// chunk goes through LDS to 16-byte row stores.
//
// A qkv workgroup takes one token slice and proj_units(C) of its 3 * C / 64
// (output tensor, channel chunk) units: all three tensors when C <= 64, so
// the slice is staged once, else two (or one).  The units of one slice are
// consecutive workgroups, which run on one XCD and re-read the slice from
// its L2; splitting wide outputs over workgroups keeps each wave's serial
// work to one weight tile, so the grid holds many short workgroups whose
// weight loads overlap.
//
// qkv: a slice is the tokens of `group` whole regions of one image when a
// region is smaller than a slice, else one region taken a slice at a time.
// For q and k each (region, channel) sums its tokens' rounded values in fp64
// -- within the span condition of row16_sum_exact (bra_device.h) every
// partial sum of bf16 values is exact, so the region means equal those of
// the pool kernel over the stored maps, bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_device.h"
#include "bra_shapes.h"

namespace bra {
namespace {

// Output channels per workgroup: one 16-channel MFMA tile per wave.
constexpr int kProjOut = 16 * kWaves;
// LDS row stride (bf16 elements) of the output chunk.
constexpr int kOutRow = kProjOut + 8;
// 32-channel steps of the contraction (C / 32), at most 16.
constexpr int kMaxProjSteps = 16;
// Parts a channel's token sum is split into (threads per channel).
constexpr int kSumParts = kThreads / kProjOut;

// Tokens a workgroup stages at a time: 64, or 32 for C > 256 (the x slice
// stays within 33 KB of LDS).
__host__ __device__ constexpr int proj_slice(int C) { return C <= 256 ? 64 : 32; }

// Output-channel chunks of C.
__host__ __device__ constexpr int proj_chunks(int C) { return (C + kProjOut - 1) / kProjOut; }

// (tensor, chunk) units a qkv workgroup computes in turn (at most 3; it
// divides the 3 * proj_chunks(C) units of a slice).
__host__ __device__ constexpr int proj_units(int C) {
    return C <= kProjOut ? 3 : proj_chunks(C) % 2 == 0 ? 2 : 1;
}
constexpr int kMaxUnits = 3;

// Regions per qkv slice: the whole regions that fit one slice, else one.
__host__ __device__ constexpr int proj_group(int C, int t) {
    return t >= proj_slice(C) ? 1 : proj_slice(C) / t;
}

// 16-byte pieces of a staged slice per thread: proj_slice(C) * C / 8 over
// the workgroup, at most 2048 / kThreads for C <= 512.
__host__ __device__ constexpr int stage_pieces(int C) {
    return C == 0 ? 2048 / kThreads : (proj_slice(C) * C / 8 + kThreads - 1) / kThreads;
}

__host__ __device__ constexpr int proj_lds_bytes(int C) {
    // the x slice (whole rounds of 16-byte slots), the output chunk, then the
    // fp64 part sums of one region
    return stage_pieces(C) * kThreads * 16 + proj_slice(C) * kOutRow * 2 +
           kSumParts * kProjOut * 8;
}

// The x slice in LDS: rows of nvec = C / 8 16-byte pieces, packed, with
// piece pv of row u in slot pv ^ (u & m) of the row.  The XOR spreads the
// 16 rows that one MFMA operand read touches (same piece, rows n = 0..15)
// over the banks; m is the largest of 15, 7, 3 that keeps the slot inside
// the row (nvec is a multiple of 4).
__device__ __forceinline__ int swizzle_mask(int nvec) {
    return nvec % 16 == 0 ? 15 : nvec % 8 == 0 ? 7 : 3;
}
__device__ __forceinline__ int x_slot(int u, int pv, int nvec, int m) {
    return u * nvec + (pv ^ (u & m));
}

// Stage nt rows of C channels into sX by LDS DMA (global_load_lds_dwordx4):
// each wave instruction fills 64 consecutive slots, lane L slot base + L, so
// lane L loads the global piece that its slot holds.  Slots past the slice
// (up to the allocation, a whole number of rounds) receive a copy of the
// last piece.  No registers hold the data and every load of a thread is in
// flight at once; the caller waits (vmcnt) and takes a barrier before
// reading.  src(u) is the address of row u.  NP: rounds, 0 = runtime.
template <int NP, typename Src>
__device__ __forceinline__ void stage_slice(uint16_t* sX, int nt, int nvec, int np, int tid,
                                            Src src) {
    const int last = nt * nvec - 1, m = swizzle_mask(nvec);
    const int wave_slot0 = __builtin_amdgcn_readfirstlane(tid & ~63);
    constexpr int kRounds = NP > 0 ? NP : 2048 / kThreads;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
        if (NP == 0 && j >= np) break;
        const int q = min(j * kThreads + tid, last);
        const int u = q / nvec, sl = q - u * nvec;
        const int pv = sl ^ (u & m);  // the swizzle is its own inverse
        __builtin_amdgcn_global_load_lds(
            src(u) + 8 * pv,
            (__attribute__((address_space(3))) void*)(sX + 8 * (j * kThreads + wave_slot0)), 16,
            0, 0);
    }
}

// Wave-held operands of one 16-channel weight tile: rows row0 .. row0 + 15
// of w (bf16 [*, C]) and the bias entries of lane (n, g)'s output channels.
struct WeightTile {
    uint4 a[kMaxProjSteps];
    float bias[4];
};

// Loads are unconditional (steps past ksteps re-read the last one), so they
// issue back to back.  KS: C / 32 when known at compile time, else 0.
template <int KS>
__device__ __forceinline__ void load_weight_tile(WeightTile& wt, const uint16_t* __restrict__ w,
                                                 const float* __restrict__ b, int row0, int C,
                                                 int ksteps, int n, int g) {
    constexpr int kSteps = KS > 0 ? KS : kMaxProjSteps;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
        wt.a[s] = *reinterpret_cast<const uint4*>(w + static_cast<size_t>(row0 + n) * C +
                                                  32 * min(s, ksteps - 1) + 8 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) wt.bias[i] = b ? b[row0 + 4 * g + i] : 0.f;
}

// The nt tokens of sX times the weight tile, plus the bias, rounded to bf16
// into columns col0 .. col0 + 15 of the output chunk sO.
__device__ __forceinline__ void tile_linear(const WeightTile& wt, const uint16_t* sX, int nvec,
                                            int nt, int ksteps, uint16_t* sO, int col0, int n,
                                            int g) {
    const int ttiles = (nt + 15) / 16, m = swizzle_mask(nvec);
    for (int tt = 0; tt < ttiles; ++tt) {
        const int row = min(tt * 16 + n, nt - 1);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kMaxProjSteps; ++s)
            if (s < ksteps) {
                const uint4 xb = *reinterpret_cast<const uint4*>(
                    sX + 8 * x_slot(row, 4 * s + g, nvec, m));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, wt.a[s]), __builtin_bit_cast(bf16x8_t, xb),
                    acc, 0, 0, 0);
            }
        if (tt * 16 + n < nt) {
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = f32_to_bf16(acc[i] + wt.bias[i]);
            *reinterpret_cast<uint2*>(sO + (tt * 16 + n) * kOutRow + col0 + 4 * g) =
                uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        }
    }
}

template <int HS, int WS, int NW, int HEADS>
__global__ __launch_bounds__(kThreads) void proj_qkv_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w_qkv,
    const float* __restrict__ b_qkv, uint16_t* __restrict__ qs, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ vs, double* __restrict__ means, const float* __restrict__ lepe_w,
    uint2* __restrict__ lepe_table, Params p_in) {
    const Params p = fold_geometry<HS, WS, NW, HEADS, 1, 8>(p_in);
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int C = p.C, ST = proj_slice(C), nch = proj_chunks(C);
    const int group = proj_group(C, p.t), U = proj_units(C);
    const int gpi = (p.R + group - 1) / group;  // slices (token groups) per image
    const int upw = 3 * nch / U;                // workgroups per slice
    const int tasks = p.B * gpi * upw;
    if (static_cast<int>(blockIdx.x) >= tasks) {
        // trailing workgroups: the Toeplitz operands of the MFMA LePE
        const int it = (blockIdx.x - tasks) * kThreads + tid;
        if (it < p.table_items) lepe_table[it] = lepe_table_entry(lepe_w, it);
        return;
    }
    uint16_t* sX = reinterpret_cast<uint16_t*>(smem);  // stage_pieces(C) rounds of slots
    uint16_t* sO = sX + stage_pieces(C) * kThreads * 8;  // [ST][kOutRow]
    double* sP = reinterpret_cast<double*>(sO + ST * kOutRow);  // [kSumParts][kProjOut]
    const int blk = xcd_logical_block(blockIdx.x, tasks);
    const int tg = blk / upw, unit0 = (blk - tg * upw) * U;
    const int b = tg / gpi, r0 = (tg - b * gpi) * group;
    const int nreg = min(group, p.R - r0);
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C;
    const int nvec = C / 8, ksteps = C / 32;
    const int n = lane & 15, g = lane >> 4;
    // token u of the workgroup: region r0 + u / t, slot u % t with several
    // regions; slot u of region r0 with one
    const int span = group > 1 ? nreg * p.t : p.t;
    auto tok_offset = [&](int u) {
        return group > 1 ? token_offset(p, r0 + u / p.t, u - (u / p.t) * p.t)
                         : token_offset(p, r0, u);
    };
    const int col0 = 16 * wu;
    // one region: thread (part, pc) sums tokens part, part + kSumParts, ...
    // of channel c0 + pc over every slice, for each unit
    const int part = tid / kProjOut, pc = tid - part * kProjOut;
    double rsum[kMaxUnits];
#pragma unroll
    for (int j = 0; j < kMaxUnits; ++j) rsum[j] = 0.0;

    for (int u0 = 0; u0 < span; u0 += ST) {
        const int nt = min(ST, span - u0);
        __syncthreads();  // the previous slice's LDS reads are done
        stage_slice<HEADS ? stage_pieces(HEADS * kHeadDim) : 0>(
            sX, nt, nvec, stage_pieces(C), tid,
            [&](int u) { return x + img + tok_offset(u0 + u); });
#pragma unroll
        for (int j = 0; j < kMaxUnits; ++j) {
            if (j >= U) break;
            const int unit = unit0 + j, which = unit / nch, ch = unit - which * nch;
            const int c0 = ch * kProjOut, cw = min(kProjOut, C - c0);  // the chunk's channels
            const int ovec = cw / 8;
            uint16_t* dst = which == 0 ? qs : which == 1 ? ks : vs;
            // wave wu's weight tile: rows which * C + c0 + 16 wu .. of w_qkv,
            // loaded while the workgroup waits at the barrier
            WeightTile wt;
            if (col0 < cw)
                load_weight_tile<HEADS * kHeadDim / 32>(wt, w_qkv, b_qkv, which * C + c0 + col0,
                                                        C, ksteps, n, g);
            // this wave's slice loads have landed; after the barrier every
            // wave's have, and the previous unit's sO reads are done
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (col0 < cw) tile_linear(wt, sX, nvec, nt, ksteps, sO, col0, n, g);
            __syncthreads();
            for (int i = tid; i < nt * ovec; i += kThreads) {
                const int u = i / ovec, pv = i - u * ovec;
                *reinterpret_cast<uint4*>(dst + img + tok_offset(u0 + u) + c0 + 8 * pv) =
                    *reinterpret_cast<const uint4*>(sO + u * kOutRow + 8 * pv);
            }
            if (which < 2) {
                if (group > 1) {
                    // whole regions in this (only) slice: the means directly
                    for (int item = tid; item < nreg * cw; item += kThreads) {
                        const int rr = item / cw, cc = item - rr * cw;
                        double sum = 0.0;
                        for (int u = rr * p.t; u < (rr + 1) * p.t; ++u)
                            sum += static_cast<double>(bf16_to_f32(sO[u * kOutRow + cc]));
                        const int c = c0 + cc, h = c / kHeadDim, d = c - h * kHeadDim;
                        const int bh = b * p.heads + h;
                        if (which == 0)
                            means[qmean_index(p, bh, r0 + rr, d)] = mean_of(sum, p.t);
                        else
                            store_kmean(p, means, bh, d, r0 + rr, mean_of(sum, p.t));
                    }
                } else if (pc < cw) {
                    for (int u = part; u < nt; u += kSumParts)
                        rsum[j] += static_cast<double>(bf16_to_f32(sO[u * kOutRow + pc]));
                }
            }
        }
    }
    if (group == 1) {
        // the parts meet in LDS; thread c adds them
#pragma unroll
        for (int j = 0; j < kMaxUnits; ++j) {
            if (j >= U) break;
            const int unit = unit0 + j, which = unit / nch, ch = unit - which * nch;
            if (which >= 2) break;
            const int c0 = ch * kProjOut, cw = min(kProjOut, C - c0);
            __syncthreads();  // sP is free (previous unit) and every sum is in
            sP[part * kProjOut + pc] = rsum[j];
            __syncthreads();
            if (tid < cw) {
                double sum = 0.0;
#pragma unroll
                for (int q = 0; q < kSumParts; ++q) sum += sP[q * kProjOut + tid];
                const int c = c0 + tid, h = c / kHeadDim, d = c - h * kHeadDim;
                const int bh = b * p.heads + h;
                if (which == 0)
                    means[qmean_index(p, bh, r0, d)] = mean_of(sum, p.t);
                else
                    store_kmean(p, means, bh, d, r0, mean_of(sum, p.t));
            }
        }
    }
}

// out = y W^T + b over the rows of y (bf16 [ntok, C]): a slice of rows and
// a chunk of output channels per workgroup; streaming stores (the result is
// the forward's output and is not re-read here).
template <int HEADS>
__global__ __launch_bounds__(kThreads) void proj_out_kernel(
    const uint16_t* y, const uint16_t* __restrict__ w, const float* __restrict__ b,
    uint16_t* __restrict__ out, int ntok, int C_in) {
    const int C = HEADS > 0 ? HEADS * kHeadDim : C_in;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ST = proj_slice(C), nch = proj_chunks(C);
    const int tasks = ((ntok + ST - 1) / ST) * nch;
    uint16_t* sX = reinterpret_cast<uint16_t*>(smem);  // stage_pieces(C) rounds of slots
    uint16_t* sO = sX + stage_pieces(C) * kThreads * 8;  // [ST][kOutRow]
    const int blk = xcd_logical_block(blockIdx.x, tasks);
    const int ch = blk % nch, row0 = (blk / nch) * ST;
    const int nt = min(ST, ntok - row0);
    const int c0 = ch * kProjOut, cw = min(kProjOut, C - c0);
    const int nvec = C / 8, ovec = cw / 8, ksteps = C / 32;
    const int n = lane & 15, g = lane >> 4, col0 = 16 * wu;
    const bool has_tile = col0 < cw;
    WeightTile wt;
    if (has_tile) load_weight_tile<HEADS * kHeadDim / 32>(wt, w, b, c0 + col0, C, ksteps, n, g);
    const uint16_t* src = y + static_cast<size_t>(row0) * C;
    stage_slice<HEADS ? stage_pieces(HEADS * kHeadDim) : 0>(
        sX, nt, nvec, stage_pieces(C), tid,
        [&](int u) { return src + static_cast<size_t>(u) * C; });
    __builtin_amdgcn_s_waitcnt(0);  // this wave's slice loads have landed
    __syncthreads();
    if (has_tile) tile_linear(wt, sX, nvec, nt, ksteps, sO, col0, n, g);
    __syncthreads();
    uint16_t* o = out + static_cast<size_t>(row0) * C + c0;
    for (int i = tid; i < nt * ovec; i += kThreads) {
        const int u = i / ovec, pv = i - u * ovec;
        const uint4 v = *reinterpret_cast<const uint4*>(sO + u * kOutRow + 8 * pv);
        __builtin_nontemporal_store(
            u32x4_t{v.x, v.y, v.z, v.w},
            reinterpret_cast<u32x4_t*>(o + static_cast<size_t>(u) * C + 8 * pv));
    }
}

}  // namespace

int proj_qkv_lds_bytes(const Params& p) { return proj_lds_bytes(p.C); }

hipError_t launch_proj_qkv(const Params& p, const void* x, const void* w_qkv,
                           const float* b_qkv, void* qs, void* ks, void* vs, double* means,
                           const float* lepe_w, uint2* lepe_table, hipStream_t stream) {
    Params pp = p;
    if (!lepe_w) pp.table_items = 0;
    const int group = proj_group(p.C, p.t);
    const int gpi = (p.R + group - 1) / group;
    const int tasks = p.B * gpi * (3 * proj_chunks(p.C) / proj_units(p.C));
    const int table_blocks = (pp.table_items + kThreads - 1) / kThreads;
    const dim3 grid(tasks + table_blocks), block(kThreads);
    const int lds = proj_lds_bytes(p.C);
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

hipError_t launch_proj_out(const Params& p, const void* y, const void* w_o, const float* b_o,
                           void* out, hipStream_t stream) {
    const int ntok = p.B * p.H * p.W;
    const int tasks = ((ntok + proj_slice(p.C) - 1) / proj_slice(p.C)) * proj_chunks(p.C);
    const uint16_t* yy = static_cast<const uint16_t*>(y);
    const uint16_t* ww = static_cast<const uint16_t*>(w_o);
    uint16_t* oo = static_cast<uint16_t*>(out);
    const dim3 grid(tasks), block(kThreads);
    const int lds = proj_lds_bytes(p.C);
#define BRA_PROJ_OUT(HEADS) \
    hipLaunchKernelGGL(proj_out_kernel<HEADS>, grid, block, lds, stream, yy, ww, b_o, oo, ntok, p.C)
    // the channel counts of the BiFormer stages are compiled with C fixed
    switch (p.C) {
        case 64: BRA_PROJ_OUT(2); break;
        case 128: BRA_PROJ_OUT(4); break;
        case 256: BRA_PROJ_OUT(8); break;
        case 512: BRA_PROJ_OUT(16); break;
        default: BRA_PROJ_OUT(0);
    }
#undef BRA_PROJ_OUT
    return hipGetLastError();
}

}  // namespace bra
