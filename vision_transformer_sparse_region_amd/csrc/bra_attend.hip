// bra_attend.hip -- token attention over the routed regions plus LePE, one
// workgroup per (image, region), all heads (page keys in bra_device.h).
//
//   1  issue every load at once: the routed region ids of this region
//      (written by a routing kernel) -- or, when this kernel routes (at most
//      64 regions, at most 4 heads), the K means of the image --, the LePE
//      weights or Toeplitz operands, the V window with its 2-token halo, the
//      first job's Q operands                                  [P5 §五 ⑤]
//   1b in-kernel routing: the Q means from the Q operands (fp64 sums, exact
//      within the span condition of row16_sum_exact),
//      the affinity with every region -- screened with fp32 K means and an
//      error bound, the fp64 affinities where the bound cannot decide --,
//      arg-max or bitonic top-k, wave h for head h
//                                              [P4 §1.2; P1 §2.1; P5 §五 ③-④]
//   2  each wave issues the gathers of its first two routed K/V chunks ...
//   3  ... the halo goes to LDS and the 5x5 depthwise LePE of V runs while
//      those loads are in flight                       [P5 §五 lepe, ⑧; P2 §2.2]
//   4  token attention over the routed tokens: S^T = K Q^T and O^T += V^T P^T
//      on bf16 MFMA (fp32 VALU for fp32 input), fp32 online softmax, the next
//      chunk's gather in flight during each chunk         [P3 §2.2; P5 §五 ⑤-⑦]
//   5  out = LePE + O, one rounding, 16-byte NHWC stores; or, with the
//      module's output projection, (LePE + O) W_o^T + b_o on MFMA  [P5 §五 ⑧]
// The routed K/V tokens are never copied to HBM: [P3 §4.2] and [P1 §2.2]
// build a dense k-fold gathered tensor with torch.gather; here the routing
// index drives the loads straight into MFMA operands.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bra_device.h"
#include "bra_shapes.h"

namespace bra {
namespace {

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
        const JobShape js = job_shape(p.t, p.heads);
        QT = js.QT;
        tpg = js.tpg;
        G = js.G;
        njobs = js.njobs;
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
// query (qt0 + jq) * 16 + li of head h.  Query slots past the window (and
// tiles past the job's) load the window's last token instead: their score
// columns are independent of the others and are never stored, and the load
// stays unconditional.
__device__ __forceinline__ void load_q_operands(const Params& p, const WaveJobs& J, int job,
                                                const uint16_t* __restrict__ qimg, int r,
                                                bf16x8_t (&qb)[kMaxQTiles]) {
    const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
    const int h = job / J.G, grp = job - h * J.G;
    const int qt0 = grp * J.tpg;
#pragma unroll
    for (int jq = 0; jq < kMaxQTiles; ++jq) {
        const int qi = min((qt0 + jq) * 16 + li, p.t - 1);
        const uint4 u = *reinterpret_cast<const uint4*>(qimg + token_offset(p, r, qi) +
                                                        h * kHeadDim + 8 * g);
        qb[jq] = __builtin_bit_cast(bf16x8_t, u);
    }
}

// Word 3 of a raw buffer descriptor on gfx9-family chips (gfx950 included).
constexpr int kBufferDword3 = 0x00020000;

// Gather of chunk c of local job jl into `g8`.  sOff holds, per (head, rank),
// the element offset of the routed region's first token.  Keys past the
// routed set (a ragged last chunk) re-read the last key: their scores are
// masked to -inf, so they weigh nothing, and every load stays unconditional.
// The K half fills g8.ka (MFMA operands as loaded), the V half g8.vv.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t image_rsrc(const Params& p,
                                                            const uint16_t* img) {
    // buffer loads: a 32-bit byte offset per lane against the image's base
    // in a buffer descriptor (no 64-bit address arithmetic per load)
    const uint32_t map_bytes = static_cast<uint32_t>(p.kH) * p.kW * p.C * 2u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(img), 0,
                                             static_cast<int>(map_bytes), kBufferDword3);
}
__device__ __forceinline__ void gather_k_chunk(const Params& p, const WaveJobs& J, int w, int jl,
                                               int c, const uint16_t* __restrict__ kimg,
                                               const int* sOff, StepRegs& g8) {
    const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
    const int h = (w + kWaves * jl) / J.G;
    const int* off = sOff + h * p.k;
    const __amdgpu_buffer_rsrc_t krs = image_rsrc(p, kimg);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int key = min(32 * c + 8 * (li >> 2) + 4 * blk + (li & 3), p.nkeys - 1);
        const int j = key / p.kt, slot = key - j * p.kt;
        const int e = off[j] + slot_offset_kv(p, slot) + h * kHeadDim + 8 * g;
        g8.ka[blk] = __builtin_bit_cast(bf16x8_t,
                                        __builtin_amdgcn_raw_buffer_load_b128(krs, 2 * e, 0, 0));
    }
}
__device__ __forceinline__ void gather_v_chunk(const Params& p, const WaveJobs& J, int w, int jl,
                                               int c, const uint16_t* __restrict__ vimg,
                                               const int* sOff, StepRegs& g8) {
    const int lane = threadIdx.x & 63;
    const int h = (w + kWaves * jl) / J.G;
    const int* off = sOff + h * p.k;
    const __amdgpu_buffer_rsrc_t vrs = image_rsrc(p, vimg);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        const int pc = lane + 64 * pp;
        const int key = min(32 * c + (pc >> 2), p.nkeys - 1);
        const int j = key / p.kt, slot = key - j * p.kt;
        const int e = off[j] + slot_offset_kv(p, slot) + h * kHeadDim + 8 * (pc & 3);
        g8.vv[pp] = __builtin_bit_cast(uint4,
                                       __builtin_amdgcn_raw_buffer_load_b128(vrs, 2 * e, 0, 0));
    }
}
__device__ __forceinline__ void gather_chunk(const Params& p, const WaveJobs& J, int w, int jl,
                                             int c, const uint16_t* __restrict__ kimg,
                                             const uint16_t* __restrict__ vimg, const int* sOff,
                                             StepRegs& g8) {
    gather_k_chunk(p, J, w, jl, c, kimg, sOff, g8);
    gather_v_chunk(p, J, w, jl, c, vimg, sOff, g8);
}

// Gathers of the shared-V windows (64 tokens, so a pair of 32-key chunks is
// exactly one routed region): within a pair every lane reads the same
// offsets from the region's first token, so they are computed once, and the
// region's base is wave-uniform (the buffer loads' scalar offset).
struct PairLanes {
    int k[2][2];  // K operand piece of chunk ch, block blk
    int v[2];     // the two V pieces of this wave's chunk
};
__device__ __forceinline__ PairLanes pair_lanes(const Params& p, int h, int mine) {
    const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
    PairLanes L;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
            L.k[ch][blk] = 2 * (slot_offset_kv(p, 32 * ch + 8 * (li >> 2) + 4 * blk + (li & 3)) +
                                h * kHeadDim + 8 * g);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        const int pc = lane + 64 * pp;
        L.v[pp] = 2 * (slot_offset_kv(p, 32 * mine + (pc >> 2)) + h * kHeadDim + 8 * (pc & 3));
    }
    return L;
}
// Byte offset of routed region j of head h (wave-uniform).
__device__ __forceinline__ int pair_base(const Params& p, const int* sOff, int h, int j) {
    return __builtin_amdgcn_readfirstlane(2 * sOff[h * p.k + j]);
}
__device__ __forceinline__ void gather_k_pair(const PairLanes& L, __amdgpu_buffer_rsrc_t krs,
                                              int base, StepRegs (&ring)[2]) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
            ring[ch].ka[blk] = __builtin_bit_cast(
                bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(krs, L.k[ch][blk], base, 0));
}
__device__ __forceinline__ void gather_v_mine(const PairLanes& L, __amdgpu_buffer_rsrc_t vrs,
                                              int base, StepRegs& g8) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
        g8.vv[pp] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, L.v[pp], base, 0));
}

// Chunk `ch` (0 or 1) of pair u of local job jl, if it exists.
__device__ __forceinline__ bool pair_chunk(const WaveJobs& J, int u, int ch) {
    return 2 * u + ch < J.nchunks;
}

// V chunk (in registers, one 16-byte piece per lane and half) through an LDS
// buffer -- the wave's own, or, for the shared-V windows, one its head's two
// waves share -- read back as the two V^T operands of O^T += V^T P^T.
// A staged row (one key) is 32 dims = 8 units of 8 bytes (dims 4u .. 4u+3);
// unit u of row r sits at slot u ^ vt_swizzle(r).  Rows two apart (and, with
// 64 banks, four and eight apart) would otherwise meet on the same banks --
// in the writes, where a 16-lane group writes units of the same parity to
// four rows, and in the transposing reads, where it reads units 4db .. 4db+3
// of four rows: bit 1 of the row flips a unit's parity and its half (5),
// bit 2 its parity (1), bit 3 its half (4).
__device__ __forceinline__ int vt_swizzle(int r) {
    return (((r >> 1) & 1) * 5) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) * 4);
}
// The staging writes (one chunk, 32 keys) and the transposing reads.
__device__ __forceinline__ void v_stage(const StepRegs& cur, uint16_t* sVt) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        const int pc = lane + 64 * pp, row = pc >> 2, q = pc & 3, sw = vt_swizzle(row);
        uint2* dst = reinterpret_cast<uint2*>(sVt + row * kVtRow);
        dst[(2 * q) ^ sw] = uint2{cur.vv[pp].x, cur.vv[pp].y};
        dst[(2 * q + 1) ^ sw] = uint2{cur.vv[pp].z, cur.vv[pp].w};
    }
}
__device__ __forceinline__ void v_read_t(const uint16_t* sVt, bf16x8_t (&va)[2]) {
    const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
    // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element
    // i % 4 of the 8-byte pieces that lanes i / 4, 4 + i / 4, 8 + i / 4 and
    // 12 + i / 4 read.  Lane 4r + a of group g reads dims 16 db + 4a .. + 3 of
    // key 8g + r (then 8g + 4 + r), so lane i gets dim 16 db + i of keys
    // 8g .. 8g + 3 (then 8g + 4 .. 8g + 7): the operand, without repacking.
    const int tr_r = li >> 2, tr_a = li & 3;
    const int r_lo = 8 * g + tr_r, r_hi = r_lo + 4;
    const int sw_lo = vt_swizzle(r_lo), sw_hi = vt_swizzle(r_hi);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const int unit = 4 * db + tr_a;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(sVt + r_lo * kVtRow + 4 * (unit ^ sw_lo)));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(sVt + r_hi * kVtRow + 4 * (unit ^ sw_hi)));
        va[db] = __builtin_bit_cast(
            bf16x8_t, u32x4_t{__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                              __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]});
        // (unscheduled, the reads of both halves bunch up and the long-key
        // loop spills)
        __builtin_amdgcn_sched_barrier(0);
    }
}
// One chunk through the wave's own buffer.  A wave's LDS operations complete
// in order; the fences keep the compiler from moving the transposed reads
// above the writes, or the next chunk's writes above these reads.
__device__ __forceinline__ void v_transpose(const StepRegs& cur, uint16_t* sVt,
                                            bf16x8_t (&va)[2]) {
    v_stage(cur, sVt);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    v_read_t(sVt, va);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Token attention of one wave's jobs.  Keys are taken 64 at a time (a pair
// of 32-key chunks, held in the two register sets of `ring`): scores of both
// chunks, one max and one exponent pass, then both P.V products.  When a
// job's routed keys fit in 64 (every BiFormer stage), this is a plain
// softmax with no rescaling; longer key lists carry an online softmax across
// pairs.  The next pair's gathers are issued as soon as this pair's K and V
// registers are consumed.
template <int N>
struct NextTag {
    static constexpr int value = N;
};
template <bool SHARE_V>
__device__ __forceinline__ void attend_mfma(const Params& p, const WaveJobs& J, const uint16_t* __restrict__ qimg,
                            const uint16_t* __restrict__ kimg, const uint16_t* __restrict__ vimg,
                            int r, uint16_t* sVt_all, float* sL, const int* sOff,
                            StepRegs (&ring)[2], bf16x8_t (&qb)[kMaxQTiles], bool sum_mfma) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    uint16_t* sVt = sVt_all + w * 32 * kVtRow;
    const int npair = (J.nchunks + 1) / 2;
    // (SHARE_V: one job per wave, whole pairs, one routed region per pair)
    const PairLanes pl = SHARE_V ? pair_lanes(p, w / J.G, w & 1) : PairLanes{};
    const __amdgpu_buffer_rsrc_t krs = image_rsrc(p, kimg), vrs = image_rsrc(p, vimg);
    const int njl = J.nchunks > 0 ? J.nsteps / J.nchunks : 0;  // this wave's jobs

    // Softmax denominator.  sum_mfma (long key lists, where the VALU softmax
    // is the bound): an all-ones A operand sums P over a chunk's 32 keys on
    // the MFMA (every row of the product is that sum; element 0 is kept and
    // rescaled).  Otherwise (one pair of chunks: latency matters more than
    // VALU slots) each lane adds up its 16 exponentials and the four lane
    // groups are summed at the end.
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u,
                                                              0x3f803f80u, 0x3f803f80u});
    float m[kMaxQTiles];
    f32x4_t o0[kMaxQTiles], o1[kMaxQTiles], l[kMaxQTiles];
    // One pair step.  NEXT: 2, the next step's gathers are issued if there
    // is one (general path); 1, always (shared-V steps before the last); 0,
    // never (the shared-V last step).  The shared-V loop then issues its
    // loads in the same order on every path into the loop's head, which the
    // compiler's counts of loads in flight need to wait for only the oldest.
    auto step = [&](int ss, auto next_tag) {
        constexpr int NEXT = decltype(next_tag)::value;
        const int jl = ss / npair, u = ss - jl * npair;
        const int job = w + kWaves * jl;
        const int h = job / J.G, grp = job - h * J.G;
        const int qt0 = grp * J.tpg;
        const int nq = min(J.tpg, J.QT - qt0);
        const int hoff = h * kHeadDim;
        const bool two = pair_chunk(J, u, 1);
        // the first job's Q operands were loaded with its first gathers
        if (u == 0 && jl > 0) load_q_operands(p, J, job, qimg, r, qb);

        bf16x8_t va[2][2];
        if constexpr (SHARE_V) {
            // this wave's chunk of the pair (ring[0].vv) into its head's
            // buffer of this pair's parity; then the next pair's V chunk goes
            // out, and both chunks are read back once both waves have written
            // (the buffer of this parity is written again two pairs on, after
            // the next pair's barrier, which every wave passes only once its
            // reads of this one have returned)
            uint16_t* hb = sVt_all + ((ss & 1) * 2 + h) * 2 * 32 * kVtRow;
            v_stage(ring[0], hb + (w & 1) * 32 * kVtRow);
            if constexpr (NEXT == 1) gather_v_mine(pl, vrs, pair_base(p, sOff, h, u + 1), ring[0]);
            __syncthreads();
            v_read_t(hb, va[0]);
            v_read_t(hb + 32 * kVtRow, va[1]);
        } else {
            v_transpose(ring[0], sVt, va[0]);
            if (two) v_transpose(ring[1], sVt, va[1]);
        }

#pragma unroll
        for (int jq = 0; jq < kMaxQTiles; ++jq) {
            if (jq >= nq) break;
            // scores of both chunks: S^T = K Q^T, keys 64u + 32ch + 8g + e on
            // this lane
            f32x4_t sc[2][2];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                if (ch == 1 && !two) break;
                const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
                sc[ch][0] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[ch].ka[0], qb[jq], z4, 0, 0, 0);
                sc[ch][1] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[ch].ka[1], qb[jq], z4, 0, 0, 0);
            }
            // after the last tile's scores the K and V registers are consumed:
            // the next pair's gathers go out now
            if (jq == nq - 1) {
                const int nss = ss + 1, njl2 = nss / npair, nu = nss - njl2 * npair;
                if (NEXT == 1 || (NEXT == 2 && njl2 < njl)) {
                    if constexpr (SHARE_V) {
                        gather_k_pair(pl, krs, pair_base(p, sOff, h, nu), ring);
                    } else {
                        gather_chunk(p, J, w, njl2, 2 * nu, kimg, vimg, sOff, ring[0]);
                        if (pair_chunk(J, nu, 1))
                            gather_chunk(p, J, w, njl2, 2 * nu + 1, kimg, vimg, sOff, ring[1]);
                    }
                }
            }
            // raw scores; the running max is kept in raw units and the
            // scale * log2(e) factor enters each exponent through one FMA
            float x[2][8];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                const int kbase = 64 * u + 32 * ch + 8 * g;
                if (ch == 1 && !two) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[ch][e] = -INFINITY;
                    continue;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[ch][e] = sc[ch][0][e];
                    x[ch][4 + e] = sc[ch][1][e];
                }
                if (kbase + 8 > p.nkeys) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (kbase + e >= p.nkeys) x[ch][e] = -INFINITY;
                }
            }
            float mx = x[0][0];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (ch | e) mx = max_f(mx, x[ch][e]);
            mx = group4_max(mx);
            const float mnew = u == 0 ? mx : max_f(m[jq], mx);
            const float mb = mnew * p.scale_log2e;
            bf16x8_t pb[2];
            float psum = 0.f;
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pe = __builtin_amdgcn_exp2f(fmaf(x[ch][e], p.scale_log2e, -mb));
                    if (!sum_mfma) psum += pe;
                    pb[ch][e] = static_cast<__bf16>(pe);
                }
            if (u == 0) {
                l[jq] = f32x4_t{sum_mfma ? 0.f : psum, 0.f, 0.f, 0.f};
                o0[jq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                o1[jq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            } else {
                const float alpha = __builtin_amdgcn_exp2f((m[jq] - mnew) * p.scale_log2e);
                l[jq][0] = sum_mfma ? l[jq][0] * alpha : fmaf(l[jq][0], alpha, psum);
                o0[jq] *= alpha;
                o1[jq] *= alpha;
            }
            m[jq] = mnew;
            o0[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[0][0], pb[0], o0[jq], 0, 0, 0);
            o1[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[0][1], pb[0], o1[jq], 0, 0, 0);
            if (sum_mfma)
                l[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[0], l[jq], 0, 0, 0);
            if (two) {
                o0[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[1][0], pb[1], o0[jq], 0, 0, 0);
                o1[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[1][1], pb[1], o1[jq], 0, 0, 0);
                if (sum_mfma)
                    l[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[1], l[jq], 0, 0, 0);
            }
        }

        if (u == npair - 1) {
#pragma unroll
            for (int jq = 0; jq < kMaxQTiles; ++jq) {
                if (jq >= nq) break;
                const float inv =
                    __builtin_amdgcn_rcpf(sum_mfma ? l[jq][0] : group4_sum(l[jq][0]));
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
        };
    if constexpr (SHARE_V) {
        // one job per wave, so the steps are the job's pairs
        for (int ss = 0; ss + 1 < npair; ++ss) step(ss, NextTag<1>{});
        if (npair > 0) step(npair - 1, NextTag<0>{});
    } else {
        for (int ss = 0; ss < njl * npair; ++ss) step(ss, NextTag<2>{});
    }
}

// fp32 VALU token attention: 8 lanes per (query token, head), 4 dims each;
// keys in routed order with an online softmax, the next key's loads in
// flight while the current one is processed; fp32 throughout.
__device__ __forceinline__ void attend_valu(const Params& p, const float* __restrict__ qimg,
                            const float* __restrict__ kimg, const float* __restrict__ vimg, int r,
                            float* sL, const int* sOff) {
    const int sub = threadIdx.x & 7;
    for (int item = threadIdx.x >> 3; item < p.t * p.heads; item += kThreads / 8) {
        const int h = item / p.t, slot = item - h * p.t;
        const int hoff = h * kHeadDim + 4 * sub;
        const float4 qv = *reinterpret_cast<const float4*>(qimg + token_offset(p, r, slot) + hoff);
        const int* roff = sOff + h * p.k;
        float m = -INFINITY, l = 0.f;
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        int off = roff[0] + hoff;
        float4 kv = *reinterpret_cast<const float4*>(kimg + off);
        float4 vv = *reinterpret_cast<const float4*>(vimg + off);
        for (int key = 0; key < p.nkeys; ++key) {
            float4 kn = kv, vn = vv;
            if (key + 1 < p.nkeys) {
                const int j = (key + 1) / p.kt, ks = key + 1 - j * p.kt;
                const int o2 = roff[j] + slot_offset_kv(p, ks) + hoff;
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
        const float inv = __builtin_amdgcn_rcpf(l);
        float4* dst = reinterpret_cast<float4*>(sL + slot * p.lstride + hoff);
        const float4 a = *dst;
        *dst = float4{a.x + acc.x * inv, a.y + acc.y * inv, a.z + acc.z * inv, a.w + acc.w * inv};
    }
}

// One LePE work item: channels c0, c0+1 of window row y, columns xs..xs+7
// (fewer at the window's right edge), bias + 25 taps from the LDS halo.
// Weights come from LDS (sW, [C][25] then the bias [C]) or from global memory.
// The 50 weights of a thread's channel pair (c0, c0 + 1), loaded in the
// prologue when each thread has at most one LePE item and the weights are
// not in LDS: rows c0 and c0 + 1 of the [C][25] weights.
struct LepePairWeights {
    float w[50];
};

// NC: output columns per item, kLepeCols, or the window width of a fixed
// shape narrower than that (no work on columns past the window).
template <typename T, bool PRE, int NC>
__device__ __forceinline__ void lepe_item(const Params& p, const T* sVh, const float* wsrc,
                                          const LepePairWeights& pre, const float* bsrc, int c0,
                                          int y, int xs, int nx, float (&acc)[2][NC]) {
    float b0 = 0.f, b1 = 0.f;
    if (p.has_lepe && bsrc) {
        b0 = bsrc[c0];
        b1 = bsrc[c0 + 1];
    }
#pragma unroll
    for (int x = 0; x < NC; ++x) {
        acc[0][x] = b0;
        acc[1][x] = b1;
    }
    if (!p.has_lepe) return;
    const int hw = p.ws + 4;
    // (the rows unroll when the weights are in registers: they are indexed
    // by the row)
#pragma unroll(PRE ? 5 : 1)
    for (int i = 0; i < 5; ++i) {
        float w0[5], w1[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            w0[j] = PRE ? pre.w[i * 5 + j] : wsrc[c0 * 25 + i * 5 + j];
            w1[j] = PRE ? pre.w[25 + i * 5 + j] : wsrc[(c0 + 1) * 25 + i * 5 + j];
        }
        const T* row = sVh + ((y + i) * hw + xs) * p.C + c0;
        float in0[NC + 4], in1[NC + 4];
#pragma unroll
        for (int xx = 0; xx < NC + 4; ++xx) {
            float2 v2 = {0.f, 0.f};
            if (xx < nx + 4) v2 = Elem<T>::pair(row + xx * p.C);
            in0[xx] = v2.x;
            in1[xx] = v2.y;
        }
#pragma unroll
        for (int x = 0; x < NC; ++x)
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                acc[0][x] = fmaf(w0[j], in0[x + j], acc[0][x]);
                acc[1][x] = fmaf(w1[j], in1[x + j], acc[1][x]);
            }
    }
}

template <int NC>
__device__ __forceinline__ void store_lepe(const Params& p, float* sL, int c0, int y, int xs,
                                           int nx, const float (&acc)[2][NC]) {
#pragma unroll
    for (int x = 0; x < NC; ++x)
        if (x < nx)
            *reinterpret_cast<float2*>(sL + (y * p.ws + xs + x) * p.lstride + c0) =
                float2{acc[0][x], acc[1][x]};
}

// The whole LePE step: every (channel pair, row, column block) item, written
// to sL.  In alias mode sL overlays the halo, so the items (at most one per
// thread) are computed first and stored after a barrier.  Ends with a barrier.
template <typename T, bool PRE, int NC>
__device__ __forceinline__ void lepe_phase(const Params& p, const T* sVh, float* sL,
                                           const float* wsrc, const LepePairWeights& pre,
                                           const float* bsrc) {
    const int npairs = p.C / 2;
    const int nxb = (p.ws + kLepeCols - 1) / kLepeCols;
    float acc[2][NC];
    int mine = -1;
    for (int it = threadIdx.x; it < p.lepe_items; it += kThreads) {
        const int cp = it % npairs, rest = it / npairs;
        const int xb = rest % nxb, y = rest / nxb;
        const int xs = xb * kLepeCols, nx = min(kLepeCols, p.ws - xs);
        lepe_item<T, PRE, NC>(p, sVh, wsrc, pre, bsrc, 2 * cp, y, xs, nx, acc);
        if (p.lepe_alias)
            mine = it;
        else
            store_lepe<NC>(p, sL, 2 * cp, y, xs, nx, acc);
    }
    if (p.lepe_alias) {
        __syncthreads();  // every halo read is done before sL overwrites it
        if (mine >= 0) {
            const int cp = mine % npairs, rest = mine / npairs;
            const int xb = rest % nxb, y = rest / nxb;
            const int xs = xb * kLepeCols;
            store_lepe<NC>(p, sL, 2 * cp, y, xs, min(kLepeCols, p.ws - xs), acc);
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
// and the lane's column n.  The pool kernel writes each channel's 25 weights
// once per forward as a 64-byte row of bf16 (lepe_table_entry); the four
// lanes of a channel load a quarter of the row each and share the quarters by
// DPP, and each lane builds its ten operands: for tap row i, the eight bf16
// [0]*n, w[i][0..4], 0.. make the B operands of ks = 0 and 1.  Weights enter
// the product as bf16 (the accumulation is fp32).

// The Toeplitz B operands and the bias of this lane's channel in each of the
// wave's channel groups, built from the weight table the pool kernel wrote.
template <int HS, int WS, int HEADS>
struct LepeOperands {
    uint4 tb[LepeMfmaShape<HS, WS, HEADS>::GPW][5];  // 10 x 8 bytes per group
    float bias[LepeMfmaShape<HS, WS, HEADS>::GPW];
};

// `bias` is never NULL (a zero vector stands in for a missing bias); groups
// past the last one re-read the last group (they are never used).  Every lane
// of the wave runs this (the quads exchange their quarters by DPP).
template <int HS, int WS, int HEADS>
__device__ __forceinline__ void lepe_mfma_load(const uint2* __restrict__ table,
                                               const float* __restrict__ bias,
                                               LepeOperands<HS, WS, HEADS>& o) {
    using S = LepeMfmaShape<HS, WS, HEADS>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 3;
    // the shift of a lane's operands: 16 bits when n is odd, one word when n >= 2
    const bool half = (n & 1) != 0, word = n >= 2;
#pragma unroll
    for (int g = 0; g < S::GPW; ++g) {
        const int cg = min(w + kWaves * g, S::NG - 1);
        // taps 8n .. 8n + 7 of channel 16 cg + lane / 4
        const uint4 x4 =
            *reinterpret_cast<const uint4*>(table + (16 * cg + (lane >> 2)) * 8 + 2 * n);
        const uint32_t x[4] = {x4.x, x4.y, x4.z, x4.w};
        // word m of the row (taps 2m, 2m + 1), from lane m / 4 of the quad
        auto row_word = [&](int m) -> uint32_t {
            const int q = m >> 2, e = m & 3;
            const int v = static_cast<int>(x[e]);
            const int r = q == 0 ? __builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false)
                        : q == 1 ? __builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false)
                        : q == 2 ? __builtin_amdgcn_mov_dpp(v, 0xAA, 0xf, 0xf, false)
                                 : __builtin_amdgcn_mov_dpp(v, 0xFF, 0xf, 0xf, false);
            return static_cast<uint32_t>(r);
        };
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            // z = w[i][0..4], 0, 0, 0 as four words (taps 5i .. 5i + 4 start on
            // a half word when i is odd)
            uint32_t z[4];
            if ((5 * i) % 2 == 0) {
                const int m = 5 * i / 2;
                z[0] = row_word(m);
                z[1] = row_word(m + 1);
                z[2] = row_word(m + 2) & 0xffffu;
            } else {
                const int m = (5 * i - 1) / 2;
                const uint32_t a = row_word(m), b = row_word(m + 1), c = row_word(m + 2);
                z[0] = __builtin_amdgcn_alignbit(b, a, 16);
                z[1] = __builtin_amdgcn_alignbit(c, b, 16);
                z[2] = c >> 16;
            }
            z[3] = 0u;
            // shifted left by 16 n bits: [0]*n, w[i][0..4], 0 ..
            uint32_t e[4];
            e[0] = half ? z[0] << 16 : z[0];
#pragma unroll
            for (int k = 1; k < 4; ++k)
                e[k] = half ? __builtin_amdgcn_alignbit(z[k], z[k - 1], 16) : z[k];
            const uint32_t o0 = word ? 0u : e[0], o1 = word ? e[0] : e[1];
            const uint32_t o2 = word ? e[1] : e[2], o3 = word ? e[2] : e[3];
            o.tb[g][i] = uint4{o0, o1, o2, o3};
        }
        o.bias[g] = bias[16 * cg + (lane >> 2)];
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
            const uint16_t* plane = sVp + lepe_plane_offset(c, S::PS);
#pragma unroll
            for (int ty = 0; ty < S::TY; ++ty)
#pragma unroll
                for (int tx = 0; tx < S::TX; ++tx) {
                    // the accumulator starts at the channel's bias
                    f32x4_t d = {o.bias[g], o.bias[g], o.bias[g], o.bias[g]};
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
                            dacc[g][ty * S::TX + tx][e];
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Region Q mean from the Q operands [P4 §1.2; P2 §2.1; P5 §五 ③].  When every
// job is some wave's first job, the first Q operands of the waves hold each
// query of the region once: wave w (< njobs) sums, in fp64, the queries of
// its job (job w) for dims 8g..8g+7 of the job's head on lane row g, and
// stores the 32 sums at sQp[w][..].  Within the span condition of
// row16_sum_exact (bra_device.h) every partial sum of bf16 values is an
// exact fp64 number, so neither this split nor the order of the additions
// can change the total: it equals the pool kernel's and the plain loop's.
__device__ __forceinline__ void qmean_partial(const Params& p, const WaveJobs& J, int w,
                                              const bf16x8_t (&qb)[kMaxQTiles], double* sQp) {
    const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
    const int grp = w - (w / J.G) * J.G;
    const int qt0 = grp * J.tpg, nq = min(J.tpg, J.QT - qt0);
    double* dst = sQp + w * kHeadDim + 8 * g;
    // the lane's sums of its 8 dims over its tiles
    double sd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        double acc = 0.0;
#pragma unroll
        for (int jq = 0; jq < kMaxQTiles; ++jq) {
            // tiles past the job's and slots past the window hold duplicates
            // (no slot is past the window when it is a whole number of tiles)
            const bool in = jq < nq && (p.t % 16 == 0 || (qt0 + jq) * 16 + li < p.t);
            const u16x8_t u = __builtin_bit_cast(u16x8_t, qb[jq]);
            acc += in ? static_cast<double>(__uint_as_float(static_cast<uint32_t>(u[e]) << 16))
                      : 0.0;
        }
        sd[e] = acc;
    }
    // A reduce-scatter over the row's 16 lanes: each step adds the DPP
    // partner's half of the dims this lane keeps (partners 15 - li, then
    // 7 - li within each half, li ^ 2, li ^ 1), 8 additions in all instead
    // of 4 per dim; lane li ends with dim 4 [li >= 8] + 2 [li & 4] + [li & 2].
    const bool ha = li >= 8, hb = (li & 4) != 0, hc = (li & 2) != 0;
    double a[4], bb[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double send = ha ? sd[j] : sd[4 + j];
        a[j] = (ha ? sd[4 + j] : sd[j]) + dpp_f64<0x140>(send);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const double send = hb ? a[j] : a[2 + j];
        bb[j] = (hb ? a[2 + j] : a[j]) + dpp_f64<0x141>(send);
    }
    double c = (hc ? bb[1] : bb[0]) + dpp_f64<0x4E>(hc ? bb[0] : bb[1]);
    c += dpp_f64<0xB1>(c);
    if ((li & 1) == 0) dst[4 * ha + 2 * hb + hc] = c;
}


// ---------------------------------------------------------------------------
// Fixed shapes whose LePE runs on MFMA need little LDS; the fixed instances
// are compiled for four waves per SIMD (more waves per SIMD did not pay: the
// extra register pressure spills), the generic ones, whose runtime sizes
// keep more registers live, for three (at 128 registers they spilled 90 to
// 140).
template <typename T, int HS, int WS, int NW, int HEADS, int KTOP, bool FUSED>
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(HS > 0 && WS > 0 && NW > 0 && HEADS > 0 && KTOP > 0 ? 4 : 2, 8))) void
attend_kernel(const T* __restrict__ q, const T* __restrict__ v, const T* __restrict__ kg,
              const T* __restrict__ vg, const double* __restrict__ means,
              int32_t* __restrict__ routing,
              const float* __restrict__ lepe_w,
              const float* __restrict__ lepe_b, const float* __restrict__ lepe_bias,
              const uint2* __restrict__ lepe_table, const uint16_t* __restrict__ w_o,
              const float* __restrict__ b_o, T* __restrict__ out, Params p_in) {
    const Params p = fold_geometry<HS, WS, NW, HEADS, KTOP, Elem<T>::kVec>(p_in);
    // Where this kernel routes windows of at least 32 tokens (fixed shapes),
    // the prologue -- loads, Q means, routing, up to the first gathers -- runs
    // at raised wave priority: that chain decides when the workgroup's
    // gathers go out (stage 1: attention 36.5 -> 35.7 us; with 16-token
    // windows it measured 0.6 us slower).
    constexpr bool kPrioPrologue = HS > 0 && WS > 0 && NW > 0 && HEADS > 0 && KTOP > 0 &&
                                   FUSED && kmean32_pays(HS * WS);
    if constexpr (kPrioPrologue) __builtin_amdgcn_s_setprio(2);
    extern __shared__ __align__(16) unsigned char smem[];
    T* sVh = reinterpret_cast<T*>(smem + p.off_vh);
    float* sL = reinterpret_cast<float*>(smem + p.off_l);
    float* sW = reinterpret_cast<float*>(smem + p.off_w);
    int* sOff = reinterpret_cast<int*>(smem + p.off_idx);  // routed region bases
    const bool w_in_lds = p.off_w >= 0;

    constexpr int VEC = Elem<T>::kVec;
    constexpr bool kLepeMfma = VEC == 8 && LepeMfmaShape<HS, WS, HEADS>::ok;
    // 64-token windows of two heads: the two waves of a head share the
    // routed V chunks through LDS (every wave holds one job, so all take the
    // same number of pair steps and workgroup barriers)
    constexpr bool kShareV = VEC == 8 && HS > 0 && WS > 0 && NW > 0 && KTOP > 0 &&
                             share_v(HS, WS, HEADS);
    const int tid = threadIdx.x, w = tid >> 6;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int b = blk / p.R, r = blk - b * p.R;
    const int y0 = (r / p.n) * p.hs, x0 = (r % p.n) * p.ws;
    const size_t img = static_cast<size_t>(b) * p.H * p.W * p.C;
    const size_t kimg = static_cast<size_t>(b) * p.kH * p.kW * p.C;  // gathered K/V map
    const int nvec = p.C / VEC;
    const int hw = p.ws + 4;

    // 1. Issue every load that does not depend on the routing first.  The
    //    loads are unconditional (clamped, in-bounds addresses) and nothing
    //    reads a loaded value until all of them are issued: a value consumed
    //    inside a branch makes the wave wait for it there, serialising the
    //    loads behind it.
    //    LePE weights and bias (nw + nb 16-byte pieces, VALU LePE with
    //    weights in LDS): the first kWRegs pieces of each thread ride in
    //    registers and are stored once all loads are issued.
    const int nw = p.C * 25 / 4, nb = lepe_b ? p.C / 4 : 0;
    const bool stage_w = !kLepeMfma && w_in_lds && p.has_lepe;
    float4 wreg[kWRegs];
    if (stage_w) {
#pragma unroll
        for (int u = 0; u < kWRegs; ++u) {
            const int i = min(tid + u * kThreads, nw + nb - 1);
            wreg[u] = i < nw ? reinterpret_cast<const float4*>(lepe_w)[i]
                             : reinterpret_cast<const float4*>(lepe_b)[i - nw];
        }
    }
    // VALU LePE with the weights outside LDS and at most one item per thread
    // (fixed bf16 shapes only: elsewhere the 50 registers would spill): the
    // thread's 50 weights load now, with everything else, rather than one
    // tap row at a time inside the LePE
    constexpr bool kFixedShape = HS > 0 && WS > 0 && NW > 0 && HEADS > 0 && KTOP > 0;
    const bool pre_w = kFixedShape && VEC == 8 && !kLepeMfma && !w_in_lds && p.has_lepe &&
                       p.lepe_items <= kThreads;
    LepePairWeights pw;
    if (pre_w) {
        const int c0 = 2 * (min(tid, p.lepe_items - 1) % (p.C / 2));
#pragma unroll
        for (int e = 0; e < 50; ++e) pw.w[e] = lepe_w[c0 * 25 + e];
    }
    const int nhk = p.heads * p.k;
    const int wu = __builtin_amdgcn_readfirstlane(w);  // w, known wave-uniform
    WaveJobs J(p, w);
    bf16x8_t qb[kMaxQTiles];
    // In-kernel routing on bf16 maps whose jobs are all first jobs: the Q
    // means come from the first Q operands, which therefore load first.
    constexpr bool kFixed = HS > 0 && WS > 0 && NW > 0 && HEADS > 0 && KTOP > 0;
    const bool qm_here =
        FUSED && VEC == 8 &&
        (kFixed ? qmean_in_attend(true, true, HS * WS, HEADS) : p.qmean_attend != 0);
    if constexpr (FUSED && VEC == 8)
        load_q_operands(p, J, min(w, J.njobs - 1), reinterpret_cast<const uint16_t*>(q) + img, r,
                        qb);
    int ridx = 0;
    // routing waves: the K mean of region lane & 63, in fp32 when the
    // routing screens with it, else in fp64
    constexpr int kScreenFixed = kFixed ? (kmean32_pays(HS * WS) ? 1 : 0) : -1;
    const bool screen = kScreenFixed >= 0 ? kScreenFixed == 1 : p.kmean32 != 0;
    double kreg[kHeadDim];
    double qmean_lane = 0.0;  // routing waves: dim lane & 31 of the region's Q mean
    if constexpr (FUSED) {
        // In-kernel routing (R <= 64, heads <= 4): wave w routes this region
        // for head w; lane s holds the fp32 K mean of region s, loaded now
        // with everything else (the fp64 means only if the screen needs them).
        if (wu < p.heads) {
            if (screen)
                load_kmean32(p, means, b * p.heads + wu, min(tid & 63, p.R - 1), kreg);
            else
                load_kmean(p, means, b * p.heads + wu, min(tid & 63, p.R - 1), kreg);
            if (!qm_here) qmean_lane = means[qmean_index(p, b * p.heads + wu, r, tid & 31)];
        }
    } else {
        // the routed region ids of this region, one per (head, rank); lanes
        // past heads * k re-read the last one
        const int i = min(tid, nhk - 1);
        const int h = i / p.k, j = i - h * p.k;
        ridx = routing[((static_cast<size_t>(b) * p.rheads + (p.shared ? 0 : h)) * p.R + r) *
                           p.k +
                       j];
    }
    // (with in-kernel routing the LePE operands load after it: the K means
    // hold 32 or 64 registers until then)
    LepeOperands<kLepeMfma ? HS : 4, kLepeMfma ? WS : 4, kLepeMfma ? HEADS : 1> lop;
    if constexpr (kLepeMfma && !FUSED) lepe_mfma_load<HS, WS, HEADS>(lepe_table, lepe_bias, lop);
    // halo pieces kept in registers: all of them for a fixed shape (when they
    // fit kHaloRegs per thread), kHaloRegs otherwise.  Cells outside the map
    // load a clamped in-map cell and are zeroed when staged (bit u of hvalid).
    // For the MFMA LePE (channel-planar halo) a task can be 4 consecutive
    // cells of one halo row times one 16-byte channel piece, so that each
    // channel plane takes one 8-byte LDS write per task instead of four
    // 2-byte ones; taken where it needs no more registers than one cell per
    // task (stage 2: 4 either way; 8 x 8 windows would need 8 instead of 5,
    // and measured slower).
    constexpr int kHaloFixed =
        (HS > 0 && WS > 0 && HEADS > 0)
            ? ((HS + 4) * (WS + 4) * (HEADS * kHeadDim / VEC) + kThreads - 1) / kThreads
            : kHaloRegs;
    constexpr int kHR1 = kHaloFixed < kHaloRegs ? kHaloFixed : kHaloRegs;
    constexpr int kHTasks4 =
        kLepeMfma ? (HS + 4) * ((WS + 4) / 4) * (HEADS * kHeadDim / 8) : 0;
    constexpr bool kHalo4 = kLepeMfma && 4 * ((kHTasks4 + kThreads - 1) / kThreads) <= kHR1;
    constexpr int kHTask = kHalo4 ? 4 : 1;  // cells per task
    constexpr int kHTasks = kHalo4 ? kHTasks4 : 0;
    constexpr int kHR = kHalo4 ? (kHTasks + kThreads - 1) / kThreads : kHR1;
    static_assert(kHR * kHTask <= 32, "one validity bit per halo register");
    uint4 hreg[kHR * kHTask];
    unsigned hvalid = 0;
    // The halo loads.  Where this kernel routes, they go out after the Q
    // means: issued before, they held each wave in the load queue that the
    // Q operands and K means, which the routing needs first, also wait on.
    auto issue_halo = [&]() {
        if constexpr (kHalo4) {
            constexpr int NV = HEADS * kHeadDim / 8, GX = (WS + 4) / 4;
#pragma unroll
            for (int u = 0; u < kHR; ++u) {
                const int task = tid + u * kThreads;
                const int tc = min(task, kHTasks - 1);
                const int pv = tc % NV, cg = tc / NV, hy = cg / GX, gx = cg - hy * GX;
                const int y = y0 + hy - 2, yc = min(max(y, 0), p.H - 1);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int x = x0 + 4 * gx + j - 2, xc = min(max(x, 0), p.W - 1);
                    hreg[u * 4 + j] =
                        *reinterpret_cast<const uint4*>(v + img + (yc * p.W + xc) * p.C + pv * 8);
                    if (task < kHTasks && y == yc && x == xc) hvalid |= 1u << (u * 4 + j);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < kHR; ++u) {
                const int i = tid + u * kThreads;
                const int ic = min(i, p.halo_pieces - 1);
                const int cell = ic / nvec, pv = ic - cell * nvec;
                const int hy = cell / hw, hx = cell - hy * hw;
                const int y = y0 + hy - 2, x = x0 + hx - 2;
                const int yc = min(max(y, 0), p.H - 1), xc = min(max(x, 0), p.W - 1);
                hreg[u] = *reinterpret_cast<const uint4*>(v + img + (yc * p.W + xc) * p.C + pv * VEC);
                if (i < p.halo_pieces && y == yc && x == xc) hvalid |= 1u << u;
            }
        }
    };
    if constexpr (!FUSED) issue_halo();
    if constexpr (!FUSED && VEC == 8)
        load_q_operands(p, J, min(w, J.njobs - 1), reinterpret_cast<const uint16_t*>(q) + img, r,
                        qb);
    // The element offset of each routed region's first token goes to LDS.
    // Region ids are clamped into range, so a routing buffer holding garbage
    // (non-finite inputs) cannot send the gather outside the image.  (Every
    // thread stores: those past heads * k rewrite the last entry with the
    // value it already gets, so the store needs no branch.)
    if constexpr (FUSED) {
        if (qm_here) {
            // partial Q sums of every wave's first job, then wave h adds up
            // those of head h's jobs (jobs h*G .. h*G + G - 1).  With one
            // group per head, wave h's own job is head h's whole region: no
            // other wave's sums are needed, and no workgroup barrier.
            double* sQp = reinterpret_cast<double*>(smem + p.off_vt);  // [kWaves][32]
            const int G = kFixed ? job_shape(HS * WS, HEADS).G : J.G;
            if (G == 1) {
                if (wu < p.heads) {
                    qmean_partial(p, J, wu, qb, sQp);
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    qmean_lane = mean_of(sQp[wu * kHeadDim + (tid & 31)], p.t);
                }
            } else {
                if (wu < J.njobs) qmean_partial(p, J, wu, qb, sQp);
                __syncthreads();
                if (wu < p.heads) {
                    double sum = 0.0;
                    for (int j = 0; j < G; ++j) sum += sQp[(wu * G + j) * kHeadDim + (tid & 31)];
                    qmean_lane = mean_of(sum, p.t);
                }
            }
        }
        issue_halo();
        if (wu < p.heads) {
            const size_t row = (static_cast<size_t>(b) * p.heads + wu) * p.R + r;
            route_row_wave(p, qmean_lane, screen, kreg, means, b * p.heads + wu,
                           sOff + wu * p.k, routing + row * p.k);
        }
        if constexpr (kLepeMfma) lepe_mfma_load<HS, WS, HEADS>(lepe_table, lepe_bias, lop);
    } else {
        sOff[min(tid, nhk - 1)] = region_base_kv(p, min(max(ridx, 0), p.R - 1));
        for (int i = tid + kThreads; i < nhk; i += kThreads) {
            const int h = i / p.k, j = i - h * p.k;
            const int x = routing[((static_cast<size_t>(b) * p.rheads + (p.shared ? 0 : h)) *
                                       p.R +
                                   r) *
                                      p.k +
                                  j];
            sOff[i] = region_base_kv(p, min(max(x, 0), p.R - 1));
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

    // 2. LePE with weights from global memory runs before the gather is
    //    issued (a load queued behind the gather would wait for it); its halo
    //    goes to LDS first.
    const float* wsrc = w_in_lds ? sW : lepe_w;
    const float* bsrc = w_in_lds ? (lepe_b ? sW + p.C * 25 : nullptr) : lepe_b;
    auto halo_store = [&](int i, uint4 val) {
        const int cell = i / nvec, pv = i - cell * nvec;
        if constexpr (kLepeMfma) {
            using S = LepeMfmaShape<HS, WS, HEADS>;
            // channels 8 pv + e (e < 8) share the 4-element step of 8 pv
            uint16_t* dst =
                reinterpret_cast<uint16_t*>(sVh) + lepe_plane_offset(8 * pv, S::PS) + cell;
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
    auto stage_halo = [&]() {
        if constexpr (kHalo4) {
            // channel c = 8 pv + e of the task's 4 cells: bf16 e of each
            // cell's piece, two cells to a 32-bit word
            using S = LepeMfmaShape<HS, WS, HEADS>;
            constexpr int NV = HEADS * kHeadDim / 8, GX = (WS + 4) / 4;
            if (p.has_lepe) {
#pragma unroll
                for (int u = 0; u < kHR; ++u) {
                    const int task = tid + u * kThreads;
                    if (task < kHTasks) {
                        const int pv = task % NV, cg = task / NV, hy = cg / GX, gx = cg - hy * GX;
                        uint32_t wd[4][4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const unsigned mk = 0u - ((hvalid >> (u * 4 + j)) & 1u);
                            wd[j][0] = hreg[u * 4 + j].x & mk;
                            wd[j][1] = hreg[u * 4 + j].y & mk;
                            wd[j][2] = hreg[u * 4 + j].z & mk;
                            wd[j][3] = hreg[u * 4 + j].w & mk;
                        }
                        uint16_t* base = reinterpret_cast<uint16_t*>(sVh) +
                                         lepe_plane_offset(8 * pv, S::PS) + hy * S::HWP +
                                         4 * gx;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int sh = 16 * (e & 1);
                            const uint32_t c0 = (wd[0][e >> 1] >> sh) & 0xffffu;
                            const uint32_t c1 = (wd[1][e >> 1] >> sh) & 0xffffu;
                            const uint32_t c2 = (wd[2][e >> 1] >> sh) & 0xffffu;
                            const uint32_t c3 = (wd[3][e >> 1] >> sh) & 0xffffu;
                            *reinterpret_cast<uint2*>(base + e * S::PS) =
                                uint2{c0 | (c1 << 16), c2 | (c3 << 16)};
                        }
                    }
                }
            }
            __syncthreads();
            return;
        }
        if (p.has_lepe) {
#pragma unroll
            for (int u = 0; u < kHR; ++u) {
                const int i = tid + u * kThreads;
                // cells outside the map are zero (a mask, not a branch)
                const unsigned mk = 0u - ((hvalid >> u) & 1u);
                if (i < p.halo_pieces)
                    halo_store(i, uint4{hreg[u].x & mk, hreg[u].y & mk, hreg[u].z & mk,
                                        hreg[u].w & mk});
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
    };
    const bool early_lepe = !kLepeMfma && !w_in_lds;
    // VALU LePE columns per item: a fixed window narrower than kLepeCols
    // computes only its own columns
    constexpr int kLepeNC = WS > 0 && WS < kLepeCols ? WS : kLepeCols;
    if (early_lepe) {
        stage_halo();
        if constexpr (kFixedShape && VEC == 8 && !kLepeMfma) {
            if (pre_w) {
                lepe_phase<T, true, kLepeNC>(p, sVh, sL, wsrc, pw, bsrc);
            } else {
                lepe_phase<T, false, kLepeNC>(p, sVh, sL, wsrc, pw, bsrc);
            }
        } else {
            lepe_phase<T, false, kLepeNC>(p, sVh, sL, wsrc, pw, bsrc);
        }
    }

    // 3. Each wave issues the gathers of its first two (job, chunk) steps;
    //    the LePE runs while they are in flight.
    StepRegs ring[2];
    if constexpr (VEC == 8) {
        if (J.nsteps > 0) {
            const uint16_t* kgi = reinterpret_cast<const uint16_t*>(kg) + kimg;
            const uint16_t* vgi = reinterpret_cast<const uint16_t*>(vg) + kimg;
            if constexpr (kShareV) {
                // V only of this wave's chunk (w & 1), then both K chunks:
                // the order the pair loop issues them in (V of a pair one pair
                // ahead of its K), so that its waits count the same loads
                const PairLanes pl = pair_lanes(p, w / J.G, w & 1);
                const int base = pair_base(p, sOff, w / J.G, 0);
                gather_v_mine(pl, image_rsrc(p, vgi), base, ring[0]);
                gather_k_pair(pl, image_rsrc(p, kgi), base, ring);
            } else {
#pragma unroll
                for (int ch = 0; ch < 2; ++ch)
                    if (ch < J.nchunks) gather_chunk(p, J, w, 0, ch, kgi, vgi, sOff, ring[ch]);
            }
        }
    }
    if constexpr (kPrioPrologue) __builtin_amdgcn_s_setprio(0);
    if (!early_lepe) {
        stage_halo();
        if constexpr (kLepeMfma) {
            if (p.has_lepe) {
                lepe_mfma_compute<HS, WS, HEADS>(p, reinterpret_cast<const uint16_t*>(sVh), sL,
                                                 lop);
            } else {
                for (int i = tid; i < p.t * p.lstride; i += kThreads) sL[i] = 0.f;
                __syncthreads();
            }
        } else {
            lepe_phase<T, false, kLepeNC>(p, sVh, sL, wsrc, pw, bsrc);
        }
    }

    // 4. Token attention over the routed tokens, added into sL.
    if constexpr (VEC == 8) {
        // the denominator on the MFMA for key lists longer than one pair of chunks
        constexpr bool kFixedKeys = HS > 0 && WS > 0 && KTOP > 0;
        const bool sum_mfma = kFixedKeys ? KTOP * HS * WS > 64 : p.nkeys > 64;
        attend_mfma<kShareV>(p, J, reinterpret_cast<const uint16_t*>(q) + img,
                    reinterpret_cast<const uint16_t*>(kg) + kimg,
                    reinterpret_cast<const uint16_t*>(vg) + kimg, r,
                    reinterpret_cast<uint16_t*>(smem + p.off_vt), sL, sOff, ring, qb, sum_mfma);
    } else {
        attend_valu(p, reinterpret_cast<const float*>(q) + img,
                    reinterpret_cast<const float*>(kg) + kimg,
                    reinterpret_cast<const float*>(vg) + kimg, r, sL, sOff);
    }
    __syncthreads();

    // 5. out = LePE + O, one rounding, 16-byte NHWC stores -- or, with the
    //    output projection [P5 §五 ⑧ proj; P4 §1.1], out = (LePE + O) W_o^T + b_o
    //    on MFMA: out^T tile = W_o[o0 .. o0+15, :] . Y^T, operand A row m the
    //    Linear weight row o0 + m, operand B column n token n of the tile (its
    //    fp32 row of LePE + O from LDS, rounded to bf16); lane (n, g) receives
    //    output channels o0 + 4g .. o0 + 4g + 3 of token n, rounded once.
    if constexpr (VEC == 8) {
        if (p.out_proj) {
            const int lane = tid & 63, n = lane & 15, g = lane >> 4;
            const int otiles = p.C / 16, ttiles = (p.t + 15) / 16, ksteps = p.C / 32;
            constexpr int kMaxSteps = kMaxChannels / 32;
            // wave w takes output tiles w, w + kWaves, ...: the tile's weight
            // operands are loaded once and serve every token tile
            for (int ot = w; ot < otiles; ot += kWaves) {
                const int o0 = ot * 16, c = o0 + 4 * g;
                uint4 a[kMaxSteps > 16 ? 16 : kMaxSteps];
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    if (s < ksteps)
                        a[s] = *reinterpret_cast<const uint4*>(
                            w_o + static_cast<size_t>(o0 + n) * p.C + 32 * s + 8 * g);
                float bo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) bo[i] = b_o ? b_o[c + i] : 0.f;
                for (int tt = 0; tt < ttiles; ++tt) {
                    const int tok = tt * 16 + n;
                    const float* yrow = sL + min(tok, p.t - 1) * p.lstride;
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        if (s < ksteps) {
                            const float4 y0 =
                                *reinterpret_cast<const float4*>(yrow + 32 * s + 8 * g);
                            const float4 y1 =
                                *reinterpret_cast<const float4*>(yrow + 32 * s + 8 * g + 4);
                            const u32x4_t yb = {f32_to_bf16(y0.x) | (f32_to_bf16(y0.y) << 16),
                                                f32_to_bf16(y0.z) | (f32_to_bf16(y0.w) << 16),
                                                f32_to_bf16(y1.x) | (f32_to_bf16(y1.y) << 16),
                                                f32_to_bf16(y1.z) | (f32_to_bf16(y1.w) << 16)};
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, a[s]),
                                __builtin_bit_cast(bf16x8_t, yb), acc, 0, 0, 0);
                        }
                    if (tok < p.t) {
                        const uint32_t lo =
                            f32_to_bf16(acc[0] + bo[0]) | (f32_to_bf16(acc[1] + bo[1]) << 16);
                        const uint32_t hi =
                            f32_to_bf16(acc[2] + bo[2]) | (f32_to_bf16(acc[3] + bo[3]) << 16);
                        __builtin_nontemporal_store(
                            u32x2_t{lo, hi},
                            reinterpret_cast<u32x2_t*>(out + img + token_offset(p, r, tok) + c));
                    }
                }
            }
            return;
        }
    }
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
            // streaming store: the output is not re-read, so it should not sit
            // dirty in L2 for the next kernel to write back
            __builtin_nontemporal_store(u32x4_t{u.x, u.y, u.z, u.w},
                                        reinterpret_cast<u32x4_t*>(dst));
        } else {
            __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(src),
                                        reinterpret_cast<f32x4_t*>(dst));
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
static long align16(long x) { return (x + 15) & ~15L; }

bool plan(Params& p, int B, int H, int W, int C, int heads, int n_win, int k, float scale,
          bool bf16, bool shared, int kv_ratio) {
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
    p.shared = shared ? 1 : 0;
    p.rheads = shared ? 1 : heads;
    p.kv_ratio = kv_ratio;
    p.kH = H / kv_ratio;
    p.kW = W / kv_ratio;
    p.khs = p.hs / kv_ratio;
    p.kws = p.ws / kv_ratio;
    p.kt = p.khs * p.kws;
    p.nkeys = k * p.kt;
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
    // per-wave V^T staging (bf16 attention); before the attention, the
    // partial Q sums of each wave (32 doubles)
    const long vt_bytes = !bf16 ? 0L
                          : (is_fixed_shape(p, bf16) && share_v(p.hs, p.ws, heads))
                              ? static_cast<long>(kVtSharedBytes)
                              : static_cast<long>(kWaves) * 32 * kVtRow * 2;
    p.off_vt = take(std::max(vt_bytes,
                             static_cast<long>(kWaves) * kHeadDim * 8));
    // The fixed bf16 shapes whose windows tile by 4x4 run LePE on MFMA with a
    // channel-planar halo; the others on VALU with an NHWC halo.
    p.lepe_mfma = bf16 && is_fixed_shape(p, bf16) && lepe_mfma_fits(p.hs, p.ws, heads);
    const long vh_bytes =
        p.lepe_mfma ? static_cast<long>(lepe_plane_offset(C, lepe_plane_stride(p.hs, p.ws))) * 2
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
    // VALU LePE: weights and bias go to LDS while four workgroups still fit a CU.
    const long w_bytes = static_cast<long>(C) * 26 * 4;
    if (!p.lepe_mfma && off + w_bytes <= 40 * 1024) {
        p.off_w = take(w_bytes);
    } else {
        p.off_w = -1;
    }
    p.lds_bytes = static_cast<int>(off);
    p.table_items = p.lepe_mfma ? C * 8 : 0;
    p.qmean_attend = qmean_in_attend(bf16, route_in_attend(p), p.t, heads) ? 1 : 0;
    p.kmean32 = route_in_attend(p) && kmean32_pays(p.t) ? 1 : 0;
    {
        // wave path: one wave per (region, tensor), four waves per workgroup
        const int nvec = C / vec;
        const bool wave_path = bf16 && 64 % nvec == 0;
        const int per_block = p.qmean_attend ? kWaves : kWaves / 2;
        p.pool_blocks = wave_path ? (B * p.R + per_block - 1) / per_block : B * p.R;
    }
    p.pool_chunk = std::max(1, std::min(p.t, kPoolChunkBytes / (C * static_cast<int>(es))));
    // LDS of the pool kernel's staged path (fp32, or C/8 not dividing 64)
    p.pool_lds_bytes = p.pool_chunk * C * static_cast<int>(es);
    return off <= kMaxLdsBytes && C <= kMaxChannels && C % 32 == 0 && p.R <= kMaxRegions;
}

hipError_t prepare_attend(const Params& p, bool bf16) {
    if (p.lds_bytes <= kDefaultLdsBytes) return hipSuccess;
    auto raise = [](const void* f) {
        return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
    };
#define BRA_ATTEND_PREP(T, HS, WS, NW, HEADS, KTOP)                                             \
    if (p.kv_ratio == 1 && matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, true)) {     \
        hipError_t e = raise(reinterpret_cast<const void*>(                                     \
            &attend_kernel<T, HS, WS, NW, HEADS, KTOP, false>));                                \
        if (e != hipSuccess || !route_fused(NW * NW, HEADS)) return e;                          \
        return raise(reinterpret_cast<const void*>(                                             \
            &attend_kernel<T, HS, WS, NW, HEADS, KTOP, route_fused(NW * NW, HEADS)>));          \
    }
    BRA_FOR_EACH_SHAPE(BRA_ATTEND_PREP)
#undef BRA_ATTEND_PREP
    hipError_t e;
    if (bf16) {
        e = raise(reinterpret_cast<const void*>(&attend_kernel<uint16_t, 0, 0, 0, 0, 0, false>));
        if (e == hipSuccess)
            e = raise(reinterpret_cast<const void*>(&attend_kernel<uint16_t, 0, 0, 0, 0, 0, true>));
    } else {
        e = raise(reinterpret_cast<const void*>(&attend_kernel<float, 0, 0, 0, 0, 0, false>));
        if (e == hipSuccess)
            e = raise(reinterpret_cast<const void*>(&attend_kernel<float, 0, 0, 0, 0, 0, true>));
    }
    return e;
}

hipError_t launch_attend(const Params& p, bool bf16, const void* q, const void* v,
                         const void* kg, const void* vg, const double* means, int32_t* routing,
                         bool use_routing, const float* lepe_w, const float* lepe_b,
                         const uint2* lepe_table, const float* zero_bias, const void* w_o,
                         const float* b_o, void* out, hipStream_t stream) {
    Params pp = p;
    pp.has_lepe = lepe_w != nullptr;
    pp.out_proj = bf16 && w_o != nullptr;
    if (!pp.has_lepe) lepe_b = nullptr;
    // the MFMA LePE loads its bias unconditionally: a zero vector stands in
    const float* lepe_bias = lepe_b ? lepe_b : zero_bias;
    const dim3 grid(p.B * p.R), block(kThreads);
    const bool fused = !use_routing && route_in_attend(p);
    const uint16_t* wo = static_cast<const uint16_t*>(w_o);
#define BRA_ATTEND_F(T, HS, WS, NW, HEADS, KTOP, F)                                             \
    hipLaunchKernelGGL((attend_kernel<T, HS, WS, NW, HEADS, KTOP, F>), grid, block,             \
                       p.lds_bytes, stream, static_cast<const T*>(q), static_cast<const T*>(v), \
                       static_cast<const T*>(kg), static_cast<const T*>(vg), means, routing,   \
                       lepe_w, lepe_b, lepe_bias, lepe_table, wo, b_o, static_cast<T*>(out), pp)
#define BRA_ATTEND(T, HS, WS, NW, HEADS, KTOP)                                                  \
    if (p.kv_ratio == 1 && matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, true)) {     \
        if constexpr (route_fused(NW * NW, HEADS)) {                                            \
            if (fused)                                                                          \
                BRA_ATTEND_F(T, HS, WS, NW, HEADS, KTOP, true);                                 \
            else                                                                                \
                BRA_ATTEND_F(T, HS, WS, NW, HEADS, KTOP, false);                                \
        } else {                                                                                \
            BRA_ATTEND_F(T, HS, WS, NW, HEADS, KTOP, false);                                    \
        }                                                                                       \
        return hipGetLastError();                                                               \
    }
    BRA_FOR_EACH_SHAPE(BRA_ATTEND)
#undef BRA_ATTEND
#undef BRA_ATTEND_F
#define BRA_GENERIC(T, F)                                                                       \
    hipLaunchKernelGGL((attend_kernel<T, 0, 0, 0, 0, 0, F>), grid, block, p.lds_bytes, stream,  \
                       static_cast<const T*>(q), static_cast<const T*>(v),                      \
                       static_cast<const T*>(kg), static_cast<const T*>(vg), means, routing,    \
                       lepe_w, lepe_b, lepe_bias, lepe_table, wo, b_o, static_cast<T*>(out), pp)
    if (bf16) {
        if (fused)
            BRA_GENERIC(uint16_t, true);
        else
            BRA_GENERIC(uint16_t, false);
    } else {
        if (fused)
            BRA_GENERIC(float, true);
        else
            BRA_GENERIC(float, false);
    }
#undef BRA_GENERIC
    return hipGetLastError();
}

}  // namespace bra
