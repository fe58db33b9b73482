// bra_image.h -- interface of the whole-image kernel (bra_image.hip): one
// workgroup per (image, head group) computes the region means, the routing,
// the token attention and LePE of that group over the whole map, with K and
// V of the group resident in LDS.  Not installed; the public ABI is
// include/bra.h.
#pragma once

#include "bra_launch.h"

namespace bra {

constexpr int kImgWaves = 16;  // waves of an image workgroup (1024 threads)

// LDS layout of an image workgroup (byte offsets; every region 16-byte
// aligned).  The region means and, once the routing is done, the waves'
// output tiles share one overlay.  Strides are padded so that the rows the
// lanes of one LDS instruction touch fall on different banks: a map row of
// K carries 16 bytes of padding, a Q-mean row 2 doubles, a K-mean block 4.
struct ImgGeo {
    int ts;       // 4 x 4 token tiles per map side
    int pw;       // row pitch of a V plane (elements): 4 ts columns + a 2-cell border each side
    int ps;       // V plane stride (elements)
    int rs;       // K (and staged Q) map row stride (elements): W * CG + 8
    int qs;       // stride (doubles) of one region-mean row
    int off_k, off_over, means_bytes, off_vp, off_tab, off_bias, off_offk, off_offv, off_regk,
        off_regv, off_misc, lds;
};

constexpr int img_align16(int x) { return (x + 15) & ~15; }
constexpr int img_max(int a, int b) { return a > b ? a : b; }

// HS: window side (2 or 4), NW: regions per side, HG: heads per workgroup.
constexpr ImgGeo img_geo(int HS, int NW, int HG, int HEADS, int KTOP) {
    ImgGeo g{};
    const int H = NW * HS, R = NW * NW, CG = HG * kHeadDim;
    (void)HEADS;
    g.ts = (H + 3) / 4;
    g.pw = 4 * g.ts + 4;
    g.ps = H * g.pw + 4;
    g.rs = H * CG + 8;
    g.qs = kHeadDim + 2;
    int off = 0;
    g.off_k = off;
    off = img_align16(off + H * g.rs * 2);
    g.off_over = off;
    // K means then Q means, [HG][R][qs] fp64 each
    g.means_bytes = 2 * HG * R * g.qs * 8;
    const int stage = kImgWaves * 16 * 36 * 4;
    off = img_align16(off + img_max(g.means_bytes, stage));
    // the V planes; before them (up to the means) the staged Q, H rows of rs
    g.off_vp = off;
    off = img_align16(off + img_max(CG * g.ps * 2, H * g.rs * 2));
    g.off_tab = off;
    off = img_align16(off + CG * 40 * 8);
    g.off_bias = off;
    off = img_align16(off + CG * 4);
    g.off_offk = off;
    off = img_align16(off + HG * R * KTOP * 4);
    g.off_offv = off;
    off = img_align16(off + HG * R * KTOP * 4);
    g.off_regk = off;
    off = img_align16(off + R * 4);
    g.off_regv = off;
    off = img_align16(off + R * 4);
    // 16 zero bytes (the LePE rows outside the map), the max |K mean| per
    // head, the count and list of rows to route exactly
    g.off_misc = off;
    off = img_align16(off + 16 + 4 * HG + 4 + 4 * HG * R);
    g.lds = off;
    return g;
}

// The image kernel takes the forward when one of its compiled geometries
// matches (bf16, per-head routing, no KV downsampling).
bool image_applies(const Params& p, bool bf16);
int image_lds_bytes(const Params& p);
// Raises the kernel's dynamic LDS limit to what it uses (once per handle).
hipError_t prepare_image(const Params& p);
// routed: read the routing from `routing` (the caller's) instead of routing.
hipError_t launch_image(const Params& p, const void* q, const void* k, const void* v,
                        const float* lepe_w, const float* lepe_b, int32_t* routing, bool routed,
                        void* out, hipStream_t stream);

}  // namespace bra
