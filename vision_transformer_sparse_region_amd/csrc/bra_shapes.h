// bra_shapes.h -- the window geometries compiled as dedicated kernel
// instances, and the host-side matching of a Params against them.
#pragma once

#include "bra_launch.h"

namespace bra {

// Shapes with a compiled instance whose geometry is folded at compile time;
// every other shape runs the generic instance.  X(T, HS, WS, NW, HEADS, KTOP):
// BiFormer-S stages 1-3 (7x7 regions of 8x8, 4x4 and 2x2 tokens), the
// 512x512 segmentation map at stride 4 (16x16 regions of 8x8 tokens), and
// the small fp32 map (7x7 regions of 4x4 tokens).
#define BRA_FOR_EACH_SHAPE(X)    \
    X(uint16_t, 8, 8, 7, 2, 1)   \
    X(uint16_t, 4, 4, 7, 4, 4)   \
    X(uint16_t, 2, 2, 7, 8, 16)  \
    X(uint16_t, 8, 8, 16, 2, 16) \
    X(float, 4, 4, 7, 2, 4)

struct GeoKey {
    bool bf16;
    int hs, ws, n, heads, k;
};

template <typename T, int HS, int WS, int NW, int HEADS, int KTOP>
struct Inst {
    static constexpr GeoKey key{sizeof(T) == 2, HS, WS, NW, HEADS, KTOP};
};

inline bool matches(const GeoKey& g, const Params& p, bool bf16, bool with_k) {
    return g.bf16 == bf16 && g.hs == p.hs && g.ws == p.ws && g.n == p.n && g.heads == p.heads &&
           (!with_k || g.k == p.k);
}

inline bool is_fixed_shape(const Params& p, bool bf16) {
    bool found = false;
#define BRA_IS_FIXED(T, HS, WS, NW, HEADS, KTOP) \
    found = found || matches(Inst<T, HS, WS, NW, HEADS, KTOP>::key, p, bf16, true);
    BRA_FOR_EACH_SHAPE(BRA_IS_FIXED)
#undef BRA_IS_FIXED
    return found;
}

}  // namespace bra
