// bra_api.cpp -- the C ABI of libbra.so (declared in include/bra.h): argument
// validation, handle registry, workspace, launches on the caller's stream and
// optional per-kernel event timing.  No compute happens on the host.
#include "bra.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <vector>

#include "bra_launch.h"

struct bra_handle_s {
    bra_config_t cfg;
    bra::Params params;
    bool bf16;
    int device;
    double* means;       // workspace: fp64 region means of Q [B, heads, R, 32], then of
                         // K [B, heads, 16, R, 2], then K in fp32 (same order); the routing
                         // [B, heads, R, k] int32; the MFMA LePE operand table; C zero floats
                         // (the bias when none is given)
    size_t means_bytes;
    int32_t* routing;
    uint2* lepe_table;
    float* zero_bias;
    void* kd;  // downsampled K and V [B, H/r, W/r, C] (KV downsampling), else NULL
    void* vd;
    void* qs;  // projected q, k, v [B, H, W, C] (handles created with projections), else NULL
    void* ks;
    void* vs;
    void* ys;  // attention output before the output projection, when that runs as its own
               // kernel (projections on shapes with small regions), else NULL
    // per-kernel timing (events recorded by bra_forward while slots remain)
    std::vector<hipEvent_t> events;  // kEventsPerCall per recorded call
    int timing_capacity;
    int timing_used;
};

namespace {

constexpr int kEventsPerCall = 4;  // before pool, route, attend; after attend

std::mutex g_mutex;
std::set<bra_handle_t> g_live;  // handles between create and destroy
thread_local std::string g_last_error;

bra_status_t fail(bra_status_t s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

bra_status_t fail_hip(hipError_t e, const char* what) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return e == hipErrorOutOfMemory ? BRA_ERR_NOMEM : BRA_ERR_HIP;
}

bool is_live(bra_handle_t h) {
    std::lock_guard<std::mutex> lock(g_mutex);
    return h != nullptr && g_live.count(h) != 0;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, const void* b, size_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + n && y < x + n;
}

void release_events(bra_handle_t h) {
    for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
    h->events.clear();
    h->timing_capacity = 0;
    h->timing_used = 0;
}

}  // namespace

extern "C" {

const char* bra_status_string(bra_status_t s) {
    switch (s) {
        case BRA_OK: return "ok";
        case BRA_ERR_NULL: return "a required pointer is NULL";
        case BRA_ERR_SHAPE: return "invalid shape";
        case BRA_ERR_UNSUPPORTED: return "unsupported configuration";
        case BRA_ERR_HIP: return "HIP runtime error";
        case BRA_ERR_NOMEM: return "out of device memory";
        case BRA_ERR_BAD_HANDLE: return "not a live handle";
        case BRA_ERR_ALIGN: return "misaligned pointer";
        case BRA_ERR_ALIAS: return "output overlaps an input";
        case BRA_ERR_DEVICE: return "current device is not the handle's device";
    }
    return "unknown status";
}

const char* bra_last_error(void) { return g_last_error.c_str(); }

bra_status_t bra_create(const bra_config_t* cfg, bra_handle_t* out) {
    if (!cfg || !out) return fail(BRA_ERR_NULL, "bra_create: cfg and out are required");
    *out = nullptr;
    const bra_config_t c = *cfg;
    if (c.batch <= 0 || c.height <= 0 || c.width <= 0 || c.channels <= 0 || c.num_heads <= 0 ||
        c.n_win <= 0)
        return fail(BRA_ERR_SHAPE, "bra_create: sizes must be positive");
    if (c.height % c.n_win || c.width % c.n_win)
        return fail(BRA_ERR_SHAPE, "bra_create: height and width must be divisible by n_win");
    if (c.channels % c.num_heads)
        return fail(BRA_ERR_SHAPE, "bra_create: channels must be divisible by num_heads");
    const double elems = static_cast<double>(c.height) * c.width * c.channels;
    if (elems >= 2147483647.0 || static_cast<double>(c.batch) * c.n_win * c.n_win >= 2147483647.0)
        return fail(BRA_ERR_SHAPE, "bra_create: one image or the region grid exceeds int32 indexing");
    if (c.channels / c.num_heads != bra::kHeadDim)
        return fail(BRA_ERR_UNSUPPORTED, "bra_create: head_dim must be 32");
    if (static_cast<double>(c.height) * c.width >= 8388608.0)  // 2^23: 24-bit token indexing
        return fail(BRA_ERR_UNSUPPORTED, "bra_create: height * width must be below 2^23");
    if (c.dtype != BRA_F32 && c.dtype != BRA_BF16)
        return fail(BRA_ERR_UNSUPPORTED, "bra_create: dtype must be BRA_F32 or BRA_BF16");
    const int R = c.n_win * c.n_win;
    const int k = (c.topk <= 0 || c.topk > R) ? R : c.topk;
    const float scale = c.scale > 0.f ? c.scale : 1.0f / std::sqrt(static_cast<float>(bra::kHeadDim));
    const bool bf16 = c.dtype == BRA_BF16;
    bra::Params p;
    if (c.shared_routing != 0 && c.shared_routing != 1)
        return fail(BRA_ERR_SHAPE, "bra_create: shared_routing must be 0 or 1");
    if (c.projections != 0 && c.projections != 1)
        return fail(BRA_ERR_SHAPE, "bra_create: projections must be 0 or 1");
    if (c.projections && !bf16)
        return fail(BRA_ERR_UNSUPPORTED, "bra_create: projections need dtype BRA_BF16");
    if (c.projections && c.channels > 512)
        return fail(BRA_ERR_UNSUPPORTED, "bra_create: projections need channels <= 512");
    const int kv_ratio = c.kv_downsample_ratio <= 1 ? 1 : c.kv_downsample_ratio;
    if (c.projections && (c.shared_routing == 1 || kv_ratio > 1))
        return fail(BRA_ERR_UNSUPPORTED,
                    "bra_create: projections combine with neither shared_routing nor KV downsampling");
    if ((c.height / c.n_win) % kv_ratio || (c.width / c.n_win) % kv_ratio)
        return fail(BRA_ERR_SHAPE,
                    "bra_create: kv_downsample_ratio must divide the window height and width");
    if (!bra::plan(p, c.batch, c.height, c.width, c.channels, c.num_heads, c.n_win, k, scale,
                   bf16, c.shared_routing == 1, kv_ratio))
        return fail(BRA_ERR_UNSUPPORTED,
                    "bra_create: a region (with its LePE halo) or the channel count is too large "
                    "for the on-chip tiles (" + std::to_string(p.lds_bytes) + " bytes of LDS)");

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "bra_create: hipGetDevice");
    bra_handle_t h = new (std::nothrow) bra_handle_s();
    if (!h) return fail(BRA_ERR_NOMEM, "bra_create: host allocation failed");
    h->cfg = c;
    h->params = p;
    h->bf16 = bf16;
    h->device = dev;
    // fp64 Q and K means, then the K means in fp32
    const size_t mean_bytes = static_cast<size_t>(c.batch) * c.channels * R *
                              (2 * sizeof(double) + sizeof(float));
    const size_t route_bytes =
        ((static_cast<size_t>(c.batch) * p.rheads * R * k * sizeof(int32_t)) + 15) & ~size_t{15};
    const size_t table_bytes = static_cast<size_t>(p.table_items) * sizeof(uint2);
    const size_t zero_bytes = ((static_cast<size_t>(c.channels) * sizeof(float)) + 15) &
                              ~size_t{15};
    // downsampled K and V (KV downsampling only)
    const size_t kv_bytes = p.kv_ratio > 1 ? static_cast<size_t>(c.batch) * p.kH * p.kW *
                                                 c.channels * (bf16 ? 2 : 4)
                                           : 0;
    // projected q, k, v (projections only)
    const size_t map_bytes = static_cast<size_t>(c.batch) * c.height * c.width * c.channels *
                             (bf16 ? 2 : 4);
    const bool proj_after = c.projections && !bra::out_proj_in_attend(p.t, c.channels);
    const size_t proj_bytes = c.projections ? (proj_after ? 4 : 3) * map_bytes : 0;
    h->means_bytes = mean_bytes + route_bytes + table_bytes + zero_bytes + 2 * kv_bytes +
                     proj_bytes;
    h->means = nullptr;
    h->routing = nullptr;
    h->lepe_table = nullptr;
    h->zero_bias = nullptr;
    h->kd = nullptr;
    h->vd = nullptr;
    h->qs = h->ks = h->vs = h->ys = nullptr;
    h->timing_capacity = 0;
    h->timing_used = 0;
    e = hipMalloc(reinterpret_cast<void**>(&h->means), h->means_bytes);
    if (e != hipSuccess) {
        delete h;
        return fail_hip(e, "bra_create: hipMalloc of the workspace");
    }
    h->routing = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(h->means) + mean_bytes);
    h->lepe_table =
        reinterpret_cast<uint2*>(reinterpret_cast<char*>(h->means) + mean_bytes + route_bytes);
    h->zero_bias = reinterpret_cast<float*>(reinterpret_cast<char*>(h->means) + mean_bytes +
                                            route_bytes + table_bytes);
    h->kd = kv_bytes ? reinterpret_cast<char*>(h->zero_bias) + zero_bytes : nullptr;
    h->vd = kv_bytes ? static_cast<char*>(h->kd) + kv_bytes : nullptr;
    if (proj_bytes) {
        h->qs = reinterpret_cast<char*>(h->zero_bias) + zero_bytes + 2 * kv_bytes;
        h->ks = static_cast<char*>(h->qs) + map_bytes;
        h->vs = static_cast<char*>(h->ks) + map_bytes;
        if (proj_after) h->ys = static_cast<char*>(h->vs) + map_bytes;
    }
    e = hipMemset(h->zero_bias, 0, zero_bytes);
    if (e != hipSuccess) {
        (void)hipFree(h->means);
        delete h;
        return fail_hip(e, "bra_create: hipMemset of the zero bias");
    }
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        g_live.insert(h);
    }
    *out = h;
    return BRA_OK;
}

bra_status_t bra_destroy(bra_handle_t h) {
    if (!h) return BRA_OK;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (!g_live.erase(h)) return fail(BRA_ERR_BAD_HANDLE, "bra_destroy: not a live handle");
    }
    release_events(h);
    hipError_t e = hipFree(h->means);
    delete h;
    if (e != hipSuccess) return fail_hip(e, "bra_destroy: hipFree");
    return BRA_OK;
}

int32_t bra_topk_effective(bra_handle_t h) {
    if (!is_live(h)) return -1;
    return h->params.k;
}

// The argument checks shared by both forward entry points (`what` names the
// caller in messages).
static bra_status_t check_forward_args(bra_handle_t h, const char* what, const void* q,
                                       const void* k, const void* v, const float* lepe_w,
                                       const float* lepe_b, const void* out,
                                       const int32_t* routing_idx) {
    const std::string w(what);
    if (!is_live(h)) return fail(BRA_ERR_BAD_HANDLE, w + ": not a live handle");
    if (!q || !k || !v || !out) return fail(BRA_ERR_NULL, w + ": q, k, v and out are required");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(BRA_ERR_ALIGN, w + ": q, k, v and out must be 16-byte aligned");
    if (!aligned(lepe_w, 4) || !aligned(lepe_b, 4) || !aligned(routing_idx, 4))
        return fail(BRA_ERR_ALIGN, w + ": lepe_w, lepe_b and routing_idx must be 4-byte aligned");
    const bra_config_t& c = h->cfg;
    const size_t bytes = static_cast<size_t>(c.batch) * c.height * c.width * c.channels *
                         (h->bf16 ? 2 : 4);
    if (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes))
        return fail(BRA_ERR_ALIAS, w + ": out must not overlap q, k or v");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, (w + ": hipGetDevice").c_str());
    if (dev != h->device) return fail(BRA_ERR_DEVICE, w + ": wrong current device");
    return BRA_OK;
}

// The forward steps on stream s.  With x (projections), the qkv projection
// writes the handle's q, k, v (and the region means), and the attention
// kernel applies the output projection w_o, b_o; otherwise the pool kernel
// reads the caller's q and k.
static bra_status_t enqueue_forward(bra_handle_t h, const char* what, const void* x,
                                    const void* w_qkv, const float* b_qkv, const void* q,
                                    const void* k, const void* v, const float* lepe_w,
                                    const float* lepe_b, const void* w_o, const float* b_o,
                                    void* out, int32_t* routing_idx, hipStream_t s) {
    const std::string wh(what);
    hipError_t e;
    const bool timed = h->timing_used < h->timing_capacity;
    hipEvent_t* ev = timed ? &h->events[kEventsPerCall * h->timing_used] : nullptr;
    if (timed && (e = hipEventRecord(ev[0], s)) != hipSuccess)
        return fail_hip(e, (wh + ": hipEventRecord").c_str());
    // the routing goes to the caller's buffer when one is given
    int32_t* routing = routing_idx ? routing_idx : h->routing;
    const bra::Params& P = h->params;
    // small region grids with many heads: means and routing in one kernel
    const bool pool_route =
        !x && bra::route_in_pool(h->bf16, P.shared != 0, P.R, P.heads, P.t);
    if (x) {
        e = bra::launch_proj_qkv(h->params, x, w_qkv, b_qkv, h->qs, h->ks, h->vs, h->means,
                                 lepe_w, h->lepe_table, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": qkv projection launch").c_str());
        q = h->qs;
        k = h->ks;
        v = h->vs;
    } else if (pool_route) {
        e = bra::launch_pool_route(h->params, q, k, lepe_w, h->lepe_table, routing, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": region-pool and routing launch").c_str());
    } else {
        e = bra::launch_pool_qk(h->params, h->bf16, q, k, lepe_w, h->means, h->lepe_table, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": region-pool launch").c_str());
    }
    if (h->kd) {
        e = bra::launch_kv_pool(h->params, h->bf16, k, v, h->kd, h->vd, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": K/V downsampling launch").c_str());
    }
    if (timed && (e = hipEventRecord(ev[1], s)) != hipSuccess)
        return fail_hip(e, (wh + ": hipEventRecord").c_str());
    // small region grids are routed inside the attention kernel
    if (!bra::route_in_attend(h->params) && !pool_route) {
        e = bra::launch_route(h->params, h->bf16, h->means, routing, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": routing launch").c_str());
    }
    if (timed && (e = hipEventRecord(ev[2], s)) != hipSuccess)
        return fail_hip(e, (wh + ": hipEventRecord").c_str());
    // the output projection: in the attention kernel's epilogue, or over y
    // in a kernel of its own (h->ys is set for the shapes that take that)
    const bool proj_after = w_o && h->ys;
    e = bra::launch_attend(h->params, h->bf16, q, v, h->kd ? h->kd : k, h->vd ? h->vd : v,
                           h->means, routing, !bra::route_in_attend(h->params), lepe_w, lepe_b,
                           h->lepe_table, h->zero_bias, proj_after ? nullptr : w_o, b_o,
                           proj_after ? h->ys : out, s);
    if (e != hipSuccess) return fail_hip(e, (wh + ": attention launch").c_str());
    if (proj_after) {
        e = bra::launch_proj_out(h->params, h->ys, w_o, b_o, out, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": output projection launch").c_str());
    }
    if (timed) {
        if ((e = hipEventRecord(ev[3], s)) != hipSuccess)
            return fail_hip(e, (wh + ": hipEventRecord").c_str());
        ++h->timing_used;
    }
    return BRA_OK;
}

bra_status_t bra_forward(bra_handle_t h, const void* q, const void* k, const void* v,
                         const float* lepe_w, const float* lepe_b, void* out,
                         int32_t* routing_idx, void* stream) {
    bra_status_t st = check_forward_args(h, "bra_forward", q, k, v, lepe_w, lepe_b, out,
                                         routing_idx);
    if (st != BRA_OK) return st;
    return enqueue_forward(h, "bra_forward", nullptr, nullptr, nullptr, q, k, v, lepe_w, lepe_b,
                           nullptr, nullptr, out, routing_idx, static_cast<hipStream_t>(stream));
}

bra_status_t bra_forward_proj(bra_handle_t h, const void* x, const void* w_qkv,
                              const float* b_qkv, const float* lepe_w, const float* lepe_b,
                              const void* w_o, const float* b_o, void* out,
                              int32_t* routing_idx, void* stream) {
    bra_status_t st = check_forward_args(h, "bra_forward_proj", x, x, x, lepe_w, lepe_b, out,
                                         routing_idx);
    if (st != BRA_OK) return st;
    if (!h->qs)
        return fail(BRA_ERR_UNSUPPORTED,
                    "bra_forward_proj: the handle was created without projections");
    if (!w_qkv || !w_o) return fail(BRA_ERR_NULL, "bra_forward_proj: w_qkv and w_o are required");
    if (!aligned(w_qkv, 16) || !aligned(w_o, 16) || !aligned(b_qkv, 4) || !aligned(b_o, 4))
        return fail(BRA_ERR_ALIGN,
                    "bra_forward_proj: w_qkv and w_o must be 16-byte aligned, the biases 4-byte");
    return enqueue_forward(h, "bra_forward_proj", x, w_qkv, b_qkv, nullptr, nullptr, nullptr,
                           lepe_w, lepe_b, w_o, b_o, out, routing_idx,
                           static_cast<hipStream_t>(stream));
}

bra_status_t bra_forward_routed(bra_handle_t h, const void* q, const void* k, const void* v,
                                const float* lepe_w, const float* lepe_b,
                                const int32_t* routing_idx, void* out, void* stream) {
    if (!routing_idx && is_live(h))
        return fail(BRA_ERR_NULL, "bra_forward_routed: routing_idx is required");
    bra_status_t st = check_forward_args(h, "bra_forward_routed", q, k, v, lepe_w, lepe_b, out,
                                         routing_idx);
    if (st != BRA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    // the MFMA LePE operand table is the region-pool kernel's side product:
    // build it alone (no means) when this shape uses it
    if (lepe_w && h->params.table_items > 0) {
        e = bra::launch_lepe_table(h->params, lepe_w, h->lepe_table, s);
        if (e != hipSuccess) return fail_hip(e, "bra_forward_routed: LePE table launch");
    }
    if (h->kd) {
        e = bra::launch_kv_pool(h->params, h->bf16, k, v, h->kd, h->vd, s);
        if (e != hipSuccess) return fail_hip(e, "bra_forward_routed: K/V downsampling launch");
    }
    e = bra::launch_attend(h->params, h->bf16, q, v, h->kd ? h->kd : k, h->vd ? h->vd : v,
                           h->means, const_cast<int32_t*>(routing_idx), true, lepe_w, lepe_b,
                           h->lepe_table, h->zero_bias, nullptr, nullptr, out, s);
    if (e != hipSuccess) return fail_hip(e, "bra_forward_routed: attention launch");
    return BRA_OK;
}

bra_status_t bra_timing_enable(bra_handle_t h, int32_t n) {
    if (!is_live(h)) return fail(BRA_ERR_BAD_HANDLE, "bra_timing_enable: not a live handle");
    if (n < 0) return fail(BRA_ERR_SHAPE, "bra_timing_enable: n must be >= 0");
    release_events(h);
    h->events.resize(static_cast<size_t>(kEventsPerCall) * n);
    for (size_t i = 0; i < h->events.size(); ++i) {
        hipError_t e = hipEventCreate(&h->events[i]);
        if (e != hipSuccess) {
            h->events.resize(i);
            release_events(h);
            return fail_hip(e, "bra_timing_enable: hipEventCreate");
        }
    }
    h->timing_capacity = n;
    h->timing_used = 0;
    return BRA_OK;
}

bra_status_t bra_timing_read(bra_handle_t h, float* ms, int32_t* count) {
    if (!is_live(h)) return fail(BRA_ERR_BAD_HANDLE, "bra_timing_read: not a live handle");
    if (!ms || !count) return fail(BRA_ERR_NULL, "bra_timing_read: ms and count are required");
    *count = 0;
    for (int i = 0; i < h->timing_used; ++i) {
        hipEvent_t* ev = &h->events[kEventsPerCall * i];
        hipError_t e = hipEventSynchronize(ev[kEventsPerCall - 1]);
        if (e != hipSuccess) return fail_hip(e, "bra_timing_read: hipEventSynchronize");
        for (int j = 0; j < kEventsPerCall - 1; ++j) {
            float x = 0.f;
            if ((e = hipEventElapsedTime(&x, ev[j], ev[j + 1])) != hipSuccess)
                return fail_hip(e, "bra_timing_read: hipEventElapsedTime");
            ms[(kEventsPerCall - 1) * i + j] = x;
        }
    }
    *count = h->timing_used;
    h->timing_used = 0;
    return BRA_OK;
}

}  // extern "C"
