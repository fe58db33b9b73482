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

#include "bra_image.h"
#include "bra_small.h"
#include "bra_launch.h"

// Device workspace of the forward: the region means (fp64 Q means
// [B, heads, R, 32], fp64 K means [B, heads, 16, R, 2], the K means again in
// fp32), the routing [B, rheads, R, k] int32 for calls that pass no
// routing_idx, the MFMA LePE operand table, C zero floats (the bias when none
// is given), the K/V downsampled by kv_downsample_ratio, and the projected
// q, k, v (and y) of the projected path.
struct bra_workspace {
    double* means;
    int32_t* routing;
    uint2* lepe_table;
    float* zero_bias;
    void* kd;  // downsampled K and V [B, H/r, W/r, C] (KV downsampling), else NULL
    void* vd;
    void* qs;  // projected q, k, v [B, H, W, C] (projections), else NULL
    void* ks;
    void* vs;
    void* ys;  // attention output before the output projection, when that runs as its own
               // kernel (projections on shapes with small regions), else NULL
    size_t zero_bytes;
};

struct bra_handle_s {
    bra_config_t cfg;
    bra::Params params;
    bool bf16;
    int device;
    void* base;          // the one device allocation holding the workspace
    size_t bytes;
    bra_workspace ws;
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
// Allocation-failure injection (bra_debug_inject_alloc_failure): the next
// g_fail_host handle allocations and the next g_fail_device workspace
// allocations of bra_create fail as if out of memory.
int g_fail_host = 0;
int g_fail_device = 0;

bool take_injected(int& counter) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (counter <= 0) return false;
    --counter;
    return true;
}

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

// Checks cfg; on success fills p and bf16 (the planned kernel geometry).
bra_status_t validate_config(const bra_config_t* cfg, const char* what, bra::Params& p,
                             bool& bf16) {
    const std::string w(what);
    if (!cfg) return fail(BRA_ERR_NULL, w + ": cfg is required");
    const bra_config_t c = *cfg;
    if (c.batch <= 0 || c.height <= 0 || c.width <= 0 || c.channels <= 0 || c.num_heads <= 0 ||
        c.n_win <= 0)
        return fail(BRA_ERR_SHAPE, w + ": sizes must be positive");
    if (c.height % c.n_win || c.width % c.n_win)
        return fail(BRA_ERR_SHAPE, w + ": height and width must be divisible by n_win");
    if (c.channels % c.num_heads)
        return fail(BRA_ERR_SHAPE, w + ": channels must be divisible by num_heads");
    const double elems = static_cast<double>(c.height) * c.width * c.channels;
    if (elems >= 2147483647.0 || static_cast<double>(c.batch) * c.n_win * c.n_win >= 2147483647.0)
        return fail(BRA_ERR_SHAPE, w + ": one image or the region grid exceeds int32 indexing");
    if (c.channels / c.num_heads != bra::kHeadDim)
        return fail(BRA_ERR_UNSUPPORTED, w + ": head_dim must be 32");
    if (static_cast<double>(c.height) * c.width >= 8388608.0)  // 2^23: 24-bit token indexing
        return fail(BRA_ERR_UNSUPPORTED, w + ": height * width must be below 2^23");
    if (c.dtype != BRA_F32 && c.dtype != BRA_BF16)
        return fail(BRA_ERR_UNSUPPORTED, w + ": dtype must be BRA_F32 or BRA_BF16");
    const int R = c.n_win * c.n_win;
    const int k = (c.topk <= 0 || c.topk > R) ? R : c.topk;
    const float scale =
        c.scale > 0.f ? c.scale : 1.0f / std::sqrt(static_cast<float>(bra::kHeadDim));
    bf16 = c.dtype == BRA_BF16;
    if (c.shared_routing != 0 && c.shared_routing != 1)
        return fail(BRA_ERR_SHAPE, w + ": shared_routing must be 0 or 1");
    if (c.projections != 0 && c.projections != 1)
        return fail(BRA_ERR_SHAPE, w + ": projections must be 0 or 1");
    if (c.projections && !bf16)
        return fail(BRA_ERR_UNSUPPORTED, w + ": projections need dtype BRA_BF16");
    if (c.projections && c.channels > 512)
        return fail(BRA_ERR_UNSUPPORTED, w + ": projections need channels <= 512");
    const int kv_ratio = c.kv_downsample_ratio <= 1 ? 1 : c.kv_downsample_ratio;
    if (c.projections && (c.shared_routing == 1 || kv_ratio > 1))
        return fail(BRA_ERR_UNSUPPORTED,
                    w + ": projections combine with neither shared_routing nor KV downsampling");
    if ((c.height / c.n_win) % kv_ratio || (c.width / c.n_win) % kv_ratio)
        return fail(BRA_ERR_SHAPE,
                    w + ": kv_downsample_ratio must divide the window height and width");
    if (!bra::plan(p, c.batch, c.height, c.width, c.channels, c.num_heads, c.n_win, k, scale,
                   bf16, c.shared_routing == 1, kv_ratio))
        return fail(BRA_ERR_UNSUPPORTED,
                    w + ": a region (with its LePE halo) or the channel count is too large "
                        "for the on-chip tiles (" + std::to_string(p.lds_bytes) + " bytes of LDS)");
    return BRA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t{255}; }

// The workspace of a forward with config c: returns its size in bytes and,
// when base is given, carves ws out of base.
size_t workspace_layout(const bra_config_t& c, const bra::Params& p, bool bf16, char* base,
                        bra_workspace* ws) {
    const size_t R = static_cast<size_t>(p.R);
    // fp64 Q and K means, then the K means in fp32 (none where the image
    // kernel computes them on chip, unless the qkv projection writes them)
    const bool on_chip = bra::image_applies(p, bf16) && !c.projections;
    const size_t mean_bytes =
        on_chip ? 0
                : align256(static_cast<size_t>(c.batch) * c.channels * R *
                           (2 * sizeof(double) + sizeof(float)));
    const size_t route_bytes =
        align256(static_cast<size_t>(c.batch) * p.rheads * R * p.k * sizeof(int32_t));
    const size_t table_bytes = align256(static_cast<size_t>(p.table_items) * sizeof(uint2));
    const size_t zero_bytes = align256(static_cast<size_t>(c.channels) * sizeof(float));
    // downsampled K and V (KV downsampling only)
    const size_t kv_bytes =
        p.kv_ratio > 1
            ? align256(static_cast<size_t>(c.batch) * p.kH * p.kW * c.channels * (bf16 ? 2 : 4))
            : 0;
    // projected q, k, v (projections only)
    const size_t map_bytes = align256(static_cast<size_t>(c.batch) * c.height * c.width *
                                      c.channels * (bf16 ? 2 : 4));
    const bool proj_after = c.projections && !bra::out_proj_in_attend(p.t, c.channels);
    const size_t proj_bytes = c.projections ? (proj_after ? 4 : 3) * map_bytes : 0;
    const size_t total =
        mean_bytes + route_bytes + table_bytes + zero_bytes + 2 * kv_bytes + proj_bytes;
    if (base && ws) {
        char* at = base;
        ws->means = reinterpret_cast<double*>(at);
        at += mean_bytes;
        ws->routing = reinterpret_cast<int32_t*>(at);
        at += route_bytes;
        ws->lepe_table = reinterpret_cast<uint2*>(at);
        at += table_bytes;
        ws->zero_bias = reinterpret_cast<float*>(at);
        ws->zero_bytes = zero_bytes;
        at += zero_bytes;
        ws->kd = kv_bytes ? at : nullptr;
        ws->vd = kv_bytes ? at + kv_bytes : nullptr;
        at += 2 * kv_bytes;
        ws->qs = ws->ks = ws->vs = ws->ys = nullptr;
        if (proj_bytes) {
            ws->qs = at;
            ws->ks = at + map_bytes;
            ws->vs = at + 2 * map_bytes;
            if (proj_after) ws->ys = at + 3 * map_bytes;
        }
    }
    return total;
}

}  // namespace

extern "C" {

const char* bra_status_string(int32_t s) {
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
    bra::Params p;
    bool bf16 = false;
    bra_status_t st = validate_config(cfg, "bra_create", p, bf16);
    if (st != BRA_OK) return st;
    bra_handle_t h = take_injected(g_fail_host) ? nullptr : new (std::nothrow) bra_handle_s();
    if (!h) return fail(BRA_ERR_NOMEM, "bra_create: host allocation failed");
    h->cfg = *cfg;
    h->params = p;
    h->bf16 = bf16;
    h->timing_capacity = 0;
    h->timing_used = 0;
    h->bytes = workspace_layout(*cfg, p, bf16, nullptr, nullptr);
    h->base = nullptr;
    if (take_injected(g_fail_device)) {
        delete h;
        return fail(BRA_ERR_NOMEM, "bra_create: hipMalloc of the workspace: out of memory "
                                   "(injected)");
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        delete h;
        return fail_hip(e, "bra_create: hipGetDevice");
    }
    h->device = dev;
    e = bra::prepare_attend(p, bf16);
    if (e == hipSuccess && bra::small_applies(p, bf16)) e = bra::prepare_small(p);
    if (e != hipSuccess) {
        delete h;
        return fail_hip(e, "bra_create: attention kernel LDS limit");
    }
    if (bra::image_applies(p, bf16)) {
        e = bra::prepare_image(p);
        if (e != hipSuccess) {
            delete h;
            return fail_hip(e, "bra_create: image kernel LDS limit");
        }
    }
    e = hipMalloc(&h->base, h->bytes);
    if (e != hipSuccess) {
        delete h;
        return fail_hip(e, "bra_create: hipMalloc of the workspace");
    }
    workspace_layout(*cfg, p, bf16, static_cast<char*>(h->base), &h->ws);
    e = hipMemset(h->ws.zero_bias, 0, h->ws.zero_bytes);
    if (e != hipSuccess) {
        (void)hipFree(h->base);
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
    hipError_t e = hipFree(h->base);
    delete h;
    if (e != hipSuccess) return fail_hip(e, "bra_destroy: hipFree");
    return BRA_OK;
}

int32_t bra_topk_effective(bra_handle_t h) {
    if (!is_live(h)) return -1;
    return h->params.k;
}

// The pointer checks of the forward entry points (`what` names the caller in
// messages); `bytes` is the size of one [B,H,W,C] map.
static bra_status_t check_pointers(const char* what, size_t bytes, const void* q, const void* k,
                                   const void* v, const float* lepe_w, const float* lepe_b,
                                   const void* out, const int32_t* routing_idx) {
    const std::string w(what);
    if (!q || !k || !v || !out) return fail(BRA_ERR_NULL, w + ": q, k, v and out are required");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(BRA_ERR_ALIGN, w + ": q, k, v and out must be 16-byte aligned");
    if (!aligned(lepe_w, 4) || !aligned(lepe_b, 4) || !aligned(routing_idx, 4))
        return fail(BRA_ERR_ALIGN, w + ": lepe_w, lepe_b and routing_idx must be 4-byte aligned");
    if (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes))
        return fail(BRA_ERR_ALIAS, w + ": out must not overlap q, k or v");
    return BRA_OK;
}

static size_t map_bytes(const bra_config_t& c) {
    return static_cast<size_t>(c.batch) * c.height * c.width * c.channels *
           (c.dtype == BRA_BF16 ? 2 : 4);
}

// The argument checks of the handle entry points.
static bra_status_t check_forward_args(bra_handle_t h, const char* what, const void* q,
                                       const void* k, const void* v, const float* lepe_w,
                                       const float* lepe_b, const void* out,
                                       const int32_t* routing_idx) {
    const std::string w(what);
    if (!is_live(h)) return fail(BRA_ERR_BAD_HANDLE, w + ": not a live handle");
    bra_status_t st =
        check_pointers(what, map_bytes(h->cfg), q, k, v, lepe_w, lepe_b, out, routing_idx);
    if (st != BRA_OK) return st;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, (w + ": hipGetDevice").c_str());
    if (dev != h->device) return fail(BRA_ERR_DEVICE, w + ": wrong current device");
    return BRA_OK;
}

// The forward steps on stream s, with the workspace ws.  With x
// (projections), the qkv projection writes the workspace's q, k, v (and the
// region means), and the attention kernel applies the output projection
// w_o, b_o; otherwise the pool kernel reads the caller's q and k.  ev: NULL,
// or kEventsPerCall events to record around the steps.
static bra_status_t enqueue_forward(const bra::Params& P, bool bf16, const bra_workspace& ws,
                                    hipEvent_t* ev, const char* what, const void* x,
                                    const void* w_qkv, const float* b_qkv, const void* q,
                                    const void* k, const void* v, const float* lepe_w,
                                    const float* lepe_b, const void* w_o, const float* b_o,
                                    void* out, int32_t* routing_idx, hipStream_t s) {
    const std::string wh(what);
    hipError_t e;
    if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess)
        return fail_hip(e, (wh + ": hipEventRecord").c_str());
    // the routing goes to the caller's buffer when one is given
    int32_t* routing = routing_idx ? routing_idx : ws.routing;
    // small fp32 problems: the whole forward in one kernel, one workgroup per
    // (image, head, region)
    const bool small = !x && !ws.kd && bra::small_applies(P, bf16);
    // maps whose head-group K and V fit LDS: the whole forward in one kernel
    const bool image = !small && bra::image_applies(P, bf16);
    // small region grids with many heads: means and routing in one kernel
    const bool pool_route = !x && !image && !small &&
                            bra::route_in_pool(bf16, P.shared != 0, P.R, P.heads, P.t);
    if (x) {
        e = bra::launch_proj_qkv(P, x, w_qkv, b_qkv, ws.qs, ws.ks, ws.vs, ws.means, lepe_w,
                                 ws.lepe_table, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": qkv projection launch").c_str());
        q = ws.qs;
        k = ws.ks;
        v = ws.vs;
    } else if (pool_route) {
        e = bra::launch_pool_route(P, q, k, lepe_w, ws.lepe_table, routing, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": region-pool and routing launch").c_str());
    } else if (!image && !small) {
        e = bra::launch_pool_qk(P, bf16, q, k, lepe_w, ws.means, ws.lepe_table, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": region-pool launch").c_str());
    }
    if (ws.kd) {
        e = bra::launch_kv_pool(P, bf16, k, v, ws.kd, ws.vd, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": K/V downsampling launch").c_str());
    }
    if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess)
        return fail_hip(e, (wh + ": hipEventRecord").c_str());
    // small region grids are routed inside the attention kernel
    if (!image && !small && !bra::route_in_attend(P) && !pool_route) {
        e = bra::launch_route(P, bf16, ws.means, routing, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": routing launch").c_str());
    }
    if (ev && (e = hipEventRecord(ev[2], s)) != hipSuccess)
        return fail_hip(e, (wh + ": hipEventRecord").c_str());
    // the output projection: in the attention kernel's epilogue, or over y
    // in a kernel of its own (ws.ys is set for the shapes that take that)
    const bool proj_after = w_o && ws.ys;
    if (small) {
        e = bra::launch_small(P, static_cast<const float*>(q), static_cast<const float*>(k),
                              static_cast<const float*>(v), lepe_w, lepe_b, routing,
                              static_cast<float*>(out), s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": small-problem kernel launch").c_str());
    } else if (image) {
        e = bra::launch_image(P, q, k, v, lepe_w, lepe_b, routing, false,
                              proj_after ? ws.ys : out, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": image kernel launch").c_str());
    } else {
        e = bra::launch_attend(P, bf16, q, v, ws.kd ? ws.kd : k, ws.vd ? ws.vd : v, ws.means,
                               routing, !bra::route_in_attend(P), lepe_w, lepe_b, ws.lepe_table,
                               ws.zero_bias, proj_after ? nullptr : w_o, b_o,
                               proj_after ? ws.ys : out, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": attention launch").c_str());
    }
    if (proj_after) {
        e = bra::launch_proj_out(P, ws.ys, w_o, b_o, out, s);
        if (e != hipSuccess) return fail_hip(e, (wh + ": output projection launch").c_str());
    }
    if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess)
        return fail_hip(e, (wh + ": hipEventRecord").c_str());
    return BRA_OK;
}

// enqueue_forward with the handle's workspace and timing slots.
static bra_status_t enqueue_handle(bra_handle_t h, const char* what, const void* x,
                                   const void* w_qkv, const float* b_qkv, const void* q,
                                   const void* k, const void* v, const float* lepe_w,
                                   const float* lepe_b, const void* w_o, const float* b_o,
                                   void* out, int32_t* routing_idx, hipStream_t s) {
    const bool timed = h->timing_used < h->timing_capacity;
    hipEvent_t* ev = timed ? &h->events[kEventsPerCall * h->timing_used] : nullptr;
    bra_status_t st = enqueue_forward(h->params, h->bf16, h->ws, ev, what, x, w_qkv, b_qkv, q,
                                      k, v, lepe_w, lepe_b, w_o, b_o, out, routing_idx, s);
    if (st == BRA_OK && timed) ++h->timing_used;
    return st;
}

bra_status_t bra_forward(bra_handle_t h, const void* q, const void* k, const void* v,
                         const float* lepe_w, const float* lepe_b, void* out,
                         int32_t* routing_idx, void* stream) {
    bra_status_t st = check_forward_args(h, "bra_forward", q, k, v, lepe_w, lepe_b, out,
                                         routing_idx);
    if (st != BRA_OK) return st;
    return enqueue_handle(h, "bra_forward", nullptr, nullptr, nullptr, q, k, v, lepe_w, lepe_b,
                          nullptr, nullptr, out, routing_idx, static_cast<hipStream_t>(stream));
}

bra_status_t bra_forward_proj(bra_handle_t h, const void* x, const void* w_qkv,
                              const float* b_qkv, const float* lepe_w, const float* lepe_b,
                              const void* w_o, const float* b_o, void* out,
                              int32_t* routing_idx, void* stream) {
    bra_status_t st = check_forward_args(h, "bra_forward_proj", x, x, x, lepe_w, lepe_b, out,
                                         routing_idx);
    if (st != BRA_OK) return st;
    if (!h->ws.qs)
        return fail(BRA_ERR_UNSUPPORTED,
                    "bra_forward_proj: the handle was created without projections");
    if (!w_qkv || !w_o) return fail(BRA_ERR_NULL, "bra_forward_proj: w_qkv and w_o are required");
    if (!aligned(w_qkv, 16) || !aligned(w_o, 16) || !aligned(b_qkv, 4) || !aligned(b_o, 4))
        return fail(BRA_ERR_ALIGN,
                    "bra_forward_proj: w_qkv and w_o must be 16-byte aligned, the biases 4-byte");
    return enqueue_handle(h, "bra_forward_proj", x, w_qkv, b_qkv, nullptr, nullptr, nullptr,
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
    if (bra::image_applies(h->params, h->bf16)) {
        e = bra::launch_image(h->params, q, k, v, lepe_w, lepe_b,
                              const_cast<int32_t*>(routing_idx), true, out, s);
        if (e != hipSuccess) return fail_hip(e, "bra_forward_routed: image kernel launch");
        return BRA_OK;
    }
    // the MFMA LePE operand table is the region-pool kernel's side product:
    // build it alone (no means) when this shape uses it
    const bra_workspace& ws = h->ws;
    if (lepe_w && h->params.table_items > 0) {
        e = bra::launch_lepe_table(h->params, lepe_w, ws.lepe_table, s);
        if (e != hipSuccess) return fail_hip(e, "bra_forward_routed: LePE table launch");
    }
    if (ws.kd) {
        e = bra::launch_kv_pool(h->params, h->bf16, k, v, ws.kd, ws.vd, s);
        if (e != hipSuccess) return fail_hip(e, "bra_forward_routed: K/V downsampling launch");
    }
    e = bra::launch_attend(h->params, h->bf16, q, v, ws.kd ? ws.kd : k, ws.vd ? ws.vd : v,
                           ws.means, const_cast<int32_t*>(routing_idx), true, lepe_w, lepe_b,
                           ws.lepe_table, ws.zero_bias, nullptr, nullptr, out, s);
    if (e != hipSuccess) return fail_hip(e, "bra_forward_routed: attention launch");
    return BRA_OK;
}

bra_status_t bra_forward_noalloc(const bra_config_t* cfg, const void* q, const void* k,
                                const void* v, const float* lepe_w, const float* lepe_b,
                                void* out, int32_t* routing_idx, void* stream) {
    const char* what = "bra_forward_noalloc";
    bra::Params p;
    bool bf16 = false;
    bra_status_t st = validate_config(cfg, what, p, bf16);
    if (st != BRA_OK) return st;
    if (cfg->projections)
        return fail(BRA_ERR_UNSUPPORTED,
                    "bra_forward_noalloc: projections run through bra_forward_proj only");
    st = check_pointers(what, map_bytes(*cfg), q, k, v, lepe_w, lepe_b, out, routing_idx);
    if (st != BRA_OK) return st;
    const size_t need = workspace_layout(*cfg, p, bf16, nullptr, nullptr);
    if (need > bra::scratch_bytes())
        return fail(BRA_ERR_UNSUPPORTED,
                    "bra_forward_noalloc: this configuration needs " + std::to_string(need) +
                        " bytes of scratch, more than the " +
                        std::to_string(bra::scratch_bytes()) + " the library holds");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "bra_forward_noalloc: hipGetDevice");
    void* base = nullptr;
    e = bra::scratch_pointer(dev, &base);
    if (e != hipSuccess) return fail_hip(e, "bra_forward_noalloc: hipGetSymbolAddress");
    e = bra::prepare_attend(p, bf16);
    if (e == hipSuccess && bra::small_applies(p, bf16)) e = bra::prepare_small(p);
    if (e != hipSuccess) return fail_hip(e, "bra_forward_noalloc: attention kernel LDS limit");
    if (bra::image_applies(p, bf16)) {
        e = bra::prepare_image(p);
        if (e != hipSuccess) return fail_hip(e, "bra_forward_noalloc: image kernel LDS limit");
    }
    bra_workspace ws;
    workspace_layout(*cfg, p, bf16, static_cast<char*>(base), &ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the stand-in bias must read zero, whatever the array held before
    if (lepe_w && !lepe_b) {
        e = bra::launch_zero_fill(ws.zero_bias, cfg->channels, s);
        if (e != hipSuccess) return fail_hip(e, "bra_forward_noalloc: zero fill launch");
    }
    return enqueue_forward(p, bf16, ws, nullptr, what, nullptr, nullptr, nullptr, q, k, v,
                           lepe_w, lepe_b, nullptr, nullptr, out, routing_idx, s);
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

bra_status_t bra_debug_inject_alloc_failure(int32_t which, int32_t count) {
    if (count < 0) return fail(BRA_ERR_SHAPE, "bra_debug_inject_alloc_failure: count must be >= 0");
    std::lock_guard<std::mutex> lock(g_mutex);
    if (which == BRA_ALLOC_HOST)
        g_fail_host = count;
    else if (which == BRA_ALLOC_DEVICE)
        g_fail_device = count;
    else
        return fail(BRA_ERR_SHAPE, "bra_debug_inject_alloc_failure: unknown allocation kind");
    return BRA_OK;
}

int32_t bra_debug_live_handles(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    return static_cast<int32_t>(g_live.size());
}

bra_status_t bra_debug_projected_qkv(bra_handle_t h, void* q, void* k, void* v, void* stream) {
    if (!is_live(h)) return fail(BRA_ERR_BAD_HANDLE, "bra_debug_projected_qkv: not a live handle");
    if (!h->ws.qs)
        return fail(BRA_ERR_UNSUPPORTED,
                    "bra_debug_projected_qkv: the handle was created without projections");
    if (!q || !k || !v) return fail(BRA_ERR_NULL, "bra_debug_projected_qkv: q, k, v are required");
    const size_t bytes = map_bytes(h->cfg);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const void* src[3] = {h->ws.qs, h->ws.ks, h->ws.vs};
    void* dst[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
        hipError_t e = hipMemcpyAsync(dst[i], src[i], bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return fail_hip(e, "bra_debug_projected_qkv: hipMemcpyAsync");
    }
    return BRA_OK;
}

}  // extern "C"
