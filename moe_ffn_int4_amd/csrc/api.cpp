// api.cpp -- the C ABI declared in include/moe_int4.h: argument validation,
// workspace carving, path choice and kernel launch order.
//
// Validation is plain host code and runs before any HIP call, so every
// invalid-argument path can be exercised without a GPU.
#include "moe_int4.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

static_assert(MOE_MAX_EXPERTS == moe::kMaxExperts, "expert limit mismatch");
static_assert(MOE_GROUP_SIZE == moe::kGroup, "group size mismatch");

namespace moe {
LaunchTiming& launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}
}  // namespace moe

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// largest P + T whose down projection splits its reduction (workspace for O2)
constexpr int64_t kSplitRows = 2048;

// Workspace sections (byte offsets from the workspace base).
struct Layout {
    size_t partials, logits, ids, gates, counts, offsets, tile_base, perm, inv, chunks, nchunks,
        routing_end, x_perm, H, O, O2, total;
    size_t xq, sxq, hq, shq, total_fp8;  // fp8 experts: quantized x and H rows, row scales
    int slices;
    int max_chunks;
};

int64_t max_decode_chunks(const moe_dims& d) {
    const int64_t P = d.T * d.top_k;
    const int64_t R = moe::kDecodeRows;
    return (d.E < P ? d.E : P) + (P + R - 1) / R + (d.T + R - 1) / R;
}

Layout layout(const moe_dims& d) {
    const size_t T = d.T, E = d.E, P = static_cast<size_t>(d.T) * d.top_k;
    Layout L{};
    const moe::RouterPlan plan = moe::router_plan(d.T, d.d, d.E);
    L.slices = plan.slices;
    L.max_chunks = static_cast<int>(max_decode_chunks(d));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += round_up(bytes);
        return at;
    };
    L.partials = take(static_cast<size_t>(plan.slices) * T * E * 4);
    L.logits = take(T * E * 4);
    L.ids = take(P * 4);
    L.gates = take(P * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.tile_base = take((E + 2) * 4);
    L.perm = take(P * 4);
    L.inv = take(P * 4);
    L.chunks = take(static_cast<size_t>(L.max_chunks) * 16);
    L.nchunks = take(4);
    L.routing_end = off;
    L.x_perm = take(T * static_cast<size_t>(d.d) * 2);
    L.H = take((P + T) * static_cast<size_t>(d.h) * 2);
    L.O = take((P + T) * static_cast<size_t>(d.d) * 4);
    // the streaming down projection's second partial sums (small batches only)
    L.O2 = take(static_cast<int64_t>(P + T) <= kSplitRows ? (P + T) * static_cast<size_t>(d.d) * 4 : 0);
    L.total = off;
    L.xq = take(T * static_cast<size_t>(d.d));
    L.sxq = take(T * 4);
    L.hq = take(P * static_cast<size_t>(d.h));
    L.shq = take(P * 4);
    L.total_fp8 = off;
    return L;
}

// The one-block routing kernel covers small batches (decode).
// The one-block routing kernel handles up to kSmallRoutePairs pairs, but its
// time grows with them (one block). Against the multi-block top-k + dispatch
// kernels (about 13 us), measured with 16 experts: 6.4 and 9.7 us at 16 and 32
// pairs, 14.7 us at 64 (with 4 experts it still wins there), 22 us at 128 and
// 53 us at 512. It is chosen up to kSmallRouteMaxPairs.
constexpr int64_t kSmallRouteMaxPairs = 64;
static_assert(kSmallRouteMaxPairs <= moe::kSmallRoutePairs, "within the kernel's capacity");

bool small_routing(const moe_dims& d) {
    return d.T * d.E <= moe::kSmallRouteLogits && d.T * d.top_k <= kSmallRouteMaxPairs;
}

// MOE_PATH_AUTO: the streaming decode path for small batches; the hybrid path
// when the pairs average under kHybridAvgPairs per routed expert.
constexpr int64_t kDecodeMaxPairs = 64;
constexpr int64_t kHybridAvgPairs = 256;
// MOE_PATH_HYBRID: routed experts with at most this many pairs stream
constexpr int kHybridRows = 32;

bool group_ok(int32_t g) { return g == 128 || g == 64 || g == 32; }

int check_dims(const moe_dims* d) {
    if (!d) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
    if (!group_ok(d->group_size))
        return fail(MOE_ERR_INVALID_ARG, "group_size %d unsupported (128, 64 or 32)", d->group_size);
    if (d->T < 1) return fail(MOE_ERR_INVALID_ARG, "T = %lld must be >= 1", (long long)d->T);
    if (d->d < 128 || d->d % 128)
        return fail(MOE_ERR_INVALID_ARG, "d = %lld must be a positive multiple of 128", (long long)d->d);
    if (d->h < 128 || d->h % 128)
        return fail(MOE_ERR_INVALID_ARG, "h = %lld must be a positive multiple of 128", (long long)d->h);
    if (d->E < 1 || d->E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_INVALID_ARG, "E = %lld outside [1, %d]", (long long)d->E, MOE_MAX_EXPERTS);
    if (d->top_k < 1 || d->top_k > d->E || d->top_k > MOE_MAX_TOP_K)
        return fail(MOE_ERR_INVALID_ARG, "top_k = %d outside [1, min(E, %d)]", d->top_k, MOE_MAX_TOP_K);
    const long long P = (long long)d->T * d->top_k;
    if (P + d->T > (1LL << 30))
        return fail(MOE_ERR_INVALID_ARG, "T * (top_k + 1) = %lld exceeds 2^30", P + d->T);
    if (d->E * d->h * (d->d / 2) > (1LL << 40))
        return fail(MOE_ERR_INVALID_ARG, "expert weights exceed 1 TiB");
    return MOE_OK;
}

int check_ptr(const void* p, const char* name, size_t align = 16) {
    if (!p) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(MOE_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
    return MOE_OK;
}

#define CHECK(expr)                   \
    do {                              \
        int rc_ = (expr);             \
        if (rc_ != MOE_OK) return rc_; \
    } while (0)

#define HIP_CHECK(expr, what)                    \
    do {                                         \
        hipError_t e_ = (expr);                  \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

// ---- optional per-stage timing (moe_profile_*)
struct Prof {
    std::mutex mu;
    bool on = false;
    struct Rec {
        int stage;
        hipEvent_t a, b;
    };
    std::vector<Rec> pending;
    std::vector<hipEvent_t> pool;
    double ms[MOE_STAGE_COUNT] = {};
    int64_t n[MOE_STAGE_COUNT] = {};
};
Prof& prof() {
    static Prof p;
    return p;
}

hipError_t prof_event(hipEvent_t* ev) {
    Prof& P = prof();
    if (!P.pool.empty()) {
        *ev = P.pool.back();
        P.pool.pop_back();
        return hipSuccess;
    }
    return hipEventCreate(ev);
}

// Launch `fn` (returning hipError_t) as `stage`; when timing is enabled its
// kernels record a pair of events at the first one's start and the last one's end.
template <typename F>
int timed(int stage, hipStream_t s, const char* what, F&& fn) {
    Prof& P = prof();
    std::unique_lock<std::mutex> lock(P.mu);
    if (!P.on) {
        lock.unlock();
        HIP_CHECK(fn(), what);
        return MOE_OK;
    }
    Prof::Rec r{stage, nullptr, nullptr};
    HIP_CHECK(prof_event(&r.a), "hipEventCreate");
    HIP_CHECK(prof_event(&r.b), "hipEventCreate");
    // the stage's kernels record the events at their own start and end
    moe::LaunchTiming& lt = moe::launch_timing();
    lt.start = r.a;
    lt.stop = r.b;
    const hipError_t e = fn();
    const bool launched = lt.start == nullptr;  // the first launch took the start event
    lt.start = lt.stop = nullptr;
    if (launched) {
        P.pending.push_back(r);
    } else {
        P.pool.push_back(r.a);
        P.pool.push_back(r.b);
    }
    HIP_CHECK(e, what);
    (void)s;
    return MOE_OK;
}

// Cached "is gfx950" per device ordinal.
int device_ok() {
    static std::mutex mu;
    static int state[64];  // 0 unknown, 1 ok, 2 unsupported
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device ordinal %d", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (state[dev] == 2) {
            return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device %d is %s, this library is built for gfx950",
                        dev, prop.gcnArchName);
        }
    }
    if (state[dev] == 2) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
    return MOE_OK;
}

int check_forward_args(const moe_dims* dims, const uint16_t* x, const float* router_w,
                       const float* router_b, void* workspace, size_t workspace_bytes,
                       bool routing_only = false, bool fp8 = false) {
    CHECK(check_dims(dims));
    CHECK(check_ptr(x, "x"));
    CHECK(check_ptr(router_w, "router_w"));
    if (router_b) CHECK(check_ptr(router_b, "router_b", 4));
    if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, kAlign)) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    const Layout L = layout(*dims);
    const size_t need = routing_only ? L.routing_end : (fp8 ? L.total_fp8 : L.total);
    if (workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    return MOE_OK;
}

struct Routing {
    float* partials;
    float* logits;
    int32_t* ids;
    float* gates;
    int32_t* counts;
    int32_t* offsets;
    int32_t* tile_base;
    int32_t* perm;
    int32_t* inv;
    int4* chunks;
    int32_t* nchunks;
};

Routing carve(const moe_dims& d, void* ws) {
    const Layout L = layout(d);
    char* b = static_cast<char*>(ws);
    Routing R;
    R.partials = reinterpret_cast<float*>(b + L.partials);
    R.logits = reinterpret_cast<float*>(b + L.logits);
    R.ids = reinterpret_cast<int32_t*>(b + L.ids);
    R.gates = reinterpret_cast<float*>(b + L.gates);
    R.counts = reinterpret_cast<int32_t*>(b + L.counts);
    R.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
    R.tile_base = reinterpret_cast<int32_t*>(b + L.tile_base);
    R.perm = reinterpret_cast<int32_t*>(b + L.perm);
    R.inv = reinterpret_cast<int32_t*>(b + L.inv);
    R.chunks = reinterpret_cast<int4*>(b + L.chunks);
    R.nchunks = reinterpret_cast<int32_t*>(b + L.nchunks);
    return R;
}

// The hybrid path's second stream: per device, a non-blocking stream of
// default priority owned by the library (kept for the life of the process)
// and the events that fork the small experts' streaming kernels off the
// caller's stream and join them back. The fork and join of one call are
// enqueued under the mutex, so calls from several host threads cannot
// interleave their event records; the GPU work of such calls then shares the
// side stream in enqueue order.
struct Side {
    std::mutex mu;
    bool ready = false;
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, mid = nullptr, quant = nullptr, join = nullptr;
};

int side_stream(Side** out) {
    static Side sides[64];
    int dev = 0;
    HIP_CHECK(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device ordinal %d", dev);
    Side& sd = sides[dev];
    std::lock_guard<std::mutex> lock(sd.mu);
    if (!sd.ready) {
        HIP_CHECK(hipStreamCreateWithFlags(&sd.stream, hipStreamNonBlocking), "hipStreamCreate");
        for (hipEvent_t* e : {&sd.fork, &sd.mid, &sd.quant, &sd.join})
            HIP_CHECK(hipEventCreateWithFlags(e, hipEventDisableTiming), "hipEventCreate");
        sd.ready = true;
    }
    *out = &sd;
    return MOE_OK;
}

// ---- scratch of the allocation-free forward (moe_forward_noalloc)
// Its workspace is this file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host code
// the array's name is a host-side stand-in, not a device address: host code
// only ever uses the address hipGetSymbolAddress returns for the current
// device (scratch_address), never the name.
constexpr size_t kScratchBytes = static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) uint8_t scratch[kScratchBytes];

// Set-up, once per device with that device current: the array's device address,
// and the hybrid path's second stream, so later calls create nothing.
int scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    HIP_CHECK(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device ordinal %d", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p || !aligned(p, kAlign))
            return fail(MOE_ERR_HIP, "scratch has no 256-byte aligned device address");
        Side* side = nullptr;
        CHECK(side_stream(&side));
        addr[dev] = p;
    }
    *out = addr[dev];
    return MOE_OK;
}

// Router partial logits, then either the one-block small-batch finish (top-k,
// dispatch, decode chunks) or the top-k kernel + the per-expert dispatch kernel.
// small_rows: which groups get streaming chunks and which GEMM tiles (build_work_lists)
int run_routing(const moe_dims& d, const uint16_t* x, const float* wr, const float* b,
                const Routing& R, int32_t* ids_out, float* gates_out, uint16_t* x_perm,
                int small_rows, int tile_rows, hipStream_t s) {
    const moe::RouterPlan plan = moe::router_plan(d.T, d.d, d.E);
    CHECK(timed(MOE_STAGE_ROUTER, s, "router launch", [&] {
        return moe::launch_router_partials(x, wr, d.T, d.d, d.E, plan, R.partials, x_perm, s);
    }));
    if (small_routing(d)) {
        CHECK(timed(MOE_STAGE_TOPK, s, "small routing launch", [&] {
            return moe::launch_route_small(R.partials, plan.slices, b, d.T, d.E, d.top_k,
                                           tile_rows, small_rows, R.logits, R.ids, R.gates, ids_out,
                                           gates_out, R.counts, R.offsets, R.tile_base, R.perm,
                                           R.inv, R.chunks, R.nchunks, s);
        }));
        return MOE_OK;
    }
    CHECK(timed(MOE_STAGE_TOPK, s, "top-k launch", [&] {
        return moe::launch_topk(R.partials, plan.slices, b, d.T, d.E, d.top_k, R.logits, R.ids,
                                R.gates, ids_out, gates_out, s);
    }));
    CHECK(timed(MOE_STAGE_DISPATCH, s, "dispatch launch", [&] {
        return moe::launch_dispatch(R.ids, d.T, d.top_k, d.E, tile_rows, small_rows, R.counts, R.offsets,
                                    R.tile_base, R.perm, R.inv, R.chunks, R.nchunks, s);
    }));
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_abi_version(void) { return MOE_INT4_ABI_VERSION; }

int moe_device_check(void) { return device_ok(); }

static int quantize(const float* w, int64_t rows, int64_t K, int32_t group_size, uint8_t* q,
                    float* scales, bool tiled, void* stream) {
    g_last_error.clear();
    if (!group_ok(group_size))
        return fail(MOE_ERR_INVALID_ARG, "group_size %d unsupported (128, 64 or 32)", group_size);
    if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows = %lld is negative", (long long)rows);
    if (K < 128 || K % 128)
        return fail(MOE_ERR_INVALID_ARG, "K = %lld must be a positive multiple of 128", (long long)K);
    if (tiled && rows % 16)
        return fail(MOE_ERR_INVALID_ARG, "rows = %lld must be a multiple of 16 for the tiled layout",
                    (long long)rows);
    if (rows == 0) return MOE_OK;
    CHECK(check_ptr(w, "w"));
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(scales, "scales", 4));
    CHECK(device_ok());
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return timed(MOE_STAGE_QUANTIZE, s, "quantize launch", [&] {
        return moe::launch_quantize_int4(w, rows, K, group_size, q, scales, tiled, s);
    });
}

int moe_quantize_int4(const float* w, int64_t rows, int64_t K, int32_t group_size, uint8_t* q,
                      float* scales, void* stream) {
    return quantize(w, rows, K, group_size, q, scales, false, stream);
}

int moe_quantize_int4_tiled(const float* w, int64_t rows, int64_t K, int32_t group_size, uint8_t* q,
                            float* scales, void* stream) {
    return quantize(w, rows, K, group_size, q, scales, true, stream);
}

int moe_tile_int4(const uint8_t* q, const float* scales, int64_t rows, int64_t K, int32_t group_size,
                  uint8_t* q_tiled, float* scales_tiled, void* stream) {
    g_last_error.clear();
    if (!group_ok(group_size))
        return fail(MOE_ERR_INVALID_ARG, "group_size %d unsupported (128, 64 or 32)", group_size);
    if (rows < 0 || rows % 16)
        return fail(MOE_ERR_INVALID_ARG, "rows = %lld must be a non-negative multiple of 16",
                    (long long)rows);
    if (K < 128 || K % 128)
        return fail(MOE_ERR_INVALID_ARG, "K = %lld must be a positive multiple of 128", (long long)K);
    if (rows == 0) return MOE_OK;
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(scales, "scales", 4));
    CHECK(check_ptr(q_tiled, "q_tiled"));
    CHECK(check_ptr(scales_tiled, "scales_tiled", 4));
    auto overlap = [](const void* a, const void* b, uintptr_t n, uintptr_t m) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
        return x < y + m && y < x + n;
    };
    const uintptr_t nq = static_cast<uintptr_t>(rows) * (K / 2);
    const uintptr_t ns = static_cast<uintptr_t>(rows) * (K / group_size) * 4;
    if (overlap(q, q_tiled, nq, nq) || overlap(q, scales_tiled, nq, ns) ||
        overlap(scales, q_tiled, ns, nq) || overlap(scales, scales_tiled, ns, ns))
        return fail(MOE_ERR_INVALID_ARG, "the row-major and tiled buffers overlap");
    CHECK(device_ok());
    HIP_CHECK(moe::launch_tile_int4(q, scales, rows, K, group_size, q_tiled, scales_tiled,
                                    static_cast<hipStream_t>(stream)),
              "tile launch");
    return MOE_OK;
}

int moe_pack_bf16_tiled(const uint16_t* src, int64_t rows, int64_t K, uint16_t* dst, void* stream) {
    g_last_error.clear();
    if (rows < 0 || rows % 16)
        return fail(MOE_ERR_INVALID_ARG, "rows = %lld must be a non-negative multiple of 16",
                    (long long)rows);
    if (K < 128 || K % 128)
        return fail(MOE_ERR_INVALID_ARG, "K = %lld must be a positive multiple of 128", (long long)K);
    if (rows == 0) return MOE_OK;
    CHECK(check_ptr(src, "src"));
    CHECK(check_ptr(dst, "dst"));
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t n = static_cast<uintptr_t>(rows) * K * 2;
    if (a < b + n && b < a + n) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
    CHECK(device_ok());
    HIP_CHECK(moe::launch_pack_bf16(src, rows, K, dst, static_cast<hipStream_t>(stream)), "pack launch");
    return MOE_OK;
}

int moe_quantize_fp8_tiled(const float* w, int64_t rows, int64_t K, uint8_t* q, float* scales,
                           void* stream) {
    g_last_error.clear();
    if (rows < 0 || rows % 16)
        return fail(MOE_ERR_INVALID_ARG, "rows = %lld must be a non-negative multiple of 16",
                    (long long)rows);
    if (K < 128 || K % 128)
        return fail(MOE_ERR_INVALID_ARG, "K = %lld must be a positive multiple of 128", (long long)K);
    if (rows == 0) return MOE_OK;
    CHECK(check_ptr(w, "w"));
    CHECK(check_ptr(q, "q", 4));
    CHECK(check_ptr(scales, "scales", 4));
    CHECK(device_ok());
    HIP_CHECK(moe::launch_quantize_fp8_weights(w, rows, K, q, scales, static_cast<hipStream_t>(stream)),
              "fp8 quantize launch");
    return MOE_OK;
}

int moe_quantize_fp8_rows(const uint16_t* x, int64_t rows, int64_t K, float ub, uint8_t* q,
                          float* scales, void* stream) {
    g_last_error.clear();
    if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows = %lld is negative", (long long)rows);
    if (K < 128 || K % 128)
        return fail(MOE_ERR_INVALID_ARG, "K = %lld must be a positive multiple of 128", (long long)K);
    if (!(ub >= 0.f) || ub > 3.0e38f) return fail(MOE_ERR_INVALID_ARG, "ub must be finite and >= 0");
    if (rows == 0) return MOE_OK;
    CHECK(check_ptr(x, "x", 8));
    CHECK(check_ptr(q, "q", 4));
    CHECK(check_ptr(scales, "scales", 4));
    CHECK(device_ok());
    HIP_CHECK(moe::launch_quantize_fp8_activations(x, rows, K, ub, q, scales,
                                                   static_cast<hipStream_t>(stream)),
              "fp8 activation quantize launch");
    return MOE_OK;
}

size_t moe_forward_workspace_bytes(const moe_dims* dims) {
    const std::string saved = g_last_error;
    if (check_dims(dims) != MOE_OK) return 0;
    g_last_error = saved;
    return layout(*dims).total;
}

size_t moe_route_workspace_bytes(const moe_dims* dims) {
    const std::string saved = g_last_error;
    if (!dims) return 0;
    moe_dims d = *dims;
    d.h = 128;
    if (check_dims(&d) != MOE_OK) return 0;
    g_last_error = saved;
    return layout(d).routing_end;
}

int moe_route(const moe_dims* dims, const uint16_t* x, const float* router_w,
              const float* router_b, int32_t* topk_ids, float* topk_gates, float* logits,
              int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, void* workspace,
              size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    CHECK(check_forward_args(dims, x, router_w, router_b, workspace, workspace_bytes, true));
    CHECK(check_ptr(topk_ids, "topk_ids", 4));
    CHECK(check_ptr(topk_gates, "topk_gates", 4));
    CHECK(device_ok());
    const moe_dims& d = *dims;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Routing R = carve(d, workspace);
    CHECK(run_routing(d, x, router_w, router_b, R, topk_ids, topk_gates, nullptr, 0, moe::kPrefillBM, s));
    const size_t P = static_cast<size_t>(d.T) * d.top_k;
    if (logits)
        HIP_CHECK(hipMemcpyAsync(logits, R.logits, d.T * d.E * 4, hipMemcpyDeviceToDevice, s), "copy");
    if (counts) HIP_CHECK(hipMemcpyAsync(counts, R.counts, d.E * 4, hipMemcpyDeviceToDevice, s), "copy");
    if (offsets)
        HIP_CHECK(hipMemcpyAsync(offsets, R.offsets, (d.E + 1) * 4, hipMemcpyDeviceToDevice, s), "copy");
    if (perm) HIP_CHECK(hipMemcpyAsync(perm, R.perm, P * 4, hipMemcpyDeviceToDevice, s), "copy");
    if (inv) HIP_CHECK(hipMemcpyAsync(inv, R.inv, P * 4, hipMemcpyDeviceToDevice, s), "copy");
    return MOE_OK;
}

// The forward for int4 (ex4), bf16 (exb) or fp8 (ex8) routed experts; exactly one is set.
static int forward_impl(const moe_dims* dims, const uint16_t* x, const float* router_w,
                        const float* router_b, const moe_experts_int4* ex4,
                        const moe_experts_bf16* exb, const moe_experts_fp8* ex8,
                        const moe_shared_bf16* sh, uint16_t* y, int32_t* topk_ids,
                        float* topk_gates, int32_t path, void* workspace, size_t workspace_bytes,
                        void* stream) {
    g_last_error.clear();
    CHECK(check_forward_args(dims, x, router_w, router_b, workspace, workspace_bytes, false,
                             ex8 != nullptr));
    if (!ex4 && !exb && !ex8) return fail(MOE_ERR_INVALID_ARG, "experts is NULL");
    if (!sh) return fail(MOE_ERR_INVALID_ARG, "shared is NULL");
    if (ex8) {
        CHECK(check_ptr(ex8->w1q, "experts->w1q", 4));
        CHECK(check_ptr(ex8->w3q, "experts->w3q", 4));
        CHECK(check_ptr(ex8->w2q, "experts->w2q", 4));
        CHECK(check_ptr(ex8->w1s, "experts->w1s", 4));
        CHECK(check_ptr(ex8->w3s, "experts->w3s", 4));
        CHECK(check_ptr(ex8->w2s, "experts->w2s", 4));
        if (!(ex8->act_ub >= 0.f) || ex8->act_ub > 3.0e38f)
            return fail(MOE_ERR_INVALID_ARG, "experts->act_ub must be finite and >= 0");
    } else if (ex4) {
        CHECK(check_ptr(ex4->w1q, "experts->w1q"));
        CHECK(check_ptr(ex4->w3q, "experts->w3q"));
        CHECK(check_ptr(ex4->w2q, "experts->w2q"));
        CHECK(check_ptr(ex4->w1s, "experts->w1s", 4));
        CHECK(check_ptr(ex4->w3s, "experts->w3s", 4));
        CHECK(check_ptr(ex4->w2s, "experts->w2s", 4));
    } else {
        CHECK(check_ptr(exb->w1, "experts->w1"));
        CHECK(check_ptr(exb->w3, "experts->w3"));
        CHECK(check_ptr(exb->w2, "experts->w2"));
    }
    CHECK(check_ptr(sh->s1, "shared->s1"));
    CHECK(check_ptr(sh->s3, "shared->s3"));
    CHECK(check_ptr(sh->s2, "shared->s2"));
    CHECK(check_ptr(y, "y"));
    if (topk_ids) CHECK(check_ptr(topk_ids, "topk_ids", 4));
    if (topk_gates) CHECK(check_ptr(topk_gates, "topk_gates", 4));
    if (path != MOE_PATH_AUTO && path != MOE_PATH_PREFILL && path != MOE_PATH_DECODE &&
        path != MOE_PATH_HYBRID && path != MOE_PATH_PREFILL_WIDE)
        return fail(MOE_ERR_INVALID_ARG, "path %d unknown", path);
    CHECK(device_ok());

    const moe_dims& d = *dims;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Layout L = layout(d);
    const Routing R = carve(d, workspace);
    char* base = static_cast<char*>(workspace);
    uint16_t* H = reinterpret_cast<uint16_t*>(base + L.H);
    float* O = reinterpret_cast<float*>(base + L.O);
    const int64_t P = d.T * d.top_k;

    const bool decode =
        path == MOE_PATH_DECODE || (path == MOE_PATH_AUTO && P <= kDecodeMaxPairs);
    // decode path, int4 experts without sliced staging (P < 4 E): the down
    // projection splits its reduction over two blocks per chunk (twice the blocks
    // of a launch that otherwise leaves HBM underused), the second half into O2
    float* O2 = (decode && ex4 && P < 4 * d.E &&
                 P + d.T <= kSplitRows && d.h >= 2 * moe::kGroup)
                    ? reinterpret_cast<float*>(base + L.O2) : nullptr;
    const bool hybrid = !decode && (path == MOE_PATH_HYBRID ||
                                    (path == MOE_PATH_AUTO && P < kHybridAvgPairs * d.E));
    const int small_rows = decode ? -1 : (hybrid ? kHybridRows : 0);
    // 256 x 256 GEMM tiles: asked for, or (AUTO) the non-hybrid prefill
    const bool wide = !decode && !hybrid &&
                      (path == MOE_PATH_PREFILL_WIDE || path == MOE_PATH_AUTO);
    const int tile_rows = wide ? moe::kPrefillBM2 : moe::kPrefillBM;
    uint16_t* x_perm = reinterpret_cast<uint16_t*>(base + L.x_perm);
    uint8_t* xq = ex8 ? reinterpret_cast<uint8_t*>(base + L.xq) : nullptr;
    float* sxq = ex8 ? reinterpret_cast<float*>(base + L.sxq) : nullptr;
    uint8_t* hq = ex8 ? reinterpret_cast<uint8_t*>(base + L.hq) : nullptr;
    float* shq = ex8 ? reinterpret_cast<float*>(base + L.shq) : nullptr;
    // the interleaved copy of x feeds only the streaming kernel's int4 experts
    CHECK(run_routing(d, x, router_w, router_b, R, topk_ids, topk_gates,
                      (decode || hybrid) && ex4 ? x_perm : nullptr, small_rows, tile_rows, s));
    // fp8 experts: quantize x per row (the routed rows' A operand); H's routed
    // rows follow once the up-projections have written them
    if (ex8)
        CHECK(timed(MOE_STAGE_ACT_QUANT, s, "fp8 x quantize launch", [&] {
            return moe::launch_quantize_fp8_activations(x, d.T, d.d, ex8->act_ub, xq, sxq, s);
        }));
    auto quantize_h = [&] {
        return timed(MOE_STAGE_ACT_QUANT, s, "fp8 H quantize launch", [&] {
            return moe::launch_quantize_fp8_activations(H, P, d.h, ex8->act_ub, hq, shq, s);
        });
    };

    // streaming projections over the chunk list: every group (decode path) or
    // the small routed experts (hybrid path)
    // streaming chunks average 4+ rows: the kernel that stages their A rows in
    // LDS slices (measured: Maverick prefill 4.35 -> 4.12 ms per step; at a
    // pair or two per expert the per-wave reads cost less, Scout decode down
    // 59.2 against 60.3 us)
    const int sliced = (ex4 && d.group_size == 128 && P >= 4 * d.E) ? 1 : 0;
    auto stream_up = [&](int max_chunks, int shared_chunks, hipStream_t st) {
        moe::DecodeArgs a{};
        a.sliced = sliced;
        a.T = d.T;
        a.P = P;
        a.top_k = d.top_k;
        a.E = static_cast<int>(d.E);
        a.perm = R.perm;
        a.chunks = R.chunks;
        a.nchunks = R.nchunks;
        a.a = x;
        a.a_perm = x_perm;
        a.K = d.d;
        a.N = d.h;
        a.spt = moe::kGroup / d.group_size;
        if (ex4) {
            a.wq0 = ex4->w1q;
            a.ws0 = ex4->w1s;
            a.wq1 = ex4->w3q;
            a.ws1 = ex4->w3s;
        } else if (ex8) {
            a.wf0 = ex8->w1q;
            a.wf1 = ex8->w3q;
            a.wfs0 = ex8->w1s;
            a.wfs1 = ex8->w3s;
            a.a8 = xq;
            a.a8s = sxq;
        } else {
            a.wb0 = exb->w1;
            a.wb1 = exb->w3;
        }
        a.sh0 = sh->s1;
        a.sh1 = sh->s3;
        a.h_out = H;
        return timed(MOE_STAGE_DECODE_UP, st, "decode up launch",
                     [&] { return moe::launch_decode_up(a, max_chunks, shared_chunks, st); });
    };
    auto stream_down = [&](int max_chunks, int shared_chunks, hipStream_t st) {
        moe::DecodeArgs a{};
        a.sliced = sliced;
        a.T = d.T;
        a.P = P;
        a.top_k = d.top_k;
        a.E = static_cast<int>(d.E);
        a.perm = R.perm;
        a.chunks = R.chunks;
        a.nchunks = R.nchunks;
        a.a = H;
        a.a_perm = H;  // routed rows of H were written interleaved by the streaming up projection
        a.K = d.h;
        a.N = d.d;
        a.spt = moe::kGroup / d.group_size;
        if (ex4) {
            a.wq0 = ex4->w2q;
            a.ws0 = ex4->w2s;
        } else if (ex8) {
            a.wf0 = ex8->w2q;
            a.wfs0 = ex8->w2s;
            a.a8 = hq;
            a.a8s = shq;
        } else {
            a.wb0 = exb->w2;
        }
        a.sh0 = sh->s2;
        a.o_out = O;
        a.o_out2 = st == s ? O2 : nullptr;  // never on the hybrid path's side stream
        return timed(MOE_STAGE_DECODE_DOWN, st, "decode down launch",
                     [&] { return moe::launch_decode_down(a, max_chunks, shared_chunks, st); });
    };
    // hybrid: at most min(E, P) small experts of at most two 16-row chunks each
    const int64_t hybrid_chunks =
        (d.E < P ? d.E : P) * ((kHybridRows + moe::kDecodeRows - 1) / moe::kDecodeRows);

    if (decode) {
        // bf16 chunks are split four ways: the shared expert's, at the head of
        // the list, or every chunk when the routed experts are bf16
        const int split = exb ? L.max_chunks
                              : static_cast<int>((d.T + moe::kDecodeRows - 1) / moe::kDecodeRows);
        CHECK(stream_up(L.max_chunks, split, s));
        if (ex8) CHECK(quantize_h());
        CHECK(stream_down(L.max_chunks, split, s));
    } else {
        moe::GroupedGemmArgs g{};
        g.T = d.T;
        g.P = P;
        g.top_k = d.top_k;
        g.E = static_cast<int>(d.E);
        g.perm = R.perm;
        g.offsets = R.offsets;
        g.counts = R.counts;
        g.tile_base = R.tile_base;
        // XCD split (time of a routed tile in eighths of a shared bf16 tile,
        // measured on the Scout and Maverick prefill layers): int4 tiles
        // dequantize their weights, fp8 256-row tiles run the 128-deep fp8
        // instruction; in the hybrid path the GEMMs share the chip with the
        // streaming kernels and equal counts balance best
        g.routed_weight = hybrid ? 8 : ex4 ? 10 : (ex8 && wide) ? 6 : 8;

        g.a = x;
        g.K = d.d;
        g.N = d.h;
        g.spt = moe::kGroup / d.group_size;
        if (ex4) {
            g.wq0 = ex4->w1q;
            g.ws0 = ex4->w1s;
            g.wq1 = ex4->w3q;
            g.ws1 = ex4->w3s;
        } else if (ex8) {
            g.wf0 = ex8->w1q;
            g.wf1 = ex8->w3q;
            g.wfs0 = ex8->w1s;
            g.wfs1 = ex8->w3s;
            g.a8 = xq;
            g.a8s = sxq;
        } else {
            g.wb0 = exb->w1;
            g.wb1 = exb->w3;
        }
        g.sh0 = sh->s1;
        g.sh1 = sh->s3;
        g.h_out = H;
        // hybrid: the small experts' streaming kernels (HBM-bound) run on the
        // side stream beside the grouped GEMMs (MFMA-bound); the two chains
        // touch disjoint rows of H and O. fp8 experts quantize all routed H
        // rows in one step between the two projections, which joins them there.
        const int hsplit = exb ? static_cast<int>(hybrid_chunks) : 0;
        const int hch = static_cast<int>(hybrid_chunks);
        Side* side = nullptr;
        std::unique_lock<std::mutex> side_lock;
        if (hybrid) {
            CHECK(side_stream(&side));
            side_lock = std::unique_lock<std::mutex>(side->mu);
            HIP_CHECK(hipEventRecord(side->fork, s), "hipEventRecord");
            HIP_CHECK(hipStreamWaitEvent(side->stream, side->fork, 0), "hipStreamWaitEvent");
            CHECK(stream_up(hch, hsplit, side->stream));
            if (ex8) {
                HIP_CHECK(hipEventRecord(side->mid, side->stream), "hipEventRecord");
            } else {
                CHECK(stream_down(hch, hsplit, side->stream));
            }
        }
        // hybrid: the large routed experts on 128-row tiles, then the shared
        // expert alone on 256-row tiles (a plain bf16 GEMM over every token,
        // which the 256-row kernel runs faster)
        auto grouped = [&](bool up) {
            if (!hybrid) {
                g.tile_mode = moe::kTilesAll;
                return wide ? (up ? moe::launch_grouped_up256(g, s) : moe::launch_grouped_down256(g, s))
                            : (up ? moe::launch_grouped_up(g, s) : moe::launch_grouped_down(g, s));
            }
            g.tile_mode = moe::kTilesRouted;
            hipError_t e = up ? moe::launch_grouped_up(g, s) : moe::launch_grouped_down(g, s);
            if (e != hipSuccess) return e;
            g.tile_mode = moe::kTilesShared;
            return up ? moe::launch_grouped_up256(g, s) : moe::launch_grouped_down256(g, s);
        };
        CHECK(timed(MOE_STAGE_UP, s, "grouped up launch", [&] { return grouped(true); }));
        if (ex8) {
            if (hybrid) HIP_CHECK(hipStreamWaitEvent(s, side->mid, 0), "hipStreamWaitEvent");
            CHECK(quantize_h());
            if (hybrid) {
                HIP_CHECK(hipEventRecord(side->quant, s), "hipEventRecord");
                HIP_CHECK(hipStreamWaitEvent(side->stream, side->quant, 0), "hipStreamWaitEvent");
                CHECK(stream_down(hch, hsplit, side->stream));
            }
        }

        g.a = H;
        g.K = d.h;
        g.N = d.d;
        g.wq0 = ex4 ? ex4->w2q : nullptr;
        g.ws0 = ex4 ? ex4->w2s : nullptr;
        g.wq1 = nullptr;
        g.ws1 = nullptr;
        g.wb0 = exb ? exb->w2 : nullptr;
        g.wb1 = nullptr;
        g.wf0 = ex8 ? ex8->w2q : nullptr;
        g.wf1 = nullptr;
        g.wfs0 = ex8 ? ex8->w2s : nullptr;
        g.wfs1 = nullptr;
        g.a8 = hq;
        g.a8s = shq;
        g.sh0 = sh->s2;
        g.sh1 = nullptr;
        g.h_out = nullptr;
        g.o_out = O;
        CHECK(timed(MOE_STAGE_DOWN, s, "grouped down launch", [&] { return grouped(false); }));
        if (hybrid) {
            HIP_CHECK(hipEventRecord(side->join, side->stream), "hipEventRecord");
            HIP_CHECK(hipStreamWaitEvent(s, side->join, 0), "hipStreamWaitEvent");
        }
    }

    CHECK(timed(MOE_STAGE_COMBINE, s, "combine launch", [&] {
        return moe::launch_combine(O, decode ? O2 : nullptr, R.gates, R.inv, d.T, P, d.top_k, d.d, y, s);
    }));
    return MOE_OK;
}

int moe_forward_path(const moe_dims* dims, const uint16_t* x, const float* router_w,
                     const float* router_b, const moe_experts_int4* experts,
                     const moe_shared_bf16* shared, uint16_t* y, int32_t* topk_ids,
                     float* topk_gates, int32_t path, void* workspace, size_t workspace_bytes,
                     void* stream) {
    if (!experts) {
        g_last_error.clear();
        return fail(MOE_ERR_INVALID_ARG, "experts is NULL");
    }
    return forward_impl(dims, x, router_w, router_b, experts, nullptr, nullptr, shared, y, topk_ids,
                        topk_gates, path, workspace, workspace_bytes, stream);
}

int moe_forward_bf16(const moe_dims* dims, const uint16_t* x, const float* router_w,
                     const float* router_b, const moe_experts_bf16* experts,
                     const moe_shared_bf16* shared, uint16_t* y, int32_t* topk_ids,
                     float* topk_gates, int32_t path, void* workspace, size_t workspace_bytes,
                     void* stream) {
    if (!experts) {
        g_last_error.clear();
        return fail(MOE_ERR_INVALID_ARG, "experts is NULL");
    }
    return forward_impl(dims, x, router_w, router_b, nullptr, experts, nullptr, shared, y, topk_ids,
                        topk_gates, path, workspace, workspace_bytes, stream);
}

size_t moe_forward_fp8_workspace_bytes(const moe_dims* dims) {
    const std::string saved = g_last_error;
    if (check_dims(dims) != MOE_OK) return 0;
    g_last_error = saved;
    return layout(*dims).total_fp8;
}

int moe_forward_fp8(const moe_dims* dims, const uint16_t* x, const float* router_w,
                    const float* router_b, const moe_experts_fp8* experts,
                    const moe_shared_bf16* shared, uint16_t* y, int32_t* topk_ids,
                    float* topk_gates, int32_t path, void* workspace, size_t workspace_bytes,
                    void* stream) {
    if (!experts) {
        g_last_error.clear();
        return fail(MOE_ERR_INVALID_ARG, "experts is NULL");
    }
    return forward_impl(dims, x, router_w, router_b, nullptr, nullptr, experts, shared, y, topk_ids,
                        topk_gates, path, workspace, workspace_bytes, stream);
}

int moe_forward(const moe_dims* dims, const uint16_t* x, const float* router_w,
                const float* router_b, const moe_experts_int4* experts,
                const moe_shared_bf16* shared, uint16_t* y, int32_t* topk_ids, float* topk_gates,
                void* workspace, size_t workspace_bytes, void* stream) {
    return moe_forward_path(dims, x, router_w, router_b, experts, shared, y, topk_ids, topk_gates,
                            MOE_PATH_AUTO, workspace, workspace_bytes, stream);
}

int moe_forward_noalloc(const moe_dims* dims, const uint16_t* x, const float* router_w,
                        const float* router_b, const moe_experts_int4* experts,
                        const moe_shared_bf16* shared, uint16_t* y, int32_t* topk_ids,
                        float* topk_gates, int32_t path, void* stream) {
    g_last_error.clear();
    CHECK(check_dims(dims));
    if (!experts) return fail(MOE_ERR_INVALID_ARG, "experts is NULL");
    const size_t need = layout(*dims).total;
    if (need > kScratchBytes)
        return fail(MOE_ERR_WORKSPACE,
                    "the layer needs %zu bytes of workspace; the allocation-free forward has %zu "
                    "(MOE_NOALLOC_SCRATCH_BYTES): use moe_forward_path with a workspace",
                    need, kScratchBytes);
    CHECK(device_ok());
    void* ws = nullptr;
    CHECK(scratch_address(&ws));
    return forward_impl(dims, x, router_w, router_b, experts, nullptr, nullptr, shared, y, topk_ids,
                        topk_gates, path, ws, kScratchBytes, stream);
}

static int stream_args(const void* a, const void* b, int64_t bytes) {
    if (!a || !b) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) % 16)
        return fail(MOE_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    if (bytes <= 0 || bytes % 16)
        return fail(MOE_ERR_INVALID_ARG, "bytes = %lld must be a positive multiple of 16", (long long)bytes);
    return MOE_OK;
}

int moe_hbm_read_sink_words(void) { return moe::kStreamBlocks; }

int moe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    g_last_error.clear();
    CHECK(device_ok());
    CHECK(stream_args(buf, sink, bytes));
    HIP_CHECK(moe::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream)), "read launch");
    return MOE_OK;
}

int moe_hbm_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    g_last_error.clear();
    CHECK(device_ok());
    CHECK(stream_args(dst, src, bytes));
    HIP_CHECK(moe::launch_stream_copy(dst, src, bytes, static_cast<hipStream_t>(stream)), "copy launch");
    return MOE_OK;
}

int moe_profile_enable(int on) {
    Prof& P = prof();
    std::lock_guard<std::mutex> lock(P.mu);
    P.on = on != 0;
    return MOE_OK;
}

int moe_profile_read(double* ms, int64_t* launches, int n) {
    g_last_error.clear();
    if (n < 0 || n > MOE_STAGE_COUNT) return fail(MOE_ERR_INVALID_ARG, "n = %d outside [0, %d]", n, MOE_STAGE_COUNT);
    Prof& P = prof();
    std::lock_guard<std::mutex> lock(P.mu);
    for (const Prof::Rec& r : P.pending) {
        HIP_CHECK(hipEventSynchronize(r.b), "hipEventSynchronize");
        float t = 0.f;
        HIP_CHECK(hipEventElapsedTime(&t, r.a, r.b), "hipEventElapsedTime");
        P.ms[r.stage] += t;
        P.n[r.stage] += 1;
        P.pool.push_back(r.a);
        P.pool.push_back(r.b);
    }
    P.pending.clear();
    for (int i = 0; i < n; ++i) {
        if (ms) ms[i] = P.ms[i];
        if (launches) launches[i] = P.n[i];
    }
    for (int i = 0; i < MOE_STAGE_COUNT; ++i) {
        P.ms[i] = 0.0;
        P.n[i] = 0;
    }
    return MOE_OK;
}

const char* moe_stage_name(int stage) {
    static const char* names[MOE_STAGE_COUNT] = {"router", "topk", "dispatch", "grouped_up",
                                                 "grouped_down", "combine", "decode_up", "decode_down",
                                                 "act_quant", "quantize"};
    return (stage >= 0 && stage < MOE_STAGE_COUNT) ? names[stage] : "unknown";
}

}  // extern "C"
