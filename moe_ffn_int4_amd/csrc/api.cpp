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

#include "kernels.h"

static_assert(MOE_MAX_EXPERTS == moe::kMaxExperts, "expert limit mismatch");
static_assert(MOE_GROUP_SIZE == moe::kGroup, "group size mismatch");

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

// Workspace sections (byte offsets from the workspace base).
struct Layout {
    size_t logits, ids, gates, counts, offsets, tile_base, perm, inv, routing_end, H, O, total;
};

Layout layout(const moe_dims& d) {
    const size_t T = d.T, E = d.E, P = static_cast<size_t>(d.T) * d.top_k;
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += round_up(bytes);
        return at;
    };
    L.logits = take(T * E * 4);
    L.ids = take(P * 4);
    L.gates = take(P * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.tile_base = take((E + 2) * 4);
    L.perm = take(P * 4);
    L.inv = take(P * 4);
    L.routing_end = off;
    L.H = take((P + T) * static_cast<size_t>(d.h) * 2);
    L.O = take((P + T) * static_cast<size_t>(d.d) * 4);
    L.total = off;
    return L;
}

int check_dims(const moe_dims* d) {
    if (!d) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
    if (d->group_size != MOE_GROUP_SIZE)
        return fail(MOE_ERR_INVALID_ARG, "group_size %d unsupported (only %d)", d->group_size,
                    MOE_GROUP_SIZE);
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
                       bool routing_only = false) {
    CHECK(check_dims(dims));
    CHECK(check_ptr(x, "x"));
    CHECK(check_ptr(router_w, "router_w"));
    if (router_b) CHECK(check_ptr(router_b, "router_b", 4));
    if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, kAlign)) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    const Layout L = layout(*dims);
    const size_t need = routing_only ? L.routing_end : L.total;
    if (workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    return MOE_OK;
}

struct Routing {
    float* logits;
    int32_t* ids;
    float* gates;
    int32_t* counts;
    int32_t* offsets;
    int32_t* tile_base;
    int32_t* perm;
    int32_t* inv;
};

Routing carve(const moe_dims& d, void* ws) {
    const Layout L = layout(d);
    char* b = static_cast<char*>(ws);
    return Routing{reinterpret_cast<float*>(b + L.logits),   reinterpret_cast<int32_t*>(b + L.ids),
                   reinterpret_cast<float*>(b + L.gates),    reinterpret_cast<int32_t*>(b + L.counts),
                   reinterpret_cast<int32_t*>(b + L.offsets), reinterpret_cast<int32_t*>(b + L.tile_base),
                   reinterpret_cast<int32_t*>(b + L.perm),   reinterpret_cast<int32_t*>(b + L.inv)};
}

int run_routing(const moe_dims& d, const uint16_t* x, const float* wr, const float* b,
                const Routing& R, int32_t* ids_out, float* gates_out, hipStream_t s) {
    HIP_CHECK(moe::launch_router_logits(x, wr, b, d.T, d.d, d.E, R.logits, s), "router launch");
    HIP_CHECK(moe::launch_topk(R.logits, d.T, d.E, d.top_k, R.ids, R.gates, ids_out, gates_out, s),
              "top-k launch");
    HIP_CHECK(moe::launch_dispatch(R.ids, d.T, d.top_k, d.E, moe::kPrefillBM, R.counts, R.offsets,
                                   R.tile_base, R.perm, R.inv, s),
              "dispatch launch");
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

int moe_quantize_int4(const float* w, int64_t rows, int64_t K, int32_t group_size, uint8_t* q,
                      float* scales, void* stream) {
    g_last_error.clear();
    if (group_size != MOE_GROUP_SIZE)
        return fail(MOE_ERR_INVALID_ARG, "group_size %d unsupported (only %d)", group_size,
                    MOE_GROUP_SIZE);
    if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows = %lld is negative", (long long)rows);
    if (K < group_size || K % group_size)
        return fail(MOE_ERR_INVALID_ARG, "K = %lld must be a positive multiple of %d", (long long)K,
                    group_size);
    if (rows == 0) return MOE_OK;
    CHECK(check_ptr(w, "w"));
    CHECK(check_ptr(q, "q", 2));
    CHECK(check_ptr(scales, "scales", 4));
    CHECK(device_ok());
    HIP_CHECK(moe::launch_quantize_int4(w, rows, K, q, scales, static_cast<hipStream_t>(stream)),
              "quantize launch");
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
    CHECK(run_routing(d, x, router_w, router_b, R, topk_ids, topk_gates, s));
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

int moe_forward_path(const moe_dims* dims, const uint16_t* x, const float* router_w,
                     const float* router_b, const moe_experts_int4* ex, const moe_shared_bf16* sh,
                     uint16_t* y, int32_t* topk_ids, float* topk_gates, int32_t path,
                     void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    CHECK(check_forward_args(dims, x, router_w, router_b, workspace, workspace_bytes));
    if (!ex) return fail(MOE_ERR_INVALID_ARG, "experts is NULL");
    if (!sh) return fail(MOE_ERR_INVALID_ARG, "shared is NULL");
    CHECK(check_ptr(ex->w1q, "experts->w1q"));
    CHECK(check_ptr(ex->w3q, "experts->w3q"));
    CHECK(check_ptr(ex->w2q, "experts->w2q"));
    CHECK(check_ptr(ex->w1s, "experts->w1s", 4));
    CHECK(check_ptr(ex->w3s, "experts->w3s", 4));
    CHECK(check_ptr(ex->w2s, "experts->w2s", 4));
    CHECK(check_ptr(sh->s1, "shared->s1"));
    CHECK(check_ptr(sh->s3, "shared->s3"));
    CHECK(check_ptr(sh->s2, "shared->s2"));
    CHECK(check_ptr(y, "y"));
    if (topk_ids) CHECK(check_ptr(topk_ids, "topk_ids", 4));
    if (topk_gates) CHECK(check_ptr(topk_gates, "topk_gates", 4));
    if (path != MOE_PATH_AUTO && path != MOE_PATH_PREFILL && path != MOE_PATH_DECODE)
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

    CHECK(run_routing(d, x, router_w, router_b, R, topk_ids, topk_gates, s));

    moe::GroupedGemmArgs g{};
    g.T = d.T;
    g.P = P;
    g.top_k = d.top_k;
    g.E = static_cast<int>(d.E);
    g.perm = R.perm;
    g.offsets = R.offsets;
    g.counts = R.counts;
    g.tile_base = R.tile_base;

    g.a = x;
    g.K = d.d;
    g.N = d.h;
    g.wq0 = ex->w1q;
    g.ws0 = ex->w1s;
    g.wq1 = ex->w3q;
    g.ws1 = ex->w3s;
    g.sh0 = sh->s1;
    g.sh1 = sh->s3;
    g.h_out = H;
    HIP_CHECK(moe::launch_grouped_up(g, s), "grouped up launch");

    g.a = H;
    g.K = d.h;
    g.N = d.d;
    g.wq0 = ex->w2q;
    g.ws0 = ex->w2s;
    g.wq1 = nullptr;
    g.ws1 = nullptr;
    g.sh0 = sh->s2;
    g.sh1 = nullptr;
    g.h_out = nullptr;
    g.o_out = O;
    HIP_CHECK(moe::launch_grouped_down(g, s), "grouped down launch");

    HIP_CHECK(moe::launch_combine(O, R.gates, R.inv, d.T, P, d.top_k, d.d, y, s), "combine launch");
    return MOE_OK;
}

int moe_forward(const moe_dims* dims, const uint16_t* x, const float* router_w,
                const float* router_b, const moe_experts_int4* experts,
                const moe_shared_bf16* shared, uint16_t* y, int32_t* topk_ids, float* topk_gates,
                void* workspace, size_t workspace_bytes, void* stream) {
    return moe_forward_path(dims, x, router_w, router_b, experts, shared, y, topk_ids, topk_gates,
                            MOE_PATH_AUTO, workspace, workspace_bytes, stream);
}

}  // extern "C"
