// fk_api.hip -- host side of the C ABI declared in include/fk.h: argument
// checks (before anything is enqueued), workspace layout and kernel sequence
// of each entry point.  No device memory is allocated here; the one static
// array (the scratch of fk_update_bias_noalloc) comes with the code object.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "fk_internal.h"

namespace fk {
hipError_t launch_assign_f16(const void*, const void*, const float*, int32_t*, float*, int64_t,
                             int64_t, int64_t, int, hipStream_t);
hipError_t launch_assign_bf16(const void*, const void*, const float*, int32_t*, float*, int64_t,
                              int64_t, int64_t, int, hipStream_t);
hipError_t launch_assign_f32(const void*, const void*, const float*, int32_t*, float*, int64_t,
                             int64_t, int64_t, int, hipStream_t);

hipError_t launch_assign(int dtype, const void* X, const void* C, const float* bias,
                         int32_t* labels, float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                         hipStream_t s) {
    switch (dtype) {
        case FK_F16: return launch_assign_f16(X, C, bias, labels, min_dist, B, N, K, d, s);
        case FK_BF16: return launch_assign_bf16(X, C, bias, labels, min_dist, B, N, K, d, s);
        default: return launch_assign_f32(X, C, bias, labels, min_dist, B, N, K, d, s);
    }
}

hipError_t launch_scores_f16(const void*, const void*, const float*, float*, int64_t, int64_t,
                             int64_t, int, hipStream_t);
hipError_t launch_scores_bf16(const void*, const void*, const float*, float*, int64_t, int64_t,
                              int64_t, int, hipStream_t);

hipError_t launch_scores(int dtype, const void* X, const void* C, const float* bias, float* D,
                         int64_t B, int64_t N, int64_t K, int d, hipStream_t s) {
    return dtype == FK_F16 ? launch_scores_f16(X, C, bias, D, B, N, K, d, s)
                           : launch_scores_bf16(X, C, bias, D, B, N, K, d, s);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Workspace workspace_layout(const fk_problem& p, char* base) {
    Workspace w{};
    size_t o = 0;
    auto take = [&](size_t bytes) -> char* {
        char* at = base ? base + o : nullptr;
        o = align256(o + bytes);
        return at;
    };
    const size_t B = (size_t)p.B, N = (size_t)p.N, K = (size_t)p.K, d = (size_t)p.d;
    const size_t tab = (size_t)sort_table_bound(p.N, p.K);
    w.bias = reinterpret_cast<float*>(take(B * K * sizeof(float)));
    w.offsets = reinterpret_cast<int32_t*>(take(B * (K + 1) * sizeof(int32_t)));
    w.table = reinterpret_cast<int32_t*>(take(B * tab * sizeof(int32_t)));
    w.radix = reinterpret_cast<int32_t*>(
        take(B * (size_t)radix_pairs_bound(p.N, p.K) * sizeof(int32_t)));
    w.nvalid = reinterpret_cast<int32_t*>(take(B * sizeof(int32_t)));
    w.sorted_idx = reinterpret_cast<int32_t*>(take(B * N * sizeof(int32_t)));
    w.poff = reinterpret_cast<int32_t*>(take(B * (K + 1) * sizeof(int32_t)));
    w.pieces = reinterpret_cast<int32_t*>(
        take(B * (1 + 2 * (size_t)piece_capacity(p.N, p.K)) * sizeof(int32_t)));
    w.part = reinterpret_cast<int32_t*>(take(B * 2 * (size_t)plan_blocks(p.K) * sizeof(int32_t)));
    w.sums = reinterpret_cast<float*>(take(B * K * d * sizeof(float)));
    w.arrive = reinterpret_cast<int32_t*>(take(B * K * sizeof(int32_t)));
    w.counts = reinterpret_cast<int32_t*>(take(B * K * sizeof(int32_t)));
    w.lowp = p.dtype == FK_F32 ? nullptr : take(B * K * d * (size_t)dtype_size(p.dtype));
    w.bad = reinterpret_cast<int32_t*>(take(B * sizeof(int32_t)));
    w.flags = reinterpret_cast<uint32_t*>(take(256));
    w.psums = (p.flags & FK_DETERMINISTIC)
                  ? reinterpret_cast<float*>(
                        take(B * (size_t)piece_capacity(p.N, p.K) * d * sizeof(float)))
                  : nullptr;
    w.total = o;
    return w;
}

StreamWorkspace stream_workspace_layout(const fk_problem& p, int64_t chunk, char* base) {
    StreamWorkspace w{};
    size_t o = 0;
    auto take = [&](size_t bytes) -> char* {
        char* at = base ? base + o : nullptr;
        o = align256(o + bytes);
        return at;
    };
    const size_t B = (size_t)p.B, K = (size_t)p.K, d = (size_t)p.d, c = (size_t)chunk;
    const size_t es = (size_t)dtype_size(p.dtype);
    w.xbuf[0] = take(c * d * es);
    w.xbuf[1] = take(c * d * es);
    w.bias = reinterpret_cast<float*>(take(B * K * sizeof(float)));
    w.lowp = p.dtype == FK_F32 ? nullptr : take(B * K * d * es);
    w.sums = reinterpret_cast<float*>(take(B * K * d * sizeof(float)));
    w.ccounts = reinterpret_cast<int32_t*>(take(K * sizeof(int32_t)));
    w.offsets = reinterpret_cast<int32_t*>(take((K + 1) * sizeof(int32_t)));
    w.table = reinterpret_cast<int32_t*>(take((size_t)sort_table_bound(chunk, p.K) * sizeof(int32_t)));
    w.radix = reinterpret_cast<int32_t*>(
        take((size_t)radix_pairs_bound(chunk, p.K) * sizeof(int32_t)));
    w.nvalid = reinterpret_cast<int32_t*>(take(256));
    w.sorted_idx = reinterpret_cast<int32_t*>(take(c * sizeof(int32_t)));
    w.poff = reinterpret_cast<int32_t*>(take((K + 1) * sizeof(int32_t)));
    w.pieces = reinterpret_cast<int32_t*>(
        take((1 + 2 * (size_t)piece_capacity(chunk, p.K)) * sizeof(int32_t)));
    w.part = reinterpret_cast<int32_t*>(take(2 * (size_t)plan_blocks(p.K) * sizeof(int32_t)));
    w.bad = reinterpret_cast<int32_t*>(take(256));
    if (p.flags & FK_DETERMINISTIC) {
        w.csums = reinterpret_cast<float*>(take(K * d * sizeof(float)));
        w.psums = reinterpret_cast<float*>(
            take((size_t)piece_capacity(chunk, p.K) * d * sizeof(float)));
    }
    w.total = o;
    return w;
}

}  // namespace fk

namespace {

using namespace fk;

thread_local char g_err[512] = "";

fk_status fail(fk_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

fk_status hip_fail(hipError_t e, const char* what) {
    return fail(FK_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

#define FK_TRY(call, what)                            \
    do {                                              \
        hipError_t fk_e_ = (call);                    \
        if (fk_e_ != hipSuccess) return hip_fail(fk_e_, what); \
    } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxIndex = 2147483646;  // N and K must leave room for N + 1 / K + 1 in int32
constexpr int64_t kMaxD = 65536;


fk_status check_problem(const fk_problem* p) {
    if (!p) return fail(FK_EINVAL, "problem is NULL");
    if (p->B < 1 || p->N < 1 || p->K < 1 || p->d < 1)
        return fail(FK_EINVAL, "sizes must be >= 1 (B=%lld N=%lld K=%lld d=%lld)", (long long)p->B,
                    (long long)p->N, (long long)p->K, (long long)p->d);
    if (p->dtype != FK_F32 && p->dtype != FK_F16 && p->dtype != FK_BF16)
        return fail(FK_EUNSUPPORTED, "unknown dtype %d", (int)p->dtype);
    if (p->flags & ~FK_DETERMINISTIC) return fail(FK_EINVAL, "unknown flag bits 0x%x", (unsigned)p->flags);
    if (p->N > kMaxIndex || p->K > kMaxIndex)
        return fail(FK_EUNSUPPORTED, "N and K must be <= %lld", (long long)kMaxIndex);
    if (p->d > kMaxD) return fail(FK_EUNSUPPORTED, "d must be <= %lld", (long long)kMaxD);
    if (p->B > 65535) return fail(FK_EUNSUPPORTED, "B must be <= 65535");
    return FK_OK;
}

fk_status check_ptr(const void* ptr, const char* name, bool required = true) {
    if (!ptr) return required ? fail(FK_EINVAL, "%s is NULL", name) : FK_OK;
    if (!aligned16(ptr)) return fail(FK_EINVAL, "%s is not 16-byte aligned", name);
    return FK_OK;
}

fk_status check_ws(const fk_problem& p, void* ws, size_t ws_bytes, Workspace* out) {
    const Workspace need = workspace_layout(p, nullptr);
    if (!ws) return fail(FK_EWORKSPACE, "workspace is NULL");
    if (!aligned16(ws)) return fail(FK_EINVAL, "workspace is not 16-byte aligned");
    if (ws_bytes < need.total)
        return fail(FK_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need.total);
    *out = workspace_layout(p, static_cast<char*>(ws));
    return FK_OK;
}

fk_status check_assign_d(const fk_problem&) { return FK_OK; }

// FK_DETERMINISTIC: every argsort is stable; nothing to check beyond flags
fk_status check_deterministic(const fk_problem&) { return FK_OK; }

#define FK_CHECK(expr)                    \
    do {                                  \
        fk_status fk_s_ = (expr);         \
        if (fk_s_ != FK_OK) return fk_s_; \
    } while (0)

// Counting-sort argsort of the labels into counts, offsets, sorted_idx and
// the pieces of the segment sums; with clear_update the sum rows and arrival
// counters a fused update accumulates into are cleared on the way, and a
// non-null move word is cleared.
fk_status enqueue_sort(const fk_problem& p, const Workspace& w, const int32_t* labels,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_idx, bool clear_update,
                       uint32_t* move, hipStream_t s) {
    SortParams sp{};
    sp.labels = labels;
    sp.counts = counts;
    sp.offsets = offsets;
    sp.sorted_idx = sorted_idx;
    sp.poff = w.poff;
    sp.pieces = w.pieces;
    sp.part = w.part;
    sp.table = w.table;
    sp.radix = w.radix;
    sp.nvalid = w.nvalid;
    sp.bad = w.bad;
    sp.move = move;
    if (clear_update) {
        sp.sums = w.sums;
        sp.arrive = w.arrive;
        sp.d = p.d;
    }
    FK_TRY(launch_sort(sp, p.B, p.N, p.K, s), "sort labels");
    return FK_OK;
}

}  // namespace

extern "C" {

int fk_abi_version(void) { return FK_ABI_VERSION; }

const char* fk_status_str(int status) {
    switch (status) {
        case FK_OK: return "FK_OK";
        case FK_EINVAL: return "FK_EINVAL: invalid argument";
        case FK_EUNSUPPORTED: return "FK_EUNSUPPORTED: unsupported dtype or size";
        case FK_EWORKSPACE: return "FK_EWORKSPACE: workspace missing or too small";
        case FK_EHIP: return "FK_EHIP: HIP runtime or launch failure";
        case FK_EHOST: return "FK_EHOST: host resource failure";
        default: return "unknown fk_status";
    }
}

const char* fk_last_error(void) { return g_err; }

fk_status fk_workspace_size(const fk_problem* p, int64_t chunk_points, size_t* bytes) {
    FK_CHECK(check_problem(p));
    if (!bytes) return fail(FK_EINVAL, "bytes is NULL");
    if (chunk_points < 0) return fail(FK_EINVAL, "chunk_points must be >= 0");
    if (chunk_points > kMaxIndex) return fail(FK_EUNSUPPORTED, "chunk_points too large");
    *bytes = chunk_points == 0
                 ? workspace_layout(*p, nullptr).total
                 : stream_workspace_layout(*p, chunk_points < p->N ? chunk_points : p->N, nullptr).total;
    return FK_OK;
}

size_t fk_workspace_bytes(const fk_problem* p, int64_t chunk_points) {
    size_t bytes = 0;
    return fk_workspace_size(p, chunk_points, &bytes) == FK_OK ? bytes : 0;
}

fk_status fk_centroid_bias(const fk_problem* p, const void* C, float* bias, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(C, "C"));
    FK_CHECK(check_ptr(bias, "bias"));
    hipStream_t s = static_cast<hipStream_t>(stream);
    FK_TRY(launch_centroid_bias(p->dtype, C, bias, p->B * p->K, (int)p->d, s), "centroid bias");
    return FK_OK;
}

fk_status fk_assign(const fk_problem* p, const void* X, const void* C, int32_t* labels,
                    float* min_dist, void* ws, size_t ws_bytes, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(X, "X"));
    FK_CHECK(check_ptr(C, "C"));
    FK_CHECK(check_ptr(labels, "labels"));
    FK_CHECK(check_ptr(min_dist, "min_dist", false));
    FK_CHECK(check_assign_d(*p));
    Workspace w;
    FK_CHECK(check_ws(*p, ws, ws_bytes, &w));
    hipStream_t s = static_cast<hipStream_t>(stream);
    FK_TRY(launch_centroid_bias(p->dtype, C, w.bias, p->B * p->K, (int)p->d, s), "centroid bias");
    FK_TRY(launch_assign(p->dtype, X, C, w.bias, labels, min_dist, p->B, p->N, p->K, (int)p->d, s),
           "assign");
    return FK_OK;
}

fk_status fk_assign_with_bias(const fk_problem* p, const void* X, const void* C,
                              const float* bias, int32_t* labels, float* min_dist, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(X, "X"));
    FK_CHECK(check_ptr(C, "C"));
    FK_CHECK(check_ptr(bias, "bias"));
    FK_CHECK(check_ptr(labels, "labels"));
    FK_CHECK(check_ptr(min_dist, "min_dist", false));
    FK_CHECK(check_assign_d(*p));
    hipStream_t s = static_cast<hipStream_t>(stream);
    FK_TRY(launch_assign(p->dtype, X, C, bias, labels, min_dist, p->B, p->N, p->K, (int)p->d, s),
           "assign");
    return FK_OK;
}

fk_status fk_sort_labels(const fk_problem* p, const int32_t* labels, int32_t* counts,
                         int32_t* offsets, int32_t* sorted_idx, void* ws, size_t ws_bytes,
                         void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(labels, "labels"));
    FK_CHECK(check_ptr(counts, "counts"));
    FK_CHECK(check_ptr(offsets, "offsets"));
    FK_CHECK(check_ptr(sorted_idx, "sorted_idx"));
    FK_CHECK(check_deterministic(*p));
    Workspace w;
    FK_CHECK(check_ws(*p, ws, ws_bytes, &w));
    hipStream_t s = static_cast<hipStream_t>(stream);
    return enqueue_sort(*p, w, labels, counts, offsets, sorted_idx, false, nullptr, s);
}

}  // extern "C"

namespace {
// Checks shared by the update entry points (everything but the workspace).
fk_status check_update(const fk_problem* p, const void* X, const int32_t* labels,
                       const float* C_prev, const float* C_next, const void* C_next_lowp,
                       const int32_t* counts) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(X, "X"));
    FK_CHECK(check_ptr(labels, "labels"));
    FK_CHECK(check_ptr(C_prev, "C_prev"));
    FK_CHECK(check_ptr(C_next, "C_next"));
    FK_CHECK(check_ptr(C_next_lowp, "C_next_lowp", false));
    FK_CHECK(check_ptr(counts, "counts"));
    if (p->dtype == FK_F32 && C_next_lowp && C_next_lowp == static_cast<const void*>(C_next))
        return fail(FK_EINVAL, "C_next_lowp must differ from C_next");
    if (p->d > 1024) return fail(FK_EUNSUPPORTED, "update supports d <= 1024");
    FK_CHECK(check_deterministic(*p));
    return FK_OK;
}

// The update's kernels (argsort, segment sums and finalize) on workspace w.
fk_status enqueue_update(const fk_problem* p, const Workspace& w, const void* X,
                         const int32_t* labels, const float* C_prev, float* C_next,
                         void* C_next_lowp, int32_t* counts, float* bias_next, hipStream_t s) {
    const int64_t rows = p->B * p->K;
    FK_CHECK(enqueue_sort(*p, w, labels, counts, w.offsets, w.sorted_idx, true, nullptr, s));
    SegParams sp{true,    w.sums,  w.arrive, C_prev, C_next,
                 p->dtype == FK_F32 ? nullptr : C_next_lowp, bias_next, nullptr, w.psums, w.poff};
    FK_TRY(launch_segment_sums(p->dtype, X, w.sorted_idx, w.offsets, w.pieces, sp, p->B, p->N,
                               p->K, (int)p->d, s),
           "segment sums");
    if (p->dtype == FK_F32 && C_next_lowp)
        FK_TRY(hipMemcpyAsync(C_next_lowp, C_next, (size_t)(rows * p->d) * sizeof(float),
                              hipMemcpyDeviceToDevice, s),
               "copy fp32 centroids");
    return FK_OK;
}

fk_status update_impl(const fk_problem* p, const void* X, const int32_t* labels,
                      const float* C_prev, float* C_next, void* C_next_lowp, int32_t* counts,
                      float* bias_next, void* ws, size_t ws_bytes, void* stream) {
    FK_CHECK(check_update(p, X, labels, C_prev, C_next, C_next_lowp, counts));
    Workspace w;
    FK_CHECK(check_ws(*p, ws, ws_bytes, &w));
    return enqueue_update(p, w, X, labels, C_prev, C_next, C_next_lowp, counts, bias_next,
                          static_cast<hipStream_t>(stream));
}

// Scratch of fk_update_bias_noalloc: part of the library's code object, so
// every GPU the library runs on holds its own copy, at its own address, from
// the library's load on that device until the process ends.  The array's
// name is a host-side stand-in: host code uses only the device address that
// hipGetSymbolAddress returns for the device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[FK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the device of stream s (the
// current device for the null stream), looked up on the first call for that
// device with that device current and kept for the process.
fk_status scratch_address(hipStream_t s, void** out) {
    int cur = 0, dev = 0;
    FK_TRY(hipGetDevice(&cur), "current device");
    dev = cur;
    if (s) FK_TRY(hipStreamGetDevice(s, &dev), "device of the stream");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(FK_EUNSUPPORTED, "device %d: static scratch is kept for devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur) FK_TRY(hipSetDevice(dev), "select the stream's device");
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess && r != hipSuccess) return hip_fail(r, "restore the current device");
        }
        if (e != hipSuccess) return hip_fail(e, "address of the static scratch");
        if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u))
            return fail(FK_EHIP, "static scratch at %p is not 256-byte aligned", ptr);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FK_OK;
}
}  // namespace

extern "C" {

fk_status fk_update(const fk_problem* p, const void* X, const int32_t* labels,
                    const float* C_prev, float* C_next, void* C_next_lowp, int32_t* counts,
                    void* ws, size_t ws_bytes, void* stream) {
    return update_impl(p, X, labels, C_prev, C_next, C_next_lowp, counts, nullptr, ws, ws_bytes,
                       stream);
}

fk_status fk_update_bias(const fk_problem* p, const void* X, const int32_t* labels,
                         const float* C_prev, float* C_next, void* C_next_lowp, int32_t* counts,
                         float* bias_next, void* ws, size_t ws_bytes, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(bias_next, "bias_next"));
    return update_impl(p, X, labels, C_prev, C_next, C_next_lowp, counts, bias_next, ws, ws_bytes,
                       stream);
}

fk_status fk_update_bias_noalloc(const fk_problem* p, const void* X, const int32_t* labels,
                                 const float* C_prev, float* C_next, void* C_next_lowp,
                                 int32_t* counts, float* bias_next, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(bias_next, "bias_next"));
    FK_CHECK(check_update(p, X, labels, C_prev, C_next, C_next_lowp, counts));
    const size_t need = workspace_layout(*p, nullptr).total;
    if (need > (size_t)FK_NOALLOC_SCRATCH_BYTES)
        return fail(FK_EUNSUPPORTED,
                    "problem needs %zu bytes of scratch, the static scratch holds %zu "
                    "(use fk_update_bias with a workspace)",
                    need, (size_t)FK_NOALLOC_SCRATCH_BYTES);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ptr = nullptr;
    FK_CHECK(scratch_address(s, &ptr));
    const Workspace w = workspace_layout(*p, static_cast<char*>(ptr));
    return enqueue_update(p, w, X, labels, C_prev, C_next, C_next_lowp, counts, bias_next, s);
}

fk_status fk_lloyd(const fk_problem* p, const void* X, float* C, int32_t* labels,
                   int32_t* counts, int max_iters, float tol, int* n_iter, void* ws,
                   size_t ws_bytes, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(X, "X"));
    FK_CHECK(check_ptr(C, "C"));
    FK_CHECK(check_ptr(labels, "labels"));
    FK_CHECK(check_ptr(counts, "counts"));
    if (max_iters < 1) return fail(FK_EINVAL, "max_iters must be >= 1");
    if (!(tol >= 0.f)) return fail(FK_EINVAL, "tol must be >= 0");
    FK_CHECK(check_assign_d(*p));
    if (p->d > 1024) return fail(FK_EUNSUPPORTED, "update supports d <= 1024");
    FK_CHECK(check_deterministic(*p));
    Workspace w;
    FK_CHECK(check_ws(*p, ws, ws_bytes, &w));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t rows = p->B * p->K;
    const bool sync = tol > 0.f || n_iter != nullptr;
    const void* Cq = p->dtype == FK_F32 ? static_cast<const void*>(C) : w.lowp;

    FK_TRY(launch_prepare(p->dtype, C, w.lowp, w.bias, rows, (int)p->d, s), "prepare centroids");
    uint32_t* move = sync ? w.flags + 1 : nullptr;
    const SegParams sp{true, w.sums, w.arrive, C, C, w.lowp, w.bias, move, w.psums, w.poff};
    int it = 0;
    while (it < max_iters) {
        FK_TRY(launch_assign(p->dtype, X, Cq, w.bias, labels, nullptr, p->B, p->N, p->K,
                             (int)p->d, s),
               "assign");
        FK_CHECK(enqueue_sort(*p, w, labels, counts, w.offsets, w.sorted_idx, true, move, s));
        FK_TRY(launch_segment_sums(p->dtype, X, w.sorted_idx, w.offsets, w.pieces, sp, p->B,
                                   p->N, p->K, (int)p->d, s),
               "segment sums");
        ++it;
        if (sync) {
            uint32_t bits = 0;
            FK_TRY(hipMemcpyAsync(&bits, w.flags + 1, sizeof(bits), hipMemcpyDeviceToHost, s),
                   "read centroid move");
            FK_TRY(hipStreamSynchronize(s), "synchronise");
            float move;
            memcpy(&move, &bits, sizeof(move));
            if (tol > 0.f && move <= tol) break;
        }
    }
    if (n_iter) *n_iter = it;
    return FK_OK;
}

fk_status fk_lloyd_streamed(const fk_problem* p, const void* X_host, int64_t chunk_points,
                            float* C, int32_t* labels, int32_t* counts, int max_iters, void* ws,
                            size_t ws_bytes, void* compute_stream, void* copy_stream) {
    FK_CHECK(check_problem(p));
    if (!X_host) return fail(FK_EINVAL, "X_host is NULL");
    FK_CHECK(check_ptr(C, "C"));
    FK_CHECK(check_ptr(labels, "labels"));
    FK_CHECK(check_ptr(counts, "counts"));
    if (chunk_points < 1) return fail(FK_EINVAL, "chunk_points must be >= 1");
    if (chunk_points > kMaxIndex) return fail(FK_EUNSUPPORTED, "chunk_points too large");
    if (max_iters < 1) return fail(FK_EINVAL, "max_iters must be >= 1");
    if (p->d > 1024) return fail(FK_EUNSUPPORTED, "update supports d <= 1024");
    const int64_t chunk = chunk_points < p->N ? chunk_points : p->N;
    const StreamWorkspace need = stream_workspace_layout(*p, chunk, nullptr);
    if (!ws) return fail(FK_EWORKSPACE, "workspace is NULL");
    if (!aligned16(ws)) return fail(FK_EINVAL, "workspace is not 16-byte aligned");
    if (ws_bytes < need.total)
        return fail(FK_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need.total);
    // the source must be pinned host memory for asynchronous copies
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, X_host) != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(FK_EINVAL, "X_host must be pinned host memory (hipHostMalloc)");
    }
    const StreamWorkspace w = stream_workspace_layout(*p, chunk, static_cast<char*>(ws));
    hipStream_t cs = static_cast<hipStream_t>(compute_stream);
    hipStream_t xs = static_cast<hipStream_t>(copy_stream);
    const int64_t B = p->B, N = p->N, K = p->K, d = p->d;
    const int64_t rows = B * K;
    const size_t es = (size_t)dtype_size(p->dtype);
    const int64_t nchunk = (N + chunk - 1) / chunk;

    hipEvent_t copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
    fk_status st = FK_OK;
    for (int i = 0; i < 2 && st == FK_OK; ++i) {
        if (hipEventCreateWithFlags(&copied[i], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&done[i], hipEventDisableTiming) != hipSuccess)
            st = fail(FK_EHOST, "cannot create events");
    }
    // the copy stream starts after everything already queued on the compute stream
    if (st == FK_OK && xs != cs) {
        hipError_t e = hipEventRecord(done[0], cs);
        if (e == hipSuccess) e = hipStreamWaitEvent(xs, done[0], 0);
        if (e != hipSuccess) st = hip_fail(e, "order streams");
    }
    auto body = [&]() -> fk_status {
        const int dt = p->dtype;
        FK_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(w.sums), rows * d, 0u, cs), "clear sums");
        FK_TRY(launch_prepare(dt, C, w.lowp, w.bias, rows, (int)d, cs), "prepare centroids");
        const void* Cq = dt == FK_F32 ? static_cast<const void*>(C) : w.lowp;
        int64_t seq = 0;  // chunk sequence number across iterations
        for (int it = 0; it < max_iters; ++it) {
            FK_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(counts), rows, 0u, cs), "clear counts");
            for (int64_t b = 0; b < B; ++b) {
                const char* Cqb = static_cast<const char*>(Cq) + (size_t)(b * K * d) * es;
                for (int64_t c = 0; c < nchunk; ++c, ++seq) {
                    const int buf = (int)(seq & 1);
                    const int64_t i0 = c * chunk;
                    const int64_t n = (N - i0) < chunk ? (N - i0) : chunk;
                    // copy stream: wait until the compute stream released this buffer
                    if (seq >= 2) FK_TRY(hipStreamWaitEvent(xs, done[buf], 0), "wait buffer");
                    const char* src = static_cast<const char*>(X_host) + (size_t)((b * N + i0) * d) * es;
                    FK_TRY(hipMemcpyAsync(w.xbuf[buf], src, (size_t)(n * d) * es, hipMemcpyHostToDevice, xs),
                           "copy chunk");
                    FK_TRY(hipEventRecord(copied[buf], xs), "record copy");
                    // compute stream: assign, sort and segment sums of this chunk
                    FK_TRY(hipStreamWaitEvent(cs, copied[buf], 0), "wait copy");
                    int32_t* lab = labels + b * N + i0;
                    FK_TRY(launch_assign(dt, w.xbuf[buf], Cqb, w.bias + b * K, lab, nullptr, 1, n, K,
                                         (int)d, cs),
                           "assign");
                    SortParams so{};
                    so.labels = lab;
                    so.counts = w.ccounts;
                    so.offsets = w.offsets;
                    so.sorted_idx = w.sorted_idx;
                    so.poff = w.poff;
                    so.pieces = w.pieces;
                    so.part = w.part;
                    so.table = w.table;
                    so.radix = w.radix;
                    so.nvalid = w.nvalid;
                    so.bad = w.bad;
                    FK_TRY(launch_sort(so, 1, n, K, cs), "sort chunk labels");
                    if (w.csums) {
                        // deterministic: this chunk's sums stored (pieces merged in
                        // order), then added to the running sums in chunk order
                        const SegParams sp{true, w.csums, nullptr, nullptr, nullptr, nullptr,
                                           nullptr, nullptr, w.psums, w.poff};
                        FK_TRY(launch_segment_sums(dt, w.xbuf[buf], w.sorted_idx, w.offsets,
                                                   w.pieces, sp, 1, n, K, (int)d, cs),
                               "segment sums");
                        FK_TRY(launch_add_f32(w.sums + b * K * d, w.csums, K * d, cs),
                               "add chunk sums");
                    } else {
                        const SegParams sp{false, w.sums + b * K * d, nullptr, nullptr, nullptr,
                                           nullptr, nullptr, nullptr};
                        FK_TRY(launch_segment_sums(dt, w.xbuf[buf], w.sorted_idx, w.offsets,
                                                   w.pieces, sp, 1, n, K, (int)d, cs),
                               "segment sums");
                    }
                    FK_TRY(launch_add_i32(counts + b * K, w.ccounts, K, cs), "add counts");
                    FK_TRY(hipEventRecord(done[buf], cs), "record done");
                }
            }
            FK_TRY(launch_finalize(dt, w.sums, counts, C, C, w.lowp, w.bias, nullptr, rows, (int)d, cs),
                   "finalize");
        }
        return FK_OK;
    };
    if (st == FK_OK) st = body();
    for (int i = 0; i < 2; ++i) {
        if (copied[i]) (void)hipEventDestroy(copied[i]);
        if (done[i]) (void)hipEventDestroy(done[i]);
    }
    return st;
}

fk_status fk_error_count(const fk_problem* p, const void* ws, size_t ws_bytes, int64_t* count,
                         void* stream) {
    FK_CHECK(check_problem(p));
    if (!count) return fail(FK_EINVAL, "count is NULL");
    Workspace w;
    FK_CHECK(check_ws(*p, const_cast<void*>(ws), ws_bytes, &w));
    hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t total = 0;
    int32_t part[256];
    for (int64_t b0 = 0; b0 < p->B; b0 += 256) {
        const int64_t nb = p->B - b0 < 256 ? p->B - b0 : 256;
        FK_TRY(hipMemcpyAsync(part, w.bad + b0, (size_t)nb * sizeof(int32_t),
                              hipMemcpyDeviceToHost, s),
               "read error count");
        FK_TRY(hipStreamSynchronize(s), "synchronise");
        for (int64_t i = 0; i < nb; ++i) total += part[i];
    }
    *count = total;
    return FK_OK;
}

// ---- tuning -------------------------------------------------------------------

fk_status fk_assign_variant(const fk_problem* p, const void* X, const void* C, const float* bias,
                            int32_t* labels, int point_blocks, int waves, int64_t grid_wgs,
                            void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(X, "X"));
    FK_CHECK(check_ptr(C, "C"));
    FK_CHECK(check_ptr(bias, "bias"));
    FK_CHECK(check_ptr(labels, "labels"));
    if (p->dtype != FK_F16) return fail(FK_EUNSUPPORTED, "assign variants are fp16 only");
    if (p->d != 64 && p->d != 128 && p->d != 256)
        return fail(FK_EUNSUPPORTED, "assign variants need d = 64, 128 or 256");
    if (p->K < 32) return fail(FK_EUNSUPPORTED, "assign variants need K >= 32");
    if (point_blocks != 1 && point_blocks != 2 && point_blocks != 4 && point_blocks != 8)
        return fail(FK_EINVAL, "point_blocks must be 1, 2, 4 or 8");
    if (waves != 2 && waves != 4 && waves != 8) return fail(FK_EINVAL, "waves must be 2, 4 or 8");
    if (grid_wgs < 0 || grid_wgs > 0x7fffffff) return fail(FK_EINVAL, "grid_wgs out of range");
    hipStream_t s = static_cast<hipStream_t>(stream);
    FK_TRY(launch_assign_variant(X, C, bias, labels, p->B, p->N, p->K, (int)p->d, point_blocks,
                                 waves, grid_wgs, s),
           "assign variant");
    return FK_OK;
}

// ---- baselines ---------------------------------------------------------------

fk_status fk_baseline_scores(const fk_problem* p, const void* X, const void* C, const float* bias,
                             float* D, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(X, "X"));
    FK_CHECK(check_ptr(C, "C"));
    FK_CHECK(check_ptr(bias, "bias"));
    FK_CHECK(check_ptr(D, "D"));
    if (p->dtype == FK_F32) return fail(FK_EUNSUPPORTED, "scores baseline takes fp16 or bf16");
    if (p->d > 256) return fail(FK_EUNSUPPORTED, "scores baseline supports d <= 256");
    hipStream_t s = static_cast<hipStream_t>(stream);
    FK_TRY(launch_scores(p->dtype, X, C, bias, D, p->B, p->N, p->K, (int)p->d, s), "scores");
    return FK_OK;
}

fk_status fk_baseline_argmin(const fk_problem* p, const float* D, int32_t* labels, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(D, "D"));
    FK_CHECK(check_ptr(labels, "labels"));
    hipStream_t s = static_cast<hipStream_t>(stream);
    FK_TRY(launch_argmin_rows(D, labels, p->B * p->N, p->K, s), "argmin");
    return FK_OK;
}

fk_status fk_baseline_update_scatter(const fk_problem* p, const void* X, const int32_t* labels,
                                     const float* C_prev, float* C_next, void* C_next_lowp,
                                     int32_t* counts, float* sums, void* stream) {
    FK_CHECK(check_problem(p));
    FK_CHECK(check_ptr(X, "X"));
    FK_CHECK(check_ptr(labels, "labels"));
    FK_CHECK(check_ptr(C_prev, "C_prev"));
    FK_CHECK(check_ptr(C_next, "C_next"));
    FK_CHECK(check_ptr(C_next_lowp, "C_next_lowp", false));
    FK_CHECK(check_ptr(counts, "counts"));
    FK_CHECK(check_ptr(sums, "sums"));
    if (p->dtype == FK_F32 && C_next_lowp && C_next_lowp == static_cast<void*>(C_next))
        return fail(FK_EINVAL, "C_next_lowp must differ from C_next");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t rows = p->B * p->K;
    FK_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(counts), rows, 0u, s), "clear counts");
    FK_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(sums), rows * p->d, 0u, s), "clear sums");
    FK_TRY(launch_scatter_add(p->dtype, X, labels, sums, counts, p->B, p->N, p->K, (int)p->d, s),
           "scatter add");
    FK_TRY(launch_finalize(p->dtype, sums, counts, C_prev, C_next,
                           p->dtype == FK_F32 ? nullptr : C_next_lowp, nullptr, nullptr, rows,
                           (int)p->d, s),
           "finalize");
    if (p->dtype == FK_F32 && C_next_lowp)
        FK_TRY(hipMemcpyAsync(C_next_lowp, C_next, (size_t)(rows * p->d) * sizeof(float),
                              hipMemcpyDeviceToDevice, s),
               "copy fp32 centroids");
    return FK_OK;
}

}  // extern "C"
