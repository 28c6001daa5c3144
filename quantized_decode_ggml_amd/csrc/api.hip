// C ABI of libqdec (declared in include/qdec.h): argument validation, the
// repack cache, error reporting and the launch counter.  All device work is in
// the kernels of the other translation units; nothing here computes on the CPU.
#include "qdec.h"
#include "qdec_internal.h"

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

namespace qdec {

namespace {

thread_local std::string t_error;
std::atomic<uint64_t> g_launches{0};

int fail(int status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(QDEC_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------------ repack cache --
// Keyed by (device, raw pointer, type, n_in, n_out), guarded by one mutex (the
// pages' weight cache is likewise a mutex-guarded global map).  The repack is
// enqueued on the caller's stream; an event records its completion so that a
// first use from another stream waits for it.
struct Key {
    int dev;
    uintptr_t ptr;
    int type;
    int64_t n_in, n_out;
    bool operator<(const Key& o) const
    {
        return std::tie(dev, ptr, type, n_in, n_out) < std::tie(o.dev, o.ptr, o.type, o.n_in, o.n_out);
    }
};

struct Entry {
    void* buf = nullptr;
    int64_t bytes = 0;
    hipEvent_t ready = nullptr;
    hipStream_t made_on = nullptr;
    bool done = false;
};

std::mutex g_mu;
std::map<Key, Entry> g_cache;

bool fail_alloc_hook()
{
    const char* v = std::getenv("QDEC_FAIL_ALLOC");
    return v && v[0] == '1';
}

// QDEC_LOG=1: one stderr line per library allocation or release (a repacked
// copy made or freed, a workspace made or grown), keys separated by '|'.
bool log_on()
{
    static const bool on = [] {
        const char* v = std::getenv("QDEC_LOG");
        return v && v[0] == '1';
    }();
    return on;
}

const char* type_name(int type)
{
    switch (type) {
        case QDEC_TYPE_F32: return "f32_bf16_copy";
        case QDEC_TYPE_Q8_0: return "q8_0";
        case QDEC_TYPE_Q4_K: return "q4_k";
        case QDEC_TYPE_Q6_K: return "q6_k";
        case kTypeQ8_0Tiled: return "q8_0_tiled";
        case kTypeQ4KTiled: return "q4_k_tiled";
        case kTypeQ6KTiled: return "q6_k_tiled";
        default: return "unknown";
    }
}

void destroy(Entry& e)
{
    if (e.ready) (void)hipEventDestroy(e.ready);
    if (e.buf) (void)hipFree(e.buf);
    e = Entry{};
}

int64_t copy_bytes(int type, int64_t n_in, int64_t n_out)
{
    return type == QDEC_TYPE_F32 ? n_in * n_out * 2
         : type == QDEC_TYPE_Q8_0 ? q8_plane_bytes(n_in, n_out)
         : type == kTypeQ8_0Tiled ? q8t_plane_bytes(n_in, n_out)
         : type == kTypeQ4KTiled ? q4kt_plane_bytes(n_in, n_out)
         : type == kTypeQ6KTiled ? q6kt_plane_bytes(n_in, n_out)
         : type == QDEC_TYPE_Q6_K ? q6k_plane_bytes(n_in, n_out)
                                  : q4k_plane_bytes(n_in, n_out);
}

hipError_t launch_copy_of(int type, const void* w, int64_t n_in, int64_t n_out, void* dst, hipStream_t s)
{
    const uint8_t* raw = static_cast<const uint8_t*>(w);
    return type == QDEC_TYPE_F32 ? launch_to_bf16(static_cast<const float*>(w), n_in * n_out, dst, s)
         : type == QDEC_TYPE_Q8_0 ? launch_repack_q8_0(raw, n_in, n_out, dst, s)
         : type == kTypeQ8_0Tiled ? launch_repack_q8_0_tiled(raw, n_in, n_out, dst, s)
         : type == kTypeQ4KTiled ? launch_repack_q4k_tiled(raw, n_in, n_out, dst, s)
         : type == kTypeQ6KTiled ? launch_repack_q6k_tiled(raw, n_in, n_out, dst, s)
         : type == QDEC_TYPE_Q6_K ? launch_repack_q6k(raw, n_in, n_out, dst, s)
                                  : launch_repack_q4k(raw, n_in, n_out, dst, s);
}

// Returns the repacked copy of w, making it on first use.  With `wait` the
// host waits until the copy is complete (qdec_prepare).  With `optional`, a
// copy that a stream capture cannot make or wait for is reported as absent
// (*out = nullptr, QDEC_OK) instead of as an error.
int repacked(const void* w, int type, int64_t n_in, int64_t n_out, hipStream_t s, const void** out,
             bool wait = false, bool optional = false, bool noalloc = false)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    const Key key{dev, reinterpret_cast<uintptr_t>(w), type, n_in, n_out};
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &capture) != hipSuccess) {
        (void)hipGetLastError();
        capture = hipStreamCaptureStatusNone;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_cache.find(key);
    if (it == g_cache.end()) {
        // the allocation-free entry point never makes a copy
        if (noalloc) {
            if (optional) return QDEC_OK;
            return fail(QDEC_EINVAL, "weight %p has no repacked copy: call qdec_prepare first (this entry point "
                                     "allocates nothing)", w);
        }
        // a repack allocates device memory, which a captured graph cannot do
        if (capture != hipStreamCaptureStatusNone) {
            if (optional) return QDEC_OK;
            return fail(QDEC_EINVAL, "weight %p has no repacked copy: call qdec_prepare before graph capture", w);
        }
        if (fail_alloc_hook()) return fail(QDEC_ENOMEM, "repack allocation refused (QDEC_FAIL_ALLOC=1)");
        Entry ent;
        ent.bytes = copy_bytes(type, n_in, n_out);
        e = hipMalloc(&ent.buf, (size_t)ent.bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(QDEC_ENOMEM, "hipMalloc(%lld bytes) for a repacked copy: %s",
                        (long long)ent.bytes, hipGetErrorString(e));
        }
        e = launch_copy_of(type, w, n_in, n_out, ent.buf, s);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ent.ready, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventRecord(ent.ready, s);
        if (e != hipSuccess) {
            destroy(ent);
            return hip_fail(e, "repack launch");
        }
        ent.made_on = s;
        it = g_cache.emplace(key, ent).first;
        if (log_on())
            std::fprintf(stderr, "qdec|repack|dev=%d|w=%p|type=%s|n_in=%lld|n_out=%lld|bytes=%lld\n", dev, w,
                         type_name(type), (long long)n_in, (long long)n_out, (long long)ent.bytes);
    }
    Entry& ent = it->second;
    if (!ent.done) {
        if (capture != hipStreamCaptureStatusNone) {
            // an event wait or query would invalidate the capture
            if (optional) return QDEC_OK;
            return fail(QDEC_EINVAL, "weight %p: its repack may still be running; call qdec_prepare for it "
                                     "before graph capture", w);
        }
        if (wait) {
            e = hipEventSynchronize(ent.ready);
            if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
            ent.done = true;
        } else if (hipEventQuery(ent.ready) == hipSuccess) {
            ent.done = true;
        } else if (s != ent.made_on) {
            e = hipStreamWaitEvent(s, ent.ready, 0);
            if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
        }
    }
    *out = ent.buf;
    return QDEC_OK;
}

// ------------------------------------------------------------ workspaces --
// Workspace (the 3..8-row GEMV's K-slice sums, top-k candidate lists,
// attention chunk partials, the batched GEMMs' bf16 x and slice partials),
// one buffer per (device, stream): calls on one stream are ordered, so they
// can share it;
// calls on different streams never do.  A buffer grows on demand outside
// stream capture; a capturing stream whose buffer is missing or too small gets
// none, and the caller then takes the VALU kernels.  A buffer that a larger
// one replaces is not freed: a graph captured earlier may still hold its
// address, so it stays on the retired list until qdec_clear_cache.
std::map<std::pair<int, uintptr_t>, Entry> g_ws;
std::vector<std::pair<int, Entry>> g_ws_retired;

int stream_workspace(hipStream_t s, int64_t bytes, void** out)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &capture) != hipSuccess) {
        (void)hipGetLastError();
        capture = hipStreamCaptureStatusNone;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    Entry& ent = g_ws[{dev, reinterpret_cast<uintptr_t>(s)}];
    if (ent.bytes >= bytes) {
        *out = ent.buf;
        return QDEC_OK;
    }
    if (capture != hipStreamCaptureStatusNone) return QDEC_OK;
    if (fail_alloc_hook()) return fail(QDEC_ENOMEM, "workspace allocation refused (QDEC_FAIL_ALLOC=1)");
    if (ent.buf) {
        // queued kernels and captured graphs may still use the old buffer
        g_ws_retired.emplace_back(dev, ent);
        ent = Entry{};
    }
    e = hipMalloc(&ent.buf, (size_t)bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        ent = Entry{};
        return fail(QDEC_ENOMEM, "hipMalloc(%lld bytes) for a workspace: %s", (long long)bytes,
                    hipGetErrorString(e));
    }
    ent.bytes = bytes;
    *out = ent.buf;
    if (log_on())
        std::fprintf(stderr, "qdec|workspace|dev=%d|stream=%p|bytes=%lld|retired=%zu\n", dev, (void*)s,
                     (long long)bytes, g_ws_retired.size());
    return QDEC_OK;
}

// ------------------------------------------------------------ validation --

int check_dims(const char* fn, int64_t n_in, int64_t n_out, int64_t batch, int64_t kmult,
               int64_t max_batch)
{
    if (n_in <= 0 || n_out <= 0) return fail(QDEC_EINVAL, "%s: n_in=%lld n_out=%lld must be > 0", fn, (long long)n_in, (long long)n_out);
    if (n_in % kmult != 0) return fail(QDEC_EINVAL, "%s: n_in=%lld is not a multiple of %lld", fn, (long long)n_in, (long long)kmult);
    if (batch < 1 || (max_batch > 0 && batch > max_batch))
        return fail(QDEC_EINVAL, "%s: batch=%lld outside [1, %lld]", fn, (long long)batch, (long long)(max_batch > 0 ? max_batch : INT32_MAX));
    if (batch > INT32_MAX || n_in > INT32_MAX / 2 || n_out > INT32_MAX)
        return fail(QDEC_EINVAL, "%s: dimension too large", fn);
    return QDEC_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, uintptr_t align)
{
    if (!p) return fail(QDEC_EINVAL, "%s: %s is NULL", fn, name);
    if (!aligned(p, align)) return fail(QDEC_EINVAL, "%s: %s is not %u-byte aligned", fn, name, (unsigned)align);
    return QDEC_OK;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)bbytes && pb < pa + (uintptr_t)abytes;
}

#define QDEC_TRY(expr)                 \
    do {                               \
        const int _rc = (expr);        \
        if (_rc != QDEC_OK) return _rc; \
    } while (0)

int finish(hipError_t e, const char* what)
{
    if (e != hipSuccess) return hip_fail(e, what);
    return QDEC_OK;
}

// fixed_ws: a caller-provided workspace of at least q8_mfma_workspace_bytes
// (the allocation-free entry point); with noalloc no repacked copy is made.
int q8_gemv_common(GemvMode mode, const char* fn, const void* const* ws, int nw, int64_t n_in,
                   const int64_t* rows, int64_t batch, const float* x, const float* residual,
                   float* const* outs, int nout, hipStream_t s, const float* norm_w = nullptr,
                   float eps = 0.0f, void* fixed_ws = nullptr, bool noalloc = false)
{
    for (int k = 0; k < nw; ++k) QDEC_TRY(check_ptr(fn, "weight", ws[k], 2));
    QDEC_TRY(check_ptr(fn, "x", x, 16));
    for (int k = 0; k < nout; ++k) {
        QDEC_TRY(check_ptr(fn, "out", outs[k], 4));
        if (overlaps(outs[k], batch * rows[k] * 4, x, batch * n_in * 4))
            return fail(QDEC_EINVAL, "%s: out overlaps x", fn);
    }
    if (mode == kResidual) {
        QDEC_TRY(check_ptr(fn, "residual", residual, 4));
        if (overlaps(residual, batch * rows[0] * 4, x, batch * n_in * 4))
            return fail(QDEC_EINVAL, "%s: residual overlaps x", fn);
    }
    Q8GemvProblem p{};
    p.mode = mode;
    p.nseg = nw;
    for (int k = 0; k < nw; ++k) {
        const void* buf = nullptr;
        QDEC_TRY(repacked(ws[k], QDEC_TYPE_Q8_0, n_in, rows[k], s, &buf, false, false, noalloc));
        p.w[k] = q8_view(buf, n_in, rows[k]);
        p.rows[k] = rows[k];
        p.out[k] = outs[k < nout ? k : 0];
    }
    p.x = x;
    p.residual = residual;
    p.n_in = n_in;
    p.batch = batch;
    if (norm_w) {
        // callers pass a norm only where it folds into the one-row kernel
        p.norm_w = norm_w;
        p.eps = eps;
        if (!q8_gemv_norm_fusable(p)) return fail(QDEC_EINVAL, "%s: RMSNorm cannot be folded here", fn);
        return finish(launch_q8_0_gemv(p, s), fn);
    }
    if (q8_mfma_supported(p)) {
        // tiled copies and a workspace; inside a capture either may be missing,
        // and the VALU kernels then run instead
        Q8TView tiles[3] = {};
        bool have = true;
        for (int k = 0; k < nw && have; ++k) {
            const void* tb = nullptr;
            QDEC_TRY(repacked(ws[k], kTypeQ8_0Tiled, n_in, rows[k], s, &tb, false, true, noalloc));
            if (tb) tiles[k] = q8t_view(tb, n_in, rows[k]);
            else have = false;
        }
        // the K slices' sums (none when every workgroup covers whole rows)
        int64_t flat = rows[0];
        if (mode == kQKV)
            for (int k = 1; k < nw; ++k) flat += rows[k];
        const int64_t need = q8_mfma_workspace_bytes(mode, n_in, flat, batch);
        void* wsp = need > 0 ? fixed_ws : nullptr;
        if (have && need > 0 && !wsp && !noalloc) QDEC_TRY(stream_workspace(s, need, &wsp));
        if (have && (need == 0 || wsp)) return finish(launch_q8_0_gemv_mfma(p, tiles, wsp, s), fn);
    }
    return finish(launch_q8_0_gemv(p, s), fn);
}

// y = RMSNorm(x) feeding a Q8_0 product of `mode`: folded into the one-row
// kernel where it can be, else normalised into `scratch` first.
int q8_normed_product(GemvMode mode, const char* fn, const void* const* ws, int nw, int64_t n_in,
                      const int64_t* rows, int64_t batch, const float* x, const float* norm_w, float eps,
                      float* const* outs, int nout, float* scratch, hipStream_t s)
{
    QDEC_TRY(check_ptr(fn, "norm_w", norm_w, 16));
    if (!(eps >= 0.0f) || eps > 1.0f) return fail(QDEC_EINVAL, "%s: eps=%g outside [0, 1]", fn, (double)eps);
    Q8GemvProblem probe{};
    probe.batch = batch;
    probe.n_in = n_in;
    if (q8_gemv_norm_fusable(probe))
        return q8_gemv_common(mode, fn, ws, nw, n_in, rows, batch, x, nullptr, outs, nout, s, norm_w, eps);
    QDEC_TRY(check_ptr(fn, "scratch", scratch, 16));
    if (overlaps(scratch, batch * n_in * 4, x, batch * n_in * 4))
        return fail(QDEC_EINVAL, "%s: scratch overlaps the input", fn);
    QDEC_TRY(finish(launch_rmsnorm(x, n_in, batch, norm_w, eps, scratch, s), fn));
    return q8_gemv_common(mode, fn, ws, nw, n_in, rows, batch, scratch, nullptr, outs, nout, s);
}

// ------------------------------------------------- allocation-free scratch --
// The scratch of q8_0_gemv_topk_noalloc: one static device array, which every
// GPU the library runs on holds (its own copy) until the process ends.  In
// host code `scratch` only names the symbol; its device address on each GPU
// comes from hipGetSymbolAddress, taken once per device (with that device
// current) on the entry point's first call there and kept.
constexpr int64_t kNoAllocScratchBytes = (int64_t)QDEC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

int noalloc_scratch(void** out)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(QDEC_EUNSUPPORTED, "device %d out of range for the static scratch", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(QDEC_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        e != hipSuccess ? hipGetErrorString(e) : "null address");
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return QDEC_OK;
}

}  // namespace

void count_launch(uint64_t n) { g_launches.fetch_add(n, std::memory_order_relaxed); }

int device_cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace qdec

using namespace qdec;

extern "C" {

int q8_0_gemv(const void* w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
              hipStream_t stream)
{
    QDEC_TRY(check_dims("q8_0_gemv", n_in, n_out, batch, 32, QDEC_GEMV_MAX_BATCH));
    const void* ws[1] = {w};
    const int64_t rows[1] = {n_out};
    float* outs[1] = {out};
    return q8_gemv_common(kPlain, "q8_0_gemv", ws, 1, n_in, rows, batch, x, nullptr, outs, 1, stream);
}

int q8_0_gemv_residual(const void* w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                       const float* residual, float* out, hipStream_t stream)
{
    QDEC_TRY(check_dims("q8_0_gemv_residual", n_in, n_out, batch, 32, QDEC_GEMV_MAX_BATCH));
    if (residual != out && residual && out && overlaps(residual, batch * n_out * 4, out, batch * n_out * 4))
        return fail(QDEC_EINVAL, "q8_0_gemv_residual: residual partially overlaps out");
    const void* ws[1] = {w};
    const int64_t rows[1] = {n_out};
    float* outs[1] = {out};
    return q8_gemv_common(kResidual, "q8_0_gemv_residual", ws, 1, n_in, rows, batch, x, residual,
                          outs, 1, stream);
}

int q8_0_qkv(const void* wq, const void* wk, const void* wv, int64_t n_in, int64_t n_q,
             int64_t n_kv, int64_t batch, const float* x, float* q_out, float* k_out, float* v_out,
             hipStream_t stream)
{
    QDEC_TRY(check_dims("q8_0_qkv", n_in, n_q, batch, 32, QDEC_GEMV_MAX_BATCH));
    if (n_kv < 1 || n_kv > n_q) return fail(QDEC_EINVAL, "q8_0_qkv: n_kv=%lld must be in [1, n_q=%lld]", (long long)n_kv, (long long)n_q);
    if (q_out && k_out && v_out &&
        (overlaps(q_out, batch * n_q * 4, k_out, batch * n_kv * 4) ||
         overlaps(q_out, batch * n_q * 4, v_out, batch * n_kv * 4) ||
         overlaps(k_out, batch * n_kv * 4, v_out, batch * n_kv * 4)))
        return fail(QDEC_EINVAL, "q8_0_qkv: output buffers overlap");
    const void* ws[3] = {wq, wk, wv};
    const int64_t rows[3] = {n_q, n_kv, n_kv};
    float* outs[3] = {q_out, k_out, v_out};
    return q8_gemv_common(kQKV, "q8_0_qkv", ws, 3, n_in, rows, batch, x, nullptr, outs, 3, stream);
}

int q8_0_swiglu(const void* w_gate, const void* w_up, int64_t n_in, int64_t n_out, int64_t batch,
                const float* x, float* out, hipStream_t stream)
{
    QDEC_TRY(check_dims("q8_0_swiglu", n_in, n_out, batch, 32, QDEC_GEMV_MAX_BATCH));
    const void* ws[2] = {w_gate, w_up};
    const int64_t rows[2] = {n_out, n_out};
    float* outs[1] = {out};
    return q8_gemv_common(kSwiGLU, "q8_0_swiglu", ws, 2, n_in, rows, batch, x, nullptr, outs, 1,
                          stream);
}

int q8_0_gemv_topk(const void* w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, int64_t k,
                   float* logits, int32_t* top_idx, float* top_val, hipStream_t stream)
{
    const char* fn = "q8_0_gemv_topk";
    QDEC_TRY(check_dims(fn, n_in, n_out, batch, 32, QDEC_GEMV_MAX_BATCH));
    if (k < 1 || k > QDEC_TOPK_MAX || k > n_out)
        return fail(QDEC_EINVAL, "%s: k=%lld outside [1, min(n_out, %d)]", fn, (long long)k, QDEC_TOPK_MAX);
    QDEC_TRY(check_ptr(fn, "top_idx", top_idx, 4));
    QDEC_TRY(check_ptr(fn, "top_val", top_val, 4));
    QDEC_TRY(check_ptr(fn, "logits", logits, 4));
    const int64_t lb = batch * n_out * 4, tb = batch * k * 4;
    if (overlaps(top_idx, tb, top_val, tb) || overlaps(top_idx, tb, logits, lb) || overlaps(top_val, tb, logits, lb) ||
        overlaps(top_idx, tb, x, batch * n_in * 4) || overlaps(top_val, tb, x, batch * n_in * 4))
        return fail(QDEC_EINVAL, "%s: top_idx, top_val, logits and x must not overlap", fn);
    // the candidate buffers are checked before anything is launched
    const int64_t need = topk_workspace_bytes(n_out, batch, (int)k);
    if (need > 0) {
        void* probe = nullptr;
        QDEC_TRY(stream_workspace(stream, need, &probe));
        if (!probe)
            return fail(QDEC_EINVAL, "%s: no top-k workspace on this capturing stream: make one call on the "
                        "stream before capturing it", fn);
    }
    const void* ws[1] = {w};
    const int64_t rows[1] = {n_out};
    float* outs[1] = {logits};
    QDEC_TRY(q8_gemv_common(kPlain, fn, ws, 1, n_in, rows, batch, x, nullptr, outs, 1, stream));
    // the projection may have grown the stream's workspace: fetch it again
    void* wsp = nullptr;
    if (need > 0) {
        QDEC_TRY(stream_workspace(stream, need, &wsp));
        if (!wsp) return fail(QDEC_EINVAL, "%s: top-k workspace vanished", fn);
    }
    return finish(launch_topk(logits, n_out, batch, (int)k, wsp, top_idx, top_val, stream), fn);
}

int q8_0_gemv_topk_noalloc(const void* w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, int64_t k,
                           float* logits, int32_t* top_idx, float* top_val, hipStream_t stream)
{
    const char* fn = "q8_0_gemv_topk_noalloc";
    QDEC_TRY(check_dims(fn, n_in, n_out, batch, 32, QDEC_GEMV_MAX_BATCH));
    if (k < 1 || k > QDEC_TOPK_MAX || k > n_out)
        return fail(QDEC_EINVAL, "%s: k=%lld outside [1, min(n_out, %d)]", fn, (long long)k, QDEC_TOPK_MAX);
    // scratch layout: the K slices' sums of the matrix-core projection (3..8
    // batch rows, when it splits K), then the top-k candidate lists
    const int64_t proj = batch >= 3 ? align_up(q8_mfma_workspace_bytes(kPlain, n_in, n_out, batch), kAlign) : 0;
    const int64_t need = proj + topk_workspace_bytes(n_out, batch, (int)k);
    if (need > kNoAllocScratchBytes)
        return fail(QDEC_EINVAL, "%s: needs %lld bytes of scratch, above the %lld-byte static array (fewer batch "
                    "rows, a smaller k or a smaller n_out fit)", fn, (long long)need, (long long)kNoAllocScratchBytes);
    QDEC_TRY(check_ptr(fn, "top_idx", top_idx, 4));
    QDEC_TRY(check_ptr(fn, "top_val", top_val, 4));
    QDEC_TRY(check_ptr(fn, "logits", logits, 4));
    const int64_t lb = batch * n_out * 4, tb = batch * k * 4;
    if (overlaps(top_idx, tb, top_val, tb) || overlaps(top_idx, tb, logits, lb) || overlaps(top_val, tb, logits, lb) ||
        overlaps(top_idx, tb, x, batch * n_in * 4) || overlaps(top_val, tb, x, batch * n_in * 4))
        return fail(QDEC_EINVAL, "%s: top_idx, top_val, logits and x must not overlap", fn);
    void* sp = nullptr;
    QDEC_TRY(noalloc_scratch(&sp));
    const void* ws[1] = {w};
    const int64_t rows[1] = {n_out};
    float* outs[1] = {logits};
    QDEC_TRY(q8_gemv_common(kPlain, fn, ws, 1, n_in, rows, batch, x, nullptr, outs, 1, stream, nullptr, 0.0f,
                            proj > 0 ? sp : nullptr, true));
    void* tk = need > proj ? static_cast<char*>(sp) + proj : nullptr;
    return finish(launch_topk(logits, n_out, batch, (int)k, tk, top_idx, top_val, stream), fn);
}

int qdec_rmsnorm(const float* x, int64_t n, int64_t batch, const float* w, float eps, float* out, hipStream_t stream)
{
    const char* fn = "qdec_rmsnorm";
    if (n < 1 || n > INT32_MAX || batch < 1 || batch > INT32_MAX)
        return fail(QDEC_EINVAL, "%s: n=%lld batch=%lld out of range", fn, (long long)n, (long long)batch);
    if (!(eps >= 0.0f) || eps > 1.0f) return fail(QDEC_EINVAL, "%s: eps=%g outside [0, 1]", fn, (double)eps);
    QDEC_TRY(check_ptr(fn, "x", x, 4));
    QDEC_TRY(check_ptr(fn, "w", w, 4));
    QDEC_TRY(check_ptr(fn, "out", out, 4));
    if (out != x && overlaps(out, batch * n * 4, x, batch * n * 4))
        return fail(QDEC_EINVAL, "%s: out overlaps x without being x", fn);
    return finish(launch_rmsnorm(x, n, batch, w, eps, out, stream), fn);
}

int q8_0_rmsnorm_qkv(const void* wq, const void* wk, const void* wv, int64_t n_in, int64_t n_q, int64_t n_kv,
                     int64_t batch, const float* h, const float* norm_w, float eps, float* q_out, float* k_out,
                     float* v_out, float* scratch, hipStream_t stream)
{
    const char* fn = "q8_0_rmsnorm_qkv";
    QDEC_TRY(check_dims(fn, n_in, n_q, batch, 32, QDEC_GEMV_MAX_BATCH));
    if (n_kv < 1 || n_kv > n_q) return fail(QDEC_EINVAL, "%s: n_kv=%lld outside [1, n_q]", fn, (long long)n_kv);
    const void* ws[3] = {wq, wk, wv};
    const int64_t rows[3] = {n_q, n_kv, n_kv};
    float* outs[3] = {q_out, k_out, v_out};
    for (int a = 0; a < 3; ++a)
        for (int b = a + 1; b < 3; ++b)
            if (outs[a] && outs[b] && overlaps(outs[a], batch * rows[a] * 4, outs[b], batch * rows[b] * 4))
                return fail(QDEC_EINVAL, "%s: outputs overlap", fn);
    if (scratch)
        for (int a = 0; a < 3; ++a)
            if (outs[a] && overlaps(outs[a], batch * rows[a] * 4, scratch, batch * n_in * 4))
                return fail(QDEC_EINVAL, "%s: an output overlaps scratch", fn);
    return q8_normed_product(kQKV, fn, ws, 3, n_in, rows, batch, h, norm_w, eps, outs, 3, scratch, stream);
}

int q8_0_attn_out_ffn(const void* wo, const void* w_gate, const void* w_up, const void* w_down, int64_t n_embd,
                      int64_t n_q, int64_t n_ff, int64_t batch, float* h, const float* attn, const float* ffn_norm,
                      float eps, float* scratch, hipStream_t stream)
{
    const char* fn = "q8_0_attn_out_ffn";
    QDEC_TRY(check_dims(fn, n_q, n_embd, batch, 32, QDEC_GEMV_MAX_BATCH));
    QDEC_TRY(check_dims(fn, n_embd, n_ff, batch, 32, QDEC_GEMV_MAX_BATCH));
    QDEC_TRY(check_dims(fn, n_ff, n_embd, batch, 32, QDEC_GEMV_MAX_BATCH));
    QDEC_TRY(check_ptr(fn, "h", h, 16));
    QDEC_TRY(check_ptr(fn, "scratch", scratch, 16));
    const int64_t hb = batch * n_embd * 4, fb = batch * n_ff * 4;
    if (overlaps(scratch, fb + hb, h, hb) || overlaps(scratch, fb + hb, attn, batch * n_q * 4))
        return fail(QDEC_EINVAL, "%s: scratch overlaps h or attn", fn);
    float* f = scratch;                 // batch x n_ff: SwiGLU output
    float* hn = scratch + batch * n_ff; // batch x n_embd: normalised h (several batch rows)
    // h += Wo attn
    {
        const void* ws[1] = {wo};
        const int64_t rows[1] = {n_embd};
        float* outs[1] = {h};
        QDEC_TRY(q8_gemv_common(kResidual, fn, ws, 1, n_q, rows, batch, attn, h, outs, 1, stream));
    }
    // f = SwiGLU(RMSNorm(h))
    {
        const void* ws[2] = {w_gate, w_up};
        const int64_t rows[2] = {n_ff, n_ff};
        float* outs[1] = {f};
        QDEC_TRY(q8_normed_product(kSwiGLU, fn, ws, 2, n_embd, rows, batch, h, ffn_norm, eps, outs, 1, hn, stream));
    }
    // h += Wd f
    const void* ws[1] = {w_down};
    const int64_t rows[1] = {n_embd};
    float* outs[1] = {h};
    return q8_gemv_common(kResidual, fn, ws, 1, n_ff, rows, batch, f, h, outs, 1, stream);
}

namespace {

int check_heads(const char* fn, int64_t n_head, int64_t n_kv, int64_t head_dim, int64_t max_seq)
{
    if (head_dim != 64 && head_dim != 128) return fail(QDEC_EINVAL, "%s: head_dim=%lld not 64 or 128", fn, (long long)head_dim);
    if (n_head < 1 || n_kv < 1 || n_head % n_kv != 0 || n_head / n_kv > 16 || n_head > 4096)
        return fail(QDEC_EINVAL, "%s: n_head=%lld n_kv=%lld: need n_kv | n_head and n_head/n_kv <= 16", fn,
                    (long long)n_head, (long long)n_kv);
    if (max_seq < 1 || max_seq > (int64_t)1 << 24) return fail(QDEC_EINVAL, "%s: max_seq=%lld out of range", fn, (long long)max_seq);
    return QDEC_OK;
}

}  // namespace

int qdec_rope_kv_append(float* q, float* k, const float* v, int64_t n_head, int64_t n_kv, int64_t head_dim, int64_t pos,
                        float base, float* k_cache, float* v_cache, int64_t max_seq, hipStream_t stream)
{
    const char* fn = "qdec_rope_kv_append";
    QDEC_TRY(check_heads(fn, n_head, n_kv, head_dim, max_seq));
    if (pos < 0 || pos >= max_seq) return fail(QDEC_EINVAL, "%s: pos=%lld outside [0, max_seq)", fn, (long long)pos);
    if (!(base > 1.0f) || !(base < 1e30f)) return fail(QDEC_EINVAL, "%s: base=%g must be > 1", fn, (double)base);
    QDEC_TRY(check_ptr(fn, "q", q, 8));
    QDEC_TRY(check_ptr(fn, "k", k, 8));
    QDEC_TRY(check_ptr(fn, "v", v, 8));
    QDEC_TRY(check_ptr(fn, "k_cache", k_cache, 16));
    QDEC_TRY(check_ptr(fn, "v_cache", v_cache, 16));
    const int64_t qb = n_head * head_dim * 4, kb = n_kv * head_dim * 4, cb = n_kv * max_seq * head_dim * 4;
    const void* bufs[5] = {q, k, v, k_cache, v_cache};
    const int64_t lens[5] = {qb, kb, kb, cb, cb};
    for (int a = 0; a < 5; ++a)
        for (int b = a + 1; b < 5; ++b)
            if (overlaps(bufs[a], lens[a], bufs[b], lens[b]))
                return fail(QDEC_EINVAL, "%s: q, k, v and the two caches must not overlap", fn);
    return finish(launch_rope_append(q, k, v, n_head, n_kv, head_dim, pos, (double)base, k_cache, v_cache, max_seq,
                                     stream), fn);
}

int qdec_attention_decode(const float* q, const float* k_cache, const float* v_cache, int64_t n_head, int64_t n_kv,
                          int64_t head_dim, int64_t n_ctx, int64_t max_seq, float scale, float* out, hipStream_t stream)
{
    const char* fn = "qdec_attention_decode";
    QDEC_TRY(check_heads(fn, n_head, n_kv, head_dim, max_seq));
    if (n_ctx < 1 || n_ctx > max_seq) return fail(QDEC_EINVAL, "%s: n_ctx=%lld outside [1, max_seq]", fn, (long long)n_ctx);
    if (!(scale > 0.0f) || !(scale < 1e30f)) return fail(QDEC_EINVAL, "%s: scale=%g must be > 0", fn, (double)scale);
    QDEC_TRY(check_ptr(fn, "q", q, 16));
    QDEC_TRY(check_ptr(fn, "k_cache", k_cache, 16));
    QDEC_TRY(check_ptr(fn, "v_cache", v_cache, 16));
    QDEC_TRY(check_ptr(fn, "out", out, 4));
    const int64_t ob = n_head * head_dim * 4, cb = n_kv * max_seq * head_dim * 4;
    if (overlaps(out, ob, q, ob) || overlaps(out, ob, k_cache, cb) || overlaps(out, ob, v_cache, cb))
        return fail(QDEC_EINVAL, "%s: out overlaps an input", fn);
    void* wsp = nullptr;
    const int64_t need = attention_workspace_bytes(n_head, head_dim, n_ctx);
    if (need > 0) {
        QDEC_TRY(stream_workspace(stream, need, &wsp));
        if (!wsp)
            return fail(QDEC_EINVAL, "%s: no workspace on this capturing stream: make one call on the stream "
                        "before capturing it", fn);
    }
    return finish(launch_attention(q, k_cache, v_cache, n_head, n_kv, head_dim, n_ctx, max_seq, scale, out, wsp,
                                   stream), fn);
}

int q4k_gemv(const void* w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
             hipStream_t stream)
{
    const char* fn = "q4k_gemv";
    QDEC_TRY(check_dims(fn, n_in, n_out, batch, 256, QDEC_GEMV_MAX_BATCH));
    QDEC_TRY(check_ptr(fn, "weight", w, 2));
    QDEC_TRY(check_ptr(fn, "x", x, 16));
    QDEC_TRY(check_ptr(fn, "out", out, 4));
    if (overlaps(out, batch * n_out * 4, x, batch * n_in * 4)) return fail(QDEC_EINVAL, "%s: out overlaps x", fn);
    const void* buf = nullptr;
    if (q4k_mfma_supported(n_in, batch)) {
        // one row on the matrix cores, from the fragment-tiled copy; inside a
        // capture that copy may be missing, and the VALU kernel then runs
        QDEC_TRY(repacked(w, kTypeQ4KTiled, n_in, n_out, stream, &buf, false, true));
        if (buf)
            return finish(launch_q4k_gemv_mfma(q4kt_view(buf, n_in, n_out), n_in, n_out, batch, x, out, stream), fn);
    }
    QDEC_TRY(repacked(w, QDEC_TYPE_Q4_K, n_in, n_out, stream, &buf));
    return finish(launch_q4k_gemv(q4k_view(buf, n_in, n_out), n_in, n_out, batch, x, out, stream), fn);
}

int q6k_gemv(const void* w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
             hipStream_t stream)
{
    const char* fn = "q6k_gemv";
    QDEC_TRY(check_dims(fn, n_in, n_out, batch, 256, QDEC_GEMV_MAX_BATCH));
    QDEC_TRY(check_ptr(fn, "weight", w, 2));
    QDEC_TRY(check_ptr(fn, "x", x, 16));
    QDEC_TRY(check_ptr(fn, "out", out, 4));
    if (overlaps(out, batch * n_out * 4, x, batch * n_in * 4)) return fail(QDEC_EINVAL, "%s: out overlaps x", fn);
    const void* buf = nullptr;
    if (q6k_mfma_supported(n_in, batch)) {
        // one row on the matrix cores, from the fragment-tiled copy; inside a
        // capture that copy may be missing, and the VALU kernel then runs
        QDEC_TRY(repacked(w, kTypeQ6KTiled, n_in, n_out, stream, &buf, false, true));
        if (buf)
            return finish(launch_q6k_gemv_mfma(q6kt_view(buf, n_in, n_out), n_in, n_out, batch, x, out, stream), fn);
    }
    QDEC_TRY(repacked(w, QDEC_TYPE_Q6_K, n_in, n_out, stream, &buf));
    return finish(launch_q6k_gemv(q6k_view(buf, n_in, n_out), n_in, n_out, batch, x, out, stream), fn);
}

int q8_0_gemm_batched(const void* w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                      float* out, hipStream_t stream)
{
    const char* fn = "q8_0_gemm_batched";
    QDEC_TRY(check_dims(fn, n_in, n_out, batch, 32, 0));
    QDEC_TRY(check_ptr(fn, "weight", w, 2));
    QDEC_TRY(check_ptr(fn, "x", x, 16));
    QDEC_TRY(check_ptr(fn, "out", out, 4));
    if (overlaps(out, batch * n_out * 4, x, batch * n_in * 4)) return fail(QDEC_EINVAL, "%s: out overlaps x", fn);
    const void* buf = nullptr;
    QDEC_TRY(repacked(w, QDEC_TYPE_Q8_0, n_in, n_out, stream, &buf));
    // the pipelined kernel rounds x to bf16 in the stream's workspace, the
    // register-staged one keeps its K-slice partials there; a capture on a
    // stream without one runs the register-staged kernel with atomics
    void* wsp = nullptr;
    const int64_t need = q8_gemm_workspace_bytes(n_in, n_out, batch);
    if (need > 0) QDEC_TRY(stream_workspace(stream, need, &wsp));
    return finish(launch_q8_0_gemm(q8_view(buf, n_in, n_out), n_in, n_out, batch, x, out, wsp, stream), fn);
}

int f32_gemm_batched(const float* w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                     float* out, hipStream_t stream)
{
    const char* fn = "f32_gemm_batched";
    QDEC_TRY(check_dims(fn, n_in, n_out, batch, 32, 0));
    QDEC_TRY(check_ptr(fn, "weight", w, 16));
    QDEC_TRY(check_ptr(fn, "x", x, 16));
    QDEC_TRY(check_ptr(fn, "out", out, 4));
    if (overlaps(out, batch * n_out * 4, x, batch * n_in * 4) ||
        overlaps(out, batch * n_out * 4, w, n_out * n_in * 4))
        return fail(QDEC_EINVAL, "%s: out overlaps an input", fn);
    // the bf16 copy is used when qdec_prepare made it (it is never made here:
    // it doubles the weight's footprint and binds the caller not to change W)
    const void* wb = nullptr;
    QDEC_TRY(repacked(w, QDEC_TYPE_F32, n_in, n_out, stream, &wb, false, /*optional*/ true, /*noalloc*/ true));
    // x in bf16 and K-split partial products go to the stream's workspace; a
    // capture on a stream without one large enough takes the register-staged
    // kernel, which adds its K slices with atomics
    void* wsp = nullptr;
    const int64_t need = f32_gemm_workspace_bytes(n_in, n_out, batch, wb != nullptr);
    if (need > 0) QDEC_TRY(stream_workspace(stream, need, &wsp));
    return finish(launch_f32_gemm(w, wb, n_in, n_out, batch, x, out, wsp, stream), fn);
}

int qdec_prepare(const void* w, int type, int64_t n_in, int64_t n_out, hipStream_t stream)
{
    const char* fn = "qdec_prepare";
    if (type != QDEC_TYPE_F32 && type != QDEC_TYPE_Q8_0 && type != QDEC_TYPE_Q4_K && type != QDEC_TYPE_Q6_K)
        return fail(QDEC_EINVAL, "%s: unknown type %d", fn, type);
    const bool blk32 = type == QDEC_TYPE_Q8_0 || type == QDEC_TYPE_F32;
    QDEC_TRY(check_dims(fn, n_in, n_out, 1, blk32 ? 32 : 256, 0));
    QDEC_TRY(check_ptr(fn, "weight", w, type == QDEC_TYPE_F32 ? 16 : 2));
    const void* buf = nullptr;
    QDEC_TRY(repacked(w, type, n_in, n_out, stream, &buf, true));
    // Q8_0 weights also get the fragment-tiled copy of the batched matrix-core
    // GEMV, Q4_K and Q6_K weights that of their one-row matrix-core GEMVs, so
    // that graphs captured later can use them
    if (type == QDEC_TYPE_Q8_0) QDEC_TRY(repacked(w, kTypeQ8_0Tiled, n_in, n_out, stream, &buf, true));
    if (type == QDEC_TYPE_Q4_K && q4k_mfma_supported(n_in, 1))
        QDEC_TRY(repacked(w, kTypeQ4KTiled, n_in, n_out, stream, &buf, true));
    if (type == QDEC_TYPE_Q6_K && q6k_mfma_supported(n_in, 1))
        QDEC_TRY(repacked(w, kTypeQ6KTiled, n_in, n_out, stream, &buf, true));
    return QDEC_OK;
}

int qdec_check_plans(int64_t n_in, int64_t n_out, int64_t batch)
{
    const char* fn = "qdec_check_plans";
    QDEC_TRY(check_dims(fn, n_in, n_out, batch, 32, 0));
    auto bad = [&](const std::string& why) { return fail(QDEC_EUNSUPPORTED, "%s: %s", fn, why.c_str()); };
    // the 3..8-row matrix-core GEMV in each of its forms (QKV: the rows as
    // q, a quarter of them as k and as v, all but the last segment whole
    // 16-row groups), with the workspace each would be given
    if (batch >= 3 && batch <= QDEC_GEMV_MAX_BATCH) {
        const int64_t q16 = n_out / 16 * 16, kv16 = n_out / 64 * 16;
        for (GemvMode mode : {kPlain, kResidual, kSwiGLU, kQKV}) {
            Q8GemvProblem p{};
            p.mode = mode;
            p.n_in = n_in;
            p.batch = batch;
            p.nseg = 1;
            p.rows[0] = n_out;
            if (mode == kQKV) {
                if (q16 == 0 || kv16 == 0) continue;
                p.nseg = 3;
                p.rows[0] = q16;
                p.rows[1] = kv16;
                p.rows[2] = n_out - q16 + kv16;
            }
            if (!q8_mfma_supported(p)) continue;
            int64_t flat = p.rows[0];
            if (mode == kQKV) flat += p.rows[1] + p.rows[2];
            const std::string why = q8_mfma_plan_check(p, q8_mfma_workspace_bytes(mode, n_in, flat, batch));
            if (!why.empty()) return bad(why);
        }
    }
    // the Q4_K and Q6_K matrix-core GEMVs (widths that are multiples of 256),
    // one row and this batch
    if (n_in % 256 == 0 && q4k_mfma_supported(n_in, 1)) {
        std::string why = q4k_mfma_plan_check(n_in, n_out, 1);
        if (why.empty() && batch > 1 && batch <= QDEC_GEMV_MAX_BATCH && q4k_mfma_supported(n_in, batch))
            why = q4k_mfma_plan_check(n_in, n_out, batch);
        if (!why.empty()) return bad(why);
    }
    if (n_in % 256 == 0 && q6k_mfma_supported(n_in, 1)) {
        std::string why = q6k_mfma_plan_check(n_in, n_out, 1);
        if (why.empty() && batch > 1 && batch <= QDEC_GEMV_MAX_BATCH && q6k_mfma_supported(n_in, batch))
            why = q6k_mfma_plan_check(n_in, n_out, batch);
        if (!why.empty()) return bad(why);
    }
    // the batched GEMMs, with and without a workspace (a capture on a stream
    // that has none), dense f32 with and without its bf16 copy
    for (bool ws : {true, false}) {
        std::string why = q8_gemm_plan_check(n_in, n_out, batch, ws ? q8_gemm_workspace_bytes(n_in, n_out, batch) : 0);
        if (!why.empty()) return bad(why);
        for (bool copy : {true, false}) {
            why = f32_gemm_plan_check(n_in, n_out, batch, copy,
                                      ws ? f32_gemm_workspace_bytes(n_in, n_out, batch, copy) : 0);
            if (!why.empty()) return bad(why);
        }
    }
    return QDEC_OK;
}

int qdec_release(const void* w)
{
    int dev = 0;
    if (!w) return fail(QDEC_EINVAL, "qdec_release: w is NULL");
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_mu);
    int n = 0;
    for (auto it = g_cache.begin(); it != g_cache.end();) {
        if (it->first.dev == dev && it->first.ptr == reinterpret_cast<uintptr_t>(w)) {
            (void)hipDeviceSynchronize();
            if (log_on())
                std::fprintf(stderr, "qdec|release|dev=%d|w=%p|type=%s|bytes=%lld\n", dev, w,
                             type_name(it->first.type), (long long)it->second.bytes);
            destroy(it->second);
            it = g_cache.erase(it);
            ++n;
        } else {
            ++it;
        }
    }
    return n ? QDEC_OK : fail(QDEC_EINVAL, "qdec_release: no repacked copy of %p", w);
}

void qdec_clear_cache(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    if (log_on())
        std::fprintf(stderr, "qdec|clear_cache|copies=%zu|workspaces=%zu|retired=%zu\n", g_cache.size(), g_ws.size(),
                     g_ws_retired.size());
    int cur = 0;
    const bool have_dev = hipGetDevice(&cur) == hipSuccess;
    for (auto& kv : g_cache) {
        if (have_dev) (void)hipSetDevice(kv.first.dev);
        (void)hipDeviceSynchronize();
        destroy(kv.second);
    }
    g_cache.clear();
    for (auto& kv : g_ws) {
        if (have_dev) (void)hipSetDevice(kv.first.first);
        (void)hipDeviceSynchronize();
        destroy(kv.second);
    }
    g_ws.clear();
    for (auto& kv : g_ws_retired) {
        if (have_dev) (void)hipSetDevice(kv.first);
        (void)hipDeviceSynchronize();
        destroy(kv.second);
    }
    g_ws_retired.clear();
    if (have_dev) (void)hipSetDevice(cur);
}

int64_t qdec_cache_len(void)
{
    // one per (weight, public type, shape): the tiled copies Q8_0, Q4_K and
    // Q6_K weights also get for the matrix-core GEMVs are not counted separately
    std::lock_guard<std::mutex> lock(g_mu);
    int64_t n = 0;
    for (const auto& kv : g_cache)
        n += kv.first.type != kTypeQ8_0Tiled && kv.first.type != kTypeQ4KTiled && kv.first.type != kTypeQ6KTiled;
    return n;
}

int q8_0_dequantize(const void* w, int64_t n_in, int64_t n_out, float* out, hipStream_t stream)
{
    const char* fn = "q8_0_dequantize";
    QDEC_TRY(check_dims(fn, n_in, n_out, 1, 32, 0));
    QDEC_TRY(check_ptr(fn, "weight", w, 2));
    QDEC_TRY(check_ptr(fn, "out", out, 16));
    const void* buf = nullptr;
    QDEC_TRY(repacked(w, QDEC_TYPE_Q8_0, n_in, n_out, stream, &buf));
    return finish(launch_dequant_q8_0(q8_view(buf, n_in, n_out), n_in, n_out, out, stream), fn);
}

int q4k_dequantize(const void* w, int64_t n_in, int64_t n_out, float* out, hipStream_t stream)
{
    const char* fn = "q4k_dequantize";
    QDEC_TRY(check_dims(fn, n_in, n_out, 1, 256, 0));
    QDEC_TRY(check_ptr(fn, "weight", w, 2));
    QDEC_TRY(check_ptr(fn, "out", out, 16));
    const void* buf = nullptr;
    QDEC_TRY(repacked(w, QDEC_TYPE_Q4_K, n_in, n_out, stream, &buf));
    return finish(launch_dequant_q4k(q4k_view(buf, n_in, n_out), n_in, n_out, out, stream), fn);
}

const char* qdec_last_error(void) { return t_error.c_str(); }

uint64_t qdec_launch_count(void) { return g_launches.load(std::memory_order_relaxed); }

int q6k_dequantize(const void* w, int64_t n_in, int64_t n_out, float* out, hipStream_t stream)
{
    const char* fn = "q6k_dequantize";
    QDEC_TRY(check_dims(fn, n_in, n_out, 1, 256, 0));
    QDEC_TRY(check_ptr(fn, "weight", w, 2));
    QDEC_TRY(check_ptr(fn, "out", out, 16));
    const void* buf = nullptr;
    QDEC_TRY(repacked(w, QDEC_TYPE_Q6_K, n_in, n_out, stream, &buf));
    return finish(launch_dequant_q6k(q6k_view(buf, n_in, n_out), n_in, n_out, out, stream), fn);
}

int qdec_empty_kernel(hipStream_t stream) { return finish(launch_empty(stream), "qdec_empty_kernel"); }

int qdec_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream)
{
    const char* fn = "qdec_copy";
    if (bytes <= 0 || bytes % 16 != 0) return fail(QDEC_EINVAL, "%s: bytes=%lld must be a positive multiple of 16", fn, (long long)bytes);
    QDEC_TRY(check_ptr(fn, "dst", dst, 16));
    QDEC_TRY(check_ptr(fn, "src", src, 16));
    if (overlaps(dst, bytes, src, bytes)) return fail(QDEC_EINVAL, "%s: buffers overlap", fn);
    return finish(launch_copy(dst, src, bytes, stream), fn);
}

int qdec_stream_read(const void* src, int64_t bytes, int loads_per_lane, uint32_t* sink, hipStream_t stream)
{
    const char* fn = "qdec_stream_read";
    if (bytes <= 0 || bytes % 16 != 0 || bytes / 16 > (int64_t)UINT32_MAX * 256)
        return fail(QDEC_EINVAL, "%s: bytes=%lld must be a positive multiple of 16", fn, (long long)bytes);
    if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8 &&
        loads_per_lane != 16)
        return fail(QDEC_EINVAL, "%s: loads_per_lane=%d not 1, 2, 4, 8 or 16", fn, loads_per_lane);
    QDEC_TRY(check_ptr(fn, "src", src, 16));
    QDEC_TRY(check_ptr(fn, "sink", sink, 4));
    if (overlaps(sink, 4, src, bytes)) return fail(QDEC_EINVAL, "%s: sink overlaps src", fn);
    return finish(launch_stream_read(src, bytes, loads_per_lane, sink, stream), fn);
}

}  // extern "C"
