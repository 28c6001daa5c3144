// Host-only driver of the libqdec C ABI, built together with an
// AddressSanitizer-instrumented copy of the library's host code (see
// test_abi_asan.py).  No GPU is needed: every call below is rejected by
// argument validation before any HIP call, or, where the arguments are valid,
// fails at its first HIP call.  ASan watches the validation code, the
// error-message formatting, the size arithmetic of the allocation-free entry
// point and the cache bookkeeping while they run, from several threads at
// once (the error string is per thread).
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "qdec.h"

namespace {

int g_failures = 0;

void expect(bool ok, const char* what)
{
    if (!ok) {
        std::printf("FAIL %s (last error: %s)\n", what, qdec_last_error());
        ++g_failures;
    }
}

// Distinct, aligned, never dereferenced addresses.
template <typename T>
T* at(uintptr_t a)
{
    return reinterpret_cast<T*>(a);
}

constexpr uintptr_t F = 0x10000;

// Every call must return QDEC_EINVAL and leave a message.
int invalid_calls()
{
    int bad = 0;
    auto einval = [&](int rc, const char* what) {
        const bool ok = rc == QDEC_EINVAL && std::strlen(qdec_last_error()) > 0;
        if (!ok) {
            std::printf("FAIL %s: rc=%d msg=%s\n", what, rc, qdec_last_error());
            ++bad;
        }
    };
    float* x = at<float>(F);
    float* out = at<float>(2 * F);
    einval(q8_0_gemv(at<void>(F), 33, 16, 1, x, out, nullptr), "n_in % 32");
    einval(q8_0_gemv(at<void>(F), 0, 16, 1, x, out, nullptr), "n_in 0");
    einval(q8_0_gemv(at<void>(F), 64, -1, 1, x, out, nullptr), "n_out < 0");
    einval(q8_0_gemv(at<void>(F), 64, 16, 0, x, out, nullptr), "batch 0");
    einval(q8_0_gemv(at<void>(F), 64, 16, 9, x, out, nullptr), "batch 9");
    einval(q8_0_gemv(nullptr, 64, 16, 1, x, out, nullptr), "null weight");
    einval(q8_0_gemv(at<void>(F), 64, 16, 1, at<float>(F + 4), out, nullptr), "x misaligned");
    einval(q8_0_gemv(at<void>(F + 1), 64, 16, 1, x, out, nullptr), "odd weight address");
    einval(q8_0_gemv(at<void>(F), 64, 16, 1, x, at<float>(F + 16), nullptr), "out overlaps x");
    einval(q8_0_gemv(at<void>(F), INT64_MAX - 31, 16, 1, x, out, nullptr), "huge n_in");
    einval(q8_0_gemv_residual(at<void>(F), 64, 16, 1, x, nullptr, out, nullptr), "null residual");
    einval(q8_0_gemv_residual(at<void>(F), 64, 16, 1, x, at<float>(2 * F + 8), out, nullptr), "residual misaligned");
    einval(q8_0_qkv(at<void>(F), at<void>(F), at<void>(F), 64, 8, 9, 1, x, out, at<float>(3 * F), at<float>(4 * F),
                    nullptr),
           "n_kv > n_q");
    einval(q8_0_qkv(at<void>(F), at<void>(F), at<void>(F), 64, 8, 4, 1, x, out, at<float>(2 * F + 16),
                    at<float>(4 * F), nullptr),
           "q and k overlap");
    einval(q8_0_swiglu(at<void>(F), nullptr, 64, 8, 1, x, out, nullptr), "null up");
    einval(q4k_gemv(at<void>(F), 128, 8, 1, x, out, nullptr), "q4k n_in % 256");
    einval(q6k_gemv(at<void>(F), 256, 8, 9, x, out, nullptr), "q6k batch 9");
    einval(q8_0_gemm_batched(at<void>(F), 64, 8, 0, x, out, nullptr), "gemm batch 0");
    einval(f32_gemm_batched(at<float>(F + 4), 64, 8, 1, at<float>(4 * F), at<float>(8 * F), nullptr),
           "f32 weight misaligned");
    einval(qdec_prepare(at<void>(F), 7, 64, 8, nullptr), "unknown type");
    einval(qdec_prepare(at<void>(F), QDEC_TYPE_Q4_K, 64, 8, nullptr), "q4k prepare n_in");
    einval(qdec_prepare(at<void>(F + 4), QDEC_TYPE_F32, 64, 8, nullptr), "f32 prepare misaligned");
    einval(q8_0_dequantize(at<void>(F), 64, 8, at<float>(2 * F + 4), nullptr), "dequant out misaligned");
    einval(qdec_copy(at<void>(F), at<void>(2 * F), 24, nullptr), "copy bytes % 16");
    einval(qdec_release(nullptr), "release null");
    einval(qdec_attention_decode(at<float>(F), at<float>(2 * F), at<float>(3 * F), 24, 8, 96, 10, 100, 0.1f,
                                 at<float>(4 * F), nullptr),
           "head_dim 96");
    einval(qdec_rope_kv_append(at<float>(F), at<float>(2 * F), at<float>(3 * F), 24, 8, 128, 100, 10000.0f,
                               at<float>(4 * F), at<float>(5 * F), 100, nullptr),
           "rope pos past the cache");
    einval(q8_0_gemv_topk(at<void>(F), 64, 400, 1, x, 257, at<float>(2 * F), at<int32_t>(3 * F),
                          at<float>(4 * F), nullptr),
           "k > 256");
    einval(q8_0_gemv_topk(at<void>(F), 64, 16, 1, x, 4, at<float>(2 * F), at<int32_t>(2 * F + 8), at<float>(4 * F),
                          nullptr),
           "top_idx inside logits");
    einval(qdec_rmsnorm(x, 64, 1, at<float>(2 * F), -1.0f, at<float>(3 * F), nullptr), "negative eps");
    // the allocation-free entry point refuses a scratch request it cannot
    // hold before touching the device: 8 rows x 8192 columns of 128256 logits
    einval(q8_0_gemv_topk_noalloc(at<void>(0x40000000), 8192, 128256, 8, at<float>(0x1000000), 256,
                                  at<float>(0x10000000), at<int32_t>(0x20000000), at<float>(0x30000000), nullptr),
           "noalloc scratch too small");
    if (std::strstr(qdec_last_error(), "static array") == nullptr) {
        std::printf("FAIL noalloc message: %s\n", qdec_last_error());
        ++bad;
    }
    return bad;
}

// Valid arguments with no device: the first HIP call fails; the call must
// report an error (not crash) and leave a message.
int no_device_calls()
{
    int bad = 0;
    auto failed = [&](int rc, const char* what) {
        if (rc == QDEC_OK || std::strlen(qdec_last_error()) == 0) {
            std::printf("FAIL %s: rc=%d msg=%s\n", what, rc, qdec_last_error());
            ++bad;
        }
    };
    failed(qdec_release(at<void>(F)), "release without a device");
    failed(q8_0_gemv_topk_noalloc(at<void>(0x40000000), 3072, 128256, 8, at<float>(0x1000000), 256,
                                  at<float>(0x10000000), at<int32_t>(0x20000000), at<float>(0x30000000), nullptr),
           "noalloc request that fits");
    if (std::strstr(qdec_last_error(), "static array") != nullptr) {
        std::printf("FAIL a fitting noalloc request was refused for size: %s\n", qdec_last_error());
        ++bad;
    }
    qdec_clear_cache();   // nothing cached; must not touch freed state
    return bad;
}

}  // namespace

int main()
{
    g_failures += invalid_calls();
    g_failures += no_device_calls();
    // the same from several threads at once: per-thread error strings
    std::vector<std::thread> ts;
    std::vector<int> res(8, 0);
    for (int t = 0; t < 8; ++t) ts.emplace_back([&res, t] { res[t] = invalid_calls(); });
    for (auto& t : ts) t.join();
    for (int r : res) g_failures += r;
    expect(qdec_launch_count() == 0, "no kernel was launched");
    expect(qdec_cache_len() == 0, "no copy was made");
    std::printf("abi_asan_driver: %d failures\n", g_failures);
    return g_failures ? 1 : 0;
}
