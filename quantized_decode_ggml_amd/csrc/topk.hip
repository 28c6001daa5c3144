// On-device top-k of vocabulary logits ("Struct QTensorEngine" page, methods
// dispatch_output_topk_chunked and dispatch_output_top1_chunked: the logits stay
// on the GPU, each chunk of the vocabulary is reduced there, and only the K
// (id, logit) candidates leave).
//
// Order: a larger logit ranks first; equal logits rank by the smaller vocabulary
// index; -0 ranks as +0.  Each (logit, index) pair becomes one 64-bit key whose
// unsigned order is exactly that order: the high word is the f32 bit pattern
// mapped monotonically onto unsigned integers (positive values get the sign
// bit set, negative values are complemented), the low word is 0xFFFFFFFF - index.
// NaN logits (only possible from non-finite inputs) rank by their bit pattern:
// a positive NaN above +inf, a negative NaN below -inf.
//
// Stages: the keys of one batch row are cut into chunks of C (1024 for k <= 128,
// 2048 for larger k); one 256-thread workgroup per (chunk, row) sorts its
// chunk's keys in LDS (bitonic network over the next power of two at or above
// the chunk's key count) and keeps the first k; the chunk winners of all chunks
// form the next stage's input, until one chunk remains, whose first k keys are
// the answer.  For k = 1 a max-reduction replaces the sort.  The network moves
// the whole chunk through LDS once per step, so chunks are kept small: LDS
// bandwidth per step, not the step count, sets the time (4096-key chunks on a
// 1024-thread group took ~30 us per stage; 1024-key chunks spread the work over
// four times as many compute units).  Each stage shrinks the candidate count at
// least 8-fold (128256 logits, k = 40: three stages).
#include "qdec_internal.h"

namespace qdec {

namespace {

constexpr int kMaxChunk = 2048;
constexpr int kThreads = 256;

__device__ inline uint64_t topk_key(float v, uint32_t idx)
{
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    if (b == 0x80000000u) b = 0;                                   // -0 ranks as +0
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ inline int32_t key_index(uint64_t key) { return (int32_t)(0xFFFFFFFFu - (uint32_t)key); }

// One stage over `n` inputs per batch row (row b of the grid's y dimension):
// logits[b * n_out + i] when FROM_LOGITS, else keys in[b * n + i], in chunks of
// `chunk` (a power of two <= kMaxChunk).  Writes the chunk's first k keys to
// out[b * out_stride + chunk_index * k + r], or, when FINAL (a single chunk),
// the indices and the logits themselves.  Key 0 pads a chunk past the end of
// the row; it is below every real key.
template <bool FROM_LOGITS, bool FINAL, bool TOP1>
__global__ __launch_bounds__(kThreads) void topk_stage(const float* __restrict__ logits, int64_t n_out,
                                                       const uint64_t* __restrict__ in, int64_t n, int k, int chunk,
                                                       uint64_t* __restrict__ out, int64_t out_stride,
                                                       int32_t* __restrict__ top_idx, float* __restrict__ top_val)
{
    __shared__ uint64_t keys[kMaxChunk];
    const int64_t b = blockIdx.y;
    const int64_t base = (int64_t)blockIdx.x * chunk;
    const int tid = threadIdx.x;
    // sort length: the next power of two holding this chunk's keys (>= 2)
    const int64_t have = n - base < chunk ? n - base : chunk;
    int len = 2;
    while (len < have) len <<= 1;

    uint64_t best = 0;
    for (int t = tid; t < (TOP1 ? chunk : len); t += kThreads) {
        const int64_t i = base + t;
        uint64_t key = 0;
        if (t < have) key = FROM_LOGITS ? topk_key(logits[b * n_out + i], (uint32_t)i) : in[b * n + i];
        if constexpr (TOP1) best = key > best ? key : best;
        else keys[t] = key;
    }
    if constexpr (TOP1) keys[tid] = best;
    __syncthreads();

    if constexpr (TOP1) {
        for (int h = kThreads / 2; h > 0; h >>= 1) {
            if (tid < h) {
                const uint64_t a = keys[tid], c = keys[tid + h];
                keys[tid] = a > c ? a : c;
            }
            __syncthreads();
        }
    } else {
        // bitonic network: blocks of `size` alternate direction so that the
        // final merge (size = len) leaves the whole sequence descending
        for (int size = 2; size <= len; size <<= 1) {
            for (int ls = __builtin_ctz(size) - 1; ls >= 0; --ls) {
                const int stride = 1 << ls;
                for (int p = tid; p < len / 2; p += kThreads) {
                    const int i = ((p >> ls) << (ls + 1)) + (p & (stride - 1));
                    const int j = i + stride;
                    const bool desc = (i & size) == 0 || size == len;
                    const uint64_t a = keys[i], c = keys[j];
                    if ((a < c) == desc) {
                        keys[i] = c;
                        keys[j] = a;
                    }
                }
                __syncthreads();
            }
        }
    }

    for (int r = tid; r < k; r += kThreads) {
        const uint64_t key = r < (TOP1 ? 1 : len) ? keys[r] : 0;
        if constexpr (FINAL) {
            const int32_t idx = key_index(key);
            top_idx[b * k + r] = idx;
            top_val[b * k + r] = logits[b * n_out + idx];   // the logit's own bits (-0 stays -0)
        } else {
            out[b * out_stride + (int64_t)blockIdx.x * k + r] = key;
        }
    }
}

using StageFn = void (*)(const float*, int64_t, const uint64_t*, int64_t, int, int, uint64_t*, int64_t,
                         int32_t*, float*);

template <bool TOP1>
StageFn pick_stage(bool from_logits, bool final_stage)
{
    if (from_logits) return final_stage ? topk_stage<true, true, TOP1> : topk_stage<true, false, TOP1>;
    return final_stage ? topk_stage<false, true, TOP1> : topk_stage<false, false, TOP1>;
}

int chunk_for(int k) { return k <= 128 ? 1024 : kMaxChunk; }

int64_t chunks(int64_t n, int c) { return (n + c - 1) / c; }

}  // namespace

int64_t topk_workspace_bytes(int64_t n_out, int64_t batch, int k)
{
    const int c = chunk_for(k);
    if (chunks(n_out, c) <= 1) return 0;
    return 2 * batch * chunks(n_out, c) * (int64_t)k * (int64_t)sizeof(uint64_t);
}

hipError_t launch_topk(const float* logits, int64_t n_out, int64_t batch, int k, void* workspace,
                       int32_t* top_idx, float* top_val, hipStream_t s)
{
    const int c = chunk_for(k);
    uint64_t* buf[2] = {static_cast<uint64_t*>(workspace), nullptr};
    if (workspace) buf[1] = buf[0] + batch * chunks(n_out, c) * (int64_t)k;
    const uint64_t* in = nullptr;
    int64_t n = n_out;
    bool from_logits = true;
    for (int which = 0;; which ^= 1) {
        const int64_t nch = chunks(n, c);
        const bool final_stage = nch == 1;
        const StageFn fn = k == 1 ? pick_stage<true>(from_logits, final_stage)
                                  : pick_stage<false>(from_logits, final_stage);
        uint64_t* out = final_stage ? nullptr : buf[which];
        hipLaunchKernelGGL(fn, dim3((unsigned)nch, (unsigned)batch), dim3(kThreads), 0, s, logits, n_out, in, n, k, c,
                           out, nch * k, top_idx, top_val);
        count_launch();
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || final_stage) return e;
        in = out;
        n = nch * k;
        from_logits = false;
    }
}

}  // namespace qdec
