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
// Two launches.  Stage 1 (topk_chunks): the keys of one batch row are cut into
// chunks of C (2048, or 4096 / 8192 when the candidate lists would not fit the
// merge); one 256-thread workgroup per (chunk, row) holds its chunk's keys in
// registers and finds its r largest, r = min(k, keys in the chunk), by a
// radix select (radix_select below: the candidates' common leading bits
// skipped, then 8-bit digits most significant first, stopping as soon as the
// kept digit's bin holds exactly the keys still wanted); those keys go to k
// slots of the row's candidate list, the rest padded with key 0 (below every
// real key).  Stage 2 (topk_merge): one workgroup per row runs the same select
// over the row's whole list for its k largest and places each by rank (the
// number of winners above it).  For k = 1 max-reductions replace both
// selects.  A list that would not fit the merge (more than 64 keys per
// thread) takes the staged path below.
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
#include "qdec.h"
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

// The logit of a key: its high word mapped back to the f32 bits, except that
// +0 may have been -0 (which ranks as +0): then the logit itself is read.
__device__ inline float key_logit(uint64_t key, const float* row)
{
    const uint32_t o = (uint32_t)(key >> 32);
    const uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return b == 0 ? row[key_index(key)] : __builtin_bit_cast(float, b);
}

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

int64_t chunks(int64_t n, int64_t c) { return (n + c - 1) / c; }

// ------------------------------------------------------ radix select --
constexpr int kSelThreads = 256;   // 4 waves
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMergeKeys = 64;     // keys per thread in the merge

struct SelState {
    int shift;       // selected keys: key != 0 and (key >> shift) >= prefix
    uint64_t prefix;
};

struct alignas(16) SelShared {
    uint32_t hist[2][kSelWaves][256];   // per digit parity, one histogram per wave
    uint64_t red[2][kSelWaves];
    uint32_t cnt;
};

template <int CTRL, int ROWS>
__device__ __attribute__((always_inline)) inline uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}

template <int CTRL>
__device__ __attribute__((always_inline)) inline uint64_t dpp64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __attribute__((always_inline)) inline uint64_t readlane64(uint64_t v, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Maximum and minimum of u64 values over the workgroup (uniform results):
// within each row of 16 lanes by lane swaps (lane ^ 1, lane ^ 2, the
// half-row and row mirrors), across the wave's 4 rows by lane reads, across
// the waves through LDS.
__device__ __attribute__((always_inline)) inline void wg_maxmin(uint64_t mx, uint64_t mn, SelShared& sh,
                                                                uint64_t* out_max, uint64_t* out_min)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#define QDEC_MAXMIN_STEP(CTRL)                                  \
    {                                                           \
        const uint64_t a = dpp64<CTRL>(mx), c = dpp64<CTRL>(mn); \
        mx = a > mx ? a : mx;                                   \
        mn = c < mn ? c : mn;                                   \
    }
    QDEC_MAXMIN_STEP(0xB1)    // quad_perm 1,0,3,2
    QDEC_MAXMIN_STEP(0x4E)    // quad_perm 2,3,0,1
    QDEC_MAXMIN_STEP(0x141)   // row_half_mirror
    QDEC_MAXMIN_STEP(0x140)   // row_mirror
#undef QDEC_MAXMIN_STEP
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const uint64_t a = readlane64(mx, r), c = readlane64(mn, r);
        mx = a > mx ? a : mx;
        mn = c < mn ? c : mn;
    }
    mx = readlane64(mx, 0);   // uniform: lane 0 now holds the wave's values
    mn = readlane64(mn, 0);
    if (lane == 0) {
        sh.red[0][wave] = mx;
        sh.red[1][wave] = mn;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        mx = sh.red[0][w] > mx ? sh.red[0][w] : mx;
        mn = sh.red[1][w] < mn ? sh.red[1][w] : mn;
    }
    *out_max = mx;
    *out_min = mn;
}

// Exactly r non-zero keys (1 <= r <= the number of non-zero keys held)
// satisfy the returned criterion: the r largest of the keys held by the
// workgroup, key[s] of each thread for s < N; key 0 is padding and never
// counted.  With SKIP the candidates' common leading bits (from their maximum
// and minimum) are skipped first.  Then 8-bit digits, most significant first:
// each wave histograms its candidates' digit in its own LDS copy; after one
// barrier every wave sums the copies, scans them (4 bins a lane, DPP) and
// finds, itself, the bin that holds the r-th largest: the keys in higher
// bins rank above, the bin's keys stay candidates.  It stops once that bin
// holds exactly the keys still wanted.  Histograms alternate between two
// buffers, each wave clearing its own next copy, so one barrier a digit
// suffices.  Every thread calls it; it synchronises the workgroup.
template <bool SKIP, int N>
__device__ __attribute__((always_inline)) SelState radix_select(const uint64_t (&key)[N], int r, SelShared& sh)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int top = 64;
    uint64_t prefix = 0;
    if constexpr (SKIP) {
        uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
        for (int s = 0; s < N; ++s) {
            if (key[s] != 0) {
                kmax = key[s] > kmax ? key[s] : kmax;
                kmin = key[s] < kmin ? key[s] : kmin;
            }
        }
        wg_maxmin(kmax, kmin, sh, &kmax, &kmin);
        if (kmax == kmin) return SelState{0, kmax};   // a single candidate (r = 1)
        top = 64 - __builtin_clzll(kmax ^ kmin);       // bits at and above top are shared
        prefix = top == 64 ? 0 : kmax >> top;
    }
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) sh.hist[0][w][tid] = 0;   // first buffer
    *reinterpret_cast<uint4*>(&sh.hist[1][wave][4 * lane]) = make_uint4(0, 0, 0, 0);
    __syncthreads();
    for (int p = 0;; p ^= 1) {
        const int sft = top > 8 ? top - 8 : 0;
        const uint32_t mask = (1u << (top - sft)) - 1u;
#pragma unroll
        for (int s = 0; s < N; ++s) {
            const bool cand = key[s] != 0 && (top == 64 || (key[s] >> top) == prefix);
            if (cand) atomicAdd(&sh.hist[p][wave][(uint32_t)(key[s] >> sft) & mask], 1u);
        }
        __syncthreads();
        // lane l: bins 255 - 4l - j, j = 0..3 (top down), summed over the waves
        uint32_t c4[4] = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) {
            const uint4 h = *reinterpret_cast<const uint4*>(&sh.hist[p][w][252 - 4 * lane]);
            c4[0] += h.w;
            c4[1] += h.z;
            c4[2] += h.y;
            c4[3] += h.x;
        }
        // this wave's copy for the next digit
        *reinterpret_cast<uint4*>(&sh.hist[p ^ 1][wave][4 * lane]) = make_uint4(0, 0, 0, 0);
        const uint32_t cnt = (c4[0] + c4[1]) + (c4[2] + c4[3]);
        uint32_t incl = cnt;
        incl += dpp<0x111, 0xF>(incl);   // row_shr:1
        incl += dpp<0x112, 0xF>(incl);   // row_shr:2
        incl += dpp<0x114, 0xF>(incl);   // row_shr:4
        incl += dpp<0x118, 0xF>(incl);   // row_shr:8
        incl += dpp<0x142, 0xA>(incl);   // row_bcast:15 into rows 1, 3
        incl += dpp<0x143, 0xC>(incl);   // row_bcast:31 into rows 2, 3
        const uint32_t above_l = incl - cnt;
        const uint64_t hit = __ballot(above_l < (uint32_t)r && (uint32_t)r <= incl);
        const int cl = __builtin_ctzll(hit);   // exactly one lane crosses
        uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)above_l, cl);
        int j = 0;
        uint32_t cb = (uint32_t)__builtin_amdgcn_readlane((int)c4[0], cl);
        while (above + cb < (uint32_t)r) {
            above += cb;
            ++j;
            cb = (uint32_t)__builtin_amdgcn_readlane((int)(j == 1 ? c4[1] : j == 2 ? c4[2] : c4[3]), cl);
        }
        const uint32_t bin = 255u - 4u * (uint32_t)cl - (uint32_t)j;
        prefix = (prefix << (top - sft)) | bin;
        top = sft;
        r -= (int)above;
        if ((int)cb == r || top == 0) {
            __syncthreads();   // the histograms and red are free for the caller
            return SelState{top, prefix};
        }
    }
}

// Appends the keys meeting c to out (positions from a counter in LDS, zero on
// entry, one atomic per wave and slot).
template <int N, typename T>
__device__ __attribute__((always_inline)) inline void compact(const uint64_t (&key)[N], SelState c, uint32_t* cnt,
                                                             T* out)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < N; ++s) {
        const bool take = key[s] != 0 && (key[s] >> c.shift) >= c.prefix;
        const uint64_t m = __ballot(take);
        if (m == 0) continue;
        uint32_t base = 0;
        if (lane == __builtin_ctzll(m)) base = atomicAdd(cnt, (uint32_t)__builtin_popcountll(m));
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, __builtin_ctzll(m));
        if (take) out[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = key[s];
    }
}

// Stage 1: grid (chunks, batch); each workgroup writes its chunk's r largest
// keys (r = min(k, keys in the chunk)) to k slots of the row's list, the
// rest 0.  KPT = chunk / kSelThreads.
template <int KPT, bool TOP1>
__global__ __launch_bounds__(kSelThreads) void topk_chunks(const float* __restrict__ logits, int64_t n_out, int k,
                                                           uint64_t* __restrict__ part)
{
    __shared__ SelShared sh;
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t chunk = (int64_t)KPT * kSelThreads;
    const int64_t base = (int64_t)blockIdx.x * chunk;
    const int have = (int)(n_out - base < chunk ? n_out - base : chunk);
    uint64_t* list = part + (b * gridDim.x + blockIdx.x) * (int64_t)k;
    uint64_t key[KPT];
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
        const int i = tid + s * kSelThreads;
        key[s] = i < have ? topk_key(logits[b * n_out + base + i], (uint32_t)(base + i)) : 0;
    }
    if constexpr (TOP1) {
        uint64_t m = key[0];
#pragma unroll
        for (int s = 1; s < KPT; ++s) m = key[s] > m ? key[s] : m;
        uint64_t mn;
        wg_maxmin(m, m, sh, &m, &mn);
        if (tid == 0) list[0] = m;
    } else {
        const int r = k < have ? k : have;
        if (tid == 0) sh.cnt = 0;
        const SelState c = radix_select<false>(key, r, sh);
        compact(key, c, &sh.cnt, list);
        for (int t = r + tid; t < k; t += kSelThreads) list[t] = 0;
    }
}

// Stage 2: grid (1, batch); the k largest of the row's nchunks * k keys,
// placed by rank (the number of winners above; keys are distinct).  KPT keys
// per thread, a power of two at or above nchunks * k / kSelThreads.
template <bool TOP1, int KPT>
__global__ __launch_bounds__(kSelThreads) void topk_merge(const float* __restrict__ logits, int64_t n_out, int k,
                                                          const uint64_t* __restrict__ part, int nchunks,
                                                          int32_t* __restrict__ top_idx,
                                                          float* __restrict__ top_val)
{
    __shared__ SelShared sh;
    __shared__ uint64_t sel[QDEC_TOPK_MAX];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int total = nchunks * k;   // <= KPT * kSelThreads (chosen on the host)
    const uint64_t* list = part + b * (int64_t)total;
    uint64_t key[KPT];
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
        const int i = tid + s * kSelThreads;
        key[s] = i < total ? list[i] : 0;
    }
    if constexpr (TOP1) {
        uint64_t m = 0;
#pragma unroll
        for (int s = 0; s < KPT; ++s) m = key[s] > m ? key[s] : m;
        uint64_t mn;
        wg_maxmin(m, m, sh, &m, &mn);
        if (tid == 0) {
            top_idx[b] = key_index(m);
            top_val[b] = key_logit(m, logits + b * n_out);   // the logit's own bits (-0 stays -0)
        }
    } else {
        const int k8 = (k + 7) & ~7;   // winners padded with key 0, below every winner
        if (tid == 0) sh.cnt = 0;
        if (tid >= k && tid < k8) sel[tid] = 0;
        const SelState c = radix_select<true>(key, k, sh);
        compact(key, c, &sh.cnt, sel);
        __syncthreads();
        for (int t = tid; t < k; t += kSelThreads) {
            const uint64_t mine = sel[t];
            int rank = 0;
            for (int j = 0; j < k8; j += 8) {
                uint64_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = sel[j + u];
#pragma unroll
                for (int u = 0; u < 8; ++u) rank += v[u] > mine;
            }
            top_idx[b * k + rank] = key_index(mine);
            top_val[b * k + rank] = key_logit(mine, logits + b * n_out);
        }
    }
}

// Keys per thread in stage 1: of 4, 8, 16, 32, the one with the fewest keys
// per thread over both stages (the merge holds a power of two at or above
// chunks * k / kSelThreads, at most kMergeKeys); 0 when none fits the merge.
int merge_kpt(int64_t total)
{
    int m = 1;
    while ((int64_t)m * kSelThreads < total) m *= 2;
    return m;
}

int select_kpt(int64_t n_out, int k)
{
    int best = 0, cost = 0;
    for (int kpt : {4, 8, 16, 32}) {
        const int m = merge_kpt(chunks(n_out, (int64_t)kpt * kSelThreads) * k);
        if (m > kMergeKeys) continue;
        if (!best || kpt + m < cost) {
            best = kpt;
            cost = kpt + m;
        }
    }
    return best;
}

using ChunkFn = void (*)(const float*, int64_t, int, uint64_t*);
using MergeFn = void (*)(const float*, int64_t, int, const uint64_t*, int, int32_t*, float*);

template <bool TOP1, int KPT = 1>
MergeFn pick_merge(int64_t total)
{
    if constexpr (KPT >= kMergeKeys) {
        return topk_merge<TOP1, kMergeKeys>;
    } else {
        return total <= (int64_t)KPT * kSelThreads ? topk_merge<TOP1, KPT> : pick_merge<TOP1, KPT * 2>(total);
    }
}

template <bool TOP1>
ChunkFn pick_chunks(int kpt)
{
    return kpt == 4 ? topk_chunks<4, TOP1> : kpt == 8 ? topk_chunks<8, TOP1>
         : kpt == 16 ? topk_chunks<16, TOP1> : topk_chunks<32, TOP1>;
}

}  // namespace

int64_t topk_workspace_bytes(int64_t n_out, int64_t batch, int k)
{
    const int kpt = select_kpt(n_out, k);
    if (kpt) return batch * chunks(n_out, (int64_t)kpt * kSelThreads) * (int64_t)k * 8;
    const int c = chunk_for(k);
    if (chunks(n_out, c) <= 1) return 0;
    return 2 * batch * chunks(n_out, c) * (int64_t)k * (int64_t)sizeof(uint64_t);
}

hipError_t launch_topk(const float* logits, int64_t n_out, int64_t batch, int k, void* workspace,
                       int32_t* top_idx, float* top_val, hipStream_t s)
{
    const int kpt = select_kpt(n_out, k);
    if (kpt) {
        if (!workspace) return hipErrorInvalidValue;
        uint64_t* part = static_cast<uint64_t*>(workspace);
        const int nch = (int)chunks(n_out, (int64_t)kpt * kSelThreads);
        const ChunkFn f1 = k == 1 ? pick_chunks<true>(kpt) : pick_chunks<false>(kpt);
        hipLaunchKernelGGL(f1, dim3((unsigned)nch, (unsigned)batch), dim3(kSelThreads), 0, s, logits, n_out, k, part);
        count_launch();
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t total = (int64_t)nch * k;
        const MergeFn f2 = k == 1 ? pick_merge<true>(total) : pick_merge<false>(total);
        hipLaunchKernelGGL(f2, dim3(1, (unsigned)batch), dim3(kSelThreads), 0, s, logits, n_out, k, part, nch,
                           top_idx, top_val);
        count_launch();
        return hipGetLastError();
    }
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
