// Device decode attention for one new token ("Module cuda_lane" page,
// try_q4k_soa_attention_device: RoPE on the new q and k, append of k and v to
// the device KV cache, GQA scaled dot-product attention; the O projection after
// it is the Q8_0 GEMV with residual).  The pages name the steps and keep an f32
// KV cache but give no formulas; the ones used:
//   RoPE   : adjacent pairs (x[2i], x[2i+1]) of a head of length d rotate by
//            pos * base^(-2i/d); angle, sine and cosine in f64, the rotated
//            pair rounded once to f32;
//   cache  : f32 [kv_head][max_seq][d], position pos written in place;
//   GQA    : q head h reads kv head h / (n_head / n_kv);
//   output : softmax over t < n_ctx of scale * (q_h . K[t]), times V.
//
// Attention is HBM-bound on the cache (2 * n_ctx * n_kv * d * 4 bytes per
// token), so each workgroup takes one kv head and a chunk of CH = 128 (or,
// up to 2048 positions, 64) positions (flash-decoding split): the G =
// n_head / n_kv query heads of the group share every K and V row it reads.
// 256 / CH threads own a position for the scores (a segment of the K row
// each, streamed as float4, the G query vectors broadcast from LDS), the
// chunk's max and sum come from a wave/LDS reduction, the
// weights go to LDS, and each wave then sums p_t V[t] over a quarter of the
// positions with its lanes across the columns (coalesced V rows), the four
// wave partials meeting in LDS.  Each chunk leaves (max, sum, unnormalised
// output) per head; a second kernel merges the chunks (log-sum-exp).  One
// chunk writes the output directly.
#include "qdec_internal.h"

namespace qdec {

namespace {

// Positions per workgroup: 128 (two threads per position for the scores), or
// 64 (four threads per position) up to 2048 positions, so that short
// contexts still spread over more compute units.
inline int attn_chunk(int64_t n_ctx) { return n_ctx <= 2048 ? 64 : 128; }
constexpr int kMaxGroup = 16;     // query heads per kv head

__global__ __launch_bounds__(64) void rope_append_kernel(float* q, float* k, const float* v, int64_t n_head,
                                                         int64_t d, int64_t pos, double log2_base,
                                                         float* k_cache, float* v_cache, int64_t max_seq)
{
    const int64_t hh = blockIdx.x;
    const bool is_q = hh < n_head;
    const int64_t kvh = hh - n_head;
    float* x = is_q ? q + hh * d : k + kvh * d;
    for (int64_t i = threadIdx.x; i < d / 2; i += blockDim.x) {
        const double ang = (double)pos * exp2(-2.0 * (double)i / (double)d * log2_base);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const double a = x[2 * i], b = x[2 * i + 1];
        const float ra = (float)(a * cs - b * sn), rb = (float)(a * sn + b * cs);
        x[2 * i] = ra;
        x[2 * i + 1] = rb;
        if (!is_q) {
            float* kc = k_cache + (kvh * max_seq + pos) * d;
            kc[2 * i] = ra;
            kc[2 * i + 1] = rb;
            const float* vv = v + kvh * d;
            float* vc = v_cache + (kvh * max_seq + pos) * d;
            vc[2 * i] = vv[2 * i];
            vc[2 * i + 1] = vv[2 * i + 1];
        }
    }
}

__device__ inline float block_reduce(float v, float* red, bool is_max)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();                          // red may still be read from the previous reduction
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
}

// The same reduction for NG values at once (one pair of barriers for all the
// query heads of a group); red holds 4 x kMaxGroup floats.  Per value the
// order of operations is that of block_reduce.
template <int NG>
__device__ inline void block_reduce_n(float (&v)[NG], float* red, bool is_max)
{
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float o = __shfl_xor(v[g], off);
            v[g] = is_max ? fmaxf(v[g], o) : v[g] + o;
        }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int g = 0; g < NG; ++g) red[w * kMaxGroup + g] = v[g];
    __syncthreads();
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float r0 = red[g], r1 = red[kMaxGroup + g], r2 = red[2 * kMaxGroup + g], r3 = red[3 * kMaxGroup + g];
        v[g] = is_max ? fmaxf(fmaxf(r0, r1), fmaxf(r2, r3)) : (r0 + r1) + (r2 + r3);
    }
}

// Partial attention of one (chunk, kv head).  part layout per (kv, chunk, g):
// [max, sum, o[0..D)].  FINAL (a single chunk): out = o / sum directly.
// Scores: position p = tid / TPP of the chunk, segment tid % TPP of the d
// columns per thread, the segments added across the TPP neighbouring lanes
// (TPP = 256 / CH threads per position).  Weighted sum: wave w
// takes positions w, w+4, ...; lane l takes columns D/64 * l ..; the four
// wave partials meet in LDS.  G > 0: the group size (query heads per kv
// head) is fixed at compile time, so every loop over the heads unrolls without
// branches and the LDS reads of a step issue together; G = 0 takes it from
// `group` (any size up to kMaxGroup), with a branch per head and step (at 24
// query / 8 kv heads that form measured 18.6 us at 1024 positions, bound by
// the serialised LDS round trips of its four waves).
typedef __attribute__((address_space(3))) void lds_void;

template <int D, bool FINAL, int G, int CH>
__global__ __launch_bounds__(256) void attn_chunk_kernel(const float* __restrict__ q, const float* __restrict__ k_cache,
                                                         const float* __restrict__ v_cache, int64_t n_kv, int group_rt,
                                                         int64_t n_ctx, int64_t max_seq, float scale,
                                                         float* __restrict__ part, float* __restrict__ out)
{
    constexpr int TPP = 256 / CH, SEG = D / TPP;   // threads per position, d columns per thread (scores)
    constexpr int GM = G > 0 ? G : kMaxGroup;     // unrolled head loops
    constexpr int CPR = D / 4;                     // 16-byte chunks per K row
    constexpr int RPI = 64 / CPR;                  // K rows per wave DMA instruction
    constexpr int QD = CH / (4 * RPI);             // K DMA instructions per wave
    constexpr int OWF = 4 * kMaxGroup * D;                   // the wave partials (floats)
    constexpr int KL = CH * D > OWF + kMaxGroup * CH ? CH * D : OWF + kMaxGroup * CH;
    const int group = G > 0 ? G : group_rt;
    __shared__ __attribute__((aligned(16))) float qs[kMaxGroup * D];
    __shared__ float red[4];
    __shared__ float redn[4 * kMaxGroup];
    __shared__ float mx[kMaxGroup], sm[kMaxGroup];
    // the chunk's K rows (scores), then the weights p and the four waves'
    // partial outputs (written only after every K read: the softmax barriers
    // lie between)
    __shared__ __attribute__((aligned(1024))) float kl[KL];
    auto ow = reinterpret_cast<float (*)[kMaxGroup][D]>(kl);
    auto ps = reinterpret_cast<float (*)[CH]>(kl + OWF);
    const int64_t chunk = blockIdx.x, kv = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nchunks = gridDim.x;
    // the group's query vectors (heads kv*group .. +group) go to LDS by DMA
    // ahead of everything else; the wait for the K rows below covers them,
    // so no load round trip precedes the cache stream
    {
        const float* qsrc = q + (kv * group) * D;
        const int nq4 = group * D / 4;   // 16-byte pieces
        for (int base = __builtin_amdgcn_readfirstlane(wave) * 64; base < nq4; base += 256)
            if (base + lane < nq4)
                __builtin_amdgcn_global_load_lds(qsrc + (base + lane) * 4, (lds_void*)(qs + base * 4), 16, 0, 0);
    }

    const int pl = tid / TPP, seg = tid % TPP;
    const int64_t t = chunk * CH + pl;
    const bool valid = t < n_ctx;
    const int64_t tbase = chunk * CH;
    const int tn = (int)(n_ctx - tbase < CH ? n_ctx - tbase : CH);
    // every load of the workgroup is issued before any arithmetic waits on one:
    // the chunk's K rows into LDS, whole rows per instruction (rows past n_ctx
    // repeat the last; lane l of an instruction lands at 16-byte slot l % CPR
    // of its row and carries the row's chunk (l % CPR) ^ (row % CPR), so that
    // the per-position reads below hit every bank once), then this wave's V
    // rows (used after the softmax)
    {
        const float* kbase = k_cache + kv * max_seq * D;
#pragma unroll
        for (int qi = 0; qi < QD; ++qi) {
            const int row = (wave * QD + qi) * RPI + lane / CPR;
            int64_t tk = tbase + row;
            tk = tk < n_ctx ? tk : n_ctx - 1;
            const int c = (lane % CPR) ^ (row % CPR);
            __builtin_amdgcn_global_load_lds(kbase + tk * D + c * 4, (lds_void*)(kl + (wave * QD + qi) * 256), 16, 0,
                                             0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // V: wave w takes positions w + 4k; each load covers RPV of them, whole
    // rows, 16 bytes (4 columns) a lane
    constexpr int VPW = CH / 4;                   // positions per wave in the weighted sum
    constexpr int LPR = D / 4;                    // lanes per V row
    constexpr int RPV = 64 / LPR;                 // V rows per load
    constexpr int VI = VPW / RPV;                 // V loads per lane
    const int vrow = lane / LPR, vcol = 4 * (lane % LPR);
    const float* vbase = v_cache + (kv * max_seq + tbase) * D + vcol;
    float4 vr[VI];
#pragma unroll
    for (int i = 0; i < VI; ++i) {
        const int tt = wave + 4 * (RPV * i + vrow);
        const int ts = tt < tn ? tt : tn - 1;     // in bounds; weight 0 past tn
        vr[i] = *reinterpret_cast<const float4*>(vbase + (int64_t)ts * D);
    }
    __builtin_amdgcn_sched_barrier(0);
    // this wave's K rows have landed once at most its V loads remain; the
    // barrier makes every wave's rows visible
    static_assert(VI < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VI & 15) | ((VI >> 4) << 14) | 0x70 | 0xF00);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    float4 kr[SEG / 4];
#pragma unroll
    for (int j4 = 0; j4 < SEG / 4; ++j4) {
        const int c = seg * (SEG / 4) + j4;
        kr[j4] = *reinterpret_cast<const float4*>(kl + pl * D + (c ^ (pl % CPR)) * 4);
    }
    float s[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) s[g] = 0.0f;
    {
#pragma unroll
        for (int j4 = 0; j4 < SEG / 4; ++j4) {
            const float4 kk = kr[j4];
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                if (G > 0 || g < group) {
                    const float4 qq = *reinterpret_cast<const float4*>(&qs[g * D + seg * SEG + 4 * j4]);
                    s[g] = __builtin_fmaf(qq.x, kk.x, s[g]);
                    s[g] = __builtin_fmaf(qq.y, kk.y, s[g]);
                    s[g] = __builtin_fmaf(qq.z, kk.z, s[g]);
                    s[g] = __builtin_fmaf(qq.w, kk.w, s[g]);
                }
            }
        }
    }
    if constexpr (G > 0) {
        float sc[G], m[G], l[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float full = s[g];
#pragma unroll
            for (int o = 1; o < TPP; o <<= 1) full += __shfl_xor(full, o);
            sc[g] = valid ? full * scale : -INFINITY;
            m[g] = sc[g];
        }
        block_reduce_n<G>(m, redn, true);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            sc[g] = valid ? expf(sc[g] - m[g]) : 0.0f;   // the weight p
            l[g] = seg == 0 ? sc[g] : 0.0f;
        }
        block_reduce_n<G>(l, redn, false);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (seg == 0) ps[g][pl] = sc[g];
            if (tid == 0) {
                mx[g] = m[g];
                sm[g] = l[g];
            }
        }
    } else {
        for (int g = 0; g < group; ++g) {
            float full = s[g];
#pragma unroll
            for (int o = 1; o < TPP; o <<= 1) full += __shfl_xor(full, o);
            const float sc = valid ? full * scale : -INFINITY;
            const float m = block_reduce(sc, red, true);
            const float p = valid ? expf(sc - m) : 0.0f;
            const float l = block_reduce(seg == 0 ? p : 0.0f, red, false);
            if (seg == 0) ps[g][pl] = p;
            if (tid == 0) {
                mx[g] = m;
                sm[g] = l;
            }
        }
    }
    __syncthreads();

    // weighted sum of V over this wave's positions (rows already in registers;
    // positions past tn have weight 0)
    float o[GM][4];
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int c = 0; c < 4; ++c) o[g][c] = 0.0f;
#pragma unroll
    for (int i = 0; i < VI; ++i) {
        const int tt = wave + 4 * (RPV * i + vrow);
        const float vv[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (G > 0 || g < group) {
                const float p = tt < tn ? ps[g][tt] : 0.0f;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[g][c] = __builtin_fmaf(p, vv[c], o[g][c]);
            }
        }
    }
    // the RPV lane groups of the wave hold the same columns: add them
#pragma unroll
    for (int g = 0; g < GM; ++g)
        if (G > 0 || g < group)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int off = LPR; off < 64; off <<= 1) o[g][c] += __shfl_xor(o[g][c], off);
    if (lane < LPR) {
#pragma unroll
        for (int g = 0; g < GM; ++g)
            if (G > 0 || g < group)
#pragma unroll
                for (int c = 0; c < 4; ++c) ow[wave][g][vcol + c] = o[g][c];
    }
    __syncthreads();
    for (int u = tid; u < group * D; u += 256) {
        const int g = u / D, j = u % D;
        const float ot = (ow[0][g][j] + ow[1][g][j]) + (ow[2][g][j] + ow[3][g][j]);
        if constexpr (FINAL) {
            out[(kv * group + g) * D + j] = ot / sm[g];
        } else {
            float* pr = part + ((kv * nchunks + chunk) * group + g) * (D + 2);
            pr[2 + j] = ot;
            if (j == 0) {
                pr[0] = mx[g];
                pr[1] = sm[g];
            }
        }
    }
}

// Merge of the chunk partials of one query head (log-sum-exp): the chunk
// maxima and sums are read in parallel (one chunk per thread, strided), each
// chunk's weight exp(m_c - m) and weighted sum l_c exp(m_c - m) kept in LDS,
// then each thread sums its column over the chunks in chunk order.  The
// column values of the first PF chunks (PF <= nchunks, chosen by the
// launcher) are loaded together with the maxima, before the maximum is known,
// so up to PF chunks cost one memory round trip instead of three (maxima;
// maxima and sums again; columns).  (A variant
// with 256 threads splitting the chunks four ways and an exp per chunk and
// thread measured slower, and so did a one-pass merge with a running maximum
// (two exponentials per chunk in one dependent chain per thread: 26 -> 42 us
// at 64 chunks).)
template <int D, int PF>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float* __restrict__ part, int64_t nchunks, int group,
                                                         float* __restrict__ out)
{
    __shared__ float wsh[1024];   // exp(m_c - m) of chunk c
    __shared__ float wl[1024];    // l_c exp(m_c - m)
    __shared__ float red[4];
    const int64_t h = blockIdx.x;
    const int64_t kv = h / group, g = h % group;
    const int j = threadIdx.x;
    auto at = [&](int64_t c) { return part + ((kv * nchunks + c) * group + g) * (D + 2); };
    float op[PF > 0 ? PF : 1];
    {
        const float* p = at(0) + 2 + j;   // per-lane address: a vector pointer step per chunk
        const int64_t step = (int64_t)group * (D + 2);
#pragma unroll
        for (int c = 0; c < PF; ++c, p += step) op[c] = *p;
    }
    // (m, l) of chunk j (8-byte aligned: D + 2 is even)
    const float2 ml0 = j < nchunks ? *reinterpret_cast<const float2*>(at(j)) : make_float2(-INFINITY, 0.0f);
    float m = ml0.x;
    for (int64_t c = j + D; c < nchunks; c += D) m = fmaxf(m, at(c)[0]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((j & 63) == 0) red[j >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < D / 64; ++w) m = fmaxf(m, red[w]);
    float l = 0.0f, o = 0.0f;
    for (int64_t c0 = 0; c0 < nchunks; c0 += 1024) {
        const int64_t cn = nchunks - c0 < 1024 ? nchunks - c0 : 1024;
        __syncthreads();                                   // wsh of the previous block is consumed
        int64_t cj = j;
        if (c0 == 0) {   // chunk j: (m, l) already loaded
            if (j < cn) {
                const float wv = expf(ml0.x - m);
                wsh[j] = wv;
                wl[j] = ml0.y * wv;
            }
            cj += D;
        }
        for (; cj < cn; cj += D) {
            const float2 ml = *reinterpret_cast<const float2*>(at(c0 + cj));
            const float wv = expf(ml.x - m);
            wsh[cj] = wv;
            wl[cj] = ml.y * wv;
        }
        __syncthreads();
        for (int64_t c = 0; c < cn; ++c) l += wl[c];
        int64_t c = 0;
        if (c0 == 0) {   // cn >= PF here
#pragma unroll
            for (int q = 0; q < PF; ++q) o = __builtin_fmaf(op[q], wsh[q], o);
            c = PF;
        }
        // the chunk sums come from LDS, so the loop below issues only the
        // vector loads of o: 16 in flight (8: one more round trip per 8
        // chunks; 32: slower again, measured)
#pragma unroll 16
        for (; c < cn; ++c) o = __builtin_fmaf(at(c0 + c)[2 + j], wsh[c], o);
    }
    out[h * D + j] = o / l;
}

using ChunkFn = void (*)(const float*, const float*, const float*, int64_t, int, int64_t, int64_t, float, float*,
                        float*);

// Compile-time group sizes for the usual GQA ratios; others take the generic
// kernel.
template <int D, bool FINAL, int CH>
ChunkFn pick_group(int group)
{
    switch (group) {
        case 1: return attn_chunk_kernel<D, FINAL, 1, CH>;
        case 2: return attn_chunk_kernel<D, FINAL, 2, CH>;
        case 3: return attn_chunk_kernel<D, FINAL, 3, CH>;
        case 4: return attn_chunk_kernel<D, FINAL, 4, CH>;
        case 6: return attn_chunk_kernel<D, FINAL, 6, CH>;
        case 8: return attn_chunk_kernel<D, FINAL, 8, CH>;
        default: return attn_chunk_kernel<D, FINAL, 0, CH>;
    }
}

using CombineFn = void (*)(const float*, int64_t, int, float*);

// Combine kernel prefetching the first pf chunks (pf <= nchunks).
template <int D>
CombineFn pick_combine(int pf)
{
    switch (pf) {
        case 64: return attn_combine_kernel<D, 64>;
        case 32: return attn_combine_kernel<D, 32>;
        case 16: return attn_combine_kernel<D, 16>;
        case 8: return attn_combine_kernel<D, 8>;
        default: return attn_combine_kernel<D, 0>;
    }
}

template <int D, bool FINAL>
ChunkFn pick_chunk(int group, int ch)
{
    return ch == 64 ? pick_group<D, FINAL, 64>(group) : pick_group<D, FINAL, 128>(group);
}

}  // namespace

int64_t attention_workspace_bytes(int64_t n_head, int64_t head_dim, int64_t n_ctx)
{
    const int ch = attn_chunk(n_ctx);
    const int64_t nchunks = (n_ctx + ch - 1) / ch;
    return nchunks > 1 ? n_head * nchunks * (head_dim + 2) * 4 : 0;
}

hipError_t launch_rope_append(float* q, float* k, const float* v, int64_t n_head, int64_t n_kv, int64_t d, int64_t pos,
                              double base, float* k_cache, float* v_cache, int64_t max_seq, hipStream_t s)
{
    hipLaunchKernelGGL(rope_append_kernel, dim3((unsigned)(n_head + n_kv)), dim3(64), 0, s, q, k, v, n_head, d, pos,
                       log2(base), k_cache, v_cache, max_seq);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_attention(const float* q, const float* k_cache, const float* v_cache, int64_t n_head, int64_t n_kv,
                            int64_t d, int64_t n_ctx, int64_t max_seq, float scale, float* out, void* workspace,
                            hipStream_t s)
{
    const int group = (int)(n_head / n_kv);
    const int ch = attn_chunk(n_ctx);
    const int64_t nchunks = (n_ctx + ch - 1) / ch;
    const dim3 grid((unsigned)nchunks, (unsigned)n_kv);
    float* part = static_cast<float*>(workspace);
    const bool final = nchunks == 1;
    const ChunkFn fn = d == 64 ? (final ? pick_chunk<64, true>(group, ch) : pick_chunk<64, false>(group, ch))
                               : (final ? pick_chunk<128, true>(group, ch) : pick_chunk<128, false>(group, ch));
    hipLaunchKernelGGL(fn, grid, dim3(256), 0, s, q, k_cache, v_cache, n_kv, group, n_ctx, max_seq, scale, part, out);
    count_launch();
    if (final) return hipGetLastError();
    const int pf = nchunks >= 64 ? 64 : nchunks >= 32 ? 32 : nchunks >= 16 ? 16 : nchunks >= 8 ? 8 : 0;
    const CombineFn cf = d == 64 ? pick_combine<64>(pf) : pick_combine<128>(pf);
    hipLaunchKernelGGL(cf, dim3((unsigned)n_head), dim3((unsigned)d), 0, s, part, nchunks, group, out);
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
