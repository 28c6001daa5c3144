// Batched prefill-shaped GEMM on gfx950 MFMA.
//
// What is computed (rustdoc source view of weight_cache.rs, try_cuda_batch_gemv
// and its doc comment): for each of `batch` packed rows of hidden (n_in wide),
// out[b][i] = sum_j W[i][j] * x[b][j], i.e. C[m x n] = A[m x k] * B[k x n] with
// m = batch, k = n_in, n = n_out and B = W transposed.  That page pads every
// dimension to a multiple of 16 with zeros and trims the result; here the tile
// loads zero-fill past the edges and the stores are predicated, which is the
// same product.
//
// Precision: both operands are rounded to bf16 (round to nearest even) and
// contracted on v_mfma_f32_16x16x32_bf16 with f32 accumulation.  The Q8_0
// weight is first dequantised exactly in f32 (d*q), then rounded.  The pages
// record that f16 tensor-core operands gave unusable results on their
// single-token path; bf16 keeps the f32 exponent range, and the error per
// product is at most about 2*2^-9 relative.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of C over a slice
// of K; each of its four waves computes 64 x 64 with 4 x 4 MFMA 16x16x32
// tiles.  K advances 64 at a time (two Q8_0 blocks).  Both operands are staged
// in LDS as bf16 rows (K contiguous, padded by 8 elements against bank
// conflicts), double-buffered: the global loads of step k+1 are in flight
// while step k runs on MFMA.
//
// Parallelism: with few output tiles (the prefill batch is 128 or 512 rows) K
// is split into S slices so that the grid has at least one workgroup per CU;
// the slices add their partial tiles into the output with fire-and-forget f32
// atomics (a fill kernel zeroes the output first).  Each atomic costs far more
// than a store, so S stays at the smallest value that fills the CUs.  Block
// ids go to the XCDs round-robin, which spreads the m-tiles that share a
// weight tile over all L2s (measured faster than grouping consecutive tiles
// on one XCD).
#include "qdec_internal.h"

namespace qdec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;  // LDS row stride in bf16 elements (144 bytes)

struct GemmArgs {
    const float* x;        // M x K f32
    const int8_t* q;       // Q8_0 q plane (N x K) or nullptr
    const uint16_t* d;     // Q8_0 d plane (N x K/32)
    const float* wf;       // dense f32 W (N x K) or nullptr
    float* out;            // M x N f32
    int64_t M, N, K;
    int64_t mtiles, ntiles;
    int64_t kslice;        // K per split (multiple of BK)
    int splits;
    float* part;           // splits > 1: slice s writes part[s][M][N] (workspace), or null: atomics into a zeroed out
};

__device__ inline float fp16_bits_to_f32(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, sizeof v);
    return static_cast<float>(v);
}

__device__ inline bf16x4 to_bf16x4(float4 v)
{
    bf16x4 r;
    r[0] = (__bf16)v.x;
    r[1] = (__bf16)v.y;
    r[2] = (__bf16)v.z;
    r[3] = (__bf16)v.w;
    return r;
}

// Global -> register staging of one 128 x 64 f32 tile (rows r0.., cols k0..):
// 2048 float4, 8 per thread, consecutive threads on consecutive float4s.
__device__ inline void load_f32_tile(const float* __restrict__ src, int64_t rows, int64_t K,
                                     int64_t kend, int64_t r0, int64_t k0, float4 (&reg)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx >> 4, c4 = idx & 15;
        const int64_t gr = r0 + row, gk = k0 + c4 * 4;
        reg[i] = (gr < rows && gk < kend) ? *reinterpret_cast<const float4*>(src + gr * K + gk)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

__device__ inline void store_f32_tile(__bf16* lds, const float4 (&reg)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx >> 4, c4 = idx & 15;
        *reinterpret_cast<bf16x4*>(lds + row * LDK + c4 * 4) = to_bf16x4(reg[i]);
    }
}

// Q8_0 weight tile: 128 rows x 64 q bytes; thread t takes row t/2, block t%2
// (32 weights = two 16-byte loads) and that block's fp16 scale.
struct QTileReg {
    uint4 q0, q1;
    uint16_t d;
};

__device__ inline void load_q8_tile(const GemmArgs& a, int64_t kend, int64_t n0, int64_t k0, QTileReg& reg)
{
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int64_t gn = n0 + row, gk = k0 + half * 32;
    if (gn < a.N && gk < kend) {
        const uint4* p = reinterpret_cast<const uint4*>(a.q + gn * a.K + gk);
        reg.q0 = p[0];
        reg.q1 = p[1];
        reg.d = a.d[gn * (a.K >> 5) + (gk >> 5)];
    } else {
        reg.q0 = make_uint4(0, 0, 0, 0);
        reg.q1 = reg.q0;
        reg.d = 0;
    }
}

__device__ inline void store_q8_tile(__bf16* lds, const QTileReg& reg)
{
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    const float d = fp16_bits_to_f32(reg.d);
    const uint32_t w[8] = {reg.q0.x, reg.q0.y, reg.q0.z, reg.q0.w, reg.q1.x, reg.q1.y, reg.q1.z, reg.q1.w};
    __bf16* dst = lds + row * LDK + half * 32;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bf16x8 v;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t word = w[2 * k + (t >> 2)];
            v[t] = (__bf16)(d * (float)(int8_t)((word >> (8 * (t & 3))) & 0xff));
        }
        *reinterpret_cast<bf16x8*>(dst + 8 * k) = v;
    }
}

template <bool QUANT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) __bf16 As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][BN * LDK];

    // block id -> (k slice, n tile, m tile), k fastest
    const int64_t id = blockIdx.x;
    const int64_t slice = id % a.splits;
    const int64_t tile = id / a.splits;
    const int64_t n0 = (tile % a.ntiles) * BN;
    const int64_t m0 = (tile / a.ntiles) * BM;
    const int64_t kbeg = slice * a.kslice;
    const int64_t kend = kbeg + a.kslice < a.K ? kbeg + a.kslice : a.K;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    float4 xr[8];
    float4 wr[8];
    QTileReg qr;
    const int64_t nk = (kend - kbeg + BK - 1) / BK;

    load_f32_tile(a.x, a.M, a.K, kend, m0, kbeg, xr);
    if (QUANT) load_q8_tile(a, kend, n0, kbeg, qr);
    else load_f32_tile(a.wf, a.N, a.K, kend, n0, kbeg, wr);
    store_f32_tile(As[0], xr);
    if (QUANT) store_q8_tile(Bs[0], qr);
    else store_f32_tile(Bs[0], wr);
    __syncthreads();

    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < nk;
        if (more) {
            const int64_t k0 = kbeg + (kt + 1) * BK;
            load_f32_tile(a.x, a.M, a.K, kend, m0, k0, xr);
            if (QUANT) load_q8_tile(a, kend, n0, k0, qr);
            else load_f32_tile(a.wf, a.N, a.K, kend, n0, k0, wr);
        }
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 af[4], bfr[4];
            const int koff = ks * 32 + (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm * 64 + i * 16 + (lane & 15)) * LDK + koff]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn * 64 + j * 16 + (lane & 15)) * LDK + koff]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            store_f32_tile(As[cur ^ 1], xr);
            if (QUANT) store_q8_tile(Bs[cur ^ 1], qr);
            else store_f32_tile(Bs[cur ^ 1], wr);
        }
        __syncthreads();
    }

    // D layout of the 16x16 MFMA: lane holds column (lane % 16) and rows
    // 4*(lane / 16) + 0..3.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 64 + j * 16 + (lane & 15);
            if (n >= a.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
                if (m >= a.M) continue;
                if (a.splits == 1) a.out[m * a.N + n] = acc[i][j][e];
                else if (a.part) a.part[(slice * a.M + m) * a.N + n] = acc[i][j][e];
                else unsafeAtomicAdd(a.out + m * a.N + n, acc[i][j][e]);
            }
        }
    }
}

// ----------------------------------------------------------- pipelined --
// Q8_0 GEMM for grids that fill the chip without K splits (>= 256 tiles of
// 128 x 128, K % 64 == 0, n_out % 8 == 0).  The register-staged kernel above
// waits a full memory latency every 64 k (one K step of prefetch); here every
// operand streams global->LDS by DMA (global_load_lds, 16 bytes a lane) into a
// ring of P = 4 super-stages of 64 k, so three super-stages are in flight
// while one is consumed:
//   x  : bf16 rows (rounded once into the workspace by x_to_bf16), 128 bytes
//        of a row per 8 lanes, chunk c of row r stored at c ^ (r & 7) against
//        LDS bank conflicts;
//   W  : raw int8 rows, 64 bytes each;
//   d  : the block-major scale plane, one 16-byte load per lane covering two
//        blocks x 128 rows.
// Each 32-k compute stage dequantises its W half-tile from LDS into one of
// three bf16 buffers (two stages ahead of the MFMAs that read it), loads the
// A and B fragments of the next stage while the current stage's MFMAs run,
// and ends with one barrier.  The scheduling fences interleave LDS reads,
// MFMAs and the dequantisation VALU work; all waits on the DMA counter are
// explicit (vmcnt counts whole super-stages of PER instructions).
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline void dma16(const void* g, lds_void* l) { __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0); }

template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

struct PipeArgs {
    const __bf16* xb;      // M x K bf16 (workspace)
    const int8_t* q;       // N x K
    const uint16_t* dT;    // (K/32) x N
    float* out;            // M x N
    int64_t M, N, K, ntiles;
    int64_t kslice;        // K per split (multiple of 64)
    int splits;            // > 1: slice s writes its partial tiles to part[s][M][N]
    float* part;           // splits * M * N f32 (workspace), summed by sum_slices
};

__global__ __launch_bounds__(256) void x_to_bf16(const float4* __restrict__ x, bf16x4* __restrict__ xb, int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) xb[i] = to_bf16x4(x[i]);
}

constexpr int kPipeStages = 4;

#define QDEC_RING(name, type, n)                                                                        \
    __shared__ __attribute__((aligned(1024))) type name##0[n], name##1[n], name##2[n], name##3[n]
#define QDEC_PICK(name, u) ((u) == 0 ? name##0 : (u) == 1 ? name##1 : (u) == 2 ? name##2 : name##3)

__global__ __launch_bounds__(256) void gemm_q8_pipe(PipeArgs a)
{
    constexpr int PBM = 128, PBN = 128, P = kPipeStages;
    constexpr int WGN = 2, NWAVE = 4, TM = 4, TN = 4;          // 2 x 2 waves of 64 x 64
    constexpr int XI = PBM * 128 / 1024, XPW = XI / NWAVE;    // x: 8 rows x 128 B per instruction
    constexpr int WI = PBN * 64 / 1024, WPW = WI / NWAVE;     // W: 16 rows x 64 B per instruction
    constexpr int PER = XPW + WPW + 1;                         // DMA instructions per super-stage and wave
    static_assert(XI % NWAVE == 0 && WI % NWAVE == 0 && PBN * 4 <= 1024, "tile split");
    QDEC_RING(XR, __bf16, PBM * 64);
    QDEC_RING(WR, int8_t, PBN * 64);
    QDEC_RING(DR, uint16_t, 512);
    __shared__ __attribute__((aligned(1024))) __bf16 WB0[PBN * 32], WB1[PBN * 32], WB2[PBN * 32];

    // block id -> (k slice, n tile, m tile), k fastest
    const int64_t id = blockIdx.x;
    const int64_t slice = id % a.splits, tile = id / a.splits;
    const int64_t n0 = (tile % a.ntiles) * PBN, m0 = (tile / a.ntiles) * PBM;
    const int64_t kbeg = slice * a.kslice;
    const int64_t klen = kbeg + a.kslice < a.K ? a.kslice : a.K - kbeg;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int nk = (int)(klen >> 5);  // 32-k compute stages of this slice
    const int ns = nk >> 1;           // 64-k super-stages

    // x rows: instruction i of this wave covers tile rows 8(wave*XPW + i) ..+7;
    // lane -> row + lane/8, its 16 bytes land at LDS chunk lane%8, which holds
    // global chunk (lane%8) ^ (row & 7)
    const __bf16* xsrc[XPW];
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
        const int r = 8 * (wave * XPW + i) + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        int64_t gr = m0 + r;
        gr = gr < a.M ? gr : a.M - 1;                          // edge rows repeat the last row
        xsrc[i] = a.xb + gr * a.K + kbeg + c * 8;
    }
    int wi[WPW];
    const int8_t* wsrc[WPW];
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
        wi[i] = wave * WPW + i;
        const int r = wi[i] * 16 + (lane >> 2);
        int64_t gn = n0 + r;
        gn = gn < a.N ? gn : a.N - 1;
        wsrc[i] = a.q + gn * a.K + kbeg + (lane & 3) * 16;
    }
    // scales: lane l < 32 loads 8 rows of block 2s + l/16 (rows 8(l%16)..); lanes
    // 32..63 repeat the load into the unused upper half of the slot
    const int dl = lane & 31;
    const int dblk = dl >> 4, drow = (dl & 15) * 8;
    int64_t gdr = n0 + drow;
    gdr = gdr + 8 <= a.N ? gdr : a.N - 8;                     // n_out % 8 == 0: only whole groups past the edge
    const uint16_t* dsrc = a.dT + (kbeg / 32 + dblk) * a.N + gdr;

    auto issue = [&](int st, int slot) {
        const int sc = st < ns ? st : ns - 1;                  // past the end: reload the last super-stage
        __bf16* xd = QDEC_PICK(XR, slot);
        int8_t* wd = QDEC_PICK(WR, slot);
        uint16_t* dd = QDEC_PICK(DR, slot);
#pragma unroll
        for (int i = 0; i < XPW; ++i) dma16(xsrc[i] + (int64_t)sc * 64, (lds_void*)(xd + (wave * XPW + i) * 512));
#pragma unroll
        for (int i = 0; i < WPW; ++i) dma16(wsrc[i] + (int64_t)sc * 64, (lds_void*)(wd + wi[i] * 1024));
        dma16(dsrc + (int64_t)(2 * sc) * a.N, (lds_void*)dd);
    };
    auto wbuf = [&](int k) -> __bf16* { return k == 0 ? WB0 : k == 1 ? WB1 : WB2; };
    // dequantisation: thread t takes row t/2 and 16 weights (half t%2) of the
    // 32-k half of the super-stage
    const int wr = threadIdx.x >> 1, wh = threadIdx.x & 1;
    auto dequant = [&](int t, int slot, int wbk) {
        __bf16* wb = wbuf(wbk);
        const int h2 = t & 1;
        const uint4 qv = *reinterpret_cast<const uint4*>(QDEC_PICK(WR, slot) + wr * 64 + h2 * 32 + wh * 16);
        const float dd = fp16_bits_to_f32(QDEC_PICK(DR, slot)[h2 * PBN + wr]);
        const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (__bf16)(dd * (float)(int8_t)((w[2 * h + (e >> 2)] >> (8 * (e & 3))) & 0xff));
            const int c = (wh * 2 + h) ^ ((wr >> 1) & 3);
            *reinterpret_cast<bf16x8*>(&wb[wr * 32 + c * 8]) = v;
        }
    };
    bf16x8 fa[2][TM], fb[2][TN];
    auto frags = [&](int t, int slot, int wbk, int f) {
        const __bf16* xs = QDEC_PICK(XR, slot);
        const __bf16* wb = wbuf(wbk);
        const int h2 = t & 1;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = (wm * TM + i) * 16 + (lane & 15);
            const int c = (h2 * 4 + (lane >> 4)) ^ (r & 7);
            fa[f][i] = *reinterpret_cast<const bf16x8*>(&xs[r * 64 + c * 8]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int r = (wn * TN + j) * 16 + (lane & 15);
            const int c = (lane >> 4) ^ ((r >> 1) & 3);
            fb[f][j] = *reinterpret_cast<const bf16x8*>(&wb[r * 32 + c * 8]);
        }
    };
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: super-stages 0..P-2 in flight; 0 and 1 landed
#pragma unroll
    for (int st = 0; st < P - 1; ++st) issue(st, st);
    wait_vm<PER * (P - 3)>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    dequant(0, 0, 0);
    dequant(1, 0, 1);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the bf16 tiles are written
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    frags(0, 0, 0, 0);
    // compute stage t (u = t mod 24, so every ring index is a compile-time constant)
    auto body = [&](const int t, const int u) {
        if ((u & 1) == 0) issue(t / 2 + P - 1, (u / 2 + P - 1) % P);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[u & 1][i], fb[u & 1][j], acc[i][j], 0, 0, 0);
        dequant(t + 2, ((u + 2) / 2) % P, (u + 2) % 3);
        frags(t + 1, ((u + 1) / 2) % P, (u + 1) % 3, (u + 1) & 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // LDS reads of the dequantisation
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);        // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);  // fragment reads
#pragma unroll
        for (int k = 0; k < TM * TN - 2; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);    // VALU between MFMAs
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);        // LDS writes
        // end of stage t: super-stage (t+3)/2 must have landed
        if ((u & 1) == 0) wait_vm<PER * (P - 2)>();
        else wait_vm<PER * (P - 3)>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    int t0 = 0;
    for (; t0 + 24 <= nk; t0 += 24) {
#pragma unroll
        for (int u = 0; u < 24; ++u) body(t0 + u, u);
    }
#pragma unroll
    for (int u = 0; u < 24; ++u)
        if (t0 + u < nk) body(t0 + u, u);
    wait_vm<0>();   // no DMA may still be writing LDS when the workgroup ends

#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + (wn * TN + j) * 16 + (lane & 15);
            if (n >= a.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + (wm * TM + i) * 16 + (lane >> 4) * 4 + e;
                if (m >= a.M) continue;
                if (a.splits == 1) a.out[m * a.N + n] = acc[i][j][e];
                else a.part[(slice * a.M + m) * a.N + n] = acc[i][j][e];
            }
        }
    }
}

// out = sum over the K slices of their partial products, slice 0 first (a
// fixed order: the split result is reproducible, unlike atomic adds).
__global__ __launch_bounds__(256) void sum_slices(const float* __restrict__ part, int splits, int64_t mn,
                                                  float* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = mn / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 t = reinterpret_cast<const float4*>(part)[i];
        for (int sl = 1; sl < splits; ++sl) {
            const float4 u = reinterpret_cast<const float4*>(part + sl * mn)[i];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
        }
        reinterpret_cast<float4*>(out)[i] = t;
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += stride) {
        float t = part[i];
        for (int sl = 1; sl < splits; ++sl) t += part[sl * mn + i];
        out[i] = t;
    }
}

#undef QDEC_RING
#undef QDEC_PICK

// The pipelined kernel holds 124 KB of LDS, so one workgroup per CU: its grid
// should be whole rounds of 256 workgroups.  K splits (slices >= 512 deep and
// multiples of 64) bring small grids up; each slice writes its M*N partial
// products to the workspace and a small kernel sums them (f32 atomics into a
// zeroed output cost ~12 us per 4M), up to 4M partial values.  Up to 4
// splits the grid must reach 256 workgroups; the 8-way split is also taken at
// 192 (three quarters of a round, one workgroup per CU).  Measured:
// 128x8192x3072 split 4: 32.0 us (36.1 unpipelined); 512x8192x3072: 52.7 us
// (74.5); 128x3072x8192 split 8 (192 workgroups, 3.1M atomics): 30.1 us
// against 36.3 unpipelined; 512x3072x8192 split 4 (6.3M atomics, 1.5
// rounds): 84 us against 70.5 unpipelined, and split 2 (192 workgroups):
// 72.3, so neither is taken.
int pipe_splits(int64_t M, int64_t N, int64_t K)
{
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    int s = 1;
    while (s < 8 && tiles * s < 256 && K % (64 * 2 * s) == 0 && K / (2 * s) >= 512) s *= 2;
    return s;
}

bool pipe_ok(int64_t M, int64_t N, int64_t K)
{
    if (K % 64 != 0 || N % 8 != 0 || N < 128) return false;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    const int s = pipe_splits(M, N, K);
    const int64_t wg = tiles * s;
    const int64_t rounds = (wg + 255) / 256;
    const bool full = (wg >= 256 || (s == 8 && wg >= 192)) && 4 * wg >= 3 * rounds * 256;   // >= 75% of the last round busy
    return full && (s == 1 || M * N * s <= (int64_t)1 << 22);
}

__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, int64_t n4, float* __restrict__ tail,
                                                   int64_t ntail)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < ntail) tail[t] = 0.f;
}

// Grid plan: K slices so that tiles * slices reaches 256 workgroups (one per
// CU), each slice at least 512 deep (8 K steps) and a multiple of BK.
GemmArgs plan(int64_t M, int64_t N, int64_t K)
{
    GemmArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.mtiles = (M + BM - 1) / BM;
    a.ntiles = (N + BN - 1) / BN;
    const int64_t tiles = a.mtiles * a.ntiles;
    int splits = 1;
    while (tiles * splits < 256 && K / (splits * 2) >= 512) splits *= 2;
    a.kslice = ((K + splits - 1) / splits + BK - 1) / BK * BK;
    a.splits = (int)((K + a.kslice - 1) / a.kslice);
    return a;
}

hipError_t launch(GemmArgs& a, bool quant, hipStream_t s)
{
    if (a.splits > 1 && !a.part) {
        const int64_t n = a.M * a.N;
        const int64_t n4 = n / 4;
        const int64_t ntail = n - n4 * 4;
        int64_t blocks = (n4 + 255) / 256;
        if (blocks > 2048) blocks = 2048;
        if (blocks < 1) blocks = 1;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<float4*>(a.out), n4, a.out + n4 * 4, ntail);
        count_launch();
    }
    const dim3 grid((unsigned)(a.mtiles * a.ntiles * a.splits));
    if (quant) hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, dim3(256), 0, s, a);
    count_launch();
    if (a.splits > 1 && a.part) {
        const int64_t mn = a.M * a.N;
        int64_t sb = (mn / 4 + 255) / 256;
        if (sb > 2048) sb = 2048;
        if (sb < 1) sb = 1;
        hipLaunchKernelGGL(sum_slices, dim3((unsigned)sb), dim3(256), 0, s, a.part, a.splits, mn, a.out);
        count_launch();
    }
    return hipGetLastError();
}

// Register-staged path: the slices' partial products (none without a K split).
int64_t reg_part_bytes(int64_t M, int64_t N, int64_t K)
{
    const GemmArgs a = plan(M, N, K);
    return a.splits > 1 ? (int64_t)a.splits * M * N * 4 : 0;
}

}  // namespace

// x rounded to bf16, then (with a K split) the slices' partial products.
static int64_t pipe_x_bytes(int64_t n_in, int64_t batch) { return align_up(batch * n_in * 2, kAlign); }

int64_t q8_gemm_workspace_bytes(int64_t n_in, int64_t n_out, int64_t batch)
{
    if (!pipe_ok(batch, n_out, n_in)) return reg_part_bytes(batch, n_out, n_in);
    const int s = pipe_splits(batch, n_out, n_in);
    return pipe_x_bytes(n_in, batch) + (s > 1 ? (int64_t)s * batch * n_out * 4 : 0);
}

int64_t f32_gemm_workspace_bytes(int64_t n_in, int64_t n_out, int64_t batch)
{
    return reg_part_bytes(batch, n_out, n_in);
}

hipError_t launch_q8_0_gemm(Q8View w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                            float* out, void* workspace, hipStream_t s)
{
    if (workspace && pipe_ok(batch, n_out, n_in)) {
        const int64_t n4 = batch * n_in / 4;   // n_in % 64 == 0
        int64_t blocks = (n4 + 255) / 256;
        if (blocks > 2048) blocks = 2048;
        hipLaunchKernelGGL(x_to_bf16, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(x),
                           static_cast<bf16x4*>(workspace), n4);
        count_launch();
        PipeArgs p{};
        p.xb = static_cast<const __bf16*>(workspace);
        p.q = w.q;
        p.dT = w.dT;
        p.out = out;
        p.M = batch;
        p.N = n_out;
        p.K = n_in;
        p.ntiles = (n_out + 127) / 128;
        p.splits = pipe_splits(batch, n_out, n_in);
        p.kslice = n_in / p.splits;
        p.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + pipe_x_bytes(n_in, batch));
        const int64_t grid = ((batch + 127) / 128) * p.ntiles * p.splits;
        hipLaunchKernelGGL(gemm_q8_pipe, dim3((unsigned)grid), dim3(256), 0, s, p);
        count_launch();
        if (p.splits > 1) {
            const int64_t mn = batch * n_out;
            int64_t sb = (mn / 4 + 255) / 256;
            if (sb > 2048) sb = 2048;
            if (sb < 1) sb = 1;
            hipLaunchKernelGGL(sum_slices, dim3((unsigned)sb), dim3(256), 0, s, p.part, p.splits, mn, out);
            count_launch();
        }
        return hipGetLastError();
    }
    GemmArgs a = plan(batch, n_out, n_in);
    a.x = x;
    a.q = w.q;
    a.d = w.d;
    a.out = out;
    // a workspace given for a shape off the pipelined path holds the slices'
    // partial products (q8_gemm_workspace_bytes sized it)
    a.part = workspace && a.splits > 1 && !pipe_ok(batch, n_out, n_in) ? static_cast<float*>(workspace) : nullptr;
    return launch(a, true, s);
}

hipError_t launch_f32_gemm(const float* wf, int64_t n_in, int64_t n_out, int64_t batch,
                           const float* x, float* out, void* workspace, hipStream_t s)
{
    GemmArgs a = plan(batch, n_out, n_in);
    a.x = x;
    a.wf = wf;
    a.out = out;
    a.part = workspace && a.splits > 1 ? static_cast<float*>(workspace) : nullptr;
    return launch(a, false, s);
}

}  // namespace qdec
