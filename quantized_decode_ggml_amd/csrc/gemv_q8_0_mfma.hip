// Q8_0 GEMV for 3..8 batch rows on the matrix cores (gfx950 MFMA), plain,
// residual, fused QKV and fused SwiGLU.  Same results as the VALU kernels to
// the f32 tolerance; used when the batch makes those VALU-bound (each weight
// then costs one multiply-add per batch row on 16-lane SIMDs).  Two kernels:
// at widths 1024, 2048, 3072 and 4096 an integer matrix-core kernel that
// keeps whole rows in one workgroup (see "integer matrix cores" below); at
// the other widths the bf16 kernel described here.
//
// What is computed is unchanged (rustdoc "Module cuda_lane", Functions
// section): out[b][i] = sum_j (d*q)[i][j] x[b][j] with the epilogues of the
// fused variants.  How:
//
// * x is split exactly into three bf16 parts, x = hi + mid + lo: hi keeps the
//   top 16 bits of the f32 pattern, mid the top 16 bits of x - hi, and
//   lo = (x - hi) - mid, whose 8 significant bits fit bf16 exactly.  Both
//   subtractions are exact (each removes a leading bit prefix), so the parts
//   sum to x with no rounding for every x whose lo part is a normal number
//   (|x| above about 2^-100).
// * The parts of all batch rows are stacked as the MFMA A rows, row
//   v = p*batch + b, so 3*batch rows fill NV = 1 (batch <= 5) or 2 fragments
//   of 16 rows.
// * q is an integer in [-127, 127], exact in bf16, so each product q * part
//   is exact in f32.  One v_mfma_f32_16x16x32_bf16 per Q8_0 block (32 k) and
//   fragment gives, for 16 weight rows, P = sum_k q * part in f32 for every
//   stacked row; the block's fp16 scale is applied in f32 afterwards,
//   acc += d * P, so the scale multiplies an exact integer-weighted sum.
// * The three part sums of a batch row are added at the end,
//   (hi + mid) + lo.
// Rounding: at most 31 roundings inside each MFMA sum, one per block in the
// scale-and-accumulate chain (NBW <= 32 blocks per slice), 2 for the parts,
// one per K slice after the first (at most 31) and one for the residual:
// below 100 units of 2^-24 of sum_j |w x|, i.e. under 6e-6, inside the 1e-5
// bound.
//
// Operands per MFMA (16x16x32): A = an x-split fragment, lane l holding
// stacked row l % 16 and k = 8*(l/16)..+8 of the block; B = the weight
// fragment, lane l holding weight row l % 16 and the same 8 k (8 int8
// bytes); the result D[v][r] lands in lane r + 16*(v/4), element v % 4.  So
// every lane scales its results with the one d of its own weight row.
//
// Layout of the work: the weights come from the fragment-tiled copy (one
// contiguous 512-byte tile per 16 rows x 32 k, scales alongside), so every
// wave load is contiguous.  A workgroup is four waves, one 16-row group each
// (x 2 matrices for SwiGLU), over one K slice of NBW blocks; all four share
// the x fragments of that slice, which the workgroup builds once in LDS: every
// thread loads 8 values of one batch row, splits them and writes the three
// parts' fragments.  The x loads go out first, then each wave's first D
// blocks of weight loads, and the split is computed while those fly (the
// in-order load counter lets a wave wait for x alone).  A wave then streams
// its NBW blocks in straight-line code, D blocks ahead, reading each block's
// A fragments from LDS one block ahead.  With one slice per row (a grid
// large enough without a K split) the workgroup stores the rows itself;
// otherwise each writes its slice's sums to the workspace and a second launch
// adds the slices in slice order and applies the epilogue (residual, QKV
// routing, SwiGLU): at most 31 more roundings, in a fixed order, so every
// result is bitwise reproducible.  (Two earlier designs: a separate launch
// that split x into the workspace, every wave reading its fragments from L2
// (x traffic 2-4x the weight bytes at 6-8 rows); and a K split whose slices
// were added with f32 atomics, or merged by the last workgroup of a row set
// behind a device-scope release fence, which writes back the whole L2.)
#include <cstdio>
#include <string>

#include "gemv_common.h"

namespace qdec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kParts = 3;

constexpr int kWaves = 4;   // row groups (one per wave) of a workgroup
constexpr int kDepth = 6;   // blocks a wave keeps in flight ahead of the one computed

// x = hi + mid + lo (see above): the top 16 bits of each part's f32 pattern.
__device__ inline void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t h = u & 0xffff0000u;
    const float r1 = x - __builtin_bit_cast(float, h);       // exact
    const uint32_t m = __builtin_bit_cast(uint32_t, r1) & 0xffff0000u;
    const float r2 = r1 - __builtin_bit_cast(float, m);      // exact, 8 significant bits
    hi = h >> 16;
    mid = m >> 16;
    lo = __builtin_bit_cast(uint32_t, r2) >> 16;
}

// 8 int8 weights -> 8 bf16 (exact).
__device__ inline bf16x8 q8_to_bf16(u32x2 w)
{
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)(float)(int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xff);
    return r;
}

// Where the tiles of the row groups live: segment k of the flat row space
// (QKV: q, k, v; SwiGLU: gate, up over the same rows) starts at tile byte
// offset tq[k] and scale element offset td[k] from segment 0; flat group G
// belongs to segment (G >= gend0) + (G >= gend1).
struct TileArgs {
    const int8_t* q0;
    const uint16_t* d0;
    int64_t tq1, tq2, td1, td2;
    int64_t gend0, gend1, groups;
    int64_t nb;
    int ksplit;   // K slices (workgroups) per row set
    float* part;  // ksplit > 1: per (set, slice) the slice's sums, kWaves x NM x batch x 16 floats
};

// Tile and scale pointers of matrix m of flat 16-row group G (clamped to the
// last group by the caller), at block blk0, for lane `lane`.
template <int MODE>
__device__ inline void group_tiles(const TileArgs& t, int64_t G, int m, int64_t blk0, int lane, const int8_t*& tq,
                                   const uint16_t*& td)
{
    const int64_t tile_stride = t.nb * 512, dtile_stride = t.nb * 16;
    int64_t oq, od, local;
    if constexpr (MODE == kSwiGLU) {
        oq = m ? t.tq1 : 0;
        od = m ? t.td1 : 0;
        local = G;
    } else {
        const int64_t s1 = G >= t.gend0, s2 = G >= t.gend1;   // 0 or 1, uniform
        oq = (s1 - s2) * t.tq1 + s2 * t.tq2;
        od = (s1 - s2) * t.td1 + s2 * t.td2;
        local = G - s1 * t.gend0 - s2 * (t.gend1 - t.gend0);
    }
    tq = t.q0 + oq + local * tile_stride + blk0 * 512 + 8 * lane;
    td = t.d0 + od + local * dtile_stride + blk0 * 16 + (lane & 15);
}

// The stacked A rows: virtual row v = p * batch + b holds part p of x[b]
// (3 * batch rows); fragment f covers rows 16f .. 16f + 15, and lane l of a
// fragment holds row 16f + l % 16 at k = 8 (l / 16) .. + 7 of its block.
// Rows past 3 * batch are left unwritten: a result row of the MFMA depends on
// its own A row only, and those results are never read.
template <int MODE, int NBW, int NV>
__global__ __launch_bounds__(kWaves * 64) void q8_0_gemv_mfma(Q8GemvArgs a, TileArgs t)
{
    constexpr int NM = (MODE == kSwiGLU) ? 2 : 1;
    constexpr int D = kDepth < NBW ? kDepth : NBW;
    constexpr int RS = D + 1;                                   // register ring slots
    constexpr int NT = kWaves * 64;
    constexpr int XSLOTS = NBW * NV * 64;                       // 16-byte x fragment slots
    constexpr int FIN = kWaves * NM * NV * 16 * 16;             // floats of the epilogue exchange
    constexpr int LBYTES = XSLOTS * 16 > FIN * 4 ? XSLOTS * 16 : FIN * 4;
    constexpr int IPT = (8 * NBW * 4 + NT - 1) / NT;            // x items per thread at batch 8
    __shared__ __attribute__((aligned(16))) char lds[LBYTES];
    u32x4* xl = reinterpret_cast<u32x4*>(lds);

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g4 = lane >> 4;
    const int64_t set = blockIdx.x / t.ksplit;
    const int kp = (int)(blockIdx.x % t.ksplit);
    const int64_t blk0 = (int64_t)kp * NBW;

    // x item (b, i, o): the 8 values of batch row b at k = 32 (blk0 + i) + 8 o,
    // loaded before any weight so that they do not queue behind the stream
    const int items = a.batch * NBW * 4;
    float4 xv[IPT][2];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = (int)threadIdx.x + j * NT;
        if (it < items) {
            const int b = it / (NBW * 4), io = it % (NBW * 4);
            const float4* src = reinterpret_cast<const float4*>(a.x + (int64_t)b * a.n_in + blk0 * 32 + io * 8);
            xv[j][0] = src[0];
            xv[j][1] = src[1];
        }
    }

    // this wave's row group: tile and scale pointers of its first block
    const int8_t* tq[NM];
    const uint16_t* td[NM];
    {
        int64_t G = set * kWaves + w;
        G = G < t.groups ? G : t.groups - 1;                  // loads stay in bounds
#pragma unroll
        for (int m = 0; m < NM; ++m) group_tiles<MODE>(t, G, m, blk0, lane, tq[m], td[m]);
    }
    u32x2 wq[RS][NM];
    uint16_t wd[RS][NM];
    auto issue = [&](int i, int slot) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            wq[slot][m] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tq[m] + i * 512));
            wd[slot][m] = __builtin_nontemporal_load(td[m] + i * 16);
        }
    };
#pragma unroll
    for (int i = 0; i < D; ++i) issue(i, i);
    asm volatile("" ::: "memory");

    // the split fragments of the slice, written while the weight loads fly
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = (int)threadIdx.x + j * NT;
        if (it < items) {
            const int b = it / (NBW * 4), io = it % (NBW * 4), i = io >> 2, o = io & 3;
            const float v8[8] = {xv[j][0].x, xv[j][0].y, xv[j][0].z, xv[j][0].w,
                                 xv[j][1].x, xv[j][1].y, xv[j][1].z, xv[j][1].w};
            uint32_t h[kParts][8];
#pragma unroll
            for (int e = 0; e < 8; ++e) split3(v8[e], h[0][e], h[1][e], h[2][e]);
#pragma unroll
            for (int p = 0; p < kParts; ++p) {
                const int v = p * a.batch + b;
                xl[(i * NV + (v >> 4)) * 64 + (v & 15) + 16 * o] =
                    u32x4{h[p][0] | (h[p][1] << 16), h[p][2] | (h[p][3] << 16), h[p][4] | (h[p][5] << 16),
                          h[p][6] | (h[p][7] << 16)};
            }
        }
    }
    __syncthreads();   // LDS only: the weight loads stay in flight

    f32x4 acc[NM][NV];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int f = 0; f < NV; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 af[2][NV];
#pragma unroll
    for (int f = 0; f < NV; ++f) af[0][f] = xl[f * 64 + lane];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        if (i + D < NBW) issue(i + D, (i + D) % RS);
        if (i + 1 < NBW) {
#pragma unroll
            for (int f = 0; f < NV; ++f) af[(i + 1) & 1][f] = xl[((i + 1) * NV + f) * 64 + lane];
        }
        const int s = i % RS;
        // Opaque from here on: without this the compiler hoists the unpacking
        // of a prefetched block next to its load, and every step then waits
        // for the load it has just issued.
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            asm volatile("" : "+v"(wq[s][m]));
            asm volatile("" : "+v"(wd[s][m]));
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const bf16x8 bw = q8_to_bf16(wq[s][m]);
            const float dsc = fp16_bits_to_f32(wd[s][m]);
#pragma unroll
            for (int f = 0; f < NV; ++f) {
                const f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i & 1][f]), bw,
                                                                        f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[m][f][e] = __builtin_fmaf(dsc, P[e], acc[m][f][e]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the block pipeline in program order
    }

    // D[v][r]: lane r + 16 (v % 16 / 4), element v % 4 of fragment v / 16; the
    // three parts of batch row b sit at v = b, batch + b, 2 batch + b
    __syncthreads();   // every wave is done with the x fragments
    float* fin = reinterpret_cast<float*>(lds) + w * (NM * NV * 256);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int f = 0; f < NV; ++f)
#pragma unroll
            for (int e = 0; e < 4; ++e) fin[(m * NV * 16 + 16 * f + 4 * g4 + e) * 16 + (lane & 15)] = acc[m][f][e];
    __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's LDS writes done (the wave reads only its own)
    __builtin_amdgcn_wave_barrier();
    const int r = lane & 15;
    auto part_sum = [&](int m, int b) {
        const float* q = fin + m * NV * 256;
        return (q[b * 16 + r] + q[(a.batch + b) * 16 + r]) + q[(2 * a.batch + b) * 16 + r];
    };
    if (t.ksplit > 1) {
        // this slice's sums; sum_slices_kernel adds the slices in order
        float* mine = t.part + ((set * t.ksplit + kp) * kWaves + w) * (int64_t)(NM * a.batch * 16);
        for (int b = g4; b < a.batch; b += 4)
#pragma unroll
            for (int m = 0; m < NM; ++m) mine[(m * a.batch + b) * 16 + r] = part_sum(m, b);
    } else {
        const int64_t row = (set * kWaves + w) * 16 + r;
        if (row < a.total_rows)
            for (int b = g4; b < a.batch; b += 4) store_row<MODE>(a, row, b, part_sum(0, b), part_sum(NM - 1, b));
    }
}

// Output (b, row) of a K-split product: the slices' sums in slice order, then
// the epilogue.  One thread per output, rows fastest.  Every slice's sum is
// loaded before the first add (a load-add loop would wait out one memory
// latency per slice).
constexpr int kMaxSlices = 32;   // n_in <= 8192 in slices of at least 8 blocks

template <int MODE>
__global__ __launch_bounds__(256) void sum_slices_kernel(Q8GemvArgs a, const float* __restrict__ part, int ksplit)
{
    constexpr int NM = (MODE == kSwiGLU) ? 2 : 1;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)a.batch * a.total_rows) return;
    const int b = (int)(t / a.total_rows);
    const int64_t row = t % a.total_rows;
    const int64_t g = row >> 4, set = g / kWaves;
    const int w = (int)(g % kWaves), r = (int)(row & 15);
    const int64_t per = (int64_t)kWaves * NM * a.batch * 16;
    const float* p = part + set * ksplit * per + ((int64_t)w * NM * a.batch + b) * 16 + r;
    float v[NM][kMaxSlices];
#pragma unroll
    for (int k = 0; k < kMaxSlices; ++k)
#pragma unroll
        for (int m = 0; m < NM; ++m) v[m][k] = k < ksplit ? p[k * per + m * a.batch * 16] : 0.f;
    float s[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        s[m] = v[m][0];
#pragma unroll
        for (int k = 1; k < kMaxSlices; ++k)
            if (k < ksplit) s[m] += v[m][k];
    }
    store_row<MODE>(a, row, b, s[0], s[NM - 1]);
}

// ------------------------------------------- integer matrix cores --
// The same products for widths up to 4096 with the whole K of a row inside
// one workgroup (one launch, no slice sums), on v_mfma_i32_16x16x32_i8.
// x enters as a 30-bit fixed-point number per (batch row, Q8_0 block):
// X = trunc(x * 2^(30 - e)), |x| < 2^e over the block's 32 values, so
// x = X 2^(e - 30) + eps, |eps| < 2^(e - 30) <= 2^-29 max |x| of the block
// (zero for every value within 2^6 of the block's largest).  X is written as
// four signed base-256 digits (the bytes of X + 0x80808080, each less 0x80).
// A fragment of the A operand stacks 4 batch rows x 4 digits as its 16 rows,
// row 4 (b % 4) + j; the B operand is the tile's 8 int8 weights of the lane
// as they stand.  One MFMA per block and fragment gives in exact int32
// D_j = sum_k q_k a_j,k for batch row b and weight row n in lane
// n + 16 (b % 4), elements j = 0..3; the lane forms
// u = (256 D3 + D2) 2^16 + (256 D1 + D0) (each bracket below 2^27, exact in
// f32 up to 2^24 and rounded once above; the fma rounds once) and
// accumulates d * (u 2^(e - 30)), the power of two exact.  Against the bf16
// split: no int8 -> bf16 conversion (17 instructions a block and matrix) and
// 4 bytes of A operand per x value instead of 6, so a workgroup holds the A
// operands of a whole row in LDS (batch x n_in x 4 bytes: 96 KB at 8 x 3072)
// and no K slice leaves the workgroup.
// A workgroup is RG 16-row groups (x 2 matrices for SwiGLU), each with its K
// over KS waves of T blocks.  Every thread loads its x items and waits for
// them (behind the grid's weight requests they would land late), then every
// weight load of its wave is issued, and while those fly the workgroup
// writes the A fragments and the exponents.  The KS wave sums of an output
// are added in wave order through LDS; then the epilogue.  A non-finite x
// makes every output of its batch row NaN.
// Rounding: per block at most 2 in u and 1 in the accumulation, KS - 1 for
// the wave sums, 1 for the residual; with T <= 16 below 60 units of 2^-24 of
// sum_j |w x|, plus the truncation of x above.
template <int MODE, int KS, int T, int NV, int RG>
__global__ __launch_bounds__(64 * KS * RG) void q8_0_gemv_i8(Q8GemvArgs a, TileArgs t)
{
    static_assert(KS * RG <= 16 && T % 4 == 0 && NV >= 1 && NV <= 2, "KS * RG waves, T blocks a wave");
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    constexpr int NM = (MODE == kSwiGLU) ? 2 : 1;
    constexpr int NB = KS * T;                          // Q8_0 blocks of a row
    constexpr int NW = KS * RG;
    constexpr int NT = 64 * NW;
    constexpr int XB = NB * NV * 512;                   // A fragments
    constexpr int RB = NW * NM * NV * 64 * 4;           // wave sums, after the products
    constexpr int LB = XB > RB ? XB : RB;
    constexpr int IPT = (4 * NV * NB * 4 + NT - 1) / NT;   // x items (8 values) a thread
    __shared__ __attribute__((aligned(16))) char lds[LB];
    __shared__ __attribute__((aligned(16))) int xe[4 * NV][NB];   // e - 30 per (batch row, block)
    __shared__ uint32_t wbad[NW];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = w / KS, kw = w % KS;
    const int64_t Gw = (int64_t)blockIdx.x * RG + rg;
    const int64_t G = Gw < t.groups ? Gw : t.groups - 1;     // a spare wave reads the last group
    const int64_t blk0 = (int64_t)kw * T;

    // x item it = (b, blk, g), g fastest: values 32 blk + 8 g .. +7 of batch row b
    const int items = a.batch * NB * 4;
    float4 xv[IPT][2];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = (int)threadIdx.x + j * NT;
        if (it < items) {
            const float4* src =
                reinterpret_cast<const float4*>(a.x + (int64_t)(it / (NB * 4)) * a.n_in) + 2 * (it % (NB * 4));
            xv[j][0] = src[0];
            xv[j][1] = src[1];
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    asm volatile("" ::: "memory");
    // every weight load of this wave
    const int8_t* tq[NM];
    const uint16_t* td[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) group_tiles<MODE>(t, G, m, blk0, lane, tq[m], td[m]);
    u32x2 wq[T][NM];
    uint16_t wd[T][NM];
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            wq[i][m] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tq[m] + i * 512));
            wd[i][m] = __builtin_nontemporal_load(td[m] + i * 16);
        }
    asm volatile("" ::: "memory");

    // A fragments: lane (m, g) of fragment (blk, f) reads the 8 bytes at
    // ((blk NV + f) 64 + 16 g + (m ^ (blk % 16))) * 8 -- digit m % 4 of
    // batch row 4 f + m / 4 at k = 8 g .. 8 g + 7 of block blk.  The XOR is a
    // permutation inside each 16-lane group (the reads stay conflict-free);
    // it spreads the writes, where the lanes of a wave hold 16 blocks x 4
    // k-groups of one digit row, over all LDS banks (unswizzled they hit two).
    u32x2* xf = reinterpret_cast<u32x2*>(lds);
    uint32_t badm = 0;   // bit b: a non-finite x in batch row b
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = (int)threadIdx.x + j * NT;
        if (it < items) {   // the 4 lanes of a block agree
            const int b = it / (NB * 4), blk = (it >> 2) % NB, g = it & 3;
            float v[8] = {xv[j][0].x, xv[j][0].y, xv[j][0].z, xv[j][0].w,
                          xv[j][1].x, xv[j][1].y, xv[j][1].z, xv[j][1].w};
            uint32_t amax = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = max(amax, __builtin_bit_cast(uint32_t, v[e]) & 0x7fffffffu);
            // over the block's 4 items (4 consecutive lanes): lane ^ 1, lane ^ 2
            amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0xB1, 0xF, 0xF, false));
            amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x4E, 0xF, 0xF, false));
            const bool fin = amax < 0x7f800000u;
            if (__builtin_amdgcn_ballot_w64(!fin) != 0) {
                // rare: a non-finite block converts zeros (its row's outputs
                // are NaN; an infinity or NaN has no defined int conversion)
                badm |= fin ? 0u : 1u << b;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = fin ? v[e] : 0.0f;
            }
            // amax = m 2^e with 0.5 <= m < 1, so every |x| < 2^e (e = 0 for zeros)
            const int ex = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, amax));
            uint32_t y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (uint32_t)(int)__builtin_amdgcn_ldexpf(v[e], 30 - ex) + 0x80808080u;
            // word dj of each half: digit dj of its 4 values
            uint32_t dg[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t t01l = __builtin_amdgcn_perm(y[4 * h + 1], y[4 * h], 0x05010400u);
                const uint32_t t01h = __builtin_amdgcn_perm(y[4 * h + 1], y[4 * h], 0x07030602u);
                const uint32_t t23l = __builtin_amdgcn_perm(y[4 * h + 3], y[4 * h + 2], 0x05010400u);
                const uint32_t t23h = __builtin_amdgcn_perm(y[4 * h + 3], y[4 * h + 2], 0x07030602u);
                dg[h][0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u) ^ 0x80808080u;
                dg[h][1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u) ^ 0x80808080u;
                dg[h][2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u) ^ 0x80808080u;
                dg[h][3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u) ^ 0x80808080u;
            }
            u32x2* frag = xf + (blk * NV + (b >> 2)) * 64 + 16 * g;
#pragma unroll
            for (int dj = 0; dj < 4; ++dj) frag[(4 * (b & 3) + dj) ^ (blk & 15)] = u32x2{dg[0][dj], dg[1][dj]};
            if (g == 0) xe[b][blk] = ex - 30;
        }
    }
    uint32_t wm = 0;
#pragma unroll
    for (int b = 0; b < 4 * NV; ++b)
        if (__builtin_amdgcn_ballot_w64(((badm >> b) & 1u) != 0) != 0) wm |= 1u << b;
    if (lane == 0) wbad[w] = wm;
    __syncthreads();   // LDS only: the weight loads stay in flight
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) bad |= wbad[k];

    // lane (n = lane % 16, b' = lane / 16) of fragment f: batch row 4 f + b'.
    // Up to 16 blocks a wave the exponents are read once into registers;
    // longer waves read each block's from LDS where it is used.
    constexpr bool EBL = T > 16;
    int eb[NV][EBL ? 1 : T];
    if constexpr (!EBL) {
#pragma unroll
        for (int f = 0; f < NV; ++f)
#pragma unroll
            for (int q = 0; q < T / 4; ++q) {
                const int4 e4 = *reinterpret_cast<const int4*>(&xe[4 * f + (lane >> 4)][blk0 + 4 * q]);
                eb[f][4 * q] = e4.x;
                eb[f][4 * q + 1] = e4.y;
                eb[f][4 * q + 2] = e4.z;
                eb[f][4 * q + 3] = e4.w;
            }
    }
    float acc[NM][NV];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int f = 0; f < NV; ++f) acc[m][f] = 0.0f;
    const u32x2* xw = xf + blk0 * NV * 64;
#pragma unroll
    for (int i = 0; i < T; ++i) {
        const int sl = lane ^ (int)((blk0 + i) & 15);
        u32x2 A[NV];
#pragma unroll
        for (int f = 0; f < NV; ++f) A[f] = xw[(i * NV + f) * 64 + sl];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const float dsc = fp16_bits_to_f32(wd[i][m]);
#pragma unroll
            for (int f = 0; f < NV; ++f) {
                const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, A[f]),
                                                                      __builtin_bit_cast(long, wq[i][m]),
                                                                      i32x4{0, 0, 0, 0}, 0, 0, 0);
                const float u =
                    __builtin_fmaf((float)(D[3] * 256 + D[2]), 65536.0f, (float)(D[1] * 256 + D[0]));
                const int e = EBL ? xe[4 * f + (lane >> 4)][blk0 + i] : eb[f][EBL ? 0 : i];
                acc[m][f] = __builtin_fmaf(dsc, __builtin_amdgcn_ldexpf(u, e), acc[m][f]);
            }
        }
    }

    // the KS wave sums of each output in wave order, then the epilogue
    __syncthreads();   // every wave is done with the A fragments
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int f = 0; f < NV; ++f) red[((w * NM + m) * NV + f) * 64 + lane] = acc[m][f];
    __syncthreads();
    if (kw != 0) return;
    const int64_t row = Gw * 16 + (lane & 15);
#pragma unroll
    for (int f = 0; f < NV; ++f) {
        float sm[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            sm[m] = red[(((rg * KS) * NM + m) * NV + f) * 64 + lane];
#pragma unroll
            for (int k = 1; k < KS; ++k) sm[m] += red[((((rg * KS + k) * NM) + m) * NV + f) * 64 + lane];
        }
        const int b = 4 * f + (lane >> 4);
        if (b < a.batch && Gw < t.groups && row < a.total_rows) {
            const float nan = __builtin_nanf("");
            const bool nb_ = (bad >> b) & 1u;
            store_row<MODE>(a, row, b, nb_ ? nan : sm[0], nb_ ? nan : sm[NM - 1]);
        }
    }
}

using MfmaFn = void (*)(Q8GemvArgs, TileArgs);

// x fragments per block: the 3 * batch stacked part rows in groups of 16
inline int frags_for(int64_t batch) { return (int)((3 * batch + 15) / 16); }

template <int MODE, int NV>
MfmaFn pick_nbw(int nbw)
{
    switch (nbw) {
        case 8: return q8_0_gemv_mfma<MODE, 8, NV>;
        case 16: return q8_0_gemv_mfma<MODE, 16, NV>;
        case 24: return q8_0_gemv_mfma<MODE, 24, NV>;
        case 32: return q8_0_gemv_mfma<MODE, 32, NV>;
        default: return nullptr;
    }
}

template <int MODE>
MfmaFn pick_mfma(int nbw, int nv)
{
    return nv == 1 ? pick_nbw<MODE, 1>(nbw) : pick_nbw<MODE, 2>(nbw);
}

// K split of the integer path: n_in = 32 KS T, T = 16 blocks a wave; two
// row groups a workgroup from 512 groups on, up to 12 waves (16 waves of
// SwiGLU would spill registers).  6144 and 8192 columns fit LDS (12 and 16
// waves, 96 and 128 KB of A operands) with one fragment, up to 4 batch rows,
// and one matrix.
bool i8_shape(int64_t n_in, int64_t batch, int mode, int* ks, int* t)
{
    *t = 16;
    switch (n_in) {
        case 1024: *ks = 2; return true;
        case 2048: *ks = 4; return true;
        case 3072: *ks = 6; return true;
        case 4096: *ks = 8; return true;
        case 6144: *ks = 12; return batch <= 4 && mode != kSwiGLU;
        case 8192: *ks = 16; return batch <= 4 && mode != kSwiGLU;
        default: return false;
    }
}

int i8_rg(int64_t groups, int ks) { return groups >= 512 && ks <= 6 ? 2 : 1; }

// 5..8 rows of a tall plain or residual product at 3072 columns (>= 2048 row
// groups): kTallRG row groups a workgroup of 4 waves x 24 blocks, so each
// workgroup's x preparation (two fragments) serves 16 kTallRG weight rows
// instead of 32.  Measured at 128256 x 3072 (graph-replayed): b8 125 -> 106
// us with four row groups (118 us with three); at 3..4 rows (one fragment)
// it was slower than two row groups of 6 waves (b4 74 -> 86 us).
constexpr int kTallRG = 4;

bool i8_tall(int64_t n_in, int64_t batch, int mode, int64_t groups)
{
    return n_in == 3072 && batch > 4 && batch <= 8 && groups >= 2048 && (mode == kPlain || mode == kResidual);
}

template <int MODE>
MfmaFn pick_i8_tall()
{
    if constexpr (MODE == kPlain || MODE == kResidual) return q8_0_gemv_i8<MODE, 4, 24, 2, kTallRG>;
    return nullptr;
}

template <int MODE, int KS, int T>
MfmaFn pick_i8_rg(int nv, int rg)
{
    if (nv == 1) return rg == 2 ? q8_0_gemv_i8<MODE, KS, T, 1, 2> : q8_0_gemv_i8<MODE, KS, T, 1, 1>;
    return rg == 2 ? q8_0_gemv_i8<MODE, KS, T, 2, 2> : q8_0_gemv_i8<MODE, KS, T, 2, 1>;
}

template <int MODE>
MfmaFn pick_i8(int ks, int nv, int rg)
{
    switch (ks) {
        case 2: return pick_i8_rg<MODE, 2, 16>(nv, rg);
        case 4: return pick_i8_rg<MODE, 4, 16>(nv, rg);
        case 6: return pick_i8_rg<MODE, 6, 16>(nv, rg);
        case 8: return nv == 1 ? q8_0_gemv_i8<MODE, 8, 16, 1, 1> : q8_0_gemv_i8<MODE, 8, 16, 2, 1>;
        case 12:
            if constexpr (MODE != kSwiGLU) return nv == 1 ? q8_0_gemv_i8<MODE, 12, 16, 1, 1> : nullptr;
            return nullptr;
        case 16:
            if constexpr (MODE != kSwiGLU) return nv == 1 ? q8_0_gemv_i8<MODE, 16, 16, 1, 1> : nullptr;
            return nullptr;
        default: return nullptr;
    }
}

// Flat 16-row groups of a problem: the segments (all but the last a multiple
// of 16 rows) back to back; SwiGLU's two matrices share their rows.
int64_t flat_rows(const Q8GemvProblem& p)
{
    if (p.mode != kQKV) return p.rows[0];
    int64_t n = 0;
    for (int k = 0; k < p.nseg; ++k) n += p.rows[k];
    return n;
}

// Blocks per K slice: the largest of 32, 24, 16, 8 that divides the row's
// n_in / 32 blocks and still gives at least kMinGrid workgroups (else 8, the
// most slices).  One slice per row needs no second launch.  Measured
// (graph-replayed, both launches, 3072x8192 with residual / SwiGLU 2x8192x3072
// at 8 rows): 8 waves, 6-8 blocks in flight, >= 224 workgroups 12.2 / 15.8 us;
// 16 in flight 13.1 / 18.1; 4 waves, >= 448 workgroups 11.0-11.4 / 15.4-16.7
// (4-8 in flight); 4 waves, >= 1024: 13.8 / 18.6; 2 waves 15.7-17.6 / 22-23.
constexpr int64_t kMinGrid = 448;

int slice_blocks(int64_t n_in, int64_t rows)
{
    const int64_t nb = n_in / 32, sets = (q8t_groups(rows) + kWaves - 1) / kWaves;
    for (int nbw : {32, 24, 16}) {
        if (nb % nbw) continue;
        if (sets * (nb / nbw) >= kMinGrid) return nbw;
    }
    return 8;
}

}  // namespace

// Host-side extent check of a launch plan: the last element each kernel
// instance reads or writes, worked out again from the plan and the kernels'
// index formulas, against the extents of the buffers the launch is given (the
// tiled planes of every segment, x, the workspace).  Returns an empty string
// when every access stays inside, else what overruns.  A failing plan is a
// library bug: the launch is refused rather than run.
std::string q8_mfma_plan_check(const Q8GemvProblem& p, int64_t ws_bytes)
{
    char why[256];
    auto over = [&](const char* what, int64_t end, int64_t size) {
        std::snprintf(why, sizeof why, "3..8-row GEMV plan: %s ends at %lld, extent %lld", what, (long long)end,
                      (long long)size);
        return std::string(why);
    };
    const int64_t nb = p.n_in / 32, rows = flat_rows(p);
    int iks = 0, it = 0;
    if (i8_shape(p.n_in, p.batch, p.mode, &iks, &it)) {
        // integer path: one workgroup per RG row groups, whole rows
        if ((int64_t)iks * it != nb) return over("waves x blocks", (int64_t)iks * it, nb);
        if (p.batch > 8) return over("batch rows", p.batch, 8);
        // x: item (b, blk, g) reads floats b n_in + 32 blk + 8 g .. +7
        const int64_t x_end = (p.batch - 1) * p.n_in + (nb - 1) * 32 + 3 * 8 + 8;
        if (x_end > p.batch * p.n_in) return over("x", x_end, p.batch * p.n_in);
        for (int k = 0; k < (p.mode == kSwiGLU ? 2 : p.nseg); ++k) {
            const int64_t segrows = p.mode == kSwiGLU ? p.rows[0] : p.rows[k];
            const int64_t g = q8t_groups(segrows), tiles = g * nb;
            const int64_t q_end = ((g - 1) * nb + nb - 1) * 512 + 8 * 63 + 8;
            const int64_t d_end = (((g - 1) * nb + nb - 1) * 16 + 15 + 1) * 2;
            if (q_end > tiles * 512) return over("weight tiles", q_end, tiles * 512);
            if (d_end > tiles * 32) return over("tile scales", d_end, tiles * 32);
        }
        return std::string();
    }
    const int nbw = slice_blocks(p.n_in, rows);
    const int64_t ksplit = nb / nbw;
    if (nbw != 8 && nbw != 16 && nbw != 24 && nbw != 32) return over("slice blocks", nbw, 32);
    if (ksplit * nbw != nb) return over("slices x slice blocks", ksplit * nbw, nb);
    if (ksplit > kMaxSlices) return over("slices", ksplit, kMaxSlices);
    const int nv = frags_for(p.batch), nm = p.mode == kSwiGLU ? 2 : 1;
    if (3 * p.batch > 16 * nv) return over("stacked x rows", 3 * p.batch, 16 * nv);
    // x: item (b, i, o) of the last slice reads floats b*n_in + 32*(blk0 + i) + 8*o .. +7
    const int64_t x_end = (p.batch - 1) * p.n_in + ((ksplit - 1) * nbw + nbw - 1) * 32 + 3 * 8 + 8;
    if (x_end > p.batch * p.n_in) return over("x", x_end, p.batch * p.n_in);
    // tiles and scales: the last group of each segment (loads clamp the row
    // group to the last one), every block of the last slice
    for (int k = 0; k < (p.mode == kSwiGLU ? 2 : p.nseg); ++k) {
        const int64_t segrows = p.mode == kSwiGLU ? p.rows[0] : p.rows[k];
        const int64_t g = q8t_groups(segrows), tiles = g * nb;
        const int64_t q_end = ((g - 1) * nb + (ksplit - 1) * nbw + nbw - 1) * 512 + 8 * 63 + 8;
        const int64_t d_end = (((g - 1) * nb + (ksplit - 1) * nbw + nbw - 1) * 16 + 15 + 1) * 2;
        if (q_end > tiles * 512) return over("weight tiles", q_end, tiles * 512);
        if (d_end > tiles * 32) return over("tile scales", d_end, tiles * 32);
    }
    if (ksplit > 1) {
        // partial sums of the last (set, slice, wave), and the slice-sum reads
        const int64_t sets = (q8t_groups(rows) + kWaves - 1) / kWaves;
        const int64_t per = (int64_t)kWaves * nm * p.batch * 16;
        const int64_t w_end = (sets * ksplit - 1) * per + (int64_t)(kWaves - 1) * nm * p.batch * 16 +
                              ((nm - 1) * p.batch + p.batch - 1) * 16 + 16;
        const int64_t r_end = (sets - 1) * ksplit * per + ((int64_t)(kWaves - 1) * nm * p.batch + p.batch - 1) * 16 +
                              15 + (ksplit - 1) * per + (nm - 1) * p.batch * 16 + 1;
        if (w_end * 4 > ws_bytes) return over("slice sums written (bytes)", w_end * 4, ws_bytes);
        if (r_end * 4 > ws_bytes) return over("slice sums read (bytes)", r_end * 4, ws_bytes);
    }
    return std::string();
}

bool q8_mfma_supported(const Q8GemvProblem& p)
{
    if (p.batch < 3 || p.batch > 8 || p.n_in % 256 || p.n_in > 8192) return false;
    // a 16-row group must not straddle two segments (only the last may be ragged)
    if (p.mode == kQKV)
        for (int k = 0; k + 1 < p.nseg; ++k)
            if (p.rows[k] % 16) return false;
    return true;
}

// The K slices' sums (none with one slice per row): per (row set, slice)
// kWaves x NM x batch x 16 floats.
int64_t q8_mfma_workspace_bytes(int mode, int64_t n_in, int64_t rows, int64_t batch)
{
    int iks = 0, it = 0;
    if (i8_shape(n_in, batch, mode, &iks, &it)) return 0;   // the integer path keeps whole rows
    const int64_t ksplit = (n_in / 32) / slice_blocks(n_in, rows);
    if (ksplit <= 1) return 0;
    const int64_t sets = (q8t_groups(rows) + kWaves - 1) / kWaves;
    const int nm = mode == kSwiGLU ? 2 : 1;
    return sets * ksplit * kWaves * nm * batch * 16 * 4;
}

hipError_t launch_q8_0_gemv_mfma(const Q8GemvProblem& p, const Q8TView* tiles, void* workspace,
                                 hipStream_t s)
{
    if (!q8_mfma_supported(p)) return hipErrorNotSupported;
    const Q8GemvArgs a = make_q8_gemv_args(p);
    TileArgs t{};
    const int last = p.nseg - 1, s1 = last < 1 ? last : 1;
    t.q0 = tiles[0].q;
    t.d0 = tiles[0].d;
    t.tq1 = tiles[s1].q - tiles[0].q;
    t.tq2 = tiles[last].q - tiles[0].q;
    t.td1 = tiles[s1].d - tiles[0].d;
    t.td2 = tiles[last].d - tiles[0].d;
    t.nb = p.n_in / 32;
    if (p.mode == kQKV) {
        t.gend0 = p.rows[0] / 16;
        t.gend1 = p.nseg > 1 ? t.gend0 + p.rows[1] / 16 : t.gend0;
        t.groups = (p.nseg > 2 ? t.gend1 : t.gend0) + q8t_groups(p.rows[last]);
        if (p.nseg == 1) t.groups = q8t_groups(p.rows[0]);
        if (p.nseg == 2) t.groups = t.gend0 + q8t_groups(p.rows[1]);
    } else {
        t.groups = q8t_groups(p.rows[0]);
        t.gend0 = t.gend1 = t.groups;
    }
    int iks = 0, it = 0;
    if (i8_shape(p.n_in, p.batch, p.mode, &iks, &it)) {
        if (!q8_mfma_plan_check(p, 0).empty()) return hipErrorInvalidConfiguration;
        int rg = i8_rg(t.groups, iks);
        const int nv = (int)((p.batch + 3) / 4);
        t.ksplit = 1;
        MfmaFn fn = nullptr;
        if (i8_tall(p.n_in, p.batch, p.mode, t.groups)) {
            iks = 4;   // 4 waves x 24 blocks = 3072 columns
            rg = kTallRG;
            fn = p.mode == kPlain ? pick_i8_tall<kPlain>() : pick_i8_tall<kResidual>();
        } else {
            switch (p.mode) {
                case kPlain: fn = pick_i8<kPlain>(iks, nv, rg); break;
                case kResidual: fn = pick_i8<kResidual>(iks, nv, rg); break;
                case kQKV: fn = pick_i8<kQKV>(iks, nv, rg); break;
                default: fn = pick_i8<kSwiGLU>(iks, nv, rg); break;
            }
        }
        if (!fn) return hipErrorNotSupported;
        hipLaunchKernelGGL(fn, dim3((unsigned)((t.groups + rg - 1) / rg)), dim3(64 * iks * rg), 0, s, a, t);
        count_launch();
        return hipGetLastError();
    }
    const int64_t rows = flat_rows(p);
    const int nbw = slice_blocks(p.n_in, rows);
    t.ksplit = (int)(t.nb / nbw);
    if (t.ksplit > kMaxSlices) return hipErrorNotSupported;
    const int64_t ws_bytes = q8_mfma_workspace_bytes(p.mode, p.n_in, rows, p.batch);
    if (!q8_mfma_plan_check(p, ws_bytes).empty()) return hipErrorInvalidConfiguration;
    if (t.ksplit > 1) {
        if (!workspace) return hipErrorInvalidValue;
        t.part = static_cast<float*>(workspace);
    }
    const int nv = frags_for(p.batch);
    MfmaFn fn = nullptr;
    switch (p.mode) {
        case kPlain: fn = pick_mfma<kPlain>(nbw, nv); break;
        case kResidual: fn = pick_mfma<kResidual>(nbw, nv); break;
        case kQKV: fn = pick_mfma<kQKV>(nbw, nv); break;
        default: fn = pick_mfma<kSwiGLU>(nbw, nv); break;
    }
    if (!fn) return hipErrorNotSupported;
    const int64_t sets = (t.groups + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(fn, dim3((unsigned)(sets * t.ksplit)), dim3(kWaves * 64), 0, s, a, t);
    count_launch();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || t.ksplit == 1) return e;
    const int64_t nout = p.batch * a.total_rows;
    const dim3 grid((unsigned)((nout + 255) / 256));
    switch (p.mode) {
        case kPlain: hipLaunchKernelGGL(sum_slices_kernel<kPlain>, grid, dim3(256), 0, s, a, t.part, t.ksplit); break;
        case kResidual:
            hipLaunchKernelGGL(sum_slices_kernel<kResidual>, grid, dim3(256), 0, s, a, t.part, t.ksplit);
            break;
        case kQKV: hipLaunchKernelGGL(sum_slices_kernel<kQKV>, grid, dim3(256), 0, s, a, t.part, t.ksplit); break;
        default: hipLaunchKernelGGL(sum_slices_kernel<kSwiGLU>, grid, dim3(256), 0, s, a, t.part, t.ksplit); break;
    }
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
