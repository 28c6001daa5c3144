// Q8_0 GEMV for 3..8 batch rows on the matrix cores (gfx950 MFMA), plain,
// residual, fused QKV and fused SwiGLU.  Same results as the VALU kernels to
// the f32 tolerance; used when the batch makes those VALU-bound (each weight
// then costs one multiply-add per batch row on 16-lane SIMDs).
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
// scale-and-accumulate chain (NBW blocks per wave), KS - 1 in the cross-wave
// sum, 2 for the parts and, with the K split, one per workgroup slice plus
// the residual: below 110 units of 2^-24 of sum_j |w x| at n_in = 8192,
// i.e. under 7e-6, inside the 1e-5 bound.
//
// Operands per MFMA (16x16x32): A = an x-split fragment, lane l holding
// stacked row l % 16 and k = 8*(l/16)..+8 of the block; B = the weight
// fragment, lane l holding weight row l % 16 and the same 8 k (8 int8
// bytes); the result D[v][r] lands in lane r + 16*(v/4), element v % 4.  So
// every lane scales its results with the one d of its own weight row.
//
// A small kernel writes the x split once per call, in fragment order
// (block, part, lane), into a workspace the caller provides; all workgroups
// then read it from L2.  The weights come from the fragment-tiled copy (one
// contiguous 512-byte tile per 16 rows x 32 k, scales alongside), so every
// wave load is contiguous.  Each workgroup owns RG groups of 16 output rows
// (x 2 matrices for SwiGLU), which share each x fragment, and splits K over
// its KS waves, NBW blocks each; a wave streams its blocks in straight-line
// code with loads D blocks ahead, then the waves add their partial sums
// through LDS.  Where that grid would not fill the chip (fewer than 512 row
// groups, plain and residual forms), K is also split over workgroups: each
// writes its slice's sums to the workspace, and a third small launch adds
// the slices in slice order and the residual: n_in/1024 - 1 more roundings,
// in a fixed order, so every result is bitwise reproducible.  (Adding the
// slices with f32 atomics into an output that the split launch had set to
// the residual was 1.5-3.5 us faster at batch 4-8 but not reproducible; so
// were merges by the last slice of each row set, found with a device-scope
// counter: after a release fence per workgroup, which writes back the whole
// L2, 3x slower; with write-through stores of the sums, 20-40% slower.)
#include "gemv_common.h"

namespace qdec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kParts = 3;

// The A operand stacks the parts of all batch rows: virtual row v = p*batch + b
// holds part p of x[b] (3*batch rows, zero beyond), in NV = ceil(3*batch/16)
// fragments of 16 rows.  One thread per (block, fragment, lane): 8 bf16 of
// virtual row 16f + lane % 16 at k = 32*block + 8*(lane/16) .. +7.
__global__ __launch_bounds__(256) void split_x_kernel(const float* __restrict__ x, int batch,
                                                      int64_t n_in, int nv, int64_t nslots,
                                                      u32x4* __restrict__ xs)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nslots) return;
    const int l = (int)(t & 63);
    const int64_t bf = t >> 6;
    const int f = (int)(bf % nv);
    const int64_t blk = bf / nv;
    const int v = 16 * f + (l & 15);
    const int p = v / batch, b = v % batch;
    uint32_t h[8];
    if (p < kParts) {
        const float4* src = reinterpret_cast<const float4*>(x + (int64_t)b * n_in + blk * 32 + 8 * (l >> 4));
        const float4 v0 = src[0], v1 = src[1];
        const float xv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t u = __builtin_bit_cast(uint32_t, xv[j]);
            const uint32_t hi = u & 0xffff0000u;
            const float r1 = xv[j] - __builtin_bit_cast(float, hi);   // exact
            const uint32_t u1 = __builtin_bit_cast(uint32_t, r1);
            const uint32_t mid = u1 & 0xffff0000u;
            const float r2 = r1 - __builtin_bit_cast(float, mid);     // exact, 8 significant bits
            const uint32_t lo = __builtin_bit_cast(uint32_t, r2);
            h[j] = (p == 0 ? hi : (p == 1 ? mid : lo)) >> 16;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = 0;
    }
    xs[t] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// The K slices' sums of the split over workgroups, added in slice order (plus
// the residual): one thread per output; part holds, per (row-group set,
// slice), RG x batch x 16 sums.
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, int ksplit, int rg_per_set,
                                                         int batch, int64_t rows, const float* residual,
                                                         float* out)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)batch * rows) return;
    const int64_t b = t / rows, row = t % rows;
    const int64_t g = row / 16, set = g / rg_per_set;
    const int rg = (int)(g % rg_per_set), r = (int)(row % 16);
    const int64_t per = (int64_t)rg_per_set * batch * 16;
    const float* p = part + set * ksplit * per + (rg * batch + b) * 16 + r;
    float v = p[0];
    for (int k = 1; k < ksplit; ++k) v += p[k * per];
    out[t] = residual ? residual[t] + v : v;
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
    int ksplit;   // workgroups per row-group set along K (AT kernels)
    float* part;  // AT: per (set, slice) the slice's sums, RG x batch x 16 floats
};

// K split over workgroups (plain and residual): kAtKs waves of kAtNbw blocks
// per workgroup, kAtRg row groups sharing every x fragment; at most
// kMaxSlices slices (n_in <= 8192).
constexpr int kAtKs = 4, kAtNbw = 8, kAtRg = 2, kMaxSlices = 8;

// AT: the workgroup covers KS * NBW blocks of K (slice blockIdx.x % ksplit)
// and writes its partial sums to the workspace; sum_slices_kernel then adds
// the slices in slice order and stores the rows (plain and residual forms).
template <int MODE, int KS, int NBW, int DP, int RG, int NV, bool AT>
__global__ __launch_bounds__(KS * 64) void q8_0_gemv_mfma(Q8GemvArgs a, TileArgs t, const u32x4* __restrict__ xs)
{
    constexpr int NM = (MODE == kSwiGLU) ? 2 : 1;
    static_assert(!AT || MODE == kPlain || MODE == kResidual, "atomic K split: linear epilogues only");
    constexpr int D = DP < NBW ? DP : NBW;   // blocks in flight ahead of the one computed
    constexpr int RS = D + 1;                 // register ring slots
    static_assert(KS > 1, "the epilogue runs on wave 0 after the K reduction");
    __shared__ float red[KS - 1][RG][NM][NV][4][64];
    __shared__ float fin[RG][NM][NV * 16][16];   // D[v][r] after the K reduction

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g4 = lane >> 4;
    const int64_t gb = AT ? blockIdx.x / t.ksplit : blockIdx.x;   // row-group set
    const int kp = AT ? (int)(blockIdx.x % t.ksplit) : 0;          // K slice
    const int blk0 = (kp * KS + w) * NBW;
    const int64_t tile_stride = t.nb * 512, dtile_stride = t.nb * 16;

    // tile and scale pointers of this wave's first block, per row group and matrix
    const int8_t* tq[RG][NM];
    const uint16_t* td[RG][NM];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        int64_t G = gb * RG + rg;
        G = G < t.groups ? G : t.groups - 1;                  // loads stay in bounds
#pragma unroll
        for (int m = 0; m < NM; ++m) {
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
            tq[rg][m] = t.q0 + oq + local * tile_stride + (int64_t)blk0 * 512 + 8 * lane;
            td[rg][m] = t.d0 + od + local * dtile_stride + (int64_t)blk0 * 16 + (lane & 15);
        }
    }
    const u32x4* xw = xs + (int64_t)blk0 * (NV * 64) + lane;

    u32x4 xf[RS][NV];
    u32x2 wq[RS][RG][NM];
    uint16_t wd[RS][RG][NM];
    auto issue = [&](int i, int slot) {
#pragma unroll
        for (int f = 0; f < NV; ++f) xf[slot][f] = xw[(i * NV + f) * 64];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                wq[slot][rg][m] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tq[rg][m] + i * 512));
                wd[slot][rg][m] = __builtin_nontemporal_load(td[rg][m] + i * 16);
            }
    };

    f32x4 acc[RG][NM][NV];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int f = 0; f < NV; ++f) acc[rg][m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < D; ++i) issue(i, i);
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        if (i + D < NBW) issue(i + D, (i + D) % RS);
        const int s = i % RS;
        // Opaque from here on: without this the compiler hoists the unpacking
        // of a prefetched block next to its load, and every step then waits
        // for the load it has just issued.
#pragma unroll
        for (int f = 0; f < NV; ++f) asm volatile("" : "+v"(xf[s][f]));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                asm volatile("" : "+v"(wq[s][rg][m]));
                asm volatile("" : "+v"(wd[s][rg][m]));
            }
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const bf16x8 bw = q8_to_bf16(wq[s][rg][m]);
                const float dsc = fp16_bits_to_f32(wd[s][rg][m]);
#pragma unroll
                for (int f = 0; f < NV; ++f) {
                    const f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, xf[s][f]), bw, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[rg][m][f][e] = __builtin_fmaf(dsc, P[e], acc[rg][m][f][e]);
                }
            }
        __builtin_amdgcn_sched_barrier(0);   // keep the block pipeline in program order
    }

    if constexpr (KS > 1) {
        if (w > 0) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int f = 0; f < NV; ++f)
#pragma unroll
                        for (int e = 0; e < 4; ++e) red[w - 1][rg][m][f][e][lane] = acc[rg][m][f][e];
        }
        __syncthreads();
        if (w != 0) return;
#pragma unroll
        for (int k = 0; k < KS - 1; ++k)
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int f = 0; f < NV; ++f)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[rg][m][f][e] += red[k][rg][m][f][e][lane];
    }
    // D[v][r]: lane r + 16*(v%16/4) element v%4 of fragment v/16; the three
    // parts of batch row b sit at v = b, batch + b, 2*batch + b
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int f = 0; f < NV; ++f)
#pragma unroll
                for (int e = 0; e < 4; ++e) fin[rg][m][16 * f + 4 * g4 + e][lane & 15] = acc[rg][m][f][e];
    __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's LDS writes done (only wave 0 is left)
    __builtin_amdgcn_wave_barrier();
    const int r = lane & 15;
    if constexpr (AT) {
        // this slice's sums; sum_slices_kernel adds the slices in order afterwards
        float* mine = t.part + (gb * t.ksplit + kp) * (int64_t)(RG * a.batch * 16);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
            for (int b = g4; b < a.batch; b += 4)
                mine[(rg * a.batch + b) * 16 + r] =
                    (fin[rg][0][b][r] + fin[rg][0][a.batch + b][r]) + fin[rg][0][2 * a.batch + b][r];
    } else {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int64_t row = (gb * RG + rg) * 16 + r;
            if (row >= a.total_rows) continue;
            for (int b = g4; b < a.batch; b += 4) {
                const float v0 = (fin[rg][0][b][r] + fin[rg][0][a.batch + b][r]) + fin[rg][0][2 * a.batch + b][r];
                const float v1 = (fin[rg][NM - 1][b][r] + fin[rg][NM - 1][a.batch + b][r]) +
                                 fin[rg][NM - 1][2 * a.batch + b][r];
                store_row<MODE>(a, row, b, v0, v1);
            }
        }
    }
}

using MfmaFn = void (*)(Q8GemvArgs, TileArgs, const u32x4*);

// x fragments per block: the 3*batch stacked part rows in groups of 16
inline int frags_for(int64_t batch) { return (int)((3 * batch + 15) / 16); }

// Blocks in flight per wave (the register ring holds D + 1 blocks of x
// fragments and weight tiles).
template <int MODE, int RG>
constexpr int depth() { return 8; }

template <int MODE, int KS, int RG, int NV>
MfmaFn pick_nbw(int nbw)
{
    switch (nbw) {
        case 8: return q8_0_gemv_mfma<MODE, KS, 8, depth<MODE, RG>(), RG, NV, false>;
        case 16: return q8_0_gemv_mfma<MODE, KS, 16, depth<MODE, RG>(), RG, NV, false>;
        case 24: return q8_0_gemv_mfma<MODE, KS, 24, depth<MODE, RG>(), RG, NV, false>;
        case 32: return q8_0_gemv_mfma<MODE, KS, 32, depth<MODE, RG>(), RG, NV, false>;
        default: return nullptr;
    }
}

// The K split over workgroups (constants above) is taken where the
// one-workgroup-per-row-group grid would leave compute units idle; measured
// on 3072x8192 with residual (graph-replayed, both launches): batch 3 / 4 / 8
// 12.9 / 13.0 / 16.7 -> 10.7 / 10.9 / 13.1 us (4 x 8 x 2 against 4 x 8 x 4,
// 4 x 16 x 2 and 4 x 8 x 1: 11.7-14.7 us).  On 8192x3072, where two row
// groups per workgroup already fill the chip, it gained nothing.


template <int MODE>
MfmaFn pick_at(int nv)
{
    return nv == 1 ? q8_0_gemv_mfma<MODE, kAtKs, kAtNbw, 8, kAtRg, 1, true>
                   : q8_0_gemv_mfma<MODE, kAtKs, kAtNbw, 8, kAtRg, 2, true>;
}

template <int MODE, int RG, int NV>
MfmaFn pick_ks(int ks, int nbw)
{
    return ks == 4 ? pick_nbw<MODE, 4, RG, NV>(nbw) : pick_nbw<MODE, 8, RG, NV>(nbw);
}

template <int MODE>
MfmaFn pick_mfma(int ks, int nbw, int rg, int nv)
{
    if constexpr (MODE != kSwiGLU) {
        if (rg == 2) return nv == 1 ? pick_ks<MODE, 2, 1>(ks, nbw) : pick_ks<MODE, 2, 2>(ks, nbw);
    }
    return nv == 1 ? pick_ks<MODE, 1, 1>(ks, nbw) : pick_ks<MODE, 1, 2>(ks, nbw);
}

// K split: KS waves of NBW blocks; 4 waves up to 96 blocks (n_in 3072),
// 8 waves beyond.
bool mfma_shape(int64_t n_in, int* ks, int* nbw)
{
    const int64_t nb = n_in / 32;
    for (int k : {4, 8}) {
        if (nb % k) continue;
        const int64_t n = nb / k;
        if ((n == 8 || n == 16 || n == 24 || n == 32) && (k == 8 || nb <= 96)) {
            *ks = k;
            *nbw = (int)n;
            return true;
        }
    }
    return false;
}

}  // namespace

// K split over workgroups: plain and residual products whose row groups
// would leave compute units idle (fewer than 512) and whose K holds 2 to
// kMaxSlices whole workgroup slices.
static bool q8_mfma_ksplit(int mode, int64_t n_in, int64_t rows0)
{
    const int64_t at_blocks = (int64_t)kAtKs * kAtNbw;
    const int64_t slices = (n_in / 32) / at_blocks;
    return (mode == kPlain || mode == kResidual) && (n_in / 32) % at_blocks == 0 && slices >= 2 &&
           slices <= kMaxSlices && q8t_groups(rows0) / 2 < 256;
}

// at most two fragments (3 * 8 stacked rows) of 64 lanes x 16 bytes per block,
// then, with the K split, the slices' sums (batch x padded rows per slice)
int64_t q8_mfma_workspace_bytes(int mode, int64_t n_in, int64_t rows0, int64_t batch)
{
    const int64_t xs = align_up((n_in / 32) * 2 * 64 * 16, kAlign);
    if (!q8_mfma_ksplit(mode, n_in, rows0)) return xs;
    const int64_t ksplit = (n_in / 32) / ((int64_t)kAtKs * kAtNbw);
    const int64_t sets = (q8t_groups(rows0) + kAtRg - 1) / kAtRg;
    return xs + sets * ksplit * kAtRg * 16 * batch * 4;
}


bool q8_mfma_supported(const Q8GemvProblem& p)
{
    int ks = 0, nbw = 0;
    if (p.batch < 3 || p.batch > 8 || !mfma_shape(p.n_in, &ks, &nbw)) return false;
    // a 16-row group must not straddle two segments (only the last may be ragged)
    if (p.mode == kQKV)
        for (int k = 0; k + 1 < p.nseg; ++k)
            if (p.rows[k] % 16) return false;
    return true;
}

hipError_t launch_q8_0_gemv_mfma(const Q8GemvProblem& p, const Q8TView* tiles, void* workspace,
                                 hipStream_t s)
{
    int ks = 0, nbw = 0;
    if (!q8_mfma_supported(p) || !mfma_shape(p.n_in, &ks, &nbw)) return hipErrorNotSupported;
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
    const int nv = frags_for(p.batch);
    MfmaFn fn = nullptr;
    int64_t blocks = 0;
    const int64_t at_blocks = (int64_t)kAtKs * kAtNbw;
    if (q8_mfma_ksplit(p.mode, p.n_in, p.rows[0])) {
        // K split over workgroups: x fragments are read by kAtRg row groups
        // per workgroup and only for its K slice; the slices' sums go to the
        // workspace after the x fragments
        t.ksplit = (int)(t.nb / at_blocks);
        t.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(t.nb * 2 * 64 * 16, kAlign));
        fn = p.mode == kPlain ? pick_at<kPlain>(nv) : pick_at<kResidual>(nv);
        blocks = (t.groups + kAtRg - 1) / kAtRg * t.ksplit;
        ks = kAtKs;
    } else {
        // two row groups per workgroup while that still gives one workgroup per CU
        // (SwiGLU already shares each x fragment between its two matrices)
        const int rg = p.mode != kSwiGLU && t.groups / 2 >= 256 ? 2 : 1;
        switch (p.mode) {
            case kPlain: fn = pick_mfma<kPlain>(ks, nbw, rg, nv); break;
            case kResidual: fn = pick_mfma<kResidual>(ks, nbw, rg, nv); break;
            case kQKV: fn = pick_mfma<kQKV>(ks, nbw, rg, nv); break;
            default: fn = pick_mfma<kSwiGLU>(ks, nbw, rg, nv); break;
        }
        blocks = (t.groups + rg - 1) / rg;
    }
    if (!fn) return hipErrorNotSupported;
    u32x4* xs = static_cast<u32x4*>(workspace);
    const int64_t nslots = (p.n_in / 32) * nv * 64;
    hipLaunchKernelGGL(split_x_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, s, p.x,
                       (int)p.batch, p.n_in, nv, nslots, xs);
    count_launch();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(ks * 64), 0, s, a, t, xs);
    count_launch();
    e = hipGetLastError();
    if (e != hipSuccess || !t.ksplit) return e;
    const int64_t nout = p.batch * p.rows[0];
    hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, s, t.part, t.ksplit,
                       kAtRg, (int)p.batch, p.rows[0], p.mode == kResidual ? p.residual : nullptr, a.out0);
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
