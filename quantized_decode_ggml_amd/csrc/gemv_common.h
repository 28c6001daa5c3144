// Pieces shared by the Q8_0 GEMV kernels (VALU and MFMA paths): the kernel
// argument block, the row -> weight-plane and row -> output mapping of the
// fused variants, and the host-side construction of the arguments.
// Included by one translation unit each; everything has internal linkage.
#pragma once

#include "qdec_internal.h"

namespace qdec {

namespace {

__device__ inline float fp16_bits_to_f32(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, sizeof v);
    return static_cast<float>(v);
}

struct Q8GemvArgs {
    // Segment 1 and 2 are addressed as element offsets from segment 0, and a
    // row picks its segment with 0/1 multipliers: selecting between argument
    // fields would make the compiler copy the arguments to scratch memory.
    const int8_t* q0;
    const uint16_t* d0;
    float* out0;
    int64_t dq1, dq2;      // q plane offsets (bytes) of segments 1, 2
    int64_t dd1, dd2;      // d plane offsets (elements)
    int64_t dout1, dout2;  // output offsets (elements)
    int64_t end0, end1;    // flat row where segment 1 and segment 2 start
    int64_t rows0, rows1, rows2;
    const float* x;
    const float* residual;
    int64_t n_in;
    int64_t total_rows;   // flat rows (output rows for SwiGLU)
    int batch;
    int lpr_log2;         // general path: lanes per row group = 1 << lpr_log2
    int nch;              // 16-byte chunks per row = n_in / 16
    const float* norm_w;  // RMSNorm weights folded into a one-row product, or null
    float eps;
};

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// Weight planes of one flat row (matrix m of SwiGLU).
struct Seg {
    const int8_t* q;
    const uint16_t* d;
};

template <int MODE>
__device__ inline Seg row_seg(const Q8GemvArgs& a, int64_t rr, int m)
{
    const int64_t nb = a.n_in >> 5;
    if constexpr (MODE == kSwiGLU) {
        return Seg{a.q0 + m * a.dq1 + rr * a.n_in, a.d0 + m * a.dd1 + rr * nb};
    } else if constexpr (MODE == kQKV) {
        const int64_t s1 = rr >= a.end0, s2 = rr >= a.end1;   // 0 or 1
        const int64_t seg1 = s1 - s2;                         // 1 in segment 1 only
        const int64_t local = rr - s1 * a.end0 - s2 * (a.end1 - a.end0);
        return Seg{a.q0 + seg1 * a.dq1 + s2 * a.dq2 + local * a.n_in,
                   a.d0 + seg1 * a.dd1 + s2 * a.dd2 + local * nb};
    } else {
        (void)m;
        return Seg{a.q0 + rr * a.n_in, a.d0 + rr * nb};
    }
}

// Rows lo and hi lie in one segment (always true outside QKV).
template <int MODE>
__device__ inline bool same_segment(const Q8GemvArgs& a, int64_t lo, int64_t hi)
{
    if constexpr (MODE == kQKV) return (lo >= a.end0) == (hi >= a.end0) && (lo >= a.end1) == (hi >= a.end1);
    else return true;
}

// Final value of output row `rw`, batch row b (v1 is the up product of SwiGLU).
template <int MODE>
__device__ inline void store_row(const Q8GemvArgs& a, int64_t rw, int b, float v0, float v1)
{
    if constexpr (MODE == kPlain) {
        a.out0[(int64_t)b * a.total_rows + rw] = v0;
    } else if constexpr (MODE == kResidual) {
        const int64_t o = (int64_t)b * a.total_rows + rw;
        a.out0[o] = a.residual[o] + v0;
    } else if constexpr (MODE == kQKV) {
        const int64_t s1 = rw >= a.end0, s2 = rw >= a.end1;
        const int64_t seg1 = s1 - s2;
        const int64_t local = rw - s1 * a.end0 - s2 * (a.end1 - a.end0);
        const int64_t rows = a.rows0 + seg1 * (a.rows1 - a.rows0) + s2 * (a.rows2 - a.rows0);
        a.out0[seg1 * a.dout1 + s2 * a.dout2 + (int64_t)b * rows + local] = v0;
    } else {
        a.out0[(int64_t)b * a.total_rows + rw] = silu(v0) * v1;
    }
}

// Host side: kernel arguments of a Q8_0 GEMV problem.
inline Q8GemvArgs make_q8_gemv_args(const Q8GemvProblem& p)
{
    Q8GemvArgs a{};
    const int last = p.nseg - 1;
    const int s1 = last < 1 ? last : 1;
    a.q0 = p.w[0].q;
    a.d0 = p.w[0].d;
    a.out0 = p.out[0];
    // byte distances between independent allocations, in elements of each type
    auto dist = [](const void* from, const void* to, int64_t elem) {
        return (int64_t)(reinterpret_cast<uintptr_t>(to) - reinterpret_cast<uintptr_t>(from)) / elem;
    };
    a.dq1 = dist(p.w[0].q, p.w[s1].q, 1);
    a.dq2 = dist(p.w[0].q, p.w[last].q, 1);
    a.dd1 = dist(p.w[0].d, p.w[s1].d, 2);
    a.dd2 = dist(p.w[0].d, p.w[last].d, 2);
    a.dout1 = dist(p.out[0], p.out[s1], 4);
    a.dout2 = dist(p.out[0], p.out[last], 4);
    a.rows0 = p.rows[0];
    a.rows1 = p.rows[s1];
    a.rows2 = p.rows[last];
    int64_t end = 0;
    for (int k = 0; k < p.nseg; ++k) end += p.rows[k];
    a.end0 = p.rows[0];
    a.end1 = p.nseg > 1 ? p.rows[0] + p.rows[1] : p.rows[0];
    a.x = p.x;
    a.residual = p.residual;
    a.n_in = p.n_in;
    a.total_rows = p.mode == kSwiGLU ? p.rows[0] : end;
    a.batch = (int)p.batch;
    a.nch = (int)(p.n_in / 16);
    a.norm_w = p.norm_w;
    a.eps = p.eps;
    return a;
}

}  // namespace

}  // namespace qdec
