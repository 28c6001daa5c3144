// Load-time repack of GGML blocks into the aligned plane layouts, the
// bit-exact dequantisation exports, and two diagnostic kernels.
//
// Block layouts (the workload definitions that accompany the rustdoc
// "Module cuda_lane" page; its Constants section names Q8_0_BLOCK_BYTES and
// Q8_0_BLOCK_ELEMS):
//   Q8_0 block, 34 bytes : fp16 d | int8 q[32]             w = d*q
//   Q4_K block, 144 bytes: fp16 d | fp16 dmin | 12 scale bytes | 128 nibble bytes
//                                                          w = d*sc*q - dmin*m
// The repack ("call once at plan build", preload_q4k_soa_weights on that page)
// splits each block into planes: the q bytes and nibbles go to one plane, the
// scales to others, so every row starts on a 16-byte boundary and the hot
// kernels read rows with aligned wide loads.  It moves bytes, except that the
// Q4_K 6-bit scales and mins are unpacked to one byte each.
#include "qdec_internal.h"

namespace qdec {

namespace {

constexpr int kQ8Bytes = 34;
constexpr int kQ4KBytes = 144;

__device__ inline float fp16_bits_to_f32(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, sizeof v);
    return static_cast<float>(v);
}

// One thread per Q8_0 block.  The raw blocks are 2-byte aligned (34 is even),
// so they are read as 17 halfwords.
__global__ __launch_bounds__(256) void repack_q8_0_kernel(const uint16_t* __restrict__ raw,
                                                          int64_t nblocks, int64_t nb_row,
                                                          int64_t n_in, int64_t n_out, int8_t* __restrict__ qp,
                                                          uint16_t* __restrict__ dp, uint16_t* __restrict__ dtp)
{
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= nblocks) return;
    const uint16_t* src = raw + blk * (kQ8Bytes / 2);
    uint32_t words[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        words[k] = (uint32_t)src[1 + 2 * k] | ((uint32_t)src[2 + 2 * k] << 16);
    const int64_t row = blk / nb_row;
    const int64_t kb = blk % nb_row;
    uint4* dst = reinterpret_cast<uint4*>(qp + row * n_in + kb * 32);
    dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
    dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
    dp[blk] = src[0];
    dtp[kb * n_out + row] = src[0];
}

// 6-bit scale and min of sub-block s from the 12 packed bytes (GGML K-quant
// packing): sub-blocks 0-3 use the low 6 bits of bytes s and s+4; sub-blocks
// 4-7 take their low 4 bits from byte s+4 (scale: low nibble, min: high
// nibble) and their high 2 bits from the top of bytes s-4 (scale) and s (min).
__device__ inline void unpack_scale_min(const uint8_t (&b)[12], int s, uint32_t& sc, uint32_t& mn)
{
    if (s < 4) {
        sc = b[s] & 63u;
        mn = b[s + 4] & 63u;
    } else {
        sc = (b[s + 4] & 15u) | ((uint32_t)(b[s - 4] >> 6) << 4);
        mn = (uint32_t)(b[s + 4] >> 4) | ((uint32_t)(b[s] >> 6) << 4);
    }
}

// One thread per Q4_K super-block (72 halfwords): nibbles to the qs plane,
// d|dmin to the dm plane, unpacked scales and mins to the sm plane.
__global__ __launch_bounds__(256) void repack_q4k_kernel(const uint16_t* __restrict__ raw,
                                                         int64_t nblocks,
                                                         uint8_t* __restrict__ qsp,
                                                         uint32_t* __restrict__ dmp,
                                                         uint32_t* __restrict__ smp)
{
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= nblocks) return;
    const uint16_t* src = raw + blk * (kQ4KBytes / 2);
    uint32_t words[36];
#pragma unroll
    for (int k = 0; k < 36; ++k)
        words[k] = (uint32_t)src[2 * k] | ((uint32_t)src[2 * k + 1] << 16);
    dmp[blk] = words[0];
    uint8_t sb[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) sb[k] = (uint8_t)(words[1 + k / 4] >> (8 * (k % 4)));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t sc0, m0, sc1, m1;
        unpack_scale_min(sb, 2 * p, sc0, m0);
        unpack_scale_min(sb, 2 * p + 1, sc1, m1);
        smp[blk * 4 + p] = sc0 | (sc1 << 8) | (m0 << 16) | (m1 << 24);
    }
    // n_in/2 bytes per row and 128 per super-block: super-block blk's nibbles
    // land at byte blk*128 of the qs plane.
    uint4* dst = reinterpret_cast<uint4*>(qsp + blk * 128);
#pragma unroll
    for (int k = 0; k < 8; ++k)
        dst[k] = make_uint4(words[4 + 4 * k], words[5 + 4 * k], words[6 + 4 * k], words[7 + 4 * k]);
}

// One thread per (row, super-block) of the tiled Q4_K copy, rows padded to a
// multiple of 16 with zeros (d = dmin = 0, so padding weights are 0): the
// super-block's four 32-byte nibble chunks go to the 8-byte slots r, r+16,
// r+32, r+48 of four tiles, its unpacked scale/min words to the sm tiles and
// d|dmin to the dm tile.
__global__ __launch_bounds__(256) void repack_q4k_tiled_kernel(const uint16_t* __restrict__ raw, int64_t n_out,
                                                               int64_t nsb, int64_t nthreads,
                                                               uint2* __restrict__ qp, uint32_t* __restrict__ smp,
                                                               uint32_t* __restrict__ dmp)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nthreads) return;
    const int64_t row = t / nsb, sb = t % nsb;
    const int64_t G = row >> 4, r = row & 15, nch = nsb * 4;
    uint32_t words[36] = {};
    if (row < n_out) {
        const uint16_t* src = raw + (row * nsb + sb) * (kQ4KBytes / 2);
#pragma unroll
        for (int k = 0; k < 36; ++k) words[k] = (uint32_t)src[2 * k] | ((uint32_t)src[2 * k + 1] << 16);
    }
    dmp[(G * nsb + sb) * 16 + r] = words[0];
    uint8_t sbytes[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) sbytes[k] = (uint8_t)(words[1 + k / 4] >> (8 * (k % 4)));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t c = sb * 4 + p;
        uint32_t sc0, m0, sc1, m1;
        unpack_scale_min(sbytes, 2 * p, sc0, m0);
        unpack_scale_min(sbytes, 2 * p + 1, sc1, m1);
        smp[(G * nch + c) * 16 + r] = sc0 | (sc1 << 8) | (m0 << 16) | (m1 << 24);
        // nibble bytes 32p + 8g .. +7 are words 4 + 8p + 2g, +1
#pragma unroll
        for (int g = 0; g < 4; ++g)
            qp[(G * nch + c) * 64 + r + 16 * g] = make_uint2(words[4 + 8 * p + 2 * g], words[5 + 8 * p + 2 * g]);
    }
}

// One thread per (row, Q8_0 block) of the tiled copy, rows padded to a
// multiple of 16 with zeros: the block's 32 weights go to the four 8-byte
// slots of its tile that the lanes r, r+16, r+32, r+48 load, its scale to the
// tile's scale slot r.
__global__ __launch_bounds__(256) void repack_q8_0_tiled_kernel(const uint16_t* __restrict__ raw,
                                                                int64_t n_out, int64_t nb,
                                                                int64_t nthreads,
                                                                uint2* __restrict__ qp,
                                                                uint16_t* __restrict__ dp)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nthreads) return;
    const int64_t row = t / nb, b = t % nb;
    const int64_t g = row >> 4;
    const int r = (int)(row & 15);
    uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint16_t d = 0;
    if (row < n_out) {
        const uint16_t* src = raw + (row * nb + b) * (kQ8Bytes / 2);
#pragma unroll
        for (int k = 0; k < 8; ++k) words[k] = (uint32_t)src[1 + 2 * k] | ((uint32_t)src[2 + 2 * k] << 16);
        d = src[0];
    }
    uint2* tile = qp + (g * nb + b) * 64;   // 64 slots of 8 bytes
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) tile[r + 16 * kg] = make_uint2(words[2 * kg], words[2 * kg + 1]);
    dp[(g * nb + b) * 16 + r] = d;
}

// One thread per 16 weights of the repacked Q8_0 matrix.
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(Q8View w, int64_t n_in, int64_t nchunks,
                                                           float* __restrict__ out)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= nchunks) return;
    const uint4 qv = *reinterpret_cast<const uint4*>(w.q + c * 16);
    // chunk c covers weights 16c..16c+15 of the flattened matrix; its block
    // is (16c)/32 because n_in is a multiple of 32.
    const float d = fp16_bits_to_f32(w.d[c >> 1]);
    const uint32_t words[4] = {qv.x, qv.y, qv.z, qv.w};
    float4* o = reinterpret_cast<float4*>(out + c * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t v = words[k];
        o[k] = make_float4(d * (float)(int8_t)(v & 0xff), d * (float)(int8_t)((v >> 8) & 0xff),
                           d * (float)(int8_t)((v >> 16) & 0xff), d * (float)(int8_t)(v >> 24));
    }
    (void)n_in;
}

// One thread per 16 nibble bytes (32 weights: 16 in sub-block 2p, 16 in 2p+1).
__global__ __launch_bounds__(256) void dequant_q4k_kernel(Q4KView w, int64_t n_in, int64_t nchunks,
                                                          float* __restrict__ out)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= nchunks) return;
    const int64_t sbg = c >> 3;          // global super-block index
    const int cc = (int)(c & 7);
    const int p = cc >> 1, h = cc & 1;
    const uint32_t dm = w.dm[sbg];
    const float d = fp16_bits_to_f32((uint16_t)(dm & 0xffff));
    const float dmin = fp16_bits_to_f32((uint16_t)(dm >> 16));
    const uint32_t sm = w.sm[sbg * 4 + p];
    const float a0 = d * (float)(sm & 0xff), b0 = dmin * (float)((sm >> 16) & 0xff);
    const float a1 = d * (float)((sm >> 8) & 0xff), b1 = dmin * (float)(sm >> 24);
    const uint4 qv = *reinterpret_cast<const uint4*>(w.qs + c * 16);
    const uint32_t words[4] = {qv.x, qv.y, qv.z, qv.w};
    // flattened element index of the first low-nibble weight
    const int64_t base = sbg * 256 + 64 * p + 16 * h;
    float* lo = out + base;
    float* hi = out + base + 32;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t byte = (words[k] >> (8 * t)) & 0xffu;
            // products are exact in f32; the subtraction rounds once
            lo[4 * k + t] = a0 * (float)(byte & 15u) - b0;
            hi[4 * k + t] = a1 * (float)(byte >> 4) - b1;
        }
    }
    (void)n_in;
}

__global__ void empty_kernel() {}

__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ dst,
                                                   const uint4* __restrict__ src, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

// Plain streaming read (the HBM read ceiling the weight-streaming kernels are
// measured against): a workgroup reads 4 KB * U contiguous bytes, each lane U
// non-temporal 16-byte loads issued before any use.  The loaded words are
// folded by XOR and written only in the (practically impossible) case that a
// lane's fold equals a fixed constant, so the loads cannot be removed while
// the kernel writes essentially nothing.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, int64_t n,
                                                          uint32_t* __restrict__ sink)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t base = (int64_t)blockIdx.x * (256 * U) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * 256;
        v[u] = i < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i)) : u32x4{0, 0, 0, 0};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

inline unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_repack_q8_0(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst,
                              hipStream_t s)
{
    const Q8View v = q8_view(dst, n_in, n_out);
    const int64_t nb = n_in / 32, nblocks = nb * n_out;
    hipLaunchKernelGGL(repack_q8_0_kernel, dim3(grid_for(nblocks, 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(raw), nblocks, nb, n_in, n_out,
                       const_cast<int8_t*>(v.q), const_cast<uint16_t*>(v.d), const_cast<uint16_t*>(v.dT));
    count_launch();
    return hipGetLastError();
}

hipError_t launch_repack_q4k(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst,
                             hipStream_t s)
{
    const Q4KView v = q4k_view(dst, n_in, n_out);
    const int64_t nblocks = (n_in / 256) * n_out;
    hipLaunchKernelGGL(repack_q4k_kernel, dim3(grid_for(nblocks, 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(raw), nblocks, const_cast<uint8_t*>(v.qs),
                       const_cast<uint32_t*>(v.dm), const_cast<uint32_t*>(v.sm));
    count_launch();
    return hipGetLastError();
}

hipError_t launch_repack_q4k_tiled(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst, hipStream_t s)
{
    const Q4KTView v = q4kt_view(dst, n_in, n_out);
    const int64_t nsb = n_in / 256, nthreads = q4kt_groups(n_out) * 16 * nsb;
    hipLaunchKernelGGL(repack_q4k_tiled_kernel, dim3(grid_for(nthreads, 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(raw), n_out, nsb, nthreads,
                       reinterpret_cast<uint2*>(const_cast<uint8_t*>(v.q)), const_cast<uint32_t*>(v.sm),
                       const_cast<uint32_t*>(v.dm));
    count_launch();
    return hipGetLastError();
}

hipError_t launch_repack_q8_0_tiled(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst,
                                    hipStream_t s)
{
    const Q8TView v = q8t_view(dst, n_in, n_out);
    const int64_t nb = n_in / 32, nthreads = q8t_groups(n_out) * 16 * nb;
    hipLaunchKernelGGL(repack_q8_0_tiled_kernel, dim3(grid_for(nthreads, 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(raw), n_out, nb, nthreads,
                       reinterpret_cast<uint2*>(const_cast<int8_t*>(v.q)), const_cast<uint16_t*>(v.d));
    count_launch();
    return hipGetLastError();
}

hipError_t launch_dequant_q8_0(Q8View w, int64_t n_in, int64_t n_out, float* out, hipStream_t s)
{
    const int64_t nchunks = n_out * n_in / 16;
    hipLaunchKernelGGL(dequant_q8_0_kernel, dim3(grid_for(nchunks, 256)), dim3(256), 0, s, w, n_in,
                       nchunks, out);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_dequant_q4k(Q4KView w, int64_t n_in, int64_t n_out, float* out, hipStream_t s)
{
    const int64_t nchunks = n_out * n_in / 32;
    hipLaunchKernelGGL(dequant_q4k_kernel, dim3(grid_for(nchunks, 256)), dim3(256), 0, s, w, n_in,
                       nchunks, out);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_empty(hipStream_t s)
{
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s)
{
    const int64_t n = bytes / 16;
    int64_t blocks = grid_for(n, 256);
    if (blocks > 256 * 16) blocks = 256 * 16;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint4*>(dst), static_cast<const uint4*>(src), n);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, int loads_per_lane, uint32_t* sink, hipStream_t s)
{
    const int64_t n = bytes / 16;
    const unsigned blocks = grid_for(n, 256 * loads_per_lane);
    const uint4* p = static_cast<const uint4*>(src);
    switch (loads_per_lane) {
        case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, s, p, n, sink); break;
        case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(256), 0, s, p, n, sink); break;
        case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, s, p, n, sink); break;
        case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, s, p, n, sink); break;
        default: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(blocks), dim3(256), 0, s, p, n, sink); break;
    }
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
