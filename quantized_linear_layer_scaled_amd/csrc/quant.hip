// Dynamic FP8 (OCP e4m3fn) quantization kernels for gfx950.
//
// Rule ("FP8 dynamic quantization" and "Block-FP8" of the page "Helion in
// vLLM: A Unified Route to Tunable Linear Kernels", section "What the
// integration changes"; scale rule absmax / 448 of the FP8 per-token
// workload): for each group of values
//     amax = max |x|,  s = amax / 448,  q = e4m3_rne(clamp(x / s, -448, 448))
// with a correctly rounded fp32 division (not a reciprocal multiply), s = 0
// and zero codes for an all-zero group, and the sign kept when a value rounds
// to zero.  The conversion uses gfx950's v_cvt_pk_fp8_f32 (OCP e4m3,
// round to nearest even) after the clamp.
//
// All three kernels are HBM-bound (read 2 bytes, write 1 byte per element):
//   quant_rows:        one wave per row, the row held in registers, max by
//                      cross-lane shuffles (very long rows: one workgroup
//                      per row, two passes, max across waves through LDS);
//   quant_groups128:   16 lanes per 1x128 group (8 bf16 per lane), shuffle
//                      max inside the 16 lanes; no LDS;
//   quant_weight_blocks: one workgroup per 128x128 weight block.
#include "qll_internal.h"

namespace qll {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const uint4& v, float* f)
{
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ float absmax8(const uint4& v)
{
    float f[8];
    unpack8(v, f);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        m = fmaxf(m, fabsf(f[i]));
    return m;
}

__device__ __forceinline__ float clamp448(float v)
{
    return fminf(fmaxf(v, -448.0f), 448.0f);
}

// 8 bf16 values -> 8 e4m3 codes (little-endian in a uint2).
__device__ __forceinline__ uint2 encode8(const uint4& v, float s)
{
    float f[8];
    unpack8(v, f);
    if (s == 0.0f)
        return make_uint2(0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        f[i] = clamp448(f[i] / s);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
    return make_uint2((uint32_t)w0, (uint32_t)w1);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// One wave per row, four rows per 256-thread workgroup: the row
// (K <= 64 * 8 * CH) stays in registers between the max and the conversion,
// the max is a wave-level shuffle reduction (no LDS, no barrier), and each
// lane keeps CH 16-byte loads in flight.
template <int CH>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s, int M, int K)
{
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= M)
        return;
    const uint16_t* xr = x + (size_t)m * K;
    uint8_t* qr = q + (size_t)m * K;
    uint4 v[CH];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int e = (c * 64 + lane) * 8;
        v[c] = make_uint4(0, 0, 0, 0);
        if (e < K)
            v[c] = *(const uint4*)(xr + e);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
        amax = fmaxf(amax, absmax8(v[c]));
    amax = wave_max(amax);
    const float sc = amax / 448.0f;
    if (lane == 0)
        s[m] = sc;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int e = (c * 64 + lane) * 8;
        if (e < K)
            *(uint2*)(qr + e) = encode8(v[c], sc);
    }
}

// Rows longer than 64 * 8 * 16 elements: one workgroup per row, two passes
// over the row (the second one hits the caches).
__global__ __launch_bounds__(256) void quant_rows_long_kernel(const uint16_t* __restrict__ x,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ s, int K)
{
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* xr = x + (size_t)m * K;
    uint8_t* qr = q + (size_t)m * K;
    float amax = 0.0f;
    for (int e = tid * 8; e < K; e += 256 * 8)
        amax = fmaxf(amax, absmax8(*(const uint4*)(xr + e)));
    amax = wave_max(amax);
    __shared__ float red[4];
    if ((tid & 63) == 0)
        red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax / 448.0f;
    if (tid == 0)
        s[m] = sc;
    for (int e = tid * 8; e < K; e += 256 * 8)
        *(uint2*)(qr + e) = encode8(*(const uint4*)(xr + e), sc);
}

// 1x128 groups: the flattened [M][K] array is a sequence of M*K/128 groups
// (K % 128 == 0), and the scale array [M][K/128] lists them in that order.
__global__ __launch_bounds__(256) void quant_groups128_kernel(const uint16_t* __restrict__ x,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ s,
                                                             long total)
{
    const long e = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
    const bool live = e < total;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (live)
        v = *(const uint4*)(x + e);
    float amax = absmax8(v);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float sc = amax / 448.0f;
    if (live) {
        if ((threadIdx.x & 15) == 0)
            s[e >> 7] = sc;
        *(uint2*)(q + e) = encode8(v, sc);
    }
}

// One workgroup per 128x128 block of the [N][K] weight: 64 values per thread.
__global__ __launch_bounds__(256) void quant_weight_blocks_kernel(const uint16_t* __restrict__ w,
                                                                 uint8_t* __restrict__ q,
                                                                 float* __restrict__ s,
                                                                 int N, int K)
{
    const int nb = blockIdx.x, kb = blockIdx.y;
    const int tid = threadIdx.x;
    const int KG = K / 128;
    uint4 v[8];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int idx = c * 256 + tid;           // 0 .. 2047 chunks of 8
        const int r = nb * 128 + (idx >> 4);     // 16 chunks per row
        const int col = kb * 128 + (idx & 15) * 8;
        v[c] = make_uint4(0, 0, 0, 0);
        if (r < N)
            v[c] = *(const uint4*)(w + (size_t)r * K + col);
        amax = fmaxf(amax, absmax8(v[c]));
    }
    amax = wave_max(amax);
    __shared__ float red[4];
    if ((tid & 63) == 0)
        red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax / 448.0f;
    if (tid == 0)
        s[nb * KG + kb] = sc;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int idx = c * 256 + tid;
        const int r = nb * 128 + (idx >> 4);
        const int col = kb * 128 + (idx & 15) * 8;
        if (r < N)
            *(uint2*)(q + (size_t)r * K + col) = encode8(v[c], sc);
    }
}

}  // namespace

hipError_t launch_quant_rows(const void* x, void* q, float* s, int M, int K,
                             hipStream_t stream)
{
    const int ch = (K + 511) / 512;  // 16-byte chunks per lane, one wave per row
    const uint16_t* xp = (const uint16_t*)x;
    uint8_t* qp = (uint8_t*)q;
    dim3 grid((M + 3) / 4), block(256);
    switch (ch) {
    case 1: hipLaunchKernelGGL(quant_rows_kernel<1>, grid, block, 0, stream, xp, qp, s, M, K); break;
    case 2: hipLaunchKernelGGL(quant_rows_kernel<2>, grid, block, 0, stream, xp, qp, s, M, K); break;
    case 3:
    case 4: hipLaunchKernelGGL(quant_rows_kernel<4>, grid, block, 0, stream, xp, qp, s, M, K); break;
    case 5:
    case 6: hipLaunchKernelGGL(quant_rows_kernel<6>, grid, block, 0, stream, xp, qp, s, M, K); break;
    case 7:
    case 8: hipLaunchKernelGGL(quant_rows_kernel<8>, grid, block, 0, stream, xp, qp, s, M, K); break;
    case 9:
    case 10:
    case 11:
    case 12: hipLaunchKernelGGL(quant_rows_kernel<12>, grid, block, 0, stream, xp, qp, s, M, K); break;
    case 13:
    case 14:
    case 15:
    case 16: hipLaunchKernelGGL(quant_rows_kernel<16>, grid, block, 0, stream, xp, qp, s, M, K); break;
    default:
        hipLaunchKernelGGL(quant_rows_long_kernel, dim3(M), block, 0, stream, xp, qp, s, K);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_quant_groups128(const void* x, void* q, float* s, int M, int K,
                                  hipStream_t stream)
{
    const long total = (long)M * K;
    const long blocks = (total / 8 + 255) / 256;
    hipLaunchKernelGGL(quant_groups128_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const uint16_t*)x, (uint8_t*)q, s, total);
    return hipGetLastError();
}

hipError_t launch_quant_weight_blocks(const void* w, void* q, float* s, int N, int K,
                                      hipStream_t stream)
{
    dim3 grid((N + 127) / 128, K / 128);
    hipLaunchKernelGGL(quant_weight_blocks_kernel, grid, dim3(256), 0, stream,
                       (const uint16_t*)w, (uint8_t*)q, s, N, K);
    return hipGetLastError();
}

}  // namespace qll
