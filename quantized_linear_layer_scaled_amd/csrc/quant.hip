// Dynamic FP8 (OCP e4m3fn) quantization kernels for gfx950.
//
// Rule ("FP8 dynamic quantization" and "Block-FP8" of the page "Helion in
// vLLM: A Unified Route to Tunable Linear Kernels", section "What the
// integration changes"; scale rule absmax / 448 of the FP8 per-token
// workload): for each group of values
//     amax = max |x|,  s = amax / 448,  q = e4m3_rne(clamp(x / s, -448, 448))
// with the correctly rounded fp32 quotient x / s, s = 0 and zero codes for an
// all-zero group, and the sign kept when a value rounds to zero.  The
// conversion uses gfx950's v_cvt_pk_fp8_f32 (OCP e4m3, round to nearest even)
// after the clamp.
//
// The quotient x / s uses the reciprocal of s with one fma correction
// (quant_encode.h), equal in effect to the correctly rounded division.
//
// All kernels are HBM-bound (read 2 bytes, write 1 byte per element):
//   quant_rows:        TPR threads (64, 128 or 256) per row, the row held in
//                      registers, max by cross-lane shuffles and, across the
//                      waves of a row, through LDS (very long rows: one
//                      workgroup per row, two passes); many rows: one wave
//                      per row up to 4096 elements, a row loop with the next
//                      row's loads in flight for longer ones;
//   quant_groups128:   16 lanes per 1x128 group (8 bf16 per lane), shuffle
//                      max inside the 16 lanes; no LDS;
//   quant_weight_blocks: one workgroup per 128x128 weight block.
#include <type_traits>

#include "qll_internal.h"
#include "quant_encode.h"

namespace qll {

namespace {

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// TPR threads per row, 256 / TPR rows per 256-thread workgroup: each thread
// holds CH 16-byte chunks of its row (chunk c of thread t covers elements
// 8 (c TPR + t) .. + 7) in registers between the max and the conversion.
// The max is a wave shuffle reduction, then (TPR > 64) a max over the row's
// waves through LDS.
template <int TPR, int CH>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s, int M, int K)
{
    constexpr int WPR = TPR / 64;
    const int tid = threadIdx.x;
    const int sub = tid / TPR, t = tid % TPR;
    const int m = blockIdx.x * (256 / TPR) + sub;
    const bool live = m < M;
    const uint16_t* xr = x + (size_t)m * K;
    uint8_t* qr = q + (size_t)m * K;
    uint4 v[CH];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int e = (c * TPR + t) * 8;
        v[c] = make_uint4(0, 0, 0, 0);
        if (live && e < K)
            v[c] = *(const uint4*)(xr + e);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
        amax = fmaxf(amax, absmax8(v[c]));
    amax = wave_max(amax);
    if constexpr (WPR > 1) {
        __shared__ float red[4];
        if ((tid & 63) == 0)
            red[tid >> 6] = amax;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < WPR; ++w)
            amax = fmaxf(amax, red[sub * WPR + w]);
    }
    if (!live)
        return;
    const float sc = amax / 448.0f;
    if (t == 0)
        s[m] = sc;
    const Quot d(sc);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int e = (c * TPR + t) * 8;
        if (e < K)
            *(uint2*)(qr + e) = encode8(v[c], d);
    }
}

// Many rows of 2048..32768 elements: a grid of G workgroups (G < M) in which
// workgroup b quantizes rows b, b + G, b + 2G, ...; the loads of its next row
// are issued before the current row is reduced, encoded and stored, so that
// reads and writes overlap (with one row per workgroup and all of them
// resident at once, every row first loads and then every row stores).  The
// arithmetic per row is quant_rows_kernel's with TPR = 256: bitwise the same
// codes and scales.  Rows are read through a buffer resource (rows past M
// read as zeros, so the next-row loads need no branch).
template <int CH>
__global__ __launch_bounds__(256) void quant_rows_loop_kernel(const uint16_t* __restrict__ x,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ s, int M,
                                                             int K)
{
    const int tid = threadIdx.x;
    const int G = gridDim.x;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, 2 * M * K, 0x00020000);
    auto load = [&](uint4* v, int m) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int e = (c * 256 + tid) * 8;
            v[c] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rx, e < K ? 2 * (m * K + e) : 0x7FFFFFF0, 0, 0));
        }
    };
    __shared__ float red[2][4];
    uint4 v[2][CH];
    auto row = [&](auto P, int m) __attribute__((always_inline)) {
        constexpr int p = decltype(P)::value;
        load(v[p ^ 1], m + G);  // the next row (zeros past M)
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            amax = fmaxf(amax, absmax8(v[p][c]));
        amax = wave_max(amax);
        if ((tid & 63) == 0)
            red[p][tid >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[p][0], red[p][1]), fmaxf(red[p][2], red[p][3]));
        const float sc = amax / 448.0f;
        if (tid == 0)
            s[m] = sc;
        const Quot d(sc);
        uint8_t* qr = q + (size_t)m * K;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int e = (c * 256 + tid) * 8;
            if (e < K)
                *(uint2*)(qr + e) = encode8(v[p][c], d);
        }
    };
    int m = blockIdx.x;
    load(v[0], m);
    for (; m < M; m += 2 * G) {
        row(std::integral_constant<int, 0>{}, m);
        if (m + G >= M)
            break;
        row(std::integral_constant<int, 1>{}, m + G);
    }
}

// Many rows of up to 4096 elements: one wave per row, four rows per
// 256-thread workgroup, lane l holding chunks l, l + 64, ... of its row (CH
// of them).  The row is read through a buffer resource of its own (chunks
// past K read as zeros), so no load is conditional and the wait before the
// maximum covers them all at once; the maximum is a shuffle reduction inside
// the wave, with no LDS and no barrier, so each wave streams on its own.
// With every row in flight at once this keeps more bytes in the air than a
// workgroup per row of 256 threads, each holding one or two chunks.  The
// arithmetic is quant_rows_kernel's with TPR = 64: bitwise the same codes and
// scales.
template <int CH>
__global__ __launch_bounds__(256) void quant_rows_wave_kernel(const uint16_t* __restrict__ x,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ s, int M,
                                                             int K)
{
    const int lane = threadIdx.x & 63;
    // (the wave's row, uniform across the wave: one descriptor per wave)
    const int m = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (m >= M)
        return;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + (size_t)m * K), (short)0, 2 * K, 0x00020000);
    uint4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
        v[c] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, (c * 64 + lane) * 16, 0, 0));
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
        amax = fmaxf(amax, absmax8(v[c]));
    amax = wave_max(amax);
    const float sc = amax / 448.0f;
    if (lane == 0)
        s[m] = sc;
    const Quot d(sc);
    uint8_t* qr = q + (size_t)m * K;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int e = (c * 64 + lane) * 8;
        if (e < K)
            *(uint2*)(qr + e) = encode8(v[c], d);
    }
}

// Rows longer than 256 * 8 * 16 elements: one workgroup per row, two passes
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
    const Quot d(sc);
    for (int e = tid * 8; e < K; e += 256 * 8)
        *(uint2*)(qr + e) = encode8(*(const uint4*)(xr + e), d);
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
        *(uint2*)(q + e) = encode8(v, Quot(sc));
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
    const Quot d(sc);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int idx = c * 256 + tid;
        const int r = nb * 128 + (idx >> 4);
        const int col = kb * 128 + (idx & 15) * 8;
        if (r < N)
            *(uint2*)(q + (size_t)r * K + col) = encode8(v[c], d);
    }
}

}  // namespace

template <int TPR, int CH>
static void launch_rows(const uint16_t* x, uint8_t* q, float* s, int M, int K,
                        hipStream_t stream)
{
    hipLaunchKernelGGL((quant_rows_kernel<TPR, CH>), dim3((M + 256 / TPR - 1) / (256 / TPR)),
                       dim3(256), 0, stream, x, q, s, M, K);
}

hipError_t launch_quant_rows(const void* x, void* q, float* s, int M, int K,
                             hipStream_t stream)
{
    const uint16_t* xp = (const uint16_t*)x;
    uint8_t* qp = (uint8_t*)q;
    // a whole workgroup per row from 2048 elements on (short per-thread
    // chains, no idle lanes), narrower rows share a workgroup
    const int chunks = (K + 7) / 8;
    // many rows of up to 2048 elements (4096 from 2048 rows on): one wave per
    // row (measured faster there, cold: M = 4096, K = 2048 8.0 against
    // 12.0 us; M = 2048, K = 4096 8.8 against 9.7 us; from K = 6144 the row
    // loop below is ahead)
    if ((M >= 512 && chunks <= 256) || (M >= 2048 && chunks <= 512)) {
        const dim3 grid((M + 3) / 4);
        switch ((chunks + 63) / 64) {
        case 1: hipLaunchKernelGGL(quant_rows_wave_kernel<1>, grid, dim3(256), 0, stream, xp, qp, s, M, K); break;
        case 2: hipLaunchKernelGGL(quant_rows_wave_kernel<2>, grid, dim3(256), 0, stream, xp, qp, s, M, K); break;
        case 3: hipLaunchKernelGGL(quant_rows_wave_kernel<3>, grid, dim3(256), 0, stream, xp, qp, s, M, K); break;
        case 4: hipLaunchKernelGGL(quant_rows_wave_kernel<4>, grid, dim3(256), 0, stream, xp, qp, s, M, K); break;
        case 5:
        case 6: hipLaunchKernelGGL(quant_rows_wave_kernel<6>, grid, dim3(256), 0, stream, xp, qp, s, M, K); break;
        default: hipLaunchKernelGGL(quant_rows_wave_kernel<8>, grid, dim3(256), 0, stream, xp, qp, s, M, K); break;
        }
        return hipGetLastError();
    }
    // many rows of 2048..8192 elements: the row loop with G = 512 workgroups
    // (two per CU, each with the next row's loads in flight)
    constexpr int kLoopGrid = 512;
    // (byte offsets of the rows up to M + G stay below 2^31)
    if (M > kLoopGrid && chunks >= 256 && chunks <= 1024 &&
        2 * ((int64_t)M + kLoopGrid) * K < ((int64_t)1 << 31)) {
        const int G = kLoopGrid;
        switch ((chunks + 255) / 256) {
        case 1: hipLaunchKernelGGL(quant_rows_loop_kernel<1>, dim3(G), dim3(256), 0, stream, xp, qp, s, M, K); break;
        case 2: hipLaunchKernelGGL(quant_rows_loop_kernel<2>, dim3(G), dim3(256), 0, stream, xp, qp, s, M, K); break;
        case 3: hipLaunchKernelGGL(quant_rows_loop_kernel<3>, dim3(G), dim3(256), 0, stream, xp, qp, s, M, K); break;
        default: hipLaunchKernelGGL(quant_rows_loop_kernel<4>, dim3(G), dim3(256), 0, stream, xp, qp, s, M, K); break;
        }
        return hipGetLastError();
    }
    if (chunks <= 64)
        launch_rows<64, 1>(xp, qp, s, M, K, stream);
    else if (chunks <= 128)
        launch_rows<64, 2>(xp, qp, s, M, K, stream);
    else if (chunks < 256)
        launch_rows<128, 2>(xp, qp, s, M, K, stream);
    else {
        switch ((chunks + 255) / 256) {
        case 1: launch_rows<256, 1>(xp, qp, s, M, K, stream); break;
        case 2: launch_rows<256, 2>(xp, qp, s, M, K, stream); break;
        case 3: launch_rows<256, 3>(xp, qp, s, M, K, stream); break;
        case 4: launch_rows<256, 4>(xp, qp, s, M, K, stream); break;
        case 5:
        case 6: launch_rows<256, 6>(xp, qp, s, M, K, stream); break;
        case 7:
        case 8: launch_rows<256, 8>(xp, qp, s, M, K, stream); break;
        case 9:
        case 10:
        case 11:
        case 12: launch_rows<256, 12>(xp, qp, s, M, K, stream); break;
        case 13:
        case 14:
        case 15:
        case 16: launch_rows<256, 16>(xp, qp, s, M, K, stream); break;
        default:
            hipLaunchKernelGGL(quant_rows_long_kernel, dim3(M), dim3(256), 0, stream, xp, qp, s,
                               K);
            break;
        }
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
