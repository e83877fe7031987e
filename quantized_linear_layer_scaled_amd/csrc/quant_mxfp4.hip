// MXFP4 quantization for gfx950: bf16 [M][K] -> E2M1 codes (two per byte)
// and one E8M0 scale per 32 consecutive elements of a row.
//
// The pages name 4-bit formats among those vLLM serves (introduction of
// "Helion in vLLM: A Unified Route to Tunable Linear Kernels") without
// defining one; MXFP4 is the block-scaled 4-bit format CDNA4's matrix cores
// read natively, with the conversion rule of the OCP Microscaling (MX) v1.0
// specification:
//     amax = max |x| over the block,
//     E = floor(log2 amax) - 2 (the exponent of E2M1's largest value 6),
//         clamped to [-127, 127], -127 for an all-zero block,
//     scale byte = E + 127,
//     code = E2M1 round-to-nearest-even of x / 2^E, saturating at 6,
//            sign bit = sign of x (also when the magnitude rounds to 0).
// Packing: element 2j of a row in bits 0-3 of byte j, element 2j+1 in 4-7.
//
// On bf16 bits this is integer work: floor(log2 amax) of a normal amax is
// its exponent field minus 127, so the scale byte is max(field - 2, 0) (a
// subnormal or zero amax gives 0); x / 2^E is exact in fp32.
//
// HBM-bound (2 bytes read, 17/32 byte written per element): four lanes per
// block, 8 elements (one 16-byte load) per lane, block max by two lane
// shuffles, a 4-byte code store per lane and a scale byte per block.
#include "qll_internal.h"

namespace qll {

namespace {

// E2M1 magnitude code of 0 <= y < 8 (y = |x| / 2^E, so y < 8 by the choice
// of E), round to nearest even, saturating at 6 (code 7):
//   y < 1:  codes 0, 1, 2 are 0, 0.5, 1.0, i.e. rint(2 y) (ties to even);
//   y >= 1: round the fp32 mantissa to one bit (ties to even); the exponent
//           and that bit, (bits >> 22) - 252, are the code (1.0 -> 2).
__device__ __forceinline__ uint32_t e2m1_mag(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t hi = (u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22;
    const uint32_t big = min(hi - 252u, 7u);
    const uint32_t small = (uint32_t)__builtin_rintf(2.0f * y);
    return y < 1.0f ? small : big;
}

// Code (with sign) of one bf16 value h scaled by inv = 2^-E.
__device__ __forceinline__ uint32_t e2m1_code(uint32_t h, float inv)
{
    const float y = __uint_as_float((h & 0x7FFFu) << 16) * inv;
    return e2m1_mag(y) | ((h >> 12) & 8u);
}

__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint4* __restrict__ x,
                                                         uint32_t* __restrict__ q,
                                                         uint8_t* __restrict__ s,
                                                         long octets)
{
    const long stride = (long)gridDim.x * 256;
    for (long o = (long)blockIdx.x * 256 + threadIdx.x; o - (threadIdx.x & 3) < octets;
         o += stride) {
        // the four lanes of a block are live together (octets % 4 == 0)
        const bool live = o < octets;
        const uint4 v = live ? x[o] : make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
        m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
        // scale byte = max(exponent field of amax - 2, 0); 2^-E as fp32
        const uint32_t sc = (uint32_t)max((int)(m >> 7) - 2, 0);
        const float inv = __uint_as_float((254u - sc) << 23);
        uint32_t out = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out |= e2m1_code(w[i] & 0xFFFFu, inv) << (8 * i);
            out |= e2m1_code(w[i] >> 16, inv) << (8 * i + 4);
        }
        if (live) {
            q[o] = out;
            if ((threadIdx.x & 3) == 0)
                s[o >> 2] = (uint8_t)sc;
        }
    }
}

}  // namespace

hipError_t launch_quant_mxfp4(const void* x, void* q, void* s, int64_t elems,
                              hipStream_t stream)
{
    const long octets = (long)(elems / 8);
    long blocks = (octets + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;  // grid-stride beyond this
    hipLaunchKernelGGL(quant_mxfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint4*)x, (uint32_t*)q, (uint8_t*)s, octets);
    return hipGetLastError();
}

}  // namespace qll
