// The FP8 (OCP e4m3fn) encode rule of the quantizer kernels ("FP8 dynamic
// quantization" of "Helion in vLLM: A Unified Route to Tunable Linear
// Kernels", section "What the integration changes"):
// q = e4m3_rne(clamp(x / s, -448, 448)) with the correctly rounded fp32
// quotient, zero codes when s == 0, and the sign kept when a value rounds to
// zero.  Every kernel that encodes calls these functions, so all codes agree
// bit for bit.
//
// The quotient.  A correctly rounded fp32 division costs about ten
// instructions (one of them quarter rate), which dominates the arithmetic of
// the quantizers.  Every value of a group shares s, so the kernels take the
// reciprocal y = 1 / s once (correctly rounded) and per value form
//     q0 = x * y,  r = fma(q0, s, -x),  q = fma(-r, y, q0)
// (one correction step from the exactly computed residual, Markstein's
// division scheme, with the residual's sign flipped: r = -(x - q0 s) exactly,
// since rounding is symmetric, and a zero x keeps its sign through both fmas,
// so the quotient needs no copysign -- the negations are free operand
// modifiers, the copysign was an instruction per value).  For bf16 x and s = amax / 448 with amax a bf16 value,
// s in [2^-64, 2^64], this q equals the correctly rounded x / s whenever
// either of them is at least 2^-10, and both are below 2^-10 otherwise, so
// the e4m3 code (+-0 below 2^-10, sign from x) is the same; this was checked
// exhaustively over all such (x, amax) pairs.  Groups with s outside that
// range take the division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qll {

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

// The quotient x / s of one group (see the header comment).
struct Quot {
    float s, y;
    bool fast;
    __device__ __forceinline__ explicit Quot(float sc) : s(sc)
    {
        fast = sc >= 0x1p-64f && sc <= 0x1p64f;
        y = fast ? 1.0f / sc : 0.0f;
    }
    // the quotient on the reciprocal path (valid when fast)
    __device__ __forceinline__ float by_reciprocal(float x) const
    {
        const float q0 = x * y;
        const float r = __builtin_fmaf(q0, s, -x);
        return __builtin_fmaf(-r, y, q0);
    }
};

// 8 bf16 values -> 8 e4m3 codes (little-endian in a uint2).
__device__ __forceinline__ uint2 encode8(const uint4& v, const Quot& d)
{
    float f[8];
    unpack8(v, f);
    if (d.s == 0.0f)
        return make_uint2(0, 0);
    // one branch per 8 values (the division path is for extreme scales only)
    if (d.fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            f[i] = clamp448(d.by_reciprocal(f[i]));
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            f[i] = clamp448(f[i] / d.s);
    }
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
    return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// Running maximum magnitude of the 8 bf16 values of a 16-byte chunk, kept
// on the packed bits (lo: the low halves, hi: the high halves): for finite
// bf16 values the magnitude order is the integer order of the low 15 bits.
__device__ __forceinline__ void absmax_bits8(const uint4& v, uint32_t& lo, uint32_t& hi)
{
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo = max(lo, u[i] & 0x7FFFu);
        hi = max(hi, u[i] & 0x7FFF0000u);
    }
}
__device__ __forceinline__ float absmax_bits_value(uint32_t lo, uint32_t hi)
{
    return fmaxf(__uint_as_float(lo << 16), __uint_as_float(hi));
}

}  // namespace qll
