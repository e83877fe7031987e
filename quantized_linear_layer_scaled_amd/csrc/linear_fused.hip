// Fused FP8 dynamic linear layer for few tokens: per-token quantization of
// the bf16 activations inside the Swap-AB decode GEMM, one launch instead of
// the quantizer's launch plus the GEMM's ("FP8 dynamic quantization" of
// "Helion in vLLM: A Unified Route to Tunable Linear Kernels", "What the
// integration changes"; each kernel transition of a decode step costs a
// launch and a round trip through memory).
//
// A workgroup owns HR weight rows (16, or 8 with the MFMA's other rows
// zero) and all M <= TOK <= 16 tokens, and its W waves split K on the grid of the
// wave-split decode GEMM (gemm_skinny.h), so that the products are summed in
// exactly that kernel's order:
//   1. each wave issues the loads of its whole K chunk of weights (e4m3)
//      and of the tokens (bf16, in the MFMA operand layout: lane l holds
//      token l % 16 and 32 consecutive K elements of each step);
//   2. the per-token maximum magnitude: within a lane, over the 4 lanes of
//      a token by shuffles, over the 8 waves through LDS (one barrier);
//   3. s = amax / 448 and the codes with the quantizer's own encode
//      (quant_encode.h), so codes and scales are bitwise the quantizer's;
//   4. the MFMAs of the chunk, the 8 partial tiles added in LDS in wave
//      order, the epilogue (acc * s[m]) * sb[n].
// The output is therefore bitwise that of quantize_per_token_fp8 followed by
// the 8-wave decode GEMM with the same row count per workgroup.  Workgroup 0
// also writes the codes and scales, which the call returns.
//
// Every workgroup reads all tokens' bf16 values (twice the bytes of their
// codes) and encodes them, so this pays off for very few tokens only; the
// dispatch table decides per shape.
#include <algorithm>

#include "gemm_tile.h"
#include "quant_encode.h"

namespace qll {


// 32 bf16 values (64 bytes) -> 32 e4m3 codes (one MFMA operand)
static __device__ __forceinline__ void encode32(const uint4* v, const Quot& d, uint4* c)
{
    uint2 e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        e[i] = encode8(v[i], d);
    c[0] = make_uint4(e[0].x, e[0].y, e[1].x, e[1].y);
    c[1] = make_uint4(e[2].x, e[2].y, e[3].x, e[3].y);
}

// V bf16 values (V / 2 words, V = 2 or 4) -> V e4m3 codes in one dword: the
// per-value arithmetic of encode8 (quant_encode.h), so the same codes.
template <int V>
static __device__ __forceinline__ uint32_t encode_small(const uint32_t* w, const Quot& d)
{
    float f[V];
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
    }
    if (d.s == 0.0f)
        return 0u;
    if (d.fast) {
#pragma unroll
        for (int i = 0; i < V; ++i)
            f[i] = clamp448(d.by_reciprocal(f[i]));
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
            f[i] = clamp448(f[i] / d.s);
    }
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    if constexpr (V == 4)
        r = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], r, true);
    return (uint32_t)r;
}

// TOK = 16: every lane holds its token's values in the MFMA operand layout
// and encodes them there (16 tokens x 32 values of a step per wave, whatever
// M is).  TOK = 1, 2, 4 or 8 (M <= TOK): the wave's lanes hold only the
// tokens there are -- VPL = 2 TOK values of a step per lane (8 from TOK = 4
// on: 16-byte chunks), lane L taking run L % (128 / VPL) of token
// L / (128 / VPL) + (64 VPL / 128) h -- so a wave encodes TOK instead of 16
// tokens' values (a wave64 VALU instruction takes four cycles: at K = 6144
// the 16-token encode of every workgroup cost ~5 us), and the codes reach
// the MFMA layout through the wave's own LDS buffer.  The maximum, the scale
// and the encode of each value are the same, so the codes, scales and output
// are bitwise those of TOK = 16.
template <int HR, int W, int D, int TOK>
__global__ __launch_bounds__(W * 64) void linear_fused_kernel(FusedArgs a)
{
    static_assert(TOK == 1 || TOK == 2 || TOK == 4 || TOK == 8 || TOK == 16,
                  "1, 2, 4, 8 or 16 tokens");
    constexpr bool DENSE = TOK < 16;
    constexpr int VPL = TOK >= 4 ? 8 : 2 * TOK;   // dense: values of a step per lane and run
    constexpr int VW = VPL / 2;                   // ... in 32-bit words
    constexpr int LPTOK = 128 / VPL;              // lanes per token
    constexpr int TPP = 64 / LPTOK;               // tokens per pass over the lanes
    constexpr int NCH = DENSE ? TOK / TPP : 1;    // passes (runs per lane per step)
    constexpr int KB = 32;          // bytes (codes) per lane per MFMA step
    constexpr int KSTEP = 4 * KB;   // 128 K elements per step
    constexpr int U = kFoldUnit / KSTEP;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int N = a.N, M = a.M, K = a.K;
    const int n0 = blockIdx.x * HR;
    const bool wrow = (lane & 15) < HR;
    // the wave's steps, as the wave-split decode GEMM cuts them
    const int T = (K + KSTEP - 1) / KSTEP;
    const int TU = (T + U - 1) / U;
    const int s0 = min(T, U * (wave * TU / W));
    const int s1 = min(T, U * ((wave + 1) * TU / W));
    const int ns = s1 - s0;  // <= D (checked on the host)

    const int t = lane & 15;                 // this lane's token
    const int koff = (lane >> 4) * KB;       // element offset within a step
    // the tokens and the workgroup's weight rows as two buffers (one
    // descriptor each, the same in every lane): a load at an offset outside
    // (the K tail, the steps past this wave's range, weight rows past N or
    // past the workgroup's HR) returns zeros, so every load is unconditional
    // and the waits below count them exactly
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, (short)0, 2 * M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.B + (size_t)n0 * K), (short)0, min(HR, N - n0) * K, 0x00020000);
    constexpr int kOut = 0x7FFFFFF0;
    // lanes of tokens past M read zeros (their output columns are
    // discarded): no load path spent on copies of another row
    const bool tok = t < M;
    const int xrow = t * K;                   // element offset of the token's row
    const int wrowoff = wrow ? t * K : kOut;  // byte offset of the weight row

    // 1. loads: the tokens (32 bf16 per step; dense: NCH chunks of 8) first,
    // then the weights (32 bytes per step): the wait for the tokens (in issue
    // order) then leaves the weight stream in flight while the maximum and
    // the codes are formed
    const int dj = lane % LPTOK;  // dense: this lane's run of each step
    const int dt = lane / LPTOK;  // dense: its token in the first pass
    uint4 wb[D][2], xb[DENSE ? 1 : D][4];
    uint32_t xd[DENSE ? D : 1][NCH][VW];
    if constexpr (DENSE) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int e = (s0 + d) * KSTEP + dj * VPL;
#pragma unroll
            for (int h = 0; h < NCH; ++h) {
                const int tk = dt + TPP * h;
                const int off = tk < M && d < ns && e < K ? 2 * (tk * K + e) : kOut;
                if constexpr (VW == 4) {
                    const uint4 v = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
                    xd[d][h][0] = v.x;
                    xd[d][h][1] = v.y;
                    xd[d][h][2] = v.z;
                    xd[d][h][3] = v.w;
                } else if constexpr (VW == 2) {
                    const uint2 v = __builtin_bit_cast(
                        uint2, __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 0));
                    xd[d][h][0] = v.x;
                    xd[d][h][1] = v.y;
                } else {
                    xd[d][h][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0);
                }
            }
        }
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int e = (s0 + d) * KSTEP + koff;  // this lane's first element
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xb[d][j] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(
                               rx, tok && d < ns && e + 8 * j < K ? 2 * (xrow + e + 8 * j) : kOut,
                               0, 0));
        }
    }
    // (empty asm with a memory clobber: the compiler keeps the three groups
    // -- token loads, weight loads, the math -- in this order)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int e = (s0 + d) * KSTEP + koff;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            wb[d][j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rw, wrow && d < ns && e + 16 * j < K ? wrowoff + e + 16 * j : kOut,
                           0, 0));
    }

    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 2. the token's maximum magnitude over K (on the bf16 bits: for finite
    // values the magnitude order is the integer order of the low 15 bits)
    __shared__ float red_max[W][16];
    float amax = 0.0f, sc = 0.0f;
    float dsc[NCH];  // dense: the scales of this lane's tokens
    if constexpr (DENSE) {
        float dmax[NCH];
#pragma unroll
        for (int h = 0; h < NCH; ++h) {
            uint32_t mlo = 0, mhi = 0;
#pragma unroll
            for (int d = 0; d < D; ++d)
#pragma unroll
                for (int i = 0; i < VW; ++i) {
                    mlo = max(mlo, xd[d][h][i] & 0x7FFFu);
                    mhi = max(mhi, xd[d][h][i] & 0x7FFF0000u);
                }
            float m = absmax_bits_value(mlo, mhi);
            // over the LPTOK lanes of the token
#pragma unroll
            for (int o = 1; o < LPTOK; o <<= 1)
                m = fmaxf(m, __shfl_xor(m, o, 64));
            dmax[h] = m;
            if (dj == 0)
                red_max[wave][dt + TPP * h] = m;
        }
        if (lane < 16 && lane >= TOK)
            red_max[wave][lane] = 0.0f;
        __syncthreads();
#pragma unroll
        for (int h = 0; h < NCH; ++h) {
#pragma unroll
            for (int w = 0; w < W; ++w)
                dmax[h] = fmaxf(dmax[h], red_max[w][dt + TPP * h]);
            dsc[h] = dmax[h] / 448.0f;
        }
        // the MFMA-layout lane's token scale (the epilogue's and workgroup
        // 0's copy): the same maximum and quotient
#pragma unroll
        for (int w = 0; w < W; ++w)
            amax = fmaxf(amax, red_max[w][t]);
        sc = amax / 448.0f;
    } else {
        uint32_t mlo = 0, mhi = 0;
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                absmax_bits8(xb[d][j], mlo, mhi);
        amax = absmax_bits_value(mlo, mhi);
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        if (lane < 16)
            red_max[wave][lane] = amax;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < W; ++w)
            amax = fmaxf(amax, red_max[w][t]);
        // 3. the quantizer's scale and codes
        sc = amax / 448.0f;
    }
    const Quot qd(sc);
    // dense: the codes of this wave's steps, [step][token][128], written in
    // the dense layout and read back in the MFMA operand layout
    __shared__ __attribute__((aligned(16))) uint8_t cbuf[DENSE ? W : 1][DENSE ? D * TOK * 128 : 16];
    if constexpr (DENSE) {
#pragma unroll
        for (int h = 0; h < NCH; ++h) {
            const Quot dq(dsc[h]);
            const int tk = dt + TPP * h;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (d >= ns)
                    break;
                uint8_t* const cdst = &cbuf[wave][(d * TOK + tk) * 128 + dj * VPL];
                const int e = (s0 + d) * KSTEP + dj * VPL;
                const bool wq = blockIdx.x == 0 && tk < M && e < K;  // workgroup 0: the codes out
                if constexpr (VPL == 8) {
                    const uint2 c8 = encode8(make_uint4(xd[d][h][0], xd[d][h][1], xd[d][h][2],
                                                        xd[d][h][3]), dq);
                    *(uint2*)cdst = c8;
                    if (wq)
                        *(uint2*)(a.q + (size_t)tk * K + e) = c8;
                } else if constexpr (VPL == 4) {
                    const uint32_t c4 = encode_small<4>(xd[d][h], dq);
                    *(uint32_t*)cdst = c4;
                    if (wq)
                        *(uint32_t*)(a.q + (size_t)tk * K + e) = c4;
                } else {
                    const uint16_t c2 = (uint16_t)encode_small<2>(xd[d][h], dq);
                    *(uint16_t*)cdst = c2;
                    if (wq)
                        *(uint16_t*)(a.q + (size_t)tk * K + e) = c2;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    v4f acc = v4f{0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (d >= ns)
            break;
        uint4 code[2];
        if constexpr (DENSE) {
            // this lane's 32 codes in the MFMA layout (tokens past TOK: zero)
            const uint8_t* cp = &cbuf[wave][(d * TOK + (t < TOK ? t : 0)) * 128 + koff];
            code[0] = t < TOK ? *(const uint4*)cp : make_uint4(0, 0, 0, 0);
            code[1] = t < TOK ? *(const uint4*)(cp + 16) : make_uint4(0, 0, 0, 0);
        } else {
            encode32(xb[d], qd, code);
        }
        if (!DENSE && blockIdx.x == 0 && t < M) {
            const int e = (s0 + d) * KSTEP + koff;
            if (e < K) {
                uint8_t* qp = a.q + (size_t)t * K + e;
                // K is a multiple of 16: the run ends at a 16-byte boundary
                *(uint4*)qp = code[0];
                if (e + 16 < K)
                    *(uint4*)(qp + 16) = code[1];
            }
        }
        // 4. the step's MFMA: weights on the row side, tokens on the column
        // side (the decode GEMM's Swap-AB orientation)
        acc = mfma_step<OP_FP8>(wb[d], code, acc);
    }
    if (blockIdx.x == 0 && wave == 0 && lane < M)
        a.sa[lane] = sc;  // lane < 16: token `lane`, its scale as computed above

    // the 8 partial tiles, added in wave order (the decode GEMM's order)
    __shared__ float red[W][256];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        red[wave][lane * 4 + v] = acc[v];
    // the scale of each output column's token, from the lanes that hold it
    __shared__ float tok_scale[16];
    if (wave == 0 && lane < 16)
        tok_scale[lane] = sc;
    __syncthreads();
    for (int e = threadIdx.x; e < 256; e += W * 64) {
        float sum = red[0][e];
#pragma unroll
        for (int w = 1; w < W; ++w)
            sum += red[w][e];
        // element (lane ln, register v): n = n0 + (ln >> 4) * 4 + v,
        // m = ln & 15
        const int ln = e >> 2, v = e & 3;
        const int n = n0 + (ln >> 4) * 4 + v;
        const int m = ln & 15;
        if (m < M && n < N && (ln >> 4) * 4 + v < HR) {
            const float u = sum * tok_scale[m];
            const float y = u * a.sb[n];
            if (a.out_dtype == OUT_BF16)
                ((uint16_t*)a.out)[(size_t)m * N + n] = bf16_rne(y);
            else
                ((float*)a.out)[(size_t)m * N + n] = y;
        }
    }
}

// K steps (of 128 elements) the busiest of W waves of a workgroup handles.
int fused_steps_per_wave(int K, int W)
{
    const int T = (K + 127) / 128;
    const int U = kFoldUnit / 128;
    const int TU = (T + U - 1) / U;
    int most = 0;
    for (int w = 0; w < W; ++w) {
        const int s0 = std::min(T, U * (w * TU / W));
        const int s1 = std::min(T, U * ((w + 1) * TU / W));
        most = std::max(most, s1 - s0);
    }
    return most;
}

template <int HR, int W, int D, int TOK>
hipError_t launch_fused(const FusedArgs& a, hipStream_t stream)
{
    if (a.M < 1 || a.M > TOK || fused_steps_per_wave(a.K, W) > D || a.N > 0x7FFFFFF0 ||
        2 * (int64_t)a.M * a.K > 0x7FFFFFF0 || (int64_t)HR * a.K > 0x7FFFFFF0)
        return hipErrorInvalidValue;  // (32-bit buffer offsets)
    hipLaunchKernelGGL((linear_fused_kernel<HR, W, D, TOK>), dim3((a.N + HR - 1) / HR),
                       dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qll

#define QLL_FOR_EACH_FUSED(X)                                                              \
    X(16, 8, 2, 16) X(8, 8, 2, 16) X(16, 8, 6, 16) X(8, 8, 6, 16) X(16, 16, 2, 16)          \
    X(8, 16, 2, 16) X(16, 16, 4, 16) X(8, 16, 4, 16)                                        \
    X(16, 8, 2, 4) X(16, 8, 2, 8) X(8, 8, 6, 4) X(8, 8, 6, 8) X(8, 16, 4, 4) X(8, 16, 4, 8) \
    X(16, 16, 2, 4) X(16, 16, 2, 8) X(16, 8, 2, 1) X(16, 8, 2, 2) X(8, 8, 6, 1) X(8, 8, 6, 2)
#define QLL_FUSED_INSTANTIATE(HR, W, D, TOK) \
    template __global__ void qll::linear_fused_kernel<HR, W, D, TOK>(qll::FusedArgs);
QLL_FOR_EACH_FUSED(QLL_FUSED_INSTANTIATE)

namespace qll {

// host-side registry (the device pass only needs the kernels above): HR
// weight rows per workgroup, W waves splitting K (the fold grid of the
// W-wave decode GEMM), D K steps of 128 per wave in registers (W = 8: D = 2
// for K <= 2048, 6 for K <= 6144; W = 16: D = 2 for K <= 4096, 4 for
// K <= 8192)
#if !defined(__HIP_DEVICE_COMPILE__)
#define QLL_FUSED_ENTRY(HR, W, D, TOK) \
    {"f" #HR "x" #TOK "_w" #W "_d" #D, HR, W, D, TOK, &launch_fused<HR, W, D, TOK>},
extern const FusedVariant kFusedVariants[] = {QLL_FOR_EACH_FUSED(QLL_FUSED_ENTRY)};
extern const int kNumFusedVariants = sizeof(kFusedVariants) / sizeof(FusedVariant);
#endif

}  // namespace qll
