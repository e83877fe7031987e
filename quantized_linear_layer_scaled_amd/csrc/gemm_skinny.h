// Skinny-M ("decode") scaled GEMM for gfx950, Swap-AB orientation: weights
// occupy the MFMA row side and the few tokens the column side, which is the
// Swap-AB strategy of "Helion in vLLM: A Unified Route to Tunable Linear
// Kernels" ("What the integration changes") for small M.
//
// For M <= 64 the GEMM streams the weight matrix once and reuses every byte
// M times only, so it is bound by HBM bandwidth and by how many loads are in
// flight.  The tiled kernel's LDS staging buys nothing here, so this kernel:
//   * loads both operands straight from global memory into registers in MFMA
//     operand layout (each lane: a contiguous 16/32-byte run of one K-major
//     row -- the weights are read exactly once, coalesced per row);
//   * gives each workgroup 16 weight rows and lets its W waves split the K
//     range among themselves (KSPLIT), so that even N = 2048 yields W x 128
//     independent streams; D MFMA steps of loads are issued before their
//     MFMAs to keep many bytes in flight per wave;
//   * HR = 8 gives a workgroup 8 weight rows only (the MFMA's other 8 rows
//     are zero): twice the workgroups, so that a weight matrix of 2048 rows
//     spreads over all 256 CUs instead of 128;
//   * adds the W partial tiles through LDS in a fixed order (wave 0, 1, ...,
//     W-1), so the result is deterministic and needs no second kernel.
//   Without KSPLIT each wave owns 16 weight rows and the whole K range (used
//   by the batch-invariant op, whose K reduction must not change with M).
// Cross-workgroup Split-K (blockIdx.z) composes with this exactly as in the
// tiled kernel: each piece is reduced in-workgroup, then the pieces are added
// in ascending order by the second-stage kernel.
#pragma once

#include "gemm_tile.h"

namespace qll {

template <int OP, int RQ, int W, int HR, bool KSPLIT, int D>
__global__ __launch_bounds__(W * 64) void gemm_skinny_kernel(GemmArgs a)
{
    static_assert(HR == 16 || (HR == 8 && KSPLIT), "8-row workgroups split K over waves");
    using Tr = OpTraits<OP>;
    using acc_t = typename Tr::acc_t;
    using elem_t = typename Tr::elem_t;
    constexpr int KB = Tr::kb;
    constexpr int KSTEP = 4 * KB;
    constexpr int NJ = KB / 16;  // 16-byte loads per operand per step

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int N = a.N, M = a.M;
    const int n0 = KSPLIT ? blockIdx.x * HR : (blockIdx.x * W + wave) * 16;
    const bool wrow = (lane & 15) < HR;  // this lane loads a weight row
    const int m0 = blockIdx.y * (16 * RQ);
    const int z = blockIdx.z;
    const int kbeg = z * a.kchunk;
    const int kend = min(a.kbytes, kbeg + a.kchunk);
    // the waves split K on the same grid of kFoldUnit-byte units as the
    // chunked summation of the other bf16 kernels
    constexpr int U = kFoldUnit / KSTEP;
    const int T = (kend - kbeg + KSTEP - 1) / KSTEP;
    const int TU = (T + U - 1) / U;
    const int s0 = KSPLIT ? min(T, U * (wave * TU / W)) : 0;
    const int s1 = KSPLIT ? min(T, U * ((wave + 1) * TU / W)) : T;
    const size_t ldk = (size_t)a.kbytes;

    // rows this lane loads (clamped: out-of-range rows are masked at the store)
    const int nrow = min(n0 + (lane & 15), N - 1);
    const uint8_t* __restrict__ bp =
        (const uint8_t*)a.B + (size_t)nrow * ldk + kbeg + (lane >> 4) * KB;
    const uint8_t* __restrict__ ap[RQ];
#pragma unroll
    for (int r = 0; r < RQ; ++r) {
        const int mrow = min(m0 + r * 16 + (lane & 15), M - 1);
        ap[r] = (const uint8_t*)a.A + (size_t)mrow * ldk + kbeg + (lane >> 4) * KB;
    }
    const int klim = kend - kbeg - (lane >> 4) * KB;  // bytes this lane may read

    // MXFP4: each row's E8M0 scales, one byte per 32 K elements (16 bytes of
    // codes); the scale dword of step t holds the four blocks of that step,
    // and this lane's block is byte lane >> 4 of it.
    constexpr bool MX = OP == OP_MXFP4;
    const int srow = a.kbytes / 16;  // scale bytes per row
    const uint8_t* __restrict__ sbp =
        (const uint8_t*)a.sb + (size_t)nrow * srow + kbeg / 16;
    const uint8_t* __restrict__ sap[RQ];
#pragma unroll
    for (int r = 0; r < RQ; ++r) {
        const int mrow = min(m0 + r * 16 + (lane & 15), M - 1);
        sap[r] = (const uint8_t*)a.sa + (size_t)mrow * srow + kbeg / 16;
    }
    const int sshift = 8 * (lane >> 4);

    acc_t acc[RQ];
#pragma unroll
    for (int r = 0; r < RQ; ++r)
        acc[r] = acc_t{0, 0, 0, 0};

    const int KG = a.K / 128;
    const int nb = (min(n0, N - 1) >> 7);  // 16 weight rows share one 128-row block

    // bf16 without the wave split: chunked K summation (kBiFold); with the
    // wave split the chunks are the waves themselves (W must equal kfold).
    constexpr bool FOLD = OP == OP_BF16 && !KSPLIT;
    KFold<acc_t, 1, RQ> fold(FOLD ? a.kfold : 1, T, U);

    // Block-FP8: the group scales of each step (weight block nb, and each
    // token row's), loaded with the operands so that they are in flight
    // together instead of one more round trip before the promotion
    constexpr bool BLK = OP == OP_BLOCK;
    for (int s = s0; s < s1; s += D) {
        uint4 fb[D][NJ], fa[D][RQ][NJ];
        uint32_t xb[MX ? D : 1], xa[MX ? D : 1][RQ];
        float gb[BLK ? D : 1], ga[BLK ? D : 1][RQ];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int off = (s + d) * KSTEP;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const bool ok = (s + d < s1) && (off + 16 * j < klim);
                fb[d][j] = ok && wrow ? *(const uint4*)(bp + off + 16 * j)
                                      : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < RQ; ++r)
                    fa[d][r][j] = ok ? *(const uint4*)(ap[r] + off + 16 * j)
                                     : make_uint4(0, 0, 0, 0);
            }
            if constexpr (BLK) {
                // step s + d is K group (kbeg >> 7) + s + d (KSTEP = 128)
                const bool ok = s + d < s1;
                const int g = (kbeg >> 7) + s + d;
                gb[d] = ok ? a.sb[nb * KG + g] : 0.0f;
#pragma unroll
                for (int r = 0; r < RQ; ++r) {
                    const int m = min(m0 + r * 16 + (lane & 15), M - 1);
                    ga[d][r] = ok ? a.sa[m * KG + g] : 0.0f;
                }
            }
            if constexpr (MX) {
                // a whole step is in range or not (K is a multiple of 128)
                const bool ok = (s + d < s1) && (off < klim);
                xb[d] = ok && wrow ? *(const uint32_t*)(sbp + 4 * (s + d)) : 0u;
#pragma unroll
                for (int r = 0; r < RQ; ++r)
                    xa[d][r] = ok ? *(const uint32_t*)(sap[r] + 4 * (s + d)) : 0u;
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (s + d >= s1)
                continue;  // (every later step is past s1 too)
            if constexpr (FOLD)
                fold.before(s + d, (acc_t(&)[1][RQ])acc);
            if constexpr (BLK) {
#pragma unroll
                for (int r = 0; r < RQ; ++r) {
                    const float sc = gb[d] * ga[d][r];
                    v4f pg = mfma_step<OP>(fb[d], fa[d][r], v4f{0, 0, 0, 0});
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[r][v] = __builtin_fmaf(sc, pg[v], acc[r][v]);
                }
            } else if constexpr (MX) {
                const int xw = (int)__builtin_amdgcn_ubfe(xb[d], sshift, 8);
#pragma unroll
                for (int r = 0; r < RQ; ++r)
                    acc[r] = mfma_mx(fb[d][0], fa[d][r][0], acc[r], xw,
                                     (int)__builtin_amdgcn_ubfe(xa[d][r], sshift, 8));
            } else {
#pragma unroll
                for (int r = 0; r < RQ; ++r)
                    acc[r] = mfma_step<OP>(fb[d], fa[d][r], acc[r]);
            }
        }
    }

    if constexpr (FOLD)
        fold.finish((acc_t(&)[1][RQ])acc);

    // Output element (r, lane, v): n = n0 + (lane >> 4) * 4 + v,
    //                              m = m0 + r * 16 + (lane & 15).
    auto emit = [&](int r, int ln, int v, elem_t e) __attribute__((always_inline)) {
        const int n = n0 + (ln >> 4) * 4 + v;
        const int m = m0 + r * 16 + (ln & 15);
        if (m < M && n < N && (ln >> 4) * 4 + v < HR) {
            if (a.splits > 1)
                ((elem_t*)a.ws)[((size_t)z * M + m) * N + n] = e;
            else
                store_one<OP>(a, (size_t)m * N + n, e, m, n);
        }
    };

    if constexpr (!KSPLIT) {
#pragma unroll
        for (int r = 0; r < RQ; ++r)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                emit(r, lane, v, acc[r][v]);
    } else {
        __shared__ elem_t red[W][RQ * 256];
#pragma unroll
        for (int r = 0; r < RQ; ++r)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[wave][r * 256 + lane * 4 + v] = acc[r][v];
        __syncthreads();
        for (int e = threadIdx.x; e < RQ * 256; e += W * 64) {
            elem_t sum = red[0][e];
#pragma unroll
            for (int w = 1; w < W; ++w)
                sum += red[w][e];
            emit(e >> 8, (e & 255) >> 2, e & 3, sum);
        }
    }
}

template <int OP, int RQ, int W, int HR, bool KSPLIT, int D>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream)
{
    const int rows = KSPLIT ? HR : 16 * W;
    dim3 grid((a.N + rows - 1) / rows, (a.M + 16 * RQ - 1) / (16 * RQ), a.splits);
    if (grid.y > 65535 || grid.z > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_skinny_kernel<OP, RQ, W, HR, KSPLIT, D>), grid, dim3(W * 64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace qll

// Registry entries of the skinny kernel.  Name: "k" (waves split K) or "r"
// (waves split rows), weight rows x tokens per workgroup, waves (the wp
// field holds the wave count).
// X(OP, RQ, TOKENS, W, KSPLIT, D, HR) is applied to every entry.
// D is the number of K steps whose loads are in flight together: enough for
// a wave's whole K chunk at K = 6144 (fp8) for the wave-split kernels, so the
// weight stream costs one memory round trip.
#define QLL_FOR_EACH_SKINNY(X, OP, DM)     \
    X(OP, 1, 16, 8, true, 6 * (DM), 16)    \
    X(OP, 2, 32, 8, true, 4 * (DM), 16)    \
    X(OP, 4, 64, 8, true, 4 * (DM), 16)    \
    X(OP, 1, 16, 16, true, 4 * (DM), 16)   \
    X(OP, 1, 16, 4, false, 4 * (DM), 16)   \
    X(OP, 2, 32, 4, false, 4 * (DM), 16)   \
    X(OP, 4, 64, 4, false, 2 * (DM), 16)   \
    X(OP, 1, 16, 8, true, 6 * (DM), 8)     \
    X(OP, 1, 16, 16, true, 4 * (DM), 8)    \
    X(OP, 2, 32, 8, true, 4 * (DM), 8)

#define QLL_SKINNY_INSTANTIATE(OP, RQ, TOK, W, KS, D, HR) \
    template __global__ void qll::gemm_skinny_kernel<OP, RQ, W, HR, KS, D>(qll::GemmArgs);
#define QLL_SKINNY_ENTRY(OP, RQ, TOK, W, KS, D, HR)                                   \
    {(KS) ? "k" #HR "x" #TOK "_w" #W : "r16x" #TOK "_w" #W, OP, 1, (KS) ? (HR) : 16 * (W), \
     TOK, W, 1, 0, (KS) ? (W) * (RQ) * 1024 : 0,                                        \
     &qll::launch_skinny<OP, RQ, W, HR, KS, D>},
