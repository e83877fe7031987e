// Tiled scaled GEMM for gfx950: one kernel template behind every GEMM of the
// library (W8A8 INT8, FP8 per-token x per-channel, Block-FP8, bf16), in the
// ordinary orientation or as Swap-AB, with or without Split-K.  These are the
// strategies of "Helion in vLLM: A Unified Route to Tunable Linear Kernels",
// section "What the integration changes".
//
// Design (CDNA4):
//   * Both operands are K-contiguous ([M][K] activations, [N][K] weights), so
//     every lane of a 16x16 MFMA reads a contiguous 16- or 32-byte run of one
//     row: int8 v_mfma_i32_16x16x64_i8 and bf16 v_mfma_f32_16x16x32_bf16 take
//     16 bytes per lane, fp8 v_mfma_f32_16x16x128_f8f6f4 takes 32 bytes.
//   * A workgroup owns a BP x BQ output tile; its waves form a WP x WQ grid and
//     each wave owns (BP/WP) x (BQ/WQ) = RP x RQ blocks of 16x16.
//   * K advances KSTAGE bytes per iteration.  Tiles are staged through LDS in
//     two buffers: 128-bit coalesced global loads for stage k+1 are in flight
//     while the MFMAs consume stage k.  Each 16-byte chunk of an LDS row is
//     XOR-swizzled with the row index so that the 16 lanes reading one column
//     of chunks from 16 rows spread over the banks.
//   * Split-K: blockIdx.y selects a contiguous K piece; the partial tile goes
//     to the caller's workspace and a second kernel adds the pieces in
//     ascending order (no atomics, deterministic).
//   * Every output element accumulates its K range in ascending k, one MFMA
//     K-slab after another, whatever the tile shape; so only the MFMA kind and
//     the split boundaries decide the rounding, which is what the
//     batch-invariant entry point relies on.
#pragma once

#include <type_traits>

#include "qll_internal.h"

namespace qll {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int OP> struct OpTraits;
template <> struct OpTraits<OP_INT8> {
    static constexpr int esz = 1, kb = 16;  // bytes per lane per MFMA
    using acc_t = v4i;
    using elem_t = int;
};
template <> struct OpTraits<OP_FP8> {
    static constexpr int esz = 1, kb = 32;
    using acc_t = v4f;
    using elem_t = float;
};
template <> struct OpTraits<OP_BLOCK> {
    static constexpr int esz = 1, kb = 32;
    using acc_t = v4f;
    using elem_t = float;
};
template <> struct OpTraits<OP_BF16> {
    static constexpr int esz = 2, kb = 16;
    using acc_t = v4f;
    using elem_t = float;
};
// MXFP4: two E2M1 codes per byte, 32 codes (16 bytes) per lane per MFMA,
// E8M0 block scales applied inside the matrix core
template <> struct OpTraits<OP_MXFP4> {
    static constexpr int esz = 1, kb = 16;
    using acc_t = v4f;
    using elem_t = float;
};
// W4A16: bf16 activations (16 bytes per lane per bf16 MFMA), int4 weights
// widened to bf16 in registers
template <> struct OpTraits<OP_W4A16> {
    static constexpr int esz = 2, kb = 16;
    using acc_t = v4f;
    using elem_t = float;
};

// Workgroup -> output tile, XCD-aware.  The dispatcher hands consecutive
// workgroup ids to the 8 XCDs in turn, and each XCD has its own L2.  The
// tiles are numbered so that the workgroups one XCD receives form one
// contiguous run t = xcd * per + local, and that run is laid out in groups of
// `group` tile rows (tile_p fastest), so an XCD works on a compact block of
// tiles that share A rows and B rows in its L2.  The map is a bijection of
// [0, tp * tq) for any tile count and group; only locality depends on the
// dispatch order.  (Groups chosen to make an XCD's block square measured
// slower than four tile rows: the workgroups running at the same time share
// rows better in the taller-than-wide arrangement.)
__device__ __forceinline__ void xcd_tile(int bid, int tp, int tq, int group,
                                         int& tile_p, int& tile_q)
{
    const int T = tp * tq;
    const int per = T >> 3, rem = T & 7;
    const int xcd = bid & 7, loc = bid >> 3;
    const int t = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    const int span = group * tq;
    const int first = (t / span) * group;
    const int gsize = min(tp - first, group);
    tile_p = first + (t % span) % gsize;
    tile_q = (t % span) / gsize;
}

template <int OP>
__device__ __forceinline__ typename OpTraits<OP>::acc_t
mfma_step(const uint4* a, const uint4* b, typename OpTraits<OP>::acc_t c)
{
    if constexpr (OP == OP_INT8) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(
            __builtin_bit_cast(v4i, a[0]), __builtin_bit_cast(v4i, b[0]), c, 0,
            0, 0);
    } else if constexpr (OP == OP_BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8bf, a[0]), __builtin_bit_cast(v8bf, b[0]), c,
            0, 0, 0);
    } else {
        // e4m3 x e4m3 (format code 0 for both operands), no block scaling:
        // the scale operands are zero, which selects the unscaled
        // v_mfma_f32_16x16x128_f8f6f4.
        v8i av, bv;
        av.lo = __builtin_bit_cast(v4i, a[0]);
        av.hi = __builtin_bit_cast(v4i, a[1]);
        bv.lo = __builtin_bit_cast(v4i, b[0]);
        bv.hi = __builtin_bit_cast(v4i, b[1]);
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0,
                                                                0, 0, 0, 0);
    }
}

// One block-scaled MXFP4 step, 16 x 16 x 128 (format code 4 = E2M1 for both
// operands; only the first four dwords of each operand carry codes).  Lane l
// supplies the 32 K elements (l >> 4) * 32 .. + 31 of row l & 15 of each
// operand and, in bits 0-7 of sa / sb (byte select 0), the E8M0 scale of
// exactly that block of 32: v_mfma_scale_f32_16x16x128_f8f6f4.
__device__ __forceinline__ v4f mfma_mx(const uint4& a, const uint4& b, v4f c, int sa, int sb)
{
    v8i av, bv;
    av.lo = __builtin_bit_cast(v4i, a);
    av.hi = v4i{0, 0, 0, 0};
    bv.lo = __builtin_bit_cast(v4i, b);
    bv.hi = v4i{0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

// XOR swizzle of the 16-byte chunks of one staged LDS row.  A fragment read
// has 16 lanes reading the same logical chunk of 16 consecutive rows; with
// NC chunks per row the physical chunk is c ^ swz(row), and swz makes both
// the first 8 and the first 16 rows of every 16-row group hit distinct
// 16-byte bank groups whether the LDS serves 8 or 16 lanes of a b128 read per
// cycle (NC = 8: swz = (row ^ row / 8) mod 8; NC = 16: swz = row mod 16).
template <int NC>
__device__ __forceinline__ int swz(int row)
{
    return (row ^ (row / NC)) & (NC - 1);
}

__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two values rounded to bf16 (nearest even) and packed, lo in bits 0..15:
// gfx950's v_cvt_pk_bf16_f32, one instruction for the pair.  For finite
// values and infinities it gives bf16_rne's bits.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi)
{
    typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
    typedef float f2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, bf2_t));
}

// The value of lane l ^ 1 (a DPP quad permute [1, 0, 3, 2]).
__device__ __forceinline__ float lane_pair_swap(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// Epilogue value of one accumulator element (before the output cast).
template <int OP>
__device__ __forceinline__ float epilogue_value(typename OpTraits<OP>::elem_t v,
                                                const GemmArgs& a, int m, int n)
{
    if constexpr (OP == OP_INT8) {
        float t = (float)v * a.sa[m];
        return t * a.sb[n];
    } else if constexpr (OP == OP_FP8) {
        float t = v * a.sa[m];
        return t * a.sb[n];
    } else {
        return v;
    }
}

template <int OP>
__device__ __forceinline__ void store_one(const GemmArgs& a, size_t idx,
                                          typename OpTraits<OP>::elem_t v,
                                          int m, int n)
{
    if constexpr (OP == OP_INT8) {
        if (a.out_dtype == OUT_INT32) {
            ((int*)a.out)[idx] = v;
            return;
        }
    }
    float y = epilogue_value<OP>(v, a, m, n);
    if (a.out_dtype == OUT_BF16)
        ((uint16_t*)a.out)[idx] = bf16_rne(y);
    else
        ((float*)a.out)[idx] = y;
}

// Chunked K summation of the bf16 kernels (see kBiFold): the T MFMA steps of
// a K piece form F chunks on a grid of U-step units (TU = ceil(T / U) units,
// chunk w = units [w*TU/F, (w+1)*TU/F), clipped to T); each chunk is summed
// from zero and the chunk sums are added in ascending order.  before(step)
// closes the running chunk when `step` is a chunk boundary; finish() closes
// the rest and leaves the result in acc.  With U a multiple of the steps per
// K stage, every boundary falls on a stage start.
template <typename acc_t, int RP, int RQ>
struct KFold {
    acc_t tot[RP][RQ];
    int next = 1, at, F, T, U, TU;
    bool first = true;
    __device__ __forceinline__ KFold(int f, int t, int u) : F(f), T(t), U(u)
    {
        TU = (T + U - 1) / U;
        at = F > 1 ? min(T, U * (TU / F)) : 0x7FFFFFFF;
    }
    __device__ __forceinline__ void close(acc_t (&acc)[RP][RQ])
    {
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int j = 0; j < RQ; ++j) {
                tot[i][j] = first ? acc[i][j] : tot[i][j] + acc[i][j];
                acc[i][j] = acc_t{0, 0, 0, 0};
            }
        first = false;
    }
    __device__ __forceinline__ void before(int step, acc_t (&acc)[RP][RQ])
    {
        while (step == at) {
            close(acc);
            ++next;
            at = next < F ? min(T, U * (next * TU / F)) : 0x7FFFFFFF;
        }
    }
    __device__ __forceinline__ void finish(acc_t (&acc)[RP][RQ])
    {
        if (F <= 1)
            return;
        while (next <= F) {
            close(acc);
            ++next;
        }
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int j = 0; j < RQ; ++j)
                acc[i][j] = tot[i][j];
    }
};

template <int OP, int SWAP, int BP, int BQ, int WP, int WQ, int KSTAGE>
__global__ __launch_bounds__(WP* WQ * 64) void gemm_tile_kernel(GemmArgs a)
{
    using Tr = OpTraits<OP>;
    using acc_t = typename Tr::acc_t;
    using elem_t = typename Tr::elem_t;
    constexpr int THREADS = WP * WQ * 64;
    constexpr int NC = KSTAGE / 16;  // 16-byte chunks per staged row
    constexpr int KB = Tr::kb;
    constexpr int KSTEP = 4 * KB;    // bytes of K per MFMA
    constexpr int NSTEP = KSTAGE / KSTEP;
    constexpr int SP = BP / WP, SQ = BQ / WQ;  // per-wave extent
    constexpr int RP = SP / 16, RQ = SQ / 16;
    constexpr int LP = (BP * NC + THREADS - 1) / THREADS;
    constexpr int LQ = (BQ * NC + THREADS - 1) / THREADS;
    constexpr int STAGE_BYTES = (BP + BQ) * KSTAGE;
    static_assert(KSTAGE % KSTEP == 0 && RP >= 1 && RQ >= 1, "bad tile");
    static_assert((NC & (NC - 1)) == 0, "KSTAGE must be a power of two");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wpi = wave % WP, wqi = wave / WP;

    const int Pdim = SWAP ? a.N : a.M;
    const int Qdim = SWAP ? a.M : a.N;
    const uint8_t* __restrict__ Pptr = (const uint8_t*)(SWAP ? a.B : a.A);
    const uint8_t* __restrict__ Qptr = (const uint8_t*)(SWAP ? a.A : a.B);
    const int tp = (Pdim + BP - 1) / BP;
    const int tile_p = blockIdx.x % tp, tile_q = blockIdx.x / tp;
    const int p0 = tile_p * BP, q0 = tile_q * BQ;
    const int z = blockIdx.y;
    const int kbeg = z * a.kchunk;
    const int kend = min(a.kbytes, kbeg + a.kchunk);
    const int nk = (kend - kbeg + KSTAGE - 1) / KSTAGE;
    const size_t ldk = (size_t)a.kbytes;

    uint4 rp[LP], rq[LQ];

    auto gload = [&](int kt) __attribute__((always_inline)) {
        const int kb0 = kbeg + kt * KSTAGE;
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const int c = tid + i * THREADS;
            const int row = c / NC, ch = c % NC;
            const int gr = p0 + row, kb = kb0 + ch * 16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if ((BP * NC % THREADS == 0 || c < BP * NC) && gr < Pdim && kb < kend)
                v = *(const uint4*)(Pptr + (size_t)gr * ldk + kb);
            rp[i] = v;
        }
#pragma unroll
        for (int i = 0; i < LQ; ++i) {
            const int c = tid + i * THREADS;
            const int row = c / NC, ch = c % NC;
            const int gr = q0 + row, kb = kb0 + ch * 16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if ((BQ * NC % THREADS == 0 || c < BQ * NC) && gr < Qdim && kb < kend)
                v = *(const uint4*)(Qptr + (size_t)gr * ldk + kb);
            rq[i] = v;
        }
    };

    auto sstore = [&](int buf) __attribute__((always_inline)) {
        uint8_t* sp = lds + buf * STAGE_BYTES;
        uint8_t* sq = sp + BP * KSTAGE;
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const int c = tid + i * THREADS;
            if (BP * NC % THREADS == 0 || c < BP * NC) {
                const int row = c / NC, ch = c % NC;
                *(uint4*)(sp + row * KSTAGE + ((ch ^ swz<NC>(row)) << 4)) = rp[i];
            }
        }
#pragma unroll
        for (int i = 0; i < LQ; ++i) {
            const int c = tid + i * THREADS;
            if (BQ * NC % THREADS == 0 || c < BQ * NC) {
                const int row = c / NC, ch = c % NC;
                *(uint4*)(sq + row * KSTAGE + ((ch ^ swz<NC>(row)) << 4)) = rq[i];
            }
        }
    };

    acc_t acc[RP][RQ];
#pragma unroll
    for (int i = 0; i < RP; ++i)
#pragma unroll
        for (int j = 0; j < RQ; ++j)
            acc[i][j] = acc_t{0, 0, 0, 0};

    constexpr bool FOLD = OP == OP_BF16;
    KFold<acc_t, RP, RQ> fold(FOLD ? a.kfold : 1, (kend - kbeg + KSTEP - 1) / KSTEP,
                              kFoldUnit / KSTEP);
    static_assert(!FOLD || (kFoldUnit / KSTEP) % NSTEP == 0, "fold grid must align to stages");

    // Block-FP8 scale bookkeeping: the rows/columns of this lane.
    const int KG = a.K / 128;
    int prow[RP][4];
    int qcol[RQ];
    if constexpr (OP == OP_BLOCK) {
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                prow[i][v] = min(p0 + wpi * SP + i * 16 + (lane >> 4) * 4 + v, Pdim - 1);
#pragma unroll
        for (int j = 0; j < RQ; ++j)
            qcol[j] = min(q0 + wqi * SQ + j * 16 + (lane & 15), Qdim - 1);
    }

    auto compute = [&](int buf, int kt) __attribute__((always_inline)) {
        if constexpr (FOLD)
            fold.before(kt * NSTEP, acc);  // chunk boundaries fall on stage starts
        const uint8_t* sp = lds + buf * STAGE_BYTES;
        const uint8_t* sq = sp + BP * KSTAGE;
#pragma unroll
        for (int ks = 0; ks < NSTEP; ++ks) {
            // steps wholly past the end of this K piece are skipped, so every
            // variant issues the same MFMA sequence for an output element
            if (kbeg + kt * KSTAGE + ks * KSTEP >= kend)
                break;
            uint4 fa[RP][KB / 16], fb[RQ][KB / 16];
            const int off = ks * KSTEP + (lane >> 4) * KB;
#pragma unroll
            for (int i = 0; i < RP; ++i) {
                const int row = wpi * SP + i * 16 + (lane & 15);
#pragma unroll
                for (int j = 0; j < KB / 16; ++j) {
                    const int ch = (off >> 4) + j;
                    fa[i][j] = *(const uint4*)(sp + row * KSTAGE + ((ch ^ swz<NC>(row)) << 4));
                }
            }
#pragma unroll
            for (int i = 0; i < RQ; ++i) {
                const int row = wqi * SQ + i * 16 + (lane & 15);
#pragma unroll
                for (int j = 0; j < KB / 16; ++j) {
                    const int ch = (off >> 4) + j;
                    fb[i][j] = *(const uint4*)(sq + row * KSTAGE + ((ch ^ swz<NC>(row)) << 4));
                }
            }
            if constexpr (OP == OP_BLOCK) {
                const int g = (kbeg + kt * KSTAGE + ks * KSTEP) >> 7;
                float ps[RP][4], qs[RQ];
#pragma unroll
                for (int i = 0; i < RP; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        ps[i][v] = SWAP ? a.sb[(prow[i][v] >> 7) * KG + g]
                                        : a.sa[prow[i][v] * KG + g];
#pragma unroll
                for (int j = 0; j < RQ; ++j)
                    qs[j] = SWAP ? a.sa[qcol[j] * KG + g]
                                 : a.sb[(qcol[j] >> 7) * KG + g];
#pragma unroll
                for (int i = 0; i < RP; ++i)
#pragma unroll
                    for (int j = 0; j < RQ; ++j) {
                        v4f pg = mfma_step<OP>(fa[i], fb[j], v4f{0, 0, 0, 0});
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[i][j][v] = __builtin_fmaf(ps[i][v] * qs[j], pg[v], acc[i][j][v]);
                    }
            } else {
#pragma unroll
                for (int i = 0; i < RP; ++i)
#pragma unroll
                    for (int j = 0; j < RQ; ++j)
                        acc[i][j] = mfma_step<OP>(fa[i], fb[j], acc[i][j]);
            }
        }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk)
            gload(kt + 1);
        compute(cur, kt);
        if (kt + 1 < nk)
            sstore(cur ^ 1);
        __syncthreads();
    }

    if constexpr (FOLD)
        fold.finish(acc);

    // Epilogue.
    const int M = a.M, N = a.N;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
#pragma unroll
        for (int j = 0; j < RQ; ++j) {
            const int pb = p0 + wpi * SP + i * 16 + (lane >> 4) * 4;
            const int q = q0 + wqi * SQ + j * 16 + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int p = pb + v;
                const int m = SWAP ? q : p;
                const int n = SWAP ? p : q;
                if (m < M && n < N) {
                    const elem_t e = acc[i][j][v];
                    if (a.splits > 1) {
                        ((elem_t*)a.ws)[((size_t)z * M + m) * N + n] = e;
                    } else {
                        store_one<OP>(a, (size_t)m * N + n, e, m, n);
                    }
                }
            }
        }
    }
}

template <int OP, int SWAP, int BP, int BQ, int WP, int WQ, int KSTAGE>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream)
{
    const int Pdim = SWAP ? a.N : a.M;
    const int Qdim = SWAP ? a.M : a.N;
    const long tiles = (long)((Pdim + BP - 1) / BP) * ((Qdim + BQ - 1) / BQ);
    if (tiles > 0x7FFFFFFFL)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)tiles, (unsigned)a.splits);
    hipLaunchKernelGGL((gemm_tile_kernel<OP, SWAP, BP, BQ, WP, WQ, KSTAGE>), grid,
                       dim3(WP * WQ * 64), 0, stream, a);
    return hipGetLastError();
}

// Second Split-K stage: each thread owns up to 4 consecutive columns of one
// row and adds the partials of the pieces s = 0, 1, ..., S-1 in that order.
// The partials were just stored by other CUs (an L2 or Infinity Cache round
// trip each), so they are loaded kReduceBatch pieces at a time, all loads of
// a batch in flight before the first add.
constexpr int kReduceThreads = 128;
constexpr int kReduceBatch = 8;

template <int OP>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(GemmArgs a)
{
    using elem_t = typename OpTraits<OP>::elem_t;
    typedef elem_t v4e __attribute__((ext_vector_type(4)));
    constexpr int ZB = kReduceBatch;
    const int NQ = (a.N + 3) / 4;
    const long idx = (long)blockIdx.x * kReduceThreads + threadIdx.x;
    if (idx >= (long)a.M * NQ)
        return;
    const int m = (int)(idx / NQ);
    const int n0 = (int)(idx % NQ) * 4;
    const elem_t* ws = (const elem_t*)a.ws;
    const size_t plane = (size_t)a.M * a.N;
    const size_t base = (size_t)m * a.N + n0;
    const bool vec = (a.N & 3) == 0;
    elem_t s[4] = {0, 0, 0, 0};
    for (int z0 = 0; z0 < a.splits; z0 += ZB) {
        v4e t[ZB];
#pragma unroll
        for (int j = 0; j < ZB; ++j) {
            t[j] = v4e{0, 0, 0, 0};
            if (z0 + j < a.splits) {
                const elem_t* src = ws + (size_t)(z0 + j) * plane + base;
                if (vec) {
                    t[j] = *(const v4e*)src;
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (n0 + c < a.N)
                            t[j][c] = src[c];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < ZB; ++j)
            if (z0 + j < a.splits)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    s[c] += t[j][c];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (n0 + j < a.N)
            store_one<OP>(a, base + j, s[j], m, n0 + j);
}

template <int OP>
hipError_t launch_reduce(const GemmArgs& a, hipStream_t stream)
{
    const long total = (long)a.M * ((a.N + 3) / 4);
    const long blocks = (total + kReduceThreads - 1) / kReduceThreads;
    if (blocks > 0x7FFFFFFFL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(splitk_reduce_kernel<OP>, dim3((unsigned)blocks),
                       dim3(kReduceThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qll

// One registry entry: orientation (n = ordinary, s = Swap-AB), tile BPxBQ,
// wave grid WPxWQ, K stage bytes.
#define QLL_VARIANT(OP, SW, BP, BQ, WP, WQ, KS)                                \
    {(SW) ? "s" #BP "x" #BQ "_w" #WP "x" #WQ "_k" #KS                            \
          : "n" #BP "x" #BQ "_w" #WP "x" #WQ "_k" #KS,                           \
     OP, SW, BP, BQ, WP, WQ, KS, 2 * ((BP) + (BQ)) * (KS),                      \
     &qll::launch_tile<OP, SW, BP, BQ, WP, WQ, KS>}
