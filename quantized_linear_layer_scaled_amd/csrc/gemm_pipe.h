// Pipelined large-M scaled GEMM for gfx950 (ordinary orientation: tokens on
// the MFMA row side), the compute-bound member of the "ordinary GEMM"
// strategy of "Helion in vLLM: A Unified Route to Tunable Linear Kernels"
// ("What the integration changes").
//
// The plain tiled kernel prefetches one stage into registers, so every K step
// waits for a full global-memory round trip.  Here:
//   * operands go from global memory straight into LDS with
//     global_load_lds_dwordx4 (no VGPR staging, no ds_write), STAGES-1 stages
//     ahead, in a ring of STAGES LDS buffers (the K loop is unrolled by
//     STAGES so that every slot is a compile-time LDS object);
//   * a wave waits only for its own oldest stage (s_waitcnt vmcnt(N) with N
//     the loads of the younger stages still allowed in flight) and then meets
//     the other waves at one s_barrier per stage -- the barrier also frees the
//     buffer that the next prefetch overwrites;
//   * each lane's 64 destination bytes are fixed by the hardware (lane i of a
//     wave writes bytes 16i..16i+15 of the wave's 1 KiB block), so the XOR
//     swizzle of 16-byte chunks is applied on the global side: the lane that
//     fills LDS chunk (row, j) fetches logical chunk j ^ swz(row);
//   * loads past the end of the K range read a 16-byte zero block, so the
//     K tail needs no masking in the MFMA loop; rows past M or N are clamped
//     (their outputs are discarded at the store).
// Output element accumulation is the same ascending sequence of MFMA K steps
// as in the other kernels, so results are bitwise equal to theirs for the
// same K split.
#pragma once

#include <type_traits>

#include "gemm_tile.h"

namespace qll {

// 16 zero bytes that loads past the K range read (one copy per translation
// unit; never written).
static __device__ __attribute__((aligned(16))) uint4 g_zero16[1];

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane i
// of the wave writes LDS bytes lds_base + 16 i .. + 15.  Issued from inline
// asm so that the compiler, which cannot tell the ring slots apart, does not
// add a wait for every copy in flight before each LDS read; the only
// synchronization is the explicit vmcnt wait + barrier below.  The asm has no
// register outputs; M0 is set inside the same block.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 ::"v"(g), "s"(lds_base)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// SPLITK only gives the first stage of a Split-K call its own kernel symbol
// (the code is the same), so that traces separate the two kinds of launch.
template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int STAGES, bool SPLITK>
__global__ __launch_bounds__(WP* WQ * 64) void gemm_pipe_kernel(GemmArgs a)
{
    using Tr = OpTraits<OP>;
    using acc_t = typename Tr::acc_t;
    using elem_t = typename Tr::elem_t;
    constexpr int WAVES = WP * WQ;
    constexpr int THREADS = WAVES * 64;
    constexpr int NC = KSTAGE / 16;
    constexpr int KB = Tr::kb;
    constexpr int KSTEP = 4 * KB;
    constexpr int NSTEP = KSTAGE / KSTEP;
    constexpr int SP = BP / WP, SQ = BQ / WQ;
    constexpr int RP = SP / 16, RQ = SQ / 16;
    constexpr int ROWS = BP + BQ;
    constexpr int LPT = ROWS * NC / THREADS;  // loads per thread per stage
    constexpr int STAGE_BYTES = ROWS * KSTAGE;
    static_assert(ROWS * NC % THREADS == 0, "stage must split evenly over the waves");
    static_assert((NC & (NC - 1)) == 0 && KSTAGE % KSTEP == 0, "bad K stage");
    static_assert(STAGES >= 2 && (STAGES - 2) * LPT < 64, "bad pipeline depth");
    static_assert(OP != OP_BLOCK, "block scaling is not pipelined here");

    // One LDS object per ring slot, the slot known at compile time in the
    // unrolled K loop (constant LDS addresses for the fragment reads).
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[STAGES >= 3 ? STAGE_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[STAGES >= 4 ? STAGE_BYTES : 16];
    static_assert(STAGES <= 4, "at most four ring slots");
    auto slot = [&](auto J) __attribute__((always_inline)) -> uint8_t* {
        constexpr int j = decltype(J)::value;
        if constexpr (j == 0)
            return lds0;
        else if constexpr (j == 1)
            return lds1;
        else if constexpr (j == 2)
            return lds2;
        else
            return lds3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wpi = wave % WP, wqi = wave / WP;
    const int M = a.M, N = a.N;
    const int tp = (M + BP - 1) / BP, tq = (N + BQ - 1) / BQ;
    int tile_p, tile_q;
    xcd_tile(blockIdx.x, tp, tq, 4, tile_p, tile_q);
    const int p0 = tile_p * BP, q0 = tile_q * BQ;
    const int z = blockIdx.y;
    const int kbeg = z * a.kchunk;
    const int kend = min(a.kbytes, kbeg + a.kchunk);
    const int nk = (kend - kbeg + KSTAGE - 1) / KSTAGE;
    const size_t ldk = (size_t)a.kbytes;

    // Source of each of this thread's LPT loads: LDS chunk index
    // L = (i * WAVES + wave) * 64 + lane holds logical chunk
    // (L % NC) ^ swz(r) of stage row L / NC, r its row within the A or B part.
    const uint8_t* src[LPT];
    int coff[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int L = (i * WAVES + wave) * 64 + lane;
        const int row = L / NC;
        // the fragment reads swizzle with the row index inside the A part or
        // the B part of the stage, so the copy must do the same
        const int c = (L % NC) ^ swz<NC>(row < BP ? row : row - BP);
        coff[i] = c * 16;
        const uint8_t* base;
        if (row < BP)
            base = (const uint8_t*)a.A + (size_t)min(p0 + row, M - 1) * ldk;
        else
            base = (const uint8_t*)a.B + (size_t)min(q0 + row - BP, N - 1) * ldk;
        src[i] = base + kbeg + c * 16;
    }

    auto issue = [&](int kt, uint8_t* buf) __attribute__((always_inline)) {
        const int kb0 = kt * KSTAGE;  // relative to kbeg
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const bool live = kbeg + kb0 + coff[i] < kend;
            const void* g = live ? (const void*)(src[i] + kb0) : (const void*)g_zero16;
            dma16(g, __builtin_amdgcn_readfirstlane(
                         (uint32_t)(uintptr_t)(buf + (i * WAVES + wave) * 1024)));
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

    auto compute = [&](const uint8_t* sp, int kt) __attribute__((always_inline)) {
        if constexpr (FOLD)
            fold.before(kt * NSTEP, acc);  // chunk boundaries fall on stage starts
        const uint8_t* sq = sp + BP * KSTAGE;
#pragma unroll
        for (int ks = 0; ks < NSTEP; ++ks) {
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
#pragma unroll
            for (int i = 0; i < RP; ++i)
#pragma unroll
                for (int j = 0; j < RQ; ++j)
                    acc[i][j] = mfma_step<OP>(fa[i], fb[j], acc[i][j]);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    // prologue: stages 0 .. STAGES-2 in flight
    if (0 < nk)
        issue(0, slot(I0{}));
    if constexpr (STAGES >= 3)
        if (1 < nk)
            issue(1, slot(I1{}));
    if constexpr (STAGES >= 4)
        if (2 < nk)
            issue(2, slot(I2{}));

    // one K stage in ring slot J
    auto stage = [&](auto J, int kt) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        // stage kt must have landed; younger stages may stay in flight
        const int younger = min(STAGES - 2, nk - 1 - kt);
        if constexpr (STAGES >= 4) {
            if (younger >= 2)
                wait_vm_barrier<2 * LPT>();
            else if (younger == 1)
                wait_vm_barrier<LPT>();
            else
                wait_vm_barrier<0>();
        } else if constexpr (STAGES == 3) {
            if (younger >= 1)
                wait_vm_barrier<LPT>();
            else
                wait_vm_barrier<0>();
        } else {
            wait_vm_barrier<0>();
        }
        // the slot consumed one stage ago is free again for all waves
        if (kt + STAGES - 1 < nk)
            issue(kt + STAGES - 1, slot(std::integral_constant<int, (j + STAGES - 1) % STAGES>{}));
        compute(slot(J), kt);
    };

    for (int kt = 0; kt < nk; kt += STAGES) {
        stage(I0{}, kt);
        if (kt + 1 < nk)
            stage(I1{}, kt + 1);
        if constexpr (STAGES >= 3)
            if (kt + 2 < nk)
                stage(I2{}, kt + 2);
        if constexpr (STAGES >= 4)
            if (kt + 3 < nk)
                stage(I3{}, kt + 3);
    }

    if constexpr (FOLD)
        fold.finish(acc);

    // Epilogue through LDS: each wave writes one 16-row block of its tile at a
    // time into a private LDS scratch, then every lane emits 8 consecutive
    // columns of one row -- a 16-byte bf16 store (two for fp32) instead of
    // eight scattered 2-byte stores.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // ring slots are free
    static_assert(WAVES * 16 * SQ * 4 <= STAGE_BYTES, "epilogue scratch must fit one slot");
    elem_t* scr = (elem_t*)(lds0 + wave * 16 * SQ * 4);
    constexpr int CPR = SQ / 8;          // 8-column groups per row
    constexpr int RPP = 64 / CPR;        // rows per pass
    const bool vec_ok = (N & 7) == 0;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
#pragma unroll
        for (int j = 0; j < RQ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                scr[((lane >> 4) * 4 + v) * SQ + j * 16 + (lane & 15)] = acc[i][j][v];
#pragma unroll
        for (int pass = 0; pass < 16 / RPP; ++pass) {
            const int r = pass * RPP + lane / CPR;
            const int c = (lane % CPR) * 8;
            const int m = p0 + wpi * SP + i * 16 + r;
            const int n = q0 + wqi * SQ + c;
            elem_t e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                e[t] = scr[r * SQ + c + t];
            if (m < M) {
                if (a.splits > 1) {
                    elem_t* dst = (elem_t*)a.ws + ((size_t)z * M + m) * N + n;
                    if (vec_ok && n + 7 < N) {
                        ((uint4*)dst)[0] = make_uint4(__builtin_bit_cast(uint32_t, e[0]), __builtin_bit_cast(uint32_t, e[1]),
                                                      __builtin_bit_cast(uint32_t, e[2]), __builtin_bit_cast(uint32_t, e[3]));
                        ((uint4*)dst)[1] = make_uint4(__builtin_bit_cast(uint32_t, e[4]), __builtin_bit_cast(uint32_t, e[5]),
                                                      __builtin_bit_cast(uint32_t, e[6]), __builtin_bit_cast(uint32_t, e[7]));
                    } else {
                        for (int t = 0; t < 8; ++t)
                            if (n + t < N)
                                dst[t] = e[t];
                    }
                } else if (vec_ok && n + 7 < N && a.out_dtype == OUT_BF16) {
                    uint32_t w[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        w[t] = (uint32_t)bf16_rne(epilogue_value<OP>(e[2 * t], a, m, n + 2 * t)) |
                               ((uint32_t)bf16_rne(epilogue_value<OP>(e[2 * t + 1], a, m, n + 2 * t + 1)) << 16);
                    *(uint4*)((uint16_t*)a.out + (size_t)m * N + n) = make_uint4(w[0], w[1], w[2], w[3]);
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            store_one<OP>(a, (size_t)m * N + n + t, e[t], m, n + t);
                }
            }
        }
    }
}

template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int STAGES>
hipError_t launch_pipe(const GemmArgs& a, hipStream_t stream)
{
    const long tiles = (long)((a.M + BP - 1) / BP) * ((a.N + BQ - 1) / BQ);
    if (tiles > 0x7FFFFFFFL)
        return hipErrorInvalidValue;
    if (a.splits > 1)
        hipLaunchKernelGGL((gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KSTAGE, STAGES, true>),
                           dim3((unsigned)tiles, (unsigned)a.splits), dim3(WP * WQ * 64), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KSTAGE, STAGES, false>),
                           dim3((unsigned)tiles, 1), dim3(WP * WQ * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qll

// X(OP, BP, BQ, WP, WQ, KSTAGE, STAGES) for every pipelined variant.
#define QLL_FOR_EACH_PIPE(X, OP)           \
    X(OP, 128, 128, 2, 2, 128, 4)          \
    X(OP, 128, 128, 2, 2, 128, 3)          \
    X(OP, 256, 128, 2, 2, 128, 3)          \
    X(OP, 128, 256, 2, 2, 128, 3)          \
    X(OP, 256, 128, 4, 2, 128, 3)          \
    X(OP, 128, 64, 2, 2, 128, 4)           \
    X(OP, 64, 128, 2, 2, 128, 4)           \
    X(OP, 32, 128, 1, 4, 128, 4)           \
    X(OP, 64, 64, 2, 2, 128, 4)            \
    X(OP, 128, 32, 4, 1, 128, 4)

#define QLL_PIPE_INSTANTIATE(OP, BP, BQ, WP, WQ, KS, ST)                                       \
    template __global__ void qll::gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KS, ST, false>(qll::GemmArgs); \
    template __global__ void qll::gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KS, ST, true>(qll::GemmArgs);
#define QLL_PIPE_ENTRY(OP, BP, BQ, WP, WQ, KS, ST)                                   \
    {"p" #BP "x" #BQ "_w" #WP "x" #WQ "_k" #KS "_s" #ST, OP, 0, BP, BQ, WP, WQ, KS,    \
     (ST) * ((BP) + (BQ)) * (KS), &qll::launch_pipe<OP, BP, BQ, WP, WQ, KS, ST>},
