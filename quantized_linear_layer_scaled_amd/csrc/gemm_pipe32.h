// Deep-ring pipelined FP8 GEMM for gfx950 on the 32x32x64 matrix-core step:
// the large-M, compute-bound member of the "ordinary GEMM" strategy of
// "Helion in vLLM: A Unified Route to Tunable Linear Kernels" ("What the
// integration changes": tile shapes and pipeline depth as tunables).
//
// The 16x16x128 step of gemm_pipe.h needs 128 bytes of K per stage, so a
// 256x256 tile stages 64 KB at a time and 160 KB of LDS holds two stages:
// one in flight while the other is computed, and the CU's global->LDS stream
// stalls at every stage boundary.  v_mfma_f32_32x32x64_f8f6f4 consumes 64
// bytes of K per step, so here a stage is 64 bytes of K of every tile row
// (32 KB for 256x256), the ring holds STAGES of them, and STAGES - 1 stages
// are always on their way while one is computed:
//   * stage j + STAGES is issued into the slot of stage j as soon as every
//     wave holds stage j's fragments in registers (one barrier per stage);
//   * the fragments of stage j + 1 are read from LDS into the second of two
//     register sets while the MFMAs of stage j run on the first;
//   * a wave waits only for its own copies of the stage it reads next
//     (s_waitcnt vmcnt with the younger stages' copies still allowed);
//   * the tile rows' 64-byte stage runs are XOR-swizzled in 16-byte chunks
//     (swz4 below) so that the 8 or 16 lanes an LDS read serves together hit
//     distinct banks; the swizzle is applied on the global side of the copy,
//     whose LDS destination per lane the hardware fixes;
//   * a 256x256 tile runs 4 waves of 128x128 (16 accumulators of 32x32 in
//     the accumulation registers, one wave per SIMD), which also reads a
//     third fewer LDS bytes per flop than 8 waves of 128x64.
// Operands are addressed through buffer resources as in gemm_pipe.h (rows
// past M or N and K past the range read zeros, no masking in the loop).
//
// Lane layout of the 32x32x64 e4m3 step (checked on the device): lane l
// supplies row l % 32 and K bytes 32 (l / 32) .. + 31 of each operand;
// accumulator r of lane l is output row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.
#pragma once

#include "gemm_pipe.h"

namespace qll {

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32_fp8(const v8i& a, const v8i& b, v16f c)
{
    // format code 0 (e4m3) for both operands, no block scaling
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Physical 16-byte chunk of logical chunk c of a 64-byte staged row:
// c ^ swz4(row).  Over any 8 (or 16) consecutive rows the pairs
// (row mod 2, chunk) (or (row mod 4, chunk)) that one chunk column maps to
// are distinct, so a fragment read is free of bank conflicts whether the LDS
// serves 8 or 16 lanes of a 16-byte read per cycle.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

constexpr int kP32Stage = 64;  // bytes of K per stage (one MFMA step)

template <int BP, int BQ, int STAGES>
constexpr int p32_ring_bytes()
{
    return STAGES * (BP + BQ) * kP32Stage;
}

template <int BP, int BQ, int STAGES>
constexpr int p32_lds_bytes()
{
    return p32_ring_bytes<BP, BQ, STAGES>() + pipe_prescale_bytes<BP, BQ>();
}

template <int BP, int BQ, int WP, int WQ, int STAGES>
constexpr int p32_waves_per_eu()
{
    constexpr int wgs = pipe_wgs_per_cu(p32_lds_bytes<BP, BQ, STAGES>());
    constexpr int w = wgs * WP * WQ / 4;
    return w < 1 ? 1 : (w > 8 ? 8 : w);
}

template <int OP, int BP, int BQ, int WP, int WQ, int STAGES, bool SPLITK>
__global__ __launch_bounds__(WP* WQ * 64)
__attribute__((amdgpu_waves_per_eu(p32_waves_per_eu<BP, BQ, WP, WQ, STAGES>())))
void gemm_p32_kernel(GemmArgs a)
{
    static_assert(OP == OP_FP8, "the 32x32x64 step here is e4m3 x e4m3");
    constexpr int WAVES = WP * WQ;
    constexpr int THREADS = WAVES * 64;
    constexpr int SP = BP / WP, SQ = BQ / WQ;
    constexpr int RP = SP / 32, RQ = SQ / 32;
    constexpr int ROWS = BP + BQ;
    constexpr int SLOT = ROWS * kP32Stage;
    constexpr int LPT = ROWS * 4 / THREADS;  // 16-byte copies per thread per stage
    static_assert(SP % 32 == 0 && SQ % 32 == 0, "waves own whole 32x32 blocks");
    static_assert(BP % 16 == 0 && (ROWS * 4) % THREADS == 0,
                  "a copy instruction fills 16 rows of one operand");
    static_assert(STAGES >= 3 && (STAGES - 1) * LPT < 64, "bad ring depth");
    static_assert(SLOT % 1024 == 0, "slots start on 1 KiB boundaries");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[STAGES * SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wpi = wave % WP, wqi = wave / WP;
    const int M = a.M, N = a.N;
    int tile_p, tile_q;
    xcd_tile(blockIdx.x, (M + BP - 1) / BP, (N + BQ - 1) / BQ, 4, tile_p, tile_q);
    const int p0 = tile_p * BP, q0 = tile_q * BQ;
    const int z = blockIdx.y;
    const int kbeg = z * a.kchunk;
    const int kend = min(a.kbytes, kbeg + a.kchunk);
    const int nk = (kend - kbeg + kP32Stage - 1) / kP32Stage;
    const uint32_t ldk = (uint32_t)a.kbytes;

    const v4i rsA = buffer_rsrc((const uint8_t*)a.A + (size_t)p0 * ldk,
                                (uint32_t)min((uint64_t)(M - p0) * ldk, (uint64_t)0x7FFFFFFF));
    const v4i rsB = buffer_rsrc((const uint8_t*)a.B + (size_t)q0 * ldk,
                                (uint32_t)min((uint64_t)(N - q0) * ldk, (uint64_t)0x7FFFFFFF));

    // Copy i of this thread fills 16-byte LDS chunk 64 (i WAVES + wave) +
    // lane of the slot: stage row 16 (i WAVES + wave) + lane / 4, physical
    // chunk lane % 4, which holds logical chunk (lane % 4) ^ swz4(r) of that
    // row (r: the row within its operand, as the fragment reads index it).
    // The row of a copy lies at 16 (i WAVES + wave) + lane / 4 of the stage;
    // within its operand r = rb + lane / 4 with rb a multiple of 16 (the
    // operand's 16-row block, wave-uniform).  swz4(r) depends on bits 1-4 of
    // r, i.e. on lane / 4 and on bit 4 of rb: two chunk offsets per lane
    // cover every copy, and the rest of the offset is wave-uniform.
    const uint32_t lrow = (uint32_t)(lane >> 2) * ldk;
    const uint32_t ch0 = (uint32_t)((lane & 3) ^ swz4(lane >> 2)) * 16u;
    const uint32_t ch1 = (uint32_t)((lane & 3) ^ swz4((lane >> 2) + 16)) * 16u;
    const int krem = kend - kbeg;
    // Stage kt into ring slot sidx.  Stages at or past the end of the K
    // range are issued too, as copies of zeros (every offset out of range),
    // so that every stage of the loop has the same number of copies in
    // flight behind it and the waits need no branches.
    auto issue = [&](int kt, int sidx) __attribute__((always_inline)) {
        const int kb0 = kt * kP32Stage;
        const bool full = kb0 + kP32Stage <= krem;
        const uint32_t base = (uint32_t)(uintptr_t)ring + (uint32_t)(sidx * SLOT);
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int blk = i * WAVES + wave;           // wave-uniform
            const bool ina = 16 * blk < BP;
            const int rb = ina ? 16 * blk : 16 * blk - BP;
            const uint32_t ch = (rb & 16) ? ch1 : ch0;
            uint32_t vo = lrow + ch + (uint32_t)rb * ldk + (uint32_t)(kbeg + kb0);
            if (!full && kb0 + (int)ch >= krem)
                vo = kOutOfRange;  // past the K range: zeros
            dma16(vo, ina ? rsA : rsB,
                  __builtin_amdgcn_readfirstlane(base + (uint32_t)(blk * 1024)));
        }
    };

    // The tile's scales into LDS ahead of the first stage (the stage waits,
    // which count only younger copies, cover them): unit u holds sa of tile
    // rows 64u .. 64u + 63 (u < UA), then sb of the tile columns.
    constexpr int UA = (BP + 63) / 64, UB = (BQ + 63) / 64;
    __shared__ __attribute__((aligned(16))) float lpre[(UA + UB) * 64];
    const bool scaled = a.splits == 1;
    if (scaled) {
        const v4i rsPa = buffer_rsrc(a.sa + p0,
                                     (uint32_t)min((uint64_t)(M - p0) * 4, (uint64_t)0x7FFFFFFF));
        const v4i rsPb = buffer_rsrc(a.sb + q0,
                                     (uint32_t)min((uint64_t)(N - q0) * 4, (uint64_t)0x7FFFFFFF));
        for (int u = wave; u < UA + UB; u += WAVES) {
            const bool ua = u < UA;
            dma4((uint32_t)((ua ? u : u - UA) * 64 + lane) * 4u, ua ? rsPa : rsPb,
                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lpre + u * 64)));
        }
    }

    v16f acc[RP][RQ];
#pragma unroll
    for (int i = 0; i < RP; ++i)
#pragma unroll
        for (int j = 0; j < RQ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    // fragments: lane l reads row l % 32 of each 32-row block, logical
    // chunks 2 (l / 32) and 2 (l / 32) + 1.  Blocks start at multiples of 32
    // rows, so swz4 of the row is swz4(l % 32) for every block: one pair of
    // chunk offsets per lane, the block and slot in the immediate offset.
    v8i fa[2][RP], fb[2][RQ];
    const int h2 = (lane >> 5) * 2;
    const int sl = swz4(lane & 31);
    const uint32_t fa_base = (uint32_t)((wpi * SP + (lane & 31)) * kP32Stage);
    const uint32_t fb_base = (uint32_t)((BP + wqi * SQ + (lane & 31)) * kP32Stage);
    const uint32_t co_lo = (uint32_t)((h2 ^ sl) << 4), co_hi = (uint32_t)(((h2 + 1) ^ sl) << 4);
    auto load_frags = [&](const uint8_t* sp, v8i* da, v8i* db) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const uint8_t* rp = sp + fa_base + i * 32 * kP32Stage;
            da[i].lo = *(const v4i*)(rp + co_lo);
            da[i].hi = *(const v4i*)(rp + co_hi);
        }
#pragma unroll
        for (int j = 0; j < RQ; ++j) {
            const uint8_t* rp = sp + fb_base + j * 32 * kP32Stage;
            db[j].lo = *(const v4i*)(rp + co_lo);
            db[j].hi = *(const v4i*)(rp + co_hi);
        }
    };
    auto compute = [&](const v8i* ca, const v8i* cb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int j = 0; j < RQ; ++j)
                acc[i][j] = mfma32_fp8(ca[i], cb[j], acc[i][j]);
    };

    // prologue: every slot receives a stage; stage 0's fragments go to set 0
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
        issue(st, st);
    wait_vm_barrier<(STAGES - 1) * LPT>();
    load_frags(ring, fa[0], fb[0]);

    // Stage kt, computed from register set P: once stage kt + 1 has landed
    // for every wave, the slot of stage kt (whose fragments every wave
    // holds) takes stage kt + STAGES, stage kt + 1's fragments are read into
    // the other set (past the last stage they are read and never used) and
    // stage kt's MFMAs run.  The loop is unrolled by two so that the register
    // sets are fixed, and runs an even number of stages (a last stage past
    // the K range holds zeros and adds nothing): a loop without an exit
    // between its two halves keeps every accumulator in place in the
    // accumulation registers.  The ring slot is a run-time index.
    int cs = 0;  // slot of stage kt
    auto step = [&](auto P, int kt) __attribute__((always_inline)) {
        constexpr int cp = decltype(P)::value;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): set cp is loaded
        wait_vm_barrier<(STAGES - 2) * LPT>();
        issue(kt + STAGES, cs);
        cs = cs + 1 == STAGES ? 0 : cs + 1;
        load_frags(ring + cs * SLOT, fa[cp ^ 1], fb[cp ^ 1]);
        compute(fa[cp], fb[cp]);
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(std::integral_constant<int, 0>{}, kt);
        step(std::integral_constant<int, 1>{}, kt + 1);
    }

    // Epilogue through LDS: each wave writes one 32-row block of its tile at
    // a time into a private scratch in the ring, then every lane emits 8
    // consecutive columns of one row (16-byte stores).  Its addresses derive
    // from an opaque zero made here, so that the compiler does not compute
    // them before the K loop and hold them (in registers the loop needs)
    // through it.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    int z0;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z0));
    static_assert(WAVES * 32 * SQ * 4 <= STAGES * SLOT, "epilogue scratch must fit the ring");
    float* scr = (float*)(ring + wave * 32 * SQ * 4);
    constexpr int CPR = SQ / 8;     // 8-column groups per row
    constexpr int RPP = 64 / CPR;   // rows per pass
    constexpr int PASSES = 32 / RPP;
    static_assert(64 % CPR == 0 && 32 % RPP == 0, "epilogue lane map");
    const bool vec_ok = (N & 7) == 0;
    const int c = (lane % CPR) * 8;
    const int n = q0 + z0 + wqi * SQ + c;
    const int pe = p0 + z0;
    float sbv[8];
    if (scaled) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            sbv[t] = lpre[UA * 64 + wqi * SQ + c + t];
    }
#pragma unroll
    for (int i = 0; i < RP; ++i) {
#pragma unroll
        for (int j = 0; j < RQ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                scr[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * SQ + j * 32 + (lane & 31)] =
                    acc[i][j][r];
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            const int rr = pass * RPP + lane / CPR;
            const int tr = wpi * SP + i * 32 + rr;  // row within the tile
            const int m = pe + tr;
            float e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                e[t] = scr[rr * SQ + c + t];
            if (m >= M)
                continue;
            if (!scaled) {
                // Split-K partials, added in order by the second stage
                float* dst = (float*)a.ws + ((size_t)z * M + m) * N + n;
                if (vec_ok && n + 7 < N) {
                    ((v4f*)dst)[0] = v4f{e[0], e[1], e[2], e[3]};
                    ((v4f*)dst)[1] = v4f{e[4], e[5], e[6], e[7]};
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = e[t];
                }
                continue;
            }
            const float sam = lpre[tr];
            float y[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float u = e[t] * sam;
                y[t] = u * sbv[t];
            }
            if (a.out_dtype == OUT_BF16) {
                uint16_t* dst = (uint16_t*)a.out + (size_t)m * N + n;
                if (vec_ok && n + 7 < N) {
                    uint32_t w[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        w[t] = (uint32_t)bf16_rne(y[2 * t]) |
                               ((uint32_t)bf16_rne(y[2 * t + 1]) << 16);
                    store16_stream(dst, w[0], w[1], w[2], w[3]);
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = bf16_rne(y[t]);
                }
            } else {
                float* dst = (float*)a.out + (size_t)m * N + n;
                if (vec_ok && n + 7 < N) {
                    store16_stream(dst, __float_as_uint(y[0]), __float_as_uint(y[1]),
                                   __float_as_uint(y[2]), __float_as_uint(y[3]));
                    store16_stream(dst + 4, __float_as_uint(y[4]), __float_as_uint(y[5]),
                                   __float_as_uint(y[6]), __float_as_uint(y[7]));
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = y[t];
                }
            }
        }
    }
}

template <int OP, int BP, int BQ, int WP, int WQ, int STAGES>
hipError_t launch_p32(const GemmArgs& a, hipStream_t stream)
{
    const long tiles = (long)((a.M + BP - 1) / BP) * ((a.N + BQ - 1) / BQ);
    if (tiles > 0x7FFFFFFFL || (long)(BP > BQ ? BP : BQ) * a.kbytes > 0x7FFFFFFFL ||
        a.out_dtype == OUT_INT32)
        return hipErrorInvalidValue;  // 32-bit buffer offsets within a tile
    if (a.splits > 1)
        hipLaunchKernelGGL((gemm_p32_kernel<OP, BP, BQ, WP, WQ, STAGES, true>),
                           dim3((unsigned)tiles, (unsigned)a.splits), dim3(WP * WQ * 64), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((gemm_p32_kernel<OP, BP, BQ, WP, WQ, STAGES, false>),
                           dim3((unsigned)tiles, 1), dim3(WP * WQ * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qll

// X(OP, BP, BQ, WP, WQ, STAGES) for every deep-ring variant.
#define QLL_FOR_EACH_P32(X, OP)  \
    X(OP, 256, 256, 2, 2, 4)     \
    X(OP, 256, 128, 2, 2, 6)     \
    X(OP, 128, 256, 2, 2, 6)     \
    X(OP, 128, 128, 2, 2, 8)     \
    X(OP, 128, 128, 2, 2, 4)     \
    X(OP, 128, 64, 2, 2, 6)      \
    X(OP, 64, 128, 2, 2, 6)

#define QLL_P32_INSTANTIATE(OP, BP, BQ, WP, WQ, ST)                                      \
    template __global__ void qll::gemm_p32_kernel<OP, BP, BQ, WP, WQ, ST, false>(qll::GemmArgs); \
    template __global__ void qll::gemm_p32_kernel<OP, BP, BQ, WP, WQ, ST, true>(qll::GemmArgs);
#define QLL_P32_ENTRY(OP, BP, BQ, WP, WQ, ST)                                      \
    {"p" #BP "x" #BQ "_w" #WP "x" #WQ "_k64_s" #ST, OP, 0, BP, BQ, WP, WQ, 64,       \
     qll::p32_lds_bytes<BP, BQ, ST>(), &qll::launch_p32<OP, BP, BQ, WP, WQ, ST>},
