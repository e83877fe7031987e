// Pipelined large-M scaled GEMM for gfx950 (ordinary orientation: tokens on
// the MFMA row side), the compute-bound member of the "ordinary GEMM"
// strategy of "Helion in vLLM: A Unified Route to Tunable Linear Kernels"
// ("What the integration changes").
//
// The plain tiled kernel prefetches one stage into registers, so every K step
// waits for a full global-memory round trip.  Here:
//   * operands go from global memory straight into LDS with
//     buffer_load_dwordx4 ... lds (no VGPR staging, no ds_write) into a ring
//     of STAGES LDS buffers, every buffer holding a stage in flight;
//   * the MFMA fragments of a stage are read from LDS into one of two
//     register sets while the MFMAs of the previous stage run on the other,
//     so a ring slot is free as soon as its fragments are in registers (the
//     K loop is unrolled by lcm(STAGES, 2) so that every slot is a
//     compile-time LDS object and every register set a fixed set);
//   * a wave waits only for its own oldest stage (s_waitcnt vmcnt(N) with N
//     the loads of the younger stages still allowed in flight) and for its
//     LDS reads, and then meets the other waves at one s_barrier per stage --
//     the barrier also frees the buffer that the next prefetch overwrites;
//   * each lane's 64 destination bytes are fixed by the hardware (lane i of a
//     wave writes bytes 16i..16i+15 of the wave's 1 KiB block), so the XOR
//     swizzle of 16-byte chunks is applied on the global side: the lane that
//     fills LDS chunk (row, j) fetches logical chunk j ^ swz(row);
//   * the A and B tiles are addressed through buffer resources whose range
//     ends at the last row of the matrix, with one 32-bit offset per load:
//     rows past M or N fall outside the range, and a load past the end of
//     the K range gets an offset outside it, so the hardware fills both with
//     zeros and the MFMA loop needs no masking (outputs of rows past M or N
//     are discarded at the store).  This needs BP * K bytes < 2^31, which the
//     host checks.
// Output element accumulation is the same ascending sequence of MFMA K steps
// as in the other kernels, so results are bitwise equal to theirs for the
// same K split.
#pragma once

#include <type_traits>

#include "gemm_tile.h"

namespace qll {

// Raw buffer resource (GFX9 layout): 48-bit base, stride 0, num_records
// bytes, 32-bit data format; loads at offsets past num_records return zeros.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    v4i r;
    r.x = (int)(uint32_t)b;
    r.y = (int)(uint32_t)(b >> 32) & 0xFFFF;
    r.z = (int)bytes;
    r.w = 0x00020000;
    return r;
}

// 16-byte store of a final output: non-temporal, so that the line goes out
// to memory instead of waiting, dirty in L2, for the write-back at the end of
// the kernel (all tiles finish together; measured 2-3 us less per call on a
// 16 MB output).  Split-K partials, read back at once, use plain stores.
__device__ __forceinline__ void store16_stream(void* p, uint32_t x, uint32_t y, uint32_t z,
                                               uint32_t w)
{
    __builtin_nontemporal_store(v4i{(int)x, (int)y, (int)z, (int)w}, (v4i*)p);
}

// bf16 output of one wave's RP x RQ accumulator blocks of 16 x 16 (lane
// element (i, j, v): row 16 i + 4 (lane >> 4) + v, column 16 j + (lane & 15)
// of the wave's block, whose first output row is m0 and first column n0).
// With SCALED, an element is (acc * sa) * sb, sa = lsa[16 i + 4 (lane >> 4)
// + v] and sb = lsb[16 j + (lane & 15)] (LDS copies of the block's row and
// column scales), else the accumulator itself.  Each value is rounded where
// the MFMA left it, to nearest even; the two lanes of a pair (neighbouring
// columns) trade values with one DPP swap, so that each lane holds two
// bf16x2 words of adjacent columns (rows 0-1 of its 4 in the even lane, 2-3
// in the odd one).  The words of BB row blocks at a time go through the
// wave's LDS scratch `scr` (16 BB rows of SQ / 2 + 4 words) -- all of their
// writes, then all of their reads, then all of their 16-byte stores of 8
// columns per lane -- so that the LDS round trips overlap instead of running
// one row block after another, with half the bytes of staging fp32 values.
// With rows of SQ / 2 + 4 words, the even and odd lanes' rows (2 apart) fall
// 8 banks apart and the lane groups (4 rows apart) 16 apart: no write
// conflicts.  N must be a multiple of 8; rows past M and columns past N are
// not stored.
template <int RP, int RQ, int BB, bool SCALED, typename Acc>
__device__ __forceinline__ void store_bf16_batched(const Acc (&acc)[RP][RQ], uint32_t* scr,
                                                   const float* lsa, const float* lsb,
                                                   int lane, int m0, int n0, int M, int N,
                                                   uint16_t* out)
{
    constexpr int SQ = RQ * 16;
    constexpr int SQB = SQ / 2 + 4;
    constexpr int CPR = SQ / 8, RPP = 64 / CPR, PASSES = 16 / RPP;
    static_assert(RP % BB == 0 && SQ % 8 == 0 && 64 % CPR == 0 && 16 % RPP == 0,
                  "epilogue lane map");
    const bool odd = lane & 1;
    float sbc[RQ];
    if constexpr (SCALED) {
#pragma unroll
        for (int j = 0; j < RQ; ++j)
            sbc[j] = lsb[j * 16 + (lane & 15)];
    }
    const int c = (lane % CPR) * 8;  // this lane's 8 output columns
    const int n = n0 + c;
#pragma unroll
    for (int i0 = 0; i0 < RP; i0 += BB) {
#pragma unroll
        for (int b = 0; b < BB; ++b) {
            const int i = i0 + b;
            float sar[4];
            if constexpr (SCALED) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    sar[v] = lsa[i * 16 + (lane >> 4) * 4 + v];
            }
            const int r0 = b * 16 + (lane >> 4) * 4 + (odd ? 2 : 0);
#pragma unroll
            for (int j = 0; j < RQ; ++j) {
                float y[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    if constexpr (SCALED) {
                        const float u = (float)acc[i][j][v] * sar[v];
                        y[v] = u * sbc[j];
                    } else {
                        y[v] = (float)acc[i][j][v];
                    }
                }
                const float t0 = lane_pair_swap(odd ? y[0] : y[2]);
                const float t1 = lane_pair_swap(odd ? y[1] : y[3]);
                const int c2 = (j * 16 + (lane & 15)) >> 1;
                scr[r0 * SQB + c2] = odd ? bf16x2_rne(t0, y[2]) : bf16x2_rne(y[0], t0);
                scr[(r0 + 1) * SQB + c2] = odd ? bf16x2_rne(t1, y[3]) : bf16x2_rne(y[1], t1);
            }
        }
        uint4 w[BB][PASSES];
#pragma unroll
        for (int b = 0; b < BB; ++b)
#pragma unroll
            for (int pass = 0; pass < PASSES; ++pass)
                w[b][pass] = *(const uint4*)&scr[(b * 16 + pass * RPP + lane / CPR) * SQB + c / 2];
#pragma unroll
        for (int b = 0; b < BB; ++b)
#pragma unroll
            for (int pass = 0; pass < PASSES; ++pass) {
                const int m = m0 + (i0 + b) * 16 + pass * RPP + lane / CPR;
                if (m < M && n < N)
                    store16_stream(out + (size_t)m * N + n, w[b][pass].x, w[b][pass].y,
                                   w[b][pass].z, w[b][pass].w);
            }
    }
}

// The most row blocks of 16 that store_bf16_batched can batch in a wave's
// share of `bytes` of scratch (RP itself, else 4 or 2 if they divide it).
template <int RP, int SQ>
constexpr int bf16_batch_blocks(int bytes)
{
    constexpr int rbb = 16 * (SQ / 2 + 4) * 4;
    return bytes / rbb >= RP ? RP
           : (bytes / rbb >= 4 && RP % 4 == 0 ? 4 : (bytes / rbb >= 2 && RP % 2 == 0 ? 2 : 1));
}

// Offset that lies outside every resource built here (num_records < 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;

// One 16-byte buffer -> LDS copy per lane (buffer_load_dwordx4 ... lds): lane
// i of the wave writes LDS bytes lds_base + 16 i .. + 15.  Issued from inline
// asm so that the compiler, which cannot tell the ring slots apart, does not
// add a wait for every copy in flight before each LDS read; the only
// synchronization is the explicit vmcnt wait + barrier below.  The asm has no
// register outputs; M0 is set inside the same block.
__device__ __forceinline__ void dma16(uint32_t voff, v4i rsrc, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 ::"v"(voff), "s"(rsrc), "s"(lds_base)
                 : "memory", "m0");
}

// One 4-byte buffer -> LDS copy per lane: lane i writes LDS bytes
// lds_base + 4 i .. + 3.
__device__ __forceinline__ void dma4(uint32_t voff, v4i rsrc, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 ::"v"(voff), "s"(rsrc), "s"(lds_base)
                 : "memory", "m0");
}

// Wait until at most N of this wave's global->LDS copies are in flight and
// all of its LDS reads have returned, then meet the other waves.  The wait is
// the s_waitcnt builtin (vmcnt(N) lgkmcnt(0), GFX9 encoding) so that the
// compiler knows the LDS reads issued before it are complete and does not
// make later MFMAs wait for reads issued after it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    asm volatile("s_barrier" ::: "memory");
}

// f(integral_constant<J>{}, kt + J) for J = J0 .. U-1 while kt + J < nk: the
// stages of one unrolled round of the K loop, each with its ring slot and
// register set known at compile time.
template <int J, int U, typename F>
__device__ __forceinline__ void for_stages(F&& f, int kt, int nk)
{
    if constexpr (J < U) {
        if (kt + J < nk) {
            f(std::integral_constant<int, J>{}, kt + J);
            for_stages<J + 1, U>(f, kt, nk);
        }
    }
}

// f(integral_constant<J>{}) for J = J0 .. U-1, unconditionally.
template <int J, int U, typename F>
__device__ __forceinline__ void unroll(F&& f)
{
    if constexpr (J < U) {
        f(std::integral_constant<int, J>{});
        unroll<J + 1, U>(f);
    }
}

// wait_vm_barrier<Y * LPT>() for the largest Y <= min(younger, YMAX).
template <int YMAX, int LPT>
__device__ __forceinline__ void wait_younger(int younger)
{
    if constexpr (YMAX <= 0) {
        wait_vm_barrier<0>();
    } else {
        if (younger >= YMAX)
            wait_vm_barrier<YMAX * LPT>();
        else
            wait_younger<YMAX - 1, LPT>(younger);
    }
}

// Waves per SIMD the register allocation has to allow: as many workgroups
// as the LDS ring lets share a CU (160 KiB of LDS, at most four), each with
// WP x WQ waves over the CU's four SIMDs.  Several resident workgroups are
// what keeps the global->LDS copies of one overlapping the barrier waits and
// MFMAs of another.
// MXFP4 stages carry the tile rows' E8M0 block scales (KSTAGE / 16 bytes per
// row) behind the codes, in whole 256-byte copy units.
template <int OP, int BP, int BQ, int KSTAGE>
constexpr int pipe_scale_bytes()
{
    return OP == OP_MXFP4 ? ((BP + BQ) * (KSTAGE / 16) + 255) / 256 * 256 : 0;
}

// LDS of the operand ring (and the Block-FP8 scale ring).
// One ring slot: a stage's operand rows (and MXFP4 scale bytes), in whole
// KiB so that every slot starts 1 KiB-aligned.
template <int OP, int BP, int BQ, int KSTAGE>
constexpr int pipe_slot_bytes()
{
    return ((BP + BQ) * KSTAGE + pipe_scale_bytes<OP, BP, BQ, KSTAGE>() + 1023) / 1024 * 1024;
}

// KGRP K groups per workgroup (see gemm_pipe_kernel) have a ring each.
template <int OP, int BP, int BQ, int KSTAGE, int STAGES, int KGRP = 1>
constexpr int pipe_ring_bytes()
{
    return KGRP * STAGES * pipe_slot_bytes<OP, BP, BQ, KSTAGE>() +
           (OP == OP_BLOCK ? (STAGES + 1) * 1280 : 0);
}

constexpr int pipe_wgs_per_cu(int lds)
{
    return 163840 / lds < 4 ? 163840 / lds : 4;
}

// The per-token x per-channel ops copy the tile's activation and weight
// scales into LDS at the start, so that the epilogue does not wait a memory
// round trip for them after the K loop -- unless the extra bytes (whole
// 64-float units per operand) would lower the number of resident workgroups.
template <int BP, int BQ>
constexpr int pipe_prescale_bytes()
{
    return ((BP + 63) / 64 + (BQ + 63) / 64) * 256;
}

template <int OP, int BP, int BQ, int KSTAGE, int STAGES, int KGRP = 1>
constexpr bool pipe_prescale()
{
    return (OP == OP_INT8 || OP == OP_FP8) &&
           pipe_wgs_per_cu(pipe_ring_bytes<OP, BP, BQ, KSTAGE, STAGES, KGRP>() +
                           pipe_prescale_bytes<BP, BQ>()) ==
               pipe_wgs_per_cu(pipe_ring_bytes<OP, BP, BQ, KSTAGE, STAGES, KGRP>());
}

template <int OP, int BP, int BQ, int KSTAGE, int STAGES, int KGRP = 1>
constexpr int pipe_lds_bytes()
{
    return pipe_ring_bytes<OP, BP, BQ, KSTAGE, STAGES, KGRP>() +
           (pipe_prescale<OP, BP, BQ, KSTAGE, STAGES, KGRP>() ? pipe_prescale_bytes<BP, BQ>()
                                                               : 0);
}

template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int STAGES, int KGRP = 1>
constexpr int pipe_waves_per_eu()
{
    constexpr int wgs = pipe_wgs_per_cu(pipe_lds_bytes<OP, BP, BQ, KSTAGE, STAGES, KGRP>());
    constexpr int w = wgs * KGRP * WP * WQ / 4;
    return w < 1 ? 1 : (w > 8 ? 8 : w);
}

// Grouped GEMM: the number of row tiles of BP rows over all experts, with
// the offsets read as group_tile reads them (every lane gets the total).
__device__ __forceinline__ int group_row_tiles(const int* __restrict__ off, int E, int M, int BP,
                                               int lane)
{
    int total = 0, carry = 0;
    for (int base = 0; base < E; base += 64) {
        const int j = base + lane;
        const bool live = j < E;
        int lo = live ? min(max(off[j], 0), M) : 0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(lo, d, 64);
            if (lane >= d)
                lo = max(lo, v);
        }
        lo = max(lo, carry);
        const int hi = live ? max(lo, min(max(off[j + 1], 0), M)) : lo;
        int tiles = live ? (hi - lo + BP - 1) / BP : 0;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1)
            tiles += __shfl_xor(tiles, d, 64);
        total += tiles;
        carry = __shfl(hi, 63, 64);
    }
    return total;
}

// Grouped GEMM: the expert that owns virtual row tile t (tiles of BP rows,
// numbered expert by expert) and its row range [m0, m1) for that tile.
// Offsets are clamped to [0, M] and made non-decreasing, so no access leaves
// the A rows whatever the offsets hold.  Lane-parallel over 64 experts at a
// time (prefix sum by shuffles); every lane gets the same answer, e = -1 past
// the last tile.
__device__ __forceinline__ void group_tile(const int* __restrict__ off, int E, int M, int t,
                                           int BP, int lane, int& e, int& m0, int& m1)
{
    int before = 0;   // tiles of the experts already scanned
    int carry = 0;    // running maximum of the offsets already scanned
    for (int base = 0; base < E; base += 64) {
        const int j = base + lane;
        const bool live = j < E;
        // c[j] = max(clamp(off[0..j])): expert j owns rows [c[j], c[j+1])
        int lo = live ? min(max(off[j], 0), M) : 0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(lo, d, 64);
            if (lane >= d)
                lo = max(lo, v);
        }
        lo = max(lo, carry);
        const int hi = live ? max(lo, min(max(off[j + 1], 0), M)) : lo;
        const int tiles = live ? (hi - lo + BP - 1) / BP : 0;
        int incl = tiles;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d)
                incl += v;
        }
        const unsigned long long hit = __ballot(live && before + incl > t);
        if (hit) {
            const int L = __ffsll((long long)hit) - 1;
            const int first = before + __shfl(incl - tiles, L, 64);
            e = base + L;
            m0 = __shfl(lo, L, 64) + (t - first) * BP;
            m1 = __shfl(hi, L, 64);
            return;
        }
        before += __shfl(incl, 63, 64);
        carry = __shfl(hi, 63, 64);
    }
    e = -1;
    m0 = m1 = 0;
}

// SPLITK only gives the first stage of a Split-K call its own kernel symbol
// (the code is the same), so that traces separate the two kinds of launch.
// GROUPED: the per-expert GEMM over rows sorted by expert (no Split-K).
// KGRP = 2: two K groups of WP x WQ waves in one workgroup, each running the
// whole pipeline on its half of the workgroup's K range (the first
// ceil(stages / 2) stages, the rest) through a ring of its own; both run
// the same number of stages, so they meet at every barrier, and at the end
// the second group's partial tile is added to the first's through LDS, in
// that order.  Twice the copy streams per tile and half its serial K depth,
// with no second launch: the Split-K of the mid-size M within a workgroup.
// RC > 0 (gemm_pipe_rc_kernel): the operand copies go through registers
// instead of the LDS copy path -- buffer_load_dwordx4 into one of RC register
// sets, RC stages ahead, then ds_write_b128 into a two-slot LDS ring one
// stage ahead of the MFMAs.  The LDS image is the same as the copy path's, so
// the fragment reads and the products are too.
template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int STAGES, bool SPLITK,
          bool GROUPED, int KGRP, int RC>
__device__ __forceinline__ void gemm_pipe_body(const GemmArgs& a)
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
    constexpr bool BLK = OP == OP_BLOCK;
    constexpr bool MX = OP == OP_MXFP4;
    constexpr int LPT0 = ROWS * NC / THREADS;      // operand loads per thread per stage
    // MXFP4: SCB scale bytes per tile row per stage, copied in NSC units of
    // 256 bytes (64 lanes x 4), LPS per wave (units repeat when there are
    // more waves than units: the copies write equal values)
    constexpr int SCB = MX ? KSTAGE / 16 : 0;
    constexpr int SC_REGION = pipe_scale_bytes<OP, BP, BQ, KSTAGE>();
    constexpr int NSC = SC_REGION / 256;
    constexpr int LPS = MX ? (NSC + WAVES - 1) / WAVES : 0;
    constexpr int LPT = LPT0 + (BLK ? 2 : 0) + LPS;  // + the scale loads
    constexpr int STAGE_BYTES = ROWS * KSTAGE + SC_REGION;
    // 256x256 tiles and the Block-FP8 tiles stream their fragments (see the
    // K loop)
    constexpr bool STREAM = (BP * BQ >= 256 * 256 || BLK) && !MX;
    static_assert(ROWS * NC % THREADS == 0, "stage must split evenly over the waves");
    static_assert((NC & (NC - 1)) == 0 && KSTAGE % KSTEP == 0, "bad K stage");
    static_assert(STAGES >= 2 && (STAGES - 1) * LPT < 64, "bad pipeline depth");
    static_assert(!GROUPED || (!SPLITK && (OP == OP_FP8 || OP == OP_INT8)),
                  "grouped: per-token x per-channel ops, no Split-K");
    static_assert(!BLK || (KSTAGE == 128 && NSTEP == 1 && BP <= 256 && WAVES >= BP / 64),
                  "block scaling: one 128-wide K group per stage");
    static_assert(!MX || ((SCB == 8 || SCB == 16) && BP % (256 / (SCB ? SCB : 1)) == 0),
                  "MXFP4: a scale copy unit must not straddle the A and B rows");

    // One LDS object per ring slot, the slot known at compile time in the
    // unrolled K loop (constant LDS addresses for the fragment reads).
    constexpr int SLOT = pipe_slot_bytes<OP, BP, BQ, KSTAGE>();
    static_assert(KGRP == 1 || (KGRP == 2 && !BLK && !MX && !GROUPED &&
                                (OP == OP_FP8 || OP == OP_INT8) && !(BP * BQ >= 256 * 256)),
                  "K groups: the per-token x per-channel tiles with a register-set K loop");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[KGRP * STAGES * SLOT];
    // Block-FP8: the K group's activation scales of the tile rows (256
    // floats) and its weight-block scales (64) per stage, in a ring of
    // STAGES + 1 entries, so that a stage's scales outlive the reuse of its
    // operand slot while its MFMAs run.
    constexpr int SC_SLOTS = BLK ? STAGES + 1 : 1;
    constexpr int SC_FLOATS = 320;
    __shared__ __attribute__((aligned(16))) float lsc[SC_SLOTS][BLK ? SC_FLOATS : 4];
    static_assert(STAGES <= 8, "at most eight ring slots");
    static_assert(RC == 0 || (STAGES == 2 && !STREAM && !MX && !BLK && !GROUPED && KGRP == 1 &&
                              RC <= 4),
                  "register-path copies: plain per-token x per-channel or bf16 tiles, two slots");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // this wave's K group and its index within the group (wave-uniform)
    const int kgi = KGRP > 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) / (WP * WQ) : 0;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) % (WP * WQ);
    uint8_t* const gring = KGRP > 1 ? ring + kgi * (STAGES * SLOT) : ring;
    auto slot = [&](auto J) __attribute__((always_inline)) -> uint8_t* {
        return gring + decltype(J)::value * SLOT;
    };
    const int wpi = wave % WP, wqi = wave / WP;
    const int N = a.N;
    const int tq = (N + BQ - 1) / BQ;
    int M = a.M;  // the tile's row limit (grouped: the end of its expert's rows)
    int tile_p, tile_q, p0;
    const uint8_t* Bp = (const uint8_t*)a.B;
    const float* sbp = a.sb;
    if constexpr (GROUPED) {
        // The grid covers the most row tiles the experts can have (one
        // partial tile each beyond ceil(M / BP)); the tiles they do have are
        // counted here and spread evenly over the XCDs, and the workgroups
        // beyond them on each XCD leave at once (else the XCDs that draw the
        // end of the range would idle).
        const int rows = __builtin_amdgcn_readfirstlane(
            group_row_tiles(a.offsets, a.E, a.M, BP, lane));
        const int T = rows * tq;
        const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
        if (loc >= (T >> 3) + (xcd < (T & 7) ? 1 : 0))
            return;  // (the same for every wave)
        xcd_tile(blockIdx.x, rows, tq, 4, tile_p, tile_q);
        int e, m0, m1;
        group_tile(a.offsets, a.E, a.M, tile_p, BP, lane, e, m0, m1);
        // equal in every lane: make them scalar (the buffer resources below
        // must live in scalar registers)
        e = __builtin_amdgcn_readfirstlane(e);
        m0 = __builtin_amdgcn_readfirstlane(m0);
        m1 = __builtin_amdgcn_readfirstlane(m1);
        if (e < 0)
            return;  // past the last tile (the same for every wave)
        p0 = m0;
        M = m1;
        Bp += (size_t)e * N * (size_t)a.kbytes;
        sbp += (size_t)e * N;
    } else {
        const int tp = (M + BP - 1) / BP;
        xcd_tile(blockIdx.x, tp, tq, 4, tile_p, tile_q);
        p0 = tile_p * BP;
    }
    const int q0 = tile_q * BQ;
    const int z = blockIdx.y;
    // the workgroup's K range [kbeg0, kend0), its group's part [kbeg, kend)
    // of nk stages (the same nk for both groups; a short or empty second
    // part reads zeros and skips its MFMAs past kend)
    const int kbeg0 = z * a.kchunk;
    const int kend0 = min(a.kbytes, kbeg0 + a.kchunk);
    const int nk0 = (kend0 - kbeg0 + KSTAGE - 1) / KSTAGE;
    const int nk = KGRP > 1 ? (nk0 + 1) / 2 : nk0;
    const int kbeg = kbeg0 + kgi * nk * KSTAGE;
    const int kend = KGRP > 1 ? min(kend0, kbeg + nk * KSTAGE) : kend0;
    const uint32_t ldk = (uint32_t)a.kbytes;

    // The tile's A rows and B rows as two buffers, each ending at the last
    // row of its matrix.
    const v4i rsA = buffer_rsrc((const uint8_t*)a.A + (size_t)p0 * ldk,
                                (uint32_t)min((uint64_t)(M - p0) * ldk, (uint64_t)0x7FFFFFFF));
    const v4i rsB = buffer_rsrc(Bp + (size_t)q0 * ldk,
                                (uint32_t)min((uint64_t)(N - q0) * ldk, (uint64_t)0x7FFFFFFF));

    // Source of each of this thread's LPT loads: LDS chunk index
    // L = (i * WAVES + wave) * 64 + lane holds logical chunk
    // (L % NC) ^ swz(r) of stage row L / NC, r its row within the A or B
    // part (the fragment reads swizzle with that row index).  One load
    // instruction fills 1024 / KSTAGE whole rows of one part, so the part is
    // wave-uniform.
    auto chunk_of = [&](int i) __attribute__((always_inline)) {
        const int L = (i * WAVES + wave) * 64 + lane;
        const int row = L / NC;
        return (L % NC) ^ swz<NC>(row < BP ? row : row - BP);
    };
    auto in_a = [&](int i) __attribute__((always_inline)) {
        return (i * WAVES + wave) * 64 / NC < BP;
    };
    uint32_t voff[LPT0];
#pragma unroll
    for (int i = 0; i < LPT0; ++i) {
        const int row = ((i * WAVES + wave) * 64 + lane) / NC;
        const int r = in_a(i) ? row : row - BP;
        voff[i] = (uint32_t)r * ldk + (uint32_t)kbeg + (uint32_t)chunk_of(i) * 16u;
    }

    // Block-FP8 scale sources: sa [M][KG] from the tile's first row, sb
    // [ceil(N/128)][KG] from the tile's first column block.  Each wave loads
    // one 64-row chunk of the tile's activation scales (chunks repeat when
    // there are more waves than chunks: the copies write equal values) and
    // the (at most four) weight-block scales, so that every wave issues the
    // same number of loads per stage.
    const int KG = a.K / 128;
    v4i rsSa{}, rsSb{};
    uint32_t sa_off = 0, sb_off = kOutOfRange;
    constexpr int SA_CHUNKS = BP >= 64 ? BP / 64 : 1;
    const int sa_chunk = wave % SA_CHUNKS;
    if constexpr (BLK) {
        rsSa = buffer_rsrc(a.sa + (size_t)p0 * KG,
                           (uint32_t)min((uint64_t)(M - p0) * KG * 4, (uint64_t)0x7FFFFFFF));
        const int nb0 = q0 >> 7, nbs = (N + 127) >> 7;
        rsSb = buffer_rsrc(a.sb + (size_t)nb0 * KG,
                           (uint32_t)min((uint64_t)(nbs - nb0) * KG * 4, (uint64_t)0x7FFFFFFF));
        sa_off = (uint32_t)((sa_chunk * 64 + lane) * KG) * 4u;
        if (lane < 4)
            sb_off = (uint32_t)(lane * KG) * 4u;
    }

    // MXFP4 scale sources: [M][K/32] and [N][K/32] bytes from the tile's
    // first row; unit c of a stage holds the bytes c*256 + 4*lane .. + 3 of
    // the stage's [ROWS][SCB] scale block.
    v4i rsXA{}, rsXB{};
    uint32_t xoff[LPS > 0 ? LPS : 1];
    int xj[LPS > 0 ? LPS : 1];
    bool xin_a[LPS > 0 ? LPS : 1];
    uint32_t xdst[LPS > 0 ? LPS : 1];
    const uint32_t srow = (uint32_t)a.kbytes / 16u;
    if constexpr (MX) {
        rsXA = buffer_rsrc((const uint8_t*)a.sa + (size_t)p0 * srow,
                           (uint32_t)min((uint64_t)(M - p0) * srow, (uint64_t)0x7FFFFFFF));
        rsXB = buffer_rsrc((const uint8_t*)a.sb + (size_t)q0 * srow,
                           (uint32_t)min((uint64_t)(N - q0) * srow, (uint64_t)0x7FFFFFFF));
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const int c = (i * WAVES + wave) % NSC;
            const int b = c * 256 + lane * 4;
            const int row = b / SCB, j = b % SCB;
            xin_a[i] = c * 256 / SCB < BP;  // wave-uniform
            const int r = row < BP ? row : row - BP;
            xoff[i] = row < ROWS ? (uint32_t)r * srow + (uint32_t)(kbeg / 16 + j) : kOutOfRange;
            xj[i] = j;
            xdst[i] = (uint32_t)(ROWS * KSTAGE + c * 256);
        }
    }

    // the operand copies i0 .. i1 - 1 of stage kt (of this wave's LPT0)
    auto issue_ops = [&](int kt, uint8_t* buf, int i0, int i1) __attribute__((always_inline)) {
        const int kb0 = kt * KSTAGE;  // relative to kbeg
        const bool full = kbeg + kb0 + KSTAGE <= kend;
#pragma unroll
        for (int i = 0; i < LPT0; ++i) {
            if (i < i0 || i >= i1)
                continue;
            uint32_t vo = voff[i] + (uint32_t)kb0;
            if (!full && kbeg + kb0 + chunk_of(i) * 16 >= kend)
                vo = kOutOfRange;  // past the K range: zeros
            dma16(vo, in_a(i) ? rsA : rsB,
                  __builtin_amdgcn_readfirstlane(
                      (uint32_t)(uintptr_t)(buf + (i * WAVES + wave) * 1024)));
        }
    };
    // the scale copies of stage kt (MXFP4 block scales, Block-FP8 scales)
    auto issue_scales = [&](int kt, uint8_t* buf) __attribute__((always_inline)) {
        const int kb0 = kt * KSTAGE;
        const bool full = kbeg + kb0 + KSTAGE <= kend;
        (void)full;
        if constexpr (MX) {
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
                // scale byte j covers code bytes 16 j .. 16 j + 15 of the stage
                uint32_t xo = xoff[i] + (uint32_t)(kt * SCB);
                if (xoff[i] == kOutOfRange || (!full && kbeg + kb0 + xj[i] * 16 >= kend))
                    xo = kOutOfRange;
                dma4(xo, xin_a[i] ? rsXA : rsXB,
                     __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(buf + xdst[i])));
            }
        }
        if constexpr (BLK) {
            const uint32_t g4 = (uint32_t)((kbeg + kb0) >> 7) * 4u;
            float* sc = lsc[kt % SC_SLOTS];
            dma4(sa_off + g4, rsSa,
                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(sc + sa_chunk * 64)));
            dma4(sb_off == kOutOfRange ? kOutOfRange : sb_off + g4, rsSb,
                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(sc + 256)));
        }
    };
    auto issue = [&](int kt, uint8_t* buf) __attribute__((always_inline)) {
        issue_ops(kt, buf, 0, LPT0);
        issue_scales(kt, buf);
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

    // The MFMA fragments of one K step (the wave's RP A blocks and RQ B
    // blocks) are read from LDS into one of two register sets while the
    // MFMAs of the previous step run on the other, so the LDS latency hides
    // behind the matrix cores.  Global step g = kt * NSTEP + ks uses set g % 2.
    struct Frag {
        uint4 a[RP][KB / 16];
        uint4 b[RQ][KB / 16];
        int xa[MX ? RP : 1];  // MXFP4: this lane's block scale per fragment
        int xb[MX ? RQ : 1];
    };
    Frag fr[2];
    auto load_step = [&](const uint8_t* sp, int ks, Frag& f) __attribute__((always_inline)) {
        const uint8_t* sq = sp + BP * KSTAGE;
        const int off = ks * KSTEP + (lane >> 4) * KB;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int row = wpi * SP + i * 16 + (lane & 15);
#pragma unroll
            for (int j = 0; j < KB / 16; ++j) {
                const int ch = (off >> 4) + j;
                f.a[i][j] = *(const uint4*)(sp + row * KSTAGE + ((ch ^ swz<NC>(row)) << 4));
            }
        }
#pragma unroll
        for (int i = 0; i < RQ; ++i) {
            const int row = wqi * SQ + i * 16 + (lane & 15);
#pragma unroll
            for (int j = 0; j < KB / 16; ++j) {
                const int ch = (off >> 4) + j;
                f.b[i][j] = *(const uint4*)(sq + row * KSTAGE + ((ch ^ swz<NC>(row)) << 4));
            }
        }
        if constexpr (MX) {
            // scale byte of step ks, block lane >> 4, of each fragment row
            const uint8_t* sc = sp + ROWS * KSTAGE + ks * 4 + (lane >> 4);
#pragma unroll
            for (int i = 0; i < RP; ++i)
                f.xa[i] = sc[(wpi * SP + i * 16 + (lane & 15)) * SCB];
#pragma unroll
            for (int i = 0; i < RQ; ++i)
                f.xb[i] = sc[(BP + wqi * SQ + i * 16 + (lane & 15)) * SCB];
        }
    };
    auto compute_step = [&](const Frag& f, int kt, int ks) __attribute__((always_inline)) {
        if (kbeg + kt * KSTAGE + ks * KSTEP >= kend)
            return;  // steps past the K range (zero-filled) are skipped
        if constexpr (BLK) {
            // promotion: a fresh MFMA partial per K group, scaled by
            // sa[m][g] * sb[n / 128][g] into the fp32 accumulator
            // The wave's SQ columns start at a multiple of SQ <= 128, so
            // they lie in one 128-column weight block: one weight scale per
            // step, and the scale product sa * sb is formed once per row.
            static_assert(SQ <= 128, "a wave's columns must share one weight block");
            const float* sc = lsc[kt % SC_SLOTS];
            const float qs = sc[256 + (((q0 & 127) + wqi * SQ) >> 7)];
            float4 ps[RP];
#pragma unroll
            for (int i = 0; i < RP; ++i) {
                ps[i] = *(const float4*)(sc + wpi * SP + i * 16 + (lane >> 4) * 4);
                ps[i].x *= qs;
                ps[i].y *= qs;
                ps[i].z *= qs;
                ps[i].w *= qs;
            }
#pragma unroll
            for (int i = 0; i < RP; ++i)
#pragma unroll
                for (int j = 0; j < RQ; ++j) {
                    const v4f pg = mfma_step<OP>(f.a[i], f.b[j], v4f{0, 0, 0, 0});
                    acc[i][j][0] = __builtin_fmaf(ps[i].x, pg[0], acc[i][j][0]);
                    acc[i][j][1] = __builtin_fmaf(ps[i].y, pg[1], acc[i][j][1]);
                    acc[i][j][2] = __builtin_fmaf(ps[i].z, pg[2], acc[i][j][2]);
                    acc[i][j][3] = __builtin_fmaf(ps[i].w, pg[3], acc[i][j][3]);
                }
        } else if constexpr (MX) {
#pragma unroll
            for (int i = 0; i < RP; ++i)
#pragma unroll
                for (int j = 0; j < RQ; ++j)
                    acc[i][j] = mfma_mx(f.a[i][0], f.b[j][0], acc[i][j], f.xa[i], f.xb[j]);
        } else {
#pragma unroll
            for (int i = 0; i < RP; ++i)
#pragma unroll
                for (int j = 0; j < RQ; ++j)
                    acc[i][j] = mfma_step<OP>(f.a[i], f.b[j], acc[i][j]);
        }
    };
    // wait for the oldest stage in flight with `younger` later stages still
    // allowed in flight
    auto wait_stage = [&](int younger) __attribute__((always_inline)) {
        wait_younger<STAGES - 1, LPT>(younger);
    };
    using I0 = std::integral_constant<int, 0>;

    // The tile's scales, into LDS ahead of the operand stages (the stage
    // waits, which count only the younger copies, also cover these): unit u
    // holds sa of tile rows 64u .. 64u + 63 (u < UA), then sb of the tile
    // columns; entries past M or N read as zero.
    constexpr bool SCALED = OP == OP_INT8 || OP == OP_FP8;
    constexpr bool PRE = pipe_prescale<OP, BP, BQ, KSTAGE, STAGES, KGRP>();
    constexpr int UA = (BP + 63) / 64, UB = (BQ + 63) / 64;
    __shared__ __attribute__((aligned(16))) float lpre[PRE ? (UA + UB) * 64 : 1];
    const bool scaled = SCALED && a.splits == 1 && a.out_dtype != OUT_INT32;
    if constexpr (PRE) {
        if (scaled && kgi == 0) {  // (the first K group writes the output)
            const v4i rsPa = buffer_rsrc(
                a.sa + p0, (uint32_t)min((uint64_t)(M - p0) * 4, (uint64_t)0x7FFFFFFF));
            const v4i rsPb = buffer_rsrc(
                sbp + q0, (uint32_t)min((uint64_t)(N - q0) * 4, (uint64_t)0x7FFFFFFF));
            for (int u = wave; u < UA + UB; u += WAVES) {
                const bool ua = u < UA;
                dma4((uint32_t)((ua ? u : u - UA) * 64 + lane) * 4u, ua ? rsPa : rsPb,
                     __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lpre + u * 64)));
            }
        }
    }

    if constexpr (RC > 0) {
        // Register-path copies.  Stage s is loaded into register set s % RC
        // (RC stages ahead), written to LDS slot s % 2 during stage s - 1, and
        // published by the barrier that ends stage s - 1, after which its
        // first step's fragments are read.  Slot s % 2 last held stage s - 2,
        // whose fragments every wave had read (and waited for) before the
        // barrier that ended stage s - 2, and every wave writing stage s has
        // passed that barrier, so the writes need no other wait.
        // The compiler tracks the loads (builtins) and waits for exactly the
        // set a ds_write needs; the only asm copies (the tile's scales) are
        // issued before them, so they only make such a wait stricter.
        const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const uint8_t*)a.A + (size_t)p0 * ldk), (short)0,
            (int)min((uint64_t)(M - p0) * ldk, (uint64_t)0x7FFFFFFF), 0x00020000);
        const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Bp + (size_t)q0 * ldk), (short)0,
            (int)min((uint64_t)(N - q0) * ldk, (uint64_t)0x7FFFFFFF), 0x00020000);
        uint4 rg[RC][LPT0];
        auto gload = [&](int kt, uint4* dst) __attribute__((always_inline)) {
            const int kb0 = kt * KSTAGE;
            const bool full = kbeg + kb0 + KSTAGE <= kend;
#pragma unroll
            for (int i = 0; i < LPT0; ++i) {
                uint32_t vo = voff[i] + (uint32_t)kb0;
                if (!full && kbeg + kb0 + chunk_of(i) * 16 >= kend)
                    vo = kOutOfRange;  // past the K range: zeros
                dst[i] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(in_a(i) ? rA : rB, (int)vo, 0, 0));
            }
        };
        auto swrite = [&](const uint4* src, uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < LPT0; ++i)
                *(uint4*)(buf + ((i * WAVES + wave) * 64 + lane) * 16) = src[i];
        };
        // Every load, write and barrier below is issued unconditionally
        // (stages past the K range load zeros and skip their MFMAs), so the
        // loop body has no branch around a load and the compiler's waits
        // stay exact: a ds_write waits only for its own stage's loads.
        unroll<0, RC>([&](auto J) __attribute__((always_inline)) {
            gload(decltype(J)::value, rg[decltype(J)::value]);
        });
        swrite(rg[0], slot(I0{}));
        gload(RC, rg[0]);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the writes have landed
        __builtin_amdgcn_s_barrier();
        load_step(slot(I0{}), 0, fr[0]);
        // J = kt mod U: LDS slot, register set and fragment set are
        // compile-time constants
        constexpr int U = RC % 2 == 0 ? RC : 2 * RC;
        auto stage = [&](auto J, int kt) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
            constexpr int cs = j % 2, ns = (j + 1) % 2, rs = (j + 1) % RC;
            if constexpr (FOLD) {
                if (kt < nk)
                    fold.before(kt * NSTEP, acc);
            }
#pragma unroll
            for (int ks = 0; ks < NSTEP; ++ks) {
                const int cp = (j * NSTEP + ks) & 1;
                if (ks + 1 < NSTEP) {
                    load_step(slot(std::integral_constant<int, cs>{}), ks + 1, fr[cp ^ 1]);
                } else {
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    swrite(rg[rs], slot(std::integral_constant<int, ns>{}));
                    gload(kt + 1 + RC, rg[rs]);
                    __builtin_amdgcn_s_waitcnt(0xC07F);
                    __builtin_amdgcn_s_barrier();
                    load_step(slot(std::integral_constant<int, ns>{}), 0, fr[cp ^ 1]);
                }
                compute_step(fr[cp], kt, ks);  // (returns for stages past the K range)
            }
        };
        for (int kt = 0; kt < nk; kt += U)
            unroll<0, U>([&](auto J) __attribute__((always_inline)) {
                stage(J, kt + decltype(J)::value);
            });
    } else if constexpr (!STREAM) {
        // prologue: every ring slot receives a stage (0 .. STAGES-1); the
        // fragments of step 0 go to register set 0
        for_stages<0, STAGES>([&](auto J, int kt) __attribute__((always_inline)) {
            issue(kt, slot(J));
        }, 0, nk);
        if (0 < nk) {
            wait_stage(min(STAGES - 1, nk - 1));
            load_step(slot(I0{}), 0, fr[0]);
        }

        // stage kt (J = kt mod U, U a multiple of STAGES with U * NSTEP even, so
        // that ring slot and register set are compile-time constants): the steps
        // of the stage run one after the other, each reading the next step's
        // fragments first.  Before the last step, once stage kt+1 has landed for
        // every wave and every wave holds its stage-kt fragments in registers,
        // slot kt % STAGES takes stage kt + STAGES and the first step of stage
        // kt+1 is read from the next slot.
        constexpr int U = (NSTEP % 2 == 0 || STAGES % 2 == 0) ? STAGES : 2 * STAGES;
        // Workgroups of up to 8 waves issue a stage's copies after the MFMAs
        // of its last K step, not before them: the texture unit takes the
        // CU's copies one after another, and a wave issuing its copies first
        // would wait for its place in that queue before its MFMAs.  The slot
        // is free from the barrier on either way.  With 16 waves (four MFMAs
        // per wave per stage) the later issue cost more in copy latency than
        // it saved (measured on 128x128 tiles: 3-5% slower; 4 and 8 waves:
        // 2-10% faster).
        constexpr bool DEFER = WAVES <= 8;
        auto stage = [&](auto J, int kt) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
            constexpr int cs = j % STAGES, ns = (j + 1) % STAGES;
            if constexpr (FOLD)
                fold.before(kt * NSTEP, acc);  // chunk boundaries fall on stage starts
    #pragma unroll
            for (int ks = 0; ks < NSTEP; ++ks) {
                const int cp = (j * NSTEP + ks) & 1;
                if (ks + 1 < NSTEP) {
                    load_step(slot(std::integral_constant<int, cs>{}), ks + 1, fr[cp ^ 1]);
                } else {
                    // the fragments of this step are in registers on every path
                    // from here on, so the compiler never holds the MFMAs for the
                    // reads issued below
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    if (kt + 1 < nk) {
                        wait_stage(min(STAGES - 2, nk - 2 - kt));
                        if (!DEFER && kt + STAGES < nk)
                            issue(kt + STAGES, slot(std::integral_constant<int, cs>{}));
                        load_step(slot(std::integral_constant<int, ns>{}), 0, fr[cp ^ 1]);
                    }
                }
                compute_step(fr[cp], kt, ks);
                if (DEFER && ks + 1 == NSTEP && kt + STAGES < nk)
                    issue(kt + STAGES, slot(std::integral_constant<int, cs>{}));
            }
        };
        for (int kt = 0; kt < nk; kt += U)
            for_stages<0, U>(stage, kt, nk);
    } else {
        // Streamed fragments, for tiles whose two register sets of a whole K
        // step would not fit next to the accumulators (256x256 tiles; the
        // Block-FP8 tiles, whose promotion needs registers of its own):
        // STAGES - 1 stages in flight ahead of the one being computed; per K
        // step each wave reads its RQ B fragments, then its A fragments one
        // row block at a time, each read issued before the MFMAs of the
        // previous row block.  The other waves on the SIMD run while one
        // waits for its reads.
        static_assert(!MX, "streamed tiles: no MXFP4");
        for_stages<0, STAGES - 1>([&](auto J, int kt) __attribute__((always_inline)) {
            issue(kt, slot(J));
        }, 0, nk);
        auto sstage = [&](auto J, int kt) __attribute__((always_inline)) {
            constexpr int cs = decltype(J)::value;
            constexpr int fs = (cs + STAGES - 1) % STAGES;  // the slot of stage kt - 1
            // stage kt has landed for every wave (younger ones may still be
            // in flight), and every wave is done with stage kt - 1: its slot
            // takes stage kt + STAGES - 1
            wait_stage(min(STAGES - 2, nk - 1 - kt));
            // The copies of stage kt + STAGES - 1 are spread over the first
            // half of the first K step's row blocks (two of RP row blocks
            // carry 2 LPT0 / RP of them each) instead of all being issued
            // here: the texture unit takes the CU's copies one after another,
            // and a wave that had to issue all its copies first would wait
            // for its place in that queue before its first MFMA.  (Step 0 of
            // a stage kt < nk always lies in the K range, so it is never
            // skipped.)
            const bool fresh = kt + STAGES - 1 < nk;
            uint8_t* const fslot = slot(std::integral_constant<int, fs>{});
            if (fresh)
                issue_scales(kt + STAGES - 1, fslot);
            auto spread = [&](int ks, int i) __attribute__((always_inline)) {
                if (ks == 0 && fresh && 2 * i < RP)
                    issue_ops(kt + STAGES - 1, fslot, 2 * i * LPT0 / RP,
                              2 * i + 2 >= RP ? LPT0 : (2 * i + 2) * LPT0 / RP);
            };
            if constexpr (FOLD)
                fold.before(kt * NSTEP, acc);
            const uint8_t* sp = slot(std::integral_constant<int, cs>{});
            const uint8_t* sq = sp + BP * KSTAGE;
#pragma unroll
            for (int ks = 0; ks < NSTEP; ++ks) {
                if (kbeg + kt * KSTAGE + ks * KSTEP >= kend)
                    continue;  // steps past the K range (zero-filled)
                const int off = ks * KSTEP + (lane >> 4) * KB;
                uint4 bv[RQ][KB / 16];
#pragma unroll
                for (int i = 0; i < RQ; ++i) {
                    const int row = wqi * SQ + i * 16 + (lane & 15);
#pragma unroll
                    for (int j = 0; j < KB / 16; ++j) {
                        const int ch = (off >> 4) + j;
                        bv[i][j] = *(const uint4*)(sq + row * KSTAGE + ((ch ^ swz<NC>(row)) << 4));
                    }
                }
                uint4 av[2][KB / 16];
                auto read_a = [&](int i, uint4* dst) __attribute__((always_inline)) {
                    const int row = wpi * SP + i * 16 + (lane & 15);
#pragma unroll
                    for (int j = 0; j < KB / 16; ++j) {
                        const int ch = (off >> 4) + j;
                        dst[j] = *(const uint4*)(sp + row * KSTAGE + ((ch ^ swz<NC>(row)) << 4));
                    }
                };
                read_a(0, av[0]);
                if constexpr (BLK) {
                    // promotion as in compute_step, pipelined by row block:
                    // the fresh partials of row block i + 1 are issued before
                    // the fmas of row block i, so the matrix cores never wait
                    // for the promotion of the previous block
                    static_assert(SQ <= 128, "a wave's columns must share one weight block");
                    const float* sc = lsc[kt % SC_SLOTS];
                    const float qs = sc[256 + (((q0 & 127) + wqi * SQ) >> 7)];
                    v4f pg[2][RQ];
#pragma unroll
                    for (int j = 0; j < RQ; ++j)
                        pg[0][j] = mfma_step<OP>(av[0], bv[j], v4f{0, 0, 0, 0});
#pragma unroll
                    for (int i = 0; i < RP; ++i) {
                        spread(ks, i);
                        if (i + 1 < RP) {
                            read_a(i + 1, av[(i + 1) & 1]);
#pragma unroll
                            for (int j = 0; j < RQ; ++j)
                                pg[(i + 1) & 1][j] =
                                    mfma_step<OP>(av[(i + 1) & 1], bv[j], v4f{0, 0, 0, 0});
                        }
                        float4 ps = *(const float4*)(sc + wpi * SP + i * 16 + (lane >> 4) * 4);
                        ps.x *= qs;
                        ps.y *= qs;
                        ps.z *= qs;
                        ps.w *= qs;
#pragma unroll
                        for (int j = 0; j < RQ; ++j) {
                            acc[i][j][0] = __builtin_fmaf(ps.x, pg[i & 1][j][0], acc[i][j][0]);
                            acc[i][j][1] = __builtin_fmaf(ps.y, pg[i & 1][j][1], acc[i][j][1]);
                            acc[i][j][2] = __builtin_fmaf(ps.z, pg[i & 1][j][2], acc[i][j][2]);
                            acc[i][j][3] = __builtin_fmaf(ps.w, pg[i & 1][j][3], acc[i][j][3]);
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < RP; ++i) {
                        spread(ks, i);
                        if (i + 1 < RP)
                            read_a(i + 1, av[(i + 1) & 1]);
#pragma unroll
                        for (int j = 0; j < RQ; ++j)
                            acc[i][j] = mfma_step<OP>(av[i & 1], bv[j], acc[i][j]);
                    }
                }
            }
        };
        for (int kt = 0; kt < nk; kt += STAGES)
            for_stages<0, STAGES>(sstage, kt, nk);
    }

    if constexpr (FOLD)
        fold.finish(acc);

    // Epilogue through LDS: each wave writes one 16-row block of its tile at a
    // time into a private LDS scratch, then every lane emits 8 consecutive
    // columns of one row -- a 16-byte bf16 store (two for fp32) instead of
    // eight scattered 2-byte stores.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // ring slots are free
    if constexpr (KGRP > 1) {
        // The second K group parks its accumulators at the end of the ring
        // (its own ring, clear of the first group's epilogue scratch); the
        // first adds them to its own, first group + second group, and goes
        // on to the epilogue alone.
        constexpr int PART = WP * WQ * RP * RQ * 4 * 64 * 4;
        static_assert(PART <= STAGES * SLOT, "the partial tile must fit the second ring");
        uint32_t* pt = (uint32_t*)(ring + KGRP * STAGES * SLOT - PART) + wave * (RP * RQ * 4 * 64);
        if (kgi == 1) {
#pragma unroll
            for (int i = 0; i < RP; ++i)
#pragma unroll
                for (int j = 0; j < RQ; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        // (through a scalar: the bit cast of a vector element
                        // in place reads the vector's first element)
                        const elem_t e = acc[i][j][v];
                        pt[((i * RQ + j) * 4 + v) * 64 + lane] = __builtin_bit_cast(uint32_t, e);
                    }
        }
        __syncthreads();
        if (kgi == 1)
            return;
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int j = 0; j < RQ; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[i][j][v] +=
                        __builtin_bit_cast(elem_t, pt[((i * RQ + j) * 4 + v) * 64 + lane]);
    }
    // bf16 output (the common case): store_bf16_batched, which scales each
    // accumulator as the general path below does -- (acc * sa[m]) * sb[n]
    // for the per-token x per-channel ops -- and rounds it the same way, so
    // the same bits.
    if constexpr (!SCALED || PRE) {
        if (a.out_dtype == OUT_BF16 && a.splits == 1 && (N & 7) == 0 && (!SCALED || scaled)) {
            constexpr int BB = bf16_batch_blocks<RP, SQ>(STAGES * SLOT / WAVES);
            constexpr int RBB = 16 * (SQ / 2 + 4) * 4;
            static_assert(STAGES * SLOT / WAVES >= RBB, "epilogue scratch must fit the ring");
            store_bf16_batched<RP, RQ, BB, SCALED>(
                acc, (uint32_t*)(ring + wave * BB * RBB), SCALED ? lpre + wpi * SP : nullptr,
                SCALED ? lpre + UA * 64 + wqi * SQ : nullptr, lane, p0 + wpi * SP,
                q0 + wqi * SQ, M, N, (uint16_t*)a.out);
            return;
        }
    }
    // Scratch rows of SQ + 4 words: a lane writes rows 4 (lane / 16) + v of
    // its column, so that each half-wave's two lane groups (4 rows apart)
    // fall on the two disjoint halves of the 32 LDS banks instead of on the
    // same 16 (with rows of SQ words, a multiple of 32, every 16-lane group
    // of a write hit the same banks).
    constexpr int SQP = SQ + 4;
    static_assert(WAVES * 16 * SQP * 4 <= STAGES * SLOT, "epilogue scratch must fit the ring");
    elem_t* scr = (elem_t*)(ring + wave * 16 * SQP * 4);
    constexpr int CPR = SQ / 8;          // 8-column groups per row
    constexpr int RPP = 64 / CPR;        // rows per pass
    constexpr int PASSES = 16 / RPP;
    const bool vec_ok = (N & 7) == 0;
    const int c = (lane % CPR) * 8;      // this lane's 8 columns, fixed
    const int n = q0 + wqi * SQ + c;
    // The per-token and per-channel scales this lane applies, read together
    // before the stores (from the LDS copy when there is one) instead of one
    // dependent load per element.
    float sbv[8], sav[RP][PASSES];
    if (SCALED && scaled) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (PRE)
                sbv[t] = lpre[UA * 64 + wqi * SQ + c + t];
            else
                sbv[t] = n + t < N ? sbp[n + t] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int pass = 0; pass < PASSES; ++pass) {
                const int r = wpi * SP + i * 16 + pass * RPP + lane / CPR;
                if constexpr (PRE)
                    sav[i][pass] = lpre[r];
                else
                    sav[i][pass] = p0 + r < M ? a.sa[p0 + r] : 0.0f;
            }
    }
    // the epilogue value of an accumulator element: (acc * sa[m]) * sb[n]
    // for the per-token x per-channel ops, the accumulator otherwise
    auto value = [&](elem_t e, int i, int pass, int t) __attribute__((always_inline)) -> float {
        if constexpr (SCALED) {
            const float u = (float)e * sav[i][pass];
            return u * sbv[t];
        } else {
            return (float)e;
        }
    };
#pragma unroll
    for (int i = 0; i < RP; ++i) {
#pragma unroll
        for (int j = 0; j < RQ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                scr[((lane >> 4) * 4 + v) * SQP + j * 16 + (lane & 15)] = acc[i][j][v];
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            const int r = pass * RPP + lane / CPR;
            const int m = p0 + wpi * SP + i * 16 + r;
            elem_t e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                e[t] = scr[r * SQP + c + t];
            if (m >= M)
                continue;
            if (a.splits > 1 || (OP == OP_INT8 && a.out_dtype == OUT_INT32)) {
                // raw accumulators: Split-K partials or the INT8 int32 output
                elem_t* dst = a.splits > 1 ? (elem_t*)a.ws + ((size_t)z * M + m) * N + n
                                           : (elem_t*)a.out + (size_t)m * N + n;
                if (vec_ok && n + 7 < N) {
                    uint32_t u[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        u[t] = __builtin_bit_cast(uint32_t, e[t]);
                    if (a.splits > 1) {
                        ((uint4*)dst)[0] = make_uint4(u[0], u[1], u[2], u[3]);
                        ((uint4*)dst)[1] = make_uint4(u[4], u[5], u[6], u[7]);
                    } else {
                        store16_stream(dst, u[0], u[1], u[2], u[3]);
                        store16_stream(dst + 4, u[4], u[5], u[6], u[7]);
                    }
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = e[t];
                }
            } else if (a.out_dtype == OUT_BF16) {
                uint16_t* dst = (uint16_t*)a.out + (size_t)m * N + n;
                if (vec_ok && n + 7 < N) {
                    uint32_t w[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        w[t] = (uint32_t)bf16_rne(value(e[2 * t], i, pass, 2 * t)) |
                               ((uint32_t)bf16_rne(value(e[2 * t + 1], i, pass, 2 * t + 1)) << 16);
                    store16_stream(dst, w[0], w[1], w[2], w[3]);
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = bf16_rne(value(e[t], i, pass, t));
                }
            } else {
                float* dst = (float*)a.out + (size_t)m * N + n;
                float y[8];
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    y[t] = value(e[t], i, pass, t);
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

template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int STAGES, bool SPLITK,
          bool GROUPED = false, int KGRP = 1>
__global__ __launch_bounds__(KGRP* WP* WQ * 64)
__attribute__((amdgpu_waves_per_eu(
    pipe_waves_per_eu<OP, BP, BQ, WP, WQ, KSTAGE, STAGES, KGRP>())))
void gemm_pipe_kernel(GemmArgs a)
{
    gemm_pipe_body<OP, BP, BQ, WP, WQ, KSTAGE, STAGES, SPLITK, GROUPED, KGRP, 0>(a);
}

// Register cap for WP x WQ / 4 waves per SIMD (one workgroup's share): the
// register sets of the copies in flight take registers a second workgroup
// would need (the 16-wave tiles run one workgroup per CU; 8-wave tiles that
// stay under 128 registers can still pair).
template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int RC, bool SPLITK>
__global__ __launch_bounds__(WP* WQ * 64)
__attribute__((amdgpu_waves_per_eu(WP * WQ >= 8 ? WP * WQ / 4 : 1)))
void gemm_pipe_rc_kernel(GemmArgs a)
{
    gemm_pipe_body<OP, BP, BQ, WP, WQ, KSTAGE, 2, SPLITK, false, 1, RC>(a);
}

template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int RC>
hipError_t launch_pipe_rc(const GemmArgs& a, hipStream_t stream)
{
    const long tiles = (long)((a.M + BP - 1) / BP) * ((a.N + BQ - 1) / BQ);
    if (tiles > 0x7FFFFFFFL || (long)(BP > BQ ? BP : BQ) * a.kbytes > 0x7FFFFFFFL)
        return hipErrorInvalidValue;  // 32-bit buffer offsets within a tile
    const dim3 block(WP * WQ * 64);
    if (a.splits > 1)
        hipLaunchKernelGGL((gemm_pipe_rc_kernel<OP, BP, BQ, WP, WQ, KSTAGE, RC, true>),
                           dim3((unsigned)tiles, (unsigned)a.splits), block, 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_pipe_rc_kernel<OP, BP, BQ, WP, WQ, KSTAGE, RC, false>),
                           dim3((unsigned)tiles, 1), block, 0, stream, a);
    return hipGetLastError();
}

template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int STAGES, int KGRP = 1>
hipError_t launch_pipe(const GemmArgs& a, hipStream_t stream)
{
    const long tiles = (long)((a.M + BP - 1) / BP) * ((a.N + BQ - 1) / BQ);
    if (tiles > 0x7FFFFFFFL || (long)(BP > BQ ? BP : BQ) * a.kbytes > 0x7FFFFFFFL)
        return hipErrorInvalidValue;  // 32-bit buffer offsets within a tile
    const dim3 block(KGRP * WP * WQ * 64);
    if (a.splits > 1)
        hipLaunchKernelGGL(
            (gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KSTAGE, STAGES, true, false, KGRP>),
            dim3((unsigned)tiles, (unsigned)a.splits), block, 0, stream, a);
    else
        hipLaunchKernelGGL(
            (gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KSTAGE, STAGES, false, false, KGRP>),
            dim3((unsigned)tiles, 1), block, 0, stream, a);
    return hipGetLastError();
}

template <int OP, int BP, int BQ, int WP, int WQ, int KSTAGE, int STAGES>
hipError_t launch_pipe_grouped(const GemmArgs& a, hipStream_t stream)
{
    const long tiles = (long)((a.M + BP - 1) / BP + a.E) * ((a.N + BQ - 1) / BQ);
    if (a.splits != 1 || tiles > 0x7FFFFFFFL ||
        (long)(BP > BQ ? BP : BQ) * a.kbytes > 0x7FFFFFFFL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KSTAGE, STAGES, false, true>),
                       dim3((unsigned)tiles, 1), dim3(WP * WQ * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qll

// X(OP, BP, BQ, WP, WQ, KSTAGE, STAGES) for every pipelined variant.
#define QLL_FOR_EACH_PIPE(X, OP)           \
    X(OP, 128, 128, 2, 2, 128, 2)          \
    X(OP, 128, 128, 2, 2, 128, 3)          \
    X(OP, 128, 128, 2, 2, 128, 4)          \
    X(OP, 256, 128, 4, 2, 128, 2)          \
    X(OP, 256, 128, 4, 2, 128, 3)          \
    X(OP, 128, 256, 2, 4, 128, 2)          \
    X(OP, 256, 128, 2, 2, 128, 3)          \
    X(OP, 128, 256, 2, 2, 128, 3)          \
    X(OP, 64, 128, 2, 2, 128, 2)           \
    X(OP, 64, 128, 2, 2, 128, 3)           \
    X(OP, 64, 128, 2, 2, 128, 4)           \
    X(OP, 128, 64, 2, 2, 128, 2)           \
    X(OP, 128, 64, 2, 2, 128, 3)           \
    X(OP, 128, 64, 2, 2, 128, 4)           \
    X(OP, 64, 64, 2, 2, 128, 2)            \
    X(OP, 64, 64, 2, 2, 128, 3)            \
    X(OP, 64, 64, 2, 2, 128, 4)            \
    X(OP, 32, 128, 1, 4, 128, 4)           \
    X(OP, 128, 32, 4, 1, 128, 4)

// Tiles over 8 and 16 waves (32x32 to 64x32 per wave): more independent
// copy streams per CU for grids of about one tile per CU.
#define QLL_FOR_EACH_PIPE_W8(X, OP)        \
    X(OP, 128, 128, 2, 4, 128, 3)          \
    X(OP, 128, 128, 4, 2, 128, 3)          \
    X(OP, 128, 128, 4, 4, 128, 3)          \
    X(OP, 128, 128, 4, 4, 128, 4)          \
    X(OP, 128, 64, 4, 2, 128, 3)           \
    X(OP, 128, 64, 4, 2, 128, 4)           \
    X(OP, 64, 128, 2, 4, 128, 3)

#define QLL_FOR_EACH_PIPE_W8_K256(X, OP)   \
    X(OP, 128, 128, 4, 4, 256, 2)          \
    X(OP, 128, 64, 4, 2, 256, 2)

// A deeper ring of 256-byte stages for 64x64 tiles (the mid-size M of
// weight-streaming shapes).  Rings of 6 and 8 128-byte stages of the small
// tiles were measured too and never won.
#define QLL_FOR_EACH_PIPE_DEEP_K256(X, OP) \
    X(OP, 64, 64, 2, 2, 256, 4)

// 256x256 tiles over 8 waves of 128x64, fragments streamed: half the
// operand bytes per flop of a 128x256 tile, for grids of many tiles per CU.
#define QLL_FOR_EACH_PIPE_BIG(X, OP)       \
    X(OP, 256, 256, 2, 4, 128, 2)

// Variants with 256-byte K stages (two fp8 / four bf16 MFMA steps per stage:
// half the barriers per K); not for Block-FP8, whose stage is one K group.
#define QLL_FOR_EACH_PIPE_K256(X, OP)      \
    X(OP, 64, 64, 2, 2, 256, 2)            \
    X(OP, 128, 64, 2, 2, 256, 2)           \
    X(OP, 64, 128, 2, 2, 256, 2)           \
    X(OP, 128, 128, 2, 2, 256, 2)

#define QLL_PIPE_INSTANTIATE(OP, BP, BQ, WP, WQ, KS, ST)                                       \
    template __global__ void qll::gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KS, ST, false>(qll::GemmArgs); \
    template __global__ void qll::gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KS, ST, true>(qll::GemmArgs);
#define QLL_PIPE_GROUPED_INSTANTIATE(OP, BP, BQ, WP, WQ, KS, ST) \
    template __global__ void qll::gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KS, ST, false, true>(qll::GemmArgs);
#define QLL_PIPE_GROUPED_ENTRY(OP, BP, BQ, WP, WQ, KS, ST)                           \
    {"p" #BP "x" #BQ "_w" #WP "x" #WQ "_k" #KS "_s" #ST, OP, 0, BP, BQ, WP, WQ, KS,    \
     qll::pipe_lds_bytes<OP, BP, BQ, KS, ST>(), &qll::launch_pipe_grouped<OP, BP, BQ, WP, WQ, KS, ST>},
#define QLL_PIPE_ENTRY(OP, BP, BQ, WP, WQ, KS, ST)                                   \
    {"p" #BP "x" #BQ "_w" #WP "x" #WQ "_k" #KS "_s" #ST, OP, 0, BP, BQ, WP, WQ, KS,    \
     qll::pipe_lds_bytes<OP, BP, BQ, KS, ST>(), &qll::launch_pipe<OP, BP, BQ, WP, WQ, KS, ST>},

// Tiles whose operand copies go through registers (gemm_pipe_rc_kernel):
// named p<BP>x<BQ>_w<WP>x<WQ>_k<KS>_r<RC>, RC the register stages in flight.
// A copy-path byte costs the LDS about twice what a ds_write byte does (a
// probe copying L2-resident rows beside four bytes of ds_read per copied
// byte: 18.9 TB/s through the copy path, 22.2 TB/s through registers), and
// the fragment reads of these tiles load the LDS that much; the FP8 sweep
// picks them by 1-4% at M = 512-2048.  INT8 and bf16 tiles gained nothing.
#define QLL_FOR_EACH_PIPE_RC(X, OP)        \
    X(OP, 128, 128, 4, 4, 128, 2)          \
    X(OP, 128, 128, 4, 2, 128, 2)          \
    X(OP, 128, 128, 2, 4, 128, 1)          \
    X(OP, 128, 128, 2, 4, 128, 2)          \
    X(OP, 128, 64, 4, 2, 128, 2)           \
    X(OP, 64, 128, 2, 4, 128, 2)
#define QLL_PIPE_RC_INSTANTIATE(OP, BP, BQ, WP, WQ, KS, RC)                                      \
    template __global__ void qll::gemm_pipe_rc_kernel<OP, BP, BQ, WP, WQ, KS, RC, false>(       \
        qll::GemmArgs);                                                                          \
    template __global__ void qll::gemm_pipe_rc_kernel<OP, BP, BQ, WP, WQ, KS, RC, true>(qll::GemmArgs);
#define QLL_PIPE_RC_ENTRY(OP, BP, BQ, WP, WQ, KS, RC)                                \
    {"p" #BP "x" #BQ "_w" #WP "x" #WQ "_k" #KS "_r" #RC, OP, 0, BP, BQ, WP, WQ, KS,    \
     qll::pipe_lds_bytes<OP, BP, BQ, KS, 2>(), &qll::launch_pipe_rc<OP, BP, BQ, WP, WQ, KS, RC>},

// Tiles of two K groups (the in-workgroup Split-K of gemm_pipe_kernel,
// KGRP = 2) for the mid-size M: named p<BP>x<BQ>_w<WP>x<WQ>_k<KS>_s<ST>_g2,
// the wave grid and ring of one group.
#define QLL_FOR_EACH_PIPE_KG2(X, OP)       \
    X(OP, 64, 64, 2, 2, 128, 2)            \
    X(OP, 64, 64, 2, 2, 128, 4)            \
    X(OP, 64, 64, 2, 2, 256, 2)            \
    X(OP, 128, 32, 4, 1, 128, 3)           \
    X(OP, 32, 128, 1, 4, 128, 3)           \
    X(OP, 128, 64, 4, 2, 128, 3)           \
    X(OP, 64, 128, 2, 4, 128, 3)
#define QLL_PIPE_KG2_INSTANTIATE(OP, BP, BQ, WP, WQ, KS, ST)                                 \
    template __global__ void qll::gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KS, ST, false, false, 2>( \
        qll::GemmArgs);                                                                          \
    template __global__ void qll::gemm_pipe_kernel<OP, BP, BQ, WP, WQ, KS, ST, true, false, 2>(  \
        qll::GemmArgs);
#define QLL_PIPE_KG2_ENTRY(OP, BP, BQ, WP, WQ, KS, ST)                                 \
    {"p" #BP "x" #BQ "_w" #WP "x" #WQ "_k" #KS "_s" #ST "_g2", OP, 0, BP, BQ, WP, WQ, KS, \
     qll::pipe_lds_bytes<OP, BP, BQ, KS, ST, 2>(),                                        \
     &qll::launch_pipe<OP, BP, BQ, WP, WQ, KS, ST, 2>},
