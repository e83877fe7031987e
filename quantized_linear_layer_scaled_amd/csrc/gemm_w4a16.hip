// INT4 weight-only (W4A16) quantizer and GEMM for gfx950.
//
// The page "Helion in vLLM: A Unified Route to Tunable Linear Kernels" names
// INT4 among the formats vLLM serves (introduction) without defining it; the
// reading here is the symmetric per-group form of the FP8 rule:
//   weights: signed 4-bit codes q (two's complement nibbles, element 2j of a
//   row in bits 0-3 of byte j), one fp32 scale per output channel and
//   128-element K group, s = amax / 7, q = clamp(rne(w / s), -8, 7);
//   GEMM: out[m][n] = sum_g s[n][g] * sum_{k in g} a[m][k] * q[n][k] with
//   bf16 activations a; every group partial sum comes fresh from the matrix
//   cores (bf16 x small integer products are exact) and is promoted with one
//   fma, as Block-FP8 promotes its groups.
//
// Matrix core: v_mfma_f32_16x16x32_bf16 with the tokens on the row side (A
// operand) and the weights on the column side (B operand), so each lane's
// four accumulator values belong to one output channel and need one scale
// per group.  The nibbles become bf16 in registers (sign-extending bit-field
// extract, int -> fp32 convert, high halves packed by v_perm: exact for
// |q| <= 8).
//
// K order inside a group: lane l of a 16x16x32 step supplies 8 consecutive K
// slots (l >> 4) * 8 .. + 7 of its row.  A lane loads its weights once per
// group as one 16-byte run -- the 32 elements (l >> 4) * 32 .. + 31 -- and
// feeds elements (l >> 4) * 32 + 8 t .. + 7 in step t = 0..3; the activation
// fragments follow the same map, so every product still pairs a[m][k] with
// q[n][k] and the group sum is unchanged.
#include "gemm_pipe.h"

namespace qll {

namespace {

// ---------------------------------------------------------------- quantizer

// 16 lanes per 128-element group (8 bf16 each); the max by shuffles within
// the 16; codes by the correctly rounded fp32 quotient and rint (ties to
// even); a 4-byte code store per lane and one scale per group.
__global__ __launch_bounds__(256) void quant_int4_kernel(const uint4* __restrict__ w,
                                                        uint32_t* __restrict__ q,
                                                        float* __restrict__ s, long octets)
{
    const long stride = (long)gridDim.x * 256;
    for (long o = (long)blockIdx.x * 256 + threadIdx.x; o - (threadIdx.x & 15) < octets;
         o += stride) {
        const uint4 v = w[o];  // a group's 16 lanes are live together (octets % 16 == 0)
        const uint32_t x[4] = {v.x, v.y, v.z, v.w};
        float e[8];
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e[2 * i] = __uint_as_float(x[i] << 16);
            e[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
            m = fmaxf(m, fmaxf(fabsf(e[2 * i]), fabsf(e[2 * i + 1])));
        }
#pragma unroll
        for (int d = 1; d < 16; d <<= 1)
            m = fmaxf(m, __shfl_xor(m, d, 64));
        const float sc = m / 7.0f;
        uint32_t out = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r = sc == 0.0f ? 0.0f : __builtin_rintf(e[i] / sc);
            r = fminf(fmaxf(r, -8.0f), 7.0f);
            out |= ((uint32_t)(int)r & 15u) << (4 * i);
        }
        q[o] = out;
        if ((threadIdx.x & 15) == 0)
            s[o >> 4] = sc;
    }
}

// ---------------------------------------------------------------- helpers

// Eight 4-bit codes (bits 4e .. 4e+3 hold element e) -> eight bf16 values in
// MFMA operand order.
__device__ __forceinline__ uint4 int4x8_to_bf16(uint32_t d)
{
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // (the builtin's result type is unsigned: convert it as the signed
        // value the bit-field extract produced)
        const float lo = (float)(int)__builtin_amdgcn_sbfe((int)d, 8 * i, 4);
        const float hi = (float)(int)__builtin_amdgcn_sbfe((int)d, 8 * i + 4, 4);
        // bytes 2-3 of lo, then bytes 2-3 of hi (the bf16 halves, exact)
        w[i] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ v4f mfma_bf16(const uint4& a, const uint4& b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// The group range [g0, g1) of K piece z (kchunk is in weight bytes, 64 per
// group).
__device__ __forceinline__ void piece_groups(const GemmArgs& a, int z, int& g0, int& g1)
{
    const int G = a.K / 128;
    g0 = z * (a.kchunk / 64);
    g1 = min(G, g0 + a.kchunk / 64);
}

}  // namespace

// ---------------------------------------------------------------- decode

// HR (16 or 8) output channels per workgroup, 16 * RQ tokens; the W waves
// split the piece's groups into W contiguous runs, D groups of a run in
// flight at a time; the wave partials are added in wave order through LDS.
// With HR = 8 the MFMA's other 8 channel columns are zero: twice the
// workgroups, so that 2048 channels spread over all 256 CUs.
template <int RQ, int W, int HR, int D>
__global__ __launch_bounds__(W * 64) void gemm_w4_skinny_kernel(GemmArgs a)
{
    static_assert(HR == 16 || HR == 8, "channels per workgroup");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int N = a.N, M = a.M, K = a.K;
    const int G = K / 128;
    const int n0 = blockIdx.x * HR;
    const int m0 = blockIdx.y * (16 * RQ);
    const int z = blockIdx.z;
    const bool wcol = (lane & 15) < HR;  // this lane loads a channel's codes
    int pg0, pg1;
    piece_groups(a, z, pg0, pg1);
    const int TG = pg1 - pg0;
    const int g0 = pg0 + wave * TG / W, g1 = pg0 + (wave + 1) * TG / W;
    const int kq = lane >> 4;

    const int nrow = min(n0 + (lane & 15), N - 1);
    const uint8_t* __restrict__ bp = (const uint8_t*)a.B + (size_t)nrow * (K / 2) + kq * 16;
    const float* __restrict__ sp = a.sb + (size_t)nrow * G;
    const uint16_t* __restrict__ ap[RQ];
#pragma unroll
    for (int r = 0; r < RQ; ++r) {
        const int mrow = min(m0 + r * 16 + (lane & 15), M - 1);
        ap[r] = (const uint16_t*)a.A + (size_t)mrow * K + kq * 32;
    }

    v4f acc[RQ];
#pragma unroll
    for (int r = 0; r < RQ; ++r)
        acc[r] = v4f{0, 0, 0, 0};

    for (int g = g0; g < g1; g += D) {
        uint4 wb[D];
        float sc[D];
        uint4 xa[D][RQ][4];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const bool ok = g + d < g1;
            wb[d] = ok && wcol ? *(const uint4*)(bp + (size_t)(g + d) * 64)
                               : make_uint4(0, 0, 0, 0);
            sc[d] = ok && wcol ? sp[g + d] : 0.0f;
#pragma unroll
            for (int r = 0; r < RQ; ++r)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    xa[d][r][t] = ok ? *(const uint4*)(ap[r] + (size_t)(g + d) * 128 + t * 8)
                                     : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (g + d >= g1)
                continue;
            const uint32_t wd[4] = {wb[d].x, wb[d].y, wb[d].z, wb[d].w};
            v4f p[RQ];
#pragma unroll
            for (int r = 0; r < RQ; ++r)
                p[r] = v4f{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 bf = int4x8_to_bf16(wd[t]);
#pragma unroll
                for (int r = 0; r < RQ; ++r)
                    p[r] = mfma_bf16(xa[d][r][t], bf, p[r]);
            }
#pragma unroll
            for (int r = 0; r < RQ; ++r)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[r][v] = __builtin_fmaf(sc[d], p[r][v], acc[r][v]);
        }
    }

    // lane element (r, v): m = m0 + 16 r + 4 (lane >> 4) + v, n = n0 + (lane & 15)
    __shared__ float red[W][RQ * 256];
#pragma unroll
    for (int r = 0; r < RQ; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[wave][r * 256 + lane * 4 + v] = acc[r][v];
    __syncthreads();
    for (int e = threadIdx.x; e < RQ * 256; e += W * 64) {
        float sum = red[0][e];
#pragma unroll
        for (int w = 1; w < W; ++w)
            sum += red[w][e];
        const int r = e >> 8, ln = (e & 255) >> 2, v = e & 3;
        const int m = m0 + r * 16 + (ln >> 4) * 4 + v;
        const int n = n0 + (ln & 15);
        if (m < M && n < N && (ln & 15) < HR) {
            if (a.splits > 1)
                ((float*)a.ws)[((size_t)z * M + m) * N + n] = sum;
            else
                store_one<OP_W4A16>(a, (size_t)m * N + n, sum, m, n);
        }
    }
}

template <int RQ, int W, int HR, int D>
hipError_t launch_w4_skinny(const GemmArgs& a, hipStream_t stream)
{
    dim3 grid((a.N + HR - 1) / HR, (a.M + 16 * RQ - 1) / (16 * RQ), a.splits);
    if (grid.y > 65535 || grid.z > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_w4_skinny_kernel<RQ, W, HR, D>), grid, dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- tiles

// BP tokens x BQ channels per workgroup, WP x WQ waves; one 128-element
// group per stage: the activations (BP rows x 256 bytes) and the codes (BQ
// rows x 64 bytes) are staged in LDS (two buffers, XOR-swizzled 16-byte
// chunks), the next group's are loaded into registers while the current one
// is computed.
template <int BP, int BQ, int WP, int WQ>
__global__ __launch_bounds__(WP* WQ * 64) void gemm_w4_tile_kernel(GemmArgs a)
{
    constexpr int THREADS = WP * WQ * 64;
    constexpr int SP = BP / WP, SQ = BQ / WQ;
    constexpr int RP = SP / 16, RQ = SQ / 16;
    constexpr int ACH = BP * 16 / THREADS;  // 16-byte activation chunks per thread
    constexpr int BCH = (BQ * 4 + THREADS - 1) / THREADS;
    static_assert(BP * 16 % THREADS == 0, "activation chunks must split evenly");

    __shared__ __attribute__((aligned(16))) uint8_t As[2][BP * 256];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BQ * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wpi = wave % WP, wqi = wave / WP;
    const int M = a.M, N = a.N, K = a.K;
    const int G = K / 128;
    int tile_p, tile_q;
    xcd_tile(blockIdx.x, (M + BP - 1) / BP, (N + BQ - 1) / BQ, 4, tile_p, tile_q);
    const int p0 = tile_p * BP, q0 = tile_q * BQ;
    const int z = blockIdx.y;
    int g0, g1;
    piece_groups(a, z, g0, g1);
    const int kq = lane >> 4;

    const uint16_t* __restrict__ A = (const uint16_t*)a.A;
    const uint8_t* __restrict__ B = (const uint8_t*)a.B;

    uint4 ra[ACH], rb[BCH];
    float rs[RQ];
    auto fetch = [&](int g) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int c = i * THREADS + tid;
            const int row = c >> 4, ch = c & 15;
            const int m = p0 + row;
            ra[i] = m < M ? *(const uint4*)(A + (size_t)m * K + g * 128 + ch * 8)
                          : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = i * THREADS + tid;
            const int row = c >> 2, ch = c & 3;
            const int n = q0 + row;
            rb[i] = (c < BQ * 4 && n < N)
                        ? *(const uint4*)(B + (size_t)n * (K / 2) + g * 64 + ch * 16)
                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < RQ; ++j) {
            const int n = q0 + wqi * SQ + j * 16 + (lane & 15);
            rs[j] = n < N ? a.sb[(size_t)n * G + g] : 0.0f;
        }
    };
    auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int c = i * THREADS + tid;
            const int row = c >> 4, ch = c & 15;
            *(uint4*)(&As[buf][row * 256 + ((ch ^ swz<16>(row)) << 4)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = i * THREADS + tid;
            if (c < BQ * 4) {
                const int row = c >> 2, ch = c & 3;
                *(uint4*)(&Bs[buf][row * 64 + ((ch ^ swz<4>(row)) << 4)]) = rb[i];
            }
        }
    };

    v4f acc[RP][RQ];
#pragma unroll
    for (int i = 0; i < RP; ++i)
#pragma unroll
        for (int j = 0; j < RQ; ++j)
            acc[i][j] = v4f{0, 0, 0, 0};

    if (g0 < g1) {
        fetch(g0);
        stash(0);
        __syncthreads();
    }
    float sc[RQ];
    for (int g = g0; g < g1; ++g) {
        const int buf = (g - g0) & 1;
#pragma unroll
        for (int j = 0; j < RQ; ++j)
            sc[j] = rs[j];
        if (g + 1 < g1)
            fetch(g + 1);
        // this wave's codes of the group, one 16-byte run per lane and column block
        uint4 wq[RQ];
#pragma unroll
        for (int j = 0; j < RQ; ++j) {
            const int row = wqi * SQ + j * 16 + (lane & 15);
            wq[j] = *(const uint4*)(&Bs[buf][row * 64 + ((kq ^ swz<4>(row)) << 4)]);
        }
        v4f p[RP][RQ];
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int j = 0; j < RQ; ++j)
                p[i][j] = v4f{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint4 af[RP], bf[RQ];
#pragma unroll
            for (int i = 0; i < RP; ++i) {
                const int row = wpi * SP + i * 16 + (lane & 15);
                const int ch = kq * 4 + t;
                af[i] = *(const uint4*)(&As[buf][row * 256 + ((ch ^ swz<16>(row)) << 4)]);
            }
#pragma unroll
            for (int j = 0; j < RQ; ++j) {
                const uint32_t wd = t == 0 ? wq[j].x : t == 1 ? wq[j].y : t == 2 ? wq[j].z : wq[j].w;
                bf[j] = int4x8_to_bf16(wd);
            }
#pragma unroll
            for (int i = 0; i < RP; ++i)
#pragma unroll
                for (int j = 0; j < RQ; ++j)
                    p[i][j] = mfma_bf16(af[i], bf[j], p[i][j]);
        }
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int j = 0; j < RQ; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[i][j][v] = __builtin_fmaf(sc[j], p[i][j][v], acc[i][j][v]);
        if (g + 1 < g1) {
            stash(buf ^ 1);
            __syncthreads();
        }
    }

    // Epilogue through LDS (the activation buffers, free once every wave is
    // past its last group): each wave writes one 16-row block of its tile at
    // a time into a private scratch, then every lane emits 8 consecutive
    // columns of one row as one 16-byte store (two for fp32).  Lane element
    // (i, j, v) is row 16 i + 4 (lane >> 4) + v, column 16 j + (lane & 15)
    // of the wave's SP x SQ block.
    __syncthreads();
    static_assert(WP * WQ * 16 * SQ * 4 <= 2 * BP * 256, "epilogue scratch must fit");
    float* scr = (float*)&As[0][0] + wave * 16 * SQ;
    constexpr int CPR = SQ / 8;    // 8-column groups per row
    constexpr int RPP = 64 / CPR;  // rows per pass
    constexpr int PASSES = 16 / RPP;
    static_assert(SQ % 8 == 0 && 64 % CPR == 0 && 16 % RPP == 0, "epilogue lane map");
    const bool vec_ok = (N & 7) == 0;
    const int c = (lane % CPR) * 8;
    const int n = q0 + wqi * SQ + c;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
#pragma unroll
        for (int j = 0; j < RQ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                scr[((lane >> 4) * 4 + v) * SQ + j * 16 + (lane & 15)] = acc[i][j][v];
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            const int r = pass * RPP + lane / CPR;
            const int m = p0 + wpi * SP + i * 16 + r;
            float e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                e[t] = scr[r * SQ + c + t];
            if (m >= M)
                continue;
            if (a.splits > 1 || a.out_dtype != OUT_BF16) {
                float* dst = a.splits > 1 ? (float*)a.ws + ((size_t)z * M + m) * N + n
                                          : (float*)a.out + (size_t)m * N + n;
                if (vec_ok && n + 7 < N) {
                    const v4f lo{e[0], e[1], e[2], e[3]}, hi{e[4], e[5], e[6], e[7]};
                    if (a.splits > 1) {
                        *(v4f*)dst = lo;
                        *(v4f*)(dst + 4) = hi;
                    } else {
                        __builtin_nontemporal_store(lo, (v4f*)dst);
                        __builtin_nontemporal_store(hi, (v4f*)(dst + 4));
                    }
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = e[t];
                }
            } else {
                uint16_t* dst = (uint16_t*)a.out + (size_t)m * N + n;
                if (vec_ok && n + 7 < N) {
                    v4i w;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        w[t] = (int)((uint32_t)bf16_rne(e[2 * t]) |
                                     ((uint32_t)bf16_rne(e[2 * t + 1]) << 16));
                    __builtin_nontemporal_store(w, (v4i*)dst);
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = bf16_rne(e[t]);
                }
            }
        }
    }
}

template <int BP, int BQ, int WP, int WQ>
hipError_t launch_w4_tile(const GemmArgs& a, hipStream_t stream)
{
    const long tiles = (long)((a.M + BP - 1) / BP) * ((a.N + BQ - 1) / BQ);
    if (tiles > 0x7FFFFFFFL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_w4_tile_kernel<BP, BQ, WP, WQ>),
                       dim3((unsigned)tiles, (unsigned)a.splits), dim3(WP * WQ * 64), 0, stream,
                       a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- pipelined

// The copy pipeline of the 8-bit GEMMs (gemm_pipe.h) applied to W4A16: one
// 128-element group per stage.  The activations (BP rows x 256 bytes) and
// the codes (BQ rows x 64 bytes) go from global memory straight into a ring
// of S LDS slots with buffer_load_dwordx4 ... lds, the group's BQ weight
// scales with buffer_load_dword ... lds beside them; S - 1 groups are in
// flight ahead of the one computed, with one wait and one barrier per
// group.  As in gemm_pipe.h, the 16-byte chunks of a staged row are
// XOR-swizzled on the global side, and rows past M or N and offsets outside
// the operand read as zeros.  Per group each wave reads its code runs and
// scales once and the activation fragments of each step while the previous
// step's MFMAs run; the products are summed per group exactly as in the
// tiled kernel above (bitwise the same results).
template <int BP, int BQ>
constexpr int w4_pipe_stage_bytes()
{
    return BP * 256 + BQ * 64;
}

template <int BP, int BQ, int WP, int WQ, int S>
constexpr int w4_pipe_waves_per_eu()
{
    constexpr int lds = S * (w4_pipe_stage_bytes<BP, BQ>() + BQ * 4);
    constexpr int wgs = 163840 / lds < 4 ? 163840 / lds : 4;
    constexpr int w = wgs * WP * WQ / 4;
    return w < 1 ? 1 : (w > 8 ? 8 : w);
}

template <int BP, int BQ, int WP, int WQ, int S>
__global__ __launch_bounds__(WP* WQ * 64)
__attribute__((amdgpu_waves_per_eu(w4_pipe_waves_per_eu<BP, BQ, WP, WQ, S>())))
void gemm_w4_pipe_kernel(GemmArgs a)
{
    constexpr int WAVES = WP * WQ;
    constexpr int SP = BP / WP, SQ = BQ / WQ;
    constexpr int RP = SP / 16, RQ = SQ / 16;
    constexpr int AB = BP * 256, STAGE = w4_pipe_stage_bytes<BP, BQ>();
    constexpr int IA = AB / 1024, IB = BQ * 64 / 1024;  // copy instructions per stage
    constexpr int LPT0 = (IA + IB) / WAVES;
    constexpr int NSC = BQ / 64;                        // scale copy units per stage
    constexpr int LPS = (NSC + WAVES - 1) / WAVES;      // (units repeat: equal values)
    constexpr int LPT = LPT0 + LPS;
    static_assert(BP % 4 == 0 && BQ % 64 == 0 && (IA + IB) % WAVES == 0,
                  "a stage must split into whole copy instructions per wave");
    static_assert(S >= 2 && S <= 4 && (S - 1) * LPT < 64, "bad pipeline depth");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[S * STAGE];
    __shared__ __attribute__((aligned(16))) float lsc[S][BQ];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpi = wave % WP, wqi = wave / WP;
    const int M = a.M, N = a.N, K = a.K;
    const int G = K / 128;
    int tile_p, tile_q;
    xcd_tile(blockIdx.x, (M + BP - 1) / BP, (N + BQ - 1) / BQ, 4, tile_p, tile_q);
    const int p0 = tile_p * BP, q0 = tile_q * BQ;
    const int z = blockIdx.y;
    int g0, g1;
    piece_groups(a, z, g0, g1);
    const int nk = max(g1 - g0, 0);
    const int kq = lane >> 4;

    // the tile's activation rows, code rows and scale rows as buffers ending
    // at the last row of each matrix
    const uint32_t lda = (uint32_t)K * 2u, ldb = (uint32_t)K / 2u;
    const v4i rsA = buffer_rsrc((const uint16_t*)a.A + (size_t)p0 * K,
                                (uint32_t)min((uint64_t)(M - p0) * lda, (uint64_t)0x7FFFFFFF));
    const v4i rsB = buffer_rsrc((const uint8_t*)a.B + (size_t)q0 * ldb,
                                (uint32_t)min((uint64_t)(N - q0) * ldb, (uint64_t)0x7FFFFFFF));
    const v4i rsS = buffer_rsrc(a.sb + (size_t)q0 * G,
                                (uint32_t)min((uint64_t)(N - q0) * G * 4, (uint64_t)0x7FFFFFFF));

    // copy instruction i of this wave: stage instruction ii = i * WAVES + wave
    // (the first IA fill the activation part, the rest the code part); lane
    // chunk L = 64 (instruction within its part) + lane holds the logical
    // chunk (L mod NC) ^ swz(row) of row L / NC
    uint32_t voff[LPT0];
#pragma unroll
    for (int i = 0; i < LPT0; ++i) {
        const int ii = i * WAVES + wave;
        if (ii < IA) {
            const int L = ii * 64 + lane, row = L / 16, c = L % 16;
            voff[i] = (uint32_t)row * lda + (uint32_t)((c ^ swz<16>(row)) << 4);
        } else {
            const int L = (ii - IA) * 64 + lane, row = L / 4, c = L % 4;
            voff[i] = (uint32_t)row * ldb + (uint32_t)((c ^ swz<4>(row)) << 4);
        }
    }
    auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
        const int g = g0 + kt;
        uint8_t* buf = lds + slot * STAGE;
#pragma unroll
        for (int i = 0; i < LPT0; ++i) {
            const int ii = i * WAVES + wave;
            const bool pa = ii < IA;  // wave-uniform
            dma16(voff[i] + (uint32_t)g * (pa ? 256u : 64u), pa ? rsA : rsB,
                  __builtin_amdgcn_readfirstlane(
                      (uint32_t)(uintptr_t)(buf + (pa ? ii * 1024 : AB + (ii - IA) * 1024))));
        }
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const int u = (i * WAVES + wave) % NSC;
            dma4((uint32_t)((u * 64 + lane) * G + g) * 4u, rsS,
                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(&lsc[slot][u * 64])));
        }
    };

    v4f acc[RP][RQ];
#pragma unroll
    for (int i = 0; i < RP; ++i)
#pragma unroll
        for (int j = 0; j < RQ; ++j)
            acc[i][j] = v4f{0, 0, 0, 0};

    // one group from ring slot J: a fresh partial over its four MFMA steps,
    // promoted with the column's scale
    auto compute = [&](auto J) __attribute__((always_inline)) {
        constexpr int slot = decltype(J)::value;
        const uint8_t* sa = lds + slot * STAGE;
        const uint8_t* sb = sa + AB;
        uint4 wq[RQ];
        float sc[RQ];
#pragma unroll
        for (int j = 0; j < RQ; ++j) {
            const int row = wqi * SQ + j * 16 + (lane & 15);
            wq[j] = *(const uint4*)(sb + row * 64 + ((kq ^ swz<4>(row)) << 4));
            sc[j] = lsc[slot][row];
        }
        uint4 af[2][RP];
        auto read_a = [&](int t, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < RP; ++i) {
                const int row = wpi * SP + i * 16 + (lane & 15);
                const int ch = kq * 4 + t;
                dst[i] = *(const uint4*)(sa + row * 256 + ((ch ^ swz<16>(row)) << 4));
            }
        };
        v4f pp[RP][RQ];
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int j = 0; j < RQ; ++j)
                pp[i][j] = v4f{0, 0, 0, 0};
        read_a(0, af[0]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t + 1 < 4)
                read_a(t + 1, af[(t + 1) & 1]);
            uint4 bf[RQ];
#pragma unroll
            for (int j = 0; j < RQ; ++j) {
                const uint32_t wd = t == 0 ? wq[j].x : t == 1 ? wq[j].y : t == 2 ? wq[j].z : wq[j].w;
                bf[j] = int4x8_to_bf16(wd);
            }
#pragma unroll
            for (int i = 0; i < RP; ++i)
#pragma unroll
                for (int j = 0; j < RQ; ++j)
                    pp[i][j] = mfma_bf16(af[t & 1][i], bf[j], pp[i][j]);
        }
#pragma unroll
        for (int i = 0; i < RP; ++i)
#pragma unroll
            for (int j = 0; j < RQ; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[i][j][v] = __builtin_fmaf(sc[j], pp[i][j][v], acc[i][j][v]);
    };

    // prologue: groups 0 .. S-2 in flight; at group kt, once it has landed
    // for every wave and every wave is done with group kt - 1, that group's
    // slot takes group kt + S - 1
#pragma unroll
    for (int kt = 0; kt < S - 1; ++kt)
        if (kt < nk)
            issue(kt, kt);
    auto group = [&](auto J, int kt) __attribute__((always_inline)) {
        constexpr int slot = decltype(J)::value;
        const int younger = min(S - 2, nk - 1 - kt);  // later groups in flight
        if (S >= 4 && younger >= 2)
            wait_vm_barrier<(S >= 4 ? 2 : 0) * LPT>();
        else if (S >= 3 && younger >= 1)
            wait_vm_barrier<(S >= 3 ? 1 : 0) * LPT>();
        else
            wait_vm_barrier<0>();
        if (kt + S - 1 < nk)
            issue(kt + S - 1, (slot + S - 1) % S);
        compute(J);
    };
    for (int kt = 0; kt < nk; kt += S) {
        group(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < nk)
            group(std::integral_constant<int, 1>{}, kt + 1);
        if constexpr (S >= 3)
            if (kt + 2 < nk)
                group(std::integral_constant<int, (S >= 3 ? 2 : 0)>{}, kt + 2);
        if constexpr (S >= 4)
            if (kt + 3 < nk)
                group(std::integral_constant<int, (S >= 4 ? 3 : 0)>{}, kt + 3);
    }

    // Epilogue through LDS.  bf16 output: several 16-row blocks at a time,
    // rounded where the MFMA left them (store_bf16_batched); otherwise, as in
    // the tiled kernel, each wave writes one 16-row block of its tile at a
    // time into a private scratch, then every lane emits 8 consecutive
    // columns of one row.  Same values and rounding either way.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // slots are free
    if (a.splits == 1 && a.out_dtype == OUT_BF16 && (N & 7) == 0) {
        constexpr int BB = bf16_batch_blocks<RP, SQ>(S * STAGE / WAVES);
        constexpr int RBB = 16 * (SQ / 2 + 4) * 4;
        static_assert(S * STAGE / WAVES >= RBB, "epilogue scratch must fit");
        store_bf16_batched<RP, RQ, BB, false>(acc, (uint32_t*)(lds + wave * BB * RBB), nullptr,
                                              nullptr, lane, p0 + wpi * SP, q0 + wqi * SQ, M, N,
                                              (uint16_t*)a.out);
        return;
    }
    static_assert(WAVES * 16 * SQ * 4 <= S * STAGE, "epilogue scratch must fit");
    float* scr = (float*)lds + wave * 16 * SQ;
    constexpr int CPR = SQ / 8;
    constexpr int RPP = 64 / CPR;
    constexpr int PASSES = 16 / RPP;
    static_assert(SQ % 8 == 0 && 64 % CPR == 0 && 16 % RPP == 0, "epilogue lane map");
    const bool vec_ok = (N & 7) == 0;
    const int c = (lane % CPR) * 8;
    const int n = q0 + wqi * SQ + c;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
#pragma unroll
        for (int j = 0; j < RQ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                scr[((lane >> 4) * 4 + v) * SQ + j * 16 + (lane & 15)] = acc[i][j][v];
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            const int r = pass * RPP + lane / CPR;
            const int m = p0 + wpi * SP + i * 16 + r;
            float e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                e[t] = scr[r * SQ + c + t];
            if (m >= M)
                continue;
            if (a.splits > 1 || a.out_dtype != OUT_BF16) {
                float* dst = a.splits > 1 ? (float*)a.ws + ((size_t)z * M + m) * N + n
                                          : (float*)a.out + (size_t)m * N + n;
                if (vec_ok && n + 7 < N) {
                    const v4f lo{e[0], e[1], e[2], e[3]}, hi{e[4], e[5], e[6], e[7]};
                    if (a.splits > 1) {
                        *(v4f*)dst = lo;
                        *(v4f*)(dst + 4) = hi;
                    } else {
                        __builtin_nontemporal_store(lo, (v4f*)dst);
                        __builtin_nontemporal_store(hi, (v4f*)(dst + 4));
                    }
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = e[t];
                }
            } else {
                uint16_t* dst = (uint16_t*)a.out + (size_t)m * N + n;
                if (vec_ok && n + 7 < N) {
                    v4i w;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        w[t] = (int)((uint32_t)bf16_rne(e[2 * t]) |
                                     ((uint32_t)bf16_rne(e[2 * t + 1]) << 16));
                    __builtin_nontemporal_store(w, (v4i*)dst);
                } else {
                    for (int t = 0; t < 8; ++t)
                        if (n + t < N)
                            dst[t] = bf16_rne(e[t]);
                }
            }
        }
    }
}

template <int BP, int BQ, int WP, int WQ, int S>
hipError_t launch_w4_pipe(const GemmArgs& a, hipStream_t stream)
{
    const long tiles = (long)((a.M + BP - 1) / BP) * ((a.N + BQ - 1) / BQ);
    if (tiles > 0x7FFFFFFFL || (long)BP * a.K * 2 > 0x7FFFFFFFL ||
        (long)BQ * (a.K / 2) > 0x7FFFFFFFL || (long)BQ * (a.K / 128) * 4 > 0x7FFFFFFFL)
        return hipErrorInvalidValue;  // 32-bit buffer offsets within a tile
    hipLaunchKernelGGL((gemm_w4_pipe_kernel<BP, BQ, WP, WQ, S>),
                       dim3((unsigned)tiles, (unsigned)a.splits), dim3(WP * WQ * 64), 0, stream,
                       a);
    return hipGetLastError();
}

// the kernels the registry launches (needed by the device pass)
// X(RQ, TOKENS, W, D, HR) for every decode variant
#define QLL_FOR_EACH_W4_SKINNY(X) \
    X(1, 16, 8, 2, 16)            \
    X(1, 16, 4, 4, 16)            \
    X(2, 32, 8, 2, 16)            \
    X(4, 64, 8, 1, 16)            \
    X(1, 16, 16, 1, 16)           \
    X(1, 16, 8, 2, 8)             \
    X(1, 16, 16, 1, 8)            \
    X(2, 32, 8, 2, 8)
#define QLL_W4_SKINNY_INSTANTIATE(RQ, TOK, W, D, HR) \
    template __global__ void gemm_w4_skinny_kernel<RQ, W, HR, D>(GemmArgs);
QLL_FOR_EACH_W4_SKINNY(QLL_W4_SKINNY_INSTANTIATE)
template __global__ void gemm_w4_tile_kernel<64, 64, 2, 2>(GemmArgs);
template __global__ void gemm_w4_tile_kernel<128, 64, 2, 2>(GemmArgs);
template __global__ void gemm_w4_tile_kernel<64, 128, 2, 2>(GemmArgs);
template __global__ void gemm_w4_tile_kernel<128, 128, 2, 2>(GemmArgs);
template __global__ void gemm_w4_tile_kernel<256, 64, 4, 1>(GemmArgs);

// X(BP, BQ, WP, WQ, S) for every pipelined W4A16 variant
#define QLL_FOR_EACH_W4_PIPE(X) \
    X(64, 64, 2, 2, 2)          \
    X(64, 64, 2, 2, 3)          \
    X(128, 64, 2, 2, 2)         \
    X(128, 64, 2, 2, 3)         \
    X(128, 64, 2, 2, 4)         \
    X(64, 128, 2, 2, 3)         \
    X(128, 128, 2, 2, 3)        \
    X(128, 128, 2, 4, 3)        \
    X(256, 64, 4, 1, 2)         \
    X(256, 128, 4, 2, 2)        \
    X(64, 128, 2, 4, 2)         \
    X(64, 128, 2, 4, 3)         \
    X(128, 128, 4, 2, 3)        \
    X(128, 128, 1, 4, 3)        \
    X(128, 256, 2, 4, 2)        \
    X(128, 256, 2, 4, 3)        \
    X(128, 256, 1, 8, 3)        \
    X(64, 256, 1, 4, 3)         \
    X(64, 256, 1, 4, 4)         \
    X(32, 128, 1, 4, 3)         \
    X(32, 128, 1, 4, 4)         \
    X(32, 256, 1, 8, 3)         \
    X(64, 128, 1, 4, 3)
#define QLL_W4_PIPE_INSTANTIATE(BP, BQ, WP, WQ, S) \
    template __global__ void gemm_w4_pipe_kernel<BP, BQ, WP, WQ, S>(GemmArgs);
QLL_FOR_EACH_W4_PIPE(QLL_W4_PIPE_INSTANTIATE)


hipError_t launch_quant_int4(const void* w, void* q, float* s, int64_t elems,
                             hipStream_t stream)
{
    const long octets = (long)(elems / 8);
    long blocks = (octets + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;  // grid-stride beyond this
    hipLaunchKernelGGL(quant_int4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint4*)w, (uint32_t*)q, s, octets);
    return hipGetLastError();
}

hipError_t launch_reduce_w4a16(const GemmArgs& a, hipStream_t stream)
{
    return launch_reduce<OP_W4A16>(a, stream);
}

// Registry.  Decode: "k<channels>x<tokens>_w<waves>" (16 or 8 channels per
// workgroup, the waves split K); tiles: "t<BP>x<BQ>_w<WP>x<WQ>" (one group per stage,
// register prefetch) and "p<BP>x<BQ>_w<WP>x<WQ>_s<S>" (one group per stage,
// S-slot LDS copy ring).
#define QLL_W4_SKINNY(RQ, TOK, W, D, HR)                                             \
    {"k" #HR "x" #TOK "_w" #W, OP_W4A16, 1, HR, TOK, W, 1, 0, (W) * (RQ) * 1024,       \
     &launch_w4_skinny<RQ, W, HR, D>},
#define QLL_W4_TILE(BP, BQ, WP, WQ)                                                  \
    {"t" #BP "x" #BQ "_w" #WP "x" #WQ, OP_W4A16, 0, BP, BQ, WP, WQ, 64,               \
     2 * ((BP) * 256 + (BQ) * 64), &launch_w4_tile<BP, BQ, WP, WQ>},

#define QLL_W4_PIPE_ENTRY(BP, BQ, WP, WQ, S)                                          \
    {"p" #BP "x" #BQ "_w" #WP "x" #WQ "_s" #S, OP_W4A16, 0, BP, BQ, WP, WQ, 64,        \
     (S) * ((BP) * 256 + (BQ) * 68), &launch_w4_pipe<BP, BQ, WP, WQ, S>},

#if !defined(__HIP_DEVICE_COMPILE__)
extern const Variant kVariantsW4a16[] = {
    QLL_FOR_EACH_W4_SKINNY(QLL_W4_SKINNY)
    QLL_W4_TILE(64, 64, 2, 2)
    QLL_W4_TILE(128, 64, 2, 2)
    QLL_W4_TILE(64, 128, 2, 2)
    QLL_W4_TILE(128, 128, 2, 2)
    QLL_W4_TILE(256, 64, 4, 1)
    QLL_FOR_EACH_W4_PIPE(QLL_W4_PIPE_ENTRY)
};
extern const int kNumVariantsW4a16 = sizeof(kVariantsW4a16) / sizeof(Variant);
#endif

template __global__ void splitk_reduce_kernel<OP_W4A16>(GemmArgs);

}  // namespace qll
