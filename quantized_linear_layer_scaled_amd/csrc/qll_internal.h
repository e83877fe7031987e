// Internal declarations shared by the host API and the kernel translation
// units of libqll.so.  Not part of the public interface (see include/qll.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qll {

enum Op : int {
    OP_INT8 = 0,
    OP_FP8 = 1,
    OP_BLOCK = 2,
    OP_BF16 = 3,
    OP_MXFP4 = 4,
    OP_W4A16 = 5,
    // the FP8 dynamic linear layer (quantizer + FP8 GEMM): its variants are
    // the FP8 GEMM's (two launches) followed by the fused ones
    OP_FP8_DYN = 6,
    OP_COUNT = 7
};
enum Out : int { OUT_BF16 = 0, OUT_FP32 = 1, OUT_INT32 = 2 };

// The K range of one Split-K piece is a multiple of this many bytes, for every
// variant, so that the split boundaries depend only on (K, splits).
constexpr int kSplitGranule = 512;
constexpr int kMaxSplits = 64;

// Everything a GEMM launch needs.  P/Q naming: the matrix-core "A" operand
// supplies the rows (P) of each 16x16 output block and the "B" operand its
// columns (Q).  In the ordinary orientation P = tokens (A, M rows) and
// Q = weights (B, N rows); Swap-AB exchanges the two.
struct GemmArgs {
    const void* A;   // [M][K]
    const void* B;   // [N][K]
    const float* sa; // per-token [M] or per-group [M][K/128]
    const float* sb; // per-channel [N] or per-block [ceil(N/128)][K/128]
                     // (MXFP4: E8M0 bytes [M][K/32] and [N][K/32];
                     // W4A16: sb fp32 [N][K/128], sa unused)
    void* out;       // [M][N]
    void* ws;        // [splits][M][N] int32 / fp32 partials (splits > 1)
    int out_dtype;
    int M, N, K;     // K in elements
    int kbytes;      // bytes of one row of A or B (K / 2 for packed MXFP4;
                     // W4A16: of B, the packed int4 weights)
    int splits;      // effective number of K pieces
    int kchunk;      // bytes of K per piece (multiple of kSplitGranule)
    int kfold;       // bf16 only: K chunks summed separately, then in order
    // grouped (per-expert) GEMM only: A rows [offsets[e], offsets[e+1]) use
    // weights B + e * N * K and scales sb + e * N (device int32 [E + 1])
    const int* offsets;
    int E;
};

// The batch-invariant bf16 op sums every K piece as kBiFold contiguous chunks
// on a grid of kFoldUnit-byte units (with TU units in the piece, chunk w holds
// units [w*TU/kBiFold, (w+1)*TU/kBiFold)), each from zero, and adds the chunk
// sums in ascending order.  Every bf16 kernel reproduces that order, so all
// of them agree bit for bit.  The skinny kernels' waves split K on the same
// grid for every op.
constexpr int kBiFold = 8;
constexpr int kFoldUnit = 256;

using LaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t);

struct Variant {
    const char* name;
    int op;
    int swap;    // 0 ordinary, 1 Swap-AB
    int bp, bq;  // tile rows along P and Q
    int wp, wq;  // wave grid
    int kstage;  // bytes of K staged per iteration
    int lds;     // LDS bytes
    LaunchFn launch;       // the tile kernel (writes out, or ws when splits > 1)
};

// Registries, one per op (defined in the kernel translation units).
const Variant* variants(int op, int* count);
// Grouped FP8 GEMM: the pipelined variants launched over experts.
const Variant* grouped_variants(int* count);

// Second Split-K stage: out = epilogue(sum_{s ascending} ws[s]).
hipError_t launch_splitk_reduce(int op, const GemmArgs& a, hipStream_t stream);

// The fused FP8 dynamic linear layer for few tokens (linear_fused.hip):
// per-token quantization inside the wave-split decode GEMM.
struct FusedArgs {
    const uint16_t* x;  // bf16 [M][K]
    const uint8_t* B;   // e4m3 [N][K]
    const float* sb;    // [N]
    uint8_t* q;         // e4m3 [M][K] (written by workgroup 0)
    float* sa;          // [M] (written by workgroup 0)
    void* out;          // [M][N]
    int out_dtype;
    int M, N, K;        // M <= the variant's tokens (<= 16)
};
struct FusedVariant {
    const char* name;
    int hr;  // weight rows per workgroup
    int w;   // waves splitting K
    int d;   // K steps of 128 a wave holds in registers
    int tok; // most tokens (M) it takes: 1, 2, 4, 8 or 16
    hipError_t (*launch)(const FusedArgs&, hipStream_t);
};
extern const FusedVariant kFusedVariants[];
extern const int kNumFusedVariants;
// K steps the busiest of W waves of a fused workgroup handles (<= d to fit)
int fused_steps_per_wave(int K, int W);

// Looks up, for the current device, the address of the static scratch array
// of gemm_fp8_scaled_noalloc (once per device).
hipError_t noalloc_setup();

// Quantizers.
hipError_t launch_quant_rows(const void* x, void* q, float* s, int M, int K,
                             hipStream_t stream);
hipError_t launch_quant_groups128(const void* x, void* q, float* s, int M,
                                  int K, hipStream_t stream);
hipError_t launch_quant_weight_blocks(const void* w, void* q, float* s, int N,
                                      int K, hipStream_t stream);
hipError_t launch_quant_mxfp4(const void* x, void* q, void* s, int64_t elems,
                              hipStream_t stream);
hipError_t launch_quant_int4(const void* w, void* q, float* s, int64_t elems,
                             hipStream_t stream);

}  // namespace qll
