// The registered tile shapes, shared by the four GEMM ops.  KS8 is the K
// stage (bytes) for the smaller variants, KSL for the larger ones; each op's
// translation unit picks values that are multiples of its MFMA K step.
//
//   Swap-AB (weights on the MFMA row side, tokens on the column side):
//     small M (1..64) with 16..64 tokens per tile.
//   Ordinary (tokens on the row side): 16..256 tokens per tile.
//
// X(OP, SWAP, BP, BQ, WP, WQ, KSTAGE) is applied to every entry.
#define QLL_FOR_EACH_VARIANT(X, OP, KS8, KSL) \
    X(OP, 1, 64, 16, 4, 1, KS8)               \
    X(OP, 1, 128, 16, 4, 1, KS8)              \
    X(OP, 1, 256, 16, 4, 1, KSL)              \
    X(OP, 1, 128, 32, 4, 1, KSL)              \
    X(OP, 1, 128, 64, 2, 2, KSL)              \
    X(OP, 0, 16, 64, 1, 4, KS8)               \
    X(OP, 0, 32, 128, 1, 4, KSL)              \
    X(OP, 0, 64, 128, 2, 2, KSL)              \
    X(OP, 0, 128, 128, 2, 2, KSL)             \
    X(OP, 0, 128, 256, 2, 2, KSL)             \
    X(OP, 0, 256, 128, 2, 2, KSL)

// explicit kernel instantiation (needed by the device pass)
#define QLL_INSTANTIATE(OP, SW, BP, BQ, WP, WQ, KS) \
    template __global__ void qll::gemm_tile_kernel<OP, SW, BP, BQ, WP, WQ, KS>(qll::GemmArgs);

// registry entry (host pass)
#define QLL_ENTRY(OP, SW, BP, BQ, WP, WQ, KS) QLL_VARIANT(OP, SW, BP, BQ, WP, WQ, KS),
