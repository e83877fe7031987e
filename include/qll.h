/*
 * qll.h -- C ABI of libqll.so, the scaled_mm quantized linear-layer GEMM
 * library for AMD Instinct MI355X (gfx950).
 *
 * Operations (all described by the page "Helion in vLLM: A Unified Route to
 * Tunable Linear Kernels", section "What the integration changes", and by
 * vLLM PR #53446 "Hopper (SM90) tuned config for batch-invariant persistent
 * matmul", sections "Summary" and "Test Plan"):
 *   quantize_per_token_fp8      FP8 dynamic (per-token / per-1x128) quantization
 *   quantize_weight_block_fp8   128x128 Block-FP8 weight quantization (offline)
 *   gemm_w8a8_int8              W8A8 INT8 GEMM, per-token x per-channel scales
 *   gemm_fp8_scaled             FP8 GEMM, per-token x per-channel scales
 *   gemm_block_fp8              Block-FP8 GEMM (1x128 and 128x128 scales)
 *   gemm_bf16_batch_invariant   bf16 GEMM whose rows do not depend on M
 *   quantize_mxfp4, gemm_mxfp4  MXFP4 (4-bit E2M1, E8M0 scale per 32) quantizer
 *                               and GEMM, the block-scaled 4-bit format of the
 *                               CDNA4 matrix cores (see below)
 *   quantize_int4_weights,      INT4 weight-only: symmetric int4 weights with a
 *   gemm_w4a16                  scale per 128-element group, bf16 activations
 * Each GEMM runs as an ordinary tiled GEMM, as Split-K or as Swap-AB (the
 * three strategies of "What the integration changes"), chosen per (M, N, K)
 * by a dispatch table that an on-device sweep fills, or forced with the _ex
 * entry points.
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers, owned by the caller, dense and
 *     row-major: activations A [M][K], weights B [N][K] (the K x N operand
 *     stored column-major, as a linear layer keeps it), output [M][N].
 *     A, B, q, x and out must be 16-byte aligned; scales 4-byte aligned.
 *     Inputs and outputs must not overlap.
 *   - e4m3 is the OCP FP8 E4M3 format (e4m3fn: bias 7, max 448, no inf).
 *     Scales are fp32.  bf16 outputs are rounded to nearest even.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream: the library never allocates, frees or
 *     synchronizes on these paths, so calls can be captured into HIP graphs.
 *   - Arguments are validated before any HIP call; a launch failure reported
 *     by hipGetLastError maps to QLL_ERR_HIP.  Faults inside a kernel surface
 *     at the caller's next synchronization, as usual in HIP.  M == 0 is a
 *     valid no-op.  No C++ exception crosses this interface.
 *   - Split-K needs a caller-owned workspace of qll_workspace_bytes() bytes
 *     (16-byte aligned); a smaller one returns QLL_ERR_WORKSPACE.  Split-K
 *     partial sums are added in a fixed, ascending order by a second kernel
 *     (no atomics), so results are deterministic run to run.
 *   - After qll_init, calls are thread-safe; qll_init itself must not race
 *     with other calls.
 */
#ifndef QLL_H
#define QLL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QLL_OK = 0,
    QLL_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad dtype, bad cfg */
    QLL_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
    QLL_ERR_MISALIGNED = 3,  /* pointer alignment below the stated minimum */
    QLL_ERR_WORKSPACE = 4,   /* Split-K workspace missing or too small */
    QLL_ERR_NO_DEVICE = 5,   /* no usable gfx950 device */
    QLL_ERR_TABLE = 6,       /* dispatch table unreadable / for another device */
    QLL_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed */
} qll_status;

typedef enum {
    QLL_OUT_BF16 = 0,
    QLL_OUT_FP32 = 1,
    QLL_OUT_INT32 = 2 /* gemm_w8a8_int8 only: the raw int32 accumulators */
} qll_out;

typedef enum {
    QLL_OP_INT8 = 0,
    QLL_OP_FP8 = 1,
    QLL_OP_BLOCK_FP8 = 2,
    QLL_OP_BF16_BI = 3,
    QLL_OP_MXFP4 = 4,
    QLL_OP_W4A16 = 5,
    QLL_OP_FP8_DYNAMIC = 6 /* linear_fp8_dynamic: quantizer + FP8 GEMM, or fused */
} qll_op;

/* A GEMM configuration: which registered kernel variant (tile shape, wave
 * layout, ordinary or Swap-AB orientation) and how many K splits.  splits is
 * the requested Split-K factor; the K range is cut into contiguous chunks of
 * ceil(K_bytes / splits) rounded up to 512 bytes, so fewer splits may result
 * (qll_effective_splits). */
typedef struct {
    int32_t variant; /* index into the op's variant registry */
    int32_t splits;  /* >= 1 */
} qll_cfg;

/* ------------------------------------------------------------------ */
/* Quantizers                                                          */
/* ------------------------------------------------------------------ */

/* FP8 dynamic activation quantization ("FP8 dynamic quantization", page
 * "Helion in vLLM ...", section "What the integration changes").
 * For each row m and each group g of `group` consecutive columns:
 *   amax = max |x|;  s = amax / 448 (fp32);  q = e4m3_rne(clamp(x / s, +-448))
 * (x / s is a correctly rounded fp32 division; an all-zero group gives s = 0
 * and zero codes; the sign of a value that rounds to zero is kept).
 *   x      bf16 [M][K] (in)
 *   q      e4m3 [M][K] (out)
 *   scales fp32 [M][K/group] (out)
 *   group  0 or K: one scale per row (per token); 128: one per 1x128 group.
 *   K      multiple of 16 (of 128 for group 128).
 * Non-finite inputs give unspecified codes. */
int quantize_per_token_fp8(const void* x, void* q, float* scales, int64_t M,
                           int64_t K, int64_t group, void* stream);

/* Block-FP8 weight quantization, one scale per 128 x 128 block of the [N][K]
 * weight ("Block-FP8", same section), with the same rule as above applied to
 * each block.  w bf16 [N][K] (in); q e4m3 [N][K] (out);
 * scales fp32 [ceil(N/128)][K/128] (out).  K must be a multiple of 128; a
 * last partial block of rows is allowed.  Weight preparation, not the hot
 * path, but kept on the device like everything else. */
int quantize_weight_block_fp8(const void* w, void* q, float* scales, int64_t N,
                              int64_t K, void* stream);

/* ------------------------------------------------------------------ */
/* GEMMs                                                               */
/* ------------------------------------------------------------------ */

/* W8A8 INT8 ("W8A8 INT8", same section):
 *   acc[m][n] = sum_k A[m][k] * B[n][k]            (exact int32)
 *   out = bf16_rne((float(acc) * sa[m]) * sb[n])   (two fp32 multiplies)
 *   or the fp32 value (QLL_OUT_FP32) or acc itself (QLL_OUT_INT32).
 *   A int8 [M][K]; B int8 [N][K]; sa fp32 [M]; sb fp32 [N].
 *   K multiple of 16 and at most 131071 (int32 accumulators cannot overflow). */
int gemm_w8a8_int8(const void* A, const void* B, const float* sa,
                   const float* sb, void* out, int out_dtype, int64_t M,
                   int64_t N, int64_t K, void* ws, size_t ws_bytes,
                   void* stream);

/* FP8 with per-token x per-channel scales ("FP8 dynamic quantization"):
 *   out = bf16_rne((acc * sa[m]) * sb[n]), acc = sum_k A[m][k] * B[n][k]
 *   accumulated in fp32 on the matrix cores.
 *   A e4m3 [M][K] (e.g. from quantize_per_token_fp8); B e4m3 [N][K];
 *   sa fp32 [M]; sb fp32 [N]; out bf16 or fp32; K multiple of 16. */
int gemm_fp8_scaled(const void* A, const void* B, const float* sa,
                    const float* sb, void* out, int out_dtype, int64_t M,
                    int64_t N, int64_t K, void* ws, size_t ws_bytes,
                    void* stream);

/* Block-FP8 ("Block-FP8"): for each 128-wide K group g
 *   P_g = sum_{k in g} A[m][k] * B[n][k]  (fp32, matrix cores)
 *   acc += (sa[m][g] * sb[n/128][g]) * P_g
 *   out = bf16_rne(acc) (or fp32).
 *   A e4m3 [M][K]; B e4m3 [N][K]; sa fp32 [M][K/128]; sb fp32
 *   [ceil(N/128)][K/128]; K multiple of 128. */
int gemm_block_fp8(const void* A, const void* B, const float* sa,
                   const float* sb, void* out, int out_dtype, int64_t M,
                   int64_t N, int64_t K, void* ws, size_t ws_bytes,
                   void* stream);

/* Batch-invariant bf16 GEMM (vLLM PR #53446, "Summary" and "Test Plan"):
 *   out = bf16_rne(sum_k A[m][k] * B[n][k]) (or fp32), fp32 accumulation.
 * Row m of the output depends only on row m of A, on B and on (N, K): the
 * matrix-core instruction, the K order and the Split-K boundaries used are a
 * function of (N, K) alone, so row m is bitwise identical for every M.
 *   A bf16 [M][K]; B bf16 [N][K]; K multiple of 8. */
int gemm_bf16_batch_invariant(const void* A, const void* B, void* out,
                              int out_dtype, int64_t M, int64_t N, int64_t K,
                              void* ws, size_t ws_bytes, void* stream);

/* The four GEMMs above with a forced configuration (the sweep and the tests
 * use these; the MXFP4 and W4A16 GEMMs below have _ex forms too).  cfg == NULL behaves like the plain entry point.  For the
 * batch-invariant entry a forced cfg is the caller's responsibility: only
 * the table / heuristic choice is guaranteed M-independent. */
int gemm_w8a8_int8_ex(const void* A, const void* B, const float* sa,
                      const float* sb, void* out, int out_dtype, int64_t M,
                      int64_t N, int64_t K, void* ws, size_t ws_bytes,
                      void* stream, const qll_cfg* cfg);
int gemm_fp8_scaled_ex(const void* A, const void* B, const float* sa,
                       const float* sb, void* out, int out_dtype, int64_t M,
                       int64_t N, int64_t K, void* ws, size_t ws_bytes,
                       void* stream, const qll_cfg* cfg);
int gemm_block_fp8_ex(const void* A, const void* B, const float* sa,
                      const float* sb, void* out, int out_dtype, int64_t M,
                      int64_t N, int64_t K, void* ws, size_t ws_bytes,
                      void* stream, const qll_cfg* cfg);
int gemm_bf16_batch_invariant_ex(const void* A, const void* B, void* out,
                                 int out_dtype, int64_t M, int64_t N,
                                 int64_t K, void* ws, size_t ws_bytes,
                                 void* stream, const qll_cfg* cfg);

/* MXFP4.  The page "Helion in vLLM: A Unified Route to Tunable Linear
 * Kernels" names 4-bit formats (INT4, NVFP4) among those vLLM serves
 * (introduction) without defining them; MXFP4 is the block-scaled 4-bit
 * format gfx950's matrix cores read natively.  Encodings and conversion rule
 * follow the OCP Microscaling Formats (MX) v1.0 specification:
 *   E2M1 codes (sign bit 3, values 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte:
 *   element 2j of a row in bits 0-3 of byte j, element 2j+1 in bits 4-7;
 *   E8M0 scale bytes, value 2^(s - 127), one per 32 consecutive elements of
 *   a row (0xFF = NaN is never produced here).
 *
 * Quantizer, for each block of 32 elements of a row of bf16 x [M][K]:
 *   amax = max |x|;  E = floor(log2 amax) - 2 clamped to [-127, 127]
 *   (-127 for an all-zero block);  scale byte = E + 127;
 *   code = round-to-nearest-even of x / 2^E on the E2M1 values, saturating
 *   at 6, sign bit = sign of x (also when the magnitude rounds to zero).
 *   x bf16 [M][K] (16-byte aligned); q [M][K/2] bytes (4-byte aligned);
 *   scales [M][K/32] bytes.  K % 32 == 0.  Non-finite inputs give
 *   unspecified codes.  Used for activations (per call) and weights. */
int quantize_mxfp4(const void* x, void* q, void* scales, int64_t M, int64_t K,
                   void* stream);

/* MXFP4 GEMM:
 *   out[m][n] = sum_k a(m,k) * b(n,k),
 *   a(m,k) = e2m1(A[m][k]) * 2^(sa[m][k/32] - 127), b likewise with sb,
 *   accumulated in fp32 on the matrix cores (each 32-element block product
 *   is exact; the block scales are applied inside the instruction);
 *   out = bf16_rne (or fp32).
 *   A [M][K/2], B [N][K/2] packed codes (16-byte aligned); sa [M][K/32],
 *   sb [N][K/32] scale bytes (4-byte aligned); K % 128 == 0, K <= 2^23.
 *   ws as for the other GEMMs (Split-K, qll_workspace_bytes(QLL_OP_MXFP4,...)).
 * gemm_mxfp4_ex forces a configuration like the other _ex entry points. */
int gemm_mxfp4(const void* A, const void* B, const void* sa, const void* sb,
               void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
               void* ws, size_t ws_bytes, void* stream);
int gemm_mxfp4_ex(const void* A, const void* B, const void* sa, const void* sb,
                  void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                  void* ws, size_t ws_bytes, void* stream, const qll_cfg* cfg);

/* INT4 weight-only (W4A16).  The same page names INT4 among vLLM's formats
 * without defining it; the reading is the symmetric per-group form of the
 * FP8 rule:
 *   weights: for each output channel n and group g of 128 consecutive K
 *   elements, amax = max |w|, s[n][g] = amax / 7 (fp32), q = clamp(
 *   rne(w / s), -8, 7) with the correctly rounded fp32 quotient (an all-zero
 *   group: s = 0, zero codes); codes are 4-bit two's complement nibbles,
 *   element 2j of a row in bits 0-3 of byte j, element 2j+1 in bits 4-7.
 *     w bf16 [N][K] (16-byte aligned); q [N][K/2] bytes (4-byte aligned);
 *     scales fp32 [N][K/128]; K % 128 == 0.  Weight preparation (offline).
 *   GEMM: out[m][n] = sum_g s[n][g] * P_g,  P_g = sum_{k in g} A[m][k] q[n][k]
 *   with each P_g a fresh fp32 matrix-core sum (bf16 x int4 products are
 *   exact) promoted by one fma per group; out bf16_rne (or fp32).
 *     A bf16 [M][K]; B packed int4 [N][K/2]; scales fp32 [N][K/128];
 *     K % 128 == 0; ws as for the other GEMMs (Split-K pieces are whole
 *     multiples of 8 groups: qll_workspace_bytes(QLL_OP_W4A16, ...)). */
int quantize_int4_weights(const void* w, void* q, float* scales, int64_t N,
                          int64_t K, void* stream);
int gemm_w4a16(const void* A, const void* B, const float* scales, void* out,
               int out_dtype, int64_t M, int64_t N, int64_t K, void* ws,
               size_t ws_bytes, void* stream);
int gemm_w4a16_ex(const void* A, const void* B, const float* scales, void* out,
                  int out_dtype, int64_t M, int64_t N, int64_t K, void* ws,
                  size_t ws_bytes, void* stream, const qll_cfg* cfg);

/* FP8 dynamic linear layer in one call ("FP8 dynamic quantization", same
 * section): per-token quantization of x (q, sa) and the scaled FP8 GEMM
 * (q, B, sa, sb -> out), in one of two forms, chosen per shape by the
 * dispatch under the op QLL_OP_FP8_DYNAMIC (or by cfg):
 *   - two launches: quantize_per_token_fp8 then gemm_fp8_scaled with an FP8
 *     GEMM variant (the first qll_num_variants(QLL_OP_FP8) indices, the same
 *     as the FP8 op's; without a table entry of its own the op takes the
 *     FP8 GEMM's choice);
 *   - fused (the indices after them, names "f<rows>x<tokens>_w<W>_d<steps>"):
 *     one launch whose workgroups quantize the tokens themselves inside the
 *     wave-split decode GEMM; M <= tokens (1, 2, 4, 8 or 16; the forms
 *     below 16 encode only that many tokens' values per wave) and K within
 *     the variant's register chunk (d steps of 128 per wave: K <= 2048 for
 *     d2, <= 6144 for d6),
 *     else QLL_ERR_UNSUPPORTED; no workspace.  Its output is bitwise that of
 *     the two launches with the W-wave decode GEMM of the same rows per
 *     workgroup ("k16x16_w8" for f16..._w8, "k8x16_w16" for f8..._w16).
 * Codes and scales are bitwise those of quantize_per_token_fp8 in both forms.
 *   x bf16 [M][K] (in); B e4m3 [N][K]; sb fp32 [N];
 *   q e4m3 [M][K] and sa fp32 [M] (out, required: the quantized activations);
 *   out bf16 / fp32 [M][N]; ws as for gemm_fp8_scaled (Split-K;
 *   qll_workspace_bytes(QLL_OP_FP8_DYNAMIC, ...)).
 * Errors: those of the two calls; nothing is launched on an invalid argument. */
int linear_fp8_dynamic(const void* x, const void* B, const float* sb, void* q,
                       float* sa, void* out, int out_dtype, int64_t M, int64_t N,
                       int64_t K, void* ws, size_t ws_bytes, void* stream);
int linear_fp8_dynamic_ex(const void* x, const void* B, const float* sb, void* q,
                          float* sa, void* out, int out_dtype, int64_t M, int64_t N,
                          int64_t K, void* ws, size_t ws_bytes, void* stream,
                          const qll_cfg* cfg);

/* Grouped (per-expert) FP8 GEMM, the expert layer of an FP8 mixture of
 * experts built from the same scaled FP8 GEMM ("FP8 dynamic quantization"
 * of "Helion in vLLM: A Unified Route to Tunable Linear Kernels", "What the
 * integration changes"; the FP8 MoE pipeline of the Hunyuan MoE backend
 * pages).  The M rows of A are sorted by expert: rows
 * [offsets[e], offsets[e+1]) go to expert e, whose weights are B + e*N*K
 * and whose per-channel scales are sb + e*N:
 *   out[m][n] = bf16_rne((acc * sa[m]) * sb[e][n]),
 *   acc = sum_k e4m3(A[m][k]) * e4m3(B[e][n][k]) in fp32.
 *   A e4m3 [M][K]; B e4m3 [E][N][K]; sa fp32 [M]; sb fp32 [E][N];
 *   offsets: DEVICE int32 [E + 1], offsets[0] = 0, offsets[E] = M,
 *   non-decreasing.  Other values are read as their running maximum clamped
 *   to [0, M] (expert e then owns rows [c[e], c[e+1]) of those values, rows
 *   that no expert owns are left unwritten), so no access leaves A, B, sa,
 *   sb or out;
 *   out bf16 / fp32 [M][N].  K % 16 == 0, 1 <= E <= 65536.  No workspace.
 * variant (the _ex form): one of the pipelined variant names
 * ("p<BP>x<BQ>_w<WP>x<WQ>_k128_s<S>", as listed by qll_variant_info for the
 * FP8 op), or NULL for the built-in rule.  M == 0 is a no-op.
 * Errors: INVALID_ARG (shapes, pointers, unknown variant), MISALIGNED,
 * UNSUPPORTED (K too long for the variant), HIP. */
int gemm_fp8_grouped(const void* A, const void* B, const float* sa, const float* sb,
                     const int32_t* offsets, void* out, int out_dtype, int64_t M,
                     int64_t N, int64_t K, int64_t E, void* stream);
int gemm_fp8_grouped_ex(const void* A, const void* B, const float* sa, const float* sb,
                        const int32_t* offsets, void* out, int out_dtype, int64_t M,
                        int64_t N, int64_t K, int64_t E, void* stream,
                        const char* variant);
/* The variant gemm_fp8_grouped picks for M rows over E experts, written as
 * a NUL-terminated name into buf (cap bytes).  INVALID_ARG on bad arguments
 * or a too small buffer. */
int qll_grouped_select(int64_t M, int64_t E, char* buf, size_t cap);

/* ------------------------------------------------------------------ */
/* Without device allocation                                           */
/* ------------------------------------------------------------------ */

/* Bytes of the static device array gemm_fp8_scaled_noalloc keeps its Split-K
 * partial sums in (one array per GPU, held until the process ends). */
#define QLL_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)

/* gemm_fp8_scaled for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments without the workspace; the configuration, the kernels and
 * the output are those of gemm_fp8_scaled for the same shape (bitwise).  When
 * the configuration splits K, the partial sums go to a static device array of
 * QLL_NOALLOC_SCRATCH_BYTES per GPU instead of a caller workspace; a shape
 * whose partials (splits x M x N x 4 bytes) exceed it returns
 * QLL_ERR_WORKSPACE before anything is enqueued.  Nothing is allocated or
 * freed; the array's address on a device is looked up at qll_init (for the
 * device current then) or at the first call on that device.  Every call on
 * one GPU uses the same array: calls that overlap on one GPU (different
 * streams or threads) race and must be serialized by the caller; the array
 * needs no clearing between calls (every partial is written before it is
 * read). */
int gemm_fp8_scaled_noalloc(const void* A_e4m3, const void* B_e4m3, const float* sa,
                            const float* sb, void* out, int out_dtype, int64_t M, int64_t N,
                            int64_t K, void* stream);

/* ------------------------------------------------------------------ */
/* Dispatch, registry and support                                      */
/* ------------------------------------------------------------------ */

/* Load the dispatch table (per-shape tuning, "What the integration changes").
 * table_path NULL: $QLL_TABLE if set, else no table (built-in heuristic).
 * A table is keyed by device, as the review of vLLM PR #53446 keys its
 * configs by device name after a table tuned on one H100 variant regressed
 * another: its one device line ("device <arch> <CUs> <MHz> <name>") must
 * match the current device's signature (see qll_device_signature) in gfx
 * arch, CU count and peak engine clock -- MI350X and MI355X are both gfx950
 * with 256 CUs and differ in clock -- and in device name when the table and
 * the runtime both give one (the runtime reports an empty name in some
 * environments, e.g. under the rocprofv3 tracer), else QLL_ERR_TABLE is
 * returned and the heuristic stays in force.  A batch-invariant section whose
 * effective Split-K factor varies with M for one (N, K) is rejected the same
 * way (tile shape and orientation may vary: every batch-invariant variant sums
 * K in the same fixed chunks, so they agree bit for bit).  Loading a table
 * equal to one loaded before reuses it.  Without a device the call returns
 * QLL_ERR_NO_DEVICE. */
int qll_init(const char* table_path);

/* Parse and check a dispatch table against a device signature (gfx arch name,
 * CU count, peak engine clock in MHz, device name) without installing it; no
 * device needed.  Returns QLL_OK or QLL_ERR_TABLE with a reason in err
 * (NUL-terminated, truncated to cap); INVALID_ARG for null arguments. */
int qll_table_validate(const char* path, const char* arch, int cus, int mhz,
                       const char* name, char* err, size_t cap);

/* The current device's signature as a table's device line holds it after the
 * keyword: "<arch> <CUs> <MHz> <name>" (NUL-terminated into buf, cap bytes;
 * the name may be empty).
 * QLL_ERR_NO_DEVICE without a gfx950 device, INVALID_ARG for a null or too
 * small buffer. */
int qll_device_signature(char* buf, size_t cap);

/* The configuration the entry point would use for this shape (table entry if
 * one exists, else the heuristic). */
int qll_select(int op, int64_t M, int64_t N, int64_t K, qll_cfg* cfg_out);

/* Workspace bytes the op needs for this shape: with cfg == NULL for the
 * configuration qll_select picks, else for cfg.  Returns 0 when no Split-K is
 * involved, a negative value (-status) for invalid arguments. */
int64_t qll_workspace_bytes(int op, int64_t M, int64_t N, int64_t K,
                            const qll_cfg* cfg);

/* Number of K splits actually used for (op, K, cfg->splits). */
int qll_effective_splits(int op, int64_t K, int32_t splits);

/* Registered kernel variants of an op.  qll_variant_info writes a one-line
 * JSON description (name, orientation, tile, waves, K stage, LDS bytes) into
 * buf (NUL-terminated, truncated to cap) and returns QLL_OK.
 * Names, as the _ex forms take them:
 *   k<rows>x<tokens>_w<W>        decode kernel, Swap-AB, its W waves split K
 *   r<rows>x<tokens>_w<W>        decode kernel, its waves split the rows
 *   n|s<BP>x<BQ>_w<WP>x<WQ>_k<KS>  register-prefetch tile, ordinary | Swap-AB
 *   p<BP>x<BQ>_w<WP>x<WQ>_k<KS>_s<S>  tile fed by an S-slot LDS copy ring of
 *                                KS-byte K stages; a "_g2" suffix: two such
 *                                wave groups split K inside the workgroup
 *   f<rows>x<T>_w<W>_d<D>        fused quantizer + decode GEMM for M <= T
 *                                (fp8_dynamic)
 *   p<BP>x<BQ>_w<WP>x<WQ>_k<KS>_r<R>  tile whose operand copies go through
 *                                R register stages into a two-slot LDS ring
 *   t<BP>x<BQ>_w<WP>x<WQ>        W4A16 register-staged tile
 * The W4A16 tiles omit _k (one 128-element group per stage); FP8 tiles with
 * _k64 run on the 32x32x64 matrix-core step. */
int qll_num_variants(int op);
int qll_variant_info(int op, int idx, char* buf, size_t cap);
int qll_variant_index(int op, const char* name);

/* Number of table entries in force (0 = heuristic only). */
int qll_table_entries(void);

const char* qll_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLL_H */
