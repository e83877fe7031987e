// C ABI of libqll.so: argument validation, the per-shape dispatch table with
// its heuristic fallback, and the launches.  Declarations and the contract of
// every entry point are in include/qll.h.
//
// Dispatch follows "Helion in vLLM: A Unified Route to Tunable Linear
// Kernels", section "What the integration changes": the algorithm (ordinary,
// Split-K, Swap-AB) is chosen per shape together with its tile configuration,
// from a table an offline on-device search fills, with a fixed rule for the
// shapes the table does not cover.  As in vLLM PR #53446 (the per-device
// configuration keys of its review), a table is used only on the device it
// was measured on.  The lookup happens on the host in O(1), with no
// allocation, no synchronization and no HIP call before the launch.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/qll.h"
#include "qll_internal.h"

namespace qll {

extern const Variant kVariantsInt8[];
extern const int kNumVariantsInt8;
extern const Variant kVariantsFp8[];
extern const int kNumVariantsFp8;
extern const Variant kVariantsFp8Grouped[];
extern const int kNumVariantsFp8Grouped;
extern const Variant kVariantsBlock[];
extern const int kNumVariantsBlock;
extern const Variant kVariantsBf16[];
extern const int kNumVariantsBf16;
extern const Variant kVariantsMxfp4[];
extern const int kNumVariantsMxfp4;
extern const Variant kVariantsW4a16[];
extern const int kNumVariantsW4a16;
hipError_t launch_reduce_int8(const GemmArgs&, hipStream_t);
hipError_t launch_reduce_fp8(const GemmArgs&, hipStream_t);
hipError_t launch_reduce_block(const GemmArgs&, hipStream_t);
hipError_t launch_reduce_bf16(const GemmArgs&, hipStream_t);
hipError_t launch_reduce_mxfp4(const GemmArgs&, hipStream_t);
hipError_t launch_reduce_w4a16(const GemmArgs&, hipStream_t);

// (for OP_FP8_DYN: its GEMM variants, i.e. the FP8 ones; the fused variants
// follow them in that op's index space, see dyn_count)
const Variant* variants(int op, int* count)
{
    switch (op) {
    case OP_INT8: *count = kNumVariantsInt8; return kVariantsInt8;
    case OP_FP8:
    case OP_FP8_DYN: *count = kNumVariantsFp8; return kVariantsFp8;
    case OP_BLOCK: *count = kNumVariantsBlock; return kVariantsBlock;
    case OP_BF16: *count = kNumVariantsBf16; return kVariantsBf16;
    case OP_MXFP4: *count = kNumVariantsMxfp4; return kVariantsMxfp4;
    case OP_W4A16: *count = kNumVariantsW4a16; return kVariantsW4a16;
    default: *count = 0; return nullptr;
    }
}

const Variant* grouped_variants(int* count)
{
    *count = kNumVariantsFp8Grouped;
    return kVariantsFp8Grouped;
}

hipError_t launch_splitk_reduce(int op, const GemmArgs& a, hipStream_t stream)
{
    switch (op) {
    case OP_INT8: return launch_reduce_int8(a, stream);
    case OP_FP8: return launch_reduce_fp8(a, stream);
    case OP_BLOCK: return launch_reduce_block(a, stream);
    case OP_MXFP4: return launch_reduce_mxfp4(a, stream);
    case OP_W4A16: return launch_reduce_w4a16(a, stream);
    default: return launch_reduce_bf16(a, stream);
    }
}

namespace {

const char* const kOpNames[OP_COUNT] = {"int8", "fp8", "block_fp8", "bf16_bi", "mxfp4",
                                         "w4a16", "fp8_dynamic"};

// The FP8 dynamic linear layer's variant index space: the FP8 GEMM variants
// (quantizer + GEMM, two launches) and then the fused variants.
int dyn_count() { return kNumVariantsFp8 + kNumFusedVariants; }
const FusedVariant* dyn_fused(int idx)
{
    return idx >= kNumVariantsFp8 && idx < dyn_count() ? &kFusedVariants[idx - kNumVariantsFp8]
                                                       : nullptr;
}
// a fused variant runs M up to its tokens (at most 16) and K up to its
// register chunk
bool fused_fits(const FusedVariant& f, int64_t M, int64_t K)
{
    return M <= f.tok && K <= 0x3FFFFFFF && fused_steps_per_wave((int)K, f.w) <= f.d &&
           2 * M * K <= 0x7FFFFFF0 && f.hr * K <= 0x7FFFFFF0;
}

// Bytes of one K-row of A or B: bf16 2 per element, packed MXFP4 one per two;
// W4A16 counts the packed weight row (its Split-K pieces are cut on those
// bytes, 512 of them = 8 groups of 128).
int64_t op_kbytes(int op, int64_t K)
{
    return op == OP_BF16 ? 2 * K : (op == OP_MXFP4 || op == OP_W4A16 ? K / 2 : K);
}

// Longest MXFP4 K: every pipelined variant's tile rows times the row bytes
// stay below 2^31 (there is no tiled fallback for this op).
constexpr int64_t kMaxKMxfp4 = (int64_t)1 << 23;

// The pipelined kernels address a tile's rows with 32-bit buffer offsets:
// for each operand, its tile rows times the bytes of one of its rows must stay
// below 2^31 (A rows of W4A16 are bf16, 2K bytes; its B rows are K/2 bytes of
// codes beside K/128 fp32 group scales).
bool variant_fits(int op, const Variant& v, int64_t K)
{
    if (v.name[0] != 'p')
        return true;
    const int64_t lim = 0x7FFFFFFF;
    if (op == OP_W4A16)
        return (int64_t)v.bp * 2 * K <= lim && (int64_t)v.bq * (K / 2) <= lim &&
               (int64_t)v.bq * (K / 128) * 4 <= lim;
    const int64_t kbytes = op_kbytes(op, K);
    return (int64_t)v.bp * kbytes <= lim && (int64_t)v.bq * kbytes <= lim;
}

// ------------------------------------------------------------------ device
// What a table is keyed by: gfx arch, compute units, peak engine clock and
// the runtime's device name.  Two parts of one arch and CU count can still
// differ in clock and power (MI350X and MI355X are both gfx950 with 256 CUs;
// MI355X runs at up to 2400 MHz), and a table tuned on one can lose on the
// other -- the cross-SKU regression that the review of vLLM PR #53446
// reports for an H100 NVL table on H100 SXM, and why its configs are keyed
// by device name.
struct DeviceSig {
    char arch[64] = {0};
    int cus = 0;
    int mhz = 0;
    char name[256] = {0};
};

struct DeviceInfo {
    bool ok = false;
    int cus = 256;
    DeviceSig sig;
};

DeviceInfo& device_info()
{
    static DeviceInfo info;
    static std::once_flag once;
    std::call_once(once, [] {
        int n = 0;
        if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            return;
        }
        int dev = 0;
        hipDeviceProp_t p;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipGetDeviceProperties(&p, dev) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        info.cus = p.multiProcessorCount;
        DeviceSig& g = info.sig;
        std::snprintf(g.arch, sizeof g.arch, "%s", p.gcnArchName);
        char* colon = std::strchr(g.arch, ':');
        if (colon)
            *colon = 0;
        g.cus = p.multiProcessorCount;
        g.mhz = p.clockRate / 1000;  // kHz
        std::snprintf(g.name, sizeof g.name, "%s", p.name);
        info.ok = std::strcmp(g.arch, "gfx950") == 0;
    });
    return info;
}

// "<arch> <cus> <mhz> <name>", the form of a table's device line after the
// keyword.
void format_sig(const DeviceSig& g, char* buf, size_t cap)
{
    std::snprintf(buf, cap, "%s %d %d %s", g.arch, g.cus, g.mhz, g.name);
}

// Parse a device line's fields (the keyword already skipped); the name is
// the rest of the line with surrounding blanks removed.
bool parse_sig(const char* p, DeviceSig* g)
{
    int used = 0;
    char arch[64];
    if (std::sscanf(p, "%63s %d %d %n", arch, &g->cus, &g->mhz, &used) != 3 || used <= 0)
        return false;
    std::snprintf(g->arch, sizeof g->arch, "%s", arch);
    const char* q = p + used;
    while (*q == ' ' || *q == '\t')
        ++q;
    size_t len = std::strlen(q);
    while (len && (q[len - 1] == '\n' || q[len - 1] == '\r' || q[len - 1] == ' ' ||
                   q[len - 1] == '\t'))
        --len;
    if (len >= sizeof g->name)
        return false;
    std::memcpy(g->name, q, len);
    g->name[len] = 0;
    return true;
}

// Arch, CU count and peak clock must match; the names too when both sides
// have one (the runtime reports an empty name in some environments -- under
// the rocprofv3 tracer, for one -- and the clock alone separates the gfx950
// parts of 256 CUs).
bool same_sig(const DeviceSig& table, const DeviceSig& dev)
{
    return std::strcmp(table.arch, dev.arch) == 0 && table.cus == dev.cus &&
           table.mhz == dev.mhz &&
           (!table.name[0] || !dev.name[0] || std::strcmp(table.name, dev.name) == 0);
}

// ------------------------------------------------------------------ table
int bucket_of(int64_t M)
{
    int b = 1;
    while (b < M && b < 4096)
        b <<= 1;
    return b;
}

// (op, N, K, M bucket); bucket 0 names the whole (op, N, K) shape.
struct Key {
    int op;
    int bucket;
    int64_t N, K;
    bool operator==(const Key& o) const
    {
        return op == o.op && bucket == o.bucket && N == o.N && K == o.K;
    }
};
struct KeyHash {
    size_t operator()(const Key& k) const
    {
        uint64_t h = (uint64_t)k.N * 0x9E3779B97F4A7C15ull;
        h ^= ((uint64_t)k.K + 0x632BE59BD9B4E019ull) * 0xC2B2AE3D27D4EB4Full + (h << 6) + (h >> 2);
        h ^= (uint64_t)(k.op * 8191 + k.bucket) * 0x165667B19E3779F9ull + (h << 6) + (h >> 2);
        return (size_t)h;
    }
};

Key table_key(int op, int64_t N, int64_t K, int bucket) { return Key{op, bucket, N, K}; }

Key shape_key(int op, int64_t N, int64_t K) { return Key{op, 0, N, K}; }

struct Table {
    std::unordered_map<Key, qll_cfg, KeyHash> entries;
    // batch-invariant: the effective Split-K factor fixed per (N, K)
    std::unordered_map<Key, std::pair<int, int>, KeyHash> bi_fixed;
};

std::atomic<Table*> g_table{nullptr};  // replaced only by qll_init

// Every table qll_init has installed stays allocated until the process ends
// (a call on another thread may still be reading the previous one), but a
// table equal to one already loaded is not kept twice, so re-initializing
// with the same file does not grow memory.
Table* retain_table(Table* t)
{
    static std::mutex mu;
    static std::vector<Table*> loaded;
    std::lock_guard<std::mutex> lock(mu);
    auto same = [](const Table& x, const Table& y) {
        if (x.entries.size() != y.entries.size() || x.bi_fixed != y.bi_fixed)
            return false;
        for (const auto& kv : x.entries) {
            auto it = y.entries.find(kv.first);
            if (it == y.entries.end() || it->second.variant != kv.second.variant ||
                it->second.splits != kv.second.splits)
                return false;
        }
        return true;
    };
    for (Table* old : loaded)
        if (same(*old, *t)) {
            delete t;
            return old;
        }
    loaded.push_back(t);
    return t;
}

int find_variant(int op, const char* name)
{
    int n = 0;
    const Variant* v = variants(op, &n);
    for (int i = 0; i < n; ++i)
        if (std::strcmp(v[i].name, name) == 0)
            return i;
    if (op == OP_FP8_DYN)
        for (int i = 0; i < kNumFusedVariants; ++i)
            if (std::strcmp(kFusedVariants[i].name, name) == 0)
                return kNumVariantsFp8 + i;
    return -1;
}

int effective_splits(int op, int64_t K, int splits)
{
    const int64_t kbytes = op_kbytes(op, K);
    if (splits <= 1)
        return 1;
    int64_t chunk = (kbytes + splits - 1) / splits;
    chunk = (chunk + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
    return (int)((kbytes + chunk - 1) / chunk);
}

int64_t split_chunk(int op, int64_t K, int splits)
{
    const int64_t kbytes = op_kbytes(op, K);
    if (splits <= 1)
        return kbytes;
    int64_t chunk = (kbytes + splits - 1) / splits;
    return (chunk + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
}

int load_table(const char* path, const DeviceSig& want, Table** out, std::string* err)
{
    FILE* f = std::fopen(path, "r");
    if (!f) {
        *err = "cannot open table";
        return QLL_ERR_TABLE;
    }
    Table* t = new Table;
    char line[512];
    bool device_ok = false, device_seen = false;
    int rc = QLL_OK;
    std::unordered_map<Key, std::pair<int, int>, KeyHash> bi_seen;
    while (std::fgets(line, sizeof line, f)) {
        char* p = line;
        while (*p == ' ' || *p == '\t')
            ++p;
        if (*p == '#' || *p == '\n' || *p == 0)
            continue;
        char a0[64], a2[64];
        if (std::strncmp(p, "device", 6) == 0 && (p[6] == ' ' || p[6] == '\t')) {
            DeviceSig g;
            if (device_seen || !parse_sig(p + 6, &g)) {
                rc = QLL_ERR_TABLE;
                *err = device_seen ? "more than one device line" : "bad device line";
                break;
            }
            device_seen = true;
            device_ok = same_sig(g, want);
            continue;
        }
        long long N = 0, K = 0;
        int bucket = 0, splits = 0;
        if (std::sscanf(p, "%63s %lld %lld %d %63s %d", a0, &N, &K, &bucket, a2,
                        &splits) != 6) {
            rc = QLL_ERR_TABLE;
            *err = std::string("bad entry: ") + p;
            break;
        }
        int op = -1;
        for (int i = 0; i < OP_COUNT; ++i)
            if (std::strcmp(a0, kOpNames[i]) == 0)
                op = i;
        const int vi = op >= 0 ? find_variant(op, a2) : -1;
        if (op < 0 || vi < 0 || splits < 1 || splits > kMaxSplits || N <= 0 ||
            K <= 0 || bucket < 1 || bucket > 4096 || (bucket & (bucket - 1))) {
            rc = QLL_ERR_TABLE;
            *err = std::string("bad entry: ") + p;
            break;
        }
        if (const FusedVariant* fv = op == OP_FP8_DYN ? dyn_fused(vi) : nullptr) {
            if (!fused_fits(*fv, bucket, K) || splits != 1) {
                rc = QLL_ERR_TABLE;
                *err = std::string("fused entry beyond its tokens, its K chunk or one split: ") + p;
                break;
            }
        } else {
            int n = 0;
            if (!variant_fits(op, variants(op, &n)[vi], K)) {
                rc = QLL_ERR_TABLE;
                *err = std::string("entry's variant does not support this K: ") + p;
                break;
            }
        }
        const int seff = effective_splits(op, K, splits);
        if (op == OP_BF16) {
            int n = 0;
            const Variant* v = variants(op, &n);
            // a variant whose waves split K must split it into the kBiFold chunks
            if (v[vi].name[0] == 'k' && v[vi].wp != kBiFold) {
                rc = QLL_ERR_TABLE;
                *err = "batch-invariant entry splits K across a number of waves other than the fixed chunk count";
                break;
            }
            const std::pair<int, int> fx(seff, 0);
            auto it = bi_seen.find(shape_key(op, N, K));
            if (it == bi_seen.end()) {
                bi_seen.emplace(shape_key(op, N, K), fx);
            } else if (it->second != fx) {
                rc = QLL_ERR_TABLE;
                *err = "batch-invariant entries vary the K split with M";
                break;
            }
        }
        t->entries[table_key(op, N, K, bucket)] = qll_cfg{vi, splits};
    }
    std::fclose(f);
    if (rc == QLL_OK && (!device_seen || !device_ok)) {
        rc = QLL_ERR_TABLE;
        *err = "table was measured on another device";
    }
    if (rc != QLL_OK || !out) {
        delete t;
        return rc;
    }
    t->bi_fixed = std::move(bi_seen);
    *out = t;
    return QLL_OK;
}

// ------------------------------------------------------------------ heuristic
// Used when the table has no entry.  M <= 64: the skinny Swap-AB kernel (for
// the ordinary ops its waves split K inside the workgroup); larger M: the
// pipelined ordinary tiles with two-stage rings (several workgroups per CU),
// growing with M, with Split-K until the grid covers the CUs once.  The batch-invariant
// op never splits K across workgroups, and every variant it uses sums K in
// the same kBiFold chunks (the skinny kernel with eight waves does so by
// construction, the others fold their accumulator at the chunk boundaries).
qll_cfg heuristic(int op, int64_t M, int64_t N, int64_t K)
{
    if (op == OP_FP8_DYN)  // two launches with the FP8 GEMM's rule
        op = OP_FP8;
    const int cus = device_info().cus;
    const char* name;
    bool exact = true;
    if (op == OP_W4A16) {
        // few tokens: the wave-split decode kernel; more: the pipelined
        // tiles (the fastest variants of the on-device sweep of the two
        // sweep shapes)
        name = M <= 16 ? "k16x16_w16"
             : M <= 64 ? "k16x32_w8"
             : M <= 512 ? "p64x64_w2x2_s3" : "p128x128_w2x4_s3";
    } else if (op == OP_MXFP4 && M > 32) {
        // 256-byte K stages (four MFMA steps of 128 elements per barrier):
        // fastest from 64 tokens up on the sweep shapes
        name = M <= 1024 ? "p64x64_w2x2_k256_s2" : "p128x128_w2x2_k256_s2";
    } else if (M <= 64) {
        if (op == OP_BF16)  // eight waves = the kBiFold chunks
            name = M <= 16 ? "k16x16_w8" : (M <= 32 ? "k16x32_w8" : "k16x64_w8");
        else if (M <= 16)  // 8-row workgroups when 16-row ones leave CUs idle
            name = (N + 15) / 16 >= 2 * cus ? "k16x16_w8"
                 : (N + 15) / 16 >= cus     ? "k16x16_w16"
                                            : "k8x16_w16";
        else
            name = M <= 32 ? "k16x32_w8" : "k16x64_w8";
    } else if (op == OP_BLOCK) {
        exact = false;
        if (M <= 128)
            name = "n64x128_w2x2_k";
        else if (M * N >= (int64_t)cus * 4 * 128 * 256)
            name = "n128x256_w2x2_k";
        else
            name = "n128x128_w2x2_k";
    } else if (M <= 512) {
        name = "p64x64_w2x2_k128_s2";
    } else if (M <= 1024) {
        name = "p128x64_w2x2_k128_s2";
    } else {
        name = "p128x128_w2x2_k128_s2";
    }
    int n = 0;
    const Variant* v = variants(op, &n);
    int vi = 0;
    for (int i = 0; i < n; ++i)
        if (exact ? std::strcmp(v[i].name, name) == 0
                  : std::strncmp(v[i].name, name, std::strlen(name)) == 0) {
            vi = i;
            break;
        }
    const int64_t kbytes = op_kbytes(op, K);
    if (!variant_fits(op, v[vi], K)) {  // very long rows: the plain tiled kernel
        const char* fb = op == OP_W4A16 ? "t128x128_w2x2" : "n128x128_w2x2_k";
        for (int i = 0; i < n; ++i)
            if (std::strncmp(v[i].name, fb, std::strlen(fb)) == 0) {
                vi = i;
                break;
            }
    }
    if (op == OP_BF16 || M <= 64)
        return qll_cfg{vi, 1};
    const int64_t tiles = ((v[vi].swap ? N : M) + v[vi].bp - 1) / v[vi].bp *
                          (((v[vi].swap ? M : N) + v[vi].bq - 1) / v[vi].bq);
    int s = 1;
    while (tiles * s < cus && (int64_t)s * 2 * 1024 <= kbytes && s < 16)
        s *= 2;
    return qll_cfg{vi, s};
}

qll_cfg select_cfg(int op, int64_t M, int64_t N, int64_t K)
{
    const Table* t = g_table.load(std::memory_order_acquire);
    if (t) {
        auto it = t->entries.find(table_key(op, N, K, bucket_of(M)));
        if (it != t->entries.end())
            return it->second;
        if (op == OP_FP8_DYN)  // no entry of its own: the FP8 GEMM's choice
            return select_cfg(OP_FP8, M, N, K);
        if (op == OP_BF16) {
            auto fx = t->bi_fixed.find(shape_key(op, N, K));
            if (fx != t->bi_fixed.end()) {
                // a covered (N, K) keeps its table's K split at every M
                qll_cfg c = heuristic(op, M, N, K);
                c.splits = fx->second.first;
                return c;
            }
        }
    }
    return heuristic(op, M, N, K);
}

// ------------------------------------------------------------------ validation
bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

int validate_gemm(int op, const void* A, const void* B, const float* sa,
                  const float* sb, const void* out, int out_dtype, int64_t M,
                  int64_t N, int64_t K)
{
    if (M < 0 || N <= 0 || K <= 0)
        return QLL_ERR_INVALID_ARG;
    if (M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x3FFFFFFF)
        return QLL_ERR_INVALID_ARG;
    if (M * K > ((int64_t)1 << 40) || N * K > ((int64_t)1 << 40) ||
        M * N > ((int64_t)1 << 40))
        return QLL_ERR_INVALID_ARG;
    if (out_dtype != QLL_OUT_BF16 && out_dtype != QLL_OUT_FP32 &&
        !(out_dtype == QLL_OUT_INT32 && op == OP_INT8))
        return QLL_ERR_INVALID_ARG;
    if (op == OP_BF16) {
        if (K % 8)
            return QLL_ERR_INVALID_ARG;
    } else if (op == OP_BLOCK) {
        if (K % 128)
            return QLL_ERR_INVALID_ARG;
    } else if (op == OP_MXFP4) {
        if (K % 128 || K > kMaxKMxfp4)
            return QLL_ERR_INVALID_ARG;
    } else if (op == OP_W4A16) {
        if (K % 128)
            return QLL_ERR_INVALID_ARG;
    } else if (K % 16) {
        return QLL_ERR_INVALID_ARG;
    }
    if (op == OP_INT8 && K > 131071)
        return QLL_ERR_INVALID_ARG;
    if (M == 0)
        return QLL_OK;
    const bool has_sa = op != OP_BF16 && op != OP_W4A16;
    if (!A || !B || !out || (has_sa && !sa) || (op != OP_BF16 && !sb))
        return QLL_ERR_INVALID_ARG;
    if (misaligned(A, 16) || misaligned(B, 16) || misaligned(out, 16))
        return QLL_ERR_MISALIGNED;
    if ((has_sa && misaligned(sa, 4)) || (op != OP_BF16 && misaligned(sb, 4)))
        return QLL_ERR_MISALIGNED;
    return QLL_OK;
}

int validate_cfg(int op, const qll_cfg* c)
{
    int n = 0;
    variants(op, &n);
    if (op == OP_FP8_DYN)
        n = dyn_count();
    if (c->variant < 0 || c->variant >= n || c->splits < 1 || c->splits > kMaxSplits)
        return QLL_ERR_INVALID_ARG;
    if (op == OP_FP8_DYN && dyn_fused(c->variant) && c->splits != 1)
        return QLL_ERR_INVALID_ARG;  // a fused variant does not split K
    return QLL_OK;
}

int run_gemm(int op, const void* A, const void* B, const float* sa,
             const float* sb, void* out, int out_dtype, int64_t M, int64_t N,
             int64_t K, void* ws, size_t ws_bytes, void* stream,
             const qll_cfg* forced)
{
    int rc = validate_gemm(op, A, B, sa, sb, out, out_dtype, M, N, K);
    if (rc != QLL_OK)
        return rc;
    if (forced && (rc = validate_cfg(op, forced)) != QLL_OK)
        return rc;
    if (M == 0)
        return QLL_OK;
    const qll_cfg cfg = forced ? *forced : select_cfg(op, M, N, K);
    int nv = 0;
    const Variant* vs = variants(op, &nv);
    const Variant& v = vs[cfg.variant];
    if (!variant_fits(op, v, K))
        return QLL_ERR_UNSUPPORTED;
    GemmArgs a;
    a.A = A;
    a.B = B;
    a.sa = sa;
    a.sb = sb;
    a.out = out;
    a.ws = ws;
    a.out_dtype = out_dtype;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.kbytes = (int)op_kbytes(op, K);
    a.splits = effective_splits(op, K, cfg.splits);
    a.kchunk = (int)split_chunk(op, K, cfg.splits);
    a.kfold = op == OP_BF16 ? kBiFold : 1;
    a.offsets = nullptr;
    a.E = 0;
    if (a.splits > 1) {
        const uint64_t need = (uint64_t)a.splits * M * N * 4;
        if (!ws || ws_bytes < need)
            return QLL_ERR_WORKSPACE;
        if (misaligned(ws, 16))
            return QLL_ERR_MISALIGNED;
    }
    hipStream_t s = (hipStream_t)stream;
    if (v.launch(a, s) != hipSuccess)
        return QLL_ERR_HIP;
    if (a.splits > 1 && launch_splitk_reduce(op, a, s) != hipSuccess)
        return QLL_ERR_HIP;
    return QLL_OK;
}

// Built-in tile rule of the grouped GEMM by the mean rows per expert (the
// fastest variant measured on the 64-expert N = 1536, K = 2048 layer with
// skewed top-8 routing at 16, 128, 1024 and 4096 tokens): thin row tiles when
// experts get a few rows, the 256x256 tile once the heavy experts get
// hundreds (the skew puts most rows on a few experts).
const char* grouped_rule(int64_t M, int64_t E)
{
    const int64_t per = M / (E > 0 ? E : 1);
    if (per <= 4)
        return "p64x128_w2x2_k128_s2";
    if (per <= 32)
        return "p32x128_w1x4_k128_s4";
    return "p256x256_w2x4_k128_s2";
}

}  // namespace

// For the entry point without a workspace argument (noalloc.hip): the
// configuration a GEMM entry point picks for this shape, the Split-K
// workspace it needs, and the common validated launch path.
int gemm_plan(int op, int64_t M, int64_t N, int64_t K, qll_cfg* cfg, uint64_t* ws_need)
{
    *cfg = select_cfg(op, M, N, K);
    const int s = effective_splits(op, K, cfg->splits);
    *ws_need = s > 1 ? (uint64_t)s * (uint64_t)M * (uint64_t)N * 4u : 0u;
    return QLL_OK;
}

int gemm_run(int op, const void* A, const void* B, const float* sa, const float* sb,
             void* out, int out_dtype, int64_t M, int64_t N, int64_t K, void* ws,
             size_t ws_bytes, void* stream, const qll_cfg* cfg)
{
    return run_gemm(op, A, B, sa, sb, out, out_dtype, M, N, K, ws, ws_bytes, stream, cfg);
}

int gemm_validate(int op, const void* A, const void* B, const float* sa, const float* sb,
                  const void* out, int out_dtype, int64_t M, int64_t N, int64_t K)
{
    return validate_gemm(op, A, B, sa, sb, out, out_dtype, M, N, K);
}

}  // namespace qll

using namespace qll;

extern "C" {

int quantize_per_token_fp8(const void* x, void* q, float* scales, int64_t M,
                           int64_t K, int64_t group, void* stream)
{
    if (M < 0 || K <= 0 || K % 16 || M > 0x7FFFFFFF || K > 0x3FFFFFFF ||
        M * K > ((int64_t)1 << 40))
        return QLL_ERR_INVALID_ARG;
    const bool per_token = group == 0 || group == K;
    if (!per_token && group != 128)
        return QLL_ERR_UNSUPPORTED;
    if (!per_token && K % 128)
        return QLL_ERR_INVALID_ARG;
    if (M == 0)
        return QLL_OK;
    if (!x || !q || !scales)
        return QLL_ERR_INVALID_ARG;
    if (misaligned(x, 16) || misaligned(q, 16) || misaligned(scales, 4))
        return QLL_ERR_MISALIGNED;
    hipError_t e = per_token
                       ? launch_quant_rows(x, q, scales, (int)M, (int)K, (hipStream_t)stream)
                       : launch_quant_groups128(x, q, scales, (int)M, (int)K,
                                                (hipStream_t)stream);
    return e == hipSuccess ? QLL_OK : QLL_ERR_HIP;
}

int quantize_weight_block_fp8(const void* w, void* q, float* scales, int64_t N,
                              int64_t K, void* stream)
{
    if (N < 0 || K <= 0 || K % 128 || N > 0x7FFFFFFF || K > 0x3FFFFFFF ||
        N * K > ((int64_t)1 << 40))
        return QLL_ERR_INVALID_ARG;
    if (N == 0)
        return QLL_OK;
    if (!w || !q || !scales)
        return QLL_ERR_INVALID_ARG;
    if (misaligned(w, 16) || misaligned(q, 16) || misaligned(scales, 4))
        return QLL_ERR_MISALIGNED;
    if ((N + 127) / 128 > 0x7FFFFFFF || K / 128 > 65535)
        return QLL_ERR_INVALID_ARG;
    hipError_t e = launch_quant_weight_blocks(w, q, scales, (int)N, (int)K,
                                              (hipStream_t)stream);
    return e == hipSuccess ? QLL_OK : QLL_ERR_HIP;
}

int gemm_w8a8_int8_ex(const void* A, const void* B, const float* sa,
                      const float* sb, void* out, int out_dtype, int64_t M,
                      int64_t N, int64_t K, void* ws, size_t ws_bytes,
                      void* stream, const qll_cfg* cfg)
{
    return run_gemm(OP_INT8, A, B, sa, sb, out, out_dtype, M, N, K, ws,
                    ws_bytes, stream, cfg);
}

int gemm_fp8_scaled_ex(const void* A, const void* B, const float* sa,
                       const float* sb, void* out, int out_dtype, int64_t M,
                       int64_t N, int64_t K, void* ws, size_t ws_bytes,
                       void* stream, const qll_cfg* cfg)
{
    return run_gemm(OP_FP8, A, B, sa, sb, out, out_dtype, M, N, K, ws, ws_bytes,
                    stream, cfg);
}

int gemm_block_fp8_ex(const void* A, const void* B, const float* sa,
                      const float* sb, void* out, int out_dtype, int64_t M,
                      int64_t N, int64_t K, void* ws, size_t ws_bytes,
                      void* stream, const qll_cfg* cfg)
{
    return run_gemm(OP_BLOCK, A, B, sa, sb, out, out_dtype, M, N, K, ws,
                    ws_bytes, stream, cfg);
}

int gemm_bf16_batch_invariant_ex(const void* A, const void* B, void* out,
                                 int out_dtype, int64_t M, int64_t N, int64_t K,
                                 void* ws, size_t ws_bytes, void* stream,
                                 const qll_cfg* cfg)
{
    return run_gemm(OP_BF16, A, B, nullptr, nullptr, out, out_dtype, M, N, K,
                    ws, ws_bytes, stream, cfg);
}

int gemm_w8a8_int8(const void* A, const void* B, const float* sa,
                   const float* sb, void* out, int out_dtype, int64_t M,
                   int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream)
{
    return run_gemm(OP_INT8, A, B, sa, sb, out, out_dtype, M, N, K, ws,
                    ws_bytes, stream, nullptr);
}

int gemm_fp8_scaled(const void* A, const void* B, const float* sa,
                    const float* sb, void* out, int out_dtype, int64_t M,
                    int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream)
{
    return run_gemm(OP_FP8, A, B, sa, sb, out, out_dtype, M, N, K, ws, ws_bytes,
                    stream, nullptr);
}

int gemm_block_fp8(const void* A, const void* B, const float* sa,
                   const float* sb, void* out, int out_dtype, int64_t M,
                   int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream)
{
    return run_gemm(OP_BLOCK, A, B, sa, sb, out, out_dtype, M, N, K, ws,
                    ws_bytes, stream, nullptr);
}

int gemm_bf16_batch_invariant(const void* A, const void* B, void* out,
                              int out_dtype, int64_t M, int64_t N, int64_t K,
                              void* ws, size_t ws_bytes, void* stream)
{
    return run_gemm(OP_BF16, A, B, nullptr, nullptr, out, out_dtype, M, N, K,
                    ws, ws_bytes, stream, nullptr);
}

int quantize_mxfp4(const void* x, void* q, void* scales, int64_t M, int64_t K, void* stream)
{
    if (M < 0 || K <= 0 || K % 32 || M > 0x7FFFFFFF || K > 0x3FFFFFFF ||
        M * K > ((int64_t)1 << 40))
        return QLL_ERR_INVALID_ARG;
    if (M == 0)
        return QLL_OK;
    if (!x || !q || !scales)
        return QLL_ERR_INVALID_ARG;
    if (misaligned(x, 16) || misaligned(q, 4))
        return QLL_ERR_MISALIGNED;
    return launch_quant_mxfp4(x, q, scales, M * K, (hipStream_t)stream) == hipSuccess
               ? QLL_OK
               : QLL_ERR_HIP;
}

int quantize_int4_weights(const void* w, void* q, float* scales, int64_t N, int64_t K,
                          void* stream)
{
    if (N < 0 || K <= 0 || K % 128 || N > 0x7FFFFFFF || K > 0x3FFFFFFF ||
        N * K > ((int64_t)1 << 40))
        return QLL_ERR_INVALID_ARG;
    if (N == 0)
        return QLL_OK;
    if (!w || !q || !scales)
        return QLL_ERR_INVALID_ARG;
    if (misaligned(w, 16) || misaligned(q, 4) || misaligned(scales, 4))
        return QLL_ERR_MISALIGNED;
    return launch_quant_int4(w, q, scales, N * K, (hipStream_t)stream) == hipSuccess
               ? QLL_OK
               : QLL_ERR_HIP;
}

int gemm_w4a16_ex(const void* A, const void* B, const float* scales, void* out, int out_dtype,
                  int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream,
                  const qll_cfg* cfg)
{
    return run_gemm(OP_W4A16, A, B, nullptr, scales, out, out_dtype, M, N, K, ws, ws_bytes,
                    stream, cfg);
}

int gemm_w4a16(const void* A, const void* B, const float* scales, void* out, int out_dtype,
               int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream)
{
    return run_gemm(OP_W4A16, A, B, nullptr, scales, out, out_dtype, M, N, K, ws, ws_bytes,
                    stream, nullptr);
}

int gemm_mxfp4_ex(const void* A, const void* B, const void* sa, const void* sb, void* out,
                  int out_dtype, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                  void* stream, const qll_cfg* cfg)
{
    return run_gemm(OP_MXFP4, A, B, (const float*)sa, (const float*)sb, out, out_dtype, M, N,
                    K, ws, ws_bytes, stream, cfg);
}

int gemm_mxfp4(const void* A, const void* B, const void* sa, const void* sb, void* out,
               int out_dtype, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
               void* stream)
{
    return run_gemm(OP_MXFP4, A, B, (const float*)sa, (const float*)sb, out, out_dtype, M, N,
                    K, ws, ws_bytes, stream, nullptr);
}

int linear_fp8_dynamic_ex(const void* x, const void* B, const float* sb, void* q,
                          float* sa, void* out, int out_dtype, int64_t M, int64_t N,
                          int64_t K, void* ws, size_t ws_bytes, void* stream,
                          const qll_cfg* cfg)
{
    if (!q || !sa || !x)
        return M == 0 && N > 0 && K > 0 ? QLL_OK : QLL_ERR_INVALID_ARG;
    int rc = validate_gemm(OP_FP8, x, B, sa, sb, out, out_dtype, M, N, K);
    if (rc != QLL_OK)
        return rc;
    if (cfg && (rc = validate_cfg(OP_FP8_DYN, cfg)) != QLL_OK)
        return rc;
    if (misaligned(q, 16))
        return QLL_ERR_MISALIGNED;
    if (M == 0)
        return QLL_OK;
    const qll_cfg c = cfg ? *cfg : select_cfg(OP_FP8_DYN, M, N, K);
    if (const FusedVariant* fv = dyn_fused(c.variant)) {
        // one launch: quantizer inside the decode GEMM
        if (!fused_fits(*fv, M, K))
            return QLL_ERR_UNSUPPORTED;
        FusedArgs f;
        f.x = (const uint16_t*)x;
        f.B = (const uint8_t*)B;
        f.sb = sb;
        f.q = (uint8_t*)q;
        f.sa = sa;
        f.out = out;
        f.out_dtype = out_dtype;
        f.M = (int)M;
        f.N = (int)N;
        f.K = (int)K;
        return fv->launch(f, (hipStream_t)stream) == hipSuccess ? QLL_OK : QLL_ERR_HIP;
    }
    // two launches: the quantizer, then the FP8 GEMM with the GEMM's own
    // checks done before anything is enqueued
    int nv = 0;
    if (!variant_fits(OP_FP8, variants(OP_FP8, &nv)[c.variant], K))
        return QLL_ERR_UNSUPPORTED;
    const int splits = effective_splits(OP_FP8, K, c.splits);
    if (splits > 1) {
        if (!ws || ws_bytes < (uint64_t)splits * M * N * 4)
            return QLL_ERR_WORKSPACE;
        if (misaligned(ws, 16))
            return QLL_ERR_MISALIGNED;
    }
    rc = quantize_per_token_fp8(x, q, sa, M, K, 0, stream);
    if (rc != QLL_OK)
        return rc;
    return run_gemm(OP_FP8, q, B, sa, sb, out, out_dtype, M, N, K, ws, ws_bytes, stream,
                    &c);
}

int linear_fp8_dynamic(const void* x, const void* B, const float* sb, void* q, float* sa,
                       void* out, int out_dtype, int64_t M, int64_t N, int64_t K, void* ws,
                       size_t ws_bytes, void* stream)
{
    return linear_fp8_dynamic_ex(x, B, sb, q, sa, out, out_dtype, M, N, K, ws, ws_bytes,
                                 stream, nullptr);
}

int qll_grouped_select(int64_t M, int64_t E, char* buf, size_t cap)
{
    if (M < 0 || E < 1 || !buf || cap == 0)
        return QLL_ERR_INVALID_ARG;
    const char* name = grouped_rule(M, E);
    if (std::strlen(name) + 1 > cap)
        return QLL_ERR_INVALID_ARG;
    std::memcpy(buf, name, std::strlen(name) + 1);
    return QLL_OK;
}

int gemm_fp8_grouped_ex(const void* A, const void* B, const float* sa, const float* sb,
                        const int32_t* offsets, void* out, int out_dtype, int64_t M,
                        int64_t N, int64_t K, int64_t E, void* stream, const char* variant)
{
    if (M < 0 || N <= 0 || K <= 0 || K % 16 || E < 1 || E > 65536 || M > 0x7FFFFFFF ||
        N > 0x7FFFFFFF || K > 0x3FFFFFFF || M * K > ((int64_t)1 << 40) ||
        E * N * K > ((int64_t)1 << 42) || M * N > ((int64_t)1 << 40))
        return QLL_ERR_INVALID_ARG;
    if (out_dtype != QLL_OUT_BF16 && out_dtype != QLL_OUT_FP32)
        return QLL_ERR_INVALID_ARG;
    int nv = 0;
    const Variant* vs = grouped_variants(&nv);
    const char* name = variant ? variant : grouped_rule(M, E);
    int vi = -1;
    for (int i = 0; i < nv; ++i)
        if (std::strcmp(vs[i].name, name) == 0)
            vi = i;
    if (vi < 0)
        return QLL_ERR_INVALID_ARG;
    if (M == 0)
        return QLL_OK;
    if (!A || !B || !sa || !sb || !offsets || !out)
        return QLL_ERR_INVALID_ARG;
    if (misaligned(A, 16) || misaligned(B, 16) || misaligned(out, 16) || misaligned(sa, 4) ||
        misaligned(sb, 4) || misaligned(offsets, 4))
        return QLL_ERR_MISALIGNED;
    if (!variant_fits(OP_FP8, vs[vi], K))
        return QLL_ERR_UNSUPPORTED;
    GemmArgs a;
    a.A = A;
    a.B = B;
    a.sa = sa;
    a.sb = sb;
    a.out = out;
    a.ws = nullptr;
    a.out_dtype = out_dtype;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.kbytes = (int)K;
    a.splits = 1;
    a.kchunk = (int)K;
    a.kfold = 1;
    a.offsets = offsets;
    a.E = (int)E;
    return vs[vi].launch(a, (hipStream_t)stream) == hipSuccess ? QLL_OK : QLL_ERR_HIP;
}

int gemm_fp8_grouped(const void* A, const void* B, const float* sa, const float* sb,
                     const int32_t* offsets, void* out, int out_dtype, int64_t M, int64_t N,
                     int64_t K, int64_t E, void* stream)
{
    return gemm_fp8_grouped_ex(A, B, sa, sb, offsets, out, out_dtype, M, N, K, E, stream,
                               nullptr);
}

int qll_init(const char* table_path)
{
    const char* path = table_path;
    if (!path || !*path)
        path = std::getenv("QLL_TABLE");
    if (!device_info().ok)
        return QLL_ERR_NO_DEVICE;
    if (noalloc_setup() != hipSuccess) {
        (void)hipGetLastError();
        return QLL_ERR_HIP;
    }
    if (!path || !*path) {
        g_table.store(nullptr, std::memory_order_release);
        return QLL_OK;
    }
    Table* t = nullptr;
    std::string err;
    int rc = load_table(path, device_info().sig, &t, &err);
    if (rc != QLL_OK) {
        if (std::getenv("QLL_LOG"))
            std::fprintf(stderr, "qll: table %s not used: %s\n", path, err.c_str());
        g_table.store(nullptr, std::memory_order_release);
        return rc;
    }
    Table* kept = retain_table(t);  // (t itself may be gone now)
    g_table.store(kept, std::memory_order_release);
    if (std::getenv("QLL_LOG"))
        std::fprintf(stderr, "qll: table %s: %zu entries\n", path, kept->entries.size());
    return QLL_OK;
}

int qll_table_validate(const char* path, const char* arch, int cus, int mhz,
                       const char* name, char* err, size_t cap)
{
    if (!path || !arch || !name)
        return QLL_ERR_INVALID_ARG;
    DeviceSig want;
    std::snprintf(want.arch, sizeof want.arch, "%s", arch);
    want.cus = cus;
    want.mhz = mhz;
    std::snprintf(want.name, sizeof want.name, "%s", name);
    std::string e;
    const int rc = load_table(path, want, nullptr, &e);
    if (err && cap)
        std::snprintf(err, cap, "%s", e.c_str());
    return rc;
}

int qll_device_signature(char* buf, size_t cap)
{
    if (!buf || cap == 0)
        return QLL_ERR_INVALID_ARG;
    if (!device_info().ok)
        return QLL_ERR_NO_DEVICE;
    char tmp[400];
    format_sig(device_info().sig, tmp, sizeof tmp);
    if (std::strlen(tmp) + 1 > cap)
        return QLL_ERR_INVALID_ARG;
    std::memcpy(buf, tmp, std::strlen(tmp) + 1);
    return QLL_OK;
}

int qll_select(int op, int64_t M, int64_t N, int64_t K, qll_cfg* cfg_out)
{
    if (op < 0 || op >= OP_COUNT || M < 0 || N <= 0 || K <= 0 || !cfg_out)
        return QLL_ERR_INVALID_ARG;
    *cfg_out = select_cfg(op, M, N, K);
    return QLL_OK;
}

int64_t qll_workspace_bytes(int op, int64_t M, int64_t N, int64_t K,
                            const qll_cfg* cfg)
{
    if (op < 0 || op >= OP_COUNT || M < 0 || N <= 0 || K <= 0)
        return -QLL_ERR_INVALID_ARG;
    qll_cfg c = cfg ? *cfg : select_cfg(op, M, N, K);
    if (validate_cfg(op, &c) != QLL_OK)
        return -QLL_ERR_INVALID_ARG;
    if (op == OP_FP8_DYN && dyn_fused(c.variant))
        return 0;
    const int s = effective_splits(op, K, c.splits);
    return s > 1 ? (int64_t)s * M * N * 4 : 0;
}

int qll_effective_splits(int op, int64_t K, int32_t splits)
{
    if (op < 0 || op >= OP_COUNT || K <= 0 || splits < 1)
        return -QLL_ERR_INVALID_ARG;
    return effective_splits(op, K, splits);
}

int qll_num_variants(int op)
{
    if (op == OP_FP8_DYN)
        return dyn_count();
    int n = 0;
    variants(op, &n);
    return n;
}

int qll_variant_info(int op, int idx, char* buf, size_t cap)
{
    if (op < 0 || op >= OP_COUNT || !buf || cap == 0)
        return QLL_ERR_INVALID_ARG;
    if (const FusedVariant* f = op == OP_FP8_DYN ? dyn_fused(idx) : nullptr) {
        std::snprintf(buf, cap,
                      "{\"name\": \"%s\", \"op\": \"%s\", \"swap\": 1, \"bp\": %d, "
                      "\"bq\": %d, \"wp\": %d, \"wq\": 1, \"kstage\": 128, \"lds\": %d, "
                      "\"fused\": 1, \"ksteps\": %d}",
                      f->name, kOpNames[op], f->hr, f->tok, f->w,
                      f->w * 1024 + f->w * 64 + 64 + (f->tok < 16 ? f->w * f->d * f->tok * 128 : 0),
                      f->d);
        return QLL_OK;
    }
    int n = 0;
    const Variant* v = variants(op, &n);
    if (idx < 0 || idx >= n)
        return QLL_ERR_INVALID_ARG;
    std::snprintf(buf, cap,
                  "{\"name\": \"%s\", \"op\": \"%s\", \"swap\": %d, \"bp\": %d, "
                  "\"bq\": %d, \"wp\": %d, \"wq\": %d, \"kstage\": %d, \"lds\": %d, "
                  "\"fused\": 0}",
                  v[idx].name, kOpNames[op], v[idx].swap, v[idx].bp, v[idx].bq,
                  v[idx].wp, v[idx].wq, v[idx].kstage, v[idx].lds);
    return QLL_OK;
}

int qll_variant_index(int op, const char* name)
{
    if (op < 0 || op >= OP_COUNT || !name)
        return -QLL_ERR_INVALID_ARG;
    return find_variant(op, name);
}

int qll_table_entries(void)
{
    const Table* t = g_table.load(std::memory_order_acquire);
    return t ? (int)t->entries.size() : 0;
}

const char* qll_status_str(int status)
{
    switch (status) {
    case QLL_OK: return "ok";
    case QLL_ERR_INVALID_ARG: return "invalid argument";
    case QLL_ERR_UNSUPPORTED: return "unsupported";
    case QLL_ERR_MISALIGNED: return "misaligned pointer";
    case QLL_ERR_WORKSPACE: return "workspace missing or too small";
    case QLL_ERR_NO_DEVICE: return "no gfx950 device";
    case QLL_ERR_TABLE: return "dispatch table not usable";
    case QLL_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

}  // extern "C"
