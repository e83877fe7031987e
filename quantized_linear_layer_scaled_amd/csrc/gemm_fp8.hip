// Kernel instantiations and variant registry of the fp8 GEMM.
#include "gemm_pipe.h"
#include "gemm_pipe32.h"
#include "gemm_skinny.h"
#include "gemm_tile.h"
#include "variant_list.h"

QLL_FOR_EACH_VARIANT(QLL_INSTANTIATE, qll::OP_FP8, 256, 128)
QLL_FOR_EACH_SKINNY(QLL_SKINNY_INSTANTIATE, qll::OP_FP8, 1)
QLL_FOR_EACH_PIPE(QLL_PIPE_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_K256(QLL_PIPE_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_W8(QLL_PIPE_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_DEEP_K256(QLL_PIPE_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_BIG(QLL_PIPE_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_W8_K256(QLL_PIPE_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_KG2(QLL_PIPE_KG2_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_RC(QLL_PIPE_RC_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_P32(QLL_P32_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE(QLL_PIPE_GROUPED_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_W8(QLL_PIPE_GROUPED_INSTANTIATE, qll::OP_FP8)
QLL_FOR_EACH_PIPE_BIG(QLL_PIPE_GROUPED_INSTANTIATE, qll::OP_FP8)
template __global__ void qll::splitk_reduce_kernel<qll::OP_FP8>(qll::GemmArgs);

namespace qll {

// host-side registry (the device pass only needs the kernels above)
#if !defined(__HIP_DEVICE_COMPILE__)
extern const Variant kVariantsFp8[] = {
    QLL_FOR_EACH_VARIANT(QLL_ENTRY, OP_FP8, 256, 128)
    QLL_FOR_EACH_SKINNY(QLL_SKINNY_ENTRY, OP_FP8, 1)
    QLL_FOR_EACH_PIPE(QLL_PIPE_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_K256(QLL_PIPE_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_W8(QLL_PIPE_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_DEEP_K256(QLL_PIPE_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_BIG(QLL_PIPE_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_W8_K256(QLL_PIPE_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_KG2(QLL_PIPE_KG2_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_RC(QLL_PIPE_RC_ENTRY, OP_FP8)
    QLL_FOR_EACH_P32(QLL_P32_ENTRY, OP_FP8)
};
extern const int kNumVariantsFp8 = sizeof(kVariantsFp8) / sizeof(Variant);
// the grouped (per-expert) GEMM runs the pipelined tiles over experts
extern const Variant kVariantsFp8Grouped[] = {
    QLL_FOR_EACH_PIPE(QLL_PIPE_GROUPED_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_W8(QLL_PIPE_GROUPED_ENTRY, OP_FP8)
    QLL_FOR_EACH_PIPE_BIG(QLL_PIPE_GROUPED_ENTRY, OP_FP8)
};
extern const int kNumVariantsFp8Grouped = sizeof(kVariantsFp8Grouped) / sizeof(Variant);
#endif

hipError_t launch_reduce_fp8(const GemmArgs& a, hipStream_t stream)
{
    return launch_reduce<OP_FP8>(a, stream);
}

}  // namespace qll
