// Kernel instantiations and variant registry of the int8 GEMM.
#include "gemm_pipe.h"
#include "gemm_skinny.h"
#include "gemm_tile.h"
#include "variant_list.h"

QLL_FOR_EACH_VARIANT(QLL_INSTANTIATE, qll::OP_INT8, 256, 128)
QLL_FOR_EACH_SKINNY(QLL_SKINNY_INSTANTIATE, qll::OP_INT8, 2)
QLL_FOR_EACH_PIPE(QLL_PIPE_INSTANTIATE, qll::OP_INT8)
QLL_FOR_EACH_PIPE_K256(QLL_PIPE_INSTANTIATE, qll::OP_INT8)
QLL_FOR_EACH_PIPE_W8(QLL_PIPE_INSTANTIATE, qll::OP_INT8)
QLL_FOR_EACH_PIPE_DEEP_K256(QLL_PIPE_INSTANTIATE, qll::OP_INT8)
QLL_FOR_EACH_PIPE_BIG(QLL_PIPE_INSTANTIATE, qll::OP_INT8)
QLL_FOR_EACH_PIPE_W8_K256(QLL_PIPE_INSTANTIATE, qll::OP_INT8)
QLL_FOR_EACH_PIPE_KG2(QLL_PIPE_KG2_INSTANTIATE, qll::OP_INT8)
template __global__ void qll::splitk_reduce_kernel<qll::OP_INT8>(qll::GemmArgs);

namespace qll {

// host-side registry (the device pass only needs the kernels above)
#if !defined(__HIP_DEVICE_COMPILE__)
extern const Variant kVariantsInt8[] = {
    QLL_FOR_EACH_VARIANT(QLL_ENTRY, OP_INT8, 256, 128)
    QLL_FOR_EACH_SKINNY(QLL_SKINNY_ENTRY, OP_INT8, 2)
    QLL_FOR_EACH_PIPE(QLL_PIPE_ENTRY, OP_INT8)
    QLL_FOR_EACH_PIPE_K256(QLL_PIPE_ENTRY, OP_INT8)
    QLL_FOR_EACH_PIPE_W8(QLL_PIPE_ENTRY, OP_INT8)
    QLL_FOR_EACH_PIPE_DEEP_K256(QLL_PIPE_ENTRY, OP_INT8)
    QLL_FOR_EACH_PIPE_BIG(QLL_PIPE_ENTRY, OP_INT8)
    QLL_FOR_EACH_PIPE_W8_K256(QLL_PIPE_ENTRY, OP_INT8)
    QLL_FOR_EACH_PIPE_KG2(QLL_PIPE_KG2_ENTRY, OP_INT8)
};
extern const int kNumVariantsInt8 = sizeof(kVariantsInt8) / sizeof(Variant);
#endif

hipError_t launch_reduce_int8(const GemmArgs& a, hipStream_t stream)
{
    return launch_reduce<OP_INT8>(a, stream);
}

}  // namespace qll
