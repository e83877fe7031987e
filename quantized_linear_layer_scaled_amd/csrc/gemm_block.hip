// Kernel instantiations and variant registry of the block GEMM.
#include "gemm_pipe.h"
#include "gemm_skinny.h"
#include "gemm_tile.h"
#include "variant_list.h"

QLL_FOR_EACH_VARIANT(QLL_INSTANTIATE, qll::OP_BLOCK, 256, 128)
QLL_FOR_EACH_SKINNY(QLL_SKINNY_INSTANTIATE, qll::OP_BLOCK, 1)
QLL_FOR_EACH_PIPE(QLL_PIPE_INSTANTIATE, qll::OP_BLOCK)
QLL_FOR_EACH_PIPE_W8(QLL_PIPE_INSTANTIATE, qll::OP_BLOCK)
template __global__ void qll::splitk_reduce_kernel<qll::OP_BLOCK>(qll::GemmArgs);

namespace qll {

// host-side registry (the device pass only needs the kernels above)
#if !defined(__HIP_DEVICE_COMPILE__)
extern const Variant kVariantsBlock[] = {
    QLL_FOR_EACH_VARIANT(QLL_ENTRY, OP_BLOCK, 256, 128)
    QLL_FOR_EACH_SKINNY(QLL_SKINNY_ENTRY, OP_BLOCK, 1)
    QLL_FOR_EACH_PIPE(QLL_PIPE_ENTRY, OP_BLOCK)
    QLL_FOR_EACH_PIPE_W8(QLL_PIPE_ENTRY, OP_BLOCK)
};
extern const int kNumVariantsBlock = sizeof(kVariantsBlock) / sizeof(Variant);
#endif

hipError_t launch_reduce_block(const GemmArgs& a, hipStream_t stream)
{
    return launch_reduce<OP_BLOCK>(a, stream);
}

}  // namespace qll
