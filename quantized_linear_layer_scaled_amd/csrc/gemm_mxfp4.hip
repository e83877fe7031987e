// Kernel instantiations and variant registry of the MXFP4 GEMM: the skinny
// Swap-AB kernels for few tokens and the pipelined tiles for many, both with
// the E8M0 block scales applied by the matrix core (no tiled fallback: the
// entry point limits K so that every pipelined variant fits).
#include "gemm_pipe.h"
#include "gemm_skinny.h"
#include "gemm_tile.h"

QLL_FOR_EACH_SKINNY(QLL_SKINNY_INSTANTIATE, qll::OP_MXFP4, 2)
QLL_FOR_EACH_PIPE(QLL_PIPE_INSTANTIATE, qll::OP_MXFP4)
QLL_FOR_EACH_PIPE_K256(QLL_PIPE_INSTANTIATE, qll::OP_MXFP4)
QLL_FOR_EACH_PIPE_W8(QLL_PIPE_INSTANTIATE, qll::OP_MXFP4)
QLL_FOR_EACH_PIPE_W8_K256(QLL_PIPE_INSTANTIATE, qll::OP_MXFP4)
template __global__ void qll::splitk_reduce_kernel<qll::OP_MXFP4>(qll::GemmArgs);

namespace qll {

// host-side registry (the device pass only needs the kernels above)
#if !defined(__HIP_DEVICE_COMPILE__)
extern const Variant kVariantsMxfp4[] = {
    QLL_FOR_EACH_SKINNY(QLL_SKINNY_ENTRY, OP_MXFP4, 2)
    QLL_FOR_EACH_PIPE(QLL_PIPE_ENTRY, OP_MXFP4)
    QLL_FOR_EACH_PIPE_K256(QLL_PIPE_ENTRY, OP_MXFP4)
    QLL_FOR_EACH_PIPE_W8(QLL_PIPE_ENTRY, OP_MXFP4)
    QLL_FOR_EACH_PIPE_W8_K256(QLL_PIPE_ENTRY, OP_MXFP4)
};
extern const int kNumVariantsMxfp4 = sizeof(kVariantsMxfp4) / sizeof(Variant);
#endif

hipError_t launch_reduce_mxfp4(const GemmArgs& a, hipStream_t stream)
{
    return launch_reduce<OP_MXFP4>(a, stream);
}

}  // namespace qll
