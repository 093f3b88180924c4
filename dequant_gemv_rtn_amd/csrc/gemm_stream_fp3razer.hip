// Weight-streaming MFMA kernels (gemm_stream_kernels.hpp) for Q_FP3_RAZER.  One
// translation unit per format so that the formats compile in parallel.
#include "gemm_stream_kernels.hpp"

namespace qg {
template StreamKernelFn stream_kernel_for<Q_FP3_RAZER>(int, int, int, bool);
template SplitKernelFn split_kernel_for<Q_FP3_RAZER>(int, int, int, bool);
}  // namespace qg
