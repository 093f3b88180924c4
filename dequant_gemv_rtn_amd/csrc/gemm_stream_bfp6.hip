// Weight-streaming MFMA kernels (gemm_stream_kernels.hpp) for Q_BFP6.  One
// translation unit per format so that the formats compile in parallel.
#include "gemm_stream_kernels.hpp"

namespace qg {
template StreamKernelFn stream_kernel_for<Q_BFP6>(int, int, int, bool);
template SplitKernelFn split_kernel_for<Q_BFP6>(int, int, int, bool);
}  // namespace qg
