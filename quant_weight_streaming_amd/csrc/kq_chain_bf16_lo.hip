// Chain kernels (persistent launches over a sequence of GEMV steps) for bf16 activations,
// batches 1 to 4; the kernel code is in kq_gemv.h.
#include "kq_gemv.h"

namespace kq {
template hipError_t launch_chain_b<1, false>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<2, false>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<3, false>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<4, false>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
}  // namespace kq
