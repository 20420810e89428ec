// Chain kernels (persistent launches over a sequence of GEMV steps) for bf16 activations,
// batches 5 to 8; the kernel code is in kq_gemv.h.
#include "kq_gemv.h"

namespace kq {
template hipError_t launch_chain_b<5, false>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<6, false>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<7, false>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<8, false>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
}  // namespace kq
