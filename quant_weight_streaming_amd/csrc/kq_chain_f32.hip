// Chain kernels (persistent launches over a sequence of GEMV steps) for fp32 activations,
// batches 1 to 4 (2 to 8 staged bf16 rows); the kernel code is in kq_gemv.h.
#include "kq_gemv.h"

namespace kq {
template hipError_t launch_chain_b<2, true>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<4, true>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<6, true>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_b<8, true>(const ChainArgs&, int, bool, int, size_t, hipStream_t, int*);
}  // namespace kq
