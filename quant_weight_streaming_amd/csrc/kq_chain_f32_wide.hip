// Chain kernels (persistent launches over a sequence of GEMV steps) for fp32 activations,
// batches 5 to 8 (10 to 16 staged bf16 rows, matrix cores); the kernel code is in kq_gemv.h.
#include "kq_gemv.h"

namespace kq {
template hipError_t launch_chain_wide<10, true>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<12, true>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<14, true>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<16, true>(const ChainArgs&, int, size_t, hipStream_t, int*);
}  // namespace kq
