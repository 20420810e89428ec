// Chain kernels (persistent launches over a sequence of GEMV steps) for bf16 activations,
// batches 9 to 16 (matrix cores, 8-wavefront workgroups); the kernel code is in kq_gemv.h.
#include "kq_gemv.h"

namespace kq {
template hipError_t launch_chain_wide<9, false>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<10, false>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<11, false>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<12, false>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<13, false>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<14, false>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<15, false>(const ChainArgs&, int, size_t, hipStream_t, int*);
template hipError_t launch_chain_wide<16, false>(const ChainArgs&, int, size_t, hipStream_t, int*);
}  // namespace kq
