// GEMV kernels for Q6_K weights (all batch sizes, activation types and
// workgroup shapes); the kernel code is in kq_gemv.h.
#include "kq_gemv.h"

namespace kq {
template hipError_t launch_gemv_type<KQ_Q6_K>(int, int, int, bool, const GemvArgs&, int, size_t, hipStream_t);
}  // namespace kq
