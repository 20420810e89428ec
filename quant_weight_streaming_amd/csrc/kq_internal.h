// Host/device interface between the C-ABI layer (kq_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kq.h"

namespace kq {

// Kernel arguments of one GEMV launch (one or several projections sharing x).
struct GemvArgs {
  const uint8_t* w[KQ_MAX_PROJ];       // repacked weights of each projection
  float* y[KQ_MAX_PROJ];               // outputs
  int64_t ldy[KQ_MAX_PROJ];            // output row strides (elements)
  int32_t rows[KQ_MAX_PROJ];           // rows of each projection
  int32_t tile_begin[KQ_MAX_PROJ + 1]; // first global tile of each projection (prefix sums)
  int32_t nproj;
  int32_t n_cols;                      // super-block columns = cols / 256
  const void* x;                       // activations (fp32 or bf16)
  int64_t ldx;                         // activation row stride (elements)
  int32_t n_units;                     // total tiles * n_cols
  int32_t upw;                         // units per wavefront
  int32_t tsb;                         // LDS capacity in staged columns per workgroup
  // Whole-tile workgroups (tiles_per_wg > 0): n_win column windows, window w
  // covers win_base (+1 for w < win_extra) columns; wg_per_win workgroups per
  // window each take tiles_per_wg whole tiles of it.  tiles_per_wg == 0: even
  // runs of upw units per wavefront over the whole unit range.
  int32_t n_win, win_base, win_extra, wg_per_win, tiles_per_wg, n_tiles;
  float* partial;                      // scratch: [workgroups][2] (windows: [n_win][n_tiles]) x [KQ_MAX_BATCH][64]
  uint32_t* counters;                  // scratch: arrival counters per split tile, zero between calls
};

// Launch the GEMV with workgroups of `nw` (4 or 8) wavefronts.
hipError_t launch_gemv(int type, int xtype, int batch, int nw, const GemvArgs& a, int grid, size_t lds,
                       hipStream_t s);
// Whether launch_gemv runs this activation type and batch on the matrix cores,
// and the dynamic LDS a workgroup of `nw` wavefronts staging `staged_cols`
// columns needs.
bool gemv_uses_mfma(int xtype, int batch);
size_t gemv_lds_bytes(int type, int xtype, int batch, int nw, int staged_cols);
hipError_t launch_repack(int type, int64_t rows, int64_t cols, const void* gguf, void* out, hipStream_t s);
hipError_t launch_dequant(int type, const void* w, int64_t rows, int64_t cols, float* out, int64_t ldo,
                          hipStream_t s);

int64_t sb_bytes(int type);

}  // namespace kq
