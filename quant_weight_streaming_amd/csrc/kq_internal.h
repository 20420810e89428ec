// Host/device interface between the C-ABI layer (kq_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kq.h"

namespace kq {


constexpr int kHeadRows = 128;        // outputs per head of a KQ_EPI_HEADNORM segment (head_dim)

// Workspace of one GEMV call (caller-owned device memory, see kq.h):
//   [0, kCounterBytes)  arrival counters: kMaxGroups for split tiles (indexed by
//                       workgroup, or by tile with column windows), then
//                       kMaxGroups for head-norm heads (indexed by first tile).
//                       Zero between calls: every call leaves them zero.
//   then the partial-sum slots of split tiles, n_slots x partial_stride(B) floats
//   (B = the call's batch): [B][64] row sums, then the piece's sums of x^2 per
//   batch row (normalised launches) at partial_q(B);
//   then, for launches with a head-norm segment, [tile][2][KQ_MAX_BATCH] floats of
//   the heads' tile sums of squares.
constexpr int kMaxGroups = 8192;
constexpr size_t kCounterBytes = (size_t)2 * kMaxGroups * sizeof(uint32_t);
__host__ __device__ constexpr int partial_q(int b) { return b * 64; }
__host__ __device__ constexpr int partial_stride(int b) { return b * 64 + 64; }
constexpr size_t kWorkspaceMax = kCounterBytes + (size_t)2 * kMaxGroups * partial_stride(KQ_MAX_BATCH) * sizeof(float) +
                                 (size_t)kMaxGroups * 2 * KQ_MAX_BATCH * sizeof(float);
static_assert(kWorkspaceMax == KQ_WORKSPACE_BYTES, "kq.h states the largest workspace a call can need");

// Kernel arguments of one GEMV launch (one or several projections sharing x).

struct GemvArgs {
  const uint8_t* w[KQ_MAX_PROJ];       // repacked weights of each projection
  float* y[KQ_MAX_PROJ];               // outputs
  int64_t ldy[KQ_MAX_PROJ];            // output row strides (elements)
  uint16_t* y16[KQ_MAX_PROJ];          // optional bf16 copies of the outputs (null: none)
  int64_t ldy16[KQ_MAX_PROJ];          // their row strides (elements)
  int32_t rows[KQ_MAX_PROJ];           // rows of each projection
  int32_t tile_begin[KQ_MAX_PROJ + 1]; // first global tile of each projection (prefix sums)
  int32_t nproj;
  int32_t n_cols;                      // super-block columns = cols / 256
  const void* x;                       // activations (fp32 or bf16)
  int64_t ldx;                         // activation row stride (elements)
  int32_t n_units;                     // total tiles * n_cols
  int32_t upw;                         // units per wavefront
  int32_t wgu;                         // units per workgroup: nw * upw, or (units taken dynamically by
                                       // the wavefronts) an even share of the units per CU
  int32_t tsb;                         // LDS capacity in staged columns per workgroup
  int32_t tpw;                         // tiles a wavefront's run of units can touch (its LDS tile sums)
  uint32_t epi;                        // epilogue code of segment i in bits 4i..4i+3 (KQ_EPI_*); KQ_EPI_SWIGLU:
                                       // one segment whose tile t holds 32 gate and 32 up rows
  float rms_eps;                       // > 0: x is normalised first, x / sqrt(mean(x^2) + rms_eps) per batch row
  float head_eps;                      // KQ_EPI_HEADNORM segments: the per-head norm's epsilon
  float* head_ss;                      // workspace: [tile][2][KQ_MAX_BATCH] sums of squares of the heads' tiles
  uint32_t* head_ctr;                  // workspace: arrival counters per head (by its first tile), zero between calls
  // Whole-tile workgroups (tiles_per_wg > 0): n_win column windows, window w
  // covers win_base (+1 for w < win_extra) columns; wg_per_win workgroups per
  // window each take tiles_per_wg whole tiles of it.  tiles_per_wg == 0: even
  // runs of upw units per wavefront over the whole unit range.
  int32_t n_win, win_base, win_extra, wg_per_win, tiles_per_wg, n_tiles;
  float* partial;                      // workspace: [workgroups][2] (windows: [n_win][n_tiles]) slots of
                                       // partial_stride(batch) floats
  uint32_t* counters;                  // workspace: arrival counters per split tile, zero between calls
};

// The two-hop step barrier's done word of a step is stored in this many
// copies, one 64-byte line each; workgroup g polls copy g % kDoneReplicas.
constexpr int kDoneReplicas = 16;

// Control words of a chain launch (device memory owned by the chain).
struct ChainCtl {
  uint32_t* arrive;    // [step][workgroup]: the run's tag once the workgroup finished the step
  uint32_t* done;      // [step][kDoneReplicas][16]: the run's tag once every workgroup finished the step
  uint32_t* epoch;     // tag of the last completed run
  uint32_t* error;     // set when a wait gave up
  uint32_t* error_host;// pinned host word, set with the error word (read by the host without a sync)
  uint64_t* tl;        // timeline builds (KQ_TIMELINE): [step][workgroup][8] device clock stamps; else null
  uint32_t groups;     // workgroups of the launch
  uint32_t spin;       // polls before a wait gives up
};

// One step of a chain, device-resident: its launch arguments, weight type,
// logical workgroups (a multiple of 8, at most the launch's), whether it
// waits for the previous step (0: a further weight type of the same step, which
// shares its x and writes other outputs), and the resident workgroup that takes
// its logical block 0 (a multiple of 8: a further weight type starts after the
// workgroups of the types before it, so they do not take both).
struct ChainStep {
  GemvArgs a;
  int32_t type;
  int32_t grid;
  int32_t wait;    // a barrier sub-step: its workgroups wait until every earlier sub-step is complete
  int32_t first;
  int32_t gate;    // the latest barrier sub-step at or before this one (0: none)
};

struct ChainArgs {
  const ChainStep* steps;
  int32_t n_steps;
  ChainCtl ctl;
};

template <int B, bool XF32>
hipError_t launch_chain_b(const ChainArgs& c, int nw, bool mf, int grid, size_t lds, hipStream_t s, int* occupancy);
template <int B, bool XF32>
hipError_t launch_chain_wide(const ChainArgs& c, int grid, size_t lds, hipStream_t s, int* occupancy);

// Launch the GEMV of one weight type over `rows` staged activation rows (the
// batch, or twice it for fp32 activations) with workgroups of `nw` (4 or 8)
// wavefronts, on the matrix cores (`mf`, from 2 staged rows) or on the dot2
// VALU path.
template <int QT>
hipError_t launch_gemv_type(int xtype, int rows, int nw, bool mf, const GemvArgs& a, int grid, size_t lds,
                            hipStream_t s);

// The dynamic LDS a workgroup of `nw` wavefronts staging `staged_cols` columns
// needs on the chosen path: per column the activations of every batch row and
// (Q4_K/Q5_K) their sub-block sums (matrix cores: rows padded to 528 bytes, the
// sums as three bf16 parts per row padded to a multiple of 4 rows, then a
// 512-byte zero block), plus each wavefront's partial sums of the tiles its run touches
// (dynamic workgroups: a counter and one slot per unit).
// Workgroups whose wavefronts take units dynamically (see gemv_block): the dot2
// path (one or two staged rows: batch 1 or 2 with bf16 x, batch 1 with fp32 x)
// in 8-wavefront workgroups.  With more staged rows the per-unit LDS slots
// would not fit beside the staged activations.
template <int B, int NW, bool MF>
__host__ __device__ constexpr bool dyn_units() { return B <= 2 && NW == 8 && !MF; }
inline bool dyn_units(int batch, int nw, bool mf) { return batch <= 2 && nw == 8 && !mf; }

// `run_units`: units of one workgroup (the per-unit slots of dynamic workgroups);
// `tpw`: tiles one wavefront's run can touch (its tile sums otherwise).
// `rows`: staged bf16 rows (the batch, or twice the batch for fp32 activations);
// norm: the launch normalises x (sums of x^2 per staged column and row).
inline size_t gemv_lds_bytes(int type, int rows, int nw, bool mf, int staged_cols, int run_units, int tpw,
                             bool norm = false) {
  const size_t partials = (dyn_units(rows, nw, mf) ? 16 + (size_t)run_units * rows * 64 * sizeof(float)
                                                   : (size_t)nw * tpw * rows * 64 * sizeof(float)) +
                          (norm ? (size_t)((staged_cols * rows + 3) & ~3) * sizeof(float) : 0);
  const int sb = type == KQ_Q6_K ? 0 : 8;   // staged sub-block activation sums per column (Q6_K has no mins)
  if (mf) {
    const int nb = (rows + 3) / 4;
    return (size_t)staged_cols * (rows * 528 + (sb ? 3 * nb * 64 : 0)) + 512 + partials;
  }
  return (size_t)staged_cols * rows * 4 * (128 + sb) + partials;
}
hipError_t launch_repack(int type, int64_t rows, int64_t cols, const void* gguf, const void* gguf2, void* out,
                         hipStream_t s);
hipError_t launch_dequant(int type, const void* w, int64_t rows, int64_t cols, float* out, int64_t ldo,
                          hipStream_t s);
hipError_t launch_gather(int type, const void* w, int64_t rows, int64_t cols, const int32_t* ids, int64_t n,
                         float* out, int64_t ldo, hipStream_t s);
// Read `bytes` (a multiple of 16) from p once with the GEMV's loads (the achievable read rate).
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, int groups, hipStream_t s);
// Zero n 32-bit words with a kernel (graph-capturable, unlike a memset node).
hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t s);

int64_t sb_bytes(int type);

}  // namespace kq
