// C ABI of the K-quant GEMV library: argument validation, launch geometry and
// the per-device scratch area.  Every step of the computation runs in the HIP
// kernels of kq_gemv.h (instantiated per weight type in kq_gemv_q*.hip) and
// kq_repack.hip.
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/kq.h"
#ifdef KQ_TIMELINE
#include "../../include/kq_timeline.h"
#endif
#include "kq_internal.h"

namespace kq {

int64_t sb_bytes(int type) {
  switch (type) {
    case KQ_Q4_K: return 144;
    case KQ_Q5_K: return 176;
    case KQ_Q6_K: return 210;
    default: return 0;
  }
}


// Workspace of kq_gemv_fused_noalloc, for callers that cannot allocate: one
// copy per GPU in the code object's static memory, held until the process
// ends.  Host code never uses the name `scratch` as an address (on the host it
// is only a stand-in for the symbol): the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is passed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
static_assert(kStaticScratchBytes == KQ_NOALLOC_SCRATCH_BYTES, "kq.h states the static scratch size");
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's `scratch` (looked up on first use).
static int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KQ_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KQ_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KQ_OK;
}

// CUs of the current device (the launch geometry is planned for them).
static int current_device_cus(int* dev_out, int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *cus < 1)
    return KQ_ERR_HIP;
  if (dev_out) *dev_out = dev;
  return KQ_OK;
}

static hipError_t launch_gemv(int type, int xtype, int batch, int nw, bool mf, const GemvArgs& a, int grid,
                              size_t lds, hipStream_t s) {
  switch (type) {
    case KQ_Q4_K: return launch_gemv_type<KQ_Q4_K>(xtype, batch, nw, mf, a, grid, lds, s);
    case KQ_Q5_K: return launch_gemv_type<KQ_Q5_K>(xtype, batch, nw, mf, a, grid, lds, s);
    case KQ_Q6_K: return launch_gemv_type<KQ_Q6_K>(xtype, batch, nw, mf, a, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Wavefronts per workgroup forced by KQ_WG_WAVES (4 or 8), else 0.
static int forced_wg_waves() {
  const char* e = getenv("KQ_WG_WAVES");
  const int x = e ? atoi(e) : 0;
  return (x == 4 || x == 8) ? x : 0;
}

// Tuning knobs, read per call: target wavefronts per CU (KQ_WAVES_PER_CU) and
// wavefronts per workgroup (KQ_WG_WAVES, 4 or 8).  From batch 2 the default is
// one 8-wavefront workgroup per CU, which stages the activations of its columns
// once for all of its wavefronts.  A single launch at batch 1 runs one
// 4-wavefront workgroup per CU with fixed runs: on the 209-launch sweep that is
// about 5% faster than two such workgroups per CU or one of 8 wavefronts (one
// wavefront per SIMD, twice the units per run).  A chain keeps 8 wavefronts per
// CU at every batch (its persistent grid and its steps' plans); so does a single
// launch whose workgroup size KQ_WG_WAVES forces, which then has the shape of a
// chain step with the same setting.
static int waves_per_cu(bool single, int srows, int nw) {
  const char* e = getenv("KQ_WAVES_PER_CU");
  const int x = e ? atoi(e) : 0;
  if (x >= 1 && x <= 32) return x;
  return single && srows == 1 && nw == 4 && !forced_wg_waves() ? 4 : 8;
}


// Whole tiles per workgroup forced for every shape (KQ_ALIGNED_TILES; 0 = automatic).
static int aligned_tiles() {
  const char* e = getenv("KQ_ALIGNED_TILES");
  const int x = e ? atoi(e) : 0;
  return (x >= 1 && x <= 8) ? x : 0;
}

// Units per CU below which a launch gives each workgroup whole tiles (KQ_WHOLE_TILES_BELOW; 0 = never).
static int64_t whole_tiles_below() {
  const char* e = getenv("KQ_WHOLE_TILES_BELOW");
  const long x = e ? atol(e) : 0;
  return (x >= 0 && x <= 4096) ? x : 0;
}

// Extra column windows the planner may add beyond the fewest that fit (KQ_WIN_SEARCH, 0..64; 3 measured
// best on the batch-8 sweep: each extra window adds a piece to every tile's hand-off).
static int64_t window_search() {
  const char* e = getenv("KQ_WIN_SEARCH");
  const long x = e ? atol(e) : 3;
  return (x >= 0 && x <= 64) ? x : 3;
}

// Batches from which column windows are used (KQ_WINDOWS_FROM overrides; 9 = never).
static int windows_from_batch() {
  const char* e = getenv("KQ_WINDOWS_FROM");
  const int x = e ? atoi(e) : 0;
  return (x >= 1 && x <= 9) ? x : 4;
}

// Batches (bf16 activations) from which the matrix cores compute the products
// (KQ_MATRIX_CORES_FROM, 1..9; 9 = never, every batch on the dot2 VALU path).
// The default, 3, is where the dot2 path becomes VALU-issue bound: at batch 2
// it is as fast or faster on every sweep shape, from batch 3 on it is slower.
static int matrix_cores_from() {
  const char* e = getenv("KQ_MATRIX_CORES_FROM");
  const int x = e ? atoi(e) : 0;
  return (x >= 1 && x <= 9) ? x : 3;
}

// Wavefronts per workgroup of a single launch (KQ_WG_WAVES = 4 or 8
// overrides): 4 at batch 1 (one workgroup per CU, see waves_per_cu), 8 above.
static int wg_waves(int batch) {
  const int x = forced_wg_waves();
  return x ? x : batch == 1 ? 4 : 8;
}

// Wavefronts per workgroup of a chain (KQ_WG_WAVES overrides): 8 at every
// batch.  With two 4-wavefront workgroups on a CU the older one's waves win the
// issue arbitration, so the pair ends a step several microseconds apart and the
// CU runs half-empty until the step barrier; at batch 1 the eight wavefronts
// of one workgroup instead take its units one at a time.
static int chain_wg_waves() {
  const int x = forced_wg_waves();
  return x ? x : 8;
}

constexpr size_t kMaxLds = 160 * 1024;   // LDS of one CU

// Argument checks shared by every GEMV entry point and every chain step.
static int validate(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x,
                    int xtype, int64_t ldx, int batch, float* const* y, const int64_t* ldy) {
  if (type != KQ_Q4_K && type != KQ_Q5_K && type != KQ_Q6_K) return KQ_ERR_TYPE;
  if (xtype != KQ_X_F32 && xtype != KQ_X_BF16) return KQ_ERR_TYPE;
  if (batch < 1 || batch > (xtype == KQ_X_F32 ? KQ_MAX_BATCH_F32 : KQ_MAX_BATCH) || n < 1 || n > KQ_MAX_PROJ)
    return KQ_ERR_BATCH;
  if (!w || !rows || !y || !ldy || !x) return KQ_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!w[i] || !y[i]) return KQ_ERR_NULL;
  if (cols <= 0 || cols % 256 != 0 || ldx < cols) return KQ_ERR_SHAPE;
  for (int i = 0; i < n; ++i)
    if (rows[i] < 1 || ldy[i] < rows[i]) return KQ_ERR_SHAPE;
  const int64_t esize = xtype == KQ_X_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * esize) % 16 != 0) return KQ_ERR_ALIGN;
  for (int i = 0; i < n; ++i)
    if (!aligned(w[i], 16) || !aligned(y[i], 4)) return KQ_ERR_ALIGN;
  return KQ_OK;
}

// Launch plan of one GEMV (or multi-projection) call.
struct Plan {
  GemvArgs a;
  int nw;            // wavefronts per workgroup
  bool mf;           // matrix-core path
  int64_t grid;      // workgroups, a multiple of 8
  size_t lds;        // dynamic LDS per workgroup
  int rows;          // staged activation rows: the batch, or twice it for fp32 activations
  int64_t slots;     // partial-sum slots of split tiles
  int slot_floats;   // floats per slot
  bool heads;        // a head-norm segment: the heads' sums of squares follow the slots
  size_t ws_bytes;   // workspace the call needs
};

// Point the plan's workspace arguments into `ws` (layout in kq_internal.h).
static void assign_workspace(Plan& p, uint8_t* ws) {
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
  float* partial = reinterpret_cast<float*>(ws + kCounterBytes);
  p.a.counters = counters;
  p.a.head_ctr = counters + kMaxGroups;
  p.a.partial = partial;
  p.a.head_ss = partial + p.slots * p.slot_floats;
}

// Launch geometry of a validated call on a device with `cus` CUs, using at most
// `max_grid` workgroups (a multiple of 8).
// epi: segment i's epilogue code in bits 4i..4i+3.  KQ_EPI_SWIGLU: one matrix
// (n == 1) from kq_repack_swiglu, rows[0] = the intermediate size, 32 outputs
// per 64-row tile.
static int plan_gemv(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x,
                     int xtype, int64_t ldx, int batch, float* const* y, const int64_t* ldy, void* const* y16,
                     const int64_t* ldy16, int cus,
                     int64_t max_grid, int force_nw, bool single, uint32_t epi, float rms_eps, float head_eps,
                     Plan* out, int64_t whole_below = -1) {
  const int64_t n_cols = cols / 256;
  const bool norm = rms_eps > 0.0f;
  GemvArgs a{};
  a.epi = epi;
  a.rms_eps = rms_eps;
  a.head_eps = head_eps;
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    if (rows[i] > (int64_t)INT32_MAX - 64) return KQ_ERR_RANGE;
    a.w[i] = static_cast<const uint8_t*>(w[i]);
    a.y[i] = y[i];
    a.ldy[i] = ldy[i];
    a.y16[i] = y16 ? static_cast<uint16_t*>(y16[i]) : nullptr;
    a.ldy16[i] = y16 && y16[i] ? ldy16[i] : 0;
    a.rows[i] = (int32_t)rows[i];
    a.tile_begin[i] = (int32_t)tiles;
    tiles += epi == (uint32_t)KQ_EPI_SWIGLU ? (rows[i] + 31) / 32 : (rows[i] + 63) / 64;
    if (tiles > INT32_MAX) return KQ_ERR_RANGE;
  }
  for (int i = n; i <= KQ_MAX_PROJ; ++i) a.tile_begin[i] = (int32_t)tiles;
  bool heads = false;
  for (int i = 0; i < n; ++i) heads |= ((epi >> (4 * i)) & 15u) == (uint32_t)KQ_EPI_HEADNORM;
  if (heads && tiles > kMaxGroups) return KQ_ERR_RANGE;   // the head scratch is indexed by tile
  const int64_t n_units = tiles * n_cols;
  if (n_units + 2 * n_cols + 8 * (int64_t)kMaxGroups >= INT32_MAX) return KQ_ERR_RANGE;
  const int64_t max_groups = max_grid < kMaxGroups ? max_grid : kMaxGroups;

  // An even run of `upw` units per wavefront, about `wpc` wavefronts per CU,
  // nw wavefronts per workgroup.  A workgroup stages the activations
  // (and sub-block sums) of the columns its nw*upw units touch in LDS, within
  // `budget` bytes (64 KiB leaves room for two 4-wavefront workgroups per CU,
  // 112 KiB is for one 8-wavefront workgroup), plus its wavefronts' partial sums.
  // The activations are staged as bf16 rows: the batch, or (fp32 activations)
  // two rows per batch row, hi = bf16(x) and lo = bf16(x - hi).  Every launch
  // decision below is taken on the staged rows.
  const int srows = xtype == KQ_X_F32 ? 2 * batch : batch;
  // above 8 staged rows only the matrix cores with 8-wavefront workgroups are built
  const int nw = srows > 8 ? 8 : force_nw ? force_nw : wg_waves(srows);
  const bool mf = srows >= matrix_cores_from() || srows > 8;
  // staging budget: what is left of the CU's LDS after the tile sums (two tiles
  // per wavefront assumed here; the final size is checked below)
  const int64_t tile_sums = (int64_t)nw * 2 * srows * 64 * sizeof(float);
  int64_t budget = nw == 8 ? 112 * 1024 : 64 * 1024;
  if (budget > (int64_t)kMaxLds - tile_sums - 2048) budget = (int64_t)kMaxLds - tile_sums - 2048;
  const int wpc = waves_per_cu(single, srows, nw);
  const int64_t target = (int64_t)cus * wpc;
  int64_t upw = (n_units + target - 1) / target;
  if (upw < 1) upw = 1;
  const int64_t per_col =
      (int64_t)(gemv_lds_bytes(type, srows, nw, mf, 1, 0, 0, norm) - gemv_lds_bytes(type, srows, nw, mf, 0, 0, 0, norm));
  const int64_t max_cols = budget / per_col;
  if (n_cols > max_cols && nw * upw > max_cols) upw = max_cols / nw > 0 ? max_cols / nw : 1;
  int64_t n_groups = (n_units + nw * upw - 1) / (nw * upw);
  bool even_ok = true;   // even runs fit the staging budget within max_groups workgroups
  if ((n_groups + 7) / 8 * 8 > max_groups) {
    upw = (n_units + nw * (max_groups / 8 * 8) - 1) / (nw * (max_groups / 8 * 8));
    even_ok = !(n_cols > max_cols && nw * upw > max_cols);
    n_groups = (n_units + nw * upw - 1) / (nw * upw);
  }
  int64_t tcols = n_cols < nw * upw ? n_cols : nw * upw;
  int64_t grid = (n_groups + 7) / 8 * 8;  // whole XCD rounds for the block remap

  // Column windows: when a long row does not fit the staging budget, split the
  // columns into n_win windows of at most max_cols and give each workgroup whole
  // tiles of one window, so its staged activations serve several row tiles
  // (worth it where the activations are large next to the weights).
  a.n_win = 1;
  a.n_tiles = (int32_t)tiles;
  a.tiles_per_wg = 0;
  const int64_t n_win = (n_cols + max_cols - 1) / max_cols;
  // small steps (fewer units than `whole_tiles_below()` per CU): one whole tile per workgroup, so no
  // tile is split between workgroups
  const int64_t small = whole_below >= 0 ? whole_below : whole_tiles_below();
  const int forced_r = n_units < (int64_t)cus * small && n_win == 1 ? 1 : aligned_tiles();
  if (((srows >= windows_from_batch() && n_win > 1) || forced_r > 0) && tiles <= kMaxGroups &&
      n_win * tiles <= 2 * (int64_t)kMaxGroups) {
    int64_t g_target = (int64_t)cus * wpc / nw;
    if (g_target < 1) g_target = 1;
    if (g_target > max_groups) g_target = max_groups;
    int64_t nwin = n_win, r = 0, g_win = 0;
    if (forced_r > 0) {
      r = forced_r;
      g_win = (tiles + r - 1) / r;
    } else {
      // the window count (at least n_win, so each window fits the staging budget) and whole tiles per
      // workgroup (at most nw, so a wavefront's run touches at most two tiles) with the least work per
      // CU: rounds of resident workgroups x the units of the largest workgroup; ties go to fewer
      // workgroups, then to fewer windows (fewer pieces per tile to hand over)
      int64_t best = -1, best_groups = 0;
      for (int64_t nwc = n_win; nwc <= n_win + window_search() && nwc <= n_cols; ++nwc) {
        if (nwc * tiles > 2 * (int64_t)kMaxGroups) break;
        const int64_t cols_w = (n_cols + nwc - 1) / nwc;
        for (int64_t rc = 1; rc <= nw; ++rc) {
          const int64_t gw = (tiles + rc - 1) / rc, groups = nwc * gw;
          if ((groups + 7) / 8 * 8 > max_groups) continue;
          const int64_t span = (groups + g_target - 1) / g_target * rc * cols_w;
          if (best < 0 || span < best || (span == best && groups < best_groups)) {
            best = span;
            best_groups = groups;
            nwin = nwc;
            r = rc;
            g_win = gw;
          }
        }
      }
      if (best < 0) {   // no plan within max_groups: the widest tiles per workgroup
        r = (tiles + (max_groups / 8 * 8) / n_win - 1) / ((max_groups / 8 * 8) / n_win);
        g_win = (tiles + r - 1) / r;
      }
    }
    const int64_t wgrid = (nwin * g_win + 7) / 8 * 8;
    if (wgrid <= max_groups) {
      even_ok = true;
      a.n_win = (int32_t)nwin;
      a.win_base = (int32_t)(n_cols / nwin);
      a.win_extra = (int32_t)(n_cols % nwin);
      a.wg_per_win = (int32_t)g_win;
      a.tiles_per_wg = (int32_t)r;
      tcols = a.win_base + (a.win_extra ? 1 : 0);
      grid = wgrid;
    }
  }
  if (!even_ok) return KQ_ERR_RANGE;
  const int64_t wgu = (int64_t)nw * upw;
  a.wgu = (int32_t)wgu;
  a.nproj = n;
  a.n_cols = (int32_t)n_cols;
  a.x = x;
  a.ldx = ldx;
  a.n_units = (int32_t)n_units;
  a.upw = (int32_t)upw;
  a.tsb = (int32_t)tcols;
  out->a = a;
  out->nw = nw;
  out->mf = mf;
  out->grid = grid;
  const int64_t run_units = a.tiles_per_wg > 0 ? (int64_t)a.tiles_per_wg * tcols : wgu;
  // a run of u units starting anywhere in a tile of c columns touches at most
  // ceil((u - 1) / c) + 1 tiles
  if (a.tiles_per_wg > 0) {
    const int64_t uw = ((int64_t)a.tiles_per_wg * (a.win_base + 1) + nw - 1) / nw;
    a.tpw = (int32_t)((uw - 1 + a.win_base - 1) / a.win_base + 1);
  } else {
    a.tpw = (int32_t)((upw - 1 + n_cols - 1) / n_cols + 1);
  }
  out->a.tpw = a.tpw;
  out->lds = gemv_lds_bytes(type, srows, nw, mf, (int)tcols, (int)run_units, a.tpw, norm);
  out->rows = srows;
  if (out->lds > kMaxLds) return KQ_ERR_RANGE;
  // workspace: the counter block, one slot per (workgroup, 0/1) of even runs or per (window, tile), and
  // the heads' sums of squares
  out->slots = a.tiles_per_wg > 0 ? (int64_t)a.n_win * a.n_tiles : 2 * grid;
  out->slot_floats = partial_stride(batch);
  out->heads = heads;
  out->ws_bytes = kCounterBytes + (size_t)out->slots * out->slot_floats * sizeof(float) +
                  (heads ? (size_t)tiles * 2 * KQ_MAX_BATCH * sizeof(float) : 0);
  return KQ_OK;
}

static bool segment_code(int32_t c) {
  return c == KQ_EPI_NONE || c == KQ_EPI_SIGMOID || c == KQ_EPI_RESIDUAL || c == KQ_EPI_HEADNORM;
}

// Packed per-segment epilogue codes are valid: SwiGLU alone on a single matrix,
// else none / sigmoid / residual / head norm on each of the n segments.
static bool valid_epilogue(int n, uint32_t epi) {
  if (epi == (uint32_t)KQ_EPI_SWIGLU) return n == 1;
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = (epi >> (4 * i)) & 15u;
    if (i >= n ? c != 0 : !segment_code((int32_t)c)) return false;
  }
  return true;
}

// Head-norm segments hold whole heads, and their epsilon is finite and > 0.
static int check_heads(int n, const int64_t* rows, uint32_t epi, float head_eps) {
  if (epi == (uint32_t)KQ_EPI_SWIGLU) return KQ_OK;
  bool heads = false;
  for (int i = 0; i < n; ++i) {
    if (((epi >> (4 * i)) & 15u) != (uint32_t)KQ_EPI_HEADNORM) continue;
    heads = true;
    if (rows[i] % kHeadRows != 0) return KQ_ERR_SHAPE;
  }
  if (heads && !(head_eps > 0.0f && head_eps <= FLT_MAX)) return KQ_ERR_SHAPE;
  return KQ_OK;
}

// Optional bf16 copies of the outputs: a row stride >= the segment's outputs, 2-byte aligned.
static int check_y16(int n, const int64_t* rows, void* const* y16, const int64_t* ldy16) {
  if (!y16) return KQ_OK;
  for (int i = 0; i < n; ++i) {
    if (!y16[i]) continue;
    if (!ldy16) return KQ_ERR_NULL;
    if (ldy16[i] < rows[i] || ldy16[i] > ((int64_t)1 << 40)) return KQ_ERR_SHAPE;
    if (!aligned(y16[i], 2)) return KQ_ERR_ALIGN;
  }
  return KQ_OK;
}

// The weight-less RMSNorm's epsilon: 0 (no normalisation) or finite and > 0.
static bool valid_rms_eps(float e) { return e == 0.0f || (e > 0.0f && e <= FLT_MAX); }

// Host-side checks of one call's arguments (every GEMV entry point).
static int validate_call(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x,
                         int xtype, int64_t ldx, int batch, float* const* y, const int64_t* ldy, uint32_t epi,
                         float rms_eps, float head_eps, void* const* y16, const int64_t* ldy16) {
  int rc = validate(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy);
  if (rc != KQ_OK) return rc;
  rc = check_y16(n, rows, y16, ldy16);
  if (rc != KQ_OK) return rc;
  if (!valid_epilogue(n, epi)) return KQ_ERR_TYPE;
  if (!valid_rms_eps(rms_eps)) return KQ_ERR_SHAPE;
  return check_heads(n, rows, epi, head_eps);
}

// Validate one call and plan it for the current device (every GEMV entry point
// and the workspace query).
static int plan_call(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x,
                     int xtype, int64_t ldx, int batch, float* const* y, const int64_t* ldy, uint32_t epi,
                     float rms_eps, float head_eps, void* const* y16, const int64_t* ldy16, Plan* p) {
  int rc = validate_call(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, epi, rms_eps, head_eps, y16, ldy16);
  if (rc != KQ_OK) return rc;
  int cus = 0;
  rc = current_device_cus(nullptr, &cus);
  if (rc != KQ_OK) return rc;
  rc = plan_gemv(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, y16, ldy16, cus, kMaxGroups, 0, true, epi,
                 rms_eps, head_eps, p);
  // too many units per 8-wavefront workgroup: 4-wavefront runs
  if (rc == KQ_ERR_RANGE && wg_waves(xtype == KQ_X_F32 ? 2 * batch : batch) == 8)
    rc = plan_gemv(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, y16, ldy16, cus, kMaxGroups, 4, true, epi,
                   rms_eps, head_eps, p);
  return rc;
}

static int gemv_impl(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x,
                     int xtype, int64_t ldx, int batch, float* const* y, const int64_t* ldy, void* ws,
                     size_t ws_bytes, void* stream, uint32_t epi = KQ_EPI_NONE, float rms_eps = 0.0f,
                     float head_eps = 0.0f, void* const* y16 = nullptr, const int64_t* ldy16 = nullptr) {
  int rc = validate_call(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, epi, rms_eps, head_eps, y16, ldy16);
  if (rc != KQ_OK) return rc;
  if (!ws || !aligned(ws, 16)) return KQ_ERR_WORKSPACE;
  Plan p{};
  rc = plan_call(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, epi, rms_eps, head_eps, y16, ldy16, &p);
  if (rc != KQ_OK) return rc;
  if (ws_bytes < p.ws_bytes) return KQ_ERR_WORKSPACE;
  assign_workspace(p, static_cast<uint8_t*>(ws));
  if (launch_gemv(type, xtype, p.rows, p.nw, p.mf, p.a, (int)p.grid, p.lds, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
}

// ---------------------------------------------------------------- chains

// `rows`: staged activation rows (the batch, or twice it for fp32 activations).
static hipError_t launch_chain(int xtype, int rows, const ChainArgs& c, int nw, bool mf, int grid, size_t lds,
                               hipStream_t s, int* occupancy) {
  if (xtype == KQ_X_F32) {
    switch (rows) {
      case 2: return launch_chain_b<2, true>(c, nw, mf, grid, lds, s, occupancy);
      case 4: return launch_chain_b<4, true>(c, nw, mf, grid, lds, s, occupancy);
      case 6: return launch_chain_b<6, true>(c, nw, mf, grid, lds, s, occupancy);
      case 8: return launch_chain_b<8, true>(c, nw, mf, grid, lds, s, occupancy);
      default: break;
    }
    if (!mf || nw != 8) return hipErrorInvalidValue;
    switch (rows) {
      case 10: return launch_chain_wide<10, true>(c, grid, lds, s, occupancy);
      case 12: return launch_chain_wide<12, true>(c, grid, lds, s, occupancy);
      case 14: return launch_chain_wide<14, true>(c, grid, lds, s, occupancy);
      case 16: return launch_chain_wide<16, true>(c, grid, lds, s, occupancy);
      default: return hipErrorInvalidValue;
    }
  }
  switch (rows) {
#define KQ_CHAIN_CASE(B) \
  case B: return launch_chain_b<B, false>(c, nw, mf, grid, lds, s, occupancy);
    KQ_CHAIN_CASE(1) KQ_CHAIN_CASE(2) KQ_CHAIN_CASE(3) KQ_CHAIN_CASE(4)
    KQ_CHAIN_CASE(5) KQ_CHAIN_CASE(6) KQ_CHAIN_CASE(7) KQ_CHAIN_CASE(8)
#undef KQ_CHAIN_CASE
    default: break;
  }
  if (!mf || nw != 8) return hipErrorInvalidValue;
  switch (rows) {
#define KQ_CHAIN_WIDE(B) \
  case B: return launch_chain_wide<B, false>(c, grid, lds, s, occupancy);
    KQ_CHAIN_WIDE(9) KQ_CHAIN_WIDE(10) KQ_CHAIN_WIDE(11) KQ_CHAIN_WIDE(12)
    KQ_CHAIN_WIDE(13) KQ_CHAIN_WIDE(14) KQ_CHAIN_WIDE(15) KQ_CHAIN_WIDE(16)
#undef KQ_CHAIN_WIDE
    default: return hipErrorInvalidValue;
  }
}

// One planned unit of a chain: a step, or the segments of one weight type of a
// step with mixed types.  `wait`: the first sub-step of a step waits at the step
// barrier; the others share its x and run without waiting.
struct SubStep {
  int type = 0, n = 0;
  int64_t cols = 0, ldx = 0;
  const void* x = nullptr;
  const void* w[KQ_MAX_PROJ] = {};
  int64_t rows[KQ_MAX_PROJ] = {};
  float* y[KQ_MAX_PROJ] = {};
  int64_t ldy[KQ_MAX_PROJ] = {};
  void* y16[KQ_MAX_PROJ] = {};
  int64_t ldy16[KQ_MAX_PROJ] = {};
  uint32_t epi = 0;
  float rms_eps = 0.0f, head_eps = 0.0f;
  bool wait = true;
  int step = 0;          // index of the chain step it belongs to
  bool overlap = false;  // the step carries KQ_STEP_OVERLAP
  bool overlapped = false;  // ... and skips the step barrier (mark_overlaps)
};

// Split a chain step into one sub-step per weight type (segment i's type is
// types[i], or the step's type where that is 0), in the order the types first
// appear; each sub-step keeps its segments' order and epilogue codes.
static int split_by_type(const kq_chain_step& st, std::vector<SubStep>& out) {
  if (!valid_epilogue(st.n, (uint32_t)st.epilogue)) return KQ_ERR_TYPE;
  int seg_type[KQ_MAX_PROJ], order[3], nt = 0;
  for (int i = 0; i < st.n; ++i) {
    seg_type[i] = st.types[i] ? st.types[i] : st.type;
    if (!sb_bytes(seg_type[i])) return KQ_ERR_TYPE;
    bool seen = false;
    for (int k = 0; k < nt; ++k) seen |= order[k] == seg_type[i];
    if (!seen) order[nt++] = seg_type[i];
  }
  const bool swiglu = (uint32_t)st.epilogue == (uint32_t)KQ_EPI_SWIGLU;
  for (int g = 0; g < nt; ++g) {
    SubStep u;
    u.type = order[g];
    u.cols = st.cols;
    u.x = st.x;
    u.ldx = st.ldx;
    u.rms_eps = st.rms_eps;
    u.head_eps = st.head_eps;
    u.wait = g == 0;
    u.overlap = (st.flags & KQ_STEP_OVERLAP) != 0;
    for (int i = 0; i < st.n; ++i) {
      if (seg_type[i] != u.type) continue;
      const int k = u.n++;
      u.w[k] = st.w[i];
      u.rows[k] = st.rows[i];
      u.y[k] = st.y[i];
      u.ldy[k] = st.ldy[i];
      u.y16[k] = st.y16[i];
      u.ldy16[k] = st.ldy16[i];
      u.epi |= swiglu ? (uint32_t)KQ_EPI_SWIGLU : (((uint32_t)st.epilogue >> (4 * i)) & 15u) << (4 * k);
    }
    out.push_back(u);
  }
  return KQ_OK;
}

// Polls before a chain step's wait gives up (KQ_CHAIN_SPIN overrides; about a
// second at the default).
static uint32_t chain_spin() {
  const char* e = getenv("KQ_CHAIN_SPIN");
  if (e) {
    const long v = atol(e);
    if (v >= 0 && v <= 0x7fffffffL) return (uint32_t)v;
  }
  return 1u << 20;
}

}  // namespace kq

struct kq_chain {
  int dev = 0;
  int xtype = 0, rows = 0, nw = 4;   // rows: staged activation rows (2 x batch for fp32 activations)
  bool mf = false;
  int grid = 0;
  size_t lds = 0;
  kq::ChainArgs args{};
  void* mem = nullptr;          // one allocation: step table, control words, the steps' workspace
  uint32_t* counters = nullptr; // the workspace (its counter blocks are reset after a run whose wait gave up)
  size_t ws_bytes = 0;
  uint32_t* flag = nullptr;     // pinned host word, set by the device when a wait gives up
  size_t tl_bytes = 0;          // timeline builds: the clock stamps after the workspace
  std::vector<uint8_t> waits;   // per chain step: 1 if it waits at the step barrier
};

using namespace kq;

extern "C" {

int kq_abi_version(void) { return KQ_ABI_VERSION; }

const char* kq_status_str(int status) {
  switch (status) {
    case KQ_OK: return "ok";
    case KQ_ERR_NULL: return "null pointer argument";
    case KQ_ERR_SHAPE: return "invalid shape or stride";
    case KQ_ERR_ALIGN: return "misaligned pointer or stride";
    case KQ_ERR_BATCH: return "batch or projection count out of range";
    case KQ_ERR_TYPE: return "unknown weight or activation format";
    case KQ_ERR_HIP: return "HIP runtime error";
    case KQ_ERR_NOMEM: return "device allocation failed";
    case KQ_ERR_RANGE: return "problem too large";
    case KQ_ERR_TIMEOUT: return "a chain step's wait for the previous step gave up";
    case KQ_ERR_DEVICE: return "chain run on another device than the one it was made on";
    case KQ_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than the call needs";
    default: return "unknown status";
  }
}

int kq_init(int device) {
  int n = 0, cus = 0, prev = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return KQ_ERR_DEVICE;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
    return KQ_ERR_HIP;
  // look up this device's static scratch now, with the device current
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess) return KQ_ERR_HIP;
  void* p = nullptr;
  const int rc = static_scratch(&p);
  (void)hipSetDevice(prev);
  return rc;
}

size_t kq_gemv_workspace_bytes(int type, int n, const int64_t* rows, int64_t cols, int xtype, int batch,
                               const int32_t* epi, float rms_eps) {
  if (n < 1 || n > KQ_MAX_PROJ || !rows) return 0;
  // the plan depends on shapes and options only; stand-in pointers pass validation
  const void* w[KQ_MAX_PROJ];
  float* y[KQ_MAX_PROJ];
  int64_t ldy[KQ_MAX_PROJ];
  for (int i = 0; i < n; ++i) {
    w[i] = reinterpret_cast<const void*>((uintptr_t)256);
    y[i] = reinterpret_cast<float*>((uintptr_t)256);
    ldy[i] = rows[i];
  }
  uint32_t packed = 0;
  if (epi) {
    if (n == 1 && epi[0] == KQ_EPI_SWIGLU) packed = KQ_EPI_SWIGLU;
    else
      for (int i = 0; i < n; ++i) packed |= ((uint32_t)epi[i] & 15u) << (4 * i);
  }
  Plan p{};
  // head-norm segments need a valid epsilon to plan; its value does not change the plan
  if (plan_call(type, n, w, rows, cols, reinterpret_cast<const void*>((uintptr_t)256), xtype, cols, batch, y, ldy,
                packed, rms_eps, 1.0f, nullptr, nullptr, &p) != KQ_OK)
    return 0;
  return p.ws_bytes;
}

int kq_workspace_init(void* ws, size_t bytes, void* stream) {
  if (!ws) return KQ_ERR_NULL;
  if (!aligned(ws, 16) || bytes < kCounterBytes) return KQ_ERR_WORKSPACE;
  if (launch_zero_words(static_cast<uint32_t*>(ws), kCounterBytes / 4, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
}

size_t kq_repacked_bytes(int type, int64_t rows, int64_t cols) {
  const int64_t sbb = sb_bytes(type);
  if (!sbb || rows < 1 || cols <= 0 || cols % 256 != 0) return 0;
  const int64_t tiles = (rows + 63) / 64;
  return (size_t)(tiles * (cols / 256) * 64 * sbb);
}

int kq_repack(int type, int64_t rows, int64_t cols, const void* gguf, void* out, void* stream) {
  if (!sb_bytes(type)) return KQ_ERR_TYPE;
  if (!gguf || !out) return KQ_ERR_NULL;
  if (rows < 1 || cols <= 0 || cols % 256 != 0) return KQ_ERR_SHAPE;
  if (!aligned(out, 16) || !aligned(gguf, type == KQ_Q6_K ? 2 : 4)) return KQ_ERR_ALIGN;
  if (rows > (int64_t)INT32_MAX - 64 || cols / 256 > INT32_MAX) return KQ_ERR_RANGE;
  if (launch_repack(type, rows, cols, gguf, nullptr, out, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
}

int kq_repack_swiglu(int type, int64_t inter, int64_t cols, const void* gate, const void* up, void* out,
                     void* stream) {
  if (!sb_bytes(type)) return KQ_ERR_TYPE;
  if (!gate || !up || !out) return KQ_ERR_NULL;
  if (inter < 1 || cols <= 0 || cols % 256 != 0) return KQ_ERR_SHAPE;
  const int align = type == KQ_Q6_K ? 2 : 4;
  if (!aligned(out, 16) || !aligned(gate, align) || !aligned(up, align)) return KQ_ERR_ALIGN;
  if (inter > (int64_t)INT32_MAX / 2 - 64 || cols / 256 > INT32_MAX) return KQ_ERR_RANGE;
  if (launch_repack(type, inter, cols, gate, up, out, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
}

int kq_gemv_fused(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x, int xtype,
                  int64_t ldx, int batch, float* const* y, const int64_t* ldy, void* const* y16, const int64_t* ldy16,
                  const int32_t* epi, float rms_eps, float head_eps, void* ws, size_t ws_bytes, void* stream) {
  if (n < 1 || n > KQ_MAX_PROJ) return KQ_ERR_BATCH;
  uint32_t packed = 0;
  if (epi) {
    if (n == 1 && epi[0] == KQ_EPI_SWIGLU) {
      packed = KQ_EPI_SWIGLU;
      if (rows && rows[0] > (int64_t)INT32_MAX / 2 - 64) return KQ_ERR_RANGE;
    } else {
      for (int i = 0; i < n; ++i) {
        if (!segment_code(epi[i])) return KQ_ERR_TYPE;
        packed |= (uint32_t)epi[i] << (4 * i);
      }
    }
  }
  return gemv_impl(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, ws, ws_bytes, stream, packed, rms_eps,
                   head_eps, y16, ldy16);
}

int kq_gemv_fused_noalloc(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x,
                          int xtype, int64_t ldx, int batch, float* const* y, const int64_t* ldy,
                          void* const* y16, const int64_t* ldy16, const int32_t* epi, float rms_eps, float head_eps,
                          void* stream) {
  if (n < 1 || n > KQ_MAX_PROJ) return KQ_ERR_BATCH;
  uint32_t packed = 0;
  if (epi) {
    if (n == 1 && epi[0] == KQ_EPI_SWIGLU) {
      packed = KQ_EPI_SWIGLU;
      if (rows && rows[0] > (int64_t)INT32_MAX / 2 - 64) return KQ_ERR_RANGE;
    } else {
      for (int i = 0; i < n; ++i) {
        if (!segment_code(epi[i])) return KQ_ERR_TYPE;
        packed |= (uint32_t)epi[i] << (4 * i);
      }
    }
  }
  int rc = validate_call(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, packed, rms_eps, head_eps, y16,
                         ldy16);
  if (rc != KQ_OK) return rc;
  Plan p{};
  rc = plan_call(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, packed, rms_eps, head_eps, y16, ldy16, &p);
  if (rc != KQ_OK) return rc;
  if (p.ws_bytes > kStaticScratchBytes) return KQ_ERR_WORKSPACE;   // beyond the static scratch: refused
  void* ws = nullptr;
  rc = static_scratch(&ws);
  if (rc != KQ_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the previous call on this GPU left the counters zero; clear them anyway (a kernel, not a memset node)
  if (launch_zero_words(static_cast<uint32_t*>(ws), kCounterBytes / 4, s) != hipSuccess) return KQ_ERR_HIP;
  assign_workspace(p, static_cast<uint8_t*>(ws));
  if (launch_gemv(type, xtype, p.rows, p.nw, p.mf, p.a, (int)p.grid, p.lds, s) != hipSuccess) return KQ_ERR_HIP;
  return KQ_OK;
}

int kq_gemv_swiglu(int type, const void* w, int64_t inter, int64_t cols, const void* x, int xtype, int64_t ldx,
                   int batch, float* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  if (inter > (int64_t)INT32_MAX / 2 - 64) return KQ_ERR_RANGE;
  return gemv_impl(type, 1, &w, &inter, cols, x, xtype, ldx, batch, &y, &ldy, ws, ws_bytes, stream, KQ_EPI_SWIGLU);
}

int kq_gemv_q4k(const void* w, int64_t rows, int64_t cols, const void* x, int xtype, int64_t ldx, int batch,
                float* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return gemv_impl(KQ_Q4_K, 1, &w, &rows, cols, x, xtype, ldx, batch, &y, &ldy, ws, ws_bytes, stream);
}

int kq_gemv_q5k(const void* w, int64_t rows, int64_t cols, const void* x, int xtype, int64_t ldx, int batch,
                float* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return gemv_impl(KQ_Q5_K, 1, &w, &rows, cols, x, xtype, ldx, batch, &y, &ldy, ws, ws_bytes, stream);
}

int kq_gemv_q6k(const void* w, int64_t rows, int64_t cols, const void* x, int xtype, int64_t ldx, int batch,
                float* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return gemv_impl(KQ_Q6_K, 1, &w, &rows, cols, x, xtype, ldx, batch, &y, &ldy, ws, ws_bytes, stream);
}

int kq_gemv_multi(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x, int xtype,
                  int64_t ldx, int batch, float* const* y, const int64_t* ldy, void* ws, size_t ws_bytes,
                  void* stream) {
  return gemv_impl(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, ws, ws_bytes, stream);
}

int kq_stream_read(const void* p, size_t bytes, uint32_t* sink, void* stream) {
  if (!p || !sink) return KQ_ERR_NULL;
  if (!aligned(p, 16) || !aligned(sink, 4) || bytes % 16 != 0) return KQ_ERR_ALIGN;
  if (bytes == 0) return KQ_OK;
  int cus = 0;
  if (current_device_cus(nullptr, &cus) != KQ_OK) return KQ_ERR_HIP;
  // workgroups of 4 wavefronts per CU (KQ_READ_WG_PER_CU overrides, 1..32)
  const char* e = getenv("KQ_READ_WG_PER_CU");
  const int per_cu = e && atoi(e) >= 1 && atoi(e) <= 32 ? atoi(e) : 16;
  if (launch_stream_read(p, bytes, sink, cus * per_cu, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
}

int kq_dequant(int type, const void* w, int64_t rows, int64_t cols, float* out, int64_t ldo, void* stream) {
  if (!sb_bytes(type)) return KQ_ERR_TYPE;
  if (!w || !out) return KQ_ERR_NULL;
  if (rows < 1 || cols <= 0 || cols % 256 != 0 || ldo < cols) return KQ_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(out, 4)) return KQ_ERR_ALIGN;
  if (rows > (int64_t)INT32_MAX - 64 || cols / 256 > INT32_MAX) return KQ_ERR_RANGE;
  if (launch_dequant(type, w, rows, cols, out, ldo, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
}

int kq_gather_rows(int type, const void* w, int64_t rows, int64_t cols, const int32_t* ids, int64_t n, float* out,
                   int64_t ldo, void* stream) {
  if (!sb_bytes(type)) return KQ_ERR_TYPE;
  if (n < 0 || n > INT32_MAX) return KQ_ERR_BATCH;
  if (!w || (n > 0 && (!ids || !out))) return KQ_ERR_NULL;
  if (rows < 1 || cols <= 0 || cols % 256 != 0 || ldo < cols) return KQ_ERR_SHAPE;
  if (!aligned(w, 16) || (n > 0 && (!aligned(out, 4) || !aligned(ids, 4)))) return KQ_ERR_ALIGN;
  if (rows > (int64_t)INT32_MAX - 64 || cols / 256 > INT32_MAX) return KQ_ERR_RANGE;
  if (n == 0) return KQ_OK;
  if (launch_gather(type, w, rows, cols, ids, n, out, ldo, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
}

static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Byte ranges a sub-step reads (x) and writes (y, y16), batch rows included.
struct ByteRange {
  uintptr_t lo, hi;
};
static bool meets(const ByteRange& a, const ByteRange& b) { return a.lo < b.hi && b.lo < a.hi; }
static ByteRange x_range(const SubStep& u, int batch, int64_t esize) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(u.x);
  return {p, p + (uintptr_t)(((int64_t)(batch - 1) * u.ldx + u.cols) * esize)};
}
static void out_ranges(const SubStep& u, int batch, std::vector<ByteRange>& out) {
  for (int i = 0; i < u.n; ++i) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(u.y[i]);
    out.push_back({p, p + (uintptr_t)(((int64_t)(batch - 1) * u.ldy[i] + u.rows[i]) * 4)});
    if (u.y16[i]) {
      const uintptr_t q = reinterpret_cast<uintptr_t>(u.y16[i]);
      out.push_back({q, q + (uintptr_t)(((int64_t)(batch - 1) * u.ldy16[i] + u.rows[i]) * 2)});
    }
  }
}

// Largest workspace of one run of overlapping steps (their regions are disjoint).
constexpr size_t kMaxOverlapWorkspace = (size_t)512 << 20;
// Units per CU below which a step that skips the barrier takes whole tiles per workgroup.  Measured on
// the sweep's 209 GEMVs overlapped (QKV 5.6 and O 5.0 units per CU, the rest 38 or more): B = 1
// 3.00-3.01 ms against 3.19-3.25 ms with split tiles, B = 8 4.30-4.32 against 4.57-4.59 ms; 40 (down
// too) gave the same.
constexpr int64_t kOverlapWholeTilesBelow = 8;

// Which steps skip the step barrier.  The steps that may still be running when
// a step starts are those since the last step that waited (a wait orders a
// step after every earlier one).  A step with KQ_STEP_OVERLAP skips its wait
// unless its x meets an output of one of them, or one of its outputs meets
// their x or outputs (read after write, write after read, write after write),
// or the run's workspace regions would pass kMaxOverlapWorkspace.  The sub-steps
// of one step (one per weight type) go together: only the first can wait.
static void mark_overlaps(std::vector<SubStep>& subs, const std::vector<Plan>& plans, int batch, int64_t esize) {
  std::vector<ByteRange> run_x, run_out;   // buffers of the steps that may still be running
  size_t run_ws = 0;
  const int n_sub = (int)subs.size();
  for (int f = 0; f < n_sub;) {
    int l = f;
    while (l + 1 < n_sub && subs[l + 1].step == subs[f].step) ++l;
    std::vector<ByteRange> xs, outs;
    size_t ws = 0;
    for (int k = f; k <= l; ++k) {
      xs.push_back(x_range(subs[k], batch, esize));
      out_ranges(subs[k], batch, outs);
      ws += round_up(plans[k].ws_bytes, 256);
    }
    bool free_to_run = f > 0 && subs[f].overlap && run_ws + ws <= kMaxOverlapWorkspace;
    for (const ByteRange& o : outs) {
      for (const ByteRange& r : run_x) free_to_run &= !meets(o, r);
      for (const ByteRange& r : run_out) free_to_run &= !meets(o, r);
    }
    for (const ByteRange& x : xs)
      for (const ByteRange& r : run_out) free_to_run &= !meets(x, r);
    if (!free_to_run) {
      run_x.clear();
      run_out.clear();
      run_ws = 0;
    }
    subs[f].wait = !free_to_run;
    for (int k = f; k <= l; ++k) subs[k].overlapped = free_to_run;
    run_x.insert(run_x.end(), xs.begin(), xs.end());
    run_out.insert(run_out.end(), outs.begin(), outs.end());
    run_ws += ws;
    f = l + 1;
  }
}

int kq_chain_create(int n_steps, const kq_chain_step* steps, int xtype, int batch, kq_chain** out) {
  if (!out) return KQ_ERR_NULL;
  *out = nullptr;
  if (n_steps < 1 || n_steps > (1 << 16)) return KQ_ERR_BATCH;
  if (!steps) return KQ_ERR_NULL;
  if (xtype != KQ_X_F32 && xtype != KQ_X_BF16) return KQ_ERR_TYPE;
  if (batch < 1 || batch > (xtype == KQ_X_F32 ? KQ_MAX_BATCH_F32 : KQ_MAX_BATCH)) return KQ_ERR_BATCH;
  const int64_t esize = xtype == KQ_X_F32 ? 4 : 2;
  // A step whose segments have different weight types becomes one sub-step per type (the segments of
  // that type, in order, with their epilogue codes): the sub-steps share the step's x and write
  // different outputs, so the later ones run without waiting for the earlier ones.
  std::vector<SubStep> subs;
  for (int j = 0; j < n_steps; ++j) {
    const kq_chain_step& st = steps[j];
    if (st.n < 1 || st.n > KQ_MAX_PROJ) return KQ_ERR_BATCH;
    if (st.flags & ~KQ_STEP_OVERLAP) return KQ_ERR_SHAPE;
    const size_t first_sub = subs.size();
    int rc = split_by_type(st, subs);
    if (rc != KQ_OK) return rc;
    for (size_t k = first_sub; k < subs.size(); ++k) subs[k].step = j;
  }
  for (const SubStep& u : subs) {
    const int rc = validate(u.type, u.n, u.w, u.rows, u.cols, u.x, xtype, u.ldx, batch, u.y, u.ldy);
    if (rc != KQ_OK) return rc;
    if (!valid_epilogue(u.n, u.epi)) return KQ_ERR_TYPE;
    if (!valid_rms_eps(u.rms_eps)) return KQ_ERR_SHAPE;
    const int hrc = check_heads(u.n, u.rows, u.epi, u.head_eps);
    if (hrc != KQ_OK) return hrc;
    const int yrc = check_y16(u.n, u.rows, u.y16, u.ldy16);
    if (yrc != KQ_OK) return yrc;
    if (((int64_t)(batch - 1) * u.ldx + u.cols) * esize >= ((int64_t)1 << 31)) return KQ_ERR_RANGE;
  }
  const int n_sub = (int)subs.size();
  int dev = 0, cus = 0;
  if (current_device_cus(&dev, &cus) != KQ_OK) return KQ_ERR_HIP;

  // Persistent grid: the designed workgroups per CU (two of 4 wavefronts, one
  // of 8), fewer if the occupancy of the chain kernel says so.
  kq_chain* c = new (std::nothrow) kq_chain;
  if (!c) return KQ_ERR_NOMEM;
  std::vector<Plan> plans(n_sub);
  const int srows = xtype == KQ_X_F32 ? 2 * batch : batch;
  int nw = chain_wg_waves();
  auto plan_all = [&](int64_t max_grid, size_t* lds) {
    *lds = 0;
    for (int j = 0; j < n_sub; ++j) {
      const SubStep& u = subs[j];
      int rc = plan_gemv(u.type, u.n, u.w, u.rows, u.cols, u.x, xtype, u.ldx, batch, u.y, u.ldy, u.y16, u.ldy16,
                         cus, max_grid, nw, false, u.epi, u.rms_eps, u.head_eps, &plans[j]);
      if (rc == KQ_ERR_RANGE && nw == 8 && srows <= 8) {   // every step then runs with 4-wavefront workgroups
        nw = 4;
        return (int)KQ_ERR_RANGE;
      }
      if (rc != KQ_OK) return rc;
      if (plans[j].lds > *lds) *lds = plans[j].lds;
    }
    return (int)KQ_OK;
  };
  // Every step is planned as its single launch would be; the persistent grid
  // (one 8-wavefront or two 4-wavefront workgroups per CU, fewer if the
  // occupancy says so) walks each step's logical blocks grid-stride.
  size_t lds = 0;
  int rc = plan_all(kMaxGroups, &lds);
  if (rc == KQ_ERR_RANGE && nw == 4 && srows <= 8) rc = plan_all(kMaxGroups, &lds);
  // Steps that skip the barrier and have fewer than kOverlapWholeTilesBelow units per CU take one
  // whole tile per workgroup: no tile is split, so no hand-off (partials, arrival counter, the last
  // arriver's reads) delays the workgroup's next step.  The step then streams on fewer CUs, which costs
  // nothing here since the other CUs run other steps meanwhile.  The workspace regions only shrink, so
  // the overlap decisions stand.
  if (rc == KQ_OK) {
    mark_overlaps(subs, plans, batch, esize);
    const int64_t whole = whole_tiles_below() > kOverlapWholeTilesBelow ? whole_tiles_below()
                                                                          : kOverlapWholeTilesBelow;
    for (int j = 0; j < n_sub && rc == KQ_OK; ++j) {
      const SubStep& u = subs[j];
      if (!u.overlapped) continue;
      rc = plan_gemv(u.type, u.n, u.w, u.rows, u.cols, u.x, xtype, u.ldx, batch, u.y, u.ldy, u.y16, u.ldy16,
                     cus, kMaxGroups, nw, false, u.epi, u.rms_eps, u.head_eps, &plans[j], whole);
      if (rc == KQ_OK && plans[j].lds > lds) lds = plans[j].lds;
    }
  }
  int64_t groups = (int64_t)cus * (8 / nw);
  int occ = 0;
  if (rc == KQ_OK &&
      launch_chain(xtype, srows, ChainArgs{}, nw, plans[0].mf, 0, lds, nullptr, &occ) != hipSuccess)
    rc = KQ_ERR_HIP;
  if (rc == KQ_OK && occ < 1) rc = KQ_ERR_RANGE;
  if (rc == KQ_OK && (int64_t)occ * cus < groups) {
    groups = (int64_t)occ * cus / 8 * 8;
    if (groups < 8) rc = KQ_ERR_RANGE;
  }
  if (rc != KQ_OK) {
    delete c;
    return rc;
  }

  const size_t steps_bytes = round_up((size_t)n_sub * sizeof(ChainStep), 256);
  // control words: arrive[n_sub][groups], done[n_sub][kDoneReplicas][16] (one 64-byte line per replica),
  // epoch, error
  const size_t ctl_bytes =
      round_up(((size_t)n_sub * (groups + kDoneReplicas * 16) + 2) * sizeof(uint32_t), 256);
  // Steps run one after another and share one workspace; the sub-steps of one step may run at the
  // same time, so each has its own region of it: the workspace is the largest step's sum of regions.
  std::vector<size_t> ws_off(n_sub);
  size_t ws_bytes = kCounterBytes;
  for (int j = 0; j < n_sub;) {
    size_t off = 0;
    int k = j;
    for (; k < n_sub && (k == j || !subs[k].wait); ++k) {
      ws_off[k] = off;
      off += round_up(plans[k].ws_bytes, 256);
    }
    ws_bytes = off > ws_bytes ? off : ws_bytes;
    j = k;
  }
#ifdef KQ_TIMELINE
  const size_t tl_bytes = (size_t)n_sub * groups * 8 * sizeof(uint64_t);
#else
  const size_t tl_bytes = 0;
#endif
  const size_t total = steps_bytes + ctl_bytes + ws_bytes + tl_bytes;
  if (hipMalloc(&c->mem, total) != hipSuccess) {
    delete c;
    return KQ_ERR_NOMEM;
  }
  if (hipHostMalloc(reinterpret_cast<void**>(&c->flag), sizeof(uint32_t),
                    hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
    (void)hipFree(c->mem);
    delete c;
    return KQ_ERR_NOMEM;
  }
  *reinterpret_cast<volatile uint32_t*>(c->flag) = 0;
  uint32_t* d_flag = nullptr;
  uint8_t* base = static_cast<uint8_t*>(c->mem);
  ChainStep* d_steps = reinterpret_cast<ChainStep*>(base);
  uint32_t* d_ctl = reinterpret_cast<uint32_t*>(base + steps_bytes);
  uint8_t* d_ws = base + steps_bytes + ctl_bytes;
  std::vector<ChainStep> h(n_sub);
  for (int j = 0; j < n_sub; ++j) {
    assign_workspace(plans[j], d_ws + ws_off[j]);
    h[j].a = plans[j].a;
    h[j].type = subs[j].type;
    h[j].grid = (int32_t)plans[j].grid;
    h[j].wait = subs[j].wait ? 1 : 0;
    h[j].gate = subs[j].wait ? j : j == 0 ? 0 : h[j - 1].gate;
    // a further weight type of a step starts on the workgroups after those of the types before it
    h[j].first = subs[j].wait || j == 0 ? 0 : (int32_t)(((int64_t)h[j - 1].first + h[j - 1].grid) % groups / 8 * 8);
  }
  rc = KQ_OK;
  if (hipHostGetDevicePointer(reinterpret_cast<void**>(&d_flag), c->flag, 0) != hipSuccess ||
      hipMemcpy(d_steps, h.data(), (size_t)n_sub * sizeof(ChainStep), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(d_ctl, 0, ctl_bytes) != hipSuccess || hipMemset(d_ws, 0, ws_bytes + tl_bytes) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess)
    rc = KQ_ERR_HIP;
  if (rc != KQ_OK) {
    (void)hipFree(c->mem);
    (void)hipHostFree(c->flag);
    delete c;
    return rc;
  }
  c->dev = dev;
  c->xtype = xtype;
  c->rows = srows;
  c->nw = nw;
  c->mf = plans[0].mf;
  c->grid = (int)groups;
  c->lds = lds;
  c->counters = reinterpret_cast<uint32_t*>(d_ws);
  c->ws_bytes = ws_bytes;
  c->args.steps = d_steps;
  c->args.n_steps = n_sub;
  uint32_t* d_done = d_ctl + (size_t)n_sub * groups;
  c->args.ctl = ChainCtl{d_ctl, d_done, d_done + (size_t)n_sub * kDoneReplicas * 16,
                         d_done + (size_t)n_sub * kDoneReplicas * 16 + 1, d_flag,
                         tl_bytes ? reinterpret_cast<uint64_t*>(d_ws + ws_bytes) : nullptr, (uint32_t)groups, 0};
  c->tl_bytes = tl_bytes;
  c->waits.assign(n_steps, 0);
  for (const SubStep& u : subs)
    if (u.wait) c->waits[u.step] = 1;
  *out = c;
  return KQ_OK;
}

int kq_chain_run(kq_chain* c, void* stream) {
  if (!c) return KQ_ERR_NULL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
  if (dev != c->dev) return KQ_ERR_DEVICE;
  // an earlier run's wait gave up: its results were invalid and the chain's counters may be
  // inconsistent; nothing runs until kq_chain_status has reset the chain
  if (*reinterpret_cast<volatile uint32_t*>(c->flag)) return KQ_ERR_TIMEOUT;
  ChainArgs args = c->args;
  args.ctl.spin = chain_spin();
  if (launch_chain(c->xtype, c->rows, args, c->nw, c->mf, c->grid, c->lds, static_cast<hipStream_t>(stream),
                   nullptr) != hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
}

#ifdef KQ_TIMELINE
int kq_chain_timeline(kq_chain* c, uint64_t* host, size_t bytes, int* groups, int* n_sub) {
  if (!c || !host || !groups || !n_sub) return KQ_ERR_NULL;
  if (bytes < c->tl_bytes) return KQ_ERR_SHAPE;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(c->dev) != hipSuccess) return KQ_ERR_HIP;
  const bool ok = hipDeviceSynchronize() == hipSuccess &&
                  hipMemcpy(host, c->args.ctl.tl, c->tl_bytes, hipMemcpyDeviceToHost) == hipSuccess;
  (void)hipSetDevice(prev);
  if (!ok) return KQ_ERR_HIP;
  *groups = (int)c->args.ctl.groups;
  *n_sub = c->args.n_steps;
  return KQ_OK;
}
#endif

int kq_chain_waits(const kq_chain* c, uint8_t* waits, int n) {
  if (!c || !waits) return KQ_ERR_NULL;
  if (n != (int)c->waits.size()) return KQ_ERR_SHAPE;
  for (int j = 0; j < n; ++j) waits[j] = c->waits[j];
  return KQ_OK;
}

int kq_chain_query(kq_chain* c) {
  if (!c) return KQ_ERR_NULL;
  return *reinterpret_cast<volatile uint32_t*>(c->flag) ? KQ_ERR_TIMEOUT : KQ_OK;
}

int kq_chain_status(kq_chain* c) {
  if (!c) return KQ_ERR_NULL;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(c->dev) != hipSuccess) return KQ_ERR_HIP;
  uint32_t err = 0;
  int rc = KQ_OK;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(&err, c->args.ctl.error, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess)
    rc = KQ_ERR_HIP;
  if (rc == KQ_OK && (err || *reinterpret_cast<volatile uint32_t*>(c->flag))) {
    // reset: the split-tile and head counters (a workgroup that stopped waiting may have entered a
    // step early and left them non-zero), the device error word and the host flag
    rc = hipMemset(c->counters, 0, c->ws_bytes) == hipSuccess &&
                 hipMemset(c->args.ctl.error, 0, sizeof(err)) == hipSuccess && hipDeviceSynchronize() == hipSuccess
             ? KQ_ERR_TIMEOUT
             : KQ_ERR_HIP;
    *reinterpret_cast<volatile uint32_t*>(c->flag) = 0;
  }
  (void)hipSetDevice(prev);
  return rc;
}

int kq_chain_destroy(kq_chain* c) {
  if (!c) return KQ_OK;
  int prev = 0, rc = KQ_OK;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(c->dev) != hipSuccess) rc = KQ_ERR_HIP;
  if (rc == KQ_OK && (hipDeviceSynchronize() != hipSuccess || hipFree(c->mem) != hipSuccess ||
                      hipHostFree(c->flag) != hipSuccess))
    rc = KQ_ERR_HIP;
  (void)hipSetDevice(prev);
  delete c;
  return rc;
}

}  // extern "C"
