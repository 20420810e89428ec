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


// Scratch for row tiles whose columns span several workgroups: two partial-sum
// slots and one arrival counter per workgroup.  The counters are zero between
// calls (the last arrival of a tile resets its counter), so they are cleared
// once, at allocation.
constexpr int kMaxGroups = 8192;
// then the per-head sums of squares of KQ_EPI_HEADNORM launches ([tile][2][KQ_MAX_BATCH]),
// and after the tile counters one counter per head
constexpr size_t kPartialFloats = (size_t)kMaxGroups * 2 * kPartialStride;
constexpr size_t kHeadSsFloats = (size_t)kMaxGroups * 2 * KQ_MAX_BATCH;
constexpr size_t kPartialBytes = (kPartialFloats + kHeadSsFloats) * sizeof(float);
constexpr size_t kCounterBytes = (size_t)2 * kMaxGroups * sizeof(uint32_t);
static_assert(kHeadRows == 2 * 64, "a head is two row tiles");
constexpr int kMaxDevices = 64;

struct DeviceState {
  bool ready = false;
  int cus = 0;
  float* partial = nullptr;
  uint32_t* counters = nullptr;
};

static std::mutex g_mu;
static DeviceState g_dev[kMaxDevices];

static int device_state(int dev, DeviceState** out) {
  if (dev < 0 || dev >= kMaxDevices) return KQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& s = g_dev[dev];
  if (!s.ready) {
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return KQ_ERR_HIP;
    if (hipSetDevice(dev) != hipSuccess) return KQ_ERR_HIP;
    int rc = KQ_OK;
    void* p = nullptr;
    void* c = nullptr;
    if (hipDeviceGetAttribute(&s.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) rc = KQ_ERR_HIP;
    if (rc == KQ_OK && hipMalloc(&p, kPartialBytes) != hipSuccess) rc = KQ_ERR_NOMEM;
    if (rc == KQ_OK && hipMalloc(&c, kCounterBytes) != hipSuccess) rc = KQ_ERR_NOMEM;
    if (rc == KQ_OK && hipMemset(c, 0, kCounterBytes) != hipSuccess) rc = KQ_ERR_HIP;
    if (rc == KQ_OK && hipDeviceSynchronize() != hipSuccess) rc = KQ_ERR_HIP;
    if (rc != KQ_OK) {
      if (p) (void)hipFree(p);
      if (c) (void)hipFree(c);
      (void)hipSetDevice(prev);
      return rc;
    }
    s.partial = static_cast<float*>(p);
    s.counters = static_cast<uint32_t*>(c);
    s.ready = true;
    (void)hipSetDevice(prev);
  }
  *out = &s;
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

// Batches from which column windows are used (KQ_WINDOWS_FROM overrides; 9 = never).
static int windows_from_batch() {
  const char* e = getenv("KQ_WINDOWS_FROM");
  const int x = e ? atoi(e) : 0;
  return (x >= 1 && x <= 9) ? x : 4;
}

// Batches (bf16 activations) from which the matrix cores compute the products
// (KQ_MATRIX_CORES_FROM, 2..9; 9 = never, every batch on the dot2 VALU path).
// The default, 3, is where the dot2 path becomes VALU-issue bound: at batch 2
// it is as fast or faster on every sweep shape, from batch 3 on it is slower.
static int matrix_cores_from() {
  const char* e = getenv("KQ_MATRIX_CORES_FROM");
  const int x = e ? atoi(e) : 0;
  return (x >= 2 && x <= 9) ? x : 3;
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
  int nw;        // wavefronts per workgroup
  bool mf;       // matrix-core path
  int64_t grid;  // workgroups, a multiple of 8
  size_t lds;    // dynamic LDS per workgroup
  int rows;      // staged activation rows: the batch, or twice it for fp32 activations
};

// Launch geometry of a validated call on a device with `cus` CUs, using at most
// `max_grid` workgroups (a multiple of 8).
// epi: segment i's epilogue code in bits 4i..4i+3.  KQ_EPI_SWIGLU: one matrix
// (n == 1) from kq_repack_swiglu, rows[0] = the intermediate size, 32 outputs
// per 64-row tile.
static int plan_gemv(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x,
                     int xtype, int64_t ldx, int batch, float* const* y, const int64_t* ldy, void* const* y16,
                     const int64_t* ldy16, int cus,
                     int64_t max_grid, int force_nw, bool single, uint32_t epi, float rms_eps, float head_eps,
                     float* partial, uint32_t* counters, Plan* out) {
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
  const int forced_r = aligned_tiles();
  if (((srows >= windows_from_batch() && n_win > 1) || forced_r > 0) && tiles <= kMaxGroups &&
      n_win * tiles <= 2 * (int64_t)kMaxGroups) {
    int64_t g_target = (int64_t)cus * wpc / nw;
    if (g_target < 1) g_target = 1;
    if (g_target > max_groups) g_target = max_groups;
    int64_t g_win = g_target / n_win > 0 ? g_target / n_win : 1;
    int64_t r = forced_r > 0 ? forced_r : (tiles + g_win - 1) / g_win;
    // at most nw tiles per workgroup (a wavefront's run then touches at most two
    // tiles) unless that needs more than max_groups workgroups
    if (r > nw && ((tiles + nw - 1) / nw * n_win + 7) / 8 * 8 <= max_groups) r = nw;
    g_win = (tiles + r - 1) / r;
    const int64_t wgrid = (n_win * g_win + 7) / 8 * 8;
    if (wgrid <= max_groups) {
      even_ok = true;
      a.n_win = (int32_t)n_win;
      a.win_base = (int32_t)(n_cols / n_win);
      a.win_extra = (int32_t)(n_cols % n_win);
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
  a.partial = partial;
  a.counters = counters;
  a.head_ss = partial ? partial + kPartialFloats : nullptr;
  a.head_ctr = counters ? counters + kMaxGroups : nullptr;
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

static int gemv_impl(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x,
                     int xtype, int64_t ldx, int batch, float* const* y, const int64_t* ldy, void* stream,
                     uint32_t epi = KQ_EPI_NONE, float rms_eps = 0.0f, float head_eps = 0.0f,
                     void* const* y16 = nullptr, const int64_t* ldy16 = nullptr) {
  int rc = validate(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy);
  if (rc != KQ_OK) return rc;
  rc = check_y16(n, rows, y16, ldy16);
  if (rc != KQ_OK) return rc;
  if (!valid_epilogue(n, epi)) return KQ_ERR_TYPE;
  if (!valid_rms_eps(rms_eps)) return KQ_ERR_SHAPE;
  rc = check_heads(n, rows, epi, head_eps);
  if (rc != KQ_OK) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
  DeviceState* st = nullptr;
  rc = device_state(dev, &st);
  if (rc != KQ_OK) return rc;
  Plan p{};
  rc = plan_gemv(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, y16, ldy16, st->cus, kMaxGroups, 0, true, epi,
                 rms_eps, head_eps,
                 st->partial,
                 st->counters, &p);
  if (rc == KQ_ERR_RANGE && wg_waves(xtype == KQ_X_F32 ? 2 * batch : batch) == 8)   // too many units per
                                                                                        // workgroup: 4-wave runs
    rc = plan_gemv(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, y16, ldy16, st->cus, kMaxGroups, 4, true, epi,
                   rms_eps, head_eps,
                   st->partial,
                   st->counters, &p);
  if (rc != KQ_OK) return rc;
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
  void* mem = nullptr;   // one allocation: step table, control words, partial sums, tile counters
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
    default: return "unknown status";
  }
}

int kq_init(int device) {
  DeviceState* st = nullptr;
  return device_state(device, &st);
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
                  const int32_t* epi, float rms_eps, float head_eps, void* stream) {
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
  return gemv_impl(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, stream, packed, rms_eps, head_eps, y16, ldy16);
}

int kq_gemv_swiglu(int type, const void* w, int64_t inter, int64_t cols, const void* x, int xtype, int64_t ldx,
                   int batch, float* y, int64_t ldy, void* stream) {
  if (inter > (int64_t)INT32_MAX / 2 - 64) return KQ_ERR_RANGE;
  return gemv_impl(type, 1, &w, &inter, cols, x, xtype, ldx, batch, &y, &ldy, stream, KQ_EPI_SWIGLU);
}

int kq_gemv_q4k(const void* w, int64_t rows, int64_t cols, const void* x, int xtype, int64_t ldx, int batch,
                float* y, int64_t ldy, void* stream) {
  return gemv_impl(KQ_Q4_K, 1, &w, &rows, cols, x, xtype, ldx, batch, &y, &ldy, stream);
}

int kq_gemv_q5k(const void* w, int64_t rows, int64_t cols, const void* x, int xtype, int64_t ldx, int batch,
                float* y, int64_t ldy, void* stream) {
  return gemv_impl(KQ_Q5_K, 1, &w, &rows, cols, x, xtype, ldx, batch, &y, &ldy, stream);
}

int kq_gemv_q6k(const void* w, int64_t rows, int64_t cols, const void* x, int xtype, int64_t ldx, int batch,
                float* y, int64_t ldy, void* stream) {
  return gemv_impl(KQ_Q6_K, 1, &w, &rows, cols, x, xtype, ldx, batch, &y, &ldy, stream);
}

int kq_gemv_multi(int type, int n, const void* const* w, const int64_t* rows, int64_t cols, const void* x, int xtype,
                  int64_t ldx, int batch, float* const* y, const int64_t* ldy, void* stream) {
  return gemv_impl(type, n, w, rows, cols, x, xtype, ldx, batch, y, ldy, stream);
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

int kq_chain_create(int n_steps, const kq_chain_step* steps, int xtype, int batch, kq_chain** out) {
  if (!out) return KQ_ERR_NULL;
  *out = nullptr;
  if (n_steps < 1 || n_steps > (1 << 16)) return KQ_ERR_BATCH;
  if (!steps) return KQ_ERR_NULL;
  if (xtype != KQ_X_F32 && xtype != KQ_X_BF16) return KQ_ERR_TYPE;
  if (batch < 1 || batch > (xtype == KQ_X_F32 ? KQ_MAX_BATCH_F32 : KQ_MAX_BATCH)) return KQ_ERR_BATCH;
  const int64_t esize = xtype == KQ_X_F32 ? 4 : 2;
  for (int j = 0; j < n_steps; ++j) {
    const kq_chain_step& st = steps[j];
    const int rc = validate(st.type, st.n, st.w, st.rows, st.cols, st.x, xtype, st.ldx, batch, st.y, st.ldy);
    if (rc != KQ_OK) return rc;
    if (!valid_epilogue(st.n, (uint32_t)st.epilogue)) return KQ_ERR_TYPE;
    if (!valid_rms_eps(st.rms_eps)) return KQ_ERR_SHAPE;
    const int hrc = check_heads(st.n, st.rows, (uint32_t)st.epilogue, st.head_eps);
    if (hrc != KQ_OK) return hrc;
    const int yrc = check_y16(st.n, st.rows, st.y16, st.ldy16);
    if (yrc != KQ_OK) return yrc;
    if (((int64_t)(batch - 1) * st.ldx + st.cols) * esize >= ((int64_t)1 << 31)) return KQ_ERR_RANGE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return KQ_ERR_HIP;

  // Persistent grid: the designed workgroups per CU (two of 4 wavefronts, one
  // of 8), fewer if the occupancy of the chain kernel says so.
  kq_chain* c = new (std::nothrow) kq_chain;
  if (!c) return KQ_ERR_NOMEM;
  std::vector<Plan> plans(n_steps);
  const int srows = xtype == KQ_X_F32 ? 2 * batch : batch;
  int nw = chain_wg_waves();
  auto plan_all = [&](int64_t max_grid, size_t* lds) {
    *lds = 0;
    for (int j = 0; j < n_steps; ++j) {
      const kq_chain_step& st = steps[j];
      int rc = plan_gemv(st.type, st.n, st.w, st.rows, st.cols, st.x, xtype, st.ldx, batch, st.y, st.ldy, st.y16,
                         st.ldy16, cus,
                         max_grid, nw, false, (uint32_t)st.epilogue, st.rms_eps, st.head_eps, nullptr, nullptr, &plans[j]);
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

  const size_t steps_bytes = round_up((size_t)n_steps * sizeof(ChainStep), 256);
  // control words: arrive[n_steps][groups], done[n_steps], epoch, error
  const size_t ctl_bytes = round_up(((size_t)n_steps * (groups + 1) + 2) * sizeof(uint32_t), 256);
  const size_t total = steps_bytes + ctl_bytes + kPartialBytes + kCounterBytes;
  if (hipMalloc(&c->mem, total) != hipSuccess) {
    delete c;
    return KQ_ERR_NOMEM;
  }
  uint8_t* base = static_cast<uint8_t*>(c->mem);
  ChainStep* d_steps = reinterpret_cast<ChainStep*>(base);
  uint32_t* d_ctl = reinterpret_cast<uint32_t*>(base + steps_bytes);
  float* d_partial = reinterpret_cast<float*>(base + steps_bytes + ctl_bytes);
  uint32_t* d_counters = reinterpret_cast<uint32_t*>(base + steps_bytes + ctl_bytes + kPartialBytes);
  std::vector<ChainStep> h(n_steps);
  for (int j = 0; j < n_steps; ++j) {
    h[j].a = plans[j].a;
    h[j].a.partial = d_partial;
    h[j].a.counters = d_counters;
    h[j].a.head_ss = d_partial + kPartialFloats;
    h[j].a.head_ctr = d_counters + kMaxGroups;
    h[j].type = steps[j].type;
    h[j].grid = (int32_t)plans[j].grid;
  }
  rc = KQ_OK;
  if (hipMemcpy(d_steps, h.data(), (size_t)n_steps * sizeof(ChainStep), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(d_ctl, 0, ctl_bytes) != hipSuccess || hipMemset(d_counters, 0, kCounterBytes) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess)
    rc = KQ_ERR_HIP;
  if (rc != KQ_OK) {
    (void)hipFree(c->mem);
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
  c->args.steps = d_steps;
  c->args.n_steps = n_steps;
  uint32_t* d_done = d_ctl + (size_t)n_steps * groups;
  c->args.ctl = ChainCtl{d_ctl, d_done, d_done + n_steps, d_done + n_steps + 1, (uint32_t)groups, chain_spin()};
  *out = c;
  return KQ_OK;
}

int kq_chain_run(kq_chain* c, void* stream) {
  if (!c) return KQ_ERR_NULL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
  if (dev != c->dev) return KQ_ERR_DEVICE;
  if (launch_chain(c->xtype, c->rows, c->args, c->nw, c->mf, c->grid, c->lds, static_cast<hipStream_t>(stream),
                   nullptr) != hipSuccess)
    return KQ_ERR_HIP;
  return KQ_OK;
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
  if (rc == KQ_OK && err) {
    rc = hipMemset(c->args.ctl.error, 0, sizeof(err)) == hipSuccess && hipDeviceSynchronize() == hipSuccess
             ? KQ_ERR_TIMEOUT
             : KQ_ERR_HIP;
  }
  (void)hipSetDevice(prev);
  return rc;
}

int kq_chain_destroy(kq_chain* c) {
  if (!c) return KQ_OK;
  int prev = 0, rc = KQ_OK;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(c->dev) != hipSuccess) rc = KQ_ERR_HIP;
  if (rc == KQ_OK && (hipDeviceSynchronize() != hipSuccess || hipFree(c->mem) != hipSuccess)) rc = KQ_ERR_HIP;
  (void)hipSetDevice(prev);
  delete c;
  return rc;
}

}  // extern "C"
