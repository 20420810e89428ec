// Decode-step K-quant GEMV: y[b, r] = sum_k dequant(W)[r, k] * x[b, k], b < B <= 8.
//
// Work decomposition.  A "unit" is one tile column: 64 rows (lane == row) x one
// 256-weight super-block column, 9 / 11 / 13 KiB of weights read as coalesced
// 1 KiB wavefront loads.  Units are ordered tile-major (all columns of tile 0,
// then tile 1, ...) and each wavefront takes a contiguous run of `upw` of them,
// so the chip is filled with an even share per wavefront whatever the matrix
// shape.  A tile whose columns span several wavefronts is finished by the last
// of them to arrive: each writes its partial row sums to scratch, bumps a
// counter, and the last one adds the partials in wavefront order (fixed order,
// so the result is deterministic) and resets the counter for the next call.
//
// Per super-block and lane the 4/5/6-bit quants become bf16 pairs (128 + q)
// with shift/and-or only, and v_dot2_f32_bf16 takes the activation pair
// straight from scalar registers: all 64 lanes of a wavefront share the column
// and so the same activations, which arrive with scalar loads.  Per sub-block
// the sum S of (128 + q) * x is corrected with T, the same chain of dot2 over
// (128, 128) (Q6_K: (160, 160) = 128 + 32), computed once per wavefront into
// LDS; when every q is zero (Q6_K: 32) S and T are bitwise equal and the
// sub-block contributes exactly zero.  Then
//   Q4_K/Q5_K: acc += (d*sc) * (S - T) - (dmin*m/128) * T
//   Q6_K     : acc += (d*sc) * (S - T).
// With fp32 activations the weights are converted to exact fp32 q and used
// with v_fma (S = sum q*x, T = sum x).
#include "kq_common.h"
#include "kq_internal.h"

namespace kq {

template <int QT>
__device__ __forceinline__ const uint8_t* unit_base(const GemvArgs& a, int t, int c) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < KQ_MAX_PROJ; ++i)
    if (i < a.nproj && t >= a.tile_begin[i]) p = i;
  return a.w[p] + ((int64_t)(t - a.tile_begin[p]) * a.n_cols + c) * tile_bytes<QT>();
}

template <int QT>
__device__ __forceinline__ void load_unit(const uint8_t* base, int lane, u32x4* buf, uint32_t& d6) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base + lane * kChunk);
#pragma unroll
  for (int k = 0; k < Fmt<QT>::kChunks; ++k) buf[k] = __builtin_nontemporal_load(p + k * kTileRows);
  if constexpr (QT == KQ_Q6_K) {
    const uint16_t* dp = reinterpret_cast<const uint16_t*>(base + 13 * kChunkStride) + lane;
    d6 = __builtin_nontemporal_load(dp);
  }
}

typedef const __attribute__((address_space(4))) uint32_t* sword_ptr;
typedef const __attribute__((address_space(4))) float* sfloat_ptr;

// T[i*B + b] for the ncols_t columns c0, c0+1, ... (mod n_cols) that this wavefront touches.
template <int QT, int B, bool XF32>
__device__ __forceinline__ void compute_T(const GemvArgs& a, float* T, int c0, int ncols_t, int lane) {
  using F = Fmt<QT>;
  if constexpr (!(XF32 && QT == KQ_Q6_K)) {
    const int n = ncols_t * F::kSubBlocks;
    for (int i = lane; i < n; i += 64) {
      const int ic = i / F::kSubBlocks, g = i - ic * F::kSubBlocks;
      int c = c0 + ic;
      if (c >= a.n_cols) c -= a.n_cols;
      const int64_t k0 = (int64_t)c * 256 + g * F::kSubW;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float t = 0.0f;
        if constexpr (!XF32) {
          const u32x4* xp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + b * a.ldx + k0);
          const uint32_t Kc = (QT == KQ_Q6_K) ? 0x43204320u : 0x43004300u;  // bf16 (160,160) / (128,128)
#pragma unroll
          for (int v = 0; v < F::kPairs / 4; ++v) {
            const u32x4 xv = xp[v];
            t = dot2_bf16(Kc, xv.x, t);
            t = dot2_bf16(Kc, xv.y, t);
            t = dot2_bf16(Kc, xv.z, t);
            t = dot2_bf16(Kc, xv.w, t);
          }
        } else {
          const float4* xp = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + b * a.ldx + k0);
#pragma unroll
          for (int v = 0; v < F::kSubW / 4; ++v) {
            const float4 xv = xp[v];
            t += xv.x;
            t += xv.y;
            t += xv.z;
            t += xv.w;
          }
        }
        T[i * B + b] = t;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Accumulate one unit (tile column c, T column index ic) into acc[B].
template <int QT, int B, bool XF32>
__device__ __forceinline__ void process_unit(const GemvArgs& a, const u32x4* buf, uint32_t d6, int c, int ic,
                                             const float* T, float* acc, uint32_t M, uint32_t K) {
  using F = Fmt<QT>;
  constexpr int SB = F::kSubBlocks, NP = F::kPairs;
  float ca[SB], cm[SB];
  sb_coeffs<QT>(buf, d6, XF32 ? 1.0f : 0.0078125f, ca, cm);
#pragma unroll
  for (int g = 0; g < SB; ++g) {
    uint32_t pr[NP];
    unpack_pairs<QT>(buf, g, M, K, pr);
    const int64_t k0 = (int64_t)c * 256 + g * F::kSubW;
    const float* Tg = T + (ic * SB + g) * B;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float s = 0.0f;
      if constexpr (!XF32) {
        sword_ptr xw = (sword_ptr)(a.x) + ((b * a.ldx + k0) >> 1);
#pragma unroll
        for (int i = 0; i < NP; ++i) s = dot2_bf16(pr[i], xw[i], s);
        const float t = Tg[b];
        acc[b] = __builtin_fmaf(ca[g], s - t, acc[b]);
        if constexpr (QT != KQ_Q6_K) acc[b] = __builtin_fmaf(-cm[g], t, acc[b]);
      } else {
        sfloat_ptr xf = (sfloat_ptr)(a.x) + (b * a.ldx + k0);
        const float off = (QT == KQ_Q6_K) ? 160.0f : 128.0f;  // (128 + q) - off = q, or q - 32
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          s = __builtin_fmaf(bf16_lo(pr[i]) - off, xf[2 * i], s);
          s = __builtin_fmaf(bf16_hi(pr[i]) - off, xf[2 * i + 1], s);
        }
        acc[b] = __builtin_fmaf(ca[g], s, acc[b]);
        if constexpr (QT != KQ_Q6_K) acc[b] = __builtin_fmaf(-cm[g], Tg[b], acc[b]);
      }
    }
  }
}

// Tile t's run of units ended in this wavefront: write y, or hand over a partial.
template <int B>
__device__ __forceinline__ void finish_tile(const GemvArgs& a, int t, bool full, int w, int u0, int lane,
                                            float* acc) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < KQ_MAX_PROJ; ++i)
    if (i < a.nproj && t >= a.tile_begin[i]) p = i;
  const int row = (t - a.tile_begin[p]) * kTileRows + lane;
  float* y = a.y[p];
  const int64_t ldy = a.ldy[p];
  const bool live = row < a.rows[p];
  if (full) {
    if (live) {
#pragma unroll
      for (int b = 0; b < B; ++b) y[b * ldy + row] = acc[b];
    }
    return;
  }
  // Hand-off without an L2 writeback: the partials are written with agent-scope
  // atomic stores (write-through to the device coherence point), the wavefront
  // waits until they are acknowledged, and only then bumps the tile's counter.
  // The last arrival reads the partials with agent-scope atomic loads, which
  // bypass the (per-XCD) caches.
  const int n_cols = a.n_cols, upw = a.upw;
  const int slot = (t == u0 / n_cols) ? 0 : 1;
  float* mine = a.partial + (int64_t)(w * 2 + slot) * kPartialStride;
#pragma unroll
  for (int b = 0; b < B; ++b)
    __hip_atomic_store(mine + b * kTileRows + lane, acc[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const int wa = (t * n_cols) / upw, wb = ((t + 1) * n_cols - 1) / upw;
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(&a.counters[wa], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != (uint32_t)(wb - wa)) return;
  asm volatile("" ::: "memory");
  float s[B];
#pragma unroll
  for (int b = 0; b < B; ++b) s[b] = 0.0f;
  for (int wc = wa; wc <= wb; ++wc) {
    const int sl = (t == (wc * upw) / n_cols) ? 0 : 1;
    float* pp = a.partial + (int64_t)(wc * 2 + sl) * kPartialStride;
#pragma unroll
    for (int b = 0; b < B; ++b)
      s[b] += __hip_atomic_load(pp + b * kTileRows + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (live) {
#pragma unroll
    for (int b = 0; b < B; ++b) y[b * ldy + row] = s[b];
  }
  if (lane == 0) __hip_atomic_store(&a.counters[wa], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int QT, int B, bool XF32>
__global__ void __launch_bounds__(256) gemv_kernel(const GemvArgs a) {
  using F = Fmt<QT>;
  constexpr int NCH = F::kChunks;
  extern __shared__ float lds_t[];
  // readfirstlane: the wavefront index is uniform across the wavefront; saying so
  // keeps all unit/column bookkeeping and the activation addresses in SGPRs.
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Blocks are dispatched round-robin over the 8 XCDs; give consecutive logical
  // blocks (which share split tiles) to one XCD so partial sums stay in its L2.
  const int nb8 = gridDim.x >> 3;
  const int lblock = (blockIdx.x & 7) * nb8 + (blockIdx.x >> 3);
  const int w = lblock * 4 + wid;
  if (w >= a.n_waves) return;
  const int n_cols = a.n_cols;
  const int u0 = w * a.upw;
  const int u1 = min(u0 + a.upw, a.n_units);
  const int c0 = u0 % n_cols;
  float* T = lds_t + wid * a.tsb * B;
  const uint32_t M = in_vgpr(0x000F000Fu), K = in_vgpr(0x43004300u);

  // Weight loads for the first two units go out before the activation sums,
  // so their latency overlaps.
  u32x4 bA[NCH], bB[NCH];
  uint32_t dA = 0, dB = 0;
  int tl = u0 / n_cols, cl = c0;  // next unit to load
  load_unit<QT>(unit_base<QT>(a, tl, cl), lane, bA, dA);
  if (++cl == n_cols) { cl = 0; ++tl; }
  if (u0 + 1 < u1) load_unit<QT>(unit_base<QT>(a, tl, cl), lane, bB, dB);
  if (++cl == n_cols) { cl = 0; ++tl; }

  compute_T<QT, B, XF32>(a, T, c0, min(n_cols, u1 - u0), lane);

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  int t = u0 / n_cols, c = c0, ic = 0;
  int u = u0;
  auto step = [&](const u32x4* buf, uint32_t d6) {
    process_unit<QT, B, XF32>(a, buf, d6, c, ic, T, acc, M, K);
    if (c == n_cols - 1 || u + 1 == u1) {
      const bool full = (t * n_cols >= u0) && (c == n_cols - 1);
      finish_tile<B>(a, t, full, w, u0, lane, acc);
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    }
    ++u;
    if (++c == n_cols) { c = 0; ++t; }
    if (++ic == n_cols) ic = 0;
  };
  while (true) {
    step(bA, dA);
    if (u + 1 < u1) {
      load_unit<QT>(unit_base<QT>(a, tl, cl), lane, bA, dA);
      if (++cl == n_cols) { cl = 0; ++tl; }
    }
    if (u >= u1) break;
    step(bB, dB);
    if (u + 1 < u1) {
      load_unit<QT>(unit_base<QT>(a, tl, cl), lane, bB, dB);
      if (++cl == n_cols) { cl = 0; ++tl; }
    }
    if (u >= u1) break;
  }
}

template <int QT, int B, bool XF32>
static hipError_t launch_one(const GemvArgs& a, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((gemv_kernel<QT, B, XF32>), dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int QT, bool XF32>
static hipError_t launch_b(const GemvArgs& a, int batch, int grid, size_t lds, hipStream_t s) {
  switch (batch) {
    case 1: return launch_one<QT, 1, XF32>(a, grid, lds, s);
    case 2: return launch_one<QT, 2, XF32>(a, grid, lds, s);
    case 3: return launch_one<QT, 3, XF32>(a, grid, lds, s);
    case 4: return launch_one<QT, 4, XF32>(a, grid, lds, s);
    case 5: return launch_one<QT, 5, XF32>(a, grid, lds, s);
    case 6: return launch_one<QT, 6, XF32>(a, grid, lds, s);
    case 7: return launch_one<QT, 7, XF32>(a, grid, lds, s);
    case 8: return launch_one<QT, 8, XF32>(a, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(int type, int xtype, int batch, const GemvArgs& a, int grid, size_t lds, hipStream_t s) {
  const bool f32 = xtype == KQ_X_F32;
  switch (type) {
    case KQ_Q4_K: return f32 ? launch_b<KQ_Q4_K, true>(a, batch, grid, lds, s) : launch_b<KQ_Q4_K, false>(a, batch, grid, lds, s);
    case KQ_Q5_K: return f32 ? launch_b<KQ_Q5_K, true>(a, batch, grid, lds, s) : launch_b<KQ_Q5_K, false>(a, batch, grid, lds, s);
    case KQ_Q6_K: return f32 ? launch_b<KQ_Q6_K, true>(a, batch, grid, lds, s) : launch_b<KQ_Q6_K, false>(a, batch, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kq
