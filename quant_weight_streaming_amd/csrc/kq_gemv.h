// Decode-step K-quant GEMV: y[b, r] = sum_k dequant(W)[r, k] * x[b, k], b < B <= 8.
//
// Work decomposition.  A "unit" is one tile column: 64 rows (lane == row) x one
// 256-weight super-block column, 9 / 11 / 13 KiB of weights read as coalesced
// 1 KiB wavefront loads.  Units are ordered tile-major (all columns of tile 0,
// then tile 1, ...).  By default a workgroup takes a contiguous run of NW * upw
// units and each of its NW (4 or 8) wavefronts an even part of that run (the
// parts differ by at most one unit, the longer ones on wavefronts 0, 1, ..., so
// on different SIMDs), so the chip gets an even share per wavefront whatever
// the matrix shape; with column windows a workgroup instead takes whole tiles
// of one window of columns, split between its wavefronts the same way.
// Per-tile sums go to LDS; after the main loop the workgroup adds its
// wavefronts' pieces of each tile in wavefront order, writes y for tiles it
// covered completely, and hands the rest to the other workgroups sharing the
// tile (the last to arrive adds all pieces in workgroup or window order).
// Fixed summation orders make y deterministic.
//
// Per super-block and lane the 4/5/6-bit quants become exact bf16 operands
// (kq_common.h: Q4_K/Q5_K q, Q6_K 4*(q-32)), and v_dot2_f32_bf16 dots them
// with the activation pair of the same position.  All 64 lanes (rows) of a
// wavefront share the column, so the activations are wavefront-uniform; the
// workgroup stages the activations of its columns in LDS once and every
// wavefront reads them with broadcast LDS loads.  Per sub-block g, with
// S = sum v*x over its elements and (Q4_K/Q5_K) X = sum x, staged alongside:
//   Q4_K/Q5_K: acc += (d*sc_g) * S - (dmin*m_g) * X
//   Q6_K     : acc += (d*sc_g/4) * S.
// S carries no offset, so its rounding error is relative to sum |v x|.
// fp32 activations are staged as two bf16 rows each, hi = bf16(x) and
// lo = bf16(x - hi), whose sums are added before the epilogue (XStage).
//
// The weight stream is buffered in registers: while one unit is computed the
// next DEPTH-1 are in flight.  The main loop issues each refill before the
// computation that needs the oldest buffer, unconditionally, and keeps global
// stores out of the loop, so the compiler waits for exactly the unit it
// consumes instead of for every load in flight.
#pragma once

#include "kq_common.h"
#include "kq_internal.h"

#ifndef KQ_DEPTH
#define KQ_DEPTH 2
#endif


namespace kq {


// Buffer resource over unit (t, c): base = its first byte, size = one unit, or
// size 0 when `live` is false, which turns every load through it into a
// zero-filled no-op that moves no data (loads past the wavefront's last unit).
template <int QT, class GA>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t unit_rsrc(GA& a, int t, int c, bool live) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < KQ_MAX_PROJ; ++i)
    if (i < a.nproj && t >= a.tile_begin[i]) p = i;
  const uint64_t addr = reinterpret_cast<uint64_t>(a.w[p]) +
                        ((int64_t)(t - a.tile_begin[p]) * a.n_cols + c) * tile_bytes<QT>();
  // every operand is wavefront-uniform; say so, so the resource stays in SGPRs
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const int n = __builtin_amdgcn_readfirstlane(live ? (int)tile_bytes<QT>() : 0);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, n,
                                           kBufferFlags);
}

// One unit's weights: chunk k of this lane's row, nontemporal (read once).
template <int QT>
__device__ __forceinline__ void load_unit(__amdgpu_buffer_rsrc_t r, int lane, u32x4* buf, uint32_t& d6) {
#pragma unroll
  for (int k = 0; k < Fmt<QT>::kChunks; ++k)
    buf[k] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * kChunk + k * kChunkStride, 0, kCacheNT);
  if constexpr (QT == KQ_Q6_K)
    d6 = __builtin_amdgcn_raw_buffer_load_b16(r, 13 * kChunkStride + 2 * lane, 0, kCacheNT);
}

// Staging of the activations of the workgroup's columns c0, c0+1, ... (mod
// n_cols) in LDS: X [ic][b][256 elements], rows RS bytes apart.  The work is cut into items of one
// sub-block of one batch row; each thread issues the loads of IPT items (128
// bytes) before it stores any of them, so a round costs one memory round trip,
// and the first round is issued ahead of the weight prologue so that waiting
// for it does not wait for the weights.  On the dot2 path of Q4_K/Q5_K the
// store also forms T, the item's activation sum X (a dot2 chain over (1, 1)),
// at T[ic * SB + g][b].
// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// A segment's bf16 copy of an output (the next product's activation): the fp32
// value rounded to the nearest bf16; COH: through the device coherence point.
template <bool COH>
__device__ __forceinline__ void store_bf16(uint16_t* p, float v) {
  const uint16_t h = (uint16_t)bf16_bits(v);
  if constexpr (COH) __hip_atomic_store(p, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = h;
}

// Staging of the activations into LDS as bf16 rows of 512 bytes (RS apart).
// B is the number of staged rows.  XF32: the activations are fp32 and each of
// the B / 2 rows read is staged as two bf16 rows, hi = bf16(x) as row b and
// lo = bf16(x - hi) as row b + B / 2, so that hi + lo is x to within 2^-18 |x|
// and the bf16 products run on both.
template <int QT, int B, bool XF32, int NW, int RS>
struct XStage {
  using F = Fmt<QT>;
  static constexpr int SB = F::kSubBlocks;
  static constexpr int BU = XF32 ? B / 2 : B;               // activation rows read
  static constexpr int ES = XF32 ? 4 : 2;                   // bytes per element read
  static constexpr int VPI = F::kSubW * ES / 16;            // 16-byte vectors per item
  static constexpr int IPT = VPI >= 8 ? 1 : 8 / VPI;        // items per thread and round
  static constexpr int NT = 64 * NW;
  static_assert(!XF32 || B % 2 == 0, "fp32 activations stage two rows each");
  u32x4 v[IPT][VPI];

  __device__ __forceinline__ static int rounds(int len) { return (len * BU * SB + IPT * NT - 1) / (IPT * NT); }

  // COH: read through the device coherence point (the activations may have been
  // written by another XCD earlier in the same launch).
  template <bool COH, class GA>
  __device__ __forceinline__ void load(GA& a, int c0, int len, int r) {
    const int n = len * BU * SB;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int i = (r * IPT + j) * NT + threadIdx.x;
      if (i < n) {
        const int g = i % SB, q = i / SB, b = q % BU, ic = q / BU;
        int c = c0 + ic;
        if (c >= a.n_cols) c -= a.n_cols;
        const int64_t off = ((int64_t)b * a.ldx + (int64_t)c * 256 + g * F::kSubW) * ES;
        if constexpr (COH) {
          const __amdgpu_buffer_rsrc_t xr =
              __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.x), (short)0, 0x7fffffff, kBufferFlags);
#pragma unroll
          for (int e = 0; e < VPI; ++e)
            v[j][e] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off + 16 * e, 0, kCacheCoherent);
        } else {
          const uint8_t* xp = static_cast<const uint8_t*>(a.x) + off;
#pragma unroll
          for (int e = 0; e < VPI; ++e) v[j][e] = reinterpret_cast<const u32x4*>(xp)[e];
        }
      }
    }
  }

  // Q2 (not null: the launch normalises x): Q2[ic * BU + b] = sum of x^2 over
  // staged column ic of activation row b (from the values read, fp32 or bf16).
  // The SB items of one (column, row) sit in SB consecutive lanes (n and every
  // round's start are multiples of SB), so their squares are added by a fixed
  // butterfly and every workgroup that stages a column gets the same bits for it.
  // WITH_T: the sub-block's sum t of staged row b.  Dot2 path (TB false):
  // T[(ic * SB + g) * TS + b] = t with TS = B.  Matrix-core path (TB): t as three
  // bf16 parts hi + mid + lo (each the rounding of what the earlier parts leave;
  // the differences are exact, so the parts hold t's 24 bits), part s at byte
  // ((ic * 3 + s) * TS + b) * 16 + 2 g of T, TS = NB * 4 rows of 8 sub-blocks.
  template <bool WITH_T, int TS = B, bool TB = false>
  __device__ __forceinline__ void store(uint8_t* X, float* T, float* Q2, int len, int r) const {
    const int n = len * BU * SB;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int i = (r * IPT + j) * NT + threadIdx.x;
      if (Q2) {
        float q = 0.0f;
        if (i < n) {
#pragma unroll
          for (int e = 0; e < VPI; ++e) {
            const u32x4 xv = v[j][e];
            if constexpr (XF32) {
              q = fmaf(__uint_as_float(xv.x), __uint_as_float(xv.x), q);
              q = fmaf(__uint_as_float(xv.y), __uint_as_float(xv.y), q);
              q = fmaf(__uint_as_float(xv.z), __uint_as_float(xv.z), q);
              q = fmaf(__uint_as_float(xv.w), __uint_as_float(xv.w), q);
            } else {
              q = dot2_bf16(xv.x, xv.x, q);
              q = dot2_bf16(xv.y, xv.y, q);
              q = dot2_bf16(xv.z, xv.z, q);
              q = dot2_bf16(xv.w, xv.w, q);
            }
          }
        }
#pragma unroll
        for (int m = 1; m < SB; m <<= 1) q += __shfl_xor(q, m);
        if (i < n && i % SB == 0) Q2[i / SB] = q;   // i / SB = ic * BU + b
      }
      if (i < n) {
        const int g = i % SB, q = i / SB, b = q % BU, ic = q / BU;
        const uint32_t kc = 0x3F803F80u;   // bf16 (1, 1)
        // T: the sub-block's activation sum X, per staged row
        auto put_t = [&](int row, float v) {
          if constexpr (TB) {
            uint8_t* tb = reinterpret_cast<uint8_t*>(T) + ((ic * 3) * TS + row) * 16 + g * 2;
            const uint32_t h = bf16_bits(v);
            const float r1 = v - __uint_as_float(h << 16);
            const uint32_t m = bf16_bits(r1);
            const uint32_t l = bf16_bits(r1 - __uint_as_float(m << 16));
            *reinterpret_cast<uint16_t*>(tb) = (uint16_t)h;
            *reinterpret_cast<uint16_t*>(tb + TS * 16) = (uint16_t)m;
            *reinterpret_cast<uint16_t*>(tb + 2 * TS * 16) = (uint16_t)l;
          } else {
            T[(ic * SB + g) * TS + row] = v;
          }
        };
        auto tsum = [&](const u32x4& w, float t) {
          t = dot2_bf16(kc, w.x, t);
          t = dot2_bf16(kc, w.y, t);
          t = dot2_bf16(kc, w.z, t);
          return dot2_bf16(kc, w.w, t);
        };
        if constexpr (XF32) {
          u32x4* xh = reinterpret_cast<u32x4*>(X + (ic * B + b) * RS + g * F::kSubW * 2);
          u32x4* xo = reinterpret_cast<u32x4*>(X + (ic * B + b + BU) * RS + g * F::kSubW * 2);
          float th = 0.0f, tl = 0.0f;
#pragma unroll
          for (int e = 0; e < VPI; e += 2) {
            u32x4 hw, lw;
            uint32_t* hp = reinterpret_cast<uint32_t*>(&hw);
            uint32_t* lp = reinterpret_cast<uint32_t*>(&lw);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const u32x4 xv = v[j][e + k / 4];
              const float f = __uint_as_float(k % 4 == 0 ? xv.x : k % 4 == 1 ? xv.y : k % 4 == 2 ? xv.z : xv.w);
              const uint32_t h = bf16_bits(f);
              const uint32_t l = bf16_bits(f - __uint_as_float(h << 16));   // the difference is exact
              if (k % 2 == 0) {
                hp[k / 2] = h;
                lp[k / 2] = l;
              } else {
                hp[k / 2] |= h << 16;
                lp[k / 2] |= l << 16;
              }
            }
            xh[e / 2] = hw;
            xo[e / 2] = lw;
            if constexpr (WITH_T) {
              th = tsum(hw, th);
              tl = tsum(lw, tl);
            }
          }
          if constexpr (WITH_T) {
            put_t(b, th);
            put_t(b + BU, tl);
          }
        } else {
          u32x4* xl = reinterpret_cast<u32x4*>(X + (ic * B + b) * RS + g * F::kSubW * 2);
          float t = 0.0f;
#pragma unroll
          for (int e = 0; e < VPI; ++e) {
            xl[e] = v[j][e];
            if constexpr (WITH_T) t = tsum(v[j][e], t);
          }
          if constexpr (WITH_T) put_t(b, t);
        }
      }
    }
  }
};

// Accumulate one unit into acc[B].  Xc / Tc: the staged (bf16) activations and
// (Q4_K/Q5_K) sub-block activation sums of the unit's column.  The (sub-block,
// batch row) steps are software-pipelined: each step reads the next step's
// activations from LDS before its own dot products, and a scheduling barrier
// keeps the compiler from hoisting reads any further (which would cost
// registers and occupancy).
template <int QT, int B>
__device__ __forceinline__ void process_unit(const u32x4* buf, uint32_t d6, const uint32_t* Xc, const float* Tc,
                                             float* acc) {
  using F = Fmt<QT>;
  constexpr int SB = F::kSubBlocks, NP = F::kPairs;
  constexpr bool MINS = QT != KQ_Q6_K;
  constexpr int XW = 128;                           // 32-bit words per staged row
  constexpr int NV = NP / 4;                        // 16-byte LDS reads per sub-block and batch row
  constexpr int SWD = F::kSubW / 2;
  float ca[SB], cm[SB];
  sb_coeffs<QT>(buf, d6, ca, cm);
  u32x4 xc[NV], xn[NV];
  float tc = 0.0f, tn = 0.0f;
  {
    const u32x4* xl = reinterpret_cast<const u32x4*>(Xc);
#pragma unroll
    for (int v = 0; v < NV; ++v) xc[v] = xl[v];
    if constexpr (MINS) tc = Tc[0];
  }
  uint32_t pr[NP];
#pragma unroll
  for (int g = 0; g < SB; ++g) {
    unpack_pairs<QT>(buf, g, pr);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int gn = (b + 1 < B) ? g : g + 1, bn = (b + 1 < B) ? b + 1 : 0;
      if (gn < SB) {
        const u32x4* xl = reinterpret_cast<const u32x4*>(Xc + bn * XW + gn * SWD);
#pragma unroll
        for (int v = 0; v < NV; ++v) xn[v] = xl[v];
        if constexpr (MINS) tn = Tc[gn * B + bn];
      }
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        s = dot2_bf16(pr[4 * v + 0], xc[v].x, s);
        s = dot2_bf16(pr[4 * v + 1], xc[v].y, s);
        s = dot2_bf16(pr[4 * v + 2], xc[v].z, s);
        s = dot2_bf16(pr[4 * v + 3], xc[v].w, s);
      }
      acc[b] = __builtin_fmaf(ca[g], s, acc[b]);
      if constexpr (MINS) acc[b] = __builtin_fmaf(-cm[g], tc, acc[b]);
#pragma unroll
      for (int v = 0; v < NV; ++v) xc[v] = xn[v];
      tc = tn;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------- matrix-core path
//
// With 3 or more staged bf16 rows (bf16 activations, or fp32 activations as
// hi and lo rows) the products q * x of a unit go through
// v_mfma_f32_16x16x32_bf16 instead of v_dot2.  The operands are arranged
// block-diagonally so that the instruction consumes the lane == row layout
// as it is: for one block of 8 consecutive columns k0..k0+7,
//   B operand: lane l supplies its own row's 8 exact bf16 operands, which is
//              B[8j + kk][n] with n = l % 16, j = l / 16;
//   A operand: A[4j + b][8j + kk] = x[b][k0 + kk] and zero for the other 24 of
//              the 32 columns of row 4j + b, so lane la holds x[la % 4] when
//              (la % 16) / 4 == la / 16 and zeros otherwise;
//   result:    D[4j + b][n] = sum_kk x[b][k0 + kk] * w[16j + n][k0 + kk], held by
//              lane 16j + n in register b: lane == row again, one register per
//              batch row (four batch rows per instruction; a second set covers
//              batch rows 4..7).
// A sub-block is 4 (Q6_K: 2) such instructions accumulating in place, then
// scaled on the VALU as in the dot2 path.  For Q4_K/Q5_K the activation sum X
// of each column's sub-blocks is taken while staging, as on the dot2 path (the
// operands are exact, so X need not round like the products).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Chains of v_mfma_f32_16x16x32_bf16 accumulating over KB blocks of 8 columns,
// one or two accumulators (operand sets), each chain a single inline-assembly
// statement: the result registers are the accumulator registers (left to
// itself this compiler can give a chained instruction a result that partially
// overlaps its own accumulator input), and nothing else touches them before the
// chain has completed.  The hazard waits are therefore ours: two wait states
// before the first instruction (for a VALU write of an operand just before it)
// and eight after the last one before the result may be read (measured on the
// device: seven suffice).
#define KQ_MF(D, A, B, C) "v_mfma_f32_16x16x32_bf16 " D ", " A ", " B ", " C "\n\t"
template <int KB>
__device__ __forceinline__ void mfma_chain(f32x4& s, const bf16x8* a, const bf16x8* b);
template <>
__device__ __forceinline__ void mfma_chain<4>(f32x4& s, const bf16x8* a, const bf16x8* b) {
  asm volatile("s_nop 1\n\t" KQ_MF("%0", "%1", "%5", "0") KQ_MF("%0", "%2", "%6", "%0") KQ_MF("%0", "%3", "%7", "%0")
                   KQ_MF("%0", "%4", "%8", "%0") "s_nop 7"
               : "=&v"(s)
               : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
}
template <>
__device__ __forceinline__ void mfma_chain<3>(f32x4& s, const bf16x8* a, const bf16x8* b) {
  asm volatile("s_nop 1\n\t" KQ_MF("%0", "%1", "%4", "0") KQ_MF("%0", "%2", "%5", "%0") KQ_MF("%0", "%3", "%6", "%0")
                   "s_nop 7"
               : "=&v"(s)
               : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(b[0]), "v"(b[1]), "v"(b[2]));
}
template <>
__device__ __forceinline__ void mfma_chain<2>(f32x4& s, const bf16x8* a, const bf16x8* b) {
  asm volatile("s_nop 1\n\t" KQ_MF("%0", "%1", "%3", "0") KQ_MF("%0", "%2", "%4", "%0") "s_nop 7"
               : "=&v"(s)
               : "v"(a[0]), "v"(a[1]), "v"(b[0]), "v"(b[1]));
}
// Two accumulators sharing the weight operands b: s0 with a0[kb], s1 with a1[kb].
template <int KB>
__device__ __forceinline__ void mfma_chain2(f32x4& s0, f32x4& s1, const bf16x8* a0, const bf16x8* a1,
                                            const bf16x8* b);
template <>
__device__ __forceinline__ void mfma_chain2<4>(f32x4& s0, f32x4& s1, const bf16x8* a0, const bf16x8* a1,
                                               const bf16x8* b) {
  asm volatile("s_nop 1\n\t" KQ_MF("%0", "%2", "%10", "0") KQ_MF("%1", "%6", "%10", "0")
                   KQ_MF("%0", "%3", "%11", "%0") KQ_MF("%1", "%7", "%11", "%1")
                   KQ_MF("%0", "%4", "%12", "%0") KQ_MF("%1", "%8", "%12", "%1")
                   KQ_MF("%0", "%5", "%13", "%0") KQ_MF("%1", "%9", "%13", "%1") "s_nop 7"
               : "=&v"(s0), "=&v"(s1)
               : "v"(a0[0]), "v"(a0[1]), "v"(a0[2]), "v"(a0[3]), "v"(a1[0]), "v"(a1[1]), "v"(a1[2]), "v"(a1[3]),
                 "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
}
template <>
__device__ __forceinline__ void mfma_chain2<2>(f32x4& s0, f32x4& s1, const bf16x8* a0, const bf16x8* a1,
                                               const bf16x8* b) {
  asm volatile("s_nop 1\n\t" KQ_MF("%0", "%2", "%6", "0") KQ_MF("%1", "%4", "%6", "0")
                   KQ_MF("%0", "%3", "%7", "%0") KQ_MF("%1", "%5", "%7", "%1") "s_nop 7"
               : "=&v"(s0), "=&v"(s1)
               : "v"(a0[0]), "v"(a0[1]), "v"(a1[0]), "v"(a1[1]), "v"(b[0]), "v"(b[1]));
}
#undef KQ_MF

// Byte offsets inside the workgroup's LDS for the matrix-core path:
//   X [ic][b][256] bf16 in rows of kXRow = 528 bytes (the 16-byte pad puts the
//   four batch rows one instruction reads in different LDS banks), then
//   (Q4_K/Q5_K) T [ic][3][NB * 4][8] bf16, the sub-block activation sums of each
//   staged row as three exact bf16 parts (the A operands of the mins' product),
//   then Z, 512 zero bytes that the inactive operand lanes read.
template <int QT, int B>
struct MfmaLds {
  static constexpr int NB = (B + 3) / 4;                       // operand sets of 4 batch rows
  static constexpr int kXRow = 528;                            // bytes per staged row of x
  static constexpr int kXCol = B * kXRow;                      // bytes of x per column
  static constexpr int kTPart = NB * 4 * 16;                  // bytes of one part of T per column
  static constexpr int kTCol = QT == KQ_Q6_K ? 0 : 3 * kTPart;  // bytes of T per column
  static constexpr int kPerCol = kXCol + kTCol;
};

// A-operand byte offset of this lane for operand set gb at column ic (see above).
template <int B>
__device__ __forceinline__ int a_operand_offset(int lane, int gb, int ic, int x_base, int z_base) {
  const int b = 4 * gb + (lane & 3);
  const bool active = ((lane & 15) >> 2) == (lane >> 4) && b < B;
  return active ? x_base + (ic * B + b) * 528 : z_base;
}

// T-operand byte offset of this lane for operand set gb at column ic, and the
// stride between T's three parts (0 for a lane that reads the zero block).
template <int QT, int B>
__device__ __forceinline__ int t_operand_offset(int lane, int gb, int ic, int t_base, int z_base, int& stride) {
  const int b = 4 * gb + (lane & 3);
  const bool active = ((lane & 15) >> 2) == (lane >> 4) && b < B;
  stride = active ? MfmaLds<QT, B>::kTPart : 0;
  return active ? t_base + ic * MfmaLds<QT, B>::kTCol + b * 16 : z_base;
}

// The mins of a Q4_K/Q5_K super-block as the B operand of the mins' product:
// lane l supplies its own row's m_0..m_7 times p, the power of two (with sign)
// of dmin, which keeps each m_g * p exact in bf16 and the product's magnitude
// that of dmin * m_g * X (no overflow where the output itself is in range).
// dmin = p * f with f = dmin's mantissa in [1, 2); f = 1 when dmin is zero.
template <int QT>
__device__ __forceinline__ bf16x8 sb_mins_operand(const u32x4* c, float& f) {
  const u32x4 h = c[0];
  const uint32_t u = __float_as_uint(f16_bits_to_f32(h.x >> 16));
  const float p = __uint_as_float(u & 0xFF800000u);
  f = __uint_as_float((u & 0x007FFFFFu) | 0x3F800000u);
  const uint32_t lo = h.z & 0x3F3F3F3Fu;
  const uint32_t hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
  auto pk = [p](uint32_t v, int i) {
    return pk_bf16((float)((v >> (16 * i)) & 0xFFu) * p, (float)((v >> (16 * i + 8)) & 0xFFu) * p);
  };
  return __builtin_bit_cast(bf16x8, u32x4{pk(lo, 0), pk(lo, 1), pk(hi, 0), pk(hi, 1)});
}

// One unit on the matrix cores: ap[gb] are this lane's A-operand pointers for
// the unit's column; tp[gb] / ts[gb] its T-operand pointers and part strides
// (Q4_K/Q5_K).  Each sub-block's products are scaled by d*sc_g on the VALU; the
// mins' term, sum over g of dmin*m_g*X_g, is one more product per operand set:
// A = the staged sums X_g of the column (three exact bf16 parts, chained), B =
// the row's eight m_g times dmin's power of two, then acc -= dmin's mantissa
// times that.  The operands of sub-block g+1 are read from LDS while sub-block
// g is on the matrix core, so the read latency is not paid per instruction.
// LEAN (chain kernels, which hold the code of every weight type and would
// otherwise spill registers at batch 5..8): with two operand sets, each
// sub-block's operands are read just before use.
template <int QT, int B, bool LEAN>
__device__ __forceinline__ void process_unit_mfma(const u32x4* buf, uint32_t d6, const uint8_t* const* ap,
                                                  const uint8_t* const* tp, const int* ts, float* acc) {
  using F = Fmt<QT>;
  constexpr int SB = F::kSubBlocks, NP = F::kPairs, KB = F::kSubW / 8, NB = MfmaLds<QT, B>::NB;
  constexpr bool MINS = QT != KQ_Q6_K;
  float ca[SB], cm[SB];
  sb_coeffs<QT>(buf, d6, ca, cm);
  auto scale = [&](int g, int gb, const f32x4& S) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * gb + r < B) acc[4 * gb + r] = __builtin_fmaf(ca[g], S[r], acc[4 * gb + r]);
  };
  uint32_t pr[NP];
  if constexpr (LEAN && NB == 2) {
#pragma unroll
    for (int g = 0; g < SB; ++g) {
      bf16x8 A[NB][KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int gb = 0; gb < NB; ++gb)
          A[gb][kb] = *reinterpret_cast<const bf16x8*>(ap[gb] + (g * F::kSubW + 8 * kb) * 2);
      unpack_pairs<QT>(buf, g, pr);
      bf16x8 bop[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        bop[kb] = __builtin_bit_cast(bf16x8, u32x4{pr[4 * kb], pr[4 * kb + 1], pr[4 * kb + 2], pr[4 * kb + 3]});
      f32x4 S[NB];
      mfma_chain2<KB>(S[0], S[1], A[0], A[1], bop);
#pragma unroll
      for (int gb = 0; gb < NB; ++gb) scale(g, gb, S[gb]);
    }
  } else if constexpr (NB <= 2) {
    bf16x8 A[2][NB][KB];
    auto read_operands = [&](int g, int h) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int gb = 0; gb < NB; ++gb)
          A[h][gb][kb] = *reinterpret_cast<const bf16x8*>(ap[gb] + (g * F::kSubW + 8 * kb) * 2);
    };
    read_operands(0, 0);
#pragma unroll
    for (int g = 0; g < SB; ++g) {
      const int h = g & 1;
      if (g + 1 < SB) read_operands(g + 1, h ^ 1);
      unpack_pairs<QT>(buf, g, pr);
      bf16x8 bop[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        bop[kb] = __builtin_bit_cast(bf16x8, u32x4{pr[4 * kb], pr[4 * kb + 1], pr[4 * kb + 2], pr[4 * kb + 3]});
      f32x4 S[NB];
      if constexpr (NB == 1) mfma_chain<KB>(S[0], A[h][0], bop);
      else mfma_chain2<KB>(S[0], S[NB - 1], A[h][0], A[h][NB - 1], bop);
#pragma unroll
      for (int gb = 0; gb < NB; ++gb) scale(g, gb, S[gb]);
    }
  } else if constexpr (LEAN) {
    // batch 9..16 in a chain kernel: operand sets two at a time, read just before use
    constexpr int NPAIR = (NB + 1) / 2;
#pragma unroll
    for (int g = 0; g < SB; ++g) {
      unpack_pairs<QT>(buf, g, pr);
      bf16x8 bop[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        bop[kb] = __builtin_bit_cast(bf16x8, u32x4{pr[4 * kb], pr[4 * kb + 1], pr[4 * kb + 2], pr[4 * kb + 3]});
#pragma unroll
      for (int q = 0; q < NPAIR; ++q) {
        bf16x8 A[2][KB];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int gb = 2 * q + i;
          if (gb < NB) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              A[i][kb] = *reinterpret_cast<const bf16x8*>(ap[gb] + (g * F::kSubW + 8 * kb) * 2);
          }
        }
        f32x4 S[2];
        if (2 * q + 1 < NB) mfma_chain2<KB>(S[0], S[1], A[0], A[1], bop);
        else mfma_chain<KB>(S[0], A[0], bop);
        scale(g, 2 * q, S[0]);
        if (2 * q + 1 < NB) scale(g, 2 * q + 1, S[1]);
      }
    }
  } else {
    // batch 9..16: three or four operand sets, taken two at a time; the next
    // pair's operands are read from LDS while the current pair computes
    constexpr int NPAIR = (NB + 1) / 2;
    bf16x8 A[2][2][KB];
    auto read_pair = [&](int g, int q, int h) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int gb = 2 * q + i;
        if (gb < NB) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            A[h][i][kb] = *reinterpret_cast<const bf16x8*>(ap[gb] + (g * F::kSubW + 8 * kb) * 2);
        }
      }
    };
    read_pair(0, 0, 0);
#pragma unroll
    for (int g = 0; g < SB; ++g) {
      unpack_pairs<QT>(buf, g, pr);
      bf16x8 bop[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        bop[kb] = __builtin_bit_cast(bf16x8, u32x4{pr[4 * kb], pr[4 * kb + 1], pr[4 * kb + 2], pr[4 * kb + 3]});
#pragma unroll
      for (int q = 0; q < NPAIR; ++q) {
        const int h = (g * NPAIR + q) & 1;
        if (q + 1 < NPAIR) read_pair(g, q + 1, h ^ 1);
        else if (g + 1 < SB) read_pair(g + 1, 0, h ^ 1);
        f32x4 S[2];
        if (2 * q + 1 < NB) mfma_chain2<KB>(S[0], S[1], A[h][0], A[h][1], bop);
        else mfma_chain<KB>(S[0], A[h][0], bop);
        scale(g, 2 * q, S[0]);
        if (2 * q + 1 < NB) scale(g, 2 * q + 1, S[1]);
      }
    }
  }
  if constexpr (MINS) {
    float f;
    const bf16x8 mb = sb_mins_operand<QT>(buf, f);
    const bf16x8 mbs[3] = {mb, mb, mb};
#pragma unroll
    for (int gb = 0; gb < NB; ++gb) {
      bf16x8 tv[3];
#pragma unroll
      for (int s = 0; s < 3; ++s) tv[s] = *reinterpret_cast<const bf16x8*>(tp[gb] + s * ts[gb]);
      f32x4 M;
      mfma_chain<3>(M, tv, mbs);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * gb + r < B) acc[4 * gb + r] = __builtin_fmaf(-f, M[r], acc[4 * gb + r]);
    }
  }
}

// Weight-less RMSNorm of each head of kHeadRows outputs of a segment (the Q
// and K heads): y = v / sqrt(mean over the head of v^2 + head_eps) per batch
// row.  A head is two tiles, whose writers may be different workgroups: each
// stores its raw values and its sum of squares (a xor butterfly, the same bits
// in every lane) through the coherence point, waits for them, and bumps the
// head's counter; the second to arrive adds the two sums in tile order, scales
// its own values and re-reads, scales and rewrites the other tile's.  The
// counter is reset for the next call.
template <int B, class GA>
__device__ __forceinline__ void head_norm_tile(GA& a, int t, int p, int lane, const float* v) {
  const int tl = t - a.tile_begin[p], par = tl & 1, h0 = t - par;
  float* y = a.y[p];
  const int64_t ldy = a.ldy[p];
  const int row = tl * kTileRows + lane;
  // the tile's sum of squares, then lane 0's value in every lane: the compiler
  // may fuse a square into the butterfly's first addition differently in each
  // lane, and the head's two halves must add the same published values
  // whichever finishes second
  float q[B];
#pragma unroll
  for (int b = 0; b < B; ++b) q[b] = v[b] * v[b];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
    for (int b = 0; b < B; ++b) q[b] += __shfl_xor(q[b], m);
#pragma unroll
  for (int b = 0; b < B; ++b) q[b] = __shfl(q[b], 0);
#pragma unroll
  for (int b = 0; b < B; ++b)
    __hip_atomic_store(y + b * ldy + row, v[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float* hs = a.head_ss + ((int64_t)h0 * 2 + par) * KQ_MAX_BATCH;
  float mine = 0.0f;
#pragma unroll
  for (int b = 0; b < B; ++b)
    if (lane == b) mine = q[b];
  if (lane < B) __hip_atomic_store(hs + lane, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(a.head_ctr + h0, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old == 0) return;                      // the head's other tile finishes it
  asm volatile("" ::: "memory");
  const float* ho = a.head_ss + ((int64_t)h0 * 2 + (par ^ 1)) * KQ_MAX_BATCH;
  const float qo = lane < B ? __hip_atomic_load(ho + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
  float sc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float other = __shfl(qo, b);
    const float tot = par ? other + q[b] : q[b] + other;   // tile 0's sum first
    sc[b] = 1.0f / sqrtf(tot / (float)kHeadRows + a.head_eps);
  }
  // every read of the other tile goes out before the first store (one round trip, not B)
  const int row_o = (tl ^ 1) * kTileRows + lane;
  float vo[B];
#pragma unroll
  for (int b = 0; b < B; ++b) vo[b] = __hip_atomic_load(y + b * ldy + row_o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int b = 0; b < B; ++b)
    __hip_atomic_store(y + b * ldy + row, v[b] * sc[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int b = 0; b < B; ++b)
    __hip_atomic_store(y + b * ldy + row_o, vo[b] * sc[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (a.y16[p]) {
    uint16_t* y16 = a.y16[p];
    const int64_t ld16 = a.ldy16[p];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      store_bf16<true>(y16 + b * ld16 + row, v[b] * sc[b]);
      store_bf16<true>(y16 + b * ld16 + row_o, vo[b] * sc[b]);
    }
  }
  if (lane == 0) __hip_atomic_store(a.head_ctr + h0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Write finished row sums of tile t (all of its columns) to y; COH: write
// through to the device coherence point (read later in the same launch).
template <int B, bool COH, class GA>
__device__ __forceinline__ void write_tile(GA& a, int t, int lane, const float* v) {
  if (a.epi == KQ_EPI_SWIGLU) {
    // lanes 0..31 hold the gate sums of outputs 32t .. 32t+31, lanes 32..63
    // the up sums of the same outputs: y = silu(gate) * up
    float u[B];
#pragma unroll
    for (int b = 0; b < B; ++b) u[b] = __shfl(v[b], lane + 32);
    const int row = t * (kTileRows / 2) + lane;
    if (lane < 32 && row < a.rows[0]) {
      float* y = a.y[0];
      const int64_t ldy = a.ldy[0];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float h = v[b] / (1.0f + expf(-v[b])) * u[b];
        if constexpr (COH) __hip_atomic_store(y + b * ldy + row, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else y[b * ldy + row] = h;
        if (a.y16[0]) store_bf16<COH>(a.y16[0] + b * a.ldy16[0] + row, h);
      }
    }
    return;
  }
  int p = 0;
#pragma unroll
  for (int i = 1; i < KQ_MAX_PROJ; ++i)
    if (i < a.nproj && t >= a.tile_begin[i]) p = i;
  const int row = (t - a.tile_begin[p]) * kTileRows + lane;
  const uint32_t code = (a.epi >> (4 * p)) & 15u;
  if (code == KQ_EPI_HEADNORM) {
    head_norm_tile<B>(a, t, p, lane, v);
    return;
  }
  if (row < a.rows[p]) {
    float* y = a.y[p];
    const int64_t ldy = a.ldy[p];
    float o[B];
#pragma unroll
    for (int b = 0; b < B; ++b) o[b] = v[b];
    if (code == KQ_EPI_SIGMOID) {                // the attention output gate
#pragma unroll
      for (int b = 0; b < B; ++b) o[b] = 1.0f / (1.0f + expf(-o[b]));
    } else if (code == KQ_EPI_RESIDUAL) {        // y holds the residual stream on entry
      float r[B];                                // every read goes out before the first store
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float* yp = y + b * ldy + row;
        r[b] = COH ? __hip_atomic_load(yp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *yp;
      }
#pragma unroll
      for (int b = 0; b < B; ++b) o[b] += r[b];
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if constexpr (COH) __hip_atomic_store(y + b * ldy + row, o[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else y[b * ldy + row] = o[b];
    }
    if (a.y16[p]) {
#pragma unroll
      for (int b = 0; b < B; ++b) store_bf16<COH>(a.y16[p] + b * a.ldy16[p] + row, o[b]);
    }
  }
}

// Weight-less RMSNorm folded into the GEMV: W (x / rms(x)) = (W x) / rms(x),
// rms(x) = sqrt(sum_k x_k^2 / K + eps) per batch row.  ss[b] is the sum of x^2
// over all K columns of row b (the same for every lane); v[b] *= 1 / rms.
template <int B, class GA>
__device__ __forceinline__ void rms_scale(const GA& a, float* v, const float* ss) {
  const float k = (float)a.n_cols * 256.0f;
#pragma unroll
  for (int b = 0; b < B; ++b) v[b] *= 1.0f / sqrtf(ss[b] / k + a.rms_eps);
}

// A piece's sums of x^2 go to the slot's words partial_q(B) + b, lane b < B.
template <int B>
__device__ __forceinline__ void publish_q(float* slot, int lane, const float* q) {
  float mine = 0.0f;
#pragma unroll
  for (int b = 0; b < B; ++b)
    if (lane == b) mine = q[b];
  if (lane < B) __hip_atomic_store(slot + partial_q(B) + lane, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup L holds its sum for tile t, whose columns other workgroups share.
// Hand it over; the last workgroup to arrive adds all of them in workgroup
// order and writes y.  No L2 writeback is needed: the partials are written with
// agent-scope atomic stores (write-through to the device coherence point), the
// wavefront waits until they are acknowledged before bumping the tile's
// counter, and the last arrival reads them with agent-scope atomic loads, which
// bypass the per-XCD caches.  The counter is reset for the next call.
template <int B, bool COH, class GA>
__device__ __forceinline__ void hand_off(GA& a, int t, int L, int wgu, int lane, const float* v, const float* q) {
  const int n_cols = a.n_cols;
  const bool norm = a.rms_eps > 0.0f;
  const int slot = (t == (L * wgu) / n_cols) ? 0 : 1;
  float* mine = a.partial + (int64_t)(L * 2 + slot) * partial_stride(B);
#pragma unroll
  for (int b = 0; b < B; ++b)
    __hip_atomic_store(mine + b * kTileRows + lane, v[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (norm) publish_q<B>(mine, lane, q);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const int la = (t * n_cols) / wgu, lb = ((t + 1) * n_cols - 1) / wgu;
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(&a.counters[la], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != (uint32_t)(lb - la)) return;
  asm volatile("" ::: "memory");
  float s[B];
#pragma unroll
  for (int b = 0; b < B; ++b) s[b] = 0.0f;
  float qs = 0.0f;   // lane b < B: the pieces' sums of x^2 for batch row b
  // read the pieces PR workgroups at a time (one round trip per PR), then add
  // them in workgroup order
  constexpr int PR = B <= 2 ? 8 : 4;
  for (int l0 = la; l0 <= lb; l0 += PR) {
    float v[PR][B], qv[PR];
#pragma unroll
    for (int j = 0; j < PR; ++j) {
      const int l = l0 + j;
      const int sl = (t == (l * wgu) / n_cols) ? 0 : 1;
      const float* pp = a.partial + (int64_t)(l * 2 + sl) * partial_stride(B);
#pragma unroll
      for (int b = 0; b < B; ++b)
        v[j][b] = l <= lb ? __hip_atomic_load(pp + b * kTileRows + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0.0f;
      qv[j] = norm && l <= lb && lane < B
                  ? __hip_atomic_load(pp + partial_q(B) + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                  : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < PR; ++j) {
#pragma unroll
      for (int b = 0; b < B; ++b)
        if (l0 + j <= lb) s[b] += v[j][b];
      if (l0 + j <= lb) qs += qv[j];
    }
  }
  if (norm) {
    float qa[B];
#pragma unroll
    for (int b = 0; b < B; ++b) qa[b] = __shfl(qs, b);
    rms_scale<B>(a, s, qa);
  }
  write_tile<B, COH>(a, t, lane, s);
  if (lane == 0) __hip_atomic_store(&a.counters[la], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Windowed variant: the workgroup of window w holds tile t's sum over that
// window's columns.  Every window contributes one piece per tile; the last to
// arrive adds them in window order.  Same publication protocol as hand_off.
template <int B, bool COH, class GA>
__device__ __forceinline__ void hand_off_windows(GA& a, int t, int w, int lane, const float* v, const float* q) {
  const bool norm = a.rms_eps > 0.0f;
  float* mine = a.partial + (int64_t)(w * a.n_tiles + t) * partial_stride(B);
#pragma unroll
  for (int b = 0; b < B; ++b)
    __hip_atomic_store(mine + b * kTileRows + lane, v[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (norm) publish_q<B>(mine, lane, q);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(&a.counters[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != (uint32_t)(a.n_win - 1)) return;
  asm volatile("" ::: "memory");
  float s[B];
#pragma unroll
  for (int b = 0; b < B; ++b) s[b] = 0.0f;
  float qs = 0.0f;
  constexpr int PR = B <= 2 ? 8 : 4;
  for (int w0 = 0; w0 < a.n_win; w0 += PR) {
    float pv[PR][B], qv[PR];
#pragma unroll
    for (int j = 0; j < PR; ++j) {
      const float* pp = a.partial + (int64_t)((w0 + j) * a.n_tiles + t) * partial_stride(B);
#pragma unroll
      for (int b = 0; b < B; ++b)
        pv[j][b] = w0 + j < a.n_win
                       ? __hip_atomic_load(pp + b * kTileRows + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0.0f;
      qv[j] = norm && w0 + j < a.n_win && lane < B
                  ? __hip_atomic_load(pp + partial_q(B) + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                  : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < PR; ++j) {
#pragma unroll
      for (int b = 0; b < B; ++b)
        if (w0 + j < a.n_win) s[b] += pv[j][b];
      if (w0 + j < a.n_win) qs += qv[j];
    }
  }
  if (norm) {
    float qa[B];
#pragma unroll
    for (int b = 0; b < B; ++b) qa[b] = __shfl(qs, b);
    rms_scale<B>(a, s, qa);
  }
  write_tile<B, COH>(a, t, lane, s);
  if (lane == 0) __hip_atomic_store(&a.counters[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Step barrier of a chain.  Workgroup g arrives at step j by storing the run's
// tag in arrive[j][g].  Two forms of the wait:
//  * two hops (the dynamic-units shape: one or two staged rows, 8 wavefronts):
//    workgroup 0 (the collector) polls the arrivals of the step and then
//    stores the tag in the kDoneReplicas copies of done[j] (a line each);
//    workgroup g polls copy g % kDoneReplicas, so the pollers spread over
//    lines instead of queueing on one;
//  * one hop (every other shape): every workgroup's first wavefront polls the
//    arrivals itself.
// Measured on a decoder's sweep of projections, the one-hop form is 3-4%
// faster at batch 8 and 1% slower at batch 1, where its releases are spread
// wider (hundreds of pollers on the same words).
// All plain stores and loads through the device coherence point: no
// read-modify-write on a shared word (hundreds of them on one address serialise
// at the memory).  Every poll loop is bounded by `spin`; one that gives up sets
// the error word.  Arriving at step j implies having arrived at every earlier
// step, so both forms also order step j+1 after all earlier steps.
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-step timeline of a chain, in measurement builds only (-DKQ_TIMELINE,
// libkq_timeline.so): the first thread of each workgroup stores the device
// clock (s_memrealtime, 100 MHz) at fixed points of every step it takes part
// in, into tl[step][workgroup][k]:
//   0 step start, 1 after the barrier wait, 2 activations staged,
//   3 main loop done (all wavefronts), 4 tiles written or handed over,
//   5 arrival stored; at step 0, slot 6 holds the XCC id and 7 the HW_ID word.
#ifdef KQ_TIMELINE
__device__ __forceinline__ void tl_stamp(const ChainCtl* c, int step, int k) {
  if (c && c->tl && threadIdx.x == 0)
    __hip_atomic_store(c->tl + ((size_t)step * c->groups + blockIdx.x) * 8 + k,
                       (uint64_t)__builtin_amdgcn_s_memrealtime(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void tl_ids(const ChainCtl* c) {
  if (c->tl && threadIdx.x == 0) {
    uint32_t x, h;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(h));
    __hip_atomic_store(c->tl + (size_t)blockIdx.x * 8 + 6, (uint64_t)x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(c->tl + (size_t)blockIdx.x * 8 + 7, (uint64_t)h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
#else
__device__ __forceinline__ void tl_stamp(const ChainCtl*, int, int) {}
__device__ __forceinline__ void tl_ids(const ChainCtl*) {}
#endif

// A wait gave up: set the device error word (later waits of the run then give
// up at once, and later runs do nothing) and the host-visible word that
// kq_chain_run and kq_chain_query read without a device synchronisation.
__device__ __forceinline__ void chain_fail(const ChainCtl& c) {
  store_coherent(c.error, 1u);
  __hip_atomic_store(c.error_host, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void chain_collect(const ChainCtl& c, int step, uint32_t tag) {
  const uint32_t* arr = c.arrive + (size_t)step * c.groups;
  uint32_t n = 0;
  int all;
  for (;;) {
    int mine = 1;
    for (uint32_t g = threadIdx.x; g < c.groups; g += blockDim.x) mine &= load_coherent(arr + g) == tag;
    all = __syncthreads_and(mine);
    if (all) break;
    // bounded: give up after `spin` polls, or at once once another wait of the run has
    const int quit = __syncthreads_or(threadIdx.x == 0 && (++n > c.spin || load_coherent(c.error) != 0u));
    if (quit) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (threadIdx.x == 0 && !all) chain_fail(c);
  if (threadIdx.x < kDoneReplicas) store_coherent(c.done + ((size_t)step * kDoneReplicas + threadIdx.x) * 16, tag);
}

// Wait before reading step `step`'s activations until every workgroup has
// finished step - 1.
template <bool ONE_HOP>
__device__ __forceinline__ void chain_wait(const ChainCtl& c, int step, uint32_t tag) {
  if (step == 0) return;
  if constexpr (ONE_HOP) {
    if (threadIdx.x < 64) {
      const uint32_t* arr = c.arrive + (size_t)(step - 1) * c.groups;
      uint32_t n = 0;
      for (;;) {
        bool mine = true;
        for (uint32_t g = threadIdx.x; g < c.groups; g += 64) mine &= load_coherent(arr + g) == tag;
        if (__all(mine)) break;
        // bounded: give up after `spin` polls, or at once once another wait of the run has
        if (++n > c.spin || __builtin_amdgcn_readfirstlane(load_coherent(c.error)) != 0u) {
          if (threadIdx.x == 0) chain_fail(c);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  } else if (blockIdx.x == 0) {
    chain_collect(c, step - 1, tag);
  } else if (threadIdx.x == 0) {
    uint32_t n = 0;
    const uint32_t* dw = c.done + ((size_t)(step - 1) * kDoneReplicas + blockIdx.x % kDoneReplicas) * 16;
    while (load_coherent(dw) != tag) {
      if (++n > c.spin || load_coherent(c.error) != 0u) {
        chain_fail(c);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// One workgroup's share (logical block `lblock`) of one GEMV launch.  CHAIN:
// the call is a step of a chain (chain_kernel): the weight prologue goes out
// before the wait for the previous step, and the activations are read, and y
// written, through the device coherence point.
template <int QT, int B, bool XF32, bool MF, int NW, int DEPTH, bool CHAIN, class GA>
__device__ __forceinline__ bool gemv_block(GA& a, int lblock, const ChainCtl* ctl, int step, uint32_t tag,
                                           bool wait = true, int gate = 0) {
  using F = Fmt<QT>;
  constexpr int NCH = F::kChunks, SB = F::kSubBlocks;
  constexpr int XW = 128;                          // 32-bit words per staged (bf16) row
  // B staged rows; fp32 activations give two per output row (XStage), which
  // are added back together before the tile's epilogue
  constexpr int BU = XF32 ? B / 2 : B;
  extern __shared__ uint32_t lds_words[];
  // readfirstlane: the wavefront index is uniform across the wavefront; saying so
  // keeps all unit/column bookkeeping in SGPRs.
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_cols = a.n_cols;
  // The workgroup's columns [cs, cs + cw) and its run of units [U0, U1),
  // numbered tile-major inside those columns (unit u: tile u / cw, column
  // cs + u % cw).  Without windows cs = 0, cw = n_cols and the runs split the
  // whole unit range evenly; with windows each workgroup takes whole tiles of
  // one window.
  int cs = 0, cw = n_cols, w = 0, U0, U1;
  if (a.tiles_per_wg > 0) {
    w = lblock / a.wg_per_win;
    const int t_first = (lblock - w * a.wg_per_win) * a.tiles_per_wg;
    if (w >= a.n_win || t_first >= a.n_tiles) return false;   // whole workgroup idle
    cs = w * a.win_base + min(w, a.win_extra);
    cw = a.win_base + (w < a.win_extra ? 1 : 0);
    U0 = t_first * cw;
    U1 = min(t_first + a.tiles_per_wg, a.n_tiles) * cw;
  } else {
    U0 = lblock * a.wgu;
    if (U0 >= a.n_units) return false;               // whole workgroup idle
    U1 = min(U0 + a.wgu, a.n_units);
  }
  const int c0w = cs + U0 % cw;                    // staged columns c0w, c0w+1, ... (mod n_cols)
  const int len = min(cw, U1 - U0);
  uint32_t* X = lds_words;
  float* T = reinterpret_cast<float*>(lds_words + a.tsb * B * XW);   // Q4_K/Q5_K sub-block sums (dot2 path)
  constexpr int TSB = QT == KQ_Q6_K ? 0 : SB;                         // T entries per column and row
  // the staged columns' sums of squares (normalised launches only), then the
  // per-wavefront tile sums [NW][tpw][B][64]
  const bool norm = a.rms_eps > 0.0f;
  float* Q2 = MF ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(lds_words) +
                                            a.tsb * MfmaLds<QT, B>::kPerCol + 512)
                 : T + a.tsb * TSB * B;
  float* P = norm ? Q2 + ((a.tsb * B + 3) & ~3) : Q2;
  if (!norm) Q2 = nullptr;
  // DYN (one or two staged rows, one 8-wavefront workgroup per CU): instead of fixed runs the
  // wavefronts take the workgroup's units one at a time from an LDS counter, so
  // a wavefront that gets fewer issue slots than its neighbours simply computes
  // fewer units; each unit's row sums go to an LDS slot of their own and a
  // tile's slots are added in unit order, so y does not depend on which
  // wavefront computed what.  P then holds the counter (16 bytes) and the slots
  // [U1 - U0][B][64].
  constexpr bool DYN = dyn_units<B, NW, MF>();
  // the dynamic prologue fills buffer k with unit wid + k * NW and the LDS
  // counter starts past them; that numbering is written for two buffers
  static_assert(!DYN || DEPTH == 2, "dynamic units assume two weight buffers");
  // wavefront i's part of the run: [run_begin(i), run_begin(i + 1))
  const int run_base = (U1 - U0) / NW, run_ext = (U1 - U0) % NW;
  auto run_begin = [&](int i) { return U0 + i * run_base + min(i, run_ext); };
  const int u0 = DYN ? U0 + wid : run_begin(wid);
  const int u1 = DYN ? U1 : run_begin(wid + 1);
  const bool active = u0 < U1;
  const int t0 = u0 / cw;                          // first tile of this wavefront
  // The weight stream runs DEPTH-1 units ahead of the unit being computed.
  // The first DEPTH-1 units' loads go out before the activations are staged,
  // so their latency overlaps the staging.
  u32x4 buf[DEPTH][NCH];
  uint32_t d6[DEPTH];
#pragma unroll
  for (int k = 0; k < DEPTH; ++k) d6[k] = 0;       // Q4_K / Q5_K never load it
  int ul = u0, tl = t0, cl = cs + u0 % cw;         // next unit to load
  auto refill = [&](int k) {
    load_unit<QT>(unit_rsrc<QT>(a, tl, cl, ul < u1), lane, buf[k], d6[k]);
    ++ul;
    if (++cl == cs + cw) { cl = cs; ++tl; }
    // keep the loads ahead of the computation that follows: neither the IR
    // passes nor the machine scheduler may move work across this point
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // first round of activation loads, then the weight prologue, then the stores
  constexpr int kRS = MF ? MfmaLds<QT, B>::kXRow : 512;
  XStage<QT, B, XF32, NW, kRS> xs;
  if constexpr (CHAIN) {
    // before the step barrier every buffer is filled (DYN: the first unit), so
    // twice as many weights stream in while the previous step drains.  (Filling
    // the last buffer after the activation loads instead, so that they do not
    // wait for its weights, measured slower.)
#pragma unroll
    for (int k = 0; k + 1 < DEPTH; ++k) refill(k);
    if constexpr (!DYN) refill(DEPTH - 1);
    if (wait) chain_wait<!DYN>(*ctl, gate, tag);
    tl_stamp(ctl, step, 1);
    xs.template load<true>(a, c0w, len, 0);
  } else {
    xs.template load<false>(a, c0w, len, 0);
#pragma unroll
    for (int k = 0; k + 1 < DEPTH; ++k) refill(k);
  }
  if constexpr (DYN) {
    if (threadIdx.x == 0) *reinterpret_cast<uint32_t*>(P) = (DEPTH - 1) * NW;   // the prologue took units 0..NW-1
  }
  {
    uint8_t* Xb = reinterpret_cast<uint8_t*>(lds_words);
    // the sub-block sums: after the dot2 path's staged rows, or in the matrix-core path's T block
    constexpr int TS = MF ? MfmaLds<QT, B>::NB * 4 : B;
    float* Ts = MF ? reinterpret_cast<float*>(Xb + len * MfmaLds<QT, B>::kXCol) : T;
    xs.template store<TSB != 0, TS, MF>(Xb, Ts, Q2, len, 0);
    const int nr = XStage<QT, B, XF32, NW, kRS>::rounds(len);
    for (int r = 1; r < nr; ++r) {
      xs.template load<CHAIN>(a, c0w, len, r);
      xs.template store<TSB != 0, TS, MF>(Xb, Ts, Q2, len, r);
    }
    if constexpr (MF) {
      const int z_base = len * MfmaLds<QT, B>::kPerCol;
      if (threadIdx.x < 32) *reinterpret_cast<u32x4*>(Xb + z_base + threadIdx.x * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
  if constexpr (CHAIN) tl_stamp(ctl, step, 2);

  if constexpr (DYN) {
    // unit indices (relative to U0) held by the buffers; >= n: nothing
    uint32_t* ctr = reinterpret_cast<uint32_t*>(P);
    float* S = P + 4;
    const int n = U1 - U0;
    int kb[DEPTH];
#pragma unroll
    for (int k = 0; k + 1 < DEPTH; ++k) kb[k] = wid + k * NW;
    auto grab = [&]() -> int {
      uint32_t v = 0;
      if (lane == 0) v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return (int)__builtin_amdgcn_readfirstlane(v);
    };
    auto refill_unit = [&](int k, int idx) {
      const int U = U0 + idx;
      const int tu = U / cw;
      load_unit<QT>(unit_rsrc<QT>(a, tu, cs + (U - tu * cw), idx < n), lane, buf[k], d6[k]);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // the index for the next refill is taken one step early, so the LDS
    // atomic's latency hides behind a unit's arithmetic
    int nxt = grab();
    bool more = true;
    while (more) {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) {
        const int nk = (k + DEPTH - 1) % DEPTH;
        kb[nk] = nxt;
        refill_unit(nk, nxt);
        nxt = grab();
        if (kb[k] >= n) {
          more = false;
          break;
        }
        const int U = U0 + kb[k];
        int ic = cs + U % cw - c0w;
        if (ic < 0) ic += cw;
        float acc[B];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = 0.0f;
        process_unit<QT, B>(buf[k], d6[k], X + ic * B * XW, T + ic * TSB * B, acc);
#pragma unroll
        for (int b = 0; b < B; ++b) S[(kb[k] * B + b) * kTileRows + lane] = acc[b];
      }
    }
  } else if (active) {
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    int t = t0, c = cs + u0 % cw;
    int ic = c - c0w;
    if (ic < 0) ic += cw;
    int u = u0;
    // consume buf[k] (unit u); at a tile's last unit or the run's end park the sum in LDS
    auto consume = [&](int k) {
      if constexpr (MF) {
        constexpr int NB = MfmaLds<QT, B>::NB;
        uint8_t* base = reinterpret_cast<uint8_t*>(lds_words);
        const int t_base = len * MfmaLds<QT, B>::kXCol, z_base = t_base + len * MfmaLds<QT, B>::kTCol;
        const uint8_t* ap[NB];
        const uint8_t* tp[NB];
        int ts[NB];
#pragma unroll
        for (int gb = 0; gb < NB; ++gb) {
          ap[gb] = base + a_operand_offset<B>(lane, gb, ic, 0, z_base);
          tp[gb] = base + t_operand_offset<QT, B>(lane, gb, ic, t_base, z_base, ts[gb]);
        }
        process_unit_mfma<QT, B, CHAIN>(buf[k], d6[k], ap, tp, ts, acc);
      } else {
        process_unit<QT, B>(buf[k], d6[k], X + ic * B * XW, T + ic * TSB * B, acc);
      }
      if (c == cs + cw - 1 || u + 1 == u1) {
        float* pw = P + ((wid * a.tpw + (t - t0)) * B) * kTileRows;
#pragma unroll
        for (int b = 0; b < B; ++b) {
          pw[b * kTileRows + lane] = acc[b];
          acc[b] = 0.0f;
        }
      }
      ++u;
      if (++c == cs + cw) { c = cs; ++t; }
      if (++ic == cw) ic = 0;
    };
    // Each step issues the load of unit u+DEPTH-1 into the buffer the previous
    // step freed, then computes unit u.  Loads past the run are issued too,
    // through a zero-size resource, so every step has the same loads in flight
    // and the wait before a computation is for its own unit only.
    if constexpr (CHAIN) {
      // every buffer was filled before the barrier: compute, then refill the
      // buffer just freed (the same loads in flight as below, one step later)
      while (u < u1) {
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
          if (u < u1) consume(k);
          refill(k);
        }
      }
    } else {
      while (u < u1) {
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
          refill((k + DEPTH - 1) % DEPTH);
          if (u < u1) consume(k);
        }
      }
    }
  }
  __syncthreads();
  if constexpr (CHAIN) tl_stamp(ctl, step, 3);

  // Each tile of the workgroup: add the wavefronts' sums in wavefront order;
  // write y if the workgroup covered the whole tile, else hand it over.
  const int tA = U0 / cw, tB = (U1 - 1) / cw;
  for (int t = tA + wid; t <= tB; t += NW) {
    const int ts = t * cw, te = ts + cw;
    float s[B];
#pragma unroll
    for (int b = 0; b < B; ++b) s[b] = 0.0f;
    if constexpr (DYN) {
      // the tile's unit slots in unit order; four slots are read before they
      // are added, so the reads overlap (the order of the additions is kept)
      const float* S = P + 4;
      int U = max(U0, ts);
      const int Ue = min(U1, te);
      for (; U + 4 <= Ue; U += 4) {
        float r[4][B];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int b = 0; b < B; ++b) r[j][b] = S[((U + j - U0) * B + b) * kTileRows + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int b = 0; b < B; ++b) s[b] += r[j][b];
      }
      for (; U < Ue; ++U)
#pragma unroll
        for (int b = 0; b < B; ++b) s[b] += S[((U - U0) * B + b) * kTileRows + lane];
    } else {
      for (int i = 0; i < NW; ++i) {
        const int a0 = run_begin(i), a1 = run_begin(i + 1);
        if (max(a0, ts) >= min(a1, te)) continue;
        const float* pw = P + ((i * a.tpw + (t - a0 / cw)) * B) * kTileRows;
#pragma unroll
        for (int b = 0; b < B; ++b) s[b] += pw[b * kTileRows + lane];
      }
    }
    // fp32 activations: each output row's hi and lo sums
    float su[BU];
#pragma unroll
    for (int b = 0; b < BU; ++b) su[b] = XF32 ? s[b] + s[b + BU] : s[b];
    // normalised launches: the sum of x^2 over the workgroup's columns of tile t.
    // Lanes take the columns, then a xor butterfly adds across the wavefront; at
    // every level both partners add the same two values, so all lanes end with
    // the same bits.
    float q[BU];
#pragma unroll
    for (int b = 0; b < BU; ++b) q[b] = 0.0f;
    if (norm) {
      for (int U = max(U0, ts) + lane; U < min(U1, te); U += 64) {
        int ic = cs + U % cw - c0w;
        if (ic < 0) ic += cw;
#pragma unroll
        for (int b = 0; b < BU; ++b) q[b] += Q2[ic * BU + b];
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
        for (int b = 0; b < BU; ++b) q[b] += __shfl_xor(q[b], m);
    }
    if (a.n_win > 1) {
      hand_off_windows<BU, CHAIN>(a, t, w, lane, su, q);
    } else if (ts >= U0 && te <= U1) {   // every tile when tiles_per_wg > 0
      if (norm) rms_scale<BU>(a, su, q);
      write_tile<BU, CHAIN>(a, t, lane, su);
    } else {
      hand_off<BU, CHAIN>(a, t, lblock, a.wgu, lane, su, q);
    }
  }
  if constexpr (CHAIN) tl_stamp(ctl, step, 4);
  return wait;
}

// ---------------------------------------------------------------- chains
//
// A chain is a sequence of GEMV steps where step j+1 may read, as its
// activations, what step j wrote (the decoder's projections, one after the
// other).  One persistent launch runs them all: every workgroup of the grid (all
// resident at once: the grid is sized from the occupancy) takes its share of
// step 0, then of step 1, and so on.  Before reading a step's activations a
// workgroup waits at the step barrier (chain_wait) for every workgroup to have
// finished the previous step; the weight prologue of the step goes out before
// that wait, so the weights stream in while the previous step drains, and
// there is no launch gap between steps.  A workgroup arrives at step j (idle or
// not) once its stores of the step are complete.  The barrier words carry the
// run's tag (one more than the last completed run's, kept in `epoch`), so they
// need no reset between runs; workgroup 0 bumps the epoch once every workgroup
// has arrived at the last step.

// The step table is read through the constant address space: it is not written
// during the launch, so its fields load into SGPRs with scalar loads and stay
// valid across the weight loop's compiler barriers.
typedef const __attribute__((address_space(4))) ChainStep ConstChainStep;

template <int B, bool XF32, bool MF, int NW>
__global__ void __launch_bounds__(64 * NW) chain_kernel(const ChainArgs c) {
  ConstChainStep* steps = (ConstChainStep*)(c.steps);
  // a wait of an earlier run gave up (and the chain has not been reset): the
  // counters may be inconsistent, so this run does nothing.  (A workgroup that
  // starts after a wait of this same run gave up returns too; that run's
  // results are invalid and reported either way.)
  if (__builtin_amdgcn_readfirstlane(load_coherent(c.ctl.error)) != 0u) return;
  const uint32_t tag = __builtin_amdgcn_readfirstlane(load_coherent(c.ctl.epoch)) + 1u;
  // the latest barrier sub-step this workgroup has passed: every sub-step before
  // it is complete on every workgroup
  int passed = 0;
  for (int j = 0; j < c.n_steps; ++j) {
    ConstChainStep& st = steps[j];
    const int g = st.grid;
    tl_stamp(&c.ctl, j, 0);
    // A sub-step reads its x once the barrier of its gate (itself, or for a
    // sub-step that is no barrier the latest barrier sub-step before it) has
    // been passed.  Not barriers: a further weight type of the same step (it
    // reads the same x as the sub-step before it and writes other outputs), and
    // a step whose buffers meet none of those of the sub-steps since its gate
    // (KQ_STEP_OVERLAP).  A workgroup that had no work in the gate sub-step has
    // not passed its barrier yet, so its first block here waits at it.
    const int gate = st.gate;
    bool waited = passed >= gate;
    // the step's logical blocks, as a single launch numbers them, grid-stride
    // over the resident workgroups from workgroup st.first on (the launch and
    // st.first are multiples of 8, so every logical block keeps the XCD it would
    // have had); the first block with work waits at the step barrier
    for (int vb = ((int)blockIdx.x + (int)gridDim.x - st.first) % (int)gridDim.x; vb < g; vb += gridDim.x) {
      const int lblock = (vb & 7) * (g >> 3) + (vb >> 3);
      if (st.type == KQ_Q4_K)
        waited |= gemv_block<KQ_Q4_K, B, XF32, MF, NW, KQ_DEPTH, true>(st.a, lblock, &c.ctl, j, tag, !waited,
                                                                             gate);
      else if (st.type == KQ_Q5_K)
        waited |= gemv_block<KQ_Q5_K, B, XF32, MF, NW, KQ_DEPTH, true>(st.a, lblock, &c.ctl, j, tag, !waited,
                                                                             gate);
      else
        waited |= gemv_block<KQ_Q6_K, B, XF32, MF, NW, KQ_DEPTH, true>(st.a, lblock, &c.ctl, j, tag, !waited,
                                                                             gate);
    }
    // the collector of the two-hop wait never skips a barrier sub-step
    if constexpr (dyn_units<B, NW, MF>()) {
      if (blockIdx.x == 0 && j > 0 && st.wait && !waited) {
        chain_collect(c.ctl, j - 1, tag);
        waited = true;
      }
    }
    if (waited && gate > passed) passed = gate;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wavefront's y / partial stores are done
    __syncthreads();
    if (threadIdx.x == 0) store_coherent(c.ctl.arrive + (size_t)j * c.ctl.groups + blockIdx.x, tag);
    tl_stamp(&c.ctl, j, 5);
  }
  tl_ids(&c.ctl);
  if (blockIdx.x == 0) {
    chain_collect(c.ctl, c.n_steps - 1, tag);
    if (threadIdx.x == 0) store_coherent(c.ctl.epoch, tag);
  }
}

template <int QT, int B, bool XF32, bool MF, int NW, int DEPTH>
__global__ void __launch_bounds__(64 * NW) gemv_kernel(const GemvArgs a) {
  // Blocks are dispatched round-robin over the 8 XCDs; consecutive logical
  // blocks (which share split tiles) go to one XCD.
  const int nb8 = gridDim.x >> 3;
  gemv_block<QT, B, XF32, MF, NW, DEPTH, false>(a, (blockIdx.x & 7) * nb8 + (blockIdx.x >> 3), nullptr, 0, 0u);
}

template <int QT, int B, bool XF32, bool MF>
static hipError_t launch_nw(const GemvArgs& a, int nw, int grid, size_t lds, hipStream_t s) {
  if (nw == 8)
    hipLaunchKernelGGL((gemv_kernel<QT, B, XF32, MF, 8, KQ_DEPTH>), dim3(grid), dim3(512), lds, s, a);
  else
    hipLaunchKernelGGL((gemv_kernel<QT, B, XF32, MF, 4, KQ_DEPTH>), dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int QT, int B, bool XF32>
static hipError_t launch_wide(const GemvArgs& a, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((gemv_kernel<QT, B, XF32, true, 8, KQ_DEPTH>), dim3(grid), dim3(512), lds, s, a);
  return hipGetLastError();
}

// Both paths exist at every batch.
template <int QT, int B, bool XF32>
static hipError_t launch_one(const GemvArgs& a, int nw, bool mf, int grid, size_t lds, hipStream_t s) {
  if (mf) return launch_nw<QT, B, XF32, true>(a, nw, grid, lds, s);
  return launch_nw<QT, B, XF32, false>(a, nw, grid, lds, s);
}

// `rows`: staged rows, the batch (bf16 activations) or twice the batch (fp32).
template <int QT, bool XF32>
static hipError_t launch_b(const GemvArgs& a, int rows, int nw, bool mf, int grid, size_t lds, hipStream_t s) {
  if constexpr (XF32) {
    switch (rows) {
      case 2: return launch_one<QT, 2, true>(a, nw, mf, grid, lds, s);
      case 4: return launch_one<QT, 4, true>(a, nw, mf, grid, lds, s);
      case 6: return launch_one<QT, 6, true>(a, nw, mf, grid, lds, s);
      case 8: return launch_one<QT, 8, true>(a, nw, mf, grid, lds, s);
      default: break;
    }
  } else {
    switch (rows) {
      case 1: return launch_one<QT, 1, false>(a, nw, mf, grid, lds, s);
      case 2: return launch_one<QT, 2, false>(a, nw, mf, grid, lds, s);
      case 3: return launch_one<QT, 3, false>(a, nw, mf, grid, lds, s);
      case 4: return launch_one<QT, 4, false>(a, nw, mf, grid, lds, s);
      case 5: return launch_one<QT, 5, false>(a, nw, mf, grid, lds, s);
      case 6: return launch_one<QT, 6, false>(a, nw, mf, grid, lds, s);
      case 7: return launch_one<QT, 7, false>(a, nw, mf, grid, lds, s);
      case 8: return launch_one<QT, 8, false>(a, nw, mf, grid, lds, s);
      default: break;
    }
  }
  // 9..16 staged rows: matrix cores, 8-wavefront workgroups
  if (!mf || nw != 8) return hipErrorInvalidValue;
  if constexpr (XF32) {
    switch (rows) {
      case 10: return launch_wide<QT, 10, true>(a, grid, lds, s);
      case 12: return launch_wide<QT, 12, true>(a, grid, lds, s);
      case 14: return launch_wide<QT, 14, true>(a, grid, lds, s);
      case 16: return launch_wide<QT, 16, true>(a, grid, lds, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (rows) {
      case 9: return launch_wide<QT, 9, false>(a, grid, lds, s);
      case 10: return launch_wide<QT, 10, false>(a, grid, lds, s);
      case 11: return launch_wide<QT, 11, false>(a, grid, lds, s);
      case 12: return launch_wide<QT, 12, false>(a, grid, lds, s);
      case 13: return launch_wide<QT, 13, false>(a, grid, lds, s);
      case 14: return launch_wide<QT, 14, false>(a, grid, lds, s);
      case 15: return launch_wide<QT, 15, false>(a, grid, lds, s);
      case 16: return launch_wide<QT, 16, false>(a, grid, lds, s);
      default: return hipErrorInvalidValue;
    }
  }
}

template <int B, bool XF32, bool MF>
static hipError_t launch_chain_nw(const ChainArgs& c, int nw, int grid, size_t lds, hipStream_t s, int* occupancy) {
  const void* k = nw == 8 ? reinterpret_cast<const void*>(&chain_kernel<B, XF32, MF, 8>)
                          : reinterpret_cast<const void*>(&chain_kernel<B, XF32, MF, 4>);
  if (occupancy) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, k, 64 * nw, lds);
  if (nw == 8) hipLaunchKernelGGL((chain_kernel<B, XF32, MF, 8>), dim3(grid), dim3(512), lds, s, c);
  else hipLaunchKernelGGL((chain_kernel<B, XF32, MF, 4>), dim3(grid), dim3(256), lds, s, c);
  return hipGetLastError();
}

// Chain launch (or, with `occupancy`, the number of its workgroups one CU
// holds) for B staged rows (the batch, or twice the batch for fp32
// activations) and one activation type.
template <int B, bool XF32>
hipError_t launch_chain_b(const ChainArgs& c, int nw, bool mf, int grid, size_t lds, hipStream_t s, int* occupancy) {
  if (mf) return launch_chain_nw<B, XF32, true>(c, nw, grid, lds, s, occupancy);
  return launch_chain_nw<B, XF32, false>(c, nw, grid, lds, s, occupancy);
}

// Chain launch for 9..16 staged rows (matrix cores, 8-wavefront workgroups).
template <int B, bool XF32>
hipError_t launch_chain_wide(const ChainArgs& c, int grid, size_t lds, hipStream_t s, int* occupancy) {
  const void* k = reinterpret_cast<const void*>(&chain_kernel<B, XF32, true, 8>);
  if (occupancy) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, k, 512, lds);
  hipLaunchKernelGGL((chain_kernel<B, XF32, true, 8>), dim3(grid), dim3(512), lds, s, c);
  return hipGetLastError();
}

// Host entry for one weight type; each type is instantiated in its own
// translation unit (kq_gemv_q4k.hip, ...), which keeps the build parallel.
template <int QT>
hipError_t launch_gemv_type(int xtype, int rows, int nw, bool mf, const GemvArgs& a, int grid, size_t lds,
                            hipStream_t s) {
  return xtype == KQ_X_F32 ? launch_b<QT, true>(a, rows, nw, mf, grid, lds, s)
                           : launch_b<QT, false>(a, rows, nw, mf, grid, lds, s);
}

}  // namespace kq
