// Shared device-side definitions of the K-quant GEMV library (gfx950).
//
// Repacked layout (see kq.h, kq_repacked_bytes): a "tile" is 64 rows x one
// super-block column; chunk k (16 B) of row r's super-block sits at
// k*1024 + 16*r inside the tile, so each chunk is one coalesced 1 KiB
// wavefront load with lane == row.
//
// Chunk contents per super-block (256 weights):
//   Q4_K (9 chunks):  0: the 16 GGUF header bytes (fp16 d, fp16 dmin, 12 bytes
//                        of packed 6-bit scale/min);
//                     1+g: the 32 four-bit quants of sub-block g (g = 0..7).
//   Q5_K (11 chunks): 0..8 as Q4_K (low four bits), 9..10: eight 32-bit words
//                     H_g holding the fifth bits of sub-block g.
//   Q6_K (13 chunks + 2 B tail): k = 0..7: low-nibble words of sub-blocks 2k and
//                     2k+1 (two words each, sub-blocks of 16); 8+k: 32-bit words
//                     H_g of the two high bits of sub-blocks 4k..4k+3;
//                     12: the 16 int8 sub-block scales; tail: fp16 d.
//
// The quants become EXACT bf16 operands, with no offset, so every sub-block's
// dot product S = sum v * x is rounded relative to sum |v x| alone:
//   Q4_K: a quant word for sub-block elements 8j .. 8j+7 holds element 8j+k
//         (k < 4) in the low nibble of byte k and element 8j+4+k in its high
//         nibble.  word & 0x0F0F0F0F and (word >> 4) & 0x0F0F0F0F put one quant
//         per byte; read as OCP fp8 e4m3, bytes 0..15 are the subnormal and
//         first normal binade, i.e. exactly q * 2^-9, and the conversion to
//         bf16 with scale 2^9 (v_cvt_scalef32_pk_bf16_fp8, two bytes per
//         instruction) yields the pair (q, q') exactly.
//   Q5_K: the same low nibbles, plus the fifth bit of element 8j+4h+k at bit
//         8k + (2j+h) of H_g; merged into bit 4 of the byte, each byte holds
//         q in 0..31 and v_cvt_f32_ubyte{0..3} + v_cvt_pk_bf16_f32 give
//         exact bf16 q.
//   Q6_K: element 8j+4h+k of a sub-block keeps its low nibble at bits 8k+4h of
//         low word j and its two high bits, with the top one inverted, at bits
//         8k+2m (m = 2j+h) of H_g.  The byte (nibble << 2) | (high << 6) is
//         then the two's-complement int8 4*(q-32); the sign-extending byte
//         conversion (v_cvt_f32_i32 with an SDWA byte select) and
//         v_cvt_pk_bf16_f32 give exact bf16 4*(q-32), and d*sc/4 scales it.
// Pairs follow the activation pairs (x_{2i}, x_{2i+1}) of the same position.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kq.h"

namespace kq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 64;
constexpr int kChunk = 16;                      // bytes per lane per chunk
constexpr int kChunkStride = kTileRows * kChunk;  // 1024 bytes between chunks of one tile
// Word 3 of a raw (untyped, stride 0) buffer resource on gfx950: 32-bit data
// format, bounds checked against num_records.
constexpr int kBufferFlags = 0x00020000;
// Cache-policy operand of buffer loads: nontemporal (the weights are read once).
constexpr int kCacheNT = 2;
// buffer-load cache policy: sc1, read through the device coherence point
constexpr int kCacheCoherent = 16;

template <int QT> struct Fmt;
template <> struct Fmt<KQ_Q4_K> {
  static constexpr int kSbBytes = 144, kChunks = 9, kSubBlocks = 8, kSubW = 32, kPairs = 16;
};
template <> struct Fmt<KQ_Q5_K> {
  static constexpr int kSbBytes = 176, kChunks = 11, kSubBlocks = 8, kSubW = 32, kPairs = 16;
};
template <> struct Fmt<KQ_Q6_K> {
  static constexpr int kSbBytes = 210, kChunks = 13, kSubBlocks = 16, kSubW = 16, kPairs = 8;
};
template <int QT> constexpr int64_t tile_bytes() { return (int64_t)kTileRows * Fmt<QT>::kSbBytes; }

// Hides a constant from the optimiser so that it stays in a VGPR; gfx9 VOP3
// encodings take no literal, and a register operand lets the compiler fuse
// shift-free extractions into one v_and_or_b32.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// (a & m) | b in one v_and_or_b32 (the compiler otherwise splits the Q6_K
// three-way merge into and/and/or3).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t b) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(b));
  return r;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ uint32_t word(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Exact bf16 operand pairs of sub-block G of one super-block held in chunks
// c[]: Q4_K/Q5_K q (16 pairs), Q6_K 4*(q-32) (8 pairs); see the layout above.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t v) {
  // scale 2^9: e4m3 bytes 0..15 are q * 2^-9, so the result is exactly q
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 512.0f, HI_WORD));
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  // small integers: exact in bf16 (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

template <int QT>
__device__ __forceinline__ void unpack_pairs(const u32x4* c, int G, uint32_t* pr) {
  if constexpr (QT == KQ_Q4_K) {
    const u32x4 q = c[1 + G];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = word(q, j);
      const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
      pr[4 * j + 0] = fp8x2_to_bf16x2<false>(lo);
      pr[4 * j + 1] = fp8x2_to_bf16x2<true>(lo);
      pr[4 * j + 2] = fp8x2_to_bf16x2<false>(hi);
      pr[4 * j + 3] = fp8x2_to_bf16x2<true>(hi);
    }
  } else if constexpr (QT == KQ_Q5_K) {
    const u32x4 q = c[1 + G];
    const uint32_t H = word(c[9 + G / 4], G % 4);
    const uint32_t M4 = in_vgpr(0x0F0F0F0Fu), M5 = in_vgpr(0x10101010u);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t v = word(q, t / 2);
      const uint32_t base = (t & 1) ? ((v >> 4) & M4) : (v & M4);
      const uint32_t hs = t <= 4 ? (H << (4 - t)) : (H >> (t - 4));
      const uint32_t b = and_or(hs, M5, base);
      pr[2 * t + 0] = pk_bf16((float)(b & 0xFFu), (float)((b >> 8) & 0xFFu));
      pr[2 * t + 1] = pk_bf16((float)((b >> 16) & 0xFFu), (float)(b >> 24));
    }
  } else {
    const u32x4 lq = c[G / 2];
    const uint32_t H = word(c[8 + G / 4], G % 4);
    const uint32_t M6 = in_vgpr(0x3C3C3C3Cu), MH = in_vgpr(0xC0C0C0C0u);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t L = word(lq, (G % 2) * 2 + m / 2);
      const uint32_t lf = ((m & 1) ? (L >> 2) : (L << 2)) & M6;
      const uint32_t b = and_or(H << (6 - 2 * m), MH, lf);   // int8 bytes 4*(q-32)
      pr[2 * m + 0] = pk_bf16((float)(int8_t)(b & 0xFFu), (float)(int8_t)((b >> 8) & 0xFFu));
      pr[2 * m + 1] = pk_bf16((float)(int8_t)((b >> 16) & 0xFFu), (float)(int8_t)(b >> 24));
    }
  }
}

// Per-sub-block coefficients from the super-block header (exact products).
//   Q4_K/Q5_K: a[g] = d*sc_g, cm[g] = dmin*m_g.
//   Q6_K     : a[g] = d*sc_g / 4 (the operands are 4*(q-32)).
template <int QT>
__device__ __forceinline__ void sb_coeffs(const u32x4* c, uint32_t d6bits, float* a, float* cm) {
  if constexpr (QT == KQ_Q4_K || QT == KQ_Q5_K) {
    const u32x4 h = c[0];
    const float d = f16_bits_to_f32(h.x);
    const float dm = f16_bits_to_f32(h.x >> 16);
    const uint32_t sc_lo = h.y & 0x3F3F3F3Fu;
    const uint32_t m_lo = h.z & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t m_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = d * (float)((sc_lo >> (8 * i)) & 0xFFu);
      a[4 + i] = d * (float)((sc_hi >> (8 * i)) & 0xFFu);
      cm[i] = dm * (float)((m_lo >> (8 * i)) & 0xFFu);
      cm[4 + i] = dm * (float)((m_hi >> (8 * i)) & 0xFFu);
    }
  } else {
    const float d = f16_bits_to_f32(d6bits) * 0.25f;
    const u32x4 s = c[12];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t sc = (int32_t)(word(s, i / 4) << (24 - 8 * (i % 4))) >> 24;
      a[i] = d * (float)sc;
    }
    (void)cm;
  }
}

}  // namespace kq
