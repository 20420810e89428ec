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
// Inside a quant word for sub-block elements 8j .. 8j+7, nibble p (bits
// 4p..4p+3) holds element 8j+2p and bits 16+4p.. hold element 8j+2p+1, so
// ((word >> 4p) & 0x000F000F) | 0x43004300 is a pair of bf16 values
// (128 + q_{8j+2p}, 128 + q_{8j+2p+1}) matching the bf16 activation pair at the
// same position.  The high-bit words put the bits of pair pi = 4j+p at bit pi
// (Q5_K; plus 16 for the second element) or bits 2pi..2pi+1 (Q6_K; plus 16).
// bf16 represents 128 + q exactly for q < 128, so every weight enters the dot
// product exactly; the 128 (Q6_K: 160 = 128 + 32) offset is removed per
// sub-block with a sum of the activations accumulated in the same order.
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

template <int S> __device__ __forceinline__ uint32_t shift_signed(uint32_t v) {
  if constexpr (S > 0) return v >> S;
  else if constexpr (S < 0) return v << (-S);
  else return v;
}

__device__ __forceinline__ uint32_t word(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// bf16 pairs (offset + q) of sub-block G of one super-block held in chunks c[].
// Q4_K/Q5_K: 16 pairs, offset 128; Q6_K: 8 pairs, offset 128 (q in 0..63).
template <int QT>
__device__ __forceinline__ void unpack_pairs(const u32x4* c, int G, uint32_t M, uint32_t K, uint32_t* pr) {
  if constexpr (QT == KQ_Q4_K || QT == KQ_Q5_K) {
    const u32x4 q = c[1 + G];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = word(q, j);
      pr[4 * j + 0] = (v & M) | K;
      pr[4 * j + 1] = ((v >> 4) & M) | K;
      pr[4 * j + 2] = ((v >> 8) & M) | K;
      pr[4 * j + 3] = ((v >> 12) & M) | K;
    }
    if constexpr (QT == KQ_Q5_K) {
      const uint32_t H = word(c[9 + G / 4], G % 4);
      const uint32_t M5 = in_vgpr(0x00100010u);
#define KQ_Q5_HB(PI) pr[PI] = and_or(shift_signed<(PI) - 4>(H), M5, pr[PI]);
      KQ_Q5_HB(0) KQ_Q5_HB(1) KQ_Q5_HB(2) KQ_Q5_HB(3) KQ_Q5_HB(4) KQ_Q5_HB(5) KQ_Q5_HB(6) KQ_Q5_HB(7)
      KQ_Q5_HB(8) KQ_Q5_HB(9) KQ_Q5_HB(10) KQ_Q5_HB(11) KQ_Q5_HB(12) KQ_Q5_HB(13) KQ_Q5_HB(14) KQ_Q5_HB(15)
#undef KQ_Q5_HB
    }
  } else {
    const u32x4 lq = c[G / 2];
    const uint32_t L0 = word(lq, (G % 2) * 2), L1 = word(lq, (G % 2) * 2 + 1);
    const uint32_t H = word(c[8 + G / 4], G % 4);
    const uint32_t M6 = in_vgpr(0x00300030u);
    // pair pi: nibbles of L_{pi/4} >> 4(pi%4), two high bits of H >> (2pi - 4)
#define KQ_Q6_PAIR(PI, L, P) pr[PI] = and_or(shift_signed<2 * (PI) - 4>(H), M6, and_or(shift_signed<4 * (P)>(L), M, K));
    KQ_Q6_PAIR(0, L0, 0) KQ_Q6_PAIR(1, L0, 1) KQ_Q6_PAIR(2, L0, 2) KQ_Q6_PAIR(3, L0, 3)
    KQ_Q6_PAIR(4, L1, 0) KQ_Q6_PAIR(5, L1, 1) KQ_Q6_PAIR(6, L1, 2) KQ_Q6_PAIR(7, L1, 3)
#undef KQ_Q6_PAIR
  }
}

// Per-sub-block coefficients from the super-block header.
//   Q4_K/Q5_K: a[g] = d*sc_g, cm[g] = dmin*m_g * cm_scale (exact products).
//   Q6_K     : a[g] = d*sc_g.
template <int QT>
__device__ __forceinline__ void sb_coeffs(const u32x4* c, uint32_t d6bits, float cm_scale, float* a, float* cm) {
  if constexpr (QT == KQ_Q4_K || QT == KQ_Q5_K) {
    const u32x4 h = c[0];
    const float d = f16_bits_to_f32(h.x);
    const float dm = f16_bits_to_f32(h.x >> 16) * cm_scale;
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
    const float d = f16_bits_to_f32(d6bits);
    const u32x4 s = c[12];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t sc = (int32_t)(word(s, i / 4) << (24 - 8 * (i % 4))) >> 24;
      a[i] = d * (float)sc;
    }
    (void)cm;
    (void)cm_scale;
  }
}

}  // namespace kq
