// One-time repack of GGUF K-quant super-blocks into the wavefront-coalesced
// tile layout (kq_common.h), and the fp32 dequantisation of that layout.
//
// GGUF super-block element order (public GGUF K-quant layout):
//   Q4_K/Q5_K: element 64c + i (i < 32) is the low nibble of qs[32c + i],
//              element 64c + 32 + i its high nibble; the Q5_K fifth bit of
//              element 32g + i is bit g of qh[i].
//   Q6_K: element 128h + 32r + i keeps its low nibble in ql[64h + 32(r&1) + i]
//         (low half for r < 2) and its top two bits in bits 2r..2r+1 of
//         qh[32h + i]; scales[e/16] is its int8 sub-block scale.
#include "kq_common.h"
#include "kq_internal.h"

namespace kq {

// byte i of a super-block held as 32-bit words
template <int N> __device__ __forceinline__ uint32_t byte_at(const uint32_t (&W)[N], int i) {
  return (W[i >> 2] >> (8 * (i & 3))) & 0xFFu;
}

template <int QT> struct Repack;

template <> struct Repack<KQ_Q4_K> {
  static constexpr int kWords = 36;
  // nibble of element e (0..255) from qs bytes starting at byte offset QS
  template <int N> static __device__ __forceinline__ uint32_t nib(const uint32_t (&W)[N], int qs_off, int e) {
    const int c = e / 64, r = e % 64;
    const uint32_t b = byte_at(W, qs_off + 32 * c + (r % 32));
    return (r < 32) ? (b & 15u) : (b >> 4);
  }
  // word j of sub-block g: element 32g + 8j + k (k < 4) in the low nibble of
  // byte k, element 32g + 8j + 4 + k in its high nibble
  template <int N> static __device__ __forceinline__ void quant_chunks(const uint32_t (&W)[N], int qs_off, u32x4* ch) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t o = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o |= nib(W, qs_off, 32 * g + 8 * j + k) << (8 * k);
          o |= nib(W, qs_off, 32 * g + 8 * j + 4 + k) << (8 * k + 4);
        }
        v[j] = o;
      }
      ch[1 + g] = u32x4{v[0], v[1], v[2], v[3]};
    }
  }
  static __device__ __forceinline__ void run(const uint8_t* sb, u32x4* ch, uint16_t& d6) {
    uint32_t W[kWords];
    const uint32_t* p = reinterpret_cast<const uint32_t*>(sb);
#pragma unroll
    for (int i = 0; i < kWords; ++i) W[i] = p[i];
    ch[0] = u32x4{W[0], W[1], W[2], W[3]};
    quant_chunks(W, 16, ch);
    d6 = 0;
  }
};

template <> struct Repack<KQ_Q5_K> {
  static constexpr int kWords = 44;
  static __device__ __forceinline__ void run(const uint8_t* sb, u32x4* ch, uint16_t& d6) {
    uint32_t W[kWords];
    const uint32_t* p = reinterpret_cast<const uint32_t*>(sb);
#pragma unroll
    for (int i = 0; i < kWords; ++i) W[i] = p[i];
    ch[0] = u32x4{W[0], W[1], W[2], W[3]};
    Repack<KQ_Q4_K>::quant_chunks(W, 48, ch);
    // fifth bit of element 32g + 8j + 4h + k at bit 8k + (2j + h) of H_g
    uint32_t H[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      uint32_t o = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = 8 * (t / 2) + 4 * (t % 2) + k;   // element 32g + i
          const uint32_t bit = (byte_at(W, 16 + i) >> g) & 1u;
          o |= bit << (8 * k + t);
        }
      }
      H[g] = o;
    }
    ch[9] = u32x4{H[0], H[1], H[2], H[3]};
    ch[10] = u32x4{H[4], H[5], H[6], H[7]};
    d6 = 0;
  }
};

template <> struct Repack<KQ_Q6_K> {
  static constexpr int kHalves = 105;
  template <int N> static __device__ __forceinline__ uint32_t b16(const uint16_t (&U)[N], int i) {
    return (U[i >> 1] >> (8 * (i & 1))) & 0xFFu;
  }
  template <int N> static __device__ __forceinline__ uint32_t lo(const uint16_t (&U)[N], int e) {
    const int h = e / 128, r = (e % 128) / 32, i = e % 32;
    const uint32_t b = b16(U, 64 * h + 32 * (r & 1) + i);
    return (r < 2) ? (b & 15u) : (b >> 4);
  }
  template <int N> static __device__ __forceinline__ uint32_t hi(const uint16_t (&U)[N], int e) {
    const int h = e / 128, r = (e % 128) / 32, i = e % 32;
    return (b16(U, 128 + 32 * h + i) >> (2 * r)) & 3u;
  }
  static __device__ __forceinline__ void run(const uint8_t* sb, u32x4* ch, uint16_t& d6) {
    uint16_t U[kHalves];
    const uint16_t* p = reinterpret_cast<const uint16_t*>(sb);
#pragma unroll
    for (int i = 0; i < kHalves; ++i) U[i] = p[i];
    // element 16g + 8j + 4h + k: low nibble at bits 8k + 4h of L[g][j]; its two
    // high bits, the top one inverted, at bits 8k + 2m (m = 2j + h) of H[g]
    uint32_t L[16][2], H[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      uint32_t h = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t o = 0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = 16 * g + 8 * j + 4 * hh + k;
            o |= lo(U, e) << (8 * k + 4 * hh);
            h |= (hi(U, e) ^ 2u) << (8 * k + 2 * (2 * j + hh));
          }
        }
        L[g][j] = o;
      }
      H[g] = h;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ch[k] = u32x4{L[2 * k][0], L[2 * k][1], L[2 * k + 1][0], L[2 * k + 1][1]};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) ch[8 + k] = u32x4{H[4 * k], H[4 * k + 1], H[4 * k + 2], H[4 * k + 3]};
    uint32_t S[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) S[k] = (uint32_t)U[96 + 2 * k] | ((uint32_t)U[97 + 2 * k] << 16);
    ch[12] = u32x4{S[0], S[1], S[2], S[3]};
    d6 = U[104];
  }
};

// gguf2 == nullptr: tile t holds rows 64t .. 64t+63 of gguf.  Otherwise (the
// SwiGLU pair) tile t holds rows 32t .. 32t+31 of gguf (gate) in lanes 0..31
// and the same rows of gguf2 (up) in lanes 32..63.  Rows past `rows` are zero.
template <int QT>
__global__ void __launch_bounds__(256) repack_kernel(const uint8_t* __restrict__ gguf, const uint8_t* __restrict__ gguf2,
                                                     uint8_t* __restrict__ out, int64_t rows, int n_cols, int64_t total) {
  using F = Fmt<QT>;
  for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < total; gid += (int64_t)gridDim.x * 256) {
    const int lane = (int)(gid & 63);
    const int64_t unit = gid >> 6;               // tile * n_cols + column
    const int64_t t = unit / n_cols;
    const int c = (int)(unit - t * n_cols);
    const uint8_t* src = gguf;
    int64_t row = t * kTileRows + lane;
    if (gguf2) {
      row = t * (kTileRows / 2) + (lane & 31);
      if (lane >= 32) src = gguf2;
    }
    u32x4 ch[F::kChunks];
    uint16_t d6 = 0;
    if (row < rows) {
      Repack<QT>::run(src + (row * n_cols + c) * F::kSbBytes, ch, d6);
    } else {
#pragma unroll
      for (int k = 0; k < F::kChunks; ++k) ch[k] = u32x4{0u, 0u, 0u, 0u};
    }
    uint8_t* tb = out + unit * tile_bytes<QT>();
#pragma unroll
    for (int k = 0; k < F::kChunks; ++k)
      *reinterpret_cast<u32x4*>(tb + k * kChunkStride + lane * kChunk) = ch[k];
    if constexpr (QT == KQ_Q6_K) reinterpret_cast<uint16_t*>(tb + 13 * kChunkStride)[lane] = d6;
  }
}

// fp32 dequantisation of one super-block (row 64t + lane, column c) of the
// repacked layout, whose unit starts at `tb`, into o[0..255].
template <int QT>
__device__ __forceinline__ void dequant_superblock(const uint8_t* tb, int lane, float* o) {
  using F = Fmt<QT>;
  u32x4 ch[F::kChunks];
#pragma unroll
  for (int k = 0; k < F::kChunks; ++k)
    ch[k] = *reinterpret_cast<const u32x4*>(tb + k * kChunkStride + lane * kChunk);
  uint32_t d6 = 0;
  if constexpr (QT == KQ_Q6_K) d6 = reinterpret_cast<const uint16_t*>(tb + 13 * kChunkStride)[lane];
  float a[F::kSubBlocks], cm[F::kSubBlocks];
  sb_coeffs<QT>(ch, d6, a, cm);
#pragma unroll
  for (int g = 0; g < F::kSubBlocks; ++g) {
    uint32_t pr[F::kPairs];
    unpack_pairs<QT>(ch, g, pr);
#pragma unroll
    for (int i = 0; i < F::kPairs; ++i) {
      const int e = g * F::kSubW + 2 * i;
      if constexpr (QT == KQ_Q6_K) {   // (d*sc/4) * 4(q-32): an exact product
        o[e] = a[g] * bf16_lo(pr[i]);
        o[e + 1] = a[g] * bf16_hi(pr[i]);
      } else {                         // one rounding of d*sc*q - dmin*m
        o[e] = __builtin_fmaf(a[g], bf16_lo(pr[i]), -cm[g]);
        o[e + 1] = __builtin_fmaf(a[g], bf16_hi(pr[i]), -cm[g]);
      }
    }
  }
}

// out[row*ldo + 256c + e] = fp32 dequantised weight, from the repacked layout,
// through the same unpacking the GEMV uses.
template <int QT>
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ w, float* __restrict__ out,
                                                      int64_t rows, int n_cols, int64_t total, int64_t ldo) {
  for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < total; gid += (int64_t)gridDim.x * 256) {
    const int lane = (int)(gid & 63);
    const int64_t unit = gid >> 6;
    const int64_t t = unit / n_cols;
    const int c = (int)(unit - t * n_cols);
    const int64_t row = t * kTileRows + lane;
    if (row >= rows) continue;
    dequant_superblock<QT>(w + unit * tile_bytes<QT>(), lane, out + row * ldo + (int64_t)c * 256);
  }
}

// Row gather (the embedding lookup): out[i*ldo + k] = dequant(W)[ids[i], k] for
// i < n, one thread per (i, super-block column).  An id outside [0, rows) gives
// a row of quiet NaNs and reads nothing.  (One thread per sub-block measured
// slower for a single token.)
template <int QT>
__global__ void __launch_bounds__(256) gather_kernel(const uint8_t* __restrict__ w, const int32_t* __restrict__ ids,
                                                     float* __restrict__ out, int64_t rows, int n_cols, int64_t total,
                                                     int64_t ldo) {
  for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < total; gid += (int64_t)gridDim.x * 256) {
    const int64_t i = gid / n_cols;
    const int c = (int)(gid - i * n_cols);
    const int64_t row = ids[i];
    float* o = out + i * ldo + (int64_t)c * 256;
    if (row < 0 || row >= rows) {
      for (int e = 0; e < 256; ++e) o[e] = __builtin_nanf("");
      continue;
    }
    const int64_t t = row / kTileRows;
    dequant_superblock<QT>(w + (t * n_cols + c) * tile_bytes<QT>(), (int)(row - t * kTileRows), o);
  }
}

// The achievable read rate: every 16-byte chunk of p read once with the
// GEMV's own load (128-bit nontemporal buffer loads), 16 loads in flight per
// wavefront, no arithmetic but an xor; *sink is written only if the xor of
// everything equals a fixed value, so the loads cannot be dropped.
__global__ void __launch_bounds__(256) stream_read_kernel(const uint8_t* __restrict__ p, int64_t chunks,
                                                          uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), waves = (int64_t)gridDim.x * 4;
  constexpr int kIn = 16;                         // chunks of 1 KiB per wavefront in flight
  uint32_t acc = 0;
  for (int64_t c0 = wave * 64 * kIn; c0 < chunks; c0 += waves * 64 * kIn) {
    // one resource per step, based at the step's first byte (offsets stay below 2^31)
    const uint64_t addr = reinterpret_cast<uint64_t>(p) + (uint64_t)c0 * kChunk;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const int64_t left = chunks - c0;
    const int n = __builtin_amdgcn_readfirstlane((int)((left < 64 * kIn ? left : 64 * kIn) * kChunk));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, n, kBufferFlags);
    u32x4 v[kIn];
#pragma unroll
    for (int k = 0; k < kIn; ++k) v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (k * 64 + lane) * kChunk, 0, kCacheNT);
#pragma unroll
    for (int k = 0; k < kIn; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

static int grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  return (int)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

hipError_t launch_repack(int type, int64_t rows, int64_t cols, const void* gguf, const void* gguf2, void* out,
                         hipStream_t s) {
  const int n_cols = (int)(cols / 256);
  const int64_t n_tiles = gguf2 ? (rows + kTileRows / 2 - 1) / (kTileRows / 2) : (rows + kTileRows - 1) / kTileRows;
  const int64_t total = n_tiles * n_cols * kTileRows;
  const uint8_t* in = static_cast<const uint8_t*>(gguf);
  const uint8_t* in2 = static_cast<const uint8_t*>(gguf2);
  uint8_t* o = static_cast<uint8_t*>(out);
  switch (type) {
    case KQ_Q4_K: hipLaunchKernelGGL(repack_kernel<KQ_Q4_K>, dim3(grid_for(total)), dim3(256), 0, s, in, in2, o, rows, n_cols, total); break;
    case KQ_Q5_K: hipLaunchKernelGGL(repack_kernel<KQ_Q5_K>, dim3(grid_for(total)), dim3(256), 0, s, in, in2, o, rows, n_cols, total); break;
    case KQ_Q6_K: hipLaunchKernelGGL(repack_kernel<KQ_Q6_K>, dim3(grid_for(total)), dim3(256), 0, s, in, in2, o, rows, n_cols, total); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(int type, const void* w, int64_t rows, int64_t cols, float* out, int64_t ldo, hipStream_t s) {
  const int n_cols = (int)(cols / 256);
  const int64_t n_tiles = (rows + kTileRows - 1) / kTileRows;
  const int64_t total = n_tiles * n_cols * kTileRows;
  const uint8_t* in = static_cast<const uint8_t*>(w);
  switch (type) {
    case KQ_Q4_K: hipLaunchKernelGGL(dequant_kernel<KQ_Q4_K>, dim3(grid_for(total)), dim3(256), 0, s, in, out, rows, n_cols, total, ldo); break;
    case KQ_Q5_K: hipLaunchKernelGGL(dequant_kernel<KQ_Q5_K>, dim3(grid_for(total)), dim3(256), 0, s, in, out, rows, n_cols, total, ldo); break;
    case KQ_Q6_K: hipLaunchKernelGGL(dequant_kernel<KQ_Q6_K>, dim3(grid_for(total)), dim3(256), 0, s, in, out, rows, n_cols, total, ldo); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gather(int type, const void* w, int64_t rows, int64_t cols, const int32_t* ids, int64_t n,
                         float* out, int64_t ldo, hipStream_t s) {
  const int n_cols = (int)(cols / 256);
  const int64_t total = n * n_cols;
  const uint8_t* in = static_cast<const uint8_t*>(w);
  switch (type) {
    case KQ_Q4_K: hipLaunchKernelGGL(gather_kernel<KQ_Q4_K>, dim3(grid_for(total)), dim3(256), 0, s, in, ids, out, rows, n_cols, total, ldo); break;
    case KQ_Q5_K: hipLaunchKernelGGL(gather_kernel<KQ_Q5_K>, dim3(grid_for(total)), dim3(256), 0, s, in, ids, out, rows, n_cols, total, ldo); break;
    case KQ_Q6_K: hipLaunchKernelGGL(gather_kernel<KQ_Q6_K>, dim3(grid_for(total)), dim3(256), 0, s, in, ids, out, rows, n_cols, total, ldo); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, int groups, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(groups), dim3(256), 0, s, static_cast<const uint8_t*>(p),
                     (int64_t)(bytes / kChunk), sink);
  return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(zero_words_kernel, dim3(grid_for((int64_t)n)), dim3(256), 0, s, p, (int64_t)n);
  return hipGetLastError();
}

}  // namespace kq
