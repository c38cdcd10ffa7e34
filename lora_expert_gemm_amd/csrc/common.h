// Device helpers shared by the gfx950 kernels of the MoE-LoRA layer.
//
// Element storage: bf16 as uint16_t bit patterns, or float.  Every MFMA
// operand a lane supplies is one 16-byte "chunk": 8 bf16 or 4 float values
// that are consecutive along the contraction dimension.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moelora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename DT> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int kPerChunk = 8;
  __device__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
  __device__ static uint16_t from_f32(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};

// The elements of a chunk, as a value (no address taken).
template <typename DT> struct Chunk {
  DT v[Elem<DT>::kPerChunk];
};
template <typename DT>
__device__ __forceinline__ Chunk<DT> chunk_elems(u32x4_t c) {
  return __builtin_bit_cast(Chunk<DT>, c);
}

// One contraction step of a 16x16 output tile:  D[i][j] += sum_k A[i][k] B[k][j]
// where the lane l supplies row i = l % 16 of A and column j = l % 16 of B,
// both as one chunk covering the same contraction indices.  bf16: one
// 16x16x32 MFMA; float: four 16x16x4 MFMAs (element q of each lane's chunk
// goes to the q-th).  Either way the 64 lanes cover 4 chunks = 32 (bf16) or
// 16 (float) contraction indices.  The result layout: lane l holds
// D[4 * (l / 16) + v][l % 16], v = 0..3.
template <typename DT> struct Mma;
template <> struct Mma<uint16_t> {
  static constexpr int kK = 32;
  __device__ __forceinline__ static void step(f32x4_t &c, u32x4_t a, u32x4_t b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int kK = 16;
  __device__ __forceinline__ static void step(f32x4_t &c, u32x4_t a, u32x4_t b) {
    f32x4_t fa = __builtin_bit_cast(f32x4_t, a), fb = __builtin_bit_cast(f32x4_t, b);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[0], fb[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[1], fb[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[2], fb[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[3], fb[3], c, 0, 0, 0);
  }
};

// Chunk of row[k .. k + kPerChunk): one 16-byte load.  The caller
// guarantees the chunk lies inside the row and is 16-byte aligned.
template <typename DT>
__device__ __forceinline__ u32x4_t load_chunk(const DT *row, int k) {
  return *reinterpret_cast<const u32x4_t *>(row + k);
}

// Cache-policy operand of a global load (direct-to-LDS form) that marks it
// non-temporal: the weight stream reads each line once, and so marked it
// streams 10-12 % faster than with the default policy (decode-sized blocks).
constexpr int kCpolNonTemporal = 2;
// Third dword of a raw buffer resource (gfx9 family): 32-bit data format,
// no swizzle, no stride; loads at offsets past num_records return zero and
// touch no memory.
constexpr int kBufferWord3 = 0x00020000;

// Chunk of row[k ..) with zeros past `len`, element by element (any
// alignment).
template <typename DT>
__device__ __forceinline__ u32x4_t load_chunk_masked(const DT *row, int k, int len) {
  constexpr int n = Elem<DT>::kPerChunk;
  DT v[n];
#pragma unroll
  for (int q = 0; q < n; ++q) v[q] = (k + q < len) ? row[k + q] : DT(0);
  return __builtin_bit_cast(u32x4_t, v);
}

// Chunk of row[k ..): vector load when VEC (row 16-byte aligned, len a
// multiple of the chunk) and the chunk is in range; otherwise masked.
template <typename DT, bool VEC>
__device__ __forceinline__ u32x4_t load_chunk_any(const DT *row, int k, int len) {
  if (VEC) {
    if (k < len) return load_chunk(row, k);
    return u32x4_t{0, 0, 0, 0};
  }
  return load_chunk_masked(row, k, len);
}

// Eight (bf16) or four (float) float values as two chunks hi + lo with
// hi + lo equal to the values to about 2^-16 relative (bf16), or one exact
// chunk (float; lo = 0).
template <typename DT> struct SplitF32;
template <> struct SplitF32<uint16_t> {
  __device__ __forceinline__ static void run(const float *v, u32x4_t &hi, u32x4_t &lo) {
    uint16_t h[8], l[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      h[q] = f32_to_bf16(v[q]);
      l[q] = f32_to_bf16(v[q] - bf16_to_f32(h[q]));
    }
    hi = __builtin_bit_cast(u32x4_t, h);
    lo = __builtin_bit_cast(u32x4_t, l);
  }
};
template <> struct SplitF32<float> {
  __device__ __forceinline__ static void run(const float *v, u32x4_t &hi, u32x4_t &lo) {
    hi = __builtin_bit_cast(u32x4_t, f32x4_t{v[0], v[1], v[2], v[3]});
    lo = u32x4_t{0, 0, 0, 0};
  }
};


__device__ __forceinline__ float silu_f32(float v) { return v / (1.0f + __expf(-v)); }

// Eight OCP E4M3 codes (code i in byte i % 4 of w[i / 4]) as one MFMA
// operand chunk of eight bf16 values.  Every E4M3 value is a bf16 value, so
// the conversion (two codes per instruction, scale 1) is exact; an in-bounds
// check of the instruction on all 256 codes, both halves of the source
// dword, matched the format's definition.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  return u32x4_t{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
}

}  // namespace moelora
