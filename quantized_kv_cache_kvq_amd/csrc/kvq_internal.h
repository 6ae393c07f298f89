// Internal helpers shared by the libkvq translation units (device + host).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kTile = 64;         // tokens per packed tile
constexpr int kWave = 64;         // gfx950 wavefront width
constexpr int kMaxSplits = 256;   // sequence splits per (batch, KV head) in decode
constexpr int kMaxGqa = 8;        // query heads per KV head supported by the kernels

// Launch geometry derived once from a validated kvq_config.
struct Geom {
  int B, H, D, C, bits, qmax, R, G, max_seg, dtype;
  float eps;
  int W;              // packed bytes per token row
  int ring;           // tail ring slots
  int64_t code_stream;  // bytes of one (b, h) code stream = C * W
};

// ---- scalar conversions (device) -------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Load element i of a K/V/Q array stored as bf16 (dtype 0) or fp32 (dtype 1).
__device__ __forceinline__ float load_elem(const void* base, int64_t i, int dtype) {
  if (dtype == KVQ_BF16)
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  return static_cast<const float*>(base)[i];
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Round-to-nearest-even fp32 -> fp16 (hardware conversion, default round mode).
__device__ __forceinline__ uint16_t f32_to_half_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Sign-extend a b-bit two's-complement field.
template <int BITS>
__device__ __forceinline__ int sext_field(uint32_t word, int shift) {
  return static_cast<int>(word << (32 - BITS - shift)) >> (32 - BITS);
}

// ---- wave reductions -------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- host helpers ----------------------------------------------------------------

kvq_status validate_config(const kvq_config* cfg, Geom* g);

}  // namespace kvq
