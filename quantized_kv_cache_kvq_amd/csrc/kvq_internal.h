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
constexpr int kRunChannels = 64;  // channels per scale in same-axis caches

// Launch geometry derived once from a validated kvq_config.
struct Geom {
  int B, H, D, C, bits, qmax, R, G, max_seg, dtype;
  float eps;
  int W;              // packed bytes per token row
  int ring;           // tail ring slots
  int64_t code_stream;  // bytes of one (b, h) code stream = C * W
  int scheme;         // kvq_scheme
  int runs;           // same-axis: scales per token (head_dim / kRunChannels); KIVI: 0
  int kernel;         // kvq_decode_kernel
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

// ---- cross-lane reductions ---------------------------------------------------------
// Within a row of 16 lanes: DPP quad permutations, then half-row and row
// mirrors (every lane of the row ends with the result).  Across the wave: the
// four row results are read into scalar registers.

// Full-row permutations only (every lane has a source), so the DPP move has
// no "old" operand and folds into the consuming add / max (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  return v;
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  v += dpp_f<kDppRowMirror>(v);
  return v;
}

// Value of lane `lane` (wave-uniform index) as a wave-uniform scalar.
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Order LDS traffic between the lanes of one wave.  A wave's LDS operations
// complete in issue order, so only the compiler needs fencing; a wider fence
// would also wait for every outstanding global load of the wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---- host helpers ----------------------------------------------------------------

// HIP reports a failed launch through the calling thread's last-error slot.
// Entry points clear whatever an earlier, unrelated HIP call left there
// before they launch, so KVQ_EDEVICE reports their own launches only.
inline void clear_stale_hip_error() { (void)hipGetLastError(); }

kvq_status validate_config(const kvq_config* cfg, Geom* g);

// Entry points built for the KIVI axes only (block attention, restore, paged
// caches): a same-axis configuration is an invalid argument there.
inline kvq_status validate_kivi_config(const kvq_config* cfg, Geom* g) {
  const kvq_status s = validate_config(cfg, g);
  return s != KVQ_OK ? s : (g->scheme == KVQ_KIVI ? KVQ_OK : KVQ_EINVAL);
}

}  // namespace kvq
