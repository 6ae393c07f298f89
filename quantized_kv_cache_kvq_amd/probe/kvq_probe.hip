// Measurement kernels: the HBM read stream and the matrix-core loop that
// calibrate the rooflines on the machine itself ("KV Cache and
// autoregressive video generation", appendix section [C]: peak bandwidth
// measured by streaming, peak arithmetic by a dense product).  Built into
// libkvq_probe.so, apart from the KV-cache library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxWorkgroups = 1 << 20;

// Workgroup w reads elements [w * per_wg, (w + 1) * per_wg) of the buffer
// (clipped to its end) in rounds of kThreads * DEPTH 16-byte elements: each
// thread issues DEPTH loads, 4 KiB apart across the workgroup, before it
// folds any of them.  One word per workgroup is stored.
template <int DEPTH>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                               int64_t per_wg, uint32_t* sink) {
  const int64_t begin = (int64_t)blockIdx.x * per_wg;
  const int64_t end = begin + per_wg < n16 ? begin + per_wg : n16;
  uint32_t acc = 0u;
  constexpr int64_t kRound = (int64_t)kThreads * DEPTH;
  const int64_t full_end = end - begin >= kRound ? begin + (end - begin) / kRound * kRound : begin;
  for (int64_t base = begin + threadIdx.x; base < full_end; base += kRound) {
    uint4 v[DEPTH];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) v[k] = p[base + (int64_t)k * kThreads];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (full_end < end) {                         // the ragged last round, DEPTH loads in flight
    uint4 v[DEPTH];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      const int64_t i = full_end + threadIdx.x + (int64_t)k * kThreads;
      v[k] = i < end ? p[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0u;
  __syncthreads();
  atomicXor(&red, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red;
}

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Eight independent accumulator chains per wave, operands in registers
// (derived from the lane id so that nothing is constant-folded).
template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, uint32_t* sink) {
  const int lane = threadIdx.x % 64;
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = 0x3C003C00u ^ ((uint32_t)(lane + 17 * i) & 0x00FF00FFu);
  const uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
  uint32_t fold = 0u;
  if constexpr (KIND == 2) {
    const i4_t a = __builtin_bit_cast(i4_t, u);
    const i4_t b = __builtin_bit_cast(i4_t, make_uint4(w[3], w[2], w[1], w[0]));
    i4_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = i4_t{j, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) fold ^= (uint32_t)(acc[j][0] ^ acc[j][1] ^ acc[j][2] ^ acc[j][3]);
  } else if constexpr (KIND == 3 || KIND == 4) {
    // 32x32x16: sixteen accumulator registers per chain
    f32x16_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] = f32x16_t{};
      acc[j][0] = (float)j;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (KIND == 3)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8_t, u),
                                                           __builtin_bit_cast(bf8_t, make_uint4(w[3], w[2], w[1], w[0])),
                                                           acc[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, u),
                                                          __builtin_bit_cast(h8_t, make_uint4(w[3], w[2], w[1], w[0])),
                                                          acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) fold ^= __float_as_uint(acc[j][e]);
  } else {
    f4_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f4_t{(float)j, 0.0f, 0.0f, 0.0f};
    if constexpr (KIND == 0) {
      const bf8_t a = __builtin_bit_cast(bf8_t, u);
      const bf8_t b = __builtin_bit_cast(bf8_t, make_uint4(w[3], w[2], w[1], w[0]));
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
      }
    } else {
      const h8_t a = __builtin_bit_cast(h8_t, u);
      const h8_t b = __builtin_bit_cast(h8_t, make_uint4(w[3], w[2], w[1], w[0]));
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      fold ^= __float_as_uint(acc[j][0]) ^ __float_as_uint(acc[j][1]) ^ __float_as_uint(acc[j][2]) ^
              __float_as_uint(acc[j][3]);
  }
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0u;
  __syncthreads();
  atomicXor(&red, fold);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red;
}

__global__ __launch_bounds__(kThreads) void empty_kernel() {}

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : 4; }

}  // namespace

extern "C" int kvq_probe_stream_read(const void* buf, int64_t bytes, int32_t workgroups, int32_t depth,
                                     uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return 1;
  if (workgroups < 1 || workgroups > kMaxWorkgroups) return 1;
  const int64_t n16 = bytes / 16;
  // Per-workgroup share, whole 128-byte lines.
  int64_t per_wg = (n16 + workgroups - 1) / workgroups;
  per_wg = (per_wg + 7) / 8 * 8;
  const uint4* p = static_cast<const uint4*>(buf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const dim3 grid(workgroups), block(kThreads);
  switch (depth) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, s, p, n16, per_wg, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, s, p, n16, per_wg, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, s, p, n16, per_wg, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, s, p, n16, per_wg, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, grid, block, 0, s, p, n16, per_wg, sink); break;
    default: return 1;
  }
  return launch_status();
}

extern "C" int kvq_probe_mfma(int32_t kind, int32_t workgroups, int32_t iters, uint32_t* sink, void* stream) {
  if (!sink || iters < 1 || workgroups < 1 || workgroups > kMaxWorkgroups) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const dim3 grid(workgroups), block(kThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_kernel<0>, grid, block, 0, s, iters, sink); break;
    case 1: hipLaunchKernelGGL(mfma_kernel<1>, grid, block, 0, s, iters, sink); break;
    case 2: hipLaunchKernelGGL(mfma_kernel<2>, grid, block, 0, s, iters, sink); break;
    case 3: hipLaunchKernelGGL(mfma_kernel<3>, grid, block, 0, s, iters, sink); break;
    case 4: hipLaunchKernelGGL(mfma_kernel<4>, grid, block, 0, s, iters, sink); break;
    default: return 1;
  }
  return launch_status();
}

extern "C" int kvq_probe_empty(int32_t workgroups, void* stream) {
  if (workgroups < 1 || workgroups > kMaxWorkgroups) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(empty_kernel, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream));
  return launch_status();
}
