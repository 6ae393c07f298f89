// Restore of the quantized prefix into a dense array: k = code / max(kscale,
// eps), v = code / max(vscale, eps) ("KV Cache Quantization Strategies",
// Step 4 ``restore``), in fp32 (IEEE division, as the reference restore
// computes it) or rounded once to bf16.
//
// This is the first half of read path (i) of "KV Cache quantization and
// compression", section 06 -- restore the whole history to HBM, then run
// ordinary attention -- which the attention kernels of this library avoid by
// restoring inside the kernel.  It exists for callers that want the dense
// history, and to measure that path against the fused one.
//
// Work: grid = (quantized tiles, batch * KV heads), 256 threads.  Keys:
// item = (token, eight channels), one 2/4/8-byte load of the token's packed
// row and one 16/32-byte store, consecutive lanes on consecutive channels;
// Values: thread = (channel c, a run of tokens), reading the channel's packed
// run, so that the stores of a token row are contiguous across lanes.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kRestoreThreads = 256;

struct RestoreArgs {
  Geom g;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* seg_index;
  void* k_out;
  void* v_out;
  int64_t ld;     // rows per (batch, head) in the outputs
  int nq;
  int out_bf16;
};

__device__ __forceinline__ void store_out(void* base, int64_t i, float x, int bf16) {
  if (bf16) static_cast<__bf16*>(base)[i] = (__bf16)x;   // round to nearest even
  else static_cast<float*>(base)[i] = x;
}

__device__ __forceinline__ float restore_one(int code, uint16_t scale_bits, float eps) {
  return __fdiv_rn((float)code, fmaxf(half_bits_to_f32(scale_bits), eps));
}

template <int D, int BITS>
__global__ __launch_bounds__(kRestoreThreads) void restore_kernel(RestoreArgs a) {
  constexpr int CG = D / 8;                             // Key groups of eight channels per token
  constexpr int TPC = kRestoreThreads / D;              // threads per Value channel
  constexpr int NTV = kTile / TPC;                      // Value tokens per thread
  constexpr int VW = NTV * BITS / 32;                   // their packed 32-bit words
  static_assert(VW >= 1 && (NTV * BITS) % 32 == 0, "restore shapes");
  const Geom& g = a.g;
  const int tile = blockIdx.x, unit = blockIdx.y, tid = threadIdx.x;
  const int t0 = tile * kTile;
  const int count = min(kTile, a.nq - t0);
  const int64_t stream = (int64_t)unit * g.code_stream + (int64_t)tile * (kTile * g.W);
  const int64_t row0 = (int64_t)unit * a.ld + t0;      // output row of the tile's first token

  // ---- Keys: item e = (token e / CG, channels 8 (e % CG) ..): consecutive
  // lanes cover consecutive channels of a row ----
  for (int e = tid; e < kTile * CG; e += kRestoreThreads) {
    const int i = e / CG, cg = e % CG;
    if (i >= count) continue;
    const int t = t0 + i;
    const int r = cg * BITS;                            // first byte of the group in the token's row
    const uint8_t* src = a.k_codes + stream + (r / 16) * 1024 + i * 16 + r % 16;
    uint64_t bits;                                      // 8 fields, low bits first
    if constexpr (BITS == 8) bits = *reinterpret_cast<const uint64_t*>(src);
    else if constexpr (BITS == 4) bits = *reinterpret_cast<const uint32_t*>(src);
    else bits = *reinterpret_cast<const uint16_t*>(src);
    const int seg = g.G > 0 ? t / g.G : a.seg_index[t];
    const uint4 sw = *reinterpret_cast<const uint4*>(a.k_scale + ((int64_t)unit * g.max_seg + seg) * D + 8 * cg);
    const uint32_t sv[4] = {sw.x, sw.y, sw.z, sw.w};
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int code = static_cast<int>(static_cast<int64_t>(bits << (64 - BITS * (j + 1))) >> (64 - BITS));
      x[j] = restore_one(code, (uint16_t)(sv[j / 2] >> (16 * (j % 2))), g.eps);
    }
    const int64_t o = (row0 + i) * D + 8 * cg;
    if (a.out_bf16) {
      __bf16 h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (__bf16)x[j];
      *reinterpret_cast<uint4*>(static_cast<__bf16*>(a.k_out) + o) = __builtin_bit_cast(uint4, h);
    } else {
      float* dst = static_cast<float*>(a.k_out) + o;
      *reinterpret_cast<float4*>(dst) = float4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<float4*>(dst + 4) = float4{x[4], x[5], x[6], x[7]};
    }
  }
  // ---- Values: channel c, tokens j0 .. j0 + NTV - 1 (the channel's packed
  // run); the stores of one token row are contiguous across lanes ----
  {
    const int c = tid % D, j0 = (tid / D) * NTV;
    const uint32_t* vt = reinterpret_cast<const uint32_t*>(a.v_codes + stream + c * (8 * BITS) + j0 * BITS / 8);
    uint32_t vw[VW];
#pragma unroll
    for (int k = 0; k < VW; ++k) vw[k] = vt[k];
    const uint16_t* vs = a.v_scale + (int64_t)unit * g.C + t0 + j0;
#pragma unroll
    for (int j = 0; j < NTV; ++j) {
      if (j0 + j < count) {
        const int code = sext_field<BITS>(vw[j * BITS / 32], (j * BITS) % 32);
        store_out(a.v_out, (row0 + j0 + j) * D + c, restore_one(code, vs[j], g.eps), a.out_bf16);
      }
    }
  }
}

template <int D, int BITS>
bool launch_restore_db(const RestoreArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (D * BITS % 128 == 0) {      // packed rows of whole 16-byte chunks (validated configs)
    hipLaunchKernelGGL((restore_kernel<D, BITS>), grid, dim3(kRestoreThreads), 0, s, a);
    return true;
  }
  return false;
}

template <int D>
bool launch_restore_d(const RestoreArgs& a, dim3 grid, hipStream_t s) {
  switch (a.g.bits) {
    case 8: return launch_restore_db<D, 8>(a, grid, s);
    case 4: return launch_restore_db<D, 4>(a, grid, s);
    case 2: return launch_restore_db<D, 2>(a, grid, s);
  }
  return false;
}

bool launch_restore(const RestoreArgs& a, dim3 grid, hipStream_t s) {
  switch (a.g.D) {
    case 16: return launch_restore_d<16>(a, grid, s);
    case 32: return launch_restore_d<32>(a, grid, s);
    case 64: return launch_restore_d<64>(a, grid, s);
    case 128: return launch_restore_d<128>(a, grid, s);
  }
  return false;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_restore(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                                  void* k_out, void* v_out, int32_t out_dtype, int64_t ld, void* stream) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!st || !cache) return KVQ_EINVAL;
  if (st->quantized < 0 || st->tail < 0 || st->total != st->quantized + st->tail || st->quantized > g.C)
    return KVQ_EINVAL;
  if (g.G > 0 && st->quantized % g.G != 0) return KVQ_EINVAL;
  if (out_dtype != KVQ_BF16 && out_dtype != KVQ_F32) return KVQ_EINVAL;
  if (ld < st->quantized) return KVQ_EINVAL;
  if (st->quantized == 0) return KVQ_OK;      // nothing to restore
  if (!k_out || !v_out || !cache->k_codes || !cache->v_codes || !cache->k_scale || !cache->v_scale ||
      (g.G == 0 && !cache->seg_index))
    return KVQ_EINVAL;
  RestoreArgs a;
  a.g = g;
  a.k_codes = static_cast<const uint8_t*>(cache->k_codes);
  a.v_codes = static_cast<const uint8_t*>(cache->v_codes);
  a.k_scale = static_cast<const uint16_t*>(cache->k_scale);
  a.v_scale = static_cast<const uint16_t*>(cache->v_scale);
  a.seg_index = static_cast<const int32_t*>(cache->seg_index);
  a.k_out = k_out;
  a.v_out = v_out;
  a.ld = ld;
  a.nq = static_cast<int>(st->quantized);
  a.out_bf16 = out_dtype == KVQ_BF16;
  const dim3 grid(static_cast<unsigned>((a.nq + kTile - 1) / kTile), static_cast<unsigned>(g.B * g.H));
  clear_stale_hip_error();
  if (!launch_restore(a, grid, static_cast<hipStream_t>(stream))) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}
