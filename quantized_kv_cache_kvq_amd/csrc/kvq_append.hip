// Append path: token accounting on the host, flush-quantize and tail-ring
// writes on the device.
//
// Method ("KV Cache Quantization Strategies", Steps 3-4): the newest
// ``residual`` tokens stay in high precision; only tokens that overflow the
// window are quantized, as new segments after the existing ones.  Keys get
// one scale per channel per segment (absmax over the segment's tokens),
// Values one scale per token (absmax over head_dim); scale = qmax /
// max(absmax, eps) in fp32, stored as fp16 clamped to 65504; codes =
// clamp(rne(fp32(x) * scale16), -qmax, qmax), packed as b-bit fields.
//
// Device work of one append, in stream order:
//   1. flush_kernel  -- one workgroup per (new segment, batch*head).  Tokens
//      are read straight from the old tail ring or from the new input (the
//      "concatenation" is virtual), reduced, scaled, rounded and packed.
//   2. tail_kernel   -- copies the new tokens that stay in the window into
//      their ring slots.  It runs after the flush because a ring slot being
//      refilled may hold a token the flush is still reading.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kFlushThreads = 256;
constexpr int kVChunk = 1024;  // tokens per Value-scale staging chunk (64-aligned)

struct FlushArgs {
  Geom g;
  const void* k_new;
  const void* v_new;
  int64_t n_new;
  const void* k_tail;
  const void* v_tail;
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_scale;
  uint16_t* v_scale;
  int32_t* seg_index;
  int64_t nq_old, nt_old;  // accounting before this append
  int64_t seg_base;        // id of the first segment written by this launch
  int64_t seg_len;         // tokens per segment (G, or the whole flush when G == 0)
};

// Token at absolute position p of stream bh, channel c: from the old tail
// ring if it was already cached, else from the new input.
__device__ __forceinline__ float flush_src(const FlushArgs& a, bool key, int bh, int64_t p, int c) {
  const Geom& g = a.g;
  const int64_t old_end = a.nq_old + a.nt_old;
  if (p < old_end) {
    const int64_t slot = p % g.ring;
    return load_elem(key ? a.k_tail : a.v_tail, ((int64_t)bh * g.ring + slot) * g.D + c, g.dtype);
  }
  const int64_t i = p - old_end;
  return load_elem(key ? a.k_new : a.v_new, ((int64_t)bh * a.n_new + i) * g.D + c, g.dtype);
}

__device__ __forceinline__ float scale_of(float absmax, int qmax, float eps) {
  // qmax / max(absmax, eps): one correctly rounded fp32 division, then the
  // fp16 storage rounding (half-to-even) after clamping to the fp16 range.
  const float s32 = __fdiv_rn(static_cast<float>(qmax), fmaxf(absmax, eps));
  return fminf(s32, 65504.0f);
}

__device__ __forceinline__ uint32_t code_field(float x, float s, int qmax, uint32_t mask) {
  const float r = __builtin_rintf(__fmul_rn(x, s));   // fp32 product, ties to even
  const float cl = fminf(fmaxf(r, -static_cast<float>(qmax)), static_cast<float>(qmax));
  return static_cast<uint32_t>(static_cast<int>(cl)) & mask;
}

template <int BITS>
__global__ __launch_bounds__(kFlushThreads) void flush_kernel(FlushArgs a) {
  constexpr int kPer = 8 / BITS;             // fields per byte
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const Geom& g = a.g;
  const int D = g.D;
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int64_t seg = a.seg_base + blockIdx.x;
  const int64_t p0 = a.nq_old + (int64_t)blockIdx.x * a.seg_len;
  const int64_t p1 = p0 + a.seg_len;

  __shared__ float red[kFlushThreads];
  __shared__ float kscale[128];
  __shared__ float vscale[kVChunk];

  // ---- Keys: per-channel absmax over the segment's tokens -----------------------
  {
    const int c = tid % D;
    const int nsub = kFlushThreads / D;
    const int sub = tid / D;
    float m = 0.0f;
    for (int64_t p = p0 + sub; p < p1; p += nsub) m = fmaxf(m, fabsf(flush_src(a, true, bh, p, c)));
    red[tid] = m;
    __syncthreads();
    if (tid < D) {
      for (int k = 1; k < nsub; ++k) m = fmaxf(m, red[k * D + tid]);
      const uint16_t h = f32_to_half_bits(scale_of(m, g.qmax, g.eps));
      a.k_scale[((int64_t)bh * g.max_seg + seg) * D + tid] = h;
      kscale[tid] = half_bits_to_f32(h);
    }
    __syncthreads();
  }

  // ---- Key codes: one 16-byte chunk of one token row per thread ------------------
  {
    uint8_t* kc = a.k_codes + (int64_t)bh * g.code_stream;
    const int chunks = g.W / 16;
    const int64_t items = (p1 - p0) * chunks;
    for (int64_t it = tid; it < items; it += kFlushThreads) {
      const int64_t p = p0 + it / chunks;
      const int j = static_cast<int>(it % chunks);
      uint32_t w4[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
        const int c0 = (j * 16 + w * 4) * kPer;
#pragma unroll
        for (int f = 0; f < 4 * kPer; ++f) {
          const int c = c0 + f;
          word |= code_field(flush_src(a, true, bh, p, c), kscale[c], g.qmax, kMask) << (f * BITS);
        }
        w4[w] = word;
      }
      const int64_t off = (p / kTile) * kTile * g.W + (int64_t)j * 1024 + (p % kTile) * 16;
      *reinterpret_cast<uint4*>(kc + off) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }

  // ---- Values: per-token scales and codes, in 64-aligned chunks of tokens --------
  uint8_t* vc = a.v_codes + (int64_t)bh * g.code_stream;
  const int wave = tid / kWave, lane = tid % kWave;
  constexpr int kTokPerWord = 32 / BITS;
  for (int64_t t0 = (p0 / kTile) * kTile; t0 < p1; t0 += kVChunk) {
    const int64_t cs = t0 > p0 ? t0 : p0;
    const int64_t ce = (t0 + kVChunk) < p1 ? (t0 + kVChunk) : p1;
    __syncthreads();
    for (int64_t p = cs + wave; p < ce; p += kFlushThreads / kWave) {
      float m = 0.0f;
      for (int c = lane; c < D; c += kWave) m = fmaxf(m, fabsf(flush_src(a, false, bh, p, c)));
      m = wave_max(m);
      if (lane == 0) {
        const uint16_t h = f32_to_half_bits(scale_of(m, g.qmax, g.eps));
        a.v_scale[(int64_t)bh * g.C + p] = h;
        vscale[p - t0] = half_bits_to_f32(h);
      }
    }
    __syncthreads();
    // Words of kTokPerWord tokens of one channel; channel fastest so that the
    // source reads of consecutive threads are contiguous.
    const int64_t w_first = cs / kTokPerWord, w_last = (ce - 1) / kTokPerWord;
    const int64_t items = (w_last - w_first + 1) * D;
    for (int64_t it = tid; it < items; it += kFlushThreads) {
      const int c = static_cast<int>(it % D);
      const int64_t wt = (w_first + it / D) * kTokPerWord;   // first token of the word
      const int64_t off = (wt / kTile) * kTile * g.W + (int64_t)c * 8 * BITS + ((wt % kTile) * BITS) / 8;
      uint32_t* dst = reinterpret_cast<uint32_t*>(vc + off);
      uint32_t word = 0;
      if (wt < cs) {
        // Only at an unaligned segment start (group == 0): keep the fields of
        // the previous segment's tokens.
        const int keep = static_cast<int>(cs - wt);
        word = *dst & ((1u << (keep * BITS)) - 1u);
      }
#pragma unroll
      for (int f = 0; f < kTokPerWord; ++f) {
        const int64_t t = wt + f;
        if (t >= cs && t < ce)
          word |= code_field(flush_src(a, false, bh, t, c), vscale[t - t0], g.qmax, kMask) << (f * BITS);
      }
      *dst = word;
    }
  }

  // ---- group == 0: record the segment id of every flushed token ------------------
  if (g.G == 0 && bh == 0) {
    for (int64_t p = p0 + tid; p < p1; p += kFlushThreads) a.seg_index[p] = static_cast<int32_t>(seg);
  }
}

struct TailArgs {
  const uint8_t* k_new;
  const uint8_t* v_new;
  uint8_t* k_tail;
  uint8_t* v_tail;
  int64_t n_new;      // tokens in the input
  int64_t first;      // first input token that stays in the window
  int64_t count;      // tokens that stay
  int64_t pos0;       // absolute position of input token 0
  int ring;
  int row16;          // 16-byte chunks per token row
  int BH;
};

__global__ __launch_bounds__(256) void tail_kernel(TailArgs a) {
  const int64_t per_bh = a.count * a.row16;
  const int64_t total = per_bh * a.BH * 2;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < total;
       it += (int64_t)gridDim.x * blockDim.x) {
    const bool val = it >= per_bh * a.BH;
    const int64_t r = val ? it - per_bh * a.BH : it;
    const int64_t bh = r / per_bh;
    const int64_t rem = r % per_bh;
    const int64_t i = a.first + rem / a.row16;        // input token
    const int64_t ch = rem % a.row16;
    const int64_t slot = (a.pos0 + i) % a.ring;
    const uint4* src = reinterpret_cast<const uint4*>(val ? a.v_new : a.k_new) +
                       (bh * a.n_new + i) * a.row16 + ch;
    uint4* dst = reinterpret_cast<uint4*>(val ? a.v_tail : a.k_tail) + (bh * a.ring + slot) * a.row16 + ch;
    *dst = *src;
  }
}

kvq_status check_state(const Geom& g, const kvq_state* st) {
  if (!st) return KVQ_EINVAL;
  if (st->quantized < 0 || st->tail < 0 || st->total != st->quantized + st->tail) return KVQ_EINVAL;
  if (st->quantized > g.C || st->tail > g.ring || st->segments < 0 || st->segments > g.max_seg)
    return KVQ_EINVAL;
  if (g.G > 0 && (st->quantized % g.G != 0 || st->segments != st->quantized / g.G)) return KVQ_EINVAL;
  if (g.G == 0 && st->quantized > 0 && st->tail != g.R) return KVQ_EINVAL;
  if (g.G == 0 && st->quantized == 0 && st->segments != 0) return KVQ_EINVAL;
  return KVQ_OK;
}

}  // namespace

kvq_status plan_append(const Geom& g, const kvq_state* st, int64_t n_new, kvq_state* next) {
  if (n_new < 0) return KVQ_EINVAL;
  kvq_status s = check_state(g, st);
  if (s != KVQ_OK) return s;
  const int64_t len = st->tail + n_new;
  const int64_t overflow = len > g.R ? len - g.R : 0;
  const int64_t flush = g.G == 0 ? overflow : (overflow / g.G) * g.G;
  kvq_state n = *st;
  n.quantized = st->quantized + flush;
  n.tail = len - flush;
  n.total = n.quantized + n.tail;
  n.flushed_last = flush;
  n.segments = st->segments + (flush == 0 ? 0 : (g.G == 0 ? 1 : flush / g.G));
  if (n.quantized > g.C || n.segments > g.max_seg) return KVQ_ECAPACITY;
  *next = n;
  return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_plan_append(const kvq_config* cfg, const kvq_state* st, int64_t n_new,
                                      kvq_state* next) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!next) return KVQ_EINVAL;
  return plan_append(g, st, n_new, next);
}

extern "C" kvq_status kvq_append(const kvq_config* cfg, kvq_state* st, const kvq_cache* cache,
                                 const void* k_new, const void* v_new, int64_t n_new, void* stream) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  kvq_state next;
  s = plan_append(g, st, n_new, &next);
  if (s != KVQ_OK) return s;
  if (n_new == 0) {  // nothing to write; the counters still report "flushed 0"
    *st = next;
    return KVQ_OK;
  }
  if (!cache || !k_new || !v_new || !cache->k_codes || !cache->v_codes || !cache->k_scale ||
      !cache->v_scale || !cache->k_tail || !cache->v_tail || (g.G == 0 && !cache->seg_index))
    return KVQ_EINVAL;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  clear_stale_hip_error();
  const int64_t flush = next.flushed_last;
  if (flush > 0) {
    FlushArgs a;
    a.g = g;
    a.k_new = k_new;
    a.v_new = v_new;
    a.n_new = n_new;
    a.k_tail = cache->k_tail;
    a.v_tail = cache->v_tail;
    a.k_codes = static_cast<uint8_t*>(cache->k_codes);
    a.v_codes = static_cast<uint8_t*>(cache->v_codes);
    a.k_scale = static_cast<uint16_t*>(cache->k_scale);
    a.v_scale = static_cast<uint16_t*>(cache->v_scale);
    a.seg_index = static_cast<int32_t*>(cache->seg_index);
    a.nq_old = st->quantized;
    a.nt_old = st->tail;
    a.seg_base = st->segments;
    a.seg_len = g.G == 0 ? flush : g.G;
    const int64_t nseg = flush / a.seg_len;
    dim3 grid(static_cast<unsigned>(nseg), static_cast<unsigned>(g.B * g.H));
    switch (g.bits) {
      case 8: hipLaunchKernelGGL(flush_kernel<8>, grid, dim3(kFlushThreads), 0, hs, a); break;
      case 4: hipLaunchKernelGGL(flush_kernel<4>, grid, dim3(kFlushThreads), 0, hs, a); break;
      default: hipLaunchKernelGGL(flush_kernel<2>, grid, dim3(kFlushThreads), 0, hs, a); break;
    }
  }
  // New tokens at absolute positions >= next.quantized stay in the window.
  const int64_t old_end = st->quantized + st->tail;
  const int64_t first = next.quantized > old_end ? next.quantized - old_end : 0;
  const int64_t count = n_new - first;
  if (count > 0) {
    TailArgs t;
    t.k_new = static_cast<const uint8_t*>(k_new);
    t.v_new = static_cast<const uint8_t*>(v_new);
    t.k_tail = static_cast<uint8_t*>(cache->k_tail);
    t.v_tail = static_cast<uint8_t*>(cache->v_tail);
    t.n_new = n_new;
    t.first = first;
    t.count = count;
    t.pos0 = old_end;
    t.ring = g.ring;
    t.row16 = g.D * (g.dtype == KVQ_BF16 ? 2 : 4) / 16;
    t.BH = g.B * g.H;
    const int64_t total = count * t.row16 * t.BH * 2;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(tail_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, hs, t);
  }
  if (hipGetLastError() != hipSuccess) return KVQ_EDEVICE;
  *st = next;
  return KVQ_OK;
}
