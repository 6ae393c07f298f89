// Decode attention over the quantized cache: one launch per call.
//
// Definition ("KV Cache and autoregressive video generation", section 3.1):
// o = sum_t softmax_t(sigma q . k_t) v_t over every cached token, query head
// h reading KV head h / g (section 04).  The quantized prefix is restored
// inside the kernel (k = code / kscale[segment, channel], v = code /
// vscale[token]; "KV Cache Quantization Strategies" Step 4 ``restore``), the
// high-precision tail is read as stored.
//
// Work decomposition (flash-decoding split, the former page, section 05):
// grid = (splits, batch * kv_heads).  The cached tokens form 64-token work
// tiles (quantized tiles, then tail tiles); split s owns a contiguous run of
// tiles, its four waves take tiles round-robin and keep online-softmax
// states (m, l, acc) in the log2 domain.  The workgroup folds its waves into
// one partial, writes it to the workspace, and the last workgroup of each
// (batch, KV head) to arrive -- counted with a device-scope atomic --
// merges all partials and writes the output.  Counters are left at zero.
//
// Scale folding: the per-channel Key scale of a segment is folded into the
// query once per tile (aq = sigma * log2(e) * q / kscale), the per-token
// Value scale into the softmax weight (p / vscale), so the inner loops
// multiply integer codes by those folded factors.
#include "kvq_internal.h"

namespace kvq {

size_t workspace_bytes(const Geom& g, int q_heads, int tq);
size_t workspace_counter_bytes(const Geom& g, int tq);

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

struct DecodeArgs {
  Geom g;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const void* k_tail;
  const void* v_tail;
  const int32_t* seg_index;
  int64_t nq, nt;
  const void* q;
  float qscale;          // sigma * log2(e)
  float* out;
  float* part;           // [unit][split][gqa][D + 2]
  int* counters;         // [unit]
  int splits;
  int tiles_q, tiles;    // quantized tiles, all tiles
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

template <int D, int BITS, int GQA>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  constexpr int W = D * BITS / 8;        // bytes per token row
  constexpr int NSLOT = W / 16;          // 16-byte units per lane per tile
  constexpr int TPU = 128 / BITS;        // tokens per Value unit
  constexpr int FPW = 32 / BITS;         // fields per 32-bit word
  const Geom& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int unit = blockIdx.y;           // b * H + kvh
  const int b = unit / g.H, kvh = unit % g.H;
  const int split = blockIdx.x;

  __shared__ float qs[GQA][D];
  __shared__ float aq[kWaves][D][GQA];
  __shared__ float pw[kWaves][kTile][GQA];
  __shared__ float red[kWaves][D][GQA];
  __shared__ float wml[kWaves][2][GQA];
  __shared__ int last_flag;

  for (int i = tid; i < GQA * D; i += kThreads) {
    const int h = i / D, c = i % D;
    qs[h][c] = load_elem(a.q, ((int64_t)b * g.H * GQA + kvh * GQA + h) * D + c, g.dtype) * a.qscale;
  }
  __syncthreads();

  float m[GQA], l[GQA], acc[NSLOT][GQA];
#pragma unroll
  for (int h = 0; h < GQA; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) acc[k][h] = 0.0f;
  }

  const int t_begin = (int)(((int64_t)a.tiles * split) / a.splits);
  const int t_end = (int)(((int64_t)a.tiles * (split + 1)) / a.splits);
  const int64_t stream_off = (int64_t)unit * g.code_stream;
  int64_t cur_seg = -1;

  for (int tile = t_begin + wave; tile < t_end; tile += kWaves) {
    const bool quant = tile < a.tiles_q;
    float logit[GQA];
#pragma unroll
    for (int h = 0; h < GQA; ++h) logit[h] = 0.0f;
    bool valid;
    float vinv = 1.0f;   // 1 / max(vscale, eps) of this lane's token

    if (quant) {
      const int64_t t = (int64_t)tile * kTile + lane;
      valid = t < a.nq;
      const uint8_t* kt = a.k_codes + stream_off + (int64_t)tile * kTile * W;
      if (g.G > 0) {
        const int64_t seg = ((int64_t)tile * kTile) / g.G;
        if (seg != cur_seg) {
          cur_seg = seg;
          const uint16_t* ks = a.k_scale + ((int64_t)unit * g.max_seg + seg) * D;
          wave_lds_sync();
          for (int c = lane; c < D; c += kWave) {
            const float r = 1.0f / fmaxf(half_bits_to_f32(ks[c]), g.eps);
#pragma unroll
            for (int h = 0; h < GQA; ++h) aq[wave][c][h] = qs[h][c] * r;
          }
          wave_lds_sync();
        }
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
          const uint4 v = *reinterpret_cast<const uint4*>(kt + j * 1024 + lane * 16);
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int f = 0; f < FPW; ++f) {
              const int c = (j * 16 + w * 4) * (8 / BITS) + f;
              const float code = static_cast<float>(sext_field<BITS>(wd[w], f * BITS));
#pragma unroll
              for (int h = 0; h < GQA; ++h) logit[h] = fmaf(aq[wave][c][h], code, logit[h]);
            }
          }
        }
      } else if (valid) {
        // One segment per flush: the segment varies per token.
        const int64_t seg = a.seg_index[t];
        const uint16_t* ks = a.k_scale + ((int64_t)unit * g.max_seg + seg) * D;
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
          const uint4 v = *reinterpret_cast<const uint4*>(kt + j * 1024 + lane * 16);
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int f = 0; f < FPW; ++f) {
              const int c = (j * 16 + w * 4) * (8 / BITS) + f;
              const float kh = static_cast<float>(sext_field<BITS>(wd[w], f * BITS)) /
                               fmaxf(half_bits_to_f32(ks[c]), g.eps);
#pragma unroll
              for (int h = 0; h < GQA; ++h) logit[h] = fmaf(qs[h][c], kh, logit[h]);
            }
          }
        }
      }
      if (valid) vinv = 1.0f / fmaxf(half_bits_to_f32(a.v_scale[(int64_t)unit * g.C + t]), g.eps);
    } else {
      const int64_t tt = (int64_t)(tile - a.tiles_q) * kTile + lane;   // index within the tail
      valid = tt < a.nt;
      if (valid) {
        const int64_t slot = (a.nq + tt) % g.ring;
        const int64_t row = ((int64_t)unit * g.ring + slot) * D;
        for (int c = 0; c < D; ++c) {
          const float kv = load_elem(a.k_tail, row + c, g.dtype);
#pragma unroll
          for (int h = 0; h < GQA; ++h) logit[h] = fmaf(qs[h][c], kv, logit[h]);
        }
      }
    }

    // Online softmax over this tile (log2 domain), one state per head.
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      const float x = valid ? logit[h] : -INFINITY;
      const float mt = wave_max(x);
      const float mn = fmaxf(m[h], mt);
      const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(m[h] - mn);
      const float p = valid ? exp2f(x - mn) : 0.0f;
      l[h] = l[h] * alpha + wave_sum(p);
      m[h] = mn;
#pragma unroll
      for (int k = 0; k < NSLOT; ++k) acc[k][h] *= alpha;
      pw[wave][lane][h] = p * vinv;
    }
    wave_lds_sync();

    // Values: lane owns NSLOT (channel, token-run) units of the tile.
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) {
      const int u = k * kWave + lane;
      const int c = u * 16 / (8 * BITS);
      const int t0 = ((u * 16) % (8 * BITS)) * 8 / BITS;
      if (quant) {
        const uint8_t* vt = a.v_codes + stream_off + (int64_t)tile * kTile * W;
        const uint4 v = *reinterpret_cast<const uint4*>(vt + u * 16);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int f = 0; f < TPU; ++f) {
          const float code = static_cast<float>(sext_field<BITS>(wd[f / FPW], (f % FPW) * BITS));
#pragma unroll
          for (int h = 0; h < GQA; ++h) acc[k][h] = fmaf(pw[wave][t0 + f][h], code, acc[k][h]);
        }
      } else {
        const int64_t base_tt = (int64_t)(tile - a.tiles_q) * kTile;
        for (int f = 0; f < TPU; ++f) {
          const int64_t tt = base_tt + t0 + f;
          if (tt >= a.nt) break;
          const int64_t slot = (a.nq + tt) % g.ring;
          const float vv = load_elem(a.v_tail, ((int64_t)unit * g.ring + slot) * D + c, g.dtype);
#pragma unroll
          for (int h = 0; h < GQA; ++h) acc[k][h] = fmaf(pw[wave][t0 + f][h], vv, acc[k][h]);
        }
      }
    }
  }

  // ---- fold the four waves into one partial ----------------------------------
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      wml[wave][0][h] = m[h];
      wml[wave][1][h] = l[h];
    }
  }
  __syncthreads();
  float M[GQA], wscale[GQA];
#pragma unroll
  for (int h = 0; h < GQA; ++h) {
    float mx = -INFINITY;
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wml[w][0][h]);
    M[h] = mx;
    wscale[h] = (mx == -INFINITY) ? 0.0f : exp2f(m[h] - mx);
  }
  // Lanes that share a channel hold different token runs of it: sum them.
#pragma unroll
  for (int k = 0; k < NSLOT; ++k) {
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      float v = acc[k][h] * wscale[h];
      if (BITS == 8) {
        v += __shfl_xor(v, 1, kWave);
        v += __shfl_xor(v, 2, kWave);
      } else if (BITS == 4) {
        v += __shfl_xor(v, 1, kWave);
      }
      acc[k][h] = v;
    }
  }
#pragma unroll
  for (int k = 0; k < NSLOT; ++k) {
    const int u = k * kWave + lane;
    if (u % (BITS / 2) == 0) {
      const int c = u * 2 / BITS;
#pragma unroll
      for (int h = 0; h < GQA; ++h) red[wave][c][h] = acc[k][h];
    }
  }
  __syncthreads();
  float* part = a.part + ((int64_t)unit * a.splits + split) * GQA * (D + 2);
  for (int i = tid; i < GQA * D; i += kThreads) {
    const int h = i / D, c = i % D;
    float s = 0.0f;
    for (int w = 0; w < kWaves; ++w) s += red[w][c][h];
    part[h * (D + 2) + c] = s;
  }
  if (tid < GQA) {
    const int h = tid;
    float L = 0.0f;
    for (int w = 0; w < kWaves; ++w)
      L += (M[h] == -INFINITY) ? 0.0f : wml[w][1][h] * exp2f(wml[w][0][h] - M[h]);
    part[h * (D + 2) + D] = M[h];
    part[h * (D + 2) + D + 1] = L;
  }

  // ---- last workgroup of this (batch, KV head) merges the splits ---------------
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(&a.counters[unit], 1);
    last_flag = (prev == a.splits - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* pu = a.part + (int64_t)unit * a.splits * GQA * (D + 2);
  for (int i = tid; i < GQA * D; i += kThreads) {
    const int h = i / D, c = i % D;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, __builtin_nontemporal_load(&pu[(s * GQA + h) * (D + 2) + D]));
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < a.splits; ++s) {
      const float* ps = pu + (s * GQA + h) * (D + 2);
      const float ms = __builtin_nontemporal_load(&ps[D]);
      if (ms == -INFINITY) continue;
      const float e = exp2f(ms - mx);
      num += __builtin_nontemporal_load(&ps[c]) * e;
      den += __builtin_nontemporal_load(&ps[D + 1]) * e;
    }
    a.out[((int64_t)b * g.H * GQA + kvh * GQA + h) * D + c] = num / den;
  }
  if (tid == 0) a.counters[unit] = 0;
}

template <int D, int BITS, int GQA>
void launch(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.splits, a.g.B * a.g.H);
  hipLaunchKernelGGL((decode_kernel<D, BITS, GQA>), grid, dim3(kThreads), 0, s, a);
}

template <int D, int BITS>
bool dispatch_gqa(const DecodeArgs& a, int gqa, hipStream_t s) {
  switch (gqa) {
    case 1: launch<D, BITS, 1>(a, s); return true;
    case 2: launch<D, BITS, 2>(a, s); return true;
    case 4: launch<D, BITS, 4>(a, s); return true;
    case 8: launch<D, BITS, 8>(a, s); return true;
  }
  return false;
}

bool dispatch(const DecodeArgs& a, int gqa, hipStream_t s) {
  const int D = a.g.D, bits = a.g.bits;
  if (D == 16 && bits == 8) return dispatch_gqa<16, 8>(a, gqa, s);
  if (D == 32 && bits == 8) return dispatch_gqa<32, 8>(a, gqa, s);
  if (D == 32 && bits == 4) return dispatch_gqa<32, 4>(a, gqa, s);
  if (D == 64 && bits == 8) return dispatch_gqa<64, 8>(a, gqa, s);
  if (D == 64 && bits == 4) return dispatch_gqa<64, 4>(a, gqa, s);
  if (D == 64 && bits == 2) return dispatch_gqa<64, 2>(a, gqa, s);
  if (D == 128 && bits == 8) return dispatch_gqa<128, 8>(a, gqa, s);
  if (D == 128 && bits == 4) return dispatch_gqa<128, 4>(a, gqa, s);
  if (D == 128 && bits == 2) return dispatch_gqa<128, 2>(a, gqa, s);
  return false;
}

}  // namespace

int auto_splits(int units, int tiles) {
  // Aim for about two workgroups per compute unit (256 CUs), at least two
  // tiles per workgroup, and never more splits than tiles.
  int s = (2 * 256 + units - 1) / units;
  const int max_by_tiles = tiles / 2 > 0 ? tiles / 2 : 1;
  if (s > max_by_tiles) s = max_by_tiles;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : s;
}

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_decode_attn(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                                      const void* q, int32_t q_heads, float softmax_scale,
                                      int32_t num_splits, float* out, void* workspace,
                                      size_t workspace_size, void* stream) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!st || !cache || !q || !out) return KVQ_EINVAL;
  if (q_heads < 1 || q_heads % g.H != 0) return KVQ_EINVAL;
  const int gqa = q_heads / g.H;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8) return KVQ_EINVAL;
  if (st->quantized < 0 || st->tail < 0 || st->total != st->quantized + st->tail || st->total < 1 ||
      st->quantized > g.C || st->tail > g.ring)
    return KVQ_EINVAL;
  if (g.G > 0 && st->quantized % g.G != 0) return KVQ_EINVAL;
  if (!(softmax_scale == softmax_scale) || num_splits < 0 || num_splits > kMaxSplits) return KVQ_EINVAL;
  if (st->quantized > 0 && (!cache->k_codes || !cache->v_codes || !cache->k_scale || !cache->v_scale ||
                            (g.G == 0 && !cache->seg_index)))
    return KVQ_EINVAL;
  if (st->tail > 0 && (!cache->k_tail || !cache->v_tail)) return KVQ_EINVAL;
  if (!workspace || workspace_size < workspace_bytes(g, q_heads, 1)) return KVQ_EWORKSPACE;

  DecodeArgs a;
  a.g = g;
  a.k_codes = static_cast<const uint8_t*>(cache->k_codes);
  a.v_codes = static_cast<const uint8_t*>(cache->v_codes);
  a.k_scale = static_cast<const uint16_t*>(cache->k_scale);
  a.v_scale = static_cast<const uint16_t*>(cache->v_scale);
  a.k_tail = cache->k_tail;
  a.v_tail = cache->v_tail;
  a.seg_index = static_cast<const int32_t*>(cache->seg_index);
  a.nq = st->quantized;
  a.nt = st->tail;
  a.q = q;
  a.qscale = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.counters = static_cast<int*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + workspace_counter_bytes(g, 1));
  a.tiles_q = static_cast<int>((st->quantized + kTile - 1) / kTile);
  a.tiles = a.tiles_q + static_cast<int>((st->tail + kTile - 1) / kTile);
  const int units = g.B * g.H;
  a.splits = num_splits > 0 ? num_splits : auto_splits(units, a.tiles);
  if (!dispatch(a, gqa, static_cast<hipStream_t>(stream))) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}
