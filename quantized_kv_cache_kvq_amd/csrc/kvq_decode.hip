// Decode attention over the quantized cache.
//
// Definition ("KV Cache and autoregressive video generation", section 3.1):
// o = sum_t softmax_t(sigma q . k_t) v_t over every cached token, query head
// h reading KV head h / g (section 04).  The quantized prefix is restored
// inside the kernel (k = code / kscale[segment, channel], v = code /
// vscale[token]; "KV Cache Quantization Strategies" Step 4 ``restore``); the
// high-precision tail is read as stored.
//
// Work decomposition (flash-decoding split, the former page, section 05):
// grid = (splits, batch * kv_heads).  The cached tokens form work items --
// 64-token quantized tiles, then 16-token tail chunks (about as many bytes
// each).  Split s owns a contiguous run of items and hands each of its four
// waves a contiguous sub-run (so a wave meets each Key segment once); every
// wave keeps one online-softmax state per query head (m, l, acc) in the log2
// domain.  The workgroup folds its waves into one partial; a second, small
// kernel merges the partials of each (batch, KV head).  With a single split
// the workgroup writes the output itself.  No device-scope fence is used: on
// gfx950 one costs a whole-L2 writeback and invalidate per workgroup.
//
// Scale folding: the per-channel Key scale of a segment is folded into the
// query once per segment (aq = sigma * log2(e) * q / kscale), the per-token
// Value scale into the softmax weight (p / vscale), so the inner products
// multiply integer codes by folded factors.
//
// Two kernels share this structure:
//   * decode_mfma_kernel (int4 codes, head_dim 64/128, whole-group segments,
//     bf16 tail):
//     both contractions of a tile run on v_mfma_f32_16x16x32_f16.  A nibble
//     field with its sign bit flipped (u = code + 8) becomes the fp16 value
//     X = 1 + u/16 by masking it into the mantissa of 1.0 (one shift and one
//     and-or per pair of fields); with the other operand a pre-scaled by 16,
//     sum a X = sum (a/16) code + 1.5 sum a, so the exact per-head term
//     1.5 sum a (summed from the same fp16 operands) is subtracted.  Query
//     heads are the MFMA M dimension (GQA <= 16).
//     The folded query is carried as two fp16 terms (hi + lo, about 22
//     significant bits): one fp16 term alone shifts the logits of outlier-
//     heavy Key channels by up to ~2e-3 of the output.
//   * decode_kernel (every other shape): the same tiles on the vector ALUs.
// Tail chunks (bf16 / fp32 values) run on the vector ALUs in both kernels.
// Hot-loop indexing is 32-bit; ring slots wrap with one subtraction.
#include "kvq_internal.h"

namespace kvq {

size_t workspace_bytes(const Geom& g, int q_heads, int tq);
size_t workspace_counter_bytes(const Geom& g, int tq);

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTailChunk = 16;

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

struct DecodeArgs {
  Geom g;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const void* k_tail;
  const void* v_tail;
  const int32_t* seg_index;
  int nq, nt;            // quantized / tail tokens
  int nq_slot;           // nq % ring: ring slot of the first tail token
  int tiles_per_seg;     // G / 64 (G > 0)
  const void* q;
  float qscale;          // sigma * log2(e)
  float* out;
  float* part;           // [unit][split][gqa][D + 2]
  int splits;
  int tiles_q, items;    // quantized tiles; work items = tiles_q + tail chunks
  uint32_t nib_mask;     // 0x03C003C0, see nibbles_to_h8
  uint32_t nib_one;      // 0x3C003C00
};

// Order LDS traffic between the lanes of one wave.  A wave's LDS operations
// complete in issue order, so only the compiler needs fencing; a wider fence
// would also wait for every outstanding global load of the wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---- shared pieces ---------------------------------------------------------------

// Fold one tile's maximum into the running maximum of a head; returns the
// factor by which every accumulator of that head is rescaled.
__device__ __forceinline__ float fold_max(float& m, float tile_max) {
  const float mn = fmaxf(m, tile_max);
  const float alpha = (mn == -INFINITY) ? 1.0f : fast_exp2(m - mn);
  m = mn;
  return alpha;
}

// Channels of the tail accumulator owned by a lane: c = lane * TCPL + k.
template <int D>
struct TailMap {
  static constexpr int TCPL = D >= kWave ? D / kWave : 1;
  __device__ static bool owns(int lane) { return lane * TCPL < D; }
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Ring slot of tail token tt (tt < nt <= ring, nq_slot < ring).
__device__ __forceinline__ int tail_slot(const DecodeArgs& a, int tt) {
  const int s = a.nq_slot + tt;
  return s >= a.g.ring ? s - a.g.ring : s;
}

// Tail chunk of 16 tokens (values stored as bf16/fp32 in the ring), on the
// vector ALUs.  Keys: lane = (token lane % 16, channel quarter lane / 16),
// partial dot products summed across the quarters.  Values: lane = channel
// owner (TailMap), sixteen tokens.  Key and Value loads are issued together
// and kept raw until use.  Updates m/l (uniform per head), returns alpha[]
// for the caller's other accumulators, accumulates into acc_tail.
// kBf16Only drops the fp32 branch (and its registers).
template <int D, int GQA, bool kBf16Only = false>
__device__ __forceinline__ void tail_chunk(const DecodeArgs& a, int unit, int chunk,
                                           const float (*qsT)[GQA], float (*pw)[GQA], float* m,
                                           float* l, float* alpha,
                                           float (&acc_tail)[TailMap<D>::TCPL][GQA]) {
  constexpr int CPQ = D / 4;               // channels per quarter
  constexpr int TCPL = TailMap<D>::TCPL;
  const Geom& g = a.g;
  const int lane = threadIdx.x % kWave;
  const int col = lane % 16, quarter = lane / 16;
  const int tt0 = chunk * kTailChunk;
  const int nvalid = a.nt - tt0 < kTailChunk ? a.nt - tt0 : kTailChunk;
  const bool bf16 = kBf16Only || g.dtype == KVQ_BF16;
  const int64_t ring_row0 = (int64_t)unit * g.ring;
  // ---- loads: Keys (CPQ channels of one token), Values (TCPL channels x 16 tokens)
  const int kslot = tail_slot(a, tt0 + (col < nvalid ? col : 0));
  const int64_t krow = (ring_row0 + kslot) * D + quarter * CPQ;
  uint32_t kraw[kBf16Only ? CPQ / 2 : CPQ];  // bf16: CPQ/2 words; fp32: CPQ words
  if (bf16) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.k_tail) + krow);
#pragma unroll
    for (int j = 0; j < CPQ / 2; ++j) kraw[j] = p[j];
  } else if constexpr (!kBf16Only) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.k_tail) + krow);
#pragma unroll
    for (int j = 0; j < CPQ; ++j) kraw[j] = p[j];
  }
  const bool owner = TailMap<D>::owns(lane);
  const int c0 = owner ? lane * TCPL : 0;
  uint32_t vraw[kTailChunk][TCPL];          // bf16: packed pair (TCPL = 2) or one value
#pragma unroll
  for (int t = 0; t < kTailChunk; ++t) {
    const int64_t base = (ring_row0 + tail_slot(a, tt0 + (t < nvalid ? t : 0))) * D + c0;
    if (bf16) {
      if constexpr (TCPL == 2) {
        vraw[t][0] = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.v_tail) + base);
      } else {
#pragma unroll
        for (int k = 0; k < TCPL; ++k) vraw[t][k] = static_cast<const uint16_t*>(a.v_tail)[base + k];
      }
    } else if constexpr (!kBf16Only) {
#pragma unroll
      for (int k = 0; k < TCPL; ++k)
        vraw[t][k] = reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.v_tail))[base + k];
    }
  }
  // ---- logits and softmax ----
  const bool valid = col < nvalid;
  wave_lds_sync();
#pragma unroll
  for (int h = 0; h < GQA; ++h) {
    float s = 0.0f;
    if (bf16) {
#pragma unroll
      for (int j = 0; j < CPQ / 2; ++j) {
        s = fmaf(qsT[quarter * CPQ + 2 * j][h], bf16_lo(kraw[j]), s);
        s = fmaf(qsT[quarter * CPQ + 2 * j + 1][h], bf16_hi(kraw[j]), s);
      }
    } else if constexpr (!kBf16Only) {
#pragma unroll
      for (int j = 0; j < CPQ; ++j) s = fmaf(qsT[quarter * CPQ + j][h], __uint_as_float(kraw[j]), s);
    }
    s += __shfl_xor(s, 16, kWave);
    s += __shfl_xor(s, 32, kWave);
    const float lg = valid ? s : -INFINITY;
    alpha[h] = fold_max(m[h], lane_value(row16_max(lg), 0));
    const float p = fast_exp2(lg - m[h]);          // exp2(-inf) = 0 for padding tokens
    l[h] = l[h] * alpha[h] + lane_value(row16_sum(p), 0);
    if (quarter == 0) pw[col][h] = p;
#pragma unroll
    for (int k = 0; k < TCPL; ++k) acc_tail[k][h] *= alpha[h];
  }
  wave_lds_sync();
  if (!owner) return;
#pragma unroll
  for (int t = 0; t < kTailChunk; ++t) {
    float v[TCPL];
    if (bf16) {
      if constexpr (TCPL == 2) {
        v[0] = bf16_lo(vraw[t][0]);
        v[1] = bf16_hi(vraw[t][0]);
      } else {
#pragma unroll
        for (int k = 0; k < TCPL; ++k) v[k] = bf16_lo(vraw[t][k]);
      }
    } else if constexpr (!kBf16Only) {
#pragma unroll
      for (int k = 0; k < TCPL; ++k) v[k] = __uint_as_float(vraw[t][k]);
    }
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      const float p = pw[t][h];
#pragma unroll
      for (int k = 0; k < TCPL; ++k) acc_tail[k][h] = fmaf(p, v[k], acc_tail[k][h]);
    }
  }
}

// Fold the four waves of a workgroup and write a partial (or the output).
// red[w][c][h] holds wave w's accumulator relative to its own maximum.
template <int D, int GQA>
__device__ __forceinline__ void fold_and_store(const DecodeArgs& a, int unit, int split,
                                               float (*red)[D][GQA], float (*wml)[2][GQA],
                                               const float* m, const float* l) {
  const Geom& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int b = unit / g.H, kvh = unit % g.H;
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      wml[wave][0][h] = m[h];
      wml[wave][1][h] = l[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < GQA * D; i += kThreads) {
    const int h = i / D, c = i % D;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wml[w][0][h]);
    float s = 0.0f, L = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      const float e = (wml[w][0][h] == -INFINITY) ? 0.0f : fast_exp2(wml[w][0][h] - M);
      s += red[w][c][h] * e;
      L += wml[w][1][h] * e;
    }
    if (a.splits == 1) {
      a.out[((int64_t)b * g.H * GQA + kvh * GQA + h) * D + c] = s / L;
    } else {
      float* part = a.part + ((int64_t)unit * a.splits + split) * GQA * (D + 2) + h * (D + 2);
      part[c] = s;
      if (c == 0) {
        part[D] = M;
        part[D + 1] = L;
      }
    }
  }
}

template <int D, int GQA>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int unit, float (*qsT)[GQA]) {
  const Geom& g = a.g;
  const int b = unit / g.H, kvh = unit % g.H;
  for (int i = threadIdx.x; i < GQA * D; i += kThreads) {
    const int h = i / D, c = i % D;
    qsT[c][h] = load_elem(a.q, ((int64_t)b * g.H * GQA + kvh * GQA + h) * D + c, g.dtype) * a.qscale;
  }
}

// The contiguous run of work items [begin, end) of this wave.
__device__ __forceinline__ void wave_items(const DecodeArgs& a, int split, int wave, int& begin, int& end) {
  const int s0 = (int)(((int64_t)a.items * split) / a.splits);
  const int s1 = (int)(((int64_t)a.items * (split + 1)) / a.splits);
  begin = s0 + ((s1 - s0) * wave) / kWaves;
  end = s0 + ((s1 - s0) * (wave + 1)) / kWaves;
}

// ---- vector-ALU kernel (every shape) ------------------------------------------------

template <int D, int BITS, int GQA>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  constexpr int W = D * BITS / 8;        // bytes per token row
  constexpr int NSLOT = W / 16;          // 16-byte units per lane per tile
  constexpr int TPU = 128 / BITS;        // tokens per Value unit
  constexpr int FPW = 32 / BITS;         // fields per 32-bit word
  constexpr int TCPL = TailMap<D>::TCPL;
  const Geom& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int unit = blockIdx.y;
  const int split = blockIdx.x;

  __shared__ float qsT[D][GQA];
  __shared__ float aq[kWaves][D][GQA];
  __shared__ float pw[kWaves][kTile][GQA];
  __shared__ float red[kWaves][D][GQA];
  __shared__ float wml[kWaves][2][GQA];

  load_q<D, GQA>(a, unit, qsT);
  __syncthreads();

  float m[GQA], l[GQA], alpha[GQA], acc[NSLOT][GQA], acc_tail[TCPL][GQA];
#pragma unroll
  for (int h = 0; h < GQA; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) acc[k][h] = 0.0f;
#pragma unroll
    for (int k = 0; k < TCPL; ++k) acc_tail[k][h] = 0.0f;
  }

  int w_begin, w_end;
  wave_items(a, split, wave, w_begin, w_end);
  const uint8_t* kbase = a.k_codes + (int64_t)unit * g.code_stream;
  const uint8_t* vbase = a.v_codes + (int64_t)unit * g.code_stream;
  const uint16_t* ksbase = a.k_scale + (int64_t)unit * g.max_seg * D;
  const uint16_t* vsbase = a.v_scale + (int64_t)unit * g.C;
  int cur_seg = -1;

  for (int tile = w_begin; tile < w_end; ++tile) {
    if (tile >= a.tiles_q) {
      tail_chunk<D, GQA>(a, unit, tile - a.tiles_q, qsT, pw[wave], m, l, alpha, acc_tail);
#pragma unroll
      for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) acc[k][h] *= alpha[h];
      continue;
    }
    const int t = tile * kTile + lane;
    const bool valid = t < a.nq;
    const uint8_t* kt = kbase + (int64_t)tile * (kTile * W);
    const uint8_t* vt = vbase + (int64_t)tile * (kTile * W);
    // Issue every load of the tile before any arithmetic.
    uint4 kc[NSLOT], vc[NSLOT];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) kc[j] = *reinterpret_cast<const uint4*>(kt + j * 1024 + lane * 16);
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) vc[k] = *reinterpret_cast<const uint4*>(vt + (k * kWave + lane) * 16);
    const float vs = valid ? half_bits_to_f32(vsbase[t]) : 1.0f;
    float logit[GQA];
#pragma unroll
    for (int h = 0; h < GQA; ++h) logit[h] = 0.0f;

    if (g.G > 0) {
      const int seg = tile / a.tiles_per_seg;
      if (seg != cur_seg) {
        cur_seg = seg;
        const uint16_t* ks = ksbase + seg * D;
        wave_lds_sync();
        for (int c = lane; c < D; c += kWave) {
          const float r = fast_rcp(fmaxf(half_bits_to_f32(ks[c]), g.eps));
#pragma unroll
          for (int h = 0; h < GQA; ++h) aq[wave][c][h] = qsT[c][h] * r;
        }
        wave_lds_sync();
      }
#pragma unroll
      for (int j = 0; j < NSLOT; ++j) {
        const uint32_t wd[4] = {kc[j].x, kc[j].y, kc[j].z, kc[j].w};
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
      const int seg = a.seg_index[t];
      const uint16_t* ks = ksbase + seg * D;
#pragma unroll
      for (int j = 0; j < NSLOT; ++j) {
        const uint32_t wd[4] = {kc[j].x, kc[j].y, kc[j].z, kc[j].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
          for (int f = 0; f < FPW; ++f) {
            const int c = (j * 16 + w * 4) * (8 / BITS) + f;
            const float kh = static_cast<float>(sext_field<BITS>(wd[w], f * BITS)) *
                             fast_rcp(fmaxf(half_bits_to_f32(ks[c]), g.eps));
#pragma unroll
            for (int h = 0; h < GQA; ++h) logit[h] = fmaf(qsT[c][h], kh, logit[h]);
          }
        }
      }
    }

    const float vinv = fast_rcp(fmaxf(vs, g.eps));
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      const float x = valid ? logit[h] : -INFINITY;
      alpha[h] = fold_max(m[h], wave_max(x));
      const float p = valid ? fast_exp2(x - m[h]) : 0.0f;
      l[h] = l[h] * alpha[h] + wave_sum(p);
#pragma unroll
      for (int k = 0; k < NSLOT; ++k) acc[k][h] *= alpha[h];
#pragma unroll
      for (int k = 0; k < TCPL; ++k) acc_tail[k][h] *= alpha[h];
      pw[wave][lane][h] = p * vinv;
    }
    wave_lds_sync();

    // Values: lane owns NSLOT (channel, token-run) units of the tile; the
    // token run starts at t0, the same for every slot of the lane.
    const int t0 = ((lane * 16) % (8 * BITS)) * 8 / BITS;
#pragma unroll
    for (int f = 0; f < TPU; ++f) {
      float pf[GQA];
#pragma unroll
      for (int h = 0; h < GQA; ++h) pf[h] = pw[wave][t0 + f][h];
#pragma unroll
      for (int k = 0; k < NSLOT; ++k) {
        const uint32_t wd[4] = {vc[k].x, vc[k].y, vc[k].z, vc[k].w};
        const float code = static_cast<float>(sext_field<BITS>(wd[f / FPW], (f % FPW) * BITS));
#pragma unroll
        for (int h = 0; h < GQA; ++h) acc[k][h] = fmaf(pf[h], code, acc[k][h]);
      }
    }
  }

  // Lanes that share a channel hold different token runs of it: sum them.
#pragma unroll
  for (int k = 0; k < NSLOT; ++k) {
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      float v = acc[k][h];
      if (BITS == 8) {
        v += dpp_f<kDppQuadXor1>(v);
        v += dpp_f<kDppQuadXor2>(v);
      } else if (BITS == 4) {
        v += dpp_f<kDppQuadXor1>(v);
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
  wave_lds_sync();
  if (TailMap<D>::owns(lane)) {
#pragma unroll
    for (int k = 0; k < TCPL; ++k)
#pragma unroll
      for (int h = 0; h < GQA; ++h) red[wave][lane * TCPL + k][h] += acc_tail[k][h];
  }
  fold_and_store<D, GQA>(a, unit, split, red, wml, m, l);
}

// ---- MFMA kernel (int4 codes, head_dim 64 / 128, whole-group segments) ---------------

// One 32-bit word of eight int4 fields -> eight fp16 values 1 + (code + 8) / 16
// in MFMA slot order: slot 2v holds field v, slot 2v+1 holds field v + 4.
// mask = 0x03C003C0 (mantissa bits 6..9 of both halves) and one = 0x3C003C00
// (two fp16 ones) arrive as kernel arguments: kept in registers, each pair of
// fields costs a shift and one v_and_or_b32 (literal operands would force a
// separate and + or).
__device__ __forceinline__ h8_t nibbles_to_h8(uint32_t w, uint32_t mask, uint32_t one) {
  const uint32_t x = w ^ 0x88888888u;          // u = code + 8 in every field
  u4_t r;
  r[0] = ((x << 6) & mask) | one;              // 1 + u / 16, fields 0 and 4
  r[1] = ((x << 2) & mask) | one;
  r[2] = ((x >> 2) & mask) | one;
  r[3] = ((x >> 6) & mask) | one;
  return __builtin_bit_cast(h8_t, r);
}

// Element (0..7) of a word held in MFMA slot r, and its inverse.
__device__ __forceinline__ constexpr int slot_elem(int r) { return (r % 2) * 4 + r / 2; }
__device__ __forceinline__ constexpr int elem_slot(int e) { return 2 * (e % 4) + e / 4; }

// Head held in MFMA result row 4q + i.  Rows >= GQA are padding; they are
// mapped onto a real head so every value they carry stays finite.
template <int GQA>
__device__ __forceinline__ int row_head(int q, int i) {
  return GQA > 4 ? (4 * (q & 1) + i) % GQA : i % GQA;
}

template <int D, int GQA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_kernel(DecodeArgs a) {
  constexpr int BITS = 4;
  constexpr int W = D * BITS / 8;         // bytes per token row
  constexpr int MK = D / 32;              // Key MFMAs per 16 tokens (32 channels each)
  constexpr int NV = D / 16;              // Value MFMA column blocks (16 channels each)
  constexpr int TCPL = TailMap<D>::TCPL;
  static_assert(GQA <= 16, "query rows must fit the MFMA M dimension");
  const Geom& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int q4 = lane / 16, col = lane % 16;
  const int unit = blockIdx.y;
  const int split = blockIdx.x;

  __shared__ float qsT[D][GQA];
  __shared__ __attribute__((aligned(16))) _Float16 pV[kWaves][16][8][8];  // [row][token block][slot]
  __shared__ h8_t aKs[kWaves][2 * MK][kWave];     // folded-query operands, [hi/lo x mk][lane]
  __shared__ float pw[kWaves][kTile][GQA];
  __shared__ float red[kWaves][D][GQA];
  __shared__ float wml[kWaves][2][GQA];

  load_q<D, GQA>(a, unit, qsT);
  for (int i = tid; i < kWaves * 16 * 8 * 8; i += kThreads) (&pV[0][0][0][0])[i] = (_Float16)0.0f;
  __syncthreads();

  float m[GQA], l[GQA], alpha[GQA], acc_tail[TCPL][GQA];
#pragma unroll
  for (int h = 0; h < GQA; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < TCPL; ++k) acc_tail[k][h] = 0.0f;
  }
  f4_t acc[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) acc[n] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  int w_begin, w_end;
  wave_items(a, split, wave, w_begin, w_end);
  const uint8_t* kbase = a.k_codes + (int64_t)unit * g.code_stream;
  const uint8_t* vbase = a.v_codes + (int64_t)unit * g.code_stream;
  const uint16_t* ksbase = a.k_scale + (int64_t)unit * g.max_seg * D;
  const uint16_t* vsbase = a.v_scale + (int64_t)unit * g.C;
  // Per-lane byte offsets inside a tile (the tile base is wave-uniform).
  const int lk = col * 16 + 4 * q4;               // Key word: token 16 grp + col, channels 8 q4..
  const int lv = col * (8 * BITS) + 8 * q4;       // Value words: channel 16 n + col, blocks 2 q4, 2 q4 + 1
  const int pv_slot = (col / 8) * 8 + elem_slot(col % 8);   // this lane's token in pV[row][.][.]
  const int hq = col < GQA ? col : 0;
  const float row_mask = col < GQA ? 16.0f : 0.0f;   // 16x pre-scale; padding rows are zero
  uint32_t nib_mask = a.nib_mask;
  const uint32_t nib_one = a.nib_one;
  // Keep the mask in a vector register (an empty statement, no instruction):
  // v_and_or_b32 may read only one scalar operand.
  asm("" : "+v"(nib_mask));
  float corrK[4];         // 1.5 * sum of the Key operand over channels, result rows 4 q4 + i
  float corrV[GQA];       // 1.5 * sum of the Value weights (running, rescaled like acc)
#pragma unroll
  for (int h = 0; h < GQA; ++h) corrV[h] = 0.0f;
  h8_t* aK = &aKs[wave][0][lane];              // [hi/lo][mk] operands of this lane, stride 64

  // Code words of one tile, as this lane needs them.
  struct TileRegs {
    uint32_t kw[4][MK];   // [token group][channel block]: 8 channels of token 16 grp + col
    uint2 vw[NV];         // channel 16 n + col, token blocks 2 q4 and 2 q4 + 1
    float vs[4];          // Value scales of tokens 16 grp + col
    bool new_seg;         // the tile opens a Key segment: ksn holds its scales
  };
  uint4 ksn[MK];          // Key scales of channels 32 mk + 8 q4 .. +7 of the next segment
  auto load_tile = [&](int tile, TileRegs& r) {
    r.new_seg = tile == w_begin || tile % a.tiles_per_seg == 0;
    if (r.new_seg) {      // first, so that waiting for it leaves the code words in flight
      const uint16_t* ks = ksbase + (tile / a.tiles_per_seg) * D;
#pragma unroll
      for (int mk = 0; mk < MK; ++mk) ksn[mk] = *reinterpret_cast<const uint4*>(ks + 32 * mk + 8 * q4);
    }
    const uint8_t* kt = kbase + (int64_t)tile * (kTile * W);
    const uint8_t* vt = vbase + (int64_t)tile * (kTile * W);
    const uint16_t* vst = vsbase + tile * kTile;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp)
#pragma unroll
      for (int mk = 0; mk < MK; ++mk)
        r.kw[grp][mk] = *reinterpret_cast<const uint32_t*>(kt + lk + grp * 256 + mk * 1024);
#pragma unroll
    for (int n = 0; n < NV; ++n) r.vw[n] = *reinterpret_cast<const uint2*>(vt + lv + n * 16 * (8 * BITS));
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) r.vs[grp] = half_bits_to_f32(vst[16 * grp + col]);
  };

  // Key operands of a segment: 16 * sigma*log2e * q / kscale as hi + lo fp16,
  // written to this wave's LDS slab (MFMA slot order).
  auto build_key_operands = [&]() {
    float rowsum = 0.0f;
#pragma unroll
    for (int mk = 0; mk < MK; ++mk) {
      const uint32_t kh[4] = {ksn[mk].x, ksn[mk].y, ksn[mk].z, ksn[mk].w};
      h8_t hi8, lo8;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int e = slot_elem(rr);
        const uint16_t bits = static_cast<uint16_t>(kh[e / 2] >> (16 * (e % 2)));
        const float rk = fast_rcp(fmaxf(half_bits_to_f32(bits), g.eps));
        const float v = row_mask * qsT[32 * mk + 8 * q4 + e][hq] * rk;
        const _Float16 hi = (_Float16)v;
        const _Float16 lo = (_Float16)(v - (float)hi);
        hi8[rr] = hi;
        lo8[rr] = lo;
        rowsum += (float)hi + (float)lo;
      }
      aK[(0 * MK + mk) * kWave] = hi8;
      aK[(1 * MK + mk) * kWave] = lo8;
    }
    // Row col's sum over all channels: its four channel quarters sit in lanes col + 16 q.
    rowsum += __shfl_xor(rowsum, 16, kWave);
    rowsum += __shfl_xor(rowsum, 32, kWave);
#pragma unroll
    for (int i = 0; i < 4; ++i) corrK[i] = 1.5f * __shfl(rowsum, 4 * q4 + i, kWave);
  };

  auto compute_tile = [&](const TileRegs& r) {
    float vsr[4];         // 16 / max(vscale, eps)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) vsr[grp] = 16.0f * fast_rcp(fmaxf(r.vs[grp], g.eps));

    // ---- logits: S[head][token] = aK . (code / 16) ----
    f4_t S[4];
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) S[grp] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int mk = 0; mk < MK; ++mk) {
      const h8_t ah = aK[(0 * MK + mk) * kWave];
      const h8_t al = aK[(1 * MK + mk) * kWave];
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const h8_t kb = nibbles_to_h8(r.kw[grp][mk], nib_mask, nib_one);
        S[grp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, kb, S[grp], 0, 0, 0);
        S[grp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, kb, S[grp], 0, 0, 0);
      }
    }
#pragma unroll
    for (int grp = 0; grp < 4; ++grp)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[grp][i] -= corrK[i];

    // ---- online softmax (rows 4 q4 + i of this lane; tokens 16 grp + col) ----
    float rmax[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rmax[i] = row16_max(fmaxf(fmaxf(S[0][i], S[1][i]), fmaxf(S[2][i], S[3][i])));
#pragma unroll
    for (int h = 0; h < GQA; ++h) alpha[h] = fold_max(m[h], lane_value(rmax[h % 4], 16 * (h / 4)));
    bool moved = false;   // did any head's running maximum change?
#pragma unroll
    for (int h = 0; h < GQA; ++h) moved |= alpha[h] != 1.0f;
    float rsum[4], rcs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = row_head<GQA>(q4, i);
      const float mrow = m[hh];
      float ps = 0.0f, cs = 0.0f;
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const float p = fast_exp2(S[grp][i] - mrow);
        ps += p;
        const _Float16 ap = (_Float16)(p * vsr[grp]);
        cs += (float)ap;
        if (4 * q4 + i < GQA) (&pV[wave][4 * q4 + i][0][0])[grp * 16 + pv_slot] = ap;
      }
      rsum[i] = row16_sum(ps);
      rcs[i] = row16_sum(cs);
    }
    if (moved) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float al = alpha[row_head<GQA>(q4, i)];
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[n][i] *= al;
      }
#pragma unroll
      for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int k = 0; k < TCPL; ++k) acc_tail[k][h] *= alpha[h];
    }
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      l[h] = l[h] * alpha[h] + lane_value(rsum[h % 4], 16 * (h / 4));
      corrV[h] = corrV[h] * alpha[h] + 1.5f * lane_value(rcs[h % 4], 16 * (h / 4));
    }
    wave_lds_sync();

    // ---- values: acc[head][channel] += (16 p / vscale) . (1 + (code + 8) / 16) ----
    const h8_t A0 = *reinterpret_cast<const h8_t*>(&pV[wave][col][2 * q4][0]);
    const h8_t A1 = *reinterpret_cast<const h8_t*>(&pV[wave][col][2 * q4 + 1][0]);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, nibbles_to_h8(r.vw[n].x, nib_mask, nib_one), acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, nibbles_to_h8(r.vw[n].y, nib_mask, nib_one), acc[n], 0, 0, 0);
    }
    wave_lds_sync();      // pV is rewritten by the next tile
  };

  // Quantized tiles, double-buffered: the next tile's loads are in flight
  // while the current one is computed.
  const int q_end = w_end < a.tiles_q ? w_end : a.tiles_q;
  int tile = w_begin;
  TileRegs bufA, bufB;
  if (tile < q_end) load_tile(tile, bufA);
  while (tile < q_end) {
    if (bufA.new_seg) {
      build_key_operands();
      wave_lds_sync();
    }
    if (tile + 1 < q_end) load_tile(tile + 1, bufB);
    compute_tile(bufA);
    if (++tile >= q_end) break;
    if (bufB.new_seg) {
      build_key_operands();
      wave_lds_sync();
    }
    if (tile + 1 < q_end) load_tile(tile + 1, bufA);
    compute_tile(bufB);
    ++tile;
  }
  // Tail chunks (bf16), after the quantized tiles of this wave.
  for (tile = tile > w_begin ? tile : w_begin; tile < w_end; ++tile) {
    if (tile < a.tiles_q) continue;
    tail_chunk<D, GQA, true>(a, unit, tile - a.tiles_q, qsT, pw[wave], m, l, alpha, acc_tail);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float al = alpha[row_head<GQA>(q4, i)];
#pragma unroll
      for (int n = 0; n < NV; ++n) acc[n][i] *= al;
    }
#pragma unroll
    for (int h = 0; h < GQA; ++h) corrV[h] *= alpha[h];
  }

  // ---- wave result into red[wave][channel][head] ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q4 + i;
    if (h < GQA) {
#pragma unroll
      for (int n = 0; n < NV; ++n) red[wave][16 * n + col][h] = acc[n][i] - corrV[h];
    }
  }
  wave_lds_sync();
  if (TailMap<D>::owns(lane)) {
#pragma unroll
    for (int k = 0; k < TCPL; ++k)
#pragma unroll
      for (int h = 0; h < GQA; ++h) red[wave][lane * TCPL + k][h] += acc_tail[k][h];
  }
  fold_and_store<D, GQA>(a, unit, split, red, wml, m, l);
}

// One workgroup per (batch, KV head): combine the splits' (m, l, acc).
template <int D, int GQA>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeArgs a) {
  const int unit = blockIdx.x;
  const int b = unit / a.g.H, kvh = unit % a.g.H;
  const float* pu = a.part + (int64_t)unit * a.splits * GQA * (D + 2);
  for (int i = threadIdx.x; i < GQA * D; i += kThreads) {
    const int h = i / D, c = i % D;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, pu[(s * GQA + h) * (D + 2) + D]);
    float num = 0.0f, den = 0.0f;
#pragma unroll 8
    for (int s = 0; s < a.splits; ++s) {
      const float* ps = pu + (s * GQA + h) * (D + 2);
      const float ms = ps[D];
      const float e = (ms == -INFINITY) ? 0.0f : fast_exp2(ms - mx);
      num = fmaf(ps[c], e, num);
      den = fmaf(ps[D + 1], e, den);
    }
    a.out[((int64_t)b * a.g.H * GQA + kvh * GQA + h) * D + c] = num / den;
  }
}

template <int D, int BITS, int GQA>
void launch(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.splits, a.g.B * a.g.H);
  if constexpr (BITS == 4 && D >= 64) {
    if (a.g.G > 0 && a.g.dtype == KVQ_BF16)
      hipLaunchKernelGGL((decode_mfma_kernel<D, GQA>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<D, BITS, GQA>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, BITS, GQA>), grid, dim3(kThreads), 0, s, a);
  }
  if (a.splits > 1)
    hipLaunchKernelGGL((merge_kernel<D, GQA>), dim3(a.g.B * a.g.H), dim3(kThreads), 0, s, a);
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

int auto_splits(int units, int items) {
  // Aim for about two workgroups per compute unit (256 CUs), at least four
  // work items per workgroup, and never more splits than that allows.
  int s = (2 * 256 + units - 1) / units;
  const int max_by_items = items / 4 > 0 ? items / 4 : 1;
  if (s > max_by_items) s = max_by_items;
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
  a.nq = static_cast<int>(st->quantized);
  a.nt = static_cast<int>(st->tail);
  a.nq_slot = static_cast<int>(st->quantized % g.ring);
  a.tiles_per_seg = g.G > 0 ? g.G / kTile : 0;
  a.q = q;
  a.qscale = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + workspace_counter_bytes(g, 1));
  a.nib_mask = 0x03C003C0u;
  a.nib_one = 0x3C003C00u;
  a.tiles_q = (a.nq + kTile - 1) / kTile;
  a.items = a.tiles_q + (a.nt + kTailChunk - 1) / kTailChunk;
  const int units = g.B * g.H;
  a.splits = num_splits > 0 ? num_splits : auto_splits(units, a.items);
  if (!dispatch(a, gqa, static_cast<hipStream_t>(stream))) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}
