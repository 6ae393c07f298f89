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
// domain.  The workgroup folds its waves into one partial; the last
// workgroup of each (batch, KV head) to finish merges the partials (see
// finish_unit; with up to eight splits and at most one appended token its
// wave 0 does the fold, the publication and the merge alone, see
// merge_in_wave), or, above 64 splits, a second, small kernel does.  With a
// single split the workgroup writes the output itself.  No device-scope
// fence is used: on gfx950 one costs a whole-L2 writeback and invalidate
// per workgroup.
//
// Same-axis caches (Keys and Values per token, one scale per run of 64
// channels) run on decode_kernel<..., kSameAxis = true>.
//
// Scale folding: the per-channel Key scale of a segment is folded into the
// query once per segment (aq = sigma * log2(e) * q / kscale), the per-token
// Value scale into the softmax weight (p / vscale), so the inner products
// multiply integer codes by folded factors.
//
// Two kernels share this structure:
//   * decode_i8_kernel (int4 / int2 codes, head_dim 64 / 128, whole-group
//     segments, bf16 window): both contractions of a quantized tile run on
//     the integer matrix cores (v_mfma_i32_16x16x64_i8, see the comment
//     above that kernel); window chunks score on v_mfma_f32_16x16x32_bf16.
//   * decode_kernel (every other shape, same-axis caches, or the vector-ALU
//     kernel chosen in the configuration): the same work items on the vector
//     ALUs.
// Hot-loop indexing is 32-bit; ring slots wrap with one subtraction.
#include <mutex>

#include "kvq_internal.h"

namespace kvq {

size_t workspace_bytes(const Geom& g, int q_heads, int tq);
size_t workspace_counter_bytes(const Geom& g, int tq);

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTailChunk = 16;
// Buffer resources: word 3 of a raw (untyped, stride 0) buffer.
constexpr int kRsrcWord3 = 0x00020000;


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
  float* part;           // [unit][split][gqa][D + 4]: acc[D], m, l, 2 pad (16-byte rows)
  int splits;
  int tiles_q, items;    // quantized tiles; work items = tiles_q + tail chunks
  int tq_div, tq_mod;    // tiles_q = splits * tq_div + tq_mod
  int ch_div, ch_mod;    // tail chunks, likewise
  uint32_t* ctr;         // per-unit arrival counters (workspace), 0 between calls
  int last_merge;        // 1: the last workgroup of a unit to arrive merges its splits;
                         // 0: partials are written for merge_kernel (more than kLastMergeSplits splits)
  // Tokens appended by the same call (kvq_decode_step), folded in by the
  // merge: keys and values [unit][n_new][D] (bf16), and the window slot of
  // the first one; the merge of query head 0 copies them into the window.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* ring_k;
  uint16_t* ring_v;
  int n_new, new_slot0;
};

constexpr int kMaxStepNew = 16;
constexpr int kWaveMergeSplits = 8;    // split counts whose merge wave 0 does alone   // appended tokens kvq_decode_step folds into the merge
constexpr int kLastMergeSplits = 64;  // split counts merged inside the attention kernel
constexpr int kMergeBatch = 16;   // partial loads in flight per output element in that merge
constexpr int kMaxPagedSeqs = 64;

// Paged caches: per-sequence lengths and the page of each tile.  A page
// holds, per KV head: Key codes (64 W bytes), Value codes (64 W), Value
// scales (64 fp16), the segment's Key-scale row (D fp16).
struct PagedDecode {
  const uint8_t* pool;
  const int32_t* table;     // [batch, stride]
  int64_t n_pages;
  int64_t page_bytes;
  int head_bytes;
  int stride;
  int per_split;            // work items per split: a sequence takes ceil(items / per_split) splits
  int nq[kMaxPagedSeqs];
  int nt[kMaxPagedSeqs];
  int wg_end[kMaxPagedSeqs];  // workgroups of sequences 0..b (H times each one's split count)
  int n_new[kMaxPagedSeqs];   // decode step: tokens appended to sequence b (rows of k_new / v_new)
  int new_slot0[kMaxPagedSeqs];  // ... and the window slot of its first one
};
struct NoPaging {};         // uniform caches: no page table

// Paged caches launch only workgroups with work, on a 1-D grid: sequence b
// owns ids [wg_end[b - 1], wg_end[b]), H units of ws splits each, consecutive
// ids on consecutive splits of one unit (so every XCD gets its share of
// every unit).
struct PagedUnit {
  int unit, split, ws;
};
__device__ __forceinline__ PagedUnit paged_unit(const PagedDecode& pd, int H, int batch, int id) {
  int b = 0;
  while (b < batch - 1 && id >= pd.wg_end[b]) ++b;
  const int start = b > 0 ? pd.wg_end[b - 1] : 0;
  PagedUnit u;
  u.ws = (pd.wg_end[b] - start) / H;
  const int local = id - start;
  u.unit = b * H + local / u.ws;
  u.split = local % u.ws;
  return u;
}

// A paged sequence's lengths and its division of work into ws splits.  The
// partials keep the layout of the largest split count (a.splits).
__device__ __forceinline__ DecodeArgs paged_args(const DecodeArgs& a0, const PagedDecode& pd, int unit, int ws) {
  DecodeArgs pa = a0;
  const int b = unit / a0.g.H;
  pa.nq = pd.nq[b];
  pa.nt = pd.nt[b];
  pa.nq_slot = pa.nq % a0.g.ring;
  pa.tiles_q = (pa.nq + kTile - 1) / kTile;
  pa.items = pa.tiles_q + (pa.nt + kTailChunk - 1) / kTailChunk;
  pa.tq_div = pa.tiles_q / ws;
  pa.tq_mod = pa.tiles_q % ws;
  pa.ch_div = (pa.items - pa.tiles_q) / ws;
  pa.ch_mod = (pa.items - pa.tiles_q) % ws;
  return pa;
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
// owner (TailMap), sixteen tokens.  tail_load issues every load of a chunk
// (kept raw in registers); tail_compute updates m/l (uniform per head),
// returns alpha[] for the caller's other accumulators and accumulates into
// acc_tail.  kBf16Only drops the fp32 branch (and its registers).
template <int D, bool kBf16Only>
struct TailRegs {
  static constexpr int CPQ = D / 4;        // channels per quarter
  uint32_t kraw[kBf16Only ? CPQ / 2 : CPQ];  // bf16: CPQ/2 words; fp32: CPQ words
  uint32_t vraw[kTailChunk][TailMap<D>::TCPL];
  int nvalid;
};

template <int D, bool kBf16Only>
__device__ __forceinline__ void tail_load(const DecodeArgs& a, int unit, int chunk, TailRegs<D, kBf16Only>& r) {
  constexpr int CPQ = D / 4;
  constexpr int TCPL = TailMap<D>::TCPL;
  const Geom& g = a.g;
  const int lane = threadIdx.x % kWave;
  const int col = lane % 16, quarter = lane / 16;
  const int tt0 = chunk * kTailChunk;
  r.nvalid = a.nt - tt0 < kTailChunk ? a.nt - tt0 : kTailChunk;
  const bool bf16 = kBf16Only || g.dtype == KVQ_BF16;
  const int64_t ring_row0 = (int64_t)unit * g.ring;
  const int kslot = tail_slot(a, tt0 + (col < r.nvalid ? col : 0));
  const int64_t krow = (ring_row0 + kslot) * D + quarter * CPQ;
  if (bf16) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.k_tail) + krow);
#pragma unroll
    for (int j = 0; j < CPQ / 2; ++j) r.kraw[j] = p[j];
    if constexpr (!kBf16Only) {     // every element defined on both paths: the array stays in registers
#pragma unroll
      for (int j = CPQ / 2; j < CPQ; ++j) r.kraw[j] = 0u;
    }
  } else if constexpr (!kBf16Only) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.k_tail) + krow);
#pragma unroll
    for (int j = 0; j < CPQ; ++j) r.kraw[j] = p[j];
  }
  const int c0 = TailMap<D>::owns(lane) ? lane * TCPL : 0;
#pragma unroll
  for (int t = 0; t < kTailChunk; ++t) {
    const int64_t base = (ring_row0 + tail_slot(a, tt0 + (t < r.nvalid ? t : 0))) * D + c0;
    if (bf16) {
      if constexpr (TCPL == 2) {   // one word holds the lane's two bf16 channels
        r.vraw[t][0] = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.v_tail) + base);
        r.vraw[t][1] = 0u;
      } else {
#pragma unroll
        for (int k = 0; k < TCPL; ++k) r.vraw[t][k] = static_cast<const uint16_t*>(a.v_tail)[base + k];
      }
    } else if constexpr (!kBf16Only) {
#pragma unroll
      for (int k = 0; k < TCPL; ++k)
        r.vraw[t][k] = reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.v_tail))[base + k];
    }
  }
}

template <int D, int GQA, bool kBf16Only>
__device__ __forceinline__ void tail_compute(const DecodeArgs& a, const TailRegs<D, kBf16Only>& r,
                                             const float (*qsT)[GQA], float (*pw)[GQA], float* m,
                                             float* l, float* alpha,
                                             float (&acc_tail)[TailMap<D>::TCPL][GQA]) {
  constexpr int CPQ = D / 4;
  constexpr int TCPL = TailMap<D>::TCPL;
  const int lane = threadIdx.x % kWave;
  const int col = lane % 16, quarter = lane / 16;
  const bool bf16 = kBf16Only || a.g.dtype == KVQ_BF16;
  const bool valid = col < r.nvalid;
  wave_lds_sync();
#pragma unroll
  for (int h = 0; h < GQA; ++h) {
    float s = 0.0f;
    if (bf16) {
#pragma unroll
      for (int j = 0; j < CPQ / 2; ++j) {
        s = fmaf(qsT[quarter * CPQ + 2 * j][h], bf16_lo(r.kraw[j]), s);
        s = fmaf(qsT[quarter * CPQ + 2 * j + 1][h], bf16_hi(r.kraw[j]), s);
      }
    } else if constexpr (!kBf16Only) {
#pragma unroll
      for (int j = 0; j < CPQ; ++j) s = fmaf(qsT[quarter * CPQ + j][h], __uint_as_float(r.kraw[j]), s);
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
  if (!TailMap<D>::owns(lane)) return;
#pragma unroll
  for (int t = 0; t < kTailChunk; ++t) {
    float v[TCPL];
    if (bf16) {
      if constexpr (TCPL == 2) {
        v[0] = bf16_lo(r.vraw[t][0]);
        v[1] = bf16_hi(r.vraw[t][0]);
      } else {
#pragma unroll
        for (int k = 0; k < TCPL; ++k) v[k] = bf16_lo(r.vraw[t][k]);
      }
    } else if constexpr (!kBf16Only) {
#pragma unroll
      for (int k = 0; k < TCPL; ++k) v[k] = __uint_as_float(r.vraw[t][k]);
    }
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      const float p = pw[t][h];
#pragma unroll
      for (int k = 0; k < TCPL; ++k) acc_tail[k][h] = fmaf(p, v[k], acc_tail[k][h]);
    }
  }
}

// Merge of the split partials (m, l, acc) of one (batch, KV head, query
// head): one workgroup, thread c owns output channel c.  Every thread issues
// its splits' acc[c] loads (up to 32 in flight) together with the split
// maxima and sums, so up to 32 splits cost one memory round trip; the
// per-split weights exp2(m_s - M) are computed once into LDS.  kBatch is 8
// when the splits fit in it (no duplicate loads), 32 otherwise.
// kNew: the call also appended n_new tokens that the partials do not cover.
// Each is one more term of the softmax: its logit q . k (log2 domain) is a
// workgroup reduction, its value row is read directly, and the workgroup of
// query head 0 copies the keys and values into their window slots.
template <int D, int GQA, int kBatch, bool kNew, typename PD = NoPaging>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a, PD pd) {
  constexpr int W = D < kWave ? D : kWave;           // lanes of one reduction
  constexpr int NW = D / W;
  const int unit = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  const Geom& g = a.g;
  const int b = unit / g.H, kvh = unit % g.H;
  const int stride = GQA * (D + 4);                  // floats between splits
  const float* pu = a.part + (int64_t)unit * a.splits * stride + h * (D + 4);
  int S = a.splits;                                  // paged: the sequence's own split count
  int nn = a.n_new;                                  // appended tokens folded in (paged: this sequence's)
  int slot0 = a.new_slot0;
  if constexpr (!__is_same(PD, NoPaging)) {
    S = (pd.wg_end[b] - (b > 0 ? pd.wg_end[b - 1] : 0)) / g.H;
    if constexpr (kNew) {
      nn = pd.n_new[b];
      slot0 = pd.new_slot0[b];
    }
  }
  const int nst = a.n_new;                           // rows per unit in k_new / v_new
  __shared__ float ew[kMaxSplits], el[kMaxSplits];
  __shared__ float lgw[kNew ? kMaxStepNew : 1][NW];  // per-wave parts of the new logits
  float v[kBatch];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sk = s0 + k < S ? s0 + k : S - 1;   // clamped: unconditional loads
      v[k] = pu[sk * stride + c];
    }
  };
  load_batch(0);
  // split maxima and sums: thread c reads split c (clamped, unconditional, in
  // flight with the partials); splits beyond D are read further down
  const int sk0 = c < S ? c : S - 1;
  const float m0 = pu[sk0 * stride + D], l0 = pu[sk0 * stride + D + 1];
  // The first kPreNew appended tokens' key and value elements are loaded with
  // the partials (clamped indices, unconditional), so one round trip covers
  // the merge; further tokens (up to kMaxStepNew) are read where used.
  constexpr int kPreNew = 4;
  uint16_t kn[kPreNew], vn[kPreNew];
  if constexpr (kNew) {
    const float qc = bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[((int64_t)b * g.H * GQA + kvh * GQA + h) * D + c]);
#pragma unroll
    for (int t = 0; t < kPreNew; ++t) {
      const int tc = t < nn ? t : (nn > 0 ? nn - 1 : 0);
      const int64_t row = ((int64_t)unit * nst + tc) * D + c;
      kn[t] = a.k_new[row];
      vn[t] = a.v_new[row];
    }
    for (int t = 0; t < nn; ++t) {
      const uint16_t kb = t < kPreNew ? kn[t < kPreNew ? t : 0] : a.k_new[((int64_t)unit * nst + t) * D + c];
      float x = qc * bf16_bits_to_f32(kb);
#pragma unroll
      for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, W);
      if (c % W == 0) lgw[t][c / W] = x;
    }
  }
  if (c < S) {
    ew[c] = m0;
    el[c] = l0;
  }
  for (int sk = c + D; sk < S; sk += D) {
    ew[sk] = pu[sk * stride + D];
    el[sk] = pu[sk * stride + D + 1];
  }
  __syncthreads();
  auto new_logit = [&](int t) {
    float x = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) x += lgw[t][w];
    return x * a.qscale;
  };
  float M = -INFINITY;
  for (int sk = 0; sk < S; ++sk) M = fmaxf(M, ew[sk]);   // -inf only for empty splits
  if constexpr (kNew) {
    for (int t = 0; t < nn; ++t) M = fmaxf(M, new_logit(t));
  }
  __syncthreads();
  for (int sk = c; sk < S; sk += D) {
    const float e = ew[sk] == -INFINITY ? 0.0f : fast_exp2(ew[sk] - M);   // empty split: weight 0
    ew[sk] = e;
    el[sk] *= e;
  }
  __syncthreads();
  float num = 0.0f, den = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    if (s0 > 0) load_batch(s0);
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (s0 + k < S) num = fmaf(v[k], ew[s0 + k], num);
  }
  for (int sk = 0; sk < S; ++sk) den += el[sk];
  if constexpr (kNew) {
    auto fold_new = [&](int t, uint16_t kb, uint16_t vb) {
      const float e = fast_exp2(new_logit(t) - M);
      num = fmaf(e, bf16_bits_to_f32(vb), num);
      den += e;
      if (h == 0) {
        int slot = slot0 + t;
        slot = slot >= g.ring ? slot - g.ring : slot;
        a.ring_k[((int64_t)unit * g.ring + slot) * D + c] = kb;
        a.ring_v[((int64_t)unit * g.ring + slot) * D + c] = vb;
      }
    };
#pragma unroll
    for (int t = 0; t < kPreNew; ++t)
      if (t < nn) fold_new(t, kn[t], vn[t]);
    for (int t = kPreNew; t < nn; ++t) {
      const int64_t row = ((int64_t)unit * nst + t) * D + c;
      fold_new(t, a.k_new[row], a.v_new[row]);
    }
  }
  a.out[((int64_t)b * g.H * GQA + kvh * GQA + h) * D + c] = num / den;
}

// Agent-scope accesses to the split partials: coherent across the XCDs
// (sc1: written through to memory, read past the XCD's L2), with no
// cache-wide writeback or invalidate (which an agent-scope fence implies on
// gfx950: a whole-L2 writeback per workgroup).  The same cache policy the
// compiler gives agent-scope relaxed atomic loads and stores, on 16-byte
// buffer accesses.
constexpr int kCoherent = 0x10;   // buffer cache policy: sc1
typedef unsigned u4v_t __attribute__((ext_vector_type(4)));
typedef unsigned u2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_agent4(__amdgpu_buffer_rsrc_t r, int off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4v_t, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ void store_agent2(__amdgpu_buffer_rsrc_t r, int off, float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2v_t, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ float4 load_agent4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ float2 load_agent2(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherent));
}
// Wait until every memory operation this wave issued has been performed:
// the partial stores above it are visible device-wide before the arrival
// counter below it moves.
__device__ __forceinline__ void wait_memory_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);      // vmcnt(0) expcnt(0) lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float4 f4_scale(float4 v, float s) { return make_float4(v.x * s, v.y * s, v.z * s, v.w * s); }
__device__ __forceinline__ float4 f4_fma(float4 v, float s, float4 acc) {
  return make_float4(fmaf(v.x, s, acc.x), fmaf(v.y, s, acc.y), fmaf(v.z, s, acc.z), fmaf(v.w, s, acc.w));
}
__device__ __forceinline__ float4 f4_add(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// End of one workgroup's share of a unit (batch, KV head).  The four waves'
// online-softmax states (m, l per head; red[w][h][c] = acc relative to the
// wave's own maximum) are folded into the split's state.  Then:
//   * one split and nothing appended: the workgroup writes the output;
//   * more than kLastMergeSplits splits: it writes its partial for merge_kernel;
//   * otherwise it publishes its partial (agent-scope stores, waited for) and
//     takes an arrival ticket from the unit's counter (agent-scope increment
//     that wraps back to 0 on the last arrival, leaving the counter ready for
//     the next call).  The last workgroup to arrive merges every split's
//     partial (flash-decoding merge, "KV Cache and autoregressive video
//     generation", section 05), adds the nn tokens appended by the same call
//     (decode step) as further softmax terms -- logit sigma log2(e) q . k_new
//     from qf(h, c) = sigma log2(e) q[h][c] -- writes them into their window
//     slots (slot0 + t, wrapped), and writes the output.
// Thread t owns output channels c0 .. c0 + 3 of head h (group t % NT) and, in
// the merge, every NSG-th split from t / NT; partial rows are D + 4 floats so
// that every access is 16 bytes.  k_new / v_new rows of unit u start at row
// u * nst.
// A decode step's first appended token as the kernel prologue prepared it
// (loaded with the query, its logits computed while the tiles stream):
// logit of head wave + kWaves i, key channels lane + kWave j, and value
// channels c0 .. c0 + 3 of the thread's output group.
// First output channel of thread tid in the merge (groups of four channels,
// head-major): the value channels a decode step's first appended token
// contributes through that thread.
// Row pitch (floats) of a wave's per-head results in LDS: rows of successive
// heads start 16 banks apart, so the sixteen-channel stores of four heads and
// the merge's 16-byte reads of consecutive channels are free of bank conflicts.
constexpr int red_pitch(int d) { return d + 16; }

template <int D, int GQA>
__device__ __forceinline__ int merge_c0(int tid) {
  return 4 * (tid % (GQA * D / 4)) % D;
}

template <int D, int GQA>
struct FirstNew {
  static constexpr int kHeads = (GQA + kWaves - 1) / kWaves;
  static constexpr int kKeys = (D + kWave - 1) / kWave;
  float lg[kHeads];
  uint16_t kr[kKeys];
  uint2 vr;
};
struct NoFirstNew {};

// The end of a unit's share done by wave 0 alone (finish_unit decides when):
// lane i folds the four waves' results of output groups i, i + 64, ... (a
// group is four channels of one head), publishes them and takes the ticket
// itself (its own stores waited for), and as the last arriver merges the
// splits' partials, weighted by a butterfly over the lanes that hold the
// splits' (m, l), and the appended token when there is one (folded in by an
// online-softmax rescale).  Partial rows and the ticket are those of
// finish_unit's workgroup-wide path.  The loops over splits are unrolled over
// NS >= S slots.
template <int D, int GQA, int GPL, int NS, bool kFirst, typename QF, typename FN>
__device__ __forceinline__ void merge_in_wave(const DecodeArgs& a, int unit, int split, int S, int nn, int slot0,
                                              float (*red)[GQA][red_pitch(D)], float (*wml)[2][GQA],
                                              float (*sm)[GQA], float (*sl)[GQA], float (*lg)[GQA], QF qf,
                                              const FN& fn) {
  constexpr int NT = GQA * D / 4;
  constexpr int RS = D + 4;
  constexpr int KPL = (D + kWave - 1) / kWave;
  constexpr int sstride = GQA * RS;
  const int lane = threadIdx.x % kWave;
  int hk[GPL], ck[GPL];
  float4 num[GPL];
  float den[GPL], mk[GPL];
#pragma unroll
  for (int k = 0; k < GPL; ++k) {
    const int gk = (lane + kWave * k) % NT;                  // lanes past NT repeat a group, write nothing
    hk[k] = 4 * gk / D;
    ck[k] = 4 * gk % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, wml[w][0][hk[k]]);
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float ll = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = (wml[w][0][hk[k]] == -INFINITY) ? 0.0f : fast_exp2(wml[w][0][hk[k]] - mm);
      acc = f4_fma(*reinterpret_cast<const float4*>(&red[w][hk[k]][ck[k]]), e, acc);
      ll += wml[w][1][hk[k]] * e;
    }
    num[k] = acc;
    den[k] = ll;
    mk[k] = mm;
  }
  auto owns = [&](int k) { return lane + kWave * k < NT; };
  if (S > 1) {
    float* pu = a.part + (int64_t)unit * a.splits * sstride;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, S * sstride * 4, kRsrcWord3);
#pragma unroll
    for (int k = 0; k < GPL; ++k) {
      if (owns(k)) {
        store_agent4(rp, (split * sstride + hk[k] * RS + ck[k]) * 4, num[k]);
        if (ck[k] == 0) store_agent2(rp, (split * sstride + hk[k] * RS + D) * 4, make_float2(mk[k], den[k]));
      }
    }
    wait_memory_done();
    uint32_t t = 0;
    if (lane == 0) t = __builtin_amdgcn_atomic_inc32(a.ctr + unit, (uint32_t)(S - 1), __ATOMIC_RELAXED, "agent");
    t = __builtin_amdgcn_readfirstlane(t);
    if (t != (uint32_t)(S - 1)) return;
    // the last arriver: every other split's partials and every (m, l)
    float4 v[GPL][NS];
#pragma unroll
    for (int sk = 0; sk < NS; ++sk) {
      if (sk < S && sk != split) {
#pragma unroll
        for (int k = 0; k < GPL; ++k) v[k][sk] = load_agent4(rp, (sk * sstride + hk[k] * RS + ck[k]) * 4);
      }
    }
    const float2 ml = lane < S * GQA ? load_agent2(rp, ((lane / GQA) * sstride + (lane % GQA) * RS + D) * 4)
                                     : make_float2(-INFINITY, 0.0f);
    // lane j holds split j / GQA, head j % GQA (GQA a power of two)
    float M = ml.x;
#pragma unroll
    for (int msk = GQA; msk < kWave; msk *= 2) M = fmaxf(M, __shfl_xor(M, msk));
    if (lane < S * GQA) {
      const float e = ml.x == -INFINITY ? 0.0f : fast_exp2(ml.x - M);   // empty split: 0
      sm[lane / GQA][lane % GQA] = e;
      sl[lane / GQA][lane % GQA] = ml.y * e;
    }
    if (lane < GQA) lg[kMaxStepNew - 1][lane] = M;             // the heads' maxima (a spare row)
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < GPL; ++k) {
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      float ll = 0.0f;
#pragma unroll
      for (int sk = 0; sk < NS; ++sk) {
        if (sk < S) {
          acc = f4_fma(sk == split ? num[k] : v[k][sk], sm[sk][hk[k]], acc);
          ll += sl[sk][hk[k]];
        }
      }
      num[k] = acc;
      den[k] = ll;
      mk[k] = lg[kMaxStepNew - 1][hk[k]];
    }
  }
  if (nn == 1) {
    // the appended token: its key and value (channels c0 .. c0 + 3, the same
    // for every group of a lane), its logits per head
    const uint16_t* kn = a.k_new + (int64_t)unit * a.n_new * D;
    const uint16_t* vn = a.v_new + (int64_t)unit * a.n_new * D;
    uint16_t kr[KPL];
    uint2 vr;
    float lgh[GQA];
    if constexpr (kFirst) {
#pragma unroll
      for (int j = 0; j < KPL; ++j) kr[j] = fn.kr[j];
      vr = fn.vr;
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) lgh[hh] = lg[0][hh];
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int c = lane + j * kWave;
        kr[j] = kn[c < D ? c : 0];
      }
      vr = *reinterpret_cast<const uint2*>(vn + ck[0]);
#pragma unroll
      for (int hh = 0; hh < GQA; ++hh) {
        float x = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int c = lane + j * kWave;
          if (c < D) x = fmaf(qf(hh, c), bf16_bits_to_f32(kr[j]), x);
        }
        lgh[hh] = wave_sum(x);
      }
    }
    const float4 vt = make_float4(bf16_lo(vr.x), bf16_hi(vr.x), bf16_lo(vr.y), bf16_hi(vr.y));
#pragma unroll
    for (int k = 0; k < GPL; ++k) {
      float x = lgh[0];
#pragma unroll
      for (int hh = 1; hh < GQA; ++hh) x = hk[k] == hh ? lgh[hh] : x;
      const float mt = fmaxf(mk[k], x);
      const float sc = mk[k] == -INFINITY ? 0.0f : fast_exp2(mk[k] - mt);   // no cached term: 0
      const float e = fast_exp2(x - mt);
      num[k] = f4_fma(vt, e, f4_scale(num[k], sc));
      den[k] = den[k] * sc + e;
    }
    // the token into its window slot
    uint16_t* rk = a.ring_k + (int64_t)unit * a.g.ring * D;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int c = lane + j * kWave;
      if (c < D) rk[slot0 * D + c] = kr[j];
    }
    if (4 * lane < D) *reinterpret_cast<uint2*>(a.ring_v + ((int64_t)unit * a.g.ring + slot0) * D + 4 * lane) = vr;
  }
#pragma unroll
  for (int k = 0; k < GPL; ++k)
    if (owns(k)) *reinterpret_cast<float4*>(a.out + (int64_t)unit * GQA * D + hk[k] * D + ck[k]) = f4_scale(num[k], 1.0f / den[k]);
}

template <int D, int GQA, typename QF, typename FN = NoFirstNew>
__device__ __forceinline__ void finish_unit(const DecodeArgs& a, int unit, int split, int S, int nn, int nst,
                                            int slot0, float (*red)[GQA][red_pitch(D)], float (*wml)[2][GQA],
                                            const float* m, const float* l, QF qf, const FN& fn = FN{}) {
  constexpr bool kFirst = !__is_same(FN, NoFirstNew);
  constexpr int NT = GQA * D / 4;                            // 16-byte output groups of a unit
  constexpr int NSG = kThreads / NT;                         // split groups of the merge
  static_assert(NT <= kThreads && kThreads % NT == 0, "output groups tile the workgroup");
  constexpr int RS = D + 4;                                  // floats per (split, head) partial row
  constexpr int KPL = (D + kWave - 1) / kWave;               // key channels per lane (new-token logits)
  const Geom& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int grp = tid % NT, sgi = tid / NT;
  const int h = 4 * grp / D, c0 = merge_c0<D, GQA>(tid);
  __shared__ float sm[kLastMergeSplits][GQA], sl[kLastMergeSplits][GQA];
  __shared__ float lg[kMaxStepNew][GQA], mx[GQA];
  __shared__ float4 racc[NSG > 1 ? NSG - 1 : 1][NT];
  __shared__ int last;
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < GQA; ++hh) {
      wml[wave][0][hh] = m[hh];
      wml[wave][1][hh] = l[hh];
    }
  }
  // Few splits and at most one appended token: after the fold's barrier wave
  // 0 does the rest alone (fold, publication, ticket, merge), with no further
  // workgroup barrier.  The appended token's logits go through LDS first.
  constexpr int GPL = (NT + kWave - 1) / kWave;              // output groups per lane of wave 0
  const bool wave_merge = GPL <= 4 && nn <= 1 && ((S > 1 && S <= kWaveMergeSplits && a.last_merge) ||
                                                 (S == 1 && nn == 1));
  if constexpr (kFirst) {
    if (wave_merge && nn == 1 && lane == 0) {
#pragma unroll
      for (int i = 0; i < FN::kHeads; ++i) {
        const int hh = wave + kWaves * i;
        if (hh < GQA) lg[0][hh] = fn.lg[i];
      }
    }
  }
  __syncthreads();
  if constexpr (GPL <= 4) {
    if (wave_merge) {
      // unrolled over NS split slots: the smallest instance that holds S
      if (wave == 0) {
        if (S <= 4) merge_in_wave<D, GQA, GPL, 4, kFirst>(a, unit, split, S, nn, slot0, red, wml, sm, sl, lg, qf, fn);
        else merge_in_wave<D, GQA, GPL, kWaveMergeSplits, kFirst>(a, unit, split, S, nn, slot0, red, wml, sm, sl, lg, qf, fn);
      }
      return;
    }
  }
  float4 fs = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float fm = -INFINITY, fl = 0.0f;
  if (sgi == 0) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) fm = fmaxf(fm, wml[w][0][h]);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = (wml[w][0][h] == -INFINITY) ? 0.0f : fast_exp2(wml[w][0][h] - fm);
      fs = f4_fma(*reinterpret_cast<const float4*>(&red[w][h][c0]), e, fs);
      fl += wml[w][1][h] * e;
    }
  }
  float4* out = reinterpret_cast<float4*>(a.out + (int64_t)unit * GQA * D + h * D + c0);
  if (S == 1 && nn == 0) {
    if (sgi == 0) *out = f4_scale(fs, 1.0f / fl);
    return;
  }
  const int sstride = GQA * RS;                              // floats between splits
  float* pu = a.part + (int64_t)unit * a.splits * sstride;
  if (!a.last_merge) {                                       // merge_kernel merges
    if (sgi == 0) {
      float* ps = pu + split * sstride + h * RS;
      *reinterpret_cast<float4*>(ps + c0) = fs;
      if (c0 == 0) *reinterpret_cast<float2*>(ps + D) = make_float2(fm, fl);
    }
    return;
  }
  // the unit's partials through one buffer resource (byte offsets)
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, S * sstride * 4, kRsrcWord3);
  if (S > 1) {
    if (sgi == 0) {
      store_agent4(rp, (split * sstride + h * RS + c0) * 4, fs);
      if (c0 == 0) store_agent2(rp, (split * sstride + h * RS + D) * 4, make_float2(fm, fl));
    }
    wait_memory_done();
    __syncthreads();
    if (tid == 0)
      last = __builtin_amdgcn_atomic_inc32(a.ctr + unit, (uint32_t)(S - 1), __ATOMIC_RELAXED, "agent") ==
             (uint32_t)(S - 1);
    __syncthreads();
    if (!last) return;
  }
  // ---- the last workgroup of the unit: merge ----
  // Every load of the merge goes out together: the first batch of partials,
  // the split maxima and sums, and the appended tokens' keys and values.
  // Only the splits that exist are read; with at most four partials per
  // thread a short path does it (the unrolled batch's skipped slots and its
  // longer code cost about half a microsecond on this serial tail).
  constexpr int kFew = 4;
  float4 v[kMergeBatch];
  const bool few = S <= kFew * NSG;
  const bool in_wave = S * GQA <= kWave;                    // every split's (m, l) in one wave
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int sk = sgi + NSG * (j0 + j);
      if (sk < S) v[j] = load_agent4(rp, (sk * sstride + h * RS + c0) * 4);
    }
  };
  if (S > 1) {
    if (few) {
#pragma unroll
      for (int j = 0; j < kFew; ++j) {
        const int sk = sgi + NSG * j;
        if (sk < S) v[j] = load_agent4(rp, (sk * sstride + h * RS + c0) * 4);
      }
    } else {
      load_batch(0);
    }
    if (in_wave) {
      // Lane j of wave 0 holds split j / GQA's (m, l) for head j % GQA: the
      // heads' maxima over the splits by a butterfly over the lanes of one
      // head (GQA is a power of two), then each split's weight.
      if (tid < kWave) {
        const float2 ml = tid < S * GQA ? load_agent2(rp, ((tid / GQA) * sstride + (tid % GQA) * RS + D) * 4)
                                        : make_float2(-INFINITY, 0.0f);
        float M = ml.x;
#pragma unroll
        for (int msk = GQA; msk < kWave; msk *= 2) M = fmaxf(M, __shfl_xor(M, msk));
        if (tid < S * GQA) {
          const float e = ml.x == -INFINITY ? 0.0f : fast_exp2(ml.x - M);   // empty split: 0
          sm[tid / GQA][tid % GQA] = e;
          sl[tid / GQA][tid % GQA] = ml.y * e;
        }
        if (tid < GQA) mx[tid] = M;
      }
    } else {
      for (int j = tid; j < S * GQA; j += kThreads) {
        const float2 ml = load_agent2(rp, ((j / GQA) * sstride + (j % GQA) * RS + D) * 4);
        sm[j / GQA][j % GQA] = ml.x;
        sl[j / GQA][j % GQA] = ml.y;
      }
    }
  } else if (sgi == 0 && c0 == 0) {                          // one split: weight 1
    const float e = fm == -INFINITY ? 0.0f : 1.0f;
    sm[0][h] = e;
    sl[0][h] = fl * e;
    mx[h] = fm;
  }
  if (S == 1) v[0] = fs;
  const uint16_t* kn = a.k_new + (int64_t)unit * nst * D;
  const uint16_t* vn = a.v_new + (int64_t)unit * nst * D;
  // Token 0 in registers (from the prologue when it prepared it); tokens
  // 1 .. nn - 1 (a step of several tokens) are read again where they are
  // used, in loops that do not run for a single token.
  uint16_t kr0[KPL];
  uint2 vr0 = make_uint2(0u, 0u);                            // channels c0 .. c0 + 3 (bf16)
  if (nn > 0) {
    if constexpr (kFirst) {
#pragma unroll
      for (int j = 0; j < KPL; ++j) kr0[j] = fn.kr[j];
      vr0 = fn.vr;
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int c = lane + j * kWave;
        kr0[j] = kn[c < D ? c : 0];
      }
      vr0 = *reinterpret_cast<const uint2*>(vn + c0);
    }
    // logits of the appended tokens, one wave per head
#pragma unroll
    for (int i = 0; i < (GQA + kWaves - 1) / kWaves; ++i) {
      const int hh = wave + kWaves * i;
      if (hh < GQA) {
        float x0 = 0.0f;
        if constexpr (kFirst) {
          x0 = fn.lg[i];
        } else {
#pragma unroll
          for (int j = 0; j < KPL; ++j) {
            const int c = lane + j * kWave;
            if (c < D) x0 = fmaf(qf(hh, c), bf16_bits_to_f32(kr0[j]), x0);
          }
          x0 = wave_sum(x0);
        }
        if (lane == 0) lg[0][hh] = x0;
        for (int t = 1; t < nn; ++t) {
          float x = 0.0f;
#pragma unroll
          for (int j = 0; j < KPL; ++j) {
            const int c = lane + j * kWave;
            if (c < D) x = fmaf(qf(hh, c), bf16_bits_to_f32(kn[t * D + c]), x);
          }
          x = wave_sum(x);
          if (lane == 0) lg[t][hh] = x;
        }
      }
    }
  }
  __syncthreads();
  if (!in_wave && S > 1) {
    // Many splits: the heads' maxima over the splits, then the weights.
    if (tid < GQA) {
      float M = -INFINITY;
      for (int sk = 0; sk < S; ++sk) M = fmaxf(M, sm[sk][tid]);   // -inf only for empty splits
      mx[tid] = M;
    }
    __syncthreads();
    for (int j = tid; j < S * GQA; j += kThreads) {
      const int sk = j / GQA, hh = j % GQA;
      const float e = sm[sk][hh] == -INFINITY ? 0.0f : fast_exp2(sm[sk][hh] - mx[hh]);   // empty split: 0
      sm[sk][hh] = e;
      sl[sk][hh] *= e;
    }
    __syncthreads();
  }
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (few) {
#pragma unroll
    for (int j = 0; j < kFew; ++j) {
      const int sk = sgi + NSG * j;
      if (sk < S) num = f4_fma(v[j], sm[sk][h], num);
    }
  } else {
    for (int j0 = 0; sgi + NSG * j0 < S; j0 += kMergeBatch) {
      if (j0 > 0) load_batch(j0);
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const int sk = sgi + NSG * (j0 + j);
        if (sk < S) num = f4_fma(v[j], sm[sk][h], num);
      }
    }
  }
  // the appended keys into their window slots, from wave 0's registers --
  // after the last barrier when all of wave 0 gets there (a barrier waits
  // for the stores before it)
  constexpr bool kKeysLate = NT >= kWave;
  auto store_keys = [&]() {
    if (nn > 0 && wave == 0) {
      uint16_t* rk = a.ring_k + (int64_t)unit * g.ring * D;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int c = lane + j * kWave;
        if (c < D) rk[slot0 * D + c] = kr0[j];
      }
      for (int t = 1; t < nn; ++t) {
        int slot = slot0 + t;
        slot = slot >= g.ring ? slot - g.ring : slot;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int c = lane + j * kWave;
          if (c < D) rk[slot * D + c] = kn[t * D + c];
        }
      }
    }
  };
  if constexpr (!kKeysLate) store_keys();
  if constexpr (NSG > 1) {
    if (sgi > 0) racc[sgi - 1][grp] = num;
    __syncthreads();
  }
  if (sgi != 0) return;
  if constexpr (kKeysLate) store_keys();
#pragma unroll
  for (int k = 0; k + 1 < NSG; ++k) num = f4_add(num, racc[k][grp]);
  float den = 0.0f;
  for (int sk = 0; sk < S; ++sk) den += sl[sk][h];
  // The appended tokens' terms (and their values into their window slots):
  // the splits' sum, relative to their maximum, is rescaled to the maximum
  // that includes the new logits (online softmax).
  float mt = mx[h];
  if (nn > 0) {
    for (int t = 0; t < nn; ++t) mt = fmaxf(mt, lg[t][h]);
    const float sc = mx[h] == -INFINITY ? 0.0f : fast_exp2(mx[h] - mt);   // no cached term: 0
    num = f4_scale(num, sc);
    den *= sc;
  }
  for (int t = 0; t < nn; ++t) {
    const uint2 vt = t == 0 ? vr0 : *reinterpret_cast<const uint2*>(vn + t * D + c0);
    const float e = fast_exp2(lg[t][h] - mt);
    num = f4_fma(make_float4(bf16_lo(vt.x), bf16_hi(vt.x), bf16_lo(vt.y), bf16_hi(vt.y)), e, num);
    den += e;
    if (h == 0) {
      int slot = slot0 + t;
      slot = slot >= g.ring ? slot - g.ring : slot;
      *reinterpret_cast<uint2*>(a.ring_v + ((int64_t)unit * g.ring + slot) * D + c0) = vt;
    }
  }
  *out = f4_scale(num, 1.0f / den);
}

template <int D, int GQA>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int unit, float (*qsT)[GQA]) {
  const Geom& g = a.g;
  const int b = unit / g.H, kvh = unit % g.H;
  const int64_t row = ((int64_t)b * g.H * GQA + kvh * GQA) * D;
  // The dtype test stays outside the loops, so that the loads of a thread
  // are unconditional and in flight together.
  if (g.dtype == KVQ_BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + row;
    for (int i = threadIdx.x; i < GQA * D; i += kThreads) qsT[i % D][i / D] = bf16_bits_to_f32(q[i]) * a.qscale;
  } else {
    const float* q = static_cast<const float*>(a.q) + row;
    for (int i = threadIdx.x; i < GQA * D; i += kThreads) qsT[i % D][i / D] = q[i] * a.qscale;
  }
}

// Work of one wave: quantized tiles [t0, t1) and window chunks [c0, c1).
// Split s owns an equal share of the tiles and of the chunks (so the window
// is spread over the splits).  The split's chunks are dealt to its waves as
// evenly as they go (one each while there are at most four), and the tiles
// fill the waves around them, a chunk counting as kChunkCost tiles: a wave
// then meets each Key segment once, and no wave has to read a second chunk
// after computing its first (a dependent round trip at the end of the call)
// unless the split holds more chunks than waves.
struct WaveWork {
  int t0, t1, c0, c1;
};
template <int kChunkCost>
__device__ __forceinline__ WaveWork wave_work(const DecodeArgs& a, int split, int wave) {
  // the first (count % splits) splits take one item more (no division here)
  const int ts0 = split * a.tq_div + (split < a.tq_mod ? split : a.tq_mod);
  const int ts1 = ts0 + a.tq_div + (split < a.tq_mod ? 1 : 0);
  const int cs0 = split * a.ch_div + (split < a.ch_mod ? split : a.ch_mod);
  const int cs1 = cs0 + a.ch_div + (split < a.ch_mod ? 1 : 0);
  const int nt = ts1 - ts0, nc = cs1 - cs0;
  const int cost = nt + kChunkCost * nc;
  // chunks before wave w, and tiles before it (clamped, non-decreasing in w)
  auto chunks_before = [&](int w) { return (nc * w) / kWaves; };
  auto tiles_before = [&](int w) {
    int tb = 0;
    for (int v = 1; v <= w; ++v) {
      int x = (cost * v) / kWaves - kChunkCost * chunks_before(v);
      x = x > nt ? nt : x;
      tb = x > tb ? x : tb;
    }
    return tb;
  };
  WaveWork ww;
  ww.t0 = ts0 + tiles_before(wave);
  ww.t1 = ts0 + tiles_before(wave + 1);
  ww.c0 = cs0 + chunks_before(wave);
  ww.c1 = cs0 + chunks_before(wave + 1);
  return ww;
}

// ---- vector-ALU kernel (every shape) ------------------------------------------------

// kSameAxis (uniform caches): Keys and Values carry one scale per token and
// run of kRunChannels channels.  A logit is then sum over runs r of
// (sum_{c in r} q[c] code[c]) / kscale[t][r], and a Value weight depends on
// the channel's run: p / vscale[t][r].
template <int D, int BITS, int GQA, bool kPaged = false, bool kSameAxis = false>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a0, PagedDecode pd) {
  static_assert(!(kPaged && kSameAxis), "paged caches use the KIVI axes");
  static_assert(!kSameAxis || D % kRunChannels == 0, "same-axis runs divide head_dim");
  constexpr int W = D * BITS / 8;        // bytes per token row
  constexpr int NSLOT = W / 16;          // 16-byte units per lane per tile
  constexpr int TPU = 128 / BITS;        // tokens per Value unit
  constexpr int FPW = 32 / BITS;         // fields per 32-bit word
  constexpr int NR = kSameAxis ? D / kRunChannels : 1;   // scales per token (same-axis)
  constexpr int TCPL = TailMap<D>::TCPL;
  const Geom& g = a0.g;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  int unit = blockIdx.y;
  int split = blockIdx.x;
  int S = a0.splits, nn = a0.n_new, slot0 = a0.new_slot0;
  // Paged caches: this sequence's lengths and work split (uniform caches:
  // the arguments as given).
  DecodeArgs pa = a0;
  if constexpr (kPaged) {
    const PagedUnit pu = paged_unit(pd, a0.g.H, a0.g.B, blockIdx.x);
    unit = pu.unit;
    split = pu.split;
    S = pu.ws;
    nn = pd.n_new[unit / g.H];
    slot0 = pd.new_slot0[unit / g.H];
    pa = paged_args(a0, pd, unit, pu.ws);
  }
  const DecodeArgs& a = pa;

  __shared__ float qsT[D][GQA];
  __shared__ float aq[kWaves][D][GQA];
  __shared__ float pw[kWaves][kTile * NR][GQA];   // same-axis: row NR t + r
  __shared__ __attribute__((aligned(16))) float red[kWaves][GQA][red_pitch(D)];
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

  const WaveWork ww = wave_work<2>(a, split, wave);
  const uint8_t* kbase = a.k_codes + (int64_t)unit * g.code_stream;
  const uint8_t* vbase = a.v_codes + (int64_t)unit * g.code_stream;
  const uint16_t* ksbase = a.k_scale + (int64_t)unit * g.max_seg * D;
  const uint16_t* vsbase = a.v_scale + (int64_t)unit * g.C;
  int cur_seg = -1;

  for (int chunk = ww.c0; chunk < ww.c1; ++chunk) {
    TailRegs<D, false> tr;
    tail_load<D, false>(a, unit, chunk, tr);
    tail_compute<D, GQA, false>(a, tr, qsT, pw[wave], m, l, alpha, acc_tail);
#pragma unroll
    for (int h = 0; h < GQA; ++h)
#pragma unroll
      for (int k = 0; k < NSLOT; ++k) acc[k][h] *= alpha[h];
  }
  for (int tile = ww.t0; tile < ww.t1; ++tile) {
    const int t = tile * kTile + lane;
    const bool valid = t < a.nq;
    const uint8_t* kt;
    const uint8_t* vt;
    const uint16_t* vs_tile;     // Value scales of the tile's tokens
    const uint16_t* ks_page;     // the tile's Key-scale row (paged)
    if constexpr (kPaged) {
      int64_t pg = pd.table[(int64_t)(unit / g.H) * pd.stride + tile];
      pg = pg < 0 ? 0 : (pg >= pd.n_pages ? pd.n_pages - 1 : pg);   // clamped into the pool
      kt = pd.pool + pg * pd.page_bytes + (int64_t)(unit % g.H) * pd.head_bytes;
      vt = kt + kTile * W;
      vs_tile = reinterpret_cast<const uint16_t*>(kt + 2 * kTile * W);
      ks_page = vs_tile + kTile;
    } else {
      kt = kbase + (int64_t)tile * (kTile * W);
      vt = vbase + (int64_t)tile * (kTile * W);
      vs_tile = vsbase + tile * kTile;
      ks_page = nullptr;
    }
    // Issue every load of the tile before any arithmetic.
    uint4 kc[NSLOT], vc[NSLOT];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) kc[j] = *reinterpret_cast<const uint4*>(kt + j * 1024 + lane * 16);
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) vc[k] = *reinterpret_cast<const uint4*>(vt + (k * kWave + lane) * 16);
    const float vs = (valid && !kSameAxis) ? half_bits_to_f32(vs_tile[lane]) : 1.0f;
    float logit[GQA];
#pragma unroll
    for (int h = 0; h < GQA; ++h) logit[h] = 0.0f;
    float rvs[NR];            // same-axis: 1 / vscale of the token's runs

    if constexpr (kSameAxis) {
      // this token's run scales (NR consecutive fp16 per token)
      const int64_t srow = ((int64_t)unit * g.C + (valid ? t : 0)) * NR;
      float rks[NR], part[NR][GQA];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        rks[r] = valid ? fast_rcp(fmaxf(half_bits_to_f32(a.k_scale[srow + r]), g.eps)) : 0.0f;
        rvs[r] = valid ? fast_rcp(fmaxf(half_bits_to_f32(a.v_scale[srow + r]), g.eps)) : 0.0f;
#pragma unroll
        for (int h = 0; h < GQA; ++h) part[r][h] = 0.0f;
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
            for (int h = 0; h < GQA; ++h) part[c / kRunChannels][h] = fmaf(qsT[c][h], code, part[c / kRunChannels][h]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int h = 0; h < GQA; ++h) logit[h] = fmaf(part[r][h], rks[r], logit[h]);
    } else if (g.G > 0) {
      const int seg = tile / a.tiles_per_seg;
      if (seg != cur_seg) {
        cur_seg = seg;
        const uint16_t* ks = kPaged ? ks_page : ksbase + seg * D;
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
      if constexpr (kSameAxis) {
#pragma unroll
        for (int r = 0; r < NR; ++r) pw[wave][lane * NR + r][h] = p * rvs[r];
      } else {
        pw[wave][lane][h] = p * vinv;
      }
    }
    wave_lds_sync();

    // Values: lane owns NSLOT (channel, token-run) units of the tile; the
    // token run starts at t0, the same for every slot of the lane.
    const int t0 = ((lane * 16) % (8 * BITS)) * 8 / BITS;
#pragma unroll
    for (int f = 0; f < TPU; ++f) {
      float pf[NR][GQA];
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int h = 0; h < GQA; ++h) pf[r][h] = pw[wave][(t0 + f) * NR + r][h];
#pragma unroll
      for (int k = 0; k < NSLOT; ++k) {
        // slot k holds channel (64 k + lane) * 2 / BITS: run 2 k / BITS (same-axis)
        const int r = kSameAxis ? (2 * k) / BITS : 0;
        const uint32_t wd[4] = {vc[k].x, vc[k].y, vc[k].z, vc[k].w};
        const float code = static_cast<float>(sext_field<BITS>(wd[f / FPW], (f % FPW) * BITS));
#pragma unroll
        for (int h = 0; h < GQA; ++h) acc[k][h] = fmaf(pf[r][h], code, acc[k][h]);
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
      for (int h = 0; h < GQA; ++h) red[wave][h][c] = acc[k][h];
    }
  }
  wave_lds_sync();
  if (TailMap<D>::owns(lane)) {
#pragma unroll
    for (int k = 0; k < TCPL; ++k)
#pragma unroll
      for (int h = 0; h < GQA; ++h) red[wave][h][lane * TCPL + k] += acc_tail[k][h];
  }
  finish_unit<D, GQA>(a, unit, split, S, nn, a.n_new, slot0, red, wml, m, l,
                      [&](int h, int c) { return qsT[c][h]; });
}

// ---- int8-MFMA kernel (int4 / int2 codes, head_dim 64 / 128, whole-group segments) ----
//
// Both contractions of a 64-token tile run on v_mfma_i32_16x16x64_i8.  Lane l
// supplies row l % 16 of A and column l % 16 of B for k-group l / 16 (16 bytes
// each); element i of the result in lane l is row 4 (l / 16) + i, column l % 16.
//
// Codes: a b-bit two's-complement field moved to the top of a byte is the
// signed int8 value 2^(8-b) * code, so a packed word unpacks with a shift and
// an and per four fields and needs no bias correction.
//
// Key side: logit[head][token] = sum_c a[head][c] code[token][c] with
// a = sigma log2(e) q / kscale (per segment).  a is rounded to the 21-bit
// fixed-point integer v = round(a F) (F per head and segment, from a bound on
// |a|) and split into three balanced base-128 digits; MFMA row 4 h + d holds
// digit d of head h, so a head's three partial sums land in one lane and
// recombine exactly in fp32 (each is below 2^24).
//
// Value side: acc[head][c] += sum_t P[head][t] code[t][c] with
// P = Fv p / vscale[t], p = exp2(logit - running max) <= 1 and Fv fixed for the
// wave's run of tiles (from the largest 1 / vscale in it), so P is an unsigned
// 21-bit integer; its three base-128 digits go in rows 4 h + d.  A tile's
// int32 digit sums start from zero and are recombined into the fp32
// accumulator at once (acc = acc * alpha + sums), so no integer state is
// carried from tile to tile.
//
// Token order: slot j of the Value operand of k-group kg holds token
// 16 kg + f(j) (f = field order of the unpacked word); column col of Key MFMA
// g is token 16 (col / 4) + f(4 (col % 4) + g), so a lane owns the four tokens
// of one Value-operand dword and stores each digit with one 32-bit LDS write.

typedef int i4_t __attribute__((ext_vector_type(4)));

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// bf16 bits of x, rounded to nearest even (x finite).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// A 16-token chunk of the bf16 window as the matrix-core path reads it:
// Keys as the B operand of the score MFMA (lane (q4, col): channels
// 32 mk + 8 q4 .. + 8 of token col), Values by channel owner (TailMap).
template <int D>
struct ChunkRegs {
  uint4 k[D / 32];
  uint32_t v[kTailChunk];
  int nvalid;
};

// Sixteen packed b-bit fields (one operand k-group) -> four dwords of int8
// values 2^(8-b) * field; field(j) = the field held in operand slot j.
template <int BITS>
struct Fields16;

template <>
struct Fields16<4> {
  typedef uint2 raw_t;
  static constexpr float kMul = 16.0f;
  __device__ static i4_t unpack(raw_t r) {
    const uint32_t m = 0xF0F0F0F0u;
    return i4_t{(int)((r.x << 4) & m), (int)(r.x & m), (int)((r.y << 4) & m), (int)(r.y & m)};
  }
  // dword j/4 = even or odd nibbles of word j/8; byte j%4
  __host__ __device__ static constexpr int field(int j) { return 8 * (j / 8) + 2 * (j % 4) + (j / 4) % 2; }
  // operand slot of field f (the inverse of field)
  __host__ __device__ static constexpr int slot(int f) { return 8 * (f / 8) + 4 * (f % 2) + (f % 8) / 2; }
};

template <>
struct Fields16<2> {
  typedef uint32_t raw_t;
  static constexpr float kMul = 64.0f;
  __device__ static i4_t unpack(raw_t w) {
    const uint32_t m = 0xC0C0C0C0u;
    return i4_t{(int)((w << 6) & m), (int)((w << 4) & m), (int)((w << 2) & m), (int)(w & m)};
  }
  // dword j/4 = field j/4 of every byte; byte j%4
  __host__ __device__ static constexpr int field(int j) { return 4 * (j % 4) + j / 4; }
  __host__ __device__ static constexpr int slot(int f) { return 4 * (f % 4) + f / 4; }
};

template <int BITS>
constexpr bool slots_invert_fields() {
  for (int j = 0; j < 16; ++j)
    if (Fields16<BITS>::slot(Fields16<BITS>::field(j)) != j) return false;
  return true;
}
static_assert(slots_invert_fields<4>() && slots_invert_fields<2>(), "slot() inverts field()");

// Low bytes of four registers -> one dword (byte k from bk).
__device__ __forceinline__ uint32_t pack_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// round(x) + 0x102040 for |x| <= 2^20, from one fma: the magic constant
// 1.5 * 2^23 places the rounded integer in the low mantissa bits.
__device__ __forceinline__ uint32_t fixed_biased(float a, float f) {
  return __float_as_uint(fmaf(a, f, 12582912.0f)) - (0x4B400000u - 0x102040u);
}

// Recombine three base-128 digit sums (rows 4 h + 0..2 of an i32 MFMA result).
__device__ __forceinline__ float digits_value(const i4_t s) {
  return fmaf((float)s[0], 16384.0f, fmaf((float)s[1], 128.0f, (float)s[2]));
}

// Two waves per SIMD (<= 256 registers); eight heads per KV head need the
// register file of one wave per SIMD.
//
// Every wave works on its own from the first instruction to the workgroup
// fold: it loads the query itself (one 16-byte load per lane for four heads
// of 128 channels), and its run's first window chunk and first two tiles
// are in flight before it waits for anything, so a run of up to two tiles
// and a chunk (the Llama-3-8B shape at 4096 tokens) is one burst of loads.
// A tile takes 18 load instructions (int4, head_dim 128), so the burst stays
// within the 63 vector-memory instructions a wave can have outstanding and
// every wait is exact.  Later tiles refill the two-tile ring as tiles are
// computed.  The Value weights' fixed-point scale is set per tile from the
// tile's own scales, so nothing has to be read ahead of the first tile.
template <int D, int BITS, int GQA, typename PD = NoPaging>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(GQA > 4 ? 1 : 2)))
void decode_i8_kernel(DecodeArgs a0, PD pd) {
  constexpr bool kPaged = !__is_same(PD, NoPaging);
  using F16 = Fields16<BITS>;
  using raw_t = typename F16::raw_t;
  constexpr int W = D * BITS / 8;         // bytes per token row
  constexpr int MK = D / 64;              // Key MFMAs per token group (64 channels each)
  constexpr int NV = D / 16;              // Value MFMAs per head group (16 channels each)
  constexpr int HG = (GQA + 3) / 4;       // head groups of four MFMA row quads
  constexpr int TCPL = TailMap<D>::TCPL;
  constexpr int RPL = D / 64;             // Key-scale slots per lane in the operand build
  constexpr float kFixQ = 1047552.0f;     // 2^20 (1 - 2^-10): |round(a F)| <= 2^20
  constexpr float kFixP = 2097150.0f;     // P < 2^21: top digit <= 127
  constexpr int NQ16 = GQA * D / 8;       // 16-byte pieces of one unit's bf16 queries
  constexpr int QPL = (NQ16 + kWave - 1) / kWave;
  const Geom& g = a0.g;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int q4 = lane / 16, col = lane % 16;
  int unit = blockIdx.y;
  int split = blockIdx.x;
  int S = a0.splits, nn = a0.n_new, slot0 = a0.new_slot0;
  DecodeArgs pa = a0;
  if constexpr (kPaged) {
    const PagedUnit pu = paged_unit(pd, a0.g.H, a0.g.B, blockIdx.x);
    unit = pu.unit;
    split = pu.split;
    S = pu.ws;
    nn = pd.n_new[unit / g.H];
    slot0 = pd.new_slot0[unit / g.H];
    pa = paged_args(a0, pd, unit, pu.ws);
  }
  const DecodeArgs& a = pa;

  // Per wave: sigma log2(e) q in fp32 (channel order), its bf16 high part and
  // the bf16 rounding of the remainder (the window-chunk score operand),
  // 1 / kscale of the current segment (slot order), operand digits (rows
  // padded to 20 dwords so that the 16-byte operand reads -- lane col reads
  // row col -- spread over all banks) and window-chunk weights.
  constexpr int kRowPad = 20;
  __shared__ __attribute__((aligned(16))) float qsC[kWaves][GQA][D];
  __shared__ __attribute__((aligned(16))) uint16_t qsHL[kWaves][2][GQA][D];
  __shared__ __attribute__((aligned(16))) float rkP[kWaves][D];
  __shared__ __attribute__((aligned(16))) uint32_t qD[kWaves][HG][MK][16][kRowPad];  // Key operand digits
  __shared__ __attribute__((aligned(16))) uint32_t pD[kWaves][HG][16][kRowPad];      // Value operand digits
  __shared__ float pw[kWaves][kTailChunk][GQA];
  __shared__ __attribute__((aligned(16))) float red[kWaves][GQA][red_pitch(D)];
  __shared__ float wml[kWaves][2][GQA];

  // Channel (or token) held in slot position p of a 64-wide group.
  auto chan = [](int p) { return (p & ~15) + F16::field(p & 15); };

  // A 16-token bf16 window chunk moves as many bytes as an int4 tile and,
  // with its scores on the matrix cores, costs about as much.
  const WaveWork ww = wave_work<2>(a, split, wave);
  const int w_begin = ww.t0, q_end = ww.t1;
  const uint8_t* kbase = a.k_codes + (int64_t)unit * g.code_stream;
  const uint8_t* vbase = a.v_codes + (int64_t)unit * g.code_stream;
  const uint16_t* ksbase = a.k_scale + (int64_t)unit * g.max_seg * D;
  const uint16_t* vsbase = a.v_scale + (int64_t)unit * g.C;

  // Token of column col of Key MFMA gg.
  auto tok = [&](int gg) { return 16 * (col / 4) + F16::field(4 * (col % 4) + gg); };
  // Byte of a Key word: chunk (r0 / 16) of token tok[gg], byte r0 % 16 in it,
  // r0 = 8 BITS mk + 2 BITS q4.
  auto koff = [&](int gg, int mk) {
    const int r0 = 8 * BITS * mk + 2 * BITS * q4;
    return (r0 / 16) * 1024 + r0 % 16 + tok(gg) * 16;
  };
  const int voff = col * (8 * BITS) + 2 * BITS * q4;

  // ---- the query: one wave's loads, issued first ----
  uint4 qraw[QPL];
  {
    const uint4* qg = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + (int64_t)unit * GQA * D);
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
      const int i = lane + k * kWave;
      qraw[k] = qg[i < NQ16 ? i : 0];
    }
  }

  // A tile's registers: Key and Value code words, the Key-scale row of its
  // segment (channels RPL * lane .. + RPL - 1, one load) and the Value scales
  // of the 8 (int4) or 16 (int2) consecutive tokens around the lane's four
  // tokens tok[0..3] (one or two 16-byte loads), kept raw: widening them at
  // load time would make the wave wait for the loads it has just issued.
  constexpr int NVS = BITS == 4 ? 1 : 2;
  struct TileRegs {
    raw_t kw[4][MK];
    raw_t vw[NV];
    uint4 vs[NVS];
    uint32_t ks;
    bool new_seg;
  };
  static_assert(RPL <= 2, "two Key-scale slots per lane at most");
  // Every load of a tile or window chunk is issued unconditionally through a
  // buffer resource; the loads of an item past the wave's run get a
  // zero-size resource, which the hardware drops (no memory access, zero
  // data).  The number of loads in flight is then the same on every path and
  // the compiler waits for exactly the ones an item needs.
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, (int)g.code_stream, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, (int)g.code_stream, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rKS = __builtin_amdgcn_make_buffer_rsrc((void*)ksbase, (short)0, g.max_seg * D * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rVS = __builtin_amdgcn_make_buffer_rsrc((void*)vsbase, (short)0, g.C * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rNull = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, 0, kRsrcWord3);
  // Paged caches: lane i holds the page of the run's tile w_begin + i (a run
  // is at most 64 tiles: the launch keeps per_split <= 4 * 64), loaded right
  // after the query; a tile's loads go through a resource over its page's
  // part for this KV head: Key codes at 0, Value codes at 64 W, Value scales
  // at 128 W, the segment's Key-scale row at 128 W + 128.
  constexpr int kPgV = kTile * W, kPgVS = 2 * kTile * W, kPgKS = 2 * kTile * W + 2 * kTile;
  int tpages = 0;
  if constexpr (kPaged) {
    const int ti = w_begin + lane < pd.stride ? w_begin + lane : pd.stride - 1;
    tpages = pd.table[(int64_t)(unit / g.H) * pd.stride + ti];
  }
  // Decode step: the first appended token's key (channels lane + kWave j)
  // and value (this thread's output channels in the merge) go out with the
  // query, so the last workgroup's merge does not wait for them.
  FirstNew<D, GQA> fnew;
  if (nn > 0) {
    const uint16_t* kn = a.k_new + (int64_t)unit * a.n_new * D;
    const uint16_t* vn = a.v_new + (int64_t)unit * a.n_new * D;
#pragma unroll
    for (int j = 0; j < FirstNew<D, GQA>::kKeys; ++j) {
      const int c = lane + j * kWave;
      fnew.kr[j] = kn[c < D ? c : 0];
    }
    fnew.vr = *reinterpret_cast<const uint2*>(vn + merge_c0<D, GQA>(tid));
  }
  __builtin_amdgcn_sched_barrier(0);          // the query (and page numbers) go out first
  auto page_rsrc = [&](int tile_, bool ok) -> __amdgpu_buffer_rsrc_t {
    if constexpr (kPaged) {
      int k = __builtin_amdgcn_readfirstlane(tile_ - w_begin);
      k = k < 0 ? 0 : (k > kWave - 1 ? kWave - 1 : k);
      int64_t pg = __builtin_amdgcn_readlane(tpages, k);
      pg = pg < 0 ? 0 : (pg >= pd.n_pages ? pd.n_pages - 1 : pg);    // clamped into the pool
      const uint8_t* base = pd.pool + pg * pd.page_bytes + (int64_t)(unit % g.H) * pd.head_bytes;
      return ok ? __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, pd.head_bytes, kRsrcWord3) : rNull;
    } else {
      return rNull;
    }
  };
  // Per-lane byte offsets inside a tile (loop invariant); the tile's own
  // offset travels in the scalar offset of each load.
  int koffv[4];
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) koffv[gg] = koff(gg, 0);
  // The lane's tokens tok[gg]: int4 16 (col / 4) + 8 (m / 2) + m % 2 + 2 gg,
  // int2 16 (col / 4) + 4 gg + m (m = col % 4): Value scales loaded from the
  // aligned run of 8 (int4) or 16 (int2) tokens that starts at vsoff / 2.
  const int m4 = col % 4;
  const int vsoff = BITS == 4 ? (16 * (col / 4) + 8 * (m4 / 2)) * 2 : 16 * (col / 4) * 2;
  const int ksoff = RPL * lane * 2;
  constexpr int kMkBytes = ((8 * BITS) / 16) * 1024;   // koff(gg, mk) - koff(gg, 0) per mk
  auto ld_raw = [&](__amdgpu_buffer_rsrc_t rs, int voff_, int soff) -> raw_t {
    if constexpr (sizeof(raw_t) == 8)
      return __builtin_bit_cast(raw_t, __builtin_amdgcn_raw_buffer_load_b64(rs, voff_, soff, 0));
    else
      return __builtin_bit_cast(raw_t, __builtin_amdgcn_raw_buffer_load_b32(rs, voff_, soff, 0));
  };
  // Tiles are loaded in order: the segment of the next one is tracked with a
  // counter (no division per tile).
  int ld_seg = w_begin / a.tiles_per_seg;
  int ld_pos = w_begin - ld_seg * a.tiles_per_seg;
  auto load_tile = [&](int tile_, TileRegs& r) {
    // Loop counters are wave-uniform; taking them through readfirstlane first
    // keeps the whole offset computation in scalar registers.
    const int tile = __builtin_amdgcn_readfirstlane(tile_);
    const int seg = __builtin_amdgcn_readfirstlane(ld_seg);
    const bool ok = tile < q_end;              // past the run: a zero-size resource, nothing read
    r.new_seg = tile == w_begin || ld_pos == 0;
    __amdgpu_buffer_rsrc_t rks, rvs, rk, rv;
    int kso, vso, to, vto;
    if constexpr (kPaged) {
      rks = rvs = rk = rv = page_rsrc(tile, ok);
      kso = kPgKS;
      vso = kPgVS;
      to = 0;
      vto = kPgV;
    } else {
      rks = ok ? rKS : rNull;
      rvs = ok ? rVS : rNull;
      rk = ok ? rK : rNull;
      rv = ok ? rV : rNull;
      kso = ok ? seg * (D * 2) : 0;
      vso = ok ? tile * (kTile * 2) : 0;
      to = ok ? tile * (kTile * W) : 0;
      vto = to;
    }
    if constexpr (RPL == 2) r.ks = __builtin_amdgcn_raw_buffer_load_b32(rks, ksoff, kso, 0);
    else r.ks = __builtin_amdgcn_raw_buffer_load_b16(rks, ksoff, kso, 0);
#pragma unroll
    for (int k = 0; k < NVS; ++k)
      r.vs[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rvs, vsoff + 16 * k, vso, 0));
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
#pragma unroll
      for (int mk = 0; mk < MK; ++mk) r.kw[gg][mk] = ld_raw(rk, koffv[gg] + mk * kMkBytes, to);
#pragma unroll
    for (int n = 0; n < NV; ++n) r.vw[n] = ld_raw(rv, voff + n * 16 * (8 * BITS), vto);
    if (++ld_pos == a.tiles_per_seg) {
      ld_pos = 0;
      ++ld_seg;
    }
  };
  // Window chunks: this unit's ring through buffer resources (byte offsets
  // below ring * D * 2 < 2^29); a chunk past the wave's run reads nothing.
  const uint16_t* ring_k = static_cast<const uint16_t*>(a.k_tail) + (int64_t)unit * g.ring * D;
  const uint16_t* ring_v = static_cast<const uint16_t*>(a.v_tail) + (int64_t)unit * g.ring * D;
  const __amdgpu_buffer_rsrc_t rRK = __builtin_amdgcn_make_buffer_rsrc((void*)ring_k, (short)0, g.ring * D * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rRV = __builtin_amdgcn_make_buffer_rsrc((void*)ring_v, (short)0, g.ring * D * 2, kRsrcWord3);
  const int vlane = TCPL * lane * 2;          // this lane's Value channels in a ring row (bytes)
  auto chunk_load = [&](int chunk_, ChunkRegs<D>& r) {
    const int chunk = __builtin_amdgcn_readfirstlane(chunk_);
    const bool ok = chunk < ww.c1;            // past the run: a zero-size resource, nothing read
    const __amdgpu_buffer_rsrc_t rk = ok ? rRK : rNull;
    const __amdgpu_buffer_rsrc_t rv = ok ? rRV : rNull;
    const int tt0 = chunk * kTailChunk;
    const int nv = a.nt - tt0 < kTailChunk ? a.nt - tt0 : kTailChunk;
    r.nvalid = nv;
    const int kro = (tail_slot(a, tt0 + (col < nv ? col : 0)) * D + 8 * q4) * 2;
#pragma unroll
    for (int mk = 0; mk < D / 32; ++mk)
      r.k[mk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, kro + 64 * mk, 0, 0));
#pragma unroll
    for (int t = 0; t < kTailChunk; ++t) {
      const int row = __builtin_amdgcn_readfirstlane(tail_slot(a, tt0 + (t < nv ? t : 0)) * D * 2);
      if constexpr (TCPL == 2) r.v[t] = __builtin_amdgcn_raw_buffer_load_b32(rv, vlane, row, 0);
      else r.v[t] = __builtin_amdgcn_raw_buffer_load_b16(rv, vlane, row, 0);
    }
  };

  __builtin_amdgcn_sched_barrier(0);        // the tile loads stay behind the query's wait

  // The run's first window chunk and first tile, before the query's wait;
  // the second tile after it.  Every load of a run of up to two tiles and a
  // chunk (the Llama-3-8B shape at 4096 tokens) goes out before the wave
  // waits for tile data.  The chunk goes first so that the wait for a tile is
  // the same on every pass of the loop below (the loads of the one tile after
  // it in flight).
  ChunkRegs<D> cr;
  chunk_load(ww.c0, cr);
  TileRegs buf0, buf1;
  load_tile(w_begin, buf0);
  __builtin_amdgcn_sched_barrier(0);
  // The query lands: sigma log2(e) q into this wave's LDS rows (fp32, and
  // the bf16 high / low pair of the chunk scores).  The run's first window
  // chunk and first tile are already on the way (issued above, after the
  // query, so the wait below is for the query alone): the query still lands
  // early, and the memory system is busy from the start.  Issuing the second
  // tile before this wait as well measured no better; with every load of the
  // run ahead of it, the query landed only as the whole burst drained.
#pragma unroll
  for (int k = 0; k < QPL; ++k) {
    const int i = lane + k * kWave;
    if (i < NQ16) {
      const uint32_t w4[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 8 * i + j, h = e / D, c = e % D;
        const float x = bf16_bits_to_f32((w4[j / 2] >> (16 * (j % 2))) & 0xFFFFu) * a.qscale;
        qsC[wave][h][c] = x;
        const uint32_t hb = bf16_rne(x);
        qsHL[wave][0][h][c] = (uint16_t)hb;
        qsHL[wave][1][h][c] = (uint16_t)bf16_rne(x - bf16_bits_to_f32(hb));
      }
    }
  }
  wave_lds_sync();

  __builtin_amdgcn_sched_barrier(0);
  load_tile(w_begin + 1, buf1);
  __builtin_amdgcn_sched_barrier(0);
  // ... and its logits (head wave + kWaves i) while the tiles are on the way
  if (nn > 0) {
#pragma unroll
    for (int i = 0; i < FirstNew<D, GQA>::kHeads; ++i) {
      const int hh = wave + kWaves * i;
      float x = 0.0f;
      if (hh < GQA) {
#pragma unroll
        for (int j = 0; j < FirstNew<D, GQA>::kKeys; ++j) {
          const int c = lane + j * kWave;
          if (c < D) x = fmaf(qsC[wave][hh][c], bf16_bits_to_f32(fnew.kr[j]), x);
        }
      }
      fnew.lg[i] = wave_sum(x);
    }
  }

  // Online-softmax state: head 4 hg + q4 of this lane's row quad.
  float m[HG], lsum[HG], inv[HG], mq[HG];
  float acc_f[HG][NV];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    m[hg] = -INFINITY;
    lsum[hg] = 0.0f;
    inv[hg] = 0.0f;
#pragma unroll
    for (int n = 0; n < NV; ++n) acc_f[hg][n] = 0.0f;
    // max |q| of head 4 hg + q4 (bounds the fixed-point query with max 1/kscale)
    const int h = 4 * hg + q4;
    float mx = 0.0f;
    if (h < GQA) {
#pragma unroll
      for (int k = 0; k < D / 16; ++k) mx = fmaxf(mx, fabsf(qsC[wave][h][col * (D / 16) + k]));
    }
    mq[hg] = row16_max(mx);
  }

  // Key operands of a segment: digit d of round(F a[head][c]) in row 4 h + d.
  // Lane items: head 4 hg + q4, k-group (lane / 4) % 4, dword lane % 4, both halves mk.
  i4_t qop[HG][MK];
  auto build_key_operands = [&](const TileRegs& r) {
    float rkmax = 0.0f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const float rk = fast_rcp(fmaxf(half_bits_to_f32((uint16_t)(r.ks >> (16 * i))), g.eps));
      const int c = RPL * lane + i;
      rkP[wave][(c & ~15) + F16::slot(c & 15)] = rk;
      rkmax = fmaxf(rkmax, rk);
    }
    rkmax = wave_max(rkmax);
    wave_lds_sync();
    const int kgi = (lane / 4) % 4, qi = lane % 4;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      const int h = 4 * hg + q4;
      // F only sets the fixed-point scale: the hardware reciprocal (about one
      // ulp) keeps |round(a F)| below 2^20 thanks to the headroom in kFixQ,
      // and inv undoes exactly the F used, up to one more ulp.
      const float F = kFixQ * fast_rcp(fmaxf(mq[hg] * rkmax, 1e-30f));   // all-zero query: any finite F
      inv[hg] = h < GQA ? fast_rcp(F * F16::kMul) : 0.0f;
      if (h < GQA) {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk) {
          const int p0 = 64 * mk + 16 * kgi + 4 * qi;
          const float4 rv = *reinterpret_cast<const float4*>(&rkP[wave][p0]);
          const uint32_t u[4] = {fixed_biased(qsC[wave][h][chan(p0)] * rv.x, F),
                                 fixed_biased(qsC[wave][h][chan(p0 + 1)] * rv.y, F),
                                 fixed_biased(qsC[wave][h][chan(p0 + 2)] * rv.z, F),
                                 fixed_biased(qsC[wave][h][chan(p0 + 3)] * rv.w, F)};
          uint32_t* dst = &qD[wave][hg][mk][4 * q4][4 * kgi + qi];
          // balanced digits: (u & 127) - 64, ((u >> 7) & 127) - 64, (u >> 14) - 64
          dst[0 * kRowPad] = pack_bytes((u[0] >> 14) - 64u, (u[1] >> 14) - 64u, (u[2] >> 14) - 64u,
                                        (u[3] >> 14) - 64u);
          dst[1 * kRowPad] = pack_bytes(((u[0] >> 7) & 127u) - 64u, ((u[1] >> 7) & 127u) - 64u,
                                        ((u[2] >> 7) & 127u) - 64u, ((u[3] >> 7) & 127u) - 64u);
          dst[2 * kRowPad] = pack_bytes((u[0] & 127u) - 64u, (u[1] & 127u) - 64u, (u[2] & 127u) - 64u,
                                        (u[3] & 127u) - 64u);
        }
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int mk = 0; mk < MK; ++mk) qop[hg][mk] = *reinterpret_cast<const i4_t*>(&qD[wave][hg][mk][col][4 * q4]);
  };

  // One quantized tile.  Value weights: P = Fv p / vscale as a 21-bit
  // integer, with Fv = kFixP / max(1 / vscale) over the tile's 64 tokens
  // (every row of 16 lanes holds all of them), so p <= 1 keeps P < 2^21; the
  // tile's digit sums are scaled back by 1 / Fv as they are folded into the
  // fp32 accumulator (acc = acc alpha + sums / Fv): nothing integer is carried
  // from tile to tile.
  auto compute_tile = [&](const TileRegs& r) {
    float x[HG][4];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      i4_t sk[HG];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) sk[hg] = i4_t{0, 0, 0, 0};
#pragma unroll
      for (int mk = 0; mk < MK; ++mk) {
        const i4_t kb = F16::unpack(r.kw[gg][mk]);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) sk[hg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qop[hg][mk], kb, sk[hg], 0, 0, 0);
      }
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) x[hg][gg] = digits_value(sk[hg]) * inv[hg];
    }
    float rv[4], rmax = 0.0f;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      uint32_t w;
      if constexpr (BITS == 4) {
        // token 2 gg + m % 2 of the run: dword gg, half m % 2
        const uint32_t d[4] = {r.vs[0].x, r.vs[0].y, r.vs[0].z, r.vs[0].w};
        w = d[gg] >> (16 * (m4 % 2));
      } else {
        // token 4 gg + m of the run: load gg / 2, dword 2 (gg % 2) + m / 2, half m % 2
        const uint4 v = r.vs[gg / 2];
        const uint32_t lo = gg % 2 ? v.z : v.x, hi = gg % 2 ? v.w : v.y;
        w = (m4 / 2 ? hi : lo) >> (16 * (m4 % 2));
      }
      rv[gg] = fast_rcp(fmaxf(half_bits_to_f32((uint16_t)w), g.eps));
      rmax = fmaxf(rmax, rv[gg]);
    }
    rmax = row16_max(rmax);
    const float fv = kFixP * fast_rcp(rmax);
    const float back = rmax * (1.0f / kFixP);              // 1 / Fv
    float alpha[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      const float tm = row16_max(fmaxf(fmaxf(x[hg][0], x[hg][1]), fmaxf(x[hg][2], x[hg][3])));
      const float mn = fmaxf(m[hg], tm);     // finite: every token of a tile is cached
      alpha[hg] = fast_exp2(m[hg] - mn);     // exp2(-inf) = 0 on the first tile
      m[hg] = mn;
      lsum[hg] *= alpha[hg];
    }
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) rv[gg] *= fv;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      uint32_t P[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const float p = fast_exp2(x[hg][gg] - m[hg]);
        lsum[hg] += p;
        P[gg] = (uint32_t)(p * rv[gg]);
      }
      uint32_t* dst = &pD[wave][hg][4 * q4][col];      // k-group col / 4, dword col % 4
      dst[0 * kRowPad] = pack_bytes(P[0] >> 14, P[1] >> 14, P[2] >> 14, P[3] >> 14);
      dst[1 * kRowPad] = pack_bytes((P[0] >> 7) & 127u, (P[1] >> 7) & 127u, (P[2] >> 7) & 127u, (P[3] >> 7) & 127u);
      dst[2 * kRowPad] = pack_bytes(P[0] & 127u, P[1] & 127u, P[2] & 127u, P[3] & 127u);
    }
    wave_lds_sync();
    i4_t pop[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) pop[hg] = *reinterpret_cast<const i4_t*>(&pD[wave][hg][col][4 * q4]);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const i4_t vb = F16::unpack(r.vw[n]);
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const i4_t d = __builtin_amdgcn_mfma_i32_16x16x64_i8(pop[hg], vb, i4_t{0, 0, 0, 0}, 0, 0, 0);
        acc_f[hg][n] = fmaf(digits_value(d), back, acc_f[hg][n] * alpha[hg]);
      }
    }
    wave_lds_sync();      // pD is rewritten by the next tile
  };

  // Window chunks (bf16).  Scores on the matrix cores: A = the query in two
  // bf16 rows per head (4 h: high part, 4 h + 1: the rounding remainder,
  // about 16 more bits), B = the chunk's Keys, so lane (q4, col) receives
  // head q4's score for token col -- the layout of the tile scores.
  // Weighted Values on the vector ALUs, each lane owning TCPL channels of
  // every head.  The chunks keep a softmax state of their own (mC, lC,
  // acc_tail), merged with the tiles' once at the end, so that the first
  // chunk can be computed before the tiles.
  float acc_tail[TCPL][GQA], mC[HG], lC[HG];
#pragma unroll
  for (int h = 0; h < GQA; ++h)
#pragma unroll
    for (int k = 0; k < TCPL; ++k) acc_tail[k][h] = 0.0f;
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    mC[hg] = -INFINITY;
    lC[hg] = 0.0f;
  }
  auto load_qa = [&](bf8_t (&qa)[HG][D / 32]) {
    const int hq = col / 4, part = col % 4;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      const int h = 4 * hg + hq;
#pragma unroll
      for (int mk = 0; mk < D / 32; ++mk) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (h < GQA && part < 2) w = *reinterpret_cast<const uint4*>(&qsHL[wave][part][h][32 * mk + 8 * q4]);
        qa[hg][mk] = __builtin_bit_cast(bf8_t, w);
      }
    }
  };
  auto compute_chunk = [&](const bf8_t (&qa)[HG][D / 32]) {
    float al_u[GQA];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      f4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int mk = 0; mk < D / 32; ++mk)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hg][mk], __builtin_bit_cast(bf8_t, cr.k[mk]), sc, 0, 0, 0);
      const float xs = col < cr.nvalid ? sc[0] + sc[1] : -INFINITY;
      const float mn = fmaxf(mC[hg], row16_max(xs));    // finite: a chunk has a valid token
      const float al = fast_exp2(mC[hg] - mn);           // exp2(-inf) = 0 before the first token
      mC[hg] = mn;
      const float pr = fast_exp2(xs - mn);               // 0 for padding tokens
      lC[hg] = lC[hg] * al + pr;
      if (4 * hg + q4 < GQA) pw[wave][col][4 * hg + q4] = pr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * hg + i < GQA) al_u[4 * hg + i] = lane_value(al, 16 * i);
    }
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < kTailChunk; ++t) {
      float v[TCPL];
      v[0] = bf16_lo(cr.v[t]);
      if constexpr (TCPL == 2) v[1] = bf16_hi(cr.v[t]);
#pragma unroll
      for (int h = 0; h < GQA; ++h) {
        const float pt = pw[wave][t][h];
#pragma unroll
        for (int k = 0; k < TCPL; ++k)
          acc_tail[k][h] = fmaf(pt, v[k], t == 0 ? acc_tail[k][h] * al_u[h] : acc_tail[k][h]);
      }
    }
    wave_lds_sync();      // pw is rewritten by the next chunk
  };

  // The run's first window chunk comes before its tiles: its loads went out
  // first, so it is computed while the tiles' data is still on the way.
  if (ww.c0 < ww.c1) {
    bf8_t qa[HG][D / 32];
    load_qa(qa);
    compute_chunk(qa);
  }

  // Quantized tiles through a ring of two: a tile is computed, then its
  // registers take the loads of the tile two ahead (issued unconditionally:
  // past the run they read nothing), so the next tile is in flight while one
  // is computed.
  for (int tile = w_begin; tile < q_end; tile += 2) {
    if (buf0.new_seg) build_key_operands(buf0);
    compute_tile(buf0);
    load_tile(tile + 2, buf0);
    if (tile + 1 >= q_end) break;
    if (buf1.new_seg) build_key_operands(buf1);
    compute_tile(buf1);
    load_tile(tile + 3, buf1);
  }

  // Further window chunks of the run (a run holds more than one only when a
  // split has more chunks than waves), after the tiles.
  if (ww.c0 + 1 < ww.c1) {
    bf8_t qa[HG][D / 32];
    load_qa(qa);
    for (int chunk = ww.c0 + 1; chunk < ww.c1; ++chunk) {
      chunk_load(chunk, cr);
      compute_chunk(qa);
    }
  }
  // Merge the chunks' softmax state into the tiles': both scaled to the
  // common maximum (a wave with neither tiles nor chunks keeps -inf and 0).
  {
    float aC[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      const float mx = fmaxf(m[hg], mC[hg]);
      const float aT = mx == -INFINITY ? 0.0f : fast_exp2(m[hg] - mx);
      aC[hg] = mx == -INFINITY ? 0.0f : fast_exp2(mC[hg] - mx);
      m[hg] = mx;
      lsum[hg] = lsum[hg] * aT + lC[hg] * aC[hg];
#pragma unroll
      for (int n = 0; n < NV; ++n) acc_f[hg][n] *= aT;
    }
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * hg + i;
        if (h < GQA) {
          const float a = lane_value(aC[hg], 16 * i);
#pragma unroll
          for (int k = 0; k < TCPL; ++k) acc_tail[k][h] *= a;
        }
      }
  }

  // Per-head state as wave-uniform values (head 4 hg + i lives in lanes 16 i..).
  float mu[GQA], lu[GQA];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const float ls = row16_sum(lsum[hg]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * hg + i;
      if (h < GQA) {
        mu[h] = lane_value(m[hg], 16 * i);
        lu[h] = lane_value(ls, 16 * i);
      }
    }
  }

  // ---- wave result into red[wave][head][channel] ----
  constexpr float kOut = 1.0f / F16::kMul;
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const int h = 4 * hg + q4;
    if (h < GQA) {
#pragma unroll
      for (int n = 0; n < NV; ++n) red[wave][h][16 * n + col] = acc_f[hg][n] * kOut;
    }
  }
  wave_lds_sync();
  if (TailMap<D>::owns(lane)) {
#pragma unroll
    for (int k = 0; k < TCPL; ++k)
#pragma unroll
      for (int h = 0; h < GQA; ++h) red[wave][h][lane * TCPL + k] += acc_tail[k][h];
  }
  finish_unit<D, GQA>(a, unit, split, S, nn, a.n_new, slot0, red, wml, mu, lu,
                      [&](int h, int c) { return qsC[0][h][c]; }, fnew);
}

template <int D, int BITS, int GQA>
void launch(const DecodeArgs& a, const PagedDecode* pd, hipStream_t s) {
  dim3 grid(a.splits, a.g.B * a.g.H);
  if (pd) {
    grid = dim3(pd->wg_end[a.g.B - 1], 1);   // the workgroups with work, 1-D
    // Matrix-core kernel: a wave's run of tiles must fit its 64-lane page
    // list.  A split holds at most per_split + 2 items (rounding of tiles and
    // chunks), a wave at most a quarter of that, rounded up.
    bool i8 = false;
    if constexpr ((BITS == 4 || BITS == 2) && D >= 64)
      i8 = a.g.dtype == KVQ_BF16 && a.g.kernel == KVQ_KERNEL_AUTO && pd->per_split + 2 <= kWaves * kWave;
    if (i8) {
      if constexpr ((BITS == 4 || BITS == 2) && D >= 64)
        hipLaunchKernelGGL((decode_i8_kernel<D, BITS, GQA, PagedDecode>), grid, dim3(kThreads), 0, s, a, *pd);
    } else {
      hipLaunchKernelGGL((decode_kernel<D, BITS, GQA, true>), grid, dim3(kThreads), 0, s, a, *pd);
    }
  } else if (a.g.scheme == KVQ_SAME_AXIS) {
    if constexpr (D % kRunChannels == 0)
      hipLaunchKernelGGL((decode_kernel<D, BITS, GQA, false, true>), grid, dim3(kThreads), 0, s, a, PagedDecode{});
  } else if constexpr ((BITS == 4 || BITS == 2) && D >= 64) {
    // The matrix-core kernel addresses a unit's streams with 32-bit buffer offsets.
    const bool offsets32 = a.g.code_stream < (int64_t(1) << 31) &&
                           (int64_t)a.g.max_seg * a.g.D * 2 < (int64_t(1) << 31);
    if (a.g.G > 0 && a.g.dtype == KVQ_BF16 && a.g.kernel == KVQ_KERNEL_AUTO && a.tiles_q > 0 && offsets32)
      hipLaunchKernelGGL((decode_i8_kernel<D, BITS, GQA>), grid, dim3(kThreads), 0, s, a, NoPaging{});
    else
      hipLaunchKernelGGL((decode_kernel<D, BITS, GQA>), grid, dim3(kThreads), 0, s, a, PagedDecode{});
  } else {
    hipLaunchKernelGGL((decode_kernel<D, BITS, GQA>), grid, dim3(kThreads), 0, s, a, PagedDecode{});
  }
  if (!a.last_merge && (a.splits > 1 || a.n_new > 0)) {
    // More splits than the in-kernel merge takes: a second kernel merges them,
    // one workgroup per (batch, KV head, query head), 64 partials per round trip.
    const dim3 mgrid(a.g.B * a.g.H, GQA);
    if (pd && a.n_new > 0)
      hipLaunchKernelGGL((merge_kernel<D, GQA, 64, true, PagedDecode>), mgrid, dim3(D), 0, s, a, *pd);
    else if (pd)
      hipLaunchKernelGGL((merge_kernel<D, GQA, 64, false, PagedDecode>), mgrid, dim3(D), 0, s, a, *pd);
    else if (a.n_new > 0)
      hipLaunchKernelGGL((merge_kernel<D, GQA, 64, true>), mgrid, dim3(D), 0, s, a, NoPaging{});
    else
      hipLaunchKernelGGL((merge_kernel<D, GQA, 64, false>), mgrid, dim3(D), 0, s, a, NoPaging{});
  }
}

template <int D, int BITS>
bool dispatch_gqa(const DecodeArgs& a, int gqa, const PagedDecode* pd, hipStream_t s) {
  switch (gqa) {
    case 1: launch<D, BITS, 1>(a, pd, s); return true;
    case 2: launch<D, BITS, 2>(a, pd, s); return true;
    case 4: launch<D, BITS, 4>(a, pd, s); return true;
    case 8: launch<D, BITS, 8>(a, pd, s); return true;
  }
  return false;
}

bool dispatch(const DecodeArgs& a, int gqa, hipStream_t s, const PagedDecode* pd = nullptr) {
  const int D = a.g.D, bits = a.g.bits;
  if (D == 16 && bits == 8) return dispatch_gqa<16, 8>(a, gqa, pd, s);
  if (D == 32 && bits == 8) return dispatch_gqa<32, 8>(a, gqa, pd, s);
  if (D == 32 && bits == 4) return dispatch_gqa<32, 4>(a, gqa, pd, s);
  if (D == 64 && bits == 8) return dispatch_gqa<64, 8>(a, gqa, pd, s);
  if (D == 64 && bits == 4) return dispatch_gqa<64, 4>(a, gqa, pd, s);
  if (D == 64 && bits == 2) return dispatch_gqa<64, 2>(a, gqa, pd, s);
  if (D == 128 && bits == 8) return dispatch_gqa<128, 8>(a, gqa, pd, s);
  if (D == 128 && bits == 4) return dispatch_gqa<128, 4>(a, gqa, pd, s);
  if (D == 128 && bits == 2) return dispatch_gqa<128, 2>(a, gqa, pd, s);
  return false;
}

}  // namespace

int auto_splits(int units, int items) {
  // Aim for one workgroup per compute unit (256 CUs): a wave then has a run
  // of several tiles, whose loads stream through the tile ring while earlier
  // tiles are computed (at two workgroups per unit the Llama-3-8B call is a
  // single burst of loads whose compute all comes after it: 16.2 us against
  // 14.9 us).  At least four work items per workgroup.
  int s = (256 + units - 1) / units;
  const int max_by_items = items / 4 > 0 ? items / 4 : 1;
  if (s > max_by_items) s = max_by_items;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : s;
}

}  // namespace kvq

using namespace kvq;

namespace kvq {
kvq_status plan_append(const Geom& g, const kvq_state* st, int64_t n_new, kvq_state* next);

namespace {

// Preconditions of attention over a cache in state `st` (every one checked
// before anything is enqueued); sets the query-group size.
kvq_status check_decode(const Geom& g, const kvq_state* st, const kvq_cache* cache, const void* q,
                        int32_t q_heads, float softmax_scale, int32_t num_splits, const float* out,
                        const void* workspace, size_t workspace_size, int* gqa) {
  if (!st || !cache || !q || !out) return KVQ_EINVAL;
  if (q_heads < 1 || q_heads % g.H != 0) return KVQ_EINVAL;
  *gqa = q_heads / g.H;
  if (*gqa != 1 && *gqa != 2 && *gqa != 4 && *gqa != 8) return KVQ_EINVAL;
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
  return KVQ_OK;
}

// Kernel arguments of attention over the cache in state `st`.
DecodeArgs decode_args(const Geom& g, const kvq_state* st, const kvq_cache* cache, const void* q,
                       float softmax_scale, int32_t num_splits, float* out, void* workspace) {
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
  a.ctr = static_cast<uint32_t*>(workspace);
  a.part = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + workspace_counter_bytes(g, 1))
                     : nullptr;
  a.tiles_q = (a.nq + kTile - 1) / kTile;
  a.items = a.tiles_q + (a.nt + kTailChunk - 1) / kTailChunk;
  const int units = g.B * g.H;
  a.splits = num_splits > 0 ? num_splits : auto_splits(units, a.items);
  a.tq_div = a.tiles_q / a.splits;
  a.tq_mod = a.tiles_q % a.splits;
  a.ch_div = (a.items - a.tiles_q) / a.splits;
  a.ch_mod = (a.items - a.tiles_q) % a.splits;
  a.last_merge = a.splits <= kLastMergeSplits;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.ring_k = nullptr;
  a.ring_v = nullptr;
  a.n_new = 0;
  a.new_slot0 = 0;
  return a;
}

}  // namespace
}  // namespace kvq

extern "C" kvq_status kvq_decode_attn(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                                      const void* q, int32_t q_heads, float softmax_scale,
                                      int32_t num_splits, float* out, void* workspace,
                                      size_t workspace_size, void* stream) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  int gqa = 0;
  s = check_decode(g, st, cache, q, q_heads, softmax_scale, num_splits, out, workspace, workspace_size, &gqa);
  if (s != KVQ_OK) return s;
  const DecodeArgs a = decode_args(g, st, cache, q, softmax_scale, num_splits, out, workspace);
  clear_stale_hip_error();
  if (!dispatch(a, gqa, static_cast<hipStream_t>(stream))) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}

// ---- decode attention without a caller workspace ---------------------------
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the split partials and arrival
// counters live in one file-scope device array of kScratchBytes per GPU,
// held until the process ends.  In host code the array's name only stands in
// for the symbol: its device address comes from hipGetSymbolAddress, taken
// once per device (with that device current) on the first call there.
namespace kvq {
namespace {
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex scratch_mu;
void* scratch_ptr[kMaxScratchDevices] = {};

// The scratch array's device address on the current device.
kvq_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return KVQ_EDEVICE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_EDEVICE;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return KVQ_OK;
}
}  // namespace
}  // namespace kvq

extern "C" kvq_status kvq_decode_attn_noalloc(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                                              const void* q, int32_t q_heads, float softmax_scale,
                                              int32_t num_splits, float* out, void* stream) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  int gqa = 0;
  // every check of kvq_decode_attn except the caller's workspace (a dummy,
  // large enough, stands in for it until the real size is known)
  const void* dummy = cfg;
  s = check_decode(g, st, cache, q, q_heads, softmax_scale, num_splits, out, dummy, SIZE_MAX, &gqa);
  if (s != KVQ_OK) return s;
  DecodeArgs a = decode_args(g, st, cache, q, softmax_scale, num_splits, out, nullptr);
  // counters, then the partials of this call's split count
  const size_t need = workspace_counter_bytes(g, 1) +
                      (size_t)g.B * q_heads * a.splits * (g.D + 4) * sizeof(float);
  if (need > kScratchBytes) return KVQ_EWORKSPACE;
  void* ws = nullptr;
  s = scratch_on_current_device(&ws);
  if (s != KVQ_OK) return s;
  a.ctr = static_cast<uint32_t*>(ws);
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + workspace_counter_bytes(g, 1));
  clear_stale_hip_error();
  if (!dispatch(a, gqa, static_cast<hipStream_t>(stream))) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}

extern "C" kvq_status kvq_decode_step(const kvq_config* cfg, kvq_state* st, const kvq_cache* cache,
                                      const void* k_new, const void* v_new, int64_t n_new,
                                      const void* q, int32_t q_heads, float softmax_scale,
                                      int32_t num_splits, float* out, void* workspace,
                                      size_t workspace_size, void* stream) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!st) return KVQ_EINVAL;
  kvq_state next;
  s = plan_append(g, st, n_new, &next);
  if (s != KVQ_OK) return s;
  int gqa = 0;
  s = check_decode(g, &next, cache, q, q_heads, softmax_scale, num_splits, out, workspace, workspace_size, &gqa);
  if (s != KVQ_OK) return s;
  if (n_new > 0 && (!k_new || !v_new || !cache->k_codes || !cache->v_codes || !cache->k_scale ||
                    !cache->v_scale || !cache->k_tail || !cache->v_tail || (g.G == 0 && !cache->seg_index)))
    return KVQ_EINVAL;      // what kvq_append requires
  // One pass when nothing is flushed: attention over the cache as it was,
  // and the appended tokens folded in (and written to the window) by the
  // merge.  Otherwise the append, then attention.
  const bool fused = n_new >= 1 && n_new <= kMaxStepNew && next.flushed_last == 0 && st->total >= 1 &&
                     g.dtype == KVQ_BF16;
  if (!fused) {
    s = kvq_append(cfg, st, cache, k_new, v_new, n_new, stream);
    if (s != KVQ_OK) return s;
    return kvq_decode_attn(cfg, st, cache, q, q_heads, softmax_scale, num_splits, out, workspace,
                           workspace_size, stream);
  }
  DecodeArgs a = decode_args(g, st, cache, q, softmax_scale, num_splits, out, workspace);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.ring_k = static_cast<uint16_t*>(cache->k_tail);
  a.ring_v = static_cast<uint16_t*>(cache->v_tail);
  a.n_new = static_cast<int>(n_new);
  a.new_slot0 = static_cast<int>((st->quantized + st->tail) % g.ring);
  clear_stale_hip_error();
  if (!dispatch(a, gqa, static_cast<hipStream_t>(stream))) return KVQ_EINVAL;
  if (hipGetLastError() != hipSuccess) return KVQ_EDEVICE;
  *st = next;
  return KVQ_OK;
}

namespace kvq {
namespace {

// Checks of a paged decode over states st[0 .. batch) and its launch
// arguments: per-sequence lengths, work-sized splits, workgroup ranges.
kvq_status paged_decode_setup(const Geom& g, const kvq_state* st, const kvq_paged_cache* cache, const void* q,
                              int32_t q_heads, float softmax_scale, int32_t num_splits, float* out,
                              void* workspace, size_t workspace_size, DecodeArgs* a_out, PagedDecode* pd_out,
                              int* gqa_out) {
  if (!st || !cache || !q || !out) return KVQ_EINVAL;
  if (g.G <= 0 || g.B > kMaxPagedSeqs) return KVQ_EINVAL;
  if (!cache->pool || !cache->block_table || cache->n_pages < 1 || cache->table_stride < 1 ||
      (int64_t)cache->table_stride * kTile < g.C)
    return KVQ_EINVAL;
  if (q_heads < 1 || q_heads % g.H != 0) return KVQ_EINVAL;
  const int gqa = q_heads / g.H;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8) return KVQ_EINVAL;
  *gqa_out = gqa;
  if (!(softmax_scale == softmax_scale) || num_splits < 0 || num_splits > kMaxSplits) return KVQ_EINVAL;
  if (!workspace || workspace_size < workspace_bytes(g, q_heads, 1)) return KVQ_EWORKSPACE;
  PagedDecode& pd = *pd_out;
  pd.pool = static_cast<const uint8_t*>(cache->pool);
  pd.table = cache->block_table;
  pd.n_pages = cache->n_pages;
  pd.head_bytes = 2 * kTile * g.W + 2 * kTile + 2 * g.D;
  pd.page_bytes = static_cast<int64_t>(g.H) * pd.head_bytes;
  pd.stride = cache->table_stride;
  int max_items = 1;
  int64_t sum_items = 0;
  bool any_tail = false;
  for (int b = 0; b < kMaxPagedSeqs; ++b) {
    pd.nq[b] = pd.nt[b] = pd.n_new[b] = pd.new_slot0[b] = 0;
    if (b >= g.B) continue;
    const kvq_state& x = st[b];
    if (x.quantized < 0 || x.tail < 0 || x.total != x.quantized + x.tail || x.total < 1 || x.quantized > g.C ||
        x.tail > g.ring || x.quantized % g.G != 0)
      return KVQ_EINVAL;
    pd.nq[b] = static_cast<int>(x.quantized);
    pd.nt[b] = static_cast<int>(x.tail);
    any_tail |= x.tail > 0;
    const int items = static_cast<int>((x.quantized + kTile - 1) / kTile + (x.tail + kTailChunk - 1) / kTailChunk);
    max_items = items > max_items ? items : max_items;
    sum_items += (int64_t)items * g.H;
  }
  if (any_tail && (!cache->k_tail || !cache->v_tail)) return KVQ_EINVAL;
  // Uniform fields from the first sequence; the kernel replaces the
  // per-sequence ones.
  kvq_cache dense = {nullptr, nullptr, nullptr, nullptr, cache->k_tail, cache->v_tail, nullptr};
  DecodeArgs& a = *a_out;
  a = decode_args(g, &st[0], &dense, q, softmax_scale, num_splits, out, workspace);
  // Splits sized by work: every split of every sequence gets about per_split
  // items (window chunks count as tiles), so a long sequence takes more
  // splits instead of setting the time for the batch.  Auto: about one
  // workgroup per compute unit (as for uniform caches), at least four items
  // each.
  int per_split;
  if (num_splits > 0) {
    per_split = (max_items + num_splits - 1) / num_splits;
  } else {
    // Each sequence rounds its split count up: grow per_split until the
    // workgroups with work fit in one per compute unit (256).  Measured on
    // the ragged Llama-3-8B batch: 17.9 us per call against 19.3 us at two
    // per compute unit.
    const int64_t target = (sum_items + 256 - 1) / 256;
    per_split = static_cast<int>(target < 4 ? 4 : target);
    for (;;) {
      int64_t wgs = 0;
      for (int b = 0; b < g.B; ++b) {
        const int items = static_cast<int>((st[b].quantized + kTile - 1) / kTile + (st[b].tail + kTailChunk - 1) / kTailChunk);
        wgs += (int64_t)g.H * ((items + per_split - 1) / per_split);
      }
      if (wgs <= 256 || per_split >= max_items) break;
      ++per_split;
    }
  }
  if ((max_items + per_split - 1) / per_split > kMaxSplits) per_split = (max_items + kMaxSplits - 1) / kMaxSplits;
  pd.per_split = per_split;
  a.splits = (max_items + per_split - 1) / per_split;
  a.last_merge = a.splits <= kLastMergeSplits;
  int wg = 0;
  for (int b = 0; b < kMaxPagedSeqs; ++b) {
    if (b < g.B) {
      const int items = static_cast<int>((st[b].quantized + kTile - 1) / kTile + (st[b].tail + kTailChunk - 1) / kTailChunk);
      wg += g.H * ((items + per_split - 1) / per_split);
    }
    pd.wg_end[b] = wg;
  }
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

extern "C" kvq_status kvq_paged_decode_attn(const kvq_config* cfg, const kvq_state* st,
                                            const kvq_paged_cache* cache, const void* q, int32_t q_heads,
                                            float softmax_scale, int32_t num_splits, float* out,
                                            void* workspace, size_t workspace_size, void* stream) {
  Geom g;
  kvq_status s = validate_kivi_config(cfg, &g);
  if (s != KVQ_OK) return s;
  DecodeArgs a;
  PagedDecode pd;
  int gqa = 0;
  s = paged_decode_setup(g, st, cache, q, q_heads, softmax_scale, num_splits, out, workspace, workspace_size, &a,
                         &pd, &gqa);
  if (s != KVQ_OK) return s;
  clear_stale_hip_error();
  if (!dispatch(a, gqa, static_cast<hipStream_t>(stream), &pd)) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}

extern "C" kvq_status kvq_paged_decode_step(const kvq_config* cfg, kvq_state* st, const kvq_paged_cache* cache,
                                            const void* k_new, const void* v_new, const int64_t* n_new,
                                            const void* q, int32_t q_heads, float softmax_scale,
                                            int32_t num_splits, float* out, void* workspace,
                                            size_t workspace_size, void* stream) {
  Geom g;
  kvq_status s = validate_kivi_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!st || !cache || !n_new) return KVQ_EINVAL;
  if (g.G <= 0 || g.B > kMaxPagedSeqs) return KVQ_EINVAL;
  kvq_state next[kMaxPagedSeqs];
  int64_t max_n = 0;
  bool fused = g.dtype == KVQ_BF16;
  for (int b = 0; b < g.B; ++b) {
    s = plan_append(g, &st[b], n_new[b], &next[b]);
    if (s != KVQ_OK) return s;
    max_n = n_new[b] > max_n ? n_new[b] : max_n;
    fused = fused && n_new[b] <= kMaxStepNew && next[b].flushed_last == 0 && st[b].total >= 1;
  }
  fused = fused && max_n >= 1;
  // Every precondition of the attention over the post-append states, and
  // of the append, before anything is enqueued.
  DecodeArgs a;
  PagedDecode pd;
  int gqa = 0;
  s = paged_decode_setup(g, next, cache, q, q_heads, softmax_scale, num_splits, out, workspace, workspace_size, &a,
                         &pd, &gqa);
  if (s != KVQ_OK) return s;
  if (max_n > 0 && (!k_new || !v_new || !cache->k_tail || !cache->v_tail)) return KVQ_EINVAL;
  if (!fused) {
    s = kvq_paged_append(cfg, st, cache, k_new, v_new, n_new, stream);
    if (s != KVQ_OK) return s;
    return kvq_paged_decode_attn(cfg, st, cache, q, q_heads, softmax_scale, num_splits, out, workspace,
                                 workspace_size, stream);
  }
  // One pass: attention over the caches as they were (every sequence holds a
  // token, none flushes), the appended tokens folded in and written to the
  // windows by the merge.
  s = paged_decode_setup(g, st, cache, q, q_heads, softmax_scale, num_splits, out, workspace, workspace_size, &a,
                         &pd, &gqa);
  if (s != KVQ_OK) return s;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.ring_k = static_cast<uint16_t*>(cache->k_tail);
  a.ring_v = static_cast<uint16_t*>(cache->v_tail);
  a.n_new = static_cast<int>(max_n);
  a.new_slot0 = 0;
  for (int b = 0; b < g.B; ++b) {
    pd.n_new[b] = static_cast<int>(n_new[b]);
    pd.new_slot0[b] = static_cast<int>((st[b].quantized + st[b].tail) % g.ring);
  }
  clear_stale_hip_error();
  if (!dispatch(a, gqa, static_cast<hipStream_t>(stream), &pd)) return KVQ_EINVAL;
  if (hipGetLastError() != hipSuccess) return KVQ_EDEVICE;
  for (int b = 0; b < g.B; ++b) st[b] = next[b];
  return KVQ_OK;
}
