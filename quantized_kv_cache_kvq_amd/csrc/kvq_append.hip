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
//   1. flush_kernel  -- grid (segments * (1 + value workgroups), batch*heads).
//      Per segment one workgroup quantizes the Keys and a few quantize the
//      Values, one group of 64-token tiles each.  Tokens are read straight
//      from the old tail ring or from the new input (the "concatenation" is
//      virtual), as 16-byte pieces of their rows.
//   2. tail_kernel   -- copies the new tokens that stay in the window into
//      their ring slots.  It runs after the flush because a ring slot being
//      refilled may hold a token the flush is still reading.
#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kFlushThreads = 256;
constexpr int kKeyBatch = 8;      // 16-byte pieces per thread in flight in the Key pass

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
  int nq_slot_old;         // nq_old % ring: ring slot of the oldest tail token
  int64_t seg_base;        // id of the first segment written by this launch
  int64_t seg_len;         // tokens per segment (G, or the whole flush when G == 0)
  int pieces;              // 16-byte pieces per token row
  int v_tiles_per_wg;      // 64-token tiles per Value workgroup
  int v_wgs;               // Value workgroups per segment
  // Paged caches (pool != null): tile j's codes and scales go to page
  // table[j] of this sequence; grid.y runs over its KV heads.
  uint8_t* pool;
  const int32_t* table;    // the sequence's row of the block table
  int64_t n_pages;
  int64_t page_bytes;
  int head_bytes;          // 128 W + 128 + 2 D
  int seq;                 // sequence index (window and input rows: seq * H + head)
};

constexpr int kMaxPagedSeqs = 64;

// Paged appends flush every sequence in one launch (grid.z = sequence):
// each sequence's accounting before the append and its segment count.
struct PagedFlushSeqs {
  int nq_old[kMaxPagedSeqs];
  int nt_old[kMaxPagedSeqs];
  int seg_base[kMaxPagedSeqs];
  int nseg[kMaxPagedSeqs];       // segments this sequence flushes (0: its workgroups exit)
  int table_stride;              // block-table row length
};
struct NoPagedSeqs {};

// Base of KV head h's part of the page holding tile `tile` (paged caches);
// out-of-range page numbers are clamped into the pool.
__device__ __forceinline__ uint8_t* page_head(const FlushArgs& a, int h, int64_t tile) {
  int64_t pg = a.table[tile];
  pg = pg < 0 ? 0 : (pg >= a.n_pages ? a.n_pages - 1 : pg);
  return a.pool + pg * a.page_bytes + (int64_t)h * a.head_bytes;
}

// Row (head_dim elements) of absolute position p of the flushed range: the
// old tail ring if p was already cached, else the new input.
__device__ __forceinline__ const uint8_t* flush_row(const FlushArgs& a, bool key, int bh, int64_t p) {
  const Geom& g = a.g;
  const int row_bytes = a.pieces * 16;
  const int64_t old_end = a.nq_old + a.nt_old;
  if (p < old_end) {
    int slot = a.nq_slot_old + static_cast<int>(p - a.nq_old);   // p - nq_old < nt_old <= ring
    if (slot >= g.ring) slot -= g.ring;
    return static_cast<const uint8_t*>(key ? a.k_tail : a.v_tail) + ((int64_t)bh * g.ring + slot) * row_bytes;
  }
  return static_cast<const uint8_t*>(key ? a.k_new : a.v_new) + ((int64_t)bh * a.n_new + (p - old_end)) * row_bytes;
}

// Element e (0 .. 16/es - 1) of a 16-byte piece as fp32 (exact).
__device__ __forceinline__ float piece_elem(const uint4& w, int e, bool bf16) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  if (bf16) return bf16_bits_to_f32((v[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
  return __uint_as_float(v[e]);
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

// Max over aligned groups of `width` consecutive lanes (width a power of two
// <= 32, wave-uniform).  Every lane of a group ends with the group's max.
__device__ __forceinline__ float lane_group_max(float v, int width) {
  if (width >= 2) v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  if (width >= 4) v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  if (width >= 8) v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  if (width >= 16) v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  if (width >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}

// Keys of one segment.  Thread (row group rg, piece q) reads piece q of the
// tokens p0 + rg + rows*i.  The per-channel absmax is reduced over the
// lanes holding the same piece, then over the four waves in LDS; the codes
// of a piece (epp fields) are stored as one 1..8-byte word of its token's
// 16-byte chunk.
template <int BITS, bool kPaged>
__device__ __forceinline__ void flush_keys(const FlushArgs& a, int bh, int64_t seg, int64_t p0, int64_t p1,
                                           float (*red)[128], float* sc) {
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const Geom& g = a.g;
  const int D = g.D, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const bool bf16 = g.dtype == KVQ_BF16;
  const int epp = bf16 ? 8 : 4;                  // elements per 16-byte piece
  const int P = a.pieces;
  const int rows = kFlushThreads / P;
  const int q = tid % P, rg = tid / P;
  const int64_t per_batch = (int64_t)rows * kKeyBatch;
  const int nb = static_cast<int>((p1 - p0 + per_batch - 1) / per_batch);
  uint4 r[kKeyBatch];
  auto load_batch = [&](int b) {
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i) {
      int64_t p = p0 + b * per_batch + rg + (int64_t)rows * i;
      p = p < p1 ? p : p1 - 1;                   // clamped: the loads stay unconditional
      r[i] = *reinterpret_cast<const uint4*>(flush_row(a, true, bh, p) + q * 16);
    }
  };
  float mx[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int b = 0; b < nb; ++b) {
    load_batch(b);
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i) {
      // a clamped duplicate of the last token leaves the max unchanged
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < epp) mx[e] = fmaxf(mx[e], fabsf(piece_elem(r[i], e, bf16)));
    }
  }
  for (int m = P; m < kWave; m <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], m));
  }
  if (lane < P) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < epp) red[wave][q * epp + e] = mx[e];
  }
  __syncthreads();
  if (tid < D) {
    const float m = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    const uint16_t h = f32_to_half_bits(scale_of(m, g.qmax, g.eps));
    if constexpr (kPaged) {    // the segment's row in each of its pages
      for (int64_t tl = p0 / kTile; tl < (p1 + kTile - 1) / kTile; ++tl)
        reinterpret_cast<uint16_t*>(page_head(a, bh % g.H, tl) + 2 * kTile * g.W + 2 * kTile)[tid] = h;
    } else {
      a.k_scale[((int64_t)bh * g.max_seg + seg) * D + tid] = h;
    }
    sc[tid] = half_bits_to_f32(h);
  }
  __syncthreads();
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = e < epp ? sc[q * epp + e] : 0.0f;
  const int cpc = 128 / BITS;                    // channels per 16-byte chunk
  const int j = (q * epp) / cpc;                 // chunk of the piece
  const int byte_in_chunk = ((q * epp - j * cpc) * BITS) / 8;
  const int bytes = epp * BITS / 8;              // 1, 2, 4 or 8
  uint8_t* kc = kPaged ? nullptr : a.k_codes + (int64_t)bh * g.code_stream + j * 1024 + byte_in_chunk;
  for (int b = 0; b < nb; ++b) {
    if (nb > 1) load_batch(b);                   // one batch: still in registers
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i) {
      const int64_t p = p0 + b * per_batch + rg + (int64_t)rows * i;
      if (p >= p1) continue;
      uint64_t bits = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < epp) bits |= static_cast<uint64_t>(code_field(piece_elem(r[i], e, bf16), s[e], g.qmax, kMask)) << (e * BITS);
      uint8_t* dst = kPaged ? page_head(a, bh % g.H, p / kTile) + j * 1024 + byte_in_chunk + (p % kTile) * 16
                            : kc + (p / kTile) * kTile * g.W + (p % kTile) * 16;
      if (bytes == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(static_cast<uint32_t>(bits), static_cast<uint32_t>(bits >> 32));
      else if (bytes == 4) *reinterpret_cast<uint32_t*>(dst) = static_cast<uint32_t>(bits);
      else if (bytes == 2) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(bits);
      else *dst = static_cast<uint8_t>(bits);
    }
  }
}

// Values of one group of 64-token tiles.  A packed word holds one channel
// of 32/BITS consecutive tokens, so unit (tile, token group wj, piece q)
// reads piece q of those tokens and builds the words of the piece's
// channels in registers.  The units of a token group sit in `pieces`
// consecutive lanes, which reduce the per-token absmax; every lane derives
// the scale itself, the piece-0 lane stores it.
template <int BITS, bool kPaged>
__device__ __forceinline__ void flush_values(const FlushArgs& a, int bh, int vw, int64_t p0, int64_t p1) {
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  constexpr int kTok = 32 / BITS;                // tokens per packed word
  constexpr int kGroups = kTile / kTok;          // words per channel in a tile
  const Geom& g = a.g;
  const bool bf16 = g.dtype == KVQ_BF16;
  const int epp = bf16 ? 8 : 4;
  const int P = a.pieces;
  const int per_tile = kGroups * P;              // units per tile
  const int units = a.v_tiles_per_wg * per_tile; // a multiple of the block size
  uint8_t* vc = kPaged ? nullptr : a.v_codes + (int64_t)bh * g.code_stream;
  for (int u = threadIdx.x; u < units; u += kFlushThreads) {
    const int q = u % P, wj = (u / P) % kGroups, tw = u / per_tile;
    const int64_t t0 = (p0 / kTile + (int64_t)vw * a.v_tiles_per_wg + tw) * kTile;
    const int64_t wt = t0 + wj * kTok;           // first token of the word
    uint4 x[kTok];
#pragma unroll
    for (int i = 0; i < kTok; ++i) {
      int64_t p = wt + i;
      p = p < p0 ? p0 : (p < p1 ? p : p1 - 1);    // clamped: the loads stay unconditional
      x[i] = *reinterpret_cast<const uint4*>(flush_row(a, false, bh, p) + q * 16);
    }
    float s[kTok];
#pragma unroll
    for (int i = 0; i < kTok; ++i) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < epp) m = fmaxf(m, fabsf(piece_elem(x[i], e, bf16)));
      m = lane_group_max(m, P);
      const uint16_t h = f32_to_half_bits(scale_of(m, g.qmax, g.eps));
      s[i] = half_bits_to_f32(h);
      const int64_t t = wt + i;
      if (q == 0 && t >= p0 && t < p1) {
        if constexpr (kPaged) reinterpret_cast<uint16_t*>(page_head(a, bh % g.H, t / kTile) + 2 * kTile * g.W)[t % kTile] = h;
        else a.v_scale[(int64_t)bh * g.C + t] = h;
      }
    }
    if (wt + kTok <= p0 || wt >= p1) continue;   // no token of this word is flushed here
    uint32_t keep_mask = 0;
    if (wt < p0) keep_mask = (1u << ((p0 - wt) * BITS)) - 1u;   // unaligned start (group == 0)
    uint32_t* dst = reinterpret_cast<uint32_t*>(
        (kPaged ? page_head(a, bh % g.H, t0 / kTile) + kTile * g.W : vc + (t0 / kTile) * kTile * g.W) + wj * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e >= epp) continue;
      const int c = q * epp + e;
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < kTok; ++i) {
        const int64_t t = wt + i;
        if (t >= p0 && t < p1) word |= code_field(piece_elem(x[i], e, bf16), s[i], g.qmax, kMask) << (i * BITS);
      }
      uint32_t* w = dst + c * 2 * BITS;          // channel c: 8*BITS bytes per tile
      if (keep_mask) word |= *w & keep_mask;     // keep the previous segment's fields
      *w = word;
    }
  }
}

// Same-axis caches: the Keys (kKey) or the Values of one group of 64-token
// tiles, both quantized per token with one scale per run of kRunChannels
// channels ("KV Cache Quantization Strategies", Step 2 table, fixed local
// group).  Units as in flush_values: (tile, token group wj, piece q) reads
// piece q of 32/BITS consecutive tokens.  A run's pieces sit in aligned
// groups of consecutive lanes, which reduce its absmax; the run's first
// piece stores the scale.  Values are packed as in flush_values, Keys into
// their tokens' 16-byte chunks as in flush_keys.  Segments are whole tiles
// (group > 0), so no packed word is shared with the previous segment.
template <int BITS, bool kKey>
__device__ __forceinline__ void flush_runs(const FlushArgs& a, int bh, int vw, int64_t p0, int64_t p1) {
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  constexpr int kTok = 32 / BITS;                // tokens per packed Value word
  constexpr int kGroups = kTile / kTok;
  const Geom& g = a.g;
  const bool bf16 = g.dtype == KVQ_BF16;
  const int epp = bf16 ? 8 : 4;
  const int P = a.pieces;
  const int rp = kRunChannels / epp;             // pieces per run: 8 (bf16) or 16 (fp32) lanes
  const int per_tile = kGroups * P;
  const int units = a.v_tiles_per_wg * per_tile; // a multiple of the block size
  uint8_t* codes = (kKey ? a.k_codes : a.v_codes) + (int64_t)bh * g.code_stream;
  uint16_t* scales = (kKey ? a.k_scale : a.v_scale) + (int64_t)bh * g.C * g.runs;
  for (int u = threadIdx.x; u < units; u += kFlushThreads) {
    const int q = u % P, wj = (u / P) % kGroups, tw = u / per_tile;
    const int64_t t0 = (p0 / kTile + (int64_t)vw * a.v_tiles_per_wg + tw) * kTile;
    const int64_t wt = t0 + wj * kTok;           // first token of the unit
    uint4 x[kTok];
#pragma unroll
    for (int i = 0; i < kTok; ++i) {
      int64_t p = wt + i;
      p = p < p0 ? p0 : (p < p1 ? p : p1 - 1);    // clamped: the loads stay unconditional
      x[i] = *reinterpret_cast<const uint4*>(flush_row(a, kKey, bh, p) + q * 16);
    }
    float s[kTok];
#pragma unroll
    for (int i = 0; i < kTok; ++i) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < epp) m = fmaxf(m, fabsf(piece_elem(x[i], e, bf16)));
      m = lane_group_max(m, rp);
      const uint16_t h = f32_to_half_bits(scale_of(m, g.qmax, g.eps));
      s[i] = half_bits_to_f32(h);
      const int64_t t = wt + i;
      if (q % rp == 0 && t >= p0 && t < p1) scales[t * g.runs + q / rp] = h;
    }
    if (wt + kTok <= p0 || wt >= p1) continue;   // no token of this unit is flushed here
    if constexpr (kKey) {
      const int cpc = 128 / BITS;                // channels per 16-byte chunk
      const int j = (q * epp) / cpc;
      const int byte_in_chunk = ((q * epp - j * cpc) * BITS) / 8;
      const int bytes = epp * BITS / 8;          // 1, 2, 4 or 8
#pragma unroll
      for (int i = 0; i < kTok; ++i) {
        const int64_t t = wt + i;
        if (t < p0 || t >= p1) continue;
        uint64_t bits = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < epp) bits |= static_cast<uint64_t>(code_field(piece_elem(x[i], e, bf16), s[i], g.qmax, kMask)) << (e * BITS);
        uint8_t* dst = codes + (t / kTile) * kTile * g.W + j * 1024 + (t % kTile) * 16 + byte_in_chunk;
        if (bytes == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(static_cast<uint32_t>(bits), static_cast<uint32_t>(bits >> 32));
        else if (bytes == 4) *reinterpret_cast<uint32_t*>(dst) = static_cast<uint32_t>(bits);
        else if (bytes == 2) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(bits);
        else *dst = static_cast<uint8_t>(bits);
      }
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (t0 / kTile) * kTile * g.W) + wj;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e >= epp) continue;
        const int c = q * epp + e;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < kTok; ++i) {
          const int64_t t = wt + i;
          if (t >= p0 && t < p1) word |= code_field(piece_elem(x[i], e, bf16), s[i], g.qmax, kMask) << (i * BITS);
        }
        dst[c * 2 * BITS] = word;                // channel c: 8*BITS bytes (2*BITS words) per tile
      }
    }
  }
}

// kPaged: codes and scales go to the sequence's pages (a.pool, a.table);
// grid.z runs over the sequences, whose accounting comes from ps.
// kSameAxis (uniform caches only): per segment, v_wgs workgroups quantize
// the Keys and v_wgs the Values, both per token in runs of channels.
template <int BITS, bool kPaged, bool kSameAxis = false>
__global__ __launch_bounds__(kFlushThreads) void flush_kernel(FlushArgs a0,
                                                              typename std::conditional<kPaged, PagedFlushSeqs, NoPagedSeqs>::type ps) {
  static_assert(!(kPaged && kSameAxis), "paged caches use the KIVI axes");
  FlushArgs a = a0;
  const int per_seg = kSameAxis ? 2 * a.v_wgs : 1 + a.v_wgs;
  const int64_t sl = blockIdx.x / per_seg;
  if constexpr (kPaged) {
    const int b = blockIdx.z;
    if (sl >= ps.nseg[b]) return;                // this sequence flushes fewer segments
    a.seq = b;
    a.nq_old = ps.nq_old[b];
    a.nt_old = ps.nt_old[b];
    a.nq_slot_old = ps.nq_old[b] % a.g.ring;
    a.seg_base = ps.seg_base[b];
    a.table = a0.table + (int64_t)b * ps.table_stride;
  }
  const int bh = kPaged ? a.seq * a.g.H + (int)blockIdx.y : (int)blockIdx.y;
  const int role = blockIdx.x % per_seg;
  const int64_t seg = a.seg_base + sl;
  const int64_t p0 = a.nq_old + sl * a.seg_len;
  const int64_t p1 = p0 + a.seg_len;
  if constexpr (kSameAxis) {
    if (role < a.v_wgs) flush_runs<BITS, true>(a, bh, role, p0, p1);
    else flush_runs<BITS, false>(a, bh, role - a.v_wgs, p0, p1);
    return;
  }
  __shared__ float red[kFlushThreads / kWave][128];
  __shared__ float sc[128];
  if (role == 0) {
    flush_keys<BITS, kPaged>(a, bh, seg, p0, p1, red, sc);
    // group == 0: record the segment id of every flushed token
    if (a.g.G == 0 && bh == 0)
      for (int64_t p = p0 + threadIdx.x; p < p1; p += kFlushThreads) a.seg_index[p] = static_cast<int32_t>(seg);
  } else {
    flush_values<BITS, kPaged>(a, bh, role - 1, p0, p1);
  }
}

struct TailArgs {
  const uint8_t* k_new;
  const uint8_t* v_new;
  uint8_t* k_tail;
  uint8_t* v_tail;
  int64_t n_new;      // tokens in the input
  int first;          // first input token that stays in the window
  int count;          // tokens that stay (<= ring)
  int slot0;          // ring slot of input token `first`
  int ring;
  int row16;          // 16-byte chunks per token row
};

// grid (chunks of count * row16, batch*heads, 2 = K / V): one 16-byte copy per thread.
__global__ __launch_bounds__(256) void tail_kernel(TailArgs a) {
  const int it = blockIdx.x * blockDim.x + threadIdx.x;
  if (it >= a.count * a.row16) return;
  const int bh = blockIdx.y;
  const bool val = blockIdx.z == 1;
  const int j = it / a.row16, ch = it % a.row16;
  int slot = a.slot0 + j;
  if (slot >= a.ring) slot -= a.ring;
  const uint4* src = reinterpret_cast<const uint4*>(val ? a.v_new : a.k_new) +
                     ((int64_t)bh * a.n_new + a.first + j) * a.row16 + ch;
  uint4* dst = reinterpret_cast<uint4*>(val ? a.v_tail : a.k_tail) + ((int64_t)bh * a.ring + slot) * a.row16 + ch;
  *dst = *src;
}

// Segment geometry of a flush of `flush` tokens after nq_old (paged: the
// most any sequence flushes), and the launch (grid.y: the (batch, head)
// units, or the heads of every paged sequence, grid.z: the sequences).
void launch_flush(const Geom& g, FlushArgs& a, int64_t flush, unsigned grid_y, hipStream_t hs,
                  const PagedFlushSeqs* ps = nullptr) {
  a.seg_len = g.G == 0 ? flush : g.G;
  a.pieces = g.D * (g.dtype == KVQ_BF16 ? 2 : 4) / 16;
  const int per_tile = (kTile / (32 / g.bits)) * a.pieces;   // Value units of one tile
  a.v_tiles_per_wg = per_tile >= kFlushThreads ? 1 : kFlushThreads / per_tile;
  // tiles touched by one segment (group > 0 segments are tile aligned)
  const int64_t p0 = a.nq_old, p1 = a.nq_old + a.seg_len;
  const int64_t seg_tiles = (p1 + kTile - 1) / kTile - p0 / kTile;
  a.v_wgs = static_cast<int>((seg_tiles + a.v_tiles_per_wg - 1) / a.v_tiles_per_wg);
  const int64_t nseg = flush / a.seg_len;
  const bool same_axis = g.scheme == KVQ_SAME_AXIS;   // uniform caches only (checked by the entry points)
  dim3 grid(static_cast<unsigned>(nseg * (same_axis ? 2 * a.v_wgs : 1 + a.v_wgs)), grid_y,
            ps ? static_cast<unsigned>(g.B) : 1u);
  const NoPagedSeqs np{};
  if (same_axis) {
    switch (g.bits) {
      case 8: hipLaunchKernelGGL((flush_kernel<8, false, true>), grid, dim3(kFlushThreads), 0, hs, a, np); break;
      case 4: hipLaunchKernelGGL((flush_kernel<4, false, true>), grid, dim3(kFlushThreads), 0, hs, a, np); break;
      default: hipLaunchKernelGGL((flush_kernel<2, false, true>), grid, dim3(kFlushThreads), 0, hs, a, np); break;
    }
    return;
  }
  switch (g.bits) {
    case 8:
      if (ps) hipLaunchKernelGGL((flush_kernel<8, true>), grid, dim3(kFlushThreads), 0, hs, a, *ps);
      else hipLaunchKernelGGL((flush_kernel<8, false>), grid, dim3(kFlushThreads), 0, hs, a, np);
      break;
    case 4:
      if (ps) hipLaunchKernelGGL((flush_kernel<4, true>), grid, dim3(kFlushThreads), 0, hs, a, *ps);
      else hipLaunchKernelGGL((flush_kernel<4, false>), grid, dim3(kFlushThreads), 0, hs, a, np);
      break;
    default:
      if (ps) hipLaunchKernelGGL((flush_kernel<2, true>), grid, dim3(kFlushThreads), 0, hs, a, *ps);
      else hipLaunchKernelGGL((flush_kernel<2, false>), grid, dim3(kFlushThreads), 0, hs, a, np);
      break;
  }
}

struct PagedTailArgs {
  const uint8_t* k_new;
  const uint8_t* v_new;
  uint8_t* k_tail;
  uint8_t* v_tail;
  int64_t max_n;      // rows per (sequence, head) of the input
  int ring;
  int row16;          // 16-byte chunks per token row
  int H;
  int first[kMaxPagedSeqs];   // per sequence: first input token that stays in the window,
  int count[kMaxPagedSeqs];   // how many stay,
  int slot0[kMaxPagedSeqs];   // and the window slot of the first
};

// grid (chunks of max count * row16, batch*heads, 2 = K / V): one 16-byte copy per thread.
__global__ __launch_bounds__(256) void paged_tail_kernel(PagedTailArgs a) {
  const int bh = blockIdx.y, b = bh / a.H;
  const int it = blockIdx.x * blockDim.x + threadIdx.x;
  if (it >= a.count[b] * a.row16) return;
  const bool val = blockIdx.z == 1;
  const int j = it / a.row16, ch = it % a.row16;
  int slot = a.slot0[b] + j;
  if (slot >= a.ring) slot -= a.ring;
  const uint4* src = reinterpret_cast<const uint4*>(val ? a.v_new : a.k_new) +
                     ((int64_t)bh * a.max_n + a.first[b] + j) * a.row16 + ch;
  uint4* dst = reinterpret_cast<uint4*>(val ? a.v_tail : a.k_tail) + ((int64_t)bh * a.ring + slot) * a.row16 + ch;
  *dst = *src;
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
    a.nq_slot_old = static_cast<int>(st->quantized % g.ring);
    a.seg_base = st->segments;
    a.pool = nullptr;
    a.table = nullptr;
    a.n_pages = 0;
    a.page_bytes = 0;
    a.head_bytes = 0;
    a.seq = 0;
    launch_flush(g, a, flush, static_cast<unsigned>(g.B * g.H), hs);
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
    t.first = static_cast<int>(first);
    t.count = static_cast<int>(count);
    t.slot0 = static_cast<int>((old_end + first) % g.ring);
    t.ring = g.ring;
    t.row16 = g.D * (g.dtype == KVQ_BF16 ? 2 : 4) / 16;
    const int64_t items = count * t.row16;
    dim3 tgrid(static_cast<unsigned>((items + 255) / 256), static_cast<unsigned>(g.B * g.H), 2);
    hipLaunchKernelGGL(tail_kernel, tgrid, dim3(256), 0, hs, t);
  }
  if (hipGetLastError() != hipSuccess) return KVQ_EDEVICE;
  *st = next;
  return KVQ_OK;
}

// ---- paged caches ------------------------------------------------------------------

extern "C" kvq_status kvq_paged_page_bytes(const kvq_config* cfg, size_t* bytes) {
  Geom g;
  kvq_status s = validate_kivi_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!bytes) return KVQ_EINVAL;
  *bytes = static_cast<size_t>(g.H) * (2 * kTile * g.W + 2 * kTile + 2 * g.D);
  return KVQ_OK;
}

extern "C" kvq_status kvq_paged_append(const kvq_config* cfg, kvq_state* st, const kvq_paged_cache* cache,
                                       const void* k_new, const void* v_new, const int64_t* n_new,
                                       void* stream) {
  Geom g;
  kvq_status s = validate_kivi_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!st || !cache || !n_new) return KVQ_EINVAL;
  if (g.G <= 0 || g.B > kMaxPagedSeqs) return KVQ_EINVAL;
  if (!cache->pool || !cache->block_table || cache->n_pages < 1 || cache->table_stride < 1 ||
      (int64_t)cache->table_stride * kTile < g.C || !cache->k_tail || !cache->v_tail)
    return KVQ_EINVAL;
  const int64_t page_bytes = static_cast<int64_t>(g.H) * (2 * kTile * g.W + 2 * kTile + 2 * g.D);
  kvq_state next[kMaxPagedSeqs];
  int64_t max_n = 0;
  for (int b = 0; b < g.B; ++b) {
    s = plan_append(g, &st[b], n_new[b], &next[b]);
    if (s != KVQ_OK) return s;
    max_n = n_new[b] > max_n ? n_new[b] : max_n;
  }
  if (max_n == 0) {
    for (int b = 0; b < g.B; ++b) st[b] = next[b];
    return KVQ_OK;
  }
  if (!k_new || !v_new) return KVQ_EINVAL;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  clear_stale_hip_error();
  // every sequence flushes its own overflow into its own pages: one launch,
  // grid.z over the sequences
  PagedFlushSeqs ps;
  int64_t max_flush = 0;
  for (int b = 0; b < kMaxPagedSeqs; ++b) {
    ps.nq_old[b] = ps.nt_old[b] = ps.seg_base[b] = ps.nseg[b] = 0;
    if (b >= g.B) continue;
    ps.nq_old[b] = static_cast<int>(st[b].quantized);
    ps.nt_old[b] = static_cast<int>(st[b].tail);
    ps.seg_base[b] = static_cast<int>(st[b].segments);
    ps.nseg[b] = static_cast<int>(next[b].flushed_last / g.G);
    max_flush = next[b].flushed_last > max_flush ? next[b].flushed_last : max_flush;
  }
  ps.table_stride = cache->table_stride;
  if (max_flush > 0) {
    FlushArgs a;
    a.g = g;
    a.k_new = k_new;
    a.v_new = v_new;
    a.n_new = max_n;
    a.k_tail = cache->k_tail;
    a.v_tail = cache->v_tail;
    a.k_codes = nullptr;
    a.v_codes = nullptr;
    a.k_scale = nullptr;
    a.v_scale = nullptr;
    a.seg_index = nullptr;
    a.nq_old = a.nt_old = 0;           // per sequence, from ps
    a.nq_slot_old = 0;
    a.seg_base = 0;
    a.pool = static_cast<uint8_t*>(cache->pool);
    a.table = cache->block_table;      // row b: table + b * table_stride
    a.n_pages = cache->n_pages;
    a.page_bytes = page_bytes;
    a.head_bytes = 2 * kTile * g.W + 2 * kTile + 2 * g.D;
    a.seq = 0;
    launch_flush(g, a, max_flush, static_cast<unsigned>(g.H), hs, &ps);
  }
  // then the tokens that stay in each window
  PagedTailArgs t;
  t.k_new = static_cast<const uint8_t*>(k_new);
  t.v_new = static_cast<const uint8_t*>(v_new);
  t.k_tail = static_cast<uint8_t*>(cache->k_tail);
  t.v_tail = static_cast<uint8_t*>(cache->v_tail);
  t.max_n = max_n;
  t.ring = g.ring;
  t.row16 = g.D * (g.dtype == KVQ_BF16 ? 2 : 4) / 16;
  t.H = g.H;
  int max_count = 0;
  for (int b = 0; b < kMaxPagedSeqs; ++b) {
    t.first[b] = t.count[b] = t.slot0[b] = 0;
    if (b >= g.B) continue;
    const int64_t old_end = st[b].quantized + st[b].tail;
    const int64_t first = next[b].quantized > old_end ? next[b].quantized - old_end : 0;
    const int64_t count = n_new[b] - first;
    if (count <= 0) continue;
    t.first[b] = static_cast<int>(first);
    t.count[b] = static_cast<int>(count);
    t.slot0[b] = static_cast<int>((old_end + first) % g.ring);
    max_count = t.count[b] > max_count ? t.count[b] : max_count;
  }
  if (max_count > 0) {
    const int64_t items = (int64_t)max_count * t.row16;
    dim3 tgrid(static_cast<unsigned>((items + 255) / 256), static_cast<unsigned>(g.B * g.H), 2);
    hipLaunchKernelGGL(paged_tail_kernel, tgrid, dim3(256), 0, hs, t);
  }
  if (hipGetLastError() != hipSuccess) return KVQ_EDEVICE;
  for (int b = 0; b < g.B; ++b) st[b] = next[b];
  return KVQ_OK;
}
