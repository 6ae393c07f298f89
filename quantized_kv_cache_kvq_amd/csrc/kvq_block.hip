// Causal block attention over the quantized cache, on the MFMA units.
//
// Definition ("KV Cache and autoregressive video generation", section 3.1,
// causal mask M_ij = -inf for j > i): a block of tq new queries at absolute
// positions N .. N + tq - 1 (N cached tokens) attends to every cached token
// and to the block's own keys and values up to its own position; query head h
// reads KV head h / g (section 04).  The quantized prefix is restored inside
// the kernel (k = code / kscale, v = code / vscale: "KV Cache Quantization
// Strategies", Step 4 ``restore``); tail and block tokens are used as stored.
//
// Work: grid = (query row tiles, KV splits, batch * KV heads).  A workgroup
// owns 256 (head_dim 128) or 128 query rows of one KV head -- a row is a
// (position, head) pair --
// and a contiguous range of 64-token KV tiles: quantized tiles, then tail
// tiles (bf16 ring), then own-block tiles (bf16, causal).  Its threads
// restore each tile once into LDS, shared by its waves (32 rows each):
//   Khi [token][channel]       bf16 hi of code / kscale (tail and block
//                              tokens: the stored value)
//   Klo8 [token][channel]      fp8 e4m3 low part (x - hi) times 2^ls, one power
//                              of two per workgroup (quantized tiles only)
//   V [channel][token]         fp16: the codes (exact), or the stored values
//   vsr [token]                1 / vscale, 1 for tail and block tokens
// Logits are computed transposed, S^T = Khat . Q^T: the hi part on
// v_mfma_f32_16x16x32_bf16 against the bf16 queries (exact), the low part on
// v_mfma_scale_f32_16x16x128_f8f6f4 against the queries in fp8 (one power-of-two
// scale per wave), the scale operands undoing both powers of two.  |lo| is at
// most 2^-8 |Khat|, so the fp8 product adds about 2^-13 relative per term:
// Khat keeps ~13 significant bits (one 16-bit rounding of an outlier
// channel's 1/kscale alone moves logits by ~1e-3).  A lane then holds four consecutive tokens of
// one query in each 16-token block -- exactly its operand of the P.V product
// on v_mfma_f32_16x16x32_f16 once that MFMA's k slots of lane group kg are the
// tokens 32 ks + 4 kg + j (j < 4) and 32 ks + 16 + 4 kg + (j - 4): no transpose
// of P.  The weights p / vscale are rounded to fp16.
// Online softmax per query row in the log2 domain.  When a running maximum
// moves, the output accumulator (whose rows live in other lanes) is rescaled
// through LDS.  With several splits, partials (m, l, acc) are merged by
// block_merge_kernel.
#include "kvq_internal.h"

namespace kvq {

size_t workspace_bytes(const Geom& g, int q_heads, int tq);
size_t workspace_counter_bytes(const Geom& g, int tq);

namespace {

constexpr int kRowsWave = 32;            // two 16-row query blocks per wave
constexpr int kMergeThreads = 256;

// Workgroup shape: eight waves (256 query rows) share each restored tile at
// head_dim 128, four at head_dim 64 (where a thread's share of a Key row
// would otherwise be narrower than the 32-bit words it loads).
template <int D>
struct BlockShape {
  static constexpr int kThreads = D >= 128 ? 512 : 256;
  static constexpr int kWaves = kThreads / kWave;
  static constexpr int kRows = kRowsWave * kWaves;   // query rows per workgroup
};
constexpr int kBlockMaxSplits = 8;       // partial slots the workspace holds for tq > 1

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int f8x32_t __attribute__((ext_vector_type(8)));   // 32 fp8 e4m3 values

struct BlockArgs {
  Geom g;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const uint16_t* k_tail;   // bf16
  const uint16_t* v_tail;
  const int32_t* seg_index;
  const uint16_t* q;        // bf16 [B, tq, Hq, D]
  const uint16_t* k_blk;    // bf16 [B, tq, Hkv, D]
  const uint16_t* v_blk;
  float* out;               // fp32 [B, tq, Hq, D]
  float* part;              // [unit][split][row][D + 2]
  int nq, nt, nq_slot;
  int tq, gqa, rows;        // rows = tq * gqa query rows per KV head
  float qscale;             // sigma * log2(e)
  int tiles_q, tiles_t, tiles_b, splits;
  int frame;                // frame length F (1 = token-causal)
  int cached;               // N = nq + nt: absolute position of the block's first query
};

// Paged caches (the page layout of kvq_paged_cache): per-sequence lengths
// and the page of each 64-token tile.  A page holds, per KV head: Key codes
// (64 W bytes), Value codes (64 W), Value scales (64 fp16), the segment's
// Key-scale row (D fp16).
constexpr int kMaxBlockSeqs = 64;
struct PagedBlock {
  const uint8_t* pool;
  const int32_t* table;     // [batch, stride]
  int64_t n_pages;
  int64_t page_bytes;
  int head_bytes;
  int stride;
  int nq[kMaxBlockSeqs];
  int nt[kMaxBlockSeqs];
};
struct NoPagedBlock {};     // uniform caches

// Token a tile slot covers, and whether it exists (per tile kind).
enum TileKind { kQuant = 0, kTail = 1, kOwn = 2 };

template <int P>
struct Par {                 // a compile-time flag passed to a generic lambda
  static constexpr int value = P;
};

template <int D, int BITS, typename PB = NoPagedBlock>
__global__ __launch_bounds__(BlockShape<D>::kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void block_kernel(BlockArgs a0, PB pb) {
  constexpr bool kPaged = !__is_same(PB, NoPagedBlock);
  constexpr int kBT = BlockShape<D>::kThreads;
  constexpr int kBWaves = BlockShape<D>::kWaves;
  constexpr int kRowsWG = BlockShape<D>::kRows;
  constexpr int CG = D / (kBT / kTile);    // channels per thread in the K fill
  constexpr int KROW = D + 8;              // LDS row pitch (bf16) of Khi: no bank conflicts
  constexpr int K8ROW = D + 16;            // LDS row pitch (bytes) of Klo8
  constexpr int VROW = kTile + 4;          // LDS row pitch (fp16) of V: 34 banks, 16 rows of a
                                           // 64-bit operand read hit 32 distinct banks
  constexpr int KS = D / 32;               // k steps of the logit MFMAs
  constexpr int CB = D / 16;               // channel blocks of the output
  constexpr int TPC = kBT / D;             // threads per channel in the V fill
  constexpr int NTV = kTile / TPC;         // tokens per thread in the V fill
  constexpr int KW = (CG * BITS + 31) / 32;   // code words per thread (K fill)
  constexpr int VW = (NTV * BITS + 31) / 32;  // code words per thread (V fill)
  const Geom& g = a0.g;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int q4 = lane / 16, col = lane % 16;
  const int unit = blockIdx.z;
  const int split = blockIdx.y;
  const int b = unit / g.H, kvh = unit % g.H;
  // Paged caches: this sequence's own lengths (uniform caches: as given).
  // (kept in scalars rather than a modified copy of the arguments, which
  // the compiler would leave in scratch memory)
  const int s_nq = [&] {
    if constexpr (kPaged) return pb.nq[b];
    else return a0.nq;
  }();
  const int s_nt = [&] {
    if constexpr (kPaged) return pb.nt[b];
    else return a0.nt;
  }();
  const int s_nq_slot = kPaged ? s_nq % g.ring : a0.nq_slot;
  const int s_cached = kPaged ? s_nq + s_nt : a0.cached;
  const int s_tiles_q = kPaged ? (s_nq + kTile - 1) / kTile : a0.tiles_q;
  const int s_tiles_t = kPaged ? (s_nt + kTile - 1) / kTile : a0.tiles_t;
  const BlockArgs& a = a0;
  // Base of this KV head's part of the page of quantized tile `item`
  // (paged); page numbers outside the pool are clamped into it.
  auto page_head = [&](int item) -> const uint8_t* {
    if constexpr (kPaged) {
      int64_t pg = pb.table[(int64_t)b * pb.stride + item];
      pg = pg < 0 ? 0 : (pg >= pb.n_pages ? pb.n_pages - 1 : pg);
      return pb.pool + pg * pb.page_bytes + (int64_t)kvh * pb.head_bytes;
    } else {
      return nullptr;
    }
  };
  const int r0 = blockIdx.x * kRowsWG;
  const int Hq = g.H * a.gqa;

  // Two tile buffers: tile j of the split's run lives in buffer j % 2, so a
  // tile is restored while the one before it is computed.
  __shared__ __attribute__((aligned(16))) __bf16 Khi[2][kTile][KROW];
  // Klo8 byte 8 KS g + 8 ks + j holds channel 32 ks + 8 g + j: lane group g
  // of the fp8 product reads its 8 KS bytes in one piece.
  __shared__ __attribute__((aligned(16))) uint8_t Klo8[2][kTile][K8ROW];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[2][D][VROW];
  __shared__ __attribute__((aligned(16))) float vsr[2][kTile];
  __shared__ __attribute__((aligned(16))) float2 rkL[2][D];  // 1 / kscale split into bf16 hi, lo (as fp32),
                                                             // by item parity (G > 0)
  __shared__ float xch[kBWaves][kRowsWave];   // per-row values exchanged inside a wave
  __shared__ float kred[kBWaves];             // per-wave minima of the Key scales

  // ---- this wave's query rows: operand B of S^T = Khat . Q^T ----
  bf8_t qop[2][KS];
  int qpos[2];        // position of query row col of block qb (or -1 past the end)
  // Last block token each of those rows sees: the end of its frame
  // floor((N + pos) / F), clipped to the block.
  auto own_limit = [&](int pos) {
    return min(a.tq - 1, ((s_cached + pos) / a.frame + 1) * a.frame - 1 - s_cached);
  };
  int qlim[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = r0 + wave * kRowsWave + qb * 16 + col;
    const bool ok = r < a.rows;
    const int pos = ok ? r / a.gqa : 0, h = ok ? r % a.gqa : 0;
    qpos[qb] = ok ? pos : -1;
    qlim[qb] = own_limit(pos);
    const uint16_t* qrow = a.q + (((int64_t)b * a.tq + pos) * Hq + kvh * a.gqa + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 w = ok ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * q4) : uint4{0u, 0u, 0u, 0u};
      qop[qb][ks] = __builtin_bit_cast(bf8_t, w);
    }
  }
  // last block token any row of the workgroup sees
  const int lim_hi = own_limit((min(r0 + kRowsWG, a.rows) - 1) / a.gqa);

  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.0f, 0.0f};
  f4_t acc[2][CB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[qb][cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int items = s_tiles_q + s_tiles_t + a.tiles_b;
  const int i0 = (int)(((int64_t)items * split) / a.splits);
  const int i1 = (int)(((int64_t)items * (split + 1)) / a.splits);
  // Tiles past the last block tile any row of the workgroup sees are skipped.
  const int i_end = min(i1, s_tiles_q + s_tiles_t + lim_hi / kTile + 1);
  const int64_t stream = (int64_t)unit * g.code_stream;
  const uint16_t* kscale_unit = a.k_scale + (int64_t)unit * g.max_seg * D;
  auto ksrow_page = [&](int item) {
    return reinterpret_cast<const uint16_t*>(page_head(item) + 2 * kTile * g.W + 2 * kTile);
  };

  // ---- power of two of the fp8 low parts ----
  // |Khat| <= qmax / min kscale over the workgroup's quantized tiles, and
  // |lo| <= 2^-8 |Khat|; with |Khat| < 2^e the low parts are stored times
  // 2^ls, ls = 16 - e, so at most 2^8 in magnitude (fp8 e4m3 reaches 448).
  float kmin = INFINITY;
  {
    constexpr int C8 = D / 8;
    auto min8 = [](uint4 w) {
      const uint32_t v[4] = {w.x, w.y, w.z, w.w};
      float m = INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fminf(m, half_bits_to_f32((uint16_t)(v[j / 2] >> (16 * (j % 2)))));
      return m;
    };
    const int qe = min(i_end, s_tiles_q);
    if (i0 < qe) {
      if constexpr (kPaged) {
        const int n = (qe - i0) * C8;
        for (int e = tid; e < n; e += kBT)
          kmin = fminf(kmin, min8(*reinterpret_cast<const uint4*>(ksrow_page(i0 + e / C8) + 8 * (e % C8))));
      } else {
        const int s0 = g.G > 0 ? i0 * kTile / g.G : a.seg_index[i0 * kTile];
        const int s1 = g.G > 0 ? (qe * kTile - 1) / g.G : a.seg_index[min(qe * kTile, s_nq) - 1];
        const int n = (s1 - s0 + 1) * C8;
        for (int e = tid; e < n; e += kBT)
          kmin = fminf(kmin, min8(*reinterpret_cast<const uint4*>(kscale_unit + (int64_t)(s0 + e / C8) * D +
                                                                  8 * (e % C8))));
      }
    }
    kmin = -wave_max(-kmin);
    if (lane == 0) kred[wave] = kmin;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kBWaves; ++w) kmin = fminf(kmin, kred[w]);
  }
  int ls = 0;
  if (kmin < INFINITY) {
    const float bound = (float)g.qmax / fmaxf(kmin, g.eps);
    const int e = (int)((__float_as_uint(bound) >> 23) & 255) - 126;    // bound < 2^e
    ls = min(max(16 - e, -100), 100);
  }
  const float lsf = __uint_as_float((uint32_t)(ls + 127) << 23);      // 2^ls
  const float lsinv = __uint_as_float((uint32_t)(127 - ls) << 23);    // 2^-ls
  const int lo_scale = 127 - ls;                                      // E8M0 2^-ls

  // ---- the wave's queries in fp8 (operand B of the low product) ----
  // times 2^-qe with max |q| * 2^-qe < 2^8; slot 8 ks + j of lane group q4 is
  // channel 32 ks + 8 q4 + j, as in qop.
  f8x32_t q8[2];
  int q_scale;
  {
    float qa = 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) qa = fmaxf(qa, fabsf((float)qop[qb][ks][j]));
    qa = wave_max(qa);
    const int qe = qa > 0.0f ? min(max((int)((__float_as_uint(qa) >> 23) & 255) - 126 - 8, -120), 120) : 0;
    const float qsf = __uint_as_float((uint32_t)(127 - qe) << 23);
    q_scale = 127 + qe;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int w = 0;
          if (ks < KS) {
            const bf8_t& v = qop[qb][ks];
            w = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[4 * h] * qsf, (float)v[4 * h + 1] * qsf, 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[4 * h + 2] * qsf, (float)v[4 * h + 3] * qsf, w, true);
          }
          q8[qb][2 * ks + h] = w;
        }
    }
  }

  // With whole-group segments every token of a tile shares one Key-scale row:
  // its reciprocals are computed once per tile (one per thread) into rkL, the
  // low part already times 2^ls.
  auto seg_rk = [&](int item) {
    const uint16_t* ksrow = kPaged ? ksrow_page(item) : kscale_unit + (item * kTile / g.G) * D;
    const float r = fast_rcp(fmaxf(half_bits_to_f32(ksrow[tid]), g.eps));
    const float hi = (float)(__bf16)r;
    return float2{hi, (float)(__bf16)(r - hi) * lsf};
  };
  if (g.G > 0 && i0 < i_end && i0 < s_tiles_q && tid < D) rkL[i0 & 1][tid] = seg_rk(i0);
  // Raw codes and the Value scale a thread restores from a quantized tile;
  // the next tile's are loaded while the current one is computed.
  struct QRaw {
    uint32_t w[KW];       // Key: token tid % 64, channels (tid / 64) * CG ..
    uint32_t vw[VW];      // Value: channel tid % D, tokens (tid / D) * NTV ..
    uint16_t vs;          // Value scale of token tid (tid < 64)
  };
  auto load_qraw = [&](int item, QRaw& r) {
    const int t0 = item * kTile;
    const int count = min(kTile, s_nq - t0);
    const int i = tid % kTile, grp = tid / kTile;
    const uint8_t* kt = kPaged ? page_head(item) : a.k_codes + stream + (int64_t)item * (kTile * g.W);
    const int rb = grp * CG * BITS / 8;
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      const int rr = rb + 4 * k;
      r.w[k] = i < count ? *reinterpret_cast<const uint32_t*>(kt + (rr / 16) * 1024 + i * 16 + rr % 16) : 0u;
    }
    const int c = tid % D, vt0 = (tid / D) * NTV;
    const uint8_t* vt = (kPaged ? kt + kTile * g.W : a.v_codes + stream + (int64_t)item * (kTile * g.W)) +
                        c * (8 * BITS) + vt0 * BITS / 8;
#pragma unroll
    for (int k = 0; k < VW; ++k) r.vw[k] = *reinterpret_cast<const uint32_t*>(vt + 4 * k);
    const uint16_t* vsrow = kPaged ? reinterpret_cast<const uint16_t*>(kt + 2 * kTile * g.W)
                                   : a.v_scale + (int64_t)unit * g.C + t0;
    r.vs = tid < count ? vsrow[tid] : (uint16_t)0;
  };
  QRaw cur;
  // ---- restore tile `item` into LDS buffer bf (a quantized tile from cur) ----
  auto restore = [&](int item, int bf) __attribute__((always_inline)) {
    const int kind = item < s_tiles_q ? kQuant : (item < s_tiles_q + s_tiles_t ? kTail : kOwn);
    const int tile = kind == kQuant ? item : (kind == kTail ? item - s_tiles_q : item - s_tiles_q - s_tiles_t);
    const int t0 = tile * kTile;
    const int count = kind == kQuant ? min(kTile, s_nq - t0)
                                     : (kind == kTail ? min(kTile, s_nt - t0) : min(kTile, a.tq - t0));
      // ---- fill: restore the tile into LDS ----
      {
        const int i = tid % kTile, grp = tid / kTile;     // K: token i, channels grp * CG ..
        const bool tv = i < count;
        if (kind == kQuant) {
          const uint32_t* w = cur.w;
          // one segment per flush (G == 0): each token reads its own Key-scale row
          const uint16_t* ks = kscale_unit + (g.G > 0 ? 0 : (tv ? a.seg_index[t0 + i] : 0)) * D + grp * CG;
          const float2* rks = &rkL[item & 1][grp * CG];
  #pragma unroll
          for (int e = 0; e < CG; e += 8) {
            __bf16 hi[8];
            float lo[8];          // low parts times 2^ls
            if (g.G > 0) {
  #pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int f = e + j;
                const float code = (float)sext_field<BITS>(w[f * BITS / 32], (f * BITS) % 32);
                const float2 rk = rks[e + j];     // 1 / kscale = rk.x + rk.y 2^-ls (rk.x, rk.y 2^-ls bf16 values)
                if constexpr (BITS == 2) {
                  // code in {-1, 0, 1}: code * rk.x and code * rk.y are exact
                  hi[j] = (__bf16)(code * rk.x);
                  lo[j] = code * rk.y;
                } else {
                  const float x = fmaf(code, rk.x, code * rk.y * lsinv);
                  hi[j] = (__bf16)x;
                  lo[j] = (x - (float)hi[j]) * lsf;
                }
              }
            } else {
              const uint4 sw = *reinterpret_cast<const uint4*>(ks + e);
              const uint32_t sv[4] = {sw.x, sw.y, sw.z, sw.w};
  #pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int f = e + j;
                const float rk = fast_rcp(fmaxf(half_bits_to_f32((uint16_t)(sv[j / 2] >> (16 * (j % 2)))), g.eps));
                const float x = (float)sext_field<BITS>(w[f * BITS / 32], (f * BITS) % 32) * rk;
                hi[j] = (__bf16)x;
                lo[j] = (x - (float)hi[j]) * lsf;
              }
            }
            *reinterpret_cast<uint4*>(&Khi[bf][i][grp * CG + e]) = __builtin_bit_cast(uint4, hi);
            // channels c0 .. c0 + 7 (c0 = 32 ks + 8 g) at byte 8 KS g + 8 ks
            const int c0 = grp * CG + e;
            int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0], lo[1], 0, false);
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[2], lo[3], w0, true);
            int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[4], lo[5], 0, false);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[6], lo[7], w1, true);
            *reinterpret_cast<uint2*>(&Klo8[bf][i][8 * KS * ((c0 % 32) / 8) + 8 * (c0 / 32)]) =
                uint2{(uint32_t)w0, (uint32_t)w1};
          }
          // V: channel c, tokens vt0 .. vt0 + NTV - 1 (a run of the channel's row)
          const int c = tid % D, vt0 = (tid / D) * NTV;
          const uint32_t* vw = cur.vw;
  #pragma unroll
          for (int j0 = 0; j0 < NTV; j0 += 8) {
            _Float16 v8[8];
  #pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int f = j0 + j;
              v8[j] = (_Float16)(float)sext_field<BITS>(vw[f * BITS / 32], (f * BITS) % 32);
            }
            const uint4 v8w = __builtin_bit_cast(uint4, v8);
            *reinterpret_cast<uint2*>(&Vs[bf][c][vt0 + j0]) = uint2{v8w.x, v8w.y};
            *reinterpret_cast<uint2*>(&Vs[bf][c][vt0 + j0 + 4]) = uint2{v8w.z, v8w.w};
          }
          if (tid < kTile) vsr[bf][tid] = tid < count ? fast_rcp(fmaxf(half_bits_to_f32(cur.vs), g.eps)) : 0.0f;
        } else {
          // bf16 rows: K copied as the hi part (lo = 0), V transposed into fp16
          const uint16_t* krow;
          const uint16_t* vrow;
          if (kind == kTail) {
            int slot = s_nq_slot + t0 + (tv ? i : 0);
            slot = slot >= g.ring ? slot - g.ring : slot;
            krow = a.k_tail + ((int64_t)unit * g.ring + slot) * D;
            vrow = a.v_tail + ((int64_t)unit * g.ring + slot) * D;
          } else {
            const int j = t0 + (tv ? i : 0);
            krow = a.k_blk + (((int64_t)b * a.tq + j) * g.H + kvh) * D;
            vrow = a.v_blk + (((int64_t)b * a.tq + j) * g.H + kvh) * D;
          }
  #pragma unroll
          for (int e = 0; e < CG; e += 8) {
            const uint4 kw = tv ? *reinterpret_cast<const uint4*>(krow + grp * CG + e) : uint4{0u, 0u, 0u, 0u};
            const uint4 vv = tv ? *reinterpret_cast<const uint4*>(vrow + grp * CG + e) : uint4{0u, 0u, 0u, 0u};
            *reinterpret_cast<uint4*>(&Khi[bf][i][grp * CG + e]) = kw;
            const uint32_t vs4[4] = {vv.x, vv.y, vv.z, vv.w};
  #pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float v = __uint_as_float((vs4[j / 2] >> (16 * (j % 2))) << 16);
              Vs[bf][grp * CG + e + j][i] = (_Float16)v;
            }
          }
          if (tid < kTile) vsr[bf][tid] = tid < count ? 1.0f : 0.0f;
        }
      }
  };
  // The raw codes and Key-scale reciprocals of quantized tile `item`; rk is
  // written to rkL[item & 1] before the barrier that precedes its restore.
  float2 rk_next = float2{0.0f, 0.0f};
  auto fetch = [&](int item) __attribute__((always_inline)) {
    if (item < i_end && item < s_tiles_q) {
      if (g.G > 0 && tid < D) rk_next = seg_rk(item);
      load_qraw(item, cur);
    }
  };
  if (i0 < i_end && i0 < s_tiles_q) load_qraw(i0, cur);
  __syncthreads();                 // rkL of the first tile
  if (i0 < i_end) restore(i0, 0);
  fetch(i0 + 1);
  if (g.G > 0 && i0 + 1 < i_end && i0 + 1 < s_tiles_q && tid < D) rkL[(i0 + 1) & 1][tid] = rk_next;
  __syncthreads();                 // the first tile is restored

  // Each step computes tile `item` from buffer b and restores tile item + 1
  // into the other buffer, with one barrier per tile.  The two waves of a
  // SIMD (wave w and w + half) take the phases in different orders --
  // logits, softmax, P.V, restore against restore, logits, softmax, P.V --
  // so that one of them is on the matrix cores while the other is on the
  // vector ALUs; the logits and the P operands are never live during a
  // restore.
  const bool restore_first = wave >= kBWaves / 2;
  for (int item = i0; item < i_end; ++item) {
    const int b = (item - i0) & 1;
    const int kind = item < s_tiles_q ? kQuant : (item < s_tiles_q + s_tiles_t ? kTail : kOwn);
    const int tile = kind == kQuant ? item : (kind == kTail ? item - s_tiles_q : item - s_tiles_q - s_tiles_t);
    const int t0 = tile * kTile;
    const int count = kind == kQuant ? min(kTile, s_nq - t0)
                                     : (kind == kTail ? min(kTile, s_nt - t0) : min(kTile, a.tq - t0));
    auto restore_next = [&]() __attribute__((always_inline)) {
      if (item + 1 < i_end) restore(item + 1, b ^ 1);
      fetch(item + 2);             // cur's restore is done: its registers are free
    };
    if (restore_first) restore_next();

    // ---- logits S^T[token][query] (token block tb, query block qb) ----
    // The Key operands of k step ks + 1 are read from LDS while the MFMAs of
    // k step ks run: scheduling barriers keep each batch of reads ahead of the
    // previous batch's products (eight independent accumulators per k step).
    f4_t S[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) S[tb][qb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto logits = [&](auto with_lo) {
      constexpr bool kLo = decltype(with_lo)::value != 0;
      bf8_t kh[2][4];
      f8x32_t kq[2];        // fp8 low operand of token block tb, one step ahead
      auto kread = [&](int ks, bf8_t (&h)[4]) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          h[tb] = *reinterpret_cast<const bf8_t*>(&Khi[b][tb * 16 + col][32 * ks + 8 * q4]);
      };
      auto lread = [&](int tb, f8x32_t& k) {
        const uint8_t* src = &Klo8[b][tb * 16 + col][8 * KS * q4];
        const uint4 w0 = *reinterpret_cast<const uint4*>(src);
        const uint4 w1 = KS == 4 ? *reinterpret_cast<const uint4*>(src + 16) : uint4{0u, 0u, 0u, 0u};
        k = f8x32_t{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
      };
      // k step ks also takes the low product of token block ks (KS = 4), or of
      // token blocks 2 ks and 2 ks + 1 (KS = 2)
      constexpr int kLoPerStep = 4 / KS;
      kread(0, kh[0]);
      if constexpr (kLo) lread(0, kq[0]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) kread(ks + 1, kh[(ks + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            S[tb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh[ks & 1][tb], qop[qb][ks], S[tb][qb], 0, 0, 0);
        if constexpr (kLo) {
#pragma unroll
          for (int u = 0; u < kLoPerStep; ++u) {
            const int tb = ks * kLoPerStep + u;
            if (tb + 1 < 4) lread(tb + 1, kq[(tb + 1) & 1]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              S[tb][qb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kq[tb & 1], q8[qb], S[tb][qb], 0, 0, 0,
                                                                           lo_scale, 0, q_scale);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (kind == kQuant) logits(Par<1>{});
    else logits(Par<0>{});

    // ---- online softmax per query (lane's column col of block qb) ----
    // S[tb][qb][i]: token t0 + 16 tb + 4 q4 + i; the logit (log2 domain) is
    // S * qscale, folded into the exponent.
    float vr[4][4];       // 1 / vscale of the lane's tokens (shared by both query blocks)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const float4 v4 = *reinterpret_cast<const float4*>(&vsr[b][16 * tb + 4 * q4]);
      vr[tb][0] = v4.x; vr[tb][1] = v4.y; vr[tb][2] = v4.z; vr[tb][3] = v4.w;
    }
    const bool full = kind == kQuant && count == kTile;   // no masking needed
    h8_t pa[2][2];        // P operands: [qb][k step] (tokens 32 ks + 4 q4 + j, 32 ks + 16 + 4 q4 + j)
    float alpha[2];
    bool moved = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
      if (!full) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tt = 16 * tb + 4 * q4 + i;
            const bool vis = tt < count && qpos[qb] >= 0 && (kind != kOwn || t0 + tt <= qlim[qb]);
            S[tb][qb][i] = vis ? S[tb][qb][i] : -INFINITY;
          }
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        mx = fmaxf(mx, fmaxf(fmaxf(S[tb][qb][0], S[tb][qb][1]), fmaxf(S[tb][qb][2], S[tb][qb][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mn = fmaxf(m[qb], mx * a.qscale);
      alpha[qb] = (mn == -INFINITY) ? 1.0f : fast_exp2(m[qb] - mn);
      moved |= alpha[qb] != 1.0f && m[qb] != -INFINITY;
      m[qb] = mn;
      const float mu = mn == -INFINITY ? 0.0f : mn;
      float ps = 0.0f;
      float pv[4][4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(fmaf(S[tb][qb][i], a.qscale, -mu));
          ps += p;
          pv[tb][i] = p * vr[tb][i];
        }
      lsum[qb] = lsum[qb] * alpha[qb] + ps;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pa[qb][ks] = h8_t{(_Float16)pv[2 * ks][0], (_Float16)pv[2 * ks][1], (_Float16)pv[2 * ks][2],
                          (_Float16)pv[2 * ks][3], (_Float16)pv[2 * ks + 1][0], (_Float16)pv[2 * ks + 1][1],
                          (_Float16)pv[2 * ks + 1][2], (_Float16)pv[2 * ks + 1][3]};
    }
    if (__any(moved)) {
      // acc row 4 q4 + i of block qb needs alpha of query 4 q4 + i (held by lanes col == 4 q4 + i)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (q4 == 0) xch[wave][qb * 16 + col] = alpha[qb];
      }
      wave_lds_sync();
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = xch[wave][qb * 16 + 4 * q4 + i];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[qb][cb][i] *= al;
        }
      wave_lds_sync();
    }


    // ---- acc[query][channel] += P' . V (k step outermost; the Value
    // operands of k step 1 are read while the MFMAs of k step 0 run) ----
    // Value operands in batches of four channel blocks, one batch ahead.
    constexpr int kVB = 4;
    constexpr int NVB = 2 * CB / kVB;     // batches (k step major)
    h8_t vop[2][kVB];
    auto vread = [&](int bi, h8_t (&v)[kVB]) {
      const int ks = bi / (CB / kVB), cb0 = (bi % (CB / kVB)) * kVB;
#pragma unroll
      for (int j = 0; j < kVB; ++j) {
        const int cb = cb0 + j;
        const h4_t v0 = *reinterpret_cast<const h4_t*>(&Vs[b][16 * cb + col][32 * ks + 4 * q4]);
        const h4_t v1 = *reinterpret_cast<const h4_t*>(&Vs[b][16 * cb + col][32 * ks + 16 + 4 * q4]);
        v[j] = h8_t{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
    };
    vread(0, vop[0]);
#pragma unroll
    for (int bi = 0; bi < NVB; ++bi) {
      if (bi + 1 < NVB) vread(bi + 1, vop[(bi + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int ks = bi / (CB / kVB), cb0 = (bi % (CB / kVB)) * kVB;
#pragma unroll
      for (int j = 0; j < kVB; ++j)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc[qb][cb0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[qb][ks], vop[bi & 1][j], acc[qb][cb0 + j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!restore_first) restore_next();
    // the Key-scale reciprocals of tile item + 2 into the slot tile item used
    if (g.G > 0 && item + 2 < i_end && item + 2 < s_tiles_q && tid < D) rkL[item & 1][tid] = rk_next;
    __syncthreads();      // tile item + 1 is restored; buffer b is free
  }

  // ---- write: rows 4 q4 + i of block qb, channel 16 cb + col ----
  // Row sums: lanes col, col + 16, col + 32, col + 48 hold parts of query col.
  float ltot[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = lsum[qb];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    ltot[qb] = l;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (q4 == 0) xch[wave][qb * 16 + col] = ltot[qb];
  }
  wave_lds_sync();
  float lrow[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) lrow[qb][i] = xch[wave][qb * 16 + 4 * q4 + i];
  wave_lds_sync();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (q4 == 0) xch[wave][qb * 16 + col] = m[qb];
  }
  wave_lds_sync();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + wave * kRowsWave + qb * 16 + 4 * q4 + i;
      if (r >= a.rows) continue;
      const float mrow = xch[wave][qb * 16 + 4 * q4 + i];
      if (a.splits == 1) {
        const int pos = r / a.gqa, h = r % a.gqa;
        float* o = a.out + (((int64_t)b * a.tq + pos) * Hq + kvh * a.gqa + h) * D;
        const float inv = 1.0f / lrow[qb][i];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[16 * cb + col] = acc[qb][cb][i] * inv;
      } else {
        float* p = a.part + (((int64_t)unit * a.splits + split) * a.rows + r) * (D + 2);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) p[16 * cb + col] = acc[qb][cb][i];
        if (col == 0) {
          p[D] = mrow;
          p[D + 1] = lrow[qb][i];
        }
      }
    }
}

// Combine the splits' partials of each query row: one thread per (row, channel).
template <int D>
__global__ __launch_bounds__(kMergeThreads) void block_merge_kernel(BlockArgs a) {
  const int unit = blockIdx.y;
  const int b = unit / a.g.H, kvh = unit % a.g.H;
  const int Hq = a.g.H * a.gqa;
  const int64_t idx = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (idx >= (int64_t)a.rows * D) return;
  const int r = (int)(idx / D), c = (int)(idx % D);
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s)
    M = fmaxf(M, a.part[(((int64_t)unit * a.splits + s) * a.rows + r) * (D + 2) + D]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < a.splits; ++s) {
    const float* p = a.part + (((int64_t)unit * a.splits + s) * a.rows + r) * (D + 2);
    const float e = p[D] == -INFINITY ? 0.0f : fast_exp2(p[D] - M);
    num = fmaf(p[c], e, num);
    den = fmaf(p[D + 1], e, den);
  }
  const int pos = r / a.gqa, h = r % a.gqa;
  a.out[(((int64_t)b * a.tq + pos) * Hq + kvh * a.gqa + h) * D + c] = num / den;
}

template <int D, int BITS>
void launch_block(const BlockArgs& a, const PagedBlock* pb, hipStream_t s) {
  constexpr int kRowsWG = BlockShape<D>::kRows;
  dim3 grid((a.rows + kRowsWG - 1) / kRowsWG, a.splits, a.g.B * a.g.H);
  if (pb)
    hipLaunchKernelGGL((block_kernel<D, BITS, PagedBlock>), grid, dim3(BlockShape<D>::kThreads), 0, s, a, *pb);
  else
    hipLaunchKernelGGL((block_kernel<D, BITS>), grid, dim3(BlockShape<D>::kThreads), 0, s, a, NoPagedBlock{});
  if (a.splits > 1) {
    dim3 mg((unsigned)(((int64_t)a.rows * D + kMergeThreads - 1) / kMergeThreads), a.g.B * a.g.H);
    hipLaunchKernelGGL((block_merge_kernel<D>), mg, dim3(kMergeThreads), 0, s, a);
  }
}

bool dispatch_block(const BlockArgs& a, hipStream_t s, const PagedBlock* pb = nullptr) {
  const int D = a.g.D, bits = a.g.bits;
  if (D == 128 && bits == 2) { launch_block<128, 2>(a, pb, s); return true; }
  if (D == 128 && bits == 4) { launch_block<128, 4>(a, pb, s); return true; }
  if (D == 128 && bits == 8) { launch_block<128, 8>(a, pb, s); return true; }
  if (D == 64 && bits == 2) { launch_block<64, 2>(a, pb, s); return true; }
  if (D == 64 && bits == 4) { launch_block<64, 4>(a, pb, s); return true; }
  if (D == 64 && bits == 8) { launch_block<64, 8>(a, pb, s); return true; }
  return false;
}

int block_auto_splits(int row_tiles, int units, int items, int threads) {
  // Aim for about eight waves per compute unit (256 CUs) and at least eight
  // tiles per split.
  const int64_t wgs = (int64_t)row_tiles * units;
  const int64_t target = 256 * 8 * kWave / threads;
  int s = (int)((target + wgs - 1) / wgs);
  if (s > kBlockMaxSplits) s = kBlockMaxSplits;
  if (s > items / 8) s = items / 8;
  return s < 1 ? 1 : s;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_block_attn(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                                     const void* q, const void* k_blk, const void* v_blk, int32_t tq,
                                     int32_t q_heads, int32_t frame_tokens, float softmax_scale,
                                     int32_t num_splits, float* out, void* workspace,
                                     size_t workspace_size, void* stream) {
  Geom g;
  kvq_status s = validate_kivi_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!st || !cache || !q || !k_blk || !v_blk || !out) return KVQ_EINVAL;
  if (g.dtype != KVQ_BF16 || (g.D != 64 && g.D != 128)) return KVQ_EINVAL;
  if (tq < 1 || q_heads < 1 || q_heads % g.H != 0) return KVQ_EINVAL;
  const int gqa = q_heads / g.H;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8) return KVQ_EINVAL;
  if (st->quantized < 0 || st->tail < 0 || st->total != st->quantized + st->tail || st->quantized > g.C ||
      st->tail > g.ring)
    return KVQ_EINVAL;
  if (g.G > 0 && st->quantized % g.G != 0) return KVQ_EINVAL;
  if (!(softmax_scale > 0.0f) || num_splits < 0 || num_splits > kBlockMaxSplits) return KVQ_EINVAL;
  if ((int64_t)tq * gqa > (1 << 30)) return KVQ_EINVAL;
  if (frame_tokens < 1 || st->total + (int64_t)tq + frame_tokens > (int64_t(1) << 31) - 1) return KVQ_EINVAL;
  if (st->quantized > 0 && (!cache->k_codes || !cache->v_codes || !cache->k_scale || !cache->v_scale ||
                            (g.G == 0 && !cache->seg_index)))
    return KVQ_EINVAL;
  if (st->tail > 0 && (!cache->k_tail || !cache->v_tail)) return KVQ_EINVAL;
  if (!workspace || workspace_size < workspace_bytes(g, q_heads, tq)) return KVQ_EWORKSPACE;

  BlockArgs a;
  a.g = g;
  a.k_codes = static_cast<const uint8_t*>(cache->k_codes);
  a.v_codes = static_cast<const uint8_t*>(cache->v_codes);
  a.k_scale = static_cast<const uint16_t*>(cache->k_scale);
  a.v_scale = static_cast<const uint16_t*>(cache->v_scale);
  a.k_tail = static_cast<const uint16_t*>(cache->k_tail);
  a.v_tail = static_cast<const uint16_t*>(cache->v_tail);
  a.seg_index = static_cast<const int32_t*>(cache->seg_index);
  a.q = static_cast<const uint16_t*>(q);
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.out = out;
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + workspace_counter_bytes(g, tq));
  a.nq = static_cast<int>(st->quantized);
  a.nt = static_cast<int>(st->tail);
  a.nq_slot = static_cast<int>(st->quantized % g.ring);
  a.tq = tq;
  a.gqa = gqa;
  a.rows = tq * gqa;
  a.qscale = softmax_scale * 1.4426950408889634f;
  a.tiles_q = (a.nq + kTile - 1) / kTile;
  a.tiles_t = (a.nt + kTile - 1) / kTile;
  a.tiles_b = (tq + kTile - 1) / kTile;
  a.frame = frame_tokens;
  a.cached = static_cast<int>(st->total);
  const int rows_wg = g.D >= 128 ? BlockShape<128>::kRows : BlockShape<64>::kRows;
  const int threads = g.D >= 128 ? BlockShape<128>::kThreads : BlockShape<64>::kThreads;
  const int row_tiles = (a.rows + rows_wg - 1) / rows_wg;
  const int items = a.tiles_q + a.tiles_t + a.tiles_b;
  a.splits = num_splits > 0 ? num_splits : block_auto_splits(row_tiles, g.B * g.H, items, threads);
  if (a.splits > items) a.splits = items;
  if (row_tiles > 65535) return KVQ_EINVAL;
  clear_stale_hip_error();
  if (!dispatch_block(a, static_cast<hipStream_t>(stream))) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}

extern "C" kvq_status kvq_paged_block_attn(const kvq_config* cfg, const kvq_state* st,
                                           const kvq_paged_cache* cache, const void* q, const void* k_blk,
                                           const void* v_blk, int32_t tq, int32_t q_heads, int32_t frame_tokens,
                                           float softmax_scale, int32_t num_splits, float* out, void* workspace,
                                           size_t workspace_size, void* stream) {
  Geom g;
  kvq_status s = validate_kivi_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!st || !cache || !q || !k_blk || !v_blk || !out) return KVQ_EINVAL;
  if (g.dtype != KVQ_BF16 || (g.D != 64 && g.D != 128)) return KVQ_EINVAL;
  if (g.G <= 0 || g.B > kMaxBlockSeqs) return KVQ_EINVAL;
  if (!cache->pool || !cache->block_table || cache->n_pages < 1 || cache->table_stride < 1 ||
      (int64_t)cache->table_stride * kTile < g.C)
    return KVQ_EINVAL;
  if (tq < 1 || q_heads < 1 || q_heads % g.H != 0) return KVQ_EINVAL;
  const int gqa = q_heads / g.H;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8) return KVQ_EINVAL;
  if (!(softmax_scale > 0.0f) || num_splits < 0 || num_splits > kBlockMaxSplits) return KVQ_EINVAL;
  if ((int64_t)tq * gqa > (1 << 30)) return KVQ_EINVAL;
  if (frame_tokens < 1) return KVQ_EINVAL;
  PagedBlock pb;
  pb.pool = static_cast<const uint8_t*>(cache->pool);
  pb.table = cache->block_table;
  pb.n_pages = cache->n_pages;
  pb.head_bytes = 2 * kTile * g.W + 2 * kTile + 2 * g.D;
  pb.page_bytes = static_cast<int64_t>(g.H) * pb.head_bytes;
  pb.stride = cache->table_stride;
  int max_items = 1;
  bool any_tail = false;
  for (int b = 0; b < kMaxBlockSeqs; ++b) {
    pb.nq[b] = pb.nt[b] = 0;
    if (b >= g.B) continue;
    const kvq_state& x = st[b];
    if (x.quantized < 0 || x.tail < 0 || x.total != x.quantized + x.tail || x.quantized > g.C ||
        x.tail > g.ring || x.quantized % g.G != 0)
      return KVQ_EINVAL;
    if (x.total + (int64_t)tq + frame_tokens > (int64_t(1) << 31) - 1) return KVQ_EINVAL;
    pb.nq[b] = static_cast<int>(x.quantized);
    pb.nt[b] = static_cast<int>(x.tail);
    any_tail |= x.tail > 0;
    const int items = static_cast<int>((x.quantized + kTile - 1) / kTile + (x.tail + kTile - 1) / kTile +
                                       (tq + kTile - 1) / kTile);
    max_items = items > max_items ? items : max_items;
  }
  if (any_tail && (!cache->k_tail || !cache->v_tail)) return KVQ_EINVAL;
  if (!workspace || workspace_size < workspace_bytes(g, q_heads, tq)) return KVQ_EWORKSPACE;

  // Uniform fields; the kernel takes each sequence's lengths from pb.
  BlockArgs a;
  a.g = g;
  a.k_codes = nullptr;
  a.v_codes = nullptr;
  a.k_scale = nullptr;
  a.v_scale = nullptr;
  a.k_tail = static_cast<const uint16_t*>(cache->k_tail);
  a.v_tail = static_cast<const uint16_t*>(cache->v_tail);
  a.seg_index = nullptr;
  a.q = static_cast<const uint16_t*>(q);
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.out = out;
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + workspace_counter_bytes(g, tq));
  a.nq = 0;
  a.nt = 0;
  a.nq_slot = 0;
  a.tq = tq;
  a.gqa = gqa;
  a.rows = tq * gqa;
  a.qscale = softmax_scale * 1.4426950408889634f;
  a.tiles_q = 0;
  a.tiles_t = 0;
  a.tiles_b = (tq + kTile - 1) / kTile;
  a.frame = frame_tokens;
  a.cached = 0;
  const int rows_wg = g.D >= 128 ? BlockShape<128>::kRows : BlockShape<64>::kRows;
  const int threads = g.D >= 128 ? BlockShape<128>::kThreads : BlockShape<64>::kThreads;
  const int row_tiles = (a.rows + rows_wg - 1) / rows_wg;
  // one split count for every sequence (the longest sets it); shorter
  // sequences leave some splits empty, which the merge weighs as zero
  a.splits = num_splits > 0 ? num_splits : block_auto_splits(row_tiles, g.B * g.H, max_items, threads);
  if (a.splits > max_items) a.splits = max_items;
  if (row_tiles > 65535) return KVQ_EINVAL;
  clear_stale_hip_error();
  if (!dispatch_block(a, static_cast<hipStream_t>(stream), &pb)) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}
