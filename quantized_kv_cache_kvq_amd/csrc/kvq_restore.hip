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

// Paged caches (the page layout of kvq_paged_cache): per-sequence prefix
// lengths and the page of each tile.
constexpr int kMaxRestoreSeqs = 64;
struct PagedRestore {
  const uint8_t* pool;
  const int32_t* table;     // [batch, stride]
  int64_t n_pages;
  int64_t page_bytes;
  int head_bytes;
  int stride;
  int nq[kMaxRestoreSeqs];
};
struct NoPagedRestore {};

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

template <int D, int BITS, typename PR = NoPagedRestore>
__global__ __launch_bounds__(kRestoreThreads) void restore_kernel(RestoreArgs a, PR pr) {
  constexpr bool kPaged = !__is_same(PR, NoPagedRestore);
  constexpr int CG = D / 8;                             // Key groups of eight channels per token
  constexpr int TPC = kRestoreThreads / D;              // threads per Value channel
  constexpr int NTV = kTile / TPC;                      // Value tokens per thread
  constexpr int VW = NTV * BITS / 32;                   // their packed 32-bit words
  static_assert(VW >= 1 && (NTV * BITS) % 32 == 0, "restore shapes");
  const Geom& g = a.g;
  const int tile = blockIdx.x, unit = blockIdx.y, tid = threadIdx.x;
  const int t0 = tile * kTile;
  int nq = a.nq;
  const uint8_t* ktile;       // the tile's Key codes, Value codes, Value scales
  const uint8_t* vtile;
  const uint16_t* vstile;
  const uint16_t* kspage = nullptr;   // paged: the tile's Key-scale row
  if constexpr (kPaged) {
    const int b = unit / g.H;
    nq = pr.nq[b];
    if (t0 >= nq) return;     // this sequence has fewer tiles (uniform per workgroup)
    int64_t pg = pr.table[(int64_t)b * pr.stride + tile];
    pg = pg < 0 ? 0 : (pg >= pr.n_pages ? pr.n_pages - 1 : pg);
    ktile = pr.pool + pg * pr.page_bytes + (int64_t)(unit % g.H) * pr.head_bytes;
    vtile = ktile + kTile * g.W;
    vstile = reinterpret_cast<const uint16_t*>(ktile + 2 * kTile * g.W);
    kspage = vstile + kTile;
  } else {
    const int64_t stream = (int64_t)unit * g.code_stream + (int64_t)tile * (kTile * g.W);
    ktile = a.k_codes + stream;
    vtile = a.v_codes + stream;
    vstile = a.v_scale + (int64_t)unit * g.C + t0;
  }
  const int count = min(kTile, nq - t0);
  const int64_t row0 = (int64_t)unit * a.ld + t0;      // output row of the tile's first token

  // ---- Keys: item e = (token e / CG, channels 8 (e % CG) ..): consecutive
  // lanes cover consecutive channels of a row ----
  for (int e = tid; e < kTile * CG; e += kRestoreThreads) {
    const int i = e / CG, cg = e % CG;
    if (i >= count) continue;
    const int t = t0 + i;
    const int r = cg * BITS;                            // first byte of the group in the token's row
    const uint8_t* src = ktile + (r / 16) * 1024 + i * 16 + r % 16;
    uint64_t bits;                                      // 8 fields, low bits first
    if constexpr (BITS == 8) bits = *reinterpret_cast<const uint64_t*>(src);
    else if constexpr (BITS == 4) bits = *reinterpret_cast<const uint32_t*>(src);
    else bits = *reinterpret_cast<const uint16_t*>(src);
    const uint16_t* ksrow;
    if constexpr (kPaged) {
      ksrow = kspage;
    } else {
      const int seg = g.G > 0 ? t / g.G : a.seg_index[t];
      ksrow = a.k_scale + ((int64_t)unit * g.max_seg + seg) * D;
    }
    const uint4 sw = *reinterpret_cast<const uint4*>(ksrow + 8 * cg);
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
    const uint32_t* vt = reinterpret_cast<const uint32_t*>(vtile + c * (8 * BITS) + j0 * BITS / 8);
    uint32_t vw[VW];
#pragma unroll
    for (int k = 0; k < VW; ++k) vw[k] = vt[k];
    const uint16_t* vs = vstile + j0;
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
bool launch_restore_db(const RestoreArgs& a, const PagedRestore* pr, dim3 grid, hipStream_t s) {
  if constexpr (D * BITS % 128 == 0) {      // packed rows of whole 16-byte chunks (validated configs)
    if (pr)
      hipLaunchKernelGGL((restore_kernel<D, BITS, PagedRestore>), grid, dim3(kRestoreThreads), 0, s, a, *pr);
    else
      hipLaunchKernelGGL((restore_kernel<D, BITS>), grid, dim3(kRestoreThreads), 0, s, a, NoPagedRestore{});
    return true;
  }
  return false;
}

template <int D>
bool launch_restore_d(const RestoreArgs& a, const PagedRestore* pr, dim3 grid, hipStream_t s) {
  switch (a.g.bits) {
    case 8: return launch_restore_db<D, 8>(a, pr, grid, s);
    case 4: return launch_restore_db<D, 4>(a, pr, grid, s);
    case 2: return launch_restore_db<D, 2>(a, pr, grid, s);
  }
  return false;
}

bool launch_restore(const RestoreArgs& a, dim3 grid, hipStream_t s, const PagedRestore* pr = nullptr) {
  switch (a.g.D) {
    case 16: return launch_restore_d<16>(a, pr, grid, s);
    case 32: return launch_restore_d<32>(a, pr, grid, s);
    case 64: return launch_restore_d<64>(a, pr, grid, s);
    case 128: return launch_restore_d<128>(a, pr, grid, s);
  }
  return false;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_restore(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                                  void* k_out, void* v_out, int32_t out_dtype, int64_t ld, void* stream) {
  Geom g;
  kvq_status s = validate_kivi_config(cfg, &g);
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

extern "C" kvq_status kvq_paged_restore(const kvq_config* cfg, const kvq_state* st, const kvq_paged_cache* cache,
                                        void* k_out, void* v_out, int32_t out_dtype, int64_t ld, void* stream) {
  Geom g;
  kvq_status s = validate_kivi_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!st || !cache) return KVQ_EINVAL;
  if (g.G <= 0 || g.B > kMaxRestoreSeqs) return KVQ_EINVAL;
  if (!cache->pool || !cache->block_table || cache->n_pages < 1 || cache->table_stride < 1 ||
      (int64_t)cache->table_stride * kTile < g.C)
    return KVQ_EINVAL;
  if (out_dtype != KVQ_BF16 && out_dtype != KVQ_F32) return KVQ_EINVAL;
  PagedRestore pr;
  pr.pool = static_cast<const uint8_t*>(cache->pool);
  pr.table = cache->block_table;
  pr.n_pages = cache->n_pages;
  pr.head_bytes = 2 * kTile * g.W + 2 * kTile + 2 * g.D;
  pr.page_bytes = static_cast<int64_t>(g.H) * pr.head_bytes;
  pr.stride = cache->table_stride;
  int64_t max_nq = 0;
  for (int b = 0; b < kMaxRestoreSeqs; ++b) {
    pr.nq[b] = 0;
    if (b >= g.B) continue;
    const kvq_state& x = st[b];
    if (x.quantized < 0 || x.tail < 0 || x.total != x.quantized + x.tail || x.quantized > g.C ||
        x.quantized % g.G != 0)
      return KVQ_EINVAL;
    pr.nq[b] = static_cast<int>(x.quantized);
    max_nq = x.quantized > max_nq ? x.quantized : max_nq;
  }
  if (ld < max_nq) return KVQ_EINVAL;
  if (max_nq == 0) return KVQ_OK;           // nothing to restore
  if (!k_out || !v_out) return KVQ_EINVAL;
  RestoreArgs a;
  a.g = g;
  a.k_codes = nullptr;
  a.v_codes = nullptr;
  a.k_scale = nullptr;
  a.v_scale = nullptr;
  a.seg_index = nullptr;
  a.k_out = k_out;
  a.v_out = v_out;
  a.ld = ld;
  a.nq = static_cast<int>(max_nq);
  a.out_bf16 = out_dtype == KVQ_BF16;
  const dim3 grid(static_cast<unsigned>((max_nq + kTile - 1) / kTile), static_cast<unsigned>(g.B * g.H));
  clear_stale_hip_error();
  if (!launch_restore(a, grid, static_cast<hipStream_t>(stream), &pr)) return KVQ_EINVAL;
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}
