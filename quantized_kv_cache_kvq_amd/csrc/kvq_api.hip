// Configuration validation, buffer and workspace sizing, status strings.
#include "kvq_internal.h"

namespace kvq {

kvq_status validate_config(const kvq_config* cfg, Geom* g) {
  if (!cfg || !g) return KVQ_EINVAL;
  const kvq_config& c = *cfg;
  if (c.batch < 1 || c.kv_heads < 1) return KVQ_EINVAL;
  if (c.head_dim != 16 && c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128) return KVQ_EINVAL;
  if (c.code_bits != 8 && c.code_bits != 4 && c.code_bits != 2) return KVQ_EINVAL;
  if ((c.head_dim * c.code_bits) % 128 != 0) return KVQ_EINVAL;
  if (c.qmax < 1 || c.qmax > (1 << (c.code_bits - 1)) - 1) return KVQ_EINVAL;
  if (c.capacity < 0 || c.capacity % kTile != 0) return KVQ_EINVAL;
  if (c.residual < 1) return KVQ_EINVAL;
  if (c.group < 0 || (c.group > 0 && c.group % kTile != 0)) return KVQ_EINVAL;
  if (c.max_segments < 1) return KVQ_EINVAL;
  if (c.group > 0 && c.max_segments < c.capacity / c.group) return KVQ_EINVAL;
  if (c.kv_dtype != KVQ_BF16 && c.kv_dtype != KVQ_F32) return KVQ_EINVAL;
  if (!(c.eps > 0.0f) || c.eps > 1.0f) return KVQ_EINVAL;
  // Keep every index of the device code inside int64 and launch limits.
  if ((int64_t)c.batch * c.kv_heads > 65535) return KVQ_EINVAL;
  if ((int64_t)c.residual + c.group > (1 << 20)) return KVQ_EINVAL;
  if (c.scheme != KVQ_KIVI && c.scheme != KVQ_SAME_AXIS) return KVQ_EINVAL;
  if (c.scheme == KVQ_SAME_AXIS && (c.head_dim % kRunChannels != 0 || c.group == 0)) return KVQ_EINVAL;
  if (c.decode_kernel != KVQ_KERNEL_AUTO && c.decode_kernel != KVQ_KERNEL_VALU) return KVQ_EINVAL;
  g->B = c.batch;
  g->H = c.kv_heads;
  g->D = c.head_dim;
  g->C = c.capacity;
  g->bits = c.code_bits;
  g->qmax = c.qmax;
  g->R = c.residual;
  g->G = c.group;
  g->max_seg = c.max_segments;
  g->dtype = c.kv_dtype;
  g->eps = c.eps;
  g->W = c.head_dim * c.code_bits / 8;
  g->ring = c.group > 0 ? c.residual + c.group : c.residual;
  g->code_stream = (int64_t)c.capacity * g->W;
  g->scheme = c.scheme;
  g->runs = c.scheme == KVQ_SAME_AXIS ? c.head_dim / kRunChannels : 0;
  g->kernel = c.decode_kernel;
  return KVQ_OK;
}

// Workspace layout (bytes), shared by the attention entry points:
//   [0, 4 * units)            int32 arrival counters, one per (batch, KV head, row tile)
//   aligned to 256            float partials: per (unit, split, row) head_dim + 4 floats
//                             (acc[head_dim], m, l and padding; 16-byte rows)
size_t workspace_bytes(const Geom& g, int q_heads, int tq) {
  const int64_t units = (int64_t)g.B * g.H * ((tq + 15) / 16 + 1);
  const int64_t counters = ((units * 4 + 255) / 256) * 256;
  const int64_t splits = tq <= 1 ? kMaxSplits : 8;
  const int64_t rows = (int64_t)g.B * q_heads * (tq < 1 ? 1 : tq);
  return static_cast<size_t>(counters + rows * splits * (g.D + 4) * 4);
}

size_t workspace_counter_bytes(const Geom& g, int tq) {
  const int64_t units = (int64_t)g.B * g.H * ((tq + 15) / 16 + 1);
  return static_cast<size_t>(((units * 4 + 255) / 256) * 256);
}

namespace {
__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
}  // namespace

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_buffer_sizes(const kvq_config* cfg, kvq_sizes* out) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!out) return KVQ_EINVAL;
  const size_t streams = static_cast<size_t>(g.B) * g.H;
  const size_t es = g.dtype == KVQ_BF16 ? 2 : 4;
  out->k_codes = streams * static_cast<size_t>(g.code_stream);
  out->v_codes = out->k_codes;
  if (g.scheme == KVQ_SAME_AXIS) {     // one scale per run of channels per token, K and V alike
    out->k_scale = streams * static_cast<size_t>(g.C) * g.runs * 2;
    out->v_scale = out->k_scale;
  } else {
    out->k_scale = streams * static_cast<size_t>(g.max_seg) * g.D * 2;
    out->v_scale = streams * static_cast<size_t>(g.C) * 2;
  }
  out->k_tail = streams * static_cast<size_t>(g.ring) * g.D * es;
  out->v_tail = out->k_tail;
  out->seg_index = g.G == 0 ? static_cast<size_t>(g.C) * 4 : 0;
  out->ring = g.ring;
  out->row_bytes = g.W;
  return KVQ_OK;
}

extern "C" kvq_status kvq_workspace_size(const kvq_config* cfg, int32_t q_heads, int32_t tq,
                                         size_t* bytes) {
  Geom g;
  kvq_status s = validate_config(cfg, &g);
  if (s != KVQ_OK) return s;
  if (!bytes || q_heads < 1 || q_heads % g.H != 0 || tq < 1) return KVQ_EINVAL;
  const int gqa = q_heads / g.H;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8) return KVQ_EINVAL;
  *bytes = workspace_bytes(g, q_heads, tq);
  return KVQ_OK;
}

extern "C" kvq_status kvq_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace || bytes < 256 || bytes % 4 != 0) return KVQ_EINVAL;
  // Clearing the whole workspace is cheap and keeps the contract simple.
  const int64_t n = static_cast<int64_t>(bytes / 4);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  clear_stale_hip_error();
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t*>(workspace), n);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EDEVICE;
}

extern "C" const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_EINVAL: return "KVQ_EINVAL: invalid argument or configuration";
    case KVQ_ECAPACITY: return "KVQ_ECAPACITY: capacity or segment table exhausted";
    case KVQ_EWORKSPACE: return "KVQ_EWORKSPACE: workspace missing or too small";
    case KVQ_EDEVICE: return "KVQ_EDEVICE: HIP launch failed";
  }
  return "KVQ_UNKNOWN";
}
