// C ABI of librlq: argument validation, split planning and kernel launches.
// Declarations and the meaning of every argument: include/rlq.h.

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "rlq_internal.h"

// Scratch of rlq_mla_decode_noalloc: one array per device, living as long as
// the process.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, looked up once per device (with
// that device current) and kept (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[RLQ_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_hip_error[256] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return RLQ_OK;
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s: %s", hipGetErrorName(e),
           hipGetErrorString(e));
  return RLQ_EHIP;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Device architecture check, cached per device ordinal.
int check_device() {
  static int known[64];  // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= 64) return RLQ_EUNSUPPORTED;
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_status(e);
    known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return known[dev] == 1 ? RLQ_OK : RLQ_EUNSUPPORTED;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

int scratch_ptr(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return RLQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr || !aligned(p, 256)) return RLQ_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return RLQ_OK;
}

// Opt-in checks of the values that live in device memory (RLQ_DEBUG set to
// anything but "0"): the call copies them to the host (synchronizing its
// stream) and returns RLQ_EINVAL if one is out of range, before any launch.
bool debug_checks() {
  const char *e = getenv("RLQ_DEBUG");
  return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
}

// Test switch of the 16-head kernel's bounded exchange wait
// (RLQ_TEST_EXCHANGE_TIMEOUT set to anything but "0"): every poll finds its
// slot empty and gives up after two tries, so each workgroup marks its
// partial lost and the call's outputs and LSE come out NaN.  Every kernel
// still runs to its end.
bool force_exchange_timeout() {
  const char *e = getenv("RLQ_TEST_EXCHANGE_TIMEOUT");
  return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
}

// Copies `n` int32 of device memory to `host` in stream order.
int fetch_i32(const int32_t *dev, size_t n, std::vector<int32_t> &host, hipStream_t stream) {
  host.resize(n);
  if (n == 0) return RLQ_OK;
  hipError_t e = hipMemcpyAsync(host.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return hip_status(e);
}

int check_cache(const rlq_cache *c, int32_t batch) {
  if (c == nullptr || c->codes == nullptr || c->meta == nullptr || c->rope == nullptr)
    return RLQ_EINVAL;
  if (!aligned(c->codes, 16) || !aligned(c->meta, 16) || !aligned(c->rope, 16)) return RLQ_EINVAL;
  if (c->page_size != RLQ_PAGE || c->num_pages < 1) return RLQ_EINVAL;
  if (c->sink != nullptr) {
    if (c->n_sink < 1 || c->max_batch < batch || !aligned(c->sink, 16)) return RLQ_EINVAL;
  }
  if (c->recent != nullptr) {
    if (c->n_recent < 1 || c->max_batch < batch || !aligned(c->recent, 16)) return RLQ_EINVAL;
  }
  if (c->n_sink < 0 || c->n_recent < 0) return RLQ_EINVAL;
  return RLQ_OK;
}

}  // namespace

extern "C" {

int rlq_abi_version(void) { return RLQ_ABI_VERSION; }

rlq_layer_params rlq_layer_params_default(void) {
  rlq_layer_params p;
  p.tau = 0.9816f;
  p.gain = 1.0f;
  p.level_inner = 0.4528f;
  p.level_outer = 1.510f;
  return p;
}

const char *rlq_status_string(int status) {
  switch (status) {
    case RLQ_OK: return "RLQ_OK";
    case RLQ_EINVAL: return "RLQ_EINVAL: invalid argument";
    case RLQ_EUNSUPPORTED: return "RLQ_EUNSUPPORTED: device is not gfx950";
    case RLQ_ENOSPC: return "RLQ_ENOSPC: workspace too small";
    case RLQ_EHIP: return "RLQ_EHIP: HIP runtime error";
    default: return "unknown rlq status";
  }
}

const char *rlq_last_hip_error(void) { return g_last_hip_error; }

float rlq_coupled_gain(float tau, float level_inner, float level_outer) {
  if (!(level_inner > 0.f) || !(level_outer > 0.f)) return NAN;
  const double inv_sqrt_2pi = 0.39894228040143267794;
  const double t = tau;
  const double phi0 = inv_sqrt_2pi;
  const double phit = inv_sqrt_2pi * exp(-0.5 * t * t);
  const double resp = 2.0 * (level_inner * phi0 + ((double)level_outer - level_inner) * phit);
  return (float)(1.0 / resp);
}

// Page ids of positions [p0, p1) of one request.
static bool pages_ok(const int32_t *row, int64_t p0, int64_t p1, int32_t max_pages, int32_t num_pages) {
  if (p1 <= p0) return true;
  const int64_t first = p0 / RLQ_PAGE, last = (p1 - 1) / RLQ_PAGE;
  if (p0 < 0 || last >= max_pages) return false;
  for (int64_t i = first; i <= last; ++i)
    if (row[i] < 0 || row[i] >= num_pages) return false;
  return true;
}

int rlq_check_decode_tables(int32_t batch, const int32_t *ctx_lens, const int32_t *block_table,
                            int32_t max_pages_per_req, int32_t num_pages, int32_t max_ctx_len) {
  if (batch < 1 || ctx_lens == nullptr || block_table == nullptr || max_pages_per_req < 1 || num_pages < 1)
    return RLQ_EINVAL;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = ctx_lens[b];
    if (n < 0 || n > max_ctx_len) return RLQ_EINVAL;
    if (!pages_ok(block_table + (int64_t)b * max_pages_per_req, 0, n, max_pages_per_req, num_pages))
      return RLQ_EINVAL;
  }
  return RLQ_OK;
}

int rlq_check_append_tables(int32_t batch, const int32_t *cu_seqlens, const int32_t *start_pos,
                            const int32_t *block_table, int32_t max_pages_per_req, int32_t num_pages,
                            int64_t n_tokens) {
  if (batch < 1 || cu_seqlens == nullptr || start_pos == nullptr || block_table == nullptr ||
      max_pages_per_req < 1 || num_pages < 1)
    return RLQ_EINVAL;
  if (cu_seqlens[0] != 0 || cu_seqlens[batch] != n_tokens) return RLQ_EINVAL;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = (int64_t)cu_seqlens[b + 1] - cu_seqlens[b];
    if (n < 0 || start_pos[b] < 0) return RLQ_EINVAL;
    if (!pages_ok(block_table + (int64_t)b * max_pages_per_req, start_pos[b], start_pos[b] + n,
                  max_pages_per_req, num_pages))
      return RLQ_EINVAL;
  }
  return RLQ_OK;
}

int rlq_check_extend_tables(int32_t batch, const int32_t *cu_seqlens_q, const int32_t *ctx_lens,
                            const int32_t *block_table, int32_t max_pages_per_req, int32_t num_pages,
                            int32_t max_q_len, int32_t max_ctx_len) {
  if (cu_seqlens_q == nullptr) return RLQ_EINVAL;
  const int st = rlq_check_decode_tables(batch, ctx_lens, block_table, max_pages_per_req, num_pages, max_ctx_len);
  if (st != RLQ_OK) return st;
  if (cu_seqlens_q[0] != 0) return RLQ_EINVAL;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t nq = (int64_t)cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    if (nq < 0 || nq > max_q_len || nq > ctx_lens[b]) return RLQ_EINVAL;
  }
  return RLQ_OK;
}

int rlq_quantize_append(const rlq_layer_params *p, const rlq_cache *cache,
                        const uint16_t *latent_bf16, const float *latent_rot_f32,
                        const uint16_t *rotation_bf16, const uint16_t *k_rope_bf16,
                        const int32_t *cu_seqlens, const int32_t *start_pos,
                        const int32_t *block_table, int32_t max_pages_per_req,
                        int32_t batch, int64_t n_tokens, float *z_debug, void *stream) {
  if (p == nullptr || batch < 1 || n_tokens < 0 || max_pages_per_req < 1) return RLQ_EINVAL;
  if (!(p->tau >= 0.f) || !isfinite(p->tau)) return RLQ_EINVAL;  // the code needs t = tau * s >= 0
  int st = check_cache(cache, batch);
  if (st != RLQ_OK) return st;
  if ((latent_bf16 == nullptr) == (latent_rot_f32 == nullptr)) return RLQ_EINVAL;
  if (latent_bf16 != nullptr && (rotation_bf16 == nullptr || !aligned(latent_bf16, 16) ||
                                 !aligned(rotation_bf16, 16)))
    return RLQ_EINVAL;
  if (latent_rot_f32 != nullptr && !aligned(latent_rot_f32, 16)) return RLQ_EINVAL;
  if (k_rope_bf16 == nullptr || !aligned(k_rope_bf16, 16)) return RLQ_EINVAL;
  if (cu_seqlens == nullptr || start_pos == nullptr || block_table == nullptr) return RLQ_EINVAL;
  if (!aligned(cu_seqlens, 4) || !aligned(start_pos, 4) || !aligned(block_table, 4)) return RLQ_EINVAL;
  if (z_debug != nullptr && !aligned(z_debug, 16)) return RLQ_EINVAL;
  st = check_device();
  if (st != RLQ_OK) return st;
  if (debug_checks()) {
    std::vector<int32_t> cu, sp, bt;
    if ((st = fetch_i32(cu_seqlens, (size_t)batch + 1, cu, (hipStream_t)stream)) != RLQ_OK) return st;
    if ((st = fetch_i32(start_pos, (size_t)batch, sp, (hipStream_t)stream)) != RLQ_OK) return st;
    if ((st = fetch_i32(block_table, (size_t)batch * max_pages_per_req, bt, (hipStream_t)stream)) != RLQ_OK)
      return st;
    st = rlq_check_append_tables(batch, cu.data(), sp.data(), bt.data(), max_pages_per_req, cache->num_pages,
                                 n_tokens);
    if (st != RLQ_OK) return st;
  }
  if (n_tokens == 0) return RLQ_OK;

  rlq::AppendArgs a;
  a.latent = latent_bf16;
  a.latent_rot = latent_rot_f32;
  a.rotation = rotation_bf16;
  a.k_rope = k_rope_bf16;
  a.cu_seqlens = cu_seqlens;
  a.start_pos = start_pos;
  a.block_table = block_table;
  a.max_pages = max_pages_per_req;
  a.batch = batch;
  a.n_tokens = n_tokens;
  a.codes = cache->codes;
  a.meta = cache->meta;
  a.rope = cache->rope;
  a.sink = cache->sink;
  a.recent = cache->recent;
  a.n_sink = cache->sink ? cache->n_sink : 0;
  a.n_recent = cache->recent ? cache->n_recent : 0;
  a.tau = p->tau;
  a.z_debug = z_debug;
  return hip_status(rlq::launch_append(a, (hipStream_t)stream));
}

// The 16-head kernel launches one workgroup row per (request, head group) in
// a grid dimension of at most 65535; the many-head kernel has no such bound.
static bool decode_shape(int32_t batch, int32_t heads) {
  if (batch < 1 || heads < 16 || heads > RLQ_MAX_HEADS || heads % 16) return false;
  return rlq::use_wide(heads) || (int64_t)batch * (heads / 16) <= 65535;
}

int rlq_mla_decode_workspace_size(int32_t batch, int32_t heads, int32_t max_ctx_len,
                                  size_t *bytes) {
  if (bytes == nullptr || !decode_shape(batch, heads) || max_ctx_len < 0 || max_ctx_len > RLQ_MAX_CTX)
    return RLQ_EINVAL;
  *bytes = rlq::use_wide(heads)
               ? rlq::wide_workspace_bytes(batch, heads, rlq::plan_wide(batch, heads, max_ctx_len))
               : rlq::decode_workspace_bytes(batch, heads, rlq::plan_splits(batch, heads, max_ctx_len));
  return RLQ_OK;
}

// The decode of rlq_mla_decode and rlq_mla_decode_noalloc.  With noalloc the
// workspace is this library's static scratch array on the current device,
// looked up only after every argument has been validated.
static int decode_call(const rlq_layer_params *p, const rlq_cache *cache,
                       const uint16_t *q_c_bf16, const uint16_t *q_r_bf16,
                       int32_t batch, int32_t heads, float sm_scale,
                       const int32_t *block_table, int32_t max_pages_per_req,
                       const int32_t *ctx_lens, int32_t max_ctx_len,
                       float *out, float *lse,
                       void *workspace, size_t workspace_bytes, bool noalloc, void *stream) {
  if (p == nullptr || !decode_shape(batch, heads)) return RLQ_EINVAL;
  if (max_ctx_len < 0 || max_ctx_len > RLQ_MAX_CTX || max_pages_per_req < 1 ||
      (int64_t)max_ctx_len > (int64_t)max_pages_per_req * RLQ_PAGE)
    return RLQ_EINVAL;
  int st = check_cache(cache, batch);
  if (st != RLQ_OK) return st;
  if (q_c_bf16 == nullptr || q_r_bf16 == nullptr || block_table == nullptr ||
      ctx_lens == nullptr || out == nullptr || (!noalloc && workspace == nullptr))
    return RLQ_EINVAL;
  if (!aligned(q_c_bf16, 16) || !aligned(q_r_bf16, 16) || !aligned(out, 16) ||
      (!noalloc && !aligned(workspace, 16)) || !aligned(block_table, 4) || !aligned(ctx_lens, 4) ||
      (lse != nullptr && !aligned(lse, 4)))
    return RLQ_EINVAL;
  const bool wide = rlq::use_wide(heads);
  const rlq::SplitPlan plan = rlq::plan_splits(batch, heads, max_ctx_len);
  const rlq::WidePlan wplan = rlq::plan_wide(batch, heads, max_ctx_len);
  const size_t need = wide ? rlq::wide_workspace_bytes(batch, heads, wplan)
                           : rlq::decode_workspace_bytes(batch, heads, plan);
  if (noalloc) workspace_bytes = RLQ_NOALLOC_SCRATCH_BYTES;
  if (workspace_bytes < need) return RLQ_ENOSPC;
  st = check_device();
  if (st != RLQ_OK) return st;
  if (debug_checks()) {
    std::vector<int32_t> cl, bt;
    if ((st = fetch_i32(ctx_lens, (size_t)batch, cl, (hipStream_t)stream)) != RLQ_OK) return st;
    if ((st = fetch_i32(block_table, (size_t)batch * max_pages_per_req, bt, (hipStream_t)stream)) != RLQ_OK)
      return st;
    st = rlq_check_decode_tables(batch, cl.data(), bt.data(), max_pages_per_req, cache->num_pages, max_ctx_len);
    if (st != RLQ_OK) return st;
  }
  if (noalloc) {
    st = scratch_ptr(&workspace);
    if (st != RLQ_OK) return st;
  }

  rlq::DecodeArgs a;
  a.codes = cache->codes;
  a.meta = cache->meta;
  a.rope = cache->rope;
  a.sink = cache->sink;
  a.recent = cache->recent;
  a.n_sink = cache->sink ? cache->n_sink : 0;
  a.n_recent = cache->recent ? cache->n_recent : 0;
  a.q_c = q_c_bf16;
  a.q_r = q_r_bf16;
  a.block_table = block_table;
  a.max_pages = max_pages_per_req;
  a.ctx_lens = ctx_lens;
  a.heads = heads;
  a.tokens_per_split = plan.tokens_per_split;
  a.splits = plan.splits;
  a.prot = ((a.sink != nullptr && a.n_sink > 0) || (a.recent != nullptr && a.n_recent > 0)) ? 1 : 0;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.gain = p->gain;
  a.level_inner = p->level_inner;
  a.level_outer = p->level_outer;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.max_ctx_len = max_ctx_len;
  a.item_slots = wplan.item_slots;
  a.item_target = wplan.item_target;
  a.cu_q = nullptr;
  a.q_heads = heads;
  a.force_xch_timeout = force_exchange_timeout() ? 1 : 0;
  a.spin_limit = a.force_xch_timeout ? 2 : (1 << 16);
  if (wide) {
    // Many heads: balanced work items, each 32-token tile decoded once per 64 heads.
    rlq::wide_workspace_layout(a, workspace, batch, heads, wplan);
    return hip_status(rlq::launch_decode_wide(a, batch, (hipStream_t)stream));
  }
  const size_t parts = (size_t)batch * (heads / 16) * (plan.splits + a.prot);
  a.part_o = (float *)workspace;
  a.part_ml = a.part_o + parts * rlq::kPartialFloats;
  a.plan = nullptr;
  return hip_status(rlq::launch_decode(a, batch, (hipStream_t)stream));
}

int rlq_mla_decode(const rlq_layer_params *p, const rlq_cache *cache,
                   const uint16_t *q_c_bf16, const uint16_t *q_r_bf16,
                   int32_t batch, int32_t heads, float sm_scale,
                   const int32_t *block_table, int32_t max_pages_per_req,
                   const int32_t *ctx_lens, int32_t max_ctx_len,
                   float *out, float *lse,
                   void *workspace, size_t workspace_bytes, void *stream) {
  return decode_call(p, cache, q_c_bf16, q_r_bf16, batch, heads, sm_scale, block_table, max_pages_per_req,
                     ctx_lens, max_ctx_len, out, lse, workspace, workspace_bytes, false, stream);
}

int rlq_mla_decode_noalloc(const rlq_layer_params *p, const rlq_cache *cache,
                           const uint16_t *q_c_bf16, const uint16_t *q_r_bf16,
                           int32_t batch, int32_t heads, float sm_scale,
                           const int32_t *block_table, int32_t max_pages_per_req,
                           const int32_t *ctx_lens, int32_t max_ctx_len,
                           float *out, float *lse, void *stream) {
  return decode_call(p, cache, q_c_bf16, q_r_bf16, batch, heads, sm_scale, block_table, max_pages_per_req,
                     ctx_lens, max_ctx_len, out, lse, nullptr, 0, true, stream);
}

// Extend: the many-head kernel over (query, head) rows, the rows of the
// largest request padded to a multiple of 64.
static bool extend_shape(int32_t batch, int32_t heads, int32_t max_q_len, int32_t max_ctx_len,
                         int64_t *rows) {
  if (batch < 1 || heads < 16 || heads > RLQ_MAX_HEADS || heads % 16 || max_q_len < 1 ||
      max_ctx_len < 0 || max_ctx_len > RLQ_MAX_CTX || max_q_len > max_ctx_len)
    return false;
  *rows = rlq::extend_rows(max_q_len, heads);
  return *rows / 64 <= 65535 && (int64_t)batch * (*rows / 16) <= (int64_t)1 << 30;
}

int rlq_mla_extend_workspace_size(int32_t batch, int32_t heads, int32_t max_q_len,
                                  int32_t max_ctx_len, size_t *bytes) {
  int64_t rows;
  if (bytes == nullptr || !extend_shape(batch, heads, max_q_len, max_ctx_len, &rows)) return RLQ_EINVAL;
  *bytes = rlq::wide_workspace_bytes(batch, (int32_t)rows, rlq::plan_wide(batch, (int32_t)rows, max_ctx_len));
  return RLQ_OK;
}

int rlq_mla_extend(const rlq_layer_params *p, const rlq_cache *cache,
                   const uint16_t *q_c_bf16, const uint16_t *q_r_bf16,
                   const int32_t *cu_seqlens_q, int32_t batch, int32_t heads,
                   int32_t max_q_len, float sm_scale,
                   const int32_t *block_table, int32_t max_pages_per_req,
                   const int32_t *ctx_lens, int32_t max_ctx_len,
                   float *out, float *lse,
                   void *workspace, size_t workspace_bytes, void *stream) {
  int64_t rows;
  if (p == nullptr || !extend_shape(batch, heads, max_q_len, max_ctx_len, &rows)) return RLQ_EINVAL;
  if (max_pages_per_req < 1 || (int64_t)max_ctx_len > (int64_t)max_pages_per_req * RLQ_PAGE)
    return RLQ_EINVAL;
  int st = check_cache(cache, batch);
  if (st != RLQ_OK) return st;
  if (q_c_bf16 == nullptr || q_r_bf16 == nullptr || cu_seqlens_q == nullptr || block_table == nullptr ||
      ctx_lens == nullptr || out == nullptr || workspace == nullptr)
    return RLQ_EINVAL;
  if (!aligned(q_c_bf16, 16) || !aligned(q_r_bf16, 16) || !aligned(out, 16) ||
      !aligned(workspace, 16) || !aligned(block_table, 4) || !aligned(ctx_lens, 4) ||
      !aligned(cu_seqlens_q, 4) || (lse != nullptr && !aligned(lse, 4)))
    return RLQ_EINVAL;
  const rlq::WidePlan wplan = rlq::plan_wide(batch, (int32_t)rows, max_ctx_len);
  if (workspace_bytes < rlq::wide_workspace_bytes(batch, (int32_t)rows, wplan)) return RLQ_ENOSPC;
  st = check_device();
  if (st != RLQ_OK) return st;
  if (debug_checks()) {
    std::vector<int32_t> cq, cl, bt;
    if ((st = fetch_i32(cu_seqlens_q, (size_t)batch + 1, cq, (hipStream_t)stream)) != RLQ_OK) return st;
    if ((st = fetch_i32(ctx_lens, (size_t)batch, cl, (hipStream_t)stream)) != RLQ_OK) return st;
    if ((st = fetch_i32(block_table, (size_t)batch * max_pages_per_req, bt, (hipStream_t)stream)) != RLQ_OK)
      return st;
    st = rlq_check_extend_tables(batch, cq.data(), cl.data(), bt.data(), max_pages_per_req, cache->num_pages,
                                 max_q_len, max_ctx_len);
    if (st != RLQ_OK) return st;
  }

  rlq::DecodeArgs a;
  a.codes = cache->codes;
  a.meta = cache->meta;
  a.rope = cache->rope;
  a.sink = cache->sink;
  a.recent = cache->recent;
  a.n_sink = cache->sink ? cache->n_sink : 0;
  a.n_recent = cache->recent ? cache->n_recent : 0;
  a.q_c = q_c_bf16;
  a.q_r = q_r_bf16;
  a.block_table = block_table;
  a.max_pages = max_pages_per_req;
  a.ctx_lens = ctx_lens;
  a.heads = (int32_t)rows;
  a.tokens_per_split = 0;
  a.splits = 0;
  a.prot = ((a.sink != nullptr && a.n_sink > 0) || (a.recent != nullptr && a.n_recent > 0)) ? 1 : 0;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.gain = p->gain;
  a.level_inner = p->level_inner;
  a.level_outer = p->level_outer;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.max_ctx_len = max_ctx_len;
  a.item_slots = wplan.item_slots;
  a.item_target = wplan.item_target;
  a.cu_q = cu_seqlens_q;
  a.q_heads = heads;
  a.force_xch_timeout = 0;
  a.spin_limit = 1 << 16;
  rlq::wide_workspace_layout(a, workspace, batch, (int32_t)rows, wplan);
  return hip_status(rlq::launch_decode_wide(a, batch, (hipStream_t)stream));
}

}  // extern "C"
