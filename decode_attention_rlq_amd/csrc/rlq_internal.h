// Internal declarations shared by the librlq translation units (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "rlq.h"

namespace rlq {

// A one-time set-up step (a kernel attribute) run once per device, safe when
// several host threads launch at once.
struct PerDeviceOnce {
  std::mutex m;
  bool done[64] = {};
};
template <class F>
hipError_t once_per_device(PerDeviceOnce &o, F &&f) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(o.m);
  if (!o.done[dev]) {
    e = f();
    if (e != hipSuccess) return e;
    o.done[dev] = true;
  }
  return hipSuccess;
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- append

struct AppendArgs {
  const uint16_t *latent;      // [N][512] bf16, or null
  const float *latent_rot;     // [N][512] fp32, or null
  const uint16_t *rotation;    // [512][512] bf16
  const uint16_t *k_rope;      // [N][64] bf16
  const int32_t *cu_seqlens;   // [B+1]
  const int32_t *start_pos;    // [B]
  const int32_t *block_table;  // [B][max_pages]
  int32_t max_pages;
  int32_t batch;
  int64_t n_tokens;
  uint32_t *codes;
  float *meta;
  uint16_t *rope;
  uint16_t *sink;
  uint16_t *recent;
  int32_t n_sink;
  int32_t n_recent;
  float tau;
  float *z_debug;
};

hipError_t launch_append(const AppendArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- decode

// Tokens of one wave iteration and of one score tile.
constexpr int kChunk = 32;
constexpr int kTile = 16;
constexpr int kDecodeWaves = 8;
constexpr int kDecodeThreads = 64 * kDecodeWaves;
// Per-(request, head group, split) partial: 16 heads x 512 latent fp32 in the
// accumulator's own order, then (max, sum) per head.
constexpr int kPartialFloats = 16 * RLQ_DC;
// Upper bound on splits per request (the merge keeps one weight per split).
constexpr int kMaxSplits = 256;
// Upper bound on pages per split (their ids are staged in LDS); together with
// kMaxSplits it bounds the context length at RLQ_MAX_CTX tokens.
constexpr int kMaxSplitPages = 256;
static_assert((int64_t)kMaxSplits * kMaxSplitPages * RLQ_PAGE == RLQ_MAX_CTX, "context bound");

struct DecodeArgs {
  const uint32_t *codes;
  const float *meta;
  const uint16_t *rope;
  const uint16_t *sink;
  const uint16_t *recent;
  int32_t n_sink;
  int32_t n_recent;
  const uint16_t *q_c;
  const uint16_t *q_r;
  const int32_t *block_table;
  int32_t max_pages;
  const int32_t *ctx_lens;
  int32_t heads;
  int32_t tokens_per_split;
  int32_t splits;
  int32_t prot;      // 1 if sink/recent buffers are given (one more partial per request)
  float scale_log2;  // sm_scale * log2(e)
  float gain;
  float level_inner;
  float level_outer;
  float *part_o;   // [B][HG][S+prot][kPartialFloats]
  float *part_ml;  // [B][HG][S+prot][16][2]
  float *out;      // [B][H][512]
  float *lse;      // [B][H] or null
  // Many-head path (heads a multiple of kWideHeads) only.
  int32_t batch;
  int32_t max_ctx_len;
  int32_t item_slots;   // workgroups per 64-head group: work items at most
  int32_t item_target;  // work items the balanced plan aims for
  int32_t *plan;        // [B][2]: first work item and item count of each request
  // Extend (many query tokens per request): null for decode.  Request b's
  // query rows are (query i, head h) for i < cu_q[b+1] - cu_q[b], stored from
  // row cu_q[b] * q_heads; `heads` is then the padded row count of the
  // largest request (a multiple of 64).
  const int32_t *cu_q;
  int32_t q_heads;
  // Bounded wait of the 16-head kernel's partial-score exchange: polls before
  // a wave gives up (and marks its partial NaN), and a test switch that makes
  // every poll find its slot empty.
  int32_t spin_limit;
  int32_t force_xch_timeout;
};

// Split policy shared by the workspace query and the launch.
struct SplitPlan {
  int32_t tokens_per_split;
  int32_t splits;
  int32_t prot;      // 1 if sink/recent buffers are given (one more partial per request)
};
SplitPlan plan_splits(int32_t batch, int32_t heads, int32_t max_ctx_len);
size_t decode_workspace_bytes(int32_t batch, int32_t heads, const SplitPlan &plan);

hipError_t launch_decode(const DecodeArgs &a, int32_t batch, hipStream_t stream);

// Many-head path: heads per workgroup, workgroups resident at once (one per
// CU), and the bounds of a work item (a run of 32-token tiles of one request).
constexpr int kWideHeads = 64;
constexpr int kResidentWide = 256;
constexpr int kMinItemTiles = 16;
constexpr int kMaxItemPages = 768;
constexpr int kMaxItemTiles = 2 * (kMaxItemPages - 1);

inline bool use_wide(int32_t heads) { return heads % kWideHeads == 0; }

struct WidePlan {
  int32_t item_slots;
  int32_t item_target;
  int32_t partials;  // 1 if a request can span several items (partials + merge)
};
WidePlan plan_wide(int32_t batch, int32_t heads, int32_t max_ctx_len);
size_t wide_workspace_bytes(int32_t batch, int32_t heads, const WidePlan &plan);
// Points a.plan / a.part_o / a.part_ml into a workspace of
// wide_workspace_bytes (part_o and part_ml null without partials).
void wide_workspace_layout(DecodeArgs &a, void *workspace, int32_t batch, int32_t heads, const WidePlan &plan);
hipError_t launch_decode_wide(const DecodeArgs &a, int32_t batch, hipStream_t stream);

// Extend: the many-head kernel over (query, head) rows.  Padded row count of
// the largest request, and the grid limits it must respect.
int64_t extend_rows(int32_t max_q_len, int32_t heads);

}  // namespace rlq
