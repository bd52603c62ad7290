/*
 * rlq.h - C ABI of librlq: RoLaQ-style 2-bit MLA latent cache on MI355X (gfx950).
 *
 * The library implements the data-parallel hot path of a 2-bit Multi-Head
 * Latent Attention cache as described in "RoLaQ: Joint Rotation and Range
 * Calibration for 2-Bit KV Caches in Multi-Head Latent Attention":
 *
 *   rlq_quantize_append  write side: rotate each token's content latent by the
 *                        fixed shared rotation (§3.3), standardize every
 *                        128-coordinate group with an fp32 mean and scale
 *                        (§A.3), assign each coordinate one of four levels by
 *                        the per-layer threshold tau (§3.2), pack the 2-bit
 *                        codes and copy the BF16 RoPE key (§2.1, §A.3);
 *                        optionally keep sink/recent tokens in BF16 (§4.1).
 *   rlq_mla_decode       read side: absorbed-MLA decode attention over the
 *                        paged cache; reconstruction = group mean + scale *
 *                        gain * level (§3.2); scores q_c.c_hat + q_R.k_R with
 *                        the read-side rotation folded into the absorbed query
 *                        (§3.3, Fig. 3a); softmax; output in latent space.
 *   rlq_mla_extend       prefill / extend: each request's newest tokens attend
 *                        causally to the same cache (§D: the method serves
 *                        prefill and decode from its cache).
 *
 * Storage per unprotected token and layer: 128 B codes + 32 B fp32 group
 * statistics + 128 B BF16 RoPE key = 288 B (§A.3; the storage-accounting
 * notebook "What does a 2-bit KV cache actually store?").
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers marked "device" are HIP device pointers; the caller allocates
 *    and owns them.  The library allocates nothing, keeps no pointer after a
 *    call returns and never synchronizes: work is enqueued on `stream` and the
 *    caller keeps every buffer alive until the stream has completed it.  Its
 *    only process-wide state is a per-device "is gfx950" check result, the
 *    one-time LDS-size attributes of the decode and bulk-append kernels, all set
 *    on first use, and the static scratch array of rlq_mla_decode_noalloc (one
 *    per device, part of the loaded code object).
 *  - Device pointers must be 16-byte aligned and their arrays contiguous in
 *    the layouts given below.
 *  - Each call returns an RLQ_* status.  Host-side validation runs before any
 *    launch; on error nothing is enqueued.  A launch failure reported by the
 *    HIP runtime returns RLQ_EHIP (text via rlq_last_hip_error()).
 *  - Values that live in device memory (block tables, lengths, positions) are
 *    trusted: out-of-range entries are undefined behaviour.  With the
 *    environment variable RLQ_DEBUG set (to anything but "0"), the decode,
 *    extend and append calls first copy them to the host (synchronizing their
 *    stream, so not under graph capture) and return RLQ_EINVAL, with nothing
 *    launched, if one is out of range (the rlq_check_*_tables rules below).
 *  - The 16-head decode kernel's two waves of a pair exchange partial scores
 *    through LDS with a bounded wait; a wave that gives up (which needs a
 *    partner stalled for milliseconds) marks its workgroup's partial, and the
 *    affected rows of out and lse come out NaN instead of a silently wrong
 *    value.  RLQ_TEST_EXCHANGE_TIMEOUT (anything but "0") forces that path
 *    for tests; every kernel still completes.
 *  - Calls on one stream run in order; calls that overlap on different
 *    streams must not write the same cache slots.
 *  - Values: content latents must stay within the fp16 range (|x| < 65504);
 *    non-finite inputs are outside the method's domain.
 */
#ifndef RLQ_H
#define RLQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RLQ_ABI_VERSION 1

/* Status codes. */
enum {
  RLQ_OK = 0,
  RLQ_EINVAL = -1,        /* bad argument: null/misaligned pointer, bad size      */
  RLQ_EUNSUPPORTED = -2,  /* current device is not gfx950                          */
  RLQ_ENOSPC = -3,        /* workspace too small                                   */
  RLQ_EHIP = -4           /* HIP runtime error while launching                     */
};

/* Fixed dimensions (DeepSeek-V2-Lite MLA: latent 512, RoPE 64; group 128). */
#define RLQ_DC 512        /* content latent width d_c                              */
#define RLQ_DR 64         /* RoPE key width d_R                                    */
#define RLQ_GROUP 128     /* coordinates per (mean, scale) group                   */
#define RLQ_NGROUPS 4     /* groups per token                                      */
#define RLQ_PAGE 64       /* tokens per cache page                                 */
#define RLQ_WORDS 32      /* uint32 code words per token (16 codes per word)       */
#define RLQ_MAX_HEADS 128
#define RLQ_MAX_CTX 4194304  /* longest context one decode call accepts (tokens)  */
#define RLQ_NOALLOC_SCRATCH_BYTES (64u << 20)  /* static scratch of rlq_mla_decode_noalloc */

/*
 * Per-layer quantizer parameters, fixed while serving (§3.3).
 *   tau          threshold on the standardized coordinate (§3.2, §C.3);
 *                finite and >= 0 (rlq_quantize_append returns RLQ_EINVAL
 *                otherwise)
 *   gain         reconstruction gain around the group mean (§3.2, §B.3)
 *   level_inner  a, level_outer b: the four levels are -b, -a, +a, +b
 * Defaults (rlq_layer_params_default): the four-level Lloyd-Max quantizer for
 * a unit Gaussian, tau 0.9816, levels 0.4528 / 1.510, gain 1 (the initial
 * threshold named in §C.3 and Fig. 8).
 */
typedef struct {
  float tau;
  float gain;
  float level_inner;
  float level_outer;
} rlq_layer_params;

/*
 * Paged cache of one layer (device memory, caller-owned).
 *   codes   uint32 [num_pages][64][32]  2-bit codes, 16 per word; coordinate
 *                                       j of a token is word j/16, bits
 *                                       2*(j%16) .. 2*(j%16)+1; code 0,1,2,3 =
 *                                       level -b, -a, +a, +b
 *   meta    float  [num_pages][64][8]   mu_0..mu_3, s_0..s_3 per token
 *   rope    uint16 [num_pages][64][64]  BF16 RoPE key per token
 *   sink    uint16 [max_batch][n_sink][512]   BF16 rotated latent of positions
 *                                       0..n_sink-1 of each request, or NULL
 *   recent  uint16 [max_batch][n_recent][512] BF16 rotated latent ring; the
 *                                       token at position p sits in slot
 *                                       p % n_recent; or NULL
 *   page_size must be 64.  Protection (§4.1, §A.3): with sink/recent given,
 *   decode reads those tokens' content from them instead of the codes.
 */
typedef struct {
  uint32_t *codes;
  float *meta;
  uint16_t *rope;
  int32_t num_pages;
  int32_t page_size;
  uint16_t *sink;
  uint16_t *recent;
  int32_t n_sink;
  int32_t n_recent;
  int32_t max_batch;
} rlq_cache;

/* Library ABI version (RLQ_ABI_VERSION). */
int rlq_abi_version(void);

/* Default quantizer parameters (see rlq_layer_params). */
rlq_layer_params rlq_layer_params_default(void);

/* Static text for a status code. */
const char *rlq_status_string(int status);

/* Text of the last HIP error seen by this thread inside the library ("" if none). */
const char *rlq_last_hip_error(void);

/*
 * Gain linked to tau for unit response of the centred signal (§3.2, §B.3),
 * for x ~ N(0,1):  g(tau) = 1 / (2 (a phi(0) + (b - a) phi(tau))).
 * Host-only helper; returns NaN for non-positive levels.
 */
float rlq_coupled_gain(float tau, float level_inner, float level_outer);

/*
 * Host-side checks of the device-resident tables, on host copies of them
 * (the RLQ_DEBUG checks; callers may also use them directly).  Each returns
 * RLQ_OK or RLQ_EINVAL.
 *   rlq_check_decode_tables   every 0 <= ctx_lens[b] <= max_ctx_len, and the
 *                             page ids of positions 0 .. ctx_lens[b]-1 lie in
 *                             [0, num_pages) within max_pages_per_req columns
 *   rlq_check_append_tables   cu_seqlens[0] = 0, non-decreasing, cu_seqlens
 *                             [batch] = n_tokens; start_pos[b] >= 0; the page
 *                             ids of the new positions in range as above
 *   rlq_check_extend_tables   the decode rules, cu_seqlens_q[0] = 0 and every
 *                             0 <= n_q <= min(max_q_len, ctx_lens[b])
 * Arrays: ctx_lens, start_pos [batch]; cu_seqlens, cu_seqlens_q [batch+1];
 * block_table [batch][max_pages_per_req] (host memory).
 */
int rlq_check_decode_tables(int32_t batch, const int32_t *ctx_lens, const int32_t *block_table,
                            int32_t max_pages_per_req, int32_t num_pages, int32_t max_ctx_len);
int rlq_check_append_tables(int32_t batch, const int32_t *cu_seqlens, const int32_t *start_pos,
                            const int32_t *block_table, int32_t max_pages_per_req, int32_t num_pages,
                            int64_t n_tokens);
int rlq_check_extend_tables(int32_t batch, const int32_t *cu_seqlens_q, const int32_t *ctx_lens,
                            const int32_t *block_table, int32_t max_pages_per_req, int32_t num_pages,
                            int32_t max_q_len, int32_t max_ctx_len);

/*
 * rlq_quantize_append - append new tokens of `batch` requests to the cache.
 *
 * Request b owns new tokens cu_seqlens[b] .. cu_seqlens[b+1]-1; its i-th new
 * token lands at position p = start_pos[b] + i, in page block_table[b][p / 64]
 * slot p % 64.  For every token:
 *   z     = R c (fp32), or the given already-rotated latent;
 *   mu_g  = S(z_g) / 128, d = z - mu_g, s_g = sqrt(S(d*d) / 128), where S is
 *           the fp32 adjacent-pair tree sum over the group, d*d is a plain
 *           fp32 product and sqrt is correctly rounded;
 *   code  = [d >= -t] + [d >= 0] + [d >= t] with t = fl32(tau * s_g);
 * and codes, meta, rope are written.  With cache->sink, positions p < n_sink
 * also write sink[b][p] = bf16(z); with cache->recent, the last n_recent
 * positions of the request after this append write recent[b][p % n_recent].
 *
 *   p              layer parameters (host pointer; tau used here)
 *   cache          cache descriptor (host pointer to device pools)
 *   latent_bf16    device [n_tokens][512] BF16 content latents, or NULL
 *   latent_rot_f32 device [n_tokens][512] fp32 rotated latents z, or NULL;
 *                  exactly one of latent_bf16 / latent_rot_f32 is non-NULL
 *   rotation_bf16  device [512][512] BF16 rotation R (row = output),
 *                  required with latent_bf16, ignored otherwise
 *   k_rope_bf16    device [n_tokens][64] BF16 RoPE keys
 *   cu_seqlens     device int32 [batch+1], cu_seqlens[0] = 0, non-decreasing
 *   start_pos      device int32 [batch], tokens already cached per request
 *   block_table    device int32 [batch][max_pages_per_req] page ids
 *   batch          number of requests, 1 .. max_batch when protection is on
 *   n_tokens       host copy of cu_seqlens[batch] (sizes the launch; 0 = no-op)
 *   z_debug        device [n_tokens][512] fp32 dump of z, or NULL
 *
 * With latent_bf16 the rotation runs as a bf16 MFMA product with fp32
 * accumulation; with identity or signed-permutation R every z is exact.
 * Errors: RLQ_EINVAL (null/misaligned pointers, page_size != 64, batch < 1,
 * n_tokens < 0, both or neither latent given, protection buffers without
 * max_batch >= batch), RLQ_EUNSUPPORTED, RLQ_EHIP.
 */
int rlq_quantize_append(const rlq_layer_params *p, const rlq_cache *cache,
                        const uint16_t *latent_bf16, const float *latent_rot_f32,
                        const uint16_t *rotation_bf16, const uint16_t *k_rope_bf16,
                        const int32_t *cu_seqlens, const int32_t *start_pos,
                        const int32_t *block_table, int32_t max_pages_per_req,
                        int32_t batch, int64_t n_tokens, float *z_debug,
                        void *stream);

/*
 * Workspace (bytes) that rlq_mla_decode needs for this batch, head count and
 * maximum context length: split-KV partials (unnormalised output, running max
 * and sum per split and head) and, when heads is a multiple of 64, a table of
 * each request's work items (two int32 per request) followed by partials per
 * work-item slot and 32 heads (64 KB + 256 bytes), which are left out when
 * every request is one work item (batch * heads / 64 >= 512 and max_ctx_len
 * <= 49,088: the requests' rows are then written directly).  Errors: RLQ_EINVAL (also
 * for max_ctx_len above RLQ_MAX_CTX, and for batch * heads / 16 above 65535
 * when heads is not a multiple of 64).
 */
int rlq_mla_decode_workspace_size(int32_t batch, int32_t heads, int32_t max_ctx_len,
                                  size_t *bytes);

/*
 * rlq_mla_decode - one decode step of absorbed MLA attention over the cache.
 *
 * For request b and head h, over positions t < ctx_lens[b]:
 *   c_hat_t = mu + s * gain * L[code]    (or the BF16 sink/recent latent)
 *   s_t     = sm_scale * (q_c[b,h] . c_hat_t + q_r[b,h] . k_R_t)
 *   out     = sum_t softmax(s)_t c_hat_t,   lse = ln sum_t exp(s_t)
 * Tokens t < n_sink read sink[b][t]; tokens t >= ctx_len - n_recent read
 * recent[b][t % n_recent] (when those buffers are given); the RoPE key always
 * comes from rope.  With protection the ring must hold the request's last
 * n_recent tokens, i.e. ctx_lens[b] equals the cached length.
 *
 *   q_c_bf16       device [batch][heads][512] absorbed content queries (BF16),
 *                  already in the rotated basis
 *   q_r_bf16       device [batch][heads][64] RoPE queries (BF16)
 *   heads          multiple of 16, at most 128 (a multiple of 64 runs the
 *                  many-head kernel: each token decoded once per 64 heads,
 *                  work items balanced over ctx_lens on the device; other
 *                  counts run the 16-head kernel, which takes at most 65535
 *                  (request, 16-head group) pairs per call)
 *   sm_scale       softmax scale
 *   block_table    device int32 [batch][max_pages_per_req]
 *   ctx_lens       device int32 [batch], 0 <= ctx_lens[b] <= max_ctx_len
 *   max_ctx_len    host bound on ctx_lens (sizes the split grid), at most
 *                  RLQ_MAX_CTX
 *   out            device fp32 [batch][heads][512]
 *   lse            device fp32 [batch][heads] natural-log LSE, or NULL
 *   workspace      device scratch of at least rlq_mla_decode_workspace_size()
 *                  bytes; its contents need no initialisation
 * ctx_lens[b] = 0 gives out = 0 and lse = -inf.
 * Errors: RLQ_EINVAL (pointers, heads, batch, max_ctx_len beyond the block
 * table or above RLQ_MAX_CTX), RLQ_ENOSPC, RLQ_EUNSUPPORTED, RLQ_EHIP.
 */
int rlq_mla_decode(const rlq_layer_params *p, const rlq_cache *cache,
                   const uint16_t *q_c_bf16, const uint16_t *q_r_bf16,
                   int32_t batch, int32_t heads, float sm_scale,
                   const int32_t *block_table, int32_t max_pages_per_req,
                   const int32_t *ctx_lens, int32_t max_ctx_len,
                   float *out, float *lse,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * rlq_mla_decode_noalloc - rlq_mla_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation and kernels, with the
 * workspace taken from a static array of RLQ_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds on each device it runs on until the process ends.
 * Arguments as for rlq_mla_decode without workspace / workspace_bytes; the
 * caller still passes the inputs and outputs.  Nothing is allocated: the
 * array's device address is looked up once per device.
 * Calls that overlap on one device (concurrent streams, or threads) share the
 * array and race; serialize them.  The array needs no initialisation.
 * Errors: as rlq_mla_decode; RLQ_ENOSPC when rlq_mla_decode_workspace_size()
 * for these arguments exceeds RLQ_NOALLOC_SCRATCH_BYTES (e.g. batch 2 at
 * RLQ_MAX_CTX with 128 heads needs 46 MB, which fits).
 */
int rlq_mla_decode_noalloc(const rlq_layer_params *p, const rlq_cache *cache,
                           const uint16_t *q_c_bf16, const uint16_t *q_r_bf16,
                           int32_t batch, int32_t heads, float sm_scale,
                           const int32_t *block_table, int32_t max_pages_per_req,
                           const int32_t *ctx_lens, int32_t max_ctx_len,
                           float *out, float *lse, void *stream);

/*
 * Workspace (bytes) that rlq_mla_extend needs: the work-item table (two int32
 * per request, padded to 256 bytes) and, when a request can span several work
 * items, split partials for (query, head) rows, max_q_len * heads rows
 * rounded up to 64 per request.  With batch * rows / 64 >= 512 and
 * max_ctx_len <= 49,088 every request is one work item and writes its rows
 * directly: the table alone (e.g. 4 requests of 8192 queries).  Otherwise the
 * partials take 64 KB + 256 bytes per 32 rows and work-item slot.  Errors:
 * RLQ_EINVAL (heads, batch, max_q_len < 1, max_ctx_len above RLQ_MAX_CTX, or
 * a row count beyond the launch limits: rows / 64 at most 65535 and
 * batch * rows / 16 at most 2^30).
 */
int rlq_mla_extend_workspace_size(int32_t batch, int32_t heads, int32_t max_q_len,
                                  int32_t max_ctx_len, size_t *bytes);

/*
 * rlq_mla_extend - prefill / extend attention of many new query tokens per
 * request over the cache ([RoLaQ] §D: the method serves prefill and decode
 * with kernels that read its cache; the attention itself is that of
 * rlq_mla_decode, §2.1, §3.2, §3.3).
 *
 * The new tokens are appended first (rlq_quantize_append), so request b's
 * cache holds ctx_lens[b] tokens and its n_q = cu_seqlens_q[b+1] -
 * cu_seqlens_q[b] queries are its last n_q positions: query i sits at
 * position p = ctx_lens[b] - n_q + i and attends causally to positions
 * 0 .. p, each read exactly as rlq_mla_decode reads it (sink and recent BF16
 * rows as the cache holds them after the append, i.e. the recent window is
 * the last n_recent positions of ctx_lens[b]).  For query row r = cu_q[b] + i
 * and head h:
 *   out[r][h] = sum_{t <= p} softmax(s)_t c_hat_t,   lse[r][h] = ln sum exp(s_t)
 * with s_t as in rlq_mla_decode.  n_q = 1 is the decode of the last token.
 *
 *   q_c_bf16       device [total_q][heads][512] absorbed content queries,
 *                  total_q = cu_seqlens_q[batch]
 *   q_r_bf16       device [total_q][heads][64] RoPE queries
 *   cu_seqlens_q   device int32 [batch+1], cu_seqlens_q[0] = 0, with
 *                  0 <= n_q <= min(ctx_lens[b], max_q_len) per request
 *   heads          multiple of 16, at most 128
 *   max_q_len      host bound on n_q (sizes the grid)
 *   block_table, ctx_lens, max_ctx_len, sm_scale   as in rlq_mla_decode
 *   out            device fp32 [total_q][heads][512]
 *   lse            device fp32 [total_q][heads], or NULL
 *   workspace      device scratch of rlq_mla_extend_workspace_size() bytes
 * Device-resident counts are trusted (as for decode): n_q above max_q_len or
 * ctx_lens[b] is undefined behaviour.
 * Errors: RLQ_EINVAL, RLQ_ENOSPC, RLQ_EUNSUPPORTED, RLQ_EHIP.
 */
int rlq_mla_extend(const rlq_layer_params *p, const rlq_cache *cache,
                   const uint16_t *q_c_bf16, const uint16_t *q_r_bf16,
                   const int32_t *cu_seqlens_q, int32_t batch, int32_t heads,
                   int32_t max_q_len, float sm_scale,
                   const int32_t *block_table, int32_t max_pages_per_req,
                   const int32_t *ctx_lens, int32_t max_ctx_len,
                   float *out, float *lse,
                   void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RLQ_H */
