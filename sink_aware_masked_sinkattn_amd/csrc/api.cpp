// C ABI of the sink-aware masked attention library (declared in
// include/sinkattn.h): argument validation (host only, before any HIP call),
// workspace layout, and dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cmath>
#include <cstdint>

#include "../../include/sinkattn.h"
#include "mask_tiles.h"

typedef __bf16 bf16;

hipError_t launch_fwd_bf16_d64(const bf16* q, const bf16* k, const bf16* v, const float* sinks,
                               bf16* o, float* lse, const int* cu_seqlens, int batch, int seqlen,
                               int total_tokens, int heads_q, int heads_kv, int window,
                               int prefix, float scale, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16_d64(const bf16* q, const bf16* k, const bf16* v,
                                    const bf16* dout, const float* l_ws, const float* d_ws,
                                    float* dk_acc, float* dv_acc, const int* cu_seqlens,
                                    int batch, int seqlen, int rows_total, int heads_q,
                                    int heads_kv, int window, int prefix, float scale, bool fold,
                                    bf16* dk, bf16* dv, hipStream_t stream);
hipError_t launch_bwd_dq_bf16_d64(const bf16* q, const bf16* k, const bf16* v, const bf16* dout,
                                  const bf16* o, const float* lse, const float* sinks,
                                  float* ds_part, int ds_stride, float* l_ws, float* d_ws, float* dk_acc,
                                  float* dv_acc, bf16* dq, const int* cu_seqlens, int batch,
                                  int seqlen, int rows_total, int heads_q, int heads_kv, int window,
                                  int prefix, float scale, long long fold_row, float* fold_part,
                                  bool clear_acc, hipStream_t stream);
bool dkdv_accumulates(int batch, int seqlen, int heads_q, int heads_kv, int window, int prefix,
                      bool fold);
bool dq_prefix_fold(int seqlen, int group, int window, int prefix);
hipError_t launch_prefix_fold_add(const float* fold_part, float* dk_acc, float* dv_acc,
                                  bf16* dk, bf16* dv, float scale, const int* cu_seqlens,
                                  int batch, int seqlen, int heads_kv, int prefix, int ds_stride,
                                  long long fold_row, hipStream_t stream);
long long dkdv_prefix_fold_row(int window);
int dq_launch_tiles(int batch, int seqlen, int total_tokens, bool varlen, int group, int window,
                    int prefix);
hipError_t launch_fwd_f32(int head_dim, const float* q, const float* k, const float* v,
                          const float* sinks, float* o, float* lse, const int* cu_seqlens,
                          int batch, int seqlen, int total_tokens, int heads_q, int heads_kv,
                          int window, int prefix, float scale, hipStream_t stream);
hipError_t launch_bwd_f32(int head_dim, const float* q, const float* k, const float* v,
                          const float* dout, const float* l_ws, const float* d_ws, float* dq,
                          float* dk, float* dv, const int* cu_seqlens, int batch, int seqlen,
                          int total_tokens, int heads_q, int heads_kv, int window, int prefix,
                          float scale, bool do_dq, bool do_dkdv, hipStream_t stream);
hipError_t launch_bwd_pre(int head_dim, const float* o, const float* dout, const float* lse,
                          const float* sinks, const int* cu_seqlens, float* dsinks, float* d_ws,
                          float* l_ws, int batch, int seqlen, int rows_total, int heads_q,
                          int lse_head_stride, hipStream_t stream);
hipError_t launch_convert(const float* dk_acc, const float* dv_acc, bf16* dk, bf16* dv,
                          long long n_kv, float scale, const float* ds_part, int ds_used,
                          int ds_stride, int heads, float* dsinks, hipStream_t stream);
hipError_t launch_zero_f32(float* p, int n, hipStream_t stream);
hipError_t launch_decode_bf16_d64(const bf16* q, const bf16* k, const bf16* v,
                                  const int* cache_seqlens, const float* sinks, bf16* o,
                                  float* lse, float* workspace, int batch, int t_max, int heads_q,
                                  int heads_kv, int window, int prefix, float scale,
                                  hipStream_t stream);
size_t decode_workspace_bytes(int batch, int t_max, int heads_q, int heads_kv, int window,
                              int prefix);
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** out);
int fwd_key_tile(int window);
int dkdv_query_tile(int window);
hipError_t launch_grpo(const float* logp_new, const float* logp_old, const float* logp_ref,
                       const uint8_t* mask, const float* rewards, const int32_t* cu_seqlens,
                       float* loss, float* grad, float* advantages, void* workspace,
                       int num_rollouts, int group_size, int total_tokens, int kl_mode,
                       float eps_adv, float eps_clip, float beta, hipStream_t stream);
size_t grpo_workspace_bytes(int num_rollouts, int total_tokens);

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Dims {
  long long rows;      // B*T or N
  bool varlen;
};

// Shape / mask / dtype checks shared by fwd and bwd.  No HIP calls.
sinkattn_status check_problem(const sinkattn_problem* pb, Dims* dims) {
  if (!pb) return SINKATTN_ERR_NULL_POINTER;
  if (pb->dtype != SINKATTN_BF16 && pb->dtype != SINKATTN_FP32) return SINKATTN_ERR_UNSUPPORTED;
  if (pb->batch < 0 || pb->seqlen < 0 || pb->heads_q <= 0 || pb->heads_kv <= 0 ||
      pb->head_dim <= 0)
    return SINKATTN_ERR_BAD_SHAPE;
  if (pb->heads_q % pb->heads_kv != 0) return SINKATTN_ERR_BAD_SHAPE;
  if (pb->window < 0 || pb->prefix < 0) return SINKATTN_ERR_BAD_MASK;
  if (pb->dtype == SINKATTN_BF16 && pb->head_dim != 64) return SINKATTN_ERR_UNSUPPORTED;
  if (pb->dtype == SINKATTN_FP32 && pb->head_dim != 32 && pb->head_dim != 64)
    return SINKATTN_ERR_UNSUPPORTED;
  if (!(pb->softmax_scale > 0.0f) || pb->softmax_scale > 1.0e30f) return SINKATTN_ERR_BAD_SHAPE;
  dims->varlen = pb->cu_seqlens != nullptr;
  if (dims->varlen) {
    if (pb->total_tokens < 0) return SINKATTN_ERR_BAD_SHAPE;
    if (pb->batch > 0 && pb->seqlen == 0 && pb->total_tokens > 0) return SINKATTN_ERR_BAD_SHAPE;
    dims->rows = pb->total_tokens;
  } else {
    dims->rows = (long long)pb->batch * pb->seqlen;
  }
  // Row * stride products inside kernels are widened to size_t, but a tile
  // copy's lane offset (up to 8 rows of the row stride, in bytes) is 32-bit:
  // heads * head_dim * 2 bytes * 8 rows must stay below 2^31.
  if ((long long)pb->heads_q * pb->head_dim > (1LL << 24)) return SINKATTN_ERR_BAD_SHAPE;
  if (dims->rows > (1LL << 31) - 1) return SINKATTN_ERR_BAD_SHAPE;
  return SINKATTN_OK;
}

struct Workspace {
  size_t d_off, l_off, dk_off, dv_off, ds_off, fold_off, total;
  int ds_stride;   // slots per head for the parts of ds_h (bf16)
  bool fold;       // the window dQ kernel takes the prefix keys' rows past the fold row
};

// window and prefix as the kernels see them: clamped to the longest sequence
int clamped_window(const sinkattn_problem* pb) { return pb->window > pb->seqlen ? pb->seqlen : pb->window; }
int clamped_prefix(const sinkattn_problem* pb) { return pb->prefix > pb->seqlen ? pb->seqlen : pb->prefix; }

Workspace workspace_layout(const sinkattn_problem* pb, const Dims& dims) {
  Workspace w;
  const size_t rows = (size_t)dims.rows;
  const size_t stat = round_up(rows * (size_t)pb->heads_q * sizeof(float));
  const bool accum = pb->dtype == SINKATTN_BF16;   // fp32 path writes outputs directly
  const size_t kvacc = accum ? round_up(rows * pb->heads_kv * pb->head_dim * sizeof(float)) : 0;
  // per-workgroup parts of ds_h: one slot per (sequence, 32-row block) and
  // head, enough for every dQ kernel's query tiles
  const long long blocks32 = (long long)pb->batch * ((pb->seqlen + 31) / 32);
  w.ds_stride = accum ? (int)blocks32 : 0;
  const size_t ds = accum ? round_up((size_t)blocks32 * pb->heads_q * sizeof(float)) : 0;
  // prefix fold: per (kv head, slot) the block's dK and dV rows of the prefix keys
  const int prefix = clamped_prefix(pb);
  w.fold = accum && dq_prefix_fold(pb->seqlen, pb->heads_q / pb->heads_kv, clamped_window(pb), prefix);
  const size_t fold = w.fold ? round_up((size_t)blocks32 * pb->heads_kv * 2 * prefix *
                                        pb->head_dim * sizeof(float)) : 0;
  w.d_off = 0;
  w.l_off = stat;
  w.dk_off = 2 * stat;
  w.dv_off = w.dk_off + kvacc;
  w.ds_off = w.dv_off + kvacc;
  w.fold_off = w.ds_off + ds;
  w.total = w.fold_off + fold;
  return w;
}

sinkattn_status hip_status(hipError_t e) { return e == hipSuccess ? SINKATTN_OK : SINKATTN_ERR_HIP; }

// Decode problem checks.  No HIP calls.
sinkattn_status check_decode(const sinkattn_decode_problem* pb) {
  if (!pb) return SINKATTN_ERR_NULL_POINTER;
  if (pb->batch < 0 || pb->cache_capacity < 0 || pb->heads_q <= 0 || pb->heads_kv <= 0 ||
      pb->head_dim <= 0)
    return SINKATTN_ERR_BAD_SHAPE;
  if (pb->heads_q % pb->heads_kv != 0) return SINKATTN_ERR_BAD_SHAPE;
  if (pb->window < 0 || pb->prefix < 0) return SINKATTN_ERR_BAD_MASK;
  if (pb->head_dim != 64 || pb->heads_q / pb->heads_kv > 16) return SINKATTN_ERR_UNSUPPORTED;
  if (!(pb->softmax_scale > 0.0f) || pb->softmax_scale > 1.0e30f) return SINKATTN_ERR_BAD_SHAPE;
  if ((long long)pb->batch * pb->cache_capacity > (1LL << 31) - 1) return SINKATTN_ERR_BAD_SHAPE;
  // as for the training problem: 8 cache rows of one sequence in bytes fit 2^31
  if ((long long)pb->heads_q * pb->head_dim > (1LL << 24)) return SINKATTN_ERR_BAD_SHAPE;
  return SINKATTN_OK;
}

int clamp_window(int window, int capacity) { return window > capacity ? capacity : window; }

}  // namespace

extern "C" {

const char* sinkattn_status_string(sinkattn_status s) {
  switch (s) {
    case SINKATTN_OK: return "ok";
    case SINKATTN_ERR_NULL_POINTER: return "null pointer argument";
    case SINKATTN_ERR_BAD_SHAPE: return "invalid shape";
    case SINKATTN_ERR_BAD_MASK: return "invalid mask parameters (window and prefix must be >= 0)";
    case SINKATTN_ERR_UNSUPPORTED: return "unsupported dtype / head_dim combination";
    case SINKATTN_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
    case SINKATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case SINKATTN_ERR_HIP: return "HIP runtime error";
    case SINKATTN_ERR_SCRATCH:
      return "problem needs more workspace than the static scratch of the allocation-free "
             "entry point holds";
  }
  return "unknown status";
}

int32_t sinkattn_tile_class(int32_t q0, int32_t q1, int32_t k0, int32_t k1, int32_t window,
                            int32_t prefix) {
  return sa_tile_class(q0, q1, k0, k1, window, prefix);
}

int32_t sinkattn_key_tile_segments(int32_t q0, int32_t q1, int32_t window, int32_t prefix,
                                   int32_t block_k, int32_t* out) {
  if (!out || block_k <= 0 || q0 < 0 || q1 < q0 || window < 0 || prefix < 0) return -1;
  int tmp[4];
  const int n = sa_key_tile_segments(q0, q1, window, prefix, block_k, tmp);
  for (int i = 0; i < 4; ++i) out[i] = tmp[i];
  return n;
}

sinkattn_status sinkattn_tile_config(const sinkattn_problem* pb, int32_t* out) {
  Dims dims;
  const sinkattn_status st = check_problem(pb, &dims);
  if (st != SINKATTN_OK) return st;
  if (!out) return SINKATTN_ERR_NULL_POINTER;
  const int window = pb->window > pb->seqlen ? pb->seqlen : pb->window;
  out[0] = fwd_key_tile(window);
  out[1] = dkdv_query_tile(window);
  return SINKATTN_OK;
}

size_t sinkattn_bwd_workspace_size(const sinkattn_problem* pb) {
  Dims dims;
  if (check_problem(pb, &dims) != SINKATTN_OK) return 0;
  return workspace_layout(pb, dims).total;
}

sinkattn_status sinkattn_fwd(const sinkattn_problem* pb, const void* q, const void* k,
                             const void* v, const float* sinks, void* o, float* lse,
                             void* stream) {
  Dims dims;
  sinkattn_status st = check_problem(pb, &dims);
  if (st != SINKATTN_OK) return st;
  if (dims.rows == 0 || pb->batch == 0) return SINKATTN_OK;
  if (!q || !k || !v || !sinks || !o) return SINKATTN_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned16(lse)) || !aligned16(sinks))
    return SINKATTN_ERR_MISALIGNED;
  const int window = pb->window > pb->seqlen ? pb->seqlen : pb->window;   // same mask
  const int prefix = pb->prefix > pb->seqlen ? pb->seqlen : pb->prefix;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pb->dtype == SINKATTN_BF16) {
    return hip_status(launch_fwd_bf16_d64(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, sinks, (bf16*)o, lse, pb->cu_seqlens,
        pb->batch, pb->seqlen, (int)dims.rows, pb->heads_q, pb->heads_kv, window, prefix,
        pb->softmax_scale, s));
  }
  return hip_status(launch_fwd_f32(pb->head_dim, (const float*)q, (const float*)k,
                                   (const float*)v, sinks, (float*)o, lse, pb->cu_seqlens,
                                   pb->batch, pb->seqlen, (int)dims.rows, pb->heads_q,
                                   pb->heads_kv, window, prefix, pb->softmax_scale, s));
}


static sinkattn_status bwd_phases(unsigned phases, const sinkattn_problem* pb, const void* q,
                                  const void* k, const void* v, const float* sinks, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                  float* dsinks, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  Dims dims;
  sinkattn_status st = check_problem(pb, &dims);
  if (st != SINKATTN_OK) return st;
  if (!sinks || !dsinks) return SINKATTN_ERR_NULL_POINTER;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool empty = dims.rows == 0 || pb->batch == 0;
  if (!empty) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
      return SINKATTN_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        !aligned16(sinks) || !aligned16(dsinks))
      return SINKATTN_ERR_MISALIGNED;
    const Workspace wl = workspace_layout(pb, dims);
    if (!workspace || workspace_bytes < wl.total) return SINKATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SINKATTN_ERR_MISALIGNED;
  }
  // ---- validation done; device work from here on
  hipError_t e = hipSuccess;
  // dsinks: fp32 accumulates into it (cleared here); bf16 forms it in FINISH
  // from the dQ kernel's per-workgroup parts (an empty problem: cleared here)
  if ((phases & SINKATTN_BWD_PREPARE) && (pb->dtype == SINKATTN_FP32 || empty)) {
    e = launch_zero_f32(dsinks, pb->heads_q, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (empty) return SINKATTN_OK;
  const Workspace wl = workspace_layout(pb, dims);
  char* ws = static_cast<char*>(workspace);
  float* d_ws = (float*)(ws + wl.d_off);
  float* l_ws = (float*)(ws + wl.l_off);
  const bool is_f32 = pb->dtype == SINKATTN_FP32;
  float* dk_acc = is_f32 ? nullptr : (float*)(ws + wl.dk_off);
  float* dv_acc = is_f32 ? nullptr : (float*)(ws + wl.dv_off);
  float* ds_part = is_f32 ? nullptr : (float*)(ws + wl.ds_off);
  const int window = clamped_window(pb);
  const int prefix = clamped_prefix(pb);
  float* fold_part = wl.fold ? (float*)(ws + wl.fold_off) : nullptr;
  // bf16: whether the dK/dV kernel adds into its accumulators (cleared by the
  // dQ kernel, converted by the finish pass) or writes dk, dv itself
  const bool dkdv_acc = !is_f32 && dkdv_accumulates(pb->batch, pb->seqlen, pb->heads_q,
                                                    pb->heads_kv, window, prefix, wl.fold);
  const int rows = (int)dims.rows;
  const int lse_stride = dims.varlen ? rows : pb->seqlen;
  // fp32: the row pass (D, L, dsinks) is its own kernel; bf16: the dQ kernel
  // computes the row statistics of its rows, writes them for the dK/dV
  // kernel and zeroes the dK/dV accumulators, so it runs first
  if (is_f32 && (phases & SINKATTN_BWD_PREPARE)) {
    e = launch_bwd_pre(pb->head_dim, (const float*)o, (const float*)dout, lse, sinks,
                       pb->cu_seqlens, dsinks, d_ws, l_ws, pb->batch, pb->seqlen, rows,
                       pb->heads_q, lse_stride, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (!is_f32 && (phases & SINKATTN_BWD_DQ)) {
    e = launch_bwd_dq_bf16_d64((const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,
                               (const bf16*)o, lse, sinks, ds_part, wl.ds_stride, l_ws, d_ws, dk_acc, dv_acc,
                               (bf16*)dq, pb->cu_seqlens, pb->batch, pb->seqlen, rows,
                               pb->heads_q, pb->heads_kv, window, prefix, pb->softmax_scale,
                               dkdv_prefix_fold_row(window), fold_part, dkdv_acc, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (is_f32 && (phases & (SINKATTN_BWD_DKDV | SINKATTN_BWD_DQ))) {
    // the fp32 path computes dQ and dK/dV in one call (both into the outputs)
    e = launch_bwd_f32(pb->head_dim, (const float*)q, (const float*)k, (const float*)v,
                       (const float*)dout, l_ws, d_ws, (float*)dq, (float*)dk, (float*)dv,
                       pb->cu_seqlens, pb->batch, pb->seqlen, rows, pb->heads_q, pb->heads_kv,
                       window, prefix, pb->softmax_scale, (phases & SINKATTN_BWD_DQ) != 0,
                       (phases & SINKATTN_BWD_DKDV) != 0, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (!is_f32 && (phases & SINKATTN_BWD_DKDV)) {
    e = launch_bwd_dkdv_bf16_d64((const bf16*)q, (const bf16*)k, (const bf16*)v,
                                 (const bf16*)dout, l_ws, d_ws, dk_acc, dv_acc, pb->cu_seqlens,
                                 pb->batch, pb->seqlen, rows, pb->heads_q, pb->heads_kv, window,
                                 prefix, pb->softmax_scale, wl.fold, (bf16*)dk, (bf16*)dv, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if ((phases & SINKATTN_BWD_FINISH) && !is_f32) {
    // the slots the dQ kernel wrote: one per workgroup of a head
    const int ds_used = dq_launch_tiles(pb->batch, pb->seqlen, rows, dims.varlen,
                                        pb->heads_q / pb->heads_kv, window, prefix);
    // dkdv_acc false: the dK/dV kernel wrote dk, dv itself (the fold's rows
    // excepted), and only ds_h is left to the convert pass
    if (wl.fold) {
      e = launch_prefix_fold_add(fold_part, dk_acc, dv_acc, dkdv_acc ? nullptr : (bf16*)dk,
                                 dkdv_acc ? nullptr : (bf16*)dv, pb->softmax_scale,
                                 pb->cu_seqlens, pb->batch, pb->seqlen, pb->heads_kv, prefix,
                                 wl.ds_stride, dkdv_prefix_fold_row(window), s);
      if (e != hipSuccess) return hip_status(e);
    }
    e = launch_convert(dk_acc, dv_acc, (bf16*)dk, (bf16*)dv,
                       dkdv_acc ? (long long)rows * pb->heads_kv * pb->head_dim : 0,
                       pb->softmax_scale, ds_part, ds_used, wl.ds_stride, pb->heads_q, dsinks, s);
  }
  return hip_status(e);
}

#define SINKATTN_BWD_ARGS                                                                   \
  const sinkattn_problem *pb, const void *q, const void *k, const void *v,                 \
      const float *sinks, const void *o, const float *lse, const void *dout, void *dq,     \
      void *dk, void *dv, float *dsinks, void *workspace, size_t workspace_bytes,          \
      void *stream
#define SINKATTN_BWD_PASS q, k, v, sinks, o, lse, dout, dq, dk, dv, dsinks, workspace, workspace_bytes, stream

sinkattn_status sinkattn_bwd(SINKATTN_BWD_ARGS) {
  return bwd_phases(SINKATTN_BWD_ALL, pb, SINKATTN_BWD_PASS);
}

sinkattn_status sinkattn_bwd_phases(uint32_t phases, SINKATTN_BWD_ARGS) {
  if (phases == 0 || (phases & ~(uint32_t)SINKATTN_BWD_ALL) != 0) return SINKATTN_ERR_BAD_SHAPE;
  return bwd_phases(phases, pb, SINKATTN_BWD_PASS);
}

}  // extern "C"

extern "C" {

size_t sinkattn_decode_workspace_size(const sinkattn_decode_problem* pb) {
  if (check_decode(pb) != SINKATTN_OK) return 0;
  return round_up(decode_workspace_bytes(pb->batch, pb->cache_capacity, pb->heads_q, pb->heads_kv,
                                         clamp_window(pb->window, pb->cache_capacity),
                                         clamp_window(pb->prefix, pb->cache_capacity)));
}

}  // extern "C"

namespace {

// Pointer checks shared by the two decode entry points.  No HIP calls.
sinkattn_status check_decode_pointers(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* cache_seqlens, const float* sinks,
                                      const void* o, const float* lse) {
  if (!q || !k_cache || !v_cache || !cache_seqlens || !sinks || !o)
    return SINKATTN_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned16(sinks) || (lse && !aligned16(lse)) ||
      (reinterpret_cast<uintptr_t>(cache_seqlens) & 3u) != 0)
    return SINKATTN_ERR_MISALIGNED;
  return SINKATTN_OK;
}

}  // namespace

extern "C" {

sinkattn_status sinkattn_decode(const sinkattn_decode_problem* pb, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* cache_seqlens, const float* sinks, void* o,
                                float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  sinkattn_status st = check_decode(pb);
  if (st != SINKATTN_OK) return st;
  if (pb->batch == 0) return SINKATTN_OK;
  st = check_decode_pointers(q, k_cache, v_cache, cache_seqlens, sinks, o, lse);
  if (st != SINKATTN_OK) return st;
  const int window = clamp_window(pb->window, pb->cache_capacity);
  const int prefix = clamp_window(pb->prefix, pb->cache_capacity);
  const size_t need = decode_workspace_bytes(pb->batch, pb->cache_capacity, pb->heads_q,
                                             pb->heads_kv, window, prefix);
  if (!workspace || workspace_bytes < need) return SINKATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SINKATTN_ERR_MISALIGNED;
  return hip_status(launch_decode_bf16_d64(
      (const bf16*)q, (const bf16*)k_cache, (const bf16*)v_cache, cache_seqlens, sinks, (bf16*)o,
      lse, (float*)workspace, pb->batch, pb->cache_capacity, pb->heads_q, pb->heads_kv, window,
      prefix, pb->softmax_scale, static_cast<hipStream_t>(stream)));
}

sinkattn_status sinkattn_decode_noalloc(const sinkattn_decode_problem* pb, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* cache_seqlens, const float* sinks,
                                        void* o, float* lse, void* stream) {
  sinkattn_status st = check_decode(pb);
  if (st != SINKATTN_OK) return st;
  if (pb->batch == 0) return SINKATTN_OK;
  st = check_decode_pointers(q, k_cache, v_cache, cache_seqlens, sinks, o, lse);
  if (st != SINKATTN_OK) return st;
  const int window = clamp_window(pb->window, pb->cache_capacity);
  const int prefix = clamp_window(pb->prefix, pb->cache_capacity);
  const size_t need = decode_workspace_bytes(pb->batch, pb->cache_capacity, pb->heads_q,
                                             pb->heads_kv, window, prefix);
  if (need > decode_scratch_bytes()) return SINKATTN_ERR_SCRATCH;
  // ---- validation done; device work from here on
  void* scratch = nullptr;
  const hipError_t e = decode_scratch(&scratch);
  if (e != hipSuccess) return SINKATTN_ERR_HIP;
  return hip_status(launch_decode_bf16_d64(
      (const bf16*)q, (const bf16*)k_cache, (const bf16*)v_cache, cache_seqlens, sinks, (bf16*)o,
      lse, (float*)scratch, pb->batch, pb->cache_capacity, pb->heads_q, pb->heads_kv, window,
      prefix, pb->softmax_scale, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

sinkattn_status check_grpo(const sinkattn_grpo_problem* pb) {
  if (!pb) return SINKATTN_ERR_NULL_POINTER;
  if (pb->num_rollouts < 0 || pb->total_tokens < 0 || pb->group_size < 1 ||
      pb->group_size > 1024 || pb->num_rollouts % pb->group_size != 0 ||
      (pb->num_rollouts == 0 && pb->total_tokens != 0) || (pb->kl_mode != 0 && pb->kl_mode != 1))
    return SINKATTN_ERR_BAD_SHAPE;
  if (!(pb->eps_adv >= 0.0f) || !std::isfinite(pb->eps_adv) || !(pb->eps_clip >= 0.0f) ||
      !(pb->eps_clip < 1.0f) || !std::isfinite(pb->beta))
    return SINKATTN_ERR_BAD_SHAPE;
  return SINKATTN_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" {

size_t sinkattn_grpo_workspace_size(const sinkattn_grpo_problem* pb) {
  if (check_grpo(pb) != SINKATTN_OK) return 0;
  return round_up(grpo_workspace_bytes(pb->num_rollouts, pb->total_tokens));
}

sinkattn_status sinkattn_grpo_loss(const sinkattn_grpo_problem* pb, const float* logp_new,
                                   const float* logp_old, const float* logp_ref,
                                   const uint8_t* action_mask, const float* rewards,
                                   const int32_t* cu_seqlens, float* loss, float* grad,
                                   float* advantages, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  const sinkattn_status st = check_grpo(pb);
  if (st != SINKATTN_OK) return st;
  const bool tokens = pb->total_tokens > 0;
  const bool rolls = pb->num_rollouts > 0;
  if (!loss || !cu_seqlens || (tokens && (!logp_new || !logp_old || !grad)) ||
      (rolls && !rewards) || (tokens && pb->beta != 0.0f && !logp_ref))
    return SINKATTN_ERR_NULL_POINTER;
  if ((tokens && (!aligned16(logp_new) || !aligned16(logp_old) || !aligned16(grad) ||
                  (pb->beta != 0.0f && !aligned16(logp_ref)) ||
                  (action_mask && !aligned16(action_mask)))) ||
      (rolls && !aligned4(rewards)) || (advantages && !aligned4(advantages)) ||
      !aligned4(cu_seqlens) || !aligned4(loss))
    return SINKATTN_ERR_MISALIGNED;
  const size_t need = grpo_workspace_bytes(pb->num_rollouts, pb->total_tokens);
  if (!workspace || workspace_bytes < need) return SINKATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SINKATTN_ERR_MISALIGNED;
  return hip_status(launch_grpo(logp_new, logp_old, logp_ref, action_mask, rewards, cu_seqlens,
                                loss, grad, advantages, workspace, pb->num_rollouts,
                                pb->group_size, pb->total_tokens, pb->kl_mode, pb->eps_adv,
                                pb->eps_clip, pb->beta, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
