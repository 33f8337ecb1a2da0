// GRPO token loss and group-normalised advantage over packed rollout groups
// (arXiv 2608.10357, section 4 "Training pipeline", paragraph "Policy
// update", eq. 3-7):
//   A_i = (R_i - mean_g R) / (std_g R + eps_A)            population std
//   rho = exp(logp_new - logp_old),  J = min(rho A, clip(rho, 1 -+ eps_c) A)
//   L_g = (-sum J + beta sum kl) / S_g over the group's optimised tokens,
//   loss = mean_g L_g,  grad = d loss / d logp_new per token.
// HBM-bound streaming work: 13 bytes read and 4 written per token.
//
// Three launches.  grpo_rollout_stats: one workgroup per rollout counts its
// optimised tokens (16 mask bytes per lane load), forms its advantage from
// the group's G rewards (fp64 mean and population std) and records, for each
// 4096-token chunk that starts inside the rollout, the rollout's index.
// grpo_tokens: one workgroup per 4096-token chunk reads the rollout its chunk
// starts in, stages the next 256 rollout boundaries, advantages and token
// weights 1 / (M S_g) in LDS (S_g summed from the group's counts), issues all
// its loads (float4 per lane: a wave moves 1 KB per load) before the
// arithmetic, finds each token's rollout by walking the LDS table forward
// (tokens come in increasing order, so the position only moves ahead), and
// writes the gradient and its loss partial.  grpo_loss_sum adds the partials
// in index order, so the loss does not depend on which workgroups finish
// first.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

constexpr int STATS_THREADS = 256;
constexpr int TOK_THREADS = 256;
constexpr int TOK_VEC = 4;                                // tokens per lane per step
constexpr int TOK_STEPS = 4;
constexpr int TOK_CHUNK = TOK_THREADS * TOK_VEC * TOK_STEPS;   // 4096 tokens per workgroup
constexpr int TABLE = 256;                       // rollouts staged per chunk

struct GrpoArgs {
  const float* logp_new;
  const float* logp_old;
  const float* logp_ref;        // null when beta == 0
  const uint8_t* mask;          // null: every token optimised
  const float* rewards;
  const int32_t* cu;            // [B + 1]
  float* loss;
  float* grad;
  float* adv_out;               // may be null
  float* adv_ws;                // [B]
  int* count_ws;                // [B]  optimised tokens per rollout
  int* chunk_roll;              // [chunks] rollout holding each chunk's first token
  double* partial;              // [chunks]
  int num_rollouts, group_size, num_groups, total_tokens, num_chunks, kl_mode;
  float eps_adv, eps_clip, beta;
  float clip_hi_log, clip_lo_log;   // fp32 log(1 + eps_c), log(1 - eps_c)
};

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
// sum over the workgroup (STATS_THREADS) in a fixed order
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < STATS_THREADS / 64; ++w) s += red[w];
  return s;
}
// nonzero bytes of a 32-bit word
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  w |= w >> 4;
  w |= w >> 2;
  w |= w >> 1;
  return __builtin_popcount(w & 0x01010101u);
}

__global__ __launch_bounds__(STATS_THREADS) void grpo_rollout_stats(GrpoArgs a) {
  __shared__ double red[STATS_THREADS / 64];
  const int i = blockIdx.x;
  if (i >= a.num_rollouts) return;
  const int n = a.total_tokens;
  // offsets clamped to [0, N], so malformed cu_seqlens cannot index past the arrays
  const int s = min(max(a.cu[i], 0), n);
  const int e = min(max(a.cu[i + 1], s), n);
  // T_i: aligned 16-byte blocks inside [s, e) by uint4 loads, the ragged ends by bytes
  int c = 0;
  if (a.mask) {
    const int a0 = (s + 15) & ~15, a1 = e & ~15;
    if (a0 < a1) {
      for (int k = a0 + 16 * (int)threadIdx.x; k < a1; k += 16 * STATS_THREADS) {
        const uint4 v = *(const uint4*)(a.mask + k);
        c += nonzero_bytes(v.x) + nonzero_bytes(v.y) + nonzero_bytes(v.z) + nonzero_bytes(v.w);
      }
      for (int t = s + (int)threadIdx.x; t < a0; t += STATS_THREADS) c += a.mask[t] != 0;
      for (int t = a1 + (int)threadIdx.x; t < e; t += STATS_THREADS) c += a.mask[t] != 0;
    } else {
      for (int t = s + (int)threadIdx.x; t < e; t += STATS_THREADS) c += a.mask[t] != 0;
    }
  } else if (threadIdx.x == 0) {
    c = e - s;
  }
  const double cnt = block_sum((double)c, red);
  // advantage from the group's rewards: fp64 mean, then population std
  const int g = a.group_size, r0 = (i / g) * g;
  double rs = 0.0;
  for (int k = threadIdx.x; k < g; k += STATS_THREADS) rs += (double)a.rewards[r0 + k];
  const double mean = block_sum(rs, red) / g;
  double vs = 0.0;
  for (int k = threadIdx.x; k < g; k += STATS_THREADS) {
    const double d = (double)a.rewards[r0 + k] - mean;
    vs += d * d;
  }
  const double var = block_sum(vs, red) / g;
  if (threadIdx.x == 0) {
    const double dr = (double)a.rewards[i] - mean;
    // a reward equal to the group mean has no advantage, also for eps_A = 0
    const float adv = dr == 0.0 ? 0.0f : (float)(dr / (sqrt(var) + (double)a.eps_adv));
    a.adv_ws[i] = adv;
    if (a.adv_out) a.adv_out[i] = adv;
    a.count_ws[i] = (int)cnt;
  }
  // chunks whose first token lies in this rollout
  for (int ch = (s + TOK_CHUNK - 1) / TOK_CHUNK + (int)threadIdx.x; ch * TOK_CHUNK < e;
       ch += STATS_THREADS)
    a.chunk_roll[ch] = i;
}

// KL estimate and its derivative in logp_new.  MODE 1: log-ratio; MODE 2:
// exp(r) - r - 1 with r = logp_ref - logp_new, by a short series near 0 (the
// direct form cancels there) and by the hardware exp2 elsewhere.
template <int MODE>
__device__ __forceinline__ void kl_term(float vn, float vr, float& kl, float& dkl) {
  if (MODE == 1) {
    kl = vn - vr;
    dkl = 1.0f;
  } else if (MODE == 2) {
    const float r = vr - vn;
    // r^2 (1/2 + r/6 + r^2/24 + ...) and r (1 + r/2 + r^2/6 + ...) for |r| < 1/4
    float p = fmaf(r, 1.0f / 5040.0f, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);                          // (e^r - 1 - r) / r^2
    const float em1_small = fmaf(r * r, p, r);    // e^r - 1
    const float e = __builtin_amdgcn_exp2f(r * 1.4426950408889634f);
    const bool small = fabsf(r) < 0.25f;
    kl = small ? r * r * p : (e - r) - 1.0f;
    dkl = -(small ? em1_small : e - 1.0f);
  } else {
    kl = 0.0f;
    dkl = 0.0f;
  }
}

// token weight 1 / (M S_g) of rollout r's group (0 if the group has no optimised token)
__device__ __forceinline__ float group_weight(const GrpoArgs& a, int r) {
  const int g0 = (r / a.group_size) * a.group_size;
  long long sg = 0;
  for (int k = 0; k < a.group_size; ++k) sg += a.count_ws[g0 + k];
  return sg > 0 ? (float)(1.0 / ((double)a.num_groups * (double)sg)) : 0.0f;
}

// rollout of token t when more than TABLE rollouts end inside the chunk:
// walk on from the table's end (rare)
__device__ __forceinline__ void far_rollout(const GrpoArgs& a, int r_from, int t,
                                                   float* adv, float* wt) {
  int r = r_from;
  while (r + 1 < a.num_rollouts && a.cu[r + 1] <= t) ++r;
  r = min(r, a.num_rollouts - 1);
  *adv = a.adv_ws[r];
  *wt = group_weight(a, r);
}

struct TokTable {
  int bound[TABLE];        // cu[r0 + 1 + j]: end of rollout r0 + j
  float adv[TABLE], w[TABLE];
};

// one token: loss contribution (into acc) and gradient
template <int MODE>
__device__ __forceinline__ float token(const GrpoArgs& a, float vn, float vo, float vr, float on,
                                       float adv, float wt, double& acc) {
  const float d = vn - vo;
  const float rho = __builtin_amdgcn_exp2f(d * 1.4426950408889634f);
  const bool clipped = (adv > 0.0f && d > a.clip_hi_log) || (adv < 0.0f && d < a.clip_lo_log);
  const float rho_used = clipped ? (adv > 0.0f ? 1.0f + a.eps_clip : 1.0f - a.eps_clip) : rho;
  const float dj = clipped ? 0.0f : rho * adv;
  float kl, dkl;
  kl_term<MODE>(vn, vr, kl, dkl);
  const float wo = wt * on;                    // on: 1 for an optimised token, else 0
  acc += (double)(wo * (a.beta * kl - rho_used * adv));
  return wo * (a.beta * dkl - dj);
}

template <int MODE, bool FULL>
__device__ __forceinline__ void chunk(const GrpoArgs& a, TokTable& tb, int base, double& acc) {
  const int n = a.total_tokens, nr = a.num_rollouts;
  // every token load of this lane first (they do not depend on the rollout table)
  float4 nw[TOK_STEPS], od[TOK_STEPS], rf[TOK_STEPS];
  uint32_t mk[TOK_STEPS];
#pragma unroll
  for (int st = 0; st < TOK_STEPS; ++st) {
    const int t0 = base + (st * TOK_THREADS + (int)threadIdx.x) * TOK_VEC;
    if (FULL || t0 + TOK_VEC <= n) {
      nw[st] = *(const float4*)(a.logp_new + t0);
      od[st] = *(const float4*)(a.logp_old + t0);
      rf[st] = MODE ? *(const float4*)(a.logp_ref + t0) : make_float4(0.f, 0.f, 0.f, 0.f);
      mk[st] = a.mask ? *(const uint32_t*)(a.mask + t0) : 0x01010101u;
    } else {
      float x[TOK_VEC], y[TOK_VEC], z[TOK_VEC];
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < TOK_VEC; ++e) {
        const int t = t0 + e < n ? t0 + e : n - 1;
        x[e] = a.logp_new[t];
        y[e] = a.logp_old[t];
        z[e] = MODE ? a.logp_ref[t] : 0.0f;
        const uint32_t on = t0 + e < n && (a.mask ? a.mask[t] != 0 : true);
        m |= on << (8 * e);
      }
      nw[st] = make_float4(x[0], x[1], x[2], x[3]);
      od[st] = make_float4(y[0], y[1], y[2], y[3]);
      rf[st] = make_float4(z[0], z[1], z[2], z[3]);
      mk[st] = m;
    }
  }
  // the rollout table of this chunk
  const int r0 = min(max(a.chunk_roll[blockIdx.x], 0), nr - 1);
  const int end = min(base + TOK_CHUNK, n);
  for (int j = threadIdx.x; j < TABLE; j += TOK_THREADS) {
    const int r = r0 + j;
    tb.bound[j] = r < nr ? (r + 1 < nr ? a.cu[r + 1] : n) : 0x7fffffff;
    // only the rollouts the chunk reaches need their group's weight
    const bool used = r < nr && (j == 0 || a.cu[r] < end);
    tb.adv[j] = used ? a.adv_ws[r] : 0.0f;
    tb.w[j] = used ? group_weight(a, r) : 0.0f;
  }
  __syncthreads();
  // this lane's tokens only increase: the table position only moves forward
  // (staged rollout r0 + pos holds token t when pos = number of ends <= t)
  int pos = 0;
#pragma unroll
  for (int st = 0; st < TOK_STEPS; ++st) {
    const int t0 = base + (st * TOK_THREADS + (int)threadIdx.x) * TOK_VEC;
    if (!FULL && t0 >= n) break;
    while (pos < TABLE && tb.bound[pos] <= t0) ++pos;
    const float vn[TOK_VEC] = {nw[st].x, nw[st].y, nw[st].z, nw[st].w};
    const float vo[TOK_VEC] = {od[st].x, od[st].y, od[st].z, od[st].w};
    const float vr[TOK_VEC] = {rf[st].x, rf[st].y, rf[st].z, rf[st].w};
    float gout[TOK_VEC];
    if (pos < TABLE && tb.bound[pos] > t0 + TOK_VEC - 1) {
      // the four tokens lie in one rollout
      const float adv = tb.adv[pos], wt = tb.w[pos];
#pragma unroll
      for (int e = 0; e < TOK_VEC; ++e) {
        const float on = (float)((mk[st] >> (8 * e)) & 0xffu ? 1 : 0);
        gout[e] = token<MODE>(a, vn[e], vo[e], vr[e], on, adv, wt, acc);
      }
    } else {
#pragma unroll
      for (int e = 0; e < TOK_VEC; ++e) {
        const int t = t0 + e;
        while (pos < TABLE && tb.bound[pos] <= t) ++pos;
        float adv = 0.0f, wt = 0.0f;
        if (pos < TABLE) {
          adv = tb.adv[pos];
          wt = tb.w[pos];
        } else if (FULL || t < n) {
          far_rollout(a, r0 + TABLE, t, &adv, &wt);
        }
        const float on = (float)((mk[st] >> (8 * e)) & 0xffu ? 1 : 0);
        gout[e] = token<MODE>(a, vn[e], vo[e], vr[e], on, adv, wt, acc);
      }
    }
    if (FULL || t0 + TOK_VEC <= n) {
      *(float4*)(a.grad + t0) = make_float4(gout[0], gout[1], gout[2], gout[3]);
    } else {
#pragma unroll
      for (int e = 0; e < TOK_VEC; ++e)
        if (t0 + e < n) a.grad[t0 + e] = gout[e];
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(TOK_THREADS) void grpo_tokens(GrpoArgs a) {
  __shared__ TokTable tb;
  __shared__ double red[TOK_THREADS / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = blockIdx.x * TOK_CHUNK;
  double acc = 0.0;               // the loss is a small difference of many terms: fp64
  if (base + TOK_CHUNK <= a.total_tokens) chunk<MODE, true>(a, tb, base, acc);
  else if (base < a.total_tokens) chunk<MODE, false>(a, tb, base, acc);
  // workgroup partial, in a fixed order; grpo_loss_sum adds the partials
  acc = wave_sum(acc);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < TOK_THREADS / 64; ++w) s += red[w];
    a.partial[blockIdx.x] = s;
  }
}

// loss = sum of the chunk partials in index order (one workgroup; a kernel of
// its own because a device-scope fence per workgroup would write back the
// XCD's L2 each time)
__global__ __launch_bounds__(TOK_THREADS) void grpo_loss_sum(GrpoArgs a) {
  __shared__ double red[TOK_THREADS / 64];
  double s = 0.0;
  for (int i = threadIdx.x; i < a.num_chunks; i += TOK_THREADS) s += a.partial[i];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < TOK_THREADS / 64; ++w) tot += red[w];
    *a.loss = (float)tot;
  }
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

int grpo_token_blocks(int total_tokens) {
  const int b = (total_tokens + TOK_CHUNK - 1) / TOK_CHUNK;
  return b > 0 ? b : 1;
}

size_t grpo_workspace_bytes(int num_rollouts, int total_tokens) {
  const size_t chunks = (size_t)grpo_token_blocks(total_tokens);
  return align256((size_t)num_rollouts * sizeof(float)) +
         align256((size_t)num_rollouts * sizeof(int)) + align256(chunks * sizeof(int)) +
         align256(chunks * sizeof(double));
}

hipError_t launch_grpo(const float* logp_new, const float* logp_old, const float* logp_ref,
                       const uint8_t* mask, const float* rewards, const int32_t* cu_seqlens,
                       float* loss, float* grad, float* advantages, void* workspace,
                       int num_rollouts, int group_size, int total_tokens, int kl_mode,
                       float eps_adv, float eps_clip, float beta, hipStream_t stream) {
  GrpoArgs a;
  a.logp_new = logp_new; a.logp_old = logp_old; a.logp_ref = beta != 0.0f ? logp_ref : nullptr;
  a.mask = mask; a.rewards = rewards; a.cu = cu_seqlens;
  a.loss = loss; a.grad = grad; a.adv_out = advantages;
  const int chunks = grpo_token_blocks(total_tokens);
  char* ws = (char*)workspace;
  a.adv_ws = (float*)ws;
  ws += align256((size_t)num_rollouts * sizeof(float));
  a.count_ws = (int*)ws;
  ws += align256((size_t)num_rollouts * sizeof(int));
  a.chunk_roll = (int*)ws;
  ws += align256((size_t)chunks * sizeof(int));
  a.partial = (double*)ws;
  a.num_rollouts = num_rollouts; a.group_size = group_size;
  a.num_groups = num_rollouts / group_size; a.total_tokens = total_tokens;
  a.num_chunks = chunks; a.kl_mode = kl_mode;
  a.eps_adv = eps_adv; a.eps_clip = eps_clip; a.beta = beta;
  a.clip_hi_log = (float)log1p((double)eps_clip);
  a.clip_lo_log = (float)log1p(-(double)eps_clip);
  if (num_rollouts > 0) {
    grpo_rollout_stats<<<num_rollouts, STATS_THREADS, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int mode = beta == 0.0f ? 0 : (kl_mode == 0 ? 1 : 2);
  if (mode == 0) grpo_tokens<0><<<chunks, TOK_THREADS, 0, stream>>>(a);
  else if (mode == 1) grpo_tokens<1><<<chunks, TOK_THREADS, 0, stream>>>(a);
  else grpo_tokens<2><<<chunks, TOK_THREADS, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  grpo_loss_sum<<<1, TOK_THREADS, 0, stream>>>(a);
  return hipGetLastError();
}
