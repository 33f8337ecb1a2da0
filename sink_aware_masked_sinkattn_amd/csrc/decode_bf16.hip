// Decode: one new query token per sequence against its key/value cache, bf16,
// head dim 64, gfx950 MFMA -- the rollout side of the same sink-aware
// attention (arXiv 2608.10357 section 4, "Rollout workers"; "GPT-OSS Agentic
// RL training: a practical retrospective", section on the training-inference
// mismatch through attention sinks: the rollout engine must give the
// trainer's token probabilities, sink included).
//
// For sequence b with n cached tokens (the new token's key and value already
// at position n - 1) the query sits at position n - 1 under the training mask
// M[q,k] = 1[k<=q] AND 1[q-k<=w OR k<p] ("Efficient Reinforcement Learning
// for Long-Horizon Tool-Use Agentic Tasks", summary page), so it sees the
// prefix keys [0, min(p, n)) and the window keys [max(0, n-1-w), n), and
//   O = sigmoid(l - s_h) * softmax(S) V,  l = log sum exp(S)   (content only)
// -- row n - 1 of the forward on the whole sequence.
//
// Work decomposition.  The visible keys are cut into 64-key chunks.  A
// workgroup (4 waves) takes one kv head of one sequence and a run of chunks
// (a split); each wave handles its own chunks with all the query heads of the
// kv head's group at once, so every K and V row is read once per group:
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 -- 16 keys (A, rows of K read
//        straight from global memory) x the group's heads (B, in registers,
//        up to 16; unused columns are zero);
//   C layout: one head per lane, 4 keys per lane and tile, so the softmax
//        state (running max m, running sum r) is per lane;
//   O^T += V^T P^T -- A = V^T by transpose reads of the chunk's V rows staged
//        in the wave's own LDS tile, B = the probabilities straight from the
//        C layout (two 16-key tiles = 32 keys), so the accumulator too has
//        one head per lane (16 of the 64 head dims per lane).
// The four waves' (m, r, acc) merge in LDS into one partial per (split, head);
// a second kernel merges the splits of a sequence and applies the sink:
//   O = acc / (r + exp(s_h - m)),  l = m + log r    (log2 units inside).
// When every sequence's visible keys fit one split (short windows) the split
// kernel applies the sink itself and no combine kernel runs.
// The decode step is bound by HBM (each visible K/V row is read once); the
// MFMA work is small next to it.
#include "common.h"
#include "mask_tiles.h"

namespace {

constexpr int D = 64;
constexpr int WAVES = 4;
constexpr int KW = 64;           // keys per chunk
constexpr int HMAX = 16;         // query heads per kv head (MFMA N columns)
constexpr int PART = D + 2;      // floats per (split, head) partial: m, r, acc[64]

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8 a, bf16x8 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct DecArgs {
  const bf16* q;            // [B, Hq, D]
  const bf16* k;            // [B, Tmax, Hkv, D]
  const bf16* v;
  const int* cache_seqlens; // [B]
  const float* sinks;       // [Hq]
  bf16* o;                  // [B, Hq, D]
  float* lse;               // [B, Hq] or null
  float* part;              // [B, Hkv, max_splits, HMAX, PART]
  int batch, tmax, heads_q, heads_kv, group, window, prefix;
  int chunks_per_wave, max_splits;
  float scale_log2;
};

constexpr int SEQ_WIN = 1024;    // sequences whose unit offsets sit in LDS at a time

// LDS of the split kernel: the waves' V tiles during a unit's chunk loop; the
// same memory then holds the four waves' results for the merge.  ustart[j]
// is the first work unit of sequence b_lo + j (relative to the window).
struct __attribute__((aligned(16))) DecSmem {
  union {
    bf16 vtile[WAVES][KW * D];          // per wave, swizzled rows (tile_off)
    float red_acc[WAVES][HMAX][D];
  };
  float red_m[WAVES][HMAX], red_r[WAVES][HMAX];
  int ustart[SEQ_WIN + 1];
};

__device__ __forceinline__ int seq_len(const DecArgs& a, int b) {
  const int n = a.cache_seqlens[b];
  return n < 0 ? 0 : (n > a.tmax ? a.tmax : n);
}

__device__ __forceinline__ int n_splits(const DecArgs& a, int n) {
  int r[4];
  const int nc = sa_decode_ranges(n, a.window, a.prefix, KW, r);
  const int per = WAVES * a.chunks_per_wave;
  return (nc + per - 1) / per;
}

// Work units of sequence b: one per (kv head, split).  FINAL: every sequence
// fits one split, and a sequence with no keys still gets its unit (it writes
// O = 0, l = -inf).
template <bool FINAL>
__device__ __forceinline__ int seq_units(const DecArgs& a, int b) {
  const int ns = n_splits(a, seq_len(a, b));
  return a.heads_kv * (FINAL ? 1 : ns);
}

// ustart[0..SEQ_WIN] = exclusive prefix sum of the unit counts of sequences
// b_lo .. b_lo + SEQ_WIN - 1 (0 past the batch).  Called by the whole
// workgroup; ends with a barrier.
template <bool FINAL>
__device__ void build_window(const DecArgs& a, DecSmem& sm, int b_lo) {
  const int tid = threadIdx.x;
  __syncthreads();   // earlier readers of ustart are done
  for (int i = tid; i < SEQ_WIN; i += WAVES * 64)
    sm.ustart[i + 1] = (b_lo + i < a.batch) ? seq_units<FINAL>(a, b_lo + i) : 0;
  __syncthreads();
  if (tid < 64) {   // wave 0: each lane sums 16 consecutive counts, then a lane scan
    constexpr int E = SEQ_WIN / 64;
    int run = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) run += sm.ustart[1 + tid * E + e];
    int inc = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(inc, off);
      if (tid >= off) inc += t;
    }
    int acc = inc - run;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc += sm.ustart[1 + tid * E + e];
      sm.ustart[1 + tid * E + e] = acc;
    }
    if (tid == 0) sm.ustart[0] = 0;
  }
  __syncthreads();
}

// One work unit: kv head kvh of sequence b, chunks [split*per, split*per+per)
// of its visible keys.  Ends with a barrier (the LDS is reused by the next).
template <bool FINAL>
__device__ __forceinline__ void decode_unit(const DecArgs& a, DecSmem& sm, int b, int kvh,
                                            int split) {
  const int n = seq_len(a, b);
  int rng[4];
  const int nc = sa_decode_ranges(n, a.window, a.prefix, KW, rng);
  const int per = WAVES * a.chunks_per_wave;
  const int tid = threadIdx.x;
  if (FINAL && nc == 0) {   // no keys: O = 0, l = -inf for the group's heads
    for (int e = tid; e < a.group * D; e += WAVES * 64) {
      const int hq = kvh * a.group + e / D;
      a.o[((size_t)b * a.heads_q + hq) * D + e % D] = (bf16)0.0f;
      if (a.lse && e % D == 0) a.lse[(size_t)b * a.heads_q + hq] = -INFINITY;
    }
    return;
  }

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;       // MFMA column: query head within the group
  const int grp = lane >> 4;       // 16-lane group
  const int kv_stride = a.heads_kv * D;
  const bf16* kbase = a.k + ((size_t)b * a.tmax * a.heads_kv + kvh) * D;
  const bf16* vbase = a.v + ((size_t)b * a.tmax * a.heads_kv + kvh) * D;

  // Q^T as the B operand: lane holds head col, head dims 32*step + 8*grp .. +7
  bf16x8 qf[2];
  {
    const bool ok = col < a.group;
    const bf16* qp = a.q + ((size_t)b * a.heads_q + kvh * a.group + col) * D;
#pragma unroll
    for (int st = 0; st < 2; ++st)
      qf[st] = ok ? *(const bf16x8*)(qp + 32 * st + 8 * grp) : bf16x8{};
  }

  float m_run = -INFINITY;   // running max of this lane's head (log2 units)
  float r_lane = 0.0f;       // this lane's share of the running sum
  f32x4_t acc[4];            // O^T: rows d = 16*mb + 4*grp + i, column = head col
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Per chunk: its V rows into this wave's LDS tile (rows past k1 repeat
  // k1-1), its K rows into registers as the A operand of S^T (lane: key
  // k0 + 16t + col, dims 32*st + 8*grp), then S^T, the online softmax and
  // O^T += V^T P^T.  (A prefetch of the next chunk does not pay here: the
  // compiler waits for every outstanding load before the first LDS read of a
  // tile filled by global_load_lds.)
  bf16* vs = sm.vtile[wave];
  const int c_begin = split * per + wave * a.chunks_per_wave;
  const int c_end = min(c_begin + a.chunks_per_wave, nc);
  for (int c = c_begin; c < c_end; ++c) {
    int k0, k1;
    sa_decode_chunk(rng, KW, c, &k0, &k1);
    tile_load_lds<KW, 1>(vs, vbase + (size_t)k0 * kv_stride, kv_stride, k1 - k0, 0, lane);
    bf16x8 kf[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = min(k0 + 16 * t + col, k1 - 1);
      const bf16* kp = kbase + (size_t)key * kv_stride + 8 * grp;
#pragma unroll
      for (int st = 0; st < 2; ++st) kf[t][st] = *(const bf16x8*)(kp + 32 * st);
    }
    // S^T: lane = head col, keys k0 + 16t + 4*grp + i
    f32x4_t s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = mfma16x16x32(kf[t][0], qf[0], f32x4_t{0.f, 0.f, 0.f, 0.f});
      s[t] = mfma16x16x32(kf[t][1], qf[1], s[t]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * t + 4 * grp + i;
        s[t][i] = key < k1 ? s[t][i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[t][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);          // finite: every chunk has a key
    const float corr = fast_exp2(m_run - m_new);   // 0 on the first chunk
    m_run = m_new;
    r_lane *= corr;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] *= corr;
    float p[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t][i] = fast_exp2(s[t][i] - m_new);
        r_lane += p[t][i];
      }
    // wait for the V tile (this wave's own loads), then O^T += V^T P^T
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const bf16x8 pb = to_bf16x8(p[2 * tp][0], p[2 * tp][1], p[2 * tp][2], p[2 * tp][3],
                                  p[2 * tp + 1][0], p[2 * tp + 1][1], p[2 * tp + 1][2],
                                  p[2 * tp + 1][3]);
      const int r0 = 32 * tp + 4 * grp + (col >> 2);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int c0 = 16 * mb + 4 * (col & 3);
        const bf16x8 va = cat8(lds_read_tr4(vs + tile_off(r0, c0)),
                               lds_read_tr4(vs + tile_off(r0 + 16, c0)));
        acc[mb] = mfma16x16x32(va, pb, acc[mb]);
      }
    }
    // the next chunk's tile load overwrites vs: all reads of it are done
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- merge the four waves in LDS (a wave without chunks has m = -inf);
  // red_acc overlays the V tiles: every wave must be done reading them
  float r_tot = r_lane + __shfl_xor(r_lane, 16);
  r_tot += __shfl_xor(r_tot, 32);
  __syncthreads();
  if (grp == 0) {
    sm.red_m[wave][col] = m_run;
    sm.red_r[wave][col] = r_tot;
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.red_acc[wave][col][16 * mb + 4 * grp + i] = acc[mb][i];
  __syncthreads();
  float* part = a.part + (((size_t)b * a.heads_kv + kvh) * a.max_splits + split) * HMAX * PART;
  for (int e = tid; e < a.group * D; e += WAVES * 64) {
    const int h = e / D, d = e % D;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) m = fmaxf(m, sm.red_m[w][h]);
    float r = 0.0f, x = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = fast_exp2(sm.red_m[w][h] - m);
        r += sm.red_r[w][h] * f;
        x += sm.red_acc[w][h][d] * f;
      }
    }
    if (FINAL) {
      const int hq = kvh * a.group + h;
      const float denom = r + fast_exp2(a.sinks[hq] * SA_LOG2E - m);
      a.o[((size_t)b * a.heads_q + hq) * D + d] = (bf16)(x / denom);
      if (a.lse && d == 0) a.lse[(size_t)b * a.heads_q + hq] = (m + fast_log2(r)) * SA_LN2;
    } else {
      float* ph = part + h * PART;
      if (d == 0) {
        ph[0] = m;
        ph[1] = r;
      }
      ph[2 + d] = x;
    }
  }
  __syncthreads();   // the next unit's tile loads overwrite red_acc
}

// Persistent grid: each workgroup takes work units blockIdx.x, + gridDim.x,
// ... of the flat list (sequence by sequence; within a sequence, split-major
// with kv heads fastest) until it passes the list's end, which every
// workgroup computes from cache_seqlens the same way -- so no workgroup is
// launched without work and every one exits.
template <bool FINAL>
__device__ __forceinline__ void decode_split(const DecArgs& a) {
  __shared__ DecSmem sm;
  int b_lo = 0;
  int base = 0;   // units before sequence b_lo
  build_window<FINAL>(a, sm, b_lo);
  for (int u = blockIdx.x;; u += gridDim.x) {
    while (u - base >= sm.ustart[SEQ_WIN]) {
      if (b_lo + SEQ_WIN >= a.batch) return;   // past the last sequence
      base += sm.ustart[SEQ_WIN];
      b_lo += SEQ_WIN;
      build_window<FINAL>(a, sm, b_lo);
    }
    const int local = u - base;
    int lo = 0, hi = SEQ_WIN;   // largest j with ustart[j] <= local
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm.ustart[mid] <= local) lo = mid; else hi = mid;
    }
    const int within = local - sm.ustart[lo];
    decode_unit<FINAL>(a, sm, b_lo + lo, within % a.heads_kv, within / a.heads_kv);
  }
}

// 4 workgroups per compute unit; the persistent grid is sized for that
constexpr int WG_PER_CU = 4;
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void sinkattn_decode_split_bf16_d64(DecArgs a) {
  decode_split<false>(a);
}
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void sinkattn_decode_single_bf16_d64(DecArgs a) {
  decode_split<true>(a);
}

// One wave per (query head, sequence): merge the sequence's splits, apply the
// sink, write O (bf16) and the content-only log-sum-exp (natural log).  Lane
// s reads split s's (m, r) so the splits' loads go out together.
__global__ __launch_bounds__(64) void sinkattn_decode_combine_bf16_d64(DecArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int n = seq_len(a, b);
  bf16* out = a.o + ((size_t)b * a.heads_q + h) * D;
  if (n == 0) {   // no keys: O = 0, l = -inf
    out[lane] = (bf16)0.0f;
    if (a.lse && lane == 0) a.lse[(size_t)b * a.heads_q + h] = -INFINITY;
    return;
  }
  const int kvh = h / a.group;
  const int hc = h - kvh * a.group;
  const int ns = n_splits(a, n);
  const float* part = a.part + ((size_t)b * a.heads_kv + kvh) * a.max_splits * HMAX * PART + hc * PART;
  const size_t sstride = (size_t)HMAX * PART;
  float m = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) m = fmaxf(m, part[(s0 + lane) * sstride]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float r = 0.0f, x = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    const float f = s < ns ? fast_exp2(part[s * sstride] - m) : 0.0f;
    r += s < ns ? part[s * sstride + 1] * f : 0.0f;
    const int cnt = min(64, ns - s0);
    for (int j = 0; j < cnt; ++j)   // lane = head dim: weight of split s0 + j from lane j
      x += __shfl(f, j) * part[(s0 + j) * sstride + 2 + lane];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) r += __shfl_xor(r, off);
  const float denom = r + fast_exp2(a.sinks[h] * SA_LOG2E - m);
  out[lane] = (bf16)(x / denom);
  if (a.lse && lane == 0) a.lse[(size_t)b * a.heads_q + h] = (m + fast_log2(r)) * SA_LN2;
}

}  // namespace

// Chunks per wave and split count for a batch of sequences of up to t_max
// tokens: about SA_DECODE_TARGET_WGS workgroups when the longest sequence
// fills the cache (many short splits keep many independent chunk loads in
// flight; the combine reads one small partial per split).
#ifndef SA_DECODE_TARGET_WGS
#define SA_DECODE_TARGET_WGS 1024
#endif
void decode_plan(int batch, int t_max, int heads_kv, int window, int prefix, int* chunks_per_wave,
                 int* max_splits) {
  const int max_chunks = sa_decode_max_chunks(t_max, window, prefix, KW);
  const long long pairs = (long long)batch * heads_kv;
  long long target = pairs > 0 ? (SA_DECODE_TARGET_WGS + pairs - 1) / pairs : 1;
  if (target < 1) target = 1;
  long long cpw = (max_chunks + WAVES * target - 1) / (WAVES * target);
  if (cpw < 1) cpw = 1;
  *chunks_per_wave = (int)cpw;
  *max_splits = (int)((max_chunks + WAVES * cpw - 1) / (WAVES * cpw));
}

size_t decode_workspace_bytes(int batch, int t_max, int heads_kv, int window, int prefix) {
  int cpw, ms;
  decode_plan(batch, t_max, heads_kv, window, prefix, &cpw, &ms);
  return (size_t)batch * heads_kv * ms * HMAX * PART * sizeof(float);
}

// Workgroups of the persistent split kernel: WG_PER_CU per compute unit (its
// occupancy), at most the number of work units.
static int decode_grid(long long units_bound) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cus[dev] = c;
  }
  const long long g = (long long)WG_PER_CU * cus[dev];
  return (int)(units_bound < g ? (units_bound > 0 ? units_bound : 1) : g);
}

hipError_t launch_decode_bf16_d64(const bf16* q, const bf16* k, const bf16* v,
                                  const int* cache_seqlens, const float* sinks, bf16* o,
                                  float* lse, float* workspace, int batch, int t_max, int heads_q,
                                  int heads_kv, int window, int prefix, float scale,
                                  hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  DecArgs a;
  a.q = q; a.k = k; a.v = v; a.cache_seqlens = cache_seqlens; a.sinks = sinks; a.o = o;
  a.lse = lse; a.part = workspace;
  a.batch = batch; a.tmax = t_max; a.heads_q = heads_q; a.heads_kv = heads_kv;
  a.group = heads_q / heads_kv; a.window = window; a.prefix = prefix;
  a.scale_log2 = scale * SA_LOG2E;
  decode_plan(batch, t_max, heads_kv, window, prefix, &a.chunks_per_wave, &a.max_splits);
  const long long units_bound = (long long)batch * heads_kv * a.max_splits;
  if (units_bound > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.max_splits <= 1) {
    // every sequence fits one split: the split kernel applies the sink itself
    // (and writes O = 0, l = -inf for empty caches); no combine kernel
    hipLaunchKernelGGL(sinkattn_decode_single_bf16_d64, dim3(decode_grid((long long)batch * heads_kv)),
                       dim3(WAVES * 64), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(sinkattn_decode_split_bf16_d64, dim3(decode_grid(units_bound)),
                     dim3(WAVES * 64), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sinkattn_decode_combine_bf16_d64, dim3(heads_q, batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}
