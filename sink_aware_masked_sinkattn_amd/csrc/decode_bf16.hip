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
// Per 64-key chunk of visible keys a wave computes, with all the query heads
// of one kv head's group at once (every K and V row is read once per group):
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 -- 16 keys (A, rows of K read
//        straight from global memory) x the group's heads (B, in registers,
//        up to 16; unused columns are zero);
//   C layout: one head per lane, 4 keys per lane and tile, so the softmax
//        state (running max m, running sum r) is per lane;
//   O^T += V^T P^T -- A = V^T by transpose reads of the chunk's V rows staged
//        in the wave's own LDS tile, B = the probabilities straight from the
//        C layout (two 16-key tiles = 32 keys), so the accumulator too has
//        one head per lane (16 of the 64 head dims per lane).
// Two ways to spread the chunks over the GPU:
//  * single pass (every sequence's visible keys fit one workgroup, e.g.
//    short windows): a workgroup (4 waves) takes one (sequence, kv head),
//    the waves' (m, r, acc) merge in LDS and the sink is applied there;
//  * stream (long caches): each (sequence, kv head) segment's chunks are cut
//    into blocks of at most qc chunks (qc chosen on the device so the blocks
//    fit the grid), listed by sequence, block and kv head; wave w takes
//    block w, so waves carry equal work, neighbouring waves read the same
//    cache rows for neighbouring kv heads, and the next chunk's loads
//    overlap the current one's arithmetic.  Each wave writes its block's
//    partial (m, r, acc); a second kernel merges a segment's blocks and
//    applies the sink:
//      O = acc / (r + exp(s_h - m)),  l = m + log r    (log2 units inside).
// The decode step is bound by HBM (each visible K/V row is read once); the
// MFMA work is small next to it.
#include <mutex>

#include "common.h"
#include "mask_tiles.h"

namespace {

constexpr int D = 64;
constexpr int WAVES = 4;
constexpr int KW = 64;           // keys per chunk
constexpr int HMAX = 16;         // query heads per kv head (MFMA N columns)
constexpr int PARTS = D + 4;     // floats per (slot, head) partial: m, r, 2 unused, acc[64]
constexpr int QMIN = 4;          // fewest chunks per wave in the stream kernel
constexpr int STREAM_WG_MAX = 1024;   // grid bound of the stream kernel (sizes its workspace)

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
  int* seq_start;           // stream: [B + 2] first block of each sequence, block count, qc
  float* part;              // stream: [slots, group, PARTS]
  int batch, tmax, heads_q, heads_kv, group, window, prefix;
  int chunks_per_wave;      // single pass: chunks per wave
  float scale_log2;
};

constexpr int SEQ_WIN = 1024;    // sequences whose prefix sums sit in LDS at a time

__device__ __forceinline__ int seq_len(const DecArgs& a, int b) {
  const int n = a.cache_seqlens[b];
  return n < 0 ? 0 : (n > a.tmax ? a.tmax : n);
}

__device__ __forceinline__ int seq_chunks(const DecArgs& a, int b) {
  int r[4];
  return sa_decode_ranges(seq_len(a, b), a.window, a.prefix, KW, r);
}

// u[1..SEQ_WIN] hold counts; make u[0..SEQ_WIN] their exclusive prefix sum.
// Called by the whole workgroup after the counts are written; starts and
// ends with a barrier.
__device__ void scan_inplace(int* u) {
  const int tid = threadIdx.x;
  __syncthreads();
  if (tid < 64) {   // wave 0: each lane sums 16 consecutive counts, then a lane scan
    constexpr int E = SEQ_WIN / 64;
    int run = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) run += u[1 + tid * E + e];
    int inc = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(inc, off);
      if (tid >= off) inc += t;
    }
    int acc = inc - run;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc += u[1 + tid * E + e];
      u[1 + tid * E + e] = acc;
    }
    if (tid == 0) u[0] = 0;
  }
  __syncthreads();
}

// u[0..SEQ_WIN] = exclusive prefix sum of count(b) over sequences
// b_lo .. b_lo + SEQ_WIN - 1 (0 past the batch).  Called by the whole
// workgroup; ends with a barrier.
template <class F>
__device__ void scan_counts(int* u, int b_lo, int batch, F count) {
  __syncthreads();   // earlier readers of u are done
  for (int i = threadIdx.x; i < SEQ_WIN; i += WAVES * 64)
    u[i + 1] = (b_lo + i < batch) ? count(b_lo + i) : 0;
  scan_inplace(u);
}

// Q^T as the B operand for kv head kvh of sequence b: lane holds head col of
// the group, head dims 32*st + 8*grp .. +7 (zero for columns past the group)
__device__ __forceinline__ void load_q(const DecArgs& a, int b, int kvh, int col, int grp,
                                       bf16x8* qf) {
  const bool ok = col < a.group;
  const bf16* qp = a.q + ((size_t)b * a.heads_q + kvh * a.group + col) * D;
#pragma unroll
  for (int st = 0; st < 2; ++st) qf[st] = ok ? *(const bf16x8*)(qp + 32 * st + 8 * grp) : bf16x8{};
}

// K rows of keys [k0, k1) as the A operand of S^T: lane holds key
// k0 + 16t + col (rows past k1 repeat k1 - 1), head dims 32*st + 8*grp .. +7
__device__ __forceinline__ void load_k(const DecArgs& a, int b, int kvh, int k0, int k1, int col,
                                       int grp, bf16x8 (&kf)[4][2]) {
  const int kv_stride = a.heads_kv * D;
  const bf16* kb = a.k + ((size_t)b * a.tmax * a.heads_kv + kvh) * D + 8 * grp;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bf16* kp = kb + (size_t)min(k0 + 16 * t + col, k1 - 1) * kv_stride;
#pragma unroll
    for (int st = 0; st < 2; ++st) kf[t][st] = *(const bf16x8*)(kp + 32 * st);
  }
}

// V rows of keys [k0, k1) into the wave's swizzled LDS tile (rows past k1
// repeat k1 - 1; their probabilities are 0): lane i of 8-row block j copies
// the 16 bytes that belong at tile chunk i % 8 of row 8j + i / 8
// (buffer_load_dwordx4 ... lds writes lane i's 16 bytes at the block's LDS
// base + 16 i).  The buffer form rather than global_load_lds: the compiler
// treats a pending global_load_lds as a flat access to both memories and
// then turns every wait for a load into a wait for all of them; with the
// buffer form it tracks each copy, so the next chunk's K and Q loads stay in
// flight across the wait for this tile.  The descriptor starts at row k0 and
// covers every byte (offsets stay below 64 rows of the cache).
__device__ __forceinline__ void load_v(const DecArgs& a, int b, int kvh, int k0, int k1, bf16* vs,
                                       int lane) {
  const int kv_stride = a.heads_kv * D;
  const bf16* vb = a.v + ((size_t)b * a.tmax + k0) * kv_stride + (size_t)kvh * D;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, -1, 0x00020000);
  const int nvalid = k1 - k0;
#pragma unroll
  for (int j = 0; j < KW / 8; ++j) {
    const int r = 8 * j + (lane >> 3);
    const int rr = r < nvalid ? r : nvalid - 1;
    const int c = (lane & 7) ^ tile_swz(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(vs + 512 * j), 16,
                                             (rr * kv_stride + 8 * c) * 2, 0, 0, 0);
  }
}

// Transposed 4 x 16-bit read of a V tile.  Deliberately without restrict
// (unlike the training kernels' reads, whose tiles a barrier publishes): the
// compiler must see that it may read what a pending copy writes, so it waits
// for that copy -- and, with the buffer-form copy, for nothing younger.
__device__ __forceinline__ bf16x4 v_read_tr4(const bf16* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

// S^T of one chunk: lane = head col, keys k0 + 16t + 4*grp + i
__device__ __forceinline__ void s_tiles(const bf16x8 (&kf)[4][2], const bf16x8* qf, f32x4_t* s) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s[t] = mfma16x16x32(kf[t][0], qf[0], f32x4_t{0.f, 0.f, 0.f, 0.f});
    s[t] = mfma16x16x32(kf[t][1], qf[1], s[t]);
  }
}

// The rest of one chunk [k0, k1) with its S^T in s and V in the LDS tile vs:
// the online softmax update of (m_run, r_lane, acc) and O^T += V^T P^T.  The
// compiler waits for the tile's copy before the first read of vs (v_read_tr4).
__device__ __forceinline__ void softmax_pv(f32x4_t* s, const bf16* vs, int k0, int k1,
                                           float scale_log2, int col, int grp, float& m_run,
                                           float& r_lane, f32x4_t* acc) {
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k0 + 16 * t + 4 * grp + i;
      s[t][i] = key < k1 ? s[t][i] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[t][i]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);          // finite: every chunk has a key
  const float corr = fast_exp2(m_run - m_new);   // 0 on a segment's first chunk
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
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    const bf16x8 pb = to_bf16x8(p[2 * tp][0], p[2 * tp][1], p[2 * tp][2], p[2 * tp][3],
                                p[2 * tp + 1][0], p[2 * tp + 1][1], p[2 * tp + 1][2],
                                p[2 * tp + 1][3]);
    const int r0 = 32 * tp + 4 * grp + (col >> 2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int c0 = 16 * mb + 4 * (col & 3);
      const bf16x8 va = cat8(v_read_tr4(vs + tile_off(r0, c0)),
                             v_read_tr4(vs + tile_off(r0 + 16, c0)));
      acc[mb] = mfma16x16x32(va, pb, acc[mb]);
    }
  }
}

// ---------------------------------------------------------------------------
// Single pass: one workgroup per (sequence, kv head); wave w takes chunks
// [w*cpw, (w+1)*cpw) of the sequence's visible keys, the four waves' (m, r,
// acc) merge in LDS and the sink is applied there.

// LDS of the single-pass kernel: the waves' V tiles during a unit's chunk
// loop; the same memory then holds the four waves' results for the merge.
// ustart[j] is the first work unit of sequence b_lo + j (relative to the
// window).
struct __attribute__((aligned(16))) DecSmem {
  union {
    bf16 vtile[WAVES][KW * D];          // per wave, swizzled rows (tile_off)
    float red_acc[WAVES][HMAX][D];
  };
  float red_m[WAVES][HMAX], red_r[WAVES][HMAX];
  int ustart[SEQ_WIN + 1];
};

// One work unit: kv head kvh of sequence b.  Ends with a barrier (the LDS is
// reused by the next).
__device__ __forceinline__ void single_unit(const DecArgs& a, DecSmem& sm, int b, int kvh) {
  const int n = seq_len(a, b);
  int rng[4];
  const int nc = sa_decode_ranges(n, a.window, a.prefix, KW, rng);
  const int tid = threadIdx.x;
  if (nc == 0) {   // no keys: O = 0, l = -inf for the group's heads
    for (int e = tid; e < a.group * D; e += WAVES * 64) {
      const int hq = kvh * a.group + e / D;
      a.o[((size_t)b * a.heads_q + hq) * D + e % D] = (bf16)0.0f;
      if (a.lse && e % D == 0) a.lse[(size_t)b * a.heads_q + hq] = -INFINITY;
    }
    return;
  }

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;       // MFMA column: query head within the group
  const int grp = lane >> 4;       // 16-lane group
  bf16x8 qf[2];
  load_q(a, b, kvh, col, grp, qf);

  float m_run = -INFINITY;   // running max of this lane's head (log2 units)
  float r_lane = 0.0f;       // this lane's share of the running sum
  f32x4_t acc[4];            // O^T: rows d = 16*mb + 4*grp + i, column = head col
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  bf16* vs = sm.vtile[wave];
  const int c_begin = wave * a.chunks_per_wave;
  const int c_end = min(c_begin + a.chunks_per_wave, nc);
  for (int c = c_begin; c < c_end; ++c) {
    int k0, k1;
    sa_decode_chunk(rng, KW, c, &k0, &k1);
    load_v(a, b, kvh, k0, k1, vs, lane);
    bf16x8 kf[4][2];
    load_k(a, b, kvh, k0, k1, col, grp, kf);
    f32x4_t st[4];
    s_tiles(kf, qf, st);
    softmax_pv(st, vs, k0, k1, a.scale_log2, col, grp, m_run, r_lane, acc);
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
  for (int e = tid; e < a.group * D; e += WAVES * 64) {
    const int h = e / D, d = e % D;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) m = fmaxf(m, sm.red_m[w][h]);
    float r = 0.0f, x = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float f = fast_exp2(sm.red_m[w][h] - m);
      r += sm.red_r[w][h] * f;
      x += sm.red_acc[w][h][d] * f;
    }
    const int hq = kvh * a.group + h;
    const float denom = r + fast_exp2(a.sinks[hq] * SA_LOG2E - m);
    a.o[((size_t)b * a.heads_q + hq) * D + d] = (bf16)(x / denom);
    if (a.lse && d == 0) a.lse[(size_t)b * a.heads_q + hq] = (m + fast_log2(r)) * SA_LN2;
  }
  __syncthreads();   // the next unit's tile loads overwrite red_acc
}

// Persistent grid: each workgroup takes units blockIdx.x, + gridDim.x, ... of
// the flat list (sequence by sequence, kv heads fastest) until it passes the
// list's end, which every workgroup computes from the batch size the same
// way -- so every one exits.  A sequence with no keys still gets its units
// (they write O = 0, l = -inf).
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void sinkattn_decode_single_bf16_d64(DecArgs a) {
  __shared__ DecSmem sm;
  int b_lo = 0;
  int base = 0;   // units before sequence b_lo
  const int hkv = a.heads_kv;
  scan_counts(sm.ustart, b_lo, a.batch, [hkv](int) { return hkv; });
  for (int u = blockIdx.x;; u += gridDim.x) {
    while (u - base >= sm.ustart[SEQ_WIN]) {
      if (b_lo + SEQ_WIN >= a.batch) return;   // past the last sequence
      base += sm.ustart[SEQ_WIN];
      b_lo += SEQ_WIN;
      scan_counts(sm.ustart, b_lo, a.batch, [hkv](int) { return hkv; });
    }
    const int local = u - base;
    int lo = 0, hi = SEQ_WIN;   // largest j with ustart[j] <= local
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm.ustart[mid] <= local) lo = mid; else hi = mid;
    }
    // uniform by construction; readfirstlane lets the compiler keep the copy
    // descriptors in scalar registers
    const int within = __builtin_amdgcn_readfirstlane(local - sm.ustart[lo]);
    single_unit(a, sm, __builtin_amdgcn_readfirstlane(b_lo + lo), within);
  }
}

// ---------------------------------------------------------------------------
// Stream: the visible chunks of each (sequence b, kv head) are cut into
// blocks of qc consecutive chunks, the blocks are listed by sequence, then
// block index, then kv head (bstart[b] = first block of sequence b), and wave
// w of the grid takes block w (and w + waves, ... if there are more blocks
// than waves).  Neighbouring waves -- the four of a workgroup -- thus read
// the same key rows of neighbouring kv heads at the same time: a cache row
// holds every kv head, so its pieces are fetched together.  qc is the
// smallest of max(QMIN, ceil(C / waves)) and max(QMIN, ceil(C / (waves - S)))
// whose block count fits the grid (C chunks in S nonempty segments: a
// segment of n chunks has ceil(n / qc) <= n / qc + 1 blocks), so no wave
// carries more than qc chunks.  Each block's partial (m, r, acc) goes to slot
// w; the combine kernel merges the blocks of a segment (slots bstart[b] +
// j*Hkv + kvh, j = 0, 1, ...) and applies the sink.

struct __attribute__((aligned(16))) StreamSmem {
  bf16 vtile[WAVES][KW * D];   // per wave, swizzled rows (tile_off)
  int bstart[SEQ_WIN + 1];     // chunks of each sequence, then its first block
  int red[WAVES];
};

// Sum over the workgroup (every thread calls; contains barriers)
__device__ __forceinline__ int wg_sum(int v, int* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();   // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) t += red[w];
  return t;
}

// This lane's share of a partial: m and the group-summed r (lanes of 16-lane
// group 0), acc rows 16*mb + 4*grp .. +3 of head col
__device__ __forceinline__ void write_partial(const DecArgs& a, int slot, int col, int grp,
                                              float m_run, float r_lane, const f32x4_t* acc) {
  float r = r_lane + __shfl_xor(r_lane, 16);
  r += __shfl_xor(r, 32);
  if (col < a.group) {
    float* ph = a.part + ((size_t)slot * a.group + col) * PARTS;
    if (grp == 0) *(float2*)ph = make_float2(m_run, r);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) *(f32x4_t*)(ph + 4 + 16 * mb + 4 * grp) = acc[mb];
  }
}

// Block w of the list (w wave-uniform).  Per chunk the next chunk's K rows
// are loaded right after S^T has used kf and its V rows right after the last
// read of the tile, so the wait for K at the top of an iteration leaves that
// chunk's V copy in flight and the wait for V leaves the next K.
__device__ __forceinline__ void stream_block(const DecArgs& a, StreamSmem& sm, int w, int qc) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  bf16* vs = sm.vtile[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];

  int lo = 0, hi = a.batch;   // bstart[lo] <= w < bstart[hi]: sequence lo holds block w
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(sm.bstart[mid]) <= w) lo = mid; else hi = mid;
  }
  const int b = __builtin_amdgcn_readfirstlane(lo);
  const int r = w - __builtin_amdgcn_readfirstlane(sm.bstart[b]);
  const int j = r / a.heads_kv;
  const int kvh = r - j * a.heads_kv;
  int rng[4];
  const int nc = sa_decode_ranges(seq_len(a, b), a.window, a.prefix, KW, rng);
  const int c0 = j * qc;
  const int c1 = min(c0 + qc, nc);

  int k0, k1;
  sa_decode_chunk(rng, KW, c0, &k0, &k1);
  bf16x8 qf[2], kf[4][2];
  load_k(a, b, kvh, k0, k1, col, grp, kf);
  load_q(a, b, kvh, col, grp, qf);
  // a previous block's reads of vs have returned before the copy overwrites it
  __builtin_amdgcn_s_waitcnt(0xc07f);
  load_v(a, b, kvh, k0, k1, vs, lane);

  float m_run = -INFINITY, r_lane = 0.0f;
  f32x4_t acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t st[4];
  for (int c = c0; c + 1 < c1; ++c) {
    s_tiles(kf, qf, st);
    int n0, n1;
    sa_decode_chunk(rng, KW, c + 1, &n0, &n1);
    load_k(a, b, kvh, n0, n1, col, grp, kf);   // kf is free once S^T has read it
    softmax_pv(st, vs, k0, k1, a.scale_log2, col, grp, m_run, r_lane, acc);
    // every read of vs has returned (lgkmcnt 0) before the next copy overwrites it
    __builtin_amdgcn_s_waitcnt(0xc07f);
    load_v(a, b, kvh, n0, n1, vs, lane);
    k0 = n0;
    k1 = n1;
  }
  s_tiles(kf, qf, st);
  softmax_pv(st, vs, k0, k1, a.scale_log2, col, grp, m_run, r_lane, acc);
  write_partial(a, w, col, grp, m_run, r_lane, acc);
}

// Grid of gridDim.x <= STREAM_WG_MAX workgroups.  Every workgroup computes
// qc and bstart from cache_seqlens the same way; workgroup 0 also stores
// them for the combine kernel.  No barrier follows, so waves finish on their
// own.
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void sinkattn_decode_stream_bf16_d64(DecArgs a) {
  __shared__ StreamSmem sm;
  const int tid = threadIdx.x;
  int mine = 0, nonempty = 0;
  for (int i = tid; i < SEQ_WIN; i += WAVES * 64) {
    const int c = i < a.batch ? seq_chunks(a, i) : 0;
    sm.bstart[i + 1] = c;
    mine += c;
    nonempty += c > 0;
  }
  const int total = a.heads_kv * wg_sum(mine, sm.red);
  const int segs = a.heads_kv * wg_sum(nonempty, sm.red);
  const int waves = gridDim.x * WAVES;
  int qc = max((total + waves - 1) / waves, QMIN);
  int nb = 0;
  for (int i = tid; i < a.batch; i += WAVES * 64) nb += (sm.bstart[i + 1] + qc - 1) / qc;
  if (a.heads_kv * wg_sum(nb, sm.red) > waves && waves > segs)
    qc = max((total + (waves - segs) - 1) / (waves - segs), QMIN);
  for (int i = tid; i < a.batch; i += WAVES * 64)
    sm.bstart[i + 1] = a.heads_kv * ((sm.bstart[i + 1] + qc - 1) / qc);
  scan_inplace(sm.bstart);
  const int nblocks = sm.bstart[a.batch];
  if (blockIdx.x == 0) {
    for (int i = tid; i <= a.batch; i += WAVES * 64) a.seq_start[i] = sm.bstart[i];
    if (tid == 0) a.seq_start[a.batch + 1] = qc;
  }
  for (int w = blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(tid >> 6); w < nblocks;
       w += waves)
    stream_block(a, sm, w, qc);
}

// One wave per (query head, sequence): merge the partials of the head's
// blocks, apply the sink, write O (bf16) and the content-only log-sum-exp
// (natural log).  Lane s reads partial s's (m, r) so their loads go out
// together.
__global__ __launch_bounds__(64) void sinkattn_decode_combine_bf16_d64(DecArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int n = seq_len(a, b);
  bf16* out = a.o + ((size_t)b * a.heads_q + h) * D;
  int rng[4];
  const int nc = sa_decode_ranges(n, a.window, a.prefix, KW, rng);
  if (nc == 0) {   // no keys: O = 0, l = -inf
    out[lane] = (bf16)0.0f;
    if (a.lse && lane == 0) a.lse[(size_t)b * a.heads_q + h] = -INFINITY;
    return;
  }
  const int kvh = h / a.group;
  const int hc = h - kvh * a.group;
  const int qc = a.seq_start[a.batch + 1];
  const int ns = (nc + qc - 1) / qc;   // blocks j = 0 .. ns-1 at slots bstart[b] + j*Hkv + kvh
  const size_t sstride = (size_t)a.heads_kv * a.group * PARTS;
  const float* part = a.part + ((size_t)(a.seq_start[b] + kvh) * a.group + hc) * PARTS;
  // 64 partials at a time (one round unless a segment has more than 64
  // blocks): lane s holds partial s's (m, r), the block's maximum
  // rescales the running sums, and eight partials' acc loads go out together
  // (lane = head dim; the weight of partial j comes from lane j).  Every
  // partial has m finite (its wave saw at least one visible key).
  float m = -INFINITY, r_lane = 0.0f, x = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    const int cnt = min(64, ns - s0);
    const float2 mr = s < ns ? *(const float2*)(part + (size_t)s * sstride)
                             : make_float2(-INFINITY, 0.0f);
    float mb = mr.x;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mb = fmaxf(mb, __shfl_xor(mb, off));
    const float m_new = fmaxf(m, mb);
    const float sc = fast_exp2(m - m_new);   // 0 on the first round
    const float f_s = s < ns ? fast_exp2(mr.x - m_new) : 0.0f;
    r_lane = r_lane * sc + mr.y * f_s;
    x *= sc;
    m = m_new;
    for (int j0 = 0; j0 < cnt; j0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = j0 + u < cnt ? part[(size_t)(s0 + j0 + u) * sstride + 4 + lane] : 0.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u) x += __shfl(f_s, j0 + u) * v[u];
    }
  }
  float r = r_lane;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) r += __shfl_xor(r, off);
  const float denom = r + fast_exp2(a.sinks[h] * SA_LOG2E - m);
  out[lane] = (bf16)(x / denom);
  if (a.lse && lane == 0) a.lse[(size_t)b * a.heads_q + h] = (m + fast_log2(r)) * SA_LN2;
}

}  // namespace

// Plan of one decode call.  single: every sequence's visible keys fit one
// workgroup of the single-pass kernel, with chunks_per_wave chunks per wave
// chosen so that about DECODE_TARGET_WGS workgroups would cover a batch
// of full caches; otherwise the stream kernel runs (then batch * heads_kv <
// DECODE_TARGET_WGS <= SEQ_WIN, so the batch's prefix sums fit its LDS).
constexpr int DECODE_TARGET_WGS = 1024;
static_assert(DECODE_TARGET_WGS <= SEQ_WIN, "the stream kernel scans the batch in one window");
struct DecodePlan {
  bool single;
  int chunks_per_wave;   // single pass
  long long max_chunks;  // per sequence and kv head, over every length <= t_max
};

static DecodePlan decode_plan(int batch, int t_max, int heads_kv, int window, int prefix) {
  DecodePlan pl;
  const int max_chunks = sa_decode_max_chunks(t_max, window, prefix, KW);
  pl.max_chunks = max_chunks;
  const long long pairs = (long long)batch * heads_kv;
  long long target = pairs > 0 ? (DECODE_TARGET_WGS + pairs - 1) / pairs : 1;
  if (target < 1) target = 1;
  long long cpw = (max_chunks + WAVES * target - 1) / (WAVES * target);
  if (cpw < 1) cpw = 1;
  pl.single = (max_chunks + WAVES * cpw - 1) / (WAVES * cpw) <= 1 || batch > SEQ_WIN ||
              pairs * max_chunks > (1LL << 30);
  // one pass over a sequence's chunks per workgroup
  if (pl.single) cpw = (max_chunks + WAVES - 1) / WAVES > cpw ? (max_chunks + WAVES - 1) / WAVES : cpw;
  pl.chunks_per_wave = (int)(cpw < 1 ? 1 : cpw);
  return pl;
}

// Stream workspace: seq_start [batch + 2] ints, then the partials of
// STREAM_WG_MAX * WAVES + batch * heads_kv slots of the group's query heads
// (the blocks number at most C / qc + S <= waves + batch * heads_kv).  The
// single pass uses none; 256 bytes are still asked for, so the workspace
// argument is required either way.
static size_t stream_part_offset(int batch) {
  return (((size_t)batch + 2) * sizeof(int) + 255) & ~(size_t)255;
}

size_t decode_workspace_bytes(int batch, int t_max, int heads_q, int heads_kv, int window,
                              int prefix) {
  const DecodePlan pl = decode_plan(batch, t_max, heads_kv, window, prefix);
  if (pl.single) return 256;
  const size_t slots = (size_t)STREAM_WG_MAX * WAVES + (size_t)batch * heads_kv;
  return stream_part_offset(batch) + slots * (size_t)(heads_q / heads_kv) * PARTS * sizeof(float);
}

// ---------------------------------------------------------------------------
// The allocation-free decode entry point's workspace: a static array of the
// library in device memory (one copy per GPU, held until the process ends).
// Host code never passes the array's name to a kernel (on the host it only
// names a stand-in); it looks up the device address once per device with
// hipGetSymbolAddress, with that device current, and passes that address.
// Size: the stream kernel runs only when batch * heads_kv < 1024, so its
// workspace is at most 4352 + (4096 + 1023) slots * 16 heads * PARTS floats
// = 22,282,240 bytes; the single pass needs none.  24 MiB so covers every
// problem sinkattn_decode accepts; the entry point still checks the size.
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)24 << 20;
static __device__ __align__(256) unsigned char scratch[DECODE_SCRATCH_BYTES];

size_t decode_scratch_bytes() { return DECODE_SCRATCH_BYTES; }

// Device address of the current device's copy of `scratch`.
hipError_t decode_scratch(void** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cus[dev] = c;
  }
  return cus[dev];
}

// 4 workgroups per compute unit (the kernels' occupancy)
constexpr int WG_PER_CU = 4;

hipError_t launch_decode_bf16_d64(const bf16* q, const bf16* k, const bf16* v,
                                  const int* cache_seqlens, const float* sinks, bf16* o,
                                  float* lse, float* workspace, int batch, int t_max, int heads_q,
                                  int heads_kv, int window, int prefix, float scale,
                                  hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  DecArgs a;
  a.q = q; a.k = k; a.v = v; a.cache_seqlens = cache_seqlens; a.sinks = sinks; a.o = o;
  a.lse = lse;
  a.batch = batch; a.tmax = t_max; a.heads_q = heads_q; a.heads_kv = heads_kv;
  a.group = heads_q / heads_kv; a.window = window; a.prefix = prefix;
  a.scale_log2 = scale * SA_LOG2E;
  const DecodePlan pl = decode_plan(batch, t_max, heads_kv, window, prefix);
  a.chunks_per_wave = pl.chunks_per_wave;
  const long long slots_wg = (long long)WG_PER_CU * device_cus();
  if (pl.single) {
    // one unit per (sequence, kv head); units with no keys write O = 0, l = -inf
    a.seq_start = nullptr;
    a.part = nullptr;
    const long long units = (long long)batch * heads_kv;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int grid = (int)(units < slots_wg ? units : slots_wg);
    hipLaunchKernelGGL(sinkattn_decode_single_bf16_d64, dim3(grid), dim3(WAVES * 64), 0, stream, a);
    return hipGetLastError();
  }
  a.seq_start = reinterpret_cast<int*>(workspace);
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + stream_part_offset(batch));
  // enough workgroups for QMIN chunks per wave over a batch of full caches,
  // at most the resident count and STREAM_WG_MAX
  const long long chunk_bound = (long long)batch * heads_kv * pl.max_chunks;
  long long grid = (chunk_bound + WAVES * QMIN - 1) / (WAVES * QMIN);
  if (grid > slots_wg) grid = slots_wg;
  if (grid > STREAM_WG_MAX) grid = STREAM_WG_MAX;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(sinkattn_decode_stream_bf16_d64, dim3((int)grid), dim3(WAVES * 64), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sinkattn_decode_combine_bf16_d64, dim3(heads_q, batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}
