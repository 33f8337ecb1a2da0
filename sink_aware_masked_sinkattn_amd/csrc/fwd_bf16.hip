// Forward of sink-aware masked attention, bf16 in / bf16 out, head dim 64,
// on gfx950 MFMA.
//
// What it computes: for each query row q of head h, over the keys that the
// mask M[q,k] = 1[k<=q] AND 1[q-k<=w OR k<p] leaves visible,
//   l[q] = log sum_k exp(scale q.k)           (content-only log-sum-exp)
//   O[q] = sigmoid(l[q] - s_h) * softmax(scale q.K) V
// ("Efficient Reinforcement Learning for Long-Horizon Tool-Use Agentic
// Tasks", summary page, sink-aware FlexAttention paragraph; the equivalence
// with an explicit zero-value sink column is arXiv 2608.10357 section 5,
// "Zero-value sink equivalence").  The score matrix is never stored: key tiles
// stream through LDS and an online softmax (running max m, running sum r)
// keeps fp32 state per row, in the blockwise exact form the same section cites
// (FlashAttention).  Because
//   sigmoid(l - s) * Obar = acc / (r + exp(s - m)) when acc = sum exp(S - m) v,
// the sink scaling costs one extra exponential per row in the epilogue.
//
// Work decomposition (one workgroup = WAVES waves x QB*32 query rows of one
// head: 4 waves x 64 rows at 2 waves per SIMD for 64-key tiles, 4 waves x 32
// rows for 32-key tiles -- or, for windows under 1024 with GQA groups of a
// multiple of 4, four query heads of one kv group x the same 32 rows, so the
// workgroup loads the key tiles of 32 rows (w/32 + 2 tiles) once for four
// heads and every wave uses every tile):
//   * each wave owns QB 32-row MFMA blocks of query rows whose Q fragments
//     stay in registers for the whole kernel; each key tile's K and V^T
//     operands are read from LDS once, up front, and shared by the blocks;
//   * key tiles of 64 rows are listed per workgroup from the mask (prefix
//     tiles + window tiles, each once), double-buffered in LDS: K row-major,
//     V row-major and read transposed with ds_read_tr16_b64;
//   * S^T = K Q^T puts one query per lane (C layout), so the row max / sum
//     need only a 32-lane swap, and the probabilities convert in registers
//     into the B operand of O^T += V^T P^T (with 64-key tiles a 16x16x32
//     MFMA against a 0/1 selector also forms the row sums from fp16 copies);
//   * each wave classifies every key tile against its own rows: skipped
//     tiles cost nothing, full tiles run mask-free, partial tiles apply the
//     element predicate (with 32-key tiles, in a one-sided form -- one
//     compare per element -- when the tile's geometry allows, mask_form);
//   * grid z runs from the last query tile to the first (longest rows start
//     first); grid x maps the heads so that one kv-group's query heads share
//     an XCD and its L2 (consecutive workgroups go to consecutive XCDs).
#include "common.h"
#include "mask_tiles.h"

namespace {

constexpr int D = 64;
// 32-row query blocks per wave of the 64-key-tile kernel: two, so every K
// and V^T operand read from LDS (and the per-tile softmax bookkeeping) serves
// 64 rows (0.619 -> 0.604 ms for a causal T=8192 layer against one block at 3
// waves per SIMD).  The 32-key-tile kernels keep one block per wave.
constexpr int QB64 = 2;
constexpr int WAVES = 4;    // waves per workgroup
// Key tiles hold NKB blocks of 32 keys: 64-key tiles in general, 32-key
// tiles for short windows, where a 32-row query block needs only w + 32 keys
// and wider tiles would mostly compute masked pairs.
constexpr int OROW = D + 8;              // padded row of the epilogue staging buffer
// LDS: two K/V tile pairs during the key loop; afterwards the same memory
// stages each wave's output rows (padded) for row-contiguous stores.
template <int NKB, int QB>
struct FwdTiles {
  static constexpr int BK = 32 * NKB;                 // key rows per LDS tile
  static constexpr int TILE_ELEMS = BK * D;           // swizzled rows (tile_off)
  static constexpr int STAGE_ELEMS = WAVES * QB * 32 * OROW;
  static constexpr int SMEM_ELEMS = (4 * TILE_ELEMS > STAGE_ELEMS) ? 4 * TILE_ELEMS : STAGE_ELEMS;
  static_assert(SMEM_ELEMS >= 4 * TILE_ELEMS && SMEM_ELEMS >= STAGE_ELEMS, "LDS sizing");
};
// Lazy rescaling: the running max used for the exponentials is only moved when
// a row's true max exceeds it by more than this (log2 units), so probabilities
// stay below 2^8 and most key tiles skip the accumulator rescale entirely.
constexpr float RESCALE_THRESHOLD = 8.0f;

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* sinks;
  bf16* o;
  float* lse;                // may be null
  const int* cu_seqlens;     // null for fixed length
  int batch, seqlen, heads_q, heads_kv, group, window, prefix;
  int lse_head_stride;       // T (fixed) or N (varlen)
  int num_q_tiles;           // fixed length: query tiles per sequence
  float scale_log2;          // softmax_scale * log2(e)
};

__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// A operand of the 16x16x32 MFMA that sums probabilities per query.  Fed a
// P^T register of the 32x32 layout (lane l: query l%32 and 8 of the 16 keys
// of a k-step, which 8 set by l/32), the 16x16x32 product reads lane l as
// column l%16 of k-group l/16, so k-groups {0,2} carry queries 0..15 and
// {1,3} queries 16..31.  Ones in A rows m = 0, 4, 8, 12 over the k-groups of
// parity (m/4)%2 put the sum for query n + 16*((m/4)%2) at row m, column n;
// since the C layout gives lane l rows 4*(l/16)+i of column l%16, register 0
// of every lane ends up holding the sum for that lane's own query.
// The probabilities enter this product as fp16 (11-bit significand, RNE):
// each is within 2^-11 of its value, so l = m + ln(sum) is within
// ln(1 + 2^-11) = 4.9e-4 of the log of the fp32 sum; with bf16 copies (the
// ones that weight V) the bound would be ln(1 + 2^-8) = 3.9e-3.
__device__ __forceinline__ f16x8 row_sum_selector(int lane) {
  const int m = lane & 15;
  const bool one = (m & 3) == 0 && ((m >> 2) & 1) == ((lane >> 4) & 1);
  const _Float16 v = one ? (_Float16)1.0f : (_Float16)0.0f;
  return f16x8{v, v, v, v, v, v, v, v};
}

__device__ __forceinline__ int map_head(int x, int heads_q) {
  // consecutive workgroups land on consecutive XCDs (8): give XCD c the
  // contiguous head range [c*Hq/8, (c+1)*Hq/8) so a kv-group stays in one L2
  if ((heads_q & 7) == 0) return (x & 7) * (heads_q >> 3) + (x >> 3);
  return x;
}

// One key tile (NKB blocks of 32 keys) against this wave's QB blocks of 32
// query rows.  MASK: apply the element predicate (partial tiles only).
template <int NKB, int QB, bool MASK>
__device__ __forceinline__ void tile_step(uint32_t ktile, const bf16x8 (&qf)[QB][4],
                                          f32x16 (&acc)[QB][2], float (&m_run)[QB],
                                          f32x4 (&rsum)[QB], f16x8 rsel, int qw0, int k0, int window,
                                          int prefix, float scale_log2, int lane) {
  // Row sums of the probabilities: for 64-key tiles on the matrix cores, from
  // fp16 copies of the P^T registers the PV product uses (8 small MFMAs and 32
  // packing converts instead of 64 fp32 adds per lane; this kernel is
  // VALU-bound).  The 32-key kernels run at 4 waves per SIMD and have no
  // registers for the extra accumulators; they add in fp32 per lane
  // (register 0 of rsum, a partial over this lane's keys).
  constexpr bool MSUM = NKB == 2;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int grp = lane >> 4;
  const int li = lane & 15;
  // ---- operands of this tile, all issued up front so the LDS latency is
  // paid once: K (keys on m, head dim on k) and V^T (head dim on m, keys on
  // k, by transpose reads).  The K tile is at LDS byte address ktile, the V
  // tile right after it; one base register per read pattern, recomputed per
  // tile (every other address is that base XOR a constant plus an immediate).
  constexpr int VOFF = NKB * 32 * 128;
  const uint32_t ra = (uint32_t)sa_opaque((int)ktile + tile_row_base(l32, g));
  const uint32_t ta =
      (uint32_t)sa_opaque((int)ktile + VOFF + tile_tr_base(4 * g + (li >> 2), 16 * (grp & 1) + 4 * (li & 3)));
  bf16x8 kf[NKB][4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int s = 0; s < 4; ++s) kf[kb][s] = lds_read8((ra ^ (32 * s)) + kb * 4096);
  // V^T: rows kb*32 + 16*hh + 4g + li/4 (+8), columns db*32 + 16*(grp&1) + 4*(li&3)
  bf16x8 vt[2][NKB][2];   // [db][kb][hh]
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int o = kb * 4096 + hh * 2048;   // folds into the immediate offset
        vt[db][kb][hh] = cat8(lds_read_tr4_at((ta ^ (64 * db)) + o),
                              lds_read_tr4_at((ta ^ (64 * db + 32)) + o + 1024));
      }
  // ---- S^T = K Q^T for both 32-key blocks and all query blocks: lane =
  // query, 16 keys per block in registers
  f32x16 st[NKB][QB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) st[kb][qb] = f32x16{};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) st[kb][qb] = mfma32x32x16(kf[kb][s], qf[qb][s], st[kb][qb]);
  if (MASK) {
    // element i of key block kb holds key kr + 8*(i/4) + i%4, kr = k0 + kb*32 + 4g
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (NKB == 1) {
          // window layers: most partial tiles take a one-sided form
          mask_query_block(st[kb][qb], qw0 + qb * 32, k0 + kb * 32, lane, window, prefix);
        } else {
          // 64-key tiles (long windows, causal): few partial tiles; the general
          // predicate keeps the kernel within its registers
          const int kr = k0 + kb * 32 + 4 * g;
          const int base = sa_opaque(qw0 + qb * 32 + l32 - kr);
          mask_query_lane<true>(st[kb][qb], base, sa_opaque(prefix - kr), window);
        }
      }
  }
  // ---- online softmax in the log2 domain, lazily rescaled
  bf16x8 pf[NKB][QB][2];
  f16x8 hf[NKB][QB][2];   // fp16 copies of the probabilities for the row sums
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = st[0][qb][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kb][qb][i]);
    mx = halves_max(mx) * scale_log2;
    if (__any(mx > m_run[qb] + RESCALE_THRESHOLD)) {
      const float m_new = fmaxf(m_run[qb], mx);
      const float corr = fast_exp2(m_run[qb] - m_new);
      m_run[qb] = m_new;
      rsum[qb][0] *= corr;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[qb][db][i] *= corr;
    }
    const float m_use = m_run[qb];
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(fmaf(st[kb][qb][i], scale_log2, -m_use));
        if (!MSUM) rs += p[i];
      }
      pf[kb][qb][0] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      pf[kb][qb][1] = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
      if (MSUM) {
        hf[kb][qb][0] = to_f16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        hf[kb][qb][1] = to_f16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
      }
    }
    if (!MSUM) rsum[qb][0] += rs;
  }
  // ---- O^T += V^T P^T
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32x32x16(vt[db][kb][hh], pf[kb][qb][hh], acc[qb][db]);
  if (MSUM) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) rsum[qb] = mfma16x16x32_f16(rsel, hf[kb][qb][hh], rsum[qb]);
  }
}

constexpr int FWD_OCC = 2;       // waves per SIMD the 64-key kernel's register budget is set for
constexpr int FWD_OCC_K32 = 4;   // the same for the 32-key kernels
// HW: waves along heads.  HW = 1: the workgroup's waves take consecutive
// row blocks of one head.  HW = 4 (short windows, GQA groups of a multiple
// of 4): they take four query heads of one kv group on the same rows, so the
// workgroup's key tiles are those of QB*32 rows only and every wave uses
// every tile (the K/V tiles are shared by the four heads).
template <int NKB, int HW, int QB>
__device__ __forceinline__ void fwd_body(const FwdArgs& a) {
  using T = FwdTiles<NKB, QB>;
  constexpr int BK = T::BK;
  constexpr int TILE_ELEMS = T::TILE_ELEMS;
  static_assert(WAVES % HW == 0, "the waves split into HW heads x row blocks");
  constexpr int BQW = (WAVES / HW) * QB * 32;   // query rows per workgroup
  __shared__ __attribute__((aligned(128))) bf16 smem[T::SMEM_ELEMS];   // K0 V0 K1 V1, then output staging

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  // h0: the workgroup's first head (uniform); the HW heads share its kv head
  const int h0 = HW == 1 ? map_head(blockIdx.x, a.heads_q) : map_head(blockIdx.x, a.heads_q / HW) * HW;
  const int h = h0 + (HW == 1 ? 0 : wave % HW);
  int z = 0, qt = 0;
  if (!launch_tile(a.cu_seqlens, a.batch, a.num_q_tiles, BQW, &z, &qt)) return;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int q_start = qt * BQW;
  if (q_start >= sv.len) return;
  const int q_last = min(q_start + BQW - 1, sv.len - 1);
  const int kvh = h0 / a.group;

  const int qw0 = q_start + (wave / HW) * (QB * 32);
  const bool wave_active = qw0 < sv.len;
  const int qw1 = min(qw0 + QB * 32 - 1, sv.len - 1);

  const int q_row_stride = a.heads_q * D;
  const int kv_row_stride = a.heads_kv * D;
  const bf16* qbase = a.q + (size_t)sv.row_base * q_row_stride + (size_t)h * D;
  const bf16* kbase = a.k + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;
  const bf16* vbase = a.v + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;

  // Q fragments (B operand of S^T = K Q^T): lane holds query l32 of each
  // block, head-dim chunk 16s + 8g .. +7.
  bf16x8 qf[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + l32;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (row < sv.len) {
        qf[qb][s] = *(const bf16x8*)(qbase + (size_t)row * q_row_stride + 16 * s + 8 * g);
      } else {
        qf[qb][s] = bf16x8{};
      }
    }
  }

  int seg[4];
  const int nseg = sa_key_tile_segments(q_start, q_last, a.window, a.prefix, BK, seg);
  const int n0 = seg[1] - seg[0];
  const int ntiles = n0 + (nseg > 1 ? seg[3] - seg[2] : 0);

  // cooperative tile load: 512 chunks of 16 B per tensor, 2 per thread
  // K / V tiles go straight from global memory into swizzled LDS tiles
  const TileLane tl = tile_lane(lane, kv_row_stride * 2);
  auto load_tile = [&](int t, int buf) {
    const int kt = t < n0 ? seg[0] + t : seg[2] + (t - n0);
    const int r0 = kt * BK;
    tile_load_lds_lane<BK, WAVES>(smem + (2 * buf) * TILE_ELEMS, kbase + (size_t)r0 * kv_row_stride,
                                  kv_row_stride * 2, sv.len - r0, wave, tl);
    tile_load_lds_lane<BK, WAVES>(smem + (2 * buf + 1) * TILE_ELEMS, vbase + (size_t)r0 * kv_row_stride,
                                  kv_row_stride * 2, sv.len - r0, wave, tl);
  };

  f32x16 acc[QB][2];
  f32x4 rsum[QB];
  float m_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    acc[qb][0] = f32x16{};
    acc[qb][1] = f32x16{};
    rsum[qb] = f32x4{};
    m_run[qb] = -1.0e30f;   // finite start: exp2(S - m) never sees (-inf) - (-inf)
  }
  const f16x8 rsel = row_sum_selector(lane);

  load_tile(0, 0);
  wait_all_mem();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1, buf ^ 1);
    const int kt = t < n0 ? seg[0] + t : seg[2] + (t - n0);
    const int k0 = kt * BK;
    const int cls = wave_active ? sa_tile_class(qw0, qw1, k0, k0 + BK - 1, a.window, a.prefix)
                                : SA_TILE_SKIP;
    const uint32_t ktile = lds_addr(smem + (2 * buf) * TILE_ELEMS);   // V tile follows
    if (cls == SA_TILE_FULL) {
      tile_step<NKB, QB, false>(ktile, qf, acc, m_run, rsum, rsel, qw0, k0, a.window, a.prefix, a.scale_log2, lane);
    } else if (cls == SA_TILE_PARTIAL) {
      tile_step<NKB, QB, true>(ktile, qf, acc, m_run, rsum, rsel, qw0, k0, a.window, a.prefix, a.scale_log2, lane);
    }
    wait_all_mem();
    __syncthreads();
  }

  // ---- epilogue: O = acc / (r + exp(s - m)), l = ln(2) * (m + log2 r)
  // Stage each wave's 64 x 64 output through LDS for row-contiguous stores.
  bf16* os = smem + wave * (QB * 32) * OROW;   // QB*32 rows x OROW per wave
  const float sink_l2 = a.sinks[h] * SA_LOG2E;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float r_tot = NKB == 2 ? rsum[qb][0] : halves_sum(rsum[qb][0]);
    const float denom = r_tot + fast_exp2(sink_l2 - m_run[qb]);
    const float inv = 1.0f / denom;
    const int qrow = qw0 + qb * 32 + l32;
    if (a.lse && wave_active && g == 0 && qrow < sv.len) {
      a.lse[sv.lse_base + (size_t)h * a.lse_head_stride + qrow] = (m_run[qb] + fast_log2(r_tot)) * SA_LN2;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * g;
        *(bf16x4*)(os + (qb * 32 + l32) * OROW + d) =
            to_bf16x4(acc[qb][db][4 * i4] * inv, acc[qb][db][4 * i4 + 1] * inv,
                      acc[qb][db][4 * i4 + 2] * inv, acc[qb][db][4 * i4 + 3] * inv);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  if (wave_active) {
    bf16* obase = a.o + (size_t)sv.row_base * q_row_stride + (size_t)h * D;
#pragma unroll
    for (int it = 0; it < (QB * 32 * D) / (64 * 8); ++it) {   // 64 lanes x 16 B per iteration
      const int chunk = it * 64 + lane;
      const int r = chunk >> 3;
      const int c = (chunk & 7) * 8;
      const int qrow = qw0 + r;
      if (qrow < sv.len) {
        *(uint4*)(obase + (size_t)qrow * q_row_stride + c) = *(const uint4*)(os + r * OROW + c);
      }
    }
  }
}

__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(FWD_OCC, FWD_OCC))) void sinkattn_fwd_bf16_d64(FwdArgs a) {
  fwd_body<2, 1, QB64>(a);
}
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(FWD_OCC_K32, FWD_OCC_K32))) void sinkattn_fwd_bf16_d64_k32(FwdArgs a) {
  fwd_body<1, 1, 1>(a);
}
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(FWD_OCC_K32, FWD_OCC_K32))) void sinkattn_fwd_bf16_d64_k32h(FwdArgs a) {
  fwd_body<1, 4, 1>(a);
}

}  // namespace

// Key-tile width of the forward and dQ kernels for a window w (already
// clamped to the sequence length): 32 keys when w < 1024, else 64.
int fwd_key_tile(int window) { return window < 1024 ? 32 : 64; }

// Host-side launcher (called from the C ABI after validation).
hipError_t launch_fwd_bf16_d64(const bf16* q, const bf16* k, const bf16* v, const float* sinks,
                               bf16* o, float* lse, const int* cu_seqlens, int batch, int seqlen,
                               int total_tokens, int heads_q, int heads_kv, int window,
                               int prefix, float scale, hipStream_t stream) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.sinks = sinks; a.o = o; a.lse = lse;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch; a.seqlen = seqlen; a.heads_q = heads_q; a.heads_kv = heads_kv;
  a.group = heads_q / heads_kv;
  a.window = window; a.prefix = prefix;
  a.lse_head_stride = cu_seqlens ? total_tokens : seqlen;
  a.scale_log2 = scale * SA_LOG2E;
  if (seqlen == 0 || batch == 0 || heads_q == 0) return hipSuccess;
  // short windows with GQA groups of a multiple of 4: four heads per workgroup
  const bool heads4 = fwd_key_tile(window) == 32 && a.group % 4 == 0;
  const bool k32 = fwd_key_tile(window) == 32;
  const int rows = heads4 ? 32 : (k32 ? WAVES * 32 : WAVES * QB64 * 32);
  a.num_q_tiles = (seqlen + rows - 1) / rows;
  // packed sequences: one linear index over every sequence's tiles
  const int tiles = cu_seqlens ? sa_packed_tiles_bound(batch, seqlen, total_tokens, rows)
                               : a.num_q_tiles;
  if (tiles > 65535) return hipErrorInvalidConfiguration;
  if (tiles == 0) return hipSuccess;
  dim3 grid(heads4 ? heads_q / 4 : heads_q, cu_seqlens ? 1 : batch, tiles);
  if (heads4)
    hipLaunchKernelGGL(sinkattn_fwd_bf16_d64_k32h, grid, dim3(WAVES * 64), 0, stream, a);
  else if (k32)
    hipLaunchKernelGGL(sinkattn_fwd_bf16_d64_k32, grid, dim3(WAVES * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(sinkattn_fwd_bf16_d64, grid, dim3(WAVES * 64), 0, stream, a);
  return hipGetLastError();
}
