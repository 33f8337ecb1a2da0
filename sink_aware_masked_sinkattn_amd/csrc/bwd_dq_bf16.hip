// dQ of sink-aware masked attention, bf16, head dim 64, gfx950 MFMA.
//
// For each query row i of head h, over the keys the mask leaves visible
// (M[q,k] = 1[k<=q] AND 1[q-k<=w OR k<p]; "Efficient Reinforcement Learning
// for Long-Horizon Tool-Use Agentic Tasks", summary page):
//   P'_ij = exp(S_ij - L_i),  S_ij = scale q_i . k_j,  L_i = logaddexp(l_i, s_h)
//   dS_ij = P'_ij (dO_i . v_j - D_i),    dQ_i = scale sum_j dS_ij k_j
// (the zero-value sink key of arXiv 2608.10357 section 5 enters only through
// L and D).  Query-stationary, like the forward: each workgroup owns the
// query rows of its waves (4 waves x QB blocks of 32 rows: 64 rows per wave
// with 64-key tiles, 32 rows with the 32-key tiles of short windows) of one
// head and walks the same key-tile list (prefix tiles + window tiles), so dQ
// accumulates in registers and is written once, with no atomics -- at the
// price of recomputing S and dP^T here (the dK/dV kernel recomputes them too).
//
// Layout per wave (QB 32-row MFMA blocks):
//   S^T = K Q^T and dP^T = V dO^T with one query per lane (C layout); Q and
//   dO fragments stay in registers as the B operand; K and V tiles come
//   from LDS as the A operand.  L and D are then per-lane scalars.  The C
//   layout of dS^T (lane = query, 16 keys in registers) is exactly the B
//   operand of dQ^T = K^T dS^T; the A operand (keys along k) is a transpose
//   read of the row-major K tile.  dQ^T's C layout gives each lane runs of 4
//   consecutive head dims of its query, stored 8 bytes at a time.
//
// Short windows with GQA groups of a multiple of 4 run a variant that keeps
// a 32-row block's key tiles resident in LDS for all the group's heads
// (sinkattn_bwd_dq_bf16_d64_win, below), which for 0 < p <= 16 also computes
// the prefix keys' dK/dV part of its rows past the fold row (the prefix
// fold).  Every kernel here also writes the backward's row statistics (D, L)
// for the dK/dV kernel and its parts of the sink gradient ds_h into
// per-workgroup slots (no atomics; the finish kernel adds them in a fixed
// order), and clears its rows of the fp32 dK/dV accumulators when the dK/dV
// launch adds into them.
#include "common.h"
#include "mask_tiles.h"

namespace {

constexpr int D = 64;
constexpr int QB64 = 2;      // 32-row query blocks per wave, 64-key-tile instance
constexpr int QB32 = 1;      // the same for the 32-key-tile (short window) instance
constexpr int WAVES = 4;     // waves per workgroup
constexpr int OROW = D + 8;            // padded row of the epilogue staging buffer
// Key tiles of NKB blocks of 32 keys (64 in general, 32 for short windows).
// LDS: two K/V tile pairs during the key loop; afterwards the same memory
// stages each wave's output rows (padded) for row-contiguous stores.
template <int NKB, int QB>
struct DqTiles {
  static constexpr int BQ = WAVES * QB * 32;   // query rows per workgroup
  static constexpr int STAGE_ELEMS = WAVES * QB * 32 * OROW;
  static constexpr int BK = 32 * NKB;
  static constexpr int TILE_ELEMS = BK * D;   // swizzled rows (tile_off)
  static constexpr int SMEM_ELEMS = (4 * TILE_ELEMS > STAGE_ELEMS) ? 4 * TILE_ELEMS : STAGE_ELEMS;
  static_assert(SMEM_ELEMS >= 4 * TILE_ELEMS && SMEM_ELEMS >= STAGE_ELEMS, "LDS sizing");
};

struct DqArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const bf16* o;
  const float* lse;       // forward log-sum-exp (natural log, content keys only)
  const float* sinks;
  float* ds_part;         // [Hq, ds_stride] this launch's per-workgroup parts of ds_h:
                          // slot grid_y_index * grid_z + grid_z_index of each head
                          // (the finish kernel adds a head's slots in index order)
  int ds_stride;
  float* l2_ws;           // [Hq, rows] L in log2 units (L * log2 e), written here
  float* d_ws;            // [Hq, rows] D, written here
  float* dk_acc;          // [rows, Hkv, D] fp32 dK / dV accumulators, zeroed here when
  float* dv_acc;          // clear_acc (the dK/dV kernel adds into them)
  int clear_acc;          // 0: the dK/dV kernel stores every key's row (one work unit per block)
  bf16* dq;
  const int* cu_seqlens;
  int batch, seqlen, heads_q, heads_kv, group, window, prefix, rows_total;
  int num_q_tiles;        // fixed length: query tiles per sequence
  int lse_head_stride;    // T (fixed length) or N (packed)
  // prefix fold (window kernel): rows at or past fold_row add the prefix keys'
  // dK/dV part of their block into fold_part[(kv head * ds_stride + slot) *
  // 2 * prefix * D]: dK (unscaled) then dV, prefix keys x head dims
  int fold;
  long long fold_row;
  float* fold_part;
  float scale_log2;
  float scale;
};

__device__ __forceinline__ int map_head(int x, int heads_q) {
  if ((heads_q & 7) == 0) return (x & 7) * (heads_q >> 3) + (x >> 3);
  return x;
}

// One key tile (NKB blocks of 32 keys) against this wave's QB blocks of 32
// query rows.  MF: the mask -- 0 none (full tiles), SA_MASK_GENERAL the
// element predicate, SA_MASK_UPPER / SA_MASK_LOWER the one-sided forms of
// mask_form with the per-lane threshold thr (32-key tiles, one row block).
//
// Issue order, per (key block, query block): S^T chain; dP^T chain with a
// quarter of the P' work after each MFMA; the first half of dS, then its two
// dQ MFMAs with the second half of dS behind them, then the last two.  A wave
// so overlaps most of its own VALU work with its MFMAs instead of leaving
// that to the other waves of its SIMD.  The next key block's operands are
// read behind the last query block's MFMAs.  sched_barrier fences hold each
// part in place.
template <int NKB, int QB, int MF>
__device__ __forceinline__ void tile_step(uint32_t ktile, const bf16x8 (&qf)[QB][4],
                                          const bf16x8 (&df)[QB][4], const float (&l2)[QB],
                                          const float (&dd)[QB], f32x16 (&acc)[QB][2], int qw0,
                                          int k0, int window, int prefix, float scale_log2,
                                          int lane, int thr = 0) {
  static_assert(MF == 0 || MF == SA_MASK_GENERAL || (NKB == 1 && QB == 1),
                "one-sided masks: 32-key tiles, one row block");
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int grp = lane >> 4;
  const int li = lane & 15;
  // LDS: the K tile at byte address ktile, the V tile right after it.  One
  // base register per read pattern (row reads, transpose reads), recomputed
  // per tile rather than kept live across the loop.
  constexpr int VOFF = NKB * 32 * 128;
  const uint32_t ra = (uint32_t)sa_opaque((int)ktile + tile_row_base(l32, g));
  const uint32_t ta =
      (uint32_t)sa_opaque((int)ktile + tile_tr_base(4 * g + (li >> 2), 16 * (grp & 1) + 4 * (li & 3)));
  // A operands of S^T = K Q^T and dP^T = V dO^T (keys on m, head dim on k)
  bf16x8 kf[4], vf[4];
  auto read_kv = [&](int kb) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kf[s] = lds_read8((ra ^ (32 * s)) + kb * 4096);
      vf[s] = lds_read8((ra ^ (32 * s)) + kb * 4096 + VOFF);
    }
  };
  // A operand of dQ^T += K^T dS^T (head dim on m, keys on k): transpose reads of
  // rows kb*32 + 16*hh + 4g + li/4 (+8), columns db*32 + 16*(grp&1) + 4*(li&3)
  bf16x8 kt[2][2];   // [hh][db]
  auto read_kt = [&](int kb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int o = kb * 4096 + hh * 2048;   // folds into the immediate offset
        kt[hh][db] = cat8(lds_read_tr4_at((ta ^ (64 * db)) + o),
                          lds_read_tr4_at((ta ^ (64 * db + 32)) + o + 1024));
      }
  };
  read_kv(0);
  read_kt(0);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    // dS^T: lane = query, rows = keys kr + 8*(i/4) + i%4, kr = k0 + kb*32 + 4g
    const int kr = k0 + kb * 32 + 4 * g;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const bool next_kb = (qb == QB - 1) && (kb + 1 < NKB);
      const int base = sa_opaque(qw0 + qb * 32 + l32 - kr);
      const int pb = prefix - kr;
      __builtin_amdgcn_sched_barrier(0);
      f32x16 st = f32x16{};
#pragma unroll
      for (int j = 0; j < 4; ++j) st = mfma32x32x16(kf[j], qf[qb][j], st);
      __builtin_amdgcn_sched_barrier(0);
      // P' = exp2(S*scale*log2e - L*log2e) (0 where hidden), a quarter after
      // each dP^T MFMA
      f32x16 dpt = f32x16{};
      float pp[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dpt = mfma32x32x16(vf[j], df[qb][j], dpt);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          float p = fast_exp2(fmaf(st[i], scale_log2, -l2[qb]));
          if (MF == SA_MASK_GENERAL) {
            const int c = 8 * j + e;
            p = sa_vis(base - c, c < pb ? SA_LIM_PREFIX : window) ? p : 0.0f;
          } else if (MF == SA_MASK_UPPER) {
            p = 8 * j + e <= thr ? p : 0.0f;
          } else if (MF == SA_MASK_LOWER) {
            p = 8 * j + e >= thr ? p : 0.0f;
          }
          pp[i] = sa_pin(p);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (next_kb) read_kv(kb + 1);   // this block's K and V operands are dead
      // dS = P' (dP - D); dQ^T += K^T dS^T, one half of dS at a time (dS^T in
      // the C layout of S^T is already the B operand: keys on k, query on n)
      bf16x8 dsb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) dsv[e] = pp[8 * hh + e] * (dpt[8 * hh + e] - dd[qb]);
        dsb[hh] = to_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < 2; ++db) acc[qb][db] = mfma32x32x16(kt[hh][db], dsb[hh], acc[qb][db]);
      }
      if (next_kb) read_kt(kb + 1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// A partial 32-key tile of one 32-row block in the cheapest exact form of
// its mask (mask_form).
__device__ __forceinline__ void partial_step(uint32_t ktile, const bf16x8 (&qf)[1][4],
                                             const bf16x8 (&df)[1][4], const float (&l2)[1],
                                             const float (&dd)[1], f32x16 (&acc)[1][2], int qw0,
                                             int k0, int window, int prefix, float scale_log2,
                                             int lane) {
  int thr;
  const int form = mask_form(qw0, k0, lane, window, prefix, &thr);
  thr = sa_opaque(thr);
  if (form == SA_MASK_UPPER)
    tile_step<1, 1, SA_MASK_UPPER>(ktile, qf, df, l2, dd, acc, qw0, k0, window, prefix, scale_log2,
                                   lane, thr);
  else if (form == SA_MASK_LOWER)
    tile_step<1, 1, SA_MASK_LOWER>(ktile, qf, df, l2, dd, acc, qw0, k0, window, prefix, scale_log2,
                                   lane, thr);
  else
    tile_step<1, 1, SA_MASK_GENERAL>(ktile, qf, df, l2, dd, acc, qw0, k0, window, prefix,
                                     scale_log2, lane);
}

// The backward's row statistics for one query row, from this lane's half
// of its dO and O (head dims 16s + 8g .. +7) and its forward l:
//   D = rowsum(dO * O),  L = logaddexp(l, s_h)  (log2 units: L * log2 e),
//   and the row's term of ds_h, -exp(s_h - L) D (counted by the g == 0 half).
// bf16 products are exact in fp32, so v_dot2_f32_bf16 changes only the
// rounding order of D.  Rows past the end (ok false) get L = +inf and D = 0.
__device__ __forceinline__ void row_stats(const bf16x8 (&o)[4], const bf16x8 (&dout)[4], float l,
                                          float sink, bool ok, int g, float& l2, float& dd,
                                          float& ds) {
  float dot = 0.0f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 8; j += 2)
      dot = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{o[s][j], o[s][j + 1]},
                                            bf16x2{dout[s][j], dout[s][j + 1]}, dot, false);
  dot = halves_sum(dot);
  // L2 = log2(2^l2 + 2^s2) = max + log2(1 + 2^-|l2 - s2|)
  const float lv2 = l * SA_LOG2E;
  const float sink2 = sink * SA_LOG2E;
  const float big_l2 = (sink == -INFINITY)
                           ? lv2
                           : fmaxf(lv2, sink2) + fast_log2(1.0f + fast_exp2(-fabsf(lv2 - sink2)));
  l2 = ok ? big_l2 : INFINITY;
  dd = ok ? dot : 0.0f;
  ds = (ok && g == 0) ? -fast_exp2(sink2 - big_l2) * dot : 0.0f;
}

constexpr int DQ_OCC = 2;   // waves per SIMD the register budget is set for
template <int NKB, int QB>
__device__ __forceinline__ void dq_body(const DqArgs& a) {
  using T = DqTiles<NKB, QB>;
  constexpr int BQ = T::BQ;
  constexpr int BK = T::BK;
  constexpr int TILE_ELEMS = T::TILE_ELEMS;
  __shared__ __attribute__((aligned(128))) bf16 smem[T::SMEM_ELEMS];   // K0 V0 K1 V1, then output staging

  const int h = map_head(blockIdx.x, a.heads_q);
  const size_t ds_slot =
      (size_t)h * a.ds_stride + (size_t)blockIdx.y * gridDim.z + blockIdx.z;
  int z = 0, qt = 0;
  const bool has_tile = launch_tile(a.cu_seqlens, a.batch, a.num_q_tiles, BQ, &z, &qt);
  const SeqView sv = seq_view(a.cu_seqlens, has_tile ? z : 0, a.seqlen, a.heads_q);
  const int q_start = qt * BQ;
  if (!has_tile || q_start >= sv.len) {   // no rows here: this workgroup's part of ds_h is 0
    if (threadIdx.x == 0) a.ds_part[ds_slot] = 0.0f;
    return;
  }
  const int q_last = min(q_start + BQ - 1, sv.len - 1);
  const int kvh = h / a.group;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int qw0 = q_start + wave * (QB * 32);
  const bool wave_active = qw0 < sv.len;
  const int qw1 = min(qw0 + QB * 32 - 1, sv.len - 1);

  const int q_row_stride = a.heads_q * D;
  const int kv_row_stride = a.heads_kv * D;
  const size_t qoff = (size_t)sv.row_base * q_row_stride + (size_t)h * D;
  const bf16* kbase = a.k + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;
  const bf16* vbase = a.v + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;

  int seg[4];
  const int nseg = sa_key_tile_segments(q_start, q_last, a.window, a.prefix, BK, seg);
  const int n0 = seg[1] - seg[0];
  const int ntiles = n0 + (nseg > 1 ? seg[3] - seg[2] : 0);

  // K / V tiles go straight from global memory into swizzled LDS tiles (the
  // lane constants are recomputed per call: a few VALU instructions instead
  // of registers held across the whole key loop)
  auto load_tile = [&](int t, int buf) {
    const int kt = t < n0 ? seg[0] + t : seg[2] + (t - n0);
    const int r0 = kt * BK;
    const TileLane tl = tile_lane(sa_opaque(lane), kv_row_stride * 2);
    tile_load_lds_lane<BK, WAVES>(smem + (2 * buf) * TILE_ELEMS, kbase + (size_t)r0 * kv_row_stride,
                                  kv_row_stride * 2, sv.len - r0, wave, tl);
    tile_load_lds_lane<BK, WAVES>(smem + (2 * buf + 1) * TILE_ELEMS, vbase + (size_t)r0 * kv_row_stride,
                                  kv_row_stride * 2, sv.len - r0, wave, tl);
  };

  // the first K/V tile load goes out before the row loads below
  load_tile(0, 0);

  // Q, dO fragments (B operands) and the row statistics of the backward for
  // this wave's rows -- the sink gradient of "GPT-OSS Agentic RL training: a
  // practical retrospective" (FlashAttention v3 implementation section),
  // with the sink as a zero-value key (arXiv 2608.10357, section 5):
  //   D = rowsum(dO * O),  L = logaddexp(l, s_h),  ds_h -= exp(s_h - L) D.
  // O is read in the layout of the dO fragment (this lane: half of the row's
  // head dim), so D is a register dot product plus one half-wave swap.  D and
  // L (log2 units) go to the workspace for the dK/dV kernel, which runs after
  // this one; those stores wait for the epilogue, so that the loads here
  // overlap with the first K/V tile load.
  bf16x8 qf[QB][4], df[QB][4];
  float l2[QB], dd[QB];
  const float sink = a.sinks[h];
  float ds_part = 0.0f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + l32;
    const bool ok = row < sv.len;
    bf16x8 of[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const size_t off = qoff + (size_t)row * q_row_stride + 16 * s + 8 * g;
      qf[qb][s] = ok ? *(const bf16x8*)(a.q + off) : bf16x8{};
      df[qb][s] = ok ? *(const bf16x8*)(a.dout + off) : bf16x8{};
      of[s] = ok ? *(const bf16x8*)(a.o + off) : bf16x8{};
    }
    const float l = ok ? a.lse[sv.lse_base + (size_t)h * a.lse_head_stride + row] : 0.0f;
    float ds;
    row_stats(of, df[qb], l, sink, ok, g, l2[qb], dd[qb], ds);
    ds_part += ds;
  }

  f32x16 acc[QB][2];   // dQ^T: C layout [m = d][n = query], lane = query
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) acc[qb][0] = acc[qb][1] = f32x16{};

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
      tile_step<NKB, QB, 0>(ktile, qf, df, l2, dd, acc, qw0, k0, a.window, a.prefix, a.scale_log2, lane);
    } else if (cls == SA_TILE_PARTIAL) {
      if constexpr (NKB == 1 && QB == 1) {
        partial_step(ktile, qf, df, l2, dd, acc, qw0, k0, a.window, a.prefix, a.scale_log2, lane);
      } else {
        tile_step<NKB, QB, SA_MASK_GENERAL>(ktile, qf, df, l2, dd, acc, qw0, k0, a.window, a.prefix,
                                            a.scale_log2, lane);
      }
    }
    wait_all_mem();
    __syncthreads();
  }

  // ---- dQ = scale * acc.  acc holds dQ^T: C layout rows = head dims
  // db*32 + 8*(i/4) + 4g + i%4, column = query qb*32 + l32, so each lane
  // holds runs of 4 consecutive head dims of its query.  Stage through LDS
  // for row-contiguous stores.
  bf16* os = smem + wave * (QB * 32) * OROW;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * g;
        *(bf16x4*)(os + (qb * 32 + l32) * OROW + d) =
            to_bf16x4(acc[qb][db][4 * i4] * a.scale, acc[qb][db][4 * i4 + 1] * a.scale,
                      acc[qb][db][4 * i4 + 2] * a.scale, acc[qb][db][4 * i4 + 3] * a.scale);
      }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  if (wave_active) {
    bf16* obase = a.dq + qoff;
#pragma unroll
    for (int it = 0; it < (QB * 32 * D) / (64 * 8); ++it) {
      const int chunk = it * 64 + lane;
      const int r = chunk >> 3;
      const int c = (chunk & 7) * 8;
      const int qrow = qw0 + r;
      if (qrow < sv.len) *(uint4*)(obase + (size_t)qrow * q_row_stride + c) = *(const uint4*)(os + r * OROW + c);
    }
  }
  // row statistics for the dK/dV kernel, and this wave's share of ds_h
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + l32;
    if (row < sv.len && g == 0) {
      const size_t wi = (size_t)h * a.rows_total + sv.row_base + row;
      a.d_ws[wi] = dd[qb];
      a.l2_ws[wi] = l2[qb];
    }
  }
  // this workgroup's part of ds_h: its waves' sums in wave order, into its
  // slot (no atomics: the finish kernel adds the slots in a fixed order)
  __shared__ float ds_red[WAVES];
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) ds_part += __shfl_xor(ds_part, w);
  if (lane == 0) ds_red[wave] = wave_active ? ds_part : 0.0f;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += ds_red[w];
    a.ds_part[ds_slot] = t;
  }
  // Zero this workgroup's share of the fp32 dK / dV accumulators (the dK/dV
  // kernel adds into them): rows of the tile congruent to h mod group, so the
  // group's query heads split the kv head's rows between them.
  if (a.clear_acc) {
    const int part = h - kvh * a.group;
    const int n_mine = (q_last - q_start + a.group - part) / a.group;   // rows part, part+group, ...
    for (int i = tid; i < n_mine * (D / 4); i += WAVES * 64) {
      const int r = q_start + part + a.group * (i / (D / 4));
      const size_t e = ((size_t)(sv.row_base + r) * a.heads_kv + kvh) * D + 4 * (i % (D / 4));
      *(float4*)(a.dk_acc + e) = make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)(a.dv_acc + e) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(DQ_OCC, DQ_OCC))) void sinkattn_bwd_dq_bf16_d64(DqArgs a) {
  dq_body<2, QB64>(a);
}
// short windows: 32-key tiles and (by default) 32 rows per wave at 3 waves
// per SIMD -- a 64-row wave would span w + 64 keys of which fewer are visible
constexpr int DQ_OCC_K32 = 3;
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(DQ_OCC_K32, DQ_OCC_K32))) void sinkattn_bwd_dq_bf16_d64_k32(DqArgs a) {
  dq_body<1, QB32>(a);
}

// ---------------------------------------------------------------------------
// Short windows with GQA groups of a multiple of 4: one workgroup per
// (32-row query block, kv head).  The block's key tiles (prefix and window,
// at most WIN_TILES tiles of 32 keys) are copied into LDS once and stay
// resident; the four waves then take the group's query heads in turn (wave
// w: heads w, w + 4, ...), each running the whole key-tile list from LDS
// with no further copies, waits or barriers.  The K/V tiles are so loaded
// once for all the group's heads, not once per head, and the tile loop has
// no per-tile latency.  Same arithmetic per tile as the streaming kernels.
constexpr int WIN_TILES = 6;
struct __attribute__((aligned(128))) DqWinSmem {
  bf16 kv[WIN_TILES][2][32 * D];    // K then V of each tile (swizzled rows, tile_off)
  bf16 stage[WAVES][32 * OROW];     // each wave's dQ rows, for row-contiguous stores
};

// The prefix fold: the prefix keys' (keys 0 .. p-1, p <= 16, all in the
// resident tile 0) part of dK and dV from this block's rows, when they lie at
// or past the fold row -- rows that see no other key of the dK/dV kernel's
// first key block, whose work stops before them; they see exactly the keys
// k < p.  Each wave takes its heads two at a time, with the heads' Q and dO
// rows copied into the block's LDS (the key tiles are no longer needed once
// the K, V operands of keys 0..15 are in registers) and their L and -D read
// back from the workspace this wave wrote them to, and runs for each head a
// 32-row x 16-key step on v_mfma_f32_16x16x32_bf16 (fold_step16).  The four
// waves' sums are added in wave order and the block's part goes to its slot;
// the finish phase adds a sequence's slots in order into the fp32 dK/dV
// accumulators.  Blocks before the fold row write nothing (the finish phase
// reads only the slots past it).
//
// LDS during the fold (the whole DqWinSmem, 66 KB): wave w's two Q / dO
// tiles at 16 KB * w (+ 8 KB for the second head; dO 4 KB after its Q),
// the heads' L and -D rows in the last 2 KB.
constexpr int FOLD_WAVE_BYTES = 2 * 2 * 32 * D * 2;
constexpr int FOLD_STAT_OFF = WAVES * FOLD_WAVE_BYTES;
constexpr int FOLD_KEYS = 16;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One head's part of the prefix keys' dK (unscaled dS^T Q) and dV (P'^T dO)
// from the block's 32 rows, keys 0..15, on the 16x16x32 MFMA (lane l: G =
// l/16, i = l%16; A: row i, k 8G..8G+7; B: column i, k 8G..8G+7; C: column i,
// rows 4G..4G+3):
//   S = Q K^T and dP = dO V^T, per 16-row half h: rows on m, keys on n, the
//     head dim on k (two k-steps of 32); dP starts from -D of its rows;
//   P' = exp2(S scale log2 e - L) for keys < p (0 otherwise), dS = P' (dP - D);
//   dV += P'^T dO and dK += dS^T Q with keys on m, d on n (four blocks of 16)
//     and the rows on k in the order 4G..4G+3, 16+4G..16+4G+3: P' and dS in
//     the C layout of S are then already the A operand, and the B operand
//     (dO, Q) is two transpose reads of four rows each.
// kb16 / vb16: B operands of S / dP (K and V rows of keys 0..15, k-step ks).
__device__ __forceinline__ void fold_step16(uint32_t qtile, uint32_t dtile, const float* l2s,
                                            const float* dds, const bf16x8 (&kb16)[2],
                                            const bf16x8 (&vb16)[2], f32x4 (&dk)[4],
                                            f32x4 (&dv)[4], int prefix, float scale_log2,
                                            int lane) {
  const int G = lane >> 4, i16 = lane & 15;
  f32x4 pq[2], dq4[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * h + i16;   // A row of this lane
    f32x4 sacc = f32x4{};
    f32x4 dacc = *(const f32x4*)(dds + 16 * h + 4 * G);   // -D of rows 16h + 4G + j
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c8 = 4 * ks + G;   // 16-byte chunk of the head dim
      const bf16x8 qa = lds_read8(qtile + (uint32_t)(r * 128 + ((c8 ^ tile_swz(r)) << 4)));
      const bf16x8 da = lds_read8(dtile + (uint32_t)(r * 128 + ((c8 ^ tile_swz(r)) << 4)));
      sacc = mfma16(qa, kb16[ks], sacc);
      dacc = mfma16(da, vb16[ks], dacc);
    }
    const f32x4 l4 = *(const f32x4*)(l2s + 16 * h + 4 * G);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float p = fast_exp2(fmaf(sacc[j], scale_log2, -l4[j]));
      p = i16 < prefix ? p : 0.0f;   // key i16 (rows past the fold see only k < p)
      pq[h][j] = p;
      dq4[h][j] = p * dacc[j];
    }
  }
  const bf16x8 pa = to_bf16x8(pq[0][0], pq[0][1], pq[0][2], pq[0][3], pq[1][0], pq[1][1], pq[1][2],
                              pq[1][3]);
  const bf16x8 sa = to_bf16x8(dq4[0][0], dq4[0][1], dq4[0][2], dq4[0][3], dq4[1][0], dq4[1][1],
                              dq4[1][2], dq4[1][3]);
  // B: rows 4G..4G+3 then 16+4G..16+4G+3 of column 16 nb + i16: lane L of the
  // 16-lane group points at row r0 + L/4, column c0 + 4 (L%4)
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    bf16x4 lo[2], hi[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int rr = 16 * half + 4 * G + (i16 >> 2);
      const int cc = 16 * nb + 4 * (i16 & 3);
      const uint32_t off = (uint32_t)(2 * tile_off(rr, cc));
      lo[half] = lds_read_tr4_at(dtile + off);
      hi[half] = lds_read_tr4_at(qtile + off);
    }
    dv[nb] = mfma16(pa, cat8(lo[0], lo[1]), dv[nb]);
    dk[nb] = mfma16(sa, cat8(hi[0], hi[1]), dk[nb]);
  }
}

__device__ __forceinline__ void prefix_fold(const DqArgs& a, DqWinSmem& sm, const SeqView& sv,
                                            int kvh, size_t slot, int q_start, int wave,
                                            int lane) {
  static_assert(FOLD_STAT_OFF + WAVES * 2 * 2 * 32 * (int)sizeof(float) <= (int)sizeof(DqWinSmem),
                "the fold's tiles and row statistics fit in the window kernel's LDS");
  static_assert(WAVES * 2 * FOLD_KEYS * D * (int)sizeof(float) <= FOLD_STAT_OFF,
                "the waves' sums fit in their tile areas");
  const int np = a.prefix;   // 1 .. FOLD_KEYS
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int G = lane >> 4, i16 = lane & 15;
  // B operands of S and dP: K and V rows of keys 0..15 (column i16), head dim
  // 32 ks + 8G .. +7
  bf16x8 kb16[2], vb16[2];
  {
    const uint32_t kt = lds_addr(sm.kv[0][0]), vt = lds_addr(sm.kv[0][1]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c8 = 4 * ks + G;
      const uint32_t off = (uint32_t)(i16 * 128 + ((c8 ^ tile_swz(i16)) << 4));
      kb16[ks] = lds_read8(kt + off);
      vb16[ks] = lds_read8(vt + off);
    }
  }
  wait_all_mem();
  __syncthreads();   // every wave is done with the key tiles and its staging rows
  f32x4 pdk[4], pdv[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) pdk[nb] = pdv[nb] = f32x4{};
  char* lds = (char*)&sm;
  bf16* qt0 = (bf16*)(lds + wave * FOLD_WAVE_BYTES);   // Q, then dO 32 * D after
  float* st0 = (float*)(lds + FOLD_STAT_OFF) + wave * 2 * 64;   // per head: L[32], -D[32]
  const int q_row_stride = a.heads_q * D;
  const TileLane tl = tile_lane(lane, q_row_stride * 2);
  const int n_valid = sv.len - q_start;
  for (int hi = wave; hi < a.group; hi += 2 * WAVES) {
    const int nh = hi + WAVES < a.group ? 2 : 1;
    for (int j = 0; j < nh; ++j) {
      const int h = kvh * a.group + hi + j * WAVES;
      const size_t off = ((size_t)sv.row_base + q_start) * q_row_stride + (size_t)h * D;
      bf16* qt = qt0 + j * 2 * 32 * D;
      tile_load_lds_lane<32, 1>(qt, a.q + off, q_row_stride * 2, n_valid, 0, tl);
      tile_load_lds_lane<32, 1>(qt + 32 * D, a.dout + off, q_row_stride * 2, n_valid, 0, tl);
    }
    // lanes 0..31: the first head's rows, 32..63: the second's
    {
      const int h = kvh * a.group + hi + g * WAVES;
      const bool ok = g < nh && q_start + l32 < sv.len;
      const size_t wi = (size_t)h * a.rows_total + sv.row_base + q_start + l32;
      const float l2v = ok ? a.l2_ws[wi] : INFINITY;
      const float ddv = ok ? -a.d_ws[wi] : 0.0f;
      st0[g * 64 + l32] = l2v;
      st0[g * 64 + 32 + l32] = ddv;
    }
    wait_all_mem();
    __builtin_amdgcn_wave_barrier();
    for (int j = 0; j < nh; ++j) {
      const uint32_t qt = lds_addr(qt0 + j * 2 * 32 * D);
      fold_step16(qt, qt + 32 * D * 2, st0 + j * 64, st0 + j * 64 + 32, kb16, vb16, pdk, pdv,
                  np, a.scale_log2, lane);
    }
    wait_all_mem();   // the tiles' reads are done before the next round's copies
    __builtin_amdgcn_wave_barrier();
  }
  // each wave's sums of keys < p into its own tile area ([dK | dV][key][d]),
  // then all threads add the four in wave order.  C layout: key 4G + j,
  // head dim 16 nb + i16.
  float* mine = (float*)qt0;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 4 * G + j;
      if (key < np) {
        mine[key * D + 16 * nb + i16] = pdk[nb][j];
        mine[(np + key) * D + 16 * nb + i16] = pdv[nb][j];
      }
    }
  __syncthreads();
  float* out = a.fold_part + ((size_t)kvh * a.ds_stride + slot) * (2 * np * D);
  for (int i = threadIdx.x; i < 2 * np * D; i += WAVES * 64) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += ((const float*)(lds + w * FOLD_WAVE_BYTES))[i];
    out[i] = t;
  }
}

__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sinkattn_bwd_dq_bf16_d64_win(DqArgs a) {
  __shared__ DqWinSmem sm;
  // consecutive workgroups go to consecutive XCDs: with 8 kv heads each XCD
  // keeps one kv head and its L2
  const int kvh = blockIdx.x;
  const size_t ds_slot = (size_t)blockIdx.y * gridDim.z + blockIdx.z;   // + h * ds_stride
  int z = 0, qt = 0;
  const bool has_tile = launch_tile(a.cu_seqlens, a.batch, a.num_q_tiles, 32, &z, &qt);
  const SeqView sv = seq_view(a.cu_seqlens, has_tile ? z : 0, a.seqlen, a.heads_q);
  const int q_start = qt * 32;
  if (!has_tile || q_start >= sv.len) {   // no rows here: the group's parts of ds_h are 0
    for (int i = threadIdx.x; i < a.group; i += WAVES * 64)
      a.ds_part[(size_t)(kvh * a.group + i) * a.ds_stride + ds_slot] = 0.0f;
    return;
  }
  const int q_last = min(q_start + 31, sv.len - 1);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int q_row_stride = a.heads_q * D;
  const int kv_row_stride = a.heads_kv * D;
  const bf16* kbase = a.k + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;
  const bf16* vbase = a.v + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;

  // the block's key tiles, all copied up front (ntiles <= WIN_TILES: the
  // host launches this kernel only when every block's list fits)
  int seg[4];
  const int nseg = sa_key_tile_segments(q_start, q_last, a.window, a.prefix, 32, seg);
  const int n0 = seg[1] - seg[0];
  const int ntiles = n0 + (nseg > 1 ? seg[3] - seg[2] : 0);
  const TileLane tl = tile_lane(lane, kv_row_stride * 2);
  for (int t = 0; t < ntiles; ++t) {
    const int r0 = (t < n0 ? seg[0] + t : seg[2] + (t - n0)) * 32;
    tile_load_lds_lane<32, WAVES>(sm.kv[t][0], kbase + (size_t)r0 * kv_row_stride,
                                  kv_row_stride * 2, sv.len - r0, wave, tl);
    tile_load_lds_lane<32, WAVES>(sm.kv[t][1], vbase + (size_t)r0 * kv_row_stride,
                                  kv_row_stride * 2, sv.len - r0, wave, tl);
  }
  wait_all_mem();
  __syncthreads();

  const int row = q_start + l32;
  const bool ok = row < sv.len;
  // a head's rows (Q, dO, O fragments, l): loaded one head ahead, so their
  // latency overlaps the previous head's tile loop
  struct HeadRows {
    bf16x8 q[4], d[4], o[4];
    float l;
  };
  // rows past the end read the last row (no branches around the loads, so
  // the compiler can count them); they get L = +inf below, so P' = dS = 0
  // there and their dQ is not stored
  const int row_c = ok ? row : sv.len - 1;
  auto load_rows = [&](int h, HeadRows& hr) {
    const size_t qoff = (size_t)sv.row_base * q_row_stride + (size_t)h * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const size_t off = qoff + (size_t)row_c * q_row_stride + 16 * s + 8 * g;
      hr.q[s] = *(const bf16x8*)(a.q + off);
      hr.d[s] = *(const bf16x8*)(a.dout + off);
      hr.o[s] = *(const bf16x8*)(a.o + off);
    }
    hr.l = a.lse[sv.lse_base + (size_t)h * a.lse_head_stride + row_c];
  };
  HeadRows nxt;
  if (wave < a.group) load_rows(kvh * a.group + wave, nxt);
  for (int hi = wave; hi < a.group; hi += WAVES) {
    const int h = kvh * a.group + hi;
    const size_t qoff = (size_t)sv.row_base * q_row_stride + (size_t)h * D;
    const HeadRows cur = nxt;
    // Q, dO fragments (B operands) and the row statistics
    bf16x8 qf[1][4], df[1][4];
    float l2[1], dd[1], ds_part;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[0][s] = cur.q[s];
      df[0][s] = cur.d[s];
    }
    row_stats(cur.o, cur.d, cur.l, a.sinks[h], ok, g, l2[0], dd[0], ds_part);
    // the next head's rows go out now, after this head's have been consumed:
    // the statistics are pinned ahead of the loads, so the one wait for this
    // head's rows comes before them and the loads stay in flight through
    // the tile loop
    asm volatile("" : "+v"(l2[0]), "+v"(dd[0]), "+v"(ds_part));
    __builtin_amdgcn_sched_barrier(0);
    if (hi + WAVES < a.group) load_rows(h + WAVES, nxt);
    __builtin_amdgcn_sched_barrier(0);

    f32x16 acc[1][2];   // dQ^T: C layout [m = d][n = query], lane = query
    acc[0][0] = acc[0][1] = f32x16{};
    for (int t = 0; t < ntiles; ++t) {
      const int k0 = (t < n0 ? seg[0] + t : seg[2] + (t - n0)) * 32;
      const int cls = sa_tile_class(q_start, q_last, k0, k0 + 31, a.window, a.prefix);
      const uint32_t ktile = lds_addr(sm.kv[t][0]);   // V tile follows
      if (cls == SA_TILE_FULL)
        tile_step<1, 1, 0>(ktile, qf, df, l2, dd, acc, q_start, k0, a.window, a.prefix,
                           a.scale_log2, lane);
      else if (cls == SA_TILE_PARTIAL)
        partial_step(ktile, qf, df, l2, dd, acc, q_start, k0, a.window, a.prefix, a.scale_log2,
                     lane);
    }

    // dQ = scale * acc through this wave's staging rows (runs of 4 head dims
    // per lane), then row-contiguous 16-byte stores
    bf16* os = sm.stage[wave];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + 8 * i4 + 4 * g;
        *(bf16x4*)(os + l32 * OROW + d) =
            to_bf16x4(acc[0][db][4 * i4] * a.scale, acc[0][db][4 * i4 + 1] * a.scale,
                      acc[0][db][4 * i4 + 2] * a.scale, acc[0][db][4 * i4 + 3] * a.scale);
      }
    // LDS writes done (lgkmcnt 0; the next head's row loads stay in flight)
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    bf16* obase = a.dq + qoff;
#pragma unroll
    for (int it = 0; it < (32 * D) / (64 * 8); ++it) {   // 64 lanes x 16 B per iteration
      const int chunk = it * 64 + lane;
      const int r = chunk >> 3;
      const int c = (chunk & 7) * 8;
      if (q_start + r < sv.len)
        *(uint4*)(obase + (size_t)(q_start + r) * q_row_stride + c) = *(const uint4*)(os + r * OROW + c);
    }
    // the staging rows are rewritten for the next head only after these reads
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // row statistics for the dK/dV kernel, and this wave's share of ds_h
    if (ok && g == 0) {
      const size_t wi = (size_t)h * a.rows_total + sv.row_base + row;
      a.d_ws[wi] = dd[0];
      a.l2_ws[wi] = l2[0];
    }
    // this head's part of ds_h from this block: one wave per head, its slot
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) ds_part += __shfl_xor(ds_part, w);
    if (lane == 0) a.ds_part[(size_t)h * a.ds_stride + ds_slot] = ds_part;
  }
  // clear the fp32 dK / dV accumulators of the block's rows for this kv head
  // (the dK/dV kernel adds into them)
  if (a.clear_acc) {
    const int nrows = q_last - q_start + 1;
    for (int i = tid; i < nrows * (D / 4); i += WAVES * 64) {
      const int r = q_start + i / (D / 4);
      const size_t e = ((size_t)(sv.row_base + r) * a.heads_kv + kvh) * D + 4 * (i % (D / 4));
      *(float4*)(a.dk_acc + e) = make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)(a.dv_acc + e) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  if (a.fold && q_start >= a.fold_row) prefix_fold(a, sm, sv, kvh, ds_slot, q_start, wave, lane);
}

}  // namespace

int fwd_key_tile(int window);

// Whether the resident-tile window kernel runs: GQA groups of a multiple of
// 4 (four waves take the group's heads) and a key-tile list of at most
// WIN_TILES tiles for every 32-row block.  A block [q0, q0 + 31] (q0 a
// multiple of 32) lists at most ceil(min(p, T) / 32) prefix tiles and
// floor(q1 / 32) - floor(max(0, q0 - w) / 32) + 1 <= ceil(w / 32) + 1
// window tiles.
bool dq_window_kernel(int seqlen, int group, int window, int prefix) {
  if (group % 4 != 0 || fwd_key_tile(window) != 32) return false;
  const long long pre = ((long long)(prefix < seqlen ? prefix : seqlen) + 31) / 32;
  const long long win = ((long long)window + 31) / 32 + 1;
  return pre + win <= WIN_TILES;
}

// Whether the window dQ kernel takes the prefix keys' dK/dV part of the rows
// past the fold row (see prefix_fold): it runs, and every prefix key lies in
// its first resident tile.
bool dq_prefix_fold(int seqlen, int group, int window, int prefix) {
  return dq_window_kernel(seqlen, group, window, prefix) && prefix > 0 && prefix <= FOLD_KEYS;
}

// Rows per query tile of the dQ kernel the launcher picks.
static int dq_query_tile(int seqlen, int group, int window, int prefix) {
  if (dq_window_kernel(seqlen, group, window, prefix)) return 32;
  return fwd_key_tile(window) == 32 ? DqTiles<1, QB32>::BQ : DqTiles<2, QB64>::BQ;
}

// Workgroups per head of the dQ launch (grid y * grid z), which is the number
// of per-workgroup sink-gradient slots per head it writes: sequences x query
// tiles (fixed length), or the packed tiles' bound (varlen).  At most
// batch * ceil(seqlen / 32), the workspace's slots per head.
int dq_launch_tiles(int batch, int seqlen, int total_tokens, bool varlen, int group, int window,
                    int prefix) {
  const int bq = dq_query_tile(seqlen, group, window, prefix);
  if (varlen) return sa_packed_tiles_bound(batch, seqlen, total_tokens, bq);
  return batch * ((seqlen + bq - 1) / bq);
}

hipError_t launch_bwd_dq_bf16_d64(const bf16* q, const bf16* k, const bf16* v, const bf16* dout,
                                  const bf16* o, const float* lse, const float* sinks,
                                  float* ds_part, int ds_stride, float* l_ws, float* d_ws, float* dk_acc,
                                  float* dv_acc, bf16* dq, const int* cu_seqlens, int batch,
                                  int seqlen, int rows_total, int heads_q, int heads_kv, int window,
                                  int prefix, float scale, long long fold_row, float* fold_part,
                                  bool clear_acc, hipStream_t stream) {
  DqArgs a;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.o = o; a.lse = lse; a.sinks = sinks;
  a.ds_part = ds_part; a.ds_stride = ds_stride; a.l2_ws = l_ws; a.d_ws = d_ws; a.dk_acc = dk_acc; a.dv_acc = dv_acc;
  a.dq = dq;
  a.lse_head_stride = cu_seqlens ? rows_total : seqlen;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch; a.seqlen = seqlen; a.heads_q = heads_q; a.heads_kv = heads_kv;
  a.group = heads_q / heads_kv; a.window = window; a.prefix = prefix;
  a.rows_total = rows_total;
  const bool k32 = fwd_key_tile(window) == 32;
  a.scale_log2 = scale * SA_LOG2E;
  a.scale = scale;
  a.fold = fold_part != nullptr;
  a.fold_row = fold_row;
  a.fold_part = fold_part;
  a.clear_acc = clear_acc ? 1 : 0;
  if (seqlen == 0 || batch == 0) return hipSuccess;
  if (a.fold && !dq_prefix_fold(seqlen, a.group, window, prefix)) return hipErrorInvalidValue;
  const int BQ = dq_query_tile(seqlen, a.group, window, prefix);
  a.num_q_tiles = (seqlen + BQ - 1) / BQ;
  // packed sequences: one linear index over every sequence's tiles
  const int tiles = cu_seqlens ? sa_packed_tiles_bound(batch, seqlen, rows_total, BQ)
                               : a.num_q_tiles;
  if (tiles > 65535) return hipErrorInvalidConfiguration;
  if (tiles == 0) return hipSuccess;
  const int gy = cu_seqlens ? 1 : batch;
  if (dq_window_kernel(seqlen, a.group, window, prefix)) {
    hipLaunchKernelGGL(sinkattn_bwd_dq_bf16_d64_win, dim3(heads_kv, gy, tiles),
                       dim3(WAVES * 64), 0, stream, a);
    return hipGetLastError();
  }
  dim3 grid(heads_q, gy, tiles);
  if (k32)
    hipLaunchKernelGGL(sinkattn_bwd_dq_bf16_d64_k32, grid, dim3(WAVES * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(sinkattn_bwd_dq_bf16_d64, grid, dim3(WAVES * 64), 0, stream, a);
  return hipGetLastError();
}
