// dK and dV of sink-aware masked attention, bf16, head dim 64, gfx950 MFMA.
//
// With L_i = logaddexp(l_i, s_h) and D_i = rowsum(dO * O) from the dQ
// kernel (which runs first), for the visible pairs of the mask
// M[q,k] = 1[k<=q] AND 1[q-k<=w OR k<p] ("Efficient Reinforcement Learning
// for Long-Horizon Tool-Use Agentic Tasks", summary page; the zero-value
// sink of arXiv 2608.10357 section 5 only enters through L and D):
//   P'_ij = exp(S_ij - L_i),  S_ij = scale q_i . k_j
//   dV_j += sum_i P'_ij dO_i
//   dK_j += scale sum_i P'_ij (dO_i . v_j - D_i) q_i
// summed over the query heads of the kv head's GQA group.  No T x T buffer:
// S and dP are recomputed tile by tile from Q, K, V, dO and L.
//
// Work decomposition.  A workgroup (4 waves) owns 128 keys of one kv head,
// 32 per wave, whose K and V
// fragments stay in registers; query tiles are BQ rows (128).  The (query
// tile, query head) pairs that can see those keys -- rows [k0, n) for a
// prefix key, [k0, k1 + w] otherwise -- form the block's iteration list
// (tiles from the last down, heads innermost; heads outermost for windows of
// at most two tiles, so neighbouring blocks read a shared tile one iteration
// apart), cut into work units of 2^chunk_shift iterations.  The grid is the
// exact list of work units (one workgroup each, the extra units of the
// longest key blocks first), so prefix keys (seen by every later row) and
// early causal keys do not leave a few workgroups running long after the
// rest, and no workgroup is launched without work.  When every key block of
// the launch is one unit, each writes its rows as bf16 (dK scaled) directly;
// otherwise a key block covered by one unit stores its fp32 result and a key
// block cut into several units adds them with one float atomic per element,
// once per unit, for the finish phase to convert.  With the prefix fold, the
// first block's query range stops at the fold row: the window dQ kernel
// takes the prefix keys' part of the rows past it.
//
// Per iteration, per wave and 32-row query block, on MFMA 32x32x16 with one
// key per lane (C layout):
//   S = Q K^T, dP = dO V^T   (A = Q, dO rows from LDS; B = K, V registers)
//   P' and dS computed in registers are already the A operand (keys on m,
//   queries on k) of dV += P'^T dO and dK += dS^T Q, whose B operands
//   (queries on k) are transpose reads of the row-major dO and Q tiles.
//   In a partial tile a wave skips the 32-row blocks that see none of its
//   keys.
// Query tiles (Q, dO, L, D) are double-buffered: registers -> LDS.  Rows
// past the end of a sequence get L = +inf, so P' = dS = 0 there.
#include "common.h"
#include "mask_tiles.h"

namespace {

constexpr int D = 64;
constexpr int WAVES = 4;
constexpr int KB = 1;                  // 32-key MFMA blocks per wave
constexpr int KW = 32 * KB;            // keys per wave
constexpr int BKW = WAVES * KW;        // keys per workgroup
// Query tiles of BQ rows (a template parameter; 128 in the launched kernel).

struct DkvArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* l2_ws;     // [Hq, rows] L in log2 units (written by the dQ kernel)
  const float* d_ws;      // [Hq, rows] D
  float* dk_acc;          // [rows, Hkv, D] sum dS^T Q (unscaled)
  float* dv_acc;          // [rows, Hkv, D] sum P'^T dO
  bf16* dk_out;           // [rows, Hkv, D] dK, dV: written here when direct
  bf16* dv_out;
  int direct;             // 1: every key block is one work unit, so each key's row is final
                          // here and goes out as bf16 (dK scaled) -- except, with the fold,
                          // the prefix keys' rows, which go to the accumulators
  float scale;
  const int* cu_seqlens;
  int seqlen, heads_q, heads_kv, group, window, prefix, rows_total;
  int batch;
  int chunk_shift;        // iterations per work unit: 2^chunk_shift
  int fold;               // 1: the window dQ kernel adds the prefix keys' part of rows past
                          // the fold row (sa_dkdv_query_range stops the blocks there)
  int heads_outer;        // iteration order: query heads outermost (short windows)
  float scale_log2;
};

template <int BQ>
struct __attribute__((aligned(128))) DkvSmem {
  bf16 qt[2][BQ * D];          // swizzled rows (tile_off)
  bf16 dot[2][BQ * D];         // dot[b] starts 2 * BQ * D * 2 bytes after qt[b]
  float l2[2][BQ];
  float dd[2][BQ];             // -D of the tile's rows
};

// One BQ-row query tile against this wave's 32 keys.  MASK: apply the
// element predicate (partial tiles); full tiles run without any mask
// arithmetic.
//
// Issue order.  Per 32-row query block the work is four MFMA chains of four
// (S, dP, dV, dK) and two stretches of VALU work that depend on them in turn
// (P' from S; dS from P' and dP).  Left to itself the compiler issues the
// MFMAs in bunches and the VALU work between them, so a wave keeps only one
// of the two units busy at a time.  Here the block is issued as
//   S chain, with L and the dV operands (transpose reads) in its shadow;
//   dP chain, each MFMA followed by a quarter of the P' work;
//   dV chain, each MFMA followed by a quarter of the dS work;
//   dK chain, with the next block's Q and dO rows read in its shadow;
// so each wave overlaps its own VALU work with MFMAs.  sched_barrier fences
// hold every part in place (the compiler may still order inside a part).
// Live registers stay those of the plain order.
template <int BQ, bool MASK>
__device__ __forceinline__ void tile_step(uint32_t qtile, const float* l2s,
                                          const float* dds, const bf16x8 (&kf)[KB][4],
                                          const bf16x8 (&vf)[KB][4], f32x16 (&dk)[KB][2],
                                          f32x16 (&dv)[KB][2], int q0, int kw0, int window,
                                          int prefix, float scale_log2, int lane) {
  static_assert(KB == 1, "the issue order is written for one 32-key block per wave");
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int k = kw0 + l32;
  const int lim = k < prefix ? SA_LIM_PREFIX : window;
  // LDS: the Q tile at byte address qtile, the dO tile DOFF bytes after it.
  // One base register per read pattern (row reads, transpose reads),
  // recomputed per tile: every other operand address is that base XOR a
  // constant plus an immediate offset.
  constexpr int DOFF = 2 * BQ * D * 2;
  const uint32_t ra = (uint32_t)sa_opaque((int)qtile + tile_row_base(l32, g));
  const uint32_t ta =
      (uint32_t)sa_opaque((int)qtile + tile_tr_base(4 * g + (li >> 2), 16 * (grp & 1) + 4 * (li & 3)));
  // A operands of S = Q K^T and dP = dO V^T (query rows, head dim along k)
  bf16x8 qa[4], da[4];
  auto read_rows = [&](int qb) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qa[s] = lds_read8((ra ^ (32 * s)) + qb * 4096);
      da[s] = lds_read8((ra ^ (32 * s)) + qb * 4096 + DOFF);
    }
  };
  // B operand (query index along k) of a dV (TOFF = DOFF) or dK (TOFF = 0)
  // MFMA: rows qb*32 + 16*hh + 4g + li/4 (+8), columns db*32 + 16*(grp&1) + 4*(li&3)
  auto read_tr = [&](int toff, int qb, int hh, int db) {
    const int o = toff + qb * 4096 + hh * 2048;   // folds into the immediate offset
    return cat8(lds_read_tr4_at((ta ^ (64 * db)) + o), lds_read_tr4_at((ta ^ (64 * db + 32)) + o + 1024));
  };
  read_rows(0);

#pragma unroll
  for (int qb = 0; qb < BQ / 32; ++qb) {
    // this lane's C rows are queries qb*32 + 8*(i/4) + 4g + i%4, its column
    // is key k: q - k = base + 8*(i/4) + i%4
    if constexpr (MASK) {
      // a 32-row block that sees none of this wave's keys (the far side of
      // the diagonal or of the window edge) is skipped
      const int ku = __builtin_amdgcn_readfirstlane(kw0);
      const int qu = __builtin_amdgcn_readfirstlane(q0 + qb * 32);
      if (sa_tile_class(qu, qu + 31, ku, ku + 31, window, prefix) == SA_TILE_SKIP) {
        if (qb + 1 < BQ / 32) read_rows(qb + 1);
        continue;
      }
    }
    const int base = sa_opaque(q0 + qb * 32 + 4 * g - k);
    __builtin_amdgcn_sched_barrier(0);
    // L and -D of the block's rows first: LDS reads complete in issue order, so
    // the dP chain (which starts from -D) then waits only for these, not for
    // the transpose reads issued after them; the counter tracks at most 15
    // reads, so the S chain's own operands must not sit behind more than that
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d4[j] = *(const f32x4*)(dds + qb * 32 + 8 * j + 4 * g);
      l4[j] = *(const f32x4*)(l2s + qb * 32 + 8 * j + 4 * g);
    }
    sa_mem_fence();
    f32x16 st = {};
    bf16x8 dob[2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      st = mfma32x32x16(qa[j], kf[0][j], st);
      asm volatile("" : "+v"(st));   // keep the MFMA in this slot
      dob[j >> 1][j & 1] = read_tr(DOFF, qb, j >> 1, j & 1);
      sa_mem_fence();
    }
    // P' = exp2(S*scale*log2e - L*log2e), a quarter after each dP MFMA.  The
    // dP chain accumulates onto -D of each element's row, so it yields dP - D.
    f32x16 dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = d4[i >> 2][i & 3];
    float pp[16];
    bf16x8 pa[2], qbt[2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dp = mfma32x32x16(da[j], vf[0][j], dp);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * j + e;
        float p = fast_exp2(fmaf(st[i], scale_log2, -l4[j][e]));
        if (MASK) p = sa_vis(base + 8 * j + e, lim) ? p : 0.0f;
        pp[i] = p;
      }
      if (j & 1) {
        const int o = 8 * (j >> 1);
        pa[j >> 1] = to_bf16x8(pp[o], pp[o + 1], pp[o + 2], pp[o + 3], pp[o + 4], pp[o + 5],
                               pp[o + 6], pp[o + 7]);
      }
      qbt[j >> 1][j & 1] = read_tr(0, qb, j >> 1, j & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // dV += P'^T dO; dS = P' (dP - D), a quarter after each dV MFMA
    float dsv[16];
    bf16x8 sa[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dv[0][j & 1] = mfma32x32x16(pa[j >> 1], dob[j >> 1][j & 1], dv[0][j & 1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * j + e;
        dsv[i] = pp[i] * dp[i];
      }
      if (j & 1) {
        const int o = 8 * (j >> 1);
        sa[j >> 1] = to_bf16x8(dsv[o], dsv[o + 1], dsv[o + 2], dsv[o + 3], dsv[o + 4], dsv[o + 5],
                               dsv[o + 6], dsv[o + 7]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // dK += dS^T Q, and the next block's rows
#pragma unroll
    for (int j = 0; j < 4; ++j) dk[0][j & 1] = mfma32x32x16(sa[j >> 1], qbt[j >> 1][j & 1], dk[0][j & 1]);
    if (qb + 1 < BQ / 32) read_rows(qb + 1);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The flat work list, sequence by sequence: chunk indices from the highest
// down, and for each index the key blocks that have that many chunks, in key
// order.  The extra chunks of the longest key blocks (prefix keys and early
// causal keys see the most rows) so come first, and the workgroups in flight
// together share a chunk index -- with the iteration order below, the same
// few query tiles, which stay in L2.  Key block 0 always has the most chunks
// (its query range starts lowest and ends highest).  Every wave of the
// workgroup finds work unit `item` with the same lane-parallel count (64 key
// blocks per step).  False if item is past the end (the grid of a packed
// batch is sized by a bound from its token count).
template <int BQ>
__device__ __forceinline__ bool dkdv_find_unit(const DkvArgs& a, int item, int lane, int* z_out,
                                               int* kb_out, int* chunk_out) {
  for (int z = 0; z < a.batch; ++z) {
    const int len = a.cu_seqlens ? a.cu_seqlens[z + 1] - a.cu_seqlens[z] : a.seqlen;
    const int nkb = (len + BKW - 1) / BKW;
    if (nkb == 0) continue;
    const int cmax = sa_dkdv_block_chunks(0, len, a.window, a.prefix, a.group, BQ, BKW,
                                          a.chunk_shift, a.fold);
    // chunk counts of this lane's key blocks are recomputed per level when
    // the sequence has more than 64 blocks, kept in a register otherwise
    const int own = lane < nkb ? sa_dkdv_block_chunks(lane, len, a.window, a.prefix, a.group, BQ,
                                                      BKW, a.chunk_shift, a.fold)
                               : 0;
    for (int c = cmax - 1; c >= 0; --c) {
      for (int kb0 = 0; kb0 < nkb; kb0 += 64) {
        const int kb = kb0 + lane;
        const int ch = kb0 == 0 ? own
                                : (kb < nkb ? sa_dkdv_block_chunks(kb, len, a.window, a.prefix,
                                                                   a.group, BQ, BKW, a.chunk_shift,
                                                                   a.fold)
                                            : 0);
        const bool has = ch > c;
        const unsigned long long m = __ballot(has);
        const int n = __builtin_popcountll(m);
        if (item < n) {
          // lane holding the item-th set bit of m
          const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
          const int L = __builtin_ctzll(__ballot(has && below == item));
          *z_out = __builtin_amdgcn_readfirstlane(z);
          *kb_out = __builtin_amdgcn_readfirstlane(kb0 + L);
          *chunk_out = __builtin_amdgcn_readfirstlane(c);
          return true;
        }
        item -= n;
      }
    }
  }
  return false;
}

constexpr int DKDV_OCC = 2;   // waves per SIMD the register budget is set for
template <int BQ>
__device__ __forceinline__ void dkdv_body(const DkvArgs& a) {
  __shared__ DkvSmem<BQ> sm;

  // grid x = heads_kv * work units, kv head fastest (consecutive workgroups
  // go to consecutive XCDs, so each XCD keeps to its kv heads)
  const int kvh = blockIdx.x % a.heads_kv;
  int z, kblk, chunk_id;
  if (!dkdv_find_unit<BQ>(a, blockIdx.x / a.heads_kv, threadIdx.x & 63, &z, &kblk, &chunk_id))
    return;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int k_start = kblk * BKW;
  if (k_start >= sv.len) return;
  int q_lo, q_hi;
  if (!sa_dkdv_query_range(kblk, sv.len, a.window, a.prefix, BQ, BKW, a.fold, &q_lo, &q_hi))
    return;
  const int qt_begin = q_lo / BQ;
  const int n_qt = q_hi / BQ - qt_begin + 1;
  const int n_iter_all = n_qt * a.group;
  const int it_begin = chunk_id << a.chunk_shift;
  if (it_begin >= n_iter_all) return;
  const int it_end = min(it_begin + (1 << a.chunk_shift), n_iter_all);
  const bool single = (it_begin == 0) && (it_end == n_iter_all);
  const int h_begin = kvh * a.group;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int kw0 = k_start + wave * KW;
  const bool wave_active = kw0 < sv.len;

  const int q_row_stride = a.heads_q * D;
  const int kv_row_stride = a.heads_kv * D;
  const bf16* kbase = a.k + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;
  const bf16* vbase = a.v + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;

  // K / V fragments, B operand of S = Q K^T and dP = dO V^T:
  // lane = key kw0 + kb*32 + l32, head-dim chunk 16s + 8g .. +7.
  bf16x8 kf[KB][4], vf[KB][4];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = kw0 + kb * 32 + l32;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (key < sv.len) {
        kf[kb][s] = *(const bf16x8*)(kbase + (size_t)key * kv_row_stride + 16 * s + 8 * g);
        vf[kb][s] = *(const bf16x8*)(vbase + (size_t)key * kv_row_stride + 16 * s + 8 * g);
      } else {
        kf[kb][s] = bf16x8{};
        vf[kb][s] = bf16x8{};
      }
    }
  }

  // Q / dO tiles go straight from global memory into swizzled LDS tiles;
  // L (in log2 units) and D go through one register per thread, with
  // L = +inf for rows past the end of the sequence so P' = dS = 0 there.
  float lreg = 0.0f;
  // Iteration order: query tiles from the last to the first, query heads
  // innermost.  All key blocks of a causal layer share the same last tile, so
  // workgroups running at the same time walk the same (tile, head) sequence
  // in step and their Q/dO tiles stay in the XCD's L2.
  const int qt_last = qt_begin + n_qt - 1;
  auto tile_of = [&](int it, int* h, int* q0) {
    if (a.heads_outer) {
      const int hi = it / n_qt;
      *h = h_begin + hi;
      *q0 = (qt_last - (it - hi * n_qt)) * BQ;
    } else {
      const int ti = it / a.group;
      *h = h_begin + (it - ti * a.group);
      *q0 = (qt_last - ti) * BQ;
    }
  };
  const TileLane tl = tile_lane(lane, q_row_stride * 2);
  auto load_tile = [&](int it, int buf) {
    int h, q0;
    tile_of(it, &h, &q0);
    const size_t off = ((size_t)sv.row_base + q0) * q_row_stride + (size_t)h * D;
    tile_load_lds_lane<BQ, WAVES>(sm.qt[buf], a.q + off, q_row_stride * 2, sv.len - q0, wave, tl);
    tile_load_lds_lane<BQ, WAVES>(sm.dot[buf], a.dout + off, q_row_stride * 2, sv.len - q0, wave, tl);
    static_assert(2 * BQ <= 256, "L and D are staged by one thread per row");
    if (tid < 2 * BQ) {
      const int r = q0 + (tid & (BQ - 1));
      const size_t wi = (size_t)h * a.rows_total + sv.row_base + r;
      if (tid < BQ) lreg = (r < sv.len) ? a.l2_ws[wi] : INFINITY;
      else lreg = (r < sv.len) ? -a.d_ws[wi] : 0.0f;   // -D: the dP chain starts from it
    }
  };
  auto store_stats = [&](int buf) {
    if (tid < BQ) sm.l2[buf][tid] = lreg;
    else if (tid < 2 * BQ) sm.dd[buf][tid - BQ] = lreg;
  };

  f32x16 dk_acc[KB][2], dv_acc[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) dk_acc[kb][0] = dk_acc[kb][1] = dv_acc[kb][0] = dv_acc[kb][1] = f32x16{};

  load_tile(it_begin, 0);
  store_stats(0);
  wait_all_mem();
  __syncthreads();

  for (int it = it_begin; it < it_end; ++it) {
    const int buf = (it - it_begin) & 1;
    int h, q0;
    tile_of(it, &h, &q0);
    (void)h;
    if (it + 1 < it_end) load_tile(it + 1, buf ^ 1);
    const int q1 = min(q0 + BQ - 1, sv.len - 1);
    const int cls = wave_active ? sa_tile_class(q0, q1, kw0, kw0 + KW - 1, a.window, a.prefix)
                                : SA_TILE_SKIP;
    if (cls == SA_TILE_FULL) {
      tile_step<BQ, false>(lds_addr(sm.qt[buf]), sm.l2[buf], sm.dd[buf], kf, vf, dk_acc, dv_acc,
                       q0, kw0, a.window, a.prefix, a.scale_log2, lane);
    } else if (cls == SA_TILE_PARTIAL) {
      tile_step<BQ, true>(lds_addr(sm.qt[buf]), sm.l2[buf], sm.dd[buf], kf, vf, dk_acc, dv_acc,
                       q0, kw0, a.window, a.prefix, a.scale_log2, lane);
    }
    if (it + 1 < it_end) store_stats(buf ^ 1);
    wait_all_mem();
    __syncthreads();
  }

  // The epilogue reads the accumulators element by element; an asm operand
  // holding each as one register tuple here keeps the register allocator
  // from carrying a second, split copy through the loop (32 v_mov per tile).
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < 2; ++db) asm volatile("" : "+v"(dk_acc[kb][db]), "+v"(dv_acc[kb][db]));
  // ---- C rows are keys kw0 + kb*32 + 8*(i/4) + 4g + i%4, column d = db*32 + l32
  if (wave_active && a.direct) {
    // every unit covers its whole block: the rows are final (but for the
    // prefix keys the fold completes)
    const int acc_below = a.fold ? a.prefix : 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const size_t e0 = ((size_t)sv.row_base * a.heads_kv + kvh) * D + db * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kw0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          const size_t e = e0 + (size_t)key * kv_row_stride;
          if (key < sv.len) {
            if (key < acc_below) {
              a.dk_acc[e] = dk_acc[kb][db][i];
              a.dv_acc[e] = dv_acc[kb][db][i];
            } else {
              a.dk_out[e] = (bf16)(dk_acc[kb][db][i] * a.scale);
              a.dv_out[e] = (bf16)dv_acc[kb][db][i];
            }
          }
        }
      }
  } else if (wave_active) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        float* dkb = a.dk_acc + ((size_t)sv.row_base * a.heads_kv + kvh) * D + db * 32 + l32;
        float* dvb = a.dv_acc + ((size_t)sv.row_base * a.heads_kv + kvh) * D + db * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kw0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key < sv.len) {
            if (single) {
              dkb[(size_t)key * kv_row_stride] = dk_acc[kb][db][i];
              dvb[(size_t)key * kv_row_stride] = dv_acc[kb][db][i];
            } else {
              unsafeAtomicAdd(dkb + (size_t)key * kv_row_stride, dk_acc[kb][db][i]);
              unsafeAtomicAdd(dvb + (size_t)key * kv_row_stride, dv_acc[kb][db][i]);
            }
          }
        }
      }
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DKDV_OCC, DKDV_OCC))) void sinkattn_bwd_dkdv_bf16_d64(DkvArgs a) {
  dkdv_body<128>(a);
}
}  // namespace

// Query-tile height of the dK/dV kernel for a window w (already clamped to
// the sequence length).  128 rows for every window: shorter tiles were
// measured slower even for w = 128 (more iterations per workgroup).
int dkdv_query_tile(int window) { (void)window; return 128; }

// First row past which the dK/dV kernel's first key block sees only its
// prefix keys (the rows it stops at when the window dQ kernel folds them).
long long dkdv_prefix_fold_row(int window) {
  return sa_prefix_fold_row(0, window, BKW, dkdv_query_tile(window));
}

// Iterations per work unit: about DKDV_TARGET_UNITS units over the whole call
// so the longest one is short next to the total (no long tail), but long
// enough that the per-unit atomic flush of dK/dV stays small (at least
// 2^4 iterations).  A power of two.
constexpr long long DKDV_TARGET_UNITS = 8192;
int bwd_dkdv_chunk_shift(long long total_iters) {
  int sh = 4;
  while (sh < 8 && ((long long)1 << sh) * DKDV_TARGET_UNITS < total_iters) ++sh;
  return sh;
}

// Iterations per work unit for a launch: from the total over every block of
// every sequence at the longest length.  *max_chunks: the most units any key
// block is cut into (a bound for every packed sequence too: a shorter
// sequence's block sees no more query tiles).
static int dkdv_plan(int batch, int seqlen, int group, int heads_kv, int window, int prefix,
                     bool fold, int* max_chunks) {
  const int nkb = (seqlen + BKW - 1) / BKW;
  const int BQ = dkdv_query_tile(window);
  long long iters = 0;
  for (int kb = 0; kb < nkb; ++kb)
    iters += (long long)sa_dkdv_block_chunks(kb, seqlen, window, prefix, group, BQ, BKW, 0, fold);
  const int shift = bwd_dkdv_chunk_shift(iters * batch * heads_kv);
  int mc = 0;
  for (int kb = 0; kb < nkb; ++kb)
    mc = max(mc, sa_dkdv_block_chunks(kb, seqlen, window, prefix, group, BQ, BKW, shift, fold));
  *max_chunks = mc;
  return shift;
}

// Whether the dK/dV launch for this problem adds into its fp32 accumulators
// (some key block is cut into several work units, whose parts are added with
// atomics) and so needs them cleared first and converted after; with one
// unit per block every key's row is final in the kernel and goes out as bf16
// directly (with the prefix fold, the prefix keys' rows excepted).
bool dkdv_accumulates(int batch, int seqlen, int heads_q, int heads_kv, int window, int prefix,
                      bool fold) {
  if (seqlen == 0 || batch == 0 || heads_kv == 0) return false;
  int mc;
  dkdv_plan(batch, seqlen, heads_q / heads_kv, heads_kv, window, prefix, fold, &mc);
  return mc > 1;
}

hipError_t launch_bwd_dkdv_bf16_d64(const bf16* q, const bf16* k, const bf16* v,
                                    const bf16* dout, const float* l_ws, const float* d_ws,
                                    float* dk_acc, float* dv_acc, const int* cu_seqlens,
                                    int batch, int seqlen, int rows_total, int heads_q,
                                    int heads_kv, int window, int prefix, float scale, bool fold,
                                    bf16* dk, bf16* dv, hipStream_t stream) {
  DkvArgs a;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.l2_ws = l_ws; a.d_ws = d_ws;
  a.dk_acc = dk_acc; a.dv_acc = dv_acc; a.cu_seqlens = cu_seqlens;
  a.seqlen = seqlen; a.heads_q = heads_q; a.heads_kv = heads_kv;
  a.group = heads_q / heads_kv; a.window = window; a.prefix = prefix;
  a.rows_total = rows_total;
  a.scale_log2 = scale * SA_LOG2E;
  a.batch = batch;
  a.fold = fold ? 1 : 0;
  const int nkb = (seqlen + BKW - 1) / BKW;
  if (nkb == 0 || batch == 0) return hipSuccess;
  const int BQ = dkdv_query_tile(window);
  a.heads_outer = window <= 2 * BQ ? 1 : 0;
  int max_chunks;   // > 1: the dQ kernel cleared the accumulators these units add into
  a.chunk_shift = dkdv_plan(batch, seqlen, a.group, heads_kv, window, prefix, fold, &max_chunks);
  a.direct = max_chunks <= 1 ? 1 : 0;
  a.dk_out = dk; a.dv_out = dv;
  a.scale = scale;
  long long units = 0;
  for (int kb = 0; kb < nkb; ++kb)
    units += sa_dkdv_block_chunks(kb, seqlen, window, prefix, a.group, BQ, BKW, a.chunk_shift,
                                  fold);
  units *= batch;   // every sequence at the longest length
  if (cu_seqlens) {
    // Packed sequences of total length rows_total: a bound from the token count (the
    // lengths stay on the device).  A block holding prefix keys (the first ceil(p / BKW))
    // sees every later row, ceil(n / BQ) query tiles, so at most
    // ceil(ceil(n / BQ) * group / 2^s) units (with the fold its range stops at the fold
    // row and it counts with the others); any other block sees at most BKW + w rows,
    // no more units than the largest count among such blocks at the longest length (the
    // same key offsets, a query range no longer).  With sum ceil(n / B) <= (N + G (B - 1)) / B
    // over the sequences, the units of the whole launch stay within the sum below.
    const int npb = fold ? 0 : min((prefix + BKW - 1) / BKW, nkb);
    long long cw = 0;
    for (int kb = npb; kb < nkb; ++kb)
      cw = max(cw, (long long)sa_dkdv_block_chunks(kb, seqlen, window, prefix, a.group, BQ, BKW,
                                                    a.chunk_shift, fold));
    const long long tiles_q = sa_packed_tiles_bound(batch, seqlen, rows_total, BQ);
    const long long blocks = sa_packed_tiles_bound(batch, seqlen, rows_total, BKW);
    const long long per_chunk = 1LL << a.chunk_shift;
    const long long packed = npb * ((a.group * tiles_q + batch * (per_chunk - 1)) / per_chunk) +
                             cw * blocks;
    if (packed < units) units = packed;
  }
  if (units * heads_kv > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (units == 0) return hipSuccess;
  dim3 grid((unsigned)(units * heads_kv));
  hipLaunchKernelGGL(sinkattn_bwd_dkdv_bf16_d64, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}
