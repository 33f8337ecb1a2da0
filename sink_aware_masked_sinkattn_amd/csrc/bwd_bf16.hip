// Backward of sink-aware masked attention, bf16, head dim 64, on gfx950 MFMA.
//
// Given the saved content-only log-sum-exp l and the preprocessing pass's
// D_i = rowsum(dO * O) and L_i = logaddexp(l_i, s_h) (sink-inclusive), the
// gradients of attention with a zero-value sink key (arXiv 2608.10357,
// section 5, "Zero-value sink equivalence"; per-head sink gradient as in
// "GPT-OSS Agentic RL training: a practical retrospective", FlashAttention
// v3 implementation section) are, for visible pairs only:
//   P'_ij = exp(S_ij - L_i)            (S_ij = scale q_i . k_j)
//   dV_j += P'_ij dO_i
//   dS_ij = P'_ij (dO_i . v_j - D_i)
//   dK_j += scale dS_ij q_i,  dQ_i += scale dS_ij k_j
// The score matrix is recomputed tile by tile from Q, K and L; nothing of
// size T x T is ever stored (the O(n^2) structure the same section warns of).
//
// Work decomposition: one workgroup = 4 waves = 128 keys of one kv head
// (32 keys per wave, K and V fragments held in registers), looping over the
// query heads it is given and, per head, over the 64-row query tiles that
// can see its keys (from the mask: the rows of a prefix key run to the end
// of the sequence, those of a window key to k + w).  Per query tile:
//   1. S = Q K^T and dP = dO V^T on MFMA with one key per lane (C layout),
//      so P' and dS come out in registers already shaped as the A operand
//      of dV += P'^T dO and dK += dS^T Q; their B operands (dO, Q with the
//      query index along k) are LDS transpose reads of the row-major tiles;
//   2. dS is written to LDS as dS^T [key][query] (8-byte stores);
//   3. dQ (64 x 64) = dS (64 x 128) K (128 x 64) is split over the 4 waves
//      (one 32 x 32 block each, both operands by transpose reads) and added
//      to the fp32 dQ accumulator with one float atomic per element, so the
//      accumulator sees one add per 128 keys instead of per 32.
// dK and dV (fp32, registers) are added to fp32 accumulators at the end; a
// conversion pass applies the scale and writes bf16.  Query/dO tiles are
// double-buffered through registers and LDS.  Rows past the end of a
// sequence get L = +inf (so P' = 0) and are never written.
#include "common.h"
#include "mask_tiles.h"

namespace {

constexpr int D = 64;
constexpr int WAVES = 4;
constexpr int KW = 32;                 // keys per wave
constexpr int BKW = WAVES * KW;        // 128 keys per workgroup
constexpr int BQ = 64;                 // query rows per tile
constexpr int LROW = D + 8;            // padded bf16 row of Q, dO, K tiles
constexpr int SROW = BQ + 8;           // padded bf16 row of dS^T [key][query]

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* l_ws;      // [Hq, rows] L = logaddexp(l, s) (natural log)
  const float* d_ws;      // [Hq, rows] D = rowsum(dO * O)
  float* dq_acc;          // [rows, Hq, D]  sum dS K (unscaled)
  float* dk_acc;          // [rows, Hkv, D] sum dS^T Q (unscaled)
  float* dv_acc;          // [rows, Hkv, D] sum P'^T dO
  const int* cu_seqlens;
  int seqlen, heads_q, heads_kv, group, window, prefix, rows_total;
  int heads_per_wg;       // query heads handled by one workgroup (divides group)
  int num_k_blocks;
  float scale_log2;       // scale * log2(e)
};

struct __attribute__((aligned(16))) BwdSmem {
  bf16 kt[BKW * LROW];          // K rows of this workgroup (for dQ)
  bf16 qt[2][BQ * LROW];        // Q tile, double buffer
  bf16 dot[2][BQ * LROW];       // dO tile, double buffer
  bf16 dst[BKW * SROW];         // dS^T [key][query]
  float l2[2][BQ];              // L * log2(e); +inf for rows past the end
  float dd[2][BQ];              // D
};

__global__ __launch_bounds__(256, 2) void sinkattn_bwd_bf16_d64(BwdArgs a) {
  __shared__ BwdSmem sm;

  const int nsplit = a.group / a.heads_per_wg;
  const int kvh = blockIdx.x % a.heads_kv;
  const int split = blockIdx.x / a.heads_kv;
  const int kblk = blockIdx.y;
  const int z = blockIdx.z;
  (void)nsplit;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int k_start = kblk * BKW;
  if (k_start >= sv.len) return;
  const int k_last = min(k_start + BKW - 1, sv.len - 1);
  int q_lo, q_hi;
  if (!sa_query_range(k_start, k_last, sv.len, a.window, a.prefix, &q_lo, &q_hi)) return;
  const int qt_begin = q_lo / BQ;
  const int n_qt = q_hi / BQ - qt_begin + 1;
  const int h_begin = kvh * a.group + split * a.heads_per_wg;
  const int n_iter = n_qt * a.heads_per_wg;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int kw0 = k_start + wave * KW;
  const bool wave_active = kw0 < sv.len;

  const int q_row_stride = a.heads_q * D;
  const int kv_row_stride = a.heads_kv * D;
  const bf16* kbase = a.k + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;
  const bf16* vbase = a.v + (size_t)sv.row_base * kv_row_stride + (size_t)kvh * D;

  // K / V fragments as the B operand of S = Q K^T, dP = dO V^T:
  // lane = key kw0 + l32, head-dim chunk 16s + 8g .. +7.
  bf16x8 kf[4], vf[4];
  {
    const int key = kw0 + l32;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (key < sv.len) {
        kf[s] = *(const bf16x8*)(kbase + (size_t)key * kv_row_stride + 16 * s + 8 * g);
        vf[s] = *(const bf16x8*)(vbase + (size_t)key * kv_row_stride + 16 * s + 8 * g);
      } else {
        kf[s] = bf16x8{};
        vf[s] = bf16x8{};
      }
    }
  }
  // K rows of the whole workgroup into LDS (row-major) for the dQ stage.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int chunk = tid + 256 * i;          // 1024 chunks of 16 B
    const int r = chunk >> 3;
    const int c = (chunk & 7) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (k_start + r < sv.len) val = *(const uint4*)(kbase + (size_t)(k_start + r) * kv_row_stride + c);
    *(uint4*)(sm.kt + r * LROW + c) = val;
  }

  // Q / dO / L / D tile loader (register prefetch, then LDS store).
  const int ld_r = tid >> 3;                  // 0..31, and +32
  const int ld_c = (tid & 7) * 8;
  uint4 qreg[2], dreg[2];
  float lreg = 0.0f;
  auto tile_of = [&](int it, int* h, int* q0) {
    const int hi = it / n_qt;
    *h = h_begin + hi;
    *q0 = (qt_begin + (it - hi * n_qt)) * BQ;
  };
  auto load_tile = [&](int it) {
    int h, q0;
    tile_of(it, &h, &q0);
    const bf16* qb = a.q + (size_t)sv.row_base * q_row_stride + (size_t)h * D;
    const bf16* db = a.dout + (size_t)sv.row_base * q_row_stride + (size_t)h * D;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = q0 + ld_r + 32 * i;
      if (r < sv.len) {
        qreg[i] = *(const uint4*)(qb + (size_t)r * q_row_stride + ld_c);
        dreg[i] = *(const uint4*)(db + (size_t)r * q_row_stride + ld_c);
      } else {
        qreg[i] = make_uint4(0, 0, 0, 0);
        dreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 2 * BQ) {
      const int r = q0 + (tid & (BQ - 1));
      const size_t wi = (size_t)h * a.rows_total + sv.row_base + r;
      if (tid < BQ) lreg = (r < sv.len) ? a.l_ws[wi] * SA_LOG2E : INFINITY;
      else lreg = (r < sv.len) ? a.d_ws[wi] : 0.0f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(uint4*)(sm.qt[buf] + (ld_r + 32 * i) * LROW + ld_c) = qreg[i];
      *(uint4*)(sm.dot[buf] + (ld_r + 32 * i) * LROW + ld_c) = dreg[i];
    }
    if (tid < BQ) sm.l2[buf][tid] = lreg;
    else if (tid < 2 * BQ) sm.dd[buf][tid - BQ] = lreg;
  };

  f32x16 dk_acc[2], dv_acc[2];
  dk_acc[0] = dk_acc[1] = dv_acc[0] = dv_acc[1] = f32x16{};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    int h, q0;
    tile_of(it, &h, &q0);
    if (it + 1 < n_iter) load_tile(it + 1);
    const int q1 = min(q0 + BQ - 1, sv.len - 1);
    const int cls = wave_active ? sa_tile_class(q0, q1, kw0, kw0 + KW - 1, a.window, a.prefix)
                                : SA_TILE_SKIP;
    const bf16* qs = sm.qt[buf];
    const bf16* ds_ = sm.dot[buf];
    bf16* dsw = sm.dst + (wave * KW + l32) * SROW;   // this lane's dS^T row
    if (cls != SA_TILE_SKIP) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 st = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 qa = *(const bf16x8*)(qs + (qb * 32 + l32) * LROW + 16 * s + 8 * g);
          const bf16x8 da = *(const bf16x8*)(ds_ + (qb * 32 + l32) * LROW + 16 * s + 8 * g);
          st = mfma32x32x16(qa, kf[s], st);
          dp = mfma32x32x16(da, vf[s], dp);
        }
        // rows of this lane's C registers: queries qb*32 + 8*(i/4) + 4g + i%4
        float pp[16], dsv[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int qr = qb * 32 + 8 * i4 + 4 * g;
          const f32x4 l4 = *(const f32x4*)(&sm.l2[buf][qr]);
          const f32x4 d4 = *(const f32x4*)(&sm.dd[buf][qr]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * i4 + e;
            float p = fast_exp2(fmaf(st[i], a.scale_log2, -l4[e]));
            if (cls == SA_TILE_PARTIAL && !sa_visible(q0 + qr + e, kw0 + l32, a.window, a.prefix)) p = 0.0f;
            pp[i] = p;
            dsv[i] = p * (dp[i] - d4[e]);
          }
        }
        // dS^T to LDS: 4 contiguous queries per 8-byte store
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          *(bf16x4*)(dsw + qb * 32 + 8 * i4 + 4 * g) =
              to_bf16x4(dsv[4 * i4], dsv[4 * i4 + 1], dsv[4 * i4 + 2], dsv[4 * i4 + 3]);
        }
        // dV += P'^T dO, dK += dS^T Q; k = 16 queries per step
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 pa = to_bf16x8(pp[8 * hh], pp[8 * hh + 1], pp[8 * hh + 2], pp[8 * hh + 3],
                                      pp[8 * hh + 4], pp[8 * hh + 5], pp[8 * hh + 6], pp[8 * hh + 7]);
          const bf16x8 sa = to_bf16x8(dsv[8 * hh], dsv[8 * hh + 1], dsv[8 * hh + 2], dsv[8 * hh + 3],
                                      dsv[8 * hh + 4], dsv[8 * hh + 5], dsv[8 * hh + 6], dsv[8 * hh + 7]);
          const int r0 = qb * 32 + 16 * hh + 4 * g + (li >> 2);
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const int c0 = db * 32 + 16 * (grp & 1) + 4 * (li & 3);
            const bf16x8 dob = cat8(lds_read_tr4(ds_ + r0 * LROW + c0), lds_read_tr4(ds_ + (r0 + 8) * LROW + c0));
            const bf16x8 qbf = cat8(lds_read_tr4(qs + r0 * LROW + c0), lds_read_tr4(qs + (r0 + 8) * LROW + c0));
            dv_acc[db] = mfma32x32x16(pa, dob, dv_acc[db]);
            dk_acc[db] = mfma32x32x16(sa, qbf, dk_acc[db]);
          }
        }
      }
    } else {
      // nothing visible for this wave: its dS^T rows are zero
#pragma unroll
      for (int c = 0; c < BQ; c += 4) *(bf16x4*)(dsw + c) = bf16x4{};
    }
    __syncthreads();
    // ---- dQ block of this wave: rows qb = wave>>1, columns db = wave&1
    const int wcls = sa_tile_class(q0, q1, k_start, k_last, a.window, a.prefix);
    if (wcls != SA_TILE_SKIP) {
      const int qb = wave >> 1, db = wave & 1;
      f32x16 dq = f32x16{};
#pragma unroll
      for (int ks = 0; ks < BKW / 16; ++ks) {
        const int r0 = ks * 16 + 8 * g + (li >> 2);
        const int ca = qb * 32 + 16 * (grp & 1) + 4 * (li & 3);
        const int cb = db * 32 + 16 * (grp & 1) + 4 * (li & 3);
        const bf16x8 sa = cat8(lds_read_tr4(sm.dst + r0 * SROW + ca), lds_read_tr4(sm.dst + (r0 + 4) * SROW + ca));
        const bf16x8 kb = cat8(lds_read_tr4(sm.kt + r0 * LROW + cb), lds_read_tr4(sm.kt + (r0 + 4) * LROW + cb));
        dq = mfma32x32x16(sa, kb, dq);
      }
      float* dqb = a.dq_acc + ((size_t)sv.row_base * a.heads_q + h) * D + db * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = q0 + qb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (qr < sv.len) unsafeAtomicAdd(dqb + (size_t)qr * q_row_stride, dq[i]);
      }
    }
    if (it + 1 < n_iter) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- dK, dV: C rows are keys kw0 + 8*(i/4) + 4g + i%4, column d = db*32 + l32
  if (wave_active) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      float* dkb = a.dk_acc + ((size_t)sv.row_base * a.heads_kv + kvh) * D + db * 32 + l32;
      float* dvb = a.dv_acc + ((size_t)sv.row_base * a.heads_kv + kvh) * D + db * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kw0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key < sv.len) {
          unsafeAtomicAdd(dkb + (size_t)key * kv_row_stride, dk_acc[db][i]);
          unsafeAtomicAdd(dvb + (size_t)key * kv_row_stride, dv_acc[db][i]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_bwd_bf16_d64(const bf16* q, const bf16* k, const bf16* v, const bf16* dout,
                               const float* l_ws, const float* d_ws, float* dq_acc, float* dk_acc,
                               float* dv_acc, const int* cu_seqlens, int batch, int seqlen,
                               int rows_total, int heads_q, int heads_kv, int window, int prefix,
                               float scale, int heads_per_wg, hipStream_t stream) {
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.l_ws = l_ws; a.d_ws = d_ws;
  a.dq_acc = dq_acc; a.dk_acc = dk_acc; a.dv_acc = dv_acc; a.cu_seqlens = cu_seqlens;
  a.seqlen = seqlen; a.heads_q = heads_q; a.heads_kv = heads_kv;
  a.group = heads_q / heads_kv; a.window = window; a.prefix = prefix;
  a.rows_total = rows_total;
  a.heads_per_wg = heads_per_wg;
  a.num_k_blocks = (seqlen + BKW - 1) / BKW;
  a.scale_log2 = scale * SA_LOG2E;
  if (a.num_k_blocks == 0 || batch == 0) return hipSuccess;
  const int nsplit = a.group / heads_per_wg;
  dim3 grid(heads_kv * nsplit, a.num_k_blocks, batch);
  hipLaunchKernelGGL(sinkattn_bwd_bf16_d64, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}
