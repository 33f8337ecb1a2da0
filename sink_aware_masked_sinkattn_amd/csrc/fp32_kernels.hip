// fp32 path: the same operation as the bf16 MFMA path (forward, dQ, dK/dV),
// in plain fp32 vector arithmetic with accurate expf/logf, for callers that
// need fp32 results (the tiny 1e-5 configuration).  One thread per query row
// (forward, dQ) or per key row (dK, dV); rows loop over exactly the keys or
// queries the mask
//   M[q,k] = 1[k<=q] AND 1[q-k<=w OR k<p]
// ("Efficient Reinforcement Learning for Long-Horizon Tool-Use Agentic
// Tasks", summary page, sink-aware FlexAttention paragraph) leaves visible,
// with an online softmax in the forward and the sink scaling
// O = acc / (r + exp(s - m)) (arXiv 2608.10357 section 5, zero-value sink
// equivalence).  Intended for short sequences; not a performance path.
#include "common.h"
#include "mask_tiles.h"

namespace {

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* sinks;
  const float* o;
  const float* dout;
  const float* l_ws;     // L = logaddexp(l, s), [Hq, rows]
  const float* d_ws;     // D = rowsum(dO * O), [Hq, rows]
  float* out_o;
  float* out_lse;
  float* dq;
  float* dk;
  float* dv;
  const int* cu_seqlens;
  int seqlen, heads_q, heads_kv, group, window, prefix, rows_total, lse_head_stride;
  float scale;
};

// Visible keys of row q: the prefix [0, min(p, q+1)) then the window keys
// [max(q-w, 0), q] that are not prefix keys.
__device__ __forceinline__ void key_ranges(int q, int w, int p, int* a0, int* a1, int* b0, int* b1) {
  *a0 = 0;
  *a1 = min(p, q + 1);
  const long long lo = (long long)q - (long long)w;
  const int wlo = lo > 0 ? (int)lo : 0;
  *b0 = max(wlo, *a1);
  *b1 = q + 1;
}

template <int D>
__global__ __launch_bounds__(64) void f32_fwd(F32Args a) {
  const int h = blockIdx.y;
  const int z = blockIdx.z;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int qi = blockIdx.x * 64 + threadIdx.x;
  if (qi >= sv.len) return;
  const int kvh = h / a.group;
  const size_t qrow = (size_t)sv.row_base + qi;
  float qv[D], acc[D];
  for (int c = 0; c < D; ++c) {
    qv[c] = a.q[(qrow * a.heads_q + h) * D + c];
    acc[c] = 0.0f;
  }
  float m = -INFINITY, r = 0.0f;
  int rng[4];
  key_ranges(qi, a.window, a.prefix, &rng[0], &rng[1], &rng[2], &rng[3]);
  for (int part = 0; part < 2; ++part) {
    for (int kj = rng[2 * part]; kj < rng[2 * part + 1]; ++kj) {
      const float* kr = a.k + (((size_t)sv.row_base + kj) * a.heads_kv + kvh) * D;
      const float* vr = a.v + (((size_t)sv.row_base + kj) * a.heads_kv + kvh) * D;
      float sc = 0.0f;
      for (int c = 0; c < D; ++c) sc = fmaf(qv[c], kr[c], sc);
      sc *= a.scale;
      const float m_new = fmaxf(m, sc);
      const float corr = expf(m - m_new);   // m = -inf only before the first key: corr = 0
      const float pj = expf(sc - m_new);
      r = r * corr + pj;
      for (int c = 0; c < D; ++c) acc[c] = fmaf(pj, vr[c], acc[c] * corr);
      m = m_new;
    }
  }
  const float s = a.sinks[h];
  const float inv = 1.0f / (r + expf(s - m));
  for (int c = 0; c < D; ++c) a.out_o[(qrow * a.heads_q + h) * D + c] = acc[c] * inv;
  if (a.out_lse) a.out_lse[sv.lse_base + (size_t)h * a.lse_head_stride + qi] = m + logf(r);
}

// dQ_i = scale * sum_j dS_ij k_j,  dS_ij = P'_ij (dO_i . v_j - D_i),  P'_ij = exp(S_ij - L_i)
template <int D>
__global__ __launch_bounds__(64) void f32_dq(F32Args a) {
  const int h = blockIdx.y;
  const int z = blockIdx.z;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int qi = blockIdx.x * 64 + threadIdx.x;
  if (qi >= sv.len) return;
  const int kvh = h / a.group;
  const size_t qrow = (size_t)sv.row_base + qi;
  float qv[D], dov[D], acc[D];
  for (int c = 0; c < D; ++c) {
    qv[c] = a.q[(qrow * a.heads_q + h) * D + c];
    dov[c] = a.dout[(qrow * a.heads_q + h) * D + c];
    acc[c] = 0.0f;
  }
  const float big_l = a.l_ws[(size_t)h * a.rows_total + qrow];
  const float dd = a.d_ws[(size_t)h * a.rows_total + qrow];
  int rng[4];
  key_ranges(qi, a.window, a.prefix, &rng[0], &rng[1], &rng[2], &rng[3]);
  for (int part = 0; part < 2; ++part) {
    for (int kj = rng[2 * part]; kj < rng[2 * part + 1]; ++kj) {
      const float* kr = a.k + (((size_t)sv.row_base + kj) * a.heads_kv + kvh) * D;
      const float* vr = a.v + (((size_t)sv.row_base + kj) * a.heads_kv + kvh) * D;
      float sc = 0.0f, dp = 0.0f;
      for (int c = 0; c < D; ++c) {
        sc = fmaf(qv[c], kr[c], sc);
        dp = fmaf(dov[c], vr[c], dp);
      }
      const float pp = expf(sc * a.scale - big_l);
      const float ds = pp * (dp - dd);
      for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, kr[c], acc[c]);
    }
  }
  for (int c = 0; c < D; ++c) a.dq[(qrow * a.heads_q + h) * D + c] = acc[c] * a.scale;
}

// dK_j = scale * sum_{h in group} sum_i dS_ij q_i,  dV_j = sum_{h in group} sum_i P'_ij dO_i
template <int D>
__global__ __launch_bounds__(64) void f32_dkdv(F32Args a) {
  const int kvh = blockIdx.y;
  const int z = blockIdx.z;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int kj = blockIdx.x * 64 + threadIdx.x;
  if (kj >= sv.len) return;
  const size_t krow = (size_t)sv.row_base + kj;
  float kv[D], vv[D], dk[D], dv[D];
  for (int c = 0; c < D; ++c) {
    kv[c] = a.k[(krow * a.heads_kv + kvh) * D + c];
    vv[c] = a.v[(krow * a.heads_kv + kvh) * D + c];
    dk[c] = 0.0f;
    dv[c] = 0.0f;
  }
  int qlo, qhi;
  if (sa_query_range(kj, kj, sv.len, a.window, a.prefix, &qlo, &qhi)) {
    for (int hh = 0; hh < a.group; ++hh) {
      const int h = kvh * a.group + hh;
      for (int qi = qlo; qi <= qhi; ++qi) {
        const size_t qrow = (size_t)sv.row_base + qi;
        const float* qr = a.q + (qrow * a.heads_q + h) * D;
        const float* dor = a.dout + (qrow * a.heads_q + h) * D;
        float sc = 0.0f, dp = 0.0f;
        for (int c = 0; c < D; ++c) {
          sc = fmaf(qr[c], kv[c], sc);
          dp = fmaf(dor[c], vv[c], dp);
        }
        const float pp = expf(sc * a.scale - a.l_ws[(size_t)h * a.rows_total + qrow]);
        const float ds = pp * (dp - a.d_ws[(size_t)h * a.rows_total + qrow]);
        for (int c = 0; c < D; ++c) {
          dk[c] = fmaf(ds, qr[c], dk[c]);
          dv[c] = fmaf(pp, dor[c], dv[c]);
        }
      }
    }
  }
  for (int c = 0; c < D; ++c) {
    a.dk[(krow * a.heads_kv + kvh) * D + c] = dk[c] * a.scale;
    a.dv[(krow * a.heads_kv + kvh) * D + c] = dv[c];
  }
}

template <int D>
hipError_t f32_fwd_launch(const F32Args& a, int batch, hipStream_t st) {
  dim3 grid((a.seqlen + 63) / 64, a.heads_q, batch);
  hipLaunchKernelGGL(f32_fwd<D>, grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t f32_bwd_launch(const F32Args& a, int batch, bool do_dq, bool do_dkdv, hipStream_t st) {
  if (do_dq) {
    dim3 gq((a.seqlen + 63) / 64, a.heads_q, batch);
    hipLaunchKernelGGL(f32_dq<D>, gq, dim3(64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (do_dkdv) {
    dim3 gk((a.seqlen + 63) / 64, a.heads_kv, batch);
    hipLaunchKernelGGL(f32_dkdv<D>, gk, dim3(64), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

F32Args make_args(const int* cu_seqlens, int seqlen, int total_tokens, int heads_q, int heads_kv,
                  int window, int prefix, float scale) {
  F32Args a = {};
  a.cu_seqlens = cu_seqlens;
  a.seqlen = seqlen; a.heads_q = heads_q; a.heads_kv = heads_kv;
  a.group = heads_q / heads_kv; a.window = window; a.prefix = prefix;
  a.rows_total = total_tokens;
  a.lse_head_stride = cu_seqlens ? total_tokens : seqlen;
  a.scale = scale;
  return a;
}

}  // namespace

hipError_t launch_fwd_f32(int head_dim, const float* q, const float* k, const float* v,
                          const float* sinks, float* o, float* lse, const int* cu_seqlens,
                          int batch, int seqlen, int total_tokens, int heads_q, int heads_kv,
                          int window, int prefix, float scale, hipStream_t stream) {
  if (batch == 0 || seqlen == 0 || heads_q == 0) return hipSuccess;
  F32Args a = make_args(cu_seqlens, seqlen, total_tokens, heads_q, heads_kv, window, prefix, scale);
  a.q = q; a.k = k; a.v = v; a.sinks = sinks; a.out_o = o; a.out_lse = lse;
  if (head_dim == 32) return f32_fwd_launch<32>(a, batch, stream);
  if (head_dim == 64) return f32_fwd_launch<64>(a, batch, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_f32(int head_dim, const float* q, const float* k, const float* v,
                          const float* dout, const float* l_ws, const float* d_ws, float* dq,
                          float* dk, float* dv, const int* cu_seqlens, int batch, int seqlen,
                          int total_tokens, int heads_q, int heads_kv, int window, int prefix,
                          float scale, bool do_dq, bool do_dkdv, hipStream_t stream) {
  if (batch == 0 || seqlen == 0 || heads_q == 0) return hipSuccess;
  F32Args a = make_args(cu_seqlens, seqlen, total_tokens, heads_q, heads_kv, window, prefix, scale);
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.l_ws = l_ws; a.d_ws = d_ws;
  a.dq = dq; a.dk = dk; a.dv = dv;
  if (head_dim == 32) return f32_bwd_launch<32>(a, batch, do_dq, do_dkdv, stream);
  if (head_dim == 64) return f32_bwd_launch<64>(a, batch, do_dq, do_dkdv, stream);
  return hipErrorInvalidValue;
}
