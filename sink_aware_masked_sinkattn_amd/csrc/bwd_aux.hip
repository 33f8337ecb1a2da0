// Backward helpers around the dK/dV and dQ kernels: the row preprocessing
// pass of the fp32 path (the bf16 dQ kernel computes the same statistics for
// its own rows), the dK/dV conversion pass and the prefix fold's sum.  All
// are HBM-bound streaming kernels.
//
// Preprocessing, per (row i, query head h) -- the sink gradient of "GPT-OSS
// Agentic RL training: a practical retrospective" (FlashAttention v3
// implementation section), written out with the sink as a zero-value key
// (arXiv 2608.10357, section 5):
//   D_i = sum_c dO_ic O_ic
//   L_i = logaddexp(l_i, s_h)                (sink-inclusive log-normaliser)
//   ds_h -= exp(s_h - L_i) D_i               (summed over all rows)
// D and L go to the workspace for the fp32 main kernel.  The ds_h partial
// sums of a wave are reduced with cross-lane shuffles, then added with one
// float atomic per wave (fp32 dsinks is reproducible to rounding only).
#include "common.h"

namespace {

// 16 bytes (4 floats) of a row per lane.
template <int D>
struct RowSplit {
  static constexpr int kElems = 4;
  static constexpr int kLanesPerRow = D / kElems;
  static constexpr int kRowsPerPass = 64 / kLanesPerRow;
};

struct PreArgs {
  const float* o;
  const float* dout;
  const float* lse;
  const float* sinks;
  const int* cu_seqlens;
  float* dsinks;
  float* d_ws;        // [Hq, rows] : D_i
  float* l_ws;        // [Hq, rows] : L_i (natural log)
  int seqlen, heads_q, rows_total;
  int lse_head_stride;
  int rows_per_wave;
};

template <int D>
__global__ __launch_bounds__(256) void sinkattn_bwd_pre(PreArgs a) {
  using RS = RowSplit<D>;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  if (h >= a.heads_q) return;
  const int z = blockIdx.z;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int r_begin = blockIdx.x * a.rows_per_wave;
  const int r_end = min(r_begin + a.rows_per_wave, sv.len);
  const float s = a.sinks[h];
  const int sub = lane % RS::kLanesPerRow;        // which 16-byte chunk of the row
  const int rsub = lane / RS::kLanesPerRow;       // which row of the pass
  float ds_part = 0.0f;
  for (int r0 = r_begin; r0 < r_end; r0 += RS::kRowsPerPass) {
    const int r = r0 + rsub;
    float dot = 0.0f;
    const size_t row = (size_t)sv.row_base + r;
    if (r < r_end) {
      const size_t off = (row * a.heads_q + h) * D + sub * RS::kElems;
      const float* po = a.o + off;
      const float* pd = a.dout + off;
#pragma unroll
      for (int e = 0; e < RS::kElems; ++e) dot += po[e] * pd[e];
    }
#pragma unroll
    for (int w = 1; w < RS::kLanesPerRow; w <<= 1) dot += __shfl_xor(dot, w);
    if (r < r_end && sub == 0) {
      const float l = a.lse[sv.lse_base + (size_t)h * a.lse_head_stride + r];
      const float mx = fmaxf(l, s);
      const float big_l = (s == -INFINITY) ? l : mx + log1pf(expf(-fabsf(l - s)));
      const size_t wi = (size_t)h * a.rows_total + row;
      a.d_ws[wi] = dot;
      a.l_ws[wi] = big_l;
      ds_part -= expf(s - big_l) * dot;
    }
  }
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) ds_part += __shfl_xor(ds_part, w);
  if (lane == 0 && r_end > r_begin) unsafeAtomicAdd(a.dsinks + h, ds_part);
}

// Same pass, one thread per (row, head): thread t of a block handles query
// head t % Hq of row (block row base) + t / Hq + k * (256 / Hq), k < passes.
// Consecutive threads read consecutive heads of a row, i.e. one contiguous
// Hq * D stretch of O and dO; every thread issues all 16-byte loads of its
// row segment at once.  Used when 256 % Hq == 0.  ds_h partials are summed
// per head in LDS, then added with one atomic per (block, head).
template <int D>
__global__ __launch_bounds__(256) void sinkattn_bwd_pre_rows(PreArgs a, int passes) {
  constexpr int kVec = 4;                            // floats per 16-byte load
  constexpr int kLoads = D / kVec;
  __shared__ float red[256];
  const int t = threadIdx.x;
  const int h = t % a.heads_q;
  const int rows_per_pass = 256 / a.heads_q;
  const int z = blockIdx.z;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int r_begin = blockIdx.x * rows_per_pass * passes + t / a.heads_q;
  const float s = a.sinks[h];
  float ds_part = 0.0f;
  for (int k = 0; k < passes; ++k) {
    const int r = r_begin + k * rows_per_pass;
    if (r >= sv.len) break;
    const size_t row = (size_t)sv.row_base + r;
    const size_t off = (row * a.heads_q + h) * D;
    uint4 ov[kLoads], dv[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      ov[j] = ((const uint4*)(a.o + off))[j];
      dv[j] = ((const uint4*)(a.dout + off))[j];
    }
    float dot = 0.0f;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const float* po = (const float*)&ov[j];
      const float* pd = (const float*)&dv[j];
#pragma unroll
      for (int e = 0; e < kVec; ++e) dot = fmaf(po[e], pd[e], dot);
    }
    const float l = a.lse[sv.lse_base + (size_t)h * a.lse_head_stride + r];
    const float mx = fmaxf(l, s);
    const float big_l = (s == -INFINITY) ? l : mx + log1pf(expf(-fabsf(l - s)));
    const size_t wi = (size_t)h * a.rows_total + row;
    a.d_ws[wi] = dot;
    a.l_ws[wi] = big_l;
    ds_part -= expf(s - big_l) * dot;
  }
  red[t] = ds_part;
  __syncthreads();
  if (t < a.heads_q) {
    float sum = 0.0f;
    for (int i = t; i < 256; i += a.heads_q) sum += red[i];
    if (sum != 0.0f) unsafeAtomicAdd(a.dsinks + t, sum);
  }
}

__global__ void sinkattn_zero_f32(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// fp32 dK / dV accumulators -> bf16 outputs, with the softmax scale folded
// into dK here (the dK/dV kernel accumulates dS^T Q unscaled).
__global__ __launch_bounds__(256) void sinkattn_convert(const float* dk_acc, const float* dv_acc,
                                                        bf16* dk, bf16* dv, long long n_kv4,
                                                        float scale, const float* ds_part,
                                                        int ds_used, int ds_stride, int heads,
                                                        float* dsinks) {
  // workgroup h < heads also forms ds_h from the dQ kernel's per-workgroup
  // parts: each thread adds slots tid, tid + 256, ... in order, then the 256
  // thread sums are added in thread order -- the same order every call
  if ((int)blockIdx.x < heads) {
    __shared__ float red[256];
    const float* src = ds_part + (size_t)blockIdx.x * ds_stride;
    float t = 0.0f;
    for (int i = threadIdx.x; i < ds_used; i += 256) t += src[i];
    red[threadIdx.x] = t;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) dsinks[blockIdx.x] = red[0];
  }
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n_kv4; i += stride) {
    const float4 k4 = ((const float4*)dk_acc)[i];
    const float4 v4 = ((const float4*)dv_acc)[i];
    *(bf16x4*)(dk + 4 * i) = to_bf16x4(k4.x * scale, k4.y * scale, k4.z * scale, k4.w * scale);
    *(bf16x4*)(dv + 4 * i) = to_bf16x4(v4.x, v4.y, v4.z, v4.w);
  }
}

// Finish phase of the prefix fold: for sequence z (grid x), kv head (grid y)
// and 64 VEC of the 2 p D values of the prefix keys' dK and dV (grid z; lane
// = VEC consecutive values), add the parts the window dQ kernel's blocks past
// the fold row wrote to their slots onto the fp32 accumulators.  The slots of
// a sequence are consecutive (z * num_q_tiles .. for fixed length, the
// sequence's run of the packed tile index) and run from its last 32-row
// block down, so its blocks past the fold row are its first slots.  Wave w
// adds slots w, w + 16, ... in order (all its loads in flight at once), then
// the 16 wave sums are added in wave order.  dk_out != nullptr: the dK/dV
// kernel stored every other row as bf16, and these rows go out here the
// same way (dK scaled); otherwise the sums are added into the accumulators
// for the convert pass.
constexpr int FOLD_D = 64;
constexpr int FOLD_ADD_WAVES = 16;
constexpr int FOLD_ADD_LOADS = 16;   // slots per wave in flight
template <int VEC>
struct FoldVec;
template <>
struct FoldVec<1> {
  typedef float T;
  static __device__ T zero() { return 0.0f; }
  static __device__ void add(T& a, const T& b) { a += b; }
  static __device__ void store_bf16(bf16* p, const T& x, float sc) { *p = (bf16)(x * sc); }
};
template <>
struct FoldVec<4> {
  typedef float4 T;
  static __device__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ void add(T& a, const T& b) { a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w; }
  static __device__ void store_bf16(bf16* p, const T& x, float sc) {
    *(bf16x4*)p = to_bf16x4(x.x * sc, x.y * sc, x.z * sc, x.w * sc);
  }
};

template <int VEC>
__global__ __launch_bounds__(FOLD_ADD_WAVES * 64) void sinkattn_prefix_fold_add(
    const float* fold_part, float* dk_acc, float* dv_acc, bf16* dk_out, bf16* dv_out,
    float scale, const int* cu_seqlens, int seqlen, int heads_kv, int prefix, int ds_stride,
    int num_q_tiles, int fold_tiles) {
  using V = FoldVec<VEC>;
  typedef typename V::T T;
  const int z = blockIdx.x;
  const int kvh = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  __shared__ int s_first;
  __shared__ T red[FOLD_ADD_WAVES][64];
  int first, count, row_base, len;
  if (!cu_seqlens) {
    first = z * num_q_tiles;
    count = num_q_tiles;
    row_base = z * seqlen;
    len = seqlen;
  } else {
    // the 32-row tiles of the sequences before z, counted 64 at a time by wave 0
    if (wave == 0) {
      int before = 0;
      for (int z0 = 0; z0 < z; z0 += 64) {
        const int zz = z0 + lane;
        const int n = zz < z ? max(cu_seqlens[zz + 1] - cu_seqlens[zz], 0) : 0;
        int t = (n + 31) / 32;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
        before += t;
      }
      if (lane == 0) s_first = before;
    }
    __syncthreads();
    first = s_first;
    row_base = cu_seqlens[z];
    len = max(cu_seqlens[z + 1] - row_base, 0);
    count = (len + 31) / 32;
  }
  const int used = count - fold_tiles;   // slots past the fold row
  if (used <= 0 && !dk_out) return;      // block-uniform
  const int per = 2 * prefix * FOLD_D;   // floats per slot (a multiple of 4)
  const int e = (blockIdx.z * 64 + lane) * VEC;
  const float* src = fold_part + ((size_t)kvh * ds_stride + first) * per + e;
  T t = V::zero();
  if (e < per) {
    for (int c0 = wave; c0 < used; c0 += FOLD_ADD_LOADS * FOLD_ADD_WAVES) {
      T v[FOLD_ADD_LOADS];
#pragma unroll
      for (int u = 0; u < FOLD_ADD_LOADS; ++u) {
        const int c = c0 + u * FOLD_ADD_WAVES;
        v[u] = *(const T*)(src + (size_t)min(c, used - 1) * per);
      }
#pragma unroll
      for (int u = 0; u < FOLD_ADD_LOADS; ++u)
        if (c0 + u * FOLD_ADD_WAVES < used) V::add(t, v[u]);
    }
  }
  red[wave][lane] = t;
  __syncthreads();
  if (wave == 0 && e < per) {
    T u = V::zero();
#pragma unroll
    for (int w = 0; w < FOLD_ADD_WAVES; ++w) V::add(u, red[w][lane]);
    const int part = e / (prefix * FOLD_D);      // 0: dK, 1: dV
    const int rem = e - part * prefix * FOLD_D;  // key * D + d
    const int key = rem / FOLD_D, d = rem - key * FOLD_D;
    if (key < len) {
      const size_t i = ((size_t)(row_base + key) * heads_kv + kvh) * FOLD_D + d;
      T* acc = (T*)((part == 0 ? dk_acc : dv_acc) + i);
      T x = *acc;
      V::add(x, u);
      if (dk_out) V::store_bf16((part == 0 ? dk_out : dv_out) + i, x, part == 0 ? scale : 1.0f);
      else *acc = x;
    }
  }
}

}  // namespace

// FINISH phase of the prefix fold (head dim 64): fold_tiles = fold_row / 32 of
// each sequence's slots are skipped; dk, dv non-null when the dK/dV kernel
// stored the other rows as bf16 itself.
hipError_t launch_prefix_fold_add(const float* fold_part, float* dk_acc, float* dv_acc,
                                  bf16* dk, bf16* dv, float scale, const int* cu_seqlens,
                                  int batch, int seqlen, int heads_kv, int prefix, int ds_stride,
                                  long long fold_row, hipStream_t stream) {
  if (batch == 0 || seqlen == 0) return hipSuccess;
  if (prefix <= 0 || prefix > 32 || fold_row % 32 != 0) return hipErrorInvalidValue;
  const long long fold_tiles = fold_row / 32;
  const int num_q_tiles = (seqlen + 31) / 32;
  // no row past the fold row: nothing to add (but rows to convert when direct)
  if (fold_tiles >= num_q_tiles && !dk) return hipSuccess;
  const int ft = (int)(fold_tiles < num_q_tiles ? fold_tiles : num_q_tiles);
  // four values per lane when that still leaves a workgroup per CU or more
  const int per = 2 * prefix * FOLD_D;
  if ((long long)batch * heads_kv * ((per + 255) / 256) >= 256) {
    hipLaunchKernelGGL(sinkattn_prefix_fold_add<4>, dim3(batch, heads_kv, (per + 255) / 256),
                       dim3(FOLD_ADD_WAVES * 64), 0, stream, fold_part, dk_acc, dv_acc, dk, dv,
                       scale, cu_seqlens, seqlen, heads_kv, prefix, ds_stride, num_q_tiles, ft);
  } else {
    hipLaunchKernelGGL(sinkattn_prefix_fold_add<1>, dim3(batch, heads_kv, (per + 63) / 64),
                       dim3(FOLD_ADD_WAVES * 64), 0, stream, fold_part, dk_acc, dv_acc, dk, dv,
                       scale, cu_seqlens, seqlen, heads_kv, prefix, ds_stride, num_q_tiles, ft);
  }
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sinkattn_zero_f32, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// fp32 row pass (D, L, dsinks); dsinks must be zero on entry.
hipError_t launch_bwd_pre(int head_dim, const float* o, const float* dout, const float* lse,
                          const float* sinks, const int* cu_seqlens, float* dsinks, float* d_ws,
                          float* l_ws, int batch, int seqlen, int rows_total, int heads_q,
                          int lse_head_stride, hipStream_t stream) {
  PreArgs a;
  a.o = o; a.dout = dout; a.lse = lse; a.sinks = sinks; a.cu_seqlens = cu_seqlens;
  a.dsinks = dsinks; a.d_ws = d_ws; a.l_ws = l_ws;
  a.seqlen = seqlen; a.heads_q = heads_q; a.rows_total = rows_total;
  a.lse_head_stride = lse_head_stride;
  if (seqlen == 0 || batch == 0) return hipSuccess;
  if (head_dim != 32 && head_dim != 64) return hipErrorInvalidValue;
  if (256 % heads_q == 0) {
    const int rows_per_pass = 256 / heads_q;
    const int passes = 4;
    dim3 grid((seqlen + rows_per_pass * passes - 1) / (rows_per_pass * passes), 1, batch);
    if (head_dim == 64)
      hipLaunchKernelGGL(sinkattn_bwd_pre_rows<64>, grid, dim3(256), 0, stream, a, passes);
    else
      hipLaunchKernelGGL(sinkattn_bwd_pre_rows<32>, grid, dim3(256), 0, stream, a, passes);
    return hipGetLastError();
  }
  a.rows_per_wave = 256;
  dim3 grid((seqlen + a.rows_per_wave - 1) / a.rows_per_wave, (heads_q + 3) / 4, batch);
  if (head_dim == 64)
    hipLaunchKernelGGL(sinkattn_bwd_pre<64>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(sinkattn_bwd_pre<32>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// bf16 FINISH phase: dk, dv from the fp32 accumulators (n_kv floats each),
// and dsinks[h] = sum of ds_part[h * ds_stride + 0 .. ds_used) for h < heads.
hipError_t launch_convert(const float* dk_acc, const float* dv_acc, bf16* dk, bf16* dv,
                          long long n_kv, float scale, const float* ds_part, int ds_used,
                          int ds_stride, int heads, float* dsinks, hipStream_t stream) {
  const long long n4 = n_kv / 4;
  if (n4 == 0 && heads <= 0) return hipSuccess;
  long long blocks = (n4 + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < heads) blocks = heads;
  hipLaunchKernelGGL(sinkattn_convert, dim3((unsigned)blocks), dim3(256), 0, stream, dk_acc,
                     dv_acc, dk, dv, n4, scale, ds_part, ds_used, ds_stride, heads, dsinks);
  return hipGetLastError();
}
