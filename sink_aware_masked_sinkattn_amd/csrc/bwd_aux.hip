// Backward helpers around the dK/dV and dQ kernels: the row preprocessing
// pass of the fp32 path (the bf16 dQ kernel computes the same statistics for
// its own rows) and the dK/dV conversion pass.  Both are HBM-bound streaming
// kernels.
//
// Preprocessing, per (row i, query head h) -- the sink gradient of "GPT-OSS
// Agentic RL training: a practical retrospective" (FlashAttention v3
// implementation section), written out with the sink as a zero-value key
// (arXiv 2608.10357, section 5):
//   D_i = sum_c dO_ic O_ic
//   L_i = logaddexp(l_i, s_h)                (sink-inclusive log-normaliser)
//   ds_h -= exp(s_h - L_i) D_i               (summed over all rows)
// D and L go to the workspace for the main kernel.  The ds_h partial sums of
// a wave are reduced with cross-lane shuffles, then added with one float
// atomic per wave.  The same pass zeroes the fp32 dK and dV accumulators
// (from the first query head of each group), so no separate memset is needed.
#include "common.h"

namespace {

// 16 bytes of a row per lane: lanes-per-row = D / (16 / sizeof(T)).
template <typename T, int D>
struct RowSplit {
  static constexpr int kElems = 16 / (int)sizeof(T);
  static constexpr int kLanesPerRow = D / kElems;
  static constexpr int kRowsPerPass = 64 / kLanesPerRow;
};

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

struct PreArgs {
  const void* o;
  const void* dout;
  const float* lse;
  const float* sinks;
  const int* cu_seqlens;
  float* dsinks;
  float* d_ws;        // [Hq, rows] : D_i
  float* l_ws;        // [Hq, rows] : L_i (natural log)
  float* dk_acc;      // [rows, Hkv, D] fp32, zeroed here (may be null)
  float* dv_acc;
  int seqlen, heads_q, heads_kv, group, rows_total;
  int lse_head_stride;
  int rows_per_wave;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void sinkattn_bwd_pre(PreArgs a) {
  using RS = RowSplit<T, D>;
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
  const T* o = (const T*)a.o;
  const T* dout = (const T*)a.dout;
  const bool zero_kv = (a.dk_acc != nullptr) && (h % a.group == 0);
  const int kvh = h / a.group;
  float ds_part = 0.0f;
  for (int r0 = r_begin; r0 < r_end; r0 += RS::kRowsPerPass) {
    const int r = r0 + rsub;
    float dot = 0.0f;
    const size_t row = (size_t)sv.row_base + r;
    if (r < r_end) {
      const size_t off = (row * a.heads_q + h) * D + sub * RS::kElems;
      const T* po = o + off;
      const T* pd = dout + off;
#pragma unroll
      for (int e = 0; e < RS::kElems; ++e) dot += to_f32(po[e]) * to_f32(pd[e]);
      if (zero_kv) {
        const size_t koff = (row * a.heads_kv + kvh) * D + sub * RS::kElems;
        float4* pk = (float4*)(a.dk_acc + koff);
        float4* pv = (float4*)(a.dv_acc + koff);
#pragma unroll
        for (int e = 0; e < RS::kElems / 4; ++e) {
          pk[e] = make_float4(0.f, 0.f, 0.f, 0.f);
          pv[e] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
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
template <typename T, int D>
__global__ __launch_bounds__(256) void sinkattn_bwd_pre_rows(PreArgs a, int passes) {
  constexpr int kVec = 16 / (int)sizeof(T);          // elements per 16-byte load
  constexpr int kLoads = D / kVec;
  __shared__ float red[256];
  const int t = threadIdx.x;
  const int h = t % a.heads_q;
  const int rows_per_pass = 256 / a.heads_q;
  const int z = blockIdx.z;
  const SeqView sv = seq_view(a.cu_seqlens, z, a.seqlen, a.heads_q);
  const int r_begin = blockIdx.x * rows_per_pass * passes + t / a.heads_q;
  const float s = a.sinks[h];
  const bool zero_kv = (a.dk_acc != nullptr) && (h % a.group == 0);
  const int kvh = h / a.group;
  float ds_part = 0.0f;
  for (int k = 0; k < passes; ++k) {
    const int r = r_begin + k * rows_per_pass;
    if (r >= sv.len) break;
    const size_t row = (size_t)sv.row_base + r;
    const size_t off = (row * a.heads_q + h) * D;
    uint4 ov[kLoads], dv[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      ov[j] = ((const uint4*)((const T*)a.o + off))[j];
      dv[j] = ((const uint4*)((const T*)a.dout + off))[j];
    }
    float dot = 0.0f;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const T* po = (const T*)&ov[j];
      const T* pd = (const T*)&dv[j];
#pragma unroll
      for (int e = 0; e < kVec; ++e) dot = fmaf(to_f32(po[e]), to_f32(pd[e]), dot);
    }
    if (zero_kv) {
      float4* pk = (float4*)(a.dk_acc + (row * a.heads_kv + kvh) * D);
      float4* pv = (float4*)(a.dv_acc + (row * a.heads_kv + kvh) * D);
#pragma unroll
      for (int j = 0; j < D / 4; ++j) {
        pk[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        pv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
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

// p[0, 4*n4) = 0, 16 bytes per store, grid-stride
__global__ __launch_bounds__(256) void sinkattn_zero_f32x4(float4* p, long long n4) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// fp32 dK / dV accumulators -> output dtype, with the softmax scale folded
// into dK here (the dK/dV kernel accumulates dS^T Q unscaled).
template <typename T>
__device__ __forceinline__ void store4(T* dst, float4 v);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* dst, float4 v) {
  *(bf16x4*)dst = to_bf16x4(v.x, v.y, v.z, v.w);
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float4 v) {
  *(float4*)dst = v;
}

template <typename T>
__global__ __launch_bounds__(256) void sinkattn_convert(const float* dk_acc, const float* dv_acc,
                                                        T* dk, T* dv, long long n_kv4, float scale,
                                                        const float* ds_part, int ds_used,
                                                        int ds_stride, int heads, float* dsinks) {
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
    float4 x = ((const float4*)dk_acc)[i];
    x.x *= scale; x.y *= scale; x.z *= scale; x.w *= scale;
    store4<T>(dk + 4 * i, x);
    store4<T>(dv + 4 * i, ((const float4*)dv_acc)[i]);
  }
}

}  // namespace

hipError_t launch_zero_f32(float* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sinkattn_zero_f32, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// Clears n floats at p (p 16-byte aligned, n a multiple of 4).
hipError_t launch_zero_f32_vec(float* p, long long n, hipStream_t stream) {
  const long long n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  long long blocks = (n4 + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;
  hipLaunchKernelGGL(sinkattn_zero_f32x4, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (float4*)p, n4);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(int dtype_is_f32, int head_dim, const void* o, const void* dout,
                          const float* lse, const float* sinks, const int* cu_seqlens,
                          float* dsinks, float* d_ws, float* l_ws, float* dk_acc, float* dv_acc,
                          int batch, int seqlen, int rows_total, int heads_q, int heads_kv,
                          int lse_head_stride, hipStream_t stream) {
  PreArgs a;
  a.o = o; a.dout = dout; a.lse = lse; a.sinks = sinks; a.cu_seqlens = cu_seqlens;
  a.dsinks = dsinks; a.d_ws = d_ws; a.l_ws = l_ws;
  a.dk_acc = dk_acc; a.dv_acc = dv_acc;
  a.seqlen = seqlen; a.heads_q = heads_q; a.heads_kv = heads_kv;
  a.group = heads_q / heads_kv; a.rows_total = rows_total;
  a.lse_head_stride = lse_head_stride;
  if (seqlen == 0 || batch == 0) return hipSuccess;
  if (256 % heads_q == 0) {
    const int rows_per_pass = 256 / heads_q;
    const int passes = 4;
    dim3 grid((seqlen + rows_per_pass * passes - 1) / (rows_per_pass * passes), 1, batch);
    if (dtype_is_f32 && head_dim == 64) {
      hipLaunchKernelGGL((sinkattn_bwd_pre_rows<float, 64>), grid, dim3(256), 0, stream, a, passes);
    } else if (dtype_is_f32 && head_dim == 32) {
      hipLaunchKernelGGL((sinkattn_bwd_pre_rows<float, 32>), grid, dim3(256), 0, stream, a, passes);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  a.rows_per_wave = 256;
  dim3 grid((seqlen + a.rows_per_wave - 1) / a.rows_per_wave, (heads_q + 3) / 4, batch);
  if (dtype_is_f32 && head_dim == 64) {
    hipLaunchKernelGGL((sinkattn_bwd_pre<float, 64>), grid, dim3(256), 0, stream, a);
  } else if (dtype_is_f32 && head_dim == 32) {
    hipLaunchKernelGGL((sinkattn_bwd_pre<float, 32>), grid, dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// heads > 0: also dsinks[h] = sum of ds_part[h * ds_stride + 0 .. ds_used).
hipError_t launch_convert(int dtype_is_f32, const float* dk_acc, const float* dv_acc, void* dk,
                          void* dv, long long n_kv, float scale, const float* ds_part,
                          int ds_used, int ds_stride, int heads, float* dsinks,
                          hipStream_t stream) {
  const long long n4 = n_kv / 4;
  if (n4 == 0 && heads <= 0) return hipSuccess;
  long long blocks = (n4 + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < heads) blocks = heads;
  if (dtype_is_f32) {
    hipLaunchKernelGGL(sinkattn_convert<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       dk_acc, dv_acc, (float*)dk, (float*)dv, n4, scale, ds_part, ds_used,
                       ds_stride, heads, dsinks);
  } else {
    hipLaunchKernelGGL(sinkattn_convert<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       dk_acc, dv_acc, (bf16*)dk, (bf16*)dv, n4, scale, ds_part, ds_used,
                       ds_stride, heads, dsinks);
  }
  return hipGetLastError();
}
