// Device-side building blocks for the gfx950 (CDNA4) kernels: vector types,
// MFMA wrappers, LDS transpose reads, cross-half-wave reductions.
//
// MFMA lane layouts (v_mfma_f32_32x32x16_bf16, wave64), checked on the device:
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) + j, j = 0..7
//   B (16 x 32): lane l holds col l%32, k = 8*(l/32) + j
//   C (32 x 32): lane l holds col l%32, rows 8*(i/4) + 4*(l/32) + i%4, i = 0..15
// Any permutation of k applied identically to A and B leaves C unchanged,
// which is how probabilities produced in C layout feed the next MFMA directly.
//
// ds_read_tr16_b64 (LDS transpose read), per 16-lane group: lane i receives,
// as element j (0..3), the 16-bit value at (address of lane 4j + i/4) + i%4.
// Pointing lane L at row r0 + L/4, column c0 + 4*(L%4) of a row-major [row][col]
// bf16 array makes lane i hold column c0 + i, rows r0 .. r0+3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define SA_LOG2E 1.4426950408889634f
#define SA_LN2 0.6931471805599453f

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposed 4 x 16-bit read from LDS (see header comment).  The builtin's
// memory operand carries no alias information of its own, and without any the
// compiler makes each such read wait (s_waitcnt vmcnt(0)) for every LDS load
// DMA in flight -- including the prefetch of the next tile into the other
// buffer, which then overlaps nothing.  A restrict parameter gives the inlined
// read an alias scope, so only the kernels' own explicit waits remain (every
// tile is waited for and published with a barrier before it is read).
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* __restrict__ p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Reduce across the two 32-lane halves of the wave (lanes l and l^32).
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 8 fp32 -> 8 bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  f32x2 p0 = {a0, a1}, p1 = {a2, a3}, p2 = {a4, a5}, p3 = {a6, a7};
  bf16x2 b0 = __builtin_convertvector(p0, bf16x2);
  bf16x2 b1 = __builtin_convertvector(p1, bf16x2);
  bf16x2 b2 = __builtin_convertvector(p2, bf16x2);
  bf16x2 b3 = __builtin_convertvector(p3, bf16x2);
  bf16x4 lo = __builtin_shufflevector(b0, b1, 0, 1, 2, 3);
  bf16x4 hi = __builtin_shufflevector(b2, b3, 0, 1, 2, 3);
  return cat8(lo, hi);
}
// 8 fp32 -> 8 fp16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ f16x8 to_f16x8(float a0, float a1, float a2, float a3, float a4,
                                          float a5, float a6, float a7) {
  f32x2 p0 = {a0, a1}, p1 = {a2, a3}, p2 = {a4, a5}, p3 = {a6, a7};
  f16x2 b0 = __builtin_convertvector(p0, f16x2);
  f16x2 b1 = __builtin_convertvector(p1, f16x2);
  f16x2 b2 = __builtin_convertvector(p2, f16x2);
  f16x2 b3 = __builtin_convertvector(p3, f16x2);
  f16x4 lo = __builtin_shufflevector(b0, b1, 0, 1, 2, 3);
  f16x4 hi = __builtin_shufflevector(b2, b3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 to_bf16x4(float a0, float a1, float a2, float a3) {
  f32x2 p0 = {a0, a1}, p1 = {a2, a3};
  bf16x2 b0 = __builtin_convertvector(p0, bf16x2);
  bf16x2 b1 = __builtin_convertvector(p1, bf16x2);
  return __builtin_shufflevector(b0, b1, 0, 1, 2, 3);
}

// The mask M[q,k] = 1[k<=q] AND 1[q-k<=w OR k<p] as one unsigned compare:
// with d = q - k (no overflow for positions in [0, 2^31)), M holds iff
// (unsigned)d <= lim where lim = INT32_MAX for a prefix key (k < p) and w
// otherwise -- a negative d wraps above every lim since w <= INT32_MAX.
__device__ __forceinline__ bool sa_vis(int d, int lim) { return (unsigned)d <= (unsigned)lim; }
constexpr int SA_LIM_PREFIX = 0x7fffffff;
// Keep v in a register as computed: stops the compiler from re-associating
// base - c_i and hoisting one loop-invariant register per element.
__device__ __forceinline__ int sa_opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Pin a value to where it is computed: instruction selection otherwise places
// side-effect-free arithmetic next to its first use, whatever sched_barrier
// fences stand in between.
__device__ __forceinline__ float sa_pin(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Scheduling fence that memory operations also respect: sched_barrier alone
// acts in the machine scheduler only, after instruction selection may already
// have moved side-effect-free LDS loads across it; the empty asm with a
// memory clobber keeps them on their side (and emits no instruction).
__device__ __forceinline__ void sa_mem_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Mask one lane's 16 C-layout elements of a 32-key block when the lane holds
// one query and element i holds key kr + c_i, c_i = 8*(i/4) + i%4, so that
// q - k = base - c_i.  Hidden elements become -inf.  GENERAL: the block may
// hold prefix keys (those with c_i < pb = p - kr); otherwise lim = w for all.
template <bool GENERAL>
__device__ __forceinline__ void mask_query_lane(f32x16& st, int base, int pb, int window) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 8 * (i >> 2) + (i & 3);
    const int lim = (GENERAL && c < pb) ? SA_LIM_PREFIX : window;
    st[i] = sa_vis(base - c, lim) ? st[i] : -INFINITY;
  }
}

// The cheapest exact form of the mask of the 32 x 32 block of rows
// [qs, qs + 31] (lane: row qs + l32) and keys [ks, ks + 31] (element i: key
// ks + 4g + c_i, c_i = 8*(i/4) + i%4), chosen from wave-uniform values
// (dq = qs - ks), with base = qs + l32 - kr, kr = ks + 4g:
//  * the window bound cannot bind (every key a prefix key, or no prefix key
//    and dq + 31 <= w): visible iff k <= q, i.e. c_i <= base   (UPPER);
//  * no key past its row (dq >= 31) and no prefix key: visible iff
//    q - k <= w, i.e. c_i >= base - w                          (LOWER);
//  * prefix keys mixed in, but every row past the window of the block's
//    other keys (dq > w + 31): visible iff k < p, i.e. c_i <= p - kr - 1
//                                                              (UPPER);
//  * otherwise the general predicate of mask_query_lane        (GENERAL).
// UPPER and LOWER cost one compare against a constant and one select per
// element.  *thr: the per-lane threshold of UPPER / LOWER.
enum { SA_MASK_UPPER = 1, SA_MASK_LOWER = 2, SA_MASK_GENERAL = 3 };
__device__ __forceinline__ int mask_form(int qs, int ks, int lane, int window, int prefix,
                                         int* thr) {
  const int dq = __builtin_amdgcn_readfirstlane(qs - ks);
  const int ku = __builtin_amdgcn_readfirstlane(ks);
  const int kr = ku + 4 * (lane >> 5);
  const int base = __builtin_amdgcn_readfirstlane(qs) + (lane & 31) - kr;
  const bool all_prefix = ku + 31 < prefix;
  const bool no_prefix = ku >= prefix;
  if (all_prefix || (no_prefix && dq <= window - 31)) {
    *thr = base;
    return SA_MASK_UPPER;
  }
  if (no_prefix && dq >= 31) {
    *thr = base - window;
    return SA_MASK_LOWER;
  }
  if (!no_prefix && dq - 31 > window) {
    *thr = prefix - kr - 1;
    return SA_MASK_UPPER;
  }
  *thr = 0;
  return SA_MASK_GENERAL;
}

// Mask the block's 16 elements of this lane to -inf in that form.
__device__ __forceinline__ void mask_query_block(f32x16& st, int qs, int ks, int lane, int window,
                                                 int prefix) {
  int thr;
  const int form = mask_form(qs, ks, lane, window, prefix, &thr);
  if (form == SA_MASK_GENERAL) {
    const int kr = ks + 4 * (lane >> 5);
    mask_query_lane<true>(st, sa_opaque(qs + (lane & 31) - kr), sa_opaque(prefix - kr), window);
    return;
  }
  const int th = sa_opaque(thr);
  if (form == SA_MASK_UPPER) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 8 * (i >> 2) + (i & 3);
      st[i] = c <= th ? st[i] : -INFINITY;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 8 * (i >> 2) + (i & 3);
      st[i] = c >= th ? st[i] : -INFINITY;
    }
  }
}

// Where a sequence lives in the packed/batched tensors.
struct SeqView {
  int row_base;  // first token row of the sequence in [B*T] or [N]
  int len;       // its length
  int lse_base;  // offset of (head 0, token 0) in the lse tensor, minus head stride
};

__device__ __forceinline__ SeqView seq_view(const int* cu_seqlens, int z, int seqlen, int heads_q) {
  SeqView s;
  if (cu_seqlens) {
    s.row_base = cu_seqlens[z];
    s.len = cu_seqlens[z + 1] - s.row_base;
    s.lse_base = s.row_base;            // lse [Hq, N]: h * N + row
  } else {
    s.row_base = z * seqlen;
    s.len = seqlen;
    s.lse_base = z * heads_q * seqlen;  // lse [B, Hq, T]: (z*Hq + h)*T + t
  }
  return s;
}

// The (sequence, query tile) of this workgroup in a launch of a
// query-stationary kernel with tiles of bq rows.  Fixed length: sequence =
// grid y, tile = num_q_tiles - 1 - grid z (tiles from the last: longest rows
// first).  Packed sequences (cu_seqlens): grid y = 1 and grid z indexes the
// packed tiles sequence by sequence, each sequence's tiles from its last
// down; the host sizes grid z with sa_packed_tiles_bound, and an index past
// the last tile returns false.  The lanes of a wave scan 64 sequences at a
// time (tile counts, prefix sum); every lane gets the same, wave-uniform result.
__device__ __forceinline__ bool launch_tile(const int* cu_seqlens, int batch, int num_q_tiles,
                                            int bq, int* z_out, int* qt_out) {
  if (!cu_seqlens) {
    *z_out = blockIdx.y;
    *qt_out = num_q_tiles - 1 - (int)blockIdx.z;
    return true;
  }
  const int lane = threadIdx.x & 63;
  int t = blockIdx.z;
  for (int z0 = 0; z0 < batch; z0 += 64) {
    const int z = z0 + lane;
    const int n = z < batch ? max(cu_seqlens[z + 1] - cu_seqlens[z], 0) : 0;
    const int nt = (n + bq - 1) / bq;
    int incl = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    // wave-uniform (readfirstlane), so the loop's branches are uniform too
    const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    if (t < total) {
      const int L = __builtin_ctzll(__ballot(incl > t));   // first sequence past index t
      const int before = __shfl(incl - nt, L);
      const int ntl = __shfl(nt, L);
      *z_out = __builtin_amdgcn_readfirstlane(z0 + L);
      *qt_out = __builtin_amdgcn_readfirstlane(ntl - 1 - (t - before));
      return true;
    }
    t -= total;
  }
  return false;
}

// ---------------------------------------------------------------------------
// LDS tiles of R rows x 64 bf16 (128 B per row, no padding).  Each row's eight
// 16-byte chunks are stored XOR-swizzled by the row index:
//   physical chunk = chunk ^ (2*(r%4) + (r/4)%2) ^ (2*((r/8)%2))
// which keeps both access patterns the kernels use free of bank conflicts
// (checked against 32- and 64-bank models): 16-byte reads of one chunk by
// 8 or 16 consecutive rows (MFMA operands with the head dim along k), and
// ds_read_tr16_b64 reads of 4 consecutive rows x 32 bytes (operands with the
// row index along k).
__device__ __forceinline__ int tile_swz(int r) {
  return (((r & 3) << 1) | ((r >> 2) & 1)) ^ ((r >> 2) & 2);
}
// element offset of (row r, column c); c's low 3 bits stay inside the chunk
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * 64 + ((((c >> 3) ^ tile_swz(r))) << 3) + (c & 7);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// Operand addresses in a swizzled tile from one per-lane base each.  In bytes
// from the tile start (checked exhaustively on the host):
//   row reads, head-dim chunk 2s + g of row r:   tile_row_base(r, g) ^ (32 s)
//   transpose reads at (r0, 32 db + c), r0 % 16 < 8, c < 32:
//       row r0:      tile_tr_base(r0, c) ^ (64 db)
//       row r0 + 8: (tile_tr_base(r0, c) ^ (64 db) ^ 32) + 1024
//   16 m rows further down (either pattern): + 2048 m.
// The tile's LDS address is a multiple of 128, so adding it before the XOR
// keeps this exact: an operand address costs at most one v_xor, and row and
// tile offsets fold into the instruction's immediate offset.
__device__ __forceinline__ int tile_row_base(int r, int g) {
  return r * 128 + ((g ^ tile_swz(r)) << 4);
}
__device__ __forceinline__ int tile_tr_base(int r0, int c) {
  return r0 * 128 + (((c >> 3) ^ tile_swz(r0)) << 4) + 2 * (c & 7);
}
// LDS byte address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const lds_void*)p;
}
// 16-byte and transposed 4 x 16-bit reads at an LDS byte address (restrict:
// see lds_read_tr4)
__device__ __forceinline__ bf16x8 lds_read8_p(const lds_bf16x8* __restrict__ p) { return *p; }
__device__ __forceinline__ bf16x8 lds_read8(uint32_t a) {
  return lds_read8_p((const lds_bf16x8*)(size_t)a);
}
__device__ __forceinline__ bf16x4 lds_read_tr4_p(lds_s16x4* __restrict__ p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}
__device__ __forceinline__ bf16x4 lds_read_tr4_at(uint32_t a) {
  return lds_read_tr4_p((lds_s16x4*)(size_t)a);
}

// Copy a ROWS x 64 bf16 tile from global memory straight into a swizzled LDS
// tile with buffer_load_dwordx4 ... lds (lane i's 16 bytes land at the
// block's LDS address + 16 i, so one instruction fills 8 rows; no VGPRs hold
// the data).  Lane i of an 8-row block reads tile row i/8 of the block and
// fetches the global chunk that belongs at physical chunk i%8 of that row.
// Rows at or past `nvalid` repeat row nvalid-1 (nvalid >= 1): callers mask
// those rows out of every result.  Completion is tracked by vmcnt:
// s_waitcnt vmcnt(0) before the barrier that publishes the tile.
//
// The address is split in two: a uniform part (tile base plus the block's
// first row, clamped to the last valid row) in the buffer descriptor, and a
// 32-bit lane offset (the lane's row, clamped the same way, plus its chunk).
// Lane constants (checked against the per-lane formula on the host for every
// lane, block and row count): the chunk offset for an even block is
// 16 * ((i%8) ^ tile_swz(i/8)), for an odd block that XOR 32 (the swizzle of
// a row r + 8 is that of r XOR 2).
//
// The buffer form rather than global_load_lds: the compiler takes a pending
// global_load_lds for a flat access to both memories and then makes every
// later wait a wait for all loads (vmcnt(0), lgkmcnt(0)); with the buffer
// form it keeps per-instruction counts, so LDS reads of the other tile
// overlap the MFMAs that consume them.  The descriptor covers every byte
// (num_records 2^32 - 1; offsets stay within 8 rows).
struct TileLane {
  int row_off;     // (lane / 8) * row_bytes
  int chunk_off;   // 16 * ((lane % 8) ^ tile_swz(lane / 8))
};
__device__ __forceinline__ TileLane tile_lane(int lane, int row_bytes) {
  TileLane t;
  t.row_off = (lane >> 3) * row_bytes;
  t.chunk_off = ((lane & 7) ^ tile_swz(lane >> 3)) << 4;
  return t;
}
template <int ROWS, int WAVES>
__device__ __forceinline__ void tile_load_lds_lane(bf16* lds_tile, const bf16* gbase, int row_bytes,
                                                   int nvalid, int wave, const TileLane& tl) {
  constexpr int PER_WAVE = ROWS / (8 * WAVES);
  static_assert(PER_WAVE * 8 * WAVES == ROWS, "tile rows must split into 8-row blocks per wave");
  const int w = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int blk = w * PER_WAVE + j;
    const int r0 = min(blk * 8, nvalid - 1);
    const int lim = max(nvalid - 1 - blk * 8, 0) * row_bytes;
    const uint32_t off = (uint32_t)(min(tl.row_off, lim) + (tl.chunk_off ^ ((blk & 1) << 5)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)gbase + (size_t)r0 * row_bytes), (short)0, -1, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_tile + blk * 512), 16, off, 0, 0, 0);
  }
}

// wait for every outstanding memory operation of this wave (vmcnt, lgkmcnt = 0)
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }
