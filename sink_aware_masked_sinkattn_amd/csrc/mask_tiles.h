// Tile-level view of the sink-aware mask
//   M[q,k] = 1[k <= q] AND 1[q - k <= w OR k < p]
// ("Efficient Reinforcement Learning for Long-Horizon Tool-Use Agentic Tasks",
// summary page, sink-aware FlexAttention paragraph).  Positions are local to
// one sequence.  Host- and device-callable, integer only.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define SA_HD __host__ __device__ __forceinline__
#else
#define SA_HD static inline
#endif

enum { SA_TILE_SKIP = 0, SA_TILE_FULL = 1, SA_TILE_PARTIAL = 2 };

// Element predicate.  w may be INT32_MAX; q - k never overflows for
// non-negative positions.
SA_HD bool sa_visible(int q, int k, int w, int p) {
  return (k <= q) && ((q - k <= w) || (k < p));
}

SA_HD int sa_max(int a, int b) { return a > b ? a : b; }
SA_HD int sa_min(int a, int b) { return a < b ? a : b; }

// Classify the block of query rows [q0, q1] x key columns [k0, k1]
// (inclusive, q0 <= q1, k0 <= k1).
//  skip:  no key is causal for any row (k0 > q1), or every key is past the
//         prefix and even the closest pair (q0, k1) is beyond the window;
//  full:  every key is causal for every row (k1 <= q0) and every key that is
//         not a prefix key lies within the window of the farthest row q1;
//  partial otherwise (the element predicate decides).
SA_HD int sa_tile_class(int q0, int q1, int k0, int k1, int w, int p) {
  if (k0 > q1) return SA_TILE_SKIP;
  if (k0 >= p && q0 - k1 > w) return SA_TILE_SKIP;
  if (k1 <= q0) {
    if (k1 < p) return SA_TILE_FULL;
    if (q1 - sa_max(k0, p) <= w) return SA_TILE_FULL;
  }
  return SA_TILE_PARTIAL;
}

// Key tiles (width bk) that query rows [q0, q1] must visit: the prefix tiles
// [0, ceil(min(p, q1+1)/bk)) and the window tiles
// [floor(max(0, q0-w)/bk), floor(q1/bk)], merged when they touch.  A tile is
// listed iff it holds at least one visible pair, and at most once.
// Writes up to two half-open ranges to out[0..3]; returns their number.
SA_HD int sa_key_tile_segments(int q0, int q1, int w, int p, int bk, int* out) {
  const long long wlo = (long long)q0 - (long long)w;
  const int win_begin = (int)((wlo > 0 ? wlo : 0) / bk);
  const int win_end = q1 / bk + 1;
  const int pre_keys = sa_min(p, q1 + 1);
  const int pre_end = (pre_keys + bk - 1) / bk;
  if (pre_end <= 0 || pre_end >= win_begin) {
    out[0] = pre_end > 0 ? 0 : win_begin;
    out[1] = win_end;
    out[2] = out[3] = 0;
    return 1;
  }
  out[0] = 0;
  out[1] = pre_end;
  out[2] = win_begin;
  out[3] = win_end;
  return 2;
}

// Query tiles of bq rows over a batch of packed sequences (total_tokens rows,
// each sequence at most seqlen): at most batch * ceil(seqlen / bq), and at
// most floor((total_tokens + batch * (bq - 1)) / bq) since
// sum ceil(len / bq) <= sum (len + bq - 1) / bq.  Sizes the grids of the
// query-stationary kernels without reading the lengths on the host.
SA_HD int sa_packed_tiles_bound(int batch, int seqlen, int total_tokens, int bq) {
  const long long per_seq = (long long)batch * ((seqlen + bq - 1) / bq);
  const long long by_tokens = ((long long)total_tokens + (long long)batch * (bq - 1)) / bq;
  return (int)(per_seq < by_tokens ? per_seq : by_tokens);
}

// Query rows that key columns [k0, k1] are visible to, within a sequence of
// n tokens: rows [k0, qmax] with qmax = n-1 if any key is a prefix key, else
// min(n-1, k1 + w).  Returns false if no row sees them.
SA_HD bool sa_query_range(int k0, int k1, int n, int w, int p, int* qlo, int* qhi) {
  if (k0 >= n) return false;
  long long hi = (k0 < p) ? (long long)(n - 1) : (long long)k1 + (long long)w;
  if (hi > n - 1) hi = n - 1;
  *qlo = k0;
  *qhi = (int)hi;
  return *qlo <= *qhi;
}

// The prefix fold.  When it is on (prefix keys all in the first 32-key tile,
// resident-tile window dQ kernel), the rows of a key block holding prefix
// keys that lie past the first query tile boundary after the block's
// window, i.e. rows >= sa_prefix_fold_row(kb, w, bkw, bq), see only the
// block's prefix keys; the window dQ kernel adds their part of the prefix
// keys' dK and dV (it holds those rows and the prefix tile anyway), and the
// dK/dV kernel's work for the block stops before them.
SA_HD long long sa_prefix_fold_row(int kb, int w, int bkw, int bq) {
  const long long last = (long long)kb * bkw + bkw - 1 + (long long)w;   // last row of the window
  return (last / bq + 1) * bq;
}

// Query rows [lo, hi] of the dK/dV kernel's work for key block kb of a
// sequence of n tokens (false if none): the rows that see it, cut at the fold
// row for blocks holding prefix keys when the fold is on.
SA_HD bool sa_dkdv_query_range(int kb, int n, int w, int p, int bq, int bkw, bool fold, int* lo,
                               int* hi) {
  const int k0 = kb * bkw;
  if (!sa_query_range(k0, sa_min(k0 + bkw - 1, n - 1), n, w, p, lo, hi)) return false;
  if (fold && k0 < p) {
    const long long cut = sa_prefix_fold_row(kb, w, bkw, bq) - 1;
    if (cut < *hi) *hi = (int)cut;
  }
  return true;
}

// Work units of the dK/dV backward: key block kb (keys [kb*bkw, kb*bkw+bkw))
// of a sequence of n tokens is paired with every (query tile of bq rows,
// query head of the group) in its query range; those iterations are cut into
// chunks of 2^chunk_shift.  Returns the number of chunks (0 if no row sees
// the block).  Host and kernel use this same count to size and walk the flat
// work list.
SA_HD int sa_dkdv_block_chunks(int kb, int n, int w, int p, int group, int bq, int bkw,
                               int chunk_shift, bool fold) {
  int lo, hi;
  if (!sa_dkdv_query_range(kb, n, w, p, bq, bkw, fold, &lo, &hi)) return 0;
  const int n_iter = (hi / bq - lo / bq + 1) * group;
  return (n_iter + (1 << chunk_shift) - 1) >> chunk_shift;
}

// Decode: the keys the query at position n - 1 of a sequence of n tokens sees
// are the prefix [0, min(p, n)) and the window [max(0, n - 1 - w), n), merged
// when they touch.  Writes the two ranges to out[0..3] (begin0, end0, begin1,
// end1; the first is empty when there is no prefix, the second when merged)
// and returns the number of chunks of kw keys, each range cut from its start.
SA_HD int sa_decode_ranges(int n, int w, int p, int kw, int* out) {
  if (n <= 0) {
    out[0] = out[1] = out[2] = out[3] = 0;
    return 0;
  }
  const int pe = sa_min(p, n);
  const long long wbl = (long long)(n - 1) - (long long)w;
  const int wb = wbl > 0 ? (int)wbl : 0;
  if (pe >= wb) {
    out[0] = 0; out[1] = n; out[2] = n; out[3] = n;
    return (n + kw - 1) / kw;
  }
  out[0] = 0; out[1] = pe; out[2] = wb; out[3] = n;
  return (pe + kw - 1) / kw + (n - wb + kw - 1) / kw;
}

// Keys [k0, k1) of chunk c (0 <= c < the count above) of the ranges r.
SA_HD void sa_decode_chunk(const int* r, int kw, int c, int* k0, int* k1) {
  const int ca = (r[1] - r[0] + kw - 1) / kw;
  if (c < ca) {
    *k0 = r[0] + c * kw;
    *k1 = sa_min(*k0 + kw, r[1]);
  } else {
    *k0 = r[2] + (c - ca) * kw;
    *k1 = sa_min(*k0 + kw, r[3]);
  }
}

// Upper bound of the chunk count over every n <= t_max: the prefix range
// holds at most min(p, t_max) keys and the window range min(w + 1, t_max);
// when the two merge, ceil((a + b) / kw) <= ceil(a / kw) + ceil(b / kw).
SA_HD int sa_decode_max_chunks(int t_max, int w, int p, int kw) {
  const int pw = sa_min(p, t_max);
  const long long win = (long long)w + 1 < (long long)t_max ? (long long)w + 1 : t_max;
  return (pw + kw - 1) / kw + (int)((win + kw - 1) / kw);
}
