// gfx950 kernels of the speculative-decoding verification step.
//
// One call is a short chain of launches on the caller's stream, with no host
// synchronisation and no cross-workgroup signalling inside a launch:
//   k_stream        the one pass over every logit the mode reads: one
//                   workgroup per tile of a row (16-byte non-temporal loads,
//                   four groups in flight per lane) leaves a small partial
//                   per tile in the workspace:
//                     ARGMAX   max + lowest index       (greedy, tree)
//                     STATS64  max + float64 sum of exp((l - max) / T)
//                                                         (plain and nucleus sampling)
//                     TOPK     the tile's top_k           (top-k sampling)
//   greedy / tree   k_greedy_final / k_tree_final: one workgroup per sequence
//   top-k           k_topk_rows (merge per row) -> k_topk_final (per sequence)
//   nucleus         k_topp_rows (exact cut per row) -> k_resid_s -> k_resid_final
//   plain sampling  k_resid_s (accept step + residual mass per segment)
//                   -> k_resid_final (draw per sequence)
//
// Every reduction that feeds an output is a fixed-order butterfly / tree, so
// repeated calls give bit-identical results.  Float64 carries every quantity
// that decides an integer output (row sums, accept test, nucleus cut,
// inverse CDF).

#include <float.h>
#include <limits.h>
#include <math.h>

#include <hip/hip_ext.h>

#include "sv_internal.h"

namespace sv {

#define DEV __device__ __forceinline__

constexpr int kWaves = kBlock / 64;
constexpr double kLog2e = 1.4426950408889634;
constexpr int kStatusInternal = 0x100;   // a numeric search did not settle (never expected)
constexpr int kTopkMax = 256;            // largest top_k

// ------------------------------------------------------------------ loads

typedef float vf4 __attribute__((ext_vector_type(4)));
typedef unsigned int vu4 __attribute__((ext_vector_type(4)));

template <typename T> struct Io;
template <> struct Io<float> {
  static DEV float at(const float* p, long i) { return p[i]; }
  static DEV void vec(const float* p, float v[kVec]) {
    const vf4* q = reinterpret_cast<const vf4*>(p);
    const vf4 a = __builtin_nontemporal_load(q);
    const vf4 b = __builtin_nontemporal_load(q + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct Io<uint16_t> {
  static DEV float at(const uint16_t* p, long i) { return __uint_as_float((uint32_t)p[i] << 16); }
  static DEV void vec(const uint16_t* p, float v[kVec]) {
    const vu4 q = __builtin_nontemporal_load(reinterpret_cast<const vu4*>(p));
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
    v[4] = __uint_as_float(q.z << 16); v[5] = __uint_as_float(q.z & 0xffff0000u);
    v[6] = __uint_as_float(q.w << 16); v[7] = __uint_as_float(q.w & 0xffff0000u);
  }
};

// Load the group of kVec logits starting at `pos` (< end).  Slots past `end`
// read as -inf.  Returns the number of real logits.
template <typename T>
DEV int load_group(const T* row, int pos, int end, int aligned, float v[kVec]) {
  int n = end - pos;
  if (n >= kVec && aligned) {
    Io<T>::vec(row + pos, v);
    return kVec;
  }
  n = n < kVec ? n : kVec;
#pragma unroll
  for (int e = 0; e < kVec; ++e) v[e] = (e < n) ? Io<T>::at(row, (long)pos + e) : -INFINITY;
  return n;
}

// ------------------------------------------------------------------ keys

// Order-preserving u32 of a float (-0 and +0 map to the same key).
DEV uint32_t ord_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
DEV float key_value(uint32_t key) {
  uint32_t b = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(b);
}
// (value desc, index asc) as one descending u64; 0 is never a real entry.
DEV uint64_t pack(float f, int idx) {
  return ((uint64_t)ord_key(f) << 32) | (uint64_t)(~(uint32_t)idx);
}
DEV int packed_idx(uint64_t pk) { return (int)(~(uint32_t)(pk & 0xffffffffu)); }
DEV float packed_val(uint64_t pk) { return key_value((uint32_t)(pk >> 32)); }

// ------------------------------------------------------------------ reductions

DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
DEV double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
DEV void wave_argmax(float& m, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o);
    int i2 = __shfl_xor(i, o);
    if (m2 > m || (m2 == m && i2 < i)) { m = m2; i = i2; }
  }
}

// Block-wide sum in a fixed order; every thread gets the same value.
DEV double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}
DEV float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}
DEV void block_argmax(float& m, int& i, float* redm, int* redi) {
  wave_argmax(m, i);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) { redm[w] = m; redi[w] = i; }
  __syncthreads();
  m = redm[0]; i = redi[0];
  for (int q = 1; q < kWaves; ++q)
    if (redm[q] > m || (redm[q] == m && redi[q] < i)) { m = redm[q]; i = redi[q]; }
  __syncthreads();
}

// Exclusive scan of one double per thread in thread order (fixed order).
// Returns the exclusive prefix; *total gets the block total.
DEV double block_exscan(double v, double* red, double* total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  double exl = __shfl_up(inc, 1);
  if (lane == 0) exl = 0.0;
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  double base = 0.0;
  for (int q = 0; q < w; ++q) base += red[q];
  double tot = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  *total = tot;
  return base + exl;
}
// Same for unsigned 64-bit integers (exact).
DEV unsigned long long block_exscan_u64(unsigned long long v, unsigned long long* red,
                                        unsigned long long* total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  unsigned long long inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    unsigned long long t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  unsigned long long base = 0;
  for (int q = 0; q < w; ++q) base += red[q];
  unsigned long long tot = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  *total = tot;
  return base + (inc - v);   // exact in integers
}

// Descending bitonic sort of n (power of two, <= LDS array size) u64 in LDS.
DEV void bitonic_desc(uint64_t* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int t = threadIdx.x; t < (n >> 1); t += kBlock) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = a[lo], y = a[hi];
        if ((x < y) == desc) { a[lo] = y; a[hi] = x; }
      }
    }
  }
  __syncthreads();
}

DEV int next_pow2(int n) {
  int p = 2;
  while (p < n) p <<= 1;
  return p;
}

// ------------------------------------------------------------------ rows

template <typename T>
DEV const T* row_ptr(const Params& p, int grow) {
  const int nt = p.B * p.rows_t;
  return grow < nt ? (const T*)p.target + (size_t)grow * p.V
                   : (const T*)p.draft + (size_t)(grow - nt) * p.V;
}

// Block-wide scan of a row for NaN or +inf (the exact test behind a probe).
template <typename T>
DEV bool row_has_nan_or_posinf(const T* row, int V) {
  int bad = 0;
  for (int i = threadIdx.x; i < V; i += kBlock) {
    const float v = Io<T>::at(row, i);
    bad |= (v != v) || (v == INFINITY);
  }
  return __syncthreads_or(bad) != 0;
}

// Combine the S tile partials of one row (one thread).
struct RowStat {
  float M;
  int amax;
  double Z;      // STATS mode: sum of exp((l - M) / T); NaN if a NaN was seen
  bool probe;    // a tile saw a non-finite value (ARGMAX / TOPK modes)
};
DEV RowStat combine_tiles(const Params& p, int grow, bool stats) {
  const TileStat* t = p.tiles + (size_t)grow * p.S;
  RowStat r;
  r.M = -INFINITY; r.amax = INT_MAX; r.Z = 0.0; r.probe = false;
  for (int s = 0; s < p.S; ++s) {
    const TileStat ts = t[s];
    if (ts.m > r.M) { r.M = ts.m; r.amax = ts.amax; }
    if (ts.s != ts.s) r.probe = true;
  }
  if (stats) {
    const double cd = kLog2e / p.T;
    double z = 0.0;
    for (int s = 0; s < p.S; ++s) {
      const TileStat ts = t[s];
      if (ts.m == -INFINITY) { z += ts.s; continue; }
      z += ts.s * exp2(((double)ts.m - (double)r.M) * cd);
    }
    r.Z = z;
  }
  return r;
}

// ================================================================== row / sequence indexing

DEV int seq_of_row(const Params& p, int grow) {
  const int nt = p.B * p.rows_t;
  return grow < nt ? grow / p.rows_t : (grow - nt) / p.rows_d;
}
DEV int trow(const Params& p, int b, int j) { return b * p.rows_t + j; }
DEV int drow(const Params& p, int b, int j) { return p.B * p.rows_t + b * p.rows_d + j; }

constexpr int kUnroll = 4;     // groups of kVec logits each thread has in flight
constexpr int kMaxTree = 1024;
constexpr int kMaxRows = 2 * 64 + 1;

// ================================================================== tile passes

template <typename T>
DEV void tile_argmax(const Params& p, const T* row, int start, int end, int ngroups, int tile) {
  __shared__ float redm[kWaves];
  __shared__ int redi[kWaves];
  float m = -INFINITY;
  int mi = INT_MAX;
  float probe = 0.f;
  for (int g0 = threadIdx.x; g0 < ngroups; g0 += kUnroll * kBlock) {
    float v[kUnroll][kVec];
    int nv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int g = g0 + u * kBlock;
      if (g < ngroups) {
        nv[u] = load_group<T>(row, start + g * kVec, end, p.aligned, v[u]);
      } else {
        nv[u] = 0;
#pragma unroll
        for (int e = 0; e < kVec; ++e) v[u][e] = -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int pos = start + (g0 + u * kBlock) * kVec;
      float gm = v[u][0];
#pragma unroll
      for (int e = 1; e < kVec; ++e) gm = fmaxf(gm, v[u][e]);
      if (nv[u] == kVec) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) probe = fmaf(v[u][e], 0.f, probe);
      } else {
        for (int e = 0; e < nv[u]; ++e) probe = fmaf(v[u][e], 0.f, probe);
      }
      if (gm > m) {
        int idx = pos;
#pragma unroll
        for (int e = kVec - 1; e >= 0; --e) if (v[u][e] == gm) idx = pos + e;
        m = gm;
        mi = idx;
      }
    }
  }
  const bool bad = __syncthreads_or(probe != probe);
  block_argmax(m, mi, redm, redi);
  if (threadIdx.x == 0) {
    TileStat ts;
    ts.m = m; ts.amax = mi; ts.s = bad ? (double)NAN : 0.0;
    p.tiles[tile] = ts;
  }
}

// Exact fallback of tile_topk for inputs that would overflow its candidate
// list: rounds of one group per lane; after each round the list is cut back
// to the best top_k and the admission threshold raised.
template <typename T>
DEV void tile_topk_rounds(const Params& p, const T* row, int start, int end, int ngroups, int tile,
                   uint64_t* buf) {
  __shared__ int cnt;
  __shared__ float tau_f;
  __shared__ uint64_t tau_p;
  const int K = p.top_k;
  const int tid = threadIdx.x;
  if (tid == 0) { cnt = 0; tau_f = -INFINITY; tau_p = 0ull; }
  __syncthreads();
  float probe = 0.f;
  for (int g0 = 0; g0 < ngroups; g0 += kBlock) {
    const float tf = tau_f;
    const uint64_t tp = tau_p;
    const int g = g0 + tid;
    if (g < ngroups) {
      const int pos = start + g * kVec;
      float v[kVec];
      const int n = load_group<T>(row, pos, end, p.aligned, v);
      float gm = v[0];
#pragma unroll
      for (int e = 1; e < kVec; ++e) gm = fmaxf(gm, v[e]);
      for (int e = 0; e < n; ++e) probe = fmaf(v[e], 0.f, probe);
      if (gm >= tf) {
        for (int e = 0; e < n; ++e) {
          if (v[e] >= tf) {
            const uint64_t pk = pack(v[e], pos + e);
            if (pk > tp) {
              const int slot = atomicAdd(&cnt, 1);
              buf[slot] = pk;
            }
          }
        }
      }
    }
    __syncthreads();
    const int c = cnt;
    const bool last = (g0 + kBlock >= ngroups);
    __syncthreads();   // every thread has read cnt before anyone appends again
    if (c > kTopkCap - kBlock * kVec || last) {
      const int P = next_pow2(c);
      for (int i = c + tid; i < P; i += kBlock) buf[i] = 0ull;
      bitonic_desc(buf, P);
      if (tid == 0) {
        cnt = c < K ? c : K;
        if (c >= K) { tau_p = buf[K - 1]; tau_f = packed_val(buf[K - 1]); }
      }
      __syncthreads();
    }
  }
  const bool bad = __syncthreads_or(probe != probe);
  const int c = cnt;
  uint64_t* out = p.cand + (size_t)tile * p.cand_w;
  for (int i = tid; i < p.cand_w; i += kBlock) out[i] = (i < c) ? buf[i] : 0ull;
  if (tid == 0) {
    TileStat ts;
    ts.m = c > 0 ? packed_val(buf[0]) : -INFINITY;
    ts.amax = c > 0 ? packed_idx(buf[0]) : INT_MAX;
    ts.s = bad ? (double)NAN : 0.0;
    p.tiles[tile] = ts;
  }
  __syncthreads();
}

// Descending bitonic sort of kBlock floats in LDS.
DEV void bitonic_desc_block_f(float* a) {
  for (int size = 2; size <= kBlock; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      const int t = threadIdx.x;
      if (t < kBlock / 2) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const float x = a[lo], y = a[hi];
        if ((x < y) == desc) { a[lo] = y; a[hi] = x; }
      }
    }
  }
  __syncthreads();
}

// Max and float64 sum of exp((l - max) / T) of a tile, for nucleus rows
// (whose cut needs the row sum to float64 accuracy).
template <typename T>
DEV void tile_stats64(const Params& p, const T* row, int start, int end, int ngroups, int tile) {
  __shared__ float redm[kWaves];
  __shared__ double redd[kWaves];
  const double invT = 1.0 / p.T;
  float m = -INFINITY;
  double s = 0.0;
  for (int g0 = threadIdx.x; g0 < ngroups; g0 += kUnroll * kBlock) {
    float v[kUnroll][kVec];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int g = g0 + u * kBlock;
      if (g < ngroups) {
        load_group<T>(row, start + g * kVec, end, p.aligned, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) v[u][e] = -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float gm = v[u][0];
#pragma unroll
      for (int e = 1; e < kVec; ++e) gm = fmaxf(gm, v[u][e]);
      if (gm > m) {
        if (m > -INFINITY) s *= exp(((double)m - (double)gm) * invT);
        m = gm;
      }
      if (m > -INFINITY) {
        const double zm = (double)m * invT;
#pragma unroll
        for (int e = 0; e < kVec; ++e) s += exp((double)v[u][e] * invT - zm);
      } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) if (v[u][e] != v[u][e]) s = (double)NAN;
      }
    }
  }
  const float M = block_max(m, redm);
  double term;
  if (m == -INFINITY) term = s;
  else term = s * exp(((double)m - (double)M) * invT);
  const double tot = block_sum(term, redd);
  if (threadIdx.x == 0) {
    TileStat ts;
    ts.m = M; ts.amax = INT_MAX; ts.s = tot;
    p.tiles[tile] = ts;
  }
}

// The tile's top_k under (value desc, index asc), written to p.cand.
//  1. Every lane loads its first kUnroll groups; the top_k-th largest of the
//     kBlock lane maxima is the admission threshold tau.  top_k distinct
//     logits reach it, so it is a lower bound of the tile's top_k-th value.
//  2. The tile streams like the other modes (kUnroll groups in flight per
//     lane, no barriers); logits >= tau go to an LDS list.
//  3. One sort of the list; its first top_k entries are the answer.
// If the list would overflow, the tile is redone by tile_topk_rounds.
template <typename T>
DEV void tile_topk(const Params& p, const T* row, int start, int end, int ngroups, int tile,
                   uint64_t* buf) {
  __shared__ int cnt, overflow;
  __shared__ float lmax[kBlock];
  const int K = p.top_k;
  const int tid = threadIdx.x;
  if (tid == 0) { cnt = 0; overflow = 0; }
  float probe = 0.f;
  float tau = -INFINITY;
  for (int base = 0; base < ngroups; base += kUnroll * kBlock) {
    float v[kUnroll][kVec];
    int nv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int g = base + tid + u * kBlock;
      if (g < ngroups) {
        nv[u] = load_group<T>(row, start + g * kVec, end, p.aligned, v[u]);
      } else {
        nv[u] = 0;
#pragma unroll
        for (int e = 0; e < kVec; ++e) v[u][e] = -INFINITY;
      }
    }
    if (base == 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int e = 0; e < kVec; ++e) mx = fmaxf(mx, v[u][e]);
      lmax[tid] = mx;
      bitonic_desc_block_f(lmax);
      tau = K <= kBlock ? lmax[K - 1] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int pos = start + (base + tid + u * kBlock) * kVec;
      float gm = v[u][0];
#pragma unroll
      for (int e = 1; e < kVec; ++e) gm = fmaxf(gm, v[u][e]);
      if (nv[u] == kVec) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) probe = fmaf(v[u][e], 0.f, probe);
      } else {
        for (int e = 0; e < nv[u]; ++e) probe = fmaf(v[u][e], 0.f, probe);
      }
      if (gm >= tau) {
        for (int e = 0; e < nv[u]; ++e) {
          if (v[u][e] >= tau) {
            const int slot = atomicAdd(&cnt, 1);
            if (slot < kTopkCap) buf[slot] = pack(v[u][e], pos + e);
            else overflow = 1;
          }
        }
      }
    }
  }
  __syncthreads();
  if (overflow) {
    // an adversarial tile: redo it exactly with the round-based path
    __syncthreads();
    tile_topk_rounds<T>(p, row, start, end, ngroups, tile, buf);
    return;
  }
  const bool bad = __syncthreads_or(probe != probe);
  const int c = cnt;
  const int P = next_pow2(c);
  for (int i = c + tid; i < P; i += kBlock) buf[i] = 0ull;
  bitonic_desc(buf, P);
  const int keep = c < K ? c : K;
  uint64_t* out = p.cand + (size_t)tile * p.cand_w;
  for (int i = tid; i < p.cand_w; i += kBlock) out[i] = (i < keep) ? buf[i] : 0ull;
  if (tid == 0) {
    TileStat ts;
    ts.m = keep > 0 ? packed_val(buf[0]) : -INFINITY;
    ts.amax = keep > 0 ? packed_idx(buf[0]) : INT_MAX;
    ts.s = bad ? (double)NAN : 0.0;
    p.tiles[tile] = ts;
  }
  __syncthreads();
}

// ================================================================== outputs

DEV void emit_invalid(const Params& p, int b, int status) {
  int32_t* ot = p.out_tokens + (size_t)b * p.out_w;
  for (int i = threadIdx.x; i < p.out_w; i += kBlock) {
    ot[i] = -1;
    if (p.out_nodes) p.out_nodes[(size_t)b * p.out_w + i] = -1;
  }
  if (p.resid_probs) {
    float* rp = p.resid_probs + (size_t)b * p.V;
    for (int i = threadIdx.x; i < p.V; i += kBlock) rp[i] = 0.f;
  }
  if (threadIdx.x == 0) {
    p.acc_len[b] = 0;
    if (p.seq_status) p.seq_status[b] = status;
  }
}

DEV void emit_tokens(const Params& p, int b, const int32_t* x, int n, int y, int status) {
  int32_t* ot = p.out_tokens + (size_t)b * p.out_w;
  for (int i = threadIdx.x; i < p.out_w; i += kBlock) ot[i] = i < n ? x[i] : (i == n ? y : -1);
  if (threadIdx.x == 0) {
    p.acc_len[b] = n;
    if (p.seq_status) p.seq_status[b] = status;
  }
}

// Adjusted probability of one entry of a row (plain softmax or nucleus).
struct RowView {
  const void* row;
  double zm;      // max z of the row (z = l / T)
  double norm;    // normaliser (Z, or nucleus mass)
  uint64_t cut;   // nucleus: v is kept iff pack(l_v, v) >= cut; 0 = no nucleus
};

DEV double prob_from(const RowView& r, double invT, float l, int v) {
  if (r.cut && pack(l, v) < r.cut) return 0.0;
  return exp((double)l * invT - r.zm) / r.norm;
}

template <typename T>
DEV double prob_of(const RowView& r, double invT, int v) {
  return prob_from(r, invT, Io<T>::at((const T*)r.row, v), v);
}

// One chunk of kResidSeg entries of the residual draw: thread t owns
// [c0 + 8t, c0 + 8t + 8), loaded as one group.  w = max(0, p'(v) - q'(v)),
// or p'(v) without q.  Returns the thread's exclusive prefix within the chunk
// (fixed order); *tot = chunk total.
template <typename T>
DEV double resid_chunk(const RowView& pr, const RowView* qr, double invT, int V, int aligned,
                       int c0, double w[kVec], double* red, double* tot) {
  const int pos = c0 + threadIdx.x * kVec;
  float lp[kVec], lq[kVec];
  int n = 0;
  if (pos < V) {
    n = load_group<T>((const T*)pr.row, pos, V, aligned, lp);
    if (qr) load_group<T>((const T*)qr->row, pos, V, aligned, lq);
  }
  double t = 0.0;
#pragma unroll
  for (int q = 0; q < kVec; ++q) {
    double wq = 0.0;
    if (q < n) {
      wq = prob_from(pr, invT, lp[q], pos + q);
      if (qr) {
        wq -= prob_from(*qr, invT, lq[q], pos + q);
        wq = wq > 0.0 ? wq : 0.0;
      }
    }
    w[q] = wq;
    t += wq;
  }
  return block_exscan(t, red, tot);
}

// Within one chunk whose total crosses t (base = mass before the chunk):
// first v with C_v > t; if rounding leaves none, the chunk's last positive entry.
DEV int pick_in_chunk(double base, double ex, const double w[kVec], int c0, double t, int* sh_int) {
  if (threadIdx.x == 0) *sh_int = INT_MAX;
  __syncthreads();
  double c = base + ex;
  int mine = INT_MAX, last_pos = -1;
#pragma unroll
  for (int q = 0; q < kVec; ++q) {
    c += w[q];
    const int v = c0 + threadIdx.x * kVec + q;
    if (w[q] > 0.0) last_pos = v;
    if (mine == INT_MAX && w[q] > 0.0 && c > t) mine = v;
  }
  atomicMin(sh_int, mine);
  __syncthreads();
  int y = *sh_int;
  __syncthreads();
  if (y == INT_MAX) {
    if (threadIdx.x == 0) *sh_int = -1;
    __syncthreads();
    atomicMax(sh_int, last_pos);
    __syncthreads();
    y = *sh_int;
    __syncthreads();
  }
  return y;
}

// Inverse CDF over a whole row inside one workgroup (the empty-residual
// fallback): y = min{v : C_v > ur * S'}.
template <typename T>
DEV int resid_draw(const RowView& pr, const RowView* qr, double invT, int V, int aligned, double ur,
                   double* red, int* sh_int, double* S_out) {
  double w[kVec];
  double S = 0.0;
  for (int c0 = 0; c0 < V; c0 += kResidSeg) {
    double tot;
    resid_chunk<T>(pr, qr, invT, V, aligned, c0, w, red, &tot);
    S += tot;
  }
  *S_out = S;
  if (!(S > 0.0)) return -1;
  const double t = ur * S;
  double base = 0.0;
  int lastc = 0;
  for (int c0 = 0; c0 < V; c0 += kResidSeg) {
    double tot;
    const double ex = resid_chunk<T>(pr, qr, invT, V, aligned, c0, w, red, &tot);
    if (tot > 0.0) lastc = c0;
    if (base + tot > t) return pick_in_chunk(base, ex, w, c0, t, sh_int);
    base += tot;
  }
  double tot;
  const double ex = resid_chunk<T>(pr, qr, invT, V, aligned, lastc, w, red, &tot);
  return pick_in_chunk(-INFINITY, ex, w, lastc, INFINITY, sh_int);
}

// Block-wide check of the rows of a sequence whose probes saw a non-finite
// value; returns true if one of them holds NaN or +inf.  `flag[r]`: 1 bad,
// 2 needs the exact scan.
template <typename T>
DEV bool rows_bad(const Params& p, int b, const int* flag, int nrows) {
  for (int r = 0; r < nrows; ++r) {
    if (flag[r] == 1) return true;
    if (flag[r] == 2) {
      const int grow = r < p.rows_t ? trow(p, b, r) : drow(p, b, r - p.rows_t);
      if (row_has_nan_or_posinf<T>(row_ptr<T>(p, grow), p.V)) return true;
    }
  }
  return false;
}

// ================================================================== greedy chain

template <typename T>
__global__ __launch_bounds__(kBlock) void k_greedy_final(Params p) {
  __shared__ int rA[kMaxRows];
  __shared__ int rBad[kMaxRows];
  __shared__ int sx[64];
  __shared__ int sh_n, sh_st;
  const int b = blockIdx.x;
  const int k = p.k, V = p.V;
  const int32_t* x = p.tokens + (size_t)b * k;
  for (int j = threadIdx.x; j <= k; j += kBlock) {
    const RowStat rs = combine_tiles(p, trow(p, b, j), false);
    rA[j] = rs.amax;
    int bad = (rs.M == INFINITY) || (rs.M == -INFINITY) || (rs.M != rs.M) || (rs.amax == INT_MAX);
    if (!bad && rs.probe) bad = 2;
    rBad[j] = bad;
    if (j < k) sx[j] = x[j];
  }
  __syncthreads();
  if (rows_bad<T>(p, b, rBad, k + 1)) { emit_invalid(p, b, 4); return; }
  if (threadIdx.x == 0) {
    int n = k, st = 0;
    for (int j = 0; j < k; ++j) {
      const int xj = sx[j];
      if (xj < 0 || xj >= V) { st |= 1; n = j; break; }
      if (xj != rA[j]) { n = j; break; }
    }
    sh_n = n; sh_st = st;
  }
  __syncthreads();
  emit_tokens(p, b, x, sh_n, rA[sh_n], sh_st);
}

// ================================================================== token tree

template <typename T>
__global__ __launch_bounds__(kBlock) void k_tree_final(Params p) {
  __shared__ int g[kMaxTree];
  __shared__ int spar[kMaxTree];
  __shared__ int stok[kMaxTree];
  __shared__ short jmp[2][kMaxTree];
  __shared__ short dep[2][kMaxTree];
  __shared__ unsigned char val[2][kMaxTree];
  __shared__ int rBad[kMaxTree];
  __shared__ int sh_st, sh_best;
  const int b = blockIdx.x;
  const int N = p.k, V = p.V, tid = threadIdx.x;
  const int32_t* par = p.parents + (size_t)b * N;
  const int32_t* tok = p.tokens + (size_t)b * N;
  if (tid == 0) { sh_st = 0; sh_best = 0; }
  for (int i = tid; i < N; i += kBlock) {
    const RowStat rs = combine_tiles(p, trow(p, b, i), false);
    g[i] = rs.amax;
    int bad = (rs.M == INFINITY) || (rs.M == -INFINITY) || (rs.M != rs.M) || (rs.amax == INT_MAX);
    if (!bad && rs.probe) bad = 2;
    rBad[i] = bad;
    spar[i] = par[i];
    stok[i] = tok[i];
  }
  __syncthreads();
  if (rows_bad<T>(p, b, rBad, N)) { emit_invalid(p, b, 4); return; }
  int st = 0;
  for (int i = tid; i < N; i += kBlock) {
    const int pi = spar[i];
    int ok, j, d;
    if (i == 0) {
      if (pi != -1) st |= 2;
      ok = 1; j = -1; d = 0;
    } else if (pi < 0 || pi >= i) {
      st |= 2; ok = 0; j = -1; d = 0;
    } else {
      const int t = stok[i];
      if (t < 0 || t >= V) { st |= 1; ok = 0; }
      else ok = (t == g[pi]);
      j = pi; d = 1;
    }
    val[0][i] = (unsigned char)ok; jmp[0][i] = (short)j; dep[0][i] = (short)d;
  }
  if (st) atomicOr(&sh_st, st);
  __syncthreads();
  // pointer jumping: val = AND of the edge tests up to the root, dep = depth
  int cur = 0;
  for (int span = 1; span < N; span <<= 1) {
    for (int i = tid; i < N; i += kBlock) {
      const int j = jmp[cur][i];
      if (j >= 0) {
        val[cur ^ 1][i] = val[cur][i] & val[cur][j];
        dep[cur ^ 1][i] = (short)(dep[cur][i] + dep[cur][j]);
        jmp[cur ^ 1][i] = jmp[cur][j];
      } else {
        val[cur ^ 1][i] = val[cur][i];
        dep[cur ^ 1][i] = dep[cur][i];
        jmp[cur ^ 1][i] = -1;
      }
    }
    cur ^= 1;
    __syncthreads();
  }
  int bestkey = -1;
  for (int i = tid; i < N; i += kBlock)
    if (val[cur][i]) bestkey = max(bestkey, ((int)dep[cur][i] << 11) | (2047 - i));
  atomicMax(&sh_best, bestkey);
  __syncthreads();
  const int best = 2047 - (sh_best & 2047);
  const int n = sh_best >> 11;
  // the path root..best, written from LDS by the lanes of one wave
  if (tid == 0) {
    int32_t* ot = p.out_tokens + (size_t)b * p.out_w;
    int32_t* on = p.out_nodes ? p.out_nodes + (size_t)b * p.out_w : nullptr;
    ot[n] = g[best];
    int node = best;
    for (int d = n; d >= 0; --d) {
      if (on) on[d] = node;
      if (d > 0) { ot[d - 1] = stok[node]; node = spar[node]; }
    }
    p.acc_len[b] = n;
    if (p.seq_status) p.seq_status[b] = sh_st;
  }
  for (int i = n + 1 + tid; i < p.out_w; i += kBlock) {
    p.out_tokens[(size_t)b * p.out_w + i] = -1;
    if (p.out_nodes) p.out_nodes[(size_t)b * p.out_w + i] = -1;
  }
}

// ================================================================== top-k

// Merge the S tile lists of one row and publish its kept set.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_topk_rows(Params p) {
  __shared__ uint64_t buf[kTopkCap];
  __shared__ double red[kWaves];
  __shared__ int sh_n, sh_kept, sh_probe;
  __shared__ double sh_mass;
  const int grow = blockIdx.x;
  const int tid = threadIdx.x;
  const int K = p.top_k;
  const int total = p.S * p.cand_w;             // <= kTopkCap (host-checked)
  const uint64_t* src = p.cand + (size_t)grow * p.S * p.cand_w;
  const int P = next_pow2(total);
  for (int i = tid; i < P; i += kBlock) buf[i] = i < total ? src[i] : 0ull;
  if (tid == 0) {
    int pr = 0;
    for (int s = 0; s < p.S; ++s) { const double ps = p.tiles[(size_t)grow * p.S + s].s; pr |= (ps != ps); }
    sh_probe = pr;
  }
  bitonic_desc(buf, P);
  if (tid == 0) {
    int n = 0;
    while (n < K && buf[n] != 0ull) ++n;
    sh_n = n;
  }
  __syncthreads();
  const int n = sh_n;
  const float v0 = n > 0 ? packed_val(buf[0]) : -INFINITY;
  bool bad = (v0 != v0) || (v0 == INFINITY) || (v0 == -INFINITY);
  if (!bad && sh_probe) bad = row_has_nan_or_posinf<T>(row_ptr<T>(p, grow), p.V);
  const double invT = 1.0 / p.T;
  const double zm = (double)v0 * invT;
  int32_t* kidx = p.k_idx + (size_t)grow * K;
  double* ke = p.k_e + (size_t)grow * K;
  double s = 0.0;
  for (int i = tid; i < n; i += kBlock) {
    const double e = bad ? 0.0 : exp((double)packed_val(buf[i]) * invT - zm);
    kidx[i] = packed_idx(buf[i]);
    ke[i] = e;
    s += e;
  }
  const double Z = block_sum(s, red);
  int kept = n;
  double norm = Z;
  if (p.top_p < 1.0 && n > 0 && !bad) {
    // nucleus on the kept set: rank order is already probability order
    __syncthreads();
    if (tid == 0) {
      double before = 0.0, mass = 0.0;
      int kk = 0;
      for (int i = 0; i < n; ++i) {
        if (!(before < p.top_p)) break;
        const double e = ke[i];
        kk = i + 1;
        mass += e;
        before += e / Z;
      }
      sh_kept = kk;
      sh_mass = mass;
    }
    __syncthreads();
    kept = sh_kept;
    norm = sh_mass;
  }
  if (tid == 0) {
    p.k_cnt[grow] = kept;
    p.k_norm[grow] = norm;
    p.k_bad[grow] = bad ? 1 : 0;
  }
}

// p'(x) of a published kept set (0 if x is not a member); one thread.
DEV double kept_prob_1(const Params& p, int grow, int x) {
  const int K = p.top_k;
  const int n = p.k_cnt[grow];
  const int32_t* kidx = p.k_idx + (size_t)grow * K;
  for (int i = 0; i < n; ++i)
    if (kidx[i] == x) return p.k_e[(size_t)grow * K + i] / p.k_norm[grow];
  return 0.0;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_topk_final(Params p) {
  __shared__ uint64_t buf[kTopkMax];
  __shared__ double rw[kTopkMax];
  __shared__ int sidx[kTopkMax];
  __shared__ int sh_dec[64];
  __shared__ int sh_bad, sh_n, sh_st, sh_y;
  __shared__ double sh_S;
  const int b = blockIdx.x;
  const int k = p.k, V = p.V, tid = threadIdx.x, K = p.top_k;
  const int32_t* x = p.tokens + (size_t)b * k;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  for (int r = tid; r < p.rows_t + p.rows_d; r += kBlock) {
    const int grow = r < p.rows_t ? trow(p, b, r) : drow(p, b, r - p.rows_t);
    if (p.k_bad[grow]) sh_bad = 1;
  }
  __syncthreads();
  if (sh_bad) { emit_invalid(p, b, 4); return; }
  for (int j = tid; j < k; j += kBlock) {
    const int xj = x[j];
    int dec;
    if (xj < 0 || xj >= V) dec = 3;
    else {
      const double a = kept_prob_1(p, trow(p, b, j), xj);
      const double bq = kept_prob_1(p, drow(p, b, j), xj);
      const double u = (double)p.u[(size_t)b * k + j];
      dec = bq > 0.0 ? (u < fmin(1.0, a / bq) ? 1 : 0) : (a > 0.0 ? 1 : 0);
    }
    sh_dec[j] = dec;
  }
  __syncthreads();
  if (tid == 0) {
    int n = k, st = 0;
    for (int j = 0; j < k; ++j) {
      if (sh_dec[j] == 3) { st |= 1; n = j; break; }
      if (sh_dec[j] == 0) { n = j; break; }
    }
    sh_n = n; sh_st = st;
  }
  __syncthreads();
  const int n = sh_n;
  const int gp = trow(p, b, n);
  const int np = p.k_cnt[gp];
  const double normp = p.k_norm[gp];
  const int32_t* pidx = p.k_idx + (size_t)gp * K;
  const double* pe = p.k_e + (size_t)gp * K;
  for (int i = tid; i < np; i += kBlock) {
    const double pa = pe[i] / normp;
    sidx[i] = pidx[i];
    if (n < k) {
      const double qa = kept_prob_1(p, drow(p, b, n), pidx[i]);
      const double d = pa - qa;
      rw[i] = d > 0.0 ? d : 0.0;
    } else {
      rw[i] = pa;
    }
  }
  // vocabulary order of the target's kept entries
  const int P = next_pow2(np);
  for (int i = tid; i < P; i += kBlock)
    buf[i] = i < np ? (((uint64_t)(~(uint32_t)pidx[i])) << 32) | (uint32_t)i : 0ull;
  bitonic_desc(buf, P);
  if (tid == 0) {
    double S = 0.0;
    for (int i = 0; i < np; ++i) S += rw[(int)(buf[i] & 0xffffffffu)];
    if (!(S > 0.0)) {   // empty residual: draw from p'_n
      S = 0.0;
      for (int i = 0; i < np; ++i) { const int sl = (int)(buf[i] & 0xffffffffu); rw[sl] = pe[sl] / normp; S += rw[sl]; }
    }
    const double t = (double)p.ur[b] * S;
    double c = 0.0;
    int y = -1, lastpos = -1;
    for (int i = 0; i < np; ++i) {
      const int sl = (int)(buf[i] & 0xffffffffu);
      c += rw[sl];
      if (rw[sl] > 0.0) lastpos = sidx[sl];
      if (y < 0 && rw[sl] > 0.0 && c > t) y = sidx[sl];
    }
    sh_y = y < 0 ? lastpos : y;
    sh_S = S;
  }
  __syncthreads();
  if (p.resid_probs) {
    float* rp = p.resid_probs + (size_t)b * V;
    for (int v = tid; v < V; v += kBlock) rp[v] = 0.f;
    __syncthreads();
    for (int i = tid; i < np; i += kBlock) rp[sidx[i]] = (float)(rw[i] / sh_S);
  }
  emit_tokens(p, b, x, n, sh_y, sh_st);
}

// ================================================================== plain and nucleus sampling
//
// After the stream pass (float64 row sums per tile) -- and, for the nucleus,
// the exact cut per row (k_topp_rows) -- two kernels finish a call:
//   k_resid_s     grid (segment, sequence): every workgroup of a sequence
//                 redoes its accept step (k tests on a few dozen partials and
//                 2k logits), then sums the residual max(0, p' - q') (or p'_k
//                 after full acceptance) over its segment of kResidSeg
//                 entries in float64; segment 0 publishes the sequence state.
//   k_resid_final one workgroup per sequence: S' = sum of the segments, the
//                 segment where ur * S' falls, the entry inside it, outputs.

// The adjusted view of row `grow` (FILT: kFiltNone or kFiltTopp).
template <typename T, int FILT>
DEV RowView sample_view(const Params& p, int grow, double invT, bool* bad) {
  if constexpr (FILT == kFiltTopp) {
    const RowNuc nu = p.nuc[grow];
    *bad = nu.ok != 1;
    return RowView{row_ptr<T>(p, grow), (double)nu.M * invT, nu.N, nu.cut};
  } else {
    const RowStat rs = combine_tiles(p, grow, true);
    *bad = (rs.Z != rs.Z) || (rs.M == INFINITY) || (rs.M == -INFINITY);
    return RowView{row_ptr<T>(p, grow), (double)rs.M * invT, rs.Z, 0ull};
  }
}

// The accept step of sequence b.  Returns false if a row is invalid (the
// outputs are then written by the workgroup with `emit`).
template <typename T, int FILT>
DEV bool accept_step(const Params& p, int b, bool emit, int* n_out, int* st_out) {
  __shared__ int rBad[kMaxRows];
  __shared__ int sh_dec[64];
  __shared__ int sh_internal;
  const int k = p.k, V = p.V, tid = threadIdx.x;
  const double invT = 1.0 / p.T;
  const int nrows = p.rows_t + p.rows_d;
  const int32_t* x = p.tokens + (size_t)b * k;
  if (tid == 0) sh_internal = 0;
  __syncthreads();
  for (int r = tid; r < nrows; r += kBlock) {
    const int grow = r < p.rows_t ? trow(p, b, r) : drow(p, b, r - p.rows_t);
    bool bad;
    sample_view<T, FILT>(p, grow, invT, &bad);
    rBad[r] = bad ? 1 : 0;
    if (FILT == kFiltTopp && p.nuc[grow].ok == 2) sh_internal = kStatusInternal;
  }
  __syncthreads();
  if (rows_bad<T>(p, b, rBad, nrows)) {
    if (emit) emit_invalid(p, b, 4 | sh_internal);
    return false;
  }
  for (int j = tid; j < k; j += kBlock) {
    const int xj = x[j];
    int dec;
    if (xj < 0 || xj >= V) dec = 3;
    else {
      bool dummy;
      const double a = prob_of<T>(sample_view<T, FILT>(p, trow(p, b, j), invT, &dummy), invT, xj);
      const double bq = prob_of<T>(sample_view<T, FILT>(p, drow(p, b, j), invT, &dummy), invT, xj);
      const double u = (double)p.u[(size_t)b * k + j];
      dec = bq > 0.0 ? (u < fmin(1.0, a / bq) ? 1 : 0) : (a > 0.0 ? 1 : 0);
    }
    sh_dec[j] = dec;
  }
  __syncthreads();
  int n = k, st = 0;
  for (int j = 0; j < k; ++j) {
    if (sh_dec[j] == 3) { st |= 1; n = j; break; }
    if (sh_dec[j] == 0) { n = j; break; }
  }
  *n_out = n;
  *st_out = st;
  __syncthreads();
  return true;
}

template <typename T, int FILT>
__global__ __launch_bounds__(kBlock) void k_resid_s(Params p) {
  __shared__ double red[kWaves];
  const int b = blockIdx.y, seg = blockIdx.x;
  int n, st;
  if (!accept_step<T, FILT>(p, b, seg == 0, &n, &st)) {
    if (seg == 0 && threadIdx.x == 0) p.seq_n[b] = -1;
    return;
  }
  const double invT = 1.0 / p.T;
  bool dummy;
  const RowView pr = sample_view<T, FILT>(p, trow(p, b, n), invT, &dummy);
  RowView qrv{nullptr, 0.0, 1.0, 0ull};
  if (n < p.k) qrv = sample_view<T, FILT>(p, drow(p, b, n), invT, &dummy);
  double w[kVec];
  double tot;
  resid_chunk<T>(pr, n < p.k ? &qrv : nullptr, invT, p.V, p.aligned, seg * kResidSeg, w, red, &tot);
  if (threadIdx.x == 0) {
    p.spart[(size_t)b * p.S2 + seg] = tot;
    if (seg == 0) { p.seq_n[b] = n; p.seq_st[b] = st; }
  }
}

template <typename T, int FILT>
__global__ __launch_bounds__(kBlock) void k_resid_final(Params p) {
  __shared__ double red[kWaves];
  __shared__ int sh_int, sh_c;
  __shared__ double sh_base;
  const int b = blockIdx.x;
  const int n = p.seq_n[b];
  if (n < 0) return;
  const int V = p.V, k = p.k;
  const double invT = 1.0 / p.T;
  bool dummy;
  const RowView pr = sample_view<T, FILT>(p, trow(p, b, n), invT, &dummy);
  RowView qrv{nullptr, 0.0, 1.0, 0ull};
  if (n < k) qrv = sample_view<T, FILT>(p, drow(p, b, n), invT, &dummy);
  const RowView* qr = n < k ? &qrv : nullptr;
  const int32_t* x = p.tokens + (size_t)b * k;
  const double ur = (double)p.ur[b];
  double S = 0.0;
  for (int s = 0; s < p.S2; ++s) S += p.spart[(size_t)b * p.S2 + s];
  int y;
  bool p_only = (qr == nullptr);
  if (S > 0.0) {
    const double t = ur * S;
    if (threadIdx.x == 0) {
      double base = 0.0, lastbase = 0.0;
      int c = -1, lastc = 0;
      for (int s = 0; s < p.S2; ++s) {
        const double ps = p.spart[(size_t)b * p.S2 + s];
        if (ps > 0.0) { lastc = s; lastbase = base; }
        if (base + ps > t) { c = s; break; }
        base += ps;
      }
      if (c < 0) { c = lastc; base = lastbase; }
      sh_c = c;
      sh_base = base;
    }
    __syncthreads();
    const int c = sh_c;
    const double base = sh_base;
    __syncthreads();
    double w[kVec];
    double tc;
    const double ex = resid_chunk<T>(pr, qr, invT, V, p.aligned, c * kResidSeg, w, red, &tc);
    y = pick_in_chunk(base, ex, w, c * kResidSeg, t, &sh_int);
  } else {
    y = resid_draw<T>(pr, nullptr, invT, V, p.aligned, ur, red, &sh_int, &S);   // empty residual: p'_n
    p_only = true;
  }
  if (p.resid_probs) {
    float* rp = p.resid_probs + (size_t)b * V;
    const RowView* q2 = p_only ? nullptr : qr;
    for (int c0 = 0; c0 < V; c0 += kResidSeg) {
      double w[kVec];
      double tot;
      resid_chunk<T>(pr, q2, invT, V, p.aligned, c0, w, red, &tot);
#pragma unroll
      for (int q = 0; q < kVec; ++q) {
        const int v = c0 + threadIdx.x * kVec + q;
        if (v < V) rp[v] = (float)(w[q] / S);
      }
    }
  }
  emit_tokens(p, b, x, n, y, p.seq_st[b]);
}

// ================================================================== stream kernel

// One workgroup per tile; the host picks about four tiles per resident
// workgroup so that the last, partial wave of workgroups is short.
template <typename T, int MODE>
__global__ __launch_bounds__(kBlock) void k_stream(Params p) {
  const int tile = blockIdx.x;
  const int grow = tile / p.S;
  const int seg = tile - grow * p.S;
  const T* row = row_ptr<T>(p, grow);
  const int start = seg * p.L;
  const int end = min(start + p.L, p.V);
  const int ngroups = (end - start + kVec - 1) / kVec;
  if constexpr (MODE == kModeTopk) {
    __shared__ uint64_t buf[kTopkCap];
    tile_topk<T>(p, row, start, end, ngroups, tile, buf);
  } else if constexpr (MODE == kModeStats64) {
    tile_stats64<T>(p, row, start, end, ngroups, tile);
  } else {
    tile_argmax<T>(p, row, start, end, ngroups, tile);
  }
}

// ================================================================== nucleus
//
// Exact nucleus cut of one row.  The rank order is (logit desc, index asc),
// i.e. the packed u64 of pack() in descending order; e_v = exp(z_v - zmax)
// with z = l / T; the kept set is the shortest rank prefix whose mass reaches
// top_p * Z.  Search: histogram the row by d = zmax - z (level 0) or, inside
// a window, by the packed key (deeper levels); locate the boundary bin from
// exact-integer fixed-point masses; take a 3-bin window; if it holds at most
// kWindowCap entries, gather them, sort, and walk with float64 prefix sums
// starting from the exact mass of everything ranked above the window.
// Otherwise the window becomes the next level's range.  Packed keys are
// distinct, so the levels always narrow down (at most ~7).  No logit with
// d >= dmax = ln(V / (1 - top_p)) + 1 can be kept (every kept entry has
// probability > (1 - top_p) / V), so those are skipped.

struct NucState {
  double zm, invT, dmax, w0, invw0;
  int level;                 // 0: bins by d; >= 1: bins by packed key
  int p0lo, p0hi;            // level-0 window (bins), used at levels >= 1
  uint64_t plo, phi;         // packed range of the current level (>= 1)
  int sh;                    // bin = (phi - pk) >> sh
  int c0, c1;                // current window, in bins of the current level
};

// Where one logit stands relative to the current level and window.
//   cls: -1 ranked above the window, 0 in the window, 1 below it, 2 never kept
//   *bin: its bin at the current level when it lies in the level's range, else -1
DEV int nuc_class(const NucState& s, float l, int idx, double d, int* bin) {
  *bin = -1;
  if (!(d < s.dmax)) return 2;
  int b0 = (int)(d * s.invw0);
  b0 = b0 < 0 ? 0 : (b0 >= kNucBins ? kNucBins - 1 : b0);
  if (s.level == 0) {
    *bin = b0;
    return b0 < s.c0 ? -1 : (b0 > s.c1 ? 1 : 0);
  }
  if (b0 < s.p0lo) return -1;
  if (b0 > s.p0hi) return 1;
  const uint64_t pk = pack(l, idx);
  if (pk > s.phi) return -1;
  if (pk < s.plo) return 1;
  const int b = (int)((s.phi - pk) >> s.sh);
  *bin = b;
  return b < s.c0 ? -1 : (b > s.c1 ? 1 : 0);
}

// Reference factor of a bin's fixed-point masses: an upper bound of e in it.
DEV double nuc_bin_ref(const NucState& s, int b) {
  if (s.level == 0) return exp(-(double)b * s.w0);
  return exp(-(double)s.p0lo * s.w0);
}

// Histogram sweep at the current level (the window fields are ignored).
// hq: sum of e / ref(bin) in 2^-32 units (exact integers, so the order of the
// LDS atomics cannot change them; float32 exponentials suffice because these
// masses only locate the boundary); hc: counts.  *A gets the exact float64
// mass of everything ranked above the level's range, *below the count ranked
// below it (and still < dmax).
template <typename T>
DEV void nuc_hist(const T* row, int V, int aligned, NucState s, unsigned long long* hq,
                  unsigned int* hc, unsigned int* below, double* red, double* A) {
  for (int b = threadIdx.x; b < kNucBins; b += kBlock) { hq[b] = 0ull; hc[b] = 0u; }
  if (threadIdx.x == 0) *below = 0u;
  __syncthreads();
  s.c0 = 0; s.c1 = kNucBins - 1;   // whole level = "window"
  const double ref1 = (double)s.p0lo * s.w0;
  double a = 0.0;
  unsigned int nb = 0;
  for (int g = threadIdx.x; g * kVec < V; g += kBlock) {
   float vv[kVec];
   const int ng = load_group<T>(row, g * kVec, V, aligned, vv);
   for (int e = 0; e < ng; ++e) {
    const int i = g * kVec + e;
    const float l = vv[e];
    const double d = s.zm - (double)l * s.invT;
    if (!(d < s.dmax)) continue;
    int bin;
    const int cls = nuc_class(s, l, i, d, &bin);
    if (cls == -1) a += exp(-d);
    else if (cls == 1) nb++;
    else if (cls == 0) {
      const double refd = s.level == 0 ? (double)bin * s.w0 : ref1;
      const float rel = __expf((float)(refd - d));   // in (e^-w, 1]
      atomicAdd(&hq[bin], (unsigned long long)(rel * 4294967296.0f));
      atomicAdd(&hc[bin], 1u);
    }
   }
  }
  if (nb) atomicAdd(below, nb);
  *A = block_sum(a, red);
  __syncthreads();
}

// First bin whose cumulative approximate mass (from A) reaches tgt.
DEV int nuc_locate(const NucState& s, const unsigned long long* hq, double A, double tgt,
                   double* red, int* sh_int) {
  double local[kNucBins / kBlock];
  double tsum = 0.0;
#pragma unroll
  for (int q = 0; q < kNucBins / kBlock; ++q) {
    const int b = threadIdx.x * (kNucBins / kBlock) + q;
    local[q] = hq[b] ? (double)hq[b] * (1.0 / 4294967296.0) * nuc_bin_ref(s, b) : 0.0;
    tsum += local[q];
  }
  double tot;
  const double ex = block_exscan(tsum, red, &tot);
  if (threadIdx.x == 0) *sh_int = kNucBins - 1;
  __syncthreads();
  double c = A + ex;
  int found = INT_MAX;
#pragma unroll
  for (int q = 0; q < kNucBins / kBlock; ++q) {
    c += local[q];
    if (found == INT_MAX && c >= tgt) found = threadIdx.x * (kNucBins / kBlock) + q;
  }
  if (found != INT_MAX) atomicMin(sh_int, found);
  __syncthreads();
  const int b = *sh_int;
  __syncthreads();
  return b;
}

// Exact nucleus cut of one valid row (see above); fills *out.
template <typename T>
DEV void topp_search(const Params& p, const T* row, float Mrow, double Z, RowNuc* outp,
                     unsigned long long* hq, unsigned int* hc, uint64_t* win, double* red,
                     unsigned long long* redu, unsigned int* below_p, unsigned int* wcnt_p,
                     int* sh_int_p, unsigned long long* sh_pmin_p, unsigned long long* sh_pmax_p) {
  unsigned int& below = *below_p;
  unsigned int& wcnt = *wcnt_p;
  int& sh_int = *sh_int_p;
  unsigned long long& sh_pmin = *sh_pmin_p;
  unsigned long long& sh_pmax = *sh_pmax_p;
  RowNuc& out = *outp;
  const int V = p.V;
  const int tid = threadIdx.x;
  NucState s;
  s.invT = 1.0 / p.T;
  s.zm = (double)Mrow * s.invT;
  // every kept entry has probability > (1 - top_p) / V, i.e. d < ln(V / ((1 - top_p) Z))
  s.dmax = log((double)V / ((1.0 - p.top_p) * Z)) + 1.0;
  if (!(s.dmax > 1.0)) s.dmax = 1.0;
  s.w0 = s.dmax / kNucBins;
  s.invw0 = 1.0 / s.w0;
  s.level = 0; s.p0lo = 0; s.p0hi = kNucBins - 1; s.plo = 0; s.phi = ~0ull; s.sh = 0;
  s.c0 = 0; s.c1 = kNucBins - 1;

  double A = 0.0;
  nuc_hist<T>(row, V, p.aligned, s, hq, hc, &below, red, &A);
  const double tgt = p.top_p * Z;
  bool located = false;
  int result = 0;   // 1 found, -1 failed
  for (int iter = 0; iter < 64 && result == 0; ++iter) {
    if (!located) {
      const int b = nuc_locate(s, hq, A, tgt, red, &sh_int);
      s.c0 = b > 0 ? b - 1 : 0;
      s.c1 = b < kNucBins - 1 ? b + 1 : kNucBins - 1;
      located = true;
    }
    // window and below-window counts at this level
    unsigned long long cw = 0, cb = 0;
    for (int b = tid; b < kNucBins; b += kBlock) {
      if (b >= s.c0 && b <= s.c1) cw += hc[b];
      else if (b > s.c1) cb += hc[b];
    }
    unsigned long long tw, tb;
    block_exscan_u64(cw, redu, &tw);
    block_exscan_u64(cb, redu, &tb);
    tb += below;

    if (tw <= (unsigned long long)kWindowCap) {
      // gather the window; exact mass ranked above it
      if (tid == 0) wcnt = 0u;
      __syncthreads();
      double a = 0.0;
      for (int g = tid; g * kVec < V; g += kBlock) {
        float vv[kVec];
        const int ng = load_group<T>(row, g * kVec, V, p.aligned, vv);
        for (int e = 0; e < ng; ++e) {
          const int i = g * kVec + e;
          const float l = vv[e];
          const double d = s.zm - (double)l * s.invT;
          if (!(d < s.dmax)) continue;
          int bin;
          const int cls = nuc_class(s, l, i, d, &bin);
          if (cls == -1) a += exp(-d);
          else if (cls == 0) {
            const unsigned slot = atomicAdd(&wcnt, 1u);
            if (slot < (unsigned)kWindowCap) win[slot] = pack(l, i);
          }
        }
      }
      const double Aw = block_sum(a, red);
      const int n = (int)min(wcnt, (unsigned)kWindowCap);
      const int P = next_pow2(n);
      for (int i = n + tid; i < P; i += kBlock) win[i] = 0ull;
      bitonic_desc(win, P);
      // exclusive float64 prefix of e in rank order
      const int per = (n + kBlock - 1) / kBlock;
      double tl = 0.0;
      for (int q = 0; q < per; ++q) {
        const int i = tid * per + q;
        if (i < n) tl += exp((double)packed_val(win[i]) * s.invT - s.zm);
      }
      double tot;
      const double ex = block_exscan(tl, red, &tot);
      double c = Aw + ex;
      int kept_local = 0;
      double mass_local = 0.0;
      for (int q = 0; q < per; ++q) {
        const int i = tid * per + q;
        if (i < n) {
          const double e = exp((double)packed_val(win[i]) * s.invT - s.zm);
          if (c < tgt) { kept_local = i + 1; mass_local = c + e; }
          c += e;
        }
      }
      if (tid == 0) sh_int = 0;
      __syncthreads();
      atomicMax(&sh_int, kept_local);
      __syncthreads();
      const int kept = sh_int;
      __syncthreads();
      if (kept == 0) {
        if (s.c0 == 0) result = -1;                     // cut above this level's range
        else { s.c1 = s.c0 - 1; s.c0 = s.c0 >= 3 ? s.c0 - 3 : 0; }
      } else if (kept == n && tb > 0 && Aw + tot < tgt) {
        // every window entry is kept and so would be the next one: cut lies below
        if (s.c1 == kNucBins - 1) result = -1;          // cut below this level's range
        else { s.c0 = s.c1 + 1; s.c1 = s.c1 + 3 < kNucBins ? s.c1 + 3 : kNucBins - 1; }
      } else {
        if (tid == (kept - 1) / per) {                  // owner of the last kept entry
          out.N = mass_local;
          out.cut = win[kept - 1];
          red[0] = mass_local;
        }
        __syncthreads();
        out.N = red[0];
        out.cut = win[kept - 1];
        result = 1;
      }
      __syncthreads();
    } else {
      // too many entries near the cut: the window becomes the next level's range
      if (tid == 0) { sh_pmin = ~0ull; sh_pmax = 0ull; }
      __syncthreads();
      unsigned long long pmin = ~0ull, pmax = 0ull;
      for (int g = tid; g * kVec < V; g += kBlock) {
        float vv[kVec];
        const int ng = load_group<T>(row, g * kVec, V, p.aligned, vv);
        for (int e = 0; e < ng; ++e) {
          const int i = g * kVec + e;
          const float l = vv[e];
          const double d = s.zm - (double)l * s.invT;
          int bin;
          if (nuc_class(s, l, i, d, &bin) == 0) {
            const unsigned long long pk = pack(l, i);
            pmin = pk < pmin ? pk : pmin;
            pmax = pk > pmax ? pk : pmax;
          }
        }
      }
      atomicMin(&sh_pmin, pmin);
      atomicMax(&sh_pmax, pmax);
      __syncthreads();
      if (s.level == 0) { s.p0lo = s.c0; s.p0hi = s.c1; }
      s.plo = sh_pmin;
      s.phi = sh_pmax;
      const unsigned long long span = s.phi - s.plo;
      int bits = span ? 64 - __clzll((long long)span) : 0;
      s.sh = bits > 11 ? bits - 11 : 0;
      s.level += 1;
      nuc_hist<T>(row, V, p.aligned, s, hq, hc, &below, red, &A);
      located = false;
    }
  }
  out.ok = result == 1 ? 1 : 2;
}


template <typename T>
__global__ __launch_bounds__(kBlock) void k_topp_rows(Params p) {
  const int grow = blockIdx.x;
  const T* row = row_ptr<T>(p, grow);
  const int V = p.V;
  const int tid = threadIdx.x;

  __shared__ unsigned long long hq[kNucBins];
  __shared__ unsigned int hc[kNucBins];
  __shared__ uint64_t win[kWindowCap];
  __shared__ double red[kWaves];
  __shared__ unsigned long long redu[kWaves];
  __shared__ unsigned int below, wcnt;
  __shared__ int sh_int;
  __shared__ unsigned long long sh_pmin, sh_pmax;

  RowNuc out;
  out.Z = 0.0; out.N = 0.0; out.cut = 0ull; out.ok = 0; out.M = 0.f;

  const RowStat rs = combine_tiles(p, grow, true);   // float64 row sum from the tiles
  const bool invalid = (rs.Z != rs.Z) || (rs.M == INFINITY) || (rs.M == -INFINITY);
  out.M = rs.M;
  out.Z = rs.Z;
  if (invalid) {
    if (tid == 0) p.nuc[grow] = out;
  } else {
    topp_search<T>(p, row, rs.M, rs.Z, &out, hq, hc, win, red, redu, &below, &wcnt, &sh_int, &sh_pmin, &sh_pmax);
    if (tid == 0) p.nuc[grow] = out;
  }
}


// ================================================================== launchers

template <typename T>
static int capacity_t(int mode) {
  int per_cu = 0;
  hipError_t e;
  if (mode == kModeStats64) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stream<T, kModeStats64>, kBlock, 0);
  else if (mode == kModeTopk) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stream<T, kModeTopk>, kBlock, 0);
  else e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stream<T, kModeArgmax>, kBlock, 0);
  return e == hipSuccess ? per_cu : 0;
}

int stream_blocks_per_cu(int mode, int bf16) {
  return bf16 ? capacity_t<uint16_t>(mode) : capacity_t<float>(mode);
}

// With ev_begin / ev_end the dispatch packet itself records the two events
// (hipExtLaunchKernelGGL), so their difference is the kernel's duration.
template <typename T>
static hipError_t launch_stream_t(const Params& p, int mode, hipStream_t st, hipEvent_t e0,
                                  hipEvent_t e1) {
  const unsigned grid = (unsigned)((long)p.B * (p.rows_t + p.rows_d) * p.S);
  const dim3 block(kBlock);
  if (mode == kModeStats64)
    hipExtLaunchKernelGGL((k_stream<T, kModeStats64>), dim3(grid), block, 0, st, e0, e1, 0, p);
  else if (mode == kModeTopk)
    hipExtLaunchKernelGGL((k_stream<T, kModeTopk>), dim3(grid), block, 0, st, e0, e1, 0, p);
  else
    hipExtLaunchKernelGGL((k_stream<T, kModeArgmax>), dim3(grid), block, 0, st, e0, e1, 0, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_finish_t(const Params& p, int filt, hipStream_t st) {
  const int rows = p.B * (p.rows_t + p.rows_d);
  const dim3 block(kBlock), gb((unsigned)p.B), gr((unsigned)rows), gs((unsigned)p.S2, (unsigned)p.B);
  switch (filt) {
    case kFiltGreedy: hipLaunchKernelGGL((k_greedy_final<T>), gb, block, 0, st, p); break;
    case kFiltTree: hipLaunchKernelGGL((k_tree_final<T>), gb, block, 0, st, p); break;
    case kFiltTopk:
      hipLaunchKernelGGL((k_topk_rows<T>), gr, block, 0, st, p);
      hipLaunchKernelGGL((k_topk_final<T>), gb, block, 0, st, p);
      break;
    case kFiltTopp:
      hipLaunchKernelGGL((k_topp_rows<T>), gr, block, 0, st, p);
      hipLaunchKernelGGL((k_resid_s<T, kFiltTopp>), gs, block, 0, st, p);
      hipLaunchKernelGGL((k_resid_final<T, kFiltTopp>), gb, block, 0, st, p);
      break;
    default:  // plain sampling
      hipLaunchKernelGGL((k_resid_s<T, kFiltNone>), gs, block, 0, st, p);
      hipLaunchKernelGGL((k_resid_final<T, kFiltNone>), gb, block, 0, st, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_stream(const Params& p, int mode, int bf16, hipStream_t st, hipEvent_t e0,
                         hipEvent_t e1) {
  return bf16 ? launch_stream_t<uint16_t>(p, mode, st, e0, e1)
              : launch_stream_t<float>(p, mode, st, e0, e1);
}

hipError_t launch_finish(const Params& p, int filt, int bf16, hipStream_t st) {
  return bf16 ? launch_finish_t<uint16_t>(p, filt, st) : launch_finish_t<float>(p, filt, st);
}

}  // namespace sv
