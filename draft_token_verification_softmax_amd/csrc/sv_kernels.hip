// gfx950 kernels of the speculative-decoding verification step.
//
// One call is a short chain of launches on the caller's stream, with no host
// synchronisation and no cross-workgroup signalling inside a launch:
//   k_stream        the one pass over every logit the mode reads: one
//                   workgroup per tile of a row (one round of 16-byte
//                   non-temporal buffer loads per lane), leaving small
//                   partials in the workspace:
//                     ARGMAX   max + lowest index, per wave   (greedy, tree)
//                     STATS64  max + sum of exp((l - max) / T), per wave,
//                              float64 terms              (nucleus rows)
//                     STATSMIX the same with float64 terms in rows whose
//                              normaliser can decide an output and float32
//                              terms in the others   (plain, tree sampling)
//                     TOPK     a certified filter: every logit above a
//                              lower bound of the tile's top_k-th, per wave
//                              (aligned rows); or the tile's exact top_k
//                              (other shapes)             (top-k sampling)
//                   Every part also records, exactly, whether it holds a
//                   NaN or +inf, so no row is ever scanned a second time
//                   for that.
//   greedy / tree   k_greedy_final / k_tree_final: one workgroup per sequence
//   top-k           k_topk_rows (merge per row) -> k_topk_final (per sequence)
//   nucleus         k_topp_rows (exact cut per row, the multi-level search inline)
//                   (rows it could not settle) -> k_resid_s -> k_resid_final
//   plain sampling  k_resid_s (accept step + residual mass per segment)
//                   -> k_resid_final (draw; one workgroup per segment)
//
// The finishing kernels are latency-bound: each one is written as a few
// rounds of independent loads (partials are combined in registers first,
// all rows of a sequence at once) rather than chains of dependent loads.
//
// Every reduction that feeds an output has a fixed order, so repeated calls
// give bit-identical results.  Float64 carries every quantity that decides
// an integer output (accept test, nucleus cut, inverse CDF, and the row sums
// they divide by); only row sums that cannot change a decision (a chain's
// bonus row, a leaf's rows) use float32 exp2 terms summed in float64.

#include <float.h>
#include <limits.h>
#include <limits>
#include <type_traits>
#include <math.h>

#include <hip/hip_ext.h>

#include "sv_internal.h"

namespace sv {

#define DEV __device__ __forceinline__

constexpr int kWaves = kBlock / 64;
constexpr double kLog2e = 1.4426950408889634;
constexpr int kStatusInternal = 0x100;   // a numeric search did not settle (never expected)
constexpr int kTopkMax = 256;            // largest top_k
constexpr int kUnroll = 4;               // groups of kVec logits each lane has in flight
constexpr int kFilterGroups = kFilterRound / (kBlock * kVec) * 2;   // groups per lane of a top-k filter tile, times sizeof(T) / 2
constexpr int kMaxTree = 1024;
constexpr int kMaxRows = 2 * 64 + 1;

// ------------------------------------------------------------------ loads

typedef float vf4 __attribute__((ext_vector_type(4)));
typedef unsigned int vu4 __attribute__((ext_vector_type(4)));
typedef unsigned int vu2 __attribute__((ext_vector_type(2)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef double d2 __attribute__((ext_vector_type(2)));

template <typename T> struct Io;
template <> struct Io<float> {
  static DEV float at(const float* p, long i) { return p[i]; }
};
template <> struct Io<uint16_t> {
  static DEV float at(const uint16_t* p, long i) { return __uint_as_float((uint32_t)p[i] << 16); }
};

// One aligned group of kVec logits as loaded (one or two 16-byte loads).
// probe() keeps, in one register, enough to tell exactly whether any logit
// seen was a NaN: the largest magnitude bit pattern (per 16-bit half for
// bf16); a NaN is the only pattern above the one of infinity.
// Buffer loads: word 3 of a gfx9 buffer resource (raw, 32-bit data format),
// and the cache-policy bit for non-temporal (single-use) loads.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNT = 2;
DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

template <typename T> struct Group;
template <> struct Group<uint16_t> {
  vu4 w;
  DEV void load(const uint16_t* p) { w = __builtin_nontemporal_load(reinterpret_cast<const vu4*>(p)); }
  // group at byte offset voff + soff of a buffer resource (non-temporal)
  DEV void load_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    w = __builtin_bit_cast(vu4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT));
  }
  static constexpr int kBytes = 16;
  // the same words through an empty asm: values() of the copy are recomputed
  // instead of kept alive from an earlier unpack (registers)
  DEV Group opaque() const {
    Group g = *this;
    asm volatile("" : "+v"(g.w.x), "+v"(g.w.y), "+v"(g.w.z), "+v"(g.w.w));
    return g;
  }
  DEV void values(float v[kVec]) const {
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
    v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xffff0000u);
    v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xffff0000u);
  }
  DEV void probe(uint32_t& acc) const {
    us2 a = __builtin_bit_cast(us2, acc);
    a = __builtin_elementwise_max(a, __builtin_bit_cast(us2, w.x & 0x7fff7fffu));
    a = __builtin_elementwise_max(a, __builtin_bit_cast(us2, w.y & 0x7fff7fffu));
    a = __builtin_elementwise_max(a, __builtin_bit_cast(us2, w.z & 0x7fff7fffu));
    a = __builtin_elementwise_max(a, __builtin_bit_cast(us2, w.w & 0x7fff7fffu));
    acc = __builtin_bit_cast(uint32_t, a);
  }
  static DEV bool has_nan(uint32_t acc) { return (acc & 0xffffu) > 0x7f80u || (acc >> 16) > 0x7f80u; }
  // the n < kVec logits at p, the rest -inf (bf16 pattern 0xff80)
  DEV void load_part(const uint16_t* p, int n) {
    uint32_t h[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) h[e] = e < n ? (uint32_t)p[e] : 0xff80u;
    w.x = h[0] | (h[1] << 16); w.y = h[2] | (h[3] << 16);
    w.z = h[4] | (h[5] << 16); w.w = h[6] | (h[7] << 16);
  }
  DEV void select(bool c, const Group& o) {
    w.x = c ? o.w.x : w.x; w.y = c ? o.w.y : w.y; w.z = c ? o.w.z : w.z; w.w = c ? o.w.w : w.w;
  }
};
template <> struct Group<float> {
  vf4 a, b;
  DEV void load(const float* p) {
    const vf4* q = reinterpret_cast<const vf4*>(p);
    a = __builtin_nontemporal_load(q);
    b = __builtin_nontemporal_load(q + 1);
  }
  DEV void load_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    a = __builtin_bit_cast(vf4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT));
    b = __builtin_bit_cast(vf4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, kNT));
  }
  static constexpr int kBytes = 32;
  // split slot: quad a at byte voff + soff, quad b kBlock * 16 bytes further
  // (a workgroup's 256 lanes read two 4 KB runs)
  DEV void load_split(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    a = __builtin_bit_cast(vf4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT));
    b = __builtin_bit_cast(vf4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + kBlock * 16, kNT));
  }
  // -inf in the quads of a split slot whose first logit (pa for a) is at or
  // past n (n a multiple of 4: quads are wholly in or out)
  DEV void pad_split(int pa, int n) {
    if (pa >= n) a = vf4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (pa + kBlock * 4 >= n) b = vf4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  DEV Group opaque() const {
    Group g = *this;
    asm volatile("" : "+v"(g.a.x), "+v"(g.a.y), "+v"(g.a.z), "+v"(g.a.w));
    asm volatile("" : "+v"(g.b.x), "+v"(g.b.y), "+v"(g.b.z), "+v"(g.b.w));
    return g;
  }
  DEV void values(float v[kVec]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  DEV void probe(uint32_t& acc) const {
    const uint32_t m = 0x7fffffffu;
    const uint32_t x0 = max(__float_as_uint(a.x) & m, __float_as_uint(a.y) & m);
    const uint32_t x1 = max(__float_as_uint(a.z) & m, __float_as_uint(a.w) & m);
    const uint32_t x2 = max(__float_as_uint(b.x) & m, __float_as_uint(b.y) & m);
    const uint32_t x3 = max(__float_as_uint(b.z) & m, __float_as_uint(b.w) & m);
    acc = max(acc, max(max(x0, x1), max(x2, x3)));
  }
  static DEV bool has_nan(uint32_t acc) { return acc > 0x7f800000u; }
  DEV void load_part(const float* p, int n) {
    float h[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) h[e] = e < n ? p[e] : -INFINITY;
    a = vf4{h[0], h[1], h[2], h[3]};
    b = vf4{h[4], h[5], h[6], h[7]};
  }
  DEV void select(bool c, const Group& o) {
    a.x = c ? o.a.x : a.x; a.y = c ? o.a.y : a.y; a.z = c ? o.a.z : a.z; a.w = c ? o.a.w : a.w;
    b.x = c ? o.b.x : b.x; b.y = c ? o.b.y : b.y; b.z = c ? o.b.z : b.z; b.w = c ? o.b.w : b.w;
  }
};

// Load the group of kVec logits starting at `pos` (< end).  Slots past `end`
// read as -inf.  Returns the number of real logits.
template <typename T>
DEV int load_group(const T* row, int pos, int end, int aligned, float v[kVec]) {
  int n = end - pos;
  if (n >= kVec && aligned) {
    Group<T> g;
    g.load(row + pos);
    g.values(v);
    return kVec;
  }
  n = n < kVec ? n : kVec;
#pragma unroll
  for (int e = 0; e < kVec; ++e) v[e] = (e < n) ? Io<T>::at(row, (long)pos + e) : -INFINITY;
  return n;
}

// One iteration of a tile pass: the kUnroll groups g0, g0 + kBlock, ... of
// the lane, all issued as plain vector loads with no per-group test.  A group
// past the tile loads the tile's last full group instead (always in bounds)
// and is then set to -inf with nv = 0.  Only a wave that holds the partial
// last group of a row whose length is not a multiple of kVec (or a row that
// is not 16-byte aligned) takes the element path.  NaN evidence goes to
// `probe` (vector path) or `nanv` (element path).
template <typename T, int U = kUnroll>
DEV void load_iter(const T* row, int start, int end, int ngroups, int nfull, int aligned, int g0,
                   float v[U][kVec], int nv[U], uint32_t& probe, bool& nanv) {
  const bool partial = nfull != ngroups;
  if (aligned && nfull > 0 && __all(!partial || g0 + (U - 1) * kBlock < nfull)) {
    Group<T> gr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * kBlock;
      gr[u].load(row + start + (g < nfull ? g : nfull - 1) * kVec);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      gr[u].values(v[u]);
      gr[u].probe(probe);
      nv[u] = kVec;
      if (g0 + u * kBlock >= nfull) {
        nv[u] = 0;
#pragma unroll
        for (int e = 0; e < kVec; ++e) v[u][e] = -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * kBlock;
      if (g < ngroups) {
        nv[u] = load_group<T>(row, start + g * kVec, end, aligned, v[u]);
      } else {
        nv[u] = 0;
#pragma unroll
        for (int e = 0; e < kVec; ++e) v[u][e] = -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < kVec; ++e) nanv |= (v[u][e] != v[u][e]);
    }
  }
}

// One pass over the groups of a tile [start, end).  Tiles of whole groups
// in 16-byte aligned rows are read through a buffer resource spanning
// exactly the tile, U groups of kVec logits per lane in flight; a slot past
// the tile reads zeros without touching memory, so no address is clamped and
// nothing outside the tile is fetched.  The groups stay as loaded (raw
// words) until the consumer unpacks them one at a time, which keeps the
// register count -- and so the number of resident waves -- low.
// f(groups, first index, n valid) gets the lane's U group slots (slot u
// holds group first + u * kBlock and is valid iff u < n valid).  Other tiles
// assemble one group per lane at a time element by element, padded with
// -inf (f gets U = 1).  Every lane of the block runs every round (lanes past
// the tile get no valid slot), so f may use wave-wide operations.
template <typename T, int U, typename F>
DEV void tile_groups(const T* row, int start, int end, int aligned, F&& f) {
  const int ngroups = (end - start + kVec - 1) / kVec;
  const int nfull = (end - start) / kVec;
  if (aligned && nfull == ngroups && nfull > 0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(row + start, (end - start) * (int)sizeof(T));
    for (int base = 0; base < ngroups; base += U * kBlock) {
      const int g0 = base + threadIdx.x;
      Group<T> gr[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        gr[u].load_buf(rs, g0 * Group<T>::kBytes, u * kBlock * Group<T>::kBytes);
      const int nv = g0 < ngroups ? (ngroups - g0 + kBlock - 1) / kBlock : 0;
      f(gr, g0, nv);
    }
  } else {
    for (int base = 0; base < ngroups; base += kBlock) {
      const int g = base + threadIdx.x;
      Group<T> gr[1];
      const int pos = start + g * kVec;
      const int n = g < ngroups ? min(kVec, end - pos) : 0;
      if (aligned && n == kVec) gr[0].load(row + pos);
      else gr[0].load_part(row + pos, n);
      f(gr, g, g < ngroups ? 1 : 0);
    }
  }
}

// Where element e of a lane's group slot u sits in a swept range (logit
// offset from the range start).  Contiguous slots hold kVec consecutive
// logits (slot u of the lane is group base + u * kBlock); split slots (float32
// sweeps) hold two quads kBlock * 4 logits apart, base being the round's
// first logit, so that every 16-byte load instruction of a wave reads 1 KB
// of consecutive memory.
struct SlotMap {
  int base;
  int split;
  DEV int index(int u, int e) const {
    if (!split) return (base + u * kBlock) * kVec + e;
    return base + u * (kBlock * kVec) + 4 * (int)threadIdx.x + (e < 4 ? e : kBlock * 4 + e - 4);
  }
};

// tile_groups for long ranges (many rounds), as one workgroup's sweep of a
// whole row: the next round's loads are issued before the current round is
// consumed (two sets of U groups in registers), and the rounds start at
// round `rot` (mod the round count) and wrap around.  Many workgroups that
// sweep equally strided rows in step would otherwise hit the same memory
// channels at the same time; a different rotation per row spreads them.
// f(groups, slot map, n valid): as tile_groups, the first index replaced by
// the slot map.  Float32 rows of whole groups are read in split slots
// (32-byte groups, two per load instruction's 2 KB span at half density, read
// a bare 1.4 GB sweep 14% slower on one MI355X); their slots past the range
// hold -inf and all count as valid.
template <typename T, int U, typename F>
DEV void tile_groups_pipe(const T* row, int start, int end, int aligned, int rot, F&& f) {
  const int ngroups = (end - start + kVec - 1) / kVec;
  const int nfull = (end - start) / kVec;
  if (!(aligned && nfull == ngroups && nfull > 0)) {
    tile_groups<T, U>(row, start, end, aligned, [&](const auto& gr, int g0, int nv) { f(gr, SlotMap{g0, 0}, nv); });
    return;
  }
  constexpr bool kSplit = sizeof(T) == 4;
  constexpr int R = U * kBlock;                 // groups per round
  const int n = end - start;
  const int nr = (ngroups + R - 1) / R;
  rot = rot % nr;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(row + start, n * (int)sizeof(T));
  const int tid = threadIdx.x;
  auto load_round = [&](Group<T>* g, int r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (kSplit) g[u].load_split(rs, tid * 16, (r * R + u * kBlock) * Group<T>::kBytes);
      else g[u].load_buf(rs, (r * R + tid) * Group<T>::kBytes, u * kBlock * Group<T>::kBytes);
    }
  };
  Group<T> cur[U], nxt[U];
  int rc = rot;
  load_round(cur, rc);
  // Take the first round's registers here, before the loop.  Left pending
  // into the loop, they make the compiler's wait inside the body (which
  // cannot tell the first iteration from the others) also wait for the
  // next round's prefetch on every iteration, and no load overlaps work.
#pragma unroll
  for (int u = 0; u < U; ++u) cur[u] = cur[u].opaque();
  for (int j = 0; j < nr; ++j) {
    int rn = rc + 1;
    if (rn >= nr) rn -= nr;
    if (j + 1 < nr) load_round(nxt, rn);
    if constexpr (kSplit) {
      if ((rc + 1) * R > ngroups) {
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u].pad_split(rc * R * kVec + u * kBlock * kVec + 4 * tid, n);
      }
      f(cur, SlotMap{rc * R * kVec, 1}, U);
    } else {
      const int g0 = rc * R + tid;
      const int nv = g0 < ngroups ? (ngroups - g0 + kBlock - 1) / kBlock : 0;
      f(cur, SlotMap{g0, 0}, nv < U ? nv : U);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    rc = rn;
  }
}

// Max of three floats as one v_max3_f32.  fmaxf would first quieten each
// operand (one more instruction per logit); NaN never needs to survive here
// because every pass probes for it separately.
DEV float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
DEV float max8(const float v[kVec]) {
  return max3_raw(max3_raw(v[0], v[1], v[2]), max3_raw(v[3], v[4], v[5]), max3_raw(v[6], v[7], v[7]));
}
// Max of three floats that is NaN if any operand is NaN (v_maximum3_f32, IEEE
// 754-2019 maximum; -0 < +0), and the max of a group built from it: one
// comparison of the result with itself then tells whether the group held a NaN.
DEV float maximum3(float a, float b, float c) {
  float r;
  asm("v_maximum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
DEV float maximum8(const float v[kVec]) {
  return maximum3(maximum3(v[0], v[1], v[2]), maximum3(v[3], v[4], v[5]), maximum3(v[6], v[7], v[7]));
}

// ------------------------------------------------------------------ float64 exp2

// 2^(y / kExpTab) to 1.5e-13 relative, for the streaming sums; callers
// scale their arguments by kExpTab (cs = kExpTab log2(e) / T).
// y = kExpTab j + f with j = rint(y), |f| <= 1/2:
//   2^(y/kExpTab) = 2^(j >> 8) * 2^((j & 255) / 256) * e^(f ln2 / 256);
// the middle factor comes from a 256-entry table in LDS, the last from its
// Taylor series to degree 3 (|r| = |f ln2 / 256| <= 0.00136: remainder
// below r^4 / 24 < 1.4e-13, plus a few ulp of rounding).  That is seven
// orders of magnitude inside the 1e-6 band of the flag rule, and one fma
// per term less than degree 4 (remainder 4e-17), where these terms are
// most of the instructions.
// Arguments below -280000 (results below 2^-1093, i.e. 0) and NaN give 0.
constexpr int kExpTabBits = 8;
constexpr int kExpTab = 1 << kExpTabBits;
constexpr double kExpScale = (double)kExpTab;
constexpr double kE1 = 0.0027076061740622863;    // (ln2/256)^i / i!
constexpr double kE2 = 3.6655655969101062e-06;
constexpr double kE3 = 3.3083026805413713e-09;
static_assert(kExpTab == kBlock, "one table entry per thread of the block");

// 2^(j / kExpTab) for j = 0 .. kExpTab - 1, each the float64 nearest the
// exact value (the device library's exp2 is one ulp off in 20 of them).
__device__ const double kExp2Tab[kExpTab] = {
    0x1.0000000000000p+0, 0x1.00b1afa5abcbfp+0, 0x1.0163da9fb3335p+0, 0x1.02168143b0281p+0,
    0x1.02c9a3e778061p+0, 0x1.037d42e11bbccp+0, 0x1.04315e86e7f85p+0, 0x1.04e5f72f654b1p+0,
    0x1.059b0d3158574p+0, 0x1.0650a0e3c1f89p+0, 0x1.0706b29ddf6dep+0, 0x1.07bd42b72a836p+0,
    0x1.0874518759bc8p+0, 0x1.092bdf66607e0p+0, 0x1.09e3ecac6f383p+0, 0x1.0a9c79b1f3919p+0,
    0x1.0b5586cf9890fp+0, 0x1.0c0f145e46c85p+0, 0x1.0cc922b7247f7p+0, 0x1.0d83b23395decp+0,
    0x1.0e3ec32d3d1a2p+0, 0x1.0efa55fdfa9c5p+0, 0x1.0fb66affed31bp+0, 0x1.1073028d7233ep+0,
    0x1.11301d0125b51p+0, 0x1.11edbab5e2ab6p+0, 0x1.12abdc06c31ccp+0, 0x1.136a814f204abp+0,
    0x1.1429aaea92de0p+0, 0x1.14e95934f312ep+0, 0x1.15a98c8a58e51p+0, 0x1.166a45471c3c2p+0,
    0x1.172b83c7d517bp+0, 0x1.17ed48695bbc0p+0, 0x1.18af9388c8deap+0, 0x1.1972658375d2fp+0,
    0x1.1a35beb6fcb75p+0, 0x1.1af99f8138a1cp+0, 0x1.1bbe084045cd4p+0, 0x1.1c82f95281c6bp+0,
    0x1.1d4873168b9aap+0, 0x1.1e0e75eb44027p+0, 0x1.1ed5022fcd91dp+0, 0x1.1f9c18438ce4dp+0,
    0x1.2063b88628cd6p+0, 0x1.212be3578a819p+0, 0x1.21f49917ddc96p+0, 0x1.22bdda27912d1p+0,
    0x1.2387a6e756238p+0, 0x1.2451ffb82140ap+0, 0x1.251ce4fb2a63fp+0, 0x1.25e85711ece75p+0,
    0x1.26b4565e27cddp+0, 0x1.2780e341ddf29p+0, 0x1.284dfe1f56381p+0, 0x1.291ba7591bb70p+0,
    0x1.29e9df51fdee1p+0, 0x1.2ab8a66d10f13p+0, 0x1.2b87fd0dad990p+0, 0x1.2c57e39771b2fp+0,
    0x1.2d285a6e4030bp+0, 0x1.2df961f641589p+0, 0x1.2ecafa93e2f56p+0, 0x1.2f9d24abd886bp+0,
    0x1.306fe0a31b715p+0, 0x1.31432edeeb2fdp+0, 0x1.32170fc4cd831p+0, 0x1.32eb83ba8ea32p+0,
    0x1.33c08b26416ffp+0, 0x1.3496266e3fa2dp+0, 0x1.356c55f929ff1p+0, 0x1.36431a2de883bp+0,
    0x1.371a7373aa9cbp+0, 0x1.37f26231e754ap+0, 0x1.38cae6d05d866p+0, 0x1.39a401b7140efp+0,
    0x1.3a7db34e59ff7p+0, 0x1.3b57fbfec6cf4p+0, 0x1.3c32dc313a8e5p+0, 0x1.3d0e544ede173p+0,
    0x1.3dea64c123422p+0, 0x1.3ec70df1c5175p+0, 0x1.3fa4504ac801cp+0, 0x1.40822c367a024p+0,
    0x1.4160a21f72e2ap+0, 0x1.423fb2709468ap+0, 0x1.431f5d950a897p+0, 0x1.43ffa3f84b9d4p+0,
    0x1.44e086061892dp+0, 0x1.45c2042a7d232p+0, 0x1.46a41ed1d0057p+0, 0x1.4786d668b3237p+0,
    0x1.486a2b5c13cd0p+0, 0x1.494e1e192aed2p+0, 0x1.4a32af0d7d3dep+0, 0x1.4b17dea6db7d7p+0,
    0x1.4bfdad5362a27p+0, 0x1.4ce41b817c114p+0, 0x1.4dcb299fddd0dp+0, 0x1.4eb2d81d8abffp+0,
    0x1.4f9b2769d2ca7p+0, 0x1.508417f4531eep+0, 0x1.516daa2cf6642p+0, 0x1.5257de83f4eefp+0,
    0x1.5342b569d4f82p+0, 0x1.542e2f4f6ad27p+0, 0x1.551a4ca5d920fp+0, 0x1.56070dde910d2p+0,
    0x1.56f4736b527dap+0, 0x1.57e27dbe2c4cfp+0, 0x1.58d12d497c7fdp+0, 0x1.59c0827ff07ccp+0,
    0x1.5ab07dd485429p+0, 0x1.5ba11fba87a03p+0, 0x1.5c9268a5946b7p+0, 0x1.5d84590998b93p+0,
    0x1.5e76f15ad2148p+0, 0x1.5f6a320dceb71p+0, 0x1.605e1b976dc09p+0, 0x1.6152ae6cdf6f4p+0,
    0x1.6247eb03a5585p+0, 0x1.633dd1d1929fdp+0, 0x1.6434634ccc320p+0, 0x1.652b9febc8fb7p+0,
    0x1.6623882552225p+0, 0x1.671c1c70833f6p+0, 0x1.68155d44ca973p+0, 0x1.690f4b19e9538p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6b052fa75173ep+0, 0x1.6c012750bdabfp+0, 0x1.6cfdcddd47645p+0,
    0x1.6dfb23c651a2fp+0, 0x1.6ef9298593ae5p+0, 0x1.6ff7df9519484p+0, 0x1.70f7466f42e87p+0,
    0x1.71f75e8ec5f74p+0, 0x1.72f8286ead08ap+0, 0x1.73f9a48a58174p+0, 0x1.74fbd35d7cbfdp+0,
    0x1.75feb564267c9p+0, 0x1.77024b1ab6e09p+0, 0x1.780694fde5d3fp+0, 0x1.790b938ac1cf6p+0,
    0x1.7a11473eb0187p+0, 0x1.7b17b0976cfdbp+0, 0x1.7c1ed0130c132p+0, 0x1.7d26a62ff86f0p+0,
    0x1.7e2f336cf4e62p+0, 0x1.7f3878491c491p+0, 0x1.80427543e1a12p+0, 0x1.814d2add106d9p+0,
    0x1.82589994cce13p+0, 0x1.8364c1eb941f7p+0, 0x1.8471a4623c7adp+0, 0x1.857f4179f5b21p+0,
    0x1.868d99b4492edp+0, 0x1.879cad931a436p+0, 0x1.88ac7d98a6699p+0, 0x1.89bd0a478580fp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8be05bad61778p+0, 0x1.8cf3216b5448cp+0, 0x1.8e06a5e0866d9p+0,
    0x1.8f1ae99157736p+0, 0x1.902fed0282c8ap+0, 0x1.9145b0b91ffc6p+0, 0x1.925c353aa2fe2p+0,
    0x1.93737b0cdc5e5p+0, 0x1.948b82b5f98e5p+0, 0x1.95a44cbc8520fp+0, 0x1.96bdd9a7670b3p+0,
    0x1.97d829fde4e50p+0, 0x1.98f33e47a22a2p+0, 0x1.9a0f170ca07bap+0, 0x1.9b2bb4d53fe0dp+0,
    0x1.9c49182a3f090p+0, 0x1.9d674194bb8d5p+0, 0x1.9e86319e32323p+0, 0x1.9fa5e8d07f29ep+0,
    0x1.a0c667b5de565p+0, 0x1.a1e7aed8eb8bbp+0, 0x1.a309bec4a2d33p+0, 0x1.a42c980460ad8p+0,
    0x1.a5503b23e255dp+0, 0x1.a674a8af46052p+0, 0x1.a799e1330b358p+0, 0x1.a8bfe53c12e59p+0,
    0x1.a9e6b5579fdbfp+0, 0x1.ab0e521356ebap+0, 0x1.ac36bbfd3f37ap+0, 0x1.ad5ff3a3c2774p+0,
    0x1.ae89f995ad3adp+0, 0x1.afb4ce622f2ffp+0, 0x1.b0e07298db666p+0, 0x1.b20ce6c9a8952p+0,
    0x1.b33a2b84f15fbp+0, 0x1.b468415b749b1p+0, 0x1.b59728de5593ap+0, 0x1.b6c6e29f1c52ap+0,
    0x1.b7f76f2fb5e47p+0, 0x1.b928cf22749e4p+0, 0x1.ba5b030a1064ap+0, 0x1.bb8e0b79a6f1fp+0,
    0x1.bcc1e904bc1d2p+0, 0x1.bdf69c3f3a207p+0, 0x1.bf2c25bd71e09p+0, 0x1.c06286141b33dp+0,
    0x1.c199bdd85529cp+0, 0x1.c2d1cd9fa652cp+0, 0x1.c40ab5fffd07ap+0, 0x1.c544778fafb22p+0,
    0x1.c67f12e57d14bp+0, 0x1.c7ba88988c933p+0, 0x1.c8f6d9406e7b5p+0, 0x1.ca3405751c4dbp+0,
    0x1.cb720dcef9069p+0, 0x1.ccb0f2e6d1675p+0, 0x1.cdf0b555dc3fap+0, 0x1.cf3155b5bab74p+0,
    0x1.d072d4a07897cp+0, 0x1.d1b532b08c968p+0, 0x1.d2f87080d89f2p+0, 0x1.d43c8eacaa1d6p+0,
    0x1.d5818dcfba487p+0, 0x1.d6c76e862e6d3p+0, 0x1.d80e316c98398p+0, 0x1.d955d71ff6075p+0,
    0x1.da9e603db3285p+0, 0x1.dbe7cd63a8315p+0, 0x1.dd321f301b460p+0, 0x1.de7d5641c0658p+0,
    0x1.dfc97337b9b5fp+0, 0x1.e11676b197d17p+0, 0x1.e264614f5a129p+0, 0x1.e3b333b16ee12p+0,
    0x1.e502ee78b3ff6p+0, 0x1.e653924676d76p+0, 0x1.e7a51fbc74c83p+0, 0x1.e8f7977cdb740p+0,
    0x1.ea4afa2a490dap+0, 0x1.eb9f4867cca6ep+0, 0x1.ecf482d8e67f1p+0, 0x1.ee4aaa2188510p+0,
    0x1.efa1bee615a27p+0, 0x1.f0f9c1cb6412ap+0, 0x1.f252b376bba97p+0, 0x1.f3ac948dd7274p+0,
    0x1.f50765b6e4540p+0, 0x1.f6632798844f8p+0, 0x1.f7bfdad9cbe14p+0, 0x1.f91d802243c89p+0,
    0x1.fa7c1819e90d8p+0, 0x1.fbdba3692d514p+0, 0x1.fd3c22b8f71f1p+0, 0x1.fe9d96b2a23d9p+0,
};

// The table in LDS: each thread's entry is read from memory first (issued
// with a kernel's first loads, so its latency overlaps theirs) and stored
// where the kernel needs the table.
DEV double exp2_table_fetch() { return kExp2Tab[threadIdx.x]; }
DEV void exp2_table_store(double* tab, double v) {
  tab[threadIdx.x] = v;
  __syncthreads();
}
DEV double exp2_64(double y, const double* tab) {
  y = fmax(y, -280000.0);
  const double j = rint(y);
  const double f = y - j;
  double q = fma(f, kE3, kE2);
  q = fma(q, f, kE1);
  q = fma(q, f, 1.0);
  const int ji = (int)j;
  return ldexp(tab[ji & (kExpTab - 1)] * q, ji >> kExpTabBits);
}

// exp2_64(fma(l, cs, n)) for a logit l, the same value to the bit for every
// argument that is not NaN (callers never pass one), in one instruction
// less: y' = -y 2^-20 = fma(l, -cs 2^-20, -n 2^-20) with the fma's clamp to
// [0, 1] in place of the lower bound (y >= -2^20; below -280000 every term
// is 0 anyway); adding y' to -1.5 2^32, whose unit in the last place is
// 2^-20, rounds it to a multiple of 2^-20 whose integer count, -j with
// j = rint(y), is the low word of the sum; f = y - j = -(y' - that
// multiple) 2^20 exactly.  The Taylor coefficients take the factor
// (-2^20)^i, so every rounding is the one of exp2_64 scaled by a power of 2.
constexpr double kMagic20 = 6442450944.0;                    // 1.5 * 2^32
constexpr double kTwoM20 = 1.0 / 1048576.0;                  // 2^-20
constexpr double kF1 = -kE1 * 1048576.0;                     // kE_i (-2^20)^i
constexpr double kF2 = kE2 * 1048576.0 * 1048576.0;
constexpr double kF3 = -kE3 * 1048576.0 * 1048576.0 * 1048576.0;
struct Exp2Split {
  double f;
  int j;
};
DEV Exp2Split exp2_split(float l, double a, double b) {   // a = -cs 2^-20, b = -n 2^-20
  const double yp = fmin(fmax(fma((double)l, a, b), 0.0), 1.0);
  const double t = kMagic20 - yp;
  const double jd = kMagic20 - t;
  return Exp2Split{yp - jd, (int)(uint32_t)(uint64_t)__double_as_longlong(t)};
}
DEV double exp2_tail(double f) {
  double q = fma(f, kF3, kF2);
  q = fma(q, f, kF1);
  return fma(q, f, 1.0);
}
DEV double exp2_64_l(float l, double cs, double n, const double* tab) {
  const Exp2Split e = exp2_split(l, -cs * kTwoM20, -n * kTwoM20);
  return ldexp(tab[e.j & (kExpTab - 1)] * exp2_tail(e.f), e.j >> kExpTabBits);
}

// 2^y for y <= 0 in float64 with few registers: y = j + f, j = rint(y),
// 2^f = e^(f ln2) by its Taylor series to degree 13 (|f ln2| <= 0.35,
// remainder below 1e-17), then scaled by 2^j.  Below -1100 the result is 0.
DEV double exp2_neg(double y) {
  if (!(y > -1100.0)) return 0.0;
  const double j = rint(y);
  const double t = (y - j) * 0.6931471805599453;
  double q = 1.0 / 6227020800.0;                 // 1/13!
  q = fma(q, t, 1.0 / 479001600.0);
  q = fma(q, t, 1.0 / 39916800.0);
  q = fma(q, t, 1.0 / 3628800.0);
  q = fma(q, t, 1.0 / 362880.0);
  q = fma(q, t, 1.0 / 40320.0);
  q = fma(q, t, 1.0 / 5040.0);
  q = fma(q, t, 1.0 / 720.0);
  q = fma(q, t, 1.0 / 120.0);
  q = fma(q, t, 1.0 / 24.0);
  q = fma(q, t, 1.0 / 6.0);
  q = fma(q, t, 0.5);
  q = fma(q, t, 1.0);
  q = fma(q, t, 1.0);
  return ldexp(q, (int)j);
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
//
// Cross-lane steps go through DPP (an operand taken from another lane of the
// same row of 16 lanes, or a row broadcast, as a modifier of an ordinary VALU
// instruction) rather than LDS permutes, whose round trips serialise a
// reduction.  Row shifts by 1, 2, 4 and 8 give every lane the inclusive
// prefix of its row (Hillis-Steele); broadcasts of lane 15 to rows 1 and 3,
// then of lane 31 to rows 2 and 3, carry the rows' totals forward.  Lane i
// then holds the inclusive prefix over lanes 0..i, lane 63 the wave's total;
// the order of operations is fixed, so results are reproducible.  Lanes
// whose source is outside the row, or not written by a broadcast, take the
// identity.  A reduction reads lane 63, so every lane must be active.
enum : int {
  kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118,
  kDppWaveShr1 = 0x138, kDppBcast15 = 0x142, kDppBcast31 = 0x143,
  kDppQuadXor1 = 0xb1, kDppQuadXor2 = 0x4e, kDppHalfMirror = 0x141, kDppMirror = 0x140,
};

template <int CTRL, int ROWS>
DEV uint32_t dpp32(uint32_t id, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWS, 0xf, false);
}
// v of the lane CTRL selects (id where there is none), for 4- and 8-byte types
template <int CTRL, int ROWS = 0xf, typename T>
DEV T dpp_move(T id, T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, dpp32<CTRL, ROWS>(__builtin_bit_cast(uint32_t, id), __builtin_bit_cast(uint32_t, v)));
  } else {
    const uint64_t a = __builtin_bit_cast(uint64_t, id), b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp32<CTRL, ROWS>((uint32_t)a, (uint32_t)b);
    const uint32_t hi = dpp32<CTRL, ROWS>((uint32_t)(a >> 32), (uint32_t)(b >> 32));
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}
// v of one lane (uniform index), in every lane
template <typename T>
DEV T read_lane(T v, int lane) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
  } else {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}
// Inclusive scan over the lanes of a wave for an associative op with
// identity id: lane i gets op over lanes 0..i.
template <typename T, typename Op>
DEV T wave_scan(T v, T id, Op op) {
  v = op(v, dpp_move<kDppShr1>(id, v));
  v = op(v, dpp_move<kDppShr2>(id, v));
  v = op(v, dpp_move<kDppShr4>(id, v));
  v = op(v, dpp_move<kDppShr8>(id, v));
  v = op(v, dpp_move<kDppBcast15, 0xa>(id, v));
  v = op(v, dpp_move<kDppBcast31, 0xc>(id, v));
  return v;
}
// op over all lanes of a wave, in every lane
template <typename T, typename Op>
DEV T wave_all(T v, T id, Op op) {
  return read_lane(wave_scan(v, id, op), 63);
}
// The value of lane - 1 (id in lane 0).
template <typename T>
DEV T lane_before(T v, T id) { return dpp_move<kDppWaveShr1>(id, v); }

DEV float wave_max(float v) {
  return wave_all(v, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
}
DEV double wave_sum(double v) {
  return wave_all(v, 0.0, [](double a, double b) { return a + b; });
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

// Block-wide integer reductions by shuffles (one LDS slot per wave); every
// thread gets the result.  Many lanes updating one LDS word with atomics
// serialise, so block-wide decisions go through these instead.
template <typename I> DEV I wave_min_t(I v) {
  return wave_all(v, std::numeric_limits<I>::max(), [](I a, I b) { return b < a ? b : a; });
}
template <typename I> DEV I wave_max_t(I v) {
  return wave_all(v, std::numeric_limits<I>::lowest(), [](I a, I b) { return b > a ? b : a; });
}
// (min a, max b) over the block in one pass
template <typename I>
DEV void block_minmax(I& a, I& b, I* red) {
  a = wave_min_t(a);
  b = wave_max_t(b);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) { red[w] = a; red[kWaves + w] = b; }
  __syncthreads();
  a = red[0]; b = red[kWaves];
  for (int q = 1; q < kWaves; ++q) {
    a = red[q] < a ? red[q] : a;
    b = red[kWaves + q] > b ? red[kWaves + q] : b;
  }
  __syncthreads();
}
DEV int block_max_i(int v, int* red) {
  int lo = INT_MAX;
  block_minmax(lo, v, red);
  return v;
}
// Wave-aggregated append: lanes with `take` get consecutive slots of a
// shared counter with one LDS atomic per wave.  Call with every lane of the
// wave that may append active.
DEV int wave_append(bool take, int* counter) {
  const unsigned long long m = __ballot(take);
  if (m == 0ull) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)m) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(m));
  base = read_lane(base, leader);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  return take ? base + below : -1;
}

// Wave-aggregated reservation of n >= 0 slots per lane: returns the lane's
// first slot (consecutive in lane order); one LDS atomic per wave.  Call
// with every lane of the wave active.
DEV int wave_reserve(int n, int* counter) {
  const int lane = threadIdx.x & 63;
  const int incl = wave_scan(n, 0, [](int a, int b) { return a + b; });
  const int total = read_lane(incl, 63);
  int base = 0;
  if (lane == 0 && total > 0) base = atomicAdd(counter, total);
  return read_lane(base, 0) + incl - n;
}

// Exclusive scan of one double per thread in thread order (fixed order).
// Returns the exclusive prefix; *total gets the block total.
DEV double block_exscan(double v, double* red, double* total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const double inc = wave_scan(v, 0.0, [](double a, double b) { return a + b; });
  const double exl = lane_before(inc, 0.0);
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
  const unsigned long long inc =
      wave_scan(v, 0ull, [](unsigned long long a, unsigned long long b) { return a + b; });
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
DEV int trow(const Params& p, int b, int j) { return b * p.rows_t + j; }
DEV int drow(const Params& p, int b, int j) { return p.B * p.rows_t + b * p.rows_d + j; }

// Combine the partials of rows 0..nrows-1 (global row ids row_of(r)).  A
// segment of W lanes (W = ceil(P / Q) rounded up to a power of two, Q =
// kLanePartials unless a kernel short of registers asks for fewer) takes one
// row; lane s holds the Q consecutive partials from s * Q, combines them in
// registers, and butterflies over xor offsets < W finish the row.  Every partial load
// is issued before any is used, unconditionally (a slot with no partial
// reads partial 0 of the workspace and is cleared: a load under a branch
// would be waited for before the branch joins).  The order of every
// operation depends only on P, so every kernel that combines a row gets the
// same bits.  sink(r, M, amax, Z, bad) is called once per row:
//   M     the row max; amax its lowest index (argmax partials)
//   Z     STATS: sum over partials of s_t * 2^((m_t - M) log2e / T), else 0
//   bad   the row holds NaN or +inf, or no finite value
constexpr int kLanePartials = 16;

template <bool STATS, int Q = kLanePartials, typename RowOf, typename Sink>
DEV void combine_rows(const Params& p, int nrows, RowOf row_of, Sink sink) {
  const int P = p.P;
  int lw = 0;
  while ((Q << lw) < P) ++lw;
  const int W = 1 << lw;                     // lanes per row
  const int per_block = kBlock >> lw;        // rows per pass of the block
  const int seg = threadIdx.x >> lw, s = threadIdx.x & (W - 1);
  const double cd = kLog2e / p.T;
  for (int base = 0; base < nrows; base += per_block) {
    const int r = base + seg;
    TileStat ts[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = s * Q + q;
      const bool ok = r < nrows && i < P;
      ts[q] = p.tiles[ok ? (size_t)row_of(ok ? r : 0) * P + i : 0];
    }
    float m = -INFINITY;
    int ai = INT_MAX;
    int bad = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = s * Q + q;
      const bool ok = r < nrows && i < P;
      if (!ok) { ts[q].m = -INFINITY; ts[q].amax = INT_MAX; ts[q].s = 0.0; }
      bad |= ts[q].s != ts[q].s;
      if (ts[q].m > m || (ts[q].m == m && ts[q].amax < ai)) { m = ts[q].m; ai = ts[q].amax; }
    }
    for (int o = W >> 1; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o);
      const int a2 = __shfl_xor(ai, o);
      if (m2 > m || (m2 == m && a2 < ai)) { m = m2; ai = a2; }
      bad |= __shfl_xor(bad, o);
    }
    double Z = 0.0;
    if (STATS) {
      double t = 0.0;
      if (m > -INFINITY && m < INFINITY) {
#pragma unroll
        for (int q = 0; q < Q; ++q)
          t += ts[q].m == -INFINITY ? ts[q].s : ts[q].s * exp2_neg(((double)ts[q].m - (double)m) * cd);
      }
      for (int o = W >> 1; o > 0; o >>= 1) t += __shfl_xor(t, o);
      Z = t;
    }
    bad |= (m == INFINITY) || (m == -INFINITY) || (Z != Z);
    if (s == 0 && r < nrows) sink(r, m, ai, Z, bad);
  }
}

// ================================================================== tile passes

// Max and lowest index of the max over the logits each wave of a tile reads
// (one partial per wave).  Each lane keeps the first of its groups that
// reached its running max (raw words, in registers), so the lane's lowest
// index of its max is found at the end without touching memory again; the
// wave then takes the largest packed (value desc, index asc) key with one
// butterfly.  NaN: the group max propagates it, one ballot per group.
template <typename T>
DEV void tile_argmax(const Params& p, const T* row, int start, int end, int grow, int seg) {
  float m = -INFINITY;
  int gbest = -1;
  Group<T> best;
  best.load_part(row, 0);
  uint64_t nanm = 0;
  tile_groups<T, kUnroll>(row, start, end, p.aligned, [&](const auto& gr, int g0, int nv) {
    constexpr int n = sizeof(gr) / sizeof(gr[0]);
#pragma unroll
    for (int u = 0; u < n; ++u) {
      float v[kVec];
      gr[u].values(v);
      const float gm = maximum8(v);
      nanm |= __ballot(gm != gm);
      const bool better = u < nv && gm > m;
      m = better ? gm : m;
      gbest = better ? g0 + u * kBlock : gbest;
      best.select(better, gr[u]);
    }
  });
  int idx = INT_MAX;
  if (gbest >= 0) {
    float v[kVec];
    best.values(v);
#pragma unroll
    for (int e = kVec - 1; e >= 0; --e) if (v[e] == m) idx = start + gbest * kVec + e;
  }
  uint64_t key = idx == INT_MAX ? 0ull : pack(m, idx);
  key = wave_max_t(key);
  if ((threadIdx.x & 63) == 0) {
    TileStat ts;
    ts.m = key ? packed_val(key) : -INFINITY;
    ts.amax = key ? packed_idx(key) : INT_MAX;
    ts.s = (nanm || ts.m == INFINITY) ? (double)NAN : 0.0;
    p.tiles[(size_t)grow * p.P + seg * kWaves + (threadIdx.x >> 6)] = ts;
  }
}

// The drafted token whose logit an accept test reads from this row, in
// every lane; *has = false for rows without one (the value is then
// meaningless).  A buffer load with no branch: it is issued ahead of a
// tile's own loads and waited for with them, so its latency overlaps theirs
// instead of preceding them.
DEV int row_token(const Params& p, int grow, bool* has) {
  const int nt = p.B * p.rows_t;
  int b, j;
  if (grow < nt) { b = grow / p.rows_t; j = grow - b * p.rows_t; }
  else { b = (grow - nt) / p.rows_d; j = (grow - nt) - b * p.rows_d; }
  *has = !p.tree && j < p.k;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.tokens, p.B * p.k * 4);
  return __builtin_amdgcn_raw_buffer_load_b32(rs, (*has ? b * p.k + j : 0) * 4, 0, 0);
}

// Whether a row of a plain-sampling chain or of a sampled tree needs float64
// row-sum terms: only rows whose normaliser can change a decision do.
//   chain: every draft row and target rows 0..k-1 (accept ratios and the
//          residual max(0, p' - q') depend on the ratio of two normalisers);
//          target row k is only ever drawn from whole (the bonus), and
//          C_v / C_{V-1} of p'_k does not depend on its normaliser.
//   tree:  the two rows of a node with children (the tests of its children
//          and the running residual after a rejection); a leaf's target row
//          is only drawn from whole and its draft row is never read.
// For a tree the answer needs the tree's parent array: tree_parents() loads
// the part of it each lane checks (buffer loads, issued before the tile's
// own loads; offsets past the array read 0 without a memory access) and
// has_child() compares after the tile's loads are in flight.
constexpr int kParentLoads = kMaxTree / kBlock;
DEV void tree_parents(const Params& p, int grow, int pv[kParentLoads], int* node) {
  const int N = p.k, nt = p.B * p.rows_t;
  const int r = grow < nt ? grow : grow - nt;
  const int b = r / N;
  *node = r - b * N;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.parents + (size_t)b * N, N * 4);
#pragma unroll
  for (int q = 0; q < kParentLoads; ++q)
    pv[q] = __builtin_amdgcn_raw_buffer_load_b32(rs, ((int)threadIdx.x + q * kBlock) * 4, 0, 0);
}
DEV int has_child(const Params& p, const int pv[kParentLoads], int node) {
  int h = 0;
#pragma unroll
  for (int q = 0; q < kParentLoads; ++q) {
    int v = pv[q];
    asm volatile("" : "+v"(v));   // first use here, after the tile's loads are issued
    const int i = (int)threadIdx.x + q * kBlock;
    h |= (i < p.k && i > node && v == node) ? 1 : 0;
  }
  return h;
}

// Max and sum of exp((l - max) / T) = 2^((l - max) c), c = log2(e) / T, over
// the logits each wave of a tile reads (one partial per wave).  Per lane:
// each round of groups first raises the lane max m over them (rescaling the
// lane sum, in float64, if it rose), then adds 2^((l - m) c) of every logit.
// Terms:
//   float64 (exp2_64 from a 256-entry table, 1.5e-13 relative; TERMS64, and
//   the rows of a TERMS_MIX pass that need them): the sum is the one of exact
//   arithmetic to about 1e-13, so every decision taken from it agrees with a
//   float64 evaluation except within 1e-13 of its threshold.
//   float32 (the other rows of a TERMS_MIX pass): the hardware float32 exp2
//   (relative error below 1e-7) of (l - m) * c with c split into two floats
//   (c_hi + c_lo carries c to about 48 bits), eight terms summed in float32 (a
//   fixed tree), groups in float64.  Used only where the normaliser cannot
//   change a decision (see row_needs_f64 / has_child).
// The wave combines its lanes in float64 by one fixed butterfly.
constexpr int kTerms64 = 1, kTermsMix = 2;
template <typename T, int TERMS>
DEV void tile_stats(const Params& p, const T* row, int start, int end, int grow, int seg) {
  __shared__ double tab[kExpTab];
  bool xhas;
  const int xt = row_token(p, grow, &xhas);
  float lx = 0.f;
  bool hx = false;
  const double tv = exp2_table_fetch();
  bool need_tab = true;   // stored once the first round's loads are in flight
  // which terms this tile takes (uniform over the workgroup)
  bool exact = TERMS == kTerms64;
  int pv[kParentLoads];
  int node = 0;
  if constexpr (TERMS == kTermsMix) {
    if (p.tree) {
      tree_parents(p, grow, pv, &node);
    } else {
      const int nt = p.B * p.rows_t;
      exact = grow >= nt || (grow % p.rows_t) < p.k;
    }
  }
  const double cd = kLog2e / p.T;
  const double cs = kExpScale * cd;
  // c_hi <= c and c_lo > 0, so that a -inf logit gives d * c_lo = -inf and
  // a term of exactly 0 (never inf - inf)
  float c_hi = (float)cd;
  if ((double)c_hi > cd) c_hi = __uint_as_float(__float_as_uint(c_hi) - 1u);   // c > 0
  const float c_lo = fmaxf((float)(cd - (double)c_hi), FLT_MIN);
  float m = -INFINITY;
  double s = 0.0;
  uint64_t nanm = 0;
  tile_groups<T, kUnroll>(row, start, end, p.aligned, [&](const auto& gr, int g0, int nv) {
    constexpr int n = sizeof(gr) / sizeof(gr[0]);
    // the token's first use stays here, after this round's loads are issued
    // (its wait then overlaps theirs)
    int xr = xt;
    asm volatile("" : "+v"(xr));
    xr = xhas ? xr - start : -kVec;
    float mi = m;
#pragma unroll
    for (int u = 0; u < n; ++u) {
      float v[kVec];
      gr[u].values(v);
      const float gm = maximum8(v);
      nanm |= __ballot(gm != gm);
      mi = (u < nv && gm > mi) ? gm : mi;
      // the drafted token's logit, from the one lane whose group holds it
      const unsigned off = (unsigned)(xr - (g0 + u * kBlock) * kVec);
      if (u < nv && off < (unsigned)kVec) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) lx = off == (unsigned)e ? v[e] : lx;
        hx = true;
      }
    }
    if (mi > m) {
      if (m > -INFINITY) s *= exp2_neg(((double)m - (double)mi) * cd);
      m = mi;
    }
    if (need_tab) {
      tab[threadIdx.x] = tv;
      if (TERMS == kTermsMix && p.tree) exact = __syncthreads_or(has_child(p, pv, node)) != 0;
      else __syncthreads();
      need_tab = false;
    }
    if (m > -INFINITY) {
      if (exact) {
#pragma unroll
        for (int u = 0; u < n; ++u) {
          float v[kVec];
          gr[u].opaque().values(v);
          const double nmc = -(double)m * cs;
          double gs = -0.0;
#pragma unroll
          for (int q = 0; q < kVec; ++q) gs += exp2_64_l(v[q], cs, nmc, tab);
          s += u < nv ? gs : 0.0;
        }
      } else if constexpr (TERMS == kTermsMix) {
#pragma unroll
        for (int u = 0; u < n; ++u) {
          float v[kVec];
          gr[u].opaque().values(v);
          float e[kVec];
#pragma unroll
          for (int q = 0; q < kVec; ++q) {
            const float d = v[q] - m;
            e[q] = __builtin_amdgcn_exp2f(fmaf(d, c_hi, d * c_lo));
          }
          const float gs = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
          s += u < nv ? (double)gs : 0.0;
        }
      }
    }
  });
  if (hx) p.row_lx[grow] = lx;
  const float M = wave_max(m);
  double term = m == -INFINITY ? 0.0 : s * exp2_neg(((double)m - (double)M) * cd);
  term = wave_sum(term);
  if ((threadIdx.x & 63) == 0) {
    TileStat ts;
    ts.m = M; ts.amax = INT_MAX; ts.s = (nanm || M == INFINITY) ? (double)NAN : term;
    p.tiles[(size_t)grow * p.P + seg * kWaves + (threadIdx.x >> 6)] = ts;
  }
}

// Exact fallback of tile_topk for inputs that would overflow its candidate
// list: rounds of one group per lane; after each round the list is cut back
// to the best top_k and the admission threshold raised.
template <typename T>
DEV void tile_topk_rounds(const Params& p, const T* row, int start, int end, int ngroups, int tile,
                          uint64_t* buf, unsigned short* rank, int* n_out = nullptr,
                          float* m_out = nullptr) {
  __shared__ int cnt;
  __shared__ float tau_f;
  __shared__ uint64_t tau_p;
  const int K = p.top_k;
  const int tid = threadIdx.x;
  if (tid == 0) { cnt = 0; tau_f = -INFINITY; tau_p = 0ull; }
  __syncthreads();
  bool badv = false;
  for (int g0 = 0; g0 < ngroups; g0 += kBlock) {
    const float tf = tau_f;
    const uint64_t tp = tau_p;
    const int g = g0 + tid;
    if (g < ngroups) {
      const int pos = start + g * kVec;
      float v[kVec];
      const int n = load_group<T>(row, pos, end, p.aligned, v);
      const float gm = max8(v);
      for (int e = 0; e < n; ++e) badv |= (v[e] != v[e]) || (v[e] == INFINITY);
      if (__any(gm >= tf)) {
        for (int e = 0; e < kVec; ++e) {
          const uint64_t pk = pack(v[e], pos + e);
          const int slot = wave_append(e < n && v[e] >= tf && pk > tp, &cnt);
          if (slot >= 0) buf[slot] = pk;
        }
      }
    }
    __syncthreads();
    const int c = cnt;
    const bool last = (g0 + kBlock >= ngroups);
    __syncthreads();   // every thread has read cnt before anyone appends again
    if (c > kTopkCap - kBlock * kVec || last) {
      // keep the best K in rank order in buf[0, K): rank = entries above.
      // Writes only reach slots < K <= kBlock, whose entries each owner
      // thread holds in a register; every other entry is read in place.
      const uint64_t key0 = tid < c ? buf[tid] : 0ull;
      for (int i = tid; i < c; i += kBlock) {
        const uint64_t key = buf[i];
        int r = 0;
        for (int j = 0; j < c; ++j) r += buf[j] > key;
        rank[i] = (unsigned short)(r < K ? r : K);
      }
      __syncthreads();
      for (int i = tid; i < c; i += kBlock)
        if (rank[i] < K) buf[rank[i]] = i == tid ? key0 : buf[i];
      __syncthreads();
      if (tid == 0) {
        cnt = c < K ? c : K;
        if (c >= K) { tau_p = buf[K - 1]; tau_f = packed_val(buf[K - 1]); }
      }
      __syncthreads();
    }
  }
  const bool bad = __syncthreads_or(badv);
  const int c = cnt;
  const float m = c >= K ? packed_val(buf[K - 1]) : -INFINITY;   // the tile's top_k-th
  uint64_t* out = p.cand + (size_t)tile * p.cand_w;
  for (int i = tid; i < c; i += kBlock) out[i] = buf[i];
  if (tid == 0 && !n_out) {   // the row merge's redo keeps the result to itself
    TileStat ts;
    ts.m = m;
    ts.amax = c;
    ts.s = bad ? (double)NAN : 0.0;
    p.tiles[tile] = ts;
  }
  if (n_out) *n_out = c;
  if (m_out) *m_out = m;
  __syncthreads();
}

// Descending sort of one value per lane across a wave (bitonic network on
// shuffles, no LDS or barriers); lane i gets the i-th largest.
template <typename V>
DEV V wave_sort_desc(V x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const V y = __shfl_xor(x, stride);
      const bool lower = (lane & stride) == 0;        // lower index of the pair
      const bool desc = (lane & size) == 0 || size == 64;
      const bool keep_max = lower == desc;            // descending runs keep the max low
      const bool ygt = y > x;
      x = (keep_max == ygt) ? y : x;
    }
  }
  return x;
}

// Orders the c distinct keys in lst (LDS, room for c rounded up to 64)
// descending and calls emit(rank, key) for ranks < K.  Runs of 64 are sorted
// in registers by the waves and written back in place (zero padded); a key's
// rank is its place in its run plus binary searches in the other runs.
template <typename Emit>
DEV void rank_top(uint64_t* lst, int c, int K, Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int nruns = (c + 63) >> 6;
  __syncthreads();
  for (int r0 = 0; r0 < nruns; r0 += kWaves) {
    const int r = r0 + (tid >> 6);
    const int i = r * 64 + lane;
    const uint64_t key = (r < nruns && i < c) ? lst[i] : 0ull;
    const uint64_t srt = wave_sort_desc(key);
    if (r < nruns) lst[i] = srt;
  }
  __syncthreads();
  for (int i = tid; i < c; i += kBlock) {
    const uint64_t key = lst[i];
    const int r = i >> 6;
    int rank = i & 63;
    for (int q = 0; q < nruns && rank < K; ++q) {
      if (q == r) continue;
      const uint64_t* run = lst + q * 64;
      int lo = 0, hi = 64;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (run[mid] > key) lo = mid + 1; else hi = mid;
      }
      rank += lo;
    }
    if (rank < K) emit(rank, key);
  }
  __syncthreads();
}

// LDS of one top-k tile workgroup (u64 words): the candidate list and the
// groups that reach the threshold; the exact fallback reuses it whole.
constexpr int kCandCap = 1024;                        // candidate entries
constexpr int kGrpCap = 480;                          // groups holding one
constexpr int kTopkLds = kTopkCap + kTopkCap / 4;     // fallback: keys + u16 ranks
static_assert(kCandCap * 8 + kGrpCap * (kVec * 4 + 4) <= kTopkLds * 8, "top-k LDS layout");

// The tile's top_k under (value desc, index asc), written to p.cand in
// rank order (zero-padded to cand_w).
//  1. Admission threshold tau, raised after every kUnroll groups per lane:
//     each wave sorts its 64 lane maxima (over those groups) in registers
//     and takes the ceil(top_k / 4)-th largest; the smallest of the four
//     waves' values has at least top_k logits at or above it in the tile,
//     so it (and the running max of such values) bounds the tile's top_k-th
//     logit from below.
//  2. The tile streams; a group whose max reaches the current tau is copied
//     to LDS (one atomic per wave and step).  Only those groups are looked
//     at again: their logits >= the final tau become the candidate list.
//  3. The candidates are ranked (rank_top) and the tile's exact top_k goes
//     out in rank order (p.cand), with its length and its top_k-th logit in
//     the tile's TileStat (amax, m).  Every entry of the row's top_k is >=
//     the largest of those values over the row's tiles, and the per-row
//     merge keeps only those.
// If an LDS list would overflow, the tile is redone by tile_topk_rounds.
template <typename T>
DEV void tile_topk(const Params& p, const T* row, int start, int end, int ngroups, int tile,
                   uint64_t* lds) {
  __shared__ int cnt, ncg, overflow;
  __shared__ float wtau[kWaves];
  uint64_t* cand = lds;                                           // [kCandCap]
  float* gval = reinterpret_cast<float*>(lds + kCandCap);         // [kGrpCap][kVec]
  unsigned* gpos = reinterpret_cast<unsigned*>(gval + kGrpCap * kVec);   // [kGrpCap]: pos | nv << 28
  const int K = p.top_k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int nfull = (end - start) / kVec;
  if (tid == 0) { cnt = 0; ncg = 0; overflow = 0; }
  uint32_t probe = 0;
  bool nanv = false, posinf = false;
  float tau = -INFINITY;
  for (int base = 0; base < ngroups; base += kUnroll * kBlock) {
    float v[kUnroll][kVec];
    int nv[kUnroll];
    load_iter<T>(row, start, end, ngroups, nfull, p.aligned, base + tid, v, nv, probe, nanv);
    if ((base / (kUnroll * kBlock)) % 4 == 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, max8(v[u]));
      const float srt = wave_sort_desc(mx);
      const float tw = read_lane(srt, (K + kWaves - 1) / kWaves - 1);
      __syncthreads();
      if (lane == 0) wtau[tid >> 6] = tw;
      __syncthreads();
      tau = fmaxf(tau, fminf(fminf(wtau[0], wtau[1]), fminf(wtau[2], wtau[3])));
    }
    bool take[kUnroll];
    int ntake = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float gm = max8(v[u]);
      posinf |= gm == INFINITY;
      take[u] = nv[u] > 0 && gm >= tau;
      ntake += take[u];
    }
    if (__any(ntake > 0)) {
      int slot = wave_reserve(ntake, &ncg);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (take[u]) {
          if (slot < kGrpCap) {
            float* d = gval + slot * kVec;
#pragma unroll
            for (int e = 0; e < kVec; ++e) d[e] = v[u][e];
            gpos[slot] = (unsigned)(start + (base + tid + u * kBlock) * kVec) | ((unsigned)nv[u] << 28);
          } else {
            overflow = 1;
          }
          ++slot;
        }
      }
    }
  }
  __syncthreads();
  // the candidate list: logits >= tau of the copied groups
  const int ng = ncg < kGrpCap ? ncg : kGrpCap;
  for (int b0 = 0; b0 < ng; b0 += kBlock) {
    const int i = b0 + tid;
    const bool act = i < ng;
    float gv[kVec];
    unsigned gp = 0u;
    if (act) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) gv[e] = gval[i * kVec + e];
      gp = gpos[i];
    }
    const int pos = (int)(gp & 0x0fffffffu), gn = (int)(gp >> 28);
    unsigned msk = 0u;
#pragma unroll
    for (int e = 0; e < kVec; ++e) msk |= (act && e < gn && gv[e] >= tau) ? (1u << e) : 0u;
    int slot = wave_reserve(__popc(msk), &cnt);
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      if ((msk >> e) & 1u) {
        if (slot < kCandCap) cand[slot] = pack(gv[e], pos + e);
        else overflow = 1;
        ++slot;
      }
    }
  }
  __syncthreads();
  if (overflow) {
    // an adversarial tile: redo it exactly with the round-based path
    __syncthreads();
    tile_topk_rounds<T>(p, row, start, end, ngroups, tile, lds,
                        reinterpret_cast<unsigned short*>(lds + kTopkCap));
    return;
  }
  const bool bad = __syncthreads_or(nanv || posinf || Group<T>::has_nan(probe));
  const int c = cnt;
  uint64_t* out = p.cand + (size_t)tile * p.cand_w;
  __shared__ float kth;
  if (tid == 0) kth = -INFINITY;
  rank_top(cand, c, K, [&](int r, uint64_t key) {
    out[r] = key;
    if (r == K - 1) kth = packed_val(key);
  });
  if (tid == 0) {
    TileStat ts;
    ts.m = kth;
    ts.amax = c < K ? c : K;
    ts.s = bad ? (double)NAN : 0.0;
    p.tiles[tile] = ts;
  }
}

// r-th largest (1 <= r <= 64 * Q) of the keys k[q] held by the lanes of one
// wave: radix select from the top bit, one ballot per key slot and bit (no
// shuffles, no LDS).  Every lane gets it.  BITS = 16 is for keys of bf16
// values, whose low 16 bits follow from the top bit (all ones for a negative
// value, zeros otherwise): only the top 16 bits are selected, the rest is
// restored, so the result is the r-th largest key exactly in both cases.
template <int Q, int BITS>
DEV uint32_t wave_kth_key(const uint32_t (&k)[Q], int r) {
  uint32_t pre = 0u;
#pragma unroll
  for (int bit = 31; bit >= 32 - BITS; --bit) {
    const uint32_t c = pre | (1u << bit);
    int n = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) n += __popcll(__ballot(k[q] >= c));
    if (n >= r) pre = c;
  }
  if (BITS < 32 && !(pre >> 31)) pre |= (1u << (32 - BITS)) - 1u;
  return pre;
}

// Exclusive prefix over the lanes of a wave of small counts c (0 <= c < 64),
// bit-sliced through ballots; *total gets the wave's sum.
DEV int wave_exclusive_small(int c, int* total) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  int ex = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const uint64_t m = __ballot((c >> b) & 1);
    ex += __popcll(m & below) << b;
    tot += __popcll(m) << b;
  }
  *total = tot;
  return ex;
}

// Certified top-k filter over a tile of one round of loads (U groups per
// lane; whole groups, 16-byte aligned row).  Every lane reduces its groups
// to a lane max.  Each wave finds the r1-th largest of its 64 lane maxima
// (r1 = max(16, ceil(top_k / 4))) by a radix select and publishes r1 lane
// maxima at or above it; after the tile's one barrier every wave takes the
// top_k-th largest, tau, of those 4 r1 values (the same in every wave).
// They are maxima of distinct lanes, so at least top_k logits of the tile
// are >= tau: tau bounds the tile's top_k-th logit from below (lanes with no
// logit hold -inf, which can only make tau -inf: then the whole tile is
// listed).  bf16 keys need only their top 16 bits.
//
// Listing: few groups reach tau (about one per wave and group slot), so a
// wave first copies its groups whose max is >= tau into its own LDS stage
// (a short predicated store per group slot), then each lane takes one staged
// group and lists its logits >= tau, unordered, in the wave's own kWaveList
// slots of the tile's list (slot from a ballot-sliced prefix count).  Each
// wave writes its own partial: m = tau, amax = its count (above kWaveList,
// or a stage overflow: the row merge then redoes the tile exactly), s = NaN
// if its logits hold a NaN or +inf.
constexpr int kWaveList = kCandSlots / kWaves;
constexpr int kStageCap = 64;   // staged groups per wave (one per lane)

template <typename T, int U>
DEV void tile_topk_filter(const Params& p, const T* row, int start, int end, int grow, int seg) {
  constexpr int BITS = sizeof(T) == 2 ? 16 : 32;
  __shared__ uint32_t pub[kBlock];
  __shared__ Group<T> stage[kWaves][kStageCap];
  __shared__ int spos[kWaves][kStageCap];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = p.top_k;
  const int r1 = max(16, (K + kWaves - 1) / kWaves);
  const int ngroups = (end - start) / kVec;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(row + start, (end - start) * (int)sizeof(T));
  Group<T> gr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) gr[u].load_buf(rs, tid * Group<T>::kBytes, u * kBlock * Group<T>::kBytes);
  // group maxima (NaN-propagating, so one test of the lane max finds a NaN);
  // groups past the tile (partial tiles only) hold -inf
  float gm[U];
  uint32_t vm = (1u << U) - 1u;   // the lane's groups inside the tile
  if (ngroups == U * kBlock) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[kVec];
      gr[u].values(v);
      gm[u] = maximum8(v);
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[kVec];
      gr[u].values(v);
      const bool in = tid + u * kBlock < ngroups;
      gm[u] = in ? maximum8(v) : -INFINITY;
      if (!in) vm &= ~(1u << u);
    }
  }
  float lm = gm[0];
#pragma unroll
  for (int u = 1; u + 1 < U; u += 2) lm = maximum3(lm, gm[u], gm[u + 1]);
  if (U % 2 == 0) lm = maximum3(lm, gm[U - 1], gm[U - 1]);
  const bool bad = __ballot(lm != lm || lm == INFINITY) != 0ull;
  // each wave publishes r1 of its largest lane maxima
  {
    const uint32_t key[1] = {ord_key(lm)};
    const uint32_t t1 = wave_kth_key<1, BITS>(key, r1);
    const bool sel = key[0] >= t1;
    const uint64_t msk = __ballot(sel);
    const int pos = __popcll(msk & ((1ull << lane) - 1ull));
    if (sel && pos < r1) pub[w * r1 + pos] = key[0];
  }
  __syncthreads();
  float tau;
  if (kWaves * r1 <= 64) {
    const uint32_t k1[1] = {lane < kWaves * r1 ? pub[lane] : 0u};
    tau = key_value(wave_kth_key<1, BITS>(k1, K));
  } else {
    uint32_t k4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) { const int i = lane + 64 * q; k4[q] = i < kWaves * r1 ? pub[i] : 0u; }
    tau = key_value(wave_kth_key<4, BITS>(k4, K));
  }
  // stage the wave's groups that reach tau
  uint32_t pm = 0u;
#pragma unroll
  for (int u = 0; u < U; ++u) pm |= (gm[u] >= tau ? 1u : 0u) << u;
  pm &= vm;
  int nstaged;
  int slot = wave_exclusive_small(__popc(pm), &nstaged);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if ((pm >> u) & 1u) {
      if (slot < kStageCap) {
        stage[w][slot] = gr[u];
        spos[w][slot] = tid + u * kBlock;
      }
      ++slot;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // one staged group per lane: its logits >= tau into the wave's sublist
  int c = 0;
  float v[kVec];
  int gpos = 0;
  const bool have = lane < nstaged && lane < kStageCap;
  if (have) {
    stage[w][lane].values(v);
    gpos = spos[w][lane];
#pragma unroll
    for (int e = 0; e < kVec; ++e) c += v[e] >= tau;
  }
  int total;
  int at = wave_exclusive_small(c, &total);
  if (nstaged > kStageCap) total = kWaveList + 1;
  const size_t tile = (size_t)grow * p.S + seg;
  uint64_t* out = p.cand + tile * p.cand_w + w * kWaveList;
  if (have && c) {
    const int pos = start + gpos * kVec;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      if (v[e] >= tau) {
        if (at < kWaveList) out[at] = pack(v[e], pos + e);
        ++at;
      }
    }
  }
  if (lane == 0) {
    TileStat ts;
    ts.m = tau;
    ts.amax = total;
    ts.s = bad ? (double)NAN : 0.0;
    p.tiles[(size_t)grow * p.P + seg * kWaves + w] = ts;
  }
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

// x: the sequence's drafted tokens (global or LDS)
DEV void emit_tokens(const Params& p, int b, const int32_t* x, int n, int y, int status) {
  int32_t* ot = p.out_tokens + (size_t)b * p.out_w;
  for (int i = threadIdx.x; i < p.out_w; i += kBlock) ot[i] = i < n ? x[i] : (i == n ? y : -1);
  if (threadIdx.x == 0) {
    p.acc_len[b] = n;
    if (p.seq_status) p.seq_status[b] = status;
  }
}

// The drawn token of a sequence whose other outputs are already written
// (tree sampling: the walk wrote the path), or every output (chain).
DEV void emit_final(const Params& p, int b, const int32_t* x, int n, int y, int status) {
  if (p.tree) {
    if (threadIdx.x == 0) p.out_tokens[(size_t)b * p.out_w + n] = y;
  } else {
    emit_tokens(p, b, x, n, y, status);
  }
}

// First rejected position of a chain from the per-position outcomes of wave
// 0's lanes (lane j < k: j-th drafted token; call from all 64 lanes of wave
// 0).  Returns n; *st gets 1 if the first failure is an invalid token.
DEV int first_failure(bool fail, bool invalid, int k, int* st) {
  const unsigned long long fm = __ballot(fail);
  const unsigned long long im = __ballot(invalid);
  const int n = fm ? (__ffsll((unsigned long long)fm) - 1) : k;
  *st = (fm && ((im >> n) & 1ull)) ? 1 : 0;
  return n;
}

// Adjusted probability of one entry of a row (plain softmax or nucleus):
// p'(v) = 2^((l_v - M) cs / kExpTab) / norm on the kept set, cs = kExpTab log2e / T.
struct RowView {
  const void* row;
  double nmc;     // -M * cs (M = max logit of the row)
  double inv;     // 1 / norm (Z, or nucleus mass)
  uint64_t cut;   // nucleus: v is kept iff pack(l_v, v) >= cut; 0 = no nucleus
};

DEV double prob_from(const RowView& r, double cs, const double* tab, float l, int v) {
  if (r.cut && pack(l, v) < r.cut) return 0.0;
  return exp2_64_l(l, cs, r.nmc, tab) * r.inv;
}

// Residual weights of the kVec entries [pos, pos + kVec) of one chunk:
// w = max(0, p'(v) - q'(v)), or p'(v) without q.  Returns their sum.
// Residual weights of kVec entries from their logits (lp: target row n,
// lq: draft row n; n valid entries): w = max(0, p'(v) - q'(v)), or p'(v)
// without q.  Returns their sum.
DEV double resid_weights_of(const RowView& pr, const RowView& qr, bool hasq, double cs,
                            const double* tab, int pos, int n, const float lp[kVec],
                            const float lq[kVec], double w[kVec]) {
  double t = 0.0;
#pragma unroll
  for (int q = 0; q < kVec; ++q) {
    double wq = 0.0;
    if (q < n) {
      wq = prob_from(pr, cs, tab, lp[q], pos + q);
      if (hasq) {
        wq -= prob_from(qr, cs, tab, lq[q], pos + q);
        wq = wq > 0.0 ? wq : 0.0;
      }
    }
    w[q] = wq;
    t += wq;
  }
  return t;
}

// The same for the kVec entries [pos, pos + kVec) loaded from the rows.
template <typename T>
DEV double resid_weights(const RowView& pr, const RowView& qr, bool hasq, double cs,
                         const double* tab, int V, int aligned, int pos, double w[kVec]) {
  float lp[kVec], lq[kVec];
  int n = 0;
  if (pos < V) {
    n = load_group<T>((const T*)pr.row, pos, V, aligned, lp);
    if (hasq) load_group<T>((const T*)qr.row, pos, V, aligned, lq);
  }
  return resid_weights_of(pr, qr, hasq, cs, tab, pos, n, lp, lq, w);
}

// The residual mass of the kVec entries [pos, pos + kVec) of nucleus rows
// (the sum resid_weights returns, in another fixed order).  Only entries
// kept in the target's nucleus can weigh anything, and those are a few
// percent of a row at the usual top_p: each wave queues them in LDS (ballot
// and lane-prefix slot, per entry) and every 64 queued ones cost one float64
// evaluation per lane instead of one per entry of the row.  Queue slots:
// 128 per wave (64 + at most 63 before a flush).
template <typename T>
DEV double resid_nuc_sparse(const RowView& pr, const RowView& qr, bool hasq, double cs,
                            const double* tab, int V, int aligned, int pos, float* qlp,
                            float* qlq, int* qix) {
  float lp[kVec], lq[kVec];
  int nv = 0;
  if (pos < V) {
    nv = load_group<T>((const T*)pr.row, pos, V, aligned, lp);
    if (hasq) load_group<T>((const T*)qr.row, pos, V, aligned, lq);
  }
  const int lane = threadIdx.x & 63;
  auto weight = [&](float a, float b, int v) {
    double w = exp2_64_l(a, cs, pr.nmc, tab) * pr.inv;
    if (hasq) {
      w -= prob_from(qr, cs, tab, b, v);
      w = w > 0.0 ? w : 0.0;
    }
    return w;
  };
  double t = 0.0;
  int qn = 0;
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    const bool kp = e < nv && (pr.cut == 0ull || pack(lp[e], pos + e) >= pr.cut);
    const uint64_t m = __builtin_amdgcn_ballot_w64(kp);
    if (m) {
      if (kp) {
        const unsigned sl = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((unsigned)m, (unsigned)qn));
        qlp[sl] = lp[e];
        qlq[sl] = hasq ? lq[e] : 0.f;
        qix[sl] = pos + e;
      }
      qn += __popcll(m);
      if (qn >= 64) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        t += weight(qlp[lane], qlq[lane], qix[lane]);
        const int rest = qn - 64;
        float a = 0.f, b = 0.f;
        int v = 0;
        if (lane < rest) { a = qlp[64 + lane]; b = qlq[64 + lane]; v = qix[64 + lane]; }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (lane < rest) { qlp[lane] = a; qlq[lane] = b; qix[lane] = v; }
        qn = rest;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (lane < qn) t += weight(qlp[lane], qlq[lane], qix[lane]);
  return t;
}

// One chunk of kResidSeg entries of the residual draw: thread t owns
// [c0 + 8t, c0 + 8t + 8).  Returns the thread's exclusive prefix within the
// chunk (fixed order); *tot = chunk total.
template <typename T>
DEV double resid_chunk(const RowView& pr, const RowView& qr, bool hasq, double cs,
                       const double* tab, int V, int aligned, int c0, double w[kVec], double* red,
                       double* tot) {
  const double t = resid_weights<T>(pr, qr, hasq, cs, tab, V, aligned, c0 + threadIdx.x * kVec, w);
  return block_exscan(t, red, tot);
}

// Within one chunk whose total crosses t (base = mass before the chunk):
// first v with C_v > t; if rounding leaves none, the chunk's last positive entry.
DEV int pick_in_chunk(double base, double ex, const double w[kVec], int c0, double t, int* redi) {
  double c = base + ex;
  int mine = INT_MAX, last_pos = -1;
#pragma unroll
  for (int q = 0; q < kVec; ++q) {
    c += w[q];
    const int v = c0 + threadIdx.x * kVec + q;
    if (w[q] > 0.0) last_pos = v;
    if (mine == INT_MAX && w[q] > 0.0 && c > t) mine = v;
  }
  block_minmax(mine, last_pos, redi);
  return mine != INT_MAX ? mine : last_pos;
}

// Inverse CDF over a whole row inside one workgroup (the empty-residual
// fallback, over p' alone): y = min{v : C_v > ur * S'}.
template <typename T>
DEV int resid_draw(const RowView& pr, double cs, const double* tab, int V, int aligned, double ur,
                   double* red, int* redi, double* S_out) {
  const RowView none{nullptr, 0.0, 1.0, 0ull};
  double w[kVec];
  double S = 0.0;
  for (int c0 = 0; c0 < V; c0 += kResidSeg) {
    double tot;
    resid_chunk<T>(pr, none, false, cs, tab, V, aligned, c0, w, red, &tot);
    S += tot;
  }
  *S_out = S;
  if (!(S > 0.0)) return -1;
  const double t = ur * S;
  double base = 0.0;
  int lastc = 0;
  for (int c0 = 0; c0 < V; c0 += kResidSeg) {
    double tot;
    const double ex = resid_chunk<T>(pr, none, false, cs, tab, V, aligned, c0, w, red, &tot);
    if (tot > 0.0) lastc = c0;
    if (base + tot > t) return pick_in_chunk(base, ex, w, c0, t, redi);
    base += tot;
  }
  double tot;
  const double ex = resid_chunk<T>(pr, none, false, cs, tab, V, aligned, lastc, w, red, &tot);
  return pick_in_chunk(-INFINITY, ex, w, lastc, INFINITY, redi);
}

// ================================================================== greedy chain

template <typename T>
__global__ __launch_bounds__(kBlock) void k_greedy_final(Params p) {
  __shared__ int rA[kMaxRows];
  __shared__ int rBad[kMaxRows];
  __shared__ int sx[64];
  __shared__ int sh_n, sh_st, sh_bad;
  const int b = blockIdx.x;
  const int k = p.k, V = p.V, tid = threadIdx.x;
  int xj = 0;
  if (tid < k) xj = p.tokens[(size_t)b * k + tid];
  combine_rows<false>(p, k + 1, [&](int r) { return trow(p, b, r); },
                      [&](int r, float, int a, double, int bad) { rA[r] = a; rBad[r] = bad; });
  if (tid < k) sx[tid] = xj;
  __syncthreads();
  if (tid < 64) {
    int bad = 0;
    for (int r = tid; r <= k; r += 64) bad |= rBad[r];
    const bool inv = tid < k && (xj < 0 || xj >= V);
    const bool fail = tid < k && (inv || xj != rA[tid]);
    int st;
    const int n = first_failure(fail, inv, k, &st);
    const unsigned long long bm = __ballot(bad);
    if (tid == 0) { sh_n = n; sh_st = st; sh_bad = bm != 0ull; }
  }
  __syncthreads();
  if (sh_bad) { emit_invalid(p, b, 4); return; }
  emit_tokens(p, b, sx, sh_n, rA[sh_n], sh_st);
}

// ================================================================== token tree

// k_tree_final for a tree of at most 64 nodes whose rows have at most
// kLanePartials partials: every step in wave 0 alone, one lane per node,
// with no barrier.  The lane combines its row's partials in registers in the
// order combine_rows takes with one lane per row (the same argmax and bad
// flag); the edge tests read the parent's argmax, and the pointer jumping
// reads the pointed-to node's state, by lane shuffles (all lanes read before
// any writes, as the double-buffered arrays of the block path); the path is
// written from the shuffled parents and tokens of the nodes on it.
DEV void tree_final_wave(const Params& p, int b) {
  const int N = p.k, V = p.V, P = p.P, lane = threadIdx.x & 63;
  const bool on = lane < N;
  const int pi = p.parents[(size_t)b * N + (on ? lane : 0)];
  const int ti = p.tokens[(size_t)b * N + (on ? lane : 0)];
  TileStat ts[kLanePartials];
#pragma unroll
  for (int q = 0; q < kLanePartials; ++q) {
    const bool ok = on && q < P;
    ts[q] = p.tiles[ok ? (size_t)trow(p, b, lane) * P + q : 0];
  }
  float m = -INFINITY;
  int ai = INT_MAX;
  int bad = 0;
#pragma unroll
  for (int q = 0; q < kLanePartials; ++q) {
    const bool ok = on && q < P;
    if (!ok) { ts[q].m = -INFINITY; ts[q].amax = INT_MAX; ts[q].s = 0.0; }
    bad |= ts[q].s != ts[q].s;
    if (ts[q].m > m || (ts[q].m == m && ts[q].amax < ai)) { m = ts[q].m; ai = ts[q].amax; }
  }
  bad |= (m == INFINITY) || (m == -INFINITY);
  int32_t* ot = p.out_tokens + (size_t)b * p.out_w;
  int32_t* onode = p.out_nodes ? p.out_nodes + (size_t)b * p.out_w : nullptr;
  if (__ballot(on && bad)) {
    for (int i = lane; i < p.out_w; i += 64) {
      ot[i] = -1;
      if (onode) onode[i] = -1;
    }
    if (lane == 0) {
      p.acc_len[b] = 0;
      if (p.seq_status) p.seq_status[b] = 4;
    }
    return;
  }
  // the edge into each node: its token against the parent row's argmax
  const int gpar = __shfl(ai, (pi >= 0 && pi < 64) ? pi : 0);
  int st = 0, ok = 0, j = -1, d = 0;
  if (on) {
    if (lane == 0) {
      if (pi != -1) st |= 2;
      ok = 1;
    } else if (pi < 0 || pi >= lane) {
      st |= 2;
    } else {
      if (ti < 0 || ti >= V) st |= 1;
      else ok = ti == gpar;
      j = pi; d = 1;
    }
  }
  const int sst = (__ballot(st & 1) ? 1 : 0) | (__ballot(st & 2) ? 2 : 0);
  // pointer jumping: ok = AND of the edge tests up to the root, d = depth
  for (int span = 1; span < N; span <<= 1) {
    const int jj = j >= 0 ? j : lane;
    const int oj = __shfl(ok, jj), dj = __shfl(d, jj), jn = __shfl(j, jj);
    if (j >= 0) { ok &= oj; d += dj; j = jn; }
  }
  const int key = on && ok ? (d << 11) | (2047 - lane) : -1;
  const int kbest = wave_max_t(key);
  const int best = 2047 - (kbest & 2047);
  const int n = kbest >> 11;
  const int ybest = __shfl(ai, best);
  int node = best;
  for (int dd = n; dd >= 0; --dd) {
    const int tk = __shfl(ti, node), pn = __shfl(pi, node);
    if (lane == 0) {
      if (onode) onode[dd] = node;
      if (dd > 0) ot[dd - 1] = tk;
    }
    if (dd > 0) node = pn;
  }
  if (lane == 0) {
    ot[n] = ybest;
    p.acc_len[b] = n;
    if (p.seq_status) p.seq_status[b] = sst;
  }
  for (int i = n + 1 + lane; i < p.out_w; i += 64) {
    ot[i] = -1;
    if (onode) onode[i] = -1;
  }
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_tree_final(Params p) {
  if (p.k <= 64 && p.P <= kLanePartials) {
    if (threadIdx.x < 64) tree_final_wave(p, blockIdx.x);
    return;
  }
  __shared__ int g[kMaxTree];
  __shared__ int spar[kMaxTree];
  __shared__ int stok[kMaxTree];
  __shared__ short jmp[2][kMaxTree];
  __shared__ short dep[2][kMaxTree];
  __shared__ unsigned char val[2][kMaxTree];
  __shared__ unsigned char rbad[kMaxTree];
  __shared__ int redi[2 * kWaves];
  const int b = blockIdx.x;
  const int N = p.k, V = p.V, tid = threadIdx.x;
  const int32_t* par = p.parents + (size_t)b * N;
  const int32_t* tok = p.tokens + (size_t)b * N;
  constexpr int kPer = kMaxTree / kBlock;
  int rp[kPer], rt[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = tid + q * kBlock;
    rp[q] = i < N ? par[i] : 0;
    rt[q] = i < N ? tok[i] : 0;
  }
  combine_rows<false>(p, N, [&](int r) { return trow(p, b, r); },
                      [&](int r, float, int a, double, int bad) { g[r] = a; rbad[r] = (unsigned char)bad; });
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = tid + q * kBlock;
    if (i < N) { spar[i] = rp[q]; stok[i] = rt[q]; }
  }
  __syncthreads();
  int anybad = 0;
  for (int i = tid; i < N; i += kBlock) anybad |= rbad[i];
  if (__syncthreads_or(anybad)) { emit_invalid(p, b, 4); return; }
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
  const int sh_st = (__syncthreads_or(st & 1) ? 1 : 0) | (__syncthreads_or(st & 2) ? 2 : 0);
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
  const int sh_best = block_max_i(bestkey, redi);
  const int best = 2047 - (sh_best & 2047);
  const int n = sh_best >> 11;
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

// Threshold of the K largest of c >= K distinct u64 keys in LDS: keys >= the
// result are exactly the K largest.  Radix select by 8-bit digits from the
// top: an LDS histogram of the digit among the keys that match the prefix
// so far, then wave 0 finds the digit where the count from the top reaches
// the rank still needed.  Stops as soon as that digit holds exactly the
// keys still needed (then the prefix with zero low bits is the threshold).
DEV uint64_t block_topk_threshold(const uint64_t* keys, int c, int K, unsigned* hist, int* shv) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint64_t prefix = 0ull, mask = 0ull;
  int need = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kBlock) hist[b] = 0u;
    __syncthreads();
    for (int i = tid; i < c; i += kBlock) {
      const uint64_t x = keys[i];
      if ((x & mask) == prefix) atomicAdd(&hist[(unsigned)(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      unsigned h[4];
      unsigned s4 = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) { h[q] = hist[255 - 4 * lane - q]; s4 += h[q]; }
      const unsigned incl = wave_scan(s4, 0u, [](unsigned a, unsigned b) { return a + b; });
      unsigned cb = incl - s4;   // keys with a larger digit
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (cb < (unsigned)need && cb + h[q] >= (unsigned)need) {
          shv[0] = 255 - 4 * lane - q;
          shv[1] = need - (int)cb;
          shv[2] = (int)h[q];
        }
        cb += h[q];
      }
    }
    __syncthreads();
    const int d = shv[0];
    need = shv[1];
    const int hd = shv[2];
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)255 << shift;
    __syncthreads();
    if (hd == need) break;   // every key with this prefix is kept
  }
  return prefix;
}

// Keeps the min(c, K) largest of c distinct keys: writes them, unordered, to
// dst[0, n) and returns n (c <= K: all of them).
DEV int block_keep_top(const uint64_t* keys, int c, int K, uint64_t* dst, unsigned* hist, int* shv,
                       int* counter) {
  if (c <= K) {
    for (int i = threadIdx.x; i < c; i += kBlock) dst[i] = keys[i];
    __syncthreads();
    return c;
  }
  const uint64_t thr = block_topk_threshold(keys, c, K, hist, shv);
  if (threadIdx.x == 0) *counter = 0;
  __syncthreads();
  for (int i0 = 0; i0 < c; i0 += kBlock) {
    const int i = i0 + threadIdx.x;
    const uint64_t x = i < c ? keys[i] : 0ull;
    const int slot = wave_append(i < c && x >= thr, counter);
    if (slot >= 0) dst[slot] = x;
  }
  __syncthreads();
  return K;
}

// Merge the S tile lists of one row and publish its kept set in rank order,
// its normaliser, and -- for the rows an accept test reads -- p'(x) of the
// drafted token.  Only list entries >= the row's largest tile tau can be in
// its top_k; they are gathered (a few more than top_k in practice) and
// ranked.  If they would overflow the LDS list, the list is cut back to its
// top_k every few tiles and the threshold raised.
static_assert(kCandSlots == kBlock, "one candidate slot per thread in the merge");
static_assert(kMergeCap % 64 == 0 && kMergeCap >= 2 * kUnroll * kBlock, "merge list size");
static_assert(kTopkCap * 8 + kTopkCap * 2 <= kMergeCap * 8, "the exact tile pass fits in the merge list");

template <typename T>
DEV void merge_row_block(const Params& p, const int grow) {
  __shared__ uint64_t surv[kMergeCap];
  __shared__ uint64_t top[kTopkMax];
  __shared__ int tcnt[kMaxTiles];
  __shared__ float ttau[kMaxTiles];
  __shared__ int wcnt4[kMaxTiles * kWaves];
  __shared__ unsigned hist[256];
  __shared__ int shv[3];
  __shared__ int cnt2;
  __shared__ uint64_t redu[kWaves];
  __shared__ double red[kWaves];
  __shared__ int redi[2 * kWaves];
  __shared__ double sh_mass, sh_px;
  __shared__ float sh_tau;
  __shared__ int ns;
  const int tid = threadIdx.x;
  const int K = p.top_k, S = p.S, cw = p.cand_w;
  const uint64_t* src = p.cand + (size_t)grow * S * cw;
  // drafted token read by this row's accept test, if any
  const int nt = p.B * p.rows_t;
  int j = -1, b = 0;
  if (grow < nt) { b = grow / p.rows_t; j = grow - b * p.rows_t; if (j >= p.k) j = -1; }
  else { b = (grow - nt) / p.rows_d; j = (grow - nt) - b * p.rows_d; }
  const int x = (j >= 0) ? p.tokens[(size_t)b * p.k + j] : -1;
  // tile lengths, taus and probes (S <= 64).  Filter tiles (P = 4 S) keep
  // one sublist of kWaveList slots per wave, with counts in wcnt4 (255 =
  // overflow) and tcnt[t] = 0; an exact tile (P = S), or a filter tile
  // redone here, has one list of tcnt[t] entries.
  const bool sub = p.P != S;
  int pr = 0;
  if (sub) {
    for (int i = tid; i < p.P; i += kBlock) {
      const TileStat ts = p.tiles[(size_t)grow * p.P + i];
      pr |= ts.s != ts.s;
      if ((i & (kWaves - 1)) == 0) ttau[i / kWaves] = ts.m;
      wcnt4[i] = ts.amax > kWaveList ? 255 : ts.amax;
    }
  } else if (tid < S) {
    const TileStat ts = p.tiles[(size_t)grow * S + tid];
    tcnt[tid] = ts.amax;
    ttau[tid] = ts.m;
    pr = ts.s != ts.s;
  }
  if (tid < kTopkMax) top[tid] = 0ull;
  if (tid == 0) { sh_px = 0.0; ns = 0; }
  const int probe = __syncthreads_or(pr);
  if (sub && tid < S) {
    int ov = 0;
    for (int q = 0; q < kWaves; ++q) ov |= wcnt4[tid * kWaves + q] == 255;
    tcnt[tid] = ov ? cw + 1 : 0;   // 0: sublists; cw + 1: redo
  }
  __syncthreads();
  // a filter list that overflowed (rare: many logits tie near the tile's
  // top_k-th): redo that tile exactly, in rank order, into its list
  for (int t = 0; t < S; ++t) {
    if (tcnt[t] > cw) {
      const T* row = row_ptr<T>(p, grow);
      const int start = t * p.L, end = min(start + p.L, p.V);
      int n;
      float m;
      tile_topk_rounds<T>(p, row, start, end, (end - start + kVec - 1) / kVec, grow * S + t, surv,
                          reinterpret_cast<unsigned short*>(surv + kTopkCap), &n, &m);
      if (tid == 0) { tcnt[t] = n; ttau[t] = m; }
      if (sub && tid < kWaves) wcnt4[t * kWaves + tid] = 0;   // now one list of n
      __syncthreads();
    }
  }
  if (tid < 64) {
    float tt = tid < S ? ttau[tid] : -INFINITY;
    tt = wave_max(tt);
    if (tid == 0) sh_tau = tt;
  }
  __syncthreads();
  float tau = sh_tau;
  for (int t0 = 0; t0 < S; t0 += kUnroll) {
    uint64_t key[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u;
      // slot tid of tile t: sublist tid / kWaveList, entry tid % kWaveList
      // (sublists), or entry tid of one list
      bool has = false;
      if (t < S) {
        has = tid < tcnt[t];
        if (sub && tcnt[t] == 0) has = (tid % kWaveList) < wcnt4[t * kWaves + tid / kWaveList];
      }
      key[u] = src[has ? (size_t)t * cw + tid : 0];
      if (!has) key[u] = 0ull;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool take = key[u] != 0ull && packed_val(key[u]) >= tau;
      const int slot = wave_append(take, &ns);
      if (take) surv[slot] = key[u];
    }
    __syncthreads();
    if (ns > kMergeCap - kUnroll * kBlock && t0 + kUnroll < S) {
      // cut the list back to its top_k and raise the threshold
      const int c = ns;
      const int n = block_keep_top(surv, c, K, top, hist, shv, &cnt2);
      uint64_t mn = ~0ull;
      for (int i = tid; i < n; i += kBlock) { surv[i] = top[i]; mn = top[i] < mn ? top[i] : mn; }
      mn = wave_min_t(mn);
      if ((tid & 63) == 0) redu[tid >> 6] = mn;
      if (tid == 0) ns = n;
      __syncthreads();
      if (c >= K) {
        const uint64_t kth = min(min(redu[0], redu[1]), min(redu[2], redu[3]));
        tau = fmaxf(tau, packed_val(kth));
      }
      __syncthreads();
    }
  }
  // the top_k of the survivors, then their ranks by counting
  const int n = block_keep_top(surv, ns, K, top, hist, shv, &cnt2);
  {
    const uint64_t key = tid < n ? top[tid] : 0ull;
    int r = 0;
    for (int j = 0; j < n; ++j) r += top[j] > key;
    __syncthreads();
    if (tid < n) surv[r] = key;
    __syncthreads();
    if (tid < n) top[tid] = surv[tid];
    __syncthreads();
  }
  const float v0 = n > 0 ? packed_val(top[0]) : -INFINITY;
  const bool bad = probe || (v0 != v0) || (v0 == INFINITY) || (v0 == -INFINITY);
  const double invT = 1.0 / p.T;
  const double zm = (double)v0 * invT;
  int32_t* kidx = p.k_idx + (size_t)grow * K;
  double* ke = p.k_e + (size_t)grow * K;
  double e = 0.0;
  int idx = -1;
  if (tid < n) {
    idx = packed_idx(top[tid]);
    e = bad ? 0.0 : exp((double)packed_val(top[tid]) * invT - zm);
    kidx[tid] = idx;
    ke[tid] = e;
  }
  double Z;
  const double ex = block_exscan(e, red, &Z);   // rank-order prefix of the kept set
  int kept = n;
  double norm = Z;
  if (p.top_p < 1.0 && n > 0 && !bad) {
    // nucleus on the kept set: rank order is already probability order;
    // entry i stays iff the mass ranked before it is below top_p
    kept = block_max_i((tid < n && ex < p.top_p * Z) ? tid + 1 : 1, redi);
    if (tid == kept - 1) sh_mass = ex + e;
    __syncthreads();
    norm = sh_mass;
  }
  if (idx >= 0 && idx == x && tid < kept) sh_px = e / norm;
  __syncthreads();
  if (tid == 0) {
    p.k_cnt[grow] = kept;
    p.k_norm[grow] = norm;
    p.k_bad[grow] = bad ? 1 : 0;
    p.k_px[grow] = sh_px;
    if (p.tfilt) {
      // tree sampling reads the adjusted row as a view: v is kept iff its
      // packed key ranks at or above the last kept one
      RowNuc nu;
      nu.Z = Z; nu.N = norm; nu.M = v0;
      nu.cut = (!bad && kept > 0) ? top[kept - 1] : 0ull;
      nu.ok = (!bad && kept > 0) ? 1 : 0;
      p.nuc[grow] = nu;
    }
  }
  __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_topk_rows(Params p) {
  merge_row_block<T>(p, blockIdx.x);
}

// The drafted token whose p'(x) the row's accept test reads (-1 if none).
DEV int merge_row_token(const Params& p, int grow) {
  const int nt = p.B * p.rows_t;
  int j, b;
  if (grow < nt) { b = grow / p.rows_t; j = grow - b * p.rows_t; if (j >= p.k) j = -1; }
  else { b = (grow - nt) / p.rows_d; j = (grow - nt) - b * p.rows_d; }
  return j >= 0 ? p.tokens[(size_t)b * p.k + j] : -1;
}

// The same merge for one row in one wave (top_k <= 64, filter lists): the
// row's partials (one round of loads), the sublists' entries at or above
// the largest tile bound (one more round) into the wave's LDS list, ranks
// by counting over that list, the kept set in rank order, and its float64
// softmax (nucleus on top if asked) with DPP scans.  Returns false, having
// written nothing, for a row the wave cannot take (a tile whose list
// overflowed, or more than kWaveCand survivors); the block merge does it.
constexpr int kWaveCand = 256;   // survivors one wave ranks (four per lane)
constexpr int kWaveSubl = 16;    // sublists whose entries are loaded per round

template <typename T>
DEV bool merge_row_wave(const Params& p, int grow, uint64_t* lst, int x) {
  const int lane = threadIdx.x & 63;
  const int K = p.top_k, S = p.S, P = p.P, cw = p.cand_w;
  constexpr int BITS = sizeof(T) == 2 ? 16 : 32;
  const uint64_t* src = p.cand + (size_t)grow * S * cw;
  // one round of loads: the partials (lane holds l, l + 64, l + 128, l + 192)
  // and, unconditionally, slot `lane` of the first kWaveSubl sublists
  // (sublist i = tile i / kWaves, wave i % kWaves; masked by the counts
  // once they arrive)
  TileStat ts[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    ts[q] = p.tiles[(size_t)grow * P + (i < P ? i : 0)];
  }
  uint64_t key[kWaveSubl];
#pragma unroll
  for (int q = 0; q < kWaveSubl; ++q) {
    const int i = q < P ? q : 0;
    key[q] = src[(size_t)(i / kWaves) * cw + (i % kWaves) * kWaveList + lane];
  }
  float tau = -INFINITY;
  int cnt[4];
  bool nanr = false, over = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    cnt[q] = i < P ? ts[q].amax : 0;
    if (i < P) {
      tau = fmaxf(tau, ts[q].m);
      nanr |= ts[q].s != ts[q].s;
      over |= ts[q].amax > kWaveList;
    }
  }
  if (__ballot(over)) return false;
  tau = wave_max(tau);
  const bool bad_partial = __ballot(nanr) != 0ull;
  // entries at or above the largest tile bound (all of the row's top_k)
  int n = 0;
  for (int i0 = 0; i0 < P; i0 += kWaveSubl) {
    if (i0 > 0) {
#pragma unroll
      for (int q = 0; q < kWaveSubl; ++q) {
        const int i = i0 + q < P ? i0 + q : 0;
        key[q] = src[(size_t)(i / kWaves) * cw + (i % kWaves) * kWaveList + lane];
      }
    }
#pragma unroll
    for (int q = 0; q < kWaveSubl; ++q) {
      const int i = i0 + q;
      const int c = read_lane(cnt[(i >> 6) & 3], i & 63);   // uniform index
      const bool take = i < P && lane < c && packed_val(key[q]) >= tau;
      const uint64_t m = __ballot(take);
      const int at = n + __popcll(m & ((1ull << lane) - 1ull));
      if (take && at < kWaveCand) lst[at] = key[q];
      n += __popcll(m);
    }
  }
  if (n > kWaveCand) return false;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint64_t mine[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) mine[q] = lane + 64 * q < n ? lst[lane + 64 * q] : 0ull;
  const int nk = n < K ? n : K;
  uint64_t key_l = 0ull;   // this lane's kept entry (lane < nk)
  if (p.top_p < 1.0) {
    // the nucleus needs rank order: ranks by counting (keys are distinct)
    int rank[4] = {0, 0, 0, 0};
    for (int j = 0; j < n; ++j) {
      const uint64_t o = lst[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) rank[q] += o > mine[q];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q < n && rank[q] < nk) lst[rank[q]] = mine[q];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    key_l = lane < nk ? lst[lane] : 0ull;
  } else {
    // any fixed order will do: the top_k-th largest key by radix selects
    // (value bits, then index bits among the ties); the kept entries are
    // compacted in list order
    uint64_t thr = 0ull;
    if (n > K) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hi[q] = (uint32_t)(mine[q] >> 32);
      const uint32_t h = wave_kth_key<4, BITS>(hi, K);
      int gt = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gt += __popcll(__ballot(hi[q] > h));
        lo[q] = hi[q] == h ? (uint32_t)mine[q] : 0u;
      }
      const uint32_t l = wave_kth_key<4, 32>(lo, K - gt);
      thr = ((uint64_t)h << 32) | l;
    }
    int at = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool kp = lane + 64 * q < n && mine[q] >= thr;
      const uint64_t m = __ballot(kp);
      const int pos = at + __popcll(m & ((1ull << lane) - 1ull));
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (kp) lst[pos] = mine[q];
      at += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    key_l = lane < nk ? lst[lane] : 0ull;
  }
  const float v0 = nk > 0 ? packed_val(wave_max_t(key_l)) : -INFINITY;
  const bool bad = bad_partial || (v0 != v0) || (v0 == INFINITY) || (v0 == -INFINITY);
  const double invT = 1.0 / p.T;
  const double zm = (double)v0 * invT;
  double e = 0.0;
  int idx = -1;
  if (lane < nk) {
    idx = packed_idx(key_l);
    e = bad ? 0.0 : exp((double)packed_val(key_l) * invT - zm);
    p.k_idx[(size_t)grow * K + lane] = idx;
    p.k_e[(size_t)grow * K + lane] = e;
  }
  const double inc = wave_scan(e, 0.0, [](double a, double b2) { return a + b2; });
  const double Z = read_lane(inc, 63);
  int kept = nk;
  double norm = Z;
  if (p.top_p < 1.0 && nk > 0 && !bad) {
    const double ex = lane_before(inc, 0.0);
    kept = wave_max_t((lane < nk && ex < p.top_p * Z) ? lane + 1 : 1);
    norm = read_lane(inc, kept - 1);
  }
  const uint64_t hit = __ballot(idx >= 0 && idx == x && lane < kept);
  const double px = hit ? read_lane(e, __ffsll((unsigned long long)hit) - 1) / norm : 0.0;
  // tree sampling: the row as a view (kept iff the packed key is at least
  // the smallest kept one; the kept lanes are 0..kept-1)
  const uint64_t cut = p.tfilt ? wave_min_t(lane < kept ? key_l : ~0ull) : 0ull;
  if (lane == 0) {
    p.k_cnt[grow] = kept;
    p.k_norm[grow] = norm;
    p.k_bad[grow] = bad ? 1 : 0;
    p.k_px[grow] = px;
    if (p.tfilt) {
      RowNuc nu;
      nu.Z = Z; nu.N = norm; nu.M = v0;
      nu.cut = (!bad && kept > 0) ? cut : 0ull;
      nu.ok = (!bad && kept > 0) ? 1 : 0;
      p.nuc[grow] = nu;
    }
  }
  return true;
}

// One row per wave, four per workgroup; rows a wave cannot take go to the
// block merge, one after another, with the whole workgroup.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_topk_rows_w(Params p) {
  __shared__ uint64_t wl[kWaves][kWaveCand];
  __shared__ int need[kWaves];
  const int w = threadIdx.x >> 6;
  const int rows = p.B * (p.rows_t + p.rows_d);
  const int grow = blockIdx.x * kWaves + w;
  bool ok = true;
  if (grow < rows) ok = merge_row_wave<T>(p, grow, wl[w], merge_row_token(p, grow));
  if ((threadIdx.x & 63) == 0) need[w] = ok ? 0 : 1;
  __syncthreads();
  for (int q = 0; q < kWaves; ++q)
    if (need[q]) merge_row_block<T>(p, blockIdx.x * kWaves + q);
}

// The same for top_k <= 64 and k < 64, in wave 0 without barriers: one
// round of loads for everything the accept step reads (and every row's
// count and normaliser), one for the two kept sets of row n; q'(v) of p's
// entries and their vocabulary ranks by lane reads; the inverse CDF by a
// DPP scan.  The other waves only help write the outputs.
constexpr int kFinalSpec = 8;   // chains up to this k load every row's kept set in round 1

template <typename T>
__global__ __launch_bounds__(kBlock) void k_topk_final_w(Params p) {
  __shared__ int sx[64];
  __shared__ int sidx[64];
  __shared__ double sw[64];
  __shared__ int sh_n, sh_st, sh_y, sh_np, sh_bad;
  __shared__ double sh_S;
  const int b = blockIdx.x;
  const int k = p.k, V = p.V, K = p.top_k, tid = threadIdx.x, lane = tid & 63;
  const int nrows = p.rows_t + p.rows_d;
  if (tid < 64) {
    int bad = 0;
    for (int r = lane; r < nrows; r += 64)
      bad |= p.k_bad[r < p.rows_t ? trow(p, b, r) : drow(p, b, r - p.rows_t)];
    const int j = lane < k ? lane : 0;
    const int jt = lane <= k ? lane : 0;
    const int xj = p.tokens[(size_t)b * k + j];
    const double a = p.k_px[trow(p, b, j)], bq = p.k_px[drow(p, b, j)];
    const double u = (double)p.u[(size_t)b * k + j];
    const double ur = (double)p.ur[b];
    const int cntp = p.k_cnt[trow(p, b, jt)];
    const double normp_l = p.k_norm[trow(p, b, jt)];
    const int cntq = p.k_cnt[drow(p, b, j)];
    const double normq_l = p.k_norm[drow(p, b, j)];
    // short chains: the kept sets of every target and draft row as well
    // (entry `lane`), so that row n's are in registers once n is known
    int tidx[kFinalSpec + 1], didx[kFinalSpec];
    double te[kFinalSpec + 1], de[kFinalSpec];
    if (k <= kFinalSpec) {
      const int e = lane < K ? lane : 0;
#pragma unroll
      for (int r = 0; r <= kFinalSpec; ++r) {
        const size_t gt = (size_t)trow(p, b, r <= k ? r : 0) * K + e;
        tidx[r] = p.k_idx[gt];
        te[r] = p.k_e[gt];
        if (r < kFinalSpec) {
          const size_t gd = (size_t)drow(p, b, r < k ? r : 0) * K + e;
          didx[r] = p.k_idx[gd];
          de[r] = p.k_e[gd];
        }
      }
    }
    if (lane < k) sx[lane] = xj;
    const bool anybad = __ballot(bad != 0) != 0ull;
    if (lane == 0) sh_bad = anybad;
    if (!anybad) {
      const bool inv = lane < k && (xj < 0 || xj >= V);
      bool acc = true;
      if (lane < k && !inv) acc = bq > 0.0 ? (u < fmin(1.0, a / bq)) : (a > 0.0);
      int st;
      const int n = first_failure(lane < k && (inv || !acc), inv, k, &st);
      const bool hq = n < k;
      const int np = read_lane(cntp, n);
      const double normp = read_lane(normp_l, n);
      const int nq = hq ? read_lane(cntq, hq ? n : 0) : 0;
      const double normq = hq ? read_lane(normq_l, n) : 1.0;
      int pidx_l, qidx_l;
      double pe_l, qe_l;
      if (k <= kFinalSpec) {
        // loaded with round 1 for every row n could be
        pidx_l = tidx[0]; pe_l = te[0]; qidx_l = didx[0]; qe_l = de[0];
#pragma unroll
        for (int r = 1; r <= kFinalSpec; ++r) {
          if (r == n) { pidx_l = tidx[r]; pe_l = te[r]; }
          if (r < kFinalSpec && r == n) { qidx_l = didx[r]; qe_l = de[r]; }
        }
      } else {
        const size_t gp = (size_t)trow(p, b, n) * K, gq = (size_t)drow(p, b, hq ? n : 0) * K;
        const int e = lane < K ? lane : 0;
        pidx_l = p.k_idx[gp + e];
        pe_l = p.k_e[gp + e];
        qidx_l = p.k_idx[gq + e];
        qe_l = p.k_e[gq + e];
      }
      const int pidx = lane < np ? pidx_l : -1;
      const double pa = lane < np ? pe_l / normp : 0.0;
      double qa = 0.0;
      for (int i = 0; i < nq; ++i) {
        const int qi = read_lane(qidx_l, i);
        const double qv = read_lane(qe_l, i);
        if (qi == pidx) qa = qv / normq;
      }
      const double d = pa - qa;
      double w = hq ? (d > 0.0 ? d : 0.0) : pa;
      if (lane >= np) w = 0.0;
      int rank = 0;
      for (int i = 0; i < np; ++i) rank += read_lane(pidx, i) < pidx;   // vocabulary order
      if (lane < np) { sidx[rank] = pidx; sw[rank] = w; }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      double ws = lane < np ? sw[lane] : 0.0;
      const int yi = lane < np ? sidx[lane] : -1;
      double inc = wave_scan(ws, 0.0, [](double x, double y) { return x + y; });
      double S = read_lane(inc, 63);
      if (!(S > 0.0)) {   // empty residual: draw from p'_n
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (lane < np) sw[rank] = pa;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        ws = lane < np ? sw[lane] : 0.0;
        inc = wave_scan(ws, 0.0, [](double x, double y) { return x + y; });
        S = read_lane(inc, 63);
      }
      const double ex = lane_before(inc, 0.0);
      const double t = ur * S;
      const uint64_t m1 = __ballot(lane < np && ws > 0.0 && ex + ws > t);
      const uint64_t m2 = __ballot(lane < np && ws > 0.0);
      const int ys = m1 ? __ffsll((unsigned long long)m1) - 1 : (m2 ? 63 - __clzll((long long)m2) : -1);
      const int y = ys >= 0 ? read_lane(yi, ys) : -1;
      if (lane == 0) { sh_n = n; sh_st = st; sh_y = y; sh_np = np; sh_S = S; }
    }
  }
  __syncthreads();
  if (sh_bad) { emit_invalid(p, b, 4); return; }
  if (p.resid_probs) {
    float* rp = p.resid_probs + (size_t)b * V;
    for (int v = tid; v < V; v += kBlock) rp[v] = 0.f;
    __syncthreads();
    if (tid < sh_np) rp[sidx[tid]] = (float)(sw[tid] / sh_S);
  }
  emit_tokens(p, b, sx, sh_n, sh_y, sh_st);
}

// Accept step and residual draw of one sequence from the published kept sets.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_topk_final(Params p) {
  __shared__ int qidx[kTopkMax];
  __shared__ double qe[kTopkMax];
  __shared__ int sidx[kTopkMax];
  __shared__ double sw[kTopkMax];
  __shared__ int sidx_all[kTopkMax];
  __shared__ double red[kWaves];
  __shared__ int sx[64];
  __shared__ int redi[2 * kWaves];
  __shared__ int sh_n, sh_st;
  const int b = blockIdx.x;
  const int k = p.k, V = p.V, tid = threadIdx.x, K = p.top_k;
  const int nrows = p.rows_t + p.rows_d;
  // round 1: row validity, drafted tokens, uniforms, p'(x) and q'(x)
  int bad = 0;
  for (int r = tid; r < nrows; r += kBlock)
    bad |= p.k_bad[r < p.rows_t ? trow(p, b, r) : drow(p, b, r - p.rows_t)];
  int xj = 0;
  double a = 0.0, bq = 0.0, u = 0.0;
  const double ur = (double)p.ur[b];
  if (tid < k) {
    xj = p.tokens[(size_t)b * k + tid];
    a = p.k_px[trow(p, b, tid)];
    bq = p.k_px[drow(p, b, tid)];
    u = (double)p.u[(size_t)b * k + tid];
    sx[tid] = xj;
  }
  if (__syncthreads_or(bad)) { emit_invalid(p, b, 4); return; }
  if (tid < 64) {
    const bool inv = tid < k && (xj < 0 || xj >= V);
    bool acc = true;
    if (tid < k && !inv) acc = bq > 0.0 ? (u < fmin(1.0, a / bq)) : (a > 0.0);
    int st;
    const int n = first_failure(tid < k && (inv || !acc), inv, k, &st);
    if (tid == 0) { sh_n = n; sh_st = st; }
  }
  __syncthreads();
  const int n = sh_n;
  // round 2: the kept sets of p'_n and (n < k) q'_n
  const int gp = trow(p, b, n);
  const int np = p.k_cnt[gp];
  const double normp = p.k_norm[gp];
  int pidx = -1;
  double pe = 0.0;
  if (tid < np) { pidx = p.k_idx[(size_t)gp * K + tid]; pe = p.k_e[(size_t)gp * K + tid]; }
  int nq = 0;
  double normq = 1.0;
  if (n < k) {
    const int gq = drow(p, b, n);
    nq = p.k_cnt[gq];
    normq = p.k_norm[gq];
    if (tid < nq) { qidx[tid] = p.k_idx[(size_t)gq * K + tid]; qe[tid] = p.k_e[(size_t)gq * K + tid]; }
  }
  if (tid < np) sidx_all[tid] = pidx;
  __syncthreads();
  double w = 0.0;
  int rank = 0;
  if (tid < np) {
    const double pa = pe / normp;
    if (n < k) {
      double qa = 0.0;
      for (int i = 0; i < nq; ++i) if (qidx[i] == pidx) { qa = qe[i] / normq; break; }
      const double d = pa - qa;
      w = d > 0.0 ? d : 0.0;
    } else {
      w = pa;
    }
    for (int i = 0; i < np; ++i) rank += sidx_all[i] < pidx;   // vocabulary order
    sidx[rank] = pidx;
    sw[rank] = w;
  }
  __syncthreads();
  // inverse CDF in vocabulary order over the target's kept entries
  double ws = tid < np ? sw[tid] : 0.0;
  double S;
  double ex = block_exscan(ws, red, &S);
  bool p_only = n == k;
  if (!(S > 0.0)) {   // empty residual: draw from p'_n
    __syncthreads();
    if (tid < np) sw[rank] = pe / normp;
    __syncthreads();
    ws = tid < np ? sw[tid] : 0.0;
    ex = block_exscan(ws, red, &S);
    p_only = true;
  }
  const double t = ur * S;
  int ymin = INT_MAX, ylast = -1;
  if (tid < np && ws > 0.0) {
    if (ex + ws > t) ymin = tid;
    ylast = tid;
  }
  block_minmax(ymin, ylast, redi);
  const int ys = ymin != INT_MAX ? ymin : ylast;
  const int y = ys >= 0 ? sidx[ys] : -1;
  if (p.resid_probs) {
    float* rp = p.resid_probs + (size_t)b * V;
    for (int v = tid; v < V; v += kBlock) rp[v] = 0.f;
    __syncthreads();
    if (tid < np) rp[sidx[tid]] = (float)(ws / S);
  }
  (void)p_only;
  emit_tokens(p, b, sx, n, y, sh_st);
}

// ================================================================== plain and nucleus sampling
//
// After the stream pass (float64 row sums per tile) -- and, for the nucleus,
// the exact cut per row (k_topp_rows) -- two kernels finish a call:
//   k_resid_s     grid (segment, sequence): every workgroup of a sequence
//                 redoes its accept step (row views from the tile partials,
//                 2k logits), then sums the residual max(0, p' - q') (or p'_k
//                 after full acceptance) over its segment of kResidSeg
//                 entries in float64 (for a nucleus target row k_nuc_rows
//                 settled, from its kept entries in the row's candidate
//                 buffer); segment 0 publishes the sequence state.
//   k_resid_final grid (segment, sequence): every workgroup finds S' and the
//                 segment where ur * S' falls; that segment's workgroup draws
//                 the token; all of them write resid_probs if asked.

// The residual mass of segment seg of a row pair from the target row's
// candidate buffer, for a row k_nuc_rows settled (every entry its nucleus
// keeps is a candidate), in one wave: the segment is half u = seg % 2 of
// round seg / 2, whose entries sit in each wave region of the buffer at the
// place the round record gives (the first half's before the second's); each
// kept entry's weight is the one resid_nuc_sparse gives it, with the draft's
// logit read at its index.  Returns the segment's sum (fixed order: the
// regions' entries in turn, 64 at a time, then the wave sum).
template <typename T>
DEV double resid_nuc_cand(const Params& p, int tg, const RowView& pr, const RowView& qr, bool hasq,
                          double cs, const double* tab, int seg) {
  constexpr int kReg = kNucSlotEntries / kNucWaves;
  const int lane = threadIdx.x & 63, V = p.V;
  const int r = seg >> 1, half = seg & 1;
  const uint32_t* bval = reinterpret_cast<const uint32_t*>(p.nucc + (size_t)tg * kNucSlotEntries);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(bval, kNucSlotEntries * 4);
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(bval + kNucSlotEntries, kNucSlotEntries * 4);
  const uint64_t ml = p.nucm[((size_t)tg * kNucWaves + (lane < kNucWaves ? lane : 0)) * p.nuc_rounds + r];
  int st[kNucWaves], len[kNucWaves], total = 0;
#pragma unroll
  for (int q = 0; q < kNucWaves; ++q) {
    const uint64_t m = read_lane(ml, q);
    const int s0 = (int)(m & 0xffffu), c0 = (int)((m >> 16) & 0xffffu), c = (int)((m >> 32) & 0xffffu);
    st[q] = q * kReg + s0 + (half ? c0 : 0);
    len[q] = half ? c - c0 : c0;
    total += len[q];
  }
  double t = 0.0;
  for (int j0 = 0; j0 < total; j0 += 64) {
    int o = j0 + lane, slot = -1;
#pragma unroll
    for (int q = 0; q < kNucWaves; ++q) {
      if (slot < 0 && o < len[q]) slot = st[q] + o;
      o -= len[q];
    }
    // (a lane past the segment reads past the buffer: the resource returns 0)
    const int off = slot >= 0 ? slot * 4 : kNucSlotEntries * 4;
    const float l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, 0));
    const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, off, 0, 0);
    if (slot >= 0 && v >= 0 && v < V && pack(l, v) >= pr.cut) {
      double w = exp2_64_l(l, cs, pr.nmc, tab) * pr.inv;
      if (hasq) {
        w -= prob_from(qr, cs, tab, Io<T>::at((const T*)qr.row, v), v);
        w = w > 0.0 ? w : 0.0;
      }
      t += w;
    }
  }
  return wave_sum(t);
}

template <typename T, int FILT>
__global__ __launch_bounds__(kBlock) void k_resid_s(Params p) {
  __shared__ double vnmc[kMaxRows], vinv[kMaxRows];
  __shared__ uint64_t vcut[kMaxRows];
  __shared__ float vlx[kMaxRows];
  __shared__ int vbad[kMaxRows];
  __shared__ double red[kWaves];
  __shared__ double tab[kExpTab];
  __shared__ int sh_n, sh_st;
  // segments blockIdx.x * rgrp .. + rgrp - 1 (the setup and the accept
  // tests once for all of them)
  const int b = blockIdx.y, seg0 = blockIdx.x * p.rgrp, tid = threadIdx.x;
  const int k = p.k, V = p.V, nrows = p.rows_t + p.rows_d;
  const double cs = kExpScale * kLog2e / p.T;
  auto row_of = [&](int r) { return r < p.rows_t ? trow(p, b, r) : drow(p, b, r - p.rows_t); };
  // one round of loads, all unconditional (clamped indices): drafted
  // tokens, uniforms, the drafted tokens' logits (recorded by the streaming
  // pass) and the row views (nrows <= kMaxRows < kBlock: one row per thread)
  const int ti = tid < k ? tid : 0, ri = tid < nrows ? tid : 0;
  const double tv = exp2_table_fetch();
  const int xj_l = p.tokens[(size_t)b * k + ti];
  const float uj_l = p.u[(size_t)b * k + ti];
  const float lx = p.row_lx[row_of(ri)];
  int internal = 0;
  if constexpr (FILT == kFiltTopp) {
    const RowNuc nu = p.nuc[row_of(ri)];
    if (tid < nrows) {
      vnmc[tid] = -(double)nu.M * cs; vinv[tid] = 1.0 / nu.N; vcut[tid] = nu.cut; vbad[tid] = nu.ok != 1;
      internal = nu.ok == 2;
    }
  } else {
    // four partials per lane: short float64 chains for this latency-bound kernel
    combine_rows<true, 4>(p, nrows, row_of, [&](int r, float M, int, double Z, int bad) {
      vnmc[r] = -(double)M * cs; vinv[r] = 1.0 / Z; vcut[r] = 0ull; vbad[r] = bad;
    });
  }
  if (tid < nrows) vlx[tid] = lx;
  const int xj = tid < k ? xj_l : 0;
  const float uj = tid < k ? uj_l : 0.f;
  // a lazy call read the rows after position 0 only where x_0 was accepted
  const bool all_read = p.lazy != 3 || p.go[b] != 0;
  exp2_table_store(tab, tv);
  int mybad = 0;
  for (int r = tid; r < nrows; r += kBlock)
    if (all_read || r == 0 || r == p.rows_t) mybad |= vbad[r];
  internal = __syncthreads_or(internal);
  if (__syncthreads_or(mybad)) {
    if (seg0 == 0) {
      emit_invalid(p, b, 4 | (internal ? kStatusInternal : 0));
      if (tid == 0) p.seq[b].n = -1;
    }
    return;
  }
  // the accept tests (no memory access)
  if (tid < 64) {
    const bool inv = tid < k && (xj < 0 || xj >= V);
    bool acc = true;
    if (tid < k && !inv) {
      const int rd = p.rows_t + tid;
      const RowView vt{nullptr, vnmc[tid], vinv[tid], vcut[tid]};
      const RowView vd{nullptr, vnmc[rd], vinv[rd], vcut[rd]};
      const double a = prob_from(vt, cs, tab, vlx[tid], xj);
      const double q = prob_from(vd, cs, tab, vlx[rd], xj);
      acc = q > 0.0 ? ((double)uj < fmin(1.0, a / q)) : (a > 0.0);
    }
    int st;
    const int n = first_failure(tid < k && (inv || !acc), inv, k, &st);
    if (tid == 0) { sh_n = n; sh_st = st; }
  }
  __syncthreads();
  const int n = sh_n;
  // residual mass of this segment
  const RowView pr{row_ptr<T>(p, trow(p, b, n)), vnmc[n], vinv[n], vcut[n]};
  RowView qr{nullptr, 0.0, 1.0, 0ull};
  if (n < k) {
    const int rd = p.rows_t + n;
    qr = RowView{row_ptr<T>(p, drow(p, b, n)), vnmc[rd], vinv[rd], vcut[rd]};
  }
  if constexpr (FILT == kFiltTopp) {
    // a target row k_nuc_rows settled: its kept entries from its candidate
    // buffer, wave w taking segments seg0 + w, seg0 + w + kWaves, ...
    if (p.nuc_keep && !p.keep_w && p.nuck[trow(p, b, n)] != 0) {
      const int w = tid >> 6;
      for (int seg = seg0 + w; seg < seg0 + p.rgrp && seg < p.S2; seg += kWaves) {
        const double t = resid_nuc_cand<T>(p, trow(p, b, n), pr, qr, n < k, cs, tab, seg);
        if ((tid & 63) == 0) p.spart[(size_t)b * p.S2 + seg] = t;
      }
      if (tid == 0 && seg0 == 0) {
        SeqState ss;
        ss.nmc_p = pr.nmc; ss.inv_p = pr.inv; ss.cut_p = pr.cut;
        ss.nmc_q = qr.nmc; ss.inv_q = qr.inv; ss.cut_q = qr.cut;
        ss.n = n; ss.st = sh_st; ss.node = n; ss.hasq = n < k;
        p.seq[b] = ss;
      }
      return;
    }
  }
  for (int seg = seg0; seg < seg0 + p.rgrp && seg < p.S2; ++seg) {
  const int pos0 = seg * kResidSeg + tid * kVec;
  double w[kVec];
  double t;
  if (FILT == kFiltTopp && !p.keep_w) {
    __shared__ float nq_lp[kWaves * 128], nq_lq[kWaves * 128];
    __shared__ int nq_ix[kWaves * 128];
    const int wo = (tid >> 6) * 128;
    t = resid_nuc_sparse<T>(pr, qr, n < k, cs, tab, V, p.aligned, pos0, nq_lp + wo, nq_lq + wo,
                            nq_ix + wo);
  } else {
    t = resid_weights<T>(pr, qr, n < k, cs, tab, V, p.aligned, pos0, w);
  }
  // small problems: the weights themselves, for k_resid_final
  if (p.keep_w) {
    d2* wp = reinterpret_cast<d2*>(p.wpart + ((size_t)b * p.S2 + seg) * kResidSeg + tid * kVec);
#pragma unroll
    for (int q = 0; q < kVec / 2; ++q) wp[q] = d2{w[2 * q], w[2 * q + 1]};
  }
  const double tot = block_sum(t, red);
  if (tid == 0) {
    p.spart[(size_t)b * p.S2 + seg] = tot;
    if (seg == 0) {
      SeqState ss;
      ss.nmc_p = pr.nmc; ss.inv_p = pr.inv; ss.cut_p = pr.cut;
      ss.nmc_q = qr.nmc; ss.inv_q = qr.inv; ss.cut_q = qr.cut;
      ss.n = n; ss.st = sh_st; ss.node = n; ss.hasq = n < k;
      p.seq[b] = ss;
    }
  }
  }
}

constexpr int kSegStage = 1024;   // residual segment masses held in registers (per sequence)

template <typename T, int FILT>
__global__ __launch_bounds__(kBlock) void k_resid_final(Params p) {
  __shared__ double red[kWaves];
  __shared__ double tab[kExpTab];
  __shared__ int sx[64];
  __shared__ int redi[2 * kWaves];
  __shared__ double sh_base;
  constexpr int kPer = kSegStage / kBlock;   // segment masses per thread
  // one workgroup per segment when resid_probs is written or the weights
  // were kept; otherwise one per sequence (gridDim.x == 1), which draws in
  // the segment it finds
  const int b = blockIdx.y, tid = threadIdx.x;
  int seg = blockIdx.x;
  const int S2 = p.S2, V = p.V, k = p.k;
  const bool single = gridDim.x == 1 && S2 > 1;
  const bool use_w = p.keep_w && !single;
  const double cs = kExpScale * kLog2e / p.T;
  // one round of loads, all unconditional: sequence state, ur, the segment
  // masses this thread owns ([tid*per, (tid+1)*per)), drafted tokens, and
  // this workgroup's own segment weights (written by k_resid_s)
  const SeqState ss = p.seq[b];
  const double tv = exp2_table_fetch();
  const double ur = (double)p.ur[b];
  const double* spg = p.spart + (size_t)b * S2;
  const int per = (S2 + kBlock - 1) / kBlock;
  double sm[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int s2 = tid * per + q;
    const bool ok = q < per && s2 < S2;
    sm[q] = spg[ok ? s2 : 0];
    if (!ok) sm[q] = 0.0;
  }
  const int xl = p.tokens[(size_t)b * k + (tid < k ? tid : 0)];
  double w[kVec];
  if (use_w) {
    const d2* wp = reinterpret_cast<const d2*>(p.wpart + ((size_t)b * S2 + seg) * kResidSeg + tid * kVec);
#pragma unroll
    for (int q = 0; q < kVec / 2; ++q) { const d2 x = wp[q]; w[2 * q] = x.x; w[2 * q + 1] = x.y; }
  }
  if (!p.tree && tid < k) sx[tid] = xl;   // chain: k <= 64
  if (ss.n < 0) return;
  const int n = ss.n, node = ss.node;
  const bool hasq = ss.hasq != 0;
  // S' = sum of the segment masses (a thread owning more than kPer reads
  // the rest from global memory: vocabularies above kSegStage * kResidSeg)
  double lsum = 0.0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) lsum += sm[q];
  for (int q = kPer; q < per; ++q) { const int s2 = tid * per + q; if (s2 < S2) lsum += spg[s2]; }
  double S;
  const double ex0 = block_exscan(lsum, red, &S);
  if (!(S > 0.0)) {
    // empty residual: p'_n, drawn and written by one workgroup
    if (seg != 0) return;
    exp2_table_store(tab, tv);
    const RowView pr{row_ptr<T>(p, trow(p, b, node)), ss.nmc_p, ss.inv_p, ss.cut_p};
    const RowView none{nullptr, 0.0, 1.0, 0ull};
    double S1;
    const int y = resid_draw<T>(pr, cs, tab, V, p.aligned, ur, red, redi, &S1);
    if (p.resid_probs) {
      float* rp = p.resid_probs + (size_t)b * V;
      for (int c0 = 0; c0 < V; c0 += kResidSeg) {
        double w1[kVec];
        resid_weights<T>(pr, none, false, cs, tab, V, p.aligned, c0 + tid * kVec, w1);
#pragma unroll
        for (int q = 0; q < kVec; ++q) {
          const int v = c0 + tid * kVec + q;
          if (v < V) rp[v] = (float)(w1[q] / S1);
        }
      }
    }
    emit_final(p, b, sx, n, y, ss.st);
    return;
  }
  // the segment where t = ur * S' falls (or the last one with mass)
  const double t = ur * S;
  int cross = INT_MAX, lastpos = -1;
  {
    double run = ex0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int s2 = tid * per + q;
      if (q < per && s2 < S2) {
        if (sm[q] > 0.0) lastpos = s2;
        if (cross == INT_MAX && run + sm[q] > t) cross = s2;
        run += sm[q];
      }
    }
    for (int q = kPer; q < per; ++q) {
      const int s2 = tid * per + q;
      if (s2 < S2) {
        const double ps = spg[s2];
        if (ps > 0.0) lastpos = s2;
        if (cross == INT_MAX && run + ps > t) cross = s2;
        run += ps;
      }
    }
  }
  block_minmax(cross, lastpos, redi);
  const int c = cross != INT_MAX ? cross : lastpos;
  if (tid == c / per) {
    double run = ex0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) if (q < per && tid * per + q < c) run += sm[q];
    for (int q = kPer; q < per && tid * per + q < c; ++q) run += spg[tid * per + q];
    sh_base = run;
  }
  if (single) seg = c;
  if (seg != c && !p.resid_probs) return;
  __syncthreads();
  const double base = sh_base;
  const int c0 = seg * kResidSeg;
  if (!use_w) {
    // large problems (or one workgroup per sequence): recompute this
    // segment's weights
    exp2_table_store(tab, tv);
    const RowView pr{row_ptr<T>(p, trow(p, b, node)), ss.nmc_p, ss.inv_p, ss.cut_p};
    const RowView qr{hasq ? row_ptr<T>(p, drow(p, b, node)) : nullptr, ss.nmc_q, ss.inv_q, ss.cut_q};
    resid_weights<T>(pr, qr, hasq, cs, tab, V, p.aligned, c0 + tid * kVec, w);
  }
  if (seg == c) {
    double tl = 0.0;
#pragma unroll
    for (int q = 0; q < kVec; ++q) tl += w[q];
    double tc;
    const double ex = block_exscan(tl, red, &tc);
    const int y = pick_in_chunk(base, ex, w, c0, t, redi);
    emit_final(p, b, sx, n, y, ss.st);
  }
  if (p.resid_probs) {
    float* rp = p.resid_probs + (size_t)b * V;
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      const int v = c0 + tid * kVec + q;
      if (v < V) rp[v] = (float)(w[q] / S);
    }
  }
}

// ================================================================== tree sampling
//
// Modified rejection sampling down a token tree: the children of the
// accepted node are tried in index order against a running target, which a
// rejected child replaces by the renormalised residual.  With p' and q' the
// node's adjusted target and draft rows, the running target after some
// rejected children is r = max(0, p' - c q') / D: (c, D) = (0, 1) at first,
// and a rejection gives (c, D) <- (c + D, F(c + D)), F(c) = sum_v max(0,
// p'(v) - c q'(v)), unless F(c + D) = 0 (then r stays), because
// max(0, r - q') = max(0, p' - (c + D) q') / D.  Every F needs a pass over
// the node's two rows, so the passes run ahead, wide: pass m (grid: segment x
// tree x node) adds one segment's share of F after m rejections at every
// node with more than m children, the states rebuilt from the earlier
// passes in a fixed order.  The walk (one workgroup per tree) then only
// reads them, unless one node rejects more than kTreePasses children.  The
// final draw is the plain-sampling draw over max(0, p' - c q') at the final
// node.

// Views of node u's target row (sv[0], sv[1]) and draft row (sv[2], sv[3]):
// -M * cs and 1 / Z from the row partials; sbad[0..1] their bad flags.
// Every thread calls it; the results are in LDS after the call.  (Four
// partials per lane, as in the residual passes, so both see the same bits.)
// With top-k or top-p (p.tfilt) every row's view comes from its RowNuc (the
// row max M, the kept mass N, the cut key): p'(v) = 2^((l - M) c) / N on the
// kept set.  scut[0..1] get the cut keys (0: no cut).
DEV void nuc_view(const Params& p, int grow, double cs, double* nmc, double* inv, uint64_t* cut, int* bad) {
  const RowNuc nu = p.nuc[grow];
  *nmc = -(double)nu.M * cs;
  *inv = 1.0 / nu.N;
  *cut = nu.cut;
  *bad = nu.ok != 1;
}
DEV void tree_views(const Params& p, int b, int u, double cs, double* sv, int* sbad, uint64_t* scut) {
  if (p.tfilt) {
    if (threadIdx.x < 2) {
      const int r = threadIdx.x;
      nuc_view(p, r == 0 ? trow(p, b, u) : drow(p, b, u), cs, &sv[2 * r], &sv[2 * r + 1], &scut[r], &sbad[r]);
    }
  } else {
    combine_rows<true, 4>(p, 2, [&](int r) { return r == 0 ? trow(p, b, u) : drow(p, b, u); },
                          [&](int r, float M, int, double Z, int bad) {
                            sv[2 * r] = -(double)M * cs;
                            sv[2 * r + 1] = 1.0 / Z;
                            scut[r] = 0ull;
                            sbad[r] = bad;
                          });
  }
  __syncthreads();
}

// Indices i < n with pred(i), in increasing order, into out; returns their
// count.  Every thread calls it.
template <typename Pred>
DEV int block_list(int n, Pred pred, int* out, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int total = 0;
  for (int base = 0; base < n; base += kBlock) {
    const int i = base + (int)threadIdx.x;
    const bool f = i < n && pred(i);
    const uint64_t msk = __ballot(f);
    if (lane == 0) wsum[w] = __popcll(msk);
    __syncthreads();
    int off = total, tot = 0;
    for (int q = 0; q < kWaves; ++q) { if (q < w) off += wsum[q]; tot += wsum[q]; }
    if (f) out[off + __popcll(msk & ((1ull << lane) - 1ull))] = i;
    total += tot;
    __syncthreads();
  }
  return total;
}

constexpr int kTreeMax = 1024;   // nodes per tree (the API's limit)
constexpr int kPassBatch = 4;    // nodes whose segment loads are in flight together

// Pass m (0-based): grid (segment, tree, G).  The nodes u with more than m
// children, listed in index order, are taken kPassBatch at a time; workgroup
// (seg, g) computes segment `seg` of F(c_m + D_m) at the nodes of batches
// g, g + G, ... (none: it returns at once).  A tree has tens of nodes with
// children, and one workgroup running them all in turn left one or two
// waves per SIMD to carry long dependent float64 chains; G is bounded by
// the largest batch count pass m can have (a node with more than m children
// has m + 1 of the other N - 1 nodes as children), and g is the slowest grid
// dimension, so the workgroups of batch 0, which every pass with work has,
// are dispatched first.  Each batch's segment loads are issued first, then
// its row views and states are gathered (all loads of a kind in one round).
constexpr int kPassGroups = 8;

// TFILT: the rows carry a top-k / top-p cut (p.tfilt); without it every
// cut is 0 at compile time and the pass keeps no keys in registers.
template <typename T, bool TFILT>
__global__ __launch_bounds__(kBlock) void k_tsample_pass(Params p, int m) {
  __shared__ int nch[kTreeMax], lst[kTreeMax];
  __shared__ double vv[kPassBatch][4];
  __shared__ uint64_t vc[kPassBatch][2];
  __shared__ double cn[kPassBatch];
  __shared__ double red[kPassBatch][kWaves];
  __shared__ double tab[kExpTab];
  __shared__ int wsum[kWaves];
  const int seg = blockIdx.x, b = blockIdx.y;
  const int N = p.k, V = p.V, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const double cs = kExpScale * kLog2e / p.T;
  const double tv = exp2_table_fetch();
  for (int i = tid; i < N; i += kBlock) nch[i] = 0;
  __syncthreads();
  for (int i = tid; i < N; i += kBlock) {
    const int q = p.parents[(size_t)b * N + i];
    if (i > 0 && q >= 0 && q < i) atomicAdd(&nch[q], 1);
  }
  __syncthreads();
  const int nl = block_list(N, [&](int i) { return nch[i] > m; }, lst, wsum);
  if ((int)blockIdx.z * kPassBatch >= nl) return;
  exp2_table_store(tab, tv);
  const int pos = seg * kResidSeg + tid * kVec;
  for (int l0 = blockIdx.z * kPassBatch; l0 < nl; l0 += gridDim.z * kPassBatch) {
    const int nbl = nl - l0 < kPassBatch ? nl - l0 : kPassBatch;   // this batch: lst[l0, l0 + nbl)
    // the batch's segments first: their loads are in flight while the row
    // views and states below are gathered
    // (raw words, unpacked one node at a time below)
    Group<T> gp[kPassBatch], gq[kPassBatch];
    const int nv = pos < V ? (V - pos < kVec ? V - pos : kVec) : 0;
#pragma unroll
    for (int q = 0; q < kPassBatch; ++q) {
      const int u = lst[l0 + (q < nbl ? q : 0)];
      const T* rp = row_ptr<T>(p, trow(p, b, u)) + pos;
      const T* rq = row_ptr<T>(p, drow(p, b, u)) + pos;
      if (p.aligned && nv == kVec) { gp[q].load(rp); gq[q].load(rq); }
      else { gp[q].load_part(rp, nv); gq[q].load_part(rq, nv); }
    }
    // the batch's row views; pass 0 covers every node with children, and the
    // walk reads their views from it
    auto put = [&](int r, double nmc, double inv, uint64_t cut) {
      const int l = r < nbl ? r : r - nbl, o = r < nbl ? 0 : 2;
      vv[l][o] = nmc;
      vv[l][o + 1] = inv;
      vc[l][o >> 1] = cut;
      if (m == 0 && seg == 0) {
        const size_t at = (size_t)b * N + lst[l0 + l];
        p.tview[at * 4 + o] = nmc;
        p.tview[at * 4 + o + 1] = inv;
        if (TFILT) p.tcut[at * 2 + (o >> 1)] = cut;
      }
    };
    if (TFILT) {
      if (tid < 2 * nbl) {
        const int r = tid;
        double nmc, inv;
        uint64_t cut;
        int bad;
        nuc_view(p, r < nbl ? trow(p, b, lst[l0 + r]) : drow(p, b, lst[l0 + r - nbl]), cs, &nmc, &inv, &cut, &bad);
        put(r, nmc, inv, cut);
      }
    } else {
      combine_rows<true, 4>(p, 2 * nbl,
                            [&](int r) { return r < nbl ? trow(p, b, lst[l0 + r]) : drow(p, b, lst[l0 + r - nbl]); },
                            [&](int r, float M, int, double Z, int) { put(r, -(double)M * cs, 1.0 / Z, 0ull); });
    }
    // states after m rejections (one wave per node): F of each earlier pass
    // j at u is its segment sums in a fixed order (lane l adds segments l,
    // l + 64, ...; then the wave's fixed-order sum), every pass's loads
    // issued together (unconditionally: a pass not yet run reads pass 0's
    // slots, unused)
    if (w < nbl) {
      const int u = lst[l0 + w];
      double f[kTreePasses - 1];
#pragma unroll
      for (int j = 0; j < kTreePasses - 1; ++j) f[j] = 0.0;
      for (int s2 = lane; s2 < p.S2; s2 += 64) {
#pragma unroll
        for (int j = 0; j < kTreePasses - 1; ++j)
          f[j] += p.tpart[(((size_t)b * kTreePasses + (j < m ? j : 0)) * N + u) * p.S2 + s2];
      }
      double c = 0.0, D = 1.0;
#pragma unroll
      for (int j = 0; j < kTreePasses - 1; ++j) {
        if (j < m) {
          const double F = wave_sum(f[j]);
          if (F > 0.0) { c = c + D; D = F; }
        }
      }
      if (lane == 0) cn[w] = c + D;
    }
    __syncthreads();
    double t[kPassBatch];
#pragma unroll
    for (int q = 0; q < kPassBatch; ++q) {
      const int l = q < nbl ? q : 0;
      const RowView pr{nullptr, vv[l][0], vv[l][1], TFILT ? vc[l][0] : 0ull};
      const RowView qr{nullptr, vv[l][2], vv[l][3] * cn[l], TFILT ? vc[l][1] : 0ull};
      float lp[kVec], lq[kVec];
      gp[q].opaque().values(lp);
      gq[q].opaque().values(lq);
      double wq[kVec];
      t[q] = resid_weights_of(pr, qr, true, cs, tab, pos, nv, lp, lq, wq);
    }
#pragma unroll
    for (int q = 0; q < kPassBatch; ++q) {
      const double ws = wave_sum(t[q]);
      if (lane == 0) red[q][w] = ws;
    }
    __syncthreads();
    if (tid < nbl) {
      const double tot = (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
      p.tpart[(((size_t)b * kTreePasses + m) * N + lst[l0 + tid]) * p.S2 + seg] = tot;
    }
    __syncthreads();   // vv, cn and red are rewritten by the next batch
  }
}


// The walk of one tree (one workgroup per tree): validity, the accept tests
// down the branches, the outputs but the drawn token, and the state of the
// final draw.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_tsample_walk(Params p) {
  __shared__ int par[kTreeMax], nch[kTreeMax], tok[kTreeMax], lst[kTreeMax], path[kTreeMax];
  __shared__ float uu[kTreeMax], lpx[kTreeMax], lqx[kTreeMax];
  __shared__ unsigned char rbad[2 * kTreeMax];
  __shared__ double red[kWaves];
  __shared__ double tab[kExpTab];
  __shared__ double sv[4];
  __shared__ int sbad[2];
  __shared__ uint64_t scut[2];
  __shared__ int wsum[kWaves];
  __shared__ double vw[kTreeMax][4];
  __shared__ uint64_t vcw[kTreeMax][2];
  __shared__ double Fv[kTreePasses][kTreeMax];
  __shared__ int pr_l[kTreePasses * kTreeMax];
  const int b = blockIdx.x, N = p.k, V = p.V, tid = threadIdx.x;
  const double cs = kExpScale * kLog2e / p.T;
  const double tv = exp2_table_fetch();
  // one round of loads: parents, tokens, uniforms
  int badpar = 0;
  for (int i = tid; i < N; i += kBlock) {
    const int q = p.parents[(size_t)b * N + i];
    const int ok = i > 0 ? (q >= 0 && q < i) : 1;
    par[i] = (i > 0 && ok) ? q : -1;
    badpar |= i > 0 ? !ok : (q != -1);
    tok[i] = p.tokens[(size_t)b * N + i];
    uu[i] = p.u[(size_t)b * N + i];
    nch[i] = 0;
  }
  __syncthreads();
  for (int i = tid; i < N; i += kBlock) if (par[i] >= 0) atomicAdd(&nch[par[i]], 1);
  __syncthreads();
  // the logits the tests read (child c's token in its parent's two rows),
  // the views of every node with children (written by pass 0) and, for the
  // first kTreePasses rejections at a node, F from the passes' segment
  // masses (summed in the order the passes use, so the bits are the same):
  // all issued before the walk needs any of them
  for (int i = tid; i < N; i += kBlock) {
    const int x = tok[i], q = par[i];
    float a = 0.f, d = 0.f;
    if (q >= 0 && x >= 0 && x < V) {
      a = Io<T>::at(row_ptr<T>(p, trow(p, b, q)), x);
      d = Io<T>::at(row_ptr<T>(p, drow(p, b, q)), x);
    }
    lpx[i] = a;
    lqx[i] = d;
  }
  for (int i = tid; i < N * 4; i += kBlock) {
    const int u = i >> 2;
    vw[u][i & 3] = nch[u] > 0 ? p.tview[((size_t)b * N + u) * 4 + (i & 3)] : 0.0;
  }
  for (int i = tid; i < N * 2; i += kBlock) {
    const int u = i >> 1;
    vcw[u][i & 1] = (p.tfilt && nch[u] > 0) ? p.tcut[((size_t)b * N + u) * 2 + (i & 1)] : 0ull;
  }
  const int passes = N - 1 < kTreePasses ? N - 1 : kTreePasses;
  const int npairs = block_list(passes * N, [&](int k) { return nch[k % N] > k / N; }, pr_l, wsum);
  constexpr int kFBatch = 8;
  const int fl = tid & 63;
  for (int k0 = tid >> 6; k0 < npairs; k0 += kWaves * kFBatch) {
    double t[kFBatch];
#pragma unroll
    for (int q = 0; q < kFBatch; ++q) {
      const int k = k0 + q * kWaves;
      const int pk = pr_l[k < npairs ? k : 0];
      const double* src = p.tpart + (((size_t)b * kTreePasses + pk / N) * N + pk % N) * p.S2;
      t[q] = 0.0;
      for (int s2 = fl; s2 < p.S2; s2 += 64) t[q] += src[s2];
    }
#pragma unroll
    for (int q = 0; q < kFBatch; ++q) {
      const int k = k0 + q * kWaves;
      const double f = wave_sum(t[q]);
      if (k < npairs && fl == 0) Fv[pr_l[k] / N][pr_l[k] % N] = f;
    }
  }
  // rows: every target row, and the draft row of every node with a child
  // (validity only: a NaN partial or an infinite maximum; no row sums)
  if (p.tfilt) {
    // with top-k or top-p the filter kernel judged each row (NaN / +inf in
    // any part, or no finite entry kept); the top-k filter pass's partials
    // carry bounds, not row maxima, so they cannot
    for (int r = tid; r < 2 * N; r += kBlock)
      rbad[r] = p.nuc[r < N ? trow(p, b, r) : drow(p, b, r - N)].ok != 1 ? 1 : 0;
  } else {
    combine_rows<false>(p, 2 * N, [&](int r) { return r < N ? trow(p, b, r) : drow(p, b, r - N); },
                        [&](int r, float, int, double, int bad) { rbad[r] = (unsigned char)bad; });
  }
  badpar = __syncthreads_or(badpar);
  int mybad = 0;
  for (int i = tid; i < N; i += kBlock) mybad |= rbad[i] | (nch[i] > 0 ? rbad[N + i] : 0);
  if (__syncthreads_or(mybad)) {
    emit_invalid(p, b, 4);
    if (tid == 0) p.seq[b].n = -1;
    return;
  }
  exp2_table_store(tab, tv);
  // the walk (every thread follows it; F values from wave 0)
  int st = 0, cur = 0, n = 0;
  double c = 0.0, D = 1.0;
  if (tid == 0) path[0] = 0;
  for (;;) {
    c = 0.0;   // a new node: the running target is p'
    D = 1.0;
    const int nk = block_list(N, [&](int i) { return par[i] == cur; }, lst, wsum);
    if (nk == 0) break;
    const double* vc = vw[cur];   // the views of cur's two rows
    int nxt = -1;
    for (int j = 0; j < nk; ++j) {
      const int ch = lst[j];
      const int x = tok[ch];
      bool acc = false;
      if (x < 0 || x >= V) {
        st |= 1;
      } else {
        const RowView vpa{nullptr, vc[0], vc[1], vcw[cur][0]};
        const RowView vqa{nullptr, vc[2], vc[3], vcw[cur][1]};
        const double pa = prob_from(vpa, cs, tab, lpx[ch], x);
        const double qa = prob_from(vqa, cs, tab, lqx[ch], x);
        const double dd = pa - c * qa;
        const double a = (dd > 0.0 ? dd : 0.0) / D;
        acc = qa > 0.0 ? ((double)uu[ch] < fmin(1.0, a / qa)) : (a > 0.0);
      }
      if (acc) { nxt = ch; break; }
      // rejected: F at c + D, from pass j, or from a pass of this workgroup
      double F;
      if (j < kTreePasses) {
        F = Fv[j][cur];
      } else {
        const double cn = c + D;
        const RowView pr{row_ptr<T>(p, trow(p, b, cur)), vc[0], vc[1], vcw[cur][0]};
        const RowView qr{row_ptr<T>(p, drow(p, b, cur)), vc[2], vc[3] * cn, vcw[cur][1]};
        double t = 0.0;
        for (int c0 = 0; c0 < V; c0 += kResidSeg) {
          double w[kVec];
          t += resid_weights<T>(pr, qr, true, cs, tab, V, p.aligned, c0 + tid * kVec, w);
        }
        F = block_sum(t, red);
      }
      if (F > 0.0) { c = c + D; D = F; }
    }
    if (nxt < 0) break;
    ++n;
    cur = nxt;
    if (tid == 0) path[n] = cur;
  }
  __syncthreads();
  // outputs but the drawn token (position n), and the draw's state
  int32_t* ot = p.out_tokens + (size_t)b * p.out_w;
  for (int i = tid; i < p.out_w; i += kBlock) {
    if (i != n) ot[i] = i < n ? tok[path[i + 1]] : -1;
    if (p.out_nodes) p.out_nodes[(size_t)b * p.out_w + i] = i <= n ? path[i] : -1;
  }
  tree_views(p, b, cur, cs, sv, sbad, scut);
  if (tid == 0) {
    p.acc_len[b] = n;
    const int status = st | (badpar ? 2 : 0);
    if (p.seq_status) p.seq_status[b] = status;
    SeqState ss;
    ss.nmc_p = sv[0]; ss.inv_p = sv[1]; ss.cut_p = scut[0];
    ss.nmc_q = sv[2]; ss.inv_q = sv[3] * c; ss.cut_q = scut[1];
    ss.n = n; ss.st = status; ss.node = cur; ss.hasq = c > 0.0;
    p.seq[b] = ss;
  }
}

// Residual mass per segment of the final draw: grid (segment, tree).
template <typename T>
__global__ __launch_bounds__(kBlock) void k_tsample_mass(Params p) {
  __shared__ double red[kWaves];
  __shared__ double tab[kExpTab];
  const int b = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const double cs = kExpScale * kLog2e / p.T;
  const double tv = exp2_table_fetch();
  const SeqState ss = p.seq[b];
  exp2_table_store(tab, tv);
  if (ss.n < 0) return;
  const RowView pr{row_ptr<T>(p, trow(p, b, ss.node)), ss.nmc_p, ss.inv_p, ss.cut_p};
  const RowView qr{ss.hasq ? row_ptr<T>(p, drow(p, b, ss.node)) : nullptr, ss.nmc_q, ss.inv_q, ss.cut_q};
  double w[kVec];
  const double t = resid_weights<T>(pr, qr, ss.hasq != 0, cs, tab, p.V, p.aligned, seg * kResidSeg + tid * kVec, w);
  if (p.keep_w) {
    d2* wp = reinterpret_cast<d2*>(p.wpart + ((size_t)b * p.S2 + seg) * kResidSeg + tid * kVec);
#pragma unroll
    for (int q = 0; q < kVec / 2; ++q) wp[q] = d2{w[2 * q], w[2 * q + 1]};
  }
  const double tot = block_sum(t, red);
  if (tid == 0) p.spart[(size_t)b * p.S2 + seg] = tot;
}

// ================================================================== lazy row reads
//
// The accept test of x_0 per sequence once row pair 0 has been streamed
// (the same row views and test as k_resid_s, so both take the same
// decision): go[b] = 1 when x_0 is accepted, and stage 2 then reads the
// sequence's other rows.  One wave per sequence.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_lazy_gate(Params p) {
  __shared__ double v[2][2];
  __shared__ int vbad[2];
  __shared__ double tab[kExpTab];
  const int b = blockIdx.x, tid = threadIdx.x;
  const double cs = kExpScale * kLog2e / p.T;
  const double tv = exp2_table_fetch();
  const int x = p.tokens[(size_t)b * p.k];
  const float u = p.u[(size_t)b * p.k];
  const float lt = p.row_lx[trow(p, b, 0)], ld = p.row_lx[drow(p, b, 0)];
  combine_rows<true, 4>(p, 2, [&](int r) { return r == 0 ? trow(p, b, 0) : drow(p, b, 0); },
                        [&](int r, float M, int, double Z, int bad) {
                          v[r][0] = -(double)M * cs;
                          v[r][1] = 1.0 / Z;
                          vbad[r] = bad;
                        });
  exp2_table_store(tab, tv);
  if (tid == 0) {
    bool acc = false;
    if (!vbad[0] && !vbad[1] && x >= 0 && x < p.V) {
      const RowView vt{nullptr, v[0][0], v[0][1], 0ull};
      const RowView vd{nullptr, v[1][0], v[1][1], 0ull};
      const double a = prob_from(vt, cs, tab, lt, x);
      const double q = prob_from(vd, cs, tab, ld, x);
      acc = q > 0.0 ? ((double)u < fmin(1.0, a / q)) : (a > 0.0);
    }
    p.go[b] = acc ? 1 : 0;
  }
}

// ================================================================== stream kernel

// One workgroup per tile; the host picks about four tiles per resident
// workgroup so that the last, partial wave of workgroups is short.
template <typename T, int MODE>
__global__ __launch_bounds__(kBlock) void k_stream(Params p) {
  const int tile = blockIdx.x;
  const int idx = tile / p.S;
  const int seg = tile - idx * p.S;
  int grow = idx;
  if (p.lazy == 1) {
    // lazy stage 1: row pair 0 of every sequence (targets, then drafts)
    grow = idx < p.B ? trow(p, idx, 0) : drow(p, idx - p.B, 0);
  } else if (p.lazy == 2) {
    // lazy stage 2: target rows 1..k and draft rows 1..k-1 of each sequence,
    // read only where x_0 was accepted
    const int per = 2 * p.k - 1;
    const int b = idx / per, r = idx - b * per;
    if (p.go[b] == 0) return;
    grow = r < p.k ? trow(p, b, r + 1) : drow(p, b, r - p.k + 1);
  }
  const T* row = row_ptr<T>(p, grow);
  const int start = seg * p.L;
  const int end = min(start + p.L, p.V);
  const int ngroups = (end - start + kVec - 1) / kVec;
  if constexpr (MODE == kModeTopk) {
    __shared__ uint64_t lds[kTopkLds];
    tile_topk<T>(p, row, start, end, ngroups, tile, lds);
  } else if constexpr (MODE == kModeTopkFilter) {
    tile_topk_filter<T, kFilterGroups / (int)sizeof(T)>(p, row, start, end, grow, seg);
  } else if constexpr (MODE == kModeStats64) {
    tile_stats<T, kTerms64>(p, row, start, end, grow, seg);
  } else if constexpr (MODE == kModeStatsMix) {
    tile_stats<T, kTermsMix>(p, row, start, end, grow, seg);
  } else {
    tile_argmax<T>(p, row, start, end, grow, seg);
  }
}

// ================================================================== nucleus
//
// Exact nucleus cut of one row.  Rank order is (logit desc, index asc), i.e.
// the packed u64 of pack() in descending order; e_v = exp(z_v - zmax) with
// z = l / T; the kept set is the shortest rank prefix whose mass reaches
// top_p * Z.
//
// Bins: d = fmaf(l, -1/T, zmax) in float32 is non-increasing in l, and so is
// the level-0 bin floor(d / w0) over [0, dmax); deeper levels split a
// window of level-0 bins by the packed key.  Bin order is therefore rank
// order, and everything in bins before a window ranks above every entry of
// the window.  No logit with d >= dmax = ln(V / ((1 - top_p) Z)) + 1 can be
// kept (every kept entry has probability > (1 - top_p) / V).
//
// Pass 1 (histogram) adds, per bin, the count and the mass of its entries as
// exact integers: e relative to the bin's reference, exp(-delta) with
// delta = d - (reference bin) w0 <= 3 w0, from its Taylor series to degree 9
// in float64 (remainder below 1e-16 for every w0 this search can have), and
// rounded to fixed point with fx fraction bits (fx leaves room for V
// entries).  The LDS atomics cannot change such sums, and the mass above any
// window is float64-accurate.  The bin where the cumulative mass
// reaches top_p * Z and its two neighbours form the window; pass 2 gathers
// the window's entries (no arithmetic beyond the bin), they are sorted, and
// a float64 walk from the mass above the window finds the cut.  A window
// with more than kWindowCap entries becomes the range of the next level.

constexpr int kNucUnroll = 4;   // groups per lane in flight in the row passes

struct NucState {
  float zm32, nit32;         // d = fmaf(l, nit32, zm32), nit32 = -1 / T
  float dmax, invw0;         // d >= dmax never kept; level-0 bin = d * invw0
  double w0;                 // level-0 bin width (in d)
  double zm, invT;           // float64 d = zm - l * invT
  double fx, ifx;            // fixed-point scale 2^fx and its inverse
  double above;              // exact mass ranked above the current level's range
  int level;                 // 0: bins by d; >= 1: bins by packed key
  int p0lo, p0hi;            // level-0 window (bins), used at levels >= 1
  uint64_t plo, phi;         // packed range of the current level (>= 1)
  int sh;                    // level >= 1: bin = (phi - pk) >> sh
  int c0, c1;                // current window, in bins of the current level
};

// Where one logit stands relative to the current level and window.
//   cls: -1 ranked above the window, 0 in the window, 1 below it, 2 never kept
//   *bin: its bin at the current level when it lies in the level's range, else -1
DEV int nuc_class(const NucState& s, float l, int idx, int* bin) {
  *bin = -1;
  const float d = fmaf(l, s.nit32, s.zm32);
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

// d of a bin's reference: level 0 b w0, deeper levels p0lo w0 (every bin
// of a level lies inside that level-0 window).  Its mass unit is exp(-ref).
DEV double nuc_ref(const NucState& s, int b) {
  return (double)(s.level == 0 ? b : s.p0lo) * s.w0;
}

// exp(x) for -0.1 <= x <= 0 (and slightly above 0) to float64 accuracy:
// Taylor series to degree 9.
DEV double exp_small(double x) {
  double q = fma(x, 2.7557319223985893e-06, 2.48015873015873e-05);
  q = fma(q, x, 0.0001984126984126984);
  q = fma(q, x, 0.001388888888888889);
  q = fma(q, x, 0.008333333333333333);
  q = fma(q, x, 0.041666666666666664);
  q = fma(q, x, 0.16666666666666666);
  q = fma(q, x, 0.5);
  q = fma(q, x, 1.0);
  return fma(q, x, 1.0);
}

// round(y) as an integer for 0 <= y < 2^52 (the addition rounds).
DEV unsigned long long to_fixed(double y) {
  const double t = y + 4503599627370496.0;   // 2^52
  return (unsigned long long)__double_as_longlong(t) - 0x4330000000000000ull;
}

// Pass 1 at the current level (window fields ignored): hq = fixed-point mass
// relative to the bin reference, hc = count.
template <typename T>
DEV void nuc_hist(const T* row, int V, int aligned, NucState s, unsigned long long* hq,
                  unsigned int* hc) {
  for (int b = threadIdx.x; b < kNucBins; b += kBlock) { hq[b] = 0ull; hc[b] = 0u; }
  __syncthreads();
  const int ngroups = (V + kVec - 1) / kVec, nfull = V / kVec;
  uint32_t probe = 0;
  bool nanv = false;
  for (int base = 0; base < ngroups; base += kNucUnroll * kBlock) {
    float v[kNucUnroll][kVec];
    int nv[kNucUnroll];
    load_iter<T, kNucUnroll>(row, 0, V, ngroups, nfull, aligned, base + threadIdx.x, v, nv, probe, nanv);
#pragma unroll
    for (int u = 0; u < kNucUnroll; ++u) {
      const int i0 = (base + threadIdx.x + u * kBlock) * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        if (e >= nv[u]) continue;
        const float l = v[u][e];
        int bin;
        const int cls = nuc_class(s, l, i0 + e, &bin);
        if (bin >= 0 && cls != 2) {
          const double d = fma(-(double)l, s.invT, s.zm);
          atomicAdd(&hq[bin], to_fixed(exp_small(nuc_ref(s, bin) - d) * s.fx));
          atomicAdd(&hc[bin], 1u);
        }
      }
    }
  }
  __syncthreads();
}

// Bin masses of the current level in float64, exclusive prefix over bins in
// bin order (fixed order), and the first bin whose cumulative mass (from
// s.above) reaches tgt (kNucBins - 1 if none).  *pre gets, for the window's
// first bin c0 (after the caller sets it), nothing: callers use nuc_prefix.
DEV int nuc_locate(const NucState& s, const unsigned long long* hq, double tgt, double* red,
                   int* redi) {
  constexpr int per = kNucBins / kBlock;
  double local[per];
  double tsum = 0.0;
#pragma unroll
  for (int q = 0; q < per; ++q) {
    const int b = threadIdx.x * per + q;
    local[q] = hq[b] ? (double)hq[b] * s.ifx * exp(-nuc_ref(s, b)) : 0.0;
    tsum += local[q];
  }
  double tot;
  const double ex = block_exscan(tsum, red, &tot);
  double c = s.above + ex;
  int found = INT_MAX;
#pragma unroll
  for (int q = 0; q < per; ++q) {
    c += local[q];
    if (found == INT_MAX && c >= tgt) found = threadIdx.x * per + q;
  }
  int none = -1;
  block_minmax(found, none, redi);
  return found != INT_MAX ? found : kNucBins - 1;
}

// Exact mass of the bins before bin c0 at the current level (same order and
// rounding as nuc_locate) plus s.above.
DEV double nuc_prefix(const NucState& s, const unsigned long long* hq, int c0, double* red) {
  constexpr int per = kNucBins / kBlock;
  double tsum = 0.0;
#pragma unroll
  for (int q = 0; q < per; ++q) {
    const int b = threadIdx.x * per + q;
    if (b < c0 && hq[b]) tsum += (double)hq[b] * s.ifx * exp(-nuc_ref(s, b));
  }
  return s.above + block_sum(tsum, red);
}

// Count of the current level's entries in bins [lo, hi] (exact).
DEV unsigned long long nuc_count(const unsigned int* hc, int lo, int hi, unsigned long long* redu) {
  unsigned long long c = 0;
  for (int b = threadIdx.x; b < kNucBins; b += kBlock) if (b >= lo && b <= hi) c += hc[b];
  unsigned long long t;
  block_exscan_u64(c, redu, &t);
  return t;
}

// Exact nucleus cut of one valid row (see above); fills *out.
template <typename T>
DEV void topp_search(const Params& p, const T* row, float Mrow, double Z, RowNuc* outp,
                     unsigned long long* hq, unsigned int* hc, uint64_t* win, double* red,
                     unsigned long long* redu, int* redi, int* wcnt_p) {
  int& wcnt = *wcnt_p;
  RowNuc& out = *outp;
  const int V = p.V;
  const int tid = threadIdx.x;
  const double invT = 1.0 / p.T;
  NucState s;
  s.zm32 = (float)((double)Mrow * invT);
  s.nit32 = (float)(-invT);
  // every kept entry has probability > (1 - top_p) / V, i.e. d < ln(V / ((1 - top_p) Z))
  double dmax = log((double)V / ((1.0 - p.top_p) * Z)) + 1.0;
  if (!(dmax > 1.0)) dmax = 1.0;
  s.dmax = (float)dmax;
  s.w0 = dmax / kNucBins;
  s.invw0 = (float)(1.0 / s.w0);
  s.zm = (double)Mrow * invT;
  s.invT = invT;
  int vbits = 0;
  while ((1 << vbits) < V + 1) ++vbits;
  s.fx = ldexp(1.0, min(61 - vbits, 50));   // sums < 2^62, one entry < 2^51
  s.ifx = 1.0 / s.fx;
  s.above = 0.0;
  s.level = 0; s.p0lo = 0; s.p0hi = kNucBins - 1; s.plo = 0; s.phi = ~0ull; s.sh = 0;
  s.c0 = 0; s.c1 = kNucBins - 1;

  nuc_hist<T>(row, V, p.aligned, s, hq, hc);
  const double tgt = p.top_p * Z;
  const double zm = (double)Mrow * invT;
  bool located = false;
  int result = 0;   // 1 found, -1 failed
  for (int iter = 0; iter < 64 && result == 0; ++iter) {
    if (!located) {
      const int b = nuc_locate(s, hq, tgt, red, redi);
      s.c0 = b > 0 ? b - 1 : 0;
      s.c1 = b < kNucBins - 1 ? b + 1 : kNucBins - 1;
      located = true;
    }
    const unsigned long long tw = nuc_count(hc, s.c0, s.c1, redu);
    const unsigned long long tb = nuc_count(hc, s.c1 + 1, kNucBins - 1, redu);
    const double Aw = nuc_prefix(s, hq, s.c0, red);   // exact mass ranked above the window

    if (tw <= (unsigned long long)kWindowCap) {
      // pass 2: gather the window
      if (tid == 0) wcnt = 0;
      __syncthreads();
      const int ngroups = (V + kVec - 1) / kVec, nfull = V / kVec;
      uint32_t probe = 0;
      bool nanv = false;
      for (int base = 0; base < ngroups; base += kNucUnroll * kBlock) {
        float v[kNucUnroll][kVec];
        int nv[kNucUnroll];
        load_iter<T, kNucUnroll>(row, 0, V, ngroups, nfull, p.aligned, base + tid, v, nv, probe, nanv);
        unsigned msk[kNucUnroll];
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < kNucUnroll; ++u) {
          msk[u] = 0u;
          const int i0 = (base + tid + u * kBlock) * kVec;
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            int bin;
            if (e < nv[u] && nuc_class(s, v[u][e], i0 + e, &bin) == 0) msk[u] |= 1u << e;
          }
          cnt += __popc(msk[u]);
        }
        if (__any(cnt > 0)) {
          int slot = wave_reserve(cnt, &wcnt);
#pragma unroll
          for (int u = 0; u < kNucUnroll; ++u) {
            const int i0 = (base + tid + u * kBlock) * kVec;
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
              if ((msk[u] >> e) & 1u) {
                if (slot < kWindowCap) win[slot] = pack(v[u][e], i0 + e);
                ++slot;
              }
            }
          }
        }
      }
      __syncthreads();
      const int n = min(wcnt, kWindowCap);
      const int P = next_pow2(n);
      for (int i = n + tid; i < P; i += kBlock) win[i] = 0ull;
      bitonic_desc(win, P);
      // exclusive float64 prefix of e in rank order
      const int per = (n + kBlock - 1) / kBlock;
      double tl = 0.0;
      for (int q = 0; q < per; ++q) {
        const int i = tid * per + q;
        if (i < n) tl += exp((double)packed_val(win[i]) * invT - zm);
      }
      double tot;
      const double ex = block_exscan(tl, red, &tot);
      double c = Aw + ex;
      int kept_local = 0;
      double mass_local = 0.0;
      for (int q = 0; q < per; ++q) {
        const int i = tid * per + q;
        if (i < n) {
          const double e = exp((double)packed_val(win[i]) * invT - zm);
          if (c < tgt) { kept_local = i + 1; mass_local = c + e; }
          c += e;
        }
      }
      const int kept = block_max_i(kept_local, redi);
      if (kept == 0) {
        if (s.c0 == 0) result = -1;                     // cut above this level's range
        else { s.c1 = s.c0 - 1; s.c0 = s.c0 >= 3 ? s.c0 - 3 : 0; }
      } else if (kept == n && tb > 0 && Aw + tot < tgt) {
        // every window entry is kept and so would be the next one: cut lies below
        if (s.c1 == kNucBins - 1) result = -1;          // cut below this level's range
        else { s.c0 = s.c1 + 1; s.c1 = s.c1 + 3 < kNucBins ? s.c1 + 3 : kNucBins - 1; }
      } else {
        if (tid == (kept - 1) / per) red[0] = mass_local;   // owner of the last kept entry
        __syncthreads();
        out.N = red[0];
        out.cut = win[kept - 1];
        result = 1;
      }
      __syncthreads();
    } else {
      // too many entries near the cut: the window becomes the next level's range
      unsigned long long pmin = ~0ull, pmax = 0ull;
      for (int g = tid; g * kVec < V; g += kBlock) {
        float vv[kVec];
        const int ng = load_group<T>(row, g * kVec, V, p.aligned, vv);
        for (int e = 0; e < ng; ++e) {
          const int i = g * kVec + e;
          int bin;
          if (nuc_class(s, vv[e], i, &bin) == 0) {
            const unsigned long long pk = pack(vv[e], i);
            pmin = pk < pmin ? pk : pmin;
            pmax = pk > pmax ? pk : pmax;
          }
        }
      }
      block_minmax(pmin, pmax, redu);
      s.above = Aw;
      if (s.level == 0) { s.p0lo = s.c0; s.p0hi = s.c1; }
      s.plo = pmin;
      s.phi = pmax;
      const unsigned long long span = s.phi - s.plo;
      int bits = span ? 64 - __clzll((long long)span) : 0;
      s.sh = bits > 11 ? bits - 11 : 0;
      s.level += 1;
      nuc_hist<T>(row, V, p.aligned, s, hq, hc);
      located = false;
    }
  }
  out.ok = result == 1 ? 1 : 2;
}

// Fast exact nucleus cut of one valid row; returns false (and leaves *out
// alone) when it cannot settle the row, which then takes topp_search.
// d = fmaf(l, -1/T, M/T) in float32 (monotone in l, so bins follow the rank
// order) over [0, dmax) with dmax = ln(V / ((1 - top_p) Z)) + 1 (every
// kept logit lies below it), kFastBins bins.
//  pass 1: a histogram of exp(-d) (hardware float32 exp2, rounded to 24
//          fraction bits, one LDS integer atomic per binned logit).  Its
//          masses only locate the bin where the mass from the top reaches
//          top_p Z; the window is that bin and its two neighbours.
//  pass 2: the exact float64 mass A of every logit binned above the window
//          (exp in float64 through a per-wave queue, per-lane sums in a
//          fixed order, fixed block reduction), and the window's logits
//          gathered as packed keys.
// The window is sorted in rank order and walked from A exactly as in
// topp_search.  A window that overflows, or a cut that falls outside it
// (the float32 masses misplaced it), returns false.
constexpr int kFastBins = 4096;
// Fixed-point scale of the pass-1 masses: LDS integer atomics are several
// times faster than float ones.  A bin whose sum would overflow (hundreds of
// logits within 1/4096 of the range of the maximum) only misplaces the
// window, which the walk detects.
constexpr int kFastFrac = 24;
constexpr float kFastScale = (float)(1 << kFastFrac);
constexpr int kNucPipe = 8;   // bytes per logit times groups per lane per round of the row sweeps (bf16 4, fp32 2)
static_assert(kFastBins * 4 <= kNucBins * 8, "the fast nucleus histogram fits in the exact one's");

template <typename T>
DEV bool topp_fast(const Params& p, const T* row, float Mrow, double Z, RowNuc* outp, float* hist,
                   uint64_t* win, float* aq, double* red, int* redi, int* wcnt_p, int rot) {
  int& wcnt = *wcnt_p;
  const int V = p.V, tid = threadIdx.x;
  const double invT = 1.0 / p.T;
  const float zm32 = (float)((double)Mrow * invT);
  const float nit32 = (float)(-invT);
  double dmaxd = log((double)V / ((1.0 - p.top_p) * Z)) + 1.0;
  if (!(dmaxd > 1.0)) dmaxd = 1.0;
  const float dmax = (float)dmaxd;
  const float invw = (float)((double)kFastBins / dmaxd);
  const double tgt = p.top_p * Z;
  const double zm = (double)Mrow * invT;
  unsigned* hfix = reinterpret_cast<unsigned*>(hist);
  for (int b = tid; b < kFastBins; b += kBlock) hfix[b] = 0u;
  __syncthreads();
  // pass 1.  The bin position d * invw and the weight's exponent
  // -d log2(e) + kFastFrac (the fixed point's fraction bits) are each one
  // fma of the logit; a position below kFastBins is one below dmax.  Near
  // the maximum the rounding of the fma can make it slightly negative: those
  // go to bin 0.
  const float a1 = nit32 * invw, b1 = zm32 * invw;
  const float a2 = (float)(invT * kLog2e), b2 = (float)(kFastFrac - zm * kLog2e);
  tile_groups_pipe<T, kNucPipe / (int)sizeof(T)>(row, 0, V, p.aligned, rot, [&](const auto& gr, const SlotMap&, int nv) {
    constexpr int n = sizeof(gr) / sizeof(gr[0]);
#pragma unroll
    for (int u = 0; u < n; ++u) {
      float v[kVec];
      gr[u].values(v);
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const float pos = fmaf(v[e], a1, b1);
        if (u < nv && pos < (float)kFastBins)
          atomicAdd(&hfix[(int)__builtin_amdgcn_fmed3f(pos, 0.f, (float)(kFastBins - 1))], (unsigned)(__builtin_amdgcn_exp2f(fmaf(v[e], a2, b2)) + 0.5f));
      }
    }
  });
  __syncthreads();
  // the bin where the (float32) mass from the top reaches top_p Z
  int bc;
  {
    constexpr int per = kFastBins / kBlock;
    double local[per];
    double ts = 0.0;
#pragma unroll
    for (int q = 0; q < per; ++q) { local[q] = (double)hfix[tid * per + q] * (1.0 / kFastScale); ts += local[q]; }
    double tot;
    const double ex = block_exscan(ts, red, &tot);
    double c = ex;   // bin masses are exp(-d): the same units as Z
    int found = INT_MAX;
#pragma unroll
    for (int q = 0; q < per; ++q) {
      c += local[q];
      if (found == INT_MAX && c >= tgt) found = tid * per + q;
    }
    int none = -1;
    block_minmax(found, none, redi);
    bc = found != INT_MAX ? found : kFastBins - 1;
  }
  const int lo = bc > 0 ? bc - 1 : 0;
  const int hi = bc < kFastBins - 1 ? bc + 1 : kFastBins - 1;
  // pass 2.  The logits above the window are queued per wave in LDS (ballot
  // and prefix count, no divergent float64 work); every 64 queued ones, each
  // lane adds the float64 exponential of one.  Each lane's sum follows the
  // queue order, which is fixed, so A is reproducible.
  if (tid == 0) wcnt = 0;
  __syncthreads();
  const int lane = tid & 63;
  float* q = aq + (tid >> 6) * 128;
  int qn = 0;
  double above = 0.0;
  // pass 2 classifies by d against the window's edges (monotone in the
  // logit, so the classes follow rank order; they need not repeat pass 1's
  // bins exactly: the walk below checks that the cut lies in the window)
  const float d_lo = (float)lo / invw, d_hi = fminf((float)(hi + 1) / invw, dmax);
  tile_groups_pipe<T, kNucPipe / (int)sizeof(T)>(row, 0, V, p.aligned, rot, [&](const auto& gr, const SlotMap& sm, int nv) {
    constexpr int n = sizeof(gr) / sizeof(gr[0]);
#pragma unroll
    for (int u = 0; u < n; ++u) {
      float v[kVec];
      gr[u].opaque().values(v);
      const bool live = u < nv;
      const uint64_t lm = __builtin_amdgcn_ballot_w64(live);
      // each logit's class from two compares, each straight into a scalar
      // lane mask: above the window -> the queue (slot = queue length +
      // the lanes below with the same class), inside it -> the window list
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const float d = fmaf(v[e], nit32, zm32);
        const bool ab = d < d_lo;
        const uint64_t m = __builtin_amdgcn_ballot_w64(ab) & lm;
        if (m) {
          if (ab && live)
            q[__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, (unsigned)qn))] = v[e];
          qn += __popcll(m);
          if (qn >= 64) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            above += exp2_neg(((double)q[lane] * invT - zm) * kLog2e);
            const float rest = lane < qn - 64 ? q[64 + lane] : 0.f;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            if (lane < qn - 64) q[lane] = rest;
            qn -= 64;
          }
        }
        const uint64_t wm = __builtin_amdgcn_ballot_w64(d < d_hi) & lm & ~m;
        if (wm) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&wcnt, (int)__popcll(wm));
          base = read_lane(base, 0);
          if ((wm >> lane) & 1ull) {
            const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(wm >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)wm, 0u));
            if (slot < kWindowCap) win[slot] = pack(v[e], sm.index(u, e));
          }
        }
      }
    }
  });
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (lane < qn) above += exp2_neg(((double)q[lane] * invT - zm) * kLog2e);
  const double A = block_sum(above, red);
  const int nw = wcnt;
  if (nw > kWindowCap || nw == 0) return false;
  const int P2 = next_pow2(nw);
  for (int i = nw + tid; i < P2; i += kBlock) win[i] = 0ull;
  bitonic_desc(win, P2);
  // exclusive float64 prefix of e in rank order, from A
  const int per = (nw + kBlock - 1) / kBlock;
  double tl = 0.0;
  for (int q = 0; q < per; ++q) {
    const int i = tid * per + q;
    if (i < nw) tl += exp2_neg(((double)packed_val(win[i]) * invT - zm) * kLog2e);
  }
  double tot;
  const double ex = block_exscan(tl, red, &tot);
  double c = A + ex;
  int kept_local = 0;
  double mass_local = 0.0;
  for (int q = 0; q < per; ++q) {
    const int i = tid * per + q;
    if (i < nw) {
      const double e = exp2_neg(((double)packed_val(win[i]) * invT - zm) * kLog2e);
      if (c < tgt) { kept_local = i + 1; mass_local = c + e; }
      c += e;
    }
  }
  const int kept = block_max_i(kept_local, redi);
  // the cut must fall inside the window: some entry kept, and not every one
  // unless the window reaches the end of the kept range
  const bool inside = kept > 0 && (kept < nw || A + tot >= tgt);
  if (!inside) return false;
  __syncthreads();
  if (tid == (kept - 1) / per) red[0] = mass_local;
  __syncthreads();
  outp->N = red[0];
  outp->cut = win[kept - 1];
  outp->ok = 1;
  __syncthreads();
  return true;
}

// Nucleus cut per row: topp_fast, and for a row it cannot settle (window
// overflow, or the cut outside the window: rare) the multi-level exact
// search in the same workgroup, so the chain has no launch that almost
// always has nothing to do.  After k_nuc_rows (p.nucrow) it takes only the
// rows that kernel left with ok = kNucFast, with their M and Z, and every
// other workgroup returns at once.
constexpr int kNucFast = 4;

template <typename T>
__global__ __launch_bounds__(kBlock) void k_topp_rows(Params p) {
  const int grow = blockIdx.x;
  const T* row = row_ptr<T>(p, grow);
  // the fast pass's histogram and the search's two histograms share their
  // LDS: the search starts after a barrier that ends the fast pass
  __shared__ uint64_t pool[kNucBins + kNucBins / 2];
  static_assert(kFastBins * sizeof(float) <= sizeof(pool) &&
                kNucBins * (sizeof(unsigned long long) + sizeof(unsigned)) <= sizeof(pool), "shared histograms");
  float* hist = reinterpret_cast<float*>(pool);
  unsigned long long* hq = reinterpret_cast<unsigned long long*>(pool);
  unsigned* hc = reinterpret_cast<unsigned*>(pool + kNucBins);
  __shared__ uint64_t win[kWindowCap];
  __shared__ float aq[kWaves * 128];
  __shared__ double red[kWaves];
  __shared__ unsigned long long redu[2 * kWaves];
  __shared__ int redi[2 * kWaves];
  __shared__ int wcnt;
  __shared__ float sh_M;
  __shared__ double sh_Z;
  __shared__ int sh_bad;
  RowNuc out;
  if (p.nucrow) {
    out = p.nuc[grow];
    if (out.ok != kNucFast) return;
  } else {
    auto sink = [&](int, float M, int, double Z, int bad) { sh_M = M; sh_Z = Z; sh_bad = bad; };
    combine_rows<true, 4>(p, 1, [grow](int) { return grow; }, sink);
    __syncthreads();
    out.Z = sh_Z; out.N = 0.0; out.cut = 0ull; out.ok = sh_bad ? 0 : 1; out.M = sh_M;
    if (out.ok == 0) {
      if (threadIdx.x == 0) p.nuc[grow] = out;
      return;
    }
  }
  out.N = 0.0; out.cut = 0ull;
  if (!topp_fast<T>(p, row, out.M, out.Z, &out, hist, win, aq, red, redi, &wcnt, grow * 7)) {
    __syncthreads();
    out.N = 0.0; out.cut = 0ull; out.ok = 0;
    topp_search<T>(p, row, out.M, out.Z, &out, hq, hc, win, red, redu, redi, &wcnt);
  }
  if (threadIdx.x == 0) p.nuc[grow] = out;
}


// ================================================================== nucleus rows in one read
//
// k_nuc_rows: persistent workgroups of kNB threads; workgroup g takes rows
// g, g + gridDim.x, ...  It reads each row once and settles its nucleus cut
// from the candidates it kept in a buffer in the workspace, the row's own
// where the workspace holds one per row (p.nuc_keep: each flush then also
// records where the round's entries sit, and k_resid_s takes a settled
// target row's kept entries from there), else the workgroup's (the cut
// kernels above read a row twice more after the streaming pass; on this chip
// a second sweep of a row finds nothing of the first one left in any cache).
// The buffer, about a tenth of the row's bytes, goes to memory and is read
// back twice (values only); that traffic is the price of four workgroups per
// compute unit, where the settle of one overlaps the sweeps of the others.
//  sweep   each lane keeps its running max m and the float64 sum of
//          2^((l - m) c) as tile_stats does (table exp2, float64 terms), and
//          every logit >= tau is staged in LDS and then goes to its wave's
//          region of the buffer: the raw value and its index (in separate
//          arrays).  A region fills in its wave's program order, so its
//          contents do not depend on timing.  tau is set from
//          the first round the workgroup reads (a random share of a large
//          row): the 16-bit key prefix at which the round's counts would put
//          about kNucFill candidates at or above tau over the row.
//  settle  M, Z (fixed-order block sums); the candidates' masses
//          e = exp((l - M) / T) go to a fixed-point histogram of
//          d = (M - l) / T (the bins of topp_fast) that locates the bin where
//          the mass from the top reaches top_p Z; the window is that bin and
//          its two neighbours.  The mass A of the candidates above it is
//          summed in float64 in a fixed order, the window's keys are ranked
//          and walked from A as topp_fast walks them.
// A row it cannot settle (a region full, the cut below tau or outside the
// window, a window over kNucWin entries) keeps M and Z with ok = kNucFast and
// k_topp_rows redoes it; an invalid row gets ok = 0.  Rows of more than
// kNucMaxV logits take the streaming pass and the cut kernels instead.
constexpr int kNB = 256;                      // threads per workgroup (four per CU)
constexpr int kNW = kNB / 64;                 // its waves
static_assert(kNW == kNucWaves, "the host sizes the round records by kNucWaves");
constexpr int kNucRegion = kNucSlotEntries / kNW;   // candidate slots per wave (3072)
constexpr int kNucFill = 14000;               // candidates aimed for over a row
constexpr int kNucHist = 2048;                // bins locating the cut among the candidates
constexpr int kNucWin = kNucHist / 2;         // window slots (the histogram's space, reused)
constexpr int kNucSample = 2 * kNucHist;      // 16-bit key-prefix bins of the sample (u32)
constexpr int kNucBatch = 16;                 // candidate loads in flight per lane in the settle
constexpr int kNucStage = 512;                // candidates one wave can stage in LDS per round
constexpr float kNucFix = 1048576.f;          // 2^20: fixed-point scale of the histogram's masses (e <= 1)
static_assert(kNucRegion * kNW == kNucSlotEntries, "regions tile the buffer");
static_assert(3 * kNucFill <= 2 * kNucSlotEntries, "aim at two thirds of the capacity or less");
static_assert(kNucWin % kNB == 0 && kNucSample % kNB == 0 && kNucHist % kNB == 0, "shapes");

template <typename T> struct NucShape;
// groups per lane per round: 16 KB (float32) or 8 KB (bf16) per round in
// flight per workgroup (bf16 with four would spill registers)
template <> struct NucShape<float> { static constexpr int U = 2; };
template <> struct NucShape<uint16_t> { static constexpr int U = 2; };

// Block-wide reductions for kNB threads, fixed order; every thread gets the
// result.  Each starts with a barrier, so `red` can be reused at once.
DEV float nb_max(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int q = 1; q < kNW; ++q) t = fmaxf(t, red[q]);
  return t;
}
DEV double nb_sum(double v, double* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int q = 1; q < kNW; ++q) t += red[q];
  return t;
}
template <typename I>
DEV I nb_min(I v, I* red) {
  v = wave_min_t(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  I t = red[0];
#pragma unroll
  for (int q = 1; q < kNW; ++q) t = red[q] < t ? red[q] : t;
  return t;
}
template <typename I>
DEV I nb_max_i(I v, I* red) {
  v = wave_max_t(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  I t = red[0];
#pragma unroll
  for (int q = 1; q < kNW; ++q) t = red[q] > t ? red[q] : t;
  return t;
}
// exclusive prefix in thread order (and the total) of one value per thread
template <typename V>
DEV V nb_exscan(V v, V* red, V* total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const V inc = wave_scan(v, (V)0, [](V a, V b) { return a + b; });
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  V base = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < kNW; ++q) {
    base += q < w ? red[q] : (V)0;
    tot += red[q];
  }
  *total = tot;
  return base + (inc - v);
}

// Where the element e of slot u of thread t sits in round r of a sweep.
//   split (float32 rows read whole): slot u holds two quads kNB * 4 logits
//   apart, so every 16-byte load of a wave reads 1 KB of consecutive logits;
//   otherwise slot u holds kVec consecutive logits (group r R + u kNB + t).
template <int U, bool kSplit>
DEV int nuc_index(int r, int t, int u, int e) {
  constexpr int R = U * kNB;
  if (!kSplit) return ((r * R + u * kNB + t) * kVec) + e;
  return r * R * kVec + u * (kNB * kVec) + 4 * t + (e < 4 ? e : kNB * 4 + e - 4);
}
template <int U, bool kSplit>
struct NucMap {
  int r;
  DEV int index(int u, int e) const { return nuc_index<U, kSplit>(r, (int)threadIdx.x, u, e); }
  // the thread whose slot (*u, *e) holds logit x this round, or -1 (x
  // uniform, so all of it is scalar work)
  DEV int holder(int x, int* u, int* e) const {
    constexpr int R = U * kNB;
    const int rel = x - r * R * kVec;
    if (rel < 0 || rel >= R * kVec) return -1;
    if (!kSplit) {
      const int g = rel / kVec;
      *u = g / kNB;
      *e = rel % kVec;
      return g % kNB;
    }
    *u = rel / (kNB * kVec);
    int o = rel % (kNB * kVec);
    int hi = 0;
    if (o >= kNB * 4) { o -= kNB * 4; hi = 4; }
    *e = hi + o % 4;
    return o / 4;
  }
};

// One workgroup's sweep of a whole row in rounds of U groups per lane,
// starting at round r0 (the rounds wrap around).  Aligned rows of whole
// groups go through a buffer resource spanning the row, the next round's
// loads issued before the current one is used; others element by element.
// f(v, map, tail) with tail a std::integral_constant: the round's values
// (slots past the row hold -inf; only a tail round may have such slots).
// pre() runs at the top of every round after the first, before the next
// round's loads are issued (a store it issues is then older than every load
// a later wait is for).
template <typename T, typename F, typename P>
DEV void nuc_sweep(const T* row, int V, int aligned, int r0, F&& f, P&& pre) {
  constexpr int U = NucShape<T>::U;
  constexpr int R = U * kNB;
  const int tid = threadIdx.x;
  const int ngroups = (V + kVec - 1) / kVec, nfull = V / kVec;
  const int nr = (ngroups + R - 1) / R;
  if (aligned && nfull == ngroups && nfull > 0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, V * (int)sizeof(T));
    constexpr bool kSplit = sizeof(T) == 4;
    auto load_round = [&](Group<T>* g, int r) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (kSplit) {
          const int soff = (r * R + u * kNB) * 32;
          g[u].a = __builtin_bit_cast(vf4, __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, soff, kNT));
          g[u].b = __builtin_bit_cast(vf4, __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, soff + kNB * 16, kNT));
        } else {
          g[u].load_buf(rs, (r * R + tid) * Group<T>::kBytes, u * kNB * Group<T>::kBytes);
        }
      }
    };
    Group<T> cur[U], nxt[U];
    int rc = r0;
    load_round(cur, rc);
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = cur[u].opaque();
    for (int j = 0; j < nr; ++j) {
      int rn = rc + 1;
      if (rn >= nr) rn = 0;
      if (j > 0) pre();
      if (j + 1 < nr) load_round(nxt, rn);
      float v[U][kVec];
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u].values(v[u]);
      if ((rc + 1) * R > ngroups) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if constexpr (kSplit) {
            const int pa = rc * R * kVec + u * kNB * kVec + 4 * tid;   // first logit of quad a
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (pa >= V) v[u][e] = -INFINITY;
              if (pa + kNB * 4 >= V) v[u][4 + e] = -INFINITY;
            }
          } else {
            if (rc * R + u * kNB + tid >= ngroups) {
#pragma unroll
              for (int e = 0; e < kVec; ++e) v[u][e] = -INFINITY;
            }
          }
        }
        f(v, NucMap<U, kSplit>{rc}, std::true_type{});
      } else {
        f(v, NucMap<U, kSplit>{rc}, std::false_type{});
      }
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
      rc = rn;
    }
  } else {
    for (int j = 0; j < nr; ++j) {
      int rc = r0 + j;
      if (rc >= nr) rc -= nr;
      if (j > 0) pre();
      float v[U][kVec];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = rc * R + u * kNB + tid;
        if (g < ngroups) {
          load_group<T>(row, g * kVec, V, aligned, v[u]);
        } else {
#pragma unroll
          for (int e = 0; e < kVec; ++e) v[u][e] = -INFINITY;
        }
      }
      f(v, NucMap<U, false>{rc}, std::true_type{});
    }
  }
}

// sum of exp2_64_l over n logits, the table reads of all n issued before any
// is used (the LDS latency once per batch, not once per term)
template <int N>
DEV double exp2_64_sum(const float* v, double cs, double nmc, const double* tab) {
  const double a = -cs * kTwoM20, b = -nmc * kTwoM20;
  Exp2Split e[N];
#pragma unroll
  for (int q = 0; q < N; ++q) e[q] = exp2_split(v[q], a, b);
  double tv[N];
#pragma unroll
  for (int q = 0; q < N; ++q) tv[q] = tab[e[q].j & (kExpTab - 1)];
  double s = -0.0;   // (-0.0 + x is x: no add for the first term)
#pragma unroll
  for (int q = 0; q < N; ++q) s += ldexp(tv[q] * exp2_tail(e[q].f), e[q].j >> kExpTabBits);
  return s;
}

// f(l, slot) for each candidate value of this lane in its wave's region
// (slots lane, lane + 64, ... below n), kNucBatch loads in flight at a time;
// the order is fixed.  n is uniform over the wave, and so is every call of
// f's loop (f may hold wave-wide operations: it is called for every batch
// slot, with valid false past n).  The loads go through the region's buffer
// resource unconditionally (a slot past the region reads 0), so they issue
// back to back.  Only the values are read: an index is fetched by its slot
// where it is needed (the window's keys).
template <typename F>
DEV void nuc_each(__amdgpu_buffer_rsrc_t rval, int n, F&& f) {
  const int lane = threadIdx.x & 63;
  for (int s0 = 0; s0 < n; s0 += 64 * kNucBatch) {
    uint32_t c[kNucBatch];
#pragma unroll
    for (int q = 0; q < kNucBatch; ++q)
      c[q] = __builtin_amdgcn_raw_buffer_load_b32(rval, (s0 + 64 * q + lane) * 4, 0, 0);
#pragma unroll
    for (int q = 0; q < kNucBatch; ++q) {
      const int sl = s0 + 64 * q + lane;
      f(sl < n, __uint_as_float(c[q]), sl);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kNB, 4) void k_nuc_rows(Params p) {
  constexpr int U = NucShape<T>::U;
  constexpr int R = U * kNB;                  // groups per round
  static_assert(R * kVec == kNucRoundLogits && U == 2 && kNB * kVec == kResidSeg,
                "a round is two residual segments, its slots u = 0 and u = 1");
  __shared__ uint64_t hist[kNucHist];         // sample counts (u32), then masses, then the window
  // each wave's candidates of its last round: values, then indices, kNucStage
  // slots each and one spare slot per lane (where lanes that do not take write)
  __shared__ uint32_t stg[kNW][2][kNucStage + 64];
  __shared__ double tab[kExpTab];
  __shared__ double redd[kNW];
  __shared__ uint64_t redu[kNW];
  __shared__ float redf[kNW];
  __shared__ int redi[kNW];
  __shared__ int sh_nw;
  __shared__ double sh_N;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int V = p.V;
  const int nrows = p.B * (p.rows_t + p.rows_d);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t* sv = stg[wu][0];
  uint32_t* si = stg[wu][1];
  if (tid < kExpTab) tab[tid] = kExp2Tab[tid];
  __syncthreads();
  const double cd = kLog2e / p.T;
  const double cs = kExpScale * cd;
  const double invT = 1.0 / p.T;
  const int ngroups = (V + kVec - 1) / kVec;
  const int nr = (ngroups + R - 1) / R;
  const int nfr = (V / kVec) / R;             // rounds of whole groups only
  for (int grow = blockIdx.x; grow < nrows; grow += gridDim.x) {
    // this wave's region of the row's buffer (p.nuc_keep: one per row, kept
    // for the residual kernel) or of the workgroup's; the flushes store
    // through a buffer resource spanning the region, which drops stores past
    // its end.  (The buffer: the candidates' values, then their indices,
    // kNucSlotEntries 32-bit words each; a wave's region of each at w kNucRegion.)
    uint32_t* bval = reinterpret_cast<uint32_t*>(p.nucc + (size_t)(p.nuc_keep ? grow : (int)blockIdx.x) * kNucSlotEntries);
    const uint32_t* bidx = bval + kNucSlotEntries;
    const __amdgpu_buffer_rsrc_t rval = make_rsrc(bval + (size_t)wu * kNucRegion, kNucRegion * 4);
    const __amdgpu_buffer_rsrc_t ridx = make_rsrc(bidx + (size_t)wu * kNucRegion, kNucRegion * 4);
    const T* row = row_ptr<T>(p, grow);
    bool xhas;
    const int xs = __builtin_amdgcn_readfirstlane(row_token(p, grow, &xhas));   // uniform over the row
    // start at a whole round (its values set tau); rows start at different
    // rounds so that workgroups in step do not hit the same memory channels
    const int r0 = nfr > 0 ? (int)(((long)grow * 7) % nfr) : 0;
    float m = -INFINITY;
    double s = 0.0;
    bool nan_seen = false;
    float lx = 0.f;
    bool hx = false;
    int cw = 0;                               // candidates met by this wave (uniform)
    int cs0 = 0;                              // ... of which flushed to the region
    bool over = false;                        // a round held more than kNucStage
    float tau = -INFINITY;
    bool first = true;
    int last_rc = 0, last_cr0 = 0;            // the last round staged, and its first half's count
    // the staged candidates of the last round to the region, entries
    // lane, lane + 64, ... (coalesced 8-byte stores; past the region dropped)
    // (the stage is the wave's own: its LDS accesses run in program order,
    // and the wave barriers keep the compiler from moving them across)
    auto flush = [&]() {
      __builtin_amdgcn_wave_barrier();
      const int n = cw - cs0 < kNucStage ? cw - cs0 : kNucStage;
      for (int i = lane; i < n; i += 64) {
        __builtin_amdgcn_raw_buffer_store_b32(sv[i], rval, (cs0 + i) * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(si[i], ridx, (cs0 + i) * 4, 0, 0);
      }
      // where the round's entries sit: the residual kernel finds a segment's
      // (the first or second half of a round) without reading the row
      if (p.nuc_keep && lane == 0) {
        const uint64_t st = (uint64_t)(cs0 < 0xffff ? cs0 : 0xffff);
        const uint64_t c = (uint64_t)(cw - cs0 < 0xffff ? cw - cs0 : 0xffff);
        p.nucm[((size_t)grow * kNW + wu) * p.nuc_rounds + last_rc] = st | ((uint64_t)last_cr0 << 16) | (c << 32);
      }
      cs0 = cw;
      __builtin_amdgcn_wave_barrier();
    };
    nuc_sweep<T>(row, V, p.aligned, r0, [&](float (&v)[U][kVec], const auto& mp, auto tailc) {
      constexpr bool kTail = decltype(tailc)::value;
      // max over the round, NaN evidence, the drafted token's logit
      float mi = m;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float gm = maximum8(v[u]);
        nan_seen |= gm != gm;
        mi = gm > mi ? gm : mi;
      }
      if (xhas) {
        // the one lane (if any) whose slots hold token xs this round
        int ux = 0, ex = 0;
        if (mp.holder(xs, &ux, &ex) == tid) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) lx = (u == ux && e == ex) ? v[u][e] : lx;
          }
          hx = true;
        }
      }
      if (mi > m) {
        // (the table exp2: exp2_neg's constants would stay in registers all loop long)
        if (m > -INFINITY) s *= exp2_64(((double)m - (double)mi) * cs, tab);
        m = mi;
      }
      if (first) {
        first = false;
        if (nr > 1) {
          // tau from this (whole) round: counts of 16-bit key prefixes below the round max's
          const float rmax = nb_max(mi, redf);
          uint32_t* hs = reinterpret_cast<uint32_t*>(hist);
          for (int b = tid; b < kNucSample; b += kNB) hs[b] = 0u;
          __syncthreads();
          const uint32_t top = ord_key(rmax) >> 16;
#pragma unroll
          for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
              const float x = v[u][e];
              if (x == x) {
                const uint32_t d = top - (ord_key(x) >> 16);
                atomicAdd(&hs[d < (uint32_t)(kNucSample - 1) ? d : (uint32_t)(kNucSample - 1)], 1u);
              }
            }
          }
          __syncthreads();
          // the first prefix bin at which the count from the top reaches want
          const int want = (int)((long)kNucFill * (long)(R * kVec) / (long)V);
          constexpr int per = kNucSample / kNB;
          uint32_t c[per];
          uint32_t tl = 0;
#pragma unroll
          for (int q = 0; q < per; ++q) { c[q] = hs[tid * per + q]; tl += c[q]; }
          uint32_t tot;
          uint32_t run = nb_exscan<uint32_t>(tl, reinterpret_cast<uint32_t*>(redi), &tot);
          int found = INT_MAX;
#pragma unroll
          for (int q = 0; q < per; ++q) {
            run += c[q];
            if (found == INT_MAX && run >= (uint32_t)want) found = tid * per + q;
          }
          const int bsel = nb_min<int>(found, redi);
          if (bsel != INT_MAX && rmax == rmax && rmax > -INFINITY) {
            // every value whose key prefix is >= top - bsel (a prefix below
            // 0x0080 would decode to a NaN: such a tau takes everything finite)
            uint32_t pk = top >= (uint32_t)bsel ? top - (uint32_t)bsel : 0u;
            pk = pk < 0x0080u ? 0x0080u : pk;
            tau = key_value(pk << 16);
          }
        }
      }
      // float64 terms, in batches of four (eight hold too many registers)
      if (m > -INFINITY) {
        const double nmc = -(double)m * cs;
        double gs = -0.0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          gs += exp2_64_sum<kVec / 2>(v[u], cs, nmc, tab);
          gs += exp2_64_sum<kVec / 2>(v[u] + kVec / 2, cs, nmc, tab);
        }
        s += gs;
      }
      // candidates to the wave's stage, without branches: one ballot per
      // element slot; a taking lane's slot is the round's count so far plus
      // the lanes below taking the same element slot (clamped: a round past
      // kNucStage has the row redone), every other lane writes its spare slot
      int cr = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
          bool take = v[u][e] >= tau;
          if constexpr (kTail) take = take && mp.index(u, e) < V;
          const uint64_t bm = __builtin_amdgcn_ballot_w64(take);
          const unsigned rank = __builtin_amdgcn_mbcnt_hi((unsigned)(bm >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bm, 0u));
          const unsigned at = (unsigned)cr + rank;
          const unsigned slot = take ? (at < (unsigned)kNucStage ? at : (unsigned)(kNucStage - 1)) : (unsigned)(kNucStage + lane);
          sv[slot] = __float_as_uint(v[u][e]);
          si[slot] = (uint32_t)mp.index(u, e);
          cr += (int)__popcll(bm);
        }
        if (u == 0) last_cr0 = cr;              // the round's first half (its first segment) comes first
      }
      over |= cr > kNucStage;
      cw += cr;
      last_rc = mp.r;
    }, flush);
    flush();
    // ---- settle (every early return is uniform over the workgroup)
    if (xhas && hx) p.row_lx[grow] = lx;
    auto settle = [&]() -> RowNuc {
      const bool bad_nan = __syncthreads_or(nan_seen) != 0;   // (also publishes the regions)
      const int nc = cw < kNucRegion ? cw : kNucRegion;
      auto each = [&](auto&& f) { nuc_each(rval, nc, f); };
      const float M = nb_max(m, redf);
      const bool bad = bad_nan || !(M > -INFINITY) || !(M < INFINITY);
      double zl = 0.0;
      if (!bad && m > -INFINITY) zl = s * exp2_neg(((double)m - (double)M) * cd);
      const double Z = nb_sum(zl, redd);
      RowNuc out;
      out.Z = Z; out.N = 0.0; out.cut = 0ull; out.M = M;
      out.ok = bad ? 0 : kNucFast;
      const bool full = __syncthreads_or(cw > kNucRegion || over) != 0;
      if (bad || full) return out;
      const double tgt = p.top_p * Z;
      const double zm = (double)M * invT;
      // bins of d = (M - l) / T over [0, dspan): every kept logit has
      // d < ln(V / ((1 - top_p) Z)) + 1 (the tokens below that hold less than
      // 1 - top_p of the mass together); candidates reach down to tau
      double dmaxd = log((double)V / ((1.0 - p.top_p) * Z)) + 1.0;
      if (!(dmaxd > 1.0)) dmaxd = 1.0;
      const double dtau = tau > -INFINITY ? ((double)M - (double)tau) * invT : dmaxd;
      double dspan = dtau < dmaxd ? dtau : dmaxd;
      if (!(dspan > 0.0)) dspan = 1e-30;
      const float invw = (float)((double)kNucHist / dspan);
      const float a1 = (float)(-invT) * invw, b1 = (float)zm * invw;
      // the bin tau falls in: bins below it hold only logits > tau (monotone
      // fma), all of them candidates
      int bin_tau = INT_MAX;
      if (tau > -INFINITY) {
        const float pt = fmaf(tau, a1, b1);
        bin_tau = pt < (float)kNucHist ? (int)__builtin_amdgcn_fmed3f(pt, 0.f, (float)(kNucHist - 1)) : kNucHist;
      }
      const bool no_fix = !(tgt < (double)kNucSlotEntries);   // the candidates cannot hold that much mass
      const uint64_t tgt_fix = no_fix ? 0ull : (uint64_t)(tgt * (double)kNucFix);
      auto bin_of = [&](float l) {
        const float pos = fmaf(l, a1, b1);
        return pos < (float)kNucHist ? (int)__builtin_amdgcn_fmed3f(pos, 0.f, (float)(kNucHist - 1)) : INT_MAX;
      };
      // e = exp((l - M) / T) = 2^((l - M) c): the table exp2, as the sweep's terms
      const double nmcM = -(double)M * cs;
      auto mass_of = [&](float l) { return exp2_64_l(l, cs, nmcM, tab); };
      // the histogram only locates the window (its bin and the two around
      // it): 32-bit fixed-point masses (2^-20 units, rounded) of the hardware
      // float32 exp2 of (l - M) c, summed in 64 bits by the scan.  A and the
      // window's walk below take float64 masses and accept a cut only inside
      // the window, so an inexact histogram (a bin past 4096 full masses
      // wraps) can only leave the row to the cut kernels.
      uint32_t* hist32 = reinterpret_cast<uint32_t*>(hist);
      const float M32 = M, c32 = (float)cd;
      for (int b = tid; b < kNucHist; b += kNB) hist[b] = 0ull;
      __syncthreads();
      each([&](bool valid, float l, int) {
        const int b = bin_of(l);
        if (valid && b != INT_MAX) {
          const float e32 = __builtin_amdgcn_exp2f((l - M32) * c32);
          atomicAdd(&hist32[b], (unsigned)fmaf(e32, kNucFix, 0.5f));
        }
      });
      __syncthreads();
      // the bin where the mass from the top reaches top_p Z
      int bc;
      {
        constexpr int per = kNucHist / kNB;
        uint64_t h[per];
        uint64_t hl = 0;
#pragma unroll
        for (int q = 0; q < per; ++q) { h[q] = hist32[tid * per + q]; hl += h[q]; }
        uint64_t tot;
        uint64_t run = nb_exscan<uint64_t>(hl, redu, &tot);
        int found = INT_MAX;
        if (!no_fix) {
#pragma unroll
          for (int q = 0; q < per; ++q) {
            run += h[q];
            if (found == INT_MAX && run >= tgt_fix) found = tid * per + q;
          }
        }
        bc = nb_min<int>(found, redi);
      }
      const int lo = bc > 0 ? bc - 1 : 0;
      const int hi = bc < kNucHist - 1 ? bc + 1 : kNucHist - 1;
      if (bc == INT_MAX || hi >= bin_tau) return out;   // the cut lies below tau
      // the exact mass above the window (fixed order: the lane's slots, then
      // the block sum), the window's keys gathered
      if (tid == 0) sh_nw = 0;
      __syncthreads();
      uint64_t* wl = hist;                 // unsorted window keys
      uint64_t* ws = hist + kNucWin;       // the same, ranked
      double al = 0.0;
      // (a window key holds the candidate's slot in the buffer until its
      // index is fetched below)
      each([&](bool valid, float l, int sl) {
        const int b = valid ? bin_of(l) : INT_MAX;
        if (b < lo) al += mass_of(l);
        const bool inw = b >= lo && b <= hi;
        const int at = wave_append(inw, &sh_nw);
        if (inw && at < kNucWin) wl[at] = pack(l, wu * kNucRegion + sl);
      });
      const double A = nb_sum(al, redd);   // (its barriers also publish the window)
      const int nw = sh_nw;
      if (nw == 0 || nw > kNucWin) return out;
      for (int i = tid; i < nw; i += kNB) {
        const uint64_t k = wl[i];
        wl[i] = pack(packed_val(k), (int)bidx[packed_idx(k)]);
      }
      __syncthreads();
      if (nw <= 128) {
        // a small window in wave 0 alone: its keys in slots lane and
        // lane + 64 (key 0, below every real key, past nw), sorted in
        // descending order by a bitonic network (position i = r 64 + lane;
        // partners in other lanes by lane exchange, at distance 64 within a
        // lane), then the masses' prefix sums from A by wave scans
        if (w == 0) {
          uint64_t k[2] = {lane < nw ? wl[lane] : 0ull, lane + 64 < nw ? wl[lane + 64] : 0ull};
#pragma unroll
          for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
            for (int j = size >> 1; j > 0; j >>= 1) {
              uint64_t o[2];
#pragma unroll
              for (int r = 0; r < 2; ++r) o[r] = j == 64 ? k[1 - r] : __shfl_xor(k[r], j);
#pragma unroll
              for (int r = 0; r < 2; ++r) {
                const int i = r * 64 + lane;
                const bool keep_max = ((i & j) == 0) == ((i & size) == 0);
                k[r] = keep_max ? (k[r] > o[r] ? k[r] : o[r]) : (k[r] < o[r] ? k[r] : o[r]);
              }
            }
          }
          double e[2], inc[2];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            e[r] = r * 64 + lane < nw ? mass_of(packed_val(k[r])) : 0.0;
            inc[r] = wave_scan(e[r], 0.0, [](double a, double b) { return a + b; });
          }
          const double t0 = read_lane(inc[0], 63);
          const double wtot = t0 + read_lane(inc[1], 63);
          const double c00 = A + (inc[0] - e[0]), c01 = A + (t0 + inc[1] - e[1]);
          const uint64_t b0 = __builtin_amdgcn_ballot_w64(lane < nw && c00 < tgt);
          const uint64_t b1 = __builtin_amdgcn_ballot_w64(lane + 64 < nw && c01 < tgt);
          const int kept = (int)__popcll(b0) + (int)__popcll(b1);   // (a prefix: c0 rises with the position)
          const bool inside = kept > 0 && (kept < nw || A + wtot >= tgt);
          if (inside) {
            const int at = kept - 1, ln = at & 63;
            out.N = at < 64 ? read_lane(c00 + e[0], ln) : read_lane(c01 + e[1], ln);
            out.cut = at < 64 ? read_lane(k[0], ln) : read_lane(k[1], ln);
            out.ok = 1;
          }
        }
        return out;
      }
      // rank of each window key (keys are distinct: the index is part of the key)
      for (int i = tid; i < nw; i += kNB) {
        const uint64_t k = wl[i];
        int r = 0;
        for (int j = 0; j < nw; ++j) r += wl[j] > k ? 1 : 0;
        ws[r] = k;
      }
      __syncthreads();
      // thread t walks ranks t kPerT .. t kPerT + kPerT - 1
      constexpr int kPerT = kNucWin / kNB;
      double e[kPerT];
      double et = 0.0;
#pragma unroll
      for (int q = 0; q < kPerT; ++q) {
        const int i = tid * kPerT + q;
        e[q] = i < nw ? mass_of(packed_val(ws[i])) : 0.0;
        et += e[q];
      }
      double wtot;
      double c0 = A + nb_exscan<double>(et, redd, &wtot);
      int kept_l = 0;
      double n_l = 0.0;
#pragma unroll
      for (int q = 0; q < kPerT; ++q) {
        const int i = tid * kPerT + q;
        if (i < nw && c0 < tgt) { kept_l = i + 1; n_l = c0 + e[q]; }
        c0 += e[q];
      }
      const int kept = nb_max_i<int>(kept_l, redi);
      const bool inside = kept > 0 && (kept < nw || A + wtot >= tgt);
      if (inside && kept_l == kept) sh_N = n_l;
      __syncthreads();
      if (inside) {
        out.N = sh_N;
        out.cut = ws[kept - 1];
        out.ok = 1;
      }
      return out;
    };
    const RowNuc out = settle();
    if (tid == 0) {
      p.nuc[grow] = out;
      if (p.nuc_keep) p.nuck[grow] = out.ok == 1 ? 1 : 0;
    }
    __syncthreads();   // the next row reuses hist and the buffer
  }
}

// ================================================================== launchers

template <typename T>
static int capacity_t(int mode) {
  int per_cu = 0;
  hipError_t e;
  if (mode == kModeStats64) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stream<T, kModeStats64>, kBlock, 0);
  else if (mode == kModeStatsMix) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stream<T, kModeStatsMix>, kBlock, 0);
  else if (mode == kModeTopk) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stream<T, kModeTopk>, kBlock, 0);
  else if (mode == kModeTopkFilter) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stream<T, kModeTopkFilter>, kBlock, 0);
  else if (mode == kModeNucRow) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_nuc_rows<T>, kNB, 0);
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
  const long rows = p.lazy == 1 ? 2L * p.B : p.lazy == 2 ? (long)p.B * (2 * p.k - 1)
                                                         : (long)p.B * (p.rows_t + p.rows_d);
  const unsigned grid = (unsigned)(rows * p.S);
  const dim3 block(kBlock);
  if (mode == kModeNucRow)   // persistent: p.grid workgroups (one candidate buffer each) or one per row
    hipExtLaunchKernelGGL((k_nuc_rows<T>), dim3((unsigned)(rows < p.grid ? rows : p.grid)), dim3(kNB), 0, st,
                          e0, e1, 0, p);
  else if (mode == kModeStats64)
    hipExtLaunchKernelGGL((k_stream<T, kModeStats64>), dim3(grid), block, 0, st, e0, e1, 0, p);
  else if (mode == kModeStatsMix)
    hipExtLaunchKernelGGL((k_stream<T, kModeStatsMix>), dim3(grid), block, 0, st, e0, e1, 0, p);
  else if (mode == kModeTopk)
    hipExtLaunchKernelGGL((k_stream<T, kModeTopk>), dim3(grid), block, 0, st, e0, e1, 0, p);
  else if (mode == kModeTopkFilter)
    hipExtLaunchKernelGGL((k_stream<T, kModeTopkFilter>), dim3(grid), block, 0, st, e0, e1, 0, p);
  else
    hipExtLaunchKernelGGL((k_stream<T, kModeArgmax>), dim3(grid), block, 0, st, e0, e1, 0, p);
  return hipGetLastError();
}

// The kernels after the streaming pass.  With ev_end, the dispatch of the
// call's last kernel records it when that kernel completes.
template <typename T>
static hipError_t launch_finish_t(const Params& p, int filt, hipStream_t st, hipEvent_t ev_end) {
  const int rows = p.B * (p.rows_t + p.rows_d);
  const dim3 block(kBlock), gb((unsigned)p.B), gr((unsigned)rows), gs((unsigned)p.S2, (unsigned)p.B),
      gb1(1u, (unsigned)p.B);
  auto run = [&](bool last, auto kernel, dim3 grid, auto... args) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, nullptr, last ? ev_end : nullptr, 0, args...);
  };
  switch (filt) {
    case kFiltGreedy: run(true, k_greedy_final<T>, gb, p); break;
    case kFiltTree: run(true, k_tree_final<T>, gb, p); break;
    case kFiltTopk:
      if (p.top_k <= 64 && p.P != p.S)
        run(false, k_topk_rows_w<T>, dim3((unsigned)((rows + kWaves - 1) / kWaves)), p);
      else
        run(false, k_topk_rows<T>, gr, p);
      if (p.top_k <= 64 && p.k < 64)
        run(true, k_topk_final_w<T>, gb, p);
      else
        run(true, k_topk_final<T>, gb, p);
      break;
    case kFiltTopp:
      run(false, k_topp_rows<T>, gr, p);
      run(false, k_resid_s<T, kFiltTopp>, dim3((unsigned)((p.S2 + p.rgrp - 1) / p.rgrp), (unsigned)p.B), p);
      run(true, k_resid_final<T, kFiltTopp>, (p.resid_probs || p.keep_w) ? gs : gb1, p);
      break;
    case kFiltTreeSample: {
      // with top-k or top-p: every row's adjusted view first
      if (p.top_k > 0) {
        if (p.top_k <= 64 && p.P != p.S)
          run(false, k_topk_rows_w<T>, dim3((unsigned)((rows + kWaves - 1) / kWaves)), p);
        else
          run(false, k_topk_rows<T>, gr, p);
      } else if (p.top_p < 1.0) {
        run(false, k_topp_rows<T>, gr, p);
      }
      const int passes = p.k - 1 < kTreePasses ? p.k - 1 : kTreePasses;
      for (int m = 0; m < passes; ++m) {
        const int most = (p.k - 1) / (m + 1);   // nodes that can have more than m children
        int G = (most + kPassBatch - 1) / kPassBatch;
        G = G < 1 ? 1 : (G > kPassGroups ? kPassGroups : G);
        if (p.tfilt) run(false, k_tsample_pass<T, true>, dim3((unsigned)p.S2, (unsigned)p.B, (unsigned)G), p, m);
        else run(false, k_tsample_pass<T, false>, dim3((unsigned)p.S2, (unsigned)p.B, (unsigned)G), p, m);
      }
      run(false, k_tsample_walk<T>, gb, p);
      run(false, k_tsample_mass<T>, gs, p);
      run(true, k_resid_final<T, kFiltNone>, (p.resid_probs || p.keep_w) ? gs : gb1, p);
      break;
    }
    default:  // plain sampling
      run(false, k_resid_s<T, kFiltNone>, dim3((unsigned)((p.S2 + p.rgrp - 1) / p.rgrp), (unsigned)p.B), p);
      run(true, k_resid_final<T, kFiltNone>, (p.resid_probs || p.keep_w) ? gs : gb1, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_stream(const Params& p, int mode, int bf16, hipStream_t st, hipEvent_t e0,
                         hipEvent_t e1) {
  return bf16 ? launch_stream_t<uint16_t>(p, mode, st, e0, e1)
              : launch_stream_t<float>(p, mode, st, e0, e1);
}

hipError_t launch_lazy_gate(const Params& p, int bf16, hipStream_t st) {
  if (bf16) hipLaunchKernelGGL((k_lazy_gate<uint16_t>), dim3((unsigned)p.B), dim3(kBlock), 0, st, p);
  else hipLaunchKernelGGL((k_lazy_gate<float>), dim3((unsigned)p.B), dim3(kBlock), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_finish(const Params& p, int filt, int bf16, hipStream_t st, hipEvent_t ev_end) {
  return bf16 ? launch_finish_t<uint16_t>(p, filt, st, ev_end) : launch_finish_t<float>(p, filt, st, ev_end);
}

}  // namespace sv
