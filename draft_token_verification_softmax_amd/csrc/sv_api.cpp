// C ABI of the verification library: argument validation (host only, before
// any HIP call), workspace ownership, and the launch sequence per mode.

#include <limits.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "specverify.h"
#include "sv_aux.h"
#include "sv_internal.h"

namespace {

constexpr int kMinTile = 8192;        // top-k pass: logits per tile, lower bound
constexpr int kRound = 4 * sv::kBlock * sv::kVec;   // argmax / sum passes: logits per round of loads
constexpr int kMinSmall = 2048;       // argmax / sum / filter passes: smallest tile of small problems
constexpr int kSmallTiles = 256;      // problems with fewer tiles than this take smaller tiles
constexpr int kStatsRoundsMax = 4;     // float32 sum / argmax passes: most rounds of loads per tile
constexpr size_t kKeepBytes = 32u << 20;   // residual weights kept for the draw up to this size
constexpr long kResidGroupWgs = 4096;      // residual workgroups that keep a launch full
constexpr long kResidCandWgs = 1024;       // ... when each wave takes a segment from the candidate buffers

struct Plan {
  int filt;        // sv::Filter
  int tile_mode;   // sv::TileMode
  int top_k;       // effective top-k (0 = off)
  double top_p;    // effective top-p (1 = off)
  int rows_t, rows_d, out_w;
  int S_max;       // most tiles per row of the top-k list passes (candidate list workspace)
  int S2_max;      // residual segments per sequence (plain sampling)
  int cand_w;
};

int check_config(const sv_config* c) {
  if (!c) return SV_ERR_NULL;
  if (c->mode != SV_MODE_SAMPLE && c->mode != SV_MODE_GREEDY && c->mode != SV_MODE_TREE_GREEDY &&
      c->mode != SV_MODE_TREE_SAMPLE)
    return SV_ERR_MODE;
  if (c->dtype != SV_DTYPE_F32 && c->dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
  if (c->max_batch < 1 || c->vocab < 1 || c->vocab > SV_MAX_VOCAB) return SV_ERR_SHAPE;
  const bool tree = c->mode == SV_MODE_TREE_GREEDY || c->mode == SV_MODE_TREE_SAMPLE;
  if (tree) {
    if (c->k < 1 || c->k > SV_MAX_TREE_NODES) return SV_ERR_SHAPE;
  } else {
    if (c->k < 1 || c->k > SV_MAX_K) return SV_ERR_SHAPE;
  }
  if (c->mode == SV_MODE_SAMPLE || c->mode == SV_MODE_TREE_SAMPLE) {
    if (!(c->temperature > 0.0) || !isfinite(c->temperature)) return SV_ERR_PARAM;
    if (c->top_k < 0) return SV_ERR_PARAM;
    if (c->top_k > SV_MAX_TOP_K && c->top_k < c->vocab) return SV_ERR_PARAM;
    if (!(c->top_p > 0.0 && c->top_p <= 1.0)) return SV_ERR_PARAM;
  }
  if (c->options & ~SV_OPT_LAZY_ROWS) return SV_ERR_PARAM;
  // lazy row reads: plain sampling only
  if ((c->options & SV_OPT_LAZY_ROWS) &&
      (c->mode != SV_MODE_SAMPLE || (c->top_k > 0 && c->top_k < c->vocab) || c->top_p < 1.0))
    return SV_ERR_PARAM;
  return SV_OK;
}

Plan make_plan(const sv_config* c) {
  Plan p;
  const bool sample = c->mode == SV_MODE_SAMPLE;
  const bool tsample = c->mode == SV_MODE_TREE_SAMPLE;
  p.top_k = ((sample || tsample) && c->top_k > 0 && c->top_k < c->vocab) ? c->top_k : 0;
  p.top_p = ((sample || tsample) && c->top_p < 1.0) ? c->top_p : 1.0;
  if (c->mode == SV_MODE_GREEDY) { p.filt = sv::kFiltGreedy; p.tile_mode = sv::kModeArgmax; }
  else if (c->mode == SV_MODE_TREE_GREEDY) { p.filt = sv::kFiltTree; p.tile_mode = sv::kModeArgmax; }
  else if (tsample) {
    // tree sampling: the adjusted rows come from the top-k merge or the
    // nucleus cut when a filter is set, else from the row sums
    p.filt = sv::kFiltTreeSample;
    p.tile_mode = p.top_k > 0 ? sv::kModeTopk : (p.top_p < 1.0 ? sv::kModeStats64 : sv::kModeStatsMix);
  }
  else if (p.top_k > 0) { p.filt = sv::kFiltTopk; p.tile_mode = sv::kModeTopk; }
  else if (p.top_p < 1.0) {
    p.filt = sv::kFiltTopp;
    p.tile_mode = c->vocab <= sv::kNucMaxV ? sv::kModeNucRow : sv::kModeStats64;
  }
  else { p.filt = sv::kFiltNone; p.tile_mode = sv::kModeStatsMix; }
  if (c->mode == SV_MODE_TREE_GREEDY) { p.rows_t = c->k; p.rows_d = 0; p.out_w = c->k; }
  else if (tsample) { p.rows_t = c->k; p.rows_d = c->k; p.out_w = c->k; }
  else { p.rows_t = c->k + 1; p.rows_d = sample ? c->k : 0; p.out_w = c->k + 1; }
  // most tiles per row of the list passes at any batch size (see the tiling
  // in specverify_run): the exact pass, or the filter pass at batch 1
  {
    const long rows1 = p.rows_t + p.rows_d;
    long s_exact = (c->vocab + kMinTile - 1) / kMinTile;
    long s_round = (c->vocab + kRound - 1) / kRound;
    long s_small = (kSmallTiles + rows1 - 1) / rows1;
    const long cap = (c->vocab + kMinSmall - 1) / kMinSmall;
    if (s_small > cap) s_small = cap;
    long sm = s_exact > s_round ? s_exact : s_round;
    if (s_small > sm) sm = s_small;
    p.S_max = (int)(sm > sv::kMaxTiles ? sv::kMaxTiles : sm);
  }
  p.cand_w = p.top_k > 0 ? sv::kCandSlots : 0;
  if (p.S_max < 1) p.S_max = 1;
  p.S2_max = (c->vocab + sv::kResidSeg - 1) / sv::kResidSeg;
  return p;
}

struct Layout {
  size_t tiles, cand, nuc, nucc, nucm, nuck, row_lx, seq, spart, wpart, tpart, tview, tcut, go;
  size_t k_idx, k_e, k_cnt, k_norm, k_bad, k_px, total;
  int nuc_slots;   // candidate buffers of k_nuc_rows (its most workgroups, or one per row)
  bool nuc_keep;   // one buffer per row: the residual kernel reads the target rows' candidates
};

// The workspace of a call of up to c->max_batch sequences.  nuc_cap bounds the
// candidate buffers of k_nuc_rows (fewer buffers: fewer resident workgroups).
int nuc_rounds(const sv_config* c) { return (c->vocab + sv::kNucRoundLogits - 1) / sv::kNucRoundLogits; }

Layout layout(const sv_config* c, const Plan& pl, int nuc_cap = INT_MAX) {
  const size_t B = (size_t)c->max_batch;
  const size_t rows = B * (size_t)(pl.rows_t + pl.rows_d);
  const size_t K = (size_t)pl.top_k;
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  L.tiles = take(rows * (size_t)sv::kMaxPartials * sizeof(sv::TileStat));
  L.cand = take(pl.top_k > 0 ? rows * (size_t)pl.S_max * (size_t)pl.cand_w * sizeof(uint64_t) : 0);
  const bool tfilt = pl.filt == sv::kFiltTreeSample && (pl.top_k > 0 || pl.top_p < 1.0);
  L.nuc = take(pl.filt == sv::kFiltTopp || tfilt ? rows * sizeof(sv::RowNuc) : 0);
  L.nuc_slots = pl.tile_mode == sv::kModeNucRow ? (int)(rows < (size_t)nuc_cap ? rows : (size_t)nuc_cap) : 0;
  L.nucc = take((size_t)L.nuc_slots * sv::kNucSlotEntries * sizeof(uint64_t));
  // with a buffer per row, where each round's candidates sit and whether the row was settled in place
  L.nuc_keep = L.nuc_slots > 0 && (size_t)L.nuc_slots >= rows;
  L.nucm = take(L.nuc_keep ? rows * (size_t)sv::kNucWaves * (size_t)nuc_rounds(c) * sizeof(uint64_t) : 0);
  L.nuck = take(L.nuc_keep ? rows * sizeof(int32_t) : 0);
  const bool sampled = pl.filt == sv::kFiltNone || pl.filt == sv::kFiltTopp || pl.filt == sv::kFiltTreeSample;
  L.row_lx = take(sampled ? rows * sizeof(float) : 0);
  L.seq = take(sampled ? B * sizeof(sv::SeqState) : 0);
  L.spart = take(sampled ? B * (size_t)pl.S2_max * sizeof(double) : 0);
  const bool keep = sampled && B * (size_t)pl.S2_max * sv::kResidSeg * sizeof(double) <= kKeepBytes;
  L.wpart = take(keep ? B * (size_t)pl.S2_max * sv::kResidSeg * sizeof(double) : 0);
  L.tpart = take(pl.filt == sv::kFiltTreeSample
                     ? B * (size_t)sv::kTreePasses * (size_t)c->k * (size_t)pl.S2_max * sizeof(double) : 0);
  L.tview = take(pl.filt == sv::kFiltTreeSample ? B * (size_t)c->k * 4 * sizeof(double) : 0);
  L.tcut = take(tfilt ? B * (size_t)c->k * 2 * sizeof(uint64_t) : 0);
  L.go = take((c->options & SV_OPT_LAZY_ROWS) ? B * sizeof(int32_t) : 0);
  L.k_idx = take(rows * K * sizeof(int32_t));
  L.k_e = take(rows * K * sizeof(double));
  L.k_cnt = take(K ? rows * sizeof(int32_t) : 0);
  L.k_norm = take(K ? rows * sizeof(double) : 0);
  L.k_bad = take(K ? rows * sizeof(int32_t) : 0);
  L.k_px = take(K ? rows * sizeof(double) : 0);
  L.total = off;
  return L;
}

// The streaming pass's tiling for `batch` sequences when the streaming kernel
// has `grid` resident workgroups: its tile mode (the top-k filter needs
// aligned rows), tiles per row S, logits per tile L (a multiple of kVec),
// partials per row P.  SV_ERR_SHAPE when it would not fit the workspace the
// plan sized (never expected; tests/test_abi_cpu.py sweeps shapes for it).
int tiling(const sv_config* c, const Plan& pl, int32_t batch, int grid, int aligned, int* tile_mode_out,
           int* S_out, int* L_out, int* P_out) {
  const size_t es = c->dtype == SV_DTYPE_BF16 ? 2 : 4;
  // top-k: the certified filter pass takes tiles of one round of loads in
  // aligned rows of whole groups; other shapes take the exact per-tile pass
  int tile_mode = pl.tile_mode;
  const long rows = (long)batch * (pl.rows_t + pl.rows_d);
  // float32 row sums and argmax of large problems: tiles of 4 (or 2) rounds
  // of loads, as long as that still fills three quarters of the resident
  // workgroup slots.  Each tile's fixed work (the float64 rescale and wave
  // sums, the partials) spreads over more logits, and the kernels after the
  // pass combine four times fewer partials per row (workload 6: pass 55.0 ->
  // 48.8 -> 45.5 us for 1, 2, 4 rounds; workload 4: pass 21.0 -> 21.1 us,
  // tree_final 7.6 -> 6.0 us; the 11 MB of workload 2 are faster with one).
  // The float64 sums of nucleus rows are bound by their exponentials and
  // stay at one round.
  int rounds = 1;
  if (tile_mode == sv::kModeStatsMix || tile_mode == sv::kModeArgmax) {
    for (int r = kStatsRoundsMax; r > 1; r >>= 1) {
      if (4L * rows * ((c->vocab + (long)r * kRound - 1) / ((long)r * kRound)) >= 3L * grid) {
        rounds = r;
        break;
      }
    }
  }
  const int round = tile_mode == sv::kModeTopk ? (int)(sv::kFilterRound * 2 / es) : rounds * kRound;
  if (tile_mode == sv::kModeTopk && aligned && c->vocab % sv::kVec == 0 &&
      c->vocab <= (long)sv::kMaxTiles * round)
    tile_mode = sv::kModeTopkFilter;
  if (tile_mode == sv::kModeNucRow) {
    // one workgroup per row reads all of it (no tile partials)
    *tile_mode_out = tile_mode;
    *S_out = 1;
    *L_out = (int)((c->vocab + sv::kVec - 1) / sv::kVec * sv::kVec);
    *P_out = 1;
    return SV_OK;
  }
  long S;
  if (tile_mode == sv::kModeTopk) {
    // about four tiles per resident workgroup, tiles of at least kMinTile logits
    S = (4L * grid + rows - 1) / rows;
    const long smax = (c->vocab + kMinTile - 1) / kMinTile;
    if (S > smax) S = smax;
  } else {
    // one round of loads per lane (kRound logits; 16 KB of bf16, 32 KB of
    // fp32); rows that need more than kMaxTiles such tiles take several
    // rounds per tile; problems with fewer than kSmallTiles tiles take
    // smaller tiles (down to kMinSmall logits)
    S = (c->vocab + round - 1) / round;
    if (rows * S < kSmallTiles) {
      long want = (kSmallTiles + rows - 1) / rows;
      const long cap = (c->vocab + kMinSmall - 1) / kMinSmall;
      if (want > cap) want = cap;
      if (want > S) S = want;
    }
  }
  if (S > sv::kMaxTiles) S = sv::kMaxTiles;
  if (S < 1) S = 1;
  int per = (int)((c->vocab + S - 1) / S);
  if (tile_mode != sv::kModeTopk && per > round) per = (per + round - 1) / round * round;
  const int Lt = (per + sv::kVec - 1) / sv::kVec * sv::kVec;
  const int St = (int)((c->vocab + Lt - 1) / Lt);
  const bool lists = tile_mode == sv::kModeTopk || tile_mode == sv::kModeTopkFilter;
  const int Pt = tile_mode == sv::kModeTopk ? St : St * (sv::kBlock / 64);
  // the workspace holds S_max candidate lists and kMaxPartials partials per row
  if ((lists && St > pl.S_max) || Pt > sv::kMaxPartials || St > sv::kMaxTiles) return SV_ERR_SHAPE;
  *tile_mode_out = tile_mode;
  *S_out = St;
  *L_out = Lt;
  *P_out = Pt;
  return SV_OK;
}

// One call's launches on the current device: the tiling of the streaming
// pass, the workspace views (ws laid out as L), the launch chain of the mode.
// Arguments are already checked.  Returns SV_OK, SV_ERR_SHAPE (the tiling
// would not fit the workspace) or SV_ERR_HIP.
int launch_call(const sv_config* c, const Plan& pl, const Layout& L, char* ws, int grid,
                const hipEvent_t ev[3], int32_t batch, const void* target_logits,
                const void* draft_logits, const int32_t* draft_tokens, const int32_t* parents,
                const float* uniforms, const float* resid_uniforms, int32_t* accepted_len,
                int32_t* out_tokens, int32_t* out_nodes, float* resid_probs, int32_t* seq_status,
                hipStream_t st) {
  sv::Params p;
  memset(&p, 0, sizeof(p));
  p.target = target_logits;
  p.draft = draft_logits;
  p.tokens = draft_tokens;
  p.parents = parents;
  p.u = uniforms;
  p.ur = resid_uniforms;
  p.acc_len = accepted_len;
  p.out_tokens = out_tokens;
  p.out_nodes = out_nodes;
  p.resid_probs = resid_probs;
  p.seq_status = seq_status;
  p.B = batch;
  p.k = c->k;
  p.V = c->vocab;
  p.rows_t = pl.rows_t;
  p.rows_d = pl.rows_d;
  p.out_w = pl.out_w;
  p.T = (c->mode == SV_MODE_SAMPLE || c->mode == SV_MODE_TREE_SAMPLE) ? c->temperature : 1.0;
  p.tree = (c->mode == SV_MODE_TREE_GREEDY || c->mode == SV_MODE_TREE_SAMPLE) ? 1 : 0;
  p.top_p = pl.top_p;
  p.top_k = pl.top_k;
  // tiling of the streaming pass
  const size_t es = c->dtype == SV_DTYPE_BF16 ? 2 : 4;
  const bool rows16 = ((size_t)c->vocab * es) % 16 == 0;
  const bool base16 = ((uintptr_t)target_logits % 16 == 0) &&
                      (!draft_logits || (uintptr_t)draft_logits % 16 == 0);
  p.aligned = (rows16 && base16) ? 1 : 0;
  int tile_mode;
  const int rc = tiling(c, pl, batch, grid, p.aligned, &tile_mode, &p.S, &p.L, &p.P);
  if (rc != SV_OK) return rc;
  p.grid = grid;
  p.tiles = (sv::TileStat*)(ws + L.tiles);
  p.cand = (uint64_t*)(ws + L.cand);
  p.cand_w = pl.cand_w;
  p.nuc = (sv::RowNuc*)(ws + L.nuc);
  p.row_lx = (float*)(ws + L.row_lx);
  p.seq = (sv::SeqState*)(ws + L.seq);
  p.spart = (double*)(ws + L.spart);
  p.wpart = (double*)(ws + L.wpart);
  p.tpart = (double*)(ws + L.tpart);
  p.tview = (double*)(ws + L.tview);
  p.tcut = (uint64_t*)(ws + L.tcut);
  p.tfilt = (pl.filt == sv::kFiltTreeSample && (pl.top_k > 0 || pl.top_p < 1.0)) ? 1 : 0;
  p.keep_w = (pl.filt == sv::kFiltNone || pl.filt == sv::kFiltTopp || pl.filt == sv::kFiltTreeSample) &&
             (size_t)c->max_batch * pl.S2_max * sv::kResidSeg * sizeof(double) <= kKeepBytes ? 1 : 0;
  p.S2 = pl.S2_max;
  // segments per workgroup of the residual kernel: its setup and accept
  // tests once for several segments, as long as 4096 workgroups remain
  // (workload 5: 19200 -> 4800 workgroups, 110 -> 85 us for the kernels
  // after the streaming pass; small problems keep one segment each)
  p.rgrp = 1;
  for (int g = 4; g > 1; g >>= 1) {
    if ((long)batch * ((pl.S2_max + g - 1) / g) >= kResidGroupWgs) { p.rgrp = g; break; }
  }
  // the nucleus residual from the target rows' candidate buffers (a wave per
  // segment, the setup and accept tests once per workgroup): up to 16
  // segments per workgroup while 1024 workgroups remain (workload 5: 4864 ->
  // 1280 workgroups, the kernels after the nucleus kernel 63 -> 58 us)
  if (L.nuc_keep && tile_mode == sv::kModeNucRow) {
    for (int g = 16; g > p.rgrp; g >>= 1) {
      if ((long)batch * ((pl.S2_max + g - 1) / g) >= kResidCandWgs) { p.rgrp = g; break; }
    }
  }
  p.k_idx = (int32_t*)(ws + L.k_idx);
  p.k_e = (double*)(ws + L.k_e);
  p.k_cnt = (int32_t*)(ws + L.k_cnt);
  p.k_norm = (double*)(ws + L.k_norm);
  p.k_bad = (int32_t*)(ws + L.k_bad);
  p.k_px = (double*)(ws + L.k_px);
  p.go = (int32_t*)(ws + L.go);
  p.nucrow = tile_mode == sv::kModeNucRow ? 1 : 0;
  p.nucc = (uint64_t*)(ws + L.nucc);
  p.nucm = (uint64_t*)(ws + L.nucm);
  p.nuck = (int32_t*)(ws + L.nuck);
  p.nuc_rounds = nuc_rounds(c);
  p.nuc_keep = (p.nucrow && L.nuc_keep) ? 1 : 0;   // (the layout's rows: at least this call's)
  if (p.nucrow && !p.nuc_keep && p.grid > L.nuc_slots) p.grid = L.nuc_slots;   // one buffer per workgroup

  const int bf16 = c->dtype == SV_DTYPE_BF16;
  hipError_t e;
  if (c->options & SV_OPT_LAZY_ROWS) {
    // stage 1: row pair 0 and the test of x_0; stage 2: the other rows of
    // the sequences that passed it (the same tiling, so the partials keep
    // the layout the finishing kernels read)
    p.lazy = 1;
    e = sv::launch_stream(p, tile_mode, bf16, st, ev[0], ev[1]);
    if (e == hipSuccess) e = sv::launch_lazy_gate(p, bf16, st);
    p.lazy = 2;
    if (e == hipSuccess) e = sv::launch_stream(p, tile_mode, bf16, st);
    p.lazy = 3;   // the finishing kernels: rows after position 0 only where go
  } else {
    e = sv::launch_stream(p, tile_mode, bf16, st, ev[0], ev[1]);
  }
  if (e == hipSuccess) e = sv::launch_finish(p, pl.filt, bf16, st, ev[2]);
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}


// Workspace of specverify_run_static: one fixed array in device memory that
// every GPU the library runs on holds until the process ends.  Host code never
// uses the array's name as an address (on the host it is a stand-in, not the
// device address): the address comes from hipGetSymbolAddress, once per device
// with that device current, and is kept per device.
static __device__ __align__(256) unsigned char scratch[SV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct StaticDevice {
  int ready;               // 0 not set up, 1 set up, -1 set-up failed
  char* ptr;               // device address of `scratch` on this device
  int cus;                 // compute units
  int per_cu[2][8];        // resident streaming workgroups per CU, [bf16][tile mode] (0: not asked yet)
};
StaticDevice g_static[kMaxDevices];
std::mutex g_static_mu;

// Set-up of the current device for specverify_run_static (first call on it):
// the scratch address and the compute-unit count; then the streaming
// kernel's resident workgroups for this mode and dtype.  No allocation.
int static_device(int tile_mode, int bf16, char** ptr, int* grid) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDevice& d = g_static[dev];
  if (d.ready == 0) {
    void* addr = nullptr;
    int cus = 0;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
      d.ready = -1;
    } else {
      d.ptr = (char*)addr;
      d.cus = cus;
      d.ready = 1;
    }
  }
  if (d.ready != 1 || tile_mode < 0 || tile_mode >= 8) return SV_ERR_HIP;
  int& pc = d.per_cu[bf16 ? 1 : 0][tile_mode];
  if (pc == 0) {
    pc = sv::stream_blocks_per_cu(tile_mode, bf16);
    if (pc < 1) pc = 1;
  }
  *ptr = d.ptr;
  *grid = d.cus * pc;
  return SV_OK;
}

}  // namespace

struct specverify_ctx {
  sv_config cfg;
  Plan plan;
  int device;
  void* ws;
  size_t ws_bytes;
  Layout L;
  int grid;                      // resident workgroups of the streaming kernel
  // optional instrumentation (caller-owned events): the streaming kernel's
  // start, its end, the end of the call's last kernel
  hipEvent_t ev_begin, ev_stream_end, ev_call_end;
};

extern "C" {

const char* specverify_status_string(int status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_NULL: return "SV_ERR_NULL: a required pointer is NULL";
    case SV_ERR_SHAPE: return "SV_ERR_SHAPE: batch, k or vocab out of range";
    case SV_ERR_DTYPE: return "SV_ERR_DTYPE: unknown dtype";
    case SV_ERR_PARAM: return "SV_ERR_PARAM: temperature, top_k or top_p out of range";
    case SV_ERR_CAPACITY: return "SV_ERR_CAPACITY: batch exceeds max_batch";
    case SV_ERR_HIP: return "SV_ERR_HIP: a HIP call failed";
    case SV_ERR_MODE: return "SV_ERR_MODE: unknown mode, or a pointer that does not fit the mode";
    case SV_ERR_SCRATCH:
      return "SV_ERR_SCRATCH: the call needs more workspace than the static scratch array holds "
             "(SV_STATIC_SCRATCH_BYTES); use a context (specverify_create / specverify_run) or a smaller batch";
    default: return "unknown status";
  }
}

size_t specverify_workspace_bytes(const sv_config* cfg) {
  if (check_config(cfg) != SV_OK) return 0;
  const Plan pl = make_plan(cfg);
  return layout(cfg, pl).total;
}

int specverify_check_args(const sv_config* cfg, int32_t batch, const void* target_logits,
                          const void* draft_logits, const int32_t* draft_tokens,
                          const int32_t* parents, const float* uniforms,
                          const float* resid_uniforms, const int32_t* accepted_len,
                          const int32_t* out_tokens, const int32_t* out_nodes) {
  const int rc = check_config(cfg);
  if (rc != SV_OK) return rc;
  if (batch < 0) return SV_ERR_SHAPE;
  if (batch > cfg->max_batch) return SV_ERR_CAPACITY;
  if (batch == 0) return SV_OK;   // nothing to read or write; pointers may be NULL
  if (!target_logits || !draft_tokens || !accepted_len || !out_tokens) return SV_ERR_NULL;
  switch (cfg->mode) {
    case SV_MODE_SAMPLE:
      if (!draft_logits || !uniforms || !resid_uniforms) return SV_ERR_NULL;
      if (parents || out_nodes) return SV_ERR_MODE;
      break;
    case SV_MODE_GREEDY:
      if (draft_logits || parents || uniforms || resid_uniforms || out_nodes) return SV_ERR_MODE;
      break;
    case SV_MODE_TREE_SAMPLE:
      if (!parents || !draft_logits || !uniforms || !resid_uniforms) return SV_ERR_NULL;
      break;
    default:  // greedy tree
      if (!parents) return SV_ERR_NULL;
      if (draft_logits || uniforms || resid_uniforms) return SV_ERR_MODE;
      break;
  }
  return SV_OK;
}

int specverify_create(const sv_config* cfg, int device, specverify_ctx** out) {
  if (!out) return SV_ERR_NULL;
  *out = nullptr;
  const int rc = check_config(cfg);
  if (rc != SV_OK) return rc;
  specverify_ctx* ctx = (specverify_ctx*)calloc(1, sizeof(specverify_ctx));
  if (!ctx) return SV_ERR_HIP;
  ctx->cfg = *cfg;
  ctx->plan = make_plan(cfg);
  ctx->device = device;
  const Layout L = layout(cfg, ctx->plan);
  ctx->ws_bytes = L.total;
  ctx->L = L;
  // the caller's current device is restored on every return path
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) { free(ctx); return SV_ERR_HIP; }
  if (cur != device && hipSetDevice(device) != hipSuccess) { free(ctx); return SV_ERR_HIP; }
  int rc2 = SV_OK;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
    rc2 = SV_ERR_HIP;
  } else {
    const int per_cu = sv::stream_blocks_per_cu(ctx->plan.tile_mode, cfg->dtype == SV_DTYPE_BF16);
    ctx->grid = prop.multiProcessorCount * (per_cu > 0 ? per_cu : 1);
    if (hipMalloc(&ctx->ws, L.total) != hipSuccess) rc2 = SV_ERR_HIP;
  }
  if (cur != device) (void)hipSetDevice(cur);
  if (rc2 != SV_OK) { free(ctx); return rc2; }
  *out = ctx;
  return SV_OK;
}

void specverify_destroy(specverify_ctx* ctx) {
  if (!ctx) return;
  if (ctx->ws) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != ctx->device) (void)hipSetDevice(ctx->device);
    (void)hipFree(ctx->ws);
    if (cur >= 0 && cur != ctx->device) (void)hipSetDevice(cur);
  }
  free(ctx);
}

int specverify_profile_events(specverify_ctx* ctx, void* ev_begin, void* ev_stream_end,
                              void* ev_call_end) {
  if (!ctx) return SV_ERR_NULL;
  if (!ev_begin && (ev_stream_end || ev_call_end)) return SV_ERR_NULL;
  if (ev_begin && !ev_stream_end && !ev_call_end) return SV_ERR_NULL;
  ctx->ev_begin = (hipEvent_t)ev_begin;
  ctx->ev_stream_end = (hipEvent_t)ev_stream_end;
  ctx->ev_call_end = (hipEvent_t)ev_call_end;
  return SV_OK;
}

int specverify_run(specverify_ctx* ctx, int32_t batch, const void* target_logits,
                   const void* draft_logits, const int32_t* draft_tokens, const int32_t* parents,
                   const float* uniforms, const float* resid_uniforms, int32_t* accepted_len,
                   int32_t* out_tokens, int32_t* out_nodes, float* resid_probs,
                   int32_t* seq_status, void* stream) {
  if (!ctx) return SV_ERR_NULL;
  const sv_config* c = &ctx->cfg;
  int rc = specverify_check_args(c, batch, target_logits, draft_logits, draft_tokens, parents,
                                 uniforms, resid_uniforms, accepted_len, out_tokens, out_nodes);
  if (rc != SV_OK) return rc;
  if (resid_probs && c->mode != SV_MODE_SAMPLE && c->mode != SV_MODE_TREE_SAMPLE) return SV_ERR_MODE;
  if (batch == 0) return SV_OK;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SV_ERR_HIP;
  if (cur != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return SV_ERR_HIP;
  const hipEvent_t ev[3] = {ctx->ev_begin, ctx->ev_stream_end, ctx->ev_call_end};
  rc = launch_call(c, ctx->plan, ctx->L, (char*)ctx->ws, ctx->grid, ev, batch, target_logits,
                   draft_logits, draft_tokens, parents, uniforms, resid_uniforms, accepted_len,
                   out_tokens, out_nodes, resid_probs, seq_status, (hipStream_t)stream);
  if (cur != ctx->device) (void)hipSetDevice(cur);
  return rc;
}

int specverify_run_static(const sv_config* cfg, int32_t batch, const void* target_logits,
                          const void* draft_logits, const int32_t* draft_tokens, const int32_t* parents,
                          const float* uniforms, const float* resid_uniforms, int32_t* accepted_len,
                          int32_t* out_tokens, int32_t* out_nodes, float* resid_probs,
                          int32_t* seq_status, void* stream) {
  int rc = specverify_check_args(cfg, batch, target_logits, draft_logits, draft_tokens, parents,
                                 uniforms, resid_uniforms, accepted_len, out_tokens, out_nodes);
  if (rc != SV_OK) return rc;
  if (resid_probs && cfg->mode != SV_MODE_SAMPLE && cfg->mode != SV_MODE_TREE_SAMPLE) return SV_ERR_MODE;
  if (batch == 0) return SV_OK;
  // the workspace laid out for this call's batch
  sv_config c = *cfg;
  c.max_batch = batch;
  const Plan pl = make_plan(&c);
  Layout L = layout(&c, pl);
  if (L.total > (size_t)SV_STATIC_SCRATCH_BYTES && L.nuc_slots > 0) {
    // fewer nucleus candidate buffers (fewer resident workgroups) to fit
    const size_t per = (size_t)sv::kNucSlotEntries * sizeof(uint64_t);
    const size_t drop = (L.total - (size_t)SV_STATIC_SCRATCH_BYTES + per - 1) / per;
    if (drop < (size_t)L.nuc_slots) L = layout(&c, pl, L.nuc_slots - (int)drop);
  }
  if (L.total > (size_t)SV_STATIC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
  char* ws = nullptr;
  int grid = 0;
  rc = static_device(pl.tile_mode, c.dtype == SV_DTYPE_BF16, &ws, &grid);
  if (rc != SV_OK) return rc;
  const hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  return launch_call(&c, pl, L, ws, grid, ev, batch, target_logits, draft_logits, draft_tokens,
                     parents, uniforms, resid_uniforms, accepted_len, out_tokens, out_nodes,
                     resid_probs, seq_status, (hipStream_t)stream);
}

int specverify_tiling(const sv_config* cfg, int32_t batch, int32_t grid, int32_t aligned, int32_t* out) {
  if (!out) return SV_ERR_NULL;
  const int rc = check_config(cfg);
  if (rc != SV_OK) return rc;
  if (batch < 1) return SV_ERR_SHAPE;
  if (batch > cfg->max_batch) return SV_ERR_CAPACITY;
  if (grid < 1) return SV_ERR_PARAM;
  const Plan pl = make_plan(cfg);
  const size_t es = cfg->dtype == SV_DTYPE_BF16 ? 2 : 4;
  const int al = (aligned && ((size_t)cfg->vocab * es) % 16 == 0) ? 1 : 0;
  int tm = 0, S = 0, L = 0, P = 0;
  const int r = tiling(cfg, pl, batch, grid, al, &tm, &S, &L, &P);
  const bool lists = tm == sv::kModeTopk || tm == sv::kModeTopkFilter;
  out[0] = tm;
  out[1] = S;
  out[2] = L;
  out[3] = P;
  out[4] = lists ? pl.S_max : sv::kMaxTiles;
  out[5] = sv::kMaxPartials;
  return r;
}

static_assert(SV_STATS_LEN == sv::kStatsLen && SV_STATS_SPEEDUP_GAMMA1 == sv::kStatsSpeedup1 &&
                  SV_STATS_ALPHA == sv::kStatsAlpha && SV_STATS_GAMMA_BEST == sv::kStatsGammaBest,
              "statistics layout");

int specverify_accept_stats(const int32_t* accepted_len, const int32_t* seq_status, int32_t batch,
                            int32_t k, double draft_cost, double* out, void* stream) {
  if (!out || (batch > 0 && !accepted_len)) return SV_ERR_NULL;
  if (batch < 0 || k < 1) return SV_ERR_SHAPE;
  if (!(draft_cost >= 0.0) || !isfinite(draft_cost)) return SV_ERR_PARAM;
  const hipError_t e = sv::launch_accept_stats(accepted_len, seq_status, batch, k, draft_cost, out,
                                               (hipStream_t)stream);
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int specverify_read_floor(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0) return SV_ERR_SHAPE;
  if (bytes == 0) return SV_OK;
  if (!src || !sink) return SV_ERR_NULL;
  if ((uintptr_t)src % 16 != 0 || bytes % 16 != 0) return SV_ERR_SHAPE;
  const hipError_t e = sv::launch_read_floor(src, (long long)bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int specverify_tree_mask(const int32_t* parents, int32_t batch, int32_t nodes, uint32_t* mask,
                         int32_t* depth, void* stream) {
  if (batch < 0 || nodes < 1 || nodes > SV_MAX_TREE_NODES) return SV_ERR_SHAPE;
  if (batch == 0) return SV_OK;
  if (!parents || !mask) return SV_ERR_NULL;
  const hipError_t e = sv::launch_tree_mask(parents, batch, nodes, mask, depth, (hipStream_t)stream);
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int specverify_tree_commit(const int32_t* path_nodes, const int32_t* accepted_len, int32_t batch,
                           int32_t nodes, int32_t* commit_pos, void* stream) {
  if (batch < 0 || nodes < 1 || nodes > SV_MAX_TREE_NODES) return SV_ERR_SHAPE;
  if (batch == 0) return SV_OK;
  if (!path_nodes || !accepted_len || !commit_pos) return SV_ERR_NULL;
  const hipError_t e = sv::launch_tree_commit(path_nodes, accepted_len, batch, nodes, commit_pos,
                                              (hipStream_t)stream);
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
