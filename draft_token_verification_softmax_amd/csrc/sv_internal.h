// Internal declarations shared by the host dispatcher (sv_api.cpp) and the
// gfx950 kernels (sv_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kBlock = 256;            // threads per workgroup (4 wave64s)
constexpr int kVec = 8;                // logits per group: 16 B of bf16, 32 B of fp32
constexpr int kTopkCap = 2560;         // LDS candidate slots of the top-k tile kernel
constexpr int kMergeCap = 4096;        // LDS slots when merging a row's top-k candidates
constexpr int kCandSlots = 256;        // per-tile top-k candidate slots in the workspace
constexpr int kWindowCap = 1024;       // LDS slots for the nucleus boundary window
constexpr int kNucBins = 2048;         // histogram bins of the nucleus search
constexpr int kResidSeg = kBlock * kVec;  // logits per workgroup in the residual kernels
constexpr int kMaxTiles = 64;          // tiles per row
constexpr int kMaxPartials = 256;      // partials per row (one wave combines a row's partials)
// logits per tile of the top-k filter pass for bf16 (one round of loads:
// sixteen 16-byte groups per lane); fp32 tiles hold half as many
constexpr int kFilterRound = 16 * kBlock * kVec;

// Partial result of the streaming pass over a part of a row: the logits one
// wave of a tile read (argmax and sum passes), or a whole tile (top-k pass).
//   m    max raw logit of the part (NaN ignored; -inf if none)
//   amax lowest index holding m (INT32_MAX if none)
//   s    NaN iff the part holds a NaN or +inf (exact, every mode); otherwise
//        STATS mode: float64 sum over the part of exp((l - m) / T), other
//        modes: 0
// Top-k passes instead: m = a lower bound of the tile's top_k-th logit such
// that the tile's list (in p.cand, amax entries) holds every logit of the
// tile >= m (-inf if the tile has fewer than top_k logits).  The exact pass
// lists the tile's top_k in rank order with m its top_k-th logit; the
// filter pass lists, unordered, every logit >= its bound, and amax above
// cand_w means the list overflowed (the row merge then redoes the tile).
struct TileStat {
  float m;
  int32_t amax;
  double s;
};

// Per-row nucleus (top-p) result.
//   Z      sum_v exp(z_v - zmax) in float64 (z = l / T)
//   N      mass of the kept set (same units); p'(v) = exp(z_v - zmax) / N on the set
//   cut    packed (value, index) key of the last kept entry: v is kept iff
//          pack(l_v, v) >= cut, i.e. it ranks at or before the cut in
//          (value desc, index asc) order
//   ok     1 found; 0 the row is invalid (NaN / +inf / all -inf); 2 the search
//          did not settle (not expected)
struct RowNuc {
  double Z;
  double N;
  uint64_t cut;
  int32_t ok;
  float M;      // max raw logit of the row
};

// State of one sequence handed from k_resid_s to k_resid_final: the
// accepted count n (-1: outputs already written), status bits, and the
// views of the rows the residual reads (target row n; draft row n if n < k).
// Row views: nmc = -M * 64 log2e / T (M = row max), inv = 1 / normaliser,
// cut = nucleus cut (0 = none).
struct SeqState {
  double nmc_p, inv_p, nmc_q, inv_q;
  uint64_t cut_p, cut_q;
  int32_t n, st;
  int32_t node;   // row index of the residual within the sequence (chain: n; tree: final node)
  int32_t hasq;   // the draft row enters the residual
};

// Passes of the streaming kernel: argmax (greedy, tree), top-k lists (exact
// per tile: any tile shape; certified filter: tiles of one round of loads in
// aligned rows), max + sum of exponentials (float64 terms for the nucleus
// rows of a sampled tree; plain and tree sampling: float64 terms in the rows
// whose normaliser can change a decision, float32 terms in the others).
// Chain sampling with top-p alone takes kModeNucRow instead (rows up to
// kNucMaxV logits): persistent workgroups read each row once and settle its
// nucleus cut (k_nuc_rows) from the candidates it keeps in a buffer of
// kNucSlotEntries entries (8 bytes: the raw value and the index) in the
// workspace: one buffer per row where the workspace holds them (the residual
// kernel then reads the target rows' kept entries there), else one per
// workgroup.
enum TileMode { kModeArgmax = 0, kModeTopk = 2, kModeStats64 = 3, kModeTopkFilter = 4, kModeStatsMix = 5,
                kModeNucRow = 6 };
constexpr int kNucMaxV = 1 << 20;        // longest rows k_nuc_rows takes (its buffer holds ~1.5% of them)
constexpr int kNucSlotEntries = 24576;   // candidate entries per buffer (192 KB)
constexpr int kNucWaves = 4;             // waves of a k_nuc_rows workgroup (a region of the buffer each)
constexpr int kNucRoundLogits = 4096;    // logits a k_nuc_rows workgroup reads per round
enum Filter { kFiltGreedy = 0, kFiltNone = 1, kFiltTopk = 2, kFiltTopp = 3, kFiltTree = 4,
              kFiltTreeSample = 5 };
// Speculative residual passes of tree sampling: pass m (1..kTreePasses)
// finds the residual normaliser after the m-th rejected child at every node
// with at least m children.  A walk that rejects more children at one node
// computes the rest itself.
constexpr int kTreePasses = 4;

struct Params {
  // inputs
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* parents;
  const float* u;
  const float* ur;
  // outputs
  int32_t* acc_len;
  int32_t* out_tokens;
  int32_t* out_nodes;
  float* resid_probs;
  int32_t* seq_status;
  // shape
  int B;        // batch
  int k;        // chain: drafts per sequence; tree: nodes per tree
  int V;
  int rows_t;   // target rows per sequence (k+1, or N for a tree)
  int rows_d;   // draft rows per sequence (k in SAMPLE mode, else 0)
  int out_w;    // width of out_tokens rows (k+1 chain, N tree)
  // sampling settings
  double T;
  double top_p;
  int top_k;    // 0 = off
  // tiling of the streaming pass
  int S;        // tiles (workgroups of the streaming pass) per row
  int L;        // logits per tile (multiple of kVec)
  int P;        // partials per row in `tiles`: S * kWaves (one per wave) for
                // the argmax and sum passes, S for the top-k pass
  int aligned;  // every row starts 16-byte aligned
  int grid;     // workgroups of the streaming launch (resident capacity)
  // lazy row reads (plain sampling, opt-in): 0 off; 1 the streaming launch
  // of stage 1 (row pair 0 of every sequence); 2 that of stage 2 (rows 1..
  // of the sequences whose first drafted token was accepted); 3 the
  // finishing kernels of a lazy call (rows after position 0 were read only
  // where go is set)
  int lazy;
  int32_t* go;       // [B] lazy: 1 if position 0 was accepted (stage 2 reads the rest)
  int nucrow;        // the nucleus rows came from k_nuc_rows (RowNuc holds M and Z of every row)
  uint64_t* nucc;    // [slots][kNucSlotEntries] k_nuc_rows: candidate buffers (values, then indices, 32 bits each)
  int nuc_keep;      // one candidate buffer per row (slot = row), kept for k_resid_s; else one per workgroup
  uint64_t* nucm;    // [rows][4 waves][nuc_rounds] with nuc_keep: where each round's candidates sit in
                     // the wave's region (start | u0 count << 16 | count << 32)
  int32_t* nuck;     // [rows] with nuc_keep: 1 if k_nuc_rows settled the row, so its buffer holds every kept entry
  int nuc_rounds;    // rounds of 4096 logits per row (the nucm stride)
  // workspace
  TileStat* tiles;   // [rows][P]
  uint64_t* cand;    // [rows][S][cand_w] (top-k): each tile's candidate list
  int cand_w;        // candidate slots per tile
  RowNuc* nuc;       // [rows] (top-p; tree sampling with top-k or top-p: every row)
  float* row_lx;     // [rows] logit of the drafted token a row's accept test reads
                     // (written by the tile holding it; sampling modes)
  // sampling: state handed from k_resid_s to k_resid_final
  SeqState* seq;     // [B]
  double* spart;     // [B][S2] residual-mass partials
  double* wpart;     // [B][S2][kResidSeg] residual weights of each segment (keep_w)
  int keep_w;        // small problem: k_resid_s keeps its weights for
                     // k_resid_final (loaded in its first round, no recompute)
  int tree;          // tree modes: rows have no single drafted token to record
  double* tpart;     // tree sampling: [B][kTreePasses][N][S2] residual masses per segment
  double* tview;     // tree sampling: [B][N][4] row views (-M c64, 1/Z of target, draft) of nodes with children
  uint64_t* tcut;    // tree sampling with top-k / top-p: [B][N][2] cut keys (target, draft) of nodes with children
  int tfilt;         // tree sampling with top-k or top-p: row views come from RowNuc (nuc, every row)
  int S2;            // residual segments per sequence (kResidSeg logits each)
  int rgrp;          // segments per workgroup of k_resid_s
  // top-k: each row's kept set, rank order
  int32_t* k_idx;    // [rows][top_k]
  double* k_e;       // [rows][top_k] exp(z - zmax)
  int32_t* k_cnt;    // [rows] entries kept (after the nucleus, if any)
  double* k_norm;    // [rows] sum of k_e over the kept entries
  int32_t* k_bad;    // [rows] 1 if the row is invalid
  double* k_px;      // [rows] p'(x_j) of the drafted token the row's accept test reads
};

// Launchers (sv_kernels.hip).  Each returns the hipError_t of its launches.
// launch_stream: the one pass over every logit (tile partials; kModeNucRow:
// each row's nucleus result).
// launch_finish: the kernels after it for `filt` (greedy / tree: decision per
// sequence; top-k: merge per row, decision per sequence; nucleus: exact cut
// per row, decision per sequence; plain sampling: residual row sums, residual
// mass per segment, draw per sequence).
hipError_t launch_stream(const Params& p, int mode, int bf16, hipStream_t st,
                         hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);
// Workgroups of the streaming kernel for `mode` one CU keeps resident.
int stream_blocks_per_cu(int mode, int bf16);
hipError_t launch_finish(const Params& p, int filt, int bf16, hipStream_t st, hipEvent_t ev_end = nullptr);
// Lazy row reads: the accept test of position 0 per sequence (after stage 1).
hipError_t launch_lazy_gate(const Params& p, int bf16, hipStream_t st);

}  // namespace sv
