// Device descriptor tables and launchers of the gfx950 kernels.
//
// Every kernel reads its per-item descriptors from a table in device memory
// (inside the caller's workspace or a plan-owned buffer) and finds its item
// with a binary search over the items' first-block (or first-row) indices,
// so one launch covers any number of tensors or matrices.
#pragma once

#include "common.hpp"

namespace mo {

constexpr int kThreads = 256;

// Scope guard: while timing is enabled (mo_timing_enable), brackets the
// launch issued inside its scope with HIP events on `st`.
class KTimer {
 public:
  KTimer(int cls, hipStream_t st);
  ~KTimer();
  KTimer(const KTimer&) = delete;
  KTimer& operator=(const KTimer&) = delete;

 private:
  int cls_;
  hipStream_t st_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  bool active_ = false;
};

// While one exists on a thread, KTimer scopes on that thread record nothing
// and create no events (launches that must not acquire resources).
class KTimerOff {
 public:
  KTimerOff();
  ~KTimerOff();
  KTimerOff(const KTimerOff&) = delete;
  KTimerOff& operator=(const KTimerOff&) = delete;
};

// ----- momentum (elementwise, 2048 elements per block) ----------------------
constexpr int kEltPerThread = 8;
constexpr int kEltIters = 1;
constexpr int kEltPerBlock = kThreads * kEltPerThread * kEltIters;

struct MomSeg {
  const void* g;       // gradient (grad dtype)
  float* b;            // momentum buffer (fp32, in-out)
  void* d;             // direction out (dir dtype) or nullptr
  int64_t numel;
  int64_t start;       // first block of this segment
  int32_t gdt, ddt;
  int32_t vec;         // g, b, d all 16-byte aligned: vector path
  int32_t pad;
};

// stats != nullptr: per-block (amax, sum d^2) of the written direction, one
// StatPartial per block at stats[block].
// phase 0: B <- mu B + G, D from it (the default step);
// phase 1: B <- mu B + G only (no D, no statistics: the buffer before the
//          spectral-cap guard);
// phase 2: B <- kappa[seg] B, then D from it (the guard's factor per segment,
//          the buffer already accumulated by phase 1).
mo_status launch_momentum(const MomSeg* segs, int nseg, int64_t nblocks, float mu, int nesterov,
                          StatPartial* stats, hipStream_t st, int phase = 0,
                          const float* kappa = nullptr);

// ----- spectral-cap guard: power iteration per matrix -------------------------
struct PowSeg {
  const float* b;          // fp32 matrix, rows x cols, row stride ld
  int64_t ld;
  int64_t rblk0;           // first block of the row pass
  int64_t cblk0;           // first block of the column pass (row chunks x column blocks)
  int64_t kblk0;           // first block of the fold of the column pass's partials
  int64_t u_off;           // offset of this matrix's u (rows entries)
  int64_t w_off;           // offset of this matrix's w (cols entries)
  int64_t wp_off;          // offset of its column-pass partials (row chunks x cols entries)
  int32_t rows, cols;
};
struct PowWork {
  double* u;               // sum of rows
  double* w;               // sum of cols
  double* wpart;           // sum of row chunks x cols: B^T u per chunk of rows
  double* rpart;           // one per row-pass block
  double* cpart;           // one per fold block
  double* inv;             // per matrix
  double* sigma;           // per matrix (nullable)
  float* kappa;            // per matrix (nullable): cap / sigma above the cap, else 1
};
// Grid sizes (sums over the matrices of the counts below) and the number of
// column-pass partials.
struct PowGrid {
  int64_t row_blocks = 0, col_blocks = 0, fold_blocks = 0, wpart = 0;
};
int64_t pow_row_blocks(int64_t rows);
int64_t pow_row_chunks(int64_t rows);
int64_t pow_col_blocks(int64_t rows, int64_t cols);
int64_t pow_fold_blocks(int64_t cols);
// `iters` power iterations on every matrix (B^T B from ones / sqrt(cols)),
// then sigma = ||B v|| and the cap factor.  rblk0 / cblk0 / kblk0 / wp_off
// of the table are the running sums of the counts above (wp_off: row chunks
// x cols).
mo_status launch_power_iteration(const PowSeg* segs, int nseg, const PowGrid& g, int iters,
                                 const PowWork& wk, float cap, hipStream_t st);

// ----- AdamW ------------------------------------------------------------------
struct AdamSeg {
  void* p;             // param (dtype)
  const void* g;       // grad (dtype)
  float* m;
  float* v;
  int64_t numel;
  int64_t start;       // first block
  int32_t dt;
  int32_t t0;          // step number for tdelta == 0
  float wd;            // decoupled decay of the item's group
  float beta1, beta2, eps;
  int32_t lr_slot;     // learning rate: lrs[lr_slot] when a table is given
  int32_t pad;
};

// k_adam_sumsq writes one fp64 partial sum per kSumsqBlocksPerPartial blocks
// of kEltPerBlock elements: sumsq_partial_count(nblocks) partials in all.
constexpr int kSumsqBlocksPerPartial = 4;
__host__ __device__ constexpr int64_t sumsq_partial_count(int64_t nblocks) {
  return (nblocks + kSumsqBlocksPerPartial - 1) / kSumsqBlocksPerPartial;
}
mo_status launch_adam_sumsq(const AdamSeg* segs, int nseg, int64_t nblocks, double* partials,
                            hipStream_t st);
// Reduces partials -> T (fp64) and kappa (fp32) at scal[0], (float*)&scal[1].
mo_status launch_adam_norm(const double* partials, int64_t nblocks, float max_norm, double* scal,
                           double* norm_out, hipStream_t st);
// lrs (nullable): per-slot learning rates in device memory, read at each
// segment's lr_slot; NULL = `lr` for every segment.  Step t of a segment is
// t0 + tdelta, or t0 + *tcount - 1 with tcount (nullable) given.
mo_status launch_adam_apply(const AdamSeg* segs, int nseg, int64_t nblocks, const double* scal,
                            float lr, const float* lrs, int32_t tdelta, hipStream_t st,
                            const int32_t* tcount = nullptr);

// Per-step learning-rate table: dst[i] = vals[i] for i < n (n <= kMaxLrSlots),
// written by a kernel from its arguments (no host copy, no memset node); the
// same kernel adds 1 to *tcount (nullable), the grouped step's device count.
constexpr int kMaxLrSlots = 2 * MO_MAX_GROUPS;
mo_status launch_set_lrs(float* dst, const float* vals, int n, hipStream_t st,
                         int32_t* tcount = nullptr);

// ----- row kernels: NorMuon row normalisation and the scaled Muon update -----
enum RowMode : int32_t {
  kRowUpdate = 0,          // W <- W (1 - lr wd) - lr scale O
  kRowNormUpdate = 1,      // NorMuon on O's rows, then the update
  kRowNormInPlace = 2      // NorMuon on O's rows, written back to O
};

struct RowSeg {
  void* w;                 // weight rows (kRowNormInPlace: unused)
  void* o;                 // O rows (read; written back for kRowNormInPlace)
  float* nv;               // NorMuon v (fp32, one per row) or nullptr
  int64_t ld_w, ld_o;
  int64_t start;           // first global row index of this segment
  int32_t rows, cols;
  int32_t w_dt, o_dt;
  float scale;             // shape scale
  float wd;                // decoupled decay of this matrix's group
  int32_t lr_slot;         // learning rate: lrs[lr_slot] when a table is given
  int32_t pad;
};

// nseg == 0: `one` is the only matrix (passed by value, no table needed).
mo_status launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t st);
// lrs (nullable): per-slot learning rates, read at each segment's lr_slot.
mo_status launch_rows(int32_t mode, const RowSeg* segs, int nseg, const RowSeg& one,
                      int64_t total_rows, float lr, const float* lrs, float beta2, float eps,
                      hipStream_t st);

// ----- Newton-Schulz ------------------------------------------------------------
constexpr int kPrepTile = 64;   // prep / stats tile edge
constexpr int kGemmTile = 128;  // small GEMM tile edge (M and N); matrices are padded to their tile

struct PrepItem {
  const void* in;          // D in stored orientation, rows r x cols c, stride ld_in
  int64_t ld_in;
  int64_t sbuf;            // pool offset of the stored-orientation copy (rp x cp), -1 = none
  int64_t stbuf;           // pool offset of the transposed copy (cp x rp), -1 = none
  int64_t start;           // first prep tile of this item
  int64_t stat_begin;      // partial-statistics range of this item
  int64_t stat_end;
  int32_t r, c;
  int32_t rp, cp;          // padded (multiples of kGemmTile)
  int32_t tiles_c;         // cp / kPrepTile
  int32_t in_dt;
  int32_t vec;             // rows of `in` allow 16-byte loads of 8 elements
  int32_t slice;           // fallback table only: the slice's index (scale and flag)
};

struct GemmProb {
  int64_t a_off;           // A operand: M x K row-major (K contiguous)
  int64_t b_off;           // B operand: N x K row-major, or K x N row-major when the
                           // launch reads B K-major
  int64_t c_off;           // direct output (M x N), -1 = none
  int64_t ct_off;          // transposed output (N x M), -1 = none
  int64_t e_off;           // epilogue input (same layout as c), -1 = none
  int32_t lda, ldb, ldc, ldct, lde;
  int32_t K;
  int32_t tiles_m, tiles_n;
  int32_t sym;             // only tiles (i <= j); mirror written through ct
  int32_t start;           // first tile of this problem
  int32_t item;            // slice index (the last update of a slice), else -1: with a
                           // weight table, the launch applies the Muon update to that
                           // slice's weights instead of writing its output
  int32_t sitem;           // slice index whose normalisation scale s multiplies the
                           // product (iteration 0 reading the unscaled D in place:
                           // s^2 for the Gram, s for the update), else -1
  int64_t alt_off;         // with sitem >= 0: the pool's X0, read instead of D (and
                           // no scaling) when the slice's range flag is set
  int64_t c2_off;          // bf16 product without E only: a second output
                           // c1b C + cdb I (layout and mirror as c), -1 = none
  int32_t a_rows, b_rows;  // > 0: rows of A (of B stored N x K) that hold data;
                           // in 128 x 128 tiles the loads of later rows read
                           // zero (the padding of a slice, or a slice read in
                           // place whose padded rows are not stored); 0: all
                           // rows.  (B stored K x N is read up to K, which
                           // stops at its data.)
};

struct FinalItem {         // NS output copy (stored orientation)
  void* out;
  int64_t ld_out;
  int64_t src;             // pool offset of the stored-orientation buffer
  int64_t start;           // first row
  int32_t rows, cols;
  int32_t ld_src;
  int32_t out_dt;
};

// Statistics of D over the prep tiles -> partials[tile].
mo_status launch_ns_stats(const PrepItem* items, int n, int64_t ntiles, StatPartial* partials,
                          hipStream_t st);
// Per-item scale = 1 / (alpha (||D||/alpha + 1e-7)), alpha = max(amax, 1e-7).
// range_fb (nullable): per item, 1 when max|D| lies outside [2^-50, 2^40],
// where products of the unscaled D could leave fp32's normal range (the
// in-place first iteration then falls back to the prepared X0), else 0.
mo_status launch_ns_scale(const PrepItem* items, int n, const StatPartial* partials,
                          float* scale, int32_t* range_fb, hipStream_t st);
// X0 (scaled, padded, both orientations) into the pool.  elem = 2 (bf16) or 4.
mo_status launch_ns_prep(const PrepItem* items, int n, int64_t ntiles, const float* scale,
                         void* pool, int elem, hipStream_t st);
// The prep copy for the items (bf16, slice index in .slice) whose range flag is
// set: a fixed grid that skips unflagged items, so the common case (no flag)
// costs one pass over the item table.
mo_status launch_ns_prep_fallback(const PrepItem* items, int n, const float* scale,
                                  const int32_t* range_fb, void* pool, hipStream_t st);
// One batched GEMM phase:  out = c0 * E + c1 * (A_op B_op^T), with square
// workgroup tiles of edge `tile` (128 or 256; the problems' padding).
// Slice-resident Newton-Schulz (all iterations in one launch) for slices whose
// padded short side is 128: one workgroup per slice.
struct SmallProb {
  int64_t x_off[2];        // pool offsets of the two iterate buffers (128 x lp each)
  int32_t lp;              // padded long side = row stride of the iterates
  int32_t tall;            // last iteration writes the result transposed (lp x 128)
  int32_t item;            // index of the slice's prep item and normalisation scale
  int32_t direct;          // the first two passes read the item's input D (bf16,
                           // 128 x lp, row stride lp) instead of the prepared X0
};
struct NsCoeffTable {
  float a[MO_NS_MAX_STEPS], b[MO_NS_MAX_STEPS], c[MO_NS_MAX_STEPS];
};
constexpr int kSmallS = 128;
// wt (nullable): per-slice weight rows (the RowSeg of the slice index); the
// last iteration then applies W <- W (1 - lr wd) - lr scale O to them instead
// of writing O.  Requires bf16 O, cols % 8 == 0 and 16-byte aligned rows.
// gspace: run the iterations in Gram space (two passes over X; see
// build_ns_layout), the result in the second iterate buffer.
// range_fb (nullable): the per-slice range flags of launch_ns_scale; an
// in-place slice whose flag is clear multiplies D unscaled and scales the
// results (otherwise X0 = bf16(s D) is formed in LDS).
mo_status launch_ns_small(const SmallProb* probs, int n, void* pool, const PrepItem* items,
                          const float* scale, const float* coeffs, int steps, const RowSeg* wt,
                          float lr, const float* lrs, hipStream_t st, int gspace = 0,
                          const int32_t* range_fb = nullptr);

// C = c1 A B (+ c0 E) (+ cd I on diagonal tiles).  has_e: 0 no E term; 1 E
// read from e_off; 2 (bf16) E is the left operand itself (e_off = a_off in
// every problem, square s x s products), added from its slabs in LDS (with
// c1 != 0; else read as for 1).  bk = 1: B is read K-major (K x N row-major)
// through LDS transpose reads; no E term, and the output goes straight from
// registers to c (or, transposed, to ct).
// wt (nullable, bf16 with bk = 1 only): problems with item >= 0 apply the Muon
// update to the weights of slice `item` (as launch_ns_small) instead of
// writing their output, at learning rate lrs[wt[item].lr_slot] (lrs given) or lr.  pscale (nullable): problems with sitem >= 0 scale
// c1 by pscale[sitem]^2 (bk = 0) or pscale[sitem] (bk = 1), unless
// pfb[sitem] is set: they then read alt_off for the X operand(s), unscaled.
// c1b, cdb: the constants of the second outputs (c2_off).
// few_max: bf16 launches of fewer 128 x 128 tiles than this use the 8-wave
// variant.  persist: every problem has the same K (equal tile times), so the
// launch may take only the workgroups that fit on the device at once, each
// running several tiles in turn.
mo_status launch_ns_gemm(const GemmProb* probs, int n, int64_t ntiles, bool persist, int tile,
                         int64_t few_max, int bk,
                         void* pool, int elem, float c0, float c1, int has_e, float cd,
                         const RowSeg* wt, float lr, const float* lrs, const float* pscale,
                         const int32_t* pfb, hipStream_t st, float c1b = 0.f, float cdb = 0.f);
mo_status launch_ns_final(const FinalItem* items, int n, int64_t total_rows, const void* pool,
                          int elem, hipStream_t st);

}  // namespace mo
