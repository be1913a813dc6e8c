// Host-side declarations shared by the library's translation units.
#pragma once

#include <vector>

#include "kernels.hpp"

namespace mo {

struct Slice {
  int64_t off;   // first stored row
  int64_t rows;
  int64_t cols;
};

mo_status expand_view(int64_t rows, int64_t cols, int32_t view_ndim, const int64_t* view,
                      int32_t nsplit, const int64_t* split, std::vector<Slice>& out);
mo_status route(const mo_param_desc* d, int32_t n, mo_route_out* out, int32_t* ngroups);

// Excluded split pieces (Qwen3.8 optimizer notes, section 4: sub-blocks of a
// fused weight that AdamW steps).  A mask is valid with split sizes, bits
// below nsplit only, and at least one piece left to Muon.  expand_view lists
// slices view matrix by view matrix, split piece by split piece, so slice j
// is piece j % nsplit.
inline bool exclude_ok(int32_t nsplit, uint32_t mask) {
  if (mask == 0) return true;
  if (nsplit <= 0 || nsplit > 31) return false;
  const uint32_t all = (1u << nsplit) - 1u;
  return (mask & ~all) == 0 && mask != all;
}
inline bool piece_excluded(uint32_t mask, int32_t nsplit, size_t j) {
  return mask != 0 && nsplit > 0 && ((mask >> (j % static_cast<size_t>(nsplit))) & 1u) != 0;
}

// Newton-Schulz layout of a batch of independent matrices: padded pool
// buffers per matrix and the GEMM / prep problem tables (pool offsets only;
// device pointers and statistics ranges are filled by the caller).  Matrices
// are bucketed by GEMM tile size: short side >= kBigTileMinS -> 256 x 256
// tiles (when the batch has at least kBigTileMinWork such Gram tiles),
// otherwise 128 x 128; each bucket has its own tables and launches.
//
// Per matrix (s = short side, l = long side, both padded to the tile): two
// iterate buffers X0, X1 (s x l, short-side rows) used in turn, P (s x s) and,
// for tables with a quintic-type row, A (s x s).  Iteration k reads X[k % 2]
// and writes X[(k + 1) % 2]; the last iteration of a tall matrix writes its
// result transposed (stored orientation, l x s) into that buffer instead.
// bf16 matrices whose padded short side is kSmallS go to the slice-resident
// kernel instead (same iterate buffers and conventions, P kept in LDS).
constexpr int kBigTile = 256;
constexpr int kBigTileMinS = 512;
constexpr int64_t kGramSpaceMinS = 64;
// Gram space carries A_k = X_k X_k^T, whose small eigenvalues are the squares
// of X's small singular values, so its bf16 rounding noise in those
// directions is amplified by the table's gain prod_k a_k^2 (p'(0) = a_k per
// iteration, squared), where the plain iteration's grows with prod_k a_k.
// Emulated bf16 rounding over spiked and prescribed-spectrum inputs stays
// within the bf16 tolerance up to a gain of about 650 and leaves it past
// about 1900; the threshold admits the cubic set for up to 8 iterations and
// the quintic for up to 5.
constexpr double kGramSpaceMaxGain = 1024.0;

// Resolved Newton-Schulz options (mo_ns_options with the defaults applied).
struct NsOpts {
  bool gram_space = true;
  int64_t big_tile_min_work = 512;   // 256-bucket Gram tiles: 2 per CU
  int64_t few_tile_max = 512;        // 8-wave 128 x 128 launches below this
};
// NULL = defaults; MO_EINVAL for out-of-range fields.
mo_status resolve_ns_options(const mo_ns_options* o, NsOpts& out);
// prod_k a_k^2 <= kGramSpaceMaxGain over the table's rows.
bool gram_gain_ok(const float* coeffs, int steps);

struct NsBucket {
  int tile = kGemmTile;
  // [parity of the iteration]; fin = the update of the last iteration.
  // gram_p0 / gram_a0 / upd0 / fin0: iteration 0, which reads the input D in
  // place (with the scale folded into the products) for slices that allow it
  std::vector<GemmProb> gram_p[2], gram_a[2], square, upd[2], fin[2];
  std::vector<GemmProb> gram_p0, gram_a0, upd0, fin0;
  int64_t gram_tiles = 0, square_tiles = 0, upd_tiles = 0;
  // Gram-space mode: one problem table per launch, in order (see NsLayout)
  std::vector<std::vector<GemmProb>> gs;
  std::vector<int32_t> gs_kind, gs_k;   // GsKind; coefficient row of the launch
  std::vector<int64_t> gs_tiles;
};

// Launch kinds of the Gram-space sequence.
enum GsKind : int32_t {
  kGsGram = 0,       // A0 = X0 X0^T, and Q1 = a0 I + b0 A0 as a second output
                     // (cubic-type row 0)
  kGsProd = 1,       // C = a E + b (U V^T) over s x s operands (symmetric result)
  kGsFinal = 2,      // X_N = Q_N X0 (K-major B), the last update
  kGsProdP = 3,      // P = c (A A^T) + b A + a I (quintic-type row, E = A)
  kGsProdPlain = 4,  // C = U V^T (quintic-type row: T = P A, A' = T P, Q' = P Q)
};

struct NsLayout {
  int elem = 2;
  bool need_a = false;
  int n = 0;
  std::vector<PrepItem> prep;
  // prep items (X0 into the pool) of the slices whose iteration 0 reads D in
  // place, run only for those whose range flag is set (slice index in .slice)
  std::vector<PrepItem> prep_fb;
  std::vector<NsBucket> buckets;
  std::vector<SmallProb> small;
  int64_t prep_tiles = 0;
  std::vector<int64_t> x_off[2];
  std::vector<int32_t> tall, sp, lp;
  std::vector<uint8_t> gspace;   // slice runs the Gram-space sequence
  std::vector<uint8_t> kind;     // 0: GEMM, 128 x 128 tiles; 1: GEMM, 256 x 256; 2: slice-resident
  std::vector<SmallProb> small_gs;   // slice-resident slices run in Gram space
  int64_t pool_elems = 0;
  int64_t few_tile_max = 512;        // 8-wave 128 x 128 launches below this many tiles

  // buffer of the final iterate (stored orientation) and its row stride
  int64_t final_off(int i, int steps) const { return x_off[gspace[i] ? 1 : steps & 1][i]; }
  int32_t final_ld(int i) const { return tall[i] ? sp[i] : lp[i]; }
};

// coeffs: the [steps][3] table (a, b, c) per iteration; its rows decide
// whether A is kept (a row with c != 0) and, with `opt`, which slices run in
// Gram space (see mo_ns_options).
//
// direct_ok[i] (nullable: none) says that slice i's input can be read in
// place: bf16, row stride equal to cols, 16-byte aligned.  Such a slice
// skips the prep copy (its prep item writes nothing, and has no tiles at all
// unless the statistics are taken over the prep tiles, stats_from_prep) when
//  * it goes to the slice-resident kernel with 128 rows and a multiple of 128
//    columns, or
//  * in_off (nullable) gives its input's element offset from the pool base,
//    it is not tall, its long side is a multiple of its GEMM tile and its
//    short side is that tile's multiple (or, in 128 x 128 tiles, 64's):
//    iteration 0 then reads D itself, the scale folded into the products
//    (the rows past a padded short side read zero, see GemmProb's a_rows).
//
// Gram space on the GEMM path (rectangular slices, l >= 1.25 s; on a square
// slice it executes the same flops as the plain iteration in one more
// launch): every iterate is P_k ... P_0 X0 with P_k = a_k I + b_k A_k +
// c_k A_k^2, A_{k+1} = P_k A_k P_k, so the iterations run on s x s matrices
// (A_0 = X0 X0^T, then T = P A, A' = T P, Q' = P Q) and X0 is multiplied
// once, by Q_N, at the end.  A cubic-type row keeps P implicit through the E
// term (T = a A + b A A, A' = a T + b T A, Q' = a Q + b Q A: three products);
// a quintic-type row materialises P = c A A + b A + a I in one product with
// an E term, then three plain products.
// The slice-resident kernel does the same with its 128 x 128 matrices in LDS
// (quintic-type rows included, P_k = a_k I + R_k with R_k = b_k A_k +
// c_k A_k^2), for slices with a short side of at least kGramSpaceMinS: on
// smaller ones the bf16 products of Gram space lose more than the plain
// iteration (O(1) entries).
void build_ns_layout(NsLayout& L, const int64_t* rows, const int64_t* cols, int n, int elem,
                     const float* coeffs, int steps, const NsOpts& opt,
                     const uint8_t* direct_ok, bool stats_from_prep,
                     const int64_t* in_off = nullptr);

// Byte offsets of the device tables inside one contiguous table block.
struct NsBucketTables {
  size_t gram_p[2] = {0, 0}, gram_a[2] = {0, 0}, square = 0, upd[2] = {0, 0}, fin[2] = {0, 0};
  size_t gram_p0 = 0, gram_a0 = 0, upd0 = 0, fin0 = 0;
  std::vector<size_t> gs;
};
struct NsTables {
  size_t prep = 0, prep_fb = 0, small = 0, small_gs = 0, bytes = 0;
  std::vector<NsBucketTables> b;
};
NsTables ns_table_offsets(const NsLayout& L);
void ns_pack_tables(const NsLayout& L, const NsTables& T, std::vector<char>& buf);

// Asynchronous host -> device copy through a pinned staging buffer; `src`
// may be released when this returns.
mo_status stage_upload(void* dst, const void* src, size_t bytes, hipStream_t st);

// Whether the layout has at least two of the independent chains of launches
// (slice-resident kernel, Gram-space GEMM sequence, plain-iteration GEMM),
// which ns_run_iterations can put on two streams.
bool ns_has_two_chains(const NsLayout& L);

// Enqueue the Newton-Schulz iterations on the prepared pool.
// `scale` holds the per-slice normalisation scales (the prep kernel's).
// wt (nullable): per-slice weight rows; the last iteration then applies the
// Muon update to them instead of writing O (bf16 pool, every slice eligible),
// at learning rate lrs[row.lr_slot] (lrs given, device) or lr.
// range_fb (nullable): the per-slice range flags of launch_ns_scale, which
// send a slice's in-place iteration 0 back to the prepared X0.
// st2 (nullable): a second stream.  The Gram-space sequence stays on `st`
// and the slice-resident and plain-iteration launches go to st2 (without a
// Gram-space sequence, the plain iteration stays on `st`).  The caller
// orders st2 after the work `st` holds so far and joins it back afterwards.
mo_status ns_run_iterations(const NsLayout& L, const char* dtab, const NsTables& T, void* pool,
                            const float* scale, const float* coeffs, int steps, const RowSeg* wt,
                            float lr, const float* lrs, const int32_t* range_fb,
                            hipStream_t st, hipStream_t st2 = nullptr);

// Validates an AdamW call (adamw_clip_step's arguments) and writes one
// AdamSeg per item with a gradient into segs (capacity max_segs, host
// memory); *nseg and *nblocks receive the counts.  MO_EWORKSPACE when more
// than max_segs items have a gradient.
mo_status adam_segments(const mo_adamw_item* items, int32_t n, float lr, float beta1, float beta2,
                        float eps, float max_norm, AdamSeg* segs, int max_segs, int* nseg,
                        int64_t* nblocks);

// Power-iteration work areas for a list of matrices, laid out by the cursor
// (byte offsets; the table of PowSeg first); pow_fill writes the table's
// block starts and vector offsets.
struct PowLayout {
  size_t tab = 0, u = 0, w = 0, wpart = 0, rpart = 0, cpart = 0, inv = 0, sigma = 0, kappa = 0;
  int64_t rows = 0, cols = 0;
  PowGrid grid;
};
PowLayout pow_layout(const int64_t* rows, const int64_t* cols, int n, WsCursor& c);
void pow_fill(PowSeg* segs, const int64_t* rows, const int64_t* cols, int n);
PowWork pow_work(const PowLayout& L, char* base);

// True while kernel timing (mo_timing_enable) is on.
bool timing_enabled();

}  // namespace mo
