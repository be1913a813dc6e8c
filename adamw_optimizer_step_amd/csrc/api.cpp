// C entry points of the individual optimizer stages.  Each validates all of
// its arguments before enqueueing anything, copies its descriptor table into
// the caller's workspace and launches one kernel per stage on `stream`.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "host.hpp"

using namespace mo;

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

mo_status upload(void* dst, const void* src, size_t bytes, hipStream_t st) {
  return stage_upload(dst, src, bytes, st);
}

mo_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MO_OK;
  if (!ws) return fail(MO_EWORKSPACE, "workspace of %zu bytes required", need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(MO_EALIGN, "workspace must be 256-byte aligned");
  if (have < need) return fail(MO_EWORKSPACE, "workspace has %zu bytes, %zu required", have, need);
  return MO_OK;
}

// ----- momentum --------------------------------------------------------------
size_t momentum_table_bytes(int32_t n) { return align_up(sizeof(MomSeg) * (n > 0 ? n : 0), 256); }

// ----- NS workspace layout ---------------------------------------------------
struct NsWs {
  NsTables tabs;
  size_t tab = 0, partials = 0, scale = 0, fin = 0, pool = 0, total = 0;
};

NsWs ns_ws_layout(const NsLayout& L) {
  NsWs w;
  w.tabs = ns_table_offsets(L);
  WsCursor c;
  w.tab = c.take(w.tabs.bytes);
  w.fin = c.take(sizeof(FinalItem) * L.n);
  w.partials = c.take(sizeof(StatPartial) * L.prep_tiles);
  w.scale = c.take(sizeof(float) * L.n);
  w.pool = c.take(static_cast<size_t>(L.pool_elems) * L.elem);
  w.total = align_up(c.off, 256);
  return w;
}

mo_status validate_ns_items(const mo_ns_item* items, int32_t n, int32_t precision) {
  if (n <= 0 || !items) return fail(MO_EINVAL, "no Newton-Schulz items");
  if (precision != MO_NS_BF16 && precision != MO_NS_F32)
    return fail(MO_EINVAL, "unknown precision %d", precision);
  for (int32_t i = 0; i < n; ++i) {
    const mo_ns_item& it = items[i];
    if (!it.in || !it.out) return fail(MO_EINVAL, "item %d: NULL pointer", i);
    if (!valid_dtype(it.in_dtype) || !valid_dtype(it.out_dtype))
      return fail(MO_EDTYPE, "item %d: bad dtype", i);
    if (it.rows < 1 || it.cols < 1 || it.rows > 65536 || it.cols > 65536)
      return fail(MO_ESHAPE, "item %d: shape (%lld, %lld) outside [1, 65536]", i,
                  (long long)it.rows, (long long)it.cols);
    if (it.ld_in < it.cols || it.ld_out < it.cols)
      return fail(MO_ESHAPE, "item %d: row stride smaller than cols", i);
  }
  return MO_OK;
}

void ns_layout_from_items(const mo_ns_item* items, int32_t n, int32_t precision,
                          const float* coeffs, int32_t steps, const NsOpts& opt, NsLayout& L) {
  std::vector<int64_t> r(n), c(n);
  std::vector<uint8_t> direct(n);
  for (int32_t i = 0; i < n; ++i) {
    r[i] = items[i].rows;
    c[i] = items[i].cols;
    // an input the slice-resident kernel can read in place (it must be the
    // pool's element type, unpadded rows, 16-byte aligned)
    direct[i] = precision == MO_NS_BF16 && items[i].in_dtype == MO_BF16 &&
                items[i].ld_in == items[i].cols && aligned16(items[i].in);
  }
  build_ns_layout(L, r.data(), c.data(), n, precision == MO_NS_F32 ? 4 : 2, coeffs, steps, opt,
                  direct.data(), true);
}

mo_status check_coeffs(const float* coeffs, int32_t steps) {
  if (steps < 1 || steps > MO_NS_MAX_STEPS || !coeffs)
    return fail(MO_EINVAL, "steps must be in [1, %d] with a coefficient table", MO_NS_MAX_STEPS);
  for (int k = 0; k < 3 * steps; ++k)
    if (!std::isfinite(coeffs[k])) return fail(MO_EINVAL, "non-finite coefficient");
  return MO_OK;
}

// ----- AdamW -----------------------------------------------------------------
struct AdamWs {
  size_t tab = 0, partials = 0, scal = 0, total = 0;
  int64_t nblocks = 0;
  int nseg = 0;
};

AdamWs adam_ws_layout(const mo_adamw_item* items, int32_t n) {
  AdamWs w;
  for (int32_t i = 0; i < n; ++i)
    if (items[i].grad && items[i].numel > 0) {
      w.nblocks += ceil_div(items[i].numel, kEltPerBlock);
      ++w.nseg;
    }
  WsCursor c;
  w.tab = c.take(sizeof(AdamSeg) * w.nseg);
  w.partials = c.take(sizeof(double) * w.nblocks);
  w.scal = c.take(2 * sizeof(double));
  w.total = align_up(c.off, 256);
  return w;
}

}  // namespace

namespace mo {

mo_status adam_segments(const mo_adamw_item* items, int32_t n, float lr, float beta1, float beta2,
                        float eps, float max_norm, AdamSeg* segs, int max_segs, int* nseg,
                        int64_t* nblocks) {
  if (n < 0 || (n > 0 && !items)) return fail(MO_EINVAL, "bad item list");
  if (!std::isfinite(lr) || !std::isfinite(beta1) || !std::isfinite(beta2) ||
      !std::isfinite(eps) || beta1 < 0.f || beta1 >= 1.f || beta2 < 0.f || beta2 >= 1.f ||
      std::isnan(max_norm))
    return fail(MO_EINVAL, "bad hyper-parameter");
  *nseg = 0;
  *nblocks = 0;
  for (int32_t i = 0; i < n; ++i) {
    const mo_adamw_item& it = items[i];
    if (it.numel < 0) return fail(MO_EINVAL, "item %d: negative numel", i);
    if (!it.grad || it.numel == 0) continue;
    if (!it.param || !it.exp_avg || !it.exp_avg_sq) return fail(MO_EINVAL, "item %d: NULL", i);
    if (!valid_dtype(it.dtype)) return fail(MO_EDTYPE, "item %d: bad dtype", i);
    if (it.step < 1) return fail(MO_EINVAL, "item %d: step must be >= 1", i);
    if (!std::isfinite(it.weight_decay)) return fail(MO_EINVAL, "item %d: bad decay", i);
    if (!aligned16(it.param) || !aligned16(it.grad) || !aligned16(it.exp_avg) ||
        !aligned16(it.exp_avg_sq))
      return fail(MO_EALIGN, "item %d: pointers must be 16-byte aligned", i);
    if (*nseg >= max_segs)
      return fail(MO_EWORKSPACE, "more than %d items with a gradient", max_segs);
    AdamSeg& s = segs[(*nseg)++];
    s.p = it.param; s.g = it.grad; s.m = it.exp_avg; s.v = it.exp_avg_sq; s.numel = it.numel;
    s.start = *nblocks; s.dt = it.dtype; s.t0 = it.step; s.wd = it.weight_decay;
    s.beta1 = beta1; s.beta2 = beta2; s.eps = eps; s.lr_slot = 0; s.pad = 0;
    *nblocks += ceil_div(it.numel, kEltPerBlock);
  }
  return MO_OK;
}

PowLayout pow_layout(const int64_t* rows, const int64_t* cols, int n, WsCursor& c) {
  PowLayout L;
  for (int i = 0; i < n; ++i) {
    L.rows += rows[i];
    L.cols += cols[i];
    L.grid.row_blocks += pow_row_blocks(rows[i]);
    L.grid.col_blocks += pow_col_blocks(rows[i], cols[i]);
    L.grid.fold_blocks += pow_fold_blocks(cols[i]);
    L.grid.wpart += align_up(pow_row_chunks(rows[i]) * cols[i], 4);   // 32-byte aligned shares
  }
  L.tab = c.take(sizeof(PowSeg) * n);
  L.u = c.take(sizeof(double) * L.rows);
  L.w = c.take(sizeof(double) * L.cols);
  L.wpart = c.take(sizeof(double) * L.grid.wpart);
  L.rpart = c.take(sizeof(double) * L.grid.row_blocks);
  L.cpart = c.take(sizeof(double) * L.grid.fold_blocks);
  L.inv = c.take(sizeof(double) * n);
  L.sigma = c.take(sizeof(double) * n);
  L.kappa = c.take(sizeof(float) * n);
  return L;
}

void pow_fill(PowSeg* segs, const int64_t* rows, const int64_t* cols, int n) {
  int64_t rb = 0, cb = 0, kb = 0, uo = 0, wo = 0, po = 0;
  for (int i = 0; i < n; ++i) {
    PowSeg& s = segs[i];
    s.rblk0 = rb;
    s.cblk0 = cb;
    s.kblk0 = kb;
    s.u_off = uo;
    s.w_off = wo;
    s.wp_off = po;
    s.rows = static_cast<int32_t>(rows[i]);
    s.cols = static_cast<int32_t>(cols[i]);
    rb += pow_row_blocks(rows[i]);
    cb += pow_col_blocks(rows[i], cols[i]);
    kb += pow_fold_blocks(cols[i]);
    uo += rows[i];
    wo += cols[i];
    po += align_up(pow_row_chunks(rows[i]) * cols[i], 4);
  }
}

PowWork pow_work(const PowLayout& L, char* base) {
  PowWork w;
  w.u = reinterpret_cast<double*>(base + L.u);
  w.w = reinterpret_cast<double*>(base + L.w);
  w.wpart = reinterpret_cast<double*>(base + L.wpart);
  w.rpart = reinterpret_cast<double*>(base + L.rpart);
  w.cpart = reinterpret_cast<double*>(base + L.cpart);
  w.inv = reinterpret_cast<double*>(base + L.inv);
  w.sigma = reinterpret_cast<double*>(base + L.sigma);
  w.kappa = reinterpret_cast<float*>(base + L.kappa);
  return w;
}

}  // namespace mo

namespace {

mo_status spectral_items(const mo_spectral_item* items, int32_t n, std::vector<int64_t>& r,
                         std::vector<int64_t>& c) {
  if (n <= 0 || !items) return fail(MO_EINVAL, "no matrices");
  r.resize(n);
  c.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    const mo_spectral_item& it = items[i];
    if (!it.b) return fail(MO_EINVAL, "item %d: NULL matrix", i);
    if (it.rows < 1 || it.cols < 1 || it.rows > 65536 || it.cols > 65536)
      return fail(MO_ESHAPE, "item %d: shape (%lld, %lld) outside [1, 65536]", i,
                  static_cast<long long>(it.rows), static_cast<long long>(it.cols));
    if (it.ld < it.cols) return fail(MO_ESHAPE, "item %d: row stride smaller than cols", i);
    r[i] = it.rows;
    c[i] = it.cols;
  }
  return MO_OK;
}

}  // namespace

extern "C" {

size_t muon_spectral_workspace_bytes(const mo_spectral_item* items, int32_t n) {
  std::vector<int64_t> r, c;
  if (spectral_items(items, n, r, c) != MO_OK) return 0;
  WsCursor cur;
  pow_layout(r.data(), c.data(), n, cur);
  return align_up(cur.off, 256);
}

mo_status muon_spectral_estimate(const mo_spectral_item* items, int32_t n, int32_t iters,
                                 double* sigma_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  std::vector<int64_t> r, c;
  mo_status s = spectral_items(items, n, r, c);
  if (s != MO_OK) return s;
  if (iters < 0 || iters > MO_NS_MAX_STEPS)
    return fail(MO_EINVAL, "iters must be in [0, %d]", MO_NS_MAX_STEPS);
  if (!sigma_out) return fail(MO_EINVAL, "NULL sigma_out");
  WsCursor cur;
  const PowLayout L = pow_layout(r.data(), c.data(), n, cur);
  if ((s = check_ws(ws, ws_bytes, align_up(cur.off, 256))) != MO_OK) return s;
  std::vector<PowSeg> segs(n);
  pow_fill(segs.data(), r.data(), c.data(), n);
  for (int32_t i = 0; i < n; ++i) {
    segs[i].b = items[i].b;
    segs[i].ld = items[i].ld;
  }
  char* base = static_cast<char*>(ws);
  hipStream_t st = as_stream(stream);
  if ((s = upload(base + L.tab, segs.data(), segs.size() * sizeof(PowSeg), st)) != MO_OK) return s;
  PowWork wk = pow_work(L, base);
  wk.sigma = sigma_out;
  wk.kappa = nullptr;
  return launch_power_iteration(reinterpret_cast<const PowSeg*>(base + L.tab), n, L.grid, iters,
                                wk, 0.f, st);
}


size_t muon_momentum_workspace_bytes(int32_t n) { return momentum_table_bytes(n); }

mo_status muon_momentum(const mo_momentum_item* items, int32_t n, float mu, int32_t nesterov,
                        void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (n < 0 || (n > 0 && !items)) return fail(MO_EINVAL, "bad item list");
  if (!std::isfinite(mu)) return fail(MO_EINVAL, "mu must be finite");
  std::vector<MomSeg> segs;
  int64_t nblocks = 0;
  for (int32_t i = 0; i < n; ++i) {
    const mo_momentum_item& it = items[i];
    if (it.numel < 0) return fail(MO_EINVAL, "item %d: negative numel", i);
    if (!it.grad || it.numel == 0) continue;
    if (!it.momentum) return fail(MO_EINVAL, "item %d: NULL momentum", i);
    if (!valid_dtype(it.grad_dtype) || (it.dir && !valid_dtype(it.dir_dtype)))
      return fail(MO_EDTYPE, "item %d: bad dtype", i);
    if (!aligned16(it.grad) || !aligned16(it.momentum) || (it.dir && !aligned16(it.dir)))
      return fail(MO_EALIGN, "item %d: pointers must be 16-byte aligned", i);
    MomSeg s;
    s.g = it.grad; s.b = it.momentum; s.d = it.dir; s.numel = it.numel; s.start = nblocks;
    s.gdt = it.grad_dtype; s.ddt = it.dir ? it.dir_dtype : MO_F32; s.vec = 1; s.pad = 0;
    nblocks += ceil_div(it.numel, kEltPerBlock);
    segs.push_back(s);
  }
  if (segs.empty()) return MO_OK;
  mo_status s = check_ws(ws, ws_bytes, momentum_table_bytes(static_cast<int32_t>(segs.size())));
  if (s != MO_OK) return s;
  hipStream_t st = as_stream(stream);
  if ((s = upload(ws, segs.data(), segs.size() * sizeof(MomSeg), st)) != MO_OK) return s;
  return launch_momentum(static_cast<const MomSeg*>(ws), static_cast<int>(segs.size()), nblocks,
                         mu, nesterov, nullptr, st);
}

void mo_ns_options_default(mo_ns_options* o) {
  if (!o) return;
  o->gram_space = 1;
  o->big_tile_min_work = -1;
  o->few_tile_max = -1;
  o->reserved = 0;
}

size_t ns_workspace_bytes(const mo_ns_item* items, int32_t n, const float* coeffs, int32_t steps,
                          int32_t precision, const mo_ns_options* opts) {
  if (validate_ns_items(items, n, precision) != MO_OK) return 0;
  NsOpts opt;
  if (resolve_ns_options(opts, opt) != MO_OK) return 0;
  if (coeffs) {
    if (check_coeffs(coeffs, steps) != MO_OK) return 0;
    NsLayout L;
    ns_layout_from_items(items, n, precision, coeffs, steps, opt, L);
    return ns_ws_layout(L).total;
  }
  // any table: the larger of the quintic-capable plain layout and the
  // Gram-space layout (whose GEMM slices keep five s x s buffers)
  const float quintic[3] = {1.875f, -1.25f, 0.375f}, cubic[3] = {1.5f, -0.5f, 0.f};
  NsLayout La, Lb;
  ns_layout_from_items(items, n, precision, quintic, 1, opt, La);
  ns_layout_from_items(items, n, precision, cubic, 1, opt, Lb);
  return std::max(ns_ws_layout(La).total, ns_ws_layout(Lb).total);
}

mo_status ns_orthogonalize_batched(const mo_ns_item* items, int32_t n, const float* coeffs,
                                   int32_t steps, int32_t precision, const mo_ns_options* opts,
                                   void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  mo_status s = validate_ns_items(items, n, precision);
  if (s != MO_OK) return s;
  if ((s = check_coeffs(coeffs, steps)) != MO_OK) return s;
  NsOpts opt;
  if ((s = resolve_ns_options(opts, opt)) != MO_OK) return s;
  NsLayout L;
  ns_layout_from_items(items, n, precision, coeffs, steps, opt, L);
  const NsWs W = ns_ws_layout(L);
  if ((s = check_ws(ws, ws_bytes, W.total)) != MO_OK) return s;

  char* base = static_cast<char*>(ws);
  std::vector<FinalItem> fin(n);
  int64_t rows = 0;
  for (int32_t i = 0; i < n; ++i) {
    PrepItem& p = L.prep[i];
    p.in = items[i].in;
    p.ld_in = items[i].ld_in;
    p.in_dt = items[i].in_dtype;
    p.vec = aligned16(p.in) && (p.ld_in * dtype_size(p.in_dt)) % 16 == 0;
    p.stat_begin = p.start;
    p.stat_end = p.start + static_cast<int64_t>(p.rp / kPrepTile) * p.tiles_c;
    FinalItem& f = fin[i];
    f.out = items[i].out;
    f.ld_out = items[i].ld_out;
    f.src = L.final_off(i, steps);
    f.ld_src = L.final_ld(i);
    f.rows = static_cast<int32_t>(items[i].rows);
    f.cols = static_cast<int32_t>(items[i].cols);
    f.out_dt = items[i].out_dtype;
    f.start = rows;
    rows += items[i].rows;
  }
  std::vector<char> tab;
  ns_pack_tables(L, W.tabs, tab);
  hipStream_t st = as_stream(stream);
  if ((s = upload(base + W.tab, tab.data(), tab.size(), st)) != MO_OK) return s;
  if ((s = upload(base + W.fin, fin.data(), fin.size() * sizeof(FinalItem), st)) != MO_OK) return s;
  const PrepItem* dprep = reinterpret_cast<const PrepItem*>(base + W.tab + W.tabs.prep);
  StatPartial* partials = reinterpret_cast<StatPartial*>(base + W.partials);
  float* scale = reinterpret_cast<float*>(base + W.scale);
  void* pool = base + W.pool;
  if ((s = launch_ns_stats(dprep, n, L.prep_tiles, partials, st)) != MO_OK) return s;
  if ((s = launch_ns_scale(dprep, n, partials, scale, nullptr, st)) != MO_OK) return s;
  if ((s = launch_ns_prep(dprep, n, L.prep_tiles, scale, pool, L.elem, st)) != MO_OK) return s;
  if ((s = ns_run_iterations(L, base + W.tab, W.tabs, pool, scale, coeffs, steps, nullptr, 0.f,
                             nullptr, nullptr, st)) != MO_OK)
    return s;
  return launch_ns_final(reinterpret_cast<const FinalItem*>(base + W.fin), n, rows, pool, L.elem,
                         st);
}

mo_status normuon_rownorm(void* O, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                          float* v, float beta2, float eps, void* stream) {
  clear_error();
  if (!O || !v) return fail(MO_EINVAL, "NULL pointer");
  if (!valid_dtype(dtype)) return fail(MO_EDTYPE, "bad dtype");
  if (rows < 0 || cols < 1 || ld < cols || rows > (int64_t(1) << 31) || cols > (1 << 30))
    return fail(MO_ESHAPE, "bad shape");
  if (!std::isfinite(beta2) || !std::isfinite(eps)) return fail(MO_EINVAL, "bad hyper-parameter");
  RowSeg one;
  std::memset(&one, 0, sizeof(one));
  one.o = O; one.nv = v; one.ld_o = ld; one.rows = static_cast<int32_t>(rows);
  one.cols = static_cast<int32_t>(cols); one.o_dt = dtype; one.w_dt = dtype; one.scale = 1.f;
  return launch_rows(kRowNormInPlace, nullptr, 0, one, rows, 0.f, nullptr, beta2, eps,
                     as_stream(stream));
}

mo_status muon_update(void* W, int32_t w_dtype, const void* U, int32_t u_dtype, int64_t rows,
                      int64_t cols, int64_t ld_w, int64_t ld_u, float lr, float wd, float scale,
                      void* stream) {
  clear_error();
  if (!W || !U) return fail(MO_EINVAL, "NULL pointer");
  if (!valid_dtype(w_dtype) || !valid_dtype(u_dtype)) return fail(MO_EDTYPE, "bad dtype");
  if (rows < 0 || cols < 1 || ld_w < cols || ld_u < cols || rows > (int64_t(1) << 31) ||
      cols > (1 << 30))
    return fail(MO_ESHAPE, "bad shape");
  if (!std::isfinite(lr) || !std::isfinite(wd) || !std::isfinite(scale))
    return fail(MO_EINVAL, "bad hyper-parameter");
  RowSeg one;
  std::memset(&one, 0, sizeof(one));
  one.w = W; one.o = const_cast<void*>(U); one.ld_w = ld_w; one.ld_o = ld_u;
  one.rows = static_cast<int32_t>(rows); one.cols = static_cast<int32_t>(cols);
  one.w_dt = w_dtype; one.o_dt = u_dtype; one.scale = scale; one.wd = wd;
  return launch_rows(kRowUpdate, nullptr, 0, one, rows, lr, nullptr, 0.f, 0.f,
                     as_stream(stream));
}

size_t adamw_workspace_bytes(const mo_adamw_item* items, int32_t n) {
  if (n < 0 || (n > 0 && !items)) return 0;
  return adam_ws_layout(items, n).total;
}

mo_status adamw_clip_step(const mo_adamw_item* items, int32_t n, float lr, float beta1,
                          float beta2, float eps, float max_norm, double* norm_out, void* ws,
                          size_t ws_bytes, void* stream) {
  clear_error();
  if (n < 0 || (n > 0 && !items)) return fail(MO_EINVAL, "bad item list");
  std::vector<AdamSeg> segs(static_cast<size_t>(n > 0 ? n : 1));
  int nseg = 0;
  int64_t nblocks = 0;
  mo_status s = adam_segments(items, n, lr, beta1, beta2, eps, max_norm, segs.data(), n, &nseg,
                              &nblocks);
  if (s != MO_OK) return s;
  const AdamWs W = adam_ws_layout(items, n);
  if ((s = check_ws(ws, ws_bytes, W.total)) != MO_OK) return s;
  hipStream_t st = as_stream(stream);
  char* base = static_cast<char*>(ws);
  double* partials = reinterpret_cast<double*>(base + W.partials);
  double* scal = reinterpret_cast<double*>(base + W.scal);
  const AdamSeg* dsegs = reinterpret_cast<const AdamSeg*>(base + W.tab);
  if ((s = upload(base + W.tab, segs.data(), nseg * sizeof(AdamSeg), st)) != MO_OK) return s;
  if ((s = launch_adam_sumsq(dsegs, nseg, nblocks, partials, st)) != MO_OK) return s;
  if ((s = launch_adam_norm(partials, nblocks, max_norm, scal, norm_out, st)) != MO_OK) return s;
  return launch_adam_apply(dsegs, nseg, nblocks, scal, lr, nullptr, 0, st);
}

mo_status mo_diag_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  clear_error();
  if (bytes < 0 || bytes % 16 != 0 || (bytes > 0 && (!src || !dst)))
    return fail(MO_EINVAL, "copy of %lld bytes: need non-NULL pointers and a multiple of 16",
                static_cast<long long>(bytes));
  if (!aligned16(src) || !aligned16(dst)) return fail(MO_EALIGN, "copy pointers must be 16-byte aligned");
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (bytes > 0 && a < b + bytes && b < a + bytes) return fail(MO_EINVAL, "copy ranges overlap");
  return launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
