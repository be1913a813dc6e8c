// Plan (parameter groups, slice tables, workspace layout) and the grouped
// hybrid Muon + AdamW step.
//
// A plan holds parameter groups, each with its own hyper-parameters (the
// group table of the kimi-k3 "build_parameter_groups" page: every group has
// its params, algorithm and weight decay; here also its learning rate and, for
// Muon, momentum, coefficient table and NorMuon setting).  Muon slices whose
// groups agree on everything that shapes the launches (momentum, Nesterov,
// coefficient table, NS precision, NorMuon and its constants) form one batch:
// groups that differ only in learning rate or decay share every launch, and
// read their rate from a per-step table.
//
// One step enqueues, on the caller's stream and without host synchronisation:
//   k_set_lrs     the step's learning rate of every group into the workspace
//   per batch:    k_momentum (B, D and per-block D statistics), k_ns_scale,
//                 k_ns_prep (X0 into the padded pool where needed)
//   [fork]        k_adam_sumsq, k_adam_norm, k_adam_apply over every AdamW
//                 item of every group (one joint clip) on a side stream
//   per batch:    the Newton-Schulz launches (k_ns_gemm / k_ns_small) and,
//                 unless the last launch applies it, k_rows (NorMuon, shape
//                 scale, weight update)
//   [join]
#include <cmath>
#include <cstring>
#include <vector>

#include "host.hpp"

using namespace mo;

struct mo_plan {
  struct SliceRec {
    int32_t param;
    int64_t off, rows, cols;
  };
  struct Group {
    int32_t algorithm;      // MO_ALG_MUON / MO_ALG_ADAMW
    mo_hparams hp;
    float wd;               // decoupled decay of the group's own algorithm
    float xwd;              // Muon groups: AdamW decay of excluded pieces
  };
  struct Batch {
    int32_t group0 = 0;               // the first group: its launch-shaping fields
    int32_t ddt = MO_BF16;            // direction / pool dtype
    std::vector<SliceRec> active;     // slices of params with a gradient
    std::vector<int32_t> active_group;
    std::vector<float> coeffs;        // [steps][3]
    NsLayout ns;
    NsTables nst;
    size_t ws_stats = 0, ws_scale = 0, ws_fb = 0, ws_pool = 0;
    int64_t mom_blocks = 0, total_rows = 0;
    size_t tab_mom = 0, tab_ns = 0, tab_rows = 0, tab_pow = 0;
    PowLayout pow;                    // spectral-cap guard (hp.spectral_cap > 0)
    // Muon update fused into the last Newton-Schulz launch (no O in the
    // workspace, no separate row pass): possible for every active slice
    bool fuse_ok = false;
    bool last_fused = false;
  };
  std::vector<mo_param> params;     // plan order
  std::vector<int32_t> pgroup;      // per param: group index, -1 when skipped
  std::vector<Group> groups;
  std::vector<mo_route_out> routes;
  std::vector<SliceRec> slices;     // all Muon slices, in param order
  std::vector<int32_t> slice_batch, slice_k;   // batch; index among its active slices or -1
  std::vector<SliceRec> excluded;   // excluded pieces of Muon params with a gradient (AdamW)
  std::vector<int32_t> excluded_group;
  std::vector<uint8_t> adam_owner;  // per param: AdamW steps it (whole or excluded pieces)
  std::vector<int32_t> steps;       // AdamW step counters (per param)
  std::vector<Batch> batches;
  NsOpts nsopt;
  float max_norm = 0.f;

  // workspace layout (byte offsets)
  std::vector<size_t> d_off;        // per param: direction buffer (Muon with grad)
  size_t ws_adam_partials = 0, ws_adam_scal = 0, ws_lr = 0;
  size_t ws_total = 0;
  int64_t adam_blocks = 0;
  int n_adam = 0;

  // plan-owned device tables
  size_t tab_adam = 0, tab_tcount = 0, tab_bytes = 0;
  char* dtab = nullptr;
  int device = -1;
  std::vector<char> htab;
  void* uploaded_ws = nullptr;
  // AdamW runs on a side stream, forked from and joined back into the
  // caller's stream, so that it overlaps the Muon path (created on first use)
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // a batch's plain-iteration launches run on a second stream beside its
  // Gram-space sequence (created on first use)
  hipStream_t side2 = nullptr;
  hipEvent_t ev_ns_fork = nullptr, ev_ns_join = nullptr;
  bool dirty = true;
  int32_t tdelta = 0;
  bool keep_ns_output = false;

  int nslots() const { return 2 * static_cast<int>(groups.size()); }
  const mo_hparams& bhp(const Batch& B) const { return groups[B.group0].hp; }
};

namespace {

// Checks every hyper-parameter of one block (group `g` for messages).
mo_status check_hparams(const mo_hparams& hp, int g) {
  if (hp.ns_steps < 1 || hp.ns_steps > MO_NS_MAX_STEPS)
    return fail(MO_EINVAL, "group %d: ns_steps must be in [1, %d]", g, MO_NS_MAX_STEPS);
  if (hp.ns_precision != MO_NS_BF16 && hp.ns_precision != MO_NS_F32)
    return fail(MO_EINVAL, "group %d: bad ns_precision", g);
  const float checks[] = {hp.muon_lr, hp.muon_wd, hp.mu, hp.normuon_beta2, hp.normuon_eps,
                          hp.adamw_lr, hp.beta1, hp.beta2, hp.eps, hp.adamw_wd};
  for (float c : checks)
    if (!std::isfinite(c)) return fail(MO_EINVAL, "group %d: non-finite hyper-parameter", g);
  if (hp.beta1 < 0.f || hp.beta1 >= 1.f || hp.beta2 < 0.f || hp.beta2 >= 1.f)
    return fail(MO_EINVAL, "group %d: betas must be in [0, 1)", g);
  if (std::isnan(hp.max_norm)) return fail(MO_EINVAL, "group %d: max_norm is NaN", g);
  if (!std::isfinite(hp.spectral_cap) || hp.spectral_cap < 0.f)
    return fail(MO_EINVAL, "group %d: spectral_cap must be finite and >= 0", g);
  if (hp.spectral_iters < 0 || hp.spectral_iters > MO_NS_MAX_STEPS)
    return fail(MO_EINVAL, "group %d: spectral_iters must be in [0, %d]", g, MO_NS_MAX_STEPS);
  for (int k = 0; k < hp.ns_steps; ++k)
    for (int j = 0; j < 3; ++j)
      if (!std::isfinite(hp.ns_coeffs[k][j]))
        return fail(MO_EINVAL, "group %d: non-finite coefficient", g);
  return MO_OK;
}

// Whether two Muon blocks shape the launches alike (same batch).
bool same_launches(const mo_hparams& a, const mo_hparams& b) {
  if (a.mu != b.mu || a.nesterov != b.nesterov || a.ns_steps != b.ns_steps ||
      a.ns_precision != b.ns_precision || (a.normuon != 0) != (b.normuon != 0))
    return false;
  if (a.normuon && (a.normuon_beta2 != b.normuon_beta2 || a.normuon_eps != b.normuon_eps))
    return false;
  if (a.spectral_cap != b.spectral_cap ||
      (a.spectral_cap > 0.f && a.spectral_iters != b.spectral_iters))
    return false;
  for (int k = 0; k < a.ns_steps; ++k)
    for (int j = 0; j < 3; ++j)
      if (a.ns_coeffs[k][j] != b.ns_coeffs[k][j]) return false;
  return true;
}

int64_t numel_of(const mo_param_desc& d) {
  int64_t n = 1;
  for (int k = 0; k < d.ndim; ++k) n *= d.shape[k];
  return n;
}

mo_status build_plan(mo_plan* P) {
  const int32_t n = static_cast<int32_t>(P->params.size());
  P->steps.assign(n, 0);
  P->adam_owner.assign(n, 0);
  P->d_off.assign(n, 0);
  WsCursor ws;
  std::vector<Slice> sl;
  bool adam_seen = false;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t g = P->pgroup[i];
    if (g < 0) continue;
    const mo_param& p = P->params[i];
    const mo_plan::Group& G = P->groups[g];
    if (!p.param) return fail(MO_EINVAL, "param %d: NULL param pointer", i);
    if (!valid_dtype(p.dtype)) return fail(MO_EDTYPE, "param %d: bad dtype", i);
    const int64_t numel = numel_of(p.desc);
    const bool has_adam = G.algorithm == MO_ALG_ADAMW || p.desc.exclude_mask != 0;
    if (has_adam && p.grad) {
      if (adam_seen && G.hp.max_norm != P->max_norm)
        return fail(MO_EINVAL, "group %d: max_norm differs from another group's (the clip "
                    "norm is joint over every AdamW item)", g);
      P->max_norm = G.hp.max_norm;
      adam_seen = true;
    }
    if (G.algorithm == MO_ALG_MUON) {
      if (p.desc.ndim != 2) return fail(MO_ESHAPE, "param %d: Muon params are 2-D", i);
      const int64_t R = p.desc.shape[0], C = p.desc.shape[1];
      if (R > 65536 || C > 65536) return fail(MO_ESHAPE, "param %d: dims above 65536", i);
      if (!p.momentum) return fail(MO_EINVAL, "param %d: Muon needs a momentum buffer", i);
      if (G.hp.normuon && !p.normuon_v) return fail(MO_EINVAL, "param %d: NorMuon needs v", i);
      // the param's registered view defines the slices
      mo_status s = expand_view(R, C, p.desc.view_ndim, p.desc.view, p.desc.nsplit,
                                p.desc.split, sl);
      if (s != MO_OK) return s;
      const uint32_t mask = p.desc.exclude_mask;
      if (!exclude_ok(p.desc.nsplit, mask))
        return fail(MO_ESHAPE, "param %d: exclude mask needs split sizes, bits below the split "
                    "count and one piece left to Muon", i);
      if (mask && (!p.exp_avg || !p.exp_avg_sq))
        return fail(MO_EINVAL, "param %d: excluded pieces need exp_avg and exp_avg_sq", i);
      // the batch of this group
      int b = 0;
      while (b < static_cast<int>(P->batches.size()) &&
             !same_launches(P->bhp(P->batches[b]), G.hp))
        ++b;
      if (b == static_cast<int>(P->batches.size())) {
        P->batches.emplace_back();
        mo_plan::Batch& B = P->batches.back();
        B.group0 = g;
        B.ddt = G.hp.ns_precision == MO_NS_F32 ? MO_F32 : MO_BF16;
        B.coeffs.assign(&G.hp.ns_coeffs[0][0], &G.hp.ns_coeffs[0][0] + 3 * G.hp.ns_steps);
      }
      mo_plan::Batch& B = P->batches[b];
      int32_t nsl = 0;
      for (size_t j = 0; j < sl.size(); ++j) {
        const Slice& x = sl[j];
        if (piece_excluded(mask, p.desc.nsplit, j)) {
          if (!p.grad) continue;
          // AdamW over the piece's elements of W, G, m and v
          const int64_t e0 = x.off * x.cols, es = dtype_size(p.dtype);
          if (!aligned16(static_cast<const char*>(p.param) + e0 * es) ||
              !aligned16(static_cast<const char*>(p.grad) + e0 * es) ||
              !aligned16(p.exp_avg + e0) || !aligned16(p.exp_avg_sq + e0))
            return fail(MO_EALIGN, "param %d: excluded piece at row %lld is not 16-byte aligned",
                        i, static_cast<long long>(x.off));
          P->excluded.push_back({i, x.off, x.rows, x.cols});
          P->excluded_group.push_back(g);
          P->adam_blocks += ceil_div(x.rows * x.cols, kEltPerBlock);
          ++P->n_adam;
          P->adam_owner[i] = 1;
          continue;
        }
        ++nsl;
        P->slices.push_back({i, x.off, x.rows, x.cols});
        P->slice_batch.push_back(b);
        if (p.grad) {
          P->slice_k.push_back(static_cast<int32_t>(B.active.size()));
          B.active.push_back({i, x.off, x.rows, x.cols});
          B.active_group.push_back(g);
        } else {
          P->slice_k.push_back(-1);
        }
      }
      P->routes[i].nslices = nsl;
      if (p.grad) P->d_off[i] = ws.take(static_cast<size_t>(numel) * dtype_size(B.ddt));
    } else {
      if (!p.exp_avg || !p.exp_avg_sq) return fail(MO_EINVAL, "param %d: AdamW needs m and v", i);
      if (p.grad && numel > 0) {
        if (!aligned16(p.param) || !aligned16(p.grad) || !aligned16(p.exp_avg) ||
            !aligned16(p.exp_avg_sq))
          return fail(MO_EALIGN, "param %d: AdamW pointers must be 16-byte aligned", i);
        P->adam_blocks += ceil_div(numel, kEltPerBlock);
        ++P->n_adam;
        P->adam_owner[i] = 1;
      }
    }
  }
  for (mo_plan::Batch& B : P->batches) {
    // The fused update needs the bf16 pool, no NorMuon (whose row statistics
    // span whole rows) and 16-byte weight chunks: cols % 8 == 0, aligned rows.
    B.fuse_ok = B.ddt == MO_BF16 && !P->bhp(B).normuon;
    for (const auto& a : B.active) {
      const mo_param& p = P->params[a.param];
      const int64_t es = static_cast<int64_t>(dtype_size(p.dtype));
      const char* w = static_cast<const char*>(p.param) + a.off * a.cols * es;
      if (a.cols % 8 != 0 || (a.cols * es) % 16 != 0 || !aligned16(w)) B.fuse_ok = false;
    }
    // momentum blocks per active slice (one statistics partial per block)
    for (const auto& a : B.active) {
      B.mom_blocks += ceil_div(a.rows * a.cols, kEltPerBlock);
      B.total_rows += a.rows;
    }
    B.ws_stats = ws.take(sizeof(StatPartial) * B.mom_blocks);
    B.ws_scale = ws.take(sizeof(float) * B.active.size());
    B.ws_fb = ws.take(sizeof(int32_t) * B.active.size());
    if (P->bhp(B).spectral_cap > 0.f && !B.active.empty()) {
      std::vector<int64_t> rr, cc;
      for (const auto& a : B.active) {
        rr.push_back(a.rows);
        cc.push_back(a.cols);
      }
      B.pow = pow_layout(rr.data(), cc.data(), static_cast<int>(rr.size()), ws);
    }
  }
  P->ws_adam_partials = ws.take(sizeof(double) * P->adam_blocks);
  P->ws_adam_scal = ws.take(2 * sizeof(double));
  P->ws_lr = ws.take(sizeof(float) * P->nslots());
  // The pools come last, one per batch.  D lives in the (256-byte aligned)
  // workspace in its batch's pool element type, rows of cols elements:
  // readable in place whenever the path is bf16.  A pool's base is known
  // before its size, so each D is addressed by its element offset from it.
  for (mo_plan::Batch& B : P->batches) {
    const size_t esz = dtype_size(B.ddt);
    const size_t pool_base = align_up(ws.off, 256);
    std::vector<int64_t> rr, cc, in_off;
    for (const auto& a : B.active) {
      rr.push_back(a.rows);
      cc.push_back(a.cols);
      in_off.push_back((static_cast<int64_t>(P->d_off[a.param]) +
                        a.off * a.cols * static_cast<int64_t>(esz) -
                        static_cast<int64_t>(pool_base)) / static_cast<int64_t>(esz));
    }
    const std::vector<uint8_t> direct(rr.size(), B.ddt == MO_BF16 ? 1 : 0);
    build_ns_layout(B.ns, rr.data(), cc.data(), static_cast<int>(rr.size()),
                    static_cast<int>(esz), B.coeffs.data(), P->bhp(B).ns_steps, P->nsopt,
                    direct.data(), false, B.ddt == MO_BF16 ? in_off.data() : nullptr);
    B.ws_pool = ws.take(static_cast<size_t>(B.ns.pool_elems) * B.ns.elem);
    if (B.ws_pool != pool_base) return fail(MO_EINVAL, "internal: pool base moved");
  }
  P->ws_total = align_up(ws.off, 256);

  WsCursor t;
  for (mo_plan::Batch& B : P->batches) {
    B.nst = ns_table_offsets(B.ns);
    B.tab_mom = t.take(sizeof(MomSeg) * B.active.size());
    B.tab_ns = t.take(B.nst.bytes);
    B.tab_rows = t.take(sizeof(RowSeg) * B.active.size());
    if (P->bhp(B).spectral_cap > 0.f) B.tab_pow = t.take(sizeof(PowSeg) * B.active.size());
  }
  P->tab_adam = t.take(sizeof(AdamSeg) * P->n_adam);
  // grouped steps since the upload (AdamW's bias correction), on the device:
  // uploaded as 0 with the tables, advanced by every step's k_set_lrs
  P->tab_tcount = t.take(sizeof(int32_t));
  P->tab_bytes = align_up(t.off, 256);
  return MO_OK;
}

// Fill the device tables (absolute pointers into `ws`) and upload them.
mo_status upload_tables(mo_plan* P, char* ws, hipStream_t st) {
  int dev = 0;
  MO_HIP_TRY(hipGetDevice(&dev));
  if (P->dtab && P->device != dev) {
    return fail(MO_EINVAL, "plan was first used on device %d, now on %d", P->device, dev);
  }
  if (!P->dtab && P->tab_bytes) {
    MO_HIP_TRY(hipMalloc(reinterpret_cast<void**>(&P->dtab), P->tab_bytes));
    P->device = dev;
  }
  P->htab.assign(P->tab_bytes, 0);
  char* h = P->htab.data();
  for (mo_plan::Batch& B : P->batches) {
    const mo_hparams& hp = P->bhp(B);
    const size_t esz = dtype_size(B.ddt);
    char* pool = ws + B.ws_pool;
    // momentum segments = active slices; NS prep items read D from the workspace
    MomSeg* mom = reinterpret_cast<MomSeg*>(h + B.tab_mom);
    RowSeg* rows = reinterpret_cast<RowSeg*>(h + B.tab_rows);
    int64_t blk = 0, row = 0;
    for (size_t k = 0; k < B.active.size(); ++k) {
      const auto& a = B.active[k];
      const mo_param& p = P->params[a.param];
      const mo_plan::Group& G = P->groups[B.active_group[k]];
      const int64_t e0 = a.off * a.cols, numel = a.rows * a.cols;
      MomSeg& m = mom[k];
      m.g = static_cast<const char*>(p.grad) + e0 * dtype_size(p.dtype);
      m.b = p.momentum + e0;
      m.d = ws + P->d_off[a.param] + e0 * esz;
      m.numel = numel;
      m.start = blk;
      m.gdt = p.dtype;
      m.ddt = B.ddt;
      m.vec = aligned16(m.g) && aligned16(m.b) && aligned16(m.d);
      m.pad = 0;
      PrepItem& pi = B.ns.prep[k];
      pi.in = m.d;
      pi.ld_in = a.cols;
      pi.in_dt = B.ddt;
      pi.vec = aligned16(pi.in) && (pi.ld_in * static_cast<int64_t>(esz)) % 16 == 0;
      pi.stat_begin = blk;
      blk += ceil_div(numel, kEltPerBlock);
      pi.stat_end = blk;
      RowSeg& r = rows[k];
      std::memset(&r, 0, sizeof(r));
      r.w = static_cast<char*>(p.param) + e0 * dtype_size(p.dtype);
      r.o = pool + B.ns.final_off(static_cast<int>(k), hp.ns_steps) * esz;
      r.nv = hp.normuon ? p.normuon_v + a.off : nullptr;
      r.ld_w = a.cols;
      r.ld_o = B.ns.final_ld(static_cast<int>(k));
      r.start = row;
      r.rows = static_cast<int32_t>(a.rows);
      r.cols = static_cast<int32_t>(a.cols);
      r.w_dt = p.dtype;
      r.o_dt = B.ddt;
      r.scale = static_cast<float>(std::sqrt(std::max(1.0, static_cast<double>(a.rows) / a.cols)));
      r.wd = G.wd;
      r.lr_slot = B.active_group[k];
      row += a.rows;
    }
    // fallback prep items: the same input as the slice's prep item
    for (PrepItem& fb : B.ns.prep_fb) {
      const PrepItem& pi = B.ns.prep[fb.slice];
      fb.in = pi.in;
      fb.ld_in = pi.ld_in;
      fb.in_dt = pi.in_dt;
      fb.vec = pi.vec;
    }
    std::vector<char> nsbuf;
    ns_pack_tables(B.ns, B.nst, nsbuf);
    if (!nsbuf.empty()) std::memcpy(h + B.tab_ns, nsbuf.data(), nsbuf.size());
    if (hp.spectral_cap > 0.f && !B.active.empty()) {
      // the guard's matrices: each active slice's rows of the fp32 buffer
      PowSeg* ps = reinterpret_cast<PowSeg*>(h + B.tab_pow);
      std::vector<int64_t> rr, cc;
      for (const auto& a : B.active) {
        rr.push_back(a.rows);
        cc.push_back(a.cols);
      }
      pow_fill(ps, rr.data(), cc.data(), static_cast<int>(rr.size()));
      for (size_t k = 0; k < B.active.size(); ++k) {
        const auto& a = B.active[k];
        ps[k].b = P->params[a.param].momentum + a.off * a.cols;
        ps[k].ld = a.cols;
      }
    }
  }
  AdamSeg* ad = reinterpret_cast<AdamSeg*>(h + P->tab_adam);
  const int ng = static_cast<int>(P->groups.size());
  int64_t ablk = 0;
  int j = 0;
  auto add_seg = [&](size_t i, int64_t e0, int64_t numel, int32_t g, bool piece) {
    const mo_param& p = P->params[i];
    const mo_plan::Group& G = P->groups[g];
    const int64_t es = static_cast<int64_t>(dtype_size(p.dtype));
    AdamSeg& s = ad[j++];
    s.p = static_cast<char*>(p.param) + e0 * es;
    s.g = static_cast<const char*>(p.grad) + e0 * es;
    s.m = p.exp_avg + e0;
    s.v = p.exp_avg_sq + e0;
    s.numel = numel;
    s.start = ablk; s.dt = p.dtype; s.t0 = P->steps[i] + 1;
    s.wd = piece ? G.xwd : G.wd;
    s.beta1 = G.hp.beta1; s.beta2 = G.hp.beta2; s.eps = G.hp.eps;
    s.lr_slot = piece ? ng + g : g;
    s.pad = 0;
    ablk += ceil_div(numel, kEltPerBlock);
  };
  size_t ex = 0;
  for (size_t i = 0; i < P->params.size(); ++i) {
    const mo_param& p = P->params[i];
    const int32_t g = P->pgroup[i];
    if (g < 0) continue;
    if (P->groups[g].algorithm == MO_ALG_MUON) {
      for (; ex < P->excluded.size() && P->excluded[ex].param == static_cast<int32_t>(i); ++ex) {
        const auto& x = P->excluded[ex];
        add_seg(i, x.off * x.cols, x.rows * x.cols, P->excluded_group[ex], true);
      }
      continue;
    }
    if (!p.grad) continue;
    const int64_t numel = numel_of(p.desc);
    if (numel == 0) continue;
    add_seg(i, 0, numel, g, false);
  }
  if (j != P->n_adam) return fail(MO_EINVAL, "internal: AdamW segment count");
  if (P->tab_bytes) {
    mo_status s = stage_upload(P->dtab, h, P->tab_bytes, st);
    if (s != MO_OK) return s;
  }
  P->uploaded_ws = ws;
  P->dirty = false;
  P->tdelta = 0;
  return MO_OK;
}

mo_status finish_create(mo_plan* P, const mo_plan_options* opts, mo_plan** out) {
  mo_status s = resolve_ns_options(opts ? &opts->ns : nullptr, P->nsopt);
  if (s == MO_OK && opts && opts->keep_ns_output != 0 && opts->keep_ns_output != 1)
    s = fail(MO_EINVAL, "keep_ns_output must be 0 or 1");
  if (s == MO_OK) {
    P->keep_ns_output = opts && opts->keep_ns_output;
    s = build_plan(P);
  }
  if (s != MO_OK) {
    delete P;
    return s;
  }
  *out = P;
  return MO_OK;
}

}  // namespace

extern "C" {

void mo_plan_options_default(mo_plan_options* o) {
  if (!o) return;
  mo_ns_options_default(&o->ns);
  o->keep_ns_output = 0;
  o->reserved = 0;
}

mo_status mo_plan_create(const mo_param* params, int32_t n, const mo_hparams* hp,
                         const mo_plan_options* opts, mo_plan** out) {
  clear_error();
  if (!out || !hp || n < 0 || (n > 0 && !params)) return fail(MO_EINVAL, "bad arguments");
  *out = nullptr;
  mo_status s = check_hparams(*hp, 0);
  if (s != MO_OK) return s;
  mo_plan* P = new (std::nothrow) mo_plan();
  if (!P) return fail(MO_EINVAL, "out of host memory");
  P->params.assign(params, params + n);
  // routing (kimi-k3 predicate, OMN reading for the embedding): one group
  // per routing key, every group on `hp`, decay where the key decays
  std::vector<mo_param_desc> descs(n);
  for (int32_t i = 0; i < n; ++i) descs[i] = params[i].desc;
  P->routes.assign(n, mo_route_out{});
  int32_t ng = 0;
  s = route(descs.data(), n, P->routes.data(), &ng);
  if (s == MO_OK && ng > MO_MAX_GROUPS)
    s = fail(MO_EINVAL, "%d routing groups (at most %d)", ng, MO_MAX_GROUPS);
  if (s != MO_OK) {
    delete P;
    return s;
  }
  P->groups.resize(ng);
  P->pgroup.assign(n, -1);
  for (int32_t i = 0; i < n; ++i) {
    const mo_route_out& r = P->routes[i];
    if (r.algorithm == MO_ALG_SKIP) continue;
    mo_plan::Group& G = P->groups[r.group];
    G.algorithm = r.algorithm;
    G.hp = *hp;
    G.wd = r.decay ? (r.algorithm == MO_ALG_MUON ? hp->muon_wd : hp->adamw_wd) : 0.f;
    G.xwd = r.decay ? hp->adamw_wd : 0.f;
    P->pgroup[i] = r.group;
    P->routes[i].nslices = 0;
  }
  return finish_create(P, opts, out);
}

mo_status mo_plan_create_groups(const mo_group* groups, int32_t ngroups,
                                const mo_plan_options* opts, mo_plan** out) {
  clear_error();
  if (!out || ngroups < 0 || (ngroups > 0 && !groups)) return fail(MO_EINVAL, "bad arguments");
  *out = nullptr;
  if (ngroups > MO_MAX_GROUPS)
    return fail(MO_EINVAL, "%d groups (at most %d)", ngroups, MO_MAX_GROUPS);
  int64_t total = 0;
  for (int32_t g = 0; g < ngroups; ++g) {
    const mo_group& G = groups[g];
    if (G.algorithm != MO_ALG_MUON && G.algorithm != MO_ALG_ADAMW)
      return fail(MO_EINVAL, "group %d: algorithm must be Muon or AdamW", g);
    if (G.nparams < 0 || (G.nparams > 0 && !G.params))
      return fail(MO_EINVAL, "group %d: bad parameter list", g);
    mo_status s = check_hparams(G.hp, g);
    if (s != MO_OK) return s;
    total += G.nparams;
  }
  if (total > (int64_t(1) << 30)) return fail(MO_EINVAL, "too many parameters");
  mo_plan* P = new (std::nothrow) mo_plan();
  if (!P) return fail(MO_EINVAL, "out of host memory");
  P->groups.resize(ngroups);
  std::vector<int64_t> seen;
  int32_t trainable = 0;
  for (int32_t g = 0; g < ngroups; ++g) {
    const mo_group& G = groups[g];
    mo_plan::Group& R = P->groups[g];
    R.algorithm = G.algorithm;
    R.hp = G.hp;
    R.wd = G.algorithm == MO_ALG_MUON ? G.hp.muon_wd : G.hp.adamw_wd;
    R.xwd = G.hp.adamw_wd;
    for (int32_t j = 0; j < G.nparams; ++j) {
      const mo_param& p = G.params[j];
      const int32_t i = static_cast<int32_t>(P->params.size());
      if (p.desc.ndim < 0 || p.desc.ndim > MO_MAX_NDIM) {
        delete P;
        return fail(MO_ESHAPE, "param %d: ndim %d", i, p.desc.ndim);
      }
      for (int64_t id : seen)
        if (id == p.desc.ident) {
          delete P;
          return fail(MO_ECONFLICT, "param %d: identity %lld appears twice in the table", i,
                      static_cast<long long>(p.desc.ident));
        }
      seen.push_back(p.desc.ident);
      P->params.push_back(p);
      mo_route_out r{};
      r.group = -1;
      r.algorithm = MO_ALG_SKIP;
      if (p.desc.requires_grad) {
        r.algorithm = G.algorithm;
        r.decay = R.wd != 0.f;
        r.group = g;
        ++trainable;
      }
      P->routes.push_back(r);
      P->pgroup.push_back(r.group);
    }
  }
  if (trainable == 0) {
    delete P;
    return fail(MO_EEMPTY, "no trainable parameter in the group table");
  }
  return finish_create(P, opts, out);
}

void mo_plan_destroy(mo_plan* plan) {
  if (!plan) return;
  if (plan->dtab) (void)hipFree(plan->dtab);
  if (plan->ev_fork) (void)hipEventDestroy(plan->ev_fork);
  if (plan->ev_join) (void)hipEventDestroy(plan->ev_join);
  if (plan->side) (void)hipStreamDestroy(plan->side);
  if (plan->ev_ns_fork) (void)hipEventDestroy(plan->ev_ns_fork);
  if (plan->ev_ns_join) (void)hipEventDestroy(plan->ev_ns_join);
  if (plan->side2) (void)hipStreamDestroy(plan->side2);
  delete plan;
}

size_t mo_plan_workspace_bytes(const mo_plan* plan) { return plan ? plan->ws_total : 0; }

int32_t mo_plan_num_params(const mo_plan* plan) {
  return plan ? static_cast<int32_t>(plan->params.size()) : 0;
}

int32_t mo_plan_num_groups(const mo_plan* plan) {
  return plan ? static_cast<int32_t>(plan->groups.size()) : 0;
}

mo_status mo_plan_route(const mo_plan* plan, mo_route_out* out, int32_t n) {
  clear_error();
  if (!plan || !out || n < static_cast<int32_t>(plan->routes.size()))
    return fail(MO_EINVAL, "bad arguments");
  std::memcpy(out, plan->routes.data(), plan->routes.size() * sizeof(mo_route_out));
  return MO_OK;
}

int32_t mo_plan_num_slices(const mo_plan* plan) {
  return plan ? static_cast<int32_t>(plan->slices.size()) : 0;
}

mo_status mo_plan_slices(const mo_plan* plan, int64_t* out4, int32_t max_slices) {
  clear_error();
  if (!plan || !out4 || max_slices < static_cast<int32_t>(plan->slices.size()))
    return fail(MO_EINVAL, "bad arguments");
  for (size_t k = 0; k < plan->slices.size(); ++k) {
    out4[4 * k] = plan->slices[k].param;
    out4[4 * k + 1] = plan->slices[k].off;
    out4[4 * k + 2] = plan->slices[k].rows;
    out4[4 * k + 3] = plan->slices[k].cols;
  }
  return MO_OK;
}

mo_status mo_plan_get_steps(const mo_plan* plan, int32_t* steps, int32_t n) {
  clear_error();
  if (!plan || !steps || n < static_cast<int32_t>(plan->steps.size()))
    return fail(MO_EINVAL, "bad arguments");
  std::memcpy(steps, plan->steps.data(), plan->steps.size() * sizeof(int32_t));
  return MO_OK;
}

mo_status mo_plan_set_steps(mo_plan* plan, const int32_t* steps, int32_t n) {
  clear_error();
  if (!plan || !steps || n < static_cast<int32_t>(plan->steps.size()))
    return fail(MO_EINVAL, "bad arguments");
  for (size_t i = 0; i < plan->steps.size(); ++i)
    if (steps[i] < 0) return fail(MO_EINVAL, "negative step counter");
  std::memcpy(plan->steps.data(), steps, plan->steps.size() * sizeof(int32_t));
  plan->dirty = true;
  return MO_OK;
}

mo_status mo_plan_keep_ns_output(mo_plan* plan, int32_t keep) {
  clear_error();
  if (!plan) return fail(MO_EINVAL, "NULL plan");
  plan->keep_ns_output = keep != 0;
  return MO_OK;
}

int32_t mo_plan_fuses_update(const mo_plan* plan) {
  if (!plan || plan->keep_ns_output) return 0;
  bool any = false;
  for (const auto& B : plan->batches) {
    if (B.active.empty()) continue;
    if (!B.fuse_ok) return 0;
    any = true;
  }
  return any ? 1 : 0;
}

int32_t mo_plan_gram_space(const mo_plan* plan) {
  if (!plan) return 0;
  for (const auto& B : plan->batches)
    for (uint8_t g : B.ns.gspace)
      if (g) return 1;
  return 0;
}

mo_status mo_plan_slice_algorithms(const mo_plan* P, int32_t* out, int32_t n) {
  clear_error();
  if (!P || !out || n < static_cast<int32_t>(P->slices.size()))
    return fail(MO_EINVAL, "bad arguments");
  for (size_t i = 0; i < P->slices.size(); ++i) {
    const int k = P->slice_k[i];
    if (k < 0) {
      out[i] = -1;
      continue;
    }
    const NsLayout& L = P->batches[P->slice_batch[i]].ns;
    out[i] = (L.gspace[k] ? 1 : 0) | (L.kind[k] << 1);
  }
  return MO_OK;
}

mo_status mo_plan_ns_output(const mo_plan* P, int32_t slice, const void* ws, void** o,
                            int64_t* ld, int32_t* dtype) {
  clear_error();
  if (!P || !ws || !o || !ld || !dtype) return fail(MO_EINVAL, "bad arguments");
  if (slice < 0 || slice >= static_cast<int32_t>(P->slices.size()))
    return fail(MO_EINVAL, "slice %d out of range", slice);
  if (P->uploaded_ws != ws || P->tdelta == 0)
    return fail(MO_EINVAL, "no grouped step has run on this workspace");
  const int k = P->slice_k[slice];
  if (k < 0) return fail(MO_EINVAL, "slice %d: param has no gradient", slice);
  const mo_plan::Batch& B = P->batches[P->slice_batch[slice]];
  if (B.last_fused)
    return fail(MO_EINVAL,
                "the last grouped step applied the update inside the Newton-Schulz launch and "
                "kept no output: call mo_plan_keep_ns_output(plan, 1) before stepping");
  const size_t esz = dtype_size(B.ddt);
  *o = const_cast<char*>(static_cast<const char*>(ws)) + B.ws_pool +
       B.ns.final_off(k, P->bhp(B).ns_steps) * esz;
  *ld = B.ns.final_ld(k);
  *dtype = B.ddt;
  return MO_OK;
}

mo_status mo_grouped_step(mo_plan* P, const mo_step_args* args, void* ws, size_t ws_bytes,
                          void* stream) {
  clear_error();
  if (!P) return fail(MO_EINVAL, "NULL plan");
  if (P->ws_total) {
    if (!ws) return fail(MO_EWORKSPACE, "workspace of %zu bytes required", P->ws_total);
    if (reinterpret_cast<uintptr_t>(ws) & 255u)
      return fail(MO_EALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < P->ws_total)
      return fail(MO_EWORKSPACE, "workspace has %zu bytes, %zu required", ws_bytes, P->ws_total);
  }
  // this step's learning rates: slot g is group g's own rate (Muon or AdamW),
  // slot ngroups + g the AdamW rate of a Muon group's excluded pieces
  const int ng = static_cast<int>(P->groups.size());
  if (args && args->n_group_lr > 0 && !args->group_lr)
    return fail(MO_EINVAL, "group_lr is NULL with n_group_lr = %d", args->n_group_lr);
  std::vector<float> lr(P->nslots(), 0.f);
  for (int g = 0; g < ng; ++g) {
    const mo_plan::Group& G = P->groups[g];
    const float muon = args && args->muon_lr >= 0.f ? args->muon_lr : G.hp.muon_lr;
    const float adamw = args && args->adamw_lr >= 0.f ? args->adamw_lr : G.hp.adamw_lr;
    lr[g] = G.algorithm == MO_ALG_MUON ? muon : adamw;
    if (args && g < args->n_group_lr && args->group_lr[g] >= 0.f) lr[g] = args->group_lr[g];
    lr[ng + g] = adamw;
  }
  for (float v : lr)
    if (!std::isfinite(v)) return fail(MO_EINVAL, "non-finite learning rate");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  mo_status s;
  if (P->dirty || P->uploaded_ws != ws) {
    if ((s = upload_tables(P, base, st)) != MO_OK) return s;
  }
  float* lrs = reinterpret_cast<float*>(base + P->ws_lr);
  int32_t* tcount = reinterpret_cast<int32_t*>(P->dtab + P->tab_tcount);
  if ((s = launch_set_lrs(lrs, lr.data(), P->nslots(), st, tcount)) != MO_OK) return s;
  // Muon: momentum and the Newton-Schulz input (HBM-bound) first
  int nsl_total = 0;
  for (mo_plan::Batch& B : P->batches) {
    const int nsl = static_cast<int>(B.active.size());
    if (nsl == 0) continue;
    nsl_total += nsl;
    const mo_hparams& hp = P->bhp(B);
    const char* dns = P->dtab + B.tab_ns;
    void* pool = base + B.ws_pool;
    StatPartial* stats = reinterpret_cast<StatPartial*>(base + B.ws_stats);
    float* scale = reinterpret_cast<float*>(base + B.ws_scale);
    const PrepItem* dprep = reinterpret_cast<const PrepItem*>(dns + B.nst.prep);
    const MomSeg* dmom = reinterpret_cast<const MomSeg*>(P->dtab + B.tab_mom);
    if (hp.spectral_cap > 0.f) {
      // spectral-cap guard: accumulate B, estimate each slice's top singular
      // value, then rescale B where it exceeds the cap and form D from it
      PowWork wk = pow_work(B.pow, base);
      if ((s = launch_momentum(dmom, nsl, B.mom_blocks, hp.mu, hp.nesterov, nullptr, st, 1)) !=
          MO_OK)
        return s;
      if ((s = launch_power_iteration(reinterpret_cast<const PowSeg*>(P->dtab + B.tab_pow), nsl,
                                      B.pow.grid, hp.spectral_iters, wk, hp.spectral_cap, st)) !=
          MO_OK)
        return s;
      if ((s = launch_momentum(dmom, nsl, B.mom_blocks, hp.mu, hp.nesterov, stats, st, 2,
                               wk.kappa)) != MO_OK)
        return s;
    } else if ((s = launch_momentum(dmom, nsl, B.mom_blocks, hp.mu, hp.nesterov, stats, st)) !=
               MO_OK) {
      return s;
    }
    int32_t* fb = reinterpret_cast<int32_t*>(base + B.ws_fb);
    if ((s = launch_ns_scale(dprep, nsl, stats, scale, fb, st)) != MO_OK) return s;
    if ((s = launch_ns_prep(dprep, nsl, B.ns.prep_tiles, scale, pool, B.ns.elem, st)) != MO_OK)
      return s;
    if ((s = launch_ns_prep_fallback(reinterpret_cast<const PrepItem*>(dns + B.nst.prep_fb),
                                     static_cast<int>(B.ns.prep_fb.size()), scale, fb, pool,
                                     st)) != MO_OK)
      return s;
  }
  // AdamW (clip norm and update) is independent of the Muon path: with both
  // present it goes to a side stream forked here, so that it overlaps the
  // MFMA-bound Newton-Schulz iterations rather than the HBM-bound kernels.
  // While kernel timing is enabled everything stays on `st`, in order, so that
  // each bracketed duration belongs to one kernel running alone.
  hipStream_t ast = st;
  const bool fork = nsl_total > 0 && P->n_adam > 0 && !timing_enabled();
  if (fork) {
    if (!P->side) {
      MO_HIP_TRY(hipStreamCreateWithFlags(&P->side, hipStreamNonBlocking));
      MO_HIP_TRY(hipEventCreateWithFlags(&P->ev_fork, hipEventDisableTiming));
      MO_HIP_TRY(hipEventCreateWithFlags(&P->ev_join, hipEventDisableTiming));
    }
    MO_HIP_TRY(hipEventRecord(P->ev_fork, st));
    MO_HIP_TRY(hipStreamWaitEvent(P->side, P->ev_fork, 0));
    ast = P->side;
  }
  // Everything after the fork runs in one function so that the side stream
  // is joined back into `st` on every path, errors included: the caller may
  // reuse the workspace and the tensors once `st` has drained.
  auto forked_work = [&]() -> mo_status {
    mo_status r;
    double* scal = reinterpret_cast<double*>(base + P->ws_adam_scal);
    if (P->n_adam > 0) {
      const AdamSeg* dad = reinterpret_cast<const AdamSeg*>(P->dtab + P->tab_adam);
      double* partials = reinterpret_cast<double*>(base + P->ws_adam_partials);
      if ((r = launch_adam_sumsq(dad, P->n_adam, P->adam_blocks, partials, ast)) != MO_OK)
        return r;
      if ((r = launch_adam_norm(partials, P->adam_blocks, P->max_norm, scal,
                                args ? args->norm_out : nullptr, ast)) != MO_OK)
        return r;
      if ((r = launch_adam_apply(dad, P->n_adam, P->adam_blocks, scal, 0.f, lrs, P->tdelta,
                                 ast, tcount)) != MO_OK)
        return r;
    } else if (args && args->norm_out) {
      // no AdamW gradient: report T = 0 (a kernel write, not a memset node)
      if ((r = launch_adam_norm(nullptr, 0, P->max_norm, scal, args->norm_out, st)) != MO_OK)
        return r;
    }
    for (mo_plan::Batch& B : P->batches) {
      const int nsl = static_cast<int>(B.active.size());
      if (nsl == 0) continue;
      const mo_hparams& hp = P->bhp(B);
      const char* dns = P->dtab + B.tab_ns;
      // the row table is the weight target of the fused update and the input
      // of the separate row pass
      const RowSeg* drows = reinterpret_cast<const RowSeg*>(P->dtab + B.tab_rows);
      const bool fuse = B.fuse_ok && !P->keep_ns_output;
      // The slice-resident launches, the Gram-space sequence and the plain
      // iteration share no data: they are split over `st` and the second
      // stream, forked here and joined back on every path, so that one
      // chain's launches fill the CUs another leaves idle (the last, partly
      // empty round of workgroups of a launch; the memory-bound slice-resident
      // kernel beside latency-bound GEMM launches).  (In order on `st` while
      // timing.)
      const bool two = !timing_enabled() && ns_has_two_chains(B.ns);
      if (two) {
        if (!P->side2) {
          MO_HIP_TRY(hipStreamCreateWithFlags(&P->side2, hipStreamNonBlocking));
          MO_HIP_TRY(hipEventCreateWithFlags(&P->ev_ns_fork, hipEventDisableTiming));
          MO_HIP_TRY(hipEventCreateWithFlags(&P->ev_ns_join, hipEventDisableTiming));
        }
        MO_HIP_TRY(hipEventRecord(P->ev_ns_fork, st));
        MO_HIP_TRY(hipStreamWaitEvent(P->side2, P->ev_ns_fork, 0));
      }
      r = ns_run_iterations(B.ns, dns, B.nst, base + B.ws_pool,
                            reinterpret_cast<const float*>(base + B.ws_scale), B.coeffs.data(),
                            hp.ns_steps, fuse ? drows : nullptr, 0.f, lrs,
                            reinterpret_cast<const int32_t*>(base + B.ws_fb), st,
                            two ? P->side2 : nullptr);
      if (two) {
        const hipError_t e1 = hipEventRecord(P->ev_ns_join, P->side2);
        const hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(st, P->ev_ns_join, 0) : e1;
        if (r == MO_OK && e2 != hipSuccess)
          return fail(MO_EHIP, "joining the second Newton-Schulz stream failed: %s",
                      hipGetErrorString(e2));
      }
      if (r != MO_OK) return r;
      if (!fuse) {
        RowSeg none;
        std::memset(&none, 0, sizeof(none));
        if ((r = launch_rows(hp.normuon ? kRowNormUpdate : kRowUpdate, drows, nsl, none,
                             B.total_rows, 0.f, lrs, hp.normuon_beta2, hp.normuon_eps,
                             st)) != MO_OK)
          return r;
      }
      B.last_fused = fuse;
    }
    return MO_OK;
  };
  s = forked_work();
  if (fork) {
    // join even after an error (the first failure's message is kept)
    const hipError_t e1 = hipEventRecord(P->ev_join, ast);
    const hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(st, P->ev_join, 0) : e1;
    if (s == MO_OK && e2 != hipSuccess)
      return fail(MO_EHIP, "joining the AdamW stream failed: %s", hipGetErrorString(e2));
  }
  if (s != MO_OK) return s;
  for (size_t i = 0; i < P->params.size(); ++i)
    if (P->adam_owner[i]) ++P->steps[i];
  ++P->tdelta;
  return MO_OK;
}

}  // extern "C"
