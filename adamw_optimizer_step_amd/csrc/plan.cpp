// Plan (routing + slice table + workspace layout) and the grouped hybrid
// Muon + AdamW step.
//
// One step enqueues, on the caller's stream and without host synchronisation:
//   k_momentum   over every Muon slice (B, D and per-block D statistics)
//   k_ns_scale   per slice (max-abs / Frobenius scale from those statistics)
//   k_ns_prep    X0 in both orientations into the padded pool
//   k_ns_gemm    2 (cubic) or 3 launches per Newton-Schulz iteration
//   k_rows       NorMuon (optional) + shape scale + weight update per row
//   k_adam_*     sum of squares, clip factor, AdamW update
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
  std::vector<mo_param> params;
  mo_hparams hp;
  std::vector<mo_route_out> routes;
  std::vector<SliceRec> slices;     // all Muon slices, in param order
  std::vector<SliceRec> active;     // slices of Muon params with a gradient
  std::vector<SliceRec> excluded;   // excluded pieces of Muon params with a gradient (AdamW)
  std::vector<uint8_t> adam_owner;  // per param: AdamW steps it (whole or excluded pieces)
  std::vector<int32_t> steps;       // AdamW step counters (per param)
  int32_t ddt = MO_BF16;            // direction / pool dtype
  NsOpts nsopt;

  NsLayout ns;
  // workspace layout (byte offsets)
  std::vector<size_t> d_off;        // per param: direction buffer (Muon with grad)
  size_t ws_stats = 0, ws_scale = 0, ws_fb = 0, ws_adam_partials = 0, ws_adam_scal = 0;
  size_t ws_pool = 0;
  size_t ws_total = 0;
  int64_t mom_blocks = 0, adam_blocks = 0, total_rows = 0;
  int n_adam = 0;

  // plan-owned device tables
  NsTables nst;
  size_t tab_mom = 0, tab_ns = 0, tab_rows = 0, tab_adam = 0, tab_bytes = 0;
  char* dtab = nullptr;
  int device = -1;
  std::vector<char> htab;
  void* uploaded_ws = nullptr;
  // AdamW runs on a side stream, forked from and joined back into the
  // caller's stream, so that it overlaps the Muon path (created on first use)
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool dirty = true;
  int32_t tdelta = 0;
  // Muon update fused into the last Newton-Schulz launch (no O in the
  // workspace, no separate row pass): possible for every active slice
  // (fuse_ok), unless the caller keeps O for mo_plan_ns_output
  bool fuse_ok = false;
  bool keep_ns_output = false;
  bool last_fused = false;
};

namespace {

mo_status build_plan(mo_plan* P) {
  const int32_t n = static_cast<int32_t>(P->params.size());
  std::vector<mo_param_desc> descs(n);
  for (int32_t i = 0; i < n; ++i) descs[i] = P->params[i].desc;
  P->routes.assign(n, mo_route_out{});
  int32_t ng = 0;
  mo_status s = route(descs.data(), n, P->routes.data(), &ng);
  if (s != MO_OK) return s;
  const mo_hparams& hp = P->hp;
  P->ddt = hp.ns_precision == MO_NS_F32 ? MO_F32 : MO_BF16;
  P->steps.assign(n, 0);
  P->adam_owner.assign(n, 0);

  WsCursor ws;
  std::vector<Slice> sl;
  P->d_off.assign(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    const mo_param& p = P->params[i];
    const mo_route_out& r = P->routes[i];
    if (r.algorithm == MO_ALG_SKIP) continue;
    if (!p.param) return fail(MO_EINVAL, "param %d: NULL param pointer", i);
    if (!valid_dtype(p.dtype)) return fail(MO_EDTYPE, "param %d: bad dtype", i);
    int64_t numel = 1;
    for (int k = 0; k < p.desc.ndim; ++k) numel *= p.desc.shape[k];
    if (r.algorithm == MO_ALG_MUON) {
      const int64_t R = p.desc.shape[0], C = p.desc.shape[1];
      if (R > 65536 || C > 65536) return fail(MO_ESHAPE, "param %d: dims above 65536", i);
      if (!p.momentum) return fail(MO_EINVAL, "param %d: Muon needs a momentum buffer", i);
      if (hp.normuon && !p.normuon_v) return fail(MO_EINVAL, "param %d: NorMuon needs v", i);
      // The routing key's view (the parameter's registered view) defines the slices.
      s = expand_view(R, C, p.desc.view_ndim, p.desc.view, p.desc.nsplit, p.desc.split, sl);
      if (s != MO_OK) return s;
      const uint32_t mask = p.desc.exclude_mask;
      if (mask && (!p.exp_avg || !p.exp_avg_sq))
        return fail(MO_EINVAL, "param %d: excluded pieces need exp_avg and exp_avg_sq", i);
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
          P->adam_blocks += ceil_div(x.rows * x.cols, kEltPerBlock);
          ++P->n_adam;
          P->adam_owner[i] = 1;
          continue;
        }
        P->slices.push_back({i, x.off, x.rows, x.cols});
        if (p.grad) P->active.push_back({i, x.off, x.rows, x.cols});
      }
      if (p.grad) P->d_off[i] = ws.take(static_cast<size_t>(numel) * dtype_size(P->ddt));
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
  // The fused update needs the bf16 pool, no NorMuon (whose row statistics
  // span whole rows) and 16-byte weight chunks: cols % 8 == 0 and aligned rows.
  P->fuse_ok = P->ddt == MO_BF16 && !hp.normuon;
  for (const auto& a : P->active) {
    const mo_param& p = P->params[a.param];
    const int64_t es = static_cast<int64_t>(dtype_size(p.dtype));
    const char* w = static_cast<const char*>(p.param) + a.off * a.cols * es;
    if (a.cols % 8 != 0 || (a.cols * es) % 16 != 0 || !aligned16(w)) P->fuse_ok = false;
  }
  // momentum blocks per active slice (one statistics partial per block)
  for (const auto& a : P->active) P->mom_blocks += ceil_div(a.rows * a.cols, kEltPerBlock);
  std::vector<int64_t> rr, cc;
  for (const auto& a : P->active) { rr.push_back(a.rows); cc.push_back(a.cols); P->total_rows += a.rows; }
  P->ws_stats = ws.take(sizeof(StatPartial) * P->mom_blocks);
  P->ws_scale = ws.take(sizeof(float) * P->active.size());
  P->ws_fb = ws.take(sizeof(int32_t) * P->active.size());
  P->ws_adam_partials = ws.take(sizeof(double) * P->adam_blocks);
  P->ws_adam_scal = ws.take(2 * sizeof(double));
  // D lives in the (256-byte aligned) workspace in the pool's element type,
  // rows of cols elements: readable in place whenever the path is bf16.  The
  // pool comes last; its base is known before its size, so each D can be
  // addressed by its element offset from the pool.
  const size_t esz_ns = dtype_size(P->ddt);
  const size_t pool_base = align_up(ws.off, 256);
  std::vector<int64_t> in_off;
  for (const auto& a : P->active)
    in_off.push_back((static_cast<int64_t>(P->d_off[a.param]) +
                      a.off * a.cols * static_cast<int64_t>(esz_ns) -
                      static_cast<int64_t>(pool_base)) / static_cast<int64_t>(esz_ns));
  const std::vector<uint8_t> direct(rr.size(), P->ddt == MO_BF16 ? 1 : 0);
  build_ns_layout(P->ns, rr.data(), cc.data(), static_cast<int>(rr.size()),
                  static_cast<int>(esz_ns), &hp.ns_coeffs[0][0], hp.ns_steps, P->nsopt,
                  direct.data(), false, P->ddt == MO_BF16 ? in_off.data() : nullptr);
  P->ws_pool = ws.take(static_cast<size_t>(P->ns.pool_elems) * P->ns.elem);
  if (P->ws_pool != pool_base) return fail(MO_EINVAL, "internal: pool base moved");
  P->ws_total = align_up(ws.off, 256);

  P->nst = ns_table_offsets(P->ns);
  WsCursor t;
  P->tab_mom = t.take(sizeof(MomSeg) * P->active.size());
  P->tab_ns = t.take(P->nst.bytes);
  P->tab_rows = t.take(sizeof(RowSeg) * P->active.size());
  P->tab_adam = t.take(sizeof(AdamSeg) * P->n_adam);
  P->tab_bytes = align_up(t.off, 256);
  return MO_OK;
}

// Fill the device tables (absolute pointers into `ws`) and upload them.
mo_status upload_tables(mo_plan* P, char* ws, hipStream_t st) {
  const mo_hparams& hp = P->hp;
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
  const size_t esz = dtype_size(P->ddt);
  char* pool = ws + P->ws_pool;
  // momentum segments = active slices; NS prep items read D from the workspace
  MomSeg* mom = reinterpret_cast<MomSeg*>(h + P->tab_mom);
  RowSeg* rows = reinterpret_cast<RowSeg*>(h + P->tab_rows);
  int64_t blk = 0, row = 0;
  for (size_t k = 0; k < P->active.size(); ++k) {
    const auto& a = P->active[k];
    const mo_param& p = P->params[a.param];
    const int64_t e0 = a.off * a.cols, numel = a.rows * a.cols;
    MomSeg& m = mom[k];
    m.g = static_cast<const char*>(p.grad) + e0 * dtype_size(p.dtype);
    m.b = p.momentum + e0;
    m.d = ws + P->d_off[a.param] + e0 * esz;
    m.numel = numel;
    m.start = blk;
    m.gdt = p.dtype;
    m.ddt = P->ddt;
    m.vec = aligned16(m.g) && aligned16(m.b) && aligned16(m.d);
    m.pad = 0;
    PrepItem& pi = P->ns.prep[k];
    pi.in = m.d;
    pi.ld_in = a.cols;
    pi.in_dt = P->ddt;
    pi.vec = aligned16(pi.in) && (pi.ld_in * static_cast<int64_t>(esz)) % 16 == 0;
    pi.stat_begin = blk;
    blk += ceil_div(numel, kEltPerBlock);
    pi.stat_end = blk;
    RowSeg& r = rows[k];
    std::memset(&r, 0, sizeof(r));
    r.w = static_cast<char*>(p.param) + e0 * dtype_size(p.dtype);
    r.o = pool + P->ns.final_off(static_cast<int>(k), hp.ns_steps) * esz;
    r.nv = hp.normuon ? p.normuon_v + a.off : nullptr;
    r.ld_w = a.cols;
    r.ld_o = P->ns.final_ld(static_cast<int>(k));
    r.start = row;
    r.rows = static_cast<int32_t>(a.rows);
    r.cols = static_cast<int32_t>(a.cols);
    r.w_dt = p.dtype;
    r.o_dt = P->ddt;
    r.scale = static_cast<float>(std::sqrt(std::max(1.0, static_cast<double>(a.rows) / a.cols)));
    r.wd = P->routes[a.param].decay ? hp.muon_wd : 0.f;
    row += a.rows;
  }
  // fallback prep items: the same input as the slice's prep item
  for (PrepItem& fb : P->ns.prep_fb) {
    const PrepItem& pi = P->ns.prep[fb.slice];
    fb.in = pi.in;
    fb.ld_in = pi.ld_in;
    fb.in_dt = pi.in_dt;
    fb.vec = pi.vec;
  }
  std::vector<char> nsbuf;
  ns_pack_tables(P->ns, P->nst, nsbuf);
  if (!nsbuf.empty()) std::memcpy(h + P->tab_ns, nsbuf.data(), nsbuf.size());
  AdamSeg* ad = reinterpret_cast<AdamSeg*>(h + P->tab_adam);
  int64_t ablk = 0;
  int j = 0;
  auto add_seg = [&](size_t i, int64_t e0, int64_t numel) {
    const mo_param& p = P->params[i];
    const int64_t es = static_cast<int64_t>(dtype_size(p.dtype));
    AdamSeg& s = ad[j++];
    s.p = static_cast<char*>(p.param) + e0 * es;
    s.g = static_cast<const char*>(p.grad) + e0 * es;
    s.m = p.exp_avg + e0;
    s.v = p.exp_avg_sq + e0;
    s.numel = numel;
    s.start = ablk; s.dt = p.dtype; s.t0 = P->steps[i] + 1;
    s.wd = P->routes[i].decay ? hp.adamw_wd : 0.f;
    s.pad = 0.f;
    ablk += ceil_div(numel, kEltPerBlock);
  };
  size_t ex = 0;
  for (size_t i = 0; i < P->params.size(); ++i) {
    const mo_param& p = P->params[i];
    if (P->routes[i].algorithm == MO_ALG_MUON) {
      for (; ex < P->excluded.size() && P->excluded[ex].param == static_cast<int32_t>(i); ++ex) {
        const auto& x = P->excluded[ex];
        add_seg(i, x.off * x.cols, x.rows * x.cols);
      }
      continue;
    }
    if (P->routes[i].algorithm != MO_ALG_ADAMW || !p.grad) continue;
    int64_t numel = 1;
    for (int k = 0; k < p.desc.ndim; ++k) numel *= p.desc.shape[k];
    if (numel == 0) continue;
    add_seg(i, 0, numel);
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
  if (hp->ns_steps < 1 || hp->ns_steps > MO_NS_MAX_STEPS)
    return fail(MO_EINVAL, "ns_steps must be in [1, %d]", MO_NS_MAX_STEPS);
  if (hp->ns_precision != MO_NS_BF16 && hp->ns_precision != MO_NS_F32)
    return fail(MO_EINVAL, "bad ns_precision");
  const float checks[] = {hp->muon_lr, hp->muon_wd, hp->mu, hp->normuon_beta2, hp->normuon_eps,
                          hp->adamw_lr, hp->beta1, hp->beta2, hp->eps, hp->adamw_wd};
  for (float c : checks)
    if (!std::isfinite(c)) return fail(MO_EINVAL, "non-finite hyper-parameter");
  if (hp->beta1 < 0.f || hp->beta1 >= 1.f || hp->beta2 < 0.f || hp->beta2 >= 1.f)
    return fail(MO_EINVAL, "betas must be in [0, 1)");
  if (std::isnan(hp->max_norm)) return fail(MO_EINVAL, "max_norm is NaN");
  for (int k = 0; k < hp->ns_steps; ++k)
    for (int j = 0; j < 3; ++j)
      if (!std::isfinite(hp->ns_coeffs[k][j])) return fail(MO_EINVAL, "non-finite coefficient");
  mo_plan* P = new (std::nothrow) mo_plan();
  if (!P) return fail(MO_EINVAL, "out of host memory");
  P->params.assign(params, params + n);
  P->hp = *hp;
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

void mo_plan_destroy(mo_plan* plan) {
  if (!plan) return;
  if (plan->dtab) (void)hipFree(plan->dtab);
  if (plan->ev_fork) (void)hipEventDestroy(plan->ev_fork);
  if (plan->ev_join) (void)hipEventDestroy(plan->ev_join);
  if (plan->side) (void)hipStreamDestroy(plan->side);
  delete plan;
}

size_t mo_plan_workspace_bytes(const mo_plan* plan) { return plan ? plan->ws_total : 0; }

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
  return plan && plan->fuse_ok && !plan->keep_ns_output ? 1 : 0;
}

int32_t mo_plan_gram_space(const mo_plan* plan) {
  if (!plan) return 0;
  for (uint8_t g : plan->ns.gspace)
    if (g) return 1;
  return 0;
}

mo_status mo_plan_slice_algorithms(const mo_plan* P, int32_t* out, int32_t n) {
  clear_error();
  if (!P || !out || n < static_cast<int32_t>(P->slices.size()))
    return fail(MO_EINVAL, "bad arguments");
  int k = 0;
  for (size_t i = 0; i < P->slices.size(); ++i) {
    if (!P->params[P->slices[i].param].grad) {
      out[i] = -1;
      continue;
    }
    out[i] = (P->ns.gspace[k] ? 1 : 0) | (P->ns.kind[k] << 1);
    ++k;
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
  if (P->last_fused)
    return fail(MO_EINVAL,
                "the last grouped step applied the update inside the Newton-Schulz launch and "
                "kept no output: call mo_plan_keep_ns_output(plan, 1) before stepping");
  const int32_t param = P->slices[slice].param;
  if (!P->params[param].grad) return fail(MO_EINVAL, "slice %d: param has no gradient", slice);
  // active slices are the slices of params with a gradient, in the same order
  int k = 0;
  for (int32_t i = 0; i < slice; ++i)
    if (P->params[P->slices[i].param].grad) ++k;
  const size_t esz = dtype_size(P->ddt);
  *o = const_cast<char*>(static_cast<const char*>(ws)) + P->ws_pool +
       P->ns.final_off(k, P->hp.ns_steps) * esz;
  *ld = P->ns.final_ld(k);
  *dtype = P->ddt;
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
  const mo_hparams& hp = P->hp;
  const float muon_lr = args && args->muon_lr >= 0.f ? args->muon_lr : hp.muon_lr;
  const float adamw_lr = args && args->adamw_lr >= 0.f ? args->adamw_lr : hp.adamw_lr;
  if (!std::isfinite(muon_lr) || !std::isfinite(adamw_lr))
    return fail(MO_EINVAL, "non-finite learning rate");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  mo_status s;
  if (P->dirty || P->uploaded_ws != ws) {
    if ((s = upload_tables(P, base, st)) != MO_OK) return s;
  }
  const int nsl = static_cast<int>(P->active.size());
  // Muon: momentum and the Newton-Schulz input (HBM-bound) first
  const char* dns = P->dtab + P->tab_ns;
  void* pool = base + P->ws_pool;
  if (nsl > 0) {
    StatPartial* stats = reinterpret_cast<StatPartial*>(base + P->ws_stats);
    float* scale = reinterpret_cast<float*>(base + P->ws_scale);
    const PrepItem* dprep = reinterpret_cast<const PrepItem*>(dns + P->nst.prep);
    if ((s = launch_momentum(reinterpret_cast<const MomSeg*>(P->dtab + P->tab_mom), nsl,
                             P->mom_blocks, hp.mu, hp.nesterov, stats, st)) != MO_OK)
      return s;
    int32_t* fb = reinterpret_cast<int32_t*>(base + P->ws_fb);
    if ((s = launch_ns_scale(dprep, nsl, stats, scale, fb, st)) != MO_OK) return s;
    if ((s = launch_ns_prep(dprep, nsl, P->ns.prep_tiles, scale, pool, P->ns.elem, st)) != MO_OK)
      return s;
    if ((s = launch_ns_prep_fallback(reinterpret_cast<const PrepItem*>(dns + P->nst.prep_fb),
                                     static_cast<int>(P->ns.prep_fb.size()), scale, fb, pool,
                                     st)) != MO_OK)
      return s;
  }
  // AdamW (clip norm and update) is independent of the Muon path: with both
  // present it goes to a side stream forked here, so that it overlaps the
  // MFMA-bound Newton-Schulz iterations rather than the HBM-bound kernels.
  // While kernel timing is enabled everything stays on `st`, in order, so that
  // each bracketed duration belongs to one kernel running alone.
  hipStream_t ast = st;
  const bool fork = nsl > 0 && P->n_adam > 0 && !timing_enabled();
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
    if (P->n_adam > 0) {
      const AdamSeg* dad = reinterpret_cast<const AdamSeg*>(P->dtab + P->tab_adam);
      double* partials = reinterpret_cast<double*>(base + P->ws_adam_partials);
      double* scal = reinterpret_cast<double*>(base + P->ws_adam_scal);
      if ((r = launch_adam_sumsq(dad, P->n_adam, P->adam_blocks, partials, ast)) != MO_OK)
        return r;
      if ((r = launch_adam_norm(partials, P->adam_blocks, hp.max_norm, scal,
                                args ? args->norm_out : nullptr, ast)) != MO_OK)
        return r;
      if ((r = launch_adam_apply(dad, P->n_adam, P->adam_blocks, scal, adamw_lr, hp.beta1,
                                 hp.beta2, hp.eps, P->tdelta, ast)) != MO_OK)
        return r;
    } else if (args && args->norm_out) {
      // no AdamW gradient: report T = 0 (a kernel write, not a memset node)
      if ((r = launch_adam_norm(nullptr, 0, hp.max_norm,
                                reinterpret_cast<double*>(base + P->ws_adam_scal), args->norm_out,
                                st)) != MO_OK)
        return r;
    }
    if (nsl > 0) {
      float coeffs[3 * MO_NS_MAX_STEPS];
      for (int k = 0; k < hp.ns_steps; ++k)
        for (int j = 0; j < 3; ++j) coeffs[3 * k + j] = hp.ns_coeffs[k][j];
      // the row table is the weight target of the fused update and the input
      // of the separate row pass
      const RowSeg* drows = reinterpret_cast<const RowSeg*>(P->dtab + P->tab_rows);
      const bool fuse = P->fuse_ok && !P->keep_ns_output;
      if ((r = ns_run_iterations(P->ns, dns, P->nst, pool,
                                 reinterpret_cast<const float*>(base + P->ws_scale), coeffs,
                                 hp.ns_steps, fuse ? drows : nullptr, muon_lr,
                                 reinterpret_cast<const int32_t*>(base + P->ws_fb), st)) != MO_OK)
        return r;
      if (!fuse) {
        RowSeg none;
        std::memset(&none, 0, sizeof(none));
        if ((r = launch_rows(hp.normuon ? kRowNormUpdate : kRowUpdate, drows, nsl, none,
                             P->total_rows, muon_lr, hp.normuon_beta2, hp.normuon_eps,
                             st)) != MO_OK)
          return r;
      }
      P->last_fused = fuse;
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
    if (s == MO_OK && e1 != hipSuccess)
      return fail(MO_EHIP, "joining the AdamW stream failed: %s", hipGetErrorString(e1));
  }
  if (s != MO_OK) return s;
  for (size_t i = 0; i < P->params.size(); ++i)
    if (P->adam_owner[i]) ++P->steps[i];
  ++P->tdelta;
  return MO_OK;
}

}  // extern "C"
