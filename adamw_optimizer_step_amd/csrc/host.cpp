// Host-only parts of the library: error strings, the routing predicate and
// view expansion.  Nothing here touches the GPU.
#include <cmath>
#include <cstring>
#include <map>
#include <set>
#include <tuple>
#include <vector>

#include "host.hpp"

namespace mo {

namespace {
thread_local std::string g_last_error;
}

mo_status fail(mo_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

// Validate a view (and split) against a stored 2-D shape and expand it into
// row slabs (kimi-k3 "build_parameter_groups": "Recording independent matrix
// geometry" for the checks; "The layout declarations are literal" for the
// row-major flattening of the leading axes and the split of each matrix's rows).
mo_status expand_view(int64_t rows, int64_t cols, int32_t view_ndim, const int64_t* view,
                      int32_t nsplit, const int64_t* split, std::vector<Slice>& out) {
  out.clear();
  if (rows <= 0 || cols <= 0) return fail(MO_ESHAPE, "stored shape (%lld, %lld) not positive",
                                          (long long)rows, (long long)cols);
  if (view_ndim == 0) {
    if (nsplit != 0) return fail(MO_ESHAPE, "split sizes need a view");
    out.push_back({0, rows, cols});
    return MO_OK;
  }
  if (view_ndim < 2 || view_ndim > MO_MAX_NDIM || !view)
    return fail(MO_ESHAPE, "view rank %d not in [2, %d]", view_ndim, MO_MAX_NDIM);
  int64_t lead = 1;
  for (int i = 0; i < view_ndim; ++i) {
    if (view[i] <= 0) return fail(MO_ESHAPE, "view entry %d is %lld (must be positive)", i,
                                  (long long)view[i]);
    if (i < view_ndim - 2) {
      if (lead > (int64_t(1) << 40) / view[i]) return fail(MO_ESHAPE, "view too large");
      lead *= view[i];
    }
  }
  const int64_t r = view[view_ndim - 2], c = view[view_ndim - 1];
  if (lead * r != rows || c != cols)
    return fail(MO_ESHAPE, "view does not flatten to the stored shape (%lld, %lld)",
                (long long)rows, (long long)cols);
  std::vector<int64_t> pieces;
  if (nsplit > 0) {
    if (nsplit > MO_MAX_SPLIT || !split) return fail(MO_ESHAPE, "too many split sizes");
    int64_t sum = 0;
    for (int i = 0; i < nsplit; ++i) {
      if (split[i] <= 0) return fail(MO_ESHAPE, "split entry %d not positive", i);
      sum += split[i];
      pieces.push_back(split[i]);
    }
    if (sum != r) return fail(MO_ESHAPE, "split sizes sum to %lld, rows are %lld",
                              (long long)sum, (long long)r);
  } else if (nsplit < 0) {
    return fail(MO_ESHAPE, "negative split count");
  } else {
    pieces.push_back(r);
  }
  for (int64_t b = 0; b < lead; ++b) {
    int64_t off = b * r;
    for (int64_t q : pieces) {
      out.push_back({off, q, c});
      off += q;
    }
  }
  return MO_OK;
}

namespace {
struct GroupKey {
  int32_t alg;
  int32_t decay;
  std::vector<int64_t> view;
  std::vector<int64_t> split;
  uint32_t exclude = 0;
  bool operator<(const GroupKey& o) const {
    return std::tie(alg, decay, view, split, exclude) <
           std::tie(o.alg, o.decay, o.view, o.split, o.exclude);
  }
};
}  // namespace

// Routing predicate (kimi-k3 "build_parameter_groups": "Exclusion and decay
// rules", "Classification happens once per original parameter identity";
// OMN "Dual-Manifold Optimization": routing paragraph).
mo_status route(const mo_param_desc* d, int32_t n, mo_route_out* out, int32_t* ngroups) {
  if (n < 0 || (n > 0 && (!d || !out))) return fail(MO_EINVAL, "bad routing arguments");
  struct ViewRec {
    std::vector<int64_t> view, split;
    uint32_t exclude;
    bool operator!=(const ViewRec& o) const {
      return view != o.view || split != o.split || exclude != o.exclude;
    }
  };
  std::map<int64_t, ViewRec> views;
  std::set<int64_t> seen;
  std::map<GroupKey, int32_t> groups;
  std::vector<Slice> sl;
  for (int32_t i = 0; i < n; ++i) {
    const mo_param_desc& p = d[i];
    if (p.ndim < 0 || p.ndim > MO_MAX_NDIM) return fail(MO_EINVAL, "param %d: bad ndim", i);
    for (int k = 0; k < p.ndim; ++k)
      if (p.shape[k] <= 0) return fail(MO_ESHAPE, "param %d: non-positive dim", i);
    if (p.view_ndim != 0 || p.nsplit != 0) {
      if (p.ndim != 2) return fail(MO_ESHAPE, "param %d: views apply to 2-D weights", i);
      mo_status s = expand_view(p.shape[0], p.shape[1], p.view_ndim, p.view, p.nsplit, p.split,
                                sl);
      if (s != MO_OK) return s;
      if (!exclude_ok(p.nsplit, p.exclude_mask))
        return fail(MO_ESHAPE, "param %d: bad exclude_mask for %d split pieces", i, p.nsplit);
      ViewRec rec{std::vector<int64_t>(p.view, p.view + p.view_ndim),
                  std::vector<int64_t>(p.split, p.split + p.nsplit), p.exclude_mask};
      auto it = views.find(p.ident);
      if (it != views.end() && it->second != rec)
        return fail(MO_ECONFLICT, "param %d: conflicting views for one parameter", i);
      views[p.ident] = rec;
    } else if (p.exclude_mask != 0) {
      return fail(MO_ESHAPE, "param %d: exclude_mask needs a view with split sizes", i);
    }
  }
  int32_t ng = 0;
  for (int32_t i = 0; i < n; ++i) {
    const mo_param_desc& p = d[i];
    out[i] = {MO_ALG_SKIP, 0, -1, 0};
    if (!p.requires_grad) continue;
    if (!seen.insert(p.ident).second) continue;
    GroupKey k;
    if (p.ndim < 2 || p.no_decay) {
      k = {MO_ALG_ADAMW, 0, {}, {}};
    } else if (p.ndim == 2 && p.role != MO_ROLE_EMBEDDING && p.role != MO_ROLE_HEAD) {
      auto it = views.find(p.ident);
      k = {MO_ALG_MUON, 1, {}, {}};
      if (it != views.end()) {
        k.view = it->second.view;
        k.split = it->second.split;
        k.exclude = it->second.exclude;
      }
    } else {
      k = {MO_ALG_ADAMW, 1, {}, {}};
    }
    auto g = groups.find(k);
    int32_t gi;
    if (g == groups.end()) { gi = ng++; groups[k] = gi; } else { gi = g->second; }
    int32_t nsl = 0;
    if (k.alg == MO_ALG_MUON) {
      expand_view(p.shape[0], p.shape[1], static_cast<int32_t>(k.view.size()), k.view.data(),
                  static_cast<int32_t>(k.split.size()), k.split.data(), sl);
      for (size_t j = 0; j < sl.size(); ++j)
        nsl += piece_excluded(k.exclude, static_cast<int32_t>(k.split.size()), j) ? 0 : 1;
    }
    out[i] = {k.alg, k.decay, gi, nsl};
  }
  if (ng == 0) return fail(MO_EEMPTY, "no trainable parameter");
  if (ngroups) *ngroups = ng;
  return MO_OK;
}

}  // namespace mo

extern "C" {

const char* mo_status_str(mo_status s) {
  switch (s) {
    case MO_OK: return "MO_OK";
    case MO_EINVAL: return "MO_EINVAL";
    case MO_ESHAPE: return "MO_ESHAPE";
    case MO_ECONFLICT: return "MO_ECONFLICT";
    case MO_EEMPTY: return "MO_EEMPTY";
    case MO_EDTYPE: return "MO_EDTYPE";
    case MO_EWORKSPACE: return "MO_EWORKSPACE";
    case MO_EHIP: return "MO_EHIP";
    case MO_EALIGN: return "MO_EALIGN";
  }
  return "MO_UNKNOWN";
}

const char* mo_last_error(void) { return mo::g_last_error.c_str(); }

const char* mo_version(void) { return "muon_adamw 0.1 (gfx950)"; }

size_t mo_abi_struct_size(int32_t which) {
  switch (which) {
    case 0: return sizeof(mo_momentum_item);
    case 1: return sizeof(mo_ns_item);
    case 2: return sizeof(mo_adamw_item);
    case 3: return sizeof(mo_param_desc);
    case 4: return sizeof(mo_route_out);
    case 5: return sizeof(mo_param);
    case 6: return sizeof(mo_hparams);
    case 7: return sizeof(mo_step_args);
    case 8: return sizeof(mo_lr_schedule);
    case 9: return sizeof(mo_ns_options);
    case 10: return sizeof(mo_plan_options);
    case 11: return sizeof(mo_group);
    case 12: return sizeof(mo_spectral_item);
  }
  return 0;
}

mo_status mo_route(const mo_param_desc* descs, int32_t n, mo_route_out* out, int32_t* ngroups) {
  mo::clear_error();
  return mo::route(descs, n, out, ngroups);
}

// Token-clock schedule (OMN "Dual-Manifold Optimization" page: warmup,
// stable phase, square-root cooldown to an absolute floor).
mo_status mo_lr_at(const mo_lr_schedule* s, double tokens, double* lr) {
  mo::clear_error();
  if (!s || !lr) return mo::fail(MO_EINVAL, "NULL schedule or output");
  const double W = s->warmup_tokens, S = s->stable_end_tokens, E = s->end_tokens;
  if (!(tokens >= 0.0) || !(W >= 0.0 && W <= S && S <= E) ||
      !(s->floor >= 0.0 && s->floor <= s->peak))
    return mo::fail(MO_EINVAL, "bad schedule (need 0 <= W <= S <= E, 0 <= floor <= peak, "
                               "tokens >= 0)");
  if (tokens < W) {
    *lr = s->peak * tokens / W;
  } else if (tokens < S) {
    *lr = s->peak;
  } else if (tokens < E) {
    const double x = (tokens - S) / (E - S);
    *lr = s->floor + (s->peak - s->floor) * (1.0 - std::sqrt(x));
  } else {
    *lr = s->floor;
  }
  return MO_OK;
}

mo_status mo_expand_view(int64_t rows, int64_t cols, int32_t view_ndim, const int64_t* view,
                         int32_t nsplit, const int64_t* split, int64_t* out_slices,
                         int32_t max_slices, int32_t* nslices) {
  mo::clear_error();
  std::vector<mo::Slice> sl;
  mo_status s = mo::expand_view(rows, cols, view_ndim, view, nsplit, split, sl);
  if (s != MO_OK) return s;
  if (nslices) *nslices = static_cast<int32_t>(sl.size());
  if (static_cast<int64_t>(sl.size()) > max_slices || (!out_slices && !sl.empty()))
    return mo::fail(MO_EINVAL, "%zu slices do not fit in %d", sl.size(), max_slices);
  for (size_t i = 0; i < sl.size(); ++i) {
    out_slices[3 * i] = sl[i].off;
    out_slices[3 * i + 1] = sl[i].rows;
    out_slices[3 * i + 2] = sl[i].cols;
  }
  return MO_OK;
}

}  // extern "C"
