// Host side of the Newton-Schulz path: pool layout, problem tables and the
// iteration driver.
#include <algorithm>
#include <cstring>

#include "host.hpp"

namespace mo {

namespace {
int32_t pad_to(int64_t x, int t) { return static_cast<int32_t>(ceil_div(x, t) * t); }

GemmProb make_prob(int64_t a, int64_t b, int64_t c, int64_t ct, int64_t e, int32_t lda,
                   int32_t ldb, int32_t ldc, int32_t ldct, int32_t lde, int32_t K, int32_t tm,
                   int32_t tn, int32_t sym, int64_t start) {
  GemmProb p;
  std::memset(&p, 0, sizeof(p));
  p.a_off = a; p.b_off = b; p.c_off = c; p.ct_off = ct; p.e_off = e;
  p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.ldct = ldct; p.lde = lde;
  p.K = K; p.tiles_m = tm; p.tiles_n = tn; p.sym = sym;
  p.start = static_cast<int32_t>(start);
  p.item = -1;
  p.sitem = -1;
  p.alt_off = -1;
  p.c2_off = -1;
  return p;
}

int64_t tiles_of(int32_t tm, int32_t tn, bool sym) {
  return sym ? static_cast<int64_t>(tm) * (tm + 1) / 2 : static_cast<int64_t>(tm) * tn;
}

// Longest tiles (largest K) first, then renumber the first-tile indices: the
// short tiles fill the end of the launch.
void order_by_k(std::vector<GemmProb>& v) {
  std::stable_sort(v.begin(), v.end(),
                   [](const GemmProb& a, const GemmProb& b) { return a.K > b.K; });
  int64_t start = 0;
  for (GemmProb& p : v) {
    p.start = static_cast<int32_t>(start);
    start += tiles_of(p.tiles_m, p.tiles_n, p.sym != 0);
  }
}
}  // namespace

mo_status resolve_ns_options(const mo_ns_options* o, NsOpts& out) {
  out = NsOpts();
  if (!o) return MO_OK;
  if (o->gram_space != 0 && o->gram_space != 1)
    return fail(MO_EINVAL, "ns options: gram_space must be 0 or 1");
  if (o->big_tile_min_work < -1 || o->few_tile_max < -1)
    return fail(MO_EINVAL, "ns options: thresholds must be >= -1 (-1 = default)");
  out.gram_space = o->gram_space != 0;
  if (o->big_tile_min_work >= 0) out.big_tile_min_work = o->big_tile_min_work;
  if (o->few_tile_max >= 0) out.few_tile_max = o->few_tile_max;
  return MO_OK;
}

bool gram_gain_ok(const float* coeffs, int steps) {
  if (!coeffs || steps <= 0) return false;
  double gain = 1.0;
  for (int k = 0; k < steps; ++k) gain *= static_cast<double>(coeffs[3 * k]) * coeffs[3 * k];
  return gain <= kGramSpaceMaxGain;
}

void build_ns_layout(NsLayout& L, const int64_t* rows, const int64_t* cols, int n, int elem,
                     const float* coeffs, int steps, const NsOpts& opt,
                     const uint8_t* direct_ok, bool stats_from_prep, const int64_t* in_off) {
  L = NsLayout();
  bool need_a = false;
  for (int k = 0; k < steps; ++k)
    if (coeffs[3 * k + 2] != 0.f) need_a = true;
  // Gram space (bf16): the table's small-singular-value gain bounded, see
  // kGramSpaceMaxGain
  const bool gram_ok = elem == 2 && opt.gram_space && gram_gain_ok(coeffs, steps);
  const bool gspace_mode = gram_ok;
  L.few_tile_max = opt.few_tile_max;
  L.elem = elem;
  L.need_a = need_a;
  L.n = n;
  L.buckets.resize(2);
  L.buckets[0].tile = kGemmTile;
  L.buckets[1].tile = kBigTile;
  int64_t pool = 0;
  auto take = [&pool](int64_t elems) { int64_t at = pool; pool += elems; return at; };
  // 256 x 256 tiles only when they give enough workgroups per launch to fill
  // the chip; otherwise 128 x 128 tiles (4x as many) finish sooner
  int64_t big_tiles = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t s_ = std::min(rows[i], cols[i]), l_ = std::max(rows[i], cols[i]);
    if (s_ < kBigTileMinS) continue;
    const int64_t ts = ceil_div(s_, kBigTile), tl = ceil_div(l_, kBigTile);
    big_tiles += std::min(ts * (ts + 1) / 2, ts * tl);
  }
  const bool use_big = big_tiles >= opt.big_tile_min_work;
  for (int i = 0; i < n; ++i) {
    const int64_t r = rows[i], c = cols[i];
    const bool tall = r > c;
    const int64_t s_ = tall ? c : r, l_ = tall ? r : c;
    NsBucket& B = L.buckets[use_big && s_ >= kBigTileMinS ? 1 : 0];
    const int tile = B.tile;
    const int32_t sp = pad_to(s_, tile), lp = pad_to(l_, tile);
    const bool small = elem == 2 && tile == kGemmTile && sp == kSmallS;
    // GEMM path: rectangular slices only; on a square one Gram space executes
    // the same flops as the plain iteration in one more launch
    const bool gs = gspace_mode && !small && 4 * l_ >= 5 * s_;
    // (the slice-resident kernel's Gram space also takes quintic-type rows)
    const bool sgs = gram_ok && small && s_ >= kGramSpaceMinS;
    const int64_t x[2] = {take(static_cast<int64_t>(sp) * lp), take(static_cast<int64_t>(sp) * lp)};
    const int64_t p = small || gs ? -1 : take(static_cast<int64_t>(sp) * sp);
    const int64_t a = need_a && !small && !gs ? take(static_cast<int64_t>(sp) * sp) : -1;
    L.gspace.push_back(gs || sgs);
    L.kind.push_back(small ? 2 : tile == kBigTile ? 1 : 0);
    L.x_off[0].push_back(x[0]);
    L.x_off[1].push_back(x[1]);
    L.tall.push_back(tall);
    L.sp.push_back(sp);
    L.lp.push_back(lp);

    // X0 = normalised D in the short-side orientation (transposed when tall)
    PrepItem pi;
    std::memset(&pi, 0, sizeof(pi));
    pi.r = static_cast<int32_t>(r);
    pi.c = static_cast<int32_t>(c);
    pi.rp = tall ? lp : sp;
    pi.cp = tall ? sp : lp;
    pi.sbuf = tall ? -1 : x[0];
    pi.stbuf = tall ? x[0] : -1;
    pi.tiles_c = pi.cp / kPrepTile;
    pi.start = L.prep_tiles;
    L.prep_tiles += static_cast<int64_t>(pi.rp / kPrepTile) * pi.tiles_c;
    L.prep.push_back(pi);

    if (small) {
      SmallProb sm;
      std::memset(&sm, 0, sizeof(sm));
      sm.x_off[0] = x[0];
      sm.x_off[1] = x[1];
      sm.lp = lp;
      sm.tall = tall;
      sm.item = i;
      sm.direct = direct_ok && direct_ok[i] && !tall && s_ == kSmallS && lp == l_;
      if (sm.direct) {
        // no X0 copy; the prep tiles stay only where they feed the statistics
        L.prep.back().sbuf = -1;
        L.prep.back().stbuf = -1;
        if (!stats_from_prep) L.prep_tiles = L.prep.back().start;
      }
      (sgs ? L.small_gs : L.small).push_back(sm);
      continue;
    }
    const int32_t ts = sp / tile, tl = lp / tile;
    // K of each product: the real extent rounded up to a 64-deep K slab (a
    // multiple of every kernel's slab), not the padded one.  The pool's
    // padding is zero and stays zero, so the K slabs past it add nothing:
    // a 192-row slice's s x s products and final update take 3 slabs instead
    // of the 4 of its 256-row padding.
    const int32_t ks = static_cast<int32_t>(pad_to(s_, 64)), kl = static_cast<int32_t>(pad_to(l_, 64));
    // Every operand of this slice's products has s rows of data (X: s x l,
    // the s x s matrices): the loads of the padded rows read zero.
    auto mk = [&](auto... args) {
      GemmProb g = make_prob(args...);
      g.a_rows = g.b_rows = static_cast<int32_t>(s_);
      return g;
    };
    // iteration 0 reads D in place when it has X0's layout (not tall, the
    // long side a multiple of the tile; in 128 x 128 tiles a padded short
    // side reads zero past its last row, and is a multiple of 64, so that
    // the K-major reads of the last product stop at its last row): no prep
    // copy, the scale folded into the products
    const bool gdirect = in_off && direct_ok && direct_ok[i] && !tall && lp == l_ &&
                         (sp == s_ || (tile == kGemmTile && s_ % 64 == 0));
    if (gdirect) {
      // the prep copy stays available for slices whose range flag is set
      PrepItem fb = L.prep.back();
      fb.slice = i;
      L.prep_fb.push_back(fb);
      L.prep.back().sbuf = -1;
      L.prep.back().stbuf = -1;
      if (!stats_from_prep) L.prep_tiles = L.prep.back().start;
    }
    const int64_t x0 = gdirect ? in_off[i] : x[0];
    const int32_t si = gdirect ? i : -1;
    auto first = [&](GemmProb g) {
      g.sitem = si;
      g.alt_off = gdirect ? x[0] : -1;
      return g;
    };
    if (gs) {
      // s x s buffers: A_k in Ab[k % 2], T_k in Tb, a quintic-type row's
      // P_k in Pb (P_0 in Qb[0], which is Q_1), Q_k in Qb[(k - 1) % 2]
      int64_t Ab[2], Tb, Pb, Qb[2];
      for (auto& v : Ab) v = take(static_cast<int64_t>(sp) * sp);
      Tb = take(static_cast<int64_t>(sp) * sp);
      Pb = need_a ? take(static_cast<int64_t>(sp) * sp) : -1;
      for (auto& v : Qb) v = take(static_cast<int64_t>(sp) * sp);
      size_t stage = 0;
      auto add = [&](int32_t kind, int32_t k, const GemmProb& g) {
        if (B.gs.size() <= stage) {
          B.gs.resize(stage + 1);
          B.gs_kind.resize(stage + 1);
          B.gs_k.resize(stage + 1);
          B.gs_tiles.resize(stage + 1);
        }
        B.gs[stage].push_back(g);
        B.gs_kind[stage] = kind;
        B.gs_k[stage] = k;
        B.gs_tiles[stage] += tiles_of(g.tiles_m, g.tiles_n, g.sym != 0);
      };
      // C = c0 E + c1 (U V^T) (+ cd I) over s x s symmetric operands; the
      // result is symmetric too (all factors are polynomials in A_0).  Every
      // product with an E term has E = U, so that E passes through LDS with
      // the left operand (see launch_ns_gemm's has_e).
      auto prod = [&](int64_t u, int64_t v, int64_t e, int64_t out) {
        return mk(u, v, out, out, e, sp, sp, sp, sp, sp, ks, ts, ts, 1, 0);
      };
      const bool quintic0 = coeffs[2] != 0.f;
      GemmProb g = first(mk(x0, x0, Ab[0], Ab[0], -1, lp, lp, sp, sp, 0, kl, ts, ts, 1, 0));
      g.c2_off = quintic0 ? -1 : Qb[0];   // Q_1 = P_0 = a_0 I + b_0 A_0 (cubic-type row 0)
      add(kGsGram, 0, g);
      ++stage;
      for (int k = 0; k < steps; ++k) {
        const bool last = k + 1 == steps;
        const int64_t Ak = Ab[k % 2], An = Ab[(k + 1) % 2];
        const int64_t Qk = k >= 1 ? Qb[(k - 1) % 2] : -1, Qn = Qb[k % 2];
        if (coeffs[3 * k + 2] == 0.f) {
          // cubic-type row, P_k = a I + b A_k kept implicit in the E term:
          // T_k = a A_k + b A_k A_k, Q_{k+1} = a Q_k + b Q_k A_k (Q_k and A_k
          // commute), A_{k+1} = a T_k + b T_k A_k
          if (!last) add(kGsProd, k, prod(Ak, Ak, Ak, Tb));
          if (k >= 1) add(kGsProd, k, prod(Qk, Ak, Qk, Qn));
          if (!last || k >= 1) ++stage;
          if (!last) {
            add(kGsProd, k, prod(Tb, Ak, Tb, An));
            ++stage;
          }
        } else {
          // quintic-type row: P_k = c A_k A_k + b A_k + a I materialised,
          // then T_k = P_k A_k, Q_{k+1} = P_k Q_k, A_{k+1} = T_k P_k
          const int64_t Pk = k == 0 ? Qb[0] : Pb;
          add(kGsProdP, k, prod(Ak, Ak, Ak, Pk));
          ++stage;
          if (!last) add(kGsProdPlain, k, prod(Pk, Ak, -1, Tb));
          if (k >= 1) add(kGsProdPlain, k, prod(Pk, Qk, -1, Qn));
          if (!last || k >= 1) ++stage;
          if (!last) {
            add(kGsProdPlain, k, prod(Tb, Pk, -1, An));
            ++stage;
          }
        }
      }
      // X_N = Q_N X0 into the second iterate buffer (transposed when tall)
      const int64_t qn = Qb[(steps - 1) % 2];
      GemmProb f = first(tall ? mk(qn, x0, -1, x[1], -1, sp, lp, 0, sp, 0, ks, ts, tl, 0, 0)
                              : mk(qn, x0, x[1], -1, -1, sp, lp, lp, 0, 0, ks, ts, tl, 0,
                                          0));
      f.item = i;
      add(kGsFinal, steps - 1, f);
      continue;
    }
    B.gram_p0.push_back(
        first(mk(x0, x0, p, p, -1, lp, lp, sp, sp, 0, kl, ts, ts, 1, B.gram_tiles)));
    if (need_a)
      B.gram_a0.push_back(
          first(mk(x0, x0, a, a, -1, lp, lp, sp, sp, 0, kl, ts, ts, 1, B.gram_tiles)));
    const GemmProb u0 =
        first(mk(p, x0, x[1], -1, -1, sp, lp, lp, 0, 0, ks, ts, tl, 0, B.upd_tiles));
    B.upd0.push_back(u0);
    GemmProb f0 = tall ? first(mk(p, x0, -1, x[1], -1, sp, lp, 0, sp, 0, ks, ts, tl, 0,
                                         B.upd_tiles))
                       : u0;
    f0.item = i;
    B.fin0.push_back(f0);
    for (int q = 0; q < 2; ++q) {
      const int64_t xc = x[q], xn = x[q ^ 1];
      // Gram X X^T (K = l), B = X read N x K: into P (scaled by b) or into A;
      // the lower triangle is written as the mirror through ct.
      B.gram_p[q].push_back(mk(xc, xc, p, p, -1, lp, lp, sp, sp, 0, kl, ts, ts, 1,
                                      B.gram_tiles));
      if (need_a)
        B.gram_a[q].push_back(mk(xc, xc, a, a, -1, lp, lp, sp, sp, 0, kl, ts, ts, 1,
                                        B.gram_tiles));
      // Update X' = P X (P = a I + b A + c A^2): A = P (s x s), B = X read
      // K-major (K = s); the next buffer receives the result.
      B.upd[q].push_back(mk(p, xc, xn, -1, -1, sp, lp, lp, 0, 0, ks, ts, tl, 0,
                                   B.upd_tiles));
      // Last iteration: a tall matrix is written transposed (l x s, stored
      // orientation) instead.
      B.fin[q].push_back(tall ? mk(p, xc, -1, xn, -1, sp, lp, 0, sp, 0, ks, ts, tl, 0,
                                          B.upd_tiles)
                              : B.upd[q].back());
      B.fin[q].back().item = i;
    }
    if (need_a) {
      // P = b A + c A A; A is exactly symmetric, so it is its own transposed
      // operand and its own E term.
      B.square.push_back(mk(a, a, p, p, a, sp, sp, sp, sp, sp, ks, ts, ts, 1,
                                   B.square_tiles));
      B.square_tiles += tiles_of(ts, ts, true);
    }
    B.gram_tiles += tiles_of(ts, ts, true);
    B.upd_tiles += tiles_of(ts, tl, false);
  }
  // slice-resident problems: longest first
  for (auto* v : {&L.small, &L.small_gs})
    std::stable_sort(v->begin(), v->end(),
                     [](const SmallProb& a, const SmallProb& b) { return a.lp > b.lp; });
  for (NsBucket& B : L.buckets) {
    for (int q = 0; q < 2; ++q) {
      order_by_k(B.gram_p[q]);
      order_by_k(B.gram_a[q]);
      order_by_k(B.upd[q]);
      order_by_k(B.fin[q]);
    }
    order_by_k(B.square);
    for (auto& v : B.gs) order_by_k(v);
    order_by_k(B.gram_p0);
    order_by_k(B.gram_a0);
    order_by_k(B.upd0);
    order_by_k(B.fin0);
  }
  L.pool_elems = pool;
}

NsTables ns_table_offsets(const NsLayout& L) {
  NsTables T;
  WsCursor c;
  T.prep = c.take(L.prep.size() * sizeof(PrepItem), 64);
  T.prep_fb = c.take(L.prep_fb.size() * sizeof(PrepItem), 64);
  T.small = c.take(L.small.size() * sizeof(SmallProb), 64);
  T.small_gs = c.take(L.small_gs.size() * sizeof(SmallProb), 64);
  for (const NsBucket& B : L.buckets) {
    NsBucketTables b;
    auto take = [&c](const std::vector<GemmProb>& v) { return c.take(v.size() * sizeof(GemmProb), 64); };
    for (int q = 0; q < 2; ++q) {
      b.gram_p[q] = take(B.gram_p[q]);
      b.gram_a[q] = take(B.gram_a[q]);
      b.upd[q] = take(B.upd[q]);
      b.fin[q] = take(B.fin[q]);
    }
    b.square = take(B.square);
    b.gram_p0 = take(B.gram_p0);
    b.gram_a0 = take(B.gram_a0);
    b.upd0 = take(B.upd0);
    b.fin0 = take(B.fin0);
    for (const auto& v : B.gs) b.gs.push_back(take(v));
    T.b.push_back(b);
  }
  T.bytes = align_up(c.off, 256);
  return T;
}

void ns_pack_tables(const NsLayout& L, const NsTables& T, std::vector<char>& buf) {
  buf.assign(T.bytes, 0);
  auto put = [&buf](size_t off, const std::vector<GemmProb>& v) {
    if (!v.empty()) std::memcpy(buf.data() + off, v.data(), v.size() * sizeof(GemmProb));
  };
  if (!L.prep.empty())
    std::memcpy(buf.data() + T.prep, L.prep.data(), L.prep.size() * sizeof(PrepItem));
  if (!L.prep_fb.empty())
    std::memcpy(buf.data() + T.prep_fb, L.prep_fb.data(), L.prep_fb.size() * sizeof(PrepItem));
  if (!L.small.empty())
    std::memcpy(buf.data() + T.small, L.small.data(), L.small.size() * sizeof(SmallProb));
  if (!L.small_gs.empty())
    std::memcpy(buf.data() + T.small_gs, L.small_gs.data(),
                L.small_gs.size() * sizeof(SmallProb));
  for (size_t k = 0; k < L.buckets.size(); ++k) {
    const NsBucket& B = L.buckets[k];
    const NsBucketTables& b = T.b[k];
    for (int q = 0; q < 2; ++q) {
      put(b.gram_p[q], B.gram_p[q]);
      put(b.gram_a[q], B.gram_a[q]);
      put(b.upd[q], B.upd[q]);
      put(b.fin[q], B.fin[q]);
    }
    put(b.square, B.square);
    put(b.gram_p0, B.gram_p0);
    put(b.gram_a0, B.gram_a0);
    put(b.upd0, B.upd0);
    put(b.fin0, B.fin0);
    for (size_t j = 0; j < B.gs.size(); ++j) put(b.gs[j], B.gs[j]);
  }
}

namespace {
// Which of the three independent chains a layout has: slice-resident
// launches, the Gram-space GEMM sequence, plain-iteration GEMM launches.
struct Chains {
  bool small = false, gs = false, plain = false;
};
Chains chains_of(const NsLayout& L) {
  Chains c;
  c.small = !L.small.empty() || !L.small_gs.empty();
  for (const NsBucket& B : L.buckets) {
    c.gs = c.gs || !B.gs.empty();
    c.plain = c.plain || !B.gram_p[0].empty();
  }
  return c;
}

// Every problem of a launch has the same K: its tiles take the same time, and
// the launch can run persistent (a workgroup per resident slot, several tiles
// each) with no workgroup left holding the long tiles.
bool one_k(const std::vector<GemmProb>& probs) {
  for (const GemmProb& g : probs)
    if (g.K != probs.front().K) return false;
  return true;
}
}  // namespace

bool ns_has_two_chains(const NsLayout& L) {
  const Chains c = chains_of(L);
  return static_cast<int>(c.small) + static_cast<int>(c.gs) + static_cast<int>(c.plain) >= 2;
}

mo_status ns_run_iterations(const NsLayout& L, const char* dtab, const NsTables& T, void* pool,
                            const float* scale, const float* coeffs, int steps, const RowSeg* wt,
                            float lr, const float* lrs, const int32_t* range_fb,
                            hipStream_t st, hipStream_t st2) {
  auto tab = [dtab](size_t off) { return reinterpret_cast<const GemmProb*>(dtab + off); };
  // With st2: the Gram-space sequence stays on st, the slice-resident and
  // plain-iteration launches go to st2; without a Gram-space sequence the
  // plain iteration stays on st.
  const Chains ch = chains_of(L);
  hipStream_t sm_st = st2 ? st2 : st;
  hipStream_t ps_st = st2 && ch.gs ? st2 : st;
  for (int gsm = 0; gsm < 2; ++gsm) {
    const std::vector<SmallProb>& v = gsm ? L.small_gs : L.small;
    if (v.empty()) continue;
    mo_status s = launch_ns_small(
        reinterpret_cast<const SmallProb*>(dtab + (gsm ? T.small_gs : T.small)),
        static_cast<int>(v.size()), pool, reinterpret_cast<const PrepItem*>(dtab + T.prep),
        scale, coeffs, steps, wt, lr, lrs, sm_st, gsm, range_fb);
    if (s != MO_OK) return s;
  }
  // Gram-space sequence (every GEMM slice of the layout, or none)
  size_t nstage = 0;
  for (const NsBucket& B : L.buckets) nstage = std::max(nstage, B.gs.size());
  for (size_t j = 0; j < nstage; ++j) {
    for (size_t i = 0; i < L.buckets.size(); ++i) {
      const NsBucket& B = L.buckets[i];
      if (j >= B.gs.size()) continue;
      const int k = B.gs_k[j];
      const float a = coeffs[3 * k], b = coeffs[3 * k + 1];
      const GemmProb* t = tab(T.b[i].gs[j]);
      const int n = static_cast<int>(B.gs[j].size());
      // E products: the E term from the left operand's slabs (has_e 2), except
      // in launches of few tiles, whose short K loops pay more for the add
      // than for reading E in the epilogue
      const bool few = B.tile == kGemmTile && B.gs_tiles[j] < L.few_tile_max;
      const int e_mode = L.elem == 2 && !few ? 2 : 1;
      mo_status s;
      if (B.gs_kind[j] == kGsGram)
        s = launch_ns_gemm(t, n, B.gs_tiles[j], one_k(B.gs[j]), B.tile, L.few_tile_max, 0, pool, L.elem, 0.f, 1.f, 0, 0.f,
                           nullptr, 0.f, nullptr, scale, range_fb, st, b, a);
      else if (B.gs_kind[j] == kGsProd)   // E = U in every problem (bf16: has_e 2)
        s = launch_ns_gemm(t, n, B.gs_tiles[j], one_k(B.gs[j]), B.tile, L.few_tile_max, 0, pool, L.elem, a, b, e_mode,
                           0.f, nullptr, 0.f, nullptr, nullptr, nullptr, st);
      else if (B.gs_kind[j] == kGsProdP)
        s = launch_ns_gemm(t, n, B.gs_tiles[j], one_k(B.gs[j]), B.tile, L.few_tile_max, 0, pool, L.elem, b,
                           coeffs[3 * k + 2], e_mode, a, nullptr, 0.f, nullptr, nullptr, nullptr, st);
      else if (B.gs_kind[j] == kGsProdPlain)
        s = launch_ns_gemm(t, n, B.gs_tiles[j], one_k(B.gs[j]), B.tile, L.few_tile_max, 0, pool, L.elem, 0.f,
                           1.f, 0, 0.f, nullptr, 0.f, nullptr, nullptr, nullptr, st);
      else
        s = launch_ns_gemm(t, n, B.gs_tiles[j], one_k(B.gs[j]), B.tile, L.few_tile_max, 1, pool, L.elem, 0.f, 1.f, 0, 0.f, wt,
                           lr, lrs, scale, range_fb, st);
      if (s != MO_OK) return s;
    }
  }
  // the plain iteration
  for (int k = 0; k < steps; ++k) {
    const float a = coeffs[3 * k], b = coeffs[3 * k + 1], c = coeffs[3 * k + 2];
    const bool cubic_step = c == 0.f || !L.need_a;
    const int q = k & 1;
    // iteration 0 has tables of its own (inputs read in place, scaled by the
    // per-slice scale); later iterations alternate between two parities
    const bool first = k == 0;
    const float* ps = first ? scale : nullptr;
    const int32_t* pfb = first ? range_fb : nullptr;
    // phase 1: P = a I + b X X^T (cubic-type step), or A = X X^T then
    // P = a I + b A + c A A.  The a X term of the update is folded into P.
    for (size_t i = 0; i < L.buckets.size(); ++i) {
      const NsBucket& B = L.buckets[i];
      if (B.gram_p[q].empty()) continue;
      const NsBucketTables& tb = T.b[i];
      const int n = static_cast<int>(B.gram_p[q].size());
      const bool uk = one_k(first ? B.gram_p0 : B.gram_p[q]);
      mo_status s;
      if (cubic_step) {
        s = launch_ns_gemm(tab(first ? tb.gram_p0 : tb.gram_p[q]), n, B.gram_tiles, uk, B.tile, L.few_tile_max, 0,
                           pool, L.elem, 0.f, b, 0, a, nullptr, 0.f, nullptr, ps, pfb, ps_st);
      } else {
        s = launch_ns_gemm(tab(first ? tb.gram_a0 : tb.gram_a[q]), n, B.gram_tiles, uk, B.tile, L.few_tile_max, 0,
                           pool, L.elem, 0.f, 1.f, 0, 0.f, nullptr, 0.f, nullptr, ps, pfb, ps_st);
        if (s == MO_OK)
          s = launch_ns_gemm(tab(tb.square), n, B.square_tiles, one_k(B.square), B.tile, L.few_tile_max, 0, pool, L.elem, b, c, 1,
                             a, nullptr, 0.f, nullptr, nullptr, nullptr, ps_st);
      }
      if (s != MO_OK) return s;
    }
    // phase 2: X' = P X
    for (size_t i = 0; i < L.buckets.size(); ++i) {
      const NsBucket& B = L.buckets[i];
      if (B.upd[q].empty()) continue;
      const NsBucketTables& tb = T.b[i];
      const bool fin = k + 1 == steps;
      const size_t off = fin ? (first ? tb.fin0 : tb.fin[q]) : (first ? tb.upd0 : tb.upd[q]);
      const std::vector<GemmProb>& probs = fin ? (first ? B.fin0 : B.fin[q]) : (first ? B.upd0 : B.upd[q]);
      mo_status s = launch_ns_gemm(tab(off), static_cast<int>(B.upd[q].size()), B.upd_tiles,
                                   one_k(probs), B.tile, L.few_tile_max, 1, pool, L.elem, 0.f, 1.f, 0, 0.f, fin ? wt : nullptr,
                                   lr, lrs, ps, pfb, ps_st);
      if (s != MO_OK) return s;
    }
  }
  return MO_OK;
}

}  // namespace mo
