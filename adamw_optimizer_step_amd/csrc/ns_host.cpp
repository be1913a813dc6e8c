// Host side of the Newton-Schulz path: pool layout, problem tables and the
// iteration driver.
#include <cstring>

#include "host.hpp"

namespace mo {

namespace {
int32_t pad_tile(int64_t x) { return static_cast<int32_t>(ceil_div(x, kGemmTile) * kGemmTile); }

GemmProb make_prob(int64_t a, int64_t b, int64_t c, int64_t ct, int64_t e, int32_t lda,
                   int32_t ldb, int32_t ldc, int32_t ldct, int32_t lde, int32_t K, int32_t tm,
                   int32_t tn, int32_t sym, int64_t& start) {
  GemmProb p;
  p.a_off = a; p.b_off = b; p.c_off = c; p.ct_off = ct; p.e_off = e;
  p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.ldct = ldct; p.lde = lde;
  p.K = K; p.tiles_m = tm; p.tiles_n = tn; p.sym = sym;
  p.start = static_cast<int32_t>(start);
  start += sym ? static_cast<int64_t>(tm) * (tm + 1) / 2 : static_cast<int64_t>(tm) * tn;
  return p;
}
}  // namespace

void build_ns_layout(NsLayout& L, const int64_t* rows, const int64_t* cols, int n, int elem,
                     bool need_a) {
  L = NsLayout();
  L.elem = elem;
  L.need_a = need_a;
  L.n = n;
  int64_t pool = 0;
  auto take = [&pool](int64_t elems) { int64_t at = pool; pool += elems; return at; };
  for (int i = 0; i < n; ++i) {
    const int64_t r = rows[i], c = cols[i];
    const bool tall = r > c;
    const int32_t sp = pad_tile(tall ? c : r), lp = pad_tile(tall ? r : c);
    const int64_t x = take(static_cast<int64_t>(sp) * lp);
    const int64_t xt0 = take(static_cast<int64_t>(lp) * sp);
    const int64_t xt1 = take(static_cast<int64_t>(lp) * sp);
    const int64_t p = take(static_cast<int64_t>(sp) * sp);
    const int64_t a = need_a ? take(static_cast<int64_t>(sp) * sp) : -1;
    L.x_off.push_back(x);
    L.xt_off0.push_back(xt0);
    L.xt_off1.push_back(xt1);
    L.tall.push_back(tall);
    L.sp.push_back(sp);
    L.lp.push_back(lp);

    PrepItem pi;
    std::memset(&pi, 0, sizeof(pi));
    pi.r = static_cast<int32_t>(r);
    pi.c = static_cast<int32_t>(c);
    pi.rp = tall ? lp : sp;
    pi.cp = tall ? sp : lp;
    pi.sbuf = tall ? xt0 : x;
    pi.stbuf = tall ? x : xt0;
    pi.tiles_c = pi.cp / kPrepTile;
    pi.start = L.prep_tiles;
    L.prep_tiles += static_cast<int64_t>(pi.rp / kPrepTile) * pi.tiles_c;
    L.prep.push_back(pi);

    const int32_t ts = sp / kGemmTile, tl = lp / kGemmTile;
    // Gram X X^T (K = l) into P (scaled by b) or into A.
    L.gram_p.push_back(make_prob(x, x, p, p, -1, lp, lp, sp, sp, 0, lp, ts, ts, 1, L.gram_tiles));
    if (need_a) {
      int64_t t = L.gram_p.back().start;
      L.gram_a.push_back(make_prob(x, x, a, a, -1, lp, lp, sp, sp, 0, lp, ts, ts, 1, t));
      L.square.push_back(make_prob(a, a, p, p, a, sp, sp, sp, sp, sp, sp, ts, ts, 1,
                                   L.square_tiles));
    }
    // Update X <- a X + P X: A_op = P (s x s), B_op = Xt (l x s), K = s;
    // X written in place, X^T into the other buffer.
    int64_t t0 = L.upd_tiles;
    L.upd0.push_back(make_prob(p, xt0, x, xt1, x, sp, sp, lp, sp, lp, sp, ts, tl, 0, t0));
    L.upd1.push_back(make_prob(p, xt1, x, xt0, x, sp, sp, lp, sp, lp, sp, ts, tl, 0, L.upd_tiles));
  }
  L.pool_elems = pool;
}

NsTables ns_table_offsets(const NsLayout& L) {
  NsTables T;
  WsCursor c;
  T.prep = c.take(L.prep.size() * sizeof(PrepItem), 64);
  T.gram_p = c.take(L.gram_p.size() * sizeof(GemmProb), 64);
  T.gram_a = c.take(L.gram_a.size() * sizeof(GemmProb), 64);
  T.square = c.take(L.square.size() * sizeof(GemmProb), 64);
  T.upd0 = c.take(L.upd0.size() * sizeof(GemmProb), 64);
  T.upd1 = c.take(L.upd1.size() * sizeof(GemmProb), 64);
  T.bytes = align_up(c.off, 256);
  return T;
}

void ns_pack_tables(const NsLayout& L, const NsTables& T, std::vector<char>& buf) {
  buf.assign(T.bytes, 0);
  auto put = [&buf](size_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(buf.data() + off, src, bytes);
  };
  put(T.prep, L.prep.data(), L.prep.size() * sizeof(PrepItem));
  put(T.gram_p, L.gram_p.data(), L.gram_p.size() * sizeof(GemmProb));
  put(T.gram_a, L.gram_a.data(), L.gram_a.size() * sizeof(GemmProb));
  put(T.square, L.square.data(), L.square.size() * sizeof(GemmProb));
  put(T.upd0, L.upd0.data(), L.upd0.size() * sizeof(GemmProb));
  put(T.upd1, L.upd1.data(), L.upd1.size() * sizeof(GemmProb));
}

mo_status ns_run_iterations(const NsLayout& L, const char* dtab, const NsTables& T, void* pool,
                            const float* coeffs, int steps, hipStream_t st) {
  const GemmProb* gram_p = reinterpret_cast<const GemmProb*>(dtab + T.gram_p);
  const GemmProb* gram_a = reinterpret_cast<const GemmProb*>(dtab + T.gram_a);
  const GemmProb* square = reinterpret_cast<const GemmProb*>(dtab + T.square);
  const GemmProb* upd[2] = {reinterpret_cast<const GemmProb*>(dtab + T.upd0),
                            reinterpret_cast<const GemmProb*>(dtab + T.upd1)};
  for (int k = 0; k < steps; ++k) {
    const float a = coeffs[3 * k], b = coeffs[3 * k + 1], c = coeffs[3 * k + 2];
    mo_status s;
    if (c == 0.f || !L.need_a) {
      // P = b X X^T   (cubic-type step)
      s = launch_ns_gemm(gram_p, L.n, L.gram_tiles, pool, L.elem, 0.f, b, 0, st);
    } else {
      // A = X X^T;  P = b A + c A A
      s = launch_ns_gemm(gram_a, L.n, L.gram_tiles, pool, L.elem, 0.f, 1.f, 0, st);
      if (s == MO_OK) s = launch_ns_gemm(square, L.n, L.square_tiles, pool, L.elem, b, c, 1, st);
    }
    if (s != MO_OK) return s;
    // X <- a X + P X
    s = launch_ns_gemm(upd[k & 1], L.n, L.upd_tiles, pool, L.elem, a, 1.f, 1, st);
    if (s != MO_OK) return s;
  }
  return MO_OK;
}

}  // namespace mo
