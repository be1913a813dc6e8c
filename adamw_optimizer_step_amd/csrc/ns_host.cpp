// Host side of the Newton-Schulz path: pool layout, problem tables and the
// iteration driver.
#include <cstring>

#include "host.hpp"

namespace mo {

namespace {
int32_t pad_to(int64_t x, int t) { return static_cast<int32_t>(ceil_div(x, t) * t); }

GemmProb make_prob(int64_t a, int64_t b, int64_t c, int64_t ct, int64_t e, int64_t et,
                   int32_t lda, int32_t ldb, int32_t ldc, int32_t ldct, int32_t lde, int32_t ldet,
                   int32_t K, int32_t tm, int32_t tn, int32_t sym, int64_t& start) {
  GemmProb p;
  std::memset(&p, 0, sizeof(p));
  p.a_off = a; p.b_off = b; p.c_off = c; p.ct_off = ct; p.e_off = e; p.et_off = et;
  p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.ldct = ldct; p.lde = lde; p.ldet = ldet;
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
  L.buckets.resize(2);
  L.buckets[0].tile = kGemmTile;
  L.buckets[1].tile = kBigTile;
  int64_t pool = 0;
  auto take = [&pool](int64_t elems) { int64_t at = pool; pool += elems; return at; };
  for (int i = 0; i < n; ++i) {
    const int64_t r = rows[i], c = cols[i];
    const bool tall = r > c;
    const int64_t s_ = tall ? c : r, l_ = tall ? r : c;
    NsBucket& B = L.buckets[s_ >= kBigTileMinS ? 1 : 0];
    const int tile = B.tile;
    const int32_t sp = pad_to(s_, tile), lp = pad_to(l_, tile);
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

    const int32_t ts = sp / tile, tl = lp / tile;
    // Gram X X^T (K = l) into P (scaled by b) or into A; mirror tiles through ct.
    B.gram_p.push_back(make_prob(x, x, p, p, -1, -1, lp, lp, sp, sp, 0, 0, lp, ts, ts, 1,
                                 B.gram_tiles));
    if (need_a) {
      int64_t t = B.gram_p.back().start;
      B.gram_a.push_back(make_prob(x, x, a, a, -1, -1, lp, lp, sp, sp, 0, 0, lp, ts, ts, 1, t));
      // P = b A + c A A; A is exactly symmetric, so it is its own transposed E
      B.square.push_back(make_prob(a, a, p, p, a, a, sp, sp, sp, sp, sp, sp, sp, ts, ts, 1,
                                   B.square_tiles));
    }
    // Update X <- a X + P X: A_op = P (s x s), B_op = Xt (l x s), K = s;
    // X written in place (E = X), X^T into the other buffer (E^T = current X^T).
    int64_t t0 = B.upd_tiles;
    B.upd0.push_back(make_prob(p, xt0, x, xt1, x, xt0, sp, sp, lp, sp, lp, sp, sp, ts, tl, 0, t0));
    B.upd1.push_back(make_prob(p, xt1, x, xt0, x, xt1, sp, sp, lp, sp, lp, sp, sp, ts, tl, 0,
                               B.upd_tiles));
  }
  L.pool_elems = pool;
}

NsTables ns_table_offsets(const NsLayout& L) {
  NsTables T;
  WsCursor c;
  T.prep = c.take(L.prep.size() * sizeof(PrepItem), 64);
  for (const NsBucket& B : L.buckets) {
    NsBucketTables b;
    b.gram_p = c.take(B.gram_p.size() * sizeof(GemmProb), 64);
    b.gram_a = c.take(B.gram_a.size() * sizeof(GemmProb), 64);
    b.square = c.take(B.square.size() * sizeof(GemmProb), 64);
    b.upd0 = c.take(B.upd0.size() * sizeof(GemmProb), 64);
    b.upd1 = c.take(B.upd1.size() * sizeof(GemmProb), 64);
    T.b.push_back(b);
  }
  T.bytes = align_up(c.off, 256);
  return T;
}

void ns_pack_tables(const NsLayout& L, const NsTables& T, std::vector<char>& buf) {
  buf.assign(T.bytes, 0);
  auto put = [&buf](size_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(buf.data() + off, src, bytes);
  };
  put(T.prep, L.prep.data(), L.prep.size() * sizeof(PrepItem));
  for (size_t k = 0; k < L.buckets.size(); ++k) {
    const NsBucket& B = L.buckets[k];
    const NsBucketTables& b = T.b[k];
    put(b.gram_p, B.gram_p.data(), B.gram_p.size() * sizeof(GemmProb));
    put(b.gram_a, B.gram_a.data(), B.gram_a.size() * sizeof(GemmProb));
    put(b.square, B.square.data(), B.square.size() * sizeof(GemmProb));
    put(b.upd0, B.upd0.data(), B.upd0.size() * sizeof(GemmProb));
    put(b.upd1, B.upd1.data(), B.upd1.size() * sizeof(GemmProb));
  }
}

mo_status ns_run_iterations(const NsLayout& L, const char* dtab, const NsTables& T, void* pool,
                            const float* coeffs, int steps, hipStream_t st) {
  for (int k = 0; k < steps; ++k) {
    const float a = coeffs[3 * k], b = coeffs[3 * k + 1], c = coeffs[3 * k + 2];
    const bool cubic_step = c == 0.f || !L.need_a;
    // phase 1: P = b X X^T (cubic-type step), or A = X X^T then P = b A + c A A
    for (size_t q = 0; q < L.buckets.size(); ++q) {
      const NsBucket& B = L.buckets[q];
      if (B.gram_p.empty()) continue;
      const NsBucketTables& tb = T.b[q];
      const int n = static_cast<int>(B.gram_p.size());
      mo_status s;
      if (cubic_step) {
        s = launch_ns_gemm(reinterpret_cast<const GemmProb*>(dtab + tb.gram_p), n, B.gram_tiles,
                           B.tile, pool, L.elem, 0.f, b, 0, st);
      } else {
        s = launch_ns_gemm(reinterpret_cast<const GemmProb*>(dtab + tb.gram_a), n, B.gram_tiles,
                           B.tile, pool, L.elem, 0.f, 1.f, 0, st);
        if (s == MO_OK)
          s = launch_ns_gemm(reinterpret_cast<const GemmProb*>(dtab + tb.square), n,
                             B.square_tiles, B.tile, pool, L.elem, b, c, 1, st);
      }
      if (s != MO_OK) return s;
    }
    // phase 2: X <- a X + P X
    for (size_t q = 0; q < L.buckets.size(); ++q) {
      const NsBucket& B = L.buckets[q];
      if (B.upd0.empty()) continue;
      const NsBucketTables& tb = T.b[q];
      const size_t off = (k & 1) ? tb.upd1 : tb.upd0;
      mo_status s = launch_ns_gemm(reinterpret_cast<const GemmProb*>(dtab + off),
                                   static_cast<int>(B.upd0.size()), B.upd_tiles, B.tile, pool,
                                   L.elem, a, 1.f, 1, st);
      if (s != MO_OK) return s;
    }
  }
  return MO_OK;
}

}  // namespace mo
