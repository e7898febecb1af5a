// Host-side layout algebra behind the C ABI: descriptor checks, text form,
// size/cosize, coalesce, composition, right inverse, zipped_divide, injectivity
// and the thread-map layouts.  Plain C++17; no device code.
//
// Pages cited (title, address):
//   [ThreadMap page]     CUTLASS 2.x PitchLinearStripminedThreadMap article, hotelren.com/news/5252042
//   [CuTe algebra page]  "CUTE布局代数：GPU张量计算的内存优化革命", jsqmd.com/news/768714
//   [print_layout page]  "CUTLASS Layout可视化：从print_layout理解GPU内存映射与性能优化",
//                        codechina.net/article/weixin_30702441/411096

#include <algorithm>
#include <cctype>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "lr_internal.h"

namespace lr {

// ---------------------------------------------------------------- checks

int validate(const lr_layout* L) {
  if (!L) return LR_ERR_INVALID;
  if (L->nleaves < 1 || L->nleaves > LR_MAX_LEAVES) return LR_ERR_INVALID;
  if (L->nmodes < 1 || L->nmodes > L->nleaves) return LR_ERR_INVALID;
  int prev = 0;
  for (int i = 0; i < L->nmodes; ++i) {
    if (L->mode_end[i] <= prev) return LR_ERR_INVALID;
    prev = L->mode_end[i];
  }
  if (prev != L->nleaves) return LR_ERR_INVALID;
  int64_t sz = 1, mx = 0;
  for (int i = 0; i < L->nleaves; ++i) {
    if (L->shape[i] < 1 || L->stride[i] < 0) return LR_ERR_INVALID;
    if (!mul_ok(sz, L->shape[i], &sz)) return LR_ERR_OVERFLOW;
    int64_t t;
    if (!mul_ok(L->shape[i] - 1, L->stride[i], &t) || !add_ok(mx, t, &mx)) return LR_ERR_OVERFLOW;
  }
  if (L->swz_b < 0) return LR_ERR_SWIZZLE;
  if (L->swz_b > 0) {
    if (L->swz_m < 0 || L->swz_s < L->swz_b || L->swz_b + L->swz_m + L->swz_s > 62) return LR_ERR_SWIZZLE;
    int top = L->swz_m + L->swz_b;
    if (top >= 62) return LR_ERR_OVERFLOW;
  }
  return LR_OK;
}

int64_t size_of(const lr_layout* L) {
  int64_t s = 1;
  for (int i = 0; i < L->nleaves; ++i) s *= L->shape[i];
  return s;
}

int64_t max_linear_offset(const lr_layout* L) {
  int64_t m = 0;
  for (int i = 0; i < L->nleaves; ++i) m += (L->shape[i] - 1) * L->stride[i];
  return m;
}

int64_t cosize_bound(const lr_layout* L) {
  int64_t m = max_linear_offset(L);
  if (L->swz_b > 0) m |= (int64_t(1) << (L->swz_m + L->swz_b)) - 1;
  return m + 1;
}

static void set_leaves(lr_layout* out, const std::vector<Leaf>& lv, const std::vector<int>& mode_end,
                       int32_t b, int32_t m, int32_t s) {
  std::memset(out, 0, sizeof(*out));
  out->nleaves = (int32_t)lv.size();
  for (size_t i = 0; i < lv.size(); ++i) {
    out->shape[i] = lv[i].n;
    out->stride[i] = lv[i].d;
  }
  out->nmodes = (int32_t)mode_end.size();
  for (size_t i = 0; i < mode_end.size(); ++i) out->mode_end[i] = mode_end[i];
  out->swz_b = b;
  out->swz_m = b ? m : 0;
  out->swz_s = b ? s : 0;
}

// one mode per leaf; an empty list becomes 1:0
static int emit_flat(lr_layout* out, std::vector<Leaf> lv, int32_t b, int32_t m, int32_t s) {
  if (lv.empty()) lv.push_back({1, 0});
  if ((int)lv.size() > LR_MAX_LEAVES) return LR_ERR_NOT_REPRESENTABLE;
  std::vector<int> ends;
  for (size_t i = 0; i < lv.size(); ++i) ends.push_back((int)i + 1);
  set_leaves(out, lv, ends, b, m, s);
  return LR_OK;
}

static std::vector<Leaf> leaves_of(const lr_layout* L, int lo, int hi) {
  std::vector<Leaf> v;
  for (int i = lo; i < hi; ++i) v.push_back({L->shape[i], L->stride[i]});
  return v;
}

static std::vector<Leaf> coalesce_leaves(const std::vector<Leaf>& in) {
  std::vector<Leaf> out;
  for (const Leaf& l : in) {
    if (l.n == 1) continue;
    if (!out.empty()) {
      int64_t want;
      if (mul_ok(out.back().n, out.back().d, &want) && want == l.d) {
        out.back().n *= l.n;
        continue;
      }
    }
    out.push_back(l);
  }
  return out;
}

bool injective(const lr_layout* L) {
  // Leaves of extent > 1 sorted by stride.  A leaf whose stride exceeds the largest
  // offset R of the smaller-stride leaves is separated: its translates of their
  // image lie in the disjoint ranges [c d, c d + R], so it keeps (or breaks)
  // injectivity exactly as the smaller leaves alone do.  The whole layout is
  // therefore injective iff the prefix up to the last leaf that is not separated
  // is, and that prefix is checked exactly over its own offsets (a swizzle is a
  // bijection and changes nothing).  A stride-0 leaf of extent > 1 repeats offsets.
  std::vector<Leaf> lv;
  for (int i = 0; i < L->nleaves; ++i)
    if (L->shape[i] > 1) lv.push_back({L->shape[i], L->stride[i]});
  std::sort(lv.begin(), lv.end(), [](const Leaf& x, const Leaf& y) { return x.d < y.d || (x.d == y.d && x.n < y.n); });
  int last = -1;
  int64_t reach = 0;
  for (int k = 0; k < (int)lv.size(); ++k) {
    if (lv[k].d == 0) return false;
    if (lv[k].d <= reach) last = k;
    reach += (lv[k].n - 1) * lv[k].d;
  }
  if (last < 0) return true;
  int64_t n = 1, cos = 1;
  for (int k = 0; k <= last; ++k) {
    n *= lv[k].n;
    cos += (lv[k].n - 1) * lv[k].d;
    if (n > kExactInjectiveElems) return false;  // not proven
  }
  // the prefix's offsets, by an odometer over its leaves: a bitmap of one bit per
  // offset when the span is at most 2^26 (8 MiB), else sorted
  std::vector<bool> seen;
  std::vector<int64_t> offs;
  const bool bitmap = cos <= (int64_t(1) << 26);
  if (bitmap)
    seen.assign((size_t)cos, false);
  else
    offs.reserve((size_t)n);
  int64_t digit[LR_MAX_LEAVES] = {0}, o = 0;
  for (int64_t k = 0; k < n; ++k) {
    if (bitmap) {
      if (seen[(size_t)o]) return false;
      seen[(size_t)o] = true;
    } else {
      offs.push_back(o);
    }
    for (int j = 0; j <= last; ++j) {
      o += lv[j].d;
      if (++digit[j] < lv[j].n) break;
      o -= lv[j].n * lv[j].d;
      digit[j] = 0;
    }
  }
  if (!bitmap) {
    std::sort(offs.begin(), offs.end());
    return std::adjacent_find(offs.begin(), offs.end()) == offs.end();
  }
  return true;
}

// ---------------------------------------------------------------- composition

// Leaves of k -> A(s*k), k < n, for coalesced A whose last leaf is unbounded.
static bool compose_leaf(const std::vector<Leaf>& A, int64_t n, int64_t s, std::vector<Leaf>* out) {
  if (n == 1) {
    out->push_back({1, 0});
    return true;
  }
  if (s == 0) {
    out->push_back({n, 0});
    return true;
  }
  std::vector<Leaf> a = A.empty() ? std::vector<Leaf>{{1, 0}} : A;
  const int na = (int)a.size();
  // 1) divide s through the leading extents
  int64_t rest = s;
  int i = 0;
  int64_t cur_n = 0, cur_d = 0;  // cur_n == 0: unbounded
  while (true) {
    if (i == na - 1) {
      cur_n = 0;
      if (!mul_ok(a[i].d, rest, &cur_d)) return false;
      break;
    }
    if (rest % a[i].n == 0) {
      rest /= a[i].n;
      ++i;
      continue;
    }
    if (a[i].n % rest == 0) {
      cur_n = a[i].n / rest;
      if (!mul_ok(a[i].d, rest, &cur_d)) return false;
      break;
    }
    return false;
  }
  // 2) take n elements
  int64_t rem = n;
  while (rem > 1) {
    if (cur_n == 0) {
      out->push_back({rem, cur_d});
      rem = 1;
      break;
    }
    if (rem % cur_n == 0) {
      out->push_back({cur_n, cur_d});
      rem /= cur_n;
      ++i;
      if (rem == 1) break;
      cur_n = (i == na - 1) ? 0 : a[i].n;
      cur_d = a[i].d;
      continue;
    }
    if (cur_n % rem == 0) {
      out->push_back({rem, cur_d});
      rem = 1;
      break;
    }
    return false;
  }
  return true;
}

static int compose_impl(const lr_layout* A, const lr_layout* B, lr_layout* out) {
  std::vector<Leaf> a = coalesce_leaves(leaves_of(A, 0, A->nleaves));
  if (B->swz_b > 0) {
    if (A->swz_b == 0 && a.size() == 1 && a[0].d == 1) {
      *out = *B;
      return LR_OK;
    }
    return LR_ERR_NOT_REPRESENTABLE;
  }
  if (a.size() > 1) {
    std::vector<Leaf> nt;
    for (int i = 0; i < B->nleaves; ++i)
      if (B->shape[i] > 1 && B->stride[i] > 0) nt.push_back({B->shape[i], B->stride[i]});
    std::sort(nt.begin(), nt.end(), [](const Leaf& x, const Leaf& y) { return x.d < y.d || (x.d == y.d && x.n < y.n); });
    for (size_t j = 0; j + 1 < nt.size(); ++j) {
      int64_t top;
      if (!mul_ok(nt[j].d, nt[j].n, &top) || top > nt[j + 1].d) return LR_ERR_NOT_REPRESENTABLE;
    }
  }
  std::vector<Leaf> lv;
  std::vector<int> ends;
  int leaf = 0;
  for (int m = 0; m < B->nmodes; ++m) {
    for (; leaf < B->mode_end[m]; ++leaf) {
      if (!compose_leaf(a, B->shape[leaf], B->stride[leaf], &lv)) return LR_ERR_NOT_REPRESENTABLE;
    }
    ends.push_back((int)lv.size());
  }
  if ((int)lv.size() > LR_MAX_LEAVES) return LR_ERR_NOT_REPRESENTABLE;
  set_leaves(out, lv, ends, A->swz_b, A->swz_m, A->swz_s);
  return validate(out) == LR_OK ? LR_OK : LR_ERR_NOT_REPRESENTABLE;
}

// ---------------------------------------------------------------- text form

namespace {

struct Node {
  bool leaf = true;
  int64_t v = 0;
  std::vector<Node> kids;
};

struct Parser {
  const char* p;
  void ws() {
    while (*p && std::isspace((unsigned char)*p)) ++p;
  }
  bool lit(const char* s) {
    ws();
    size_t n = std::strlen(s);
    if (std::strncmp(p, s, n) == 0) {
      p += n;
      return true;
    }
    return false;
  }
  bool integer(int64_t* out) {
    ws();
    if (*p == '_') ++p;
    bool neg = false;
    if (*p == '-') {
      neg = true;
      ++p;
    }
    if (!std::isdigit((unsigned char)*p)) return false;
    int64_t v = 0;
    while (std::isdigit((unsigned char)*p)) {
      if (!mul_ok(v, 10, &v) || !add_ok(v, *p - '0', &v)) return false;
      ++p;
    }
    *out = neg ? -v : v;
    return true;
  }
  bool tuple(Node* n, int depth) {
    if (depth > 32) return false;
    ws();
    if (*p == '(') {
      ++p;
      n->leaf = false;
      do {
        n->kids.emplace_back();
        if (!tuple(&n->kids.back(), depth + 1)) return false;
      } while (lit(","));
      return lit(")");
    }
    n->leaf = true;
    return integer(&n->v);
  }
};

void flatten(const Node& n, std::vector<int64_t>* out) {
  if (n.leaf) {
    out->push_back(n.v);
    return;
  }
  for (const Node& k : n.kids) flatten(k, out);
}

bool congruent(const Node& a, const Node& b) {
  if (a.leaf != b.leaf) return false;
  if (a.leaf) return true;
  if (a.kids.size() != b.kids.size()) return false;
  for (size_t i = 0; i < a.kids.size(); ++i)
    if (!congruent(a.kids[i], b.kids[i])) return false;
  return true;
}

}  // namespace

static int parse_impl(const char* text, lr_layout* out) {
  Parser ps{text};
  int64_t b = 0, m = 0, s = 0;
  ps.ws();
  if (ps.lit("Swizzle") || ps.lit("Sw")) {
    if (!ps.lit("<") || !ps.integer(&b) || !ps.lit(",") || !ps.integer(&m) || !ps.lit(",") ||
        !ps.integer(&s) || !ps.lit(">"))
      return LR_ERR_INVALID;
    if (!ps.lit("o") && !ps.lit("\xE2\x88\x98")) return LR_ERR_INVALID;  // 'o' or U+2218
    if (b < 0 || m < 0 || s < 0 || b > 62 || m > 62 || s > 62) return LR_ERR_SWIZZLE;
  }
  Node sh, st;
  if (!ps.tuple(&sh, 0) || !ps.lit(":") || !ps.tuple(&st, 0)) return LR_ERR_INVALID;
  ps.ws();
  if (*ps.p) return LR_ERR_INVALID;
  if (!congruent(sh, st)) return LR_ERR_INVALID;
  std::vector<int64_t> ns, ds;
  std::vector<int> ends;
  if (sh.leaf) {
    ns.push_back(sh.v);
    ds.push_back(st.v);
    ends.push_back(1);
  } else {
    for (size_t i = 0; i < sh.kids.size(); ++i) {
      flatten(sh.kids[i], &ns);
      flatten(st.kids[i], &ds);
      ends.push_back((int)ns.size());
    }
  }
  if ((int)ns.size() > LR_MAX_LEAVES) return LR_ERR_INVALID;
  std::vector<Leaf> lv;
  for (size_t i = 0; i < ns.size(); ++i) lv.push_back({ns[i], ds[i]});
  set_leaves(out, lv, ends, (int32_t)b, (int32_t)m, (int32_t)s);
  return validate(out);
}

static void put_mode(std::string* o, const int64_t* v, int lo, int hi) {
  if (hi - lo == 1) {
    *o += std::to_string(v[lo]);
    return;
  }
  *o += "(";
  for (int i = lo; i < hi; ++i) {
    if (i > lo) *o += ",";
    *o += std::to_string(v[i]);
  }
  *o += ")";
}

static std::string format_impl(const lr_layout* L) {
  std::string o;
  if (L->swz_b > 0)
    o += "Sw<" + std::to_string(L->swz_b) + "," + std::to_string(L->swz_m) + "," + std::to_string(L->swz_s) + "> o ";
  for (int part = 0; part < 2; ++part) {
    const int64_t* v = part == 0 ? L->shape : L->stride;
    if (part == 1) o += ":";
    if (L->nmodes == 1 && L->nleaves == 1) {
      o += std::to_string(v[0]);
      continue;
    }
    o += "(";
    int lo = 0;
    for (int m = 0; m < L->nmodes; ++m) {
      if (m) o += ",";
      put_mode(&o, v, lo, L->mode_end[m]);
      lo = L->mode_end[m];
    }
    o += ")";
  }
  return o;
}

// ---------------------------------------------------------------- complement,
// logical divide and products ([CuTe algebra page, section 3.2]: tiles and the
// rest; [section 4.1]: a tile repeated over a grid)

// Leaves of the positions A leaves out up to size M (A unswizzled, strides nested).
static int complement_leaves(const lr_layout* A, int64_t M, std::vector<Leaf>* out) {
  std::vector<Leaf> lv;
  for (int i = 0; i < A->nleaves; ++i)
    if (A->shape[i] > 1 && A->stride[i] > 0) lv.push_back({A->shape[i], A->stride[i]});
  std::sort(lv.begin(), lv.end(), [](const Leaf& x, const Leaf& y) { return x.d < y.d || (x.d == y.d && x.n < y.n); });
  std::vector<Leaf> res;
  int64_t cur = 1;
  for (const Leaf& l : lv) {
    if (l.d % cur) return LR_ERR_NOT_REPRESENTABLE;
    res.push_back({l.d / cur, cur});
    if (!mul_ok(l.n, l.d, &cur)) return LR_ERR_OVERFLOW;
  }
  res.push_back({(M + cur - 1) / cur, cur});
  *out = coalesce_leaves(res);
  if (out->empty()) out->push_back({1, 0});
  return LR_OK;
}

// Two top-level modes: all leaves of x, then all leaves of y.
static int concat2(const std::vector<Leaf>& x, const std::vector<Leaf>& y, lr_layout* out) {
  if (x.size() + y.size() > LR_MAX_LEAVES) return LR_ERR_NOT_REPRESENTABLE;
  std::vector<Leaf> all = x;
  all.insert(all.end(), y.begin(), y.end());
  std::vector<int> ends{(int)x.size(), (int)all.size()};
  set_leaves(out, all, ends, 0, 0, 0);
  return LR_OK;
}

static int logical_product_impl(const lr_layout* A, const lr_layout* B, lr_layout* rep) {
  if (A->swz_b > 0 || B->swz_b > 0) return LR_ERR_NOT_REPRESENTABLE;
  int64_t m;
  if (!mul_ok(size_of(A), max_linear_offset(B) + 1, &m)) return LR_ERR_OVERFLOW;
  std::vector<Leaf> c;
  int rc = complement_leaves(A, m, &c);
  if (rc) return rc;
  lr_layout C;
  std::vector<int> ends;
  for (size_t i = 0; i < c.size(); ++i) ends.push_back((int)i + 1);
  set_leaves(&C, c, ends, 0, 0, 0);
  return compose_impl(&C, B, rep);  // B's top-level modes, repeated A's footprint
}

}  // namespace lr

using namespace lr;

// ==================================================================== C ABI

extern "C" {

int lr_layout_validate(const lr_layout* L) { return validate(L); }

int lr_layout_parse(const char* text, lr_layout* out) {
  if (!text || !out) return LR_ERR_INVALID;
  lr_layout tmp;
  int rc = parse_impl(text, &tmp);
  if (rc == LR_OK) *out = tmp;
  return rc;
}

int lr_layout_format(const lr_layout* L, char* buf, size_t cap) {
  int rc = validate(L);
  if (rc) return rc;
  if (!buf) return LR_ERR_INVALID;
  std::string s = format_impl(L);
  if (s.size() + 1 > cap) return LR_ERR_CAPACITY;
  std::memcpy(buf, s.c_str(), s.size() + 1);
  return LR_OK;
}

int lr_size(const lr_layout* L, int64_t* n) {
  int rc = validate(L);
  if (rc) return rc;
  if (!n) return LR_ERR_INVALID;
  *n = size_of(L);
  return LR_OK;
}

int lr_cosize(const lr_layout* L, int64_t* n) {
  int rc = validate(L);
  if (rc) return rc;
  if (!n) return LR_ERR_INVALID;
  *n = cosize_bound(L);
  return LR_OK;
}

int lr_coalesce(const lr_layout* in, lr_layout* out) {
  int rc = validate(in);
  if (rc) return rc;
  if (!out) return LR_ERR_INVALID;
  return emit_flat(out, coalesce_leaves(leaves_of(in, 0, in->nleaves)), in->swz_b, in->swz_m, in->swz_s);
}

int lr_composition(const lr_layout* a, const lr_layout* b, lr_layout* out) {
  int rc = validate(a);
  if (rc) return rc;
  if ((rc = validate(b))) return rc;
  if (!out) return LR_ERR_INVALID;
  lr_layout tmp;
  rc = compose_impl(a, b, &tmp);
  if (rc == LR_OK) *out = tmp;
  return rc;
}

int lr_right_inverse(const lr_layout* in, lr_layout* out) {
  int rc = validate(in);
  if (rc) return rc;
  if (!out) return LR_ERR_INVALID;
  if (in->swz_b > 0) return LR_ERR_NOT_REPRESENTABLE;
  struct Cand {
    int64_t n, d, w;
    bool used;
  };
  std::vector<Cand> c;
  int64_t w = 1;
  for (int i = 0; i < in->nleaves; ++i) {
    if (in->shape[i] > 1 && in->stride[i] != 0) c.push_back({in->shape[i], in->stride[i], w, false});
    w *= in->shape[i];
  }
  std::vector<Leaf> lv;
  int64_t expect = 1;
  while (true) {
    Cand* hit = nullptr;
    for (Cand& x : c)
      if (!x.used && x.d == expect) {
        hit = &x;
        break;
      }
    if (!hit) break;
    hit->used = true;
    lv.push_back({hit->n, hit->w});
    if (!mul_ok(expect, hit->n, &expect)) break;
  }
  return emit_flat(out, lv, 0, 0, 0);
}

int lr_zipped_divide(const lr_layout* in, const int64_t* tiler, int32_t ntiler, lr_layout* out) {
  int rc = validate(in);
  if (rc) return rc;
  if (!out || ntiler < 0 || ntiler > in->nmodes || (ntiler > 0 && !tiler)) return LR_ERR_INVALID;
  std::vector<Leaf> tiles, rests;
  int lo = 0;
  for (int m = 0; m < in->nmodes; ++m) {
    lr_layout mode;
    std::vector<Leaf> lv = leaves_of(in, lo, in->mode_end[m]);
    std::vector<int> ends{(int)lv.size()};
    set_leaves(&mode, lv, ends, 0, 0, 0);
    lo = in->mode_end[m];
    int64_t n = size_of(&mode);
    int64_t t = m < ntiler ? tiler[m] : 1;
    if (t < 1 || n % t) return LR_ERR_NOT_REPRESENTABLE;
    lr_layout bt, br, rt, rr;
    std::vector<Leaf> l1{{t, 1}}, l2{{n / t, t}};
    std::vector<int> e1{1};
    set_leaves(&bt, l1, e1, 0, 0, 0);
    set_leaves(&br, l2, e1, 0, 0, 0);
    if ((rc = compose_impl(&mode, &bt, &rt))) return rc;
    if ((rc = compose_impl(&mode, &br, &rr))) return rc;
    for (int i = 0; i < rt.nleaves; ++i) tiles.push_back({rt.shape[i], rt.stride[i]});
    for (int i = 0; i < rr.nleaves; ++i) rests.push_back({rr.shape[i], rr.stride[i]});
  }
  std::vector<Leaf> all = tiles;
  all.insert(all.end(), rests.begin(), rests.end());
  if ((int)all.size() > LR_MAX_LEAVES) return LR_ERR_NOT_REPRESENTABLE;
  std::vector<int> ends{(int)tiles.size(), (int)all.size()};
  set_leaves(out, all, ends, in->swz_b, in->swz_m, in->swz_s);
  return LR_OK;
}

int lr_slice(const lr_layout* L, const int64_t* coord, int32_t ncoord, lr_layout* out, int64_t* offset) {
  int rc = validate(L);
  if (rc) return rc;
  if (!coord || !out || !offset) return LR_ERR_INVALID;
  if (ncoord != L->nmodes && ncoord != L->nleaves) return LR_ERR_INVALID;
  const bool per_mode = ncoord == L->nmodes;  // the same reading when every mode is one leaf
  std::vector<Leaf> kept;
  std::vector<int> ends;
  int64_t off = 0;
  int lo = 0;
  for (int m = 0; m < L->nmodes; ++m) {
    const int hi = L->mode_end[m];
    bool any = false;
    if (per_mode && coord[m] == -1) {
      for (int i = lo; i < hi; ++i) kept.push_back({L->shape[i], L->stride[i]});
      any = true;
    } else if (per_mode) {
      // one integer for the whole mode, split colexicographically over its leaves
      int64_t c = coord[m], size = 1;
      for (int i = lo; i < hi; ++i) size *= L->shape[i];
      if (c < 0 || c >= size) return LR_ERR_INVALID;
      for (int i = lo; i < hi; ++i) {
        off += (c % L->shape[i]) * L->stride[i];
        c /= L->shape[i];
      }
    } else {
      for (int i = lo; i < hi; ++i) {
        if (coord[i] == -1) {
          kept.push_back({L->shape[i], L->stride[i]});
          any = true;
        } else if (coord[i] < 0 || coord[i] >= L->shape[i]) {
          return LR_ERR_INVALID;
        } else {
          off += coord[i] * L->stride[i];
        }
      }
    }
    if (any) ends.push_back((int)kept.size());
    lo = hi;
  }
  if (kept.empty()) {
    kept.push_back({1, 0});
    ends.push_back(1);
  } else if (ends.size() == 1) {
    // one mode survives: its leaves are the result's modes (tile (3,5) of the
    // zipped_divide is a 4 x 8 layout of its own)
    ends.clear();
    for (size_t i = 0; i < kept.size(); ++i) ends.push_back((int)i + 1);
  }
  // The swizzle reads bits [M+S, M+S+B) and rewrites bits [M, M+B) of the whole
  // offset; a base that is a multiple of 2^(M+S+B) leaves all of them to the kept
  // part, so Sw(base + o) = base + Sw(o).  Any other base: not a layout plus offset.
  if (L->swz_b > 0 && off % (int64_t(1) << (L->swz_m + L->swz_s + L->swz_b)) != 0)
    return LR_ERR_NOT_REPRESENTABLE;
  set_leaves(out, kept, ends, L->swz_b, L->swz_m, L->swz_s);
  *offset = off;
  return LR_OK;
}

int lr_complement(const lr_layout* A, int64_t M, lr_layout* out) {
  int rc = validate(A);
  if (rc) return rc;
  if (!out || M < 1) return LR_ERR_INVALID;
  if (A->swz_b > 0) return LR_ERR_NOT_REPRESENTABLE;
  std::vector<Leaf> c;
  if ((rc = complement_leaves(A, M, &c))) return rc;
  return emit_flat(out, c, 0, 0, 0);
}

int lr_logical_divide(const lr_layout* A, const lr_layout* B, lr_layout* out) {
  int rc;
  if ((rc = validate(A)) || (rc = validate(B))) return rc;
  if (!out) return LR_ERR_INVALID;
  if (B->swz_b > 0) return LR_ERR_NOT_REPRESENTABLE;
  std::vector<Leaf> c;
  if ((rc = complement_leaves(B, size_of(A), &c))) return rc;
  lr_layout D;
  if ((rc = concat2(leaves_of(B, 0, B->nleaves), c, &D))) return rc;
  lr_layout tmp;
  if ((rc = compose_impl(A, &D, &tmp))) return rc;
  *out = tmp;
  return LR_OK;
}

int lr_logical_product(const lr_layout* A, const lr_layout* B, lr_layout* out) {
  int rc;
  if ((rc = validate(A)) || (rc = validate(B))) return rc;
  if (!out) return LR_ERR_INVALID;
  lr_layout rep;
  if ((rc = logical_product_impl(A, B, &rep))) return rc;
  lr_layout tmp;
  if ((rc = concat2(leaves_of(A, 0, A->nleaves), leaves_of(&rep, 0, rep.nleaves), &tmp))) return rc;
  *out = tmp;
  return LR_OK;
}

int lr_blocked_product(const lr_layout* A, const lr_layout* B, lr_layout* out) {
  int rc;
  if ((rc = validate(A)) || (rc = validate(B))) return rc;
  if (!out || A->nmodes != B->nmodes) return LR_ERR_INVALID;
  lr_layout rep;
  if ((rc = logical_product_impl(A, B, &rep))) return rc;
  if (A->nleaves + rep.nleaves > LR_MAX_LEAVES) return LR_ERR_NOT_REPRESENTABLE;
  std::vector<Leaf> all;
  std::vector<int> ends;
  int la = 0, lb = 0;
  for (int m = 0; m < A->nmodes; ++m) {  // mode m: A's mode m, then the repeats' mode m
    for (; la < A->mode_end[m]; ++la) all.push_back({A->shape[la], A->stride[la]});
    for (; lb < rep.mode_end[m]; ++lb) all.push_back({rep.shape[lb], rep.stride[lb]});
    ends.push_back((int)all.size());
  }
  lr_layout tmp;
  set_leaves(&tmp, all, ends, 0, 0, 0);
  *out = tmp;
  return LR_OK;
}

int lr_is_injective(const lr_layout* L, int32_t* result) {
  int rc = validate(L);
  if (rc) return rc;
  if (!result) return LR_ERR_INVALID;
  *result = injective(L) ? 1 : 0;
  return LR_OK;
}

int lr_thread_map(int64_t pitch, int64_t strips, int64_t krow, int64_t threads, lr_layout* out) {
  if (!out || pitch < 1 || strips < 0 || krow < 0 || threads < 1) return LR_ERR_INVALID;
  std::vector<Leaf> lv;
  if (strips == 0) {
    lv = {{pitch, 1}, {(threads + pitch - 1) / pitch, krow}};
  } else {
    int64_t ps, jump;
    if (!mul_ok(pitch, strips, &ps) || !mul_ok(ps, krow, &jump)) return LR_ERR_OVERFLOW;
    lv = {{pitch, 1}, {strips, krow}, {(threads + ps - 1) / ps, jump}};
  }
  std::vector<int> ends;
  for (size_t i = 0; i < lv.size(); ++i) ends.push_back((int)i + 1);
  lr_layout tmp;
  set_leaves(&tmp, lv, ends, 0, 0, 0);
  int rc = validate(&tmp);
  if (rc == LR_OK) *out = tmp;
  return rc;
}

const char* lr_strerror(int code) {
  switch (code) {
    case LR_OK: return "ok";
    case LR_ERR_INVALID: return "invalid argument";
    case LR_ERR_SIZE_MISMATCH: return "layout sizes differ";
    case LR_ERR_BOUNDS: return "layout reaches beyond its buffer";
    case LR_ERR_OVERFLOW: return "size or offset overflows int64";
    case LR_ERR_ALIAS: return "destination layout is not injective (or beyond the ordered-alias limits)";
    case LR_ERR_NOT_REPRESENTABLE: return "result is not representable as a layout";
    case LR_ERR_SWIZZLE: return "invalid swizzle parameters";
    case LR_ERR_ELEM_BYTES: return "elem_bytes must be 1, 2, 4, 8 or 16";
    case LR_ERR_HIP: return "HIP runtime error";
    case LR_ERR_PATH: return "forced copy path does not apply";
    case LR_ERR_OVERLAP: return "source and destination storage overlap";
    case LR_ERR_CAPACITY: return "output buffer too small";
    default: return "unknown status";
  }
}

const char* lr_version(void) { return "0.1.0"; }

}  // extern "C"
