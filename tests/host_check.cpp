// Host-only checks of the library's C++ sources (built with g++, no HIP):
//   host_check fastdiv  -- the multiply-high division constants are exact
//   host_check fuzz     -- random walk through the host algebra (run under
//                          AddressSanitizer/UBSan by the test suite)
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "layout_remap.h"
#include "lr_internal.h"

static inline uint32_t qdiv(uint32_t x, lr::FastDiv f) {
  if (f.m == 0) return x;
  uint32_t hi = (uint32_t)(((uint64_t)x * f.m) >> 32);
  return hi >> f.s;
}

static int check_div(uint32_t d, uint32_t x, lr::FastDiv f) {
  if (qdiv(x, f) != x / d) {
    std::printf("fastdiv mismatch d=%u x=%u got=%u want=%u\n", d, x, qdiv(x, f), x / d);
    return 1;
  }
  return 0;
}

static int run_fastdiv() {
  const uint32_t lim = 0x80000000u;  // dividends below 2^31
  // exhaustive for a few divisors
  for (uint32_t d : {3u, 7u, 3136u, 0x7FFFFFFFu}) {
    lr::FastDiv f = lr::make_fastdiv(d);
    for (uint32_t x = 0; x < lim; ++x)
      if (qdiv(x, f) != x / d) return check_div(d, x, f);
  }
  // every quotient boundary (up to 2^17 quotients), the top of the range and
  // random dividends for many more divisors
  std::vector<uint32_t> ds;
  for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
  for (int k = 12; k < 31; ++k) {
    ds.push_back(1u << k);
    ds.push_back((1u << k) - 1);
    ds.push_back((1u << k) + 1);
  }
  for (uint32_t d : {3136u, 802816u, 524288u, 1048576u, 16777216u, 14336u, 100352u, 65535u, 65537u}) ds.push_back(d);
  std::mt19937_64 rng(12345);
  for (int i = 0; i < 2000; ++i) ds.push_back(1 + (uint32_t)(rng() % 0x7FFFFFFFu));
  for (uint32_t d : ds) {
    lr::FastDiv f = lr::make_fastdiv(d);
    uint64_t qmax = (lim - 1) / d;
    uint64_t step = qmax > 131072 ? qmax / 131072 : 1;
    for (uint64_t q = 0; q <= qmax; q += step) {
      uint64_t x0 = q * d;
      for (uint64_t x : {x0, x0 + d - 1, x0 ? x0 - 1 : 0})
        if (x < lim && check_div(d, (uint32_t)x, f)) return 1;
    }
    for (uint32_t x = lim - 4096; x < lim; ++x)
      if (check_div(d, x, f)) return 1;
    for (int r = 0; r < 2000; ++r)
      if (check_div(d, (uint32_t)(rng() % lim), f)) return 1;
  }
  std::printf("fastdiv ok (%zu divisors)\n", ds.size());
  return 0;
}

static std::string rand_layout(std::mt19937_64& rng, bool swz) {
  int nl = 1 + (int)(rng() % 6);
  std::vector<int> ext(nl), st(nl);
  for (int i = 0; i < nl; ++i) {
    ext[i] = 1 + (int)(rng() % 6);
    st[i] = (int)(rng() % 40);
  }
  std::string s = "(", d = "(";
  int i = 0;
  bool first = true;
  while (i < nl) {
    int j = i + 1 + (int)(rng() % (nl - i));
    if (!first) {
      s += ",";
      d += ",";
    }
    first = false;
    if (j - i == 1) {
      s += std::to_string(ext[i]);
      d += std::to_string(st[i]);
    } else {
      s += "(";
      d += "(";
      for (int k = i; k < j; ++k) {
        if (k > i) {
          s += ",";
          d += ",";
        }
        s += std::to_string(ext[k]);
        d += std::to_string(st[k]);
      }
      s += ")";
      d += ")";
    }
    i = j;
  }
  std::string out = s + "):" + d + ")";
  if (swz && rng() % 3 == 0) {
    int b = 1 + (int)(rng() % 3);
    out = "Sw<" + std::to_string(b) + "," + std::to_string(rng() % 4) + "," + std::to_string(b + rng() % 3) + "> o " +
          out;
  }
  return out;
}

// A random lr_copy_tuning: every field at one of its valid values or -1.
static lr_copy_tuning rand_tuning(std::mt19937_64& rng) {
  lr_copy_tuning t;
  lr_copy_tuning_init(&t);
  auto pick = [&](std::initializer_list<int32_t> v) { return *(v.begin() + rng() % v.size()); };
  t.load_policy = pick({-1, 0, 2});
  t.store_policy = pick({-1, 0, 2, 18});
  t.units_per_lane = pick({-1, 1, 4});
  t.vector_order = pick({-1, 0, 1, 2, 3});
  t.interleave_form = pick({-1, 0, 1, 2});
  t.tile_shape = pick({-1, 0, 1, 2, 3, 4, 5, 6, 7, 8});
  t.tile_order = pick({-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9});
  t.element_tiles = pick({-1, 0, 1});
  t.direct_loads = pick({-1, 0, 1});
  t.gather_chunks = pick({-1, 1, 2, 4, 8, 16, 32});
  t.pipeline_tiles = pick({-1, 0, 2, 3, 5, 64});
  t.transpose_reads = pick({-1, 0, 1});
  t.chunk_bytes = pick({-1, 8, 16});
  t.batch_swizzle = pick({-1, 0, 3, 7, 15});
  t.batch_order = pick({-1, 0, 1});
  t.workgroup_lanes = pick({-1, 64, 128, 256});
  t.transpose_blocks = pick({-1, 1, 2});
  return t;
}

// Plans a copy with the given overrides; a plan the planner accepts must pass its own
// invariant check (the check every launch runs).
static bool tuned_plan_ok(const lr_layout* a, int64_t cap_a, size_t align_a, const lr_layout* b, int64_t cap_b,
                          size_t align_b, int eb, uint32_t fl, const lr_copy_tuning& t) {
  lr::Plan p;
  if (lr::plan_copy(a, cap_a, align_a, b, cap_b, align_b, eb, fl, &t, &p) != LR_OK) return true;
  return lr::verify_plan(p, cap_a, cap_b) == LR_OK;
}

// A tiled pair: an atom of w elements continued by mode a in the source and by mode
// b in the destination, a batch mode, padding on either side, sometimes a swizzle
// that keeps 16-byte chunks (the structure of the vector path's tiles of atoms).
static void rand_atom_pair(std::mt19937_64& rng, int eb, lr_layout* s, lr_layout* d) {
  const int64_t w = (int64_t)((16 << (rng() % 6)) / eb), A = 1 + (int64_t)(rng() % 40), B = 1 + (int64_t)(rng() % 40),
                C = 1 + (int64_t)(rng() % 3);
  const int64_t pa = (rng() % 3 == 0) ? (int64_t)(16 / eb) * (int64_t)(rng() % 3) : 0;
  const int64_t pb = (rng() % 3 == 0) ? (int64_t)(16 / eb) * (int64_t)(rng() % 3) : 0;
  std::memset(s, 0, sizeof(*s));
  s->nleaves = s->nmodes = 4;
  const int64_t shape[4] = {w, A, B, C};
  for (int i = 0; i < 4; ++i) {
    s->shape[i] = shape[i];
    s->mode_end[i] = i + 1;
  }
  *d = *s;
  s->stride[0] = 1;
  s->stride[1] = w;
  s->stride[2] = w * A + pa;
  s->stride[3] = (w * A + pa) * B;
  d->stride[0] = 1;
  d->stride[2] = w;
  d->stride[1] = w * B + pb;
  d->stride[3] = (w * B + pb) * A;
  if (rng() % 4 == 0 && w * eb >= 64) {  // Sw<B,M,S> with M at least the 16-byte chunk
    d->swz_b = 1 + (int)(rng() % 2);
    d->swz_m = 4 - (eb >= 16 ? 4 : eb >= 8 ? 3 : eb >= 4 ? 2 : eb >= 2 ? 1 : 0) + (int)(rng() % 2);
    d->swz_s = d->swz_b + 1 + (int)(rng() % 3);
  }
}

static int run_fuzz() {
  std::mt19937_64 rng(777);
  char buf[1024];
  int n_ok = 0;
  for (int it = 0; it < 20000; ++it) {
    std::string ta = rand_layout(rng, true), tb = rand_layout(rng, true);
    lr_layout a, b, r;
    if (lr_layout_parse(ta.c_str(), &a) || lr_layout_parse(tb.c_str(), &b)) {
      std::printf("parse failed: %s / %s\n", ta.c_str(), tb.c_str());
      return 1;
    }
    if (lr_layout_format(&a, buf, sizeof(buf))) return 1;
    lr_layout a2;
    if (lr_layout_parse(buf, &a2) || std::memcmp(&a, &a2, sizeof(a)) != 0) {
      std::printf("round trip failed: %s -> %s\n", ta.c_str(), buf);
      return 1;
    }
    int64_t n;
    lr_size(&a, &n);
    lr_cosize(&a, &n);
    lr_coalesce(&a, &r);
    lr_composition(&a, &b, &r);
    lr_right_inverse(&a, &r);
    int64_t tiler[2] = {1 + (int64_t)(rng() % 4), 1 + (int64_t)(rng() % 4)};
    lr_zipped_divide(&a, tiler, a.nmodes < 2 ? a.nmodes : 2, &r);
    int32_t inj;
    lr_is_injective(&a, &inj);
    lr_complement(&a, 1 + (int64_t)(rng() % 100), &r);
    lr_logical_divide(&a, &b, &r);
    lr_logical_product(&a, &b, &r);
    lr_blocked_product(&a, &b, &r);
    int64_t v;
    lr_max_common_vector(&a, &b, 4, &v);
    {
      static char text[1 << 16];
      size_t need = 0;
      lr_layout_print(&a, text, sizeof(text), &need);
      lr_layout_print(&a, nullptr, 0, &need);
      lr_layout_print_table(&a, 1 + (int64_t)(rng() % 70), text, sizeof(text), &need);
      lr_access_report rep;
      for (int eb : {1, 2, 4, 8, 16})
        lr_access_check(&a, eb, 1 + (int)(rng() % 64), (int)(rng() % 4), (int)(rng() % 3) * 32,
                        (int)(rng() % 3) * 16, (int)(rng() % 3) * 64, &rep);
    }
    lr_plan p;
    // a compact destination over a's extents in a random order: a bijective copy
    lr_layout c = a;
    c.swz_b = 0;
    {
      int perm[LR_MAX_LEAVES];
      for (int i = 0; i < a.nleaves; ++i) perm[i] = i;
      for (int i = a.nleaves - 1; i > 0; --i) std::swap(perm[i], perm[rng() % (i + 1)]);
      int64_t w = 1;
      for (int i = 0; i < a.nleaves; ++i) {
        c.stride[perm[i]] = w;
        w *= a.shape[perm[i]];
      }
    }
    for (uint32_t fl : {0u, 1u, 2u}) {
      for (int eb : {1, 2, 4, 8, 16}) {
        // the planner's own choice must always pass its invariant check
        if (lr_copy_plan(&a, 1 << 20, 16, &b, 1 << 20, 16, eb, fl, &p) == LR_ERR_PATH ||
            lr_copy_plan(&a, 1 << 20, 4, &a, 1 << 20, 8, eb, fl, &p) == LR_ERR_PATH ||
            lr_copy_plan(&a, 1 << 20, 16, &c, 1 << 20, 16, eb, fl, &p) == LR_ERR_PATH ||
            lr_copy_plan(&c, 1 << 20, 16, &a, 1 << 20, 16, eb, fl, &p) == LR_ERR_PATH) {
          std::printf("planner chose a path its check rejects: %s -> %s eb=%d\n", ta.c_str(), tb.c_str(), eb);
          return 1;
        }
      }
    }
    for (int path = 0; path < 8; ++path) lr_copy_plan(&a, 1 << 20, 16, &a, 1 << 20, 16, 1, LR_COPY_FORCE_PATH(path), &p);
    // random overrides
    for (int k = 0; k < 4; ++k) {
      const lr_copy_tuning t = rand_tuning(rng);
      const int eb = 1 << (rng() % 5);
      const uint32_t fl = (uint32_t)(rng() % 3);
      if (!tuned_plan_ok(&a, 1 << 20, 16, &c, 1 << 20, 16, eb, fl, t) ||
          !tuned_plan_ok(&c, 1 << 20, 16, &a, 1 << 20, 16, eb, fl, t) ||
          !tuned_plan_ok(&a, 1 << 20, 16, &b, 1 << 20, 16, eb, fl, t)) {
        std::printf("a tuned plan fails its check: %s -> %s eb=%d\n", ta.c_str(), tb.c_str(), eb);
        return 1;
      }
    }
    ++n_ok;
  }
  // tiled pairs (tiles of atoms where they apply) under random overrides
  int atoms = 0;
  for (int it = 0; it < 20000; ++it) {
    const int eb = 1 << (rng() % 5);
    lr_layout s, d;
    rand_atom_pair(rng, eb, &s, &d);
    int64_t cs, cd;
    lr_cosize(&s, &cs);
    lr_cosize(&d, &cd);
    const lr_copy_tuning t = rand_tuning(rng);
    lr::Plan p;
    const int rc = lr::plan_copy(&s, cs, 16, &d, cd, 16, eb, 0, (it % 2) ? &t : nullptr, &p);
    if (rc == LR_OK) {
      if (lr::verify_plan(p, cs, cd) != LR_OK) {
        std::printf("tiled pair: plan fails its check (eb=%d w=%lld)\n", eb, (long long)s.shape[0]);
        return 1;
      }
      atoms += p.vorder == 3;
    }
  }
  if (atoms < 1000) {
    std::printf("tiled pairs: only %d took tiles of atoms\n", atoms);
    return 1;
  }
  // copies too large for 32-bit offsets: the blocks cover every index once and fit
  for (int it = 0; it < 3000; ++it) {
    int nl = 1 + (int)(rng() % 4);
    lr_layout a, b;
    std::memset(&a, 0, sizeof(a));
    a.nleaves = a.nmodes = nl;
    int64_t n = 1;
    for (int i = 0; i < nl; ++i) {
      a.shape[i] = 1 + (int64_t)(rng() % (1u << (8 + rng() % 16)));
      if (n > (int64_t(1) << 40) / a.shape[i]) a.shape[i] = 1;
      n *= a.shape[i];
      a.mode_end[i] = i + 1;
    }
    // source: compact in a random order, sometimes padded; destination: compact
    int perm[LR_MAX_LEAVES];
    for (int i = 0; i < nl; ++i) perm[i] = i;
    for (int i = nl - 1; i > 0; --i) std::swap(perm[i], perm[rng() % (i + 1)]);
    b = a;
    int64_t w = 1, wd = 1;
    for (int i = 0; i < nl; ++i) {
      a.stride[perm[i]] = w;
      w *= a.shape[perm[i]] + (rng() % 4 == 0 ? (int64_t)(rng() % 5) : 0);
      b.stride[i] = wd;
      wd *= b.shape[i];
    }
    lr::Plan p;
    if (lr::plan_copy(&a, w, 16, &b, wd, 16, 2, 0, nullptr, &p) != LR_OK) continue;
    int64_t cext[lr::kMaxJoint], nb = 0;
    if (!lr::block_extents(p, 0, cext, &nb)) continue;
    int64_t start[lr::kMaxJoint] = {0}, covered = 0;
    for (int64_t k = 0; k < nb; ++k) {
      lr_layout ls, ld;
      int64_t os, od;
      lr::make_block(p, cext, start, &ls, &ld, &os, &od);
      int64_t bn = 1;
      for (int i = 0; i < ls.nleaves; ++i) bn *= ls.shape[i];
      lr::Plan pb;
      if (bn >= (int64_t(1) << 31) || lr::cosize_bound(&ls) >= (int64_t(1) << 31) ||
          lr::cosize_bound(&ld) >= (int64_t(1) << 31) || os + lr::cosize_bound(&ls) > w ||
          od + lr::cosize_bound(&ld) > wd ||
          lr::plan_copy(&ls, lr::cosize_bound(&ls), 16, &ld, lr::cosize_bound(&ld), 16, 2, 0, nullptr, &pb) != LR_OK ||
          pb.wide || lr::verify_plan(pb, lr::cosize_bound(&ls), lr::cosize_bound(&ld)) != LR_OK) {
        std::printf("bad block %lld of %lld\n", (long long)k, (long long)nb);
        return 1;
      }
      covered += bn;
      for (int i = 0; i < p.rank; ++i) {
        start[i] += cext[i];
        if (start[i] < p.m[i].ext) break;
        start[i] = 0;
      }
    }
    if (covered != n) {
      std::printf("blocks cover %lld of %lld\n", (long long)covered, (long long)n);
      return 1;
    }
    ++n_ok;
  }
  // malformed and adversarial descriptors
  const char* bad[] = {"", "(", "()", "(1,2):(3)", "Sw<1,2> o 4:1", "((((((((((((((((((((((((((((((((((4))))))))))"
                       "))))))))))))))))))))))):1", "99999999999999999999:1", "(4,2):(1,2) trailing", "Sw<70,0,80> o 4:1"};
  lr_layout x;
  for (const char* t : bad) lr_layout_parse(t, &x);
  std::memset(&x, 0, sizeof(x));
  x.nleaves = 17;
  lr_layout_validate(&x);
  x.nleaves = 2;
  x.nmodes = 1;
  x.mode_end[0] = 2;
  x.shape[0] = x.shape[1] = int64_t(1) << 40;
  x.stride[0] = 1;
  x.stride[1] = int64_t(1) << 40;
  if (lr_layout_validate(&x) != LR_ERR_OVERFLOW) return 1;
  std::printf("fuzz ok (%d; %d tiled pairs on tiles of atoms)\n", n_ok, atoms);
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "fastdiv") == 0) return run_fastdiv();
  if (argc > 1 && std::strcmp(argv[1], "fuzz") == 0) return run_fuzz();
  std::printf("usage: host_check fastdiv|fuzz\n");
  return 2;
}
