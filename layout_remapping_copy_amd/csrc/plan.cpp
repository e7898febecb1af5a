// Copy planner: joint flat form of the two layouts, the common vector width,
// path selection and launch shapes.  Host only.
//
// The copy is dst[Ld(k)] = src[Ls(k)] for every index k ([CuTe algebra page,
// jsqmd.com/news/768714, sections 2.3 and 5.1]).  For an injective Ld the order of
// k is free, so the planner rewrites the pair of layouts as one list of joint
// modes (extent, src stride, dst stride), sorted by dst stride, and picks a
// kernel from the shape of that list:
//   * the first mode contiguous on both sides  -> 16-byte vectors along it;
//   * contiguous modes differ, the dst one short -> in-register interleave;
//   * contiguous modes differ                    -> register-blocked tile transpose;
//   * small compact source footprints per tile   -> footprint staged in LDS;
//   * anything else                               -> one unit per lane.
// [CuTe algebra page, section 2.3] motivates the first rule (the common part of
// the inverse layouts gives the widest copy); [print_layout page, sections 5.1
// and 5.2] the other two (adjacent lanes on adjacent addresses, bank-spread
// staging).

#include <algorithm>
#include <array>
#include <cstring>
#include <initializer_list>
#include <unordered_map>
#include <vector>

#include "lr_internal.h"

namespace lr {

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{0, 0};
  if (d <= 1) return f;
  int l = 0;
  while ((uint64_t(1) << l) < d) ++l;  // l = ceil(log2 d), 1..31
  uint64_t p = uint64_t(1) << (31 + l);
  uint64_t m = (p + d - 1) / d;  // ceil(2^(31+l)/d) < 2^32
  f.m = (uint32_t)m;
  f.s = (uint32_t)(l - 1);
  return f;
}

static bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
static int log2i(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

bool joint_flat(const lr_layout* s, const lr_layout* d, JMode* out, int* rank, bool sort_by_dst) {
  Leaf a[LR_MAX_LEAVES], b[LR_MAX_LEAVES];
  int na = 0, nb = 0;
  for (int i = 0; i < s->nleaves; ++i)
    if (s->shape[i] > 1) a[na++] = {s->shape[i], s->stride[i]};
  for (int i = 0; i < d->nleaves; ++i)
    if (d->shape[i] > 1) b[nb++] = {d->shape[i], d->stride[i]};
  int r = 0;
  int i = 0, j = 0;
  int64_t pa = 1, pb = 1, pos = 1;  // pa/pb: start of current leaf; pos: current cut
  while (i < na && j < nb) {
    int64_t ea = pa * a[i].n, eb = pb * b[j].n;
    int64_t nxt = std::min(ea, eb);
    if (nxt % pos) return false;
    out[r].ext = nxt / pos;
    out[r].ss = a[i].d * (pos / pa);
    out[r].sd = b[j].d * (pos / pb);
    ++r;
    pos = nxt;
    if (nxt == ea) {
      pa = ea;
      ++i;
    }
    if (nxt == eb) {
      pb = eb;
      ++j;
    }
  }
  if (i != na || j != nb) return false;  // sizes differ (checked by the caller)
  auto merge = [](JMode* m, int n) {
    int w = 0;
    for (int k = 0; k < n; ++k) {
      if (m[k].ext == 1) continue;
      if (w > 0 && m[k].ss == m[w - 1].ext * m[w - 1].ss && m[k].sd == m[w - 1].ext * m[w - 1].sd) {
        m[w - 1].ext *= m[k].ext;
        continue;
      }
      m[w++] = m[k];
    }
    return w;
  };
  r = merge(out, r);
  if (sort_by_dst) {
    while (true) {
      JMode tmp[kMaxJoint];
      std::memcpy(tmp, out, sizeof(JMode) * r);
      std::stable_sort(tmp, tmp + r, [](const JMode& x, const JMode& y) {
        return x.sd < y.sd || (x.sd == y.sd && x.ss < y.ss);
      });
      int r2 = merge(tmp, r);
      bool same = r2 == r && std::memcmp(tmp, out, sizeof(JMode) * r) == 0;
      std::memcpy(out, tmp, sizeof(JMode) * r2);
      r = r2;
      if (same) break;
    }
  }
  *rank = r;
  return true;
}

// largest power of two v with v | x (x > 0)
static int64_t pow2_divisor(int64_t x) { return x & (-x); }

static bool swz_keeps(const Swz& z, int64_t v) { return z.b == 0 || (int64_t(1) << z.m) >= v; }

// Largest unit (power of two elements, unit*eb <= 16) for the generic/vector kernel.
static int64_t unit_width(const Plan& p, size_t align_s, size_t align_d) {
  if (p.rank == 0 || p.m[0].ss != 1 || p.m[0].sd != 1) return 1;
  int64_t v = std::min<int64_t>(16 / p.eb, pow2_divisor(p.m[0].ext));
  for (int k = 1; k < p.rank; ++k) {
    if (p.m[k].ss) v = std::min(v, pow2_divisor(p.m[k].ss));
    if (p.m[k].sd) v = std::min(v, pow2_divisor(p.m[k].sd));
  }
  while (v > 1 && (!swz_keeps(p.sw_s, v) || !swz_keeps(p.sw_d, v) || (align_s % (size_t)(v * p.eb)) ||
                   (align_d % (size_t)(v * p.eb))))
    v >>= 1;
  return v;
}

// An override of lr_copy_tuning, or the planner's own choice when it is -1.
static int32_t knob(int32_t v, int32_t dflt) { return v < 0 ? dflt : v; }

static bool tuning_valid(const lr_copy_tuning& t) {
  auto in = [](int32_t v, std::initializer_list<int32_t> ok) {
    if (v == -1) return true;
    for (int32_t o : ok)
      if (v == o) return true;
    return false;
  };
  if (!in(t.load_policy, {0, 2}) || !in(t.store_policy, {0, 2, 18}) || !in(t.units_per_lane, {1, 4}) ||
      !in(t.vector_order, {0, 1, 2, 3}) || !in(t.interleave_form, {0, 1, 2}) ||
      !in(t.tile_shape, {0, 1, 2, 3, 4, 5, 6, 7, 8}) || !in(t.tile_order, {0, 1, 2, 3, 4, 5, 6, 7, 8, 9}) ||
      !in(t.element_tiles, {0, 1}) || !in(t.direct_loads, {0, 1}) || !in(t.gather_chunks, {1, 2, 4, 8, 16, 32}))
    return false;
  if (t.pipeline_tiles != -1 && (t.pipeline_tiles < 0 || t.pipeline_tiles == 1 || t.pipeline_tiles > 64)) return false;
  if (!in(t.transpose_reads, {0, 1})) return false;
  if (!in(t.chunk_bytes, {8, 16})) return false;
  if (t.batch_swizzle != -1 && (t.batch_swizzle < 0 || t.batch_swizzle > 15)) return false;
  if (!in(t.batch_order, {0, 1})) return false;
  if (!in(t.workgroup_lanes, {64, 128, 256})) return false;
  if (!in(t.transpose_blocks, {1, 2})) return false;
  return true;
}

// One past the highest destination byte the joint modes reach (a destination
// swizzle changes only the bits under 2^(M+B)).
static int64_t dst_span_bytes(const Plan& p) {
  int64_t md = 0;
  for (int k = 0; k < p.rank; ++k) md += (p.m[k].ext - 1) * p.m[k].sd;
  if (p.sw_d.b) md |= (int64_t(1) << (p.sw_d.m + p.sw_d.b)) - 1;
  return (md + 1) * p.eb;
}

// The element-granular channel shuffle (few channels whose planes have no whole
// 16-byte chunks: odd image sizes, unaligned strides): `interleave` planes -> pixels
// (a: the pixel mode, b: the channel mode), else pixels -> planes (a: channels, b:
// pixels).  False when the layouts are not of that form.
static bool plan_chan_elements(Plan* p, int a, int b, bool interleave, size_t src_align, size_t dst_align) {
  if (a < 0 || b < 0 || a == b || p->sw_s.b || p->sw_d.b) return false;
  const int pm = interleave ? a : b, cm = interleave ? b : a;
  const int64_t C = p->m[cm].ext;
  const bool form = interleave ? p->m[a].sd == C : p->m[b].ss == C;
  // element-aligned buffers: the kernel splits each range at 16-byte boundaries
  if (!chan_supported(p->eb, C) || !form || src_align % (size_t)p->eb || dst_align % (size_t)p->eb) return false;
  p->path = interleave ? LR_PATH_INTERLEAVE : LR_PATH_DEINTERLEAVE;
  p->a = a;
  p->b = b;
  p->v = 1;
  p->inarrow = interleave ? 3 : 0;
  p->tile_a = chan_el_pixels(p->eb);
  p->tile_b = C;
  int64_t batch = 1;
  for (int k = 0; k < p->rank; ++k)
    if (k != a && k != b) batch *= p->m[k].ext;
  p->grid = ((p->m[pm].ext + p->tile_a - 1) / p->tile_a) * batch;
  // Its ranges start unaligned, so their partial lines at both ends merge in the
  // cache under ordinary accesses: streaming only from the 256 MiB last-level cache
  // size (source plus destination), unless the caller chose a policy.
  if (!p->policy_set) p->nt = p->nt_ld = p->n >= (int64_t(128) << 20) / p->orig_eb;
  return true;
}

// The staged gather's lane grouping.  Job idx (one 16-byte destination chunk) of a
// workgroup belongs to 32-lane slice q = idx / 32; a slice covers G = 32 / cps
// tiles x cps chunks of each: tile (q / slices) * G + l / cps, chunk (q % slices) * cps
// + l % cps with l = idx % 32 and slices = cpt / cps.  With cps = min(cpt, 32) this is
// tile idx / cpt, chunk idx % cpt.  Each lane gathers its chunk's V elements from the
// staged footprint one LDS read at a time; the LDS serves the lanes of a slice
// together ([print_layout page, sections 4.3 and 5.2]: distinct words in one bank are
// served one after another), so the grouping decides the bank conflicts.  The planner
// evaluates the gfx950 bank model over every wave of one workgroup's first round for
// each admissible cps and keeps the cheapest, the widest on a tie (longer contiguous
// destination runs per store instruction).
static int64_t staged_gather_cps(const Plan& p, int inner, int64_t cpt, int64_t K, int64_t Fc, int64_t L) {
  const int V = 16 / p.eb;
  int64_t g[16];  // element offset in the footprint of element x of chunk c: filled per c
  auto offs = [&](int64_t c, int64_t* out) {
    for (int x = 0; x < V; ++x) {
      int64_t e = c * V + x, off = 0;
      for (int k = 0; k < inner; ++k) {
        off += (e % p.m[k].ext) * p.m[k].ss;
        e /= p.m[k].ext;
      }
      out[x] = off;
    }
  };
  int32_t banks, lpp;
  gfx950_lds_model((size_t)p.eb, false, &banks, &lpp);
  const int64_t dflt = std::min<int64_t>(cpt, 32);
  int64_t best = dflt, best_cost = -1;
  for (int64_t cps = dflt; cps >= 1; cps >>= 1) {
    const int64_t slices = cpt / cps, G = 32 / cps;
    // a lane's chunk stays fixed across rounds of L jobs (slices | L / 32); a
    // narrower grouping needs whole groups of G tiles (the default one is tile
    // idx / cpt for any K)
    if (slices > L / 32 || (L / 32) % slices || (cps != dflt && K % G)) continue;
    int64_t cost = 0;
    const int64_t jobs = std::min<int64_t>(L, K * cpt);
    for (int64_t w0 = 0; w0 < jobs; w0 += 64) {
      int64_t addr[16][64];
      int lanes = (int)std::min<int64_t>(64, jobs - w0);
      for (int l = 0; l < lanes; ++l) {
        const int64_t idx = w0 + l, q = idx >> 5, li = idx & 31;
        const int64_t kk = (q / slices) * G + li / cps, c = (q % slices) * cps + li % cps;
        offs(c, g);
        for (int x = 0; x < V; ++x) addr[x][l] = (kk * Fc * 16) + g[x] * p.eb;
      }
      for (int x = 0; x < V; ++x) cost += lds_cycles(addr[x], lanes, p.eb, banks, lpp, nullptr, nullptr);
    }
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = cps;
    }
  }
  return best;
}

static int plan_alias(Plan* p, int64_t n, int64_t cos_s, int64_t cos_d) {
  const int64_t win = 8192;  // dst offsets owned by one workgroup (LDS owner table)
  int64_t windows = (cos_d + win - 1) / win;
  if (cos_d > (int64_t(1) << 26) || n >= (int64_t(1) << 31) || cos_s >= (int64_t(1) << 31)) return LR_ERR_ALIAS;
  if ((double)n * (double)windows > (double)(int64_t(1) << 36)) return LR_ERR_ALIAS;
  p->path = LR_PATH_ALIAS;
  p->nt = p->nt_ld = false;  // plain accesses: every workgroup re-reads the source
  p->alias_windows = windows;
  p->block = 1024;
  p->grid = windows;
  return LR_OK;
}

// Traversal order 2 of the vector path: the lanes of a wave walk the source's
// order (after the common contiguous mode), the four waves of a workgroup the
// destination's, and everything after that the source's again.  A workgroup then
// reads a few long source runs and writes a few long destination runs, where either
// order alone makes one side a scatter of short runs (the 128-byte tile rows of a
// retile).  Modes are split where a wave or workgroup boundary falls inside one; a
// mode that does not divide there is taken whole.  Any order of the joint modes is
// the same copy when the destination is injective.
static void block_vector_order(Plan* p) {
  if (p->rank + 2 > kMaxKernelModes) {
    std::stable_sort(p->m + 1, p->m + p->rank, [](const JMode& x, const JMode& y) {
      return x.ss < y.ss || (x.ss == y.ss && x.sd < y.sd);
    });
    return;
  }
  JMode rest[kMaxJoint];
  int nr = 0;
  for (int k = 1; k < p->rank; ++k) rest[nr++] = p->m[k];
  JMode out[kMaxJoint];
  int no = 0;
  out[no++] = p->m[0];
  int64_t lanes = p->m[0].ext / p->v;  // units along the common mode
  auto first = [&](bool by_src) {
    int best = 0;
    for (int k = 1; k < nr; ++k) {
      const int64_t a = by_src ? rest[k].ss : rest[k].sd, b = by_src ? rest[best].ss : rest[best].sd;
      if (a < b) best = k;
    }
    return best;
  };
  auto fill = [&](int64_t target, bool by_src) {
    while (lanes < target && nr > 0) {
      const int k = first(by_src);
      const int64_t need = target / lanes;
      JMode m = rest[k];
      if (target % lanes == 0 && m.ext > need && m.ext % need == 0) {
        out[no++] = {need, m.ss, m.sd};
        rest[k] = {m.ext / need, m.ss * need, m.sd * need};
        lanes *= need;
      } else {
        out[no++] = m;
        lanes *= m.ext;
        for (int j = k; j + 1 < nr; ++j) rest[j] = rest[j + 1];
        --nr;
      }
    }
  };
  fill(64, true);    // a wave's lanes
  fill(p->block, false);  // a workgroup's waves
  std::stable_sort(rest, rest + nr, [](const JMode& x, const JMode& y) {
    return x.ss < y.ss || (x.ss == y.ss && x.sd < y.sd);
  });
  for (int k = 0; k < nr; ++k) out[no++] = rest[k];
  std::memcpy(p->m, out, sizeof(JMode) * no);
  p->rank = no;
}

// Tiles of atoms through LDS (vector order 3): the common contiguous mode is an atom
// of K = 2..32 16-byte chunks (32-512 bytes), a mode a continues it in the source (source stride
// equal to the atom's extent) and another mode b in the destination.  Without
// regrouping, one side is a scatter of atom-sized runs whichever order the lanes walk
// (the 128-byte tile rows of a retile); a tile of T x T atoms (a x b) staged in LDS
// is loaded as T source runs of T atoms and stored as T destination runs of T atoms
// (T from atom_tile).  Taken for atoms up to 256 bytes, and beyond for atoms that
// are not whole 128-byte lines (the one-unit-per-lane orders then write runs that
// end inside a line); measured on (b,s,h,d) -> (b,h,s,d) bf16 head splits: 80- and
// 96-byte atoms 3.0x and 2.5x faster than the source order, 128 bytes 1.17x, 192 bytes
// 1.07x, 256 bytes 1.04x, 320 bytes 1.01x, 384 and 512 bytes 0.98-0.99x.  Needs
// 16-byte units, 32-bit offsets, at
// least T atoms along a and b, and the other modes within a kernel's batch modes.
static bool atom_tiles(const Plan& p, int* a, int* b, int64_t* T) {
  if (p.v * p.eb != 16 || p.unroll != 1 || p.wide || p.rank < 3 || p.rank - 3 > kMaxKernelModes) return false;
  if (p.m[0].ss != 1 || p.m[0].sd != 1) return false;
  const int64_t e0 = p.m[0].ext, K = e0 / p.v;
  if (e0 % p.v || K < 2 || K > 32 || (K > 16 && K % 8 == 0)) return false;
  *a = *b = -1;
  for (int k = 1; k < p.rank; ++k) {
    if (*a < 0 && p.m[k].ss == e0) *a = k;
    if (*b < 0 && p.m[k].sd == e0) *b = k;
  }
  if (*a < 0 || *b < 0 || *a == *b) return false;
  *T = atom_tile(K);
  return p.m[*a].ext >= *T && p.m[*b].ext >= *T;
}

// The staged path: a compact block of the inner destination modes whose source
// footprint is small, staged in LDS and gathered into 16-byte stores.  b is the
// destination-contiguous mode.  Fills *p and returns true when it applies.
static bool plan_staged(Plan* p, int b, size_t src_align, size_t dst_align, int64_t src_cap,
                        const lr_copy_tuning& tun) {
  const int V16 = 16 / p->eb;
  bool ok = b == 0 && p->sw_s.b == 0 && src_align >= 16 && dst_align >= 16;
  int inner = 0;
  int64_t P = 1, F = 1;
  if (ok) {
    // the longest compact dst prefix (at most 4 KiB) whose source footprint is small;
    // a prefix can be compact where a shorter one is not (a whole small matrix)
    int64_t want = 1, P2 = 1, F2 = 1;
    for (int k = 0; k < p->rank - 1 && p->m[k].sd == want; ++k) {
      P2 *= p->m[k].ext;
      F2 += (p->m[k].ext - 1) * p->m[k].ss;
      if (P2 * p->eb > 4096) break;
      want = P2;
      if (F2 <= 2 * P2 + 64) {
        P = P2;
        F = F2;
        inner = k + 1;
      }
    }
    ok = inner >= 1 && inner < p->rank && p->m[inner].sd == P && (P * p->eb) % 16 == 0 &&
         is_pow2(P * p->eb / 16) && swz_keeps(p->sw_d, V16);
    for (int k = inner; ok && k < p->rank; ++k) {
      if ((p->m[k].ss * p->eb) % 16) ok = false;
      if ((p->m[k].sd * p->eb) % 16) ok = false;
    }
    if (ok) {
      const int64_t Fc = (F * p->eb + 15) / 16;
      // the padded footprint of the last tile must stay inside the buffer
      int64_t maxbase = 0;
      for (int k = inner; k < p->rank; ++k) maxbase += (p->m[k].ext - 1) * p->m[k].ss;
      ok = (maxbase + Fc * 16 / p->eb) <= src_cap;
      if (ok) {
        const int64_t cpt = P * p->eb / 16;  // 16-byte dst chunks per tile
        // L lanes per workgroup, at least one per dst chunk of a tile (a lane's
        // chunk position in the gather is then the same in every round)
        int64_t L = knob(tun.workgroup_lanes, 256);
        while (L < cpt) L *= 2;
        // about two dst chunks per lane (padded tiles: 5.85 TB/s, against 5.79 with
        // four and 5.57 with eight; one measured 4.8-5.1), and at most 10 KiB of LDS
        // per 64 lanes.  Stores with the sc1 bit measured no faster here.
        const int64_t K = std::max<int64_t>(1, std::min<int64_t>(2 * L / cpt, 10 * L / Fc));
        p->block = L;
        p->path = LR_PATH_STAGED;
        // direct global -> LDS loads measured 2.6 % faster on the padded tiles
        // (5.79 vs 5.64 TB/s): the footprint never passes through registers, so
        // every load of it is in flight at once.
        p->direct = knob(tun.direct_loads, 1) != 0;
        p->staged_inner = inner;
        p->staged_P = P;
        p->staged_F = F;
        p->staged_Fc = Fc;
        p->staged_cpt = cpt;
        p->staged_K = K;
        p->staged_cps = staged_gather_cps(*p, inner, cpt, K, Fc, L);
        if (tun.gather_chunks > 0 && tun.gather_chunks <= cpt && cpt % tun.gather_chunks == 0 &&
            (L / 32) % (cpt / tun.gather_chunks) == 0 &&
            (tun.gather_chunks == std::min<int64_t>(cpt, 32) || K % (32 / tun.gather_chunks) == 0))
          p->staged_cps = tun.gather_chunks;
        p->v = V16;
        p->tile_a = K;
        int64_t batch = 1;
        for (int k = inner + 1; k < p->rank; ++k) batch *= p->m[k].ext;
        p->grid = ((p->m[inner].ext + K - 1) / K) * batch;
        return true;
      }
    }
  }
  return false;
}

// Cycles of one wavefront's 16-byte LDS accesses to 16-byte slots, in the gfx950
// model (lds_cycles): a slot covers 4 consecutive banks, so a phase costs the most
// distinct slots that share one group of 4 banks (slot modulo banks / 4).
static int64_t slot_cycles(const int64_t* slot, int lanes, int32_t banks, int32_t per) {
  int64_t cycles = 0;
  const int groups = banks / 4;
  for (int p0 = 0; p0 < lanes; p0 += per) {
    const int n = std::min(lanes, p0 + per) - p0;
    int cnt[LR_WAVE_LANES] = {0};
    int ways = 0;
    for (int t = 0; t < n; ++t) {
      bool seen = false;  // a slot several lanes read is served once
      for (int q = 0; q < t && !seen; ++q) seen = slot[p0 + q] == slot[p0 + t];
      if (!seen) ways = std::max(ways, ++cnt[slot[p0 + t] % groups]);
    }
    cycles += ways;
  }
  return cycles;
}

// LDS cycles of the batched kernel's two exchanges (the blocks' source-row reads and
// destination-row writes, 16 bytes a lane) over one wavefront region, in the gfx950
// model, for the chunk swizzle sw (two XOR terms of shift, mask, target shift) and
// block order.
static int64_t batched_lds_cycles(int64_t P, int64_t Q, int64_t V, int64_t mpw, const int sw[6], int order) {
  int32_t rb, rl, wb, wl;
  gfx950_lds_model(16, false, &rb, &rl);
  gfx950_lds_model(16, true, &wb, &wl);
  auto swz = [&](int64_t c) { return c ^ (((c >> sw[0]) & sw[1]) << sw[2]) ^ (((c >> sw[3]) & sw[4]) << sw[5]); };
  const int64_t pq = P * Q, cpm = pq * V, nblk = mpw * pq;
  int64_t cycles = 0;
  int64_t ra[LR_WAVE_LANES], wa[LR_WAVE_LANES];
  for (int64_t u0 = 0; u0 < nblk; u0 += LR_WAVE_LANES) {
    const int lanes = (int)std::min<int64_t>(LR_WAVE_LANES, nblk - u0);
    for (int64_t j = 0; j < V; ++j) {
      for (int l = 0; l < lanes; ++l) {
        const int64_t u = u0 + l, mi = u / pq, rest = u % pq;
        const int64_t ba = order ? rest / Q : rest % P, bb = order ? rest % Q : rest / P;
        ra[l] = swz(mi * cpm + (V * bb + j) * P + ba);
        wa[l] = swz(mi * cpm + (V * ba + j) * Q + bb);
      }
      cycles += slot_cycles(ra, lanes, rb, rl) + slot_cycles(wa, lanes, wb, wl);
    }
  }
  return cycles;
}

// Batched small matrices: modes a (source-contiguous) and b (destination-contiguous)
// form a matrix that is compact on both sides (b's source stride is a's extent, a's
// destination stride b's extent), both extents multiples of V = 16 / eb, at most
// 8 KiB, over any other (batch) modes whose strides keep 16-byte chunks.  Fills *p and
// returns true when it applies.
// The LDS swizzle and block order are left to batched_swizzle.
static bool plan_batched(Plan* p, int a, int b, size_t src_align, size_t dst_align) {
  if (p->eb != 2 && p->eb != 4 && p->eb != 8) return false;
  if (p->sw_s.b || p->sw_d.b || src_align < 16 || dst_align < 16 || p->rank - 2 > kMaxKernelModes) return false;
  const int64_t V = 16 / p->eb, A = p->m[a].ext, B = p->m[b].ext;
  if (A % V || B % V || p->m[b].ss != A || p->m[a].sd != B || A * B * p->eb > 8192) return false;
  int64_t count = 1;
  for (int k = 0; k < p->rank; ++k) {
    if (k == a || k == b) continue;
    if (p->m[k].ss % V || p->m[k].sd % V) return false;
    count *= p->m[k].ext;
  }
  const int64_t P = A / V, Q = B / V, cpm = P * Q * V, mpw = 512 / cpm;
  p->path = LR_PATH_BATCHED;
  p->a = a;
  p->b = b;
  p->b2 = -1;
  p->v = (int)V;
  p->tile_a = A;
  p->tile_b = B;
  p->block = 64;  // one wavefront per workgroup
  p->direct = true;
  p->bufst = false;
  p->tel = p->twin = p->tr = false;
  p->pipe = 0;
  p->bt_mpw = mpw;
  p->bt_count = count;
  p->grid = (count + mpw - 1) / mpw;
  return true;
}

// The LDS swizzle and block order of a batched plan: the cheapest in the bank model.
// The first eight candidates (each with the order it is tried in first) cover,
// between them, every power-of-two matrix of 2-, 4- and 8-byte elements that some
// two-term XOR swizzle inside 16-chunk groups leaves without conflicts in the model
// (a greedy cover found by exhaustive search); the rest are single terms for other
// sizes.  A conflict-free candidate ends the search (reads take 4 cycles per row of
// blocks, writes 8).  Measured, the choice moves the kernel by 3 % at most, even
// against no swizzle at 4-8 times the LDS cycles (the exchange is far from the
// limit), and the model misses some conflicts the counters show; the search costs
// up to ~100 us of host time, so its result is kept per matrix shape and override.
static void batched_swizzle(Plan* p, const lr_copy_tuning& tun) {
  static const int kCand[][7] = {
      {3, 7, 0, 4, 7, 0, 0}, {4, 7, 1, 4, 15, 0, 1}, {3, 3, 1, 3, 7, 0, 0}, {5, 1, 2, 5, 15, 0, 1},
      {4, 3, 2, 4, 7, 0, 0}, {3, 1, 2, 4, 3, 1, 0}, {3, 1, 2, 4, 3, 0, 1}, {3, 3, 1, 4, 7, 0, 0},
      {4, 7, 1, 0, 0, 0, 0}, {4, 15, 0, 0, 0, 0, 0}, {4, 3, 2, 0, 0, 0, 0}, {4, 3, 1, 0, 0, 0, 0},
      {3, 3, 1, 0, 0, 0, 0}, {3, 3, 0, 0, 0, 0, 0}, {5, 15, 0, 0, 0, 0, 0}, {0, 0, 0, 0, 0, 0, 0}};
  const int64_t V = p->v, P = p->tile_a / V, Q = p->tile_b / V, mpw = p->bt_mpw;
  const uint64_t key = (uint64_t)P | ((uint64_t)Q << 16) | ((uint64_t)V << 32) |
                       ((uint64_t)(tun.batch_swizzle + 1) << 40) | ((uint64_t)(tun.batch_order + 1) << 48);
  thread_local std::unordered_map<uint64_t, std::array<int, 7>> cache;
  const auto hit = cache.find(key);
  if (hit != cache.end()) {
    for (int i = 0; i < 6; ++i) p->bt_sw[i] = hit->second[i];
    p->bt_order = hit->second[6];
    return;
  }
  const int64_t ideal = ((mpw * P * Q + LR_WAVE_LANES - 1) / LR_WAVE_LANES) * V * (4 + 8);
  int64_t best = -1;
  for (int ci = 0; ci < 16 && !(best >= 0 && best <= ideal); ++ci) {
    if (tun.batch_swizzle >= 0 && ci != tun.batch_swizzle) continue;
    for (int o = 0; o < 2; ++o) {
      const int order = o ? 1 - kCand[ci][6] : kCand[ci][6];
      if (tun.batch_order >= 0 && order != tun.batch_order) continue;
      const int64_t cy = batched_lds_cycles(P, Q, V, mpw, kCand[ci], order);
      if (best < 0 || cy < best) {
        best = cy;
        for (int i = 0; i < 6; ++i) p->bt_sw[i] = kCand[ci][i];
        p->bt_order = order;
      }
      if (best <= ideal) break;
    }
  }
  std::array<int, 7> r;
  for (int i = 0; i < 6; ++i) r[i] = p->bt_sw[i];
  r[6] = p->bt_order;
  if (cache.size() > 4096) cache.clear();
  cache.emplace(key, r);
}

// Lanes per workgroup of the vector / generic kernel with one unit per lane: one
// wavefront for a single contiguous run from a 64 MiB footprint (measured on plain
// copies: 64 MiB 12.9-13.1 -> 12.8 us, 256 MiB 43.1 -> 41.0, 1 GiB 164.7 -> 161.7; at
// 16 MiB 256 lanes stay ahead, 7.9 against 8.3 us), 256 otherwise (a 3-D permute over
// three modes lost 2-4 % with one wavefront, row gathers tied).
static int stream_lanes(const Plan& p, bool big_footprint) { return big_footprint && p.rank == 1 ? 64 : 256; }

static int plan_path(const lr_layout* Ls, int64_t src_cap, size_t src_align, const lr_layout* Ld, int64_t dst_cap,
                     size_t dst_align, size_t elem_bytes, uint32_t flags, const lr_copy_tuning& tun, Plan* p) {
  int rc;
  if ((rc = validate(Ls))) return rc;
  if ((rc = validate(Ld))) return rc;
  if (!p) return LR_ERR_INVALID;
  if (!(elem_bytes == 1 || elem_bytes == 2 || elem_bytes == 4 || elem_bytes == 8 || elem_bytes == 16))
    return LR_ERR_ELEM_BYTES;
  if (src_cap < 0 || dst_cap < 0) return LR_ERR_INVALID;
  std::memset(p, 0, sizeof(*p));
  p->a = p->b = p->b2 = -1;
  const int64_t n = size_of(Ls);
  if (size_of(Ld) != n) return LR_ERR_SIZE_MISMATCH;
  const int64_t cos_s = cosize_bound(Ls), cos_d = cosize_bound(Ld);
  if (cos_s > src_cap || cos_d > dst_cap) return LR_ERR_BOUNDS;
  int64_t t;
  if (!mul_ok(src_cap, (int64_t)elem_bytes, &t) || !mul_ok(dst_cap, (int64_t)elem_bytes, &t)) return LR_ERR_OVERFLOW;
  p->n = n;
  p->eb = (int)elem_bytes;
  p->orig_eb = (int)elem_bytes;
  p->sw_s = {Ls->swz_b, Ls->swz_m, Ls->swz_s};
  p->sw_d = {Ld->swz_b, Ld->swz_m, Ld->swz_s};
  if (src_align == 0) src_align = 1;
  if (dst_align == 0) dst_align = 1;
  src_align = std::min<size_t>(src_align & (~src_align + 1), 16);
  dst_align = std::min<size_t>(dst_align & (~dst_align + 1), 16);

  const uint32_t forced_raw = (flags >> 8) & 0xFFu;
  const int forced = forced_raw ? (int)forced_raw - 1 : -1;
  if (forced > LR_PATH_BATCHED) return LR_ERR_INVALID;
  const int64_t lim32 = int64_t(1) << 31;
  p->wide = (flags & LR_COPY_WIDE_INDEX) || n >= lim32 || cos_s >= lim32 || cos_d >= lim32;
  p->block = 256;
  // Non-temporal loads and stores when the footprint (source plus destination
  // bytes) is at least 64 MiB, a quarter of the 256 MiB last-level cache.  From
  // there a copy from memory runs faster streaming: 5-15 % on every workload of
  // 256 MiB and more, 7 % on the 64 MiB retile (13.6 against 14.6 us), whose plain
  // stores would leave the result cached for a reader that follows at once (the
  // caller can ask for that with the store policy).  Smaller copies keep plain
  // accesses, which keep the data cache-resident.  An override of one of the two
  // policies alone sets the other to match.  Stores carry the sc1 scope bit
  // (buffer stores) where a kernel has them, unless the store policy asks for nt
  // alone.
  const bool big_footprint = n >= (int64_t(32) << 20) / (int64_t)elem_bytes;
  const int32_t lp = tun.load_policy, sp = tun.store_policy;
  p->nt_ld = lp >= 0 ? lp == 2 : (sp >= 0 ? sp != 0 : big_footprint);
  p->nt = sp >= 0 ? sp != 0 : (lp >= 0 ? lp == 2 : big_footprint);
  p->policy_set = lp >= 0 || sp >= 0;
  const bool sc1_ok = sp != 2;
  // one unit per lane measured fastest for streaming copies on MI355X (more waves
  // in flight beat more loads per wave)
  p->unroll = knob(tun.units_per_lane, 1);

  // --- non-injective destination: sequential semantics
  const bool inj = injective(Ld);
  if (!inj || forced == LR_PATH_ALIAS) {
    if (!inj && !(flags & LR_COPY_ORDERED_ALIAS)) return LR_ERR_ALIAS;
    if (forced >= 0 && forced != LR_PATH_ALIAS) return LR_ERR_PATH;
    p->wide = false;
    return plan_alias(p, n, cos_s, cos_d);
  }

  // --- joint flat form
  int rank = 0;
  const bool have_joint = joint_flat(Ls, Ld, p->m, &rank, true);
  if (have_joint && rank == 0) {  // a single element: one trivial mode
    p->m[0] = {1, 1, 1};
    rank = 1;
  }
  p->rank = have_joint ? rank : 0;
  if (!have_joint || forced == LR_PATH_DUAL || (have_joint && rank > kMaxKernelModes)) {
    if (forced >= 0 && forced != LR_PATH_DUAL) return LR_ERR_PATH;
    p->path = LR_PATH_DUAL;
    p->nt = p->nt_ld = false;  // the per-element fallback keeps plain accesses
    p->rank = 0;
    p->v = 1;
    p->n_units = n;
    p->grid = (n + 1023) / 1024;
    return LR_OK;
  }
  if (p->wide) {
    // 64-bit index arithmetic: the unit-per-lane kernel, four units per lane, with
    // 16-byte vectors along a common contiguous mode when there is one
    if (forced >= 0 && forced != LR_PATH_GENERIC && forced != LR_PATH_VECTOR) return LR_ERR_PATH;
    const bool c0 = p->m[0].ss == 1 && p->m[0].sd == 1;
    const int64_t v = (c0 && forced != LR_PATH_GENERIC) ? unit_width(*p, src_align, dst_align) : 1;
    if (forced == LR_PATH_VECTOR && v <= 1) return LR_ERR_PATH;
    p->path = v > 1 ? LR_PATH_VECTOR : LR_PATH_GENERIC;
    p->v = (int)v;
    p->unroll = 4;
    p->n_units = n / v;
    p->grid = (p->n_units + 1023) / 1024;
    return LR_OK;
  }

  // --- long common contiguous mode: 16-byte vectors straight through
  const bool common0 = p->rank > 0 && p->m[0].ss == 1 && p->m[0].sd == 1;
  const int64_t v0 = unit_width(*p, src_align, dst_align);
  // 32- and 48-byte common runs go the vector way only as tiles of atoms
  bool short_atoms = false;
  if (common0 && p->m[0].ext * p->eb < 64 && v0 * p->eb == 16 && p->unroll == 1 && !p->wide) {
    Plan q = *p;
    q.v = (int)v0;
    int qa, qb;
    int64_t qt;
    short_atoms = atom_tiles(q, &qa, &qb, &qt);
  }
  const bool want_vector = common0 && (p->m[0].ext * p->eb >= 64 || short_atoms) && v0 * p->eb >= 4;
  if (forced == LR_PATH_VECTOR && !(common0 && v0 > 1)) return LR_ERR_PATH;
  if (forced == LR_PATH_VECTOR || forced == LR_PATH_GENERIC || (forced < 0 && want_vector)) {
    p->path = forced == LR_PATH_GENERIC ? LR_PATH_GENERIC : (v0 > 1 ? LR_PATH_VECTOR : LR_PATH_GENERIC);
    p->v = (int)v0;
    p->n_units = n / v0;
    p->block = (p->unroll == 1 && !p->wide) ? knob(tun.workgroup_lanes, stream_lanes(*p, big_footprint)) : 256;
    p->grid = (p->n_units + p->block * p->unroll - 1) / (p->block * p->unroll);
    // Traversal order after the common contiguous mode.  Any order of the joint
    // modes is the same copy when the destination is injective; walking the source
    // order (reads in long runs, writes in runs of the common mode) measured
    // faster than the destination order when the common run is short (the 128-byte
    // rows of the 4096^2 retile).
    // Tiles of atoms through LDS where they apply (measured on the 4096^2 retile,
    // 128-byte atoms: 13.5 -> 12.0 us, a copy of the same bytes 12.1); the source
    // order otherwise.
    int aa = -1, ab = -1;
    int64_t at = 0;
    const bool atoms = atom_tiles(*p, &aa, &ab, &at);
    p->vorder = knob(tun.vector_order, atoms ? 3 : 1);
    if (p->vorder == 3 && !atoms) p->vorder = 1;
    if (p->vorder == 3) {
      p->block = knob(tun.workgroup_lanes, 256);
      p->a = aa;
      p->b = ab;
      p->tile_a = p->tile_b = at;
      int64_t batch = 1;
      for (int k = 1; k < p->rank; ++k)
        if (k != aa && k != ab) batch *= p->m[k].ext;
      p->grid = ((p->m[aa].ext + at - 1) / at) * ((p->m[ab].ext + at - 1) / at) * batch;
    } else if (p->vorder >= 1 && p->rank > 2) {
      if (p->vorder == 2 && p->unroll == 1 && !p->wide)
        block_vector_order(p);
      else
        std::stable_sort(p->m + 1, p->m + p->rank, [](const JMode& x, const JMode& y) {
          return x.ss < y.ss || (x.ss == y.ss && x.sd < y.sd);
        });
    }
    // Streaming 16-byte units are stored as buffer stores with the nt and sc1
    // cache-policy bits (a 512 MiB copy: 6.41 -> 6.55 TB/s), addressed by one 32-bit
    // byte offset from the destination base: the destination's span must stay
    // under 4 GiB.  LR_SC1=0 keeps global stores.
    p->bufst = p->v * p->eb == 16 && p->unroll == 1 && !p->wide && sc1_ok &&
               dst_span_bytes(*p) < (int64_t(1) << 32);
    return LR_OK;
  }

  // --- fuse a short common contiguous prefix into a wider element
  if (common0) {
    const int64_t e = p->m[0].ext;
    bool ok = is_pow2(e) && e * p->eb <= 16 && swz_keeps(p->sw_s, e) && swz_keeps(p->sw_d, e) &&
              src_align % (size_t)(e * p->eb) == 0 && dst_align % (size_t)(e * p->eb) == 0;
    for (int k = 1; ok && k < p->rank; ++k) ok = (p->m[k].ss % e == 0) && (p->m[k].sd % e == 0);
    if (ok) {
      const int sh = log2i(e);
      for (int k = 1; k < p->rank; ++k) p->m[k - 1] = {p->m[k].ext, p->m[k].ss / e, p->m[k].sd / e};
      p->rank -= 1;
      p->eb *= (int)e;
      if (p->sw_s.b) p->sw_s.m -= sh;
      if (p->sw_d.b) p->sw_d.m -= sh;
      if (p->rank == 0) {  // the whole copy was one contiguous run
        p->m[0] = {1, 1, 1};
        p->rank = 1;
      }
    }
  }

  // --- a: contiguous in src, b: contiguous in dst
  int a = -1, b = -1;
  for (int k = 0; k < p->rank; ++k) {
    if (b < 0 && p->m[k].sd == 1) b = k;
    if (a < 0 && p->m[k].ss == 1) a = k;
  }
  const int V16 = 16 / p->eb;

  // interleave: the dst-contiguous mode b is short and a follows it in dst
  if (a >= 0 && b >= 0 && a != b && (forced < 0 || forced == LR_PATH_INTERLEAVE)) {
    const int64_t nb = p->m[b].ext, V = V16;
    // NB a power of two: the register kernels; other NB from 3 to 8 (three colour
    // channels, say): the channel shuffle through LDS, which applies no swizzle
    const int32_t inarrow_env = knob(tun.interleave_form, 1);
    const bool chan = chan_supported(p->eb, nb) && p->sw_s.b == 0 && p->sw_d.b == 0 &&
                      (!is_pow2(nb) || inarrow_env == 2);
    bool ok = (is_pow2(nb) || chan) && nb >= 2 && nb * p->eb <= 16 && p->m[a].sd == nb && p->m[a].ext % V == 0 &&
              swz_keeps(p->sw_s, V) && swz_keeps(p->sw_d, V) && src_align >= 16 && dst_align >= 16;
    if (ok) {
      for (int k = 0; k < p->rank && ok; ++k) {
        if (k != a && p->m[k].ss % V) ok = false;
        if (k != a && k != b && p->m[k].sd % V) ok = false;
      }
    }
    if (ok) {
      p->path = LR_PATH_INTERLEAVE;
      p->a = a;
      p->b = b;
      p->v = (int)V;
      // one 16-byte store per lane from NB narrow loads measured faster (every store
      // instruction covers 1 KiB of contiguous dst; NB 16-byte stores per lane from NB
      // wide loads write every NB-th chunk per instruction: 3.8 against 6.1 TB/s)
      p->inarrow = chan ? 2 : (int)(inarrow_env & 1);
      // a-elements per workgroup, matching the kernel's per-lane unroll (one dst
      // chunk per lane on the narrow variant, V pixels per lane on the shuffle)
      // one wavefront per workgroup from a 64 MiB footprint: the (16,32,4096,128) head
      // interleave 162.4 -> 159.0-160.2 us back to back, a (16,64,4096,64) one with four
      // heads 24.3 -> 17.1 us
      p->block = p->inarrow == 1 ? knob(tun.workgroup_lanes, big_footprint ? 64 : 256)
                 : p->inarrow == 2 ? knob(tun.workgroup_lanes, 256) : 256;
      p->tile_a = p->inarrow == 2 ? p->block * V : p->inarrow ? p->block * (V / nb) : (nb >= 8 ? 1 : 8 / nb) * 256 * V;
      // the narrow variant's streaming stores as buffer stores with the nt and sc1
      // bits from the destination base (head interleave 6.27 -> 6.55 TB/s)
      p->bufst = p->inarrow != 0 && sc1_ok && dst_span_bytes(*p) < (int64_t(1) << 32);
      p->tile_b = nb;
      int64_t batch = 1;
      for (int k = 0; k < p->rank; ++k)
        if (k != a && k != b) batch *= p->m[k].ext;
      p->grid = ((p->m[a].ext + p->tile_a - 1) / p->tile_a) * batch;
      return LR_OK;
    }
    if (forced == LR_PATH_INTERLEAVE) return plan_chan_elements(p, a, b, true, src_align, dst_align) ? LR_OK : LR_ERR_PATH;
  }

  // de-interleave: the mirror of the above.  The src-contiguous mode a is short (C
  // channels of at most 16 bytes together) and the dst-contiguous mode b follows it
  // in src (the pixels of NHWC -> NCHW with few channels): each lane turns V pixels
  // of C interleaved channels into C chunks of one plane each.
  if (a >= 0 && b >= 0 && a != b && (forced < 0 || forced == LR_PATH_DEINTERLEAVE)) {
    const int64_t C = p->m[a].ext, V = V16;
    bool ok = chan_supported(p->eb, C) && p->m[b].ss == C && p->m[b].ext % V == 0 && p->m[a].sd % V == 0 &&
              p->sw_s.b == 0 && p->sw_d.b == 0 && src_align >= 16 && dst_align >= 16;
    for (int k = 0; k < p->rank && ok; ++k)
      if (k != a && k != b && (p->m[k].ss % V || p->m[k].sd % V)) ok = false;
    if (ok) {
      p->path = LR_PATH_DEINTERLEAVE;
      p->a = a;
      p->b = b;
      p->v = (int)V;
      p->block = knob(tun.workgroup_lanes, 256);
      p->tile_a = p->block * V;  // pixels per workgroup (V per lane)
      p->tile_b = C;
      p->bufst = sc1_ok && dst_span_bytes(*p) < (int64_t(1) << 32);
      int64_t batch = 1;
      for (int k = 0; k < p->rank; ++k)
        if (k != a && k != b) batch *= p->m[k].ext;
      p->grid = ((p->m[b].ext + p->tile_a - 1) / p->tile_a) * batch;
      return LR_OK;
    }
    if (forced == LR_PATH_DEINTERLEAVE) return plan_chan_elements(p, a, b, false, src_align, dst_align) ? LR_OK : LR_ERR_PATH;
  }

  // batched small matrices (each at most 8 KiB, compact on both sides): whole matrices
  // per wavefront.  Taken at once for 2-byte elements (over 2^27 elements, back to
  // back: 16 x 16 46.1 us against 46.8 staged, 32 x 32 46.5 against 47.2, 16 x 32 46.2
  // against 46.7, 64 x 64 46.5 against 47.9 for the transpose); other small matrices
  // take it below when the staged path does not apply.
  Plan batched = *p;
  const bool bt_ok = a >= 0 && b >= 0 && a != b && (forced < 0 || forced == LR_PATH_BATCHED) &&
                     plan_batched(&batched, a, b, src_align, dst_align);
  if (forced == LR_PATH_BATCHED) {
    if (!bt_ok) return LR_ERR_PATH;
    *p = batched;
    batched_swizzle(p, tun);
    return LR_OK;
  }
  if (bt_ok && forced < 0 && p->eb == 2) {
    *p = batched;
    batched_swizzle(p, tun);
    return LR_OK;
  }

  // transpose: register blocks of V x V elements over the src-contiguous mode a and
  // the dst-contiguous run b.  When the dst-contiguous mode is short (a power of
  // two under 16 bytes) and another mode b2 continues it in dst (dst stride equal
  // to b's extent), the pair acts as one b of extent ext_b * ext_b2 whose source
  // row offsets split over the two modes (a three-way remap such as head pairs
  // interleaved inside column-major tiles).
  const bool want_t = forced < 0 || forced == LR_PATH_TRANSPOSE || forced == LR_PATH_TRANSPOSE_DIRECT;
  if (a >= 0 && b >= 0 && a != b && want_t) {
    const Plan before_transpose = *p;
    int b2 = -1;
    if (is_pow2(p->m[b].ext) && p->m[b].ext * p->eb < 16)
      for (int k = 0; k < p->rank && b2 < 0; ++k)
        if (k != a && k != b && p->m[k].sd == p->m[b].ext) b2 = k;
    const int64_t ext_b = p->m[b].ext * (b2 >= 0 ? p->m[b2].ext : 1);
    auto strides_ok = [&](int64_t V) {
      for (int k = 0; k < p->rank; ++k) {
        if (k != a && p->m[k].ss % V) return false;
        if (k != b && k != b2 && p->m[k].sd % V) return false;
      }
      return true;
    };
    // 1-byte elements: 8-byte chunks (8 x 8 byte register blocks, 32 VGPRs of data
    // against 128 for 16 x 16), measured faster in wide tiles: u8 4096^2 3.49 -> 3.91
    // TB/s, 6144^2 3.65 -> 4.07, 8192 x 16384 5.23 -> 5.44, 8192^2 4.71 -> 4.78
    // (16-byte chunks for 1-byte elements on request, and by default when their tile
    // is read back with the transpose reads)
    const bool chunk16 = tun.chunk_bytes == 16 || (tun.chunk_bytes < 0 && tun.transpose_reads == 1);
    int64_t V = (p->eb == 1 && !chunk16) ? 8 : V16;
    while (V > 1) {
      bool ok = p->m[a].ext % V == 0 && ext_b % V == 0 && strides_ok(V) && swz_keeps(p->sw_s, V) &&
                swz_keeps(p->sw_d, V) && src_align % (size_t)(V * p->eb) == 0 &&
                dst_align % (size_t)(V * p->eb) == 0;
      if (ok) break;
      V >>= 1;
    }
    const bool long_b = ext_b * p->eb > 16 && p->m[a].ext * p->eb > 16;
    if (long_b || forced >= 0) {
      p->path = forced == LR_PATH_TRANSPOSE_DIRECT ? LR_PATH_TRANSPOSE_DIRECT : LR_PATH_TRANSPOSE;
      p->a = a;
      p->b = b;
      p->b2 = b2;
      p->v = (int)V;
      // source distance between nearby b rows
      const int64_t pitch = (b2 >= 0 ? std::min(p->m[b].ss, p->m[b2].ss) : p->m[b].ss) * p->eb;
      // tile shape in 16-byte chunks (a x b): wider tiles only for full chunks on
      // the LDS variant.  Measured with streaming (non-temporal) accesses, back to
      // back against every other shape:
      //  - when one tile spans the whole a extent and consecutive b rows are
      //    adjacent in the source (each tile reads one contiguous block, e.g.
      //    NHWC -> NCHW), 32 x 8 chunks: small workgroups, many per CU;
      //  - its mirror, one tile spanning the whole b extent of 17-32 chunks with
      //    consecutive a rows adjacent in the destination (each tile writes one
      //    contiguous block, e.g. NCHW -> NHWC with 256 fp16 channels), 8 x 32
      //    chunks: 67.6 against 72.7 us for 32 x 32 over 128 images of 56 x 56;
      //  - otherwise the longest runs on both sides, 32 x 32 chunks (16 x 32 when
      //    16 chunks already cover the a extent); 16 x 32 for 8-byte elements (two a
      //    chunk: 3.6 % faster than 32 x 16 over seven fp64 transposes from 2048 x
      //    8192 to 4096 x 16384, 10 % at best, 3 % slower at worst); 64 x 16 for
      //    16-byte elements (9 % faster than 16 x 16 over six transposes from 2048^2
      //    to 8192 x 2048, 5-13 % each); 1-byte elements in 8-byte chunks 32 x 16
      //    (level with 32 x 32 and 64 x 16 over six transposes, each ahead on some).
      const bool wide_ok = (V * p->eb == 16 || (p->eb == 1 && V == 8)) && p->path == LR_PATH_TRANSPOSE;
      const int64_t ext_a = p->m[a].ext;
      const bool block_rows = ext_a <= 32 * V && p->m[b].ss == ext_a;
      const bool block_cols =
          V * p->eb == 16 && b2 < 0 && ext_b > 16 * V && ext_b <= 32 * V && p->m[a].sd == ext_b;
      // the share of a tile's lanes with work in a shape, over both sides' ragged edges
      auto lane_share = [&](int s) {
        const int64_t ta = kTileTA[s] * V, tb = kTileTB[s] * V;
        return (double)ext_a / (double)(((ext_a + ta - 1) / ta) * ta) * (double)ext_b /
               (double)(((ext_b + tb - 1) / tb) * tb);
      };
      if (!wide_ok)
        p->tshape = 0;
      else if (block_rows && !(block_cols && lane_share(8) > lane_share(ext_a > 16 * V ? 4 : 0)))
        p->tshape = ext_a > 16 * V ? 4 : 0;
      else if (block_cols)  // whole matrices both ways take the shape with more lanes at work
        p->tshape = 8;      // (batched fp32 128 x 96: 65.5 against 70.4 us for 32 x 8)
      else if (p->eb == 1)
        p->tshape = ext_a > 16 * V ? 1 : 0;  // 8-byte chunks: 32 x 16 (u8 8192^2 4.78 against 4.56 with 32 x 32)
      else if (V >= 4)
        p->tshape = ext_a > 16 * V ? 3 : 2;
      else if (V == 2)
        p->tshape = 2;
      else
        p->tshape = ext_a > 32 ? 6 : 0;
      // A short destination-contiguous extent: no tile taller along b than it needs,
      // else most of a tile's lanes idle.  Measured on NCHW -> NHWC fp16 (256 images of
      // 112 x 112): 32 channels 145.0 -> 69.3 us with 32 x 8 chunks instead of 32 x 32,
      // 64 channels 189.1 -> 137.2 us.
      if (wide_ok && !block_rows) {
        const int64_t nbc = (ext_b + V - 1) / V;  // b extent in chunks
        if (nbc <= 8 && kTileTB[p->tshape] > 8)
          p->tshape = 4;
        else if (nbc <= 16 && kTileTB[p->tshape] > 16)
          p->tshape = ext_a > 16 * V ? 1 : 0;
      }
      // Fewer tiles than compute units (a 16 MiB transpose in 256 x 256 tiles is 128
      // workgroups): 32 x 8 chunks, four times as many workgroups.  Measured on
      // fp16 1024 x 8192 and 8192 x 1024, the 8-way shard pack of 1024 x 8192 and u8
      // 4096^2 in 16-byte chunks: +2 to +8 % (16 MiB copies run near a plain copy's
      // 3.2-3.6 TB/s).
      if (wide_ok && !block_rows && !block_cols) {
        int64_t tiles = ((ext_a + kTileTA[p->tshape] * V - 1) / (kTileTA[p->tshape] * V)) *
                        ((ext_b + kTileTB[p->tshape] * V - 1) / (kTileTB[p->tshape] * V));
        for (int k = 0; k < p->rank; ++k)
          if (k != a && k != b && k != b2) tiles *= p->m[k].ext;
        if (tiles < 256) p->tshape = 4;
      }
      if (tun.tile_shape >= 0) p->tshape = wide_ok ? tun.tile_shape : 0;
      // 16-element chunks (1-byte elements): the 32 x 32 and 64 x 16 tiles would
      // need 256 KiB of LDS; take the largest that fits
      if (!shape_fits(p->tshape, (int)V)) p->tshape = p->tshape == 6 ? 5 : 1;
      p->tile_a = kTileTA[p->tshape] * V;
      p->tile_b = kTileTB[p->tshape] * V;
      p->block = kTileTA[p->tshape] * kTileTB[p->tshape];
      // Rows that do not allow aligned 16-byte chunks (odd pitches, ragged extents):
      // element-granular tiles with 256-byte rows on both sides instead of narrow
      // chunks in small tiles.  Measured on fp16 8191^2: 1.13 -> 2.80 TB/s; it wins
      // for single elements of any size and for 2- to 8-byte elements in chunks of
      // up to 8 bytes; 1-byte elements in chunks of 2 take them too (through the
      // windowed kernel below), in chunks of 4 or 8 keep the chunks (u8 8188^2 2.55
      // TB/s against 2.22-2.36, 8184^2 2.96 against 2.25-2.39).
      const bool tel_wins = V <= 2 || p->eb >= 2;
      p->tel = p->path == LR_PATH_TRANSPOSE && V * p->eb < 16 && p->eb <= 8 &&
               (tun.element_tiles == 1 || (tun.element_tiles < 0 && tel_wins));
      if (p->tel) {
        p->v = 1;
        p->tshape = 0;
        p->tile_a = p->tile_b = 256 / p->eb;
        p->block = 512;
        // The windowed kernel (16-byte accesses inside each tile row) on element-aligned
        // buffers without swizzles, with ordinary (cached) accesses at every size: the
        // partial lines at the unaligned ends of the row segments then merge in L2.
        // Measured on odd-pitch squares and rectangles of 1- to 8-byte elements, from
        // 32 MiB to 512 MiB, against the per-element kernel with streaming accesses past
        // 128 MiB: fp16 8191^2 3.34 -> 4.10 TB/s, 12287^2 3.45 -> 4.16, 4097 x 16383
        // 2.78 -> 3.89; fp32 8191^2 3.22 -> 4.92; 8-byte 4095^2 3.57 -> 5.06; u8 16383^2
        // 2.08 -> 2.40.  Streaming accesses alone cost the per-element kernel 8-18 %.
        p->twin = !p->sw_s.b && !p->sw_d.b && src_align % (size_t)p->eb == 0 && dst_align % (size_t)p->eb == 0;
        if (!p->policy_set) p->nt = p->nt_ld = false;  // an explicit policy still applies
      }
      // Workgroup order (measured on fp16, fp32, 1-, 8- and 16-byte transposes from
      // 2048 x 32768 to 16384^2).  b-tiles fastest by default: consecutive
      // workgroups then write adjacent column blocks of the same destination rows
      // and read adjacent row bands of one source column strip.  With pitches that
      // are power-of-two heavy (a multiple of 16 KiB, or a power of two from 4 KiB)
      // the rows of such a strip, or of a tile band, share their low address bits
      // and the workgroups in flight camp on a few HBM channels (fp16 8192^2: 4.3
      // TB/s); a diagonal order then spreads them (5.6).  Of the two diagonals, the
      // one with b fastest (4) wins for tiles with equal row bytes on both sides
      // (fp16 16384^2: 6.33 against 6.20; 2048 x 32768: 5.49 against 4.70); the one
      // with a fastest (2) wins for tiles whose source rows are longer (1- and
      // 8-byte elements: 4.65 against 4.40 on 1-byte 8192^2) unless there are more
      // a-tiles than b-tiles, when its workgroups sharing a b-tile would read
      // columns a power-of-two distance apart.  Other pitches keep b fastest:
      // 11264^2 fp16 5.42 against 4.94 for the diagonal.  Chunk tiles whose pitch is
      // within 64 bytes of a multiple of 16 KiB take the diagonal too (fp16 8224^2 4.33
      // against 3.44, 8184^2 3.84 against 3.47, fp32 4100^2 3.91 against 3.66; 8200^2
      // 3.71 against 3.74).  Element tiles whose pitch lies up to 64 bytes past a
      // multiple of 8 KiB take the diagonal with b fastest (fp16 8193^2 3.80 against
      // 3.22, 8196^2 4.13 against 3.12, 12289^2 3.71 against 3.18; fp32 4097 x 8193 4.43
      // against 3.40), unless a pitch lies just short of one: 8191^2 takes a fastest (4.05
      // against 2.83), 16383 x 4097 b fastest (3.37 against 2.59).  Element tiles with at least
      // as many a-tiles as b-tiles take a fastest: fp32 8191^2 4.92 against 3.63, fp16
      // 12287^2 4.16 against 3.39, u8 4097 x 16383 2.15 against 1.58; the tall mirror
      // shapes lost with it (u8 16383 x 4097 1.93 against 2.28).
      {
        const int64_t pitch_d = p->m[a].sd * p->eb;
        auto pow2_heavy = [](int64_t q) { return q % 16384 == 0 || (q >= 4096 && (q & (q - 1)) == 0); };
        // chunk tiles: within 64 bytes of a multiple of 16 KiB behaves as a multiple
        auto near_16k = [](int64_t q) { return q >= 16384 - 64 && (q % 16384 <= 64 || q % 16384 >= 16384 - 64); };
        // element tiles: up to 64 bytes past a multiple of 8 KiB, unless the other pitch
        // is up to 64 bytes short of one
        auto past_8k = [](int64_t q) { return q >= 8192 && q % 8192 != 0 && q % 8192 <= 64; };
        auto short_8k = [](int64_t q) { return q >= 8192 - 64 && q % 8192 >= 8192 - 64; };
        const int64_t nta0 = (p->m[a].ext + p->tile_a - 1) / p->tile_a;
        const int64_t ntb0 = (ext_b + p->tile_b - 1) / p->tile_b;
        const bool camp = pow2_heavy(pitch) || pow2_heavy(pitch_d) ||
                          (!p->tel && (near_16k(pitch) || near_16k(pitch_d)));
        // chunk tiles whose pitches lie just past a multiple of 16 KiB (none on or
        // just short of one): the diagonal with a fastest, remeasured back to back
        // on eight transposes whose pitches are 16-64 bytes past one (fp16 8200^2
        // 67.1 against 71.5 us for the diagonal with b fastest, 16400^2 225.5 against
        // 235.6, fp32 8200^2 113.8 against 121.1; fastest or within 0.5 % of it on
        // seven, 1.3 % behind order 4 on fp32 4104 x 8200); on or just short of a
        // multiple the diagonal with b fastest stays ahead (fp16 8184^2 64.4 against 68.4).
        auto past_16k = [](int64_t q) { return q > 16384 && q % 16384 != 0 && q % 16384 <= 64; };
        const bool past_only = !p->tel && !pow2_heavy(pitch) && !pow2_heavy(pitch_d) &&
                               (past_16k(pitch) || !near_16k(pitch)) && (past_16k(pitch_d) || !near_16k(pitch_d));
        if (nta0 > 1 && camp && past_only)
          p->torder = 2u;
        else if (nta0 > 1 && camp)
          p->torder = (p->tile_a > p->tile_b && nta0 <= ntb0) ? 2u : 4u;
        else if (nta0 > 1 && p->eb == 1 && !p->tel && p->v == 8 && p->tile_a > p->tile_b && nta0 <= ntb0)
          p->torder = 2u;  // 1-byte elements in 8-byte chunks: the diagonal at any pitch (u8 6144^2 4.07 against 3.73)
        else if (nta0 > 1 && p->tel && (past_8k(pitch) || past_8k(pitch_d)) && !short_8k(pitch) && !short_8k(pitch_d))
          p->torder = 4u;
        else if (p->tel && nta0 >= ntb0)
          p->torder = 0u;  // element tiles, at least as many a-tiles as b-tiles: a fastest
        else
          p->torder = 1u;  // (with a single a-tile, order 4 is order 1)
      }
      if (tun.tile_order >= 0) p->torder = (uint32_t)tun.tile_order;
      // direct global -> LDS loads: full chunks, tiles 16 or 32 chunks wide along a
      // and at least 16 along b
      p->direct = tun.direct_loads == 1 && p->path == LR_PATH_TRANSPOSE && V * p->eb == 16 &&
                  p->tshape <= 3 && shape_fits(p->tshape, (int)V);
      // Streaming stores of the LDS tile transpose go out as buffer stores with the
      // nt and sc1 cache-policy bits: fp16 8192^2 5.62 -> 5.67 TB/s, the column-major
      // head interleave 6.19 -> 6.35, NHWC -> NCHW 6.03 -> 6.11, fp32 8192^2 6.07 ->
      // 6.26 (the interleave and staged kernels measured slower with them, 1-1.5 %).
      // Buffer offsets are 32-bit: each workgroup stores relative to its tile's
      // lowest destination offset, so the tile's destination span must stay under
      // 4 GiB.
      {
        // rounding the base down and swizzling the highest offset up each add less
        // than one swizzle block (2^(M+B) elements)
        const int64_t swz_blk = p->sw_d.b ? (int64_t(1) << (p->sw_d.m + p->sw_d.b)) : 0;
        const int64_t span = ((p->tile_a - 1) * p->m[a].sd + p->tile_b + 2 * swz_blk) * p->eb;
        p->bufst = p->path == LR_PATH_TRANSPOSE && !p->tel && !p->direct && V * p->eb == 16 &&
                   span < (int64_t(1) << 32) && sc1_ok;
      }
      const int64_t nta = (p->m[a].ext + p->tile_a - 1) / p->tile_a;
      const int64_t ntb = (ext_b + p->tile_b - 1) / p->tile_b;
      if (p->torder % 5 == 3 && (nta % 4 || ntb % 4)) p->torder -= 1;  // grouped order needs 4 | tiles
      int64_t batch = 1;
      for (int k = 0; k < p->rank; ++k)
        if (k != a && k != b && k != b2) batch *= p->m[k].ext;
      p->grid = nta * ntb * batch;
      p->tiles_total = p->grid;
      // software pipelining over two LDS tiles (tile shapes whose exchange fits twice):
      // a workgroup takes pipeline_tiles consecutive tiles in the chosen order
      if (tun.pipeline_tiles >= 2 && p->path == LR_PATH_TRANSPOSE && !p->tel && V * p->eb == 16 &&
          pipe_fits(p->tshape, (int)V)) {
        p->pipe = tun.pipeline_tiles;
        p->direct = true;
        p->bufst = false;
        p->grid = (p->tiles_total + p->pipe - 1) / p->pipe;
        if (p->torder >= 5) p->torder -= 5;  // XCD grouping renumbers workgroups, not tiles
      }
      // gfx950 transpose reads of the LDS tile: 1- or 2-byte elements in 16-byte
      // chunks, tiles 16 or 32 chunks on each side, loaded directly (or pipelined)
      if (tun.transpose_reads == 1 && p->path == LR_PATH_TRANSPOSE && !p->tel && p->eb <= 2 && V * p->eb == 16 &&
          p->tshape <= 3 && (p->direct || p->pipe)) {
        p->tr = true;
        p->bufst = false;
      }
      // two register blocks per lane (half the lanes for the same tile) on the
      // register-loaded LDS transpose.  Taken for 1024-lane tiles of 2-byte elements:
      // back to back, the fp16 8192^2 transpose 46.2-47.2 against 47.1-47.7 us over
      // three runs, fp16 16384^2 and the bf16 KV-cache reorder 0.5-1 % faster; 4-byte
      // elements and smaller tiles lose 1-5 %.
      const bool two_blocks = tun.transpose_blocks >= 0
                                  ? tun.transpose_blocks == 2
                                  : p->eb == 2 && kTileTA[p->tshape] * kTileTB[p->tshape] == 1024;
      if (two_blocks && p->path == LR_PATH_TRANSPOSE && !p->tel && !p->direct && !p->pipe &&
          (V * p->eb == 16 || (p->eb == 1 && V == 8)) && kTileTB[p->tshape] % 2 == 0 &&
          kTileTA[p->tshape] * kTileTB[p->tshape] >= 128) {  // whole wavefronts
        p->tblocks = 2;
        p->block = kTileTA[p->tshape] * kTileTB[p->tshape] / 2;
      }
      // Small matrices in a batch (a whole matrix at most a quarter of the tile): the
      // staged path where it applies, which moves each compact matrix as one block,
      // else (under a quarter) the batched path.  Measured on batched fp16 transposes:
      // 32 x 32 115.6 -> 49.6 us, 16 x 16 406.6 -> 68.6 us (fp32 32 x 32, a quarter of
      // its tile, ties: 46.1 us; fp64 16 x 16, a quarter too, 58.8 -> 45.6 us); over 2^26
      // 4-byte and 2^25 8-byte elements the staged path beats the batched one (fp32 8 x 8
      // 45.4 against 46.6 us, 16 x 16 45.6 against 46.2, 32 x 32 45.0 against 46.8, fp64
      // 16 x 16 45.7 against 46.1).
      if (forced < 0 && tun.tile_shape < 0 && !p->tel) {
        const int64_t fa = std::min<int64_t>(p->m[a].ext, p->tile_a), fb = std::min<int64_t>(ext_b, p->tile_b);
        Plan st = before_transpose;
        if (4 * fa * fb <= p->tile_a * p->tile_b && plan_staged(&st, b, src_align, dst_align, src_cap, tun)) {
          *p = st;
          return LR_OK;
        }
        // (a matrix of exactly a quarter keeps the transpose: fp16 64 x 64 48.6 us
        // against 50.2 batched)
        if (4 * fa * fb < p->tile_a * p->tile_b && bt_ok && b2 < 0) {
          *p = batched;
          batched_swizzle(p, tun);
          return LR_OK;
        }
      }
      return LR_OK;
    }
  }
  if (forced == LR_PATH_TRANSPOSE || forced == LR_PATH_TRANSPOSE_DIRECT) return LR_ERR_PATH;

  // staged: a compact dst block of inner modes whose source footprint is small
  if (forced < 0 || forced == LR_PATH_STAGED) {
    if (plan_staged(p, b, src_align, dst_align, src_cap, tun)) return LR_OK;
    if (forced == LR_PATH_STAGED) return LR_ERR_PATH;
  }

  // few channels whose planes have no whole 16-byte chunks (odd image sizes): the
  // element-granular channel shuffle, given at least one pixel per lane.  Measured
  // on 299^2 and 331^2 images with 2 to 8 channels, both directions, against the
  // generic kernel: fp16 RGB 4.3-4.8 TB/s against 1.4-1.5, 1-byte RGB 4.3-4.6
  // against 0.8, fp32 RGB 5.4-5.7 against 2.3-2.6, fp16 with four channels 3.8-4.2
  // against 1.4-1.6, 8-byte pairs 4.9-5.1 against 4.0-4.3.
  if (forced < 0 && a >= 0 && b >= 0 && a != b) {
    if (p->m[a].ext >= 256 && plan_chan_elements(p, a, b, true, src_align, dst_align)) return LR_OK;
    if (p->m[b].ext >= 256 && plan_chan_elements(p, a, b, false, src_align, dst_align)) return LR_OK;
  }

  // generic: one unit per lane over the (fused) joint modes
  if (forced >= 0 && forced != LR_PATH_GENERIC) return LR_ERR_PATH;
  p->path = LR_PATH_GENERIC;
  p->a = p->b = -1;
  int64_t v = unit_width(*p, src_align, dst_align);
  p->v = (int)v;
  int64_t ne = 1;
  for (int k = 0; k < p->rank; ++k) ne *= p->m[k].ext;
  p->n_units = ne / v;
  p->block = (p->unroll == 1 && !p->wide) ? knob(tun.workgroup_lanes, stream_lanes(*p, big_footprint)) : 256;
  p->grid = (p->n_units + p->block * p->unroll - 1) / (p->block * p->unroll);
  // 16-byte units (fused elements) take the vector path's buffer stores too
  p->bufst = v * p->eb == 16 && p->unroll == 1 && !p->wide && sc1_ok && dst_span_bytes(*p) < (int64_t(1) << 32);
  return LR_OK;
}

static int plan_uncached(const lr_layout* Ls, int64_t src_cap, size_t src_align, const lr_layout* Ld,
                         int64_t dst_cap, size_t dst_align, size_t elem_bytes, uint32_t flags,
                         const lr_copy_tuning& tun, Plan* p) {
  const int rc = plan_path(Ls, src_cap, src_align, Ld, dst_cap, dst_align, elem_bytes, flags, tun, p);
  if (rc) return rc;
  // different load and store policies: the generic kernel only
  if (p->nt_ld != p->nt && p->path != LR_PATH_GENERIC && p->path != LR_PATH_VECTOR) return LR_ERR_PATH;
  if (p->path != LR_PATH_GENERIC && p->path != LR_PATH_VECTOR) p->vorder = -1;
  if (p->path != LR_PATH_STAGED) p->staged_cps = -1;
  return LR_OK;
}

// The planner's inputs as a flat key: the layouts' defined fields, capacities,
// alignments as the planner reads them (the lowest set bit, at most 16), element
// size, flags and tuning.
static void plan_key(const lr_layout* L, std::vector<int64_t>* k) {
  k->push_back(L->nleaves);
  k->push_back(L->nmodes);
  for (int i = 0; i < L->nleaves && i < LR_MAX_LEAVES; ++i) {
    k->push_back(L->shape[i]);
    k->push_back(L->stride[i]);
  }
  for (int i = 0; i < L->nmodes && i < LR_MAX_LEAVES; ++i) k->push_back(L->mode_end[i]);
  k->push_back(L->swz_b);
  k->push_back(L->swz_m);
  k->push_back(L->swz_s);
}

// Plans are kept per thread for the last 32 distinct inputs: the same copy issued
// again (a training step, a serving loop) skips the planner, whose bank-model
// searches take tens of microseconds, as long as a small copy's kernel.
int plan_copy(const lr_layout* Ls, int64_t src_cap, size_t src_align, const lr_layout* Ld, int64_t dst_cap,
              size_t dst_align, size_t elem_bytes, uint32_t flags, const lr_copy_tuning* tuning, Plan* p) {
  lr_copy_tuning tun;
  lr_copy_tuning_init(&tun);
  if (tuning) {
    if (!tuning_valid(*tuning)) return LR_ERR_INVALID;
    tun = *tuning;
  }
  if (Ls->nleaves < 1 || Ls->nleaves > LR_MAX_LEAVES || Ld->nleaves < 1 || Ld->nleaves > LR_MAX_LEAVES)
    return plan_uncached(Ls, src_cap, src_align, Ld, dst_cap, dst_align, elem_bytes, flags, tun, p);
  auto norm = [](size_t a) -> int64_t { return a == 0 ? 1 : (int64_t)std::min<size_t>(a & (~a + 1), 16); };
  std::vector<int64_t> key;
  key.reserve(160);
  plan_key(Ls, &key);
  plan_key(Ld, &key);
  key.push_back(src_cap);
  key.push_back(dst_cap);
  key.push_back(norm(src_align));
  key.push_back(norm(dst_align));
  key.push_back((int64_t)elem_bytes);
  key.push_back(flags);
  const int32_t* t = (const int32_t*)&tun;
  for (size_t i = 0; i < sizeof(tun) / sizeof(int32_t); ++i) key.push_back(t[i]);
  struct Entry {
    std::vector<int64_t> key;
    Plan plan;
    int rc;
  };
  thread_local std::array<Entry, 32> cache;
  thread_local int next = 0;
  for (const Entry& e : cache)
    if (e.key == key) {
      if (e.rc == LR_OK) *p = e.plan;
      return e.rc;
    }
  const int rc = plan_uncached(Ls, src_cap, src_align, Ld, dst_cap, dst_align, elem_bytes, flags, tun, p);
  Entry& e = cache[next];
  next = (next + 1) % 32;
  e.key = std::move(key);
  e.rc = rc;
  if (rc == LR_OK) e.plan = *p;
  return rc;
}

// Re-checks, independently of the choices above, the invariants each kernel's
// indexing relies on; a violation means a planner bug and nothing is launched.
int verify_plan(const Plan& p, int64_t src_cap, int64_t dst_cap) {
  auto bad = [] { return LR_ERR_PATH; };
  if (p.bufst && p.path != LR_PATH_GENERIC && p.path != LR_PATH_VECTOR && p.path != LR_PATH_TRANSPOSE &&
      p.path != LR_PATH_INTERLEAVE && p.path != LR_PATH_DEINTERLEAVE)
    return bad();
  if (p.nt_ld != p.nt && p.path != LR_PATH_GENERIC && p.path != LR_PATH_VECTOR) return bad();
  if (p.path == LR_PATH_DUAL || p.path == LR_PATH_ALIAS) return LR_OK;  // evaluate the validated layouts
  if (p.rank < 1 || p.rank > kMaxKernelModes) return bad();
  int64_t ms = 0, md = 0, prod = 1;
  for (int k = 0; k < p.rank; ++k) {
    if (p.m[k].ext < 1 || p.m[k].ss < 0 || p.m[k].sd < 0) return bad();
    ms += (p.m[k].ext - 1) * p.m[k].ss;
    md += (p.m[k].ext - 1) * p.m[k].sd;
    prod *= p.m[k].ext;
  }
  // bytes touched on each side (strides are in fused elements of p.eb bytes;
  // capacities in elements of the caller's elem_bytes)
  auto bound = [](int64_t m, const Swz& z) {
    return z.b ? (m | ((int64_t(1) << (z.m + z.b)) - 1)) + 1 : m + 1;
  };
  if (bound(ms, p.sw_s) * p.eb > src_cap * p.orig_eb) return bad();
  if (bound(md, p.sw_d) * p.eb > dst_cap * p.orig_eb) return bad();
  const int64_t v = p.v;
  if (v < 1 || v * p.eb > 16) return bad();
  switch (p.path) {
    case LR_PATH_GENERIC:
    case LR_PATH_VECTOR:
      if (v > 1) {
        if (p.m[0].ss != 1 || p.m[0].sd != 1 || p.m[0].ext % v) return bad();
        for (int k = 1; k < p.rank; ++k)
          if (p.m[k].ss % v || p.m[k].sd % v) return bad();
      }
      if (p.n_units * v != prod) return bad();
      // workgroup lanes: 64, 128 or 256 for one unit per lane with 32-bit indices (and
      // for the tiles of atoms)
      if (p.block != 256 && !((p.block == 64 || p.block == 128) && p.unroll == 1 && !p.wide)) return bad();
      if (p.vorder == 3) {  // tiles of atoms: see atom_tiles
        int a = -1, b = -1;
        int64_t T = 0;
        if (!atom_tiles(p, &a, &b, &T) || a != p.a || b != p.b || p.tile_a != T || p.tile_b != T) return bad();
        int64_t batch = 1;
        for (int k = 1; k < p.rank; ++k)
          if (k != a && k != b) batch *= p.m[k].ext;
        if (p.grid != ((p.m[a].ext + T - 1) / T) * ((p.m[b].ext + T - 1) / T) * batch || p.grid > 0x7FFFFFFF)
          return bad();
      }
      // buffer stores: one 32-bit byte offset from the destination base
      if (p.bufst && (v * p.eb != 16 || p.unroll != 1 || p.wide || (bound(md, p.sw_d) * p.eb >> 32) != 0))
        return bad();
      return LR_OK;
    case LR_PATH_TRANSPOSE:
    case LR_PATH_TRANSPOSE_DIRECT: {
      if (p.a < 0 || p.b < 0 || p.a == p.b || p.a >= p.rank || p.b >= p.rank) return bad();
      if (p.b2 >= p.rank || p.b2 == p.a || p.b2 == p.b) return bad();
      if (p.m[p.a].ss != 1 || p.m[p.b].sd != 1) return bad();
      int64_t ext_b = p.m[p.b].ext;
      if (p.b2 >= 0) {
        const int64_t e0 = p.m[p.b].ext;
        if ((e0 & (e0 - 1)) || p.m[p.b2].sd != e0) return bad();
        ext_b *= p.m[p.b2].ext;
      }
      if (p.m[p.a].ext % v || ext_b % v) return bad();
      if (p.tshape < 0 || p.tshape >= kTileShapes ||
          (p.tshape != 0 && ((v * p.eb != 16 && !(p.eb == 1 && v == 8)) || !shape_fits(p.tshape, (int)v) ||
                             p.path != LR_PATH_TRANSPOSE)))
        return bad();
      if (p.torder > 9 || (p.torder >= 5 && p.pipe)) return bad();  // XCD grouping: one tile per workgroup
      if (p.bufst) {  // buffer stores: full chunks of the LDS kernel, tile span under 4 GiB
        const int64_t swz_blk = p.sw_d.b ? (int64_t(1) << (p.sw_d.m + p.sw_d.b)) : 0;
        const int64_t span = ((p.tile_a - 1) * p.m[p.a].sd + p.tile_b + 2 * swz_blk) * p.eb;
        if (p.path != LR_PATH_TRANSPOSE || p.tel || p.direct || v * p.eb != 16 || span >= (int64_t(1) << 32))
          return bad();
      }
      // direct-load kernel: full 16-byte chunks, tiles 16 or 32 chunks along a, >= 16 along b
      if (p.direct && (p.path != LR_PATH_TRANSPOSE || v * p.eb != 16 || p.tshape > 3 || !shape_fits(p.tshape, (int)v)))
        return bad();
      // two register blocks per lane: the register-loaded LDS kernel, whole block rows per lane group
      if (p.tblocks == 2 &&
          (p.path != LR_PATH_TRANSPOSE || p.tel || p.direct || p.pipe || kTileTB[p.tshape] % 2 ||
           (v * p.eb != 16 && !(p.eb == 1 && v == 8)) || p.block != kTileTA[p.tshape] * kTileTB[p.tshape] / 2 ||
           p.block < 64))
        return bad();
      if (p.tblocks != 0 && p.tblocks != 1 && p.tblocks != 2) return bad();
      if (p.tel) {  // element-granular tiles of 256-byte rows
        if (p.path != LR_PATH_TRANSPOSE || p.eb > 8 || v != 1 || p.direct || p.tile_a != 256 / p.eb ||
            p.tile_b != 256 / p.eb || p.block != 512)
          return bad();
        if (p.twin && (p.sw_s.b || p.sw_d.b)) return bad();  // rows: contiguous ranges
      } else if (p.twin || p.tile_a != kTileTA[p.tshape] * v || p.tile_b != kTileTB[p.tshape] * v) {
        return bad();
      }
      const int64_t nta = (p.m[p.a].ext + p.tile_a - 1) / p.tile_a, ntb = (ext_b + p.tile_b - 1) / p.tile_b;
      if (p.torder % 5 == 3 && (nta % 4 || ntb % 4)) return bad();
      // one workgroup per tile and batch index, all launched (no grid cap)
      int64_t batch = 1;
      for (int k = 0; k < p.rank; ++k)
        if (k != p.a && k != p.b && k != p.b2) batch *= p.m[k].ext;
      if (p.tiles_total != nta * ntb * batch || p.grid > 0x7FFFFFFF) return bad();
      if (p.pipe) {  // pipelined: full chunks, tile shapes 0-2, direct loads into two LDS tiles
        if (p.pipe < 2 || p.pipe > 64 || p.path != LR_PATH_TRANSPOSE || p.tel || v * p.eb != 16 ||
            !pipe_fits(p.tshape, (int)v) ||
            !p.direct || p.bufst || p.grid != (p.tiles_total + p.pipe - 1) / p.pipe)
          return bad();
      } else if (p.grid != p.tiles_total) {
        return bad();
      }
      if (p.tr) {  // transpose reads: 16-byte chunks of 1- or 2-byte elements, direct loads, shapes 0-3
        if (p.path != LR_PATH_TRANSPOSE || p.tel || p.eb > 2 || v * p.eb != 16 || p.tshape > 3 || !p.direct ||
            p.bufst)
          return bad();
      }
      for (int k = 0; k < p.rank; ++k) {
        if (k != p.a && p.m[k].ss % v) return bad();
        if (k != p.b && k != p.b2 && p.m[k].sd % v) return bad();
      }
      return LR_OK;
    }
    case LR_PATH_INTERLEAVE: {
      if (p.a < 0 || p.b < 0 || p.a == p.b || p.a >= p.rank || p.b >= p.rank) return bad();
      const int64_t nb = p.m[p.b].ext;
      if (p.m[p.a].ss != 1 || p.m[p.b].sd != 1 || p.m[p.a].sd != nb || p.tile_b != nb) return bad();
      if (p.inarrow == 3) {  // element-granular channel shuffle: no chunk conditions
        if (!chan_supported(p.eb, nb) || p.sw_s.b || p.sw_d.b || v != 1 || p.bufst ||
            p.tile_a != chan_el_pixels(p.eb))
          return bad();
        return LR_OK;
      }
      if (v * p.eb != 16 || p.m[p.a].ext % v || nb * p.eb > 16) return bad();
      // the kernel's per-lane unroll
      if (p.inarrow == 2) {  // channel shuffle: any NB it was built for, no swizzle
        if (!chan_supported(p.eb, nb) || p.sw_s.b || p.sw_d.b || p.tile_a != p.block * v ||
            (p.block != 64 && p.block != 128 && p.block != 256))
          return bad();
      } else if (!is_pow2(nb) || p.tile_a != (p.inarrow ? p.block * (v / nb) : (nb >= 8 ? 1 : 8 / nb) * 256 * v) ||
                 (p.block != 256 && !(p.inarrow == 1 && (p.block == 64 || p.block == 128)))) {
        return bad();
      }
      if (p.bufst && (!p.inarrow || (bound(md, p.sw_d) * p.eb >> 32) != 0)) return bad();
      for (int k = 0; k < p.rank; ++k) {
        if (k != p.a && p.m[k].ss % v) return bad();
        if (k != p.a && k != p.b && p.m[k].sd % v) return bad();
      }
      return LR_OK;
    }
    case LR_PATH_DEINTERLEAVE: {
      if (p.a < 0 || p.b < 0 || p.a == p.b || p.a >= p.rank || p.b >= p.rank) return bad();
      const int64_t C = p.m[p.a].ext;
      if (p.m[p.a].ss != 1 || p.m[p.b].sd != 1 || p.m[p.b].ss != C || !chan_supported(p.eb, C)) return bad();
      if (v == 1)  // element-granular form
        return (p.sw_s.b || p.sw_d.b || p.bufst ||
                p.tile_a != chan_el_pixels(p.eb) || p.tile_b != C)
                   ? bad()
                   : LR_OK;
      if (v * p.eb != 16 || p.m[p.b].ext % v || p.m[p.a].sd % v || p.sw_s.b || p.sw_d.b) return bad();
      if (p.bufst && (dst_span_bytes(p) >> 32) != 0) return bad();
      if (p.tile_a != p.block * v || p.tile_b != C || (p.block != 64 && p.block != 128 && p.block != 256)) return bad();
      for (int k = 0; k < p.rank; ++k)
        if (k != p.a && k != p.b && (p.m[k].ss % v || p.m[k].sd % v)) return bad();
      return LR_OK;
    }
    case LR_PATH_BATCHED: {
      if (p.a < 0 || p.b < 0 || p.a == p.b || p.a >= p.rank || p.b >= p.rank) return bad();
      if (p.eb != 2 && p.eb != 4 && p.eb != 8) return bad();
      const int64_t A = p.m[p.a].ext, B = p.m[p.b].ext;
      if (v * p.eb != 16 || p.m[p.a].ss != 1 || p.m[p.b].sd != 1 || p.m[p.b].ss != A || p.m[p.a].sd != B ||
          A % v || B % v || A * B * p.eb > 8192 || p.sw_s.b || p.sw_d.b || p.bufst || !p.direct)
        return bad();
      int64_t count = 1;
      for (int k = 0; k < p.rank; ++k) {
        if (k == p.a || k == p.b) continue;
        if (p.m[k].ss % v || p.m[k].sd % v) return bad();
        count *= p.m[k].ext;
      }
      const int64_t cpm = A * B / v;
      if (p.bt_count != count || p.bt_mpw != 512 / cpm || p.bt_mpw < 1) return bad();
      if (p.grid != (count + p.bt_mpw - 1) / p.bt_mpw || p.grid > 0x7FFFFFFF || p.block != 64) return bad();
      // the swizzle only permutes chunks inside aligned groups of 16 and is an
      // involution: checked over two whole regions
      if (p.bt_order < 0 || p.bt_order > 1) return bad();
      for (int i = 0; i < 6; ++i)
        if (p.bt_sw[i] < 0 || p.bt_sw[i] > 15) return bad();
      auto swz = [&](int64_t c) {
        return c ^ (((c >> p.bt_sw[0]) & p.bt_sw[1]) << p.bt_sw[2]) ^ (((c >> p.bt_sw[3]) & p.bt_sw[4]) << p.bt_sw[5]);
      };
      for (int64_t c = 0; c < 1024; ++c)
        if (swz(swz(c)) != c || (swz(c) >> 4) != (c >> 4)) return bad();
      return LR_OK;
    }
    case LR_PATH_STAGED: {
      const int in = p.staged_inner;
      if (in < 1 || in >= p.rank || v * p.eb != 16) return bad();
      int64_t P = 1, F = 1;
      for (int k = 0; k < in; ++k) {
        if (p.m[k].sd != P) return bad();
        P *= p.m[k].ext;
        F += (p.m[k].ext - 1) * p.m[k].ss;
      }
      if (P != p.staged_P || F != p.staged_F || p.m[in].sd != P) return bad();
      if (p.staged_Fc * 16 < F * p.eb || p.staged_cpt * 16 != P * p.eb || 256 % p.staged_cpt) return bad();
      if (p.staged_K < 1 || p.staged_K * p.staged_Fc * 16 > 65536) return bad();
      if ((p.block != 64 && p.block != 128 && p.block != 256) || p.block < p.staged_cpt) return bad();
      {  // gather grouping: cps | cpt, cps | 32, cpt / cps | block / 32, and whole slices of tiles
        const int64_t cps = p.staged_cps;
        if (cps < 1 || cps > 32 || (cps & (cps - 1)) || p.staged_cpt % cps || (p.block / 32) % (p.staged_cpt / cps) ||
            (cps != std::min<int64_t>(p.staged_cpt, 32) && p.staged_K % (32 / cps)))
          return bad();
      }
      int64_t maxbase = 0;
      for (int k = in; k < p.rank; ++k) {
        if ((p.m[k].ss * p.eb) % 16 || (p.m[k].sd * p.eb) % 16) return bad();
        maxbase += (p.m[k].ext - 1) * p.m[k].ss;
      }
      if ((maxbase * p.eb + p.staged_Fc * 16) > src_cap * p.orig_eb) return bad();
      return LR_OK;
    }
  }
  return bad();
}

bool block_extents(const Plan& p, uint32_t flags, int64_t* cext, int64_t* nblocks) {
  if (!p.wide || (flags & (LR_COPY_WIDE_INDEX | 0xFF00u)) || p.path == LR_PATH_DUAL || p.path == LR_PATH_ALIAS)
    return false;
  if (p.sw_s.b || p.sw_d.b || p.rank < 1) return false;  // a base offset would move the swizzle's bits
  const int64_t lim = int64_t(1) << 31;
  for (int k = 0; k < p.rank; ++k) cext[k] = p.m[k].ext;
  for (;;) {
    int64_t n = 1, rs = 0, rd = 0;
    for (int k = 0; k < p.rank; ++k) {
      n *= cext[k];
      rs += (cext[k] - 1) * p.m[k].ss;
      rd += (cext[k] - 1) * p.m[k].sd;
    }
    if (n < lim && rs < lim - 1 && rd < lim - 1) break;
    // halve the mode reaching furthest on either side (by count when strides are 0)
    int best = -1;
    int64_t reach = -1;
    for (int k = 0; k < p.rank; ++k) {
      if (cext[k] < 2) continue;
      const int64_t r = (cext[k] - 1) * std::max<int64_t>(1, std::max(p.m[k].ss, p.m[k].sd));
      if (r > reach) {
        reach = r;
        best = k;
      }
    }
    if (best < 0) return false;
    const int64_t c = cext[best], h = (c + 1) / 2;
    // keep block starts on multiples of 64 elements (vector units and tiles stay whole)
    cext[best] = c > 128 ? (h + 63) / 64 * 64 : h;
  }
  int64_t nb = 1;
  for (int k = 0; k < p.rank; ++k) {
    nb *= (p.m[k].ext + cext[k] - 1) / cext[k];
    if (nb > 65536) return false;
  }
  if (nb < 2) return false;
  *nblocks = nb;
  return true;
}

void inherit_policy(const Plan& whole, Plan* blk) {
  const bool plain = blk->path == LR_PATH_DUAL || blk->path == LR_PATH_ALIAS;
  blk->nt = whole.nt && !plain;
  blk->nt_ld = whole.nt_ld && !plain;
  if (blk->nt_ld != blk->nt && blk->path != LR_PATH_GENERIC && blk->path != LR_PATH_VECTOR) blk->nt_ld = blk->nt;
}

void make_block(const Plan& p, const int64_t* cext, const int64_t* start, lr_layout* ls, lr_layout* ld,
                int64_t* src_off, int64_t* dst_off) {
  std::memset(ls, 0, sizeof(*ls));
  std::memset(ld, 0, sizeof(*ld));
  ls->nleaves = ld->nleaves = ls->nmodes = ld->nmodes = p.rank;
  int64_t os = 0, od = 0;
  for (int k = 0; k < p.rank; ++k) {
    const int64_t e = std::min(cext[k], p.m[k].ext - start[k]);
    ls->shape[k] = ld->shape[k] = e;
    ls->stride[k] = p.m[k].ss;
    ld->stride[k] = p.m[k].sd;
    ls->mode_end[k] = ld->mode_end[k] = k + 1;
    os += start[k] * p.m[k].ss;
    od += start[k] * p.m[k].sd;
  }
  *src_off = os;
  *dst_off = od;
}

}  // namespace lr

using namespace lr;

extern "C" {

void lr_copy_tuning_init(lr_copy_tuning* t) {
  if (!t) return;
  t->load_policy = t->store_policy = t->units_per_lane = t->vector_order = t->interleave_form = -1;
  t->tile_shape = t->tile_order = t->element_tiles = t->direct_loads = t->gather_chunks = t->pipeline_tiles = -1;
  t->transpose_reads = -1;
  t->chunk_bytes = -1;
  t->batch_swizzle = -1;
  t->batch_order = -1;
  t->workgroup_lanes = -1;
  t->transpose_blocks = -1;
}

int lr_copy_plan(const lr_layout* Ls, int64_t src_capacity_elems, size_t src_align, const lr_layout* Ld,
                 int64_t dst_capacity_elems, size_t dst_align, size_t elem_bytes, uint32_t flags, lr_plan* out) {
  return lr_copy_plan_tuned(Ls, src_capacity_elems, src_align, Ld, dst_capacity_elems, dst_align, elem_bytes, flags,
                            nullptr, out);
}

int lr_copy_plan_tuned(const lr_layout* Ls, int64_t src_capacity_elems, size_t src_align, const lr_layout* Ld,
                       int64_t dst_capacity_elems, size_t dst_align, size_t elem_bytes, uint32_t flags,
                       const lr_copy_tuning* tuning, lr_plan* out) {
  if (!out) return LR_ERR_INVALID;
  Plan p;
  int rc = plan_copy(Ls, src_capacity_elems, src_align, Ld, dst_capacity_elems, dst_align, elem_bytes, flags, tuning,
                     &p);
  if (rc) return rc;
  if ((rc = verify_plan(p, src_capacity_elems, dst_capacity_elems))) return rc;
  std::memset(out, 0, sizeof(*out));
  out->blocks = 1;
  int64_t cext[kMaxJoint], nblocks = 0;
  if (block_extents(p, flags, cext, &nblocks)) {
    // report the first block's plan (it starts at offset 0 on both sides)
    int64_t start[kMaxJoint] = {0}, os = 0, od = 0;
    lr_layout ls, ld;
    make_block(p, cext, start, &ls, &ld, &os, &od);
    Plan pb;
    if ((rc = plan_copy(&ls, cosize_bound(&ls), src_align, &ld, cosize_bound(&ld), dst_align, elem_bytes, flags,
                        tuning, &pb)))
      return rc;
    if (pb.wide) return LR_ERR_PATH;
    inherit_policy(p, &pb);
    if ((rc = verify_plan(pb, cosize_bound(&ls), cosize_bound(&ld)))) return rc;
    pb.n = p.n;
    pb.rank = p.rank;
    std::memcpy(pb.m, p.m, sizeof(p.m));
    out->blocks = nblocks;
    p = pb;
  }
  out->path = p.path;
  out->elem_bytes = p.eb;
  out->vec_elems = p.v;
  out->wide = p.wide ? 1 : 0;
  out->joint_rank = p.rank;
  out->a_mode = p.a;
  out->b_mode = p.b;
  out->b2_mode = p.b2;
  out->block = p.block;
  out->streaming = p.nt ? 1 : 0;
  out->order = (p.path == LR_PATH_TRANSPOSE || p.path == LR_PATH_TRANSPOSE_DIRECT) ? (int32_t)p.torder : -1;
  out->direct = p.direct ? 1 : 0;
  out->load_policy = p.nt_ld ? 2 : 0;
  out->store_policy = p.nt ? (p.bufst ? 18 : 2) : 0;
  out->vector_order = p.vorder;
  out->gather_chunks = (int32_t)p.staged_cps;
  out->pipeline_tiles = p.pipe;
  out->transpose_reads = p.tr ? 1 : 0;
  const bool bt = p.path == LR_PATH_BATCHED;
  out->batch_matrices = bt ? (int32_t)p.bt_mpw : -1;
  for (int i = 0; i < 6; ++i) out->batch_swizzle[i] = bt ? p.bt_sw[i] : 0;
  out->batch_order = bt ? p.bt_order : -1;
  out->tile_a = p.tile_a;
  out->tile_b = p.tile_b;
  out->grid = p.grid;
  out->n_elems = p.n;
  for (int k = 0; k < p.rank && k < 2 * LR_MAX_LEAVES; ++k) {
    out->ext[k] = p.m[k].ext;
    out->s_src[k] = p.m[k].ss;
    out->s_dst[k] = p.m[k].sd;
  }
  return LR_OK;
}

int lr_max_common_vector(const lr_layout* src, const lr_layout* dst, size_t elem_bytes, int64_t* elems) {
  int rc;
  if ((rc = validate(src))) return rc;
  if ((rc = validate(dst))) return rc;
  if (!elems) return LR_ERR_INVALID;
  if (!(elem_bytes == 1 || elem_bytes == 2 || elem_bytes == 4 || elem_bytes == 8 || elem_bytes == 16))
    return LR_ERR_ELEM_BYTES;
  if (size_of(src) != size_of(dst)) return LR_ERR_SIZE_MISMATCH;
  *elems = 1;
  if (!injective(dst)) return LR_OK;
  Plan p;
  std::memset(&p, 0, sizeof(p));
  p.eb = (int)elem_bytes;
  p.sw_s = {src->swz_b, src->swz_m, src->swz_s};
  p.sw_d = {dst->swz_b, dst->swz_m, dst->swz_s};
  int rank = 0;
  if (!joint_flat(src, dst, p.m, &rank, true)) return LR_OK;
  p.rank = rank;
  *elems = unit_width(p, 16, 16);
  return LR_OK;
}

}  // extern "C"
