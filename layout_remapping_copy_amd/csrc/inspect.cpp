// Host-side inspection of layouts: the printed grid, the thread-to-offset table
// and the access check of one wavefront (LDS bank cycles, adjacency of lane
// offsets, cache lines touched).  Plain C++17; no device code.
//
// Pages cited (title, address):
//   [ThreadMap page]     CUTLASS 2.x PitchLinearStripminedThreadMap article, hotelren.com/news/5252042
//   [print_layout page]  "CUTLASS Layout可视化：从print_layout理解GPU内存映射与性能优化",
//                        codechina.net/article/weixin_30702441/411096

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "lr_internal.h"

namespace lr {
namespace {

constexpr int64_t kMaxCells = int64_t(1) << 20;

// Offset of 1-D index k (colex over the leaves, then the swizzle); k < size(L).
int64_t offset_at(const lr_layout* L, int64_t k) {
  int64_t o = 0;
  for (int i = 0; i < L->nleaves; ++i) {
    o += (k % L->shape[i]) * L->stride[i];
    k /= L->shape[i];
  }
  if (L->swz_b > 0) o ^= (o >> L->swz_s) & (((int64_t(1) << L->swz_b) - 1) << L->swz_m);
  return o;
}

int64_t mode_size(const lr_layout* L, int m) {
  int lo = m ? L->mode_end[m - 1] : 0;
  int64_t s = 1;
  for (int i = lo; i < L->mode_end[m]; ++i) s *= L->shape[i];
  return s;
}

int digits(int64_t v) {
  int d = 1;
  while (v >= 10) {
    v /= 10;
    ++d;
  }
  return d;
}

void put_right(std::string* out, int64_t v, int width) {
  char tmp[32];
  std::snprintf(tmp, sizeof(tmp), "%*lld", width, (long long)v);
  *out += tmp;
}

int emit(const std::string& s, char* buf, size_t cap, size_t* needed) {
  if (needed) *needed = s.size() + 1;
  if (!buf || s.size() + 1 > cap) return LR_ERR_CAPACITY;
  std::memcpy(buf, s.c_str(), s.size() + 1);
  return LR_OK;
}

}  // namespace

void gfx950_lds_model(size_t elem_bytes, bool write, int32_t* banks, int32_t* lanes_per_phase) {
  if (elem_bytes <= 4) {
    *banks = 32;
    *lanes_per_phase = 32;
  } else if (!write) {
    *banks = 64;
    *lanes_per_phase = elem_bytes == 8 ? 32 : 16;
  } else {
    *banks = 32;
    *lanes_per_phase = elem_bytes == 8 ? 16 : 8;
  }
}

int32_t lds_cycles(const int64_t* byte_addr, int lanes, int64_t elem_bytes, int32_t banks, int32_t lanes_per_phase,
                   int32_t* ways_max, int32_t* worst_bank_words) {
  // [print_layout page, sections 4.3 and 5.2]: distinct 4-byte words in one bank
  // are served one after another, the same word once for every lane.  Lanes are
  // served in phases of lanes_per_phase consecutive lanes.
  int32_t cycles = 0, wmax = 0;
  std::vector<int64_t> words;
  for (int p = 0; p < lanes; p += lanes_per_phase) {
    words.clear();
    for (int t = p; t < std::min(lanes, p + lanes_per_phase); ++t) {
      const int64_t a = byte_addr[t];
      for (int64_t w = a / 4; w <= (a + elem_bytes - 1) / 4; ++w) words.push_back(w);
    }
    std::sort(words.begin(), words.end());
    words.erase(std::unique(words.begin(), words.end()), words.end());
    int32_t count[LR_WAVE_LANES] = {0};
    int32_t ways = 0;
    for (int64_t w : words) ways = std::max(ways, ++count[w % banks]);
    cycles += ways;
    if (ways > wmax) {
      wmax = ways;
      if (worst_bank_words) std::memcpy(worst_bank_words, count, sizeof(count));
    }
  }
  if (ways_max) *ways_max = wmax;
  return cycles;
}

}  // namespace lr

using namespace lr;

extern "C" {

int lr_layout_print(const lr_layout* L, char* buf, size_t cap, size_t* needed) {
  int rc = validate(L);
  if (rc) return rc;
  if (L->nmodes != 2) return LR_ERR_INVALID;
  const int64_t rows = mode_size(L, 0), cols = mode_size(L, 1);
  if (rows * cols > kMaxCells) return LR_ERR_INVALID;
  // [print_layout page, sections 2.3 and 3.1]: the outer loop walks mode 0, the
  // inner loop mode 1; the cell (r, c) is the 1-D index r + rows*c.
  std::vector<int64_t> v((size_t)(rows * cols));
  int64_t widest = 0;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      int64_t o = offset_at(L, r + rows * c);
      v[(size_t)(r * cols + c)] = o;
      widest = std::max(widest, o);
    }
  // [print_layout page, section 6.3]: a fixed column width keeps large grids aligned
  const int w = digits(widest);
  char head[4096];
  rc = lr_layout_format(L, head, sizeof(head));
  if (rc) return rc;
  std::string s = head;
  s += '\n';
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      if (c) s += ' ';
      put_right(&s, v[(size_t)(r * cols + c)], w);
    }
    s += '\n';
  }
  return emit(s, buf, cap, needed);
}

int lr_layout_print_table(const lr_layout* L, int64_t n, char* buf, size_t cap, size_t* needed) {
  int rc = validate(L);
  if (rc) return rc;
  if (n < 1 || n > size_of(L) || n > kMaxCells) return LR_ERR_INVALID;
  std::vector<int64_t> v((size_t)n);
  int64_t widest = 0;
  for (int64_t t = 0; t < n; ++t) widest = std::max(widest, v[(size_t)t] = offset_at(L, t));
  const int wt = digits(n - 1), wo = digits(widest);
  std::string s;
  for (int64_t t = 0; t < n; ++t) {
    s += "thread ";
    put_right(&s, t, wt);
    s += " -> offset ";
    put_right(&s, v[(size_t)t], wo);
    s += '\n';
  }
  return emit(s, buf, cap, needed);
}

int lr_access_check(const lr_layout* L, size_t elem_bytes, int32_t lanes, int32_t lds_model, int32_t banks,
                    int32_t lanes_per_phase, int32_t line_bytes, lr_access_report* out) {
  int rc = validate(L);
  if (rc) return rc;
  if (!out) return LR_ERR_INVALID;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8 && elem_bytes != 16)
    return LR_ERR_ELEM_BYTES;
  if (lanes < 1 || lanes > LR_WAVE_LANES || lanes > size_of(L)) return LR_ERR_INVALID;
  if (lds_model == LR_LDS_GFX950_READ || lds_model == LR_LDS_GFX950_WRITE) {
    if (banks != 0 || lanes_per_phase != 0) return LR_ERR_INVALID;
    gfx950_lds_model(elem_bytes, lds_model == LR_LDS_GFX950_WRITE, &banks, &lanes_per_phase);
  } else if (lds_model != LR_LDS_CUSTOM) {
    return LR_ERR_INVALID;
  }
  if (banks < 1 || banks > LR_WAVE_LANES || lanes_per_phase < 1 || lanes_per_phase > LR_WAVE_LANES)
    return LR_ERR_INVALID;
  if (line_bytes == 0) line_bytes = 128;
  if (line_bytes < 1) return LR_ERR_INVALID;
  // every byte address below must fit in int64
  int64_t top;
  if (!mul_ok(cosize_bound(L), (int64_t)elem_bytes, &top)) return LR_ERR_OVERFLOW;

  lr_access_report r;
  std::memset(&r, 0, sizeof(r));
  r.lanes = lanes;
  r.elem_bytes = (int32_t)elem_bytes;
  r.banks = banks;
  r.lanes_per_phase = lanes_per_phase;
  r.line_bytes = line_bytes;
  r.first_gap = -1;
  for (int t = 0; t < lanes; ++t) r.offsets[t] = offset_at(L, t);

  const int64_t eb = (int64_t)elem_bytes;
  int64_t addr[LR_WAVE_LANES];
  for (int t = 0; t < lanes; ++t) addr[t] = r.offsets[t] * eb;
  r.cycles = lds_cycles(addr, lanes, eb, banks, lanes_per_phase, &r.ways_max, r.bank_words);
  r.phases = (lanes + lanes_per_phase - 1) / lanes_per_phase;
  r.conflict_cycles = r.cycles - r.phases;

  // [print_layout page, section 6.4]: consecutive lanes on consecutive offsets
  for (int t = 0; t + 1 < lanes; ++t)
    if (r.offsets[t + 1] != r.offsets[t] + 1) {
      r.first_gap = t;
      break;
    }
  r.adjacent = r.first_gap < 0;

  // lines touched, and the fewest lines the same distinct bytes could fill
  std::vector<std::pair<int64_t, int64_t>> spans;  // byte ranges [lo, hi)
  for (int t = 0; t < lanes; ++t) spans.push_back({r.offsets[t] * eb, r.offsets[t] * eb + eb});
  std::sort(spans.begin(), spans.end());
  int64_t bytes = 0, cur_lo = -1, cur_hi = -1, last_line = -1;
  for (const auto& sp : spans) {
    if (sp.first > cur_hi) {
      bytes += cur_hi - cur_lo;
      cur_lo = sp.first;
      cur_hi = sp.second;
    } else {
      cur_hi = std::max(cur_hi, sp.second);
    }
    for (int64_t ln = std::max(sp.first / line_bytes, last_line + 1); ln <= (sp.second - 1) / line_bytes; ++ln) {
      r.lines += 1;
      last_line = ln;
    }
  }
  bytes += cur_hi - cur_lo;
  r.min_lines = (bytes + line_bytes - 1) / line_bytes;
  *out = r;
  return LR_OK;
}

}  // extern "C"
