// lds_bank_probe: measures how the LDS of a gfx950 compute unit serves one
// wavefront access pattern, next to what lr_access_check predicts for it.
//
// Each pattern is a layout over the lane id and an element size: lane t reads (or
// writes) the elem_bytes bytes at element offset L(t) of a 64 KiB LDS array, over
// and over, in every wave of 1024 workgroups of 1024 threads.  The library gives
// the lane offsets and the predicted cycles per access (lr_access_check with its
// gfx950 read or write model); the probe times the kernel with HIP events.  Run under
// `rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS`, the counter gives the
// conflict cycles of each launch directly (three launches per pattern, in the
// order printed).
//
// Output: one JSON object per pattern and line.
//
// Pages cited (title, address):
//   [print_layout page]  "CUTLASS Layout可视化：从print_layout理解GPU内存映射与性能优化",
//                        codechina.net/article/weixin_30702441/411096
//   ([print_layout page, section 6.2]: put a swizzle on a printed layout and count
//   the bank conflicts before and after.)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "layout_remap.h"

namespace {

constexpr int kLdsBytes = 65536;
constexpr int kBatches = 2048;  // 8 accesses per batch, then a wait
constexpr int kBlocks = 1024;
constexpr int kThreads = 1024;

#define PROBE_CHECK(x)                                                             \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned lds_word;

// Eight back-to-back LDS accesses at byte address `a`, then a wait for all of them.
template <int EB, bool WRITE>
__device__ __forceinline__ unsigned batch(unsigned a, unsigned x) {
  if constexpr (WRITE) {
    if constexpr (EB == 1) {
      asm volatile(
          "ds_write_b8 %0, %1\n ds_write_b8 %0, %1\n ds_write_b8 %0, %1\n ds_write_b8 %0, %1\n"
          "ds_write_b8 %0, %1\n ds_write_b8 %0, %1\n ds_write_b8 %0, %1\n ds_write_b8 %0, %1\n"
          "s_waitcnt lgkmcnt(0)" ::"v"(a), "v"(x) : "memory");
    } else if constexpr (EB == 2) {
      asm volatile(
          "ds_write_b16 %0, %1\n ds_write_b16 %0, %1\n ds_write_b16 %0, %1\n ds_write_b16 %0, %1\n"
          "ds_write_b16 %0, %1\n ds_write_b16 %0, %1\n ds_write_b16 %0, %1\n ds_write_b16 %0, %1\n"
          "s_waitcnt lgkmcnt(0)" ::"v"(a), "v"(x) : "memory");
    } else if constexpr (EB == 4) {
      asm volatile(
          "ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n"
          "ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n"
          "s_waitcnt lgkmcnt(0)" ::"v"(a), "v"(x) : "memory");
    } else if constexpr (EB == 8) {
      v2u d = {x, x + 1};
      asm volatile(
          "ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n"
          "ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n"
          "s_waitcnt lgkmcnt(0)" ::"v"(a), "v"(d) : "memory");
    } else {
      v4u d = {x, x + 1, x + 2, x + 3};
      asm volatile(
          "ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n"
          "ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n"
          "s_waitcnt lgkmcnt(0)" ::"v"(a), "v"(d) : "memory");
    }
    return x + 1;
  } else {
    if constexpr (EB <= 4) {
      unsigned r0, r1, r2, r3, r4, r5, r6, r7;
#define PROBE_READ8(OP)                                                                                   \
  asm volatile(OP " %0, %8\n " OP " %1, %8\n " OP " %2, %8\n " OP " %3, %8\n " OP " %4, %8\n " OP          \
                  " %5, %8\n " OP " %6, %8\n " OP " %7, %8\n s_waitcnt lgkmcnt(0)"                          \
               : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7) \
               : "v"(a)                                                                                   \
               : "memory")
      if constexpr (EB == 1) PROBE_READ8("ds_read_u8");
      else if constexpr (EB == 2) PROBE_READ8("ds_read_u16");
      else PROBE_READ8("ds_read_b32");
#undef PROBE_READ8
      return x ^ r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
    } else if constexpr (EB == 8) {
      v2u r0, r1, r2, r3, r4, r5, r6, r7;
      asm volatile(
          "ds_read_b64 %0, %8\n ds_read_b64 %1, %8\n ds_read_b64 %2, %8\n ds_read_b64 %3, %8\n"
          "ds_read_b64 %4, %8\n ds_read_b64 %5, %8\n ds_read_b64 %6, %8\n ds_read_b64 %7, %8\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
          : "v"(a)
          : "memory");
      v2u s = r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
      return x ^ s.x ^ s.y;
    } else {
      v4u r0, r1, r2, r3, r4, r5, r6, r7;
      asm volatile(
          "ds_read_b128 %0, %8\n ds_read_b128 %1, %8\n ds_read_b128 %2, %8\n ds_read_b128 %3, %8\n"
          "ds_read_b128 %4, %8\n ds_read_b128 %5, %8\n ds_read_b128 %6, %8\n ds_read_b128 %7, %8\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
          : "v"(a)
          : "memory");
      v4u s = r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
      return x ^ s.x ^ s.y ^ s.z ^ s.w;
    }
  }
}

// lane_bytes: byte address of each lane's access inside the LDS array (64 entries,
// each + EB <= kLdsBytes and a multiple of EB, checked on the host).
template <int EB, bool WRITE>
__global__ __launch_bounds__(kThreads) void k_lds_probe(const unsigned* __restrict__ lane_bytes,
                                                        unsigned* __restrict__ sink) {
  __shared__ unsigned lds[kLdsBytes / 4];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += kThreads) lds[i] = (unsigned)i;
  __syncthreads();
  const unsigned a = lane_bytes[threadIdx.x & 63] + (unsigned)(uintptr_t)(lds_word*)lds;
  unsigned x = threadIdx.x;
  for (int r = 0; r < kBatches; ++r) x = batch<EB, WRITE>(a, x);
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;  // keeps the reads live; never true in practice
}

struct Pattern {
  const char* layout;
  int eb;
};

const Pattern kPatterns[] = {
    // 32-bit: the page's column read (8-way on 32 banks), its padded and swizzled fixes
    {"64:1", 4}, {"64:2", 4}, {"64:4", 4}, {"64:8", 4}, {"64:9", 4}, {"64:32", 4}, {"64:33", 4},
    {"64:0", 4}, {"(32,2):(1,64)", 4}, {"(32,2):(32,1)", 4}, {"Sw<3,0,3> o (32,8):(8,1)", 4},
    // 16-bit and 8-bit: several lanes in one 4-byte word
    {"64:1", 2}, {"64:2", 2}, {"64:4", 2}, {"64:64", 2}, {"(2,32):(1,64)", 2}, {"64:0", 2},
    {"64:1", 1}, {"64:4", 1}, {"64:8", 1}, {"64:128", 1}, {"64:0", 1},
    // 64-bit
    {"64:1", 8}, {"64:2", 8}, {"64:32", 8}, {"64:33", 8}, {"(32,2):(1,64)", 8}, {"(16,4):(1,32)", 8},
    {"(16,4):(1,64)", 8},
    // 128-bit
    {"64:1", 16}, {"64:2", 16}, {"64:4", 16}, {"64:8", 16}, {"64:16", 16}, {"64:17", 16}, {"64:9", 16},
    {"(8,8):(1,16)", 16}, {"(8,2,4):(1,8,32)", 16}, {"(4,16):(1,16)", 16}, {"(16,4):(1,64)", 16},
};

template <int EB, bool WRITE>
void launch(const unsigned* lane_bytes, unsigned* sink) {
  k_lds_probe<EB, WRITE><<<kBlocks, kThreads>>>(lane_bytes, sink);
}

void launch_any(int eb, bool write, const unsigned* lane_bytes, unsigned* sink) {
  switch (eb * 2 + (write ? 1 : 0)) {
    case 2: launch<1, false>(lane_bytes, sink); break;
    case 3: launch<1, true>(lane_bytes, sink); break;
    case 4: launch<2, false>(lane_bytes, sink); break;
    case 5: launch<2, true>(lane_bytes, sink); break;
    case 8: launch<4, false>(lane_bytes, sink); break;
    case 9: launch<4, true>(lane_bytes, sink); break;
    case 16: launch<8, false>(lane_bytes, sink); break;
    case 17: launch<8, true>(lane_bytes, sink); break;
    case 32: launch<16, false>(lane_bytes, sink); break;
    default: launch<16, true>(lane_bytes, sink); break;
  }
}

}  // namespace

int main(int argc, char** argv) {
  bool do_read = true, do_write = true;
  if (argc > 1 && std::strcmp(argv[1], "read") == 0) do_write = false;
  if (argc > 1 && std::strcmp(argv[1], "write") == 0) do_read = false;

  // lane offsets and predictions from the library, checked before any launch
  struct Prepared {
    const Pattern* p;
    lr_access_report rep[2];  // read model, write model
    unsigned bytes[64];
  };
  std::vector<Prepared> prep;
  for (const Pattern& p : kPatterns) {
    Prepared q;
    q.p = &p;
    lr_layout L;
    int rc = lr_layout_parse(p.layout, &L);
    if (rc == LR_OK) rc = lr_access_check(&L, (size_t)p.eb, 64, LR_LDS_GFX950_READ, 0, 0, 0, &q.rep[0]);
    if (rc == LR_OK) rc = lr_access_check(&L, (size_t)p.eb, 64, LR_LDS_GFX950_WRITE, 0, 0, 0, &q.rep[1]);
    if (rc != LR_OK) {
      std::fprintf(stderr, "pattern %s: %s\n", p.layout, lr_strerror(rc));
      return 1;
    }
    for (int t = 0; t < 64; ++t) {
      const int64_t b = q.rep[0].offsets[t] * p.eb;
      if (b < 0 || b + p.eb > kLdsBytes || b % p.eb) {
        std::fprintf(stderr, "pattern %s: lane %d outside the LDS array\n", p.layout, t);
        return 1;
      }
      q.bytes[t] = (unsigned)b;
    }
    prep.push_back(q);
  }

  unsigned *d_bytes = nullptr, *d_sink = nullptr;
  PROBE_CHECK(hipMalloc(&d_bytes, 64 * sizeof(unsigned)));
  PROBE_CHECK(hipMalloc(&d_sink, kBlocks * sizeof(unsigned)));
  hipEvent_t e0, e1;
  PROBE_CHECK(hipEventCreate(&e0));
  PROBE_CHECK(hipEventCreate(&e1));
  for (int w = 0; w < 2; ++w) {
    const bool write = w == 1;
    if ((write && !do_write) || (!write && !do_read)) continue;
    for (const Prepared& q : prep) {
      PROBE_CHECK(hipMemcpy(d_bytes, q.bytes, sizeof(q.bytes), hipMemcpyHostToDevice));
      float best = 1e30f;
      for (int it = 0; it < 3; ++it) {
        PROBE_CHECK(hipEventRecord(e0));
        launch_any(q.p->eb, write, d_bytes, d_sink);
        PROBE_CHECK(hipGetLastError());
        PROBE_CHECK(hipEventRecord(e1));
        PROBE_CHECK(hipEventSynchronize(e1));
        float ms = 0;
        PROBE_CHECK(hipEventElapsedTime(&ms, e0, e1));
        if (ms < best) best = ms;
      }
      const double accesses = (double)kBlocks * (kThreads / 64) * kBatches * 8;  // wave instructions
      std::printf(
          "{\"layout\": \"%s\", \"elem_bytes\": %d, \"op\": \"%s\", \"model_cycles\": %d, \"model_phases\": %d, "
          "\"model_conflict_cycles\": %d, \"ms\": %.4f, \"wave_accesses\": %.0f}\n",
          q.p->layout, q.p->eb, write ? "write" : "read", q.rep[w].cycles, q.rep[w].phases, q.rep[w].conflict_cycles,
          best,
          accesses);
      std::fflush(stdout);
    }
  }
  PROBE_CHECK(hipFree(d_bytes));
  PROBE_CHECK(hipFree(d_sink));
  return 0;
}
