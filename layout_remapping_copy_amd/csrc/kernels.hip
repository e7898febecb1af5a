// HIP kernels for gfx950 (MI355X) and the device-side C ABI entry points:
// lr_layout_eval, lr_layout_eval_coords, lr_layout_copy.
//
// Pages cited (title, address):
//   [ThreadMap page]     CUTLASS 2.x PitchLinearStripminedThreadMap article, hotelren.com/news/5252042
//   [CuTe algebra page]  "CUTE布局代数：GPU张量计算的内存优化革命", jsqmd.com/news/768714
//   [print_layout page]  "CUTLASS Layout可视化：从print_layout理解GPU内存映射与性能优化",
//                        codechina.net/article/weixin_30702441/411096
//
// All work here is integer index arithmetic and byte movement: elements are moved
// as opaque bit patterns in units of 1, 2, 4, 8 or 16 bytes.  Divisions by layout
// extents use multiply-high constants computed on the host (make_fastdiv), exact
// for dividends below 2^31.  Copies beyond 31-bit indices and offsets are cut
// into blocks that fit (lr_layout_copy); the 64-bit ("wide") kernels with ordinary
// division remain for the cases that cannot be cut (a swizzle, an aliased
// destination, a forced path or an explicit request).
//
// Wavefronts are 64 lanes.  Workgroups have 256 lanes (4 waves, one per SIMD),
// except the tile transposes (TA*TB lanes, 256 to 1024; 512 for element tiles) and
// the ordered-alias kernel (1024 lanes, one window per workgroup).
//
// Cache policy: streaming copies (by default when source plus destination reach
// the 256 MiB last-level cache) load and store with the non-temporal bit; element
// tiles keep ordinary accesses at every size, so the partial lines at their
// unaligned row ends merge in L2.  The streaming stores of the vector path, the
// head interleave, the channel shuffle and the LDS tile transpose are buffer
// stores that also carry the sc1 scope bit, which HIP's global stores cannot
// express; their 32-bit offsets run from a base the host has checked (the
// destination, or a transpose tile's lowest offset).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "lr_internal.h"

namespace lr {

// ------------------------------------------------------------------ helpers

static thread_local char g_hip_err[256];

void set_hip_error(const char* text) {
  std::snprintf(g_hip_err, sizeof(g_hip_err), "%s", text ? text : "");
}

struct FD {  // device copy of FastDiv
  uint32_t m, s;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t x, FD f) { return f.m ? (__umulhi(x, f.m) >> f.s) : x; }

struct SwzArg {  // o ^ ((o >> shift) & mask); mask == 0: none
  uint32_t mask, shift;
};

__device__ __forceinline__ uint32_t swz32(uint32_t o, SwzArg z) { return o ^ ((o >> z.shift) & z.mask); }
__device__ __forceinline__ uint64_t swz64(uint64_t o, uint64_t mask, uint32_t shift) {
  return o ^ ((o >> shift) & mask);
}

static SwzArg swz_arg(const Swz& z) {
  SwzArg a{0, 0};
  if (z.b > 0) {
    a.mask = ((1u << z.b) - 1u) << z.m;
    a.shift = (uint32_t)z.s;
  }
  return a;
}

static FD fd_of(int64_t d) {
  FastDiv f = make_fastdiv((uint32_t)d);
  return FD{f.m, f.s};
}

// element and chunk types, moved as raw bits
template <int B> struct Raw;
template <> struct Raw<1> { using T = uint8_t; };
template <> struct Raw<2> { using T = uint16_t; };
template <> struct Raw<4> { using T = uint32_t; };
template <> struct Raw<8> { using T = uint2; };
template <> struct Raw<16> { using T = uint4; };

template <typename T, int V>
struct alignas(V * sizeof(T) >= 16 ? 16 : V * sizeof(T)) Chunk {
  T e[V];
};


// Global loads/stores of a raw element or chunk.  NT: non-temporal (streaming data
// that will not be re-read soon).  The policy is a template parameter: chosen at
// run time between two otherwise identical accesses, the compiler merges them
// into one plain access and the hint is lost.
template <int S> struct NativeOf;
template <> struct NativeOf<1> { using T = uint8_t; };
template <> struct NativeOf<2> { using T = uint16_t; };
template <> struct NativeOf<4> { using T = uint32_t; };
template <> struct NativeOf<8> { using T = unsigned int __attribute__((ext_vector_type(2))); };
template <> struct NativeOf<16> { using T = unsigned int __attribute__((ext_vector_type(4))); };
using U4 = NativeOf<16>::T;  // one 16-byte chunk

template <bool NT, typename C>
__device__ __forceinline__ C gload(const void* p) {
  using N = typename NativeOf<sizeof(C)>::T;
  N x;
  if constexpr (NT)
    x = __builtin_nontemporal_load((const N*)p);
  else
    x = *(const N*)p;
  return __builtin_bit_cast(C, x);
}

template <bool NT, typename C>
__device__ __forceinline__ void gstore(void* p, const C& v) {
  using N = typename NativeOf<sizeof(C)>::T;
  N x = __builtin_bit_cast(N, v);
  if constexpr (NT)
    __builtin_nontemporal_store(x, (N*)p);
  else
    *(N*)p = x;
}

// Buffer resources for raw (unformatted, stride 0) accesses: the descriptor's last
// word for gfx950, and the cache-policy bits of a streaming store: nt (2) marks the
// data non-temporal, sc1 (16) selects the wider coherence scope.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kPolicyNtSc1 = 2 | 16;

// gfx950 direct global -> LDS load of 16 bytes per lane: lane i of the wave writes
// its bytes at lds_wave + 16*i (lds_wave is the wave's common LDS base).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;
// NT: the non-temporal cache-policy bit (2 on gfx950).
template <bool NT>
__device__ __forceinline__ void load_to_lds16(const void* g, void* lds_wave) {
  __builtin_amdgcn_global_load_lds((const global_void_t*)g, (lds_void_t*)lds_wave, 16, 0, NT ? 2 : 0);
}

// Write counting for lr_layout_copy_count_writes: every store of nbytes at p adds
// one to the counter of each destination element (of 2^shift bytes) it covers.
// Ordinary copies pass wc == NULL and skip it with one uniform branch.
struct WriteCount {
  int32_t* wc;
  uint32_t shift;
};

__device__ __forceinline__ void count_store(const WriteCount& w, const void* dst_base, const void* p,
                                            uint32_t nbytes) {
  if (w.wc == nullptr) return;
  const size_t b = (size_t)((const char*)p - (const char*)dst_base);
  for (uint32_t i = 0; i < nbytes; i += (1u << w.shift)) atomicAdd(w.wc + ((b + i) >> w.shift), 1);
}

// ------------------------------------------------------------------ eval

struct EvalArgs {
  int32_t nleaves, nmodes;
  int64_t shape[LR_MAX_LEAVES];
  int64_t stride[LR_MAX_LEAVES];
  int32_t mode_end[LR_MAX_LEAVES];
  FD fd[LR_MAX_LEAVES];
  uint64_t swz_mask;
  uint32_t swz_shift;
  int32_t small;  // size < 2^31: fast division
  int64_t size;
  int64_t mode_size[LR_MAX_LEAVES];
  const int64_t* idx;
  const int64_t* coords;
  int32_t ncols;
  int64_t n;
  int64_t* out;
  int32_t s32;   // the size and every offset (swizzled too) fit 31 bits: 32-bit arithmetic
};

// 1-D index -> offset: colex digits over the leaves, sum of digit*stride, swizzle
// ([print_layout page, section 2.1]: offset = sum of coordinate * stride;
//  [print_layout page, section 4.3]: the XOR swizzle on the offset).
__device__ __forceinline__ int64_t eval_leaves(const EvalArgs& a, int lo, int hi, int64_t k) {
  int64_t off = 0;
  if (a.small) {
    uint32_t r = (uint32_t)k;
    for (int i = lo; i < hi; ++i) {
      uint32_t q = (i == hi - 1) ? 0u : fdiv(r, a.fd[i]);
      uint32_t dgt = (i == hi - 1) ? r : r - q * (uint32_t)a.shape[i];
      off += (int64_t)dgt * a.stride[i];
      r = q;
    }
  } else {
    uint64_t r = (uint64_t)k;
    for (int i = lo; i < hi; ++i) {
      uint64_t n = (uint64_t)a.shape[i];
      uint64_t q = (i == hi - 1) ? 0 : r / n;
      off += (int64_t)(r - q * n) * a.stride[i];
      r = q;
    }
  }
  return off;
}

// 32-bit form of eval_leaves for layouts whose offsets stay under 2^31: the
// unswizzled offset of index r, and r's first digit (colex, leaf 0 fastest).
__device__ __forceinline__ uint32_t eval32(const EvalArgs& a, uint32_t r, uint32_t* digit0) {
  uint32_t off = 0;
  for (int i = 0; i < a.nleaves; ++i) {
    const uint32_t q = (i == a.nleaves - 1) ? 0u : fdiv(r, a.fd[i]);
    const uint32_t d = r - q * (uint32_t)a.shape[i];
    if (i == 0) *digit0 = d;
    off += d * (uint32_t)a.stride[i];
    r = q;
  }
  return off;
}

__device__ __forceinline__ int64_t swz32_eval(const EvalArgs& a, uint32_t off) {
  return (int64_t)(off ^ ((off >> a.swz_shift) & (uint32_t)a.swz_mask));
}

// Indices 0..n-1 of a layout with 31-bit offsets: each lane evaluates two
// consecutive indices and writes them with one 16-byte store.  The second offset
// is the first plus leaf 0's stride while leaf 0's digit does not wrap, else a
// full evaluation.  `out` is 16-byte aligned (the host checks).
__global__ void __launch_bounds__(256) k_eval_range32(EvalArgs a) {
  typedef long long ll2 __attribute__((ext_vector_type(2)));
  const int64_t np = a.n >> 1;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < np; p += (int64_t)gridDim.x * 256) {
    const int64_t k = 2 * p;
    ll2 v;
    v.x = v.y = -1;
    if (k < a.size) {
      uint32_t d0;
      const uint32_t o0 = eval32(a, (uint32_t)k, &d0);
      v.x = swz32_eval(a, o0);
      if (k + 1 < a.size) {
        uint32_t d1;
        const uint32_t o1 = d0 + 1 < (uint32_t)a.shape[0] ? o0 + (uint32_t)a.stride[0] : eval32(a, (uint32_t)k + 1, &d1);
        v.y = swz32_eval(a, o1);
      }
    }
    *(ll2*)(a.out + k) = v;
  }
  if ((a.n & 1) && blockIdx.x == 0 && threadIdx.x == 0) {  // an odd count's last index
    const int64_t k = a.n - 1;
    uint32_t d;
    a.out[k] = k < a.size ? swz32_eval(a, eval32(a, (uint32_t)k, &d)) : -1;
  }
}

__global__ void __launch_bounds__(256) k_eval_index(EvalArgs a) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.n; i += (int64_t)gridDim.x * 256) {
    int64_t k = a.idx ? a.idx[i] : i;
    int64_t off = -1;
    if (k >= 0 && k < a.size) {
      if (a.s32) {
        uint32_t d;
        off = swz32_eval(a, eval32(a, (uint32_t)k, &d));
      } else {
        off = (int64_t)swz64((uint64_t)eval_leaves(a, 0, a.nleaves, k), a.swz_mask, a.swz_shift);
      }
    }
    a.out[i] = off;
  }
}

__global__ void __launch_bounds__(256) k_eval_coords(EvalArgs a) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.n; i += (int64_t)gridDim.x * 256) {
    const int64_t* c = a.coords + i * a.ncols;
    int64_t off = 0;
    bool ok = true;
    if (a.ncols == a.nleaves) {  // natural coordinate: one integer per leaf
      for (int l = 0; l < a.nleaves; ++l) {
        int64_t x = c[l];
        ok = ok && x >= 0 && x < a.shape[l];
        off += x * a.stride[l];
      }
    } else {  // one integer per top-level mode, colex inside the mode
      int lo = 0;
      for (int m = 0; m < a.nmodes; ++m) {
        int64_t x = c[m];
        ok = ok && x >= 0 && x < a.mode_size[m];
        if (ok) {
          if (a.s32) {  // 32-bit digits when every offset fits 31 bits
            uint32_t r = (uint32_t)x, o = 0;
            for (int i = lo; i < a.mode_end[m]; ++i) {
              const uint32_t q = (i == a.mode_end[m] - 1) ? 0u : fdiv(r, a.fd[i]);
              o += (r - q * (uint32_t)a.shape[i]) * (uint32_t)a.stride[i];
              r = q;
            }
            off += o;
          } else {
            off += eval_leaves(a, lo, a.mode_end[m], x);
          }
        }
        lo = a.mode_end[m];
      }
    }
    a.out[i] = ok ? (int64_t)swz64((uint64_t)off, a.swz_mask, a.swz_shift) : -1;
  }
}

// ------------------------------------------------------------------ generic / vector copy

struct ModeArg {
  uint32_t ext;
  FD fd;
  uint32_t ss, sd;
};

struct ModeArg64 {
  int64_t ext, ss, sd;
};

struct GenericArgs {
  const void* src;
  void* dst;
  int32_t rank;
  ModeArg m[kMaxKernelModes];
  ModeArg64 w[kMaxKernelModes];
  SwzArg sws, swd;
  uint64_t sws_mask64, swd_mask64;
  int64_t n_units;
  int64_t n_chunks;  // groups of 256 * U units, U the per-lane unroll
  uint32_t bufst;    // 1: streaming 16-byte stores as buffer stores from dst (span < 4 GiB)
  WriteCount wcnt;
};

// One unit (UB bytes) per lane and step, one or four units per lane (U); with four,
// each lane issues all four loads before its stores.  Lanes of a wave take
// consecutive units, i.e. consecutive positions of the fastest joint mode.
template <bool WIDE>
__device__ __forceinline__ void generic_offsets(const GenericArgs& a, int64_t idx, uint64_t* so, uint64_t* dof) {
  if (WIDE) {
    uint64_t r = (uint64_t)idx, s = 0, d = 0;
    for (int k = 0; k < a.rank; ++k) {
      uint64_t e = (uint64_t)a.w[k].ext;
      uint64_t q = r / e;
      uint64_t g = r - q * e;
      s += g * (uint64_t)a.w[k].ss;
      d += g * (uint64_t)a.w[k].sd;
      r = q;
    }
    *so = swz64(s, a.sws_mask64, a.sws.shift);
    *dof = swz64(d, a.swd_mask64, a.swd.shift);
  } else {
    uint32_t r = (uint32_t)idx, s = 0, d = 0;
    for (int k = 0; k < a.rank; ++k) {
      uint32_t q = (k == a.rank - 1) ? 0u : fdiv(r, a.m[k].fd);
      uint32_t g = r - q * a.m[k].ext;
      s += g * a.m[k].ss;
      d += g * a.m[k].sd;
      r = q;
    }
    *so = swz32(s, a.sws);
    *dof = swz32(d, a.swd);
  }
}

// Compile-time loop: f(integral_constant<int, I>) for I = 0..N-1, so per-lane
// values live in named registers (a runtime-indexed local array of vectors would
// be placed in LDS or scratch, serialising the loads behind it).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// LNT / SNT: non-temporal loads / stores (chosen apart: a source read once with a
// destination that should stay cached for its next reader).  L lanes per workgroup
// (64, 128 or 256 with one unit per lane; 256 otherwise).
template <int UB, bool WIDE, int U, bool LNT, bool SNT, int L = 256>
__global__ void __launch_bounds__(L) k_generic(GenericArgs a) {
  static_assert(U == 1 || U == 4, "one or four units per lane");
  static_assert(L == 256 || (U == 1 && !WIDE), "narrower workgroups with one unit per lane");
  using T = typename Raw<UB>::T;
  const T* __restrict__ src = (const T*)a.src;
  T* __restrict__ dst = (T*)a.dst;
  if constexpr (SNT && UB == 16 && U == 1 && !WIDE) {
    if (a.bufst) {
      // Streaming stores as buffer stores with the nt and sc1 policy bits (measured
      // faster than nt alone on large copies); the host checks that every
      // destination byte lies under 4 GiB from the base.
      const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(a.dst, 0, -1, kBufferWord3);
      for (int64_t ch = blockIdx.x; ch < a.n_chunks; ch += gridDim.x) {
        const int64_t i0 = ch * L + threadIdx.x;
        if (i0 < a.n_units) {
          uint64_t s0, d0;
          generic_offsets<false>(a, i0, &s0, &d0);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(typename NativeOf<16>::T, gload<LNT, T>(src + s0)),
                                                 rd, (uint32_t)(d0 * 16), 0, kPolicyNtSc1);
          count_store(a.wcnt, a.dst, (const char*)a.dst + d0 * 16, 16);
        }
      }
      return;
    }
  }
  for (int64_t ch = blockIdx.x; ch < a.n_chunks; ch += gridDim.x) {
    const int64_t i0 = ch * (L * U) + threadIdx.x;
    if constexpr (U == 1) {
      if (i0 < a.n_units) {
        uint64_t s0, d0;
        generic_offsets<WIDE>(a, i0, &s0, &d0);
        gstore<SNT, T>(dst + d0, gload<LNT, T>(src + s0));
        count_store(a.wcnt, a.dst, dst + d0, UB);
      }
    } else {
      uint64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0, d0 = 0, d1 = 0, d2 = 0, d3 = 0;
      const bool k0 = i0 < a.n_units, k1 = i0 + 256 < a.n_units, k2 = i0 + 512 < a.n_units,
                 k3 = i0 + 768 < a.n_units;
      if (k0) generic_offsets<WIDE>(a, i0, &s0, &d0);
      if (k1) generic_offsets<WIDE>(a, i0 + 256, &s1, &d1);
      if (k2) generic_offsets<WIDE>(a, i0 + 512, &s2, &d2);
      if (k3) generic_offsets<WIDE>(a, i0 + 768, &s3, &d3);
      T v0, v1, v2, v3;
      if (k0) v0 = gload<LNT, T>(src + s0);
      if (k1) v1 = gload<LNT, T>(src + s1);
      if (k2) v2 = gload<LNT, T>(src + s2);
      if (k3) v3 = gload<LNT, T>(src + s3);
      if (k0) gstore<SNT, T>(dst + d0, v0);
      if (k1) gstore<SNT, T>(dst + d1, v1);
      if (k2) gstore<SNT, T>(dst + d2, v2);
      if (k3) gstore<SNT, T>(dst + d3, v3);
      if (k0) count_store(a.wcnt, a.dst, dst + d0, UB);
      if (k1) count_store(a.wcnt, a.dst, dst + d1, UB);
      if (k2) count_store(a.wcnt, a.dst, dst + d2, UB);
      if (k3) count_store(a.wcnt, a.dst, dst + d3, UB);
    }
  }
}

// ------------------------------------------------------------------ dual evaluation

struct SideArg {
  int32_t nleaves;
  uint32_t ext[LR_MAX_LEAVES];
  FD fd[LR_MAX_LEAVES];
  uint32_t stride[LR_MAX_LEAVES];
  int64_t ext64[LR_MAX_LEAVES];
  int64_t stride64[LR_MAX_LEAVES];
  SwzArg sw;
  uint64_t mask64;
};

template <bool WIDE>
__device__ __forceinline__ uint64_t side_eval(const SideArg& s, int64_t k) {
  if (WIDE) {
    uint64_t r = (uint64_t)k, o = 0;
    for (int i = 0; i < s.nleaves; ++i) {
      uint64_t n = (uint64_t)s.ext64[i];
      uint64_t q = r / n;
      o += (r - q * n) * (uint64_t)s.stride64[i];
      r = q;
    }
    return swz64(o, s.mask64, s.sw.shift);
  }
  uint32_t r = (uint32_t)k, o = 0;
  for (int i = 0; i < s.nleaves; ++i) {
    uint32_t q = (i == s.nleaves - 1) ? 0u : fdiv(r, s.fd[i]);
    o += (r - q * s.ext[i]) * s.stride[i];
    r = q;
  }
  return swz32(o, s.sw);
}

struct DualArgs {
  const void* src;
  void* dst;
  SideArg s, d;
  int64_t n;
  int64_t n_chunks;
  WriteCount wcnt;
};

// Each lane evaluates both layouts from the index (used when the two layouts have
// no common refinement into joint modes).
template <int EB, bool WIDE>
__global__ void __launch_bounds__(256) k_dual(DualArgs a) {
  using T = typename Raw<EB>::T;
  const T* __restrict__ src = (const T*)a.src;
  T* __restrict__ dst = (T*)a.dst;
  for (int64_t ch = blockIdx.x; ch < a.n_chunks; ch += gridDim.x) {
    const int64_t i0 = ch * 1024 + threadIdx.x;
    const bool k0 = i0 < a.n, k1 = i0 + 256 < a.n, k2 = i0 + 512 < a.n, k3 = i0 + 768 < a.n;
    T v0, v1, v2, v3;
    if (k0) v0 = gload<false, T>(src + side_eval<WIDE>(a.s, i0));
    if (k1) v1 = gload<false, T>(src + side_eval<WIDE>(a.s, i0 + 256));
    if (k2) v2 = gload<false, T>(src + side_eval<WIDE>(a.s, i0 + 512));
    if (k3) v3 = gload<false, T>(src + side_eval<WIDE>(a.s, i0 + 768));
    T* q0 = k0 ? dst + side_eval<WIDE>(a.d, i0) : dst;
    T* q1 = k1 ? dst + side_eval<WIDE>(a.d, i0 + 256) : dst;
    T* q2 = k2 ? dst + side_eval<WIDE>(a.d, i0 + 512) : dst;
    T* q3 = k3 ? dst + side_eval<WIDE>(a.d, i0 + 768) : dst;
    if (k0) gstore<false, T>(q0, v0);
    if (k1) gstore<false, T>(q1, v1);
    if (k2) gstore<false, T>(q2, v2);
    if (k3) gstore<false, T>(q3, v3);
    if (k0) count_store(a.wcnt, a.dst, q0, EB);
    if (k1) count_store(a.wcnt, a.dst, q1, EB);
    if (k2) count_store(a.wcnt, a.dst, q2, EB);
    if (k3) count_store(a.wcnt, a.dst, q3, EB);
  }
}

// ------------------------------------------------------------------ ordered aliased copy

constexpr int kAliasWindow = 8192;

// Non-injective destination with sequential semantics: for every dst offset the
// greatest index k that writes it wins.  Workgroup w owns dst offsets
// [w*8192, (w+1)*8192): it records the greatest writer of each offset in an LDS
// table (atomic max), then lets only that writer store.  Deterministic; no
// device scratch memory.
template <int EB>
__global__ void __launch_bounds__(1024) k_alias(DualArgs a) {
  using T = typename Raw<EB>::T;
  __shared__ int owner[kAliasWindow];
  const T* __restrict__ src = (const T*)a.src;
  T* __restrict__ dst = (T*)a.dst;
  const int64_t w0 = (int64_t)blockIdx.x * kAliasWindow;
  for (int i = threadIdx.x; i < kAliasWindow; i += 1024) owner[i] = -1;
  __syncthreads();
  for (int64_t k = threadIdx.x; k < a.n; k += 1024) {
    int64_t o = (int64_t)side_eval<false>(a.d, k) - w0;
    if (o >= 0 && o < kAliasWindow) atomicMax(&owner[o], (int)k);
  }
  __syncthreads();
  for (int64_t k = threadIdx.x; k < a.n; k += 1024) {
    int64_t o = (int64_t)side_eval<false>(a.d, k) - w0;
    if (o >= 0 && o < kAliasWindow && owner[o] == (int)k) {
      dst[w0 + o] = src[side_eval<false>(a.s, k)];
      count_store(a.wcnt, a.dst, dst + w0 + o, EB);
    }
  }
}

// ------------------------------------------------------------------ batch modes

struct BatchArg {
  int32_t rank;
  uint32_t ext[kMaxKernelModes];
  FD fd[kMaxKernelModes];
  uint32_t ss[kMaxKernelModes], sd[kMaxKernelModes];
};

__device__ __forceinline__ void batch_offsets(const BatchArg& b, uint32_t r, uint32_t* so, uint32_t* sd) {
  uint32_t s = 0, d = 0;
  for (int k = 0; k < b.rank; ++k) {
    uint32_t q = (k == b.rank - 1) ? 0u : fdiv(r, b.fd[k]);
    uint32_t g = r - q * b.ext[k];
    s += g * b.ss[k];
    d += g * b.sd[k];
    r = q;
  }
  *so = s;
  *sd = d;
}

// ------------------------------------------------------------------ tiles of atoms

// The vector path's fourth traversal order: the common contiguous mode is an atom
// of K 16-byte chunks, mode a continues it in the source and mode b in the
// destination ([CuTe algebra page, section 3.2]: the copy is a zipped divide of the
// (a, b) plane into T x T tiles of atoms, each tile moved as one unit).  A
// 256-lane workgroup loads its tile as T source runs of T atoms (a wave instruction
// reads consecutive chunks of one run), regroups it in LDS and stores it as T
// destination runs of T atoms (T = atom_tile(K); a tile that is not a whole number
// of 256-lane rounds leaves the last round partial).  LDS slot of chunk q of atom
// (a = i, b = j) in the tile: (j * T + (i ^ (j % T))) * K + q.  For power-of-two K
// the stores' 16 lanes of a 16-byte read phase cover 256 bytes of atoms j, j + 1, ...
// of one i, and the XOR puts those atoms in distinct 256/K-chunk slots modulo 256
// bytes; the loads' 8 lanes of a write phase stay inside aligned groups of atoms,
// i.e. 128 contiguous bytes.  All offsets are in 16-byte chunks, swizzles included.
struct AtomArgs {
  const void* src;
  void* dst;
  uint32_t ext_a, ext_b;   // atoms along a and b
  uint32_t ss_b, sd_a;     // chunk strides of b in the source and of a in the destination
  uint32_t tiles_a, tiles_b;
  FD fd_ta, fd_tb;
  BatchArg batch;          // the other modes (chunk strides)
  SwzArg sws, swd;
  uint32_t bufst;          // streaming stores as buffer stores (destination span < 4 GiB)
  WriteCount wcnt;
};

template <int K, bool LNT, bool SNT, int LANES = 256>
__global__ void __launch_bounds__(LANES) k_atoms(AtomArgs t) {
  constexpr int T = (int)atom_tile(K);
  constexpr int RUN = T * K;         // chunks in one run of T atoms
  constexpr int CH = T * RUN, PER = (CH + LANES - 1) / LANES;
  constexpr bool WHOLE = CH % LANES == 0;  // else the last round of lanes is partial
  __shared__ U4 tile[CH];
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;
  const uint32_t r1 = fdiv(blockIdx.x, t.fd_ta), ta = blockIdx.x - r1 * t.tiles_a;
  const uint32_t r2 = fdiv(r1, t.fd_tb), tb = r1 - r2 * t.tiles_b;
  uint32_t bs, bd;
  batch_offsets(t.batch, r2, &bs, &bd);
  const int tid = threadIdx.x;
  U4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int L = k * LANES + tid;                 // source order: run j, atom i, chunk q
    const int j = L / RUN, i = (L % RUN) / K, q = L % K;
    const uint32_t a = ta * T + i, b = tb * T + j;
    if ((WHOLE || L < CH) && a < t.ext_a && b < t.ext_b)
      v[k] = gload<LNT, U4>(src + (size_t)swz32(a * K + q + b * t.ss_b + bs, t.sws) * 16);
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int L = k * LANES + tid;
    const int j = L / RUN, i = (L % RUN) / K, q = L % K;
    if ((WHOLE || L < CH) && ta * T + i < t.ext_a && tb * T + j < t.ext_b) tile[(j * T + (i ^ (j % T))) * K + q] = v[k];
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst, 0, -1, kBufferWord3);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int S = k * LANES + tid;                 // destination order: run i, atom j, chunk q
    const int i = S / RUN, j = (S % RUN) / K, q = S % K;
    const uint32_t a = ta * T + i, b = tb * T + j;
    if ((WHOLE || S < CH) && a < t.ext_a && b < t.ext_b) {
      const U4 x = tile[(j * T + (i ^ (j % T))) * K + q];
      const uint32_t dof = swz32(b * K + q + a * t.sd_a + bd, t.swd);
      if (SNT && t.bufst)
        __builtin_amdgcn_raw_buffer_store_b128(x, rd, dof * 16u, 0, kPolicyNtSc1);
      else
        gstore<SNT, U4>(dst + (size_t)dof * 16, x);
      count_store(t.wcnt, t.dst, dst + (size_t)dof * 16, 16);
    }
  }
}

// ------------------------------------------------------------------ tile transpose

// Head, interior and tail of the EB-aligned byte range [g, g + len): `head` single
// elements up to the first 16-byte boundary, `nint` whole chunks from `a0` bytes
// into the range, `tail` single elements after them.  A range without a whole chunk
// is all head.
template <int EB>
struct WinSplit {
  uint32_t head, nint, tail, a0, a1;
  __device__ __forceinline__ WinSplit(const void* g, uint32_t len) {
    const uint32_t mis = (uint32_t)((uintptr_t)g & 15u);
    const uint32_t first = (16u - mis) & 15u;                // bytes to the first boundary
    const bool inner = len >= first + 16u;
    a0 = inner ? first : len;
    nint = inner ? (len - first) >> 4 : 0u;
    a1 = a0 + 16u * nint;
    head = a0 / EB;
    tail = (len - a1) / EB;
  }
};

struct TransposeArgs {
  const void* src;
  void* dst;
  uint32_t ext_a, ext_b;  // a: src-contiguous mode, b: dst-contiguous mode
  uint32_t ss_b, sd_a;    // the other stride of each
  // b may be a group of two joint modes that run on in dst (the first of extent
  // 2^bshift at dst stride 1, the second at dst stride 2^bshift): the source offset
  // of row b is then (b & bmask) * ss_b + (b >> bshift) * ss_b2.  For a single
  // mode bmask is all ones, bshift 31 and ss_b2 0.
  uint32_t bmask, bshift, ss_b2;
  uint32_t tiles_a, tiles_b;
  FD fd_ta, fd_tb;
  BatchArg batch;
  SwzArg sws, swd;
  uint32_t order;  // 0: tiles along a vary fastest across workgroups, 1: along b, 2: diagonal,
                   // 3: diagonal over 4 x 4 groups of tiles, 4: diagonal with b fastest;
                   // 5..9: orders 0..4 over workgroup numbers grouped by XCD
  uint32_t nwg;    // orders 5..9: workgroups launched
  uint32_t gta, gtb;  // order 3: groups along a and b
  FD fd_gta, fd_gtb;
  // streaming stores of the LDS tile transpose: 1 = buffer stores relative to the
  // tile's lowest destination offset (rounded down by bufmask, which clears the
  // bits a destination swizzle may change); the host checks that every offset of a
  // tile lies less than 4 GiB above that base
  uint32_t bufst, bufmask;
  WriteCount wcnt;
  // pipelined transpose: tiles per workgroup (0: one tile, not pipelined) and the
  // total number of tiles (tiles_a * tiles_b * batch)
  uint32_t pipe, ntiles;
};

// Workgroup number -> (a-tile, b-tile, batch index) in the order t.order selects.
// Orders 5..9 first renumber the workgroups by XCD: the dispatcher hands workgroup
// w to XCD w % 8, so w -> (w % 8) * ceil-share + w / 8 gives each XCD a contiguous
// run of numbers (the XCDs with index below nwg % 8 take one more), i.e. the
// workgroups one XCD runs together take neighbouring tiles and share its L2.
__device__ __forceinline__ void transpose_tile(const TransposeArgs& t, uint32_t blk, uint32_t& ta, uint32_t& tb,
                                               uint32_t& r2) {
  uint32_t order = t.order;
  if (order >= 5) {
    const uint32_t x = blk & 7u, q = t.nwg >> 3, r = t.nwg & 7u;
    blk = x * q + (x < r ? x : r) + (blk >> 3);
    order -= 5;
  }
  if (order == 0) {
    uint32_t r1 = fdiv(blk, t.fd_ta);
    ta = blk - r1 * t.tiles_a;
    r2 = fdiv(r1, t.fd_tb);
    tb = r1 - r2 * t.tiles_b;
  } else if (order == 1) {
    uint32_t r1 = fdiv(blk, t.fd_tb);
    tb = blk - r1 * t.tiles_b;
    r2 = fdiv(r1, t.fd_ta);
    ta = r1 - r2 * t.tiles_a;
  } else if (order == 2) {
    // diagonal: consecutive workgroups take consecutive a-tiles and, with them,
    // shifted b-tiles, so that neither the rows they read nor the rows they write
    // share one column offset (power-of-two pitches otherwise land every row of a
    // tile band on the same HBM channels)
    uint32_t r1 = fdiv(blk, t.fd_ta);
    ta = blk - r1 * t.tiles_a;
    r2 = fdiv(r1, t.fd_tb);
    uint32_t ta_mod = ta - fdiv(ta, t.fd_tb) * t.tiles_b;  // ta % tiles_b
    uint32_t d = (r1 - r2 * t.tiles_b) + ta_mod;            // < 2 * tiles_b
    tb = d >= t.tiles_b ? d - t.tiles_b : d;
  } else if (order == 4) {
    // the diagonal with the roles of a and b swapped: consecutive workgroups take
    // consecutive b-tiles and, with them, shifted a-tiles
    uint32_t r1 = fdiv(blk, t.fd_tb);
    tb = blk - r1 * t.tiles_b;
    r2 = fdiv(r1, t.fd_ta);
    uint32_t tb_mod = tb - fdiv(tb, t.fd_ta) * t.tiles_a;  // tb % tiles_a
    uint32_t d = (r1 - r2 * t.tiles_a) + tb_mod;            // < 2 * tiles_a
    ta = d >= t.tiles_a ? d - t.tiles_a : d;
  } else {
    // grouped diagonal: 16 consecutive workgroups cover a 4 x 4 group of tiles,
    // so the workgroups in flight read and write 4 adjacent tile rows' worth of
    // contiguous bytes per row (DRAM page locality on both sides), and the groups
    // themselves are laid out diagonally as above (channel spread).  Needs
    // tiles_a and tiles_b to be multiples of 4; gta = tiles_a / 4, gtb = tiles_b / 4.
    const uint32_t g = blk >> 4, w = blk & 15u;
    uint32_t r1 = fdiv(g, t.fd_gta);
    const uint32_t ga = g - r1 * t.gta;
    r2 = fdiv(r1, t.fd_gtb);
    const uint32_t ga_mod = ga - fdiv(ga, t.fd_gtb) * t.gtb;
    const uint32_t d = (r1 - r2 * t.gtb) + ga_mod;
    const uint32_t gb = d >= t.gtb ? d - t.gtb : d;
    ta = 4 * ga + (w & 3u);
    tb = 4 * gb + (w >> 2);
  }
}

// Tile of (TA*V) x (TB*V) elements per workgroup of TA*TB/R lanes; each lane owns R
// V x V register blocks (the second TB/R block rows further along b): V chunk loads
// of V elements along a per block (one per b row), an in-register transpose, V chunk
// stores of V elements along b (one per a row).  V*EB == 16 normally, so every
// global access is a 16-byte vector.
//
// LDS == true: the transposed chunks go through LDS so that a wave's stores run
// along TB consecutive chunks of one dst row (TB*16 contiguous bytes per row for
// 16-B chunks).  The LDS tile is addressed [row][chunk ^ ((row / V) % TB)], an XOR
// swizzle of the 16-byte chunk index ([print_layout page, sections 4.3 and 5.2]:
// XOR spreads a column across banks, where padding would also do), so both the
// chunk writes (lanes of one chunk column) and the row reads (lanes of one row)
// touch distinct chunk slots of a bank window.
// LDS == false (TA == TB == 16 only): lanes are arranged 8 x 8 per wave so each
// load and store instruction covers eight full 128-byte lines, with no LDS.
template <int EB, int V, bool LDS, int TA, int TB, bool NT, int R = 1>
__global__ void __launch_bounds__(TA * TB / R) k_transpose(TransposeArgs t) {
  using T = typename Raw<EB>::T;
  using C = Chunk<T, V>;
  constexpr int NTH = TA * TB / R;  // threads: R register blocks per lane
  static_assert(LDS || (TA == 16 && TB == 16 && R == 1), "the direct variant uses 16 x 16 blocks");
  static_assert(R == 1 || R == 2, "one or two blocks per lane");
  static_assert(TB % R == 0, "whole rows of blocks per lane group");
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;

  uint32_t ta, tb, r2;
  transpose_tile(t, blockIdx.x, ta, tb, r2);
  uint32_t bs, bd;
  batch_offsets(t.batch, r2, &bs, &bd);

  const int tid = threadIdx.x;
  int alpha, beta;  // the lane's first block; its others lie TB / R block rows further along b
  if (LDS) {
    alpha = tid % TA;
    beta = tid / TA;
  } else {
    const int lane = tid & 63, w = tid >> 6;
    alpha = (lane & 7) + 8 * (w & 1);
    beta = (lane >> 3) + 8 * (w >> 1);
  }
  const uint32_t a0 = ta * (TA * V), b0 = tb * (TB * V);
  const uint32_t a_blk = a0 + V * alpha;
  bool valid[R];
  C in[R][V];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t b_blk = b0 + V * (beta + (TB / R) * r);
    valid[r] = a_blk < t.ext_a && b_blk < t.ext_b;
    if (valid[r]) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const uint32_t b = b_blk + j;
        uint32_t so = swz32(a_blk + (b & t.bmask) * t.ss_b + (b >> t.bshift) * t.ss_b2 + bs, t.sws);
        in[r][j] = gload<NT, C>(src + (size_t)so * EB);
      }
    }
  }
  C out[R][V];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int j = 0; j < V; ++j) out[r][i].e[j] = in[r][j].e[i];

  if (!LDS) {
    if (valid[0]) {
      const uint32_t b_blk = b0 + V * beta;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        uint32_t dof = swz32((a_blk + i) * t.sd_a + b_blk + bd, t.swd);
        gstore<NT, C>(dst + (size_t)dof * EB, out[0][i]);
        count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, sizeof(C));
      }
    }
    return;
  }

  __shared__ C tile[TA * V][TB];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (valid[r]) {
      const int bt = beta + (TB / R) * r;
#pragma unroll
      for (int i = 0; i < V; ++i) tile[V * alpha + i][bt ^ (alpha % TB)] = out[r][i];
    }
  }
  __syncthreads();
  const int c = tid % TB;
  if constexpr (NT && sizeof(C) == 16) {
    if (t.bufst) {
      // Streaming 16-byte stores as buffer stores with the nt and sc1 policy bits,
      // which measured faster than nt alone for this access pattern.  Offsets are
      // taken from the tile's lowest destination offset (every stored offset of
      // the tile is at or above it: a >= a0, b >= b0, and the swizzle changes only
      // bits under ~bufmask).
      const uint32_t tbase = (a0 * t.sd_a + b0 + bd) & t.bufmask;
      const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst + (size_t)tbase * EB, 0, -1, kBufferWord3);
#pragma unroll
      for (int k = 0; k < V * R; ++k) {
        const int row = tid / TB + (NTH / TB) * k;
        const uint32_t a = a0 + row, b = b0 + V * c;
        if (a < t.ext_a && b < t.ext_b) {
          C v = tile[row][c ^ ((row / V) % TB)];
          const uint32_t dof = swz32(a * t.sd_a + b + bd, t.swd);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(typename NativeOf<16>::T, v), rd,
                                                 (dof - tbase) * EB, 0, kPolicyNtSc1);
          count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, 16);
        }
      }
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < V * R; ++k) {
    const int row = tid / TB + (NTH / TB) * k;
    const uint32_t a = a0 + row, b = b0 + V * c;
    if (a < t.ext_a && b < t.ext_b) {
      C v = tile[row][c ^ ((row / V) % TB)];
      uint32_t dof = swz32(a * t.sd_a + b + bd, t.swd);
      gstore<NT, C>(dst + (size_t)dof * EB, v);
      count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, sizeof(C));
    }
  }
}

// Element-granular tile transpose, for copies whose rows do not allow aligned
// chunks of several elements (odd pitches, ragged extents): a tile of E x E
// elements with E = 256 / EB, so every row segment on either side is 256 bytes.
// Load: consecutive lanes read consecutive elements of a source row (a wave
// instruction covers whole 128-byte lines); the elements go to LDS as rows of the
// source.  Store: consecutive lanes take consecutive elements of a destination row,
// i.e. one column of the LDS tile, whose rows are padded by one 4-byte word (two
// for 8-byte elements) so that the lanes of a phase fall on distinct banks.
template <int EB, bool NT>
__global__ void __launch_bounds__(512) k_transpose_el(TransposeArgs t) {
  using T = typename Raw<EB>::T;
  static_assert(EB <= 8, "16-byte elements use the chunk transpose");
  constexpr int E = 256 / EB;                 // tile extent in elements, both axes
  constexpr int PITCH = 256 + (EB > 4 ? 8 : 4);  // LDS bytes per tile row
  constexpr int NTH = 512;
  constexpr int PER = E * E / NTH;            // elements per lane and phase
  constexpr int BATCH = PER < 8 ? PER : 8;    // loads in flight per lane
  static_assert(PER % BATCH == 0, "whole batches");
  __shared__ __align__(16) char tile[E * PITCH];
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;

  uint32_t ta, tb, r2;
  transpose_tile(t, blockIdx.x, ta, tb, r2);
  uint32_t bs, bd;
  batch_offsets(t.batch, r2, &bs, &bd);
  const uint32_t a0 = ta * E, b0 = tb * E;
  const int tid = threadIdx.x;

  // source rows b, elements a along each row
#pragma unroll
  for (int i0 = 0; i0 < PER; i0 += BATCH) {
    T v[BATCH] = {};
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int e = tid + NTH * (i0 + i);
      const uint32_t a = a0 + e % E, b = b0 + e / E;
      if (a < t.ext_a && b < t.ext_b) {
        const uint32_t so = swz32(a + (b & t.bmask) * t.ss_b + (b >> t.bshift) * t.ss_b2 + bs, t.sws);
        v[i] = gload<NT, T>(src + (size_t)so * EB);
      }
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int e = tid + NTH * (i0 + i);
      *(T*)(tile + (e / E) * PITCH + (e % E) * EB) = v[i];
    }
  }
  __syncthreads();
  // destination rows a, elements b along each row
#pragma unroll
  for (int i0 = 0; i0 < PER; i0 += BATCH) {
    T v[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int e = tid + NTH * (i0 + i);
      v[i] = *(const T*)(tile + (e % E) * PITCH + (e / E) * EB);
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int e = tid + NTH * (i0 + i);
      const uint32_t a = a0 + e / E, b = b0 + e % E;
      if (a < t.ext_a && b < t.ext_b) {
        const uint32_t dof = swz32(a * t.sd_a + b + bd, t.swd);
        gstore<NT, T>(dst + (size_t)dof * EB, v[i]);
        count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, EB);
      }
    }
  }
}

// The same element tiles with 16-byte accesses inside each row, for layouts without
// swizzles on element-aligned buffers.  Every tile row on either side is one
// contiguous range of at most 256 bytes (unaligned in general: an odd pitch moves
// each row's start by EB bytes modulo 16); it moves as its aligned interior in
// 16-byte chunks plus single elements at its two ends.  A lane takes chunk j of a
// row, 16 lanes a row.  The LDS tile keeps the source rows in element order, so a
// chunk goes in, or is gathered out, one element at a time at fixed offsets from
// the lane's address.  Its row pitch of 256 + EB bytes spreads the lanes that
// gather destination chunks (rows V apart) over the banks: two lanes a bank.
template <int EB, bool NT>
__global__ void __launch_bounds__(512) k_transpose_win(TransposeArgs t) {
  using T = typename Raw<EB>::T;
  static_assert(EB <= 8, "16-byte elements use the chunk transpose");
  constexpr uint32_t V = 16 / EB;
  using Ch = Chunk<T, V>;
  constexpr uint32_t E = 256 / EB;        // tile extent in elements, both axes
  constexpr uint32_t P = 256 + EB;        // LDS bytes per tile row
  constexpr uint32_t ROWS = E / 32;       // rows per lane on either side
  constexpr uint32_t NE = V > 8 ? 2 : 1;  // edge elements per lane and row (under 2 V a row)
  __shared__ __align__(16) char tile[E * P];
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;

  uint32_t ta, tb, r2;
  transpose_tile(t, blockIdx.x, ta, tb, r2);
  uint32_t bs, bd;
  batch_offsets(t.batch, r2, &bs, &bd);
  const uint32_t a0 = ta * E, b0 = tb * E;
  const uint32_t na = t.ext_a - a0 < E ? t.ext_a - a0 : E;  // tile extents (ragged at the ends)
  const uint32_t nb = t.ext_b - b0 < E ? t.ext_b - b0 : E;
  const uint32_t j = threadIdx.x & 15u, rl = threadIdx.x >> 4;

  // source rows b (elements a0 .. a0 + na - 1 of each) -> LDS rows in element order;
  // 1-byte elements in two batches of rows, so that the bytes unpacked for the LDS
  // writes stay under 128 VGPRs (two workgroups a CU)
  constexpr uint32_t BATCHES = EB == 1 ? 2 : 1;
  constexpr uint32_t RB = ROWS / BATCHES;
#pragma unroll
  for (uint32_t h = 0; h < BATCHES; ++h) {
    Ch v[RB];
    T e[RB][NE];
    uint32_t hd[RB], ni[RB], ht[RB], a1[RB];
#pragma unroll
    for (uint32_t i = 0; i < RB; ++i) {
      const uint32_t b = rl + 32u * (h * RB + i), bb = b0 + b;
      ni[i] = 0;
      ht[i] = 0;
      if (b < nb) {
        const char* g = src + (size_t)(a0 + (bb & t.bmask) * t.ss_b + (bb >> t.bshift) * t.ss_b2 + bs) * EB;
        const WinSplit<EB> w(g, na * EB);
        hd[i] = w.head;
        ni[i] = w.nint;
        ht[i] = w.head + w.tail;
        a1[i] = w.a1;
        if (j < w.nint) v[i] = gload<NT, Ch>(g + w.a0 + 16u * j);
#pragma unroll
        for (uint32_t u = 0; u < NE; ++u) {
          const uint32_t k = j + 16u * u;
          if (k < ht[i]) e[i][u] = gload<NT, T>(g + (k < w.head ? k * EB : w.a1 + (k - w.head) * EB));
        }
      }
    }
#pragma unroll
    for (uint32_t i = 0; i < RB; ++i) {
      char* row = tile + (rl + 32u * (h * RB + i)) * P;
      if (j < ni[i]) {
        const uint32_t x = hd[i] * EB + 16u * j;  // byte of the chunk's first element in the row
#pragma unroll
        for (uint32_t k = 0; k < V; ++k) *(T*)(row + x + k * EB) = v[i].e[k];
      }
#pragma unroll
      for (uint32_t u = 0; u < NE; ++u) {
        const uint32_t k = j + 16u * u;
        if (k < ht[i]) *(T*)(row + (k < hd[i] ? k * EB : a1[i] + (k - hd[i]) * EB)) = e[i][u];
      }
    }
  }
  __syncthreads();
  // destination rows a (elements b0 .. b0 + nb - 1 of each), gathered down LDS columns
#pragma unroll
  for (uint32_t i = 0; i < ROWS; ++i) {
    const uint32_t a = rl + 32u * i;
    if (a < na) {
      char* g = dst + (size_t)((a0 + a) * t.sd_a + b0 + bd) * EB;
      const WinSplit<EB> w(g, nb * EB);
      const char* col = tile + a * EB;
      if (j < w.nint) {
        const char* c0 = col + (w.head + V * j) * P;
        Ch o;
#pragma unroll
        for (uint32_t k = 0; k < V; ++k) o.e[k] = *(const T*)(c0 + k * P);
        gstore<NT, Ch>(g + w.a0 + 16u * j, o);
        count_store(t.wcnt, t.dst, g + w.a0 + 16u * j, 16);
      }
#pragma unroll
      for (uint32_t u = 0; u < NE; ++u) {
        const uint32_t k = j + 16u * u;
        if (k < w.head + w.tail) {
          const uint32_t b = k < w.head ? k : w.head + V * w.nint + (k - w.head);
          gstore<NT, T>(g + (size_t)b * EB, *(const T*)(col + b * P));
          count_store(t.wcnt, t.dst, g + (size_t)b * EB, EB);
        }
      }
    }
  }
}

// Transpose of a V x V block of EB-byte elements held as V 16-byte rows (V * EB ==
// 16): element j of out[i] is element i of in[j].  Written on 32-bit words with
// v_perm_b32 so that the rows stay whole 16-byte values: read from LDS element by
// element, the compiler splits each row into unaligned 2- and 12-byte pieces.
// __builtin_amdgcn_perm(a, b, sel): byte k of the result is byte sel_k of the
// 8-byte value a:b (b holds bytes 0-3, a bytes 4-7); selector 12 gives zero.
template <int EB>
__device__ __forceinline__ void transpose_rows16(const U4* in, U4* out) {
  if constexpr (EB == 16) {
    out[0] = in[0];
  } else if constexpr (EB == 8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) out[i] = U4{in[0][2 * i], in[0][2 * i + 1], in[1][2 * i], in[1][2 * i + 1]};
  } else if constexpr (EB == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = U4{in[0][i], in[1][i], in[2][i], in[3][i]};
  } else if constexpr (EB == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of two words
#pragma unroll
      for (int q = 0; q < 4; ++q) out[i][q] = __builtin_amdgcn_perm(in[2 * q + 1][i / 2], in[2 * q][i / 2], sel);
    }
  } else {
    static_assert(EB == 1, "elements of 1, 2, 4, 8 or 16 bytes");
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t pair = 0x0c0c0000u | (uint32_t)(i % 4) | ((uint32_t)(4 + i % 4) << 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = __builtin_amdgcn_perm(in[4 * q + 1][i / 4], in[4 * q][i / 4], pair);
        const uint32_t hi = __builtin_amdgcn_perm(in[4 * q + 3][i / 4], in[4 * q + 2][i / 4], pair);
        out[i][q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
    }
  }
}

// The same tile with its source chunks loaded straight into LDS (gfx950 direct
// loads): the tile's TB*V source rows of TA chunks land in LDS without passing
// through registers.  A direct load fills 64 consecutive 16-byte slots per wave, so
// lane l of load k of wave w takes slot 64 * (w * V + k) + l and loads the source
// chunk that belongs there: slot r * TA + (c ^ lds_swz(r)) holds chunk column c of
// tile row r (b index b0 + r).  Two ways to read the tile back:
//  - whole rows (TR false): lane tid = beta + TB * alpha reads its V x V block (V
//    chunks of chunk column alpha, rows V*beta .. V*beta+V-1) as V 16-byte rows,
//    transposes it in registers and stores V chunks; TB consecutive lanes store TB
//    consecutive chunks of one destination row.  lds_swz(r) = (r / V) % 16, so the 16
//    lanes of a 16-byte read phase (consecutive beta) fall on 16 distinct slots
//    modulo 16, i.e. all 64 banks.
//  - gfx950 transpose reads (TR true, 2-byte elements): ds_read_b64_tr_b16 hands lane
//    i of each 16-lane group element i % 4 of the 8 bytes that lane 4k + i / 4 of the
//    group addresses, as its element k (k = 0..3).  Lane j of a group addresses row
//    j / 4 of b-chunk j % 4 (and, in a second read, row j / 4 + 4), in the 8-byte half
//    of the chunk column its group owns, so lane i receives one column (element i % 4
//    of that half) of the 8 rows of b-chunk i / 4: a whole 16-byte destination chunk
//    from two reads, with no register transpose.  The four groups of a wave cover both
//    halves of one chunk column and 8 b-chunks (8 destination rows x 128 bytes per
//    store instruction).  lds_swz(r) = (r % 4) + 4 * ((r / 8) % 4), so the 16 rows a
//    group addresses fall on 16 distinct slots modulo 16 and, with the two groups of a
//    32-lane phase on different halves, the phase's 32 8-byte reads on all 64 banks.
//  - the same for 1-byte elements (TR true, V = 16) with ds_read_b64_tr_b8, which
//    hands lane i of each group byte i % 8 of the 8 bytes that lane 2k + i / 8
//    addresses, as its byte k (k = 0..7); see dl_consume.  lds_swz(r) = (r % 8) +
//    8 * ((r / 16) % 2).
// Needs full 16-byte chunks (V * EB == 16), TB >= 16 and TA in {16, 32}.
template <int EB, int V, bool TR>
__device__ __forceinline__ int lds_swz(int r) {
  if constexpr (TR && EB == 2)
    return (r & 3) | (((r >> 3) & 3) << 2);
  else if constexpr (TR)
    return (r & 7) | (((r >> 4) & 1) << 3);
  else
    return (r / V) % 16;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// gfx950 transpose read of 2-byte elements (ds_read_b64_tr_b16), as two 32-bit words.
__device__ __forceinline__ NativeOf<8>::T lds_read_tr16(const char* p) {
  return __builtin_bit_cast(NativeOf<8>::T, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)const_cast<char*>(p)));
}

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

// gfx950 transpose read of 1-byte elements (ds_read_b64_tr_b8): lane i of each
// 16-lane group receives, as its byte k (k = 0..7), byte i % 8 of the 8 bytes that
// lane 2k + i / 8 of the group addresses.
__device__ __forceinline__ NativeOf<8>::T lds_read_tr8(const char* p) {
  return __builtin_bit_cast(NativeOf<8>::T, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)const_cast<char*>(p)));
}

// Direct loads of tile blk into buf.  ALL: every lane issues its V loads, a chunk
// outside the layout loading the chunk at offset 0 into a slot no output reads (the
// pipelined kernel counts outstanding loads); otherwise such lanes load nothing.
// The chunk at offset 0 is in the source buffer: the a mode is contiguous in the
// source with an extent that is a multiple of V.
template <int EB, int V, int TA, int TB, bool NT, bool TR, bool ALL>
__device__ __forceinline__ void dl_issue(const TransposeArgs& t, uint32_t blk, Chunk<typename Raw<EB>::T, V>* buf) {
  const char* __restrict__ src = (const char*)t.src;
  uint32_t ta, tb, r2;
  transpose_tile(t, blk, ta, tb, r2);
  uint32_t bs, bd;
  batch_offsets(t.batch, r2, &bs, &bd);
  const uint32_t a0 = ta * (TA * V), b0 = tb * (TB * V);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const int base = 64 * (wave * V + k);  // first slot of this wave's load
    const int s = base + lane;
    const int r = s / TA, cs = s % TA;
    const int c = cs ^ lds_swz<EB, V, TR>(r);   // chunk column stored in slot s
    const uint32_t a = a0 + V * c, b = b0 + r;
    const bool in = a < t.ext_a && b < t.ext_b;
    if (!ALL && !in) continue;
    uint32_t so = 0;
    if (in) so = swz32(a + (b & t.bmask) * t.ss_b + (b >> t.bshift) * t.ss_b2 + bs, t.sws);
    load_to_lds16<NT>(src + (size_t)so * EB, buf + __builtin_amdgcn_readfirstlane(base));
  }
}

// Reads tile blk back from buf (see above for the two forms) and stores it.
template <int EB, int V, int TA, int TB, bool NT, bool TR>
__device__ __forceinline__ void dl_consume(const TransposeArgs& t, uint32_t blk,
                                           const Chunk<typename Raw<EB>::T, V>* buf) {
  char* __restrict__ dst = (char*)t.dst;
  uint32_t ta, tb, r2;
  transpose_tile(t, blk, ta, tb, r2);
  uint32_t bs, bd;
  batch_offsets(t.batch, r2, &bs, &bd);
  const uint32_t a0 = ta * (TA * V), b0 = tb * (TB * V);
  if constexpr (!TR) {
    const int beta = threadIdx.x % TB, alpha = threadIdx.x / TB;
    const U4* rows = (const U4*)buf;
    U4 in[V], out[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int r = V * beta + j;
      in[j] = rows[r * TA + (alpha ^ lds_swz<EB, V, false>(r))];
    }
    transpose_rows16<EB>(in, out);
    const uint32_t b = b0 + V * beta;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const uint32_t a = a0 + V * alpha + i;
      if (a < t.ext_a && b < t.ext_b) {
        const uint32_t dof = swz32(a * t.sd_a + b + bd, t.swd);
        gstore<NT, U4>(dst + (size_t)dof * EB, out[i]);
        count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, 16);
      }
    }
  } else if constexpr (EB == 1) {
    // 1-byte elements in 16-byte chunks (V = 16).  A unit is one 8-byte half h of chunk
    // column c by 8 b-chunks from 8 * bq: 8 destination rows of 128 bytes, one whole
    // line each, over the wave's 64 lanes.  Lane j of group g addresses row j / 2 (and
    // j / 2 + 8) of b-chunk 2g + j % 2 in half h, so lane i receives destination row
    // 16c + 8h + i % 8, b-chunk 2g + i / 8: one whole 16-byte destination chunk from
    // two reads.  A 32-lane phase reads 32 rows in one half, so its reads land two to
    // a bank at best; the row swizzle (r % 8) + 8 * ((r / 16) % 2) makes it exactly two.
    // (Units of both halves of a column over 16 rows, conflict-free, stored 64-byte
    // row segments and ran 25 % slower.)
    static_assert(V == 16, "transpose reads: 1-byte elements in 16-byte chunks");
    constexpr int UB = TB / 8;              // units of 8 b-chunks along b
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int sk = i >> 1, sp = i & 1;      // addressed: row sk (and sk + 8) of b-chunk 2g + sp
    const int e = i & 7, q = i >> 3;        // received: row 8h + e of the column, b-chunk 2g + q
    const char* base = (const char*)buf;
    // a wave's 16 units (the tile's TA * 2 * UB units over its TA * TB / 64 waves); all
    // 32 reads go out before the first store
    NativeOf<8>::T lo[16], hi[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int u = w * 16 + it;
      const int bq = u % UB, h = (u / UB) & 1, c = u / (2 * UB);
      const int r0 = 16 * (8 * bq + 2 * g + sp) + sk, r1 = r0 + 8;
      lo[it] = lds_read_tr8(base + (r0 * TA + (c ^ lds_swz<EB, V, true>(r0))) * 16 + 8 * h);
      hi[it] = lds_read_tr8(base + (r1 * TA + (c ^ lds_swz<EB, V, true>(r1))) * 16 + 8 * h);
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int u = w * 16 + it;
      const int bq = u % UB, h = (u / UB) & 1, c = u / (2 * UB);
      const uint32_t a = a0 + V * c + 8 * h + e;
      const uint32_t b = b0 + V * (8 * bq + 2 * g + q);
      if (a < t.ext_a && b < t.ext_b) {
        const U4 o = {lo[it][0], lo[it][1], hi[it][0], hi[it][1]};
        const uint32_t dof = swz32(a * t.sd_a + b + bd, t.swd);
        gstore<NT, U4>(dst + (size_t)dof * EB, o);
        count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, 16);
      }
    }
  } else {
    static_assert(EB == 2 && V == 8, "transpose reads: 2-byte elements in 16-byte chunks");
    constexpr int UB = TB / 8;              // units of 8 b-chunks along b
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int half = g & 1, bh = g >> 1;     // the group's 8-byte half of the chunk column; its 4 of the 8 b-chunks
    const int sk = i >> 2, sq = i & 3;       // addressed: row sk (and sk + 4) of b-chunk sq
    const int e = i & 3, q = i >> 2;         // received: element e of the half, b-chunk q
    const char* base = (const char*)buf;
    // a wave's 8 units: chunk column c, 8 b-chunks from 8 * ub (the tile's TA * UB
    // units over its TA * TB / 64 waves).  All 16 reads go out before the first store
    // (the compiler keeps these reads in order with the stores).
    NativeOf<8>::T lo[8], hi[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int u = w * 8 + it;
      const int c = u / UB, ub = u % UB;
      const int r0 = 64 * ub + 8 * (4 * bh + sq) + sk, r1 = r0 + 4;
      lo[it] = lds_read_tr16(base + (r0 * TA + (c ^ lds_swz<EB, V, true>(r0))) * 16 + 8 * half);
      hi[it] = lds_read_tr16(base + (r1 * TA + (c ^ lds_swz<EB, V, true>(r1))) * 16 + 8 * half);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int u = w * 8 + it;
      const int c = u / UB, ub = u % UB;
      const uint32_t a = a0 + V * c + 4 * half + e;
      const uint32_t b = b0 + V * (8 * ub + 4 * bh + q);
      if (a < t.ext_a && b < t.ext_b) {
        const U4 o = {lo[it][0], lo[it][1], hi[it][0], hi[it][1]};
        const uint32_t dof = swz32(a * t.sd_a + b + bd, t.swd);
        gstore<NT, U4>(dst + (size_t)dof * EB, o);
        count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, 16);
      }
    }
  }
}

template <int EB, int V, int TA, int TB, bool NT, bool TR>
__global__ void __launch_bounds__(TA * TB) k_transpose_dl(TransposeArgs t) {
  using C = Chunk<typename Raw<EB>::T, V>;
  static_assert(V * EB == 16 && TB >= 16 && (TA == 16 || TA == 32), "full chunks, 16-wide phases");
  __shared__ C tile[TB * V * TA];
  dl_issue<EB, V, TA, TB, NT, TR, false>(t, blockIdx.x, tile);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
  __syncthreads();
  dl_consume<EB, V, TA, TB, NT, TR>(t, blockIdx.x, tile);
}

// Vector-memory wait counts for s_waitcnt on gfx950 (vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Software-pipelined transpose ([CuTe algebra page, section 5.2]: the next tile's
// copy is issued while the current one is consumed).  A workgroup takes t.pipe
// consecutive tiles (in the order t.order selects) and alternates two LDS tiles:
// the gfx950 direct global -> LDS loads of tile i+1 are issued before tile i is
// read from LDS and stored, so each CU has loads and stores in flight together.
// LDS arrangement and lane roles as k_transpose_dl.  Every lane issues exactly V
// loads per tile, so "at most V vector-memory operations outstanding" means the
// current tile has landed: loads complete in the order they were issued.  The two
// buffers are distinct LDS objects and the loop names them statically, so the
// compiler's own LDS-DMA tracking waits for the right one only.  Barriers are plain
// s_barrier with explicit waits: a __syncthreads() fence would drain the next tile's
// loads too.
template <int EB, int V, int TA, int TB, bool NT, bool TR>
__global__ void __launch_bounds__(TA * TB) k_transpose_pipe(TransposeArgs t) {
  using C = Chunk<typename Raw<EB>::T, V>;
  static_assert(V * EB == 16 && TB >= 16 && (TA == 16 || TA == 32), "full chunks, 16-wide phases");
  static_assert(2 * TB * V * TA * 16 <= 160 * 1024, "two tiles fit the LDS");
  __shared__ C bufA[TB * V * TA];
  __shared__ C bufB[TB * V * TA];
  const uint32_t first = blockIdx.x * t.pipe;
  const uint32_t last = first + t.pipe < t.ntiles ? first + t.pipe : t.ntiles;
  uint32_t i = first;
  dl_issue<EB, V, TA, TB, NT, TR, true>(t, i, bufA);
  // Steady state, three or more tiles left: tile i is landing in A.  The waits are
  // unconditional so that the compiler's own LDS-DMA tracking sees, on every path
  // to a read, the wait that covers it.
  while (i + 2 < last) {
    dl_issue<EB, V, TA, TB, NT, TR, true>(t, i + 1, bufB);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(V));  // all but tile i + 1's loads: A has landed
    __builtin_amdgcn_s_barrier();
    dl_consume<EB, V, TA, TB, NT, TR>(t, i, bufA);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);     // this wave's reads of A are done
    __builtin_amdgcn_s_barrier();
    dl_issue<EB, V, TA, TB, NT, TR, true>(t, i + 2, bufA);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(V));
    __builtin_amdgcn_s_barrier();
    dl_consume<EB, V, TA, TB, NT, TR>(t, i + 1, bufB);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    i += 2;
  }
  // one or two tiles left, the first of them landing in A
  if (i + 1 < last) {
    dl_issue<EB, V, TA, TB, NT, TR, true>(t, i + 1, bufB);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(V));
    __builtin_amdgcn_s_barrier();
    dl_consume<EB, V, TA, TB, NT, TR>(t, i, bufA);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    dl_consume<EB, V, TA, TB, NT, TR>(t, i + 1, bufB);
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    dl_consume<EB, V, TA, TB, NT, TR>(t, i, bufA);
  }
}

// ------------------------------------------------------------------ interleave

struct InterleaveArgs {
  const void* src;
  void* dst;
  uint32_t ext_a;        // src-contiguous mode; dst stride of a == NB
  uint32_t ss_b;         // src stride of the short dst-contiguous mode b (extent NB)
  uint32_t tiles_a;
  FD fd_ta;
  BatchArg batch;
  SwzArg sws, swd;
  uint32_t bufst;        // 1: streaming stores as buffer stores from dst (span < 4 GiB)
  WriteCount wcnt;
};

// The dst-contiguous mode b is short (NB * EB <= 16 bytes) and a follows it in
// dst, so V consecutive a positions times NB form NB contiguous dst chunks.  This
// is the pairing of [print_layout page, section 4.2] (two heads side by side so
// one wide load brings both), done in registers.
//   NARROW == false: each lane loads NB 16-byte chunks (one per b) and writes
//     them interleaved as NB chunks;
//   NARROW == true: each lane writes one 16-byte dst chunk, built from NB loads of
//     16/NB bytes (P = V/NB positions of a, one load per b), so that every store
//     instruction of a wave covers 1 KiB of contiguous dst.  One chunk per lane:
//     more per lane measured slower.
template <int EB, int NB, bool NARROW, bool NT, int L = 256>
__global__ void __launch_bounds__(L) k_interleave(InterleaveArgs t) {
  static_assert(L == 256 || NARROW, "narrower workgroups on the narrow form");
  using T = typename Raw<EB>::T;
  constexpr int V = 16 / EB;
  using C = Chunk<T, V>;
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;

  uint32_t blk = blockIdx.x;
  uint32_t r1 = fdiv(blk, t.fd_ta);
  uint32_t ta = blk - r1 * t.tiles_a;
  uint32_t bs, bd;
  batch_offsets(t.batch, r1, &bs, &bd);

  if constexpr (NARROW) {
    constexpr int P = V / NB;  // a positions per dst chunk
    using H = Chunk<T, P>;
    constexpr int U = 1;  // dst chunks per lane: one measured fastest (6.55 against 6.27 TB/s for two)
    H in[U][NB];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = ta * (L * U) + u * L + threadIdx.x;  // dst chunk index
      const uint32_t a0 = j * P;
      ok[u] = a0 < t.ext_a;
      if (ok[u]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          uint32_t so = swz32(a0 + b * t.ss_b + bs, t.sws);
          in[u][b] = gload<NT, H>(src + (size_t)so * EB);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      const uint32_t j = ta * (L * U) + u * L + threadIdx.x;
      C o;
#pragma unroll
      for (int x = 0; x < V; ++x) o.e[x] = in[u][x % NB].e[x / NB];
      uint32_t dof = swz32(j * V + bd, t.swd);
      if constexpr (NT) {
        if (t.bufst) {  // nt and sc1 policy bits; the host checks the 4 GiB span
          const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst, 0, -1, kBufferWord3);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(typename NativeOf<16>::T, o), rd, dof * EB, 0,
                                                 kPolicyNtSc1);
          count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, 16);
          continue;
        }
      }
      gstore<NT, C>(dst + (size_t)dof * EB, o);
      count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, sizeof(C));
    }
  } else {
    constexpr int U = NB >= 8 ? 1 : 8 / NB;  // a-chunks per lane: U * NB loads in flight
    C in[U][NB];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t a0 = (ta * (256 * U) + u * 256 + threadIdx.x) * V;
      ok[u] = a0 < t.ext_a;
      if (ok[u]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          uint32_t so = swz32(a0 + b * t.ss_b + bs, t.sws);
          in[u][b] = gload<NT, C>(src + (size_t)so * EB);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      uint32_t a0 = (ta * (256 * U) + u * 256 + threadIdx.x) * V;
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        C o;
#pragma unroll
        for (int x = 0; x < V; ++x) {
          const int e = c * V + x;  // element a0*NB + e: a = a0 + e / NB, b = e % NB
          o.e[x] = in[u][e % NB].e[e / NB];
        }
        uint32_t dof = swz32(a0 * NB + c * V + bd, t.swd);
        gstore<NT, C>(dst + (size_t)dof * EB, o);
        count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, sizeof(C));
      }
    }
  }
}

// ------------------------------------------------------------------ channel shuffle

struct ChanArgs {
  const void* src;
  void* dst;
  uint32_t pixels;   // extent of the pixel mode (a multiple of the chunk's V elements)
  uint32_t plane;    // stride of the channel mode on the planar side (elements)
  uint32_t tiles;    // workgroups per batch index: pixels / (256 V), rounded up
  FD fd_tiles;
  BatchArg batch;
  uint32_t bufst;    // 1: streaming stores as buffer stores from dst (span < 4 GiB)
  WriteCount wcnt;
};

// A 16-byte streaming store: a buffer store with the nt and sc1 bits from `base`
// when `buf` (the host has checked the 4 GiB span), else a global store.
// The byte offset is 64-bit: a destination may span more than 4 GiB (element
// offsets stay under 2^31, bytes do not); only the buffer store, whose span the
// host has checked, narrows it to its 32-bit offset.
template <bool NT, typename C>
__device__ __forceinline__ void store16(char* base, size_t byte_off, const C& v, bool buf) {
  static_assert(sizeof(C) == 16, "16-byte chunks");
  if constexpr (NT) {
    if (buf) {
      const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(base, 0, -1, kBufferWord3);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(typename NativeOf<16>::T, v), rd,
                                             (uint32_t)byte_off, 0, kPolicyNtSc1);
      return;
    }
  }
  gstore<NT, C>(base + byte_off, v);
}

// Pixels with C channels side by side (the interleaved side: pixel stride C,
// channel stride 1) <-> C planes (the planar side: channel stride `plane`, pixel
// stride 1): image layouts such as NHWC <-> NCHW with few channels, where neither
// side has a contiguous run of 16 bytes per channel on the interleaved side.  The
// pairing is that of [print_layout page, section 4.2], for any C from 2 to 8.
// Lane l of a workgroup (L lanes) owns V = 16/EB consecutive pixels of all C channels: C
// chunks on either side, exchanged by a C x V transpose in registers.  On the
// interleaved side those C chunks are contiguous per lane, so that side goes
// through LDS: a wave instruction then moves 64 consecutive chunks on both sides.
//   INTERLEAVE == false (de-interleave): loads of the contiguous interleaved block
//     into LDS, C LDS reads per lane, stores of one chunk per plane;
//   INTERLEAVE == true: loads of one chunk per plane, C LDS writes per lane,
//     stores of the contiguous interleaved block.
template <int EB, int C, bool INTERLEAVE, bool NT, int L = 256>
__global__ void __launch_bounds__(L) k_chan(ChanArgs t) {
  using T = typename Raw<EB>::T;
  constexpr int V = 16 / EB;
  using Ch = Chunk<T, V>;
  __shared__ Ch lds[L * C];
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;

  const uint32_t blk = blockIdx.x;
  const uint32_t r = fdiv(blk, t.fd_tiles);
  const uint32_t tile = blk - r * t.tiles;
  uint32_t bs, bd;
  batch_offsets(t.batch, r, &bs, &bd);
  const uint32_t p0 = tile * (L * V);  // the workgroup's first pixel
  const uint32_t left = (t.pixels - p0) / V;
  const uint32_t nblk = left < (uint32_t)L ? left : (uint32_t)L;  // pixel blocks of V in this workgroup
  const uint32_t l = threadIdx.x;
  const bool mine = l < nblk;

  if constexpr (!INTERLEAVE) {
    // LDS slot of chunk q.  Lane l reads chunks l*C + j: for C odd a 16-lane phase
    // touches 16 distinct chunk slots mod 16 (all 64 banks once); for C = 2, 4, 8 the
    // XOR of bits 4-7 into bits 0-3 (Sw<4,0,4> on chunk indices, [print_layout page,
    // section 4.3]) spreads them the same way, where plain slots would collide C-fold.
    auto slot = [](uint32_t q) { return (C & (C - 1)) == 0 ? q ^ ((q >> 4) & 15u) : q; };
    const char* sb = src + (size_t)(p0 * C + bs) * EB;  // interleaved block: nblk * C chunks
    Ch tmp[C];
#pragma unroll
    for (int j = 0; j < C; ++j)
      if (l + (uint32_t)L * j < nblk * C) tmp[j] = gload<NT, Ch>(sb + (size_t)(l + (uint32_t)L * j) * 16);
#pragma unroll
    for (int j = 0; j < C; ++j)
      if (l + (uint32_t)L * j < nblk * C) lds[slot(l + (uint32_t)L * j)] = tmp[j];
    __syncthreads();
    if (!mine) return;
    Ch in[C], out[C];
#pragma unroll
    for (int j = 0; j < C; ++j) in[j] = lds[slot(l * C + j)];
#pragma unroll
    for (int e = 0; e < C * V; ++e) out[e % C].e[e / C] = in[e / V].e[e % V];  // element e: pixel e / C, channel e % C
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const size_t off = (size_t)(c * t.plane + p0 + V * l + bd) * EB;
      store16<NT>(dst, off, out[c], t.bufst);
      count_store(t.wcnt, t.dst, dst + off, 16);
    }
  } else {
    if (mine) {
      Ch in[C], out[C];
#pragma unroll
      for (int c = 0; c < C; ++c) in[c] = gload<NT, Ch>(src + (size_t)(c * t.plane + p0 + V * l + bs) * EB);
#pragma unroll
      for (int e = 0; e < C * V; ++e) out[e / V].e[e % V] = in[e % C].e[e / C];
#pragma unroll
      for (int j = 0; j < C; ++j) lds[l * C + j] = out[j];
    }
    __syncthreads();
    const size_t db = (size_t)(p0 * C + bd) * EB;
#pragma unroll
    for (int j = 0; j < C; ++j)
      if (l + (uint32_t)L * j < nblk * C) {
        store16<NT>(dst, db + (size_t)(l + (uint32_t)L * j) * 16, lds[l + (uint32_t)L * j], t.bufst);
        count_store(t.wcnt, t.dst, dst + db + (size_t)(l + (uint32_t)L * j) * 16, 16);
      }
  }
}

// Element-granular form of the same exchange, for pixel counts, plane strides or
// batch offsets that leave the planes without aligned 16-byte chunks (a 299 x 299
// image, say), still with 16-byte accesses wherever a range allows them (element-
// aligned pointers).  A workgroup's pixels are one contiguous byte range on the interleaved side
// and one range per channel on the planar side, in general none of them 16-byte
// aligned.  LDS holds the workgroup's pixels as an interleaved image placed at the
// interleaved range's address modulo 16, so that range moves as its aligned interior
// in 16-byte chunks plus single elements at its two ends.  Each planar range moves the
// same way in global memory; its chunks are scattered into (INTERLEAVE) or gathered
// from (de-interleave) the image element by element, at a stride of C elements.  For
// even C that stride would put the lanes of a wave on few LDS banks: the image then
// has one 16-byte pad slot after every 32 (512 bytes), which spreads them.
template <int C>
__device__ __forceinline__ uint32_t win_pos(uint32_t x) {
  if constexpr ((C & 1) == 0) return x + ((x >> 9) << 4);
  return x;
}

template <int EB, int C, bool INTERLEAVE, bool NT>
__global__ void __launch_bounds__(256) k_chan_win(ChanArgs t) {
  using T = typename Raw<EB>::T;
  constexpr uint32_t V = 16 / EB;
  using Ch = Chunk<T, V>;
  constexpr uint32_t PT = 256 * V;                       // pixels per workgroup
  constexpr uint32_t IMG = PT * C * EB + 16;             // image bytes (+ alignment)
  constexpr uint32_t LB = (C & 1) ? IMG : IMG + ((IMG >> 9) + 1) * 16;
  __shared__ __align__(16) unsigned char lds[LB];
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;

  const uint32_t blk = blockIdx.x;
  const uint32_t r = fdiv(blk, t.fd_tiles);
  const uint32_t tile = blk - r * t.tiles;
  uint32_t bs, bd;
  batch_offsets(t.batch, r, &bs, &bd);
  const uint32_t p0 = tile * PT;
  const uint32_t left = t.pixels - p0;
  const uint32_t np = left < PT ? left : PT;  // pixels in this workgroup
  const uint32_t l = threadIdx.x;

  // the interleaved range and its place in the image: image byte m + (p C + c) EB
  // holds pixel p, channel c
  const char* gi = INTERLEAVE ? dst + (size_t)(p0 * C + bd) * EB : src + (size_t)(p0 * C + bs) * EB;
  const uint32_t m = (uint32_t)((uintptr_t)gi & 15u);
  const uint32_t ilen = np * C * EB;
  const WinSplit<EB> wi(gi, ilen);

  if constexpr (!INTERLEAVE) {
    // interleaved range -> image
    Ch v[C];
#pragma unroll
    for (uint32_t j = 0; j < (uint32_t)C; ++j)
      if (l + 256u * j < wi.nint) v[j] = gload<NT, Ch>(gi + wi.a0 + 16u * (l + 256u * j));
    T e{};
    const bool edge = l < wi.head + wi.tail;
    const uint32_t eo = l < wi.head ? l * EB : wi.a1 + (l - wi.head) * EB;  // byte in the range
    if (edge) e = gload<NT, T>(gi + eo);
#pragma unroll
    for (uint32_t j = 0; j < (uint32_t)C; ++j)
      if (l + 256u * j < wi.nint) *(Ch*)(lds + win_pos<C>(m + wi.a0 + 16u * (l + 256u * j))) = v[j];
    if (edge) *(T*)(lds + win_pos<C>(m + eo)) = e;
    __syncthreads();
    // image -> planar ranges: chunk l of each channel, gathered at a stride of C
#pragma unroll
    for (uint32_t c = 0; c < (uint32_t)C; ++c) {
      char* gp = dst + (size_t)(c * t.plane + p0 + bd) * EB;
      const WinSplit<EB> wp(gp, np * EB);
      if (l < wp.nint) {
        const uint32_t x = m + ((wp.head + V * l) * C + c) * EB;  // image byte of its first element
        Ch o;
#pragma unroll
        for (uint32_t k = 0; k < V; ++k) o.e[k] = *(const T*)(lds + win_pos<C>(x + k * C * EB));
        gstore<NT, Ch>(gp + wp.a0 + 16u * l, o);
        count_store(t.wcnt, t.dst, gp + wp.a0 + 16u * l, 16);
      }
      if (l < wp.head + wp.tail) {
        const uint32_t px = l < wp.head ? l : wp.head + V * wp.nint + (l - wp.head);
        gstore<NT, T>(gp + (size_t)px * EB, *(const T*)(lds + win_pos<C>(m + (px * C + c) * EB)));
        count_store(t.wcnt, t.dst, gp + (size_t)px * EB, EB);
      }
    }
  } else {
    // planar ranges -> image: chunk l of each channel scattered at a stride of C
    Ch v[C];
    T e[C];
#pragma unroll
    for (uint32_t c = 0; c < (uint32_t)C; ++c) {
      const char* gp = src + (size_t)(c * t.plane + p0 + bs) * EB;
      const WinSplit<EB> wp(gp, np * EB);
      if (l < wp.nint) v[c] = gload<NT, Ch>(gp + wp.a0 + 16u * l);
      if (l < wp.head + wp.tail) {
        const uint32_t px = l < wp.head ? l : wp.head + V * wp.nint + (l - wp.head);
        e[c] = gload<NT, T>(gp + (size_t)px * EB);
      }
    }
#pragma unroll
    for (uint32_t c = 0; c < (uint32_t)C; ++c) {
      const char* gp = src + (size_t)(c * t.plane + p0 + bs) * EB;
      const WinSplit<EB> wp(gp, np * EB);
      if (l < wp.nint) {
        const uint32_t x = m + ((wp.head + V * l) * C + c) * EB;
#pragma unroll
        for (uint32_t k = 0; k < V; ++k) *(T*)(lds + win_pos<C>(x + k * C * EB)) = v[c].e[k];
      }
      if (l < wp.head + wp.tail) {
        const uint32_t px = l < wp.head ? l : wp.head + V * wp.nint + (l - wp.head);
        *(T*)(lds + win_pos<C>(m + (px * C + c) * EB)) = e[c];
      }
    }
    __syncthreads();
    // image -> interleaved range
#pragma unroll
    for (uint32_t j = 0; j < (uint32_t)C; ++j) {
      const uint32_t q = l + 256u * j;
      if (q < wi.nint) {
        gstore<NT, Ch>((char*)gi + wi.a0 + 16u * q, *(const Ch*)(lds + win_pos<C>(m + wi.a0 + 16u * q)));
        count_store(t.wcnt, t.dst, gi + wi.a0 + 16u * q, 16);
      }
    }
    if (l < wi.head + wi.tail) {
      const uint32_t eo = l < wi.head ? l * EB : wi.a1 + (l - wi.head) * EB;
      gstore<NT, T>((char*)gi + eo, *(const T*)(lds + win_pos<C>(m + eo)));
      count_store(t.wcnt, t.dst, gi + eo, EB);
    }
  }
}

// ------------------------------------------------------------------ staged footprint gather

struct StagedArgs {
  const void* src;
  void* dst;
  int32_t inner;                       // inner modes (compact in dst, in dst order)
  uint32_t in_ext[kMaxKernelModes];
  FD in_fd[kMaxKernelModes];
  uint32_t in_ss[kMaxKernelModes];
  uint32_t T;                          // tiles along the tile mode
  uint32_t Ts, Td;                     // tile strides (elements)
  uint32_t Fc;                         // 16-byte chunks of one tile's source footprint
  FD fd_Fc;
  uint32_t K;                          // tiles per workgroup
  uint32_t cpt;                        // 16-byte dst chunks per tile (power of two <= 256)
  uint32_t cpt_shift;                  // log2(cpt)
  uint32_t cps_shift;                  // log2 of the chunks per 32-lane slice of the gather
  uint32_t tgroups;
  FD fd_tg;
  BatchArg batch;
  SwzArg swd;
  WriteCount wcnt;
};

// Padded or gathered tiles ([CuTe algebra page, section 2.2]: composing a padded
// layout skips the pad).  A workgroup stages the whole 16-byte-aligned source
// footprint of K tiles in LDS with 16-byte loads (pad words included: DRAM
// fetches them with their lines anyway), then each lane builds 16-byte dst chunks
// by gathering elements from LDS and stores them contiguously.  L lanes per
// workgroup (64, 128 or 256).
template <int EB, bool NT, bool DL, int L = 256>
__global__ void __launch_bounds__(L) k_staged(StagedArgs t) {
  static_assert(L == 64 || L == 128 || L == 256, "64, 128 or 256 lanes");
  using T = typename Raw<EB>::T;
  constexpr int V = 16 / EB;
  using C = Chunk<T, V>;
  extern __shared__ uint4 lds[];
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;

  uint32_t blk = blockIdx.x;
  uint32_t r1 = fdiv(blk, t.fd_tg);
  uint32_t tg = blk - r1 * t.tgroups;
  uint32_t bs, bd;
  batch_offsets(t.batch, r1, &bs, &bd);
  const uint32_t t0 = tg * t.K;

  // Four independent 16-byte loads per lane per round, all issued before any LDS
  // write, so each lane keeps four loads in flight (a load-then-store loop body
  // would wait for every load before issuing the next).
  const uint32_t nload = t.K * t.Fc;
  auto chunk_ok = [&](uint32_t idx, size_t* byte) {
    if (idx >= nload) return false;
    const uint32_t kk = fdiv(idx, t.fd_Fc);
    const uint32_t tile = t0 + kk;
    *byte = (size_t)(tile * t.Ts + bs) * EB + (size_t)(idx - kk * t.Fc) * 16;
    return tile < t.T;
  };
  if constexpr (DL) {
    // Direct loads: chunk idx goes to lds[idx]; the 64 lanes of a wave take 64
    // consecutive chunks, so the wave's LDS base is the chunk of its lane 0.  No
    // registers hold the data, so every load of the footprint is issued at once.
    const uint32_t lane = threadIdx.x & 63u;
    for (uint32_t idx = threadIdx.x; idx < nload + lane; idx += L) {
      const uint32_t base = __builtin_amdgcn_readfirstlane(idx - lane);
      size_t b = 0;
      if (chunk_ok(idx, &b)) load_to_lds16<NT>(src + b, lds + base);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS writes have landed
  } else {
    for (uint32_t i0 = threadIdx.x; i0 < nload; i0 += 4 * L) {
      size_t b0 = 0, b1 = 0, b2 = 0, b3 = 0;
      const bool k0 = chunk_ok(i0, &b0), k1 = chunk_ok(i0 + L, &b1), k2 = chunk_ok(i0 + 2 * L, &b2),
                 k3 = chunk_ok(i0 + 3 * L, &b3);
      uint4 v0, v1, v2, v3;
      if (k0) v0 = gload<NT, uint4>(src + b0);
      if (k1) v1 = gload<NT, uint4>(src + b1);
      if (k2) v2 = gload<NT, uint4>(src + b2);
      if (k3) v3 = gload<NT, uint4>(src + b3);
      if (k0) lds[i0] = v0;
      if (k1) lds[i0 + L] = v1;
      if (k2) lds[i0 + 2 * L] = v2;
      if (k3) lds[i0 + 3 * L] = v3;
    }
  }
  __syncthreads();

  // Gather grouping: the 32-lane slice q = idx / 32 covers 32 / cps tiles x cps
  // chunks of each (tile (q / slices) * (32 / cps) + l / cps, chunk (q % slices) * cps
  // + l % cps, l = idx % 32, slices = cpt / cps); the planner picks cps from the LDS
  // bank model.  slices divides L / 32, so this lane's chunk position is the same
  // in every round of L jobs.
  const uint32_t slice_shift = t.cpt_shift - t.cps_shift, g_shift = 5u - t.cps_shift;
  const uint32_t c = (((threadIdx.x >> 5) & ((1u << slice_shift) - 1u)) << t.cps_shift) +
                     (threadIdx.x & ((1u << t.cps_shift) - 1u));
  uint32_t g[V];
#pragma unroll
  for (int x = 0; x < V; ++x) {
    uint32_t e = c * V + x, off = 0;
    for (int k = 0; k < t.inner; ++k) {
      uint32_t q = (k == t.inner - 1) ? 0u : fdiv(e, t.in_fd[k]);
      off += (e - q * t.in_ext[k]) * t.in_ss[k];
      e = q;
    }
    g[x] = off;
  }
  const T* ldsT = (const T*)lds;
  const uint32_t nstore = t.K * t.cpt;
  for (uint32_t idx = threadIdx.x; idx < nstore; idx += L) {
    const uint32_t kk = (((idx >> 5) >> slice_shift) << g_shift) + ((idx & 31u) >> t.cps_shift);
    uint32_t tile = t0 + kk;
    if (tile >= t.T) continue;
    C o;
    const uint32_t base = kk * t.Fc * V;  // tile's first element in LDS
#pragma unroll
    for (int x = 0; x < V; ++x) o.e[x] = ldsT[base + g[x]];
    uint32_t dof = swz32(tile * t.Td + bd + c * V, t.swd);
    gstore<NT, C>(dst + (size_t)dof * EB, o);
    count_store(t.wcnt, t.dst, dst + (size_t)dof * EB, sizeof(C));
  }
}

// ------------------------------------------------------------------ batched small matrices

struct BatchedArgs {
  const void* src;
  void* dst;
  uint32_t P, Q;        // 16-byte chunks along a and V-row blocks along b: A = V * P, B = V * Q
  uint32_t cpm;         // 16-byte chunks of one matrix (P * Q * V)
  FD fd_cpm;
  uint32_t pq;          // V x V blocks of one matrix (P * Q)
  FD fd_pq;
  uint32_t inner;       // the faster block index's extent: P (order 0, a-blocks fastest) or Q
  FD fd_inner;
  uint32_t order;
  uint32_t mpw;         // whole matrices per wavefront (mpw * cpm <= 512)
  uint32_t nblk;        // blocks per wavefront (mpw * pq)
  uint32_t count;       // matrices
  uint32_t sw[6];       // LDS slot of chunk c: c ^ (((c >> sw[0]) & sw[1]) << sw[2])
                        //                        ^ (((c >> sw[3]) & sw[4]) << sw[5])
  BatchArg batch;       // the matrix index over the other modes (element strides)
  WriteCount wcnt;
};

// Batched small matrices ([CuTe algebra page, section 4.1]: a blocked product of one
// small transpose over the batch modes).  Each matrix is compact on both sides: A
// elements along a (source-contiguous) by B along b (destination-contiguous), rows of
// A adjacent in the source and rows of B adjacent in the destination, A and B
// multiples of V = 16 / EB.  A wavefront owns mpw whole matrices (up to 8 KiB) in an
// LDS region of its own:
//  1. direct global -> LDS loads, lane l of load k taking region slot 64k + l, which
//     holds source chunk c = swz(slot) (the swizzle is an involution that permutes
//     chunks inside aligned groups of 16, so each load instruction still reads 1 KiB
//     of whole lines);
//  2. each lane reads the V source rows of its V x V blocks (16-byte LDS reads) and
//     transposes them in registers;
//  3. it writes the V destination rows of each block back into the region, at the
//     slots of their destination chunk indices;
//  4. lane l of store k takes slot 64k + l, i.e. destination chunk swz(slot), and
//     stores it: 1 KiB of whole lines per store instruction.
// The planner picks the swizzle and the block order that its gfx950 bank model
// finds cheapest for steps 2 and 3.  A workgroup is one wavefront (1-3 % faster than
// four independent ones sharing barriers, over 2^27 elements of 2-, 4- and 8-byte
// matrices from 8 x 8 to 64 x 64), with 8 KiB of LDS.
template <int EB, bool NT>
__global__ void __launch_bounds__(64) k_batched(BatchedArgs t) {
  constexpr int V = 16 / EB;
  constexpr int BPL = 8 / V;  // blocks per lane: 512 chunks of V-chunk blocks over 64 lanes
  static_assert(V >= 2 && V <= 8, "2-, 4- and 8-byte elements");
  __shared__ U4 reg[512];
  const char* __restrict__ src = (const char*)t.src;
  char* __restrict__ dst = (char*)t.dst;
  const int lane = threadIdx.x;
  const uint32_t m0 = blockIdx.x * t.mpw;
  const uint32_t nch = t.mpw * t.cpm;
  auto swz = [&](uint32_t c) {
    return c ^ (((c >> t.sw[0]) & t.sw[1]) << t.sw[2]) ^ (((c >> t.sw[3]) & t.sw[4]) << t.sw[5]);
  };
  // matrix of region chunk c, and c's element offset inside its matrix
  auto locate = [&](uint32_t c, uint32_t* m, uint32_t* off) {
    const uint32_t mi = fdiv(c, t.fd_cpm);
    *m = m0 + mi;
    *off = (c - mi * t.cpm) * V;
    return c < nch && *m < t.count;
  };

  // 1. loads
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t slot = 64u * k + lane;
    uint32_t m, off;
    if (!locate(swz(slot), &m, &off)) continue;
    uint32_t bs, bd;
    batch_offsets(t.batch, m, &bs, &bd);
    load_to_lds16<NT>(src + (size_t)(bs + off) * EB, reg + 64 * k);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 2. the blocks' source rows, transposed in registers
  U4 in[BPL][V], out[BPL][V];
  uint32_t mi_[BPL], ba_[BPL], bb_[BPL];
#pragma unroll
  for (int r = 0; r < BPL; ++r) {
    const uint32_t u = 64u * r + lane;
    const uint32_t mi = fdiv(u, t.fd_pq), rest = u - mi * t.pq;
    const uint32_t hi = fdiv(rest, t.fd_inner), lo = rest - hi * t.inner;
    mi_[r] = mi;
    ba_[r] = t.order ? hi : lo;
    bb_[r] = t.order ? lo : hi;
    if (u < t.nblk) {
#pragma unroll
      for (int j = 0; j < V; ++j) in[r][j] = reg[swz(mi * t.cpm + (V * bb_[r] + j) * t.P + ba_[r])];
      transpose_rows16<EB>(in[r], out[r]);
    }
  }
  __syncthreads();
  // 3. destination rows back into the region
#pragma unroll
  for (int r = 0; r < BPL; ++r) {
    if (64u * r + lane < t.nblk) {
#pragma unroll
      for (int i = 0; i < V; ++i) reg[swz(mi_[r] * t.cpm + (V * ba_[r] + i) * t.Q + bb_[r])] = out[r][i];
    }
  }
  __syncthreads();

  // 4. stores
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t slot = 64u * k + lane;
    uint32_t m, off;
    if (!locate(swz(slot), &m, &off)) continue;
    uint32_t bs, bd;
    batch_offsets(t.batch, m, &bs, &bd);
    char* p = dst + (size_t)(bd + off) * EB;
    gstore<NT, U4>(p, reg[slot]);
    count_store(t.wcnt, t.dst, p, 16);
  }
}

// ------------------------------------------------------------------ launch helpers

static int check_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_hip_error(hipGetErrorString(e));
    return LR_ERR_HIP;
  }
  return LR_OK;
}

static unsigned grid_cap(int64_t g) {
  if (g < 1) g = 1;
  return (unsigned)(g > 0x7FFFFFFF ? 0x7FFFFFFF : g);
}

static void fill_side(SideArg* s, const lr_layout* L, bool wide) {
  std::memset(s, 0, sizeof(*s));
  s->nleaves = L->nleaves;
  for (int i = 0; i < L->nleaves; ++i) {
    s->ext64[i] = L->shape[i];
    s->stride64[i] = L->stride[i];
    if (!wide) {
      s->ext[i] = (uint32_t)L->shape[i];
      s->fd[i] = fd_of(L->shape[i]);
      s->stride[i] = (uint32_t)L->stride[i];
    }
  }
  Swz z{L->swz_b, L->swz_m, L->swz_s};
  s->sw = swz_arg(z);
  s->mask64 = L->swz_b > 0 ? (((uint64_t(1) << L->swz_b) - 1) << L->swz_m) : 0;
}

static void fill_batch(BatchArg* b, const Plan& p, int skip0, int skip1, int skip2 = -1) {
  std::memset(b, 0, sizeof(*b));
  for (int k = 0; k < p.rank; ++k) {
    if (k == skip0 || k == skip1 || k == skip2) continue;
    int r = b->rank++;
    b->ext[r] = (uint32_t)p.m[k].ext;
    b->fd[r] = fd_of(p.m[k].ext);
    b->ss[r] = (uint32_t)p.m[k].ss;
    b->sd[r] = (uint32_t)p.m[k].sd;
  }
}

// The staged gather in 64-, 128- or 256-lane workgroups.
template <int EB, bool NT, bool DL>
static void launch_staged_l(const StagedArgs& a, int lanes, unsigned grid, size_t shm, hipStream_t st) {
  if (lanes == 64)
    hipLaunchKernelGGL((k_staged<EB, NT, DL, 64>), dim3(grid), dim3(64), shm, st, a);
  else if (lanes == 128)
    hipLaunchKernelGGL((k_staged<EB, NT, DL, 128>), dim3(grid), dim3(128), shm, st, a);
  else
    hipLaunchKernelGGL((k_staged<EB, NT, DL, 256>), dim3(grid), dim3(256), shm, st, a);
}

template <int EB>
static void launch_batched_eb(const BatchedArgs& a, bool nt, unsigned grid, hipStream_t st) {
  if (nt)
    hipLaunchKernelGGL((k_batched<EB, true>), dim3(grid), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((k_batched<EB, false>), dim3(grid), dim3(64), 0, st, a);
}

static bool launch_batched(const BatchedArgs& a, int eb, bool nt, unsigned grid, hipStream_t st) {
  switch (eb) {
    case 2: launch_batched_eb<2>(a, nt, grid, st); return true;
    case 4: launch_batched_eb<4>(a, nt, grid, st); return true;
    case 8: launch_batched_eb<8>(a, nt, grid, st); return true;
    default: return false;
  }
}

// One kernel per atom size K = KK..32 chunks, with 64, 128 or 256 lanes.
template <int KK, bool LNT, bool SNT>
static bool launch_atoms_nt(const AtomArgs& a, int K, int lanes, unsigned grid, hipStream_t st) {
  if constexpr (KK > 32) {
    return false;
  } else {
    if (K == KK) {
      if (lanes == 64)
        hipLaunchKernelGGL((k_atoms<KK, LNT, SNT, 64>), dim3(grid), dim3(64), 0, st, a);
      else if (lanes == 128)
        hipLaunchKernelGGL((k_atoms<KK, LNT, SNT, 128>), dim3(grid), dim3(128), 0, st, a);
      else
        hipLaunchKernelGGL((k_atoms<KK, LNT, SNT>), dim3(grid), dim3(256), 0, st, a);
      return true;
    }
    return launch_atoms_nt<KK + 1, LNT, SNT>(a, K, lanes, grid, st);
  }
}

// Tiles of atoms (vector order 3), from the vector path's arguments in 16-byte units:
// mode 0 is the atom, p.a and p.b the modes that continue it in the source and in
// the destination.
static bool launch_atoms(const Plan& p, const GenericArgs& g, unsigned grid, hipStream_t st) {
  AtomArgs a;
  std::memset(&a, 0, sizeof(a));
  a.src = g.src;
  a.dst = g.dst;
  a.wcnt = g.wcnt;
  const int K = (int)g.m[0].ext;
  const int64_t T = atom_tile(K);
  a.ext_a = g.m[p.a].ext;
  a.ext_b = g.m[p.b].ext;
  a.ss_b = g.m[p.b].ss;
  a.sd_a = g.m[p.a].sd;
  a.tiles_a = (uint32_t)((a.ext_a + T - 1) / T);
  a.tiles_b = (uint32_t)((a.ext_b + T - 1) / T);
  a.fd_ta = fd_of(a.tiles_a);
  a.fd_tb = fd_of(a.tiles_b);
  for (int k = 1; k < p.rank; ++k) {
    if (k == p.a || k == p.b) continue;
    const int r = a.batch.rank++;
    a.batch.ext[r] = g.m[k].ext;
    a.batch.fd[r] = g.m[k].fd;
    a.batch.ss[r] = g.m[k].ss;
    a.batch.sd[r] = g.m[k].sd;
  }
  a.sws = g.sws;
  a.swd = g.swd;
  a.bufst = g.bufst;
  if (p.nt_ld && p.nt) return launch_atoms_nt<2, true, true>(a, K, p.block, grid, st);
  if (p.nt_ld) return launch_atoms_nt<2, true, false>(a, K, p.block, grid, st);
  if (p.nt) return launch_atoms_nt<2, false, true>(a, K, p.block, grid, st);
  return launch_atoms_nt<2, false, false>(a, K, p.block, grid, st);
}

template <int UB, bool LNT, bool SNT>
static void launch_generic_nt(const GenericArgs& a, bool wide, int unroll, int lanes, unsigned grid,
                              hipStream_t st) {
  if (wide)
    hipLaunchKernelGGL((k_generic<UB, true, 4, LNT, SNT>), dim3(grid), dim3(256), 0, st, a);
  else if (unroll == 1 && lanes == 64)
    hipLaunchKernelGGL((k_generic<UB, false, 1, LNT, SNT, 64>), dim3(grid), dim3(64), 0, st, a);
  else if (unroll == 1 && lanes == 128)
    hipLaunchKernelGGL((k_generic<UB, false, 1, LNT, SNT, 128>), dim3(grid), dim3(128), 0, st, a);
  else if (unroll == 1)
    hipLaunchKernelGGL((k_generic<UB, false, 1, LNT, SNT>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_generic<UB, false, 4, LNT, SNT>), dim3(grid), dim3(256), 0, st, a);
}

template <int UB>
static void launch_generic(const GenericArgs& a, bool wide, int unroll, int lanes, bool nt_ld, bool nt_st,
                           unsigned grid, hipStream_t st) {
  if (nt_ld && nt_st)
    launch_generic_nt<UB, true, true>(a, wide, unroll, lanes, grid, st);
  else if (nt_ld)
    launch_generic_nt<UB, true, false>(a, wide, unroll, lanes, grid, st);
  else if (nt_st)
    launch_generic_nt<UB, false, true>(a, wide, unroll, lanes, grid, st);
  else
    launch_generic_nt<UB, false, false>(a, wide, unroll, lanes, grid, st);
}

template <int EB>
static void launch_dual(const DualArgs& a, bool wide, unsigned grid, hipStream_t st) {
  if (wide)
    hipLaunchKernelGGL((k_dual<EB, true>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_dual<EB, false>), dim3(grid), dim3(256), 0, st, a);
}

template <int EB, int V, int TA, int TB, bool NT, int R = 1>
static void launch_transpose_shape(const TransposeArgs& a, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((k_transpose<EB, V, true, TA, TB, NT, R>), dim3(grid), dim3(TA * TB / R), 0, st, a);
}

// The direct-load kernels: pipelined (a.pipe) or one tile per workgroup.
template <int EB, int V, bool NT, bool TR>
static bool launch_dl(const TransposeArgs& a, int shape, unsigned grid, hipStream_t st) {
  if (a.pipe) {
    switch (shape) {
      case 0:
        if constexpr (pipe_fits(0, V)) {
          hipLaunchKernelGGL((k_transpose_pipe<EB, V, 16, 16, NT, TR>), dim3(grid), dim3(256), 0, st, a);
          return true;
        }
        return false;
      case 1:
        if constexpr (pipe_fits(1, V)) {
          hipLaunchKernelGGL((k_transpose_pipe<EB, V, 32, 16, NT, TR>), dim3(grid), dim3(512), 0, st, a);
          return true;
        }
        return false;
      case 2:
        if constexpr (pipe_fits(2, V)) {
          hipLaunchKernelGGL((k_transpose_pipe<EB, V, 16, 32, NT, TR>), dim3(grid), dim3(512), 0, st, a);
          return true;
        }
        return false;
      default: return false;
    }
  }
  switch (shape) {
    case 0: hipLaunchKernelGGL((k_transpose_dl<EB, V, 16, 16, NT, TR>), dim3(grid), dim3(256), 0, st, a); return true;
    case 1: hipLaunchKernelGGL((k_transpose_dl<EB, V, 32, 16, NT, TR>), dim3(grid), dim3(512), 0, st, a); return true;
    case 2: hipLaunchKernelGGL((k_transpose_dl<EB, V, 16, 32, NT, TR>), dim3(grid), dim3(512), 0, st, a); return true;
    case 3:
      if constexpr (shape_fits(3, V)) {
        hipLaunchKernelGGL((k_transpose_dl<EB, V, 32, 32, NT, TR>), dim3(grid), dim3(1024), 0, st, a);
        return true;
      }
      return false;
    default: return false;
  }
}

// dl: 0 through registers, 1 direct loads, 2 direct loads read back with the gfx950
// transpose reads, 3 through registers with two blocks per lane
template <int EB, int V, bool NT>
static bool launch_transpose_v(const TransposeArgs& a, bool lds, int shape, int dl, unsigned grid,
                               hipStream_t st) {
  if constexpr (V * EB == 16 || (EB == 1 && V == 8)) {
    if (dl == 3) {
      if (!lds) return false;
#define LR_TSHAPE2_CASE(S)                                                               \
  case S:                                                                                \
    if constexpr (shape_fits(S, V) && kTileTB[S] % 2 == 0 && kTileTA[S] * kTileTB[S] >= 128) { \
      launch_transpose_shape<EB, V, kTileTA[S], kTileTB[S], NT, 2>(a, grid, st);         \
      return true;                                                                       \
    }                                                                                    \
    return false;
      switch (shape) {
        case 0: launch_transpose_shape<EB, V, 16, 16, NT, 2>(a, grid, st); return true;
        LR_TSHAPE2_CASE(1)
        LR_TSHAPE2_CASE(2)
        LR_TSHAPE2_CASE(3)
        LR_TSHAPE2_CASE(4)
        LR_TSHAPE2_CASE(5)
        LR_TSHAPE2_CASE(6)
        LR_TSHAPE2_CASE(7)
        LR_TSHAPE2_CASE(8)
        default: return false;
      }
#undef LR_TSHAPE2_CASE
    }
  } else {
    if (dl == 3) return false;
  }
  if constexpr (V * EB == 16) {
    if (dl == 2 && lds) {
      if constexpr (EB <= 2) return launch_dl<EB, V, NT, true>(a, shape, grid, st);
      return false;
    }
    if (dl == 1 && lds) return launch_dl<EB, V, NT, false>(a, shape, grid, st);
  }
  if (!lds) {
    if (shape != 0) return false;
    hipLaunchKernelGGL((k_transpose<EB, V, false, 16, 16, NT>), dim3(grid), dim3(256), 0, st, a);
    return true;
  }
  if constexpr (V * EB == 16 || (EB == 1 && V == 8)) {  // other shapes: 16-byte chunks (8-byte for 1-byte elements), tiles that fit LDS
#define LR_TSHAPE_CASE(S)                                                                \
  case S:                                                                                \
    if constexpr (shape_fits(S, V)) {                                                    \
      launch_transpose_shape<EB, V, kTileTA[S], kTileTB[S], NT>(a, grid, st);            \
      return true;                                                                       \
    }                                                                                    \
    break;
    switch (shape) {
      LR_TSHAPE_CASE(1)
      LR_TSHAPE_CASE(2)
      LR_TSHAPE_CASE(3)
      LR_TSHAPE_CASE(4)
      LR_TSHAPE_CASE(5)
      LR_TSHAPE_CASE(6)
      LR_TSHAPE_CASE(7)
      LR_TSHAPE_CASE(8)
      default: break;
    }
#undef LR_TSHAPE_CASE
  }
  if (shape != 0) return false;
  launch_transpose_shape<EB, V, 16, 16, NT>(a, grid, st);
  return true;
}

template <int EB, bool NT>
static bool launch_tel(const TransposeArgs& a, bool win, unsigned grid, hipStream_t st) {
  if (win) {
    hipLaunchKernelGGL((k_transpose_win<EB, NT>), dim3(grid), dim3(512), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_transpose_el<EB, NT>), dim3(grid), dim3(512), 0, st, a);
  }
  return true;
}

template <int EB, bool NT>
static bool launch_transpose_nt(const TransposeArgs& a, int v, bool lds, int shape, int dl, unsigned grid,
                                hipStream_t st) {
  switch (v) {
    case 1: return launch_transpose_v<EB, 1, NT>(a, lds, shape, dl, grid, st);
    case 2: if constexpr (EB <= 8) return launch_transpose_v<EB, 2, NT>(a, lds, shape, dl, grid, st); break;
    case 4: if constexpr (EB <= 4) return launch_transpose_v<EB, 4, NT>(a, lds, shape, dl, grid, st); break;
    case 8: if constexpr (EB <= 2) return launch_transpose_v<EB, 8, NT>(a, lds, shape, dl, grid, st); break;
    case 16: if constexpr (EB == 1) return launch_transpose_v<EB, 16, NT>(a, lds, shape, dl, grid, st); break;
  }
  return false;
}

template <int EB>
static bool launch_transpose(const TransposeArgs& a, int v, bool lds, int shape, bool nt, int dl, unsigned grid,
                             hipStream_t st) {
  return nt ? launch_transpose_nt<EB, true>(a, v, lds, shape, dl, grid, st)
            : launch_transpose_nt<EB, false>(a, v, lds, shape, dl, grid, st);
}

template <int EB, bool NARROW, bool NT, int L>
static bool launch_interleave_l(const InterleaveArgs& a, int nb, unsigned grid, hipStream_t st) {
  switch (nb) {
    case 2: if constexpr (EB <= 8) { hipLaunchKernelGGL((k_interleave<EB, 2, NARROW, NT, L>), dim3(grid), dim3(L), 0, st, a); return true; } break;
    case 4: if constexpr (EB <= 4) { hipLaunchKernelGGL((k_interleave<EB, 4, NARROW, NT, L>), dim3(grid), dim3(L), 0, st, a); return true; } break;
    case 8: if constexpr (EB <= 2) { hipLaunchKernelGGL((k_interleave<EB, 8, NARROW, NT, L>), dim3(grid), dim3(L), 0, st, a); return true; } break;
    case 16: if constexpr (EB == 1) { hipLaunchKernelGGL((k_interleave<EB, 16, NARROW, NT, L>), dim3(grid), dim3(L), 0, st, a); return true; } break;
  }
  return false;
}

// lanes: workgroup lanes of the narrow form (64, 128 or 256; the wide form takes 256)
template <int EB, bool NARROW, bool NT>
static bool launch_interleave_n(const InterleaveArgs& a, int nb, int lanes, unsigned grid, hipStream_t st) {
  if constexpr (NARROW) {
    if (lanes == 64) return launch_interleave_l<EB, true, NT, 64>(a, nb, grid, st);
    if (lanes == 128) return launch_interleave_l<EB, true, NT, 128>(a, nb, grid, st);
  }
  if (lanes != 256) return false;
  return launch_interleave_l<EB, NARROW, NT, 256>(a, nb, grid, st);
}

template <int EB, int CC, bool INTERLEAVE, bool NT>
static bool launch_chan_one(const ChanArgs& a, bool elem, int lanes, unsigned grid, hipStream_t st) {
  if constexpr (chan_supported(EB, CC)) {
    if (elem)
      hipLaunchKernelGGL((k_chan_win<EB, CC, INTERLEAVE, NT>), dim3(grid), dim3(256), 0, st, a);
    else if (lanes == 64)
      hipLaunchKernelGGL((k_chan<EB, CC, INTERLEAVE, NT, 64>), dim3(grid), dim3(64), 0, st, a);
    else if (lanes == 128)
      hipLaunchKernelGGL((k_chan<EB, CC, INTERLEAVE, NT, 128>), dim3(grid), dim3(128), 0, st, a);
    else
      hipLaunchKernelGGL((k_chan<EB, CC, INTERLEAVE, NT>), dim3(grid), dim3(256), 0, st, a);
    return true;
  }
  return false;
}

template <int EB, bool INTERLEAVE, bool NT>
static bool launch_chan_c(const ChanArgs& a, int c, bool elem, int lanes, unsigned grid, hipStream_t st) {
  switch (c) {
    case 2: return launch_chan_one<EB, 2, INTERLEAVE, NT>(a, elem, lanes, grid, st);
    case 3: return launch_chan_one<EB, 3, INTERLEAVE, NT>(a, elem, lanes, grid, st);
    case 4: return launch_chan_one<EB, 4, INTERLEAVE, NT>(a, elem, lanes, grid, st);
    case 5: return launch_chan_one<EB, 5, INTERLEAVE, NT>(a, elem, lanes, grid, st);
    case 6: return launch_chan_one<EB, 6, INTERLEAVE, NT>(a, elem, lanes, grid, st);
    case 7: return launch_chan_one<EB, 7, INTERLEAVE, NT>(a, elem, lanes, grid, st);
    case 8: return launch_chan_one<EB, 8, INTERLEAVE, NT>(a, elem, lanes, grid, st);
    default: return false;
  }
}

template <int EB>
static bool launch_chan(const ChanArgs& a, int c, bool interleave, bool elem, bool nt, int lanes, unsigned grid,
                        hipStream_t st) {
  if (interleave)
    return nt ? launch_chan_c<EB, true, true>(a, c, elem, lanes, grid, st)
              : launch_chan_c<EB, true, false>(a, c, elem, lanes, grid, st);
  return nt ? launch_chan_c<EB, false, true>(a, c, elem, lanes, grid, st)
            : launch_chan_c<EB, false, false>(a, c, elem, lanes, grid, st);
}

template <int EB>
static bool launch_interleave(const InterleaveArgs& a, int nb, bool narrow, bool nt, int lanes, unsigned grid,
                              hipStream_t st) {
  if (nt)
    return narrow ? launch_interleave_n<EB, true, true>(a, nb, lanes, grid, st)
                  : launch_interleave_n<EB, false, true>(a, nb, lanes, grid, st);
  return narrow ? launch_interleave_n<EB, true, false>(a, nb, lanes, grid, st)
                : launch_interleave_n<EB, false, false>(a, nb, lanes, grid, st);
}

#define LR_DISPATCH_EB(eb, CALL)          \
  switch (eb) {                            \
    case 1: { constexpr int EBV = 1; CALL; } break;   \
    case 2: { constexpr int EBV = 2; CALL; } break;   \
    case 4: { constexpr int EBV = 4; CALL; } break;   \
    case 8: { constexpr int EBV = 8; CALL; } break;   \
    case 16: { constexpr int EBV = 16; CALL; } break; \
    default: return LR_ERR_ELEM_BYTES;     \
  }

static size_t ptr_align(const void* p) {
  uintptr_t a = (uintptr_t)p;
  if (a == 0) return 16;
  size_t al = (size_t)(a & (~a + 1));
  return al > 16 ? 16 : al;
}

static int run_copy(const void* src, const lr_layout* Ls, void* dst, const lr_layout* Ld, const Plan& p,
                    hipStream_t st, WriteCount wc) {
  const unsigned grid = grid_cap(p.grid);
  switch (p.path) {
    case LR_PATH_GENERIC:
    case LR_PATH_VECTOR: {
      GenericArgs a;
      std::memset(&a, 0, sizeof(a));
      a.wcnt = wc;
      a.src = src;
      a.dst = dst;
      a.rank = p.rank;
      const int64_t v = p.v;
      for (int k = 0; k < p.rank; ++k) {
        // mode 0 is the common contiguous mode when v > 1: it is counted in units
        int64_t ext = (k == 0) ? p.m[0].ext / v : p.m[k].ext;
        int64_t ss = (k == 0 && v > 1) ? 1 : p.m[k].ss / v;
        int64_t sd = (k == 0 && v > 1) ? 1 : p.m[k].sd / v;
        a.w[k] = {ext, ss, sd};
        if (!p.wide) a.m[k] = {(uint32_t)ext, fd_of(ext), (uint32_t)ss, (uint32_t)sd};
      }
      const int sh = (v == 1) ? 0 : (v == 2 ? 1 : v == 4 ? 2 : v == 8 ? 3 : 4);
      Swz zs = p.sw_s, zd = p.sw_d;
      if (zs.b) zs.m -= sh;
      if (zd.b) zd.m -= sh;
      a.sws = swz_arg(zs);
      a.swd = swz_arg(zd);
      a.sws_mask64 = zs.b ? (((uint64_t(1) << zs.b) - 1) << zs.m) : 0;
      a.swd_mask64 = zd.b ? (((uint64_t(1) << zd.b) - 1) << zd.m) : 0;
      a.n_units = p.n_units;
      a.n_chunks = (p.n_units + p.block * p.unroll - 1) / (p.block * p.unroll);
      a.bufst = p.bufst ? 1u : 0u;
      const int ub = p.v * p.eb;
      if (p.vorder == 3) return launch_atoms(p, a, grid, st) ? check_launch() : LR_ERR_PATH;
      LR_DISPATCH_EB(ub, launch_generic<EBV>(a, p.wide, p.unroll, p.block, p.nt_ld, p.nt, grid, st));
      return check_launch();
    }
    case LR_PATH_DUAL:
    case LR_PATH_ALIAS: {
      DualArgs a;
      std::memset(&a, 0, sizeof(a));
      a.wcnt = wc;
      a.src = src;
      a.dst = dst;
      fill_side(&a.s, Ls, p.wide);
      fill_side(&a.d, Ld, p.wide);
      a.n = p.n;
      a.n_chunks = (p.n + 1023) / 1024;
      if (p.path == LR_PATH_ALIAS) {
        LR_DISPATCH_EB(p.eb, hipLaunchKernelGGL((k_alias<EBV>), dim3(grid), dim3(1024), 0, st, a));
      } else {
        LR_DISPATCH_EB(p.eb, launch_dual<EBV>(a, p.wide, grid, st));
      }
      return check_launch();
    }
    case LR_PATH_TRANSPOSE:
    case LR_PATH_TRANSPOSE_DIRECT: {
      TransposeArgs a;
      std::memset(&a, 0, sizeof(a));
      a.wcnt = wc;
      a.src = src;
      a.dst = dst;
      const int64_t ext_b = p.m[p.b].ext * (p.b2 >= 0 ? p.m[p.b2].ext : 1);
      a.ext_a = (uint32_t)p.m[p.a].ext;
      a.ext_b = (uint32_t)ext_b;
      a.ss_b = (uint32_t)p.m[p.b].ss;
      a.sd_a = (uint32_t)p.m[p.a].sd;
      if (p.b2 >= 0) {
        uint32_t sh = 0;
        while ((int64_t(1) << sh) < p.m[p.b].ext) ++sh;
        a.bmask = (1u << sh) - 1u;
        a.bshift = sh;
        a.ss_b2 = (uint32_t)p.m[p.b2].ss;
      } else {
        a.bmask = 0xFFFFFFFFu;
        a.bshift = 31;
        a.ss_b2 = 0;
      }
      a.tiles_a = (uint32_t)((p.m[p.a].ext + p.tile_a - 1) / p.tile_a);
      a.tiles_b = (uint32_t)((ext_b + p.tile_b - 1) / p.tile_b);
      a.fd_ta = fd_of(a.tiles_a);
      a.fd_tb = fd_of(a.tiles_b);
      fill_batch(&a.batch, p, p.a, p.b, p.b2);
      a.sws = swz_arg(p.sw_s);
      a.swd = swz_arg(p.sw_d);
      a.order = p.torder;
      a.nwg = (uint32_t)p.grid;
      a.bufst = p.bufst ? 1u : 0u;
      a.bufmask = p.sw_d.b ? ~((1u << (p.sw_d.m + p.sw_d.b)) - 1u) : ~0u;
      if (p.torder % 5 == 3) {
        a.gta = a.tiles_a / 4;
        a.gtb = a.tiles_b / 4;
        a.fd_gta = fd_of(a.gta);
        a.fd_gtb = fd_of(a.gtb);
      }
      a.pipe = (uint32_t)p.pipe;
      a.ntiles = (uint32_t)p.tiles_total;
      const bool lds = p.path == LR_PATH_TRANSPOSE;
      if (p.tel) {
        if (p.eb > 8) return LR_ERR_PATH;
        bool ok = false;
        switch (p.eb) {
          case 1: ok = p.nt ? launch_tel<1, true>(a, p.twin, grid, st) : launch_tel<1, false>(a, p.twin, grid, st); break;
          case 2: ok = p.nt ? launch_tel<2, true>(a, p.twin, grid, st) : launch_tel<2, false>(a, p.twin, grid, st); break;
          case 4: ok = p.nt ? launch_tel<4, true>(a, p.twin, grid, st) : launch_tel<4, false>(a, p.twin, grid, st); break;
          default: ok = p.nt ? launch_tel<8, true>(a, p.twin, grid, st) : launch_tel<8, false>(a, p.twin, grid, st); break;
        }
        if (!ok) return LR_ERR_PATH;
        return check_launch();
      }
      bool ok = false;
      const int dl = p.direct ? (p.tr ? 2 : 1) : (p.tblocks == 2 ? 3 : 0);
      LR_DISPATCH_EB(p.eb, ok = launch_transpose<EBV>(a, p.v, lds, p.tshape, p.nt, dl, grid, st));
      if (!ok) return LR_ERR_PATH;
      return check_launch();
    }
    case LR_PATH_DEINTERLEAVE:
    case LR_PATH_INTERLEAVE:
      if (p.path == LR_PATH_DEINTERLEAVE || p.inarrow >= 2) {
        // channel shuffle: the pixel mode is the one contiguous on the planar side
        const bool il = p.path == LR_PATH_INTERLEAVE;
        const int pm = il ? p.a : p.b, cm = il ? p.b : p.a;
        ChanArgs a;
        std::memset(&a, 0, sizeof(a));
        a.wcnt = wc;
        a.src = src;
        a.dst = dst;
        a.pixels = (uint32_t)p.m[pm].ext;
        a.plane = (uint32_t)(il ? p.m[cm].ss : p.m[cm].sd);
        a.tiles = (uint32_t)((p.m[pm].ext + p.tile_a - 1) / p.tile_a);
        a.fd_tiles = fd_of(a.tiles);
        fill_batch(&a.batch, p, p.a, p.b);
        a.bufst = p.bufst ? 1u : 0u;
        bool ok = false;
        // one element per lane unit (v == 1): the element-granular form
        LR_DISPATCH_EB(p.eb, ok = launch_chan<EBV>(a, (int)p.m[cm].ext, il, p.v == 1, p.nt, p.block, grid, st));
        if (!ok) return LR_ERR_PATH;
        return check_launch();
      }
      {
      InterleaveArgs a;
      std::memset(&a, 0, sizeof(a));
      a.wcnt = wc;
      a.src = src;
      a.dst = dst;
      a.ext_a = (uint32_t)p.m[p.a].ext;
      a.ss_b = (uint32_t)p.m[p.b].ss;
      a.tiles_a = (uint32_t)((p.m[p.a].ext + p.tile_a - 1) / p.tile_a);
      a.fd_ta = fd_of(a.tiles_a);
      fill_batch(&a.batch, p, p.a, p.b);
      a.sws = swz_arg(p.sw_s);
      a.swd = swz_arg(p.sw_d);
      a.bufst = p.bufst ? 1u : 0u;
      bool ok = false;
      LR_DISPATCH_EB(p.eb, ok = launch_interleave<EBV>(a, (int)p.tile_b, p.inarrow != 0, p.nt, p.block, grid, st));
      if (!ok) return LR_ERR_PATH;
      return check_launch();
    }
    case LR_PATH_BATCHED: {
      BatchedArgs a;
      std::memset(&a, 0, sizeof(a));
      a.wcnt = wc;
      a.src = src;
      a.dst = dst;
      const uint32_t V = (uint32_t)p.v;
      a.P = (uint32_t)(p.m[p.a].ext / V);
      a.Q = (uint32_t)(p.m[p.b].ext / V);
      a.cpm = a.P * a.Q * V;
      a.fd_cpm = fd_of(a.cpm);
      a.pq = a.P * a.Q;
      a.fd_pq = fd_of(a.pq);
      a.order = (uint32_t)p.bt_order;
      a.inner = a.order ? a.Q : a.P;
      a.fd_inner = fd_of(a.inner);
      a.mpw = (uint32_t)p.bt_mpw;
      a.nblk = a.mpw * a.pq;
      a.count = (uint32_t)p.bt_count;
      for (int i = 0; i < 6; ++i) a.sw[i] = (uint32_t)p.bt_sw[i];
      fill_batch(&a.batch, p, p.a, p.b);
      if (!launch_batched(a, p.eb, p.nt, grid, st)) return LR_ERR_PATH;
      return check_launch();
    }
    case LR_PATH_STAGED: {
      StagedArgs a;
      std::memset(&a, 0, sizeof(a));
      a.wcnt = wc;
      a.src = src;
      a.dst = dst;
      a.inner = p.staged_inner;
      for (int k = 0; k < p.staged_inner; ++k) {
        a.in_ext[k] = (uint32_t)p.m[k].ext;
        a.in_fd[k] = fd_of(p.m[k].ext);
        a.in_ss[k] = (uint32_t)p.m[k].ss;
      }
      const JMode& tm = p.m[p.staged_inner];
      a.T = (uint32_t)tm.ext;
      a.Ts = (uint32_t)tm.ss;
      a.Td = (uint32_t)tm.sd;
      a.Fc = (uint32_t)p.staged_Fc;
      a.fd_Fc = fd_of(p.staged_Fc);
      a.K = (uint32_t)p.staged_K;
      a.cpt = (uint32_t)p.staged_cpt;
      while ((1u << a.cpt_shift) < a.cpt) ++a.cpt_shift;
      while ((int64_t(1) << a.cps_shift) < p.staged_cps) ++a.cps_shift;
      a.tgroups = (uint32_t)((tm.ext + p.staged_K - 1) / p.staged_K);
      a.fd_tg = fd_of(a.tgroups);
      std::memset(&a.batch, 0, sizeof(a.batch));
      for (int k = p.staged_inner + 1; k < p.rank; ++k) {
        int r = a.batch.rank++;
        a.batch.ext[r] = (uint32_t)p.m[k].ext;
        a.batch.fd[r] = fd_of(p.m[k].ext);
        a.batch.ss[r] = (uint32_t)p.m[k].ss;
        a.batch.sd[r] = (uint32_t)p.m[k].sd;
      }
      a.swd = swz_arg(p.sw_d);
      const size_t shm = (size_t)p.staged_K * (size_t)p.staged_Fc * 16;
      if (p.direct) {
        if (p.nt) {
          LR_DISPATCH_EB(p.eb, (launch_staged_l<EBV, true, true>(a, (int)p.block, grid, shm, st)));
        } else {
          LR_DISPATCH_EB(p.eb, (launch_staged_l<EBV, false, true>(a, (int)p.block, grid, shm, st)));
        }
      } else if (p.nt) {
        LR_DISPATCH_EB(p.eb, (launch_staged_l<EBV, true, false>(a, (int)p.block, grid, shm, st)));
      } else {
        LR_DISPATCH_EB(p.eb, (launch_staged_l<EBV, false, false>(a, (int)p.block, grid, shm, st)));
      }
      return check_launch();
    }
  }
  return LR_ERR_PATH;
}

// LR_LOG=1 (read once): every lr_layout_copy prints its plan to stderr -- path,
// element and unit sizes, tiles, grid, policies and the joint modes -- the
// library's counterpart of printing a layout's thread-to-offset map
// ([ThreadMap page, section 5.3]).  It changes nothing else.
static bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("LR_LOG");
    return e && *e && std::strcmp(e, "0") != 0;
  }();
  return on;
}

static void log_plan(const Plan& p, int64_t blocks) {
  static const char* names[] = {"generic", "vector", "transpose", "interleave", "staged",
                                "dual", "alias", "transpose_direct", "deinterleave", "batched"};
  char modes[1024];
  int at = 0;
  for (int k = 0; k < p.rank && at < (int)sizeof(modes) - 64; ++k)
    at += std::snprintf(modes + at, sizeof(modes) - at, "%s(%lld:%lld:%lld)", k ? " " : "", (long long)p.m[k].ext,
                        (long long)p.m[k].ss, (long long)p.m[k].sd);
  if (at == 0) modes[0] = 0;
  std::fprintf(stderr,
               "lr plan: path=%s elem_bytes=%d vec=%d wide=%d a=%d b=%d b2=%d tile=%lldx%lld shape=%d order=%d "
               "block=%d grid=%lld blocks=%lld nt_load=%d nt_store=%d sc1=%d direct=%d elem_tiles=%d "
               "vorder=%d gather_chunks=%lld pipeline_tiles=%d transpose_reads=%d batched=%lld/%d/%d,%d,%d,%d,%d,%d "
               "joint=[%s]\n",
               p.path >= 0 && p.path <= 9 ? names[p.path] : "?", p.eb, p.v, p.wide ? 1 : 0, p.a, p.b, p.b2,
               (long long)p.tile_a, (long long)p.tile_b, p.tshape, (int)p.torder, p.block, (long long)p.grid,
               (long long)blocks, p.nt_ld ? 1 : 0, p.nt ? 1 : 0, (p.nt && p.bufst) ? 1 : 0, p.direct ? 1 : 0,
               p.tel ? 1 : 0, p.vorder, (long long)p.staged_cps, p.pipe, p.tr ? 1 : 0, (long long)p.bt_mpw,
               p.bt_order, p.bt_sw[0], p.bt_sw[1], p.bt_sw[2], p.bt_sw[3], p.bt_sw[4], p.bt_sw[5], modes);
}

static int fill_eval(EvalArgs* a, const lr_layout* L) {
  std::memset(a, 0, sizeof(*a));
  a->nleaves = L->nleaves;
  a->nmodes = L->nmodes;
  a->size = size_of(L);
  a->small = a->size < (int64_t(1) << 31);
  for (int i = 0; i < L->nleaves; ++i) {
    a->shape[i] = L->shape[i];
    a->stride[i] = L->stride[i];
    if (a->small) a->fd[i] = fd_of(L->shape[i]);
  }
  int lo = 0;
  for (int m = 0; m < L->nmodes; ++m) {
    a->mode_end[m] = L->mode_end[m];
    int64_t s = 1;
    for (int i = lo; i < L->mode_end[m]; ++i) s *= L->shape[i];
    a->mode_size[m] = s;
    lo = L->mode_end[m];
  }
  if (L->swz_b > 0) {
    a->swz_mask = ((uint64_t(1) << L->swz_b) - 1) << L->swz_m;
    a->swz_shift = (uint32_t)L->swz_s;
  }
  // the highest offset (a swizzle changes only bits under 2^(M+B))
  int64_t maxo = 0;
  for (int i = 0; i < L->nleaves; ++i) maxo += (L->shape[i] - 1) * L->stride[i];
  if (L->swz_b > 0) maxo |= (int64_t(1) << (L->swz_m + L->swz_b)) - 1;
  a->s32 = a->small && maxo < (int64_t(1) << 31);
  return LR_OK;
}

}  // namespace lr

using namespace lr;

extern "C" {

const char* lr_last_hip_error(void) { return g_hip_err; }

int lr_layout_eval(const lr_layout* L, const int64_t* idx, int64_t n, int64_t* offsets, void* stream) {
  int rc = validate(L);
  if (rc) return rc;
  if (n < 0 || (n > 0 && !offsets)) return LR_ERR_INVALID;
  if (n == 0) return LR_OK;
  EvalArgs a;
  if ((rc = fill_eval(&a, L))) return rc;
  a.idx = idx;
  a.n = n;
  a.out = offsets;
  if (!idx && a.s32 && ((uintptr_t)offsets & 15u) == 0) {
    // 32-bit arithmetic, two indices per lane: 2^27 indices of a swizzled four-leaf
    // layout in 164 us against 213 us for the 64-bit form
    hipLaunchKernelGGL(k_eval_range32, dim3(grid_cap(std::min<int64_t>((n / 2 + 255) / 256, 65536))), dim3(256), 0,
                       (hipStream_t)stream, a);
    return check_launch();
  }
  hipLaunchKernelGGL(k_eval_index, dim3(grid_cap(std::min<int64_t>((n + 255) / 256, 65536))), dim3(256), 0,
                     (hipStream_t)stream, a);
  return check_launch();
}

int lr_layout_eval_coords(const lr_layout* L, const int64_t* coords, int64_t n, int32_t ncols, int64_t* offsets,
                          void* stream) {
  int rc = validate(L);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!offsets || !coords))) return LR_ERR_INVALID;
  if (ncols != L->nmodes && ncols != L->nleaves) return LR_ERR_INVALID;
  if (n == 0) return LR_OK;
  EvalArgs a;
  if ((rc = fill_eval(&a, L))) return rc;
  a.coords = coords;
  a.ncols = ncols;
  a.n = n;
  a.out = offsets;
  hipLaunchKernelGGL(k_eval_coords, dim3(grid_cap(std::min<int64_t>((n + 255) / 256, 65536))), dim3(256), 0,
                     (hipStream_t)stream, a);
  return check_launch();
}

static int copy_impl(const void* src, const lr_layout* Ls, int64_t src_capacity_elems, void* dst,
                     const lr_layout* Ld, int64_t dst_capacity_elems, size_t elem_bytes, uint32_t flags,
                     const lr_copy_tuning* tuning, int32_t* counts, void* stream);

int lr_layout_copy(const void* src, const lr_layout* Ls, int64_t src_capacity_elems, void* dst, const lr_layout* Ld,
                   int64_t dst_capacity_elems, size_t elem_bytes, uint32_t flags, void* stream) {
  return copy_impl(src, Ls, src_capacity_elems, dst, Ld, dst_capacity_elems, elem_bytes, flags, nullptr, nullptr,
                   stream);
}

int lr_layout_copy_tuned(const void* src, const lr_layout* Ls, int64_t src_capacity_elems, void* dst,
                         const lr_layout* Ld, int64_t dst_capacity_elems, size_t elem_bytes, uint32_t flags,
                         const lr_copy_tuning* tuning, void* stream) {
  return copy_impl(src, Ls, src_capacity_elems, dst, Ld, dst_capacity_elems, elem_bytes, flags, tuning, nullptr,
                   stream);
}

int lr_layout_copy_count_writes(const void* src, const lr_layout* Ls, int64_t src_capacity_elems, void* dst,
                                const lr_layout* Ld, int64_t dst_capacity_elems, size_t elem_bytes, uint32_t flags,
                                const lr_copy_tuning* tuning, int32_t* counts, void* stream) {
  if (!counts) return LR_ERR_INVALID;
  return copy_impl(src, Ls, src_capacity_elems, dst, Ld, dst_capacity_elems, elem_bytes, flags, tuning, counts,
                   stream);
}

static int copy_impl(const void* src, const lr_layout* Ls, int64_t src_capacity_elems, void* dst,
                     const lr_layout* Ld, int64_t dst_capacity_elems, size_t elem_bytes, uint32_t flags,
                     const lr_copy_tuning* tuning, int32_t* counts, void* stream) {
  if (!src || !dst) return LR_ERR_INVALID;
  Plan p;
  int rc = plan_copy(Ls, src_capacity_elems, ptr_align(src), Ld, dst_capacity_elems, ptr_align(dst), elem_bytes,
                     flags, tuning, &p);
  if (rc) return rc;
  // storage overlap: [src, src + cap*eb) vs [dst, dst + cap*eb)
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  const uintptr_t s1 = s0 + (uintptr_t)src_capacity_elems * elem_bytes;
  const uintptr_t d1 = d0 + (uintptr_t)dst_capacity_elems * elem_bytes;
  if (s0 < d1 && d0 < s1) return LR_ERR_OVERLAP;
  if ((rc = verify_plan(p, src_capacity_elems, dst_capacity_elems))) return rc;
  int64_t cext[kMaxJoint], nblocks = 0;
  const bool cut = block_extents(p, flags, cext, &nblocks);
  if (log_enabled()) log_plan(p, cut ? nblocks : 1);
  uint32_t wshift = 0;
  while ((size_t(1) << wshift) < elem_bytes) ++wshift;
  if (!cut) return run_copy(src, Ls, dst, Ld, p, (hipStream_t)stream, WriteCount{counts, wshift});
  // too large for 32-bit offsets: blocks of the joint modes, each within 32 bits,
  // launched one after another on the stream (disjoint parts of an injective copy)
  int64_t start[kMaxJoint] = {0};
  for (int64_t blk = 0; blk < nblocks; ++blk) {
    lr_layout ls, ld;
    int64_t os = 0, od = 0;
    make_block(p, cext, start, &ls, &ld, &os, &od);
    const char* s = (const char*)src + os * (int64_t)elem_bytes;
    char* d = (char*)dst + od * (int64_t)elem_bytes;
    const int64_t cs = cosize_bound(&ls), cd = cosize_bound(&ld);
    Plan pb;
    if ((rc = plan_copy(&ls, cs, ptr_align(s), &ld, cd, ptr_align(d), elem_bytes, flags, tuning, &pb))) return rc;
    if (pb.wide) return LR_ERR_PATH;
    inherit_policy(p, &pb);  // the whole copy's load and store policies
    if ((rc = verify_plan(pb, cs, cd))) return rc;
    if (log_enabled() && blk == 0) log_plan(pb, -1);
    if ((rc = run_copy(s, &ls, d, &ld, pb, (hipStream_t)stream, WriteCount{counts ? counts + od : nullptr, wshift})))
      return rc;
    for (int k = 0; k < p.rank; ++k) {  // next block, mode 0 fastest
      start[k] += cext[k];
      if (start[k] < p.m[k].ext) break;
      start[k] = 0;
    }
  }
  return LR_OK;
}

}  // extern "C"
