// Lane layouts of the gfx950 transpose reads of 2-byte and 1-byte elements
// (ds_read_b64_tr_b16, ds_read_b64_tr_b8), as the direct-load transpose uses them.
// One wave fills 512 bytes of LDS, then every lane reads 8 bytes at a host-chosen
// address and writes what it receives.  The 2-byte form holds the 16-bit values
// 0..255 (each its own element index); the 1-byte form runs twice, over the low and
// then the high byte of each byte's own index (0..511), and the host joins the two.
// Printed one JSON line per read and address pattern:
// {"read": "tr16" | "tr8", "pattern": name, "addr": [...], "got": [...]}.  Every
// address is checked on the host to lie in [0, 504] and be a multiple of 8, so every
// read stays inside the 512-byte array.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

__global__ void __launch_bounds__(64) k_tr_probe(const int* addr, uint16_t* out) {
  __shared__ uint16_t lds[256];
  const int l = threadIdx.x;
  for (int i = l; i < 256; i += 64) lds[i] = (uint16_t)i;
  __syncthreads();
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((char*)lds + addr[l]));
  for (int e = 0; e < 4; ++e) out[4 * l + e] = (uint16_t)v[e];
}

// hi = 0: each byte holds the low byte of its index, hi = 1 the high byte
__global__ void __launch_bounds__(64) k_tr8_probe(const int* addr, int hi, uint16_t* out) {
  __shared__ uint8_t lds[512];
  const int l = threadIdx.x;
  for (int i = l; i < 512; i += 64) lds[i] = (uint8_t)(hi ? i >> 8 : i & 255);
  __syncthreads();
  const v2i32 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)((char*)lds + addr[l]));
  for (int e = 0; e < 8; ++e) out[8 * l + e] = (uint16_t)((uint32_t)v[e / 4] >> (8 * (e % 4)) & 255);
}

static void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

int main() {
  int* daddr = nullptr;
  uint16_t* dout = nullptr;
  check(hipMalloc(&daddr, 64 * sizeof(int)), "hipMalloc");
  check(hipMalloc(&dout, 512 * sizeof(uint16_t)), "hipMalloc");
  const char* names[5] = {"identity", "reversed", "times5", "broadcast", "shuffled"};
  for (int run = 0; run < 10; ++run) {
    const int pat = run % 5;
    const bool tr8 = run >= 5;
    int addr[64];
    int perm[64];
    for (int l = 0; l < 64; ++l) perm[l] = l;
    uint32_t x = 12345u;  // a fixed shuffle (linear congruential draws)
    for (int l = 63; l > 0; --l) {
      x = x * 1664525u + 1013904223u;
      const int j = (int)((x >> 8) % (uint32_t)(l + 1));
      const int tmp = perm[l];
      perm[l] = perm[j];
      perm[j] = tmp;
    }
    for (int l = 0; l < 64; ++l) {
      const int row = pat == 0 ? l : pat == 1 ? 63 - l : pat == 2 ? (5 * l) % 64 : pat == 3 ? 7 : perm[l];
      addr[l] = 8 * row;
      if (addr[l] < 0 || addr[l] > 504 || addr[l] % 8) {
        std::fprintf(stderr, "address out of range\n");
        return 1;
      }
    }
    check(hipMemcpy(daddr, addr, sizeof addr, hipMemcpyHostToDevice), "copy in");
    uint16_t got[512];
    int n = 256;
    if (!tr8) {
      k_tr_probe<<<1, 64>>>(daddr, dout);
      check(hipGetLastError(), "launch");
      check(hipMemcpy(got, dout, 256 * sizeof(uint16_t), hipMemcpyDeviceToHost), "copy out");
    } else {
      n = 512;
      uint16_t lo[512];
      k_tr8_probe<<<1, 64>>>(daddr, 0, dout);
      check(hipGetLastError(), "launch");
      check(hipMemcpy(lo, dout, sizeof lo, hipMemcpyDeviceToHost), "copy out");
      k_tr8_probe<<<1, 64>>>(daddr, 1, dout);
      check(hipGetLastError(), "launch");
      check(hipMemcpy(got, dout, sizeof got, hipMemcpyDeviceToHost), "copy out");
      for (int i = 0; i < 512; ++i) got[i] = (uint16_t)(got[i] << 8 | lo[i]);
    }
    std::printf("{\"read\": \"%s\", \"pattern\": \"%s\", \"addr\": [", tr8 ? "tr8" : "tr16", names[pat]);
    for (int l = 0; l < 64; ++l) std::printf("%s%d", l ? ", " : "", addr[l]);
    std::printf("], \"got\": [");
    for (int i = 0; i < n; ++i) std::printf("%s%d", i ? ", " : "", got[i]);
    std::printf("]}\n");
    std::fflush(stdout);
  }
  check(hipFree(daddr), "hipFree");
  check(hipFree(dout), "hipFree");
  return 0;
}
