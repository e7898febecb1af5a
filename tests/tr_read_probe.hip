// Lane layout of the gfx950 transpose read of 2-byte elements (ds_read_b64_tr_b16),
// as the direct-load transpose uses it.  One wave fills 512 bytes of LDS with the
// 16-bit values 0..255 (each value its own element index), then every lane reads
// 8 bytes at a host-chosen address and writes the 4 values it receives.  Printed
// one JSON line per address pattern: {"pattern": name, "addr": [...], "got": [...]}.
// Every address is checked on the host to lie in [0, 504] and be a multiple of 8,
// so every read stays inside the 512-byte array.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__global__ void __launch_bounds__(64) k_tr_probe(const int* addr, uint16_t* out) {
  __shared__ uint16_t lds[256];
  const int l = threadIdx.x;
  for (int i = l; i < 256; i += 64) lds[i] = (uint16_t)i;
  __syncthreads();
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((char*)lds + addr[l]));
  for (int e = 0; e < 4; ++e) out[4 * l + e] = (uint16_t)v[e];
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
  check(hipMalloc(&dout, 256 * sizeof(uint16_t)), "hipMalloc");
  const char* names[5] = {"identity", "reversed", "times5", "broadcast", "shuffled"};
  for (int pat = 0; pat < 5; ++pat) {
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
    k_tr_probe<<<1, 64>>>(daddr, dout);
    check(hipGetLastError(), "launch");
    uint16_t got[256];
    check(hipMemcpy(got, dout, sizeof got, hipMemcpyDeviceToHost), "copy out");
    std::printf("{\"pattern\": \"%s\", \"addr\": [", names[pat]);
    for (int l = 0; l < 64; ++l) std::printf("%s%d", l ? ", " : "", addr[l]);
    std::printf("], \"got\": [");
    for (int i = 0; i < 256; ++i) std::printf("%s%d", i ? ", " : "", got[i]);
    std::printf("]}\n");
    std::fflush(stdout);
  }
  check(hipFree(daddr), "hipFree");
  check(hipFree(dout), "hipFree");
  return 0;
}
