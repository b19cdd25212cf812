// LDS bank behaviour of this GPU for the access patterns the latent decode kernel uses.
// One workgroup of 16 waves; every wave issues the same per-lane address pattern with one
// instruction kind (16-byte read, 8-byte read, 8-byte transposed read) 4096 times, and the
// rate is reported in bytes per clock for the whole CU.  Conflict-free 16-byte reads run at
// about 250 B/clk; a 2-way conflict halves that.
// Usage: lds_probe   (prints one line per pattern)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <functional>
#include <string>
#include <vector>

namespace {

constexpr int kLds = 65536;
constexpr int kUnroll = 16;
constexpr int kReps = 256;
constexpr int kWaves = 16;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// kind 0: ds_read_b128, 1: ds_read_b64, 2: ds_read_b64_tr_b16
__global__ __launch_bounds__(kWaves * 64) void probe_kernel(const int* offs, int kind,
                                                            long long* cycles, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  for (int i = threadIdx.x; i < kLds / 4; i += blockDim.x) ((uint32_t*)lds)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t addr =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds + offs[lane];
  uint32_t acc = 0;
  __syncthreads();
  const long long t0 = clock64();
  for (int r = 0; r < kReps; ++r) {
    if (kind == 0) {
      u32x4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        asm volatile("ds_read_b128 %0, %1" : "=v"(x[u]) : "v"(addr) : "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= x[u][0] + x[u][3];
    } else {
      u32x2 x[kUnroll];
      if (kind == 1) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          asm volatile("ds_read_b64 %0, %1" : "=v"(x[u]) : "v"(addr) : "memory");
      } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(x[u]) : "v"(addr) : "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= x[u][0] + x[u][1];
    }
  }
  const long long t1 = clock64();
  if (lane == 0) cycles[w] = t1 - t0;
  sink[threadIdx.x] = acc;
}

struct Pattern {
  std::string name;
  int kind;
  std::function<int(int)> off;  // lane -> byte offset
};

// Latent stage rows: 1152 bytes = 72 chunks of 16 bytes.
int old_swizzle(int t) { return (t & 7) ^ ((t >> 3) & 1); }
int new_swizzle(int t) { return (((t >> 1) & 3) << 1) | ((t >> 3) & 1); }

}  // namespace

int main() {
  std::vector<Pattern> pats;
  pats.push_back({"b128 linear (lane * 16)", 0, [](int l) { return 16 * l; }});
  pats.push_back({"b128 rows of 1152 B, same chunk", 0,
                  [](int l) { return 16 * ((l & 15) * 72 + (l >> 4)); }});
  // lanes l and l + 16: group 1 reads slot (j ^ x) of another row where group 0 reads slot j
  for (int x : {0, 1, 2, 3, 4, 8, 12, 15})
    pats.push_back({"b128 lanes l, l+16 on slots j, j^" + std::to_string(x), 0, [x](int l) {
                      const int G = l >> 4, j = l & 15;
                      return 1280 * G + 16 * (G == 1 ? (j ^ x) : j);
                    }});
  // score tile (16 consecutive rows, one chunk per 16-lane group g)
  pats.push_back({"b128 score tile, old swizzle", 0, [](int l) {
                    const int t = l & 15, g = l >> 4;
                    return 16 * (t * 72 + (g ^ old_swizzle(t)));
                  }});
  for (int ks : {0, 7, 15, 16, 17})
    pats.push_back({"b128 score tile, new swizzle, product " + std::to_string(ks), 0, [ks](int l) {
                      const int t = 16 + (l & 15), g = l >> 4;
                      const int L = ks < 16 ? ks + 16 * g : 64 + 4 * (ks - 16) + 2 * (g & 1) + (g >> 1);
                      return 16 * (t * 72 + (L ^ new_swizzle(t)));
                    }});
  pats.push_back({"b128 P read, 80-byte head rows", 0,
                  [](int l) { return (l & 15) * 80 + 16 * (l >> 4); }});
  pats.push_back({"b128 P read, 1 KiB slabs", 0,
                  [](int l) { return 1024 * (l >> 4) + 256 + 16 * (l & 15); }});
  pats.push_back({"b64 linear (lane * 8)", 1, [](int l) { return 8 * l; }});
  pats.push_back({"b64 lanes l, l+32 on pairs j, j^16", 1, [](int l) {
                    const int H = l >> 5, j = l & 31;
                    return 1280 * H + 8 * (H ? j ^ 16 : j);
                  }});
  pats.push_back({"tr64 linear (lane * 8)", 2, [](int l) { return 8 * l; }});
  pats.push_back({"tr64 V read, old rows 8 g + 4 h + i/4, old swizzle", 2, [](int l) {
                    const int i = l & 15, g = l >> 4, t = 8 * g + (i >> 2);
                    return 16 * (t * 72 + (((i & 3) >> 1) ^ old_swizzle(t))) + 8 * (i & 1);
                  }});
  for (int h = 0; h < 2; ++h)
    for (int n4 : {0, 3})
      pats.push_back({"tr64 V read, new rows, new swizzle, h " + std::to_string(h) + " n4 " +
                          std::to_string(n4), 2, [h, n4](int l) {
                        const int i = l & 15, g = l >> 4;
                        const int t = 4 * (4 * (g >> 1) + 2 * h + (g & 1)) + (i >> 2);
                        return 16 * (t * 72 + 48 + ((2 * n4 + ((i & 3) >> 1)) ^ new_swizzle(t))) +
                               8 * (i & 1);
                      }});

  int* d_off = nullptr;
  long long* d_cycles = nullptr;
  uint32_t* d_sink = nullptr;
  if (hipMalloc(&d_off, 64 * sizeof(int)) != hipSuccess ||
      hipMalloc(&d_cycles, kWaves * sizeof(long long)) != hipSuccess ||
      hipMalloc(&d_sink, kWaves * 64 * sizeof(uint32_t)) != hipSuccess) {
    fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }
  printf("%-56s %10s\n", "pattern (16 waves, same addresses in every wave)", "B/clk/CU");
  for (const Pattern& p : pats) {
    int off[64];
    const int align = p.kind == 0 ? 16 : 8, width = p.kind == 0 ? 16 : 8;
    for (int l = 0; l < 64; ++l) {
      off[l] = p.off(l);
      if (off[l] < 0 || off[l] + width > kLds || off[l] % align) {
        fprintf(stderr, "offset out of range in pattern %s\n", p.name.c_str());
        return 1;
      }
    }
    if (hipMemcpy(d_off, off, sizeof(off), hipMemcpyHostToDevice) != hipSuccess) return 1;
    double best = 1e30;
    for (int it = 0; it < 3; ++it) {
      hipLaunchKernelGGL(probe_kernel, dim3(1), dim3(kWaves * 64), 0, 0, d_off, p.kind, d_cycles,
                         d_sink);
      if (hipDeviceSynchronize() != hipSuccess) {
        fprintf(stderr, "kernel failed\n");
        return 1;
      }
      long long c[kWaves];
      if (hipMemcpy(c, d_cycles, sizeof(c), hipMemcpyDeviceToHost) != hipSuccess) return 1;
      long long mx = 0;
      for (long long v : c) mx = v > mx ? v : mx;
      best = mx < best ? (double)mx : best;
    }
    const double per_inst = best / (double)(kReps * kUnroll);  // cycles per instruction per wave
    printf("%-56s %10.1f\n", p.name.c_str(), kWaves * 64.0 * width / per_inst);
  }
  return 0;
}
