// Achievable HBM read bandwidth on this GPU: a grid-stride kernel reading a 4 GiB buffer
// with 16-byte loads (plain and nontemporal), and scattered whole-chunk reads as a paged KV
// cache does, for comparison with the decode kernels.  Every configuration runs twice: on a
// buffer of one repeated byte and on pseudo-random bits (KV data is random; the two agree to
// about 1 %, so the ceiling does not depend on the data).
// Usage: read_ceiling   (prints one line per configuration, GB/s)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

template <int UNROLL, bool NT>
__global__ void read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  size_t i = (size_t)blockIdx.x * blockDim.x * UNROLL + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x * UNROLL;
  uint32_t acc = 0;
  for (; i + (size_t)(UNROLL - 1) * blockDim.x < n16; i += stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      v[u] = NT ? __builtin_nontemporal_load(p + i + u * blockDim.x) : p[i + u * blockDim.x];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x12345678u) out[blockIdx.x] = acc;  // keeps the loads live
}

// Chunked variant: each wave reads whole CHUNK-byte pieces (1 KiB per load instruction) at
// scattered chunk indices (a fixed odd-multiplier permutation), as a paged KV cache does.
template <int CHUNK, bool NT>
__global__ void chunk_kernel(const u32x4* __restrict__ p, size_t nchunks, uint32_t* out) {
  constexpr int PER = CHUNK / 1024;   // load instructions per chunk per wave
  const int lane = threadIdx.x & 63;
  const size_t wave = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const size_t nwaves = ((size_t)gridDim.x * blockDim.x) >> 6;
  uint32_t acc = 0;
  for (size_t i = wave; i < nchunks; i += nwaves) {
    const size_t c = (i * 2654435761ull) % nchunks;   // odd multiplier: a permutation when nchunks is a power of two
    const u32x4* q = p + c * (CHUNK / 16) + lane;
    u32x4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = NT ? __builtin_nontemporal_load(q + u * 64) : q[u * 64];
#pragma unroll
    for (int u = 0; u < PER; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x12345678u) out[blockIdx.x] = acc;
}

// Pseudo-random 32-bit words (an integer hash of the index; any well-mixed bits will do).
__global__ void fill_random(uint32_t* p, size_t n, uint32_t seed) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    uint32_t x = (uint32_t)i * 2654435761u ^ seed;
    x ^= x >> 13;
    x *= 0x5bd1e995u;
    x ^= x >> 15;
    p[i] = x;
  }
}

template <int CHUNK, bool NT>
static void run_chunks(const u32x4* p, size_t bytes, uint32_t* out, int blocks) {
  const size_t nchunks = bytes / CHUNK;
  hipEvent_t a, b;
  (void)hipEventCreate(&a);
  (void)hipEventCreate(&b);
  for (int w = 0; w < 2; ++w)
    hipLaunchKernelGGL((chunk_kernel<CHUNK, NT>), dim3(blocks), dim3(256), 0, 0, p, nchunks, out);
  (void)hipEventRecord(a);
  const int iters = 10;
  for (int w = 0; w < iters; ++w)
    hipLaunchKernelGGL((chunk_kernel<CHUNK, NT>), dim3(blocks), dim3(256), 0, 0, p, nchunks, out);
  (void)hipEventRecord(b);
  (void)hipEventSynchronize(b);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  printf("scattered %d KiB chunks, loads=%s workgroups=%d: %.1f GB/s\n", CHUNK / 1024,
         NT ? "nontemporal" : "plain", blocks, (double)nchunks * CHUNK * iters / (ms * 1e-3) / 1e9);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
}

template <int U, bool NT>
static void run(const u32x4* p, size_t n16, uint32_t* out, int blocks) {
  hipEvent_t a, b;
  (void)hipEventCreate(&a);
  (void)hipEventCreate(&b);
  for (int w = 0; w < 2; ++w)
    hipLaunchKernelGGL((read_kernel<U, NT>), dim3(blocks), dim3(256), 0, 0, p, n16, out);
  (void)hipEventRecord(a);
  const int iters = 10;
  for (int w = 0; w < iters; ++w)
    hipLaunchKernelGGL((read_kernel<U, NT>), dim3(blocks), dim3(256), 0, 0, p, n16, out);
  (void)hipEventRecord(b);
  (void)hipEventSynchronize(b);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  printf("loads=%s unroll=%d workgroups=%d: %.1f GB/s\n", NT ? "nontemporal" : "plain", U, blocks,
         n16 * 16.0 * iters / (ms * 1e-3) / 1e9);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
}

int main() {
  const size_t bytes = 4ull << 30, n16 = bytes / 16;
  u32x4* p = nullptr;
  uint32_t* out = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess || hipMalloc(&out, 8192 * sizeof(uint32_t)) != hipSuccess) {
    printf("allocation failed\n");
    return 1;
  }
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 0) {
      (void)hipMemset(p, 1, bytes);
      printf("-- data: every byte 0x01\n");
    } else {
      hipLaunchKernelGGL(fill_random, dim3(4096), dim3(256), 0, 0, (uint32_t*)p, bytes / 4, 12345u);
      printf("-- data: pseudo-random bits\n");
    }
    (void)hipDeviceSynchronize();
    for (int blocks : {1024, 2048, 4096, 8192}) {
      run<4, false>(p, n16, out, blocks);
      run<8, false>(p, n16, out, blocks);
      run<4, true>(p, n16, out, blocks);
    }
    for (int blocks : {2048, 8192}) {
      run_chunks<4096, false>(p, bytes, out, blocks);
      run_chunks<4096, true>(p, bytes, out, blocks);
      run_chunks<8192, true>(p, bytes, out, blocks);
      run_chunks<16384, true>(p, bytes, out, blocks);
    }
  }
  (void)hipFree(p);
  (void)hipFree(out);
  return 0;
}
