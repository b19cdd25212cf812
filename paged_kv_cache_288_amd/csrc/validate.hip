// Debug check of the caller's side of the interface contract: the device-resident block
// tables, context lengths and append slots that the decode and append calls trust.
//
// The paging of "深入LLM推理：从KV Cache到PD分离的Serving全景解析", section
// "PagedAttention与Cache管理", is correct only if every table entry a sequence uses names a
// block of the pool and no two new tokens are written to the same slot.  The kernels never
// fault on a bad value (out-of-range ids and slots are skipped, lengths clamped), but their
// results are then unspecified; this call counts such values so that a caller can find
// them.  Counting is by vector atomics into four device ints, zeroed by the first kernel.
#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

__global__ void validate_zero_kernel(int32_t* counts) {
  if (threadIdx.x < 4) counts[threadIdx.x] = 0;
}

// One thread per (sequence, table entry): counts[1] gets lengths outside
// [0, max_blocks * block_size] (entry 0's thread), counts[0] entries among the first
// ceil(L / block_size) outside [0, num_blocks), L clamped to the table.
__global__ __launch_bounds__(256) void validate_tables_kernel(ValidateArgs a) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.B * a.max_blocks) return;
  const int b = (int)(idx / a.max_blocks), j = (int)(idx % a.max_blocks);
  const int cap = a.max_blocks * a.block_size;
  int L = a.context_lens[b];
  if (j == 0 && (L < 0 || L > cap)) atomicAdd(&a.counts[1], 1);
  L = L < 0 ? 0 : (L > cap ? cap : L);
  if (j < (L + a.block_size - 1) / a.block_size) {
    const int phys = a.block_table[(size_t)b * a.max_blocks + j];
    if (phys < 0 || phys >= a.num_blocks) atomicAdd(&a.counts[0], 1);
  }
}

// One thread per new token: counts[2] gets slots at or past num_blocks * block_size,
// counts[3] non-negative slots already used by an earlier token of the call (O(T^2)).
__global__ __launch_bounds__(256) void validate_slots_kernel(ValidateArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.T) return;
  const int64_t s = a.slots[i];
  if (s >= (int64_t)a.num_blocks * a.block_size) atomicAdd(&a.counts[2], 1);
  if (s < 0) return;
  for (int j = 0; j < i; ++j)
    if (a.slots[j] == s) {
      atomicAdd(&a.counts[3], 1);
      break;
    }
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(validate_zero_kernel, dim3(1), dim3(64), 0, s, a.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long entries = (long long)a.B * a.max_blocks;
  if (entries > 0) {
    hipLaunchKernelGGL(validate_tables_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0,
                       s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.T > 0 && a.slots) {
    hipLaunchKernelGGL(validate_slots_kernel, dim3((unsigned)((a.T + 255) / 256)), dim3(256), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pkv
