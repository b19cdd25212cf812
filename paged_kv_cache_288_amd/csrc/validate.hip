// Debug check of the caller's side of the interface contract: the device-resident block
// tables, context lengths and append slots that the decode and append calls trust.
//
// The paging of "深入LLM推理：从KV Cache到PD分离的Serving全景解析", section
// "PagedAttention与Cache管理", is correct only if every table entry a sequence uses names a
// block of the pool and no two new tokens are written to the same slot.  The kernels never
// fault on a bad value (out-of-range ids and slots are skipped, lengths clamped), but their
// results are then unspecified; this call counts such values so that a caller can find
// them.  It also counts what the kernels would silently truncate or lose: context lengths
// above the max_context_len a decode call is given (the kernels clamp to it) and bf16
// values of V at or above fp16's largest finite magnitude (the p.V step widens V to fp16).
// Counting is by vector atomics into six device ints, zeroed by the first kernel.
#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

constexpr int kCounts = 6;

__global__ void validate_zero_kernel(int32_t* counts) {
  if (threadIdx.x < kCounts) counts[threadIdx.x] = 0;
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
  if (j == 0 && a.max_context_len >= 0 && L > a.max_context_len) atomicAdd(&a.counts[4], 1);
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

// One workgroup per (sequence, table entry in use): counts[5] gets the bf16 values among
// the first d_v dims of every KV head's rows of that block's tokens in use (L clamped to
// the table and to max_context_len) whose magnitude is 65504 or more, infinities included
// (bf16 has no value between 65280 and 65536, so that is |bits| in [0x4780, 0x7F80]).
__global__ __launch_bounds__(256) void validate_values_kernel(ValidateArgs a) {
  const int b = blockIdx.x / a.max_blocks, j = blockIdx.x % a.max_blocks;
  const int cap = a.max_blocks * a.block_size;
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  if (a.max_context_len >= 0 && L > a.max_context_len) L = a.max_context_len;
  const int t0 = j * a.block_size;
  if (t0 >= L) return;
  const int phys = a.block_table[(size_t)b * a.max_blocks + j];
  if (phys < 0 || phys >= a.num_blocks) return;
  const int ntok = min(a.block_size, L - t0);
  const long long n = (long long)a.Hkv * ntok * a.d_v;
  int found = 0;
  for (long long e = threadIdx.x; e < n; e += blockDim.x) {
    const int i = (int)(e % a.d_v);
    const long long r = e / a.d_v;
    const int t = (int)(r % ntok), h = (int)(r / ntok);
    const uint16_t x = a.v_pool[(((size_t)phys * a.Hkv + h) * a.block_size + t) * a.d + i] & 0x7FFF;
    found += (x >= 0x4780 && x <= 0x7F80);
  }
  if (found) atomicAdd(&a.counts[5], found);
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
    if (e != hipSuccess) return e;
  }
  if (a.v_pool && entries > 0) {
    hipLaunchKernelGGL(validate_values_kernel, dim3((unsigned)entries), dim3(256), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pkv
