// Slot-mapped append of new K/V rows into the block pool (bit-exact 16-byte copies).
//
// Addressing follows the block table of "深入LLM推理：从KV Cache到PD分离的Serving全景解析",
// section "PagedAttention与Cache管理": slot = physical block * block_size + offset.
// Pool layout [num_blocks][Hkv][block_size][row], row = d elements.
#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

// One thread per 16-byte chunk of one (token, head) row; blockIdx.y selects K (0) or V (1).
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int chunks_per_row = a.row_bytes >> 4;
  const long long total = (long long)a.T * a.Hkv * chunks_per_row;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int chunk = (int)(idx % chunks_per_row);
  const long long th = idx / chunks_per_row;  // token * Hkv + head
  const int h = (int)(th % a.Hkv);
  const int i = (int)(th / a.Hkv);
  const int64_t slot = a.slots[i];
  const int64_t nslots = (int64_t)a.num_blocks * a.block_size;
  if (slot < 0 || slot >= nslots) return;
  const int64_t phys = slot / a.block_size;
  const int64_t off = slot % a.block_size;
  const bool is_v = blockIdx.y == 1;
  const uint8_t* src = (const uint8_t*)(is_v ? a.v_new : a.k_new);
  uint8_t* dst = (uint8_t*)(is_v ? a.v_pool : a.k_pool);
  const size_t src_off = ((size_t)th * chunks_per_row + chunk) * 16;
  const size_t dst_off = (((size_t)phys * a.Hkv + h) * a.block_size + off) * (size_t)a.row_bytes +
                         (size_t)chunk * 16;
  *(uint4*)(dst + dst_off) = *(const uint4*)(src + src_off);
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  const long long total = (long long)a.T * a.Hkv * (a.row_bytes >> 4);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  dim3 grid((unsigned)((total + threads - 1) / threads), a.v_pool ? 2u : 1u);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
