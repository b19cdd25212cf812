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

// ---- Quantizing append: bf16 rows -> FP8 E4M3 codes with one fp32 scale per KV head
// ("PD 分离下的 KV Cache", "优化三：KV 传输优化": KV carried as FP8).  The code of x is the
// E4M3 value nearest to the fp32 quotient x / scale (IEEE division), ties to the even code;
// magnitudes >= 448 (the largest finite E4M3) and infinities saturate to +-448, NaN stays
// NaN.  The rounding is done on the quotient's bits, so it does not depend on a hardware
// conversion's saturation or rounding mode.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |v| >= 448 (and infinity)
  if (a < 0x3C800000u) {                       // |v| < 2^-6: multiples of 2^-9 (0x08 = 2^-6)
    const float units = __uint_as_float(a) * 512.0f;  // exact
    return sign | (uint32_t)__builtin_rintf(units);    // nearest, ties to even
  }
  // normal: biased exponent 1..15, keep 3 of the 23 mantissa bits, round to nearest even
  uint32_t code = ((((a >> 23) - 127u + 7u) << 3)) | ((a >> 20) & 7u);
  const uint32_t rest = a & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) ++code;  // carries into the exponent
  return sign | code;
}

// One thread per 16 elements of one (token, head) row; blockIdx.y selects K (0) or V (1).
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(AppendFp8Args a) {
  const int groups = a.d >> 4;
  const long long total = (long long)a.T * a.Hkv * groups;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int grp = (int)(idx % groups);
  const long long th = idx / groups;  // token * Hkv + head
  const int h = (int)(th % a.Hkv);
  const int i = (int)(th / a.Hkv);
  const int64_t slot = a.slots[i];
  if (slot < 0 || slot >= (int64_t)a.num_blocks * a.block_size) return;
  const bool is_v = blockIdx.y == 1;
  const uint16_t* src = (is_v ? a.v_new : a.k_new) + (size_t)th * a.d + 16 * grp;
  const float scale = (is_v ? a.v_scale : a.k_scale)[h];
  const uint4 lo = *(const uint4*)src, hi = *(const uint4*)(src + 8);
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t packed[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
    const uint32_t code = f32_to_e4m3(__fdiv_rn(__uint_as_float(bits), scale));
    packed[e >> 2] |= code << (8 * (e & 3));
  }
  const int64_t phys = slot / a.block_size, off = slot % a.block_size;
  uint8_t* dst = (is_v ? a.v_pool : a.k_pool) +
                 (((size_t)phys * a.Hkv + h) * a.block_size + off) * (size_t)a.d + 16 * grp;
  *(uint4*)dst = uint4{packed[0], packed[1], packed[2], packed[3]};
}

hipError_t launch_kv_append_fp8(const AppendFp8Args& a, hipStream_t s) {
  const long long total = (long long)a.T * a.Hkv * (a.d >> 4);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  dim3 grid((unsigned)((total + threads - 1) / threads), a.v_pool ? 2u : 1u);
  hipLaunchKernelGGL(kv_append_fp8_kernel, grid, dim3(threads), 0, s, a);
  return hipGetLastError();
}

// ---- Block copy for copy-on-write ("深入LLM推理：从KV Cache到PD分离的Serving全景解析",
// "PagedAttention与Cache管理": shared physical blocks): block dst[i] <- block src[i], every
// head and row, 16 bytes per thread; pairs with an id outside the pool are skipped.
// blockIdx.y selects the K (0) or V (1) pool.
__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(CopyBlocksArgs a) {
  const long long chunks = a.block_bytes >> 4;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.n * chunks) return;
  const int i = (int)(idx / chunks);
  const long long c = idx - (long long)i * chunks;
  const int32_t sb = a.src[i], db = a.dst[i];
  if ((unsigned)sb >= (unsigned)a.num_blocks || (unsigned)db >= (unsigned)a.num_blocks) return;
  uint8_t* pool = blockIdx.y == 1 ? a.v_pool : a.k_pool;
  *(uint4*)(pool + (size_t)db * a.block_bytes + 16 * c) =
      *(const uint4*)(pool + (size_t)sb * a.block_bytes + 16 * c);
}

hipError_t launch_kv_copy_blocks(const CopyBlocksArgs& a, hipStream_t s) {
  const long long total = (long long)a.n * (a.block_bytes >> 4);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  dim3 grid((unsigned)((total + threads - 1) / threads), a.v_pool ? 2u : 1u);
  hipLaunchKernelGGL(kv_copy_blocks_kernel, grid, dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
