// Latent (MLA) paged decode attention on gfx950 with bf16 MFMA.
//
// What is computed ("深入LLM推理：从KV Cache到PD分离的Serving全景解析", section
// "KV Cache：Transformer的循环状态"; "GPU推理深度拆解：KV Cache视角", "KV Cache 大小与分配演进"):
// every token caches one latent row of 576 dims (512 latent + 64 RoPE); all query heads
// attend to it, using the whole row as key and its first 512 dims as value:
//     out[b][h] = softmax_t(scale * q[b][h] . C_t) C_t[0:512].
// With 128 heads sharing each latent row this is a dense contraction (about 240 flop
// per byte read), so both products run on MFMA (v_mfma_f32_16x16x32_bf16 for the scores,
// v_mfma_f32_16x16x32_f16 for P V; fp32 accumulate).
//
// Work decomposition: one workgroup of 4 waves per (sequence, context partition, group of
// 64 query heads); wave w owns 16 heads.  The partition is walked in stages of 32 tokens
// (half a 64-token block).  Each stage is staged into LDS twice by all 256 threads:
//  * token-major K[32][576] (rows padded to 1168 bytes): A operand of S^T = K Q^T, where a
//    lane needs 8 consecutive dims of one token;
//  * dim-major V^T[512][32] in fp16 (rows padded to 72 bytes), built with an in-register
//    transpose: B operand of O = P V, where a lane needs 8 tokens of one dim.
// Scores are produced transposed (tokens x heads), which leaves each lane holding one head
// and 8 tokens: after the online-softmax update these 8 probabilities, rounded to bf16, are
// exactly that lane's A operand for P V, so no data moves between the two products.  P V
// runs on the fp16 MFMA (probabilities and V in fp16: 10-bit mantissas, so rounding the
// weights costs 2^-11 relative instead of bf16's 2^-9).
// The token order inside a P V contraction step is (4g..4g+3, 16+4g..16+4g+3) for lane group
// g; the V^T reads use the same order.  The running max moves lazily (only when a score
// exceeds it by more than 2^8).  Partitions of a split context write (m, l, o) partials
// that the shared merge kernel combines.
#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBlock = 64;
constexpr int kStage = 32;                  // tokens per LDS stage
constexpr int kWaves = 4;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerGroup = kWaves * kHeadsPerWave;
constexpr int kRowBytes = kDqk * 2;         // 1152
constexpr int kKStride = 1168;              // padded K row in LDS (bytes)
constexpr int kVtStride = 72;               // padded V^T row in LDS (bytes)
constexpr int kKLds = kStage * kKStride;    // 37376
constexpr int kVtLds = kDv * kVtStride;     // 36864
constexpr float kSlack = 8.0f;

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_h(const f16x8_t& a, const f16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t dword(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ float shfl(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// Max / sum over the 4 lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_max4(float x) {
  float lo, hi, e, o;
  halves_pair32(x, lo, hi);
  x = fmaxf(lo, hi);
  rows_pair16(x, e, o);
  return fmaxf(e, o);
}
__device__ __forceinline__ float group_sum4(float x) {
  float lo, hi, e, o;
  halves_pair32(x, lo, hi);
  x = lo + hi;
  rows_pair16(x, e, o);
  return e + o;
}

}  // namespace

__global__ __launch_bounds__(kWaves * kWave, 2) void mla_decode_kernel(MlaArgs a, int head_groups,
                                                                        int units) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kKLds + kVtLds];
  uint8_t* ldsK = lds;
  uint8_t* ldsVt = lds + kKLds;

  // Workgroup id -> (unit = sequence * P + partition, head group).  Eight consecutive ids
  // share a head group and cover eight units; the next eight cover the same units with the
  // next head group, so with round-robin dispatch over the 8 XCDs all head groups of a unit
  // run on the same XCD and share its L2.
  const int x = blockIdx.x;
  const int unit = (x / (8 * head_groups)) * 8 + (x & 7);
  const int hg = (x >> 3) % head_groups;
  if (unit >= units) return;
  const int b = unit / a.num_partitions, part = unit % a.num_partitions;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int h0 = hg * kHeadsPerGroup + w * kHeadsPerWave;
  const bool active = h0 < a.Hq;

  int L = a.context_lens[b];
  const int cap = min(a.max_blocks * a.block_size, a.max_context_len);
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int t0 = part * a.partition;
  if (t0 >= L) {
    if (a.num_partitions == 1 && part == 0 && active) {
      for (int i = lane; i < kHeadsPerWave * kDv; i += kWave)
        a.out[((size_t)b * a.Hq + h0) * kDv + i] = 0.f;
    }
    return;
  }
  const int t1 = min(L, t0 + a.partition);

  // q fragments: B operand of S^T = K Q^T, lane (g, c16): head h0 + c16, dims 32*ks + 8g..+8.
  bf16x8_t qf[kDqk / 32];
  {
    const int h = active ? h0 + c16 : 0;
    const uint8_t* qrow = (const uint8_t*)(a.q + ((size_t)b * a.Hq + h) * kDqk);
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qrow + ks * 64 + 16 * g));
  }

  f32x4_t o[kDv / 16];
#pragma unroll
  for (int n = 0; n < kDv / 16; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;   // this lane's head (c16), identical in the 4 lane groups
  float l_part = 0.f;      // this lane's share of the head's probability sum
  const float cscale = a.scale * kLog2e;

  for (int ts = t0; ts < t1; ts += kStage) {
    const int valid_raw = min(kStage, t1 - ts);
    const int phys = a.block_table[(size_t)b * a.max_blocks + ts / kBlock];
    const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
    const int valid = ok ? valid_raw : 0;
    const uint8_t* src = (const uint8_t*)a.kv_pool +
                         ((size_t)(ok ? phys : 0) * kBlock + (ts % kBlock)) * kRowBytes;

    __syncthreads();  // the previous stage's readers are done with the LDS
    {
      // latent dims 0..511: 8 groups of 4 tokens x 64 chunks of 8 dims, two per thread;
      // each is written token-major (K) and, after a 4x8 transpose, dim-major (V^T)
      const int dc = tid & 63;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tq = (tid >> 6) + 4 * half;   // token quad 0..7
        uint4 X[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int tok = 4 * tq + tt;
          X[tt] = *(const uint4*)(src + tok * kRowBytes + dc * 16);
          if (tok >= valid) X[tt] = uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          *(uint4*)(ldsK + (4 * tq + tt) * kKStride + dc * 16) = X[tt];
#pragma unroll
        for (int dd2 = 0; dd2 < 4; ++dd2) {  // V^T is kept in fp16 (exact for |v| < 65504)
          const uint32_t x0 = dword(X[0], dd2), x1 = dword(X[1], dd2);
          const uint32_t x2 = dword(X[2], dd2), x3 = dword(X[3], dd2);
          uint8_t* r0 = ldsVt + (8 * dc + 2 * dd2) * kVtStride + tq * 8;
          *(uint2*)(r0) = uint2{pack_f16(bf16_lo(x0), bf16_lo(x1)), pack_f16(bf16_lo(x2), bf16_lo(x3))};
          *(uint2*)(r0 + kVtStride) =
              uint2{pack_f16(bf16_hi(x0), bf16_hi(x1)), pack_f16(bf16_hi(x2), bf16_hi(x3))};
        }
      }
      // RoPE dims 512..575: thread -> (token tid/8, chunk tid%8)
      const int rt = tid >> 3, rc = tid & 7;
      uint4 R = *(const uint4*)(src + rt * kRowBytes + 1024 + rc * 16);
      if (rt >= valid) R = uint4{0, 0, 0, 0};
      *(uint4*)(ldsK + rt * kKStride + 1024 + rc * 16) = R;
    }
    __syncthreads();
    if (!active) continue;

    // ---- S^T = K Q^T for the stage's two 16-token tiles
    f32x4_t s[2];
    s[0] = s[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* krow0 = ldsK + c16 * kKStride + 16 * g;
      const uint8_t* krow1 = krow0 + 16 * kKStride;
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks) {
        const bf16x8_t k0 = __builtin_bit_cast(bf16x8_t, *(const uint4*)(krow0 + ks * 64));
        const bf16x8_t k1 = __builtin_bit_cast(bf16x8_t, *(const uint4*)(krow1 + ks * 64));
        s[0] = mfma(k0, qf[ks], s[0]);
        s[1] = mfma(k1, qf[ks], s[1]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // then 2 MFMA
      }
    }

    // ---- online softmax (log2 domain); lane holds tokens tile*16 + 4g + i of head c16
    float sv[8];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tile * 16 + 4 * g + i;
        sv[4 * tile + i] = tok < valid ? s[tile][i] * cscale : kNegInf;
      }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
    mt = group_max4(mt);
    if (wave_any(mt > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_part *= alpha;
      m_run = m_new;
      // o rows are heads 4g+i: fetch those heads' factors
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = shfl(alpha, 4 * g + i);
#pragma unroll
        for (int n = 0; n < kDv / 16; ++n) o[n][i] *= ai;
      }
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    // probabilities in fp16 (p <= 2^8 after the lazy max; 2^-11 relative rounding)
    uint32_t pp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pp[j] = pack_f16(fast_exp2(sv[2 * j] - m_use), fast_exp2(sv[2 * j + 1] - m_use));
#pragma unroll
    for (int j = 0; j < 4; ++j) l_part = dot2h(pp[j], kOnesF16x2, l_part);
    const f16x8_t pf = __builtin_bit_cast(f16x8_t, uint4{pp[0], pp[1], pp[2], pp[3]});

    // ---- O += P V over the stage's 32 tokens, 32 tiles of 16 output dims
#pragma unroll
    for (int n = 0; n < kDv / 16; ++n) {
      const uint8_t* vrow = ldsVt + (16 * n + c16) * kVtStride;
      const uint2 v0 = *(const uint2*)(vrow + 8 * g);        // tokens 4g..4g+3
      const uint2 v1 = *(const uint2*)(vrow + 32 + 8 * g);   // tokens 16+4g..16+4g+3
      const f16x8_t vf = __builtin_bit_cast(f16x8_t, uint4{v0.x, v0.y, v1.x, v1.y});
      o[n] = mfma_h(pf, vf, o[n]);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // the next tiles' LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // interleaved with the MFMAs
    }
  }
  if (!active) return;

  // ---- epilogue: per-head sum, then output rows (heads 4g+i) or partials
  const float l_head = group_sum4(l_part);        // head c16
  float li[4], mi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    li[i] = shfl(l_head, 4 * g + i);
    mi[i] = shfl(m_run, 4 * g + i);
  }
  if (a.num_partitions == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv = li[i] > 0.f ? 1.f / li[i] : 0.f;
      float* orow = a.out + ((size_t)b * a.Hq + h0 + 4 * g + i) * kDv;
#pragma unroll
      for (int n = 0; n < kDv / 16; ++n) orow[16 * n + c16] = o[n][i] * inv;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t pi = ((size_t)b * a.Hq + h0 + 4 * g + i) * a.num_partitions + part;
      float* orow = a.ws_o + pi * kDv;
#pragma unroll
      for (int n = 0; n < kDv / 16; ++n) orow[16 * n + c16] = o[n][i];
      if (c16 == 0) {
        a.ws_m[pi] = mi[i];
        a.ws_l[pi] = li[i];
      }
    }
  }
}

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t s) {
  if (a.d_qk != kDqk || a.d_v != kDv || a.block_size != kBlock || a.Hq % kHeadsPerWave ||
      a.partition % kBlock)
    return hipErrorNotSupported;
  const int head_groups = (a.Hq + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int units = a.B * a.num_partitions;
  const int units8 = (units + 7) / 8 * 8;
  hipLaunchKernelGGL(mla_decode_kernel, dim3((unsigned)(units8 * head_groups)),
                     dim3(kWaves * kWave), 0, s, a, head_groups, units);
  return hipGetLastError();
}

}  // namespace pkv
