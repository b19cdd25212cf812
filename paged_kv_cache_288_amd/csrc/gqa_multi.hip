// Multi-token paged decode attention (the verify step of speculative decoding) on gfx950.
//
// "深入LLM推理：从KV Cache到PD分离的Serving全景解析", section "投机解码：打破每步一token的假设":
// the target model checks several drafted tokens in one pass, which is nearly free because
// the step is bound by reading memory.  Here each sequence brings q_len new query tokens
// whose K/V rows are already in the cache (counted by context_lens); query token j of a
// sequence of length L sees its first L - q_len + 1 + j tokens (causal among the new ones):
//     out[b][j][h] = softmax_t<L-q_len+1+j (scale * q[b][j][h] . K_t) V_t.
//
// All q_len * G query rows of a (sequence, KV head) pair share every K/V tile, so per byte
// read the step does q_len times the arithmetic of a single-token decode (32 flop/byte at
// G = 8, q_len = 4): past what the VALU sustains at HBM speed, and a dense contraction, so
// both products run on the MFMA:
//  * scores S^T[16 tokens x 16 rows] = K Q^T on v_mfma_f32_16x16x32_bf16 (D / 32 steps), K
//    as the A operand straight from the 16-byte loads (lane l: token l % 16, 8 dims of a
//    32-dim step chosen by l / 16), Q^T as the B operand held in registers for a piece;
//  * the result gives lane l four tokens (4 (l / 16) + i) of query row l % 16, which is
//    exactly the B operand layout of v_mfma_f32_16x16x16_f16, so the probabilities feed
//    O^T[16 dims x 16 rows] += V^T P^T without moving across lanes, and each lane's output
//    values and online-softmax state belong to its own row (rescales stay lane-local);
//  * V^T (A operand: lane l holds dim l % 16 of 4 tokens) comes from LDS: each wave writes
//    its V tile there token-major and reads it back with ds_read_b64_tr_b16, which
//    transposes 4x4 blocks of 16-bit values across lanes; 32-byte pieces are XOR-swizzled
//    per row so that the eight rows one half-wave reads lie in eight different bank groups.
// Probabilities and V run through the fp16 MFMA (fp32 accumulate), as in the single-token
// kernels: p <= 2^8 after the lazy max, V widened from bf16 exactly for 2^-14 <= |v| <
// 65504.
//
// Division of work is the balanced mode of gqa_stream.hip: the 16-token tiles of all
// (KV head, sequence) segments laid end to end, cut into equal ranges, one per wave; each
// range yields one (m, l, o) piece per segment it meets, and multi_merge_kernel combines
// the pieces of each segment.
#include "gqa_multi_body.hpp"

namespace pkv {

template <int D, int RT, bool FP8>
__global__ __launch_bounds__(kMW * kWave, multi_waves_per_simd(D, RT)) void gqa_multi_kernel(MultiArgs a) {
  __shared__ int s_pre[kMultiSeqs + 1];
  __shared__ int s_sum[kMW * kWave];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kMW * MLayout<D, FP8>::LTILE];
  gqa_multi_body<D, RT, FP8>(a, blockIdx.x, s_pre, s_sum, s_v);
}

// out[b][j][hq] = merge of the pieces of segment (g = hq / G, b), row j * G + hq % G.
// One wave per output row, kMergeWaves per workgroup.
constexpr int kMultiMergeWaves = 4;
template <int D>
__global__ __launch_bounds__(kMultiMergeWaves * kWave) void multi_merge_kernel(MultiArgs a) {
  constexpr int PER = D / kWave;
  const int G = a.Hq / a.Hkv, R = G * a.q_len;
  const int idx = blockIdx.x * kMultiMergeWaves + (int)(threadIdx.x / kWave);
  if (idx >= a.B * a.q_len * a.Hq) return;
  const int b = idx / (a.q_len * a.Hq), rem = idx - b * (a.q_len * a.Hq);
  const int jq = rem / a.Hq, hq = rem - jq * a.Hq, g = hq / G, row = jq * G + (hq - g * G);
  const int lane = threadIdx.x & (kWave - 1);
  float* out = a.out + (size_t)idx * D;
  const int c0 = a.ws_seg[2 * (g * a.B + b)], np = a.ws_seg[2 * (g * a.B + b) + 1];
  const int T_head = a.ws_prefix[a.B];
  if (np == 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) out[lane + kWave * i] = 0.f;
    return;
  }
  const long long T = (long long)a.Hkv * T_head;
  const size_t slot0 = (size_t)c0 + (size_t)g * a.B + b;  // slot of piece i: slot0 + i
  // with fewer tiles than chunks some chunks are empty and wrote nothing
  const bool all_live = T >= a.chunks;
  auto live = [&](int i) {
    if (all_live) return true;
    const long long cc = c0 + i;
    return T * cc / a.chunks != T * (cc + 1) / a.chunks;
  };
  float M = kNegInf;
  for (int p0 = 0; p0 < np; p0 += kWave)
    if (p0 + lane < np && live(p0 + lane)) M = fmaxf(M, a.ws_m[(slot0 + p0 + lane) * R + row]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
  RowAcc<D> acc;
  rows_clear(acc);
  float den = 0.f;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    float f = 0.f, lp = 0.f;
    if (p0 + lane < np && live(p0 + lane)) {
      const size_t si = (slot0 + p0 + lane) * R + row;
      const float mp = a.ws_m[si];
      lp = a.ws_l[si];
      f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
    }
    float fl = f * lp;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) fl += __shfl_xor(fl, s);
    den += fl;
    rows_accumulate<D>(acc, a.ws_o + ((slot0 + p0) * R + row) * D, (size_t)R * D, f,
                       min(kWave, np - p0), lane);
  }
  rows_store<D>(acc, out, den > 0.f ? 1.f / den : 0.f, lane);
}

template <int D, int RT, bool FP8>
static hipError_t launch_multi_one(const MultiArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gqa_multi_kernel<D, RT, FP8>), dim3(a.chunks / kMW), dim3(kMW * kWave), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(((long long)a.B * a.q_len * a.Hq + kMultiMergeWaves - 1) / kMultiMergeWaves));
  hipLaunchKernelGGL(multi_merge_kernel<D>, grid, dim3(kMultiMergeWaves * kWave), 0, s, a);
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_multi_d(const MultiArgs& a, hipStream_t s) {
  const int R = a.Hq / a.Hkv * a.q_len;
  if (R <= 16) return launch_multi_one<D, 1, FP8>(a, s);
  if (R <= 32) return launch_multi_one<D, 2, FP8>(a, s);
  if (R <= 64) return launch_multi_one<D, 4, FP8>(a, s);
  return hipErrorInvalidValue;
}

int multi_waves_per_cu(int d, int rows) {
  const int rt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  if (d == 128) return kMW * multi_waves_per_simd(128, rt);
  return kMW * multi_waves_per_simd(64, rt);
}

hipError_t launch_gqa_multi(const MultiArgs& a, hipStream_t s) {
  if (a.B > kMultiSeqs || a.chunks % 32 || a.block_size % kTile) return hipErrorInvalidValue;
  if (a.d == 128) return a.fp8 ? launch_multi_d<128, true>(a, s) : launch_multi_d<128, false>(a, s);
  if (a.d == 64) return a.fp8 ? launch_multi_d<64, true>(a, s) : launch_multi_d<64, false>(a, s);
  return hipErrorInvalidValue;
}




}  // namespace pkv
