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
//
// Two kernels do this.  For bf16 K/V of 128 dims and up to 32 rows, gqa_multi_ring_kernel
// streams K, V and q through an LDS ring (gqa_multi_ring_body.hpp), one wave per SIMD;
// otherwise (FP8, 64 dims, 64 rows, the cascade's prefix role) gqa_multi_kernel holds its
// tiles in registers, two waves per SIMD (gqa_multi_body.hpp).
#include "gqa_multi_ring_body.hpp"

namespace pkv {

template <int RT>
__global__ __launch_bounds__(kRingWaves * kWave, 1) void gqa_multi_ring_kernel(MultiArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[multi_ring_lds_bytes<RT>()];
  gqa_multi_ring_body<RT>(a, blockIdx.x, (lds_u8_t*)s_lds);
}

// The ring kernel serves bf16 K/V, d = 128, up to 32 rows, every q row its own (not the
// cascade's prefix mode).
bool multi_uses_ring(int d, int rows, bool fp8) { return d == 128 && rows <= 32 && !fp8; }
int multi_ring_waves_per_cu() { return kRingWaves; }

template <int D, int RT, bool FP8>
__global__ __launch_bounds__(kMW * kWave, multi_waves_per_simd(D, RT)) void gqa_multi_kernel(MultiArgs a) {
  __shared__ int s_pre[kMultiSeqs + 1];
  __shared__ int s_sum[kMW * kWave];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kMW * MLayout<D, FP8>::LTILE];
  gqa_multi_body<D, RT, FP8>(a, blockIdx.x, s_pre, s_sum, s_v);
}

// out[b][j][g*G .. g*G + G) = merge of the pieces of segment (g, b), rows j*G .. j*G + G.
// One wave per (sequence, query token, KV head): the G rows are contiguous both in every
// piece slot and in the output, so each piece is one G*D-float run read by the whole wave
// (float4 per lane), and the output one run written by it.  Piece weights: lane q*G + h
// holds piece p0 + q, row h, for 64/G pieces per pass.  Segments of up to kMultiFastPieces
// pieces (the usual case: a few chunks per segment) are merged in one round trip: every
// piece's m, l and run requested at once, the weights formed afterwards.
constexpr int kMultiMergeWaves = 4;
constexpr int kMultiFastPieces = 4;
template <int D, int G>
__global__ __launch_bounds__(kMultiMergeWaves * kWave) void multi_merge_kernel(MultiArgs a) {
  constexpr int RUN = G * D;                      // floats per piece run
  constexpr int NF4 = RUN >= 4 * kWave ? RUN / (4 * kWave) : 1;  // float4 per lane per run
  constexpr int ACTIVE = RUN >= 4 * kWave ? kWave : RUN / 4;     // lanes holding data
  constexpr int PP = kWave / G;                   // pieces per weight pass
  constexpr int U = PP < 8 ? PP : 8;              // pieces whose loads are in flight together
  const int R = G * a.q_len;
  const int wv = blockIdx.x * kMultiMergeWaves + (int)(threadIdx.x / kWave);
  if (wv >= a.B * a.q_len * a.Hkv) return;
  const int g = wv % a.Hkv, bj = wv / a.Hkv, b = bj / a.q_len, jq = bj - b * a.q_len;
  const int lane = threadIdx.x & (kWave - 1);
  const int hw = lane % G, qw = lane / G;         // weight lane: row hw of piece p0 + qw
  float* out = a.out + ((size_t)bj * a.Hq + (size_t)g * G) * D;
  const int c0 = a.ws_seg[2 * (g * a.B + b)], np = a.ws_seg[2 * (g * a.B + b) + 1];
  if (np == 0) {
    if (lane < ACTIVE)
#pragma unroll
      for (int k = 0; k < NF4; ++k)
        *(float4*)(out + 4 * (lane + kWave * k)) = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const long long T = (long long)a.Hkv * a.ws_prefix[a.B];
  const size_t slot0 = (size_t)c0 + (size_t)g * a.B + b;  // slot of piece i: slot0 + i
  const size_t row0 = (size_t)jq * G;
  // with fewer tiles than chunks some chunks are empty and wrote nothing
  const bool all_live = T >= a.chunks;
  auto live = [&](int i) {
    if (all_live) return true;
    const long long cc = c0 + i;
    return T * cc / a.chunks != T * (cc + 1) / a.chunks;
  };
  // reduce over the lanes of one row (lane bits above log2 G)
  auto row_max = [](float x) {
#pragma unroll
    for (int s = G; s < kWave; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
    return x;
  };
  auto row_sum = [](float x) {
#pragma unroll
    for (int s = G; s < kWave; s <<= 1) x += __shfl_xor(x, s);
    return x;
  };
  constexpr int NPF = kMultiFastPieces < PP ? kMultiFastPieces : PP;
  if (np <= NPF) {
    float mp = kNegInf, lp = 0.f;
    if (qw < np && live(qw)) {
      const size_t si = (slot0 + qw) * R + row0 + hw;
      mp = a.ws_m[si];
      lp = a.ws_l[si];
    }
    float4 x[NPF][NF4];
#pragma unroll
    for (int q = 0; q < NPF; ++q) {
      const float* run = a.ws_o + ((slot0 + (q < np ? q : 0)) * R + row0) * D;
#pragma unroll
      for (int k = 0; k < NF4; ++k)
        x[q][k] = (lane < ACTIVE && q < np) ? *(const float4*)(run + 4 * (lane + kWave * k))
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float M = row_max(mp);
    const float f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
    const float den = row_sum(f * lp);
    float4 acc[NF4];
    float sc[NF4];
#pragma unroll
    for (int k = 0; k < NF4; ++k) {
      const int hk = (4 * (lane + kWave * k) / D) % G;  // the row this float4 belongs to
      acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int q = 0; q < NPF; ++q) {
        const float fq = __shfl(f, q * G + hk);
        if (fq != 0.f) {  // runs of pieces without weight (never written) are not used
          acc[k].x += fq * x[q][k].x;
          acc[k].y += fq * x[q][k].y;
          acc[k].z += fq * x[q][k].z;
          acc[k].w += fq * x[q][k].w;
        }
      }
      const float d = __shfl(den, hk);
      sc[k] = d > 0.f ? 1.f / d : 0.f;
    }
    if (lane < ACTIVE) {
#pragma unroll
      for (int k = 0; k < NF4; ++k)
        *(float4*)(out + 4 * (lane + kWave * k)) =
            make_float4(acc[k].x * sc[k], acc[k].y * sc[k], acc[k].z * sc[k], acc[k].w * sc[k]);
    }
    return;
  }
  float M = kNegInf;
  for (int p0 = 0; p0 < np; p0 += PP)
    if (p0 + qw < np && live(p0 + qw)) M = fmaxf(M, a.ws_m[(slot0 + p0 + qw) * R + row0 + hw]);
  M = row_max(M);

  // data lanes: float4 k of a run covers row (4 lane + 4 kWave k) / D
  float4 acc[NF4];
#pragma unroll
  for (int k = 0; k < NF4; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  for (int p0 = 0; p0 < np; p0 += PP) {
    float f = 0.f, lp = 0.f;
    if (p0 + qw < np && live(p0 + qw)) {
      const size_t si = (slot0 + p0 + qw) * R + row0 + hw;
      const float mp = a.ws_m[si];
      lp = a.ws_l[si];
      f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
    }
    den += row_sum(f * lp);
    const int cnt = min(PP, np - p0);
    // U pieces' loads issued together, then their products
    for (int q0 = 0; q0 < cnt; q0 += U) {
      float fk[U][NF4];
      float4 x[U][NF4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u;
        const float* run = a.ws_o + ((slot0 + p0 + (q < cnt ? q : 0)) * R + row0) * D;
#pragma unroll
        for (int k = 0; k < NF4; ++k) {
          const int e = 4 * (lane + kWave * k);
          fk[u][k] = __shfl(f, (q < cnt ? q : 0) * G + (e / D) % G);
          if (q >= cnt) fk[u][k] = 0.f;
          x[u][k] = (lane < ACTIVE && fk[u][k] != 0.f) ? *(const float4*)(run + e)
                                                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < NF4; ++k) {
          acc[k].x += fk[u][k] * x[u][k].x;
          acc[k].y += fk[u][k] * x[u][k].y;
          acc[k].z += fk[u][k] * x[u][k].z;
          acc[k].w += fk[u][k] * x[u][k].w;
        }
    }
  }
  // the row sums, from the lanes that hold them, in every lane (all lanes shuffle)
  float sc[NF4];
#pragma unroll
  for (int k = 0; k < NF4; ++k) {
    const float d = __shfl(den, (4 * (lane + kWave * k) / D) % G);
    sc[k] = d > 0.f ? 1.f / d : 0.f;
  }
  if (lane < ACTIVE) {
#pragma unroll
    for (int k = 0; k < NF4; ++k)
      *(float4*)(out + 4 * (lane + kWave * k)) =
          make_float4(acc[k].x * sc[k], acc[k].y * sc[k], acc[k].z * sc[k], acc[k].w * sc[k]);
  }
}

// The decode kernel alone: the LDS ring on MFMA for bf16 with d = 128 and up to 32 rows,
// else the register-tile kernel.
template <int D, int RT, bool FP8>
static hipError_t launch_multi_decode(const MultiArgs& a, hipStream_t s) {
  const int R = a.Hq / a.Hkv * a.q_len;
  if (multi_uses_ring(D, R, FP8)) {  // chunks were sized for it (up to 480 tiles each)
    if constexpr (D == 128 && RT <= 2 && !FP8) {
      // chunk = (XCD eighth) + (workgroup within it) * 4 + wave: whole workgroups per eighth
      if (a.chunks % (8 * kRingWaves) || a.B > kRingMaxSeqs || a.q_rows != a.B * a.q_len ||
          a.fixed_len >= 0)
        return hipErrorInvalidValue;
      hipLaunchKernelGGL((gqa_multi_ring_kernel<RT>), dim3(a.chunks / kRingWaves),
                         dim3(kRingWaves * kWave), 0, s, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL((gqa_multi_kernel<D, RT, FP8>), dim3(a.chunks / kMW), dim3(kMW * kWave), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int RT, bool FP8>
static hipError_t launch_multi_one(const MultiArgs& a, hipStream_t s, bool merge) {
  hipError_t e = launch_multi_decode<D, RT, FP8>(a, s);
  if (e != hipSuccess || !merge) return e;
  const dim3 grid((unsigned)(((long long)a.B * a.q_len * a.Hkv + kMultiMergeWaves - 1) / kMultiMergeWaves));
  const dim3 block(kMultiMergeWaves * kWave);
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((multi_merge_kernel<D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((multi_merge_kernel<D, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((multi_merge_kernel<D, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((multi_merge_kernel<D, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_multi_d(const MultiArgs& a, hipStream_t s, bool merge) {
  const int R = a.Hq / a.Hkv * a.q_len;
  if (R <= 16) return launch_multi_one<D, 1, FP8>(a, s, merge);
  if (R <= 32) return launch_multi_one<D, 2, FP8>(a, s, merge);
  if (R <= 64) return launch_multi_one<D, 4, FP8>(a, s, merge);
  return hipErrorInvalidValue;
}

static hipError_t launch_multi_impl(const MultiArgs& a, hipStream_t s, bool merge) {
  if (a.B > kMultiSeqs || a.chunks % 32 || a.block_size % kTile) return hipErrorInvalidValue;
  if (a.d == 128)
    return a.fp8 ? launch_multi_d<128, true>(a, s, merge) : launch_multi_d<128, false>(a, s, merge);
  if (a.d == 64)
    return a.fp8 ? launch_multi_d<64, true>(a, s, merge) : launch_multi_d<64, false>(a, s, merge);
  return hipErrorInvalidValue;
}

int multi_waves_per_cu(int d, int rows) {
  const int rt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  if (d == 128) return kMW * multi_waves_per_simd(128, rt);
  return kMW * multi_waves_per_simd(64, rt);
}

hipError_t launch_gqa_multi_pieces(const MultiArgs& a, hipStream_t s) {
  return launch_multi_impl(a, s, false);
}

hipError_t launch_gqa_multi(const MultiArgs& a, hipStream_t s) {
  return launch_multi_impl(a, s, true);
}

}  // namespace pkv
