// Paged decode attention for GQA/MQA/MHA on gfx950, and the split-context merge.
//
// What is computed ("深入LLM推理：从KV Cache到PD分离的Serving全景解析", sections
// "KV Cache：Transformer的循环状态" and "PagedAttention与Cache管理"): for every sequence b
// and query head h, softmax(scale * q K^T) V over the sequence's cached tokens, whose K/V
// rows are found through the block table; the G = Hq/Hkv query heads of a group share one
// K/V head.  Long contexts are split into partitions and the partial online-softmax
// states merged afterwards ("GPU推理深度拆解：KV Cache视角", "长上下文优化" / "算子优化要点").
//
// Work decomposition: one workgroup of 4 waves per (KV head g, partition p, sequence b).
// The partition's 16-token tiles are dealt round-robin to the 4 waves.  Each wave streams
// its tiles' K and V straight from HBM into VGPRs with 16-byte loads, one tile ahead of
// the arithmetic; every K/V byte is read once and used for all G query heads.  A tile of
// one (block, KV head) is 16 contiguous rows of d elements (head-major block layout).
//
// Lane layouts inside a wave (d = 128 shown; d = 64 is analogous):
//  * q.K  : lane = (k = lane>>3, c = lane&7).  Pass pi in {0,1} covers token 8*pi + k; the
//           lane holds 16 of its dims (two 16-byte pieces, so each load instruction reads
//           8 full 128-byte lines).  Partial dot products for the G heads are reduced over
//           the 8 lanes of the token with a DPP reduce-scatter, leaving lane c with head c.
//  * p.V  : lane = (r = lane>>4, dc = lane&15).  Row r owns tokens {8*pi + 2r + e} and dims
//           8*dc..8*dc+7; its accumulators o[h][8] cover those tokens only (4 independent
//           row states, merged once at the end).  The tokens a row needs for p.V are the
//           ones its own lanes scored, so probabilities move by DPP row broadcasts.
//  * q.K runs on v_dot2_f32_bf16 over adjacent dims; p.V on v_dot2_f32_f16 over two tokens
//           (probabilities rounded to fp16, V rows widened bf16 -> fp16 and paired token by
//           token in registers).  FP8 E4M3 K is widened to bf16 pairs and V to fp16 pairs
//           (both exact); the per-head K scale folds into the score scale and the V scale
//           into the output.
//  * K/V are read through range-checked buffer resources whose range ends at the tile's
//           last valid token, so rows past a sequence's end are read as zeros (and carry
//           zero probability), whatever the pool holds there.
// Online softmax runs in the log2 domain with a lazy rescale: the running max only moves
// (rescaling o and l) when a new score exceeds it by more than 2^8, which keeps every
// probability <= 256 and skips almost all rescales after the first tile.
#include "gqa_tile.hpp"

namespace pkv {

template <int D, int G, bool FP8>
__global__ __launch_bounds__(kWaves * kWave, 2) void gqa_decode_kernel(DecodeArgs a) {
  using Lo = Layout<D, FP8>;
  const int g = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int k = lane >> 3, c = lane & 7, r = lane / Lo::LPT, dc = lane % Lo::LPT;
  const int t0 = part * a.partition;
  const int tiles_per_block = a.block_size / kTile;
  const int tile_begin = t0 / kTile;
  const size_t head_bytes = (size_t)a.block_size * Lo::ROW;
  const size_t block_bytes = head_bytes * a.Hkv;

  // Issued before the sequence length is known, so the three loads overlap: this wave's
  // block ids (one tile per lane, at most 64 tiles per wave; the table row is readable up
  // to max_blocks entries whatever the length), the length, and q.
  const int my_tile = tile_begin + w + kWaves * lane;
  const int nt_full = (a.partition / kTile - w + kWaves - 1) / kWaves;
  int phys = -1;
  if (lane < nt_full && my_tile / tiles_per_block < a.max_blocks)
    phys = a.block_table[(size_t)b * a.max_blocks + my_tile / tiles_per_block];
  int L = a.context_lens[b];

  WaveState<D, G, FP8> S;
  load_q_reset<D, G, FP8>(S, a.q + ((size_t)b * a.Hq + (size_t)g * G) * D, c);

  const int cap = min(a.max_blocks * a.block_size, a.max_context_len);
  L = L < 0 ? 0 : (L > cap ? cap : L);
  if (t0 >= L) {
    if (a.num_partitions == 1 && part == 0) {  // empty sequence: output 0
      for (int idx = threadIdx.x; idx < G * D; idx += kWaves * kWave)
        a.out[((size_t)b * a.Hq + (size_t)g * G) * D + idx] = 0.f;
    }
    return;
  }
  const int t1 = min(L, t0 + a.partition);
  const int tile_end = (t1 + kTile - 1) / kTile;
  const int nt = tile_end - tile_begin > w ? (tile_end - tile_begin - w + kWaves - 1) / kWaves : 0;

  // Byte offset (within a head's pool slice) and valid-token count of this wave's tiles,
  // one tile per lane.  A block id outside the pool is never dereferenced: its tile reads
  // block 0 and counts no valid token.
  uint32_t off_lo = 0, off_hi = 0;
  int nv_lane = 0;
  if (lane < nt) {
    const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
    const uint64_t off = (uint64_t)(ok ? phys : 0) * block_bytes +
                         (uint64_t)(my_tile % tiles_per_block) * (kTile * Lo::ROW);
    off_lo = (uint32_t)off;
    off_hi = (uint32_t)(off >> 32);
    nv_lane = ok ? min(kTile, t1 - my_tile * kTile) : 0;
  }
  const uint8_t* kbase = a.k_pool + (size_t)g * head_bytes;
  const uint8_t* vbase = a.v_pool + (size_t)g * head_bytes;
  const float cscale = a.scale * kLog2e * (FP8 ? a.k_scale[g] : 1.f);

  // Source of this wave's tile n, or an empty one (all loads return zeros) for n >= nt.
  auto tile_at = [&](int n, int& nv) -> TileSrc {
    if (n >= nt) {
      nv = 0;
      return tile_src<D, FP8>(kbase, vbase, 0);
    }
    const uint64_t off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_lo, n) |
                         ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_hi, n) << 32);
    nv = __builtin_amdgcn_readlane(nv_lane, n);
    return tile_src<D, FP8>(kbase + off, vbase + off, nv);
  };

  // Two tile buffers, refilled half by half: a tile's K is replaced by the tile two ahead
  // as soon as its scores are done, its V once p.V is done, so one and a half to two tiles
  // are always in flight.
  const uint32_t koff = k_lane_offset<D, FP8>(k, c), voff = v_lane_offset<D, FP8>(r, dc);
  TileRegs<D, FP8> RA, RB;
  int nvA, nvB;
  TileSrc A = tile_at(0, nvA), Bt = tile_at(1, nvB);
  // issued in this order (the scheduling fences keep it), so the loop's waits are counts of
  // the loads issued after the data it needs
  load_k<D, FP8>(RA, A.k, koff);
  sched_fence();
  load_v<D, FP8>(RA, A.v, voff);
  sched_fence();
  load_k<D, FP8>(RB, Bt.k, koff);
  sched_fence();
  load_v<D, FP8>(RB, Bt.v, voff);
  sched_fence();
  // Pairs of tiles, then a last single tile: no exit from the middle of the loop, so every
  // path around it issues the same loads and its waits stay exact.
  int n = 0;
  for (; n + 1 < nt; n += 2) {
    {
      uint32_t pairs[Lo::NPS];
      qk_softmax<D, G, FP8>(S, RA, nvA, cscale, lane, pairs);
      sched_fence();
      A = tile_at(n + 2, nvA);
      load_k<D, FP8>(RA, A.k, koff);
      sched_fence();
      pv_accumulate<D, G, FP8>(S, RA, lane, pairs);
      sched_fence();
      load_v<D, FP8>(RA, A.v, voff);
    }
    {
      uint32_t pairs[Lo::NPS];
      qk_softmax<D, G, FP8>(S, RB, nvB, cscale, lane, pairs);
      sched_fence();
      Bt = tile_at(n + 3, nvB);
      load_k<D, FP8>(RB, Bt.k, koff);
      sched_fence();
      pv_accumulate<D, G, FP8>(S, RB, lane, pairs);
      sched_fence();
      load_v<D, FP8>(RB, Bt.v, voff);
    }
  }
  if (n < nt) {
    uint32_t pairs[Lo::NPS];
    qk_softmax<D, G, FP8>(S, RA, nvA, cscale, lane, pairs);
    pv_accumulate<D, G, FP8>(S, RA, lane, pairs);
  }

  // ---- merge the wave's row groups: every lane ends with the wave's state for its dims
  GroupStats<G> X;
  wave_merge_rows<D, G, FP8>(X, S, lane);

  // ---- merge the 4 waves through LDS and write the output or the partition's partials
  __shared__ float s_o[kWaves][G][D];
  __shared__ float s_m[kWaves][G], s_l[kWaves][G];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *(float4*)&s_o[w][h][8 * dc] = make_float4(S.o[h][0], S.o[h][1], S.o[h][2], S.o[h][3]);
      *(float4*)&s_o[w][h][8 * dc + 4] = make_float4(S.o[h][4], S.o[h][5], S.o[h][6], S.o[h][7]);
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_m[w][h] = X.m[h];
        s_l[w][h] = X.l[h];
      }
    }
  }
  __syncthreads();
  const float vs = FP8 ? a.v_scale[g] : 1.f;
  for (int idx = threadIdx.x; idx < G * D; idx += kWaves * kWave) {
    const int h = idx / D, dd = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = s_m[ww][h];
      const float f = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      lsum += f * s_l[ww][h];
      osum += f * s_o[ww][h][dd];
    }
    const size_t hq = (size_t)g * G + h;
    if (a.num_partitions == 1) {
      a.out[((size_t)b * a.Hq + hq) * D + dd] = lsum > 0.f ? osum * vs / lsum : 0.f;
    } else {
      const size_t pi = ((size_t)b * a.Hq + hq) * a.num_partitions + part;
      a.ws_o[pi * D + dd] = osum * vs;
      if (dd == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = lsum;
      }
    }
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
  return x;
}

// out[b][h] = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p over the sequence's partitions.
// One wave per (sequence, head): the partitions' statistics are loaded one per lane, then
// the partial outputs are streamed several rows per load (rows_accumulate).
template <int D>
__global__ __launch_bounds__(kWave) void partition_merge_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, const int32_t* __restrict__ context_lens,
    float* __restrict__ out, int Hq, int partition, int P, int max_ctx_clamp) {
  constexpr int PER = D / kWave;
  const int bh = blockIdx.x, b = bh / Hq, lane = threadIdx.x;
  int L = context_lens[b];
  L = L < 0 ? 0 : (L > max_ctx_clamp ? max_ctx_clamp : L);
  const int nP = min(P, (L + partition - 1) / partition);
  float* o = out + (size_t)bh * D;
  if (nP == 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) o[lane + kWave * i] = 0.f;
    return;
  }
  const size_t base = (size_t)bh * P;
  float M = kNegInf;
  for (int p0 = 0; p0 < nP; p0 += kWave)
    if (p0 + lane < nP) M = fmaxf(M, ws_m[base + p0 + lane]);
  M = wave_max(M);
  RowAcc<D> acc;
  rows_clear(acc);
  float den = 0.f;
  for (int p0 = 0; p0 < nP; p0 += kWave) {
    float f = 0.f, lp = 0.f;
    if (p0 + lane < nP) {
      const float mp = ws_m[base + p0 + lane];
      lp = ws_l[base + p0 + lane];
      f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
    }
    den += wave_sum(f * lp);
    rows_accumulate<D>(acc, ws_o + (base + p0) * D, D, f, min(kWave, nP - p0), lane);
  }
  rows_store<D>(acc, o, den > 0.f ? 1.f / den : 0.f, lane);
}

template <int D, int G, bool FP8>
static hipError_t launch_one(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.Hkv, a.num_partitions, a.B);
  hipLaunchKernelGGL((gqa_decode_kernel<D, G, FP8>), grid, dim3(kWaves * kWave), 0, s, a);
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_one<D, 1, FP8>(a, s);
    case 2: return launch_one<D, 2, FP8>(a, s);
    case 4: return launch_one<D, 4, FP8>(a, s);
    case 8: return launch_one<D, 8, FP8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gqa_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.d == 128) return a.fp8 ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
  if (a.d == 64 && !a.fp8) return launch_d<64, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_partition_merge(const float* ws_m, const float* ws_l, const float* ws_o,
                                  const int32_t* context_lens, float* out, int32_t B,
                                  int32_t Hq, int32_t d, int32_t partition,
                                  int32_t num_partitions, int32_t max_context_len,
                                  int32_t max_ctx_clamp, hipStream_t s) {
  (void)max_context_len;
  dim3 grid((unsigned)B * Hq);
  if (d == 128)
    hipLaunchKernelGGL(partition_merge_kernel<128>, grid, dim3(kWave), 0, s, ws_m, ws_l, ws_o,
                       context_lens, out, Hq, partition, num_partitions, max_ctx_clamp);
  else if (d == 64)
    hipLaunchKernelGGL(partition_merge_kernel<64>, grid, dim3(kWave), 0, s, ws_m, ws_l, ws_o,
                       context_lens, out, Hq, partition, num_partitions, max_ctx_clamp);
  else if (d == 512)
    hipLaunchKernelGGL(partition_merge_kernel<512>, grid, dim3(kWave), 0, s, ws_m, ws_l, ws_o,
                       context_lens, out, Hq, partition, num_partitions, max_ctx_clamp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
