// Balanced paged decode attention for GQA/MQA/MHA on gfx950 (the library's default mode).
//
// Same arithmetic as gqa_decode.hip (scores, online softmax and p.V per 16-token tile, see
// gqa_tile.hpp), different division of work.  The cached tiles of all (KV head, sequence)
// pairs are laid end to end - head-major, then sequence, then tile - and the resulting
// flattened space is cut into `chunks` equal contiguous ranges, one per wave.  A wave walks
// its range tile by tile with the same two-buffer prefetch; wherever its range meets a
// (head, sequence) segment it produces one piece: the (m, l, o) online-softmax state of
// those tiles for the G query heads of the group, written to slot `chunk + g*B + b` (slots
// grow strictly along the flattened space, so they are unique).  The merge kernel then
// combines the pieces of each segment (the online-softmax combine of "GPU推理深度拆解：KV
// Cache视角", sections "长上下文优化" / "算子优化要点").
//
// Compared with fixed partitions this keeps every wave streaming for the whole kernel with
// the same amount of work (+-1 tile), without per-partition start-up, barriers or a ragged
// last round.  Chunks are numbered so that each XCD (workgroups go to the 8 XCDs in turn, so
// those with equal ids mod 8 share one) gets a contiguous eighth of the space - one KV head
// when Hkv = 8 - so a shared prefix's re-reads stay in that XCD's L2.
#include "gqa_ring_body.hpp"
#include "gqa_stream_body.hpp"

namespace pkv {

template <int D, int G, bool FP8>
__global__ __launch_bounds__(kWaves * kWave, 2) void gqa_stream_kernel(DecodeArgs a) {
  __shared__ int s_pre[kMaxStreamSeqs + 1];
  __shared__ int s_sum[kWaves * kWave];
  gqa_stream_body<D, G, FP8>(a, blockIdx.x, s_pre, s_sum);
}

// out[b][h] = sum over the pieces of segment (g = h / G, b) of 2^(m - M) o / 2^(m - M) l.
// One wave per (sequence, query head), kMergeWaves of them per workgroup.
constexpr int kMergeWaves = 4;
constexpr int kFastPieces = 16;  // pieces per segment merged in a single round trip
constexpr int kFastLatentPieces = 8;  // the same for the latent (512-dim) rows
template <int D>
__global__ __launch_bounds__(kMergeWaves * kWave) void stream_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / kWave;
  const int G = a.Hq / a.Hkv;
  const int bh = blockIdx.x * kMergeWaves + (int)(threadIdx.x / kWave);
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq, hq = bh - b * a.Hq, g = hq / G, h = hq - g * G;
  const int lane = threadIdx.x & (kWave - 1);
  float* out = a.out + (size_t)bh * D;
  const int c0 = a.ws_seg[2 * (g * a.B + b)], np = a.ws_seg[2 * (g * a.B + b) + 1];
  const int T_head = a.ws_prefix[a.B];
  if (np == 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) out[lane + kWave * i] = 0.f;
    return;
  }
  const long long T = (long long)a.Hkv * T_head;
  const size_t slot0 = (size_t)c0 + (size_t)g * a.B + b;  // slot of piece i: slot0 + i
  // Chunks c0 .. c0 + np - 1 cover the segment.  With fewer tiles than chunks some of them
  // are empty and wrote nothing: those carry no weight and are never read.
  const bool all_live = T >= a.chunks;
  auto live = [&](int i) {
    if (all_live) return true;
    const long long cc = c0 + i;
    return T * cc / a.chunks != T * (cc + 1) / a.chunks;
  };
  if constexpr (D == 512) {
    // Latent rows (2 KiB) of up to kFastLatentPieces pieces: every piece's m, l and row
    // requested at once, as below; rows of pieces without weight are loaded but not used.
    constexpr int NP = kFastLatentPieces, V4 = D / 4 / kWave;
    if (np <= NP) {
      float mp = kNegInf, lp = 0.f;
      if (lane < np && live(lane)) {
        mp = a.ws_m[(slot0 + lane) * G + h];
        lp = a.ws_l[(slot0 + lane) * G + h];
      }
      float4 x[NP][V4];
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const float* row = a.ws_o + ((slot0 + (u < np ? u : 0)) * G + h) * D;
#pragma unroll
        for (int i = 0; i < V4; ++i)
          x[u][i] = u < np ? *(const float4*)(row + 4 * (lane + kWave * i))
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float M = mp;
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
      const float f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
      float den = f * lp;
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) den += __shfl_xor(den, s);
      float4 acc[V4];
#pragma unroll
      for (int i = 0; i < V4; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const float fu = __shfl(f, u);
        if (fu != 0.f) {
#pragma unroll
          for (int i = 0; i < V4; ++i) {
            acc[i].x += fu * x[u][i].x;
            acc[i].y += fu * x[u][i].y;
            acc[i].z += fu * x[u][i].z;
            acc[i].w += fu * x[u][i].w;
          }
        }
      }
      const float sc = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
      for (int i = 0; i < V4; ++i)
        *(float4*)(out + 4 * (lane + kWave * i)) =
            make_float4(acc[i].x * sc, acc[i].y * sc, acc[i].z * sc, acc[i].w * sc);
      return;
    }
  }
  if constexpr (D <= 128) {
    // Up to kFastPieces pieces: every piece's m, l and o row requested at once (one round
    // trip), the weights formed afterwards; rows of pieces that carry no weight (empty
    // chunks: never written) are loaded but not used.
    constexpr int LPR = D / 4, RPW = kWave / LPR, U = kFastPieces / RPW;
    if (np <= kFastPieces) {
      const int sub = lane / LPR, col = lane % LPR;
      float mp = kNegInf, lp = 0.f;
      if (lane < np && live(lane)) {
        mp = a.ws_m[(slot0 + lane) * G + h];
        lp = a.ws_l[(slot0 + lane) * G + h];
      }
      float4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = u * RPW + sub;
        x[u] = j < np ? *(const float4*)(a.ws_o + ((slot0 + j) * G + h) * D + 4 * col)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float M = mp;
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
      const float f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
      float den = f * lp;
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) den += __shfl_xor(den, s);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float fj = __shfl(f, u * RPW + sub);
        if (fj != 0.f) {
          acc.x += fj * x[u].x;
          acc.y += fj * x[u].y;
          acc.z += fj * x[u].z;
          acc.w += fj * x[u].w;
        }
      }
#pragma unroll
      for (int m = LPR; m < kWave; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m);
        acc.y += __shfl_xor(acc.y, m);
        acc.z += __shfl_xor(acc.z, m);
        acc.w += __shfl_xor(acc.w, m);
      }
      const float sc = den > 0.f ? 1.f / den : 0.f;
      if (lane < LPR)
        *(float4*)(out + 4 * lane) = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
      return;
    }
  }
  float M = kNegInf;
  for (int p0 = 0; p0 < np; p0 += kWave)
    if (p0 + lane < np && live(p0 + lane)) M = fmaxf(M, a.ws_m[(slot0 + p0 + lane) * G + h]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
  RowAcc<D> acc;
  rows_clear(acc);
  float den = 0.f;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    float f = 0.f, lp = 0.f;
    if (p0 + lane < np && live(p0 + lane)) {
      const size_t si = (slot0 + p0 + lane) * G + h;
      const float mp = a.ws_m[si];
      lp = a.ws_l[si];
      f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
    }
    float fl = f * lp;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) fl += __shfl_xor(fl, s);
    den += fl;
    // zero weights (empty chunks, pieces without a valid token) are skipped
    rows_accumulate<D>(acc, a.ws_o + ((slot0 + p0) * G + h) * D, (size_t)G * D, f,
                       min(kWave, np - p0), lane);
  }
  rows_store<D>(acc, out, den > 0.f ? 1.f / den : 0.f, lane);
}

// The library's default single-token decode: one workgroup per CU, each wave streaming its
// chunk through an LDS ring (gqa_ring_body.hpp) of 2 tiles (3 measured 0.7 % slower on
// the 70B-shaped batch, 4 no faster).  With 8 query heads per KV head a tile's arithmetic
// keeps one wave busy while its next tile is in flight: 4 waves (one per SIMD), up to 512
// registers each.  Smaller groups have lighter tiles, whose arithmetic a single wave cannot
// hide when their data comes from L2 (a shared prefix re-read): there two waves per SIMD
// hide each other's arithmetic.
template <int D, int G, bool FP8>
struct RingShape {
  static constexpr int WPG = G == 8 ? 4 : 8;
  static constexpr int NS = 2;
};
int ring_waves_per_cu(int d, int G, bool fp8) {
  (void)d;
  (void)fp8;
  return G == 8 ? 4 : 8;
}

template <int D, int G, bool FP8>
__global__ __launch_bounds__((RingShape<D, G, FP8>::WPG * kWave), 1) void gqa_ring_kernel(DecodeArgs a) {
  using RS = RingShape<D, G, FP8>;
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[ring_lds_bytes<D, G, FP8, RS::NS, RS::WPG>()];
  gqa_ring_body<D, G, FP8, RS::NS, RS::WPG>(a, blockIdx.x, (lds_u8_t*)s_lds);
}

template <int D, int G, bool FP8>
static hipError_t launch_stream_one(const DecodeArgs& a, hipStream_t s, bool merge) {
  if (merge) {
    constexpr int WPG = RingShape<D, G, FP8>::WPG;
    // chunk = (XCD eighth) + (workgroup within it) * WPG + wave: whole workgroups per eighth
    if (a.chunks % (8 * WPG) || a.B > kRingMaxSeqs) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gqa_ring_kernel<D, G, FP8>), dim3(a.chunks / WPG), dim3(WPG * kWave), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL((gqa_stream_kernel<D, G, FP8>), dim3(a.chunks / kWaves),
                       dim3(kWaves * kWave), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !merge) return e;
  return launch_stream_merge(a, s);
}

template <int D, bool FP8>
static hipError_t launch_stream_d(const DecodeArgs& a, hipStream_t s, bool merge) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_stream_one<D, 1, FP8>(a, s, merge);
    case 2: return launch_stream_one<D, 2, FP8>(a, s, merge);
    case 4: return launch_stream_one<D, 4, FP8>(a, s, merge);
    case 8: return launch_stream_one<D, 8, FP8>(a, s, merge);
    default: return hipErrorInvalidValue;
  }
}

// The same merge for segments of many pieces (a few long contexts): one workgroup per
// output row, its four waves each taking a contiguous quarter of the pieces.  Spreads the
// latency-bound chain of loads over four waves when there are too few rows to fill the GPU.
// Up to kFastPieces pieces per wave: each wave requests its pieces' m, l and rows at once
// and weighs them against its own maximum; the four (maximum, sum of weights, weighted row)
// triples are then rescaled to the common maximum through LDS.  More pieces: the quarter
// maxima first, then the weighted sums.
template <int D>
__global__ __launch_bounds__(kMergeWaves * kWave) void stream_merge_long_kernel(DecodeArgs a) {
  constexpr int PER = D / kWave;
  __shared__ float s_m[kMergeWaves], s_den[kMergeWaves];
  __shared__ __attribute__((aligned(16))) float s_acc[kMergeWaves][D];
  const int G = a.Hq / a.Hkv;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, hq = bh - b * a.Hq, g = hq / G, h = hq - g * G;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  float* out = a.out + (size_t)bh * D;
  const int c0 = a.ws_seg[2 * (g * a.B + b)], np = a.ws_seg[2 * (g * a.B + b) + 1];
  if (np == 0) {  // workgroup-uniform
    if (w == 0)
#pragma unroll
      for (int i = 0; i < PER; ++i) out[lane + kWave * i] = 0.f;
    return;
  }
  const long long T = (long long)a.Hkv * a.ws_prefix[a.B];
  const size_t slot0 = (size_t)c0 + (size_t)g * a.B + b;
  const bool all_live = T >= a.chunks;
  auto live = [&](int i) {
    if (all_live) return true;
    const long long cc = c0 + i;
    return T * cc / a.chunks != T * (cc + 1) / a.chunks;
  };
  const int lo = (int)((long long)np * w / kMergeWaves), hi = (int)((long long)np * (w + 1) / kMergeWaves);
  if constexpr (D <= 128) {
    constexpr int LPR = D / 4, RPW = kWave / LPR, U = kFastPieces / RPW;
    if (np <= kMergeWaves * kFastPieces) {  // workgroup-uniform; hi - lo <= kFastPieces
      const int n = hi - lo, sub = lane / LPR, col = lane % LPR;
      float mp = kNegInf, lp = 0.f;
      if (lane < n && live(lo + lane)) {
        mp = a.ws_m[(slot0 + lo + lane) * G + h];
        lp = a.ws_l[(slot0 + lo + lane) * G + h];
      }
      float4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = u * RPW + sub;
        x[u] = j < n ? *(const float4*)(a.ws_o + ((slot0 + lo + j) * G + h) * D + 4 * col)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float Mw = mp;
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) Mw = fmaxf(Mw, __shfl_xor(Mw, s));
      const float f = (mp == kNegInf) ? 0.f : fast_exp2(mp - Mw);
      float den = f * lp;
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) den += __shfl_xor(den, s);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float fj = __shfl(f, u * RPW + sub);
        if (fj != 0.f) {  // rows of pieces without weight (never written) are not used
          acc.x += fj * x[u].x;
          acc.y += fj * x[u].y;
          acc.z += fj * x[u].z;
          acc.w += fj * x[u].w;
        }
      }
#pragma unroll
      for (int m = LPR; m < kWave; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m);
        acc.y += __shfl_xor(acc.y, m);
        acc.z += __shfl_xor(acc.z, m);
        acc.w += __shfl_xor(acc.w, m);
      }
      if (lane < LPR) *(float4*)(&s_acc[w][4 * lane]) = acc;
      if (lane == 0) {
        s_m[w] = Mw;
        s_den[w] = den;
      }
      __syncthreads();
      if (w == 0) {
        const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
        float wk[kMergeWaves], d = 0.f;
#pragma unroll
        for (int k = 0; k < kMergeWaves; ++k) {
          wk[k] = s_m[k] == kNegInf ? 0.f : fast_exp2(s_m[k] - M);
          d += wk[k] * s_den[k];
        }
        const float sc = d > 0.f ? 1.f / d : 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int e = lane + kWave * i;
          float v = 0.f;
#pragma unroll
          for (int k = 0; k < kMergeWaves; ++k) v += wk[k] * s_acc[k][e];
          out[e] = v * sc;
        }
      }
      return;
    }
  }
  float M = kNegInf;
  for (int p0 = lo; p0 < hi; p0 += kWave)
    if (p0 + lane < hi && live(p0 + lane)) M = fmaxf(M, a.ws_m[(slot0 + p0 + lane) * G + h]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
  if (lane == 0) s_m[w] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  RowAcc<D> acc;
  rows_clear(acc);
  float den = 0.f;
  for (int p0 = lo; p0 < hi; p0 += kWave) {
    float f = 0.f, lp = 0.f;
    if (p0 + lane < hi && live(p0 + lane)) {
      const size_t si = (slot0 + p0 + lane) * G + h;
      const float mp = a.ws_m[si];
      lp = a.ws_l[si];
      f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
    }
    float fl = f * lp;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) fl += __shfl_xor(fl, s);
    den += fl;
    rows_accumulate<D>(acc, a.ws_o + ((slot0 + p0) * G + h) * D, (size_t)G * D, f,
                       min(kWave, hi - p0), lane);
  }
  // this wave's weighted sum (scale 1) into LDS, then wave 0 adds the four
  rows_store<D>(acc, s_acc[w], 1.f, lane);
  if (lane == 0) s_den[w] = den;
  __syncthreads();
  if (w == 0) {
    const float d = s_den[0] + s_den[1] + s_den[2] + s_den[3];
    const float sc = d > 0.f ? 1.f / d : 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + kWave * i;
      out[e] = (s_acc[0][e] + s_acc[1][e] + s_acc[2][e] + s_acc[3][e]) * sc;
    }
  }
}

hipError_t launch_stream_merge(const DecodeArgs& a, hipStream_t s) {
  const long long segs = (long long)a.Hkv * a.B;
  if ((a.d == 128 || a.d == 64) && a.chunks + segs > 16 * segs) {
    const dim3 grid((unsigned)(a.B * a.Hq)), block(kMergeWaves * kWave);
    if (a.d == 128) hipLaunchKernelGGL(stream_merge_long_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(stream_merge_long_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.B * a.Hq + kMergeWaves - 1) / kMergeWaves)), block(kMergeWaves * kWave);
  if (a.d == 128) hipLaunchKernelGGL(stream_merge_kernel<128>, grid, block, 0, s, a);
  else if (a.d == 64) hipLaunchKernelGGL(stream_merge_kernel<64>, grid, block, 0, s, a);
  else if (a.d == 512) hipLaunchKernelGGL(stream_merge_kernel<512>, grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

static hipError_t launch_gqa_stream_impl(const DecodeArgs& a, hipStream_t s, bool merge) {
  if (a.B > kMaxStreamSeqs || a.chunks % 32) return hipErrorInvalidValue;
  if (a.d == 128)
    return a.fp8 ? launch_stream_d<128, true>(a, s, merge) : launch_stream_d<128, false>(a, s, merge);
  if (a.d == 64 && !a.fp8) return launch_stream_d<64, false>(a, s, merge);
  return hipErrorInvalidValue;
}

hipError_t launch_gqa_stream(const DecodeArgs& a, hipStream_t s) {
  return launch_gqa_stream_impl(a, s, true);
}

hipError_t launch_gqa_stream_pieces(const DecodeArgs& a, hipStream_t s) {
  return launch_gqa_stream_impl(a, s, false);
}

}  // namespace pkv
