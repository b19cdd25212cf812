// Shared-prefix cascade on gfx950: the tail pass and the prefix pass in one launch, and the
// merge of their pieces.
//
// "深入LLM推理：从KV Cache到PD分离的Serving全景解析", section "PagedAttention与Cache管理": the
// sequences of a batch may point at the same physical blocks of a common prefix.  The
// cascade call attends each sequence's own blocks (tail) with the single-token balanced
// body (VALU, HBM-bound) and the prefix, once per group of 32 / G sequences, with the
// multi-token body (MFMA on 32 query rows, its re-reads of the prefix served by L2).  The
// two have nothing to wait for in each other, and they use different units, so they run
// in one launch: each workgroup takes one role, tail and prefix workgroups interleaved in
// groups of 8 (one of each per XCD round of dispatch), and both sets are sized to be
// resident together.  cascade_merge_kernel then combines, per output row, the tail pieces
// and the prefix pieces.
#include "gqa_multi_body.hpp"
#include "gqa_stream_body.hpp"

namespace pkv {

static_assert(kMaxStreamSeqs == kMultiSeqs && kWaves == kMW, "shared LDS and workgroup shape");

constexpr int kPrefixBuffers = 2;  // tiles in flight per prefix wave (3 or 4: same time)

// Workgroup v of the grid: tail workgroup (v / 16) * 8 + v % 8 when v % 16 < 8, else
// prefix workgroup (v / 16) * 8 + v % 8, while both kinds last; then the rest of the larger
// kind in order.  Either way the workgroup id keeps v's residue mod 8 (its XCD).
template <int D, int G, bool FP8>
__global__ __launch_bounds__(kWaves * kWave, 2) void cascade_kernel(DecodeArgs ta, MultiArgs pa,
                                                                    int tail_groups,
                                                                    int prefix_groups) {
  __shared__ int s_pre[kMaxStreamSeqs + 1];
  __shared__ int s_sum[kWaves * kWave];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kMW * MLayout<D, FP8>::LTILE];
  const int v = blockIdx.x;
  const int both = min(tail_groups, prefix_groups);
  bool tail;
  int id;
  if (v < 16 * both) {
    tail = (v & 15) < 8;
    id = (v >> 4) * 8 + (v & 7);
  } else {
    tail = tail_groups > prefix_groups;
    id = 8 * both + (v - 16 * both);
  }
  if (tail) gqa_stream_body<D, G, FP8>(ta, id, s_pre, s_sum);
  else gqa_multi_body<D, 2, FP8, kPrefixBuffers>(pa, id, s_pre, s_sum, s_v);
}

// out[b][h] = merge of the tail pieces of segment (g = h / G, b) (rows of G, from the
// single-token balanced kernel) and the prefix pieces of segment (g, b / J), row
// (b % J) * G + h % G (rows of J * G, from the multi-token kernel).  One wave per output row.
constexpr int kCascadeMergeWaves = 4;
constexpr int kCascadeFastPieces = 8;  // per set, merged in one round trip
template <int D>
__global__ __launch_bounds__(kCascadeMergeWaves * kWave) void cascade_merge_kernel(CascadeMergeArgs a) {
  constexpr int PER = D / kWave;
  const int G = a.Hq / a.Hkv;
  const int idx = blockIdx.x * kCascadeMergeWaves + (int)(threadIdx.x / kWave);
  if (idx >= a.B * a.Hq) return;
  const int b = idx / a.Hq, hq = idx - b * a.Hq, g = hq / G, h = hq - g * G;
  const int lane = threadIdx.x & (kWave - 1);
  float* out = a.out + (size_t)idx * D;

  // the two piece sets: first slot, count, rows per slot, row, and liveness of each chunk
  struct Set {
    const float *m, *l, *o;
    size_t slot0;
    int np, rows, row, c0, chunks;
    long long T;
  };
  auto make_set = [&](const float* m, const float* l, const float* o, const int32_t* prefix,
                      const int32_t* segr, int chunks, int nseq, int rows, int sb, int row) {
    Set st{m, l, o, 0, 0, rows, row, 0, chunks, 0};
    if (!m) return st;
    const int sg = g * nseq + sb;
    st.c0 = segr[2 * sg];
    st.np = segr[2 * sg + 1];
    st.slot0 = (size_t)st.c0 + sg;
    st.T = (long long)a.Hkv * prefix[nseq];
    return st;
  };
  const Set sets[2] = {
      make_set(a.t_m, a.t_l, a.t_o, a.t_prefix, a.t_seg, a.t_chunks, a.B, G, b, h),
      make_set(a.p_m, a.p_l, a.p_o, a.p_prefix, a.p_seg, a.p_chunks, a.p_B, a.p_J * G,
               a.p_J ? b / a.p_J : 0, a.p_J ? (b % a.p_J) * G + h : 0)};
  // with fewer tiles than chunks some chunks are empty and wrote nothing
  auto live = [](const Set& st, int i) {
    if (st.T >= st.chunks) return true;
    const long long cc = st.c0 + i;
    return st.T * cc / st.chunks != st.T * (cc + 1) / st.chunks;
  };
  // Up to kCascadeFastPieces pieces in each set: every piece's m, l and row requested at
  // once (one round trip instead of one per set and step); rows of pieces without weight
  // (empty chunks: never written) are loaded but not used.
  if (sets[0].np <= kCascadeFastPieces && sets[1].np <= kCascadeFastPieces) {
    constexpr int NP = 2 * kCascadeFastPieces, LPR = D / 4, RPW = kWave / LPR, U = NP / RPW;
    const int sub = lane / LPR, col = lane % LPR;
    // lane j < NP: piece j of set j / kCascadeFastPieces
    const int ks = lane / kCascadeFastPieces, kp = lane % kCascadeFastPieces;
    float mp = kNegInf, lp = 0.f;
    const Set& sl = (ks & 1) ? sets[1] : sets[0];
    if (lane < NP && kp < sl.np && live(sl, kp)) {
      const Set& st = sl;
      const size_t si = (st.slot0 + kp) * st.rows + st.row;
      mp = st.m[si];
      lp = st.l[si];
    }
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = u * RPW + sub, k = j / kCascadeFastPieces, p = j % kCascadeFastPieces;
      const Set& st = sets[k];
      x[u] = p < st.np ? *(const float4*)(st.o + ((st.slot0 + p) * st.rows + st.row) * D + 4 * col)
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
    const float sc = den > 0.f ? 1.f / den : 0.f;  // no token at all: zeros
    if (lane < LPR)
      *(float4*)(out + 4 * lane) = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
    return;
  }
  float M = kNegInf;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    for (int p0 = 0; p0 < sets[k].np; p0 += kWave)
      if (p0 + lane < sets[k].np && live(sets[k], p0 + lane))
        M = fmaxf(M, sets[k].m[(sets[k].slot0 + p0 + lane) * sets[k].rows + sets[k].row]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
  RowAcc<D> acc;
  rows_clear(acc);
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const Set& st = sets[k];
    for (int p0 = 0; p0 < st.np; p0 += kWave) {
      float f = 0.f, lp = 0.f;
      if (p0 + lane < st.np && live(st, p0 + lane)) {
        const size_t si = (st.slot0 + p0 + lane) * st.rows + st.row;
        const float mp = st.m[si];
        lp = st.l[si];
        f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
      }
      float fl = f * lp;
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) fl += __shfl_xor(fl, s);
      den += fl;
      rows_accumulate<D>(acc, st.o + ((st.slot0 + p0) * st.rows + st.row) * D,
                         (size_t)st.rows * D, f, min(kWave, st.np - p0), lane);
    }
  }
  if (den == 0.f) {  // no token at all
#pragma unroll
    for (int i = 0; i < PER; ++i) out[lane + kWave * i] = 0.f;
    return;
  }
  rows_store<D>(acc, out, 1.f / den, lane);
}

template <int D, bool FP8>
static hipError_t launch_cascade_d(const DecodeArgs& ta, const MultiArgs& pa, hipStream_t s) {
  const dim3 grid((unsigned)((ta.chunks + pa.chunks) / kWaves)), block(kWaves * kWave);
  const int tg = ta.chunks / (8 * kWaves), pg = pa.chunks / (8 * kWaves);
  switch (ta.Hq / ta.Hkv) {
    case 1: hipLaunchKernelGGL((cascade_kernel<D, 1, FP8>), grid, block, 0, s, ta, pa, tg, pg); break;
    case 2: hipLaunchKernelGGL((cascade_kernel<D, 2, FP8>), grid, block, 0, s, ta, pa, tg, pg); break;
    case 4: hipLaunchKernelGGL((cascade_kernel<D, 4, FP8>), grid, block, 0, s, ta, pa, tg, pg); break;
    case 8: hipLaunchKernelGGL((cascade_kernel<D, 8, FP8>), grid, block, 0, s, ta, pa, tg, pg); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cascade(const DecodeArgs& ta, const MultiArgs& pa, hipStream_t s) {
  if (ta.B > kMaxStreamSeqs || pa.B > kMultiSeqs || ta.chunks % 32 || pa.chunks % 32 ||
      ta.block_size % kTile || pa.Hq / pa.Hkv * pa.q_len > 32 || ta.fp8 != pa.fp8 || ta.d != pa.d)
    return hipErrorInvalidValue;
  if (ta.d == 128) return ta.fp8 ? launch_cascade_d<128, true>(ta, pa, s) : launch_cascade_d<128, false>(ta, pa, s);
  if (ta.d == 64 && !ta.fp8) return launch_cascade_d<64, false>(ta, pa, s);
  return hipErrorInvalidValue;
}

hipError_t launch_cascade_merge(const CascadeMergeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(((long long)a.B * a.Hq + kCascadeMergeWaves - 1) / kCascadeMergeWaves));
  if (a.d == 128) hipLaunchKernelGGL(cascade_merge_kernel<128>, grid, dim3(kCascadeMergeWaves * kWave), 0, s, a);
  else if (a.d == 64) hipLaunchKernelGGL(cascade_merge_kernel<64>, grid, dim3(kCascadeMergeWaves * kWave), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
