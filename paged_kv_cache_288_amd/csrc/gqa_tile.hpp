// Per-tile building blocks of the GQA decode kernels (see gqa_decode.hip for the layouts):
// register tiles, nontemporal K/V loads, scores + online softmax, p.V, and the merges of
// online-softmax states.
#pragma once

#include <utility>

#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

constexpr int kTile = 16;          // tokens per tile
constexpr int kWaves = 4;          // waves per workgroup
constexpr float kRescaleSlack = 8.0f;

template <int D, bool FP8>
struct Layout {
  static constexpr int ES = FP8 ? 1 : 2;        // bytes per element
  static constexpr int ROW = D * ES;            // bytes per token row
  static constexpr int KL = ROW / 128;          // 16-byte K loads per lane per pass
  static constexpr int NP = D / 16;             // bf16 pairs per lane per pass (q.K)
  static constexpr int LPT = D / 8;             // p.V lanes per token row (8 dims each)
  static constexpr int NG = kWave / LPT;        // p.V row groups per wave
  static constexpr int TPG = kTile / NG;        // tokens per group per tile
  static constexpr int NPS = TPG / 2;           // token pairs per group per tile
  static constexpr int VB = 8 * ES;             // V bytes per lane per token
  static_assert(KL >= 1 && TPG >= 2, "layout");
};

template <bool FP8> struct VReg;
template <> struct VReg<false> { typedef uint4 T; };
template <> struct VReg<true> { typedef uint2 T; };

template <int D, bool FP8>
struct TileRegs {
  uint4 k[2][Layout<D, FP8>::KL];
  typename VReg<FP8>::T v[Layout<D, FP8>::TPG];
};

// Token (0..15) of p.V slot u for row group r.
template <int D>
__device__ __forceinline__ int pv_token(int u, int r) {
  if constexpr (D == 128) return 8 * (u >> 1) + 2 * r + (u & 1);
  else return 8 * u + r;
}

// After the q.K reduction (reduce8 below) lane c of a token's 8 lanes holds head
// head_of_lane<G>(c); lane_of_head(H) is a lane that holds head H.  The map is c with bits
// 0-1 flipped when bit 2 is set: it makes each DPP step's partner (lanes c^7, c^2, c^1)
// hold, at the same register index, the head this lane keeps.
template <int G>
__device__ __forceinline__ int head_of_lane(int c) {
  return ((c & 4) ? c ^ 3 : c) & (G - 1);
}
constexpr int lane_of_head(int H) { return (H & 4) ? H ^ 3 : H; }

// Value that the lane holding head H in this lane's p.V group has, in every lane.
template <int D, int H>
__device__ __forceinline__ float group_bcast(float x, int lane) {
  constexpr int LH = lane_of_head(H);
  if constexpr (D == 128) {
    return row_bcast<LH>(x);
  } else {
    float lo = row_bcast<LH>(x), hi = row_bcast<8 + LH>(x);
    return (lane & 8) ? hi : lo;
  }
}
template <int D, int H>
__device__ __forceinline__ uint32_t group_bcast_u(uint32_t x, int lane) {
  constexpr int LH = lane_of_head(H);
  if constexpr (D == 128) {
    return row_bcast_u<LH>(x);
  } else {
    uint32_t lo = row_bcast_u<LH>(x), hi = row_bcast_u<8 + LH>(x);
    return (lane & 8) ? hi : lo;
  }
}

// Sum over the 8 lanes of a q.K token of x[0..G-1], where lane c holds head
// j ^ head_of_lane<G>(c) in x[j] (q is loaded in that order); lane c receives head
// head_of_lane<G>(c) in x[0].  Steps over the partners c^7, c^2, c^1; while more values are
// left than the remaining steps can separate, a step all-reduces, otherwise it
// reduce-scatters: x[i] += partner's x[i + N/2], which by the head order above is the same
// head, so no lane-dependent selection is needed.
template <int N, int CTRL>
__device__ __forceinline__ void rs_step(float* x) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) x[i] += dpp<CTRL>(x[i + N / 2]);
}
template <int N, int CTRL>
__device__ __forceinline__ void ar_step(float* x) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp<CTRL>(x[i]);
}
template <int G>
__device__ __forceinline__ float reduce8(float* x) {
  if constexpr (G == 8) {
    rs_step<8, kDppHalfMirror>(x);
    rs_step<4, kDppQuadXor2>(x);
    rs_step<2, kDppQuadXor1>(x);
  } else if constexpr (G == 4) {
    ar_step<4, kDppHalfMirror>(x);
    rs_step<4, kDppQuadXor2>(x);
    rs_step<2, kDppQuadXor1>(x);
  } else if constexpr (G == 2) {
    ar_step<2, kDppHalfMirror>(x);
    ar_step<2, kDppQuadXor2>(x);
    rs_step<2, kDppQuadXor1>(x);
  } else {
    ar_step<1, kDppHalfMirror>(x);
    ar_step<1, kDppQuadXor2>(x);
    ar_step<1, kDppQuadXor1>(x);
  }
  return x[0];
}

template <int D, int G, bool FP8>
struct WaveState {
  uint32_t q[G][Layout<D, FP8>::NP];  // bf16 pairs of the G query heads, this lane's dims
  float o[G][8];                      // p.V accumulators of this lane's row group
  float m;                            // running max (log2 domain), this lane's head, this group
  float l;                            // running sum of probabilities, same head and group
};

// ---- K/V tile sources.  A tile's K and V rows are read through buffer resources whose
// range is the tile's valid rows: rows past it (a sequence's last, partial tile, a block id
// outside the pool, a tile past the end of a walk) load as zeros without a memory access.
// So every load is unconditional, and padding never reaches p.V.  K and V are streamed once
// and never re-read: the loads are nontemporal, which keeps them from displacing q,
// block-table and partial data in the caches.
struct TileSrc {
  rsrc_t k, v;
};
template <int D, bool FP8>
__device__ __forceinline__ TileSrc tile_src(const uint8_t* kt, const uint8_t* vt, int nv) {
  const int bytes = nv * Layout<D, FP8>::ROW;
  return TileSrc{make_rsrc(kt, bytes), make_rsrc(vt, bytes)};
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadNontemporal);
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadNontemporal);
  return uint2{v[0], v[1]};
}

// Per-lane byte offsets inside a tile, constant for the whole walk.
template <int D, bool FP8>
__device__ __forceinline__ uint32_t k_lane_offset(int k, int c) {
  return (uint32_t)(k * Layout<D, FP8>::ROW + 16 * c);
}
template <int D, bool FP8>
__device__ __forceinline__ uint32_t v_lane_offset(int r, int dc) {
  return (uint32_t)(pv_token<D>(0, r) * Layout<D, FP8>::ROW + dc * Layout<D, FP8>::VB);
}

template <int D, bool FP8>
__device__ __forceinline__ void load_k(TileRegs<D, FP8>& R, rsrc_t src, uint32_t koff) {
  using Lo = Layout<D, FP8>;
#pragma unroll
  for (int pi = 0; pi < 2; ++pi)
#pragma unroll
    for (int j = 0; j < Lo::KL; ++j) R.k[pi][j] = buf_load16(src, koff + 8 * pi * Lo::ROW + j * 128);
}
template <int D, bool FP8>
__device__ __forceinline__ void load_v(TileRegs<D, FP8>& R, rsrc_t src, uint32_t voff) {
  using Lo = Layout<D, FP8>;
#pragma unroll
  for (int u = 0; u < Lo::TPG; ++u) {
    // token of slot u minus token of slot 0 does not depend on the row group
    const uint32_t o = voff + (pv_token<D>(u, 0) - pv_token<D>(0, 0)) * Lo::ROW;
    if constexpr (FP8) R.v[u] = buf_load8(src, o);
    else R.v[u] = buf_load16(src, o);
  }
}

template <int D, int G, bool FP8, int H>
__device__ __forceinline__ void rescale_head(WaveState<D, G, FP8>& S, float alpha, int lane) {
  float a = group_bcast<D, H>(alpha, lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) S.o[H][i] *= a;
}

template <int D, int G, bool FP8, int H>
__device__ __forceinline__ void pv_head(WaveState<D, G, FP8>& S, uint32_t pair,
                                        const uint32_t (&vp)[8], int lane) {
  uint32_t P = group_bcast_u<D, H>(pair, lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) S.o[H][i] = dot2h(P, vp[i], S.o[H][i]);
}

template <int D, int G, bool FP8, int... Hs>
__device__ __forceinline__ void rescale_all(WaveState<D, G, FP8>& S, float alpha, int lane,
                                            std::integer_sequence<int, Hs...>) {
  (rescale_head<D, G, FP8, Hs>(S, alpha, lane), ...);
}
template <int D, int G, bool FP8, int... Hs>
__device__ __forceinline__ void pv_all(WaveState<D, G, FP8>& S, uint32_t pair,
                                       const uint32_t (&vp)[8], int lane,
                                       std::integer_sequence<int, Hs...>) {
  (pv_head<D, G, FP8, Hs>(S, pair, vp, lane), ...);
}

// First half of a 16-token tile: scores and the online-softmax update; returns the
// probabilities as fp16 token pairs (in `pairs`).  Consumes only R.k, so the caller can
// refill R.k before the second half.  nv = valid tokens in the tile (16 except a
// sequence's last tile).
template <int D, int G, bool FP8>
__device__ __forceinline__ void qk_softmax(WaveState<D, G, FP8>& S, const TileRegs<D, FP8>& R,
                                           int nv, float cscale, int lane,
                                           uint32_t (&pairs)[Layout<D, FP8>::NPS]) {
  using Lo = Layout<D, FP8>;
  const int k = lane >> 3;
  const bool partial = nv < kTile;
  constexpr auto heads = std::make_integer_sequence<int, G>{};

  // ---- scores for tokens 8*pi + k, head head_of_lane(c) of this lane
  float s[2];
#pragma unroll
  for (int pi = 0; pi < 2; ++pi) {
    uint32_t kp[Lo::NP];
    if constexpr (FP8) {
      const uint32_t w4[4] = {R.k[pi][0].x, R.k[pi][0].y, R.k[pi][0].z, R.k[pi][0].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kp[2 * w] = fp8x2_to_bf16x2<false>(w4[w]);
        kp[2 * w + 1] = fp8x2_to_bf16x2<true>(w4[w]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < Lo::KL; ++j) {
        kp[4 * j + 0] = R.k[pi][j].x;
        kp[4 * j + 1] = R.k[pi][j].y;
        kp[4 * j + 2] = R.k[pi][j].z;
        kp[4 * j + 3] = R.k[pi][j].w;
      }
    }
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = dot2_zero(S.q[h][0], kp[0]);
#pragma unroll
      for (int p = 1; p < Lo::NP; ++p) a = dot2(S.q[h][p], kp[p], a);
      acc[h] = a;
    }
    float sc = reduce8<G>(acc) * cscale;
    if (partial && (8 * pi + k) >= nv) sc = kNegInf;
    s[pi] = sc;
  }

  // ---- running max of this group for the lane's head; lazy rescale
  float mt = fmaxf(s[0], s[1]);
  if constexpr (D == 128) mt = fmaxf(mt, dpp<kDppRowRor8>(mt));
  if (wave_any(mt > S.m + kRescaleSlack)) {
    const float m_new = fmaxf(S.m, mt);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(S.m - m_new);
    S.l *= alpha;
    S.m = m_new;
    rescale_all(S, alpha, lane, heads);
  }
  const float m_use = (S.m == kNegInf) ? 0.f : S.m;
  const float p0 = fast_exp2(s[0] - m_use), p1 = fast_exp2(s[1] - m_use);

  // ---- probability pairs (two tokens of a p.V pair slot) as fp16, and the running sum of
  // the rounded values.  p <= 2^8 after the lazy max, well inside fp16; its 10-bit mantissa
  // keeps the rounding of the weights below 2^-11 relative.
  if constexpr (D == 128) {
    pairs[0] = pack_f16(p0, dpp<kDppRowRor8>(p0));
    pairs[1] = pack_f16(p1, dpp<kDppRowRor8>(p1));
    S.l = dot2h(pairs[0], kOnesF16x2, S.l);
    S.l = dot2h(pairs[1], kOnesF16x2, S.l);
  } else {
    pairs[0] = pack_f16(p0, p1);
    S.l = dot2h(pairs[0], kOnesF16x2, S.l);
  }

}

// Second half of a tile: p.V accumulation.  Consumes only R.v (rows past the tile's valid
// tokens were loaded as zeros and carry zero probability).
template <int D, int G, bool FP8>
__device__ __forceinline__ void pv_accumulate(WaveState<D, G, FP8>& S, const TileRegs<D, FP8>& R,
                                              int lane,
                                              const uint32_t (&pairs)[Layout<D, FP8>::NPS]) {
  using Lo = Layout<D, FP8>;
  constexpr auto heads = std::make_integer_sequence<int, G>{};
#pragma unroll
  for (int j = 0; j < Lo::NPS; ++j) {
    uint32_t vp[8];
    if constexpr (FP8) {
      const uint2 A = R.v[2 * j], B = R.v[2 * j + 1];
      const uint32_t a2[2] = {A.x, A.y}, b2[2] = {B.x, B.y};
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t t0 = byte_perm(b2[w], a2[w], 0x05010400u);  // A0 B0 A1 B1
        const uint32_t t1 = byte_perm(b2[w], a2[w], 0x07030602u);  // A2 B2 A3 B3
        vp[4 * w + 0] = fp8x2_to_f16x2<false>(t0);
        vp[4 * w + 1] = fp8x2_to_f16x2<true>(t0);
        vp[4 * w + 2] = fp8x2_to_f16x2<false>(t1);
        vp[4 * w + 3] = fp8x2_to_f16x2<true>(t1);
      }
    } else {
      const uint4 A = R.v[2 * j], B = R.v[2 * j + 1];
      const uint32_t a4[4] = {A.x, A.y, A.z, A.w}, b4[4] = {B.x, B.y, B.z, B.w};
#pragma unroll
      // bf16 -> fp16: exact for 2^-14 <= |v| < 65504 (the supported range of bf16 V),
      // rounded to fp16's subnormal grid below 2^-14 (absolute error <= 2^-25)
      for (int w = 0; w < 4; ++w) {
        vp[2 * w] = pack_f16(bf16_lo(a4[w]), bf16_lo(b4[w]));      // (A[2w],   B[2w])
        vp[2 * w + 1] = pack_f16(bf16_hi(a4[w]), bf16_hi(b4[w]));  // (A[2w+1], B[2w+1])
      }
    }
    pv_all(S, pairs[j], vp, lane, heads);
  }
}

// Online-softmax statistics of the G heads for the lane's row group (or, after
// wave_merge_rows, for the whole wave); the accumulators stay in WaveState::o.
template <int G>
struct GroupStats {
  float m[G], l[G];
};

// Merge, head by head and in place, each lane's state with the state `pairer` pairs it
// with (pairer(x, a, b) returns in a and b the two values being combined).
template <int G, typename F>
__device__ __forceinline__ void exchange_merge(float (&m)[G], float (&l)[G], float (&o)[G][8],
                                               F&& pairer) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float ma, mb, la, lb, oa[8], ob[8];
    pairer(m[h], ma, mb);
    pairer(l[h], la, lb);
#pragma unroll
    for (int i = 0; i < 8; ++i) pairer(o[h][i], oa[i], ob[i]);
    const float M = fmaxf(ma, mb);
    const float fa = (ma == kNegInf) ? 0.f : fast_exp2(ma - M);
    const float fb = (mb == kNegInf) ? 0.f : fast_exp2(mb - M);
    l[h] = fa * la + fb * lb;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[h][i] = fa * oa[i] + fb * ob[i];
    m[h] = M;
  }
}

template <int D, int G, bool FP8, int H>
__device__ __forceinline__ void take_head_stats(GroupStats<G>& X, const WaveState<D, G, FP8>& S,
                                                int lane) {
  X.m[H] = group_bcast<D, H>(S.m, lane);
  X.l[H] = group_bcast<D, H>(S.l, lane);
}
template <int D, int G, bool FP8, int... Hs>
__device__ __forceinline__ void take_stats(GroupStats<G>& X, const WaveState<D, G, FP8>& S,
                                           int lane, std::integer_sequence<int, Hs...>) {
  (take_head_stats<D, G, FP8, Hs>(X, S, lane), ...);
}

// Merge the wave's row groups in place: afterwards every lane holds, in S.o and X, the
// wave's state for its dims.
template <int D, int G, bool FP8>
__device__ __forceinline__ void wave_merge_rows(GroupStats<G>& X, WaveState<D, G, FP8>& S,
                                                int lane) {
  take_stats(X, S, lane, std::make_integer_sequence<int, G>{});
  if constexpr (D == 64) {  // half-rows -> rows
    exchange_merge<G>(X.m, X.l, S.o, [](float x, float& e, float& o) {
      e = x;
      o = dpp<kDppRowRor8>(x);
    });
  }
  exchange_merge<G>(X.m, X.l, S.o, [](float x, float& e, float& o) { rows_pair16(x, e, o); });
  exchange_merge<G>(X.m, X.l, S.o, [](float x, float& e, float& o) { halves_pair32(x, e, o); });
}

// q pairs of the G heads starting at qg ([G][D] bf16) for this lane's dims (the same dims
// as its K pieces), S.q[j] holding head j ^ head_of_lane<G>(c) (the order reduce8 needs);
// clears the accumulators.
template <int D, int G, bool FP8>
__device__ __forceinline__ void load_q_reset(WaveState<D, G, FP8>& S, const uint16_t* qg, int c) {
  using Lo = Layout<D, FP8>;
  const int hm = head_of_lane<G>(c);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint8_t* qh = (const uint8_t*)(qg + (size_t)(h ^ hm) * D);
    if constexpr (FP8) {
      const uint4 x0 = *(const uint4*)(qh + 32 * c), x1 = *(const uint4*)(qh + 32 * c + 16);
      const uint32_t v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int p = 0; p < 8; ++p) S.q[h][p] = v[p];
    } else {
#pragma unroll
      for (int j = 0; j < Lo::KL; ++j) {
        const uint4 x = *(const uint4*)(qh + j * 128 + 16 * c);
        S.q[h][4 * j + 0] = x.x;
        S.q[h][4 * j + 1] = x.y;
        S.q[h][4 * j + 2] = x.z;
        S.q[h][4 * j + 3] = x.w;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) S.o[h][i] = 0.f;
  }
  S.m = kNegInf;
  S.l = 0.f;
}

// ---- merging partial states
// acc += sum over j < cnt (<= 64) of f_j * row_j, with row_j = base + j * stride floats and
// f_j held by lane j.  A zero weight skips its row (that row may never have been written).
// Rows are read as float4: D/4 lanes per row (all 64 lanes, D/256 loads each, for wider
// rows), so one load instruction covers several rows, and eight instructions are in flight
// per lane.  Afterwards the lanes of row slot 0 (lane < LPR) hold the sum.
template <int D>
struct RowAcc {
  static constexpr int LPR = D / 4 < kWave ? D / 4 : kWave;  // lanes per row
  static constexpr int RPW = kWave / LPR;                     // rows per load instruction
  static constexpr int V4 = D / 4 / LPR;                      // float4 per lane per row
  float4 v[V4];
};

template <int D>
__device__ __forceinline__ void rows_clear(RowAcc<D>& A) {
#pragma unroll
  for (int i = 0; i < RowAcc<D>::V4; ++i) A.v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int D>
__device__ __forceinline__ void rows_accumulate(RowAcc<D>& A, const float* base, size_t stride,
                                                float f, int cnt, int lane) {
  using R = RowAcc<D>;
  constexpr int U = 8;
  const int sub = lane / R::LPR, col = lane % R::LPR;
  for (int j0 = 0; j0 < cnt; j0 += R::RPW * U) {
    float fj[U];
    float4 x[U][R::V4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * R::RPW + sub;
      fj[u] = __shfl(f, j & (kWave - 1));
      if (j >= cnt) fj[u] = 0.f;
      const float* row = base + (size_t)(j < cnt ? j : 0) * stride;
#pragma unroll
      for (int i = 0; i < R::V4; ++i)
        x[u][i] = fj[u] != 0.f ? *(const float4*)(row + 4 * (col + R::LPR * i))
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < R::V4; ++i) {
        A.v[i].x += fj[u] * x[u][i].x;
        A.v[i].y += fj[u] * x[u][i].y;
        A.v[i].z += fj[u] * x[u][i].z;
        A.v[i].w += fj[u] * x[u][i].w;
      }
  }
}

// Sums the row slots into slot 0 and writes scale * sum to out[0..D) from lanes < LPR.
template <int D>
__device__ __forceinline__ void rows_store(RowAcc<D>& A, float* out, float scale, int lane) {
  using R = RowAcc<D>;
#pragma unroll
  for (int m = R::LPR; m < kWave; m <<= 1)
#pragma unroll
    for (int i = 0; i < R::V4; ++i) {
      A.v[i].x += __shfl_xor(A.v[i].x, m);
      A.v[i].y += __shfl_xor(A.v[i].y, m);
      A.v[i].z += __shfl_xor(A.v[i].z, m);
      A.v[i].w += __shfl_xor(A.v[i].w, m);
    }
  if (lane < R::LPR) {
#pragma unroll
    for (int i = 0; i < R::V4; ++i)
      *(float4*)(out + 4 * (lane + R::LPR * i)) =
          make_float4(A.v[i].x * scale, A.v[i].y * scale, A.v[i].z * scale, A.v[i].w * scale);
  }
}

}  // namespace pkv
