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

// Value of lane "head h of this lane's p.V group" (see layouts above) in every lane.
template <int D, int H>
__device__ __forceinline__ float group_bcast(float x, int lane) {
  if constexpr (D == 128) {
    return row_bcast<H>(x);
  } else {
    float lo = row_bcast<H>(x), hi = row_bcast<8 + H>(x);
    return (lane & 8) ? hi : lo;
  }
}
template <int D, int H>
__device__ __forceinline__ uint32_t group_bcast_u(uint32_t x, int lane) {
  if constexpr (D == 128) {
    return row_bcast_u<H>(x);
  } else {
    uint32_t lo = row_bcast_u<H>(x), hi = row_bcast_u<8 + H>(x);
    return (lane & 8) ? hi : lo;
  }
}

// Sum over the 8 lanes of a q.K token of x[0..G-1]; lane c receives head c & (G-1).
// Steps over lane bits 2, 1, 0; a step halves the value count (reduce-scatter) while more
// values than remaining steps' capacity are left, otherwise it is a plain all-reduce.
template <int N, int CTRL>
__device__ __forceinline__ void rs_step(float* x, bool upper) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    float keep = upper ? x[i + N / 2] : x[i];
    float send = upper ? x[i] : x[i + N / 2];
    x[i] = keep + dpp<CTRL>(send);
  }
}
template <int N, int CTRL>
__device__ __forceinline__ void ar_step(float* x) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp<CTRL>(x[i]);
}
template <int G>
__device__ __forceinline__ float reduce8(float* x, int c) {
  if constexpr (G == 8) {
    rs_step<8, kDppHalfMirror>(x, c & 4);
    rs_step<4, kDppQuadXor2>(x, c & 2);
    rs_step<2, kDppQuadXor1>(x, c & 1);
  } else if constexpr (G == 4) {
    ar_step<4, kDppHalfMirror>(x);
    rs_step<4, kDppQuadXor2>(x, c & 2);
    rs_step<2, kDppQuadXor1>(x, c & 1);
  } else if constexpr (G == 2) {
    ar_step<2, kDppHalfMirror>(x);
    ar_step<2, kDppQuadXor2>(x);
    rs_step<2, kDppQuadXor1>(x, c & 1);
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
  float m;                            // running max (log2 domain), head c, this group
  float l;                            // running sum of probabilities, head c, this group
};

// K and V of a tile are streamed once and never re-read: nontemporal loads keep them from
// displacing q, block-table and partial data in the caches.
__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint2 load_nt8(const uint8_t* p) {
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
  return uint2{v[0], v[1]};
}

// Per-lane byte offsets inside a tile, constant for the whole walk: with the tile base
// uniform, every K/V load is "SGPR base + this VGPR + immediate".
template <int D, bool FP8>
__device__ __forceinline__ uint32_t k_lane_offset(int k, int c) {
  return (uint32_t)(k * Layout<D, FP8>::ROW + 16 * c);
}
template <int D, bool FP8>
__device__ __forceinline__ uint32_t v_lane_offset(int r, int dc) {
  return (uint32_t)(pv_token<D>(0, r) * Layout<D, FP8>::ROW + dc * Layout<D, FP8>::VB);
}

template <int D, bool FP8>
__device__ __forceinline__ void load_k(TileRegs<D, FP8>& R, const uint8_t* kt, uint32_t koff) {
  using Lo = Layout<D, FP8>;
  const uint8_t* p = kt + koff;
#pragma unroll
  for (int pi = 0; pi < 2; ++pi)
#pragma unroll
    for (int j = 0; j < Lo::KL; ++j) R.k[pi][j] = load_nt16(p + 8 * pi * Lo::ROW + j * 128);
}
template <int D, bool FP8>
__device__ __forceinline__ void load_v(TileRegs<D, FP8>& R, const uint8_t* vt, uint32_t voff) {
  using Lo = Layout<D, FP8>;
  const uint8_t* p = vt + voff;
#pragma unroll
  for (int u = 0; u < Lo::TPG; ++u) {
    // token of slot u minus token of slot 0 does not depend on the row group
    const uint8_t* q = p + (pv_token<D>(u, 0) - pv_token<D>(0, 0)) * Lo::ROW;
    if constexpr (FP8) R.v[u] = load_nt8(q);
    else R.v[u] = load_nt16(q);
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
// probabilities as bf16 token pairs (in `pairs`).  Consumes only R.k, so the caller can
// refill R.k before the second half.  nv = valid tokens in the tile (16 except a
// sequence's last tile).
template <int D, int G, bool FP8>
__device__ __forceinline__ void qk_softmax(WaveState<D, G, FP8>& S, const TileRegs<D, FP8>& R,
                                           int nv, float cscale, int lane,
                                           uint32_t (&pairs)[Layout<D, FP8>::NPS]) {
  using Lo = Layout<D, FP8>;
  const int k = lane >> 3, c = lane & 7;
  const bool partial = nv < kTile;
  constexpr auto heads = std::make_integer_sequence<int, G>{};

  // ---- scores for tokens 8*pi + k, head c of this lane
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
      float a = 0.f;
#pragma unroll
      for (int p = 0; p < Lo::NP; ++p) a = dot2(S.q[h][p], kp[p], a);
      acc[h] = a;
    }
    float sc = reduce8<G>(acc, c) * cscale;
    if (partial && (8 * pi + k) >= nv) sc = kNegInf;
    s[pi] = sc;
  }

  // ---- running max of this group for head c; lazy rescale
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

// Second half of a tile: p.V accumulation.  Consumes only R.v.
template <int D, int G, bool FP8>
__device__ __forceinline__ void pv_accumulate(WaveState<D, G, FP8>& S, TileRegs<D, FP8>& R,
                                              int nv, int lane,
                                              const uint32_t (&pairs)[Layout<D, FP8>::NPS]) {
  using Lo = Layout<D, FP8>;
  const int r = lane / Lo::LPT;
  constexpr auto heads = std::make_integer_sequence<int, G>{};
  if (nv < kTile) {
#pragma unroll
    for (int u = 0; u < Lo::TPG; ++u)
      if (pv_token<D>(u, r) >= nv) R.v[u] = typename VReg<FP8>::T{};
  }
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
      // bf16 -> fp16 (exact for |v| < 65504, the supported range of bf16 V)
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
// as its K pieces); clears the accumulators.
template <int D, int G, bool FP8>
__device__ __forceinline__ void load_q_reset(WaveState<D, G, FP8>& S, const uint16_t* qg, int c) {
  using Lo = Layout<D, FP8>;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint8_t* qh = (const uint8_t*)(qg + (size_t)h * D);
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

}  // namespace pkv
