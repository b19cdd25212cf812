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
//  * Both products use v_dot2c_f32_bf16: q.K pairs adjacent dims, p.V pairs two tokens
//           (probabilities rounded to bf16, V rows interleaved with v_perm_b32).  FP8 E4M3
//           K/V are widened to bf16 pairs with v_cvt_scalef32_pk_bf16_fp8 (exact); the
//           per-head K scale folds into the score scale and the V scale into the output.
// Online softmax runs in the log2 domain with a lazy rescale: the running max only moves
// (rescaling o and l) when a new score exceeds it by more than 2^8, which keeps every
// probability <= 256 and skips almost all rescales after the first tile.
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

template <int D, bool FP8>
__device__ __forceinline__ void load_k(TileRegs<D, FP8>& R, const uint8_t* kt, int k, int c) {
  using Lo = Layout<D, FP8>;
#pragma unroll
  for (int pi = 0; pi < 2; ++pi)
#pragma unroll
    for (int j = 0; j < Lo::KL; ++j)
      R.k[pi][j] = load_nt16(kt + (8 * pi + k) * Lo::ROW + j * 128 + 16 * c);
}
template <int D, bool FP8>
__device__ __forceinline__ void load_v(TileRegs<D, FP8>& R, const uint8_t* vt, int r, int dc) {
  using Lo = Layout<D, FP8>;
#pragma unroll
  for (int u = 0; u < Lo::TPG; ++u) {
    const uint8_t* p = vt + pv_token<D>(u, r) * Lo::ROW + dc * Lo::VB;
    if constexpr (FP8) R.v[u] = load_nt8(p);
    else R.v[u] = load_nt16(p);
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
  for (int i = 0; i < 8; ++i) S.o[H][i] = dot2(P, vp[i], S.o[H][i]);
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

  // ---- probability pairs (two tokens of a p.V pair slot) as bf16, and the running sum
  if constexpr (D == 128) {
    pairs[0] = pack_bf16(p0, dpp<kDppRowRor8>(p0));
    pairs[1] = pack_bf16(p1, dpp<kDppRowRor8>(p1));
    S.l = dot2(pairs[0], kOnesBf16x2, S.l);
    S.l = dot2(pairs[1], kOnesBf16x2, S.l);
  } else {
    pairs[0] = pack_bf16(p0, p1);
    S.l = dot2(pairs[0], kOnesBf16x2, S.l);
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
        vp[4 * w + 0] = fp8x2_to_bf16x2<false>(t0);
        vp[4 * w + 1] = fp8x2_to_bf16x2<true>(t0);
        vp[4 * w + 2] = fp8x2_to_bf16x2<false>(t1);
        vp[4 * w + 3] = fp8x2_to_bf16x2<true>(t1);
      }
    } else {
      const uint4 A = R.v[2 * j], B = R.v[2 * j + 1];
      const uint32_t a4[4] = {A.x, A.y, A.z, A.w}, b4[4] = {B.x, B.y, B.z, B.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vp[2 * w] = byte_perm(b4[w], a4[w], 0x05040100u);      // (A[2w],   B[2w])
        vp[2 * w + 1] = byte_perm(b4[w], a4[w], 0x07060302u);  // (A[2w+1], B[2w+1])
      }
    }
    pv_all(S, pairs[j], vp, lane, heads);
  }
}

// Merge two online-softmax states (max m, sum l, accumulators o) into the first.
template <int G>
__device__ __forceinline__ void merge_state(float (&ma)[G], float (&la)[G], float (&oa)[G][8],
                                            const float (&mb)[G], const float (&lb)[G],
                                            const float (&ob)[G][8]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = fmaxf(ma[h], mb[h]);
    const float fa = (ma[h] == kNegInf) ? 0.f : fast_exp2(ma[h] - M);
    const float fb = (mb[h] == kNegInf) ? 0.f : fast_exp2(mb[h] - M);
    la[h] = fa * la[h] + fb * lb[h];
#pragma unroll
    for (int i = 0; i < 8; ++i) oa[h][i] = fa * oa[h][i] + fb * ob[h][i];
    ma[h] = M;
  }
}

template <int G>
struct GroupState {
  float m[G], l[G], o[G][8];
};

template <int G, typename F>
__device__ __forceinline__ void exchange_merge(GroupState<G>& X, F&& pairer) {
  GroupState<G> A, B;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    pairer(X.m[h], A.m[h], B.m[h]);
    pairer(X.l[h], A.l[h], B.l[h]);
#pragma unroll
    for (int i = 0; i < 8; ++i) pairer(X.o[h][i], A.o[h][i], B.o[h][i]);
  }
  merge_state<G>(A.m, A.l, A.o, B.m, B.l, B.o);
  X = A;
}

template <int D, int G, bool FP8, int H>
__device__ __forceinline__ void take_head_stats(GroupState<G>& X, const WaveState<D, G, FP8>& S,
                                                int lane) {
  X.m[H] = group_bcast<D, H>(S.m, lane);
  X.l[H] = group_bcast<D, H>(S.l, lane);
}
template <int D, int G, bool FP8, int... Hs>
__device__ __forceinline__ void take_stats(GroupState<G>& X, const WaveState<D, G, FP8>& S,
                                           int lane, std::integer_sequence<int, Hs...>) {
  (take_head_stats<D, G, FP8, Hs>(X, S, lane), ...);
}

template <int D, int G, bool FP8>
__global__ __launch_bounds__(kWaves * kWave, 2) void gqa_decode_kernel(DecodeArgs a) {
  using Lo = Layout<D, FP8>;
  const int g = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
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
  // q pairs for this lane's dims (same dims as its K pieces)
  const uint16_t* qg = a.q + ((size_t)b * a.Hq + (size_t)g * G) * D;
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

  L = L < 0 ? 0 : (L > a.max_blocks * a.block_size ? a.max_blocks * a.block_size : L);
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

  auto tile_addr = [&](int n, const uint8_t*& kt, const uint8_t*& vt) -> int {
    const uint64_t off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_lo, n) |
                         ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_hi, n) << 32);
    kt = kbase + off;
    vt = vbase + off;
    return __builtin_amdgcn_readlane(nv_lane, n);
  };

  // Two tile buffers, refilled half by half: a tile's K is replaced by the tile two ahead
  // as soon as its scores are done, its V once p.V is done, so one and a half to two tiles
  // are always in flight.
  TileRegs<D, FP8> RA, RB;
  const uint8_t *ktA, *vtA, *ktB, *vtB;
  int nvA = 0, nvB = 0;
  if (nt > 0) {
    nvA = tile_addr(0, ktA, vtA);
    load_k<D, FP8>(RA, ktA, k, c);
    load_v<D, FP8>(RA, vtA, r, dc);
  }
  if (nt > 1) {
    nvB = tile_addr(1, ktB, vtB);
    load_k<D, FP8>(RB, ktB, k, c);
    load_v<D, FP8>(RB, vtB, r, dc);
  }
  for (int n = 0; n < nt; n += 2) {
    {
      uint32_t pairs[Lo::NPS];
      qk_softmax<D, G, FP8>(S, RA, nvA, cscale, lane, pairs);
      int nv_next = 0;
      if (n + 2 < nt) {
        nv_next = tile_addr(n + 2, ktA, vtA);
        load_k<D, FP8>(RA, ktA, k, c);
      }
      pv_accumulate<D, G, FP8>(S, RA, nvA, lane, pairs);
      if (n + 2 < nt) load_v<D, FP8>(RA, vtA, r, dc);
      nvA = nv_next;
    }
    if (n + 1 >= nt) break;
    {
      uint32_t pairs[Lo::NPS];
      qk_softmax<D, G, FP8>(S, RB, nvB, cscale, lane, pairs);
      int nv_next = 0;
      if (n + 3 < nt) {
        nv_next = tile_addr(n + 3, ktB, vtB);
        load_k<D, FP8>(RB, ktB, k, c);
      }
      pv_accumulate<D, G, FP8>(S, RB, nvB, lane, pairs);
      if (n + 3 < nt) load_v<D, FP8>(RB, vtB, r, dc);
      nvB = nv_next;
    }
  }

  // ---- merge the wave's row groups: every lane ends with the wave's state for its dims
  GroupState<G> X;
  take_stats(X, S, lane, std::make_integer_sequence<int, G>{});
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) X.o[h][i] = S.o[h][i];
  if constexpr (D == 64) {  // half-rows -> rows
    exchange_merge<G>(X, [](float x, float& e, float& o) {
      e = x;
      o = dpp<kDppRowRor8>(x);
    });
  }
  exchange_merge<G>(X, [](float x, float& e, float& o) { rows_pair16(x, e, o); });
  exchange_merge<G>(X, [](float x, float& e, float& o) { halves_pair32(x, e, o); });

  // ---- merge the 4 waves through LDS and write the output or the partition's partials
  __shared__ float s_o[kWaves][G][D];
  __shared__ float s_m[kWaves][G], s_l[kWaves][G];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *(float4*)&s_o[w][h][8 * dc] = make_float4(X.o[h][0], X.o[h][1], X.o[h][2], X.o[h][3]);
      *(float4*)&s_o[w][h][8 * dc + 4] = make_float4(X.o[h][4], X.o[h][5], X.o[h][6], X.o[h][7]);
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
// One wave per (sequence, head): the partitions' statistics are loaded one per lane, their
// factors broadcast by readlane while the lanes stream the partial outputs.
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
  float acc[PER] = {};
  float den = 0.f;
  for (int p0 = 0; p0 < nP; p0 += kWave) {
    float f = 0.f, lp = 0.f;
    if (p0 + lane < nP) {
      const float mp = ws_m[base + p0 + lane];
      lp = ws_l[base + p0 + lane];
      f = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
    }
    den += wave_sum(f * lp);
    const int cnt = min(kWave, nP - p0);
    const float* op = ws_o + (base + p0) * D + lane;
    for (int j = 0; j < cnt; ++j) {
      const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += fj * op[(size_t)j * D + kWave * i];
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[lane + kWave * i] = acc[i] * inv;
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
