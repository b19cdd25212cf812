// Body of the multi-token paged decode (gqa_multi.hip describes the arithmetic and the
// register/LDS layouts): one workgroup's walk over its four chunks, leaving (m, l, o)
// pieces of q_len * G query rows.  A device function so that the shared-prefix cascade can
// run it (its prefix pass) in the same launch as the single-token tail pass.
#pragma once

#include "gqa_tile.hpp"

namespace pkv {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kMultiSeqs = 4096;      // sequences whose tile counts fit the LDS prefix
constexpr int kMultiChunkTiles = 128; // tiles per chunk: two per lane
constexpr int kMW = 4;                // waves per workgroup

template <int D, bool FP8>
struct MLayout {
  static constexpr int ROW = FP8 ? D : 2 * D;              // bytes per K or V row in HBM
  static constexpr int LROW = 2 * D;                       // bytes per V row in LDS (16-bit)
  static constexpr int KS = D / 32;                        // score MFMA steps
  static constexpr int KL = FP8 ? D / 64 : D / 32;         // 16-byte K loads per lane per tile
  static constexpr int NT = D / 16;                        // p.V MFMA dim blocks
  static constexpr int VL = kTile * ROW / (16 * kWave);    // 16-byte V loads per lane per tile
  static constexpr int TILE = kTile * ROW;                 // bytes of one K or V tile in HBM
  static constexpr int LTILE = kTile * LROW;               // bytes of one V tile in LDS
};

// LDS position of the 32-byte piece p of V row t is p ^ vswz(t): the rows a half-wave's
// transposed read touches (4 per 16-lane group, two groups) fall in distinct bank groups.
template <int D>
__device__ __forceinline__ int vswz(int t) {
  if constexpr (D == 128) return t & 7;
  else return (t >> 1) & 3;
}

__device__ __forceinline__ f32x4_t mfma_qk(const bf16x8_t& k, const bf16x8_t& q, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, q, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_pv(const f16x4_t& v, const f16x4_t& p, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(v, p, c, 0, 0, 0);
}

// Max / sum over the 4 lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max4(float x) {
  float lo, hi, e, o;
  halves_pair32(x, lo, hi);
  x = fmaxf(lo, hi);
  rows_pair16(x, e, o);
  return fmaxf(e, o);
}
__device__ __forceinline__ float sum4(float x) {
  float lo, hi, e, o;
  halves_pair32(x, lo, hi);
  x = lo + hi;
  rows_pair16(x, e, o);
  return e + o;
}

template <int D, bool FP8>
struct MTile {
  uint4 k[MLayout<D, FP8>::KL];
  uint4 v[MLayout<D, FP8>::VL];
};

// K pieces of lane l: token l % 16; the dims of MFMA step ks for lane group g = l / 16 are
// 32 ks + 8 g .. + 7 (bf16: one 16-byte load per step) or D/4 g + 8 ks .. + 7 (FP8: the
// group's D/4 contiguous bytes in D/64 loads).  q is read with the same map.
template <int D, bool FP8>
__device__ __forceinline__ uint32_t k_offset(int i16, int g, int j) {
  using Lo = MLayout<D, FP8>;
  return FP8 ? (uint32_t)(i16 * Lo::ROW + g * (D / 4) + 16 * j)
             : (uint32_t)(i16 * Lo::ROW + 16 * g + 64 * j);
}
template <int D, bool FP8>
__device__ __forceinline__ uint32_t q_offset(int g, int ks) {  // bytes into a bf16 q row
  return FP8 ? (uint32_t)(g * (D / 2) + 16 * ks) : (uint32_t)(64 * ks + 16 * g);
}
template <int D, bool FP8>
__device__ __forceinline__ void mload_k(MTile<D, FP8>& R, rsrc_t src, uint32_t koff) {
#pragma unroll
  for (int j = 0; j < MLayout<D, FP8>::KL; ++j) R.k[j] = buf_load16(src, koff + (FP8 ? 16 : 64) * j);
}
template <int D, bool FP8>
__device__ __forceinline__ void mload_v(MTile<D, FP8>& R, rsrc_t src, uint32_t lane) {
#pragma unroll
  for (int u = 0; u < MLayout<D, FP8>::VL; ++u) R.v[u] = buf_load16(src, 1024 * u + 16 * lane);
}
// A operand of score step ks: 8 bf16 K values (FP8 codes widened exactly).
template <int D, bool FP8>
__device__ __forceinline__ bf16x8_t k_frag(const MTile<D, FP8>& R, int ks) {
  if constexpr (FP8) {
    const uint4 x = R.k[ks >> 1];
    const uint32_t w0 = (ks & 1) ? x.z : x.x, w1 = (ks & 1) ? x.w : x.y;
    return __builtin_bit_cast(bf16x8_t, uint4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                                              fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1)});
  } else {
    return __builtin_bit_cast(bf16x8_t, R.k[ks]);
  }
}

}  // namespace

// Tiles in flight per wave (each a K and a V register buffer) and waves per SIMD: two
// buffers at two waves per SIMD, except for 64 rows of 128 dims (q and accumulators alone
// take 192 registers), which get the whole register file.
constexpr int multi_buffers(int D, int RT) { return 2; }
constexpr int multi_waves_per_simd(int D, int RT) {
  return (D * RT > 256 || multi_buffers(D, RT) > 2) ? 1 : 2;
}

// The multi-token decode of one workgroup: `bid` is its index in the grid of chunks / 4
// workgroups; its LDS is s_pre [kMultiSeqs + 1], s_sum [kMW * kWave] and s_v (kMW V tiles
// of MLayout::LTILE bytes, 16-byte aligned).  Per wave: the state of RT row tiles (16 query
// rows each) of the current piece; NB tiles in flight.
template <int D, int RT, bool FP8, int NB = multi_buffers(D, RT)>
__device__ __forceinline__ void gqa_multi_body(const MultiArgs& a, int bid, int* s_pre,
                                               int* s_sum, uint8_t* s_v) {
  using Lo = MLayout<D, FP8>;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int i16 = lane & 15, gq = lane >> 4;
  const int B = a.B, G = a.Hq / a.Hkv, R = G * a.q_len;
  const int cap = min(a.max_blocks * a.block_size, a.max_len);
  auto seq_len = [&](int bi) {  // clamped to the table; one length for all in prefix mode
    int L = a.fixed_len >= 0 ? a.fixed_len : a.context_lens[bi];
    return L < 0 ? 0 : (L > cap ? cap : L);
  };

  // ---- tiles per sequence and their exclusive prefix, scanned across the workgroup
  auto ntiles = [&](int bi) { return (seq_len(bi) + kTile - 1) / kTile; };
  const int per = (B + kMW * kWave - 1) / (kMW * kWave);
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (tid * per + i < B) local += ntiles(tid * per + i);
  s_sum[tid] = local;
  __syncthreads();
  for (int off = 1; off < kMW * kWave; off <<= 1) {
    const int v = tid >= off ? s_sum[tid - off] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  int run = tid == 0 ? 0 : s_sum[tid - 1];
  for (int i = 0; i < per; ++i) {
    const int bi = tid * per + i;
    if (bi < B) {
      s_pre[bi] = run;
      run += ntiles(bi);
    }
  }
  if (tid == 0) s_pre[B] = s_sum[kMW * kWave - 1];
  __syncthreads();
  if (bid == 0) {
    for (int i = tid; i <= B; i += kMW * kWave) a.ws_prefix[i] = s_pre[i];
    write_segment_ranges(a.ws_seg, s_pre, B, a.Hkv, a.chunks, tid, kMW * kWave);
  }

  // ---- this wave's chunk (each XCD gets a contiguous eighth of the chunks)
  const int T_head = __builtin_amdgcn_readfirstlane(s_pre[B]);
  const long long T = (long long)a.Hkv * T_head;
  const int C = a.chunks;
  const int ch = (bid & 7) * (C / 8) + (bid >> 3) * kMW + w;
  const long long tb = T * ch / C, te = T * (ch + 1) / C;
  const int ntl = (int)min(te - tb, (long long)kMultiChunkTiles);
  if (ntl <= 0) return;

  // ---- per tile: byte offset / 256, valid tokens | segment << 5; and the first tile's
  // index inside its sequence
  const int tiles_per_block = a.block_size / kTile;
  const size_t head_bytes = (size_t)a.block_size * Lo::ROW;
  const size_t block_bytes = head_bytes * a.Hkv;
  uint32_t off_l[2] = {0, 0};
  int info_l[2] = {0, 0};
  int tt_l = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = kWave * j + lane;
    if (n < ntl) {
      const long long t = tb + n;
      const int gg = (int)(t / T_head);
      const int rem = (int)(t - (long long)gg * T_head);
      int lo = 0, hi = B - 1;  // last sequence whose first tile is <= rem
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= rem) lo = mid;
        else hi = mid - 1;
      }
      const int tt = rem - s_pre[lo];
      const int L = seq_len(lo);
      const int phys = a.block_table[(size_t)lo * a.table_stride + tt / tiles_per_block];
      const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
      const uint64_t off = (uint64_t)(ok ? phys : 0) * block_bytes + (uint64_t)gg * head_bytes +
                           (uint64_t)(tt % tiles_per_block) * Lo::TILE;
      off_l[j] = (uint32_t)(off >> 8);
      info_l[j] = (ok ? min(kTile, L - tt * kTile) : 0) | ((gg * B + lo) << 5);
      if (j == 0) tt_l = tt;
    }
  }
  const int tt_first = __builtin_amdgcn_readlane(tt_l, 0);
  auto pick = [](int j, int x0, int x1) { return j ? x1 : x0; };
  // Source of chunk tile n, or an empty one (all loads return zeros) for n >= end.
  auto tile_at = [&](int n, int end) -> TileSrc {
    if (n >= end) return TileSrc{make_rsrc(a.k_pool, 0), make_rsrc(a.v_pool, 0)};
    const int j = n >> 6, ln = n & (kWave - 1);
    const uint64_t off =
        (uint64_t)(uint32_t)__builtin_amdgcn_readlane(pick(j, (int)off_l[0], (int)off_l[1]), ln) << 8;
    const int nv = __builtin_amdgcn_readlane(pick(j, info_l[0], info_l[1]), ln) & 31;
    return TileSrc{make_rsrc(a.k_pool + off, nv * Lo::ROW), make_rsrc(a.v_pool + off, nv * Lo::ROW)};
  };
  auto tile_seg = [&](int n) {
    return __builtin_amdgcn_readlane(pick(n >> 6, info_l[0], info_l[1]), n & (kWave - 1)) >> 5;
  };
  uint64_t starts[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = kWave * j + lane;
    const int seg = info_l[j] >> 5;
    int prev = __shfl_up(seg, 1);
    if (lane == 0) prev = j ? __builtin_amdgcn_readlane(info_l[0], kWave - 1) >> 5 : -1;
    starts[j] = __builtin_amdgcn_ballot_w64(n < ntl && seg != prev);
  }
  auto next_start = [&](int n) {  // first piece start after tile n (or ntl)
    for (int j = (n + 1) >> 6; j < 2; ++j) {
      const int lo = (n + 1) - kWave * j;
      const uint64_t m = lo <= 0 ? starts[j] : (lo >= kWave ? 0 : starts[j] & (~0ull << lo));
      if (m) return kWave * j + (int)__builtin_ctzll(m);
    }
    return ntl;
  };

  // ---- LDS addresses of this lane's V writes and transposed reads
  uint8_t* sv = s_v + w * Lo::LTILE;
  const lds_char_t* lsv = (const lds_char_t*)((lds_void_t*)sv);
  // V load u of this lane holds 16 bytes at 1024 u + 16 lane of the tile: 8 bf16 (half a
  // 32-byte LDS piece) or 16 FP8 codes (a whole piece once widened to fp16)
  uint32_t vw_off[Lo::VL];
#pragma unroll
  for (int u = 0; u < Lo::VL; ++u) {
    const int gb = 1024 * u + 16 * lane, t = gb / Lo::ROW, e0 = (gb % Lo::ROW) / (FP8 ? 1 : 2);
    vw_off[u] = t * Lo::LROW + 32 * ((e0 >> 4) ^ vswz<D>(t)) + 2 * (e0 & 15);
  }
  const int tr_row = 4 * gq + (i16 >> 2);
  const uint32_t tr_base = tr_row * Lo::LROW + 8 * (i16 & 3);
  const int tr_swz = vswz<D>(tr_row);
  const uint32_t koff = k_offset<D, FP8>(i16, gq, 0);

  MTile<D, FP8> Rb[NB];
  for (int n0 = 0; n0 < ntl;) {
    const int n1 = next_start(n0);
    const int seg = tile_seg(n0), gg = seg / B, bb = seg - gg * B;
    const int L = seq_len(bb);
    const int t_first = (n0 == 0 ? tt_first : 0) * kTile;  // sequence position of tile n0
    const float cscale = a.scale * kLog2e * (FP8 ? a.k_scale[gg] : 1.f);
    const float vs = FP8 ? a.v_scale[gg] : 1.f;

    // q rows of the piece as the B operand; row limits relative to tile n0's first token
    bf16x8_t qf[RT][Lo::KS];
    int lim[RT];
    f32x4_t o[RT][Lo::NT];
    float m[RT], l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int n = 16 * rt + i16;
      const int jq = n / G;
      const bool real = n < R && bb * a.q_len + jq < a.q_rows;
      lim[rt] = real ? L - (a.causal ? a.q_len - 1 - jq : 0) - t_first : -1;
      const uint8_t* qrow =
          (const uint8_t*)(a.q + (((size_t)bb * a.q_len + (real ? jq : 0)) * a.Hq + (size_t)gg * G +
                                  (real ? n - jq * G : 0)) * D);
#pragma unroll
      for (int ks = 0; ks < Lo::KS; ++ks) {
        uint4 x = real ? *(const uint4*)(qrow + q_offset<D, FP8>(gq, ks)) : uint4{0, 0, 0, 0};
        qf[rt][ks] = __builtin_bit_cast(bf16x8_t, x);
      }
#pragma unroll
      for (int nt = 0; nt < Lo::NT; ++nt) o[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m[rt] = kNegInf;
      l[rt] = 0.f;
    }

    // One tile of the piece (held in X): scores, online softmax, V through LDS, p.V; X is
    // refilled with tile n_next (an empty tile past the piece's end).  pos0 = first token of
    // the tile relative to tile n0.
    auto step = [&](MTile<D, FP8>& X, int pos0, int n_next, int end) {
      f32x4_t s[RT];
      bf16x8_t kf[Lo::KS];
#pragma unroll
      for (int ks = 0; ks < Lo::KS; ++ks) kf[ks] = k_frag<D, FP8>(X, ks);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        s[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < Lo::KS; ++ks) s[rt] = mfma_qk(kf[ks], qf[rt][ks], s[rt]);
      }
      sched_fence();
      const TileSrc nx = tile_at(n_next, end);
      mload_k<D, FP8>(X, nx.k, koff);
      sched_fence();
      // scores of tokens pos0 + 4 gq + i for this lane's row; masked past the row's limit
      float mt[RT];
      bool up = false;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float x = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = (pos0 + 4 * gq + i < lim[rt]) ? s[rt][i] * cscale : kNegInf;
          s[rt][i] = v;
          x = fmaxf(x, v);
        }
        mt[rt] = max4(x);
        up |= mt[rt] > m[rt] + kRescaleSlack;
      }
      if (wave_any(up)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float m_new = fmaxf(m[rt], mt[rt]);
          const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m[rt] - m_new);
          l[rt] *= alpha;
          m[rt] = m_new;
#pragma unroll
          for (int nt = 0; nt < Lo::NT; ++nt) o[rt][nt] *= alpha;
        }
      }
      f16x4_t p[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float mu = (m[rt] == kNegInf) ? 0.f : m[rt];
        const uint32_t p01 = pack_f16(fast_exp2(s[rt][0] - mu), fast_exp2(s[rt][1] - mu));
        const uint32_t p23 = pack_f16(fast_exp2(s[rt][2] - mu), fast_exp2(s[rt][3] - mu));
        l[rt] = dot2h(p01, kOnesF16x2, l[rt]);
        l[rt] = dot2h(p23, kOnesF16x2, l[rt]);
        p[rt] = __builtin_bit_cast(f16x4_t, uint2{p01, p23});
      }
      // V tile -> LDS (token-major, swizzled; FP8 codes widened to fp16 on the way), then
      // refill X.v with the next tile
#pragma unroll
      for (int u = 0; u < Lo::VL; ++u) {
        if constexpr (FP8) {
          const uint4 x = X.v[u];
          *(uint4*)(sv + vw_off[u]) = uint4{fp8x2_to_f16x2<false>(x.x), fp8x2_to_f16x2<true>(x.x),
                                            fp8x2_to_f16x2<false>(x.y), fp8x2_to_f16x2<true>(x.y)};
          *(uint4*)(sv + vw_off[u] + 16) = uint4{fp8x2_to_f16x2<false>(x.z), fp8x2_to_f16x2<true>(x.z),
                                                 fp8x2_to_f16x2<false>(x.w), fp8x2_to_f16x2<true>(x.w)};
        } else {
          *(uint4*)(sv + vw_off[u]) = X.v[u];
        }
      }
      sched_fence();
      mload_v<D, FP8>(X, nx.v, lane);
      sched_fence();
#pragma unroll
      for (int nt = 0; nt < Lo::NT; ++nt) {
        const uint2 raw = __builtin_bit_cast(
            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                       (lds_s16x4_t*)(lsv + tr_base + 32 * (nt ^ tr_swz))));
        const f16x4_t vf = FP8 ? __builtin_bit_cast(f16x4_t, raw)
                               : __builtin_bit_cast(
                                     f16x4_t, uint2{pack_f16(bf16_lo(raw.x), bf16_hi(raw.x)),
                                                    pack_f16(bf16_lo(raw.y), bf16_hi(raw.y))});
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[rt][nt] = mfma_pv(vf, p[rt], o[rt][nt]);
      }
    };

    // tile n lives in buffer (n - n0) % NB; loads are issued in tile order (the scheduling
    // fences keep it), so the waits the compiler derives stay exact
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const TileSrc S = tile_at(n0 + b, n1);
      mload_k<D, FP8>(Rb[b], S.k, koff);
      sched_fence();
      mload_v<D, FP8>(Rb[b], S.v, lane);
      sched_fence();
    }
    int n = n0;
    for (; n + NB - 1 < n1; n += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) step(Rb[b], kTile * (n + b - n0), n + b + NB, n1);
    }
#pragma unroll
    for (int b = 0; b < NB - 1; ++b)
      if (n + b < n1) step(Rb[b], kTile * (n + b - n0), n + b + NB, n1);

    // ---- the piece: rows n < R of slot ch + seg
    const size_t slot = (size_t)ch + seg;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int nrow = 16 * rt + i16;
      const float lt = sum4(l[rt]);
      if (nrow < R) {
        float* orow = a.ws_o + (slot * R + nrow) * D + 4 * gq;
#pragma unroll
        for (int nt = 0; nt < Lo::NT; ++nt)
          *(float4*)(orow + 16 * nt) =
              make_float4(o[rt][nt][0] * vs, o[rt][nt][1] * vs, o[rt][nt][2] * vs, o[rt][nt][3] * vs);
        if (gq == 0) {
          a.ws_m[slot * R + nrow] = m[rt];
          a.ws_l[slot * R + nrow] = lt;
        }
      }
    }
    n0 = n1;
  }
}

}  // namespace pkv
