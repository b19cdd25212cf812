// Multi-token (speculative verify) decode streamed through an LDS ring: the division of work
// and the tile stream of the single-token ring kernel (gqa_ring_body.hpp), the arithmetic of
// the multi-token kernel (gqa_multi_body.hpp: scores S^T = K Q^T and O^T += V^T P^T on the
// matrix cores, q_len * G query rows per KV head).
//
// "深入LLM推理：从KV Cache到PD分离的Serving全景解析", section "投机解码：打破每步一token的假设":
// the target model checks the drafted tokens in one pass over the cache.
//
// What the ring changes: K and V tiles, and the q rows of each piece, are copied HBM -> LDS
// by LDS-direct buffer loads (no registers), two tiles per wave in flight, and the MFMA
// operands are read from the ring: K as the A operand of the scores (16-byte reads), V^T as
// the A operand of p.V (transposed 8-byte reads), q as the B operand once per piece.  One
// wave per SIMD (4 per CU), so a CU holds 1024 chunks' worth of waves and the pieces are
// half as many as with the register-tile kernel's 8.  bf16 K/V, d = 128, up to 32 rows.
#pragma once

#include "gqa_multi_body.hpp"
#include "gqa_ring_body.hpp"

namespace pkv {

// Ring of one wave: kMRingSlots slots of [K tile | V tile], then as many q slots of RT*16
// rows.  Rows are 256 bytes (bf16, d = 128).  Inside the K tile and the q slots the 16-byte
// chunk c of row t sits at c ^ (t & 15), so a 16-lane group reading one chunk of 16 rows
// meets 16 distinct bank slots (and lanes l, l + 16 read slots that agree in bits 2 and 3);
// inside the V tile the 32-byte piece p of row t sits at p ^ (t & 7), so each 32-lane half
// of a transposed read meets 32 distinct 8-byte bank pairs.
constexpr int kMRingSlots = 2;
template <int RT>
struct MRing {
  static constexpr int ROW = 256;                    // bf16 row of 128 dims
  static constexpr int TILE = kTile * ROW;           // 4 KiB
  static constexpr int COPIES = TILE / 1024;         // LDS-direct copies per K (or V) tile
  static constexpr int LOADS = 2 * COPIES;           // vector-memory ops per tile
  static constexpr int SLOT = 2 * TILE;
  static constexpr int QROWS = 16 * RT;
  static constexpr int QSLOT = QROWS * ROW;
  static constexpr int QCOPIES = QSLOT / 1024;
  static constexpr int WAVE_BYTES = kMRingSlots * (SLOT + QSLOT);
};
template <int RT>
constexpr int multi_ring_lds_bytes() {
  return kRingWaves * MRing<RT>::WAVE_BYTES > kRingPrefixBytes ? kRingWaves * MRing<RT>::WAVE_BYTES
                                                                : kRingPrefixBytes;
}

template <int RT>
__device__ __forceinline__ void gqa_multi_ring_body(const MultiArgs& a, int bid, lds_u8_t* lds) {
  constexpr int D = 128, NS = kMRingSlots, WPG = kRingWaves;
  using M = MRing<RT>;
  constexpr int KS = D / 32, NTD = D / 16;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int i16 = lane & 15, gq = lane >> 4;
  const int B = a.B, G = a.Hq / a.Hkv, R = G * a.q_len;

  const RingWalk gw{a.fixed_len >= 0 ? nullptr : a.context_lens, a.fixed_len, a.block_table,
                    (size_t)a.table_stride, B, a.Hkv, a.block_size, a.num_blocks,
                    min(a.max_blocks * a.block_size, a.max_len), a.chunks, a.ws_prefix, a.ws_seg,
                    a.xcd8};
  RingTiles tl;
  // XCD-weighted ranges for large calls
  ring_setup<M::ROW, WPG, true, RingWeights<RT>>(gw, bid, lds, true, tl);
  const int ntl = tl.ntl, ch = tl.ch;
  if (ntl <= 0) return;
  uint32_t (&off_l)[kRingTilesPerLane] = tl.off;
  int (&info_l)[kRingTilesPerLane] = tl.info;
  int (&len_l)[kRingTilesPerLane] = tl.len;
  uint64_t (&starts)[kRingTilesPerLane] = tl.starts;

  // ---- LDS: this wave's ring; per-lane copy sources and read offsets
  lds_u8_t* const ring = lds + w * M::WAVE_BYTES;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
  uint32_t ksrc[M::COPIES], vsrc[M::COPIES], qsrc[M::QCOPIES];
#pragma unroll
  for (int j = 0; j < M::COPIES; ++j) {
    const uint32_t t = 4 * j + (lane >> 4), p = lane & 15;  // copy j, lane: row t, 16-byte slot p
    ksrc[j] = t * M::ROW + 16 * (p ^ (t & 15));
    vsrc[j] = t * M::ROW + 32 * ((p >> 1) ^ (t & 7)) + 16 * (p & 1);
  }
  // q row n of a piece (query token n / G, head n % G of the group) from the rows of the
  // piece's sequence; rows past R read past the range: zeros
#pragma unroll
  for (int j = 0; j < M::QCOPIES; ++j) {
    const int n = 4 * j + (lane >> 4), p = lane & 15;
    const int jq = n / G, h = n - jq * G;
    qsrc[j] = n < R ? (uint32_t)((jq * a.Hq + h) * D * 2 + 16 * (p ^ (n & 15))) : 0xFFFFFFF0u;
  }
  const uint32_t q_bytes = (uint32_t)(((a.q_len - 1) * a.Hq + G) * D * 2);
  const int tr_row = 4 * gq + (i16 >> 2);
  const uint32_t tr_base = M::TILE + tr_row * M::ROW + 8 * (i16 & 3);
  const int tr_swz = tr_row & 7;

  auto next_block = [&]() {
#pragma unroll
    for (int q = 0; q + 1 < kRingTilesPerLane; ++q) {
      info_l[q] = info_l[q + 1];
      off_l[q] = off_l[q + 1];
      len_l[q] = len_l[q + 1];
      starts[q] = starts[q + 1];
    }
    info_l[kRingTilesPerLane - 1] = 0;
    off_l[kRingTilesPerLane - 1] = 0;
    len_l[kRingTilesPerLane - 1] = 0;
    starts[kRingTilesPerLane - 1] = 0;
  };
  // Copies of tile `p` of the current block (p >= 64: the next block) into slot s, preceded
  // by its piece's q rows into q slot qs when it opens a piece.
  auto copy_tile = [&](int info, uint64_t off, bool opens, int s, int& qs) {
    if (opens) {
      const int sg = info >> 5, gg = sg / B, bb = sg - gg * B;
      const uint16_t* qg = a.q + (((size_t)bb * a.q_len) * a.Hq + (size_t)gg * G) * D;
      const i32x4_t qr = ring_rsrc(qg, q_bytes);
      const uint32_t qd = ring_addr + NS * M::SLOT + qs * M::QSLOT;
#pragma unroll
      for (int j = 0; j < M::QCOPIES; ++j) ring_copy16(qr, qsrc[j], qd + 1024 * j);
      qs = qs + 1 == NS ? 0 : qs + 1;
    }
    const uint32_t bytes = (uint32_t)(info & 31) * M::ROW;
    const i32x4_t kr = ring_rsrc(a.k_pool + off, bytes);
    const i32x4_t vr = ring_rsrc(a.v_pool + off, bytes);
    const uint32_t sd = ring_addr + s * M::SLOT;
#pragma unroll
    for (int j = 0; j < M::COPIES; ++j) ring_copy16(kr, ksrc[j], sd + 1024 * j);
#pragma unroll
    for (int j = 0; j < M::COPIES; ++j) ring_copy16(vr, vsrc[j], sd + M::TILE + 1024 * j);
  };
  auto issue = [&](int ln, int s, bool opens, int& qs) {
    const int p = ln + NS, pl = p & (kWave - 1);
    const bool nb = p >= kWave;
    const int info = __builtin_amdgcn_readlane(nb ? info_l[1] : info_l[0], pl);
    const uint64_t off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(nb ? off_l[1] : off_l[0]), pl) << 8;
    copy_tile(info, off, opens, s, qs);
  };

  int q_issue = 0, q_read = 0;
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int info = __builtin_amdgcn_readlane(info_l[0], t);
    const uint64_t off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_l[0], t) << 8;
    copy_tile(info, off, (starts[0] >> t) & 1, t, q_issue);
  }

  // state of the open piece
  bf16x8_t qf[RT][KS];
  f32x4_t o[RT][NTD];
  float m[RT], l[RT];
  int lim[RT];
  int seg = 0, n0 = 0, t_first = 0;
  const float cscale = a.scale * kLog2e;
  constexpr uint64_t kAheadMask = ((1ull << NS) - 1) & ~1ull;
  int s = 0;
  for (int n = 0; n < ntl; ++n) {
    const int ln = n & (kWave - 1);
    if (ln == 0 && n) next_block();
    const uint64_t win = (starts[0] >> ln) | (ln ? starts[1] << (kWave - ln) : 0ull);
    wait_vm_dyn<(NS - 1) * M::LOADS, M::QCOPIES, NS - 1>(__builtin_popcountll(win & kAheadMask));
    compiler_fence();
    const lds_u8_t* sp = ring + s * M::SLOT;
    bf16x8_t kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = __builtin_bit_cast(bf16x8_t, lds_ld16(sp, i16 * M::ROW + 16 * ((4 * ks + gq) ^ i16)));
    uint2 vraw[NTD];
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt)
      vraw[nt] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (lds_s16x4_t*)(sp + tr_base + 32 * (nt ^ tr_swz))));
    if (win & 1) {  // tile n opens a piece: its q rows, row limits, cleared state
      const int info = __builtin_amdgcn_readlane(info_l[0], ln);
      seg = info >> 5;
      const int gg = seg / B, bb = seg - gg * B;
      const int L = __builtin_amdgcn_readlane(len_l[0], ln);
      t_first = (n == 0 ? tl.tt_first : 0) * kTile;
      n0 = n;
      const lds_u8_t* qp = ring + NS * M::SLOT + q_read * M::QSLOT;
      q_read = q_read + 1 == NS ? 0 : q_read + 1;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int nr = 16 * rt + i16, jq = nr / G;
        const bool real = nr < R && bb * a.q_len + jq < a.q_rows;
        lim[rt] = real ? L - (a.causal ? a.q_len - 1 - jq : 0) - t_first : -1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qf[rt][ks] = __builtin_bit_cast(bf16x8_t, lds_ld16(qp, nr * M::ROW + 16 * ((4 * ks + gq) ^ i16)));
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt) o[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m[rt] = kNegInf;
        l[rt] = 0.f;
      }
    }
    // every LDS read of the slot (and of the q slot) is complete before it is refilled
    __builtin_amdgcn_s_waitcnt(0xC07F);
    compiler_fence();
    issue(ln, s, (win >> NS) & 1, q_issue);
    s = s + 1 == NS ? 0 : s + 1;

    // scores of tokens pos0 + 4 gq + i for this lane's row, masked past the row's limit
    const int pos0 = kTile * (n - n0);
    f32x4_t sc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      sc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sc[rt] = mfma_qk(kf[ks], qf[rt][ks], sc[rt]);
    }
    float mt[RT];
    bool up = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (pos0 + 4 * gq + i < lim[rt]) ? sc[rt][i] * cscale : kNegInf;
        sc[rt][i] = v;
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
        for (int nt = 0; nt < NTD; ++nt) o[rt][nt] *= alpha;
      }
    }
    f16x4_t pf[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float mu = (m[rt] == kNegInf) ? 0.f : m[rt];
      const uint32_t p01 = pack_f16(fast_exp2(sc[rt][0] - mu), fast_exp2(sc[rt][1] - mu));
      const uint32_t p23 = pack_f16(fast_exp2(sc[rt][2] - mu), fast_exp2(sc[rt][3] - mu));
      l[rt] = dot2h(p01, kOnesF16x2, l[rt]);
      l[rt] = dot2h(p23, kOnesF16x2, l[rt]);
      pf[rt] = __builtin_bit_cast(f16x4_t, uint2{p01, p23});
    }
    // p.V: V^T of 4 tokens of dim 16 nt + i16 per lane, bf16 widened to fp16 (exact for
    // 2^-14 <= |v| < 65504)
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt) {
      const f16x4_t vf = __builtin_bit_cast(
          f16x4_t, uint2{pack_f16(bf16_lo(vraw[nt].x), bf16_hi(vraw[nt].x)),
                         pack_f16(bf16_lo(vraw[nt].y), bf16_hi(vraw[nt].y))});
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) o[rt][nt] = mfma_pv(vf, pf[rt], o[rt][nt]);
    }

    if (n + 1 >= ntl || ((win >> 1) & 1)) {  // end of a piece: rows n < R of slot ch + seg
      const size_t slot = (size_t)ch + seg;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int nrow = 16 * rt + i16;
        const float lt = sum4(l[rt]);
        if (nrow < R) {
          float* orow = a.ws_o + (slot * R + nrow) * D + 4 * gq;
#pragma unroll
          for (int nt = 0; nt < NTD; ++nt)
            *(float4*)(orow + 16 * nt) = make_float4(o[rt][nt][0], o[rt][nt][1], o[rt][nt][2], o[rt][nt][3]);
          if (gq == 0) {
            a.ws_m[slot * R + nrow] = m[rt];
            a.ws_l[slot * R + nrow] = lt;
          }
        }
      }
    }
  }
  // no copy may still be writing this workgroup's LDS when it ends
  wait_vm<0>();
}

}  // namespace pkv
