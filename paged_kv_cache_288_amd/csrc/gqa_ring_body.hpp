// Balanced single-token GQA decode with an LDS ring (the body of gqa_stream_kernel).
//
// Division of work as in gqa_stream_body.hpp: the 16-token tiles of all (KV head, sequence)
// segments laid end to end, head-major, cut into `chunks` ranges, one per wave, and a
// piece of (m, l, o) partials written wherever a range meets a segment.  For large calls
// the ranges are weighted by XCD (xcd_chunk_start).  What differs is how a wave is fed.
// One workgroup runs per CU, of 4 waves (one per SIMD, so no wave waits behind another for
// its loads) or, for light tiles, 8 waves (two per SIMD).  Each wave streams its range
// through a ring of NS tile slots in LDS, filled by buffer loads that write LDS directly
// (no registers): the K and V rows of tile n + NS are requested as soon as tile n has
// been read out of its slot, whether or not n + NS belongs to the same piece.  The q rows
// of a piece are copied the same way, just before the piece's first tile, into one of
// NS q slots, so a piece boundary never drains the loads in flight.  The arithmetic of a
// tile (scores, online softmax, p.V, merge of row groups) is that of gqa_tile.hpp.
//
// Reading the pages: "GPU推理深度拆解：KV Cache视角", section "性能指标与瓶颈" (decode is bound by
// memory bandwidth, so the measure is the fraction of it reached), and "PD 分离下的 KV Cache",
// section "先回顾：LLM 推理的两个阶段" (every decode step reads the whole cache once).
#pragma once

#include "gqa_tile.hpp"

namespace pkv {

constexpr int kRing = 2;           // tiles in flight per wave (default)
constexpr int kRingWaves = 4;      // waves per workgroup, one workgroup per CU (default)
constexpr int kRingTilesPerLane = 8;
constexpr int kRingMaxChunkTiles = kWave * kRingTilesPerLane;  // 512
constexpr int kRingMaxSeqs = 4096;

// Ranges weighted by XCD (xcd_chunk_start in pkv_device.hpp) when the 4-wave shape's
// chunks hold at least kRingWeightMinTiles tiles on average (with fewer, as for a few
// 32K-token sequences, the weighting was measured to cost more than it saved).  Only in
// the 4-wave shape, whose heavy tiles stream from HBM: the 8-wave shape serves groups whose
// tiles are light, where a shared prefix re-read from each XCD's own L2 sets the pace.
constexpr int kRingWeightMinTiles = 128;
// XCD weights (parts of the tiles per chunk on even : odd XCDs) by kernel, RT its MFMA row
// tiles (0: the VALU ring).  Single-token calls, on the VALU ring or on the MFMA ring with
// one 16-row tile, take 17:15 (on the 70B-shaped batch 18:14 and 33:31 measured 2-6 us
// slower per call with the VALU ring, and 33:31 about 1.3 us slower with the MFMA ring);
// the MFMA ring with two row tiles (32 query rows: the verify pass), whose tiles carry more
// arithmetic per byte, 33:31 (17:15 and even ranges 1-2 us slower per verify call, 18:14
// too).
template <int RT>
struct RingWeights {
  static constexpr int E = RT >= 2 ? 33 : 17, O = RT >= 2 ? 31 : 15;
};

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) const u32x2_t lds_u32x2_t;

// 16 (8) bytes of LDS at a 16 (8) byte aligned offset from a 16-byte aligned base.
__device__ __forceinline__ uint4 lds_ld16(const lds_u8_t* base, uint32_t off) {
  const u32x4_t v = ((lds_u32x4_t*)base)[off >> 4];
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint2 lds_ld8(const lds_u8_t* base, uint32_t off) {
  const u32x2_t v = ((lds_u32x2_t*)base)[off >> 3];
  return uint2{v[0], v[1]};
}

// Index (0..7) of the XCD running this wave, from the XCC_ID hardware register.
__device__ __forceinline__ int xcd_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return (int)(x & 7u);
}

// Raw buffer resource words over [base, base + bytes), for loads issued from assembly.
__device__ __forceinline__ i32x4_t ring_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return i32x4_t{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), (int)bytes,
                 kRawBufferWord3};
}
// 16 bytes per lane from byte offset voff of the buffer into LDS at lds_addr + 16 * lane,
// nontemporal.  Offsets past the buffer's range write zeros without touching memory.  The
// leading s_nop 4 covers the wait states between an SGPR written by a VALU instruction
// (readlane) and a vector-memory read of it, and M0's.
__device__ __forceinline__ void ring_copy16(i32x4_t rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc),
               "{m0}"(lds_addr)
               : "memory");
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// LDS layout of one wave's ring: NS slots of [K tile | V tile], then NS q slots.
// Inside a slot the K rows of 256 bytes (bf16, d = 128) have their two 128-byte halves
// swapped on odd tokens, and the V rows of 128 bytes (FP8, d = 128) are stored at row
// t ^ ((t >> 1) & 1): with those, every 16-lane group of the K reads and every 32-lane
// group of the 8-byte V reads meets distinct LDS banks.  Other rows are stored as they are.
template <int D, int G, bool FP8, int NS = kRing>
struct Ring {
  using Lo = Layout<D, FP8>;
  static constexpr int TILE = kTile * Lo::ROW;            // bytes of a K (or V) tile
  static constexpr int COPIES = TILE / 1024;              // LDS-direct copies per K (or V) tile
  static constexpr int QB = G * D * 2;                    // q rows of a head group (bf16)
  static constexpr int QSLOT = QB < 1024 ? 1024 : QB;     // a copy writes whole KiB
  static constexpr int QCOPIES = QSLOT / 1024;
  static constexpr int SLOT = 2 * TILE;
  static constexpr int WAVE_BYTES = NS * (SLOT + QSLOT);
  static constexpr int LOADS = 2 * COPIES;                // vector-memory ops per tile
  static_assert(TILE % 1024 == 0 && (QB % 1024 == 0 || QB < 1024), "copy granularity");
  static constexpr bool KSWZ = (Lo::ROW == 256);
  static constexpr bool VSWZ = FP8;
};

// LDS of a workgroup: the rings, or the tile prefix of the set-up when that is larger.
constexpr int kRingPrefixBytes = (2 * kRingMaxSeqs + 1 + 16) * 4;
template <int D, int G, bool FP8, int NS = kRing, int WPG = kRingWaves>
constexpr int ring_lds_bytes() {
  return WPG * Ring<D, G, FP8, NS>::WAVE_BYTES > kRingPrefixBytes
             ? WPG * Ring<D, G, FP8, NS>::WAVE_BYTES
             : kRingPrefixBytes;
}

// Source offset inside a tile of the byte that lands at LDS byte x of the K (kv = 0) or V
// (kv = 1) part of a slot.
template <int D, int G, bool FP8>
__device__ __forceinline__ uint32_t ring_src(uint32_t x, int kv) {
  using R = Ring<D, G, FP8, 1>;
  using Lo = Layout<D, FP8>;
  const uint32_t t = x / Lo::ROW, b = x % Lo::ROW;
  if (kv == 0 && R::KSWZ) return t * Lo::ROW + (b ^ (128u * (t & 1u)));
  if (kv == 1 && R::VSWZ) return (t ^ ((t >> 1) & 1u)) * Lo::ROW + b;
  return x;
}

// Wait until at most N vector-memory operations of this wave are outstanding, N one of a
// few values known only at run time (the q copies in the window vary).
template <int BASE, int STEP, int MAXK>
__device__ __forceinline__ void wait_vm_dyn(int k) {
  static_assert(BASE + STEP * MAXK < 64, "vmcnt range");
  if constexpr (MAXK >= 3) {
    if (k >= 3) { wait_vm<BASE + 3 * STEP>(); return; }
  }
  if constexpr (MAXK >= 2) {
    if (k >= 2) { wait_vm<BASE + 2 * STEP>(); return; }
  }
  if constexpr (MAXK >= 1) {
    if (k >= 1) { wait_vm<BASE + STEP>(); return; }
  }
  wait_vm<BASE>();
}

// ---- set-up of a ring walk, common to the single- and the multi-token ring kernels
struct RingWalk {
  const int32_t* context_lens;  // per-sequence lengths, or nullptr: every sequence fixed_len
  int fixed_len;
  const int32_t* block_table;
  size_t table_stride;          // elements between the rows of sequences (0: one shared row)
  int B, Hkv, block_size, num_blocks;
  int cap;                      // lengths are clamped to [0, cap]
  int chunks;
  int32_t* ws_prefix;           // written by workgroup 0: tile prefix [B + 1]
  int32_t* ws_seg;              //   and per segment its first chunk and chunk count
  int xcd8;                     // the grid is spread over 8 XCDs in turn (weighting by XCD id)
};
// One wave's chunk: per lane, kRingTilesPerLane tiles (tile n of the chunk in entry n / 64 of
// lane n % 64): byte offset / 256 of its first row in the pools, valid tokens | segment << 5,
// and one bit per tile that opens a piece (its segment differs from the previous tile's).
struct RingTiles {
  uint32_t off[kRingTilesPerLane];
  int info[kRingTilesPerLane];
  int len[kRingTilesPerLane];  // length of the tile's sequence (clamped)
  uint64_t starts[kRingTilesPerLane];
  int ntl;       // tiles in the chunk
  int ch;        // the chunk
  int tt_first;  // index inside its sequence of the chunk's first tile
};
// Tiles per sequence and their exclusive prefix in LDS (which the ring aliases: the function
// ends with a workgroup barrier after its last LDS read), this wave's chunk (XCD-weighted
// when `may_weight` and the call is large), and the tables.  ROW = bytes per K or V row;
// MULTI: also the lengths and the first tile's index (RingTiles::len, tt_first), and lengths
// from fixed_len when context_lens is null (the single-token kernel needs none of these).
template <int ROW, int WPG, bool MULTI, typename Wt>
__device__ __forceinline__ void ring_setup(const RingWalk& g, int bid, lds_u8_t* lds,
                                           bool may_weight, RingTiles& t) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int B = g.B;
  const int cap = g.cap;
  constexpr int NT = WPG * kWave;
  __attribute__((address_space(3))) int* s_pre =
      (__attribute__((address_space(3))) int*)lds;        // [B + 1]
  __attribute__((address_space(3))) int* s_len = s_pre + (kRingMaxSeqs + 1);  // [B] lengths
  __attribute__((address_space(3))) int* s_wsum = s_len + kRingMaxSeqs;        // [WPG]
  const int per = (B + NT - 1) / NT;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int bi = tid * per + i;
    if (bi < B) {
      int L = (!MULTI || g.context_lens) ? g.context_lens[bi] : g.fixed_len;
      L = L < 0 ? 0 : (L > cap ? cap : L);
      s_len[bi] = L;
      local += (L + kTile - 1) / kTile;
    }
  }
  // inclusive scan of `local` over the workgroup: within the wave, then across waves
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) s_wsum[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < w; ++i) wbase += s_wsum[i];
  int run = wbase + incl - local;
  for (int i = 0; i < per; ++i) {
    const int bi = tid * per + i;
    if (bi < B) {
      s_pre[bi] = run;
      run += (s_len[bi] + kTile - 1) / kTile;
    }
  }
  if (tid == NT - 1) s_pre[B] = run;
  __syncthreads();
  const int T_head = __builtin_amdgcn_readfirstlane(s_pre[B]);
  const long long T = (long long)g.Hkv * T_head;
  const int C = g.chunks;
  const bool wtd =
      may_weight && xcd_weighted<Wt::E, Wt::O>(T, C, kRingWeightMinTiles, kRingMaxChunkTiles);
  if (bid == 0) {
    for (int i = tid; i <= B; i += NT) g.ws_prefix[i] = s_pre[i];
    write_segment_ranges_xcd<Wt::E, Wt::O>(g.ws_seg, s_pre, B, g.Hkv, C, wtd, tid, NT);
  }

  // ---- this wave's chunk and, per lane, kRingTilesPerLane tiles' offset, length, segment
  // The workgroup's eighth of the chunks is bid mod 8.  Workgroups go to the 8 XCDs in turn,
  // but which XCD takes workgroup 0 depends on the dispatches before this one, so weighted
  // ranges (the heavier eighths meant for even XCDs) take the parity from the XCD that runs
  // the workgroup: eighth (bid mod 8) xor f, f = (XCD id xor bid) & 1.  Workgroups 2j and
  // 2j + 1 run on neighbouring XCDs, so both find the same f and still share the two eighths
  // 2j mod 8 and 2j mod 8 + 1 between them.
  int eighth = bid & 7;
  if (wtd && g.xcd8) eighth ^= (xcd_id() ^ bid) & 1;
  const int ch = eighth * (C / 8) + (bid >> 3) * WPG + w;
  const long long tb = xcd_chunk_start<Wt::E, Wt::O>(ch, T, C, wtd),
                  te = xcd_chunk_start<Wt::E, Wt::O>(ch + 1, T, C, wtd);
  const int ntl = (int)min(te - tb, (long long)kRingMaxChunkTiles);
  t.ntl = ntl;
  t.ch = ch;

  const int tiles_per_block = g.block_size / kTile;
  const size_t head_bytes = (size_t)g.block_size * ROW;
  const size_t block_bytes = head_bytes * g.Hkv;
  int tt_l = 0;
  {
    // head and tile-in-head of the lane's tiles: the chunk starts at head gg0, tile rem0 of
    // it, and a lane's tile lies fewer than kRingMaxChunkTiles tiles further
    const int Th = T_head > 0 ? T_head : 1;
    const int gg0 = (int)(tb / Th), rem0 = (int)(tb - (long long)gg0 * Th);
    int lo_[kRingTilesPerLane], rem_[kRingTilesPerLane], gg_[kRingTilesPerLane];
#pragma unroll
    for (int j = 0; j < kRingTilesPerLane; ++j) {
      const uint32_t rr = (uint32_t)rem0 + kWave * j + lane;
      if (Th >= kRingMaxChunkTiles) {  // at most one head boundary inside a chunk
        const bool past = rr >= (uint32_t)Th;
        gg_[j] = gg0 + past;
        rem_[j] = (int)(past ? rr - Th : rr);
      } else {
        gg_[j] = gg0 + (int)(rr / (uint32_t)Th);
        rem_[j] = (int)(rr % (uint32_t)Th);
      }
      lo_[j] = 0;
    }
    // last sequence whose first tile is <= rem, for all of the lane's tiles at once
    int hi_[kRingTilesPerLane];
#pragma unroll
    for (int j = 0; j < kRingTilesPerLane; ++j) hi_[j] = B - 1;
    // branch-free: with lo == hi, mid = lo and s_pre[lo] <= rem, so a step changes nothing
#pragma unroll 1
    for (int step = 0; step < 13; ++step) {
      bool any = false;
#pragma unroll
      for (int j = 0; j < kRingTilesPerLane; ++j) {
        const int mid = (lo_[j] + hi_[j] + 1) >> 1;
        const bool go = s_pre[mid] <= rem_[j];
        lo_[j] = go ? mid : lo_[j];
        hi_[j] = go ? hi_[j] : mid - 1;
        any |= lo_[j] < hi_[j];
      }
      if (!wave_any(any)) break;
    }
#pragma unroll
    for (int j = 0; j < kRingTilesPerLane; ++j) {
      t.off[j] = 0;
      t.info[j] = 0;
      if constexpr (MULTI) t.len[j] = 0;
      const int n = kWave * j + lane;
      if (n < ntl) {
        const int tt = rem_[j] - s_pre[lo_[j]];
        if (MULTI && j == 0) tt_l = tt;
        const int L = s_len[lo_[j]];
        const int blk = tiles_per_block == 1 ? tt : tt / tiles_per_block;
        const int tin = tiles_per_block == 1 ? 0 : tt - blk * tiles_per_block;
        const int phys = g.block_table[(size_t)lo_[j] * g.table_stride + blk];
        const bool ok = (unsigned)phys < (unsigned)g.num_blocks;
        const uint64_t off = (uint64_t)(ok ? phys : 0) * block_bytes +
                             (uint64_t)gg_[j] * head_bytes +
                             (uint64_t)tin * (kTile * ROW);
        t.off[j] = (uint32_t)(off >> 8);
        t.info[j] = (ok ? min(kTile, L - tt * kTile) : 0) | ((gg_[j] * B + lo_[j]) << 5);
        if constexpr (MULTI) t.len[j] = L;
      }
    }
  }
  if constexpr (MULTI) t.tt_first = __builtin_amdgcn_readlane(tt_l, 0);
  // the prefix area is reused by the ring from here on
  __syncthreads();

#pragma unroll
  for (int j = 0; j < kRingTilesPerLane; ++j) {
    const int n = kWave * j + lane;
    const int sg = t.info[j] >> 5;
    int prev = __shfl_up(sg, 1);
    if (lane == 0) prev = j ? __builtin_amdgcn_readlane(t.info[j - 1], kWave - 1) >> 5 : -1;
    t.starts[j] = __builtin_amdgcn_ballot_w64(n < ntl && sg != prev);
  }
}

template <int D, int G, bool FP8, int NS = kRing, int WPG = kRingWaves>
__device__ __forceinline__ void gqa_ring_body(const DecodeArgs& a, int bid, lds_u8_t* lds) {
  using Lo = Layout<D, FP8>;
  using R = Ring<D, G, FP8, NS>;
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  static_assert(WPG == 4 || WPG == 8, "waves per workgroup");
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int k = lane >> 3, c = lane & 7, r = lane / Lo::LPT, dc = lane % Lo::LPT;
  const int B = a.B;
  const RingWalk gw{a.context_lens, 0, a.block_table, (size_t)a.max_blocks, B, a.Hkv, a.block_size,
                    a.num_blocks, min(a.max_blocks * a.block_size, a.max_context_len), a.chunks,
                    a.ws_prefix, a.ws_seg, a.xcd8};
  RingTiles tl;
  ring_setup<Lo::ROW, WPG, false, RingWeights<0>>(gw, bid, lds, WPG == 4, tl);
  const int ntl = tl.ntl, ch = tl.ch;
  if (ntl <= 0) return;
  uint32_t (&off_l)[kRingTilesPerLane] = tl.off;
  int (&info_l)[kRingTilesPerLane] = tl.info;
  uint64_t (&starts)[kRingTilesPerLane] = tl.starts;

  // ---- LDS: this wave's ring and q slots; per-lane copy and read offsets
  lds_u8_t* const ring = lds + w * R::WAVE_BYTES;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
  uint32_t ksrc[R::COPIES], vsrc[R::COPIES];
#pragma unroll
  for (int j = 0; j < R::COPIES; ++j) {
    ksrc[j] = ring_src<D, G, FP8>(1024 * j + 16 * lane, 0);
    vsrc[j] = ring_src<D, G, FP8>(1024 * j + 16 * lane, 1);
  }
  // K reads: token 8 pi + k, bytes 16 c + 128 j of the row; with the odd-token swap of the
  // 128-byte halves the two j of a lane sit at kb[0] and kb[1] (+ 8 rows for pi = 1)
  uint32_t kb[Lo::KL];
#pragma unroll
  for (int j = 0; j < Lo::KL; ++j) {
    const uint32_t g = 16 * c + 128 * j;
    kb[j] = k * Lo::ROW + (R::KSWZ ? (g ^ (128u * (k & 1))) : g);
  }
  // V reads: token pv_token(u, r) (row-permuted for FP8), bytes dc * VB
  uint32_t vrd[Lo::TPG];
#pragma unroll
  for (int u = 0; u < Lo::TPG; ++u) {
    const uint32_t t = pv_token<D>(u, r);
    vrd[u] = R::TILE + (R::VSWZ ? (t ^ ((t >> 1) & 1u)) : t) * Lo::ROW + dc * Lo::VB;
  }
  auto read_tile = [&](TileRegs<D, FP8>& T_, int s) {
    const lds_u8_t* sp = ring + s * R::SLOT;
#pragma unroll
    for (int pi = 0; pi < 2; ++pi)
#pragma unroll
      for (int j = 0; j < Lo::KL; ++j)
        T_.k[pi][j] = lds_ld16(sp, kb[j] + 8 * pi * Lo::ROW);
#pragma unroll
    for (int u = 0; u < Lo::TPG; ++u) {
      if constexpr (FP8) T_.v[u] = lds_ld8(sp, vrd[u]);
      else T_.v[u] = lds_ld16(sp, vrd[u]);
    }
  };
  // q of a piece from q slot qs, in the lane's head order (as load_q_reset); accumulators
  // cleared
  const int hm = head_of_lane<G>(c);
  auto read_q = [&](WaveState<D, G, FP8>& S, int qs) {
    const lds_u8_t* qp = ring + NS * R::SLOT + qs * R::QSLOT;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint32_t qh = (h ^ hm) * D * 2;
      if constexpr (FP8) {
        const uint4 x0 = lds_ld16(qp, qh + 32 * c);
        const uint4 x1 = lds_ld16(qp, qh + 32 * c + 16);
        S.q[h][0] = x0.x; S.q[h][1] = x0.y; S.q[h][2] = x0.z; S.q[h][3] = x0.w;
        S.q[h][4] = x1.x; S.q[h][5] = x1.y; S.q[h][6] = x1.z; S.q[h][7] = x1.w;
      } else {
#pragma unroll
        for (int j = 0; j < Lo::KL; ++j) {
          const uint4 x = lds_ld16(qp, qh + j * 128 + 16 * c);
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
  };

  // ---- per-tile tables of the 64-tile block holding the current tile (entry 0 of the
  // per-lane arrays) and of the next one (entry 1): at each block boundary the arrays move
  // down by one entry, so every lookup below is a readlane of a fixed register
  auto next_block = [&]() {
#pragma unroll
    for (int q = 0; q + 1 < kRingTilesPerLane; ++q) {
      info_l[q] = info_l[q + 1];
      off_l[q] = off_l[q + 1];
      starts[q] = starts[q + 1];
    }
    info_l[kRingTilesPerLane - 1] = 0;
    off_l[kRingTilesPerLane - 1] = 0;
    starts[kRingTilesPerLane - 1] = 0;
  };
  // Requests tile ln + NS of the current block (past the chunk's end: zeros) into ring slot
  // s, preceded by the q rows of its piece when it opens one (into q slot qs).
  auto issue = [&](int ln, int s, bool opens, int& qs) {
    const int p = ln + NS, pl = p & (kWave - 1);
    const bool nb = p >= kWave;
    const int info = __builtin_amdgcn_readlane(nb ? info_l[1] : info_l[0], pl);
    const uint64_t off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(nb ? off_l[1] : off_l[0]), pl) << 8;
    if (opens) {
      const int sg = info >> 5, gg = sg / B, bb = sg - gg * B;
      const uint16_t* qg = a.q + ((size_t)bb * a.Hq + (size_t)gg * G) * D;
      const i32x4_t qr = ring_rsrc(qg, R::QB);
      const uint32_t qd = ring_addr + NS * R::SLOT + qs * R::QSLOT;
#pragma unroll
      for (int j = 0; j < R::QCOPIES; ++j) ring_copy16(qr, 1024 * j + 16 * lane, qd + 1024 * j);
      qs = qs + 1 == NS ? 0 : qs + 1;
    }
    // a tile past the chunk has info 0: no valid rows, so its copies only write zeros
    const uint32_t bytes = (uint32_t)(info & 31) * Lo::ROW;
    const i32x4_t kr = ring_rsrc(a.k_pool + off, bytes);
    const i32x4_t vr = ring_rsrc(a.v_pool + off, bytes);
    const uint32_t sd = ring_addr + s * R::SLOT;
#pragma unroll
    for (int j = 0; j < R::COPIES; ++j) ring_copy16(kr, ksrc[j], sd + 1024 * j);
#pragma unroll
    for (int j = 0; j < R::COPIES; ++j) ring_copy16(vr, vsrc[j], sd + R::TILE + 1024 * j);
  };

  // ---- the walk.  The first NS tiles are requested up front; then per tile: wait for its
  // slot, read it (and at a piece start the piece's q), request tile n + NS into the slot,
  // compute, and at a piece end write the piece.
  int q_issue = 0, q_read = 0;
  {
    // tiles 0 .. NS-1, as issue() would for ln = -NS .. -1
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int info = __builtin_amdgcn_readlane(info_l[0], t);
      const uint64_t off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_l[0], t) << 8;
      if ((starts[0] >> t) & 1) {
        const int sg = info >> 5, gg = sg / B, bb = sg - gg * B;
        const uint16_t* qg = a.q + ((size_t)bb * a.Hq + (size_t)gg * G) * D;
        const i32x4_t qr = ring_rsrc(qg, R::QB);
        const uint32_t qd = ring_addr + NS * R::SLOT + q_issue * R::QSLOT;
#pragma unroll
        for (int j = 0; j < R::QCOPIES; ++j) ring_copy16(qr, 1024 * j + 16 * lane, qd + 1024 * j);
        q_issue = q_issue + 1 == NS ? 0 : q_issue + 1;
      }
      const uint32_t bytes = (uint32_t)(info & 31) * Lo::ROW;
      const uint32_t sd = ring_addr + t * R::SLOT;
      const i32x4_t kr = ring_rsrc(a.k_pool + off, bytes);
      const i32x4_t vr = ring_rsrc(a.v_pool + off, bytes);
#pragma unroll
      for (int j = 0; j < R::COPIES; ++j) ring_copy16(kr, ksrc[j], sd + 1024 * j);
#pragma unroll
      for (int j = 0; j < R::COPIES; ++j) ring_copy16(vr, vsrc[j], sd + R::TILE + 1024 * j);
    }
  }
  WaveState<D, G, FP8> S;
  int seg = -1;
  float cscale = 0.f, vs = 1.f;
  constexpr uint64_t kAheadMask = ((1ull << NS) - 1) & ~1ull;  // tiles n+1 .. n+NS-1
  int s = 0;
  for (int n = 0; n < ntl; ++n) {
    const int ln = n & (kWave - 1);
    if (ln == 0 && n) next_block();
    // start bits of tiles n, n+1, ... (the next 64)
    const uint64_t win = (starts[0] >> ln) | (ln ? starts[1] << (kWave - ln) : 0ull);
    // outstanding after tile n's copies: tiles n+1 .. n+NS-1 and the q copies among them
    wait_vm_dyn<(NS - 1) * R::LOADS, R::QCOPIES, NS - 1>(__builtin_popcountll(win & kAheadMask));
    compiler_fence();
    TileRegs<D, FP8> RT;
    read_tile(RT, s);
    const int info = __builtin_amdgcn_readlane(info_l[0], ln);
    if (win & 1) {
      seg = info >> 5;
      read_q(S, q_read);
      q_read = q_read + 1 == NS ? 0 : q_read + 1;
      const int gg = seg / B;
      cscale = a.scale * kLog2e * (FP8 ? a.k_scale[gg] : 1.f);
      vs = FP8 ? a.v_scale[gg] : 1.f;
    }
    // every LDS read of the slot (and of the q slot) is complete before it is refilled
    __builtin_amdgcn_s_waitcnt(0xC07F);
    compiler_fence();
    issue(ln, s, (win >> NS) & 1, q_issue);
    s = s + 1 == NS ? 0 : s + 1;
    uint32_t pairs[Lo::NPS];
    qk_softmax<D, G, FP8>(S, RT, info & 31, cscale, lane, pairs);
    pv_accumulate<D, G, FP8>(S, RT, lane, pairs);
    if (n + 1 >= ntl || ((win >> 1) & 1)) {
      // end of a piece: merge the row groups, write the partial to slot chunk + segment
      GroupStats<G> X;
      wave_merge_rows<D, G, FP8>(X, S, lane);
      const size_t slot = (size_t)ch + seg;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (h % Lo::NG == r) {
          float* o = a.ws_o + (slot * G + h) * D + 8 * dc;
          *(float4*)o = make_float4(S.o[h][0] * vs, S.o[h][1] * vs, S.o[h][2] * vs, S.o[h][3] * vs);
          *(float4*)(o + 4) =
              make_float4(S.o[h][4] * vs, S.o[h][5] * vs, S.o[h][6] * vs, S.o[h][7] * vs);
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          a.ws_m[slot * G + h] = X.m[h];
          a.ws_l[slot * G + h] = X.l[h];
        }
      }
    }
  }
  // no copy may still be writing this workgroup's LDS when it ends
  wait_vm<0>();
}

}  // namespace pkv
