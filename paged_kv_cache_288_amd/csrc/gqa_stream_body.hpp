// Body of the balanced single-token GQA decode (gqa_stream.hip describes the division of
// work): one workgroup's walk over its four chunks of the flattened tile space, leaving
// (m, l, o) pieces for the merge.  A device function so that the shared-prefix cascade can
// run it in the same launch as the prefix pass.
#pragma once

#include "gqa_tile.hpp"

namespace pkv {

constexpr int kMaxStreamSeqs = 4096;  // sequences whose tile counts fit the LDS prefix
constexpr int kMaxChunkTiles = 128;   // tiles per chunk: two per lane

// The balanced decode of one workgroup: `bid` is its index in the grid of chunks / 4
// workgroups; s_pre [kMaxStreamSeqs + 1] and s_sum [kWaves * kWave] are its LDS.
template <int D, int G, bool FP8>
__device__ __forceinline__ void gqa_stream_body(const DecodeArgs& a, int bid, int* s_pre,
                                                int* s_sum) {
  using Lo = Layout<D, FP8>;
  // w and everything derived from it are wave-uniform: readfirstlane tells the compiler so,
  // which keeps the per-tile buffer resources in scalar registers
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int k = lane >> 3, c = lane & 7, r = lane / Lo::LPT, dc = lane % Lo::LPT;
  const int B = a.B;
  const int cap = min(a.max_blocks * a.block_size, a.max_context_len);

  // ---- tiles per sequence and their exclusive prefix, scanned across the workgroup
  auto ntiles = [&](int bi) {
    int L = a.context_lens[bi];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    return (L + kTile - 1) / kTile;
  };
  const int per = (B + kWaves * kWave - 1) / (kWaves * kWave);
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (tid * per + i < B) local += ntiles(tid * per + i);
  s_sum[tid] = local;
  __syncthreads();
  for (int off = 1; off < kWaves * kWave; off <<= 1) {
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
  if (tid == 0) s_pre[B] = s_sum[kWaves * kWave - 1];
  __syncthreads();
  if (bid == 0) {
    for (int i = tid; i <= B; i += kWaves * kWave) a.ws_prefix[i] = s_pre[i];
    write_segment_ranges(a.ws_seg, s_pre, B, a.Hkv, a.chunks, tid, kWaves * kWave);
  }

  // ---- this wave's chunk
  const int T_head = __builtin_amdgcn_readfirstlane(s_pre[B]);
  const long long T = (long long)a.Hkv * T_head;
  const int C = a.chunks;
  const int ch = (bid & 7) * (C / 8) + (bid >> 3) * kWaves + w;
  const long long tb = T * ch / C, te = T * (ch + 1) / C;
  const int ntl = (int)min(te - tb, (long long)kMaxChunkTiles);
  if (ntl <= 0) return;

  // ---- per-tile byte offset, valid-token count and segment, two tiles per lane
  const int tiles_per_block = a.block_size / kTile;
  const size_t head_bytes = (size_t)a.block_size * Lo::ROW;
  const size_t block_bytes = head_bytes * a.Hkv;
  // Per tile: byte offset / 256 (tiles start on 2 KiB boundaries; pools up to 1 TiB), and
  // valid tokens (5 bits) | segment << 5.
  uint32_t off_l[2] = {0, 0};
  int info_l[2] = {0, 0};
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
      int L = a.context_lens[lo];
      L = L < 0 ? 0 : (L > cap ? cap : L);
      const int phys = a.block_table[(size_t)lo * a.max_blocks + tt / tiles_per_block];
      const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
      const uint64_t off = (uint64_t)(ok ? phys : 0) * block_bytes + (uint64_t)gg * head_bytes +
                           (uint64_t)(tt % tiles_per_block) * (kTile * Lo::ROW);
      off_l[j] = (uint32_t)(off >> 8);
      info_l[j] = (ok ? min(kTile, L - tt * kTile) : 0) | ((gg * B + lo) << 5);
    }
  }
  auto pick = [](int j, int x0, int x1) { return j ? x1 : x0; };
  // Source of chunk tile n, or an empty one (all loads return zeros) for n >= end.
  auto tile_at = [&](int n, int end, int& nv) -> TileSrc {
    if (n >= end) {
      nv = 0;
      return tile_src<D, FP8>(a.k_pool, a.v_pool, 0);
    }
    const int j = n >> 6, ln = n & (kWave - 1);
    const uint64_t off =
        (uint64_t)(uint32_t)__builtin_amdgcn_readlane(pick(j, (int)off_l[0], (int)off_l[1]), ln) << 8;
    nv = __builtin_amdgcn_readlane(pick(j, info_l[0], info_l[1]), ln) & 31;
    return tile_src<D, FP8>(a.k_pool + off, a.v_pool + off, nv);
  };
  auto tile_seg = [&](int n) {
    return __builtin_amdgcn_readlane(pick(n >> 6, info_l[0], info_l[1]), n & (kWave - 1)) >> 5;
  };

  // Tiles that open a new piece (their segment differs from the previous tile's), as two
  // 64-bit masks over the chunk's tiles.
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

  // ---- pieces: each is a pipelined walk over its tiles, then one partial
  const uint32_t koff = k_lane_offset<D, FP8>(k, c), voff = v_lane_offset<D, FP8>(r, dc);
  TileRegs<D, FP8> RA, RB;
  for (int n0 = 0; n0 < ntl;) {
    const int n1 = next_start(n0);
    const int seg = tile_seg(n0), gg = seg / B, bb = seg - gg * B;
    WaveState<D, G, FP8> S;
    load_q_reset<D, G, FP8>(S, a.q + ((size_t)bb * a.Hq + (size_t)gg * G) * D, c);
    const float cscale = a.scale * kLog2e * (FP8 ? a.k_scale[gg] : 1.f);
    const float vs = FP8 ? a.v_scale[gg] : 1.f;

    // Two tile buffers, refilled half by half: a tile's K is replaced by the tile two
    // ahead as soon as its scores are done, its V once p.V is done.
    int nvA, nvB;
    TileSrc A = tile_at(n0, n1, nvA), Bt = tile_at(n0 + 1, n1, nvB);
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
    int n = n0;
    for (; n + 1 < n1; n += 2) {
      {
        uint32_t pairs[Lo::NPS];
        qk_softmax<D, G, FP8>(S, RA, nvA, cscale, lane, pairs);
        sched_fence();
        A = tile_at(n + 2, n1, nvA);
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
        Bt = tile_at(n + 3, n1, nvB);
        load_k<D, FP8>(RB, Bt.k, koff);
        sched_fence();
        pv_accumulate<D, G, FP8>(S, RB, lane, pairs);
        sched_fence();
        load_v<D, FP8>(RB, Bt.v, voff);
      }
    }
    if (n < n1) {
      uint32_t pairs[Lo::NPS];
      qk_softmax<D, G, FP8>(S, RA, nvA, cscale, lane, pairs);
      pv_accumulate<D, G, FP8>(S, RA, lane, pairs);
    }

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
    n0 = n1;
  }
}

}  // namespace pkv
