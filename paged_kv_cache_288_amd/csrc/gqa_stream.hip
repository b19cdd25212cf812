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
// last round.  Chunks are numbered so that each XCD (workgroup id mod 8 under round-robin
// dispatch) gets a contiguous eighth of the space - one KV head when Hkv = 8 - so a shared
// prefix's re-reads stay in that XCD's L2.
#include "gqa_tile.hpp"

namespace pkv {

constexpr int kMaxStreamSeqs = 4096;  // sequences whose tile counts fit the LDS prefix
constexpr int kMaxChunkTiles = 128;   // tiles per chunk: two per lane

template <int D, int G, bool FP8>
__global__ __launch_bounds__(kWaves * kWave, 2) void gqa_stream_kernel(DecodeArgs a) {
  using Lo = Layout<D, FP8>;
  __shared__ int s_pre[kMaxStreamSeqs + 1];
  __shared__ int s_sum[kWaves * kWave];
  // w and everything derived from it are wave-uniform: readfirstlane tells the compiler so,
  // which keeps the per-tile buffer resources in scalar registers
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int k = lane >> 3, c = lane & 7, r = lane / Lo::LPT, dc = lane % Lo::LPT;
  const int B = a.B;
  const int cap = a.max_blocks * a.block_size;

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
  if (blockIdx.x == 0) {
    for (int i = tid; i <= B; i += kWaves * kWave) a.ws_prefix[i] = s_pre[i];
    write_segment_ranges(a.ws_seg, s_pre, B, a.Hkv, a.chunks, tid, kWaves * kWave);
  }

  // ---- this wave's chunk
  const int T_head = __builtin_amdgcn_readfirstlane(s_pre[B]);
  const long long T = (long long)a.Hkv * T_head;
  const int C = a.chunks;
  const int ch = (blockIdx.x & 7) * (C / 8) + (blockIdx.x >> 3) * kWaves + w;
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

// out[b][h] = sum over the pieces of segment (g = h / G, b) of 2^(m - M) o / 2^(m - M) l.
// One wave per (sequence, query head), kMergeWaves of them per workgroup.
constexpr int kMergeWaves = 4;
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

template <int D, int G, bool FP8>
static hipError_t launch_stream_one(const DecodeArgs& a, hipStream_t s, bool merge) {
  hipLaunchKernelGGL((gqa_stream_kernel<D, G, FP8>), dim3(a.chunks / kWaves), dim3(kWaves * kWave),
                     0, s, a);
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

hipError_t launch_stream_merge(const DecodeArgs& a, hipStream_t s) {
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
