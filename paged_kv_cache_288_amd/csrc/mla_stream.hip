// Balanced latent (MLA) decode attention on gfx950 (the library's default MLA mode).
//
// Same arithmetic as mla_decode.hip: every token caches one latent row C_t of 576 dims
// (512 latent + 64 RoPE) that all query heads attend to, the whole row as key and its first
// 512 dims as value ("深入LLM推理：从KV Cache到PD分离的Serving全景解析", section
// "KV Cache：Transformer的循环状态"; "GPU推理深度拆解：KV Cache视角", "KV Cache 大小与分配演进"):
//     out[b][h] = softmax_t(scale * q[b][h] . C_t) C_t[0:512].
// Scores run on the bf16 MFMA, p.V on the fp16 MFMA (weights and value dims in fp16, fp32
// accumulate), with the lazy online softmax of the other kernels.
//
// Division of work.  Each sequence's context is cut into stages of 32 tokens (half a
// 64-token block, one contiguous 36 KiB run of the pool).  The stages of all sequences are
// laid end to end and the resulting space is cut into `chunks` equal ranges; a workgroup
// takes one range for one group of 16*HT query heads, so grid = head groups x chunks and
// every workgroup gets the same work (+-1 stage).  Where a range meets a sequence it
// produces a piece: the (m, l, o) state of those tokens for its heads, written to slot
// chunk + b; the merge kernel (shared with the GQA balanced mode) combines the pieces.  The
// head groups of one chunk are numbered to land on one XCD, so a stage read from HBM by one
// of them is found in that XCD's L2 by the others.
//
// Per workgroup (4 waves), per stage:
//  * the stage is copied HBM -> LDS by buffer loads that write LDS directly (no registers),
//    NBUF - 1 stages ahead; the buffer range is the stage's valid rows, so rows past a
//    sequence's end (or a block id outside the pool) are never read;
//  * LDS rows are token-major with the 16-byte chunks of row t XOR-permuted by
//    (t & 7) ^ ((t >> 3) & 1) within groups of 8, which makes both read patterns below free
//    of bank conflicts;
//  * scores: S^T = K Q^T on v_mfma_f32_16x16x32_bf16, K as the A operand read straight from
//    the token-major rows, Q (B operand) held in registers.  A wave owns one 16-head tile and
//    2 / (4 / HT) of the stage's two 16-token tiles; waves sharing a head tile exchange
//    their tile maxima through LDS;
//  * probabilities P = 2^(s - m) are rounded to fp16 and stored [head][token] in LDS;
//  * p.V: O += P V on v_mfma_f32_16x16x32_f16.  A wave owns 128 of the 512 output dims for
//    all heads of the group.  The B operand (8 tokens of one dim per lane) is read from the
//    token-major rows with ds_read_b64_tr_b16, which transposes 4x4 blocks of 16-bit values
//    across lanes, and widened bf16 -> fp16 in registers (exact in fp16's normal range,
//    below 2^-14 rounded to its subnormal grid; |v| must stay below 65504).
#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBlock = 64;
constexpr int kStage = 32;                          // tokens per stage
constexpr int kRow = kDqk * 2;                      // 1152 bytes per latent row
constexpr int kRowChunks = kRow / 16;               // 72
constexpr int kStageBytes = kStage * kRow;          // 36864
constexpr int kMWaves = 4;                          // waves of mla_stream_kernel
constexpr int kMThreads = kMWaves * kWave;
constexpr int kDmaWaves = 4;                        // waves that copy the stages
constexpr int kDmaPerWave = kStageBytes / (16 * kWave) / kDmaWaves;  // 9 loads per wave per stage
constexpr int kMaxMlaSeqs = 4096;
constexpr int kMaxChunkStages = 128;                // two per lane
constexpr int kPRow = 80;                           // bytes per head row of P (32 fp16 + pad)
constexpr float kSlack = 8.0f;
constexpr int kScoreGroup = 2;                      // score products per group of K reads
constexpr int kPvWaves = 8;                         // p.V waves of mla_split_kernel
constexpr int kPieceStartStages = 5;                // measured cost of a piece start, in stages
static_assert(kStageBytes % (16 * kWave * kDmaWaves) == 0, "stage split");

__device__ __forceinline__ f32x4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16(const f16x8_t& a, const f16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// XOR permutation of the 16-byte chunks inside groups of 8 for LDS row t.
__device__ __forceinline__ int row_swizzle(int t) { return (t & 7) ^ ((t >> 3) & 1); }

// Stage layout of mla_split_kernel: chunk L of row t sits at position L ^ split_swizzle(t)
// (an involution that only touches the low three bits, so the 8-chunk tail stays in place).
// gfx950's LDS serves a 16-byte read per lane as four 16-lane groups over 64 banks, and
// lanes l and l + 16 must fall in 16-byte bank slots that agree in bits 2 and 3.  With
// this swizzle:
// * a score-tile read (16 consecutive rows, one chunk per 16-lane group, groups 0/1 and
//   2/3 taking chunks 16 apart, or tail chunks a and a ^ 2) hits 16 distinct slots per
//   group, with the same slot, or one flipped in bit 1, for lanes l and l + 16;
// * a transposed V read (per 32-lane half: rows 8k .. 8k + 7, two adjacent chunks) hits
//   32 distinct 8-byte bank pairs.
__device__ __forceinline__ int split_swizzle(int t) {
  return (((t >> 1) & 3) << 1) | ((t >> 3) & 1);
}

// Max / sum over the 4 lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_max4(float x) {
  float lo, hi, e, o;
  halves_pair32(x, lo, hi);
  x = fmaxf(lo, hi);
  rows_pair16(x, e, o);
  return fmaxf(e, o);
}
__device__ __forceinline__ float group_sum4(float x) {
  float lo, hi, e, o;
  halves_pair32(x, lo, hi);
  x = lo + hi;
  rows_pair16(x, e, o);
  return e + o;
}

// Raw buffer resource words over [base, base + bytes) (out-of-range loads return zeros).
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return i32x4_t{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), (int)bytes, kRawBufferWord3};
}

// 16 bytes per lane from byte offset voff of the buffer into LDS at lds_base + 16 * lane.
// Issued as assembly so that the compiler does not make every later LDS read wait for all
// such copies (it cannot tell the stage buffers apart); the kernel waits for each stage
// itself with s_waitcnt vmcnt.  The copy reads its LDS address from M0 and its resource from
// SGPRs; the leading s_nop 4 gives the five wait states that an SGPR written by a VALU
// instruction (readlane) needs before a vector-memory read, which also covers M0's one.
__device__ __forceinline__ void lds_copy16(i32x4_t rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "{m0}"(lds_base)
               : "memory");
}

// Two bf16 in one dword -> the same two values as fp16 (exact for |v| < 65504).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  return pack_f16(bf16_lo(x), bf16_hi(x));
}



}  // namespace

template <int HT, int NBUF>
__global__ __launch_bounds__(kMThreads, 1) void mla_stream_kernel(MlaArgs a) {
  constexpr int HPU = 16 * HT;   // heads per workgroup
  constexpr int WPH = 4 / HT;    // waves per head tile in the score phase
  constexpr int TT = 2 / WPH;    // token tiles per wave in the score phase
  static_assert(HT == 2 || HT == 4, "head tiles per workgroup");
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[NBUF * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sP[HPU * kPRow];
  __shared__ __attribute__((aligned(16))) float sMax[2][HPU];
  __shared__ __attribute__((aligned(16))) float sAlpha[HPU];
  __shared__ float sL[kMWaves][16];
  static_assert((kMaxMlaSeqs + 1 + kMThreads) * 4 <= NBUF * kStageBytes, "prefix scratch");

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int i16 = lane & 15, g = lane >> 4;
  const int B = a.B, Hq = a.Hq, HG = Hq / HPU, C = a.chunks;
  const int cap = min(a.max_blocks * kBlock, a.max_context_len);

  // ---- stages per sequence and their exclusive prefix (scratch in the stage buffers)
  int* s_pre = (int*)sbuf;
  int* s_sum = s_pre + kMaxMlaSeqs + 1;
  auto nstages = [&](int bi) {
    int L = a.context_lens[bi];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    return (L + kStage - 1) / kStage;
  };
  {
    const int per = (B + kMThreads - 1) / kMThreads;
    int local = 0;
    for (int i = 0; i < per; ++i)
      if (tid * per + i < B) local += nstages(tid * per + i);
    s_sum[tid] = local;
    __syncthreads();
    for (int off = 1; off < kMThreads; off <<= 1) {
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
        run += nstages(bi);
      }
    }
    if (tid == 0) s_pre[B] = s_sum[kMThreads - 1];
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int i = tid; i <= B; i += kMThreads) a.ws_prefix[i] = s_pre[i];
      write_segment_ranges(a.ws_seg, s_pre, B, 1, C, tid, kMThreads);
    }
  }

  // ---- this workgroup's head group and chunk: the HG head groups of chunk ch are
  // consecutive multiples of 8 apart, i.e. on one XCD under round-robin dispatch
  const int T = __builtin_amdgcn_readfirstlane(s_pre[B]);
  const int x = blockIdx.x, xcd = x & 7, kx = x >> 3;
  const int hg = kx % HG, ch = (kx / HG) * 8 + xcd;
  const long long tb = (long long)T * ch / C, te = (long long)T * (ch + 1) / C;
  const int ns = (int)min(te - tb, (long long)kMaxChunkStages);

  // ---- per-stage first token (pool row index) and valid-token count | sequence << 6,
  // two stages per lane
  uint32_t row_l[2] = {0, 0};
  int info_l[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = kWave * j + lane;
    if (n < ns) {
      const int t = (int)(tb + n);
      int lo = 0, hi = B - 1;  // last sequence whose first stage is <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      const int js = t - s_pre[lo];
      int L = a.context_lens[lo];
      L = L < 0 ? 0 : (L > cap ? cap : L);
      const int phys = a.block_table[(size_t)lo * a.max_blocks + js / 2];
      const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
      row_l[j] = (uint32_t)(ok ? phys : 0) * kBlock + (js & 1) * kStage;
      info_l[j] = (ok ? min(kStage, L - js * kStage) : 0) | (lo << 6);
    }
  }
  uint64_t starts[2];  // stages that open a new piece
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = kWave * j + lane;
    const int seq = info_l[j] >> 6;
    int prev = __shfl_up(seq, 1);
    if (lane == 0) prev = j ? __builtin_amdgcn_readlane(info_l[0], kWave - 1) >> 6 : -1;
    starts[j] = __builtin_amdgcn_ballot_w64(n < ns && seq != prev);
  }
  auto stage_info = [&](int n) {
    return __builtin_amdgcn_readlane(n >> 6 ? info_l[1] : info_l[0], n & (kWave - 1));
  };
  auto stage_src = [&](int n) -> i32x4_t {
    if (n >= ns) return rsrc_words(a.kv_pool, 0);
    const uint32_t row =
        (uint32_t)__builtin_amdgcn_readlane((int)(n >> 6 ? row_l[1] : row_l[0]), n & (kWave - 1));
    const int valid = stage_info(n) & 63;
    return rsrc_words((const uint8_t*)a.kv_pool + (uint64_t)row * kRow, valid * kRow);
  };

  // The prefix scratch is dead from here on; clear the stage buffers once so that rows a
  // stage does not load hold zeros or earlier valid rows, never garbage.
  __syncthreads();
  for (int i = tid; i < NBUF * kStageBytes / 16; i += kMThreads)
    *(uint4*)(sbuf + 16 * i) = uint4{0, 0, 0, 0};
  __syncthreads();
  if (ns <= 0) return;

  // ---- LDS-direct copy of a stage: load j of wave w fills bytes [1024 (9w + j), +1024) of
  // the buffer; lane -> chunk c = 64 (9w + j) + lane = row t, permuted chunk p'; it loads
  // chunk p' ^ swizzle(t) of row t from the pool.
  uint32_t dma_off[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int c = (w * kDmaPerWave + j) * kWave + lane;
    const int t = c / kRowChunks, pp = c % kRowChunks;
    dma_off[j] = (uint32_t)(16 * (t * kRowChunks + (pp ^ row_swizzle(t))));
  }
  const uint32_t sbuf_lds = (uint32_t)(uintptr_t)(lds_void_t*)sbuf;
  auto issue_stage = [&](int n) {
    const i32x4_t src = stage_src(n);
    const uint32_t base = sbuf_lds + (n % NBUF) * kStageBytes + w * kDmaPerWave * 1024;
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) lds_copy16(src, dma_off[j], base + j * 1024);
  };

  // ---- score-phase roles and per-lane LDS offsets
  const int hw = w / WPH;             // head tile of this wave in the score phase
  const int tt0 = (w % WPH) * TT;     // its first token tile
  // K (A operand): token tt*16 + i16, chunk 4 ks + g  ->  even / odd ks base offsets
  int k_off[TT][2];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int t = (tt0 + tt) * 16 + i16;
    const int xm = g ^ row_swizzle(t);
    k_off[tt][0] = 16 * (t * kRowChunks + xm);
    k_off[tt][1] = 16 * (t * kRowChunks + (xm ^ 4));
  }
  // V (B operand, transposed reads): lane s = i16 reads token 8 g + 4 h + (s >> 2), dims
  // 128 w + 16 nt + 4 (s & 3) .. +3; the chunk term depends on nt & 3 (plus 8 (nt >> 2))
  int v_off[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 8 * g + 4 * h + (i16 >> 2);
    const int qd = (i16 & 3) >> 1, half8 = 8 * (i16 & 1);
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4)
      v_off[h][n4] = 16 * (t * kRowChunks + 16 * w + ((2 * n4 + qd) ^ row_swizzle(t))) + half8;
  }

  // ---- state
  bf16x8_t qf[kDqk / 32];
  f32x4_t o[HT][8];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[ht][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};  // finite for alpha = 0
  float m_run = kNegInf, l_part = 0.f;
  const float cscale = a.scale * kLog2e;
  int seq = -1;

  auto flush = [&]() {  // write the finished piece (slot ch + seq) to the workspace
    const float l_head = group_sum4(l_part);
    if (g == 0) sL[w][i16] = l_head;
    barrier_vm<63>();
    const size_t slot = (size_t)ch + seq;
    const size_t row0 = slot * Hq + (size_t)hg * HPU;
    if (tt0 == 0 && g == 0) {
      float l = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < WPH; ++k2) l += sL[hw * WPH + k2][i16];
      a.ws_m[row0 + hw * 16 + i16] = m_run;
      a.ws_l[row0 + hw * 16 + i16] = l;
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a.ws_o[(row0 + ht * 16 + 4 * g + r) * kDv + 128 * w + 16 * nt + i16] = o[ht][nt][r];
  };

  for (int n = 0; n < NBUF - 1; ++n) issue_stage(n);

  // Pieces one after another (the stage copies run on across them); within a piece the
  // accumulators are touched only by MFMAs.
  auto next_start = [&](int n) {  // first stage after n that opens a piece (or ns)
    for (int j = (n + 1) >> 6; j < 2; ++j) {
      const int lo = (n + 1) - kWave * j;
      const uint64_t m = lo <= 0 ? starts[j] : (lo >= kWave ? 0 : starts[j] & (~0ull << lo));
      if (m) return kWave * j + (int)__builtin_ctzll(m);
    }
    return ns;
  };
  for (int n = 0; n < ns;) {
    const int n_end = next_start(n);
    seq = stage_info(n) >> 6;
    {
      const uint8_t* qrow =
          (const uint8_t*)(a.q + ((size_t)seq * Hq + (size_t)hg * HPU + hw * 16 + i16) * kDqk);
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qrow + ks * 64 + 16 * g));
      // Wait for q here, once per piece: otherwise the compiler's count-based waits for q
      // (which do not know about the stage copies) would drain the copy pipeline at every
      // stage.
      wait_vm<0>();
    }
    // O is not cleared: with the running max back at -inf, the piece's first stage with a
    // valid token rescales every head by alpha = 2^(-inf) = 0.  (A piece without valid
    // tokens keeps m = -inf, and the merge gives it no weight.)
    m_run = kNegInf;
    l_part = 0.f;
    for (; n < n_end; ++n) {
      const int valid = stage_info(n) & 63;
      // stage n has landed once this wave's loads of it are done (NBUF - 2 newer stages may
      // still be in flight) and every wave got here, which also means every wave is done
      // reading the buffer that stage n + NBUF - 1 now overwrites
      barrier_vm<kDmaPerWave * (NBUF - 2)>();
      issue_stage(n + NBUF - 1);
      const uint8_t* buf = sbuf + (n % NBUF) * kStageBytes;

      // ---- S^T = K Q^T for this wave's token tiles and head tile; K fragments are read in
      // groups of six ahead of their MFMAs
      f32x4_t s[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) s[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < kDqk / 32; k0 += 6) {
        bf16x8_t kf[TT][6];
#pragma unroll
        for (int ks = 0; ks < 6; ++ks)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            kf[tt][ks] = __builtin_bit_cast(
                bf16x8_t, *(const uint4*)(buf + k_off[tt][(k0 + ks) & 1] + 128 * ((k0 + ks) >> 1)));
#pragma unroll
        for (int ks = 0; ks < 6; ++ks)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) s[tt] = mfma_bf16(kf[tt][ks], qf[k0 + ks], s[tt]);
      }

      // ---- online softmax (log2 domain); lane holds tokens tt*16 + 4g + r of head i16
      float sv[TT * 4];
      float mt = kNegInf;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = (tt0 + tt) * 16 + 4 * g + r;
          const float v = tok < valid ? s[tt][r] * cscale : kNegInf;
          sv[tt * 4 + r] = v;
          mt = fmaxf(mt, v);
        }
      mt = group_max4(mt);
      if constexpr (WPH > 1) {  // the other token tile of this head tile is another wave's
        if (g == 0) sMax[tt0 / TT][hw * 16 + i16] = mt;
        barrier_vm<63>();
        mt = fmaxf(sMax[0][hw * 16 + i16], sMax[1][hw * 16 + i16]);
      }
      float alpha = 1.f;
      if (wave_any(mt > m_run + kSlack)) {
        const float m_new = fmaxf(m_run, mt);
        alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
        l_part *= alpha;
        m_run = m_new;
      }
      if (tt0 == 0 && g == 0) sAlpha[hw * 16 + i16] = alpha;
      const float m_use = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const uint32_t p01 = pack_f16(fast_exp2(sv[tt * 4 + 0] - m_use), fast_exp2(sv[tt * 4 + 1] - m_use));
        const uint32_t p23 = pack_f16(fast_exp2(sv[tt * 4 + 2] - m_use), fast_exp2(sv[tt * 4 + 3] - m_use));
        l_part = dot2h(p01, kOnesF16x2, l_part);
        l_part = dot2h(p23, kOnesF16x2, l_part);
        *(uint2*)(sP + (hw * 16 + i16) * kPRow + ((tt0 + tt) * 16 + 4 * g) * 2) = uint2{p01, p23};
      }
      barrier_vm<63>();

      // ---- O += P V for dims [128 w, 128 w + 128) of all HPU heads, after scaling O's rows
      // by their heads' alpha when some head's running max moved (rare).  The accumulators
      // live in ordinary VGPRs (this file is built with -amdgpu-mfma-vgpr-form): in the
      // accumulator registers the compiler would copy them around this branch every stage.
      auto pv_phase = [&]() {
        // all P and V fragments are read first (V widened to fp16 as it arrives), then the
        // HT x 8 MFMAs run back to back
        f16x8_t pf[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          pf[ht] = __builtin_bit_cast(f16x8_t, *(const uint4*)(sP + (ht * 16 + i16) * kPRow + 16 * g));
        const lds_char_t* lbuf = (const lds_char_t*)((lds_void_t*)buf);
        uint2 vr[8][2];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            vr[nt][h] = __builtin_bit_cast(
                uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (lds_s16x4_t*)(lbuf + v_off[h][nt & 3] + 128 * (nt >> 2))));
        sched_fence();
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const f16x8_t vf = __builtin_bit_cast(
              f16x8_t, uint4{bf16x2_to_f16x2(vr[nt][0].x), bf16x2_to_f16x2(vr[nt][0].y),
                             bf16x2_to_f16x2(vr[nt][1].x), bf16x2_to_f16x2(vr[nt][1].y)});
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) o[ht][nt] = mfma_f16(pf[ht], vf, o[ht][nt]);
        }
      };
      float4 alv[HT];
      bool anyr = false;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        alv[ht] = *(const float4*)&sAlpha[ht * 16 + 4 * g];
        anyr |= alv[ht].x != 1.f || alv[ht].y != 1.f || alv[ht].z != 1.f || alv[ht].w != 1.f;
      }
      if (wave_any(anyr)) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const float4 al = alv[ht];
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) {
            o[ht][nt][0] *= al.x;
            o[ht][nt][1] *= al.y;
            o[ht][nt][2] *= al.z;
            o[ht][nt][3] *= al.w;
          }
        }
      }
      pv_phase();
    }
    flush();
  }
  // Copies of stages past the end (empty ranges) may still be in flight: they must land
  // before this workgroup's LDS can be handed to another one.
  wait_vm<0>();
}

// Role-split variant for 64-head groups, 4 + PVW waves: waves 0-3 ("scorers") take stage n -
// scores for one 16-head tile over all 32 tokens, the online softmax, P into LDS - while the
// PVW waves after them ("accumulators") run p.V of stage n - 1 for 512 / PVW output dims
// each, the first four also copying the stages HBM -> LDS.  Each SIMD holds one score wave
// and PVW / 4 p.V waves, so score and p.V products overlap, and there is one workgroup
// barrier per stage.  P and the rescale factors are double-buffered by stage parity; the copy
// of stage n + NBUF - 2 reuses the buffer of stage n - 2, which every wave is done with by
// the barrier of iteration n.
template <int NBUF, int PVW>
__global__ __launch_bounds__((4 + PVW) * kWave, 1) void mla_split_kernel(MlaArgs a) {
  constexpr int THREADS = (4 + PVW) * kWave;
  constexpr int HT = 4, HPU = 64;  // head tiles and heads per workgroup
  constexpr int DPW = kDv / PVW, NT = DPW / 16;  // accumulator: output dims, p.V products per head tile
  static_assert(PVW == 4 || PVW == 8, "p.V waves");
  static_assert(NBUF >= 4, "two stages in flight");
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[NBUF * kStageBytes];
  // P of a stage in four 1 KiB slabs: slab k holds k-operand positions 8 k .. 8 k + 7 of
  // every head (16 bytes per head), so that a p.V operand read is one 16-byte slot per lane
  // with lanes l and l + 16 on the same bank slot.
  __shared__ __attribute__((aligned(16))) uint8_t sP[2][4 * 16 * HPU];
  __shared__ __attribute__((aligned(16))) float sAlpha[2][HPU];
  __shared__ __attribute__((aligned(4))) uint8_t sRescale[2][4];  // per score wave: alpha != 1
  static_assert((kMaxMlaSeqs + 1 + THREADS) * 4 <= NBUF * kStageBytes, "prefix scratch");

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const bool scorer = w < 4;
  const int r4 = w & 3;                // head tile of a score wave
  const int pvj = scorer ? 0 : w - 4;  // output-dim slice of a p.V wave
  const bool copier = !scorer && pvj < 4;  // the first four p.V waves copy the stages
  const int i16 = lane & 15, g = lane >> 4;
  const int B = a.B, Hq = a.Hq, HG = Hq / HPU, C = a.chunks;
  const int cap = min(a.max_blocks * kBlock, a.max_context_len);

  // ---- stages per sequence and their exclusive prefix.  Up to 64 sequences every wave
  // scans them in registers (lane i: sequence i), so that no workgroup barrier or LDS round
  // trip sits between the context lengths and the first stage copies; more sequences take a
  // workgroup-wide scan with scratch in the stage buffers.
  int* s_pre = (int*)sbuf;
  int* s_sum = s_pre + kMaxMlaSeqs + 1;
  auto clamp_len = [&](int L) { return L < 0 ? 0 : (L > cap ? cap : L); };
  auto nstages = [&](int bi) { return (clamp_len(a.context_lens[bi]) + kStage - 1) / kStage; };
  const bool wave_scan = B <= kWave;
  int pre_l = 0, len_l = 0;  // register scan: sequence `lane`'s first stage and length
  int T, PV;
  // Virtual stages placed before every sequence, so that a chunk in which a piece starts
  // (q loaded, the closed piece's partials stored) gets correspondingly fewer stages.  Only
  // with at least one stage per chunk (the merge takes every chunk of a segment's range as
  // written) and while every chunk stays within kMaxChunkStages.
  auto piece_pad = [&](int T_) {
    return T_ >= C && (long long)T_ + (long long)kPieceStartStages * B <=
                          (long long)(kMaxChunkStages - 1) * C
               ? kPieceStartStages
               : 0;
  };
  if (wave_scan) {
    len_l = lane < B ? clamp_len(a.context_lens[lane]) : 0;
    const int ns_l = (len_l + kStage - 1) / kStage;
    int incl = ns_l;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    pre_l = incl - ns_l;
    T = __builtin_amdgcn_readlane(incl, kWave - 1);
    PV = piece_pad(T);
    if (blockIdx.x == 0 && w == 0) {
      if (lane < B) {
        a.ws_prefix[lane] = pre_l;
        segment_range(pre_l + (long long)PV * (lane + 1), ns_l, (long long)T + (long long)PV * B, C,
                      a.ws_seg + 2 * lane);
      }
      if (lane == 0) a.ws_prefix[B] = T;
    }
  } else {
    const int per = (B + THREADS - 1) / THREADS;
    int local = 0;
    for (int i = 0; i < per; ++i)
      if (tid * per + i < B) local += nstages(tid * per + i);
    s_sum[tid] = local;
    __syncthreads();
    for (int off = 1; off < THREADS; off <<= 1) {
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
        run += nstages(bi);
      }
    }
    if (tid == 0) s_pre[B] = s_sum[THREADS - 1];
    __syncthreads();
    T = __builtin_amdgcn_readfirstlane(s_pre[B]);
    PV = piece_pad(T);
    if (blockIdx.x == 0) {
      for (int i = tid; i <= B; i += THREADS) a.ws_prefix[i] = s_pre[i];
      for (int b = tid; b < B; b += THREADS)
        segment_range(s_pre[b] + (long long)PV * (b + 1), s_pre[b + 1] - s_pre[b],
                      (long long)T + (long long)PV * B, C, a.ws_seg + 2 * b);
    }
  }

  // ---- this workgroup's head group and chunk (head groups of a chunk on one XCD).  The
  // chunks are equal ranges of the stage space with PV virtual stages before each sequence
  // (sequence b's stages sit at virtual positions pre[b] + PV (b + 1) ..); a chunk takes the
  // real stages inside its range, which are contiguous.
  const int x = blockIdx.x, xcd = x & 7, kx = x >> 3;
  const int hg = kx % HG, ch = (kx / HG) * 8 + xcd;
  const long long Tv = (long long)T + (long long)PV * B;
  auto real_before = [&](long long v) -> long long {  // real stages before virtual position v
    if (PV == 0) return v;
    int pads;
    if (wave_scan) {  // all lanes take part: sum over sequences of their pads before v
      const long long vp = (long long)pre_l + (long long)PV * lane;
      pads = lane < B ? (int)min(max(v - vp, 0LL), (long long)PV) : 0;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) pads += __shfl_xor(pads, off);
    } else {  // the last sequence whose pads start at or before v (sequence 0's start at 0)
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((long long)s_pre[mid] + (long long)PV * mid <= v) lo = mid;
        else hi = mid - 1;
      }
      pads = PV * lo + (int)min(v - ((long long)s_pre[lo] + (long long)PV * lo), (long long)PV);
    }
    return v - __builtin_amdgcn_readfirstlane(pads);  // the same in every lane
  };
  const long long tb = real_before(Tv * ch / C), te = real_before(Tv * (ch + 1) / C);
  const int ns = (int)min(te - tb, (long long)kMaxChunkStages);

  // ---- per-stage first token (pool row index) and valid-token count | sequence << 6,
  // two stages per lane
  uint32_t row_l[2] = {0, 0};
  int info_l[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = kWave * j + lane;
    const int t = (int)(tb + min(n, max(ns - 1, 0)));
    int lo = 0, js = 0, L = 0;  // last sequence whose first stage is <= t
    if (wave_scan) {            // all lanes take part in the shuffles
#pragma unroll
      for (int step = kWave / 2; step >= 1; step >>= 1) {
        const int cand = lo + step;
        const int v = __shfl(pre_l, cand < B ? cand : 0);
        if (cand < B && v <= t) lo = cand;
      }
      js = t - __shfl(pre_l, lo);
      L = __shfl(len_l, lo);
    }
    if (n < ns) {
      if (!wave_scan) {
        int hi = B - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_pre[mid] <= t) lo = mid;
          else hi = mid - 1;
        }
        js = t - s_pre[lo];
        L = clamp_len(a.context_lens[lo]);
      }
      const int phys = a.block_table[(size_t)lo * a.max_blocks + js / 2];
      const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
      row_l[j] = (uint32_t)(ok ? phys : 0) * kBlock + (js & 1) * kStage;
      info_l[j] = (ok ? min(kStage, L - js * kStage) : 0) | (lo << 6);
    }
  }
  uint64_t starts[2];  // stages that open a new piece
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = kWave * j + lane;
    const int sq = info_l[j] >> 6;
    int prev = __shfl_up(sq, 1);
    if (lane == 0) prev = j ? __builtin_amdgcn_readlane(info_l[0], kWave - 1) >> 6 : -1;
    starts[j] = __builtin_amdgcn_ballot_w64(n < ns && sq != prev);
  }
  auto stage_info = [&](int n) {
    return __builtin_amdgcn_readlane(n >> 6 ? info_l[1] : info_l[0], n & (kWave - 1));
  };
  auto opens_piece = [&](int n) {  // n < ns
    return ((n >> 6 ? starts[1] : starts[0]) >> (n & (kWave - 1))) & 1;
  };
  auto stage_src = [&](int n) -> i32x4_t {
    if (n >= ns) return rsrc_words(a.kv_pool, 0);
    const uint32_t row =
        (uint32_t)__builtin_amdgcn_readlane((int)(n >> 6 ? row_l[1] : row_l[0]), n & (kWave - 1));
    const int valid = stage_info(n) & 63;
    return rsrc_words((const uint8_t*)a.kv_pool + (uint64_t)row * kRow, valid * kRow);
  };

  // The prefix scratch is dead from here on; clear the stage buffers once so that rows a
  // stage does not load hold zeros or earlier valid rows, never garbage.
  if (!wave_scan) __syncthreads();
  for (int i = tid; i < NBUF * kStageBytes / 16; i += THREADS)
    *(uint4*)(sbuf + 16 * i) = uint4{0, 0, 0, 0};
  __syncthreads();
  if (ns <= 0) return;

  // ---- LDS-direct stage copies by the accumulators: load j of accumulator r4 fills bytes
  // [1024 (9 r4 + j), +1024) of the buffer; position pp of row t receives chunk
  // pp ^ split_swizzle(t) of that row
  uint32_t dma_off[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int c = (pvj * kDmaPerWave + j) * kWave + lane;
    const int t = c / kRowChunks, pp = c % kRowChunks;
    dma_off[j] = (uint32_t)(16 * (t * kRowChunks + (pp ^ split_swizzle(t))));
  }
  const uint32_t sbuf_lds = (uint32_t)(uintptr_t)(lds_void_t*)sbuf;
  auto issue_stage = [&](int n) {
    if (!copier) return;
    const i32x4_t src = stage_src(n);
    const uint32_t base = sbuf_lds + (n % NBUF) * kStageBytes + pvj * kDmaPerWave * 1024;
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) lds_copy16(src, dma_off[j], base + j * 1024);
  };

  // ---- scorer: K (A operand) of token tile tt.  Product ks < 16 contracts chunk ks + 16 g
  // (lane group g), products 16 and 17 the tail chunks 64 + 4 (ks - 16) + split_tail(g);
  // q is loaded with the same chunk assignment.  k_main[e] is the offset of chunk 16 g + e of
  // row i16 (e < 8; chunks 16 g + 8 + e are 128 bytes further), k_tail[ks - 16] of the tail
  // chunk; row i16 + 16 (token tile 1) has the same swizzle, kTileRows bytes further.
  const int tail_g = 2 * (g & 1) + (g >> 1);
  constexpr int kTileRows = 16 * kRow;
  int k_main[8], k_tail[2];
  {
    const int t = i16, sw = split_swizzle(t);
#pragma unroll
    for (int e = 0; e < 8; ++e) k_main[e] = 16 * (t * kRowChunks + 16 * g + (e ^ sw));
#pragma unroll
    for (int k = 0; k < 2; ++k) k_tail[k] = 16 * (t * kRowChunks + 64 + ((4 * k + tail_g) ^ sw));
  }
  // ---- accumulator: V (B operand, transposed reads) for dims 128 r4 + 16 nt + i16.  Read h
  // of lane group g takes the 4-token block 4 (g >> 1) + 2 h + (g & 1) (so that each 32-lane
  // half reads 8 consecutive rows); P is stored in the matching k order.
  int v_off[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 4 * (4 * (g >> 1) + 2 * h + (g & 1)) + (i16 >> 2);
    const int qd = (i16 & 3) >> 1, half8 = 8 * (i16 & 1);
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4)
      v_off[h][n4] = 16 * (t * kRowChunks + (DPW / 8) * pvj + ((2 * n4 + qd) ^ split_swizzle(t))) + half8;
  }

  const float cscale = a.scale * kLog2e;
  auto row0_of = [&](int sq) { return ((size_t)ch + sq) * Hq + (size_t)hg * HPU; };

  // Each kind of wave runs its own loop (so that its state is all the compiler keeps live);
  // both pass the same ns + 1 workgroup barriers.  At iteration n: stage n has landed (the
  // accumulators' copies of it are older than the newest NBUF - 3 stages'), P and alpha of
  // stage n - 1 are in LDS, and every wave is done with the buffer of stage n - 2, which the
  // copy issued next overwrites.
  if (scorer) {
    bf16x8_t qf[kDqk / 32];  // q of head r4 * 16 + i16, this lane's dims
    float m_run = kNegInf, l_part = 0.f;
    auto load_q = [&](int sq) {  // q of head r4 * 16 + i16 of sequence sq, no wait
      const uint8_t* qrow =
          (const uint8_t*)(a.q + ((size_t)sq * Hq + (size_t)hg * HPU + r4 * 16 + i16) * kDqk);
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks) {
        const int chunk = ks < 16 ? ks + 16 * g : 64 + 4 * (ks - 16) + tail_g;
        qf[ks] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qrow + 16 * chunk));
      }
    };
    // The first piece's q is requested before the first barrier, alongside the first stage
    // copies.  O is not cleared at a piece start: with the running max back at -inf, the
    // piece's first stage with a valid token sends alpha = 2^(-inf) = 0, which clears the
    // accumulators' rows.
    int seq = stage_info(0) >> 6;  // sequence of the open piece
    load_q(seq);
    auto flush_ml = [&]() {  // m and l of the open piece (slot ch + seq)
      const float l_head = group_sum4(l_part);
      if (g == 0) {
        a.ws_m[row0_of(seq) + r4 * 16 + i16] = m_run;
        a.ws_l[row0_of(seq) + r4 * 16 + i16] = l_head;
      }
    };
    for (int n = 0; n <= ns; ++n) {
      barrier_vm<kDmaPerWave * (NBUF - 3)>();
      if (n == ns) break;
      const int info = stage_info(n), valid = info & 63, sq = info >> 6;
      if (sq != seq) {
        flush_ml();
        seq = sq;
        load_q(sq);
        wait_vm<0>();  // scorers issue no stage copies: this only waits for q
        m_run = kNegInf;
        l_part = 0.f;
      }
      const uint8_t* buf = sbuf + (n % NBUF) * kStageBytes;
      // S^T = K Q^T for both token tiles (two independent accumulation chains).  The K
      // fragments are read in groups of KG products, each group's reads issued before the
      // previous group's products (two groups in registers, at most 4 KG reads in flight:
      // within the LDS counter's range), so that no product waits on a read issued just
      // before it.
      f32x4_t s[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
      constexpr int KG = kScoreGroup, NGRP = kDqk / 32 / KG;
      bf16x8_t kf[2][2][KG];  // [group parity][token tile][product]
      auto read_group = [&](int grp, bf16x8_t (&dst)[2][KG]) {
#pragma unroll
        for (int ks = 0; ks < KG; ++ks)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int kk = grp * KG + ks;
            const int off =
                tt * kTileRows + (kk < 16 ? k_main[kk & 7] + 128 * (kk >> 3) : k_tail[kk - 16]);
            dst[tt][ks] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(buf + off));
          }
      };
      read_group(0, kf[0]);
#pragma unroll
      for (int grp = 0; grp < NGRP; ++grp) {
        if (grp + 1 < NGRP) read_group(grp + 1, kf[(grp + 1) & 1]);
        sched_fence();
#pragma unroll
        for (int ks = 0; ks < KG; ++ks)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) s[tt] = mfma_bf16(kf[grp & 1][tt][ks], qf[grp * KG + ks], s[tt]);
        sched_fence();
      }

      // online softmax (log2 domain): lane holds tokens tt * 16 + 4 g + r of head i16.  The
      // maximum is taken over the raw scores and scaled once (cscale > 0).
      float sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = s[i >> 2][i & 3];
      if (valid < kStage) {  // last stage of a sequence: tokens past its end get p = 0
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i >> 2) * 16 + 4 * g + (i & 3) >= valid) sv[i] = kNegInf;
      }
      float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mt = group_max4(mt) * cscale;
      float alpha = 1.f;
      const bool rescale = wave_any(mt > m_run + kSlack);
      if (rescale) {
        const float m_new = fmaxf(m_run, mt);
        alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
        l_part *= alpha;
        m_run = m_new;
      }
      if (g == 0) sAlpha[n & 1][r4 * 16 + i16] = alpha;
      if (lane == 0) sRescale[n & 1][r4] = rescale;
      const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;
      // P in fp16 (bf16's 8-bit significand is too coarse for the weights of short
      // contexts); tokens tt * 16 + 4 g .. + 3 are k positions 8 (2 tt + (g & 1)) + 4 (g >> 1) .. + 3
      uint8_t* prow = sP[n & 1] + 1024 * (g & 1) + 16 * (r4 * 16 + i16) + 8 * (g >> 1);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint32_t p01 = pack_f16(fast_exp2(fmaf(sv[tt * 4 + 0], cscale, neg_m)),
                                      fast_exp2(fmaf(sv[tt * 4 + 1], cscale, neg_m)));
        const uint32_t p23 = pack_f16(fast_exp2(fmaf(sv[tt * 4 + 2], cscale, neg_m)),
                                      fast_exp2(fmaf(sv[tt * 4 + 3], cscale, neg_m)));
        l_part = dot2h(p01, kOnesF16x2, l_part);
        l_part = dot2h(p23, kOnesF16x2, l_part);        *(uint2*)(prow + 2048 * tt) = uint2{p01, p23};
      }
    }
    flush_ml();
  } else {
    f32x4_t o[HT][NT];  // O^T rows 4 g + r of each head tile, dims 128 r4 + 16 nt + i16
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[ht][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};  // finite for alpha = 0
    for (int n = 0; n < NBUF - 2; ++n) issue_stage(n);
    for (int n = 0; n <= ns; ++n) {
      if (copier) barrier_vm<kDmaPerWave * (NBUF - 3)>();  // this wave's copies of stage n
      else barrier_vm<63>();
      issue_stage(n + NBUF - 2);
      if (n == 0) continue;
      const int pn = n - 1;
      // scale O's rows by their heads' alpha when some score wave moved its running max (rare)
      if (__builtin_amdgcn_readfirstlane(*(const uint32_t*)sRescale[pn & 1])) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const float4 al = *(const float4*)&sAlpha[pn & 1][ht * 16 + 4 * g];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            o[ht][nt][0] *= al.x;
            o[ht][nt][1] *= al.y;
            o[ht][nt][2] *= al.z;
            o[ht][nt][3] *= al.w;
          }
        }
      }
      f16x8_t pf[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        pf[ht] = __builtin_bit_cast(f16x8_t, *(const uint4*)(sP[pn & 1] + 1024 * g + 16 * (ht * 16 + i16)));
      const lds_char_t* lbuf = (const lds_char_t*)((lds_void_t*)(sbuf + (pn % NBUF) * kStageBytes));
      uint2 vr[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          vr[nt][h] = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                         (lds_s16x4_t*)(lbuf + v_off[h][nt & 3] + 128 * (nt >> 2))));
      sched_fence();
      // widen all of V first, in place, then issue the 32 products back to back (widening
      // slice by slice into shared registers makes each slice wait for the products
      // still reading the previous one)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          vr[nt][h].x = bf16x2_to_f16x2(vr[nt][h].x);
          vr[nt][h].y = bf16x2_to_f16x2(vr[nt][h].y);
        }
      sched_fence();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f16x8_t vf = __builtin_bit_cast(
            f16x8_t, uint4{vr[nt][0].x, vr[nt][0].y, vr[nt][1].x, vr[nt][1].y});
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) o[ht][nt] = mfma_f16(pf[ht], vf, o[ht][nt]);
      }
      if (n == ns || opens_piece(n)) {  // stage pn closed its piece: write o (slot ch + seq)
        const size_t row0 = row0_of(stage_info(pn) >> 6);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              a.ws_o[(row0 + ht * 16 + 4 * g + r) * kDv + DPW * pvj + 16 * nt + i16] = o[ht][nt][r];
      }
    }
  }
  // Copies of stages past the end may still be in flight: they must land before this
  // workgroup's LDS can be handed to another one.
  wait_vm<0>();
}

// 64 heads per workgroup (two waves' worth of p.V accumulators per wave) where Hq allows,
// else 32.
int mla_stream_heads_per_group(int Hq) {
  if (Hq > 128) return 0;
  return Hq % 64 == 0 ? 64 : (Hq % 32 == 0 ? 32 : 0);
}

hipError_t launch_mla_stream(const MlaArgs& a, hipStream_t s) {
  constexpr int NBUF = 4;
  const int hpu = mla_stream_heads_per_group(a.Hq);
  if (a.d_qk != kDqk || a.d_v != kDv || a.block_size != kBlock || a.B > kMaxMlaSeqs || !hpu ||
      a.chunks % 8)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.Hq / hpu * a.chunks));
  if (hpu == 64)
    hipLaunchKernelGGL((mla_split_kernel<NBUF, kPvWaves>), grid, dim3((4 + kPvWaves) * kWave), 0, s, a);
  else
    hipLaunchKernelGGL((mla_stream_kernel<2, NBUF>), grid, dim3(kMThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecodeArgs m{};
  m.out = a.out;
  m.ws_m = a.ws_m;
  m.ws_l = a.ws_l;
  m.ws_o = a.ws_o;
  m.B = a.B;
  m.Hq = a.Hq;
  m.Hkv = 1;
  m.d = kDv;
  m.chunks = a.chunks;
  m.ws_prefix = a.ws_prefix;
  m.ws_seg = a.ws_seg;
  return launch_stream_merge(m, s);
}

}  // namespace pkv
