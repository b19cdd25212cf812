// Device helpers for the gfx950 (CDNA4) kernels: wave64 cross-lane moves, bf16 pairs
// for v_dot2c_f32_bf16, FP8 E4M3 -> bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------- DPP controls (gfx9 encoding)
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <- lane 7-i within 8 lanes
constexpr int kDppRowRor8 = 0x128;     // row_ror:8: lane i <- lane (i+8)%16 within a row
constexpr int kDppRowNewBcast = 0x150; // row_newbcast:n: every lane of a row <- lane n of it

// Every control used here reads a valid lane for every lane, so bound_ctrl never applies;
// setting it lets the compiler skip initialising the destination.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

// Broadcast lane n (0..15) of each 16-lane row to the whole row.
template <int N>
__device__ __forceinline__ float row_bcast(float x) { return dpp<kDppRowNewBcast + N>(x); }
template <int N>
__device__ __forceinline__ uint32_t row_bcast_u(uint32_t x) { return dpp_u<kDppRowNewBcast + N>(x); }

// Exchange between row pairs (0<->1, 2<->3): returns {value of the even row, value of the
// odd row} of each pair, in every lane of both rows.
__device__ __forceinline__ void rows_pair16(float x, float& even, float& odd) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  even = __builtin_bit_cast(float, (uint32_t)r[0]);
  odd = __builtin_bit_cast(float, (uint32_t)r[1]);
}
// Exchange between wave halves: returns {lower-half value, upper-half value} in every lane.
__device__ __forceinline__ void halves_pair32(float x, float& lo, float& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  lo = __builtin_bit_cast(float, (uint32_t)r[0]);
  hi = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// ---------------------------------------------------------------- arithmetic helpers
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
// dot2(a, b, 0) in the three-operand encoding, whose accumulator can be the constant 0
// (the two-operand form accumulates in place and would need a zeroed register).
__device__ __forceinline__ float dot2_zero(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}
// (lo, hi) -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
// Two FP8 E4M3 bytes (low or high 16 bits of x) -> two fp16 (exact).
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HIGH));
}
// bf16 halves of x as fp32 values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __builtin_bit_cast(float, x & 0xFFFF0000u); }
// (lo, hi) -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// Two FP8 E4M3 bytes (low or high 16 bits of x) -> two bf16 (exact).
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HIGH));
}
__device__ __forceinline__ uint32_t byte_perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // (1.0, 1.0) in bf16
constexpr uint32_t kOnesF16x2 = 0x3C003C00u;    // (1.0, 1.0) in fp16

// ---------------------------------------------------------------- buffer resources
// A raw buffer resource over [base, base + bytes): loads at offsets past `bytes` return zeros
// without a memory access (stores there are dropped).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 resource word 3: raw 32-bit data
constexpr int kLoadNontemporal = 2;          // cache-policy operand: nt
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRawBufferWord3);
}

// s_waitcnt with vmcnt <= VM (0..63) only.
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14));
}
// s_waitcnt with vmcnt <= VM (0..63) and lgkmcnt = 0 (expcnt not waited for).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
}
// Workgroup barrier that waits only for this wave's LDS operations and its vector memory
// operations beyond the newest VM (HIP's __syncthreads also drains every global access).
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  asm volatile("" ::: "memory");
  wait_vm_lgkm0<VM>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Nothing is scheduled across this point (keeps loads where the source puts them).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// ---------------------------------------------------------------- balanced-mode bookkeeping
// The balanced kernels lay the units of work (16-token tiles, or stages) of all (head g,
// sequence b) segments end to end, head-major, and cut the T units into C equal ranges:
// range c covers [T c / C, T (c + 1) / C).  First range holding unit t:
__device__ __forceinline__ int chunk_of(long long t, long long T, int C) {
  return (int)(((t + 1) * (long long)C - 1) / T);
}
// For the merge kernel, per segment s = g * B + b: the first range holding its units and the
// number of ranges it spans (0 for a sequence without units).  pre[0..B] is the exclusive
// prefix of units per sequence; threads tid, tid + nthreads, ... of one workgroup write.
// First range and number of ranges of a segment of nb units starting at unit `first`.
__device__ __forceinline__ void segment_range(long long first, int nb, long long T, int C,
                                              int32_t* out) {
  int c0 = 0, n = 0;
  if (nb > 0) {
    c0 = chunk_of(first, T, C);
    n = chunk_of(first + nb - 1, T, C) - c0 + 1;
  }
  out[0] = c0;
  out[1] = n;
}
template <typename PRE>  // any pointer to int (generic or LDS)
__device__ __forceinline__ void write_segment_ranges(int32_t* ws_seg, PRE pre, int B,
                                                     int H, int C, int tid, int nthreads) {
  const int T_head = pre[B];
  const long long T = (long long)H * T_head;
  for (int sg = tid; sg < H * B; sg += nthreads) {
    const int g = sg / B, b = sg - g * B;
    segment_range((long long)g * T_head + pre[b], pre[b + 1] - pre[b], T, C, ws_seg + 2 * sg);
  }
}

// ---- XCD-weighted ranges.  On MI355X the odd-numbered XCDs were measured to stream the
// single-token decode 6-10 % slower than the even ones on most boxes (their waves finished
// 15-20 us later on a 200 us call).  Workgroups go to the XCDs in turn: workgroup i runs on
// XCD (i + r) mod 8, r the same for the whole grid but set by the dispatches before it.  The
// balanced kernels give wave w of workgroup i the chunk e * C/8 + (i / 8) * waves + w, with
// e = i mod 8 (weighted: with its lowest bit matched to the parity of the XCD it runs on), so
// each XCD owns C/8 consecutive chunks.  (The register-tile multi-token kernel, at 8 waves
// per CU and about 74 tiles per chunk on the 70B-shaped verify batch, measured 2.6 % slower
// weighted, and splits evenly.)  Weighted WE:WO, the chunks of even XCDs take WE parts of
// the tiles for the odd ones' WO, H = (WE + WO) / 2 parts on average: W(c) counts the parts
// of chunks 0 .. c-1, and chunk c covers tiles [T W(c) / HC, T W(c+1) / HC).  Unweighted,
// W(c) = H c: the equal split above.
template <int WE, int WO>
__device__ __forceinline__ long long xcd_chunk_start(int c, long long T, int C, bool wtd) {
  static_assert(WE > WO && (WE + WO) % 2 == 0, "XCD weights");
  constexpr int H = (WE + WO) / 2;
  if (!wtd) return T * c / C;
  const int E = C / 8, x = c / E, r = c - x * E;
  const long long W = (long long)E * (WE * ((x + 1) >> 1) + WO * (x >> 1)) +
                      (long long)r * ((x & 1) ? WO : WE);
  return T * W / ((long long)H * C);
}
// The chunk holding tile t (0 <= t < T): the last c with xcd_chunk_start(c) <= t.
template <int WE, int WO>
__device__ __forceinline__ int xcd_chunk_of(long long t, long long T, int C, bool wtd) {
  constexpr int H = (WE + WO) / 2;
  if (!wtd) return chunk_of(t, T, C);
  const long long E = C / 8;
  const long long ws = ((t + 1) * H * C - 1) / T;  // largest W(c) that still starts <= t
  const long long pair = ws / (2 * H * E), rem = ws - pair * 2 * H * E;
  if (rem < WE * E) return (int)(2 * pair * E + rem / WE);
  return (int)((2 * pair + 1) * E + (rem - WE * E) / WO);
}
// Whether to weight: chunks hold at least min_tiles tiles on average (below that the
// weighting was measured to cost more than it saved), and the heavier chunks, up to
// T * WE / HC + 1 tiles, still fit a wave's max_tiles.
template <int WE, int WO>
__device__ __forceinline__ bool xcd_weighted(long long T, int C, int min_tiles, int max_tiles) {
  constexpr int H = (WE + WO) / 2;
  return T >= (long long)min_tiles * C && WE * T <= (long long)H * C * (max_tiles - 1);
}
// write_segment_ranges over the (possibly weighted) ranges.
template <int WE, int WO, typename PRE>
__device__ __forceinline__ void write_segment_ranges_xcd(int32_t* ws_seg, PRE pre, int B, int H,
                                                         int C, bool wtd, int tid, int nthreads) {
  const int T_head = pre[B];
  const long long T = (long long)H * T_head;
  for (int sg = tid; sg < H * B; sg += nthreads) {
    const int g = sg / B, b = sg - g * B;
    const int nb = pre[b + 1] - pre[b];
    int c0 = 0, n = 0;
    if (nb > 0) {
      const long long first = (long long)g * T_head + pre[b];
      c0 = xcd_chunk_of<WE, WO>(first, T, C, wtd);
      n = xcd_chunk_of<WE, WO>(first + nb - 1, T, C, wtd) - c0 + 1;
    }
    ws_seg[2 * sg] = c0;
    ws_seg[2 * sg + 1] = n;
  }
}

}  // namespace pkv
