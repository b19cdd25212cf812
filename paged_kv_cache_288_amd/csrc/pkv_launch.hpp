// Internal host-side launchers; each kernel translation unit defines its own.  Arguments
// are validated by the C-ABI layer (pkv_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct AppendArgs {
  void* k_pool;
  void* v_pool;
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
  int32_t T, num_blocks, Hkv, block_size;
  int32_t row_bytes;  // d * element bytes
};
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);

struct AppendFp8Args {
  uint8_t* k_pool;  // [num_blocks][Hkv][block_size][d] E4M3 codes
  uint8_t* v_pool;  // may be null (K only)
  const uint16_t* k_new;  // [T][Hkv][d] bf16
  const uint16_t* v_new;
  const float* k_scale;  // [Hkv]
  const float* v_scale;
  const int64_t* slots;
  int32_t T, num_blocks, Hkv, block_size, d;
};
hipError_t launch_kv_append_fp8(const AppendFp8Args& a, hipStream_t s);

struct CopyBlocksArgs {
  uint8_t* k_pool;
  uint8_t* v_pool;  // may be null
  const int32_t* src;
  const int32_t* dst;
  int32_t n, num_blocks;
  int64_t block_bytes;  // bytes of one physical block of one pool (multiple of 16)
};
hipError_t launch_kv_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);

struct DecodeArgs {
  float* out;
  const uint16_t* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* ws_m;  // [B][Hq][P]
  float* ws_l;  // [B][Hq][P]
  float* ws_o;  // [B][Hq][P][d]
  int32_t B, Hq, Hkv, d, block_size, num_blocks, max_blocks, max_context_len;
  int32_t partition, num_partitions;  // num_partitions == 1: no split, out written directly
  float scale;
  int32_t fp8;
  // balanced mode: number of equal chunks (one per wave, a multiple of 32), and what the
  // decode kernel leaves for the merge kernel: the per-sequence tile prefix [B + 1] and per
  // segment (first chunk, chunks spanned) [Hkv * B][2]
  int32_t chunks;
  int32_t* ws_prefix;
  int32_t* ws_seg;
  // 1 when the device hands a grid's workgroups to 8 XCDs in turn (the whole chip as one
  // partition): the balanced kernels then read which XCD runs them to place weighted ranges
  int32_t xcd8;
};
hipError_t launch_gqa_decode(const DecodeArgs& a, hipStream_t s);
// Balanced mode: decode kernel + merge kernel (always both).
hipError_t launch_gqa_stream(const DecodeArgs& a, hipStream_t s);
// Waves per CU (one workgroup per CU) of the balanced single-token decode kernel.
int ring_waves_per_cu(int d, int G, bool fp8);
// Merge of balanced-mode pieces for d_v = D (128, 64 or 512); reads a.ws_* and a.ws_prefix.
hipError_t launch_stream_merge(const DecodeArgs& a, hipStream_t s);
hipError_t launch_partition_merge(const float* ws_m, const float* ws_l, const float* ws_o,
                                  const int32_t* context_lens, float* out, int32_t B,
                                  int32_t Hq, int32_t d, int32_t partition,
                                  int32_t num_partitions, int32_t max_context_len,
                                  int32_t max_ctx_clamp, hipStream_t s);

struct MlaArgs {
  float* out;
  const uint16_t* q;
  const uint16_t* kv_pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int32_t B, Hq, d_qk, d_v, block_size, num_blocks, max_blocks, max_context_len;
  int32_t partition, num_partitions;
  float scale;
  // balanced mode: chunks per head group (a multiple of 8), and what the decode kernel leaves
  // for the merge kernel: the per-sequence stage prefix [B + 1] and per sequence (first
  // chunk, chunks spanned) [B][2]
  int32_t chunks;
  int32_t* ws_prefix;
  int32_t* ws_seg;
};
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t s);
// Balanced mode: decode kernel + merge kernel.  Heads per workgroup for a given Hq
// (0 = the balanced mode does not support this Hq).
int mla_stream_heads_per_group(int Hq);
hipError_t launch_mla_stream(const MlaArgs& a, hipStream_t s);

// Debug check of block tables, context lengths and append slots (counts into counts[4]).
struct ValidateArgs {
  int32_t* counts;  // [6]
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t B, max_blocks, num_blocks, block_size;
  int32_t max_context_len;  // < 0: not checked
  const int64_t* slots;     // may be null
  int32_t T;
  const uint16_t* v_pool;   // bf16 [num_blocks][Hkv][block_size][d], may be null
  int32_t Hkv, d, d_v;      // first d_v dims of each row are the values checked
};
hipError_t launch_validate(const ValidateArgs& a, hipStream_t s);

// Multi-token decode (q_len query tokens per sequence, causal among them), balanced mode
// only.  Row n of segment (g, b) is query token n / G, head g * G + n % G.  The same kernel
// serves the shared-prefix pass of the cascade call: there the "sequences" are groups of
// q_len real sequences (q row b * q_len + j is real sequence b * q_len + j), all of them
// reading the same block-table row (table_stride 0) of fixed_len tokens, without the
// causal mask.
struct MultiArgs {
  float* out;           // [B][q_len][Hq][d] (merged output; unused when only pieces are made)
  const uint16_t* q;    // [B][q_len][Hq][d] bf16
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const float* k_scale;  // [Hkv] (FP8) or null
  const float* v_scale;
  const int32_t* block_table;   // row b at b * table_stride
  const int32_t* context_lens;  // [B], unused when fixed_len >= 0
  float* ws_m;  // [S][R], S = chunks + Hkv * B piece slots, R = q_len * Hq / Hkv rows
  float* ws_l;  // [S][R]
  float* ws_o;  // [S][R][d]
  int32_t* ws_prefix;  // [B + 1]
  int32_t* ws_seg;     // [Hkv * B][2]
  int32_t B, q_len, Hq, Hkv, d, block_size, num_blocks;
  int32_t max_blocks;    // valid table entries per sequence
  int32_t max_len;       // cap on context lengths (the host's max_context_len)
  int32_t table_stride;  // elements between table rows (0: one row shared by all)
  int32_t fixed_len;     // >= 0: every sequence has this length
  int32_t q_rows;        // real q rows along (b, j): B * q_len, fewer in prefix mode
  int32_t causal, fp8;
  float scale;
  int32_t chunks;  // one per resident wave, a multiple of 32
  int32_t xcd8;    // as DecodeArgs::xcd8
};
// Decode kernel + merge kernel.
hipError_t launch_gqa_multi(const MultiArgs& a, hipStream_t s);
// The decode kernel only (the ring or the register-tile kernel, as launch_gqa_multi picks),
// leaving its pieces (rows of q_len * G per slot) for a later merge.  With q_len = 1 they
// are laid out as the single-token balanced kernel's, so launch_stream_merge combines them.
hipError_t launch_gqa_multi_pieces(const MultiArgs& a, hipStream_t s);
// Resident waves per CU of the multi-token decode kernel for head dim d and q_len * G rows.
int multi_waves_per_cu(int d, int rows);
// Whether the multi-token call runs the LDS-ring kernel (then multi_ring_waves_per_cu()
// waves per CU, up to 512 tiles per wave).
bool multi_uses_ring(int d, int rows, bool fp8);
int multi_ring_waves_per_cu();

// Balanced-mode single-token decode kernel only (pieces for a later merge).
hipError_t launch_gqa_stream_pieces(const DecodeArgs& a, hipStream_t s);

// Cascade merge: out[b][h] combines the tail pieces of (h / G, b) from the single-token
// balanced kernel with the prefix pieces of row (b % J) * G + h % G of segment
// (h / G, b / J) from the multi-token kernel (J = q_len of the prefix pass).
struct CascadeMergeArgs {
  float* out;  // [B][Hq][d]
  int32_t B, Hq, Hkv, d;
  const float *t_m, *t_l, *t_o;          // tail pieces: rows of G
  const int32_t *t_prefix, *t_seg;
  int32_t t_chunks;
  const float *p_m, *p_l, *p_o;          // prefix pieces: rows of J * G (null: no prefix)
  const int32_t *p_prefix, *p_seg;
  int32_t p_chunks, p_B, p_J;
};
hipError_t launch_cascade_merge(const CascadeMergeArgs& a, hipStream_t s);
// Tail pass (ta, single-token balanced) and prefix pass (pa, multi-token with 32 rows) of
// the cascade in one launch: grid (ta.chunks + pa.chunks) / 4, pieces only.
hipError_t launch_cascade(const DecodeArgs& ta, const MultiArgs& pa, hipStream_t s);

}  // namespace pkv
