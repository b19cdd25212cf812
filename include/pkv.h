/*
 * pkv.h — decode attention over a paged KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *  - "深入LLM推理：从KV Cache到PD分离的Serving全景解析", section "KV Cache：Transformer的循环状态":
 *    each decode step computes softmax(q K^T * scale) V for one new query token per head
 *    over every cached position; under GQA a group of query heads shares one K/V head.
 *  - same page, section "PagedAttention与Cache管理": the cache is a pool of fixed-size
 *    physical blocks; a per-sequence block table maps logical blocks to physical ones,
 *    blocks may be shared between sequences, and the kernel has to read this layout.
 *  - "PD 分离下的 KV Cache", section "先回顾：两个阶段": a decode step adds one token and
 *    reads the whole cache, so the step is bound by memory bandwidth.
 *
 * Conventions for every call:
 *  - All buffer pointers are DEVICE pointers to row-major, contiguous arrays, 16-byte
 *    aligned, allocated and owned by the caller.  The library keeps no pointer after
 *    returning and allocates nothing.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on it and
 *    the call returns without synchronising; buffers must stay alive until the stream
 *    has passed the work.
 *  - Host-checkable errors (NULL pointers, bad sizes, misalignment, unsupported shapes or
 *    dtypes, a too-small workspace) are returned before anything is launched.  A failed
 *    launch returns PKV_ERR_HIP.  No C++ exception crosses this interface.
 *  - Device-resident indices are the caller's contract, but a bad value never causes an
 *    out-of-bounds access: block ids outside [0, num_blocks) are not read (their tokens
 *    are skipped and that sequence's output is then unspecified), context lengths are
 *    clamped to [0, max_blocks_per_seq * block_size], and append slots outside
 *    [0, num_blocks * block_size) are skipped.
 *  - Calls on different streams may overlap; the library has no global mutable state.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 2

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL                              */
  PKV_ERR_SHAPE = -2,       /* a size is non-positive or inconsistent                  */
  PKV_ERR_DTYPE = -3,       /* unknown element type                                    */
  PKV_ERR_UNSUPPORTED = -4, /* valid but not implemented (head dim, block size, group) */
  PKV_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                        */
  PKV_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required              */
  PKV_ERR_HIP = -7          /* the HIP runtime reported an error at launch             */
};

/* Element types of the KV pools. */
enum {
  PKV_BF16 = 1,             /* bfloat16                                                */
  PKV_FP8_E4M3 = 2          /* OCP FP8 E4M3 ("e4m3fn": bias 7, max 448, no inf), with
                               one fp32 scale per KV head for K and one for V; the
                               stored value is e4m3(byte) * scale                      */
};

/* Returns PKV_ABI_VERSION of the built library. */
int pkv_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* pkv_status_str(pkv_status s);

/*
 * pkv_kv_append — write T new tokens' K and V rows into the block pool.
 *
 * Cites: "深入LLM推理…" section "PagedAttention与Cache管理" (block + offset addressing) and
 * section "KV Cache：Transformer的循环状态" (history is never rewritten, only appended).
 *
 * For token i with s = slot_mapping[i] in [0, num_blocks*block_size):
 *     k_pool[s / block_size][h][s % block_size][0:d] = k_new[i][h][0:d]   for every h < Hkv
 * and the same for V.  Slots < 0 (and out-of-range slots) are skipped.  Every other byte
 * of the pools is left unchanged; the copy is bit-exact.  Duplicate slots in one call
 * are a caller error (the surviving row is unspecified).
 *
 *   k_pool, v_pool  [num_blocks][Hkv][block_size][d], element type kv_dtype.
 *                   v_pool may be NULL (then v_new must be NULL too): this is the
 *                   latent (MLA) cache, written with Hkv = 1.
 *   k_new, v_new    [T][Hkv][d], same element type as the pools.
 *   slot_mapping    [T] int64.
 * Requires d * element_bytes to be a multiple of 16.  T = 0 is a no-op.
 */
pkv_status pkv_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int32_t T, int32_t num_blocks,
                         int32_t Hkv, int32_t d, int32_t block_size, int32_t kv_dtype,
                         void* stream);

/*
 * pkv_decode_partition_size — how pkv_paged_decode_attn divides the work for these
 * arguments.  With partition_size > 0 each sequence's context is cut into partitions of
 * that many tokens (a result >= max_context_len means no split).  With partition_size = 0
 * the result is 0: the balanced mode, where the cached tiles of all (KV head, sequence)
 * pairs are laid end to end and cut into equal ranges, one per wave of the current device
 * (B up to 4096; larger batches fall back to a library-chosen partition, which is then
 * returned).  Negative = error code.
 */
int32_t pkv_decode_partition_size(int32_t B, int32_t Hkv, int32_t max_context_len,
                                  int32_t partition_size);

/*
 * pkv_decode_workspace_bytes — bytes of workspace pkv_paged_decode_attn needs for these
 * arguments on the current device (0 when a partitioned context is not split).  The
 * workspace holds the partial online-softmax states (running max, sum and unnormalised
 * output per query head) of partitions, or of the balanced mode's pieces, plus (balanced
 * mode) the per-sequence tile prefix and per-segment piece ranges the merge step reads.
 */
size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d_v,
                                  int32_t max_context_len, int32_t partition_size);

/*
 * pkv_paged_decode_attn — one decode step of GQA/MQA/MHA attention over the paged cache.
 *
 * Cites: "深入LLM推理…" section "KV Cache：Transformer的循环状态" (softmax(q K^T / sqrt d) V,
 * GQA head sharing) and "PagedAttention与Cache管理" (block table).  Long contexts are
 * split into partitions whose online-softmax partials are merged afterwards ("GPU推理深度
 * 拆解：KV Cache视角", sections "长上下文优化" and "算子优化要点").
 *
 * For sequence b with L = context_lens[b] and query head h (KV head g = h / (Hq/Hkv)):
 *     token t (0 <= t < L) lives at block block_table[b][t / block_size], offset
 *     t % block_size;  s_t = scale * k_scale[g] * dot(q[b][h], K_t)
 *     out[b][h] = v_scale[g] * sum_t softmax(s)_t V_t        (out = 0 when L = 0)
 * k_scale / v_scale are taken as 1 for bf16 pools.
 *
 *   out          [B][Hq][d] float32 (written)
 *   q            [B][Hq][d] bfloat16
 *   k_pool       [num_blocks][Hkv][block_size][d], kv_dtype
 *   v_pool       [num_blocks][Hkv][block_size][d], kv_dtype
 *   k_scale, v_scale  [Hkv] float32 for PKV_FP8_E4M3, ignored (may be NULL) for bf16
 *   block_table  [B][max_blocks_per_seq] int32 (entries past a sequence's end unused)
 *   context_lens [B] int32
 *   max_context_len   host-side upper bound of context_lens (sizes the grid)
 *   partition_size    tokens per partition (a multiple of 16, at most 4096), or 0 for the
 *                     balanced mode (see pkv_decode_partition_size)
 *   workspace, workspace_bytes  >= pkv_decode_workspace_bytes(...) with the same
 *                     arguments on the same device; may be NULL/0 when that is 0.
 * Supported: d = 128 with bf16 or FP8 pools, d = 64 with bf16 pools; block_size a
 * multiple of 16 (16, 32, 64, ...); Hq / Hkv in {1, 2, 4, 8}.  Other shapes return
 * PKV_ERR_UNSUPPORTED.  q and out must not alias the pools.
 * Precision: scores accumulate exact bf16 (or widened FP8) products in fp32; the
 * softmax weights are rounded to fp16 and V widened to fp16 for p.V, accumulated in fp32.
 * bf16 V values must therefore lie within fp16's range (|v| < 65504); FP8 values always do.
 * (bf16 values below 2^-14 in magnitude land on fp16's subnormal grid: absolute error
 * at most 2^-25 per value.)
 */
pkv_status pkv_paged_decode_attn(float* out, const void* q, const void* k_pool,
                                 const void* v_pool, const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, const int32_t* context_lens,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 float scale, int32_t kv_dtype, int32_t partition_size,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_attn_noalloc — pkv_paged_decode_attn for callers that cannot allocate
 * device memory: code running under HIP graph capture, serving loops that must not call
 * hipMalloc, harnesses that forbid it.  Same arguments, meaning, layouts, precision and
 * errors as pkv_paged_decode_attn, without the workspace: the call uses a device-resident
 * scratch array of the library, PKV_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the
 * first call on that GPU until the process ends.  Nothing is allocated by the call.
 *
 * Returns PKV_ERR_WORKSPACE when pkv_decode_workspace_bytes for these arguments exceeds
 * PKV_NOALLOC_SCRATCH_BYTES (e.g. the balanced mode of 64 sequences x 8 KV heads x 64
 * query heads needs 6.4 MB), and PKV_ERR_HIP when the scratch's device address cannot be
 * obtained.  Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents (the kernels need it in no particular state): calls that overlap in time on
 * one GPU (on different streams, or from different threads) race and give unspecified
 * results.  The call keeps one device address per GPU; it is safe to call from several
 * host threads as long as their GPU work does not overlap.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16 << 20)
pkv_status pkv_paged_decode_attn_noalloc(float* out, const void* q, const void* k_pool,
                                         const void* v_pool, const float* k_scale,
                                         const float* v_scale, const int32_t* block_table,
                                         const int32_t* context_lens, int32_t B, int32_t Hq,
                                         int32_t Hkv, int32_t d, int32_t block_size,
                                         int32_t num_blocks, int32_t max_blocks_per_seq,
                                         int32_t max_context_len, float scale, int32_t kv_dtype,
                                         int32_t partition_size, void* stream);

/*
 * pkv_mla_workspace_bytes — workspace bytes for pkv_paged_decode_attn_mla with these
 * arguments (0 when the context is not split).
 */
size_t pkv_mla_workspace_bytes(int32_t B, int32_t Hq, int32_t d_v, int32_t max_context_len,
                               int32_t partition_size);

/*
 * pkv_paged_decode_attn_mla — decode attention over a latent (MLA) cache.
 *
 * Cites: "深入LLM推理…" section "KV Cache：Transformer的循环状态" and "GPU推理深度拆解：KV Cache
 * 视角" section "KV Cache 大小与分配演进": one cached latent row per token (512 latent + 64
 * RoPE dims) serves every query head.  Reading: the key is the whole latent row and the
 * value its first d_v dims (MQA over the latent).
 *
 *     s_t = scale * dot(q[b][h][0:d_qk], C_t[0:d_qk]);  out[b][h] = sum_t softmax(s)_t C_t[0:d_v]
 *
 *   out      [B][Hq][d_v] float32;  q [B][Hq][d_qk] bfloat16
 *   kv_pool  [num_blocks][block_size][d_qk] bfloat16
 *   block_table, context_lens, max_context_len, partition_size, workspace: as above
 *   (partition_size a multiple of block_size, or 0 for the library's choice).
 * Supported: d_qk = 576, d_v = 512, block_size = 64, Hq a multiple of 16 (<= 128).
 * Precision: scores on the bf16 MFMA (fp32 accumulate); weights and the value dims in fp16
 * on the fp16 MFMA for p.V, so latent values must satisfy |v| < 65504 (values below 2^-14
 * in magnitude are rounded to fp16's subnormal grid, absolute error at most 2^-25).
 */
pkv_status pkv_paged_decode_attn_mla(float* out, const void* q, const void* kv_pool,
                                     const int32_t* block_table, const int32_t* context_lens,
                                     int32_t B, int32_t Hq, int32_t d_qk, int32_t d_v,
                                     int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * pkv_multi_workspace_bytes — workspace bytes for pkv_paged_decode_attn_multi with these
 * arguments (0 for an unsupported combination).
 */
size_t pkv_multi_workspace_bytes(int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t d,
                                 int32_t max_context_len);

/*
 * pkv_paged_decode_attn_multi — decode step with q_len query tokens per sequence, the
 * verify pass of speculative decoding.
 *
 * Cites: "深入LLM推理…" section "投机解码：打破每步一token的假设" (the target model checks
 * the drafted tokens in one forward pass; nearly free while decode is memory-bound) and
 * section "KV Cache：Transformer的循环状态" (softmax attention, GQA grouping).  The q_len new
 * tokens' K/V rows are already in the cache (appended with pkv_kv_append) and counted by
 * context_lens; the new tokens are causal among themselves:
 *
 *     L_j = context_lens[b] - q_len + 1 + j     (tokens that query token j sees)
 *     out[b][j][h] = sum_{t < L_j} softmax_t(scale * dot(q[b][j][h], K[h / G][t])) V[h / G][t]
 *
 * (out = 0 where L_j <= 0).
 *   out      [B][q_len][Hq][d] float32;  q [B][q_len][Hq][d] bfloat16
 *   k_pool, v_pool, k_scale, v_scale, kv_dtype, block_table, context_lens,
 *   max_context_len, workspace: as for pkv_paged_decode_attn (the workspace size from
 *   pkv_multi_workspace_bytes).
 * Supported: bf16 or FP8 K/V, d in {64, 128}, block_size a multiple of 16,
 * Hq / Hkv in {1, 2, 4, 8}, (Hq / Hkv) * q_len <= 64, B <= 4096.  Precision: scores on the bf16 MFMA (FP8 codes
 * widened exactly to bf16), weights and V in fp16 on the fp16 MFMA (fp32 accumulate), so
 * |v| < 65504 as for the latent call.
 */
pkv_status pkv_paged_decode_attn_multi(float* out, const void* q, const void* k_pool,
                                       const void* v_pool, const float* k_scale,
                                       const float* v_scale, const int32_t* block_table,
                                       const int32_t* context_lens, int32_t B, int32_t q_len,
                                       int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_context_len, float scale, int32_t kv_dtype,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_cascade_workspace_bytes — workspace bytes for pkv_paged_decode_attn_cascade with
 * these arguments (0 for an invalid combination).
 */
size_t pkv_cascade_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                   int32_t prefix_len, int32_t max_tail_len);

/*
 * pkv_paged_decode_attn_cascade — decode step for a batch whose sequences all start with
 * the same cached prefix.
 *
 * Cites: "深入LLM推理…" section "PagedAttention与Cache管理" (several sequences' block tables
 * point at the same physical blocks of a common prefix) and "PD 分离下的 KV Cache" section
 * "优化一：Prefix Cache（前缀缓存）" (requests sharing a system prompt reuse its KV).  The
 * result is exactly that of pkv_paged_decode_attn with block_table[b] = prefix_blocks
 * followed by tail_table[b] and context_lens[b] = prefix_len + tail_lens[b]:
 *
 *     out[b][h] = sum_t softmax_t(scale * dot(q[b][h], K_t)) V_t over the prefix's tokens
 *                 and then sequence b's own tail tokens (KV head h / G).
 *
 * The prefix is read once per group of 32 / G sequences, with the whole group's query rows
 * as one dense product on the matrix cores, instead of once per sequence; the tails run
 * through the single-token kernel, and one merge combines both.
 *   out            [B][Hq][d] float32;  q [B][Hq][d] bfloat16
 *   k_pool, v_pool, k_scale, v_scale, kv_dtype, scale: as for pkv_paged_decode_attn
 *   prefix_blocks  [prefix_len / block_size] int32 physical block ids (device); NULL
 *                  allowed when prefix_len = 0.  prefix_len: a multiple of block_size
 *                  (a partially filled shared block belongs to the tails).
 *   tail_table     [B][max_tail_blocks] int32;  tail_lens [B] int32 in
 *                  [0, max_tail_blocks * block_size] (clamped); max_tail_len >= every
 *                  tail length (sizes the work split and the workspace).
 *   workspace      >= pkv_cascade_workspace_bytes(...) device bytes, 16-byte aligned.
 * A sequence with no token at all (prefix_len = 0 and an empty tail) gets out = 0.
 * Supported: Hq / Hkv in {1, 2, 4, 8}, d = 128 (bf16 or FP8) or 64 (bf16), block_size a
 * multiple of 16, B <= 4096.  Precision: tails as pkv_paged_decode_attn; the prefix as
 * pkv_paged_decode_attn_multi (bf16 MFMA scores, fp16 MFMA p.V, FP8 codes widened
 * exactly).
 */
pkv_status pkv_paged_decode_attn_cascade(float* out, const void* q, const void* k_pool,
                                         const void* v_pool, const float* k_scale,
                                         const float* v_scale, const int32_t* prefix_blocks,
                                         int32_t prefix_len, const int32_t* tail_table,
                                         const int32_t* tail_lens, int32_t B, int32_t Hq,
                                         int32_t Hkv, int32_t d, int32_t block_size,
                                         int32_t num_blocks, int32_t max_tail_blocks,
                                         int32_t max_tail_len, float scale, int32_t kv_dtype,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_validate — count violations of the caller's contract on the device (a debug aid).
 *
 * Cites: "深入LLM推理…" section "PagedAttention与Cache管理" (a sequence's table entries name
 * physical blocks of the pool; each new token gets its own slot).  The decode and append
 * calls never fault on bad values but their results are then unspecified; this call finds
 * them, and the values the decode calls would silently truncate or lose.  Writes six
 * int32 counts to the device array counts[6]:
 *   counts[0]  table entries in use (the first ceil(L / block_size) of each row, L clamped to
 *              the table) outside [0, num_blocks)
 *   counts[1]  context lengths outside [0, max_blocks_per_seq * block_size]
 *   counts[2]  slots at or past num_blocks * block_size (negative slots mean "skip", legal)
 *   counts[3]  non-negative slots already used by an earlier token of the same append
 *              (quadratic in T: meant for checking, not for every step)
 *   counts[4]  context lengths above max_context_len (the decode calls attend to the first
 *              max_context_len tokens only); not checked when max_context_len < 0
 *   counts[5]  bf16 values of V in use (the first d_v dims of each KV head's row of every
 *              token within the clamped lengths, in blocks whose id is valid) of magnitude
 *              65504 or more, infinities included: the p.V step widens V to fp16, where
 *              they would become infinite; not checked when v_pool is NULL
 * block_table [B][max_blocks_per_seq], context_lens [B] int32; slot_mapping [T] int64 (may
 * be NULL when T = 0); v_pool: a bf16 pool [num_blocks][Hkv][block_size][d] (the V pool,
 * or a latent pool with Hkv = 1, d = 576, d_v = 512), or NULL; FP8 pools never overflow
 * fp16 and need no check.  Enqueued on `stream` like the other calls; counts are valid once
 * the stream has passed the work.  Errors: PKV_ERR_SHAPE, PKV_ERR_NULL, PKV_ERR_ALIGN,
 * PKV_ERR_HIP.
 */
pkv_status pkv_validate(int32_t* counts, const int32_t* block_table,
                        const int32_t* context_lens, int32_t B, int32_t max_blocks_per_seq,
                        int32_t num_blocks, int32_t block_size, int32_t max_context_len,
                        const int64_t* slot_mapping, int32_t T, const void* v_pool, int32_t Hkv,
                        int32_t d, int32_t d_v, void* stream);

/*
 * pkv_kv_append_fp8 — quantizing append ("PD 分离下的 KV Cache", "优化三：KV 传输优化": KV
 * kept as FP8): token i's bf16 rows k_new/v_new [T][Hkv][d] are written as FP8 E4M3 (OCP
 * e4m3fn) codes into slot_mapping[i] of the FP8 pools [num_blocks][Hkv][block_size][d],
 * with the pools' per-KV-head scales k_scale/v_scale [Hkv] (fp32, device):
 * code = the E4M3 value nearest to the fp32 quotient x / scale[h] (IEEE division), ties
 * to the even code; magnitudes >= 448 and infinities saturate to +-448, NaN stays NaN.
 * The decode call then reads code * scale[h].  v_pool and v_new may both be NULL (K only).
 * Slots < 0 or outside the pool are skipped.  d must be a multiple of 16; pools and new
 * rows 16-byte aligned, scales 4-byte aligned.  Errors as pkv_kv_append.
 */
pkv_status pkv_kv_append_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                             const float* k_scale, const float* v_scale,
                             const int64_t* slot_mapping, int32_t T, int32_t num_blocks,
                             int32_t Hkv, int32_t d, int32_t block_size, void* stream);

/*
 * pkv_kv_copy_blocks — copy-on-write support ("深入LLM推理：从KV Cache到PD分离的Serving全景
 * 解析", "PagedAttention与Cache管理": physical blocks shared between requests): for i < n,
 * physical block dst_blocks[i] of each pool becomes a copy of block src_blocks[i] (every
 * KV head and row).  src_blocks/dst_blocks are device int32 arrays [n]; pairs with an id
 * outside [0, num_blocks) are skipped; a block must not be both a source and a
 * destination of one call.  Pools [num_blocks][Hkv][block_size][d] of kv_dtype (an MLA
 * latent pool: Hkv = 1, v_pool NULL).  Errors: PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_NULL,
 * PKV_ERR_ALIGN (pools 16-byte aligned, rows a multiple of 16 bytes), PKV_ERR_HIP.
 */
pkv_status pkv_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_blocks,
                              const int32_t* dst_blocks, int32_t n, int32_t num_blocks,
                              int32_t Hkv, int32_t d, int32_t block_size, int32_t kv_dtype,
                              void* stream);

/*
 * pkv_block_hashes — host function, the prefix-cache key chain ("PD 分离下的 KV Cache",
 * "优化一：Prefix Cache（前缀缓存）"): hash_i = H(hash_{i-1}, tokens of block i) for each of
 * the n_tokens / block_size full blocks of `tokens` (host int32 array), hash_{-1} =
 * `parent` (0 for a sequence start, or the hash of the block before, to continue a
 * chain).  H is 64-bit FNV-1a over hash_{i-1} as 8 little-endian bytes followed by the
 * block's tokens as little-endian int32.  Writes the hashes to `hashes` (host, room for
 * n_tokens / block_size values) and returns their number; PKV_ERR_NULL / PKV_ERR_SHAPE on
 * bad arguments.  No GPU work.
 */
int32_t pkv_block_hashes(const int32_t* tokens, int32_t n_tokens, int32_t block_size,
                         uint64_t parent, uint64_t* hashes);

/* ---- Graph capture of a decode step ("GPU推理深度拆解：KV Cache视角", "算子优化要点":
 * replaying a captured step removes the per-kernel launch overhead, at the price of static
 * shapes and addresses, so steps are padded to the nearest bucket).
 *
 * pkv_graph_begin starts capturing what is enqueued on `stream` (not the null stream) from
 * this thread; the library calls made on that stream until pkv_graph_end are recorded, not
 * run.  pkv_graph_end stops the capture and instantiates it into *graph (caller-owned,
 * released by pkv_graph_destroy).  pkv_graph_launch enqueues one replay on `stream`.
 *
 * A replay runs the recorded kernels with the pointers and sizes they were given: the
 * caller updates the buffers' contents in place (q, new rows, slot mapping, block table,
 * context lengths) between replays and keeps every buffer and the workspace alive until
 * the graph is destroyed.  The library's calls record kernel launches only (no memory set
 * or copy nodes), so a replay needs no clearing.  Errors: PKV_ERR_NULL for a missing
 * stream or graph pointer, PKV_ERR_HIP when the runtime rejects the capture (a library call
 * that fails while capturing returns its own status; the capture must still be ended and
 * the resulting graph destroyed). */
typedef struct pkv_graph* pkv_graph_t;
pkv_status pkv_graph_begin(void* stream);
pkv_status pkv_graph_end(void* stream, pkv_graph_t* graph);
pkv_status pkv_graph_launch(pkv_graph_t graph, void* stream);
pkv_status pkv_graph_destroy(pkv_graph_t graph);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
