// C-ABI of the paged decode-attention library: argument validation, partition choice,
// workspace sizing and dispatch to the kernel launchers.  Validation touches no HIP API,
// so every error return happens before anything is enqueued.  Also the capture and replay
// of decode steps as HIP graphs.
#include <stdint.h>

#include <mutex>
#include <new>

#include "../../include/pkv.h"
#include "pkv_launch.hpp"

// Device-resident scratch for pkv_paged_decode_attn_noalloc: every GPU the library runs on
// holds one copy until the process ends.  Host code never passes `scratch` itself to a
// kernel (in host code the name stands for a host-side shadow, not a device address): the
// per-device address comes from hipGetSymbolAddress, taken once per device with that
// device current.
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

constexpr int kMaxPartitionTokens = 4096;  // 64 tiles of 16 tokens per wave, 4 waves
constexpr int kMaxStreamSeqs = 4096;       // balanced mode: sequences per call
constexpr long long kMaxChunkTiles = 128;  // balanced mode: tiles per wave
constexpr int kRingMaxWavesPerCu = 8;      // the default decode kernel: 4 or 8 waves per CU
// and about 480 tiles per wave, so that a chunk weighted 17/16 (single-token) or 33/32
// (multi-token) by XCD still fits the 512 tiles a wave's tables hold
constexpr long long kRingChunkTiles = 480;

int32_t ring_chunks(int32_t B, int32_t Hkv, int32_t max_ctx, int waves_per_cu);
constexpr int kGridYZMax = 65535;
constexpr long long kTargetWorkgroups = 1024;  // ~4 workgroups per CU on 256 CUs

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

int elem_bytes(int32_t dtype) {
  return dtype == PKV_BF16 ? 2 : (dtype == PKV_FP8_E4M3 ? 1 : 0);
}

// Longest partition (up to 1024 tokens) that still gives every CU several workgroups:
// each workgroup pays a fixed start (table, q, first tile latency) and end (merge) cost.
int32_t auto_partition(int32_t B, int32_t heads, int32_t max_ctx) {
  int32_t ps = 1024;
  while (ps > 64) {
    const long long parts = (max_ctx + ps - 1) / ps;
    if ((long long)B * heads * (parts > 0 ? parts : 1) >= kTargetWorkgroups) break;
    ps /= 2;
  }
  return ps;
}

// Latent decode: one workgroup covers 64 query heads of a partition, and a partition's
// partial output (128 heads x 512 fp32) is large next to its latent rows, so split only
// as far as needed for about two workgroups per CU.
int32_t mla_auto_partition(int32_t B, int32_t Hq, int32_t max_ctx) {
  const long long groups = (long long)B * ((Hq + 63) / 64);
  long long parts = (2 * 256 + groups - 1) / (groups > 0 ? groups : 1);
  if (parts < 1) parts = 1;
  long long ps = (max_ctx + parts - 1) / parts;
  ps = (ps + 63) / 64 * 64;
  return (int32_t)(ps < 64 ? 64 : ps);
}

int32_t num_parts(int32_t max_ctx, int32_t ps) {
  const int32_t p = (max_ctx + ps - 1) / ps;
  return p < 1 ? 1 : p;
}

// Workspace layout, shared by both decode entry points: m [R], l [R], o [R][d_v] (fp32),
// R = B * Hq * P, each section 256-byte aligned.
size_t ws_bytes(int32_t B, int32_t Hq, int32_t d_v, int32_t P) {
  if (P <= 1) return 0;
  const size_t rows = (size_t)B * Hq * P;
  return 2 * round256(rows * sizeof(float)) + round256(rows * d_v * sizeof(float));
}

void ws_split(void* ws, int32_t B, int32_t Hq, int32_t P, float** m, float** l, float** o) {
  const size_t rows = (size_t)B * Hq * P;
  char* base = (char*)ws;
  *m = (float*)base;
  *l = (float*)(base + round256(rows * sizeof(float)));
  *o = (float*)(base + 2 * round256(rows * sizeof(float)));
}

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Whether the current device hands a grid's workgroups to 8 XCDs in turn: the whole MI355X
// as one partition (cached per device; false when the query fails).
bool device_xcd8() {
  static int cached[64] = {0};  // 0 unknown, 1 no, 2 yes
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (!cached[dev]) {
    int n = 0;
    const bool ok = hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess;
    cached[dev] = ok && n == 8 ? 2 : 1;
  }
  return cached[dev] == 2;
}

// Balanced mode: one chunk per resident wave (two 4-wave workgroups per CU for the
// single-token kernel), and enough chunks that
// none holds more than kMaxChunkTiles tiles even if every context were max_context_len;
// never more chunks than that bound on the tiles (rounded up to 8 workgroups), so that a
// small batch is not spread over thousands of empty chunks the merge would walk.
int32_t stream_chunks(int32_t B, int32_t Hkv, int32_t max_ctx, int waves_per_cu = 8,
                      long long max_chunk_tiles = kMaxChunkTiles, int waves_per_group = 4) {
  const long long tmax = (long long)Hkv * B * ((max_ctx + 15) / 16);
  long long c = (long long)waves_per_cu * device_cus();
  if (tmax < c) c = tmax;
  const long long need = (tmax + max_chunk_tiles - 1) / max_chunk_tiles;
  if (need > c) c = need;
  // a multiple of 8 workgroups' worth: each of the 8 XCDs takes whole workgroups of an eighth
  const long long unit = 8LL * waves_per_group;
  c = (c + unit - 1) / unit * unit;
  if (c < unit) c = unit;
  return c > (1LL << 30) ? -1 : (int32_t)c;
}

// The decode kernel's chunks; the workspace query sizes for the largest count (8 waves per
// CU), since it does not know the element type that selects the kernel's shape.
int32_t ring_chunks(int32_t B, int32_t Hkv, int32_t max_ctx, int waves_per_cu) {
  return stream_chunks(B, Hkv, max_ctx, waves_per_cu, kRingChunkTiles, waves_per_cu);
}

// Balanced-mode workspace: m [S][G], l [S][G], o [S][G][d], prefix [B + 1] (int32) and
// per-segment (first chunk, chunks spanned) [Hkv * B][2] (int32), S = chunks + Hkv * B piece
// slots; sections 256-byte aligned.
size_t stream_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t chunks) {
  const size_t rows = ((size_t)chunks + (size_t)Hkv * B) * (size_t)(Hq / Hkv);
  return 2 * round256(rows * sizeof(float)) + round256(rows * d * sizeof(float)) +
         round256(((size_t)B + 1) * sizeof(int32_t)) +
         round256((size_t)Hkv * B * 2 * sizeof(int32_t));
}

// Latent balanced mode: one workgroup per CU, Hq / 32 or Hq / 64 head groups, chunks a
// multiple of 8, enough of them that none holds more than 128 stages of 32 tokens, and no
// more than the bound on the stages (rounded up to 8).
int32_t mla_stream_chunks(int32_t B, int32_t Hq, int32_t max_ctx) {
  const long long hg = Hq / pkv::mla_stream_heads_per_group(Hq);
  const long long smax = (long long)B * ((max_ctx + 31) / 32);
  long long c = (device_cus() + hg - 1) / hg;
  if (smax < c) c = smax;
  const long long need = (smax + 127) / 128;
  if (need > c) c = need;
  c = (c + 7) / 8 * 8;
  if (c < 8) c = 8;
  return c > (1LL << 24) ? -1 : (int32_t)c;
}

bool mla_stream_mode(int32_t B, int32_t Hq, int32_t partition_size) {
  return partition_size == 0 && B <= kMaxStreamSeqs && pkv::mla_stream_heads_per_group(Hq) > 0;
}

bool stream_mode(int32_t B, int32_t partition_size) {
  return partition_size == 0 && B <= kMaxStreamSeqs;
}

pkv_status hip_status(hipError_t e) {
  if (e == hipSuccess) return PKV_OK;
  if (e == hipErrorNotSupported) return PKV_ERR_UNSUPPORTED;
  return PKV_ERR_HIP;
}

// Multi-token workspace: the balanced layout with R = q_len * Hq / Hkv rows per piece slot.
size_t multi_ws_bytes(int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t d,
                      int32_t chunks) {
  const size_t rows = ((size_t)chunks + (size_t)Hkv * B) * (size_t)(Hq / Hkv) * q_len;
  return 2 * round256(rows * sizeof(float)) + round256(rows * d * sizeof(float)) +
         round256(((size_t)B + 1) * sizeof(int32_t)) +
         round256((size_t)Hkv * B * 2 * sizeof(int32_t));
}

// The workspace query does not know the element type: it sizes for the register-tile
// kernel (8 waves per CU, 128 tiles per wave), which never has fewer chunks than the ring
// kernel (4 waves per CU, 480 tiles per wave).
int32_t multi_chunks(int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t d,
                     int32_t max_context_len, bool ring) {
  if (ring)
    return stream_chunks(B, Hkv, max_context_len, pkv::multi_ring_waves_per_cu(), kRingChunkTiles,
                         pkv::multi_ring_waves_per_cu());
  return stream_chunks(B, Hkv, max_context_len,
                       pkv::multi_waves_per_cu(d, (Hq / Hkv) * q_len));
}

// Multi-token workspace sections (m, l, o, tile prefix, segment ranges) into a.
void multi_ws_split(void* ws, int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t d,
                    int32_t chunks, pkv::MultiArgs& a) {
  const size_t rows = ((size_t)chunks + (size_t)Hkv * B) * (size_t)(Hq / Hkv) * q_len;
  char* base = (char*)ws;
  a.ws_m = (float*)base;
  a.ws_l = (float*)(base + round256(rows * sizeof(float)));
  a.ws_o = (float*)(base + 2 * round256(rows * sizeof(float)));
  a.ws_prefix = (int32_t*)(base + 2 * round256(rows * sizeof(float)) +
                           round256(rows * d * sizeof(float)));
  a.ws_seg = (int32_t*)((char*)a.ws_prefix + round256(((size_t)B + 1) * sizeof(int32_t)));
}

// Cascade call: the tail pass's balanced workspace, then the prefix pass's multi-token
// workspace for groups of J = 32 / G sequences (32 query rows per KV head and group: two
// waves per SIMD; 64-row groups read the prefix half as often but take the whole register
// file and measured slower).  With a prefix both passes run in one launch, sized to be
// resident together: kCascadeTailWaves + kCascadePrefixWaves waves per CU (of the splits
// 4+4, 5+3, 6+2, 7+1, 6+1, 7+2, 8+2 and 8+4 on the FP8 shared-prefix batch, 6+2 was the
// fastest: 69 us against 74-101 us).
constexpr int kCascadeTailWaves = 6;
constexpr int kCascadePrefixWaves = 2;
struct CascadePlan {
  bool ok;
  int32_t t_chunks, p_chunks, J, p_B;
  size_t t_bytes, p_bytes;
};
CascadePlan cascade_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t prefix_len,
                         int32_t max_tail_len) {
  CascadePlan c{false, 0, 0, 0, 0, 0, 0};
  const int32_t G = Hq / Hkv;
  if (G < 1 || G > 32) return c;
  c.t_chunks = stream_chunks(B, Hkv, max_tail_len, prefix_len > 0 ? kCascadeTailWaves : 8);
  if (c.t_chunks < 0) return c;
  c.t_bytes = stream_ws_bytes(B, Hq, Hkv, d, c.t_chunks);
  c.J = 32 / G;
  c.p_B = (B + c.J - 1) / c.J;
  if (prefix_len > 0) {
    c.p_chunks = stream_chunks(c.p_B, Hkv, prefix_len, kCascadePrefixWaves);
    if (c.p_chunks < 0) return c;
    c.p_bytes = multi_ws_bytes(c.p_B, c.J, Hq, Hkv, d, c.p_chunks);
  }
  c.ok = true;
  return c;
}

bool multi_shape_ok(int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t d,
                    int32_t max_context_len) {
  return B >= 0 && q_len > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && d > 0 &&
         max_context_len >= 0;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_str(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is non-positive or inconsistent";
    case PKV_ERR_DTYPE: return "unknown element type";
    case PKV_ERR_UNSUPPORTED: return "shape or type combination not supported";
    case PKV_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

pkv_status pkv_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int32_t T, int32_t num_blocks,
                         int32_t Hkv, int32_t d, int32_t block_size, int32_t kv_dtype,
                         void* stream) {
  if (T < 0 || num_blocks <= 0 || Hkv <= 0 || d <= 0 || block_size <= 0) return PKV_ERR_SHAPE;
  const int es = elem_bytes(kv_dtype);
  if (!es) return PKV_ERR_DTYPE;
  if (T == 0) return PKV_OK;
  if (!k_pool || !k_new || !slot_mapping) return PKV_ERR_NULL;
  if ((v_pool == nullptr) != (v_new == nullptr)) return PKV_ERR_NULL;
  if (((long long)d * es) % 16) return PKV_ERR_UNSUPPORTED;
  if (!aligned16(k_pool) || !aligned16(k_new) || (v_pool && (!aligned16(v_pool) || !aligned16(v_new))) ||
      ((uintptr_t)slot_mapping & 7u))
    return PKV_ERR_ALIGN;
  pkv::AppendArgs a{k_pool, v_pool, k_new, v_new, slot_mapping, T, num_blocks, Hkv, block_size,
                    d * es};
  return hip_status(pkv::launch_kv_append(a, (hipStream_t)stream));
}

int32_t pkv_decode_partition_size(int32_t B, int32_t Hkv, int32_t max_context_len,
                                  int32_t partition_size) {
  if (B < 0 || Hkv <= 0 || max_context_len < 0) return PKV_ERR_SHAPE;
  if (partition_size < 0 || partition_size % 16 || partition_size > kMaxPartitionTokens)
    return PKV_ERR_SHAPE;
  // balanced mode packs (segment << 5) into 32 bits: Hkv * B must stay below 2^26
  if (stream_mode(B, partition_size) && (long long)Hkv * B < (1LL << 26)) return 0;
  return partition_size > 0 ? partition_size : auto_partition(B, Hkv, max_context_len);
}

size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d_v,
                                  int32_t max_context_len, int32_t partition_size) {
  const int32_t ps = pkv_decode_partition_size(B, Hkv, max_context_len, partition_size);
  if (ps < 0 || Hq <= 0 || d_v <= 0 || Hq % Hkv) return 0;
  if (ps == 0) {
    // the most chunks any balanced kernel of the call can take: the VALU ring at 8 waves per
    // CU, or for d = 128 (FP8 K/V: the register-tile MFMA kernel) up to 128 tiles per chunk
    int32_t chunks = ring_chunks(B, Hkv, max_context_len, kRingMaxWavesPerCu);
    if (d_v == 128 && chunks >= 0) {
      const int32_t tile_chunks = multi_chunks(B, 1, Hq, Hkv, d_v, max_context_len, false);
      chunks = tile_chunks < 0 ? -1 : (tile_chunks > chunks ? tile_chunks : chunks);
    }
    return chunks < 0 ? 0 : stream_ws_bytes(B, Hq, Hkv, d_v, chunks);
  }
  return ws_bytes(B, Hq, d_v, num_parts(max_context_len, ps));
}

pkv_status pkv_paged_decode_attn(float* out, const void* q, const void* k_pool,
                                 const void* v_pool, const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, const int32_t* context_lens,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 float scale, int32_t kv_dtype, int32_t partition_size,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0)
    return PKV_ERR_SHAPE;
  if (Hq % Hkv) return PKV_ERR_SHAPE;
  if (!elem_bytes(kv_dtype)) return PKV_ERR_DTYPE;
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens) return PKV_ERR_NULL;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  const int32_t G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PKV_ERR_UNSUPPORTED;
  if (!((d == 128) || (d == 64 && !fp8))) return PKV_ERR_UNSUPPORTED;
  if (block_size % 16) return PKV_ERR_UNSUPPORTED;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(block_table) || !aligned4(context_lens) ||
      (fp8 && (!aligned4(k_scale) || !aligned4(v_scale))))
    return PKV_ERR_ALIGN;
  if (B > kGridYZMax) return PKV_ERR_SHAPE;
  // Grid and workspace follow max_context_len exactly as pkv_decode_workspace_bytes does;
  // each sequence's own length is clamped to its table inside the kernels.
  const int32_t ctx = max_context_len;
  const int32_t ps = pkv_decode_partition_size(B, Hkv, ctx, partition_size);
  if (ps < 0) return PKV_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (ps == 0) {  // balanced mode
    // d = 128: the multi-token kernels with q_len = 1 (each sequence's G query rows in one
    // 16-row MFMA tile): for bf16 K/V the LDS ring, for FP8 the register-tile kernel; d = 64:
    // the VALU ring
    const bool mfma = d == 128;
    const int32_t chunks = mfma ? multi_chunks(B, 1, Hq, Hkv, d, ctx, !fp8)
                                : ring_chunks(B, Hkv, ctx, pkv::ring_waves_per_cu(d, G, fp8));
    if (chunks < 0) return PKV_ERR_SHAPE;
    const size_t need = stream_ws_bytes(B, Hq, Hkv, d, chunks);
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    const size_t rows = ((size_t)chunks + (size_t)Hkv * B) * (size_t)(Hq / Hkv);
    char* base = (char*)workspace;
    float* ws_m = (float*)base;
    float* ws_l = (float*)(base + round256(rows * sizeof(float)));
    float* ws_o = (float*)(base + 2 * round256(rows * sizeof(float)));
    int32_t* ws_p = (int32_t*)(base + 2 * round256(rows * sizeof(float)) +
                               round256(rows * d * sizeof(float)));
    int32_t* ws_s = (int32_t*)((char*)ws_p + round256(((size_t)B + 1) * sizeof(int32_t)));
    pkv::DecodeArgs a{out, (const uint16_t*)q, (const uint8_t*)k_pool, (const uint8_t*)v_pool,
                      k_scale, v_scale, block_table, context_lens, ws_m, ws_l, ws_o,
                      B, Hq, Hkv, d, block_size, num_blocks, max_blocks_per_seq, ctx,
                      0, 0, scale, fp8 ? 1 : 0, chunks, ws_p, ws_s, device_xcd8() ? 1 : 0};
    if (!mfma) return hip_status(pkv::launch_gqa_stream(a, s));
    pkv::MultiArgs m{};
    m.out = nullptr;
    m.q = (const uint16_t*)q;
    m.k_pool = (const uint8_t*)k_pool;
    m.v_pool = (const uint8_t*)v_pool;
    m.k_scale = k_scale;
    m.v_scale = v_scale;
    m.block_table = block_table;
    m.context_lens = context_lens;
    m.ws_m = ws_m, m.ws_l = ws_l, m.ws_o = ws_o, m.ws_prefix = ws_p, m.ws_seg = ws_s;
    m.B = B, m.q_len = 1, m.Hq = Hq, m.Hkv = Hkv, m.d = d, m.block_size = block_size;
    m.num_blocks = num_blocks, m.max_blocks = max_blocks_per_seq, m.max_len = ctx;
    m.table_stride = max_blocks_per_seq, m.fixed_len = -1, m.q_rows = B;
    m.causal = 1, m.fp8 = fp8 ? 1 : 0, m.scale = scale, m.chunks = chunks, m.xcd8 = a.xcd8;
    const pkv_status st = hip_status(pkv::launch_gqa_multi_pieces(m, s));
    if (st != PKV_OK) return st;
    return hip_status(pkv::launch_stream_merge(a, s));
  }
  const int32_t P = num_parts(ctx, ps);
  if (P > kGridYZMax) return PKV_ERR_SHAPE;
  float *ws_m = nullptr, *ws_l = nullptr, *ws_o = nullptr;
  if (P > 1) {
    if (!workspace || workspace_bytes < ws_bytes(B, Hq, d, P)) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    ws_split(workspace, B, Hq, P, &ws_m, &ws_l, &ws_o);
  }
  pkv::DecodeArgs a{out, (const uint16_t*)q, (const uint8_t*)k_pool, (const uint8_t*)v_pool,
                    k_scale, v_scale, block_table, context_lens, ws_m, ws_l, ws_o,
                    B, Hq, Hkv, d, block_size, num_blocks, max_blocks_per_seq, ctx,
                    ps, P, scale, fp8 ? 1 : 0, 0, nullptr};
  pkv_status st = hip_status(pkv::launch_gqa_decode(a, s));
  if (st != PKV_OK || P == 1) return st;
  return hip_status(pkv::launch_partition_merge(ws_m, ws_l, ws_o, context_lens, out, B, Hq, d,
                                                ps, P, ctx,
                                                min(max_blocks_per_seq * block_size, ctx), s));
}

pkv_status pkv_paged_decode_attn_noalloc(float* out, const void* q, const void* k_pool,
                                         const void* v_pool, const float* k_scale,
                                         const float* v_scale, const int32_t* block_table,
                                         const int32_t* context_lens, int32_t B, int32_t Hq,
                                         int32_t Hkv, int32_t d, int32_t block_size,
                                         int32_t num_blocks, int32_t max_blocks_per_seq,
                                         int32_t max_context_len, float scale, int32_t kv_dtype,
                                         int32_t partition_size, void* stream) {
  // the same argument checks and the same kernels as pkv_paged_decode_attn, with the
  // library's device scratch as the workspace (no allocation anywhere on this path)
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_context_len < 0 || Hq % Hkv)
    return PKV_ERR_SHAPE;
  const size_t need = pkv_decode_workspace_bytes(B, Hq, Hkv, d, max_context_len, partition_size);
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && B > 0) {
    ws = scratch_on_current_device();
    if (!ws) return PKV_ERR_HIP;
  }
  return pkv_paged_decode_attn(out, q, k_pool, v_pool, k_scale, v_scale, block_table,
                               context_lens, B, Hq, Hkv, d, block_size, num_blocks,
                               max_blocks_per_seq, max_context_len, scale, kv_dtype,
                               partition_size, ws, ws ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0,
                               stream);
}

size_t pkv_mla_workspace_bytes(int32_t B, int32_t Hq, int32_t d_v, int32_t max_context_len,
                               int32_t partition_size) {
  if (B < 0 || Hq <= 0 || d_v <= 0 || max_context_len < 0 || partition_size < 0) return 0;
  if (mla_stream_mode(B, Hq, partition_size)) {
    const int32_t chunks = mla_stream_chunks(B, Hq, max_context_len);
    return chunks < 0 ? 0 : stream_ws_bytes(B, Hq, 1, d_v, chunks);
  }
  const int32_t ps = partition_size > 0 ? partition_size : mla_auto_partition(B, Hq, max_context_len);
  return ws_bytes(B, Hq, d_v, num_parts(max_context_len, ps));
}

pkv_status pkv_paged_decode_attn_mla(float* out, const void* q, const void* kv_pool,
                                     const int32_t* block_table, const int32_t* context_lens,
                                     int32_t B, int32_t Hq, int32_t d_qk, int32_t d_v,
                                     int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (B < 0 || Hq <= 0 || d_qk <= 0 || d_v <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0 || partition_size < 0)
    return PKV_ERR_SHAPE;
  if (d_v > d_qk) return PKV_ERR_SHAPE;
  if (B == 0) return PKV_OK;
  if (!out || !q || !kv_pool || !block_table || !context_lens) return PKV_ERR_NULL;
  if (d_qk != 576 || d_v != 512 || block_size != 64 || Hq % 16 || Hq > 128)
    return PKV_ERR_UNSUPPORTED;
  if (partition_size % block_size) return PKV_ERR_SHAPE;
  if (!aligned16(out) || !aligned16(q) || !aligned16(kv_pool) || !aligned4(block_table) ||
      !aligned4(context_lens))
    return PKV_ERR_ALIGN;
  if (B > kGridYZMax) return PKV_ERR_SHAPE;
  const int32_t ctx = max_context_len;
  hipStream_t s = (hipStream_t)stream;
  if (mla_stream_mode(B, Hq, partition_size)) {  // balanced mode
    const int32_t chunks = mla_stream_chunks(B, Hq, ctx);
    if (chunks < 0) return PKV_ERR_SHAPE;
    if (!workspace || workspace_bytes < stream_ws_bytes(B, Hq, 1, d_v, chunks))
      return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    const size_t rows = ((size_t)chunks + (size_t)B) * (size_t)Hq;
    char* base = (char*)workspace;
    float* ws_m = (float*)base;
    float* ws_l = (float*)(base + round256(rows * sizeof(float)));
    float* ws_o = (float*)(base + 2 * round256(rows * sizeof(float)));
    int32_t* ws_p = (int32_t*)(base + 2 * round256(rows * sizeof(float)) +
                               round256(rows * d_v * sizeof(float)));
    int32_t* ws_s = (int32_t*)((char*)ws_p + round256(((size_t)B + 1) * sizeof(int32_t)));
    pkv::MlaArgs a{out, (const uint16_t*)q, (const uint16_t*)kv_pool, block_table, context_lens,
                   ws_m, ws_l, ws_o, B, Hq, d_qk, d_v, block_size, num_blocks,
                   max_blocks_per_seq, ctx, 0, 0, scale, chunks, ws_p, ws_s};
    return hip_status(pkv::launch_mla_stream(a, s));
  }
  const int32_t ps = partition_size > 0 ? partition_size : mla_auto_partition(B, Hq, ctx);
  const int32_t P = num_parts(ctx, ps);
  if (P > kGridYZMax) return PKV_ERR_SHAPE;
  float *ws_m = nullptr, *ws_l = nullptr, *ws_o = nullptr;
  if (P > 1) {
    if (!workspace || workspace_bytes < ws_bytes(B, Hq, d_v, P)) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    ws_split(workspace, B, Hq, P, &ws_m, &ws_l, &ws_o);
  }
  pkv::MlaArgs a{out, (const uint16_t*)q, (const uint16_t*)kv_pool, block_table, context_lens,
                 ws_m, ws_l, ws_o, B, Hq, d_qk, d_v, block_size, num_blocks, max_blocks_per_seq,
                 ctx, ps, P, scale, 0, nullptr};
  pkv_status st = hip_status(pkv::launch_mla_decode(a, s));
  if (st != PKV_OK || P == 1) return st;
  return hip_status(pkv::launch_partition_merge(ws_m, ws_l, ws_o, context_lens, out, B, Hq, d_v,
                                                ps, P, ctx,
                                                min(max_blocks_per_seq * block_size, ctx), s));
}

size_t pkv_multi_workspace_bytes(int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t d,
                                 int32_t max_context_len) {
  if (!multi_shape_ok(B, q_len, Hq, Hkv, d, max_context_len)) return 0;
  const int32_t G = Hq / Hkv;
  if ((long long)G * q_len > 64 || (G != 1 && G != 2 && G != 4 && G != 8) ||
      (long long)Hkv * B >= (1LL << 26))
    return 0;
  const int32_t chunks = multi_chunks(B, q_len, Hq, Hkv, d, max_context_len, false);
  return chunks < 0 ? 0 : multi_ws_bytes(B, q_len, Hq, Hkv, d, chunks);
}

pkv_status pkv_paged_decode_attn_multi(float* out, const void* q, const void* k_pool,
                                       const void* v_pool, const float* k_scale,
                                       const float* v_scale, const int32_t* block_table,
                                       const int32_t* context_lens, int32_t B, int32_t q_len,
                                       int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_context_len, float scale, int32_t kv_dtype,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!multi_shape_ok(B, q_len, Hq, Hkv, d, max_context_len) || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_SHAPE;
  if (!elem_bytes(kv_dtype)) return PKV_ERR_DTYPE;
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens) return PKV_ERR_NULL;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  const int32_t G = Hq / Hkv;
  if ((d != 128 && d != 64) || block_size % 16 || (long long)G * q_len > 64 ||
      (G != 1 && G != 2 && G != 4 && G != 8))
    return PKV_ERR_UNSUPPORTED;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(block_table) || !aligned4(context_lens) ||
      (fp8 && (!aligned4(k_scale) || !aligned4(v_scale))))
    return PKV_ERR_ALIGN;
  if (B > kMaxStreamSeqs || (long long)Hkv * B >= (1LL << 26)) return PKV_ERR_SHAPE;
  const int32_t chunks = multi_chunks(B, q_len, Hq, Hkv, d, max_context_len,
                                      pkv::multi_uses_ring(d, G * q_len, fp8));
  if (chunks < 0) return PKV_ERR_SHAPE;
  if (!workspace || workspace_bytes < multi_ws_bytes(B, q_len, Hq, Hkv, d, chunks))
    return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  pkv::MultiArgs a{};
  multi_ws_split(workspace, B, q_len, Hq, Hkv, d, chunks, a);
  a.out = out;
  a.q = (const uint16_t*)q;
  a.k_pool = (const uint8_t*)k_pool;
  a.v_pool = (const uint8_t*)v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.B = B, a.q_len = q_len, a.Hq = Hq, a.Hkv = Hkv, a.d = d, a.block_size = block_size;
  a.num_blocks = num_blocks, a.max_blocks = max_blocks_per_seq;
  a.table_stride = max_blocks_per_seq, a.fixed_len = -1, a.q_rows = B * q_len;
  a.max_len = max_context_len;
  a.causal = 1, a.fp8 = fp8 ? 1 : 0, a.scale = scale, a.chunks = chunks;
  a.xcd8 = device_xcd8() ? 1 : 0;
  return hip_status(pkv::launch_gqa_multi(a, (hipStream_t)stream));
}

size_t pkv_cascade_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                   int32_t prefix_len, int32_t max_tail_len) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || prefix_len < 0 || max_tail_len < 0)
    return 0;
  const CascadePlan c = cascade_plan(B, Hq, Hkv, d, prefix_len, max_tail_len);
  return c.ok ? c.t_bytes + c.p_bytes : 0;
}

pkv_status pkv_paged_decode_attn_cascade(float* out, const void* q, const void* k_pool,
                                         const void* v_pool, const float* k_scale,
                                         const float* v_scale, const int32_t* prefix_blocks,
                                         int32_t prefix_len, const int32_t* tail_table,
                                         const int32_t* tail_lens, int32_t B, int32_t Hq,
                                         int32_t Hkv, int32_t d, int32_t block_size,
                                         int32_t num_blocks, int32_t max_tail_blocks,
                                         int32_t max_tail_len, float scale, int32_t kv_dtype,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_tail_blocks <= 0 || max_tail_len < 0 || prefix_len < 0)
    return PKV_ERR_SHAPE;
  if (Hq % Hkv || prefix_len % block_size) return PKV_ERR_SHAPE;
  if (!elem_bytes(kv_dtype)) return PKV_ERR_DTYPE;
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !tail_table || !tail_lens ||
      (prefix_len > 0 && !prefix_blocks))
    return PKV_ERR_NULL;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  const int32_t G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PKV_ERR_UNSUPPORTED;
  if (!((d == 128) || (d == 64 && !fp8)) || block_size % 16) return PKV_ERR_UNSUPPORTED;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(tail_table) || !aligned4(tail_lens) || (prefix_len > 0 && !aligned4(prefix_blocks)) ||
      (fp8 && (!aligned4(k_scale) || !aligned4(v_scale))))
    return PKV_ERR_ALIGN;
  if (B > kMaxStreamSeqs || (long long)Hkv * B >= (1LL << 26)) return PKV_ERR_SHAPE;
  const CascadePlan c = cascade_plan(B, Hq, Hkv, d, prefix_len, max_tail_len);
  if (!c.ok) return PKV_ERR_SHAPE;
  if (!workspace || workspace_bytes < c.t_bytes + c.p_bytes) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;

  // tails: the single-token balanced kernel over each sequence's own blocks, pieces only
  const size_t rows = ((size_t)c.t_chunks + (size_t)Hkv * B) * (size_t)G;
  char* base = (char*)workspace;
  float* t_m = (float*)base;
  float* t_l = (float*)(base + round256(rows * sizeof(float)));
  float* t_o = (float*)(base + 2 * round256(rows * sizeof(float)));
  int32_t* t_p = (int32_t*)(base + 2 * round256(rows * sizeof(float)) + round256(rows * d * sizeof(float)));
  int32_t* t_s = (int32_t*)((char*)t_p + round256(((size_t)B + 1) * sizeof(int32_t)));
  pkv::DecodeArgs ta{out, (const uint16_t*)q, (const uint8_t*)k_pool, (const uint8_t*)v_pool,
                     k_scale, v_scale, tail_table, tail_lens, t_m, t_l, t_o,
                     B, Hq, Hkv, d, block_size, num_blocks, max_tail_blocks, max_tail_len,
                     0, 0, scale, fp8 ? 1 : 0, c.t_chunks, t_p, t_s, device_xcd8() ? 1 : 0};
  // prefix: groups of J sequences as the q_len rows of the multi-token kernel, all reading
  // the prefix blocks, no causal mask; launched together with the tails
  pkv::MultiArgs pa{};
  pkv_status st = PKV_OK;
  if (prefix_len == 0) {
    st = hip_status(pkv::launch_gqa_stream_pieces(ta, s));
  } else {
    multi_ws_split(base + c.t_bytes, c.p_B, c.J, Hq, Hkv, d, c.p_chunks, pa);
    pa.out = nullptr;
    pa.q = (const uint16_t*)q;
    pa.k_pool = (const uint8_t*)k_pool;
    pa.v_pool = (const uint8_t*)v_pool;
    pa.k_scale = k_scale;
    pa.v_scale = v_scale;
    pa.block_table = prefix_blocks;
    pa.context_lens = nullptr;
    pa.B = c.p_B, pa.q_len = c.J, pa.Hq = Hq, pa.Hkv = Hkv, pa.d = d;
    pa.block_size = block_size, pa.num_blocks = num_blocks;
    pa.max_blocks = prefix_len / block_size, pa.table_stride = 0, pa.fixed_len = prefix_len;
    pa.max_len = prefix_len;
    pa.q_rows = B, pa.causal = 0, pa.fp8 = fp8 ? 1 : 0, pa.scale = scale, pa.chunks = c.p_chunks;
    pa.xcd8 = device_xcd8() ? 1 : 0;
    st = hip_status(pkv::launch_cascade(ta, pa, s));
  }
  if (st != PKV_OK) return st;

  pkv::CascadeMergeArgs ma{out, B, Hq, Hkv, d, t_m, t_l, t_o, t_p, t_s, c.t_chunks,
                           prefix_len > 0 ? pa.ws_m : nullptr, pa.ws_l, pa.ws_o, pa.ws_prefix,
                           pa.ws_seg, c.p_chunks, c.p_B, c.J};
  return hip_status(pkv::launch_cascade_merge(ma, s));
}

pkv_status pkv_validate(int32_t* counts, const int32_t* block_table,
                        const int32_t* context_lens, int32_t B, int32_t max_blocks_per_seq,
                        int32_t num_blocks, int32_t block_size, int32_t max_context_len,
                        const int64_t* slot_mapping, int32_t T, const void* v_pool, int32_t Hkv,
                        int32_t d, int32_t d_v, void* stream) {
  if (B < 0 || T < 0 || num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq < 0)
    return PKV_ERR_SHAPE;
  if (v_pool && (Hkv <= 0 || d <= 0 || d_v <= 0 || d_v > d)) return PKV_ERR_SHAPE;
  if (!counts || (B > 0 && max_blocks_per_seq > 0 && (!block_table || !context_lens)) ||
      (T > 0 && !slot_mapping))
    return PKV_ERR_NULL;
  if (!aligned4(counts) || (B > 0 && (!aligned4(block_table) || !aligned4(context_lens))) ||
      ((uintptr_t)slot_mapping & 7u) || ((uintptr_t)v_pool & 1u))
    return PKV_ERR_ALIGN;
  pkv::ValidateArgs a{counts, block_table, context_lens, B, max_blocks_per_seq, num_blocks,
                      block_size, max_context_len, slot_mapping, T, (const uint16_t*)v_pool,
                      Hkv, d, d_v};
  return hip_status(pkv::launch_validate(a, (hipStream_t)stream));
}

pkv_status pkv_kv_append_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                             const float* k_scale, const float* v_scale,
                             const int64_t* slot_mapping, int32_t T, int32_t num_blocks,
                             int32_t Hkv, int32_t d, int32_t block_size, void* stream) {
  if (T < 0 || num_blocks <= 0 || Hkv <= 0 || d <= 0 || block_size <= 0) return PKV_ERR_SHAPE;
  if (T == 0) return PKV_OK;
  if (!k_pool || !k_new || !k_scale || !slot_mapping) return PKV_ERR_NULL;
  if ((v_pool == nullptr) != (v_new == nullptr) || (v_pool && !v_scale)) return PKV_ERR_NULL;
  if (d % 16) return PKV_ERR_UNSUPPORTED;
  if (!aligned16(k_pool) || !aligned16(k_new) || !aligned4(k_scale) ||
      (v_pool && (!aligned16(v_pool) || !aligned16(v_new) || !aligned4(v_scale))) ||
      ((uintptr_t)slot_mapping % 8))
    return PKV_ERR_ALIGN;
  pkv::AppendFp8Args a{(uint8_t*)k_pool, (uint8_t*)v_pool, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, k_scale, v_scale, slot_mapping, T,
                       num_blocks, Hkv, block_size, d};
  return hip_status(pkv::launch_kv_append_fp8(a, (hipStream_t)stream));
}

pkv_status pkv_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_blocks,
                              const int32_t* dst_blocks, int32_t n, int32_t num_blocks,
                              int32_t Hkv, int32_t d, int32_t block_size, int32_t kv_dtype,
                              void* stream) {
  if (n < 0 || num_blocks <= 0 || Hkv <= 0 || d <= 0 || block_size <= 0) return PKV_ERR_SHAPE;
  const int es = elem_bytes(kv_dtype);
  if (!es) return PKV_ERR_DTYPE;
  if (n == 0) return PKV_OK;
  if (!k_pool || !src_blocks || !dst_blocks) return PKV_ERR_NULL;
  if (((long long)d * es) % 16) return PKV_ERR_UNSUPPORTED;
  if (!aligned16(k_pool) || (v_pool && !aligned16(v_pool)) || !aligned4(src_blocks) ||
      !aligned4(dst_blocks))
    return PKV_ERR_ALIGN;
  pkv::CopyBlocksArgs a{(uint8_t*)k_pool, (uint8_t*)v_pool, src_blocks, dst_blocks, n,
                        num_blocks, (int64_t)Hkv * block_size * d * es};
  return hip_status(pkv::launch_kv_copy_blocks(a, (hipStream_t)stream));
}

int32_t pkv_block_hashes(const int32_t* tokens, int32_t n_tokens, int32_t block_size,
                         uint64_t parent, uint64_t* hashes) {
  if (n_tokens < 0 || block_size <= 0) return PKV_ERR_SHAPE;
  const int32_t nb = n_tokens / block_size;
  if (nb == 0) return 0;
  if (!tokens || !hashes) return PKV_ERR_NULL;
  uint64_t h = parent;
  for (int32_t i = 0; i < nb; ++i) {
    uint64_t x = 0xCBF29CE484222325ull;  // FNV-1a 64 offset basis
    auto mix = [&x](uint8_t byte) { x = (x ^ byte) * 0x100000001B3ull; };
    for (int k = 0; k < 8; ++k) mix((uint8_t)(h >> (8 * k)));
    for (int32_t t = 0; t < block_size; ++t) {
      const uint32_t v = (uint32_t)tokens[(size_t)i * block_size + t];
      for (int k = 0; k < 4; ++k) mix((uint8_t)(v >> (8 * k)));
    }
    h = x;
    hashes[i] = h;
  }
  return nb;
}

struct pkv_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

pkv_status pkv_graph_begin(void* stream) {
  if (!stream) return PKV_ERR_NULL;
  return hip_status(hipStreamBeginCapture((hipStream_t)stream, hipStreamCaptureModeThreadLocal));
}

pkv_status pkv_graph_end(void* stream, pkv_graph_t* graph) {
  if (!stream || !graph) return PKV_ERR_NULL;
  *graph = nullptr;
  hipGraph_t g = nullptr;
  if (hipStreamEndCapture((hipStream_t)stream, &g) != hipSuccess || !g) return PKV_ERR_HIP;
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return PKV_ERR_HIP;
  }
  pkv_graph* h = new (std::nothrow) pkv_graph{g, exec};
  if (!h) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(g);
    return PKV_ERR_HIP;
  }
  *graph = h;
  return PKV_OK;
}

pkv_status pkv_graph_launch(pkv_graph_t graph, void* stream) {
  if (!graph) return PKV_ERR_NULL;
  return hip_status(hipGraphLaunch(graph->exec, (hipStream_t)stream));
}

pkv_status pkv_graph_destroy(pkv_graph_t graph) {
  if (!graph) return PKV_OK;
  const hipError_t e1 = hipGraphExecDestroy(graph->exec);
  const hipError_t e2 = hipGraphDestroy(graph->graph);
  delete graph;
  return (e1 == hipSuccess && e2 == hipSuccess) ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
