"""fp64 oracle for decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Sources (cited by page title and section):

* [Serving] "深入LLM推理：从KV Cache到PD分离的Serving全景解析" (kongchang.com)
  - section "KV Cache：Transformer的循环状态": attention is softmax(Q K^T / sqrt(d)) V;
    under GQA several query heads share one K/V head, MQA is the limit with a
    single K/V head, MLA caches a low-rank latent (512 latent + 64 RoPE dims).
    History K/V never changes once written (causal mask), which is what makes
    the cache, and an append-only write, legal.
  - section "PagedAttention与Cache管理": the cache lives in fixed-size
    physical blocks (16 or 32 tokens); a per-sequence block table maps logical
    blocks to physical ones; physical blocks may be shared across requests.
* [GPU-KV] "GPU推理深度拆解：KV Cache视角" (cutenote.app)
  - section "KV Cache 大小与分配演进": per-token KV size of a 70B GQA model,
    block table logical -> physical.
  - sections "长上下文优化" and "算子优化要点": online softmax keeps a split
    computation (ring attention, FlashAttention) mathematically equal to the
    single pass.
* [PD-KV] "PD 分离下的 KV Cache" (zer0e-github-io, ai-infra-7)
  - section "KV Cache 到底有多大？", Eq. KV Size = 2 * L * H_kv * d * S * b and
    its worked example (327680 B per token for 80 layers, 8 KV heads, d=128,
    2-byte elements).
  - section "优化三：KV 传输优化": KV carried as FP8 (half the FP16 bytes) and
    possibly computed on directly in low precision.

Readings taken where the pages are silent:

* query head h uses KV head h // G with G = Hq / Hkv (contiguous grouping);
* a block's physical layout is [num_blocks][Hkv][block_size][d] (head-major
  inside a block); an MLA pool is [num_blocks][block_size][d_qk], one latent
  "head", with V = the first d_v dims of the same latent row;
* FP8 means OCP E4M3 ("e4m3fn": bias 7, no infinities, S.1111.111 is NaN),
  one fp32 scale per KV head, separately for K and V: value = e4m3(byte)*scale;
* a sequence of length 0 has output 0;
* slot_mapping entries < 0 are skipped by the append.

Inputs are the stored bits the device path also reads, decoded exactly to
float64, so that any disagreement is kernel arithmetic alone.
"""

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


# --------------------------------------------------------------------------
# Exact decoding of stored element formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """bfloat16 is the top 16 bits of an IEEE binary32: widen exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):                  # NaN codes stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def fp8_e4m3fn_table():
    """Value of each of the 256 codes of OCP FP8 E4M3 (e4m3fn).

    Built from the format definition: sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^(1-7); there
    are no infinities and only S.1111.111 is NaN (largest finite = 448).
    The pages only say "FP8" ([PD-KV], section "优化三：KV 传输优化"); this
    variant is the reading taken.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            table[code] = np.nan
        elif e == 0:
            table[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            table[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return table


def decode_kv_bits(bits, kv_dtype, scale=None, head_axis=1):
    """Decode a pool (or a slice of one) of stored bits to float64 values.

    kv_dtype "bf16": bits is uint16. kv_dtype "fp8": bits is uint8 and
    ``scale`` holds one fp32 scale per KV head, applied along ``head_axis``.
    """
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if kv_dtype == "fp8":
        vals = fp8_e4m3fn_table()[np.asarray(bits, dtype=np.uint8)]
        shape = [1] * vals.ndim
        shape[head_axis] = -1
        return vals * np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(shape)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


# --------------------------------------------------------------------------
# Paging: block table -> contiguous history
# --------------------------------------------------------------------------

def gather_sequence(pool, block_ids, length, block_size):
    """Logical history of one sequence, gathered out of the block pool.

    [Serving] "PagedAttention与Cache管理": logical block i of the sequence is
    physical block block_ids[i]; token t sits at offset t % block_size of
    logical block t // block_size.  Only the first ceil(length / block_size)
    table entries are read.

    pool: [num_blocks, H, block_size, d] -> returns [H, length, d].
    """
    if length == 0:
        return pool[:0].transpose(1, 0, 2, 3).reshape(pool.shape[1], 0, pool.shape[3])
    n = -(-length // block_size)
    ids = np.asarray(block_ids[:n], dtype=np.int64)
    blocks = pool[ids]                                   # [n, H, bs, d]
    hist = blocks.transpose(1, 0, 2, 3).reshape(pool.shape[1], n * block_size, pool.shape[3])
    return hist[:, :length]


# --------------------------------------------------------------------------
# The attention itself
# --------------------------------------------------------------------------

def paged_decode_attention(q, k_pool, v_pool, block_table, context_lens, scale):
    """One decode step: every query head attends to its sequence's whole history.

    [Serving] "KV Cache：Transformer的循环状态": out = softmax(q K^T * scale) V,
    query head h reading KV head h // G (GQA; G = Hq / Hkv; MQA when Hkv = 1).
    The history is first gathered out of the pool (see ``gather_sequence``),
    then plain softmax attention runs on the contiguous arrays.

    q [B, Hq, d], k_pool [nb, Hkv, bs, d], v_pool [nb, Hkv, bs, d_v] (float64)
    block_table [B, max_blocks] int, context_lens [B] int -> out [B, Hq, d_v].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    _, Hkv, bs, _ = k_pool.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    out = np.zeros((B, Hq, v_pool.shape[3]), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = gather_sequence(k_pool, block_table[b], L, bs)     # [Hkv, L, d]
        V = gather_sequence(v_pool, block_table[b], L, bs)     # [Hkv, L, d_v]
        for h in range(Hq):
            g = h // G
            s = scale * (K[g] @ q[b, h])                        # [L]
            w = np.exp(s - s.max())
            out[b, h] = (w @ V[g]) / w.sum()
    return out


def mla_decode_attention(q, kv_pool, block_table, context_lens, scale, d_v):
    """Latent (MLA) decode: all query heads attend to one shared latent cache.

    [Serving] "KV Cache：Transformer的循环状态" and [GPU-KV] "KV Cache 大小与分配演进":
    the cache holds one compressed latent row per token (512 latent + 64 RoPE
    dims).  Reading taken: the score uses the whole latent row as the key and
    the output uses its first d_v dims as the value; this is MQA (one KV head)
    over the latent.

    q [B, Hq, d_qk], kv_pool [nb, bs, d_qk] -> out [B, Hq, d_v].
    """
    kv = np.asarray(kv_pool, dtype=np.float64)[:, None, :, :]    # [nb, 1, bs, d_qk]
    return paged_decode_attention(q, kv, kv[..., :d_v], block_table, context_lens, scale)


def multi_token_decode_attention(q, k_pool, v_pool, block_table, context_lens, scale):
    """Decode step with q_len query tokens per sequence (speculative verify).

    [Serving] "投机解码：打破每步一token的假设": the large model checks the K drafted tokens
    in one pass.  The new tokens' K/V are already in the cache and counted by
    context_lens; causally, query token j of sequence b sees its first
    context_lens[b] - q_len + 1 + j tokens (none: output 0).  q [B, q_len, Hq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    B, q_len = q.shape[:2]
    lens = np.asarray(context_lens, dtype=np.int64)
    out = np.zeros(q.shape[:3] + (np.asarray(v_pool).shape[-1],), dtype=np.float64)
    for j in range(q_len):
        lens_j = np.maximum(lens - (q_len - 1 - j), 0)
        out[:, j] = paged_decode_attention(q[:, j], k_pool, v_pool, block_table, lens_j, scale)
    return out


# --------------------------------------------------------------------------
# Append (the write half of a decode step)
# --------------------------------------------------------------------------

def kv_append(pool, new, slot_mapping, block_size):
    """Write each new token's rows into its slot; returns a new pool.

    [Serving] "PagedAttention与Cache管理" (block/offset addressing) and
    "KV Cache：Transformer的循环状态" (the past is never rewritten): token i
    goes to physical block slot // block_size, offset slot % block_size, every
    KV head at once.  Slots < 0 are skipped.  Works on raw bits of any dtype.

    pool [nb, H, bs, d], new [T, H, d], slot_mapping [T] int.
    """
    out = np.array(pool, copy=True)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        out[slot // block_size, :, slot % block_size, :] = new[i]
    return out


# --------------------------------------------------------------------------
# Split-context partials and their merge (online-softmax combine)
# --------------------------------------------------------------------------

def partition_partials(q_vec, K, V, scale, part):
    """Per-partition softmax statistics of one query row over one history.

    Splits positions [0, L) into consecutive partitions of ``part`` tokens and
    returns, per partition p, (m_p, l_p, o_p) with m_p = max score,
    l_p = sum exp(s - m_p), o_p = sum exp(s - m_p) v (unnormalised).  The
    online-softmax combine of [GPU-KV] "长上下文优化" / "算子优化要点" then
    recovers the single-pass result exactly (see ``merge_partials``).
    """
    L = K.shape[0]
    ms, ls, os_ = [], [], []
    for start in range(0, L, part):
        s = scale * (K[start:start + part] @ q_vec)
        m = s.max()
        w = np.exp(s - m)
        ms.append(m)
        ls.append(w.sum())
        os_.append(w @ V[start:start + part])
    return np.array(ms), np.array(ls), np.array(os_)


def merge_partials(m, l, o):
    """Combine partition partials: rescale each to the global max and normalise.

    out = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p with M = max_p m_p;
    partitions with l_p = 0 (empty) contribute nothing.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    live = l > 0
    if not live.any():
        return np.zeros(o.shape[-1])
    M = m[live].max()
    w = np.where(live, np.exp(np.where(live, m, M) - M), 0.0)
    return (w @ o) / (w @ l)


# --------------------------------------------------------------------------
# Closed form for the cache size
# --------------------------------------------------------------------------

def kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_elem, tensors=2):
    """Eq. KV Size of [PD-KV] "KV Cache 到底有多大？" per token (S = 1).

    The leading factor counts K and V; a latent (MLA) cache stores one shared
    row, tensors=1.
    """
    return tensors * n_layers * n_kv_heads * head_dim * bytes_per_elem
