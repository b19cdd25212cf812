"""Oracle for the cache-management operations around the decode kernel.

TEST INFRASTRUCTURE ONLY: imported by the test suite; never by the product path.

Sources (cited by page title and section):

* [PD-KV] "PD 分离下的 KV Cache" (zer0e-github-io, ai-infra-7)
  - section "优化三：KV 传输优化", item "传输量化": KV is compressed to FP8 before it
    moves and decompressed (or used directly in low precision) where it lands;
  - section "优化一：Prefix Cache（前缀缓存）": the cache is reused per fixed-size token
    block; block i's hash is H(hash_{i-1}, tokens of block i), so two requests share a
    block's hash exactly when all tokens up to the end of that block agree.
* [Serving] "深入LLM推理：从KV Cache到PD分离的Serving全景解析", section
  "PagedAttention与Cache管理": physical blocks can be shared between requests, which
  is what prefix caching and copy-on-write build on.

Readings taken where the pages are silent:

* FP8 is OCP E4M3 with one fp32 scale per KV head (as for the decode path); the stored
  code of a value x is the E4M3 value nearest to the fp32 quotient x / scale (IEEE
  binary32 division), ties to the even code; magnitudes at or above 448 (the largest
  finite value) and infinities become +-448; NaN stays NaN (code S.1111.111);
* H is 64-bit FNV-1a over the previous hash's 8 bytes (little-endian) followed by the
  block's tokens as little-endian int32; the hash before the first block is a caller-
  given parent (0 for a sequence start); a trailing partial block has no hash.
"""

import numpy as np

from .paged_attention import fp8_e4m3fn_table

FP8_MAX = 448.0


def quantize_e4m3(quotient_f32):
    """E4M3 codes (uint8) of fp32 values: nearest representable value, ties to the even
    code, +-448 for magnitudes >= 448 and infinities, NaN -> S.1111.111.

    Nearest-value search over the 127 non-negative finite codes of the format's value
    table (codes 0..126 are increasing in value), done in float64 on the fp32 inputs.
    """
    v = np.asarray(quotient_f32, dtype=np.float32).astype(np.float64)
    table = fp8_e4m3fn_table()[:127]                       # codes 0..126, increasing
    a = np.abs(v)
    neg = np.signbit(v)
    codes = np.empty(v.shape, dtype=np.uint8)
    nan = np.isnan(v)
    sat = ~nan & (a >= FP8_MAX)
    mid = ~nan & ~sat
    am = a[mid]
    hi = np.searchsorted(table, am, side="left")          # first code with value >= a
    hi = np.clip(hi, 1, 126)
    lo = hi - 1
    d_lo = am - table[lo]
    d_hi = table[hi] - am
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(am == table[hi], hi, pick)
    codes[mid] = pick.astype(np.uint8)
    codes[sat] = 0x7E
    codes[nan] = 0x7F
    return np.where(neg, codes | np.uint8(0x80), codes).astype(np.uint8)


def kv_append_fp8(pool_codes, new_bf16_bits, scale, slot_mapping, block_size):
    """Quantizing append: token i's rows (bf16 bits [T, H, d]) become E4M3 codes
    quantize_e4m3(fp32(x) / fp32(scale[h])) in slot slot_mapping[i] of the pool
    [nb, H, bs, d]; slots < 0 are skipped.  Returns a new pool."""
    x = (np.asarray(new_bf16_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16))
    x = x.view(np.float32)
    s = np.asarray(scale, dtype=np.float32).reshape(1, -1, 1)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        q = (x / s).astype(np.float32)                     # IEEE binary32 division
    codes = quantize_e4m3(q)
    out = np.array(pool_codes, copy=True)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        out[slot // block_size, :, slot % block_size, :] = codes[i]
    return out


def copy_blocks(pool, src_blocks, dst_blocks):
    """Copy-on-write support: physical block dst[i] becomes a copy of block src[i] (all
    heads, all rows); pairs whose ids fall outside the pool are skipped."""
    out = np.array(pool, copy=True)
    nb = out.shape[0]
    for s, d in zip(np.asarray(src_blocks).tolist(), np.asarray(dst_blocks).tolist()):
        if 0 <= s < nb and 0 <= d < nb:
            out[d] = pool[s]
    return out


def fnv1a64(data):
    """64-bit FNV-1a of a byte string (offset basis 14695981039346656037, prime
    1099511628211)."""
    h = 14695981039346656037
    for byte in bytes(data):
        h ^= byte
        h = (h * 1099511628211) % (1 << 64)
    return h


def block_hashes(tokens, block_size, parent=0):
    """hash_i = H(hash_{i-1}, tokens of block i) for every full block of `tokens`."""
    toks = [int(t) for t in tokens]
    out = []
    prev = int(parent) % (1 << 64)
    for i in range(len(toks) // block_size):
        blk = toks[i * block_size:(i + 1) * block_size]
        data = prev.to_bytes(8, "little") + b"".join(
            (t % (1 << 32)).to_bytes(4, "little") for t in blk)
        prev = fnv1a64(data)
        out.append(prev)
    return out
