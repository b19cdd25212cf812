"""Seeded synthetic inputs for paged decode attention.

This module only draws and lays out inputs; it holds none of the attention
arithmetic, and both the HIP path (through the tests and bench) and the CPU
oracle read what it returns.  Every array is numpy on the host; the stored
K/V/q are the raw bits (bf16 as uint16, FP8 E4M3 as uint8).

Shapes follow the workloads the pages talk about:

* 70B-class GQA (80 layers, 8 KV heads, head dim 128, bf16): "深入LLM推理：从KV
  Cache到PD分离的Serving全景解析", section "KV Cache：Transformer的循环状态", and
  "PD 分离下的 KV Cache", section "KV Cache 到底有多大？" (worked example);
  one layer of it is one launch here.
* block size 16 tokens: "PD 分离下的 KV Cache", section "优化一：Prefix Cache"
  (typical block size) and the PagedAttention section of the first page.
* shared prefixes through shared physical blocks: first page, section
  "PagedAttention与Cache管理"; FP8 KV: "PD 分离下的 KV Cache", "优化三".
* MLA latent of 512 + 64 dims: first page, "KV Cache：Transformer的循环状态".

Recipe (fixed order of draws from ``numpy.random.default_rng([288, index, seed])``):
 1. context lengths (integers, both ends inclusive);
 2. pool size, then a permutation of the pool's block ids;
 3. block tables: each sequence takes the next ids of the permutation in
    order (a shared prefix takes the first ids once, for every sequence);
 4. q ~ N(0, 1) fp32 -> bf16 (round to nearest even);
 5. K then V ~ N(0, 1) fp32 for written slots only, sequence by sequence;
 6. workload transform (1% of keys x8 per (sequence, KV head); or FP8
    quantisation with per-KV-head scale = amax / 448, separately for K and V);
 7. rounding to the stored format; every other slot holds NaN bits
    (bf16 0x7FC0, FP8 0x7F) and unused block-table entries hold -1.
"""

from dataclasses import dataclass, field
import math

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
FP8_MAX = 448.0


@dataclass
class Workload:
    name: str
    kind: str                    # "gqa" or "mla"
    B: int
    Hq: int
    Hkv: int
    d: int                       # head dim of q and K (d_qk for MLA)
    d_v: int                     # head dim of V and out
    bs: int                      # tokens per physical block
    kv_dtype: str                # "bf16" or "fp8"
    scale: float
    partition_size: int          # 0 = library default
    q: np.ndarray                # uint16 [B, Hq, d] ([B, q_len, Hq, d] when q_len > 1)
    k_pool: np.ndarray           # [nb, Hkv, bs, d] (MLA: [nb, bs, d])
    v_pool: object               # [nb, Hkv, bs, d_v] or None for MLA
    k_scale: object              # float32 [Hkv] (FP8) or None
    v_scale: object
    block_table: np.ndarray      # int32 [B, max_blocks], -1 padded
    context_lens: np.ndarray     # int32 [B]
    new_k: np.ndarray            # bits [B * q_len, Hkv, d]: the tokens at L_b - q_len .. L_b - 1
    new_v: object                # bits [B * q_len, Hkv, d_v] or None (MLA)
    slot_mapping: np.ndarray     # int64 [B * q_len] (-1 for a position before the sequence)
    meta: dict = field(default_factory=dict)
    q_len: int = 1               # new query tokens per sequence (multi-token decode)

    @property
    def num_blocks(self):
        return self.k_pool.shape[0]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if self.B else 0

    @property
    def elem_bytes(self):
        return 1 if self.kv_dtype == "fp8" else 2


# name -> (index, spec).  The index is part of the seed.
SPECS = {
    "tiny-gqa-b2-h4x1-d64": (0, dict(
        kind="gqa", B=2, Hq=4, Hkv=1, d=64, bs=16, kv_dtype="bf16", scale=1.0 / 8.0,
        lens=("fixed", [200, 256]), pool=("fixed", 40), partition_size=0)),
    "gqa70b-b64-h64x8-d128-ctx1k-8k": (1, dict(
        kind="gqa", B=64, Hq=64, Hkv=8, d=128, bs=16, kv_dtype="bf16", scale=1.0 / math.sqrt(128),
        lens=("uniform", 1024, 8192), pool=("factor", 1.25), partition_size=0)),
    "gqa-splitk-b4-h64x8-d128-ctx32k": (2, dict(
        kind="gqa", B=4, Hq=64, Hkv=8, d=128, bs=16, kv_dtype="bf16", scale=1.0 / math.sqrt(128),
        # split-K into 512-token partitions: the library's default (balanced) mode cuts this
        # batch's 65,536 tiles into 2048 chunks of 32 tiles on a 256-CU MI355X, i.e. exactly
        # 64 partitions of 512 tokens per (sequence, KV head); partition_size=512 selects
        # the same split through the partitioned kernel
        lens=("fixed", [32768] * 4), pool=("factor", 1.25), partition_size=0,
        key_boost=(0.01, 8.0))),
    "gqa-fp8-prefix4k-b128-h32x8-d128": (3, dict(
        kind="gqa", B=128, Hq=32, Hkv=8, d=128, bs=16, kv_dtype="fp8", scale=1.0 / math.sqrt(128),
        lens=("prefix", 4096, 256, 2048), pool=("factor", 1.25), partition_size=0)),
    "mla-b32-h128-d576-ctx2k-8k": (4, dict(
        kind="mla", B=32, Hq=128, Hkv=1, d=576, d_v=512, bs=64, kv_dtype="bf16",
        scale=1.0 / math.sqrt(192), lens=("uniform", 2048, 8192), pool=("factor", 1.25),
        partition_size=0)),
    # The 70B-shaped batch verifying 4 new tokens per sequence (speculative decoding:
    # "深入LLM推理…", section "投机解码：打破每步一token的假设"); context lengths include them.
    "gqa70b-verify4-b64-h64x8-d128-ctx1k-8k": (5, dict(
        kind="gqa", B=64, Hq=64, Hkv=8, d=128, bs=16, kv_dtype="bf16", scale=1.0 / math.sqrt(128),
        lens=("uniform", 1024, 8192), pool=("factor", 1.25), partition_size=0, q_len=4)),
}

# Short aliases used on command lines.
ALIASES = {
    "tiny": "tiny-gqa-b2-h4x1-d64",
    "gqa70b": "gqa70b-b64-h64x8-d128-ctx1k-8k",
    "splitk": "gqa-splitk-b4-h64x8-d128-ctx32k",
    "fp8prefix": "gqa-fp8-prefix4k-b128-h32x8-d128",
    "mla": "mla-b32-h128-d576-ctx2k-8k",
    "verify4": "gqa70b-verify4-b64-h64x8-d128-ctx1k-8k",
}


def to_bf16_bits(x):
    """fp32 -> bf16 bits, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def to_fp8_bits(x):
    """fp32 -> OCP E4M3 bits via torch's conversion (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _lengths(rng, spec, B):
    kind = spec["lens"][0]
    if kind == "fixed":
        lens = list(spec["lens"][1])
        if len(lens) != B:
            lens = [lens[i % len(lens)] for i in range(B)]
        return np.array(lens, dtype=np.int64)
    if kind == "uniform":
        lo, hi = spec["lens"][1], spec["lens"][2]
        return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    if kind == "prefix":
        prefix, lo, hi = spec["lens"][1:]
        return prefix + rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    raise ValueError(kind)


def make_workload(name, seed=0, B=None, lens=None, pool=None, heads=None, q_len=None):
    """Build a workload by name (or alias); ``B``/``lens``/``pool``/``heads`` (a pair
    Hq, Hkv)/``q_len`` override the spec to make reduced-size variants of the same
    structure.  With q_len > 1, q holds q_len query tokens per sequence."""
    name = ALIASES.get(name, name)
    index, spec = SPECS[name]
    spec = dict(spec)
    if B is not None:
        spec["B"] = B
    if lens is not None:
        spec["lens"] = lens
    if pool is not None:
        spec["pool"] = pool
    if heads is not None:
        spec["Hq"], spec["Hkv"] = heads
    if q_len is not None:
        spec["q_len"] = q_len
    q_len = int(spec.get("q_len", 1))
    rng = np.random.default_rng([288, index, seed])
    kind = spec["kind"]
    B, Hq, Hkv, d, bs = spec["B"], spec["Hq"], spec["Hkv"], spec["d"], spec["bs"]
    d_v = spec.get("d_v", d)
    fp8 = spec["kv_dtype"] == "fp8"

    # 1. lengths
    lens = _lengths(rng, spec, B)
    prefix_tokens = spec["lens"][1] if spec["lens"][0] == "prefix" else 0
    prefix_blocks = prefix_tokens // bs
    nblk = -(-lens // bs)
    own_blocks = nblk - prefix_blocks
    needed = prefix_blocks + int(own_blocks.sum())

    # 2. pool size and permutation
    if spec["pool"][0] == "fixed":
        num_blocks = int(spec["pool"][1])
    else:
        num_blocks = int(math.ceil(spec["pool"][1] * needed))
    if num_blocks < needed:
        raise ValueError("pool too small")
    perm = rng.permutation(num_blocks).astype(np.int64)

    # 3. block tables
    # Table width covers the longest length the spec allows, not just the drawn one.
    if spec["lens"][0] == "uniform":
        max_len = spec["lens"][2]
    elif spec["lens"][0] == "prefix":
        max_len = prefix_tokens + spec["lens"][3]
    else:
        max_len = 0
    max_len = max(int(max_len), int(lens.max()) if B else 0)
    max_blocks = max(1, -(-max_len // bs))
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    shared = perm[:prefix_blocks]
    cursor = prefix_blocks
    for b in range(B):
        table[b, :prefix_blocks] = shared
        k = int(own_blocks[b])
        table[b, prefix_blocks:prefix_blocks + k] = perm[cursor:cursor + k]
        cursor += k

    # 4. q
    qshape = (B, Hq, d) if q_len == 1 else (B, q_len, Hq, d)
    q = to_bf16_bits(rng.standard_normal(qshape, dtype=np.float32))

    # 5.-7. K and V, sequence by sequence over written slots only
    heads = 1 if kind == "mla" else Hkv
    if kind == "mla":
        k_pool = np.full((num_blocks, bs, d), BF16_NAN, dtype=np.uint16)
        v_pool = None
    else:
        nan = FP8_NAN if fp8 else BF16_NAN
        dt = np.uint8 if fp8 else np.uint16
        k_pool = np.full((num_blocks, Hkv, bs, d), nan, dtype=dt)
        v_pool = np.full((num_blocks, Hkv, bs, d_v), nan, dtype=dt)

    # Values in logical order: a shared prefix once, then each sequence's own tokens.
    segs = []                               # (block ids, first logical token, K fp32, V fp32)
    if prefix_blocks:
        kp = rng.standard_normal((prefix_tokens, heads, d), dtype=np.float32)
        vp = rng.standard_normal((prefix_tokens, heads, d_v), dtype=np.float32)
        segs.append((shared, 0, kp, vp, None))
    boost = spec.get("key_boost")
    for b in range(B):
        n_own = int(lens[b]) - prefix_tokens
        kb = rng.standard_normal((n_own, heads, d), dtype=np.float32)
        vb = None if kind == "mla" else rng.standard_normal((n_own, heads, d_v), dtype=np.float32)
        segs.append((table[b, prefix_blocks:prefix_blocks + int(own_blocks[b])], prefix_tokens, kb, vb, b))
    if boost is not None:
        frac, factor = boost
        for (_, _, kb, _, b) in segs:
            L = kb.shape[0]
            n = int(round(frac * L))
            for g in range(heads):
                pos = rng.choice(L, size=n, replace=False)
                kb[pos, g, :] *= np.float32(factor)

    k_scale = v_scale = None
    if fp8:
        k_amax = np.max([np.abs(s[2]).max(axis=(0, 2)) for s in segs], axis=0)
        v_amax = np.max([np.abs(s[3]).max(axis=(0, 2)) for s in segs], axis=0)
        k_scale = (k_amax / np.float32(FP8_MAX)).astype(np.float32)
        v_scale = (v_amax / np.float32(FP8_MAX)).astype(np.float32)

    def store(pool, ids, vals, sc):
        n = len(ids)
        if vals.shape[0] == 0:
            return
        if fp8:
            bits = to_fp8_bits(vals / sc[None, :, None])
        else:
            bits = to_bf16_bits(vals)
        if kind == "mla":
            pad = np.full((n * bs, bits.shape[-1]), BF16_NAN, dtype=bits.dtype)
            pad[:bits.shape[0]] = bits[:, 0, :]
            pool[ids] = pad.reshape(n, bs, -1)
        else:
            pad = np.full((n * bs,) + bits.shape[1:], FP8_NAN if fp8 else BF16_NAN, dtype=bits.dtype)
            pad[:bits.shape[0]] = bits
            pool[ids] = pad.reshape(n, bs, bits.shape[1], bits.shape[2]).transpose(0, 2, 1, 3)

    for (ids, _, kb, vb, _) in segs:
        store(k_pool, ids, kb, k_scale)
        if v_pool is not None:
            store(v_pool, ids, vb, v_scale)

    # The decode step's own tokens: positions L_b - q_len .. L_b - 1 (already in the
    # pool, so appending them again leaves the pool unchanged).
    pos = (lens[:, None] - q_len + np.arange(q_len)[None, :]).reshape(-1)
    seq = np.repeat(np.arange(B), q_len)
    live = pos >= 0
    posc = np.where(live, pos, 0)
    phys = table[seq, posc // bs].astype(np.int64)
    off = posc % bs
    slot_mapping = np.where(live, phys * bs + off, -1).astype(np.int64)
    if kind == "mla":
        new_k = k_pool[phys, off][:, None, :].copy()
        new_v = None
    else:
        new_k = k_pool[phys, :, off, :].copy()
        new_v = v_pool[phys, :, off, :].copy()
        if not live.all():
            new_k[~live] = new_k.dtype.type(0)
            new_v[~live] = new_v.dtype.type(0)

    return Workload(
        name=name, kind=kind, B=B, Hq=Hq, Hkv=Hkv, d=d, d_v=d_v, bs=bs,
        kv_dtype=spec["kv_dtype"], scale=float(spec["scale"]),
        partition_size=int(spec.get("partition_size", 0)),
        q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
        block_table=table, context_lens=lens.astype(np.int32),
        new_k=new_k, new_v=new_v, slot_mapping=slot_mapping,
        meta=dict(prefix_blocks=prefix_blocks, seed=seed), q_len=q_len,
    )
