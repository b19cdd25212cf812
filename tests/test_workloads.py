"""Host-side checks of the seeded input generator (CPU only)."""

import numpy as np
import pytest

from paged_kv_cache_288_amd.workloads import make_workload, SPECS, ALIASES, BF16_NAN, FP8_NAN


def _used_blocks(w):
    out = []
    for b in range(w.B):
        n = -(-int(w.context_lens[b]) // w.bs)
        out.append(w.block_table[b, :n])
    return out


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("gqa70b", dict(B=3, lens=("uniform", 40, 300))),
    ("splitk", dict(B=2, lens=("fixed", [1000, 1000]))),
    ("fp8prefix", dict(B=3, lens=("prefix", 64, 5, 40))),
    ("mla", dict(B=2, lens=("uniform", 65, 200))),
])
def test_structure_and_determinism(name, kw):
    w = make_workload(name, seed=1, **kw)
    w2 = make_workload(name, seed=1, **kw)
    for a, b in [(w.q, w2.q), (w.k_pool, w2.k_pool), (w.block_table, w2.block_table)]:
        assert np.array_equal(a, b)
    used = _used_blocks(w)
    flat = np.concatenate(used)
    assert flat.min() >= 0 and flat.max() < w.num_blocks
    # unused table entries are -1
    for b in range(w.B):
        assert (w.block_table[b, len(used[b]):] == -1).all()
    pb = w.meta["prefix_blocks"]
    if pb:
        for b in range(w.B):
            assert np.array_equal(used[b][:pb], used[0][:pb])
        tails = np.concatenate([u[pb:] for u in used])
        assert len(set(tails.tolist())) == len(tails)
        assert not set(tails.tolist()) & set(used[0][:pb].tolist())
    else:
        assert len(set(flat.tolist())) == len(flat), "no block is used twice"
    nan = FP8_NAN if w.kv_dtype == "fp8" else BF16_NAN
    # slots past each length, and unused blocks, hold NaN bits
    for b in range(w.B):
        L = int(w.context_lens[b])
        last = used[b][-1]
        tail = L % w.bs
        if tail:
            blk = w.k_pool[last]
            rows = blk[tail:] if w.kind == "mla" else blk[:, tail:]
            assert (rows == nan).all()
    unused = np.setdiff1d(np.arange(w.num_blocks), flat)
    if len(unused):
        assert (w.k_pool[unused] == nan).all()
    # the decode step's own token is the one at position L - 1, already stored
    for b in range(w.B):
        L = int(w.context_lens[b])
        phys = w.block_table[b, (L - 1) // w.bs]
        assert w.slot_mapping[b] == phys * w.bs + (L - 1) % w.bs
    if w.kv_dtype == "fp8":
        assert w.k_scale.shape == (w.Hkv,) and (w.k_scale > 0).all()


def test_full_size_specs_are_the_stated_shapes():
    assert set(ALIASES.values()) == set(SPECS)
    w = make_workload("tiny")
    assert w.q.shape == (2, 4, 64) and list(w.context_lens) == [200, 256] and w.num_blocks == 40
    assert w.block_table.shape == (2, 16) and w.scale == 1 / 8


def test_key_boost_scales_one_percent_of_keys():
    w = make_workload("splitk", B=1, lens=("fixed", [1600]))
    # boosted rows have |k| about 8x larger: their mean |k| stands out
    from oracle import gather_sequence, bf16_bits_to_f64   # test may use the oracle's decoders
    K = bf16_bits_to_f64(gather_sequence(w.k_pool, w.block_table[0], 1600, 16))
    norms = np.abs(K).mean(axis=2)                        # [Hkv, L]
    assert ((norms > 3.0).sum(axis=1) == 16).all()


def test_multi_token_workload_structure():
    """q_len > 1: q [B, q_len, Hq, d]; the step's tokens are the last q_len positions of
    each sequence, their slots and rows read back from the pool (-1 before position 0)."""
    w = make_workload("gqa70b", seed=3, B=5, lens=("fixed", [0, 2, 16, 17, 300]), q_len=4)
    assert w.q.shape == (5, 4, 64, 128) and w.q_len == 4
    assert w.slot_mapping.shape == (20,) and w.new_k.shape == (20, 8, 128)
    for b, L in enumerate(w.context_lens):
        for j in range(4):
            pos, i = int(L) - 4 + j, 4 * b + j
            if pos < 0:
                assert w.slot_mapping[i] == -1
                continue
            phys = int(w.block_table[b, pos // 16])
            assert w.slot_mapping[i] == phys * 16 + pos % 16
            assert np.array_equal(w.new_k[i], w.k_pool[phys, :, pos % 16])
            assert np.array_equal(w.new_v[i], w.v_pool[phys, :, pos % 16])
    full = make_workload("verify4")
    assert (full.B, full.q_len, full.Hq, full.Hkv, full.d) == (64, 4, 64, 8, 128)
