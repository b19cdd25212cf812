"""Pins for the fp64 oracle (CPU only).

Every check compares the oracle with something other than itself: brute force
in 50-digit decimal arithmetic that walks the block table position by
position, a library routine (torch's CPU float64 scaled_dot_product_attention,
torch's bfloat16/float8 decoders), a closed form or a value the pages print, or
an invariant the mathematics fixes.  ``test_planted_mistakes_are_caught`` runs
the same pins against copies of the oracle with one plausible mistake each
(a wrong index, a dropped term, a flipped sign, a transposed operand) and
requires that each copy fails at least one pin.
"""

import decimal
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle as REAL
from oracle import paged_attention as PA

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# Tiny fixtures: a contiguous history scattered into a shuffled pool by the test
# --------------------------------------------------------------------------

def scatter_history(hists, bs, rng, spare=3, fill=np.nan):
    """hists: list over sequences of arrays [H, L_b, d].  Returns (pool, table, lens)
    with each sequence's blocks drawn from a random permutation of the pool."""
    H, d = hists[0].shape[0], hists[0].shape[2]
    nblk = [-(-h.shape[1] // bs) for h in hists]
    num_blocks = sum(nblk) + spare
    perm = rng.permutation(num_blocks)
    pool = np.full((num_blocks, H, bs, d), fill)
    table = np.full((len(hists), max(max(nblk), 1)), -1, dtype=np.int64)
    cur = 0
    for b, h in enumerate(hists):
        for t in range(h.shape[1]):
            blk = t // bs
            if t % bs == 0:
                table[b, blk] = perm[cur]
                cur += 1
            pool[table[b, blk], :, t % bs, :] = h[:, t, :]
    return pool, table, np.array([h.shape[1] for h in hists])


def tiny_case(seed=0, B=2, Hq=4, Hkv=2, d=5, d_v=3, bs=4, lens=(7, 8)):
    rng = np.random.default_rng(seed)
    K = [rng.standard_normal((Hkv, L, d)) for L in lens]
    V = [rng.standard_normal((Hkv, L, d_v)) for L in lens]
    q = rng.standard_normal((B, Hq, d))
    state = np.random.default_rng(seed + 1000)
    kp, table, lens_a = scatter_history(K, bs, state)
    state = np.random.default_rng(seed + 1000)           # same permutation for V
    vp, _, _ = scatter_history(V, bs, state)
    return dict(q=q, K=K, V=V, k_pool=kp, v_pool=vp, table=table, lens=lens_a, bs=bs,
                scale=1.0 / math.sqrt(d), G=Hq // Hkv)


def brute_attention(q, k_pool, v_pool, table, lens, scale, G, bs):
    """Position-by-position walk of the block table, exact products and 50-digit exp."""
    ctx = decimal.Context(prec=50)
    D = decimal.Decimal
    B, Hq, d = q.shape
    d_v = v_pool.shape[3]
    out = np.zeros((B, Hq, d_v))
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            g = h // G
            weights, rows = [], []
            for t in range(L):
                phys, off = int(table[b][t // bs]), t % bs
                s = sum((ctx.multiply(D(float(q[b, h, i])), D(float(k_pool[phys, g, off, i])))
                         for i in range(d)), D(0))
                weights.append(ctx.exp(ctx.multiply(s, D(float(scale)))))
                rows.append([D(float(v_pool[phys, g, off, j])) for j in range(d_v)])
            den = sum(weights, D(0))
            for j in range(d_v):
                num = sum((ctx.multiply(w, r[j]) for w, r in zip(weights, rows)), D(0))
                out[b, h, j] = float(ctx.divide(num, den))
    return out


def sdpa(qv, K, V, scale):
    """torch CPU float64 attention of one query row set over a contiguous history."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qv)[None, :, None, :], torch.from_numpy(K)[None],
        torch.from_numpy(V)[None], scale=scale)
    return out[0, :, 0, :].numpy()


def close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and bool(np.all(np.abs(a - b) <= tol * (1.0 + np.abs(b))))


# --------------------------------------------------------------------------
# Pins, each a function of an oracle namespace O (raises AssertionError on failure)
# --------------------------------------------------------------------------

def pin_attention_brute_force(O):
    for seed, lens, bs in [(0, (7, 8), 4), (1, (1, 6), 2), (2, (5, 3), 4)]:
        c = tiny_case(seed, lens=lens, bs=bs)
        got = O.paged_decode_attention(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], c["scale"])
        ref = brute_attention(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], c["scale"], c["G"], bs)
        assert close(got, ref, 1e-13), "oracle vs decimal brute force"


def pin_attention_vs_sdpa(O):
    # d == d_v here so that a K/V mix-up cannot hide behind a shape error.
    for seed, (Hq, Hkv) in enumerate([(4, 2), (8, 2), (3, 3), (4, 1)]):
        c = tiny_case(seed + 10, Hq=Hq, Hkv=Hkv, d=6, d_v=6, bs=4, lens=(9, 13))
        got = O.paged_decode_attention(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], c["scale"])
        G = Hq // Hkv
        for b in range(2):
            ref = sdpa(c["q"][b], np.repeat(c["K"][b], G, axis=0), np.repeat(c["V"][b], G, axis=0), c["scale"])
            assert close(got[b], ref, 1e-12), "oracle vs torch SDPA (GQA by repeat_interleave)"


def pin_mla_vs_sdpa(O):
    rng = np.random.default_rng(5)
    d_qk, d_v, bs, Hq = 10, 7, 4, 3
    lat = [rng.standard_normal((1, L, d_qk)) for L in (11, 4)]
    pool4, table, lens = scatter_history(lat, bs, np.random.default_rng(6))
    q = rng.standard_normal((2, Hq, d_qk))
    got = O.mla_decode_attention(q, pool4[:, 0], table, lens, 0.3, d_v)
    for b in range(2):
        C = lat[b][0]
        ref = sdpa(q[b], np.repeat(C[None], Hq, 0), np.repeat(C[None, :, :d_v], Hq, 0), 0.3)
        assert close(got[b], ref, 1e-12), "MLA oracle vs SDPA with V = first d_v latent dims"


def pin_block_permutation_invariance(O):
    c = tiny_case(3, lens=(10, 7), bs=4)
    base = O.paged_decode_attention(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], c["scale"])
    rng = np.random.default_rng(9)
    nb = c["k_pool"].shape[0]
    for _ in range(3):
        p = rng.permutation(nb)
        kp, vp = np.empty_like(c["k_pool"]), np.empty_like(c["v_pool"])
        kp[p], vp[p] = c["k_pool"], c["v_pool"]
        table = np.where(c["table"] >= 0, p[np.maximum(c["table"], 0)], -1)
        got = O.paged_decode_attention(c["q"], kp, vp, table, c["lens"], c["scale"])
        assert np.array_equal(got, base), "output must not depend on where blocks live"


def pin_single_token_returns_v(O):
    c = tiny_case(4, lens=(1, 1), bs=4)
    got = O.paged_decode_attention(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], c["scale"])
    for b in range(2):
        for h in range(4):
            assert np.array_equal(got[b, h], c["V"][b][h // c["G"], 0]), "L = 1 must return v exactly"


def pin_constant_v(O):
    c = tiny_case(5, lens=(9, 6), bs=4)
    vp = np.full_like(c["v_pool"], np.nan)
    const = np.array([0.75, -1.5, 3.0])
    for g in range(2):
        vp[:, g, :, :] = const * (g + 1)
    got = O.paged_decode_attention(c["q"], c["k_pool"], vp, c["table"], c["lens"], c["scale"])
    for h in range(4):
        assert close(got[:, h], np.broadcast_to(const * (h // 2 + 1), (2, 3)), 1e-15), "constant V"


def pin_gqa_equals_replicated_mha(O):
    c = tiny_case(6, Hq=6, Hkv=2, lens=(8, 5), bs=4)
    got = O.paged_decode_attention(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], c["scale"])
    rep = O.paged_decode_attention(c["q"], np.repeat(c["k_pool"], 3, axis=1), np.repeat(c["v_pool"], 3, axis=1),
                                   c["table"], c["lens"], c["scale"])
    assert close(got, rep, 1e-15), "GQA(G) == MHA with each KV head repeated G times"


def pin_linearity_in_v(O):
    c = tiny_case(7, lens=(11, 3), bs=4)
    a = O.paged_decode_attention(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], c["scale"])
    b = O.paged_decode_attention(c["q"], c["k_pool"], 2.0 * c["v_pool"], c["table"], c["lens"], c["scale"])
    assert np.array_equal(b, 2.0 * a), "out(2V) == 2 out(V) exactly"


def pin_two_token_closed_form(O):
    # scores (0, ln 3) -> weights (1/4, 3/4)
    d, bs, scale = 4, 2, 0.5
    q = np.zeros((1, 1, d)); q[0, 0, 0] = 1.0
    K = np.zeros((1, 2, d)); K[0, 1, 0] = math.log(3.0) / scale
    V = np.array([[[1.0, -2.0, 0.5, 4.0], [5.0, 2.0, -0.5, 0.0]]])
    kp, table, lens = scatter_history([K], bs, np.random.default_rng(0))
    vp, _, _ = scatter_history([V], bs, np.random.default_rng(0))
    got = O.paged_decode_attention(q, kp, vp, table, lens, scale)[0, 0]
    assert close(got, (V[0, 0] + 3.0 * V[0, 1]) / 4.0, 1e-15), "two-token closed form"


def pin_empty_sequence_is_zero(O):
    c = tiny_case(8, lens=(5, 3), bs=4)
    lens = np.array([0, 3])
    got = O.paged_decode_attention(c["q"], c["k_pool"], c["v_pool"], c["table"], lens, c["scale"])
    assert np.array_equal(got[0], np.zeros_like(got[0])), "reading: L = 0 gives 0"


def pin_append_brute_force(O):
    rng = np.random.default_rng(11)
    nb, H, bs, d = 6, 2, 4, 3
    pool = rng.integers(0, 2 ** 16, size=(nb, H, bs, d), dtype=np.uint16)
    new = rng.integers(0, 2 ** 16, size=(6, H, d), dtype=np.uint16)
    slots = np.array([0, 9, -1, 6, 14, 3])      # block/offset swaps of these stay in range
    got = O.kv_append(pool, new, slots, bs)
    ref = pool.copy()
    for i in range(len(slots)):
        if slots[i] < 0:
            continue
        for h in range(H):
            for j in range(d):
                ref[slots[i] // bs, h, slots[i] % bs, j] = new[i, h, j]
    assert got.dtype == pool.dtype and np.array_equal(got, ref), "append vs element loop"
    assert not np.shares_memory(got, pool), "append returns a new pool"


def pin_split_merge_equals_direct(O):
    rng = np.random.default_rng(12)
    L, d, d_v = 37, 5, 4
    K, V, qv = rng.standard_normal((L, d)) * 3, rng.standard_normal((L, d_v)), rng.standard_normal(d)
    direct = sdpa(qv[None], K[None], V[None], 0.7)[0]
    for part in (1, 5, 16, 36, 37, 64):
        m, l, o = O.partition_partials(qv, K, V, 0.7, part)
        assert len(m) == -(-L // part)
        assert close(O.merge_partials(m, l, o), direct, 1e-12), "split + merge == single pass"
    m, l, o = O.partition_partials(qv, K, V, 0.7, 8)
    m2 = np.append(m, -np.inf)
    l2 = np.append(l, 0.0)
    o2 = np.vstack([o, np.zeros(d_v)])
    assert close(O.merge_partials(m2, l2, o2), direct, 1e-12), "empty partition ignored"


def pin_bf16_decode(O):
    codes = np.arange(2 ** 16, dtype=np.uint16)
    got = O.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "bf16 decode vs torch"
    assert O.bf16_bits_to_f64(np.uint16(0x3F80)) == 1.0 and O.bf16_bits_to_f64(np.uint16(0xC000)) == -2.0
    assert O.bf16_bits_to_f64(np.uint16(0x0001)) == 2.0 ** -133


def pin_fp8_decode(O):
    gold = json.load(open(os.path.join(GOLD, "fp8_e4m3fn_points.json")))
    t = O.fp8_e4m3fn_table()
    for code, val in gold["points"].items():
        assert t[int(code, 16)] == val and math.copysign(1, t[int(code, 16)]) == math.copysign(1, val)
    for code in gold["nan_codes"]:
        assert np.isnan(t[int(code, 16)])
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(t[ok], ref[ok]), "fp8 table vs torch float8_e4m3fn"
    bits = np.array([[[[0x38, 0x40]]], [[[0x3c, 0xb8]]]], dtype=np.uint8).reshape(1, 2, 1, 2)
    vals = O.decode_kv_bits(bits, "fp8", np.array([0.5, 4.0], dtype=np.float32))
    assert np.array_equal(vals.reshape(-1), [0.5, 1.0, 6.0, -4.0]), "per-head scale on axis 1"


def pin_kv_size_worked_example(O):
    g = json.load(open(os.path.join(GOLD, "kv_size_70b.json")))
    per_tok = O.kv_bytes_per_token(g["n_layers"], g["n_kv_heads"], g["head_dim"], g["bytes_per_elem"])
    assert per_tok == g["bytes_per_token"]
    assert per_tok == 320 * 1024
    assert per_tok * g["context_tokens"] == g["bytes_per_context_approx_gb"] * 2 ** 30
    # MLA: one shared 576-dim latent row per token and layer, bf16
    assert O.kv_bytes_per_token(1, 1, 576, 2, tensors=1) == 1152


PINS = [pin_attention_brute_force, pin_attention_vs_sdpa, pin_mla_vs_sdpa,
        pin_block_permutation_invariance, pin_single_token_returns_v, pin_constant_v,
        pin_gqa_equals_replicated_mha, pin_linearity_in_v, pin_two_token_closed_form,
        pin_empty_sequence_is_zero, pin_append_brute_force, pin_split_merge_equals_direct,
        pin_bf16_decode, pin_fp8_decode, pin_kv_size_worked_example]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(REAL)


# --------------------------------------------------------------------------
# Planted mistakes: each copy of the oracle below carries one, and must fail a pin
# --------------------------------------------------------------------------

def _namespace(**over):
    ns = types.SimpleNamespace(**{n: getattr(PA, n) for n in REAL.__all__}) if hasattr(REAL, "__all__") else \
        types.SimpleNamespace(**{n: getattr(PA, n) for n in dir(PA) if not n.startswith("_")})
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _attn(gather=PA.gather_sequence, group="div", scale_on=True, sign=1.0, normalize=True, use_v=True):
    def f(q, k_pool, v_pool, block_table, context_lens, scale):
        B, Hq, _ = q.shape
        Hkv, bs = k_pool.shape[1], k_pool.shape[2]
        G = Hq // Hkv
        out = np.zeros((B, Hq, v_pool.shape[3]))
        for b in range(B):
            L = int(context_lens[b])
            if L == 0:
                continue
            K = gather(k_pool, block_table[b], L, bs)
            V = gather(v_pool, block_table[b], L, bs) if use_v else K
            for h in range(Hq):
                g = h // G if group == "div" else h % Hkv
                s = (scale if scale_on else 1.0) * (K[g] @ q[b, h])
                w = np.exp(sign * (s - s.max()))
                o = w @ V[g][:, :v_pool.shape[3]]
                out[b, h] = o / w.sum() if normalize else o
        return out
    return f


def _gather_drop_partial(pool, ids, L, bs):
    n = L // bs
    hist = pool[np.asarray(ids[:n], dtype=np.int64)].transpose(1, 0, 2, 3).reshape(pool.shape[1], n * bs, -1)
    return hist[:, :L]


def _gather_no_transpose(pool, ids, L, bs):
    n = -(-L // bs)
    hist = pool[np.asarray(ids[:n], dtype=np.int64)].reshape(pool.shape[1], n * bs, -1)
    return hist[:, :L]


def _gather_shifted(pool, ids, L, bs):
    n = -(-L // bs) + 1
    idx = np.asarray(ids[:n], dtype=np.int64)
    hist = pool[idx].transpose(1, 0, 2, 3).reshape(pool.shape[1], len(idx) * bs, -1)
    return hist[:, 1:L + 1] if hist.shape[1] > L else hist[:, :L]


def _gather_reversed(pool, ids, L, bs):
    n = -(-L // bs)
    idx = np.asarray(ids[:n], dtype=np.int64)[::-1]
    hist = pool[idx].transpose(1, 0, 2, 3).reshape(pool.shape[1], n * bs, -1)
    return hist[:, :L]


def _append_swapped(pool, new, slots, bs):
    out = np.array(pool, copy=True)
    for i, s in enumerate(slots):
        if s >= 0:
            out[s % bs, :, s // bs, :] = new[i]
    return out


def _append_no_skip(pool, new, slots, bs):
    out = np.array(pool, copy=True)
    for i, s in enumerate(slots):
        out[s // bs, :, s % bs, :] = new[i]
    return out


def _merge_no_rescale(m, l, o):
    return np.asarray(o).sum(0) / np.asarray(l).sum()


def _partials_drop_tail(q_vec, K, V, scale, part):
    L = K.shape[0]
    keep = max(part, (L // part) * part)
    return PA.partition_partials(q_vec, K[:keep], V[:keep], scale, part)


def _bf16_shift15(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)


def _fp8_bias8():
    t = PA.fp8_e4m3fn_table()
    return t / 2.0


def _fp8_bad_subnormal():
    t = PA.fp8_e4m3fn_table().copy()
    for code in range(256):
        if (code >> 3) & 0xF == 0:
            t[code] = (-1.0 if code & 0x80 else 1.0) * (code & 7) / 8.0 * 2.0 ** -7
    return t


def _mla_last_dims(q, kv_pool, block_table, context_lens, scale, d_v):
    kv = np.asarray(kv_pool, dtype=np.float64)[:, None]
    return PA.paged_decode_attention(q, kv, kv[..., -d_v:], block_table, context_lens, scale)


MUTANTS = {
    "grouping h % Hkv": dict(paged_decode_attention=_attn(group="mod")),
    "scale dropped": dict(paged_decode_attention=_attn(scale_on=False)),
    "exp sign flipped": dict(paged_decode_attention=_attn(sign=-1.0)),
    "no normalisation": dict(paged_decode_attention=_attn(normalize=False)),
    "K used as V": dict(paged_decode_attention=_attn(use_v=False)),
    "partial last block dropped": dict(paged_decode_attention=_attn(gather=_gather_drop_partial)),
    "block layout not transposed": dict(paged_decode_attention=_attn(gather=_gather_no_transpose)),
    "history off by one": dict(paged_decode_attention=_attn(gather=_gather_shifted)),
    "block table reversed": dict(paged_decode_attention=_attn(gather=_gather_reversed)),
    "append block/offset swapped": dict(kv_append=_append_swapped),
    "append ignores slot < 0": dict(kv_append=_append_no_skip),
    "merge without rescale": dict(merge_partials=_merge_no_rescale),
    "partials drop the tail": dict(partition_partials=_partials_drop_tail),
    "bf16 widened by 15 bits": dict(bf16_bits_to_f64=_bf16_shift15),
    "fp8 exponent bias 8": dict(fp8_e4m3fn_table=_fp8_bias8),
    "fp8 subnormal scale": dict(fp8_e4m3fn_table=_fp8_bad_subnormal),
    "kv size without the K/V factor": dict(
        kv_bytes_per_token=lambda L, H, d, b, tensors=2: L * H * d * b),
    "MLA value = last dims": dict(mla_decode_attention=_mla_last_dims),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_are_caught(name):
    ns = _namespace(**MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            pin(ns)
        except Exception as e:      # AssertionError, or a crash caused by the mistake
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"no pin catches the planted mistake {name!r}"


def test_unmutated_namespace_passes_every_pin():
    ns = _namespace()
    for pin in PINS:
        pin(ns)
    # and the test-side re-implementation with no mistake is also clean
    ns2 = _namespace(paged_decode_attention=_attn())
    for pin in PINS:
        pin(ns2)


def _pin_multi_token(multi_fn):
    """Pin of the multi-token decode: dense attention with an explicit causal mask over
    the gathered sequence (the new tokens are its last q_len positions), q_len = 1 against
    the single-token oracle, and a token whose context is empty against 0."""
    rng = np.random.default_rng(21)
    B, q_len, Hq, Hkv, d, bs = 3, 4, 4, 2, 8, 4
    lens = np.array([9, 4, 2])
    nb = 8
    k_pool = rng.standard_normal((nb, Hkv, bs, d))
    v_pool = rng.standard_normal((nb, Hkv, bs, d))
    table = np.array([[3, 0, 6], [5, 1, 7], [2, 4, 7]])
    q = rng.standard_normal((B, q_len, Hq, d))
    got = multi_fn(q, k_pool, v_pool, table, lens, 0.3)
    G = Hq // Hkv
    for b in range(B):
        L = int(lens[b])
        K = np.concatenate([k_pool[table[b, i]] for i in range(3)], axis=1)[:, :L]   # [Hkv, L, d]
        V = np.concatenate([v_pool[table[b, i]] for i in range(3)], axis=1)[:, :L]
        for h in range(Hq):
            S = q[b, :, h] @ K[h // G].T * 0.3                      # [q_len, L]
            pos = np.arange(L)[None, :]
            row = (L - q_len + np.arange(q_len))[:, None]            # position of each new token
            S = np.where(pos <= row, S, -np.inf)
            for j in range(q_len):
                if not np.isfinite(S[j]).any():
                    assert np.all(got[b, j, h] == 0)
                    continue
                p = np.exp(S[j] - S[j].max())
                assert np.allclose(got[b, j, h], p @ V[h // G] / p.sum(), rtol=1e-12, atol=1e-12)
    one = multi_fn(q[:, :1], k_pool, v_pool, table, lens, 0.3)
    assert np.array_equal(one[:, 0], REAL.paged_decode_attention(q[:, 0], k_pool, v_pool,
                                                                    table, lens, 0.3))


def test_multi_token_decode_is_causal_attention_over_the_new_tokens():
    _pin_multi_token(REAL.multi_token_decode_attention)


def _multi_mutant(shift=0, reverse=False, causal=True):
    """The multi-token oracle with one plausible mistake: the visible length off by
    `shift`, the query tokens taken in reverse order, or no causal mask at all."""
    def fn(q, k_pool, v_pool, block_table, context_lens, scale):
        q = np.asarray(q, dtype=np.float64)
        B, q_len = q.shape[:2]
        lens = np.asarray(context_lens, dtype=np.int64)
        out = np.zeros(q.shape[:3] + (np.asarray(v_pool).shape[-1],))
        for j in range(q_len):
            jj = q_len - 1 - j if reverse else j
            seen = lens - (q_len - 1 - jj) + shift if causal else lens
            out[:, j] = REAL.paged_decode_attention(q[:, j], k_pool, v_pool, block_table,
                                                    np.clip(seen, 0, lens), scale)
        return out
    return fn


@pytest.mark.parametrize("mutant", [dict(shift=-1), dict(shift=1), dict(reverse=True),
                                    dict(causal=False)])
def test_multi_token_pin_catches_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _pin_multi_token(_multi_mutant(**mutant))


def test_multi_token_mutant_without_mistake_passes():
    _pin_multi_token(_multi_mutant())
