"""GPU parity of pkv_paged_decode_attn_multi (multi-token decode, the verify pass of
speculative decoding) through the C-ABI against the fp64 oracle.

Every row count the kernel specialises on (q_len * G up to 16, 32 and 64 query rows per
KV head) is compared element by element on reduced workloads spanning many tiles and
ragged tails; the full-size 70B-shaped verify batch, as benchmarked, on every output
row.  Edge cases: contexts shorter than q_len (early query tokens see nothing and
give zeros), empty sequences, one long sequence spread over many chunks, q_len = 1
against the single-token oracle, and block-permutation invariance (bitwise)."""

import numpy as np
import pytest

import oracle
from gpu_common import _subset, assert_close, bits_to_device, log, make_workload, torch_cuda

pytestmark = pytest.mark.gpu


def gpu_multi(torch, w, out=None):
    import paged_kv_cache_288_amd as pkv
    q = bits_to_device(torch, w.q.reshape(w.B, w.q_len, w.Hq, w.d))
    kp = bits_to_device(torch, w.k_pool)
    vp = bits_to_device(torch, w.v_pool)
    bt = torch.from_numpy(w.block_table).to("cuda")
    cl = torch.from_numpy(w.context_lens).to("cuda")
    if out is None:
        out = torch.empty((w.B, w.q_len, w.Hq, w.d_v), dtype=torch.float32, device="cuda")
    ks = None if w.k_scale is None else torch.from_numpy(w.k_scale).to("cuda")
    vs = None if w.v_scale is None else torch.from_numpy(w.v_scale).to("cuda")
    pkv.paged_decode_attn_multi(out, q, kp, vp, bt, cl, w.scale, w.max_context_len,
                                kv_dtype=w.kv_dtype, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_multi(w, seqs=None):
    seqs = range(w.B) if seqs is None else list(seqs)
    kp, vp, table, lens, _ = _subset(w, seqs)
    q = oracle.bf16_bits_to_f64(w.q.reshape(w.B, w.q_len, w.Hq, w.d)[list(seqs)])
    K = oracle.decode_kv_bits(kp, w.kv_dtype, w.k_scale)
    V = oracle.decode_kv_bits(vp, w.kv_dtype, w.v_scale)
    return oracle.multi_token_decode_attention(q, K, V, table, lens, w.scale)


@pytest.mark.parametrize("q_len", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("gqa70b", dict(B=5, lens=("uniform", 1, 1500))),
])
def test_multi_matches_oracle(name, over, q_len):
    torch = torch_cuda()
    for seed in (0, 1):
        w = make_workload(name, seed=seed, q_len=q_len, **over)
        log(f"[multi] {w.name} q_len={q_len} seed={seed} G={w.Hq // w.Hkv} "
            f"lens={w.context_lens.tolist()}")
        assert_close(gpu_multi(torch, w), oracle_multi(w), "bf16", f"{name} q_len={q_len}/{seed}")


@pytest.mark.parametrize("heads,q_len", [((64, 8), 2), ((16, 8), 16), ((32, 8), 16),
                                         ((8, 8), 64), ((8, 1), 5), ((4, 1), 16)])
def test_multi_row_counts(heads, q_len):
    """Rows per KV head from 4 to 64 with several group sizes (padding rows included)."""
    torch = torch_cuda()
    w = make_workload("gqa70b", seed=9, B=3, lens=("uniform", 40, 900), heads=heads,
                      q_len=q_len)
    log(f"[multi] heads={heads} q_len={q_len} lens={w.context_lens.tolist()}")
    assert_close(gpu_multi(torch, w), oracle_multi(w), "bf16", f"heads {heads} q_len {q_len}")


@pytest.mark.parametrize("q_len,heads", [(4, (32, 8)), (2, (64, 8)), (16, (32, 8))])
def test_multi_fp8(q_len, heads):
    """FP8 E4M3 K/V with per-head scales (codes widened exactly on the way to the MFMA)."""
    torch = torch_cuda()
    w = make_workload("fp8prefix", seed=6, B=5, lens=("prefix", 64, 1, 700), q_len=q_len,
                      heads=heads)
    log(f"[multi] fp8 q_len={q_len} heads={heads} lens={w.context_lens.tolist()}")
    assert_close(gpu_multi(torch, w), oracle_multi(w), "fp8", f"fp8 q_len={q_len}")


def test_multi_short_and_empty_contexts():
    """Contexts shorter than q_len: query token j of a sequence of length L sees
    L - q_len + 1 + j tokens, none (output 0) when that is not positive."""
    torch = torch_cuda()
    w = make_workload("gqa70b", seed=4, B=12, q_len=8, heads=(32, 4), pool=("factor", 1.5),
                      lens=("fixed", [0, 1, 2, 7, 8, 3, 9, 15, 16, 17, 20, 33]))
    log(f"[multi] short lens={w.context_lens.tolist()}")
    got = gpu_multi(torch, w)
    ref = oracle_multi(w)
    assert (got[0] == 0).all()
    assert (got[5, :5] == 0).all() and (np.abs(got[5, 5:]) > 0).any()
    assert_close(got, ref, "bf16", "short/empty")


def test_multi_one_long_sequence():
    """One 20000-token sequence: its tiles spread over many chunks and pieces."""
    torch = torch_cuda()
    w = make_workload("gqa70b", seed=11, B=1, lens=("fixed", [20000]), q_len=4)
    log(f"[multi] long lens={w.context_lens.tolist()}")
    assert_close(gpu_multi(torch, w), oracle_multi(w), "bf16", "one long sequence")


def test_multi_q_len_one_is_single_token_decode():
    torch = torch_cuda()
    w = make_workload("gqa70b", seed=2, B=4, lens=("uniform", 1, 800), q_len=1)
    got = gpu_multi(torch, w)[:, 0]
    kp, vp, table, lens, _ = _subset(w, range(w.B))
    ref = oracle.paged_decode_attention(oracle.bf16_bits_to_f64(w.q), oracle.decode_kv_bits(kp, "bf16"),
                                        oracle.decode_kv_bits(vp, "bf16"), table, lens, w.scale)
    assert_close(got, ref, "bf16", "q_len 1 vs single-token oracle")


def test_multi_block_permutation_is_bitwise_invisible():
    torch = torch_cuda()
    w = make_workload("gqa70b", seed=13, B=3, lens=("uniform", 100, 700), q_len=4)
    a = gpu_multi(torch, w)
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.num_blocks)            # new position of each physical block
    kp = np.empty_like(w.k_pool)
    vp = np.empty_like(w.v_pool)
    kp[perm] = w.k_pool
    vp[perm] = w.v_pool
    table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w.k_pool, w.v_pool, w.block_table = kp, vp, table
    b = gpu_multi(torch, w)
    assert np.array_equal(a, b)


def test_multi_full_size():
    """The benchmarked 70B-shaped verify batch (64 sequences, 4 new tokens each), every
    output row against the oracle."""
    torch = torch_cuda()
    w = make_workload("verify4")
    log(f"[multi] full size {w.name}: B={w.B} q_len={w.q_len} max_ctx={w.max_context_len}")
    got = gpu_multi(torch, w)
    assert_close(got, oracle_multi(w), "bf16", f"verify4, all {w.B} sequences")


def test_multi_weighted_ranges_do_not_depend_on_the_first_xcd():
    """The verify batch is large enough for XCD-weighted ranges, where a workgroup reads
    which XCD runs it.  The call is repeated after 1 to 7 extra one-workgroup launches of
    other work (which move the XCD that takes workgroup 0): every output must equal the
    first bit for bit, and the first matches the oracle on sampled sequences."""
    torch = torch_cuda()
    import paged_kv_cache_288_amd as pkv
    w = make_workload("verify4")
    q = bits_to_device(torch, w.q.reshape(w.B, w.q_len, w.Hq, w.d))
    kp, vp = bits_to_device(torch, w.k_pool), bits_to_device(torch, w.v_pool)
    bt = torch.from_numpy(w.block_table).to("cuda")
    cl = torch.from_numpy(w.context_lens).to("cuda")
    out = torch.empty((w.B, w.q_len, w.Hq, w.d_v), dtype=torch.float32, device="cuda")

    def call():
        pkv.paged_decode_attn_multi(out, q, kp, vp, bt, cl, w.scale, w.max_context_len)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    first = call()
    x = torch.zeros(64, device="cuda")
    for extra in range(1, 8):
        for _ in range(extra):
            x.add_(1.0)
        got = call()
        log(f"[multi] after {extra} extra launches: equal={np.array_equal(got, first)}")
        assert np.array_equal(got.view(np.uint32), first.view(np.uint32)), extra
    seqs = [0, 40]
    assert_close(first[seqs], oracle_multi(w, seqs), "bf16", "verify4 sampled sequences")


def test_multi_rejects_unsupported():
    torch = torch_cuda()
    import paged_kv_cache_288_amd as pkv
    w = make_workload("gqa70b", seed=1, B=2, lens=("uniform", 10, 50), q_len=9)   # 72 rows
    with pytest.raises(pkv.PkvError) as e:
        gpu_multi(torch, w)
    assert e.value.status == pkv.PKV_ERR_UNSUPPORTED


def test_multi_block_size_64():
    """64-token blocks (four 16-token tiles per block): the same histories re-blocked."""
    torch = torch_cuda()
    w = make_workload("gqa70b", seed=12, B=3, lens=("uniform", 5, 700), q_len=3)
    ref = oracle_multi(w)
    bs, L = 64, w.context_lens
    nb = int(sum(-(-int(x) // bs) for x in L)) + 2
    perm = np.random.default_rng(64).permutation(nb)
    kp = np.full((nb, w.Hkv, bs, w.d), 0x7FC0, np.uint16)
    vp = kp.copy()
    table = np.full((w.B, -(-int(L.max()) // bs)), -1, np.int32)
    cur = 0
    for b in range(w.B):
        n = -(-int(L[b]) // bs)
        table[b, :n] = perm[cur:cur + n]
        cur += n
        for t in range(int(L[b])):
            pb, off = w.block_table[b, t // 16], t % 16
            kp[table[b, t // bs], :, t % bs] = w.k_pool[pb, :, off]
            vp[table[b, t // bs], :, t % bs] = w.v_pool[pb, :, off]
    w.k_pool, w.v_pool, w.block_table, w.bs = kp, vp, table, bs
    assert_close(gpu_multi(torch, w), ref, "bf16", "multi block size 64")


def test_multi_linearity_in_v_is_exact():
    """V x 2 (exact in bf16 and in the fp16 the products use) doubles every output bit for
    bit: the weights do not depend on V and every rounding scales by the power of two."""
    torch = torch_cuda()
    w = make_workload("gqa70b", seed=14, B=3, lens=("uniform", 30, 600), q_len=4)
    w.v_pool, doubled = _double_v_exactly(w.v_pool)
    a = gpu_multi(torch, w)
    w.v_pool = doubled
    b = gpu_multi(torch, w)
    assert np.array_equal(b, 2 * a)


def _double_v_exactly(v_pool):
    """V with the N(0,1) draws below 2^-14 in magnitude zeroed (p.V widens V to fp16, exact
    only in fp16's normal range), and that V times 2 (exponent + 1, exact in bf16)."""
    v = v_pool.view(np.uint16).copy()
    exp = (v >> 7) & 0xFF
    v = np.where((exp != 0xFF) & (exp < 127 - 14), np.uint16(0), v).astype(np.uint16)
    exp = (v >> 7) & 0xFF
    ok = (exp != 0xFF) & (exp > 0) & (exp < 0xFE)
    return v, np.where(ok, v + np.uint16(1 << 7), v).astype(np.uint16)


def test_multi_lengths_above_max_context_len_are_truncated():
    """Lengths above max_context_len are clamped to it before the causal window of the new
    tokens is placed (query j sees the first min(L, max) - q_len + 1 + j tokens)."""
    torch = torch_cuda()
    import paged_kv_cache_288_amd as pkv
    w = make_workload("gqa70b", seed=15, B=4, lens=("uniform", 300, 1200), q_len=3)
    cap = 500
    q = bits_to_device(torch, w.q.reshape(w.B, w.q_len, w.Hq, w.d))
    kp, vp = bits_to_device(torch, w.k_pool), bits_to_device(torch, w.v_pool)
    bt, cl = torch.from_numpy(w.block_table).to("cuda"), torch.from_numpy(w.context_lens).to("cuda")
    out = torch.empty((w.B, w.q_len, w.Hq, w.d_v), dtype=torch.float32, device="cuda")
    pkv.paged_decode_attn_multi(out, q, kp, vp, bt, cl, w.scale, cap)
    torch.cuda.synchronize()
    w.context_lens = np.minimum(w.context_lens, cap).astype(np.int32)
    assert_close(out.cpu().numpy(), oracle_multi(w), "bf16", f"multi truncated at {cap}")
