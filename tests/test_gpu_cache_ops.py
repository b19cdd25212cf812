"""Cache-management operations on the GPU against the oracle: the quantizing append
(bf16 rows -> FP8 E4M3 codes, bit-exact), the block copy behind copy-on-write (bit-exact),
an FP8 cache built by the quantizing append and then decoded, and a copy-on-write fork
driven by the host allocator."""

import numpy as np
import pytest

import oracle
from oracle import cache_management as cm
from gpu_common import assert_close, log, torch_cuda

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def test_quantizing_append_bit_exact():
    torch = torch_cuda()
    import paged_kv_cache_288_amd as pkv
    rng = np.random.default_rng(11)
    nb, H, bs, d, T = 12, 3, 16, 256, 6
    table = oracle.fp8_e4m3fn_table()
    # head 0 of token 0: every midpoint between neighbouring positive codes (exact ties with
    # scale 1), then their negatives; the other rows random with special values
    mids = [(table[c] + table[c + 1]) / 2 for c in range(126)]
    x = rng.standard_normal((T, H, d)).astype(np.float32) * np.float32(30)
    x[0, 0, :126] = mids
    x[0, 0, 126:252] = -np.array(mids)
    x[1, 1, :12] = [np.nan, np.inf, -np.inf, 1e30, -1e30, 0.0, -0.0, 1e-40, -1e-40, 448.0,
                    464.0, 2.0 ** -10]
    k_bits = _bf16_bits(x)
    v_bits = _bf16_bits(rng.standard_normal((T, H, d)).astype(np.float32) * 3)
    k_scale = np.array([1.0, 0.37, 0.0019], np.float32)
    v_scale = np.array([0.25, 1.9, 7.5], np.float32)
    slots = np.array([5, 17, -1, 100, 191, 40], np.int64)
    kp0 = np.full((nb, H, bs, d), 0x55, np.uint8)
    vp0 = np.full((nb, H, bs, d), 0xAA, np.uint8)
    kp, vp = _dev(torch, kp0), _dev(torch, vp0)
    pkv.kv_append_fp8(kp, vp, _dev(torch, k_bits), _dev(torch, v_bits), _dev(torch, k_scale),
                      _dev(torch, v_scale), _dev(torch, slots))
    torch.cuda.synchronize()
    want_k = cm.kv_append_fp8(kp0, k_bits, k_scale, slots, bs)
    want_v = cm.kv_append_fp8(vp0, v_bits, v_scale, slots, bs)
    got_k, got_v = kp.cpu().numpy(), vp.cpu().numpy()
    bad = np.argwhere(got_k != want_k)
    assert bad.size == 0, f"K codes differ at {bad[:5].tolist()}"
    assert np.array_equal(got_v, want_v)
    # ties went to the even code
    assert got_k[0, 0, 5, :126].tolist() == [c if c % 2 == 0 else c + 1 for c in range(126)]
    # slots outside the pool are skipped: the whole pool else is untouched
    pkv.kv_append_fp8(kp, vp, _dev(torch, k_bits), _dev(torch, v_bits), _dev(torch, k_scale),
                      _dev(torch, v_scale), _dev(torch, np.array([-5, nb * bs, 10**9, -1,
                                                                  nb * bs + 3, -2], np.int64)))
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), want_k) and np.array_equal(vp.cpu().numpy(), want_v)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "mla"])
def test_block_copy_bit_exact(kind):
    torch = torch_cuda()
    import paged_kv_cache_288_amd as pkv
    rng = np.random.default_rng(12)
    if kind == "mla":
        shape, dt, v = (9, 64, 576), np.uint16, False
    else:
        shape, dt, v = ((10, 4, 16, 128), np.uint16 if kind == "bf16" else np.uint8, True)
    kp0 = rng.integers(0, np.iinfo(dt).max, shape, dtype=dt)
    vp0 = rng.integers(0, np.iinfo(dt).max, shape, dtype=dt) if v else None
    src = np.array([1, 3, 99, 0, -1], np.int32)
    dst = np.array([4, 7, 2, 8, 6], np.int32)
    kp = _dev(torch, kp0)
    vp = _dev(torch, vp0) if v else None
    pkv.kv_copy_blocks(kp, vp, _dev(torch, src), _dev(torch, dst),
                       kv_dtype="fp8" if kind == "fp8" else "bf16")
    torch.cuda.synchronize()
    got = kp.cpu().numpy().view(dt)
    assert np.array_equal(got, cm.copy_blocks(kp0, src, dst))
    if v:
        assert np.array_equal(vp.cpu().numpy().view(dt), cm.copy_blocks(vp0, src, dst))


def test_fp8_cache_from_quantizing_append_decodes_like_the_oracle():
    """Every cached token of a small GQA batch goes through the quantizing append; the
    decode of the resulting FP8 cache matches the oracle on the oracle's own codes."""
    torch = torch_cuda()
    import paged_kv_cache_288_amd as pkv
    rng = np.random.default_rng(13)
    B, Hq, H, d, bs = 3, 8, 2, 128, 16
    lens = np.array([37, 160, 91], np.int32)
    nblk = -(-lens // bs)
    nb = int(nblk.sum()) + 3
    perm = rng.permutation(nb)
    table = np.full((B, int(nblk.max())), -1, np.int32)
    slots = []
    at = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += nblk[b]
        for p in range(lens[b]):
            slots.append(int(table[b, p // bs]) * bs + p % bs)
    T = len(slots)
    k = rng.standard_normal((T, H, d)).astype(np.float32) * 2
    vv = rng.standard_normal((T, H, d)).astype(np.float32)
    k_bits, v_bits = _bf16_bits(k), _bf16_bits(vv)
    kf = (k_bits.astype(np.uint32) << 16).view(np.float32)
    vf = (v_bits.astype(np.uint32) << 16).view(np.float32)
    k_scale = (np.abs(kf).max(axis=(0, 2)) / 448).astype(np.float32)
    v_scale = (np.abs(vf).max(axis=(0, 2)) / 448).astype(np.float32)
    slots = np.array(slots, np.int64)
    kp0 = np.zeros((nb, H, bs, d), np.uint8)
    kp, vp = _dev(torch, kp0), _dev(torch, kp0)
    ks, vs = _dev(torch, k_scale), _dev(torch, v_scale)
    pkv.kv_append_fp8(kp, vp, _dev(torch, k_bits), _dev(torch, v_bits), ks, vs, _dev(torch, slots))
    q_bits = _bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32))
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    scale = 1 / np.sqrt(d)
    pkv.paged_decode_attn(out, _dev(torch, q_bits), kp, vp, _dev(torch, table), _dev(torch, lens),
                          scale, int(lens.max()), kv_dtype="fp8", k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    want_kp = cm.kv_append_fp8(kp0, k_bits, k_scale, slots, bs)
    want_vp = cm.kv_append_fp8(kp0, v_bits, v_scale, slots, bs)
    assert np.array_equal(kp.cpu().numpy(), want_kp) and np.array_equal(vp.cpu().numpy(), want_vp)
    K = oracle.decode_kv_bits(want_kp, "fp8", k_scale)
    V = oracle.decode_kv_bits(want_vp, "fp8", v_scale)
    ref = oracle.paged_decode_attention(oracle.bf16_bits_to_f64(q_bits), K, V, table, lens, scale)
    assert_close(out.cpu().numpy(), ref, "fp8", "decode of a quantized-append cache")


def test_copy_on_write_fork_keeps_both_histories():
    """A sequence forks (beam search): both branches share its blocks, the branch that
    writes into the shared partial block gets a copy first, then each appends its own
    rows; each branch must decode to its own history."""
    torch = torch_cuda()
    import paged_kv_cache_288_amd as pkv
    from paged_kv_cache_288_amd.cache import BlockAllocator
    rng = np.random.default_rng(14)
    nb, H, bs, d, Hq = 16, 2, 16, 64, 4
    alloc = BlockAllocator(nb, bs)
    kp = torch.zeros((nb, H, bs, d), dtype=torch.int16, device="cuda")
    vp = torch.zeros_like(kp)
    hist = {}

    def append(name, blocks, length, n):
        slots, copies = alloc.slots_for_append(blocks, length, n)
        if copies:
            src = torch.tensor([c[0] for c in copies], dtype=torch.int32, device="cuda")
            dst = torch.tensor([c[1] for c in copies], dtype=torch.int32, device="cuda")
            pkv.kv_copy_blocks(kp, vp, src, dst)
        k = _bf16_bits(rng.standard_normal((n, H, d)))
        v = _bf16_bits(rng.standard_normal((n, H, d)))
        pkv.kv_append(kp, vp, _dev(torch, k), _dev(torch, v),
                      torch.tensor(slots, dtype=torch.int64, device="cuda"))
        hk, hv = hist.get(name, (np.zeros((0, H, d), np.uint16),) * 2)
        hist[name] = (np.concatenate([hk, k]), np.concatenate([hv, v]))
        return copies

    a_blocks = []
    append("a", a_blocks, 0, 21)                       # blocks 0, 1 (block 1: 5 rows)
    b_blocks = [alloc.share(b) for b in a_blocks]
    hist["b"] = hist["a"]
    assert append("b", b_blocks, 21, 4) == [(a_blocks[1], b_blocks[1])]
    assert append("a", a_blocks, 21, 30) == []         # a owns block 1 alone now
    log(f"[cow] a blocks {a_blocks}, b blocks {b_blocks}")
    lens = np.array([51, 25], np.int32)
    table = np.full((2, 4), -1, np.int32)
    table[0, :len(a_blocks)] = a_blocks
    table[1, :len(b_blocks)] = b_blocks
    q = _bf16_bits(rng.standard_normal((2, Hq, d)))
    out = torch.empty((2, Hq, d), dtype=torch.float32, device="cuda")
    pkv.paged_decode_attn(out, _dev(torch, q), kp, vp, _dev(torch, table), _dev(torch, lens),
                          0.125, 64)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i, name in enumerate(["a", "b"]):
        # the branch's own history, laid out contiguously for the oracle
        hk, hv = hist[name]
        L = hk.shape[0]
        n = -(-L // bs)
        pk = np.zeros((n * bs, H, d), np.uint16)
        pv = np.zeros((n * bs, H, d), np.uint16)
        pk[:L], pv[:L] = hk, hv
        K = oracle.bf16_bits_to_f64(pk.reshape(n, bs, H, d).transpose(0, 2, 1, 3))
        V = oracle.bf16_bits_to_f64(pv.reshape(n, bs, H, d).transpose(0, 2, 1, 3))
        ref = oracle.paged_decode_attention(oracle.bf16_bits_to_f64(q[i:i + 1]), K, V,
                                            np.arange(n)[None, :], np.array([L]), 0.125)
        assert L == lens[i]
        assert_close(got[i:i + 1], ref, "bf16", f"branch {name}")
