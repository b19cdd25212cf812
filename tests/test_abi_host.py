"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before anything is enqueued."""

import ctypes
import os
import re

import numpy as np

import pytest

import paged_kv_cache_288_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.library_path()):
        from paged_kv_cache_288_amd import build
        build.build(verbose=False)
    return pkv.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    declared = header_functions()
    assert declared, "no declarations found"
    assert sorted(declared) == sorted(pkv.EXPORTED), "binding signatures out of sync with pkv.h"
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
    nm = os.popen(f"nm -D --defined-only {pkv.library_path()}").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", nm), f"{name} is not a defined text symbol"


def test_abi_version_and_status_strings(lib):
    ver = re.search(r"#define PKV_ABI_VERSION (\d+)", open(HEADER).read()).group(1)
    assert lib.pkv_abi_version() == int(ver)
    for code in range(-7, 1):
        assert lib.pkv_status_str(code)
    assert lib.pkv_status_str(0) == b"ok"


FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: every call below returns early
MIS = ctypes.c_void_p(0x1004)       # misaligned


def decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, bt=FAKE, cl=FAKE, B=2, Hq=8,
             Hkv=1, d=128, bs=16, nb=10, mb=4, ctx=64, scale=0.1, dt=pkv.PKV_BF16, ps=0,
             ws=None, wsb=0)
    a.update(kw)
    return lib.pkv_paged_decode_attn(a["out"], a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"],
                                     a["cl"], a["B"], a["Hq"], a["Hkv"], a["d"], a["bs"], a["nb"],
                                     a["mb"], a["ctx"], a["scale"], a["dt"], a["ps"], a["ws"],
                                     a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=0), -2), (dict(Hq=12, Hkv=8), -2), (dict(d=-1), -2), (dict(ctx=-5), -2),
    (dict(dt=7), -3),
    (dict(out=None), -1), (dict(bt=None), -1), (dict(dt=pkv.PKV_FP8_E4M3), -1),
    (dict(Hq=16, Hkv=1), -4), (dict(Hq=3, Hkv=1), -4), (dict(d=96), -4), (dict(bs=8), -4),
    (dict(d=64, dt=pkv.PKV_FP8_E4M3, ks=FAKE, vs=FAKE), -4),
    (dict(q=MIS), -5), (dict(k=MIS), -5),
    (dict(ctx=8192, ps=512, mb=512), -6),                       # split needs a workspace
    (dict(ctx=8192, ps=512, mb=512, ws=FAKE, wsb=100), -6),     # too small
    (dict(ctx=8192, ps=0, mb=512), -6),                         # balanced mode needs one too
    (dict(ps=24), -2), (dict(ps=8192), -2),
])
def test_decode_rejects_bad_arguments_before_launch(lib, kw, code):
    assert decode(lib, **kw) == code


def test_decode_empty_batch_is_a_noop(lib):
    assert decode(lib, B=0, out=None, q=None) == 0


def test_append_rejects_bad_arguments_before_launch(lib):
    f = lib.pkv_kv_append
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, 4, 10, 8, 128, 16, pkv.PKV_BF16, None)
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a5=-1) == -2
    assert call(a10=9) == -3
    assert call(a0=None) == -1
    assert call(a1=None) == -1           # v_pool without v_new
    assert call(a8=7) == -4              # 7 * 2 bytes is not a multiple of 16
    assert call(a2=MIS) == -5
    assert call(a5=0, a0=None, a2=None) == 0   # T = 0 is a no-op


def test_partition_and_workspace_sizing(lib):
    # explicit partition: 32768 tokens / 512 = 64 partitions of [m, l, o[128]] per head
    assert lib.pkv_decode_partition_size(4, 8, 32768, 512) == 512
    rows = 4 * 64 * 64
    r256 = lambda x: (x + 255) // 256 * 256
    assert lib.pkv_decode_workspace_bytes(4, 64, 8, 128, 32768, 512) == 2 * r256(rows * 4) + r256(rows * 128 * 4)
    # no split needed -> no workspace
    assert lib.pkv_decode_workspace_bytes(4, 64, 8, 128, 512, 512) == 0
    # partition_size 0 selects the balanced mode (reported as 0) up to 4096 sequences,
    # beyond which the library picks a partition (a power of two in [64, 1024])
    for B, H, ctx in [(64, 8, 8192), (2, 1, 256), (1, 8, 32768), (128, 8, 6144)]:
        assert lib.pkv_decode_partition_size(B, H, ctx, 0) == 0
    assert lib.pkv_decode_partition_size(5000, 8, 256, 0) in (64, 128, 256, 512, 1024)
    assert lib.pkv_decode_partition_size(1, 8, 100, 20) < 0


def _stream_chunks(B, Hkv, ctx, cus, waves_per_cu=8, max_tiles=480):
    """One chunk per wave (the workspace query sizes for the decode kernel's larger shape, 8
    waves per CU in 8-wave workgroups), at most the bound on the tiles, at most 480 tiles
    each, a whole number of workgroups on each of the 8 XCDs."""
    tmax = Hkv * B * ((ctx + 15) // 16)
    c = max(min(waves_per_cu * cus, tmax), -(-tmax // max_tiles))
    unit = 8 * waves_per_cu
    return max(unit, -(-c // unit) * unit)


def test_balanced_mode_workspace_size(lib):
    r256 = lambda x: (x + 255) // 256 * 256
    # this container has no GPU: the library assumes 256 CUs when the device query fails
    for B, Hq, Hkv, d, ctx in [(64, 64, 8, 128, 8192), (2, 4, 1, 64, 256), (4, 64, 8, 128, 32768),
                               (1, 8, 1, 128, 0), (3, 12, 3, 64, 700)]:
        C = _stream_chunks(B, Hkv, ctx, 256)
        if d == 128:  # FP8 calls run the register-tile MFMA kernel: up to 128 tiles per chunk
            tmax = Hkv * B * ((ctx + 15) // 16)
            c = max(min(8 * 256, tmax), -(-tmax // 128))
            C = max(C, max(32, -(-c // 32) * 32))
        rows = (C + Hkv * B) * (Hq // Hkv)
        want = 2 * r256(rows * 4) + r256(rows * d * 4) + r256((B + 1) * 4) + r256(Hkv * B * 8)
        assert lib.pkv_decode_workspace_bytes(B, Hq, Hkv, d, ctx, 0) == want


def chunk_of(t, T, C):
    return ((t + 1) * C - 1) // T


@pytest.mark.parametrize("lens,Hkv,C", [([7, 0, 300, 1, 16, 17], 2, 32), ([4096] * 3, 8, 64),
                                        ([1, 1, 1], 1, 32), ([5000, 33], 4, 2048)])
def test_balanced_mode_piece_slots(lens, Hkv, C):
    """Host mirror of the balanced mode's bookkeeping: every tile lies in exactly one chunk,
    pieces (chunk x segment) get unique slots below C + Hkv*B, and the non-empty chunks of
    the merge's chunk range for each segment are exactly the chunks that hold its tiles
    (with fewer tiles than chunks, empty chunks sit inside that range)."""
    B = len(lens)
    nt = [-(-L // 16) for L in lens]
    pre = [0]
    for n in nt:
        pre.append(pre[-1] + n)
    T = Hkv * pre[-1]
    seen_slots = set()
    owner = {}
    for ch in range(C):
        tb, te = T * ch // C, T * (ch + 1) // C
        assert te - tb <= max(1, -(-T // C))
        for t in range(tb, te):
            g, rem = divmod(t, pre[-1])
            b = max(i for i in range(B) if pre[i] <= rem)
            assert chunk_of(t, T, C) == ch
            owner.setdefault((g, b), set()).add(ch)
            seen_slots.add(ch + g * B + b)
    assert all(s < C + Hkv * B for s in seen_slots)
    assert len(seen_slots) == sum(len(v) for v in owner.values())
    for (g, b), chunks in owner.items():
        s0 = g * pre[-1] + pre[b]
        c0, c1 = chunk_of(s0, T, C), chunk_of(s0 + nt[b] - 1, T, C)
        live = {c for c in range(c0, c1 + 1) if T * c // C != T * (c + 1) // C}
        assert chunks == live   # the merge reads exactly these pieces


def _xcd_chunk_start(c, T, C, wtd, we=17, wo=15):
    if not wtd:
        return T * c // C
    h = (we + wo) // 2
    E = C // 8
    x, r = divmod(c, E)
    W = E * (we * ((x + 1) // 2) + wo * (x // 2)) + r * (wo if x & 1 else we)
    return T * W // (h * C)


def _xcd_chunk_of(t, T, C, wtd, we=17, wo=15):
    if not wtd:
        return chunk_of(t, T, C)
    h = (we + wo) // 2
    E = C // 8
    ws = ((t + 1) * h * C - 1) // T
    pair, rem = divmod(ws, 2 * h * E)
    if rem < we * E:
        return 2 * pair * E + rem // we
    return (2 * pair + 1) * E + (rem - we * E) // wo


def _xcd_weighted(T, C, min_tiles, max_tiles, we=17, wo=15):
    return T >= min_tiles * C and we * T <= (we + wo) // 2 * C * (max_tiles - 1)


@pytest.mark.parametrize("we,wo", [(17, 15), (33, 31)])
@pytest.mark.parametrize("T,C", [(128 * 64, 64), (70001, 64), (262144, 1024), (480 * 1024, 1024),
                                 (159952, 1024), (99991, 512), (152000, 2048), (2048 * 119, 2048)])
def test_xcd_weighted_chunks(T, C, we, wo):
    """Host mirror of the balanced kernels' XCD-weighted ranges (17:15 for single-token
    calls, 33:31 for the 32-row tiles of the verify pass): they tile [0, T) in order, the inverse used
    for the merge's bookkeeping names the range that holds each tile, chunks of even XCDs
    hold about we/wo of the odd ones' tiles, and whenever the weighting is switched on (512
    tiles per wave, chunk counts for 480) no range exceeds what a wave's tables hold."""
    for max_tiles in (512, 128):
        if _xcd_weighted(T, C, 64, max_tiles, we, wo):
            starts = [_xcd_chunk_start(c, T, C, True, we, wo) for c in range(C + 1)]
            assert max(b - a for a, b in zip(starts, starts[1:])) <= max_tiles
    starts = [_xcd_chunk_start(c, T, C, True, we, wo) for c in range(C + 1)]
    assert starts[0] == 0 and starts[-1] == T
    assert all(b > a for a, b in zip(starts, starts[1:]))   # every chunk non-empty
    if T <= 480 * C:   # the chunk count keeps T within this bound
        assert max(b - a for a, b in zip(starts, starts[1:])) <= 512
    E = C // 8
    size = [starts[c + 1] - starts[c] for c in range(C)]
    even = sum(size[c] for c in range(C) if (c // E) % 2 == 0)
    assert abs(even / (T - even) - we / wo) < 0.01
    step = max(1, T // 20000)
    for t in list(range(0, T, step)) + [s for s in starts[1:-1]] + [s - 1 for s in starts[1:]]:
        c = _xcd_chunk_of(t, T, C, True, we, wo)
        assert starts[c] <= t < starts[c + 1], (t, c)


@pytest.mark.parametrize("groups", [1, 2, 4])
def test_xcd_parity_assignment(groups):
    """Host mirror of how a balanced kernel's workgroup picks its eighth of the chunks when
    the ranges are weighted: eighth = (bid mod 8) xor f, f = (XCD id xor bid) & 1.  For every
    XCD r that may take workgroup 0 (workgroup i then runs on XCD (i + r) mod 8), each chunk
    goes to exactly one wave, and every eighth with the heavier (even) weight runs on an even
    XCD.  With the parity taken from bid alone, an odd r puts every heavy eighth on an odd
    XCD."""
    WPG = 4
    C = 8 * WPG * groups
    for r in range(8):
        owner = {}
        for bid in range(C // WPG):
            xcd = (bid + r) % 8
            eighth = (bid % 8) ^ ((xcd ^ bid) & 1)
            assert eighth % 2 == xcd % 2
            for w in range(WPG):
                ch = eighth * (C // 8) + (bid // 8) * WPG + w
                assert ch not in owner
                owner[ch] = xcd
        assert sorted(owner) == list(range(C))
        blind = [((bid + r) % 8) % 2 == (bid % 8) % 2 for bid in range(8)]
        assert all(blind) == (r % 2 == 0)


def test_mla_rejects_bad_arguments_before_launch(lib):
    f = lib.pkv_paged_decode_attn_mla
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 128, 576, 512, 64, 10, 4, 200, 0.1, 0, None, 0, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a6=0) == -2
    assert call(a8=600) == -2            # d_v > d_qk
    assert call(a0=None) == -1
    assert call(a7=512, a8=256) == -4
    assert call(a9=32) == -4
    assert call(a6=100) == -4
    assert call(a14=96) == -2            # partition not a multiple of the block size
    assert call(a1=MIS) == -5
    assert call(a12=8192, a14=64) == -6  # split without a workspace


def test_binding_rejects_pools_that_do_not_match_kv_dtype():
    """The library trusts the pool geometry it is given, so a pool whose element size
    differs from kv_dtype's would be addressed past its end; the binding refuses such calls
    before any launch (CPU tensors: nothing reaches the library)."""
    torch = pytest.importorskip("torch")
    q = torch.zeros((2, 8, 128), dtype=torch.int16)
    out = torch.zeros((2, 8, 128), dtype=torch.float32)
    bt = torch.zeros((2, 4), dtype=torch.int32)
    cl = torch.zeros((2,), dtype=torch.int32)
    fp8_pool = torch.zeros((10, 1, 16, 128), dtype=torch.uint8)
    bf16_pool = torch.zeros((10, 1, 16, 128), dtype=torch.int16)
    with pytest.raises(ValueError, match="1-byte elements"):
        pkv.paged_decode_attn(out, q, fp8_pool, fp8_pool, bt, cl, 0.1, 64)        # FP8 pool as bf16
    with pytest.raises(ValueError, match="2-byte elements"):
        pkv.paged_decode_attn(out, q, bf16_pool, bf16_pool, bt, cl, 0.1, 64, kv_dtype="fp8")
    with pytest.raises(ValueError, match="differs"):
        pkv.paged_decode_attn(out, q, bf16_pool, bf16_pool[:5], bt, cl, 0.1, 64)
    with pytest.raises(ValueError, match="dimensions"):
        pkv.paged_decode_attn_mla(out, q, bf16_pool, bt, cl, 0.1, 64)            # latent pools are 3-D
    with pytest.raises(ValueError, match="1-byte elements"):
        pkv.paged_decode_attn_multi(out, q[:, None], fp8_pool, fp8_pool, bt, cl, 0.1, 64)
    with pytest.raises(ValueError, match="2-byte elements"):
        pkv.kv_append_fp8(bf16_pool, bf16_pool, q, q, None, None, cl.long())


def test_binding_refuses_to_run_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(pkv, "_LIB", None)
    monkeypatch.setattr(pkv, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        pkv.load_library()


def _mla_chunks(B, Hq, ctx, cus):
    hg = Hq // (64 if Hq % 64 == 0 else 32)   # head groups of 64 (or 32) heads
    smax = B * -(-ctx // 32)                   # bound on the 32-token stages
    c = max(min(-(-cus // hg), smax), -(-smax // 128))
    return max(8, -(-c // 8) * 8)


def test_mla_balanced_workspace_size(lib):
    """Latent balanced mode (partition_size 0, Hq a multiple of 32): pieces (chunks + B) x Hq
    rows of m, l and o[512], the stage prefix and per-sequence chunk ranges; 256 CUs assumed
    without a GPU."""
    r256 = lambda x: (x + 255) // 256 * 256
    for B, Hq, ctx in [(32, 128, 8192), (1, 32, 8192), (200, 64, 100), (5, 96, 1500),
                       (4, 128, 131072), (3, 128, 700), (2, 64, 0)]:
        C = _mla_chunks(B, Hq, ctx, 256)
        assert B * -(-ctx // 32) <= 128 * C            # no range exceeds 128 stages
        rows = (C + B) * Hq
        want = 2 * r256(rows * 4) + r256(rows * 512 * 4) + r256((B + 1) * 4) + r256(B * 8)
        assert lib.pkv_mla_workspace_bytes(B, Hq, 512, ctx, 0) == want
    # Hq not a multiple of 32 (and explicit partitions) use the partitioned kernel
    assert lib.pkv_mla_workspace_bytes(2, 48, 512, 8192, 0) > 0
    assert lib.pkv_mla_workspace_bytes(2, 128, 512, 512, 1024) == 0


def _mla_padded_split(ns_b, C, pad, max_stages=128):
    """Mirror of the latent kernel's chunking: `pad` virtual stages before every sequence
    (when the total allows), chunk c takes the real stages inside [Tv c / C, Tv (c+1) / C);
    returns the pad used, each chunk's real [tb, te) and each sequence's (first chunk, count)
    as the kernel writes them for the merge."""
    B, T = len(ns_b), int(sum(ns_b))
    pre = [0]
    for n in ns_b:
        pre.append(pre[-1] + int(n))
    pv = pad if (T >= C and T + pad * B <= (max_stages - 1) * C) else 0
    tv = T + pv * B

    def real_before_sum(v):            # the register-scan form (sequences up to 64)
        return v - sum(min(max(v - (pre[b] + pv * b), 0), pv) for b in range(B))

    def real_before_search(v):         # the binary-search form (more sequences)
        if pv == 0:
            return v
        lo, hi = 0, B - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if pre[mid] + pv * mid <= v:
                lo = mid
            else:
                hi = mid - 1
        return v - (pv * lo + min(v - (pre[lo] + pv * lo), pv))

    chunks = []
    for c in range(C):
        a, b = tv * c // C, tv * (c + 1) // C
        tb, te = real_before_sum(a), real_before_sum(b)
        assert (tb, te) == (real_before_search(a), real_before_search(b))
        chunks.append((tb, te))
    chunk_of = lambda t: ((t + 1) * C - 1) // tv
    segs = []
    for b in range(B):
        if ns_b[b] == 0:
            segs.append((0, 0))
            continue
        first = pre[b] + pv * (b + 1)
        c0 = chunk_of(first)
        segs.append((c0, chunk_of(first + ns_b[b] - 1) - c0 + 1))
    return pv, pre, chunks, segs


def test_latent_chunks_with_piece_padding():
    """Latent chunking with virtual stages before each sequence: the chunks' real ranges
    tile the stages in order, every chunk in a sequence's merge range holds stages of it
    (and no other chunk does), and no chunk exceeds 128 stages."""
    rng = np.random.default_rng(5)
    cases = [([64, 116, 236, 220, 108, 175] * 5 + [100, 90], 128, 4),   # latent batch-like
             ([10] * 200, 128, 4), ([0, 0, 50, 0, 300], 16, 4), ([1] * 300, 8, 4),
             ([128 * 8 - 10], 8, 4), ([5, 5], 64, 4)]
    for _ in range(60):
        B = int(rng.integers(1, 90))
        ns_b = [int(x) for x in rng.integers(0, 260, size=B)]
        C = int(rng.choice([8, 16, 64, 128, 256]))
        cases.append((ns_b, C, int(rng.integers(1, 6))))
    for ns_b, C, pad in cases:
        T = sum(ns_b)
        if T > 127 * C:
            continue
        pv, pre, chunks, segs = _mla_padded_split(ns_b, C, pad)
        assert chunks[0][0] == 0 and chunks[-1][1] == T
        for c in range(C - 1):
            assert chunks[c][1] == chunks[c + 1][0]
        if pv:
            assert T >= C and max(te - tb for tb, te in chunks) <= 128
        for b, (c0, n) in enumerate(segs):
            lo, hi = pre[b], pre[b + 1]
            holding = [c for c, (tb, te) in enumerate(chunks) if max(tb, lo) < min(te, hi)]
            if T >= C:
                assert holding == list(range(c0, c0 + n)), (ns_b, C, pad, b)
            else:  # fewer stages than chunks (never padded): the merge skips empty chunks
                assert pv == 0 and set(holding) <= set(range(c0, c0 + n))


def test_graph_calls_reject_null_arguments(lib):
    """The graph entry points check their pointers before any HIP call."""
    assert lib.pkv_graph_begin(None) == pkv.PKV_ERR_NULL
    handle = ctypes.c_void_p()
    assert lib.pkv_graph_end(None, ctypes.byref(handle)) == pkv.PKV_ERR_NULL
    assert lib.pkv_graph_end(FAKE, None) == pkv.PKV_ERR_NULL
    assert lib.pkv_graph_launch(None, None) == pkv.PKV_ERR_NULL
    assert lib.pkv_graph_destroy(None) == pkv.PKV_OK


def test_graph_buckets():
    from paged_kv_cache_288_amd.graph import bucket_batch, bucket_context
    assert [bucket_batch(b) for b in (1, 2, 3, 4, 5, 64, 65)] == [1, 2, 4, 4, 8, 64, 128]
    assert bucket_context(1, 16) == 256 and bucket_context(257, 16) == 512
    assert bucket_context(8192, 16) == 8192 and bucket_context(8133, 64) == 8192
    with pytest.raises(ValueError):
        bucket_batch(0)


def test_quantizing_append_and_block_copy_reject_bad_arguments(lib):
    f = lib.pkv_kv_append_fp8
    #          k_pool v_pool k_new v_new ks  vs  slots T  nb  H  d   bs  stream
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 2, 64, 16, None) == pkv.PKV_OK
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 4, 2, 64, 16, None) == pkv.PKV_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 3, 4, 2, 64, 16, None) == pkv.PKV_ERR_NULL
    assert f(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 3, 4, 2, 64, 16, None) == pkv.PKV_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 3, 4, 2, 64, 16, None) == pkv.PKV_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 4, 2, 40, 16, None) == \
        pkv.PKV_ERR_UNSUPPORTED
    assert f(MIS, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 4, 2, 64, 16, None) == pkv.PKV_ERR_ALIGN
    g = lib.pkv_kv_copy_blocks
    #          k_pool v_pool src dst n nb H d bs dtype stream
    assert g(FAKE, FAKE, FAKE, FAKE, 0, 4, 2, 64, 16, pkv.PKV_BF16, None) == pkv.PKV_OK
    assert g(FAKE, FAKE, FAKE, FAKE, 2, 4, 2, 64, 16, 9, None) == pkv.PKV_ERR_DTYPE
    assert g(FAKE, FAKE, None, FAKE, 2, 4, 2, 64, 16, pkv.PKV_BF16, None) == pkv.PKV_ERR_NULL
    assert g(FAKE, FAKE, FAKE, FAKE, -1, 4, 2, 64, 16, pkv.PKV_BF16, None) == pkv.PKV_ERR_SHAPE
    assert g(FAKE, MIS, FAKE, FAKE, 2, 4, 2, 64, 16, pkv.PKV_BF16, None) == pkv.PKV_ERR_ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, 2, 4, 2, 4, 16, pkv.PKV_FP8_E4M3, None) == \
        pkv.PKV_ERR_UNSUPPORTED


def test_multi_rejects_bad_arguments_before_launch(lib):
    f = lib.pkv_paged_decode_attn_multi
    # out q k v ks vs bt cl B q_len Hq Hkv d bs nb mb ctx scale dtype ws wsb stream
    base = [FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 2, 4, 64, 8, 128, 16, 10, 4, 64,
            0.1, pkv.PKV_BF16, None, 0, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a9=0) == -2              # q_len
    assert call(a10=60) == -2            # Hq not a multiple of Hkv
    assert call(a18=9) == -3
    assert call(a8=0) == 0               # empty batch
    assert call(a0=None) == -1
    assert call(a18=pkv.PKV_FP8_E4M3) == -1   # FP8 needs its scales
    assert call(a9=9) == -4              # 72 rows per KV head
    assert call(a10=48) == -4            # group of 6 query heads
    assert call(a12=96) == -4
    assert call(a13=8) == -4
    assert call(a1=MIS) == -5
    assert call() == -6                  # needs a workspace
    assert call(a19=FAKE, a20=64) == -6
    assert call(a18=pkv.PKV_FP8_E4M3, a4=FAKE, a5=FAKE) == -6


def test_multi_workspace_size(lib):
    """Balanced layout with q_len * G rows per piece slot; 256 CUs assumed without a GPU."""
    r256 = lambda x: (x + 255) // 256 * 256
    for B, q_len, Hq, Hkv, d, ctx in [(64, 4, 64, 8, 128, 8192), (2, 8, 4, 1, 64, 256),
                                      (1, 1, 8, 8, 128, 20000), (3, 16, 32, 8, 128, 900)]:
        tmax = Hkv * B * -(-ctx // 16)
        rows = (Hq // Hkv) * q_len
        waves = 4 if d * -(-rows // 16) > 256 else 8      # resident waves per CU
        C = max(min(waves * 256, tmax), -(-tmax // 128))
        C = max(32, -(-C // 32) * 32)
        rows = (C + Hkv * B) * (Hq // Hkv) * q_len
        want = 2 * r256(rows * 4) + r256(rows * d * 4) + r256((B + 1) * 4) + r256(Hkv * B * 8)
        assert lib.pkv_multi_workspace_bytes(B, q_len, Hq, Hkv, d, ctx) == want
    assert lib.pkv_multi_workspace_bytes(2, 9, 64, 8, 128, 100) == 0     # 72 rows
    assert lib.pkv_multi_workspace_bytes(2, 0, 64, 8, 128, 100) == 0


def test_cascade_rejects_bad_arguments_before_launch(lib):
    f = lib.pkv_paged_decode_attn_cascade
    # out q k v ks vs prefix plen tail_t tail_l B Hq Hkv d bs nb mtb mtl scale dtype ws wsb stream
    base = [FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 64, FAKE, FAKE, 4, 32, 8, 128, 16, 100,
            8, 128, 0.1, pkv.PKV_BF16, None, 0, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a7=40) == -2               # prefix not whole blocks
    assert call(a11=30) == -2              # Hq not a multiple of Hkv
    assert call(a16=0) == -2
    assert call(a19=5) == -3
    assert call(a10=0) == 0
    assert call(a6=None) == -1             # prefix_len > 0 needs its blocks
    assert call(a19=pkv.PKV_FP8_E4M3) == -1
    assert call(a11=128) == -4             # G = 16
    assert call(a13=64, a19=pkv.PKV_FP8_E4M3, a4=FAKE, a5=FAKE) == -4
    assert call(a1=MIS) == -5
    assert call() == -6
    assert call(a6=None, a7=0) == -6       # no prefix is fine, the workspace is still needed


def test_cascade_workspace_size(lib):
    """Tail pass (balanced, rows of G) and prefix pass (multi-token, 32 / G sequences per
    group, 32 rows); 256 CUs assumed without a GPU."""
    r256 = lambda x: (x + 255) // 256 * 256
    def chunks(tiles, waves):
        c = max(min(waves * 256, tiles), -(-tiles // 128))
        return max(32, -(-c // 32) * 32)
    for B, Hq, Hkv, d, plen, tmax in [(128, 32, 8, 128, 4096, 2048), (37, 8, 8, 128, 320, 401),
                                      (9, 4, 1, 64, 0, 90), (5, 64, 8, 128, 512, 0)]:
        G = Hq // Hkv
        # with a prefix both passes share one launch: 6 + 2 waves per CU
        ct = chunks(Hkv * B * -(-tmax // 16), 6 if plen else 8)
        rows = (ct + Hkv * B) * G
        want = 2 * r256(rows * 4) + r256(rows * d * 4) + r256((B + 1) * 4) + r256(Hkv * B * 8)
        if plen:
            J = 32 // G
            pB = -(-B // J)
            cp = chunks(Hkv * pB * -(-plen // 16), 2)
            prow = (cp + Hkv * pB) * 32
            want += 2 * r256(prow * 4) + r256(prow * d * 4) + r256((pB + 1) * 4) + r256(Hkv * pB * 8)
        assert lib.pkv_cascade_workspace_bytes(B, Hq, Hkv, d, plen, tmax) == want, (B, Hq)


def test_validate_rejects_bad_arguments_before_launch(lib):
    f = lib.pkv_validate
    # counts table lens B mb nb bs max_ctx slots T v_pool Hkv d d_v stream
    base = [FAKE, FAKE, FAKE, 4, 8, 100, 16, 128, FAKE, 10, None, 0, 0, 0, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a3=-1) == -2
    assert call(a5=0) == -2
    assert call(a6=0) == -2
    assert call(a0=None) == -1
    assert call(a1=None) == -1
    assert call(a8=None) == -1           # T > 0 needs slots
    assert call(a0=ctypes.c_void_p(0x1002)) == -5   # counts must be 4-byte aligned
    assert call(a8=ctypes.c_void_p(0x1004)) == -5   # slots must be 8-byte aligned
    assert call(a10=FAKE, a11=0, a12=128, a13=128) == -2   # a V pool needs its shape
    assert call(a10=FAKE, a11=8, a12=128, a13=129) == -2   # d_v <= d
    assert call(a10=ctypes.c_void_p(0x1001), a11=8, a12=128, a13=128) == -5

def test_noalloc_rejects_what_exceeds_its_scratch(lib):
    """The allocation-free decode call refuses, before any GPU work, an argument set whose
    workspace would exceed the library's scratch (4096 sequences of 32K tokens, 8 KV heads)."""
    scratch = int(re.search(r"#define PKV_NOALLOC_SCRATCH_BYTES \((\d+) << (\d+)\)",
                            open(HEADER).read()).expand(r"\1")) << 20
    assert lib.pkv_decode_workspace_bytes(4096, 64, 8, 128, 32768, 0) > scratch
    st = lib.pkv_paged_decode_attn_noalloc(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 4096,
                                           64, 8, 128, 16, 10, 2048, 32768, 0.1, pkv.PKV_BF16,
                                           0, None)
    assert st == pkv.PKV_ERR_WORKSPACE
    assert lib.pkv_paged_decode_attn_noalloc(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 4,
                                             64, 12, 128, 16, 10, 64, 1024, 0.1, pkv.PKV_BF16,
                                             0, None) == pkv.PKV_ERR_SHAPE
