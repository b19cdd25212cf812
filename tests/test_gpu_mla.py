"""GPU parity of pkv_paged_decode_attn_mla (latent decode on MFMA) against the fp64 oracle."""

import numpy as np
import pytest

from gpu_common import assert_close, gpu_decode, log, make_workload, oracle_decode, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ps", [0, 64, 128, 256, 4096])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mla_matches_oracle_reduced(seed, ps):
    torch = torch_cuda()
    w = make_workload("mla", seed=seed, B=3, lens=("uniform", 1, 700))
    log(f"[mla] seed={seed} partition={ps} lens={w.context_lens.tolist()}")
    assert_close(gpu_decode(torch, w, partition_size=ps), oracle_decode(w), "bf16",
                 f"mla seed {seed} partition {ps}")


@pytest.mark.parametrize("hq", [16, 48, 64, 128])
def test_mla_head_counts(hq):
    torch = torch_cuda()
    w = make_workload("mla", seed=4, B=2, lens=("uniform", 30, 400), heads=(hq, 1))
    log(f"[mla] Hq={hq} lens={w.context_lens.tolist()}")
    assert_close(gpu_decode(torch, w), oracle_decode(w), "bf16", f"mla Hq {hq}")


def test_mla_full_size():
    """The 32-sequence latent batch as benchmarked, every output row against the oracle."""
    torch = torch_cuda()
    w = make_workload("mla")
    log(f"[mla] full size: B={w.B} max_ctx={w.max_context_len}")
    got = gpu_decode(torch, w)
    assert_close(got, oracle_decode(w), "bf16", f"mla full size, all {w.B} sequences")


def test_mla_single_token_returns_latent_exactly():
    torch = torch_cuda()
    w = make_workload("mla", seed=5, B=3, lens=("fixed", [1, 1, 1]))
    got = gpu_decode(torch, w)
    assert np.array_equal(got.astype(np.float64), oracle_decode(w))


def test_mla_block_permutation_is_bitwise_invisible():
    torch = torch_cuda()
    w = make_workload("mla", seed=6, B=3, lens=("uniform", 100, 900))
    base = gpu_decode(torch, w, partition_size=256)
    p = np.random.default_rng(1).permutation(w.num_blocks)
    kp = np.empty_like(w.k_pool)
    kp[p] = w.k_pool
    w.k_pool = kp
    w.block_table = np.where(w.block_table >= 0, p[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    assert np.array_equal(gpu_decode(torch, w, partition_size=256), base)


def test_mla_empty_sequence_gives_zero():
    torch = torch_cuda()
    w = make_workload("mla", seed=7, B=3, lens=("uniform", 100, 500))
    w.context_lens[2] = 0
    for ps in (0, 4096):
        got = gpu_decode(torch, w, partition_size=ps)
        assert (got[2] == 0).all()
        assert_close(got, oracle_decode(w), "bf16", f"mla empty sequence, partition {ps}")


# ---- balanced mode (partition_size 0, Hq a multiple of 32): stage ranges cut across
# sequences, pieces merged per sequence

def test_mla_balanced_many_short_sequences():
    """Many pieces per workgroup range: short contexts, partial 32-token stages, empties."""
    torch = torch_cuda()
    w = make_workload("mla", seed=11, B=200, lens=("uniform", 0, 100), heads=(64, 1))
    log(f"[mla] balanced B=200 lens<=100 (zeros: {int((w.context_lens == 0).sum())})")
    got = gpu_decode(torch, w, partition_size=0)
    assert_close(got, oracle_decode(w), "bf16", "mla balanced, 200 short sequences")


def test_mla_balanced_one_long_sequence():
    """One sequence spread over every workgroup range (one piece each)."""
    torch = torch_cuda()
    w = make_workload("mla", seed=12, B=1, lens=("fixed", [8192]))
    log("[mla] balanced B=1 L=8192")
    got = gpu_decode(torch, w, partition_size=0)
    assert_close(got, oracle_decode(w), "bf16", "mla balanced, one 8192-token sequence")


@pytest.mark.parametrize("B", [64, 65])
def test_mla_balanced_batch_scan_boundary(B):
    """64 sequences are the most the 64-head kernel scans in registers; 65 take the
    workgroup-wide scan.  Both must give the same stage map and merge bookkeeping."""
    torch = torch_cuda()
    w = make_workload("mla", seed=16 + B, B=B, lens=("uniform", 0, 300))
    w.context_lens[B - 1] = 0
    log(f"[mla] balanced B={B} lens<=300 (zeros: {int((w.context_lens == 0).sum())})")
    assert_close(gpu_decode(torch, w, partition_size=0), oracle_decode(w), "bf16",
                 f"mla balanced B={B}")


@pytest.mark.parametrize("hq", [32, 96])
def test_mla_balanced_head_groups(hq):
    torch = torch_cuda()
    w = make_workload("mla", seed=13, B=5, lens=("uniform", 1, 1500), heads=(hq, 1))
    log(f"[mla] balanced Hq={hq} lens={w.context_lens.tolist()}")
    assert_close(gpu_decode(torch, w, partition_size=0), oracle_decode(w), "bf16",
                 f"mla balanced Hq {hq}")


def test_mla_balanced_matches_partitioned():
    torch = torch_cuda()
    w = make_workload("mla", seed=14, B=6, lens=("uniform", 200, 3000))
    a = gpu_decode(torch, w, partition_size=0)
    b = gpu_decode(torch, w, partition_size=1024)
    ref = oracle_decode(w)
    assert_close(a, ref, "bf16", "mla balanced")
    assert_close(b, ref, "bf16", "mla partitioned")


def test_mla_balanced_large_latent_values():
    """Latent values up to ~2e4 (inside fp16's range, which p.V uses): compared in units of
    4096 so that the absolute bound scales with the data."""
    torch = torch_cuda()
    w = make_workload("mla", seed=15, B=3, lens=("uniform", 50, 900))
    from oracle.paged_attention import bf16_bits_to_f64
    vals = bf16_bits_to_f64(w.k_pool) * 4096.0
    w.k_pool = (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w.q = (np.asarray(bf16_bits_to_f64(w.q) / 4096.0, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = gpu_decode(torch, w, partition_size=0)
    ref = oracle_decode(w)
    assert np.isfinite(got).all()
    assert_close(got / 4096.0, ref / 4096.0, "bf16", "mla balanced, large latent values")


@pytest.mark.parametrize("ps", [0, 256])
def test_mla_lengths_above_max_context_len_are_truncated(ps):
    """As for the GQA call: lengths above max_context_len are attended up to it."""
    torch = torch_cuda()
    import paged_kv_cache_288_amd as pkv
    from gpu_common import to_device
    w = make_workload("mla", seed=8, B=4, lens=("uniform", 200, 1400))
    cap = 600
    dev = to_device(torch, w)
    out = torch.empty((w.B, w.Hq, w.d_v), dtype=torch.float32, device="cuda")
    pkv.paged_decode_attn_mla(out, dev["q"], dev["k_pool"], dev["block_table"],
                              dev["context_lens"], w.scale, cap, d_v=w.d_v, partition_size=ps)
    torch.cuda.synchronize()
    w.context_lens = np.minimum(w.context_lens, cap).astype(np.int32)
    assert_close(out.cpu().numpy(), oracle_decode(w), "bf16", f"mla truncated at {cap}, partition {ps}")
