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


def test_mla_full_size_sampled():
    torch = torch_cuda()
    w = make_workload("mla")
    log(f"[mla] full size: B={w.B} max_ctx={w.max_context_len}")
    got = gpu_decode(torch, w)
    seqs = [0, 7, 19, 31]
    assert_close(got[seqs], oracle_decode(w, seqs), "bf16", f"mla full size sampled {seqs}")
    assert np.isfinite(got).all()


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
