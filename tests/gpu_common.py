"""Shared helpers for the GPU parity tests: move a workload to the device, run the HIP path
through the binding, and run the fp64 oracle on the same stored bits (optionally on a
sample of sequences, for full-size workloads)."""

import sys

import numpy as np
import pytest

import oracle
from paged_kv_cache_288_amd.workloads import make_workload  # noqa: F401  (re-export)

# Acceptance bounds: |gpu - ref| <= ABS + REL * |ref| element by element.
# bf16 K/V with fp32 accumulation: 2e-3 + 1e-2 |ref|; FP8 K/V: 2e-3 + 3e-2 |ref|.
TOL = {"bf16": (2e-3, 1e-2), "fp8": (2e-3, 3e-2)}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_device(torch, arr, device="cuda"):
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def to_device(torch, w):
    d = dict(
        q=bits_to_device(torch, w.q),
        k_pool=bits_to_device(torch, w.k_pool),
        v_pool=bits_to_device(torch, w.v_pool),
        block_table=torch.from_numpy(w.block_table).to("cuda"),
        context_lens=torch.from_numpy(w.context_lens).to("cuda"),
        k_scale=None if w.k_scale is None else torch.from_numpy(w.k_scale).to("cuda"),
        v_scale=None if w.v_scale is None else torch.from_numpy(w.v_scale).to("cuda"),
        new_k=bits_to_device(torch, w.new_k),
        new_v=bits_to_device(torch, w.new_v),
        slot_mapping=torch.from_numpy(w.slot_mapping).to("cuda"),
    )
    return d


def gpu_decode(torch, w, dev=None, partition_size=None, out=None):
    import paged_kv_cache_288_amd as pkv
    dev = dev or to_device(torch, w)
    ps = w.partition_size if partition_size is None else partition_size
    if out is None:
        out = torch.empty((w.B, w.Hq, w.d_v), dtype=torch.float32, device="cuda")
    if w.kind == "mla":
        pkv.paged_decode_attn_mla(out, dev["q"], dev["k_pool"], dev["block_table"],
                                  dev["context_lens"], w.scale, w.max_context_len, d_v=w.d_v,
                                  partition_size=ps)
    else:
        pkv.paged_decode_attn(out, dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                              dev["context_lens"], w.scale, w.max_context_len,
                              kv_dtype=w.kv_dtype, k_scale=dev["k_scale"],
                              v_scale=dev["v_scale"], partition_size=ps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _subset(w, seqs):
    """Pools restricted to the blocks the given sequences use, with their tables remapped.
    (Test plumbing only: what the oracle then computes is unchanged.)"""
    seqs = list(seqs)
    used = []
    for b in seqs:
        n = -(-int(w.context_lens[b]) // w.bs)
        used.append(w.block_table[b, :n].astype(np.int64))
    uniq = np.unique(np.concatenate(used)) if used else np.zeros(0, np.int64)
    remap = {int(x): i for i, x in enumerate(uniq)}
    table = np.full((len(seqs), w.max_blocks), -1, dtype=np.int64)
    for i, u in enumerate(used):
        table[i, :len(u)] = [remap[int(x)] for x in u]
    kp = w.k_pool[uniq]
    vp = None if w.v_pool is None else w.v_pool[uniq]
    return kp, vp, table, w.context_lens[seqs], w.q[seqs]


def oracle_decode(w, seqs=None):
    seqs = range(w.B) if seqs is None else seqs
    kp, vp, table, lens, q = _subset(w, seqs)
    qf = oracle.bf16_bits_to_f64(q)
    if w.kind == "mla":
        kv = oracle.bf16_bits_to_f64(kp)
        return oracle.mla_decode_attention(qf, kv, table, lens, w.scale, w.d_v)
    K = oracle.decode_kv_bits(kp, w.kv_dtype, w.k_scale)
    V = oracle.decode_kv_bits(vp, w.kv_dtype, w.v_scale)
    return oracle.paged_decode_attention(qf, K, V, table, lens, w.scale)


def assert_close(got, ref, kv_dtype, what=""):
    ab, rel = TOL[kv_dtype]
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ab + rel * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    normwise = err.max() / max(np.abs(ref).max(), 1e-30)
    log(f"  {what}: max|err|={err.max():.3e} normwise={normwise:.3e} "
        f"worst at {worst}: got {got[worst]:.6g} ref {ref[worst]:.6g}")
    assert (err <= bound).all(), f"{what}: {int((err > bound).sum())} elements out of tolerance"
    if kv_dtype == "fp8":
        # the FP8 bound is relative; the absolute floor above is a large share of the small
        # outputs of long contexts, so the bound is also checked normwise
        assert err.max() <= rel * np.abs(ref).max(), f"{what}: normwise error {normwise:.3e} > {rel}"
