"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C-ABI library ``libpkv.so`` (declared in
``include/pkv.h``).  It only marshals arguments: tensor data pointers, sizes and
the current HIP stream go to the library, whose HIP kernels do every step of
the computation.  PyTorch supplies device memory and streams.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""

import ctypes
import os

__all__ = [
    "PKV_BF16", "PKV_FP8_E4M3", "PkvError", "library_path", "load_library",
    "abi_version", "kv_append", "decode_partition_size", "decode_workspace_bytes",
    "paged_decode_attn", "paged_decode_attn_noalloc", "mla_workspace_bytes", "paged_decode_attn_mla", "Graph",
    "graph_begin", "graph_end", "graph_launch", "graph_destroy", "kv_append_fp8",
    "kv_copy_blocks", "block_hashes", "multi_workspace_bytes", "paged_decode_attn_multi",
    "cascade_workspace_bytes", "paged_decode_attn_cascade", "validate",
]

PKV_BF16 = 1
PKV_FP8_E4M3 = 2
# status codes (include/pkv.h)
PKV_OK, PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_UNSUPPORTED = 0, -1, -2, -3, -4
PKV_ERR_ALIGN, PKV_ERR_WORKSPACE, PKV_ERR_HIP = -5, -6, -7
_DTYPES = {"bf16": PKV_BF16, "fp8": PKV_FP8_E4M3}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_c_int32, _c_size, _p = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p

# (name, restype, argtypes), in the order of include/pkv.h
_SIGNATURES = [
    ("pkv_abi_version", ctypes.c_int, []),
    ("pkv_status_str", ctypes.c_char_p, [_c_int32]),
    ("pkv_kv_append", _c_int32, [_p, _p, _p, _p, _p, _c_int32, _c_int32, _c_int32, _c_int32,
                                 _c_int32, _c_int32, _p]),
    ("pkv_decode_partition_size", _c_int32, [_c_int32, _c_int32, _c_int32, _c_int32]),
    ("pkv_decode_workspace_bytes", _c_size, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                             _c_int32]),
    ("pkv_paged_decode_attn", _c_int32, [_p, _p, _p, _p, _p, _p, _p, _p, _c_int32, _c_int32,
                                         _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                         _c_int32, ctypes.c_float, _c_int32, _c_int32, _p,
                                         _c_size, _p]),
    ("pkv_paged_decode_attn_noalloc", _c_int32, [_p, _p, _p, _p, _p, _p, _p, _p, _c_int32,
                                                 _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                                 _c_int32, _c_int32, ctypes.c_float, _c_int32,
                                                 _c_int32, _p]),
    ("pkv_mla_workspace_bytes", _c_size, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32]),
    ("pkv_paged_decode_attn_mla", _c_int32, [_p, _p, _p, _p, _p, _c_int32, _c_int32, _c_int32,
                                             _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                             ctypes.c_float, _c_int32, _p, _c_size, _p]),
    ("pkv_multi_workspace_bytes", _c_size, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                            _c_int32]),
    ("pkv_paged_decode_attn_multi", _c_int32, [_p, _p, _p, _p, _p, _p, _p, _p, _c_int32,
                                               _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                               _c_int32, _c_int32, _c_int32, ctypes.c_float,
                                               _c_int32, _p, _c_size, _p]),
    ("pkv_cascade_workspace_bytes", _c_size, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                              _c_int32]),
    ("pkv_paged_decode_attn_cascade", _c_int32, [_p, _p, _p, _p, _p, _p, _p, _c_int32, _p, _p,
                                                 _c_int32, _c_int32, _c_int32, _c_int32,
                                                 _c_int32, _c_int32, _c_int32, _c_int32,
                                                 ctypes.c_float, _c_int32, _p, _c_size, _p]),
    ("pkv_validate", _c_int32, [_p, _p, _p, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _p,
                                _c_int32, _p, _c_int32, _c_int32, _c_int32, _p]),
    ("pkv_kv_append_fp8", _c_int32, [_p, _p, _p, _p, _p, _p, _p, _c_int32, _c_int32, _c_int32,
                                     _c_int32, _c_int32, _p]),
    ("pkv_kv_copy_blocks", _c_int32, [_p, _p, _p, _p, _c_int32, _c_int32, _c_int32, _c_int32,
                                      _c_int32, _c_int32, _p]),
    ("pkv_block_hashes", _c_int32, [_p, _c_int32, _c_int32, ctypes.c_uint64, _p]),
    ("pkv_graph_begin", _c_int32, [_p]),
    ("pkv_graph_end", _c_int32, [_p, ctypes.POINTER(ctypes.c_void_p)]),
    ("pkv_graph_launch", _c_int32, [_p, _p]),
    ("pkv_graph_destroy", _c_int32, [_p]),
]
EXPORTED = [name for name, _, _ in _SIGNATURES]


class PkvError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def library_path():
    return os.path.join(_HERE, "libpkv.so")


def load_library():
    """Load libpkv.so (built in-tree by ``python -m paged_kv_cache_288_amd.build``)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m paged_kv_cache_288_amd.build`")
        lib = ctypes.CDLL(path)
        for name, res, args in _SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(fn, status):
    if status != 0:
        raise PkvError(fn, status, load_library().pkv_status_str(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(kv_dtype):
    if kv_dtype not in _DTYPES:
        raise ValueError(f"kv_dtype must be one of {sorted(_DTYPES)}")
    return _DTYPES[kv_dtype]


def _check_pools(k_pool, v_pool, kv_dtype, latent=False):
    """The library trusts the pool geometry it is given; a pool whose element size differs
    from kv_dtype's would be addressed past its end.  Reject such calls here, before any
    launch: element size 2 for bf16, 1 for FP8 codes; [num_blocks, Hkv, block_size, d]
    (latent: [num_blocks, block_size, d]); V shaped and typed like K."""
    want = 1 if kv_dtype == "fp8" else 2
    dims = 3 if latent else 4
    for name, pool in (("k_pool", k_pool), ("v_pool", v_pool)):
        if pool is None:
            continue
        if pool.dim() != dims:
            raise ValueError(f"{name} must have {dims} dimensions, got shape {tuple(pool.shape)}")
        if pool.element_size() != want:
            raise ValueError(f"{name} has {pool.element_size()}-byte elements; kv_dtype "
                             f"{kv_dtype!r} stores {want}-byte ones")
    if v_pool is not None and tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError(f"v_pool shape {tuple(v_pool.shape)} differs from k_pool's {tuple(k_pool.shape)}")


def abi_version():
    return load_library().pkv_abi_version()


def kv_append(k_pool, v_pool, k_new, v_new, slot_mapping, kv_dtype="bf16"):
    """Scatter new rows into the pool in place (pkv_kv_append).

    k_pool/v_pool [num_blocks, Hkv, block_size, d] (v_pool None for an MLA latent pool
    [num_blocks, block_size, d]), k_new/v_new [T, Hkv, d], slot_mapping [T] int64.
    Tensors hold the raw element bits (bf16 as torch.bfloat16/int16/uint16, FP8 as uint8
    or torch.float8_e4m3fn) on the current device.
    """
    mla = v_pool is None
    _check_pools(k_pool, v_pool, kv_dtype, latent=mla)
    if mla:
        num_blocks, bs, d = k_pool.shape
        Hkv = 1
    else:
        num_blocks, Hkv, bs, d = k_pool.shape
    T = slot_mapping.shape[0]
    st = load_library().pkv_kv_append(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T,
        num_blocks, Hkv, d, bs, _dtype_code(kv_dtype), _stream(k_pool.device))
    _check("pkv_kv_append", st)


def decode_partition_size(B, Hkv, max_context_len, partition_size=0):
    return load_library().pkv_decode_partition_size(B, Hkv, max_context_len, partition_size)


def decode_workspace_bytes(B, Hq, Hkv, d, max_context_len, partition_size=0):
    return load_library().pkv_decode_workspace_bytes(B, Hq, Hkv, d, max_context_len, partition_size)


def _workspace(nbytes, device, workspace):
    import torch
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def paged_decode_attn(out, q, k_pool, v_pool, block_table, context_lens, scale, max_context_len,
                      kv_dtype="bf16", k_scale=None, v_scale=None, partition_size=0,
                      workspace=None):
    """out[B, Hq, d] (fp32) = paged decode attention (pkv_paged_decode_attn).

    q [B, Hq, d] bf16; pools [num_blocks, Hkv, block_size, d]; block_table
    [B, max_blocks] int32; context_lens [B] int32; k_scale/v_scale [Hkv] fp32 for FP8.
    The workspace (device bytes) is allocated here with torch when not given.
    """
    _check_pools(k_pool, v_pool, kv_dtype)
    B, Hq, d = q.shape
    num_blocks, Hkv, bs, _ = k_pool.shape
    lib = load_library()
    nbytes = lib.pkv_decode_workspace_bytes(B, Hq, Hkv, d, max_context_len, partition_size)
    workspace, wsize = _workspace(nbytes, q.device, workspace)
    st = lib.pkv_paged_decode_attn(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), _ptr(context_lens), B, Hq, Hkv, d, bs, num_blocks,
        block_table.shape[1], max_context_len, float(scale), _dtype_code(kv_dtype),
        partition_size, _ptr(workspace), wsize, _stream(q.device))
    _check("pkv_paged_decode_attn", st)
    return out


def paged_decode_attn_noalloc(out, q, k_pool, v_pool, block_table, context_lens, scale,
                              max_context_len, kv_dtype="bf16", k_scale=None, v_scale=None,
                              partition_size=0):
    """out[B, Hq, d] (fp32) = paged decode attention through pkv_paged_decode_attn_noalloc:
    the same computation as paged_decode_attn, with the library's device scratch
    (PKV_NOALLOC_SCRATCH_BYTES per GPU) as the workspace; nothing is allocated."""
    _check_pools(k_pool, v_pool, kv_dtype)
    B, Hq, d = q.shape
    num_blocks, Hkv, bs, _ = k_pool.shape
    st = load_library().pkv_paged_decode_attn_noalloc(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), _ptr(context_lens), B, Hq, Hkv, d, bs, num_blocks,
        block_table.shape[1], max_context_len, float(scale), _dtype_code(kv_dtype),
        partition_size, _stream(q.device))
    _check("pkv_paged_decode_attn_noalloc", st)
    return out


def mla_workspace_bytes(B, Hq, d_v, max_context_len, partition_size=0):
    return load_library().pkv_mla_workspace_bytes(B, Hq, d_v, max_context_len, partition_size)


def paged_decode_attn_mla(out, q, kv_pool, block_table, context_lens, scale, max_context_len,
                          d_v=512, partition_size=0, workspace=None):
    """out[B, Hq, d_v] (fp32) = latent decode attention (pkv_paged_decode_attn_mla).

    q [B, Hq, d_qk] bf16; kv_pool [num_blocks, block_size, d_qk] bf16.
    """
    _check_pools(kv_pool, None, "bf16", latent=True)
    B, Hq, d_qk = q.shape
    num_blocks, bs, _ = kv_pool.shape
    lib = load_library()
    nbytes = lib.pkv_mla_workspace_bytes(B, Hq, d_v, max_context_len, partition_size)
    workspace, wsize = _workspace(nbytes, q.device, workspace)
    st = lib.pkv_paged_decode_attn_mla(
        _ptr(out), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(context_lens), B, Hq, d_qk,
        d_v, bs, num_blocks, block_table.shape[1], max_context_len, float(scale),
        partition_size, _ptr(workspace), wsize, _stream(q.device))
    _check("pkv_paged_decode_attn_mla", st)
    return out


def multi_workspace_bytes(B, q_len, Hq, Hkv, d, max_context_len):
    return load_library().pkv_multi_workspace_bytes(B, q_len, Hq, Hkv, d, max_context_len)


def paged_decode_attn_multi(out, q, k_pool, v_pool, block_table, context_lens, scale,
                            max_context_len, kv_dtype="bf16", k_scale=None, v_scale=None,
                            workspace=None):
    """out[B, q_len, Hq, d] (fp32) = multi-token decode attention, causal among each
    sequence's q_len new tokens (pkv_paged_decode_attn_multi).

    q [B, q_len, Hq, d] bf16; pools [num_blocks, Hkv, block_size, d]; context_lens count
    the new tokens, whose K/V are already in the pools; k_scale/v_scale [Hkv] for FP8.
    """
    _check_pools(k_pool, v_pool, kv_dtype)
    B, q_len, Hq, d = q.shape
    num_blocks, Hkv, bs, _ = k_pool.shape
    lib = load_library()
    nbytes = lib.pkv_multi_workspace_bytes(B, q_len, Hq, Hkv, d, max_context_len)
    workspace, wsize = _workspace(nbytes, q.device, workspace)
    st = lib.pkv_paged_decode_attn_multi(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), _ptr(context_lens), B, q_len, Hq, Hkv, d, bs, num_blocks,
        block_table.shape[1], max_context_len, float(scale), _dtype_code(kv_dtype),
        _ptr(workspace), wsize, _stream(q.device))
    _check("pkv_paged_decode_attn_multi", st)
    return out


def cascade_workspace_bytes(B, Hq, Hkv, d, prefix_len, max_tail_len):
    return load_library().pkv_cascade_workspace_bytes(B, Hq, Hkv, d, prefix_len, max_tail_len)


def paged_decode_attn_cascade(out, q, k_pool, v_pool, prefix_blocks, prefix_len, tail_table,
                              tail_lens, scale, max_tail_len, kv_dtype="bf16", k_scale=None,
                              v_scale=None, workspace=None):
    """out[B, Hq, d] (fp32) = decode attention over a shared prefix (prefix_blocks
    [prefix_len / block_size] int32) followed by each sequence's tail (tail_table
    [B, max_tail_blocks] int32, tail_lens [B] int32) (pkv_paged_decode_attn_cascade)."""
    _check_pools(k_pool, v_pool, kv_dtype)
    B, Hq, d = q.shape
    num_blocks, Hkv, bs, _ = k_pool.shape
    lib = load_library()
    nbytes = lib.pkv_cascade_workspace_bytes(B, Hq, Hkv, d, prefix_len, max_tail_len)
    workspace, wsize = _workspace(nbytes, q.device, workspace)
    st = lib.pkv_paged_decode_attn_cascade(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(prefix_blocks), prefix_len, _ptr(tail_table), _ptr(tail_lens), B, Hq, Hkv, d, bs,
        num_blocks, tail_table.shape[1], max_tail_len, float(scale), _dtype_code(kv_dtype),
        _ptr(workspace), wsize, _stream(q.device))
    _check("pkv_paged_decode_attn_cascade", st)
    return out


def validate(block_table, context_lens, num_blocks, block_size, slot_mapping=None,
             max_context_len=-1, v_pool=None, d_v=None):
    """Count caller-contract violations on the device (pkv_validate): returns a dict with
    the table entries in use outside the pool, context lengths outside the table, slots
    past the pool, slots written twice, context lengths above max_context_len (when it is
    given, >= 0) and bf16 V values in use of magnitude 65504 or more (when v_pool, a bf16
    pool [num_blocks, Hkv, block_size, d] or a latent pool [num_blocks, block_size, d], is
    given; d_v leading dims checked, default all).  Synchronises the current stream."""
    import torch
    counts = torch.empty(6, dtype=torch.int32, device=block_table.device)
    B, mb = block_table.shape
    T = 0 if slot_mapping is None else slot_mapping.shape[0]
    Hkv = d = 0
    if v_pool is not None:
        _check_pools(v_pool, None, "bf16", latent=v_pool.dim() == 3)
        if v_pool.dim() == 3:
            Hkv, d = 1, v_pool.shape[2]
        else:
            Hkv, d = v_pool.shape[1], v_pool.shape[3]
    dv = d if d_v is None else d_v
    st = load_library().pkv_validate(
        _ptr(counts), _ptr(block_table), _ptr(context_lens), B, mb, num_blocks, block_size,
        int(max_context_len), _ptr(slot_mapping), T, _ptr(v_pool), Hkv, d, dv,
        _stream(block_table.device))
    _check("pkv_validate", st)
    c = counts.cpu().tolist()
    return {"bad_block_ids": c[0], "bad_context_lens": c[1], "slots_past_pool": c[2],
            "duplicate_slots": c[3], "lengths_above_max": c[4], "v_out_of_fp16_range": c[5]}


def kv_append_fp8(k_pool, v_pool, k_new, v_new, k_scale, v_scale, slot_mapping):
    """Quantizing append (pkv_kv_append_fp8): bf16 rows k_new/v_new [T, Hkv, d] stored as
    FP8 E4M3 codes of x / scale[h] into the uint8 pools [num_blocks, Hkv, block_size, d];
    k_scale/v_scale [Hkv] fp32.  v_pool/v_new/v_scale may be None (K only)."""
    _check_pools(k_pool, v_pool, "fp8")
    num_blocks, Hkv, bs, d = k_pool.shape
    T = slot_mapping.shape[0]
    st = load_library().pkv_kv_append_fp8(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(k_scale), _ptr(v_scale),
        _ptr(slot_mapping), T, num_blocks, Hkv, d, bs, _stream(k_pool.device))
    _check("pkv_kv_append_fp8", st)


def kv_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks, kv_dtype="bf16"):
    """Copy-on-write support (pkv_kv_copy_blocks): block dst[i] <- block src[i] in each pool.
    Pools [num_blocks, Hkv, block_size, d] (an MLA latent pool [num_blocks, block_size,
    d] with v_pool None); src/dst int32 device tensors [n]."""
    _check_pools(k_pool, v_pool, kv_dtype, latent=k_pool.dim() == 3)
    if k_pool.dim() == 3:
        num_blocks, bs, d = k_pool.shape
        Hkv = 1
    else:
        num_blocks, Hkv, bs, d = k_pool.shape
    st = load_library().pkv_kv_copy_blocks(
        _ptr(k_pool), _ptr(v_pool), _ptr(src_blocks), _ptr(dst_blocks), src_blocks.shape[0],
        num_blocks, Hkv, d, bs, _dtype_code(kv_dtype), _stream(k_pool.device))
    _check("pkv_kv_copy_blocks", st)


def block_hashes(tokens, block_size, parent=0):
    """Prefix-cache keys of the full blocks of `tokens` (pkv_block_hashes, host): a numpy
    uint64 array, hash_i = H(hash_{i-1}, tokens of block i), hash_{-1} = parent."""
    import numpy as np
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    out = np.zeros(max(len(toks) // block_size, 0) if block_size > 0 else 0, dtype=np.uint64)
    n = load_library().pkv_block_hashes(
        toks.ctypes.data_as(ctypes.c_void_p), len(toks), block_size, int(parent) % (1 << 64),
        out.ctypes.data_as(ctypes.c_void_p))
    if n < 0:
        _check("pkv_block_hashes", n)
    return out[:n]


class Graph:
    """Library calls captured on a stream (pkv_graph_end), replayed by launch()."""

    def __init__(self, handle, device):
        self._handle = handle
        self.device = device

    def launch(self):
        """Enqueue one replay on the device's current stream (pkv_graph_launch)."""
        if self._handle is None:
            raise RuntimeError("graph already destroyed")
        _check("pkv_graph_launch",
               load_library().pkv_graph_launch(self._handle, _stream(self.device)))

    def destroy(self):
        if self._handle is not None:
            st = load_library().pkv_graph_destroy(self._handle)
            self._handle = None
            _check("pkv_graph_destroy", st)

    def __del__(self):
        if getattr(self, "_handle", None) is not None and _LIB is not None:
            _LIB.pkv_graph_destroy(self._handle)
            self._handle = None


def graph_begin(device=None):
    """Start capturing the device's current stream (pkv_graph_begin); it must not be the
    default stream.  Calls made on it until graph_end are recorded, not run."""
    import torch
    device = torch.device("cuda") if device is None else torch.device(device)
    _check("pkv_graph_begin", load_library().pkv_graph_begin(_stream(device)))


def graph_end(device=None):
    """Stop the capture started by graph_begin and instantiate it (pkv_graph_end)."""
    import torch
    device = torch.device("cuda") if device is None else torch.device(device)
    handle = ctypes.c_void_p()
    _check("pkv_graph_end", load_library().pkv_graph_end(_stream(device), ctypes.byref(handle)))
    return Graph(handle, device)


def graph_launch(graph):
    graph.launch()


def graph_destroy(graph):
    graph.destroy()

