"""Decode steps replayed as captured graphs, with the batch and context padded to buckets.

Replaying a captured step removes the per-kernel launch overhead, at the price of static
shapes and addresses, so a step is padded to the nearest bucket ("GPU推理深度拆解：KV
Cache视角", "算子优化要点").  A `DecodeStep` owns the static buffers of one bucket, captures
the append of the new rows plus the attention call once, and on every call copies the
caller's inputs into its buffers and replays the capture.  Padded batch rows carry
context length 0 (their output rows are zero) and slot -1 (their new rows are not
written).  The cache pools are the caller's: the capture records their addresses, so one
`DecodeStep` serves one set of pools (one layer).
"""

import paged_kv_cache_288_amd as pkv


def _bits(t):
    """The tensor's raw element bits (element values are never converted on copy)."""
    import torch
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def bucket_batch(B):
    """Smallest power of two >= B."""
    if B < 1:
        raise ValueError("batch must be positive")
    return 1 << (B - 1).bit_length()


def bucket_context(max_context_len, block_size):
    """Smallest power of two >= max_context_len, at least 256 tokens and one block."""
    n = max(256, block_size, int(max_context_len))
    return 1 << (n - 1).bit_length()


class DecodeStep:
    """One bucket's captured append + decode step.

    kind "gqa": pools [num_blocks, Hkv, block_size, d] (k_pool, v_pool), q [B, Hq, d];
    kind "mla": latent pool [num_blocks, block_size, d_qk] (k_pool; v_pool None),
    q [B, Hq, d_qk], output width d_v.  B_bucket and ctx_bucket fix the capture's shapes;
    calls with B <= B_bucket and every context <= ctx_bucket replay it (the block table's
    columns past ctx_bucket / block_size are not copied).
    """

    def __init__(self, kind, k_pool, v_pool, Hq, scale, B_bucket, ctx_bucket, kv_dtype="bf16",
                 k_scale=None, v_scale=None, d_v=512, partition_size=0):
        import torch
        if kind not in ("gqa", "mla"):
            raise ValueError("kind must be 'gqa' or 'mla'")
        self.kind, self.k_pool, self.v_pool = kind, k_pool, v_pool
        self.kv_dtype, self.k_scale, self.v_scale = kv_dtype, k_scale, v_scale
        self.Hq, self.scale, self.partition_size = Hq, float(scale), partition_size
        self.B_bucket, self.ctx_bucket = int(B_bucket), int(ctx_bucket)
        dev = k_pool.device
        if kind == "mla":
            num_blocks, bs, d = k_pool.shape
            Hkv, self.d_v = 1, d_v
            new_shape = (self.B_bucket, 1, d)
        else:
            num_blocks, Hkv, bs, d = k_pool.shape
            self.d_v = d
            new_shape = (self.B_bucket, Hkv, d)
        self.Hkv, self.d, self.block_size = Hkv, d, bs
        self.max_blocks = -(-self.ctx_bucket // bs)
        B = self.B_bucket
        self.q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device=dev)
        self.out = torch.zeros((B, Hq, self.d_v), dtype=torch.float32, device=dev)
        self.k_new = torch.zeros(new_shape, dtype=k_pool.dtype, device=dev)
        self.v_new = None if v_pool is None else torch.zeros(new_shape, dtype=v_pool.dtype,
                                                             device=dev)
        self.slots = torch.full((B,), -1, dtype=torch.int64, device=dev)
        self.block_table = torch.zeros((B, self.max_blocks), dtype=torch.int32, device=dev)
        self.context_lens = torch.zeros((B,), dtype=torch.int32, device=dev)
        if kind == "mla":
            nbytes = pkv.mla_workspace_bytes(B, Hq, self.d_v, self.ctx_bucket, partition_size)
        else:
            nbytes = pkv.decode_workspace_bytes(B, Hq, Hkv, d, self.ctx_bucket, partition_size)
        self.workspace = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev)
        self.graph = None
        self._capture()

    def _run(self):
        pkv.kv_append(self.k_pool, self.v_pool, self.k_new, self.v_new, self.slots,
                      kv_dtype=self.kv_dtype)
        if self.kind == "mla":
            pkv.paged_decode_attn_mla(self.out, self.q, self.k_pool, self.block_table,
                                      self.context_lens, self.scale, self.ctx_bucket,
                                      d_v=self.d_v, partition_size=self.partition_size,
                                      workspace=self.workspace)
        else:
            pkv.paged_decode_attn(self.out, self.q, self.k_pool, self.v_pool, self.block_table,
                                  self.context_lens, self.scale, self.ctx_bucket,
                                  kv_dtype=self.kv_dtype, k_scale=self.k_scale,
                                  v_scale=self.v_scale, partition_size=self.partition_size,
                                  workspace=self.workspace)

    def _capture(self):
        import torch
        side = torch.cuda.Stream(device=self.k_pool.device)
        side.wait_stream(torch.cuda.current_stream(self.k_pool.device))
        with torch.cuda.stream(side):
            pkv.graph_begin(self.k_pool.device)
            try:
                self._run()
            finally:
                graph = pkv.graph_end(self.k_pool.device)
        torch.cuda.current_stream(self.k_pool.device).wait_stream(side)
        self.graph = graph

    def __call__(self, q, k_new, v_new, slot_mapping, block_table, context_lens):
        """Append the new rows and attend, by replaying the capture; returns out[:B]."""
        B = q.shape[0]
        if B > self.B_bucket:
            raise ValueError(f"batch {B} exceeds the bucket {self.B_bucket}")
        _bits(self.q)[:B].copy_(_bits(q))
        _bits(self.k_new)[:B].copy_(_bits(k_new).reshape(self.k_new[:B].shape))
        if self.v_new is not None:
            _bits(self.v_new)[:B].copy_(_bits(v_new).reshape(self.v_new[:B].shape))
        self.slots[:B].copy_(slot_mapping)
        self.slots[B:].fill_(-1)
        width = min(block_table.shape[1], self.max_blocks)  # contexts fit the bucket
        self.block_table[:B, :width].copy_(block_table[:, :width])
        self.context_lens[:B].copy_(context_lens)
        self.context_lens[B:].zero_()
        self.graph.launch()
        return self.out[:B]

    def close(self):
        if self.graph is not None:
            self.graph.destroy()
            self.graph = None
