"""Host-side block management around the paged cache (the caller's side of the library).

"深入LLM推理：从KV Cache到PD分离的Serving全景解析", "PagedAttention与Cache管理": the cache is
cut into fixed-size physical blocks handed out on demand, a per-sequence block table maps
logical blocks to physical ones, and blocks can be shared between requests, which prefix
caching and copy-on-write build on.  "PD 分离下的 KV Cache", "优化一：Prefix Cache（前缀缓
存）": full blocks are found again by the chain hash of their tokens and all tokens before
them (`pkv_block_hashes`).

`BlockAllocator` keeps the free list, per-block reference counts and the hash -> block map
of full, registered blocks.  It does no GPU work: when a sequence is about to write into a
block it shares, `writable_last_block` hands out a fresh block and returns the (source,
destination) pair, and the caller copies such pairs with `kv_copy_blocks` before appending.
"""

import paged_kv_cache_288_amd as pkv


class BlockAllocator:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks, self.block_size = num_blocks, block_size
        self.free = list(range(num_blocks - 1, -1, -1))   # pop() hands out 0, 1, 2, ...
        self.refs = [0] * num_blocks
        self.by_hash = {}                                  # chain hash -> block
        self.hash_of = {}                                  # block -> chain hash

    # ---- reference counting
    def allocate(self):
        if not self.free:
            raise MemoryError("no free KV blocks")
        b = self.free.pop()
        self.refs[b] = 1
        return b

    def share(self, block):
        if self.refs[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self.refs[block] += 1
        return block

    def release(self, block):
        if self.refs[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self.refs[block] -= 1
        if self.refs[block] == 0:
            h = self.hash_of.pop(block, None)
            if h is not None and self.by_hash.get(h) == block:
                del self.by_hash[h]
            self.free.append(block)

    # ---- prefix cache
    def register(self, tokens, blocks, parent=0):
        """Record the chain hashes of the full blocks of `tokens`, stored in `blocks`."""
        hashes = pkv.block_hashes(tokens, self.block_size, parent)
        for h, b in zip(hashes.tolist(), blocks):
            self.by_hash.setdefault(h, b)
            self.hash_of.setdefault(b, h)
        return hashes

    def match_prefix(self, tokens, parent=0):
        """Blocks holding the longest cached run of full blocks at the start of `tokens`;
        each returned block gains a reference (the caller's sequence now shares it)."""
        out = []
        for h in pkv.block_hashes(tokens, self.block_size, parent).tolist():
            b = self.by_hash.get(h)
            if b is None:
                break
            out.append(self.share(b))
        return out

    # ---- growth of one sequence
    def slots_for_append(self, blocks, length, n_new):
        """Slots of tokens length .. length + n_new - 1 of a sequence whose block table is
        `blocks` (extended in place with fresh blocks as needed).  Returns (slots, copies):
        if the block receiving the first new token is shared, it is replaced by a fresh one
        and (old, new) is in `copies` for the caller to copy before appending."""
        copies = []
        bs = self.block_size
        if n_new > 0 and length % bs and self.refs[blocks[length // bs]] > 1:
            old = blocks[length // bs]
            new = self.allocate()
            self.release(old)
            blocks[length // bs] = new
            copies.append((old, new))
        slots = []
        for pos in range(length, length + n_new):
            if pos // bs == len(blocks):
                blocks.append(self.allocate())
            slots.append(blocks[pos // bs] * bs + pos % bs)
        return slots, copies
