"""Paged KV-cache bookkeeping: block counts, slot mapping, free-block stack.

Test infrastructure only. Pages followed:

* mini-infer README, "Project overview": the KV cache is a set of fixed-size
  blocks handed out from a free-block pool, and a per-request BlockTable maps
  the request's logical blocks to physical ones.
* nxmr.cn inference-techniques article, section 2.1: a request of seq_len
  tokens needs ceil(seq_len / PAGE_SIZE) pages, each popped from the list of
  free pages. (The article grows the pool when the list is empty; a fixed
  free-block pool cannot, so exhaustion is an error here.)
* MegEngine/InferLLM article, section 4.2 "problem two": the KV-cache size is
  2 * batch * layers * max_seq_len * hidden * sizeof(dtype); under grouped-
  query attention the cached width per token is num_kv_heads * head_dim.

Pool layout (a reading: the pages fix none): per layer one K pool and one V
pool, each [num_blocks, num_kv_heads, block_size, head_dim], row-major.
"""
import numpy as np


def blocks_needed(num_tokens, block_size):
    """Pages needed for num_tokens tokens: ceil(num_tokens / block_size)."""
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens >= 0 and block_size > 0 required")
    return -(-num_tokens // block_size)


def slot(block_table_row, pos, block_size):
    """Physical (block id, offset in block) of logical token position ``pos``.

    The logical block is pos // block_size; the BlockTable row maps it to a
    physical block; the token sits at offset pos % block_size inside it.
    """
    return int(block_table_row[pos // block_size]), pos % block_size


def element_offset(blk, head, off, d, num_kv_heads, block_size, head_dim):
    """Flat element index of (block, kv head, offset, dim) in a row-major pool."""
    return ((blk * num_kv_heads + head) * block_size + off) * head_dim + d


def kv_cache_bytes(batch, layers, max_seq_len, hidden, dtype_bytes):
    """KV-cache size formula of the InferLLM article, section 4.2 problem two.

    The leading 2 counts K and V. For grouped-query attention ``hidden`` is
    the cached width num_kv_heads * head_dim.
    """
    return 2 * batch * layers * max_seq_len * hidden * dtype_bytes


def pool_bytes(num_blocks, num_kv_heads, block_size, head_dim, dtype_bytes=2):
    """Bytes of ONE pool (K or V) of one layer."""
    return num_blocks * num_kv_heads * block_size * head_dim * dtype_bytes


class FreeBlockStack:
    """Free-block pool as a LIFO stack (mini-infer "FreeBlockPool").

    Reading of the pages: the nxmr.cn article pops pages from the end of a
    Python list of free pages, so the pool is a stack. It is initialised so the
    first pop returns block 0, then 1, ...; freed ids are pushed back in the
    order given, so the last id freed is the next one handed out. An
    allocation that cannot be met in full fails and leaves the stack as it
    was.
    """

    def __init__(self, num_blocks):
        if num_blocks <= 0:
            raise ValueError("num_blocks > 0 required")
        self.num_blocks = num_blocks
        self._stack = list(range(num_blocks - 1, -1, -1))   # top of stack = end = 0
        self._free = np.ones(num_blocks, dtype=bool)

    def num_free(self):
        return len(self._stack)

    def alloc(self, n):
        if n < 0:
            raise ValueError("n >= 0 required")
        if n > len(self._stack):
            raise MemoryError("free-block pool exhausted")
        ids = [self._stack.pop() for _ in range(n)]
        self._free[ids] = False
        return ids

    def free(self, ids):
        ids = list(ids)
        seen = set()
        for i in ids:
            if not (0 <= i < self.num_blocks):
                raise ValueError("block id out of range")
            if self._free[i] or i in seen:
                raise ValueError("double free")
            seen.add(i)
        for i in ids:
            self._stack.append(i)
            self._free[i] = True


def append_model_positions(context_len, block_size, table_row):
    """Brute-force model of a growing cache: the (block, offset) reached by each
    appended token when tokens are appended one at a time to an empty cache and
    a new block is taken exactly when the current one is full.

    This is the list-of-blocks picture of the course project (KV-cache append,
    section 2.1) combined with the ceil(n / PAGE_SIZE) allocation of the
    nxmr.cn article, section 2.1; it contains no division or modulo, so it
    pins ``slot`` independently.
    """
    positions = []
    blocks_used = 0
    fill = block_size          # current block "full" before the first token
    for _ in range(context_len):
        if fill == block_size:
            blocks_used += 1
            fill = 0
        positions.append((int(table_row[blocks_used - 1]), fill))
        fill += 1
    return positions, blocks_used


def kv_pool_shape(num_blocks, num_kv_heads, block_size, head_dim):
    return (num_blocks, num_kv_heads, block_size, head_dim)


def expected_algorithmic_bytes_attention(context_lens, num_q_heads, num_kv_heads,
                                         head_dim, block_size, elem_bytes=2):
    """Bytes paged decode attention must move: every cached K and V element of
    the L = ctx + 1 attended tokens once per (sequence, kv head), q in and out
    once, the used block-table entries and the lengths."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    L = ctx + 1
    kv = 2 * elem_bytes * num_kv_heads * head_dim * int(L.sum())
    qo = 2 * elem_bytes * len(ctx) * num_q_heads * head_dim
    table = 4 * int(sum(blocks_needed(int(x), block_size) for x in L))
    return kv + qo + table + 4 * len(ctx)


def ceil_div(a, b):
    return -(-a // b)


__all__ = [
    "blocks_needed", "slot", "element_offset", "kv_cache_bytes", "pool_bytes",
    "FreeBlockStack", "append_model_positions", "kv_pool_shape",
    "expected_algorithmic_bytes_attention", "ceil_div",
]
