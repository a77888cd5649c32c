"""Block management with a prefix cache, written out plainly — TEST INFRASTRUCTURE.

Nothing in the HIP library imports or mirrors this file.  It states the
host-side rules of block management in plain Python, to check the native
block manager of the library against them call by call.

What it follows:
  - datawhalechina page "17. vLLM PagedAttention", Step 4 and its reference
    solution: a free list; ceil(len / block_size) blocks per prompt; one more
    block whenever a sequence grows past its last block; OOM when the free
    list runs short;
  - ybb.press page "vLLM 与 LLM 推理部署实战" §2.2: a reference count per
    block; a write into a block that several sequences reference copies the
    block first; a block whose prefix hash matches a cached one is reused;
  - bogosort page §16 Prefix Caching: the cache key is a hash, tenants are
    isolated, blocks are reference counted; §17 Parallel Sampling: forks
    share the prompt's blocks.

Where the pages leave the policy open, the plainest deterministic one is
taken (and the native manager documents the same):
  - the free list is first-in first-out, in a given initial order;
  - the key of a full block is FNV-1a-64 (the published Fowler-Noll-Vo
    definition) over the little-endian bytes of the parent block's key
    (uint64, 0 for a prompt's first block), the namespace (uint64) and the
    block's token ids (int32 each); a hit also needs equal namespace, parent
    key and tokens, so equal keys alone never share a block;
  - only full blocks are cached; a fresh full block is cached unless its key
    is already in the cache; blocks that decode steps fill are cached the
    same way when the caller registers them;
  - a cached block nobody uses stays cached; fresh blocks come from the free
    list, else from evicting the least recently released cached block;
  - a finished sequence releases its blocks last first;
  - a call that fails changes nothing.
"""

from __future__ import annotations

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64-bit: for each byte, xor it in, then multiply by the prime."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_key(parent: int, namespace: int, tokens) -> int:
    data = parent.to_bytes(8, "little") + namespace.to_bytes(8, "little")
    for t in tokens:
        data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    return fnv1a64(data)


class OutOfBlocks(RuntimeError):
    pass


class PrefixBlockManager:
    def __init__(self, num_blocks: int, block_size: int, order=None):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks)) if order is None else [int(b) for b in order]
        self.ref = [0] * num_blocks
        self.cache = {}          # key -> block
        self.entry = {}          # block -> (key, parent, namespace, tokens tuple)
        self.lru = []            # cached blocks with no user, oldest release first

    # -- helpers
    def _available(self) -> int:
        return len(self.free) + len(self.lru)

    def _take(self) -> int:
        if self.free:
            b = self.free.pop(0)
        else:
            b = self.lru.pop(0)
            key = self.entry.pop(b)[0]
            del self.cache[key]
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.entry:
                self.lru.append(b)
            else:
                self.free.append(b)

    # -- calls
    def allocate_prompt(self, namespace: int, tokens):
        """Returns (blocks, number of leading cache hits)."""
        bs = self.block_size
        n = len(tokens)
        nblocks = -(-n // bs)
        full = n // bs
        keys, hits, parent = [], 0, 0
        for i in range(full):
            chunk = tuple(int(t) for t in tokens[i * bs:(i + 1) * bs])
            k = block_key(parent, namespace, chunk)
            keys.append(k)
            if hits == i and k in self.cache:
                b = self.cache[k]
                if self.entry[b][1:] == (parent, namespace, chunk):
                    hits += 1
            parent = k
        hit_blocks = [self.cache[keys[i]] for i in range(hits)]
        if nblocks - hits > self._available() - sum(b in self.lru for b in hit_blocks):
            raise OutOfBlocks("OOM")
        out = []
        for b in hit_blocks:
            if b in self.lru:
                self.lru.remove(b)
            self.ref[b] += 1
            out.append(b)
        parent = keys[hits - 1] if hits else 0
        for i in range(hits, nblocks):
            b = self._take()
            out.append(b)
            if i < full:
                if keys[i] not in self.cache:
                    chunk = tuple(int(t) for t in tokens[i * bs:(i + 1) * bs])
                    self.cache[keys[i]] = b
                    self.entry[b] = (keys[i], parent, namespace, chunk)
                parent = keys[i]
        return out, hits

    def register_blocks(self, namespace: int, tokens, table: list) -> int:
        """Cache the full blocks of ``tokens`` held by ``table`` (blocks filled by
        decode steps; intelliparadigm §6.2, prefix sharing across turns of a
        dialogue): block i is cached under the key of the first (i + 1) full
        blocks, unless it is already cached or the key is taken."""
        bs = self.block_size
        full = len(tokens) // bs
        added, parent = 0, 0
        for i in range(full):
            chunk = tuple(int(t) for t in tokens[i * bs:(i + 1) * bs])
            k = block_key(parent, namespace, chunk)
            b = table[i]
            if b not in self.entry and k not in self.cache:
                self.cache[k] = b
                self.entry[b] = (k, parent, namespace, chunk)
                added += 1
            parent = k
        return added

    def append(self, table: list, new_len: int) -> None:
        need = -(-new_len // self.block_size)
        if need - len(table) > self._available():
            raise OutOfBlocks("OOM")
        while len(table) < need:
            table.append(self._take())

    def fork(self, table: list) -> list:
        for b in table:
            self.ref[b] += 1
        return list(table)

    def copy_on_write(self, table: list, logical: int):
        b = table[logical]
        if self.ref[b] <= 1:
            return None
        if self._available() < 1:
            raise OutOfBlocks("OOM")
        dst = self._take()
        self.ref[b] -= 1
        table[logical] = dst
        return (b, dst)

    def release(self, table: list) -> None:
        for b in reversed(table):
            self._drop(b)

    # -- counters
    def num_free(self) -> int:
        return len(self.free)

    def num_evictable(self) -> int:
        return len(self.lru)

    def num_cached(self) -> int:
        return len(self.cache)
