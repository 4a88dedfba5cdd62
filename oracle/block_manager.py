"""KV block manager, plain Python reference (oracle; test infrastructure).

What the pages fix:
  - blocks of 16 tokens and a per-sequence table from logical to physical blocks; a new
    physical block is taken from a free list only when the sequence's last block is full
    (vLLM-PagedAttention与连续批处理技术拆解, section 3.2; intelliparadigm article, section
    3.1); so the only waste is the unfilled tail of each last block (serving-engine article,
    section 2);
  - shared blocks carry a reference count and are read-only; a sequence that must write into
    one copies it first (copy-on-write: vLLM-PagedAttention与连续批处理技术拆解, section 3.4;
    serving-engine article, section 2);
  - prefix caching (serving-engine article, section 4): each full block gets a key made from
    the previous block's key, the block's token ids and extra data, so a key stands for the
    whole prefix; only full blocks are cached; released blocks keep their contents in a
    queue evicted least-recently-used first, a finished request's blocks entering it from
    the tail first.

Readings where the pages leave the policy open (the same as the C ABI states):
  - free list first-in first-out, initially 0..N-1; allocation takes the free list's head,
    else evicts the evictable queue's head; with neither, the operation fails unchanged;
  - key = FNV-1a-64(prev_key as 8 little-endian bytes, salt as 8, each token id as 4);
    prev_key = 0 for the first block; a hit also needs equal token ids; the first block
    to cache a key keeps it;
  - keys are registered when a block becomes full (prompt blocks at add, later ones when
    an appended token fills them);
  - release walks a sequence's blocks from the last to the first; a count reaching zero
    sends a cached block to the evictable queue's tail, any other to the free list's tail;
    a cache hit takes the block out of the queue.
  - preemption by swapping (vLLM-PagedAttention与连续批处理技术拆解, section 4.3: a victim's
    KV moves to CPU memory and comes back later): a host pool with its own first-in
    first-out free list; swap-out gives every block of an unshared sequence a host block in
    order and releases the device blocks as a finished sequence's are; swap-in allocates
    fresh device blocks, returns the host blocks to the tail of the host free list and
    registers the full blocks' keys when free.
"""
from __future__ import annotations

FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
MASK64 = (1 << 64) - 1


class NoBlocks(Exception):
    """Not enough free or evictable blocks (state unchanged)."""


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit: for each byte, xor it in, then multiply by the prime mod 2^64."""
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_key(prev: int, salt: int, tokens) -> int:
    data = prev.to_bytes(8, "little") + (salt & MASK64).to_bytes(8, "little")
    for t in tokens:
        data += (t & 0xFFFFFFFF).to_bytes(4, "little")
    return fnv1a64(data)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16, prefix_cache: bool = True):
        self.N, self.bs, self.prefix = num_blocks, block_size, prefix_cache
        self.ref = [0] * num_blocks
        self.free = list(range(num_blocks))     # head = index 0
        self.evictable = []                     # head = index 0 (least recently used)
        self.cache = {}                         # key -> block
        self.block_key = {}                     # cached block -> key
        self.block_tokens = {}                  # cached block -> its token ids
        self.seqs = {}                          # id -> dict(blocks, tokens, keys, salt, swapped)
        self.host_free = None                   # host pool free list, once configured

    # -- helpers
    def available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _allocate(self) -> int:
        if self.free:
            blk = self.free.pop(0)
        else:
            blk = self.evictable.pop(0)
            del self.cache[self.block_key.pop(blk)]
            del self.block_tokens[blk]
        self.ref[blk] = 1
        return blk

    def _register(self, blk, key, tokens):
        if self.prefix and blk not in self.block_key and key not in self.cache:
            self.cache[key] = blk
            self.block_key[blk] = key
            self.block_tokens[blk] = list(tokens)

    def _lookup(self, key, tokens):
        if not self.prefix or key not in self.cache:
            return None
        blk = self.cache[key]
        return blk if self.block_tokens[blk] == list(tokens) else None

    # -- operations
    def add(self, seq_id, tokens, salt: int = 0) -> int:
        """Returns the number of leading prompt tokens already cached."""
        if seq_id in self.seqs:
            raise KeyError(seq_id)
        bs, n = self.bs, len(tokens)
        nfull, nb = n // bs, -(-n // bs)
        keys, prev = [], 0
        for j in range(nfull):
            prev = block_key(prev, salt, tokens[j * bs:(j + 1) * bs])
            keys.append(prev)
        hits = []
        for j in range(nfull):
            blk = self._lookup(keys[j], tokens[j * bs:(j + 1) * bs])
            if blk is None:
                break
            hits.append(blk)
        in_queue = sum(1 for b in hits if b in self.evictable)
        if nb - len(hits) > self.available() - in_queue:
            raise NoBlocks()
        blocks = []
        for blk in hits:
            if blk in self.evictable:
                self.evictable.remove(blk)
            self.ref[blk] += 1
            blocks.append(blk)
        for j in range(len(hits), nb):
            blk = self._allocate()
            blocks.append(blk)
            if j < nfull:
                self._register(blk, keys[j], tokens[j * bs:(j + 1) * bs])
        self.seqs[seq_id] = dict(blocks=blocks, tokens=list(tokens), keys=keys, salt=salt,
                                 swapped=False)
        return len(hits) * bs

    def append(self, seq_id, token):
        """Returns (slot, cow_src, cow_dst); the pair is (-1, -1) without a copy."""
        s = self.seqs[seq_id]
        if s["swapped"]:
            raise ValueError("sequence is swapped out")
        bs = self.bs
        off = len(s["tokens"]) % bs
        src = dst = -1
        if off == 0:
            if self.available() < 1:
                raise NoBlocks()
            s["blocks"].append(self._allocate())
        elif self.ref[s["blocks"][-1]] > 1:
            if self.available() < 1:
                raise NoBlocks()
            old = s["blocks"][-1]
            new = self._allocate()
            self.ref[old] -= 1
            s["blocks"][-1] = new
            src, dst = old, new
        s["tokens"].append(token)
        last = s["blocks"][-1]
        if off == bs - 1:
            prev = s["keys"][-1] if s["keys"] else 0
            blk_tokens = s["tokens"][-bs:]
            key = block_key(prev, s["salt"], blk_tokens)
            s["keys"].append(key)
            self._register(last, key, blk_tokens)
        return last * bs + off, src, dst

    def fork(self, parent, child):
        if child in self.seqs:
            raise KeyError(child)
        p = self.seqs[parent]
        if p["swapped"]:
            raise ValueError("sequence is swapped out")
        for blk in p["blocks"]:
            self.ref[blk] += 1
        self.seqs[child] = dict(blocks=list(p["blocks"]), tokens=list(p["tokens"]),
                                keys=list(p["keys"]), salt=p["salt"], swapped=False)

    def free_seq(self, seq_id):
        s = self.seqs.pop(seq_id)
        if s["swapped"]:
            self.host_free.extend(s["blocks"])
            return
        for blk in reversed(s["blocks"]):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                (self.evictable if blk in self.block_key else self.free).append(blk)

    def set_host_blocks(self, n):
        if self.host_free is not None or n < 1:
            raise ValueError("host pool already set or empty")
        self.host_free = list(range(n))

    def swap_out(self, seq_id):
        """Returns the (device block, host block) pairs."""
        s = self.seqs[seq_id]
        if s["swapped"] or any(self.ref[b] > 1 for b in s["blocks"]):
            raise ValueError("cannot swap out")
        if len(self.host_free) < len(s["blocks"]):
            raise NoBlocks()
        host = [self.host_free.pop(0) for _ in s["blocks"]]
        pairs = list(zip(s["blocks"], host))
        for blk in reversed(s["blocks"]):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                (self.evictable if blk in self.block_key else self.free).append(blk)
        s["blocks"], s["swapped"] = host, True
        return pairs

    def swap_in(self, seq_id):
        """Returns the (host block, device block) pairs."""
        s = self.seqs[seq_id]
        if not s["swapped"]:
            raise ValueError("not swapped out")
        if self.available() < len(s["blocks"]):
            raise NoBlocks()
        dev = []
        for j, h in enumerate(s["blocks"]):
            blk = self._allocate()
            dev.append(blk)
            if j < len(s["keys"]):
                self._register(blk, s["keys"][j], s["tokens"][j * self.bs:(j + 1) * self.bs])
        pairs = list(zip(s["blocks"], dev))
        self.host_free.extend(s["blocks"])
        s["blocks"], s["swapped"] = dev, False
        return pairs

    # -- queries
    def slots(self, seq_id, first, count):
        s = self.seqs[seq_id]
        return [s["blocks"][p // self.bs] * self.bs + p % self.bs
                for p in range(first, first + count)]

    def table(self, seq_id, width):
        b = self.seqs[seq_id]["blocks"]
        if width < len(b):
            raise ValueError("table width too small")
        return b + [-1] * (width - len(b))

    def seq_len(self, seq_id):
        return len(self.seqs[seq_id]["tokens"])

    def stats(self):
        return len(self.free), len(self.evictable), len(self.cache)
