"""Host prefix cache: chained block hashes and shared full prompt blocks.

Semantics follow the pages ("PagedAttention from First Principles", section 9,
prefix caching; "PagedAttention Explained" (sevydevy), "How vLLM shares blocks
today" and "What full-block sharing means for a system prompt"):

* A full block's hash covers its parent block's hash, its own token ids and
  extra keys such as a cache salt, so two blocks with the same tokens match
  only when everything before them matches too.  The first block's parent is
  a fixed root.
* A table maps hashes to physical blocks.  A new prompt walks its full
  blocks: a hit shares the block (one more reference), a miss takes a fresh
  block and registers its hash.
* Only full blocks are cached; a partly filled last block is private.
* A block whose count reaches zero stays registered and can be revived by a
  later hit until the pool hands it out again, which drops its registration.
  The pool's free list is first-in first-out, so the least recently freed
  block goes first (least-recently-used eviction).

The hash function itself is not given on the pages: SHA-256 over the parent
digest, the token ids as little-endian int64 and the extra key bytes.

Host bookkeeping only; it never touches K/V values.
"""

import hashlib
import struct

from .blockpool import Sequence, reserve_slots

ROOT_HASH = bytes(32)


def block_hash(parent, token_ids, extra=b""):
    """Chained hash of one full block."""
    h = hashlib.sha256()
    h.update(parent)
    h.update(struct.pack(f"<{len(token_ids)}q", *[int(t) for t in token_ids]))
    h.update(extra)
    return h.digest()


class PrefixCache:
    def __init__(self, pool):
        self.pool = pool
        self.by_hash = {}   # hash -> physical block
        self.hash_of = {}   # physical block -> hash
        pool.on_take = self._forget

    def _forget(self, b):
        """The pool reused block b: its old contents, and so its hash, are gone."""
        h = self.hash_of.pop(b, None)
        if h is not None:
            del self.by_hash[h]

    def _share(self, b):
        if self.pool.ref.get(b, 0) == 0:
            self.pool.revive(b)
        else:
            self.pool.share(b)

    def allocate_prompt(self, token_ids, salt=b""):
        """A sequence holding ``token_ids``: full blocks through the cache, the
        rest private.  Returns the sequence and the number of cache hits (blocks
        whose K/V need not be computed again)."""
        B = self.pool.block_size
        seq = Sequence()
        parent, hits = ROOT_HASH, 0
        for i in range(len(token_ids) // B):
            h = block_hash(parent, token_ids[i * B:(i + 1) * B], salt)
            b = self.by_hash.get(h)
            if b is not None:
                self._share(b)
                hits += 1
            else:
                b = self.pool.take()
                self.by_hash[h] = b
                self.hash_of[b] = h
            seq.table.append(b)
            seq.length += B
            parent = h
        reserve_slots(self.pool, seq, len(token_ids) - seq.length)
        return seq, hits
