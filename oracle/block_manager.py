"""Plain-Python oracle of the paged KV cache's block manager.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, the smoke check of the package entry file and the CPU-baseline
leg of the benchmark may import or call it. It shares no code with the native
library and imports nothing from it; the content hash comes from the `xxhash`
package (the library routine the pages name).

What it follows ("Nano-vLLM System Architecture Analysis"):
* section 2, "Paged KV Cache": fixed-size blocks, a free list, a table from
  content hash to block id for prefix caching, reference counts for shared
  blocks;
* section 2, "Scheduler": preemption releases a sequence's blocks;
* section 3, "Lifecycle of a Request": prepare_inputs builds positions, block
  tables and slot mappings;
* "Differences from Normal nanoGPT Inference", item 2: blocks are allocated
  on demand; identical prompt prefixes share blocks, found with xxhash.

The pages give the parts, not the rules; this is the reading taken:
1. The free list is a queue: take from the front, release to the back; it
   starts as 0..N-1.
2. Full block b of a sequence hashes as xxh64(its token ids as little-endian
   int32, seed = hash of block b-1, 0 for b = 0). Partial blocks never hash.
3. A full block enters the table when a prepare call emits its last row's
   slot; an existing entry for the same hash is kept. A block taken from the
   free list for new content leaves the table.
4. Allocation reuses the prompt's leading full blocks found in the table with
   identical token ids, stopping at the first miss and never reusing all of a
   prompt (at least one token stays to compute). Reused blocks in use gain a
   reference; reused released blocks come back off the free list.
5. Release drops blocks last to first; a block at zero references goes to the
   back of the free list.
6. Every call checks its inputs first and changes nothing when it fails.
"""
from __future__ import annotations

import struct
from typing import Dict, List, Optional, Sequence

import xxhash

OK = "ok"
NO_BLOCKS = "no_blocks"
INVALID = "invalid"


def block_hash(tokens: Sequence[int], seed: int) -> int:
    """xxh64 of one block's token ids (little-endian int32), chained on seed."""
    return xxhash.xxh64(struct.pack("<%di" % len(tokens), *tokens), seed=seed).intdigest()


class OracleBlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        assert num_blocks > 0 and block_size > 0
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: List[int] = list(range(num_blocks))
        self.ref = [0] * num_blocks
        self.block_key: List[Optional[int]] = [None] * num_blocks  # hash the block is registered under
        self.block_tokens: List[Optional[List[int]]] = [None] * num_blocks
        self.table: Dict[int, int] = {}
        self.seqs: Dict[int, dict] = {}

    # -- helpers ------------------------------------------------------------
    def _chunk(self, tokens, b):
        bs = self.block_size
        return list(tokens[b * bs:(b + 1) * bs])

    def _hits(self, tokens):
        bs = self.block_size
        full = len(tokens) // bs
        if full * bs == len(tokens):
            full -= 1  # never the whole prompt
        ids, hashes, h = [], [], 0
        for b in range(full):
            h = block_hash(self._chunk(tokens, b), h)
            blk = self.table.get(h)
            if blk is None or self.block_tokens[blk] != self._chunk(tokens, b):
                break
            ids.append(blk)
            hashes.append(h)
        return ids, hashes

    def _needed(self, tokens):
        ids, hashes = self._hits(tokens)
        total = -(-len(tokens) // self.block_size)
        return total - sum(1 for b in ids if self.ref[b] > 0), ids, hashes

    def _take_fresh(self):
        b = self.free.pop(0)
        key = self.block_key[b]
        if key is not None and self.table.get(key) == b:
            del self.table[key]
        self.block_key[b] = None
        self.block_tokens[b] = None
        self.ref[b] = 1
        return b

    def _emit(self, seq, upto):
        """Tokens [computed, upto) are emitted; register the blocks they fill."""
        bs = self.block_size
        for b in range(len(seq["hashes"]), upto // bs):
            seed = seq["hashes"][b - 1] if b else 0
            h = block_hash(self._chunk(seq["tokens"], b), seed)
            seq["hashes"].append(h)
            blk = seq["blocks"][b]
            if h not in self.table and self.block_key[blk] is None:
                self.table[h] = blk
                self.block_key[blk] = h
                self.block_tokens[blk] = self._chunk(seq["tokens"], b)
        seq["computed"] = upto

    def _row(self, seq, width):
        return [seq["blocks"][j] if j < len(seq["blocks"]) else -1 for j in range(width)]

    def _slot(self, seq, pos):
        bs = self.block_size
        return seq["blocks"][pos // bs] * bs + pos % bs

    # -- calls --------------------------------------------------------------
    def num_free_blocks(self) -> int:
        return len(self.free)

    def can_allocate(self, tokens) -> bool:
        return self._needed(list(tokens))[0] <= len(self.free)

    def allocate(self, seq_id, tokens):
        tokens = list(tokens)
        if not tokens or seq_id in self.seqs:
            return INVALID, None
        need, ids, hashes = self._needed(tokens)
        if need > len(self.free):
            return NO_BLOCKS, None
        blocks = []
        for b in ids:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            blocks.append(b)
        while len(blocks) < -(-len(tokens) // self.block_size):
            blocks.append(self._take_fresh())
        cached = len(ids) * self.block_size
        self.seqs[seq_id] = {"tokens": tokens, "blocks": blocks, "hashes": list(hashes), "computed": cached}
        return OK, cached

    def append_token(self, seq_id, token):
        seq = self.seqs.get(seq_id)
        if seq is None or seq["computed"] != len(seq["tokens"]):
            return INVALID
        if len(seq["tokens"]) % self.block_size == 0:
            if not self.free:
                return NO_BLOCKS
            seq["blocks"].append(self._take_fresh())
        seq["tokens"].append(token)
        return OK

    def append_tokens(self, seq_ids, tokens):
        """One token for each of several distinct sequences, all or nothing."""
        if len(set(seq_ids)) != len(seq_ids):
            return INVALID
        for i in seq_ids:
            s = self.seqs.get(i)
            if s is None or s["computed"] != len(s["tokens"]):
                return INVALID
        opening = sum(1 for i in seq_ids if len(self.seqs[i]["tokens"]) % self.block_size == 0)
        if opening > len(self.free):
            return NO_BLOCKS
        for i, t in zip(seq_ids, tokens):
            assert self.append_token(i, t) == OK
        return OK

    def free_seq(self, seq_id):
        seq = self.seqs.pop(seq_id, None)
        if seq is None:
            return INVALID
        for b in reversed(seq["blocks"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        return OK

    def block_table(self, seq_id):
        return list(self.seqs[seq_id]["blocks"])

    def seq_info(self, seq_id):
        s = self.seqs[seq_id]
        return len(s["tokens"]), s["computed"], len(s["blocks"])

    def prepare_prefill(self, seq_ids, max_new=None, max_blocks_per_seq=1, max_total_q=1 << 30):
        if len(set(seq_ids)) != len(seq_ids) or any(i not in self.seqs for i in seq_ids):
            return INVALID, None
        counts = []
        for k, i in enumerate(seq_ids):
            s = self.seqs[i]
            n = len(s["tokens"]) - s["computed"]
            if max_new is not None:
                n = min(n, max_new[k])
            if n <= 0 or len(s["blocks"]) > max_blocks_per_seq:
                return INVALID, None
            counts.append(n)
        if sum(counts) > max_total_q:
            return INVALID, None
        out = {"positions": [], "slot_mapping": [], "block_tables": [], "context_lens": [], "cu_seqlens": [0]}
        for i, n in zip(seq_ids, counts):
            s = self.seqs[i]
            c = s["computed"]
            out["positions"] += list(range(c, c + n))
            out["slot_mapping"] += [self._slot(s, p) for p in range(c, c + n)]
            out["block_tables"].append(self._row(s, max_blocks_per_seq))
            out["context_lens"].append(c + n)
            out["cu_seqlens"].append(out["cu_seqlens"][-1] + n)
            self._emit(s, c + n)
        return OK, out

    def prepare_decode(self, seq_ids, max_blocks_per_seq=1):
        if len(set(seq_ids)) != len(seq_ids) or any(i not in self.seqs for i in seq_ids):
            return INVALID, None
        for i in seq_ids:
            s = self.seqs[i]
            if s["computed"] != len(s["tokens"]) - 1 or len(s["blocks"]) > max_blocks_per_seq:
                return INVALID, None
        out = {"positions": [], "slot_mapping": [], "block_tables": [], "context_lens": []}
        for i in seq_ids:
            s = self.seqs[i]
            p = s["computed"]
            out["positions"].append(p)
            out["slot_mapping"].append(self._slot(s, p))
            out["context_lens"].append(p + 1)
            out["block_tables"].append(self._row(s, max_blocks_per_seq))
            self._emit(s, p + 1)
        return OK, out
