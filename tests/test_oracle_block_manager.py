"""Pins of the block-manager oracle (CPU only).

1. A hand-worked scenario (block size 4, 6 blocks): every block id, slot,
   reference count and free-list state below was derived by hand from the
   rules the oracle states (FIFO free list starting 0..N-1, chained xxh64 of
   full blocks registered when their last row is emitted, hits stop at the
   first miss and never cover a whole prompt, release last block first), not
   produced by running any code.
2. Seeded serving traces (admission, chunked prefill, decode, preemption,
   finishing) with invariants checked after every call: reference counts
   equal the number of holders, the free list holds exactly the unreferenced
   blocks, chain hashes equal a from-scratch recomputation, shared blocks sit
   at the same index over identical prefixes, the metadata obeys the slot
   formula, and every emitted position reads back its own token through the
   simulated pool.
3. Planted mistakes in copies of the oracle, each caught by 1. or 2.
"""
import pytest
import xxhash

import oracle.block_manager as obm
from bm_trace import run_trace

A_TOK = [1, 2, 3, 4, 5, 6, 7, 8, 9]
B_TOK = [1, 2, 3, 4, 5, 6, 7, 8, 10, 11]


def hand_scenario(m):
    """Runs the scenario on manager m, asserting the hand-derived results."""
    assert m.allocate(1, A_TOK) == (obm.OK, 0)           # no table entries: blocks 0, 1, 2
    assert m.block_table(1) == [0, 1, 2] and m.free == [3, 4, 5]
    st, meta = m.prepare_prefill([1], None, 4)
    assert st == obm.OK
    assert meta["positions"] == list(range(9)) and meta["slot_mapping"] == list(range(9))
    assert meta["block_tables"] == [[0, 1, 2, -1]] and meta["context_lens"] == [9] and meta["cu_seqlens"] == [0, 9]
    h0 = xxhash.xxh64(b"".join(x.to_bytes(4, "little") for x in [1, 2, 3, 4]), seed=0).intdigest()
    h1 = xxhash.xxh64(b"".join(x.to_bytes(4, "little") for x in [5, 6, 7, 8]), seed=h0).intdigest()
    assert m.table == {h0: 0, h1: 1}                      # blocks 0 and 1 are full; block 2 is not

    assert m.allocate(2, B_TOK) == (obm.OK, 8)           # hits 0, 1; one fresh block (3)
    assert m.block_table(2) == [0, 1, 3] and m.ref[:4] == [2, 2, 1, 1] and m.free == [4, 5]
    st, meta = m.prepare_prefill([2], None, 4)
    assert meta["positions"] == [8, 9] and meta["slot_mapping"] == [12, 13] and meta["context_lens"] == [10]

    assert m.allocate(3, [1, 2, 3, 4]) == (obm.OK, 0)    # a whole-prompt hit is refused: fresh block 4
    assert m.block_table(3) == [4] and m.free == [5]
    assert m.allocate(4, [7, 7, 7, 7, 7]) == (obm.NO_BLOCKS, None)
    assert m.free == [5] and 4 not in m.seqs

    assert m.free_seq(1) == obm.OK                       # release 2, then 1, then 0
    assert m.free == [5, 2] and m.ref[:3] == [1, 1, 0]

    assert m.append_token(2, 12) == obm.OK               # position 10: same block 3
    st, meta = m.prepare_decode([2], 4)
    assert meta == {"positions": [10], "slot_mapping": [14], "block_tables": [[0, 1, 3, -1]], "context_lens": [11]}
    assert m.append_token(2, 13) == obm.OK
    st, meta = m.prepare_decode([2], 4)
    assert meta["slot_mapping"] == [15] and meta["context_lens"] == [12]
    h2 = xxhash.xxh64(b"".join(x.to_bytes(4, "little") for x in [10, 11, 12, 13]), seed=h1).intdigest()
    assert m.table[h2] == 3                               # block 3 filled by this step
    assert m.append_token(2, 14) == obm.OK               # position 12 opens a block: head of [5, 2]
    assert m.block_table(2) == [0, 1, 3, 5] and m.free == [2]
    st, meta = m.prepare_decode([2], 4)
    assert meta["slot_mapping"] == [20] and meta["context_lens"] == [13]

    assert m.allocate(5, [1, 2, 3, 4, 5, 6, 7, 8, 10, 11, 12, 13, 99]) == (obm.OK, 12)  # hits 0, 1, 3
    assert m.block_table(5) == [0, 1, 3, 2] and m.free == []
    assert [m.ref[b] for b in (0, 1, 2, 3)] == [2, 2, 1, 2]
    assert m.free_seq(3) == obm.OK and m.free == [4]
    assert m.can_allocate(A_TOK)                          # hits 0 and 1 in use: needs one block

    assert m.free_seq(5) == obm.OK and m.free == [4, 2]
    assert m.free_seq(2) == obm.OK and m.free == [4, 2, 5, 3, 1, 0]
    # released blocks keep their entries: a new prompt takes 0, 1, 3 back, then the head (4)
    assert m.allocate(6, [1, 2, 3, 4, 5, 6, 7, 8, 10, 11, 12, 13, 50]) == (obm.OK, 12)
    assert m.block_table(6) == [0, 1, 3, 4] and m.free == [2, 5]
    assert m.allocate(7, [9] * 9) == (obm.NO_BLOCKS, None)  # three blocks needed, two free
    assert m.allocate(7, [9] * 8) == (obm.OK, 0)
    assert m.block_table(7) == [2, 5] and m.free == []


def test_hand_worked_scenario():
    m = obm.OracleBlockManager(6, 4)
    hand_scenario(m)


def reuse_scenario(m):
    """Blocks 0 and 1 hold prompt [1..8]; after release, new content that
    takes them from the free list must erase their entries, so the old prompt
    no longer hits (hand-derived)."""
    assert m.allocate(1, A_TOK) == (obm.OK, 0)
    m.prepare_prefill([1], None, 3)
    assert len(m.table) == 2
    m.free_seq(1)                                         # free list [2, 1, 0]
    assert m.free == [2, 1, 0]
    assert m.allocate(2, [5] * 12) == (obm.OK, 0)         # takes 2, 1, 0 for new content
    assert m.table == {}
    m.free_seq(2)
    assert m.allocate(3, A_TOK) == (obm.OK, 0)            # no hit any more


def test_taking_a_registered_block_drops_its_entry():
    reuse_scenario(obm.OracleBlockManager(3, 4))


@pytest.mark.parametrize("seed", range(6))
def test_trace_invariants(seed):
    stats = run_trace(seed, num_blocks=40, bs=8, steps=150)
    assert stats["prefill"] > 0 and stats["decode"] > 0


def test_traces_exercise_hits_and_preemption():
    tot = {"hits": 0, "preempt": 0, "finished": 0}
    for seed in range(6):
        st = run_trace(seed, num_blocks=40, bs=8, steps=150)
        for k in tot:
            tot[k] += st[k]
    assert tot["hits"] > 5 and tot["preempt"] > 0 and tot["finished"] > 5, tot


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
class KeepsEntryOnReuse(obm.OracleBlockManager):
    """Forgets to drop a reused block's table entry."""

    def _take_fresh(self):
        b = self.free.pop(0)
        self.ref[b] = 1
        return b


class RegistersAtAllocation(obm.OracleBlockManager):
    """Registers full blocks when a prompt is admitted, before their K/V exist."""

    def allocate(self, seq_id, tokens):
        st, cached = super().allocate(seq_id, tokens)
        if st == obm.OK:
            s = self.seqs[seq_id]
            comp = s["computed"]
            self._emit(s, len(tokens))
            s["computed"] = comp
        return st, cached


class ReleasesFirstBlockFirst(obm.OracleBlockManager):
    def free_seq(self, seq_id):
        seq = self.seqs.pop(seq_id, None)
        if seq is None:
            return obm.INVALID
        for b in seq["blocks"]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        return obm.OK


class HitsWholePrompt(obm.OracleBlockManager):
    def _hits(self, tokens):
        bs = self.block_size
        ids, hashes, h = [], [], 0
        for b in range(len(tokens) // bs):
            h = obm.block_hash(self._chunk(tokens, b), h)
            blk = self.table.get(h)
            if blk is None:
                break
            ids.append(blk)
            hashes.append(h)
        return ids, hashes


class LastInFirstOut(obm.OracleBlockManager):
    def _take_fresh(self):
        self.free.insert(0, self.free.pop())
        return super()._take_fresh()


class SlotOffByBlock(obm.OracleBlockManager):
    def _slot(self, seq, pos):
        bs = self.block_size
        return seq["blocks"][min(pos // bs + (pos % bs == bs - 1), len(seq["blocks"]) - 1)] * bs + pos % bs


@pytest.mark.parametrize("cls", [KeepsEntryOnReuse, RegistersAtAllocation, ReleasesFirstBlockFirst, HitsWholePrompt,
                                 LastInFirstOut, SlotOffByBlock])
def test_planted_mistakes_are_caught(cls, monkeypatch):
    caught = False
    for scenario, size in ((hand_scenario, 6), (reuse_scenario, 3)):
        try:
            scenario(cls(size, 4))
        except AssertionError:
            caught = True
    if not caught:
        monkeypatch.setattr(obm, "OracleBlockManager", cls)
        for seed in range(6):
            try:
                run_trace(seed, num_blocks=40, bs=8, steps=150)
            except AssertionError:
                caught = True
                break
    assert caught, cls.__name__
