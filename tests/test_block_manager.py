"""Host tests of the prefix-caching block manager (C++ behind the C ABI; no GPU needed).

The central check is a content invariant: a simulated cache records which
token each slot holds. Freshly allocated slots are written, cached (hit)
blocks must already hold the right tokens, and copy-on-write copies are
applied. After every operation, every slot of every live sequence must hold
that sequence's token at that position. Reference counts must equal the number
of live owners, and the free-block count must equal the blocks nobody
references.
"""

from __future__ import annotations

import pytest
from hypothesis import HealthCheck, settings, strategies as st
from hypothesis.stateful import RuleBasedStateMachine, initialize, invariant, precondition, rule

import paged_attention_decode_amd as pa


def test_prefix_blocks_are_shared_and_partial_blocks_are_not():
    m = pa.BlockManager(64, 16)
    a = list(range(100))
    assert m.add_sequence(1, a) == 0
    b = a[:70] + [7] * 30
    assert m.add_sequence(2, b) == 64            # four full 16-token blocks match
    ta, tb = m.block_table(1), m.block_table(2)
    assert ta[:4] == tb[:4] and not set(ta[4:]) & set(tb[4:])
    assert all(m.block_ref(x) == 2 for x in ta[:4]) and m.block_ref(ta[4]) == 1
    assert m.slots(2, 60, 8) == [tb[3] * 16 + 12, tb[3] * 16 + 13, tb[3] * 16 + 14, tb[3] * 16 + 15,
                                 tb[4] * 16, tb[4] * 16 + 1, tb[4] * 16 + 2, tb[4] * 16 + 3]


def test_freed_blocks_stay_cached_until_evicted():
    m = pa.BlockManager(8, 4)
    m.add_sequence(1, list(range(16)))           # 4 full blocks
    m.free_sequence(1)
    assert m.stats()["free_blocks"] == 8 and m.stats()["cached_blocks"] == 4
    assert m.add_sequence(2, list(range(16))) == 16   # all four come back from the cache
    m.free_sequence(2)
    m.add_sequence(3, list(range(100, 132)))     # needs all 8 blocks: evicts the cached ones
    assert m.stats()["evictions"] == 4
    m.free_sequence(3)
    assert m.add_sequence(4, list(range(16))) == 0


def test_capacity_error_changes_nothing():
    m = pa.BlockManager(4, 4)
    m.add_sequence(1, list(range(12)))
    before = m.stats()
    with pytest.raises(pa.PagedAttnError) as ei:
        m.add_sequence(2, list(range(50, 60)))
    assert ei.value.code == 7
    assert m.stats() == before
    with pytest.raises(pa.PagedAttnError):
        m.block_table(2)


def test_decode_appends_fill_and_register_blocks():
    m = pa.BlockManager(16, 4)
    m.add_sequence(1, [5, 6, 7])
    slots = [m.append_token(1, t)[0] for t in (8, 9, 10, 11, 12)]
    table = m.block_table(1)
    assert len(table) == 2 and slots == [table[0] * 4 + 3, table[1] * 4, table[1] * 4 + 1,
                                        table[1] * 4 + 2, table[1] * 4 + 3]
    # the blocks filled by decoding are now reusable by an identical prompt
    assert m.add_sequence(2, [5, 6, 7, 8, 9, 10, 11, 12, 1]) == 8


def test_fork_shares_and_copy_on_write_splits():
    m = pa.BlockManager(16, 4)
    m.add_sequence(1, list(range(6)))            # blocks: full, partial (2 of 4)
    m.fork(1, 2)
    t1 = m.block_table(1)
    assert m.block_table(2) == t1 and m.block_ref(t1[1]) == 2
    slot, copy = m.append_token(2, 42)
    t2 = m.block_table(2)
    assert copy == (t1[1], t2[1]) and t2[0] == t1[0] and t2[1] != t1[1]
    assert slot == t2[1] * 4 + 2
    slot1, copy1 = m.append_token(1, 43)          # the parent's block is no longer shared
    assert copy1 is None and slot1 == t1[1] * 4 + 2


def test_hash_chain_distinguishes_equal_blocks_after_different_prefixes():
    m = pa.BlockManager(16, 4)
    m.add_sequence(1, [1, 2, 3, 4, 9, 9, 9, 9])
    assert m.add_sequence(2, [0, 2, 3, 4, 9, 9, 9, 9]) == 0   # same second block, different first
    assert not set(m.block_table(1)) & set(m.block_table(2))


def test_errors():
    with pytest.raises(pa.PagedAttnError):
        pa.BlockManager(0, 16)
    m = pa.BlockManager(4, 4)
    m.add_sequence(1, [1])
    with pytest.raises(pa.PagedAttnError):
        m.add_sequence(1, [2])
    with pytest.raises(pa.PagedAttnError):
        m.append_token(9, 1)
    with pytest.raises(pa.PagedAttnError):
        m.fork(1, 1)
    with pytest.raises(pa.PagedAttnError):
        m.slots(1, 0, 2)
    assert m.block_ref(99) == -1


VOCAB = st.integers(0, 3)  # tiny vocabulary: many equal blocks, many prefix hits


class ManagerMachine(RuleBasedStateMachine):
    BS = 4
    NB = 24

    @initialize()
    def setup(self):
        self.m = pa.BlockManager(self.NB, self.BS)
        self.content = {}     # slot -> token held there
        self.seqs = {}        # seq id -> token list
        self.next_id = 0

    def _write(self, sid, first):
        toks = self.seqs[sid]
        for t, slot in enumerate(self.m.slots(sid, first, len(toks) - first), start=first):
            self.content[slot] = toks[t]

    @rule(prompt=st.lists(VOCAB, min_size=0, max_size=14), reuse=st.booleans())
    def add(self, prompt, reuse):
        if reuse and self.seqs:
            base = self.seqs[sorted(self.seqs)[0]]
            prompt = base[:len(prompt)] + prompt[len(base):]
        sid = self.next_id
        self.next_id += 1
        try:
            cached = self.m.add_sequence(sid, prompt)
        except pa.PagedAttnError as e:
            assert e.code == 7
            return
        assert cached % self.BS == 0 and cached <= len(prompt)
        self.seqs[sid] = list(prompt)
        # cached blocks must already hold the prompt's tokens
        for t, slot in enumerate(self.m.slots(sid, 0, cached)):
            assert self.content.get(slot) == prompt[t]
        self._write(sid, cached)

    @precondition(lambda self: self.seqs)
    @rule(data=st.data(), token=VOCAB)
    def append(self, data, token):
        sid = data.draw(st.sampled_from(sorted(self.seqs)))
        try:
            slot, copy = self.m.append_token(sid, token)
        except pa.PagedAttnError as e:
            assert e.code == 7
            return
        if copy is not None:
            src, dst = copy
            for o in range(self.BS):
                if src * self.BS + o in self.content:
                    self.content[dst * self.BS + o] = self.content[src * self.BS + o]
        self.seqs[sid].append(token)
        self.content[slot] = token

    @precondition(lambda self: self.seqs)
    @rule(data=st.data())
    def fork(self, data):
        sid = data.draw(st.sampled_from(sorted(self.seqs)))
        child = self.next_id
        self.next_id += 1
        self.m.fork(sid, child)
        self.seqs[child] = list(self.seqs[sid])

    @precondition(lambda self: self.seqs)
    @rule(data=st.data())
    def free(self, data):
        sid = data.draw(st.sampled_from(sorted(self.seqs)))
        self.m.free_sequence(sid)
        del self.seqs[sid]

    @invariant()
    def every_slot_holds_its_token(self):
        if not hasattr(self, "m"):
            return
        for sid, toks in self.seqs.items():
            for t, slot in enumerate(self.m.slots(sid, 0, len(toks))):
                assert self.content.get(slot) == toks[t], (sid, t)

    @invariant()
    def reference_counts_and_free_blocks(self):
        if not hasattr(self, "m"):
            return
        owners = {}
        for sid in self.seqs:
            table = self.m.block_table(sid)
            assert len(table) == -(-len(self.seqs[sid]) // self.BS)
            assert len(set(table)) == len(table)
            for b in table:
                owners[b] = owners.get(b, 0) + 1
        for b in range(self.NB):
            assert self.m.block_ref(b) == owners.get(b, 0)
        assert self.m.stats()["free_blocks"] == self.NB - len(owners)

    def teardown(self):
        if hasattr(self, "m"):
            self.m.close()


TestManagerMachine = ManagerMachine.TestCase
TestManagerMachine.settings = settings(max_examples=60, stateful_step_count=40, deadline=None,
                                       suppress_health_check=[HealthCheck.too_slow])
