"""The scheduler / block-manager oracle against the pages' worked examples and
invariants, and planted mistakes that those checks must catch."""

import pytest

import sched_pins as pins
from oracle import sched as S


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


# ---- planted mistakes -----------------------------------------------------

def _release_hashed_to_head(self, block_ids):
    for bid in reversed(block_ids):
        b = self.blocks[bid]
        b.ref_cnt -= 1
        if b.ref_cnt == 0:
            self.free.insert(0, bid)


def _release_forward(self, block_ids):
    for bid in block_ids:
        b = self.blocks[bid]
        b.ref_cnt -= 1
        if b.ref_cnt == 0:
            if b.hash is None:
                self.free.insert(0, bid)
            else:
                self.free.append(bid)


def _hits_whole_prompt(self, r):
    hits, parent = [], None
    for k in range(len(r.tokens) // self.B):
        parent = S.block_hash(parent, r.tokens[k * self.B:(k + 1) * self.B])
        bid = self.pool.cached.get(parent)
        if bid is None:
            break
        hits.append(bid)
    return hits


_orig_alloc = S.Scheduler._allocate_slots


def _alloc_no_cow(self, r, num_new, copies):
    need_total = -(-(r.num_computed + num_new) // self.B)
    need_new = need_total - len(r.blocks)
    if self.pool.num_free() < need_new:
        return False
    for _ in range(need_new):
        r.blocks.append(self.pool.take_fresh())
    return True


def _alloc_floor_plus_one(self, r, num_new, copies):
    need_total = (r.num_computed + num_new) // self.B + 1
    need_new = need_total - len(r.blocks)
    if self.pool.num_free() < need_new:
        return False
    for _ in range(max(0, need_new)):
        r.blocks.append(self.pool.take_fresh())
    return True


def _hash_unchained(parent, tokens):
    return _orig_hash(None, tokens)


_orig_hash = S.block_hash
_orig_cap = S.Scheduler._cap


def _cap_no_threshold(self, computed, num_new, budget):
    return min(num_new, budget, self.max_model_len - computed)


_orig_schedule = S.Scheduler.schedule


def _preempt_oldest(self):
    # the running list is reversed around the step, so pop() takes the oldest
    self.running.reverse()
    try:
        return _orig_schedule(self)
    finally:
        self.running.reverse()


MUTATIONS = {
    "hashed_blocks_freed_to_head": ("BlockPool", "release", _release_hashed_to_head),
    "release_first_block_first": ("BlockPool", "release", _release_forward),
    "prefix_hit_covers_whole_prompt": ("Scheduler", "_prefix_hits", _hits_whole_prompt),
    "no_copy_on_write": ("Scheduler", "_allocate_slots", _alloc_no_cow),
    "block_count_floor_plus_one": ("Scheduler", "_allocate_slots", _alloc_floor_plus_one),
    "threshold_ignored": ("Scheduler", "_cap", _cap_no_threshold),
    "preempt_oldest": ("Scheduler", "schedule", _preempt_oldest),
    "hash_not_chained": (None, "block_hash", _hash_unchained),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    owner, attr, bad = MUTATIONS[name]
    target = S if owner is None else getattr(S, owner)
    monkeypatch.setattr(target, attr, bad)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception:
            caught.append(check.__name__)
    assert caught, f"mutation {name} passed every pin"
