"""Pins of crop, snapshot and restore ([HB14] rollback: truncation for a KV cache,
copy and restore for a recurrent state; [DLM] item 2: crop after the first
rejected guess)."""
import numpy as np
import pytest

import oracle as O
from synth import make_state


def test_restore_is_bitwise_and_only_where_a_draft_was_rejected():
    D = 4
    st = make_state(5, 1000)
    snap = O.state_snapshot(st)
    assert snap is not st and np.array_equal(snap, st)
    st[:] = 7                                     # the verification pass rewrites the state
    n_acc = np.array([4, 0, 3, 4, 1])
    O.state_restore(st, snap, n_acc, D)
    for b in range(5):
        if n_acc[b] < D:
            assert np.array_equal(st[b], snap[b])
        else:
            assert np.all(st[b] == 7)


def test_crop_sets_lengths_and_rejects_out_of_range():
    class C:
        pass
    from synth import MTPConfig
    cfg = MTPConfig(93, "s", 8, 1, 1, 8, 8, 8, 1, 1e4, 1e-6, "f32", 1.0, 3, 1, 0, 0, 1, 1.0)
    c = O.KVCache(cfg, 3, 10)
    c.len[:] = [9, 5, 7]
    O.kv_crop(c, [4, 5, 0])
    assert list(c.len) == [4, 5, 0]
    with pytest.raises(ValueError):
        O.kv_crop(c, [11, 0, 0])


def test_crop_len_counts_the_settled_token_and_the_accepted_drafts():
    tl = np.zeros((3, 4, 5))
    tl[0, :, 1] = 1      # all three drafts (1, 1, 1) hold
    tl[1, 0, 1] = 1      # first holds, second does not
    tl[1, 1, 2] = 1
    tl[2, 0, 3] = 1      # first rejected
    r = O.greedy_verify(tl, np.ones((3, 3), int), [10, 20, 30])
    assert list(r.n_accept) == [3, 1, 0]
    assert list(r.crop_len) == [14, 22, 31]
