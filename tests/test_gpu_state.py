"""GPU checks of kv_crop, state snapshot/restore (bitwise, against the oracle) and the error paths."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, make_state, make_weights

pytestmark = pytest.mark.gpu

M = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import config, f32, i32, upload_weights  # noqa: E402


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, 19 * 1024 * 1024 + 48])
def test_snapshot_restore_bitwise(nbytes):
    B, D = 5, 3
    st = make_state(B, nbytes)
    g_state = torch.from_numpy(st).cuda()
    g_snap = torch.zeros_like(g_state)
    M.mtp_state_snapshot(g_state, g_snap, nbytes, B)
    torch.cuda.synchronize()
    assert torch.equal(g_snap.cpu(), torch.from_numpy(st))
    g_state.fill_(7)
    n_acc = np.array([3, 0, 2, 3, 1], np.int32)
    M.mtp_state_restore(g_state, g_snap, nbytes, B, i32(n_acc), D)
    ref = np.full_like(st, 7)
    O.state_restore(ref, O.state_snapshot(st), n_acc, D)
    assert np.array_equal(g_state.cpu().numpy(), ref)


def test_kv_crop_truncates_only():
    c = config(CONFIGS["tiny"])
    kv = M.KVCache(c, 4, 64)
    kv.len.copy_(i32([10, 20, 30, 40]))
    M.kv_crop(kv, i32([5, 25, -3, 40]))
    assert kv.len.cpu().tolist() == [5, 20, 0, 40]


def _tiny():
    cfg = CONFIGS["tiny"].replace(batch=2)
    w = make_weights(cfg)
    return cfg, config(cfg), upload_weights(cfg, w)


def test_capacity_overflow_is_reported_and_skipped():
    cfg, c, gw = _tiny()
    kv = M.KVCache(c, 2, 8)
    kv.len.copy_(i32([6, 0]))
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, 2, 4, 1, 8))
    toks = i32([[1, 2, 3, 4], [5, 6, -1, -1]])
    hid = torch.randn(2, 4, cfg.hidden, device="cuda")
    hout = torch.zeros_like(hid)
    d = torch.zeros(2, dtype=torch.int32, device="cuda")
    M.mtp_draft_step(c, gw, kv, 4, toks, hid, hout, d, None, ws)
    with pytest.raises(M.MTPError) as e:
        M.mtp_check(ws)
    assert e.value.code == -4
    assert kv.len.cpu().tolist() == [8, 2]          # sequence 0 took the two rows that fit
    M.mtp_check(ws)                                 # the status word was cleared


def test_token_outside_vocab_is_reported():
    cfg, c, gw = _tiny()
    kv = M.KVCache(c, 2, 16)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, 2, 2, 1, 16))
    toks = i32([[1, cfg.vocab], [5, 6]])
    hid = torch.randn(2, 2, cfg.hidden, device="cuda")
    d = torch.zeros(2, dtype=torch.int32, device="cuda")
    M.mtp_draft_step(c, gw, kv, 2, toks, hid, torch.zeros_like(hid), d, None, ws)
    with pytest.raises(M.MTPError) as e:
        M.mtp_check(ws)
    assert e.value.code == -7
    assert kv.len.cpu().tolist() == [1, 2]


def test_host_side_errors_launch_nothing():
    cfg, c, gw = _tiny()
    kv = M.KVCache(c, 2, 16)
    need = M.mtp_draft_workspace_size(c, 2, 2, 1, 16)
    small = M.new_workspace(need - 256)
    toks = i32([[1, 2], [3, 4]])
    hid = torch.randn(2, 2, cfg.hidden, device="cuda")
    d = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MTPError) as e:
        M.mtp_draft_step(c, gw, kv, 2, toks, hid, torch.zeros_like(hid), d, None, small)
    assert e.value.code == -5
    with pytest.raises(M.MTPError) as e:
        M.mtp_draft_step(c, gw, kv, 2, toks, hid, hid, d, None, M.new_workspace(need))
    assert e.value.code == -1
    bad = M.Config(**{**c.__dict__, "head_dim": 96})
    with pytest.raises(M.MTPError) as e:
        M.mtp_draft_workspace_size(bad, 2, 2, 1, 16)
    assert e.value.code == -2
    assert kv.len.cpu().tolist() == [0, 0]
    with pytest.raises(M.MTPError):
        M.spec_verify_workspace_size(2, 0, 100, M.sampling(1.0, 0, 0.9))  # D must be positive
