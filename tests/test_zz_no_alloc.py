"""spec_verify_noalloc (no workspace: the library's own per-GPU scratch array) against spec_verify
with a workspace, through the C ABI: bit-identical accept counts, emitted tokens and crop lengths
on two calls in a row, the second with a smaller input, greedy and sampling; a call that needs
more scratch than the array holds is refused before anything is launched."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

M = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import f32, i32  # noqa: E402


def _inputs(seed, B, D, V):
    g = np.random.default_rng(seed)
    tl = g.standard_normal((B, D + 1, V), dtype=np.float32) * 2.0
    drafts = g.integers(0, V, size=(B, D), dtype=np.int32)
    # plant agreement with the target's argmax on part of the drafts so that acceptance varies
    arg = tl[:, :D].argmax(-1)
    keep = g.random((B, D)) < 0.6
    drafts[keep] = arg[keep]
    ua = g.random((B, D), dtype=np.float32)
    us = g.random(B, dtype=np.float32)
    ctx = g.integers(1, 5000, size=B, dtype=np.int32)
    return tl, drafts, ua, us, ctx


def _both(B, D, V, sp, seed):
    tl, drafts, ua, us, ctx = _inputs(seed, B, D, V)
    outs = []
    for use_ws in (True, False):
        n = torch.full((B,), -9, dtype=torch.int32, device="cuda")
        out = torch.full((B, D + 1), -9, dtype=torch.int32, device="cuda")
        crop = torch.full((B,), -9, dtype=torch.int32, device="cuda")
        args = (B, D, V, f32(tl), i32(drafts), None, sp, f32(ua), f32(us), i32(ctx), n, out, crop)
        if use_ws:
            ws = M.new_workspace(M.spec_verify_workspace_size(B, D, V, sp))
            M.spec_verify(*args, ws)
        else:
            M.spec_verify_noalloc(*args)
        torch.cuda.synchronize()
        outs.append((n.cpu().numpy(), out.cpu().numpy(), crop.cpu().numpy()))
    return outs


@pytest.mark.parametrize("sampling", [None, (0.8, 40, 0.9, 0)])
def test_noalloc_matches_workspace_verify_on_two_calls(sampling):
    sp = None if sampling is None else M.sampling(*sampling)
    for (B, D, V), seed in (((24, 4, 50000), 1), ((3, 2, 3000), 2)):   # the second call is smaller
        a, b = _both(B, D, V, sp, seed)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), (B, D, V, sampling)
        assert np.all(a[0] >= 0) and np.all(a[0] <= D)
        assert (a[1] >= 0).sum() == (a[0] + 1).sum()


def test_noalloc_refuses_a_call_larger_than_its_scratch():
    B, D, V = 1100, 3, 512          # sampling at top-k 128: 4400 rows x 128 x 8 bytes > 4 MiB
    sp = M.sampling(1.0, 128, 1.0, 0)
    tl, drafts, ua, us, ctx = _inputs(3, B, D, V)
    n = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.full((B, D + 1), -9, dtype=torch.int32, device="cuda")
    crop = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MTPError) as e:
        M.spec_verify_noalloc(B, D, V, f32(tl), i32(drafts), None, sp, f32(ua), f32(us), i32(ctx), n, out, crop)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert int((out != -9).sum()) == 0     # nothing was launched
