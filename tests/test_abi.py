"""The C-ABI library loads and exports every entry point include/mtp.h declares; host-side
argument checks work without a GPU (they return before anything is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtp.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["mtp_draft_step", "mtp_draft_loop", "spec_verify", "kv_crop", "mtp_state_snapshot",
              "mtp_state_restore", "mtp_draft_workspace_size", "spec_verify_workspace_size", "mtp_check",
              "mtp_last_error", "mtp_timer_start", "mtp_timer_read", "mtp_target_workspace_size",
              "mtp_target_forward", "mtp_draft_loop_shared_kv", "mtp_draft_loop_multi"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    M = pytest.importorskip("speculative_decoding_mtp_amd")
    lib = ctypes.CDLL(M.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(M.EXPORTED)


def test_host_side_checks_without_a_gpu():
    M = pytest.importorskip("speculative_decoding_mtp_amd")
    from synth import CONFIGS
    from tests.gpu_util import config
    c = config(CONFIGS["qwen"])
    assert M.mtp_draft_workspace_size(c, 1, 2, 1, 4500) > 0
    with pytest.raises(M.MTPError) as e:
        M.mtp_draft_workspace_size(M.Config(**{**c.__dict__, "wdtype": 7}), 1, 2, 1, 16)
    assert e.value.code == -3
    with pytest.raises(M.MTPError) as e:
        M.mtp_draft_workspace_size(c, 0, 2, 1, 16)
    assert e.value.code == -1
    # top-k off or above the candidate buffer takes the whole-vocabulary path
    assert M.spec_verify_workspace_size(4, 2, 1000, M.sampling(1.0, 500, 0.9)) > 0
    assert M.spec_verify_workspace_size(4, 2, 1000, M.sampling(1.0, 0, 0.9)) > 0
    assert M.spec_verify_workspace_size(4, 2, 1000, M.sampling(1.0, 50, 0.9)) > 0
    with pytest.raises(M.MTPError):
        M.spec_verify_workspace_size(4, 0, 1000, M.sampling(1.0, 50, 0.9))


def test_host_side_checks_of_the_widened_loops_without_a_gpu():
    # NULL device pointers: every check below fails on the host, before any launch
    M = pytest.importorskip("speculative_decoding_mtp_amd")
    from synth import CONFIGS
    from tests.gpu_util import config
    c = config(CONFIGS["tiny"]).c()
    lib = M._lib
    rc = lib.mtp_draft_loop_multi(ctypes.byref(c), None, 0, None, 2, 1, None, None, None, None, None, None, 0, None)
    assert rc == -1
    assert b"M >= 1" in M._lib.mtp_last_error()
    w = (M.MtpWeights * 1)()
    kv = (M.MtpKV * 1)()
    rc = lib.mtp_draft_loop_multi(ctypes.byref(c), w, 1, kv, 2, 1, None, None, None, None, None, None, 0, None)
    assert rc == -1                                  # NULL weights
    layers = (ctypes.c_int32 * 1)(0)
    rc = lib.mtp_draft_loop_shared_kv(ctypes.byref(c), None, None, 1, layers, 2, None, None, None, None, None,
                                      None, 0, None)
    assert rc == -1
    rc = lib.mtp_target_forward(ctypes.byref(c), None, None, 1, None, None, None, None, 0, None)
    assert rc == -1
