"""The allocation-free selection entry point (hsa_select_noalloc) against
hsa_select with a caller workspace, through the C ABI: the same lists on two
calls in a row, the second on a smaller problem (the static workspace keeps
the first call's contents, which must not leak into the second)."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _scores(nh, nb, seed):
    rng = np.random.default_rng(seed)
    S = rng.random((nh, nb, nb)) ** 4
    S[0, 1, :] = 1.0                       # an all-tied row
    S /= S.sum(axis=2, keepdims=True)
    return torch.from_numpy(S.astype(np.float32)).cuda()


@pytest.mark.parametrize("mode", ["thresh_global", "topk"])
def test_noalloc_select_equals_workspace_select(mode):
    import block_sparse_attention_hilbert3d_amd as hsa
    hsa.lib()
    # the 720p threshold shape first, then a smaller one on the same array
    for nh, nb, tau, ratio, seed in ((24, 929, 0.25, 0.30, 1), (3, 70, 0.5, 0.1, 2)):
        _say(f"noalloc select {mode} nh={nh} nb={nb}")
        S = _scores(nh, nb, seed)
        if mode == "topk":
            p = hsa.make_params("topk", k=min(38, nb))
            cap = p.k
        else:
            p = hsa.make_params("thresh_global", tau=tau, budget_ratio=ratio)
            cap = nb
        want = hsa.hsa_select(S, nh, nb, p, cap)
        got = (torch.full((nh, nb, cap), 7, dtype=torch.int32, device="cuda"),
               torch.full((nh, nb), 7, dtype=torch.int32, device="cuda"))
        hsa.hsa_select_noalloc(S, nh, nb, p, cap, outs=got)
        torch.cuda.synchronize()
        assert torch.equal(got[1], want[1])
        # each row's first kv_cnt entries (the rest of a row is not written)
        valid = torch.arange(cap, device="cuda")[None, None, :] < want[1][..., None]
        assert torch.equal(torch.where(valid, got[0], -1), torch.where(valid, want[0], -1))


def test_noalloc_select_rejects_oversize():
    """More workspace than the static array holds is refused before launch."""
    import ctypes
    import block_sparse_attention_hilbert3d_amd as hsa
    L = hsa.lib()
    p = hsa.make_params("thresh_global", tau=0.25, budget_ratio=0.3)
    fake = ctypes.c_void_p(0x10000)
    assert L.hsa_select_noalloc(fake, 512, 1024, ctypes.byref(p), fake, fake, 1024, None) == 4
    assert b"static scratch" in L.hsa_last_error()
