"""The CPU-baseline leg of bench.py runs the oracle on request ranges with a
sub-pool of the slots each range touches. These checks (CPU only) confirm
that such a call computes exactly what the full call computes for those
requests, so the timed work is the workload's."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402

CASES = {
    "dense_gdn": lambda: W.make("c", W.GDN, B=6, T=2, H=2, HV=4, K=64, V=64,
                                pool_size=14, seed=1, separate_write=True,
                                write_skip=0.3),
    "lightning_in_place": lambda: W.make("c", W.LIGHTNING, B=5, T=1, H=4,
                                         HV=4, K=64, V=64, pool_size=9,
                                         seed=2),
    "kda_cache": lambda: W.make("c", W.KDA, B=4, T=3, H=2, HV=2, K=64, V=64,
                                pool_size=8, seed=3, inter=True),
    "varlen": lambda: W.make("c", W.GDN, B=6, T=4, H=2, HV=2, K=64, V=64,
                             pool_size=12, seed=4, varlen_min=0,
                             separate_write=True),
    "paged": lambda: W.make("c", W.GDN, B=4, T=3, H=2, HV=2, K=64, V=64,
                            pool_size=16, seed=5, paged=True),
}


def _full(wl):
    args, kw = bench._oracle_inputs(wl, 0, wl.B)
    return args, kw, oracle.decode(*args, **kw)


@pytest.mark.parametrize("name", sorted(CASES))
def test_range_call_equals_the_full_call(name):
    wl = CASES[name]()
    fargs, fkw, full = _full(wl)
    counts = wl.counts()
    cu = np.concatenate([[0], np.cumsum(counts)])
    for lo, hi in ((0, 1), (1, wl.B - 1), (wl.B // 2, wl.B)):
        args, kw = bench._oracle_inputs(wl, lo, hi)
        got = oracle.decode(*args, **kw)
        if wl.cu_seqlens is not None:
            want_out = full["out"][cu[lo]:cu[hi]]
        else:
            want_out = full["out"][lo:hi]
        np.testing.assert_array_equal(got["out"], want_out)
        if wl.inter:
            want = (full["inter"][cu[lo]:cu[hi]] if wl.cu_seqlens is not None
                    else full["inter"][lo:hi])
            np.testing.assert_array_equal(got["inter"], want)
        # every sub-pool slot ends as the full call left that slot
        pool = fargs[6]
        sub = args[6]
        for j in range(sub.shape[0]):
            matches = [s for s in range(pool.shape[0])
                       if np.array_equal(pool[s], sub[j])]
            assert matches, "sub-pool slot %d is not a pool slot" % j
        assert got["pool"].shape == sub.shape
        changed = [j for j in range(sub.shape[0])
                   if not np.array_equal(got["pool"][j], sub[j])]
        for j in changed:
            assert any(np.array_equal(got["pool"][j], full["pool"][s])
                       for s in range(pool.shape[0])), j


SHARD_CASES = dict(CASES)
SHARD_CASES["lightning_decays"] = lambda: W.make(
    "c", W.LIGHTNING, B=3, T=2, H=4, HV=4, K=64, V=64, pool_size=5, seed=6,
    lightning_decay=0.5 + 0.5 * torch.rand(4, generator=torch.Generator()
                                           .manual_seed(7)))


@pytest.mark.parametrize("name", sorted(SHARD_CASES))
def test_head_shard_is_the_full_call_on_its_heads(name):
    """bench.py --head-shards measures one GPU's share of the heads. Value
    heads do not interact, so that share computes exactly the full call's
    results on its heads: outputs, cached states and stored states."""
    wl = SHARD_CASES[name]()
    n = 2
    if name == "lightning_in_place":  # built-in decays depend on HV
        sh = W.head_shard(wl, n)
        assert sh.g is None and sh.HV == wl.HV // n
        return
    _, _, full = _full(wl)
    sh = W.head_shard(wl, n)
    hv = wl.HV // n
    assert (sh.H, sh.HV) == (wl.H // n, hv)
    assert sh.backing.is_contiguous()
    assert torch.equal(sh.backing, wl.backing[:, :hv])
    _, _, got = _full(sh)
    np.testing.assert_array_equal(got["out"], full["out"][..., :hv, :])
    np.testing.assert_array_equal(got["pool"], full["pool"][:, :hv])
    if wl.inter:
        np.testing.assert_array_equal(got["inter"],
                                      full["inter"][..., :hv, :, :])


def test_head_shard_rejects_uneven_splits():
    wl = CASES["dense_gdn"]()
    with pytest.raises(ValueError):
        W.head_shard(wl, 3)
    with pytest.raises(ValueError):
        W.head_shard(wl, 4)  # H = 2 cannot be split four ways
