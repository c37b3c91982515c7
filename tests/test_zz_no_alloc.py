"""The split verify that allocates nothing (kda_verify_split_noalloc, for
callers that cannot allocate device memory) against the split verify with a
caller workspace (kda_verify_split): two calls in a row on the library's
static scratch, the second with a smaller batch, each compared bit for bit
with the workspace entry point and element by element with the oracle."""

import sys

import numpy as np
import pytest

import oracle
from linear_attention_decode_03_amd import inputs
from linear_attention_decode_03_amd.inputs import copy_problem

from . import _parity

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _args(d):
    return (d["x"], d["conv_w"], d["conv_b"], d["conv_state"], d["f_a"], d["beta"], d["a_log"],
            d["dt_bias"], d["slots"], d["state"], d["out"], d["gate"], d["norm_w"],
            d["lower_bound"], d["scale"], d["eps"], d["f_b"], d["accepted"])


def test_noalloc_matches_workspace_entry_point():
    import torch

    from linear_attention_decode_03_amd import device, kda

    assert torch.cuda.is_available(), "no GPU visible"
    kda.load_library()
    # the second call is smaller (fewer items, fewer tokens) and runs on the
    # scratch the first one left behind
    for label, cfg, split in (("first", dict(B=4, H=16, T=8, seed=801), 4),
                              ("second", dict(B=1, H=8, T=4, seed=802), 2)):
        B, H, T = cfg["B"], cfg["H"], cfg["T"]
        p = inputs.make_problem(dict(cfg, N=B * T + 1, W=T + 2))
        p["slots"][0, T - 1] = 0  # one skipped write target
        say(f"[noalloc] {label}: B={B} H={H} T={T} split={split}")
        before, ref = copy_problem(p), copy_problem(p)
        taps = oracle.run(ref, taps=True)
        d = device.to_device(p)
        kda.kda_verify_split_noalloc(*_args(d), T=T, split=split)
        torch.cuda.synchronize()
        got = device.to_host(d)
        d2 = device.to_device(p)
        ws = kda.split_workspace(B, H, T, d2["state"].device)
        kda.kda_verify_split(*_args(d2), ws, T=T, split=split)
        torch.cuda.synchronize()
        want = device.to_host(d2)
        for k in ("state", "conv_state", "out"):
            assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), (label, k)
        rep = _parity.compare_step(before, ref, got, taps)
        say(f"[noalloc] {label}: ok {rep}")
    # a call beyond the static scratch is refused before any device work
    p = inputs.make_problem(dict(B=64, H=32, T=4, N=257, W=6, seed=803))
    d = device.to_device(p)
    with pytest.raises(ValueError, match="static scratch"):
        kda.kda_verify_split_noalloc(*_args(d), T=4, split=4)
