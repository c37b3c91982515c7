"""GPU parity of the RecoverSSM replay (kda_replay) against the oracle, and
the whole recovery flow on the GPU: record-mode verify, then replay of the
accepted prefix, against a plain verify of the same inputs."""

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


@pytest.fixture(scope="module")
def gpu():
    import torch

    assert torch.cuda.is_available(), "no GPU visible"
    from . import _gpu
    from linear_attention_decode_03_amd import kda

    kda.load_library()
    return _gpu


def replay_gpu(gpu, r):
    import torch

    d = gpu.to_device(r)
    gpu.run_replay(d)
    torch.cuda.synchronize()
    return d["state"].cpu().numpy()


@pytest.mark.parametrize("cfg", ["replay_t8", dict(B=5, H=3, T=3, N=13, seed=21),
                                 dict(B=7, H=2, T=8, N=17, seed=22, lower_bound=-12.0),
                                 dict(B=4, H=128, T=6, N=11, seed=24),
                                 dict(B=3, H=1, T=1, N=7, seed=25)])
def test_replay_parity(gpu, cfg):
    r = inputs.make_replay_problem(cfg)
    if not isinstance(cfg, str):
        r["n"][0] = 0                # a plain copy
        r["src"][1] = -2             # skipped
        r["n"][2] = r["T"] + 1       # skipped
    say(f"[replay] B={r['B']} H={r['H']} T={r['T']} N={r['N']}")
    ref = copy_problem(r)
    oracle.replay(ref)
    got = replay_gpu(gpu, copy_problem(r))
    worst = _parity.compare_replay(r, ref, got)
    say(f"[replay] ok, worst {worst:.2e}")


def test_replay_in_place(gpu):
    r = inputs.make_replay_problem(dict(B=6, H=4, T=5, N=13, seed=23))
    r["dst"] = r["src"].copy()
    ref = copy_problem(r)
    oracle.replay(ref)
    got = replay_gpu(gpu, copy_problem(r))
    _parity.compare_replay(r, ref, got)


def test_recovery_flow_gpu(gpu):
    import torch

    """Record-mode verify, then replay of n accepted tokens into fresh slots,
    equals the state a plain verify writes after token n.  The oracle's
    replay and plain verify agree bit for bit, and each GPU side is within
    1e-4 of the oracle, so the two GPU results are held to 2e-4."""
    T, B, H = 8, 6, 4
    p = inputs.make_problem(dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=31, record=1))
    plain = copy_problem(p)
    plain.update(record=0, rec_u=None, rec_kg=None)

    say("[recovery] record verify, replay, plain verify")
    d = gpu.to_device(p)
    gpu.run(d)
    torch.cuda.synchronize()
    rec = gpu.to_host(d)
    q = gpu.to_device(plain)
    gpu.run(q)
    torch.cuda.synchronize()
    plain_state = q["state"].cpu().numpy()
    n = np.array([1, 3, 8, 5, 0, 2], np.int32)
    N = p["N"]
    src = np.array([int(p["slots"][b, p["accepted"][b] - 1]) for b in range(B)], np.int32)
    state = np.concatenate([p["state"], np.zeros((B,) + p["state"].shape[1:], np.float32)])
    r = dict(B=B, H=H, T=T, N=N + B, lower_bound=p["lower_bound"], rec_u=rec["rec_u"],
             rec_kg=rec["rec_kg"], a_log=p["a_log"], dt_bias=p["dt_bias"], src=src,
             dst=np.arange(N, N + B, dtype=np.int32), n=n, state=state)
    got = replay_gpu(gpu, r)
    for b in range(B):
        want = p["state"][src[b]] if n[b] == 0 else plain_state[int(p["slots"][b, n[b] - 1])]
        g = got[N + b].reshape(H, -1).astype(np.float64)
        w = want.reshape(H, -1).astype(np.float64)
        rms = np.sqrt((w * w).mean(axis=1, keepdims=True))
        m = float((np.abs(g - w) / (np.abs(w) + rms)).max())
        assert m <= 2e-4, f"request {b} (n={n[b]}): relative error {m:.3e}"
