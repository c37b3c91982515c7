"""GPU parity: the HIP path through the C ABI against the CPU oracle,
element by element, on seeded inputs (contract in tests/_parity.py).

Covers the five workloads at their full sizes (every item compared), ragged
and degenerate shapes, padding and out-of-range tables, the invariants of
the method on the GPU, and the launch on a non-default stream.
"""

import sys

import numpy as np
import pytest

import oracle
from linear_attention_decode_03_amd import inputs
from linear_attention_decode_03_amd.inputs import copy_problem, to_bf16

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


def gpu_step(gpu, p, ahead=-1, stream=None):
    import torch

    d = gpu.to_device(p)
    gpu.run(d, ahead=ahead, stream=stream)
    torch.cuda.synchronize()
    return gpu.to_host(d)


def check(gpu, p, label, ahead=-1):
    say(f"[parity] {label}: B={p['B']} H={p['H']} T={p['T']} N={p['N']} W={p['W']} "
        f"record={p['record']} gate_mode={p['gate_mode']}")
    before = copy_problem(p)
    ref = copy_problem(p)
    taps = oracle.run(ref, taps=True)
    got = gpu_step(gpu, p, ahead=ahead)
    rep = _parity.compare_step(before, ref, got, taps)
    say(f"[parity] {label}: ok {rep}")
    return rep, got, ref


# --------------------------------------------------------------------------
# the five workloads at full size


@pytest.mark.parametrize("name", list(inputs.CONFIGS))
def test_config_parity(gpu, name):
    p = inputs.make_problem(name)
    rep, _, _ = check(gpu, p, name)
    live = len(_parity._live_items(p))
    assert rep["out_ties_used"] <= max(4, 0.002 * live * p["T"] * 128)


@pytest.mark.parametrize("name,steps", [("decode_b256", 4), ("verify_t4", 3)])
def test_chained_launches(gpu, name, steps):
    """Several launches back to back on the same pools (the state evolves),
    compared with the oracle after every launch.  A store whose data is
    corrupted in flight shows up here even when it strikes a few pages per
    launch."""
    import torch

    p = inputs.make_problem(name)
    ref = copy_problem(p)
    d = gpu.to_device(p)
    for k in range(steps):
        before = copy_problem(ref)
        taps = oracle.run(ref, taps=True)
        gpu.run(d)
        torch.cuda.synchronize()
        got = gpu.to_host(d)
        say(f"[chain] {name} launch {k}")
        _parity.compare_step(before, ref, got, taps)
        # the next launch starts from the GPU's own pools, as a caller's would
        ref["state"] = got["state"].copy()
        ref["conv_state"] = got["conv_state"].copy()
        ref["out"] = got["out"].copy()


# --------------------------------------------------------------------------
# ragged shapes, padding, out-of-range tables, bias


def test_ragged_decode_with_padding(gpu):
    p = inputs.make_problem(dict(B=7, H=3, T=1, N=20, W=3, seed=101))
    p["slots"][[1, 4]] = [0, -3]
    p["slots"][5] = p["N"] + 2  # beyond the pool: treated as padding
    check(gpu, p, "ragged decode")


@pytest.mark.parametrize("T", [2, 3, 5, 6, 7, 8])
def test_ragged_verify(gpu, T):
    B, H = 5, 3
    p = inputs.make_problem(dict(B=B, H=H, T=T, N=B * T + 1, W=T + 3, seed=200 + T))
    p["slots"][1, T - 1] = 0      # a skipped write target
    p["accepted"][2] = T + 1      # out of range: padding
    p["slots"][3, 0] = -1         # convolution slot out of range: padding
    check(gpu, p, f"ragged verify T={T}")


@pytest.mark.parametrize("T", [2, 3, 5, 8])
def test_record_ragged(gpu, T):
    B, H = 4, 5
    p = inputs.make_problem(dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=300 + T, record=1))
    p["accepted"][2] = 0          # padding in record mode leaves the records untouched
    check(gpu, p, f"record T={T}")


@pytest.mark.parametrize("B,H,T", [(45, 32, 5), (250, 5, 3), (40, 48, 8)])
def test_record_more_items_than_resident(gpu, B, H, T):
    """More items than record workgroups resident at once (4 per CU, 1024
    on 256 CUs): the items past the first round run on workgroups started
    as earlier ones finish; padding in both rounds (items numbered
    b * H + h)."""
    p = inputs.make_problem(dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=330 + T, record=1))
    p["accepted"][3] = 0              # first round
    p["accepted"][B - 5] = T + 1      # second round
    p["slots"][B - 2, 0] = -1         # second round: convolution slot out of range
    p["slots"][B - 1, T - 1] = 0      # an unused entry of the row (record mode writes no page)
    check(gpu, p, f"record B={B} H={H} T={T}")


@pytest.mark.parametrize("B,T,record", [(3, 1, 0), (5, 1, 0), (3, 4, 0), (5, 8, 0), (5, 8, 1),
                                         (3, 3, 1)])
def test_many_heads(gpu, B, T, record):
    # H = 128: 16384 channels per row of x, gate and out, 49152 convolution
    # channels; 384 items run the latency kernel, 640 the full-occupancy one
    # (record mode: the closed-form kernel at either size)
    H = 128
    cfg = dict(B=B, H=H, T=T, N=B * T + 2, W=T + 2 if T > 1 else 3, seed=700 + B + T,
               record=record)
    p = inputs.make_problem(cfg)
    if B > 3:
        if T == 1:
            p["slots"][1] = 0
        else:
            p["accepted"][1] = 0
    check(gpu, p, f"many heads B={B} T={T} record={record}")


@pytest.mark.parametrize("T,record", [(1, 0), (4, 0), (8, 1)])
def test_deterministic(gpu, T, record):
    # no atomics and no order that depends on timing: the same inputs give
    # the same bits on every launch (640 items: the full-occupancy kernels)
    cfg = dict(B=20, H=32, T=T, N=20 * T + 1, W=T + 2 if T > 1 else 3, seed=900 + T,
               record=record)
    p = inputs.make_problem(cfg)
    say(f"[determinism] T={T} record={record}")
    a = gpu_step(gpu, copy_problem(p))
    b = gpu_step(gpu, copy_problem(p))
    for k in ("state", "conv_state", "out", "rec_u", "rec_kg"):
        if a[k] is not None:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_replay_deterministic(gpu):
    import torch

    r = inputs.make_replay_problem(dict(B=20, H=32, T=8, N=41, seed=905))
    say("[determinism] replay")
    got = []
    for _ in range(2):
        d = gpu.to_device(copy_problem(r))
        gpu.run_replay(d)
        torch.cuda.synchronize()
        got.append(d["state"].cpu().numpy())
    assert np.array_equal(got[0].view(np.uint8), got[1].view(np.uint8))


def test_largest_grid(gpu):
    # B*H = 2^24 - 1 items (H = 1): the largest grid the host checks accept
    # (B*H*256 work-items below 2^32).  One live request near the end of
    # the grid on slot 1 of a 2-slot pool, every other request padding;
    # operands (~26 GB) are made on the device.  The live item is compared
    # with the oracle on that request alone (items are independent), every
    # other output row must be +0.
    import torch

    from linear_attention_decode_03_amd import kda

    B, live = (1 << 24) - 1, (1 << 24) - 5
    small = inputs.make_problem(dict(B=1, H=1, T=1, N=2, W=3, seed=1201))
    before = copy_problem(small)
    ref = copy_problem(small)
    taps = oracle.run(ref, taps=True)
    d = gpu.to_device(small)
    say(f"[largest grid] B={B} H=1, live request {live}")
    big = {}
    for k in ("x", "f_a", "beta", "gate"):
        t = d[k]
        big[k] = torch.zeros((B,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
        big[k][live] = t[0]
    slots = torch.zeros(B, dtype=torch.int32, device="cuda")
    slots[live] = 1
    out = torch.full((B, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    kda.kda_decode(big["x"], d["conv_w"], d["conv_b"], d["conv_state"], big["f_a"], big["beta"],
                   d["a_log"], d["dt_bias"], slots, d["state"], out, big["gate"], d["norm_w"],
                   small["lower_bound"], small["scale"], small["eps"], d["f_b"])
    torch.cuda.synchronize()
    got = gpu.to_host(dict(state=d["state"], conv_state=d["conv_state"], out=out[live:live + 1],
                           rec_u=None, rec_kg=None))
    _parity.compare_step(before, ref, got, taps)
    bits = out.view(torch.int16)
    bits[live] = 0
    assert int(torch.count_nonzero(bits)) == 0, "a padded row is not +0"
    del big, slots, out, bits
    torch.cuda.empty_cache()


def test_conv_bias(gpu):
    for T in (1, 4):
        cfg = dict(B=3, H=2, T=T, N=3 * T + 2, W=T + 2, seed=400 + T)
        p = inputs.make_problem(cfg)
        rng = np.random.default_rng(7)
        p["conv_b"] = to_bf16(rng.standard_normal(3 * p["H"] * 128).astype(np.float32) * 0.3)
        p["has_bias"] = 1
        check(gpu, p, f"bias T={T}")


# --------------------------------------------------------------------------
# FP32 convolution pool (kda_decode_f32conv / kda_verify_f32conv)


@pytest.mark.parametrize("name", ["decode_b256", "verify_t4", "verify_record_t8"])
def test_conv_f32_parity(gpu, name):
    """Full-size workloads with the convolution pool in FP32 (taps not BF16
    values): windows bit-exact, the rest under the same contract."""
    p = inputs.make_problem(name, conv_f32=1)
    assert p["conv_state"].dtype == np.float32
    check(gpu, p, f"{name} conv_f32")


@pytest.mark.parametrize("T", [1, 3, 8])
def test_conv_f32_ragged_bias(gpu, T):
    B, H = 5, 3
    cfg = dict(B=B, H=H, T=T, N=B * T + 2, W=T + 3, seed=600 + T, conv_f32=1,
               record=int(T == 8))
    p = inputs.make_problem(cfg)
    rng = np.random.default_rng(8)
    p["conv_b"] = to_bf16(rng.standard_normal(3 * H * 128).astype(np.float32) * 0.3)
    p["has_bias"] = 1
    if T == 1:
        p["slots"][2] = 0
    else:
        p["accepted"][1] = T + 1  # padding
    check(gpu, p, f"conv_f32 bias T={T}")


@pytest.mark.parametrize("name,ahead", [("decode_b256", 256), ("verify_t4", 64),
                                        ("decode_b64", 1024), ("verify_record_t8", 8)])
def test_prefetch_parity(gpu, name, ahead):
    """With the prefetch on, the step matches the oracle (the full workload,
    every item compared)."""
    check(gpu, inputs.make_problem(name), f"{name} ahead={ahead}", ahead=ahead)


@pytest.mark.parametrize("name", ["decode_b64", "verify_t4", "verify_record_t8"])
def test_prefetch_changes_nothing(gpu, name):
    """The prefetch distance is a hint: every value gives identical bits."""
    p = inputs.make_problem(name)
    say(f"[prefetch] {name}")
    base = gpu_step(gpu, copy_problem(p), ahead=0)
    for ahead in (8, 100, 1024, 2**31 - 1):   # the last: beyond any grid
        got = gpu_step(gpu, copy_problem(p), ahead=ahead)
        for k in ("state", "conv_state", "out", "rec_u", "rec_kg"):
            if base[k] is not None:
                assert np.array_equal(base[k].view(np.uint8), got[k].view(np.uint8)), (ahead, k)


def test_empty_batch(gpu):
    import torch

    p = inputs.make_problem(dict(B=0, H=2, T=1, N=3, W=3, seed=1))
    before = copy_problem(p)
    got = gpu_step(gpu, p)
    assert np.array_equal(got["state"], before["state"])
    assert np.array_equal(got["conv_state"], before["conv_state"])
    torch.cuda.synchronize()


def test_contract_errors_raise(gpu):
    p = inputs.make_problem(dict(B=2, H=2, T=2, N=5, W=4, seed=3))
    d = gpu.to_device(p)
    with pytest.raises(ValueError):
        d2 = dict(d)
        d2["gate_mode"] = 2
        gpu.run(d2)
    with pytest.raises(ValueError):
        d2 = dict(d)
        d2["W"] = 3
        d2["conv_state"] = d["conv_state"][:, :, :3].contiguous()
        gpu.run(d2)   # W < T + 2


@pytest.mark.parametrize("name,shift", [("state", 1), ("f_a", 2), ("x", 1)])
def test_misaligned_operand_raises(gpu, name, shift):
    """A contiguous view that starts `shift` elements past an aligned address
    (state: 4 bytes off 16; f_a: 4 bytes off 16; x: 2 bytes off 4) is refused
    before any device work: the pools keep their bits."""
    import torch

    p = inputs.make_problem(dict(B=2, H=2, T=1, N=5, W=3, seed=5))
    d = gpu.to_device(p)
    t = d[name]
    buf = torch.empty(t.numel() + shift, dtype=t.dtype, device=t.device)
    mis = buf[shift:].view(t.shape)
    mis.copy_(t)
    state0, conv0 = d["state"].clone(), d["conv_state"].clone()
    d2 = dict(d)
    d2[name] = mis
    with pytest.raises(ValueError, match="aligned"):
        gpu.run(d2)
    torch.cuda.synchronize()
    assert torch.equal(d["state"], state0) and torch.equal(d["conv_state"], conv0)
    assert torch.equal(mis, t)


# --------------------------------------------------------------------------
# the method's invariants, on the GPU


@pytest.mark.parametrize("T", [1, 4])
def test_identity_invariant_gpu(gpu, T):
    """Decay 1 (lower_bound 0) and beta 0: every written page equals the
    page read, bit for bit."""
    cfg = dict(B=4, H=4, T=T, N=4 * T + 2, W=T + 2, seed=500 + T, lower_bound=0.0)
    p = inputs.make_problem(cfg)
    p["beta"][:] = to_bf16(np.full(p["beta"].shape, -200.0, np.float32))
    say(f"[invariant] identity T={T}")
    got = gpu_step(gpu, p)
    for b in range(p["B"]):
        src = p["slots"][b] if T == 1 else p["slots"][b, p["accepted"][b] - 1]
        tgts = [p["slots"][b]] if T == 1 else list(p["slots"][b, :T])
        for tgt in tgts:
            assert np.array_equal(got["state"][tgt].view(np.uint32), p["state"][src].view(np.uint32))


def test_delta_rule_beta_one_gpu(gpu):
    """beta = 1: after the update S^T k_hat = v (k, v from the oracle, which
    the GPU matches bit for bit)."""
    p = inputs.make_problem(dict(B=4, H=4, T=1, N=10, W=3, seed=601))
    p["beta"][:] = to_bf16(np.full(p["beta"].shape, 30.0, np.float32))
    ref = copy_problem(p)
    taps = oracle.run(ref, taps=True)
    say("[invariant] delta rule beta=1")
    got = gpu_step(gpu, p)
    for b in range(p["B"]):
        for h in range(p["H"]):
            S = got["state"][p["slots"][b], h].astype(np.float64)
            k = taps["k"][b, h, 0].astype(np.float64)
            kh = k / np.sqrt((k * k).sum() + 1e-6)
            v = taps["v"][b, h, 0].astype(np.float64)
            u = taps["u"][b, h, 0].astype(np.float64)
            assert np.all(np.abs(S @ kh - v) <= 1e-5 * (np.abs(v) + np.abs(u) + 1e-3))


@pytest.mark.parametrize("T", [2, 4, 8])
def test_verify_equals_chained_decode_gpu(gpu, T):
    """A T-token verify (accepted = 1) equals T chained decodes, on the GPU."""
    import torch

    B, H = 3, 4
    p = inputs.make_problem(dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=700 + T))
    p["accepted"][:] = 1
    say(f"[invariant] verify vs chained decode T={T}")
    got_v = gpu_step(gpu, p)
    chain = dict(p)
    chain.update(T=1, W=3, slot_stride=1, record=0, accepted=None, rec_u=None, rec_kg=None)
    chain["slots"] = np.ascontiguousarray(p["slots"][:, 0])
    chain["conv_state"] = np.ascontiguousarray(p["conv_state"][:, :, :3])
    d = gpu.to_device(chain)
    for t in range(T):
        rows = torch.as_tensor(np.arange(B) * T + t, device="cuda")
        step = dict(d)
        for key in ("x", "f_a", "beta", "gate"):
            step[key] = d[key][rows].contiguous()
        step["out"] = torch.zeros((B, H * 128), dtype=torch.bfloat16, device="cuda")
        gpu.run(step)
        torch.cuda.synchronize()
        out_t = step["out"].view(torch.int16).cpu().numpy().view(np.uint16)
        st = d["state"].cpu().numpy()
        for b in range(B):
            r = st[chain["slots"][b]].astype(np.float64)
            g = got_v["state"][p["slots"][b, t]].astype(np.float64)
            rms = np.sqrt((r * r).mean())
            assert np.all(np.abs(g - r) <= 1e-5 * (np.abs(r) + rms))
        o_r = inputs.from_bf16(out_t).astype(np.float64)
        o_g = inputs.from_bf16(got_v["out"][np.arange(B) * T + t]).astype(np.float64)
        assert np.all(np.abs(o_g - o_r) <= 2 * _parity.ulp_bf16(np.maximum(np.abs(o_r), 1e-3)))
    conv = d["conv_state"].view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        cs = chain["slots"][b]
        assert np.array_equal(got_v["conv_state"][cs][:, T - 1:T + 2], conv[cs])


def test_gate_modes_agree_gpu(gpu):
    """gate_mode selects the accumulation structure; the projection is exact
    here, so both modes give identical bits."""
    p = inputs.make_problem(dict(B=6, H=4, T=3, N=19, W=5, seed=801))
    say("[gate_mode] 0 vs 1")
    a = gpu_step(gpu, copy_problem(p))
    p["gate_mode"] = 1
    b = gpu_step(gpu, p)
    for k in ("state", "conv_state", "out"):
        assert np.array_equal(a[k], b[k])


@pytest.mark.parametrize("T,record,gate_mode", [(1, 0, 0), (1, 0, 1), (4, 0, 0), (4, 0, 1),
                                                 (8, 1, 0), (8, 1, 1)])
def test_gate_sum_exact_on_cancelling_rows_gpu(gpu, T, record, gate_mode):
    """Kernel body, gate projection: raw_g is the exact sum rounded once to
    FP32, then to BF16.  With F_B rows 2^20, 1, 2^-8, 2^-20, -2^20 and
    f_a = 1 every feature's exact raw_g is 1 + 2^-7, while an FP32 running
    sum ends at 1: the decay then differs by far more than the state
    tolerance, and in record mode the stored raw_g is compared bit for bit."""
    cfg = dict(B=4, H=2, T=T, N=4 * T + 3, W=T + 2, seed=811, record=record,
               gate_mode=gate_mode)
    p = inputs.make_problem(cfg)
    p["f_b"] = _parity.cancelling_gate_rows(p["H"], 128, 5)
    p["f_a"][:] = to_bf16(np.float32(1.0))
    rep, got, ref = check(gpu, p, f"cancelling gate T={T} record={record} mode={gate_mode}")
    if record:
        g = got["rec_kg"][..., 128:].transpose(0, 2, 1, 3)  # [B, T, H, 128]
        live = np.arange(T)[None, :] < p["accepted"][:, None]
        assert np.all(g[live] == to_bf16(np.float32(1.0 + 2.0 ** -7)))


@pytest.mark.parametrize("T,record,kind", [(1, 0, "overflow"), (4, 0, "overflow"),
                                            (8, 1, "overflow"), (3, 1, "tiny"), (8, 1, "tiny")])
def test_gate_products_beyond_fp32_gpu(gpu, T, record, kind):
    """Kernel body, gate projection: every product exact, also where FP32
    would overflow (2^140 - 2^140 + 0.5: raw_g 0.5, seen through the
    decay by the state) or underflow (a sum just off a BF16 midpoint at
    2^-120, seen in record mode's stored raw_g)."""
    B, H = 3, 2
    if T == 1:
        cfg = dict(B=B, H=H, T=1, N=2 * B + 2, W=3, seed=821)
    else:
        cfg = dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=822 + T, record=record)
    p = inputs.make_problem(cfg)
    p["f_b"], fa = _parity.wide_range_gate_operands(H, 128, kind)
    p["f_a"][:] = fa
    rep, got, ref = check(gpu, p, f"wide-range gate {kind} T={T} record={record}")
    if record:
        want = 0.5 if kind == "overflow" else 2.0 ** -120 + 2.0 ** -127
        g = got["rec_kg"][..., 128:].transpose(0, 2, 1, 3)  # [B, T, H, 128]
        live = np.arange(T)[None, :] < p["accepted"][:, None]
        assert np.all(g[live] == to_bf16(np.float32(want)))


def test_record_matches_plain_gpu(gpu):
    """Record mode (closed-form kernel) and a plain verify of the same inputs
    both match the oracle; record mode writes no state page, leaves the same
    convolution windows, and its records replay to the plain states."""
    T = 4
    p = inputs.make_problem(dict(B=5, H=4, T=T, N=21, W=6, seed=901, record=1))
    plain = copy_problem(p)
    plain.update(record=0, rec_u=None, rec_kg=None)
    say("[record] vs plain")
    rep_r, r, _ = check(gpu, copy_problem(p), "record T=4")
    rep_q, q, _ = check(gpu, plain, "plain T=4")
    assert np.array_equal(r["conv_state"], q["conv_state"])
    assert np.array_equal(r["state"].view(np.uint32), p["state"].view(np.uint32))
    for b in range(p["B"]):
        for h in range(p["H"]):
            S = p["state"][p["slots"][b, p["accepted"][b] - 1], h].astype(np.float64)
            dt = p["dt_bias"][h * 128:(h + 1) * 128]
            for t in range(T):
                k = inputs.from_bf16(r["rec_kg"][b, h, t, :128]).astype(np.float64)
                g = inputs.from_bf16(r["rec_kg"][b, h, t, 128:])
                a = np.array([oracle.decay(float(p["a_log"][h]), float(g[f]), float(dt[f]),
                                           p["lower_bound"]) for f in range(128)])
                kh = k / np.sqrt((k * k).sum() + 1e-6)
                S = S * a[None, :] + np.outer(r["rec_u"][b, h, t].astype(np.float64), kh)
                ref = q["state"][p["slots"][b, t], h].astype(np.float64)
                rms = np.sqrt((ref ** 2).mean())
                assert np.all(np.abs(S - ref) <= 1e-4 * (np.abs(ref) + rms))


@pytest.mark.parametrize("lb", [-12.0, 10.0, -10.0])
def test_record_decay_bound_paths(gpu, lb):
    """|lower_bound| > 10 takes the token-by-token record kernel, <= 10 the
    closed-form one; both match the oracle (10 is the edge of the closed form)."""
    T = 8
    p = inputs.make_problem(dict(B=6, H=3, T=T, N=49, W=10, seed=950, record=1,
                                 lower_bound=lb))
    check(gpu, p, f"record lower_bound={lb}")


def test_silu_every_bf16_input_gpu(gpu):
    """The kernel's SiLU (fast FP32 path with a rounding-boundary test, FP64
    otherwise) against the oracle's, for every finite BF16 convolution sum:
    tap weights [0, 0, 0, 1] make the k-channel sum equal x exactly, and
    record mode stores k."""
    B, H, T = 64, 4, 8
    p = inputs.make_problem(dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=960, record=1))
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    vals = bits[finite]
    dim = H * 128
    n = B * T * dim
    xk = np.resize(vals, n).reshape(B * T, dim)
    p["x"][:, dim:2 * dim] = xk
    p["conv_w"][1] = to_bf16(np.array([0, 0, 0, 1], np.float32))[:, None]
    say(f"[silu] {vals.size} BF16 inputs")
    got = gpu_step(gpu, p)
    k_gpu = got["rec_kg"][..., :128]                                    # [B, H, T, 128]
    xs = inputs.from_bf16(xk).reshape(B, T, H, 128).transpose(0, 2, 1, 3)
    # The convolution's FP32 sum fma(x, 1, +0) is x, except that -0 becomes +0.
    sums = inputs.from_bf16(vals) + np.float32(0.0)
    want = np.array([oracle.silu_bf16(float(x)) for x in sums], dtype=np.float32)
    lut = dict(zip(vals.tolist(), to_bf16(want).tolist()))
    xb = xk.reshape(B, T, H, 128).transpose(0, 2, 1, 3)
    ref = np.vectorize(lut.__getitem__, otypes=[np.uint16])(xb)
    bad = np.nonzero(k_gpu != ref)
    assert bad[0].size == 0, (f"{bad[0].size} SiLU mismatches, first x="
                              f"{xs[tuple(d[0] for d in bad)]}")


def test_nondefault_stream(gpu):
    import torch

    p = inputs.make_problem(dict(B=4, H=8, T=1, N=9, W=3, seed=1001))
    before = copy_problem(p)
    ref = copy_problem(p)
    taps = oracle.run(ref, taps=True)
    s = torch.cuda.Stream()
    d = gpu.to_device(p)
    torch.cuda.synchronize()
    say("[stream] non-default stream")
    with torch.cuda.stream(s):
        gpu.run(d, stream=s)
    s.synchronize()
    _parity.compare_step(before, ref, gpu.to_host(d), taps)


_LOAD_FIRST = r"""
import sys
sys.path.insert(0, {root!r})
from linear_attention_decode_03_amd import kda
kda.load_library()          # before the caller has imported torch
import numpy as np
import torch
from linear_attention_decode_03_amd import inputs
from tests import _gpu
p = inputs.make_problem(dict(B=3, H=4, T=4, N=13, W=6, seed=1003))
d = _gpu.to_device(p)
s = torch.cuda.Stream()
torch.cuda.synchronize()
with torch.cuda.stream(s):
    _gpu.run(d, stream=s)
s.synchronize()
h = _gpu.to_host(d)
np.savez({out!r}, **{{k: v for k, v in h.items() if v is not None}})
print("done", flush=True)
"""


def test_library_loaded_before_torch(gpu, tmp_path):
    # A fresh process that loads the library before importing torch, then
    # launches a verify step on a torch stream: the library must share
    # torch's HIP runtime (one runtime in the process), so the launch runs.
    import os
    import subprocess

    out = str(tmp_path / "load_first.npz")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("[load-first] subprocess: library loaded before torch, verify T=4 on a torch stream")
    r = subprocess.run([sys.executable, "-c", _LOAD_FIRST.format(root=root, out=out)],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-1000:] + r.stderr[-2000:]
    p = inputs.make_problem(dict(B=3, H=4, T=4, N=13, W=6, seed=1003))
    before = copy_problem(p)
    ref = copy_problem(p)
    taps = oracle.run(ref, taps=True)
    got = dict(np.load(out))
    for k in ("rec_u", "rec_kg"):
        got.setdefault(k, None)
    _parity.compare_step(before, ref, got, taps)


# --------------------------------------------------------------------------
# HIP graph capture: a decode and a verify step recorded once, replayed


def test_graph_capture_replays_match_eager(gpu):
    """The entry points enqueue on the caller's stream and allocate nothing,
    so a decode + verify pair can be captured in a HIP graph and replayed.
    Every replay (with unrelated eager work and synchronisations between
    them) must give the eager launches' bits."""
    import torch

    dec = inputs.make_problem("decode_b64")
    ver = inputs.make_problem(dict(B=16, H=32, T=4, N=65, W=6, seed=41))
    eager = [gpu.to_device(copy_problem(dec)), gpu.to_device(copy_problem(ver))]
    graphed = [gpu.to_device(copy_problem(dec)), gpu.to_device(copy_problem(ver))]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for d in graphed:
            gpu.run(d)
    torch.cuda.synchronize()
    for k in range(4):
        say(f"[graph] replay {k}")
        for d in eager:
            gpu.run(d)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        scratch = torch.arange(1 << 20, device="cuda", dtype=torch.float32)
        assert float(scratch.sum()) > 0
        for e, r in zip(eager, graphed):
            he, hr = gpu.to_host(e), gpu.to_host(r)
            for key in ("state", "conv_state", "out"):
                a, b = he[key], hr[key]
                bits = np.uint32 if a.dtype == np.float32 else np.uint16
                assert np.array_equal(a.view(bits), b.view(bits)), (k, key)


def silu_inputs(n, rng):
    """FP32 SiLU arguments: wide random magnitudes, tiny and large values,
    and values whose SiLU lies within a few FP32 ulps of a BF16 rounding
    midpoint (found by Newton steps in float64 from random midpoints)."""
    parts = [rng.standard_normal(n // 5) * 3.0,
             rng.uniform(-90.0, 90.0, n // 5),
             np.sign(rng.standard_normal(n // 10)) * 10.0 ** rng.uniform(-38, 1.9, n // 10)]
    # near-midpoint arguments
    m = n - sum(len(q) for q in parts)
    hb = rng.integers(0, 1 << 16, size=m).astype(np.uint32)
    hb = hb[((hb & 0x7F80) != 0x7F80) & ((hb & 0x7F80) > 0x0000)]
    lo = (hb << 16).view(np.float32).astype(np.float64)
    spacing = 2.0 ** (np.floor(np.log2(np.abs(lo))) - 7)   # BF16 spacing at lo
    mid = lo + np.sign(lo) * spacing / 2                  # halfway to the next BF16 value
    ok = (mid > -0.278) & (np.abs(mid) < 80.0)             # SiLU's range
    mid = mid[ok]
    x = np.where(mid > 0, mid + 0.3, -0.5 + 0 * mid)
    for _ in range(60):
        e = np.exp(-x)
        f = x / (1.0 + e) - mid
        df = (1.0 + e + x * e) / (1.0 + e) ** 2
        x = x - f / np.where(np.abs(df) < 1e-30, 1e-30, df)
    x = x[np.isfinite(x)].astype(np.float32)
    step = rng.integers(-3, 4, size=x.size).astype(np.int32)
    x = (x.view(np.int32) + step).view(np.float32)
    parts.append(x.astype(np.float64))
    v = np.concatenate(parts).astype(np.float32)
    return v[np.isfinite(v) & (np.abs(v) < 3.0e38)]


def test_silu_fp32_inputs_gpu(gpu):
    """The kernel's SiLU against the oracle's for ~2 M FP32 arguments,
    including arguments whose SiLU sits next to a BF16 rounding midpoint:
    an FP32 convolution pool with k tap weights [1, 0, 0, 0] makes the
    convolution sum of token t the pool's tap t exactly, and record mode
    stores BF16(silu(tap))."""
    B, H, T = 1024, 8, 2
    rng = np.random.default_rng(970)
    p = inputs.make_problem(dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=970, record=1,
                                 conv_f32=1))
    dim = H * 128
    p["accepted"][:] = 1                       # window taps at columns 0, 1, 2
    vals = silu_inputs(B * H * 128 * T, rng)
    say(f"[silu32] {vals.size} FP32 inputs")
    cs = p["slots"][:, 0]
    k = np.resize(vals, B * H * 128 * T).reshape(B, H, 128, T)
    pool = p["conv_state"]
    for t in range(T):
        pool[cs, dim:2 * dim, t] = k[..., t].reshape(B, dim)
    p["conv_w"][1] = to_bf16(np.array([1, 0, 0, 0], np.float32))[:, None]
    got = gpu_step(gpu, p)
    k_gpu = got["rec_kg"][..., :128]                       # [B, H, T, 128]
    xs = k.transpose(0, 1, 3, 2)                           # [B, H, T, 128]
    # fma(tap, 1, +0) is the tap, except that -0 becomes +0
    flat = (xs + np.float32(0.0)).reshape(-1)
    want = to_bf16(np.array([oracle.silu_bf16(float(x)) for x in flat], dtype=np.float32))
    bad = np.nonzero(k_gpu.reshape(-1) != want)[0]
    assert bad.size == 0, f"{bad.size} SiLU mismatches, first x={flat[bad[0]]!r}"


# --------------------------------------------------------------------------
# slot tables wider than T, pools beyond 4 GiB


def test_slot_stride_wider_than_tokens(gpu):
    """slot_stride 7 for T = 4: the read slot is slots[b, accepted - 1] with
    accepted <= 4, the write targets are the first 4 columns, and the pages
    of columns 4-6 are untouched."""
    B, H, T, S = 6, 4, 4, 7
    p = inputs.make_problem(dict(B=B, H=H, T=T, N=B * S + 1, W=T + 2, seed=1100, slot_stride=S))
    assert p["slots"].shape == (B, S)
    check(gpu, p, "slot_stride 7, T 4")


@pytest.mark.parametrize("T", [1, 2])
def test_pool_beyond_4gib(gpu, T):
    """A 4.4 GB state pool (2100 slots x 32 heads x 64 KiB) with the live
    pages at the top slots, so every page offset exceeds 2^32 bytes; the
    rest of the pool is zero and must stay so."""
    B, H, N = 8, 32, 2100
    small = inputs.make_problem(dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=1200 + T))
    p = dict(small)
    p["N"] = N
    remap = np.zeros(small["N"], np.int32)
    remap[1:] = np.arange(N - small["N"] + 1, N, dtype=np.int32)  # slot s -> N - small_N + s
    p["slots"] = np.where(small["slots"] > 0, remap[np.maximum(small["slots"], 0)], small["slots"])
    p["slots"] = np.ascontiguousarray(p["slots"].astype(np.int32))
    state = np.zeros((N, H, 128, 128), np.float32)
    state[remap[1:]] = small["state"][1:]
    p["state"] = state
    conv = np.zeros((N,) + small["conv_state"].shape[1:], small["conv_state"].dtype)
    conv[remap[1:]] = small["conv_state"][1:]
    p["conv_state"] = conv
    assert (int(p["slots"].min()) * H) * 65536 >= 1 << 32
    say(f"[4gib] T={T} pool {state.nbytes / 2**30:.1f} GiB")
    check(gpu, p, f"pool beyond 4 GiB, T={T}")


# --------------------------------------------------------------------------
# a seeded sweep of small random configurations over every axis


def random_configs(n=36, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 9))
        B = int(rng.integers(1, 9))
        H = int(rng.choice([1, 2, 3, 5, 7, 8, 12]))
        record = int(T > 1 and rng.random() < 0.35)
        stride = T if T == 1 else T + int(rng.integers(0, 3))
        W = (3 if T == 1 else T + 2) + int(rng.integers(0, 3))
        cfg = dict(B=B, H=H, T=T, W=W, seed=3000 + i, record=record,
                   gate_mode=int(rng.integers(0, 2)), conv_f32=int(rng.random() < 0.3),
                   lower_bound=float(rng.choice([-5.0, -5.0, -1.0, -9.5, -12.0, 0.0])))
        if T > 1:
            cfg["slot_stride"] = stride
            cfg["N"] = B * stride + 1 + int(rng.integers(0, 5))
        else:
            cfg["N"] = B + 1 + int(rng.integers(0, 5))
        out.append((cfg, bool(rng.random() < 0.3), bool(rng.random() < 0.3)))
    return out


@pytest.mark.parametrize("k", range(36))
def test_random_small_configs(gpu, k):
    cfg, bias, pad = random_configs()[k]
    p = inputs.make_problem(cfg)
    rng = np.random.default_rng(cfg["seed"])
    if bias:
        p["conv_b"] = to_bf16(rng.standard_normal(3 * p["H"] * 128).astype(np.float32) * 0.3)
        p["has_bias"] = 1
    if pad and p["B"] > 1:
        b = int(rng.integers(0, p["B"]))
        if p["T"] == 1:
            p["slots"][b] = 0
        else:
            p["accepted"][b] = 0
            if p["B"] > 2:       # and a skipped write target elsewhere
                p["slots"][(b + 1) % p["B"], p["T"] - 1] = 0
    check(gpu, p, f"random {k}: {cfg} bias={bias} pad={pad}")


# --------------------------------------------------------------------------
# the two launch shapes of the step: up to 512 items every workgroup is
# resident at 2 per CU and the latency kernel runs (all operands ahead of the
# page); above, the full-occupancy kernel


def _request_slice(d, lo, hi):
    """The device operands of requests lo .. hi-1 (views; pools and weights shared)."""
    T = d["T"]
    out = dict(d)
    for k in ("x", "f_a", "beta", "gate", "out"):
        out[k] = d[k][lo * T:hi * T]
    for k in ("slots", "accepted", "rec_u", "rec_kg"):
        if d.get(k) is not None:
            out[k] = d[k][lo:hi]
    return out


@pytest.mark.parametrize("T,record,conv_f32,lower_bound", [
    (1, 0, 0, -5.0), (2, 0, 0, -5.0), (3, 0, 1, -5.0), (5, 0, 0, -5.0), (6, 0, 0, -5.0),
    (7, 0, 1, -5.0), (8, 0, 0, -5.0), (8, 1, 0, -12.0), (4, 1, 0, -5.0), (8, 1, 1, -5.0)])
def test_full_occupancy_kernel_and_latency_kernel(gpu, T, record, conv_f32, lower_bound):
    """B*H = 640 items: the full-occupancy kernel against the oracle, then the
    same requests as two calls of 320 items each (the latency kernel) must
    leave every pool, output and record bit for bit as the single call did
    (the gate projection is exact in both, every other operation the same).
    Record mode with lower_bound -12 takes the token-by-token path, with -5
    the closed-form record kernel."""
    import torch

    cfg = dict(B=40, H=16, T=T, W=3 if T == 1 else T + 2, seed=4100 + 10 * record + T,
               record=record, conv_f32=conv_f32, lower_bound=lower_bound)
    if T > 1:
        cfg.update(slot_stride=T, N=40 * T + 3)
    else:
        cfg.update(N=43)
    p = inputs.make_problem(cfg)
    if T > 1:
        p["accepted"][3] = 0      # a padded request in each half
        p["accepted"][27] = 0
    else:
        p["slots"][3] = 0
        p["slots"][27] = 0
    check(gpu, p, f"full occupancy T={T} record={record} conv_f32={conv_f32} lb={lower_bound}")

    one = gpu.to_device(p)
    gpu.run(one)
    two = gpu.to_device(p)
    gpu.run(_request_slice(two, 0, 20))
    gpu.run(_request_slice(two, 20, 40))
    torch.cuda.synchronize()
    a, b = gpu.to_host(one), gpu.to_host(two)
    for k in ("state", "conv_state", "out", "rec_u", "rec_kg"):
        if a[k] is None:
            continue
        va, vb = a[k].view(np.uint8), b[k].view(np.uint8)
        assert np.array_equal(va, vb), f"{k}: the latency kernel differs from the full-occupancy kernel"
