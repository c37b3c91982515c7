"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Sources: the vLLM API page vllm.models.kimi_k3.nvidia.specialized_decode.
cutedsl.kda.wide (class KdaWide: docstring, constructor, kernel body, helpers
silu and decay).  The page prints no worked example, so the pins are
invariants, closed forms, special cases and an independent float64 matrix
formulation.  Which step each pin covers:

  slot resolution, padding ............ test_padding_*, test_contract_errors
  convolution (tap order, window) ..... test_conv_tap_selection, test_conv_window_update
  FP32 convolution pool ............... the same two with conv_f32, test_conv_f32_reduces_to_bf16
  SiLU stage .......................... test_silu_textbook
  L2 norm, q/k roles, o = S^T q ....... test_zero_state_closed_form, test_delta_rule_*
  gate projection (indexing) .......... test_gate_one_hot
  decay (formula, per-key axis) ....... test_decay_golden, test_decay_through_state
  beta = sigmoid(logit) ............... test_identity_invariant, test_zero_state_closed_form
  recurrence order and orientation .... test_delta_rule_*, test_zero_state_closed_form
  verify slots / per-token writes ..... test_verify_equals_chained_decode
  record outputs ...................... test_record_replay
  RecoverSSM replay ................... test_replay_*
  gated RMSNorm ....................... test_rmsnorm_closed_form, test_zero_state_closed_form
  everything together ................. test_matrix_form_cross_check
"""

import math
import os

import numpy as np
import pytest

from linear_attention_decode_03_amd import inputs
from linear_attention_decode_03_amd.inputs import from_bf16, to_bf16

from . import _matrix_form, _parity

D = 128
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LOGIT_ONE = 30.0     # sigmoid(30) rounds to 1.0 in FP32
LOGIT_ZERO = -200.0  # sigmoid(-200) rounds to 0.0 in FP32


def small(T=1, B=3, H=2, seed=11, **kw):
    if T == 1:
        cfg = dict(B=B, H=H, T=1, N=2 * B + 2, W=3, seed=seed)
    else:
        cfg = dict(B=B, H=H, T=T, N=B * T + 1, W=T + 2, seed=seed)
    cfg.update(kw)
    return inputs.make_problem(cfg)


def read_slot(p, b):
    return int(p["slots"][b]) if p["T"] == 1 else int(p["slots"][b, p["accepted"][b] - 1])


def bf16_of_f64(x):
    """FP32 value of a float64, then BF16 (the page's rounding points)."""
    return from_bf16(to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32)))


def silu64(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def set_conv_taps(p, part, taps):
    """Sets the 4 convolution weights of one part (0 q, 1 k, 2 v) for every channel."""
    p["conv_w"][part] = to_bf16(np.asarray(taps, dtype=np.float32))[:, None]


# --------------------------------------------------------------------------
# contract and padding


def test_contract_errors(oracle_lib):
    p = small()
    for T, rec, gm in ((0, 0, 0), (9, 0, 0), (1, 0, 2), (1, 1, 0)):
        q = inputs.copy_problem(p)
        q["T"], q["record"], q["gate_mode"] = T, rec, gm
        with pytest.raises(ValueError):
            oracle_lib.run(q)


def test_padding_leaves_everything_but_zero_output(oracle_lib):
    p = small(B=5)
    p["slots"][1] = 0
    p["slots"][3] = -7
    before = inputs.copy_problem(p)
    oracle_lib.run(p)
    for b in (1, 3):
        assert np.all(p["out"][b] == 0)  # +0 in BF16, bit-exact
    for b in (0, 2, 4):
        assert not np.any(p["out"][b] == inputs.BF16_SENTINEL)
        s = int(p["slots"][b])
        assert not np.array_equal(p["state"][s], before["state"][s])
    live = {int(p["slots"][b]) for b in (0, 2, 4)}
    for s in range(p["N"]):
        if s not in live:
            assert np.array_equal(p["state"][s], before["state"][s])
            assert np.array_equal(p["conv_state"][s], before["conv_state"][s])


def test_padding_verify_per_token_target(oracle_lib):
    """A verify target <= 0 skips only that token's state write."""
    p = small(T=3, B=2)
    p["accepted"][:] = 1
    skipped = int(p["slots"][0, 1])
    p["slots"][0, 1] = 0
    before = inputs.copy_problem(p)
    oracle_lib.run(p)
    assert np.array_equal(p["state"][skipped], before["state"][skipped])
    assert np.array_equal(p["state"][0], before["state"][0])
    for t in (0, 2):
        s = int(p["slots"][0, t])
        assert not np.array_equal(p["state"][s], before["state"][s])


# --------------------------------------------------------------------------
# invariant (1): decay = 1 and beta = 0 leave the state unchanged


@pytest.mark.parametrize("T", [1, 4])
def test_identity_invariant(oracle_lib, T):
    p = small(T=T, lower_bound=0.0)
    p["beta"][:] = to_bf16(np.full(p["beta"].shape, LOGIT_ZERO, np.float32))
    before = inputs.copy_problem(p)
    oracle_lib.run(p)
    for b in range(p["B"]):
        src = before["state"][read_slot(before, b)]
        targets = [int(p["slots"][b])] if T == 1 else [int(s) for s in p["slots"][b, :T]]
        for tgt in targets:
            assert np.array_equal(p["state"][tgt].view(np.uint32), src.view(np.uint32))


# --------------------------------------------------------------------------
# invariant (2) and the textbook delta-rule recall


def test_delta_rule_beta_one(oracle_lib):
    """beta = 1: after the update S^T k_hat = v for every value row."""
    p = small(B=4)
    p["beta"][:] = to_bf16(np.full(p["beta"].shape, LOGIT_ONE, np.float32))
    taps = oracle_lib.run(p, taps=True)
    for b in range(p["B"]):
        for h in range(p["H"]):
            S = p["state"][int(p["slots"][b]), h].astype(np.float64)  # [v][k]
            k = taps["k"][b, h, 0].astype(np.float64)
            kh = k / np.sqrt((k * k).sum() + 1e-6)
            v = taps["v"][b, h, 0].astype(np.float64)
            u = taps["u"][b, h, 0].astype(np.float64)
            lhs = S @ kh
            assert np.all(np.abs(lhs - v) <= 1e-5 * (np.abs(v) + np.abs(u) + 1e-3))


def test_delta_rule_recall_one_hot_keys(oracle_lib):
    """Associative-memory recall: with no decay (lb = 0), beta = 1 and
    orthonormal keys e_{j_t}, after T tokens S^T e_{j_t} = v_t for every t."""
    T = 4
    p = small(T=T, B=2, H=2, lower_bound=0.0)
    p["accepted"][:] = 1
    p["beta"][:] = to_bf16(np.full(p["beta"].shape, LOGIT_ONE, np.float32))
    set_conv_taps(p, 1, [0, 0, 0, 1])  # k_t = silu(x_k,t)
    set_conv_taps(p, 2, [0, 0, 0, 1])  # v_t = silu(x_v,t)
    dim = p["H"] * D
    keys = [5, 77, 31, 120]
    for b in range(p["B"]):
        for t in range(T):
            row = p["x"][b * T + t]
            row[dim:2 * dim] = 0
            for h in range(p["H"]):
                row[dim + h * D + keys[t]] = to_bf16(np.float32(3.0)).item()
    before = inputs.copy_problem(p)
    oracle_lib.run(p)
    for b in range(p["B"]):
        for h in range(p["H"]):
            S = p["state"][int(p["slots"][b, T - 1]), h].astype(np.float64)  # [v][k]
            for t in range(T):
                xv = from_bf16(before["x"][b * T + t, 2 * dim + h * D:2 * dim + (h + 1) * D])
                v_t = bf16_of_f64(silu64(xv)).astype(np.float64)
                col = S[:, keys[t]]
                # k_hat_j = s / sqrt(s^2 + 1e-6), 1 - k_hat_j ~ 6e-8
                assert np.allclose(col, v_t, rtol=2e-6, atol=1e-7)


# --------------------------------------------------------------------------
# invariant (3): a T-token verify equals T chained single-token decodes


@pytest.mark.parametrize("T", [2, 4, 8])
def test_verify_equals_chained_decode(oracle_lib, T):
    p = small(T=T, B=3, H=2, seed=20 + T)
    p["accepted"][:] = 1
    B, H = p["B"], p["H"]
    dim = H * D
    chain = dict(p)
    chain.update(T=1, W=3, slot_stride=1, record=0, accepted=None, rec_u=None, rec_kg=None)
    chain["slots"] = np.ascontiguousarray(p["slots"][:, 0])
    chain["state"] = p["state"].copy()
    chain["conv_state"] = np.ascontiguousarray(p["conv_state"][:, :, :3])
    outs = []
    states = []
    for t in range(T):
        rows = np.arange(B) * T + t
        step = dict(chain)
        for key in ("x", "f_a", "beta", "gate"):
            step[key] = np.ascontiguousarray(p[key][rows])
        step["out"] = np.zeros((B, dim), np.uint16)
        oracle_lib.run(step)
        outs.append(step["out"])
        states.append({b: chain["state"][int(chain["slots"][b])].copy() for b in range(B)})
    conv_before = p["conv_state"].copy()
    oracle_lib.run(p)
    for t in range(T):
        assert np.array_equal(p["out"][np.arange(B) * T + t], outs[t])
        for b in range(B):
            got = p["state"][int(p["slots"][b, t])]
            assert np.array_equal(got.view(np.uint32), states[t][b].view(np.uint32))
    for b in range(B):
        cs = int(p["slots"][b, 0])
        assert np.array_equal(p["conv_state"][cs][:, T - 1:T + 2], chain["conv_state"][cs])
    assert conv_before.shape == p["conv_state"].shape


# --------------------------------------------------------------------------
# (5) the decay formula


def test_decay_golden(oracle_lib):
    rows = [line.split() for line in open(os.path.join(GOLDEN, "decay_special_values.txt"))
            if line.strip() and not line.startswith("#")]
    assert len(rows) >= 10
    for a_log, g, dt, lb, hexv in rows:
        got = np.float32(oracle_lib.decay(float(a_log), float(g), float(dt), float(lb)))
        assert got.view(np.uint32) == np.uint32(int(hexv, 16)), (a_log, g, dt, lb)


def test_decay_through_state(oracle_lib):
    """State all ones and beta = 0: the new state holds the decay, identical
    for every value row and varying along the key axis.  F_B rows are one-hot
    through a permutation with no fixed points, so raw_g[f] = f_a[pi(f)]."""
    p = small(B=2, H=2)
    p["beta"][:] = to_bf16(np.full(p["beta"].shape, LOGIT_ZERO, np.float32))
    p["state"][:] = 1.0
    pi = (np.arange(D) * 37 + 11) % D
    fb = np.zeros((p["H"] * D, D), np.float32)
    for h in range(p["H"]):
        fb[h * D + np.arange(D), pi] = 1.0
    p["f_b"] = to_bf16(fb)
    oracle_lib.run(p)
    for b in range(p["B"]):
        for h in range(p["H"]):
            S = p["state"][int(p["slots"][b]), h]
            assert np.all(S == S[0:1, :])          # every value row identical
            fa = from_bf16(p["f_a"][b]).astype(np.float64)
            z = fa[pi] + p["dt_bias"][h * D:(h + 1) * D].astype(np.float64)
            lb = p["lower_bound"]
            y = math.exp(float(p["a_log"][h])) * z
            sig = 1.0 / (1.0 + np.exp(-y))
            a = np.exp(lb * sig)
            # FP32 rounding bound of the five-step chain z, e, y, sigma, g, exp
            # (unit roundoff u): |dy| <= 3u|y|, |ds| <= s(1-s)|dy| + u s,
            # |dg| <= |lb||ds| + u|lb s|, |da|/a <= |dg| + u.
            u = 2.0 ** -24
            ds = sig * (1 - sig) * 3 * u * np.abs(y) + u * sig
            bound = a * (abs(lb) * ds + u * abs(lb) * sig + u)
            assert np.all(np.abs(S[0].astype(np.float64) - a) <= 1.5 * bound + 1e-300)


# --------------------------------------------------------------------------
# convolution, SiLU and gate special cases


def test_silu_textbook(oracle_lib):
    xs = np.concatenate([np.linspace(-12, 12, 2001), [-100.0, -88.0, 0.0, 1e-3, 50.0]])
    xs = from_bf16(to_bf16(xs.astype(np.float32)))  # BF16-exact inputs, as the conv sees
    want = bf16_of_f64(silu64(xs.astype(np.float64)))
    for x, w in zip(xs, want):
        got = oracle_lib.silu_bf16(float(x))
        assert got == float(w) or (math.isnan(got) and math.isnan(w)), x


def pool_values(p, cs, ch, col):
    """FP32 values of convolution-pool entries (BF16 bits or FP32)."""
    v = p["conv_state"][cs][ch, col]
    return v.astype(np.float32) if p.get("conv_f32") else from_bf16(v)


@pytest.mark.parametrize("T,conv_f32", [(1, 0), (3, 0), (1, 1), (3, 1)])
def test_conv_tap_selection(oracle_lib, T, conv_f32):
    """One-hot tap weights select one window entry: weight i selects
    window[t + i] of [conv[off], conv[off+1], conv[off+2], x_0, ..., x_{T-1}].
    With an FP32 pool the taps enter the SiLU unrounded (the pool draws are
    not BF16 values)."""
    p = small(T=T, B=2, H=2, conv_f32=conv_f32)
    if T > 1:
        p["accepted"][:] = [2, 3]
    dim = p["H"] * D
    for tap in range(4):
        q = inputs.copy_problem(p)
        for part in range(3):
            w = [0.0] * 4
            w[tap] = 1.0
            set_conv_taps(q, part, w)
        taps = oracle_lib.run(q, taps=True)
        for b in range(p["B"]):
            off = 0 if T == 1 else int(p["accepted"][b]) - 1
            cs = int(p["slots"][b]) if T == 1 else int(p["slots"][b, 0])
            for h in range(p["H"]):
                for part, name in enumerate(("q", "k", "v")):
                    ch = part * dim + h * D + np.arange(D)
                    window = [pool_values(p, cs, ch, off + i) for i in range(3)]
                    window += [from_bf16(p["x"][b * T + t, ch]) for t in range(T)]
                    for t in range(T):
                        want = bf16_of_f64(silu64(window[t + tap]))
                        assert np.array_equal(taps[name][b, h, t], want)


@pytest.mark.parametrize("conv_f32", [0, 1])
def test_conv_window_update(oracle_lib, conv_f32):
    """Window after the step: [tap1, tap2, x_0, ..., x_{T-1}] in the pool's
    type: taps keep their bits, the BF16 inputs are stored exactly (as BF16
    bits, or as their FP32 values in an FP32 pool)."""
    for T in (1, 3):
        p = small(T=T, B=2, H=1, conv_f32=conv_f32)
        if T > 1:
            p["accepted"][:] = [3, 2]
        before = inputs.copy_problem(p)
        oracle_lib.run(p)
        dim = D
        for b in range(2):
            off = 0 if T == 1 else int(p["accepted"][b]) - 1
            cs = int(p["slots"][b]) if T == 1 else int(p["slots"][b, 0])
            old = before["conv_state"][cs]
            new = p["conv_state"][cs]
            assert np.array_equal(new[:, 0], old[:, off + 1])
            assert np.array_equal(new[:, 1], old[:, off + 2])
            for t in range(T):
                x = before["x"][b * T + t, :3 * dim]
                assert np.array_equal(new[:, 2 + t], from_bf16(x) if conv_f32 else x)
            assert np.array_equal(new[:, 2 + T:], old[:, 2 + T:])


@pytest.mark.parametrize("T", [1, 4])
def test_conv_f32_reduces_to_bf16(oracle_lib, T):
    """An FP32 pool holding BF16 values (exactly) gives the BF16 pool's step
    bit for bit, and its window afterwards holds the BF16 window's values."""
    p = small(T=T, B=3, H=2)
    q = inputs.copy_problem(p)
    q["conv_f32"] = 1
    q["conv_state"] = from_bf16(p["conv_state"]).reshape(p["conv_state"].shape).copy()
    oracle_lib.run(p)
    oracle_lib.run(q)
    assert np.array_equal(q["out"], p["out"])
    assert np.array_equal(q["state"].view(np.uint32), p["state"].view(np.uint32))
    assert np.array_equal(q["conv_state"], from_bf16(p["conv_state"]).reshape(p["conv_state"].shape))


# The kernel body accumulates the convolution as one FP32 chain that starts
# at the bias (or 0) and takes an fma with the weight of tap i = 0, 1, 2, 3 in
# turn (the convolution block, stock tap order).  The cases below are built
# by hand so that the chain's order and its fused multiply-add show in the
# BF16 result; any other order or a separate multiply and add lands on a
# different value.
BIG = float(2 ** 24)  # 2^24 + 1 is a tie in FP32 and rounds to 2^24 (even)


def _conv_window_setter(p, part, b, h):
    """Returns a function set(col, value) that writes window column `col`
    (0-2: the pool taps at off + col, 3 + t: input x_t) of every channel of
    `part` of item (b, h)."""
    T, dim = p["T"], p["H"] * D
    off = 0 if T == 1 else int(p["accepted"][b]) - 1
    cs = int(p["slots"][b]) if T == 1 else int(p["slots"][b, 0])
    ch = part * dim + h * D + np.arange(D)

    def put(col, value):
        if col < 3:
            if p.get("conv_f32"):
                p["conv_state"][cs, ch, off + col] = np.float32(value)
            else:
                p["conv_state"][cs, ch, off + col] = to_bf16(np.float32(value))
        else:
            p["x"][b * T + col - 3, ch] = to_bf16(np.float32(value))
    return put


@pytest.mark.parametrize("T,t", [(1, 0), (3, 0), (3, 1), (5, 2)])
def test_conv_chain_order_bf16(oracle_lib, T, t):
    """Window [.., 2^24, 1, -2^24, 1 ..] at positions t .. t+3, weights all 1:
    the chain i = 0..3 gives ((2^24 + 1) - 2^24) + 1 = 1 (the first add
    rounds away the 1); the reversed chain gives ((1 - 2^24) + 1) + 2^24 = 2
    (every step exact).  So k = BF16(silu(1)), not BF16(silu(2))."""
    p = small(T=T, B=2, H=2, seed=71 + T)
    if T > 1:
        p["accepted"][:] = 1
    set_conv_taps(p, 1, [1, 1, 1, 1])
    for b in range(p["B"]):
        for h in range(p["H"]):
            put = _conv_window_setter(p, 1, b, h)
            for i, value in enumerate((BIG, 1.0, -BIG, 1.0)):
                put(t + i, value)
    taps = oracle_lib.run(p, taps=True)
    want = bf16_of_f64(silu64(1.0))
    assert want != bf16_of_f64(silu64(2.0))
    assert np.all(taps["k"][:, :, t, :] == want)


@pytest.mark.parametrize("T", [1, 4])
def test_conv_chain_starts_at_bias(oracle_lib, T):
    """Bias 2^24 and window [1, -2^24, 0, 0]: starting from the bias,
    (2^24 + 1) rounds to 2^24 and the chain ends at 0; a bias added after
    the taps would give (1 - 2^24) + 2^24 = 1."""
    p = small(T=T, B=2, H=2, seed=81 + T)
    if T > 1:
        p["accepted"][:] = 1
    dim = p["H"] * D
    p["has_bias"] = 1
    bias = np.zeros(3 * dim, np.float32)
    bias[dim:2 * dim] = BIG
    p["conv_b"] = to_bf16(bias)
    set_conv_taps(p, 1, [1, 1, 1, 1])
    for b in range(p["B"]):
        for h in range(p["H"]):
            put = _conv_window_setter(p, 1, b, h)
            for i, value in enumerate((1.0, -BIG, 0.0, 0.0)):
                put(i, value)
    taps = oracle_lib.run(p, taps=True)
    assert np.all(taps["k"][:, :, 0, :] == 0.0)


@pytest.mark.parametrize("T", [1, 3])
def test_conv_chain_is_fused_fp32_pool(oracle_lib, T):
    """FP32 pool: taps [-(1 + 2^-7 + 2^-23), 1 + 2^-23, 0], weights
    [1, 1 + 2^-7, 0, 0].  The second product is 1 + 2^-7 + 2^-23 + 2^-30;
    an fma keeps it exactly, so the chain leaves 2^-30 and k = BF16(silu(2^-30));
    a product rounded to FP32 first loses the 2^-30 and would give 0."""
    p = small(T=T, B=2, H=2, seed=91 + T, conv_f32=1)
    if T > 1:
        p["accepted"][:] = 1
    set_conv_taps(p, 1, [1.0, 1.0 + 2.0 ** -7, 0.0, 0.0])
    a = -(1.0 + 2.0 ** -7 + 2.0 ** -23)
    for b in range(p["B"]):
        for h in range(p["H"]):
            put = _conv_window_setter(p, 1, b, h)
            for i, value in enumerate((a, 1.0 + 2.0 ** -23, 0.0)):
                put(i, value)
    taps = oracle_lib.run(p, taps=True)
    want = bf16_of_f64(silu64(2.0 ** -30))
    assert want > 0
    assert np.all(taps["k"][:, :, 0, :] == want)


def test_q_scale_applied_after_the_norm_factor(oracle_lib):
    """q_hat = (q * fq) * scale, two FP32 products in that order (kernel
    body, normalised q): then q_hat at scale s is exactly the FP32 product
    of q_hat at scale 1 and s.  Multiplying q by the FP32 product fq * s
    instead breaks that relation for some channels."""
    p = small(B=4, H=2, seed=95)
    s = np.float32(0.0883883476)
    q1 = inputs.copy_problem(p)
    q1["scale"] = 1.0
    qs = inputs.copy_problem(p)
    qs["scale"] = float(s)
    t1 = oracle_lib.run(q1, taps=True)
    ts = oracle_lib.run(qs, taps=True)
    want = (t1["q_hat"].astype(np.float32) * s).astype(np.float32)
    assert np.array_equal(ts["q_hat"].view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("T", [1, 4])
def test_gate_sum_is_exact_before_rounding(oracle_lib, T):
    """raw_g = BF16(FP32(exact sum)) (kernel body, gate projection: the FP32
    accumulation order is free, so the reading takes the exact sum; it is
    rounded to FP32 once, then to BF16): every feature of the cancelling rows
    gives 1 + 2^-7, whose decay a test reads through an all-ones state with
    beta = 0.  An FP32 running sum in column order would give 1 for most."""
    p = small(T=T, B=2, H=2, seed=97, record=0)
    if T > 1:
        p["accepted"][:] = 1
    p["f_b"] = _parity.cancelling_gate_rows(p["H"], D, 5)
    p["f_a"][:] = to_bf16(np.float32(1.0))
    p["beta"][:] = to_bf16(np.full(p["beta"].shape, LOGIT_ZERO, np.float32))
    p["state"][:] = 1.0
    taps = oracle_lib.run(p, taps=True)
    want = np.float32(1.0 + 2.0 ** -7)
    assert np.all(taps["raw_g"] == want)
    a = oracle_lib.decay(float(p["a_log"][0]), float(want), float(p["dt_bias"][0]),
                         p["lower_bound"])
    assert taps["decay"][0, 0, 0, 0] == np.float32(a)


@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("kind,want", [("overflow", 0.5), ("tiny", 2.0 ** -120 + 2.0 ** -127)])
def test_gate_products_exact_beyond_fp32(oracle_lib, T, kind, want):
    """Each gate product is exact (kernel body, gate projection: products of
    BF16 values, summed; the reading takes the exact sum): products beyond
    FP32's range cancel exactly (raw_g = 0.5), and products below its
    smallest subnormal still move a sum off a BF16 midpoint (raw_g =
    2^-120 + 2^-127).  Forming the products in FP32 gives NaN and 2^-120."""
    p = small(T=T, B=2, H=2, seed=98, record=0)
    if T > 1:
        p["accepted"][:] = 1
    p["f_b"], fa = _parity.wide_range_gate_operands(p["H"], D, kind)
    p["f_a"][:] = fa
    taps = oracle_lib.run(p, taps=True)
    assert np.all(taps["raw_g"] == np.float32(want))


def test_output_norm_association(oracle_lib):
    """out = BF16(((o * rstd) * nw) * sigma(gate)) in that order (kernel body,
    output norm block).  Hand-built case, derived with exact rational
    arithmetic and round-to-nearest-even at each FP32 step: all 128 o equal
    x = 1.7578125 (BF16 0x3fe1) and eps = FP32(1e-6), so Σo² = 128 x² exactly,
    variance = x² + eps = 3.0899057388305664 and rstd = 0.568888783454895
    (FP32), x * rstd = 0.9999998211860657.  Channel 0 (nw 0x3f87, gate
    0xbe42) gives BF16 0x3ef4 and channel 1 (nw 0x3f11, gate 0xbea2) 0x3e74
    in the page's order; o * (rstd * nw) * σ, (o * rstd) * (nw * σ) and
    o * ((rstd * nw) * σ) all give 0x3ef5 and 0x3e75."""
    o = np.full(D, 1.7578125, np.float32)
    gate = np.zeros(D, np.uint16)
    nw = np.full(D, 0x3F80, np.uint16)
    gate[0], nw[0] = 0xBE42, 0x3F87
    gate[1], nw[1] = 0xBEA2, 0x3F11
    out = oracle_lib.gated_rmsnorm(o, gate, nw, float(np.float32(1e-6)))
    assert int(out[0]) == 0x3EF4 and int(out[1]) == 0x3E74


def test_gate_one_hot(oracle_lib):
    """One-hot F_B rows: raw_g[f] = f_a[pi(f)] bit for bit (record output)."""
    T = 2
    p = small(T=T, B=2, H=2, record=1)
    pi = (np.arange(D) * 53 + 7) % D
    fb = np.zeros((p["H"] * D, D), np.float32)
    for h in range(p["H"]):
        fb[h * D + np.arange(D), (pi + h) % D] = 1.0
    p["f_b"] = to_bf16(fb)
    oracle_lib.run(p)
    for b in range(p["B"]):
        for h in range(p["H"]):
            for t in range(T):
                want = p["f_a"][b * T + t][(pi + h) % D]
                assert np.array_equal(p["rec_kg"][b, h, t, D:], want)


# --------------------------------------------------------------------------
# closed forms through the whole step


def test_zero_state_closed_form(oracle_lib):
    """S = 0 and q = k: S_new = k_hat u^T with u = v * beta, and
    o_v = u_v * (k_hat . q_hat) = u_v * scale * |k_hat|^2; the output is the
    gated RMSNorm of that o."""
    p = small(B=3, H=2, seed=31)
    p["state"][:] = 0.0
    dim = p["H"] * D
    p["conv_w"][0] = p["conv_w"][1]
    p["x"][:, :dim] = p["x"][:, dim:2 * dim]
    p["conv_state"][:, :dim] = p["conv_state"][:, dim:2 * dim]
    taps = oracle_lib.run(p, taps=True)
    for b in range(p["B"]):
        for h in range(p["H"]):
            k = taps["k"][b, h, 0].astype(np.float64)
            v = taps["v"][b, h, 0].astype(np.float64)
            beta = 1.0 / (1.0 + np.exp(-float(from_bf16(p["beta"][b:b + 1, h])[0])))
            kh = k / np.sqrt((k * k).sum() + 1e-6)
            S = p["state"][int(p["slots"][b]), h].astype(np.float64)
            assert np.allclose(S, np.outer(v * beta, kh), rtol=1e-6, atol=1e-9)
            o = v * beta * p["scale"] * (kh * kh).sum()
            assert np.allclose(taps["o_exact"][b, h, 0], o, rtol=1e-5, atol=1e-9)
            o_bf = bf16_of_f64(o).astype(np.float64)
            g = from_bf16(p["gate"][b, h * D:(h + 1) * D]).astype(np.float64)
            nw = from_bf16(p["norm_w"]).astype(np.float64)
            want = o_bf / np.sqrt((o_bf ** 2).mean() + p["eps"]) * nw / (1 + np.exp(-g))
            got = from_bf16(p["out"][b, h * D:(h + 1) * D]).astype(np.float64)
            assert np.all(np.abs(got - want) <= 2 * 2.0 ** (np.floor(np.log2(np.abs(want) + 1e-30)) - 7))


def test_norm_epsilon_small_keys(oracle_lib):
    """The 1e-6 of the L2 norm is added to the sum of squares: with q = k of
    sum of squares m ~ 1e-6, zero state and beta = 1, S_new = v k_hat^T and
    o = v * scale * m / (m + 1e-6)."""
    p = small(B=2, H=2, seed=33)
    p["state"][:] = 0.0
    p["beta"][:] = to_bf16(np.full(p["beta"].shape, LOGIT_ONE, np.float32))
    dim = p["H"] * D
    for part in (0, 1):
        set_conv_taps(p, part, [0, 0, 0, 1])
    small_x = to_bf16(from_bf16(p["x"][:, dim:2 * dim]) * np.float32(2e-4))
    p["x"][:, :dim] = small_x
    p["x"][:, dim:2 * dim] = small_x
    taps = oracle_lib.run(p, taps=True)
    for b in range(p["B"]):
        for h in range(p["H"]):
            k = taps["k"][b, h, 0].astype(np.float64)
            v = taps["v"][b, h, 0].astype(np.float64)
            m = (k * k).sum()
            assert 1e-7 < m < 1e-5
            kh = k / np.sqrt(m + 1e-6)
            S = p["state"][int(p["slots"][b]), h].astype(np.float64)
            assert np.allclose(S, np.outer(v, kh), rtol=1e-5, atol=1e-12)
            o = v * p["scale"] * m / (m + 1e-6)
            assert np.allclose(taps["o_exact"][b, h, 0], o, rtol=1e-5, atol=1e-12)


def test_rmsnorm_closed_form(oracle_lib):
    rng = np.random.default_rng(3)
    o = from_bf16(to_bf16(rng.standard_normal(D).astype(np.float32)))
    one = to_bf16(np.ones(D, np.float32))
    sig1 = to_bf16(np.full(D, LOGIT_ONE, np.float32))
    # eps = 0, nw = 1, gate sigma = 1: out = o / rms(o), so rms(out) = 1
    out = from_bf16(oracle_lib.gated_rmsnorm(o, sig1, one, 0.0)).astype(np.float64)
    assert abs(math.sqrt((out ** 2).mean()) - 1.0) < 2 ** -8
    assert np.all(np.sign(out) == np.sign(o))
    # eps = m: rms(out) = sqrt(m / (m + eps)) = sqrt(1/2)
    m = float((o.astype(np.float64) ** 2).mean())
    out = from_bf16(oracle_lib.gated_rmsnorm(o, sig1, one, m)).astype(np.float64)
    assert abs(math.sqrt((out ** 2).mean()) - math.sqrt(0.5)) < 2 ** -8
    # nw = 2 doubles the output exactly; a gate logit of -200 zeroes a channel
    two = to_bf16(np.full(D, 2.0, np.float32))
    base = from_bf16(oracle_lib.gated_rmsnorm(o, sig1, one, 1e-6))
    dbl = from_bf16(oracle_lib.gated_rmsnorm(o, sig1, two, 1e-6))
    assert np.array_equal(dbl, 2 * base)
    gz = sig1.copy()
    gz[[3, 64, 127]] = to_bf16(np.float32(LOGIT_ZERO))
    zed = from_bf16(oracle_lib.gated_rmsnorm(o, gz, one, 1e-6))
    assert np.all(zed[[3, 64, 127]] == 0) and np.array_equal(np.delete(zed, [3, 64, 127]),
                                                             np.delete(base, [3, 64, 127]))


# --------------------------------------------------------------------------
# record mode (RecoverSSM): same outputs, no state write, replayable records


def test_record_replay(oracle_lib):
    T = 4
    p = small(T=T, B=3, H=2, record=1, seed=41)
    plain = inputs.copy_problem(p)
    plain.update(record=0, rec_u=None, rec_kg=None)
    before_state = p["state"].copy()
    oracle_lib.run(p)
    oracle_lib.run(plain)
    assert np.array_equal(p["out"], plain["out"])
    assert np.array_equal(p["conv_state"], plain["conv_state"])
    assert np.array_equal(p["state"].view(np.uint32), before_state.view(np.uint32))  # no writes
    for b in range(p["B"]):
        for h in range(p["H"]):
            S = before_state[read_slot(p, b), h].astype(np.float64)   # the checkpoint
            dt = p["dt_bias"][h * D:(h + 1) * D]
            for t in range(T):
                k = from_bf16(p["rec_kg"][b, h, t, :D]).astype(np.float64)
                g = from_bf16(p["rec_kg"][b, h, t, D:])
                u = p["rec_u"][b, h, t].astype(np.float64)
                a = np.array([oracle_lib.decay(float(p["a_log"][h]), float(g[f]), float(dt[f]),
                                               p["lower_bound"]) for f in range(D)])
                kh = k / np.sqrt((k * k).sum() + 1e-6)
                S = S * a[None, :] + np.outer(u, kh)
                ref = plain["state"][int(plain["slots"][b, t]), h].astype(np.float64)
                rms = math.sqrt((ref ** 2).mean())
                assert np.all(np.abs(S - ref) <= 1e-5 * (np.abs(ref) + rms))


# --------------------------------------------------------------------------
# the whole step against an independent float64 matrix formulation


@pytest.mark.parametrize("name,T", [("tiny_decode", 1), ("small_verify", 4), ("small_verify8", 8)])
def test_matrix_form_cross_check(oracle_lib, name, T):
    """Where a BF16 rounding input sits within FP32 noise of a midpoint the two
    formulations may round differently (the page fixes FP32 operations, the
    matrix form is float64); there the matrix form takes the oracle's
    neighbour, and such points must stay rare."""
    if name == "tiny_decode":
        p = inputs.make_problem("tiny_decode")
    else:
        p = small(T=T, B=2, H=2, seed=50 + T)
    before = inputs.copy_problem(p)
    taps = oracle_lib.run(p, taps=True)
    ties = [0]
    for b in range(p["B"]):
        for h in range(p["H"]):
            out, states = _matrix_form.step(before, b, h, taps=taps, counter=ties)
            got = from_bf16(p["out"][b * T:(b + 1) * T, h * D:(h + 1) * D]).astype(np.float64)
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(out), 1e-30))) - 7)
            assert np.all(np.abs(got - out) <= 2 * ulp)
            for t in range(T):
                tgt = int(p["slots"][b]) if T == 1 else int(p["slots"][b, t])
                ref = states[t].T  # back to [value row][key]
                g = p["state"][tgt, h].astype(np.float64)
                rms = math.sqrt((ref ** 2).mean())
                assert np.all(np.abs(g - ref) <= 1e-5 * (np.abs(ref) + rms))
    assert ties[0] <= 0.05 * p["B"] * p["H"] * T * 5 * D


# --------------------------------------------------------------------------
# RecoverSSM replay: checkpoint + records -> the state after n tokens


def replay_from_record(p, n):
    """A replay problem that applies the records of record-mode problem p
    (after its run) to the pages p read, writing to fresh slots."""
    B, H, T, N = p["B"], p["H"], p["T"], p["N"]
    src = np.array([int(p["slots"][b, p["accepted"][b] - 1]) for b in range(B)], np.int32)
    state = np.concatenate([p["state"], np.zeros((B,) + p["state"].shape[1:], np.float32)])
    return dict(B=B, H=H, T=T, N=N + B, lower_bound=p["lower_bound"], rec_u=p["rec_u"],
                rec_kg=p["rec_kg"], a_log=p["a_log"], dt_bias=p["dt_bias"], src=src,
                dst=np.arange(N, N + B, dtype=np.int32), n=np.asarray(n, np.int32), state=state)


def test_replay_matches_plain_verify(oracle_lib):
    """Replaying the first n records from the checkpoint gives, bit for bit,
    the state a plain verify of the same inputs writes after token n; n = 0
    copies the checkpoint."""
    T = 6
    p = small(T=T, B=5, H=2, seed=61, record=1)
    plain = inputs.copy_problem(p)
    plain.update(record=0, rec_u=None, rec_kg=None)
    oracle_lib.run(p)
    oracle_lib.run(plain)
    n = [0, 1, 3, 6, 4]
    r = replay_from_record(p, n)
    before = r["state"].copy()
    oracle_lib.replay(r)
    for b in range(p["B"]):
        got = r["state"][r["dst"][b]]
        want = before[r["src"][b]] if n[b] == 0 else plain["state"][int(plain["slots"][b, n[b] - 1])]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), b
    assert np.array_equal(r["state"][:p["N"]], before[:p["N"]])  # checkpoints untouched


def test_replay_skips_invalid(oracle_lib):
    r = inputs.make_replay_problem(dict(B=4, H=2, T=3, N=12, seed=7))
    r["src"][0] = 0
    r["dst"][1] = r["N"]
    r["n"][2] = 4
    before = r["state"].copy()
    oracle_lib.replay(r)
    for b in (0, 1, 2):
        assert np.array_equal(r["state"][r["dst"][b] % r["N"]], before[r["dst"][b] % r["N"]])
    assert not np.array_equal(r["state"][r["dst"][3]], before[r["dst"][3]]) or r["n"][3] == 0


def test_replay_closed_form(oracle_lib):
    """No decay (lower_bound 0): S_n = S_0 + sum_t k_hat_t u_t^T, an
    independent float64 sum of outer products."""
    r = inputs.make_replay_problem(dict(B=3, H=2, T=5, N=10, seed=9, lower_bound=0.0))
    r["n"][:] = [5, 2, 3]
    before = r["state"].copy()
    oracle_lib.replay(r)
    for b in range(r["B"]):
        for h in range(r["H"]):
            S = before[r["src"][b], h].astype(np.float64)
            for t in range(int(r["n"][b])):
                k = from_bf16(r["rec_kg"][b, h, t, :D]).astype(np.float64)
                kh = k / np.sqrt((k * k).sum() + 1e-6)
                S = S + np.outer(r["rec_u"][b, h, t].astype(np.float64), kh)
            got = r["state"][r["dst"][b], h].astype(np.float64)
            rms = math.sqrt((S ** 2).mean())
            assert np.all(np.abs(got - S) <= 1e-5 * (np.abs(S) + rms))
