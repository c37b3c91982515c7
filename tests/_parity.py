"""Element-wise comparison of a GPU step with the oracle's step.

The contract:
  * slot and index handling bit-exact: which pages and output rows are
    written; untouched pages (slot 0, unused slots, skipped targets, every
    page in record mode) keep their bits; padded outputs are +0; the
    convolution windows are exact bit copies; record buffers of padded
    items are untouched;
  * BF16 k and raw gate (record mode) bit-exact: both sides compute them as
    correctly rounded values of the same FP32 operations;
  * FP32 state pages and rec_u: |g - r| <= 1e-4 (|r| + rms(r) over the page,
    or over the 128 u of a token);
  * BF16 outputs: |g - r| <= 2 ulp_bf16(max(|r|, 2^-8 rms(row))), where the
    recurrence output o of a channel lies within 2^-18 sum_k |S q_hat| of a
    BF16 midpoint, the output computed with the other rounding of that o is
    accepted too (FP32 summation order decides such a rounding).
"""

import numpy as np

import oracle
from linear_attention_decode_03_amd.inputs import from_bf16, to_bf16

D = 128
TIE_BAND = 2.0 ** -18


def ulp_bf16(x):
    x = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(x)) - 7)


def cancelling_gate_rows(H, D, seed):
    """F_B rows (H*D of them, D columns, BF16) for a test of the gate's exact
    sum: each row holds 2^20, 1, 2^-8, 2^-20 and -2^20 at five columns drawn
    per row, zero elsewhere.  Against f_a = 1 the exact projection is
    1 + 2^-8 + 2^-20, an FP32 value just above the midpoint between the BF16
    values 1 and 1 + 2^-7, so the exact sum rounds to 1 + 2^-7.  An FP32 sum
    that meets 2^20 before the small terms loses them (the FP32 spacing at
    2^20 is 2^-3) and ends at 1; one that loses only 2^-20 ends on the
    midpoint, which rounds to even, also 1.  An input generator only: no
    step of the method is computed here."""
    rng = np.random.default_rng(seed)
    fb = np.zeros((H * D, D), np.float32)
    terms = np.array([2.0 ** 20, 1.0, 2.0 ** -8, 2.0 ** -20, -(2.0 ** 20)], np.float32)
    for r in range(H * D):
        fb[r, rng.choice(D, size=5, replace=False)] = terms
    return to_bf16(fb)



def wide_range_gate_operands(H, D, kind):
    """F_B rows (H*D of them, all alike) and one f_a row for a test that the
    gate's products are formed exactly, also beyond FP32's range.  An input
    generator only: no step of the method is computed here.

    kind "overflow": columns 0 and 1 give the products 2^140 and -2^140
    (beyond FP32, exact in FP64) and column 2 gives 1 * 0.5, so the exact
    projection is 0.5; products formed in FP32 overflow to +-inf and sum
    to NaN.

    kind "tiny": columns 0 and 1 give 2^-120 and 2^-128, whose sum M is the
    midpoint between the BF16 values 2^-120 and 2^-120 + 2^-127, and the
    other 126 columns give (1 + 77/128) 2^-151 each (below FP32's smallest
    subnormal, 2^-149, by a factor 0.4004).  The exact sum is M plus 0.788
    FP32 ulps at that magnitude (2^-143): it rounds to M + 2^-143 in FP32
    and up to 2^-120 + 2^-127 in BF16.  Products formed in FP32 round the
    small ones to 0, leave the midpoint M and round to even, 2^-120."""
    fb = np.zeros((H * D, D), np.float32)
    fa = np.zeros(D, np.float32)
    if kind == "overflow":
        fb[:, 0], fa[0] = 2.0 ** 70, 2.0 ** 70
        fb[:, 1], fa[1] = -(2.0 ** 70), 2.0 ** 70
        fb[:, 2], fa[2] = 1.0, 0.5
    elif kind == "tiny":
        fb[:, 0], fa[0] = 2.0 ** -60, 2.0 ** -60
        fb[:, 1], fa[1] = 2.0 ** -64, 2.0 ** -64
        fb[:, 2:], fa[2:] = (1.0 + 77.0 / 128.0) * 2.0 ** -76, 2.0 ** -75
    else:
        raise ValueError(kind)
    return to_bf16(fb), to_bf16(fa)


def written_targets(p):
    """{slot: [(b, h, t), ...]} of the state pages the step writes."""
    B, H, T = p["B"], p["H"], p["T"]
    writes = {}
    if p["record"]:
        return writes
    for b in range(B):
        if T == 1:
            rs = int(p["slots"][b])
            if 0 < rs < p["N"]:
                writes.setdefault(rs, []).append(b)
        else:
            acc = int(p["accepted"][b])
            if not 1 <= acc <= min(T, p["slot_stride"]):
                continue
            rs = int(p["slots"][b, acc - 1])
            cs = int(p["slots"][b, 0])
            if not (0 < rs < p["N"] and 0 <= cs < p["N"]):
                continue
            for t in range(T):
                tgt = int(p["slots"][b, t])
                if 0 < tgt < p["N"]:
                    writes.setdefault(tgt, []).append(b)
    return writes


def compare_step(before, ref, got, taps, items=None, report=None):
    """before: the host problem before the step; ref: the oracle's results
    (problem dict after oracle.run); got: the GPU's results (dict with state,
    conv_state, out, rec_u, rec_kg as numpy); taps: the oracle's taps.
    `items` limits the output and record comparison to those item ids
    (the state and conv pools are always compared whole).  Raises
    AssertionError with a description on the first violation.  Fills
    `report` (a dict) with counts."""
    B, H, T = before["B"], before["H"], before["T"]
    rep = {} if report is None else report
    # conv windows: exact bits everywhere (BF16 bits, or FP32 bits of an FP32 pool)
    bits = np.uint32 if ref["conv_state"].dtype == np.float32 else np.uint16
    diff = np.nonzero(ref["conv_state"].view(bits) != got["conv_state"].view(bits))
    assert diff[0].size == 0, f"conv_state differs at {len(diff[0])} places, first {[d[0] for d in diff]}"
    # state pages
    writes = written_targets(before)
    pages_ref = ref["state"].reshape(before["N"], H, -1)
    pages_got = got["state"].reshape(before["N"], H, -1)
    untouched = np.ones(before["N"], dtype=bool)
    untouched[list(writes)] = False
    u_idx = np.nonzero(untouched)[0]
    if u_idx.size:
        same = pages_got[u_idx].view(np.uint32) == before["state"].reshape(before["N"], H, -1)[u_idx].view(np.uint32)
        assert same.all(), f"an unwritten state page changed (slots {u_idx[~same.all(axis=(1, 2))][:8]})"
    worst = 0.0
    for s in writes:
        r = pages_ref[s].astype(np.float64)
        g = pages_got[s].astype(np.float64)
        rms = np.sqrt((r * r).mean(axis=1, keepdims=True))
        err = np.abs(g - r) / (np.abs(r) + rms)
        m = float(err.max())
        worst = max(worst, m)
        assert m <= 1e-4, f"state page {s}: relative error {m:.3e} > 1e-4"
    rep["state_worst_rel"] = worst
    rep["pages_written"] = len(writes)

    # outputs and records, item by item
    if items is None:
        items = np.arange(B * H)
    live = set(_live_items(before).tolist())
    out_r, out_g = ref["out"], got["out"]
    nties = nflag = 0
    worst_ulp = 0.0
    for it in np.asarray(items):
        b, h = divmod(int(it), H)
        rows = slice(b * T, (b + 1) * T)
        cols = slice(h * D, (h + 1) * D)
        if int(it) not in live:
            assert np.all(out_g[rows, cols] == 0), f"padded item {it}: output not +0"
            if before["record"]:
                assert np.array_equal(got["rec_kg"][b, h], before["rec_kg"][b, h])
                assert np.array_equal(got["rec_u"][b, h].view(np.uint32),
                                      before["rec_u"][b, h].view(np.uint32))
            continue
        for t in range(T):
            r = from_bf16(out_r[b * T + t, cols]).astype(np.float64)
            g = from_bf16(out_g[b * T + t, cols]).astype(np.float64)
            rms = np.sqrt((r * r).mean())
            tol = 2 * ulp_bf16(np.maximum(np.abs(r), 2.0 ** -8 * rms))
            bad = np.abs(g - r) > tol
            o_ex = taps["o_exact"][b, h, t]
            band = TIE_BAND * taps["o_abs"][b, h, t]
            ul = ulp_bf16(o_ex)
            lo = np.floor(o_ex / ul) * ul
            flagged = np.abs(np.abs(o_ex - lo) - ul / 2) <= band
            nflag += int(flagged.sum())
            if bad.any():
                for c in np.nonzero(bad)[0]:
                    assert flagged[c], (f"item {it} token {t} channel {c}: out {g[c]!r} vs "
                                        f"{r[c]!r} (tol {tol[c]:.3g}), o not near a tie")
                    o_row = taps["o_bf"][b, h, t].copy()
                    o_row[c] = lo[c] if o_row[c] == lo[c] + ul[c] else lo[c] + ul[c]
                    alt = from_bf16(oracle.gated_rmsnorm(
                        o_row, before["gate"][b * T + t, cols], before["norm_w"],
                        before["eps"]))[c]
                    ok = abs(g[c] - alt) <= 2 * ulp_bf16(max(abs(alt), 2.0 ** -8 * rms))
                    assert ok, f"item {it} token {t} channel {c}: out {g[c]} vs {r[c]} or {alt}"
                    nties += 1
            worst_ulp = max(worst_ulp, float((np.abs(g - r) / ulp_bf16(np.maximum(np.abs(r), 2.0 ** -8 * rms))).max()))
        if before["record"]:
            assert np.array_equal(got["rec_kg"][b, h], ref["rec_kg"][b, h]), \
                f"item {it}: record k | raw_g differ"
            ru = ref["rec_u"][b, h].astype(np.float64)
            gu = got["rec_u"][b, h].astype(np.float64)
            rms = np.sqrt((ru * ru).mean(axis=1, keepdims=True))
            m = float((np.abs(gu - ru) / (np.abs(ru) + rms)).max())
            assert m <= 1e-4, f"item {it}: rec_u relative error {m:.3e}"
    rep["out_ties_used"] = nties
    rep["o_flagged"] = nflag
    rep["out_worst_ulp"] = worst_ulp
    return rep


def _live_items(p):
    B, H, T = p["B"], p["H"], p["T"]
    live = []
    for b in range(B):
        if T == 1:
            rs = int(p["slots"][b])
            ok = 0 < rs < p["N"]
        else:
            acc = int(p["accepted"][b])
            ok = 1 <= acc <= min(T, p["slot_stride"])
            if ok:
                rs, cs = int(p["slots"][b, acc - 1]), int(p["slots"][b, 0])
                ok = 0 < rs < p["N"] and 0 <= cs < p["N"]
        if ok:
            live.extend(b * H + h for h in range(H))
    return np.asarray(live, dtype=np.int64)


def compare_replay(before, ref, got_state):
    """Replay contract: every valid request's dst pages within 1e-4 of the
    oracle (relative to |r| + rms of the page); every other page keeps its
    bits.  Returns the worst relative error."""
    N, H = before["N"], before["H"]
    valid = [b for b in range(before["B"])
             if 0 < before["src"][b] < N and 0 < before["dst"][b] < N and 0 <= before["n"][b] <= before["T"]]
    dst = {int(before["dst"][b]) for b in valid}
    for s in range(N):
        if s not in dst:
            assert np.array_equal(got_state[s].view(np.uint32), before["state"][s].view(np.uint32)), \
                f"page {s} changed but is no replay target"
    worst = 0.0
    for s in dst:
        r = ref["state"][s].reshape(H, -1).astype(np.float64)
        g = got_state[s].reshape(H, -1).astype(np.float64)
        rms = np.sqrt((r * r).mean(axis=1, keepdims=True))
        m = float((np.abs(g - r) / (np.abs(r) + rms)).max())
        worst = max(worst, m)
        assert m <= 1e-4, f"replay page {s}: relative error {m:.3e}"
    return worst
