"""Seeded synthetic inputs for the KDA decode / verify step.

This module only draws random numbers and stores them in the operand layouts;
it holds none of the method's arithmetic.  The same host arrays feed the GPU
library and the CPU oracle.

Layouts (row-major, contiguous; "bf16" arrays are uint16 bit patterns):
    x          bf16  [B*T, 3*H*128]   q | k | v channels before the convolution
    conv_w     bf16  [3, 4, H*128]    (part, tap, channel)
    conv_state bf16  [N, 3*H*128, W]  per-slot window of past inputs
               (f32 when the problem has conv_f32 = 1)
    f_a        bf16  [B*T, 128]       low-rank gate input
    beta       bf16  [B*T, H]         beta logits
    a_log      f32   [H]
    dt_bias    f32   [H*128]
    slots      i32   [B] (decode) or [B, slot_stride] (verify)
    accepted   i32   [B] (verify only)
    state      f32   [N, H, 128, 128] (slot, head, value row, key)
    out        bf16  [B*T, H*128]
    gate       bf16  [B*T, H*128]     output-gate logits
    norm_w     bf16  [128]
    f_b        bf16  [H*128, 128]     gate projection
    rec_u      f32   [B, H, T, 128]   (record mode)
    rec_kg     bf16  [B, H, T, 256]   (record mode)

Distributions (the KDA page's workload, real Kimi-K3 decode traffic, has no
public dataset; these stand in for it): state ~N(0, 0.02), conv weights
~N(0, 0.5), x ~N(0, 1), F_B ~N(0, 0.05), A_log ~U(-1, 1), dt_bias ~N(0, 0.1),
beta logits ~N(0, 1), lower_bound = -5, eps = 1e-6, scale = 1/sqrt(128);
conv pool, f_a and gate ~N(0, 1), norm weight ~N(1, 0.1).  Draws come from
numpy's PCG64 in this fixed order: state pool, conv pool, conv weights, x, f_a,
F_B, A_log, dt_bias, beta, gate, norm weight, slots, accepted.  Normal draws
are made in float32 and rounded to BF16 (nearest-even) where the operand is BF16.
"""

from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128

# The five workloads: a tiny case, a padded decode batch, the throughput
# decode batch, a speculative verify and a record-mode verify.
CONFIGS = {
    "tiny_decode": dict(B=2, H=2, T=1, N=4, W=3, seed=0, fixed_slots=[1, 3]),
    "decode_b64": dict(B=64, H=32, T=1, N=160, W=3, seed=1, padded=8),
    "decode_b256": dict(B=256, H=32, T=1, N=512, W=3, seed=2),
    "verify_t4": dict(B=64, H=32, T=4, N=257, W=6, seed=3),
    "verify_record_t8": dict(B=128, H=32, T=8, N=1025, W=10, seed=4, record=1, gate_mode=1),
}

# A value no correct kernel writes: a BF16 NaN and an FP32 NaN bit pattern,
# used to fill outputs so that an element left unwritten is visible.
BF16_SENTINEL = np.uint16(0x7FC1)
F32_SENTINEL_BITS = np.uint32(0x7FC00123)


def to_bf16(a) -> np.ndarray:
    """float array -> BF16 bit patterns (uint16), round to nearest even."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def from_bf16(h) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32 (exact)."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    return (h.astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std, mean=0.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    if mean:
        a += np.float32(mean)
    return a


def make_problem(name_or_cfg="tiny_decode", seed=None, **override) -> dict:
    """Builds one seeded problem.  `name_or_cfg` names an entry of CONFIGS or is
    a dict of the same keys; `override` replaces any key (B, H, T, N, W, seed,
    record, gate_mode, padded, fixed_slots, slot_stride, lower_bound, eps,
    scale, conv_f32).  conv_f32 = 1 keeps the convolution pool in FP32 (the
    same draws, not rounded to BF16)."""
    cfg = dict(CONFIGS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    if seed is not None:
        cfg["seed"] = seed
    B, H, T, N, W = (int(cfg[k]) for k in ("B", "H", "T", "N", "W"))
    record = int(cfg.get("record", 0))
    gate_mode = int(cfg.get("gate_mode", 0))
    conv_f32 = int(cfg.get("conv_f32", 0))
    stride = int(cfg.get("slot_stride", T if T > 1 else 1))
    dim = H * HEAD_DIM
    rng = np.random.default_rng(int(cfg.get("seed", 0)))

    p = dict(B=B, H=H, T=T, N=N, W=W, slot_stride=stride, record=record,
             gate_mode=gate_mode, has_bias=0, conv_f32=conv_f32,
             lower_bound=float(cfg.get("lower_bound", -5.0)),
             scale=float(cfg.get("scale", 1.0 / math.sqrt(HEAD_DIM))),
             eps=float(cfg.get("eps", 1e-6)))

    p["state"] = _normal(rng, (N, H, HEAD_DIM, HEAD_DIM), 0.02)
    pool = _normal(rng, (N, 3 * dim, W), 1.0)
    p["conv_state"] = pool if conv_f32 else to_bf16(pool)
    p["conv_w"] = to_bf16(_normal(rng, (3, 4, dim), 0.5))
    p["x"] = to_bf16(_normal(rng, (B * T, 3 * dim), 1.0))
    p["f_a"] = to_bf16(_normal(rng, (B * T, HEAD_DIM), 1.0))
    p["f_b"] = to_bf16(_normal(rng, (dim, HEAD_DIM), 0.05))
    p["a_log"] = rng.uniform(-1.0, 1.0, size=H).astype(np.float32)
    p["dt_bias"] = _normal(rng, (dim,), 0.1)
    p["beta"] = to_bf16(_normal(rng, (B * T, H), 1.0))
    p["gate"] = to_bf16(_normal(rng, (B * T, dim), 1.0))
    p["norm_w"] = to_bf16(_normal(rng, (HEAD_DIM,), 0.1, mean=1.0))
    p["conv_b"] = None

    if T == 1:
        if "fixed_slots" in cfg:
            slots = np.asarray(cfg["fixed_slots"], dtype=np.int32)
        else:
            slots = rng.choice(np.arange(1, N, dtype=np.int32), size=B, replace=False)
            npad = int(cfg.get("padded", 0))
            if npad:
                slots[rng.choice(B, size=npad, replace=False)] = 0
        p["slots"] = np.ascontiguousarray(slots.astype(np.int32).reshape(B))
        p["accepted"] = None
    else:
        if "fixed_slots" in cfg:
            slots = np.asarray(cfg["fixed_slots"], dtype=np.int32).reshape(B, stride)
        else:
            pool = rng.permutation(np.arange(1, N, dtype=np.int32))
            slots = pool[: B * stride].reshape(B, stride)
        p["slots"] = np.ascontiguousarray(slots.astype(np.int32))
        p["accepted"] = rng.integers(1, min(T, stride) + 1, size=B).astype(np.int32)

    p["out"] = np.full((B * T, dim), BF16_SENTINEL, dtype=np.uint16)
    if record:
        p["rec_u"] = np.full((B, H, T, HEAD_DIM), F32_SENTINEL_BITS, dtype=np.uint32).view(np.float32)
        p["rec_kg"] = np.full((B, H, T, 2 * HEAD_DIM), BF16_SENTINEL, dtype=np.uint16)
    else:
        p["rec_u"] = None
        p["rec_kg"] = None
    return p


def copy_problem(p: dict) -> dict:
    """Deep copy (arrays copied, scalars shared)."""
    return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}


def live_items(p: dict) -> np.ndarray:
    """Item ids (b * H + h) whose read slot is live (> 0), for sampling."""
    B, H, T = p["B"], p["H"], p["T"]
    if T == 1:
        rs = p["slots"].reshape(B)
    else:
        rs = p["slots"][np.arange(B), p["accepted"] - 1]
    live_b = np.nonzero(rs > 0)[0]
    return (live_b[:, None] * H + np.arange(H)[None, :]).reshape(-1).astype(np.int32)


# The replay workload: a record-mode verify's records applied to checkpoint
# pages.  B=128 requests, H=32 heads, T=8 recorded tokens, accepted counts
# n ~ U{0..8}; checkpoint and target slots are distinct pool entries.
REPLAY_CONFIGS = {
    "replay_t8": dict(B=128, H=32, T=8, N=257, seed=5),
}


def make_replay_problem(name_or_cfg="replay_t8", seed=None, **override) -> dict:
    """Seeded replay operands: state pool ~N(0, 0.02), records with k ~N(0, 1)
    and raw_g ~N(0, 0.57) in BF16 (the spread of a BF16 projection of the
    verify workload), u ~N(0, 0.5) in FP32, A_log ~U(-1, 1),
    dt_bias ~N(0, 0.1), lower_bound = -5; src and dst slots are 2B distinct
    entries of 1..N-1."""
    cfg = dict(REPLAY_CONFIGS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(override)
    if seed is not None:
        cfg["seed"] = seed
    B, H, T, N = (int(cfg[k]) for k in ("B", "H", "T", "N"))
    rng = np.random.default_rng(int(cfg.get("seed", 0)))
    r = dict(B=B, H=H, T=T, N=N, lower_bound=float(cfg.get("lower_bound", -5.0)))
    r["state"] = _normal(rng, (N, H, HEAD_DIM, HEAD_DIM), 0.02)
    k = to_bf16(_normal(rng, (B, H, T, HEAD_DIM), 1.0))
    g = to_bf16(_normal(rng, (B, H, T, HEAD_DIM), 0.57))
    r["rec_kg"] = np.ascontiguousarray(np.concatenate([k, g], axis=3))
    r["rec_u"] = _normal(rng, (B, H, T, HEAD_DIM), 0.5)
    r["a_log"] = rng.uniform(-1.0, 1.0, size=H).astype(np.float32)
    r["dt_bias"] = _normal(rng, (H * HEAD_DIM,), 0.1)
    slots = rng.permutation(np.arange(1, N, dtype=np.int32))[: 2 * B]
    r["src"] = np.ascontiguousarray(slots[:B])
    r["dst"] = np.ascontiguousarray(slots[B:])
    r["n"] = rng.integers(0, T + 1, size=B).astype(np.int32)
    return r
