"""Device-side plumbing for the binding: moves a host problem (see
`inputs`) to the GPU as torch tensors, runs one step through the C ABI
binding (`kda`), and brings the results back.  Marshalling only; every step
of the computation runs in the library's kernels."""

import numpy as np
import torch

from . import kda

_BF16 = ("x", "conv_w", "conv_b", "conv_state", "f_a", "beta", "out", "gate", "norm_w", "f_b",
         "rec_kg")


def to_device(p, device="cuda"):
    d = {}
    for k, v in p.items():
        if not isinstance(v, np.ndarray):
            d[k] = v
        elif k in _BF16 and v.dtype == np.uint16:
            d[k] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to(device).view(torch.bfloat16)
        else:
            d[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
    return d


def to_host(d, keys=("state", "conv_state", "out", "rec_u", "rec_kg")):
    h = {}
    for k in keys:
        t = d.get(k)
        if t is None:
            h[k] = None
        elif t.dtype == torch.bfloat16:
            h[k] = t.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            h[k] = t.cpu().numpy()
    return h


def run(d, ahead=-1, stream=None):
    """One step on the device problem d (in place)."""
    args = (d["x"], d["conv_w"], d["conv_b"], d["conv_state"], d["f_a"], d["beta"], d["a_log"],
            d["dt_bias"], d["slots"], d["state"], d["out"], d["gate"], d["norm_w"],
            d["lower_bound"], d["scale"], d["eps"], d["f_b"])
    if d["T"] == 1:
        kda.kda_decode(*args, gate_mode=d["gate_mode"], ahead=ahead, stream=stream)
    else:
        kda.kda_verify(*args, d["accepted"], d.get("rec_u"), d.get("rec_kg"), T=d["T"],
                       record=bool(d["record"]), gate_mode=d["gate_mode"], ahead=ahead,
                       stream=stream)



def run_replay(d, stream=None):
    """One replay on the device operands d (to_device of a replay problem)."""
    kda.kda_replay(d["rec_u"], d["rec_kg"], d["a_log"], d["dt_bias"], d["src"], d["dst"], d["n"],
                   d["state"], d["lower_bound"], stream=stream)


def run_split(d, workspace, split=0, stream=None):
    """One split step (plain decode or verify) on the device problem d."""
    args = (d["x"], d["conv_w"], d["conv_b"], d["conv_state"], d["f_a"], d["beta"], d["a_log"],
            d["dt_bias"], d["slots"], d["state"], d["out"], d["gate"], d["norm_w"],
            d["lower_bound"], d["scale"], d["eps"], d["f_b"])
    if d["T"] == 1:
        kda.kda_decode_split(*args, workspace, split=split, gate_mode=d["gate_mode"],
                             stream=stream)
    else:
        kda.kda_verify_split(*args, d["accepted"], workspace, T=d["T"], split=split,
                             gate_mode=d["gate_mode"], stream=stream)
