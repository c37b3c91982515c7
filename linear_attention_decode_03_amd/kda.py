"""Python binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: every step of the KDA decode / verify computation
runs in the HIP kernels of the library.  Operands are torch tensors on the
GPU (PyTorch provides device memory and streams); BF16 operands are
torch.bfloat16 tensors.  Argument errors (status codes 1-5, and 7 for a
misaligned operand) raise ValueError, like the constructor checks of the
KdaWide class on the vLLM kda.wide page; code 6 (launch) raises
RuntimeError.  If the built library is missing the binding raises: it
has no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")
HEAD_DIM = 128

KDA_OK, KDA_ERR_TOKENS, KDA_ERR_GATE_MODE, KDA_ERR_RECORD_T1, KDA_ERR_NULL, KDA_ERR_SHAPE, \
    KDA_ERR_LAUNCH, KDA_ERR_ALIGN, KDA_ERR_WORKSPACE, KDA_ERR_SCRATCH = range(10)

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
# the 17 shared operands: x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots,
# state, out, gate, norm_w, lower_bound, scale, eps, f_b
_OPERANDS = [_P] * 13 + [_F] * 3 + [_P]


def load_library(path: str = LIB_PATH):
    """Loads libkda.so (once) and declares its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        # torch carries its own HIP runtime (soname libamdhip64.so.7, loaded
        # by torch under the name libamdhip64.so).  It has to be in the
        # process before the library, whose libamdhip64.so.7 dependency then
        # binds to it; loaded the other way round the process holds two HIP
        # runtimes, and torch's streams and allocations are not the
        # library's (launches on a torch stream fail).
        import torch  # noqa: F401

        lib = ctypes.CDLL(path)
        lib.kda_decode.restype = _I
        lib.kda_decode.argtypes = _OPERANDS + [_I] * 6 + [_P]
        lib.kda_verify.restype = _I
        lib.kda_verify.argtypes = _OPERANDS + [_P] * 3 + [_I] * 9 + [_P]
        lib.kda_decode_f32conv.restype = _I
        lib.kda_decode_f32conv.argtypes = lib.kda_decode.argtypes
        lib.kda_verify_f32conv.restype = _I
        lib.kda_verify_f32conv.argtypes = lib.kda_verify.argtypes
        lib.kda_validate.restype = _I
        lib.kda_validate.argtypes = _OPERANDS + [_P] * 3 + [_I] * 8
        lib.kda_replay.restype = _I
        lib.kda_replay.argtypes = [_P] * 8 + [_F] + [_I] * 4 + [_P]
        lib.kda_split_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_split_workspace_bytes.argtypes = [_I, _I, _I]
        lib.kda_decode_split.restype = _I
        lib.kda_decode_split.argtypes = _OPERANDS + [_I] * 6 + [_P, ctypes.c_size_t, _P]
        lib.kda_verify_split.restype = _I
        lib.kda_verify_split.argtypes = _OPERANDS + [_P] + [_I] * 8 + [_P, ctypes.c_size_t, _P]
        lib.kda_verify_split_noalloc.restype = _I
        lib.kda_verify_split_noalloc.argtypes = _OPERANDS + [_P] + [_I] * 8 + [_P]
        lib.kda_page_copy.restype = _I
        lib.kda_page_copy.argtypes = [_P] * 3 + [_I] * 4 + [_P]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [_I]
        _lib = lib
    return _lib


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _raise(status: int):
    if status == KDA_OK:
        return
    msg = f"kda: {kda_status_string(status)} (status {status})"
    if status == KDA_ERR_LAUNCH:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(name, t, dtype, ndim, device=None):
    import torch

    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise ValueError(f"{name}: expected a {dtype} tensor")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {ndim}-d tensor, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _sizes(x, state, conv_state, T):
    rows, xcols = x.shape
    N, H = state.shape[0], state.shape[1]
    if tuple(state.shape[2:]) != (HEAD_DIM, HEAD_DIM):
        raise ValueError("state: expected [N, H, 128, 128]")
    if xcols != 3 * H * HEAD_DIM or rows % T:
        raise ValueError("x: expected [B*T, 3*H*128]")
    if conv_state.shape[0] != N or conv_state.shape[1] != 3 * H * HEAD_DIM:
        raise ValueError("conv_state: expected [N, 3*H*128, W]")
    return rows // T, H, N, conv_state.shape[2]


def _gpu_device(state):
    """The GPU the call runs on: that of the state pool.  Host tensors are
    refused here, before any library call (their pointers are not device
    memory)."""
    import torch

    if not isinstance(state, torch.Tensor) or state.device.type != "cuda":
        raise ValueError("state: expected a tensor on a GPU (every operand is device memory)")
    return state.device


def _check_common(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                  gate, norm_w, f_b, B, H, T):
    import torch

    dev = _gpu_device(state)
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    for name, t, dt, nd in (("x", x, bf, 2), ("conv_w", conv_w, bf, 3), ("conv_b", conv_b, bf, 1),
                            ("conv_state", conv_state, conv_state.dtype if conv_state.dtype in
                             (bf, f32) else bf, 3), ("f_a", f_a, bf, 2),
                            ("beta", beta, bf, 2), ("a_log", a_log, f32, 1),
                            ("dt_bias", dt_bias, f32, 1), ("state", state, f32, 4),
                            ("out", out, bf, 2), ("gate", gate, bf, 2), ("norm_w", norm_w, bf, 1),
                            ("f_b", f_b, bf, 2)):
        _check(name, t, dt, nd, dev)
    _check("slots", slots, i32, 1 if T == 1 else 2, dev)
    dim = H * HEAD_DIM
    want = {"conv_w": (conv_w, (3, 4, dim)), "f_a": (f_a, (B * T, HEAD_DIM)),
            "beta": (beta, (B * T, H)), "a_log": (a_log, (H,)), "dt_bias": (dt_bias, (dim,)),
            "out": (out, (B * T, dim)), "gate": (gate, (B * T, dim)),
            "norm_w": (norm_w, (HEAD_DIM,)), "f_b": (f_b, (dim, HEAD_DIM))}
    if conv_b is not None:
        want["conv_b"] = (conv_b, (3 * dim,))
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape:
            raise ValueError(f"{name}: expected shape {shape}, got {tuple(t.shape)}")
    if slots.shape[0] != B:
        raise ValueError("slots: expected B rows")


def _stream(stream, device):
    """The hipStream_t handle: torch's current stream of `device` by default;
    a torch stream must belong to `device`; an int is taken as a raw handle."""
    import torch

    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if hasattr(stream, "cuda_stream"):
        if getattr(stream, "device", device) != device:
            raise ValueError(f"stream: on {stream.device}, operands on {device}")
        return stream.cuda_stream
    return int(stream)


def kda_decode(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
               gate, norm_w, lower_bound, scale, eps, f_b, gate_mode=0, ahead=-1, stream=None):
    """One decode step (T = 1); see kda_decode in include/kda.h (an FP32
    conv_state runs kda_decode_f32conv).  Enqueued on `stream` (default:
    torch's current stream); returns without waiting."""
    import torch

    B, H, N, W = _sizes(x, state, conv_state, 1)
    _check_common(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                  gate, norm_w, f_b, B, H, 1)
    lib = load_library()
    entry = lib.kda_decode_f32conv if conv_state.dtype == torch.float32 else lib.kda_decode
    with torch.cuda.device(state.device):
        status = entry(
            _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(f_a), _ptr(beta),
            _ptr(a_log), _ptr(dt_bias), _ptr(slots), _ptr(state), _ptr(out), _ptr(gate),
            _ptr(norm_w), float(lower_bound), float(scale), float(eps), _ptr(f_b),
            B, H, N, W, int(gate_mode), int(ahead), _stream(stream, state.device))
    _raise(status)


def kda_verify(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
               gate, norm_w, lower_bound, scale, eps, f_b, accepted, rec_u=None, rec_kg=None,
               T=None, record=False, gate_mode=0, ahead=-1, stream=None):
    """One verify step over T = slots.shape[1] tokens unless given; see
    kda_verify in include/kda.h (an FP32 conv_state runs
    kda_verify_f32conv)."""
    import torch

    if slots.dim() != 2:
        raise ValueError("slots: expected [B, slot_stride]")
    T = int(T if T is not None else slots.shape[1])
    if not 1 <= T <= 8:
        _raise(KDA_ERR_TOKENS)
    B, H, N, W = _sizes(x, state, conv_state, T)
    _check_common(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                  gate, norm_w, f_b, B, H, T)
    _check("accepted", accepted, torch.int32, 1, state.device)
    if accepted.shape[0] != B:
        raise ValueError("accepted: expected [B]")
    if record:
        _check("rec_u", rec_u, torch.float32, 4, state.device)
        _check("rec_kg", rec_kg, torch.bfloat16, 4, state.device)
        if tuple(rec_u.shape) != (B, H, T, HEAD_DIM) or \
                tuple(rec_kg.shape) != (B, H, T, 2 * HEAD_DIM):
            raise ValueError("rec_u / rec_kg: expected [B, H, T, 128] / [B, H, T, 256]")
    lib = load_library()
    entry = lib.kda_verify_f32conv if conv_state.dtype == torch.float32 else lib.kda_verify
    with torch.cuda.device(state.device):
        status = entry(
            _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(f_a), _ptr(beta),
            _ptr(a_log), _ptr(dt_bias), _ptr(slots), _ptr(state), _ptr(out), _ptr(gate),
            _ptr(norm_w), float(lower_bound), float(scale), float(eps), _ptr(f_b),
            _ptr(accepted), _ptr(rec_u), _ptr(rec_kg), B, H, N, W, T, int(slots.shape[1]),
            int(bool(record)), int(gate_mode), int(ahead), _stream(stream, state.device))
    _raise(status)


def split_workspace(B, H, T, device):
    """A zero-filled workspace for kda_decode_split / kda_verify_split with B
    requests of H heads and T tokens; calls leave its counters zero, so it
    can be kept and reused on one stream."""
    import torch

    n = int(load_library().kda_split_workspace_bytes(int(B), int(H), int(T)))
    return torch.zeros(max(1, n // 4), dtype=torch.int32, device=device)


def _workspace(workspace):
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def kda_decode_split(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                     out, gate, norm_w, lower_bound, scale, eps, f_b, workspace, split=0,
                     gate_mode=0, stream=None):
    """One decode step with each item split over `split` workgroups (0: the
    library chooses); see kda_decode_split in include/kda.h.  `workspace`:
    a tensor from split_workspace (zero-filled device memory)."""
    import torch

    B, H, N, W = _sizes(x, state, conv_state, 1)
    _check_common(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                  gate, norm_w, f_b, B, H, 1)
    if conv_state.dtype != torch.bfloat16:
        raise ValueError("conv_state: the split step takes a BF16 convolution pool")
    if workspace is not None:
        _check("workspace", workspace, workspace.dtype, 1, state.device)
    ws, ws_bytes = _workspace(workspace)
    with torch.cuda.device(state.device):
        status = load_library().kda_decode_split(
            _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(f_a), _ptr(beta),
            _ptr(a_log), _ptr(dt_bias), _ptr(slots), _ptr(state), _ptr(out), _ptr(gate),
            _ptr(norm_w), float(lower_bound), float(scale), float(eps), _ptr(f_b),
            B, H, N, W, int(gate_mode), int(split), ws, ws_bytes, _stream(stream, state.device))
    _raise(status)


def kda_verify_split(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state,
                     out, gate, norm_w, lower_bound, scale, eps, f_b, accepted, workspace,
                     T=None, split=0, gate_mode=0, stream=None):
    """One plain verify step (no record mode) with each item split over
    `split` workgroups (0: the library chooses); see kda_verify_split in
    include/kda.h."""
    import torch

    if slots.dim() != 2:
        raise ValueError("slots: expected [B, slot_stride]")
    T = int(T if T is not None else slots.shape[1])
    if not 1 <= T <= 8:
        _raise(KDA_ERR_TOKENS)
    B, H, N, W = _sizes(x, state, conv_state, T)
    _check_common(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                  gate, norm_w, f_b, B, H, T)
    if conv_state.dtype != torch.bfloat16:
        raise ValueError("conv_state: the split step takes a BF16 convolution pool")
    _check("accepted", accepted, torch.int32, 1, state.device)
    if accepted.shape[0] != B:
        raise ValueError("accepted: expected [B]")
    if workspace is not None:
        _check("workspace", workspace, workspace.dtype, 1, state.device)
    ws, ws_bytes = _workspace(workspace)
    with torch.cuda.device(state.device):
        status = load_library().kda_verify_split(
            _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(f_a), _ptr(beta),
            _ptr(a_log), _ptr(dt_bias), _ptr(slots), _ptr(state), _ptr(out), _ptr(gate),
            _ptr(norm_w), float(lower_bound), float(scale), float(eps), _ptr(f_b),
            _ptr(accepted), B, H, N, W, T, int(slots.shape[1]), int(gate_mode), int(split),
            ws, ws_bytes, _stream(stream, state.device))
    _raise(status)


def kda_verify_split_noalloc(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots,
                             state, out, gate, norm_w, lower_bound, scale, eps, f_b, accepted,
                             T=None, split=0, gate_mode=0, stream=None):
    """kda_verify_split with the library's static scratch instead of a
    workspace: allocates nothing (see kda_verify_split_noalloc in
    include/kda.h; calls that may overlap on one GPU race)."""
    import torch

    if slots.dim() != 2:
        raise ValueError("slots: expected [B, slot_stride]")
    T = int(T if T is not None else slots.shape[1])
    if not 1 <= T <= 8:
        _raise(KDA_ERR_TOKENS)
    B, H, N, W = _sizes(x, state, conv_state, T)
    _check_common(x, conv_w, conv_b, conv_state, f_a, beta, a_log, dt_bias, slots, state, out,
                  gate, norm_w, f_b, B, H, T)
    if conv_state.dtype != torch.bfloat16:
        raise ValueError("conv_state: the split step takes a BF16 convolution pool")
    _check("accepted", accepted, torch.int32, 1, state.device)
    if accepted.shape[0] != B:
        raise ValueError("accepted: expected [B]")
    with torch.cuda.device(state.device):
        status = load_library().kda_verify_split_noalloc(
            _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(f_a), _ptr(beta),
            _ptr(a_log), _ptr(dt_bias), _ptr(slots), _ptr(state), _ptr(out), _ptr(gate),
            _ptr(norm_w), float(lower_bound), float(scale), float(eps), _ptr(f_b),
            _ptr(accepted), B, H, N, W, T, int(slots.shape[1]), int(gate_mode), int(split),
            _stream(stream, state.device))
    _raise(status)


def kda_replay(rec_u, rec_kg, a_log, dt_bias, src_slots, dst_slots, n_tokens, state,
               lower_bound, stream=None):
    """RecoverSSM replay: the state after the first n_tokens[b] recorded
    tokens, rebuilt from the checkpoint pages src_slots into dst_slots; see
    kda_replay in include/kda.h."""
    import torch

    if rec_u.dim() != 4:
        raise ValueError("rec_u: expected [B, H, T, 128]")
    B, H, T = int(rec_u.shape[0]), int(rec_u.shape[1]), int(rec_u.shape[2])
    dev = _gpu_device(state)
    _check("rec_u", rec_u, torch.float32, 4, dev)
    _check("rec_kg", rec_kg, torch.bfloat16, 4, dev)
    _check("a_log", a_log, torch.float32, 1, dev)
    _check("dt_bias", dt_bias, torch.float32, 1, dev)
    _check("state", state, torch.float32, 4, dev)
    for name, t in (("src_slots", src_slots), ("dst_slots", dst_slots), ("n_tokens", n_tokens)):
        _check(name, t, torch.int32, 1, dev)
        if t.shape[0] != B:
            raise ValueError(f"{name}: expected [B]")
    if tuple(rec_u.shape) != (B, H, T, HEAD_DIM) or tuple(rec_kg.shape) != (B, H, T, 2 * HEAD_DIM):
        raise ValueError("rec_u / rec_kg: expected [B, H, T, 128] / [B, H, T, 256]")
    if tuple(a_log.shape) != (H,) or tuple(dt_bias.shape) != (H * HEAD_DIM,):
        raise ValueError("a_log / dt_bias: expected [H] / [H*128]")
    if state.shape[1] != H or tuple(state.shape[2:]) != (HEAD_DIM, HEAD_DIM):
        raise ValueError("state: expected [N, H, 128, 128]")
    lib = load_library()
    with torch.cuda.device(dev):
        status = lib.kda_replay(
            _ptr(rec_u), _ptr(rec_kg), _ptr(a_log), _ptr(dt_bias), _ptr(src_slots),
            _ptr(dst_slots), _ptr(n_tokens), _ptr(state), float(lower_bound), B, H,
            int(state.shape[0]), T, _stream(stream, dev))
    _raise(status)


def kda_page_copy(state, src_slots, dst_slots, n_dst, stream=None):
    """A measurement aid: the step's state-page reads and writes without the
    compute (see kda_page_copy in include/kda.h).  src_slots [B], dst_slots
    [B, n_dst] int32 on the GPU of `state`."""
    import torch

    dev = _gpu_device(state)
    _check("state", state, torch.float32, 4, dev)
    _check("src_slots", src_slots, torch.int32, 1, dev)
    B, H, N = int(src_slots.shape[0]), int(state.shape[1]), int(state.shape[0])
    if n_dst:
        _check("dst_slots", dst_slots, torch.int32, 2, dev)
        if tuple(dst_slots.shape) != (B, n_dst):
            raise ValueError("dst_slots: expected [B, n_dst]")
    with torch.cuda.device(dev):
        status = load_library().kda_page_copy(_ptr(state), _ptr(src_slots), _ptr(dst_slots),
                                              int(n_dst), B, H, N, _stream(stream, dev))
    _raise(status)


def kda_validate(*, B, H, N, W, T, slot_stride=1, record=0, gate_mode=0, lower_bound=-5.0,
                 scale=0.08838834764831845, eps=1e-6, pointers=None):
    """The library's host-side argument checks, with no device work.
    `pointers` maps operand names to integers (NULL when missing; by default
    every operand gets a dummy non-NULL value).  Returns the status code."""
    names = ["x", "conv_w", "conv_b", "conv_state", "f_a", "beta", "a_log", "dt_bias", "slots",
             "state", "out", "gate", "norm_w", "f_b", "accepted", "rec_u", "rec_kg"]
    ptrs = {n: 0x1000 for n in names}
    ptrs["conv_b"] = 0
    if pointers:
        ptrs.update(pointers)
    p = lambda n: ptrs[n] or None  # noqa: E731
    return load_library().kda_validate(
        p("x"), p("conv_w"), p("conv_b"), p("conv_state"), p("f_a"), p("beta"), p("a_log"),
        p("dt_bias"), p("slots"), p("state"), p("out"), p("gate"), p("norm_w"),
        float(lower_bound), float(scale), float(eps), p("f_b"), p("accepted"), p("rec_u"),
        p("rec_kg"), int(B), int(H), int(N), int(W), int(T), int(slot_stride), int(record),
        int(gate_mode))
