"""Host logic of bench.py (no GPU): the algorithmic byte counts the roofline
divides by, and the threaded CPU baseline of the oracle.

The byte counts are checked against totals worked out by hand from the
operand sizes of the KDA step (a 64 KiB FP32 state page per item, a BF16
convolution window of 3 read and T+2 written columns over 3x128 channels,
and the per-token BF16 activations), not against a second copy of the
bench's own expression."""

import numpy as np

import bench
import oracle
from linear_attention_decode_03_amd import inputs


def _tables(B, H, T, slots, accepted=None, record=0):
    p = {"B": B, "H": H, "T": T, "record": record, "slots": np.asarray(slots, np.int32)}
    if accepted is not None:
        p["accepted"] = np.asarray(accepted, np.int32)
    return p


def test_decode_b256_bytes():
    # 8192 live items, each: page read + page written (131072), window taps
    # read 3*384*2 = 2304 and 3 columns written 2304, x 768 + gate 256 +
    # beta 2 + out 256; f_a 256 B per request; slots 1 KiB; weights per head
    # 3*4*128*2 + 128*128*2 + 128*4 + 4 = 36356, plus the norm weight 256.
    slots = np.arange(1, 257)
    got = bench.algorithmic_bytes(_tables(256, 32, 1, slots))
    per_item = 131072 + 2304 + 2304 + 768 + 256 + 2 + 256
    assert got == 8192 * per_item + 256 * 256 + 1024 + 32 * 36356 + 256 == 1123222912


def test_padding_and_record_bytes():
    # decode with two padded requests: each padded item moves its 256 B of
    # zeros only, and no f_a.
    got = bench.algorithmic_bytes(_tables(4, 2, 1, [1, 0, 3, -2]))
    live = 4 * (131072 + 2304 + 2304 + 1282) + 2 * 256
    assert got == live + 4 * 256 + 16 + 2 * 36356 + 256
    # record mode, T = 8: no state written, 1 KiB of records per token,
    # 10 window columns written; accepted picks the read slot's column.
    slots = [[1, 2, 3, 4, 5, 6, 7, 8], [9, 10, 0, 11, 12, 13, 14, 15]]
    got = bench.algorithmic_bytes(_tables(2, 2, 8, slots, accepted=[3, 3], record=1))
    per_item = 65536 + 8 * 1024 + 2304 + 10 * 768 + 8 * (768 + 256 + 2 + 256)
    # request 1 reads slot 0 (column 2): padded, 8 rows of zeros per head
    assert got == 2 * per_item + 2 * 256 * 8 + 256 * 8 + 64 + 8 + 2 * 36356 + 256


def test_threaded_oracle_equals_single_thread():
    p = inputs.make_problem(dict(B=6, H=3, T=4, N=25, W=6, seed=11))
    a, b = inputs.copy_problem(p), inputs.copy_problem(p)
    oracle.run(a)
    r = bench.cpu_baseline_threaded(b, min_seconds=0.0, max_threads=4)
    assert r["cores"] == min(4, len(__import__("os").sched_getaffinity(0)))
    for k in ("state", "conv_state", "out"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_more_than_one_gpu_is_refused():
    # the step has no cross-GPU exchange; the bench measures one GPU and
    # says so for any other count (before touching a device)
    import subprocess
    import sys

    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
