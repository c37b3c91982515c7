"""The package's device plumbing, under the name the GPU tests use."""

from linear_attention_decode_03_amd.device import (run, run_replay, run_split, to_device,  # noqa: F401
                                                   to_host)
