"""The page-copy measurement kernel (kda_page_copy) moves what it claims:
every destination page is a bit copy of its item's source page, padding
entries (slot <= 0 or >= N) read and write nothing, and pages no entry
names keep their bits.  The figures it gives are the traffic ceiling quoted
beside the step kernels, so a copy that skipped or duplicated traffic would
make them meaningless."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("n_dst", [0, 1, 3])
def test_page_copy_copies_pages(n_dst):
    import torch

    from linear_attention_decode_03_amd import kda

    assert torch.cuda.is_available(), "no GPU visible"
    kda.load_library()
    rng = np.random.default_rng(900 + n_dst)
    B, H, N = 6, 3, 1 + 6 * (1 + n_dst) + 2
    pool = rng.standard_normal((N, H, 128, 128)).astype(np.float32)
    perm = rng.permutation(np.arange(1, N, dtype=np.int32))
    src = perm[:B].copy()
    dst = perm[B:B + B * n_dst].reshape(B, n_dst).copy()
    src[1] = 0          # padding: nothing read or written for this request
    src[4] = N + 3      # beyond the pool: padding as well
    if n_dst:
        dst[2, 0] = 0   # a skipped target
    say(f"[page copy] B={B} H={H} N={N} n_dst={n_dst}")
    state = torch.from_numpy(pool).cuda()
    src_t = torch.from_numpy(src).cuda()
    dst_t = torch.from_numpy(np.ascontiguousarray(dst)).cuda() if n_dst else None
    kda.kda_page_copy(state, src_t, dst_t, n_dst)
    torch.cuda.synchronize()
    got = state.cpu().numpy()
    want = pool.copy()
    for b in range(B):
        if not 0 < src[b] < N:
            continue
        for w in range(n_dst):
            if 0 < dst[b, w] < N:
                want[dst[b, w]] = pool[src[b]]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
