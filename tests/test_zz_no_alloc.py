"""The allocation-free statistics entry point (awq_act_stats_noalloc), called
through the C ABI, against the workspace entry point awq_act_stats and the
oracle: bit-exact saliency on two calls in a row, the second with a smaller
input, both on the two-pass path whose partial sums go to the library's fixed
per-GPU scratch; then a one-launch shape that needs none."""
import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_bit_weight_awq_amd as m
    m.load()
    return m


def _noalloc(awq, Xd, out):
    n, k = Xd.shape
    stream = torch.cuda.current_stream().cuda_stream
    return awq.load().awq_act_stats_noalloc(ctypes.c_void_p(Xd.data_ptr()), n, k,
                                            ctypes.c_void_p(out.data_ptr()),
                                            ctypes.c_void_p(stream))


# (4096, 13824): 3.5 MiB of partials; (2048, 4096): 8M elements, smaller, still
# two-pass; (512, 4096): one launch, no scratch
@pytest.mark.parametrize("shapes", [[(4096, 13824, 1), (2048, 4096, 2), (512, 4096, 3)]])
def test_noalloc_matches_workspace_entry_point(awq, shapes):
    for (n, k, seed) in shapes:
        _say(f"noalloc stats {n}x{k}")
        _, X, _ = synth.make_custom(n, k, 1, seed=seed, kind="heavy" if seed == 2 else "normal")
        Xd = torch.from_numpy(X).cuda()
        want = awq.awq_act_stats(Xd)
        out = torch.full((k,), float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc(awq, Xd, out) == 0, awq.load().awq_last_error()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.cpu().numpy().view(np.uint32))
        assert np.array_equal(got.view(np.uint32), O.act_stats(X).view(np.uint32))


def test_noalloc_rejects_shapes_beyond_its_scratch(awq):
    """More partial sums than the fixed scratch holds: rejected on the host
    with AWQ_ERR_WORKSPACE, nothing enqueued (the pointers are never used)."""
    fake = ctypes.c_void_p(0x1000)
    rc = awq.load().awq_act_stats_noalloc(fake, 8193, 1 << 20, fake, None)
    assert rc == awq._lib.AWQ_ERR_WORKSPACE
    assert b"scratch" in awq.load().awq_last_error()
