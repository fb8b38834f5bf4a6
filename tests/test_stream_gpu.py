"""Launches on a caller's stream other than the default one.

Every entry point enqueues its kernels on the stream it is given (torch's
current stream in the Python binding, or an explicit HIP stream handle) and
nothing else.  The same forward and backward computed on a side stream,
queued behind unrelated work on that stream, and on the default stream must
agree bit for bit (the kernels are deterministic).
"""
import pytest

torch = pytest.importorskip("torch")

import io_aware_exact_03_amd as fa  # noqa: E402
from workloads import random_qkv  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_side_stream_matches_default_stream(d, causal):
    q, k, v, rng = random_qkv(2, 4, 777, d, 500 + d, "bf16")
    do = rng.standard_normal(q.shape).astype("float32")
    tq, tk, tv, tdo = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v, do))
    o0, l0 = fa.fwd(tq, tk, tv, causal=causal)
    g0 = fa.bwd(tq, tk, tv, o0, tdo, l0, causal=causal)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        busy = torch.randn(2048, 2048, device="cuda")
        for _ in range(4):
            busy = (busy @ busy) * 1e-3  # unrelated work queued ahead
        o1, l1 = fa.fwd(tq, tk, tv, causal=causal)
        g1 = fa.bwd(tq, tk, tv, o1, tdo, l1, causal=causal)
    # explicit stream handle, outputs preallocated
    o2 = torch.full_like(tq, float("nan"))
    l2 = torch.full(tq.shape[:3], float("nan"), device="cuda")
    fa.fwd(tq, tk, tv, causal=causal, out=o2, lse=l2, stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(o0, o2) and torch.equal(l0, l2)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)
