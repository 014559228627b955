"""The stream argument of the C ABI: forward and backward enqueued on a
non-default stream, and captured into a graph that is replayed, give the
same bits as the eager calls on the default stream."""

import pytest

from tests.gpu_util import ensure_library, upload
from workloads import DTYPE_BF16, make_inputs_shape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_library()


def _inputs():
    inp = make_inputs_shape(DTYPE_BF16, 1, 4, 2, 700, 700, 128, seed=321, with_grad=True)
    return upload(inp, ("q", "k", "v", "do"))


def _eager(q, k, v, do):
    import torch
    import exact_attention_109_amd as fa
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def test_side_stream_matches_default_stream():
    import torch
    import exact_attention_109_amd as fa
    q, k, v, do = _inputs()
    ref = _eager(q, k, v, do)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o, lse = fa.fwd(q, k, v, causal=True)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    side.synchronize()
    for a, b in zip((o, lse, dq, dk, dv), ref):
        assert torch.equal(a, b)


def test_graph_replays_match_eager():
    import torch
    import exact_attention_109_amd as fa
    q, k, v, do = _inputs()
    ref = _eager(q, k, v, do)
    # warm up on a side stream before capture (torch's recommended pattern)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _eager(q, k, v, do)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, lse = fa.fwd(q, k, v, causal=True)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    for rep in range(3):
        # eager work of the program itself between the replays
        junk = (q.float() * 2).sum()
        torch.cuda.synchronize()
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}: junk {float(junk):.3f}", flush=True)
        for a, b in zip((o, lse, dq, dk, dv), ref):
            assert torch.equal(a, b), rep
