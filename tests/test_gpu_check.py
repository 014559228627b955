"""On-GPU self-check (fa_fwd_check): near zero on the forward's own
logsumexp, and exactly the closed form |exp(-delta) - 1| when the
logsumexp is shifted by delta; sampled rows of the full-size c3 forward."""

import numpy as np
import pytest

from tests.gpu_util import default_scale, ensure_library, to_f64, upload
from workloads import DTYPE_BF16, DTYPE_F32, WORKLOADS, make_inputs, make_inputs_shape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_library()


CASES = [(DTYPE_BF16, 2, 4, 2, 300, 300, 128, True), (DTYPE_BF16, 1, 2, 2, 77, 513, 64, False),
         (DTYPE_F32, 1, 4, 1, 130, 130, 64, True), (DTYPE_F32, 2, 2, 2, 64, 200, 128, False)]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_check_of_forward_and_of_shifted_lse(case):
    import exact_attention_109_amd as fa
    import torch
    dtype, B, Hq, Hkv, nq, nkv, d, causal = case
    inp = make_inputs_shape(dtype, B, Hq, Hkv, nq, nkv, d, seed=1100 + nq)
    q, k, v = upload(inp)
    o, lse = fa.fwd(q, k, v, causal=causal)
    rows = torch.tensor(sorted({0, 1, nq // 2, nq - 1}), dtype=torch.int32, device="cuda")
    err = to_f64(fa.fwd_check(q, k, lse, rows, causal=causal))
    bound = 2e-3 if dtype == DTYPE_BF16 else 1e-4
    assert np.all(err <= bound), float(err.max())
    for delta in (0.05, -0.2):
        err = to_f64(fa.fwd_check(q, k, lse + delta, rows, causal=causal))
        # sum_j exp(s - lse - delta) = exp(-delta) * (1 + e), |e| <= bound
        expected = abs(np.exp(-delta) - 1.0)
        assert np.all(np.abs(err - expected) <= bound * 1.3), (delta, float(np.abs(err - expected).max()))


def test_check_full_size_c3_sampled_rows():
    import exact_attention_109_amd as fa
    import torch
    w = WORKLOADS["c3"]
    inp = make_inputs(w)
    q, k, v = upload(inp)
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    rows = torch.tensor([0, 1, 255, 256, 4095, 4096, 8190, 8191], dtype=torch.int32, device="cuda")
    err = to_f64(fa.fwd_check(q, k, lse, rows, causal=w.causal, scale=w.scale))
    assert err.shape == (w.B, w.H_q, 8)
    assert np.all(err <= 2e-3), float(err.max())
