"""fp8_quant_colwise_grouped_noalloc, the entry point that allocates nothing: through the C ABI
(via the binding), its bytes and scales equal those of fp8_quant_colwise_grouped (itself held
bit-exact to the oracle) on two calls in a row, the second on a smaller input, so that the
shared static maxima array must be cleared between calls; too large a problem is rejected."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_grouped_amd as m
    m.lib()
    return m


CASES = [
    # rows, cols, offsets: the first call larger than the second
    (3000, 520, [100, 1100, 1100, 2999, 3000]),
    (700, 64, [300, 300, 700]),
]


@pytest.mark.parametrize("fmt", [0, 1])
def test_noalloc_equals_workspace_entry_on_two_calls(fq, fmt):
    for i, (rows, cols, off) in enumerate(CASES):
        x = workloads.to_torch_bf16(workloads.make_matrix(4000 + i, rows, cols, 1.0, 0.01), DEV)
        offd = torch.tensor(np.asarray(off, np.int32), device=DEV)
        q_ref, s_ref = fq.fp8_quant_colwise_grouped(x, offd, fmt)
        q_na, s_na = fq.fp8_quant_colwise_grouped_noalloc(x, offd, fmt)
        torch.cuda.synchronize()
        assert torch.equal(q_na, q_ref), (i, fmt)
        assert torch.equal(s_na.view(torch.int32), s_ref.view(torch.int32)), (i, fmt)
    # and the last call against the oracle itself
    oq, os_ = oracle.quant_colwise_grouped(workloads.make_matrix(4001, 700, 64, 1.0, 0.01),
                                           np.asarray(CASES[1][2], np.int32), fmt)
    assert np.array_equal(q_na.cpu().numpy(), oq) and np.array_equal(s_na.cpu().numpy(), os_)


def test_noalloc_rejects_problems_beyond_its_array(fq):
    """groups * cols * 4 bytes of maxima beyond the 8 MiB array: FP8Q_ERR_WORKSPACE, nothing
    launched (the outputs keep their fill)."""
    rows, cols, groups = 4, 32768, 128      # 16 MiB of maxima
    x = torch.zeros((rows, cols), dtype=torch.bfloat16, device=DEV)
    off = torch.full((groups,), rows, dtype=torch.int32, device=DEV)
    q = torch.full((cols, rows), 0xAB, dtype=torch.uint8, device=DEV)
    s = torch.full((groups, cols), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(RuntimeError, match="status 3"):
        fq.fp8_quant_colwise_grouped_noalloc(x, off, 1, q_t=q, scales=s)
    torch.cuda.synchronize()
    assert torch.all(q == 0xAB) and torch.all(s == 7.0)
