"""GPU: the achievable-MFMA-rate diagnostic runs and keeps its products live.

Every chain adds the same product A.B of fixed register operands each round,
so each workgroup's word grows linearly with the number of rounds."""
import pytest
import torch

import adaptive_sparse_attention_amd as ea

from parity_util import require_gpu, say

pytestmark = pytest.mark.gpu


def test_mfma_peak_is_linear_in_rounds():
    require_gpu()
    say("mfma_peak: 8 workgroups, 1 and 3 rounds")
    one = torch.zeros(8, dtype=torch.float32, device="cuda")
    three = torch.zeros(8, dtype=torch.float32, device="cuda")
    f1 = ea.mfma_peak(one, 8, 1)
    f3 = ea.mfma_peak(three, 8, 3)
    torch.cuda.synchronize()
    assert f3 == 3 * f1 == 3 * 2 * 32 * 32 * 16 * 8 * 4 * 8
    assert torch.all(one != 0)
    assert torch.all(one == one[0])
    torch.testing.assert_close(three, 3 * one, rtol=1e-5, atol=0)
