"""The allocation-free worst-group scan (for callers that cannot allocate)
through the C ABI on an MI355X, against the entry point with a caller
workspace: the same group, maximum and X_worst, bit for bit, on calls in a
row that shrink (so the shared scratch of a larger earlier call must not leak
into a later one), at the scratch's maximum size, and the refusal above it."""
import numpy as np
import pytest
import torch

import mxfp4_activation_rotation_amd as mxq
import workloads as W
from oracle import calibration as CAL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mxq.load()
    return torch.device("cuda:0")


def both(x, lam, dev):
    xd = x.to(dev)
    lam_d = None if lam is None else torch.from_numpy(np.ascontiguousarray(lam, np.float32)).to(dev)
    a = mxq.calib_worst_group(xd, lam_d)
    b = mxq.calib_worst_group_noalloc(xd, lam_d)
    torch.cuda.synchronize()
    a = tuple(t.cpu().numpy() for t in a)
    b = tuple(t.cpu().numpy() for t in b)
    assert int(a[1]) == int(b[1]) and a[2].tobytes() == b[2].tobytes()
    assert np.array_equal(a[0], b[0])
    g_o, linf_o, xw_o = CAL.worst_group(x, lam)
    assert int(b[1]) == g_o and float(b[2]) == linf_o and np.array_equal(b[0], xw_o)
    return int(b[1]), float(b[2])


def test_noalloc_calls_in_a_row(dev):
    rng = np.random.default_rng(9100)
    # 1: large, smoothed, its maximum in group 5 (a large entry the later
    #    calls must not see in the shared scratch)
    x1 = rng.standard_normal((600, 8192))
    x1[17, 5 * 32 + 3] = 900.0
    lam1 = np.exp(0.3 * rng.standard_normal(8192)).astype(np.float32)
    g, _ = both(W.to_dtype(x1, torch.bfloat16), lam1, dev)
    assert g == 5
    # 2: smaller, fp16, no smoothing, its maximum in group 30
    x2 = rng.standard_normal((300, 2048)) * 0.01
    x2[250, 30 * 32 + 31] = 3.0
    g, linf = both(W.to_dtype(x2, torch.float16), None, dev)
    assert g == 30 and linf == float(np.float16(3.0))
    # 3: smaller still, fp32, ragged token count
    x3 = (rng.standard_normal((7, 96)) * 1e-3).astype(np.float32)
    x3[6, 64] = -2.5
    g, _ = both(torch.from_numpy(x3), None, dev)
    assert g == 2


def test_noalloc_at_the_scratch_limit_and_beyond(dev):
    rng = np.random.default_rng(9200)
    C = 262144
    x = rng.standard_normal((4, C))
    x[3, C - 1] = 77.0
    g, _ = both(W.to_dtype(x, torch.bfloat16), None, dev)
    assert g == C // 32 - 1
    big = torch.zeros((1, C + 32), dtype=torch.bfloat16, device=dev)
    with pytest.raises(mxq.MXQError) as e:
        mxq.calib_worst_group_noalloc(big)
    assert e.value.status == 2
    torch.cuda.synchronize()
