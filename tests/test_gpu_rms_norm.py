"""GPU parity of rms_norm_bf16 (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
import linear_attention_recurrence_step_amd as gdn
from gpu_util import dev, f64, note

pytestmark = pytest.mark.gpu

# float32 output of a float32 computation: the sum of squares over up to ~10^4
# terms and three roundings per element stay far inside 1e-5 relative.
RTOL = 1e-5


def _check(x, w, eps, what, out=None):
    note("rms_norm %s" % what)
    xd, wd = x.to(dev()), w.to(dev())
    got = gdn.rms_norm_bf16(xd, wd, eps, out=out(xd) if out else None)
    torch.cuda.synchronize()
    ref = oracle.rms_norm_bf16(x.reshape(-1, x.shape[-1]), w, eps).reshape(x.shape)
    g = f64(got)
    err = np.abs(g - ref) / (1e-30 + np.abs(ref) + 1e-6)
    assert np.all(np.isfinite(g)), what
    assert float(err.max()) <= RTOL, "%s: worst relative error %.2e" % (what, float(err.max()))
    return got


@pytest.mark.parametrize("n,dim", [(1, 4), (3, 12), (257, 100), (5, 2048), (4096, 2048),
                                   (7, 4096), (2, 8192), (3, 6), (4, 1001), (2, 10000)])
def test_rms_norm_matches_oracle(n, dim):
    x, w = gi.norm_inputs(n, dim, seed=n + dim)
    _check(x, w, 1e-6, "n=%d dim=%d" % (n, dim))


def test_rms_norm_large_eps_batch_dims_and_scale():
    x, w = gi.norm_inputs(6 * 5, 512, seed=11)
    _check(x.reshape(6, 5, 512) * 1e3, w, 0.5, "batched, eps 0.5, scaled")


def test_rms_norm_in_place_and_unaligned_views():
    x, w = gi.norm_inputs(9, 2048, seed=12)
    ref = oracle.rms_norm_bf16(x, w, 1e-6)
    xd = x.to(dev())
    note("rms_norm in place")
    got = gdn.rms_norm_bf16(xd, w.to(dev()), 1e-6, out=xd)
    torch.cuda.synchronize()
    assert got.data_ptr() == xd.data_ptr()
    assert np.max(np.abs(f64(got) - ref) / (np.abs(ref) + 1e-6)) <= RTOL
    # a row view one float in: 4-byte aligned only, so the general path runs
    big = torch.zeros(9 * 2048 + 1, dtype=torch.float32, device=dev())
    view = big[1:].view(9, 2048)
    view.copy_(x.to(dev()))
    wbig = torch.zeros(2049, dtype=torch.bfloat16, device=dev())
    wv = wbig[1:]
    wv.copy_(w.to(dev()))
    note("rms_norm on unaligned views")
    got = gdn.rms_norm_bf16(view, wv, 1e-6)
    torch.cuda.synchronize()
    assert np.max(np.abs(f64(got) - ref) / (np.abs(ref) + 1e-6)) <= RTOL


def test_rms_norm_paths_agree_and_runs_repeat_bitwise():
    """The register path (aligned, dim % 4 == 0) and the general path (the same
    data at an odd offset) compute the same sums in different orders: equal
    within rounding; each path is deterministic."""
    x, w = gi.norm_inputs(33, 1024, seed=13)
    xd, wd = x.to(dev()), w.to(dev())
    a = gdn.rms_norm_bf16(xd, wd, 1e-6)
    b = gdn.rms_norm_bf16(xd, wd, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    big = torch.zeros(33 * 1024 + 1, dtype=torch.float32, device=dev())
    view = big[1:].view(33, 1024)
    view.copy_(xd)
    c = gdn.rms_norm_bf16(view, wd, 1e-6)
    torch.cuda.synchronize()
    assert torch.allclose(a, c, rtol=2e-6, atol=1e-7)


def test_rms_norm_golden_case_exact():
    """The hand-worked case has dyadic results: exact on the GPU too."""
    import json, os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rms_norm_hand.json")))
    x = torch.tensor(gold["x"], dtype=torch.float32)
    w = torch.tensor(gold["weight"]).to(torch.bfloat16)
    note("rms_norm golden case")
    got = gdn.rms_norm_bf16(x.to(dev()), w.to(dev()), gold["eps"])
    torch.cuda.synchronize()
    ref = np.array(gold["out"])
    np.testing.assert_allclose(f64(got)[[0, 2]], ref[[0, 2]], rtol=0, atol=0)
    np.testing.assert_allclose(f64(got)[1], ref[1], rtol=1e-6)


# Past 65536 tokens each workgroup takes several tokens in turn (a launch
# covers at most 2^32 - 1 threads); rows on both sides of the wrap are checked
# against the oracle, for every thread count and for the general path.
@pytest.mark.parametrize("dim", [4, 2048, 4096, 8192, 3])
def test_rms_norm_more_tokens_than_workgroups(dim):
    n = 65536 + 37
    note("rms_norm n=%d dim=%d (workgroups take several tokens)" % (n, dim))
    xd, w = gi.norm_inputs_on_device(n, dim, dev(), seed=dim)
    got = gdn.rms_norm_bf16(xd, w.to(dev()), 1e-6)
    torch.cuda.synchronize()
    rows = [0, 1, 65535, 65536, 65537, n - 1]
    x = xd[rows].cpu()
    ref = oracle.rms_norm_bf16(x, w, 1e-6)
    out = f64(got[rows])
    assert np.max(np.abs(out - ref) / (np.abs(ref) + 1e-6)) <= RTOL
    del xd, got
