"""cce_forward_static (the forward that allocates nothing: the library's own
device scratch is its workspace) against cce_forward on a caller workspace:
two calls in a row through the C ABI, the second with a smaller input, each
bit for bit equal to cce_forward's result; and the size limit."""
import numpy as np
import pytest

from linear_cross_entropy_libcce_amd import cce
from linear_cross_entropy_libcce_amd import synthetic as syn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cce.load()
    return torch


def test_static_forward_matches_cce_forward_twice(torch_cuda):
    torch = torch_cuda
    # the same head, a larger then a smaller token batch (masks, softcap, an
    # affine head: the bias block runs); the second call reuses the scratch
    # the first one left behind
    big = syn.make_custom(M=700, H=1024, V=5000, bits=8, seed=91, softcap=30.0, mask="random", mask_frac=0.2,
                          bias="affine")
    small = syn.make_custom(M=37, H=1024, V=5000, bits=8, seed=92, softcap=30.0, bias="affine")
    small.update(wq=big["wq"], scales=big["scales"], biases=big["biases"])
    head = cce.head_from_numpy(big)
    assert cce.forward_workspace_bytes(head, 700) <= cce.STATIC_SCRATCH_BYTES
    for inp in (big, small):
        h, t, m = cce.tokens_from_numpy(inp)
        logp0, lse0 = cce.cce_forward(h, head, t, m)
        logp1, lse1 = cce.cce_forward_static(h, head, t, m)
        torch.cuda.synchronize()
        assert torch.equal(logp0, logp1) and torch.equal(lse0, lse1)
        assert bool(torch.isfinite(logp1).all()) and float(logp1.abs().sum()) > 0


def test_static_forward_rejects_what_does_not_fit(torch_cuda):
    # a plan larger than the scratch: CCE_ERR_WORKSPACE before any launch, and
    # the outputs left as they were
    torch = torch_cuda
    inp = syn.make_custom(M=8, H=4096, V=200000, bits=8, seed=93)
    head = cce.head_from_numpy(inp)
    assert cce.forward_workspace_bytes(head, 8) > cce.STATIC_SCRATCH_BYTES
    h, t, m = cce.tokens_from_numpy(inp)
    logp = torch.full((8,), 7.0, device="cuda")
    lse = torch.full((8,), 7.0, device="cuda")
    with pytest.raises(cce.CceError) as e:
        cce.cce_forward_static(h, head, t, m, out=(logp, lse))
    assert e.value.status == cce.CCE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((logp == 7.0).all()) and bool((lse == 7.0).all())
