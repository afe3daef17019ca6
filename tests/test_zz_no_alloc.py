"""GPU test of pab_attention_backward_noalloc, the backward entry point that
takes its workspace from the library's own device array instead of a caller
buffer (for callers that cannot allocate): through the C ABI its gradients
equal those of pab_attention_backward with a caller workspace, bit for bit
(the same kernels on the same inputs), on two calls in a row where the second
is smaller, and the call itself allocates no device memory through torch.
pab_attention_backward has its own parity tests against the oracle."""
import numpy as np
import pytest
import torch

from tests.test_gpu_backward import _inputs, _quantize

pytestmark = pytest.mark.gpu


def _compare(lib, B, H, N, recipe, causal, seed):
    print("noalloc case B=%d H=%d N=%d %s causal=%s" % (B, H, N, recipe, causal), flush=True)
    _, ts, do = _inputs(B, H, N, 128, seed)
    q, k, v = _quantize(lib, [t.cuda() for t in ts], recipe, 64)
    out, lse = lib.attention_dense(q, k, v, causal=causal, lse=True)
    dout = do.cuda()
    ref = lib.attention_backward(q, k, v, out, dout, lse, causal=causal)
    grads = tuple(torch.full_like(out, float("nan")) for _ in range(3))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = lib.attention_backward_noalloc(q, k, v, out, dout, lse, causal=causal, grads=grads)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for name, a, b in zip("QKV", ref, got):
        assert torch.equal(a, b), name


def test_noalloc_backward_equals_workspace_backward(gpu_lib):
    _compare(gpu_lib, 1, 2, 700, "fp8", True, 11)
    _compare(gpu_lib, 1, 1, 300, "mxfp4", False, 12)     # second call, smaller input


def test_noalloc_backward_rejects_a_problem_beyond_its_array(gpu_lib):
    """A problem whose workspace exceeds the array is refused before any
    launch (PAB_UNSUPPORTED), and the next call still works."""
    N, H = 8192, 8
    assert gpu_lib.backward_workspace_bytes(1, H, N, 128) > gpu_lib.NOALLOC_SCRATCH_BYTES
    z = torch.zeros((1, H, N, 128), dtype=torch.bfloat16, device="cuda")
    q, k, v = _quantize(gpu_lib, [z, z, z], "fp8", 128)
    out = torch.zeros((1, H, N, 128), device="cuda")
    lse = torch.zeros((1, H, N), device="cuda")
    with pytest.raises(gpu_lib.PabError) as e:
        gpu_lib.attention_backward_noalloc(q, k, v, out, out, lse)
    assert e.value.status == gpu_lib.PAB_UNSUPPORTED
    _compare(gpu_lib, 1, 1, 256, "fp8", False, 13)
