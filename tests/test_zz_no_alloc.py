"""The allocation-free grouped call (bsq_grouped_qgemm_noalloc) against the
workspace form (bsq_grouped_qgemm) through the C ABI: the same kernels run
on the same inputs, so the outputs and the status must be bit-identical.  Two
calls in a row, the second smaller (fewer rows, fewer experts, a different
format, an id outside the stack), so the second reads nothing the first left
in the shared routing table."""
import numpy as np
import pytest
import torch

from block_scaled_bit_e2m1_amd import bsq, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(fmt, E, n, k, m, seed, bad=()):
    stack = bsq.to_device(bsq.pack(fmt, workloads.random_weights(E * n, k, seed=seed, sigma=0.02)), DEV)
    ids = np.random.default_rng(seed + 1).integers(0, E, m).astype(np.int32)
    for i in bad:
        ids[i] = E + 3
    x = torch.from_numpy(workloads.random_activations(m, k, seed=seed + 2, act="bf16")).to(torch.bfloat16).to(DEV)
    return stack, torch.from_numpy(ids).to(DEV), x


def _noalloc(stack, E, eids, x, out, status):
    m, k = x.shape
    return bsq.bsq_grouped_qgemm_noalloc(stack.fmt, 0, m, stack.n // E, k, E, bsq._ptr(stack.codes),
                                         bsq._ptr(stack.scales), bsq._ptr(stack.biases), stack.global_scale,
                                         bsq._ptr(eids), bsq._ptr(x), bsq._ptr(out), bsq.BF16, bsq._ptr(status),
                                         bsq._stream(DEV))


def test_noalloc_equals_workspace_entry_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = [("mxfp4", 8, 512, 1024, 1500, 201, ()), ("nvfp8", 3, 200, 512, 300, 211, (5, 77))]
    for fmt, E, n, k, m, seed, bad in cases:
        stack, eids, x = _case(fmt, E, n, k, m, seed, bad)
        ref_status = torch.zeros(1, dtype=torch.int32, device=DEV)
        ref = bsq.grouped_qmm(stack, E, eids, x, status=ref_status)
        out = torch.full((m, n), 3.0, dtype=torch.bfloat16, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        assert _noalloc(stack, E, eids, x, out, status) == bsq.OK, bsq.bsq_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{fmt} m={m}"
        assert int(status.item()) == int(ref_status.item()) == (bsq.ERR_ARG if bad else 0)


def test_noalloc_rejects_tables_beyond_its_array():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    st, need = bsq.bsq_grouped_qgemm_workspace(300000, 8)
    assert st == bsq.OK and need > (1 << 20)
    q = torch.zeros(16, dtype=torch.uint8, device=DEV)
    p = bsq._ptr(q)
    assert bsq.bsq_grouped_qgemm_noalloc(bsq.MXFP4, 0, 300000, 64, 64, 8, p, p, None, 1.0, p, p, p, bsq.BF16, None,
                                         bsq._stream(DEV)) == bsq.ERR_SHAPE
    assert "1048576" in bsq.bsq_last_error()
