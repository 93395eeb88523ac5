"""GPU parity of the expert-grouped quantized matmul (bsq_grouped_qgemm).

Its result is the routed gather's, out[i] = x[i] . dequant(expert ids[i])^T,
so the oracle is oracle.gather_matmul on the same seeded inputs, to the
bf16 bound |gpu - ref| <= 2e-3 * sum|x*w| per output.  The cases span experts
with no rows, one row, a ragged multiple of the 128-row tile, ragged n and k
(both tile configurations), the largest expert count, ids outside the stack,
graph replay, the decode form (m <= 32: routed inside the GEMV kernel, one
round or guarded rounds of the k split) with shared, lone and bad ids, and
the prefill MoE workload at full size on sampled rows.  The
output and the workspace sit between guard bands that must come back
untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_bit_e2m1_amd import bsq, workloads
from tests.test_gpu_parity import ALL, DEV, check_bound

pytestmark = pytest.mark.gpu

CANARY = -12352.0  # exactly representable in bf16 (-193 * 2^6) and f32
WS_CANARY = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsq.lib()
    oracle.lib()
    yield
    torch.cuda.synchronize()


def _stack(fmt, E, n, k, seed, W=None):
    if W is None:
        W = workloads.random_weights(E * n, k, seed=seed, sigma=0.02)
    p = oracle.pack(fmt, W)
    pw = bsq.PackedWeight(p["fmt"], E * n, k, torch.from_numpy(p["codes"]), torch.from_numpy(p["scales"]),
                          None if p["biases"] is None else torch.from_numpy(p["biases"]), p["global"])
    return p, bsq.to_device(pw, DEV)


def _ids_with_counts(counts, seed):
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    return np.random.default_rng(seed).permutation(ids).astype(np.int32)


def _run(stack, E, ids, X, out_dtype=torch.bfloat16):
    """The grouped matmul with guard rows around the output and a guard tail
    after the workspace; returns (out f32 numpy, status)."""
    m, n = len(ids), stack.n // E
    x = torch.from_numpy(np.ascontiguousarray(X, np.float32)).to(torch.bfloat16).to(DEV)
    eids = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(DEV)
    st, need = bsq.bsq_grouped_qgemm_workspace(m, E)
    assert st == bsq.OK
    ws = torch.full((need + 256,), WS_CANARY, dtype=torch.uint8, device=DEV)
    buf = torch.full((m + 2, n), CANARY, dtype=out_dtype, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    bsq.grouped_qmm(stack, E, eids, x, out=buf[1:m + 1], status=status, workspace=ws[:need])
    torch.cuda.synchronize()
    b = buf.float().cpu().numpy()
    assert (b[0] == CANARY).all() and (b[m + 1] == CANARY).all(), "output guard rows overwritten"
    assert (ws[need:].cpu().numpy() == WS_CANARY).all(), "workspace guard tail overwritten"
    return b[1:m + 1], int(status.item())


def _check(fmt, p, X, ids, n, out, rows=None, what=""):
    rows = np.arange(len(ids)) if rows is None else rows
    ref, den = oracle.gather_matmul(X[rows], oracle.dequant_packed(p), ids[rows], n)
    check_bound(out[rows], ref, den, 2e-3, f"grouped {fmt} {what}", True)


@pytest.mark.parametrize("fmt", ALL)
def test_grouped_parity_narrow_tiles(fmt):
    """6 experts of 200 x 512: counts 140 (two tiles, ragged), 0, 1, 129, 30,
    0 in a shuffled order; 128x64 tiles; bf16 and f32 output."""
    E, n, k = 6, 200, 512
    p, stack = _stack(fmt, E, n, k, seed=71)
    ids = _ids_with_counts([140, 0, 1, 129, 30, 0], seed=72)
    X = workloads.random_activations(len(ids), k, seed=73, act="bf16")
    for dt in (torch.bfloat16, torch.float32):
        out, st = _run(stack, E, ids, X, dt)
        assert st == 0
        if dt == torch.bfloat16:
            _check(fmt, p, X, ids, n, out, what="bf16 out")
        else:
            ref, den = oracle.gather_matmul(X, oracle.dequant_packed(p), ids, n)
            check_bound(out, ref, den, 2e-3, f"grouped {fmt} f32 out")


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("k", [512, 384])
def test_grouped_parity_wide_tiles(fmt, k):
    """4 experts of 3900 x k with 600 rows: the 128x256 step-ahead tiles
    (k = 512 takes the three-slice scale path where the format has one,
    k = 384 the other), ragged in n against 256."""
    E, n = 4, 3900
    p, stack = _stack(fmt, E, n, k, seed=81)
    ids = _ids_with_counts([300, 17, 0, 283], seed=82)
    X = workloads.random_activations(len(ids), k, seed=83, act="bf16")
    out, st = _run(stack, E, ids, X)
    assert st == 0
    rows = np.sort(np.random.default_rng(84).choice(len(ids), 160, replace=False))
    _check(fmt, p, X, ids, n, out, rows, f"wide k={k}")


@pytest.mark.parametrize("fmt", ALL)
def test_grouped_parity_few_rows_per_expert(fmt):
    """Few rows per expert on the 128-row MFMA tiles: 8 experts of 300 x 512
    with 100 rows (experts of 30, 33 and 1 rows, empty experts) and 4
    experts with 200 rows (70, 64, 1, 65); every row, bf16 and f32 output."""
    n, k = 300, 512
    for E, counts, seed in ((8, [30, 0, 1, 33, 12, 24, 0, 0], 75), (4, [70, 64, 1, 65], 78)):
        p, stack = _stack(fmt, E, n, k, seed=seed)
        ids = _ids_with_counts(counts, seed=seed + 1)
        X = workloads.random_activations(len(ids), k, seed=seed + 2, act="bf16")
        ref, den = oracle.gather_matmul(X, oracle.dequant_packed(p), ids, n)
        for dt in (torch.bfloat16, torch.float32):
            out, st = _run(stack, E, ids, X, dt)
            assert st == 0
            check_bound(out, ref, den, 2e-3, f"grouped few rows {fmt} E={E} m={len(ids)} {dt}", dt == torch.bfloat16)


@pytest.mark.parametrize("fmt", ALL)
def test_grouped_parity_more_than_one_round(fmt):
    """8 experts of 3900 x 256 with 2100 rows: more than 256 wide tiles, where
    the float formats switch to 128x128 tiles (two workgroups per CU) and
    int4 / int8 keep the 128x256 ones; ragged n and ragged expert groups."""
    E, n, k = 8, 3900, 256
    p, stack = _stack(fmt, E, n, k, seed=91)
    ids = _ids_with_counts([400, 129, 0, 383, 1, 500, 300, 387], seed=92)
    X = workloads.random_activations(len(ids), k, seed=93, act="bf16")
    out, st = _run(stack, E, ids, X)
    assert st == 0
    rows = np.sort(np.random.default_rng(94).choice(len(ids), 200, replace=False))
    _check(fmt, p, X, ids, n, out, rows, "more than one round")


@pytest.mark.parametrize("fmt", ALL)
def test_grouped_decode_form(fmt):
    """m <= 32 routed rows take the decode form (routed in the kernel, tiles
    of up to 4 rows of one expert, one weight pass per tile); at k = 4096 its
    one-round kernel: 4 experts of 1000 x 4096 (ragged against every
    row group) with rows shared between tokens; m = 1, 5 (tiles of 2 and 3
    rows), 19 (an expert with 9 rows spans three tiles) and 32; bf16 and f32
    output."""
    E, n, k = 4, 1000, 4096
    p, stack = _stack(fmt, E, n, k, seed=61)
    W = oracle.dequant_packed(p)
    for counts in ([1, 0, 0, 0], [2, 0, 3, 0], [9, 4, 0, 6], [8, 8, 8, 8]):
        ids = _ids_with_counts(counts, seed=62 + sum(counts))
        X = workloads.random_activations(len(ids), k, seed=63 + len(ids), act="bf16")
        ref, den = oracle.gather_matmul(X, W, ids, n)
        for dt in (torch.bfloat16, torch.float32):
            out, st = _run(stack, E, ids, X, dt)
            assert st == 0
            check_bound(out, ref, den, 2e-3, f"grouped decode {fmt} m={len(ids)} {dt}", dt == torch.bfloat16)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("k", [64, 4160, 14336])
def test_grouped_decode_form_any_k(fmt, k):
    """The decode form away from k = 4096: guarded rounds of the k split.
    k = 64 (fewer chunks than one round, some waves add nothing), 4160 (one
    full round and a partial one) and 14336 (3.5 rounds, an MoE down
    projection's k); 4 experts of 300 rows, 9 routed rows in tiles of 4 + 1,
    3 and 1; bf16 and f32 output."""
    E, n = 4, 300
    p, stack = _stack(fmt, E, n, k, seed=69)
    ids = _ids_with_counts([5, 0, 3, 1], seed=70)
    X = workloads.random_activations(len(ids), k, seed=71, act="bf16")
    ref, den = oracle.gather_matmul(X, oracle.dequant_packed(p), ids, n)
    for dt in (torch.bfloat16, torch.float32):
        out, st = _run(stack, E, ids, X, dt)
        assert st == 0
        check_bound(out, ref, den, 2e-3, f"grouped decode {fmt} k={k} {dt}", dt == torch.bfloat16)


def test_grouped_decode_form_bad_ids_and_equal_to_gather():
    """Decode-sized m with ids outside [0, E): those rows are zero and the
    status is set; every other row meets the bound against the oracle, as
    the per-row gather of the same rows does.  Calls with no valid id at all
    give all-zero outputs."""
    E, n, k = 6, 600, 4096
    p, stack = _stack("mxfp4", E, n, k, seed=64)
    ids = np.array([3, -1, 3, 5, 0, 6, 3, 5, 0, 3], np.int32)
    X = workloads.random_activations(len(ids), k, seed=65, act="bf16")
    out, st = _run(stack, E, ids, X)
    assert st == 1
    bad = (ids < 0) | (ids >= E)
    assert (out[bad] == 0).all()
    good = ~bad
    x = torch.from_numpy(np.ascontiguousarray(X[good])).to(torch.bfloat16).to(DEV)
    g = bsq.gather_qmm(stack, E, torch.from_numpy(ids[good]).to(DEV), x).float().cpu().numpy()
    ref, den = oracle.gather_matmul(X[good], oracle.dequant_packed(p), ids[good], n)
    check_bound(out[good], ref, den, 2e-3, "grouped decode vs oracle", True)
    check_bound(g, ref, den, 2e-3, "gather vs oracle", True)
    for ids in (np.array([7], np.int32), np.array([-3, 6, 99], np.int32)):  # no valid row at all
        out, st = _run(stack, E, ids, X[:len(ids)], torch.float32)
        assert st == 1 and (out == 0).all()


def test_grouped_max_experts_and_single_expert():
    """1024 experts (the most the routing takes) with 1500 random rows, most
    experts holding 0-3 rows; and one expert holding every row."""
    E, n, k = 1024, 64, 256
    p, stack = _stack("nvfp4", E, n, k, seed=91)
    ids = np.random.default_rng(92).integers(0, E, 1500).astype(np.int32)
    X = workloads.random_activations(len(ids), k, seed=93, act="bf16")
    out, st = _run(stack, E, ids, X)
    assert st == 0
    _check("nvfp4", p, X, ids, n, out, what="1024 experts")
    p1, stack1 = _stack("mxfp8_e4m3", 1, 300, 256, seed=94)
    ids1 = np.zeros(333, np.int32)
    X1 = workloads.random_activations(333, 256, seed=95, act="bf16")
    out1, st1 = _run(stack1, 1, ids1, X1)
    assert st1 == 0
    _check("mxfp8_e4m3", p1, X1, ids1, 300, out1, what="one expert")


def test_grouped_bad_ids_zero_rows_and_set_status():
    E, n, k = 4, 96, 256
    p, stack = _stack("mxfp4", E, n, k, seed=101)
    ids = np.array([1, 7, 0, -1, 3, 3, 4], np.int32)  # 7, -1 and 4 are outside [0, 4)
    X = workloads.random_activations(len(ids), k, seed=102, act="bf16")
    out, st = _run(stack, E, ids, X)
    assert st == bsq.ERR_ARG
    bad = np.array([1, 3, 6])
    good = np.array([0, 2, 4, 5])
    assert (out[bad] == 0).all()
    _check("mxfp4", p, X, ids, n, out, good, "good rows")
    out2, st2 = _run(stack, E, np.array([9, 9, -3], np.int32), X[:3])  # no row routes anywhere
    assert st2 == bsq.ERR_ARG and (out2 == 0).all()


def test_grouped_deterministic():
    """The order of rows inside an expert's group varies with the atomics; the
    result does not."""
    E, n, k = 3, 256, 512
    _, stack = _stack("int4_affine", E, n, k, seed=111)
    ids = np.random.default_rng(112).integers(0, E, 700).astype(np.int32)
    X = workloads.random_activations(700, k, seed=113, act="bf16")
    a, _ = _run(stack, E, ids, X)
    b, _ = _run(stack, E, ids, X)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_grouped_degenerate_and_rejected():
    E, n, k = 2, 64, 256
    _, stack = _stack("mxfp4", E, n, k, seed=121)
    s = bsq._stream(DEV)
    ws = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    x = torch.zeros((3, k), dtype=torch.bfloat16, device=DEV)
    eids = torch.zeros(3, dtype=torch.int32, device=DEV)
    out = torch.full((3, n), 7.0, dtype=torch.bfloat16, device=DEV)
    P = bsq._ptr
    # k = 0: the empty sum, zeros
    st = bsq.bsq_grouped_qgemm(stack.fmt, 0, 3, n, 0, E, None, None, None, 1.0, None, None, P(out), bsq.BF16,
                               None, 0, None, s)
    assert st == bsq.OK
    torch.cuda.synchronize()
    assert (out == 0).all()
    # m = 0: nothing to do
    st = bsq.bsq_grouped_qgemm(stack.fmt, 0, 0, n, k, E, P(stack.codes), P(stack.scales), None, 1.0, None, None,
                               None, bsq.BF16, None, 0, None, s)
    assert st == bsq.OK
    args = (P(stack.codes), P(stack.scales), None, 1.0, P(eids), P(x), P(out), bsq.BF16)
    assert bsq.bsq_grouped_qgemm(stack.fmt, 0, 3, n, k, 0, *args, P(ws), 4096, None, s) == bsq.ERR_ARG
    assert bsq.bsq_grouped_qgemm(stack.fmt, 0, 3, n, k, 1025, *args, P(ws), 4096, None, s) == bsq.ERR_SHAPE
    assert bsq.bsq_grouped_qgemm(stack.fmt, 0, 3, n, k, E, *args, P(ws), 8, None, s) == bsq.ERR_ARG
    assert bsq.bsq_grouped_qgemm(stack.fmt, 0, 3, n, k, E, *args, None, 4096, None, s) == bsq.ERR_ARG
    xo = torch.zeros(3 * k + 8, dtype=torch.bfloat16, device=DEV)[1:1 + 3 * k]
    assert bsq.bsq_grouped_qgemm(stack.fmt, 0, 3, n, k, E, P(stack.codes), P(stack.scales), None, 1.0, P(eids),
                                 P(xo), P(out), bsq.BF16, P(ws), 4096, None, s) == bsq.ERR_ALIGN
    with pytest.raises(ValueError):
        bsq.grouped_qmm(stack, E, eids, x.float())
    torch.cuda.synchronize()
    assert (out == 0).all()  # no rejected call wrote anything


def test_grouped_graph_replay():
    """Routing and matmul captured in a HIP graph: every replay, with eager
    work between replays, equals the eager result; so does the decode form
    (12 rows, routed inside the kernel, one bad id) in the same graph."""
    E, n, k = 5, 320, 512
    _, stack = _stack("mxfp8_e5m2", E, n, k, seed=131)
    ids = np.random.default_rng(132).integers(0, E, 400).astype(np.int32)
    x = torch.from_numpy(workloads.random_activations(400, k, seed=133, act="bf16")).to(torch.bfloat16).to(DEV)
    eids = torch.from_numpy(ids).to(DEV)
    _, need = bsq.bsq_grouped_qgemm_workspace(400, E)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ref = bsq.grouped_qmm(stack, E, eids, x, workspace=ws).clone()
    out = torch.empty_like(ref)
    dids = torch.tensor([4, 0, 4, 2, 9, 4, 0, 1, 4, 2, 3, 4], dtype=torch.int32, device=DEV)  # 9 is outside [0, 5)
    dx = x[:12]
    dws = torch.empty(max(bsq.bsq_grouped_qgemm_workspace(12, E)[1], 4), dtype=torch.uint8, device=DEV)
    dst = torch.zeros(1, dtype=torch.int32, device=DEV)
    dref = bsq.grouped_qmm(stack, E, dids, dx, workspace=dws).clone()
    dout = torch.empty_like(dref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bsq.grouped_qmm(stack, E, eids, x, out=out, workspace=ws)
        bsq.grouped_qmm(stack, E, dids, dx, out=dout, workspace=dws, status=dst)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        bsq.grouped_qmm(stack, E, eids, x, out=out, workspace=ws)
        bsq.grouped_qmm(stack, E, dids, dx, out=dout, workspace=dws, status=dst)
    for _ in range(3):
        out.fill_(0)
        dout.fill_(7)
        dst.zero_()
        ws.fill_(0xFF)
        bsq.qgemv(stack, x[:1])  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(dout, dref) and (dout[4] == 0).all() and int(dst.item()) == bsq.ERR_ARG


def test_grouped_workload_moe_prefill_sampled():
    """The prefill MoE workload at full size (1024 tokens, top-2 of 8 mxfp4
    experts of 4096 x 4096) in the configuration the benchmark times, against
    the oracle on 64 seeded rows."""
    wl = workloads.MOE_WORKLOADS["mxfp4_moe_prefill_8x4096"]
    W, X, ids = workloads.generate_moe(wl)
    p, stack = _stack(wl.fmt, wl.experts, wl.n, wl.k, 0, W=W)
    del W
    out, st = _run(stack, wl.experts, ids, X)
    assert st == 0
    rows = np.sort(np.random.default_rng(wl.seed + 7).choice(wl.m, 64, replace=False))
    _check(wl.fmt, p, X, ids, wl.n, out, rows, "moe prefill workload")
