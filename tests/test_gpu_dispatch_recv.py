"""GPU parity of the dispatch's expert side (bounded wait for the counts to
add up, then the per-expert unpack) through the C ABI, against the oracle
on the same seeded inputs: payload rows, fp8 scales, source tokens and
counts byte for byte, with sentinel-filled outputs so that a stray write
shows; run after the dispatch in stream order, and started beside a held
dispatch on a second stream."""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("no GPU", allow_module_level=True)

import combine_ll_moe_amd as ll  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402
from _gpu import DEV, Step, random_case, say, to_dev  # noqa: E402

SENT = 0xA5
FULL_COMPARE_BYTES = 256 << 20
# a hold of about 0.5 ms on the dispatch's stream, so that the receiver is
# already waiting when the dispatch starts
HOLD_CYCLES = 1_200_000


class Outputs:
    """The four output arrays on the GPU, sentinel-filled."""

    def __init__(self, w):
        rows = w.num_experts * w.capacity
        self.pb = 2 * w.hidden if w.dtype == W.BF16 else w.hidden
        self.rows = rows
        self.payload = torch.full((rows, self.pb), SENT, dtype=torch.uint8, device=DEV)
        self.scales = None
        if w.dtype == W.FP8_E4M3:
            self.scales = torch.full((rows, w.hidden // 128), float("nan"), dtype=torch.float32,
                                     device=DEV)
        self.src = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
        self.counts = torch.full((w.num_experts,), -7, dtype=torch.int32, device=DEV)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def launch(self, st: Step, q, expected, max_spins=1 << 20, stream=None):
        w = st.w
        ll.ll_moe_dispatch_recv(st.lay, w.capacity, w.hidden, w.num_experts, w.dtype, q, expected,
                                self.payload, self.scales, self.src, self.counts, max_spins,
                                self.status, stream=stream)


def _check(st: Step, q, outs: Outputs, expected, filled_rows):
    """Compare with the oracle's expert side on the same image."""
    w = st.w
    ref_out = (np.full((outs.rows, outs.pb), SENT, np.uint8),
               np.full((outs.rows, w.hidden // 128), np.nan, np.float32) if outs.scales is not None
               else None,
               np.full(outs.rows, -7, np.int32), np.full(w.num_experts, -7, np.int32))
    payload, scales, src, counts = oracle.dispatch_recv(
        st.img, w.capacity, w.hidden, w.num_experts, w.dtype, q, expected, out=ref_out)
    torch.cuda.synchronize()
    assert int(outs.status.item()) & ~ll.RECV_WAITED == ll.RECV_READY
    assert np.array_equal(outs.counts.cpu().numpy(), counts)
    assert np.array_equal(outs.src.cpu().numpy(), src)
    if outs.rows * outs.pb <= FULL_COMPARE_BYTES:
        g = outs.payload.cpu().numpy()
        if not np.array_equal(g, payload):
            bad = np.argwhere(g != payload)
            raise AssertionError(f"payload differs at {bad.shape[0]} bytes, first {bad[0]}")
        if scales is not None:
            gs = outs.scales.cpu().numpy()
            assert np.array_equal(gs.view(np.uint32), scales.view(np.uint32))
    else:
        # filled rows whole, and a seeded sample of the others for the sentinel
        rows = torch.from_numpy(filled_rows).to(DEV)
        assert np.array_equal(outs.payload.index_select(0, rows).cpu().numpy(),
                              payload[filled_rows])
        if scales is not None:
            assert np.array_equal(outs.scales.index_select(0, rows).cpu().numpy().view(np.uint32),
                                  scales[filled_rows].view(np.uint32))
        rest = np.setdiff1d(np.arange(outs.rows), filled_rows)
        pick = np.random.default_rng(0).choice(rest, size=min(4096, rest.size), replace=False)
        assert (outs.payload.index_select(0, torch.from_numpy(pick).to(DEV)) == SENT).all()
    st.check_signals()


def _filled(w, idx):
    _, cnt = oracle.route(idx, w.num_experts, w.capacity)
    return np.concatenate([e * w.capacity + np.arange(int(cnt[e])) for e in range(w.num_experts)])


def _step(st: Step, q, x, idx, overlapped=False):
    w = st.w
    expected = int(((idx >= 0) & (idx < w.num_experts)).sum())
    outs = Outputs(w)
    if overlapped:
        n, k = idx.shape
        xd, idd = to_dev(x), to_dev(idx)
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(main)  # the output fills and earlier launches come first
        # the dispatch is enqueued (held) before the receiver, so that a
        # shared hardware queue would run it first instead of behind the
        # waiting receiver
        torch.cuda._sleep(HOLD_CYCLES)
        ll.ll_moe_dispatch(st.lay, w.capacity, n, w.hidden, w.num_experts, k, w.dtype, q, xd, idd,
                           stream=main)
        outs.launch(st, q, expected, max_spins=1 << 22, stream=side)
        oracle.dispatch(st.img, w.capacity, w.hidden, w.num_experts, w.dtype, q, x, idx)
        torch.cuda.synchronize()
    else:
        st.dispatch(q, x, idx)
        outs.launch(st, q, expected)
    _check(st, q, outs, expected, _filled(w, idx))
    return int(outs.status.item())


@pytest.mark.parametrize("name", ["tiny", "decode", "decode_fp8", "wide_zipf", "worst_fill"])
def test_unpack_workloads(name):
    w = W.WORKLOADS[name]
    say(f"[expert side] {name}")
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=(name == "tiny"))
    for q in (0, 1):
        _step(st, q, x, idx)
        say(f"[expert side] {name} parity {q} ok")


@pytest.mark.parametrize("name", ["tiny", "decode", "decode_fp8", "wide_zipf", "worst_fill"])
def test_unpack_beside_a_running_dispatch(name):
    w = W.WORKLOADS[name]
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=False)
    waited = 0
    for rep in range(4):
        q = rep & 1
        status = _step(st, q, x, idx, overlapped=True)
        waited += bool(status & ll.RECV_WAITED)
        say(f"[expert side] {name} overlapped parity {q} ok (status {status:#x})")
    # the receiver must really have started before the dispatch finished at
    # least once, or the runs above say nothing about reading during it
    assert waited > 0, "the receiver never found the set incomplete"


@pytest.mark.parametrize("n", [0, 1, 77])
@pytest.mark.parametrize("dtype", [W.BF16, W.FP8_E4M3])
def test_unpack_ragged(n, dtype):
    w = W.Workload("ragged", n, 7168, 256, 8, dtype, "uniform", max_tokens=128, seed=n + 3)
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=False)
    for q in (1, 0):
        _step(st, q, x, idx)


@pytest.mark.parametrize("shape", [
    # (N, Nmax, h, E, K, dtype)
    (5, 8, 8, 1, 1, W.BF16),
    (33, 40, 1032, 17, 5, W.BF16),
    (40, 48, 64, 1000, 4, W.BF16),
    (40, 40, 64, 4096, 4, W.BF16),
    (24, 24, 256, 300, 12, W.FP8_E4M3),
    (3, 3, 128, 5, 4, W.FP8_E4M3),
    (6, 6, 22520, 4, 2, W.BF16),
])
@pytest.mark.parametrize("pad", [0, 48])
def test_unpack_shapes_and_phases(shape, pad):
    n, cap, h, e, k, dt = shape
    w = W.Workload("shape", n, h, e, k, dt, "uniform", max_tokens=cap, seed=h + k + e + 1)
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=True, base_pad=pad)
    for q in (0, 1):
        _step(st, q, x, idx)


def test_unpack_many_rows_per_workgroup():
    """131072 received rows over 256 workgroups: several batches of 64 each."""
    w = W.Workload("many_rows", 8192, 8, 256, 16, W.BF16, "uniform", max_tokens=8192, seed=6)
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=False)
    _step(st, 0, x, idx)


@pytest.mark.parametrize("dtype", [W.BF16, W.FP8_E4M3])
def test_unpack_wide_grid(dtype):
    """Steps that route 64 MiB of messages or more take the receiver's wider
    grid and deeper loads: 16384 messages of 4228 (fp8) or 8196 (bf16)
    bytes, queued and beside a running dispatch."""
    w = W.Workload("wide", 2048, 4096, 64, 8, dtype, "uniform", max_tokens=2048, seed=21 + dtype)
    md, _ = oracle.message_bytes(w.hidden, w.dtype)
    assert w.num_tokens * w.topk * md >= 64 << 20
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=False)
    _step(st, 0, x, idx)
    _step(st, 1, x, idx, overlapped=True)


def test_unpack_masked_entries():
    w = W.Workload("masked", 64, 1024, 16, 4, W.FP8_E4M3, "uniform", seed=12)
    x, idx = W.tokens(w), W.routing(w)
    idx[3, 1] = -1
    idx[10, 0] = w.num_experts
    idx[40, 3] = -5
    st = Step(w, full_image=True)
    _step(st, 1, x, idx)


@pytest.mark.parametrize("delta", [-1, 1])
def test_refusal_when_the_counts_never_add_up(delta):
    """An expected number the counts never reach runs the wait out after
    max_spins polls; the launch ends and the refusal word says so."""
    w = W.WORKLOADS["tiny"]
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=True)
    st.dispatch(0, x, idx)
    outs = Outputs(w)
    outs.launch(st, 0, idx.size + delta, max_spins=8)
    torch.cuda.synchronize()
    assert int(outs.status.item()) & ll.REFUSAL_COUNT_WAIT
    with pytest.raises(oracle.CountsIncomplete):
        oracle.dispatch_recv(st.img, w.capacity, w.hidden, w.num_experts, w.dtype, 0,
                             idx.size + delta)
    st.check_signals()
    # the next step is exact again
    _step(st, 1, x, idx)


@pytest.mark.parametrize("name", ["tiny", "decode_fp8"])
def test_unpack_graph_replays(name):
    """dispatch + dispatch_recv for parity 0 then 1, with the status words
    cleared by a fill kernel inside the graph, replayed three times with
    sentinel fills between replays: every replay unpacks the same bytes."""
    w = W.WORKLOADS[name]
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=False)
    xd, idd = to_dev(x), to_dev(idx)
    expected = int(idx.size)
    outs = [Outputs(w) for _ in range(2)]
    for q in (0, 1):  # eager, checked against the oracle
        st.dispatch(q, x, idx, x_dev=xd, idx_dev=idd)
        outs[q].launch(st, q, expected)
        _check(st, q, outs[q], expected, _filled(w, idx))
    refs = [(o.payload.clone(), None if o.scales is None else o.scales.clone(), o.src.clone(),
             o.counts.clone()) for o in outs]
    n, k = idx.shape
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            gs = torch.cuda.current_stream().cuda_stream
            for q in (0, 1):
                outs[q].status.zero_()
                ll.ll_moe_dispatch(st.lay, w.capacity, n, w.hidden, w.num_experts, k, w.dtype, q,
                                   xd, idd, gs)
                outs[q].launch(st, q, expected, stream=gs)
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:  # eager work between replays
            o.payload.fill_(SENT)
            o.src.fill_(-7)
            o.counts.fill_(-7)
            o.status.fill_(5)
            if o.scales is not None:
                o.scales.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for q in (0, 1):
            o, ref = outs[q], refs[q]
            assert int(o.status.item()) & ~ll.RECV_WAITED == ll.RECV_READY, (r, q)
            assert torch.equal(o.payload, ref[0]) and torch.equal(o.src, ref[2])
            assert torch.equal(o.counts, ref[3])
            if ref[1] is not None:
                assert torch.equal(o.scales.view(torch.int32), ref[1].view(torch.int32))
        say(f"[unpack graph] {name} replay {r} ok")


@pytest.mark.parametrize("block", range(2))
def test_unpack_random_shapes(block):
    """20 seeded random cases (10 per block; any dtype, hidden, expert count,
    top-k, batch and capacity, with repeats, masks and overflow) through the
    dispatch and the expert side, both parities, each against the oracle;
    every layout at a random 16-byte phase of its allocation."""
    for case in range(10):
        rng = np.random.default_rng(4000 + 10 * block + case)
        w, idx = random_case(rng)
        pad = int(rng.choice([0, 16, 32, 48]))
        _, cnt = oracle.route(idx, w.num_experts, w.capacity)
        expected = int(cnt.sum())  # routed messages: masked and overflowing picks excluded
        say(f"[unpack] random case {10 * block + case}: N={w.num_tokens} cap={w.capacity} "
            f"h={w.hidden} E={w.num_experts} K={w.topk} dtype={w.dtype} pad={pad} "
            f"messages={expected}")
        x = W.tokens(w)
        st = Step(w, full_image=False, base_pad=pad)
        for q in (0, 1):
            outs = Outputs(w)
            st.dispatch(q, x, idx)
            outs.launch(st, q, expected)
            _check(st, q, outs, expected, _filled(w, idx))
        del st
        torch.cuda.empty_cache()


# LL_MOE_SWEEP_CASES=n runs n more seeded random cases (seeds 30000 on); the
# default runs none, so that the GPU suite stays short
SWEEP_CASES = int(os.environ.get("LL_MOE_SWEEP_CASES", "0"))


@pytest.mark.skipif(SWEEP_CASES == 0, reason="set LL_MOE_SWEEP_CASES for a longer random sweep")
def test_unpack_random_sweep():
    """A longer sweep of seeded random cases through the dispatch and the
    expert side, both parities, each against the oracle."""
    for seed in range(30000, 30000 + SWEEP_CASES):
        rng = np.random.default_rng(seed)
        w, idx = random_case(rng)
        pad = int(rng.choice([0, 16, 32, 48]))
        _, cnt = oracle.route(idx, w.num_experts, w.capacity)
        expected = int(cnt.sum())
        say(f"[unpack sweep] case {seed}: N={w.num_tokens} cap={w.capacity} h={w.hidden} "
            f"E={w.num_experts} K={w.topk} dtype={w.dtype} pad={pad} messages={expected}")
        x = W.tokens(w)
        st = Step(w, full_image=False, base_pad=pad)
        for q in (0, 1):
            outs = Outputs(w)
            st.dispatch(q, x, idx)
            outs.launch(st, q, expected)
            _check(st, q, outs, expected, _filled(w, idx))
        del st
        torch.cuda.empty_cache()
