"""GPU parity of the two-phase combine (expert-side put with per-expert
flags, then the token side's bounded wait and fold) through the C ABI,
against the oracle on the same seeded inputs: staging rows and signal words
byte for byte (the whole layout where the image is small), the folded
output bit for bit, and equal to the one-shot combine's output."""
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
from _gpu import DEV, Step, check_combine, filled_mask, random_case, say, to_dev  # noqa: E402

# a hold of about 0.5 ms on the expert side's stream, so that the token side
# is already waiting when the staging starts
HOLD_CYCLES = 1_200_000


def _inputs(w: W.Workload):
    x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    return x, idx, wt, y


def _two_phase_step(st: Step, q, x, idx, wt, y, y_dev=None):
    st.dispatch(q, x, idx)
    st.check_dispatch(q, idx, restore=False)
    st.combine_send(q, y, y_dev)
    st.check_staging(q, idx)
    out, status, ref = st.combine_recv(q, idx, wt)
    assert status & ~ll.RECV_WAITED == ll.RECV_READY, f"status word {status:#x}"
    st.check_signals()
    diff = check_combine(out, ref)
    assert diff == 0, f"{diff} outputs differ in bits"
    return out


@pytest.mark.parametrize("name", ["tiny", "decode", "decode_fp8", "wide_zipf", "worst_fill"])
def test_two_phase_workloads(name):
    w = W.WORKLOADS[name]
    say(f"[two-phase] {name}: N={w.num_tokens} h={w.hidden} E={w.num_experts} K={w.topk}")
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=(name == "tiny"))
    y_dev = to_dev(y)
    for q in (0, 1):
        out = _two_phase_step(st, q, x, idx, wt, y, y_dev)
        # the same bits as the one-shot combine of the same dispatch
        fused, _ = st.combine(q, y, idx, wt, y_dev=y_dev)
        assert np.array_equal(out.view(np.uint32), fused.view(np.uint32))
        say(f"[two-phase] {name} parity {q} ok")


@pytest.mark.parametrize("n", [0, 1, 77])
@pytest.mark.parametrize("dtype", [W.BF16, W.FP8_E4M3])
def test_two_phase_ragged(n, dtype):
    w = W.Workload("ragged", n, 7168, 256, 8, dtype, "uniform", max_tokens=128, seed=n + 7)
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    for q in (1, 0):
        _two_phase_step(st, q, x, idx, wt, y)


@pytest.mark.parametrize("shape", [
    # (N, Nmax, h, E, K, dtype)
    (5, 8, 8, 1, 1, W.BF16),          # smallest combine message: 20 bytes
    (33, 40, 1032, 17, 5, W.BF16),    # ragged chunk counts
    (16, 16, 512, 64, 16, W.BF16),    # 16 picks
    (40, 48, 64, 1000, 4, W.BF16),    # count prefix in 4 rounds
    (40, 40, 64, 4096, 4, W.BF16),    # largest expert count: 16 rounds
    (24, 24, 256, 300, 12, W.FP8_E4M3),
    (6, 6, 22520, 4, 2, W.BF16),      # largest message, rows from registers past one round
    (9, 9, 10240, 3, 2, W.FP8_E4M3),  # rows from registers past one round
])
@pytest.mark.parametrize("pad", [0, 16, 48])
def test_two_phase_shapes_and_phases(shape, pad):
    n, cap, h, e, k, dt = shape
    w = W.Workload("shape", n, h, e, k, dt, "uniform", max_tokens=cap, seed=h + k + e)
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=True, base_pad=pad)
    for q in (0, 1):
        _two_phase_step(st, q, x, idx, wt, y)


@pytest.mark.parametrize("shape", [
    # (N, h, E, K): the token side's equal runs of columns, as the fused
    # combine's: one run of 160 threads (129 chunks; the last wavefront half
    # there), two of 160, and two streamed runs of 288
    (128, 1032, 16, 4),
    (128, 2056, 16, 8),
    (1024, 4104, 64, 8),
])
def test_two_phase_column_runs(shape):
    n, h, e, k = shape
    w = W.Workload("runs", n, h, e, k, W.BF16, "hotset", seed=h + n)
    say(f"[two-phase] column runs: N={n} h={h} E={e} K={k}")
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    for q in (0, 1):
        _two_phase_step(st, q, x, idx, wt, y)


@pytest.mark.parametrize("pad", [0, 16])
def test_two_phase_staging_through_lds(pad):
    """64 MiB of staged rows or more go through LDS with whole-line stores:
    2048 rows of the largest message (one LDS buffer, rows past four
    rounds)."""
    w = W.Workload("lds_stage", 1024, 22520, 16, 2, W.BF16, "uniform", max_tokens=1024, seed=31)
    mc = 4 + 2 * w.hidden
    assert w.num_tokens * w.topk * mc >= 64 << 20
    x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    st = Step(w, full_image=False, base_pad=pad)
    for q in (0, 1):
        _two_phase_step(st, q, x, idx, wt, y)
        say(f"[two-phase] staging through LDS, pad {pad}, parity {q} ok")


def test_two_phase_many_rows_per_workgroup():
    """131072 received rows: every expert-side workgroup takes more than one
    batch of 64."""
    w = W.Workload("many_rows", 8192, 8, 256, 16, W.BF16, "uniform", max_tokens=8192, seed=4)
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    _two_phase_step(st, 0, x, idx, wt, y)


def test_two_phase_decode_steps():
    base = W.WORKLOADS["decode"]
    st = Step(base, full_image=False)
    y = W.expert_outputs(base)
    y_dev = to_dev(y)
    for s in range(20):
        w = base.with_(seed=3000 + s)
        x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
        _two_phase_step(st, s & 1, x, idx, wt, y, y_dev)
    say("[two-phase] decode 20 steps ok")


@pytest.mark.parametrize("name", ["decode", "wide_zipf", "worst_fill"])
def test_token_side_waits_for_the_flags(name):
    """The token side is launched on its own stream right after the dispatch,
    while the expert side is held back on the main stream: it has to wait
    for the flags, and still folds the staged rows exactly."""
    w = W.WORKLOADS[name]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    yd, idd, wd = to_dev(y), to_dev(idx), to_dev(wt)
    n, k = idx.shape
    waited = 0
    for q in (0, 1):
        st.dispatch(q, x, idx)
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(main)  # the dispatch is complete before the wait starts
        out = torch.full((n, w.hidden), float("nan"), dtype=torch.float32, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        # expert side first (held), so that a shared hardware queue would run
        # it before the waiting token side instead of behind it
        torch.cuda._sleep(HOLD_CYCLES)
        ll.ll_moe_combine_send(st.lay, w.capacity, w.hidden, w.num_experts, w.dtype, q, yd,
                               stream=main)
        ll.ll_moe_combine_recv(st.lay, w.capacity, n, w.hidden, w.num_experts, k, w.dtype, q,
                               idd, wd, out, 1 << 22, status, stream=side)
        oracle.combine_send(st.img, w.capacity, w.hidden, w.num_experts, w.dtype, q, y)
        ref = oracle.combine_recv(st.img, w.capacity, w.hidden, w.num_experts, w.dtype, q, idx, wt)
        torch.cuda.synchronize()
        assert int(status.item()) & ~ll.RECV_WAITED == ll.RECV_READY
        waited += bool(int(status.item()) & ll.RECV_WAITED)
        assert check_combine(out.cpu().numpy(), ref) == 0
        st.check_staging(q, idx)
        say(f"[two-phase] {name} concurrent parity {q} ok (status {int(status.item()):#x})")
    # the token side must really have waited for the flags at least once
    assert waited > 0, "the token side never found a flag down"


def test_refusal_without_expert_side():
    """No expert side: every wait runs out after max_spins polls and the
    status word says so; the launch ends, the other set's words are zeroed,
    and a normal step afterwards is exact."""
    w = W.WORKLOADS["tiny"]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=True)
    st.dispatch(0, x, idx)
    st.check_dispatch(0, idx, restore=False)
    with pytest.raises(oracle.FlagNotRaised):
        oracle.combine_recv(st.img, w.capacity, w.hidden, w.num_experts, w.dtype, 0, idx, wt)
    _, status, _ = st.combine_recv(0, idx, wt, max_spins=16, with_oracle=False)
    assert status & ll.REFUSAL_FLAG_WAIT
    st.check_signals()
    _two_phase_step(st, 1, x, idx, wt, y)


def test_refusal_on_a_short_flag():
    """One expert's flag is left one row short (its count raised by one on
    the host after the expert side): the token side refuses."""
    w = W.WORKLOADS["tiny"]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=True)
    st.dispatch(1, x, idx)
    st.combine_send(1, y)
    st.check_staging(1, idx)
    e = int(idx[0, 0])
    off = st.L["sig"][1] + 8 * e
    word = st.lay[off:off + 8].view(torch.int64)
    word += 1
    st.img[off:off + 8].view(np.int64)[0] += 1
    with pytest.raises(oracle.FlagNotRaised):
        oracle.combine_recv(st.img, w.capacity, w.hidden, w.num_experts, w.dtype, 1, idx, wt)
    _, status, _ = st.combine_recv(1, idx, wt, max_spins=16, with_oracle=False)
    assert status & ll.REFUSAL_FLAG_WAIT


def test_bad_header_stages_nothing():
    """A receive row whose header is outside [0, max_tokens) is not staged
    and not counted, so its expert's flag stays down: the token side refuses
    and no byte outside the other staging rows is written."""
    w = W.WORKLOADS["tiny"]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=True)
    st.dispatch(0, x, idx)
    st.check_dispatch(0, idx, restore=False)
    e = int(idx[5, 1])
    row = st.L["recv"][0] + (e * w.capacity) * st.md  # slot 0 of expert e
    bad = torch.tensor([w.capacity], dtype=torch.int32, device=DEV).view(torch.uint8)
    st.lay[row:row + 4] = bad
    st.img[row:row + 4] = np.array([w.capacity], np.int32).view(np.uint8)
    torch.cuda.synchronize()
    ll.ll_moe_combine_send(st.lay, w.capacity, w.hidden, w.num_experts, w.dtype, 0, to_dev(y))
    # expected image: every other row staged, expert e's flag one short
    lay = oracle.layout(w.capacity, w.hidden, w.num_experts, w.dtype)
    sig = st.img[lay["sig"][0]:lay["sig"][0] + 8 * w.num_experts].view(np.int64)
    counts = sig & 0xFFFFFFFF
    stage = lay["send"][0]
    mc = st.mc
    st.img[lay["sig"][1]:lay["sig"][1] + 8 * w.num_experts] = 0
    for ex in range(w.num_experts):
        staged = 0
        for j in range(int(counts[ex])):
            src = ex * w.capacity + j
            r0 = lay["recv"][0] + src * st.md
            t = int(st.img[r0:r0 + 4].view(np.int32)[0])
            if not 0 <= t < w.capacity:
                continue
            d = stage + (ex * w.capacity + t) * mc
            st.img[d:d + 4] = np.array([t], np.int32).view(np.uint8)
            st.img[d + 4:d + mc] = y[src].view(np.uint8)
            staged += 1
        sig[ex] = counts[ex] | (staged << 32)
    torch.cuda.synchronize()
    st.check_staging(0, idx)
    _, status, _ = st.combine_recv(0, idx, wt, max_spins=16, with_oracle=False)
    assert status & ll.REFUSAL_FLAG_WAIT


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_two_phase_graph_replays(name):
    """Two two-phase steps (parity 0, then 1) captured into a HIP graph with
    the status words cleared by a fill kernel inside it, replayed three
    times with eager work between replays: every replay gives the eager
    bits and a ready status."""
    w = W.WORKLOADS[name]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    xd, idd, wtd, yd = to_dev(x), to_dev(idx), to_dev(wt), to_dev(y)
    refs = [_two_phase_step(st, q, x, idx, wt, y, yd) for q in (0, 1)]
    n, k = idx.shape
    outs = [torch.empty((n, w.hidden), dtype=torch.float32, device=DEV) for _ in range(2)]
    statuses = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(2)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            gs = torch.cuda.current_stream().cuda_stream
            for q in (0, 1):
                statuses[q].zero_()
                ll.ll_moe_dispatch(st.lay, w.capacity, n, w.hidden, w.num_experts, k, w.dtype, q,
                                   xd, idd, gs)
                ll.ll_moe_combine_send(st.lay, w.capacity, w.hidden, w.num_experts, w.dtype, q,
                                       yd, gs)
                ll.ll_moe_combine_recv(st.lay, w.capacity, n, w.hidden, w.num_experts, k,
                                       w.dtype, q, idd, wtd, outs[q], 1 << 20, statuses[q], gs)
    torch.cuda.synchronize()
    for r in range(3):
        for q in (0, 1):  # eager work between replays
            outs[q].fill_(float("nan"))
            statuses[q].fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for q in (0, 1):
            assert int(statuses[q].item()) & ~ll.RECV_WAITED == ll.RECV_READY, (r, q)
            got = outs[q].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), refs[q].view(np.uint32)), (r, q)
        say(f"[two-phase graph] {name} replay {r} ok")


def test_two_phase_masked_entries():
    """Entries outside [0, num_experts) are not dispatched, not staged and
    not folded; the other picks of the same tokens still are."""
    w = W.Workload("masked", 64, 1024, 16, 4, W.BF16, "uniform", seed=13)
    x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
    idx[3, 1] = -1
    idx[10, 0] = w.num_experts
    idx[40, 3] = -5
    idx[41] = -1  # a token with no routed pick: its output row is all +0
    y = W.expert_outputs(w, filled_mask(w, idx))
    st = Step(w, full_image=True)
    for q in (0, 1):
        out = _two_phase_step(st, q, x, idx, wt, y)
        assert (out[41].view(np.uint32) == 0).all()


@pytest.mark.parametrize("n", [64, 2048])
def test_two_phase_fully_masked_tokens(n):
    """Tokens whose every pick is masked write +0.0f through the two-phase
    combine too: alone, as the first or second token of a two-token tile
    (N=2048 with 8 columns of chunks: one run per row, so tiles of two), and
    both tokens of a tile."""
    w = W.Workload("masked", n, 64, 8, 4, W.BF16, "uniform", seed=n + 1)
    rng = np.random.default_rng(n + 1)
    idx = np.stack([rng.permutation(8)[:4] for _ in range(n)]).astype(np.int32)
    for t in (0, 1, 5, 6, 7, n - 2, n - 1):  # tiles (0,1), (6,7), (n-2,n-1) whole; 5 alone
        idx[t] = -1
    idx[9] = [8, -1, 100, -5]
    x, wt = W.tokens(w), W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    say(f"[two-phase] fully masked tokens: N={n}")
    st = Step(w, full_image=True)
    for q in (0, 1):
        out = _two_phase_step(st, q, x, idx, wt, y)
        for t in (0, 1, 5, 6, 7, 9, n - 2, n - 1):
            assert not out[t].view(np.uint32).any(), f"token {t} is not +0.0f"


@pytest.mark.parametrize("block", range(2))
def test_two_phase_random_shapes(block):
    """20 seeded random cases (10 per block; any dtype, hidden, expert count,
    top-k, batch and capacity, with masks and overflow) through the dispatch
    and the two-phase combine, both parities, each against the oracle; every
    layout at a random 16-byte phase of its allocation. The two-phase
    combine takes at most one pick per (token, expert): a repeated expert
    is masked here."""
    for case in range(10):
        rng = np.random.default_rng(3000 + 10 * block + case)
        w, idx = random_case(rng)
        idx = _mask_repeats(idx)
        pad = int(rng.choice([0, 16, 32, 48]))
        say(f"[two-phase] random case {10 * block + case}: N={w.num_tokens} cap={w.capacity} "
            f"h={w.hidden} E={w.num_experts} K={w.topk} dtype={w.dtype} pad={pad}")
        x, wt = W.tokens(w), W.weights(w)
        y = W.expert_outputs(w, filled_mask(w, idx))
        st = Step(w, full_image=False, base_pad=pad)
        y_dev = to_dev(y)
        for q in (0, 1):
            _two_phase_step(st, q, x, idx, wt, y, y_dev)
        del st, y_dev
        torch.cuda.empty_cache()


# LL_MOE_SWEEP_CASES=n runs n more seeded random cases (seeds 20000 on); the
# default runs none, so that the GPU suite stays short
SWEEP_CASES = int(os.environ.get("LL_MOE_SWEEP_CASES", "0"))


def _mask_repeats(idx):
    """The two-phase combine takes at most one pick per (token, expert)."""
    idx = idx.copy()
    for t in range(idx.shape[0]):
        _, first = np.unique(idx[t], return_index=True)
        again = np.ones(idx.shape[1], bool)
        again[first] = False
        idx[t, again] = -1
    return idx


@pytest.mark.skipif(SWEEP_CASES == 0, reason="set LL_MOE_SWEEP_CASES for a longer random sweep")
def test_random_sweep():
    """A longer sweep of seeded random cases (the generator of the random
    shape tests): both parities through the dispatch and the fused combine,
    and every third case also through the two-phase combine with repeated
    experts masked, each against the oracle."""
    for seed in range(20000, 20000 + SWEEP_CASES):
        rng = np.random.default_rng(seed)
        w, idx = random_case(rng)
        pad = int(rng.choice([0, 16, 32, 48]))
        say(f"[sweep] case {seed}: N={w.num_tokens} cap={w.capacity} h={w.hidden} "
            f"E={w.num_experts} K={w.topk} dtype={w.dtype} pad={pad}")
        x, wt = W.tokens(w), W.weights(w)
        y = W.expert_outputs(w, filled_mask(w, idx))
        st = Step(w, full_image=False, base_pad=pad)
        y_dev = to_dev(y)
        for q in (0, 1):
            st.dispatch(q, x, idx)
            st.check_dispatch(q, idx)
            out, ref = st.combine(q, y, idx, wt, y_dev=y_dev)
            st.check_signals()
            assert check_combine(out, ref) == 0, f"case {seed}: combine outputs differ"
        if seed % 3 == 0:
            idx1 = _mask_repeats(idx)
            y1 = W.expert_outputs(w, filled_mask(w, idx1))
            st1 = Step(w, full_image=False, base_pad=pad)
            for q in (0, 1):
                _two_phase_step(st1, q, x, idx1, wt, y1)
            del st1
        del st, y_dev
        torch.cuda.empty_cache()
