"""CPU pins of the oracle's two-phase combine (expert-side put plus flag
hand-off, then the token-side fma chain).

The expected values come from the definition, not from the function under
test: the staged rows are checked against the expert outputs picked through
the routing, the flags against the dispatch counts, and the result against
the oracle's one-shot gather, which forms the same fma chain over the same
values when every token names distinct experts."""
import numpy as np
import pytest

import oracle
import workloads as W

SENT = 0xA5


def _setup(w, q):
    x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
    slot, cnt = oracle.route(idx, w.num_experts, w.capacity)
    rng = np.random.default_rng(w.seed + 11)
    y = rng.integers(0, 1 << 16, size=(w.num_experts * w.capacity, w.hidden), dtype=np.uint16)
    y[(y & 0x7F80) == 0x7F80] = 0x3F80  # no NaN / inf patterns: compare values freely
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype, fill=SENT)
    for p in (0, 1):
        oracle.clean(img, w.capacity, w.hidden, w.num_experts, w.dtype, p)
    oracle.dispatch(img, w.capacity, w.hidden, w.num_experts, w.dtype, q, x, idx)
    return x, idx, wt, y, slot, cnt, img


CASES = [W.WORKLOADS["tiny"],
         W.Workload("tp_fp8", 24, 256, 12, 3, W.FP8_E4M3, "uniform", seed=3),
         W.Workload("tp_zipf", 40, 64, 9, 4, W.BF16, "zipf", max_tokens=48, seed=5)]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("q", [0, 1])
def test_staging_rows_flags_and_untouched_bytes(w, q):
    x, idx, wt, y, slot, cnt, img = _setup(w, q)
    before = img.copy()
    oracle.combine_send(img, w.capacity, w.hidden, w.num_experts, w.dtype, q, y)
    L = oracle.layout(w.capacity, w.hidden, w.num_experts, w.dtype)
    _, mc = oracle.message_bytes(w.hidden, w.dtype)
    stage = L["send"][q]
    changed = np.zeros(img.size, bool)
    for t in range(idx.shape[0]):
        for k in range(idx.shape[1]):
            e = int(idx[t, k])
            if not 0 <= e < w.num_experts:
                continue
            row = stage + (e * w.capacity + t) * mc
            assert int(img[row:row + 4].view(np.int32)[0]) == t
            want = y[e * w.capacity + slot[t, k]]
            assert np.array_equal(img[row + 4:row + mc].view(np.uint16), want)
            changed[row:row + mc] = True
    sig = oracle.signals(img, w.capacity, w.hidden, w.num_experts, w.dtype, q)
    assert np.array_equal(sig, cnt.astype(np.int64) * ((1 << 32) + 1))
    assert not oracle.signals(img, w.capacity, w.hidden, w.num_experts, w.dtype, 1 - q).any()
    for p in (0, 1):
        changed[L["sig"][p]:L["sig"][p] + 8 * w.num_experts] = True
    assert np.array_equal(img[~changed], before[~changed])


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_two_phase_equals_one_shot_gather(w):
    q = 1
    x, idx, wt, y, slot, cnt, img = _setup(w, q)
    fused = oracle.combine(img.copy(), w.capacity, w.hidden, w.num_experts, w.dtype, q, y, idx, wt)
    oracle.combine_send(img, w.capacity, w.hidden, w.num_experts, w.dtype, q, y)
    two = oracle.combine_recv(img, w.capacity, w.hidden, w.num_experts, w.dtype, q, idx, wt)
    assert np.array_equal(two.view(np.uint32), fused.view(np.uint32))


def test_receiver_refuses_without_flags():
    w = CASES[0]
    x, idx, wt, y, slot, cnt, img = _setup(w, 0)
    with pytest.raises(oracle.FlagNotRaised):
        oracle.combine_recv(img, w.capacity, w.hidden, w.num_experts, w.dtype, 0, idx, wt)
    # tokens whose picks are all masked need no flag
    masked = np.full_like(idx, -1)
    out = oracle.combine_recv(img, w.capacity, w.hidden, w.num_experts, w.dtype, 0, masked, wt)
    assert not out.any()


def test_parity_schedule_with_two_phase_combine():
    """dispatch(q), combine_send(q), combine_recv(q) per step: every
    dispatch finds its set's words zero, and each step's words are the
    dispatch counts in both halves."""
    w = CASES[1]
    x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
    _, cnt = oracle.route(idx, w.num_experts, w.capacity)
    y = np.full((w.num_experts * w.capacity, w.hidden), 0x3F80, np.uint16)
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype, fill=SENT)
    args = (w.capacity, w.hidden, w.num_experts, w.dtype)
    for p in (0, 1):
        oracle.clean(img, *args, p)
    for s in range(6):
        q = s & 1
        assert not oracle.signals(img, *args, q).any()
        oracle.dispatch(img, *args, q, x, idx)
        oracle.combine_send(img, *args, q, y)
        out = oracle.combine_recv(img, *args, q, idx, wt)
        assert np.array_equal(oracle.signals(img, *args, q), cnt * ((1 << 32) + 1))
        assert not oracle.signals(img, *args, 1 - q).any()
        # y is all ones, so fmaf(w, 1, acc) is the fp32 sum acc + w: each
        # output is the token's weights summed in ascending k
        ref = np.zeros(w.num_tokens, np.float32)
        for k in range(w.topk):
            ref = (ref + wt[:, k]).astype(np.float32)
        assert np.array_equal(out, np.repeat(ref[:, None], w.hidden, axis=1))
