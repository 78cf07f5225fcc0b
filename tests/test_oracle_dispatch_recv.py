"""CPU pins of the oracle's expert side of the dispatch (wait for the counts
to add up, then unpack the received messages per expert).

Expected values come from the inputs and the definition, not from the
function under test: the source tokens of expert e are the tokens that name
e, in ascending order (an independent numpy walk of the routing); a bf16
payload row is the token's x row; an fp8 payload row and its scales are the
message the oracle's encoder makes for that token (the encoder has its own
pins); counts are a bincount of the routing."""
import numpy as np
import pytest

import oracle
import workloads as W

SENT = 0xA5


def _dispatched(w, q, idx=None):
    x = W.tokens(w)
    idx = W.routing(w) if idx is None else idx
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype, fill=SENT)
    for p in (0, 1):
        oracle.clean(img, w.capacity, w.hidden, w.num_experts, w.dtype, p)
    oracle.dispatch(img, w.capacity, w.hidden, w.num_experts, w.dtype, q, x, idx)
    return x, idx, img


def _filled_outputs(w):
    rows = w.num_experts * w.capacity
    pb = 2 * w.hidden if w.dtype == W.BF16 else w.hidden
    return (np.full((rows, pb), SENT, np.uint8),
            np.full((rows, w.hidden // 128), np.nan, np.float32) if w.dtype == W.FP8_E4M3 else None,
            np.full(rows, -7, np.int32), np.full(w.num_experts, -7, np.int32))


def _sources(idx, e):
    """Tokens naming expert e, ascending, with one entry per naming pick."""
    t, k = np.nonzero(idx == e)
    order = np.lexsort((k, t))
    return t[order]


CASES = [W.WORKLOADS["tiny"],
         W.Workload("dr_fp8", 24, 256, 12, 3, W.FP8_E4M3, "uniform", seed=3),
         W.Workload("dr_zipf", 40, 64, 9, 4, W.BF16, "zipf", max_tokens=48, seed=5),
         W.Workload("dr_ragged", 5, 128, 6, 2, W.FP8_E4M3, "uniform", max_tokens=9, seed=8)]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("q", [0, 1])
def test_unpacked_rows_sources_and_counts(w, q):
    x, idx, img = _dispatched(w, q)
    before = img.copy()
    valid = (idx >= 0) & (idx < w.num_experts)
    out = _filled_outputs(w)
    payload, scales, src, counts = oracle.dispatch_recv(
        img, w.capacity, w.hidden, w.num_experts, w.dtype, q, int(valid.sum()), out=out)
    assert np.array_equal(counts, np.bincount(idx[valid], minlength=w.num_experts))
    msgs = None
    if w.dtype == W.FP8_E4M3:
        msgs = oracle.encode_messages(x, w.dtype)
    h = w.hidden
    for e in range(w.num_experts):
        ts = _sources(idx, e)
        base = e * w.capacity
        assert np.array_equal(src[base:base + ts.size], ts)
        assert (src[base + ts.size:base + w.capacity] == -7).all()
        assert (payload[base + ts.size:base + w.capacity] == SENT).all()
        for j, t in enumerate(ts):
            if w.dtype == W.BF16:
                assert np.array_equal(payload[base + j], x[t].view(np.uint8))
            else:
                assert np.array_equal(payload[base + j], msgs[t, 4:4 + h])
                assert np.array_equal(scales[base + j].view(np.uint8), msgs[t, 4 + h:])
        if scales is not None:
            assert np.isnan(scales[base + ts.size:base + w.capacity]).all()
    # the layout: set 1-q's words zeroed, nothing else changed
    L = oracle.layout(w.capacity, w.hidden, w.num_experts, w.dtype)
    other = L["sig"][1 - q]
    assert (img[other:other + 8 * w.num_experts] == 0).all()
    before[other:other + 8 * w.num_experts] = 0
    assert np.array_equal(img, before)


def test_masked_entries_are_not_expected():
    w = W.Workload("dr_mask", 16, 64, 5, 3, W.BF16, "uniform", seed=11)
    idx = W.routing(w)
    idx[2, 1] = -1
    idx[7, 0] = w.num_experts
    idx[9, 2] = -100
    x, idx, img = _dispatched(w, 0, idx)
    n_valid = int(((idx >= 0) & (idx < w.num_experts)).sum())
    assert n_valid == w.num_tokens * w.topk - 3
    with pytest.raises(oracle.CountsIncomplete):
        oracle.dispatch_recv(img, w.capacity, w.hidden, w.num_experts, w.dtype, 0,
                             w.num_tokens * w.topk)
    _, _, src, counts = oracle.dispatch_recv(img, w.capacity, w.hidden, w.num_experts, w.dtype,
                                             0, n_valid)
    assert counts.sum() == n_valid
    for e in range(w.num_experts):
        ts = _sources(idx, e)
        assert np.array_equal(src[e * w.capacity:e * w.capacity + ts.size], ts)


@pytest.mark.parametrize("delta", [-1, 1])
def test_refusal_leaves_outputs_alone(delta):
    w = W.WORKLOADS["tiny"]
    _, idx, img = _dispatched(w, 1)
    out = _filled_outputs(w)
    copies = [a.copy() for a in out if a is not None]
    with pytest.raises(oracle.CountsIncomplete):
        oracle.dispatch_recv(img, w.capacity, w.hidden, w.num_experts, w.dtype, 1,
                             idx.size + delta, out=out)
    for a, b in zip([a for a in out if a is not None], copies):
        assert np.array_equal(a, b)


def test_clean_set_unpacks_nothing():
    """Right after a clean, zero messages are expected and none unpacked."""
    w = W.WORKLOADS["tiny"]
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype, fill=SENT)
    for p in (0, 1):
        oracle.clean(img, w.capacity, w.hidden, w.num_experts, w.dtype, p)
    out = _filled_outputs(w)
    payload, _, src, counts = oracle.dispatch_recv(img, w.capacity, w.hidden, w.num_experts,
                                                   w.dtype, 0, 0, out=out)
    assert (counts == 0).all() and (src == -7).all() and (payload == SENT).all()


def test_count_above_capacity_is_taken_as_capacity():
    """A count word above max_tokens (not something a dispatch writes) is
    read as max_tokens, in the completion sum and in the unpacking."""
    w = W.WORKLOADS["tiny"]
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype, fill=SENT)
    for p in (0, 1):
        oracle.clean(img, w.capacity, w.hidden, w.num_experts, w.dtype, p)
    L = oracle.layout(w.capacity, w.hidden, w.num_experts, w.dtype)
    sig = img[L["sig"][0]:L["sig"][0] + 8 * w.num_experts].view(np.int64)
    sig[3] = w.capacity + 50
    sig[5] = 7 | (123 << 32)  # a flag in the high half does not count
    with pytest.raises(oracle.CountsIncomplete):
        oracle.dispatch_recv(img, w.capacity, w.hidden, w.num_experts, w.dtype, 0,
                             w.capacity + 57)
    _, _, src, counts = oracle.dispatch_recv(img, w.capacity, w.hidden, w.num_experts, w.dtype,
                                             0, w.capacity + 7)
    assert counts.tolist() == [0, 0, 0, w.capacity, 0, 7, 0, 0]
    rows = 3 * w.capacity + np.arange(w.capacity)
    recv = L["recv"][0]
    md, _ = oracle.message_bytes(w.hidden, w.dtype)
    hdr = [int(img[recv + r * md:recv + r * md + 4].view(np.int32)[0]) for r in rows]
    assert src[rows].tolist() == hdr
