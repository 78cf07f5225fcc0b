"""Publish order of the dispatch's counts, seen by a concurrent consumer.

A count may rise only after the messages it counts are visible at device
scope (mscclpp.h, the put-then-signal contract above struct mscclppDevConn).
No value left behind by a finished dispatch can show this order, so a
consumer kernel (ll_moe_diag_watch) runs on a second stream while the
dispatch runs: it acquires the counts over and over and checks, each time,
that every expert has at least as many complete receive rows as its
acquired count, a row being complete when every byte equals the message of
the token its slot belongs to (the oracle's encoding, bf16 or fp8). The
receive rows start as a sentinel that is no message. The dispatch output is
then compared with the oracle as in the parity tests.
"""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("no GPU", allow_module_level=True)

import numpy as np  # noqa: E402

import combine_ll_moe_amd as ll  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402
from _gpu import DEV, Step, say, to_dev  # noqa: E402

# each pass takes microseconds, so the watcher gives up after well under a
# second if it never sees the whole count
MAX_PASSES = 20000


# a hold of about 0.5 ms on the dispatch's stream, so that the watcher is
# already polling when the dispatch starts
HOLD_CYCLES = 1_200_000


def _watched_dispatch(st: Step, q: int, x: np.ndarray, idx: np.ndarray, messages):
    w = st.w
    n, k = idx.shape
    xd, idd = to_dev(x), to_dev(idx)
    report = torch.zeros(4, dtype=torch.int64, device=DEV)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)  # the sentinel fill and the cleans come first
    # The dispatch is enqueued before the watcher: should the two streams
    # share a hardware queue, the watcher then runs after it (and sees only
    # the final counts) instead of holding it back.
    torch.cuda._sleep(HOLD_CYCLES)
    ll.ll_moe_dispatch(st.lay, w.capacity, n, w.hidden, w.num_experts, k, w.dtype, q, xd, idd,
                       stream=main)
    ll.ll_moe_diag_watch(st.lay, w.capacity, n, w.hidden, w.num_experts, k, w.dtype, q, messages,
                         idd, MAX_PASSES, report, stream=side)
    oracle.dispatch(st.img, w.capacity, w.hidden, w.num_experts, w.dtype, q, x, idx)
    torch.cuda.synchronize()
    return [int(v) for v in report.cpu()]


@pytest.mark.parametrize("name,num_tokens", [("decode", 128), ("decode", 512),
                                             ("wide_zipf", 512), ("decode_fp8", 128),
                                             ("decode_fp8", 512)])
def test_counts_never_run_ahead_of_messages(name, num_tokens):
    w = W.WORKLOADS[name].with_(num_tokens=num_tokens)
    x, idx = W.tokens(w), W.routing(w)
    _, cnt = oracle.route(idx, w.num_experts, w.capacity)
    routed = int(cnt.sum())
    # the messages the rows must hold, from the oracle's encoder
    messages = to_dev(np.ascontiguousarray(oracle.encode_messages(x, w.dtype)))
    st = Step(w, full_image=False)
    partial = 0
    for rep in range(4):
        q = rep & 1
        say(f"[publish] {name} N={num_tokens} rep {rep} parity {q}")
        passes, part, violations, last = _watched_dispatch(st, q, x, idx, messages)
        say(f"[publish]   passes {passes}, partial views {part}, violations {violations}, "
            f"last total {last} of {routed}")
        assert violations == 0, "a count was visible before its messages"
        assert last == routed and passes < MAX_PASSES, "the watcher never saw every count"
        st.check_dispatch(q, idx)  # byte parity; puts the sentinel back
        partial += part
    # the watcher must really have overlapped the dispatch at least once,
    # or the check above says nothing about the order
    assert partial > 0, "the watcher never saw a partial total"
