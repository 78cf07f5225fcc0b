"""The measurement probes do what their floors claim.

gather_rows runs the combine's own gather over rows handed in, so over the
oracle's rows its output must be the oracle's combine, bit for bit.
store_rows writes its pattern to the listed rows and nowhere else.
The contiguous stream copy reproduces its source.
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
from _gpu import DEV, filled_mask, say, to_dev  # noqa: E402


@pytest.mark.parametrize("name", ["tiny", "decode", "wide_zipf"])
def test_gather_probe_is_the_combine(name):
    w = W.WORKLOADS[name]
    idx, wt = W.routing(w), W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    slot, _ = oracle.route(idx, w.num_experts, w.capacity)
    rows = (idx.astype(np.int64) * w.capacity + slot).astype(np.int32)
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype)
    ref = oracle.combine(img, w.capacity, w.hidden, w.num_experts, w.dtype, 0, y, idx, wt)
    out = torch.full((w.num_tokens, w.hidden), float("nan"), dtype=torch.float32, device=DEV)
    say(f"[probe] gather_rows {name}")
    ll.ll_moe_diag_gather_rows(to_dev(y), w.num_experts * w.capacity, w.hidden, to_dev(rows),
                               to_dev(wt), w.num_tokens, w.topk, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_gather_probe_skips_rows_out_of_range():
    w = W.WORKLOADS["tiny"]
    idx, wt = W.routing(w), W.weights(w)
    y = W.expert_outputs(w)
    slot, _ = oracle.route(idx, w.num_experts, w.capacity)
    rows = (idx.astype(np.int64) * w.capacity + slot).astype(np.int32)
    rows[::3, 0] = -1
    rows[1::5, 1] = w.num_experts * w.capacity  # one past the end
    keep = (rows >= 0) & (rows < w.num_experts * w.capacity)
    yf = W.bf16_bits_to_f32(y).astype(np.float64)
    ref = np.zeros((w.num_tokens, w.hidden), np.float32)
    for t in range(w.num_tokens):
        acc = np.zeros(w.hidden, np.float32)
        for k in range(w.topk):
            if keep[t, k]:
                # fmaf: the product of an fp32 and a bf16 is exact in fp64; the
                # sum with the fp32 accumulator is checked exact in fp64
                # (two-sum error 0), so rounding it to fp32 is the fma's one
                # rounding
                p = np.float64(wt[t, k]) * yf[rows[t, k]]
                a = acc.astype(np.float64)
                s = p + a
                bp = s - a
                assert np.all((p - bp) + (a - (s - bp)) == 0)
                acc = s.astype(np.float32)
        ref[t] = acc
    out = torch.full((w.num_tokens, w.hidden), float("nan"), dtype=torch.float32, device=DEV)
    ll.ll_moe_diag_gather_rows(to_dev(y), w.num_experts * w.capacity, w.hidden, to_dev(rows),
                               to_dev(wt), w.num_tokens, w.topk, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


G_, W_, D_ = ll.PROBE_ROWS_GROUP, ll.PROBE_ROWS_WAVE, ll.PROBE_ROWS_DIRECT


@pytest.mark.parametrize("line,rows_mode,policy,row_bytes", [
    (False, G_, 0, 2004), (True, G_, 0, 2004), (False, W_, 0, 2004), (True, W_, 0, 2004),
    (False, G_, 1, 2004), (False, W_, 2, 2004), (True, G_, 3, 2004),
    (False, D_, 0, 2004), (False, D_, 1, 2004), (True, D_, 3, 2004),
    (False, D_, 0, 4 + 16 * 1500),  # two rounds of register chunks
])
def test_store_probe_writes_only_its_rows(line, rows_mode, policy, row_bytes):
    # rows of a 4-byte header and whole 16-byte chunks: 4-byte phases, as
    # message rows
    nrows, space = 37, 64
    rng = np.random.default_rng(1)
    slots = np.sort(rng.choice(space, nrows, replace=False))
    offs = (slots * row_bytes).astype(np.int64)
    buf = torch.full((space * row_bytes + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    base = buf[16:]
    say(f"[probe] store_rows line={line} rows={rows_mode} policy={policy} row_bytes={row_bytes}")
    ll.ll_moe_diag_store_rows(base, to_dev(offs), nrows, row_bytes, 6, line, rows_mode, policy)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    want = np.full_like(got, 0xA5)
    pattern = (0xC3C30000 ^ np.arange(0, row_bytes, 4, dtype=np.uint32)).view(np.uint8)
    for o in offs:
        want[16 + o:16 + o + row_bytes] = pattern
    assert np.array_equal(got, want)


@pytest.mark.parametrize("nt", [False, True])
def test_stream_copy_reproduces_its_source(nt):
    n = (3 << 20) + 48
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ll.ll_moe_diag_stream(ll.PROBE_COPY, nt, dst, src, n, 37)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    sink = torch.zeros(16, dtype=torch.uint8, device=DEV)
    ll.ll_moe_diag_stream(ll.PROBE_READ, nt, sink, src, n, 37)
    ll.ll_moe_diag_stream(ll.PROBE_WRITE, nt, dst, None, n, 5)
    torch.cuda.synchronize()
    words = dst.cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert (words[:, 0] == 0x5A5A5A5A).all() and (words[:, 1] == 0x5A5A5A5B).all()


@pytest.mark.parametrize("nt", [False, True])
def test_stream_fold_sums_its_four_regions(nt):
    n = (1 << 20) + 48  # bytes written: several tiles and a ragged tail
    src = torch.randint(0, 256, (4 * n,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros(n + 16, dtype=torch.uint8, device=DEV)
    say(f"[probe] stream fold4 nt={nt} bytes={n}")
    ll.ll_moe_diag_stream(ll.PROBE_FOLD4, nt, dst, src, n, 37)
    torch.cuda.synchronize()
    words = src.cpu().numpy().view(np.uint32).reshape(4, -1).astype(np.uint64)
    want = (words.sum(axis=0) & 0xFFFFFFFF).astype(np.uint32)
    got = dst.cpu().numpy()
    assert np.array_equal(got[:n].view(np.uint32), want)
    assert not got[n:].any()  # nothing past the bytes asked for
