"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs. Dispatch buffers and signal words must match byte for
byte, with no byte written outside them; combine outputs must be within
1e-6 relative error of the oracle (and are expected to be bit-identical)."""
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


def _inputs(w: W.Workload, dense_y=False):
    x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
    y = W.expert_outputs(w, None if dense_y else filled_mask(w, idx))
    return x, idx, wt, y


def _run_step(st: Step, q, x, idx, wt, y, y_dev=None):
    st.dispatch(q, x, idx)
    st.check_dispatch(q, idx)
    out, ref = st.combine(q, y, idx, wt, y_dev=y_dev)
    st.check_signals()
    diff = check_combine(out, ref)
    assert diff == 0, f"{diff} combine outputs differ in bits"
    return out


@pytest.mark.parametrize("name", ["tiny", "decode", "decode_fp8", "wide_zipf", "worst_fill"])
def test_workload_both_parities(name):
    w = W.WORKLOADS[name]
    say(f"[parity] {name}: N={w.num_tokens} h={w.hidden} E={w.num_experts} K={w.topk} "
        f"dtype={w.dtype}")
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=(name == "tiny"))
    y_dev = to_dev(y)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y, y_dev)
        say(f"[parity] {name} parity {q} ok")


def test_hundred_steps_tiny_every_byte():
    base = W.WORKLOADS["tiny"]
    st = Step(base, full_image=True)
    for s in range(100):
        w = base.with_(seed=1000 + s)
        x, idx, wt, y = _inputs(w)
        _run_step(st, s & 1, x, idx, wt, y)
    say("[seq] tiny 100 steps ok")


def test_hundred_steps_decode():
    base = W.WORKLOADS["decode"]
    st = Step(base, full_image=False)
    y = W.expert_outputs(base)          # every row filled: one upload for all steps
    y_dev = to_dev(y)
    for s in range(100):
        w = base.with_(seed=2000 + s)
        x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
        q = s & 1
        st.dispatch(q, x, idx)
        st.check_dispatch(q, idx)
        out, ref = st.combine(q, y, idx, wt, y_dev=y_dev)
        assert check_combine(out, ref) == 0
    say("[seq] decode 100 steps ok")


@pytest.mark.parametrize("n", [0, 1, 77, 127])
@pytest.mark.parametrize("dtype", [W.BF16, W.FP8_E4M3])
def test_ragged_batches(n, dtype):
    w = W.Workload("ragged", n, 7168, 256, 8, dtype, "uniform", max_tokens=128, seed=n)
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    for q in (1, 0):
        _run_step(st, q, x, idx, wt, y)


@pytest.mark.parametrize("shape", [
    # (N, Nmax, h, E, K, dtype)
    (5, 8, 8, 1, 1, W.BF16),        # smallest message: 20 bytes
    (9, 9, 24, 3, 2, W.BF16),       # odd capacity, short rows
    (33, 40, 1032, 17, 5, W.BF16),  # ragged chunk counts
    (16, 16, 512, 64, 16, W.BF16),  # the 16-pick path
    (16, 16, 512, 64, 9, W.BF16),   # 16-pick path with 9 picks
    (3, 3, 128, 5, 4, W.FP8_E4M3),  # one fp8 block
    (64, 64, 384, 32, 3, W.FP8_E4M3),
    (300, 300, 2048, 128, 8, W.BF16),
    (40, 40, 64, 4096, 4, W.BF16),   # largest expert count of the LDS histogram
    (40, 48, 64, 4097, 4, W.BF16),   # ballot path beyond it
    (24, 24, 256, 5000, 12, W.FP8_E4M3),
    (2048, 2048, 256, 64, 8, W.BF16),    # two-token tiles of rows from registers
    (2048, 2048, 128, 64, 4, W.FP8_E4M3),
])
@pytest.mark.parametrize("pad", [0, 16, 48])
def test_shapes_and_base_phases(shape, pad):
    n, cap, h, e, k, dt = shape
    w = W.Workload("shape", n, h, e, k, dt, "uniform", max_tokens=cap, seed=h + k)
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=True, base_pad=pad)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y)


@pytest.mark.parametrize("shape", [
    (1024, 1024, 4104, 64, 8, W.BF16, "uniform"),
    (1000, 1024, 4104, 64, 8, W.BF16, "hotset"),
    (2048, 2048, 7168, 32, 8, W.FP8_E4M3, "uniform"),
])
def test_large_dispatch_whole_line_stores(shape):
    """Dispatches that write 64 MiB or more deal store chunks to lanes by
    whole 128-byte lines. Message lengths 8212 and 7396 (not multiples of
    128) start the rows at every 4-byte phase of a line."""
    n, cap, h, e, k, dt, routing = shape
    w = W.Workload("lines", n, h, e, k, dt, routing, max_tokens=cap, seed=n + h)
    md, _ = oracle.message_bytes(h, dt)
    assert n * (k + 1) * md >= 64 << 20
    say(f"[parity] whole-line stores: N={n} cap={cap} h={h} E={e} K={k} dtype={dt}")
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y)


@pytest.mark.parametrize("shape", [
    # (N, h, E, K, dtype, routing): the combine splits a row into equal runs
    # of columns, one 16-byte chunk per thread, blocks a multiple of 32
    (128, 1032, 16, 4, W.BF16, "uniform"),      # 129 chunks: one run of 160 threads
    (96, 7168, 32, 8, W.FP8_E4M3, "uniform"),   # four runs of 224 (a half wavefront each)
    (128, 2056, 16, 8, W.BF16, "uniform"),      # 257 chunks: two runs of 160, the last 97
    (1024, 4104, 64, 8, W.BF16, "hotset"),      # streamed rows: two runs of 288, the last 225
])
def test_combine_column_runs(shape):
    n, h, e, k, dt, routing = shape
    w = W.Workload("runs", n, h, e, k, dt, routing, seed=h + k)
    say(f"[parity] combine column runs: N={n} h={h} E={e} K={k} dtype={dt}")
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y)


@pytest.mark.parametrize("n", [64, 2048])
def test_fully_masked_tokens(n):
    """Tokens whose every pick is masked (out of range or -1) write +0.0f and
    load nothing that matters: alone, as the first or second token of a
    two-token tile (N=2048), and both tokens of a tile."""
    w = W.Workload("masked", n, 64, 8, 4, W.BF16, "uniform", seed=n)
    rng = np.random.default_rng(n)
    idx = np.stack([rng.permutation(8)[:4] for _ in range(n)]).astype(np.int32)
    for t in (0, 1, 5, 6, 7, n - 2, n - 1):  # tiles (0,1), (6,7), (n-2,n-1) whole; 5 alone
        idx[t] = -1
    idx[9] = [8, -1, 100, -5]
    x, wt = W.tokens(w), W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    say(f"[parity] fully masked tokens: N={n}")
    st = Step(w, full_image=True)
    for q in (0, 1):
        out = _run_step(st, q, x, idx, wt, y)
        for t in (0, 1, 5, 6, 7, 9, n - 2, n - 1):
            assert not out[t].view(np.uint32).any(), f"token {t} is not +0.0f"


def test_masked_repeated_and_overflowing_picks():
    w = W.Workload("mask", 6, 64, 4, 3, W.BF16, "uniform", max_tokens=6, seed=9)
    x = W.tokens(w)
    idx = np.array([[0, -1, 2], [2, 2, 7], [0, 0, 0], [1, 3, 0], [0, 0, 2**31 - 1],
                    [-2**31, 0, 0]], np.int32)
    wt = W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    st = Step(w, full_image=True)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y)
    _, cnt = oracle.route(idx, 4, 6)
    assert cnt[0] == 6  # capacity reached: later picks of expert 0 dropped


@pytest.mark.parametrize("shape", [
    # (N, Nmax, h, E, K, dtype): messages near the 45056-byte limit leave LDS
    # room for one message buffer; the N=1024 cases take one-token tiles and
    # whole-line stores, the N=2048 cases two-token tiles (the dispatch grows
    # tiles past 1024 workgroups; the single buffer is reused with a
    # barrier); fp8 at h=43648 quantizes in six batches of four rounds
    (64, 64, 22520, 16, 4, W.BF16),
    (1024, 1024, 22520, 16, 2, W.BF16),
    (2048, 2048, 22520, 16, 2, W.BF16),
    (32, 32, 43648, 8, 2, W.FP8_E4M3),
    (1024, 1024, 43648, 8, 2, W.FP8_E4M3),
    (2048, 2048, 43648, 8, 2, W.FP8_E4M3),
    # whole-line stores with a token's rows shared by two workgroups: bf16
    # rows by workgroup, fp8 rows by wavefront
    (200, 200, 22520, 64, 8, W.BF16),
    (200, 200, 43648, 64, 8, W.FP8_E4M3),
])
def test_largest_messages(shape):
    n, cap, h, e, k, dt = shape
    md, _ = oracle.message_bytes(h, dt)
    # LDS of a dispatch workgroup: 64 KiB less the tile entries (512 B) and
    # the histogram (4 bytes per expert): no room for a second buffer
    assert 2 * (((12 + md) + 15) // 16 * 16) > 65536 - 512 - 4 * e and md <= ll.MAX_MESSAGE_BYTES
    say(f"[parity] largest messages: N={n} h={h} E={e} K={k} dtype={dt} md={md}")
    w = W.Workload("big", n, h, e, k, dt, "uniform", max_tokens=cap, seed=h + n)
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y)


@pytest.mark.parametrize("n,k,e,shift", [
    (1024, 8, 64, 0),    # 8192 entries, 16-byte aligned: four entries per load
    (1024, 8, 64, 1),    # the same table 4 bytes off 16-byte alignment: one per load
    (1025, 5, 64, 0),    # 5125 entries, not a whole number of 4-entry loads
    (3000, 4, 64, 0),    # 12000 entries: two rounds of four-entry loads
    (1024, 8, 5000, 0),  # four-entry loads in both histogram passes (5000 experts)
    (128, 8, 256, 0),    # 1024 entries, aligned: four per load on the register path
    (128, 8, 256, 1),    # the same, misaligned: one per load
])
def test_routing_table_load_widths(n, k, e, shift):
    """The dispatch and the combine read the routing table four entries per
    load only when it is 16-byte aligned and a multiple of 4 entries long
    (the dispatch of 64 MiB or more only when it is also longer than 4096
    entries); every case must route exactly as the oracle does, through
    both kernels, with the table at the same (mis)aligned address."""
    w = W.Workload("tab", n, 64, e, k, W.BF16, "hotset", seed=n + k + shift)
    x, idx, wt, y = _inputs(w)
    buf = torch.zeros(idx.size + 4, dtype=torch.int32, device=DEV)
    idx_dev = buf[shift:shift + idx.size].view(n, k)
    idx_dev.copy_(torch.from_numpy(idx))
    assert (idx_dev.data_ptr() % 16 == 0) == (shift == 0)
    say(f"[parity] routing table widths: N={n} K={k} E={e} shift={4 * shift} bytes")
    st = Step(w, full_image=e <= 64)
    for q in (0, 1):
        st.dispatch(q, x, idx, idx_dev=idx_dev)
        st.check_dispatch(q, idx)
        out, ref = st.combine(q, y, idx, wt, idx_dev=idx_dev)
        assert check_combine(out, ref) == 0, "combine outputs differ in bits"


@pytest.mark.parametrize("shape", [
    # (N, E, K): one-token tiles of 8 and 16 entries (DPP-row ranks), and
    # two-token tiles of 32 entries (the register walk: the combine's at
    # N=1024, the dispatch's at N=2048); experts drawn with replacement, so
    # tokens repeat experts, plus masked entries and experts that overflow
    # their capacity
    (64, 8, 8),
    (1024, 32, 16),
    (2048, 32, 16),
])
def test_repeated_picks_in_every_rank_path(shape):
    n, e, k = shape
    w = W.Workload("rep", n, 64, e, k, W.BF16, "uniform", seed=n + k)
    rng = np.random.default_rng(n * 31 + k)
    idx = rng.integers(-1, e + 1, size=(n, k)).astype(np.int32)  # -1 and e are masked
    x = W.tokens(w)
    wt = W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    _, cnt = oracle.route(idx, e, n)
    say(f"[parity] repeated picks: N={n} E={e} K={k}, max count {int(cnt.max())} of {n}")
    st = Step(w, full_image=True)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y)


def test_fp8_special_blocks():
    w = W.Workload("fp8s", 8, 1024, 8, 2, W.FP8_E4M3, "uniform", seed=4)
    x = W.tokens(w)
    x[0, :128] = 0                                                   # amax 0
    x[0, 128:256] = 0x8000                                           # all -0
    x[1, :128] = W.f32_to_bf16_bits(np.full(128, 3e-38, np.float32))  # tiny normal
    x[1, 128:256] = np.arange(128, dtype=np.uint16)                  # subnormals, amax 2^-126 * ...
    x[2, :128] = 0x0001                                              # smallest subnormal: inv overflows
    x[2, 1] = 0
    x[3, 5] = 0x7F80                                                 # +inf in a block
    x[3, 200] = 0xFF80                                               # -inf
    x[4, 7] = 0x7FC0                                                 # quiet NaN
    x[4, 300] = 0x7F81                                               # signalling NaN pattern
    x[5, :128] = W.f32_to_bf16_bits(np.linspace(-448, 448, 128).astype(np.float32))
    x[6, 256:384] = W.f32_to_bf16_bits(np.full(128, 65504.0, np.float32))
    idx = W.routing(w)
    wt = W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    st = Step(w, full_image=True)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y)


def test_fp8_special_blocks_in_every_round():
    """hidden = 9216: 1152 eight-element units, so a 256-thread workgroup
    quantizes four rounds (blocks 0-15, 16-31, 32-47, 48-63) and then a
    second batch (blocks 64-71). Special blocks sit in each of them."""
    w = W.Workload("fp8r", 16, 9216, 16, 4, W.FP8_E4M3, "uniform", seed=5)
    x = W.tokens(w)

    def blk(t, b):
        return x[t, 128 * b:128 * (b + 1)]

    blk(0, 20)[:] = 0                                   # round 1: amax 0
    blk(0, 40)[17] = 0x7FC0                             # round 2: a NaN
    blk(0, 50)[3] = 0x7F80                              # round 3: +inf
    blk(0, 66)[100] = 0xFFC1                            # second batch: negative NaN
    blk(1, 33)[:] = np.arange(1, 129, dtype=np.uint16)  # round 2: subnormals
    blk(1, 49)[:] = 0x0001                              # round 3: inv overflows
    blk(1, 49)[5] = 0                                   #   with a zero: 0 * inf
    blk(1, 70)[:] = 0x8000                              # second batch: all -0
    for b in range(72):                                 # every block holds a NaN
        blk(2, b)[(7 * b) % 128] = 0x7FC0
    blk(3, 17)[:] = 0x7FC0                              # round 1: all NaN
    blk(3, 63)[:] = 0xFF80                              # round 3: all -inf
    for k, b in enumerate([0, 16, 32, 48, 64]):         # amax 448 * 2^k in each round
        v = np.linspace(-1.0, 1.0, 128).astype(np.float32) * np.float32(448.0 * 2.0 ** (k - 2))
        blk(4, b)[:] = W.f32_to_bf16_bits(v)
    idx = W.routing(w)
    wt = W.weights(w)
    y = W.expert_outputs(w, filled_mask(w, idx))
    st = Step(w, full_image=True)
    for q in (0, 1):
        _run_step(st, q, x, idx, wt, y)


def test_dispatch_accumulates_when_set_not_cleaned():
    """dispatch(q) adds to set q's words; without a launch of the other
    parity in between they are not cleaned, on both sides alike."""
    w = W.WORKLOADS["tiny"]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    st.dispatch(0, x, idx)
    st.dispatch(0, x, idx)
    torch.cuda.synchronize()
    st.check_signals()
    g, _ = st.signals(0)
    assert g.sum() == 2 * idx.size


def test_clean_only_touches_its_set():
    w = W.WORKLOADS["tiny"]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=True)
    st.dispatch(1, x, idx)
    st.clean(0)
    st.clean(1)
    st.check_dispatch(1, idx)


def test_identity_round_trip_exact():
    """Experts that return their input and weights 1/8: every partial sum
    is exact, so combine(dispatch(x)) returns f32(x) exactly (a -0 input
    returns +0, the chain's starting value)."""
    w = W.WORKLOADS["decode"]
    x, idx = W.tokens(w), W.routing(w)
    st = Step(w, full_image=False)
    st.dispatch(0, x, idx)
    st.check_dispatch(0, idx, restore=False)
    md = st.md
    r0 = st.L["recv"][0]
    nrow = w.num_experts * w.capacity
    recv = st.img[r0:r0 + nrow * md].reshape(nrow, md)
    y = np.zeros((nrow, w.hidden), np.uint16)
    mask = filled_mask(w, idx)
    y[mask] = np.ascontiguousarray(recv[mask][:, 4:]).view(np.uint16)
    wt = np.full(idx.shape, 1.0 / 8, np.float32)
    out, ref = st.combine(0, y, idx, wt)
    xf = W.bf16_bits_to_f32(x)
    # the chain starts from +0.0f, so an input -0 comes back as +0
    nz = xf != 0
    for o in (ref, out):
        assert np.array_equal(o, xf)
        assert np.array_equal(o[nz].view(np.uint32), xf[nz].view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "decode_fp8"])
def test_graph_capture_replays(name):
    """Two steps (parity 0, then 1) captured into a HIP graph and replayed
    three times, with eager kernels and synchronizations between replays:
    every replay writes the same bytes and bits as the eager steps. The
    two-step sequence is idempotent under the parity schedule (each
    parity's launches zero the other set's words before it is reused)."""
    w = W.WORKLOADS[name]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    xd, idd, wtd, yd = to_dev(x), to_dev(idx), to_dev(wt), to_dev(y)
    refs = []
    for q in (0, 1):  # eager, checked against the oracle
        st.dispatch(q, x, idx, x_dev=xd, idx_dev=idd)
        st.check_dispatch(q, idx, restore=False)
        out, ref = st.combine(q, y, idx, wt, y_dev=yd)
        assert check_combine(out, ref) == 0
        refs.append(out)
    n, k = idx.shape
    outs = [torch.empty((n, w.hidden), dtype=torch.float32, device=DEV) for _ in range(2)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            gs = torch.cuda.current_stream().cuda_stream
            for q in (0, 1):
                ll.ll_moe_dispatch(st.lay, w.capacity, n, w.hidden, w.num_experts, k, w.dtype, q,
                                   xd, idd, gs)
                ll.ll_moe_combine(st.lay, w.capacity, n, w.hidden, w.num_experts, k, w.dtype, q,
                                  yd, idd, wtd, outs[q], gs)
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:  # eager work between replays
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for q in (0, 1):
            got = outs[q].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), refs[q].view(np.uint32)), (r, q)
            st.check_dispatch(q, idx, restore=False)
        say(f"[graph] {name} replay {r} ok")


def _all_rounding_inputs():
    top = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = [0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xFEDC]
    return np.concatenate([top | np.uint32(lo) for lo in lows]).view(np.float32)


def test_e4m3_encoder_against_oracle():
    rng = np.random.default_rng(3)
    rnd = rng.integers(0, 1 << 32, 1 << 24, dtype=np.uint64).astype(np.uint32).view(np.float32)
    for v in (_all_rounding_inputs(), rnd):
        d_in = torch.from_numpy(v.copy()).to(DEV)
        d_out = torch.empty(v.size, dtype=torch.uint8, device=DEV)
        ll.ll_moe_diag_e4m3(d_in, d_out, v.size)
        got = d_out.cpu().numpy()
        want = oracle.e4m3(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(hex(v.view(np.uint32)[i]), got[i], want[i]) for i in bad[:8]]


# largest fp32 magnitude the fast encoder sees: 448 * (1 + 2^-23) rounded
# down to a float is 448 + 2^-15, the bit pattern 0x43E00001
FAST_DOMAIN_BITS = 0x43E00001


def test_e4m3_fast_path_against_oracle_on_its_domain():
    """The encoder ordinary fp8 waves run (no clamp, no NaN patch) on every
    input of the rounding cover inside its domain, the domain's edges, and
    16M random inputs inside it."""
    rng = np.random.default_rng(4)
    cover = _all_rounding_inputs()
    mag = cover.view(np.uint32) & np.uint32(0x7FFFFFFF)
    cover = cover[mag <= FAST_DOMAIN_BITS]
    edges = np.array([0x43E00001, 0x43E00000, 0x43DFFFFF, 0x43D00000, 0x43C00000, 0x43B00000,
                      0x3B000000, 0x3A800000, 0x3A800001, 1, 0], np.uint32)
    edges = np.concatenate([edges, edges | np.uint32(0x80000000)]).view(np.float32)
    rnd = rng.integers(0, FAST_DOMAIN_BITS + 1, 1 << 24, dtype=np.uint64).astype(np.uint32)
    rnd |= rng.integers(0, 2, rnd.size, dtype=np.uint32) << np.uint32(31)
    for v in (cover, edges, rnd.view(np.float32)):
        assert np.isfinite(v).all() and (np.abs(v) <= np.float32(448 + 2.0 ** -15)).all()
        d_in = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
        d_out = torch.empty(v.size, dtype=torch.uint8, device=DEV)
        ll.ll_moe_diag_e4m3_in_range(d_in, d_out, v.size)
        got = d_out.cpu().numpy()
        want = oracle.e4m3(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(hex(v.view(np.uint32)[i]), got[i], want[i]) for i in bad[:8]]
    say(f"[e4m3] fast path: {cover.size} cover inputs, {edges.size} edges, {rnd.size} random")


def test_repeated_calls_same_bits():
    """Fixed operand order: the same inputs give the same bits every call."""
    w = W.WORKLOADS["wide_zipf"]
    x, idx, wt, y = _inputs(w)
    st = Step(w, full_image=False)
    y_dev = to_dev(y)
    outs = []
    for s in range(4):
        st.dispatch(s & 1, x, idx)
        o, ref = st.combine(s & 1, y, idx, wt, y_dev=y_dev)
        outs.append(o)
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("block", range(4))
def test_random_shapes(block):
    """40 seeded random cases (10 per block) through dispatch and combine,
    both parities, each against the oracle; every layout starts at a random
    16-byte phase of its allocation."""
    for case in range(10):
        rng = np.random.default_rng(1000 + 10 * block + case)
        w, idx = random_case(rng)
        pad = int(rng.choice([0, 16, 32, 48]))
        say(f"[parity] random case {10 * block + case}: N={w.num_tokens} cap={w.capacity} "
            f"h={w.hidden} E={w.num_experts} K={w.topk} dtype={w.dtype} pad={pad}")
        x, wt = W.tokens(w), W.weights(w)
        y = W.expert_outputs(w, filled_mask(w, idx))
        st = Step(w, full_image=False, base_pad=pad)
        y_dev = to_dev(y)
        for q in (0, 1):
            _run_step(st, q, x, idx, wt, y, y_dev)
        del st, y_dev
        torch.cuda.empty_cache()
