"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Each test checks the oracle against something the pages or mathematics fix:
hand-evaluated layout sizes, invariants of the layout and of dispatch, an
independent sort-based slot assignment on every tiny routing, an encoder built
from the e4m3 code table, torch's own e4m3 cast, an exact-sum error bound for
the combine, and exact identity round trips.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_bytes.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            p = line.split()
            rows.append((p[0], *map(int, p[1:])))
    return rows


# --------------------------------------------------------------------------
# Layout (LL_MoE_Buffers.hpp, LLMoEBufferLayout constructor)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_layout_matches_hand_values(row):
    name, n, h, e, dt, md, mc, send, recv, sig, total = row
    assert oracle.message_bytes(h, dt) == (md, mc)
    L = oracle.layout(n, h, e, dt)
    assert L["total"] == total
    assert L["send"] == (0, send)
    assert L["recv"] == (2 * send, 2 * send + recv)
    assert L["sig"] == (2 * send + 2 * recv, 2 * send + 2 * recv + sig)


@pytest.mark.parametrize("n,h,e,dt", [(1, 8, 1, 0), (5, 24, 3, 0), (7, 256, 9, 1),
                                      (128, 7168, 256, 1), (33, 1000, 17, 0)])
def test_layout_regions_tile_the_buffer(n, h, e, dt):
    """Six regions, two sets, disjoint, in order, covering [0, total) exactly;
    each send region can hold N dispatch messages and E*N combine messages,
    each recv region E*N of either; signals are E int64 words, 8-aligned."""
    L = oracle.layout(n, h, e, dt)
    md, mc = oracle.message_bytes(h, dt)
    s0, s1 = L["send"]
    r0, r1 = L["recv"]
    g0, g1 = L["sig"]
    send, recv = s1 - s0, r1 - r0
    assert s0 == 0 and r0 == s1 + send and g0 == r1 + recv
    assert g1 - g0 == 8 * e and L["total"] == g1 + 8 * e
    assert send >= n * md and send >= e * n * mc
    assert recv >= e * n * md and recv >= e * n * mc
    assert send in (n * md, e * n * mc) and recv in (e * n * md, e * n * mc)
    assert send % 4 == 0 and recv % 4 == 0 and g0 % 8 == 0


def test_layout_rejects_what_the_constructor_asserts():
    # h odd, E*N odd: the send size is not a multiple of sizeof(int)
    with pytest.raises(ValueError):
        oracle.layout(1, 1, 1, 0)
    with pytest.raises(ValueError):
        oracle.layout(4, 100, 8, 1)   # fp8 needs whole 128-element blocks
    # the fp8 reading leaves the layout equal to the bf16 one
    assert oracle.layout(128, 7168, 256, 1) == oracle.layout(128, 7168, 256, 0)


# --------------------------------------------------------------------------
# Slot assignment: brute force over every tiny routing, against a
# sort-based formulation written independently of the oracle's counters.
# --------------------------------------------------------------------------
def _slots_by_sort(idx, E, Nmax):
    N, K = idx.shape
    triples = [(int(idx[t, k]), t, k) for t in range(N) for k in range(K)
               if 0 <= idx[t, k] < E]
    triples.sort()  # by expert, then token, then k
    slot = -np.ones((N, K), np.int32)
    cnt = np.zeros(E, np.int64)
    prev, rank = None, 0
    for e, t, k in triples:
        rank = rank + 1 if e == prev else 0
        prev = e
        if rank < Nmax:
            slot[t, k] = rank
            cnt[e] += 1
    return slot, cnt


@pytest.mark.parametrize("N,K,E", [(1, 1, 1), (2, 2, 2), (3, 2, 3), (4, 1, 3), (2, 3, 3)])
def test_route_every_tiny_routing(N, K, E):
    values = list(range(-1, E + 1))  # includes both out-of-range kinds
    for combo in itertools.product(values, repeat=N * K):
        idx = np.array(combo, np.int32).reshape(N, K)
        for Nmax in sorted({N, max(1, N - 1)}):
            slot, cnt = oracle.route(idx, E, Nmax)
            s2, c2 = _slots_by_sort(idx, E, Nmax)
            assert np.array_equal(slot, s2), (idx, Nmax)
            assert np.array_equal(cnt, c2), (idx, Nmax)


# --------------------------------------------------------------------------
# Dispatch invariants on a full host image filled with a sentinel.
# --------------------------------------------------------------------------
SENT = 0xA5


def _check_dispatch_image(img, w, x, idx, parity, sig_before):
    N, K = idx.shape
    Nmax, h, E, dt = w.capacity, w.hidden, w.num_experts, w.dtype
    md, _ = oracle.message_bytes(h, dt)
    L = oracle.layout(Nmax, h, E, dt)
    touched = np.zeros(img.size, bool)

    # counts: equal to a plain histogram of the valid entries
    valid = (idx >= 0) & (idx < E)
    hist = np.bincount(idx[valid].ravel(), minlength=E).astype(np.int64)
    sig = img[L["sig"][parity]:L["sig"][parity] + 8 * E].view(np.int64)
    assert np.array_equal(sig, sig_before + hist)
    if (idx < E).all() and (idx >= 0).all():
        assert hist.sum() == N * K
    other = img[L["sig"][parity ^ 1]:L["sig"][parity ^ 1] + 8 * E].view(np.int64)
    assert (other == 0).all()
    touched[L["sig"][0]:L["sig"][1] + 8 * E] = True

    # send rows: header t, then the payload
    send = L["send"][parity]
    rows = img[send:send + N * md].reshape(N, md)
    assert np.array_equal(rows[:, :4].copy().view(np.int32).ravel(), np.arange(N))
    if dt == W.BF16:
        assert np.array_equal(rows[:, 4:].copy().view(np.uint16), x)
    touched[send:send + N * md] = True

    # every routed (t, k) exactly once in expert e's rows, headers strictly
    # increasing within an expert, payload equal to the send row of its header
    recv = L["recv"][parity]
    seen = []
    for e in range(E):
        for j in range(int(hist[e])):
            off = recv + (e * Nmax + j) * md
            m = img[off:off + md]
            t = int(m[:4].view(np.int32)[0])
            assert 0 <= t < N
            assert np.array_equal(m, rows[t])
            seen.append((e, t))
            touched[off:off + md] = True
        ts = [t for (ee, t) in seen if ee == e]
        assert ts == sorted(ts)
    want = sorted((int(idx[t, k]), t) for t in range(N) for k in range(K) if valid[t, k])
    assert sorted(seen) == want

    # nothing else changed
    assert (img[~touched] == SENT).all()


@pytest.mark.parametrize("dtype", [W.BF16, W.FP8_E4M3])
@pytest.mark.parametrize("parity", [0, 1])
def test_dispatch_invariants_small(dtype, parity):
    w = W.Workload("t", 24, 256, 6, 3, dtype, "uniform", max_tokens=32, seed=3)
    x, idx = W.tokens(w), W.routing(w)
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, dtype, fill=SENT)
    oracle.clean(img, w.capacity, w.hidden, w.num_experts, dtype, parity)
    sig_before = np.zeros(w.num_experts, np.int64)
    oracle.dispatch(img, w.capacity, w.hidden, w.num_experts, dtype, parity, x, idx)
    _check_dispatch_image(img, w, x, idx, parity, sig_before)


def test_dispatch_invariants_tiny_workload():
    w = W.WORKLOADS["tiny"]
    x, idx = W.tokens(w), W.routing(w)
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype, fill=SENT)
    oracle.clean(img, w.capacity, w.hidden, w.num_experts, w.dtype, 0)
    oracle.dispatch(img, w.capacity, w.hidden, w.num_experts, w.dtype, 0, x, idx)
    _check_dispatch_image(img, w, x, idx, 0, np.zeros(w.num_experts, np.int64))


def test_dispatch_masked_and_repeated_entries():
    w = W.Workload("t", 4, 16, 3, 3, W.BF16, "uniform", max_tokens=4, seed=5)
    x = W.tokens(w)
    idx = np.array([[0, -1, 2], [2, 2, 7], [0, 0, 0], [1, 3, 0]], np.int32)
    img = oracle.new_image(4, 16, 3, W.BF16, fill=SENT)
    oracle.clean(img, 4, 16, 3, W.BF16, 1)
    oracle.dispatch(img, 4, 16, 3, W.BF16, 1, x, idx)
    # expert 0 gets (0,0), (2,0), (2,1), (2,2) -> four rows; (3,2) would be
    # a fifth and is dropped (capacity 4)
    sig = oracle.signals(img, 4, 16, 3, W.BF16, 1)
    assert list(sig) == [4, 1, 3]
    slot, cnt = oracle.route(idx, 3, 4)
    assert slot[3, 2] == -1 and slot[0, 1] == -1 and slot[1, 2] == -1
    assert list(slot[2]) == [1, 2, 3] and list(slot[1][:2]) == [1, 2]


def test_dispatch_empty_batch():
    img = oracle.new_image(8, 64, 4, W.BF16, fill=SENT)
    oracle.dispatch(img, 8, 64, 4, W.BF16, 0, np.zeros((0, 64), np.uint16),
                    np.zeros((0, 2), np.int32))
    L = oracle.layout(8, 64, 4, W.BF16)
    assert (img[:L["sig"][0]] == SENT).all()
    # sig_0 was sentinel and got +0 for every expert; sig_1 was cleaned
    assert (img[L["sig"][0]:L["sig"][1]] == SENT).all()
    assert (oracle.signals(img, 8, 64, 4, W.BF16, 1) == 0).all()


# --------------------------------------------------------------------------
# e4m3 encoder against a table-driven nearest-value search
# --------------------------------------------------------------------------
def _e4m3_table():
    """Exact value of every finite e4m3fn code (S.EEEE.MMM, bias 7)."""
    vals = {}
    for code in range(256):
        s, ex, m = code >> 7, (code >> 3) & 15, code & 7
        if ex == 15 and m == 7:
            continue  # NaN
        if ex == 0:
            v = Fraction(m, 8) * Fraction(1, 64)
        else:
            v = (1 + Fraction(m, 8)) * Fraction(2) ** (ex - 7)
        vals[code] = -v if s else v
    return vals


def _table_encode(values: np.ndarray) -> np.ndarray:
    table = _e4m3_table()
    pos = sorted((v, c) for c, v in table.items() if v >= 0 and c < 128)
    pv = np.array([float(v) for v, _ in pos])      # exact in fp64
    pc = np.array([c for _, c in pos], np.uint8)
    with np.errstate(invalid="ignore"):
        a = values.astype(np.float64)
    out = np.empty(a.shape, np.uint8)
    nan = np.isnan(a)
    mag = np.abs(np.where(nan, 0.0, a))
    mag = np.minimum(mag, 448.0)  # saturate (also the infinities)
    hi = np.clip(np.searchsorted(pv, mag, side="left"), 0, len(pv) - 1)
    lo = np.clip(hi - 1, 0, len(pv) - 1)
    dlo, dhi = mag - pv[lo], pv[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((pc[hi] & 1) == 0))
    code = np.where(pick_hi, pc[hi], pc[lo])
    code = np.where(mag == pv[hi], pc[hi], code)
    sign = np.signbit(a) & ~nan
    out[:] = code | (sign.astype(np.uint8) << 7)
    out[nan] = 0x7F
    return out


def _cover_all_roundings():
    """Every top-16-bit fp32 pattern with low halves {0, 1, 0x7fff, 0x8000,
    0x8001, 0xffff, two random}. e4m3 rounding looks at bits >= 16 and at
    whether anything below is nonzero, so this set meets every case."""
    top = np.arange(1 << 16, dtype=np.uint32) << 16
    rng = np.random.default_rng(1)
    lows = [0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF] + list(rng.integers(1, 1 << 16, 2))
    bits = np.concatenate([top | np.uint32(lo) for lo in lows])
    return bits.view(np.float32)


def test_e4m3_against_code_table():
    v = _cover_all_roundings()
    got = oracle.e4m3(v)
    want = _table_encode(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), got[i], want[i]) for i in bad[:5]]


def test_e4m3_random_sample_against_code_table():
    rng = np.random.default_rng(7)
    v = rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    assert np.array_equal(oracle.e4m3(v), _table_encode(v))


def test_e4m3_special_points():
    pts = [(448.0, 0x7E), (464.0, 0x7E), (465.0, 0x7E), (1e30, 0x7E), (math.inf, 0x7E),
           (-math.inf, 0xFE), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (1.5 * 2 ** -10, 0x01),
           (2.0 ** -6, 0x08), (1.0, 0x38), (240.0, 0x77), (0.0, 0x00), (-0.0, 0x80),
           (1.0625, 0x38), (1.1875, 0x3A), (math.nan, 0x7F), (-math.nan, 0x7F)]
    for v, code in pts:
        assert oracle.e4m3(np.array([v], np.float32))[0] == code, v


def test_e4m3_matches_torch_cast_inside_range():
    torch = pytest.importorskip("torch")
    v = _cover_all_roundings()
    v = v[np.isfinite(v)]
    v = np.clip(v, -448.0, 448.0).astype(np.float32)
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3(v), t)


# --------------------------------------------------------------------------
# fp8 message: scales and codes against the dequantization error bound
# --------------------------------------------------------------------------
def _decode_e4m3(codes):
    table = _e4m3_table()
    lut = np.array([float(table.get(c, math.nan)) for c in range(256)])
    return lut[codes]


def test_fp8_message_dequantizes_within_e4m3_error():
    w = W.Workload("t", 16, 1024, 4, 2, W.FP8_E4M3, "uniform", seed=11)
    x = W.tokens(w)
    x[3, :128] = 0                     # an all-zero block
    x[4, 128:256] = W.f32_to_bf16_bits(np.full(128, 1e-3, np.float32))
    x[5, 256:384] = W.f32_to_bf16_bits(np.linspace(-8, 2, 128).astype(np.float32))
    msgs = oracle.encode_messages(x, W.FP8_E4M3)
    h = w.hidden
    assert msgs.shape[1] == 4 + h + 4 * (h // 128)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    for t in range(w.num_tokens):
        m = msgs[t]
        assert m[:4].view(np.int32)[0] == t
        q = _decode_e4m3(m[4:4 + h])
        sc = m[4 + h:].view(np.float32).astype(np.float64)
        for b in range(h // 128):
            xb = xf[t, 128 * b:128 * (b + 1)]
            amax = np.abs(xb).max()
            if amax == 0:
                assert sc[b] == 0 and (m[4 + 128 * b:4 + 128 * (b + 1)] == 0).all()
                continue
            # scale is amax/448 to fp32 rounding; the largest element maps to 448
            assert abs(sc[b] - amax / 448) <= 2 ** -23 * amax / 448
            assert np.abs(q[128 * b:128 * (b + 1)]).max() == 448.0
            deq = q[128 * b:128 * (b + 1)] * sc[b]
            # half an e4m3 spacing: 2^-4 relative on normals, 2^-10 * 448/amax
            # absolute in code units on subnormals, plus the fp32 roundings
            err = np.abs(deq - xb)
            bound = np.maximum(np.abs(xb) * 2 ** -4, 2 ** -10 * sc[b]) * (1 + 2 ** -20) \
                + np.abs(xb) * 2 ** -22
            assert (err <= bound).all(), (t, b, err.max())


def test_fp8_block_max_at_power_of_two_multiple_of_448():
    # amax = 448 * 2^-3 = 56: inv = 8 and scale = 1/8 are exact, so every
    # code is the e4m3 rounding of 8*x exactly, and the maximum is 0x7E
    x = np.zeros((1, 128), np.float32)
    x[0, :] = np.linspace(-56, 56, 128, dtype=np.float32)
    xb = W.f32_to_bf16_bits(x)
    m = oracle.encode_messages(xb, W.FP8_E4M3)[0]
    assert m[4 + 127] == 0x7E and m[4 + 0] == 0xFE
    assert m[4 + 128:].view(np.float32)[0] == np.float32(0.125)
    want = _table_encode((W.bf16_bits_to_f32(xb[0]) * 8).astype(np.float32))
    assert np.array_equal(m[4:4 + 128], want)


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------
def _round_f32(fr: Fraction) -> float:
    """Nearest fp32 to an exact rational, ties to even (no double rounding)."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # subnormal spacing floor
    ulp = Fraction(2) ** (e - 23)
    q = a / ulp
    m = q.numerator // q.denominator
    rem = q - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return sign * float(m * ulp)


def _fma32(a, b, c) -> float:
    return _round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def _small_combine_case(seed, N=40, h=64, E=5, K=3, Nmax=48):
    w = W.Workload("t", N, h, E, K, W.BF16, "uniform", max_tokens=Nmax, seed=seed)
    idx, wt = W.routing(w), W.weights(w)
    slot, cnt = oracle.route(idx, E, Nmax)
    filled = np.zeros(E * Nmax, bool)
    for e in range(E):
        filled[e * Nmax:e * Nmax + cnt[e]] = True
    y = W.expert_outputs(w, filled)
    img = oracle.new_image(Nmax, h, E, W.BF16)
    out = oracle.combine(img, Nmax, h, E, W.BF16, 0, y, idx, wt)
    return w, idx, wt, slot, y, out


def test_combine_within_fma_chain_bound_of_exact_sum():
    for seed in range(3):
        w, idx, wt, slot, y, out = _small_combine_case(seed)
        yf = W.bf16_bits_to_f32(y).astype(np.float64)
        N, K = idx.shape
        Nmax = w.capacity
        for t in range(N):
            for c in range(w.hidden):
                terms = [Fraction(float(wt[t, k])) * Fraction(float(yf[idx[t, k] * Nmax + slot[t, k], c]))
                         for k in range(K)]
                exact = sum(terms, Fraction(0))
                absum = sum(abs(x) for x in terms)
                err = abs(Fraction(float(out[t, c])) - exact)
                # K fused steps, one rounding each: |err| <= ((1+u)^K - 1) sum|w y|
                u = Fraction(1, 2 ** 24)
                assert err <= ((1 + u) ** K - 1) * absum, (t, c)


def test_combine_never_reads_unfilled_rows():
    # unfilled rows hold NaN; any stray read would leave a NaN in out
    for seed in range(3):
        *_, out = _small_combine_case(seed)
        assert np.isfinite(out).all()


@pytest.mark.parametrize("K", [2, 4, 8])
def test_identity_round_trip_is_exact(K):
    """Experts that return their input, weights 1/K (a power of two): every
    partial sum m*x/K is exact in fp32, so combine(dispatch(x)) == x (a -0
    input returns +0, the chain's starting value)."""
    E, N, h = 9, 30, 96
    w = W.Workload("t", N, h, E, K, W.BF16, "uniform", seed=K)
    x, idx = W.tokens(w), W.routing(w)
    x[0, :3] = [0x8000, 0x0000, 0x0001]  # -0, +0, the smallest subnormal
    img = oracle.new_image(N, h, E, W.BF16, fill=0)
    oracle.dispatch(img, N, h, E, W.BF16, 0, x, idx)
    md, _ = oracle.message_bytes(h, W.BF16)
    r0 = oracle.layout(N, h, E, W.BF16)["recv"][0]
    recv = img[r0:r0 + E * N * md].reshape(E * N, md)
    y = np.ascontiguousarray(recv[:, 4:]).view(np.uint16)   # expert = identity
    wt = np.full((N, K), 1.0 / K, np.float32)
    out = oracle.combine(img, N, h, E, W.BF16, 0, y, idx, wt)
    xf = W.bf16_bits_to_f32(x)
    # the chain starts from +0.0f: a -0 input returns +0; every other value
    # returns with its exact bits
    assert np.array_equal(out, xf)
    nz = xf != 0
    assert np.array_equal(out[nz].view(np.uint32), xf[nz].view(np.uint32))
    assert out[0, 0] == 0 and not np.signbit(out[0, 0])


def test_one_hot_weights_gather_exactly():
    w, idx, wt, slot, y, out = _small_combine_case(4)
    N, K = idx.shape
    pick = np.arange(N) % K
    oh = np.zeros_like(wt)
    oh[np.arange(N), pick] = 1.0
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, W.BF16)
    out = oracle.combine(img, w.capacity, w.hidden, w.num_experts, W.BF16, 0, y, idx, oh)
    rows = idx[np.arange(N), pick] * w.capacity + slot[np.arange(N), pick]
    assert np.array_equal(out, W.bf16_bits_to_f32(y[rows]))


def test_masked_entries_add_nothing():
    w, idx, wt, slot, y, out = _small_combine_case(5)
    idx2 = idx.copy()
    idx2[::3, 1] = -1
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, W.BF16)
    out2 = oracle.combine(img, w.capacity, w.hidden, w.num_experts, W.BF16, 0, y, idx2, wt)
    # masking shifts later slots of that expert; compare with the explicit
    # sum of the remaining terms, each against its own slot
    slot2, _ = oracle.route(idx2, w.num_experts, w.capacity)
    yf = W.bf16_bits_to_f32(y)
    for t in range(0, w.num_tokens, 3):
        acc = np.zeros(w.hidden, np.float32)
        for k in range(w.topk):
            if slot2[t, k] < 0:
                continue
            row = yf[idx2[t, k] * w.capacity + slot2[t, k]]
            acc = np.array([_fma32(wt[t, k], row[c], acc[c]) for c in range(w.hidden)],
                           np.float32)
        assert np.array_equal(out2[t], acc)


# --------------------------------------------------------------------------
# Parity sequences: signal words across 100 alternating steps
# --------------------------------------------------------------------------
def _sequence_violations(schedule, w, x, idx):
    """Replay `schedule` (list of (op, parity)) on the oracle and count the
    launches after which the signal words are not (histogram, 0) for the
    dispatched parity and its other set."""
    E = w.num_experts
    img = oracle.new_image(w.capacity, w.hidden, E, w.dtype, fill=0x5A)
    for q in (0, 1):
        oracle.clean(img, w.capacity, w.hidden, E, w.dtype, q)
    hist = np.bincount(idx.ravel(), minlength=E)
    wt = np.full(idx.shape, 0.5, np.float32)
    y = np.zeros((E * w.capacity, w.hidden), np.uint16)
    bad = 0
    for op, q in schedule:
        if op == "d":
            oracle.dispatch(img, w.capacity, w.hidden, E, w.dtype, q, x, idx)
            ok = (oracle.signals(img, w.capacity, w.hidden, E, w.dtype, q) == hist).all()
        else:
            oracle.combine(img, w.capacity, w.hidden, E, w.dtype, q, y, idx, wt)
            ok = (oracle.signals(img, w.capacity, w.hidden, E, w.dtype, q) == hist).all()
        ok = ok and (oracle.signals(img, w.capacity, w.hidden, E, w.dtype, q ^ 1) == 0).all()
        bad += int(not ok)
    return bad


def test_hundred_alternating_steps_keep_counts_exact():
    w = W.Workload("t", 16, 64, 8, 2, W.BF16, "uniform", seed=2)
    x, idx = W.tokens(w), W.routing(w)
    sched = [(op, s & 1) for s in range(100) for op in ("d", "c")]
    assert _sequence_violations(sched, w, x, idx) == 0


def test_sequence_check_catches_a_missing_clean():
    # the same parity twice in a row has no launch in between that cleans it:
    # the counts double, and the replay check must see that
    w = W.Workload("t", 16, 64, 8, 2, W.BF16, "uniform", seed=2)
    x, idx = W.tokens(w), W.routing(w)
    sched = [("d", 0), ("c", 0), ("d", 0), ("c", 0)]
    assert _sequence_violations(sched, w, x, idx) > 0


ALG_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "algorithmic_bytes.txt")


def _alg_rows():
    rows = []
    for line in open(ALG_GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, *nums = line.split()
            rows.append((name, *map(int, nums)))
    return rows


@pytest.mark.parametrize("row", _alg_rows(), ids=lambda r: r[0])
def test_algorithmic_bytes_match_hand_evaluation(row):
    """The roofline's byte accounting (bench.algorithmic_bytes) against the
    hand-evaluated table; every seeded workload routes all N*K picks."""
    import bench
    name, n, h, e, k, dt, md, routed, disp, comb = row
    w = W.WORKLOADS[name]
    assert (w.num_tokens, w.hidden, w.num_experts, w.topk, w.dtype) == (n, h, e, k, dt)
    assert oracle.message_bytes(h, dt)[0] == md
    _, cnt = oracle.route(W.routing(w), e, w.capacity)
    assert int(cnt.sum()) == routed == n * k
    ab = bench.algorithmic_bytes(w, md, routed)
    assert (ab["dispatch"], ab["combine"], ab["total"]) == (disp, comb, disp + comb)
