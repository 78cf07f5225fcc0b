"""Helpers of the GPU parity tests: run a step through the C ABI on the GPU
and compare it, region by region, with the oracle on the same seeded inputs.

Not collected by pytest (no test_ prefix). Imported only by GPU tests.
"""
import sys

import numpy as np
import torch

import combine_ll_moe_amd as ll
import oracle
import workloads as W

SENT = 0xA5
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8)


def filled_mask(w: W.Workload, idx: np.ndarray) -> np.ndarray:
    """Rows of the receive-slot order that some routed pick fills (oracle)."""
    _, cnt = oracle.route(idx, w.num_experts, w.capacity)
    m = np.zeros(w.num_experts * w.capacity, bool)
    for e in range(w.num_experts):
        m[e * w.capacity:e * w.capacity + int(cnt[e])] = True
    return m


class Step:
    """One layout on the GPU and its oracle image, kept in lockstep."""

    def __init__(self, w: W.Workload, full_image: bool, base_pad: int = 0):
        self.w = w
        self.L = oracle.layout(w.capacity, w.hidden, w.num_experts, w.dtype)
        self.md, self.mc = oracle.message_bytes(w.hidden, w.dtype)
        total = self.L["total"]
        assert ll.ll_moe_layout_bytes(w.capacity, w.hidden, w.num_experts, w.dtype) == total
        # base_pad shifts the layout inside its allocation (16-byte steps) so
        # that destination phases differ from the 256-byte-aligned case
        self.buf = torch.full((total + base_pad,), SENT, dtype=torch.uint8, device=DEV)
        self.lay = self.buf[base_pad:]
        self.full = full_image
        self.img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype,
                                    fill=SENT if full_image else None)
        for q in (0, 1):
            self.clean(q)

    # -- launches, mirrored on both sides ---------------------------------
    def clean(self, q):
        w = self.w
        ll.ll_moe_clean_signals(self.lay, w.capacity, w.hidden, w.num_experts, w.dtype, q)
        oracle.clean(self.img, w.capacity, w.hidden, w.num_experts, w.dtype, q)

    def dispatch(self, q, x: np.ndarray, idx: np.ndarray, x_dev=None, idx_dev=None):
        w = self.w
        n = idx.shape[0]
        xd = to_dev(x) if x_dev is None else x_dev
        idd = to_dev(idx) if idx_dev is None else idx_dev
        ll.ll_moe_dispatch(self.lay, w.capacity, n, w.hidden, w.num_experts, idx.shape[1],
                           w.dtype, q, xd, idd)
        oracle.dispatch(self.img, w.capacity, w.hidden, w.num_experts, w.dtype, q, x, idx)

    def combine(self, q, y: np.ndarray, idx: np.ndarray, wt: np.ndarray, y_dev=None,
                idx_dev=None):
        w = self.w
        n = idx.shape[0]
        yd = to_dev(y) if y_dev is None else y_dev
        idd = to_dev(idx) if idx_dev is None else idx_dev
        out = torch.full((n, w.hidden), float("nan"), dtype=torch.float32, device=DEV)
        ll.ll_moe_combine(self.lay, w.capacity, n, w.hidden, w.num_experts, idx.shape[1],
                          w.dtype, q, yd, idd, to_dev(wt), out)
        ref = oracle.combine(self.img, w.capacity, w.hidden, w.num_experts, w.dtype, q, y, idx, wt)
        torch.cuda.synchronize()
        return out.cpu().numpy(), ref

    def combine_send(self, q, y: np.ndarray, y_dev=None, stream=None):
        w = self.w
        yd = to_dev(y) if y_dev is None else y_dev
        ll.ll_moe_combine_send(self.lay, w.capacity, w.hidden, w.num_experts, w.dtype, q, yd,
                               stream=stream)
        oracle.combine_send(self.img, w.capacity, w.hidden, w.num_experts, w.dtype, q, y)

    def combine_recv(self, q, idx: np.ndarray, wt: np.ndarray, max_spins=1 << 22, stream=None,
                     with_oracle=True):
        """Token side on the GPU (and the oracle's, unless with_oracle is
        False); returns (out, status word, oracle out or None) once the GPU
        is done."""
        w = self.w
        n = idx.shape[0]
        out = torch.full((n, w.hidden), float("nan"), dtype=torch.float32, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        ll.ll_moe_combine_recv(self.lay, w.capacity, n, w.hidden, w.num_experts, idx.shape[1],
                               w.dtype, q, to_dev(idx), to_dev(wt), out, max_spins, status,
                               stream=stream)
        ref = None
        if with_oracle:
            ref = oracle.combine_recv(self.img, w.capacity, w.hidden, w.num_experts, w.dtype, q,
                                      idx, wt)
        torch.cuda.synchronize()
        return out.cpu().numpy(), int(status.item()), ref

    def check_staging(self, q, idx: np.ndarray):
        """Set q's staging rows of every routed (t, k) against the oracle,
        and the whole layout when the image is kept in full."""
        torch.cuda.synchronize()
        self.check_signals()
        w, mc = self.w, self.mc
        if self.full:
            gi = host_u8(self.lay)
            if not np.array_equal(gi, self.img):
                bad = np.nonzero(gi != self.img)[0]
                raise AssertionError(f"layout image differs at {bad.size} bytes, first {bad[0]}")
            return
        e = idx.astype(np.int64)
        t = np.broadcast_to(np.arange(idx.shape[0])[:, None], idx.shape)
        ok = (e >= 0) & (e < w.num_experts)
        rows = np.unique(e[ok] * w.capacity + t[ok])
        nrow = w.num_experts * w.capacity
        stage = self.L["send"][q]
        sv = self.lay[stage:stage + nrow * mc].view(nrow, mc)
        g = host_u8(sv.index_select(0, torch.from_numpy(rows).to(DEV)))
        r = self.img[stage:stage + nrow * mc].reshape(nrow, mc)[rows]
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"staging rows differ: {bad.shape[0]} bytes, first (row "
                                 f"{rows[bad[0][0]]}, col {bad[0][1]})")

    # -- comparisons ---------------------------------------------------------
    def signals(self, q):
        off = self.L["sig"][q]
        g = host_u8(self.lay[off:off + 8 * self.w.num_experts]).view(np.int64)
        r = self.img[off:off + 8 * self.w.num_experts].view(np.int64)
        return g, r

    def check_signals(self):
        for q in (0, 1):
            g, r = self.signals(q)
            assert np.array_equal(g, r), (q, np.nonzero(g != r)[0][:8], g[:8], r[:8])

    def check_dispatch(self, q, idx: np.ndarray, restore=True):
        """Compare set q's written regions with the oracle; then (restore)
        put the sentinel back over them on the GPU and require the whole
        layout except the signal words to be sentinel again."""
        torch.cuda.synchronize()
        self.check_signals()
        w, md, L = self.w, self.md, self.L
        n = idx.shape[0]
        send = L["send"][q]
        g = host_u8(self.lay[send:send + n * md])
        r = self.img[send:send + n * md]
        if not np.array_equal(g, r):
            bad = np.nonzero(g != r)[0]
            raise AssertionError(f"send rows differ at {bad.size} bytes, first byte {bad[0]} "
                                 f"(row {bad[0] // md}, col {bad[0] % md})")
        rows = np.nonzero(filled_mask(w, idx))[0]
        recv = L["recv"][q]
        nrow = w.num_experts * w.capacity
        rv = self.lay[recv:recv + nrow * md].view(nrow, md)
        rows_t = torch.from_numpy(rows).to(DEV)
        g = host_u8(rv.index_select(0, rows_t))
        r = self.img[recv:recv + nrow * md].reshape(nrow, md)[rows]
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"recv rows differ: {bad.shape[0]} bytes, first (row "
                                 f"{rows[bad[0][0]]}, col {bad[0][1]})")
        if self.full:
            gi = host_u8(self.lay)
            if not np.array_equal(gi, self.img):
                bad = np.nonzero(gi != self.img)[0]
                raise AssertionError(f"layout image differs at {bad.size} bytes, first {bad[0]}")
        if restore:
            self.lay[send:send + n * md] = SENT
            rv.index_fill_(0, rows_t, SENT)
            sig0 = L["sig"][0]
            saved = self.lay[sig0:sig0 + 16 * w.num_experts].clone()
            self.lay[sig0:sig0 + 16 * w.num_experts] = SENT
            stray = count_not(self.lay, SENT)
            self.lay[sig0:sig0 + 16 * w.num_experts] = saved
            assert stray == 0, f"{stray} bytes written outside the expected regions"
            if self.full:
                self.img[send:send + n * md] = SENT
                self.img[recv:recv + nrow * md].reshape(nrow, md)[rows] = SENT


def count_not(t: torch.Tensor, value: int, chunk: int = 1 << 30) -> int:
    n = 0
    for i in range(0, t.numel(), chunk):
        n += int((t[i:i + chunk] != value).sum().item())
    return n


def check_combine(out: np.ndarray, ref: np.ndarray, rel: float = 1e-6):
    """The bar: max relative error <= rel where the oracle is nonzero, exact
    where it is zero; reported alongside the count of differing bits."""
    assert out.shape == ref.shape
    nz = ref != 0
    assert np.array_equal(out[~nz], ref[~nz]), "nonzero where the oracle is zero"
    if nz.any():
        err = np.abs(out[nz].astype(np.float64) - ref[nz]) / np.abs(ref[nz].astype(np.float64))
        assert np.isfinite(out).all()
        assert err.max() <= rel, f"max rel err {err.max()}"
    return int((out.view(np.uint32) != ref.view(np.uint32)).sum())


def random_case(rng):
    """A seeded random shape and routing: any dtype, hidden, expert count,
    top-k, batch and capacity the ABI accepts (layouts up to ~256 MiB), with
    repeated experts, masked entries and capacity overflow."""
    while True:
        dt = W.FP8_E4M3 if rng.random() < 0.4 else W.BF16
        kind = rng.random()
        if kind < 0.2:    # long batches: tiles of two tokens
            n = int(rng.integers(1025, 2100))
            h = 128 * int(rng.integers(1, 4))
            e = int(rng.integers(1, 65))
        else:
            n = int(rng.integers(0, 700))
            h = 128 * int(rng.integers(1, 80)) if dt == W.FP8_E4M3 else 8 * int(rng.integers(1, 1600))
            # few experts in some cases: picks repeat and overflow the capacity
            e = int(rng.integers(1, 5)) if kind < 0.35 else int(rng.integers(1, 300))
        k = int(rng.integers(1, min(e, ll.MAX_TOPK) + 1))
        cap = max(1, n + (0 if kind < 0.35 else int(rng.integers(0, 40))))
        md, mc = oracle.message_bytes(h, dt)
        if n <= cap and md <= ll.MAX_MESSAGE_BYTES and e * cap * max(md, mc) <= 1 << 26:
            break
    idx = rng.integers(0, e, (n, k)).astype(np.int32)  # repeats allowed
    mask = rng.random((n, k)) < 0.03
    idx[mask] = np.where(rng.random(int(mask.sum())) < 0.5, -1, e + 3).astype(np.int32)
    return W.Workload("random", n, h, e, k, dt, "uniform", max_tokens=cap,
                      seed=int(rng.integers(1 << 30))), idx
