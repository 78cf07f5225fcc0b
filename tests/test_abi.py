"""The C ABI without a GPU: the library loads, exports every declared entry
point, computes the layout the oracle computes, and rejects bad arguments
before it enqueues anything."""
import ctypes
import glob
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(ll_moe_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    import combine_ll_moe_amd as ll
    lib = ctypes.CDLL(ll.LIB_PATH)
    names = _declared_symbols()
    assert {"ll_moe_layout_bytes", "ll_moe_dispatch", "ll_moe_combine",
            "ll_moe_clean_signals"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


SHAPES = [(128, 1024, 8, 0), (128, 7168, 256, 0), (128, 7168, 256, 1), (512, 4096, 64, 0),
          (1024, 7168, 256, 0), (1, 8, 1, 0), (3, 128, 5, 1), (77, 7168, 256, 1),
          (33, 1000, 17, 0), (4096, 8192, 512, 1)]


@pytest.mark.parametrize("shape", SHAPES)
def test_layout_matches_oracle(shape):
    import combine_ll_moe_amd as ll
    n, h, e, dt = shape
    L = oracle.layout(n, h, e, dt)
    assert ll.ll_moe_layout_bytes(n, h, e, dt) == L["total"]
    md, _ = oracle.message_bytes(h, dt)
    for q in (0, 1):
        o = ll.ll_moe_layout_offsets(n, h, e, dt, q)
        assert (o["send"], o["recv"], o["sig"], o["msg_bytes"]) == \
            (L["send"][q], L["recv"][q], L["sig"][q], md)


def test_layout_rejections():
    import combine_ll_moe_amd as ll
    for args in [(0, 8, 1, 0), (1, 0, 1, 0), (1, 8, 0, 0), (1, 8, 1, 2), (4, 100, 8, 1),
                 (1, 1, 1, 0), (2**31 - 1, 2**30, 2**31 - 1, 0)]:
        with pytest.raises(ll.LLMoEError) as ei:
            ll.ll_moe_layout_bytes(*args)
        assert ei.value.status == ll.INVALID_ARGUMENT


FAKE = 0x10000  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("case", [
    dict(parity=2), dict(parity=-1), dict(num_tokens=129), dict(num_tokens=-1),
    dict(topk=0), dict(topk=9, num_experts=8), dict(topk=17, num_experts=64),
    dict(hidden=1020), dict(dtype=1, hidden=1000), dict(dtype=7), dict(layout=0),
    dict(layout=FAKE + 8), dict(x=0), dict(x=FAKE + 4), dict(idx=0), dict(idx=FAKE + 2),
    dict(max_tokens=0), dict(hidden=8 * 2816), dict(num_experts=(1 << 20) + 1),
])
def test_dispatch_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(layout=FAKE, max_tokens=128, num_tokens=128, hidden=1024, num_experts=8, topk=2,
             dtype=0, parity=0, x=FAKE, idx=FAKE)
    a.update(case)
    rc = ll.raw_status("ll_moe_dispatch", a["layout"], a["max_tokens"], a["num_tokens"],
                       a["hidden"], a["num_experts"], a["topk"], a["dtype"], a["parity"],
                       a["x"], a["idx"], None)
    assert rc == ll.INVALID_ARGUMENT


@pytest.mark.parametrize("case", [
    dict(parity=3), dict(num_tokens=200), dict(topk=0), dict(hidden=1020), dict(y=0),
    dict(w=0), dict(out=0), dict(out=FAKE + 4), dict(y=FAKE + 8), dict(w=FAKE + 1),
    dict(out=FAKE + 64),  # overlaps expert_out
])
def test_combine_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(layout=FAKE, max_tokens=128, num_tokens=128, hidden=1024, num_experts=8, topk=2,
             dtype=0, parity=0, y=FAKE, idx=FAKE, w=FAKE, out=FAKE * 1024)
    a.update(case)
    rc = ll.raw_status("ll_moe_combine", a["layout"], a["max_tokens"], a["num_tokens"],
                       a["hidden"], a["num_experts"], a["topk"], a["dtype"], a["parity"],
                       a["y"], a["idx"], a["w"], a["out"], None)
    assert rc == ll.INVALID_ARGUMENT


def test_clean_rejects_bad_arguments():
    import combine_ll_moe_amd as ll
    assert ll.raw_status("ll_moe_clean_signals", FAKE, 8, 64, 4, 0, 2, None) == ll.INVALID_ARGUMENT
    assert ll.raw_status("ll_moe_clean_signals", 0, 8, 64, 4, 0, 0, None) == ll.INVALID_ARGUMENT
    assert ll.raw_status("ll_moe_clean_signals", FAKE, 0, 64, 4, 0, 0, None) == ll.INVALID_ARGUMENT
    assert ll.raw_status("ll_moe_diag_e4m3", 0, FAKE, 4, None) == ll.INVALID_ARGUMENT


@pytest.mark.parametrize("case", [
    dict(parity=2), dict(num_tokens=129), dict(topk=0), dict(hidden=1020),
    dict(num_experts=2049, topk=2), dict(max_passes=0), dict(report=0), dict(report=FAKE + 4),
    dict(layout=0), dict(msgs=0), dict(msgs=FAKE + 2), dict(idx=FAKE + 1), dict(dtype=7),
    dict(dtype=1, hidden=1000), dict(max_tokens=4097, num_tokens=4097, topk=1),
])
def test_watch_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(layout=FAKE, max_tokens=128, num_tokens=128, hidden=1024, num_experts=8, topk=2,
             dtype=0, parity=0, msgs=FAKE, idx=FAKE, max_passes=10, report=FAKE)
    a.update(case)
    rc = ll.raw_status("ll_moe_diag_watch", a["layout"], a["max_tokens"], a["num_tokens"],
                       a["hidden"], a["num_experts"], a["topk"], a["dtype"], a["parity"],
                       a["msgs"], a["idx"], a["max_passes"], a["report"], None)
    assert rc == ll.INVALID_ARGUMENT


@pytest.mark.parametrize("case", [
    dict(rows=3), dict(rows=-1), dict(rows=2, row_bytes=2008), dict(row_bytes=2002),
    dict(per=0), dict(per=257), dict(policy=4), dict(base=0), dict(base=FAKE + 4),
    dict(offs=FAKE + 4),
])
def test_store_probe_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(base=FAKE, offs=FAKE, nrows=3, row_bytes=2004, per=1, line=0, rows=0, policy=0)
    a.update(case)
    rc = ll.raw_status("ll_moe_diag_store_rows", a["base"], a["offs"], a["nrows"], a["row_bytes"],
                       a["per"], a["line"], a["rows"], a["policy"], None)
    assert rc == ll.INVALID_ARGUMENT


@pytest.mark.parametrize("case", [
    dict(y_rows=0), dict(y_rows=-1), dict(n=-1), dict(hidden=0), dict(hidden=1020),
    dict(topk=0), dict(topk=17), dict(y=0), dict(y=FAKE + 8), dict(rows=0), dict(w=0),
    dict(out=0), dict(out=FAKE + 4),
])
def test_gather_probe_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(y=FAKE, y_rows=64, hidden=1024, rows=FAKE, w=FAKE, n=16, topk=8, out=FAKE)
    a.update(case)
    rc = ll.raw_status("ll_moe_diag_gather_rows", a["y"], a["y_rows"], a["hidden"], a["rows"],
                       a["w"], a["n"], a["topk"], a["out"], None)
    assert rc == ll.INVALID_ARGUMENT


@pytest.mark.parametrize("case", [
    dict(mode=4), dict(mode=-1), dict(nbytes=1000), dict(blocks=0), dict(dst=0),
    dict(dst=FAKE + 4), dict(src=0), dict(src=FAKE + 8), dict(mode=1, src=0),
    dict(mode=2, src=FAKE + 4),
])
def test_stream_probe_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(mode=3, nt=0, dst=FAKE, src=FAKE, nbytes=1024, blocks=4)
    a.update(case)
    rc = ll.raw_status("ll_moe_diag_stream", a["mode"], a["nt"], a["dst"], a["src"], a["nbytes"],
                       a["blocks"], None)
    assert rc == ll.INVALID_ARGUMENT


BIG = 1 << 36  # far above any FAKE layout: never overlaps it


@pytest.mark.parametrize("case", [
    dict(parity=2), dict(hidden=1020), dict(dtype=7), dict(dtype=1, hidden=1000),
    dict(layout=0), dict(layout=FAKE + 8), dict(y=0), dict(y=BIG + 8),
    dict(num_experts=4097), dict(max_tokens=0), dict(hidden=22528),
    dict(y=FAKE + 64),  # overlaps the layout
    dict(max_tokens=1 << 20, num_experts=4096),  # num_experts * max_tokens >= 2^31
])
def test_combine_send_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(layout=FAKE, max_tokens=128, hidden=1024, num_experts=8, dtype=0, parity=0, y=BIG)
    a.update(case)
    rc = ll.raw_status("ll_moe_combine_send", a["layout"], a["max_tokens"], a["hidden"],
                       a["num_experts"], a["dtype"], a["parity"], a["y"], None)
    assert rc == ll.INVALID_ARGUMENT


@pytest.mark.parametrize("case", [
    dict(parity=2), dict(num_tokens=129), dict(num_tokens=-1), dict(topk=0), dict(topk=9),
    dict(hidden=1020), dict(hidden=22528), dict(num_experts=4097, topk=2), dict(layout=0),
    dict(layout=FAKE + 4), dict(idx=0), dict(idx=BIG + 2), dict(w=0), dict(w=BIG + 1),
    dict(out=0), dict(out=2 * BIG + 4), dict(out=FAKE + 64), dict(max_spins=0),
    dict(max_spins=-5), dict(status=0), dict(status=3 * BIG + 2), dict(status=0, num_tokens=0),
])
def test_combine_recv_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(layout=FAKE, max_tokens=128, num_tokens=128, hidden=1024, num_experts=8, topk=2,
             dtype=0, parity=0, idx=BIG, w=BIG, out=2 * BIG, max_spins=100, status=3 * BIG)
    a.update(case)
    rc = ll.raw_status("ll_moe_combine_recv", a["layout"], a["max_tokens"], a["num_tokens"],
                       a["hidden"], a["num_experts"], a["topk"], a["dtype"], a["parity"],
                       a["idx"], a["w"], a["out"], a["max_spins"], a["status"], None)
    assert rc == ll.INVALID_ARGUMENT


@pytest.mark.parametrize("case", [
    dict(parity=2), dict(hidden=1020), dict(dtype=7), dict(dtype=1, hidden=1000),
    dict(layout=0), dict(layout=FAKE + 8), dict(payload=0), dict(payload=BIG + 4),
    dict(src=0), dict(src=2 * BIG + 2), dict(counts=0), dict(counts=3 * BIG + 1),
    dict(status=0), dict(status=4 * BIG + 2), dict(dtype=1, scales=0),
    dict(dtype=1, scales=5 * BIG + 2), dict(expected=-1), dict(expected=8 * 128 + 1),
    dict(max_spins=0), dict(num_experts=4097), dict(max_tokens=1 << 20, num_experts=4096),
    dict(payload=FAKE + 64), dict(src=FAKE + 4), dict(counts=FAKE + 4),
    dict(dtype=1, scales=FAKE + 4),
])
def test_dispatch_recv_rejects_bad_arguments(case):
    import combine_ll_moe_amd as ll
    a = dict(layout=FAKE, max_tokens=128, hidden=1024, num_experts=8, dtype=0, parity=0,
             expected=16, payload=BIG, scales=5 * BIG, src=2 * BIG, counts=3 * BIG,
             max_spins=10, status=4 * BIG)
    a.update(case)
    rc = ll.raw_status("ll_moe_dispatch_recv", a["layout"], a["max_tokens"], a["hidden"],
                       a["num_experts"], a["dtype"], a["parity"], a["expected"], a["payload"],
                       a["scales"], a["src"], a["counts"], a["max_spins"], a["status"], None)
    assert rc == ll.INVALID_ARGUMENT


def test_binding_routes_through_the_library_only():
    """The binding imports neither the oracle nor the workload generators."""
    src = open(os.path.join(ROOT, "combine_ll_moe_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no fallback", "")
    assert "import workloads" not in src
    for f in glob.glob(os.path.join(ROOT, "combine_ll_moe_amd", "csrc", "*")):
        text = open(f).read()
        assert "oracle" not in text and "ll_moe_oracle" not in text, f
