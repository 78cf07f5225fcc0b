"""CPU oracle for the low-latency MoE dispatch + combine step (numpy front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its binding) never imports it, and it imports nothing of the product.

The arithmetic lives in ll_moe_oracle.c (plain C, compiled with gcc); this
module only marshals numpy arrays into it. Each C function cites the passage
of the pages it follows.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16 = 0
FP8_E4M3 = 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        vp = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_message_bytes.argtypes = [i, i, u64p, u64p]
        L.oracle_layout.argtypes = [i, i, i, i, u64p]
        L.oracle_e4m3.argtypes = [ctypes.c_float]
        L.oracle_e4m3.restype = ctypes.c_uint8
        L.oracle_e4m3_many.argtypes = [vp, vp, ctypes.c_uint64]
        L.oracle_e4m3_many.restype = None
        L.oracle_encode_messages.argtypes = [i, i, i, vp, vp]
        L.oracle_route.argtypes = [i, i, i, i, vp, vp, vp]
        L.oracle_dispatch.argtypes = [vp, i, i, i, i, i, i, i, vp, vp]
        L.oracle_combine.argtypes = [vp, i, i, i, i, i, i, i, vp, vp, vp, vp]
        L.oracle_clean.argtypes = [vp, i, i, i, i, i]
        L.oracle_combine_send.argtypes = [vp, i, i, i, i, i, vp]
        L.oracle_combine_recv.argtypes = [vp, i, i, i, i, i, i, i, vp, vp, vp]
        L.oracle_dispatch_recv.argtypes = [vp, i, i, i, i, i, i, vp, vp, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def message_bytes(hidden: int, dtype: int):
    """(dispatch message bytes, combine message bytes)."""
    md, mc = ctypes.c_uint64(), ctypes.c_uint64()
    rc = lib().oracle_message_bytes(hidden, dtype, ctypes.byref(md), ctypes.byref(mc))
    if rc != 0:
        raise ValueError("invalid hidden/dtype")
    return md.value, mc.value


def layout(max_tokens: int, hidden: int, num_experts: int, dtype: int) -> dict:
    out = (ctypes.c_uint64 * 7)()
    rc = lib().oracle_layout(max_tokens, hidden, num_experts, dtype, out)
    if rc != 0:
        raise ValueError("invalid layout arguments")
    return {
        "total": out[0],
        "send": (out[1], out[2]),
        "recv": (out[3], out[4]),
        "sig": (out[5], out[6]),
    }


def e4m3(values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_many(_ptr(v), _ptr(out), v.size)
    return out


def encode_messages(x: np.ndarray, dtype: int) -> np.ndarray:
    """x: uint16 bf16 bits [N, h] -> uint8 [N, md] messages."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n, h = x.shape
    md, _ = message_bytes(h, dtype)
    out = np.empty((n, md), dtype=np.uint8)
    if lib().oracle_encode_messages(n, h, dtype, _ptr(x), _ptr(out)) != 0:
        raise ValueError("encode failed")
    return out


def route(idx: np.ndarray, num_experts: int, max_tokens: int):
    """idx int32 [N, K] -> (slot int32 [N, K] with -1 for masked, cnt int64 [E])."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n, k = idx.shape
    slot = np.empty((n, k), dtype=np.int32)
    cnt = np.empty(num_experts, dtype=np.int64)
    if lib().oracle_route(n, k, num_experts, max_tokens, _ptr(idx), _ptr(slot), _ptr(cnt)) != 0:
        raise ValueError("route failed")
    return slot, cnt


def new_image(max_tokens, hidden, num_experts, dtype, fill=None) -> np.ndarray:
    """Host image of a whole layout. Without `fill` the pages stay untouched
    (and uncommitted) until the oracle writes them."""
    total = layout(max_tokens, hidden, num_experts, dtype)["total"]
    img = np.empty(total, dtype=np.uint8)
    if fill is not None:
        img.fill(fill)
    return img


def dispatch(image, max_tokens, hidden, num_experts, dtype, parity, x, idx):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n, k = idx.shape
    assert x.shape == (n, hidden)
    rc = lib().oracle_dispatch(_ptr(image), max_tokens, n, hidden, num_experts, k,
                               dtype, parity, _ptr(x), _ptr(idx))
    if rc != 0:
        raise ValueError("oracle dispatch rejected its arguments")


def combine(image, max_tokens, hidden, num_experts, dtype, parity, expert_out, idx, weights):
    y = np.ascontiguousarray(expert_out, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    n, k = idx.shape
    assert y.shape == (num_experts * max_tokens, hidden)
    assert w.shape == (n, k)
    out = np.empty((n, hidden), dtype=np.float32)
    rc = lib().oracle_combine(_ptr(image), max_tokens, n, hidden, num_experts, k, dtype,
                              parity, _ptr(y), _ptr(idx), _ptr(w), _ptr(out))
    if rc != 0:
        raise ValueError("oracle combine rejected its arguments")
    return out


class FlagNotRaised(RuntimeError):
    """The two-phase combine's receiver needs a flag the expert side has not
    raised (the GPU reports this in its refusal word)."""


def combine_send(image, max_tokens, hidden, num_experts, dtype, parity, expert_out):
    """Two-phase combine, expert side: stage the outputs per (expert, token)
    and raise the flags (high halves of set `parity`'s signal words)."""
    y = np.ascontiguousarray(expert_out, dtype=np.uint16)
    assert y.shape == (num_experts * max_tokens, hidden)
    rc = lib().oracle_combine_send(_ptr(image), max_tokens, hidden, num_experts, dtype, parity,
                                   _ptr(y))
    if rc != 0:
        raise ValueError("oracle combine_send rejected its arguments or the image")


def combine_recv(image, max_tokens, hidden, num_experts, dtype, parity, idx, weights):
    """Two-phase combine, token side: the fma chain over the staged rows."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    n, k = idx.shape
    assert w.shape == (n, k)
    out = np.empty((n, hidden), dtype=np.float32)
    rc = lib().oracle_combine_recv(_ptr(image), max_tokens, n, hidden, num_experts, k, dtype,
                                   parity, _ptr(idx), _ptr(w), _ptr(out))
    if rc == -2:
        raise FlagNotRaised("a routed expert's flag is not raised")
    if rc != 0:
        raise ValueError("oracle combine_recv rejected its arguments")
    return out


class CountsIncomplete(RuntimeError):
    """The dispatch's expert side needs counts that add up to the expected
    number of messages (the GPU reports this in its refusal word)."""


def dispatch_recv(image, max_tokens, hidden, num_experts, dtype, parity, expected, out=None):
    """Expert side of the dispatch: unpack set `parity`'s received messages.
    Returns (payload u8 [E*Nmax, row bytes], scales f32 [E*Nmax, h/128] or
    None, src int32 [E*Nmax], counts int32 [E]); `out` may hold those four
    arrays pre-filled (rows the step does not write keep their contents)."""
    rows = num_experts * max_tokens
    pb = 2 * hidden if dtype == 0 else hidden
    if out is None:
        out = (np.zeros((rows, pb), np.uint8),
               np.zeros((rows, hidden // 128), np.float32) if dtype == 1 else None,
               np.zeros(rows, np.int32), np.zeros(num_experts, np.int32))
    payload, scales, src, counts = out
    assert payload.shape == (rows, pb) and payload.dtype == np.uint8
    assert src.shape == (rows,) and counts.shape == (num_experts,)
    if dtype == 1:
        assert scales.shape == (rows, hidden // 128) and scales.dtype == np.float32
    rc = lib().oracle_dispatch_recv(_ptr(image), max_tokens, hidden, num_experts, dtype, parity,
                                    expected, _ptr(payload),
                                    _ptr(scales) if scales is not None else None, _ptr(src),
                                    _ptr(counts))
    if rc == -2:
        raise CountsIncomplete("the counts do not add up to the expected messages")
    if rc != 0:
        raise ValueError("oracle dispatch_recv rejected its arguments")
    return payload, scales, src, counts


def clean(image, max_tokens, hidden, num_experts, dtype, parity):
    rc = lib().oracle_clean(_ptr(image), max_tokens, hidden, num_experts, dtype, parity)
    if rc != 0:
        raise ValueError("oracle clean rejected its arguments")


def signals(image, max_tokens, hidden, num_experts, dtype, parity) -> np.ndarray:
    off = layout(max_tokens, hidden, num_experts, dtype)["sig"][parity]
    return image[off:off + 8 * num_experts].view(np.int64).copy()
