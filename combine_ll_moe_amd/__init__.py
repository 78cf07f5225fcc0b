"""Python binding of libllmoe.so, the MI355X low-latency MoE dispatch + combine.

Argument marshalling only: every function forwards to the C entry point of
the same name (include/ll_moe.h) and raises LLMoEError on a non-zero status.
Device buffers may be passed as torch tensors (their data_ptr is used) or as
raw integer addresses; `stream` defaults to torch's current stream.
There is no fallback: without the built library this package does not
import.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libllmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python combine_ll_moe_amd/build.py` "
        "(hipcc, gfx950) before importing combine_ll_moe_amd")

_lib = ctypes.CDLL(LIB_PATH)

BF16 = 0
FP8_E4M3 = 1
MAX_TOPK = 16
MAX_MESSAGE_BYTES = 45056
MAX_EXPERTS = 1 << 20
SEND_MAX_EXPERTS = 4096
REFUSAL_FLAG_WAIT = 1
REFUSAL_COUNT_WAIT = 2
RECV_READY = 0x100
RECV_WAITED = 0x200

SUCCESS = 0
HIP_ERROR = 1
INTERNAL_ERROR = 3
INVALID_ARGUMENT = 4
INVALID_USAGE = 5

PROBE_WRITE = 0
PROBE_READ = 1
PROBE_COPY = 2
PROBE_FOLD4 = 3
PROBE_ROWS_GROUP = 0
PROBE_ROWS_WAVE = 1
PROBE_ROWS_DIRECT = 2
PROBE_SC1 = 0
PROBE_WRITE_BACK = 1
PROBE_NT = 2
PROBE_SC1_NT = 3

_i = ctypes.c_int
_vp = ctypes.c_void_p
_szp = ctypes.POINTER(ctypes.c_size_t)

_lib.ll_moe_layout_bytes.argtypes = [_i, _i, _i, _i, _szp]
_lib.ll_moe_layout_offsets.argtypes = [_i, _i, _i, _i, _i, _szp, _szp, _szp, _szp]
_lib.ll_moe_dispatch.argtypes = [_vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]
_lib.ll_moe_combine.argtypes = [_vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]
_lib.ll_moe_combine_send.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp]
_lib.ll_moe_combine_recv.argtypes = [_vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _vp,
                                     _vp]
_lib.ll_moe_dispatch_recv.argtypes = [_vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp,
                                      _vp]
_lib.ll_moe_clean_signals.argtypes = [_vp, _i, _i, _i, _i, _i, _vp]
_lib.ll_moe_diag_e4m3.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
_lib.ll_moe_diag_e4m3_in_range.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
_lib.ll_moe_diag_watch.argtypes = [_vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp]
_lib.ll_moe_diag_stream.argtypes = [_i, _i, _vp, _vp, ctypes.c_size_t, _i, _vp]
_lib.ll_moe_diag_store_rows.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
_lib.ll_moe_diag_gather_rows.argtypes = [_vp, ctypes.c_longlong, _i, _vp, _vp, _i, _i, _vp, _vp]
_lib.ll_moe_status_string.argtypes = [_i]
_lib.ll_moe_status_string.restype = ctypes.c_char_p
for _f in ("ll_moe_layout_bytes", "ll_moe_layout_offsets", "ll_moe_dispatch",
           "ll_moe_combine", "ll_moe_combine_send", "ll_moe_combine_recv", "ll_moe_dispatch_recv",
           "ll_moe_clean_signals", "ll_moe_diag_e4m3", "ll_moe_diag_e4m3_in_range",
           "ll_moe_diag_watch", "ll_moe_diag_stream",
           "ll_moe_diag_store_rows", "ll_moe_diag_gather_rows"):
    getattr(_lib, _f).restype = _i


class LLMoEError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        name = _lib.ll_moe_status_string(status).decode()
        super().__init__(f"{call} returned {name} ({status})")


def _check(status: int, call: str) -> None:
    if status != SUCCESS:
        raise LLMoEError(status, call)


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def ll_moe_layout_bytes(max_tokens: int, hidden: int, num_experts: int, dtype: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.ll_moe_layout_bytes(max_tokens, hidden, num_experts, dtype, ctypes.byref(out)),
           "ll_moe_layout_bytes")
    return out.value


def ll_moe_layout_offsets(max_tokens: int, hidden: int, num_experts: int, dtype: int,
                          parity: int) -> dict:
    s, r, g, m = (ctypes.c_size_t() for _ in range(4))
    _check(_lib.ll_moe_layout_offsets(max_tokens, hidden, num_experts, dtype, parity,
                                      ctypes.byref(s), ctypes.byref(r), ctypes.byref(g),
                                      ctypes.byref(m)), "ll_moe_layout_offsets")
    return {"send": s.value, "recv": r.value, "sig": g.value, "msg_bytes": m.value}


def ll_moe_dispatch(layout, max_tokens: int, num_tokens: int, hidden: int, num_experts: int,
                    topk: int, dtype: int, parity: int, x, topk_idx, stream=None) -> None:
    _check(_lib.ll_moe_dispatch(_ptr(layout), max_tokens, num_tokens, hidden, num_experts, topk,
                                dtype, parity, _ptr(x), _ptr(topk_idx), _stream(stream)),
           "ll_moe_dispatch")


def ll_moe_combine(layout, max_tokens: int, num_tokens: int, hidden: int, num_experts: int,
                   topk: int, dtype: int, parity: int, expert_out, topk_idx, topk_weights, out,
                   stream=None) -> None:
    _check(_lib.ll_moe_combine(_ptr(layout), max_tokens, num_tokens, hidden, num_experts, topk,
                               dtype, parity, _ptr(expert_out), _ptr(topk_idx),
                               _ptr(topk_weights), _ptr(out), _stream(stream)),
           "ll_moe_combine")


def ll_moe_combine_send(layout, max_tokens: int, hidden: int, num_experts: int, dtype: int,
                        parity: int, expert_out, stream=None) -> None:
    _check(_lib.ll_moe_combine_send(_ptr(layout), max_tokens, hidden, num_experts, dtype, parity,
                                    _ptr(expert_out), _stream(stream)), "ll_moe_combine_send")


def ll_moe_combine_recv(layout, max_tokens: int, num_tokens: int, hidden: int, num_experts: int,
                        topk: int, dtype: int, parity: int, topk_idx, topk_weights, out,
                        max_spins: int, status, stream=None) -> None:
    _check(_lib.ll_moe_combine_recv(_ptr(layout), max_tokens, num_tokens, hidden, num_experts,
                                    topk, dtype, parity, _ptr(topk_idx), _ptr(topk_weights),
                                    _ptr(out), max_spins, _ptr(status), _stream(stream)),
           "ll_moe_combine_recv")


def ll_moe_dispatch_recv(layout, max_tokens: int, hidden: int, num_experts: int, dtype: int,
                         parity: int, expected: int, payload, scales, src_tokens, counts,
                         max_spins: int, status, stream=None) -> None:
    _check(_lib.ll_moe_dispatch_recv(_ptr(layout), max_tokens, hidden, num_experts, dtype, parity,
                                     expected, _ptr(payload), _ptr(scales), _ptr(src_tokens),
                                     _ptr(counts), max_spins, _ptr(status), _stream(stream)),
           "ll_moe_dispatch_recv")


def ll_moe_clean_signals(layout, max_tokens: int, hidden: int, num_experts: int, dtype: int,
                         parity: int, stream=None) -> None:
    _check(_lib.ll_moe_clean_signals(_ptr(layout), max_tokens, hidden, num_experts, dtype, parity,
                                     _stream(stream)), "ll_moe_clean_signals")


def ll_moe_diag_e4m3(inp, out, n: int, stream=None) -> None:
    """Diagnostic: the fp8 dispatch's e4m3 encoder applied to n fp32 values."""
    _check(_lib.ll_moe_diag_e4m3(_ptr(inp), _ptr(out), n, _stream(stream)), "ll_moe_diag_e4m3")


def ll_moe_diag_e4m3_in_range(inp, out, n: int, stream=None) -> None:
    """Diagnostic: the fp8 dispatch's fast e4m3 encoder (no clamp, no NaN
    patch), defined for |x| <= 448 * (1 + 2^-23)."""
    _check(_lib.ll_moe_diag_e4m3_in_range(_ptr(inp), _ptr(out), n, _stream(stream)),
           "ll_moe_diag_e4m3_in_range")


def ll_moe_diag_watch(layout, max_tokens: int, num_tokens: int, hidden: int, num_experts: int,
                      topk: int, dtype: int, parity: int, messages, topk_idx, max_passes: int,
                      report, stream=None) -> None:
    """Diagnostic: a concurrent consumer of a dispatch's counts that compares
    whole receive rows with the expected messages; report is a zeroed
    int64[4] (most passes of a workgroup, passes that saw a partial total,
    violations, last total acquired)."""
    _check(_lib.ll_moe_diag_watch(_ptr(layout), max_tokens, num_tokens, hidden, num_experts, topk,
                                  dtype, parity, _ptr(messages), _ptr(topk_idx), max_passes,
                                  _ptr(report), _stream(stream)), "ll_moe_diag_watch")


def ll_moe_diag_stream(mode: int, non_temporal: bool, dst, src, nbytes: int, blocks: int,
                       stream=None) -> None:
    """Measurement probe: a contiguous write / read / copy of nbytes, or a
    fold of 4 * nbytes read into nbytes written."""
    _check(_lib.ll_moe_diag_stream(mode, int(bool(non_temporal)), _ptr(dst), _ptr(src), nbytes,
                                   blocks, _stream(stream)), "ll_moe_diag_stream")


def ll_moe_diag_store_rows(base, row_offsets, nrows: int, row_bytes: int, rows_per_block: int,
                           line: bool, rows: int, policy: int, stream=None) -> None:
    """Measurement probe: the dispatch's message stores alone, to listed rows
    (rows: PROBE_ROWS_GROUP, PROBE_ROWS_WAVE or PROBE_ROWS_DIRECT)."""
    _check(_lib.ll_moe_diag_store_rows(_ptr(base), _ptr(row_offsets), nrows, row_bytes,
                                       rows_per_block, int(bool(line)), int(rows),
                                       policy, _stream(stream)), "ll_moe_diag_store_rows")


def ll_moe_diag_gather_rows(y, y_rows: int, hidden: int, rows, weights, num_tokens: int,
                            topk: int, out, stream=None) -> None:
    """Measurement probe: the combine's gather alone, rows handed in."""
    _check(_lib.ll_moe_diag_gather_rows(_ptr(y), y_rows, hidden, _ptr(rows), _ptr(weights),
                                        num_tokens, topk, _ptr(out), _stream(stream)),
           "ll_moe_diag_gather_rows")


def raw_status(name: str, *args) -> int:
    """Call a C entry point with raw ctypes-compatible arguments and return
    its status without raising (for argument-checking tests)."""
    return getattr(_lib, name)(*args)
