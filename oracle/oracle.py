"""ctypes front end of the plain-C oracle in ``hisparse_oracle.c``.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  Argument
marshalling only; every step of the computation is in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hisparse_oracle.c")
# HISPARSE_ORACLE_LIB names another build of the same source (the tests'
# sanitizer run loads an ASan/UBSan build this way).
_LIB = os.environ.get("HISPARSE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile the oracle with gcc (single-threaded, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load_oracle():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build_oracle(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_resolve.restype = ctypes.c_int
    lib.oracle_resolve.argtypes = [i32, i32, i32, i32, i32, i64, i64, i32, i32,
                                   P, P, P, P, P, P, P, P, P, P, P, P, P, i64,
                                   ctypes.c_int]
    lib.oracle_sparse_mla_decode.restype = ctypes.c_int
    lib.oracle_sparse_mla_decode.argtypes = [i32, i32, i32, P, P, P, i64, i32,
                                             ctypes.c_float, P]
    lib.oracle_mirror_rows.restype = ctypes.c_int
    lib.oracle_mirror_rows.argtypes = [i32, i32, P, P, P, i64, P, P, i32, i32, P, ctypes.c_int]
    lib.oracle_invalidate_tokens.restype = ctypes.c_int
    lib.oracle_invalidate_tokens.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_invalidate_host_rows.restype = ctypes.c_int
    lib.oracle_invalidate_host_rows.argtypes = [i32, i32, i64, i32, P, P, P, P, ctypes.c_int]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


@dataclass
class OracleState:
    """Resolver state of R request rows with S hot slots each, plus the
    simulated device pools (host arrays) of L layers."""
    R: int
    S: int
    L: int
    row_bytes: int
    dev_pool_rows: int
    slot_tokens: np.ndarray = field(default=None)
    lru_slots: np.ndarray = field(default=None)
    lru_clock: np.ndarray = field(default=None)
    stats: np.ndarray = field(default=None)
    dev_pools: list = field(default=None)

    def __post_init__(self):
        if self.slot_tokens is None:
            self.slot_tokens = np.full((self.R, self.S), -1, dtype=np.int32)
        if self.lru_slots is None:
            self.lru_slots = np.zeros((self.R, self.S), dtype=np.int32)
        if self.lru_clock is None:
            self.lru_clock = np.zeros((self.R,), dtype=np.int32)
        if self.stats is None:
            self.stats = np.zeros((5,), dtype=np.uint64)
        if self.dev_pools is None:
            self.dev_pools = [np.zeros((self.dev_pool_rows, self.row_bytes), dtype=np.uint8)
                              for _ in range(self.L)]


def oracle_resolve(state: OracleState, *, page_size: int, max_seq_len: int,
                   resident_pages: int, req_idx, top_k_tokens, seq_lens,
                   host_cache_locs, block_table, host_pools, host_pool_rows,
                   validate: bool = False) -> np.ndarray:
    """One resolver call on the oracle; returns device_buffer_locs [B, k]."""
    lib = load_oracle()
    req_idx = np.ascontiguousarray(req_idx, dtype=np.int32)
    top_k_tokens = np.ascontiguousarray(top_k_tokens, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    host_cache_locs = np.ascontiguousarray(host_cache_locs, dtype=np.int64)
    if block_table is not None:
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    B, k = top_k_tokens.shape
    out = np.empty((B, k), dtype=np.int32)
    hp = (ctypes.c_void_p * state.L)(*[int(_host_addr(h)) for h in host_pools])
    dp = (ctypes.c_void_p * state.L)(*[d.ctypes.data for d in state.dev_pools])
    hrows = np.ascontiguousarray(host_pool_rows, dtype=np.int64)
    rc = lib.oracle_resolve(state.R, state.S, state.row_bytes, state.L, page_size,
                            max_seq_len, resident_pages, B, k, _ptr(req_idx),
                            _ptr(top_k_tokens), _ptr(seq_lens), _ptr(host_cache_locs),
                            _ptr(block_table), _ptr(state.slot_tokens),
                            _ptr(state.lru_slots), _ptr(state.lru_clock), _ptr(out),
                            _ptr(state.stats), ctypes.cast(hp, ctypes.c_void_p),
                            _ptr(hrows), ctypes.cast(dp, ctypes.c_void_p),
                            state.dev_pool_rows, 1 if validate else 0)
    if rc != 0:
        raise ValueError("oracle_resolve rejected its input (code %d)" % rc)
    return out


def _host_addr(h):
    """Address of a host buffer given as a numpy array or a CPU torch tensor."""
    if isinstance(h, np.ndarray):
        assert h.flags["C_CONTIGUOUS"]
        return h.ctypes.data
    # torch CPU tensor (pinned or not)
    assert not h.is_cuda and h.is_contiguous()
    return h.data_ptr()


def oracle_sparse_mla_decode(q_bf16_bits, locs, dev_pool, softmax_scale: float,
                             row_bytes: int = 656, threads: int = 0) -> np.ndarray:
    """Float64 attention output [B, H, 512] for bf16 queries given as uint16
    bit patterns [B, H, 576] over the rows of ``dev_pool`` named by ``locs``.

    ``threads`` > 1 runs batch rows concurrently, each through the same C
    function on its own rows (ctypes releases the GIL during the call); the
    rows are independent, so the result is the same as one call over all
    of them.  0 picks min(batch, CPU count, 16)."""
    lib = load_oracle()
    q = np.ascontiguousarray(q_bf16_bits, dtype=np.uint16)
    locs = np.ascontiguousarray(locs, dtype=np.int32)
    B, H, D = q.shape
    assert D == 576
    k = locs.shape[1]
    out = np.empty((B, H, 512), dtype=np.float64)
    pool_addr = _host_addr(dev_pool)
    rows = dev_pool.shape[0]

    def run(b0, b1):
        rc = lib.oracle_sparse_mla_decode(b1 - b0, H, k, _ptr(q[b0:b1]), _ptr(locs[b0:b1]),
                                          pool_addr, rows, row_bytes,
                                          ctypes.c_float(softmax_scale), _ptr(out[b0:b1]))
        if rc != 0:
            raise ValueError("oracle_sparse_mla_decode failed (code %d)" % rc)

    if threads == 0:
        threads = min(B, os.cpu_count() or 1, 16)
    if threads <= 1 or B <= 1:
        run(0, B)
        return out
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for f in [ex.submit(run, b, b + 1) for b in range(B)]:
            f.result()
    return out


def e4m3_to_double(code: int) -> float:
    return load_oracle().oracle_e4m3_to_double(code)


def bf16_to_double(bits: int) -> float:
    return load_oracle().oracle_bf16_to_double(bits)


def oracle_mirror_rows(state: OracleState, *, dev_rows, host_rows, host_pools, host_pool_rows,
                       layer_begin: int = 0, layer_end=None, validate: bool = False):
    """Copy the oracle's device rows ``dev_rows`` to ``host_rows`` of the host
    pools (numpy arrays or CPU tensors, modified in place) in each layer."""
    lib = load_oracle()
    dev_rows = np.ascontiguousarray(dev_rows, dtype=np.int32)
    host_rows = np.ascontiguousarray(host_rows, dtype=np.int64)
    assert dev_rows.shape == host_rows.shape
    layer_end = state.L if layer_end is None else layer_end
    hp = (ctypes.c_void_p * state.L)(*[int(_host_addr(h)) for h in host_pools])
    dp = (ctypes.c_void_p * state.L)(*[d.ctypes.data for d in state.dev_pools])
    hrows = np.ascontiguousarray(host_pool_rows, dtype=np.int64)
    rc = lib.oracle_mirror_rows(state.row_bytes, len(dev_rows), _ptr(dev_rows), _ptr(host_rows),
                                ctypes.cast(dp, ctypes.c_void_p), state.dev_pool_rows,
                                ctypes.cast(hp, ctypes.c_void_p), _ptr(hrows), layer_begin,
                                layer_end, _ptr(state.stats), 1 if validate else 0)
    if rc != 0:
        raise ValueError("oracle_mirror_rows rejected its input (code %d)" % rc)


def oracle_invalidate_tokens(state: OracleState, *, req_rows, tok_begin, tok_end):
    """Clear the hot slots of the given request rows holding tokens in the ranges."""
    lib = load_oracle()
    req_rows = np.ascontiguousarray(req_rows, dtype=np.int32)
    tok_begin = np.ascontiguousarray(tok_begin, dtype=np.int32)
    tok_end = np.ascontiguousarray(tok_end, dtype=np.int32)
    rc = lib.oracle_invalidate_tokens(state.R, state.S, len(req_rows), _ptr(req_rows),
                                      _ptr(tok_begin), _ptr(tok_end), _ptr(state.slot_tokens),
                                      _ptr(state.lru_slots), _ptr(state.stats))
    if rc != 0:
        raise ValueError("oracle_invalidate_tokens rejected its input (code %d)" % rc)


def oracle_invalidate_host_rows(state: OracleState, *, rows, host_cache_locs, max_seq_len: int,
                                validate: bool = False):
    """Clear every hot slot whose token's host row is in ``rows`` (sorted)."""
    lib = load_oracle()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    host_cache_locs = np.ascontiguousarray(host_cache_locs, dtype=np.int64)
    rc = lib.oracle_invalidate_host_rows(state.R, state.S, max_seq_len, len(rows), _ptr(rows),
                                         _ptr(host_cache_locs), _ptr(state.slot_tokens),
                                         _ptr(state.lru_slots), 1 if validate else 0)
    if rc != 0:
        raise ValueError("oracle_invalidate_host_rows rejected its input (code %d)" % rc)
