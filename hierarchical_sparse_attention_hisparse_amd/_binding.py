"""ctypes binding of libhisparse.so: argument marshalling and host-side shape
checks only.  Names match the C entry points of include/hisparse.h."""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HISPARSE_LIBRARY=diag loads the diagnostic build (the same entry points, the
# plan kernel's phase trace compiled in, and the floor kernels).
_DIAG = os.environ.get("HISPARSE_LIBRARY", "") == "diag"
_LIB_PATH = os.path.join(_HERE, "libhisparse_diag.so" if _DIAG else "libhisparse.so")
_lib = None

STAT_NAMES = ("hot_hits", "misses", "resident_hits", "fast_path", "tripwires")


class HisparseError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__("%s failed (code %d): %s" % (where, code, msg))
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [
        ("max_requests", ctypes.c_int32), ("slots", ctypes.c_int32),
        ("max_top_k", ctypes.c_int32), ("max_batch", ctypes.c_int32),
        ("row_bytes", ctypes.c_int32), ("num_layers", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_steps", ctypes.c_int32),
        ("max_heads", ctypes.c_int32),
        ("resident_pages", ctypes.c_int64), ("max_seq_len", ctypes.c_int64),
    ]


@dataclass
class PoolConfig:
    max_requests: int
    slots: int
    max_top_k: int
    max_batch: int
    row_bytes: int = 656
    num_layers: int = 1
    page_size: int = 0
    resident_pages: int = 0
    max_seq_len: int = 0
    max_steps: int = 1
    max_heads: int = 0   # largest decode `heads` (multiple of 16); 0 = no decode workspace

    def _c(self) -> _Config:
        return _Config(self.max_requests, self.slots, self.max_top_k, self.max_batch,
                       self.row_bytes, self.num_layers, self.page_size, self.max_steps,
                       self.max_heads, self.resident_pages, self.max_seq_len)


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load the built library; raises if it is missing (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(os.path.basename(_LIB_PATH) + " is not built: run `python -m "
                          "hierarchical_sparse_attention_hisparse_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    V, I, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64
    lib.hisparse_last_error.restype = ctypes.c_char_p
    lib.hisparse_last_error.argtypes = []
    lib.hisparse_host_alloc.restype = I
    lib.hisparse_host_alloc.argtypes = [ctypes.c_size_t, ctypes.POINTER(V)]
    lib.hisparse_host_free.restype = I
    lib.hisparse_host_free.argtypes = [V]
    lib.hisparse_init_pool.restype = I
    lib.hisparse_init_pool.argtypes = [ctypes.POINTER(_Config), V, V, V, I64, ctypes.POINTER(V)]
    lib.hisparse_destroy_pool.restype = None
    lib.hisparse_destroy_pool.argtypes = [V]
    resolve_args = [V, V, I32, I32, V, V, V, V, V, V, V, V, V, V]
    lib.hisparse_resolve.restype = I
    lib.hisparse_resolve.argtypes = resolve_args
    lib.hisparse_resolve_plan.restype = I
    lib.hisparse_resolve_plan.argtypes = resolve_args
    lib.hisparse_gather_copy.restype = I
    lib.hisparse_gather_copy.argtypes = [V, V, I32, I32, I32, V]
    lib.hisparse_resolve_steps.restype = ctypes.c_int
    lib.hisparse_resolve_steps.argtypes = [V, V, I32] + resolve_args[2:]
    lib.hisparse_gather_copy_step.restype = ctypes.c_int
    lib.hisparse_gather_copy_step.argtypes = [V, V, I32, I32, I32, I32, V]
    lib.hisparse_mirror_rows.restype = ctypes.c_int
    lib.hisparse_mirror_rows.argtypes = [V, V, I32, V, V, I32, I32, V]
    lib.hisparse_invalidate_tokens.restype = ctypes.c_int
    lib.hisparse_invalidate_tokens.argtypes = [V, V, I32, V, V, V, V, V, V]
    lib.hisparse_invalidate_host_rows.restype = ctypes.c_int
    lib.hisparse_invalidate_host_rows.argtypes = [V, V, I32, V, V, V, V]
    lib.hisparse_decode_layers_overlapped.restype = I
    lib.hisparse_decode_layers_overlapped.argtypes = [V, V, I32, I32, I32, V, V,
                                                      ctypes.c_float, V, V]
    lib.hisparse_sparse_mla_decode.restype = I
    lib.hisparse_sparse_mla_decode.argtypes = [V, V, I32, I32, I32, I32, V, V,
                                               ctypes.c_float, V]
    lib.hisparse_sparse_mla_decode_noalloc.restype = I
    lib.hisparse_sparse_mla_decode_noalloc.argtypes = [V, I32, I32, I32, V, I64, I32, V, V,
                                                       ctypes.c_float, V]
    if _DIAG:
        lib.hisparse_diag_phase_clear.restype = I
        lib.hisparse_diag_phase_clear.argtypes = []
        lib.hisparse_diag_phase_read.restype = I
        lib.hisparse_diag_phase_read.argtypes = [V, ctypes.c_size_t]
        lib.hisparse_diag_floor.restype = I
        lib.hisparse_diag_floor.argtypes = [V, I32, I32, I32, I32, I32, I64, V, V, V, V, V, V, I32]
        lib.hisparse_diag_hit_detection.restype = I
        lib.hisparse_diag_hit_detection.argtypes = [V, I32, I32, I32, I32, I32, I64, V, V, V, V, V, I32]
        lib.hisparse_diag_exchange.restype = I
        lib.hisparse_diag_exchange.argtypes = [V, I32, I32, V, I32]
    _lib = lib
    return lib


def is_diag_library() -> bool:
    return _DIAG


def hisparse_last_error() -> str:
    return load_library().hisparse_last_error().decode("utf-8", "replace")


def _check_rc(rc: int, where: str):
    if rc != 0:
        raise HisparseError(rc, where, hisparse_last_error())


# ------------------------------------------------------------ host memory --

def hisparse_host_alloc(nbytes: int) -> int:
    p = ctypes.c_void_p()
    _check_rc(load_library().hisparse_host_alloc(nbytes, ctypes.byref(p)), "hisparse_host_alloc")
    return int(p.value)


def hisparse_host_free(ptr: int):
    _check_rc(load_library().hisparse_host_free(ctypes.c_void_p(ptr)), "hisparse_host_free")


class HostBuffer:
    """Pinned, device-mapped host memory from hisparse_host_alloc, viewable as
    a numpy array or a CPU torch tensor (views must not outlive it)."""

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.ptr = hisparse_host_alloc(self.nbytes)

    def numpy(self, shape=None, dtype=np.uint8) -> np.ndarray:
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        a = np.frombuffer(buf, dtype=np.uint8)
        a = a.view(dtype)
        return a.reshape(shape) if shape is not None else a

    def torch(self, shape=None, dtype=np.uint8):
        import torch
        return torch.from_numpy(self.numpy(shape, dtype))

    def free(self):
        if self.ptr:
            hisparse_host_free(self.ptr)
            self.ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


# ------------------------------------------------------------- marshalling --

def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t, dtype, shape: Optional[Sequence[int]], name: str, allow_none=False, device=None):
    """Checks one device tensor and returns its address.  `device`: the
    pool's device index (the library checks that it is the current one)."""
    import torch
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device (cuda) tensor" % name)
    if device is not None and t.get_device() != device:
        raise ValueError("%s is on cuda:%d, not on the pool's device cuda:%d"
                         % (name, t.get_device(), device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t.data_ptr()


class _Pool:
    def __init__(self, handle: int, cfg: PoolConfig, device_pool_rows: int, device: int, keep=()):
        self.handle = handle
        self.cfg = cfg
        self.device_pool_rows = device_pool_rows
        self.device = device
        # The library keeps raw pointers to the device pools and host buffers:
        # hold them for as long as the pool lives.
        self._keep = tuple(keep)


def hisparse_init_pool(config: PoolConfig, host_pools, host_pool_rows, device_pools,
                       device_pool_rows: int) -> _Pool:
    """host_pools: HostBuffer objects or pinned host addresses (one per layer);
    device_pools: uint8 cuda tensors [device_pool_rows, row_bytes]."""
    import torch
    L = config.num_layers
    if len(host_pools) != L or len(host_pool_rows) != L or len(device_pools) != L:
        raise ValueError("need one host pool, row count and device pool per layer")
    hp = (ctypes.c_void_p * L)()
    for l, h in enumerate(host_pools):
        addr = h.ptr if isinstance(h, HostBuffer) else int(h)
        if isinstance(h, HostBuffer) and h.nbytes < host_pool_rows[l] * config.row_bytes:
            raise ValueError("host pool %d holds fewer than host_pool_rows rows" % l)
        hp[l] = addr
    rows = (ctypes.c_int64 * L)(*[int(x) for x in host_pool_rows])
    dp = (ctypes.c_void_p * L)()
    cur = torch.cuda.current_device()
    for l, d in enumerate(device_pools):
        dp[l] = _dev(d, torch.uint8, (device_pool_rows, config.row_bytes), "device_pools[%d]" % l,
                     device=cur)
    c = config._c()
    out = ctypes.c_void_p()
    _check_rc(load_library().hisparse_init_pool(ctypes.byref(c), ctypes.cast(hp, ctypes.c_void_p),
                                                 ctypes.cast(rows, ctypes.c_void_p),
                                                 ctypes.cast(dp, ctypes.c_void_p),
                                                 device_pool_rows, ctypes.byref(out)),
              "hisparse_init_pool")
    return _Pool(int(out.value), config, device_pool_rows, cur,
                 keep=list(device_pools) + list(host_pools))


def hisparse_destroy_pool(pool: _Pool):
    if pool is not None and pool.handle:
        load_library().hisparse_destroy_pool(ctypes.c_void_p(pool.handle))
        pool.handle = 0
        pool._keep = ()


def _resolve_ptrs(pool, batch, top_k, req_idx, top_k_tokens, seq_lens, host_cache_locs,
                  resident_block_table, slot_tokens, lru_slots, lru_clock,
                  device_buffer_locs, stats, steps=None):
    import torch
    c = pool.cfg
    R, S = c.max_requests, c.slots
    max_pages = (c.max_seq_len + c.page_size - 1) // c.page_size if c.page_size > 0 else 0
    lead = () if steps is None else (steps,)
    return [
        _dev(req_idx, torch.int32, (batch,), "req_idx", device=pool.device),
        _dev(top_k_tokens, torch.int32, lead + (batch, top_k), "top_k_tokens", device=pool.device),
        _dev(seq_lens, torch.int32, lead + (batch,), "seq_lens", device=pool.device),
        _dev(host_cache_locs, torch.int64, (R, c.max_seq_len), "host_cache_locs", device=pool.device),
        _dev(resident_block_table, torch.int32, (R, max_pages), "resident_block_table",
             allow_none=True, device=pool.device),
        _dev(slot_tokens, torch.int32, (R, S), "slot_tokens", device=pool.device),
        _dev(lru_slots, torch.int32, (R, S), "lru_slots", device=pool.device),
        _dev(lru_clock, torch.int32, (R,), "lru_clock", device=pool.device),
        _dev(device_buffer_locs, torch.int32, lead + (batch, top_k), "device_buffer_locs", device=pool.device),
        _dev(stats, torch.int64, (5,), "stats", allow_none=True, device=pool.device),
    ]


def hisparse_resolve_steps(pool, stream, steps, batch, top_k, req_idx, top_k_tokens, seq_lens,
                           host_cache_locs, resident_block_table, slot_tokens, lru_slots,
                           lru_clock, device_buffer_locs, stats=None):
    """The verification steps of one speculative decode step: top_k_tokens
    [steps, batch, top_k], seq_lens [steps, batch], device_buffer_locs
    [steps, batch, top_k]."""
    ptrs = _resolve_ptrs(pool, batch, top_k, req_idx, top_k_tokens, seq_lens, host_cache_locs,
                         resident_block_table, slot_tokens, lru_slots, lru_clock,
                         device_buffer_locs, stats, steps=steps)
    _check_rc(load_library().hisparse_resolve_steps(pool.handle, _stream_handle(stream), steps,
                                                    batch, top_k, *ptrs), "hisparse_resolve_steps")


def hisparse_gather_copy_step(pool, stream, step, batch, layer_begin=0, layer_end=None,
                              stats=None):
    import torch
    if layer_end is None:
        layer_end = pool.cfg.num_layers
    sp = _dev(stats, torch.int64, (5,), "stats", allow_none=True, device=pool.device)
    _check_rc(load_library().hisparse_gather_copy_step(pool.handle, _stream_handle(stream), step,
                                                       batch, layer_begin, layer_end, sp),
              "hisparse_gather_copy_step")


def hisparse_resolve(pool, stream, batch, top_k, req_idx, top_k_tokens, seq_lens,
                     host_cache_locs, resident_block_table, slot_tokens, lru_slots,
                     lru_clock, device_buffer_locs, stats=None):
    """One decode step (plan + miss copy); stats is an int64 cuda tensor [5]
    holding the uint64 counters, or None."""
    ptrs = _resolve_ptrs(pool, batch, top_k, req_idx, top_k_tokens, seq_lens, host_cache_locs,
                         resident_block_table, slot_tokens, lru_slots, lru_clock,
                         device_buffer_locs, stats)
    _check_rc(load_library().hisparse_resolve(pool.handle, _stream_handle(stream), batch, top_k,
                                              *ptrs), "hisparse_resolve")


def hisparse_resolve_plan(pool, stream, batch, top_k, req_idx, top_k_tokens, seq_lens,
                          host_cache_locs, resident_block_table, slot_tokens, lru_slots,
                          lru_clock, device_buffer_locs, stats=None):
    ptrs = _resolve_ptrs(pool, batch, top_k, req_idx, top_k_tokens, seq_lens, host_cache_locs,
                         resident_block_table, slot_tokens, lru_slots, lru_clock,
                         device_buffer_locs, stats)
    _check_rc(load_library().hisparse_resolve_plan(pool.handle, _stream_handle(stream), batch,
                                                   top_k, *ptrs), "hisparse_resolve_plan")


def hisparse_gather_copy(pool, stream, batch, layer_begin=0, layer_end=None, stats=None):
    import torch
    if layer_end is None:
        layer_end = pool.cfg.num_layers
    sp = _dev(stats, torch.int64, (5,), "stats", allow_none=True, device=pool.device)
    _check_rc(load_library().hisparse_gather_copy(pool.handle, _stream_handle(stream), batch,
                                                  layer_begin, layer_end, sp),
              "hisparse_gather_copy")


def hisparse_mirror_rows(pool, stream, dev_rows, host_rows, layer_begin=0, layer_end=None,
                         stats=None):
    """Copy device rows ``dev_rows`` (int32 [n]) to host rows ``host_rows``
    (int64 [n]) of every layer in [layer_begin, layer_end)."""
    import torch
    if layer_end is None:
        layer_end = pool.cfg.num_layers
    n = int(dev_rows.shape[0])
    dp = _dev(dev_rows, torch.int32, (n,), "dev_rows", device=pool.device)
    hp = _dev(host_rows, torch.int64, (n,), "host_rows", device=pool.device)
    sp = _dev(stats, torch.int64, (5,), "stats", allow_none=True, device=pool.device)
    _check_rc(load_library().hisparse_mirror_rows(pool.handle, _stream_handle(stream), n, dp, hp,
                                                  layer_begin, layer_end, sp),
              "hisparse_mirror_rows")


def hisparse_invalidate_tokens(pool, stream, req_rows, tok_begin, tok_end, slot_tokens,
                               lru_slots, stats=None):
    """Empty the hot slots of ``req_rows`` holding tokens in [tok_begin, tok_end)."""
    import torch
    n = int(req_rows.shape[0])
    R, S = pool.cfg.max_requests, pool.cfg.slots
    rp = _dev(req_rows, torch.int32, (n,), "req_rows", device=pool.device)
    bp = _dev(tok_begin, torch.int32, (n,), "tok_begin", device=pool.device)
    ep = _dev(tok_end, torch.int32, (n,), "tok_end", device=pool.device)
    stp = _dev(slot_tokens, torch.int32, (R, S), "slot_tokens", device=pool.device)
    lp = _dev(lru_slots, torch.int32, (R, S), "lru_slots", device=pool.device)
    sp = _dev(stats, torch.int64, (5,), "stats", allow_none=True, device=pool.device)
    _check_rc(load_library().hisparse_invalidate_tokens(pool.handle, _stream_handle(stream), n, rp,
                                                        bp, ep, stp, lp, sp),
              "hisparse_invalidate_tokens")


def hisparse_invalidate_host_rows(pool, stream, rows_sorted, host_cache_locs, slot_tokens,
                                  lru_slots):
    """Empty every hot slot whose token's host row is in ``rows_sorted``."""
    import torch
    n = int(rows_sorted.shape[0])
    R, S = pool.cfg.max_requests, pool.cfg.slots
    rp = _dev(rows_sorted, torch.int64, (n,), "rows_sorted", device=pool.device)
    lp_ = _dev(host_cache_locs, torch.int64, (R, pool.cfg.max_seq_len), "host_cache_locs", device=pool.device)
    stp = _dev(slot_tokens, torch.int32, (R, S), "slot_tokens", device=pool.device)
    lp = _dev(lru_slots, torch.int32, (R, S), "lru_slots", device=pool.device)
    _check_rc(load_library().hisparse_invalidate_host_rows(pool.handle, _stream_handle(stream), n,
                                                           rp, lp_, stp, lp),
              "hisparse_invalidate_host_rows")


def hisparse_sparse_mla_decode(pool, stream, batch, heads, top_k, layer, q_bf16,
                               device_buffer_locs, softmax_scale, out_bf16):
    import torch
    qp = _dev(q_bf16, torch.bfloat16, (batch, heads, 576), "q_bf16", device=pool.device)
    lp = _dev(device_buffer_locs, torch.int32, (batch, top_k), "device_buffer_locs", device=pool.device)
    op = _dev(out_bf16, torch.bfloat16, (batch, heads, 512), "out_bf16", device=pool.device)
    _check_rc(load_library().hisparse_sparse_mla_decode(pool.handle, _stream_handle(stream),
                                                        batch, heads, top_k, layer, qp, lp,
                                                        ctypes.c_float(softmax_scale), op),
              "hisparse_sparse_mla_decode")


def hisparse_sparse_mla_decode_noalloc(stream, batch, heads, top_k, device_pool, q_bf16,
                                       device_buffer_locs, softmax_scale, out_bf16):
    """The decode without a pool: ``device_pool`` is one layer's uint8 cuda
    tensor [rows, row_bytes]; nothing is allocated (static split workspace)."""
    import torch
    if device_pool.dim() != 2:
        raise ValueError("device_pool must be [rows, row_bytes]")
    dev = device_pool.get_device()
    pp = _dev(device_pool, torch.uint8, None, "device_pool", device=dev)
    qp = _dev(q_bf16, torch.bfloat16, (batch, heads, 576), "q_bf16", device=dev)
    lp = _dev(device_buffer_locs, torch.int32, (batch, top_k), "device_buffer_locs", device=dev)
    op = _dev(out_bf16, torch.bfloat16, (batch, heads, 512), "out_bf16", device=dev)
    _check_rc(load_library().hisparse_sparse_mla_decode_noalloc(
        _stream_handle(stream), batch, heads, top_k, pp, int(device_pool.shape[0]),
        int(device_pool.shape[1]), qp, lp, ctypes.c_float(softmax_scale), op),
        "hisparse_sparse_mla_decode_noalloc")


def hisparse_decode_layers_overlapped(pool, stream, batch, heads, top_k, q_per_layer,
                                      device_buffer_locs, softmax_scale, out_per_layer,
                                      stats=None):
    """Per-layer miss copy pipelined with per-layer decode, after a plan on
    ``stream``: layer 0's copy, then one launch per layer that decodes layer
    l while spare workgroups copy layer l + 1 and combine layer l - 1, all
    enqueued on ``stream`` alone."""
    import torch
    L = pool.cfg.num_layers
    if len(q_per_layer) != L or len(out_per_layer) != L:
        raise ValueError("need one query and one output tensor per layer")
    qs = (ctypes.c_void_p * L)(*[_dev(q, torch.bfloat16, (batch, heads, 576), "q_bf16[%d]" % l, device=pool.device)
                                 for l, q in enumerate(q_per_layer)])
    outs = (ctypes.c_void_p * L)(*[_dev(o, torch.bfloat16, (batch, heads, 512), "out_bf16[%d]" % l, device=pool.device)
                                   for l, o in enumerate(out_per_layer)])
    lp = _dev(device_buffer_locs, torch.int32, (batch, top_k), "device_buffer_locs", device=pool.device)
    sp = _dev(stats, torch.int64, (5,), "stats", allow_none=True, device=pool.device)
    _check_rc(load_library().hisparse_decode_layers_overlapped(
        pool.handle, _stream_handle(stream), batch, heads, top_k, ctypes.cast(qs, ctypes.c_void_p), lp, ctypes.c_float(softmax_scale),
        ctypes.cast(outs, ctypes.c_void_p), sp), "hisparse_decode_layers_overlapped")



# ------------------------------------------------- diagnostic library only --
TRACE_ROWS, TRACE_WAVES, TRACE_POINTS = 256, 16, 9   # include/hisparse_diag.h
EXCHANGE_ROW_INTS = 64 + 64 * 16


def _diag_library():
    if not _DIAG:
        raise RuntimeError("the diagnostic entry points need HISPARSE_LIBRARY=diag "
                           "(libhisparse_diag.so) set before the package is imported")
    return load_library()


def hisparse_diag_phase_clear():
    _check_rc(_diag_library().hisparse_diag_phase_clear(), "hisparse_diag_phase_clear")


def hisparse_diag_phase_read() -> np.ndarray:
    """The plan kernel's phase trace as uint64 [rows, waves, points, 2]."""
    out = np.zeros((TRACE_ROWS, TRACE_WAVES, TRACE_POINTS, 2), dtype=np.uint64)
    _check_rc(_diag_library().hisparse_diag_phase_read(out.ctypes.data, out.size),
              "hisparse_diag_phase_read")
    return out


def hisparse_diag_floor(stream, kind, batch, top_k=1, slots=1, max_requests=1, max_seq_len=1,
                        req_idx=None, top_k_tokens=None, slot_tokens=None, lru_slots=None,
                        host_cache_locs=None, out=None, launches=1):
    """``launches`` back-to-back launches of a floor kernel of the plan's
    shape (kind 0-3, see include/hisparse_diag.h) on ``stream``; tensors as
    hisparse_resolve takes them, ``out`` int32 [batch, top_k] scratch."""
    import torch
    req = _dev(req_idx, torch.int32, (batch,), "req_idx", allow_none=kind == 0)
    tk = _dev(top_k_tokens, torch.int32, (batch, top_k), "top_k_tokens", allow_none=kind != 3)
    st = _dev(slot_tokens, torch.int32, (max_requests, slots), "slot_tokens", allow_none=kind < 2)
    lru = _dev(lru_slots, torch.int32, (max_requests, slots), "lru_slots", allow_none=kind < 2)
    locs = _dev(host_cache_locs, torch.int64, (max_requests, max_seq_len), "host_cache_locs",
                allow_none=kind != 3)
    op = _dev(out, torch.int32, (batch, top_k), "out", allow_none=kind == 0)
    _check_rc(_diag_library().hisparse_diag_floor(
        _stream_handle(stream), kind, batch, top_k, slots, max_requests, max_seq_len,
        req, tk, st, lru, locs, op, launches), "hisparse_diag_floor")


def hisparse_diag_exchange(stream, batch, groups, scratch, launches=1):
    """``launches`` back-to-back launches of the last-arriver exchange among
    ``groups`` workgroups per batch row; ``scratch`` int32 cuda tensor
    [batch, EXCHANGE_ROW_INTS], zero before the first call."""
    import torch
    sp = _dev(scratch, torch.int32, (batch, EXCHANGE_ROW_INTS), "scratch")
    _check_rc(_diag_library().hisparse_diag_exchange(_stream_handle(stream), batch, groups, sp,
                                                      launches), "hisparse_diag_exchange")


def hisparse_diag_hit_detection(stream, mode, batch, top_k, slots, max_requests, max_seq_len,
                                req_idx, top_k_tokens, seq_lens, slot_tokens, out, launches=1):
    """Hit detection alone (mode 0: positions table probed by the slots; mode 1:
    slot -> token map probed by the entries; modes 2 and 3: the same with
    bucketed tables); ``out`` int32 [batch, top_k]."""
    import torch
    rp = _dev(req_idx, torch.int32, (batch,), "req_idx")
    tp = _dev(top_k_tokens, torch.int32, (batch, top_k), "top_k_tokens")
    sp = _dev(seq_lens, torch.int32, (batch,), "seq_lens")
    stp = _dev(slot_tokens, torch.int32, (max_requests, slots), "slot_tokens")
    op = _dev(out, torch.int32, (batch, top_k), "out")
    _check_rc(_diag_library().hisparse_diag_hit_detection(
        _stream_handle(stream), mode, batch, top_k, slots, max_requests, max_seq_len, rp, tp, sp,
        stp, op, launches), "hisparse_diag_hit_detection")
