"""Python binding of the tile-signaled GEMM library (``libtsg.so``).

Argument marshalling only: every step of every path runs in the library's HIP
kernels.  Tensors are passed by device address (``tensor.data_ptr()``);
streams by their HIP handle (``torch.cuda.current_stream().cuda_stream``).
Anything with a ``data_ptr()`` method (a torch tensor) or a plain integer
address is accepted.  The library must have been built
(``python tile_level_communication_signaled_amd/build.py``); importing this
package without it raises ImportError.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsg.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python tile_level_communication_signaled_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

# status codes
OK, E_INVALID, E_SHAPE, E_ALIGN, E_HIP, E_TIMEOUT, E_UNSUPPORTED, E_WORKSPACE = 0, -1, -2, -3, -4, -5, -6, -7
_NAMES = {0: "OK", -1: "E_INVALID", -2: "E_SHAPE", -3: "E_ALIGN", -4: "E_HIP", -5: "E_TIMEOUT",
          -6: "E_UNSUPPORTED", -7: "E_WORKSPACE"}
# modes
OVERLAP, SERIAL, COMPUTE_ONLY, COMM_ONLY = 0, 1, 2, 3
# dtypes
F32, BF16 = 0, 1
# ops (workspace sizing)
OP_AG, OP_RS, OP_MLP2, OP_MOE, OP_MOE_AG = 0, 1, 2, 3, 4

EXPORTS = (
    "tsg_ctx_create", "tsg_ctx_destroy", "tsg_last_error", "tsg_check", "tsg_device_info",
    "tsg_enable_kernel_timing", "tsg_kernel_ms", "tsg_timeline", "tsg_workspace_bytes",
    "tsg_moe_workspace_layout",
    "gemm_ag_overlap", "gemm_rs_overlap", "mlp2_pipelined", "moe_expert_combine",
    "moe_expert_combine_noalloc", "moe_ag_group_gemm", "ag_kv_attention",
)
MOE_NOALLOC_BYTES = 64 << 20   # the static workspace of moe_expert_combine_noalloc, per GPU

# fields of tsg_moe_workspace_layout, in order
MOE_LAYOUT_FIELDS = ("meta", "offs", "poffs", "rb_expert", "row_pair", "row_token", "pair_row", "h", "y",
                     "total", "rows_max", "rb_max", "bm", "rb_order", "rb_mask")


class Opts(ctypes.Structure):
    _fields_ = [
        ("aux_cus", ctypes.c_int),
        ("main_cus", ctypes.c_int),
        ("tile", ctypes.c_int),
        ("order", ctypes.c_int),
        ("timeout_ms", ctypes.c_uint32),
        ("debug_skip_mask", ctypes.c_uint32),
        ("timeline", ctypes.c_int),
        ("aux_wgs", ctypes.c_int),
        ("comm_tile", ctypes.c_int),
        ("pull_units", ctypes.c_int),
        ("stage_dtype", ctypes.c_int),
        ("arrival_gbps", ctypes.c_int),
        ("copy_engine", ctypes.c_int),
        ("channels", ctypes.c_int),
        ("ep_ranks", ctypes.c_int),
        ("ep_rank", ctypes.c_int),
    ]


_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_P = ctypes.POINTER
_lib.tsg_ctx_create.argtypes = [_i, _P(_vp)]
_lib.tsg_ctx_destroy.argtypes = [_vp]
_lib.tsg_ctx_destroy.restype = None
_lib.tsg_last_error.argtypes = [_vp]
_lib.tsg_last_error.restype = ctypes.c_char_p
_lib.tsg_check.argtypes = [_vp, _vp]
_lib.tsg_device_info.argtypes = [_vp, _P(_i), _P(_i)]
_lib.tsg_enable_kernel_timing.argtypes = [_vp, _i]
_lib.tsg_kernel_ms.argtypes = [_vp, _i, _P(ctypes.c_float)]
_lib.tsg_timeline.argtypes = [_vp, _P(ctypes.c_uint64), _sz, _P(_sz)]
_lib.tsg_workspace_bytes.argtypes = [_i, _P(ctypes.c_int64)]
_lib.tsg_workspace_bytes.restype = _sz
_lib.tsg_moe_workspace_layout.argtypes = [_P(ctypes.c_int64), _P(ctypes.c_int64), _i]
_lib.gemm_ag_overlap.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _P(_i), _P(Opts), _i, _vp]
_lib.gemm_rs_overlap.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _P(Opts), _i, _vp]
_lib.mlp2_pipelined.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _P(Opts), _i, _vp]
_lib.moe_expert_combine.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                    _i, _i, _i, _i, _i, _P(Opts), _i, _vp]
_lib.moe_ag_group_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                   _i, _i, _i, _i, _i, _i, _i, _P(_i), _P(Opts), _i, _vp]
_lib.ag_kv_attention.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _P(_i),
                                 _P(Opts), _i, _vp]
_lib.moe_expert_combine_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _i, _i, _i, _i, _i, _P(Opts), _i, _vp]
for _f in ("tsg_ctx_create", "tsg_check", "tsg_device_info", "tsg_enable_kernel_timing", "tsg_kernel_ms",
           "tsg_timeline", "tsg_moe_workspace_layout", "gemm_ag_overlap", "gemm_rs_overlap", "mlp2_pipelined",
           "moe_expert_combine", "moe_expert_combine_noalloc", "moe_ag_group_gemm", "ag_kv_attention"):
    getattr(_lib, _f).restype = _i


class TsgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_NAMES.get(status, status)}: {msg}")
        self.status = status


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _opts(o):
    if o is None:
        return None
    if isinstance(o, Opts):
        return ctypes.byref(o)
    return ctypes.byref(Opts(**o))


# Contexts still open, closed by _close_all() at interpreter exit.  A context
# owns HIP streams (CU-masked ones among them) and events; destroying them
# must happen while the HIP runtime is fully alive.  Left to garbage
# collection, a context can be destroyed during interpreter finalisation,
# after a profiler's or the runtime's own exit handlers have started to tear
# down the state those handles refer to.
_LIVE = weakref.WeakSet()


def _close_all():
    for ctx in list(_LIVE):
        ctx.close()


atexit.register(_close_all)


class Context:
    """Owns one library context (signal words, side streams, timeline).

    Closed by close(), when collected, or at the latest from an atexit hook,
    before the interpreter (and with it the HIP runtime) shuts down."""

    def __init__(self, device: int = 0):
        h = _vp()
        st = _lib.tsg_ctx_create(device, ctypes.byref(h))
        if st != OK:
            raise TsgError(st, f"tsg_ctx_create(device={device}) failed")
        self._h = h
        _LIVE.add(self)

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None):
            _lib.tsg_ctx_destroy(self._h)
            self._h = None
        _LIVE.discard(self)

    def __del__(self, _finalizing=sys.is_finalizing):
        # During interpreter shutdown the atexit hook has already closed every
        # context; a collection this late must not call into the runtime (nor
        # rely on module globals, which may already be cleared).
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def last_error(self) -> str:
        return _lib.tsg_last_error(self._h).decode()

    def _raise(self, st):
        if st != OK:
            raise TsgError(st, self.last_error())
        return st

    def check(self, stream=None) -> int:
        """Synchronise and return the device-side status (OK, E_TIMEOUT, ...)."""
        return _lib.tsg_check(self._h, _stream(stream))

    def device_info(self):
        """(number of CUs, number of XCDs)"""
        n, x = _i(), _i()
        self._raise(_lib.tsg_device_info(self._h, ctypes.byref(n), ctypes.byref(x)))
        return n.value, x.value

    def enable_kernel_timing(self, on: bool = True):
        self._raise(_lib.tsg_enable_kernel_timing(self._h, int(on)))

    def kernel_ms(self, which: int) -> float:
        v = ctypes.c_float()
        self._raise(_lib.tsg_kernel_ms(self._h, which, ctypes.byref(v)))
        return v.value

    def timeline(self, cap: int = 1 << 16):
        buf = (ctypes.c_uint64 * (4 * cap))()
        n = _sz()
        self._raise(_lib.tsg_timeline(self._h, buf, cap, ctypes.byref(n)))
        return [tuple(buf[4 * i:4 * i + 4]) for i in range(n.value)]


def workspace_bytes(op: int, dims) -> int:
    arr = (ctypes.c_int64 * len(dims))(*dims)
    return _lib.tsg_workspace_bytes(op, arr)


def moe_workspace_layout(dims) -> dict:
    """Regions of the MoE workspace for dims (T, H, I, E, k): byte offsets of
    meta, offs, poffs, rb_expert, row_pair, row_token, pair_row, h and y, the
    total size, and rows_max, rb_max and bm (see tsg_moe_workspace_layout)."""
    arr = (ctypes.c_int64 * 5)(*dims)
    out = (ctypes.c_int64 * len(MOE_LAYOUT_FIELDS))()
    st = _lib.tsg_moe_workspace_layout(arr, out, len(MOE_LAYOUT_FIELDS))
    if st != OK:
        raise TsgError(st, f"no MoE workspace layout for dims {tuple(dims)}")
    return dict(zip(MOE_LAYOUT_FIELDS, out))


def gemm_ag_overlap(ctx: Context, a_local, a_peers, a_full, b, c, c_dtype, M, N, K, R, rank,
                    arrival_order=None, opts=None, mode=OVERLAP, stream=None, raise_on_error=True):
    order = None
    if arrival_order is not None:
        order = (_i * len(arrival_order))(*arrival_order)
    st = _lib.gemm_ag_overlap(ctx.handle, _ptr(a_local), _ptr(a_peers), _ptr(a_full), _ptr(b), _ptr(c),
                              c_dtype, M, N, K, R, rank, order, _opts(opts), mode, _stream(stream))
    return ctx._raise(st) if raise_on_error else st


def gemm_rs_overlap(ctx: Context, x, w, partial, peer_partials, out, M, N, K, R, rank,
                    opts=None, mode=OVERLAP, stream=None, raise_on_error=True):
    st = _lib.gemm_rs_overlap(ctx.handle, _ptr(x), _ptr(w), _ptr(partial), _ptr(peer_partials), _ptr(out),
                              M, N, K, R, rank, _opts(opts), mode, _stream(stream))
    return ctx._raise(st) if raise_on_error else st


def mlp2_pipelined(ctx: Context, x, w1, h, w2, y, M, K1, N1, N2, opts=None, mode=OVERLAP, stream=None,
                   raise_on_error=True):
    st = _lib.mlp2_pipelined(ctx.handle, _ptr(x), _ptr(w1), _ptr(h), _ptr(w2), _ptr(y), M, K1, N1, N2,
                             _opts(opts), mode, _stream(stream))
    return ctx._raise(st) if raise_on_error else st


def moe_expert_combine(ctx: Context, x, topk_ids, topk_w, w_up, w_down, out, expert_counts, sorted_ids,
                       workspace, workspace_bytes_, T, H, I, E, k, opts=None, mode=OVERLAP, stream=None,
                       raise_on_error=True):
    st = _lib.moe_expert_combine(ctx.handle, _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_up), _ptr(w_down),
                                 _ptr(out), _ptr(expert_counts), _ptr(sorted_ids), _ptr(workspace),
                                 workspace_bytes_, T, H, I, E, k, _opts(opts), mode, _stream(stream))
    return ctx._raise(st) if raise_on_error else st


def moe_expert_combine_noalloc(ctx: Context, x, topk_ids, topk_w, w_up, w_down, out, expert_counts, sorted_ids,
                               T, H, I, E, k, opts=None, mode=OVERLAP, stream=None, raise_on_error=True):
    """moe_expert_combine with its workspace in the library's static device
    buffer (MOE_NOALLOC_BYTES per GPU): the call allocates nothing."""
    st = _lib.moe_expert_combine_noalloc(ctx.handle, _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w_up),
                                         _ptr(w_down), _ptr(out), _ptr(expert_counts), _ptr(sorted_ids),
                                         T, H, I, E, k, _opts(opts), mode, _stream(stream))
    return ctx._raise(st) if raise_on_error else st


def moe_ag_group_gemm(ctx: Context, x_local, x_peers, x_full, topk_ids, w_up, h, expert_counts, sorted_ids,
                      workspace, workspace_bytes_, T, H, I, E, k, R, rank, arrival_order=None, opts=None,
                      mode=OVERLAP, stream=None, raise_on_error=True):
    order = None
    if arrival_order is not None:
        order = (_i * len(arrival_order))(*arrival_order)
    st = _lib.moe_ag_group_gemm(ctx.handle, _ptr(x_local), _ptr(x_peers), _ptr(x_full), _ptr(topk_ids),
                                _ptr(w_up), _ptr(h), _ptr(expert_counts), _ptr(sorted_ids), _ptr(workspace),
                                workspace_bytes_, T, H, I, E, k, R, rank, order, _opts(opts), mode,
                                _stream(stream))
    return ctx._raise(st) if raise_on_error else st


def ag_kv_attention(ctx: Context, q, k_local, k_peers, v_local, v_peers, k_full, v_full, out, S, heads, head_dim,
                    R, rank, arrival_order=None, opts=None, mode=OVERLAP, stream=None, raise_on_error=True):
    order = None
    if arrival_order is not None:
        order = (_i * len(arrival_order))(*arrival_order)
    st = _lib.ag_kv_attention(ctx.handle, _ptr(q), _ptr(k_local), _ptr(k_peers), _ptr(v_local), _ptr(v_peers),
                              _ptr(k_full), _ptr(v_full), _ptr(out), S, heads, head_dim, R, rank, order,
                              _opts(opts), mode, _stream(stream))
    return ctx._raise(st) if raise_on_error else st
