"""Python binding of libstepq.so (argument marshalling only).

Every step of the decode path runs in the library's HIP kernels; this module checks shapes,
dtypes, devices and sizes on the host, then passes raw pointers.  PyTorch provides device memory
and streams.  There is no fallback: if the library is missing or was built for another target,
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstepq.so")

GDN, KDA = 0, 1
FUSED, SPLIT = 0, 1
DELTA_FIRST, DECAY_FIRST = 0, 1   # gate order: A = Diag(a)(I - b k k^T) or (I - b k k^T) Diag(a)
FLAG_NONFINITE, FLAG_SCALE_OVF, FLAG_PIVOT_OVF, FLAG_BAD_SLOT = 1, 2, 4, 8

_lib = None


class StepqError(RuntimeError):
    pass


class _Desc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("n_heads", ctypes.c_int), ("d_k", ctypes.c_int),
                ("d_v", ctypes.c_int), ("bits", ctypes.c_void_p), ("pivot", ctypes.c_void_p),
                ("omega", ctypes.c_void_p), ("mode", ctypes.c_int), ("max_batch", ctypes.c_int),
                ("device", ctypes.c_int), ("order", ctypes.c_int)]


def lib() -> ctypes.CDLL:
    """Load libstepq.so.  torch is imported first so that the library binds to the HIP runtime
    torch already loaded (same SONAME), sharing its streams and allocations."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (HIP runtime first)
    if not os.path.exists(LIB_PATH):
        raise StepqError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    P, i, sz, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
    sigs = {
        "stepq_plan_create": (i, [ctypes.POINTER(_Desc), ctypes.POINTER(P)]),
        "stepq_plan_destroy": (i, [P]),
        "stepq_pool_bytes": (i, [P, ctypes.POINTER(sz), ctypes.POINTER(d)]),
        "stepq_head_segment": (i, [P, i, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "stepq_encode_state": (i, [P, P, P, i, P]),
        "stepq_decode_step": (i, [P, P, i, P, P, P, P, P, P, P]),
        "stepq_decode_step_noalloc": (i, [P, P, i, P, P, P, P, P, P, P]),
        "stepq_encode_state_slots": (i, [P, P, P, i, P, i, P]),
        "stepq_decode_step_slots": (i, [P, P, i, P, i, P, P, P, P, P, P, P]),
        "stepq_unpack_debug": (i, [P, P, i, P, P, P, P, P]),
        "stepq_get_status": (i, [P, ctypes.POINTER(ctypes.c_uint32), i]),
        "stepq_sync": (i, [P]),
        "stepq_debug_side_delay": (i, [P, ctypes.c_longlong]),
        "stepq_last_error": (ctypes.c_char_p, []),
        "stepq_lifetime_weights": (i, [P, i, i, P]),
        "stepq_row_impact_accumulate": (i, [i, i, P, P, P, P, i, P]),
        "stepq_row_impact_gpu": (i, [i, i, i, i, i, P, P, P, P, P, P]),
        "stepq_select_pivots": (i, [P, i, i, P]),
        "stepq_alloc_mcdp": (i, [P, i, P, i, ctypes.c_long, P, ctypes.POINTER(d)]),
        "stepq_alloc_lagrangian": (i, [P, P, P, i, P, i, d, i, P, ctypes.POINTER(d)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(rc: int, what: str):
    if rc != 0:
        msg = lib().stepq_last_error().decode()
        raise StepqError(f"{what} failed ({rc}): {msg}")


def _np(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _dev_tensor(t, name, dtype, numel, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda" or t.device.index != device:
        raise ValueError(f"{name} must live on cuda:{device} (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """One layer's packed-state plan: widths, pivots and row impact per head (Method 1-2 of the
    STEPQuant digest), the derived packed layout, and (split mode) the side stream."""

    def __init__(self, kind, bits, pivot, omega, mode=FUSED, max_batch=1, device=0,
                 order=DELTA_FIRST):
        bits = _np(bits, np.int8)
        pivot = _np(pivot, np.uint8)
        omega = _np(omega, np.float32)
        if bits.ndim != 2 or pivot.shape != bits.shape or omega.shape != bits.shape:
            raise ValueError("bits, pivot and omega must all be [n_heads, d_k]")
        self.kind, self.mode, self.device, self.order = int(kind), int(mode), int(device), int(order)
        self.H, self.d = bits.shape
        self.max_batch = int(max_batch)
        self.bits, self.pivot, self.omega = bits, pivot, omega
        desc = _Desc(self.kind, self.H, self.d, self.d, bits.ctypes.data, pivot.ctypes.data,
                     omega.ctypes.data, self.mode, self.max_batch, self.device, self.order)
        h = ctypes.c_void_p()
        _check(lib().stepq_plan_create(ctypes.byref(desc), ctypes.byref(h)), "plan_create")
        self._h = h
        bpr, bpv = ctypes.c_size_t(), ctypes.c_double()
        _check(lib().stepq_pool_bytes(h, ctypes.byref(bpr), ctypes.byref(bpv)), "pool_bytes")
        self.bytes_per_request, self.bits_per_value = int(bpr.value), float(bpv.value)

    # -- housekeeping ----------------------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            _check(lib().stepq_plan_destroy(self._h), "plan_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def head_segment(self, h):
        off, n = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().stepq_head_segment(self._h, int(h), ctypes.byref(off), ctypes.byref(n)),
               "head_segment")
        return int(off.value), int(n.value)

    def alloc_pool(self, B):
        import torch
        return torch.zeros(B * self.bytes_per_request, dtype=torch.uint8,
                           device=f"cuda:{self.device}")

    def _pool(self, pool, B):
        import torch
        p = _dev_tensor(pool, "pool", torch.uint8, pool.numel(), self.device)
        if pool.numel() < B * self.bytes_per_request:
            raise ValueError(f"pool holds {pool.numel()} bytes, needs {B * self.bytes_per_request}")
        if pool.data_ptr() % 256:
            raise ValueError("pool must be 256-byte aligned")
        return p

    def _batch(self, B):
        if B < 0 or (self.mode == SPLIT and B > self.max_batch):
            raise ValueError(f"batch {B} outside [0, {self.max_batch if self.mode == SPLIT else 'inf'}]")

    # -- the path --------------------------------------------------------------------------
    def encode(self, S, pool, B, stream=None):
        import torch
        self._batch(B)
        sp = _dev_tensor(S, "S", torch.float32, B * self.H * self.d * self.d, self.device)
        _check(lib().stepq_encode_state(self._h, sp, self._pool(pool, B), int(B),
                                        _stream_ptr(stream)), "encode_state")

    def _step_args(self, B, q, k, v, alpha, beta, out):
        import torch
        n = B * self.H * self.d
        na = B * self.H * (self.d if self.kind == KDA else 1)
        f = torch.float32
        return [_dev_tensor(q, "q", f, n, self.device), _dev_tensor(k, "k", f, n, self.device),
                _dev_tensor(v, "v", f, n, self.device),
                _dev_tensor(alpha, "alpha", f, na, self.device),
                _dev_tensor(beta, "beta", f, B * self.H, self.device),
                _dev_tensor(out, "out", f, n, self.device)]

    def step(self, pool, B, q, k, v, alpha, beta, out, stream=None):
        self._batch(B)
        args = self._step_args(B, q, k, v, alpha, beta, out)
        _check(lib().stepq_decode_step(self._h, self._pool(pool, B), int(B), *args,
                                       _stream_ptr(stream)), "decode_step")

    def step_noalloc(self, pool, B, q, k, v, alpha, beta, out, stream=None):
        """stepq_decode_step_noalloc: the same step with no device allocation (split plans
        hand over through the library's static device scratch; B may exceed max_batch up to
        that scratch's size)."""
        if B < 0:
            raise ValueError("B must be >= 0")
        args = self._step_args(B, q, k, v, alpha, beta, out)
        _check(lib().stepq_decode_step_noalloc(self._h, self._pool(pool, B), int(B), *args,
                                               _stream_ptr(stream)), "decode_step_noalloc")

    # -- slot-indexed pools: batch row b uses pool slot slots[b] (-1 = padding row) --------
    def _slots(self, slots, B):
        import torch
        return _dev_tensor(slots, "slots", torch.int32, B, self.device)

    def encode_slots(self, S, pool, n_slots, slots, B, stream=None):
        import torch
        self._batch(B)
        sp = _dev_tensor(S, "S", torch.float32, B * self.H * self.d * self.d, self.device)
        _check(lib().stepq_encode_state_slots(self._h, sp, self._pool(pool, n_slots),
                                              int(n_slots), self._slots(slots, B), int(B),
                                              _stream_ptr(stream)), "encode_state_slots")

    def step_slots(self, pool, n_slots, slots, B, q, k, v, alpha, beta, out, stream=None):
        self._batch(B)
        args = self._step_args(B, q, k, v, alpha, beta, out)
        _check(lib().stepq_decode_step_slots(self._h, self._pool(pool, n_slots), int(n_slots),
                                             self._slots(slots, B), int(B), *args,
                                             _stream_ptr(stream)), "decode_step_slots")

    def unpack(self, pool, B, stream=None):
        """Returns S_hat [B,H,d,d] f32, r [B,H,d] u16 bits, c [B,H,d] u16 bits, z [B,H,d,d] i8."""
        import torch
        dev = f"cuda:{self.device}"
        S = torch.empty((B, self.H, self.d, self.d), dtype=torch.float32, device=dev)
        r = torch.empty((B, self.H, self.d), dtype=torch.int16, device=dev)
        c = torch.empty((B, self.H, self.d), dtype=torch.int16, device=dev)
        z = torch.empty((B, self.H, self.d, self.d), dtype=torch.int8, device=dev)
        _check(lib().stepq_unpack_debug(self._h, self._pool(pool, B), int(B),
                                        ctypes.c_void_p(S.data_ptr()), ctypes.c_void_p(r.data_ptr()),
                                        ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(z.data_ptr()),
                                        _stream_ptr(stream)), "unpack_debug")
        return S, r, c, z

    def status(self, reset=False):
        f = ctypes.c_uint32()
        _check(lib().stepq_get_status(self._h, ctypes.byref(f), int(bool(reset))), "get_status")
        return int(f.value)

    def sync(self):
        _check(lib().stepq_sync(self._h), "sync")

    def debug_side_delay(self, cycles):
        _check(lib().stepq_debug_side_delay(self._h, int(cycles)), "debug_side_delay")


# -- offline planning (host, binary64) ------------------------------------------------------

def lifetime_weights(l_u, H):
    l_u = _np(l_u, np.float64)
    out = np.empty_like(l_u)
    _check(lib().stepq_lifetime_weights(l_u.ctypes.data, l_u.size, int(H), out.ctypes.data),
           "lifetime_weights")
    return out


def row_impact_accumulate(q, k, a, beta, acc, order=DELTA_FIRST):
    q, k, a = _np(q, np.float32), _np(k, np.float32), _np(a, np.float32)
    beta = _np(beta, np.float32)
    n, d = q.shape
    assert k.shape == a.shape == (n, d) and beta.shape == (n,) and acc.shape == (d,)
    assert acc.dtype == np.float64 and acc.flags.c_contiguous
    _check(lib().stepq_row_impact_accumulate(n, d, q.ctypes.data, k.ctypes.data, a.ctypes.data,
                                             beta.ctypes.data, int(order), acc.ctypes.data),
           "row_impact_accumulate")
    return acc


def row_impact_gpu(kind, q, k, alpha, beta, acc, stream=None, order=DELTA_FIRST):
    """acc [H*d] float64 (device) += sum over requests of g_i^2, g = A^T q, for one step of one
    layer: q, k [B, H, d], alpha [B, H] (GDN) or [B, H, d] (KDA), beta [B, H] (device fp32)."""
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d]")
    B, H, d = q.shape
    dev = q.device.index
    f = torch.float32
    na = B * H * (d if kind == KDA else 1)
    args = [_dev_tensor(q, "q", f, B * H * d, dev), _dev_tensor(k, "k", f, B * H * d, dev),
            _dev_tensor(alpha, "alpha", f, na, dev), _dev_tensor(beta, "beta", f, B * H, dev),
            _dev_tensor(acc, "acc", torch.float64, H * d, dev)]
    _check(lib().stepq_row_impact_gpu(int(kind), int(order), int(H), int(d), int(B), *args,
                                      _stream_ptr(stream)), "row_impact_gpu")


def select_pivots(risk, n_pivots):
    risk = _np(risk, np.float64)
    out = np.empty(max(int(n_pivots), 1), np.int32)
    _check(lib().stepq_select_pivots(risk.ctypes.data, risk.size, int(n_pivots),
                                     out.ctypes.data), "select_pivots")
    return out[: int(n_pivots)].astype(np.int64)


def alloc_mcdp(cost, choices, capacity_bits):
    cost = _np(cost, np.float64)
    ch = _np(choices, np.int32)
    n = cost.shape[0]
    out = np.empty(max(n, 1), np.int32)
    obj = ctypes.c_double()
    _check(lib().stepq_alloc_mcdp(cost.ctypes.data, n, ch.ctypes.data, ch.size,
                                  int(capacity_bits), out.ctypes.data, ctypes.byref(obj)),
           "alloc_mcdp")
    return out[:n].astype(np.int64), float(obj.value)


def alloc_lagrangian(L, d, n, choices, budget_bits, iters=100):
    L, d, n = _np(L, np.float64), _np(d, np.float64), _np(n, np.float64)
    ch = _np(choices, np.int32)
    N = L.size
    out = np.empty(max(N, 1), np.int32)
    obj = ctypes.c_double()
    _check(lib().stepq_alloc_lagrangian(L.ctypes.data, d.ctypes.data, n.ctypes.data, N,
                                        ch.ctypes.data, ch.size, float(budget_bits), int(iters),
                                        out.ctypes.data, ctypes.byref(obj)), "alloc_lagrangian")
    return out[:N].astype(np.int64), float(obj.value)
