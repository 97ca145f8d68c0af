"""Argument errors at the C boundary on a real device: each call below must return its error
code and message without enqueuing work, and leave the plan usable (a valid step afterwards
runs and keeps the status word clear).  Calls go straight through ctypes, past the Python
binding's own checks."""
import ctypes

import numpy as np
import pytest

import paritylib as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_delta_rule_amd import stepq
    L = stepq.lib()
    dev = torch.device("cuda:0")
    H, d, B = 2, 128, 3
    bits = np.full((H, d), 6, np.int8)
    piv = np.zeros((H, d), np.uint8)
    om = np.ones((H, d), np.float32)
    fused = stepq.Plan(stepq.GDN, bits, piv, om)
    split = stepq.Plan(stepq.GDN, bits, piv, om, mode=stepq.SPLIT, max_batch=B)
    pool = fused.alloc_pool(B)
    S0 = (torch.randn(B * H, d, d, generator=torch.Generator().manual_seed(5)) * 0.1).to(dev)
    fused.encode(S0, pool, B)
    t = {n: torch.randn(B, H, d, device=dev) * 0.1 for n in ("q", "k", "v")}
    t["alpha"] = torch.full((B, H), 0.9, device=dev)
    t["beta"] = torch.full((B, H), 0.5, device=dev)
    t["out"] = torch.empty(B, H, d, device=dev)
    torch.cuda.synchronize()
    return torch, stepq, L, fused, split, pool, S0, t, B


def _ptrs(t):
    V = ctypes.c_void_p
    return [V(t[n].data_ptr()) for n in ("q", "k", "v", "alpha", "beta", "out")]


def _err(L, rc, code, text):
    msg = L.stepq_last_error().decode()
    assert rc == code, (rc, msg)
    assert text in msg, msg


def test_decode_argument_errors(env):
    torch, stepq, L, fused, split, pool, S0, t, B = env
    V = ctypes.c_void_p
    P.log("[errors] decode argument checks")
    before = pool.clone()
    q, k, v, a, b, o = _ptrs(t)
    pp = V(pool.data_ptr())
    s = V(torch.cuda.current_stream().cuda_stream)
    _err(L, L.stepq_decode_step(fused._h, pp, B, None, k, v, a, b, o, s), -1, "non-NULL")
    _err(L, L.stepq_decode_step(fused._h, pp, B, q, k, v, a, b, None, s), -1, "non-NULL")
    _err(L, L.stepq_decode_step(fused._h, V(pool.data_ptr() + 16), B, q, k, v, a, b, o, s), -1,
         "256-byte aligned")
    _err(L, L.stepq_decode_step(fused._h, None, B, q, k, v, a, b, o, s), -1, "pool is NULL")
    _err(L, L.stepq_decode_step(fused._h, pp, -1, q, k, v, a, b, o, s), -1, "B must be >= 0")
    _err(L, L.stepq_decode_step(None, pp, B, q, k, v, a, b, o, s), -1, "plan is NULL")
    _err(L, L.stepq_decode_step(split._h, pp, B + 1, q, k, v, a, b, o, s), -1, "max_batch")
    _err(L, L.stepq_decode_step(fused._h, pp, 2 ** 31 - 1, q, k, v, a, b, o, s), -1,
         "launch grid")
    _err(L, L.stepq_encode_state(fused._h, None, pp, B, s), -1, "S is NULL")
    _err(L, L.stepq_encode_state(fused._h, V(S0.data_ptr()), pp, 2 ** 31 - 1, s), -1,
         "launch grid")
    _err(L, L.stepq_unpack_debug(fused._h, pp, 2 ** 31 - 1, None, None, None, None, s), -1,
         "launch grid")
    _err(L, L.stepq_decode_step_slots(fused._h, pp, 0, V(t["q"].data_ptr()), B, q, k, v, a, b,
                                      o, s), -1, "n_slots")
    _err(L, L.stepq_decode_step_slots(fused._h, pp, B, None, B, q, k, v, a, b, o, s), -1,
         "slots is NULL")
    torch.cuda.synchronize()
    assert torch.equal(pool, before), "a refused call changed the pool"
    # the plan is still usable
    assert L.stepq_decode_step(fused._h, pp, B, q, k, v, a, b, o, s) == 0
    torch.cuda.synchronize()
    assert not torch.equal(pool, before)
    assert fused.status() == 0


def test_empty_batch_needs_no_pointers(env):
    torch, stepq, L, fused, split, pool, S0, t, B = env
    P.log("[errors] B = 0 with NULL pointers")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.stepq_decode_step(fused._h, None, 0, None, None, None, None, None, None, s) == 0
    assert L.stepq_encode_state(fused._h, None, None, 0, s) == 0
    assert L.stepq_unpack_debug(fused._h, None, 0, None, None, None, None, s) == 0
    torch.cuda.synchronize()
    assert fused.status() == 0
