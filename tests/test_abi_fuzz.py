"""Host-side checks of the C ABI under seeded random parameters (no GPU).

For thousands of parameter draws, edge values included (negative, zero, one,
each limit and one past it, values near 2^31), the calls must not crash and
must agree with their size queries: a size query returns 0 exactly for the
parameters its call rejects.  The calls run with batch 0, which validates
every argument and then returns before touching a pointer or the GPU.
Run under tests/sanitize.py this also exercises the host code with
AddressSanitizer and UndefinedBehaviorSanitizer.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import pytest

import eagle_tree_verification_draft_amd as E

FAKE = C.c_void_p(1 << 24)       # never dereferenced with batch 0
WS = C.c_void_p(1 << 21)         # 256-byte aligned stand-in for a workspace
EDGE = [-(1 << 31), -1, 0, 1, 2, 7, 8, 16, 17, 60, 63, 64, 65, 127, 128, 129, 1023, 1024, 1025,
        (1 << 17), (1 << 17) + 1, (1 << 24), (1 << 30), (1 << 31) - 1]


def _draw(rng, lo, hi):
    """Mostly a value in [lo, hi], sometimes an edge value."""
    if rng.random() < 0.25:
        return int(rng.choice(EDGE))
    return int(rng.integers(lo, hi + 1))


@pytest.mark.parametrize("chunk", range(4))
def test_tree_params_calls_agree_with_size_queries(chunk):
    L = E.lib()
    rng = np.random.default_rng(1234 + chunk)
    n_ok = 0
    for _ in range(1500):
        p = E.TreeParams(_draw(rng, 1, 8), _draw(rng, 1, 20), _draw(rng, 1, 18), _draw(rng, 1, 70),
                         _draw(rng, 0, 70), _draw(rng, 1, 140000), _draw(rng, 1, 66), _draw(rng, 1, 130),
                         _draw(rng, 0, 4))
        st = L.eagle_build_tree(C.byref(p), 0, FAKE, E.EAGLE_BF16, max(p.vocab, 1), None, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, WS, 1 << 30, None)
        size = L.eagle_build_tree_workspace_size(C.byref(p), 1)
        assert (st == E.EAGLE_OK) == (size > 0), (st, size, [getattr(p, f[0]) for f in p._fields_])
        if st != E.EAGLE_OK:
            assert st in (E.EAGLE_ERR_INVALID, E.EAGLE_ERR_UNSUPPORTED)
            assert L.eagle_last_error()
        n_ok += st == E.EAGLE_OK
    assert n_ok > 10   # the draws reach valid parameters too


@pytest.mark.parametrize("chunk", range(4))
def test_attn_params_calls_agree_with_size_queries(chunk):
    L = E.lib()
    rng = np.random.default_rng(4321 + chunk)
    n_ok = 0
    for _ in range(1500):
        a = E.AttnParams(_draw(rng, 1, 64), _draw(rng, 1, 16), int(rng.choice([64, 128, 96, 0, -64, 256])),
                         _draw(rng, 1, 66), int(rng.choice([0, 8, 16, 24, 32, 64, 5, -16, 1 << 20])),
                         _draw(rng, 0, 3000), _draw(rng, 0, 40000),
                         float(rng.choice([0.0, 0.088, -1.0, 1e30])),
                         int(rng.choice([E.EAGLE_BF16, E.EAGLE_F32, 7, -1])))
        st = L.eagle_tree_attn(C.byref(a), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               WS, 1 << 30, None)
        size = L.eagle_tree_attn_workspace_size(C.byref(a), 1)
        assert (st == E.EAGLE_OK) == (size > 0), (st, size, [getattr(a, f[0]) for f in a._fields_])
        if st != E.EAGLE_OK:
            assert st in (E.EAGLE_ERR_INVALID, E.EAGLE_ERR_UNSUPPORTED)
        n_ok += st == E.EAGLE_OK
    assert n_ok >= 5
