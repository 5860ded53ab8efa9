"""GPU checks of the generator behind spec_accept and draft_sample: the library's device
Philox4x32-10 against the oracle's (each written from Salmon et al., SC'11) on 2^20 seeded
counters, bit-exact on all four output words; the acceptance and sampler counter layouts give
exactly the oracle's uniforms; and rocRAND's device Philox4x32-10, a third implementation run
through its documented state API (subsequence and offset), agrees word for word."""

import ctypes
import os

import numpy as np
import pytest
import torch

from oracle.philox import (accept_uniform, draft_uniforms, philox4x32_10, race_uniforms,
                           to_uniform)
from kv_sparse_speculative_amd import kvss

pytestmark = pytest.mark.gpu

HELPER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librocrand_philox.so")
N = 1 << 20


def _counters(n, seed, c1_bits=32):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 2 ** 32, size=(n, 4), dtype=np.uint64)
    c[:, 1] &= (1 << c1_bits) - 1
    return c.astype(np.uint32)


def _library(c, seed):
    t = torch.from_numpy(c.view(np.int32)).cuda()
    out = kvss.kvss_philox4x32_10(t, seed)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def _oracle(c, seed):
    key = (seed & 0xFFFFFFFF, seed >> 32)
    words = philox4x32_10(tuple(c[:, i] for i in range(4)), key)
    return np.stack(words, axis=1).astype(np.uint32)


@pytest.mark.parametrize("seed", [0, 1234, 0xDEADBEEFCAFEF00D])
def test_library_philox_equals_oracle(seed):
    c = _counters(N, 7)
    c[:4] = [[0, 0, 0, 0], [0xFFFFFFFF] * 4, [1, 0, 0, 0], [0, 0, 0, 0xFFFFFFFF]]
    np.testing.assert_array_equal(_library(c, seed), _oracle(c, seed))


def test_draw_layouts_give_the_oracle_uniforms():
    """u_i of the acceptance (stream 0), u'_x of the race (stream 1) and the draft sampler's
    uniforms (stream 2), read back through the library's generator at their documented
    counters."""
    seed, offset, vocab = 0x0123456789ABCDEF, 0x1_0000_0007, 1001
    nblk = (vocab + 3) // 4
    for b, pos in ((0, 0), (5, 3), (65534, 30)):
        c = np.array([[0, pos, b, offset & 0xFFFFFFFF]], dtype=np.uint32)
        u = to_uniform(_library(c, seed)[:, 0])[0]
        assert u == accept_uniform(seed, offset, b, pos)
        for stream, ref in ((1, race_uniforms), (2, draft_uniforms)):
            c = np.zeros((nblk, 4), dtype=np.uint32)
            c[:, 0] = np.arange(nblk)
            c[:, 1] = (stream << 16) | pos
            c[:, 2] = b
            c[:, 3] = offset & 0xFFFFFFFF
            u = to_uniform(_library(c, seed).reshape(-1))[:vocab]
            np.testing.assert_array_equal(u, ref(seed, offset, b, pos, vocab))


def test_rocrand_philox_agrees():
    assert os.path.exists(HELPER), f"{HELPER} is missing: build it with __graft_entry__.build()"
    lib = ctypes.CDLL(HELPER)
    lib.rocrand_philox.restype = ctypes.c_int
    lib.rocrand_philox.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_ulonglong,
                                   ctypes.c_void_p]
    c = _counters(N, 11, c1_bits=30)        # offset 4 * (c0 + 2^32 c1) stays below 2^64
    for seed in (0, 0x0123456789ABCDEF):
        t = torch.from_numpy(c.view(np.int32)).cuda()
        o = torch.empty_like(t)
        torch.cuda.synchronize()
        assert lib.rocrand_philox(t.data_ptr(), N, seed, o.data_ptr()) == 0
        np.testing.assert_array_equal(o.cpu().numpy().view(np.uint32), _library(c, seed))
