"""CPU checks of the C-ABI library: it loads, exports every function include/kvss.h declares,
and rejects bad arguments with the documented codes before any HIP call (so these run on a
machine without a GPU; no compute call is made)."""

import ctypes
import os

import pytest

from kv_sparse_speculative_amd import kvss

pytestmark = pytest.mark.skipif(not os.path.exists(kvss.LIB_PATH),
                                reason="libkvss.so not built")

FAKE = 0x1000     # a non-NULL address that is never dereferenced on the failure paths


def _desc(**kw):
    d = dict(k=FAKE, v=FAKE, block_table=FAKE, kv_lens=FAKE, batch=2, num_kv_heads=2,
             head_dim=128, block_size=16, max_blocks=4, num_blocks=8, max_kv_len=64,
             dtype=kvss.KVSS_BF16)
    d.update(kw)
    return kvss.kvss_kv(**d)


def test_exports_every_declared_function():
    names = kvss.declared_functions()
    assert set(names) == set(kvss._SIGNATURES), names
    lib = ctypes.CDLL(kvss.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert kvss.lib().kvss_version() == 1


def _verify(d, Hq=8, T=5, ws=None, wsb=0, q=FAKE, out=FAKE, scale=0.1):
    return kvss.lib().verify_attn_full(ctypes.byref(d), q, Hq, T, scale, out, None, ws, wsb, None)


@pytest.mark.parametrize("field,value,code", [
    ("dtype", 7, kvss.KVSS_EUNSUPPORTED),
    ("head_dim", 96, kvss.KVSS_EUNSUPPORTED),
    ("block_size", 8, kvss.KVSS_EUNSUPPORTED),
    ("batch", -1, kvss.KVSS_EINVAL),
    ("num_kv_heads", 0, kvss.KVSS_EINVAL),
    ("max_kv_len", 65, kvss.KVSS_EINVAL),       # > max_blocks * block_size
    ("k", None, kvss.KVSS_EINVAL),
    ("block_table", None, kvss.KVSS_EINVAL),
    ("batch", 70000, kvss.KVSS_EUNSUPPORTED),   # indexes a grid dimension
    ("num_blocks", 1 << 28, kvss.KVSS_EUNSUPPORTED),   # rows beyond 32-bit indexing
])
def test_kv_descriptor_validation(field, value, code):
    assert _verify(_desc(**{field: value})) == code
    assert kvss.lib().kvss_last_error().decode()


def test_verify_argument_validation():
    d = _desc()
    assert _verify(d, Hq=7) == kvss.KVSS_EINVAL              # not a multiple of Hkv
    assert _verify(d, T=0) == kvss.KVSS_EINVAL
    assert _verify(d, Hq=16, T=5) == kvss.KVSS_EUNSUPPORTED   # G * T = 40 > 32
    assert _verify(d, q=None) == kvss.KVSS_EINVAL
    assert _verify(d, scale=float("inf")) == kvss.KVSS_EINVAL
    assert kvss.lib().verify_attn_full(None, FAKE, 8, 5, 0.1, FAKE, None, None, 0, None) == kvss.KVSS_EINVAL


def test_workspace_too_small_is_rejected():
    d = _desc(batch=64, num_kv_heads=8, max_blocks=2001, num_blocks=128064, max_kv_len=32005)
    need = kvss.lib().kvss_verify_workspace_bytes(ctypes.byref(d), 32, 5)
    assert need > 0                  # long contexts are split
    assert _verify(d, Hq=32, T=5, ws=FAKE, wsb=need - 1) == kvss.KVSS_EWORKSPACE
    assert _verify(d, Hq=32, T=5, ws=None, wsb=need) == kvss.KVSS_EWORKSPACE
    assert "workspace" in kvss.lib().kvss_last_error().decode()


def test_empty_batch_is_a_no_op():
    d = _desc(batch=0, k=None, v=None, block_table=None, kv_lens=None)
    assert _verify(d) == kvss.KVSS_OK
    assert kvss.lib().kvss_last_error().decode() == ""


def test_draft_and_snapkv_validation():
    d = _desc()
    L = kvss.lib()
    assert L.draft_attn_sparse(ctypes.byref(d), FAKE, 8, None, None, 4, FAKE, 10, 0.1, FAKE, None,
                               None, 0, None) == kvss.KVSS_EINVAL          # k_max > 0 needs a list
    assert L.draft_attn_sparse(ctypes.byref(d), FAKE, 8, FAKE, FAKE, -1, FAKE, 10, 0.1, FAKE, None,
                               None, 0, None) == kvss.KVSS_EINVAL
    assert L.draft_attn_sparse(ctypes.byref(d), FAKE, 8, FAKE, FAKE, 4, FAKE, -2, 0.1, FAKE, None,
                               None, 0, None) == kvss.KVSS_EINVAL
    assert L.snapkv_select(ctypes.byref(d), FAKE, 8, 16, 7, 16, 0.1, FAKE, FAKE, None, None, 0,
                           None) == kvss.KVSS_EINVAL                       # budget <= w
    assert L.snapkv_select(ctypes.byref(d), FAKE, 8, 16, 6, 64, 0.1, FAKE, FAKE, None, None, 0,
                           None) == kvss.KVSS_EINVAL                       # even pool
    assert L.snapkv_select(ctypes.byref(d), FAKE, 8, 80, 7, 96, 0.1, FAKE, FAKE, None, None, 0,
                           None) == kvss.KVSS_EUNSUPPORTED                 # G * w > 256
    need = L.kvss_snapkv_workspace_bytes(ctypes.byref(d), 8, 16, 64)
    assert need > 0
    assert L.snapkv_select(ctypes.byref(d), FAKE, 8, 16, 7, 64, 0.1, FAKE, FAKE, None, FAKE,
                           need - 1, None) == kvss.KVSS_EWORKSPACE


def test_accept_and_streaming_validation():
    L = kvss.lib()
    args = [FAKE, FAKE, FAKE, 4, 3, 100, 1.0, 1, 0, FAKE, FAKE, None, None, 0, None]
    assert L.spec_accept(*args) == kvss.KVSS_EWORKSPACE
    bad = list(args); bad[6] = -1.0
    assert L.spec_accept(*bad) == kvss.KVSS_EINVAL
    bad = list(args); bad[5] = 1 << 24
    assert L.spec_accept(*bad) == kvss.KVSS_EINVAL
    bad = list(args); bad[1] = None
    assert L.spec_accept(*bad) == kvss.KVSS_EINVAL                         # temperature > 0 needs q
    bad = list(args); bad[3] = 65536
    assert L.spec_accept(*bad) == kvss.KVSS_EUNSUPPORTED                   # grid z holds the batch
    assert L.kvss_accept_workspace_bytes(4, 3, 100) >= 4 * 7 * 16
    assert L.kvss_streaming_set(FAKE, 2, 2, -1, 4, FAKE, FAKE, FAKE, None) == kvss.KVSS_EINVAL
    assert L.kvss_streaming_set(None, 2, 2, 4, 4, FAKE, FAKE, FAKE, None) == kvss.KVSS_EINVAL


def test_append_validation():
    lib = kvss.lib()
    d = _desc()
    app = lambda d, T=3, k=FAKE, v=FAKE, start=FAKE: lib.kvss_kv_append(ctypes.byref(d), k, v, T,
                                                                         start, None)
    assert app(d, T=-1) == kvss.KVSS_EINVAL
    assert app(d, k=None) == kvss.KVSS_EINVAL
    assert app(d, start=None) == kvss.KVSS_EINVAL
    assert app(d, k=FAKE + 8) == kvss.KVSS_EINVAL            # not 16-byte aligned
    assert app(_desc(dtype=5)) == kvss.KVSS_EUNSUPPORTED
    assert app(d, T=0) == kvss.KVSS_OK                       # nothing to write: no launch
    assert app(_desc(batch=0)) == kvss.KVSS_OK


def test_draft_cache_build_validation():
    lib = kvss.lib()
    src = _desc()
    dst = _desc(k=0x2000, v=0x3000, max_blocks=4, num_blocks=8, max_kv_len=0)

    def build(src=src, dst=dst, sel=FAKE, cnt=FAKE, k_max=16, tail=FAKE, max_tail=32, lens=FAKE):
        return lib.kvss_draft_cache_build(ctypes.byref(src), sel, cnt, k_max, tail, max_tail,
                                          ctypes.byref(dst), lens, None)
    assert build(k_max=-1) == kvss.KVSS_EINVAL
    assert build(max_tail=-1) == kvss.KVSS_EINVAL
    assert build(max_tail=64) == kvss.KVSS_EINVAL            # 16 + 64 > 4 * 16 slots
    assert build(sel=None) == kvss.KVSS_EINVAL
    assert build(cnt=None) == kvss.KVSS_EINVAL
    assert build(tail=None) == kvss.KVSS_EINVAL
    assert build(lens=None) == kvss.KVSS_EINVAL
    assert build(dst=_desc(k=0x2000, v=0x3000, num_kv_heads=1)) == kvss.KVSS_EINVAL
    assert build(dst=_desc(k=0x2000, v=0x3000, dtype=kvss.KVSS_F32)) == kvss.KVSS_EINVAL
    assert build(dst=_desc(k=0x2000, v=0x3000, batch=3)) == kvss.KVSS_EINVAL
    assert build(dst=_desc()) == kvss.KVSS_EINVAL            # aliases src
    assert build(dst=_desc(k=0x2008, v=0x3000)) == kvss.KVSS_EINVAL   # misaligned
    assert build(src=_desc(batch=0), dst=_desc(k=0x2000, v=0x3000, batch=0)) == kvss.KVSS_OK


def test_draft_sample_and_topk_validation():
    lib = kvss.lib()
    smp = lambda B=2, V=10, t=1.0, step=0, logits=FAKE, tok=FAKE, ws=FAKE, wsb=1 << 20: lib.draft_sample(
        logits, B, V, t, 1, 2, step, tok, None, ws, wsb, None)
    assert smp(B=-1) == kvss.KVSS_EINVAL
    assert smp(V=0) == kvss.KVSS_EINVAL
    assert smp(V=1 << 24) == kvss.KVSS_EINVAL
    assert smp(t=-1.0) == kvss.KVSS_EINVAL
    assert smp(t=float("nan")) == kvss.KVSS_EINVAL
    assert smp(t=1e-45) == kvss.KVSS_EINVAL                  # 1 / t overflows float
    assert smp(step=1 << 16) == kvss.KVSS_EINVAL
    assert smp(logits=None) == kvss.KVSS_EINVAL
    assert smp(ws=None) == kvss.KVSS_EWORKSPACE
    assert smp(wsb=8) == kvss.KVSS_EWORKSPACE
    assert smp(B=0) == kvss.KVSS_OK
    assert smp(B=65536) == kvss.KVSS_EUNSUPPORTED
    assert lib.kvss_sample_workspace_bytes(4, 1000) > 0
    d = _desc()
    topk = lambda d=d, Hq=8, k=16, ws=FAKE, wsb=1 << 30: lib.draft_attn_topk(
        ctypes.byref(d), FAKE, Hq, k, 0.1, FAKE, None, None, None, ws, wsb, None)
    assert topk(k=0) == kvss.KVSS_EINVAL
    assert topk(Hq=7) == kvss.KVSS_EINVAL
    assert topk(Hq=2 * 33) == kvss.KVSS_EUNSUPPORTED          # G = 33 > 32
    assert topk(wsb=16) == kvss.KVSS_EWORKSPACE
    assert lib.kvss_topk_workspace_bytes(ctypes.byref(d), 8, 16) > 0



def test_snapkv_workspace_holds_stored_scores_for_few_rows():
    """With bf16 and R = G * w <= 16 rows and 4 R < head_dim, the query adds the first pass's
    scaled scores: R floats per candidate, the candidate count rounded up to 4. Nothing else in
    the layout depends on head_dim, so the difference between head_dim 128 and 64 isolates it."""
    L = kvss.lib()

    def need(head_dim, w, dtype=kvss.KVSS_BF16):
        d = _desc(batch=3, num_kv_heads=2, head_dim=head_dim, max_blocks=40, num_blocks=120,
                  max_kv_len=601, dtype=dtype)
        return L.kvss_snapkv_workspace_bytes(ctypes.byref(d), 8, w, w + 32)

    # G = 4. w = 4: R = 16 is stored at head_dim 128 (64 < 128) but not at 64 (64 < 64 fails)
    n4 = (601 - 4 + 3) // 4 * 4
    extra = need(128, 4) - need(64, 4)
    assert 3 * 2 * 16 * n4 * 4 <= extra < 3 * 2 * 16 * n4 * 4 + 4096, extra
    assert need(128, 1) == need(64, 1)              # R = 4: stored at both head sizes
    assert need(128, 5) == need(64, 5)              # R = 20: never stored
    assert need(128, 4, kvss.KVSS_F32) == need(64, 4, kvss.KVSS_F32)   # fp32: never stored


def test_philox_validation():
    L = kvss.lib()
    assert L.kvss_philox4x32_10(FAKE, -1, 0, FAKE, None) == kvss.KVSS_EINVAL
    assert L.kvss_philox4x32_10(None, 4, 0, FAKE, None) == kvss.KVSS_EINVAL
    assert L.kvss_philox4x32_10(FAKE, 4, 0, None, None) == kvss.KVSS_EINVAL
    assert L.kvss_philox4x32_10(FAKE + 4, 4, 0, FAKE, None) == kvss.KVSS_EINVAL    # misaligned
    assert L.kvss_philox4x32_10(None, 0, 0, None, None) == kvss.KVSS_OK
    assert L.kvss_philox4x32_10(FAKE, (1 << 31) + 1, 0, FAKE, None) == kvss.KVSS_EUNSUPPORTED


def _verify_noalloc(d, Hq=8, T=5, q=FAKE, out=FAKE, scale=0.1):
    return kvss.lib().verify_attn_full_noalloc(ctypes.byref(d), q, Hq, T, scale, out, None, None)


def test_noalloc_verify_validation_and_scratch_limit():
    d = _desc()
    assert _verify_noalloc(d, Hq=7) == kvss.KVSS_EINVAL
    assert _verify_noalloc(d, T=0) == kvss.KVSS_EINVAL
    assert _verify_noalloc(d, Hq=16, T=5) == kvss.KVSS_EUNSUPPORTED
    assert _verify_noalloc(d, out=None) == kvss.KVSS_EINVAL
    assert _verify_noalloc(_desc(head_dim=96)) == kvss.KVSS_EUNSUPPORTED
    assert _verify_noalloc(_desc(batch=0, k=None, v=None, block_table=None, kv_lens=None)) == kvss.KVSS_OK
    # 1023 (sequence, KV head) pairs with 32 query rows each, split in two: 34,045,440 bytes of
    # partials, beyond the 32 MiB scratch -> rejected before any HIP call
    big = _desc(batch=1023, num_kv_heads=1, max_blocks=1300, num_blocks=1 << 20, max_kv_len=20000)
    need = kvss.lib().kvss_verify_workspace_bytes(ctypes.byref(big), 4, 8)
    assert need > 32 << 20
    assert _verify_noalloc(big, Hq=4, T=8) == kvss.KVSS_EWORKSPACE
    msg = kvss.lib().kvss_last_error().decode()
    assert "scratch" in msg and str(need) in msg
