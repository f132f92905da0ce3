"""The C ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host before any HIP call (these tests run with
no GPU: a HIP call would fail with KVQ_EHIP, not the code checked here)."""
import ctypes
import os
import re

import pytest

import quantized_kv_cache_group_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kvq.LIB_PATH), reason="libkvq.so not built")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(kvq_\w+)\s*\(", src, re.M)))


def test_header_symbols_exported():
    names = _declared()
    assert set(names) == set(kvq.SYMBOLS)
    L = kvq.lib()
    for n in names:
        assert getattr(L, n) is not None


def _needed(path):
    """DT_NEEDED entries of a shared library (readelf -d)."""
    import subprocess
    out = subprocess.run(["readelf", "-d", path], capture_output=True, text=True, check=True).stdout
    return re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out)


def test_library_links_hip_and_not_oracle():
    """libkvq.so depends on the HIP runtime and not on the oracle: its
    DT_NEEDED list names libamdhip64 and nothing of libkvq_ref, and loading
    it maps the HIP runtime but not the oracle."""
    needed = _needed(kvq.LIB_PATH)
    assert any(n.startswith("libamdhip64") for n in needed), needed
    assert not any("kvq_ref" in n for n in needed), needed
    import sys
    before = "oracle" in sys.modules
    kvq.lib()
    maps = open(f"/proc/{os.getpid()}/maps").read()
    assert os.path.basename(kvq.LIB_PATH) in maps
    assert "libamdhip64" in maps
    if not before:                      # nothing in this process has loaded the oracle yet
        assert "libkvq_ref" not in maps


def test_block_bytes():
    assert kvq.block_bytes(4, 8, 128) == 36864
    assert [kvq.block_bytes(b, 8, 256) for b in (2, 3, 4, 8)] == [40960, 57344, 73728, 139264]
    assert kvq.block_bytes(4, 1, 512) == 512 * 36
    assert kvq.block_bytes(5, 8, 128) == 0
    assert kvq.block_bytes(4, 8, 96) == 0
    assert kvq.block_bytes(4, 0, 128) == 0
    assert kvq.block_bytes(4, 8, 576) == 0


def test_strerror():
    L = kvq.lib()
    for c in (0, -1, -2, -3, -4, 7):
        assert L.kvq_strerror(c)


FAKE = 0x100000  # a 256-aligned non-null address; never dereferenced on error paths


def _layout(**kw):
    d = dict(n_seqs=1, n_heads=2, head_dim=64, max_blocks=4, window_cap=0,
             n_blocks=FAKE, n_window=FAKE, bits=FAKE)
    d.update(kw)
    return kvq.Layout(**d)


def _store(**kw):
    d = dict(offset=FAKE, pool=FAKE, window=FAKE)
    d.update(kw)
    return kvq.Store(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(n_seqs=0), kvq.KVQ_EINVAL),
    (dict(n_heads=0), kvq.KVQ_EINVAL),
    (dict(head_dim=100), kvq.KVQ_EINVAL),
    (dict(head_dim=0), kvq.KVQ_EINVAL),
    (dict(head_dim=576), kvq.KVQ_EUNSUPPORTED),
    (dict(max_blocks=-1), kvq.KVQ_EINVAL),
    (dict(n_blocks=None), kvq.KVQ_EINVAL),
    (dict(bits=None), kvq.KVQ_EINVAL),
    (dict(window_cap=8, n_window=None), kvq.KVQ_EINVAL),
    (dict(n_blocks=FAKE + 2), kvq.KVQ_EINVAL),
])
def test_quantize_rejects_bad_layout(kw, code):
    L, S = _layout(**kw), _store()
    assert kvq.lib().kvq_quantize(ctypes.byref(L), ctypes.byref(S), ctypes.c_void_p(FAKE), 256,
                                  None) == code


def test_quantize_rejects_bad_buffers():
    L = _layout()
    q = kvq.lib().kvq_quantize
    assert q(ctypes.byref(L), ctypes.byref(_store(pool=FAKE + 16)), ctypes.c_void_p(FAKE), 256, None) == kvq.KVQ_EINVAL
    assert q(ctypes.byref(L), ctypes.byref(_store(offset=None)), ctypes.c_void_p(FAKE), 256, None) == kvq.KVQ_EINVAL
    assert q(ctypes.byref(L), ctypes.byref(_store()), None, 256, None) == kvq.KVQ_EINVAL
    assert q(ctypes.byref(L), ctypes.byref(_store()), ctypes.c_void_p(FAKE + 2), 256, None) == kvq.KVQ_EINVAL
    assert q(ctypes.byref(L), ctypes.byref(_store()), ctypes.c_void_p(FAKE), 255, None) == kvq.KVQ_EINVAL
    assert q(None, ctypes.byref(_store()), ctypes.c_void_p(FAKE), 256, None) == kvq.KVQ_EINVAL


def test_quantize_kv_rejects():
    L = _layout()
    q = kvq.lib().kvq_quantize_kv
    K, V = _store(), _store()
    src = ctypes.c_void_p(FAKE)
    assert q(ctypes.byref(L), ctypes.byref(K), ctypes.byref(V), src, None, 256, None) == kvq.KVQ_EINVAL
    assert q(ctypes.byref(L), ctypes.byref(K), ctypes.byref(_store(pool=FAKE + 16)), src, src, 256,
             None) == kvq.KVQ_EINVAL
    assert q(ctypes.byref(L), ctypes.byref(K), ctypes.byref(V), src, ctypes.c_void_p(FAKE + 2), 256,
             None) == kvq.KVQ_EINVAL
    assert q(ctypes.byref(L), None, ctypes.byref(V), src, src, 256, None) == kvq.KVQ_EINVAL
    assert q(ctypes.byref(L), ctypes.byref(K), ctypes.byref(V), src, src, 255, None) == kvq.KVQ_EINVAL
    big = _layout(n_seqs=40000)
    assert q(ctypes.byref(big), ctypes.byref(K), ctypes.byref(V), src, src, 256, None) == kvq.KVQ_EUNSUPPORTED
    assert q(ctypes.byref(_layout(max_blocks=0)), ctypes.byref(K), ctypes.byref(V), src, src, 0,
             None) == kvq.KVQ_OK


def test_quantize_empty_layout_is_noop():
    L = _layout(max_blocks=0)
    assert kvq.lib().kvq_quantize(ctypes.byref(L), ctypes.byref(_store()), ctypes.c_void_p(FAKE), 0,
                                  None) == kvq.KVQ_OK


def test_dequantize_rejects():
    L = _layout()
    d = kvq.lib().kvq_dequantize
    assert d(ctypes.byref(L), ctypes.byref(_store()), 7, ctypes.c_void_p(FAKE), 256, None) == kvq.KVQ_EUNSUPPORTED
    assert d(ctypes.byref(L), ctypes.byref(_store()), 0, None, 256, None) == kvq.KVQ_EINVAL
    assert d(ctypes.byref(L), ctypes.byref(_store()), 0, ctypes.c_void_p(FAKE), 100, None) == kvq.KVQ_EINVAL
    Lw = _layout(window_cap=8)
    assert d(ctypes.byref(Lw), ctypes.byref(_store(window=None)), 0, ctypes.c_void_p(FAKE), 264, None) == kvq.KVQ_EINVAL


def _decode(L, K, V=None, rope=None, rope_dim=0, q=FAKE, Hq=8, scale=0.125, out=FAKE, ws=FAKE,
            ws_bytes=1 << 40):
    return kvq.lib().kvq_attend_decode(ctypes.byref(L), ctypes.byref(K),
                                       None if V is None else ctypes.byref(V),
                                       None if rope is None else ctypes.c_void_p(rope), rope_dim,
                                       None if q is None else ctypes.c_void_p(q), Hq, scale,
                                       None if out is None else ctypes.c_void_p(out),
                                       None if ws is None else ctypes.c_void_p(ws), ws_bytes, None)


def test_decode_rejects():
    L, K = _layout(), _store()
    assert _decode(L, K, Hq=7) == kvq.KVQ_EINVAL            # not a multiple of KV heads
    assert _decode(L, K, Hq=0) == kvq.KVQ_EINVAL
    assert _decode(L, K, Hq=34) == kvq.KVQ_EUNSUPPORTED     # 17 query heads per KV head
    assert _decode(L, K, q=None) == kvq.KVQ_EINVAL
    assert _decode(L, K, out=None) == kvq.KVQ_EINVAL
    assert _decode(L, K, q=FAKE + 4) == kvq.KVQ_EINVAL
    assert _decode(L, K, scale=float("nan")) == kvq.KVQ_EINVAL
    assert _decode(L, K, scale=0.0) == kvq.KVQ_EINVAL        # scales must be positive
    assert _decode(L, K, scale=-0.125) == kvq.KVQ_EINVAL
    assert _decode(L, K, scale=float("inf")) == kvq.KVQ_EINVAL
    assert _decode(L, K, rope_dim=64) == kvq.KVQ_EINVAL     # rope_dim without a rope buffer
    assert _decode(L, K, rope=FAKE, rope_dim=0) == kvq.KVQ_EINVAL
    assert _decode(L, K, rope=FAKE, rope_dim=32) == kvq.KVQ_EUNSUPPORTED
    assert _decode(L, K, ws_bytes=0) == kvq.KVQ_ENOSPC
    assert _decode(L, K, ws=None) == kvq.KVQ_EINVAL
    assert _decode(L, K, ws=FAKE + 64) == kvq.KVQ_EINVAL
    assert _decode(L, _store(pool=None)) == kvq.KVQ_EINVAL
    assert _decode(L, K, V=_store(offset=FAKE + 4)) == kvq.KVQ_EINVAL


def test_workspace_queries():
    L = _layout()
    n = ctypes.c_size_t(0)
    assert kvq.lib().kvq_decode_workspace(ctypes.byref(L), 8, 0, ctypes.byref(n)) == kvq.KVQ_OK
    assert n.value > 0 and n.value % 256 == 0
    assert kvq.lib().kvq_decode_workspace(ctypes.byref(L), 8, 0, None) == kvq.KVQ_EINVAL
    assert kvq.lib().kvq_decode_workspace(ctypes.byref(L), 5, 0, ctypes.byref(n)) == kvq.KVQ_EINVAL
    m = ctypes.c_size_t(0)
    assert kvq.lib().kvq_chunk_workspace(ctypes.byref(L), 8, 16, ctypes.byref(m)) == kvq.KVQ_OK
    assert m.value > 0
    assert kvq.lib().kvq_chunk_workspace(ctypes.byref(L), 8, -1, ctypes.byref(m)) == kvq.KVQ_EINVAL


def test_chunk_rejects():
    L, K, V = _layout(), _store(), _store()
    c = kvq.lib().kvq_attend_chunk
    args = lambda **kw: dict(dict(q=FAKE, k=FAKE, v=FAKE, n=16, Hq=8, scale=0.1, out=FAKE, ws=FAKE,
                                  wsb=1 << 40), **kw)

    def call(Vs=V, **kw):
        a = args(**kw)
        P = lambda x: None if x is None else ctypes.c_void_p(x)
        return c(ctypes.byref(L), ctypes.byref(K), None if Vs is None else ctypes.byref(Vs),
                 P(a["q"]), P(a["k"]), P(a["v"]), a["n"], a["Hq"], a["scale"], P(a["out"]),
                 P(a["ws"]), a["wsb"], None)
    assert call(Vs=None) == kvq.KVQ_EUNSUPPORTED
    assert call(q=None) == kvq.KVQ_EINVAL
    assert call(k=FAKE + 2) == kvq.KVQ_EINVAL
    assert call(n=-1) == kvq.KVQ_EINVAL
    assert call(Hq=3) == kvq.KVQ_EINVAL
    assert call(wsb=16) == kvq.KVQ_ENOSPC
    assert call(scale=0.0) == kvq.KVQ_EINVAL
    assert call(scale=-0.1) == kvq.KVQ_EINVAL
    assert call(n=0) == kvq.KVQ_OK                            # nothing to do, nothing launched


def _topk(L, K, V=None, Hq=8, scale=0.125, top_k=4, selected=None, ws=FAKE, ws_bytes=1 << 40):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return kvq.lib().kvq_attend_decode_topk(ctypes.byref(L), ctypes.byref(K),
                                            None if V is None else ctypes.byref(V), None, 0,
                                            P(FAKE), Hq, scale, top_k, P(FAKE), P(selected), P(ws),
                                            ws_bytes, None)


def test_topk_rejects():
    L, K, V = _layout(), _store(), _store()
    assert _topk(L, K, V, scale=0.0) == kvq.KVQ_EINVAL
    assert _topk(L, K, V, scale=-1.0) == kvq.KVQ_EINVAL
    assert _topk(L, K, V, top_k=0) == kvq.KVQ_EINVAL
    assert _topk(L, K, V, selected=FAKE + 2) == kvq.KVQ_EINVAL
    assert _topk(L, K, V, ws_bytes=16) == kvq.KVQ_ENOSPC
    assert _topk(L, K, V, ws=FAKE + 64) == kvq.KVQ_EINVAL


def test_topk_window_only_layout_with_null_tables():
    """A window-only layout may pass null widths, offsets and pools: the
    workspace query succeeds and argument checks reach the workspace size
    with no table dereferenced (on the GPU the call keeps no block)."""
    L = _layout(max_blocks=0, window_cap=64, bits=None)
    K = _store(offset=None, pool=None)
    V = _store(offset=None, pool=None)
    n = ctypes.c_size_t(0)
    assert kvq.lib().kvq_topk_workspace(ctypes.byref(L), 8, 0, 4, ctypes.byref(n)) == kvq.KVQ_OK
    assert n.value > 0 and n.value % 256 == 0
    assert _topk(L, K, V, ws_bytes=n.value - 1) == kvq.KVQ_ENOSPC
    assert _topk(L, K, V, scale=0.0, ws_bytes=n.value) == kvq.KVQ_EINVAL


def test_sensitivity_rejects_nonpositive_scale():
    f = kvq.lib().kvq_block_sensitivity
    P = ctypes.c_void_p
    for sc in (0.0, -0.5, float("nan")):
        assert f(P(FAKE), P(FAKE), 1, 64, 1, 2, 64, P(FAKE), 8, sc, P(FAKE), None) == kvq.KVQ_EINVAL


def test_append_rejects():
    L, K, V = _layout(window_cap=191), _store(), _store()
    ap = kvq.lib().kvq_append
    P = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(Lx=L, Vs=V, k=FAKE, v=FAKE, rope=None, rope_new=None, rope_dim=0, n=1, keep=128,
             nbo=FAKE, nwo=FAKE):
        return ap(ctypes.byref(Lx), ctypes.byref(K), None if Vs is None else ctypes.byref(Vs), P(k),
                  P(v), P(rope), P(rope_new), rope_dim, n, keep, P(nbo), P(nwo), None)
    assert call(n=-1) == kvq.KVQ_EINVAL
    assert call(keep=-1) == kvq.KVQ_EINVAL
    assert call(keep=129) == kvq.KVQ_EINVAL                  # keep + 63 > window_cap
    assert call(k=None) == kvq.KVQ_EINVAL
    assert call(v=None) == kvq.KVQ_EINVAL
    assert call(k=FAKE + 2) == kvq.KVQ_EINVAL
    assert call(nbo=None) == kvq.KVQ_EINVAL
    assert call(nwo=None) == kvq.KVQ_EINVAL
    assert call(nbo=FAKE + 2) == kvq.KVQ_EINVAL
    assert call(rope_dim=32, rope=FAKE, rope_new=FAKE) == kvq.KVQ_EUNSUPPORTED
    assert call(rope_dim=64) == kvq.KVQ_EINVAL                # no rope buffers
    assert call(rope_dim=64, rope=FAKE) == kvq.KVQ_EINVAL
    L0 = _layout(window_cap=0)
    assert call(Lx=L0, keep=0, n=5) == kvq.KVQ_EINVAL        # no window: whole blocks only
    assert call(Lx=L0, keep=1, n=64) == kvq.KVQ_EINVAL
    assert ap(None, ctypes.byref(K), ctypes.byref(V), P(FAKE), P(FAKE), None, None, 0, 1, 0, P(FAKE),
              P(FAKE), None) == kvq.KVQ_EINVAL
