"""C-ABI checks that need no GPU: the library loads and exports every declared
symbol, the host arithmetic (sizes, bytes per token, constants) agrees with the
oracle and the pages, and every validation error is returned before any launch.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from bit_kv_cache_04_amd import kvq
from oracle.bytes import per_token_head
from oracle.lloyd_max import canonical_codebook
from oracle.numerics import round_bf16
from oracle.rotation import canonical_hadamard_rotation, canonical_rotation

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

OK, EINVAL, ECAP, EUNSUP, EWS = 0, -1, -2, -3, -4


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(kv_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(kvq.EXPORTED), names
    L = kvq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_bytes_per_token_bf16_pages(golden):
    for layers, heads, d, tokens, want, _ in golden("bytes_per_token.txt"):
        lay = kvq.make_layout("bf16", 1, int(heads), int(d), 1)
        assert kvq.kv_bytes_per_token(lay, int(layers)) * int(tokens) == int(want)


@pytest.mark.parametrize("fmt,H,d,rope", [("fp4", 8, 128, 0), ("fp4", 4, 64, 0), ("kivi2", 2, 64, 0),
                                          ("kivi2", 8, 128, 0), ("turbo", 8, 128, 0), ("qjl1", 8, 128, 0),
                                          ("latent", 1, 512, 64)])
def test_bytes_per_token_matches_oracle(fmt, H, d, rope):
    lay = kvq.make_layout(fmt, 3, H, d, 96, rope)
    for layers in (1, 40, 80):
        assert kvq.kv_bytes_per_token(lay, layers) == layers * H * per_token_head(fmt, d, rope)
    # the per-token buffers (the bf16 windows and KIVI staging are per sequence)
    total = sum(kvq.kv_buffer_bytes(lay, i) for i in range(kvq.BUFFERS.index("sink_k")))
    assert total == 3 * H * 96 * per_token_head(fmt, d, rope)


def test_bytes_per_token_invalid():
    assert kvq.kv_bytes_per_token(kvq.make_layout("fp4", 1, 8, 96, 16), 1) == 0   # unsupported d
    assert kvq.kv_bytes_per_token(kvq.make_layout("fp4", 1, 8, 128, 16), 0) == 0  # no layers


def test_codebook_matches_oracle():
    for d in (64, 128):
        lv, th = kvq.kv_lloyd_max_gaussian(2, d)
        olv, oth = canonical_codebook(2, d)
        np.testing.assert_array_equal(lv.astype(np.float64), olv)
        np.testing.assert_array_equal(th.astype(np.float64), oth)
    for b in (1, 3, 4):
        lv, th = kvq.kv_lloyd_max_gaussian(b, 128)
        olv, oth = canonical_codebook(b, 128)
        np.testing.assert_allclose(lv, olv, rtol=2 ** -23)
        np.testing.assert_allclose(th, oth, rtol=2 ** -23, atol=1e-30)
    assert kvq.lib().kv_lloyd_max_gaussian(0, 128, None, None) == EINVAL


@pytest.mark.parametrize("seed,d", [(0, 128), (1, 128), (2, 64), (3, 16)])
def test_rotation_and_projection_match_oracle(seed, d):
    g = np.random.default_rng(seed).standard_normal((d, d))
    np.testing.assert_array_equal(kvq.kv_make_rotation(g).astype(np.float64), canonical_rotation(g))
    p = np.random.default_rng(seed + 100).standard_normal((128, d))
    np.testing.assert_array_equal(kvq.kv_make_projection(p).astype(np.float64), round_bf16(p))


@pytest.mark.parametrize("d", [1, 2, 16, 64, 128, 512])
def test_hadamard_rotation_matches_oracle(d):
    for rev in (True, False):
        np.testing.assert_array_equal(kvq.kv_make_hadamard_rotation(d, rev).astype(np.float64),
                                      canonical_hadamard_rotation(d, rev))


def test_hadamard_rotation_invalid():
    out = np.zeros(96 * 96, np.float32)
    for d in (0, -4, 96, 2048):
        assert kvq.lib().kv_make_hadamard_rotation(d, 1, out.ctypes.data) == EINVAL
    assert kvq.lib().kv_make_hadamard_rotation(8, 1, None) == EINVAL


def test_rotation_rank_deficient():
    g = np.zeros((8, 8))
    out = np.zeros((8, 8), np.float32)
    assert kvq.lib().kv_make_rotation(g.ctypes.data, 8, out.ctypes.data) == EINVAL


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert kvq.kv_status_string(s) != "unknown status"
    assert kvq.kv_status_string(7) == "unknown status"


# ---------------------------------------------------------------- validation (no launch)

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _cache(fmt="fp4", B=2, H=2, d=128, T=64, rope=0, fill=True, consts=True, recent=0):
    lay = kvq.make_layout(fmt, B, H, d, T, rope, recent=recent)
    bufs = (ctypes.c_void_p * len(kvq.BUFFERS))(
        *[(FAKE if fill and kvq.kv_buffer_bytes(lay, i) else None) for i in range(len(kvq.BUFFERS))])
    c = FAKE if consts else None
    return kvq.KVCache(lay, bufs, c, c, c, c)


def _append(c, k=FAKE, v=FAKE, dt=kvq.DT_BF16, start=0, n=1):
    nb = ctypes.c_size_t(99)
    return kvq.lib().kv_quant_append(ctypes.byref(c), k, v, dt, start, n, None, ctypes.byref(nb), None)


def _decode(c, q=FAKE, qdt=kvq.DT_BF16, hq=4, lens=FAKE, maxlen=64, scale=1.0, out=FAKE, ws=None,
            wsb=0, splits=0, nq=0, flags=0):
    nb = ctypes.c_size_t(wsb)
    opts = kvq.KVDecodeOpts(splits, None, None, nq, flags)
    st = kvq.lib().kv_decode_attention(ctypes.byref(c), q, qdt, hq, lens, maxlen, ctypes.c_float(scale), out,
                                       ws, ctypes.byref(nb), ctypes.byref(opts), None)
    return st, nb.value


def test_append_validation():
    assert _append(_cache(), start=60, n=5) == ECAP
    assert _append(_cache(), start=-1) == EINVAL
    assert _append(_cache(), dt=7) == EUNSUP
    assert _append(_cache(), k=None) == EINVAL
    assert _append(_cache(), v=None) == EINVAL
    assert _append(_cache(), k=FAKE + 2) == EINVAL                     # misaligned input
    assert _append(_cache(fill=False)) == EINVAL                      # NULL buffers
    assert _append(_cache("kivi2", d=64), start=40, n=25) == ECAP      # partial KIVI groups are fine, capacity is not
    assert _append(_cache("latent", H=1, d=512, rope=64)) == EINVAL   # latent takes no v
    assert _append(_cache("turbo", consts=False)) == EINVAL           # constants missing
    c = _cache("qjl1")
    c.proj = FAKE + 8
    assert _append(c) == EINVAL                                       # misaligned projection
    assert _append(_cache("fp4", d=96)) == EUNSUP
    assert _append(_cache("fp4", B=0)) == EINVAL
    assert _append(_cache(), n=0) == OK                               # nothing to do, nothing launched


def test_decode_validation_and_size_query():
    c = _cache()
    st, nb = _decode(c, ws=None)
    assert st == OK and nb > 0 and nb % 256 == 0
    st, nb2 = _decode(c, ws=None, splits=3)
    assert st == OK and nb2 >= nb or nb2 > 0
    assert _decode(c, ws=FAKE, wsb=nb - 1)[0] == EWS
    assert _decode(c, ws=FAKE + 16, wsb=nb)[0] == EINVAL                # workspace misaligned
    assert _decode(c, hq=3)[0] == EINVAL                               # not a multiple of H
    assert _decode(c, maxlen=65)[0] == EINVAL                          # beyond capacity
    assert _decode(c, maxlen=0)[0] == EINVAL
    assert _decode(c, qdt=5)[0] == EUNSUP
    assert _decode(c, scale=float("nan"))[0] == EINVAL
    assert _decode(c, splits=-1)[0] == EINVAL
    assert _decode(c, ws=FAKE, wsb=nb, q=None)[0] == EINVAL
    assert _decode(c, ws=FAKE, wsb=nb, out=None)[0] == EINVAL
    assert _decode(c, ws=FAKE, wsb=nb, lens=None)[0] == EINVAL
    assert _decode(_cache("bf16"))[0] == EUNSUP


def test_decode_num_queries_validation_and_size():
    c = _cache()
    _, nb1 = _decode(c, ws=None, splits=4)
    st, nb5 = _decode(c, ws=None, splits=4, nq=5)
    assert st == OK and nb5 > nb1                                     # five rows of partials per head
    assert _decode(c, ws=None, splits=4, nq=1)[1] == nb1              # 1 and 0 both mean one query
    assert _decode(c, nq=-1)[0] == EINVAL
    assert _decode(c, nq=65, maxlen=64)[0] == EINVAL                  # more queries than tokens
    assert _decode(_cache(T=128), nq=65, maxlen=128)[0] == EUNSUP     # beyond 64 queries


def test_mixed_precision_layout_validation_and_sizes():
    lay = kvq.make_layout("fp4", 2, 4, 128, 256, sink=8, recent=32)
    assert kvq.kv_buffer_bytes(lay, kvq.BUFFERS.index("sink_k")) == 2 * 4 * 8 * 128 * 2
    assert kvq.kv_buffer_bytes(lay, kvq.BUFFERS.index("recent_v")) == 2 * 4 * 32 * 128 * 2
    # the windows are a fixed cost per sequence, not counted per token
    assert kvq.kv_bytes_per_token(lay, 1) == kvq.kv_bytes_per_token(kvq.make_layout("fp4", 2, 4, 128, 256), 1)
    assert kvq.kv_buffer_bytes(kvq.make_layout("fp4", 2, 4, 128, 256), kvq.BUFFERS.index("sink_k")) == 0
    # every per-head format takes windows, the shared latent cache none; sizes within the capacity
    for fmt in ("kivi2", "turbo", "qjl1"):
        lay = kvq.make_layout(fmt, 1, 1, 128, 64, sink=4, recent=8)
        assert kvq.kv_buffer_bytes(lay, kvq.BUFFERS.index("recent_k")) == 8 * 128 * 2
    assert kvq.kv_buffer_bytes(kvq.make_layout("latent", 1, 1, 512, 64, rope_dim=64, sink=4), 0) == 0
    assert kvq.kv_buffer_bytes(kvq.make_layout("fp4", 1, 1, 128, 64, recent=65), 0) == 0
    assert kvq.kv_buffer_bytes(kvq.make_layout("fp4", 1, 1, 128, 64, sink=-1), 0) == 0
    c = _cache("latent", d=512, rope=64)
    c.layout.sink_tokens = 4
    assert _append(c) == EUNSUP
    for fmt in ("kivi2", "turbo"):
        c = _cache(fmt, recent=16)
        c.layout.sink_tokens = 0
        st, nb_win = _decode(c, ws=None, splits=4)
        assert st == OK and nb_win > _decode(_cache(fmt), ws=None, splits=4)[1]
    c = _cache()
    c.layout.recent_tokens = 16
    assert _append(c) == EINVAL                                        # window buffers missing
    c = _cache()
    c.layout.sink_tokens = 4
    c.layout.recent_tokens = 16
    c.buf[kvq.BUFFERS.index("sink_k")] = FAKE
    c.buf[kvq.BUFFERS.index("sink_v")] = FAKE
    c.buf[kvq.BUFFERS.index("recent_k")] = FAKE
    c.buf[kvq.BUFFERS.index("recent_v")] = FAKE
    st, nb_win = _decode(c, ws=None, splits=4)
    assert st == OK and nb_win > _decode(_cache(), ws=None, splits=4)[1]   # one more split of partials


def _append_ragged(c, starts, k=FAKE, v=FAKE, dt=kvq.DT_BF16, n=1):
    arr = None if starts is None else (ctypes.c_int32 * len(starts))(*starts)
    nb = ctypes.c_size_t(99)
    return kvq.lib().kv_quant_append_ragged(ctypes.byref(c), k, v, dt, arr, n, None, ctypes.byref(nb), None)


def test_ragged_append_validation():
    c = _cache(B=2, T=64)
    assert _append_ragged(c, None) == EINVAL
    assert _append_ragged(c, [0, -1]) == EINVAL
    assert _append_ragged(c, [0, 60], n=5) == ECAP
    assert _append_ragged(c, [0, 59], n=5, k=None) == EINVAL          # checks pass, then the NULL input
    assert _append_ragged(c, [3, 7], n=0) == OK                        # nothing to do, nothing launched
    k2 = _cache("kivi2", B=2, d=64, T=64)
    assert _append_ragged(k2, [0, 50], n=16) == ECAP                  # a partial KIVI group is fine, capacity is not
    # the staging buffer of a KIVI cache holds one 32-token key group per sequence-head
    lay = kvq.make_layout("kivi2", 2, 2, 64, 64)
    assert kvq.kv_buffer_bytes(lay, kvq.BUFFERS.index("k_stage")) == 2 * 2 * (4 + 32 * 64) * 4
    assert kvq.kv_buffer_bytes(kvq.make_layout("fp4", 2, 2, 64, 64), kvq.BUFFERS.index("k_stage")) == 0
    assert _append_ragged(_cache("fp4", d=96), [0, 0]) == EUNSUP


def test_paged_layout_validation_and_sizes():
    ok = kvq.make_layout("fp4", 4, 2, 128, 1024, page_tokens=64, num_pages=70)
    assert kvq.kv_buffer_bytes(ok, 0) == 70 * 2 * 64 * 64          # K_CODES: pages x H x P x d/2
    assert kvq.kv_buffer_bytes(ok, 1) == 70 * 2 * 64 * 8 * 2       # K_SCALE bf16 per 16 channels
    contiguous = kvq.make_layout("fp4", 4, 2, 128, 1024)
    assert kvq.kv_bytes_per_token(ok, 1) == kvq.kv_bytes_per_token(contiguous, 1)
    kl = kvq.make_layout("kivi2", 2, 2, 64, 256, page_tokens=64, num_pages=9)
    assert kvq.kv_buffer_bytes(kl, 1) == 9 * 2 * 2 * 64 * 4       # K_SCALE: P/32 rows a page
    assert kvq.kv_buffer_bytes(kl, 15) == 2 * 2 * (4 + 32 * 64) * 4  # K_STAGE stays per sequence
    ll = kvq.make_layout("latent", 3, 1, 512, 128, 64, page_tokens=32, num_pages=5)
    assert kvq.kv_buffer_bytes(ll, 0) == 5 * 32 * 256 and kvq.kv_buffer_bytes(ll, 10) == 5 * 32 * 64 * 2
    wl = kvq.make_layout("fp4", 4, 2, 128, 1024, sink=40, recent=100, page_tokens=64, num_pages=70)
    assert kvq.kv_buffer_bytes(wl, 11) == 4 * 2 * 40 * 128 * 2    # SINK_K per sequence
    for P, n in ((48, 10), (64, 0), (0, 5), (-32, 4), (96, 10), (64, -1), (16, 80), (192, 10)):
        bad = kvq.make_layout("fp4", 4, 2, 128, 1024, page_tokens=P, num_pages=n)
        assert kvq.kv_buffer_bytes(bad, 0) == 0, (P, n)
    # a paged cache needs its block table; calls fail before any launch
    lay = kvq.make_layout("fp4", 2, 2, 128, 128, page_tokens=64, num_pages=4)
    bufs = (ctypes.c_void_p * len(kvq.BUFFERS))(
        *[(FAKE if kvq.kv_buffer_bytes(lay, i) else None) for i in range(len(kvq.BUFFERS))])
    c = kvq.KVCache(lay, bufs, None, None, None, None, None)
    assert _append(c) == EINVAL
    assert _decode(c, hq=4, maxlen=128, ws=FAKE, wsb=1 << 30)[0] == EINVAL
    c.block_table = FAKE
    assert _append(c, start=100, n=29) == ECAP                      # capacity stays per sequence


def test_hsi_validation_and_sizes():
    L = kvq.lib()
    nb = ctypes.c_size_t(0)
    assert L.kv_hsi_candidates(None, 3, 1000, None, 8, 2048, None, None, None, ctypes.byref(nb), None) == OK
    assert nb.value == 3 * 125 * 4
    assert L.kv_hsi_candidates(None, 1, 1001, None, 8, 16, None, None, None, ctypes.byref(nb), None) == OK
    assert nb.value == 126 * 4
    for args in ((0, 100, 8, 4), (2, 0, 8, 4), (2, 100, 0, 4), (2, 100, 65, 4), (2, 100, 8, 0)):
        B, S, blk, top = args
        assert L.kv_hsi_candidates(None, B, S, None, blk, top, None, None, None, ctypes.byref(nb), None) == EINVAL
    small = ctypes.c_size_t(8)
    assert L.kv_hsi_candidates(FAKE, 3, 1000, FAKE, 8, 16, FAKE, FAKE, FAKE, ctypes.byref(small), None) == EWS
    assert L.kv_hsi_select(FAKE, FAKE, FAKE, 0, 100, 8, FAKE, FAKE, None) == EINVAL
    assert L.kv_hsi_select(FAKE, FAKE, FAKE, 2, 100, 0, FAKE, FAKE, None) == EINVAL
    assert L.kv_hsi_select(None, FAKE, FAKE, 2, 100, 8, FAKE, FAKE, None) == EINVAL


def test_sparse_decode_validation_and_size():
    def sparse(c, sel=FAKE, seln=FAKE, cap=512, ws=None, wsb=0, nq=0):
        nb = ctypes.c_size_t(wsb)
        opts = kvq.KVDecodeOpts(0, None, None, nq)
        st = kvq.lib().kv_decode_attention_sparse(ctypes.byref(c), FAKE, kvq.DT_BF16, 4, sel, seln, cap,
                                                  ctypes.c_float(1.0), FAKE, ws, ctypes.byref(nb),
                                                  ctypes.byref(opts), None)
        return st, nb.value
    st, need = sparse(_cache(T=1024))
    assert st == OK and need > 0
    assert sparse(_cache(T=1024), cap=0)[0] == EINVAL
    assert sparse(_cache(T=1024), nq=2)[0] == EUNSUP
    assert sparse(_cache(T=1024), ws=FAKE, wsb=need - 1)[0] == EWS
    assert sparse(_cache(T=1024), sel=None, ws=FAKE, wsb=need)[0] == EINVAL
    lay = kvq.make_layout("fp4", 2, 2, 128, 256, sink=16, recent=16)
    bufs = (ctypes.c_void_p * len(kvq.BUFFERS))(
        *[(FAKE if kvq.kv_buffer_bytes(lay, i) else None) for i in range(len(kvq.BUFFERS))])
    assert sparse(kvq.KVCache(lay, bufs, None, None, None, None, None))[0] == EUNSUP


def test_stream_read_validation():
    L = kvq.lib()
    assert L.kv_stream_read(None, 1024, FAKE, None) == EINVAL
    assert L.kv_stream_read(FAKE, 1024, None, None) == EINVAL
    assert L.kv_stream_read(FAKE + 8, 1024, FAKE, None) == EINVAL       # misaligned
    assert L.kv_stream_read(FAKE, 1000, FAKE, None) == EINVAL           # not whole 16-byte words
    assert L.kv_stream_read(FAKE, 0, FAKE, None) == EINVAL


def test_rotation_kind_validation():
    # a structured rotation is TURBO's alone, and lets the cache go without a matrix
    assert kvq.kv_bytes_per_token(kvq.make_layout("turbo", 1, 8, 128, 64, rotation=kvq.ROT_HADAMARD_BITREV), 1) > 0
    assert kvq.kv_bytes_per_token(kvq.make_layout("turbo", 1, 8, 128, 64, rotation=3), 1) == 0
    assert kvq.kv_bytes_per_token(kvq.make_layout("turbo", 1, 8, 128, 64, rotation=-1), 1) == 0
    assert kvq.kv_bytes_per_token(kvq.make_layout("fp4", 1, 8, 128, 64, rotation=kvq.ROT_HADAMARD), 1) == 0
    L = kvq.lib()
    for kind, ok in ((kvq.ROT_DENSE, False), (kvq.ROT_HADAMARD_BITREV, True), (kvq.ROT_HADAMARD, True)):
        lay = kvq.make_layout("turbo", 1, 1, 128, 64, rotation=kind)
        bufs = (ctypes.c_void_p * len(kvq.BUFFERS))(
            *[(FAKE if kvq.kv_buffer_bytes(lay, i) else None) for i in range(len(kvq.BUFFERS))])
        cache = kvq.KVCache(lay, bufs, None, FAKE, FAKE, FAKE, None)   # no rotation matrix
        need = ctypes.c_size_t(0)
        st = L.kv_decode_attention(ctypes.byref(cache), FAKE, 0, 8, FAKE, 64, ctypes.c_float(0.1), FAKE, None,
                                   ctypes.byref(need), None, None)
        assert (st == 0) == ok, (kind, st)


def test_compute_probe_validation():
    L = kvq.lib()
    for fn in (L.kv_mfma_probe, L.kv_lds_probe):
        assert fn(0, 16, FAKE, None) == EINVAL          # no workgroups
        assert fn(65536, 16, FAKE, None) == EINVAL      # past the grid limit
        assert fn(4, 0, FAKE, None) == EINVAL           # no iterations
        assert fn(4, (1 << 20) + 1, FAKE, None) == EINVAL
        assert fn(4, 16, None, None) == EINVAL          # no sink


def test_decode_split_cap_with_windows():
    # the merge holds at most 1024 partial rows per query: the packed splits
    # yield to the window's 64-position splits, and a window of 1024 such
    # splits or more is refused
    T = 1 << 17
    _, nb_plain = _decode(_cache("fp4", T=T), ws=None, splits=1024, maxlen=T)
    st, nb_win = _decode(_cache("fp4", T=T, recent=64 * 8), ws=None, splits=1024, maxlen=T)
    assert st == OK and nb_win <= nb_plain                            # at most 1016 packed + 8 window splits
    assert _decode(_cache("fp4", T=T, recent=64 * 1024), ws=None, maxlen=T)[0] == EUNSUP
    assert _decode(_cache("fp4", T=T, recent=64 * 1023), ws=None, maxlen=T)[0] == OK


def test_decode_flags_validation():
    c = _cache()
    assert _decode(c, ws=None, flags=kvq.DECODE_FP32)[0] == OK
    assert _decode(c, flags=2)[0] == EINVAL                            # unknown flag bits
    assert _decode(c, flags=-1)[0] == EINVAL


def test_static_decode_validation_before_any_gpu_call():
    # the size and argument checks come before the workspace lookup: no GPU needed
    L = kvq.lib()
    c = _cache("latent", B=64, H=1, d=512, T=1 << 16, rope=64)
    opts = kvq.KVDecodeOpts(0, None, None, 4, 0)                     # four queries: 4x the partial rows
    st = L.kv_decode_attention_static(ctypes.byref(c), FAKE, kvq.DT_BF16, 128, FAKE, 1 << 16, ctypes.c_float(1.0),
                                      FAKE, ctypes.byref(opts), None)
    assert st == EWS                                                  # beyond the 128 MiB array
    c = _cache()
    assert L.kv_decode_attention_static(ctypes.byref(c), None, kvq.DT_BF16, 4, FAKE, 64, ctypes.c_float(1.0),
                                        FAKE, None, None) == EINVAL
    assert L.kv_decode_attention_static(ctypes.byref(c), FAKE, kvq.DT_BF16, 3, FAKE, 64, ctypes.c_float(1.0),
                                        FAKE, None, None) == EINVAL
