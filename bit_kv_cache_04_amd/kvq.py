"""ctypes binding of libkvq (include/kvq.h): same names, argument marshalling only.

Every step of append and decode runs in the library's HIP kernels; torch is
used only to own device memory and to name the stream.  Loading fails loudly
when libkvq.so has not been built.
"""

import ctypes
import os

import numpy as np

# KVQ_LIBRARY names another build of the same library (e.g. a debug build).
_LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

# enum kv_format
FMT = {"bf16": 0, "kivi2": 1, "fp4": 2, "turbo": 3, "qjl1": 4, "latent": 5}
DT_F32, DT_BF16 = 0, 1
STATUS = {0: "KV_OK", -1: "KV_EINVAL", -2: "KV_ECAPACITY", -3: "KV_EUNSUPPORTED",
          -4: "KV_EWORKSPACE", -5: "KV_EDEVICE"}
BUFFERS = ["k_codes", "k_scale", "k_zero", "k_sketch", "k_norm", "k_rnorm",
           "v_codes", "v_scale", "v_zero", "v_norm", "rope", "sink_k", "sink_v", "recent_k", "recent_v",
           "k_stage"]
EXPORTED = ["kv_buffer_bytes", "kv_bytes_per_token", "kv_quant_append", "kv_quant_append_ragged", "kv_decode_attention",
            "kv_lloyd_max_gaussian", "kv_make_rotation", "kv_make_hadamard_rotation",
            "kv_make_projection", "kv_status_string", "kv_hsi_candidates", "kv_hsi_select",
            "kv_decode_attention_sparse", "kv_stream_read", "kv_decode_attention_static", "kv_mfma_probe",
            "kv_lds_probe"]


class KvError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


class KVLayout(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("group", ctypes.c_int32), ("qjl_m", ctypes.c_int32), ("lm_bits", ctypes.c_int32),
                ("sink_tokens", ctypes.c_int32), ("recent_tokens", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("rotation", ctypes.c_int32)]


# enum kv_rotation: how TURBO applies R (a dense matrix, or the Hadamard butterfly
# with or without the bit-reversal of the channels)
ROT_DENSE, ROT_HADAMARD_BITREV, ROT_HADAMARD = 0, 1, 2


class KVCache(ctypes.Structure):
    _fields_ = [("layout", KVLayout), ("buf", ctypes.c_void_p * len(BUFFERS)),
                ("rot", ctypes.c_void_p), ("proj", ctypes.c_void_p),
                ("lm_levels", ctypes.c_void_p), ("lm_thresh", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p)]


DECODE_FP32 = 1  # enum kv_decode_flags


class KVDecodeOpts(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("ev_begin", ctypes.c_void_p), ("ev_end", ctypes.c_void_p),
                ("num_queries", ctypes.c_int32), ("flags", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libkvq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libkvq.so not built at {_LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.kv_buffer_bytes.argtypes = [ctypes.POINTER(KVLayout), i32]
        L.kv_buffer_bytes.restype = sz
        L.kv_bytes_per_token.argtypes = [ctypes.POINTER(KVLayout), i32]
        L.kv_bytes_per_token.restype = sz
        L.kv_quant_append.argtypes = [ctypes.POINTER(KVCache), vp, vp, i32, i32, i32, vp,
                                      ctypes.POINTER(sz), vp]
        L.kv_quant_append.restype = ctypes.c_int
        L.kv_quant_append_ragged.argtypes = [ctypes.POINTER(KVCache), vp, vp, i32, ctypes.POINTER(i32), i32, vp,
                                             ctypes.POINTER(sz), vp]
        L.kv_quant_append_ragged.restype = ctypes.c_int
        L.kv_decode_attention.argtypes = [ctypes.POINTER(KVCache), vp, i32, i32, vp, i32, ctypes.c_float,
                                          vp, vp, ctypes.POINTER(sz), ctypes.POINTER(KVDecodeOpts), vp]
        L.kv_decode_attention.restype = ctypes.c_int
        L.kv_lloyd_max_gaussian.argtypes = [i32, i32, vp, vp]
        L.kv_lloyd_max_gaussian.restype = ctypes.c_int
        L.kv_make_rotation.argtypes = [vp, i32, vp]
        L.kv_make_rotation.restype = ctypes.c_int
        L.kv_make_hadamard_rotation.argtypes = [i32, i32, vp]
        L.kv_make_hadamard_rotation.restype = ctypes.c_int
        L.kv_make_projection.argtypes = [vp, i32, i32, vp]
        L.kv_make_projection.restype = ctypes.c_int
        L.kv_hsi_candidates.argtypes = [vp, i32, i32, vp, i32, i32, vp, vp, vp, ctypes.POINTER(sz), vp]
        L.kv_hsi_candidates.restype = ctypes.c_int
        L.kv_hsi_select.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp]
        L.kv_hsi_select.restype = ctypes.c_int
        L.kv_decode_attention_sparse.argtypes = [ctypes.POINTER(KVCache), vp, i32, i32, vp, vp, i32, ctypes.c_float,
                                                 vp, vp, ctypes.POINTER(sz), ctypes.POINTER(KVDecodeOpts), vp]
        L.kv_decode_attention_sparse.restype = ctypes.c_int
        L.kv_decode_attention_static.argtypes = [ctypes.POINTER(KVCache), vp, i32, i32, vp, i32, ctypes.c_float, vp,
                                                 ctypes.POINTER(KVDecodeOpts), vp]
        L.kv_decode_attention_static.restype = ctypes.c_int
        L.kv_stream_read.argtypes = [vp, sz, vp, vp]
        L.kv_stream_read.restype = ctypes.c_int
        L.kv_mfma_probe.argtypes = [i32, i32, vp, vp]
        L.kv_mfma_probe.restype = ctypes.c_int
        L.kv_lds_probe.argtypes = [i32, i32, vp, vp]
        L.kv_lds_probe.restype = ctypes.c_int
        L.kv_status_string.argtypes = [ctypes.c_int]
        L.kv_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_layout(fmt, batch, num_kv_heads, head_dim, capacity, rope_dim=0, sink=0, recent=0, page_tokens=0,
                num_pages=0, rotation=ROT_DENSE):
    """A kv_layout with the format's fixed group / sketch / codebook parameters
    (sink / recent: tokens kept bf16 at the start and end of each sequence;
    page_tokens / num_pages: paged storage in a pool of pages; rotation: the
    TURBO rotation's kind, enum kv_rotation)."""
    f = FMT[fmt] if isinstance(fmt, str) else int(fmt)
    group = {1: 32, 2: 16, 4: 16, 5: 16}.get(f, 0)
    qjl_m = 128 if f in (3, 4) else 0
    lm_bits = 2 if f == 3 else 0
    return KVLayout(f, batch, num_kv_heads, head_dim, rope_dim, capacity, group, qjl_m, lm_bits, sink, recent,
                    page_tokens, num_pages, rotation)


def _check(fn, st):
    if st != 0:
        raise KvError(fn, st)


# ---------------------------------------------------------------- same-name wrappers

def kv_buffer_bytes(layout: KVLayout, which: int) -> int:
    return lib().kv_buffer_bytes(ctypes.byref(layout), which)


def kv_bytes_per_token(layout: KVLayout, num_layers: int) -> int:
    return lib().kv_bytes_per_token(ctypes.byref(layout), num_layers)


def kv_quant_append(cache: KVCache, k_ptr, v_ptr, in_dtype, start, n_new, stream=0):
    nbytes = ctypes.c_size_t(0)
    st = lib().kv_quant_append(ctypes.byref(cache), k_ptr, v_ptr, in_dtype, start, n_new, None,
                               ctypes.byref(nbytes), stream)
    _check("kv_quant_append", st)


def kv_quant_append_ragged(cache: KVCache, k_ptr, v_ptr, in_dtype, starts, n_new, stream=0):
    """starts: one first position per sequence (host ints)."""
    arr = (ctypes.c_int32 * len(starts))(*[int(s) for s in starts])
    nbytes = ctypes.c_size_t(0)
    st = lib().kv_quant_append_ragged(ctypes.byref(cache), k_ptr, v_ptr, in_dtype, arr, n_new, None,
                                      ctypes.byref(nbytes), stream)
    _check("kv_quant_append_ragged", st)


def kv_decode_attention(cache: KVCache, q_ptr, q_dtype, num_q_heads, seq_lens_ptr, max_seq_len, scale,
                        out_ptr, ws_ptr, ws_bytes, opts=None, stream=0):
    """ws_ptr None: returns the workspace size; else runs and returns ws_bytes."""
    nbytes = ctypes.c_size_t(ws_bytes or 0)
    st = lib().kv_decode_attention(ctypes.byref(cache), q_ptr, q_dtype, num_q_heads, seq_lens_ptr,
                                   max_seq_len, ctypes.c_float(scale), out_ptr, ws_ptr, ctypes.byref(nbytes),
                                   ctypes.byref(opts) if opts is not None else None, stream)
    _check("kv_decode_attention", st)
    return nbytes.value


def kv_lloyd_max_gaussian(bits: int, dim: int):
    lv = np.zeros(1 << bits, np.float32)
    th = np.zeros((1 << bits) - 1, np.float32)
    _check("kv_lloyd_max_gaussian", lib().kv_lloyd_max_gaussian(bits, dim, lv.ctypes.data, th.ctypes.data))
    return lv, th


def kv_make_rotation(gauss) -> np.ndarray:
    g = np.ascontiguousarray(gauss, dtype=np.float64)
    d = g.shape[0]
    out = np.zeros((d, d), np.float32)
    _check("kv_make_rotation", lib().kv_make_rotation(g.ctypes.data, d, out.ctypes.data))
    return out


def kv_make_hadamard_rotation(d: int, bit_reverse: bool = True) -> np.ndarray:
    out = np.zeros((d, d), np.float32)
    _check("kv_make_hadamard_rotation", lib().kv_make_hadamard_rotation(d, int(bool(bit_reverse)), out.ctypes.data))
    return out


def kv_make_projection(gauss) -> np.ndarray:
    g = np.ascontiguousarray(gauss, dtype=np.float64)
    m, d = g.shape
    out = np.zeros((m, d), np.float32)
    _check("kv_make_projection", lib().kv_make_projection(g.ctypes.data, m, d, out.ctypes.data))
    return out


def kv_hsi_candidates(scores_ptr, batch, score_stride, seq_lens_ptr, block, top_blocks, pool_ptr, pool_n_ptr,
                      ws_ptr, ws_bytes, stream=0):
    """ws_ptr None: returns the workspace size; else runs."""
    nbytes = ctypes.c_size_t(ws_bytes or 0)
    _check("kv_hsi_candidates", lib().kv_hsi_candidates(scores_ptr, batch, score_stride, seq_lens_ptr, block,
                                                        top_blocks, pool_ptr, pool_n_ptr, ws_ptr,
                                                        ctypes.byref(nbytes), stream))
    return nbytes.value


def kv_hsi_select(pool_scores_ptr, pool_ptr, pool_n_ptr, batch, pool_cap, top_k, sel_ptr, sel_n_ptr, stream=0):
    _check("kv_hsi_select", lib().kv_hsi_select(pool_scores_ptr, pool_ptr, pool_n_ptr, batch, pool_cap, top_k,
                                                sel_ptr, sel_n_ptr, stream))


def kv_decode_attention_sparse(cache: KVCache, q_ptr, q_dtype, num_q_heads, sel_ptr, sel_n_ptr, sel_cap, scale,
                               out_ptr, ws_ptr, ws_bytes, opts=None, stream=0):
    """ws_ptr None: returns the workspace size; else runs and returns ws_bytes."""
    nbytes = ctypes.c_size_t(ws_bytes or 0)
    st = lib().kv_decode_attention_sparse(ctypes.byref(cache), q_ptr, q_dtype, num_q_heads, sel_ptr, sel_n_ptr,
                                          sel_cap, ctypes.c_float(scale), out_ptr, ws_ptr, ctypes.byref(nbytes),
                                          ctypes.byref(opts) if opts is not None else None, stream)
    _check("kv_decode_attention_sparse", st)
    return nbytes.value


def kv_status_string(status: int) -> str:
    return lib().kv_status_string(status).decode()


def kv_stream_read(src_ptr, nbytes, sink_ptr, stream=0):
    """The streaming-read reference kernel (kvq_probe.h)."""
    _check("kv_stream_read", lib().kv_stream_read(src_ptr, nbytes, sink_ptr, stream))


def kv_mfma_probe(blocks, iters, sink_ptr, stream=0):
    """The matrix-core reference kernel (kvq_probe.h): blocks * 4 * iters * 8 products of 32 x 32 x 16."""
    _check("kv_mfma_probe", lib().kv_mfma_probe(blocks, iters, sink_ptr, stream))


def kv_lds_probe(blocks, iters, sink_ptr, stream=0):
    """The LDS read reference kernel (kvq_probe.h): blocks * 4 * iters * 8 KiB read from LDS."""
    _check("kv_lds_probe", lib().kv_lds_probe(blocks, iters, sink_ptr, stream))


def kv_decode_attention_static(cache: KVCache, q_ptr, q_dtype, num_q_heads, seq_lens_ptr, max_seq_len, scale,
                               out_ptr, opts=None, stream=0):
    """kv_decode_attention on the library's own device workspace (allocates nothing)."""
    st = lib().kv_decode_attention_static(ctypes.byref(cache), q_ptr, q_dtype, num_q_heads, seq_lens_ptr,
                                          max_seq_len, ctypes.c_float(scale), out_ptr,
                                          ctypes.byref(opts) if opts is not None else None, stream)
    _check("kv_decode_attention_static", st)
