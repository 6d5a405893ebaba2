"""A packed KV cache held in torch device memory, driven through the C ABI.

torch owns the buffers, the constants and the workspace; every quantisation
and attention step runs in libkvq's kernels via the same-name wrappers of
`kvq`.  Nothing here computes on the data.
"""

import ctypes

import numpy as np
import torch

from . import kvq
from .kvq import BUFFERS, DT_BF16, DT_F32, FMT, KVCache, KVDecodeOpts, make_layout

_TORCH_DT = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream_ptr(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def buffer_view_spec(fmt, B, H, T, d, rope=0, m=128, sink=0, recent=0, page_tokens=0, num_pages=0):
    """{name: (torch dtype, shape)} of each buffer's natural element view (paged
    storage: the per-token buffers as [num_pages][H][page_tokens] pools)."""
    u16 = torch.uint16
    win = {}
    if page_tokens:
        spec = _packed_view_spec(fmt, num_pages, H, page_tokens, d, rope, m)
        if "k_stage" in spec:
            spec["k_stage"] = (torch.float32, (B, H, 4 + 32 * d))
    else:
        spec = _packed_view_spec(fmt, B, H, T, d, rope, m)
    if sink:
        win.update(sink_k=(u16, (B, H, sink, d)), sink_v=(u16, (B, H, sink, d)))
    if recent:
        win.update(recent_k=(u16, (B, H, recent, d)), recent_v=(u16, (B, H, recent, d)))
    return {**spec, **win}


def _packed_view_spec(fmt, B, H, T, d, rope, m):
    u8, u16, f32 = torch.uint8, torch.uint16, torch.float32
    if fmt == "kivi2":
        return dict(k_codes=(u8, (B, H, T, d // 4)), k_scale=(f32, (B, H, T // 32, d)),
                    k_zero=(f32, (B, H, T // 32, d)), v_codes=(u8, (B, H, T, d // 4)),
                    v_scale=(f32, (B, H, T, d // 32)), v_zero=(f32, (B, H, T, d // 32)),
                    k_stage=(f32, (B, H, 4 + 32 * d)))
    if fmt == "fp4":
        return dict(k_codes=(u8, (B, H, T, d // 2)), k_scale=(u16, (B, H, T, d // 16)),
                    v_codes=(u8, (B, H, T, d // 2)), v_scale=(u16, (B, H, T, d // 16)))
    if fmt == "turbo":
        return dict(k_codes=(u8, (B, H, T, d // 4)), k_sketch=(u8, (B, H, T, m // 8)),
                    k_norm=(u16, (B, H, T)), k_rnorm=(u16, (B, H, T)),
                    v_codes=(u8, (B, H, T, d // 4)), v_norm=(u16, (B, H, T)))
    if fmt == "qjl1":
        return dict(k_sketch=(u8, (B, H, T, m // 8)), k_norm=(u16, (B, H, T)),
                    v_codes=(u8, (B, H, T, d // 2)), v_scale=(u16, (B, H, T, d // 16)))
    if fmt == "latent":
        return dict(k_codes=(u8, (B, T, d // 2)), k_scale=(u16, (B, T, d // 16)), rope=(u16, (B, T, rope)))
    raise ValueError(fmt)


def make_constants(fmt, head_dim, rot_gauss=None, proj_gauss=None, rotation="haar"):
    """The method's constants from caller-drawn Gaussians, made by libkvq's host helpers
    (rotation: "haar" from rot_gauss, or "hadamard" / "hadamard_plain", the structured
    rotation with and without the bit-reversal permutation, which needs no draws)."""
    out = {}
    if fmt == "turbo":
        if rotation == "haar":
            out["rot"] = kvq.kv_make_rotation(rot_gauss)
        elif rotation in ("hadamard", "hadamard_plain"):
            out["rot"] = kvq.kv_make_hadamard_rotation(head_dim, rotation == "hadamard")
        else:
            raise ValueError(rotation)
        out["levels"], out["thresholds"] = kvq.kv_lloyd_max_gaussian(2, head_dim)
    if fmt in ("turbo", "qjl1"):
        out["proj"] = kvq.kv_make_projection(proj_gauss)
    return out


def hsi_candidates(scores, seq_lens, block=8, top_blocks=2048, out=None, ws=None):
    """HSI full mode through libkvq: scores fp32 [B, S] and seq_lens int32 [B] on
    the device; returns (pool int32 [B, top_blocks * block], pool_n int32 [B])."""
    B, S = scores.shape
    dev = scores.device
    need = kvq.kv_hsi_candidates(None, B, S, None, block, top_blocks, None, None, None, 0)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    pool, pool_n = out if out is not None else (
        torch.empty(B, top_blocks * block, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
    kvq.kv_hsi_candidates(_ptr(scores), B, S, _ptr(seq_lens), block, top_blocks, _ptr(pool), _ptr(pool_n), _ptr(ws),
                          ws.numel(), _stream_ptr(dev))
    return pool, pool_n


def hsi_select(pool_scores, pool, pool_n, top_k=512, out=None):
    """HSI reindex mode through libkvq: pool_scores fp32 [B, pool_cap] (entry i's
    score), pool / pool_n as hsi_candidates returns them; returns (sel int32
    [B, top_k] positions ascending, sel_n int32 [B])."""
    B, cap = pool_scores.shape
    dev = pool_scores.device
    sel, sel_n = out if out is not None else (
        torch.empty(B, top_k, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
    kvq.kv_hsi_select(_ptr(pool_scores), _ptr(pool), _ptr(pool_n), B, cap, top_k, _ptr(sel), _ptr(sel_n),
                      _stream_ptr(dev))
    return sel, sel_n


class PackedKVCache:
    def __init__(self, fmt, batch, num_kv_heads, head_dim, capacity, rope_dim=0, device="cuda",
                 constants=None, sink_tokens=0, recent_tokens=0, page_tokens=0, num_pages=0, block_table=None,
                 rotation=0):
        """Paged storage: page_tokens > 0, a pool of num_pages pages, and block_table
        int [batch][capacity // page_tokens] naming each sequence's pages (default:
        sequence b's page j is pool page b * capacity // page_tokens + j).  rotation:
        TURBO's kind of R (kvq.ROT_*); with a Hadamard kind the constants need no "rot"."""
        self.fmt, self.device = fmt, torch.device(device)
        self.B, self.H, self.d, self.T, self.rope = batch, num_kv_heads, head_dim, capacity, rope_dim
        self.sink, self.recent = sink_tokens, recent_tokens
        self.P, self.num_pages = page_tokens, num_pages
        self.rotation = rotation
        self.table = None
        if page_tokens:
            per_seq = capacity // page_tokens
            if block_table is None:
                block_table = np.arange(batch * per_seq, dtype=np.int32).reshape(batch, per_seq)
            self.table = torch.as_tensor(np.ascontiguousarray(block_table, dtype=np.int32)).to(self.device)
        self.layout = make_layout(fmt, batch, num_kv_heads, head_dim, capacity, rope_dim, sink_tokens,
                                  recent_tokens, page_tokens, num_pages, rotation)
        self.bufs = {}
        ptrs = []
        for i, name in enumerate(BUFFERS):
            nb = kvq.kv_buffer_bytes(self.layout, i)
            if nb:
                self.bufs[name] = torch.zeros(nb, dtype=torch.uint8, device=self.device)
            ptrs.append(self.bufs[name].data_ptr() if nb else None)
        if not self.bufs:
            raise kvq.KvError("kv_buffer_bytes", -3)
        self.consts = {}
        for k, v in (constants or {}).items():
            self.consts[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(self.device)
        cp = lambda k: self.consts[k].data_ptr() if k in self.consts else None  # noqa: E731
        self.struct = KVCache(self.layout, (ctypes.c_void_p * len(BUFFERS))(*ptrs),
                              cp("rot"), cp("proj"), cp("levels"), cp("thresholds"),
                              self.table.data_ptr() if self.table is not None else None)
        self._ws = None

    def sequence(self, b):
        """A one-sequence cache sharing sequence b's slice of every buffer (appends at
        a position of its own, e.g. for ragged prefill)."""
        sub = PackedKVCache.__new__(PackedKVCache)
        sub.__dict__.update(self.__dict__)
        sub.B = 1
        sub.layout = make_layout(self.fmt, 1, self.H, self.d, self.T, self.rope, self.sink, self.recent, self.P,
                                 self.num_pages, self.rotation)
        # a paged pool is shared; per-sequence buffers (windows, staging) are sliced
        pool = lambda n: self.P and BUFFERS.index(n) < BUFFERS.index("sink_k")  # noqa: E731
        sub.bufs = {n: (t if pool(n) else t.view(self.B, -1)[b]) for n, t in self.bufs.items()}
        sub.table = self.table[b:b + 1] if self.table is not None else None
        ptrs = [sub.bufs[n].data_ptr() if n in sub.bufs else None for n in BUFFERS]
        c = self.struct
        sub.struct = KVCache(sub.layout, (ctypes.c_void_p * len(BUFFERS))(*ptrs), c.rot, c.proj,
                             c.lm_levels, c.lm_thresh, sub.table.data_ptr() if sub.table is not None else None)
        sub._ws = None
        return sub

    # ---- views of the packed bytes
    def view(self, name):
        dt, shape = buffer_view_spec(self.fmt, self.B, self.H, self.T, self.d, self.rope, sink=self.sink,
                                     recent=self.recent, page_tokens=self.P, num_pages=self.num_pages)[name]
        return self.bufs[name].view(dt).view(shape)

    def bytes_per_token(self, num_layers=1):
        return kvq.kv_bytes_per_token(self.layout, num_layers)

    # ---- the two device entry points
    def append(self, k, v, start):
        """k, v: contiguous [B, H, n, d] (latent: k [B, n, d + rope], v None), fp32 or bf16;
        start: one first position for every sequence, or a sequence of B of them."""
        if not k.is_contiguous() or (v is not None and not v.is_contiguous()):
            raise ValueError("append inputs must be contiguous")
        if v is not None and v.dtype != k.dtype:
            raise ValueError("k and v must share a dtype")
        n = k.shape[-2]
        if isinstance(start, (int, np.integer)):
            kvq.kv_quant_append(self.struct, _ptr(k), _ptr(v), _TORCH_DT[k.dtype], int(start), n,
                                _stream_ptr(self.device))
        else:
            kvq.kv_quant_append_ragged(self.struct, _ptr(k), _ptr(v), _TORCH_DT[k.dtype], list(start), n,
                                       _stream_ptr(self.device))

    def workspace_bytes(self, num_q_heads, max_seq_len, splits=0, q_dtype=torch.bfloat16, num_queries=1, flags=0):
        opts = KVDecodeOpts(splits, None, None, num_queries, flags)
        return kvq.kv_decode_attention(self.struct, None, _TORCH_DT[q_dtype], num_q_heads, None, max_seq_len,
                                       1.0, None, None, 0, opts)

    def decode_sparse(self, q, sel, sel_n, scale, splits=0, out=None, ws=None, events=None, flags=0):
        """q: [B, Hq, d(+rope)]; sel int32 [B, K] positions, sel_n int32 [B] (device):
        query (b, hq) attends over sel[b, :sel_n[b]] only.  Returns fp32 [B, Hq, d].
        flags: kvq.DECODE_FP32 for the fp32 vector kernel."""
        q = q.contiguous()
        Hq, K = q.shape[-2], sel.shape[1]
        opts = KVDecodeOpts(splits, None, None, 1, flags)
        need = kvq.kv_decode_attention_sparse(self.struct, None, _TORCH_DT[q.dtype], Hq, None, None, K, 1.0, None,
                                              None, 0, opts)
        if ws is None:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
            ws = self._ws
        if out is None:
            out = torch.empty((self.B, Hq, self.d), dtype=torch.float32, device=self.device)
        if events is not None:
            opts = KVDecodeOpts(splits, ctypes.c_void_p(events[0].cuda_event), ctypes.c_void_p(events[1].cuda_event), 1,
                                flags)
        kvq.kv_decode_attention_sparse(self.struct, _ptr(q), _TORCH_DT[q.dtype], Hq, _ptr(sel), _ptr(sel_n), K,
                                       float(scale), _ptr(out), _ptr(ws), ws.numel(), opts,
                                       _stream_ptr(self.device))
        return out

    def decode(self, q, seq_lens, scale, max_seq_len=None, splits=0, out=None, ws=None, events=None, flags=0):
        """q: [B, Hq, d(+rope)] fp32/bf16, or [B, nq, Hq, d(+rope)] for nq query tokens per
        sequence (query j sees the first seq_lens[b] - (nq - 1 - j) tokens); seq_lens: int32
        device [B]. Returns fp32 [B, Hq, d] (or [B, nq, Hq, d]).  flags: kvq.DECODE_FP32 for
        the fp32 vector kernel (exact for any magnitude)."""
        q = q.contiguous()
        nq = q.shape[1] if q.dim() == 4 else 1
        Hq = q.shape[-2]
        max_seq_len = self.T if max_seq_len is None else max_seq_len
        need = self.workspace_bytes(Hq, max_seq_len, splits, q.dtype, nq, flags)
        if ws is None:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
            ws = self._ws
        if out is None:
            shape = (self.B, nq, Hq, self.d) if q.dim() == 4 else (self.B, Hq, self.d)
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        ev = (None, None) if events is None else (ctypes.c_void_p(events[0].cuda_event),
                                                  ctypes.c_void_p(events[1].cuda_event))
        opts = KVDecodeOpts(splits, ev[0], ev[1], nq, flags)
        kvq.kv_decode_attention(self.struct, _ptr(q), _TORCH_DT[q.dtype], Hq, _ptr(seq_lens), max_seq_len,
                                float(scale), _ptr(out), _ptr(ws), ws.numel(), opts,
                                _stream_ptr(self.device))
        return out
