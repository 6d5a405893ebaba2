"""Decode attention over a packed cache: the plain definition (one query token
per sequence, or several with a causal tail mask).

During decoding every new token attends over the keys and values of all cached
tokens, and the whole cache is streamed from HBM for each of them (page
"TurboQuant vs OSCAR vs EpiCache", section on the KV-cache memory bottleneck).
A fused streaming kernel reaches exactly this result, so the oracle is the
definition, materialised in fp64:

  for each sequence b and query head hq, with KV head g = hq // (Hq / H)
  (reading: contiguous query-head groups share a KV head):
      l_t = scale * logit(q[b, hq], cache[b, g, t])      for t < L_b
      p   = softmax(l)      (max subtracted, fp64)
      o   = sum_t p_t * value(cache[b, g, t])

Reading: a single query sees all L_b cached tokens with no mask (its own key
and value were appended before the call); the softmax scale is an argument.

Per format, logit() and value() are:
  fp4, kivi2   <q, k_hat>,  v_hat                 (dequantised in fp64)
  latent       <q_c, c_hat> + <q_r, k_rope>,  c_hat (value = the latent)
  turbo        n_k * ( <R q, u_tilde> + kappa * gamma * <S R q, sigma> ),
               value n_v * R^T u_tilde_v
  qjl1         kappa * n_k * <S q, sigma>,  v_hat (FP4)
with sigma = +-1 from the sketch bits and kappa = sqrt(pi/2) / m.  kappa follows
from E[ sign(<g, r>) <g, q> ] = sqrt(2/pi) <q, r> / ||r|| for g ~ N(0, I): the
QJL estimate of <q, r> is kappa * ||r|| * <S q, sign(S r)>, unbiased over S
(page "TurboQuant vs OSCAR vs EpiCache", section "quantization frontiers",
stage two).  The turbo logit rests on <q, k> = n <R q, u> for orthogonal R
and u = R k / n = u_tilde + r.

Several query tokens per sequence (decode_attention_multi): a draft model can
propose several next positions at once for the main model to check in one pass
(page "How DeepSeek-V4.1-Flash cut KV-cache storage by 4x via CSA2", section
"numerical precision & hardware efficiency": five draft positions predicted in
parallel).  Reading: the nq queries are the last nq tokens of the sequence,
their keys and values already appended, and query j (0-based) sees every token
up to and including its own position, t < L_b - (nq - 1 - j); nq = 1 is the
single-query case above.

Mixed precision (decode_attention_mixed): the first `sink` tokens of each
sequence and its last `recent` tokens are kept in BF16 while the rest of the
history is compressed (page "TurboQuant vs OSCAR vs EpiCache", section
"quantization frontiers: TurboQuant and OSCAR": sink and recent tokens stay in
BF16, the history goes to a low-bit code; about 0.24% of a 128K context stays
BF16).  Reading: token t of a sequence of length L attends through bf16(k_t),
bf16(v_t) when t < sink or t >= L - recent, and through its packed code
otherwise; a window token's logit is the plain <q, bf16(k_t)> for every format.

KIVI-2 staging (decode_attention_kivi_staged): KIVI quantises keys per channel
over 32-token groups (page "TurboQuant vs OSCAR vs EpiCache", section
"quantization frontiers", KIVI paragraph), so the keys of a sequence's last,
incomplete group have no code yet.  Reading: they are kept as they came in and
attend exactly; token t of a sequence appended up to A tokens (decoded over its
first L <= A) uses its input key when t >= 32 * floor(A / 32), its packed key
otherwise, and its packed value always.

Logits and dequantised values are computed in token chunks only to bound
memory; the softmax is taken over the full logit vector.
"""

import math

import numpy as np

from . import formats as F
from .numerics import bf16_from_bits, fp16_from_bits, round_bf16

CHUNK = 65536


def qjl_kappa(m: int) -> float:
    return math.sqrt(math.pi / 2.0) / m


def _key_logits(fmt, cache, b, h, t0, t1, qg, consts, latent_dim):
    """Unscaled logits [G, t1-t0] of query rows qg [G, key_width] against tokens t0..t1."""
    if fmt == "fp4":
        kh = F.fp4_decode(cache["k_codes"][b, h, t0:t1], cache["k_scale"][b, h, t0:t1])
        return qg @ kh.T
    if fmt == "kivi2":
        g0, g1 = t0 // F.KIVI_GROUP, -(-t1 // F.KIVI_GROUP)
        kh = F.kivi2_decode_keys(cache["k_codes"][b, h, g0 * F.KIVI_GROUP:g1 * F.KIVI_GROUP],
                                 cache["k_scale"][b, h, g0:g1], cache["k_zero"][b, h, g0:g1])
        kh = kh[t0 - g0 * F.KIVI_GROUP:t1 - g0 * F.KIVI_GROUP]
        return qg @ kh.T
    if fmt == "latent":
        ch = F.fp4_decode(cache["k_codes"][b, t0:t1], cache["k_scale"][b, t0:t1])
        kr = bf16_from_bits(cache["rope"][b, t0:t1])
        return qg[:, :latent_dim] @ ch.T + qg[:, latent_dim:] @ kr.T
    if fmt == "turbo":
        rot = np.asarray(consts["rot"], np.float64)
        proj = np.asarray(consts["proj"], np.float64)
        lv = np.asarray(consts["levels"], np.float64)
        q_rot = qg @ rot.T
        q_s = q_rot @ proj.T
        ut = lv[F.unpack_2bit(cache["k_codes"][b, h, t0:t1])]
        sig = 2.0 * F.unpack_bits(cache["k_sketch"][b, h, t0:t1]).astype(np.float64) - 1.0
        n = fp16_from_bits(cache["k_norm"][b, h, t0:t1])
        gam = fp16_from_bits(cache["k_rnorm"][b, h, t0:t1])
        kap = qjl_kappa(proj.shape[0])
        return n[None, :] * (q_rot @ ut.T + kap * gam[None, :] * (q_s @ sig.T))
    if fmt == "qjl1":
        proj = np.asarray(consts["proj"], np.float64)
        q_s = qg @ proj.T
        sig = 2.0 * F.unpack_bits(cache["k_sketch"][b, h, t0:t1]).astype(np.float64) - 1.0
        n = fp16_from_bits(cache["k_norm"][b, h, t0:t1])
        return qjl_kappa(proj.shape[0]) * n[None, :] * (q_s @ sig.T)
    raise ValueError(fmt)


def _values(fmt, cache, b, h, t0, t1, consts, latent_dim):
    """Dequantised values [t1-t0, dv] (turbo: in the rotated space, times n_v)."""
    if fmt in ("fp4", "qjl1"):
        return F.fp4_decode(cache["v_codes"][b, h, t0:t1], cache["v_scale"][b, h, t0:t1])
    if fmt == "kivi2":
        return F.kivi2_decode_values(cache["v_codes"][b, h, t0:t1], cache["v_scale"][b, h, t0:t1],
                                     cache["v_zero"][b, h, t0:t1])
    if fmt == "latent":
        return F.fp4_decode(cache["k_codes"][b, t0:t1], cache["k_scale"][b, t0:t1])
    if fmt == "turbo":
        lv = np.asarray(consts["levels"], np.float64)
        ut = lv[F.unpack_2bit(cache["v_codes"][b, h, t0:t1])]
        n = fp16_from_bits(cache["v_norm"][b, h, t0:t1])
        return n[:, None] * ut
    raise ValueError(fmt)


def decode_attention_row_group(fmt, cache, b, h, qg, L, scale, consts=None, latent_dim=512,
                               chunk=CHUNK):
    """Outputs [G, dv] for the query rows qg of sequence b, KV head h, over L tokens."""
    qg = np.asarray(qg, dtype=np.float64)
    if L <= 0:
        raise ValueError("decode over an empty context is undefined")
    logits = np.concatenate([
        _key_logits(fmt, cache, b, h, t0, min(L, t0 + chunk), qg, consts, latent_dim)
        for t0 in range(0, L, chunk)], axis=1) * scale
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    out = None
    for t0 in range(0, L, chunk):
        t1 = min(L, t0 + chunk)
        part = p[:, t0:t1] @ _values(fmt, cache, b, h, t0, t1, consts, latent_dim)
        out = part if out is None else out + part
    if fmt == "turbo":
        out = out @ np.asarray(consts["rot"], np.float64)   # R^T applied to each row
    return out


def decode_attention(fmt, cache, q, seq_lens, scale, hkv, consts=None, latent_dim=512,
                     rows=None):
    """fp64 outputs [B, Hq, dv] (or only the (b, hq) pairs in `rows`, as a dict)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq = q.shape[:2]
    G = Hq // hkv
    if rows is None:
        outs = []
        for b in range(B):
            per_b = [decode_attention_row_group(fmt, cache, b, h, q[b, h * G:(h + 1) * G],
                                                int(seq_lens[b]), scale, consts, latent_dim)
                     for h in range(hkv)]
            outs.append(np.concatenate(per_b, 0))
        return np.stack(outs, 0)
    res = {}
    for (b, hq) in rows:
        h = hq // G
        res[(b, hq)] = decode_attention_row_group(fmt, cache, b, h, q[b, hq:hq + 1],
                                                  int(seq_lens[b]), scale, consts, latent_dim)[0]
    return res


def decode_attention_multi(fmt, cache, q, seq_lens, scale, hkv, consts=None, latent_dim=512, chunk=CHUNK):
    """fp64 outputs [B, nq, Hq, dv] for q [B, nq, Hq, dk]: query j of sequence b
    sees the tokens t < seq_lens[b] - (nq - 1 - j)."""
    q = np.asarray(q, dtype=np.float64)
    B, nq, Hq = q.shape[:3]
    G = Hq // hkv
    out = None
    for b in range(B):
        L = int(seq_lens[b])
        if L < nq:
            raise ValueError("every query must see at least its own token")
        # row (j, g) of the group: query token j, query head h * G + g
        limit = L - (nq - 1 - np.repeat(np.arange(nq), G))
        visible = np.arange(L)[None, :] < limit[:, None]
        for h in range(hkv):
            qg = q[b, :, h * G:(h + 1) * G].reshape(nq * G, -1)
            logits = np.concatenate([
                _key_logits(fmt, cache, b, h, t0, min(L, t0 + chunk), qg, consts, latent_dim)
                for t0 in range(0, L, chunk)], axis=1) * scale
            logits = np.where(visible, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            p /= p.sum(axis=1, keepdims=True)
            o = None
            for t0 in range(0, L, chunk):
                t1 = min(L, t0 + chunk)
                part = p[:, t0:t1] @ _values(fmt, cache, b, h, t0, t1, consts, latent_dim)
                o = part if o is None else o + part
            if fmt == "turbo":
                o = o @ np.asarray(consts["rot"], np.float64)
            if out is None:
                out = np.zeros((B, nq, Hq, o.shape[1]))
            out[b, :, h * G:(h + 1) * G] = o.reshape(nq, G, -1)
    return out


def decode_attention_mixed(fmt, cache, q, seq_lens, scale, hkv, K_in, V_in, sink, recent, consts=None,
                           appended=None):
    """fp64 outputs [B, nq, Hq, d] for q [B, nq, Hq, d] over a cache whose tokens
    t < sink and t >= L - recent are read as bf16 of the inputs K_in, V_in
    ([B, H, T, d]) and the others through their packed codes; query j sees the
    first L - (nq - 1 - j) tokens.

    Reading for the 2-bit histories (page "TurboQuant vs OSCAR vs EpiCache",
    OSCAR deployment list: sink and recent tokens BF16, the history INT2):
      * TURBO: a packed token's value is n_v R^T u~ (in the original basis, as in
        decode_attention), a window token's the bf16 input; the logit of a
        window token is <q, bf16 k> with the caller's query;
      * KIVI2: keys of a sequence's last incomplete group (from
        32 * floor(appended[b] / 32) on, appended defaulting to the length) have
        no code yet and are read from the inputs unrounded, unless the token is
        in a window (bf16 there too)."""
    if fmt not in ("fp4", "qjl1", "kivi2", "turbo"):
        raise ValueError("mixed precision is defined here for the fp4, qjl1, kivi2 and turbo caches")
    q = np.asarray(q, dtype=np.float64)
    B, nq, Hq = q.shape[:3]
    G = Hq // hkv
    appended = seq_lens if appended is None else appended
    out = np.zeros((B, nq, Hq, K_in.shape[-1]))
    for b in range(B):
        L = int(seq_lens[b])
        if L < nq:
            raise ValueError("every query must see at least its own token")
        t = np.arange(L)
        window = (t < sink) | (t >= L - recent)
        staged = (t >= F.KIVI_GROUP * (int(appended[b]) // F.KIVI_GROUP)) if fmt == "kivi2" else np.zeros(L, bool)
        limit = L - (nq - 1 - np.repeat(np.arange(nq), G))
        visible = t[None, :] < limit[:, None]
        for h in range(hkv):
            qg = q[b, :, h * G:(h + 1) * G].reshape(nq * G, -1)
            kin = np.asarray(K_in[b, h, :L], np.float64)
            kb = round_bf16(kin)
            vb = round_bf16(np.asarray(V_in[b, h, :L], np.float64))
            packed = _key_logits(fmt, cache, b, h, 0, L, qg, consts, 0)
            if fmt == "kivi2":
                packed = np.where(staged[None, :], qg @ kin.T, packed)
            logits = np.where(window[None, :], qg @ kb.T, packed) * scale
            logits = np.where(visible, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            p /= p.sum(axis=1, keepdims=True)
            hist = _values(fmt, cache, b, h, 0, L, consts, 0)
            if fmt == "turbo":
                hist = hist @ np.asarray(consts["rot"], np.float64)   # R^T applied to each value
            vals = np.where(window[:, None], vb, hist)
            out[b, :, h * G:(h + 1) * G] = (p @ vals).reshape(nq, G, -1)
    return out


def decode_attention_kivi_staged(cache, q, seq_lens, scale, hkv, K_in, appended=None):
    """fp64 outputs [B, nq, Hq, d] for q [B, nq, Hq, d] over a KIVI-2 cache whose
    last incomplete key group of each sequence (appended[b] tokens appended, by
    default seq_lens[b]) is read from the input keys K_in ([B, H, T, d]); query
    j sees the first L - (nq - 1 - j) tokens."""
    appended = seq_lens if appended is None else appended
    q = np.asarray(q, dtype=np.float64)
    B, nq, Hq = q.shape[:3]
    G = Hq // hkv
    out = np.zeros((B, nq, Hq, K_in.shape[-1]))
    for b in range(B):
        L = int(seq_lens[b])
        if L < nq:
            raise ValueError("every query must see at least its own token")
        t = np.arange(L)
        staged = t >= F.KIVI_GROUP * (int(appended[b]) // F.KIVI_GROUP)
        limit = L - (nq - 1 - np.repeat(np.arange(nq), G))
        visible = t[None, :] < limit[:, None]
        for h in range(hkv):
            qg = q[b, :, h * G:(h + 1) * G].reshape(nq * G, -1)
            exact = qg @ np.asarray(K_in[b, h, :L], np.float64).T
            logits = np.where(staged[None, :], exact, _key_logits("kivi2", cache, b, h, 0, L, qg, None, 0)) * scale
            logits = np.where(visible, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h * G:(h + 1) * G] = (p @ _values("kivi2", cache, b, h, 0, L, None, 0)).reshape(nq, G, -1)
    return out
