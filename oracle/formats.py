"""Encoders and decoders of every cache format, into the packed byte layout.

All arrays are C-contiguous, token-major: sequence b, head h, token t.  Stored
arrays come back in their storage dtype (uint8 codes; uint16 bit patterns for
bf16/fp16 metadata; float32 for fp32 metadata) so that a byte comparison with
another implementation is a plain array equality.

Bit order (a reading: the pages do not fix one), all least significant first:
  * FP4: channel 2j in the low nibble of byte j, channel 2j+1 in the high one;
  * 2-bit codes: channel 4j+i in bits [2i+1 : 2i] of byte j;
  * sign sketches: row 8j+i in bit i of byte j.
"""

import numpy as np

from . import e2m1
from .lloyd_max import quantize_index
from .numerics import (bf16_bits, bf16_from_bits, fp16_bits, fp16_from_bits,
                       round_bf16, round_fp16)

FP4_GROUP = 16
KIVI_GROUP = 32


# ----------------------------------------------------------------- bit packing

def pack_nibbles(nib):
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def pack_2bit(c):
    c = np.asarray(c, dtype=np.uint8)
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).astype(np.uint8)


def unpack_2bit(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 4,), dtype=np.uint8)
    for i in range(4):
        out[..., i::4] = (codes >> (2 * i)) & 3
    return out


def pack_bits(b):
    b = np.asarray(b, dtype=np.uint8)
    out = np.zeros(b.shape[:-1] + (b.shape[-1] // 8,), dtype=np.uint8)
    for i in range(8):
        out |= (b[..., i::8] & 1) << i
    return out


def unpack_bits(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 8,), dtype=np.uint8)
    for i in range(8):
        out[..., i::8] = (codes >> i) & 1
    return out


# ----------------------------------------------------------------- FP4 E2M1

def fp4_encode(x):
    """FP4 E2M1 with one bf16 scale per 16 channels.

    Page "How DeepSeek-V4.1-Flash cut KV-cache storage by 4x via CSA2", section
    on numerical precision: E2M1 elements, one scale per 16 channels, no second
    level scale.  Reading for the scale: s = bf16_RNE(absmax / 6), so the group's
    largest magnitude maps to the top E2M1 value; s = 0 encodes all nibbles 0.
    x: fp64 [..., d] -> (codes uint8 [..., d/2], scale bf16 bits uint16 [..., d/16]).
    """
    x = np.asarray(x, dtype=np.float64)
    g = x.reshape(x.shape[:-1] + (x.shape[-1] // FP4_GROUP, FP4_GROUP))
    absmax = np.abs(g).max(-1)
    s = round_bf16(absmax / 6.0)
    nib = e2m1.encode(g, s[..., None]).reshape(x.shape)
    return pack_nibbles(nib), bf16_bits(s)


def fp4_decode(codes, scale_bits):
    nib = unpack_nibbles(codes)
    s = bf16_from_bits(scale_bits)
    v = e2m1.decode(nib)
    v = v.reshape(v.shape[:-1] + (v.shape[-1] // FP4_GROUP, FP4_GROUP)) * s[..., None]
    return v.reshape(nib.shape)


# ----------------------------------------------------------------- KIVI 2-bit

def _kivi_codes(x32, mn, mx):
    """2-bit asymmetric codes of fp32 x against group min/max (fp32 arithmetic).

    Reading: s = fl32(fl32(max - min) / 3), z = min,
             c = clamp(RNE(fl32(fl32(x - z) / s)), 0, 3), and c = 0 where s == 0.
    """
    f = np.float32
    s = (mx - mn).astype(f) / f(3.0)
    s = s.astype(f)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = ((x32 - mn).astype(f) / s).astype(f)
    c = np.clip(np.rint(q), 0, 3)
    c = np.where(s > 0, c, 0).astype(np.uint8)
    return c, s, mn.astype(f)


def kivi2_encode_keys(k):
    """Keys quantised per channel over groups of 32 tokens.

    Page "TurboQuant vs OSCAR vs EpiCache", section "quantization frontiers":
    KIVI keeps keys per channel (their outlier channels are fixed across
    tokens) and values per token, at four levels (2 bits).
    k: [..., T, d] with T a multiple of 32 -> codes uint8 [..., T, d/4],
    scale f32 [..., T/32, d], zero f32 [..., T/32, d].
    """
    k32 = np.asarray(k, dtype=np.float32)
    T, d = k32.shape[-2:]
    g = k32.reshape(k32.shape[:-2] + (T // KIVI_GROUP, KIVI_GROUP, d))
    mn = g.min(-2, keepdims=True)
    mx = g.max(-2, keepdims=True)
    c, s, z = _kivi_codes(g, mn, mx)
    return pack_2bit(c.reshape(k32.shape)), s[..., 0, :], z[..., 0, :]


def kivi2_encode_values(v):
    """Values quantised per token over groups of 32 channels.

    v: [..., T, d] -> codes uint8 [..., T, d/4], scale f32 [..., T, d/32], zero f32 [..., T, d/32].
    """
    v32 = np.asarray(v, dtype=np.float32)
    d = v32.shape[-1]
    g = v32.reshape(v32.shape[:-1] + (d // KIVI_GROUP, KIVI_GROUP))
    mn = g.min(-1, keepdims=True)
    mx = g.max(-1, keepdims=True)
    c, s, z = _kivi_codes(g, mn, mx)
    return pack_2bit(c.reshape(v32.shape)), s[..., 0], z[..., 0]


def kivi2_decode_keys(codes, scale, zero):
    c = unpack_2bit(codes).astype(np.float64)
    T, d = c.shape[-2:]
    c = c.reshape(c.shape[:-2] + (T // KIVI_GROUP, KIVI_GROUP, d))
    out = c * np.asarray(scale, np.float64)[..., None, :] + np.asarray(zero, np.float64)[..., None, :]
    return out.reshape(c.shape[:-3] + (T, d))


def kivi2_decode_values(codes, scale, zero):
    c = unpack_2bit(codes).astype(np.float64)
    d = c.shape[-1]
    c = c.reshape(c.shape[:-1] + (d // KIVI_GROUP, KIVI_GROUP))
    out = c * np.asarray(scale, np.float64)[..., None] + np.asarray(zero, np.float64)[..., None]
    return out.reshape(c.shape[:-2] + (d,))


# ----------------------------------------------------------------- TurboQuant

def norms_fp16(x):
    """Euclidean norm of each row, in fp64, stored as fp16 bits (RNE)."""
    x = np.asarray(x, dtype=np.float64)
    return fp16_bits(round_fp16(np.sqrt((x * x).sum(-1))))


def turbo_stage1(x, rot, levels, thresholds):
    """Rotate, normalise and scalar-quantise rows of x.

    Stage one of TurboQuant (page "TurboQuant vs OSCAR vs EpiCache", section
    "quantization frontiers"): a random rotation makes coordinates nearly
    independent Gaussians, then each coordinate gets the Lloyd-Max code.
    Reading: the rotated vector is divided by its exact norm n = ||x|| (so its
    coordinates are close to N(0, 1/d)); n = 0 gives u = 0.
    Returns (n fp64, u fp64 [..., d], idx uint8 [..., d]).
    """
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt((x * x).sum(-1))
    y = x @ np.asarray(rot, dtype=np.float64).T
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n[..., None] > 0, y / safe[..., None], 0.0)
    idx = quantize_index(u, thresholds)
    return n, u, idx


def turbo_encode_keys(k, rot, proj, levels, thresholds):
    """TurboQuant keys: Lloyd-Max codes of the rotated unit vector, then a 1-bit
    QJL sketch of the residual and the residual's norm.

    Stage two (same page and section): a 1-bit quantised JL transform of the
    residual gives an unbiased estimate of the attention logit.  Reading: the
    residual is r = u - levels[idx] in the rotated unit space; the sketch bit
    of row i is [ (S r)_i >= 0 ]; the residual norm gamma = ||r|| and the
    vector norm n are stored as fp16.
    Returns dict(k_codes, k_sketch, k_norm, k_rnorm).
    """
    lv = np.asarray(levels, dtype=np.float64)
    n, u, idx = turbo_stage1(k, rot, lv, thresholds)
    r = u - lv[idx]
    gamma = np.sqrt((r * r).sum(-1))
    sr = r @ np.asarray(proj, dtype=np.float64).T
    bits = (sr >= 0).astype(np.uint8)
    return dict(
        k_codes=pack_2bit(idx),
        k_sketch=pack_bits(bits),
        k_norm=fp16_bits(round_fp16(n)),
        k_rnorm=fp16_bits(round_fp16(gamma)),
    )


def turbo_encode_values(v, rot, levels, thresholds):
    """TurboQuant values: rotated, normalised, Lloyd-Max coded (no residual sketch).

    Reading: the sketch estimates logits, which values do not enter, so values
    keep stage one only; their norm is stored as fp16.
    """
    n, u, idx = turbo_stage1(v, rot, levels, thresholds)
    return dict(v_codes=pack_2bit(idx), v_norm=fp16_bits(round_fp16(n)))


# ----------------------------------------------------------------- QJL 1-bit keys

def qjl_encode_keys(k, proj):
    """1-bit keys: the QJL sign sketch of k itself plus its fp16 norm.

    Reading: the 1-bit QJL stage applied directly to the key (no rotation and
    no scalar stage): bit i = [ (S k)_i >= 0 ].
    """
    k = np.asarray(k, dtype=np.float64)
    sk = k @ np.asarray(proj, dtype=np.float64).T
    return dict(k_sketch=pack_bits((sk >= 0).astype(np.uint8)), k_norm=norms_fp16(k))


# ----------------------------------------------------------------- full caches

def encode_cache(fmt, K=None, V=None, latent=None, consts=None, latent_dim=512):
    """Encode whole K/V (or latent) arrays into the named format's buffers.

    K, V: fp64 [B, H, T, d]; latent: fp64 [B, T, latent_dim + rope_dim].
    consts: dict(rot, proj, levels, thresholds) as needed.
    """
    if fmt == "fp4":
        kc, ks = fp4_encode(K)
        vc, vs = fp4_encode(V)
        return dict(k_codes=kc, k_scale=ks, v_codes=vc, v_scale=vs)
    if fmt == "kivi2":
        kc, ks, kz = kivi2_encode_keys(K)
        vc, vs, vz = kivi2_encode_values(V)
        return dict(k_codes=kc, k_scale=ks, k_zero=kz, v_codes=vc, v_scale=vs, v_zero=vz)
    if fmt == "turbo":
        out = turbo_encode_keys(K, consts["rot"], consts["proj"], consts["levels"], consts["thresholds"])
        out.update(turbo_encode_values(V, consts["rot"], consts["levels"], consts["thresholds"]))
        return out
    if fmt == "qjl1":
        out = qjl_encode_keys(K, consts["proj"])
        vc, vs = fp4_encode(V)
        out.update(v_codes=vc, v_scale=vs)
        return out
    if fmt == "latent":
        lat = np.asarray(latent, dtype=np.float64)
        cc, cs = fp4_encode(lat[..., :latent_dim])
        return dict(k_codes=cc, k_scale=cs, rope=bf16_bits(lat[..., latent_dim:]))
    raise ValueError(fmt)
