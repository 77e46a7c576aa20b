"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module draws random numbers and lays them out; it holds none of the
operator's arithmetic.  Both sides of every parity check receive the same
bytes from here.

Generator (published definitions, restated):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014), in its counter form: draw i of stream s is
    mix64(s + (i + 1) * 0x9E3779B97F4A7C15), with the finaliser
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
    z *= 0x94D049BB133111EB; z ^= z >> 31.
  * uniform u = (z >> 11) * 2**-53 in [0, 1).
  * Box-Muller (1958): normals 2j and 2j+1 of a stream are
    r*cos(t) and r*sin(t) with r = sqrt(-2 ln(1 - u_{2j})), t = 2*pi*u_{2j+1}.
  * Draws are made in float64, rounded to float32, then rounded
    (round-to-nearest-even) to the storage dtype.

Each tensor has its own stream, seeded ``seed * 16 + tensor_id`` with
tensor_id 0 = value, 1 = offset_mask (or the locations and logits of flash
deformable attention), 2 = grad_output, 3 = the attention reference points;
elements are drawn in memory order.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
TENSOR_VALUE, TENSOR_OFFSET_MASK, TENSOR_GRAD_OUT, TENSOR_REFERENCE = 0, 1, 2, 3
_CHUNK = 1 << 22  # pairs per chunk


def splitmix64(stream_seed: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of the SplitMix64 stream (uint64)."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(stream_seed & 0xFFFFFFFFFFFFFFFF) + i * GAMMA
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform(stream_seed: int, start: int, count: int) -> np.ndarray:
    z = splitmix64(stream_seed, start, count)
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal_f32(stream_seed: int, count: int) -> np.ndarray:
    """First ``count`` standard normals of a stream, rounded to float32."""
    out = np.empty(count, np.float32)
    npairs = (count + 1) // 2
    for p0 in range(0, npairs, _CHUNK):
        np_ = min(_CHUNK, npairs - p0)
        u = uniform(stream_seed, 2 * p0, 2 * np_)
        r = np.sqrt(-2.0 * np.log1p(-u[0::2]))
        t = (2.0 * np.pi) * u[1::2]
        z = np.empty(2 * np_, np.float64)
        z[0::2] = r * np.cos(t)
        z[1::2] = r * np.sin(t)
        e0 = 2 * p0
        e1 = min(count, e0 + 2 * np_)
        out[e0:e1] = z[: e1 - e0]
    return out


def stream(seed: int, tensor_id: int) -> int:
    return seed * 16 + tensor_id


def value_f32(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return (normal_f32(stream(seed, TENSOR_VALUE), n) * np.float32(sigma)).reshape(shape)


def grad_out_f32(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return (normal_f32(stream(seed, TENSOR_GRAD_OUT), n) * np.float32(sigma)).reshape(shape)


def offset_mask_f32(N: int, Ho: int, Wo: int, G: int, K: int, P: int, seed: int,
                    sigma_off: float, sigma_m: float, pad_fill: float = float("nan"),
                    integer_offsets: bool = False) -> np.ndarray:
    """Fused offset/mask tensor (N, Ho, Wo, P).

    Channel layout per pixel: for each group g, K (dx, dy) pairs then K mask
    values; channels [3*G*K, P) are padding filled with ``pad_fill``.

    ``integer_offsets``: for (pixel, g, k) with (pixel + 3g + k) % 4 == 0 the
    pair (dx, dy) is rounded to the nearest integer (ties to even), and set to
    (0, 0) when (pixel + 3g + k) % 64 == 0 -- this puts sampling coordinates
    exactly on integers, on -1 and on size-1.
    """
    n = N * Ho * Wo * P
    z = normal_f32(stream(seed, TENSOR_OFFSET_MASK), n).reshape(N * Ho * Wo, P)
    body = z[:, : 3 * G * K].reshape(N * Ho * Wo, G, 3 * K)
    body[:, :, : 2 * K] *= np.float32(sigma_off)
    body[:, :, 2 * K:] *= np.float32(sigma_m)
    if integer_offsets:
        pix = np.arange(N * Ho * Wo, dtype=np.int64)[:, None, None]
        gg = np.arange(G, dtype=np.int64)[None, :, None]
        kk = np.arange(K, dtype=np.int64)[None, None, :]
        key = pix + 3 * gg + kk
        sel = (key % 4) == 0
        zero = (key % 64) == 0
        d = body[:, :, : 2 * K].reshape(N * Ho * Wo, G, K, 2)
        rounded = np.rint(d)
        d[...] = np.where(sel[..., None], rounded, d)
        d[...] = np.where(zero[..., None], np.float32(0.0), d)
        body[:, :, : 2 * K] = d.reshape(N * Ho * Wo, G, 2 * K)
    z[:, : 3 * G * K] = body.reshape(N * Ho * Wo, 3 * G * K)
    z[:, 3 * G * K:] = np.float32(pad_fill)
    return z.reshape(N, Ho, Wo, P)


def om_channels(G: int, K: int) -> int:
    """Padded channel count of the fused offset/mask tensor (multiple of 8)."""
    return (3 * G * K + 7) // 8 * 8


def to_storage(a_f32: np.ndarray, dtype: str):
    """Round a float32 array to the storage dtype (RNE).

    Returns (torch CPU tensor in the storage dtype, float32 numpy copy of the
    rounded values) -- the second is what the oracle consumes.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a_f32))
    if dtype == "fp32":
        st = t.clone()
    elif dtype == "fp16":
        st = t.to(torch.float16)
    elif dtype == "bf16":
        st = t.to(torch.bfloat16)
    else:
        raise ValueError(dtype)
    return st, st.to(torch.float32).numpy()


def fdattn_channels(L: int, K: int) -> int:
    """Padded entry count of a (query, head) row of loc_attn (multiple of 8)."""
    return (3 * L * K + 7) // 8 * 8


def fdattn_loc_attn_f32(N: int, Q: int, M: int, shapes, K: int, P: int, seed: int,
                        sigma_px: float, sigma_logit: float, encoder_queries: bool = True,
                        pad_fill: float = float("nan")) -> np.ndarray:
    """Locations and logits of flash deformable attention, (N, Q, M, P).

    Row of (query, head): L*K normalised (u, v) pairs (level-major, point
    inner), then L*K logits, then padding up to P filled with ``pad_fill``.

    Locations are a reference point plus a normal offset of ``sigma_px``
    pixels of the sampled level: u = ref_u + sigma_px * z / W_l.  With
    ``encoder_queries`` (Q must equal sum H_l*W_l) query q is pixel q of the
    concatenated levels and its reference point is that pixel's centre;
    otherwise reference points are uniform in [0, 1)^2 (stream 3).
    Logits are sigma_logit * N(0, 1).  Drawn in float64, rounded to float32.
    """
    shapes = [(int(h), int(w)) for h, w in shapes]
    L = len(shapes)
    LK = L * K
    if encoder_queries:
        S = sum(h * w for h, w in shapes)
        if Q != S:
            raise ValueError("encoder queries need Q == sum H_l*W_l")
        ref = np.empty((Q, 2), np.float64)
        q0 = 0
        for h, w in shapes:
            r, c = np.divmod(np.arange(h * w, dtype=np.float64), w)
            ref[q0:q0 + h * w, 0] = (c + 0.5) / w
            ref[q0:q0 + h * w, 1] = (r + 0.5) / h
            q0 += h * w
        ref = np.broadcast_to(ref[None], (N, Q, 2))
    else:
        ref = uniform(stream(seed, TENSOR_REFERENCE), 0, N * Q * 2).reshape(N, Q, 2)
    z = normal_f32(stream(seed, TENSOR_OFFSET_MASK), N * Q * M * P).reshape(N, Q, M, P).astype(np.float64)
    out = np.empty((N, Q, M, P), np.float64)
    wl = np.array([w for _, w in shapes], np.float64)
    hl = np.array([h for h, _ in shapes], np.float64)
    zl = z[..., :2 * LK].reshape(N, Q, M, L, K, 2)
    u = ref[:, :, None, None, None, 0] + sigma_px * zl[..., 0] / wl[None, None, None, :, None]
    v = ref[:, :, None, None, None, 1] + sigma_px * zl[..., 1] / hl[None, None, None, :, None]
    loc = np.stack([u, v], -1).reshape(N, Q, M, 2 * LK)
    out[..., :2 * LK] = loc
    out[..., 2 * LK:3 * LK] = sigma_logit * z[..., 2 * LK:3 * LK]
    out[..., 3 * LK:] = pad_fill
    return out.astype(np.float32)
