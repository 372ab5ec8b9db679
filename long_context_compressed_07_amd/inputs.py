"""Seeded synthetic inputs in their storage formats.

This module holds none of the layer's arithmetic. It only draws random numbers and casts them to
storage formats with PyTorch's dtype casts; both the HIP path and the CPU oracle consume what it
returns (the oracle after decoding the bytes itself).

Recipe (per tensor): a child of numpy.random.SeedSequence(seed) in the fixed order of
`_ORDER[kind]`, a PCG64 generator, float32 standard normals drawn in row chunks, multiplied by
1/sqrt(dim) where dim is the tensor's vector length (d for x, g, q and cache rows; d_I for indexer
vectors; H_I for indexer head weights; m for the position bias; d_model for the hidden state and
the projection weights) and cast to the storage dtype:
  * bf16 / f32: round-to-nearest-even cast of the float32 draw;
  * e4m3 rows: codes = e4m3(clip(z, +-3.9) * 112) (never saturates), one fp32 scale per row
    drawn from the same stream as (sigma / 112) * U(0.75, 1.25), so the dequantised rows have
    std ~ sigma.
  * MXFP4 rows (the low-precision indexer): float32 draws cast per block of 32 consecutive values
    to a shared power-of-two scale 2^(floor(log2 amax) - 2) (E8M0 code) and E2M1 codes of
    value / scale, round to nearest even with saturation to +-6 (the OCP MX conversion), two
    codes per byte, low nibble first.
"Sharp" inputs (parity only) draw q with std 1 and gate logits and bias with std 1; used with
sm_scale = 1 they give attention logits of std ~1 instead of ~1/d.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Workload

_CHUNK = 1 << 24  # elements per draw chunk

_ORDER = {
    "csa_decode_proj": ["hidden", "w_x", "w_g", "bias", "q_i", "w_i", "k_i", "q"],
    "csa_decode": ["ent_c", "ent_r", "raw_c", "raw_r", "k_i", "q_i", "w_i", "q"],
    "csa_prefill": ["x", "g", "bias", "k_i", "q_i", "w_i", "q"],
    "hca_prefill": ["x", "g", "bias", "q"],
    "hybrid_decode": ["ent_c", "ent_r", "raw_c", "raw_r", "k_i", "q_i", "w_i", "q",
                      "hca_c", "hca_r", "q_hca"],
}


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    out *= np.float32(std)
    return out.reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 codes (uint16) through torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3_rows(rng: np.random.Generator, shape, std: float):
    """fp8 rows: (codes uint8 [..., d], scale float32 [...])."""
    z = _normal(rng, shape, 1.0)
    np.clip(z, -3.9, 3.9, out=z)
    z *= np.float32(112.0)
    codes = torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    u = rng.uniform(0.75, 1.25, size=shape[:-1]).astype(np.float32)
    scale = (np.float32(std / 112.0) * u).astype(np.float32)
    return codes, scale


def to_mxfp4(x: np.ndarray):
    """float32 [..., d] (d % 32 == 0) -> (packed E2M1 codes uint8 [..., d/2], E8M0 scales uint8
    [..., d/32]): the storage cast of MXFP4 rows."""
    x = np.asarray(x, dtype=np.float32)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32)).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    y = np.abs(blk) / np.ldexp(1.0, e)[..., None]
    # nearest E2M1 magnitude, ties to the even fraction bit: steps of 0.5 below 2, 1 below 4, 2 up
    # to 6 (saturating)
    q = np.where(y < 2, np.rint(2 * y) / 2, np.where(y < 4, np.rint(y), 2 * np.rint(y / 2)))
    q = np.minimum(q, 6.0)
    mag_code = np.select([q == v for v in (0, .5, 1, 1.5, 2, 3, 4, 6)], np.arange(8), 0)
    code = (mag_code + 8 * ((blk < 0) & (q > 0))).astype(np.uint8)
    code = code.reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def to_e4m3_rows(x: np.ndarray):
    """float32 [..., d] -> (E4M3 codes uint8 [..., d], float32 row scales [...]): the storage cast of
    fp8 rows with one scale per row, sigma = amax / 448 and codes = e4m3(x / sigma) (torch's cast;
    an all-zero row stores sigma 0)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    sigma = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(sigma > 0, sigma, np.float32(1.0))
    codes = torch.from_numpy(np.ascontiguousarray(x / safe[..., None])).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).numpy(), sigma


def mxfp4_rows(rng: np.random.Generator, shape, std: float):
    """MXFP4 rows of Gaussian draws with the given std: (packed codes, scales)."""
    return to_mxfp4(_normal(rng, shape, std))


def _vec(wl_dtype: str, rng, shape, std):
    a = _normal(rng, shape, std)
    if wl_dtype == "bf16":
        return to_bf16_bits(a)
    if wl_dtype == "f32":
        return a
    raise ValueError(wl_dtype)


def make_inputs(wl: Workload, seed: int, sharp: bool = False) -> dict:
    """All inputs of one workload, as numpy arrays in storage format.

    bf16 tensors are uint16 codes, e4m3 tensors uint8 codes with a float32 `*_scale` companion,
    f32 tensors float32. Shapes: see the per-kind blocks below.
    """
    kind = wl.kind
    key = "csa_decode_proj" if (kind == "csa_decode" and wl.d_model) else kind
    names = _ORDER[key]
    kids = np.random.SeedSequence(seed).spawn(len(names))
    rngs = {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, kids)}
    d, B, T, N = wl.d, wl.B, wl.T, wl.n_entries
    qstd = 1.0 if sharp else 1.0 / np.sqrt(d)
    gstd = 1.0 if sharp else 1.0 / np.sqrt(d)
    bstd = 1.0 if sharp else 1.0 / np.sqrt(wl.m)
    nq_total = B * wl.nq
    out = {}
    if key == "csa_decode_proj":
        dm = wl.d_model
        out["hidden"] = _normal(rngs["hidden"], (B, T, dm), 1.0 / np.sqrt(dm))
        out["w_x"] = _normal(rngs["w_x"], (dm, d), 1.0 / np.sqrt(dm))
        wg_std = 1.0 if sharp else 1.0 / np.sqrt(dm)   # std of g equals std of w_g
        out["w_g"] = _normal(rngs["w_g"], (dm, d), wg_std)
        out["bias"] = _normal(rngs["bias"], (wl.m,), bstd)
        out["q_i"] = _normal(rngs["q_i"], (nq_total, wl.H_I, wl.d_I), 1.0 / np.sqrt(wl.d_I))
        out["w_i"] = _normal(rngs["w_i"], (nq_total, wl.H_I), 1.0 / np.sqrt(wl.H_I))
        out["k_i"] = _normal(rngs["k_i"], (B, N, wl.d_I), 1.0 / np.sqrt(wl.d_I))
        out["q"] = _normal(rngs["q"], (nq_total, wl.H, d), qstd)
        return out
    if kind in ("csa_decode", "hybrid_decode"):
        std = 1.0 / np.sqrt(d)
        assert wl.kv_dtype == "e4m3" and wl.idx_dtype == "e4m3"
        out["ent_c"], out["ent_scale"] = _e4m3_rows(rngs["ent_c"], (B, N, wl.d_c), std)
        out["ent_r"] = to_bf16_bits(_normal(rngs["ent_r"], (B, N, wl.d_r), std))
        out["raw_c"], out["raw_scale"] = _e4m3_rows(rngs["raw_c"], (B, wl.window, wl.d_c), std)
        out["raw_r"] = to_bf16_bits(_normal(rngs["raw_r"], (B, wl.window, wl.d_r), std))
        out["k_i"], out["k_i_scale"] = _e4m3_rows(rngs["k_i"], (B, N, wl.d_I),
                                                  1.0 / np.sqrt(wl.d_I))
        out["q_i"], out["q_i_scale"] = _e4m3_rows(rngs["q_i"], (nq_total, wl.H_I, wl.d_I),
                                                  1.0 / np.sqrt(wl.d_I))
        out["w_i"] = _normal(rngs["w_i"], (nq_total, wl.H_I), 1.0 / np.sqrt(wl.H_I))
        out["q"] = to_bf16_bits(_normal(rngs["q"], (nq_total, wl.H, d), qstd))
        if kind == "hybrid_decode":
            nh = wl.n_hca
            out["hca_c"], out["hca_scale"] = _e4m3_rows(rngs["hca_c"], (B, nh, wl.d_c), std)
            out["hca_r"] = to_bf16_bits(_normal(rngs["hca_r"], (B, nh, wl.d_r), std))
            out["q_hca"] = to_bf16_bits(_normal(rngs["q_hca"], (nq_total, wl.H, d), qstd))
        return out
    if kind in ("csa_prefill", "hca_prefill"):
        out["x"] = _vec(wl.kv_dtype, rngs["x"], (B, T, d), 1.0 / np.sqrt(d))
        out["g"] = _vec(wl.kv_dtype, rngs["g"], (B, T, d), gstd)
        out["bias"] = _normal(rngs["bias"], (wl.m,), bstd)
        if kind == "csa_prefill":
            out["k_i"] = _vec(wl.idx_dtype, rngs["k_i"], (B, N, wl.d_I), 1.0 / np.sqrt(wl.d_I))
            out["q_i"] = _vec(wl.idx_dtype, rngs["q_i"], (nq_total, wl.H_I, wl.d_I),
                              1.0 / np.sqrt(wl.d_I))
            out["w_i"] = _normal(rngs["w_i"], (nq_total, wl.H_I), 1.0 / np.sqrt(wl.H_I))
        out["q"] = _vec(wl.q_dtype, rngs["q"], (nq_total, wl.H, d), qstd)
        return out
    raise ValueError(kind)


def query_positions(wl: Workload) -> tuple[np.ndarray, np.ndarray]:
    """(seq [B*nq] int32, pos [B*nq] int64): each sequence's last nq positions, in order."""
    seq = np.repeat(np.arange(wl.B, dtype=np.int32), wl.nq)
    pos = np.tile(np.arange(wl.T - wl.nq, wl.T, dtype=np.int64), wl.B)
    return seq, pos
