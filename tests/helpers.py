"""Test-side glue: layout conversion between the library's state records and the
oracle's plain arrays, host <-> device transfer of synthetic inputs, and the
error metric. Written from the layout documented in include/bha.h; the library
itself never uses this code.
"""
from __future__ import annotations

import numpy as np

import synth


def s_index(d: int, F: int) -> np.ndarray:
    """[F][d] array of float offsets of S[f][c] inside one state record: the S
    part is stored in 32 x 4 tiles, tile (c // 32, f // 4) at
    ((c // 32) * (F // 4) + f // 4) * 128, column c % 32 at 4 * (c % 32) in it,
    feature f % 4 last."""
    f = np.arange(F)[:, None]
    c = np.arange(d)[None, :]
    return ((c // 32) * (F // 4) + f // 4) * 128 + (c % 32) * 4 + (f % 4)


def record_to_plain(rec: np.ndarray, d: int, F: int):
    """Records [..., (d+1)F] -> (S [..., F, d], Z [..., F]) as float64."""
    rec = np.asarray(rec, dtype=np.float64)
    idx = s_index(d, F)
    return rec[..., idx], rec[..., d * F:(d + 1) * F]


def plain_to_record(S: np.ndarray, Z: np.ndarray, d: int, F: int) -> np.ndarray:
    """(S [..., F, d], Z [..., F]) -> records [..., (d+1)F] float32."""
    lead = S.shape[:-2]
    rec = np.zeros(lead + ((d + 1) * F,), dtype=np.float32)
    idx = s_index(d, F)
    rec[..., idx] = S
    rec[..., d * F:] = Z
    return rec


def normwise_err(got: np.ndarray, ref: np.ndarray, axes) -> float:
    """max over tiles of max|got - ref| / max|ref| (tile = the given trailing axes)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def to_device(x: np.ndarray, io: str, device):
    """Exact host float32 values (already representable in ``io``) -> torch tensor."""
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    if io == "bf16":
        bits = synth.bf16_bits(x)
        assert np.array_equal(synth.bf16_to_f32(bits), x), "value not representable in bf16"
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def to_host(t) -> np.ndarray:
    """torch tensor (bf16 / f32) -> exact float64 numpy array."""
    import torch

    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def pairs(x: np.ndarray) -> np.ndarray:
    """[R][B][H][d] token layout -> the oracle's pair-major [R][H][B][d]."""
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))
