"""Seeded synthetic inputs for block-hybrid attention.

This module only draws random numbers and converts them to the storage dtype
(bf16 by round-to-nearest-even on the host). It holds none of the method's
arithmetic, so both the HIP path's tests and the oracle can take their inputs
from it without sharing any computation.

Workloads (d = head dim, FW = columns of the Hedgehog matrix W, F = 2 FW,
B = block length; prefix lengths are whole blocks):

==========  =====  ==  ===  ===  ==  ==============================  =====
name        R      H   d    FW   B   prefix blocks per request        I/O
==========  =====  ==  ===  ===  ==  ==============================  =====
tiny        1      1   64   32   8   4                                fp32
b16         16     16  128  64   32  64 (2,048 tokens)                bf16
decode256   256    16  128  64   32  UniformInt{8..256} (256..8,192)  bf16
longctx     64     16  128  64   32  512 or 1,024 (16K / 32K tokens)  bf16
wide2048    2048   16  128  128  32  UniformInt{16..128}             bf16
==========  =====  ==  ===  ===  ==  ==============================  =====

Distributions: Q, K, V ~ N(0, 1); W ~ N(0, 1/d) (so xW ~ N(0, 1) for x ~ N(0, I));
the gate is 0.5 in ``tiny`` and U(0, 1) per head elsewhere. Request slots are a
seeded sample without replacement from a pool of 2R slots, so the slots a batch
touches are not contiguous, as under continuous batching.

Streams: ``numpy.random.Generator(PCG64(SeedSequence(1000 + config_id)))``
spawned into children in a fixed order: lengths, slots, W, gamma, prefix K/V,
step Q/K/V. Device-side generation (for prefixes too large to draw on the host)
uses ``torch.Generator`` seeded from the same config id and the block index.
"""
from __future__ import annotations

import dataclasses

import numpy as np

CONFIGS = {
    "tiny": dict(cid=0, R=1, H=1, d=64, FW=32, B=8, blocks=(4, 4), io="f32", gamma="half"),
    "b16": dict(cid=1, R=16, H=16, d=128, FW=64, B=32, blocks=(64, 64), io="bf16", gamma="uniform"),
    "decode256": dict(cid=2, R=256, H=16, d=128, FW=64, B=32, blocks=(8, 256), io="bf16",
                      gamma="uniform"),
    "longctx16k": dict(cid=3, R=64, H=16, d=128, FW=64, B=32, blocks=(512, 512), io="bf16",
                       gamma="uniform"),
    "longctx32k": dict(cid=3, R=64, H=16, d=128, FW=64, B=32, blocks=(1024, 1024), io="bf16",
                       gamma="uniform"),
    "longctx2k": dict(cid=3, R=64, H=16, d=128, FW=64, B=32, blocks=(64, 64), io="bf16",
                      gamma="uniform"),
    "wide2048": dict(cid=4, R=2048, H=16, d=128, FW=128, B=32, blocks=(16, 128), io="bf16",
                     gamma="uniform"),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value (returned as float32)."""
    return bf16_to_f32(bf16_bits(x))


@dataclasses.dataclass
class Case:
    """One batch of inputs in the library's layouts, as exact float32 host values.

    q, k, v : [R][B][H][d]   active block (values already representable in ``io``)
    w       : [H][FW][d]     row j of head h = column j of that head's d x FW matrix
    gamma   : [H]
    slot_ids: [R] int32      state slot of each request, unique, in [0, num_slots)
    n_blocks: [R] int64      committed prefix blocks of each request
    prefix_k, prefix_v : list (per request) of [N_r][H][d] arrays, or None
    """
    name: str
    R: int
    H: int
    d: int
    FW: int
    B: int
    io: str
    num_slots: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    w: np.ndarray
    gamma: np.ndarray
    slot_ids: np.ndarray
    n_blocks: np.ndarray
    prefix_k: list | None
    prefix_v: list | None

    @property
    def F(self) -> int:
        return 2 * self.FW


def _streams(cid: int):
    ss = np.random.SeedSequence(1000 + cid)
    names = ("lengths", "slots", "w", "gamma", "prefix", "step")
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, ss.spawn(len(names)))}


def _cast(x: np.ndarray, io: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if io == "bf16" else x


def make_case(name: str, *, R=None, with_prefix=True, with_qkv=True, step=0, **over) -> Case:
    """Draw a whole case on the host. ``R`` (and any shape key) may be overridden,
    e.g. to take the first requests of a large config; ``step`` selects which
    denoising step's Q/K/V is drawn (each step draws fresh values)."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    if R is not None:
        cfg["R"] = R
    R, H, d, FW, B, io = cfg["R"], cfg["H"], cfg["d"], cfg["FW"], cfg["B"], cfg["io"]
    st = _streams(cfg["cid"])
    lo, hi = cfg["blocks"]
    n_blocks = st["lengths"].integers(lo, hi + 1, size=R).astype(np.int64)
    num_slots = 2 * R
    slot_ids = st["slots"].choice(num_slots, size=R, replace=False).astype(np.int32)
    w = _cast(st["w"].standard_normal((H, FW, d), dtype=np.float32) / np.float32(np.sqrt(d)), io)
    if cfg["gamma"] == "half":
        gamma = np.full((H,), 0.5, dtype=np.float32)
    else:
        gamma = st["gamma"].random(H, dtype=np.float32)
    prefix_k = prefix_v = None
    if with_prefix:
        prefix_k, prefix_v = [], []
        for r in range(R):
            n = int(n_blocks[r]) * B
            prefix_k.append(_cast(st["prefix"].standard_normal((n, H, d), dtype=np.float32), io))
            prefix_v.append(_cast(st["prefix"].standard_normal((n, H, d), dtype=np.float32), io))
    g = st["step"]
    if with_qkv:
        for _ in range(step):
            g.standard_normal((3, R, B, H, d), dtype=np.float32)
        qkv = _cast(g.standard_normal((3, R, B, H, d), dtype=np.float32), io)
    else:
        qkv = np.zeros((3, 0, B, H, d), dtype=np.float32)
    return Case(name=name, R=R, H=H, d=d, FW=FW, B=B, io=io, num_slots=num_slots,
                q=qkv[0], k=qkv[1], v=qkv[2], w=w, gamma=gamma, slot_ids=slot_ids,
                n_blocks=n_blocks, prefix_k=prefix_k, prefix_v=prefix_v)


def _device_gen(device, *keys):
    import torch

    gen = torch.Generator(device=device)
    seed = 0
    for k in keys:
        seed = (seed * 1_000_003 + int(k)) % (1 << 62)
    gen.manual_seed(seed)
    return gen


def _io_torch(io):
    import torch

    return torch.bfloat16 if io == "bf16" else torch.float32


def device_layer_params(name: str, layer: int, device, **over):
    """W ([H][FW][d], N(0, 1/d)) and gate ([H], U(0, 1)) of one layer instance,
    drawn on ``device``."""
    import torch

    cfg = dict(CONFIGS[name])
    cfg.update(over)
    H, d, FW = cfg["H"], cfg["d"], cfg["FW"]
    gen = _device_gen(device, 1000 + cfg["cid"], 11, layer)
    w = torch.randn((H, FW, d), generator=gen, device=device, dtype=torch.float32) / float(np.sqrt(d))
    gamma = torch.rand((H,), generator=gen, device=device, dtype=torch.float32)
    return w.to(_io_torch(cfg["io"])), gamma


def device_blocks(name: str, block_index: int, rows: int, device, *, layer: int = 0, **over):
    """Prefix K and V of one block index for ``rows`` requests, drawn on ``device``
    with a torch generator seeded from the config id, the layer and the block
    index. Returns two [rows][B][H][d] tensors in the config's I/O dtype."""
    import torch

    cfg = dict(CONFIGS[name])
    cfg.update(over)
    B, H, d = cfg["B"], cfg["H"], cfg["d"]
    gen = _device_gen(device, 1000 + cfg["cid"], 22, layer, block_index)
    kv = torch.randn((2, rows, B, H, d), generator=gen, device=device, dtype=torch.float32)
    kv = kv.to(_io_torch(cfg["io"]))
    return kv[0], kv[1]


def device_step_qkv(name: str, step: int, R: int, device, *, layer: int = 0, **over):
    """Fresh Q, K, V ([R][B][H][d] each) of one denoising step, drawn on ``device``."""
    import torch

    cfg = dict(CONFIGS[name])
    cfg.update(over)
    B, H, d = cfg["B"], cfg["H"], cfg["d"]
    gen = _device_gen(device, 1000 + cfg["cid"], 33, layer, step)
    qkv = torch.randn((3, R, B, H, d), generator=gen, device=device, dtype=torch.float32)
    qkv = qkv.to(_io_torch(cfg["io"]))
    return qkv[0], qkv[1], qkv[2]


def device_packed_prefix(name: str, n_blocks, device, *, layer: int = 0, **over):
    """Every request's whole prefix packed token-major for a ragged prefill:
    returns (k, v, seq_offsets) with k, v [T][H][d] and seq_offsets int32 [R+1],
    request r owning rows seq_offsets[r] .. seq_offsets[r+1]-1. The tokens are
    exactly those ``device_blocks`` draws for block indices 0 .. n_blocks[r]-1
    (same seeds), so a prefill over them and chained commits of those blocks
    fold the same values."""
    import torch

    cfg = dict(CONFIGS[name])
    cfg.update(over)
    B, H, d = cfg["B"], cfg["H"], cfg["d"]
    n_blocks = np.asarray(n_blocks, dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(n_blocks * B)])
    T = int(offs[-1])
    k = torch.empty((T, H, d), dtype=_io_torch(cfg["io"]), device=device)
    v = torch.empty_like(k)
    offs_dev = torch.from_numpy(offs).to(device)
    tok = torch.arange(B, device=device)
    for i in range(int(n_blocks.max(initial=0))):
        act = torch.from_numpy(np.nonzero(n_blocks > i)[0]).to(device)
        kb, vb = device_blocks(name, i, int(act.numel()), device, layer=layer, **over)
        rows = (offs_dev[act][:, None] + i * B + tok[None, :]).reshape(-1)
        k[rows] = kb.reshape(-1, H, d)
        v[rows] = vb.reshape(-1, H, d)
    return k, v, torch.from_numpy(offs.astype(np.int32)).to(device)
