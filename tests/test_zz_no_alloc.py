"""The allocation-free prefix attention (bha_prefix_attention_noalloc) against
bha_prefix_attention with a full caller workspace, through the C ABI.

Both calls take the same split, so the outputs must agree bit for bit (and so
within the 2e-2 / 1e-4 bars). Two calls in a row on one device, the second
with a smaller batch: the static buffer then holds the first call's partials,
which must not leak into the second. Cases: a few pairs over long packed
prefixes (the key sequence split over many work-groups), bf16 and fp32, and a
batch with enough pairs that no split is taken.
"""
import numpy as np
import pytest
import torch

import linear_attention_block_amd as bha
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    bha.load_library()
    return torch.device("cuda:0")


def _batch(dev, io, R, H, B, lengths, layer):
    over = dict(H=H, d=128, FW=64, B=B, io=io)
    q, k, v = synth.device_step_qkv("longctx2k", 0, R, dev, layer=layer, **over)
    nb = np.asarray(lengths, dtype=np.int64)
    pk, pv, offs = synth.device_packed_prefix("longctx2k", nb, dev, layer=layer, **dict(over, B=32))
    return q, k, v, pk, pv, offs


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_equals_workspace_call_twice(dev, io):
    cases = [  # (R, H, B, prefix blocks of 32 tokens per request)
        (3, 2, 32, [600, 17, 250]),    # 6 pairs: a many-way split
        (1, 2, 20, [130]),             # second call, smaller: fewer splits, shorter rows
    ]
    assert bha.prefix_attention_noalloc_scratch_bytes() == 9 << 20
    for i, (R, H, B, lengths) in enumerate(cases):
        q, k, v, pk, pv, offs = _batch(dev, io, R, H, B, lengths, layer=i)
        need = bha.prefix_attention_workspace(R, H, 128, B, pk.shape[0], dtype=q.dtype)
        ref = bha.prefix_attention(q, k, v, pk, pv, offs)
        out = torch.full_like(q, float("nan"))
        bha.prefix_attention_noalloc(q, k, v, pk, pv, offs, out=out)
        torch.cuda.synchronize()
        same = torch.equal(out, ref)
        err = float(((out.double() - ref.double()).abs().amax() / ref.double().abs().amax()).item())
        print(f"[noalloc] call {i + 1}: io={io} R={R} H={H} B={B} prefix tokens {pk.shape[0]}, workspace "
              f"{need} bytes: {'bit-identical' if same else f'err {err:.2e}'}", flush=True)
        assert need > 0, "the case must take the split path"
        assert same and err <= (2e-2 if io == "bf16" else 1e-4)


def test_noalloc_without_split(dev):
    # 64 x 16 pairs fill the GPU: no split, the static buffer is not touched
    q, k, v, pk, pv, offs = _batch(dev, "bf16", 64, 16, 32, [8] * 64, layer=3)
    assert bha.prefix_attention_workspace(64, 16, 128, 32, pk.shape[0]) == 0
    ref = bha.prefix_attention(q, k, v, pk, pv, offs)
    out = torch.empty_like(q)
    bha.prefix_attention_noalloc(q, k, v, pk, pv, offs, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
