"""Seeded random GPU parity cases over the supported sizes (through the C ABI).

Each case draws a shape (requests, heads, d, FW, block size, I/O dtype, K/V
head grouping), a ragged prefix per request, the gate (zero allowed), the
token layout (contiguous or a view of a fused [R][B][3][H][d] tensor) and the
batch's slots from a pool, then checks against the fp64 oracle:
  * the state built by one ragged prefill;
  * bha_block_forward (or bha_block_forward_gqa) from those state bytes;
  * bha_block_forward_commit on a copy (the output equal to the forward's, the
    committed state against the oracle's commit);
  * bha_state_commit;
  * bha_feature_map of the queries.
Bars: normwise 1e-4 (fp32 I/O), 2e-2 (bf16 I/O, fp32 accumulation).
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_block_amd as bha
import oracle
import synth
from helpers import normwise_err, pairs, record_to_plain, to_device, to_host

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
TOL = {"f32": 1e-4, "bf16": 2e-2}
N_CASES = 24


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    bha.load_library()
    return torch.device("cuda:0")


def _draw(seed):
    rng = np.random.default_rng(7000 + seed)
    io = "bf16" if rng.random() < 0.75 else "f32"
    d = int(rng.choice([64, 128]))
    fw = int(rng.choice([32, 64, 128]))
    b = int(rng.integers(1, 65))
    g = int(rng.choice([1, 1, 2, 4, 8]))
    hk = int(rng.integers(1, 4))
    R = int(rng.integers(1, 9))
    fused = bool(rng.random() < 0.5)
    return rng, dict(io=io, d=d, fw=fw, b=b, g=g, hk=hk, H=hk * g, R=R, fused=fused)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(dev, seed):
    rng, c = _draw(seed)
    io, d, fw, B, G, HK, H, R = c["io"], c["d"], c["fw"], c["b"], c["g"], c["hk"], c["H"], c["R"]
    F = 2 * fw
    tol = TOL[io]
    cast = (lambda x: synth.round_bf16(x)) if io == "bf16" else (lambda x: np.asarray(x, np.float32))
    f32 = np.float32
    # inputs (exact values in the I/O dtype)
    q = cast(rng.standard_normal((R, B, H, d)).astype(f32))
    k = cast(rng.standard_normal((R, B, HK, d)).astype(f32))
    v = cast(rng.standard_normal((R, B, HK, d)).astype(f32))
    w = cast((rng.standard_normal((HK, fw, d)) / np.sqrt(d)).astype(f32))
    gamma = rng.random(H).astype(f32)
    gamma[rng.random(H) < 0.2] = 0.0
    lens = rng.integers(0, 3 * 32 + 1, size=R)
    lens[rng.random(R) < 0.2] = 0
    pool = 2 * R + 3
    slots_np = rng.choice(pool, size=R, replace=False).astype(np.int32)
    kp = cast(rng.standard_normal((int(lens.sum()), HK, d)).astype(f32))
    vp = cast(rng.standard_normal((int(lens.sum()), HK, d)).astype(f32))
    offs_np = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    print(f"[random {seed}] io={io} d={d} FW={fw} B={B} R={R} H={H} K/V heads={HK} fused-view={c['fused']} "
          f"prefix lens {lens.tolist()}", flush=True)

    # device tensors; q (and k, v when G = 1) as views of one fused tensor
    if c["fused"] and G == 1:
        qkv = to_device(np.stack([q, k, v], axis=2), io, dev)
        qd, kd, vd = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    else:
        qd, kd, vd = (to_device(x, io, dev) for x in (q, k, v))
    wd = to_device(w, io, dev)
    gd = torch.from_numpy(gamma).to(dev)
    sd = torch.from_numpy(slots_np).to(dev)
    state = bha.new_state(pool, HK, d, fw, dev)
    if lens.sum() > 0:
        bha.state_prefill(to_device(kp, io, dev), to_device(vp, io, dev), torch.from_numpy(offs_np).to(dev), wd,
                          state, sd)
    torch.cuda.synchronize()
    S, Z = record_to_plain(state.cpu().numpy()[slots_np], d, F)  # [R][HK][F][d]
    errs = {}
    # the prefill against the oracle's build
    e = 0.0
    for r in range(R):
        for h in range(HK):
            a_, b_ = offs_np[r], offs_np[r + 1]
            S_ref, Z_ref = oracle.state_build(kp[a_:b_, h].astype(np.float64), vp[a_:b_, h].astype(np.float64), w[h])
            if b_ > a_:
                e = max(e, normwise_err(S[r, h], S_ref, None), normwise_err(Z[r, h], Z_ref, None))
            else:
                assert not np.any(S[r, h]) and not np.any(Z[r, h])
    errs["prefill"] = e

    # the forward from the same state bytes, through the oracle per query head
    if G == 1:
        y = bha.block_forward(qd, kd, vd, wd, gd, state, sd)
    else:
        y = bha.block_forward_gqa(qd, kd, vd, wd, gd, state, sd)
    torch.cuda.synchronize()
    rep = lambda a: np.repeat(a, G, axis=1)  # noqa: E731
    ref = oracle.block_forward_batch(pairs(q), rep(pairs(k)), rep(pairs(v)), np.repeat(w, G, axis=0), gamma,
                                     rep(S), rep(Z), nthreads=NTHREADS)
    errs["forward"] = normwise_err(pairs(to_host(y)), ref, (2, 3))

    # the commit, and (one K/V head per query head) the fused step on a copy
    S_c, Z_c = np.ascontiguousarray(S), np.ascontiguousarray(Z)
    oracle.state_commit_batch(S_c, Z_c, pairs(k), pairs(v), w, nthreads=NTHREADS)
    if G == 1:
        st2 = state.clone()
        y2 = bha.block_forward_commit(qd, kd, vd, wd, gd, st2, sd)
        torch.cuda.synchronize()
        assert torch.equal(y2, y), "the fused step's output must equal the forward's"
        S2, Z2 = record_to_plain(st2.cpu().numpy()[slots_np], d, F)
        errs["fused commit"] = max(normwise_err(S2, S_c, (2, 3)), normwise_err(Z2, Z_c, (2,)))
    bha.state_commit(kd, vd, wd, state, sd)
    torch.cuda.synchronize()
    S3, Z3 = record_to_plain(state.cpu().numpy()[slots_np], d, F)
    errs["commit"] = max(normwise_err(S3, S_c, (2, 3)), normwise_err(Z3, Z_c, (2,)))

    # the feature map of the queries (W of K/V head 0 for every query head)
    w_shared = to_device(w[0], io, dev)
    phi = to_host(bha.feature_map(qd, w_shared))
    phi_ref = oracle.phi(q.reshape(-1, d), w[0]).reshape(R, B, H, F)
    errs["feature map"] = normwise_err(phi, phi_ref, (3,))
    print(f"[random {seed}] " + ", ".join(f"{k_} {v_:.2e}" for k_, v_ in errs.items()), flush=True)
    for k_, v_ in errs.items():
        bar = 1e-5 if k_ == "feature map" else tol
        assert v_ <= bar, f"{k_}: {v_:.3e} > {bar}"
