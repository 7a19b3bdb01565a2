"""GPU parity at full workload sizes, on sampled (request, head) pairs.

The batch is the one bench.py times: every request's state is built on the GPU
by chained commits of its whole prefix (drawn on the device), then one forward
of the whole batch and one commit run in the same launch configuration. The
oracle then checks, one pair at a time:
  * the forward output of every pair, from the same fp32 state bytes the
    kernel read;
  * the commit of every pair, from the same pre-commit state;
  * the chained GPU state of the shortest and longest requests against the
    oracle's state built from scratch over their whole prefix;
  * one ragged prefill launch over the same prefix tokens (packed): every pair
    against the chained state, the tracked requests against the oracle;
  * one softmax prefix-attention launch over the same packed prefix and block,
    on sampled pairs (the shortest and longest prefixes among them).
Bars: normwise 2e-2 (bf16 I/O, fp32 accumulation and state).
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_block_amd as bha
import oracle
import synth
from helpers import normwise_err, pairs, record_to_plain, to_host

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
TOL = 2e-2
CHUNK = 256  # requests per oracle batch


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    bha.load_library()
    return torch.device("cuda:0")


def _pairwise_err(got, ref, d, F):
    # normwise error per (request, head) record, max over pairs: (S part, Z part)
    got, ref = got.double(), ref.double()
    out = []
    for lo, hi in ((0, d * F), (d * F, (d + 1) * F)):
        num = (got[..., lo:hi] - ref[..., lo:hi]).abs().amax(dim=-1)
        den = ref[..., lo:hi].abs().amax(dim=-1).clamp_min(1e-300)
        out.append(float((num / den).max()))
    return out


def _check_prefix_attention(name, q, k, v, pk, pv, offs, y, track, seed, n_pairs=6):
    # sampled (request, head) pairs, the shortest and longest prefixes among them
    R, B, H, d = q.shape
    rng = np.random.default_rng(seed + 1)
    rs = list(track) + [int(x) for x in rng.integers(0, R, size=n_pairs - len(track))]
    hs = rng.integers(0, H, size=len(rs))
    o = offs.cpu().numpy()
    err = 0.0
    for r, h in zip(rs, hs):
        a, b = int(o[r]), int(o[r + 1])
        ref = oracle.prefix_attention(to_host(q[r, :, h]), to_host(k[r, :, h]), to_host(v[r, :, h]),
                                      to_host(pk[a:b, h]), to_host(pv[a:b, h]))
        err = max(err, normwise_err(to_host(y[r, :, h]), ref, None))
    lens = [int(o[r + 1] - o[r]) for r in rs]
    print(f"[{name}] softmax prefix attention err {err:.2e} over {len(rs)} sampled pairs "
          f"(prefix tokens {min(lens)}..{max(lens)})", flush=True)
    assert err <= TOL


def _run_full(name, dev, seed=0):
    case = synth.make_case(name, with_prefix=False, with_qkv=False)
    R, H, d, FW, B = case.R, case.H, case.d, case.FW, case.B
    F = 2 * FW
    print(f"[{name}] R={R} H={H} d={d} FW={FW} B={B} prefix blocks {case.n_blocks.min()}..{case.n_blocks.max()}",
          flush=True)
    slots = torch.from_numpy(case.slot_ids).to(dev)
    w, gamma = synth.device_layer_params(name, 0, dev)
    state = bha.new_state(case.num_slots, H, d, FW, dev)
    track = sorted({int(np.argmin(case.n_blocks)), int(np.argmax(case.n_blocks))})
    kept = {r: ([], []) for r in track}
    for i in range(int(case.n_blocks.max())):
        act = np.nonzero(case.n_blocks > i)[0]
        kb, vb = synth.device_blocks(name, i, len(act), dev, layer=0)
        bha.state_commit(kb, vb, w, state, torch.from_numpy(case.slot_ids[act]).to(dev))
        for r in track:
            if case.n_blocks[r] > i:
                j = int(np.searchsorted(act, r))
                kept[r][0].append(kb[j].float().cpu().numpy())
                kept[r][1].append(vb[j].float().cpu().numpy())
    sel = torch.from_numpy(case.slot_ids.astype(np.int64)).to(dev)
    q, k, v = synth.device_step_qkv(name, 0, R, dev, layer=0)
    pk, pv, offs = synth.device_packed_prefix(name, case.n_blocks, dev, layer=0)
    state_p = bha.new_state(case.num_slots, H, d, FW, dev)
    bha.state_prefill(pk, pv, offs, w, state_p, slots)
    # the softmax attention over the whole prefix that the hybrid step replaces
    y_sm = bha.prefix_attention(q, k, v, pk, pv, offs)
    torch.cuda.synchronize()
    _check_prefix_attention(name, q, k, v, pk, pv, offs, y_sm, track, seed)
    del pk, pv, y_sm
    e_pc = _pairwise_err(state_p[sel], state[sel], d, F)
    prefilled = state_p[sel].cpu().numpy()
    del state_p
    print(f"[{name}] prefill vs chained commits over all {R * H} pairs: S err {e_pc[0]:.2e}, Z err {e_pc[1]:.2e}",
          flush=True)
    assert e_pc[0] <= TOL and e_pc[1] <= TOL

    out = bha.block_forward(q, k, v, w, gamma, state, slots)
    torch.cuda.synchronize()
    pre = state[torch.from_numpy(case.slot_ids.astype(np.int64)).to(dev)].cpu().numpy()  # [R][H][rec]
    state_f = state.clone()
    bha.state_commit(k, v, w, state, slots)
    torch.cuda.synchronize()
    post = state[torch.from_numpy(case.slot_ids.astype(np.int64)).to(dev)].cpu().numpy()

    # the fused last step on a copy of the same states: the same output, and the
    # same committed states on every pair
    out_f = bha.block_forward_commit(q, k, v, w, gamma, state_f, slots)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out)
    e_fc = _pairwise_err(state_f[sel], state[sel], d, F)
    del state_f, out_f
    print(f"[{name}] fused forward+commit vs forward then commit over all {R * H} pairs: output identical, "
          f"S err {e_fc[0]:.2e}, Z err {e_fc[1]:.2e}", flush=True)
    assert e_fc[0] <= 1e-5 and e_fc[1] <= 1e-5

    # every (request, head) pair against the oracle, in chunks of requests:
    # the forward from the same fp32 state bytes the kernel read, the commit
    # from the same pre-commit state
    w64 = w.float().cpu().numpy().astype(np.float64)
    g64 = gamma.cpu().numpy().astype(np.float64)
    err_f = err_c = 0.0
    for r0 in range(0, R, CHUNK):
        r1 = min(R, r0 + CHUNK)
        qh, kh, vh = (pairs(to_host(t[r0:r1])) for t in (q, k, v))
        S, Z = record_to_plain(pre[r0:r1], d, F)
        S, Z = np.ascontiguousarray(S), np.ascontiguousarray(Z)
        ref = oracle.block_forward_batch(qh, kh, vh, w64, g64, S, Z, nthreads=NTHREADS)
        err_f = max(err_f, normwise_err(pairs(to_host(out[r0:r1])), ref, (2, 3)))
        oracle.state_commit_batch(S, Z, kh, vh, w64, nthreads=NTHREADS)
        Sg, Zg = record_to_plain(post[r0:r1], d, F)
        err_c = max(err_c, normwise_err(Sg, S, (2, 3)), normwise_err(Zg, Z, (2,)))
    print(f"[{name}] forward err {err_f:.2e}, commit err {err_c:.2e} over all {R * H} pairs", flush=True)
    assert err_f <= TOL and err_c <= TOL

    for r in track:
        kp = np.concatenate(kept[r][0]).astype(np.float64)  # [N][H][d]
        vp = np.concatenate(kept[r][1]).astype(np.float64)
        S_ref = np.zeros((1, H, F, d))
        Z_ref = np.zeros((1, H, F))
        oracle.state_commit_batch(S_ref, Z_ref, np.ascontiguousarray(kp.transpose(1, 0, 2))[None],
                                  np.ascontiguousarray(vp.transpose(1, 0, 2))[None], w64, nthreads=NTHREADS)
        Sg, Zg = record_to_plain(pre[r], d, F)
        e_s = normwise_err(Sg, S_ref[0], (1, 2))
        e_z = normwise_err(Zg, Z_ref[0], (1,))
        print(f"[{name}] chained state of request {r} ({kp.shape[0]} prefix tokens): S err {e_s:.2e}, "
              f"Z err {e_z:.2e}", flush=True)
        assert e_s <= TOL and e_z <= TOL
        Sp, Zp = record_to_plain(prefilled[r], d, F)
        e_s = normwise_err(Sp, S_ref[0], (1, 2))
        e_z = normwise_err(Zp, Z_ref[0], (1,))
        print(f"[{name}] prefilled state of request {r}: S err {e_s:.2e}, Z err {e_z:.2e}", flush=True)
        assert e_s <= TOL and e_z <= TOL


def test_decode256_full_size(dev):
    # 256 requests x 16 heads, d=128, FW=64, B=32, ragged prefixes 256..8,192 tokens
    _run_full("decode256", dev)


def test_long_context_16k_full_size(dev):
    # 64 requests x 16 heads with 16,384-token prefixes
    _run_full("longctx16k", dev)


def test_long_context_32k_full_size(dev):
    # 64 requests x 16 heads with 32,768-token prefixes
    _run_full("longctx32k", dev)


def test_wide2048_full_size(dev):
    # 2,048 requests x 16 heads, FW=128 (F=256), prefixes 512..4,096 tokens
    _run_full("wide2048", dev)
