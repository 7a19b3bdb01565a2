"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Inputs come from ``synth`` (seeded); the same exact values go to the device and
to the oracle. Errors use the normwise metric max over (request, head) of
max|got - ref| / max|ref|. Bars: 1e-4 with float32 I/O, 2e-2 with bf16 I/O
(bf16 matrix-core inputs, fp32 accumulation).
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


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    bha.load_library()  # raises if libbha.so is missing: no fallback
    return torch.device("cuda:0")


def _log(msg):
    print(msg, flush=True)


class Run:
    """One case on the GPU: state built by chained commits, then one forward
    and one commit of the active block; plus the oracle's view of each step."""

    def __init__(self, case: synth.Case, dev):
        self.c = case
        self.dev = dev
        c = case
        self.w = to_device(c.w, c.io, dev)
        self.gamma = torch.from_numpy(c.gamma).to(dev)
        self.slots = torch.from_numpy(c.slot_ids).to(dev)
        self.state = bha.new_state(c.num_slots, c.H, c.d, c.FW, dev)

    def build_state(self):
        c = self.c
        for i in range(int(c.n_blocks.max(initial=0))):
            act = np.nonzero(c.n_blocks > i)[0]
            kb = np.stack([c.prefix_k[r][i * c.B:(i + 1) * c.B] for r in act])
            vb = np.stack([c.prefix_v[r][i * c.B:(i + 1) * c.B] for r in act])
            bha.state_commit(to_device(kb, c.io, self.dev), to_device(vb, c.io, self.dev), self.w,
                             self.state, torch.from_numpy(c.slot_ids[act]).to(self.dev))
        torch.cuda.synchronize()

    def plain_state(self):
        """(S [R][H][F][d], Z [R][H][F]) float64 of the batch's slots."""
        rec = self.state.cpu().numpy()[self.c.slot_ids]
        return record_to_plain(rec, self.c.d, self.c.F)

    def oracle_state(self):
        c = self.c
        S = np.zeros((c.R, c.H, c.F, c.d))
        Z = np.zeros((c.R, c.H, c.F))
        w64 = c.w.astype(np.float64)
        for r in range(c.R):
            if c.n_blocks[r] == 0:
                continue
            k = np.ascontiguousarray(np.transpose(c.prefix_k[r], (1, 0, 2)))[None]
            v = np.ascontiguousarray(np.transpose(c.prefix_v[r], (1, 0, 2)))[None]
            s1, z1 = S[r:r + 1].copy(), Z[r:r + 1].copy()
            oracle.state_commit_batch(s1, z1, k, v, w64, nthreads=NTHREADS)
            S[r], Z[r] = s1[0], z1[0]
        return S, Z

    def forward(self, out=None):
        c = self.c
        q, k, v = (to_device(x, c.io, self.dev) for x in (c.q, c.k, c.v))
        y = bha.block_forward(q, k, v, self.w, self.gamma, self.state, self.slots, out=out)
        torch.cuda.synchronize()
        return y

    def oracle_forward(self, S, Z):
        c = self.c
        return oracle.block_forward_batch(pairs(c.q), pairs(c.k), pairs(c.v), c.w, c.gamma, S, Z,
                                          nthreads=NTHREADS)

    def commit_active(self):
        c = self.c
        bha.state_commit(to_device(c.k, c.io, self.dev), to_device(c.v, c.io, self.dev), self.w,
                         self.state, self.slots)
        torch.cuda.synchronize()


def _full_check(case, dev):
    tol = TOL[case.io]
    run = Run(case, dev)
    run.build_state()
    S_gpu, Z_gpu = run.plain_state()
    S_ora, Z_ora = run.oracle_state()
    e_s = normwise_err(S_gpu, S_ora, (2, 3))
    e_z = normwise_err(Z_gpu, Z_ora, (2,))
    _log(f"[{case.name}] state build  S err {e_s:.2e}  Z err {e_z:.2e}")
    assert e_s <= tol and e_z <= tol

    y = to_host(run.forward())
    ref_same = run.oracle_forward(S_gpu, Z_gpu)  # the same fp32 state bytes
    ref_ora = run.oracle_forward(S_ora, Z_ora)   # the oracle's own state
    e1 = normwise_err(pairs(y), ref_same, (2, 3))
    e2 = normwise_err(pairs(y), ref_ora, (2, 3))
    _log(f"[{case.name}] forward  err(same state) {e1:.2e}  err(oracle state) {e2:.2e}")
    assert np.all(np.isfinite(y))
    assert e1 <= tol and e2 <= tol

    run.commit_active()
    S2, Z2 = run.plain_state()
    S_ref, Z_ref = S_gpu.copy(), Z_gpu.copy()
    oracle.state_commit_batch(S_ref, Z_ref, pairs(case.k), pairs(case.v), case.w.astype(np.float64),
                              nthreads=NTHREADS)
    e_s = normwise_err(S2, S_ref, (2, 3))
    e_z = normwise_err(Z2, Z_ref, (2,))
    _log(f"[{case.name}] commit  S err {e_s:.2e}  Z err {e_z:.2e}")
    assert e_s <= tol and e_z <= tol
    return run


def test_tiny_fp32_end_to_end(dev):
    # 1 request, 1 head, d=64, FW=32, B=8, 4 committed blocks, gate 0.5, fp32 I/O
    _full_check(synth.make_case("tiny"), dev)


def test_b16_bf16_end_to_end(dev):
    # 16 requests x 16 heads, d=128, FW=64, B=32, 2,048-token prefixes, bf16 I/O
    _full_check(synth.make_case("b16"), dev)


SWEEP = [
    # (io, d, FW, B): bf16 takes the matrix-core kernels (B <= 32: one query tile
    # and the commit kernel; 33..64: two query tiles and commits through the
    # prefill kernel), fp32 the fp32-arithmetic kernels
    ("bf16", 128, 64, 32), ("bf16", 128, 64, 1), ("bf16", 128, 64, 17), ("bf16", 128, 32, 32),
    ("bf16", 128, 128, 32), ("bf16", 64, 32, 8), ("bf16", 64, 64, 31), ("bf16", 64, 128, 32),
    ("bf16", 128, 64, 33), ("bf16", 64, 32, 64), ("bf16", 128, 64, 48), ("bf16", 128, 128, 64),
    ("bf16", 128, 32, 63), ("bf16", 64, 64, 40), ("bf16", 64, 128, 57),
    ("f32", 128, 64, 32), ("f32", 64, 128, 5), ("f32", 128, 32, 64), ("f32", 64, 64, 1), ("f32", 128, 128, 40),
]


@pytest.mark.parametrize("io,d,fw,b", SWEEP)
def test_shape_sweep(dev, io, d, fw, b):
    # ragged prefixes of 0..3 blocks (0 = empty state), 5 requests, 3 heads
    case = synth.make_case("tiny", R=5, H=3, d=d, FW=fw, B=b, io=io, blocks=(0, 3), gamma="uniform")
    _log(f"[sweep] io={io} d={d} FW={fw} B={b} n_blocks={case.n_blocks.tolist()}")
    _full_check(case, dev)


FEATURE_MAP = [
    # (io, d, FW, R, B, strided): bf16 takes the matrix-core kernel (tiles of
    # 32 d / 32 tokens of one head: one partial tile, several tiles with a
    # ragged tail, token rows seen through a view of a fused tensor), fp32 the
    # fp32-arithmetic kernel
    ("bf16", 128, 64, 3, 7, False), ("f32", 64, 32, 3, 7, False), ("bf16", 64, 128, 3, 7, False),
    ("bf16", 128, 128, 9, 33, False), ("bf16", 128, 32, 5, 64, True), ("bf16", 64, 64, 7, 19, True),
    ("f32", 128, 128, 4, 9, True),
]


@pytest.mark.parametrize("io,d,fw,R,b,strided", FEATURE_MAP)
def test_feature_map(dev, io, d, fw, R, b, strided):
    case = synth.make_case("tiny", R=R, H=3, d=d, FW=fw, B=b, io=io, with_prefix=False)
    if strided:
        # x = q, a view of a fused [R][B][3][H][d] tensor
        x = to_device(np.stack([case.q, case.k, case.v], axis=2), io, dev)[:, :, 0]
    else:
        x = to_device(case.q, io, dev)
    phi = to_host(bha.feature_map(x, to_device(case.w, io, dev)))
    ref = np.empty_like(phi)
    for h in range(case.H):
        ref[:, :, h] = oracle.phi(case.q[:, :, h].reshape(-1, d), case.w[h]).reshape(R, b, 2 * fw)
    err = normwise_err(phi, ref, (3,))
    _log(f"[feature_map] io={io} d={d} FW={fw} R={R} B={b} strided={strided} err {err:.2e}")
    assert err <= 1e-5


def test_strided_views_and_shared_map(dev):
    # q, k, v as views of one fused [R][B][3][H][d] tensor; out as a [R][H][B][d]
    # tensor seen through a permute; one W shared by every head
    case = synth.make_case("tiny", R=4, H=3, d=128, FW=64, B=32, io="bf16", blocks=(1, 2),
                           gamma="uniform")
    case.w[:] = case.w[0]
    run = Run(case, dev)
    run.w = to_device(case.w[0], case.io, dev)  # [FW][d]: head stride 0
    run.build_state()
    fused = to_device(np.stack([case.q, case.k, case.v], axis=2), case.io, dev)
    q, k, v = fused[:, :, 0], fused[:, :, 1], fused[:, :, 2]
    out = torch.empty((case.R, case.H, case.B, case.d), dtype=torch.bfloat16, device=dev)
    out_v = out.permute(0, 2, 1, 3)
    bha.block_forward(q, k, v, run.w, run.gamma, run.state, run.slots, out=out_v)
    torch.cuda.synchronize()
    S, Z = run.plain_state()
    err = normwise_err(pairs(to_host(out_v)), run.oracle_forward(S, Z), (2, 3))
    _log(f"[strided] err {err:.2e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("io,b", [("bf16", 32), ("bf16", 48), ("f32", 8)])
def test_out_of_range_slot_is_isolated(dev, io, b):
    case = synth.make_case("tiny", R=4, H=2, d=64, FW=32, B=b, io=io, blocks=(1, 2), gamma="uniform")
    run = Run(case, dev)
    run.build_state()
    before = run.state.clone()
    bad = case.slot_ids.copy()
    bad[2] = case.num_slots  # out of range
    run.slots = torch.from_numpy(bad).to(dev)
    y = to_host(run.forward())
    assert np.all(np.isnan(y[2]))
    good = [0, 1, 3]
    S, Z = record_to_plain(before.cpu().numpy()[case.slot_ids], case.d, case.F)
    ref = run.oracle_forward(S, Z)
    assert normwise_err(pairs(y)[good], ref[good], (2, 3)) <= TOL[io]
    run.commit_active()  # the bad request is skipped, the others commit
    after = run.state.cpu().numpy()
    untouched = np.setdiff1d(np.arange(case.num_slots), case.slot_ids[good])
    assert np.array_equal(after[untouched], before.cpu().numpy()[untouched])


def test_gate_zero_is_block_softmax(dev):
    case = synth.make_case("tiny", R=3, H=2, d=128, FW=64, B=32, io="bf16", blocks=(2, 3),
                           gamma="uniform")
    case.gamma[:] = 0.0
    run = Run(case, dev)
    run.build_state()
    y = pairs(to_host(run.forward()))
    ref = oracle.block_forward_batch(pairs(case.q), pairs(case.k), pairs(case.v), case.w, case.gamma,
                                     np.zeros((3, 2, 128, 128)), np.zeros((3, 2, 128)))
    assert normwise_err(y, ref, (2, 3)) <= TOL["bf16"]


def test_large_gate(dev):
    case = synth.make_case("tiny", R=2, H=2, d=128, FW=64, B=32, io="bf16", blocks=(2, 3),
                           gamma="uniform")
    case.gamma[:] = 1e6
    run = Run(case, dev)
    run.build_state()
    y = pairs(to_host(run.forward()))
    S, Z = run.plain_state()
    assert normwise_err(y, run.oracle_forward(S, Z), (2, 3)) <= TOL["bf16"]


def test_bitwise_deterministic(dev):
    case = synth.make_case("tiny", R=6, H=4, d=128, FW=64, B=32, io="bf16", blocks=(1, 3),
                           gamma="uniform")
    run = Run(case, dev)
    run.build_state()
    y1 = run.forward().clone()
    y2 = run.forward()
    assert torch.equal(y1, y2)
    s0 = run.state.clone()
    run.commit_active()
    s1 = run.state.clone()
    run.state.copy_(s0)
    run.commit_active()
    assert torch.equal(run.state, s1)


@pytest.mark.parametrize("io,d,fw", [("bf16", 128, 64), ("bf16", 64, 128), ("bf16", 128, 32), ("bf16", 128, 128),
                                     ("f32", 64, 32), ("f32", 128, 64)])
def test_prefill_ragged_matches_oracle_build(dev, io, d, fw):
    # ragged prompts of 0..100 tokens (packed), folded in two prefill calls
    # (first part, then the rest, so the second call adds to a non-empty
    # state), against the oracle's state built from scratch over all tokens
    case = synth.make_case("tiny", R=7, H=2, d=d, FW=fw, B=1, io=io, blocks=(0, 100), gamma="uniform")
    lens = case.n_blocks.copy()
    lens[:3] = [0, 1, 33]
    H, F = case.H, case.F
    first = lens // 2
    parts = []
    for lo_frac in (0, 1):
        ks, vs, offs = [], [], [0]
        for r in range(case.R):
            a, b = (0, int(first[r])) if lo_frac == 0 else (int(first[r]), int(lens[r]))
            ks.append(case.prefix_k[r][a:b])
            vs.append(case.prefix_v[r][a:b])
            offs.append(offs[-1] + (b - a))
        parts.append((np.concatenate(ks), np.concatenate(vs), np.array(offs, dtype=np.int32)))
    w = to_device(case.w, io, dev)
    slots = torch.from_numpy(case.slot_ids).to(dev)
    state = bha.new_state(case.num_slots, H, d, fw, dev)
    for kp, vp, offs in parts:
        bha.state_prefill(to_device(kp, io, dev), to_device(vp, io, dev), torch.from_numpy(offs).to(dev), w,
                          state, slots)
    torch.cuda.synchronize()
    S, Z = record_to_plain(state.cpu().numpy()[case.slot_ids], d, F)
    worst = 0.0
    for r in range(case.R):
        n = int(lens[r])
        k_all = case.prefix_k[r][:n].astype(np.float64)
        v_all = case.prefix_v[r][:n].astype(np.float64)
        for h in range(H):
            S_ref, Z_ref = oracle.state_build(k_all[:, h], v_all[:, h], case.w[h])
            if n == 0:
                assert np.all(S[r, h] == 0) and np.all(Z[r, h] == 0)
                continue
            worst = max(worst, normwise_err(S[r, h], S_ref, None), normwise_err(Z[r, h], Z_ref, None))
    _log(f"[prefill] io={io} d={d} FW={fw} lens={lens.tolist()} err {worst:.2e}")
    assert worst <= TOL[io]


@pytest.mark.parametrize("io,R,H", [("bf16", 2048, 1), ("bf16", 2049, 1), ("f32", 585, 14), ("f32", 586, 14)])
def test_prefill_many_requests(dev, io, R, H):
    # up to 2048 requests and 8192 (request, head) pairs the work-groups take
    # the requests longest first (selected in the kernel), beyond either in
    # request order; lengths 0..12 give many ties and empty ranges. Each
    # request's state against the oracle's build over its own tokens.
    case = synth.make_case("tiny", R=R, H=H, d=64, FW=32, B=1, io=io, blocks=(0, 12), gamma="uniform")
    lens = case.n_blocks.copy()
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kp = np.concatenate([case.prefix_k[r][:lens[r]] for r in range(R)])
    vp = np.concatenate([case.prefix_v[r][:lens[r]] for r in range(R)])
    state = bha.new_state(case.num_slots, H, case.d, case.FW, dev)
    bha.state_prefill(to_device(kp, io, dev), to_device(vp, io, dev), torch.from_numpy(offs).to(dev),
                      to_device(case.w, io, dev), state, torch.from_numpy(case.slot_ids).to(dev))
    torch.cuda.synchronize()
    S, Z = record_to_plain(state.cpu().numpy()[case.slot_ids], case.d, case.F)
    worst = 0.0
    for r in range(R):
        n = int(lens[r])
        if n == 0:
            assert not S[r].any() and not Z[r].any()
            continue
        for h in range(H):
            S_ref, Z_ref = oracle.state_build(case.prefix_k[r][:n, h].astype(np.float64),
                                              case.prefix_v[r][:n, h].astype(np.float64), case.w[h])
            worst = max(worst, normwise_err(S[r, h], S_ref, None), normwise_err(Z[r, h], Z_ref, None))
    _log(f"[prefill-many] io={io} R={R} H={H} empty={(lens == 0).sum()} err {worst:.2e}")
    assert worst <= TOL[io]


def test_prefill_long_prompts_fused_kv(dev):
    # prompts of several thousand tokens (many 32-token chunks per work-group),
    # k and v as views of one fused [T][2][H][d] tensor, slots in shuffled order
    case = synth.make_case("tiny", R=4, H=4, d=128, FW=64, B=64, io="bf16", blocks=(20, 70),
                           gamma="uniform")
    lens = case.n_blocks * case.B - np.array([0, 7, 31, 33])[:case.R]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kp = np.concatenate([case.prefix_k[r][:lens[r]] for r in range(case.R)])
    vp = np.concatenate([case.prefix_v[r][:lens[r]] for r in range(case.R)])
    fused = to_device(np.stack([kp, vp], axis=1), "bf16", dev)
    state = bha.new_state(case.num_slots, case.H, case.d, case.FW, dev)
    bha.state_prefill(fused[:, 0], fused[:, 1], torch.from_numpy(offs).to(dev), to_device(case.w, "bf16", dev),
                      state, torch.from_numpy(case.slot_ids).to(dev))
    torch.cuda.synchronize()
    S, Z = record_to_plain(state.cpu().numpy()[case.slot_ids], case.d, case.F)
    S_ref = np.zeros_like(S)
    Z_ref = np.zeros_like(Z)
    k_all = np.ascontiguousarray(np.transpose(kp, (1, 0, 2))).astype(np.float64)
    v_all = np.ascontiguousarray(np.transpose(vp, (1, 0, 2))).astype(np.float64)
    for r in range(case.R):
        for h in range(case.H):
            S_ref[r, h], Z_ref[r, h] = oracle.state_build(k_all[h, offs[r]:offs[r + 1]],
                                                          v_all[h, offs[r]:offs[r + 1]], case.w[h])
    e_s = normwise_err(S, S_ref, (2, 3))
    e_z = normwise_err(Z, Z_ref, (2,))
    _log(f"[prefill-long] lens={lens.tolist()} S err {e_s:.2e} Z err {e_z:.2e}")
    assert e_s <= TOL["bf16"] and e_z <= TOL["bf16"]
    # untouched slots stay zero
    rest = np.setdiff1d(np.arange(case.num_slots), case.slot_ids)
    assert not state.cpu().numpy()[rest].any()


FUSED = [("bf16", 128, 64, 32), ("bf16", 128, 64, 17), ("bf16", 64, 32, 32), ("bf16", 128, 128, 32),
         ("bf16", 64, 128, 8), ("bf16", 128, 64, 40), ("bf16", 128, 64, 64), ("f32", 128, 64, 32),
         ("f32", 64, 32, 5)]


@pytest.mark.parametrize("io,d,fw,b", FUSED)
def test_forward_commit_matches_oracle(dev, io, d, fw, b):
    # last denoising step of a block: the forward from the committed state, then
    # the commit of the block's k, v for the requests flagged in the mask; one
    # request has an out-of-range slot (NaN output, no commit)
    case = synth.make_case("tiny", R=6, H=3, d=d, FW=fw, B=b, io=io, blocks=(0, 3), gamma="uniform")
    run = Run(case, dev)
    run.build_state()
    S0, Z0 = run.plain_state()
    bad = case.slot_ids.copy()
    bad[4] = case.num_slots
    run.slots = torch.from_numpy(bad).to(dev)
    before = run.state.cpu().numpy()
    mask = np.array([1, 0, 1, 1, 1, 1], dtype=np.uint8)
    q, k, v = (to_device(x, io, dev) for x in (case.q, case.k, case.v))
    y = to_host(bha.block_forward_commit(q, k, v, run.w, run.gamma, run.state, run.slots,
                                         commit_mask=torch.from_numpy(mask).to(dev)))
    torch.cuda.synchronize()
    after = run.state.cpu().numpy()
    good = np.array([0, 1, 2, 3, 5])
    assert np.all(np.isnan(y[4]))
    ref = run.oracle_forward(S0, Z0)
    err_f = normwise_err(pairs(y)[good], ref[good], (2, 3))
    S1, Z1 = record_to_plain(after[case.slot_ids], d, case.F)
    S_ref, Z_ref = S0.copy(), Z0.copy()
    oracle.state_commit_batch(S_ref, Z_ref, pairs(case.k), pairs(case.v), case.w.astype(np.float64),
                              nthreads=NTHREADS)
    on = np.array([0, 2, 3, 5])
    err_s = normwise_err(S1[on], S_ref[on], (2, 3))
    err_z = normwise_err(Z1[on], Z_ref[on], (2,))
    _log(f"[fused] io={io} d={d} FW={fw} B={b} forward err {err_f:.2e}, commit S err {err_s:.2e} Z err {err_z:.2e}")
    # masked-off request, the request with the bad slot's own slot, and unused slots are untouched
    keep = np.concatenate([case.slot_ids[[1, 4]], np.setdiff1d(np.arange(case.num_slots), case.slot_ids)])
    assert np.array_equal(after[keep], before[keep])
    assert err_f <= TOL[io] and err_s <= TOL[io] and err_z <= TOL[io]


@pytest.mark.parametrize("io,b", [("bf16", 32), ("bf16", 9), ("f32", 32)])
def test_forward_commit_equals_forward_then_commit(dev, io, b):
    case = synth.make_case("tiny", R=5, H=4, d=128, FW=64, B=b, io=io, blocks=(1, 3), gamma="uniform")
    run = Run(case, dev)
    run.build_state()
    s0 = run.state.clone()
    q, k, v = (to_device(x, io, dev) for x in (case.q, case.k, case.v))
    y_sep = bha.block_forward(q, k, v, run.w, run.gamma, run.state, run.slots).clone()
    bha.state_commit(k, v, run.w, run.state, run.slots)
    s_sep = run.state.clone()
    run.state.copy_(s0)
    y_fused = bha.block_forward_commit(q, k, v, run.w, run.gamma, run.state, run.slots)
    torch.cuda.synchronize()
    # same forward arithmetic; the commit's sums may run in another order
    assert torch.equal(y_fused, y_sep)
    S_f, Z_f = record_to_plain(run.state.cpu().numpy()[case.slot_ids], case.d, case.F)
    S_s, Z_s = record_to_plain(s_sep.cpu().numpy()[case.slot_ids], case.d, case.F)
    assert normwise_err(S_f, S_s, (2, 3)) <= 1e-5 and normwise_err(Z_f, Z_s, (2,)) <= 1e-5


PREFIX = [("bf16", 128, 32), ("bf16", 128, 17), ("bf16", 64, 32), ("bf16", 64, 5), ("bf16", 128, 40),
          ("bf16", 64, 64), ("f32", 128, 32), ("f32", 64, 9), ("f32", 128, 40), ("f32", 64, 64)]


@pytest.mark.parametrize("io,d,b", PREFIX)
def test_prefix_attention_matches_oracle(dev, io, d, b):
    # softmax attention over ragged packed prefixes of 0, 1, 33, 127, 300 and
    # ~330 tokens plus the block; q, k, v as views of one fused tensor and the
    # prefix k, v as views of another
    nb = -(-330 // b)
    case = synth.make_case("tiny", R=6, H=2, d=d, FW=64, B=b, io=io, blocks=(nb, nb + 1), gamma="uniform")
    lens = np.minimum(np.array([0, 1, 33, 127, 300, 10**6]), case.n_blocks * b)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kp = np.concatenate([case.prefix_k[r][:lens[r]] for r in range(case.R)])
    vp = np.concatenate([case.prefix_v[r][:lens[r]] for r in range(case.R)])
    kvp = to_device(np.stack([kp, vp], axis=1), io, dev)  # [T][2][H][d]
    qkv = to_device(np.stack([case.q, case.k, case.v], axis=2), io, dev)  # [R][B][3][H][d]
    y = to_host(bha.prefix_attention(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], kvp[:, 0], kvp[:, 1],
                                     torch.from_numpy(offs).to(dev)))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(y))
    worst = 0.0
    for r in range(case.R):
        for h in range(case.H):
            ref = oracle.prefix_attention(case.q[r, :, h], case.k[r, :, h], case.v[r, :, h],
                                          kp[offs[r]:offs[r + 1], h], vp[offs[r]:offs[r + 1], h])
            worst = max(worst, normwise_err(y[r, :, h], ref, None))
    _log(f"[prefix-attn] io={io} d={d} B={b} lens={lens.tolist()} err {worst:.2e}")
    assert worst <= TOL[io]


def test_prefix_attention_empty_prefix_is_block_softmax(dev):
    # with no prefix rows (total_tokens 0, kp/vp empty) the result is plain
    # softmax attention within the block: the oracle's block forward at gate 0
    case = synth.make_case("tiny", R=3, H=2, d=128, FW=64, B=32, io="bf16", blocks=(0, 0), gamma="uniform")
    q, k, v = (to_device(x, "bf16", dev) for x in (case.q, case.k, case.v))
    empty = torch.empty((0, case.H, case.d), dtype=torch.bfloat16, device=dev)
    offs = torch.zeros(case.R + 1, dtype=torch.int32, device=dev)
    y = to_host(bha.prefix_attention(q, k, v, empty, empty, offs))
    S = np.zeros((case.R, case.H, case.F, case.d))
    Z = np.zeros((case.R, case.H, case.F))
    ref = oracle.block_forward_batch(pairs(case.q), pairs(case.k), pairs(case.v), case.w,
                                     np.zeros(case.H, dtype=np.float32), S, Z, nthreads=NTHREADS)
    err = normwise_err(pairs(y), ref, (2, 3))
    _log(f"[prefix-attn] empty prefix err {err:.2e}")
    assert err <= TOL["bf16"]


def test_prefix_attention_offsets_are_clamped(dev):
    # each request's range is clamped on the device to
    # 0 <= seq_offsets[r] <= seq_offsets[r+1] <= total_tokens; every request's
    # output equals a one-request call over its clamped range
    case = synth.make_case("tiny", R=4, H=2, d=64, FW=64, B=16, io="bf16", blocks=(6, 6), gamma="uniform")
    kp = np.concatenate([case.prefix_k[r] for r in range(case.R)])
    vp = np.concatenate([case.prefix_v[r] for r in range(case.R)])
    T = kp.shape[0]
    q, k, v = (to_device(x, "bf16", dev) for x in (case.q, case.k, case.v))
    kd, vd = to_device(kp, "bf16", dev), to_device(vp, "bf16", dev)
    bad = [-5, 40, 20, T + 50, T + 100]
    clamped = [(0, 40), (40, 40), (20, T), (T, T)]
    y = bha.prefix_attention(q, k, v, kd, vd, torch.tensor(bad, dtype=torch.int32, device=dev))
    for r, (a, b) in enumerate(clamped):
        y_r = bha.prefix_attention(q[r:r + 1], k[r:r + 1], v[r:r + 1], kd, vd,
                                   torch.tensor([a, b], dtype=torch.int32, device=dev))
        torch.cuda.synchronize()
        assert torch.equal(y[r], y_r[0]), r


@pytest.mark.parametrize("io,d,b", [("bf16", 128, 32), ("bf16", 64, 32), ("bf16", 128, 48), ("f32", 128, 32),
                                    ("f32", 64, 48)])
def test_prefix_attention_split_matches_oracle(dev, io, d, b):
    # few pairs with long prefixes: the keys of each pair are split over several
    # work-groups (the request with no prefix leaves some splits without keys);
    # the same call with a workspace too small to split, and with one that
    # allows half the splits, agree with the oracle too
    case = synth.make_case("tiny", R=3, H=2, d=d, FW=64, B=b, io=io, blocks=(20000 // b + 1, 20000 // b + 1),
                           gamma="uniform")
    lens = np.array([0, 20000, 40])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kp = np.concatenate([case.prefix_k[r][:lens[r]] for r in range(case.R)])
    vp = np.concatenate([case.prefix_v[r][:lens[r]] for r in range(case.R)])
    T = kp.shape[0]
    q, k, v = (to_device(x, io, dev) for x in (case.q, case.k, case.v))
    kd, vd, od = to_device(kp, io, dev), to_device(vp, io, dev), torch.from_numpy(offs).to(dev)
    full = bha.prefix_attention_workspace(case.R, case.H, d, b, T, dtype=q.dtype)
    part = case.R * case.H * ((b + 31) // 32) * (32 * d + 64) * 4
    assert full > 0 and full % part == 0
    n_split = full // part
    assert n_split >= 4
    results = {}
    for name, ws_bytes in (("full", full), ("half", (n_split // 2) * part), ("none", 16)):
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        results[name] = to_host(bha.prefix_attention(q, k, v, kd, vd, od, workspace=ws))
    torch.cuda.synchronize()
    for name, y in results.items():
        assert np.all(np.isfinite(y)), name
        worst = 0.0
        for r in range(case.R):
            for h in range(case.H):
                ref = oracle.prefix_attention(case.q[r, :, h], case.k[r, :, h], case.v[r, :, h],
                                              kp[offs[r]:offs[r + 1], h], vp[offs[r]:offs[r + 1], h])
                worst = max(worst, normwise_err(y[r, :, h], ref, None))
        _log(f"[prefix-attn split] io={io} d={d} workspace={name} ({n_split} splits in full) "
             f"lens={lens.tolist()} err {worst:.2e}")
        assert worst <= TOL[io]


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_normaliser_halves_count_the_tokens(dev, io):
    # each half of phi sums to 1 per token, so each half of Z sums to the
    # number of tokens folded in: a ragged prefill (0..300 tokens), then a
    # 32-token block commit, then a fused forward + commit of another block
    R, H, d, FW, B = 7, 3, 128, 64, 32
    case = synth.make_case("tiny", R=R, H=H, d=d, FW=FW, B=1, io=io, blocks=(0, 300), gamma="uniform")
    lens = case.n_blocks.copy()
    lens[:2] = [0, 1]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kp = np.concatenate([case.prefix_k[r][:lens[r]] for r in range(R)])
    vp = np.concatenate([case.prefix_v[r][:lens[r]] for r in range(R)])
    w = to_device(case.w, io, dev)
    slots = torch.from_numpy(case.slot_ids).to(dev)
    state = bha.new_state(case.num_slots, H, d, FW, dev)
    bha.state_prefill(to_device(kp, io, dev), to_device(vp, io, dev), torch.from_numpy(offs).to(dev), w, state,
                      slots)
    g = np.random.default_rng(3)
    blk = [synth.bf16_to_f32(synth.bf16_bits(g.standard_normal((R, B, H, d)).astype(np.float32)))
           for _ in range(5)]
    q1, k1, v1, k2, v2 = (to_device(x, io, dev) for x in blk)
    bha.state_commit(k1, v1, w, state, slots)
    out = torch.empty_like(q1)
    bha.block_forward_commit(q1, k2, v2, w, torch.from_numpy(case.gamma).to(dev), state, slots, out=out)
    torch.cuda.synchronize()
    _, Z = record_to_plain(state.cpu().numpy()[case.slot_ids], d, 2 * FW)
    n_tok = (lens + 2 * B).astype(np.float64)[:, None]
    err = max(np.abs(Z[..., :FW].sum(-1) - n_tok).max(), np.abs(Z[..., FW:].sum(-1) - n_tok).max())
    rel = err / n_tok.max()
    _log(f"[Z halves] io={io} max |sum Z half - tokens| {err:.2e} ({rel:.1e} of {int(n_tok.max())})")
    assert rel <= 1e-5


def test_large_token_strides_take_the_fp32_kernels(dev):
    # bf16 tokens 2^25 elements (64 MiB) apart: past the 32-bit in-chunk
    # offsets of the matrix-core kernels, so prefill, forward, commit and
    # prefix attention run on the fp32-arithmetic kernels; each against the
    # oracle
    R, H, d, FW, B, TS = 2, 1, 64, 32, 3, 1 << 25
    case = synth.make_case("tiny", R=R, H=H, d=d, FW=FW, B=B, io="bf16", blocks=(1, 1), gamma="uniform")
    F = case.F
    buf = torch.zeros(R * B * TS, dtype=torch.bfloat16, device=dev)
    pbuf = torch.zeros(R * B * TS, dtype=torch.bfloat16, device=dev)

    def tok_view(i, x):  # [R][B][H][d], the i-th H*d run at the start of each token's slot
        t = buf.as_strided((R, B, H, d), (B * TS, TS, d, 1), i * H * d)
        if x is not None:
            t.copy_(to_device(x, "bf16", dev))
        return t

    q, k, v = (tok_view(i, x) for i, x in enumerate((case.q, case.k, case.v)))
    out = tok_view(3, None)
    kp_h = np.concatenate([case.prefix_k[r] for r in range(R)])
    vp_h = np.concatenate([case.prefix_v[r] for r in range(R)])
    T = kp_h.shape[0]
    kp = pbuf.as_strided((T, H, d), (TS, d, 1), 0)
    vp = pbuf.as_strided((T, H, d), (TS, d, 1), H * d)
    kp.copy_(to_device(kp_h, "bf16", dev))
    vp.copy_(to_device(vp_h, "bf16", dev))
    offs_h = np.concatenate([[0], np.cumsum([case.prefix_k[r].shape[0] for r in range(R)])]).astype(np.int32)
    offs = torch.from_numpy(offs_h).to(dev)
    w = to_device(case.w, "bf16", dev)
    gamma = torch.from_numpy(case.gamma).to(dev)
    slots = torch.from_numpy(case.slot_ids).to(dev)
    state = bha.new_state(case.num_slots, H, d, FW, dev)

    def plain():
        torch.cuda.synchronize()
        return record_to_plain(state.cpu().numpy()[case.slot_ids], d, F)

    def built(with_block):
        S = np.zeros((R, H, F, d))
        Z = np.zeros((R, H, F))
        for r in range(R):
            for h in range(H):
                kk, vv = case.prefix_k[r][:, h], case.prefix_v[r][:, h]
                if with_block:
                    kk, vv = np.concatenate([kk, case.k[r, :, h]]), np.concatenate([vv, case.v[r, :, h]])
                S[r, h], Z[r, h] = oracle.state_build(kk.astype(np.float64), vv.astype(np.float64), case.w[h])
        return S, Z

    errs = {}
    bha.state_prefill(kp, vp, offs, w, state, slots)
    S, Z = plain()
    S_ref, Z_ref = built(False)
    errs["prefill"] = max(normwise_err(S, S_ref, (2, 3)), normwise_err(Z, Z_ref, (2,)))
    bha.block_forward(q, k, v, w, gamma, state, slots, out=out)
    y = to_host(out)
    ref = oracle.block_forward_batch(pairs(case.q), pairs(case.k), pairs(case.v), case.w, case.gamma, S, Z,
                                     nthreads=NTHREADS)
    errs["forward"] = normwise_err(pairs(y), ref, (2, 3))
    bha.state_commit(k, v, w, state, slots)
    S, Z = plain()
    S_ref, Z_ref = built(True)
    errs["commit"] = max(normwise_err(S, S_ref, (2, 3)), normwise_err(Z, Z_ref, (2,)))
    bha.prefix_attention(q, k, v, kp, vp, offs, out=out)
    y = to_host(out)
    errs["prefix_attention"] = max(
        normwise_err(y[r, :, h], oracle.prefix_attention(case.q[r, :, h], case.k[r, :, h], case.v[r, :, h],
                                                         kp_h[offs_h[r]:offs_h[r + 1], h],
                                                         vp_h[offs_h[r]:offs_h[r + 1], h]), None)
        for r in range(R) for h in range(H))
    _log(f"[large strides] {', '.join(f'{k_} err {e:.2e}' for k_, e in errs.items())}")
    assert max(errs.values()) <= TOL["bf16"]


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_state_is_consistent_across_block_sizes(dev, io):
    # blocks of 32, 16, 8, 1, 64 and 5 tokens committed in turn into one state
    # (each commit a separate call with its own B, both kernel families), then
    # forwards with B = 16 and B = 48 from it: the state equals the oracle's
    # build over all 126 tokens, and each forward the oracle's forward from
    # that state -- the state does not depend on how the prefix was cut into
    # blocks
    R, H, d, FW = 3, 2, 128, 64
    sizes = [32, 16, 8, 1, 64, 5]
    n = sum(sizes)
    case = synth.make_case("tiny", R=R, H=H, d=d, FW=FW, B=n, io=io, blocks=(1, 1), gamma="uniform")
    w = to_device(case.w, io, dev)
    slots = torch.from_numpy(case.slot_ids).to(dev)
    state = bha.new_state(case.num_slots, H, d, FW, dev)
    pk = np.stack([case.prefix_k[r][:n] for r in range(R)])  # [R][n][H][d]
    pv = np.stack([case.prefix_v[r][:n] for r in range(R)])
    t0 = 0
    for b in sizes:
        bha.state_commit(to_device(pk[:, t0:t0 + b], io, dev), to_device(pv[:, t0:t0 + b], io, dev), w, state, slots)
        t0 += b
    torch.cuda.synchronize()
    S, Z = record_to_plain(state.cpu().numpy()[case.slot_ids], d, case.F)
    worst_s = 0.0
    for r in range(R):
        for h in range(H):
            S_ref, Z_ref = oracle.state_build(pk[r, :, h], pv[r, :, h], case.w[h])
            worst_s = max(worst_s, normwise_err(S[r, h], S_ref, None), normwise_err(Z[r, h], Z_ref, None))
    worst_f = 0.0
    for b in (16, 48):
        q, k, v = (case.q[:, :b], case.k[:, :b], case.v[:, :b])
        y = to_host(bha.block_forward(*(to_device(np.ascontiguousarray(x), io, dev) for x in (q, k, v)), w,
                                      torch.from_numpy(case.gamma).to(dev), state, slots))
        ref = oracle.block_forward_batch(pairs(q), pairs(k), pairs(v), case.w, case.gamma, S, Z, nthreads=NTHREADS)
        worst_f = max(worst_f, normwise_err(pairs(y), ref, (2, 3)))
    _log(f"[block sizes] io={io} commits of {sizes}: state err {worst_s:.2e}; forwards B=16, 48 err {worst_f:.2e}")
    assert worst_s <= TOL[io] and worst_f <= TOL[io]


GQA = [("bf16", 128, 64, 32, 2), ("bf16", 128, 64, 17, 4), ("bf16", 64, 32, 32, 4), ("bf16", 128, 32, 9, 2),
       ("bf16", 128, 128, 32, 2), ("bf16", 128, 128, 32, 4), ("bf16", 128, 64, 48, 2), ("f32", 128, 64, 8, 2),
       ("bf16", 128, 64, 32, 8), ("bf16", 64, 32, 17, 8), ("bf16", 128, 128, 32, 8), ("bf16", 64, 64, 32, 8),
       ("bf16", 128, 32, 5, 8)]


@pytest.mark.parametrize("io,d,fw,b,g", GQA)
def test_forward_gqa_matches_oracle(dev, io, d, fw, b, g):
    # H = 2 g query heads over 2 K/V heads; the K/V heads' states built by
    # chained commits (bha_state_commit over the K/V heads); query head h reads
    # K/V head h // g. Against the oracle from the same fp32 state bytes, and
    # against bha_block_forward on K/V, W and states repeated for every query
    # head. Request 3 has an out-of-range slot (NaN rows for all its heads).
    HK, R = 2, 5
    H = HK * g
    case = synth.make_case("tiny", R=R, H=H, d=d, FW=fw, B=b, io=io, blocks=(0, 3), gamma="uniform")
    kv_w = to_device(case.w[:HK], io, dev)
    slots_np = case.slot_ids.copy()
    state = bha.new_state(case.num_slots, HK, d, fw, dev)
    for i in range(int(case.n_blocks.max(initial=0))):
        act = np.nonzero(case.n_blocks > i)[0]
        kb = np.stack([case.prefix_k[r][i * b:(i + 1) * b, :HK] for r in act])
        vb = np.stack([case.prefix_v[r][i * b:(i + 1) * b, :HK] for r in act])
        bha.state_commit(to_device(kb, io, dev), to_device(vb, io, dev), kv_w, state,
                         torch.from_numpy(slots_np[act]).to(dev))
    torch.cuda.synchronize()
    bad = slots_np.copy()
    bad[3] = case.num_slots
    slots = torch.from_numpy(bad).to(dev)
    q = to_device(case.q, io, dev)
    k, v = (to_device(np.ascontiguousarray(x[:, :, :HK]), io, dev) for x in (case.k, case.v))
    gamma = torch.from_numpy(case.gamma).to(dev)
    y = bha.block_forward_gqa(q, k, v, kv_w, gamma, state, slots)
    # the same through the one-K/V-head-per-query-head call on repeated operands
    rep = lambda t: t.repeat_interleave(g, dim=2)
    state_rep = state.view(case.num_slots, HK, -1).repeat_interleave(g, dim=1).contiguous()
    y_mha = bha.block_forward(q, rep(k).contiguous(), rep(v).contiguous(),
                              kv_w.repeat_interleave(g, dim=0).contiguous(), gamma, state_rep, slots)
    torch.cuda.synchronize()
    yh = to_host(y)
    assert np.all(np.isnan(yh[3]))
    good = [0, 1, 2, 4]
    S, Z = record_to_plain(state.cpu().numpy()[slots_np], d, case.F)  # [R][HK][F][d]
    worst = 0.0
    for r in good:
        for h in range(H):
            hk = h // g
            ref = oracle.block_forward(case.q[r, :, h], case.k[r, :, hk], case.v[r, :, hk], case.w[hk], case.gamma[h],
                                       S[r, hk], Z[r, hk])
            worst = max(worst, normwise_err(yh[r, :, h], ref, None))
    same = torch.equal(y[good], y_mha[good])
    e_mha = normwise_err(yh[good], to_host(y_mha)[good], (1, 3))
    _log(f"[gqa] io={io} d={d} FW={fw} B={b} G={g}: err {worst:.2e}; vs repeated-head forward "
         f"{'identical' if same else f'{e_mha:.1e}'}")
    assert worst <= TOL[io]
    # both calls on the matrix-core kernels run the same arithmetic per query
    # head; otherwise (B > 32 with G > 1, or G = 8 at FW = 128: the fp32
    # kernel) the two paths agree to the bf16 bar
    both_mfma = io == "bf16" and b <= 32 and (g in (2, 4) or (g == 8 and fw <= 64))
    if both_mfma:
        assert same
    else:
        assert e_mha <= TOL[io]


@pytest.mark.parametrize("io,b", [("bf16", 32), ("bf16", 48), ("f32", 16)])
def test_pending_hip_error_does_not_change_a_commit(dev, io, b):
    # An error left pending on the thread by an unrelated HIP call (here an
    # invalid hipSetDevice) must not decide what a library call does: one
    # bha_state_commit after it returns BHA_OK and folds the block in exactly
    # once -- bit-identical to the same commit with nothing pending. The HIP
    # runtime's symbols are resolved through libbha.so's own dependencies, so
    # the error is set in the runtime the library uses.
    import ctypes

    case = synth.make_case("tiny", R=4, H=2, d=128, FW=64, B=b, io=io, blocks=(1, 2), gamma="uniform")
    run = Run(case, dev)
    run.build_state()
    k, v = to_device(case.k, io, dev), to_device(case.v, io, dev)
    ref = run.state.clone()
    bha.state_commit(k, v, run.w, ref, run.slots)
    com = bha.prepare_commit(k, v, run.w, run.state, run.slots)
    torch.cuda.synchronize()
    hip = bha.load_library()
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipGetLastError.argtypes = []
    hip.hipGetLastError.restype = ctypes.c_int
    hip.hipGetLastError()
    assert hip.hipSetDevice(1 << 20) != 0  # leaves hipErrorInvalidDevice pending
    try:
        com()  # raises BhaError unless the call returns BHA_OK
    finally:
        pending = hip.hipGetLastError()  # cleared before torch looks at it
    torch.cuda.synchronize()
    _log(f"[pending error] io={io} B={b}: commit returned BHA_OK with error {pending} pending before it")
    assert torch.equal(run.state, ref)
