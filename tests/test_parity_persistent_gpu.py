"""GPU parity of the persistent forward kernels, and of the commit, at production grid sizes.

The matrix-core forwards run a persistent grid of (resident work-groups per
CU) x CUs work-groups, each taking pairs b, b + G, b + 2G, ... with the next
pair's slot id, operands and state slice issued ahead of the current pair's
arithmetic. A small batch gives every work-group one pair and never reaches
that loop; these tests run 256 requests x 16 heads (4,096 pairs, or 512 to
2,048 (request, K/V head) units), so every work-group takes several (eight
query heads per K/V head: 512 requests for that), and
compare EVERY pair with the fp64 oracle computed from the same fp32 state
bytes the kernel read. One request carries an out-of-range slot in the middle
of the batch: its rows must come out NaN while the pairs around it, whose
look-ahead loads run through it, stay exact.

Also the feature map at 256 x 32 tokens x 16 heads (several tiles per
work-group) and with a ragged last tile. Covered: blocks of 48 and 64 tokens (two 32-token query tiles) at FW = 32, 64
and 128 (d = 128, and d = 64 at FW = 64 and 128); grouped K/V heads with 2, 4
and 8 query heads per K/V head; the one-tile forward at 64, 256 and 512
requests (d = 128) and d = 64 at FW = 32, 64 and 128; the commit at 256 and
512 requests with skipped requests scattered through the batch.
States: one ragged prefill over 0..4 blocks of 32 tokens per request (zero
records included). Bar: normwise 2e-2 (bf16 I/O, fp32 accumulation).
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
R, H, D = 256, 16, 128
BAD = 77  # request given an out-of-range slot (77 mod R in smaller batches)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    bha.load_library()
    return torch.device("cuda:0")


def _states(dev, fw, hk, R=R, d=D, nq=H):
    """Slots, W (hk heads), gates (nq query heads), and states built by one ragged prefill."""
    case = synth.make_case("decode256", R=R, with_prefix=False, with_qkv=False, FW=fw, d=d)
    nb = np.random.default_rng(5).integers(0, 5, size=R)
    w, _ = synth.device_layer_params("decode256", 0, dev, FW=fw, H=hk, d=d)
    _, gamma = synth.device_layer_params("decode256", 0, dev, FW=fw, H=nq, d=d)
    slots = torch.from_numpy(case.slot_ids).to(dev)
    state = bha.new_state(case.num_slots, hk, d, fw, dev)
    pk, pv, offs = synth.device_packed_prefix("decode256", nb, dev, FW=fw, H=hk, d=d)
    bha.state_prefill(pk, pv, offs, w, state, slots)
    torch.cuda.synchronize()
    bad = case.slot_ids.copy()
    bad[BAD % R] = case.num_slots
    return case, w, gamma, slots, torch.from_numpy(bad).to(dev), state


def _check_all_pairs(y, q, k, v, w, gamma, state, slot_ids, g, fw, tag):
    R, nq, d = q.shape[0], q.shape[2], q.shape[3]
    hk = nq // g
    rec = state.cpu().numpy()[slot_ids]  # [R][hk][rec]
    S, Z = record_to_plain(rec, d, 2 * fw)
    rep = lambda a: np.repeat(a, g, axis=1)  # noqa: E731  K/V head -> its query heads
    kq = rep(pairs(to_host(k)))
    vq = rep(pairs(to_host(v)))
    ref = oracle.block_forward_batch(pairs(to_host(q)), kq, vq, np.repeat(to_host(w), g, axis=0),
                                     gamma.cpu().numpy().astype(np.float64), rep(S), rep(Z), nthreads=NTHREADS)
    yh = pairs(to_host(y))  # [R][H][B][d]
    assert np.all(np.isnan(yh[BAD % R])), f"[{tag}] request with an out-of-range slot must be NaN"
    good = np.ones(R, dtype=bool)
    good[BAD % R] = False
    assert np.all(np.isfinite(yh[good])), f"[{tag}] non-finite outputs outside the bad request"
    err = normwise_err(yh[good], ref[good], (2, 3))
    cus = torch.cuda.get_device_properties(y.device).multi_processor_count
    print(f"[{tag}] {R * hk} units on a persistent grid over {cus} CUs: err {err:.2e} over all "
          f"{int(good.sum()) * nq} (request, query head) pairs", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("d,fw,b", [(128, 32, 48), (128, 32, 64), (128, 64, 48), (128, 64, 64), (128, 128, 48),
                                    (128, 128, 64), (64, 64, 64), (64, 128, 48)])
def test_two_tile_forward_every_pair(dev, d, fw, b):
    case, w, gamma, _, slots_bad, state = _states(dev, fw, H, d=d)
    q, k, v = synth.device_step_qkv("decode256", 0, R, dev, FW=fw, B=b, d=d)
    y = bha.block_forward(q, k, v, w, gamma, state, slots_bad)
    torch.cuda.synchronize()
    _check_all_pairs(y, q, k, v, w, gamma, state, case.slot_ids, 1, fw, f"two-tile d={d} FW={fw} B={b}")


@pytest.mark.parametrize("d,fw,hk", [(128, 64, 8), (128, 64, 4), (128, 64, 2), (128, 32, 4), (128, 32, 2),
                                     (128, 128, 8), (128, 128, 4), (64, 64, 2), (64, 32, 2), (64, 64, 4)])
def test_grouped_forward_every_pair(dev, d, fw, hk):
    g = H // hk
    case, w, gamma, _, slots_bad, state = _states(dev, fw, hk, d=d)
    q = synth.device_step_qkv("decode256", 0, R, dev, FW=fw, d=d)[0]
    _, k, v = synth.device_step_qkv("decode256", 0, R, dev, FW=fw, H=hk, d=d)
    y = bha.block_forward_gqa(q, k, v, w, gamma, state, slots_bad)
    torch.cuda.synchronize()
    _check_all_pairs(y, q, k, v, w, gamma, state, case.slot_ids, g, fw, f"grouped d={d} FW={fw} G={g}")


@pytest.mark.parametrize("d,fw", [(128, 64), (64, 32)])
def test_eight_head_groups_several_units_per_work_group(dev, d, fw):
    # eight query heads per K/V head: at 256 requests every work-group of the
    # two-per-CU grid has one unit (the variant that issues the slice after
    # the operands); at 512 requests each takes two, through the loop that
    # loads the next unit's slice during the current unit's last head
    g, hk, nreq = 8, H // 8, 512
    case, w, gamma, _, slots_bad, state = _states(dev, fw, hk, R=nreq, d=d)
    q = synth.device_step_qkv("decode256", 0, nreq, dev, FW=fw, d=d)[0]
    _, k, v = synth.device_step_qkv("decode256", 0, nreq, dev, FW=fw, H=hk, d=d)
    y = bha.block_forward_gqa(q, k, v, w, gamma, state, slots_bad)
    torch.cuda.synchronize()
    _check_all_pairs(y, q, k, v, w, gamma, state, case.slot_ids, g, fw, f"grouped d={d} FW={fw} G={g} R={nreq}")


@pytest.mark.parametrize("nheads,nreq", [(20, 128), (12, 192)])
def test_one_tile_forward_every_pair_other_head_counts(dev, nheads, nreq):
    # the persistent grid is rounded down to a multiple of H so that a
    # work-group keeps one head: at one wave per SIMD (d = 128, 256 CUs)
    # 20 heads give 240 work-groups (10 or 11 pairs each) and 12 give 252
    # (9 or 10), so work-groups end after different numbers of pairs
    case, w, gamma, _, slots_bad, state = _states(dev, 64, nheads, R=nreq, nq=nheads)
    q, k, v = synth.device_step_qkv("decode256", 0, nreq, dev, H=nheads)
    y = bha.block_forward(q, k, v, w, gamma, state, slots_bad)
    torch.cuda.synchronize()
    _check_all_pairs(y, q, k, v, w, gamma, state, case.slot_ids, 1, 64, f"one-tile H={nheads} R={nreq}")


def _draw_grid_case(seed):
    rng = np.random.default_rng(9100 + seed)
    d = int(rng.choice([64, 128]))
    fw = int(rng.choice([32, 64]))
    g = int(rng.choice([1, 1, 2, 4, 8]))
    b = int(rng.integers(1, 65 if g == 1 else 33))
    hk = int(rng.integers(8, 25)) if g == 1 else int(rng.integers(1, 32 // g + 1))
    nreq = int(rng.integers(64, 401))
    return dict(d=d, fw=fw, g=g, b=b, hk=hk, nq=hk * g, nreq=nreq)


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_on_production_grids(dev, seed):
    # seeded shapes whose pair counts fall on both sides of the
    # one-wave-per-SIMD threshold (8 pairs per CU), with head counts that do
    # not divide the grid evenly: the one-tile, two-tile and grouped forwards
    # (1, 2, 4 or 8 query heads per K/V head), every pair against the oracle
    c = _draw_grid_case(seed)
    d, fw, g, b, hk, nq, nreq = c["d"], c["fw"], c["g"], c["b"], c["hk"], c["nq"], c["nreq"]
    case, w, gamma, _, slots_bad, state = _states(dev, fw, hk, R=nreq, d=d, nq=nq)
    q = synth.device_step_qkv("decode256", 0, nreq, dev, FW=fw, d=d, B=b, H=nq)[0]
    _, k, v = synth.device_step_qkv("decode256", 0, nreq, dev, FW=fw, d=d, B=b, H=hk)
    if g == 1:
        y = bha.block_forward(q, k, v, w, gamma, state, slots_bad)
    else:
        y = bha.block_forward_gqa(q, k, v, w, gamma, state, slots_bad)
    torch.cuda.synchronize()
    _check_all_pairs(y, q, k, v, w, gamma, state, case.slot_ids, g, fw, f"random grid case {seed}: {c}")


@pytest.mark.parametrize("d,fw,nreq,b", [(128, 64, 256, 32), (128, 64, 255, 31), (64, 32, 256, 32)])
def test_feature_map_every_token(dev, d, fw, nreq, b):
    # the persistent feature map at production size: 128-token (64 at
    # d = 64) tiles x 16 heads on two waves per SIMD, two units per
    # work-group (some one, with a ragged last tile, at 255 x 31 tokens);
    # every token and head against the oracle's phi
    case = synth.make_case("decode256", R=nreq, with_prefix=False, with_qkv=False, FW=fw, d=d, B=b)
    w, _ = synth.device_layer_params("decode256", 0, dev, FW=fw, d=d)
    x = synth.device_step_qkv("decode256", 0, nreq, dev, FW=fw, d=d, B=b)[0]
    phi = to_host(bha.feature_map(x, w))  # [R][B][H][2 FW]
    xh, wh = to_host(x), to_host(w)
    ref = np.empty_like(phi)
    for h in range(H):
        ref[:, :, h] = oracle.phi(xh[:, :, h].reshape(-1, d), wh[h]).reshape(nreq, b, 2 * fw)
    err = normwise_err(phi, ref, (3,))
    print(f"[feature map d={d} FW={fw} {nreq} x {b} tokens x {H} heads] err {err:.2e}", flush=True)
    assert err <= 1e-5


@pytest.mark.parametrize("d,fw,nreq", [(128, 64, 256), (128, 64, 512), (128, 64, 64), (64, 64, 512),
                                       (64, 32, 256), (64, 128, 256), (64, 32, 64)])
def test_one_tile_forward_every_pair(dev, d, fw, nreq):
    # the headline kernel (B = 32, FW = 64) at the decode256 grid (one
    # four-wave work-group per CU, 16 pairs each), at 512 requests (32 pairs
    # each) and at 64 requests (two work-groups per CU, 2 pairs each); d = 64
    # (two-wave work-groups, two or four per CU) at FW = 32, 64 and 128; every
    # pair
    case, w, gamma, _, slots_bad, state = _states(dev, fw, H, R=nreq, d=d)
    q, k, v = synth.device_step_qkv("decode256", 0, nreq, dev, d=d, FW=fw)
    y = bha.block_forward(q, k, v, w, gamma, state, slots_bad)
    torch.cuda.synchronize()
    _check_all_pairs(y, q, k, v, w, gamma, state, case.slot_ids, 1, fw, f"one-tile d={d} FW={fw} B=32 R={nreq}")


@pytest.mark.parametrize("d,fw,nreq", [(128, 64, 256), (128, 32, 256), (128, 64, 512), (64, 64, 512), (64, 32, 256)])
def test_commit_every_pair_with_skipped_requests(dev, d, fw, nreq):
    # bha_state_commit at production size with requests whose slots are out
    # of range (negative or past the pool) scattered through the batch:
    # nothing of theirs is written, every record outside the committed
    # requests stays unchanged bit for bit, and every committed pair matches
    # the oracle's commit from the same pre-commit bytes.
    case, w, _, _, _, state = _states(dev, fw, H, R=nreq, d=d)
    bads = np.array([3, 77, 78, 130, nreq - 1])
    slot_np = case.slot_ids.copy()
    slot_np[bads] = [-1, case.num_slots, case.num_slots + 5, -7, 2**31 - 1]
    _, k, v = synth.device_step_qkv("decode256", 0, nreq, dev, FW=fw, d=d)
    pre = state.cpu().numpy()
    bha.state_commit(k, v, w, state, torch.from_numpy(slot_np).to(dev))
    torch.cuda.synchronize()
    post = state.cpu().numpy()
    good = np.setdiff1d(np.arange(nreq), bads)
    touched = case.slot_ids[good]
    untouched = np.setdiff1d(np.arange(case.num_slots), touched)
    assert np.array_equal(post[untouched].view(np.uint32), pre[untouched].view(np.uint32)), \
        "records outside the committed requests changed"
    F = 2 * fw
    S, Z = record_to_plain(pre[touched], d, F)
    S, Z = np.ascontiguousarray(S), np.ascontiguousarray(Z)
    oracle.state_commit_batch(S, Z, np.ascontiguousarray(pairs(to_host(k))[good]),
                              np.ascontiguousarray(pairs(to_host(v))[good]), to_host(w), nthreads=NTHREADS)
    S2, Z2 = record_to_plain(post[touched], d, F)
    err = max(normwise_err(S2, S, (2, 3)), normwise_err(Z2, Z, (2,)))
    print(f"[commit d={d} FW={fw} R={nreq}] {len(good) * H} pairs committed, "
          f"{len(bads)} requests skipped: err {err:.2e}", flush=True)
    assert err <= TOL
