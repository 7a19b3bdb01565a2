"""GPU invariants of the block-hybrid kernels (no oracle arithmetic needed).

* Pair isolation: every (request, head) pair is independent in the forward
  and the commit, so a NaN planted in one pair's inputs (a key, a query row,
  its state record) must show up in that pair's outputs only, and every other
  output must be bit-identical to the clean run.
* Slot indirection: permuting the requests of a batch (their Q, K, V rows and
  slot ids together) permutes the outputs and leaves every state record as it
  was -- bit for bit.
* Checkpoint round trip: a request's state is its (d + 1) F H float32 record
  per block-hybrid layer (the S and Z states of the gist.science explainer,
  "Architecture Design"), so saving the records after block n, restoring them
  into a fresh state pool under other slots, and continuing must give the
  same outputs and states, bit for bit, as the uninterrupted run.
* Store policy: the commit and the fused last step write the state back
  with device-scope non-temporal stores from 16 pairs per CU (at F <= 128)
  and with plain non-temporal stores below that; a batch that takes the
  first path must give the same states and outputs, bit for bit, as its two
  halves committed separately (each taking the second). The feature map
  stores its rows at device scope up to 4 units (128 tokens x head) per CU
  at d = 128, FW = 64, and plainly above: a batch above that must give the
  rows of its halves, bit for bit.
Shapes: the decode-like 64 x 16 batch on the matrix-core path (d = 128,
FW = 64, B = 32), the two-tile path (B = 48) and the fp32 path.
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


CASES = [("bf16", 32), ("bf16", 48), ("f32", 32)]


def _batch(dev, io, b, R=64, H=16, FW=64):
    over = dict(FW=FW, B=b, io=io, H=H)
    case = synth.make_case("decode256", R=R, with_prefix=False, with_qkv=False, **over)
    nb = np.random.default_rng(3).integers(0, 6, size=R)
    w, gamma = synth.device_layer_params("decode256", 0, dev, **over)
    slots = torch.from_numpy(case.slot_ids).to(dev)
    state = bha.new_state(case.num_slots, H, 128, FW, dev)
    pk, pv, offs = synth.device_packed_prefix("decode256", nb, dev, **dict(over, B=32))
    bha.state_prefill(pk, pv, offs, w, state, slots)
    q, k, v = (t.contiguous() for t in synth.device_step_qkv("decode256", 0, R, dev, **over))
    torch.cuda.synchronize()
    return case, w, gamma, slots, state, q, k, v


def _nan_mask(t):
    return torch.isnan(t.float())


@pytest.mark.parametrize("io,b", CASES)
def test_nan_stays_in_its_pair(dev, io, b):
    case, w, gamma, slots, state, q, k, v = _batch(dev, io, b)
    R, H = case.R, case.H
    y0 = bha.block_forward(q, k, v, w, gamma, state, slots)
    st0 = state.clone()
    bha.state_commit(k, v, w, st0, slots)
    # plant: a NaN key in pair (5, 3); a NaN query row 7 in pair (20, 9); a NaN
    # in the state record of pair (41, 0)
    k2, q2, state2 = k.clone(), q.clone(), state.clone()
    k2[5, b // 2, 3, 17] = float("nan")
    q2[20, 7, 9, 100] = float("nan")
    rec = state2.view(case.num_slots, H, -1)
    rec[int(case.slot_ids[41]), 0, 1234] = float("nan")
    y1 = bha.block_forward(q2, k2, v, w, gamma, state2, slots)
    torch.cuda.synchronize()
    expect = torch.zeros_like(y0, dtype=torch.bool)
    expect[5, :, 3] = True      # every query of the pair reads the poisoned key
    expect[20, 7, 9] = True     # only the poisoned query row
    expect[41, :, 0] = True     # every query of the pair reads the poisoned record
    got = _nan_mask(y1)
    assert torch.equal(got.any(dim=-1), expect.any(dim=-1)), "NaN outside the planted pairs (forward)"
    assert torch.equal(y1[~expect], y0[~expect]), "clean outputs changed (forward)"
    # the commit: the poisoned key's record becomes NaN, the poisoned record
    # stays NaN, every other record is bit-identical to the clean commit
    bha.state_commit(k2, v, w, state2, slots)
    torch.cuda.synchronize()
    recs0 = st0.view(case.num_slots, H, -1)
    recs1 = state2.view(case.num_slots, H, -1)
    bad = torch.zeros(case.num_slots, H, dtype=torch.bool, device=dev)
    bad[int(case.slot_ids[5]), 3] = True
    bad[int(case.slot_ids[41]), 0] = True
    assert torch.equal(torch.isnan(recs1).any(dim=-1), bad), "NaN outside the planted records (commit)"
    assert torch.equal(recs1[~bad], recs0[~bad]), "clean records changed (commit)"
    print(f"[nan isolation] io={io} B={b}: {int(got.any(dim=-1).sum())} NaN rows, all in the planted pairs",
          flush=True)


@pytest.mark.parametrize("io,b", CASES)
def test_request_permutation_permutes_outputs(dev, io, b):
    case, w, gamma, slots, state, q, k, v = _batch(dev, io, b)
    perm = torch.from_numpy(np.random.default_rng(11).permutation(case.R)).to(dev)
    y0 = bha.block_forward(q, k, v, w, gamma, state, slots)
    yp = bha.block_forward(q[perm].contiguous(), k[perm].contiguous(), v[perm].contiguous(), w, gamma, state,
                           slots[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(yp, y0[perm])
    st_a, st_b = state.clone(), state.clone()
    bha.state_commit(k, v, w, st_a, slots)
    bha.state_commit(k[perm].contiguous(), v[perm].contiguous(), w, st_b, slots[perm].contiguous())
    ya = bha.block_forward_commit(q, k, v, w, gamma, state.clone(), slots)
    yb = bha.block_forward_commit(q[perm].contiguous(), k[perm].contiguous(), v[perm].contiguous(), w, gamma,
                                  state.clone(), slots[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b)
    assert torch.equal(yb, ya[perm])
    print(f"[permutation] io={io} B={b}: forward, commit and fused step bit-identical under a request permutation",
          flush=True)


@pytest.mark.parametrize("io,b", CASES)
def test_checkpoint_round_trip(dev, io, b, tmp_path):
    case, w, gamma, slots, state, q, k, v = _batch(dev, io, b)
    R, H = case.R, case.H
    over = dict(FW=64, B=b, io=io, H=H)

    def cycle(st, sl, step):
        # one block: two denoising forwards, then the fused last step
        qs, ks, vs = synth.device_step_qkv("decode256", step, R, dev, layer=1, **over)
        ys = [bha.block_forward(qs, ks, vs, w, gamma, st, sl) for _ in range(2)]
        ys.append(bha.block_forward_commit(qs, ks, vs, w, gamma, st, sl))
        return ys

    # uninterrupted: blocks 0..3
    run = state.clone()
    ys_run = [cycle(run, slots, i) for i in range(4)]
    # checkpoint after block 1: copy the requests' records to the host and
    # through a file; restore them into a fresh pool under different slots
    cp = state.clone()
    for i in range(2):
        cycle(cp, slots, i)
    records = cp.view(case.num_slots, H, -1)[slots.long()].cpu().numpy()
    path = tmp_path / "bha_state_checkpoint.npy"
    np.save(path, records)
    del cp
    restored = np.load(path)
    pool = 3 * R
    new_slots = torch.from_numpy(np.random.default_rng(9).choice(pool, size=R, replace=False).astype(np.int32)).to(dev)
    fresh = bha.new_state(pool, H, 128, 64, dev)
    fresh.view(pool, H, -1)[new_slots.long()] = torch.from_numpy(restored).to(dev)
    ys_res = [cycle(fresh, new_slots, i) for i in range(2, 4)]
    torch.cuda.synchronize()
    for a, bb in zip(ys_run[2:], ys_res):
        for ya, yb in zip(a, bb):
            assert torch.equal(ya, yb)
    assert torch.equal(run.view(case.num_slots, H, -1)[slots.long()], fresh.view(pool, H, -1)[new_slots.long()])
    print(f"[checkpoint] io={io} B={b}: resumed after block 1 under new slots; outputs and states of blocks 2-3 "
          "bit-identical to the uninterrupted run", flush=True)


@pytest.mark.parametrize("fused", [False, True])
def test_store_policy_keeps_the_bits(dev, fused):
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    H = 16
    R = 16 * cus // H  # the smallest batch that takes the device-scope stores
    case, w, gamma, slots, state, q, k, v = _batch(dev, "bf16", 32, R=R, H=H)
    half = R // 2
    print(f"[store-policy] fused={fused} R={R} H={H} ({R * H} pairs; halves of {half * H})", flush=True)
    whole, parts = state.clone(), state.clone()
    if fused:
        y_whole = bha.block_forward_commit(q, k, v, w, gamma, whole, slots)
        y_parts = torch.cat([bha.block_forward_commit(q[i:i + half], k[i:i + half], v[i:i + half], w, gamma, parts,
                                                      slots[i:i + half].contiguous()) for i in (0, half)])
    else:
        bha.state_commit(k, v, w, whole, slots)
        for i in (0, half):
            bha.state_commit(k[i:i + half], v[i:i + half], w, parts, slots[i:i + half].contiguous())
    torch.cuda.synchronize()
    assert not torch.equal(whole, state), "the commit changed nothing"
    assert torch.equal(whole.view(torch.int32), parts.view(torch.int32))
    if fused:
        assert torch.equal(y_whole.view(torch.int16), y_parts.view(torch.int16))


def test_feature_map_store_policy_keeps_the_bits(dev):
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    H, B = 16, 32
    R = 2 * (4 * cus * 128 // (H * B))  # twice the largest batch with device-scope stores
    _, w, _, _, _, q, _, _ = _batch(dev, "bf16", B, R=R, H=H)
    half = R // 2
    print(f"[store-policy] feature map R={R} H={H} ({R * B // 128 * H} units; halves of {half * B // 128 * H})",
          flush=True)
    whole = bha.feature_map(q, w)
    parts = torch.cat([bha.feature_map(q[i:i + half], w) for i in (0, half)])
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int32), parts.view(torch.int32))
