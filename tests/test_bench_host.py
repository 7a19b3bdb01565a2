"""Host-side checks of bench.py (no GPU): the algorithmic byte counts behind
the roofline figures, worked out term by term from the state and token
layouts, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_forward_bytes_per_pair():
    # d = 128, FW = 64 (F = 128), B = 32, bf16: S 4 d F = 65,536 B, Z 4 F = 512 B,
    # Q, K, V read and O written 4 * 2 B d = 32,768 B -> 98,816 B per pair;
    # W 2 FW d = 16,384 B once per head
    assert bench.forward_bytes(1, 1, 128, 64, 32) == 98_816 + 16_384
    # the 256 x 16 decode batch: 4,096 pairs + 16 heads' W = 405,012,480 B
    assert bench.forward_bytes(256, 16, 128, 64, 32) == 4096 * 98_816 + 16 * 16_384 == 405_012_480
    # F = 256: S 131,072 + Z 1,024 + 32,768 -> 164,864 B per pair
    assert bench.forward_bytes(1, 1, 128, 128, 32) - 2 * 128 * 128 == 164_864
    # fp32 I/O, d = 64, FW = 32, B = 8: S 16,384 + Z 256 + 4 * 4 B * 8 * 64 = 8,192
    # and W 4 B * 32 * 64 = 8,192 -> 33,024 B
    assert bench.forward_bytes(1, 1, 64, 32, 8, es=4) == 33_024


def test_commit_bytes_per_pair():
    # the record read and written (2 * 66,048 B) and K, V read (2 * 8,192 B)
    assert bench.commit_bytes(1, 1, 128, 64, 32) == 148_480 + 16_384
    assert bench.commit_bytes(256, 16, 128, 64, 32) == 4096 * 148_480 + 16 * 16_384
    # F = 256: 2 * 132,096 + 16,384 = 280,576 B per pair
    assert bench.commit_bytes(1, 1, 128, 128, 32) - 2 * 128 * 128 == 280_576
    assert bench.commit_bytes(1, 1, 64, 32, 8, es=4) == 45_568


def test_fused_and_grouped_bytes():
    # the fused last step writes the record back on top of the forward's bytes
    assert bench.forward_commit_bytes(256, 16, 128, 64, 32) == bench.forward_bytes(256, 16, 128, 64, 32) + 4096 * 66_048
    # grouped K/V heads with one K/V head per query head are the forward
    for d, fw, b in ((128, 64, 32), (64, 32, 8), (128, 128, 17)):
        assert bench.forward_gqa_bytes(7, 8, 8, d, fw, b) == bench.forward_bytes(7, 8, d, fw, b)
    # 16 query heads over 4 K/V heads: 4 records and K, V per request, 16 Q and O
    got = bench.forward_gqa_bytes(1, 16, 4, 128, 64, 32)
    assert got == 4 * (66_048 + 2 * 8_192) + 16 * 2 * 8_192 + 4 * 16_384


def test_prefill_and_prefix_attention_bytes():
    # T packed tokens: K, V of every token and head (2 * 2 B * d), each record read
    # and written, W once per head, the offsets (R + 1) and slot ids (R) as int32
    assert bench.prefill_bytes(100, 3, 2, 128, 64) == 100 * 2 * 512 + 3 * 2 * 2 * 66_048 + 2 * 16_384 + 7 * 4
    # prefix attention: the prefix K, V rows, the block's Q, K, V, O, the offsets
    assert bench.prefix_attention_bytes(100, 3, 2, 128, 32) == 100 * 2 * 512 + 3 * 2 * 4 * 8_192 + 4 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
