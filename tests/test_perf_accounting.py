"""The algorithmic work behind bench.py's roofline fractions
(top_routing_expert_amd/perf.py), pinned to numbers worked out by hand from
the layer shapes, so that a change of the accounting shows up as a failing
test rather than as a silently different fraction."""

import pytest

from top_routing_expert_amd import perf, presets


def test_mixtral_shaped_ffn_work():
    # 4096 tokens, top-2, dropless: R = 8192 rows; 8 SwiGLU experts, d = 4096,
    # F = 14336, bf16 weights.
    p = presets.get("c3")
    R = 8192
    # 2 * 3 matrices * d * F * R
    assert perf.ffn_flops(p, R, shared=False) == 2 * 3 * 4096 * 14336 * 8192 == 2886218022912
    # weights 8 * 3 * d * F * 2 B + x_perm R * d * 2 B + fp32 output R * d * 4 B
    assert perf.ffn_bytes(p, R, 8, shared=False) == 2818572288 + 67108864 + 134217728
    t, bound = perf.ffn_roofline_s(p, R, 8)
    assert bound == "mfma"
    assert t == pytest.approx(2886218022912 / 2.5e15, rel=1e-12)
    # the activation written and read back is reported beside, not counted
    assert perf.ffn_bytes_unfused(p, R, 8) - perf.ffn_bytes(p, R, 8, shared=False) == 2 * 8192 * 14336 * 2


def test_router_roofline_bytes_or_three_planes():
    # 4096 tokens, d = 4096, 8 experts: x 32 MiB + Wg 128 KiB + indices and
    # gates 4096 * 2 * 8 B; HBM-bound (the three-plane MFMA work is 0.32 us).
    p = presets.get("c3")
    assert perf.route_bytes(p) == 33554432 + 131072 + 65536
    assert perf.route_roofline_s(p) == pytest.approx(33751040 / 8e12, rel=1e-12)
    # 16384 tokens, d = 2048, 256 experts: three bf16 planes of 2 T d E flops
    # each at 2.5 PFLOP/s (20.6 us) exceed the 70 MB at 8 TB/s (8.8 us).
    q = presets.get("c5")
    assert perf.route_bytes(q) == 67108864 + 2097152 + 1048576
    assert perf.route_roofline_s(q) == pytest.approx(3 * 2 * 16384 * 2048 * 256 / 2.5e15, rel=1e-12)


def test_permute_and_combine_bytes():
    # 16384 tokens, top-8, d = 2048, bf16, 131072 kept rows, a shared expert
    p = presets.get("c4")
    R = 131072
    # x once + R rows written + indices read (T k 8 B) + row map (R 4 B)
    assert perf.permute_bytes(p, R) == 67108864 + 536870912 + 1048576 + 524288
    # fp32 rows read + y written + gates and rows read + the shared expert's rows
    assert perf.combine_bytes(p, R) == 1073741824 + 134217728 + 1048576 + 134217728


def test_gemm_source_digest_is_a_sha256():
    h = perf.gemm_source_sha256()
    assert len(h) == 64 and int(h, 16) >= 0
