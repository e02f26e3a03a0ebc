"""The byte / roofline accounting against the Lecture 15 notes' printed numbers.

tests/golden/lecture15_numbers.json holds the values as the page prints them
(rounded as printed); each check allows the page's own rounding.
"""
import pytest

from conftest import load_golden
from w4a8_quantized_linear_amd import accounting as A

L = load_golden("lecture15_numbers.json")


def close(x, printed, rel=None, digits=None):
    if digits is not None:
        return abs(x - printed) <= 0.5 * 10 ** (-digits) + 1e-12
    return abs(x - printed) <= rel * abs(printed)


def test_effective_bits_and_floor():
    assert A.effective_bits(128, 16) == L["effective_bits_g128_fp16_scale"]
    b = A.format_bytes(L["params_7b"], A.effective_bits(128, 16))
    assert close(b / 1e9, L["int4_g128_bytes_GB"], rel=0.005)
    assert close(A.floor_seconds(b, L["h100_hbm_Bps"]) * 1e3, L["int4_floor_ms"], digits=2)


@pytest.mark.parametrize("g", [32, 128, 256])
def test_exercise1_group_size_tax(g):
    bits = A.effective_bits(g, 20)
    assert close(bits, L["ex1_bits"][str(g)], digits=3)
    gb = A.format_bytes(L["params_7b"], bits) / 1e9
    assert close(gb, L["ex1_GB"][str(g)], digits=2)
    assert close(A.floor_seconds(gb * 1e9, L["h100_hbm_Bps"]) * 1e3, L["ex1_floor_ms"][str(g)], digits=2)


def test_board_model_and_exercise2():
    n = L["params_7b"]
    assert close(L["board_instr_per_weight"] * n, L["board_instr_total"], rel=0.01)
    t = A.dequant_issue_seconds(L["board_instr_per_weight"], n, L["h100_issue_instr_per_s"])
    assert close(t * 1e3, L["board_ms"], digits=1)
    assert close(L["int4_floor_ms"] + t * 1e3, L["board_unoverlapped_ms"], digits=2)
    k = A.break_even_instr_per_weight(L["int4_floor_ms"] * 1e-3, n, L["h100_issue_instr_per_s"])
    assert close(k, L["ex2_break_even_k"], digits=1)
    t2 = A.dequant_issue_seconds(2, n, L["h100_issue_instr_per_s"])
    assert close(t2 * 1e3, L["ex2_k2_ms"], digits=2)
    assert close(t2 * 1e3 / L["int4_floor_ms"], L["ex2_k2_fraction_of_floor"], digits=2)


def test_ridge_and_crossover():
    r = A.ridge_ops_per_byte(L["h100_int8_ops"], L["h100_hbm_Bps"])
    assert close(r, L["int8_ridge_ops_per_byte"], digits=0)
    assert A.w4a8_ops_per_weight_byte(1) == L["w4a8_ops_per_byte_per_token"]
    assert close(A.crossover_tokens(r), L["crossover_batch"], digits=0)


def test_two_level_storage():
    n = L["params_7b"]
    group_bytes = n / 128 * 1          # one int8 scale per group of 128
    assert close(group_bytes / 1e6, L["two_level_group_scale_MB"], digits=0)
    assert close((n * 0.5 + group_bytes) / 1e9, L["two_level_total_GB"], digits=2)


def test_exercise4_prefill():
    t_bf16 = A.time_at_fraction_of_peak(L["ex4_prefill_tflop"] * 1e12, L["h100_bf16_flops"], 0.5)
    t_w4a8 = A.time_at_fraction_of_peak(L["ex4_prefill_tflop"] * 1e12, L["h100_int8_ops"], 0.5)
    assert close(t_bf16 * 1e3, L["ex4_bf16_ms"], digits=0)
    assert close(t_w4a8 * 1e3, L["ex4_w4a8_ms"], digits=0)
    assert close(L["board_ms"] / (t_w4a8 * 1e3), L["ex4_dequant_share_prefill"], digits=3)
    assert close(L["board_ms"] / L["int4_floor_ms"], L["ex4_dequant_share_decode"], digits=2)


def test_library_traffic_formulas():
    # 7B MLP projection at one token: codes + 1 B per group + fp16 scales + activations + output
    M, N, K = 1, 11008, 4096
    assert A.weight_stream_bytes(N, K) == N * K // 2 + N * (K // 128) + 2 * N
    assert A.gemm_bytes(M, N, K) == A.weight_stream_bytes(N, K) + K + 4 + 2 * N
    assert A.gemm_ops(M, N, K) == 2 * N * K
    # the per-weight byte cost of this format is 4 + 8/128 bits (+ the channel scale)
    assert abs(A.weight_stream_bytes(N, K) * 8 / (N * K) - (A.effective_bits(128, 8) + 16 / K)) < 1e-12
