"""Bytes, operations and roofline arithmetic for the W4A8 linear layer.

Host-side accounting only (no GPU, no method arithmetic).  The formulas follow
the byte and roofline accounting of the Lecture 15 notes: decode time floor =
weight bytes / HBM bandwidth (15.1, "Numbers worth memorizing"), effective bits
of a grouped int4 format = 4 + parameter bits / group size (Exercise 1), the
dequant issue-time model (15.5, Exercise 2), the int8 ridge point and the
W4A8 crossover batch (15.7), and the prefill time at a fraction of peak
(Exercise 4).
"""
from __future__ import annotations

GROUP = 128

# MI355X (gfx950) published peaks used for roofline fractions.
MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_INT8_OPS_PER_S = 5.0e15          # dense INT8 MFMA
MI355X_FP16_FLOPS_PER_S = 2.5e15        # dense fp16/bf16 MFMA
MI355X_CUS = 256
MI355X_CLOCK_HZ = 2.4e9


def effective_bits(group: int = GROUP, param_bits: float = 16.0, code_bits: int = 4) -> float:
    """Bits per weight of a grouped code format: code bits + per-group parameter bits / group."""
    return code_bits + param_bits / group


def format_bytes(n_weights: float, bits_per_weight: float) -> float:
    return n_weights * bits_per_weight / 8.0


def floor_seconds(n_bytes: float, bytes_per_s: float) -> float:
    """Time to stream n_bytes once at the given bandwidth."""
    return n_bytes / bytes_per_s


def dequant_issue_seconds(instr_per_weight: float, n_weights: float, instr_per_s: float) -> float:
    """Unoverlapped issue time of a per-weight dequant costing k instructions."""
    return instr_per_weight * n_weights / instr_per_s


def break_even_instr_per_weight(floor_s: float, n_weights: float, instr_per_s: float) -> float:
    """k at which unoverlapped dequant time equals the byte floor."""
    return floor_s * instr_per_s / n_weights


def ridge_ops_per_byte(peak_ops_per_s: float, bytes_per_s: float) -> float:
    return peak_ops_per_s / bytes_per_s


def w4a8_ops_per_weight_byte(tokens: int) -> float:
    """2 ops per MAC, one MAC per token per weight, half a byte per weight -> 4 ops/byte per token."""
    return 2.0 * tokens / 0.5


def crossover_tokens(ridge: float) -> float:
    """Token count at which the weight stream stops being the bound."""
    return ridge / w4a8_ops_per_weight_byte(1)


def time_at_fraction_of_peak(ops: float, peak_ops_per_s: float, fraction: float) -> float:
    return ops / (peak_ops_per_s * fraction)


# ---------------------------------------------------------------------------
# per-call algorithmic traffic and work of this library's entry points
# ---------------------------------------------------------------------------
def weight_stream_bytes(N: int, K: int, group_param_bytes: int = 1) -> int:
    """Packed UINT4 codes + one parameter byte per (n, group) + fp16 channel scales."""
    return N * K // 2 + N * (K // GROUP) * group_param_bytes + 2 * N


def gemm_bytes(M: int, N: int, K: int) -> int:
    """gemm_w4a8: weight stream + int8 activations + fp32 token scales + fp16 output."""
    return weight_stream_bytes(N, K) + M * K + 4 * M + 2 * M * N


def w4a16_bytes(M: int, N: int, K: int) -> int:
    """gemm_w4a16: weight stream + fp16 activations + fp16 output."""
    return weight_stream_bytes(N, K) + 2 * M * K + 2 * M * N


def kv4_row_bytes(head_dim: int = 128) -> int:
    """One (token, head) row of the 4-bit cache: head_dim / 2 code bytes + one parameter dword."""
    return head_dim // 2 + 4


def kv4_attention_bytes(lens, Hq: int, Hkv: int, head_dim: int = 128) -> int:
    """attention_kv4_decode: the keys and values of every live token (codes + parameters) once,
    the fp16 queries in and the fp16 outputs out (chunk partial sums excluded)."""
    B = len(lens)
    return 2 * Hkv * int(sum(int(x) for x in lens)) * kv4_row_bytes(head_dim) + 2 * 2 * B * Hq * head_dim


def kv4_quant_bytes(B: int, T: int, Hkv: int, head_dim: int = 128) -> int:
    """quantize_kv4: fp16 keys and values in, their 4-bit rows out."""
    return 2 * B * T * Hkv * (2 * head_dim + kv4_row_bytes(head_dim))


def act_quant_bytes(M: int, K: int) -> int:
    """quantize_act_per_token_i8: fp16 in (absmax pass + quantize pass read the same row) counted once, int8 + fp32 out."""
    return 2 * M * K + M * K + 4 * M


def norm_quant_bytes(M: int, K: int, beta: bool = True) -> int:
    """norm_quantize_act_i8: fp16 rows in once, int8 + fp32 out, plus the fp16 gamma (and beta) rows."""
    return 2 * M * K + M * K + 4 * M + 2 * K * (2 if beta else 1)


def unfused_norm_quant_bytes(M: int, K: int, beta: bool = True) -> int:
    """The same result without the fusion: a normalization pass that writes fp16 rows, then the quantizer."""
    return 2 * M * K + 2 * M * K + 2 * K * (2 if beta else 1) + act_quant_bytes(M, K)


def gemm_ops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def linear_bytes(M: int, N: int, K: int) -> int:
    """One serving-time call: activation quantization + GEMM."""
    return act_quant_bytes(M, K) + gemm_bytes(M, N, K)
