"""Work and traffic accounting of the fused linear log-prob (closed forms).

Used by the benchmark for throughput and roofline figures; pinned in the tests
by the numbers the pages print.
"""

from __future__ import annotations

GiB = float(1 << 30)
MiB = float(1 << 20)


def linear_fwd_bwd_flops(N: int, D: int, V: int) -> int:
    """Four N x V x D contractions: logits (forward), logits recomputed in the
    backward, dH = dlogits W and dW = dlogits^T h; 2 flops per multiply-add."""
    return 8 * N * V * D


def linear_model_flops(N: int, D: int, V: int) -> int:
    """Three contractions (a method that kept the logits would skip the recompute)."""
    return 6 * N * V * D


def contraction_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def dw_table_traffic(V: int, D: int, K: int) -> dict:
    """Gradient-table bytes over K chunks with an FP32 [V, D] table.

    RL-Kernel issue #261, "Static traffic model": zero fill 4VD, then per chunk
    either a materialised GEMM result added into the table (write 4VD, read it
    back 4VD, read+write the table 8VD: 16VD) or an in-place accumulation
    (read+write the table: 8VD).
    """
    return {
        "current": 4 * V * D + 16 * K * V * D,
        "candidate": 4 * V * D + 8 * K * V * D,
        "saving": 8 * K * V * D,
    }


def rows_per_chunk(chunk_elems: int, V: int) -> int:
    """Token rows in a chunk of at most ``chunk_elems`` logits."""
    return chunk_elems // V


def logits_bytes(N: int, V: int, esize: int) -> int:
    return N * V * esize


def dw_temporary_bytes(V: int, H: int, esize: int) -> int:
    """The [V, H] temporaries of a same-dtype ``table += mm(...).float()`` update:
    the product in the operand dtype, plus its FP32 copy when that dtype is 16-bit
    (Liger-Kernel PR #1324, "Details")."""
    return V * H * esize + (V * H * 4 if esize != 4 else 0)


def tokens_per_s(N: int, ms: float) -> float:
    return N / (ms / 1e3)


def logits_only_bytes(N: int, V: int, esize: int) -> int:
    """Algorithmic HBM bytes of logits-only forward + backward with a saved lse:
    read the logits once in the forward, once in the backward, write dlogits."""
    return 3 * N * V * esize
