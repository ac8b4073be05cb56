"""FLOP and byte model of attention, used to price kernels against a roofline.

Sources:
  * "FlashAttention" (interactiveprimer), "A concrete example: 10,000 tokens":
    the standard path holds N*N score entries per head; at 2 bytes per entry
    N = 10,000 gives 1e8 entries, about 200 MB; a 128-token tile of queries
    against a 128-token tile of keys holds 128*128 = 16,384 entries.
  * "What FlashAttention actually buys", "The actual problem": the arithmetic
    stays quadratic in sequence length while the tiled path's traffic is linear.
  * "FlashAttention, simplified", "The problem": the standard path writes the
    scores, reads them for the softmax, writes the probabilities and reads
    them again for the product with V.

FLOPs count the two contractions only (2*N*N*d each per head); the pages give
no other count and padding is never credited.
"""
from __future__ import annotations

from math import ceil

LSE_BYTES = 4  # one float32 logsumexp per query row


def attention_flops(B: int, H: int, N: int, d: int) -> int:
    """4*B*H*N^2*d: S = Q K^T and O = P V, 2*N*N*d each per head."""
    return 4 * B * H * N * N * d


def score_entries(N: int) -> int:
    """Entries of one head's N x N score matrix."""
    return N * N


def score_bytes(N: int, bytes_per_entry: int) -> int:
    return score_entries(N) * bytes_per_entry


def tile_entries(br: int, bc: int) -> int:
    """Score entries held on chip for one query tile against one key tile."""
    return br * bc


def compulsory_bytes(B: int, H: int, N: int, d: int, e: int) -> int:
    """Read Q, K, V once, write O once (element size e) and the LSE (float32)."""
    return 4 * B * H * N * d * e + B * H * N * LSE_BYTES


def tiled_request_bytes(B: int, H: int, N: int, d: int, e: int, br: int) -> int:
    """Bytes a one-pass-per-query-tile schedule asks for: Q, O, LSE once plus
    all of K and V once per query tile (ceil(N/br) passes per head)."""
    t_r = ceil(N / br) if N else 0
    qo = 2 * B * H * N * d * e + B * H * N * LSE_BYTES
    return qo + t_r * 2 * B * H * N * d * e


def naive_bytes(B: int, H: int, N: int, d: int, e: int, s_bytes: int = 4) -> int:
    """Three-pass standard attention: compulsory bytes plus S written and read
    once (s_bytes per entry) and P written and read once (e bytes per entry)."""
    per_head = score_entries(N)
    return compulsory_bytes(B, H, N, d, e) + B * H * per_head * 2 * (s_bytes + e)


def naive_workspace_bytes_per_head(N: int, e: int, s_bytes: int = 4) -> int:
    """Workspace one head needs in the three-pass path: S and P."""
    return score_entries(N) * (s_bytes + e)
