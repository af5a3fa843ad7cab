"""Storage and traffic calculator (test infrastructure only).

Closed forms for the effective bit width, the bytes a decode step moves per
cached token, and the logical component-access counts, following the paper
"KV Cache Quantization for Looped Transformers with 2-Bit Residuals"
(ResidualQuant): App. A.3 (effective KV bitwidth), §3.4 (mixed precision and
the 5.2x reduction), §5.1 (LS coefficients add about 0.1 bit) and App. D
(logical reference count).

Pinned by tests/test_oracle_storage.py against the numbers the pages print.
"""
from __future__ import annotations


def beff(bits, group, D: int, meta_bits_per_group: int = 16, alpha_bits: int = 16,
         residual: bool = True, anchor: int | None = None) -> float:
    """Bits per stored KV element, averaged over the loops of one tensor.

    Counts codes, per-group metadata and (for residual quantization) one LS
    coefficient per token, head and non-anchor loop; excludes rotations and
    means (App. A.3).
    """
    L = len(bits)
    groups = list(group) if isinstance(group, (list, tuple)) else [group] * L
    per_loop = [b + meta_bits_per_group / g for b, g in zip(bits, groups)]
    total = sum(per_loop) / L
    if residual:
        total += alpha_bits * (L - 1) / (L * D)
    return total


def alpha_bits_per_element(L: int, D: int, alpha_bits: int = 16) -> float:
    """Extra bits per element from LS coefficients (App. A.3: 0.094 at L=4, D=128)."""
    return alpha_bits * (L - 1) / (L * D)


def component_bytes(D: int, bits: int, group: int, meta_bytes_per_group: int = 4,
                    alpha_bytes: int = 2, with_alpha: bool = False) -> int:
    """Bytes one token's component (codes + metadata [+ alpha]) occupies for one head."""
    return D * bits // 8 + (D // group) * meta_bytes_per_group + (alpha_bytes if with_alpha else 0)


def components_read(L: int, r: int, policy: str, loop_group: int = 0) -> list:
    """Loops whose stored component loop r's reconstruction reads (App. D), within
    r's loop group of loop_group loops (0: one group of all L loops; §5 "Models").

    'last':  the group's last loop is the anchor; loop r reads the anchor plus its
             own residual; the anchor reads itself only.
    'first': the same with the group's first loop as the anchor (§3.2).
    'prev':  the group's first loop is the anchor and loop r reads the chain of
             residuals back to it.
    Loops are 0-based here.
    """
    G = loop_group or L
    g0 = r // G * G
    if policy == "last":
        a = g0 + G - 1
        return [a] if r == a else [a, r]
    if policy == "first":
        return [g0] if r == g0 else [g0, r]
    if policy == "prev":
        return list(range(g0, r + 1))
    raise ValueError(policy)


def logical_reads(L: int, policy: str, loop_group: int = 0) -> int:
    """Components read to reconstruct every loop once: 2G-1 shared or G(G+1)/2
    chained per group of G loops."""
    return sum(len(components_read(L, r, policy, loop_group)) for r in range(L))


def decode_bytes_per_token(D: int, bits, group=32, policy: str = "last", meta_bytes_per_group: int = 4,
                           alpha_bytes: int = 2) -> int:
    """Bytes read per cached token, per head and per layer, over one decode step
    (all L loops, K and V): each loop reads the components of components_read()."""
    L = len(bits)
    groups = list(group) if isinstance(group, (list, tuple)) else [group] * L
    anchor = L - 1 if policy == "last" else 0
    total = 0
    for r in range(L):
        for c in components_read(L, r, policy):
            total += component_bytes(D, bits[c], groups[c], meta_bytes_per_group, alpha_bytes,
                                     with_alpha=(c != anchor))
    return 2 * total  # K and V


def bf16_decode_bytes_per_token(D: int, L: int) -> int:
    """BF16 cache: every loop reads its own K and V rows."""
    return 2 * L * D * 2
