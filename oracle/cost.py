"""Algorithmic cost counters of one ESA decode step and of MoBA gating.

Source: ESA write-up, the paragraph on compute reduction (the formula is
dropped; the text gives about 1.6% of full attention per step for long
inputs at about 3.2% q/k compression), and the MoBA write-up's experiments
section (95.31% sparsity with 64 blocks and top-k 3).

The counts follow the oracle's own definitions: one decode step compresses
the query (D*d_c multiply-adds), scores every middle candidate in the
compressed space (d_c each) and runs attention over the fixed attended set
(2*D per key: q.k and p*v), against 2*D per key over all T keys for full
attention.
"""


def esa_decode_macs(T, D, d_c, n_init, k_sel, window):
    n_mid = max(0, (T - 1 - window) - n_init)
    attended = n_init + min(k_sel, n_mid) + window + 1
    return D * d_c + n_mid * d_c + 2 * D * attended


def full_decode_macs(T, D):
    return 2 * D * T


def esa_step_ratio(T, D=4096, d_c=128, n_init=128, k_sel=2048, window=4096):
    return esa_decode_macs(T, D, d_c, n_init, k_sel, window) / full_decode_macs(T, D)


def moba_sparsity(n_blocks, topk):
    """Fraction of a long sequence's blocks a late query does not attend."""
    return 1.0 - min(topk, n_blocks) / n_blocks
