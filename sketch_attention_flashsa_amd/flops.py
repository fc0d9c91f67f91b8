"""Closed-form FLOP model of the SequenceO1 paper, appendix G (G.1-G.7).

Counting convention (G.1): a product of [m x r] and [r x p] matrices costs
2*m*r*p FLOPs; only GEMM-shaped terms are counted.  The SA layer (G.3, single
head, width d, L history tokens, L_s prototypes) costs
    key projection 2*L*d^2 + prototype projection 2*L_s*d^2
    + affinity and aggregation 4*L_s*L*d + sketch SwiGLU FFN 12*L_s*d^2.
The benchmark counts the on-path part of that model per head: the affinity and
aggregation term 4*L*m*dh (plus 2*L*d_model*(H*dh) per projected tensor on the
fused-projection entry).
"""
from __future__ import annotations


def swiglu(n_tokens: float, width: float, inner: float) -> float:
    """SwiGLU FFN (G.1): two [n x width]x[width x inner] and one [n x inner]x[inner x width]."""
    return 2 * n_tokens * width * inner * 2 + 2 * n_tokens * inner * width


def sa_layer(L: float, Ls: float, d: float) -> float:
    """One single-head SA layer (G.3): 2Ld^2 + 14 L_s d^2 + 4 L_s L d."""
    key_proj = 2 * L * d * d
    proto_proj = 2 * Ls * d * d
    affinity_and_aggregation = 4 * Ls * L * d
    ffn = swiglu(Ls, d, 2 * d)
    return key_proj + proto_proj + affinity_and_aggregation + ffn


def sa(L: float, n_sa: int, Ls: float, d: float) -> float:
    """Stacked SA (G.3)."""
    return n_sa * sa_layer(L, Ls, d)


def attn_reordered(L: float, D: float, h: int) -> float:
    """Single-query reordered attention, all heads (G.2.1): per head three
    D x d_h products (q W_Q, (q W_Q) W_K^T, (alpha X) W_V) and two L x D
    products (u X^T, alpha X), with d_h = D / h."""
    dh = D / h
    return h * (3 * 2 * D * dh + 2 * 2 * L * D)


def stca_layer(L: float, D: float, h: int) -> float:
    """One STCA layer (G.2): history pre-FFN + reordered attention + output
    projection 2D^2 + one-token FFN 12D^2 = 12LD^2 + 4LDh + 20D^2."""
    return swiglu(L, D, 2 * D) + attn_reordered(L, D, h) + 2 * D * D + swiglu(1, D, 2 * D)


def stca(L: float, n_stca: int, D: float, h: int) -> float:
    """Stacked STCA (G.2): N (12LD^2 + 4LDh + 20D^2)."""
    return n_stca * stca_layer(L, D, h)


def adapter(Ls: float, d: float, D: float) -> float:
    """Sketch adapter X^ = X~ W_A (G.4): 2 L_s d D."""
    return 2 * Ls * d * D


def stca_mrlb(L: float, R: float, n_stca: int, D: float, h: int) -> float:
    """Direct STCA under reuse ratio R (G.6/G.7): only the history pre-FFN is shared."""
    return 12 * n_stca * L * D * D / R + n_stca * (4 * L * D * h + 20 * D * D)


def seqo1_expected_mrlb(L: float, R: float, p_hit: float, n_sa: int, Ls: float, d: float,
                        n_stca: int, D: float, h: int) -> float:
    """Expected SequenceO1 cost per target under reuse R and hit rate p (G.6)."""
    per_target = n_stca * (4 * Ls * D * h + 20 * D * D)
    shared = adapter(Ls, d, D) + 12 * n_stca * Ls * D * D + (1 - p_hit) * sa(L, n_sa, Ls, d)
    return per_target + shared / R


# Hyper-parameters of appendix G.5.
G5 = dict(L=100_000, Ls=1024, d=128, n_sa=2, D=1024, h=16, n_stca=4)


def g7_numbers() -> dict:
    """The appendix G.7 comparison at the G.5 instantiation."""
    p = G5
    stca_inf = stca_mrlb(p["L"], 300, p["n_stca"], p["D"], p["h"])
    seq_inf = seqo1_expected_mrlb(p["L"], 300, 0.6, p["n_sa"], p["Ls"], p["d"], p["n_stca"], p["D"], p["h"])
    stca_tr = stca_mrlb(p["L"], 40, p["n_stca"], p["D"], p["h"])
    seq_tr = seqo1_expected_mrlb(p["L"], 40, 0.5, p["n_sa"], p["Ls"], p["d"], p["n_stca"], p["D"], p["h"])
    return {
        "stca_infer_gflops": stca_inf / 1e9,
        "seqo1_infer_gflops": seq_inf / 1e9,
        "ratio_infer": stca_inf / seq_inf,
        "ratio_train": stca_tr / seq_tr,
    }


# ------------------------------------------------------------ on-path counters
def sa_forward_flops(total_tokens: int, H: int, m: int, dh: int) -> float:
    """Affinity + aggregation FLOPs of one SA forward: 4 * L * m * dh per head."""
    return 4.0 * total_tokens * H * m * dh


def projection_flops(total_tokens: int, d_model: int, n_cols: int, n_mats: int = 2) -> float:
    """Key (and value) projection FLOPs: 2 * L * d_model * n_cols per matrix."""
    return 2.0 * total_tokens * d_model * n_cols * n_mats


def fold_keys_flops(H: int, m: int, dh: int, d_model: int) -> float:
    """Prototypes moved through the key projection once per call,
    P_h W_K,h^T for every head: 2 * m * dh * d_model per head.  With it the
    scores P_h (X W_K,h)^T are (P_h W_K,h^T) X^T and the per-row projection
    (projection_flops) is not performed (appendix G.2.1's reordering)."""
    return 2.0 * H * m * dh * d_model


def stca_attention_flops(rows_per_target, D: int, h: int) -> float:
    """Reordered single-query attention (G.2.1) summed over targets: target t
    sees rows_per_target[t] history rows and costs attn_reordered(L_t, D, h)."""
    return float(sum(attn_reordered(float(L), D, h) for L in rows_per_target))


def refine_flops(total_tokens: int, B: int, m: int, d: int, n_layers: int) -> float:
    """Stacked refinement over a batch (G.3's SA layer summed over users, with
    L the user's rows and L_s = m): n_sa * (2 L d^2 + 14 L_s d^2 + 4 L_s L d)
    per user.  Linear in L, so the batch total uses the row total."""
    return n_layers * (2.0 * total_tokens * d * d + 14.0 * B * m * d * d + 4.0 * m * total_tokens * d)
