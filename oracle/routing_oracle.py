"""CPU oracle for sigmoid top-k routing with an expert bias.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the tests and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP library.

Written from the Megatron-Core developer guide page
"core.inference.moe.sigmoid_topk" (the module summary, the description of
``_sigmoid_topk_kernel`` and the API of ``sigmoid_topk_routing``), which fixes:

* the score of expert e for a token is sigmoid(logit); the selection key adds
  the expert bias to it, the bias serving the selection only;
* the k-th largest key is found in the total (radix) order of fp32 values; the
  output lists every expert whose key is above it in ascending expert order,
  then the experts whose key equals it, in ascending expert order, until k;
* the probabilities are the selected scores divided by their sum plus 1e-20,
  the sum folded left in output order, then multiplied by the optional
  scaling factor; probabilities are fp32 and the indices int64.

Readings taken where the page is open (each repeated at its function):

* R1 sigmoid in fp32 is the fp64 value 1/(1+exp(-z)) rounded once to fp32
  (the page's sigmoid is whatever fp32 kernel the compiled graph used; a
  correctly rounded value is the one both sides can reproduce);
* R2 the key is that fp32 score plus the fp32 bias, one fp32 addition;
* R3 the left fold is used for every k (the page allows the last bit to differ
  from the compiled sum for k of eight or more, where its own kernel uses a
  tree);
* R4 1e-20 and the scaling factor are the nearest fp32 values, applied as one
  fp32 addition and one fp32 multiplication.

Pinned by ``tests/test_oracle_routing.py`` against torch.topk and
torch.sigmoid (library routines), hand-worked cases and invariants.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def sigmoid_fp32(logits) -> np.ndarray:
    """R1: fp32 sigmoid = round_to_fp32(1 / (1 + exp(-z))) evaluated in fp64."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def near_rounding_boundary(logits, rel: float = 2.0 ** -48) -> np.ndarray:
    """True where the fp64 sigmoid lies within ``rel`` (relative) of the
    midpoint between two fp32 values, i.e. where two fp64 evaluations that
    differ by a few fp64 ulps may round to different fp32 scores.  Tests use
    it to exempt those (rare) entries from bitwise comparison."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        v = 1.0 / (1.0 + np.exp(-z))
    f = v.astype(np.float32)
    other = np.where(v >= f.astype(np.float64), np.nextafter(f, F32(np.inf)), np.nextafter(f, F32(-np.inf)))
    mid = (f.astype(np.float64) + other.astype(np.float64)) / 2.0
    return np.abs(v - mid) <= rel * np.abs(v)


def total_order_key(values) -> np.ndarray:
    """uint32 image of fp32 values that orders them as the radix top-k does:
    negative values have every bit flipped, non-negative ones only the sign
    bit, so -0.0 sorts just below +0.0 (finite values only)."""
    bits = np.asarray(values, dtype=np.float32).view(np.uint32)
    neg = (bits >> np.uint32(31)).astype(bool)
    return np.where(neg, ~bits, bits | np.uint32(0x80000000)).astype(np.uint32)


def select_row(keys_u32: np.ndarray, k: int) -> np.ndarray:
    """Output order of one row: the experts above the k-th largest key in
    ascending expert order, then those equal to it in ascending order, k in
    all."""
    tau = np.sort(keys_u32)[::-1][k - 1]          # k-th largest in total order
    above = np.nonzero(keys_u32 > tau)[0]
    ties = np.nonzero(keys_u32 == tau)[0][: k - above.size]
    return np.concatenate([above, ties]).astype(np.int64)


def fold_normalize(scores_sel: np.ndarray, scaling=None) -> np.ndarray:
    """Probabilities of one row from its selected scores in output order:
    s_j / (((s_0 + s_1) + ...) + 1e-20) [* scaling], every operation in fp32."""
    total = F32(0.0)
    for v in scores_sel:
        total = F32(total + F32(v))
    denom = F32(total + F32(1e-20))
    p = (scores_sel.astype(np.float32) / denom).astype(np.float32)
    if scaling is not None:
        p = (p * F32(scaling)).astype(np.float32)
    return p


def sigmoid_topk_routing(logits, expert_bias, topk: int, scaling=None):
    """probs fp32 [T, k] and indices int64 [T, k] for fp32 logits [T, E] and
    an fp32 bias [E]."""
    logits = np.asarray(logits, dtype=np.float32)
    bias = np.asarray(expert_bias, dtype=np.float32)
    T, E = logits.shape
    if bias.shape != (E,):
        raise ValueError("expert_bias must hold one value per expert")
    if not 1 <= topk <= E:
        raise ValueError("topk must be in 1..num_experts")
    if not (np.isfinite(logits).all() and np.isfinite(bias).all()):
        raise ValueError("logits and bias must be finite")
    s = sigmoid_fp32(logits)
    keys = (s + bias[None, :]).astype(np.float32)     # R2: one fp32 addition
    u = total_order_key(keys)
    probs = np.empty((T, topk), dtype=np.float32)
    idx = np.empty((T, topk), dtype=np.int64)
    for t in range(T):
        sel = select_row(u[t], topk)
        idx[t] = sel
        probs[t] = fold_normalize(s[t, sel], scaling)
    return probs, idx
