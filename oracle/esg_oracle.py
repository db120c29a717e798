"""CPU oracle for the group-sparse SwiGLU feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the tests, the package's ``smoke()`` check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library.

It is a plain, slow, dense-masked implementation in float64 (numpy), written
from the eugen_sparse README ("eugen_sparse -- sparse SwiGLU FFN in Triton"),
section "What it does", which defines the four operations, and its section
"Parameters and how to choose them", which gives the shape rules and the
balancing constants.  Where that page leaves a step open, the reading taken is
stated at the function.  Inputs are the exact stored values (bf16 and fp32
upcast to float64 exactly).

Every function here is pinned by a test in ``tests/test_oracle_*.py`` against
something other than itself (library routines, brute force, closed forms,
finite differences, invariants).
"""
from __future__ import annotations

import numpy as np

_MASK64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# Subsample of gate rows (eugen_sparse README, "What it does":
# make_subsample_index; "Pitfalls and limitations": the subsample is drawn once
# per layer and kept fixed).
#
# The page gives only the signature.  Reading taken: for each group in order, a
# partial Fisher-Yates shuffle of the group's local row ids 0..gs-1 driven by a
# SplitMix64 stream seeded with ``seed``; the first ``spg`` ids after the
# shuffle are kept, offset by g*gs and sorted ascending.
# ---------------------------------------------------------------------------

class SplitMix64:
    """SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014; the 64-bit mixing constants of Vigna's public
    splitmix64.c).  The state advances by the golden-ratio increment and each
    output is the state passed through two xor-shift-multiply rounds and a
    final xor-shift."""

    GAMMA = 0x9E3779B97F4A7C15

    def __init__(self, seed: int):
        self.state = seed & _MASK64

    def next(self) -> int:
        self.state = (self.state + self.GAMMA) & _MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        return z ^ (z >> 31)


def make_subsample_index(d_ff: int, group_size: int, spg: int, seed: int) -> np.ndarray:
    """Absolute W_gate row ids, int32 [G * spg], grouped by group, ascending
    within a group."""
    if group_size <= 0 or d_ff % group_size != 0:
        raise ValueError("d_ff must be a positive multiple of group_size")
    if not 1 <= spg <= group_size:
        raise ValueError("samples_per_group must be in 1..group_size")
    groups = d_ff // group_size
    rng = SplitMix64(seed)
    out = []
    for g in range(groups):
        pool = list(range(group_size))
        for i in range(spg):
            j = i + rng.next() % (group_size - i)
            pool[i], pool[j] = pool[j], pool[i]
        out.extend(sorted(g * group_size + r for r in pool[:spg]))
    return np.asarray(out, dtype=np.int32)


# ---------------------------------------------------------------------------
# Selection (eugen_sparse README, "What it does": grouped_topk_select).
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def group_rows(d_ff: int, group_size: int, sub=None, spg=None):
    """The gate rows whose responses estimate each group's energy.

    With a subsample, group g uses sub[g*spg:(g+1)*spg]; without one it uses
    all of its rows [g*gs, (g+1)*gs) (the README's parameter table: no
    subsample, or spg = group_size, is the exact selection)."""
    groups = d_ff // group_size
    if sub is None:
        return [np.arange(g * group_size, (g + 1) * group_size) for g in range(groups)]
    sub = np.asarray(sub, dtype=np.int64)
    if spg is None or sub.shape[0] != groups * spg:
        raise ValueError("subsample must hold G * spg row ids")
    return [sub[g * spg:(g + 1) * spg] for g in range(groups)]


def group_energy(x, w_gate, group_size: int, sub=None, spg=None, dtype=np.float64) -> np.ndarray:
    """E[t, g] = sum over the group's rows r of |SiLU(x[t] . W_gate[r])|, fp64
    (``dtype`` float32 gives the same steps in float32, for the timed CPU
    baseline only; parity always uses float64).

    Reading taken: with a subsample the sum runs over the sampled rows only and
    is not rescaled (the README defines the energy as this sum and says the
    subsample estimates it; a uniform rescale would not change the ranking
    without a bias, and the unscaled sum is the plain reading)."""
    x = np.asarray(x, dtype=dtype)
    w_gate = np.asarray(w_gate, dtype=dtype)
    rows = group_rows(w_gate.shape[0], group_size, sub, spg)
    energy = np.empty((x.shape[0], len(rows)), dtype=dtype)
    for g, r in enumerate(rows):
        h = x @ w_gate[r].T
        energy[:, g] = np.abs(silu(h)).sum(axis=1)
    return energy


def selection_scores(x, w_gate, group_size: int, sub=None, spg=None, bias=None, dtype=np.float64) -> np.ndarray:
    """s = E + bias.  Reading taken: the balancing bias re-weights the ranking
    additively and is used for the selection only (DeepSeek-V3 style, as the
    README names it; the Megatron-Core sigmoid_topk page likewise adds its
    expert bias to the key and not to the probabilities)."""
    s = group_energy(x, w_gate, group_size, sub, spg, dtype)
    if bias is not None:
        s = s + np.asarray(bias, dtype=dtype)[None, :]
    return s


def topk_from_scores(scores: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k groups with the largest score, int32 [T, k], listed in
    ascending group id.

    Readings taken: equal scores are ordered by ascending group id (the order
    torch.topk gives equal keys, as the Megatron-Core sigmoid_topk page
    describes it); the output order within a token is ascending group id,
    because the FFN sum does not depend on it."""
    scores = np.asarray(scores)
    T, G = scores.shape
    if not 1 <= k <= G:
        raise ValueError("k must be in 1..G")
    # a stable sort on the negated score keeps equal scores in ascending id
    order = np.argsort(-scores, axis=1, kind="stable")
    return np.sort(order[:, :k], axis=1).astype(np.int32)


def grouped_topk_select(x, w_gate, group_size: int, k: int, sub=None, spg=None, bias=None, dtype=np.float64):
    """Hard top-k group routing.  Returns (idx int32 [T, k], scores [T, G] in
    ``dtype``, float64 unless the float32 timing variant is asked for)."""
    s = selection_scores(x, w_gate, group_size, sub, spg, bias, dtype)
    return topk_from_scores(s, k), s


def near_tie_tokens(scores: np.ndarray, k: int, rel: float = 1e-5) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th largest scores differ by at most
    rel * max(|s_k|, |s_k+1|): any choice among the near-tied groups at that
    boundary is a correct selection."""
    scores = np.asarray(scores, dtype=np.float64)
    if k >= scores.shape[1]:
        return np.zeros(scores.shape[0], dtype=bool)
    srt = -np.sort(-scores, axis=1)
    a, b = srt[:, k - 1], srt[:, k]
    return np.abs(a - b) <= rel * np.maximum(np.abs(a), np.abs(b))


def group_counts(idx: np.ndarray, groups: int) -> np.ndarray:
    """How many tokens selected each group (int32 [G])."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=groups).astype(np.int32)


# ---------------------------------------------------------------------------
# CSR bucketing (eugen_sparse README, "Pitfalls and limitations": the
# selection and the CSR bucketing are deterministic).  The page does not give
# the layout; reading taken: the (token, slot) pairs are ordered by
# (group, token), offsets are the exclusive prefix sums of the group counts,
# perm_token[pos] is the token at bucket position pos and inv[t, j] is the
# position of token t's slot j.
# ---------------------------------------------------------------------------

def bucket_by_group(idx: np.ndarray, groups: int):
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    check_routing(idx, groups)
    tok = np.repeat(np.arange(T), k)
    slot = np.tile(np.arange(k), T)
    grp = idx.reshape(-1)
    order = np.lexsort((tok, grp))      # primary key group, then token
    counts = np.bincount(grp, minlength=groups)
    offsets = np.zeros(groups + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm_token = tok[order]
    inv = np.empty(T * k, dtype=np.int64)
    inv[order] = np.arange(T * k)
    return (offsets.astype(np.int32), perm_token.astype(np.int32),
            inv.reshape(T, k).astype(np.int32))


def check_routing(idx: np.ndarray, groups: int) -> None:
    """Precondition of the FFN (README, "Pitfalls and limitations"): each
    token's group ids are distinct and in range."""
    idx = np.asarray(idx)
    if idx.size and (idx.min() < 0 or idx.max() >= groups):
        raise ValueError("group id out of range")
    srt = np.sort(idx, axis=1)
    if idx.shape[1] > 1 and np.any(srt[:, 1:] == srt[:, :-1]):
        raise ValueError("duplicate group id in a token")


# ---------------------------------------------------------------------------
# Sparse SwiGLU FFN, dense-masked (README, "What it does": sparse_swiglu_ffn
# and reference_sparse_swiglu_ffn).  nn.Linear layout: W_gate, W_up [F, d],
# W_down [d, F]; group g owns neurons [g*gs, (g+1)*gs).
# ---------------------------------------------------------------------------

def group_mask(idx, tokens: int, d_ff: int, group_size: int, dtype=np.float64) -> np.ndarray:
    """M[t, f] = 1 when neuron f's group is among token t's groups.  idx=None
    means every group is active (the dense limit)."""
    if idx is None:
        return np.ones((tokens, d_ff), dtype=dtype)
    idx = np.asarray(idx, dtype=np.int64)
    groups = d_ff // group_size
    check_routing(idx, groups)
    gm = np.zeros((tokens, groups), dtype=dtype)
    np.put_along_axis(gm, idx, 1.0, axis=1)
    return np.repeat(gm, group_size, axis=1)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sparse_swiglu_forward(x, w_gate, w_up, w_down, idx, group_size: int, chunk: int = 4096, dtype=np.float64):
    """y = (SiLU(x W_gate^T) * (x W_up^T) * M) W_down^T, fp64, [T, d]
    (``dtype`` float32: the same steps in float32, for the timed CPU baseline)."""
    x, w_gate, w_up, w_down = (np.asarray(a, dtype=dtype) for a in (x, w_gate, w_up, w_down))
    T = x.shape[0]
    F = w_gate.shape[0]
    y = np.zeros((T, w_down.shape[0]), dtype=dtype)
    for t0 in range(0, T, chunk):
        xs = x[t0:t0 + chunk]
        m = group_mask(None if idx is None else np.asarray(idx)[t0:t0 + chunk],
                       xs.shape[0], F, group_size, dtype)
        hg = xs @ w_gate.T
        hu = xs @ w_up.T
        a = silu(hg) * hu * m
        y[t0:t0 + chunk] = a @ w_down.T
    return y


def sparse_swiglu_backward(dy, x, w_gate, w_up, w_down, idx, group_size: int, chunk: int = 4096,
                           dtype=np.float64):
    """Gradients of L = sum(y * dy) with the routing held fixed (hard top-k: no
    gradient reaches the routing; README, "Pitfalls and limitations").

    With s = sigmoid(Hg), SiLU'(Hg) = s * (1 + Hg * (1 - s)):
      dA = (dy W_down) * M
      dHu = dA * SiLU(Hg);  dHg = dA * Hu * SiLU'(Hg)
      dx = dHg W_gate + dHu W_up
      dW_gate = dHg^T x;  dW_up = dHu^T x;  dW_down = dy^T A
    Returns (dx, dw_gate, dw_up, dw_down) in fp64 (``dtype`` float32: the
    same steps in float32, for the timed CPU baseline)."""
    dy, x, w_gate, w_up, w_down = (np.asarray(a, dtype=dtype) for a in (dy, x, w_gate, w_up, w_down))
    T = x.shape[0]
    F = w_gate.shape[0]
    dx = np.zeros_like(x)
    dwg = np.zeros_like(w_gate)
    dwu = np.zeros_like(w_up)
    dwd = np.zeros_like(w_down)
    for t0 in range(0, T, chunk):
        xs = x[t0:t0 + chunk]
        dys = dy[t0:t0 + chunk]
        m = group_mask(None if idx is None else np.asarray(idx)[t0:t0 + chunk],
                       xs.shape[0], F, group_size, dtype)
        hg = xs @ w_gate.T
        hu = xs @ w_up.T
        s = sigmoid(hg)
        act = hg * s
        a = act * hu * m
        da = (dys @ w_down) * m
        dhu = da * act
        dhg = da * hu * s * (1.0 + hg * (1.0 - s))
        dx[t0:t0 + chunk] = dhg @ w_gate + dhu @ w_up
        dwg += dhg.T @ xs
        dwu += dhu.T @ xs
        dwd += dys.T @ a
    return dx, dwg, dwu, dwd


def swiglu_rows(x_rows, w_gate, w_up, w_down, idx_rows, group_size: int):
    """y for a few tokens only (each token's output depends on that token
    alone), for sampled checks at full sizes."""
    return sparse_swiglu_forward(x_rows, w_gate, w_up, w_down, idx_rows, group_size)


def dx_rows(dy_rows, x_rows, w_gate, w_up, w_down, idx_rows, group_size: int):
    """dx for a few tokens only."""
    return sparse_swiglu_backward(dy_rows, x_rows, w_gate, w_up, w_down, idx_rows, group_size)[0]


def dw_neuron_rows(neurons, dy, x, w_gate, w_up, w_down, idx, group_size: int, chunk: int = 8192):
    """Rows f of dW_gate and dW_up and columns f of dW_down for the listed
    neurons, summed over all tokens.  Each needs only the activations of
    neuron f, so full-size runs can be checked on a sample of neurons.
    Returns (dwg_rows [n, d], dwu_rows [n, d], dwd_cols [d, n])."""
    dy, x, w_gate, w_up, w_down = map(_f64, (dy, x, w_gate, w_up, w_down))
    neurons = np.asarray(neurons, dtype=np.int64)
    T = x.shape[0]
    d = x.shape[1]
    dwg = np.zeros((len(neurons), d))
    dwu = np.zeros((len(neurons), d))
    dwd = np.zeros((d, len(neurons)))
    groups_of = neurons // group_size
    for t0 in range(0, T, chunk):
        xs = x[t0:t0 + chunk]
        dys = dy[t0:t0 + chunk]
        if idx is None:
            m = np.ones((xs.shape[0], len(neurons)))
        else:
            ids = np.asarray(idx)[t0:t0 + chunk]
            m = (ids[:, :, None] == groups_of[None, None, :]).any(axis=1).astype(np.float64)
        hg = xs @ w_gate[neurons].T
        hu = xs @ w_up[neurons].T
        s = sigmoid(hg)
        act = hg * s
        da = (dys @ w_down[:, neurons]) * m
        dhu = da * act
        dhg = da * hu * s * (1.0 + hg * (1.0 - s))
        dwg += dhg.T @ xs
        dwu += dhu.T @ xs
        dwd += dys.T @ (act * hu * m)
    return dwg, dwu, dwd


# ---------------------------------------------------------------------------
# Load-balance bias update (README, "What it does": update_load_balance_bias,
# auxiliary-loss-free in the style of DeepSeek-V3, once per optimizer step;
# "Parameters and how to choose them": gamma 1e-3, bias_max 0.5, momentum
# 0.99, target = k / G).
#
# The page does not give the formula.  Reading taken: the frequency EMA is
# updated first, ema <- ema + (1 - momentum) * (cur - ema) (the usual EMA,
# written so that cur == ema leaves it unchanged exactly); then the bias moves
# by a fixed step gamma toward balance, bias <- clamp(bias + gamma *
# sign(target - ema), -bias_max, bias_max), with sign(0) = 0.  A step
# proportional to (target - ema) would move by ~1e-5 per call and could never
# approach the page's bias_max of 0.5, so the sign step is the reading the
# constants support.
# ---------------------------------------------------------------------------

def update_load_balance_bias(bias, freq_ema, current_freq, target_freq: float, gamma: float,
                             bias_max: float, momentum: float, dtype=np.float64):
    """Returns (new_bias, new_ema).  ``dtype`` selects the precision in which
    the sign decision is taken (float32 to match a float32 implementation
    operation for operation)."""
    t = np.dtype(dtype).type
    bias = np.asarray(bias, dtype=dtype)
    ema = np.asarray(freq_ema, dtype=dtype)
    cur = np.asarray(current_freq, dtype=dtype)
    one_minus = t(1.0) - t(momentum)
    new_ema = (ema + one_minus * (cur - ema)).astype(dtype)
    step = np.sign(t(target_freq) - new_ema).astype(dtype) * t(gamma)
    new_bias = np.clip(bias + step, -t(bias_max), t(bias_max)).astype(dtype)
    return new_bias, new_ema


def frequency_from_counts(counts, tokens: int, dtype=np.float64):
    """Fraction of tokens that selected each group; sums to k."""
    t = np.dtype(dtype).type
    return (np.asarray(counts, dtype=dtype) / t(tokens)).astype(dtype)
