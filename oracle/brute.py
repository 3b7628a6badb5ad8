"""Pure-Python constructions for tiny cases, independent of ``bda_oracle.c``.

TEST INFRASTRUCTURE ONLY (used by the oracle pin tests).  Each function builds
the same object as the C oracle by a different route, so that a slip in one
(a wrong inequality, a swapped half, a dropped term) shows up as a mismatch.
"""
from __future__ import annotations

import itertools
import math


def blocks_of(L: int, b: int):
    """Block partition of positions 0..L-1 into runs of b (last one short)."""
    return [list(range(s, min(L, s + b))) for s in range(0, L, b)]


def hybrid_mask_kron(L: int, b: int):
    """Hybrid mask from its block-matrix form over [x_t ; x_0]:

        [[ I_K (x) J_b ,  Lstrict_K (x) J_b ],
         [      0      ,  Lincl_K   (x) J_b ]]

    with K = ceil(L/b) blocks, J_b the all-ones b x b block, I_K the identity,
    Lstrict / Lincl the strictly / non-strictly lower-triangular K x K ones
    matrices; built at size K*b and then trimmed to L per half (short last
    block).  Names follow the training-form mask of the Nemotron-Labs-Diffusion
    3x page, sec. 1 (block-diagonal, offset block-causal, block-causal).
    """
    K = -(-L // b)
    n = K * b

    def kron(A, size):
        return [[A[i // b][j // b] for j in range(size)] for i in range(size)]

    I = [[1 if i == j else 0 for j in range(K)] for i in range(K)]
    Ls = [[1 if j < i else 0 for j in range(K)] for i in range(K)]
    Li = [[1 if j <= i else 0 for j in range(K)] for i in range(K)]
    BD, OBC, BC = kron(I, n), kron(Ls, n), kron(Li, n)
    M = [[0] * (2 * L) for _ in range(2 * L)]
    for i in range(L):
        for j in range(L):
            M[i][j] = BD[i][j]            # x_t -> x_t
            M[i][L + j] = OBC[i][j]       # x_t -> x_0
            M[L + i][L + j] = BC[i][j]    # x_0 -> x_0
            M[L + i][j] = 0               # x_0 -> x_t never
    return M


def hybrid_mask_enum(L: int, b: int):
    """Hybrid mask by enumerating, for each query, the key SET that the BDLM
    conditioning names (LLaDA2.0-Uni page, training objective): the noisy
    block k is predicted from the clean blocks before k and from itself; a
    clean block k sees the clean blocks up to and including k."""
    blks = blocks_of(L, b)
    M = [[0] * (2 * L) for _ in range(2 * L)]
    for k, members in enumerate(blks):
        clean_before = [L + p for kk in range(k) for p in blks[kk]]
        noisy_k = list(members)
        clean_upto = clean_before + [L + p for p in members]
        for p in members:
            for j in noisy_k + clean_before:
                M[p][j] = 1
            for j in clean_upto:
                M[L + p][j] = 1
    return M


def decode_mask_enum(L: int, n: int):
    return [[1] * L for _ in range(n)]


def causal_mask_enum(L: int, n: int):
    """Query i is the key at position L-n+i; it sees that key and all before."""
    return [[1 if j <= L - n + i else 0 for j in range(L)] for i in range(n)]


def attention_loops(q, k, v, M, scale):
    """Plain loops over one head: q [R][d], k/v [S][d], M [R][S] of 0/1."""
    out = []
    for i, qi in enumerate(q):
        s = {j: scale * sum(a * c for a, c in zip(qi, k[j])) for j in range(len(k)) if M[i][j]}
        m = max(s.values())
        w = {j: math.exp(x - m) for j, x in s.items()}
        Z = sum(w.values())
        out.append([sum(w[j] * v[j][c] for j in w) / Z for c in range(len(v[0]))])
    return out


def commit_subset(p, masked, tau, k_min):
    """The committed set by search over all subsets of the masked rows.

    A subset S is admissible when (SPRINT's acceptance rule with its per-step
    minimum, LLaDA2.0-Uni page, and the block-refinement scheduler's
    threshold-plus-quota rule, DiffusionGemma page):
      * every masked row with p > tau is in S (threshold rows are never capped);
      * |S| = max(#{p > tau}, min(k_min, #masked));
      * every row of S that is not above tau has p at least that of every
        masked row left out, and on equal p the lower row index is taken first.
    Returns the unique admissible S as a sorted tuple (raises if not unique).
    """
    rows = [r for r in range(len(p)) if masked[r]]
    above = {r for r in rows if p[r] > tau}
    size = max(len(above), min(k_min, len(rows)))
    found = []
    for S in itertools.combinations(rows, size):
        S = set(S)
        if not above <= S:
            continue
        out = [r for r in rows if r not in S]
        ok = True
        for r in S - above:
            for o in out:
                if p[o] > p[r] or (p[o] == p[r] and o < r):
                    ok = False
        if ok:
            found.append(tuple(sorted(S)))
    if len(found) != 1:
        raise AssertionError(f"admissible sets: {found}")
    return found[0]
