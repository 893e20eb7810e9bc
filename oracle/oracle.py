"""Plain, slow fp64 CPU oracle of the hybrid block-sparse attention path.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of bench.py may import this module.  It shares no code with the
GPU library (no kernels, headers, helpers or constants) and imports nothing from
it; the two meet only in the seeded inputs from ``synth``.

What it computes, step by step, in float64 (bfloat16 inputs convert exactly):

1. Cube re-indexing of row-major video tokens.  VSA summary page ("VSA: Faster
   Video Diffusion with Trainable Sparse Attention"), section "Cube Partitioning
   and Token Re-Indexing": the block of token (t, h, w) is
   (t//ct)*Nh*Nw + (h//ch)*Nw + (w//cw); the within-cube term of that formula
   did not survive extraction, and row-major (t, h, w) order inside the cube is
   the reading taken here.  Grids whose sides are not multiples of the cube are
   padded per side ("Improving Video Sparse Attention with Fine-grained Router
   and Sparse Rebasing", section 2.2, "Kernel Implementation"); pad slots are
   excluded from pooling and masked out of attention.
2. Mean pooling of Q and K per block (SpargeAttention2 summary page, section
   "Block-Pooled Attention for Efficient Mask Construction", step 2; VSA page,
   "The Coarse Stage"), over the block's real tokens only.
3. Block scores S = Qbar Kbar^T / sqrt(d) and their row softmax P (SpargeAttention2
   page, same section, step 3).
4. Hybrid mask (SpargeAttention2 page, "The Hybrid Top-k+Top-p Masking Rule",
   Eq. 9): per row, the union of Top-k (the ceil(k*Tn) largest entries) and
   Top-p (the shortest prefix of the descending order whose cumulative
   probability reaches or exceeds p).  Both are prefixes of one order (score
   descending, lower block index first on equal scores), so the union is the
   longer prefix, max(kc, pc).  Kept blocks are listed in ascending id.
5. Block-sparse attention (SpargeAttention2 page, "Kernel Implementation of the
   Hybrid-Masked Block-Sparse Attention", Algorithm 1, and the renormalised
   sparse output o_s = (p*m/tau) V of "The Sparse Attention Error
   Decomposition"): each real query token attends, with a softmax over exactly
   the real keys of its row's kept blocks, to those keys; the natural-log
   log-sum-exp of its scaled scores is returned beside it.  This is the plain
   definition written out: no online softmax, no tiling.

6. Coarse branch output (VSA summary page, "The Coarse Stage"; "Improving
   Video Sparse Attention ...", section 2.2): attention at block granularity on
   the pooled Q, K and V, O_c = softmax(Qbar Kbar^T / sqrt(d)) Vbar, whose row i
   is repeated to every real token of block i.  The gate that mixes it with the
   fine output needs trained weights and is not part of this oracle.

7. Fine-grained router ("Improving Video Sparse Attention with Fine-grained
   Router and Sparse Rebasing", section 2.2, Figure 2, the router equations):
   Q and K are mean-pooled over sub-cubes of R = (rt, rh, rw) tokens (G = 64/R
   sub-cubes per cube), the router attention Softmax(Q_r K_r^T / sqrt(d)) is
   taken over all sub-cube keys of the head, and a G x G aggregation turns it
   into block-level scores P_r.  Readings: the aggregation sums over the key
   sub-cubes of a block and averages over the query sub-cubes, so each row of
   P_r is a probability row (it sums to 1) and the hybrid rule applies to it
   unchanged; sub-cubes holding only pad slots of a partial cube take no part
   (as keys or as queries).  The scores handed to the selection are log P_r,
   whose row softmax is P_r itself.

8. Backward pass of the block-sparse attention (the pages require the kernel
   to be differentiable for fine-tuning: SpargeAttention2 summary page, "Why
   this implementation is trainable"): the gradients of step 5's outputs with
   respect to Q, K and V, by the chain rule through the renormalised softmax
   over each row's kept real keys (the mask itself carries no gradient).

9. Mask-quality diagnostics (SpargeAttention2 summary page, "The Sparse
   Attention Error Decomposition", Eq. 8, and Table 1's L1 error; VSA summary
   page on the attention mass the selected cubes capture): per row the pooled
   probability mass the kept blocks hold; per query the true retained mass
   tau = sum of the dense softmax over the kept keys (the tau of Eq. 8); per
   query block the relative L1 error sum|o - o_s| / sum|o| of the sparse output
   against dense attention.

10. Asymmetric blocks (SpargeAttention2 summary page, "Block-Pooled Attention
   for Efficient Mask Construction": query blocks of b_q tokens and key blocks
   of b_kv tokens, b_q = 128 and b_kv = 64 there).  Reading in the cube-major
   order: a query block is qg consecutive cubes (qg = 2 gives 128 query
   slots), pooled over its real tokens; key blocks stay single cubes.  Each
   query block's row of nblk block scores is selected with the unchanged rule
   (kc = ceil(k * nblk)), and every cube of the group attends through that
   one list.

11. Per-sequence Top-K ("Improving Video Sparse Attention ...", section 1 and
   the ablation on the scope of the TopK selection): the budget is fixed for
   the whole sequence (one head) rather than per query block, so rows get
   different counts.  Reading: the budget equals per-row Top-k's total,
   T = rows * ceil(k * nblk); the T largest entries of the head's row-softmax
   block probabilities win, equal probabilities going to the lower row-major
   index first; each row's count c_i is how many of its entries won, and the
   row keeps its c_i top-scoring blocks (the Top-k rule with c_i for kc, so
   the selection within a row follows the scores as everywhere else).  A row
   may get no block at all.

12. Ideal block scores and mask recall ("Improving Video Sparse Attention ...",
   section 2.2: the oracle block scores MeanPool of the full attention matrix,
   the target a router approximates): P_ideal[i, j] is the full softmax mass
   that block i's real queries put on block j's real keys, averaged over those
   queries (every row sums to 1).  Recall of a kept list of c blocks: the share
   of the c blocks with the largest P_ideal (lower id first on equal values)
   that the list holds.  The retained mass of the list under P_ideal is the
   block mean of the tau of item 9.

13. Eq. 8's two error terms and a mask summary (SpargeAttention2 summary
   page, "The Sparse Attention Error Decomposition"; the sink rows of "Where
   Prior Approaches Fall Short"): per query block, the L1 norms of the dropped
   term p(1 - m)V and of the renormalisation term (1 - 1/tau)(p m)V relative
   to the dense output; per head, the realised block density, the mean block
   probability on block 0 and the mean row entropy of the block softmax.

Where the pages are silent or garbled, the reading taken is stated at the
function that depends on it.
Every function here is pinned by the CPU tests (worked examples, closed forms,
brute force, invariants, special cases).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

NEAR_TIE = 1e-6


# ----------------------------------------------------------------------------
# 1. geometry and re-indexing
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    frames: int
    height: int
    width: int
    ct: int = 4
    ch: int = 4
    cw: int = 4

    @property
    def block(self) -> int:
        return self.ct * self.ch * self.cw

    @property
    def nt(self) -> int:
        return -(-self.frames // self.ct)

    @property
    def nh(self) -> int:
        return -(-self.height // self.ch)

    @property
    def nw(self) -> int:
        return -(-self.width // self.cw)

    @property
    def nblk(self) -> int:
        return self.nt * self.nh * self.nw

    @property
    def n_real(self) -> int:
        return self.frames * self.height * self.width

    @property
    def n_pad(self) -> int:
        return self.nblk * self.block


def token_slots(g: Geometry) -> np.ndarray:
    """Cube-major padded slot of every row-major token n = t*H*W + h*W + w."""
    t, h, w = np.meshgrid(np.arange(g.frames), np.arange(g.height),
                          np.arange(g.width), indexing="ij")
    t, h, w = t.reshape(-1), h.reshape(-1), w.reshape(-1)
    blk = (t // g.ct) * (g.nh * g.nw) + (h // g.ch) * g.nw + (w // g.cw)
    within = ((t % g.ct) * g.ch + (h % g.ch)) * g.cw + (w % g.cw)
    return blk * g.block + within


def real_slots(g: Geometry) -> np.ndarray:
    """Boolean [n_pad]: True where a slot holds a real token."""
    m = np.zeros(g.n_pad, dtype=bool)
    m[token_slots(g)] = True
    return m


def reorder(x: np.ndarray, g: Geometry) -> np.ndarray:
    """[..., N, d] row-major tokens -> [..., n_pad, d] cube-major, pads = 0."""
    out = np.zeros(x.shape[:-2] + (g.n_pad, x.shape[-1]), dtype=x.dtype)
    out[..., token_slots(g), :] = x
    return out


def unreorder(xc: np.ndarray, g: Geometry) -> np.ndarray:
    """Inverse of reorder: [..., n_pad, d] -> [..., N, d] (pad slots dropped)."""
    return xc[..., token_slots(g), :]


def unreorder_rows(xc: np.ndarray, g: Geometry) -> np.ndarray:
    """Inverse re-indexing of a per-token scalar: [..., n_pad] -> [..., N]."""
    return xc[..., token_slots(g)]


# ----------------------------------------------------------------------------
# 2.-3. pooling, block scores, block softmax
# ----------------------------------------------------------------------------
def pool(xc: np.ndarray, g: Geometry) -> np.ndarray:
    """Mean of each block's real tokens: [..., n_pad, d] -> [..., nblk, d]."""
    xc = np.asarray(xc, dtype=np.float64)
    d = xc.shape[-1]
    blocks = xc.reshape(xc.shape[:-2] + (g.nblk, g.block, d))
    real = real_slots(g).reshape(g.nblk, g.block)
    total = (blocks * real[..., None]).sum(axis=-2)
    return total / real.sum(axis=1)[:, None]


def block_scores(qbar: np.ndarray, kbar: np.ndarray, d: int) -> np.ndarray:
    """S = Qbar Kbar^T / sqrt(d) over the last two axes."""
    return np.matmul(qbar, np.swapaxes(kbar, -1, -2)) / math.sqrt(d)


def block_softmax(s: np.ndarray) -> np.ndarray:
    """Row softmax in float64."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# 4. hybrid Top-k U Top-p selection
# ----------------------------------------------------------------------------
def ceil_k(k_frac: float, n: int) -> int:
    """Top-k count ceil(k * n).  Reading: k * n is meant in decimal arithmetic,
    so a binary-representation excess below 1e-9 does not round up (0.07 * 100
    is 7, not 8); the SpargeAttention2 page's worked count, 3% of 1562 blocks
    being 47, holds either way."""
    if n <= 0:
        return 0
    c = math.ceil(k_frac * n - 1e-9)
    return int(min(max(c, 0), n))


def rank_order(s_row: np.ndarray) -> np.ndarray:
    """Block ids sorted by score descending, lower id first on equal scores."""
    j = np.arange(s_row.shape[0])
    return np.lexsort((j, -s_row))


@dataclass
class RowSelection:
    kept: np.ndarray        # ascending block ids
    kc: int
    pc: int
    near_tie: bool
    order: np.ndarray
    cum: np.ndarray         # cumulative probability along `order`


def top_p_count(cum: np.ndarray, p: float) -> int:
    """Length of the shortest prefix whose cumulative probability >= p.
    p <= 0 keeps nothing and p >= 1 keeps everything (the exact-arithmetic
    answer, since no softmax entry is 0)."""
    n = cum.shape[0]
    if p <= 0.0:
        return 0
    if p >= 1.0:
        return n
    hit = np.nonzero(cum >= p)[0]
    return int(hit[0]) + 1 if hit.size else n


def select_row(s_row: np.ndarray, kc: int, p: float,
               probs: Optional[np.ndarray] = None) -> RowSelection:
    """Hybrid selection for one query block's row of block scores.

    ``probs`` defaults to the row softmax of ``s_row``; a test may pass exact
    probabilities for a worked example (the order still comes from s_row)."""
    s_row = np.asarray(s_row, dtype=np.float64)
    n = s_row.shape[0]
    if probs is None:
        probs = block_softmax(s_row)
    order = rank_order(s_row)
    cum = np.cumsum(probs[order])
    pc = top_p_count(cum, p)
    keep = max(kc, pc)
    kept = np.sort(order[:keep])
    near = _near_tie(s_row, order, cum, kc, pc, keep, p)
    return RowSelection(kept, kc, pc, near, order, cum)


def _near_tie(s_row, order, cum, kc, pc, keep, p) -> bool:
    """True when a perturbation of relative size < 1e-6 could change the kept
    set: (i) the last kept and first dropped scores differ by less than 1e-6 of
    the row's largest |score|; (ii) some prefix length whose cumulative
    probability lies within 1e-6 of p would give a different max(kc, pc)."""
    n = s_row.shape[0]
    scale = float(np.max(np.abs(s_row))) if n else 0.0
    if 0 < keep < n:
        gap = s_row[order[keep - 1]] - s_row[order[keep]]
        if gap <= NEAR_TIE * scale:
            return True
    if 0.0 < p < 1.0:
        prefix = np.concatenate(([0.0], cum))          # prefix[m] = sum of first m
        close = np.nonzero(np.abs(prefix - p) < NEAR_TIE)[0]
        for m in close:
            # the perturbed Top-p count is m (if prefix[m] >= p) or m + 1
            for alt in (int(m), int(m) + 1):
                if 0 <= alt <= n and max(kc, alt) != keep:
                    return True
    return False


@dataclass
class MaskResult:
    lut: np.ndarray         # [B, H, nblk, nblk] int32, -1 beyond counts
    counts: np.ndarray      # [B, H, nblk] int32
    near_tie: np.ndarray    # [B, H, nblk] bool
    kc: np.ndarray          # [B, H, nblk] int32
    pc: np.ndarray          # [B, H, nblk] int32
    scores: np.ndarray      # [B, H, nblk, nblk] float64
    qbar: np.ndarray
    kbar: np.ndarray


def build_mask(qc: np.ndarray, kc_: np.ndarray, g: Geometry, k_frac: float,
               p: float, row_budget: Optional[np.ndarray] = None) -> MaskResult:
    """Pool -> block scores -> hybrid selection for cube-major Q, K
    [B, H, n_pad, d].  With ``row_budget`` [B, H, nblk] each row keeps exactly
    its own count of top-scoring blocks (p must be 0): a per-query budget drawn
    independently of the scores, the variable-count case of the VSA2 page."""
    d = qc.shape[-1]
    qbar = pool(qc, g)
    kbar = pool(kc_, g)
    s = block_scores(qbar, kbar, d)
    B, H, n, _ = s.shape
    lut = np.full((B, H, n, n), -1, dtype=np.int32)
    counts = np.zeros((B, H, n), dtype=np.int32)
    flags = np.zeros((B, H, n), dtype=bool)
    kcs = np.zeros((B, H, n), dtype=np.int32)
    pcs = np.zeros((B, H, n), dtype=np.int32)
    k_default = ceil_k(k_frac, n)
    for b in range(B):
        for h in range(H):
            probs = block_softmax(s[b, h])
            for i in range(n):
                kc_i = k_default if row_budget is None else int(row_budget[b, h, i])
                sel = select_row(s[b, h, i], kc_i, p, probs[i])
                c = sel.kept.shape[0]
                lut[b, h, i, :c] = sel.kept
                counts[b, h, i] = c
                flags[b, h, i] = sel.near_tie
                kcs[b, h, i] = kc_i
                pcs[b, h, i] = sel.pc
    return MaskResult(lut, counts, flags, kcs, pcs, s, qbar, kbar)


def select_rows(s: np.ndarray, kc: int, p: float) -> List[RowSelection]:
    """Hybrid selection of every row of one head's [nblk, nblk] score matrix."""
    probs = block_softmax(s)
    return [select_row(s[i], kc, p, probs[i]) for i in range(s.shape[0])]


# ----------------------------------------------------------------------------
# 5. block-sparse attention (renormalised over the kept real keys)
# ----------------------------------------------------------------------------
def attention_block(qc_h: np.ndarray, kc_h: np.ndarray, vc_h: np.ndarray,
                    kept: Sequence[int], g: Geometry, i: int,
                    scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O [block, d] and LSE [block] of query block i of one (batch, head).

    Each real query attends to the real keys of the kept blocks with a softmax
    over exactly those keys; pad query slots, and every slot of a row that keeps
    no block, get O = 0 and LSE = -inf."""
    B_ = g.block
    d = qc_h.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    real = real_slots(g)
    o = np.zeros((B_, d), dtype=np.float64)
    lse = np.full(B_, -np.inf, dtype=np.float64)
    kept = list(kept)
    if not kept:
        return o, lse
    key_slots = np.concatenate([np.arange(j * B_, (j + 1) * B_) for j in kept])
    key_slots = key_slots[real[key_slots]]
    k = np.asarray(kc_h[key_slots], dtype=np.float64)
    v = np.asarray(vc_h[key_slots], dtype=np.float64)
    q_slots = np.arange(i * B_, (i + 1) * B_)
    qmask = real[q_slots]
    q = np.asarray(qc_h[q_slots[qmask]], dtype=np.float64)
    s = (q @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o[qmask] = (e @ v) / l
    lse[qmask] = (m + np.log(l))[:, 0]
    return o, lse


def sparse_attention(qc: np.ndarray, kc_: np.ndarray, vc: np.ndarray,
                     lut: np.ndarray, counts: np.ndarray, g: Geometry,
                     scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Block-sparse attention of every row: O [B, H, n_pad, d], LSE [B, H, n_pad]."""
    B, H, n_pad, d = qc.shape
    o = np.zeros((B, H, n_pad, d), dtype=np.float64)
    lse = np.full((B, H, n_pad), -np.inf, dtype=np.float64)
    blk = g.block
    for b in range(B):
        for h in range(H):
            for i in range(g.nblk):
                kept = lut[b, h, i, :counts[b, h, i]]
                ob, lb = attention_block(qc[b, h], kc_[b, h], vc[b, h], kept, g, i, scale)
                o[b, h, i * blk:(i + 1) * blk] = ob
                lse[b, h, i * blk:(i + 1) * blk] = lb
    return o, lse


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Full softmax attention over the last two axes, O and natural-log LSE."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * scale
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return np.matmul(e, v) / l, (m + np.log(l))[..., 0]


# ----------------------------------------------------------------------------
# 6. coarse branch output
# ----------------------------------------------------------------------------
def coarse_output(qc: np.ndarray, kc_: np.ndarray, vc: np.ndarray, g: Geometry,
                  scale: Optional[float] = None) -> np.ndarray:
    """Block-level attention on pooled tokens: [..., n_pad, d] x3 -> [..., nblk, d].

    VSA summary page, "The Coarse Stage": queries, keys and values are
    mean-pooled per cube (real tokens only, as in step 2) and attend to each
    other at block granularity; row i is the coarse output of every token of
    block i."""
    qbar, kbar, vbar = pool(qc, g), pool(kc_, g), pool(vc, g)
    d = qbar.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    p = block_softmax(np.matmul(qbar, np.swapaxes(kbar, -1, -2)) * scale)
    return np.matmul(p, vbar)


def expand_blocks(xb: np.ndarray, g: Geometry) -> np.ndarray:
    """Repeat each block row to the block's real token slots (pads get 0):
    [..., nblk, d] -> [..., n_pad, d] in cube-major slot order."""
    out = np.repeat(np.asarray(xb, dtype=np.float64), g.block, axis=-2)
    out[..., ~real_slots(g), :] = 0.0
    return out


# ----------------------------------------------------------------------------
# 7. fine-grained router (sub-cube pooling, softmax, G x G aggregation)
# ----------------------------------------------------------------------------
def subcube_of_slot(g: Geometry, R: Tuple[int, int, int]) -> np.ndarray:
    """Sub-cube index a in [0, G) of each of the 64 slots of a cube, for
    sub-cubes of rt x rh x rw tokens (row-major over the sub-cube grid)."""
    rt, rh, rw = R
    if g.ct % rt or g.ch % rh or g.cw % rw:
        raise ValueError("the sub-cube must tile the cube")
    s = np.arange(g.block)
    tt, rem = np.divmod(s, g.ch * g.cw)
    hh, ww = np.divmod(rem, g.cw)
    return ((tt // rt) * (g.ch // rh) + hh // rh) * (g.cw // rw) + ww // rw


def pool_r(xc: np.ndarray, g: Geometry, R: Tuple[int, int, int]):
    """Sub-cube means over real tokens: [..., n_pad, d] -> ([..., nblk*G, d],
    present [nblk*G]); a sub-cube with no real token has mean 0 and is absent."""
    xc = np.asarray(xc, dtype=np.float64)
    d = xc.shape[-1]
    G = g.block // (R[0] * R[1] * R[2])
    sub = subcube_of_slot(g, R)
    real = real_slots(g).reshape(g.nblk, g.block)
    blocks = xc.reshape(xc.shape[:-2] + (g.nblk, g.block, d))
    sums = np.zeros(xc.shape[:-2] + (g.nblk, G, d))
    cnt = np.zeros((g.nblk, G))
    for a in range(G):
        w = real & (sub == a)[None, :]
        sums[..., a, :] = (blocks * w[..., None]).sum(axis=-2)
        cnt[:, a] = w.sum(axis=1)
    present = cnt > 0
    means = np.where(present[..., None], sums / np.maximum(cnt, 1)[..., None], 0.0)
    return means.reshape(xc.shape[:-2] + (g.nblk * G, d)), present.reshape(-1)


def router_scores(qc: np.ndarray, kc_: np.ndarray, g: Geometry, R: Tuple[int, int, int] = (2, 2, 2),
                  scale: Optional[float] = None) -> np.ndarray:
    """log P_r of one or more heads: [..., n_pad, d] x2 -> [..., nblk, nblk].

    P_hat = Softmax(Q_r K_r^T * scale) over the present sub-cube keys of the
    head; P_r[i, j] = mean over the present query sub-cubes a of block i of
    sum over the key sub-cubes b of block j of P_hat[(i, a), (j, b)]."""
    qr, present = pool_r(qc, g, R)
    kr, _ = pool_r(kc_, g, R)
    d = qr.shape[-1]
    G = g.block // (R[0] * R[1] * R[2])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = np.matmul(qr, np.swapaxes(kr, -1, -2)) * scale
    s = np.where(present[None, :], s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p = p / p.sum(axis=-1, keepdims=True)
    lead = p.shape[:-2]
    p = p.reshape(lead + (g.nblk, G, g.nblk, G))
    per_query = p.sum(axis=-1)                                   # [..., i, a, j]
    pres = present.reshape(g.nblk, G)
    pr = (per_query * pres[:, :, None]).sum(axis=-2) / pres.sum(axis=1)[:, None]
    with np.errstate(divide="ignore"):
        return np.log(pr)


# ----------------------------------------------------------------------------
# 8. backward pass of the block-sparse attention
# ----------------------------------------------------------------------------
def sparse_attention_backward(qc: np.ndarray, kc_: np.ndarray, vc: np.ndarray, doc: np.ndarray,
                              lut: np.ndarray, counts: np.ndarray, g: Geometry,
                              scale: Optional[float] = None):
    """dQ, dK, dV [B, H, n_pad, d] of L = sum(dO * O) for step 5's O.

    Per query block i with kept real keys y and its real queries x:
    P = softmax(q k^T * scale) over those keys, O = P v, D_x = sum_c dO_xc O_xc,
    dV_y += P^T dO, dP = dO v^T, dS = P * (dP - D), dQ_x = scale dS k,
    dK_y += scale dS^T q.  Pad slots get zero gradients."""
    B, H, n_pad, d = qc.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    real = real_slots(g)
    blk = g.block
    dq = np.zeros((B, H, n_pad, d))
    dk = np.zeros((B, H, n_pad, d))
    dv = np.zeros((B, H, n_pad, d))
    for b in range(B):
        for h in range(H):
            q_h = np.asarray(qc[b, h], dtype=np.float64)
            k_h = np.asarray(kc_[b, h], dtype=np.float64)
            v_h = np.asarray(vc[b, h], dtype=np.float64)
            do_h = np.asarray(doc[b, h], dtype=np.float64)
            for i in range(g.nblk):
                kept = list(lut[b, h, i, :counts[b, h, i]])
                if not kept:
                    continue
                ys = np.concatenate([np.arange(j * blk, (j + 1) * blk) for j in kept])
                ys = ys[real[ys]]
                xs = np.arange(i * blk, (i + 1) * blk)
                xs = xs[real[xs]]
                s = (q_h[xs] @ k_h[ys].T) * scale
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                o = p @ v_h[ys]
                dO = do_h[xs]
                D = (dO * o).sum(axis=1, keepdims=True)
                dv[b, h, ys] += p.T @ dO
                dp = dO @ v_h[ys].T
                ds = p * (dp - D)
                dq[b, h, xs] += scale * (ds @ k_h[ys])
                dk[b, h, ys] += scale * (ds.T @ q_h[xs])
    return dq, dk, dv


# ----------------------------------------------------------------------------
# 9. mask-quality diagnostics
# ----------------------------------------------------------------------------
def pooled_mass(scores: np.ndarray, lut: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """Per row: sum over the kept blocks of the row softmax of the scores."""
    p = block_softmax(np.asarray(scores, dtype=np.float64))
    out = np.zeros(counts.shape)
    for idx in np.ndindex(counts.shape):
        out[idx] = p[idx][lut[idx][:counts[idx]]].sum()
    return out


def mask_error(qc: np.ndarray, kc_: np.ndarray, vc: np.ndarray, lut: np.ndarray, counts: np.ndarray,
               g: Geometry, scale: Optional[float] = None):
    """tau [B, H, n_pad] (dense softmax mass on the kept real keys; 0 on pad
    slots) and rel_l1 [B, H, nblk] (sum|o - o_s| / sum|o| over the block's real
    queries) of the sparse output o_s against dense attention o."""
    B, H, n_pad, d = qc.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    real = real_slots(g)
    blk = g.block
    tau = np.zeros((B, H, n_pad))
    rel = np.zeros((B, H, g.nblk))
    o_s, _ = sparse_attention(qc, kc_, vc, lut, counts, g, scale)
    for b in range(B):
        for h in range(H):
            q = np.asarray(qc[b, h], dtype=np.float64)[real]
            k = np.asarray(kc_[b, h], dtype=np.float64)[real]
            v = np.asarray(vc[b, h], dtype=np.float64)[real]
            s = (q @ k.T) * scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = np.zeros((n_pad, d))
            o[real] = p @ v
            key_blk = np.nonzero(real)[0] // blk
            t = np.zeros(n_pad)
            for i in range(g.nblk):
                kept = np.zeros(g.nblk, dtype=bool)
                kept[lut[b, h, i, :counts[b, h, i]]] = True
                rows = np.arange(i * blk, (i + 1) * blk)
                rows = rows[real[rows]]
                ridx = np.searchsorted(np.nonzero(real)[0], rows)
                t[rows] = p[ridx][:, kept[key_blk]].sum(axis=1)
                num = np.abs(o[rows] - o_s[b, h, rows]).sum()
                den = np.abs(o[rows]).sum()
                rel[b, h, i] = num / den if den > 0 else 0.0
            tau[b, h] = t
    return tau, rel


def error_terms(qc: np.ndarray, kc_: np.ndarray, vc: np.ndarray, lut: np.ndarray, counts: np.ndarray,
                g: Geometry, scale: Optional[float] = None):
    """The two terms of Eq. 8 (SpargeAttention2 summary page, "The Sparse
    Attention Error Decomposition") per query block, as L1 norms relative to
    the dense output: for each real query with dense softmax p over the real
    keys, kept-key indicator m and tau = sum(p * m),
        dropped term       e_drop = (p * (1 - m)) V,
        renormalisation    e_ren  = (1 - 1/tau) (p * m) V,
    and per block rel_drop = sum|e_drop| / sum|o|, rel_ren = sum|e_ren| / sum|o|
    with o = p V, summed over the block's real queries and the d channels.
    A query whose kept keys hold no mass (tau = 0) has no renormalised output;
    its renormalisation term is taken as 0.  Returns [B, H, nblk] twice."""
    B, H, n_pad, d = qc.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    real = real_slots(g)
    real_idx = np.nonzero(real)[0]
    key_blk = real_idx // g.block
    drop = np.zeros((B, H, g.nblk))
    ren = np.zeros((B, H, g.nblk))
    for b in range(B):
        for h in range(H):
            q = np.asarray(qc[b, h], dtype=np.float64)
            k = np.asarray(kc_[b, h], dtype=np.float64)[real]
            v = np.asarray(vc[b, h], dtype=np.float64)[real]
            for i in range(g.nblk):
                m = np.isin(key_blk, lut[b, h, i, :counts[b, h, i]]).astype(np.float64)
                num_d = num_r = den = 0.0
                for x in range(i * g.block, (i + 1) * g.block):
                    if not real[x]:
                        continue
                    s = (k @ q[x]) * scale
                    p = np.exp(s - s.max())
                    p /= p.sum()
                    tau = float((p * m).sum())
                    e_drop = (p * (1.0 - m)) @ v
                    e_ren = (1.0 - 1.0 / tau) * ((p * m) @ v) if tau > 0 else np.zeros(d)
                    num_d += np.abs(e_drop).sum()
                    num_r += np.abs(e_ren).sum()
                    den += np.abs(p @ v).sum()
                drop[b, h, i] = num_d / den if den > 0 else 0.0
                ren[b, h, i] = num_r / den if den > 0 else 0.0
    return drop, ren


def mask_report(scores: np.ndarray, counts: np.ndarray):
    """Per (batch, head) summary of a mask and the block softmax it was chosen
    on: realised block density sum(counts) / nblk^2, the mean sink mass
    P[:, 0] (the share of each row's block probability on block 0, where the
    SpargeAttention2 page's skewed "sink" rows put most of it), and the mean
    row entropy -sum_j P_ij ln P_ij (ln nblk for a uniform row, near 0 for a
    row held by one block).  Returns (density, sink, entropy), each [B, H]."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[-1]
    p = block_softmax(s)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    density = np.asarray(counts, dtype=np.float64).sum(axis=-1) / float(n * n)
    sink = p[..., 0].mean(axis=-1)
    entropy = (-plogp.sum(axis=-1)).mean(axis=-1)
    return density, sink, entropy


# ----------------------------------------------------------------------------
# 10. asymmetric blocks: query blocks of qg cubes, key blocks of one cube
# ----------------------------------------------------------------------------
def group_count(nblk: int, qg: int) -> int:
    """Query blocks per head when each holds qg consecutive cubes (the last
    one may hold fewer)."""
    return -(-nblk // qg)


def pool_groups(xc: np.ndarray, g: Geometry, qg: int) -> np.ndarray:
    """Mean over the real tokens of each group of qg consecutive blocks:
    [..., n_pad, d] -> [..., ceil(nblk / qg), d]."""
    xc = np.asarray(xc, dtype=np.float64)
    d = xc.shape[-1]
    real = real_slots(g)
    nq = group_count(g.nblk, qg)
    out = np.zeros(xc.shape[:-2] + (nq, d))
    for a in range(nq):
        lo, hi = a * qg * g.block, min((a + 1) * qg, g.nblk) * g.block
        keep = np.nonzero(real[lo:hi])[0] + lo
        out[..., a, :] = xc[..., keep, :].sum(axis=-2) / keep.size
    return out


def build_mask_groups(qc: np.ndarray, kc_: np.ndarray, g: Geometry, qg: int,
                      k_frac: float, p: float) -> MaskResult:
    """Pool (queries per group of qg cubes, keys per cube) -> block scores
    [B, H, nq, nblk] -> hybrid selection of every query block's row with
    kc = ceil(k_frac * nblk).  Lists are [B, H, nq, nblk]."""
    d = qc.shape[-1]
    qbar = pool_groups(qc, g, qg)
    kbar = pool(kc_, g)
    s = block_scores(qbar, kbar, d)
    B, H, nq, n = s.shape
    lut = np.full((B, H, nq, n), -1, dtype=np.int32)
    counts = np.zeros((B, H, nq), dtype=np.int32)
    flags = np.zeros((B, H, nq), dtype=bool)
    pcs = np.zeros((B, H, nq), dtype=np.int32)
    kc = ceil_k(k_frac, n)
    for b in range(B):
        for h in range(H):
            probs = block_softmax(s[b, h])
            for i in range(nq):
                sel = select_row(s[b, h, i], kc, p, probs[i])
                c = sel.kept.shape[0]
                lut[b, h, i, :c] = sel.kept
                counts[b, h, i] = c
                flags[b, h, i] = sel.near_tie
                pcs[b, h, i] = sel.pc
    return MaskResult(lut, counts, flags, np.full((B, H, nq), kc, dtype=np.int32), pcs, s, qbar, kbar)


def expand_group_lists(lut: np.ndarray, counts: np.ndarray, qg: int, nblk: int):
    """Per-cube lists for sparse_attention: cube i uses the list of its query
    block i // qg."""
    rows = np.arange(nblk) // qg
    return lut[..., rows, :], counts[..., rows]


# ----------------------------------------------------------------------------
# 11. per-sequence Top-K: one budget per head, variable counts per row
# ----------------------------------------------------------------------------
def sequence_budget(rows: int, nblk: int, k_frac: float) -> int:
    """The head's total: what per-row Top-k would keep."""
    return rows * ceil_k(k_frac, nblk)


def per_sequence_counts(s: np.ndarray, total: int) -> np.ndarray:
    """Per-row counts of the `total` largest entries of the row softmax of one
    head's scores [rows, nblk]; equal probabilities go to the lower row-major
    index first."""
    prob = block_softmax(np.asarray(s, dtype=np.float64))
    flat = prob.reshape(-1)
    order = np.lexsort((np.arange(flat.size), -flat))
    won = np.zeros(flat.size, dtype=bool)
    won[order[:max(0, min(total, flat.size))]] = True
    return won.reshape(prob.shape).sum(axis=1).astype(np.int32)


def per_sequence_near_tie(s: np.ndarray, total: int) -> np.ndarray:
    """Rows whose count could change under a relative perturbation below 1e-6
    of the probabilities: rows holding an entry within that margin of the
    last winning probability (when a losing entry lies within it too)."""
    prob = block_softmax(np.asarray(s, dtype=np.float64))
    flat = np.sort(prob.reshape(-1))[::-1]
    if total <= 0 or total >= flat.size:
        return np.zeros(prob.shape[0], dtype=bool)
    last, first_out = flat[total - 1], flat[total]
    if last - first_out > NEAR_TIE * last:
        return np.zeros(prob.shape[0], dtype=bool)
    close = np.abs(prob - last) <= NEAR_TIE * last
    return close.any(axis=1)


def build_mask_per_sequence(qc: np.ndarray, kc_: np.ndarray, g: Geometry, k_frac: float) -> MaskResult:
    """Pool -> block scores -> per-head budget T = nblk * ceil(k * nblk) ->
    per-row counts -> each row's top-scoring blocks (lists [B, H, nblk, nblk])."""
    d = qc.shape[-1]
    qbar = pool(qc, g)
    kbar = pool(kc_, g)
    s = block_scores(qbar, kbar, d)
    B, H, n, _ = s.shape
    lut = np.full((B, H, n, n), -1, dtype=np.int32)
    counts = np.zeros((B, H, n), dtype=np.int32)
    flags = np.zeros((B, H, n), dtype=bool)
    kcs = np.zeros((B, H, n), dtype=np.int32)
    total = sequence_budget(n, n, k_frac)
    for b in range(B):
        for h in range(H):
            c = per_sequence_counts(s[b, h], total)
            flags[b, h] = per_sequence_near_tie(s[b, h], total)
            probs = block_softmax(s[b, h])
            for i in range(n):
                sel = select_row(s[b, h, i], int(c[i]), 0.0, probs[i])
                lut[b, h, i, :sel.kept.size] = sel.kept
                counts[b, h, i] = sel.kept.size
                flags[b, h, i] |= sel.near_tie
                kcs[b, h, i] = c[i]
    return MaskResult(lut, counts, flags, kcs, np.zeros((B, H, n), dtype=np.int32), s, qbar, kbar)


# ----------------------------------------------------------------------------
# 12. ideal block scores (block-pooled full attention) and mask recall
# ----------------------------------------------------------------------------
def ideal_block_mass(qc: np.ndarray, kc_: np.ndarray, g: Geometry,
                     scale: Optional[float] = None) -> np.ndarray:
    """P_ideal [B, H, nblk, nblk]: mean over block i's real queries of the
    full softmax mass on block j's real keys."""
    B, H, n_pad, d = qc.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    real = real_slots(g)
    blk_of = np.nonzero(real)[0] // g.block
    out = np.zeros((B, H, g.nblk, g.nblk))
    for b in range(B):
        for h in range(H):
            q = np.asarray(qc[b, h], dtype=np.float64)[real]
            k = np.asarray(kc_[b, h], dtype=np.float64)[real]
            s_ = (q @ k.T) * scale
            p = np.exp(s_ - s_.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            per_key_block = np.zeros((p.shape[0], g.nblk))
            np.add.at(per_key_block.T, blk_of, p.T)
            for i in range(g.nblk):
                out[b, h, i] = per_key_block[blk_of == i].mean(axis=0)
    return out


def mask_recall(mass: np.ndarray, lut: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """Per row: |kept & top-c of mass| / c (c = the row's count; 1 when c = 0)."""
    out = np.ones(counts.shape)
    for idx in np.ndindex(counts.shape):
        c = int(counts[idx])
        if c == 0:
            continue
        top = rank_order(np.asarray(mass[idx], dtype=np.float64))[:c]
        out[idx] = np.intersect1d(top, lut[idx][:c]).size / c
    return out
