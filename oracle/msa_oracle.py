"""MSA oracle: a plain, slow, fp64 CPU statement of what the hot path computes.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call this module.  It shares no
code, tables or helpers with the HIP library, and imports nothing from it.

Sources (the pages on MiniMax Sparse Attention, "MSA"):

* [GUIDE/roles]   ai-tool-zukan.com/minimax-msa-guide, section
  "Index BranchとMain Branchの役割分担" and its pseudocode figure: one index-query
  head per GQA group plus one shared index-key head; score -> top_k(k=16) ->
  ensure_local_block -> exact softmax attention over the selection.
* [GUIDE/two-stage] same page, section "2段階構造の中身": index scores on the
  visible key tokens, max-pooled to block level; top-k blocks per (query,
  group); the query's own block always included; exact softmax over the
  selected blocks.
* [GUIDE/group]   same page, section "GQAグループ単位の選択共有とは": one block
  set per group, shared by the group's query heads, independent across groups.
* [GUIDE/local]   same page, section "クエリを含むローカルブロックの強制取り込み".
* [GUIDE/numbers] same page, table in section "ブロック単位選択の数値設計":
  B_k = 128 tokens, k = 16 blocks, fixed budget k*B_k = 2,048 tokens.
* [GUIDE/what]    same page, section "MiniMax MSAとは何か": GQA backbone; exact
  softmax attention over only the selected blocks.
* [TNK/impl]      tnkblog.net MiniMax M3 MSA post, section "MSA の実装": KV block
  as the outer loop, gather the queries that hit it.

Readings taken where the pages are silent (each is the plainest reading):

R1  score = raw dot product q_idx . k_idx (no scale, no activation; any strictly
    increasing per-row transform leaves the selection unchanged).
R2  the forced local block is one of the k (local + top-(k-1) others), which
    keeps the 2,048-token budget of [GUIDE/numbers].
R3  visibility is causal (j <= p) in both branches, inside the local block too.
R4  fewer than k visible blocks: take them all; pad the output with -1.
R5  ties between equal block scores: the lower block id wins.
R6  selection output is in ascending block id.
R7  head h belongs to group h // (Hq / Hkv).
R8  softmax scale defaults to 1/sqrt(head_dim).
R9  the Main Branch output is plain softmax attention (no gate, no weighting by
    index scores).
R10 blocks start at position 0 of each sequence; query i of a sequence with
    Lq queries and Lk keys sits at position Lk - Lq + i.
R11 inputs are bf16; the oracle computes in fp64 on their exact values.

Every function below is pinned by ``tests/test_oracle_*.py`` against closed
forms, constructed inputs with known answers, brute force, and library
routines (torch's scaled_dot_product_attention in float64) -- see each test.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 128          # B_k  [GUIDE/numbers]
TOP_K = 16           # k    [GUIDE/numbers]
ENTRY_SLOT_BITS = 5  # list entries pack (query row, slot) as row * 32 + slot


# ----------------------------------------------------------------------------
# positions (reading R10)
# ----------------------------------------------------------------------------
def query_positions(cu_seqlens_q, cu_seqlens_k):
    """Per global query row: (sequence id, position in its sequence, key offset)."""
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    seq, pos, koff = [], [], []
    for b in range(len(cu_q) - 1):
        lq = cu_q[b + 1] - cu_q[b]
        lk = cu_k[b + 1] - cu_k[b]
        for i in range(lq):
            seq.append(b)
            pos.append(lk - lq + i)
            koff.append(cu_k[b])
    return (np.asarray(seq, dtype=np.int64), np.asarray(pos, dtype=np.int64),
            np.asarray(koff, dtype=np.int64))


# ----------------------------------------------------------------------------
# Index Branch  [GUIDE/roles], [GUIDE/two-stage]
# ----------------------------------------------------------------------------
def index_token_scores(q_idx_row, k_idx_seq, p):
    """s[g, j] = q_idx[p, g, :] . k_idx[j, :] for the visible keys 0 <= j <= p.

    One index-query head per group against the single shared index-key head
    ([GUIDE/roles]); only visible (causal) keys are scored ([GUIDE/two-stage],
    R1, R3).  Returns fp64 [G, p + 1].
    """
    q = np.asarray(q_idx_row, dtype=np.float64)                # [G, d_idx]
    k = np.asarray(k_idx_seq[: p + 1], dtype=np.float64)       # [p+1, d_idx]
    return q @ k.T


def block_max_pool(s, p, block=BLOCK):
    """S[g, beta] = max of s[g, j] over the visible tokens j of block beta.

    Max-pooling of token scores to block level ([GUIDE/two-stage]).  Covers
    blocks 0 .. beta(p); the local block's entry uses only j <= p.
    """
    nbv = p // block + 1
    G = s.shape[0]
    S = np.empty((G, nbv), dtype=np.float64)
    for beta in range(nbv):
        lo = beta * block
        hi = min((beta + 1) * block, p + 1)
        S[:, beta] = s[:, lo:hi].max(axis=1)
    return S


def select_blocks(S_g, beta_p, top_k):
    """Selected blocks of one (query, group), ascending ([GUIDE/two-stage]).

    The query's own block beta_p is always in ([GUIDE/local]); the other
    top_k - 1 are the best non-local visible blocks by (score descending,
    block id ascending) (R2, R5).  With fewer than top_k - 1 non-local blocks
    all of them are taken (R4).  Uses a full sort, the definition of top-k.
    """
    if top_k < 1:
        raise ValueError("top_k >= 1")
    others = list(range(beta_p))
    if len(others) > top_k - 1:
        others = sorted(others, key=lambda b: (-float(S_g[b]), b))[: top_k - 1]
    return sorted(others + [beta_p])


# ----------------------------------------------------------------------------
# Main Branch  [GUIDE/what], [GUIDE/two-stage], [GUIDE/group]
# ----------------------------------------------------------------------------
def selected_keys(sel_blocks, p, block=BLOCK):
    """J = { j <= p : beta(j) in Sel } in ascending order (R3)."""
    idx = []
    for beta in sorted(sel_blocks):
        lo = beta * block
        hi = min((beta + 1) * block, p + 1)
        idx.extend(range(lo, hi))
    return np.asarray(idx, dtype=np.int64)


def attend_row(q_row, k_seq, v_seq, p, sel_by_group, scale, block=BLOCK):
    """Exact softmax attention of one query over its selected keys.

    For head h of group g = h // (Hq/G) (R7), the keys are J(p, g) =
    visible tokens of the group's selected blocks, shared by all heads of
    the group ([GUIDE/group]); the output is plain softmax attention over J
    ([GUIDE/what], R9).  Returns (out [Hq, d], lse [Hq]) in fp64.
    """
    q = np.asarray(q_row, dtype=np.float64)                     # [Hq, d]
    Hq, d = q.shape
    G = len(sel_by_group)
    hpg = Hq // G
    out = np.empty((Hq, d), dtype=np.float64)
    lse = np.empty((Hq,), dtype=np.float64)
    for g in range(G):
        J = selected_keys(sel_by_group[g], p, block)
        K = np.asarray(k_seq[J, g], dtype=np.float64)           # [|J|, d]
        V = np.asarray(v_seq[J, g], dtype=np.float64)
        for h in range(g * hpg, (g + 1) * hpg):
            z = scale * (K @ q[h])
            m = z.max()
            w = np.exp(z - m)
            tot = w.sum()
            out[h] = (w @ V) / tot
            lse[h] = m + math.log(tot)
    return out, lse


def block_partial(q_vec, k_seq, v_seq, p, beta, g, scale, block=BLOCK):
    """Softmax partial (m, l, acc) of one query head over one block's visible keys."""
    J = selected_keys([beta], p, block)
    K = np.asarray(k_seq[J, g], dtype=np.float64)
    V = np.asarray(v_seq[J, g], dtype=np.float64)
    z = scale * (K @ np.asarray(q_vec, dtype=np.float64))
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ V


def merge_partials(parts):
    """Log-sum-exp merge of per-block partials into (out, lse).

    M = max m_s; L = sum l_s e^(m_s - M); out = sum acc_s e^(m_s - M) / L;
    lse = M + log L.  Equal to one softmax over the union of the blocks.
    """
    M = max(m for m, _, _ in parts)
    L = sum(l * math.exp(m - M) for m, l, _ in parts)
    acc = sum(a * math.exp(m - M) for m, _, a in parts)
    return acc / L, M + math.log(L)


# ----------------------------------------------------------------------------
# whole rows / whole problems
# ----------------------------------------------------------------------------
def default_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)   # R8


class Problem:
    """Host copies of one problem's inputs (any float dtype; bf16 values are
    held as float32 or float64 numpy, which represent them exactly)."""

    def __init__(self, q, k, v, q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, top_k,
                 scale=None, block=BLOCK):
        self.q, self.k, self.v = q, k, v
        self.q_idx, self.k_idx = q_idx, k_idx
        self.cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
        self.cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
        self.top_k = int(top_k)
        self.block = int(block)
        self.Hq, self.d = q.shape[1], q.shape[2]
        self.G = k.shape[1]
        self.scale = default_scale(self.d) if scale is None else float(scale)
        self.seq, self.pos, self.koff = query_positions(self.cu_q, self.cu_k)

    @property
    def batch(self):
        return len(self.cu_q) - 1

    @property
    def total_q(self):
        return int(self.cu_q[-1])

    @property
    def nb_max(self):
        lk = np.diff(self.cu_k)
        return int((lk.max() + self.block - 1) // self.block) if len(lk) else 0

    def row(self, r, want_scores=False):
        """Index Branch + Main Branch for global query row r.

        Returns dict(sel [G, top_k] int (ascending, -1 padded),
        sel_score [G, top_k] (block score, +inf for the local block, nan pad),
        out [Hq, d], lse [Hq]) and, if asked, S [G, beta(p)+1].
        """
        b, p, ko = int(self.seq[r]), int(self.pos[r]), int(self.koff[r])
        lk = int(self.cu_k[b + 1] - self.cu_k[b])
        kseq = self.k_idx[ko:ko + lk]
        s = index_token_scores(self.q_idx[r], kseq, p)
        S = block_max_pool(s, p, self.block)
        beta_p = p // self.block
        sel = np.full((self.G, self.top_k), -1, dtype=np.int64)
        sel_score = np.full((self.G, self.top_k), np.nan, dtype=np.float64)
        groups = []
        for g in range(self.G):
            chosen = select_blocks(S[g], beta_p, self.top_k)
            groups.append(chosen)
            sel[g, :len(chosen)] = chosen
            for i, beta in enumerate(chosen):
                sel_score[g, i] = math.inf if beta == beta_p else S[g, beta]
        out, lse = attend_row(self.q[r], self.k[ko:ko + lk], self.v[ko:ko + lk], p, groups,
                              self.scale, self.block)
        res = dict(sel=sel, sel_score=sel_score, out=out, lse=lse)
        if want_scores:
            res["S"] = S
        return res

    def attend_with_selection(self, r, sel_row):
        """Main Branch for row r on a given selection sel_row [G, top_k] (-1 padded)."""
        b, p, ko = int(self.seq[r]), int(self.pos[r]), int(self.koff[r])
        lk = int(self.cu_k[b + 1] - self.cu_k[b])
        groups = [[int(x) for x in sel_row[g] if x >= 0] for g in range(self.G)]
        return attend_row(self.q[r], self.k[ko:ko + lk], self.v[ko:ko + lk], p, groups,
                          self.scale, self.block)

    def run(self, rows=None, want_scores=False):
        """Row results for `rows` (default: every row) stacked into arrays."""
        rows = range(self.total_q) if rows is None else rows
        res = [self.row(int(r), want_scores) for r in rows]
        out = dict(
            sel=np.stack([x["sel"] for x in res]) if res else np.zeros((0, self.G, self.top_k), np.int64),
            sel_score=np.stack([x["sel_score"] for x in res]) if res else np.zeros((0, self.G, self.top_k)),
            out=np.stack([x["out"] for x in res]) if res else np.zeros((0, self.Hq, self.d)),
            lse=np.stack([x["lse"] for x in res]) if res else np.zeros((0, self.Hq)),
        )
        if want_scores:
            out["S"] = [x["S"] for x in res]
        return out


# ----------------------------------------------------------------------------
# inverse map: per (sequence, group, block) query lists  [TNK/impl]
# ----------------------------------------------------------------------------
def build_block_query_lists(sel, seq_of_row, batch, G, nb_max):
    """Invert per-row selections into per-KV-block query lists.

    For every bucket u = (b * G + g) * nb_max + beta the entries
    row * 32 + slot with sel[row, g, slot] == beta and row in sequence b,
    in ascending row order ([TNK/impl]: the KV block is the outer loop and
    gathers the queries that hit it).  Returns (offsets [U + 1], entries).
    Uses a stable library sort by bucket over the row-major selection.
    """
    sel = np.asarray(sel, dtype=np.int64)
    T, Gs, k = sel.shape
    assert Gs == G and k <= (1 << ENTRY_SLOT_BITS)
    rows = np.repeat(np.arange(T, dtype=np.int64), G * k)
    gs = np.tile(np.repeat(np.arange(G, dtype=np.int64), k), T)
    slots = np.tile(np.arange(k, dtype=np.int64), T * G)
    beta = sel.reshape(-1)
    keep = beta >= 0
    rows, gs, slots, beta = rows[keep], gs[keep], slots[keep], beta[keep]
    bucket = (np.asarray(seq_of_row, dtype=np.int64)[rows] * G + gs) * nb_max + beta
    order = np.argsort(bucket, kind="stable")
    U = batch * G * nb_max
    counts = np.bincount(bucket, minlength=U)
    offsets = np.zeros(U + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    entries = (rows * (1 << ENTRY_SLOT_BITS) + slots)[order]
    return offsets, entries


# ----------------------------------------------------------------------------
# near-tie classification (for comparing a float32 selection to this one)
# ----------------------------------------------------------------------------
def _tie_tolerance(S_g, beta_p, top_k, rel):
    """(S_(k-1), S_(k), rel * max(|S_(k-1)|, |S_(k)|, 1e-30)) over the
    non-local blocks 0 .. beta_p - 1, sorted by score descending (1-based
    order statistics).  Only defined when more than k-1 such blocks exist."""
    v = np.sort(np.asarray(S_g[:beta_p], dtype=np.float64))[::-1]
    a, b = float(v[top_k - 2]), float(v[top_k - 1])
    return a, b, rel * max(abs(a), abs(b), 1e-30)


def near_tie(S_g, beta_p, top_k, rel=1e-4):
    """True when the (k-1)-th and k-th best non-local block scores are within
    `rel` (relative): then more than one selection is correct.

    Rows with at most k-1 non-local blocks take every block, and k = 1 takes
    only the local block: neither has a choice to tie over.
    """
    if beta_p <= top_k - 1 or top_k < 2:
        return False
    a, b, tol = _tie_tolerance(S_g, beta_p, top_k, rel)
    return (a - b) <= tol


def valid_selection(S_g, beta_p, top_k, chosen, rel=1e-4):
    """Whether `chosen` (block ids, -1 padding ignored) is a correct selection
    of one (query, group) up to the near-tie tolerance.

    It must hold the local block beta_p, min(top_k, beta_p + 1) distinct ids,
    none after beta_p, and no unchosen earlier block may score more than
    tol = rel * max(|S_(k-1)|, |S_(k)|) above a chosen earlier block.  Away
    from a near-tie only the exact top-(k-1) passes; on a near-tie the blocks
    inside the tie band may be exchanged, and nothing else.
    """
    chosen = [int(x) for x in chosen if x >= 0]
    if beta_p not in chosen or len(chosen) != min(top_k, beta_p + 1):
        return False
    if len(set(chosen)) != len(chosen) or max(chosen) > beta_p:
        return False
    if beta_p <= top_k - 1:
        return True
    _, _, tol = _tie_tolerance(S_g, beta_p, top_k, rel)
    mine = [c for c in chosen if c != beta_p]
    rest = [u for u in range(beta_p) if u not in set(mine)]
    if not mine or not rest:
        return True
    return max(float(S_g[u]) for u in rest) - min(float(S_g[c]) for c in mine) <= tol
