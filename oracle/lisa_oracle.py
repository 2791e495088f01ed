"""Plain float64 CPU oracle for one LISA attention layer.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and the library never calls it.

Source: "LISA: Linear-Indexed Sparse Attention for Efficient Long-Context
Reasoning" (arXiv 2607.19358v1), cited below as [LISA] with its section or
equation.

Everything is computed in float64 from the exact values of the inputs
(bf16 or fp32 storage values upcast without rounding).  The code follows the
plain definitions one row at a time; numpy matrix products serve as single
steps.  Conventions fixed where the paper is silent are listed next to the
function that uses them:

* Indexer score of key j for query t: sum over index heads h of
  ``w_h * ReLU(q_I[t,h] . k_I[j, h*H_Ik//H_I])`` ([LISA] §3.2 Stage 2, the
  ReLU dot-product score under Eq. 2, summed over the K indexer heads).
* Candidate keys of query t are positions 0..t (the current token included).
* Top-M keeps the min(M, t+1) largest scores; equal scores are ordered by
  position, the larger position first; -0.0 equals +0.0.  The index set is
  returned in ascending order.
* Sparse attention is softmax attention with scale 1/sqrt(d) over the
  selected keys, query head h reading KV head h*H_kv//H_q ([LISA] §3.1
  Softmax Attention; §3.2 Stage 2).
* Linear branch: feature map phi(x) = elu(x)+1, state
  ``S_t = S_0 + sum_{i<=t} phi(k_i)^T v_i``, normaliser
  ``z_t = z_0 + sum_{i<=t} phi(k_i)``, output
  ``phi(q_t) S_t / (phi(q_t) . z_t)`` ([LISA] §3.1 Linear Attention; §3.3
  Eqs. 3-4, read as inclusive of the current token).  With
  ``normalized=False`` the output is ``phi(q_t) S_t`` (Eq. 4 literally).
* Sliding-window mode ([LISA] §3.2 Stage 1, Eq. 1: a fixed budget of the M
  most recent tokens): query t attends to positions max(0, t+1-M)..t and no
  indexer runs.  With every indexer score equal this is exactly what top-M
  selects (ties go to the larger position).
* Gate ``g = sigmoid(x . W_g[:, h])``, one scalar per token and query head,
  and ``out = g * O_sparse + (1-g) * O_linear`` ([LISA] §3.2 Eq. 1 and §3.3
  Eq. 5; the gate weights the sparse branch here, which is Eq. 1 with W_g
  negated).
* Attention coverage ([LISA] §4, "Optimal Window Size M and Attention
  Coverage", Eq. 10): the share of a query head's dense causal softmax
  weight that falls on a selected set; its upper bound is the share of that
  head's own M largest weights.
* Indexer training objective ([LISA] §3.2 Stage 2, Eq. 2): per indexer head
  j and row t, KL(T || softmax(S)) over the causal keys, where S is head j's
  unweighted ReLU score row and T the mean of the causal attention rows of
  the teacher heads j*H_q/H_I .. (j+1)*H_q/H_I - 1 (the layer's own query
  heads; a sum of distributions renormalised is their mean).  Candidate
  dropout ([LISA] §3.2 Stage 2): the top C candidates (1.2 M in the paper),
  each dropped when its caller-drawn uniform is below p, and the M best of
  the survivors kept.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

__all__ = [
    "phi", "index_scores", "select_topm", "sparse_attention", "gate",
    "linear_recurrent", "linear_rows", "linear_chunked", "linear_state_update",
    "prefill", "prefill_rows", "decode_step", "dense_decode", "window_positions",
    "segment_correct", "attention_mass", "indexer_kl", "candidate_dropout",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------
def phi(x) -> np.ndarray:
    """elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise."""
    x = _f64(x)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def gate(x, w_gate) -> np.ndarray:
    """g[..., h] = 1 / (1 + exp(-(x . W_g[:, h]))).  [LISA] §3.3 Eq. 5.

    x: [..., hidden]; w_gate: [hidden, H_q].
    """
    a = _f64(x) @ _f64(w_gate)
    return 1.0 / (1.0 + np.exp(-a))


# ----------------------------------------------------------------------------
# indexer and selection ([LISA] §3.2 Stage 2)
# ----------------------------------------------------------------------------
def index_scores(q_idx, k_idx, w_idx) -> np.ndarray:
    """Scores of every key for one query.

    q_idx: [H_I, d_I]; k_idx: [L, H_Ik, d_I]; w_idx: [H_I].
    Returns s[j] = sum_h w_h * max(0, q_idx[h] . k_idx[j, h*H_Ik//H_I]).
    """
    q = _f64(q_idx)
    k = _f64(k_idx)
    w = _f64(w_idx)
    H_I = q.shape[0]
    H_Ik = k.shape[1]
    s = np.zeros(k.shape[0], dtype=np.float64)
    for h in range(H_I):
        dots = k[:, (h * H_Ik) // H_I, :] @ q[h]
        s += w[h] * np.maximum(dots, 0.0)
    return s


def select_topm(scores, M: int) -> np.ndarray:
    """Ascending positions of the min(M, L) largest scores.

    Order: score descending, then position descending (a tie goes to the
    later token).  Comparison is numeric, so -0.0 and +0.0 tie.
    """
    s = np.asarray(scores)
    L = s.shape[0]
    m = min(int(M), L)
    if m <= 0:
        return np.zeros((0,), dtype=np.int64)
    pos = np.arange(L, dtype=np.int64)
    # np.lexsort: the last key is the primary key, each sorted ascending.
    order = np.lexsort((-pos, -s.astype(np.float64)))
    return np.sort(order[:m])


# ----------------------------------------------------------------------------
# sparse softmax attention ([LISA] §3.1 Softmax Attention, §3.2 SA_M)
# ----------------------------------------------------------------------------
def sparse_attention(q, K, V, P) -> np.ndarray:
    """Softmax attention of one token's query heads over the keys in P.

    q: [H_q, d]; K, V: [L, H_kv, d]; P: positions (any order, no repeats).
    Query head h reads KV head h*H_kv//H_q; scale 1/sqrt(d).
    """
    q = _f64(q)
    H_q, d = q.shape
    H_kv = K.shape[1]
    P = np.asarray(P, dtype=np.int64)
    out = np.zeros((H_q, d), dtype=np.float64)
    if P.size == 0:
        return out
    for g in range(H_kv):
        heads = [h for h in range(H_q) if (h * H_kv) // H_q == g]
        Kg = _f64(K[P, g, :])            # [m, d]
        Vg = _f64(V[P, g, :])
        a = q[heads] @ Kg.T / np.sqrt(d)   # [heads, m]
        a -= a.max(axis=1, keepdims=True)
        p = np.exp(a)
        p /= p.sum(axis=1, keepdims=True)
        out[heads] = p @ Vg
    return out


# ----------------------------------------------------------------------------
# linear-attention branch ([LISA] §3.1 Linear Attention, §3.3 Eqs. 3-4)
# ----------------------------------------------------------------------------
def _linear_out(fq, S, z, normalized: bool) -> np.ndarray:
    num = np.einsum("hd,hde->he", fq, S)
    if not normalized:
        return num
    den = np.einsum("hd,hd->h", fq, z)
    return num / den[:, None]


def linear_recurrent(q_lin, k_lin, v_lin, S0, z0, normalized: bool = True):
    """Token-by-token recurrence: update with token t, then read with q_t.

    q_lin, k_lin, v_lin: [n, H, d]; S0: [H, d, d] (rows index phi(k),
    columns index v); z0: [H, d].  Returns (O [n, H, d], S_n, z_n).
    """
    S = _f64(S0).copy()
    z = _f64(z0).copy()
    n, H, d = np.shape(q_lin)
    out = np.zeros((n, H, d), dtype=np.float64)
    for t in range(n):
        fk = phi(k_lin[t])
        v = _f64(v_lin[t])
        S += fk[:, :, None] * v[:, None, :]
        z += fk
        out[t] = _linear_out(phi(q_lin[t]), S, z, normalized)
    return out, S, z


def linear_rows(q_lin, k_lin, v_lin, S0, z0, rows: Iterable[int],
                normalized: bool = True):
    """Outputs of selected rows from the closed form of Eq. 3.

    ``S_t = S_0 + phi(K[:t+1])^T V[:t+1]``, accumulated over the gaps
    between consecutive requested rows.  Returns (dict row -> [H, d],
    S_n, z_n) where S_n, z_n cover all n tokens.
    """
    rows = sorted(set(int(r) for r in rows))
    n = np.shape(k_lin)[0]
    S = _f64(S0).copy()
    z = _f64(z0).copy()
    done = 0
    res: Dict[int, np.ndarray] = {}

    def absorb(lo, hi):
        if hi <= lo:
            return
        fk = phi(k_lin[lo:hi])            # [m, H, d]
        v = _f64(v_lin[lo:hi])
        S[...] += np.einsum("mhd,mhe->hde", fk, v, optimize=True)
        z[...] += fk.sum(axis=0)

    for t in rows:
        absorb(done, t + 1)
        done = t + 1
        res[t] = _linear_out(phi(q_lin[t]), S, z, normalized)
    absorb(done, n)
    return res, S, z


def linear_chunked(q_lin, k_lin, v_lin, S0, z0, chunk: int = 64,
                   normalized: bool = True):
    """Chunked-parallel form of the same recurrence (self-check only).

    Per chunk: A = (phi(Q_c) phi(K_c)^T) masked to j <= i (diagonal kept);
    numerator A V_c + phi(Q_c) S, denominator A 1 + phi(Q_c) z; then the
    chunk's phi(K_c)^T V_c and phi(K_c)^T 1 are added to S and z.
    """
    S = _f64(S0).copy()
    z = _f64(z0).copy()
    n, H, d = np.shape(q_lin)
    out = np.zeros((n, H, d), dtype=np.float64)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        fq = phi(q_lin[c0:c1]).transpose(1, 0, 2)   # [H, c, d]
        fk = phi(k_lin[c0:c1]).transpose(1, 0, 2)
        v = _f64(v_lin[c0:c1]).transpose(1, 0, 2)
        A = fq @ fk.transpose(0, 2, 1)               # [H, c, c]
        A = np.tril(A)
        num = A @ v + fq @ S
        if normalized:
            den = A.sum(axis=2) + np.einsum("hcd,hd->hc", fq, z)
            o = num / den[:, :, None]
        else:
            o = num
        out[c0:c1] = o.transpose(1, 0, 2)
        S += fk.transpose(0, 2, 1) @ v
        z += fk.sum(axis=1)
    return out, S, z


def linear_state_update(k_lin, v_lin, S0, z0):
    """S += sum_t phi(k_t)^T v_t, z += sum_t phi(k_t).  k_lin, v_lin: [n, H, d]."""
    fk = phi(k_lin)
    v = _f64(v_lin)
    S = _f64(S0) + np.einsum("nhd,nhe->hde", fk, v, optimize=True)
    z = _f64(z0) + fk.sum(axis=0)
    return S, z


def segment_correct(S, z, S_start, z_start, mean_S, mean_z, t: int, alpha: float):
    """Segment state correction at the end of the t-th segment (t >= 1)
    ([LISA] §3.3 "Segment State Update", Eqs. 6-9).

    * Eq. 6: the segment's direction is the state change over it,
      ``grad = S - S_start`` (S: the state reached at the segment's end).
    * Eq. 7: the global direction is the plain mean of the raw directions
      of the segments before it (``mean_S`` holds that mean over segments
      1..t-1; zero for t = 1).
    * Eq. 8: ``corrected = (1 - alpha) grad + alpha mean``.
    * Eq. 9: the state becomes ``S_start + corrected``.

    Readings: the mean averages the raw directions of Eq. 6 (Eq. 7 as
    printed), and the normaliser z is corrected exactly like S, the pair
    (S, z) being the state that the branch carries.
    Returns (S_new, z_new, mean_S_new, mean_z_new): the corrected state, and
    the mean over segments 1..t; the corrected state is also where the next
    segment starts.
    """
    out = []
    for cur, start, mean in ((S, S_start, mean_S), (z, z_start, mean_z)):
        grad = _f64(cur) - _f64(start)
        prev = _f64(mean) if t > 1 else np.zeros_like(grad)
        corrected = (1.0 - alpha) * grad + alpha * prev
        out.append((_f64(start) + corrected, prev + (grad - prev) / t))
    (S_new, mS), (z_new, mz) = out
    return S_new, z_new, mS, mz


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------
def window_positions(t: int, M: int) -> np.ndarray:
    """The sliding window of query t: the min(M, t+1) positions ending at t,
    ascending ([LISA] §3.2 Stage 1, the fixed-budget window of Eq. 1)."""
    return np.arange(max(0, t + 1 - M), t + 1, dtype=np.int64)


def _row_select(q_idx_t, k_idx, w_idx, t: int, M: int, scores_dtype=None):
    s = index_scores(q_idx_t, k_idx[: t + 1], w_idx)
    if scores_dtype is not None:
        s = s.astype(scores_dtype)
    return select_topm(s, M), s


def prefill_rows(inp: Dict[str, np.ndarray], M: int, rows: Sequence[int],
                 b: int = 0, normalized: bool = True,
                 select_on=None, window: bool = False) -> Dict[str, object]:
    """Outputs of chosen query rows of a causal prefill of sequence ``b``.

    ``inp`` holds the arrays of a prefill input set (shapes [B, n, ...]).
    ``select_on``: None selects on float64 scores; np.float32 selects on the
    scores rounded to float32 (as a GPU select kernel sees them).
    Returns dict with 'out' {row: [H_q, d]}, 'idx' {row: positions},
    'scores' {row: float64 scores}, 'S', 'z' (state after all n tokens).
    """
    q, K, V = inp["q"][b], inp["k"][b], inp["v"][b]
    q_idx, k_idx, w_idx = inp["q_idx"][b], inp["k_idx"][b], inp["w_idx"]
    rows = sorted(set(int(r) for r in rows))
    lin, S, z = linear_rows(inp["q_lin"][b], inp["k_lin"][b], inp["v_lin"][b],
                            inp["S0"][b], inp["z0"][b], rows, normalized)
    g = gate(inp["x"][b][rows], inp["w_gate"])      # [r, H_q]
    out, idx, sc = {}, {}, {}
    for i, t in enumerate(rows):
        if window:
            P, s = window_positions(t, M), None
        else:
            P, s = _row_select(q_idx[t], k_idx, w_idx, t, M, select_on)
        o_s = sparse_attention(q[t], K, V, P)
        o_l = lin[t]
        out[t] = g[i][:, None] * o_s + (1.0 - g[i][:, None]) * o_l
        idx[t] = P
        sc[t] = s
    return {"out": out, "idx": idx, "scores": sc, "S": S, "z": z}


def prefill(inp: Dict[str, np.ndarray], M: int, normalized: bool = True,
            select_on=None, window: bool = False) -> Dict[str, object]:
    """Full causal prefill of every sequence (small sizes).

    Returns 'out' [B, n, H_q, d], 'idx' list (per b) of lists of arrays,
    'S' [B, H, d, d], 'z' [B, H, d], plus 'o_sparse', 'o_linear', 'g'.
    """
    B, n = inp["q"].shape[:2]
    H_q, d = inp["q"].shape[2:]
    out = np.zeros((B, n, H_q, d))
    o_sp = np.zeros((B, n, H_q, d))
    o_li = np.zeros((B, n, H_q, d))
    gs = np.zeros((B, n, H_q))
    S_all, z_all, idx_all = [], [], []
    for b in range(B):
        o_l, S, z = linear_recurrent(inp["q_lin"][b], inp["k_lin"][b], inp["v_lin"][b],
                                     inp["S0"][b], inp["z0"][b], normalized)
        g = gate(inp["x"][b], inp["w_gate"])
        idx_b = []
        for t in range(n):
            if window:
                P = window_positions(t, M)
            else:
                P, _ = _row_select(inp["q_idx"][b][t], inp["k_idx"][b], inp["w_idx"], t, M,
                                   select_on)
            o_s = sparse_attention(inp["q"][b][t], inp["k"][b], inp["v"][b], P)
            o_sp[b, t] = o_s
            idx_b.append(P)
        o_li[b] = o_l
        gs[b] = g
        out[b] = g[:, :, None] * o_sp[b] + (1.0 - g[:, :, None]) * o_l
        S_all.append(S)
        z_all.append(z)
        idx_all.append(idx_b)
    return {"out": out, "idx": idx_all, "S": np.stack(S_all), "z": np.stack(z_all),
            "o_sparse": o_sp, "o_linear": o_li, "g": gs}


def decode_step(inp: Dict[str, np.ndarray], M: int, normalized: bool = True,
                select_on=None, batch: Optional[Iterable[int]] = None,
                window: bool = False) -> Dict[str, object]:
    """One decode step for every sequence (or those in ``batch``).

    The caches hold rows 0..L_b-2; the new token's k, v, k_I become row
    L_b-1 ([LISA] §3.2 Stage 2: the KV cache covers the full context).
    The indexer then scores rows 0..L_b-1, the top-M rows feed the sparse
    attention, the linear state absorbs the new token before it is read,
    and the gate mixes the two branches.
    Returns 'out' [B', H_q, d], 'idx' list, 'scores' list, 'S', 'z'.
    """
    seq_lens = np.asarray(inp["seq_lens"])
    bs = list(range(len(seq_lens))) if batch is None else list(batch)
    outs, idxs, scs, Ss, zs, osp, oli, gg = [], [], [], [], [], [], [], []
    for b in bs:
        L = int(seq_lens[b])
        k_idx = np.array(inp["k_idx_cache"][b, :L], dtype=np.float64)
        k_idx[L - 1] = inp["k_idx_new"][b]
        K = np.array(inp["k_cache"][b, :L], dtype=np.float64)
        V = np.array(inp["v_cache"][b, :L], dtype=np.float64)
        K[L - 1] = inp["k_new"][b]
        V[L - 1] = inp["v_new"][b]
        if window:  # the new token's window: rows L-m .. L-1, no indexer
            s = None
            P = window_positions(L - 1, M)
        else:
            s = index_scores(inp["q_idx"][b], k_idx, inp["w_idx"])
            P = select_topm(s if select_on is None else s.astype(select_on), M)
        o_s = sparse_attention(inp["q"][b], K, V, P)
        fk = phi(inp["k_lin"][b])
        S = _f64(inp["S0"][b]) + fk[:, :, None] * _f64(inp["v_lin"][b])[:, None, :]
        z = _f64(inp["z0"][b]) + fk
        o_l = _linear_out(phi(inp["q_lin"][b]), S, z, normalized)
        g = gate(inp["x"][b], inp["w_gate"])          # [H_q]
        outs.append(g[:, None] * o_s + (1.0 - g[:, None]) * o_l)
        idxs.append(P)
        scs.append(s)
        Ss.append(S)
        zs.append(z)
        osp.append(o_s)
        oli.append(o_l)
        gg.append(g)
    return {"out": np.stack(outs), "idx": idxs, "scores": scs, "S": np.stack(Ss),
            "z": np.stack(zs), "o_sparse": np.stack(osp), "o_linear": np.stack(oli),
            "g": np.stack(gg)}


def dense_decode(inp: Dict[str, np.ndarray], batch: Optional[Iterable[int]] = None) -> np.ndarray:
    """Full causal softmax attention of the new token over rows 0..L_b-1.

    Caches as in ``decode_step`` (the new k, v appended at row L_b-1).
    Returns [B', H_q, d].
    """
    seq_lens = np.asarray(inp["seq_lens"])
    bs = list(range(len(seq_lens))) if batch is None else list(batch)
    outs = []
    for b in bs:
        L = int(seq_lens[b])
        K = np.array(inp["k_cache"][b, :L], dtype=np.float64)
        V = np.array(inp["v_cache"][b, :L], dtype=np.float64)
        K[L - 1] = inp["k_new"][b]
        V[L - 1] = inp["v_new"][b]
        outs.append(sparse_attention(inp["q"][b], K, V, np.arange(L)))
    return np.stack(outs)


# ----------------------------------------------------------------------------
# attention coverage ([LISA] §4, Eq. 10)
# ----------------------------------------------------------------------------
def attention_mass(q, K, P, M: int):
    """Coverage of one query row by a selected set, per query head.

    q: [H_q, d]; K: [L, H_kv, d], the keys of positions 0..L-1 (every key at
    or before the query); P: selected positions (distinct, any order).  For
    query head h reading KV head g = h*H_kv//H_q, the dense weights are
    a_j = exp(q_h . K[j, g] / sqrt(d)) over all L keys, and
      mass[h]  = sum_{j in P} a_j / sum_j a_j                    (Eq. 10)
      bound[h] = (sum of the M largest a_j) / sum_j a_j
    The bound is the coverage of the head's own best M-set, which no set of
    M positions shared by the heads can exceed (the paper's upper bound of
    the indexer's mass, read here per head).  Returns (mass, bound), [H_q].
    """
    q = _f64(q)
    H_q, d = q.shape
    H_kv = K.shape[1]
    P = np.asarray(P, dtype=np.int64)
    mass = np.zeros(H_q)
    bound = np.zeros(H_q)
    for h in range(H_q):
        g = (h * H_kv) // H_q
        a = _f64(K[:, g, :]) @ q[h] / np.sqrt(d)   # logits of every key
        w = np.exp(a - a.max())                    # the common factor cancels
        total = w.sum()
        mass[h] = w[P].sum() / total
        bound[h] = np.sort(w)[::-1][: int(M)].sum() / total
    return mass, bound


# ----------------------------------------------------------------------------
# indexer training ([LISA] §3.2 Stage 2, Eq. 2 and the candidate dropout)
# ----------------------------------------------------------------------------
def _log_softmax(x) -> np.ndarray:
    x = _f64(x)
    m = x.max()
    return x - (m + np.log(np.exp(x - m).sum()))


def indexer_kl(q, K, q_idx, k_idx, rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Per-row, per-indexer-head KL of Eq. 2 for one sequence.

    q: [n, H_q, d]; K: [n, H_kv, d] (the teacher's queries and keys);
    q_idx: [n, H_I, d_I]; k_idx: [n, H_Ik, d_I].  For row t and indexer head
    j, over the keys 0..t:
      S_k      = max(0, q_idx[t, j] . k_idx[k, j*H_Ik//H_I])    (no head weight)
      log Q    = log softmax(S)
      A_h      = softmax(q[t, h] . K[:, h*H_kv//H_q] / sqrt(d)) for the G_T =
                 H_q/H_I teacher heads h = j*G_T .. (j+1)*G_T - 1
      T        = (sum_h A_h) / G_T                   (the renormalised sum)
      KL[t, j] = sum_k T_k (log T_k - log Q_k), with 0 log 0 = 0.
    Returns [len(rows), H_I].  The loss of Eq. 2 is the mean over rows and
    heads.
    """
    q = _f64(q)
    n, H_q, d = q.shape
    H_kv = K.shape[1]
    H_I = q_idx.shape[1]
    H_Ik = k_idx.shape[1]
    assert H_q % H_I == 0, "teacher heads split evenly over the indexer heads"
    G_T = H_q // H_I
    rows = list(range(n)) if rows is None else list(rows)
    out = np.zeros((len(rows), H_I))
    for i, t in enumerate(rows):
        for j in range(H_I):
            S = np.maximum(0.0, _f64(k_idx[: t + 1, (j * H_Ik) // H_I]) @ _f64(q_idx[t, j]))
            logQ = _log_softmax(S)
            T = np.zeros(t + 1)
            for h in range(j * G_T, (j + 1) * G_T):
                a = _f64(K[: t + 1, (h * H_kv) // H_q]) @ q[t, h] / np.sqrt(d)
                T += np.exp(_log_softmax(a))
            T /= G_T
            pos = T > 0
            out[i, j] = float(np.sum(T[pos] * (np.log(T[pos]) - logQ[pos])))
    return out


def candidate_dropout(scores, M: int, n_cand: int, p, u) -> np.ndarray:
    """Indexer candidates with dropout, ascending positions.

    The top C = min(L, n_cand) positions by (score desc, position desc) are
    the candidates (the paper takes n_cand = 1.2 M early in training);
    candidate j is dropped when u[j] < p (u holds the caller's uniform draws
    in [0, 1), one per position; p is the dropout ratio, annealed by the
    caller); of the survivors the min(M, #survivors) best in the same order
    are kept.
    """
    s = np.asarray(scores)
    u = np.asarray(u)
    C = min(s.shape[0], int(n_cand))
    cand = select_topm(s, C)
    surv = np.array([j for j in cand if u[j] >= p], dtype=np.int64)
    if surv.size <= M:
        return surv
    keep = select_topm(s[surv], M)   # indices into surv, in survivor order
    return np.sort(surv[keep])
