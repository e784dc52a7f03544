"""Oracle: float64 attention of absorbed-MLA decode, per stripe, and the LSE merge.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed (no blocking, fusion or online rescaling is added):

* Absorbed MLA decode is multi-query attention with one shared 576-dim latent
  row per token: the key is the whole row [c^K (512) || k^R (64)], the value
  is its first 512 dims, and each query head brings its own 576-dim row
  [q^C_hat (512) || q^R (64)] (page "MLA 的 Decode Context Parallelism",
  sections 1 and 2: the two absorption identities).
* Scores s_p = scale * q . k_p; output o = sum_p exp(s_p) v_p / sum_p exp(s_p)
  over the visible positions, evaluated with the maximum subtracted;
  lse = log sum_p exp(s_p) (page "DCP", section "theory", merge identity and
  numerical stability).
* A query at global position t sees positions p <= t (causal mask; page "DCP",
  mergeability table: a mask only shrinks the visible set).  The q_len queries
  of a request sit at S-q_len, ..., S-1 (SGLang DCP docs, "DCP x speculative
  decoding": global lengths keep causality over the whole sequence).
* A stripe's local result is the same definition restricted to the positions
  the rank owns: o_r is normalised inside the stripe, lse_r its log-sum-exp;
  an empty visible set gives o_r = 0 and lse_r = -inf, i.e. zero weight
  (page "DCP", idea two; page "PCP/DCP" section 4.1: an empty shard must act
  as a zero-weight normalisation state).
* Merge: m = max_r lse_r, w_r = exp(lse_r - m), o = sum w_r o_r / sum w_r,
  lse = m + log sum w_r; with base-2 LSE the pair is 2^x / log2 (page "DCP",
  "merge operator and numerical stability"; SGLang DCP docs, "MLA decode
  dataflow").

"Base-2 LSE" is read as log2 of the same natural-softmax partition function
(lse_2 = lse_e * log2(e)); the attention output does not depend on the base.

Variants that keep the merge exact (page "DCP", "conditions for merging and
where they fail": a mask only shrinks the visible set, a sink or position bias
is one extra logit term in one shard, an elementwise logit transform couples
no positions):

* sliding window W: a query at t sees p with t - W < p <= t;
* logit softcap c: each scaled score s becomes c * tanh(s / c);
* attention sink: one extra logit sigma per query row with value zero, i.e.
  exp(sigma) joins the denominator; in a sharded run exactly one shard adds it.
* position bias (linear in the distance, ALiBi style): the logit of position p
  for a query at t gains slope * (p - t), after the softcap; it depends only
  on the pair's own positions, so each shard adds it for its own positions.
"""

from __future__ import annotations

import math

import numpy as np

LN2 = math.log(2.0)


def attention_rows(q: np.ndarray, q_pos: np.ndarray, kv: np.ndarray, kv_pos: np.ndarray,
                   scale: float, v_dim: int = 512, chunk: int | None = None,
                   window: int = 0, softcap: float = 0.0, sink=None, slope=None):
    """Softmax attention of R query rows over n latent rows, in float64.

    q      [R, D] query rows (D = 576)
    q_pos  [R]    global position of each query (it sees kv rows with kv_pos <= q_pos)
    kv     [n, D] latent rows; the key is the whole row, the value its first v_dim dims
    kv_pos [n]    global position of each latent row
    window > 0    also hides rows with kv_pos <= q_pos - window
    softcap > 0   replaces each scaled score s by softcap * tanh(s / softcap)
    sink   [R]    natural-log logit of an extra zero-valued term per row (None: none)
    slope  [R]    position bias slope per row: logit += slope * (kv_pos - q_pos) (None: none)
    Returns o [R, v_dim] and the natural-log lse [R]; a query that sees no row
    (and has no sink) gets o = 0 and lse = -inf.

    ``chunk`` only splits the two sums over rows into pieces (a first pass
    finds the exact maximum, a second adds up exp(s - max) and the weighted
    values); it does not change the formula.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    R = q.shape[0]
    n = kv.shape[0]
    if chunk is None or chunk <= 0:
        chunk = max(n, 1)

    def scores(lo, hi):
        s = (kv[lo:hi] @ q.T) * scale                       # [rows, R]
        if softcap > 0:
            s = softcap * np.tanh(s / softcap)
        if slope is not None:
            s = s + np.asarray(slope, dtype=np.float64)[None, :] * (kv_pos[lo:hi, None] - q_pos[None, :])
        hidden = kv_pos[lo:hi, None] > q_pos[None, :]
        if window > 0:
            hidden |= kv_pos[lo:hi, None] <= q_pos[None, :] - window
        s[hidden] = -np.inf
        return s

    m = np.full(R, -np.inf)
    for lo in range(0, n, chunk):
        s = scores(lo, min(n, lo + chunk))
        if s.size:
            m = np.maximum(m, s.max(axis=0))
    if sink is not None:
        sink = np.asarray(sink, dtype=np.float64).reshape(R)
        m = np.maximum(m, sink)
    seen = np.isfinite(m)
    m_safe = np.where(seen, m, 0.0)
    Z = np.zeros(R)
    acc = np.zeros((R, v_dim))
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        s = scores(lo, hi)
        e = np.exp(s - m_safe[None, :])                      # exp(-inf) = 0 for hidden rows
        Z += e.sum(axis=0)
        acc += e.T @ kv[lo:hi, :v_dim]
    if sink is not None:
        Z += np.exp(sink - m_safe)                           # exp(-inf) = 0: no sink on that row
    o = np.zeros((R, v_dim))
    o[seen] = acc[seen] / Z[seen, None]
    lse = np.full(R, -np.inf)
    lse[seen] = m[seen] + np.log(Z[seen])
    return o, lse


def query_positions(S: int, q_len: int) -> np.ndarray:
    """Global positions of the q_len queries of a request with S cached tokens."""
    return np.arange(S - q_len, S, dtype=np.int64)


def _row_sinks(sinks, q_len: int, H: int):
    """Per-head values [H] (sink logits, bias slopes) as one value per query row (t, h), or None."""
    if sinks is None:
        return None
    return np.tile(np.asarray(sinks, dtype=np.float64).reshape(H), q_len)


def full_attention(q_req: np.ndarray, kv_req: np.ndarray, S: int, scale: float,
                   v_dim: int = 512, chunk: int | None = None,
                   window: int = 0, softcap: float = 0.0, sinks=None, slopes=None):
    """Unsharded attention of one request.

    q_req [q_len, H, D], kv_req [S, D] (logical order, position p at row p).
    window / softcap as in ``attention_rows``; sinks [H] per-head sink logits;
    slopes [H] per-head position-bias slopes.
    Returns o [q_len, H, v_dim] and natural-log lse [q_len, H].
    """
    q_len, H, D = q_req.shape
    qp = np.repeat(query_positions(S, q_len), H)
    o, lse = attention_rows(q_req.reshape(q_len * H, D), qp, kv_req[:S],
                            np.arange(S, dtype=np.int64), scale, v_dim, chunk,
                            window, softcap, _row_sinks(sinks, q_len, H), _row_sinks(slopes, q_len, H))
    return o.reshape(q_len, H, v_dim), lse.reshape(q_len, H)


def stripe_attention(q_req: np.ndarray, kv_req: np.ndarray, S: int, positions: np.ndarray,
                     scale: float, v_dim: int = 512, chunk: int | None = None,
                     window: int = 0, softcap: float = 0.0, sinks=None, slopes=None):
    """Local attention of one request on one stripe.

    ``positions`` are the global positions the rank owns (as handed out by
    ``oracle.layout.stripe_positions``); only those rows of ``kv_req`` enter.
    window / softcap as in ``attention_rows``; ``sinks`` [H] is given to the
    one stripe that carries the sink term.
    Returns the locally normalised o_r [q_len, H, v_dim] and lse_r [q_len, H]
    (natural log; -inf where the stripe holds no visible row and no sink).
    """
    q_len, H, D = q_req.shape
    positions = np.asarray(positions, dtype=np.int64)
    positions = positions[positions < S]
    qp = np.repeat(query_positions(S, q_len), H)
    o, lse = attention_rows(q_req.reshape(q_len * H, D), qp, kv_req[positions],
                            positions, scale, v_dim, chunk,
                            window, softcap, _row_sinks(sinks, q_len, H), _row_sinks(slopes, q_len, H))
    return o.reshape(q_len, H, v_dim), lse.reshape(q_len, H)


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray, base: str = "e"):
    """Exact merge of per-stripe results.

    o_parts [N, ..., V], lse_parts [N, ...] with lse in ``base`` ("e" or "2").
    Stripes with lse = -inf carry zero weight.  If every stripe is empty the
    result is o = 0 and lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if base == "e":
        power = np.exp
        log = np.log
    elif base == "2":
        power = np.exp2
        log = np.log2
    else:
        raise ValueError("base must be 'e' or '2'")
    finite = np.isfinite(lse_parts)
    m = np.where(finite, lse_parts, -np.inf).max(axis=0)
    any_seen = np.isfinite(m)
    m_safe = np.where(any_seen, m, 0.0)
    w = np.where(finite, power(np.where(finite, lse_parts, 0.0) - m_safe[None]), 0.0)
    wsum = w.sum(axis=0)
    o = (w[..., None] * o_parts).sum(axis=0)
    o = np.where(any_seen[..., None], o / np.where(any_seen, wsum, 1.0)[..., None], 0.0)
    lse = np.where(any_seen, m_safe + log(np.where(any_seen, wsum, 1.0)), -np.inf)
    return o, lse


def to_base(lse_e: np.ndarray, base: str) -> np.ndarray:
    """Natural-log LSE expressed in ``base`` ("e" or "2")."""
    lse_e = np.asarray(lse_e, dtype=np.float64)
    if base == "e":
        return lse_e
    if base == "2":
        return lse_e / LN2
    raise ValueError("base must be 'e' or '2'")


# ---- head-return exchange: packed (o bf16, lse fp32) all-to-all payload ------
#
# Page "DCP" (zdszero), "merge: All-to-All": each rank cuts its partial O_r by
# head into N slices and sends slice d, together with the matching LSE, to the
# rank that owns those heads, in one packed buffer; the receiver merges the N
# partials of its H/N heads.  Page "MLA 的 Decode Context Parallelism",
# section 4: the payload is 64 x 96 x (512 + 4) x 2 bytes at B = 64, i.e. a
# record of 516 16-bit slots per (row, head): the output in bf16, then the LSE
# as a float32 in two slots and two slots of padding (8-byte records).

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float32 values, rounded to nearest, ties to even
    (NaN stays a quiet NaN).  Written from the definition: keep the top 16 bits
    of the float32 pattern after adding half an ulp of the kept part, plus one
    more when the kept part is odd."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, ((b >> 16) | 0x40).astype(np.uint16), rounded)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pack_heads(o_r: np.ndarray, lse_r: np.ndarray, N: int) -> np.ndarray:
    """One rank's packed send buffer.

    o_r [rows, H, v] and lse_r [rows, H] (float32 values); H % N == 0.
    Returns uint16 [N, rows, H/N, v + 4]: record (d, row, j) holds head
    d*H/N + j -- its output as bf16, then its lse as the two 16-bit halves of
    the float32 pattern (low half first), then two zero slots."""
    o_r = np.asarray(o_r, dtype=np.float32)
    lse_r = np.asarray(lse_r, dtype=np.float32)
    rows, H, v = o_r.shape
    if H % N:
        raise ValueError("heads must split evenly over the ranks")
    Hl = H // N
    out = np.zeros((N, rows, Hl, v + 4), dtype=np.uint16)
    lb = lse_r.view(np.uint32)
    for d in range(N):
        heads = slice(d * Hl, (d + 1) * Hl)
        out[d, :, :, :v] = to_bf16_bits(o_r[:, heads, :])
        out[d, :, :, v] = (lb[:, heads] & 0xFFFF).astype(np.uint16)
        out[d, :, :, v + 1] = (lb[:, heads] >> 16).astype(np.uint16)
    return out


def unpack_merge(recv: np.ndarray, base: str = "e"):
    """The owner's merge of what it received: recv [N, rows, Hl, v + 4] (record
    layout of ``pack_heads``, part r from rank r) -> o [rows, Hl, v],
    lse [rows, Hl] by the exact LSE merge, in float64."""
    recv = np.asarray(recv, dtype=np.uint16)
    v = recv.shape[-1] - 4
    o_parts = bf16_bits_to_float(recv[..., :v])
    lse_bits = recv[..., v].astype(np.uint32) | (recv[..., v + 1].astype(np.uint32) << 16)
    lse_parts = lse_bits.view(np.float32).astype(np.float64)
    return lse_merge(o_parts, lse_parts, base)


def merge_bf16_parts(o_parts: np.ndarray, lse_parts: np.ndarray, base: str = "e"):
    """Exact merge of partial results whose outputs travel in bfloat16 and
    whose LSE travels in float32: each part's o is rounded to bf16 (nearest,
    ties to even), its lse to float32, then merged in float64.  Page "DCP",
    "unification with online softmax": the split of a stripe's rows into
    chunks is the same monoid as the split across stripes, so the chunk
    partials merge with the same identity; page "MLA 的 DCP", section 5: the
    partial payload is (512 + 4) x 2 bytes per (row, head), i.e. bf16 o.
    o_parts [P, ..., V], lse_parts [P, ...] in ``base``."""
    o16 = bf16_bits_to_float(to_bf16_bits(np.asarray(o_parts, dtype=np.float64).astype(np.float32)))
    l32 = np.asarray(lse_parts, dtype=np.float64).astype(np.float32).astype(np.float64)
    return lse_merge(o16, l32, base)


# ---- sparse attention with a global top-k selection -------------------------
#
# Page "DCP", "conditions for merging and where they fail": sparse attention
# such as DSA's top-k stays mergeable when the top-k selection is made
# globally; each rank then attends only to the selected tokens it owns.

def sparse_attention(q_req: np.ndarray, kv_req: np.ndarray, S: int, topk: np.ndarray, scale: float,
                     positions=None, v_dim: int = 512):
    """Attention of one request over a per-query-token selection.

    q_req [q_len, H, D]; kv_req [S, D]; topk [q_len, K] global positions chosen
    for each query token (shared by its H heads; -1 = unused slot; the valid
    entries of a token are distinct).  Query t sees the selected positions
    p <= S - q_len + t.  ``positions`` (a rank's owned positions) restricts the
    selection to that stripe.  Returns o [q_len, H, v_dim], natural-log lse
    [q_len, H] (o = 0, lse = -inf for an empty selection)."""
    q_len, H, D = q_req.shape
    topk = np.asarray(topk, dtype=np.int64).reshape(q_len, -1)
    own = None if positions is None else set(np.asarray(positions, dtype=np.int64).tolist())
    o = np.zeros((q_len, H, v_dim))
    lse = np.full((q_len, H), -np.inf)
    for t in range(q_len):
        qp = S - q_len + t
        sel = [int(p) for p in topk[t] if 0 <= p <= qp and (own is None or int(p) in own)]
        sel = np.asarray(sel, dtype=np.int64)
        ot, lt = attention_rows(q_req[t], np.full(H, qp), kv_req[sel] if len(sel) else kv_req[:0], sel,
                                scale, v_dim)
        o[t], lse[t] = ot, lt
    return o, lse
