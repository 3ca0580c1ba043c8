"""Plain float64 attention forward on the CPU (test infrastructure, see package doc).

Every input is widened exactly to float64 before any arithmetic (bf16 and fp32
values are exactly representable), so the only rounding here is float64's.
No function here tiles the key axis except ``online_attention``, whose whole
point is to run the tiled recurrence; ``attention`` and ``mla_decode`` compute
each query row's complete score vector and its softmax by the definition.
Rows are independent under that definition, so computing several rows with
one matrix product changes no arithmetic.
"""

import numpy as np

_NEG_INF = -np.inf


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _allowed_count(i, Sq, Skv, causal):
    """How many leading keys query row ``i`` may see.

    Non-causal: all ``Skv`` keys. Causal: key j is visible to row i when
    j <= i + (Skv - Sq), i.e. the mask is aligned to the bottom-right corner
    of the Sq x Skv score block; with Sq == Skv this is the usual j <= i.
    The pages never state a causal rule (the workloads ask for causal runs);
    this is the reading adopted and documented with the design.
    """
    if not causal:
        return Skv
    return int(min(Skv, max(0, i + (Skv - Sq) + 1)))


def _softmax_rows(s, counts):
    """Two-pass softmax of each row of ``s`` over its first ``counts[r]`` entries.

    Pass 1 takes the row max m over the visible entries; pass 2 forms
    exp(s - m), its sum l, and returns (P, m, l). Subtracting m is the
    numerical-stability step the study notes insist on (leaving it out
    overflows to NaN). Rows with no visible entry get P = 0, m = -inf, l = 0.
    """
    n_rows, n_cols = s.shape
    col = np.arange(n_cols)[None, :]
    visible = col < np.asarray(counts)[:, None]
    masked = np.where(visible, s, _NEG_INF)
    m = masked.max(axis=1) if n_cols > 0 else np.full(n_rows, _NEG_INF)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(visible, np.exp(masked - safe_m[:, None]), 0.0)
    l = p.sum(axis=1)
    return p, m, l


def _finish(p, m, l, v):
    """O = P*V / l and LSE = m + ln l; empty rows give O = 0, LSE = -inf."""
    o = p @ v
    empty = l == 0.0
    denom = np.where(empty, 1.0, l)
    o = o / denom[:, None]
    o[empty] = 0.0
    lse = np.where(empty, _NEG_INF, m + np.log(np.where(empty, 1.0, l)))
    return o, lse


def attention(q, k, v, scale, causal=False, rows=None, row_group=1024):
    """Multi-head attention forward by its definition.

    Follows the standard attention definition in "TileLang study notes",
    section "FlashAttention implementation": S = Q*K^T (here scaled by
    ``scale``), P = softmax(S) along each row, O = P*V. The log-sum-exp
    written beside O is LSE_i = ln sum_j exp(S_ij), the natural log; the
    FlashMLA walk-through keeps this quantity as its running "logsum"
    (section 3.1).

    Shapes: q [B, H, Sq, D]; k [B, Hkv, Skv, D]; v [B, Hkv, Skv, Dv] with
    H a multiple of Hkv (query head h reads KV head h // (H // Hkv)).
    ``rows`` optionally restricts the query rows computed (a sample).
    Returns (O [B, H, n_rows, Dv], LSE [B, H, n_rows]) as float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    scale = float(scale)
    B, H, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = H // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    Dv = v.shape[3]
    out = np.zeros((B, H, rows.size, Dv))
    lse = np.zeros((B, H, rows.size))
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, h // group], v[b, h // group]
            for r0 in range(0, rows.size, row_group):
                rr = rows[r0:r0 + row_group]
                s = scale * (q[b, h, rr] @ kh.T)
                counts = [_allowed_count(int(i), Sq, Skv, causal) for i in rr]
                p, m, l = _softmax_rows(s, counts)
                o_blk, lse_blk = _finish(p, m, l, vh)
                out[b, h, r0:r0 + rr.size] = o_blk
                lse[b, h, r0:r0 + rr.size] = lse_blk
    return out, lse


def online_attention(q, k, v, scale, causal=False, block=64):
    """The tiled online-softmax recurrence, in float64, for self-checks only.

    Follows "TileLang study notes", subsection "Online Softmax": for every
    new key block with scores S_blk, m_new = max(m_prev, rowmax S_blk),
    l_new = l_prev*exp(m_prev - m_new) + rowsum exp(S_blk - m_new), and
    O_new = O_prev*exp(m_prev - m_new) + exp(S_blk - m_new)*V_blk; at the end
    O = O/l. Same shapes and return values as ``attention``. While a row has
    seen no visible key (m = -inf) the rescale factor is taken as 1, which
    leaves the still-zero accumulators unchanged.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    scale = float(scale)
    B, H, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    group = H // Hkv
    Dv = v.shape[3]
    out = np.zeros((B, H, Sq, Dv))
    lse = np.zeros((B, H, Sq))
    counts = np.array([_allowed_count(i, Sq, Skv, causal) for i in range(Sq)])
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, h // group], v[b, h // group]
            m = np.full(Sq, _NEG_INF)
            l = np.zeros(Sq)
            acc = np.zeros((Sq, Dv))
            for j0 in range(0, Skv, block):
                j1 = min(Skv, j0 + block)
                s = scale * (q[b, h] @ kh[j0:j1].T)
                visible = (np.arange(j0, j1)[None, :] < counts[:, None])
                s = np.where(visible, s, _NEG_INF)
                m_new = np.maximum(m, s.max(axis=1))
                alive = np.isfinite(m_new)
                alpha = np.where(alive, np.exp(np.where(alive, m - m_new, 0.0)), 1.0)
                p = np.where(visible, np.exp(s - np.where(alive, m_new, 0.0)[:, None]), 0.0)
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + p @ vh[j0:j1]
                m = m_new
            empty = l == 0.0
            out[b, h] = np.where(empty[:, None], 0.0, acc / np.where(empty, 1.0, l)[:, None])
            lse[b, h] = np.where(empty, _NEG_INF, m + np.log(np.where(empty, 1.0, l)))
    return out, lse


def attention_partial(q, k, v, scale, key_lo, key_hi, causal=False):
    """Attention restricted to keys [key_lo, key_hi): normalised O_s and lse_s.

    The causal rule is applied with the keys' global indices. A range with
    no visible key gives O_s = 0 and lse_s = -inf. Shapes as ``attention``.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    group = H // Hkv
    out = np.zeros((B, H, Sq, v.shape[3]))
    lse = np.zeros((B, H, Sq))
    scale = float(scale)
    for b in range(B):
        for h in range(H):
            kh = k[b, h // group, key_lo:key_hi]
            vh = v[b, h // group, key_lo:key_hi]
            s = scale * (q[b, h] @ kh.T)
            counts = [max(0, min(key_hi, _allowed_count(i, Sq, Skv, causal)) - key_lo)
                      for i in range(Sq)]
            p, m, l = _softmax_rows(s, counts)
            out[b, h], lse[b, h] = _finish(p, m, l, vh)
    return out, lse


def visible_keys(i, Sq, Skv, causal=False, window=0, block_row=None, block=64):
    """Boolean vector over the Skv keys: which keys query row ``i`` sees.

    Key j is visible when 0 <= j < Skv and, with off = Skv - Sq (the
    bottom-right alignment used for the causal rule),
      * causal: j <= i + off;
      * window W > 0: i + off - W <= j < i + off + W. "TileLang programming
        model and FlashMLA", section 5.1 (local attention), makes a sliding window by running the
        key loop over the positions from the query position minus the window
        size up to (not including) the query position plus the window size;
      * block mask: block_row[j // block] != 0, where ``block_row`` is the
        mask row of the query block i // block. The same section makes sparse
        attention by a mask matrix that decides which parts are computed;
        the reading here is one bit per (query block, key block) pair.
    """
    j = np.arange(Skv)
    vis = np.ones(Skv, dtype=bool)
    pos = i + (Skv - Sq)
    if causal:
        vis &= j <= pos
    if window > 0:
        vis &= (j >= pos - window) & (j < pos + window)
    if block_row is not None:
        vis &= np.asarray(block_row)[j // block] != 0
    return vis


def attention_masked(q, k, v, scale, causal=False, window=0, block_mask=None, block=64, rows=None):
    """Attention with grouped KV heads, a sliding window and a block mask.

    The same definition as ``attention`` (S = scale*Q*K^T, softmax over each
    row's visible keys, O = P*V, natural-log LSE), with the visible set of
    ``visible_keys``. KV heads are shared by groups of query heads as in
    ``attention`` (query head h reads KV head h // (H // Hkv)); with one KV
    head this is the multi-query form of "TileLang programming model and
    FlashMLA", section 5.1.
    ``block_mask`` is [B, H, ceil(Sq/block), ceil(Skv/block)] (nonzero =
    computed) or None. A row that sees no key gets O = 0 and LSE = -inf.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    scale = float(scale)
    B, H, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = H // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    Dv = v.shape[3]
    out = np.zeros((B, H, rows.size, Dv))
    lse = np.zeros((B, H, rows.size))
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, h // group], v[b, h // group]
            s = scale * (q[b, h, rows] @ kh.T)
            vis = np.stack([visible_keys(int(i), Sq, Skv, causal, window,
                                         None if block_mask is None else block_mask[b, h, int(i) // block],
                                         block) for i in rows]) if rows.size else np.zeros((0, Skv), bool)
            masked = np.where(vis, s, _NEG_INF)
            m = masked.max(axis=1) if Skv > 0 else np.full(rows.size, _NEG_INF)
            safe_m = np.where(np.isfinite(m), m, 0.0)
            p = np.where(vis, np.exp(masked - safe_m[:, None]), 0.0)
            l = p.sum(axis=1)
            out[b, h], lse[b, h] = _finish(p, m, l, vh)
    return out, lse


def combine_partials(o_parts, lse_parts):
    """Exact merge of per-range partials (the split-KV reading).

    With lse = ln sum_s exp(lse_s), the full result is
    O = sum_s exp(lse_s - lse) * O_s, because each O_s is normalised by its
    own sum exp(lse_s). Ranges with lse_s = -inf carry weight 0; if every
    range is empty the result is O = 0, lse = -inf.
    ``o_parts`` [n_split, ..., Dv], ``lse_parts`` [n_split, ...].
    """
    o_parts, lse_parts = _as64(o_parts), _as64(lse_parts)
    mx = lse_parts.max(axis=0)
    alive = np.isfinite(mx)
    safe = np.where(alive, mx, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe[None]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(alive, safe + np.log(np.where(alive, tot, 1.0)), _NEG_INF)
    o = (w[..., None] * o_parts).sum(axis=0) / np.where(alive, tot, 1.0)[..., None]
    o = np.where(alive[..., None], o, 0.0)
    return o, lse


def mla_decode(q, q_pe, kv, k_pe, indptr, scale, batches=None):
    """MLA decode forward by its definition (one query position per batch).

    Follows "TileLang programming model and FlashMLA", sections 2.1-2.2 and
    3.1: the query heads of batch b share one KV head made of a latent part
    KV (width Dl) and a rotary part K_pe (width Dr); the score of head h
    against key j is scale*(Q[b,h]*KV[j] + Q_pe[b,h]*K_pe[j]) -- the two
    products the walk-through accumulates into one score tile -- and, as the
    variant fixes, the values are the latent rows KV[j] themselves.
    Batch b owns keys indptr[b] <= j < indptr[b+1] of the packed arrays.

    Shapes: q [B, H, Dl], q_pe [B, H, Dr], kv [N, Dl], k_pe [N, Dr],
    indptr [B+1]. Returns (O [nb, H, Dl], LSE [nb, H]) as float64 for the
    selected ``batches`` (all by default).
    """
    q, q_pe, kv, k_pe = _as64(q), _as64(q_pe), _as64(kv), _as64(k_pe)
    indptr = np.asarray(indptr, dtype=np.int64)
    scale = float(scale)
    B, H, Dl = q.shape
    batches = np.arange(B) if batches is None else np.asarray(batches, dtype=np.int64)
    out = np.zeros((batches.size, H, Dl))
    lse = np.zeros((batches.size, H))
    for n, b in enumerate(batches):
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        s = scale * (q[b] @ kv[lo:hi].T + q_pe[b] @ k_pe[lo:hi].T)
        p, m, l = _softmax_rows(s, [hi - lo] * H)
        out[n], lse[n] = _finish(p, m, l, kv[lo:hi])
    return out, lse


def mla_decode_rows(q, q_pe, kv, k_pe, indptr, scale, pairs):
    """``mla_decode`` for a sample of (batch, head) pairs, one at a time.

    Returns (O [n, Dl], LSE [n]). Used where the full output is too costly.
    """
    q, q_pe = _as64(q), _as64(q_pe)
    indptr = np.asarray(indptr, dtype=np.int64)
    out = np.zeros((len(pairs), q.shape[2]))
    lse = np.zeros(len(pairs))
    for n, (b, h) in enumerate(pairs):
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        kvb, kpb = _as64(kv[lo:hi]), _as64(k_pe[lo:hi])
        s = float(scale) * (kvb @ q[b, h] + kpb @ q_pe[b, h])
        p, m, l = _softmax_rows(s[None, :], [hi - lo])
        o, ls = _finish(p, m, l, kvb)
        out[n], lse[n] = o[0], ls[0]
    return out, lse
