"""Plain float64 Mamba-2 state-space scan on the CPU (test infrastructure only;
see the package doc for who may import it).

The pages name Mamba-2's chunk-scan and chunk-state functions as the
linear-attention workload their tiled kernels were measured on ("TileLang
paper summary", appendix A.4, the linear attention results) and sketch a
tiled selective scan that walks the sequence in tiles of 64 steps with a
decay exp(delta*A) and an input term delta*B*x ("TileLang programming model
and FlashMLA" page set, the Mamba scan example in "From FlashAttention to
general kernels", section 4). They give no formula, so this module takes the
plainest reading of Mamba-2's scalar-decay state-space layer, per batch b
and head h (head h uses group h // (H / G) of B and C):

    state_t = exp(dt_t * A_h) * state_{t-1} + dt_t * x_t (outer) B_t   (P x N)
    y_t     = state_t @ C_t                                            (P)

with state_{-1} = 0 unless an initial state is given; the state after the
last step is the final state. ``ssd_recurrence`` is that definition, one step
at a time. ``chunk_state`` / ``chunk_scan`` / ``ssd_chunked`` are the chunked
form the two named functions compute (a chunk's own contribution to its
outputs, its end state, and the state carried in from earlier chunks); the
tests pin them to the recurrence. Inputs are widened to float64 first.

Shapes: x [Bt, L, H, P]; dt [Bt, L, H] (positive); A [H] (negative);
B, C [Bt, L, G, N]; y [Bt, L, H, P]; initial / final state [Bt, H, P, N].
"""

import numpy as np


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def _group_of(H, G):
    if G < 1 or H % G:
        raise ValueError("H must be a multiple of the group count G")
    return H // G


def _step(st, dt_t, a, x_t, b_t):
    """One step of the recurrence: decay the state, add the step's input."""
    return np.exp(dt_t * a) * st + dt_t * np.outer(x_t, b_t)


def ssd_recurrence(x, dt, A, B, C, init_state=None):
    """(y, final state) by the step-by-step definition, one (batch, head)
    state at a time."""
    x, dt, A, B, C = (_as64(a) for a in (x, dt, A, B, C))
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = _group_of(H, G)
    y = np.zeros((Bt, L, H, P))
    final = np.zeros((Bt, H, P, N))
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            st = np.zeros((P, N)) if init_state is None else _as64(init_state)[b, h].copy()
            for t in range(L):
                st = _step(st, dt[b, t, h], A[h], x[b, t, h], B[b, t, g])
                y[b, t, h] = st @ C[b, t, g]
            final[b, h] = st
    return y, final


def _chunk_cumsum(dt, A, lo, hi):
    """Inclusive cumulative sum of dt_t * A over steps lo .. hi-1: [Bt, hi-lo, H]."""
    return np.cumsum(dt[:, lo:hi, :] * A[None, None, :], axis=1)


def chunk_state(x, dt, A, B, chunk):
    """End state of every chunk from its own steps only (zero state entering):
    S_c = sum_{s in c} exp(Acs_last - Acs_s) * dt_s * x_s (outer) B_s.
    Returns [Bt, n_chunks, H, P, N] and the chunk's total decay exponent
    Acs_last [Bt, n_chunks, H]."""
    x, dt, A, B = (_as64(a) for a in (x, dt, A, B))
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = _group_of(H, G)
    nc = -(-L // chunk)
    S = np.zeros((Bt, nc, H, P, N))
    tot = np.zeros((Bt, nc, H))
    for c in range(nc):
        lo, hi = c * chunk, min(L, (c + 1) * chunk)
        acs = _chunk_cumsum(dt, A, lo, hi)                      # [Bt, Q, H]
        w = np.exp(acs[:, -1:, :] - acs) * dt[:, lo:hi, :]     # [Bt, Q, H]
        for h in range(H):
            g = h // hpg
            xs = x[:, lo:hi, h, :] * w[:, :, h, None]           # [Bt, Q, P]
            S[:, c, h] = np.einsum("bqp,bqn->bpn", xs, B[:, lo:hi, g, :])
        tot[:, c] = acs[:, -1, :]
    return S, tot


def state_passing(S, tot, init_state=None):
    """States entering each chunk and the final state: prev_0 = initial state
    (zero if none), prev_{c+1} = exp(tot_c) * prev_c + S_c; the final state is
    prev_{n_chunks}."""
    prev = np.zeros_like(S)
    run = np.zeros_like(S[:, 0]) if init_state is None else _as64(init_state).copy()
    for c in range(S.shape[1]):
        prev[:, c] = run
        run = np.exp(tot[:, c])[:, :, None, None] * run + S[:, c]
    return prev, run


def chunk_scan(x, dt, A, B, C, prev, chunk):
    """Outputs of every chunk from its own steps (causal within the chunk) and
    the state carried in: y_t = sum_{s<=t in c} (C_t . B_s) exp(Acs_t - Acs_s)
    dt_s x_s + exp(Acs_t) * prev_c @ C_t."""
    x, dt, A, B, C = (_as64(a) for a in (x, dt, A, B, C))
    Bt, L, H, P = x.shape
    G = B.shape[2]
    hpg = _group_of(H, G)
    y = np.zeros((Bt, L, H, P))
    for c in range(prev.shape[1]):
        lo, hi = c * chunk, min(L, (c + 1) * chunk)
        Q = hi - lo
        acs = _chunk_cumsum(dt, A, lo, hi)                      # [Bt, Q, H]
        causal = np.tril(np.ones((Q, Q), dtype=bool))
        for h in range(H):
            g = h // hpg
            cb = np.einsum("btn,bsn->bts", C[:, lo:hi, g], B[:, lo:hi, g])
            decay = np.exp(acs[:, :, h, None] - acs[:, None, :, h])
            gmat = np.where(causal[None], cb * decay, 0.0) * dt[:, None, lo:hi, h]
            y[:, lo:hi, h] = np.einsum("bts,bsp->btp", gmat, x[:, lo:hi, h])
            y[:, lo:hi, h] += np.exp(acs[:, :, h])[:, :, None] * np.einsum(
                "bpn,btn->btp", prev[:, c, h], C[:, lo:hi, g])
    return y


def ssd_chunked(x, dt, A, B, C, chunk=64, init_state=None):
    """(y, final state) through chunk_state, state_passing and chunk_scan
    (equal to the recurrence up to rounding)."""
    Bt, L, H, P = np.shape(x)
    N = np.shape(B)[3]
    if L == 0:
        final = np.zeros((Bt, H, P, N)) if init_state is None else _as64(init_state).copy()
        return np.zeros((Bt, 0, H, P)), final
    S, tot = chunk_state(x, dt, A, B, chunk)
    prev, final = state_passing(S, tot, init_state)
    return chunk_scan(x, dt, A, B, C, prev, chunk), final


def ssd_rows(x, dt, A, B, C, pairs, chunk=64, init_state=None):
    """(y, final state) of selected (batch, head) pairs only (the chunked form
    restricted to one head at a time), for sampled checks on large inputs:
    [len(pairs), L, P] and [len(pairs), P, N]."""
    x, dt, B, C = (np.asarray(a) for a in (x, dt, B, C))
    H, G = x.shape[2], B.shape[2]
    hpg = _group_of(H, G)
    ys, fs = [], []
    A = _as64(A)
    for b, h in pairs:
        g = h // hpg
        s0 = None if init_state is None else np.asarray(init_state)[b:b + 1, h:h + 1]
        y, f = ssd_chunked(x[b:b + 1, :, h:h + 1], dt[b:b + 1, :, h:h + 1], A[h:h + 1],
                           B[b:b + 1, :, g:g + 1], C[b:b + 1, :, g:g + 1], chunk, s0)
        ys.append(y[0, :, 0])
        fs.append(f[0, 0])
    return np.stack(ys), np.stack(fs)
