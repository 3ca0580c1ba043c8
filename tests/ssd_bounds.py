"""Error bounds for the bf16 Mamba-2 scan, derived term by term from where a
chunked bf16 kernel rounds (test infrastructure; computed in float64 from the
inputs and the exact chunked quantities, never from a kernel's output).

A chunked scan in bf16 (64-step chunks; the form of the chunk-scan and
chunk-state functions, "TileLang paper summary", appendix A.4) rounds to bf16
at four points besides its bf16 inputs:

1. G_ts = (C_t . B_s) exp(Acs_t - Acs_s) dt_s, the decay-weighted scores inside
   a chunk, before they multiply x_s;
2. the state entering a chunk, where it meets C_t (y_t += exp(Acs_t) prev . C_t);
3. B_s exp(Acs_last - Acs_s) dt_s, the decay-weighted B of the state update
   (the carried state itself stays fp32, so this error propagates to later
   chunks with the state's decay);
4. y itself.

Rounding to nearest makes each of 1-3 a relative error d with |d| <= u = 2^-8
on one term of a sum. Taking those errors as independent and of mean zero
(probabilistic rounding error analysis, Higham and Mary, SIAM J. Sci. Comput.
41 (2019)), Hoeffding's inequality bounds the error of a sum sum_i d_i t_i by
lam * u * sqrt(sum_i t_i^2) except with probability 2 exp(-lam^2 / 2)
(3e-8 per element at lam = 6). For y_tp the squared terms are

    sum_s (G_ts x_sp)^2                                  (point 1)
  + exp(2 Acs_t) sum_n C_tn^2 (state_pn^2 + E2_pn)       (points 2 and 3)

where E2 carries the squared point-3 terms of earlier chunks forward:
E2 <- exp(2 Acs_last) E2 + sum_s (coef_s B_sn x_sp)^2. Point 4 adds at most
half a bf16 ulp of the computed value. Besides rounding to bf16 the kernel
works in fp32; those errors are bounded in the worst case, not statistically:

* the chunk's running sum of dt*A is formed in fp32, and a decay exponent
  Acs_t - Acs_s is a difference of two such sums, so it can carry an absolute
  error of up to 2 (Q + 1) 2^-24 sum_chunk |dt A| (Q = 64 steps), i.e. that
  relative error on every decayed term (plus 2^-20 for exp2 and the products);
  applied to sum_s |G_ts x_sp| + exp(Acs_t) sum_n |C_tn| S_pn with S the state
  of absolute values (S <- exp(Acs_last) S + |x|^T |coef B|, S_0 = |init|);
* fp32 dot products and accumulation: (320 + 4 n_chunks) 2^-24 times the same
  sums with |C_t||B_s| in place of |C_t . B_s| (128-term C.B, 64-term G.x and
  128-term C.prev products, two roundings per chunk of the carried state).

The fp32 final state sees point 3 only: lam u sqrt(E2) plus the same fp32
terms on S.
"""

import numpy as np

U = 2.0 ** -8          # unit roundoff of bf16 (8 significant bits)
LAM = 6.0              # Hoeffding multiplier: 2 exp(-18) ~ 3e-8 per element
CHUNK = 64


def half_ulp(x):
    """Half a bf16 ulp at |x|."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def head_scales(x, dt, a, B, C, init=None, chunk=CHUNK):
    """Error scales of one (batch, head): x [L, P], dt [L], a (scalar), B and
    C [L, N] (the group's), init [P, N] or None, all exact values. Returns
    (sig_y, abs_g, abs_y) [L, P] and (sig_f, abs_f) [P, N], plus rho and the
    fp32 factors (see the module doc)."""
    x, dt, B, C = (np.asarray(v, dtype=np.float64) for v in (x, dt, B, C))
    a = float(a)
    L, P = x.shape
    N = B.shape[1]
    st = np.zeros((P, N)) if init is None else np.asarray(init, dtype=np.float64).copy()
    S = np.abs(st)
    E2 = np.zeros((P, N))
    sig2 = np.zeros((L, P))
    abs_g = np.zeros((L, P))
    abs_y = np.zeros((L, P))
    s_max = 0.0
    for lo in range(0, L, chunk):
        hi = min(L, lo + chunk)
        xs, Bs, Cs, d = x[lo:hi], B[lo:hi], C[lo:hi], dt[lo:hi]
        acs = np.cumsum(d * a)
        s_max = max(s_max, float(np.abs(d * a).sum()))
        W = np.tril(np.exp(acs[:, None] - acs[None, :])) * d[None, :]
        G = (Cs @ Bs.T) * W
        G_abs = (np.abs(Cs) @ np.abs(Bs).T) * W
        ey = np.exp(acs)[:, None]
        state_part = ey * (np.abs(Cs) @ S.T)
        sig2[lo:hi] = (G * G) @ (xs * xs) + ey ** 2 * ((Cs * Cs) @ (st * st + E2).T)
        abs_g[lo:hi] = np.abs(G) @ np.abs(xs) + state_part
        abs_y[lo:hi] = G_abs @ np.abs(xs) + state_part
        coef = np.exp(acs[-1] - acs) * d
        wB = coef[:, None] * Bs
        dec = np.exp(acs[-1])
        st = dec * st + xs.T @ wB
        S = dec * S + np.abs(xs).T @ np.abs(wB)
        E2 = dec * dec * E2 + (xs * xs).T @ (wB * wB)
    nc = -(-L // chunk)
    rho = 2 * (chunk + 1) * 2.0 ** -24 * s_max + 2.0 ** -20
    fp_y = (320 + 4 * nc) * 2.0 ** -24
    fp_f = (64 + 4 * nc) * 2.0 ** -24
    return {"sig_y": np.sqrt(sig2), "abs_g": abs_g, "abs_y": abs_y, "sig_f": np.sqrt(E2), "abs_f": S,
            "rho": rho, "fp_y": fp_y, "fp_f": fp_f}


def y_bound(ref, sc, lam=LAM):
    """Per-element bound on |y - ref| for one head's y [L, P]."""
    stat = lam * U * sc["sig_y"]
    return stat + half_ulp(np.abs(ref) + stat) + sc["rho"] * sc["abs_g"] + sc["fp_y"] * sc["abs_y"]


def y_mean_bound(ref, sc, lam=LAM):
    """Bound on the mean of |y - ref| over one head: E|sum d_i t_i| <= u sqrt(sum t_i^2)
    per element, plus the worst-case terms."""
    stat = lam * U * sc["sig_y"]
    return float(np.mean(U * sc["sig_y"] + half_ulp(np.abs(ref) + stat) + sc["rho"] * sc["abs_g"]
                         + sc["fp_y"] * sc["abs_y"]))


def f_bound(sc, lam=LAM):
    """Per-element bound on the fp32 final state's error [P, N]."""
    return lam * U * sc["sig_f"] + (sc["rho"] + sc["fp_f"]) * sc["abs_f"]


def check_head(y, ref_y, sc, what, f=None, ref_f=None):
    """Assert the per-element and mean bounds for one head; returns a message."""
    err = np.abs(y - ref_y)
    bnd = y_bound(ref_y, sc)
    worst = float((err / np.maximum(bnd, 1e-300)).max()) if err.size else 0.0
    mean_err = float(err.mean()) if err.size else 0.0
    mean_bnd = y_mean_bound(ref_y, sc) if err.size else 0.0
    msg = f"{what}: max|dy|={err.max() if err.size else 0:.3g} worst |dy|/bound={worst:.3g} " \
          f"mean|dy|={mean_err:.3g} (bound {mean_bnd:.3g})"
    if f is not None:
        ef = np.abs(f - ref_f)
        wf = float((ef / np.maximum(f_bound(sc), 1e-300)).max())
        msg += f"; final state max|d|={ef.max():.3g} worst/bound={wf:.3g}"
        assert wf <= 1.0, msg
    print(msg, flush=True)
    assert worst <= 1.0, msg
    assert mean_err <= mean_bnd, msg
    return msg
