"""Independent fp64 statement of the chunked Gated Delta Rule formulas.

TEST INFRASTRUCTURE ONLY: used by the CPU tests to pin the recurrence oracle
(``gdr_oracle.c``).  The two are written from different passages of the
pages -- this file from the chunked formulas of the "Qwen3Next Samples"
(PyPTO) page, the oracle from the per-token recurrence of the
"lite_boost.ops.recurrent_gated_delta_rule" page -- so their agreement on
brute-force inputs pins the signs, masks and gate indices of both.

It follows the "Qwen3Next Samples" page, section Mathematical Formulas, in
its order, for each chunk of L tokens (the page fixes L = 128; any L >= 1
gives the same result, which the tests use):

  L2 Normalization      q, k <- x / sqrt(sum x^2 + eps), eps = 1e-6;
                        q is then multiplied by `scale`.
  Gate Cumulative Sum   g_cum = T_tril g  (chunk-local inclusive prefix).
  Decay Mask            D = exp((g_cum_i - g_cum_j) for i >= j), 0 above.
  Pre-Attention Matrix  k_beta = k * beta;  A = (k_beta k^T) . D . M_mask.
  Matrix Inversion      "A^-1" := (I - A)^-1 = I + A + A^2 + ... (finite,
                        A is strictly lower triangular), or equivalently the
                        row recurrence (forward substitution).
  Value and Key Cumulative Decay
                        v_out = A^-1 (v * beta);
                        k_cumdecay = A^-1 (k_beta * exp(g_cum)).
  Recurrent State Attention
                        v' = k_cumdecay S^T;  o_inter = (q * exp(g_cum)) S^T;
                        o = o_inter + (q k^T . D . T_tril)(v_out - v').
  State Update          S_new = S exp(g_last) + v_new^T k_gexp,
                        k_gexp = k * exp(g_last - g_cum).

Readings of passages the page leaves open (each one is the only reading under
which the chunked form equals the recurrence of the decode page; the tests
show the alternatives disagree):
  * M_mask ("lower triangular negative value mask") is -1 strictly below the
    diagonal and 0 elsewhere.
  * T_tril in the output term keeps the diagonal (inclusive lower triangle),
    as it does for the cumulative sum.
  * g_last is the chunk-local cumulative gate at the last valid row, and the
    `g` inside k_gexp is g_cum.
  * v_new = v_out - v'.
  * The page writes the state as S [Dv, Dk] (so that k S^T has shape [L, Dv]);
    the boundary layout used everywhere else is S [Dk, Dv] = the page's S^T.
    This module takes and returns [Dk, Dv] and transposes internally.
  * A ragged last chunk is processed with its r < L valid rows only.

Per-key gate (the decode page's gk, read as applying to every prefill token):
state row d decays by exp(g_t + gk_t[d]) at token t, so every scalar decay of
the chunk becomes a per-key one, with G = T_tril (g + gk) [r, Dk]:
  A[i,j] = -beta_i sum_d k_i[d] k_j[d] exp(G_i[d] - G_j[d])   (j < i)
  k_cumdecay = A^-1 (k_beta * exp(G));  o_inter = (q * exp(G)) S
  o += (sum_d q_i[d] k_j[d] exp(G_i[d] - G_j[d]), j <= i) v_new
  S_new = diag(exp(G_last)) S + (k * exp(G_last - G))^T v_new
(chunk_step_gk; with gk = 0 it is chunk_step).

Update rules ("LinearAttention" page, attribute update_rule): the rules
without a gate (delta, linear) take g = 0; the rules without the delta term
(gated, linear) have no pre-attention matrix, so its inverse is I, v_out = v
and k_cumdecay = 0 (v_new = v).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def l2norm(x, eps=EPS):
    """Row-wise x / sqrt(sum x^2 + eps) (L2 Normalization formula)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def inverse_neumann(A):
    """(I - A)^-1 as the finite Neumann series I + A + A^2 + ... (A nilpotent)."""
    n = A.shape[0]
    T = np.eye(n)
    P = np.eye(n)
    for _ in range(n):
        P = P @ A
        T = T + P
        if not np.any(P):
            break
    return T


def inverse_rows(A):
    """(I - A)^-1 by the row recurrence: row i of the strict lower part is
    A[i,:i] + A[i,:i] @ Tinv[:i,:i]; the unit diagonal is added at the end."""
    n = A.shape[0]
    T = np.zeros((n, n))
    for i in range(n):
        T[i, :i] = A[i, :i] + A[i, :i] @ T[:i, :i]
    return T + np.eye(n)


def chunk_step(q, k, v, g, beta, S_dkdv, inverse=inverse_rows,
               mask_sign=-1.0, strict_out_tril=False, raw_g_last=False, raw_g_in_kgexp=False, delta=True):
    """One chunk of r rows (already L2-normalised q, k; q already scaled).

    q, k [r, Dk]; v [r, Dv]; g, beta [r]; S_dkdv [Dk, Dv].
    Returns (o [r, Dv], S_new [Dk, Dv]).  The keyword switches select the
    alternative readings that the tests show to be wrong.
    """
    r = q.shape[0]
    tril = np.tril(np.ones((r, r)))
    g_cum = tril @ g                                         # Gate Cumulative Sum
    diff = g_cum[:, None] - g_cum[None, :]
    D = np.exp(np.where(tril > 0, diff, 0.0)) * tril         # Decay Mask (0 above)
    k_beta = k * beta[:, None]                               # Pre-Attention Matrix
    M_mask = mask_sign * np.tril(np.ones((r, r)), -1)
    A = (k_beta @ k.T) * D * M_mask
    if delta:
        Ainv = inverse(A)                                    # Matrix Inversion
        v_out = Ainv @ (v * beta[:, None])                   # Value and Key Cumulative Decay
        k_cumdecay = Ainv @ (k_beta * np.exp(g_cum)[:, None])
    else:                                                    # no delta term: v_new = v
        v_out = v
        k_cumdecay = np.zeros_like(k)
    S = S_dkdv.T                                             # the page's S is [Dv, Dk]
    v_prime = k_cumdecay @ S.T                               # Recurrent State Attention
    o_inter = (q * np.exp(g_cum)[:, None]) @ S.T
    out_mask = np.tril(np.ones((r, r)), -1) if strict_out_tril else tril
    v_new = v_out - v_prime
    o = o_inter + ((q @ k.T) * D * out_mask) @ v_new
    g_last = g[-1] if raw_g_last else g_cum[-1]              # State Update
    g_in = g if raw_g_in_kgexp else g_cum
    k_gexp = k * np.exp(g_last - g_in)[:, None]
    S_new = S * np.exp(g_last) + v_new.T @ k_gexp
    return o, S_new.T


def chunk_step_gk(q, k, v, g, gk, beta, S_dkdv, delta=True):
    """One chunk with the per-key gate gk [r, Dk] (module docstring); the
    decay factors are formed directly, exp(G_i[d] - G_j[d]) per (i, j, d)."""
    r = q.shape[0]
    tril = np.tril(np.ones((r, r)))
    G = tril @ (g[:, None] + gk)                                           # [r, Dk]
    E = np.exp(np.where(tril[:, :, None] > 0, G[:, None, :] - G[None, :, :], 0.0)) * tril[:, :, None]
    k_beta = k * beta[:, None]
    if delta:
        A = -np.einsum("id,jd,ijd->ij", k_beta, k, E) * np.tril(np.ones((r, r)), -1)
        Ainv = inverse_rows(A)
        v_out = Ainv @ (v * beta[:, None])
        k_cumdecay = Ainv @ (k_beta * np.exp(G))
    else:
        v_out = v
        k_cumdecay = np.zeros_like(k)
    v_new = v_out - k_cumdecay @ S_dkdv
    o = (q * np.exp(G)) @ S_dkdv + (np.einsum("id,jd,ijd->ij", q, k, E) * tril) @ v_new
    S_new = np.exp(G[-1])[:, None] * S_dkdv + (k * np.exp(G[-1][None, :] - G)).T @ v_new
    return o, S_new


def prefill(q, k, v, g, beta, state_in, cu_seqlens, scale, L=128, rule="gated_delta", gk=None, **readings):
    """Chunked prefill over packed varlen sequences, fp64.

    q, k [T,Nqk,Dk]; v [T,Nv,Dv]; g, beta [T,Nv]; state_in [B,Nv,Dk,Dv] or
    None; cu_seqlens [B+1]; gk [T,Nv,Dk] or None.  Value head h uses qk head
    h // (Nv // Nqk).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    if rule in ("delta", "linear"):
        g = np.zeros_like(g)
        gk = None
    if gk is not None:
        gk = np.asarray(gk, np.float64)
    beta = np.asarray(beta, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    readings = dict(readings, delta=rule in ("gated_delta", "delta"))
    T, Nqk, Dk = q.shape
    Nv, Dv = v.shape[1], v.shape[2]
    B = len(cu) - 1
    G = Nv // Nqk
    qn = l2norm(q) * scale
    kn = l2norm(k)
    out = np.zeros((T, Nv, Dv))
    state_out = np.zeros((B, Nv, Dk, Dv))
    for b in range(B):
        for h in range(Nv):
            hq = h // G
            S = np.zeros((Dk, Dv)) if state_in is None else np.array(state_in[b, h], np.float64)
            for c0 in range(cu[b], cu[b + 1], L):
                c1 = min(c0 + L, cu[b + 1])
                if gk is None:
                    o, S = chunk_step(qn[c0:c1, hq], kn[c0:c1, hq], v[c0:c1, h], g[c0:c1, h],
                                      beta[c0:c1, h], S, **readings)
                else:
                    o, S = chunk_step_gk(qn[c0:c1, hq], kn[c0:c1, hq], v[c0:c1, h], g[c0:c1, h],
                                         gk[c0:c1, h], beta[c0:c1, h], S, delta=readings["delta"])
                out[c0:c1, h] = o
            state_out[b, h] = S
    return out, state_out
