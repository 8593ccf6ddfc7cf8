"""Float64 reference gradients of the masked attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward is the one ``attention_ref`` defines: for query row i and key j,
``y_ij = scale * q_i . k_j``, the logit ``z_ij = cap * tanh(y_ij / cap)``
(or ``z = y`` without a cap), ``p_ij = exp(z_ij) / sum_{j' allowed} exp(z_ij')``
over the allowed keys (0 elsewhere), and ``o_i = sum_j p_ij v_j``.  Given the
upstream gradient ``do = dL/do``, the gradients below are that definition
differentiated by the chain rule, written out on the materialised matrices
with no blocking:

* ``dv_j = sum_i p_ij do_i``;
* ``dp_ij = do_i . v_j``;
* the softmax Jacobian gives ``dz_ij = p_ij (dp_ij - D_i)`` with
  ``D_i = sum_j p_ij dp_ij`` (which equals ``do_i . o_i``);
* the cap multiplies by ``dz/dy = 1 - tanh(y / cap)^2``: ``dy_ij = dz_ij (1 - t_ij^2)``;
* ``dq_i = scale * sum_j dy_ij k_j`` and ``dk_j = scale * sum_i dy_ij q_i``.

With GQA the gradients of a K/V head sum over the query heads that read it.
A row with no allowed key has p = 0 and contributes nothing.

Sources: the forward recomputation from the stored lse residual (Lecture 13
"Pallas Kernels and Splash Attention", section 6.3: the forward writes the
per-row logsumexp for the backward; joto.ai "LSE 与 Online Softmax": the
backward rebuilds p = exp(s - lse) on chip).  The pages print no gradient
formulas; the ones above are the plain calculus of the forward definition
and are pinned in ``tests/test_backward_oracle.py`` by central finite
differences of ``attention_ref`` itself.
"""

from __future__ import annotations

import numpy as np

from .attention import _seg_for_batch, allowed


def attention_bwd_ref(q, k, v, do, *, scale: float, soft_cap: float = 0.0,
                      causal: bool = False, window_left: int = -1,
                      window_right: int = -1, seg_q=None, seg_kv=None,
                      q_offset: int = 0):
    """Gradients (dq, dk, dv) in float64 of ``sum(do * o)`` with
    ``o = attention_ref(q, k, v, ...)``.

    Shapes as in ``attention_ref``: q [B, Hq, L_q, d_qk], k [B, Hkv, L_kv,
    d_qk], v [B, Hkv, L_kv, d_v], do [B, Hq, L_q, d_v].  Returns dq like q,
    dk like k and dv like v, all float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    B, Hq, L_q, d_qk = q.shape
    _, Hkv, L_kv, _ = k.shape
    if Hq % Hkv != 0 or do.shape != (B, Hq, L_q, v.shape[3]):
        raise ValueError("shapes do not agree")
    group = Hq // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    i = np.arange(L_q)[:, None]
    j = np.arange(L_kv)[None, :]
    for b in range(B):
        a = allowed(i, j, L_q=L_q, L_kv=L_kv, causal=causal, window_left=window_left,
                    window_right=window_right, seg_q=_seg_for_batch(seg_q, b),
                    seg_kv=_seg_for_batch(seg_kv, b), q_offset=q_offset)
        has = a.any(axis=1)
        for h in range(Hq):
            kh = h // group
            qf = q[b, h].astype(np.float64)
            kf = k[b, kh].astype(np.float64)
            vf = v[b, kh].astype(np.float64)
            dof = do[b, h].astype(np.float64)
            y = scale * (qf @ kf.T)
            if soft_cap > 0:
                t = np.tanh(y / soft_cap)
                z = soft_cap * t
            else:
                z = y
            z_a = np.where(a, z, -np.inf)
            m = np.where(has, z_a.max(axis=1), 0.0)
            e = np.where(a, np.exp(z_a - m[:, None]), 0.0)
            l = np.where(has, e.sum(axis=1), 1.0)
            p = e / l[:, None]
            dv[b, kh] += p.T @ dof
            dp = dof @ vf.T
            D = (p * dp).sum(axis=1)
            dz = p * (dp - D[:, None])
            dy = dz * (1.0 - t * t) if soft_cap > 0 else dz
            dq[b, h] = scale * (dy @ kf)
            dk[b, kh] += scale * (dy.T @ qf)
    return dq, dk, dv
