"""The compute-friendly MLA formulation in NumPy fp64 (test infrastructure only).

vLLM API docs, vllm.model_executor.layers.attention.mla_attention, module
docstring, section "Compute Friendly Approach (i.e. forward_mha)": the latent
rows are up-projected per head, k_nope = kv_c @ W_UK and v = kv_c @ W_UV, and
ordinary multi-head attention runs with QK head width P + R and V head width V
(k_pe is shared by all heads).  Section "Data-Movement Friendly Approach (i.e.
forward_mqa)" absorbs W_UK into the query instead, ql_nope = q_nope . W_UK
(contracting P), attends over the latent rows with value kv_c, and applies
W_UV to the latent output afterwards.

The two are algebraically equal when both use the same softmax scale, which
makes the forward_mha path an independent check of the decode oracle: the
tests run this file's MHA, absorb the query with ``absorb_query``, run the
decode oracle on the latent cache and up-project with ``up_project``.
"""
from __future__ import annotations

import numpy as np


def mha_decode(q_nope, q_pe, kv_c, k_pe, W_UK, W_UV, softmax_scale):
    """Multi-head attention of one query token per head over Skv latent rows.

    q_nope [N, P], q_pe [N, R], kv_c [Skv, Lkv], k_pe [Skv, R],
    W_UK [Lkv, N, P], W_UV [Lkv, N, V].  Returns o [N, V] and lse [N].
    """
    Lkv, N, P = W_UK.shape
    V = W_UV.shape[2]
    Skv = kv_c.shape[0]
    k_nope = (kv_c @ W_UK.reshape(Lkv, N * P)).reshape(Skv, N, P)
    v = (kv_c @ W_UV.reshape(Lkv, N * V)).reshape(Skv, N, V)
    o = np.zeros((N, V))
    lse = np.empty(N)
    for n in range(N):
        # keys of head n: cat[k_nope[:, n], k_pe]; query cat[q_nope[n], q_pe[n]]
        scores = softmax_scale * (k_nope[:, n, :] @ q_nope[n] + k_pe @ q_pe[n])
        m = scores.max()
        w = np.exp(scores - m)
        z = w.sum()
        lse[n] = m + np.log(z)
        o[n] = (w / z) @ v[:, n, :]
    return o, lse


def absorb_query(q_nope, q_pe, W_UK):
    """ql_nope[n, l] = sum_p q_nope[n, p] * W_UK[l, n, p]; returns cat[ql_nope, q_pe]."""
    ql_nope = np.einsum("np,lnp->nl", q_nope, W_UK)
    return np.concatenate([ql_nope, q_pe], axis=-1)


def up_project(latent_out, W_UV):
    """o[n, v] = sum_l latent_out[n, l] * W_UV[l, n, v]."""
    return np.einsum("nl,lnv->nv", latent_out, W_UV)
