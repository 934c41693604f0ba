"""Dual-timescale query summaries, float64.

GrowPage Eq. 6: qbar^x_t = beta_x qbar^x_{t-1} + (1 - beta_x) q_t for x in {S, L}, with
beta_S < beta_L, kept per request, layer and query head in the pre-RoPE space. GrowPage
App. E.1: the state lives in a pre-allocated pool [M, 2, H_q, d] (index 0 short, 1 long)
addressed by the request's slot id; on the first decoding step of a newly bound slot both
summaries are set to q_t, overwriting whatever the slot held.

Pinned by: the closed form beta^(n-1) q_1 + (1 - beta) sum_{k>=2} beta^(n-k) q_k; beta_S = 0
reduces the short summary to the current query (GrowPage Sec. 5.3, Table 2 discussion); a
fresh slot ignores stale contents; a hand-computed sequence (tests/golden/ema_sequence.txt).
"""
import numpy as np


def update_query_summaries(q, slot_ids, fresh, qstate, beta_s, beta_l):
    """Apply one decoding step to the state pool in place (float64 array [M, 2, H_q, d])."""
    q = np.asarray(q, dtype=np.float64)
    for r in range(q.shape[0]):
        s = int(slot_ids[r])
        if fresh[r]:
            qstate[s, 0] = q[r]
            qstate[s, 1] = q[r]
        else:
            qstate[s, 0] = beta_s * qstate[s, 0] + (1.0 - beta_s) * q[r]
            qstate[s, 1] = beta_l * qstate[s, 1] + (1.0 - beta_l) * q[r]
    return qstate
