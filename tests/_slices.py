"""Oracle outputs of a slice of chunk rows, for parity checks at sizes where the full
oracle is out of reach (test infrastructure; calls only oracle/).

Chunk row i of a (window, KV head) attends to the cache rows and to chunk keys 0..i.
So rows [a, a + n) are exactly the whole chunk of a call whose cache is
[cache ; chunk keys 0..a-1] and whose chunk is keys / rows a..a+n-1: that call gives
their O, LSE and dQ. The chunk dK/dV of that call counts the contributions of rows
>= a only, which is all of them for keys [a, C) when a + n == C.
"""
import numpy as np

import oracle


def chunk_slice(q, kc, vc, kp, vp, do, scale, a, n):
    """One group: q, do [G][C][D]; kc, vc [C][D]; kp, vp [P][D] (fp64).

    Returns O, LSE, dQ of chunk rows [a, a + n) ([G][n][D], [G][n], [G][n][D]) and
    dKc, dVc [n][D] of chunk keys [a, a + n) from rows >= a.
    """
    kp2 = np.concatenate([kp, kc[:a]])
    vp2 = np.concatenate([vp, vc[:a]])
    qs, dos = q[:, a:a + n], do[:, a:a + n]
    kcs, vcs = kc[a:a + n], vc[a:a + n]
    o, lse = oracle.group_fwd(qs, kcs, vcs, kp2, vp2, scale)
    dq, dk, dv, _ = oracle.group_bwd(qs, kcs, vcs, kp2, vp2, scale, dos)
    return o, lse, dq, dk, dv
