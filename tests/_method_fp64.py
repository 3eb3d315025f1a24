"""fp64 re-statements of the method's algebra, used only to pin the oracle.

These are independent of ``oracle/`` (they do not import it) and of the GPU
library.  They restate, in plain NumPy, the steps the pages give for the fused
method so that tests can check "online = two-pass" and the associativity of
the ⊕ merge:

* ``merge_ml`` / ``merge_mlo``: the ⊕ merge of two summaries (m, ℓ) or
  (m, ℓ, o) ([15-779 L5] §4.4–4.5): the merged max is the larger max, and
  each side's sum (and unnormalised output) is rebased by exp(its max − the
  merged max) before adding.
* ``blocked_forward``: FA-2 loop order ([15-779 L5] §5.1; [cicada] §3.2.1–
  3.2.3): outer loop over query blocks, inner loop over key/value blocks with
  the running (m, ℓ, acc) update, one division by ℓ at the end and
  L = m + ln ℓ.  Fully masked causal tiles are skipped ([15-779 L5] §6.2).
"""

import numpy as np


def summary(s, v=None):
    """(m, ℓ[, o]) of one block of logits s (1-D) and its values v ([n, d])."""
    m = s.max()
    e = np.exp(s - m)
    if v is None:
        return (m, e.sum())
    return (m, e.sum(), e @ v)


def merge_ml(a, b):
    m = max(a[0], b[0])
    return (m, a[1] * np.exp(a[0] - m) + b[1] * np.exp(b[0] - m))


def merge_mlo(a, b):
    m = max(a[0], b[0])
    fa = np.exp(a[0] - m)
    fb = np.exp(b[0] - m)
    return (m, a[1] * fa + b[1] * fb, a[2] * fa + b[2] * fb)


def blocked_forward(q, k, v, scale, causal, br, bc):
    """FA-2 forward for one head in fp64.  q, k, v: [N, d] float64."""
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i0 in range(0, n, br):
        i1 = min(i0 + br, n)
        qi = q[i0:i1]
        rows = np.arange(i0, i1)
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        acc = np.zeros((i1 - i0, v.shape[1]))
        j_end = min(n, i1) if causal else n           # tiles past the block's last query are skipped
        for j0 in range(0, j_end, bc):
            j1 = min(j0 + bc, n)
            s = scale * (qi @ k[j0:j1].T)
            if causal:
                s = np.where(np.arange(j0, j1)[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            p = np.exp(s - m_new[:, None])
            alpha = np.exp(m - m_new)
            l = l * alpha + p.sum(axis=1)
            acc = acc * alpha[:, None] + p @ v[j0:j1]
            m = m_new
        o[i0:i1] = acc / l[:, None]
        lse[i0:i1] = m + np.log(l)
    return o, lse


def count_rescales(x):
    """Number of times the running max changes after the first element ([15-779 L5] §4.3)."""
    cnt = 0
    m = x[0]
    for t in x[1:]:
        if t > m:
            m = t
            cnt += 1
    return cnt
