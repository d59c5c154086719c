"""CPU fp64 oracle for exact attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this module; only the
test suite, the smoke check of ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP path and imports nothing from the product package.

What it computes, and where the pages define it:

* The result of attention is ``softmax(Q Kᵀ / √d) · V`` with the softmax taken along each query's row
  of scores ("Anatomy of a FlashAttention Kernel", section "Why is attention memory-bound, and how does
  FlashAttention fix it?").  The scale is a parameter here; the workloads pass 1/√d.
* The tiled method reaches that result exactly ("flash attention" glossary entry, table row "Result";
  "FlashAttention: where it matters", section "The Real Complexity", last bullet).  So the oracle is the
  plain definition written out: it materialises the full N×N score matrix S and probability matrix P per
  (batch, head), in fp64, which is precisely what the GPU path avoids.
* The forward keeps the per-row softmax statistics for the backward ("Anatomy ...", section "How does
  FlashAttention save memory in the backward pass?": maximum and denominator).  They are exported folded
  into one number per row, the natural-log logsumexp LSE_i = m_i + ln l_i of the scaled scores.
* The backward is the chain rule of O = softmax(S)·V written out term by term (no shortcut through O).
* ``online_attention64`` follows the online-softmax recurrence of "Anatomy ...", section "What is online
  softmax and how does tiling keep it exact?": a running maximum m and denominator l per query row, and a
  rescale of the accumulated denominator and output by exp(m_old − m_new) whenever a new tile raises m.
* Causal masking (key j may be used by query i only when j ≤ i) is not on the pages; it is the plain
  reading used for the causal workloads.
* Decoding against a key/value cache (the inference use the pages pair FlashAttention with: glossary
  entry "flash attention", paragraph on long-context training and serving; "FlashAttention: where it
  matters", section "Where It Matters", long-context inference and speculative decoding): a few new
  queries attend over Nk cached keys.  The queries are the last Nq positions of the sequence, so with
  the causal mask query i (0-based) sits at position q_offset + i with q_offset = Nk − Nq and may use
  key j when j ≤ q_offset + i.  ``q_offset`` is a parameter of the score functions (0 reproduces the
  square case).
* Splitting the keys into chunks, attending to each chunk on its own and combining the per-chunk
  results is the online-softmax recurrence applied to whole chunks: per row, with partial results
  (O_s, LSE_s), LSE = log Σ_s exp(LSE_s) and O = Σ_s exp(LSE_s − LSE) · O_s (``merge_partials64``).

Layout: every tensor argument is a numpy array [B, H, N, d] (LSE: [B, H, N]); arithmetic is float64.
Per-head ("_head") functions take 2-D [N, d] arrays.
"""

import math

import numpy as np

__all__ = [
    "scores_head64",
    "probabilities_head64",
    "attention_head_fwd64",
    "attention_head_bwd64",
    "attention_fwd64",
    "attention_bwd64",
    "attention_rows64",
    "attention_rows_dq64",
    "online_attention_head64",
    "brute_attention_head",
    "brute_attention_head_bwd",
    "merge_partials64",
    "split_attention_head64",
]


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def scores_head64(q, k, causal, scale, q_offset=0):
    """Scaled scores S = scale · Q Kᵀ for one head, with masked entries set to −inf.

    Masking: causal keeps key j for query i only when j ≤ q_offset + i, query i being at position
    q_offset + i of the key sequence (0 for the square case, Nk − Nq for decoding).
    """
    q = _as64(q)
    k = _as64(k)
    s = scale * (q @ k.T)
    if causal:
        n_q, n_k = s.shape
        i = np.arange(n_q)[:, None]
        j = np.arange(n_k)[None, :]
        s = np.where(j > q_offset + i, -np.inf, s)
    return s


def probabilities_head64(s):
    """Row softmax of a score matrix: returns P, the row maxima m and the row denominators l.

    m_i = max_j S_ij, E = exp(S − m), l_i = Σ_j E_ij, P = E / l.  Entries at −inf give exactly 0.
    """
    m = np.max(s, axis=1)
    e = np.exp(s - m[:, None])
    l = np.sum(e, axis=1)
    p = e / l[:, None]
    return p, m, l


def attention_head_fwd64(q, k, v, causal, scale, q_offset=0):
    """Forward for one head: O = P V and LSE_i = m_i + ln l_i (natural log, of the scaled scores).

    ``q_offset``: position of query 0 in the key sequence for the causal mask (see scores_head64).
    """
    s = scores_head64(q, k, causal, scale, q_offset)
    p, m, l = probabilities_head64(s)
    o = p @ _as64(v)
    lse = m + np.log(l)
    return o, lse


def attention_head_bwd64(q, k, v, do, causal, scale):
    """Backward for one head by the explicit chain rule of O = softmax(scale · Q Kᵀ) · V.

    With P from the forward definition and upstream gradient dO:
      dV = Pᵀ dO
      dP = dO Vᵀ
      dS_ij = P_ij · (dP_ij − Σ_k P_ik dP_ik)        (Jacobian of the row softmax)
      dQ = scale · dS K,   dK = scale · dSᵀ Q        (S = scale · Q Kᵀ)
    Returns (dq, dk, dv).
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    do = _as64(do)
    s = scores_head64(q, k, causal, scale)
    p, _, _ = probabilities_head64(s)
    dv = p.T @ do
    dp = do @ v.T
    row_dot = np.sum(p * dp, axis=1)
    ds = p * (dp - row_dot[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_fwd64(q, k, v, causal, scale):
    """Forward over [B, H, N, d] arrays, one head at a time.  Returns (o [B,H,N,d], lse [B,H,N])."""
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    b_, h_, n, d = q.shape
    o = np.empty((b_, h_, n, v.shape[-1]), dtype=np.float64)
    lse = np.empty((b_, h_, n), dtype=np.float64)
    for b in range(b_):
        for h in range(h_):
            o[b, h], lse[b, h] = attention_head_fwd64(q[b, h], k[b, h], v[b, h], causal, scale)
    return o, lse


def attention_bwd64(q, k, v, do, causal, scale):
    """Backward over [B, H, N, d] arrays, one head at a time.  Returns (dq, dk, dv)."""
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    do = _as64(do)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    b_, h_ = q.shape[:2]
    for b in range(b_):
        for h in range(h_):
            dq[b, h], dk[b, h], dv[b, h] = attention_head_bwd64(
                q[b, h], k[b, h], v[b, h], do[b, h], causal, scale)
    return dq, dk, dv


def attention_rows64(q, k, v, rows, causal, scale):
    """Forward outputs for selected query rows of one head, each computed on its own.

    For query i: s_j = scale · q_i·k_j over the allowed keys (all keys, or j ≤ i when causal),
    o_i = Σ_j softmax(s)_j v_j, lse_i = logsumexp(s).  Cost O(N·d) per row, for sampled checks of
    long sequences.  Returns (o [len(rows), d], lse [len(rows)]).
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    rows = list(rows)
    o = np.empty((len(rows), v.shape[1]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for r, i in enumerate(rows):
        end = i + 1 if causal else k.shape[0]
        s = scale * (k[:end] @ q[i])
        m = np.max(s)
        e = np.exp(s - m)
        l = np.sum(e)
        o[r] = (e / l) @ v[:end]
        lse[r] = m + np.log(l)
    return o, lse


def attention_rows_dq64(q, k, v, do, rows, causal, scale):
    """dQ for selected query rows of one head, each computed on its own.

    Row i of dQ depends only on row i of P and of dP, so the chain rule of attention_head_bwd64
    restricted to one row reads: over the allowed keys (all, or j ≤ i when causal),
    p = softmax(scale · k_j·q_i), dp_j = dO_i·v_j, ds_j = p_j (dp_j − Σ_k p_k dp_k),
    dq_i = scale · Σ_j ds_j k_j.  Cost O(N·d) per row, for sampled checks of long sequences.
    Returns dq [len(rows), d].
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    do = _as64(do)
    rows = list(rows)
    dq = np.empty((len(rows), k.shape[1]), dtype=np.float64)
    for r, i in enumerate(rows):
        end = i + 1 if causal else k.shape[0]
        s = scale * (k[:end] @ q[i])
        e = np.exp(s - np.max(s))
        p = e / np.sum(e)
        dp = v[:end] @ do[i]
        ds = p * (dp - np.sum(p * dp))
        dq[r] = scale * (ds @ k[:end])
    return dq


def online_attention_head64(q, k, v, causal, scale, tile_r, tile_c):
    """Tiled forward for one head by the online-softmax recurrence, in fp64.

    Queries are taken tile_r rows at a time and keys tile_c at a time, in key order.  Per query row the
    state is (m, l, acc): m the largest scaled score seen so far, l the running sum of exp(s − m), acc the
    running Σ exp(s − m) v.  For each key tile with scores s (masked entries −inf):
      m_new = max(m_old, max_j s_j)
      l     = exp(m_old − m_new) · l + Σ_j exp(s_j − m_new)
      acc   = exp(m_old − m_new) · acc + Σ_j exp(s_j − m_new) v_j
    and after the last tile O = acc / l, LSE = m + ln l.  A key tile whose entries are all masked for a row
    leaves that row's state unchanged.
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    n_q, n_k, d_v = q.shape[0], k.shape[0], v.shape[1]
    o = np.empty((n_q, d_v), dtype=np.float64)
    lse = np.empty(n_q, dtype=np.float64)
    for r0 in range(0, n_q, tile_r):
        r1 = min(r0 + tile_r, n_q)
        qi = q[r0:r1]
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, d_v))
        for c0 in range(0, n_k, tile_c):
            c1 = min(c0 + tile_c, n_k)
            s = scale * (qi @ k[c0:c1].T)
            if causal:
                i = np.arange(r0, r1)[:, None]
                j = np.arange(c0, c1)[None, :]
                s = np.where(j > i, -np.inf, s)
            m_new = np.maximum(m, np.max(s, axis=1))
            live = np.isfinite(m_new)
            # rows with nothing allowed so far keep m = -inf, l = 0, acc = 0
            alpha = np.where(live, np.exp(np.where(live, m - m_new, 0.0)), 1.0)
            alpha = np.where(np.isfinite(m), alpha, 0.0)
            p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
            l = alpha * l + np.sum(p, axis=1)
            acc = alpha[:, None] * acc + p @ v[c0:c1]
            m = m_new
        o[r0:r1] = acc / l[:, None]
        lse[r0:r1] = m + np.log(l)
    return o, lse


def brute_attention_head(q, k, v, causal, scale, q_offset=0):
    """Forward for one head with plain Python loops and the math module (tiny inputs only).

    Written independently of the numpy functions above, entry by entry from the definition; with the
    causal mask query i may use key j when j ≤ q_offset + i.  Returns (o, lse) as nested lists.
    """
    n_q, n_k = len(q), len(k)
    d = len(q[0])
    d_v = len(v[0])
    o = []
    lse = []
    for i in range(n_q):
        allowed = [j for j in range(n_k) if (not causal) or j <= q_offset + i]
        s = {}
        for j in allowed:
            acc = 0.0
            for t in range(d):
                acc += float(q[i][t]) * float(k[j][t])
            s[j] = scale * acc
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in allowed}
        den = sum(w.values())
        row = []
        for t in range(d_v):
            row.append(sum(w[j] * float(v[j][t]) for j in allowed) / den)
        o.append(row)
        lse.append(mx + math.log(den))
    return o, lse


def brute_attention_head_bwd(q, k, v, do, causal, scale):
    """Backward for one head with plain Python loops (tiny inputs only).

    Entry by entry: P from the definition; dV_jt = Σ_i P_ij dO_it; dP_ij = Σ_t dO_it V_jt;
    dS_ij = P_ij (dP_ij − Σ_k P_ik dP_ik); dQ_it = scale Σ_j dS_ij K_jt; dK_jt = scale Σ_i dS_ij Q_it.
    Returns (dq, dk, dv) as nested lists.
    """
    n_q, n_k = len(q), len(k)
    d = len(q[0])
    d_v = len(v[0])
    p = [[0.0] * n_k for _ in range(n_q)]
    for i in range(n_q):
        allowed = [j for j in range(n_k) if (not causal) or j <= i]
        s = {j: scale * sum(float(q[i][t]) * float(k[j][t]) for t in range(d)) for j in allowed}
        mx = max(s.values())
        den = sum(math.exp(s[j] - mx) for j in allowed)
        for j in allowed:
            p[i][j] = math.exp(s[j] - mx) / den
    dv = [[sum(p[i][j] * float(do[i][t]) for i in range(n_q)) for t in range(d_v)] for j in range(n_k)]
    dp = [[sum(float(do[i][t]) * float(v[j][t]) for t in range(d_v)) for j in range(n_k)]
          for i in range(n_q)]
    ds = [[0.0] * n_k for _ in range(n_q)]
    for i in range(n_q):
        rd = sum(p[i][j] * dp[i][j] for j in range(n_k))
        for j in range(n_k):
            ds[i][j] = p[i][j] * (dp[i][j] - rd)
    dq = [[scale * sum(ds[i][j] * float(k[j][t]) for j in range(n_k)) for t in range(d)]
          for i in range(n_q)]
    dk = [[scale * sum(ds[i][j] * float(q[i][t]) for i in range(n_q)) for t in range(d)]
          for j in range(n_k)]
    return dq, dk, dv


def merge_partials64(parts):
    """Combine per-chunk attention results of the same query rows into the result over all chunks.

    ``parts``: list of (O_s [Nq, d], LSE_s [Nq]) where chunk s attended to its own keys only (a row with
    no usable key in a chunk has LSE_s = −inf and any finite O_s).  With M = max_s LSE_s,
      LSE = M + ln Σ_s exp(LSE_s − M),   O = Σ_s exp(LSE_s − LSE) · O_s,
    i.e. each chunk's output weighted by its share of the row's total softmax mass.
    """
    lses = np.stack([_as64(l) for _, l in parts])          # [S, Nq]
    outs = np.stack([_as64(o) for o, _ in parts])          # [S, Nq, d]
    mx = np.max(lses, axis=0)
    w = np.exp(lses - mx[None, :])                          # exp(−inf) = 0 drops empty chunks
    tot = np.sum(w, axis=0)
    lse = mx + np.log(tot)
    outs = np.where(np.isfinite(lses)[:, :, None], outs, 0.0)
    o = np.sum((w / tot[None, :])[:, :, None] * outs, axis=0)
    return o, lse


def split_attention_head64(q, k, v, causal, scale, bounds, q_offset=0):
    """Forward for one head with the keys split at ``bounds`` (0 = b_0 < b_1 < … < b_S = Nk): each chunk
    [b_s, b_{s+1}) is attended to on its own (plain definition, mask positions shifted by the chunk
    start), then the chunks are merged with merge_partials64.  Rows with no usable key in a chunk get
    LSE_s = −inf there.  Returns (o, lse).
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    parts = []
    for b0, b1 in zip(bounds[:-1], bounds[1:]):
        s = scores_head64(q, k[b0:b1], causal, scale, q_offset - b0)
        m = np.max(s, axis=1)
        live = np.isfinite(m)
        e = np.where(live[:, None], np.exp(s - np.where(live, m, 0.0)[:, None]), 0.0)
        l = np.sum(e, axis=1)
        o = np.where(live[:, None], (e @ v[b0:b1]) / np.where(live, l, 1.0)[:, None], 0.0)
        lse = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
        parts.append((o, lse))
    return merge_partials64(parts)
