"""Checks that pin the CPU oracle to facts fixed outside itself.

Each ``pin_*`` takes the oracle module and raises AssertionError when the oracle disagrees with a
closed form, a library routine, an invariance, finite differences, or the brute-force loops.  The
same functions run against the real oracle (tests/test_oracle.py) and against deliberately broken
copies of it (tests/test_oracle_mutants.py), which shows that each plausible mistake is caught.

Sources of the facts:
  * definition softmax(scale·QKᵀ)·V — "Anatomy of a FlashAttention Kernel", section "Why is attention
    memory-bound, and how does FlashAttention fix it?";
  * exactness of the tiled online softmax — same page, section "What is online softmax and how does
    tiling keep it exact?";
  * statistics kept for the backward (max and denominator, folded into LSE) — same page, section "How
    does FlashAttention save memory in the backward pass?";
  * decoding against a key/value cache — glossary entry "flash attention" (paragraph on long-context
    training and serving) and "FlashAttention: where it matters", section "Where It Matters": the last
    Nq queries of a sequence against all its keys, checked against the square result's last rows;
  * merging chunk results — the online-softmax recurrence applied to whole key chunks ("Anatomy ...",
    section "What is online softmax and how does tiling keep it exact?"), checked in closed form and
    against attention over all keys;
  * everything else is mathematics: rows of a softmax sum to 1, equal scores give the mean, one key
    gives its value row, shifting all keys by u shifts every score of row i by scale·q_i·u, attention
    is linear in V, a joint key/value permutation is harmless without a mask, and the chain rule,
    checked with central differences.
"""

import math

import numpy as np
import scipy.special

RNG_SEED = 1234


def _rng(offset=0):
    return np.random.default_rng(RNG_SEED + offset)


def _qkv(n, d, offset=0, n_k=None):
    r = _rng(offset)
    n_k = n if n_k is None else n_k
    return r.standard_normal((n, d)), r.standard_normal((n_k, d)), r.standard_normal((n_k, d))


def pin_softmax_rows(orc):
    """Rows of P sum to 1, entries are ≥ 0, and masked (future) keys get exactly 0."""
    q, k, _ = _qkv(37, 8, 1)
    for causal in (False, True):
        s = orc.scores_head64(q, k, causal, 0.35)
        p, _, _ = orc.probabilities_head64(s)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-14
        assert np.all(p >= 0.0)
        if causal:
            assert np.all(p[np.triu_indices(37, k=1)] == 0.0)
            assert np.all(p[np.tril_indices(37)] > 0.0)


def pin_library_softmax(orc):
    """P and LSE equal scipy's softmax / logsumexp of the masked, scaled scores QKᵀ·scale."""
    q, k, v = _qkv(29, 6, 2)
    scale = 0.41
    for causal in (False, True):
        raw = scale * np.einsum("id,jd->ij", q, k)
        if causal:
            raw = np.where(np.tril(np.ones((29, 29), dtype=bool)), raw, -np.inf)
        p_ref = scipy.special.softmax(raw, axis=1)
        lse_ref = scipy.special.logsumexp(raw, axis=1)
        p, _, _ = orc.probabilities_head64(orc.scores_head64(q, k, causal, scale))
        assert np.max(np.abs(p - p_ref)) <= 1e-14
        o, lse = orc.attention_head_fwd64(q, k, v, causal, scale)
        assert np.max(np.abs(lse - lse_ref)) <= 1e-12
        o_ref = np.einsum("ij,jd->id", p_ref, v)
        assert np.max(np.abs(o - o_ref)) <= 1e-12


def pin_equal_scores(orc):
    """Q = 0 makes every allowed score equal: O_i is the mean of the allowed V rows and
    LSE_i = ln(number of allowed keys) — ln N without a mask, ln(i + 1) under the causal mask."""
    n, d = 23, 5
    _, k, v = _qkv(n, d, 3)
    q = np.zeros((n, d))
    o, lse = orc.attention_head_fwd64(q, k, v, False, 0.7)
    assert np.max(np.abs(o - v.mean(axis=0)[None, :])) <= 1e-13
    assert np.max(np.abs(lse - math.log(n))) <= 1e-13
    o, lse = orc.attention_head_fwd64(q, k, v, True, 0.7)
    means = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(o - means)) <= 1e-13
    assert np.max(np.abs(lse - np.log(np.arange(1, n + 1)))) <= 1e-13


def pin_single_key(orc):
    """N = 1: O = V_0 and LSE = scale·q·k.  Under the causal mask row 0 always has this form."""
    q, k, v = _qkv(1, 7, 4)
    for causal in (False, True):
        o, lse = orc.attention_head_fwd64(q, k, v, causal, 0.3)
        assert np.max(np.abs(o - v)) <= 1e-15
        assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) <= 1e-14
    q, k, v = _qkv(19, 7, 5)
    o, lse = orc.attention_head_fwd64(q, k, v, True, 0.3)
    assert np.max(np.abs(o[0] - v[0])) <= 1e-15
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) <= 1e-14


def pin_key_shift(orc):
    """Adding one vector u to every key adds scale·q_i·u to every score of row i: O is unchanged and
    LSE_i moves by exactly that amount."""
    q, k, v = _qkv(17, 4, 6)
    u = _rng(7).standard_normal(4) * 3.0
    for causal in (False, True):
        o1, l1 = orc.attention_head_fwd64(q, k, v, causal, 0.5)
        o2, l2 = orc.attention_head_fwd64(q, k + u[None, :], v, causal, 0.5)
        assert np.max(np.abs(o1 - o2)) <= 1e-12
        assert np.max(np.abs((l2 - l1) - 0.5 * (q @ u))) <= 1e-12


def pin_large_scores(orc):
    """Scores far beyond exp's range (|s| ~ 1e4) still give a finite softmax (max subtraction), equal
    to the result for the same scores shifted per row."""
    q, k, v = _qkv(11, 3, 8)
    q = q * 2000.0
    o, lse = orc.attention_head_fwd64(q, k, v, False, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    raw = q @ k.T
    o_ref = scipy.special.softmax(raw, axis=1) @ v
    assert np.max(np.abs(o - o_ref)) <= 1e-10


def pin_linear_in_v(orc):
    """O is linear in V."""
    q, k, v1 = _qkv(13, 4, 9)
    v2 = _rng(10).standard_normal(v1.shape)
    for causal in (False, True):
        o1, _ = orc.attention_head_fwd64(q, k, v1, causal, 0.6)
        o2, _ = orc.attention_head_fwd64(q, k, v2, causal, 0.6)
        o3, _ = orc.attention_head_fwd64(q, k, v1 - 2.5 * v2, causal, 0.6)
        assert np.max(np.abs(o3 - (o1 - 2.5 * o2))) <= 1e-12


def pin_joint_permutation(orc):
    """Without a mask, permuting keys and values together leaves O and LSE unchanged and permutes the
    rows of dK and dV the same way (dQ unchanged)."""
    q, k, v = _qkv(15, 4, 11)
    do = _rng(12).standard_normal(q.shape)
    perm = _rng(13).permutation(15)
    o1, l1 = orc.attention_head_fwd64(q, k, v, False, 0.45)
    o2, l2 = orc.attention_head_fwd64(q, k[perm], v[perm], False, 0.45)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12
    dq1, dk1, dv1 = orc.attention_head_bwd64(q, k, v, do, False, 0.45)
    dq2, dk2, dv2 = orc.attention_head_bwd64(q, k[perm], v[perm], do, False, 0.45)
    assert np.max(np.abs(dq1 - dq2)) <= 1e-12
    assert np.max(np.abs(dk1[perm] - dk2)) <= 1e-12
    assert np.max(np.abs(dv1[perm] - dv2)) <= 1e-12


def pin_online_recurrence(orc):
    """The tiled online-softmax recurrence equals the dense result for any tile sizes (fp64)."""
    q, k, v = _qkv(29, 6, 14)
    for causal in (False, True):
        o_ref, l_ref = orc.attention_head_fwd64(q, k, v, causal, 0.4)
        for tr in (1, 4, 29):
            for tc in (1, 2, 3, 7, 29):
                o, lse = orc.online_attention_head64(q, k, v, causal, 0.4, tr, tc)
                assert np.max(np.abs(o - o_ref)) <= 1e-12
                assert np.max(np.abs(lse - l_ref)) <= 1e-12


def pin_online_rising_max(orc):
    """Keys whose scores grow tile after tile force a rescale at every tile; the recurrence must still
    equal the dense result."""
    n, d = 24, 3
    q = np.ones((n, d))
    k = np.outer(np.arange(n, dtype=np.float64), np.ones(d)) * 0.5
    v = _rng(15).standard_normal((n, d))
    for causal in (False, True):
        o_ref, l_ref = orc.attention_head_fwd64(q, k, v, causal, 1.0)
        o, lse = orc.online_attention_head64(q, k, v, causal, 1.0, 5, 4)
        assert np.max(np.abs(o - o_ref)) <= 1e-12
        assert np.max(np.abs(lse - l_ref)) <= 1e-12


def _fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        xp = x.copy()
        xm = x.copy()
        xp[idx] += h
        xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


def pin_finite_differences(orc):
    """dQ, dK, dV equal central finite differences of f = Σ(O ∘ dO) (fp64, relative error ≤ 1e-7)."""
    for n in (1, 3, 5):
        for d in (2, 4):
            q, k, v = _qkv(n, d, 16 + n + d)
            do = _rng(17 + n * d).standard_normal((n, d))
            for causal in (False, True):
                scale = 0.8

                def f(qq, kk, vv):
                    return float(np.sum(orc.attention_head_fwd64(qq, kk, vv, causal, scale)[0] * do))

                dq, dk, dv = orc.attention_head_bwd64(q, k, v, do, causal, scale)
                for got, ref in ((dq, _fd_grad(lambda x: f(x, k, v), q)),
                                 (dk, _fd_grad(lambda x: f(q, x, v), k)),
                                 (dv, _fd_grad(lambda x: f(q, k, x), v))):
                    denom = max(np.linalg.norm(ref), 1e-3)
                    assert np.linalg.norm(got - ref) / denom <= 1e-7, (n, d, causal)


def pin_backward_identities(orc):
    """Σ_k P_ik dP_ik = dO_i · O_i; Σ_j dV_j = Σ_i dO_i (rows of P sum to 1); Σ_j dK_j = 0 (rows of
    dS sum to 0)."""
    q, k, v = _qkv(21, 5, 18)
    do = _rng(19).standard_normal(q.shape)
    for causal in (False, True):
        p, _, _ = orc.probabilities_head64(orc.scores_head64(q, k, causal, 0.5))
        o, _ = orc.attention_head_fwd64(q, k, v, causal, 0.5)
        dp = do @ v.T
        assert np.max(np.abs(np.sum(p * dp, axis=1) - np.sum(do * o, axis=1))) <= 1e-12
        dq, dk, dv = orc.attention_head_bwd64(q, k, v, do, causal, 0.5)
        assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) <= 1e-12
        assert np.max(np.abs(dk.sum(axis=0))) <= 1e-12


def pin_brute_force(orc):
    """The numpy functions equal the pure-Python loops on tiny inputs (≤ 1e-13)."""
    for n, d in ((1, 1), (3, 2), (5, 4), (8, 8)):
        q, k, v = _qkv(n, d, 20 + n)
        do = _rng(21 + n).standard_normal((n, d))
        for causal in (False, True):
            o, lse = orc.attention_head_fwd64(q, k, v, causal, 0.6)
            ob, lb = orc.brute_attention_head(q.tolist(), k.tolist(), v.tolist(), causal, 0.6)
            assert np.max(np.abs(o - np.array(ob))) <= 1e-13
            assert np.max(np.abs(lse - np.array(lb))) <= 1e-13
            g = orc.attention_head_bwd64(q, k, v, do, causal, 0.6)
            gb = orc.brute_attention_head_bwd(q.tolist(), k.tolist(), v.tolist(), do.tolist(),
                                              causal, 0.6)
            for a, b in zip(g, gb):
                assert np.max(np.abs(a - np.array(b))) <= 1e-13


def pin_batched_and_rows(orc):
    """The [B,H,N,d] drivers apply the per-head functions head by head, and the single-row functions
    agree with the full forward and with the rows of the full backward's dQ."""
    r = _rng(22)
    q, k, v, do = (r.standard_normal((2, 3, 9, 4)) for _ in range(4))
    for causal in (False, True):
        o, lse = orc.attention_fwd64(q, k, v, causal, 0.5)
        dq, dk, dv = orc.attention_bwd64(q, k, v, do, causal, 0.5)
        for b in range(2):
            for h in range(3):
                oh, lh = orc.attention_head_fwd64(q[b, h], k[b, h], v[b, h], causal, 0.5)
                assert np.array_equal(oh, o[b, h]) and np.array_equal(lh, lse[b, h])
                gh = orc.attention_head_bwd64(q[b, h], k[b, h], v[b, h], do[b, h], causal, 0.5)
                assert np.array_equal(gh[0], dq[b, h]) and np.array_equal(gh[1], dk[b, h])
                assert np.array_equal(gh[2], dv[b, h])
                rows = [0, 4, 8]
                orow, lrow = orc.attention_rows64(q[b, h], k[b, h], v[b, h], rows, causal, 0.5)
                assert np.max(np.abs(orow - oh[rows])) <= 1e-13
                assert np.max(np.abs(lrow - lh[rows])) <= 1e-13
                dqrow = orc.attention_rows_dq64(q[b, h], k[b, h], v[b, h], do[b, h], rows, causal,
                                                0.5)
                assert np.max(np.abs(dqrow - gh[0][rows])) <= 1e-13


def pin_decode_rows_of_full(orc):
    """Decoding the last Nq queries of a sequence against all its keys (query offset Nk − Nq) gives
    exactly the last Nq rows of the square attention over the whole sequence, causal or not."""
    for n, n_q, d in ((9, 1, 4), (13, 4, 3), (20, 7, 8), (6, 6, 2)):
        q, k, v = _qkv(n, d, 40 + n)
        for causal in (False, True):
            o, lse = orc.attention_head_fwd64(q, k, v, causal, 0.45)
            od, ld = orc.attention_head_fwd64(q[n - n_q:], k, v, causal, 0.45, q_offset=n - n_q)
            assert np.max(np.abs(od - o[n - n_q:])) <= 1e-13
            assert np.max(np.abs(ld - lse[n - n_q:])) <= 1e-13


def pin_decode_single_query(orc):
    """One query at the end of the sequence sees every key: the causal decode result equals the
    library softmax over all keys (scipy), and equals the non-causal result."""
    q, k, v = _qkv(1, 6, 50, n_k=17)
    s = 0.7 * (k @ q[0])
    p = scipy.special.softmax(s)
    o, lse = orc.attention_head_fwd64(q, k, v, True, 0.7, q_offset=16)
    assert np.max(np.abs(o[0] - p @ v)) <= 1e-13
    assert abs(lse[0] - scipy.special.logsumexp(s)) <= 1e-13
    o2, lse2 = orc.attention_head_fwd64(q, k, v, False, 0.7)
    assert np.max(np.abs(o - o2)) <= 1e-14 and np.max(np.abs(lse - lse2)) <= 1e-14


def pin_decode_brute(orc):
    """With a query offset the numpy forward equals the pure-Python loops (rectangular, causal)."""
    for n_q, n_k, d in ((1, 5, 2), (3, 7, 3), (4, 4, 2), (2, 9, 4)):
        r = _rng(60 + n_k)
        q, k, v = r.standard_normal((n_q, d)), r.standard_normal((n_k, d)), r.standard_normal((n_k, d))
        for off in sorted({n_k - n_q, 0, 1}):
            o, lse = orc.attention_head_fwd64(q, k, v, True, 0.8, q_offset=off)
            ob, lb = orc.brute_attention_head(q.tolist(), k.tolist(), v.tolist(), True, 0.8, off)
            assert np.max(np.abs(o - np.array(ob))) <= 1e-13
            assert np.max(np.abs(lse - np.array(lb))) <= 1e-13


def pin_merge_closed_form(orc):
    """Merging chunk results by their softmax mass: chunks with LSE ln 1 and ln 3 and outputs e_0 and
    e_1 give LSE ln 4 and O = (1/4, 3/4); a chunk with no usable key (LSE −inf) changes nothing."""
    o, lse = orc.merge_partials64([(np.array([[1.0, 0.0]]), np.array([0.0])),
                                   (np.array([[0.0, 1.0]]), np.array([math.log(3.0)]))])
    assert np.max(np.abs(o - np.array([[0.25, 0.75]]))) <= 1e-15
    assert abs(lse[0] - math.log(4.0)) <= 1e-15
    o2, lse2 = orc.merge_partials64([(np.array([[0.3, -2.0]]), np.array([1.5])),
                                     (np.array([[7.0, 7.0]]), np.array([-np.inf]))])
    assert np.array_equal(o2, np.array([[0.3, -2.0]])) and lse2[0] == 1.5


def pin_split_merge(orc):
    """Attending to key chunks separately and merging the chunk results equals attending to all keys
    at once, for any chunking, with and without the causal mask and a query offset (chunks that are
    fully masked for some rows included)."""
    r = _rng(70)
    n_q, n_k, d = 5, 23, 4
    q, k, v = r.standard_normal((n_q, d)), r.standard_normal((n_k, d)), r.standard_normal((n_k, d))
    for bounds in ([0, 23], [0, 1, 23], [0, 8, 16, 23], [0, 5, 6, 7, 20, 22, 23]):
        for causal, off in ((False, 0), (True, 18), (True, 3), (True, 0)):
            o, lse = orc.attention_head_fwd64(q, k, v, causal, 0.55, q_offset=off)
            os_, ls_ = orc.split_attention_head64(q, k, v, causal, 0.55, bounds, q_offset=off)
            assert np.max(np.abs(os_ - o)) <= 1e-13, (bounds, causal, off)
            assert np.max(np.abs(ls_ - lse)) <= 1e-13, (bounds, causal, off)


ALL_PINS = [
    pin_softmax_rows,
    pin_library_softmax,
    pin_equal_scores,
    pin_single_key,
    pin_key_shift,
    pin_large_scores,
    pin_linear_in_v,
    pin_joint_permutation,
    pin_online_recurrence,
    pin_online_rising_max,
    pin_finite_differences,
    pin_backward_identities,
    pin_brute_force,
    pin_batched_and_rows,
    pin_decode_rows_of_full,
    pin_decode_single_query,
    pin_decode_brute,
    pin_merge_closed_form,
    pin_split_merge,
]
