"""Pins that tie the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an oracle module (the real one, or a copy with
a planted mistake) and raises AssertionError when the oracle disagrees with
the fact it checks.  The facts are closed forms and invariants of softmax
attention, finite differences of the oracle's own forward, an independent
pure-Python brute force, and PyTorch's float64 CPU attention with autograd.
"""

from __future__ import annotations

import math

import numpy as np

from brute_attention import brute_backward, brute_forward


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if not a.size:
        return
    # Infinities must match exactly; a NaN anywhere (e.g. -inf - -inf from a
    # row that lost every key) is a failure, not a warning.
    same_inf = np.isinf(a) & (a == b)
    with np.errstate(invalid="ignore"):
        diff = np.where(same_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)), f"{what}: non-finite mismatch"
    err = float(np.max(diff))
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# forward closed forms
# --------------------------------------------------------------------------

def pin_constant_v(orc):
    """Every V row equal to c gives O_i = c (softmax weights sum to one)."""
    rng = np.random.default_rng(11)
    B, N, H, d = 2, 19, 3, 8
    q, k = _rand(rng, B, N, H, d), _rand(rng, B, N, H, d)
    c = _rand(rng, d)
    v = np.broadcast_to(c, (B, N, H, d)).copy()
    for causal in (False, True):
        o, _ = orc.attention_forward(q, k, v, 0.7, causal)
        _close(o, v, 1e-13, f"constant V causal={causal}")


def pin_uniform_scores(orc):
    """Q = 0 (or scale = 0): equal scores give the mean of the visible V rows.

    Non-causal: O_i = mean_j V_j and LSE_i = ln N.  Causal: O_i = mean of
    V_0..V_i and LSE_i = ln(i + 1).
    """
    rng = np.random.default_rng(12)
    B, N, H, d = 1, 128, 1, 64
    k, v = _rand(rng, B, N, H, d), _rand(rng, B, N, H, d)
    q = _rand(rng, B, N, H, d)
    for qq, scale in ((np.zeros_like(q), 0.125), (q, 0.0)):
        o, lse = orc.attention_forward(qq, k, v, scale, False)
        _close(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), 1e-13, "mean V")
        _close(lse, np.full((B, H, N), math.log(N)), 1e-13, "LSE = ln N")
        assert abs(math.log(128) - 4.852030263919617) < 1e-15
        o, lse = orc.attention_forward(qq, k, v, scale, True)
        run_mean = np.cumsum(v, axis=1) / np.arange(1, N + 1)[None, :, None, None]
        _close(o, run_mean, 1e-13, "causal running mean of V")
        _close(lse[0, 0], np.log(np.arange(1, N + 1)), 1e-13, "causal LSE = ln(i+1)")


def pin_causal_first_row(orc):
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(13)
    B, N, H, d = 2, 33, 2, 16
    q, k, v = (_rand(rng, B, N, H, d) for _ in range(3))
    scale = 0.3
    o, lse = orc.attention_forward(q, k, v, scale, True)
    _close(o[:, 0], v[:, 0], 1e-14, "causal O_0 = V_0")
    want = scale * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])
    _close(lse[:, :, 0], want, 1e-13, "causal LSE_0")


def pin_single_key(orc):
    """N = 1: O = V and LSE = scale * q . k."""
    rng = np.random.default_rng(14)
    q, k, v = (_rand(rng, 3, 1, 2, 8) for _ in range(3))
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 0.5, causal)
        _close(o, v, 1e-15, "N=1 O=V")
        _close(lse, 0.5 * np.einsum("bnhd,bnhd->bhn", q, k), 1e-14, "N=1 LSE")


def pin_dominant_key(orc):
    """q_i = alpha * k_j with large alpha and orthogonal other keys -> O_i = V_j."""
    d, N = 16, 16
    k = np.eye(N, d)[None, :, None, :] * 1.0       # orthonormal keys
    rng = np.random.default_rng(15)
    v = _rand(rng, 1, N, 1, d)
    perm = rng.permutation(N)
    q = 60.0 * k[:, perm]                           # query i points at key perm[i]
    o, lse = orc.attention_forward(q, k, v, 1.0, False)
    # weight of the other keys is (N-1) e^{-60} ~ 1.3e-25
    _close(o, v[:, perm], 1e-15, "dominant key")
    _close(lse, np.full((1, 1, N), 60.0), 1e-13, "dominant key LSE")


# --------------------------------------------------------------------------
# forward invariants
# --------------------------------------------------------------------------

def pin_rows_sum_to_one(orc):
    """P = rowsoftmax(S) over visible keys: every row sums to 1, masked = 0."""
    rng = np.random.default_rng(21)
    n, m, d = 40, 40, 12
    q, k = _rand(rng, n, d), _rand(rng, m, d)
    for causal in (False, True):
        vis = orc.visible_mask(n, m, causal)
        p, mx, l = orc.row_softmax(orc.scaled_scores(q, k, 0.9), vis)
        assert np.all(p[~vis] == 0.0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-13
        s = 0.9 * (q @ k.T)
        assert np.allclose(mx, np.where(vis, s, -np.inf).max(axis=1), rtol=0, atol=1e-14)


def pin_mask_shape(orc):
    """Causal: exactly the keys j <= i are visible (lower triangle incl. diagonal)."""
    vis = orc.visible_mask(7, 7, True)
    assert np.array_equal(vis, np.tril(np.ones((7, 7), dtype=bool)))
    assert orc.visible_mask(5, 5, False).all()


def pin_kv_permutation(orc):
    """Non-causal attention is unchanged when K and V rows move together."""
    rng = np.random.default_rng(22)
    B, N, H, d = 2, 31, 2, 8
    q, k, v = (_rand(rng, B, N, H, d) for _ in range(3))
    perm = rng.permutation(N)
    o1, l1 = orc.attention_forward(q, k, v, 0.4, False)
    o2, l2 = orc.attention_forward(q, k[:, perm], v[:, perm], 0.4, False)
    _close(o1, o2, 1e-13, "permute K,V: O")
    _close(l1, l2, 1e-13, "permute K,V: LSE")


def pin_key_shift(orc):
    """k_j -> k_j + u for all j: O unchanged, LSE_i shifts by scale * q_i . u."""
    rng = np.random.default_rng(23)
    B, N, H, d = 1, 24, 2, 8
    q, k, v = (_rand(rng, B, N, H, d) for _ in range(3))
    u = _rand(rng, d)
    for causal in (False, True):
        o1, l1 = orc.attention_forward(q, k, v, 0.6, causal)
        o2, l2 = orc.attention_forward(q, k + u, v, 0.6, causal)
        _close(o1, o2, 1e-12, "key shift: O")
        shift = 0.6 * np.einsum("bnhd,d->bhn", q, u)
        with np.errstate(invalid="ignore"):
            dl = l2 - l1
        _close(dl, shift, 1e-12, "key shift: LSE")


def pin_linear_in_v(orc):
    """O is linear in V: O(aV1 + bV2) = a O(V1) + b O(V2)."""
    rng = np.random.default_rng(24)
    B, N, H, d = 1, 20, 2, 8
    q, k, v1, v2 = (_rand(rng, B, N, H, d) for _ in range(4))
    for causal in (False, True):
        o1, _ = orc.attention_forward(q, k, v1, 0.5, causal)
        o2, _ = orc.attention_forward(q, k, v2, 0.5, causal)
        o3, _ = orc.attention_forward(q, k, 2.0 * v1 - 3.0 * v2, 0.5, causal)
        _close(o3, 2.0 * o1 - 3.0 * o2, 1e-12, "linear in V")


def pin_lse_bounds(orc):
    """max_j s_ij <= LSE_i <= max_j s_ij + ln(#visible keys of row i)."""
    rng = np.random.default_rng(25)
    B, N, H, d = 1, 50, 1, 8
    q, k, v = (_rand(rng, B, N, H, d) for _ in range(3))
    for causal in (False, True):
        _, lse = orc.attention_forward(q, k, v, 1.3, causal)
        s = 1.3 * (q[0, :, 0] @ k[0, :, 0].T)
        vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
        mx = np.where(vis, s, -np.inf).max(axis=1)
        cnt = vis.sum(axis=1)
        assert np.all(lse[0, 0] >= mx - 1e-12)
        assert np.all(lse[0, 0] <= mx + np.log(cnt) + 1e-12)


def pin_row_subset(orc):
    """Computing a subset of query rows gives exactly those rows of the full result."""
    rng = np.random.default_rng(26)
    B, N, H, d = 2, 45, 2, 8
    q, k, v = (_rand(rng, B, N, H, d) for _ in range(3))
    rows = np.array([0, 7, 44, 13, 30])
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 0.7, causal)
        o_s, lse_s = orc.attention_forward(q, k, v, 0.7, causal, rows=rows, row_block=2)
        _close(o_s, o[:, rows], 1e-14, "row subset O")
        _close(lse_s, lse[:, :, rows], 1e-14, "row subset LSE")


# --------------------------------------------------------------------------
# independent implementations
# --------------------------------------------------------------------------

def pin_brute_force_forward(orc):
    """Pure-Python fsum loops agree with the oracle to 1e-12 (N <= 16, d <= 8)."""
    rng = np.random.default_rng(31)
    for (n_q, n_k, d, causal) in ((9, 9, 4, False), (13, 13, 8, True), (6, 11, 5, True),
                                  (11, 6, 3, True), (16, 16, 8, False)):
        q, k, v = _rand(rng, 1, n_q, 1, d), _rand(rng, 1, n_k, 1, d), _rand(rng, 1, n_k, 1, d)
        o, lse = orc.attention_forward(q, k, v, 0.8, causal)
        bo, blse = brute_forward(q[0, :, 0].tolist(), k[0, :, 0].tolist(),
                                 v[0, :, 0].tolist(), 0.8, causal)
        _close(o[0, :, 0], np.array(bo), 1e-12, f"brute O {n_q}x{n_k} causal={causal}")
        want = np.array(blse)
        got = lse[0, 0]
        assert np.array_equal(np.isinf(got), np.isinf(want))
        fin = np.isfinite(want)
        _close(got[fin], want[fin], 1e-12, "brute LSE")


def pin_brute_force_backward(orc):
    """Pure-Python chain rule agrees with the oracle's gradients to 1e-12."""
    rng = np.random.default_rng(32)
    for (n_q, n_k, d, causal) in ((7, 7, 4, False), (10, 10, 6, True), (16, 16, 8, True),
                                  (5, 9, 4, False), (6, 11, 5, True), (11, 6, 3, True)):
        q, do = _rand(rng, 1, n_q, 1, d), _rand(rng, 1, n_q, 1, d)
        k, v = _rand(rng, 1, n_k, 1, d), _rand(rng, 1, n_k, 1, d)
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.7, causal)
        bq, bk, bv = brute_backward(q[0, :, 0].tolist(), k[0, :, 0].tolist(),
                                    v[0, :, 0].tolist(), do[0, :, 0].tolist(), 0.7, causal)
        _close(dq[0, :, 0], np.array(bq), 1e-12, "brute dQ")
        _close(dk[0, :, 0], np.array(bk), 1e-12, "brute dK")
        _close(dv[0, :, 0], np.array(bv), 1e-12, "brute dV")


def pin_torch_float64_cross(orc):
    """N_q != N_k: torch CPU float64 attention with an explicit mask that aligns
    the keys to the end of the query block agrees to 1e-12, gradients too.
    (Only shapes where every query sees a key: torch returns NaN otherwise.)"""
    import torch

    rng = np.random.default_rng(34)
    for (n_q, n_k, causal) in ((19, 41, True), (19, 41, False), (41, 19, False)):
        B, H, d = 1, 2, 8
        q, do = _rand(rng, B, n_q, H, d), _rand(rng, B, n_q, H, d)
        k, v = _rand(rng, B, n_k, H, d), _rand(rng, B, n_k, H, d)
        tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64,
                                   requires_grad=True) for x in (q, k, v))
        i = torch.arange(n_q)[:, None]
        j = torch.arange(n_k)[None, :]
        mask = (j <= i + (n_k - n_q)) if causal else torch.ones(n_q, n_k, dtype=torch.bool)
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.6)
        to.backward(torch.tensor(do.transpose(0, 2, 1, 3), dtype=torch.float64))
        o, lse = orc.attention_forward(q, k, v, 0.6, causal)
        _close(o, to.detach().numpy().transpose(0, 2, 1, 3), 1e-12, f"torch O {n_q}x{n_k}")
        s_ = (0.6 * torch.matmul(tq.detach(), tk.detach().transpose(-1, -2))).masked_fill(~mask, -float("inf"))
        _close(lse, torch.logsumexp(s_, dim=-1).numpy(), 1e-12, f"torch LSE {n_q}x{n_k}")
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.6, causal)
        for name, mine, ref in (("dQ", dq, tq.grad), ("dK", dk, tk.grad), ("dV", dv, tv.grad)):
            _close(mine, ref.numpy().transpose(0, 2, 1, 3), 1e-12, f"torch {name} {n_q}x{n_k}")


def pin_suffix_queries(orc):
    """Causal with N_q < N_k is the last N_q rows of square causal attention
    over all N_k positions; the gradients are those of the square problem with
    dO = 0 on its first N_k - N_q rows.  With N_q > N_k the first N_q - N_k
    rows see no key: O = 0, LSE = -inf, dQ = 0, and they add nothing to dK, dV."""
    rng = np.random.default_rng(35)
    n_q, n_k, H, d = 6, 15, 2, 5
    qq, kk, vv = (_rand(rng, 1, n_k, H, d) for _ in range(3))
    do = _rand(rng, 1, n_q, H, d)
    o_full, lse_full = orc.attention_forward(qq, kk, vv, 0.45, True)
    o, lse = orc.attention_forward(qq[:, n_k - n_q:], kk, vv, 0.45, True)
    _close(o, o_full[:, n_k - n_q:], 1e-13, "suffix O")
    _close(lse, lse_full[:, :, n_k - n_q:], 1e-13, "suffix LSE")
    do_full = np.zeros((1, n_k, H, d))
    do_full[:, n_k - n_q:] = do
    gq_full, gk_full, gv_full = orc.attention_backward(qq, kk, vv, do_full, 0.45, True)
    gq, gk, gv = orc.attention_backward(qq[:, n_k - n_q:], kk, vv, do, 0.45, True)
    _close(gq, gq_full[:, n_k - n_q:], 1e-13, "suffix dQ")
    _close(gk, gk_full, 1e-13, "suffix dK")
    _close(gv, gv_full, 1e-13, "suffix dV")

    # N_q > N_k: the rows past the first N_q - N_k are the square problem
    n_q, n_k = 13, 4
    q, do = _rand(rng, 1, n_q, H, d), _rand(rng, 1, n_q, H, d)
    k, v = _rand(rng, 1, n_k, H, d), _rand(rng, 1, n_k, H, d)
    o, lse = orc.attention_forward(q, k, v, 0.45, True)
    gq, gk, gv = orc.attention_backward(q, k, v, do, 0.45, True)
    e = n_q - n_k
    assert np.all(o[:, :e] == 0.0) and np.all(np.isneginf(lse[:, :, :e])), "empty rows: O = 0, LSE = -inf"
    assert np.all(gq[:, :e] == 0.0), "empty rows: dQ = 0"
    o_sq, lse_sq = orc.attention_forward(q[:, e:], k, v, 0.45, True)
    _close(o[:, e:], o_sq, 1e-13, "tail O")
    _close(lse[:, :, e:], lse_sq, 1e-13, "tail LSE")
    sq_q, sq_k, sq_v = orc.attention_backward(q[:, e:], k, v, do[:, e:], 0.45, True)
    _close(gq[:, e:], sq_q, 1e-13, "tail dQ")
    _close(gk, sq_k, 1e-13, "tail dK")
    _close(gv, sq_v, 1e-13, "tail dV")


def pin_torch_float64(orc):
    """torch CPU float64 scaled_dot_product_attention + autograd agree to 1e-12."""
    import torch

    rng = np.random.default_rng(33)
    B, N, H, d = 2, 37, 3, 16
    q, k, v, do = (_rand(rng, B, N, H, d) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64,
                                   requires_grad=True) for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=0.35)
        to.backward(torch.tensor(do.transpose(0, 2, 1, 3), dtype=torch.float64))
        o, lse = orc.attention_forward(q, k, v, 0.35, causal)
        _close(o, to.detach().numpy().transpose(0, 2, 1, 3), 1e-12, "torch O")
        s = 0.35 * torch.matmul(tq.detach(), tk.detach().transpose(-1, -2))
        if causal:
            s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), -float("inf"))
        _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, "torch LSE")
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.35, causal)
        for name, mine, ref in (("dQ", dq, tq.grad), ("dK", dk, tk.grad), ("dV", dv, tv.grad)):
            _close(mine, ref.numpy().transpose(0, 2, 1, 3), 1e-12, f"torch {name}")


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def pin_finite_differences(orc):
    """Central differences of L = sum(O * dO) match the gradients (rel 1e-6)."""
    rng = np.random.default_rng(41)
    eps = 1e-6
    for (n_q, n_k, d, causal) in ((5, 5, 3, False), (6, 6, 4, True), (8, 8, 4, True),
                                  (4, 7, 3, True), (7, 4, 3, True), (3, 6, 2, False)):
        q, do = _rand(rng, 1, n_q, 1, d), _rand(rng, 1, n_q, 1, d)
        k, v = _rand(rng, 1, n_k, 1, d), _rand(rng, 1, n_k, 1, d)
        scale = 0.9
        grads = orc.attention_backward(q, k, v, do, scale, causal)

        def loss(qq, kk, vv):
            o, _ = orc.attention_forward(qq, kk, vv, scale, causal)
            return float(np.sum(o * do))

        for which, g in zip(range(3), grads):
            fd = np.zeros_like(g)
            for idx in np.ndindex(*g.shape):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][idx] += eps
                args_m[which][idx] -= eps
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            rel = np.max(np.abs(fd - g)) / max(np.max(np.abs(g)), 1e-300)
            assert rel <= 1e-6, f"finite differences arg {which} causal={causal}: rel {rel:.2e}"


def pin_gradient_identities(orc):
    """sum_j dV_j = sum_i dO_i;  sum_j dK_j = 0;  causal dQ_0 = 0;
    constant V gives dQ = dK = 0;  dV is linear in dO."""
    rng = np.random.default_rng(42)
    B, N, H, d = 2, 23, 2, 8
    q, k, v, do, do2 = (_rand(rng, B, N, H, d) for _ in range(5))
    for causal in (False, True):
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.5, causal)
        _close(dv.sum(axis=1), do.sum(axis=1), 1e-12, "sum dV = sum dO")
        _close(dk.sum(axis=1), np.zeros((B, H, d)), 1e-12, "sum dK = 0")
        if causal:
            _close(dq[:, 0], np.zeros((B, H, d)), 1e-14, "causal dQ_0 = 0")
        vc = np.broadcast_to(_rand(rng, d), v.shape).copy()
        dq_c, dk_c, _ = orc.attention_backward(q, k, vc, do, 0.5, causal)
        _close(dq_c, np.zeros_like(dq_c), 1e-12, "constant V: dQ = 0")
        _close(dk_c, np.zeros_like(dk_c), 1e-12, "constant V: dK = 0")
        _, _, dv2 = orc.attention_backward(q, k, v, do2, 0.5, causal)
        _, _, dv3 = orc.attention_backward(q, k, v, 3.0 * do - do2, 0.5, causal)
        _close(dv3, 3.0 * dv - dv2, 1e-12, "dV linear in dO")


# --------------------------------------------------------------------------
# sliding window and grouped-query attention
# --------------------------------------------------------------------------

def pin_window_closed_forms(orc):
    """W = 1: every row sees only its own position, so O_i = V_i', LSE_i =
    s_ii', dV = dO scattered to those keys, dQ = dK = 0 (a one-key softmax is
    constant).  W = 2 causal: row i sees keys i - 1 and i, so O_i = sig V_i +
    (1 - sig) V_{i-1} with sig = 1 / (1 + exp(s_i,i-1 - s_ii)).  A window
    wider than every distance changes nothing."""
    rng = np.random.default_rng(51)
    B, H, d, scale = 1, 2, 4, 0.7
    for (n_q, n_k, causal) in ((9, 9, True), (9, 9, False), (4, 9, True), (4, 9, False)):
        q, do = _rand(rng, B, n_q, H, d), _rand(rng, B, n_q, H, d)
        k, v = _rand(rng, B, n_k, H, d), _rand(rng, B, n_k, H, d)
        pos = np.arange(n_q) + (n_k - n_q)
        o, lse = orc.attention_forward(q, k, v, scale, causal, window=1)
        _close(o, v[:, pos], 1e-14, "W=1: O = V at the own position")
        _close(lse, scale * np.einsum("bihc,bihc->bhi", q, k[:, pos]), 1e-13, "W=1: LSE = own score")
        dq, dk, dv = orc.attention_backward(q, k, v, do, scale, causal, window=1)
        want_dv = np.zeros_like(v)
        want_dv[:, pos] = do
        _close(dv, want_dv, 1e-14, "W=1: dV = dO at the own position")
        _close(dq, np.zeros_like(dq), 1e-14, "W=1: dQ = 0")
        _close(dk, np.zeros_like(dk), 1e-14, "W=1: dK = 0")
        o_w, lse_w = orc.attention_forward(q, k, v, scale, causal, window=n_q + n_k)
        o_f, lse_f = orc.attention_forward(q, k, v, scale, causal)
        _close(o_w, o_f, 1e-15, "wide window = no window (O)")
        _close(lse_w, lse_f, 1e-15, "wide window = no window (LSE)")
    n = 7
    q, k, v = _rand(rng, 1, n, 1, d), _rand(rng, 1, n, 1, d), _rand(rng, 1, n, 1, d)
    o, _ = orc.attention_forward(q, k, v, scale, True, window=2)
    s_self = scale * np.sum(q[0, 1:, 0] * k[0, 1:, 0], axis=1)
    s_prev = scale * np.sum(q[0, 1:, 0] * k[0, :-1, 0], axis=1)
    sig = 1.0 / (1.0 + np.exp(s_prev - s_self))
    want = sig[:, None] * v[0, 1:, 0] + (1.0 - sig[:, None]) * v[0, :-1, 0]
    _close(o[0, 1:, 0], want, 1e-13, "W=2 causal: two-key softmax")
    _close(o[0, 0, 0], v[0, 0, 0], 1e-14, "W=2 causal: first row sees one key")


def pin_brute_force_window(orc):
    """Pure-Python loops with a window agree with the oracle to 1e-12,
    forward and backward, square and cross shapes."""
    rng = np.random.default_rng(52)
    for (n_q, n_k, d, causal, window) in ((12, 12, 3, True, 3), (12, 12, 3, False, 3), (5, 13, 4, True, 4),
                                          (13, 5, 2, False, 2), (10, 10, 4, True, 1), (8, 11, 3, False, 6)):
        q, do = _rand(rng, 1, n_q, 1, d), _rand(rng, 1, n_q, 1, d)
        k, v = _rand(rng, 1, n_k, 1, d), _rand(rng, 1, n_k, 1, d)
        o, lse = orc.attention_forward(q, k, v, 0.8, causal, window=window)
        bo, blse = brute_forward(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(), 0.8, causal,
                                 window)
        tag = f"{n_q}x{n_k} causal={causal} W={window}"
        _close(o[0, :, 0], np.array(bo), 1e-12, f"brute O {tag}")
        want = np.array(blse)
        assert np.array_equal(np.isinf(lse[0, 0]), np.isinf(want)), tag
        fin = np.isfinite(want)
        _close(lse[0, 0][fin], want[fin], 1e-12, f"brute LSE {tag}")
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.8, causal, window=window)
        bq, bk, bv = brute_backward(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(),
                                    do[0, :, 0].tolist(), 0.8, causal, window)
        _close(dq[0, :, 0], np.array(bq), 1e-12, f"brute dQ {tag}")
        _close(dk[0, :, 0], np.array(bk), 1e-12, f"brute dK {tag}")
        _close(dv[0, :, 0], np.array(bv), 1e-12, f"brute dV {tag}")


def pin_torch_float64_gqa_window(orc):
    """torch CPU float64 attention with enable_gqa (query heads grouped over
    fewer K/V heads) and an explicit band mask, plus autograd, agrees to
    1e-12, including dK / dV summed over each group."""
    import torch

    rng = np.random.default_rng(53)
    for (H, H_kv, n_q, n_k, causal, window) in ((6, 2, 21, 21, True, 0), (8, 1, 17, 30, False, 0),
                                                (4, 2, 25, 25, True, 7), (4, 4, 19, 33, False, 5),
                                                (6, 3, 25, 19, False, 8)):
        B, d = 2, 8
        q, do = _rand(rng, B, n_q, H, d), _rand(rng, B, n_q, H, d)
        k, v = _rand(rng, B, n_k, H_kv, d), _rand(rng, B, n_k, H_kv, d)
        tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
                      for x in (q, k, v))
        pos = torch.arange(n_q)[:, None] + (n_k - n_q)
        j = torch.arange(n_k)[None, :]
        mask = torch.ones(n_q, n_k, dtype=torch.bool)
        if causal:
            mask &= j <= pos
        if window:
            mask &= (pos - j).abs() < window
        assert bool(mask.any(dim=1).all()), "every row must see a key (torch gives NaN otherwise)"
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.5,
                                                              enable_gqa=True)
        to.backward(torch.tensor(do.transpose(0, 2, 1, 3), dtype=torch.float64))
        tag = f"H={H}/{H_kv} {n_q}x{n_k} causal={causal} W={window}"
        o, _ = orc.attention_forward(q, k, v, 0.5, causal, window=window)
        _close(o, to.detach().numpy().transpose(0, 2, 1, 3), 1e-12, f"torch O {tag}")
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.5, causal, window=window)
        for name, mine, ref in (("dQ", dq, tq.grad), ("dK", dk, tk.grad), ("dV", dv, tv.grad)):
            _close(mine, ref.numpy().transpose(0, 2, 1, 3), 1e-12, f"torch {name} {tag}")


def pin_gqa_is_repeated_heads(orc):
    """Grouped-query attention equals multi-head attention on K / V heads
    repeated over each group, and the shared heads' gradients are the sums
    of the repeated heads' gradients."""
    rng = np.random.default_rng(54)
    B, H, H_kv, n, d = 2, 6, 2, 11, 4
    q, do = _rand(rng, B, n, H, d), _rand(rng, B, n, H, d)
    k, v = _rand(rng, B, n, H_kv, d), _rand(rng, B, n, H_kv, d)
    kr, vr = np.repeat(k, H // H_kv, axis=2), np.repeat(v, H // H_kv, axis=2)
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 0.6, causal)
        o_r, lse_r = orc.attention_forward(q, kr, vr, 0.6, causal)
        _close(o, o_r, 1e-15, "GQA O = repeated-head O")
        _close(lse, lse_r, 1e-15, "GQA LSE = repeated-head LSE")
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.6, causal)
        dq_r, dk_r, dv_r = orc.attention_backward(q, kr, vr, do, 0.6, causal)
        _close(dq, dq_r, 1e-15, "GQA dQ")
        _close(dk, dk_r.reshape(B, n, H_kv, H // H_kv, d).sum(axis=3), 1e-14, "GQA dK = group sum")
        _close(dv, dv_r.reshape(B, n, H_kv, H // H_kv, d).sum(axis=3), 1e-14, "GQA dV = group sum")


ALL_PINS = [
    pin_constant_v,
    pin_uniform_scores,
    pin_causal_first_row,
    pin_single_key,
    pin_dominant_key,
    pin_rows_sum_to_one,
    pin_mask_shape,
    pin_kv_permutation,
    pin_key_shift,
    pin_linear_in_v,
    pin_lse_bounds,
    pin_row_subset,
    pin_brute_force_forward,
    pin_brute_force_backward,
    pin_torch_float64,
    pin_torch_float64_cross,
    pin_suffix_queries,
    pin_window_closed_forms,
    pin_brute_force_window,
    pin_torch_float64_gqa_window,
    pin_gqa_is_repeated_heads,
    pin_finite_differences,
    pin_gradient_identities,
]
