"""Pins of the float64 oracle against what the pages and mathematics fix.

CPU only.  Every oracle function is checked against something other than
itself: values printed on the pages (tests/golden/), closed forms,
invariants, central finite differences, and independent library routines
(torch's float64 scaled_dot_product_attention and autograd, scipy's
logsumexp).  The cases are chosen so that a dropped term, a wrong sign, a
wrong index, a transposed operand or a reversed mask fails at least one.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle

RNG = np.random.default_rng(20240611)


def rand(*shape):
    return RNG.standard_normal(shape)


# --------------------------------------------------------------------------
# Softmax and online softmax (Lensa ML explainer, Step 4 "Online Softmax")
# --------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", range(1, 9))
def test_eight_score_example_matches_printed_values(golden, chunk):
    g = golden("online_softmax_8scores.txt")
    x = np.array(g["scores"])
    printed = np.array(g["softmax_2dp"])
    p, _, _ = oracle.softmax_online(x, chunk)
    # printed to two decimals: each value within half a unit of the last place
    assert np.all(np.abs(p - printed) <= 0.005 + 1e-12), (chunk, p)
    # same result for every chunk size, up to float64 rounding
    assert np.max(np.abs(p - oracle.softmax(x))) <= 1e-15


def test_eight_score_default_run_running_stats(golden):
    g = golden("online_softmax_8scores.txt")
    x = np.array(g["scores"])
    chunk = int(g["default_chunk"])
    p, mt, lt = oracle.softmax_online(x, chunk)
    assert len(mt) == int(g["default_chunks"])
    # invariant of the running statistics after chunk c: m is the maximum of
    # the scores seen so far and l = sum over seen scores of e^{x - m}
    for c in range(len(mt)):
        seen = x[: (c + 1) * chunk]
        assert mt[c] == seen.max()
        assert abs(lt[c] - math.fsum(math.exp(t - seen.max()) for t in seen)) <= 1e-15
    # the first two running sums in closed form: e^{1.2-3} + 1, then + e^{.4-3} + e^{2.1-3}
    assert abs(lt[0] - (math.exp(-1.8) + 1.0)) <= 1e-15
    assert abs(lt[1] - (math.exp(-1.8) + 1.0 + math.exp(-2.6) + math.exp(-0.9))) <= 1e-15
    # the global log-sum-exp agrees with scipy
    assert abs(mt[-1] + math.log(lt[-1]) - scipy.special.logsumexp(x)) <= 1e-14


def test_fp16_overflow_threshold(golden):
    g = golden("online_softmax_8scores.txt")
    # e^x overflows fp16 just above ln(65504) = 11.09, which the page rounds to 11.1
    assert abs(math.log(g["fp16_max"]) - g["fp16_overflow_exponent_approx"]) < 0.05
    with np.errstate(over="ignore"):
        assert np.isinf(np.float16(math.exp(11.1)))
    assert np.isfinite(np.float16(math.exp(11.08)))
    # the max-subtracted softmax stays finite and exact for huge scores
    x = np.array([1000.0, 1000.5, -1000.0])  # exactly representable scores
    e = math.exp(0.5)
    expect = [1 / (1 + e), e / (1 + e), 0.0]
    p = oracle.softmax(x)
    assert np.allclose(p, expect, rtol=0, atol=1e-15)
    p2, _, _ = oracle.softmax_online(x, 1)
    assert np.allclose(p2, expect, rtol=0, atol=1e-15)


def test_softmax_rows_sum_to_one_and_match_scipy():
    for n in (1, 2, 7, 64, 1000):
        x = rand(n) * 5
        p = oracle.softmax(x)
        assert abs(p.sum() - 1.0) <= 1e-12
        assert np.max(np.abs(p - scipy.special.softmax(x))) <= 1e-15
        for chunk in (1, 3, 16, n):
            po, _, _ = oracle.softmax_online(x, chunk)
            assert np.max(np.abs(po - p)) <= 1e-15


def test_softmax_masked_entries_are_zero():
    x = np.array([-np.inf, 0.5, -np.inf, 1.5])
    p = oracle.softmax(x)
    assert p[0] == 0 and p[2] == 0
    assert np.allclose(p[[1, 3]], scipy.special.softmax([0.5, 1.5]), atol=1e-16)


# --------------------------------------------------------------------------
# Forward: three-step attention (frontier notes "Le problème"; P1 pseudocode)
# --------------------------------------------------------------------------

def sdpa64(q, k, v, scale, causal):
    t = [torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=scale)
    return o.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 4), (7, 8), (33, 16), (130, 64)])
def test_fwd_matches_torch_sdpa_float64(n, d, causal):
    q, k, v = rand(2, 3, n, d), rand(2, 3, n, d), rand(2, 3, n, d)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attn_fwd(q, k, v, scale, causal)
    assert np.max(np.abs(o - sdpa64(q, k, v, scale, causal))) <= 1e-13
    s = scale * q @ np.swapaxes(k, -1, -2)
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    assert np.max(np.abs(lse - scipy.special.logsumexp(s, axis=-1))) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_permutation_closed_form(causal):
    # Q_i = t e_i and K_j = e_{pi(j)}: score a = scale*t where i == pi(j), else 0.
    n, d, t = 12, 16, 3.0
    scale = 0.7
    a = scale * t
    perm = RNG.permutation(n)
    eye = np.eye(d)
    q = t * eye[:n]
    k = eye[perm]
    v = rand(n, d)
    o, lse = oracle.attn_fwd(q, k, v, scale, causal)
    inv = np.argsort(perm)  # key j* with pi(j*) = i
    for i in range(n):
        vis = list(range(i + 1)) if causal else list(range(n))
        js = inv[i]
        if js in vis:
            z = math.exp(a) + (len(vis) - 1)
            expect = (math.exp(a) * v[js] + sum(v[j] for j in vis if j != js)) / z
        else:
            z = float(len(vis))
            expect = sum(v[j] for j in vis) / z
        assert np.max(np.abs(o[i] - expect)) <= 1e-14
        assert abs(lse[i] - math.log(z)) <= 1e-14


def test_fwd_causal_first_row_is_first_value():
    n, d = 9, 8
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o, lse = oracle.attn_fwd(q, k, v, 0.3, True)
    assert np.array_equal(o[0], v[0])
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_identical_keys_give_mean_of_visible_values(causal):
    n, d = 11, 8
    q, v = rand(n, d), rand(n, d)
    kappa = rand(d)
    k = np.tile(kappa, (n, 1))
    scale = 0.4
    o, lse = oracle.attn_fwd(q, k, v, scale, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        assert np.max(np.abs(o[i] - v[:cnt].mean(axis=0))) <= 1e-14
        assert abs(lse[i] - (scale * float(q[i] @ kappa) + math.log(cnt))) <= 1e-13


def test_fwd_constant_values_and_zero_scale():
    n, d = 10, 4
    q, k = rand(n, d) * 3, rand(n, d) * 3
    v = np.full((n, d), 2.5)
    o, _ = oracle.attn_fwd(q, k, v, 1.0, False)
    assert np.max(np.abs(o - 2.5)) <= 1e-14
    v = rand(n, d)
    o, lse = oracle.attn_fwd(q, k, v, 0.0, True)
    for i in range(n):
        assert np.max(np.abs(o[i] - v[: i + 1].mean(axis=0))) <= 1e-14
        assert abs(lse[i] - math.log(i + 1)) <= 1e-15


def test_fwd_query_positions_select_rows():
    n, d = 40, 8
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    rows = np.array([0, 5, 17, 39])
    o2, lse2 = oracle.attn_fwd(q[rows], k, v, 0.5, True, qpos=rows)
    assert np.array_equal(o2, o[rows]) and np.array_equal(lse2, lse[rows])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", [(1, 1), (4, 4), (16, 5), (64, 64), (7, 128)])
def test_tiled_equals_standard(br, bc, causal):
    n, d = 77, 16
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o, lse = oracle.attn_fwd(q, k, v, 0.25, causal)
    ot, lset = oracle.attn_fwd_tiled(q, k, v, 0.25, causal, br, bc)
    assert np.max(np.abs(ot - o)) <= 1e-14
    assert np.max(np.abs(lset - lse)) <= 1e-14


def test_tiled_exactness_demo_size(golden):
    g = golden("tiled_exactness.txt")
    d, tiles, per = int(g["head_dim"]), int(g["tiles"]), int(g["keys_per_tile_max"])
    worst = 0.0
    for seed in range(20):
        r = np.random.default_rng(seed)
        nk = r.integers(tiles * per - per + 1, tiles * per + 1)  # 4 tiles of <= 4 keys
        q, k, v = r.standard_normal((1, d)), r.standard_normal((nk, d)), r.standard_normal((nk, d))
        o, _ = oracle.attn_fwd(q, k, v, 1 / math.sqrt(d), False)
        ot, _ = oracle.attn_fwd_tiled(q, k, v, 1 / math.sqrt(d), False, 1, per)
        worst = max(worst, float(np.max(np.abs(ot - o))))
    # pure rounding: the same order as the page's 2.2e-16, far from any real error
    assert worst <= 8 * g["max_abs_diff"], worst


# --------------------------------------------------------------------------
# Backward (recomputation; plain calculus of the three-step definition)
# --------------------------------------------------------------------------

def loss_fd_grads(q, k, v, do, scale, causal, h=1e-6):
    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, scale, causal)
        return float(np.sum(o * do))
    grads = []
    for idx, x in enumerate((q, k, v)):
        g = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][pos] += h
            up = loss(*args)
            args[idx][pos] -= 2 * h
            dn = loss(*args)
            g[pos] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 3), (5, 4), (16, 8)])
def test_bwd_finite_differences(n, d, causal):
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    scale = 1 / math.sqrt(d)
    got = oracle.attn_bwd(q, k, v, do, scale, causal)
    ref = loss_fd_grads(q, k, v, do, scale, causal)
    for g, r in zip(got, ref):
        den = max(np.linalg.norm(r), 1e-30)
        assert np.linalg.norm(g - r) / den <= 1e-6 or np.linalg.norm(g - r) <= 1e-9


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_torch_autograd_float64(causal):
    b, h, n, d = 2, 2, 37, 16
    q, k, v, do = (rand(b, h, n, d) for _ in range(4))
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_() for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.from_numpy(do))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal)
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(g - t.grad.numpy())) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    n, d = 50, 16
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    scale = 0.3
    dq, dk, dv, drow = oracle.attn_bwd(q, k, v, do, scale, causal, return_drow=True)
    o, _ = oracle.attn_fwd(q, k, v, scale, causal)
    # D_i = sum_j P_ij dP_ij equals the row dot product of dO and O
    assert np.max(np.abs(drow - np.sum(do * o, axis=-1))) <= 1e-13
    # rows of dS sum to zero, so the key gradients sum to zero
    assert np.max(np.abs(dk.sum(axis=0))) <= 1e-12
    # rows of P sum to one, so the value gradients sum to the output gradients
    assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) <= 1e-12


def test_bwd_causal_last_key_gets_only_last_query():
    n, d = 8, 4
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.5, True)
    _, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    p_last = math.exp(0.5 * float(q[-1] @ k[-1]) - lse[-1])
    # only the last query sees the last key
    assert np.max(np.abs(dv[-1] - p_last * do[-1])) <= 1e-14


# --------------------------------------------------------------------------
# Sliding window ("03. FlashAttention", § "Variantes et extensions": the
# variant only considers the keys inside the window; reading: key j is
# visible to query i iff i - w < j <= i)
# --------------------------------------------------------------------------

def window_mask(n, w):
    """Boolean [n, n] mask built from band matrices (lower triangle minus the
    part more than w - 1 below the diagonal)."""
    ones = np.ones((n, n), dtype=bool)
    return np.tril(ones) & ~np.tril(ones, -w)


@pytest.mark.parametrize("n,d,w", [(9, 4, 3), (40, 8, 7), (64, 16, 1), (33, 8, 32)])
def test_window_fwd_bwd_match_torch_masked_sdpa(n, d, w):
    q, k, v, do = (rand(2, 2, n, d) for _ in range(4))
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_() for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(window_mask(n, w)), scale=scale)
    o.backward(torch.from_numpy(do))
    got, _ = oracle.attn_fwd(q, k, v, scale, True, window=w)
    assert np.max(np.abs(got - o.detach().numpy())) <= 1e-13
    for g, t in zip(oracle.attn_bwd(q, k, v, do, scale, True, window=w), (tq, tk, tv)):
        assert np.max(np.abs(g - t.grad.numpy())) <= 1e-12


@pytest.mark.parametrize("w", [1, 2, 5, 11])
def test_window_rows_are_unmasked_attention_over_their_keys(w):
    n, d = 23, 8
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o, lse = oracle.attn_fwd(q, k, v, 0.4, True, window=w)
    for i in range(n):
        lo = max(0, i - w + 1)
        oi, li = oracle.attn_fwd(q[i:i + 1], k[lo:i + 1], v[lo:i + 1], 0.4, False)
        assert np.max(np.abs(o[i] - oi[0])) <= 1e-14 and abs(lse[i] - li[0]) <= 1e-14


def test_window_one_closed_form():
    n, d = 17, 8
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    o, lse = oracle.attn_fwd(q, k, v, 0.7, True, window=1)
    # each query sees only its own key: O = V, lse = scale q_i . k_i
    assert np.array_equal(o, v)
    assert np.max(np.abs(lse - 0.7 * np.sum(q * k, axis=1))) <= 1e-14
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.7, True, window=1)
    # P = 1 on the diagonal, so dS = P (dP - D) vanishes and dV = dO
    assert np.array_equal(dv, do) and not np.any(dq) and not np.any(dk)


@pytest.mark.parametrize("w", [40, 41, 1000])
def test_window_covering_the_sequence_is_causal(w):
    n, d = 40, 8
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    a = oracle.attn_fwd(q, k, v, 0.5, True, window=w)
    c = oracle.attn_fwd(q, k, v, 0.5, True)
    assert all(np.array_equal(x, y) for x, y in zip(a, c))
    ga = oracle.attn_bwd(q, k, v, do, 0.5, True, window=w)
    gc = oracle.attn_bwd(q, k, v, do, 0.5, True)
    assert all(np.array_equal(x, y) for x, y in zip(ga, gc))


@pytest.mark.parametrize("w", [2, 4])
def test_window_bwd_finite_differences(w):
    n, d = 7, 3
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    scale = 0.6
    got = oracle.attn_bwd(q, k, v, do, scale, True, window=w)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, scale, True, window=w)
        return float(np.sum(o * do))
    for idx, g in enumerate(got):
        x0 = (q, k, v)[idx]
        ref = np.zeros_like(x0)
        for pos in np.ndindex(x0.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][pos] += 1e-6
            up = loss(*args)
            args[idx][pos] -= 2e-6
            ref[pos] = (up - loss(*args)) / 2e-6
        assert np.linalg.norm(g - ref) <= 1e-6 * max(np.linalg.norm(ref), 1e-3)


# --------------------------------------------------------------------------
# Grouped key/value heads ("FlashAttention ontleed", § "Interactie met de
# KV-cache tijdens inferentie": several query heads share one key/value head;
# reading: query head h reads key/value head h // (H / H_kv))
# --------------------------------------------------------------------------

@pytest.mark.parametrize("h,hkv,causal", [(4, 2, True), (6, 3, False), (8, 1, True), (4, 4, False)])
def test_gqa_fwd_bwd_match_torch_sdpa(h, hkv, causal):
    b, n, d = 2, 19, 8
    q, do = rand(b, h, n, d), rand(b, h, n, d)
    k, v = rand(b, hkv, n, d), rand(b, hkv, n, d)
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_() for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                         enable_gqa=True)
    o.backward(torch.from_numpy(do))
    got, _ = oracle.attn_fwd(q, k, v, scale, causal)
    assert np.max(np.abs(got - o.detach().numpy())) <= 1e-13
    for g, t in zip(oracle.attn_bwd(q, k, v, do, scale, causal), (tq, tk, tv)):
        assert g.shape == t.shape and np.max(np.abs(g - t.grad.numpy())) <= 1e-12


def test_gqa_heads_are_plain_attention_on_their_group_head():
    b, h, hkv, n, d = 2, 6, 2, 13, 8
    q, do = rand(b, h, n, d), rand(b, h, n, d)
    k, v = rand(b, hkv, n, d), rand(b, hkv, n, d)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True, window=5)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.5, True, window=5)
    g = h // hkv
    sk, sv = np.zeros_like(k), np.zeros_like(v)
    for bi in range(b):
        for hi in range(h):
            kv = hi // g
            oh, lh = oracle.attn_fwd(q[bi, hi], k[bi, kv], v[bi, kv], 0.5, True, window=5)
            assert np.array_equal(oh, o[bi, hi]) and np.array_equal(lh, lse[bi, hi])
            gq, gk, gv = oracle.attn_bwd(q[bi, hi], k[bi, kv], v[bi, kv], do[bi, hi], 0.5, True,
                                         window=5)
            assert np.array_equal(gq, dq[bi, hi])
            sk[bi, kv] += gk
            sv[bi, kv] += gv
    # a shared head's gradient is the sum of its group's per-head gradients
    assert np.max(np.abs(sk - dk)) <= 1e-14 and np.max(np.abs(sv - dv)) <= 1e-14


def test_gqa_identical_query_heads_scale_the_shared_gradient():
    n, d, g = 11, 4, 3
    q1, do1 = rand(n, d), rand(n, d)
    k, v = rand(1, 1, n, d), rand(1, 1, n, d)
    q = np.broadcast_to(q1, (1, g, n, d)).copy()
    do = np.broadcast_to(do1, (1, g, n, d)).copy()
    _, dk, dv = oracle.attn_bwd(q, k, v, do, 0.5, False)
    _, dk1, dv1 = oracle.attn_bwd(q1, k[0, 0], v[0, 0], do1, 0.5, False)
    assert np.max(np.abs(dk[0, 0] - g * dk1)) <= 1e-13
    assert np.max(np.abs(dv[0, 0] - g * dv1)) <= 1e-13


def test_gqa_decode_matches_torch():
    b, h, hkv, nkv, d = 2, 8, 2, 200, 16
    q, k, v = rand(b, h, 1, d), rand(b, hkv, nkv, d), rand(b, hkv, nkv, d)
    o, lse = oracle.attn_decode(q, k, v, 0.25)
    t = [torch.from_numpy(a) for a in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, scale=0.25, enable_gqa=True)
    assert o.shape == (b, h, d) and lse.shape == (b, h)
    assert np.max(np.abs(o - ref.numpy()[:, :, 0])) <= 1e-13
    ref_lse = scipy.special.logsumexp(0.25 * np.einsum("bhd,bhnd->bhn", q[:, :, 0],
                                                       np.repeat(k, h // hkv, axis=1)), axis=-1)
    assert np.max(np.abs(lse - ref_lse)) <= 1e-13


# --------------------------------------------------------------------------
# Decode and the split-history merge
# --------------------------------------------------------------------------

def test_decode_matches_torch_and_forward():
    b, h, nkv, d = 3, 2, 300, 32
    q, k, v = rand(b, h, 1, d), rand(b, h, nkv, d), rand(b, h, nkv, d)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attn_decode(q, k, v, scale)
    ref = sdpa64(q, k, v, scale, False)[:, :, 0]
    assert np.max(np.abs(o - ref)) <= 1e-13
    of, lsef = oracle.attn_fwd(q, k, v, scale, False)
    assert np.array_equal(of[:, :, 0], o) and np.array_equal(lsef[:, :, 0], lse)


def test_decode_ragged_lengths():
    """Per-sequence history lengths ("FlashAttention ontleed", § "Interactie met de
    KV-cache tijdens inferentie": K and V span each sequence's own history)."""
    b, h, hkv, nkv, d = 4, 4, 2, 50, 8
    q, k, v = rand(b, h, 1, d), rand(b, hkv, nkv, d), rand(b, hkv, nkv, d)
    full = oracle.attn_decode(q, k, v, 0.3)
    same = oracle.attn_decode(q, k, v, 0.3, kv_lens=[nkv] * b)
    assert all(np.array_equal(x, y) for x, y in zip(full, same))
    lens = [50, 1, 0, 17]
    o, lse = oracle.attn_decode(q, k, v, 0.3, kv_lens=lens)
    # torch with a key-padding mask
    mask = torch.from_numpy(np.arange(nkv)[None, :] < np.array(lens)[:, None])[:, None, None, :]
    t = [torch.from_numpy(a) for a in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=mask, scale=0.3,
                                                           enable_gqa=True).numpy()[:, :, 0]
    for bi in (0, 1, 3):
        assert np.max(np.abs(o[bi] - ref[bi])) <= 1e-13
    # one key: o is that key's value row, lse its scaled score
    assert np.array_equal(o[1], np.repeat(v[1, :, 0], h // hkv, axis=0))
    assert np.max(np.abs(lse[1] - 0.3 * np.einsum("hd,hd->h", q[1, :, 0],
                                                  np.repeat(k[1, :, 0], h // hkv, axis=0)))) <= 1e-14
    # no keys: o = 0, lse = -inf
    assert not np.any(o[2]) and np.all(lse[2] == -np.inf)


@pytest.mark.parametrize("nkv,splits", [(100, 1), (100, 3), (1024, 16), (1000, 16), (5, 16)])
def test_merge_of_any_partition_equals_full_row(nkv, splits):
    d = 16
    q, k, v = rand(d), rand(nkv, d), rand(nkv, d)
    scale = 0.5
    full_o, full_lse = oracle.attn_decode(q, k, v, scale)
    chunk = -(-nkv // splits)
    parts_o, parts_lse = [], []
    for c in range(splits):
        lo, hi = c * chunk, min(nkv, (c + 1) * chunk)
        if lo >= hi:  # an empty chunk carries weight zero
            parts_o.append(np.zeros(d))
            parts_lse.append(-np.inf)
            continue
        oc, lc = oracle.attn_decode(q, k[lo:hi], v[lo:hi], scale)
        parts_o.append(oc)
        parts_lse.append(float(lc))
    o, lse = oracle.lse_merge(np.array(parts_o), np.array(parts_lse))
    assert np.max(np.abs(o - full_o)) <= 1e-14
    assert abs(lse - float(full_lse)) <= 1e-13
