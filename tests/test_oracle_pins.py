"""Pins of the CPU oracle against facts fixed outside it (no GPU).

Each ``check_*`` function compares the oracle with something it does not
compute itself: brute-force enumeration, an independent library routine
(torch SDPA, torch's float32->bfloat16 cast), exact rational arithmetic, a
closed form of the mathematics, or numbers printed on the pages (fixtures
under tests/golden/).  The ``test_mutation_*`` tests plant plausible mistakes
in the oracle (on the CPU) and show that a pin fails.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import rtp_oracle as O
from oracle.problem import Problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ rounding
def check_bf16_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(ref, got)


def round_fraction(v: Fraction, sig_bits: int) -> Fraction:
    """Exact round-half-even of a rational to ``sig_bits`` significant bits (normal range)."""
    if v == 0:
        return Fraction(0)
    sgn = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (e - sig_bits + 1)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * q


def check_project_exact(dtype, n=300, seed=2):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((16, 128)).astype(np.float32).astype(np.float64)
    x = O.round_to(rng.standard_normal((n, 128)), dtype)
    got = O.project(x, w, dtype)
    bits = 8 if dtype == "bf16" else 24
    for i in range(n):
        for j in range(16):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[i], w[j]))
            assert Fraction(float(got[i, j])) == round_fraction(exact, bits), (i, j)


def check_single_rounding():
    # exact dot = 1 + 2^-8 + 2^-30 sits just above the bf16 midpoint between
    # 1 and 1 + 2^-7: one rounding gives 1 + 2^-7, rounding through float32
    # first would land on the midpoint and give 1.
    w = np.zeros((16, 128))
    w[0, 0] = 1.0
    w[1, 1] = 1.0
    x = np.zeros((1, 128))
    x[0, 0] = 1.0 + 2.0 ** -8
    x[0, 1] = 1.0 + 3 * 2.0 ** -8
    x2 = x.copy()
    x2[0, 0] = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert O.project(x, w, "bf16")[0, 0] == 1.0                   # tie -> even
    assert O.project(x, w, "bf16")[0, 1] == 1.0 + 2.0 ** -6        # tie -> even (up)
    assert O.project(x2, w, "bf16")[0, 0] == 1.0 + 2.0 ** -7       # above the tie


def test_bf16_matches_torch():
    check_bf16_matches_torch()


def test_project_exact_bf16():
    check_project_exact("bf16")


def test_project_exact_f32():
    check_project_exact("f32", n=100)


def test_project_single_rounding():
    check_single_rounding()


# ------------------------------------------------------------------ top-p
def brute_force_min_count(prob, p):
    n = len(prob)
    for k in range(1, n + 1):
        for sub in itertools.combinations(range(n), k):
            if sum(prob[list(sub)]) >= p:
                return k
    return n


def check_bruteforce(trials=120, seed=3):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(1, 11))
        s = rng.standard_normal(n) * rng.uniform(0.1, 4.0)
        if t % 5 == 0:
            s = np.round(s)                    # force ties
        p = float(rng.choice([0.3, 0.5, 0.8, 0.9, 0.95, 0.99, rng.uniform(0.01, 0.999)]))
        res = O.top_p(s, p)
        prob = np.exp(s - s.max())
        prob /= prob.sum()
        kmin = brute_force_min_count(prob, p)
        assert res.count == kmin, (s, p, res.count, kmin)
        assert prob[res.selected].sum() >= p - 1e-12
        # the set is a top-|S| prefix: every selected score >= every unselected one,
        # and among equal scores the earlier positions are the selected ones
        sel = set(res.selected.tolist())
        for a in sel:
            for b in range(n):
                if b not in sel:
                    assert s[a] > s[b] or (s[a] == s[b] and a < b)


def check_uniform_exact():
    # four equal scores: masses are exactly 1/4; p = 1/2 is reached by two
    # tokens (the earliest positions), p just above needs three
    r = O.top_p(np.zeros(4), 0.5)
    assert r.count == 2 and r.selected.tolist() == [0, 1]
    r = O.top_p(np.zeros(4), 0.5 + 1e-12)
    assert r.count == 3 and r.selected.tolist() == [0, 1, 2]


def check_gaussian_closed_form():
    # q_idx = (4, 0, ..., 0) and k_idx ~ N(0, I_16) give s = q.k / 4 ~ N(0, 1).
    # Under the tilted measure the mass above tau is Phi_bar(tau - 1), so the
    # minimal top-p set covers a fraction Phi_bar(1 - Phi^-1(p)) of the keys.
    from scipy.stats import norm
    rng = np.random.default_rng(4)
    n = 400000
    k_idx = rng.standard_normal((n, 16))
    q_idx = np.zeros(16)
    q_idx[0] = 4.0
    s = O.indexer_scores(q_idx, k_idx)
    for p in (0.8, 0.9, 0.95):
        frac = O.top_p(s, p).count / n
        expect = norm.sf(1.0 - norm.ppf(p))
        assert abs(frac - expect) < 0.006, (p, frac, expect)


def test_topp_bruteforce():
    check_bruteforce()


def test_topp_uniform_exact():
    check_uniform_exact()


def test_topp_gaussian_closed_form():
    check_gaussian_closed_form()


def test_topp_extremes():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(50)
    assert O.top_p(s, 1.0).count == 50
    r = O.top_p(s, 1e-9)
    assert r.count == 1 and r.selected[0] == int(np.argmax(s))


def test_topp_permutation_equivariant():
    rng = np.random.default_rng(6)
    s = rng.standard_normal(300)
    perm = rng.permutation(300)
    a = O.top_p(s, 0.9).selected
    b = O.top_p(s[perm], 0.9).selected
    assert sorted(perm[b].tolist()) == a.tolist()


def test_near_threshold_rule():
    s = np.zeros(4)
    r = O.top_p(s, 0.5)
    # token 2 (cum 0.75, prob 0.25): its cumulative mass minus its own mass is
    # exactly p, so it is near the threshold; token 3 (cum 1.0) is not.
    assert O.set_ok(r, 0.5, [0, 1, 2])[0]
    assert not O.set_ok(r, 0.5, [0, 1, 2, 3])[0]
    assert O.set_ok(r, 0.5, [0])[0]          # token 1 reaches p exactly: near
    assert not O.set_ok(r, 0.5, [0, 3])[0]   # token 3 is far from the threshold
    assert O.set_ok(r, 0.5, [0, 1])[0]


# ------------------------------------------------------------------ top-k
def check_topk_rank(trials=200, seed=13):
    # rank by pairwise counting: token n is in the set iff fewer than k tokens
    # beat it (a higher score, or an equal score at an earlier position)
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(1, 40))
        s = rng.standard_normal(n) * rng.uniform(0.1, 4.0)
        if t % 3 == 0:
            s = np.round(s)                    # force ties
        k = int(rng.integers(-1, n + 3))
        res = O.top_k(s, k)
        beaten = np.array([sum(1 for m in range(n) if s[m] > s[a] or (s[m] == s[a] and m < a))
                           for a in range(n)])
        expect = np.nonzero(beaten < max(k, 1))[0]
        assert res.count == min(max(k, 1), n), (n, k, res.count)
        assert res.selected.tolist() == expect.tolist(), (s, k)


def test_topk_pairwise_rank():
    check_topk_rank()


def test_topk_extremes():
    rng = np.random.default_rng(14)
    s = np.round(rng.standard_normal(64) * 2)
    assert O.top_k(s, 1).selected.tolist() == [int(np.argmax(s))]   # argmax: first of the maxima
    assert O.top_k(s, 0).selected.tolist() == [int(np.argmax(s))]
    assert O.top_k(s, 64).count == 64 and O.top_k(s, 10 ** 6).selected.tolist() == list(range(64))


def test_topk_equals_topp_of_same_size():
    # the top-p set is a descending-score prefix, so it is the top-k set with k = |S|
    rng = np.random.default_rng(15)
    for t in range(50):
        s = rng.standard_normal(500) * rng.uniform(0.2, 3.0)
        if t % 4 == 0:
            s = np.round(s, 1)
        p = float(rng.uniform(0.05, 0.999))
        tp = O.top_p(s, p)
        assert O.top_k(s, tp.count).selected.tolist() == tp.selected.tolist()


def test_topk_shift_and_permutation():
    rng = np.random.default_rng(16)
    s = rng.standard_normal(300)
    a = O.top_k(s, 37).selected
    assert O.top_k(s + 8.0, 37).selected.tolist() == a.tolist()
    perm = rng.permutation(300)
    b = O.top_k(s[perm], 37).selected
    assert sorted(perm[b].tolist()) == a.tolist()


# ------------------------------------------------------------------ block top-p
def check_block_worked_example():
    # three full blocks with constant scores 0, 5, 1: block maxima 0, 5, 1 give
    # bins 0, 255 (the top value) and floor(256 / 5) = 51; the block masses are
    # 64 e^0, 64 e^5, 64 e^1, so block 1 alone holds e^5 / (1 + e + e^5) = 0.9756
    # and blocks 1 + 2 hold (e^5 + e) / (1 + e + e^5) = 0.9934
    s = np.concatenate([np.zeros(64), np.full(64, 5.0), np.ones(64)])
    r = O.block_top_p(s, 0.9)
    assert r.bins.tolist() == [0, 255, 51]
    assert r.blocks.tolist() == [1] and r.selected.tolist() == list(range(64, 128))
    r = O.block_top_p(s, 0.99)
    assert r.blocks.tolist() == [1, 2] and r.j_star == 51 and r.count == 128
    r = O.block_top_p(s, 0.995)
    assert r.blocks.tolist() == [0, 1, 2] and r.j_star == 0
    e = math.e
    assert abs(r.block_mass[1] / r.Z - e ** 5 / (1 + e + e ** 5)) < 1e-12
    # a block's mass is the sum over its tokens: one token at 3 and 63 at 0 carry
    # e^3 + 63 = 83.1 against 64 e^2.9 = 1162.3 for a flat block at 2.9, so at
    # p = 1/2 the top bin (block 0, 6.7 % of the mass) does not suffice
    s2 = np.concatenate([[3.0], np.zeros(63), np.full(64, 2.9)])
    r = O.block_top_p(s2, 0.5)
    assert r.bins.tolist() == [255, 0] and r.blocks.tolist() == [0, 1]
    assert abs(r.block_mass[0] / r.Z - (e ** 3 + 63) / (e ** 3 + 63 + 64 * e ** 2.9)) < 1e-12


def check_block_reduces_to_token_exact(trials=40, seed=21):
    # one-token blocks and bins far finer than the gaps between scores: the
    # histogram scan walks the tokens in descending score order, i.e. Eq. 5
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        n = int(rng.integers(1, 400))
        sc = rng.standard_normal(n) * rng.uniform(0.3, 3.0)
        p = float(rng.uniform(0.05, 0.999))
        b = O.block_top_p(sc, p, block=1, nbins=2 ** 40)
        assert b.selected.tolist() == O.top_p(sc, p).selected.tolist(), (n, p)


def test_block_topp_worked_example():
    check_block_worked_example()


def test_block_topp_reduces_to_token_exact():
    check_block_reduces_to_token_exact()


def test_block_topp_cut_is_the_highest_reaching_bin():
    # brute force over every cut: the kept blocks are those at or above the
    # highest bin whose upper-tail mass reaches p, whole blocks, the tail short
    rng = np.random.default_rng(22)
    for t in range(60):
        n = int(rng.integers(1, 1500))
        sc = rng.standard_normal(n) * rng.uniform(0.3, 3.0)
        if t % 5 == 0:
            sc = np.round(sc)
        p = float(rng.choice([0.5, 0.8, 0.9, 0.95, rng.uniform(0.01, 0.999)]))
        r = O.block_top_p(sc, p)
        tail = [r.block_mass[r.bins >= j].sum() for j in range(257)]
        reach = [j for j in range(256) if tail[j] >= p * r.Z]
        assert r.j_star == max(reach)
        assert r.blocks.tolist() == np.nonzero(r.bins >= r.j_star)[0].tolist()
        expect = [x for bb in r.blocks for x in range(64 * bb, min(64 * bb + 64, n))]
        assert r.selected.tolist() == expect
        assert r.selected.size == r.count


def test_block_topp_extremes():
    rng = np.random.default_rng(23)
    sc = rng.standard_normal(1000)
    assert O.block_top_p(sc, 1.0).count == 1000
    r = O.block_top_p(sc, 1e-9)
    assert r.blocks.tolist() == np.nonzero(r.bins == 255)[0].tolist()
    assert int(np.argmax(sc)) // 64 in r.blocks.tolist()
    flat = np.concatenate([np.full(64, 2.0)] * 5 + [np.full(10, 2.0)])
    assert O.block_top_p(flat, 0.3).count == flat.size      # one shared block max: every block
    a = O.block_top_p(sc, 0.6).count
    b = O.block_top_p(sc, 0.9).count
    assert a <= b


# ------------------------------------------------------------------ attention
def _problem(L, Hq, Hkv, ret, window, n_sink, p, dtype="f32", seed=7, decode=False, B=1):
    rng = np.random.default_rng(seed)
    R = len(ret)
    lk = [L] * B
    lq = [1] * B if decode else [L] * B
    Tq, Tk = sum(lq), sum(lk)
    q = O.round_to(rng.standard_normal((Tq, Hq, 128)), dtype)
    k = O.round_to(rng.standard_normal((Tk, Hkv, 128)), dtype)
    v = O.round_to(rng.standard_normal((Tk, Hkv, 128)), dtype)
    q_pre = O.round_to(rng.standard_normal((Tq, R, 128)), dtype)
    k_pre = O.round_to(rng.standard_normal((Tk, Hkv, 128)), dtype)
    w = rng.standard_normal((R, 16, 128)).astype(np.float32).astype(np.float64)
    return Problem(q=q, k=k, v=v, q_pre=q_pre, k_pre=k_pre, w_q=w, w_k=w,
                   cu_q=np.cumsum([0] + lq).tolist(), cu_k=np.cumsum([0] + lk).tolist(),
                   ret_heads=ret, top_p=[p] * B, window=window, n_sink=n_sink, dtype=dtype)


def check_dense_equivalence():
    L, Hq, Hkv = 40, 4, 2
    pr = _problem(L, Hq, Hkv, ret=[0, 3], window=L, n_sink=4, p=1.0)
    q = torch.from_numpy(pr.q).permute(1, 0, 2)[None]                 # [1, Hq, L, d]
    k = torch.from_numpy(pr.k).permute(1, 0, 2)[None].repeat_interleave(Hq // Hkv, dim=1)
    v = torch.from_numpy(pr.v).permute(1, 0, 2)[None].repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)[0]
    for h in range(Hq):
        for i in range(L):
            got = pr.row(0, i, h).attn.out
            assert np.allclose(got, ref[h, i].numpy(), atol=1e-12, rtol=0), (h, i)


def check_decode_dense():
    L, Hq, Hkv = 33, 4, 1
    pr = _problem(L, Hq, Hkv, ret=[1], window=L, n_sink=0, p=1.0, decode=True, B=2)
    for b in range(2):
        k0 = pr.cu_k[b]
        for h in range(Hq):
            q = torch.from_numpy(pr.q[b, h])[None, None, None]
            k = torch.from_numpy(pr.k[k0:k0 + L, 0])[None, None]
            v = torch.from_numpy(pr.v[k0:k0 + L, 0])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, 0, 0].numpy()
            assert np.allclose(pr.row(b, 0, h).attn.out, ref, atol=1e-12, rtol=0)


def test_dense_equivalence_prefill():
    check_dense_equivalence()


def test_dense_equivalence_decode():
    check_decode_dense()


def test_weights_and_closed_forms():
    pr = _problem(64, 2, 1, ret=[0], window=8, n_sink=2, p=0.9)
    for i in range(64):
        for h in range(2):
            r = pr.row(0, i, h)
            assert abs(r.attn.weights.sum() - 1.0) < 1e-12
    pr.v[:] = 1.0
    for i in range(64):
        assert np.allclose(pr.row(0, i, 0).attn.out, 1.0, atol=1e-14)
        assert np.allclose(pr.row(0, i, 1).attn.out, 1.0, atol=1e-14)
    pr2 = _problem(64, 2, 1, ret=[0], window=1, n_sink=0, p=0.9)
    for i in range(64):
        assert np.array_equal(pr2.row(0, i, 1).attn.out, pr2.v[i, 0])


def test_local_pattern_counts():
    g = _golden("local_pattern.json")
    keys = O.local_keys(100000, g["window"], g["n_sink"])
    assert keys.size == g["max_attended"]
    for pos in range(0, 40):
        kk = O.local_keys(pos, 8, 4)
        assert kk.size <= 12 and kk.max() == pos and np.all(np.diff(kk) > 0)
        assert set(range(max(0, pos - 7), pos + 1)) <= set(kk.tolist())


# ------------------------------------------------------------------ retrieval-row wiring
# The whole retrieval row at p < 1 with every operand distinct: post-RoPE q and
# pre-RoPE q_pre drawn independently, W^Q_r != W^K_r and a different pair per
# slot, two KV groups.  The expected result is written out here from the
# definition alone (section 3.4, "Low-Dimensional Projection Mechanism and
# Stage-1 Training" and "Dynamic Top-p Selection Mechanism", Eq. 5 and the
# attention equation after it): exact rational projections rounded once, exact
# rational scores, then the minimal-cardinality subset of the causal prefix
# whose softmax mass reaches p (the heaviest one when several have that size),
# found by enumerating subsets, then softmax attention of the post-RoPE q over
# it.  It shares nothing with the oracle's functions.
def _wiring_problem(dtype, decode, seed=31):
    rng = np.random.default_rng(seed)
    Hq, Hkv, ret = 4, 2, [1, 2]                    # kv(1) = 0, kv(2) = 1
    lk = [7, 10] if decode else [9]
    lq = [1] * len(lk) if decode else list(lk)
    Tq, Tk, R = sum(lq), sum(lk), len(ret)

    def draw(*shape):
        return O.round_to(rng.standard_normal(shape), dtype)
    q, q_pre = draw(Tq, Hq, 128), draw(Tq, R, 128)
    k, k_pre, v = draw(Tk, Hkv, 128), draw(Tk, Hkv, 128), draw(Tk, Hkv, 128)
    # rows of norm about 1, so that the scores have unit scale and the sets several members
    w_q = (rng.standard_normal((R, 16, 128)) / math.sqrt(128)).astype(np.float32).astype(np.float64)
    w_k = (rng.standard_normal((R, 16, 128)) / math.sqrt(128)).astype(np.float32).astype(np.float64)
    p = [0.75, 0.9] if decode else [0.8]
    return Problem(q=q, k=k, v=v, q_pre=q_pre, k_pre=k_pre, w_q=w_q, w_k=w_k,
                   cu_q=np.cumsum([0] + lq).tolist(), cu_k=np.cumsum([0] + lk).tolist(),
                   ret_heads=ret, top_p=p, window=3, n_sink=1, dtype=dtype)


def _brute_retrieval_row(raw, b, i, h):
    """Expected (q_idx, set, output) of one retrieval row from the definition."""
    bits = 8 if raw["dtype"] == "bf16" else 24
    cu_q, cu_k = raw["cu_q"], raw["cu_k"]
    Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
    pos = Lk - Lq + i
    qi, k0 = cu_q[b] + i, cu_k[b]
    Hq, Hkv = raw["q"].shape[1], raw["k"].shape[1]
    g = h * Hkv // Hq
    r = raw["ret"].index(h)

    def rdot(a, c):
        return sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, c))
    qx = [round_fraction(rdot(raw["w_q"][r, j], raw["q_pre"][qi, r]), bits) for j in range(16)]
    s = []
    for n in range(pos + 1):
        kx = [round_fraction(rdot(raw["w_k"][r, j], raw["k_pre"][k0 + n, g]), bits) for j in range(16)]
        s.append(sum(a * c for a, c in zip(qx, kx)) / 4)
    top = max(s)
    e = np.array([math.exp(float(x - top)) for x in s])
    mass = e / e.sum()
    p = raw["top_p"][b]
    best = None
    for size in range(1, pos + 2):
        for sub in itertools.combinations(range(pos + 1), size):
            m = float(sum(mass[list(sub)]))
            if m >= p and (best is None or m > best[0]):
                best = (m, sub)
        if best is not None:
            break
    S = list(best[1])
    a = [float(rdot(raw["q"][qi, h], raw["k"][k0 + n, g])) / math.sqrt(128) for n in S]
    am = max(a)
    wts = [math.exp(x - am) for x in a]
    tot = sum(wts)
    out = np.zeros(128)
    for wn, n in zip(wts, S):
        out += (wn / tot) * raw["v"][k0 + n, g]
    return np.array([float(x) for x in qx]), S, out


def check_retrieval_wiring(dtype, decode):
    pr = _wiring_problem(dtype, decode)
    raw = dict(q=pr.q, q_pre=pr.q_pre, k=pr.k, k_pre=pr.k_pre, v=pr.v, w_q=pr.w_q, w_k=pr.w_k,
               cu_q=pr.cu_q, cu_k=pr.cu_k, ret=list(pr.ret_heads), top_p=list(pr.top_p), dtype=dtype)
    nb = len(pr.cu_q) - 1
    n_strict = 0
    for b in range(nb):
        for i in range(pr.cu_q[b + 1] - pr.cu_q[b]):
            for h in pr.ret_heads:
                qx, S, out = _brute_retrieval_row(raw, b, i, h)
                got = pr.row(b, i, h)
                assert np.array_equal(got.q_idx, qx), (b, i, h, "q_idx")
                assert got.topp.selected.tolist() == S, (b, i, h, got.topp.selected.tolist(), S)
                assert np.allclose(got.attn.out, out, atol=1e-12, rtol=0), (b, i, h, "out")
                n_strict += 2 <= len(S) < pr.pos_of(b, i) + 1
    # the pin is only as good as its rows whose set is a strict subset of two or more keys
    assert n_strict >= (3 if decode else 8), n_strict


def test_retrieval_wiring_prefill_f32():
    check_retrieval_wiring("f32", decode=False)


def test_retrieval_wiring_decode_bf16():
    check_retrieval_wiring("bf16", decode=True)


# ------------------------------------------------------------------ metrics (pages' numbers)
def test_table6_compute_sparsity():
    g = _golden("table6_sparsity.json")
    for c in g["cases"]:
        att = [c["active_tokens"]] * g["n_retrieval_heads"] + \
              [g["local_attended"]] * (g["n_q_heads"] - g["n_retrieval_heads"])
        got = 100.0 * O.compute_sparsity(att, c["context"])
        assert round(got, 1) == c["compute_sparsity_pct"], (c, got)


def test_gqa_union_example():
    g = _golden("gqa_union.json")
    assert O.kv_union(g["sets"]).tolist() == g["union"]
    assert O.memory_sparsity([g["sets"]], 20) == 1.0 - 4 / 20


# ------------------------------------------------------------------ generator
def test_generator_rope_shift_invariance():
    from synth.gen import rope_inplace
    rng = np.random.default_rng(8)
    q = torch.from_numpy(rng.standard_normal((1, 1, 128)))
    k = torch.from_numpy(rng.standard_normal((1, 1, 128)))
    def score(m, n):
        a = rope_inplace(q.clone(), torch.tensor([m]), 1e6)
        b = rope_inplace(k.clone(), torch.tensor([n]), 1e6)
        return float((a * b).sum())
    for (m, n, t) in [(5, 3, 100), (1000, 10, 77777), (0, 0, 5)]:
        assert abs(score(m, n) - score(m + t, n + t)) < 1e-9


def test_generator_projection_orthonormal():
    from synth.gen import orthonormal_projection
    w = orthonormal_projection(0).numpy()
    assert np.allclose(w @ w.T, np.eye(16), atol=1e-12)


# ------------------------------------------------------------------ planted mistakes
def test_mutation_strict_threshold_caught(monkeypatch):
    real = O.top_p

    def strict(scores, p):
        r = real(scores, p)
        s = np.asarray(scores, dtype=np.float64)
        cs = np.cumsum(r.prob[r.order])
        k = min(int(np.searchsorted(cs, p, side="right")) + 1, s.size) if p < 1 else s.size
        return O.TopP(np.sort(r.order[:k]), k, r.order, r.prob, r.cum, s)
    monkeypatch.setattr(O, "top_p", strict)
    with pytest.raises(AssertionError):
        check_uniform_exact()


def test_mutation_ascending_order_caught(monkeypatch):
    real = O.top_p
    monkeypatch.setattr(O, "top_p", lambda s, p: real(-np.asarray(s), p))
    with pytest.raises(AssertionError):
        check_bruteforce(trials=40)


def test_mutation_missing_scale_caught(monkeypatch):
    monkeypatch.setattr(O, "IDX_SCALE", 1.0)
    with pytest.raises(AssertionError):
        check_gaussian_closed_form()


def test_mutation_double_rounding_caught(monkeypatch):
    monkeypatch.setattr(O, "round_to", lambda x, dt: O.round_bf16(np.asarray(x).astype(np.float32))
                        if dt == "bf16" else np.asarray(x, np.float64).astype(np.float32).astype(np.float64))
    with pytest.raises(AssertionError):
        check_single_rounding()


def test_mutation_window_off_by_one_caught(monkeypatch):
    real = O.local_keys
    monkeypatch.setattr(O, "local_keys", lambda pos, w, ns: real(pos, w + 1, ns))
    with pytest.raises(AssertionError):
        test_local_pattern_counts()


def test_mutation_attention_scale_caught(monkeypatch):
    monkeypatch.setattr(O, "HEAD_DIM", 64)
    with pytest.raises(AssertionError):
        check_dense_equivalence()


def test_mutation_topk_tie_order_caught(monkeypatch):
    # equal scores taken by descending position instead of ascending
    real = O.top_k

    def late_ties(scores, k):
        s = np.asarray(scores, dtype=np.float64)
        r = real(s[::-1], k)
        return O.TopP(np.sort(s.size - 1 - r.selected), r.count, r.order, r.prob, r.cum, s)
    monkeypatch.setattr(O, "top_k", late_ties)
    with pytest.raises(AssertionError):
        check_topk_rank(trials=60)


def test_mutation_topk_off_by_one_caught(monkeypatch):
    real = O.top_k
    monkeypatch.setattr(O, "top_k", lambda s, k: real(s, k + 1))
    with pytest.raises(AssertionError):
        check_topk_rank(trials=60)


def test_mutation_block_scan_from_bottom_caught(monkeypatch):
    # the scan walks the bins from the lowest up instead of from the highest down
    real = O.block_top_p

    def from_bottom(scores, p, block=64, nbins=256):
        neg = -np.asarray(scores, dtype=np.float64)
        r = real(neg, p, block, nbins)
        return r
    monkeypatch.setattr(O, "block_top_p", from_bottom)
    with pytest.raises(AssertionError):
        check_block_worked_example()


def test_mutation_block_crossing_bin_dropped_caught(monkeypatch):
    real = O.block_top_p

    def drop_crossing(scores, p, block=64, nbins=256):
        r = real(scores, p, block, nbins)
        if p >= 1.0:
            return r
        keep = r.blocks[r.bins[r.blocks] > r.j_star]
        n = np.asarray(scores).size
        sel = np.concatenate([np.arange(b * block, min((b + 1) * block, n)) for b in keep]) if keep.size \
            else np.zeros(0, dtype=np.int64)
        return O.BlockTopP(sel, int(sel.size), keep, r.j_star, r.block_max, r.block_mass, r.pos, r.bins, r.lo, r.hi, r.Z)
    monkeypatch.setattr(O, "block_top_p", drop_crossing)
    with pytest.raises(AssertionError):
        check_block_worked_example()


def test_mutation_block_mass_from_max_caught(monkeypatch):
    # a block's mass taken as its length times exp(its maximum) instead of the
    # sum of its tokens' masses
    real = O.block_top_p

    def mass_from_max(scores, p, block=64, nbins=256):
        sc = np.asarray(scores, dtype=np.float64)
        flat = np.concatenate([np.full(min(block, sc.size - b), sc[b:b + block].max())
                               for b in range(0, sc.size, block)])
        r = real(flat, p, block, nbins)
        return r
    monkeypatch.setattr(O, "block_top_p", mass_from_max)
    with pytest.raises(AssertionError):
        check_block_worked_example()


# mistakes in the wiring of a retrieval row: each must fail the brute-force wiring pin
def test_mutation_projects_post_rope_query_caught(monkeypatch):
    monkeypatch.setattr(Problem, "q_pre_row", lambda self, qi, r: self.q_row(qi, self.ret_heads[r]))
    with pytest.raises(AssertionError):
        check_retrieval_wiring("f32", decode=False)


def test_mutation_attends_with_pre_rope_query_caught(monkeypatch):
    real = O.retrieval_row
    monkeypatch.setattr(O, "retrieval_row", lambda q, q_pre, *a, **kw: real(q_pre, q_pre, *a, **kw))
    with pytest.raises(AssertionError):
        check_retrieval_wiring("f32", decode=False)


def test_mutation_swapped_projections_caught(monkeypatch):
    real = Problem.w
    monkeypatch.setattr(Problem, "w", lambda self, which, r: real(self, {"w_q": "w_k", "w_k": "w_q"}[which], r))
    with pytest.raises(AssertionError):
        check_retrieval_wiring("bf16", decode=True)


def test_mutation_slot0_projection_for_every_slot_caught(monkeypatch):
    real = Problem.w
    monkeypatch.setattr(Problem, "w", lambda self, which, r: real(self, which, 0))
    with pytest.raises(AssertionError):
        check_retrieval_wiring("bf16", decode=True)


def test_mutation_wrong_kv_group_caught(monkeypatch):
    monkeypatch.setattr(Problem, "kv_of", lambda self, h: h % self.n_kv_heads)
    with pytest.raises(AssertionError):
        check_retrieval_wiring("f32", decode=False)


def test_mutation_keys_projected_with_query_matrix_caught(monkeypatch):
    # only the key side is wrong (W^Q_r applied to k_pre): q_idx is still right, so the
    # set or the output has to catch it
    real = Problem.w
    monkeypatch.setattr(Problem, "w", lambda self, which, r: real(self, "w_q", r))
    with pytest.raises(AssertionError, match=r"\[|out"):
        check_retrieval_wiring("f32", decode=False)
