"""Pins of the CPU oracle against closed forms, invariants and brute force.

The pages print no worked example of the decode step, so each pin is a
special case whose exact answer follows from mathematics (tests/golden/
closed_forms.txt holds the constants), an invariant the definition implies,
or an integer brute force.  They are chosen so a plausible slip in the oracle
(a dropped term, a wrong sign, index or scale, a transposed operand, a
swapped operand) fails at least one of them.
"""
import math

import numpy as np
import pytest

from conftest import golden
from oracle import bf16_to_f32
from oracle import lo as L
from synth import workloads as W


def bf16_exact(a):
    """bf16 bits of values that bf16 represents exactly."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def small_shape(**kw):
    s = dict(W.TINY)
    s.update(kw)
    return s


# ------------------------------------------------------------------ bf16

def test_bf16_round_to_nearest_even(orc):
    assert orc.bf16_round(1.0) == 0x3F80
    assert orc.bf16_round(1.0 + 2 ** -8) == 0x3F80          # tie -> even (…80)
    assert orc.bf16_round(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (…82)
    assert orc.bf16_round(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81  # just above the tie
    assert orc.bf16_round(-2.0) == 0xC000
    assert orc.bf16_round(3.140625) == 0x4049
    assert orc.bf16_widen(0x4049) == 3.140625
    assert orc.bf16_widen(0xBF80) == -1.0


# ------------------------------------------------------------- generator

def test_generator_matches_python_mirror(orc):
    shape = small_shape()
    m = orc.model(shape, seed=W.SEED_WEIGHTS, w_std=0.02)
    kap = W.kappa(0.02)
    cases = [(L.W_EMBED, 0, W.T_EMBED), (L.W_Q, 0, W.t_layer(0, W.K_WQ)),
             (L.W_DOWN, 1, W.t_layer(1, W.K_WD)), (L.W_LM_HEAD, 0, W.T_LM_HEAD),
             (L.W_GATE, 1, W.t_layer(1, W.K_WG))]
    rng = np.random.default_rng(0)
    for kind, layer, tensor in cases:
        w = m.weight(kind, layer)
        k = W.key(W.SEED_WEIGHTS, tensor)
        for idx in rng.integers(0, w.size, 40):
            assert int(w.flat[idx]) == W.normal_bf16(k, int(idx), kap)
    # norm gains are 1.0
    assert np.all(m.weight(L.W_ATTN_NORM, 1) == 0x3F80)
    assert np.all(m.weight(L.W_FINAL_NORM) == 0x3F80)


def test_generator_kv_matches_python_mirror(orc):
    shape = small_shape()
    kv = orc.kv(shape, 2, 64, seed=W.SEED_KV, kv_std=1.0, prefill=[40, 7])
    kap = W.kappa(1.0)
    d, nkv = shape["head_dim"], shape["n_kv_heads"]
    for layer, b, h, pos, i in [(0, 0, 0, 0, 0), (1, 0, 1, 39, 63), (0, 1, 1, 6, 5)]:
        idx = W.kv_index(b, nkv, h, pos, d, i)
        assert int(kv.k(layer, b, h)[pos, i]) == W.normal_bf16(W.key(W.SEED_KV, W.t_kcache(layer)),
                                                               idx, kap)
        assert int(kv.v(layer, b, h)[pos, i]) == W.normal_bf16(W.key(W.SEED_KV, W.t_vcache(layer)),
                                                               idx, kap)
    # beyond the prefill length nothing is written
    assert np.all(kv.k(0, 1, 0)[7:] == 0)


def test_generator_moments(orc):
    shape = small_shape()
    m = orc.model(shape, seed=W.SEED_WEIGHTS, w_std=0.02)
    w = bf16_to_f32(m.weight(L.W_GATE, 0)).astype(np.float64)  # 196,608 samples
    n = w.size
    assert abs(w.mean()) < 4 * 0.02 / math.sqrt(n)
    assert abs(w.std() / 0.02 - 1) < 0.01
    # Irwin-Hall(4) support: |z| <= 131070 -> |w| <= sqrt(3) * 2 * sigma (plus bf16 rounding)
    assert np.abs(w).max() <= 0.02 * 2 * math.sqrt(3) * 1.01
    # excess kurtosis of Irwin-Hall(4) is -1.2/4 = -0.3
    kurt = ((w - w.mean()) ** 4).mean() / w.var() ** 2 - 3
    assert abs(kurt + 0.3) < 0.05


def test_uniform_ints_in_range():
    toks = W.first_tokens(64, 1024)
    assert all(0 <= t < 1024 for t in toks) and len(set(toks)) > 50
    lens = W.kv_lengths(64, 256, 1024)
    assert all(256 <= x <= 1024 for x in lens) and len(set(lens)) > 50


# ---------------------------------------------------------------- matvec

@pytest.mark.parametrize("rows,cols", [(1, 1), (5, 7), (13, 3), (64, 130), (3, 1000)])
def test_matvec_integer_brute_force(orc, rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    Wi = rng.integers(-8, 9, size=(rows, cols))
    xi = rng.integers(-16, 17, size=cols)
    y = orc.matvec(bf16_exact(Wi.astype(np.float32)), xi.astype(np.float32))
    expect = [sum(int(Wi[r, c]) * int(xi[c]) for c in range(cols)) for r in range(rows)]
    assert np.array_equal(y, np.array(expect, dtype=np.float32))  # |sums| < 2^24: exact


def test_matvec_row_major_not_transposed(orc):
    # W = [[1, 2, 3], [4, 5, 6]] (2x3): W x with x = (1, 10, 100) is (321, 654)
    Wb = bf16_exact(np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float32))
    y = orc.matvec(Wb, [1, 10, 100])
    assert list(y) == [321.0, 654.0]


# --------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_form_with_large_eps(orc64):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(300) * 3
    eps = 0.5
    out = orc64.rmsnorm(x, None, eps)
    m = np.mean(x ** 2)
    # out = x / sqrt(m + eps)  =>  mean(out^2) = m / (m + eps)
    assert abs(np.mean(out ** 2) - m / (m + eps)) < 1e-12
    assert np.allclose(out * math.sqrt(m + eps), x, rtol=1e-12, atol=0)


def test_rmsnorm_unit_rms_and_gain(orc):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(256) * 5).astype(np.float32)
    out = orc.rmsnorm(x, None, 1e-5)
    m = float(np.mean(x.astype(np.float64) ** 2))
    assert abs(float(np.mean(out.astype(np.float64) ** 2)) - m / (m + 1e-5)) < 2e-6
    # gains multiply elementwise (powers of two: exact)
    g = np.array([0.5, 1.0, 2.0, 4.0] * 64, dtype=np.float32)
    out_g = orc.rmsnorm(x, bf16_exact(g), 1e-5)
    assert np.array_equal(out_g, out * g)


def test_rmsnorm_scale_invariant_at_zero_eps(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(128).astype(np.float32)
    assert np.array_equal(orc.rmsnorm(x, None, 0.0), orc.rmsnorm(4 * x, None, 0.0))


# ------------------------------------------------------------------ RoPE

def test_rope_identity_at_position_zero(orc):
    h = np.random.default_rng(4).standard_normal(64).astype(np.float32)
    assert np.array_equal(orc.rope(h, 0, 500000.0), h)


def test_rope_pair0_turns_by_p_radians(orc):
    d = 64
    h = np.zeros(d, dtype=np.float32)
    h[0] = 1.0
    r = orc.rope(h, 1, 10000.0)
    assert r[0] == np.float32(golden("cos_1"))
    assert r[d // 2] == np.float32(golden("sin_1"))   # sign fixes the direction
    assert np.count_nonzero(r) == 2


def test_rope_frequency_of_channel_quarter(orc):
    # theta = 10^4, d = 64, channel i = 16: frequency 10^4^(-2*16/64) = 0.01,
    # so at p = 100 the pair (16, 48) turns by exactly 1 radian.
    d = 64
    h = np.zeros(d, dtype=np.float32)
    h[16] = 1.0
    r = orc.rope(h, 100, 10000.0)
    assert abs(r[16] - golden("cos_1")) < 1e-7
    assert abs(r[48] - golden("sin_1")) < 1e-7


def test_rope_preserves_pair_norms(orc64):
    h = np.random.default_rng(5).standard_normal(128)
    r = orc64.rope(h, 12345, 500000.0)
    n0 = h[:64] ** 2 + h[64:] ** 2
    n1 = r[:64] ** 2 + r[64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-13)


@pytest.mark.parametrize("kind,tol", [("f32", 2e-5), ("f64", 1e-12)])
def test_rope_relative_position(kind, tol, orc, orc64):
    o = orc if kind == "f32" else orc64
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    p, s, delta = 37, 5, 211
    a = float(np.dot(o.rope(q, p, 10000.0).astype(np.float64), o.rope(k, s, 10000.0)))
    b = float(np.dot(o.rope(q, p + delta, 10000.0).astype(np.float64),
                     o.rope(k, s + delta, 10000.0)))
    assert abs(a - b) <= tol * math.sqrt(np.dot(q, q) * np.dot(k, k))


# --------------------------------------------------------------- softmax

def test_softmax_properties(orc):
    rng = np.random.default_rng(7)
    s = (rng.standard_normal(333) * 4).astype(np.float32)
    p = orc.softmax(s)
    assert abs(float(p.astype(np.float64).sum()) - 1.0) < 1e-6
    assert np.allclose(orc.softmax(s + 17.0), p, rtol=1e-5, atol=1e-9)  # shift invariance
    assert np.all(orc.softmax(np.full(64, 3.0)) == np.float32(1 / 64))  # equal scores
    two = orc.softmax([0.0, math.log(3.0)])
    assert abs(two[0] - 0.25) < 1e-7 and abs(two[1] - 0.75) < 1e-7


# ------------------------------------------------------------- attention

def test_attention_length_one_returns_v_exactly(orc):
    rng = np.random.default_rng(8)
    q = rng.standard_normal(64)
    K = orc_bf16_random(rng, (1, 64))
    V = orc_bf16_random(rng, (1, 64))
    out = orc.attention_head(q, K, V)
    assert np.array_equal(out, bf16_to_f32(V[0]))


def orc_bf16_random(rng, shape):
    a = rng.standard_normal(shape).astype(np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def test_attention_two_positions_scale(orc):
    # q = 8 e0, K0 = e0, K1 = 0, d = 64: scores (8/sqrt(64), 0) = (1, 0), so
    # the weight of position 0 is sigmoid(1); V0 = 1, V1 = 0.
    d = 64
    q = np.zeros(d)
    q[0] = 8.0
    K = np.zeros((2, d), dtype=np.float32)
    K[0, 0] = 1.0
    V = np.zeros((2, d), dtype=np.float32)
    V[0, :] = 1.0
    out = orc.attention_head(q, bf16_exact(K), bf16_exact(V))
    assert np.allclose(out, golden("sigmoid_1"), atol=2e-7)


def test_attention_constant_and_uniform(orc):
    rng = np.random.default_rng(9)
    d, n = 64, 100
    K = orc_bf16_random(rng, (n, d))
    Vc = bf16_exact(np.full((n, d), 0.75, dtype=np.float32))
    out = orc.attention_head(rng.standard_normal(d), K, Vc)
    assert np.allclose(out, 0.75, atol=1e-6)
    V = orc_bf16_random(rng, (n, d))
    out = orc.attention_head(np.zeros(d), K, V)  # all scores 0: mean of V rows
    assert np.allclose(out, bf16_to_f32(V).astype(np.float64).mean(0), atol=1e-6)


# ------------------------------------------------------------------ SiLU

def test_silu_closed_forms(orc):
    assert orc.silu(0.0) == 0.0
    assert abs(orc.silu(1.0) - golden("sigmoid_1")) < 1e-7
    assert abs(orc.silu(2.0) - 2 * golden("sigmoid_2")) < 2e-7
    assert abs(orc.silu(30.0) - 30.0) < 1e-5
    assert abs(orc.silu(-30.0)) < 1e-10
    xs = np.linspace(-3, 0, 30001)
    ys = np.array([orc.silu(x) for x in xs])
    i = int(np.argmin(ys))
    assert abs(xs[i] - golden("silu_argmin")) < 2e-3
    assert abs(ys[i] - golden("silu_min")) < 1e-6


def test_swiglu_applies_silu_to_gate(orc):
    # xn = (1, 0); gate rows give a = (2, -1, 0.5), up rows give u = (3, 4, -2)
    Wg = bf16_exact(np.array([[2, 0], [-1, 7], [0.5, 3]], dtype=np.float32))
    Wu = bf16_exact(np.array([[3, 5], [4, 1], [-2, 9]], dtype=np.float32))
    h = orc.swiglu(Wg, Wu, [1.0, 0.0])
    assert abs(h[0] - 6 * golden("sigmoid_2")) < 1e-6       # silu(2) * 3
    expect1 = -1 / (1 + math.exp(1)) * 4                       # silu(-1) * 4
    expect2 = 0.5 / (1 + math.exp(-0.5)) * -2                  # silu(0.5) * -2
    assert abs(h[1] - expect1) < 1e-6 and abs(h[2] - expect2) < 1e-6


def test_argmax_lowest_index_on_ties(orc):
    assert orc.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert orc.argmax([5.0]) == 0
    assert orc.argmax([-1.0, -1.0]) == 0
    assert orc.argmax([0.0, 0.0, 1e-30]) == 2


# ------------------------------------------------------------ whole step

def _zero(m, kind, layers):
    for l in layers:
        m.weight(kind, l)[:] = 0


def test_step_identity_layers_tied_closed_form(orc):
    # Wo = Wd = 0 makes every layer an identity, so logits = E n(E[tok]);
    # with gains 1: logits[tok] = |e|^2 / sqrt(|e|^2/H + eps).
    shape = small_shape(tied=1)
    m = orc.model(shape, seed=1, w_std=0.02)
    _zero(m, L.W_O, range(2))
    _zero(m, L.W_DOWN, range(2))
    kv = orc.kv(shape, 1, 256, seed=2, prefill=[128])
    tok = 77
    logits, nxt = orc.decode_step(m, kv, [tok], [128])
    E = bf16_to_f32(m.weight(L.W_EMBED)).astype(np.float64)
    e = E[tok]
    ss = float(e @ e)
    r = 1 / math.sqrt(ss / shape["hidden"] + 1e-5)
    assert abs(logits[0, tok] - ss * r) < 1e-5 * ss * r
    assert np.allclose(logits[0], E @ e * r, atol=1e-5)
    assert nxt[0] == int(np.argmax(logits[0]))


def test_step_untied_uses_lm_head(orc):
    shape = small_shape(tied=0)
    m = orc.model(shape, seed=1, w_std=0.02)
    _zero(m, L.W_O, range(2))
    _zero(m, L.W_DOWN, range(2))
    kv = orc.kv(shape, 1, 256, seed=2, prefill=[128])
    logits, _ = orc.decode_step(m, kv, [5], [128])
    e = bf16_to_f32(m.weight(L.W_EMBED)[5]).astype(np.float64)
    xf = e / math.sqrt(e @ e / shape["hidden"] + 1e-5)
    Wlm = bf16_to_f32(m.weight(L.W_LM_HEAD)).astype(np.float64)
    assert np.allclose(logits[0], Wlm @ xf, atol=1e-5)
    E = bf16_to_f32(m.weight(L.W_EMBED)).astype(np.float64)
    assert not np.allclose(logits[0], E @ xf, atol=1e-3)


def test_step_attention_range_append_and_gqa(orc):
    # One layer.  Wq = 0 makes every score 0, so each head's output is the mean
    # of its KV head's V rows over positions 0..p inclusive; Wv = 0 appends a
    # zero V row at p.  Heads 0,1 read KV head 0 and heads 2,3 KV head 1.
    shape = small_shape(n_layers=1)
    m = orc.model(shape, seed=1, w_std=0.02)
    _zero(m, L.W_Q, [0])
    _zero(m, L.W_V, [0])
    p = 50
    kv = orc.kv(shape, 1, 128, seed=2, prefill=[p])
    tr = orc.trace(shape, 0, 0)
    orc.decode_step(m, kv, [9], [p], trace=tr)
    d = shape["head_dim"]
    for hq in range(4):
        Vc = bf16_to_f32(kv.v(0, 0, hq // 2)[:p + 1]).astype(np.float64)
        assert np.all(Vc[p] == 0)
        assert np.allclose(tr["o"][hq * d:(hq + 1) * d], Vc.sum(0) / (p + 1), atol=1e-6)
    # new K at slot p is bf16 of the rotated k; later slots untouched
    for hk in range(2):
        Kc = kv.k(0, 0, hk)
        expect = [orc.bf16_round(float(x)) for x in tr["k"][hk * d:(hk + 1) * d]]
        assert list(Kc[p]) == expect
        assert np.all(Kc[p + 1:] == 0)


def test_step_residuals_and_mlp_structure(orc):
    # One layer, H = n_q*d = 256.  Wo = I gives x_attn = x + o exactly; the
    # MLP reads n(x_attn); Wg = [I; 0], Wu = [2I; 0] give hh_i = silu(xn2_i)*2*xn2_i
    # for i < H and 0 above; Wd = [I | 0] gives x_out = x_attn + hh[:H] exactly.
    shape = small_shape(n_layers=1)
    H, I = shape["hidden"], shape["intermediate"]
    m = orc.model(shape, seed=1, w_std=0.02)
    eye = np.eye(H, dtype=np.float32)
    m.weight(L.W_O, 0)[:] = bf16_exact(eye)
    m.weight(L.W_GATE, 0)[:] = bf16_exact(np.vstack([eye, np.zeros((I - H, H), np.float32)]))
    m.weight(L.W_UP, 0)[:] = bf16_exact(np.vstack([2 * eye, np.zeros((I - H, H), np.float32)]))
    m.weight(L.W_DOWN, 0)[:] = bf16_exact(np.hstack([eye, np.zeros((H, I - H), np.float32)]))
    kv = orc.kv(shape, 1, 64, seed=2, prefill=[20])
    tr = orc.trace(shape, 0, 0)
    tok = 3
    orc.decode_step(m, kv, [tok], [20], trace=tr)
    x = bf16_to_f32(m.weight(L.W_EMBED)[tok])
    assert np.array_equal(tr["x_attn"], x + tr["o"])
    xa = tr["x_attn"].astype(np.float64)
    xn2 = xa / math.sqrt(xa @ xa / H + 1e-5)
    assert np.allclose(tr["xn2"], xn2, atol=1e-6)
    s = tr["xn2"].astype(np.float64)
    assert np.allclose(tr["hh"][:H], s / (1 + np.exp(-s)) * 2 * s, atol=1e-6)
    assert np.all(tr["hh"][H:] == 0)
    assert np.array_equal(tr["x_out"], tr["x_attn"] + tr["hh"][:H])


def test_step_batch_independence(orc):
    shape = small_shape()
    m = orc.model(shape, seed=1, w_std=0.02)
    kv2 = orc.kv(shape, 2, 256, seed=2, prefill=[130, 140])
    kv1 = orc.kv(shape, 2, 256, seed=2, prefill=[130, 140])
    l2, _ = orc.decode_step(m, kv2, [11, 500], [130, 140])
    l1, _ = orc.decode_step(m, kv1, [11], [130])
    assert np.array_equal(l2[0], l1[0])


def test_step_deterministic(orc):
    shape = small_shape()
    m = orc.model(shape, seed=1, w_std=0.02)
    outs = []
    for _ in range(2):
        kv = orc.kv(shape, 1, 256, seed=2, prefill=[128])
        outs.append(orc.decode_step(m, kv, [42], [128])[0])
    assert np.array_equal(outs[0], outs[1])


def test_step_float_build_matches_double_build(orc, orc64):
    # The float oracle's own rounding, 16 teacher-forced greedy steps of the
    # tiny workload: relative L2 of the logits <= 1e-5 against the double build.
    shape = small_shape()
    m32 = orc.model(shape, seed=1, w_std=0.02)
    m64 = orc64.model(shape, seed=1, w_std=0.02)
    kv32 = orc.kv(shape, 1, 256, seed=2, prefill=[128])
    kv64 = orc64.kv(shape, 1, 256, seed=2, prefill=[128])
    tok = W.first_tokens(1, shape["vocab"])[0]
    for step in range(16):
        l32, _ = orc.decode_step(m32, kv32, [tok], [128 + step])
        l64, n64 = orc64.decode_step(m64, kv64, [tok], [128 + step])
        rel = np.linalg.norm(l32 - l64) / np.linalg.norm(l64)
        assert rel <= 1e-5, (step, rel)
        tok = int(n64[0])


def _score_from_mass(o_marker, mass_rest, n_rest):
    """Softmax score recovered from attention outputs: n_rest positions score 0
    (K = 0) and carry V = e_1, so o_1 = n_rest / Z; a position whose V is e_0
    has weight o_0 = e^s / Z, hence s = ln(o_0 * n_rest / o_1)."""
    return math.log(float(o_marker) * n_rest / float(mass_rest))


def test_step_rope_applied_to_q_and_k_at_the_position(orc):
    # One layer.  q head 0 and kv head 0 share one weight row in channel 0 and
    # every other Q/K/V row is zero, so before rotation q = k = c e_0: only the
    # pair (0, d/2) is non-zero, and it turns by exactly p radians (frequency
    # theta^0 = 1).  The cache holds K = 0 and V = e_1 at positions 0..p-1.
    #  - step at p: the new key must score |q|^2 / sqrt(d) (a rotation keeps
    #    the product of q and k at equal positions), and the stored key must
    #    point at angle p;
    #  - step at p + 1 with the same token (same c), reading the key stored at
    #    p: that key must score cos(1) |q|^2 / sqrt(d), the new one |q|^2 / sqrt(d).
    # A key left unrotated scores cos(p) |q|^2 / sqrt(d) (p = 20: 0.41), a q or
    # k rotated at p +- 1 changes the angle of the stored key or the relative
    # score, so each such slip fails one of the checks below.
    shape = small_shape(n_layers=1)
    d, H = shape["head_dim"], shape["hidden"]
    m = orc.model(shape, seed=1, w_std=0.02)
    for kind in (L.W_Q, L.W_K, L.W_V):
        m.weight(kind, 0)[:] = 0
    p, tok = 20, 7
    # probe: the normalised layer input (independent of the Q/K/V weights)
    probe = orc.trace(shape, 0, 0)
    orc.decode_step(m, orc.kv(shape, 1, 64, seed=2, prefill=[p]), [tok], [p], trace=probe)
    xn = probe["xn"].astype(np.float64)
    j = int(np.argmax(np.abs(xn)))
    row = np.zeros(H, dtype=np.float32)
    row[j] = 4.0 / xn[j]  # c = row . xn close to 4, so |q|^2 / sqrt(d) is about 2
    row = bf16_to_f32(np.array([orc.bf16_round(float(v)) for v in row], dtype=np.uint16))
    m.weight(L.W_Q, 0)[0] = bf16_exact(row)
    m.weight(L.W_K, 0)[0] = bf16_exact(row)
    kv = orc.kv(shape, 1, 64, seed=2, prefill=[p])
    one = orc.bf16_round(1.0)
    for h in range(shape["n_kv_heads"]):
        kv.k(0, 0, h)[:] = 0
        kv.v(0, 0, h)[:] = 0
        kv.v(0, 0, h)[:p, 1] = one
    scale = 1 / math.sqrt(d)

    tr = orc.trace(shape, 0, 0)
    orc.decode_step(m, kv, [tok], [p], trace=tr)
    q = tr["q"][:d].astype(np.float64)
    assert np.count_nonzero(q) == 2 and q[0] != 0 and q[d // 2] != 0
    q2 = float(q @ q)
    # stored key: angle p (mod 2 pi), length |q| (to bf16 rounding)
    kp = bf16_to_f32(kv.k(0, 0, 0)[p]).astype(np.float64)
    assert np.count_nonzero(kp) == 2
    ang = math.atan2(kp[d // 2], kp[0])
    assert abs(math.remainder(ang - p, 2 * math.pi)) < 1e-2
    assert abs(math.hypot(kp[0], kp[d // 2]) ** 2 / q2 - 1) < 1e-2
    # the new key at the same position: |q|^2 / sqrt(d)
    o = tr["o"][:d].astype(np.float64)
    w_new = 1.0 - o[1]  # V at p is zero (Wv = 0): the rest of the mass is p's
    s_same = math.log(w_new * p / o[1])
    assert abs(s_same / (q2 * scale) - 1) < 1e-2, (s_same, q2 * scale)

    # next step, same token: mark the row stored at p with V = e_0
    kv.v(0, 0, 0)[p, :] = 0
    kv.v(0, 0, 0)[p, 0] = one
    tr2 = orc.trace(shape, 0, 0)
    orc.decode_step(m, kv, [tok], [p + 1], trace=tr2)
    o2 = tr2["o"][:d].astype(np.float64)
    q2b = float(tr2["q"][:d].astype(np.float64) @ tr2["q"][:d].astype(np.float64))
    assert abs(q2b / q2 - 1) < 1e-6  # same token, same |q|
    s_prev = _score_from_mass(o2[0], o2[1], p)
    s_new = math.log((1.0 - o2[0] - o2[1]) * p / o2[1])
    assert abs(s_prev / (golden("cos_1") * q2 * scale) - 1) < 1e-2, (s_prev, q2 * scale)
    assert abs(s_new / (q2 * scale) - 1) < 1e-2, (s_new, q2 * scale)
