"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these compare the oracle with itself: each checks a closed form, an
invariant, a library routine (torch's own bf16 / fp8 casts), a printed figure
or a brute-force count on tiny inputs, chosen so that a dropped term, a wrong
sign or index, or a transposed operand in the oracle fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import get_config, flash_ratio as wl_flash_ratio

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch_rne():
    x32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        np.array([1e-40, -3e-39, 3.3e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32),
    ])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = O.bf16_round(x32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    # encode / decode round trip on the bit level
    bits = O.bf16_encode(x32.astype(np.float64))
    np.testing.assert_array_equal(O.bf16_decode(bits), ref)


def test_bf16_round_is_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-30 is just above the bf16 midpoint; rounding through
    # float32 first would land on the midpoint and round to even (1.0).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert O.bf16_round(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert O.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0


def test_e4m3_table_against_ocp_fixture():
    g = json.load(open(os.path.join(GOLD, "e4m3_ocp_codes.json")))
    for code, val in g["codes"].items():
        v = O.e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        assert v == val and math.copysign(1, v) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert np.isnan(O.e4m3_decode(np.array([int(code, 16)], np.uint8))[0])
    for x, code, why in g["rne_cases"]:
        assert O.e4m3_encode(np.array([x]))[0] == int(code, 16), why


def test_e4m3_all_codes_round_trip_and_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    np.testing.assert_array_equal(O.e4m3_encode(vals[finite]), codes[finite])
    tv = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    np.testing.assert_array_equal(vals[finite], tv[finite].astype(np.float64))
    assert np.nanmax(vals) == 448.0
    # random in-range values: encode agrees with torch's RNE cast
    x = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-3, 2.6, 50000)).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(x.astype(np.float64)), ref)


def test_fp8_row_record_layout_and_scale():
    d, n_rot = 512, 64
    z = rng.standard_normal(d) * 3
    rec, val = O.encode_row(z, "e4m3", d, n_rot)
    assert rec.size == 640
    dn = d - n_rot
    s = rec[dn + 128:dn + 132].copy().view(np.float32)[0]
    assert s == np.float32(np.max(np.abs(z[:dn])) / 448.0)
    # the largest non-RoPE channel lands on the top code
    j = int(np.argmax(np.abs(z[:dn])))
    assert rec[j] & 0x7F == 0x7E
    # tail is the bf16 value of the input, untouched by the scale
    np.testing.assert_array_equal(val[dn:], O.bf16_round(z[dn:]))
    assert np.max(np.abs(val[:dn] - z[:dn]) / np.max(np.abs(z[:dn]))) <= 2.0 ** -4
    np.testing.assert_array_equal(O.decode_rows(rec, "e4m3", d, n_rot), val)
    # all-zero non-RoPE part -> scale 1
    rec0, _ = O.encode_row(np.zeros(d), "e4m3", d, n_rot)
    assert rec0[dn + 128:dn + 132].copy().view(np.float32)[0] == 1.0


# ---------------------------------------------------------------------------
# RoPE on the tail only
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,n_rot,base", [(512, 64, 160000.0), (128, 64, 10000.0), (64, 64, 160000.0)])
def test_rope_tail_invariants(d, n_rot, base):
    x = rng.standard_normal((5, d))
    p = 123457
    y = O.rope_tail(x, p, base, n_rot)
    dn = d - n_rot
    np.testing.assert_array_equal(y[:, :dn], x[:, :dn])                  # head untouched
    n_x = x[:, dn:].reshape(5, -1, 2)
    n_y = y[:, dn:].reshape(5, -1, 2)
    np.testing.assert_allclose(np.hypot(n_y[..., 0], n_y[..., 1]),
                               np.hypot(n_x[..., 0], n_x[..., 1]), rtol=1e-13)
    np.testing.assert_array_equal(O.rope_tail(x, 0, base, n_rot), x)      # position 0
    np.testing.assert_allclose(O.rope_tail(O.rope_tail(x, 777, base, n_rot), 1234, base, n_rot),
                               O.rope_tail(x, 2011, base, n_rot), atol=1e-12)
    np.testing.assert_allclose(O.rope_tail(y, -p, base, n_rot), x, atol=1e-10)
    # relative position: <R(p) a, R(s) b> depends on p - s only
    a, b = rng.standard_normal(d), rng.standard_normal(d)
    s1 = O.rope_tail(a, 1000, base, n_rot) @ O.rope_tail(b, 937, base, n_rot)
    s2 = O.rope_tail(a, 5063, base, n_rot) @ O.rope_tail(b, 5000, base, n_rot)
    assert abs(s1 - s2) < 1e-9


def test_rope_pair_rotation_closed_form():
    # pair j = 0 turns by exactly pos radians; the last pair by pos * base^(-(n_rot-2)/n_rot)
    d, n_rot, base = 128, 64, 10000.0
    for j, theta in ((0, 1.0), (n_rot // 2 - 1, base ** (-(n_rot - 2) / n_rot)), (16, base ** -0.5)):
        x = np.zeros(d)
        x[d - n_rot + 2 * j] = 1.0
        y = O.rope_tail(x, 3, base, n_rot)
        assert abs(y[d - n_rot + 2 * j] - math.cos(3 * theta)) < 1e-13
        assert abs(y[d - n_rot + 2 * j + 1] - math.sin(3 * theta)) < 1e-13
        assert np.count_nonzero(y) <= 2


# ---------------------------------------------------------------------------
# compressor pooling and norm
# ---------------------------------------------------------------------------

def _linear_history_layer(ratio, width=8, relu=True):
    """Layer whose kappa_t = (t + 1) * v and sigma_t = 0 (hidden size 1)."""
    v = np.linspace(-1.0, 2.0, width)
    L = O.OracleLayer(ratio=ratio, head_dim=width, n_heads=1, idx_heads=0, idx_dim=0, top_k=0,
                      n_rot=2, swa=128, rope_base=10000.0, norm_eps=1e-6, kv_fmt="f32",
                      idx_fmt="f32", act_fmt="f32")
    L.wkv = v[:, None].copy()
    L.wgate = np.zeros((width, 1))
    L.ape = np.zeros((L.window, width))
    L.gamma = np.ones(width)
    return L, v


@pytest.mark.parametrize("ratio", [4, 128])
def test_uniform_scores_reduce_pooling_to_mean(ratio):
    L, v = _linear_history_layer(ratio)
    seq = O.OracleSequence(L)
    n = 3 * ratio + 5
    seq.feed(0, np.arange(1, n + 1, dtype=np.float32)[:, None], np.zeros((n, 8), np.float32))
    for i in range((n) // ratio):
        y = seq.pooled(i)
        if ratio == 4:
            mean = 2.5 if i == 0 else 4 * i + 0.5
        else:
            mean = 128 * i + 64.5
        np.testing.assert_allclose(y, mean * v, rtol=1e-12, atol=1e-12)


def test_ape_slot_order_picks_window_ends():
    # a dominant APE bias on one slot makes the row that slot's token
    L, v = _linear_history_layer(4)
    seq = O.OracleSequence(L)
    seq.feed(0, np.arange(1, 33, dtype=np.float32)[:, None], np.zeros((32, 8), np.float32))
    for slot, tok_of_row in ((7, lambda i: 4 * i + 3), (0, lambda i: 4 * i - 4), (4, lambda i: 4 * i)):
        L.ape = np.zeros((8, 8))
        L.ape[slot] = 60.0
        for i in (1, 2, 5):
            np.testing.assert_allclose(seq.pooled(i), (tok_of_row(i) + 1) * v, rtol=1e-12)
    # row 0: slots 0-3 hold no token; a bias there must not select anything
    L.ape = np.zeros((8, 8))
    L.ape[0] = 60.0
    np.testing.assert_allclose(seq.pooled(0), 2.5 * v, rtol=1e-12)


def test_pooling_invariants():
    W, c = 8, 16
    kap = rng.standard_normal((W, c))
    sc = rng.standard_normal((W, c)) * 3
    y = O.softmax_pool(kap, sc)
    # shift of the scores per channel does not matter
    np.testing.assert_allclose(O.softmax_pool(kap, sc + rng.standard_normal(c) * 50), y, rtol=1e-11, atol=1e-12)
    # convex combination per channel
    assert np.all(y <= kap.max(0) + 1e-12) and np.all(y >= kap.min(0) - 1e-12)
    # two-slot closed form: weight sigmoid(s0 - s1)
    k2 = np.array([[1.0], [3.0]])
    s2 = np.array([[0.7], [-0.4]])
    w0 = 1 / (1 + math.exp(-(0.7 + 0.4)))
    assert abs(O.softmax_pool(k2, s2)[0] - (w0 * 1 + (1 - w0) * 3)) < 1e-14


def test_rmsnorm_closed_form():
    y = rng.standard_normal((4, 64)) * rng.uniform(0.01, 10, (4, 1))
    gamma = rng.uniform(0.5, 1.5, 64)
    eps = 1e-6
    z = O.rmsnorm(y, gamma, eps)
    rms = np.sqrt(np.mean((z / gamma) ** 2, axis=1))
    np.testing.assert_allclose(rms, (1 + eps / np.mean(y * y, axis=1)) ** -0.5, rtol=1e-12)
    # direction preserved channel-wise: z / gamma is a positive multiple of y
    ratio = (z / gamma) / y
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones_like(ratio), rtol=1e-12)


def _small_layer(ratio, d=16, D=12, DI=8, n_rot=4, fmt="f32", seed=0):
    r = np.random.default_rng(seed)
    W = {4: 8, 128: 128}.get(ratio, 0)
    L = O.OracleLayer(ratio=ratio, head_dim=d, n_heads=3, idx_heads=2, idx_dim=DI, top_k=4,
                      n_rot=n_rot, swa=128, rope_base=10000.0, norm_eps=1e-6, kv_fmt=fmt,
                      idx_fmt=fmt, act_fmt="f32")
    if ratio:
        L.wkv, L.wgate = r.standard_normal((d, D)) * 0.3, r.standard_normal((d, D)) * 0.3
        L.ape, L.gamma = r.standard_normal((W, d)) * 0.2, np.ones(d)
        if ratio == 4:
            L.idx_wkv, L.idx_wgate = r.standard_normal((DI, D)) * 0.3, r.standard_normal((DI, D)) * 0.3
            L.idx_ape, L.idx_gamma = r.standard_normal((8, DI)) * 0.2, np.ones(DI)
    return L


@pytest.mark.parametrize("ratio", [4, 128])
def test_window_membership_by_perturbation(ratio):
    L = _small_layer(ratio)
    n = 4 * ratio + (3 if ratio == 4 else 0)
    X = rng.standard_normal((n, 12)).astype(np.float32)
    U = rng.standard_normal((n, 16)).astype(np.float32)
    base = O.OracleSequence(L)
    base.feed(0, X, U)
    V = n // ratio
    rows0 = [base.comp_row(i)[0] for i in range(V)]
    for t in (0, 3, 4, 5, 9, n - 1) if ratio == 4 else (0, 127, 128, 300, n - 1):
        X2 = X.copy()
        X2[t] += 1.0
        s2 = O.OracleSequence(L)
        s2.feed(0, X2, U)
        changed = {i for i in range(V) if not np.array_equal(s2.comp_row(i)[0], rows0[i])}
        expect = {t // 4, t // 4 + 1} if ratio == 4 else {t // 128}
        assert changed == {i for i in expect if i < V}, (t, changed)


def test_row_counts_and_swa_cap():
    # V = floor(n / r): 256, 16384, 8192, 32768, 1024 rows
    L4 = _small_layer(4)
    L128 = _small_layer(128)
    s4, s128 = O.OracleSequence(L4), O.OracleSequence(L128)
    assert s4.visible_rows(1023) == 256
    assert s4.visible_rows(65535) == 16384
    assert s128.visible_rows((1 << 20) - 1) == 8192
    assert s4.visible_rows(131071) == 32768 and s128.visible_rows(131071) == 1024
    # a 256-token block holds 64 c4a rows and 2 c128a rows (vLLM page)
    assert s4.visible_rows(256 * 7 - 1) - s4.visible_rows(256 * 6 - 1) == 64
    assert s128.visible_rows(256 * 7 - 1) - s128.visible_rows(256 * 6 - 1) == 2
    # 1M tokens -> 262144 c4a rows ("250k")
    assert s4.visible_rows((1 << 20) - 1) == 262144
    # emission: row i appears exactly when token i*r + r - 1 is seen
    for p in range(0, 40):
        assert s4.visible_rows(p) == (p + 1) // 4
    for p in (0, 5, 127, 128, 300):
        assert len(s4.raw_window(p)) == min(128, p + 1)
        assert s4.raw_window(p)[-1] == p


# ---------------------------------------------------------------------------
# indexer and top-k
# ---------------------------------------------------------------------------

def _brute_topk(scores, k):
    """Row s is selected iff fewer than k rows beat it (higher score, or equal
    score at a lower index)."""
    V = len(scores)
    sel = []
    for s in range(V):
        beats = sum(1 for t in range(V) if scores[t] > scores[s] or (scores[t] == scores[s] and t < s))
        if beats < k:
            sel.append(s)
    return sel


def test_topk_against_brute_force_tiny_exhaustive():
    for V in range(0, 65, 3):
        for k in (1, 2, 5, 8):
            for trial in range(3):
                if trial == 0:
                    sc = rng.integers(0, 4, V).astype(np.float64)   # forced ties
                else:
                    sc = rng.standard_normal(V)
                got = O.topk_select(sc, k)
                ref = _brute_topk(sc, k)
                assert list(got[got >= 0]) == ref
                assert np.all(got[len(ref):] == -1) and len(got) == k
                assert list(got[:len(ref)]) == sorted(got[:len(ref)])


def test_indexer_score_closed_form_and_relu():
    qh = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 0.0]])
    w = np.array([0.5, 0.25])
    rows = np.array([[2.0, 1.0, 9.0], [-3.0, 4.0, 0.0], [-1.0, -1.0, 5.0]])
    # row0: 0.5*2 + 0.25*2 = 1.5; row1: 0.5*0 + 0.25*8 = 2; row2: 0
    np.testing.assert_allclose(O.indexer_scores(qh, w, rows), [1.5, 2.0, 0.0])
    np.testing.assert_allclose(O.indexer_scores(qh, w, rows, relu=False), [1.5, 0.5, -1.0])


def test_topk_invariant_under_positive_head_weight_scale():
    qh = rng.standard_normal((4, 16))
    w = rng.uniform(0, 1, 4)
    rows = rng.standard_normal((200, 16))
    a = O.topk_select(O.indexer_scores(qh, w, rows), 20)
    b = O.topk_select(O.indexer_scores(qh, 7.5 * w, rows), 20)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def test_attention_special_cases():
    rows = rng.standard_normal((7, 32))
    np.testing.assert_allclose(O.attention(np.zeros((3, 32)), rows, 0.17), np.tile(rows.mean(0), (3, 1)), rtol=1e-13)
    np.testing.assert_allclose(O.attention(rng.standard_normal((2, 32)), rows[:1], 1.0), np.tile(rows[0], (2, 1)), rtol=1e-14)
    # two rows with logits l0, l1 -> weight sigmoid(l0 - l1)
    r2 = np.array([[1.0, 0.0], [0.0, 1.0]])
    q = np.array([[2.0, -1.0]])
    a0 = 1 / (1 + math.exp(-(0.5 * 2.0 - 0.5 * -1.0)))
    np.testing.assert_allclose(O.attention(q, r2, 0.5), [[a0, 1 - a0]], rtol=1e-14)
    # permutation of the row set does not matter
    perm = rng.permutation(7)
    qq = rng.standard_normal((4, 32))
    np.testing.assert_allclose(O.attention(qq, rows[perm], 0.2), O.attention(qq, rows, 0.2), rtol=1e-12)


def test_attention_translation_invariance_with_inverse_rope():
    # same un-rotated rows and query; every position shifted by delta ->
    # identical output once the output tail is rotated back (vLLM page: the
    # inverse RoPE keeps shared K=V attention translation invariant)
    d, n_rot, base = 64, 16, 160000.0
    R = rng.standard_normal((20, d))
    q = rng.standard_normal((3, d))
    t = np.sort(rng.choice(5000, 20, replace=False))
    p = 5000

    def out(shift):
        rows = O.rope_tail(R, t + shift, base, n_rot)
        qh = O.rope_tail(q, p + shift, base, n_rot)
        return O.rope_tail(O.attention(qh, rows, d ** -0.5), -(p + shift), base, n_rot)

    np.testing.assert_allclose(out(0), out(4 * 12345), atol=1e-9)
    # without the inverse rotation the tails differ
    rows0 = O.rope_tail(R, t, base, n_rot)
    o_plain = O.attention(O.rope_tail(q, p, base, n_rot), rows0, d ** -0.5)
    assert not np.allclose(o_plain[:, -n_rot:], out(0)[:, -n_rot:], atol=1e-6)


def test_swa_only_layer_first_token_returns_its_row():
    # ratio 0, p = 0: the only visible row is u_0, so every head returns u_0
    L = _small_layer(0)
    seq = O.OracleSequence(L)
    u0 = rng.standard_normal(16).astype(np.float32)
    res = seq.step(0, np.zeros(12, np.float32), u0, rng.standard_normal((3, 16)).astype(np.float32))
    np.testing.assert_allclose(res["out_f64"], np.tile(u0.astype(np.float64), (3, 1)), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_attended_rows():
    L = _small_layer(4)
    seq = O.OracleSequence(L)
    n = 60
    X = rng.standard_normal((n, 12)).astype(np.float32)
    U = rng.standard_normal((n, 16)).astype(np.float32)
    seq.feed(0, X, U)
    p = n - 1
    topk = np.array([3, 7, 11, -1], np.int32)
    res = seq.query(p, np.zeros((3, 16), np.float32), rng.standard_normal((2, 8)).astype(np.float32),
                    rng.uniform(0, 1, 2), topk_override=topk)
    rows = [seq.raw_row(t)[2] for t in range(0, p + 1)] + [seq.comp_row(i)[2] for i in (3, 7, 11)]
    mean = O.rope_tail(np.mean(rows, axis=0), -p, L.rope_base, L.n_rot)
    np.testing.assert_allclose(res["out_f64"], np.tile(mean, (3, 1)), rtol=1e-11, atol=1e-12)
    # -1 entries and any order of the list give the same output
    qx = rng.standard_normal((3, 16)).astype(np.float32)
    a = seq.query(p, qx, np.zeros((2, 8), np.float32), np.ones(2), topk_override=[11, -1, 3, 7])["out_f64"]
    b = seq.query(p, qx, np.zeros((2, 8), np.float32), np.ones(2), topk_override=[3, 7, 11, -1])["out_f64"]
    np.testing.assert_allclose(a, b, rtol=1e-13)


# ---------------------------------------------------------------------------
# prefill vs decode, schedule, cache sizes
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# position bookkeeping through OracleSequence
# ---------------------------------------------------------------------------
#
# Each class of vector carries its position in its RoPE tail: raw row t at t,
# compressed / indexer row i at i*r, the query at p, the output rotated back
# by -p (vLLM page, "Shared Key and Value": the inverse rotation makes the
# attention depend on relative positions only).  The pins below fix each of
# these positions from outside the oracle: closed forms whose expected values
# come from trigonometry written here, translation of a whole history, and the
# resume of a sequence from its stored cache.


def _softmax_out(logits, vecs):
    """sum_j softmax(logits)_j vecs_j in plain Python floats."""
    m = max(logits)
    e = [math.exp(v - m) for v in logits]
    s = sum(e)
    out = np.zeros(len(vecs[0]))
    for w, v in zip(e, vecs):
        out += (w / s) * np.asarray(v, np.float64)
    return out


def _pin_layer(ratio, base, base_comp, d=16, D=4, DI=8, n_rot=8, top_k=4):
    return O.OracleLayer(ratio=ratio, head_dim=d, n_heads=1, idx_heads=1 if ratio == 4 else 0,
                         idx_dim=DI if ratio == 4 else 0, top_k=top_k if ratio == 4 else 0, n_rot=n_rot, swa=128,
                         rope_base=base, norm_eps=1e-6, kv_fmt="f64", idx_fmt="f64", act_fmt="f64",
                         rope_base_comp=base_comp)


@pytest.mark.parametrize("ratio", [0, 4, 128])
@pytest.mark.parametrize("bases", [(10000.0, None), (10000.0, 160000.0)])
def test_positions_of_every_class_closed_form(ratio, bases):
    """Every vector lives in tail pair 1 (channels d_n+2, d_n+3), where RoPE at
    position s turns it by s*theta_1, theta_1 = base^(-2/n_rot).  Raw rows are
    A*(cos t*th_r, sin t*th_r); the compressor sees a constant kappa (wgate = 0,
    APE = 0), so every pooled row is the same unit vector, RMS-normalised to
    amplitude c = (1/d + eps)^(-1/2) and turned by i*r*th_c; the indexer lane
    likewise with c_I over D_I channels.  The query is Aq*e and q^I = e.  Then

      raw logit        tau*Aq*A*cos((p - t) th_r)
      compressed logit tau*Aq*c*cos((p - i r) th_c)
      indexer score    relu(c_I cos((p - 4 i) th_c))

    and the output, rotated back by -p class by class, is
    sum a_t A (cos, sin)((t - p) th_r) + sum a_i c (cos, sin)((i r - p) th_c).
    Rotating any class at another position (t + 1, i*r + 1, 2p, +p for the
    inverse), or with the other class's base, moves these values."""
    base, base_comp = bases
    L = _pin_layer(ratio, base, base_comp)
    d, n_rot, D, DI = L.head_dim, L.n_rot, 4, 8
    dn = d - n_rot
    th_r = base ** (-2.0 / n_rot)
    th_c = (base if base_comp is None else base_comp) ** (-2.0 / n_rot)
    A, Aq, tau = 3.0, 2.0, d ** -0.5
    ch = dn + 2                                         # x channel of pair 1
    if ratio:
        W = L.window
        L.wkv = np.zeros((d, D))
        L.wkv[ch, 0] = 1.0
        L.wgate = np.zeros((d, D))
        L.ape = np.zeros((W, d))
        L.gamma = np.ones(d)
        if ratio == 4:
            L.idx_wkv = np.zeros((DI, D))
            L.idx_wkv[2, 0] = 1.0                     # D_I = n_rot: every indexer channel rotates
            L.idx_wgate = np.zeros((DI, D))
            L.idx_ape = np.zeros((8, DI))
            L.idx_gamma = np.ones(DI)
    N = 700 if ratio == 128 else 420
    X = np.zeros((N, D))
    X[:, 0] = 1.0
    U = np.zeros((N, d))
    U[:, ch] = A
    seq = O.OracleSequence(L)
    seq.feed(0, X, U)
    c = (1.0 / d + 1e-6) ** -0.5
    cI = (1.0 / DI + 1e-6) ** -0.5
    q = np.zeros((1, d))
    q[0, ch] = Aq
    qI = np.zeros((1, DI))
    qI[0, 2] = 1.0
    for p in (5, 130, 259, 263, N - 1):
        res = seq.query(p, q, qI if ratio == 4 else None, np.ones(1) if ratio == 4 else None)
        logits, vecs = [], []
        for t in range(max(0, p - 127), p + 1):
            logits.append(tau * Aq * A * math.cos((p - t) * th_r))
            v = np.zeros(d)
            v[ch], v[ch + 1] = A * math.cos((t - p) * th_r), A * math.sin((t - p) * th_r)
            vecs.append(v)
        V = (p + 1) // ratio if ratio else 0
        if ratio == 4:
            sc = [max(0.0, cI * math.cos((p - 4 * i) * th_c)) for i in range(V)]
            np.testing.assert_allclose(res["scores"], sc, rtol=1e-12, atol=1e-12)
            order = sorted(range(V), key=lambda i: (-sc[i], i))[:L.top_k]
            assert sorted(order) == [int(i) for i in res["topk"] if i >= 0], p
            rows = sorted(order)
        else:
            rows = range(V)
        for i in rows:
            logits.append(tau * Aq * c * math.cos((p - i * ratio) * th_c))
            v = np.zeros(d)
            v[ch], v[ch + 1] = c * math.cos((i * ratio - p) * th_c), c * math.sin((i * ratio - p) * th_c)
            vecs.append(v)
        np.testing.assert_allclose(res["out_f64"][0], _softmax_out(logits, vecs), rtol=1e-11, atol=1e-12)


def _rand_layer(ratio, seed, base_comp=None):
    """Small layer with fp64 storage, channel 0 of every computed row held at
    zero (wkv row 0 = 0); the translation pin uses that channel."""
    r = np.random.default_rng(seed)
    d, D, DI = 16, 12, 8
    L = O.OracleLayer(ratio=ratio, head_dim=d, n_heads=3, idx_heads=2 if ratio == 4 else 0,
                      idx_dim=DI if ratio == 4 else 0, top_k=4 if ratio == 4 else 0, n_rot=8, swa=128,
                      rope_base=10000.0, norm_eps=1e-6, kv_fmt="f64", idx_fmt="f64", act_fmt="f64",
                      rope_base_comp=base_comp)
    if ratio:
        W = L.window
        L.wkv = r.standard_normal((d, D)) * 0.4
        L.wkv[0] = 0.0
        L.wgate = r.standard_normal((d, D)) * 0.4
        L.ape = r.standard_normal((W, d)) * 0.3
        L.gamma = 1.0 + 0.1 * r.standard_normal(d)
        if ratio == 4:
            L.idx_wkv = r.standard_normal((DI, D)) * 0.4
            L.idx_wgate = r.standard_normal((DI, D)) * 0.4
            L.idx_ape = r.standard_normal((8, DI)) * 0.3
            L.idx_gamma = 1.0 + 0.1 * r.standard_normal(DI)
    return L


def _history(L, N, seed):
    r = np.random.default_rng(seed)
    X = r.standard_normal((N, 12))
    U = r.standard_normal((N, L.head_dim))
    U[:, 0] = 0.0
    Q = r.standard_normal((N, L.n_heads, L.head_dim))
    Q[..., 0] = 1.0
    QI = r.standard_normal((N, max(L.idx_heads, 1), max(L.idx_dim, 1)))
    Wt = r.uniform(0.0, 1.0, (N, max(L.idx_heads, 1)))
    return X, U, Q, QI, Wt


def _shifted_sequence(L, delta, cap):
    """A sequence whose first live token is ``delta``, with nothing before it:
    the pending compressor slots carry score -inf (no weight, as slots before
    token 0 do), indexer rows before it are zero (score 0: never selected
    while the k-th best score is positive), and each compressed row before it
    holds -1e200 in channel 0, where every query has 1 and every live row 0,
    so its logit is about -1e199 and its softmax weight exactly 0."""
    d = L.head_dim
    W = L.window
    comp = np.zeros((cap, 8 * d), np.uint8)
    if L.ratio:
        for i in range(delta // L.ratio):
            v = np.zeros(d)
            v[0] = -1e200
            comp[i] = v.view(np.uint8)
    kw = {}
    if L.ratio:
        kw.update(st_kv=np.zeros((W, d)), st_sc=np.full((W, d), -np.inf))
    if L.ratio == 4:
        kw.update(ist_kv=np.zeros((8, L.idx_dim)), ist_sc=np.full((8, L.idx_dim), -np.inf))
    return O.OracleSequence(L, raw_rec=None, comp_rec=comp, idx_vals=None, first_live=delta, **kw)


@pytest.mark.parametrize("ratio,delta", [(4, 4 * 1237), (128, 128 * 29), (0, 3001)])
@pytest.mark.parametrize("base_comp", [None, 160000.0])
def test_translation_of_a_whole_history(ratio, delta, base_comp):
    """The same un-rotated history (x, u, q, q^I, w) fed at positions 0.. and
    at delta.., with delta a multiple of r: every query's top-k set shifts by
    delta / r and its output is unchanged (fp64 storage; queries at p >= 127
    so that both raw windows hold live tokens only).  This holds only when
    raw rows, compressed rows, indexer rows, the query and the inverse
    rotation all carry consistent positions, per class."""
    L = _rand_layer(ratio, 7 + ratio, base_comp)
    N = 700 if ratio == 128 else 300
    X, U, Q, QI, Wt = _history(L, N, 99 + ratio)
    A = O.OracleSequence(L)
    A.feed(0, X, U)
    B = _shifted_sequence(L, delta, (delta + N) // max(ratio, 1) + 1)
    B.feed(delta, X, U)
    for p in (127, 200, 263, N - 1):
        qi, w = (QI[p], Wt[p]) if ratio == 4 else (None, None)
        ra = A.query(p, Q[p], qi, w)
        rb = B.query(delta + p, Q[p], qi, w)
        if ratio == 4:
            assert np.sort(ra["scores"])[::-1][L.top_k - 1] > 0.0
            ta, tb = ra["topk"], rb["topk"]
            np.testing.assert_array_equal(tb[tb >= 0], ta[ta >= 0] + delta // 4)
        np.testing.assert_allclose(rb["out_f64"], ra["out_f64"], rtol=0, atol=1e-9)
    if ratio:
        # control: a shift that is not a multiple of r moves the absolute
        # window boundaries, and the outputs change
        B2 = _shifted_sequence(L, delta + 1, (delta + N) // ratio + 2)
        B2.feed(delta + 1, X, U)
        p = N - 1
        qi, w = (QI[p], Wt[p]) if ratio == 4 else (None, None)
        o1 = B2.query(delta + 1 + p, Q[p], qi, w)["out_f64"]
        assert np.max(np.abs(o1 - A.query(p, Q[p], qi, w)["out_f64"])) > 1e-6


@pytest.mark.parametrize("ratio,t0", [(4, 4 * 57 + 2), (4, 4 * 60), (128, 128 * 3 + 37), (0, 200)])
@pytest.mark.parametrize("fmt", ["f64", "f32"])
def test_resume_from_stored_cache_equals_full_history(ratio, t0, fmt):
    """A sequence resumed at token t0 from the cache a full run left behind --
    raw ring slot t % 128, compressed and indexer rows 0 .. t0//r - 1, and the
    compressor windows' pending (kappa, sigma) in slot t % W -- continues
    exactly as the full run does (P1 s3: chunks carry the compressor window
    and the raw rows across their edges)."""
    L = _rand_layer(ratio, 3 + ratio)
    L.kv_fmt = L.idx_fmt = fmt
    N = 700 if ratio == 128 else 320
    X, U, Q, QI, Wt = _history(L, N, 5 + ratio)
    A = O.OracleSequence(L)
    A.feed(0, X, U)
    d = L.head_dim
    rb = O.stored_row_bytes(fmt, d, L.n_rot)
    raw = np.zeros((128, rb), np.uint8)
    for t in range(max(0, t0 - 127), t0):
        raw[t % 128] = A.raw_row(t)[1]
    kw = dict(raw_rec=raw, first_live=t0)
    if ratio:
        cap = N // ratio + 1
        comp = np.zeros((cap, rb), np.uint8)
        for i in range(t0 // ratio):
            comp[i] = A.comp_row(i)[1]
        W = L.window
        st_kv, st_sc = np.zeros((W, d)), np.zeros((W, d))
        for t in range(max(0, t0 - W), t0):
            st_kv[t % W], st_sc[t % W] = A.kap[t], A.sig[t]
        kw.update(comp_rec=comp, st_kv=st_kv, st_sc=st_sc)
        if ratio == 4:
            idx = np.zeros((cap, L.idx_dim))
            for i in range(t0 // 4):
                idx[i] = A.idx_row(i)[1]
            ist_kv, ist_sc = np.zeros((8, L.idx_dim)), np.zeros((8, L.idx_dim))
            for t in range(max(0, t0 - 8), t0):
                ist_kv[t % 8], ist_sc[t % 8] = A.ikap[t], A.isig[t]
            kw.update(idx_vals=idx, ist_kv=ist_kv, ist_sc=ist_sc)
    B = O.OracleSequence(L, **kw)
    B.feed(t0, X[t0:], U[t0:])
    for p in sorted({t0, t0 + 1, t0 + 3, min(t0 + 130, N - 2), N - 1}):
        qi, w = (QI[p], Wt[p]) if ratio == 4 else (None, None)
        ra, rb_ = A.query(p, Q[p], qi, w), B.query(p, Q[p], qi, w)
        if ratio == 4:
            np.testing.assert_array_equal(rb_["topk"], ra["topk"])
        np.testing.assert_allclose(rb_["out_f64"], ra["out_f64"], rtol=1e-13, atol=1e-13)


def test_sliding_window_holds_exactly_the_last_128_tokens():
    """Ratio 0: the output at p changes when any of the tokens p-127 .. p
    changes (the query's own token included: it is appended before it is
    attended) and does not change for p-128 or for any later token."""
    L = _rand_layer(0, 1)
    N = 400
    X, U, Q, QI, Wt = _history(L, N, 2)
    p = 300

    def out(U2):
        s = O.OracleSequence(L)
        s.feed(0, X, U2)
        return s.query(p, Q[p])["out_f64"]

    base = out(U)
    for t, moves in ((p, True), (p - 127, True), (p - 60, True), (p - 128, False), (p + 1, False),
                     (0, False)):
        U2 = U.copy()
        U2[t, 1:] += 0.5
        assert (np.max(np.abs(out(U2) - base)) > 1e-9) == moves, t


def test_flash_schedule():
    r = [O.flash_ratio(i) for i in range(43)]
    assert r[:2] == [0, 0] and r.count(4) == 21 and r.count(128) == 20
    assert r == [wl_flash_ratio(i) for i in range(43)]
    rp = [O.pro_ratio(i) for i in range(61)]
    assert rp.count(4) == 30 and rp.count(128) == 31


def test_kv_cache_size_figures_of_the_vllm_page():
    g = json.load(open(os.path.join(GOLD, "kv_cache_sizes.json")))
    n = g["n_tokens"]
    pro = [O.pro_ratio(i) for i in range(g["pro_layers"])]
    v4 = O.kv_bytes_per_sequence(n, pro) / 2 ** 30
    # V3.2-style: every layer keeps every token (576-wide MLA latent + 128 indexer, bf16)
    v32 = g["pro_layers"] * n * (576 + 128) * 2 / 2 ** 30
    tol = g["print_precision"]
    assert abs(v4 - g["v4_bf16_gib"]) <= tol["v4_bf16_gib"]
    assert abs(v32 - g["v32_bf16_gib"]) <= tol["v32_bf16_gib"]
    assert abs(v32 / v4 - g["ratio"]) <= tol["ratio"]
    fp = O.kv_bytes_per_sequence(n, pro, attn_bytes_per_row=448 + 128, idx_bytes_per_row=64) / 2 ** 30
    assert abs(fp / v4 - g["fp8_fp4_factor"]) <= tol["fp8_fp4_factor"]


def test_workload_row_counts():
    assert get_config("c2").comp_cap == 16384
    assert get_config("c5").comp_cap == 32768 and get_config("c5_c128a").comp_cap == 1024
    assert get_config("c3").comp_cap == 8192


# ---------------------------------------------------------------- debug stage skips
# The boundary's SKIP_NORM / SKIP_ROPE flags turn the RMSNorm (with its gamma)
# and every tail rotation off.  With both off and wgate = APE = 0 every
# compressor score is equal, so each stored row is the plain mean of
# kappa_t = W_kv x_t over its window's live tokens (P1 s4 steps 3-5 with the
# scores uniform), the raw row of token t is u_t, and the output is the plain
# softmax average of the attended rows with the query as given.


@pytest.mark.parametrize("ratio", [4, 128])
def test_debug_skips_leave_window_means_and_plain_attention(ratio):
    rng = np.random.default_rng(11 + ratio)
    L = _pin_layer(ratio, 10000.0, 160000.0)
    L.skip_norm = L.skip_rope = True
    d, D, W = L.head_dim, 4, L.window
    L.wkv = rng.standard_normal((d, D))
    L.wgate = np.zeros((d, D))
    L.ape = np.zeros((W, d))
    L.gamma = rng.uniform(0.5, 1.5, d)           # ignored under SKIP_NORM
    if ratio == 4:
        DI = L.idx_dim
        L.idx_wkv = rng.standard_normal((DI, D))
        L.idx_wgate = np.zeros((DI, D))
        L.idx_ape = np.zeros((8, DI))
        L.idx_gamma = rng.uniform(0.5, 1.5, DI)
    N = 300 if ratio == 4 else 700
    X = rng.standard_normal((N, D))
    U = rng.standard_normal((N, d))
    seq = O.OracleSequence(L)
    seq.feed(0, X, U)
    kap = X @ L.wkv.T
    rows = []
    for i in range(N // ratio):
        toks = [t for t in range(i * ratio - (W - ratio), i * ratio + ratio) if 0 <= t < N]
        want = kap[toks].mean(axis=0)
        np.testing.assert_allclose(seq.comp_row(i)[0], want, rtol=1e-12, atol=1e-12)
        rows.append(want)
        if ratio == 4:
            iw = (X[toks] @ L.idx_wkv.T).mean(axis=0)
            np.testing.assert_allclose(seq.idx_row(i)[0], iw, rtol=1e-12, atol=1e-12)
    p = N - 1
    for t in range(p - 127, p + 1):
        np.testing.assert_array_equal(seq.raw_row(t)[0], U[t])
    q = rng.standard_normal((1, d))
    V = seq.visible_rows(p)
    sel = [0, 5, 17, V - 1] if ratio == 4 else list(range(V))
    topk = np.array(sel, np.int32) if ratio == 4 else None
    vecs = [U[t] for t in range(p - 127, p + 1)] + [rows[i] for i in sel]
    logits = [float(q[0] @ v) * d ** -0.5 for v in vecs]
    np.testing.assert_allclose(seq.attend(p, q, topk)[0], _softmax_out(logits, vecs), rtol=1e-12, atol=1e-12)
    # the same layer with RoPE on moves the output (the skip is not vacuous)
    L.skip_rope = False
    seq2 = O.OracleSequence(L)
    seq2.feed(0, X, U)
    assert np.max(np.abs(seq2.attend(p, q, topk)[0] - _softmax_out(logits, vecs))) > 1e-3


# ---------------------------------------------------------------- indexer QAT (fp4)
# P1 s9: the indexer's rows and query pass through Hadamard-128 and an FP4
# round trip.  Readings (the pages give no format): orthonormal Sylvester
# Hadamard; OCP MXFP4 (E2M1 elements, blocks of 32, power-of-two scale
# 2^(floor(log2 max|x|) - 2), round to nearest even, saturate at 6).  The pins
# below rebuild each piece independently: H from Kronecker products, the E2M1
# values from the bit layout (1 sign, 2 exponent bits with bias 1, 1 mantissa
# bit), rounding by brute force over the representable values.


def _kron_hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    return h / math.sqrt(n)


def _e2m1_value(code):
    s = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    return s * (m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1))


def _fp4_brute(v):
    """Nearest E2M1 value of v (already scaled): ties to the even mantissa bit,
    |v| above 6 saturates."""
    a = min(abs(v), 6.0)
    best, code = None, None
    for c in range(8):
        val = _e2m1_value(c)
        dist = abs(a - val)
        if best is None or dist < best - 1e-15 or (abs(dist - best) <= 1e-15 and (c & 1) == 0):
            best, code = dist, c
    out = _e2m1_value(code)
    return -out if v < 0 else out


def test_hadamard_is_orthonormal_and_keeps_dot_products():
    H = _kron_hadamard(128)
    np.testing.assert_allclose(O.hadamard(np.eye(128)), H, atol=1e-15)
    np.testing.assert_allclose(H @ H, np.eye(128), atol=1e-12)      # symmetric and orthonormal
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((5, 128)), rng.standard_normal((7, 128))
    np.testing.assert_allclose(O.hadamard(q) @ O.hadamard(k).T, q @ k.T, rtol=1e-12, atol=1e-12)
    # without the FP4 step the indexer scores are those of the plain vectors
    w = rng.uniform(0, 1, 5)
    np.testing.assert_allclose(O.indexer_scores(O.hadamard(q), w, O.hadamard(k)), O.indexer_scores(q, w, k),
                               rtol=1e-12, atol=1e-12)


def test_e2m1_codes_from_the_bit_layout():
    for c in range(16):
        assert O.fp4_decode(np.array([c]))[0] == _e2m1_value(c), c


def test_fp4_rounding_by_brute_force():
    rng = np.random.default_rng(4)
    vals = list(rng.uniform(-8, 8, 4000)) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -2.5, -5.0, 6.0, 6.5,
                                             -7.9, 0.0, 1e-9, -1e-9]
    got = O.fp4_decode(O.fp4_encode(np.array(vals)))
    for v, g in zip(vals, got):
        assert g == _fp4_brute(v), (v, g, _fp4_brute(v))


def test_mxfp4_block_scale_and_error_bound():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)) * 10.0 ** rng.uniform(-4, 4, (64, 1))
    codes, e = O.mxfp4_encode(x)
    blk = x.reshape(64, 4, 32)
    amax = np.abs(blk).max(axis=-1)
    ratio = amax / np.ldexp(1.0, e)
    assert np.all((ratio >= 4.0) & (ratio < 8.0))                   # e = floor(log2 amax) - 2
    rt = O.mxfp4_round_trip(x)
    err = np.abs(rt - x).reshape(64, 4, 32)
    step = np.ldexp(1.0, e)[..., None]
    assert np.all(err <= 2 * step)                                   # saturation above 6 * 2^e
    unsat = np.abs(blk) <= 6 * step
    assert np.all(err[unsat] <= step.repeat(32, -1)[unsat])         # largest half-gap (between 4 and 6)
    np.testing.assert_array_equal(O.mxfp4_round_trip(rt), rt)       # the grid is a fixed point
    # exact block values survive, a zero block stays zero
    exact = np.zeros((1, 32))
    exact[0, :8] = [6, -4, 3, 1.5, 0.5, 0, 2, -6]
    np.testing.assert_array_equal(O.mxfp4_round_trip(exact * 2.0 ** -5), exact * 2.0 ** -5)
    np.testing.assert_array_equal(O.mxfp4_round_trip(np.zeros((1, 32))), np.zeros((1, 32)))


def test_fp4_row_record_layout():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 128))
    rec = O.fp4_encode_rows(x)
    assert rec.shape == (3, 68) and O.fp4_row_bytes(128) == 68
    codes, e = O.mxfp4_encode(x)
    np.testing.assert_array_equal(rec[:, :64] & 15, codes[:, 0::2])
    np.testing.assert_array_equal(rec[:, :64] >> 4, codes[:, 1::2])
    np.testing.assert_array_equal(rec[:, 64:].astype(np.int64) - 127, e)
    np.testing.assert_array_equal(O.decode_values(rec, "fp4"), O.mxfp4_round_trip(x))


def test_fp4_indexer_scores_by_brute_force():
    """An fp4 layer's indexer: rows and query rounded in the Hadamard domain;
    scores against a brute-force rebuild (Kronecker H, per-element nearest
    E2M1 value with the block scale from max |x|)."""
    rng = np.random.default_rng(7)
    L = _pin_layer(4, 10000.0, None, d=16, D=4, DI=128, n_rot=8, top_k=4)
    L.idx_fmt = "fp4"
    L.idx_heads = 2
    L.wkv = rng.standard_normal((16, 4))
    L.wgate = rng.standard_normal((16, 4))
    L.ape = rng.standard_normal((8, 16)) * 0.1
    L.gamma = np.ones(16)
    L.idx_wkv = rng.standard_normal((128, 4))
    L.idx_wgate = rng.standard_normal((128, 4))
    L.idx_ape = rng.standard_normal((8, 128)) * 0.1
    L.idx_gamma = rng.uniform(0.5, 1.5, 128)
    N = 60
    seq = O.OracleSequence(L)
    seq.feed(0, rng.standard_normal((N, 4)), rng.standard_normal((N, 16)))
    H = _kron_hadamard(128)

    def brute_rt(v):
        out = np.empty_like(v)
        for b in range(0, 128, 32):
            blk = v[b:b + 32]
            amax = np.max(np.abs(blk))
            sc = 2.0 ** (math.floor(math.log2(amax)) - 2) if amax > 0 else 0.0
            out[b:b + 32] = [(_fp4_brute(t / sc) * sc if sc else 0.0) for t in blk]
        return out

    p = N - 1
    qI = rng.standard_normal((2, 128))
    w = rng.uniform(0, 1, 2)
    qr = L.rope(qI, p, L.base_comp, 8)
    qt = np.stack([brute_rt(H @ qr[h]) for h in range(2)])
    V = seq.visible_rows(p)
    rows = np.stack([brute_rt(H @ seq._pool_row(i, "idx")) for i in range(V)])
    want = np.array([sum(w[h] * max(float(qt[h] @ rows[i]), 0.0) for h in range(2)) for i in range(V)])
    np.testing.assert_allclose(seq.index_scores(p, qI, w), want, rtol=1e-12, atol=1e-12)


def test_out_fp8_scale_rule_and_error_bound():
    """Attention output in fp8 (group-of-128 E4M3 with an fp32 scale
    max|o|/448): each group's largest element takes the largest code (448),
    a zero group keeps scale 1 and zero codes, the record holds d codes then
    d/128 scales, and the round trip is within half an E4M3 step of its group
    (2^-4 relative above 2^-6 s, 2^-10 s below)."""
    rng = np.random.default_rng(1234)
    o = rng.standard_normal((3, 512)) * np.array([[1.0], [1e-3], [50.0]])
    o[1, 128:256] = 0.0
    rec, val = O.encode_out_fp8(o)
    assert rec.shape == (3, 512 + 16) and O.out_fp8_record_bytes(512) == 528
    s = rec[:, 512:].copy().view(np.float32).reshape(3, 4).astype(np.float64)
    g = o.reshape(3, 4, 128)
    for r in range(3):
        for k in range(4):
            codes = rec[r, 128 * k:128 * (k + 1)]
            if not np.any(g[r, k]):
                assert s[r, k] == 1.0 and not np.any(codes & 0x7F)
                continue
            assert s[r, k] == np.float32(np.abs(g[r, k]).max() / 448.0)
            assert (codes & 0x7F).max() == 0x7E          # 448 = exponent 15, mantissa 6
            err = np.abs(val[r, 128 * k:128 * (k + 1)] - g[r, k])
            bound = np.maximum(2.0 ** -4 * np.abs(g[r, k]), 2.0 ** -10 * s[r, k]) * (1 + 1e-6)
            assert np.all(err <= bound)
    assert np.allclose(O.decode_out_fp8(rec, 512), val)


# ---------------------------------------------------------------- query norm
# P4 "GPU compute saturation" names a query norm fused with the raw keys'
# RoPE and insertion.  Reading: each head's query divided by its RMS over the
# head's channels (no learned weight, eps = the layer's RMSNorm eps), before
# the RoPE.


def test_query_norm_closed_forms():
    # one head (3, 4): mean square 12.5
    got = O.query_rms_norm(np.array([[3.0, 4.0]]), 0.0)
    np.testing.assert_allclose(got, [[3.0 / math.sqrt(12.5), 4.0 / math.sqrt(12.5)]], rtol=1e-15)
    # with eps the output's mean square is ms / (ms + eps), head by head:
    # heads of very different size are each brought to RMS ~1 (not one
    # norm over all heads)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 64)) * np.array([[1e-3], [1.0], [30.0], [1e3]])
    eps = 1e-6
    out = O.query_rms_norm(q, eps)
    ms = np.mean(q * q, axis=-1)
    np.testing.assert_allclose(np.mean(out * out, axis=-1), ms / (ms + eps), rtol=1e-12)
    # scale invariance at eps = 0 (a negative factor flips the sign)
    np.testing.assert_allclose(O.query_rms_norm(-7.5 * q, 0.0), -O.query_rms_norm(q, 0.0), rtol=1e-13)
    # a head whose entries are all +-1 is already at RMS 1
    pm = np.where(rng.standard_normal((2, 32)) > 0, 1.0, -1.0)
    np.testing.assert_array_equal(O.query_rms_norm(pm, 0.0), pm)


@pytest.mark.parametrize("ratio", [4, 128])
def test_query_norm_in_attention_is_per_head_and_before_rope(ratio):
    """With the query norm on and eps = 0, a query whose head h holds
    c_h * (+-1) entries attends exactly like the +-1 query without the norm
    (each head rescaled by its own factor, the tail still rotated at p); and
    the norm commutes with the RoPE: normalising the rotated query gives the
    rotated normalised query."""
    L = _rand_layer(ratio, seed=40 + ratio)
    L.norm_eps = 0.0
    X, U, Q, QI, Wt = _history(L, 260, seed=41)
    seq = O.OracleSequence(L)
    seq.feed(0, X, U)
    p = 259
    topk = O.topk_select(seq.index_scores(p, QI[p], Wt[p]), L.top_k) if ratio == 4 else None
    rng = np.random.default_rng(42)
    pm = np.where(rng.standard_normal((L.n_heads, L.head_dim)) > 0, 1.0, -1.0)
    c = np.array([0.01, 3.0, 250.0])[:, None]
    plain = seq.attend(p, pm, topk)
    L.q_norm = True
    np.testing.assert_allclose(seq.attend(p, c * pm, topk), plain, rtol=1e-12, atol=1e-13)
    # the norm is not vacuous: a random query moves
    qr = rng.standard_normal((L.n_heads, L.head_dim)) * 4.0
    on = seq.attend(p, qr, topk)
    L.q_norm = False
    assert np.max(np.abs(on - seq.attend(p, qr, topk))) > 1e-3
    # RoPE keeps each pair's sum of squares, so norm and rotation commute
    rot = O.rope_tail(qr, p, L.base_raw, L.n_rot)
    np.testing.assert_allclose(O.query_rms_norm(rot, 1e-6),
                               O.rope_tail(O.query_rms_norm(qr, 1e-6), p, L.base_raw, L.n_rot), rtol=1e-12)


# ---------------------------------------------------------------- two-lane c4a compressor
# P1 s5: a ratio-4 compressor is twice as wide as its rows.  Reading (the
# alternative to one lane): each token projects to lanes A and B; a row's
# window takes lane A of the previous block's four tokens (slots 0-3) and lane
# B of its own block's (slots 4-7); APE [4, 2 w] holds lane A's slot s in
# row s, channels :w, lane B's in channels w:.


def _two_lane_from(L1):
    """The two-lane layer whose lanes are both the one-lane layer's weights."""
    import copy
    L2 = copy.copy(L1)
    L2.two_lane = True
    L2.wkv, L2.wgate = np.vstack([L1.wkv, L1.wkv]), np.vstack([L1.wgate, L1.wgate])
    L2.ape = np.hstack([L1.ape[:4], L1.ape[4:]])
    L2.idx_wkv, L2.idx_wgate = np.vstack([L1.idx_wkv, L1.idx_wkv]), np.vstack([L1.idx_wgate, L1.idx_wgate])
    L2.idx_ape = np.hstack([L1.idx_ape[:4], L1.idx_ape[4:]])
    return L2


def test_two_lane_with_tied_lanes_is_the_one_lane_compressor():
    L1 = _rand_layer(4, seed=61)
    L2 = _two_lane_from(L1)
    X, U, Q, QI, Wt = _history(L1, 300, seed=62)
    s1, s2 = O.OracleSequence(L1), O.OracleSequence(L2)
    s1.feed(0, X, U)
    s2.feed(0, X, U)
    for i in range(75):
        np.testing.assert_allclose(s2.comp_row(i)[0], s1.comp_row(i)[0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(s2.idx_row(i)[0], s1.idx_row(i)[0], rtol=1e-13, atol=1e-13)
    p = 299
    np.testing.assert_allclose(s2.query(p, Q[p], QI[p], Wt[p])["out_f64"], s1.query(p, Q[p], QI[p], Wt[p])["out_f64"],
                               rtol=1e-12, atol=1e-13)


def test_two_lane_windows_take_each_lane_once():
    """Lane B of token t enters row t // 4 only, lane A row t // 4 + 1 only
    (perturbation of one token's projection, attention and indexer lanes)."""
    rng = np.random.default_rng(63)
    L = _two_lane_from(_rand_layer(4, seed=64))
    L.wkv = L.wkv + 0.3 * rng.standard_normal(L.wkv.shape)        # untie the lanes
    L.idx_wkv = L.idx_wkv + 0.3 * rng.standard_normal(L.idx_wkv.shape)
    X, U, *_ = _history(L, 120, seed=65)
    d, DI = L.head_dim, L.idx_dim
    t = 53                                                         # row 13, slot 5 of its window
    for lane, half in (("B", slice(d, 2 * d)), ("A", slice(0, d))):
        for kind in ("attn", "idx"):
            base, moved = O.OracleSequence(L), O.OracleSequence(L)
            base.feed(0, X, U)
            moved.feed(0, X, U)
            h = half if kind == "attn" else slice(half.start // d * DI, half.start // d * DI + DI)
            tab = moved.kap if kind == "attn" else moved.ikap
            tab[t] = tab[t].copy()
            tab[t][h] += 5.0
            moved._row_cache.clear()
            get = (lambda s, i: s.comp_row(i)[0]) if kind == "attn" else (lambda s, i: s.idx_row(i)[0])
            own, nxt = t // 4, t // 4 + 1
            changed = {i for i in range(own - 2, own + 4) if not np.allclose(get(base, i), get(moved, i))}
            assert changed == ({own} if lane == "B" else {nxt}), (lane, kind, changed)


def test_two_lane_ape_slots():
    """A dominant APE entry picks one token's lane: lane A's slot s is token
    4 i - 4 + s, lane B's slot s token 4 i + s (one channel, no norm / RoPE)."""
    L = _two_lane_from(_rand_layer(4, seed=66))
    L.skip_norm = L.skip_rope = True
    rng = np.random.default_rng(67)
    L.wkv = rng.standard_normal(L.wkv.shape)
    X, U, *_ = _history(L, 80, seed=68)
    d = L.head_dim
    i, c = 10, 3
    for lane, s in (("A", 1), ("B", 2), ("A", 3), ("B", 0)):
        L.ape = np.zeros((4, 2 * d))
        L.ape[s, c + (d if lane == "B" else 0)] = 80.0
        seq = O.OracleSequence(L)
        seq.feed(0, X, U)
        t = 4 * i - 4 + s if lane == "A" else 4 * i + s
        want = seq.kap[t][c + (d if lane == "B" else 0)]
        assert seq.comp_row(i)[0][c] == pytest.approx(want, rel=1e-12, abs=1e-12), (lane, s)
