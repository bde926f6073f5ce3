"""Pins for the float64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, an invariant the method must satisfy, a library routine, or the
independent explicit-loop twin (oracle/brute.py) on tiny shapes. They run on
the CPU only.
"""
import copy
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import dflash as O
from oracle.brute import brute_propose
from oracle.numerics import e4m3_decode

HERE = os.path.dirname(os.path.abspath(__file__))


def tiny_case(seed=0, **geo_over):
    geo = synth.TINY
    if geo_over:
        from dataclasses import replace
        geo = replace(geo, **geo_over)
    w = synth.make_weights(geo, seed=seed)
    stack = synth.make_stack(geo, 32, tag=seed)
    return geo, w, stack


# --------------------------------------------------------------------------
# elementary steps
# --------------------------------------------------------------------------

def test_rmsnorm_unit_rms_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 333)) * 3.0
    eps = 1e-6
    y = O.rms_norm(x, np.ones(333), eps)
    m = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), m / (m + eps), rtol=1e-13)
    # the gain multiplies elementwise
    g = rng.standard_normal(333)
    assert np.allclose(O.rms_norm(x, g, eps), y * g, rtol=1e-13)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(1)
    d, theta = 16, 1e6
    x = rng.standard_normal((5, 3, d))
    pos = np.array([0, 1, 7, 100, 4095])
    f = O.rope_inv_freq(theta, d)
    # inv_freq[i] = theta^(-2i/d): f[0] = 1, f[i+1]/f[i] = theta^(-2/d)
    assert f[0] == 1.0 and np.allclose(f[1:] / f[:-1], theta ** (-2.0 / d))
    y = O.rope(x, pos, f)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    zr = z * np.exp(1j * pos[:, None, None] * f[None, None, :])
    assert np.allclose(y[..., : d // 2], zr.real, atol=1e-12)
    assert np.allclose(y[..., d // 2:], zr.imag, atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    # position 0 is the identity
    assert np.array_equal(O.rope(x[:1], np.array([0]), f), x[:1])


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    d = 128
    f = O.rope_inv_freq(1e7, d)
    q = rng.standard_normal((4, 1, d))
    k = rng.standard_normal((6, 1, d))
    pq, pk = np.array([10, 11, 12, 13]), np.array([0, 3, 5, 8, 9, 10])
    s0 = O.rope(q, pq, f)[:, 0] @ O.rope(k, pk, f)[:, 0].T
    for shift in (1, 77, 3000):
        s1 = O.rope(q, pq + shift, f)[:, 0] @ O.rope(k, pk + shift, f)[:, 0].T
        assert np.allclose(s0, s1, atol=1e-9)


def test_attention_identical_keys_gives_mean_v():
    rng = np.random.default_rng(3)
    R, n_q, n_kv, d, S = 5, 8, 2, 16, 37
    q = rng.standard_normal((R, n_q, d))
    key = rng.standard_normal((1, n_kv, d))
    k = np.repeat(key, S, axis=0)
    v = rng.standard_normal((S, n_kv, d))
    out = O.gqa_attention(q, k, v, n_kv)
    for hq in range(n_q):
        g = hq // (n_q // n_kv)
        assert np.allclose(out[:, hq, :], v[:, g, :].mean(axis=0)[None, :], atol=1e-12)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(4)
    R, n_q, n_kv, d, S = 16, 32, 4, 128, 300
    q = rng.standard_normal((R, n_q, d))
    k = rng.standard_normal((S, n_kv, d))
    v = rng.standard_normal((S, n_kv, d))
    ours = O.gqa_attention(q, k, v, n_kv)
    rep = n_q // n_kv
    qt = torch.from_numpy(q).permute(1, 0, 2)                    # [n_q, R, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(rep, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(rep, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).permute(1, 0, 2).numpy()
    assert np.allclose(ours, ref, atol=1e-12)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 10001)
    assert np.allclose(O.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), atol=1e-14)


# --------------------------------------------------------------------------
# output selection
# --------------------------------------------------------------------------

def test_select_ties_lowest_id_and_probabilities():
    lg = np.array([[0.0, 2.0, 1.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, 3.0, 3.0, 0.0]])
    out = O.select(lg, None, 2)
    assert out["ids"].tolist() == [1, 0, 1]
    p = out["row_prob"]
    assert p[1] == pytest.approx(0.25)
    assert p[0] == pytest.approx(1.0 / (math.exp(-2) + 1 + math.exp(-1) + 1))
    assert out["conf"] == pytest.approx(min(p[1], p[2]))


def test_select_bitmask_cases():
    rng = np.random.default_rng(6)
    V = 96
    lg = rng.standard_normal((3, V))
    words = (V + 31) // 32
    # all ones == no mask, bit for bit
    ones = np.full(words, -1, dtype=np.int32)
    a, b = O.select(lg, ones, 2), O.select(lg, None, 2)
    assert np.array_equal(a["ids"], b["ids"]) and np.array_equal(a["row_prob"], b["row_prob"])
    # a single allowed token: id is that token, p1 exactly 1
    for tok in (0, 31, 32, 95):
        m = np.zeros(words, dtype=np.int32)
        m[tok >> 5] = np.int32(np.uint32(1 << (tok & 31)).view(np.int32))
        s = O.select(lg, m, 2)
        assert s["ids"].tolist() == [tok] * 3 and s["row_prob"].tolist() == [1.0] * 3
    # nothing allowed: no token, p1 = 0
    s = O.select(lg, np.zeros(words, np.int32), 2)
    assert s["ids"].tolist() == [O.NO_TOKEN] * 3 and s["row_prob"].tolist() == [0.0] * 3


# --------------------------------------------------------------------------
# whole propose on the tiny geometry
# --------------------------------------------------------------------------

def _head_with_ctx(geo, w, stack, n=None):
    head = O.OracleHead(geo.as_dict(), w)
    st = head.new_state()
    head.precompute(st, stack if n is None else stack[:n])
    return head, st


def test_brute_force_twin_matches_vectorised():
    geo, w, stack = tiny_case(0)
    head, st = _head_with_ctx(geo, w, stack)
    tok = int(synth.make_tokens(geo, 1)[0])
    res = head.propose(st, tok, 32, 3)
    ids, probs, conf, logits = brute_propose(geo.as_dict(), w, stack, tok, 32, 3)
    assert np.allclose(res["logits"], np.array(logits), rtol=1e-9, atol=1e-12)
    assert res["ids"].tolist() == ids
    assert np.allclose(res["row_prob"], probs, rtol=1e-9)
    assert res["conf"] == pytest.approx(conf, rel=1e-9)


def test_brute_force_twin_with_window_and_mask():
    geo, w, stack = tiny_case(1, ctx_window=8)
    head, st = _head_with_ctx(geo, w, stack, 21)
    bm = synth.make_bitmask(geo.vocab, 0.5)
    res = head.propose(st, 7, 25, 2, bm)
    ids, probs, conf, logits = brute_propose(geo.as_dict(), w, stack[:21], 7, 25, 2, bm)
    assert np.allclose(res["logits"], np.array(logits), rtol=1e-9, atol=1e-12)
    assert res["ids"].tolist() == ids
    assert np.allclose(res["row_prob"], probs, rtol=1e-9)


def test_zero_final_gain_gives_uniform():
    geo, w, stack = tiny_case(0)
    w = dict(w)
    w["norm"] = np.zeros_like(w["norm"])
    head, st = _head_with_ctx(geo, w, stack)
    res = head.propose(st, 3, 32, 3)
    assert np.all(res["logits"] == 0.0)
    assert res["ids"].tolist() == [0] * geo.gamma
    assert np.allclose(res["row_prob"], 1.0 / geo.vocab, rtol=1e-14)


def test_duplicate_lm_rows_tie_to_lowest_id():
    """A copy of the argmax row a placed at b gives bit-identical logits and
    the lower of a and b wins, with the copy below a and above it."""
    geo, w, stack = tiny_case(2)
    head, st = _head_with_ctx(geo, w, stack)
    base = head.propose(st, 5, 32, 3)
    a = int(base["ids"][1])
    for b in ((a + 1) % geo.vocab, (a - 1) % geo.vocab, 0 if a else geo.vocab - 1):
        w2 = dict(w)
        lm = w["lm_head"].copy()
        lm[b] = lm[a]
        w2["lm_head"] = lm
        head2, st2 = _head_with_ctx(geo, w2, stack)
        res = head2.propose(st2, 5, 32, 3)
        assert res["logits"][1, a] == res["logits"][1, b]
        assert int(res["ids"][1]) == min(a, b)


def test_window_zero_ignores_ctx():
    geo, w, stack = tiny_case(0, ctx_window=0)
    head, st = _head_with_ctx(geo, w, stack)
    other = synth.make_stack(geo, 32, tag=99)
    _, st2 = _head_with_ctx(geo, w, other)
    empty = head.new_state()
    r1 = head.propose(st, 9, 32, 3)
    r2 = head.propose(st2, 9, 32, 3)
    r3 = head.propose(empty, 9, 32, 3)
    assert np.array_equal(r1["logits"], r2["logits"]) and np.array_equal(r1["logits"], r3["logits"])


def test_window_truncation_equals_shifted_short_context():
    """With c > W the block sees the last W rows; a state holding only those
    rows, with the block shifted by the same amount, gives the same result
    (RoPE scores depend on relative positions only)."""
    W = 8
    geo, w, stack = tiny_case(3, ctx_window=W)
    head, st = _head_with_ctx(geo, w, stack)              # c = 32
    r_full = head.propose(st, 11, 32, 3)
    geo_w, _, _ = tiny_case(3, ctx_window=4096)
    head_w = O.OracleHead(geo_w.as_dict(), w)
    # the last W rows recomputed at positions 0..W-1 differ from positions
    # 24..31 only by a global rotation, which cancels in the scores
    st_w = head_w.new_state()
    head_w.precompute(st_w, stack[32 - W:])
    r_short = head_w.propose(st_w, 11, 32 - (32 - W), 3)
    # equal up to the bf16 rounding of the cached K, which is taken after the
    # rotation (about 3e-5 on the logits), and the bf16 operands of the dense
    # products, which that difference can tip into the neighbouring bf16 value
    # (2^-9 relative each; at most ~7e-4 on the logits over seeds 3..6); a
    # window off by one row moves the logits by 4e-2 or more
    assert np.allclose(r_full["logits"], r_short["logits"], atol=2e-3)
    st_w1 = head_w.new_state()
    head_w.precompute(st_w1, stack[32 - W - 1:])
    r_off = head_w.propose(st_w1, 11, W + 1, 3)
    assert np.abs(r_full["logits"] - r_off["logits"]).max() > 1e-2


def test_trim_equals_recompute():
    geo, w, stack = tiny_case(4)
    extra = synth.make_stack(geo, 8, tag=55)
    head = O.OracleHead(geo.as_dict(), w)
    for a in range(0, 9):
        st = head.new_state()
        head.precompute(st, stack[:20])
        head.after_verify(st, 20)
        head.precompute(st, extra)
        head.after_verify(st, a)
        ref = head.new_state()
        head.precompute(ref, np.concatenate([stack[:20], extra[:a]]))
        assert st.ctx_len == ref.ctx_len == 20 + a
        r1 = head.propose(st, 4, st.ctx_len, 3)
        r2 = head.propose(ref, 4, ref.ctx_len, 3)
        assert np.allclose(r1["logits"], r2["logits"], rtol=1e-12, atol=1e-13)
        r3 = head.propose(head.rebuilt(st), 4, st.ctx_len, 3)
        assert np.allclose(r1["logits"], r3["logits"], rtol=1e-12, atol=1e-13)
    st = head.new_state()
    head.precompute(st, stack[:4])
    with pytest.raises(ValueError):
        head.after_verify(st, 5)


def test_batch_equals_single():
    geo, w, stack = tiny_case(5)
    head = O.OracleHead(geo.as_dict(), w)
    states = []
    for i, n in enumerate((3, 17, 32)):
        st = head.new_state()
        head.precompute(st, synth.make_stack(geo, n, tag=100 + i))
        states.append(st)
    toks = synth.make_tokens(geo, 3)
    pos = [s.ctx_len for s in states]
    batch = head.propose_batch(states, toks, pos, 3)
    for i, st in enumerate(states):
        single = head.propose(st, toks[i], pos[i], 3)
        assert np.array_equal(batch[i]["logits"], single["logits"])


def test_fused_kv_rows_equal_per_layer_projection():
    """The fused ctx-K/V weight, rows [K0; V0; K1; V1; ...], applied once,
    equals the per-layer k/v projections (fused_kv_weight field)."""
    from dataclasses import replace
    geo = replace(synth.TINY, num_layers=3)
    w = synth.make_weights(geo)
    head = O.OracleHead(geo.as_dict(), w)
    c = head.ctx_features(synth.make_stack(geo, 9))
    fused = np.concatenate([np.concatenate([lw["k"], lw["v"]]) for lw in head.layers])
    kv = geo.num_kv_heads * geo.head_dim
    out = c @ fused.T
    for l, lw in enumerate(head.layers):
        assert np.allclose(out[:, (2 * l) * kv:(2 * l + 1) * kv], c @ lw["k"].T, rtol=1e-13)
        assert np.allclose(out[:, (2 * l + 1) * kv:(2 * l + 2) * kv], c @ lw["v"].T, rtol=1e-13)


def test_fp8_head_mirror_properties():
    rng = np.random.default_rng(8)
    w32 = (rng.standard_normal((64, 48)) * 0.02).astype(np.float32)
    w32[3] = 0.0
    bits = synth.to_bf16_bits(w32)
    codes, scale = O.fp8_head_mirror(bits)
    w = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    deq = e4m3_decode(codes) * scale[:, None].astype(np.float64)
    amax = np.abs(w).max(axis=1)
    # each row's largest magnitude maps to the largest code (+-448)
    for v in range(64):
        if amax[v] > 0:
            assert np.abs(e4m3_decode(codes[v])).max() == 448.0
            assert np.float32(scale[v]) == np.float32(np.float32(amax[v]) / np.float32(448.0))
    assert scale[3] == 1.0 and np.all(codes[3] & 0x7F == 0)
    # round-to-nearest error bound: half an E4M3 step, at most 2^-4 relative
    # for normals, 2^-10 * scale absolute in the subnormal range
    err = np.abs(deq - w)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, scale[:, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))


def test_fp8_kv_roundtrip_error_bound():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1000, 4)) * 0.9
    s = np.array([0.01, 0.011, 0.009, 0.0105], dtype=np.float32)
    y = O.fp8_roundtrip(x, s[None, :])
    inrange = np.abs(x) <= 448 * s[None, :]
    err = np.abs(y - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s[None, :].astype(np.float64) * 2.0 ** -10) * 1.0001
    assert np.all(err[inrange] <= bound[inrange])
    # outside the range the value saturates to +-448 s
    big = np.array([[100.0, -100.0, 0.0, 0.0]])
    yb = O.fp8_roundtrip(big, s[None, :])
    assert yb[0, 0] == 448 * np.float64(s[0]) and yb[0, 1] == -448 * np.float64(s[1])


def test_page_geometry_facts():
    """Geometry the pages print for the Qwen3.6-DFlash drafter (fixture cites
    each value) against the full synthetic geometry and the oracle's shapes."""
    with open(os.path.join(HERE, "golden", "page_geometry.json")) as f:
        facts = json.load(f)["facts"]
    g = synth.FULL
    assert g.vocab == facts["vocab_size"]["value"]
    assert g.hidden == facts["hidden_size"]["value"]
    assert g.num_layers == facts["num_layers"]["value"]
    assert g.head_dim == facts["head_dim"]["value"] == facts["rotary_dim"]["value"]
    assert g.rope_theta == facts["rope_theta"]["value"]
    assert g.rms_eps == facts["rms_norm_eps"]["value"]
    assert g.num_target_layers == facts["target_hidden_stack_layers"]["value"]
    assert g.ctx_window == facts["ctx_window_default"]["value"]
    assert (g.vocab + 31) // 32 == facts["bitmask_words_full_vocab"]["value"]
    kv = g.num_kv_heads * g.head_dim
    assert 2 * g.num_layers * kv == facts["fused_kv_rows"]["value"]
    assert g.num_target_layers * g.target_hidden == facts["fc_input_width"]["value"]


@pytest.mark.parametrize("theta,d", [(1e7, 128), (1e6, 64), (1e6, 16)])
def test_yarn_table_limits(theta, d):
    """The YaRN table pinned by its limits rather than its formula: with
    factor 1 it is the plain table; pairs whose wavelength fits more than
    beta_fast times into the original context keep the plain frequency
    exactly, pairs that fit fewer than beta_slow times are divided by the
    factor exactly, the pairs between lie between the two and the table
    falls monotonically. Each regime is present at these geometries."""
    L, bf, bs, f = 4096, 32.0, 1.0, 64.0
    plain64 = O.rope_inv_freq(theta, d)
    plain = plain64.astype(np.float32).astype(np.float64)
    assert np.allclose(O.yarn_inv_freq(theta, d, 1.0, bf, bs, L), plain, rtol=2.0 ** -23, atol=0.0)
    y = O.yarn_inv_freq(theta, d, f, bf, bs, L)
    turns = L / (2.0 * math.pi / plain64)  # how often each pair's wavelength fits into L
    fast, slow = turns > bf, turns < bs
    mid = ~fast & ~slow
    assert fast.any() and slow.any() and mid.any()
    assert np.array_equal(y[fast], plain[fast])
    assert np.array_equal(y[slow], (plain64 / f).astype(np.float32).astype(np.float64)[slow])
    assert np.all(y[mid] <= plain[mid]) and np.all(y[mid] >= (plain64 / f)[mid] * (1 - 2.0 ** -23))
    assert np.all(np.diff(y) < 0)


def test_shifted_rows_read_out():
    """The shifted-row convention changes only the read-out: the block's
    logits are the same, entry 1 (the first draft) is row 0's argmax, entry 0
    holds the last row, and the chain confidence is the least top-1 softmax
    probability (scipy) of rows 0..num_drafts-1."""
    from scipy.special import softmax
    geo, w, stack = tiny_case()
    out = {}
    for sh in (0, 1):
        g = dict(geo.as_dict(), shifted_rows=sh)
        orc = O.OracleHead(g, w)
        st = orc.new_state()
        orc.precompute(st, stack)
        out[sh] = orc.propose(st, 7, st.ctx_len, 2)
    lg = out[0]["logits"]
    assert np.array_equal(out[1]["logits"], lg)
    assert out[1]["ids"][1] == int(np.argmax(lg[0])) and out[1]["ids"][0] == int(np.argmax(lg[-1]))
    p1 = softmax(lg, axis=1).max(axis=1)
    assert math.isclose(out[1]["conf"], float(p1[0:2].min()), rel_tol=1e-12)
    assert math.isclose(out[0]["conf"], float(p1[1:3].min()), rel_tol=1e-12)


def test_fp8_drafter_weight_quantisation():
    """FP8 drafter weights: each row's largest magnitude is kept exactly (it
    maps to the code 448), every element is within half an E4M3 step of its
    bf16 value, fp32 weights are taken at their bf16 value, and a zero row
    stays zero."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((48, 96)) * 0.02).astype(np.float32)
    w[7] = 0.0
    q = O.fp8_weight(w)
    b = O.bf16_round(w.astype(np.float64))
    amax = np.abs(b).max(axis=1)
    assert np.allclose(np.abs(q).max(axis=1), amax, rtol=2.0 ** -23, atol=0.0)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    # E4M3 keeps 3 mantissa bits: a half step is 2^-4 of the value (normals) or 2^-10 of the scale (subnormals)
    assert np.all(np.abs(q - b) <= np.maximum(np.abs(b) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 2.0 ** -20))
    assert np.array_equal(q[7], np.zeros(96))
    bits = (b.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(O.fp8_weight(bits), q)



def test_fp8_activation_rows():
    """E4M3 activation rows of the W8A8 head: each row's largest magnitude is
    kept (code 448), every element lies within half an E4M3 step of its
    float32 value, a zero row stays zero, and on bf16 values the recipe is
    the drafter-weight quantisation (the same per-row absmax mirror)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 256)) * np.exp(rng.uniform(-3, 3, size=(40, 1)))
    x[5] = 0.0
    q = O.fp8_rows(x)
    x32 = x.astype(np.float32).astype(np.float64)
    amax = np.abs(x32).max(axis=1)
    assert np.allclose(np.abs(q).max(axis=1), amax, rtol=2.0 ** -22, atol=0.0)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    assert np.all(np.abs(q - x32) <= np.maximum(np.abs(x32) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 2.0 ** -20))
    assert np.array_equal(q[5], np.zeros(256))
    # sign symmetry: enc(-x) = -enc(x)
    assert np.array_equal(O.fp8_rows(-x), -q)
    b = O.bf16_round(x32)
    assert np.array_equal(O.fp8_rows(b), O.fp8_weight(b.astype(np.float32)))


def test_w8a8_logits_within_activation_error_bound():
    """W8A8 head logits differ from the weight-only FP8 head's by at most the
    activation quantisation error carried through |W~|: for every vocab row v,
    |l8_v - l_v| <= sum_k |s_v dec(q_vk)| e_k with e_k the half-step bound of
    row k's E4M3 activation. A dropped activation scale, a transposed operand
    or quantising the wrong tensor breaks it by orders of magnitude; the bound
    is also not vacuous (the observed error is a sizeable fraction of it)."""
    from dataclasses import replace
    geo = replace(synth.TINY, lm_head_dtype="fp8")
    w = synth.make_weights(geo)
    h_w = O.OracleHead(geo.as_dict(), w)
    h_a = O.OracleHead(replace(geo, lm_act_dtype="fp8").as_dict(), w)
    rng = np.random.default_rng(12)
    hid = rng.standard_normal((6, geo.hidden))
    lw, la = h_w.logits(hid), h_a.logits(hid)
    # the head's operand: the final-normed row as bf16 (exact in float32)
    z = O.gemm_input(O.rms_norm(hid, h_w.final_norm, h_w.eps))
    s = np.abs(z).max(axis=1) / 448.0
    e = np.maximum(np.abs(z) * 2.0 ** -4, s[:, None] * 2.0 ** -10)
    wabs = np.abs(h_w.lm) * h_w.lm_scale.astype(np.float64)[:, None]
    bound = e @ wabs.T
    # float64 summation order only
    slack = (np.abs(z) * 2.0 ** -40) @ wabs.T
    diff = np.abs(la - lw)
    assert np.all(diff <= bound + slack)
    assert diff.max() > 0.05 * bound.max()
    with pytest.raises(ValueError):
        O.OracleHead(replace(synth.TINY, lm_act_dtype="fp8").as_dict(), synth.make_weights(synth.TINY))
