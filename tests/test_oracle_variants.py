"""Pins for the oracle's storage-format variants, its margin helper and the
interior of its YaRN table (CPU only).

* The FP8 KV cache, the FP8 LM-head mirror (weight-only and with E4M3
  activation rows), FP8 drafter weights, a given RoPE table and the shifted
  draft-row convention are each checked against the explicit-loop twin
  (oracle/brute.py), which has its own scalar E4M3 codec. Planted mistakes
  (K and V scales swapped, kv heads' scales swapped, the mirror's row scale
  dropped) are shown to break the agreement, so the comparison is not
  vacuous.
* ``top2_margin`` decides which rows' ids the GPU tests compare; it is
  checked on hand-built rows and against a scan.
* The YaRN table is checked at every pair index against YaRN's
  NTK-by-parts definition evaluated in its wavelength-ratio form: the pairs
  that turn at least beta_fast times over the original context keep their
  frequency, those that turn at most beta_slow times are divided by the
  factor, and the blend weight between them falls linearly in the pair index
  (the reading), not linearly in the number of turns.
"""
import math
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import dflash as O
from oracle.brute import _e4m3, brute_propose
from oracle.numerics import e4m3_decode, e4m3_encode


def _case(geo, seed=0, n_ctx=32, **w_over):
    w = synth.make_weights(geo, seed=seed)
    w.update(w_over)
    stack = synth.make_stack(geo, n_ctx, tag=seed)
    return w, stack


def _oracle_propose(geo_d, w, stack, tok, pos, nd, mask=None):
    head = O.OracleHead(geo_d, w)
    st = head.new_state()
    head.precompute(st, stack)
    return head.propose(st, tok, pos, nd, mask)


def _agree(res, brute, rtol=1e-9):
    ids, probs, conf, logits = brute
    return (np.allclose(res["logits"], np.array(logits), rtol=rtol, atol=1e-12)
            and res["ids"].tolist() == ids
            and np.allclose(res["row_prob"], probs, rtol=rtol)
            and math.isclose(res["conf"], conf, rel_tol=rtol))


# --------------------------------------------------------------------------
# the twin's own codec
# --------------------------------------------------------------------------

def test_brute_e4m3_codec_matches_torch_and_numerics():
    """The twin's scalar E4M3 rounding equals torch.float8_e4m3fn in range and
    the oracle's codec everywhere (saturation included), on random values
    spanning the subnormal and normal range and on exact ties."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 9, 20000))
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = e4m3_decode(codes)
    ties = (vals[:-1] + vals[1:]) / 2  # halfway between neighbouring codes
    x = np.concatenate([x, ties, -ties, vals, [500.0, -1e4, 449.0, 464.0]])
    ours = np.array([_e4m3(float(v)) for v in x])
    assert np.array_equal(ours, e4m3_decode(e4m3_encode(x)))
    inr = np.abs(x) <= 448.0
    t = torch.from_numpy(x[inr]).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours[inr], t)


# --------------------------------------------------------------------------
# FP8 KV cache
# --------------------------------------------------------------------------

def _distinct_kv_scales(geo):
    """One scale per (layer, K|V, kv head), all different: V's grid twice as
    coarse as K's, head g's 1.5^g times head 0's. K's is small enough that
    a few percent of the K values saturate at +-448 s."""
    sigma = 0.02 * math.sqrt(geo.hidden)
    s = np.empty((geo.num_layers, 2, geo.num_kv_heads), dtype=np.float32)
    for l in range(geo.num_layers):
        for g in range(geo.num_kv_heads):
            s[l, 0, g] = sigma * 2.0 / 448.0 * 1.5 ** g * (1 + 0.1 * l)
            s[l, 1, g] = sigma * 4.0 / 448.0 * 1.5 ** g * (1 + 0.1 * l)
    return s


def test_brute_twin_fp8_kv_cache():
    geo = replace(synth.TINY, kv_dtype="fp8")
    scales = _distinct_kv_scales(geo)
    w, stack = _case(geo, seed=3, kv_scale=scales)
    gd = geo.as_dict()
    res = _oracle_propose(gd, w, stack, 17, 32, 3)
    brute = brute_propose(gd, w, stack, 17, 32, 3)
    assert _agree(res, brute)
    # some K values do saturate under these scales
    head = O.OracleHead(gd, w)
    st = head.new_state()
    head.precompute(st, stack)
    k = np.stack(head.ctx_kv(head.ctx_features(stack), np.arange(32))[0][0])
    assert np.any(np.abs(k) == 448.0 * scales[0, 0][None, :, None].astype(np.float64))
    # planted mistakes in the oracle's inputs break the agreement
    swapped_kv = dict(w, kv_scale=scales[:, ::-1, :].copy())
    assert not _agree(_oracle_propose(gd, swapped_kv, stack, 17, 32, 3), brute, rtol=1e-6)
    swapped_heads = dict(w, kv_scale=scales[:, :, ::-1].copy())
    assert not _agree(_oracle_propose(gd, swapped_heads, stack, 17, 32, 3), brute, rtol=1e-6)


def test_brute_twin_fp8_kv_cache_window_and_mask():
    geo = replace(synth.TINY, kv_dtype="fp8", ctx_window=8, num_layers=2)
    w, stack = _case(geo, seed=4, n_ctx=21, kv_scale=_distinct_kv_scales(geo))
    bm = synth.make_bitmask(geo.vocab, 0.5, tag=4)
    gd = geo.as_dict()
    assert _agree(_oracle_propose(gd, w, stack, 9, 23, 2, bm), brute_propose(gd, w, stack, 9, 23, 2, bm))


# --------------------------------------------------------------------------
# FP8 LM head, W8A8 head, FP8 drafter weights
# --------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_brute_twin_fp8_lm_head(act):
    geo = replace(synth.TINY, lm_head_dtype="fp8", lm_act_dtype=act)
    w, stack = _case(geo, seed=5)
    bm = synth.make_bitmask(geo.vocab, 0.5, tag=5)
    gd = geo.as_dict()
    brute = brute_propose(gd, w, stack, 100, 32, 3, bm)
    assert _agree(_oracle_propose(gd, w, stack, 100, 32, 3, bm), brute)
    # dropping the mirror's row scale breaks it
    head = O.OracleHead(gd, w)
    head.lm_scale = np.ones_like(head.lm_scale)
    st = head.new_state()
    head.precompute(st, stack)
    assert not _agree(head.propose(st, 100, 32, 3, bm), brute, rtol=1e-6)


def test_brute_twin_fp8_drafter_weights():
    geo = replace(synth.TINY, layer_dtype="fp8", lm_head_dtype="fp8")
    w, stack = _case(geo, seed=6)
    gd = geo.as_dict()
    brute = brute_propose(gd, w, stack, 3, 32, 3)
    assert _agree(_oracle_propose(gd, w, stack, 3, 32, 3), brute)
    # the drafter matrices are quantised (the bf16-weight head differs)
    plain = replace(synth.TINY, lm_head_dtype="fp8").as_dict()
    assert not _agree(_oracle_propose(plain, w, stack, 3, 32, 3), brute, rtol=1e-6)


def test_brute_twin_yarn_table_and_shifted_rows():
    geo = replace(synth.TINY, shifted_rows=1)
    w, stack = _case(geo, seed=7)
    gd = geo.as_dict()
    gd["inv_freq"] = O.yarn_inv_freq(geo.rope_theta, geo.head_dim, 64.0, 32.0, 1.0, 4096)
    assert _agree(_oracle_propose(gd, w, stack, 44, 32, 3), brute_propose(gd, w, stack, 44, 32, 3))


# --------------------------------------------------------------------------
# top-2 margin
# --------------------------------------------------------------------------

def test_top2_margin_hand_built_rows():
    ninf = -np.inf
    lg = np.array([[3.0, 1.0, 2.0, 0.5],      # 3 - 2
                   [5.0, 5.0, 1.0, 0.0],      # a tie: 0
                   [-1.0, -3.0, -2.0, -9.0],  # negatives: -1 - (-2)
                   [0.0, 7.0, 0.0, 6.75]])    # 7 - 6.75
    m = O.top2_margin(lg)
    assert m.tolist() == [1.0, 0.0, 1.0, 0.25]
    # the margin is taken on the masked logits: masking the top of row 0
    # leaves 2 - 1; a single allowed token leaves +inf; nothing allowed, nan
    words = np.array([np.uint32(0b1110).view(np.int32)])
    assert O.top2_margin(lg[:1], words).tolist() == [1.0]
    one = np.array([np.uint32(0b0100).view(np.int32)])
    assert O.top2_margin(lg[:1], one).tolist() == [np.inf]
    with np.errstate(invalid="ignore"):
        none = O.top2_margin(lg[:1], np.zeros(1, np.int32))
    assert np.isnan(none[0])
    # -inf entries already in the logits are ignored the same way
    assert O.top2_margin(np.array([[ninf, 4.0, ninf, 3.5]])).tolist() == [0.5]


def test_top2_margin_matches_scan():
    rng = np.random.default_rng(8)
    V = 248320
    lg = rng.standard_normal((3, V)) * 0.9
    lg[1, 1234] = lg[1, 99] = lg[1].max() + 1.0  # tie at the top
    bm = synth.make_bitmask(V, 0.5, tag=3)
    allowed = ((bm.view(np.uint32)[np.arange(V) >> 5] >> (np.arange(V) & 31)) & 1) == 1
    got = O.top2_margin(lg, bm)
    for r in range(3):
        best = second = -math.inf
        for x in lg[r][allowed].tolist():
            if x > best:
                best, second = x, best
            elif x > second:
                second = x
        assert got[r] == best - second


# --------------------------------------------------------------------------
# YaRN table, every pair
# --------------------------------------------------------------------------

@pytest.mark.parametrize("theta,d", [(1e7, 128), (1e6, 64), (1e6, 16)])
def test_yarn_table_every_pair_against_wavelength_form(theta, d):
    L, beta_fast, beta_slow, factor = 4096, 32.0, 1.0, 64.0
    y = O.yarn_inv_freq(theta, d, factor, beta_fast, beta_slow, L)
    half = d // 2
    w = [theta ** (-2.0 * i / d) for i in range(half)]
    turns = [L * wi / (2.0 * math.pi) for wi in w]   # r = L / wavelength
    # regime edges from the turns themselves (no pair-index formula)
    lo = max(i for i in range(half) if turns[i] >= beta_fast)
    hi = min(i for i in range(half) if turns[i] <= beta_slow)
    assert 0 <= lo < hi < half
    for i in range(half):
        # NTK-by-parts: y = (1 - g) w / s + g w; recover the weight g of the
        # unchanged frequency (exact up to the table's float32 rounding)
        g = (y[i] / w[i] - 1.0 / factor) / (1.0 - 1.0 / factor)
        want = 1.0 if i <= lo else 0.0 if i >= hi else (hi - i) / (hi - lo)
        assert abs(g - want) <= 2.0 ** -22, (i, g, want)
    # the reading's ramp is linear in the pair index; a ramp linear in the
    # number of turns (clamp((r - beta_slow) / (beta_fast - beta_slow))) differs
    # inside the band, so it would not pass the check above
    gw = [min(1.0, max(0.0, (turns[i] - beta_slow) / (beta_fast - beta_slow))) for i in range(half)]
    assert max(abs(gw[i] - (hi - i) / (hi - lo)) for i in range(lo + 1, hi)) > 0.05
