"""GPU parity on the tiny geometry (1 layer, hidden 64, 4q/2kv heads of 16,
vocab 512, block 4, fp32 weights): the HIP library through the C ABI against
the float64 oracle on the same seeded inputs, plus the exact GPU invariants
(trim == recompute and block-table permutation, bit for bit)."""
import sys
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle.dflash import NO_TOKEN, OracleHead
from oracle.numerics import bf16_to_f64
from parity import Tally, as_u32, check_propose, split_batch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_draft_03_amd import load_library
    load_library()


def build(geo, w, **kw):
    from block_diffusion_draft_03_amd import Head
    kw.setdefault("kv_pool_blocks", 64)
    kw.setdefault("max_batch", 4)
    say(f"[build] {geo.num_layers}L h{geo.hidden} V{geo.vocab} W{geo.ctx_window} kv={geo.kv_dtype} head={geo.lm_head_dtype}")
    return Head(geo, w, **kw)


@pytest.fixture(scope="module")
def tiny():
    geo = synth.TINY
    w = synth.make_weights(geo)
    return geo, w, build(geo, w), OracleHead(geo.as_dict(), w)


@pytest.mark.parametrize("window", [4096, 8, 0])
@pytest.mark.parametrize("n_ctx", [32, 21, 0])
def test_tiny_propose_matches_oracle(window, n_ctx):
    geo = replace(synth.TINY, ctx_window=window)
    w = synth.make_weights(geo)
    head = build(geo, w)
    orc = OracleHead(geo.as_dict(), w)
    stack = synth.make_stack(geo, 32)[:n_ctx]
    st = head.state_create()
    os_ = orc.new_state()
    if n_ctx:
        head.precompute([st], [n_ctx], stack)
        orc.precompute(os_, stack)
    tally = Tally(f"tiny W={window} c={n_ctx}")
    for tok in synth.make_tokens(geo, 8, tag=window + n_ctx):
        say(f"[case] tiny W={window} c={n_ctx} tok={tok}")
        res = head.propose(st, int(tok), n_ctx, 3, logits=True)
        torch.cuda.synchronize()
        ref = orc.propose(os_, int(tok), n_ctx, 3)
        tally.add(check_propose(res, ref, label=f"W={window} c={n_ctx} tok={tok}"))
    tally.finish(min_pinned=1)
    head.destroy()


def test_tiny_kv_cache_matches_oracle(tiny):
    geo, w, head, orc = tiny
    stack = synth.make_stack(geo, 37, tag=7)
    st = head.state_create()
    os_ = orc.new_state()
    head.precompute([st], [20], stack[:20])
    head.precompute([st], [17], stack[20:])
    orc.precompute(os_, stack)
    k, v = head.read_kv(st, 0, 0, 37)
    torch.cuda.synchronize()
    kg = bf16_to_f64(k.cpu().numpy().view(np.uint16))
    vg = bf16_to_f64(v.cpu().numpy().view(np.uint16))
    kr = np.stack(os_.k[0])
    vr = np.stack(os_.v[0])
    # bf16 storage on both sides; the GPU's GEMM inputs are bf16-rounded
    assert np.abs(kg - kr).max() <= 2e-2 * np.abs(kr).max()
    assert np.abs(vg - vr).max() <= 2e-2 * np.abs(vr).max()
    st.free()


def test_tiny_multi_step_with_trim_matches_oracle(tiny):
    geo, w, head, orc = tiny
    st = head.state_create()
    os_ = orc.new_state()
    stacks = synth.make_stack(geo, 80, tag=11)
    used = 0
    acc = synth.make_accepted(6, 8, tag=3)
    tally = Tally("tiny multi-step trim")
    for step in range(6):
        n = 8
        head.precompute([st], [n], stacks[used:used + n])
        orc.precompute(os_, stacks[used:used + n])
        used += n
        head.after_verify(st, int(acc[step]))
        orc.after_verify(os_, int(acc[step]))
        assert st.ctx_len == os_.ctx_len
        tok = int(synth.make_tokens(geo, 1, tag=100 + step)[0])
        say(f"[case] tiny step {step} ctx {st.ctx_len}")
        res = head.propose(st, tok, st.ctx_len, 3, logits=True)
        torch.cuda.synchronize()
        tally.add(check_propose(res, orc.propose(os_, tok, os_.ctx_len, 3), label=f"step {step}"))
    tally.finish(min_pinned=1)
    st.free()


def _logits_of(head, st, tok=5):
    r = head.propose(st, tok, st.ctx_len, 3, logits=True)
    torch.cuda.synchronize()
    return r["logits"].cpu().numpy()


def test_tiny_trim_equals_recompute_bit_exact(tiny):
    geo, w, head, orc = tiny
    stack = synth.make_stack(geo, 28, tag=21)
    extra = stack[20:28]
    for a in (0, 3, 8):
        sa = head.state_create()
        head.precompute([sa], [20], stack[:20])
        head.after_verify(sa, 20)
        head.precompute([sa], [8], extra)
        head.after_verify(sa, a)
        sb = head.state_create()
        head.precompute([sb], [20 + a], np.concatenate([stack[:20], extra[:a]]))
        assert sa.ctx_len == sb.ctx_len == 20 + a
        la, lb = _logits_of(head, sa), _logits_of(head, sb)
        assert np.array_equal(la, lb), f"a={a}: max diff {np.abs(la - lb).max()}"
        sa.free()
        sb.free()


def test_tiny_shifted_rows_match_oracle():
    """The shifted-row convention: against the oracle with the same
    convention, and bit for bit the z-lab head's ids and probabilities
    rotated right by one (same logits)."""
    geo = synth.TINY
    w = synth.make_weights(geo)
    stack = synth.make_stack(geo, 32)
    res = {}
    for sh in (0, 1):
        g = replace(geo, shifted_rows=sh)
        head = build(g, w)
        orc = OracleHead(g.as_dict(), w)
        st, os_ = head.state_create(), orc.new_state()
        head.precompute([st], [32], stack)
        orc.precompute(os_, stack)
        say(f"[case] tiny shifted_rows={sh}")
        r = head.propose(st, 9, 32, 2, logits=True)
        torch.cuda.synchronize()
        check_propose(r, orc.propose(os_, 9, 32, 2), label=f"shifted={sh}")
        res[sh] = {k: r[k].cpu().numpy() for k in ("ids", "row_prob", "logits")}
        head.destroy()
    assert np.array_equal(res[1]["logits"], res[0]["logits"])
    assert np.array_equal(res[1]["ids"], np.roll(res[0]["ids"], 1))
    assert np.array_equal(res[1]["row_prob"], np.roll(res[0]["row_prob"], 1))


def test_tiny_kv_carry_across_turns(tiny):
    """take / install / free of a sequence's drafter KV ([DraftProposer]
    take_drafter_kv, install_drafter_kv, free_drafter_kv): a state given the
    carried blocks proposes bit for bit what the original state did (and
    matches the oracle); the emptied state proposes as a fresh one; blocks a
    live state holds are refused; freed blocks are free pool blocks again."""
    from block_diffusion_draft_03_amd import DflashError
    geo, w, head, orc = tiny
    stack = synth.make_stack(geo, 40, tag=51)
    a = head.state_create()
    head.precompute([a], [40], stack)
    head.after_verify(a, 40)
    la = _logits_of(head, a)
    blocks, rows, key = head.take_kv(a)
    assert rows == 40 and key == -1 and len(blocks) == 3 and a.ctx_len == 0
    assert head.take_kv(a) is None
    b = head.state_create()
    head.install_kv(b, blocks, rows, last_pair_key=7)
    assert b.ctx_len == 40
    say("[case] tiny carried KV")
    assert np.array_equal(_logits_of(head, b), la)
    os_ = orc.new_state()
    orc.precompute(os_, stack)
    res = head.propose(b, 5, 40, 3, logits=True)
    torch.cuda.synchronize()
    check_propose(res, orc.propose(os_, 5, 40, 3), label="carried")
    res = head.propose(a, 5, 0, 3, logits=True)
    torch.cuda.synchronize()
    check_propose(res, orc.propose(orc.new_state(), 5, 0, 3), label="emptied")
    with pytest.raises(DflashError):
        head.install_kv(a, blocks, rows)  # b holds them
    blocks2, rows2, key2 = head.take_kv(b)
    assert key2 == 7 and rows2 == 40 and np.array_equal(blocks2, blocks)
    head.free_kv(blocks2)
    with pytest.raises(DflashError):
        head.free_kv(blocks2)  # already free
    c = head.state_create(block_ids=blocks2)  # explicit blocks must be free pool blocks
    for s in (a, b, c):
        s.free()


def test_tiny_block_permutation_bit_exact(tiny):
    geo, w, head, orc = tiny
    stack = synth.make_stack(geo, 40, tag=31)
    s1 = head.state_create()
    perm = synth.make_block_permutation(3, 64, tag=1)
    s2 = head.state_create(block_ids=perm)
    head.precompute([s1], [40], stack)
    head.precompute([s2], [40], stack)
    assert np.array_equal(_logits_of(head, s1), _logits_of(head, s2))
    s1.free()
    s2.free()


def test_tiny_batch_matches_single_and_oracle(tiny):
    geo, w, head, orc = tiny
    lens = [3, 17, 32, 0]
    states, ostates = [], []
    for i, n in enumerate(lens):
        st = head.state_create()
        os_ = orc.new_state()
        if n:
            stk = synth.make_stack(geo, n, tag=200 + i)
            head.precompute([st], [n], stk)
            orc.precompute(os_, stk)
        states.append(st)
        ostates.append(os_)
    toks = synth.make_tokens(geo, 4, tag=9)
    pos = [s.ctx_len for s in states]
    masks = np.stack([synth.make_bitmask(geo.vocab, 0.5, tag=i) for i in range(4)])
    say("[case] tiny batch of 4 with masks")
    res = head.propose_batch(states, toks, pos, 3, bitmasks=masks, logits=True)
    torch.cuda.synchronize()
    tally = Tally("tiny batch of 4")
    for i in range(4):
        ref = orc.propose(ostates[i], int(toks[i]), pos[i], 3, masks[i])
        tally.add(check_propose(split_batch(res, i), ref, bitmask=masks[i], label=f"batch seq {i}"))
        single = head.propose(states[i], int(toks[i]), pos[i], 3, bitmask=masks[i], logits=True)
        torch.cuda.synchronize()
        assert np.array_equal(as_u32(single["ids"]), as_u32(res["ids"][i]))
        assert np.allclose(single["logits"].cpu().numpy(), res["logits"][i].cpu().numpy(), atol=1e-5)
    tally.finish(min_pinned=1)
    for s in states:
        s.free()


def test_tiny_mask_special_cases(tiny):
    geo, w, head, orc = tiny
    stack = synth.make_stack(geo, 32)
    st = head.state_create()
    head.precompute([st], [32], stack)
    words = (geo.vocab + 31) // 32
    base = head.propose(st, 5, 32, 3)
    ones = np.full(words, -1, dtype=np.int32)
    allm = head.propose(st, 5, 32, 3, bitmask=ones)
    torch.cuda.synchronize()
    assert np.array_equal(as_u32(base["ids"]), as_u32(allm["ids"]))
    assert np.array_equal(base["row_prob"].cpu().numpy(), allm["row_prob"].cpu().numpy())
    for tok in (0, 31, 32, 511):
        m = np.zeros(words, dtype=np.int32)
        m[tok >> 5] = np.uint32(1 << (tok & 31)).view(np.int32)
        r = head.propose(st, 5, 32, 3, bitmask=m)
        torch.cuda.synchronize()
        assert as_u32(r["ids"]).tolist() == [tok] * geo.gamma
        assert r["row_prob"].cpu().numpy().tolist() == [1.0] * geo.gamma
    r = head.propose(st, 5, 32, 3, bitmask=np.zeros(words, dtype=np.int32))
    torch.cuda.synchronize()
    assert as_u32(r["ids"]).tolist() == [NO_TOKEN] * geo.gamma
    assert r["row_prob"].cpu().numpy().tolist() == [0.0] * geo.gamma
    assert float(r["conf"].cpu()[0]) == 0.0
    st.free()


def test_tiny_zero_final_gain_and_ties():
    geo = synth.TINY
    w = synth.make_weights(geo)
    w0 = dict(w)
    w0["norm"] = np.zeros_like(w["norm"])
    head = build(geo, w0)
    st = head.state_create()
    head.precompute([st], [32], synth.make_stack(geo, 32))
    r = head.propose(st, 3, 32, 3, logits=True)
    torch.cuda.synchronize()
    assert np.all(r["logits"].cpu().numpy() == 0.0)
    assert as_u32(r["ids"]).tolist() == [0] * geo.gamma
    assert np.allclose(r["row_prob"].cpu().numpy(), 1.0 / geo.vocab, rtol=1e-5)
    head.destroy()
    # duplicate LM rows: identical logits, the lower id wins, whichever of the
    # two is the copy (the copy placed below the observed argmax a, and above)
    head = build(geo, w)
    st = head.state_create()
    head.precompute([st], [32], synth.make_stack(geo, 32))
    r = head.propose(st, 3, 32, 3)
    torch.cuda.synchronize()
    a = int(as_u32(r["ids"])[1])
    head.destroy()
    for b in ((a + 1) % geo.vocab, (a - 1) % geo.vocab, (a + 37) % geo.vocab):
        w2 = dict(w)
        lm = w["lm_head"].copy()
        lm[b] = lm[a]
        w2["lm_head"] = lm
        head = build(geo, w2)
        st = head.state_create()
        head.precompute([st], [32], synth.make_stack(geo, 32))
        say(f"[case] tiny tie a={a} b={b}")
        r = head.propose(st, 3, 32, 3, logits=True)
        torch.cuda.synchronize()
        lg = r["logits"].cpu().numpy()
        assert lg[1, b] == lg[1, a]
        assert int(as_u32(r["ids"])[1]) == min(a, b)
        head.destroy()


def test_tiny_error_paths(tiny):
    from block_diffusion_draft_03_amd import DflashError
    geo, w, head, orc = tiny
    st = head.state_create(budget_tokens=16)
    with pytest.raises(DflashError, match="E_NO_BLOCKS"):
        head.precompute([st], [17], synth.make_stack(geo, 17))
    assert st.ctx_len == 0
    with pytest.raises(DflashError, match="E_INVALID"):
        head.propose(st, geo.vocab, 0, 3)           # token out of range
    with pytest.raises(DflashError, match="E_INVALID"):
        head.propose(st, 1, 0, geo.gamma)           # num_drafts > gamma - 1
    with pytest.raises(DflashError, match="E_INVALID"):
        head.after_verify(st, 1)                    # nothing pending
    with pytest.raises(DflashError, match="E_DECLINED"):
        head.propose_batch([st] * 5, [1] * 5, [0] * 5, 3)   # max_batch is 4
    st.free()
