"""GPU parity on mid-size geometries that the tiny and full ones leave out:
head_dim 32 and 64 with a bf16 KV cache, head_dim 64 with an E4M3 KV cache
and LM head, a ctx window shorter than the context, and blocks of 64 and 33
rows (two block tiles in the attention, the second full or holding one row). Two layers, hidden
256, vocab 2048, block of 16. A ragged batch of six sequences (0 to 300 ctx
rows, so several 32-key tiles, partial blocks and an empty context) runs
through the batched path (96 rows: tiled GEMMs and LM head), and one
sequence through the single-sequence path; both are checked against the
float64 oracle on the same seeded inputs."""
import sys
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle.dflash import OracleHead
from parity import Tally, as_u32, check_propose, split_batch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MID = synth.Geometry(num_layers=2, hidden=256, intermediate=512, num_q_heads=8, num_kv_heads=2, head_dim=32,
                     vocab=2048, gamma=16, mask_token_id=2047, num_target_layers=2, target_hidden=256,
                     ctx_window=4096, rope_theta=1e6, rms_eps=1e-6)
CASES = {
    "d32": MID,
    "d64": replace(MID, num_q_heads=4, head_dim=64),
    "d64_window100": replace(MID, num_q_heads=4, head_dim=64, ctx_window=100),
    "d64_fp8": replace(MID, num_q_heads=4, head_dim=64, kv_dtype="fp8", lm_head_dtype="fp8"),
    # the largest block (two 32-row block tiles; the single-sequence forward has 64 rows) and
    # a ragged one (the second block tile holds one row)
    "d64_gamma64": replace(MID, num_q_heads=4, head_dim=64, gamma=64),
    "d64_gamma33_fp8": replace(MID, num_q_heads=4, head_dim=64, gamma=33, kv_dtype="fp8", lm_head_dtype="fp8"),
    # one query head per kv head, and one kv head for all query heads
    "d64_mha": replace(MID, num_q_heads=4, num_kv_heads=4, head_dim=64),
    "d64_mqa": replace(MID, num_q_heads=4, num_kv_heads=1, head_dim=64),
    # a vocabulary that the tiled LM head's 256-row blocks do not divide: the
    # batch takes the weight-streaming LM head in 64-row chunks
    "d64_vocab2176": replace(MID, num_q_heads=4, head_dim=64, vocab=2176, mask_token_id=2175),
    # the YaRN-corrected RoPE table of the drafter's rope_scaling (factor 64, beta_fast 32,
    # beta_slow 1, 4096 original positions): at head_dim 64 and theta 1e6 pairs 0-6 keep their
    # frequency, 7-15 blend, 16-31 are divided by 64
    "d64_yarn": replace(MID, num_q_heads=4, head_dim=64),
    # FP8 drafter weights (every drafter matrix as E4M3 + row scales; bf16 head and cache);
    # the batch of 96 rows takes the weight-streaming GEMMs in 64-row chunks
    "d64_fp8w": replace(MID, num_q_heads=4, head_dim=64, layer_dtype="fp8"),
    # W8A8 LM head (E4M3 activation rows on the E4M3 matrix cores; every propose, the single
    # one included, takes the tiled head), with a full and a ragged block
    "d64_fp8a8": replace(MID, num_q_heads=4, head_dim=64, kv_dtype="fp8", lm_head_dtype="fp8", lm_act_dtype="fp8"),
    "d64_gamma33_fp8a8": replace(MID, num_q_heads=4, head_dim=64, gamma=33, lm_head_dtype="fp8",
                                 lm_act_dtype="fp8"),
}
YARN = {"d64_yarn": (64.0, 32.0, 1.0, 4096)}
LENS = [0, 17, 64, 300, 129, 45]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_draft_03_amd import load_library
    load_library()


@pytest.mark.parametrize("case", list(CASES))
def test_mid_batch_and_single_match_oracle(case):
    from block_diffusion_draft_03_amd import Head, yarn_inv_freq
    from oracle.dflash import yarn_inv_freq as oracle_yarn
    geo = CASES[case]
    fp8 = geo.lm_head_dtype == "fp8"
    w = synth.make_weights(geo)
    say(f"[build] mid {case}")
    table, ogeo = None, geo.as_dict()
    if case in YARN:
        table = yarn_inv_freq(geo.head_dim, geo.rope_theta, *YARN[case])
        ogeo["inv_freq"] = oracle_yarn(geo.rope_theta, geo.head_dim, *YARN[case])
        assert np.allclose(table.astype(np.float64), ogeo["inv_freq"], rtol=2.0 ** -23, atol=0.0)
    head = Head(geo, w, kv_pool_blocks=160, max_batch=len(LENS), max_seq_len=1024, inv_freq=table)
    orc = OracleHead(ogeo, w)
    states, ostates = [], []
    for i, n in enumerate(LENS):
        st = head.state_create()
        os_ = orc.new_state()
        if n:
            stk = synth.make_stack(geo, n, tag=900 + i)
            head.precompute([st], [n], stk)
            orc.precompute(os_, stk)
        states.append(st)
        ostates.append(os_)
    toks = synth.make_tokens(geo, len(LENS), tag=31)
    pos = [s.ctx_len for s in states]
    masks = np.stack([synth.make_bitmask(geo.vocab, 0.5, tag=40 + i) for i in range(len(LENS))]) if fp8 else None
    tol = 6e-2 if fp8 else 2e-2
    say(f"[case] mid {case} batch of {len(LENS)}")
    res = head.propose_batch(states, toks, pos, geo.gamma - 1, bitmasks=masks, logits=True)
    torch.cuda.synchronize()
    tally = Tally(f"mid {case}")
    for i in range(len(LENS)):
        mk = None if masks is None else masks[i]
        ref = orc.propose(ostates[i], int(toks[i]), pos[i], geo.gamma - 1, mk)
        tally.add(check_propose(split_batch(res, i), ref, bitmask=mk, logit_tol=tol,
                                label=f"{case} batch seq {i} ctx {pos[i]}"))
    say(f"[case] mid {case} single")
    i = 3
    mk = None if masks is None else masks[i]
    res1 = head.propose(states[i], int(toks[i]), pos[i], geo.gamma - 1, bitmask=mk, logits=True)
    torch.cuda.synchronize()
    ref = orc.propose(ostates[i], int(toks[i]), pos[i], geo.gamma - 1, mk)
    tally.add(check_propose(res1, ref, bitmask=mk, logit_tol=tol, label=f"{case} single ctx {pos[i]}"))
    tally.finish(min_pinned=1)
    for s in states:
        s.free()
    head.destroy()


@pytest.mark.parametrize("case", ["d64", "d64_fp8", "d64_fp8w"])
def test_mid_prompt_scale_precompute_matches_oracle(case):
    """Precompute of many rows in one call (passes of up to 1024 rows through
    the tiled GEMMs: 300 rows in one pass; 1100 rows over two sequences in two
    passes, the second a ragged 76): the cache against the oracle's K/V, then a
    propose over it."""
    from oracle.numerics import bf16_to_f64, e4m3_decode
    from block_diffusion_draft_03_amd import Head
    geo = CASES[case]
    fp8 = geo.kv_dtype == "fp8"
    w = synth.make_weights(geo)
    say(f"[build] mid prefill {case}")
    head = Head(geo, w, kv_pool_blocks=200, max_batch=2, max_seq_len=2048)
    orc = OracleHead(geo.as_dict(), w)
    for lens in ([300], [700, 400]):
        say(f"[case] mid prefill {case} rows {lens}")
        sts = [head.state_create() for _ in lens]
        oss = [orc.new_state() for _ in lens]
        stacks = [synth.make_stack(geo, n, tag=1200 + i + len(lens)) for i, n in enumerate(lens)]
        head.precompute(sts, lens, np.concatenate(stacks))
        for os_, stk in zip(oss, stacks):
            orc.precompute(os_, stk)
        for i, n in enumerate(lens):
            for layer in (0, geo.num_layers - 1):
                k, v = head.read_kv(sts[i], layer, 0, n)
                torch.cuda.synchronize()
                kr = np.stack(oss[i].k[layer])
                vr = np.stack(oss[i].v[layer])
                if fp8:
                    sk = w["kv_scale"][layer, 0].astype(np.float64)
                    sv = w["kv_scale"][layer, 1].astype(np.float64)
                    kg = e4m3_decode(k.cpu().numpy()) * sk[None, :, None]
                    vg = e4m3_decode(v.cpu().numpy()) * sv[None, :, None]
                    # one E4M3 step (2^-3 relative) plus the bf16 rounding of the GEMM inputs
                    assert np.all(np.abs(kg - kr) <= np.maximum(np.abs(kr) * 2.0 ** -3, sk[None, :, None] * 2.0 ** -9) + 1e-2)
                    assert np.all(np.abs(vg - vr) <= np.maximum(np.abs(vr) * 2.0 ** -3, sv[None, :, None] * 2.0 ** -9) + 1e-2)
                else:
                    kg = bf16_to_f64(k.cpu().numpy().view(np.uint16))
                    vg = bf16_to_f64(v.cpu().numpy().view(np.uint16))
                    assert np.abs(kg - kr).max() <= 2e-2 * np.abs(kr).max()
                    assert np.abs(vg - vr).max() <= 2e-2 * np.abs(vr).max()
        tok = int(synth.make_tokens(geo, 1, tag=55)[0])
        tally = Tally(f"mid prefill {case} {lens}")
        for st, os_ in zip(sts, oss):
            res = head.propose(st, tok, st.ctx_len, geo.gamma - 1, logits=True)
            torch.cuda.synchronize()
            ref = orc.propose(os_, tok, os_.ctx_len, geo.gamma - 1)
            tally.add(check_propose(res, ref, logit_tol=6e-2 if geo.lm_head_dtype == "fp8" else 2e-2,
                                    label=f"{case} after {lens}"))
        tally.finish(min_pinned=1)
        for st in sts:
            st.free()
    head.destroy()


@pytest.mark.parametrize("case", ["bf16", "fp8a8"])
def test_mid_largest_batch_matches_oracle(case):
    """The largest call the library takes: 64 sequences (the batch ceiling) of
    64 block rows (the block ceiling), 4096 rows in one propose_batch, so the
    tiled LM head runs sixteen 256-row activation blocks per vocab range;
    contexts of 0..40 rows (empty ones included). bf16 head, and the W8A8
    head over an E4M3 cache with grammar masks. Every sequence is checked."""
    from block_diffusion_draft_03_amd import Head
    geo = replace(MID, num_q_heads=4, head_dim=64, gamma=64)
    if case == "fp8a8":
        geo = replace(geo, kv_dtype="fp8", lm_head_dtype="fp8", lm_act_dtype="fp8")
    fp8 = geo.lm_head_dtype == "fp8"
    n = 64
    w = synth.make_weights(geo)
    say(f"[build] mid largest batch {case}")
    head = Head(geo, w, kv_pool_blocks=n * 8, max_batch=n, max_seq_len=256)
    orc = OracleHead(geo.as_dict(), w)
    lens = synth.make_ctx_lengths(n, 0, 40, tag=77)
    lens[0] = 0
    states, ostates = [], []
    for i in range(n):
        st, os_ = head.state_create(), orc.new_state()
        if lens[i]:
            stk = synth.make_stack(geo, int(lens[i]), tag=1200 + i)
            head.precompute([st], [int(lens[i])], stk)
            orc.precompute(os_, stk)
        states.append(st)
        ostates.append(os_)
    toks = synth.make_tokens(geo, n, tag=78)
    pos = [s.ctx_len for s in states]
    masks = np.stack([synth.make_bitmask(geo.vocab, 0.5, tag=300 + i) for i in range(n)]) if fp8 else None
    say(f"[case] mid largest batch {case}: {n} x {geo.gamma} rows")
    res = head.propose_batch(states, toks, pos, geo.gamma - 1, bitmasks=masks, logits=True)
    torch.cuda.synchronize()
    tally = Tally(f"mid largest batch {case}")
    for i in range(n):
        mk = None if masks is None else masks[i]
        ref = orc.propose(ostates[i], int(toks[i]), pos[i], geo.gamma - 1, mk)
        tally.add(check_propose(split_batch(res, i), ref, bitmask=mk, logit_tol=6e-2 if fp8 else 2e-2,
                                label=f"largest {case} seq {i} ctx {pos[i]}"))
    tally.finish(min_pinned=1)
    for s in states:
        s.free()
    head.destroy()


# vocab offsets from the argmax a that place its copy, in the tiled LM head's
# 256-row vocab blocks (local row (wave * 8 + tile) * 16 + 4 * lane group + r),
# in the same lane, the neighbouring lane group, another 16-row tile of the
# same lanes, the other wave of the row, another vocab block of the workgroup
# and another workgroup's vocab range
TIE_XOR = {"same lane": 1, "lane group": 4, "tile": 16, "wave": 128, "vocab block": 256, "vocab range": 1024}


@pytest.mark.parametrize("case", ["d64", "d64_fp8", "d64_fp8a8"])
def test_mid_tiled_head_ties_and_empty_mask(case):
    """The tiled LM head (a batch of six sequences, 96 rows; bf16, E4M3 and
    W8A8 heads): a copy of a row's argmax vocab row at each of the placements
    above gives bit-identical logits and the lower id wins; a sequence whose
    mask allows nothing gets DFLASH_NO_TOKEN, p1 = 0 and confidence 0 on
    every entry while the others match the oracle."""
    from block_diffusion_draft_03_amd import Head
    from oracle.dflash import NO_TOKEN
    geo = CASES[case]
    w = synth.make_weights(geo)
    words = (geo.vocab + 31) // 32
    n = len(LENS)
    masks = np.full((n, words), -1, dtype=np.int32)
    masks[2] = 0
    stacks = [synth.make_stack(geo, ln, tag=900 + i) for i, ln in enumerate(LENS)]
    toks = synth.make_tokens(geo, n, tag=31)

    def run(wts):
        head = Head(geo, wts, kv_pool_blocks=160, max_batch=n, max_seq_len=1024)
        states = [head.state_create() for _ in range(n)]
        for st, stk, ln in zip(states, stacks, LENS):
            if ln:
                head.precompute([st], [ln], stk)
        res = head.propose_batch(states, toks, list(LENS), geo.gamma - 1, bitmasks=masks, logits=True)
        torch.cuda.synchronize()
        out = {k: v.cpu().numpy() for k, v in res.items()}
        for st in states:
            st.free()
        head.destroy()
        return out

    say(f"[case] mid tiled head {case}: base and empty mask")
    base = run(w)
    assert as_u32(base["ids"][2]).tolist() == [NO_TOKEN] * geo.gamma
    assert base["row_prob"][2].tolist() == [0.0] * geo.gamma and float(base["conf"][2]) == 0.0
    orc = OracleHead(geo.as_dict(), w)
    tally = Tally(f"mid tiled head {case}")
    for i in range(n):
        os_ = orc.new_state()
        if LENS[i]:
            orc.precompute(os_, stacks[i])
        ref = orc.propose(os_, int(toks[i]), LENS[i], geo.gamma - 1, masks[i])
        tally.add(check_propose(split_batch(base, i), ref, bitmask=masks[i], logit_tol=6e-2 if "fp8" in case else 2e-2,
                                label=f"{case} seq {i}"))
    tally.finish(min_pinned=1)
    seq, row = 1, 1
    a = int(as_u32(base["ids"][seq])[row])
    for where, x in TIE_XOR.items():
        b = a ^ x
        w2 = dict(w)
        lm = w["lm_head"].copy()
        lm[b] = lm[a]
        w2["lm_head"] = lm
        say(f"[case] mid tiled head {case}: tie {where} a={a} b={b}")
        out = run(w2)
        lg = out["logits"][seq, row]
        assert lg[a] == lg[b], where
        assert int(as_u32(out["ids"][seq])[row]) == min(a, b), where
        assert as_u32(out["ids"][2]).tolist() == [NO_TOKEN] * geo.gamma
