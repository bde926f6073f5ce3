"""GPU parity on mid-size geometries that the tiny and full ones leave out:
head_dim 32 and 64 with a bf16 KV cache, head_dim 64 with an E4M3 KV cache
and LM head, and a ctx window shorter than the context. Two layers, hidden
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
from parity import check_propose, split_batch

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
}
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
    from block_diffusion_draft_03_amd import Head
    geo = CASES[case]
    fp8 = geo.lm_head_dtype == "fp8"
    w = synth.make_weights(geo)
    say(f"[build] mid {case}")
    head = Head(geo, w, kv_pool_blocks=160, max_batch=len(LENS), max_seq_len=1024)
    orc = OracleHead(geo.as_dict(), w)
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
    for i in range(len(LENS)):
        mk = None if masks is None else masks[i]
        ref = orc.propose(ostates[i], int(toks[i]), pos[i], geo.gamma - 1, mk)
        check_propose(split_batch(res, i), ref, bitmask=mk, logit_tol=tol, label=f"{case} batch seq {i} ctx {pos[i]}")
    say(f"[case] mid {case} single")
    i = 3
    mk = None if masks is None else masks[i]
    res1 = head.propose(states[i], int(toks[i]), pos[i], geo.gamma - 1, bitmask=mk, logits=True)
    torch.cuda.synchronize()
    ref = orc.propose(ostates[i], int(toks[i]), pos[i], geo.gamma - 1, mk)
    check_propose(res1, ref, bitmask=mk, logit_tol=tol, label=f"{case} single ctx {pos[i]}")
    for s in states:
        s.free()
    head.destroy()
