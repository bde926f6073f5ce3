"""dflash_propose_noalloc (the propose whose scratch lives in the library's
static device array, for callers that cannot allocate) against
dflash_propose, through the C ABI: the same outputs bit for bit on two calls
in a row, the second with a smaller input (a smaller geometry, block and
context, so stale contents of the shared array from the first call would
show), then a W8A8 head; no device memory is allocated by the call; a
propose that needs more scratch than the array holds is refused before
anything is enqueued."""
import sys
from dataclasses import replace

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MID = synth.Geometry(num_layers=2, hidden=256, intermediate=512, num_q_heads=4, num_kv_heads=2, head_dim=64,
                     vocab=2048, gamma=16, mask_token_id=2047, num_target_layers=2, target_hidden=256,
                     ctx_window=4096, rope_theta=1e6, rms_eps=1e-6)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(geo, dev="cuda"):
    g = geo.gamma
    return {"ids": torch.full((g,), -7, dtype=torch.int32, device=dev),
            "conf": torch.full((1,), -7.0, dtype=torch.float32, device=dev),
            "row_prob": torch.full((g,), -7.0, dtype=torch.float32, device=dev),
            "logits": torch.full((g, geo.vocab), -7.0, dtype=torch.float32, device=dev)}


def _compare(head, geo, n_ctx, tag, label):
    """One state of n_ctx rows; dflash_propose, then dflash_propose_noalloc
    (twice), all bit for bit equal."""
    st = head.state_create()
    if n_ctx:
        head.precompute([st], [n_ctx], synth.make_stack(geo, n_ctx, tag=tag))
    tok = int(synth.make_tokens(geo, 1, tag=tag)[0])
    mask = synth.make_bitmask(geo.vocab, 0.5, tag=tag) if geo.lm_head_dtype == "fp8" else None
    say(f"[case] {label}: propose, ctx {n_ctx}")
    ref = head.propose(st, tok, n_ctx, geo.gamma - 1, bitmask=mask, logits=True)
    torch.cuda.synchronize()
    out = _outputs(geo)
    dmask = None if mask is None else torch.from_numpy(mask).cuda()
    free0 = alloc0 = None
    for rep in range(3):
        say(f"[case] {label}: propose_noalloc #{rep}")
        head.propose_noalloc(st, tok, n_ctx, geo.gamma - 1, bitmask=dmask, out=out)
        torch.cuda.synchronize()
        for k in ("ids", "row_prob", "conf", "logits"):
            assert torch.equal(out[k], ref[k]), f"{label} {k} differs"
        if rep == 0:  # after a first call (the runtime's own first-launch work) ...
            free0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    # ... the calls allocated nothing: neither through torch nor on the device
    assert torch.cuda.memory_allocated() == alloc0
    assert torch.cuda.mem_get_info()[0] == free0
    st.free()


def test_noalloc_matches_propose_two_calls_then_smaller():
    from block_diffusion_draft_03_amd import Head
    # first call: the full DFlash geometry, 1024 ctx rows (16 block rows, 17 splits per kv head)
    geo = synth.FULL
    say("[build] full geometry")
    w = synth.make_weights(geo)
    head = Head(geo, w, kv_pool_blocks=80, max_batch=1, max_seq_len=1100)
    _compare(head, geo, 1024, tag=1, label="full ctx1024")
    head.destroy()
    del w
    # second call, smaller: hidden 256, 2 layers, 17 ctx rows
    say("[build] mid geometry")
    w = synth.make_weights(MID)
    head = Head(MID, w, kv_pool_blocks=16, max_batch=1, max_seq_len=256)
    _compare(head, MID, 17, tag=2, label="mid ctx17")
    # and a 33-row block over an empty context, with the W8A8 head and FP8 cache
    geo8 = replace(MID, gamma=33, kv_dtype="fp8", lm_head_dtype="fp8", lm_act_dtype="fp8")
    head.destroy()
    w8 = synth.make_weights(geo8)
    head = Head(geo8, w8, kv_pool_blocks=16, max_batch=1, max_seq_len=256)
    _compare(head, geo8, 0, tag=3, label="mid W8A8 gamma33 empty ctx")
    head.destroy()


def test_noalloc_refuses_more_than_the_static_scratch():
    from block_diffusion_draft_03_amd import DflashError, Head
    # an SwiGLU width of 131072 with a 64-row block: 16 MiB for the MLP activations alone
    geo = synth.Geometry(num_layers=1, hidden=64, intermediate=131072, num_q_heads=2, num_kv_heads=1, head_dim=32,
                         vocab=512, gamma=64, mask_token_id=511, num_target_layers=1, target_hidden=64,
                         ctx_window=64, rope_theta=1e6, rms_eps=1e-6)
    head = Head(geo, synth.make_weights(geo), kv_pool_blocks=4, max_batch=1, max_seq_len=64)
    st = head.state_create()
    out = _outputs(geo)
    say("[case] too much scratch")
    with pytest.raises(DflashError, match="E_INVALID"):
        head.propose_noalloc(st, 1, 0, geo.gamma - 1, out=out)
    torch.cuda.synchronize()
    assert bool((out["ids"] == -7).all()) and bool((out["conf"] == -7.0).all())  # nothing was enqueued
    # the head's own propose still runs it
    res = head.propose(st, 1, 0, geo.gamma - 1)
    torch.cuda.synchronize()
    assert int(res["ids"][0]) >= 0
    st.free()
    head.destroy()
