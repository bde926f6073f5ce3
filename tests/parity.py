"""The GPU-vs-oracle acceptance rule for one propose.

* logits: per row, max_v |l_gpu - l_ref| <= tol * max_v |l_ref| (tol 2e-2 for
  a bf16 LM head, 6e-2 for an FP8 head);
* ids: equal on every row whose oracle top-2 margin (on masked logits) is
  larger than 0.05; a row the mask empties must be DFLASH_NO_TOKEN on both
  (ids and probabilities are compared entry by entry, each entry against the
  row the draft-row convention puts there);
* confidence and every row's top-1 probability within 1e-2 absolute.
"""
import numpy as np

from oracle.dflash import NO_TOKEN, top2_margin

MARGIN = 0.05
CONF_TOL = 1e-2


def as_u32(t):
    a = t.detach().cpu().numpy() if hasattr(t, "detach") else np.asarray(t)
    return a.astype(np.int64).astype(np.uint32) if a.dtype != np.uint32 else a


def check_propose(gpu, ref, bitmask=None, logit_tol=2e-2, label=""):
    """gpu: dict of torch tensors from Head.propose (one sequence); ref: the
    oracle's dict. Returns (pinned rows, agreeing unpinned rows, rows)."""
    ids = as_u32(gpu["ids"]).reshape(-1)
    rp = gpu["row_prob"].detach().cpu().numpy().reshape(-1).astype(np.float64)
    conf = float(gpu["conf"].detach().cpu().numpy().reshape(-1)[0])
    lr = ref["logits"]
    if gpu.get("logits") is not None:
        lg = gpu["logits"].detach().cpu().numpy().reshape(lr.shape).astype(np.float64)
        err = np.abs(lg - lr).max(axis=1)
        scale = np.abs(lr).max(axis=1)
        bad = err > logit_tol * scale
        assert not bad.any(), f"{label} logits: rel err {(err / scale).max():.3e} > {logit_tol}"
    # ids and row_prob are per entry; entry j holds row row_of_entry[j]
    lr = lr[ref["row_of_entry"]] if "row_of_entry" in ref else lr
    empty = ref["ids"] == NO_TOKEN
    assert np.array_equal(ids[empty], ref["ids"][empty]), f"{label} emptied rows"
    with np.errstate(invalid="ignore"):
        margin = top2_margin(lr, bitmask)
    pinned = (~empty) & (margin > MARGIN)
    mism = np.flatnonzero(pinned & (ids != ref["ids"]))
    assert mism.size == 0, f"{label} ids differ on pinned rows {mism.tolist()}: gpu {ids[mism]} ref {ref['ids'][mism]}"
    assert np.abs(rp - ref["row_prob"]).max() <= CONF_TOL, f"{label} row_prob err {np.abs(rp - ref['row_prob']).max()}"
    # p1 = 1 / sum exp(l - max): a logit error e moves log p1 by at most 2e,
    # so the logit tolerance bounds the relative error of p1 as well
    live = ~empty
    if live.any():
        lim = 2 * logit_tol * np.abs(lr[live]).max(axis=1)
        dlog = np.abs(np.log(rp[live]) - np.log(ref["row_prob"][live]))
        assert np.all(dlog <= lim), f"{label} log p1 err {dlog.max():.3e}"
    assert abs(conf - ref["conf"]) <= CONF_TOL, f"{label} conf gpu {conf} ref {ref['conf']}"
    agree_unpinned = int(((~pinned) & (ids == ref["ids"])).sum())
    return int(pinned.sum()), agree_unpinned, len(ids)


def split_batch(gpu, i):
    return {k: (None if v is None else v[i]) for k, v in gpu.items()} | {"conf": gpu["conf"][i:i + 1]}
