"""The GPU-vs-oracle acceptance rule for one propose, and a per-test tally.

Per call (``check_propose``):

* logits: per row, max_v |l_gpu - l_ref| <= tol * max_v |l_ref| (tol 2e-2 for
  a bf16 LM head, 6e-2 for an FP8 head);
* ids: equal on every row whose oracle top-2 margin (on masked logits) is
  larger than 0.05; a row the mask empties must be DFLASH_NO_TOKEN on both;
* every other live row is checked too, so no call passes on ids vacuously:
  the GPU's id must be an allowed token whose oracle logit is within twice
  the row's logit error of the oracle's maximum (what the logit bound allows
  when the top is closer than that), and when the GPU returned its logits,
  its id must be the lowest index of the maximum of its own masked logits
  (bit for bit) and its top-1 probability the softmax of those logits;
* confidence and every row's top-1 probability within 1e-2 absolute.

ids and probabilities are per entry, each entry compared against the row the
draft-row convention puts there.

``strict_ids=False`` is for the W8A8 LM head (E4M3 activation rows, a reading
of this library, not a configured workload): its activation codes are decided
on the final-normed row, which any two bf16 implementations of the eight
layers give only to ~1% (bf16 operand roundings land differently once values
differ by more than a bf16 step; measured: GPU against oracle 0.015 RMS on the
bf16 logits), so a sizeable share of the codes differ and the top-2 difference
of the logits carries ~0.045 RMS of noise. There, ids must be equal where the
stated logit tolerance itself forces it (margin above twice tol * max|l_ref|);
rows above the 0.05 margin are counted (``pinned_agree``) and the test
asserts a floor on their agreement.

``Tally`` adds up the margin-pinned rows of a test's calls, asserts a floor
(at least one pinned row per test; at the full geometry at least half of the
rows, against about three quarters expected from the logit spread), reports
the id agreement on rows below the margin, and appends a JSON line per test
to the file named by DFLASH_PARITY_LOG when that is set.
"""
import json
import os
import sys

import numpy as np

from oracle.dflash import NO_TOKEN, apply_bitmask, top2_margin

MARGIN = 0.05
CONF_TOL = 1e-2


def as_u32(t):
    a = t.detach().cpu().numpy() if hasattr(t, "detach") else np.asarray(t)
    return a.astype(np.int64).astype(np.uint32) if a.dtype != np.uint32 else a


def _np(t):
    return t.detach().cpu().numpy() if hasattr(t, "detach") else np.asarray(t)


def check_propose(gpu, ref, bitmask=None, logit_tol=2e-2, label="", strict_ids=True):
    """gpu: dict of tensors or arrays from Head.propose (one sequence); ref:
    the oracle's dict. Returns a dict of counts: rows, live, pinned (live rows
    above the 0.05 margin), pinned_agree (of those, ids equal: all of them
    when strict_ids), low (live rows at or below the margin), low_agree (of
    those, ids equal), and max_rel_err, the largest per-row logit error over
    max|l_ref| (when the GPU returned logits)."""
    ids = as_u32(gpu["ids"]).reshape(-1)
    rp = _np(gpu["row_prob"]).reshape(-1).astype(np.float64)
    conf = float(_np(gpu["conf"]).reshape(-1)[0])
    lr_rows = ref["logits"]
    R = lr_rows.shape[0]
    lg_rows = None
    scale = np.abs(lr_rows).max(axis=1)
    err = logit_tol * scale  # per-row logit error allowed
    max_rel = None
    if gpu.get("logits") is not None:
        lg_rows = _np(gpu["logits"]).reshape(lr_rows.shape).astype(np.float64)
        obs = np.abs(lg_rows - lr_rows).max(axis=1)
        max_rel = float((obs / scale).max())
        bad = obs > err
        assert not bad.any(), f"{label} logits: rel err {max_rel:.3e} > {logit_tol}"
        err = obs
    forced = 2.0 * logit_tol * scale  # a margin above this forces equal ids under the tolerance
    # entry j holds row row_of_entry[j]
    roe = ref.get("row_of_entry", np.arange(R))
    lr = lr_rows[roe]
    err = err[roe]
    lrm = lr if bitmask is None else apply_bitmask(lr, bitmask)
    empty = ref["ids"] == NO_TOKEN
    assert np.array_equal(ids[empty], ref["ids"][empty]), f"{label} emptied rows"
    with np.errstate(invalid="ignore"):
        margin = top2_margin(lr, bitmask)
    live = ~empty
    pinned = live & (margin > MARGIN)
    must = pinned if strict_ids else live & (margin > forced[roe])
    mism = np.flatnonzero(must & (ids != ref["ids"]))
    assert mism.size == 0, f"{label} ids differ on pinned rows {mism.tolist()}: gpu {ids[mism]} ref {ref['ids'][mism]}"
    # every live entry: an allowed id within twice the row's logit error of the top
    for j in np.flatnonzero(live):
        v = int(ids[j])
        assert v < lr.shape[1] and np.isfinite(lrm[j, v]), f"{label} entry {j}: id {v} not an allowed token"
        top = lrm[j].max()
        assert lrm[j, v] >= top - 2.0 * err[j] - 1e-12, \
            f"{label} entry {j}: id {v} logit {lrm[j, v]:.5f} below top {top:.5f} - 2 x {err[j]:.2e}"
    if lg_rows is not None:
        # the selection agrees bit for bit with the GPU's own logits
        lgm = lg_rows[roe] if bitmask is None else apply_bitmask(lg_rows[roe], bitmask)
        for j in np.flatnonzero(live):
            top = lgm[j].max()
            first = int(np.flatnonzero(lgm[j] == top)[0])
            assert int(ids[j]) == first, f"{label} entry {j}: id {ids[j]} is not the first argmax {first} of its own logits"
            p_own = 1.0 / np.sum(np.exp(lgm[j] - top))
            assert abs(rp[j] - p_own) <= 1e-3 * p_own + 1e-7, f"{label} entry {j}: p1 {rp[j]} vs own softmax {p_own}"
    assert np.abs(rp - ref["row_prob"]).max() <= CONF_TOL, f"{label} row_prob err {np.abs(rp - ref['row_prob']).max()}"
    # p1 = 1 / sum exp(l - max): a logit error e moves log p1 by at most 2e,
    # so the logit tolerance bounds the relative error of p1 as well
    if live.any():
        lim = 2 * logit_tol * np.abs(lr[live]).max(axis=1)
        dlog = np.abs(np.log(rp[live]) - np.log(ref["row_prob"][live]))
        assert np.all(dlog <= lim), f"{label} log p1 err {dlog.max():.3e}"
    assert abs(conf - ref["conf"]) <= CONF_TOL, f"{label} conf gpu {conf} ref {ref['conf']}"
    low = live & ~pinned
    return {"rows": int(R), "live": int(live.sum()), "pinned": int(pinned.sum()),
            "pinned_agree": int((pinned & (ids == ref["ids"])).sum()), "low": int(low.sum()),
            "low_agree": int((low & (ids == ref["ids"])).sum()), "max_rel_err": max_rel}


class Tally:
    """Counts of one test's check_propose calls."""

    def __init__(self, label):
        self.label = label
        self.calls = 0
        self.c = {"rows": 0, "live": 0, "pinned": 0, "pinned_agree": 0, "low": 0, "low_agree": 0}
        self.max_rel_err = None

    def add(self, counts):
        self.calls += 1
        for k in self.c:
            self.c[k] += counts[k]
        if counts.get("max_rel_err") is not None:
            self.max_rel_err = max(self.max_rel_err or 0.0, counts["max_rel_err"])
        return counts

    def finish(self, min_pinned=1, min_share=0.0, min_pinned_agree=1.0):
        c = self.c
        share = c["pinned"] / max(1, c["live"])
        agree = c["pinned_agree"] / c["pinned"] if c["pinned"] else 1.0
        rec = {"test": self.label, "calls": self.calls, **c, "pinned_share": round(share, 4),
               "pinned_agree_rate": round(agree, 4),
               "low_agree_rate": round(c["low_agree"] / c["low"], 4) if c["low"] else None,
               "max_rel_logit_err": None if self.max_rel_err is None else round(self.max_rel_err, 5)}
        print(f"[parity] {json.dumps(rec)}", file=sys.stderr, flush=True)
        path = os.environ.get("DFLASH_PARITY_LOG")
        if path:
            with open(path, "a") as f:
                f.write(json.dumps(rec) + "\n")
        assert c["pinned"] >= min_pinned, f"{self.label}: {c['pinned']} margin-pinned rows < {min_pinned}"
        assert share >= min_share, f"{self.label}: pinned share {share:.3f} < {min_share}"
        assert agree >= min_pinned_agree, f"{self.label}: ids equal on {agree:.3f} of the pinned rows < {min_pinned_agree}"
        return rec


def split_batch(gpu, i):
    return {k: (None if v is None else v[i]) for k, v in gpu.items()} | {"conf": gpu["conf"][i:i + 1]}
