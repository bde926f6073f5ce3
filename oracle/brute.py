"""Explicit-loop float64 twin of the propose path, for tiny shapes only.

TEST INFRASTRUCTURE (see the package docstring).

Written independently of ``oracle.dflash`` so that it pins it: every sum is a
``math.fsum`` over explicit products, RoPE is a complex multiplication,
softmax normalises through a log-sum-exp, the bf16 / FP8 storage formats are
handled by their own bit-level code, and the argmax is a scan. It recomputes
the whole context from the hidden-stack rows on every call. Only the bf16
KV-cache format is supported here (the FP8 paths are pinned by codec tests).

Same readings as ``oracle.dflash`` (RMSNorm gain multiplies directly,
rotate-half pairs (i, i + d/2), q-head -> kv-head hq // (n_q/n_kv), block
row j at position + j, ctx row i at position i, window [max(0,c-W), c),
block = [last, mask, ...], ties to the lowest id).
"""
import cmath
import math
import struct


def _bf16_bits_to_float(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _to_lists(a):
    """Stored array -> nested Python floats (bf16 bits widened bit-wise)."""
    import numpy as np
    a = np.asarray(a)
    if a.dtype == np.uint16:
        flat = [_bf16_bits_to_float(b) for b in a.reshape(-1).tolist()]
    else:
        flat = [float(x) for x in a.reshape(-1).tolist()]
    if a.ndim == 1:
        return flat
    cols = a.shape[-1]
    return [flat[i:i + cols] for i in range(0, len(flat), cols)]


def _store_bf16(x):
    """Round a float through float32 then to the nearest bf16 (ties even)."""
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return _bf16_bits_to_float(u)


def _matvec(W, x):
    return [math.fsum(wi * xi for wi, xi in zip(row, x)) for row in W]


def _rmsnorm(x, g, eps):
    ms = math.fsum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gi for v, gi in zip(x, g)]


def _rope_head(x, pos, theta):
    d = len(x)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        f = theta ** (-(2.0 * i) / d)
        z = complex(x[i], x[i + half]) * cmath.exp(1j * pos * f)
        out[i] = z.real
        out[i + half] = z.imag
    return out


def _silu(x):
    return x / (1.0 + math.exp(-x))


def brute_propose(geo, weights, ctx_stack_rows, last_token, position, num_drafts, bitmask=None):
    """Full propose from scratch with explicit loops.

    ``ctx_stack_rows`` are all ctx rows of the sequence (row i at position i).
    Returns (ids, row_prob, conf, logits) as Python lists.
    """
    L = geo["num_layers"]
    n_q, n_kv, d = geo["num_q_heads"], geo["num_kv_heads"], geo["head_dim"]
    V, gamma, eps = geo["vocab"], geo["gamma"], geo["rms_eps"]
    theta, W = geo["rope_theta"], geo["ctx_window"]
    fc = _to_lists(weights["fc"])
    gh = _to_lists(weights["hidden_norm"])
    layers = [{k: _to_lists(v) for k, v in lw.items()} for lw in weights["layers"]]

    # context: every layer's K/V for every ctx row, from scratch
    S = _to_lists(ctx_stack_rows) if len(ctx_stack_rows) else []
    c = len(S)
    ctxK = [[None] * c for _ in range(L)]
    ctxV = [[None] * c for _ in range(L)]
    for i in range(c):
        # the fused ctx K/V projection is a bf16 GEMM: its input enters as bf16
        feat = [_store_bf16(x) for x in _rmsnorm(_matvec(fc, S[i]), gh, eps)]
        for l in range(L):
            kr = _matvec(layers[l]["k"], feat)
            vr = _matvec(layers[l]["v"], feat)
            heads_k, heads_v = [], []
            for g in range(n_kv):
                kh = _rope_head(kr[g * d:(g + 1) * d], i, theta)
                heads_k.append([_store_bf16(x) for x in kh])
                heads_v.append([_store_bf16(x) for x in vr[g * d:(g + 1) * d]])
            ctxK[l][i] = heads_k
            ctxV[l][i] = heads_v
    lo = max(0, c - W) if W > 0 else c

    # block
    E = weights["embed"]
    ids_in = [last_token] + [geo["mask_token_id"]] * (gamma - 1)
    hid = [_to_lists(E[t]) for t in ids_in]
    rep = n_q // n_kv
    for l in range(L):
        lw = layers[l]
        a = [_rmsnorm(hrow, lw["in_norm"], eps) for hrow in hid]
        qs, ks, vs = [], [], []
        for j in range(gamma):
            qr = _matvec(lw["q"], a[j])
            kr = _matvec(lw["k"], a[j])
            vr = _matvec(lw["v"], a[j])
            qs.append([_rope_head(qr[h * d:(h + 1) * d], position + j, theta) for h in range(n_q)])
            ks.append([_rope_head(kr[g * d:(g + 1) * d], position + j, theta) for g in range(n_kv)])
            vs.append([vr[g * d:(g + 1) * d] for g in range(n_kv)])
        attn = []
        for j in range(gamma):
            row = []
            for hq in range(n_q):
                g = hq // rep
                keys = [ctxK[l][i][g] for i in range(lo, c)] + [ks[t][g] for t in range(gamma)]
                vals = [ctxV[l][i][g] for i in range(lo, c)] + [vs[t][g] for t in range(gamma)]
                sc = [math.fsum(qa * kb for qa, kb in zip(qs[j][hq], key)) / math.sqrt(d) for key in keys]
                m = max(sc)
                lse = m + math.log(math.fsum(math.exp(s - m) for s in sc))
                p = [math.exp(s - lse) for s in sc]
                row.extend(math.fsum(p[t] * vals[t][e] for t in range(len(vals))) for e in range(d))
            attn.append(row)
        for j in range(gamma):
            o = _matvec(lw["o"], attn[j])
            hid[j] = [x + y for x, y in zip(hid[j], o)]
        for j in range(gamma):
            b = _rmsnorm(hid[j], lw["post_norm"], eps)
            gt = _matvec(lw["gate"], b)
            up = _matvec(lw["up"], b)
            m = [_silu(x) * y for x, y in zip(gt, up)]
            dn = _matvec(lw["down"], m)
            hid[j] = [x + y for x, y in zip(hid[j], dn)]

    gn = _to_lists(weights["norm"])
    LM = _to_lists(weights["lm_head"])
    logits = [_matvec(LM, _rmsnorm(hrow, gn, eps)) for hrow in hid]

    ids, probs = [], []
    for j in range(gamma):
        best, best_v = None, None
        allowed = []
        for v in range(V):
            ok = True
            if bitmask is not None:
                ok = ((int(bitmask[v // 32]) & 0xFFFFFFFF) >> (v % 32)) & 1 == 1
            allowed.append(ok)
            if ok and (best is None or logits[j][v] > best):
                best, best_v = logits[j][v], v
        if best is None:
            ids.append(0xFFFFFFFF)
            probs.append(0.0)
            continue
        ids.append(best_v)
        probs.append(1.0 / math.fsum(math.exp(logits[j][v] - best) for v in range(V) if allowed[v]))
    conf = min(probs[1:1 + num_drafts])
    return ids, probs, conf, logits
