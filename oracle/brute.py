"""Explicit-loop float64 twin of the propose path, for tiny shapes only.

TEST INFRASTRUCTURE (see the package docstring).

Written independently of ``oracle.dflash`` and ``oracle.numerics`` so that it
pins them: every sum is a ``math.fsum`` over explicit products, RoPE is a
complex multiplication, softmax normalises through a log-sum-exp, the argmax
is a scan, and the storage formats have their own scalar code here: bf16 by
bit arithmetic on the float32 pattern, FP8 E4M3FN by exponent and quantum
(``_e4m3``), float32 arithmetic by rounding through ``struct``. It recomputes
the whole context from the hidden-stack rows on every call.

Covers every variant of the oracle: bf16 or FP8 KV cache (one scale per
layer, K|V and kv head), bf16 or FP8 LM head (per-row absmax mirror of the
bf16 head), E4M3 activation rows into the FP8 head (W8A8), FP8 drafter
weights, a given RoPE table, the shifted draft-row convention.

Same readings as ``oracle.dflash`` (RMSNorm gain multiplies directly,
rotate-half pairs (i, i + d/2), q-head -> kv-head hq // (n_q/n_kv), block
row j at position + j, ctx row i at position i, window [max(0,c-W), c),
block = [last, mask, ...], ties to the lowest id, every dense product takes
its activation operand rounded to bf16, FP8 codes decided in float32).
"""
import cmath
import math
import struct

E4M3_LARGEST = 448.0


def _f32(x):
    """Round a Python float to the nearest float32 (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


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


def _e4m3(x):
    """Nearest E4M3FN value to x (ties to the even mantissa), saturated to
    +-448. A normal value with exponent e (2^e <= |x| < 2^(e+1), e >= -6)
    has quantum 2^(e-3); below 2^-6 the subnormal quantum 2^-9 applies. The
    quotient by the quantum is rounded half to even by Python's round()."""
    a = abs(x)
    if a == 0.0:
        return 0.0
    m, e2 = math.frexp(a)          # a = m * 2^e2, 0.5 <= m < 1, so e = e2 - 1
    e = max(e2 - 1, -6)
    quantum = math.ldexp(1.0, e - 3)
    v = min(round(a / quantum) * quantum, E4M3_LARGEST)
    return -v if x < 0 else v


def _fp8_store(x, scale):
    """FP8 storage with one f32 scale: scale * e4m3(f32(f32(x) / scale))."""
    s = _f32(scale)
    return s * _e4m3(_f32(_f32(x) / s))


def _absmax_rows(rows):
    """Per-row absmax E4M3 quantisation of float32 rows, dequantised:
    s = f32(amax / 448) (1 for an all-zero row), value s * e4m3(f32(w / s))."""
    out = []
    for row in rows:
        r32 = [_f32(w) for w in row]
        amax = max(abs(w) for w in r32)
        s = _f32(amax / E4M3_LARGEST) if amax > 0 else 1.0
        out.append([s * _e4m3(_f32(w / s)) for w in r32])
    return out


def _matvec(W, x):
    return [math.fsum(wi * xi for wi, xi in zip(row, x)) for row in W]


def _bf16_vec(x):
    return [_store_bf16(v) for v in x]


def _rmsnorm(x, g, eps):
    ms = math.fsum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gi for v, gi in zip(x, g)]


def _rope_head(x, pos, freqs):
    d = len(x)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        z = complex(x[i], x[i + half]) * cmath.exp(1j * pos * freqs[i])
        out[i] = z.real
        out[i + half] = z.imag
    return out


def _silu(x):
    return x / (1.0 + math.exp(-x))


def brute_propose(geo, weights, ctx_stack_rows, last_token, position, num_drafts, bitmask=None):
    """Full propose from scratch with explicit loops.

    ``ctx_stack_rows`` are all ctx rows of the sequence (row i at position i).
    Returns (ids, row_prob, conf, logits) as Python lists; ids and row_prob
    per entry (entry j holds row j, or row j - 1 mod gamma with the shifted
    convention), logits per row.
    """
    L = geo["num_layers"]
    n_q, n_kv, d = geo["num_q_heads"], geo["num_kv_heads"], geo["head_dim"]
    V, gamma, eps = geo["vocab"], geo["gamma"], geo["rms_eps"]
    theta, W = geo["rope_theta"], geo["ctx_window"]
    kv_fp8 = geo.get("kv_dtype", "bf16") == "fp8"
    head_fp8 = geo.get("lm_head_dtype", "bf16") == "fp8"
    act_fp8 = geo.get("lm_act_dtype", "bf16") == "fp8"
    layer_fp8 = geo.get("layer_dtype", "bf16") == "fp8"
    if geo.get("inv_freq") is not None:
        freqs = [float(f) for f in geo["inv_freq"]]
    else:
        freqs = [theta ** (-(2.0 * i) / d) for i in range(d // 2)]

    def matrix(a):
        m = _to_lists(a)
        if layer_fp8:  # FP8 drafter weights: the bf16 value of each matrix, quantised per row
            m = _absmax_rows([[_store_bf16(w) for w in row] for row in m])
        return m

    fc = matrix(weights["fc"])
    gh = _to_lists(weights["hidden_norm"])
    layers = []
    for lw in weights["layers"]:
        layers.append({k: (_to_lists(v) if k in ("in_norm", "post_norm") else matrix(v)) for k, v in lw.items()})
    kv_scale = weights.get("kv_scale") if kv_fp8 else None

    def cache(x, l, kind, g):
        if kv_fp8:
            return _fp8_store(x, float(kv_scale[l][kind][g]))
        return _store_bf16(x)

    # context: every layer's K/V for every ctx row, from scratch
    S = _to_lists(ctx_stack_rows) if len(ctx_stack_rows) else []
    c = len(S)
    ctxK = [[None] * c for _ in range(L)]
    ctxV = [[None] * c for _ in range(L)]
    for i in range(c):
        feat = _bf16_vec(_rmsnorm(_matvec(fc, _bf16_vec(S[i])), gh, eps))
        for l in range(L):
            kr = _matvec(layers[l]["k"], feat)
            vr = _matvec(layers[l]["v"], feat)
            heads_k, heads_v = [], []
            for g in range(n_kv):
                kh = _rope_head(kr[g * d:(g + 1) * d], i, freqs)
                heads_k.append([cache(x, l, 0, g) for x in kh])
                heads_v.append([cache(x, l, 1, g) for x in vr[g * d:(g + 1) * d]])
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
        a = [_bf16_vec(_rmsnorm(hrow, lw["in_norm"], eps)) for hrow in hid]
        qs, ks, vs = [], [], []
        for j in range(gamma):
            qr = _matvec(lw["q"], a[j])
            kr = _matvec(lw["k"], a[j])
            vr = _matvec(lw["v"], a[j])
            qs.append([_rope_head(qr[h * d:(h + 1) * d], position + j, freqs) for h in range(n_q)])
            ks.append([_rope_head(kr[g * d:(g + 1) * d], position + j, freqs) for g in range(n_kv)])
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
            o = _matvec(lw["o"], _bf16_vec(attn[j]))
            hid[j] = [x + y for x, y in zip(hid[j], o)]
        for j in range(gamma):
            b = _bf16_vec(_rmsnorm(hid[j], lw["post_norm"], eps))
            gt = _matvec(lw["gate"], b)
            up = _matvec(lw["up"], b)
            m = _bf16_vec([_silu(x) * y for x, y in zip(gt, up)])
            dn = _matvec(lw["down"], m)
            hid[j] = [x + y for x, y in zip(hid[j], dn)]

    gn = _to_lists(weights["norm"])
    LM = _to_lists(weights["lm_head"])
    if head_fp8:  # per-row absmax mirror of the bf16 head, values including the row scale
        LM = _absmax_rows([[_store_bf16(w) for w in row] for row in LM])
    logits = []
    for hrow in hid:
        z = _bf16_vec(_rmsnorm(hrow, gn, eps))
        if act_fp8:
            z = _absmax_rows([z])[0]
        logits.append(_matvec(LM, z))

    row_ids, row_p = [], []
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
            row_ids.append(0xFFFFFFFF)
            row_p.append(0.0)
            continue
        row_ids.append(best_v)
        row_p.append(1.0 / math.fsum(math.exp(logits[j][v] - best) for v in range(V) if allowed[v]))
    shift = 1 if geo.get("shifted_rows", 0) else 0
    ids = [row_ids[(j - shift) % gamma] for j in range(gamma)]
    probs = [row_p[(j - shift) % gamma] for j in range(gamma)]
    conf = min(probs[1:1 + num_drafts])
    return ids, probs, conf, logits
