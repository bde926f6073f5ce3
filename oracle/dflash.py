"""Float64 numpy definition of the DFlash draft head's propose path.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the benchmark's CPU-baseline leg use this module.

Every step is the plain definition, in the order the pages describe the
head's data flow, computed in float64 on the stored values (bf16 bit patterns
are widened exactly; the tiny workload's fp32 weights are used as given).
Where a storage format is part of the method, it is emulated: the FP8 LM-head
mirror and the FP8 paged KV cache quantise and dequantise through the E4M3FN
codec in ``numerics``.

Geometry is a plain mapping with the keys

    num_layers hidden intermediate num_q_heads num_kv_heads head_dim vocab
    gamma mask_token_id num_target_layers target_hidden ctx_window
    rope_theta rms_eps kv_dtype lm_head_dtype

and optionally ``inv_freq`` (a RoPE table, e.g. ``yarn_inv_freq``'s, used in
place of the plain theta table), ``shifted_rows`` (draft-row convention) and
``layer_dtype`` ("fp8": FP8 drafter weights, ``fp8_weight``) and
``lm_act_dtype`` ("fp8": the FP8 LM head takes E4M3 activations, ``fp8_rows``).

Weights are a mapping with ``fc hidden_norm norm embed lm_head`` and
``layers`` (a list of mappings with ``in_norm q k v o post_norm gate up
down``), each a matrix in PyTorch Linear layout ``[out, in]`` or a gain
vector; ``kv_scale`` ``[L, 2, n_kv]`` f32 when the KV cache is FP8.

Parity status: each step is pinned by tests/test_oracle_*.py (closed forms,
library routines, the explicit-loop twin in ``brute`` with its own storage
codecs, on every variant: bf16 / FP8 KV cache, bf16 / FP8 / W8A8 LM head, FP8
drafter weights, a given RoPE table, both draft-row conventions); the YaRN
table at every pair index against the wavelength-ratio form of its
definition; ``top2_margin`` on hand-built rows and against a scan. The
composition of the steps at full geometry is the reading stated in each
docstring and is otherwise unpinned (the pages print no worked example), as is
the RoPE pairing convention itself.
"""
import math

import numpy as np

from .numerics import E4M3_MAX, bf16_round, e4m3_decode, e4m3_encode, stored_to_f64

NO_TOKEN = 0xFFFFFFFF


# ----------------------------------------------------------------------------
# elementary steps
# ----------------------------------------------------------------------------

def rms_norm(x, gain, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gain.

    The head has three kinds of RMSNorm: ``hidden_norm`` on the projected
    target context, the per-layer norms, and the final ``norm`` before the LM
    head ([Head/atlas], fields ``hidden_norm`` and ``norm``); epsilon is 1e-6
    ([Head/atlas], field ``rms_norm_eps``). Reading: the gain multiplies
    directly (not 1 + gain), the Qwen3 convention the pages cite.
    Pinned: unit RMS for gain 1 (closed form), brute-force twin.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope_inv_freq(theta, rotary_dim):
    """Plain RoPE inverse frequencies: inv_freq[i] = theta^(-2i/rotary_dim),
    i in [0, rotary_dim/2) ([Head/atlas], fields ``yarn_inv_freq``,
    ``rope_theta``, ``rotary_dim``; [Head/metrale], field ``yarn_inv_freq``:
    the YaRN correction applies only when the drafter config has
    rope_scaling, which the synthetic workloads do not)."""
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / rotary_dim)


def yarn_inv_freq(theta, rotary_dim, factor, beta_fast, beta_slow, original_max):
    """YaRN-corrected RoPE inverse frequencies, f32 [rotary_dim/2] widened to
    float64 ([Head/atlas], field ``yarn_inv_freq``: a precomputed f32 table
    of head_dim/2 entries, from the drafter's rope_scaling with factor 64,
    beta_fast 32, beta_slow 1 and original_max_position_embeddings 4096;
    [Head/metrale], field ``yarn_inv_freq``: YaRN-corrected when the config
    has rope_scaling). The pages give the parameters, not the formula; the
    reading taken is YaRN's "NTK-by-parts" interpolation (Peng et al.,
    "YaRN: Efficient Context Window Extension of Large Language Models",
    section 3.2) with its ramp laid over the pair index, the form a
    rope_scaling block with those four keys configures:

    * pair i rotates at w_i = theta^(-2i/d) (wavelength 2 pi / w_i); the
      fractional pair index whose wavelength fits r times into the original
      context L is i(r) = d ln(L / (2 pi r)) / (2 ln theta);
    * pairs up to lo = floor(i(beta_fast)) (more than beta_fast turns over L)
      keep w_i; pairs from hi = ceil(i(beta_slow)) on (fewer than beta_slow
      turns) are interpolated to w_i / factor; in between the weight of the
      unchanged frequency falls linearly in i from lo to hi (lo clamped to
      >= 0, hi to <= d - 1, hi nudged by 0.001 when equal to lo);
    * no magnitude scaling of cos / sin (the pages name none).

    Computed in float64 and rounded once to float32 (the table's dtype)."""
    d = int(rotary_dim)
    theta = float(theta)
    i = np.arange(d // 2, dtype=np.float64)
    w = np.power(theta, -2.0 * i / d)

    def pair_index(turns):
        return d * math.log(original_max / (turns * 2.0 * math.pi)) / (2.0 * math.log(theta))

    lo = max(math.floor(pair_index(beta_fast)), 0)
    hi = min(math.ceil(pair_index(beta_slow)), d - 1)
    if hi == lo:
        hi += 0.001
    ramp = np.clip((i - lo) / (hi - lo), 0.0, 1.0)
    keep = 1.0 - ramp  # weight of the unchanged frequency
    table = (w / float(factor)) * (1.0 - keep) + w * keep
    return table.astype(np.float32).astype(np.float64)


def rope(x, positions, inv_freq):
    """Rotate-half RoPE over the whole head (rotary_dim == head_dim,
    [Head/atlas] field ``rotary_dim``).

    x is ``[rows, heads, d]``; row r sits at ``positions[r]``. Dimension
    pairs are (i, i + d/2): with a = pos * inv_freq[i],
    y_i = x_i cos a - x_{i+d/2} sin a and y_{i+d/2} = x_{i+d/2} cos a +
    x_i sin a. Reading: the pairing convention is not on the pages
    (parity unpinned for the pairing itself; the rotation is pinned against
    complex multiplication).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x):
    """SiLU, x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def gemm_input(x):
    """The activation operand of one of the head's dense products, as that
    product takes it: rounded to bf16 (round to nearest, ties to even).

    Reading R10, applied to every dense product of the head (fc, the fused
    ctx K/V projection, Q/K/V, o_proj, gate/up, down, the LM head): the pages
    describe the head's products as bf16 dense GEMMs over BF16 weights (the
    fused K/V projection as a single dense GEMM over a BF16 weight,
    [Head/atlas] field ``fused_kv_weight``; the logits product over the
    target's BF16 LM head as a BF16 dense GEMM, [Head/atlas] field
    ``lm_head_nvfp4``), so both operands are
    bf16 and only the accumulation is wider. The weights are used as stored
    (bf16 for the full geometry; the tiny workload's fp32 weights as given);
    the products themselves are exact float64 sums. The residual stream, the
    norms, RoPE and attention stay in float64 (they are not dense GEMMs)."""
    return bf16_round(x)


def gqa_attention(q, k, v, num_kv_heads):
    """Grouped-query attention without a mask.

    q is ``[R, n_q, d]``; k and v are ``[S, n_kv, d]`` (ctx window rows then
    block rows). Query head hq reads kv head hq // (n_q / n_kv). Scores are
    scaled by 1/sqrt(d); softmax over all S keys. Reading: the block rows see
    each other bidirectionally and every ctx row in the window, so no mask
    applies. Pinned: identical keys give the mean of V; matches
    torch.nn.functional.scaled_dot_product_attention in float64.
    """
    R, n_q, d = q.shape
    rep = n_q // num_kv_heads
    out = np.empty((R, n_q, d), dtype=np.float64)
    scale = 1.0 / np.sqrt(d)
    for hq in range(n_q):
        g = hq // rep
        s = (q[:, hq, :] @ k[:, g, :].T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, hq, :] = p @ v[:, g, :]
    return out


def fp8_roundtrip(x, scale):
    """Emulate FP8 storage with one f32 scale: scale * dec(enc(x / scale)).
    The code is decided in float32 (the value and the scale are float32 and
    the quotient is an IEEE float32 division), the precision the cache's
    producer holds them in."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(scale, dtype=np.float32)
    q = (x32 / s32).astype(np.float64)
    return s32.astype(np.float64) * e4m3_decode(e4m3_encode(q))


def fp8_head_mirror(lm_head_bf16_bits):
    """FP8 copy of the bf16 LM head: E4M3 codes ``[V, h]`` plus one f32 scale
    per vocab row ([Head/atlas], field ``lm_head_shared_fp8``; [Head/metrale]:
    an FP8 copy of ``lm_head_shared`` when no native FP8 head is given).

    Reading (the recipe is not on the pages): per-row absmax scaling,
    s_v = amax_v / 448 and q_vk = enc(w_vk / s_v). Both the scale and the
    quotient are computed in float32, the precision of the stored scale, so
    the integer codes are a deterministic function of the bf16 head. An
    all-zero row gets scale 1. The mirror is of the bf16 head ([Head/atlas]
    field ``lm_head_shared``: the target's bf16 LM head), so a head given in
    fp32 (the tiny workload) is taken at its bf16 value first. Rows are
    independent, so they are processed in blocks of 2048 on a thread pool
    (memory and time only).
    """
    src = np.asarray(lm_head_bf16_bits)
    if src.dtype != np.uint16:
        src = (bf16_round(stored_to_f64(src)).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    V, h = src.shape
    codes = np.empty((V, h), dtype=np.uint8)
    scale = np.empty(V, dtype=np.float32)

    def rows(r0):
        r1 = min(V, r0 + 2048)
        w = stored_to_f64(src[r0:r1]).astype(np.float32)
        amax = np.max(np.abs(w), axis=1)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = w / s[:, None]  # float32 IEEE division
        codes[r0:r1] = e4m3_encode(q.astype(np.float64))
        scale[r0:r1] = s

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(16) as ex:
        list(ex.map(rows, range(0, V, 2048)))
    return codes, scale


# ----------------------------------------------------------------------------
# per-sequence state and the head
# ----------------------------------------------------------------------------

class OracleState:
    """One sequence's drafter context.

    Holds, for every ctx row appended and not trimmed, the row's K and V for
    every layer (after RoPE and, for an FP8 cache, after the FP8 round trip),
    plus the raw hidden-stack row so the whole context can be rebuilt from
    scratch. Ctx row i sits at RoPE position i (reading). ``pending_base`` is
    the ctx length at the last ``after_verify``; rows appended since then are
    the ones ``after_verify`` may trim ([DraftProposer], ``after_verify``).
    """

    def __init__(self, num_layers):
        self.k = [[] for _ in range(num_layers)]
        self.v = [[] for _ in range(num_layers)]
        self.stack_rows = []
        self.pending_base = 0

    @property
    def ctx_len(self):
        return len(self.stack_rows)


def fp8_weight(stored):
    """FP8 drafter weight ([Head/metrale], field ``lm_head_shared_fp8``: the
    LM head used with FP8 drafter weights, so the drafter's own matrices are
    FP8 then as well; the pages give no recipe for them). Reading: the same
    per-row absmax E4M3 quantisation as the LM-head mirror (fp8_head_mirror),
    applied to the bf16 value of each matrix (fp32 weights are rounded to
    bf16 first, as the library stores them) and dequantised: w~ = s_r dec(q).
    Weight-only: activations stay as they are."""
    x = np.asarray(stored)
    if x.dtype != np.uint16:
        # bf16 bit patterns of the rounded values
        b = bf16_round(stored_to_f64(x)).astype(np.float32).view(np.uint32) >> np.uint32(16)
        x = b.astype(np.uint16)
    codes, scale = fp8_head_mirror(x)
    return e4m3_decode(np.arange(256, dtype=np.uint8))[codes] * scale.astype(np.float64)[:, None]


def fp8_rows(x):
    """FP8 activations of the LM head (W8A8 head; the pages give an FP8 LM
    head, [Head/atlas] field ``lm_head_shared_fp8``, but no activation
    format). Reading: each activation row is quantised with the LM-head
    mirror's recipe (fp8_head_mirror) applied to its float32 value,
    a_m = amax_m / 448 (1 for an all-zero row) and c_mk = enc(z_mk / a_m) with
    float32 division, and used dequantised: z~_mk = a_m dec(c_mk)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = x32 / s[..., None]  # float32 IEEE division
    return s.astype(np.float64)[..., None] * e4m3_decode(e4m3_encode(q.astype(np.float64)))


class OracleHead:
    """The draft head over float64 numpy arrays.

    ``geo`` and ``weights`` as described in the module docstring. The shared
    embedding and LM head are the target's tensors ([Head/atlas], struct
    description and fields ``embed_tokens_shared``, ``lm_head_shared``).
    """

    def __init__(self, geo, weights):
        self.geo = dict(geo)
        g = self.geo
        self.L = int(g["num_layers"])
        self.h = int(g["hidden"])
        self.n_q = int(g["num_q_heads"])
        self.n_kv = int(g["num_kv_heads"])
        self.d = int(g["head_dim"])
        self.V = int(g["vocab"])
        self.gamma = int(g["gamma"])
        self.eps = float(g["rms_eps"])
        self.W = int(g["ctx_window"])
        self.mask_id = int(g["mask_token_id"])
        self.kv_fp8 = g.get("kv_dtype", "bf16") == "fp8"
        self.head_fp8 = g.get("lm_head_dtype", "bf16") == "fp8"
        # W8A8 head: the final-normed rows enter the FP8 head as E4M3 (fp8_rows)
        self.head_a8 = g.get("lm_act_dtype", "bf16") == "fp8"
        if self.head_a8 and not self.head_fp8:
            raise ValueError("lm_act_dtype fp8 needs lm_head_dtype fp8")
        fc_in = int(g["num_target_layers"]) * int(g["target_hidden"])
        # a given table (e.g. yarn_inv_freq) replaces the plain one
        self.inv_freq = (np.asarray(g["inv_freq"], dtype=np.float64) if g.get("inv_freq") is not None
                         else rope_inv_freq(g["rope_theta"], self.d))

        w = weights
        # FP8 drafter weights: every drafter matrix quantised (norm gains, the
        # target's embedding and the LM head are not drafter matrices)
        self.layers_fp8 = g.get("layer_dtype", "bf16") == "fp8"
        mat = fp8_weight if self.layers_fp8 else stored_to_f64
        self.fc = mat(w["fc"])
        if self.fc.shape != (self.h, fc_in):
            # the fc input width is num_target_layers * target_hidden
            # ([Head/atlas], fields target_hidden_size and fc; a mismatch is a
            # hard error per validate_against_target)
            raise ValueError(f"fc shape {self.fc.shape} != {(self.h, fc_in)}")
        self.hidden_norm = stored_to_f64(w["hidden_norm"])
        self.final_norm = stored_to_f64(w["norm"])
        self.embed_stored = w["embed"]  # gathered row by row; widened lazily
        self.layers = []
        for lw in w["layers"]:
            self.layers.append({key: (stored_to_f64 if key in ("in_norm", "post_norm") else mat)(lw[key]) for key in
                                ("in_norm", "q", "k", "v", "o", "post_norm", "gate", "up", "down")})
        if self.head_fp8:
            if "lm_head_fp8" in w and w["lm_head_fp8"] is not None:
                codes, scale = np.asarray(w["lm_head_fp8"], np.uint8), np.asarray(w["lm_head_scale"], np.float32)
            else:
                codes, scale = fp8_head_mirror(w["lm_head"])
            self.lm_codes, self.lm_scale = codes, scale
            # dequantised without the row scale (table of the 256 decoded codes)
            self.lm = e4m3_decode(np.arange(256, dtype=np.uint8))[codes]
        else:
            self.lm = stored_to_f64(w["lm_head"])
        if self.kv_fp8:
            self.kv_scale = np.asarray(w["kv_scale"], dtype=np.float32).astype(np.float64)
            assert self.kv_scale.shape == (self.L, 2, self.n_kv)

    # --- ctx (target-hidden) path -------------------------------------------

    def ctx_features(self, stack_rows):
        """fc projection plus hidden_norm of captured target hidden stacks.

        ``stack_rows`` is ``[rows, T*Ht]`` (shallow-to-deep concatenation of
        the hiddens at the target layers, [DraftProposer] ``propose``
        argument ``target_hidden_stack``). u = S fc^T, c = RMSNorm(u;
        hidden_norm) ([Head/atlas], fields ``fc`` and ``hidden_norm``). The
        stack is stored as bf16, so it already is the fc product's bf16
        operand (``gemm_input``).
        """
        s = stored_to_f64(stack_rows)
        return rms_norm(gemm_input(s) @ self.fc.T, self.hidden_norm, self.eps)

    def ctx_kv(self, c_hat, positions):
        """Every layer's ctx K and V from one normalised ctx feature.

        Reading: the same c feeds each layer's k_proj / v_proj with no
        per-layer norm, because the fused weight is a plain row-stitch of the
        per-layer k_proj and v_proj applied to one input ([Head/atlas] and
        [Head/metrale], field ``fused_kv_weight``). K is rotated at the ctx
        positions and cached after rotation ([Head/atlas], field
        ``kv_cache``: the cache is written by reshape_and_cache). The cached
        values pass through the cache's storage format: bf16 ([Head/metrale],
        field ``kv_cache``) or FP8 E4M3 with one f32 scale per (layer, K|V,
        kv head) ([Head/atlas], field ``kv_cache``).

        The fused projection is a bf16 dense GEMM (``gemm_input``): c enters
        rounded to bf16 and the products are exact float64 sums of those
        bf16 values.
        Returns lists over layers of ``[rows, n_kv, d]`` K and V.
        """
        ks, vs = [], []
        n = c_hat.shape[0]
        c_in = gemm_input(c_hat)
        for l, lw in enumerate(self.layers):
            k = (c_in @ lw["k"].T).reshape(n, self.n_kv, self.d)
            v = (c_in @ lw["v"].T).reshape(n, self.n_kv, self.d)
            k = rope(k, positions, self.inv_freq)
            if self.kv_fp8:
                k = fp8_roundtrip(k, self.kv_scale[l, 0][None, :, None])
                v = fp8_roundtrip(v, self.kv_scale[l, 1][None, :, None])
            else:
                k = bf16_round(k)
                v = bf16_round(v)
            ks.append(k)
            vs.append(v)
        return ks, vs

    def new_state(self):
        return OracleState(self.L)

    def precompute(self, state, stack_rows):
        """Append ctx rows: K/V for every layer at positions ctx_len.. ."""
        stack_rows = np.asarray(stack_rows)
        n = stack_rows.shape[0]
        if n == 0:
            return
        pos = np.arange(state.ctx_len, state.ctx_len + n)
        ks, vs = self.ctx_kv(self.ctx_features(stack_rows), pos)
        for l in range(self.L):
            state.k[l].extend(list(ks[l]))
            state.v[l].extend(list(vs[l]))
        state.stack_rows.extend(list(stack_rows))

    def after_verify(self, state, num_accepted):
        """Keep the first ``num_accepted`` rows appended since the last
        ``after_verify`` and drop the rest ([DraftProposer], ``after_verify``:
        trim the state to match the accepted count). Reading: 0 <= a <=
        pending rows; anything else is an error."""
        pending = state.ctx_len - state.pending_base
        if not 0 <= num_accepted <= pending:
            raise ValueError(f"num_accepted {num_accepted} outside [0, {pending}]")
        keep = state.pending_base + num_accepted
        for l in range(self.L):
            del state.k[l][keep:]
            del state.v[l][keep:]
        del state.stack_rows[keep:]
        state.pending_base = keep

    def rebuilt(self, state):
        """A fresh state holding exactly ``state``'s rows, recomputed."""
        fresh = self.new_state()
        if state.ctx_len:
            self.precompute(fresh, np.stack(state.stack_rows))
        fresh.pending_base = fresh.ctx_len
        return fresh

    # --- block forward -------------------------------------------------------

    def window(self, state):
        """Ctx rows the block attends to: [max(0, c - W), c); W = 0 keeps
        none ([Head/atlas] and [Head/metrale], field ``ctx_window``)."""
        c = state.ctx_len
        lo = max(0, c - self.W) if self.W > 0 else c
        return lo, c

    def block_tokens(self, last_token):
        """Block of gamma ids: the last verified token, then mask tokens.
        Reading from ``mask_token_id`` ([Head/atlas] struct) and the draft
        count gamma - 1 ([Head/metrale], ``block_gamma``)."""
        return np.array([last_token] + [self.mask_id] * (self.gamma - 1), dtype=np.int64)

    def embed(self, ids):
        """Rows of the target's shared embedding table."""
        return stored_to_f64(np.asarray(self.embed_stored)[ids])

    def layer(self, l, hid, positions, ctx_k, ctx_v):
        """One drafter layer, pre-norm residual (reading of the layer form):
        a = RMSNorm(h), q/k/v projections, RoPE on q and k, GQA attention over
        [ctx window ; block], h += o_proj(o); b = RMSNorm(h),
        h += down(silu(gate b) * up b). The operands a, o, b and the SwiGLU
        product enter their dense products as bf16 (``gemm_input``)."""
        lw = self.layers[l]
        R = hid.shape[0]
        a = gemm_input(rms_norm(hid, lw["in_norm"], self.eps))
        q = (a @ lw["q"].T).reshape(R, self.n_q, self.d)
        k = (a @ lw["k"].T).reshape(R, self.n_kv, self.d)
        v = (a @ lw["v"].T).reshape(R, self.n_kv, self.d)
        q = rope(q, positions, self.inv_freq)
        k = rope(k, positions, self.inv_freq)
        kk = np.concatenate([ctx_k, k], axis=0)
        vv = np.concatenate([ctx_v, v], axis=0)
        o = gqa_attention(q, kk, vv, self.n_kv)
        hid = hid + gemm_input(o.reshape(R, self.n_q * self.d)) @ lw["o"].T
        b = gemm_input(rms_norm(hid, lw["post_norm"], self.eps))
        m = gemm_input(silu(b @ lw["gate"].T) * (b @ lw["up"].T))
        return hid + m @ lw["down"].T

    def logits(self, hid):
        """Final RMSNorm then the shared LM head ([Head/atlas], fields
        ``norm``, ``lm_head_shared``). FP8 head: l_v = s_v * sum_k dec(q_vk)
        z_k ([Head/atlas], field ``lm_head_shared_fp8``); W8A8 head: z is
        replaced by its per-row E4M3 value fp8_rows(z). z enters the product
        as bf16 (``gemm_input``), so the W8A8 head quantises that bf16 row."""
        z = gemm_input(rms_norm(hid, self.final_norm, self.eps))
        if self.head_a8:
            z = fp8_rows(z)
        l = z @ self.lm.T
        if self.head_fp8:
            l = l * self.lm_scale.astype(np.float64)[None, :]
        return l

    def forward_block(self, state, last_token, position):
        """Block forward for one sequence; returns logits ``[gamma, V]``.
        Block row j sits at RoPE position ``position + j`` ([DraftProposer],
        ``propose`` argument ``position``)."""
        ids = self.block_tokens(last_token)
        hid = self.embed(ids)
        pos = position + np.arange(self.gamma)
        lo, hi = self.window(state)
        for l in range(self.L):
            if hi > lo:
                ck = np.stack(state.k[l][lo:hi])
                cv = np.stack(state.v[l][lo:hi])
            else:
                ck = np.zeros((0, self.n_kv, self.d))
                cv = np.zeros((0, self.n_kv, self.d))
            hid = self.layer(l, hid, pos, ck, cv)
        return self.logits(hid)

    def propose(self, state, last_token, position, num_drafts, bitmask=None):
        """One propose: ids for every block row, their top-1 probabilities and
        the chain confidence. Returns a dict with ``ids`` (uint32 [gamma]),
        ``row_prob`` [gamma], ``conf`` and ``logits`` [gamma, V]."""
        if not 1 <= num_drafts <= self.gamma - 1:
            raise ValueError("num_drafts must be in [1, gamma - 1]")
        lg = self.forward_block(state, last_token, position)
        return select(lg, bitmask, num_drafts, shifted=bool(self.geo.get("shifted_rows", 0)))

    def propose_batch(self, states, last_tokens, positions, num_drafts, bitmasks=None):
        """Batched propose: by definition the per-sequence result for each
        sequence ([Head/atlas], ``propose_batch``: one forward over n * gamma
        rows instead of n forwards, never a different answer)."""
        out = []
        for i, st in enumerate(states):
            bm = None if bitmasks is None else bitmasks[i]
            out.append(self.propose(st, last_tokens[i], positions[i], num_drafts, bm))
        return out


def apply_bitmask(logits, bitmask):
    """Grammar bitmask: ceil(V/32) int32 words, bit v & 31 of word v >> 5 set
    means token v is allowed ([DraftProposer], ``propose`` argument
    ``grammar_bitmask``). Disallowed logits become -inf."""
    V = logits.shape[-1]
    words = np.asarray(bitmask).astype(np.int64) & 0xFFFFFFFF
    v = np.arange(V)
    allowed = ((words[v >> 5] >> (v & 31)) & 1) == 1
    return np.where(allowed[None, :], logits, -np.inf)


def select(logits, bitmask, num_drafts, shifted=False):
    """Per-row argmax (ties to the lowest id), top-1 softmax probability
    p1 = 1 / sum_v exp(l_v - max l), and chain confidence = min p1 over the
    draft entries 1..num_drafts ([Head/atlas], ``last_confidence``). A row
    with every token masked gets id 0xFFFFFFFF and p1 = 0 (reading).

    Entry j of ``ids`` / ``row_prob`` is the draft for position + j. With the
    z-lab convention that is row j; with the shifted-row convention
    ([Head/atlas] and [Head/metrale], field ``shifted_rows``: row j's output is
    the token at position j + 1, and the draft vector is rotated right by one)
    entry j holds row j - 1 and entry 0 the last row. ``row_of_entry`` says
    which row each entry holds."""
    lg = logits if bitmask is None else apply_bitmask(logits, bitmask)
    R = lg.shape[0]
    ids = np.empty(R, dtype=np.uint32)
    p1 = np.empty(R, dtype=np.float64)
    for j in range(R):
        row = lg[j]
        mx = row.max()
        if mx == -np.inf:
            ids[j] = NO_TOKEN
            p1[j] = 0.0
            continue
        ids[j] = np.flatnonzero(row == mx)[0]
        p1[j] = 1.0 / np.sum(np.exp(row - mx))
    row_of_entry = np.arange(R)
    if shifted:
        row_of_entry = np.roll(row_of_entry, 1)
        ids, p1 = ids[row_of_entry], p1[row_of_entry]
    conf = float(p1[1:1 + num_drafts].min())
    return {"ids": ids, "row_prob": p1, "conf": conf, "logits": logits, "row_of_entry": row_of_entry}


def top2_margin(logits, bitmask=None):
    """Per-row gap between the largest and second-largest (masked) logit: 0
    for a tie at the top, +inf when one token is allowed, nan when none is.
    The GPU acceptance rule compares ids on rows whose margin exceeds 0.05
    (the tolerance stated for this path)."""
    lg = logits if bitmask is None else apply_bitmask(logits, bitmask)
    part = np.partition(lg, -2, axis=1)
    return part[:, -1] - part[:, -2]
