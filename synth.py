"""Seeded synthetic inputs for the DFlash draft-head propose path.

Shared by the tests, the smoke check and the benchmark; used by both the HIP
library's callers and the CPU oracle. It holds none of the method's
arithmetic: it only draws numbers and rounds them once to their stored dtype.

Recipe (every draw is numpy ``default_rng`` float32, one child stream per
tensor, so a tensor does not depend on which others were drawn):

* matrices (fc, q/k/v/o, gate/up/down, embedding, LM head) ~ N(0, 0.02);
* norm gains ~ 1 + N(0, 0.02) (a small perturbation of 1, so a dropped or
  misindexed gain is visible without collapsing the activations);
* hidden-stack rows ~ N(0, 1), bf16;
* tokens uniform in [0, vocab);
* grammar bitmasks: exactly ``frac`` of the vocab allowed, chosen by a seeded
  permutation, packed LSB-first into int32 words;
* FP8 KV scales: five standard deviations of a ctx K/V element
  (0.02 * sqrt(hidden)) over 448, times 1 + U[0, 0.1);
* ctx lengths and accepted counts uniform integers in the stated ranges;
* physical block tables: a seeded permutation of pool block ids.

Stored dtypes: bf16 as uint16 bit patterns (round to nearest, ties to even,
from the float32 draw), fp32 as float32.

Seeds: 0 weights, 1 hidden stacks, 2 tokens, 3 block tables, 4 accepted
counts, 5 bitmasks, 6 ctx lengths, 7 KV scales.
"""
from dataclasses import asdict, dataclass, replace

import numpy as np

SEED_WEIGHTS, SEED_STACK, SEED_TOKENS, SEED_BLOCKS, SEED_ACCEPT, SEED_MASK, SEED_CTX, SEED_KVSCALE = range(8)


@dataclass(frozen=True)
class Geometry:
    num_layers: int
    hidden: int
    intermediate: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    vocab: int
    gamma: int
    mask_token_id: int
    num_target_layers: int
    target_hidden: int
    ctx_window: int
    rope_theta: float
    rms_eps: float
    kv_block: int = 16
    weight_dtype: str = "bf16"    # "f32" | "bf16"
    lm_head_dtype: str = "bf16"   # "bf16" | "fp8"
    kv_dtype: str = "bf16"        # "bf16" | "fp8"
    shifted_rows: int = 0         # draft-row convention: 0 z-lab, 1 shifted
    layer_dtype: str = "bf16"     # drafter matrices streamed as "bf16" or "fp8" (E4M3 + row scales)
    lm_act_dtype: str = "bf16"    # rows entering the FP8 LM head: "bf16", or "fp8" (E4M3 + row scales)

    def as_dict(self):
        return asdict(self)


# Tiny oracle-check geometry: one drafter layer, hidden 64, 4 q / 2 kv heads of
# 16, intermediate 128, vocab 512, block 4, 3 target layers of 64, fp32
# weights, mask id 511, theta 1e6.
TINY = Geometry(num_layers=1, hidden=64, intermediate=128, num_q_heads=4, num_kv_heads=2,
                head_dim=16, vocab=512, gamma=4, mask_token_id=511, num_target_layers=3,
                target_hidden=64, ctx_window=4096, rope_theta=1e6, rms_eps=1e-6,
                weight_dtype="f32")

# Full DFlash drafter geometry: 8 layers, hidden 2048, 32 q / 4 kv heads of
# 128, intermediate 6144, vocab 248320, block 16, 5 target layers of 2048,
# bf16, theta 1e7, ctx window 4096, mask id vocab - 1.
FULL = Geometry(num_layers=8, hidden=2048, intermediate=6144, num_q_heads=32, num_kv_heads=4,
                head_dim=128, vocab=248320, gamma=16, mask_token_id=248319, num_target_layers=5,
                target_hidden=2048, ctx_window=4096, rope_theta=1e7, rms_eps=1e-6)

FULL_FP8 = replace(FULL, lm_head_dtype="fp8", kv_dtype="fp8")
# FP8 drafter weights: every drafter matrix and the LM head as E4M3 + row scales, bf16 KV
FULL_FP8W = replace(FULL, lm_head_dtype="fp8", layer_dtype="fp8")
# W8A8 LM head: as FULL_FP8, and the final-normed rows enter the head as E4M3 + row scales
FULL_FP8A8 = replace(FULL_FP8, lm_act_dtype="fp8")


@dataclass(frozen=True)
class Workload:
    """A named workload: geometry plus how its sequences are filled."""
    name: str
    geo: Geometry
    n_seqs: int
    ctx_lo: int          # ctx length range, inclusive
    ctx_hi: int
    new_rows: int        # ctx rows appended per sequence per step
    trim: bool = False   # after_verify with num_accepted ~ U[0, new_rows]
    mask_frac: float = 0.0
    permute_blocks: bool = False


WORKLOADS = {
    "tiny": Workload("tiny", TINY, 1, 32, 32, 8),
    "single_ctx1024": Workload("single_ctx1024", FULL, 1, 1024, 1024, 8),
    "single_ctx4096_trim": Workload("single_ctx4096_trim", FULL, 1, 4096, 4096, 16, trim=True,
                                    permute_blocks=True),
    "single_ctx1024_fp8w": Workload("single_ctx1024_fp8w", FULL_FP8W, 1, 1024, 1024, 8),
    "batch32_ctx512_4096": Workload("batch32_ctx512_4096", FULL, 32, 512, 4096, 8),
    "batch64_fp8_ctx256_4096": Workload("batch64_fp8_ctx256_4096", FULL_FP8, 64, 256, 4096, 8,
                                        mask_frac=0.5),
    "batch64_fp8a8_ctx256_4096": Workload("batch64_fp8a8_ctx256_4096", FULL_FP8A8, 64, 256, 4096, 8,
                                          mask_frac=0.5),
}


def _rng(seed, *tags):
    return np.random.default_rng([int(seed), *[int(t) for t in tags]])


def to_bf16_bits(x32):
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties even."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    if b.size < (1 << 22):
        return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    flat = b.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)

    def conv(i):
        s = slice(i, min(flat.size, i + (1 << 22)))
        x = flat[s]
        out[s] = (x + np.uint32(0x7FFF) + ((x >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(16) as ex:
        list(ex.map(conv, range(0, flat.size, 1 << 22)))
    return out.reshape(b.shape)


def _store(x32, dtype):
    return np.ascontiguousarray(x32, dtype=np.float32) if dtype == "f32" else to_bf16_bits(x32)


ROW_BLOCK = 4096  # rows drawn from one child stream (fixed, so values do not depend on threading)


def _normal(seed, tag, shape, std):
    """N(0, std) float32 of the given shape. Matrices are drawn in blocks of
    ROW_BLOCK rows, block b from child stream (seed, tag, b), on a thread
    pool; a vector is one block."""
    if len(shape) == 1:
        return _rng(seed, tag, 0).standard_normal(shape, dtype=np.float32) * np.float32(std)
    rows, cols = shape
    out = np.empty(shape, dtype=np.float32)

    def fill(b):
        r0 = b * ROW_BLOCK
        r1 = min(rows, r0 + ROW_BLOCK)
        blk = out[r0:r1]
        _rng(seed, tag, b).standard_normal((r1 - r0, cols), dtype=np.float32, out=blk)
        blk *= np.float32(std)

    nb = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    if nb == 1:
        fill(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(16, nb)) as ex:
            list(ex.map(fill, range(nb)))
    return out


def make_weights(geo: Geometry, seed: int = SEED_WEIGHTS, std: float = 0.02):
    """Drafter weights plus the target's shared embedding and LM head."""
    h, I, d = geo.hidden, geo.intermediate, geo.head_dim
    q_dim, kv_dim = geo.num_q_heads * d, geo.num_kv_heads * d
    fc_in = geo.num_target_layers * geo.target_hidden
    wd = geo.weight_dtype
    tag = iter(range(1000))

    def mat(rows, cols):
        return _store(_normal(seed, next(tag), (rows, cols), std), wd)

    def gain(n):
        return _store(1.0 + _normal(seed, next(tag), (n,), std), wd)

    w = {"fc": mat(h, fc_in), "hidden_norm": gain(h), "norm": gain(h)}
    w["embed"] = mat(geo.vocab, h)
    w["lm_head"] = mat(geo.vocab, h)
    layers = []
    for _ in range(geo.num_layers):
        layers.append({
            "in_norm": gain(h), "q": mat(q_dim, h), "k": mat(kv_dim, h), "v": mat(kv_dim, h),
            "o": mat(h, q_dim), "post_norm": gain(h), "gate": mat(I, h), "up": mat(I, h),
            "down": mat(h, I),
        })
    w["layers"] = layers
    if geo.kv_dtype == "fp8":
        w["kv_scale"] = make_kv_scales(geo)
    return w


def make_kv_scales(geo: Geometry, seed: int = SEED_KVSCALE):
    sigma = 0.02 * np.sqrt(geo.hidden)
    u = _rng(seed).uniform(0.0, 0.1, size=(geo.num_layers, 2, geo.num_kv_heads))
    return (sigma * 5.0 / 448.0 * (1.0 + u)).astype(np.float32)


def make_stack(geo: Geometry, rows: int, seed: int = SEED_STACK, tag: int = 0):
    """Captured target hidden stacks, [rows, T * Ht] bf16 ~ N(0, 1)."""
    x = _rng(seed, tag).standard_normal((rows, geo.num_target_layers * geo.target_hidden), dtype=np.float32)
    return to_bf16_bits(x)


def make_tokens(geo: Geometry, n: int, seed: int = SEED_TOKENS, tag: int = 0):
    return _rng(seed, tag).integers(0, geo.vocab, size=n, dtype=np.int64).astype(np.uint32)


def make_bitmask(vocab: int, frac: float, seed: int = SEED_MASK, tag: int = 0):
    """int32 words [ceil(vocab/32)]: exactly round(frac * vocab) bits set."""
    words = (vocab + 31) // 32
    n_on = int(round(frac * vocab))
    on = _rng(seed, tag).permutation(vocab)[:n_on]
    bits = np.zeros(words * 32, dtype=np.uint8)
    bits[on] = 1
    packed = np.packbits(bits.reshape(words, 32), axis=1, bitorder="little")
    return packed.view(np.uint32).reshape(words).view(np.int32).copy()


def make_ctx_lengths(n: int, lo: int, hi: int, seed: int = SEED_CTX, tag: int = 0):
    return _rng(seed, tag).integers(lo, hi + 1, size=n, dtype=np.int64)


def make_accepted(n: int, hi: int, seed: int = SEED_ACCEPT, tag: int = 0):
    return _rng(seed, tag).integers(0, hi + 1, size=n, dtype=np.int64)


def make_block_permutation(n_blocks: int, pool_blocks: int, seed: int = SEED_BLOCKS, tag: int = 0):
    """n_blocks distinct physical block ids drawn from [0, pool_blocks)."""
    return _rng(seed, tag).permutation(pool_blocks)[:n_blocks].astype(np.int32)
