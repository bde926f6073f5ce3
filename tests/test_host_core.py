"""CPU tests of the HIP-free host core (config validation, block pool,
append / trim bookkeeping) through libdflash_host.so, and of the HIP
library's exported C ABI (symbols only: no device calls without a GPU)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_diffusion_draft_03_amd")
HOST_LIB = os.path.join(PKG, "libdflash_host.so")
INT64_MAX = (1 << 63) - 1

OK, E_INVALID, E_SHAPE, E_NOMEM, E_NO_BLOCKS, E_DECLINED, E_HIP = 0, -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def host():
    if not os.path.exists(HOST_LIB):
        from block_diffusion_draft_03_amd import build
        build.build_host_lib()
    lib = C.CDLL(HOST_LIB)
    vp = C.c_void_p
    lib.dfh_last_error.restype = C.c_char_p
    lib.dfh_validate.argtypes = [vp]
    lib.dfh_pool_new.restype = vp
    lib.dfh_pool_new.argtypes = [C.c_int32]
    lib.dfh_pool_delete.argtypes = [vp]
    lib.dfh_pool_free_count.argtypes = [vp]
    lib.dfh_seq_new.restype = vp
    lib.dfh_seq_new.argtypes = [vp, C.c_int64, vp, C.c_int32, C.c_int32, C.POINTER(C.c_int)]
    lib.dfh_seq_append.argtypes = [vp, vp, C.c_int32]
    lib.dfh_seq_trim.argtypes = [vp, C.c_int32]
    lib.dfh_seq_ctx_len.argtypes = [vp]
    lib.dfh_seq_pending.argtypes = [vp]
    lib.dfh_seq_blocks.argtypes = [vp, vp, C.c_int32]
    lib.dfh_seq_release.argtypes = [vp, vp]
    lib.dfh_seq_delete.argtypes = [vp]
    lib.dfh_seq_take.argtypes = [vp, vp, C.c_int32, C.POINTER(C.c_int32)]
    lib.dfh_seq_install.argtypes = [vp, vp, vp, C.c_int32, C.c_int32, C.c_int32]
    lib.dfh_reserve_rows.argtypes = [vp, C.c_int32, vp, vp, vp]
    lib.dfh_attn_tiles.argtypes = [C.c_int32, C.c_int32]
    lib.dfh_attn_plan.argtypes = [C.c_int32, vp, C.c_int32, C.c_int32, C.c_int64, C.c_int32, C.POINTER(C.c_int32),
                                  C.POINTER(C.c_int32), vp, vp]
    lib.dfh_build_check.argtypes = [vp, C.c_int32]
    lib.dflash_yarn_inv_freq.argtypes = [C.c_int32, C.c_float, C.c_float, C.c_float, C.c_float, C.c_int32, vp]
    return lib


def make_cfg(geo=synth.FULL, **over):
    from block_diffusion_draft_03_amd.binding import Config, DTYPE
    d = dict(num_layers=geo.num_layers, hidden=geo.hidden, intermediate=geo.intermediate,
             num_q_heads=geo.num_q_heads, num_kv_heads=geo.num_kv_heads, head_dim=geo.head_dim, vocab=geo.vocab,
             gamma=geo.gamma, mask_token_id=geo.mask_token_id, num_target_layers=geo.num_target_layers,
             target_hidden=geo.target_hidden, ctx_window=geo.ctx_window, rope_theta=geo.rope_theta,
             rms_eps=geo.rms_eps, kv_block_size=16, kv_pool_blocks=1024, max_batch=64, max_seq_len=8192,
             weight_dtype=DTYPE[geo.weight_dtype], lm_head_dtype=DTYPE[geo.lm_head_dtype], kv_dtype=DTYPE[geo.kv_dtype])
    d.update(over)
    return Config(**d)


def test_valid_configs(host):
    for geo in (synth.TINY, synth.FULL, synth.FULL_FP8):
        assert host.dfh_validate(C.byref(make_cfg(geo))) == OK, host.dfh_last_error()


@pytest.mark.parametrize("field,value", [
    ("num_layers", 0), ("hidden", 100), ("intermediate", 96), ("head_dim", 48), ("num_kv_heads", 3),
    ("gamma", 1), ("gamma", 65), ("vocab", 1), ("mask_token_id", 248320), ("ctx_window", -1),
    ("kv_block_size", 32), ("kv_pool_blocks", 0), ("max_batch", 0), ("max_batch", 65), ("max_seq_len", 0),
    ("rope_theta", 0.5), ("rms_eps", -1.0), ("weight_dtype", 2), ("lm_head_dtype", 0), ("kv_dtype", 0),
    ("target_hidden", 0), ("gamma", 32), ("shifted_rows", 2), ("shifted_rows", -1),
    ("lm_act_fp8", 2)])
def test_invalid_configs(host, field, value):
    # gamma 32 with 8 query heads per kv head gives 256 query rows per kv head
    cfg = make_cfg(**{field: value})
    assert host.dfh_validate(C.byref(cfg)) == E_INVALID
    assert host.dfh_last_error().decode().startswith("config:")


def test_fp8_kv_needs_wide_heads(host):
    # E4M3 K rows are read 16 dims per lane group, so head_dim must be >= 64
    cfg = make_cfg(head_dim=32, kv_dtype=2)
    assert host.dfh_validate(C.byref(cfg)) == E_INVALID
    assert "head_dim" in host.dfh_last_error().decode()
    assert host.dfh_validate(C.byref(make_cfg(head_dim=64, kv_dtype=2))) == OK


def test_w8a8_head_needs_fp8_head_and_tiled_shapes(host):
    # E4M3 activations go into the tiled E4M3 head only
    assert host.dfh_validate(C.byref(make_cfg(lm_act_fp8=1, lm_head_dtype=1))) == E_INVALID
    assert "FP8_E4M3 LM head" in host.dfh_last_error().decode()
    assert host.dfh_validate(C.byref(make_cfg(lm_act_fp8=1, lm_head_dtype=2, vocab=248000))) == E_INVALID
    assert host.dfh_validate(C.byref(make_cfg(lm_act_fp8=1, lm_head_dtype=2))) == OK


def _seq(host, pool, budget=INT64_MAX, ids=None, max_seq_len=8192):
    st = C.c_int()
    arr = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
    s = host.dfh_seq_new(pool, budget, None if arr is None else arr.ctypes.data_as(C.c_void_p),
                         0 if arr is None else len(arr), max_seq_len, C.byref(st))
    return s, st.value


def _blocks(host, s):
    out = np.zeros(4096, dtype=np.int32)
    n = host.dfh_seq_blocks(s, out.ctypes.data_as(C.c_void_p), 4096)
    return out[:n].tolist()


def test_pool_lowest_free_first_and_release(host):
    pool = host.dfh_pool_new(8)
    a, st = _seq(host, pool, budget=40)           # 3 blocks now
    assert st == OK and _blocks(host, a) == [0, 1, 2]
    b, st = _seq(host, pool, budget=16)
    assert st == OK and _blocks(host, b) == [3]
    host.dfh_seq_release(a, pool)
    assert host.dfh_pool_free_count(pool) == 7
    c, st = _seq(host, pool, budget=17)           # reuses the lowest ids
    assert st == OK and _blocks(host, c) == [0, 1]
    for s in (a, b, c):
        host.dfh_seq_delete(s)
    host.dfh_pool_delete(pool)


def test_budget_and_pool_exhaustion(host):
    pool = host.dfh_pool_new(4)
    s, st = _seq(host, pool, budget=100)          # needs 7 blocks
    assert s is None and st == E_NO_BLOCKS
    assert host.dfh_pool_free_count(pool) == 4    # nothing taken
    g, st = _seq(host, pool)                       # grow mode, unknown budget
    assert st == OK
    assert host.dfh_seq_append(g, pool, 33) == OK and _blocks(host, g) == [0, 1, 2]
    assert host.dfh_seq_append(g, pool, 40) == E_NO_BLOCKS      # pool has one block left
    assert host.dfh_seq_ctx_len(g) == 33 and _blocks(host, g) == [0, 1, 2]
    assert host.dfh_seq_append(g, pool, 15) == OK and _blocks(host, g) == [0, 1, 2]   # 48 rows fit
    assert host.dfh_seq_append(g, pool, 1) == OK and _blocks(host, g) == [0, 1, 2, 3]
    h, st = _seq(host, pool, max_seq_len=10)
    host.dfh_seq_release(g, pool)
    assert host.dfh_seq_append(h, pool, 10) == OK
    assert host.dfh_seq_append(h, pool, 1) == E_NO_BLOCKS       # max_seq_len ceiling
    host.dfh_seq_delete(g)
    host.dfh_seq_delete(h)
    host.dfh_pool_delete(pool)


def test_explicit_blocks(host):
    pool = host.dfh_pool_new(16)
    ids = [9, 3, 14]
    s, st = _seq(host, pool, ids=ids)
    assert st == OK and _blocks(host, s) == ids and host.dfh_pool_free_count(pool) == 13
    assert host.dfh_seq_append(s, pool, 48) == OK
    assert host.dfh_seq_append(s, pool, 1) == E_NO_BLOCKS        # capacity = 3 blocks
    t, st = _seq(host, pool, ids=[2, 3])                          # 3 is taken
    assert t is None and st == E_NO_BLOCKS and host.dfh_pool_free_count(pool) == 13
    host.dfh_seq_delete(s)
    host.dfh_pool_delete(pool)


def test_trim_semantics(host):
    pool = host.dfh_pool_new(64)
    s, _ = _seq(host, pool)
    assert host.dfh_seq_append(s, pool, 20) == OK
    assert host.dfh_seq_trim(s, 20) == OK                          # commit all
    assert host.dfh_seq_pending(s) == 0
    assert host.dfh_seq_append(s, pool, 16) == OK
    assert host.dfh_seq_trim(s, 17) == E_INVALID                   # more than pending
    assert host.dfh_seq_trim(s, -1) == E_INVALID
    assert host.dfh_seq_ctx_len(s) == 36
    assert host.dfh_seq_trim(s, 5) == OK
    assert host.dfh_seq_ctx_len(s) == 25 and host.dfh_seq_pending(s) == 0
    assert host.dfh_seq_append(s, pool, 8) == OK and host.dfh_seq_append(s, pool, 8) == OK
    assert host.dfh_seq_pending(s) == 16                           # two appends since the verify
    assert host.dfh_seq_trim(s, 0) == OK and host.dfh_seq_ctx_len(s) == 25
    host.dfh_seq_delete(s)
    host.dfh_pool_delete(pool)


def test_kv_carry_take_and_install(host):
    """Carrying a sequence's KV ([DraftProposer] take_drafter_kv /
    install_drafter_kv): take moves every block and the row count out and
    leaves the state empty and growing; install gives them to a state with
    no rows (whose own blocks go back to the pool) and refuses bad lists."""
    pool = host.dfh_pool_new(64)
    a, _ = _seq(host, pool)
    assert host.dfh_seq_append(a, pool, 40) == OK and host.dfh_seq_trim(a, 40) == OK
    before = host.dfh_pool_free_count(pool)
    out, rows = np.zeros(8, dtype=np.int32), C.c_int32()
    n = host.dfh_seq_take(a, out.ctypes.data_as(C.c_void_p), 8, C.byref(rows))
    assert n == 3 and rows.value == 40
    assert host.dfh_seq_ctx_len(a) == 0 and host.dfh_seq_blocks(a, None, 0) == 0
    assert host.dfh_pool_free_count(pool) == before              # carried blocks stay allocated
    assert host.dfh_seq_append(a, pool, 5) == OK                  # the emptied state grows again
    carried = out[:3].copy()
    p = lambda arr: arr.ctypes.data_as(C.c_void_p)
    assert host.dfh_seq_install(a, pool, p(carried), 3, 40, 8192) == E_INVALID     # the state holds rows
    b, _ = _seq(host, pool, budget=32)                             # a fresh state with 2 own blocks
    free_before = host.dfh_pool_free_count(pool)
    assert host.dfh_seq_install(b, pool, p(carried), 3, 49, 8192) == E_INVALID     # 49 rows > 3 blocks
    assert host.dfh_seq_install(b, pool, p(np.array([carried[0], carried[0]], np.int32)), 2, 10, 8192) == E_INVALID
    free_id = np.array([63], np.int32)
    assert host.dfh_seq_install(b, pool, p(free_id), 1, 1, 8192) == E_INVALID      # not an allocated block
    assert host.dfh_pool_free_count(pool) == free_before          # errors change nothing
    assert host.dfh_seq_install(b, pool, p(carried), 3, 40, 39) == E_INVALID  # > max_seq_len
    assert host.dfh_seq_install(b, pool, p(carried), 3, 40, 8192) == OK
    assert host.dfh_seq_ctx_len(b) == 40 and host.dfh_seq_pending(b) == 0
    got = np.zeros(8, dtype=np.int32)
    assert host.dfh_seq_blocks(b, p(got), 8) == 3 and np.array_equal(got[:3], carried)
    assert host.dfh_pool_free_count(pool) == free_before + 2     # b's own two blocks returned
    # b's row capacity grew from its 32-token budget to the 48 rows of the installed blocks
    assert host.dfh_seq_append(b, pool, 8) == OK and host.dfh_seq_ctx_len(b) == 48
    assert host.dfh_seq_append(b, pool, 1) == E_NO_BLOCKS
    for s in (a, b):
        host.dfh_seq_release(s, pool)
        host.dfh_seq_delete(s)
    assert host.dfh_pool_free_count(pool) == 64
    host.dfh_pool_delete(pool)


def test_hip_library_exports_every_declared_symbol():
    """libdflash.so loads without a GPU and exports every function
    include/dflash.h declares (no compute calls are made here)."""
    from block_diffusion_draft_03_amd.binding import EXPORTED_SYMBOLS, load_library
    with open(os.path.join(ROOT, "include", "dflash.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", header))
    assert declared == set(EXPORTED_SYMBOLS)
    lib = load_library()
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.dflash_last_error() == b""


@pytest.mark.parametrize("theta,d", [(1e7, 128), (1e6, 64), (1e6, 16)])
def test_yarn_table_matches_oracle(host, theta, d):
    """The library's YaRN table (host code, the same in libdflash.so) equals
    the oracle's f32 table to one float32 rounding step; bad arguments are
    refused."""
    from oracle.dflash import yarn_inv_freq
    out = np.zeros(d // 2, dtype=np.float32)
    assert host.dflash_yarn_inv_freq(d, theta, 64.0, 32.0, 1.0, 4096, out.ctypes.data_as(C.c_void_p)) == OK
    ref = yarn_inv_freq(theta, d, 64.0, 32.0, 1.0, 4096)
    assert np.allclose(out.astype(np.float64), ref, rtol=2.0 ** -23, atol=0.0)
    for args in ((d + 1, theta, 64.0, 32.0, 1.0, 4096), (d, 1.0, 64.0, 32.0, 1.0, 4096),
                 (d, theta, 0.5, 32.0, 1.0, 4096), (d, theta, 64.0, 1.0, 32.0, 4096),
                 (d, theta, 64.0, 32.0, 1.0, 0)):
        assert host.dflash_yarn_inv_freq(*args, out.ctypes.data_as(C.c_void_p)) == E_INVALID
    assert host.dflash_yarn_inv_freq(d, theta, 64.0, 32.0, 1.0, 4096, None) == E_INVALID



# --------------------------------------------------------------------------
# error contract: what the library checks before it enqueues anything
# --------------------------------------------------------------------------

def test_multi_state_reservation_is_all_or_nothing(host):
    """A precompute over several states reserves blocks for all of them or
    for none: when a later state cannot take its rows, the blocks the earlier
    ones took go back and the pool and every state are as before."""
    pool = host.dfh_pool_new(20)
    a, _ = _seq(host, pool)                     # grows from the pool
    b, _ = _seq(host, pool, budget=16)          # one block, 16 rows at most
    c, _ = _seq(host, pool)
    assert host.dfh_seq_append(a, pool, 5) == OK
    blocks_a = _blocks(host, a)
    free0 = host.dfh_pool_free_count(pool)
    seqs = (C.c_void_p * 3)(a, c, b)
    p = lambda arr: arr.ctypes.data_as(C.c_void_p)
    # a and c fit, b's 20 rows exceed its budget: nothing is kept
    assert host.dfh_reserve_rows(seqs, 3, p(np.array([40, 33, 20], np.int32)), None, pool) == E_NO_BLOCKS
    assert "state 2" in host.dfh_last_error().decode()
    assert host.dfh_pool_free_count(pool) == free0
    assert _blocks(host, a) == blocks_a and _blocks(host, c) == []
    # the pool runs dry at the second state (6 + 13 blocks > 18 free)
    assert host.dfh_reserve_rows(seqs, 3, p(np.array([100, 200, 0], np.int32)), None, pool) == E_NO_BLOCKS
    assert "state 1" in host.dfh_last_error().decode()
    assert host.dfh_pool_free_count(pool) == free0 and _blocks(host, a) == blocks_a
    # a block-table capacity below what a state needs is refused the same way
    caps = np.array([8, 1, 1], np.int32)
    assert host.dfh_reserve_rows(seqs, 3, p(np.array([40, 33, 0], np.int32)), p(caps), pool) == E_NO_BLOCKS
    assert host.dfh_pool_free_count(pool) == free0 and _blocks(host, c) == []
    # and when everything fits, all states get their blocks
    assert host.dfh_reserve_rows(seqs, 3, p(np.array([40, 33, 16], np.int32)), None, pool) == OK
    assert len(_blocks(host, a)) == 3 and len(_blocks(host, c)) == 3
    for s in (a, b, c):
        host.dfh_seq_release(s, pool)
        host.dfh_seq_delete(s)
    assert host.dfh_pool_free_count(pool) == 20
    host.dfh_pool_delete(pool)


def test_state_rows_capped_at_max_seq_len(host):
    pool = host.dfh_pool_new(64)
    s, st = _seq(host, pool, budget=1000, max_seq_len=100)   # budget above the ceiling: 7 blocks, 100 rows
    assert st == OK and len(_blocks(host, s)) == 7
    assert host.dfh_seq_append(s, pool, 100) == OK and host.dfh_seq_append(s, pool, 1) == E_NO_BLOCKS
    t, st = _seq(host, pool, ids=np.arange(20, 30), max_seq_len=100)  # 10 blocks, still 100 rows
    assert st == OK
    assert host.dfh_seq_append(t, pool, 101) == E_NO_BLOCKS and host.dfh_seq_append(t, pool, 100) == OK
    for x in (s, t):
        host.dfh_seq_release(x, pool)
        host.dfh_seq_delete(x)
    host.dfh_pool_delete(pool)


def _plan(host, tiles, n_kv=4, max_tps=64, cap=1 << 20, target=512, split0=None):
    t = np.ascontiguousarray(tiles, dtype=np.int32)
    tps, n_split = C.c_int32(), C.c_int32()
    per = np.zeros(len(t), np.int32)
    s0 = np.full(len(t), -1, np.int32)
    rc = host.dfh_attn_plan(len(t), t.ctypes.data_as(C.c_void_p), n_kv, max_tps, cap, target, C.byref(tps),
                            C.byref(n_split), per.ctypes.data_as(C.c_void_p), s0.ctypes.data_as(C.c_void_p))
    if split0 is not None:
        split0[:] = s0.tolist()
    return rc, tps.value, n_split.value, per.tolist()


def test_attention_split_plan(host):
    """Tiles from the 16-aligned window start; one sequence of 1024 ctx rows:
    32 tiles in 16 splits of 2 plus the block tile's split; the preferred split
    count yields to the tile limit for long windows; too many sequences of
    long windows have no plan."""
    assert host.dfh_attn_tiles(1024, 4096) == 32
    assert host.dfh_attn_tiles(0, 4096) == 0 and host.dfh_attn_tiles(500, 0) == 0
    assert host.dfh_attn_tiles(4100, 4096) == 129      # rows [4, 4100) from aligned start 0
    assert host.dfh_attn_tiles(4112, 4096) == 128      # rows [16, 4112)
    assert _plan(host, [32]) == (OK, 2, 17, [17])
    assert _plan(host, [0]) == (OK, 1, 1, [1])           # the block tile alone
    # a batch: splits grow until the launch fits two workgroups per CU
    rc, tps, n_split, per = _plan(host, [32] * 32)
    assert rc == OK and n_split * 4 <= 512 and per == [(32 + tps) // tps] * 32
    # a larger target: shorter splits, at most 768 workgroups
    rc8, tps8, n_split8, _ = _plan(host, [32] * 32, target=768)
    assert rc8 == OK and tps8 < tps and 512 < n_split8 * 4 <= 768
    assert _plan(host, [32], target=0)[0] == E_INVALID
    # 1025 tiles (a 32768-row window): 64 tiles per split, 17 splits
    assert _plan(host, [1025]) == (OK, 64, 17, [17])
    # 64 such sequences need 1088 splits > 1024
    rc, *_ = _plan(host, [1025] * 64)
    assert rc == E_INVALID and "attention splits" in host.dfh_last_error().decode()
    # more than 64 splits of 64 tiles for one sequence
    assert _plan(host, [64 * 64])[0] == E_INVALID


def test_attention_split_order(host):
    """Each sequence's splits are one run of split numbers; the runs cover
    [0, n_split) exactly, go out in non-increasing order of split length (the
    kernel divides T + 2 units among a sequence's splits), and keep the
    sequence order between equal lengths."""
    rng = np.random.default_rng(5)
    for tiles in ([32, 8, 120, 0, 64, 8, 127, 31], list(rng.integers(0, 128, 64)), [16] * 10):
        s0 = [0] * len(tiles)
        rc, tps, n_split, per = _plan(host, tiles, target=768, split0=s0)
        assert rc == OK
        runs = sorted((s0[i], per[i], i) for i in range(len(tiles)))
        pos = 0
        for start, cnt, _ in runs:
            assert start == pos
            pos += cnt
        assert pos == n_split
        # split length (T + 2) / nsplit, in dispatch order
        lens = [((tiles[i] + 2) / per[i], i) for _, _, i in runs]
        for (a, ia), (b, ib) in zip(lens, lens[1:]):
            assert a > b or (a == b and ia < ib)


def test_build_rejects_configs_beyond_the_attention_splits(host):
    """dflash_build's capacity check (the same host code): 64 sequences of a
    32768-row window cannot be planned, 32 can, and the full workloads'
    configs pass."""
    assert host.dfh_build_check(C.byref(make_cfg(max_batch=64, ctx_window=32768, max_seq_len=32768)), 64) == E_INVALID
    assert "attention splits" in host.dfh_last_error().decode()
    assert host.dfh_build_check(C.byref(make_cfg(max_batch=32, ctx_window=32768, max_seq_len=32768)), 64) == OK
    # a long window with short states is fine: the states bound the tiles
    assert host.dfh_build_check(C.byref(make_cfg(max_batch=64, ctx_window=32768, max_seq_len=8192)), 64) == OK
    for geo in (synth.TINY, synth.FULL, synth.FULL_FP8):
        assert host.dfh_build_check(C.byref(make_cfg(geo, max_batch=64, max_seq_len=8192)), 64) == OK
