"""ctypes binding of libdflash.so (include/dflash.h).

Argument marshalling only: every step of the propose path runs in the HIP
library. ``load_library()`` exposes the raw C functions under their C names
(``lib.dflash_build`` ...); ``Head`` / ``State`` wrap them for callers that
hold PyTorch device tensors.
"""
import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))

DFLASH_OK = 0
STATUS = {0: "OK", -1: "E_INVALID", -2: "E_SHAPE", -3: "E_NOMEM", -4: "E_NO_BLOCKS", -5: "E_DECLINED", -6: "E_HIP"}
DTYPE = {"f32": 0, "bf16": 1, "fp8": 2}
NO_TOKEN = 0xFFFFFFFF
INT64_MAX = (1 << 63) - 1

EXPORTED_SYMBOLS = (
    "dflash_build", "dflash_destroy", "dflash_block_gamma", "dflash_propose_batch_max",
    "dflash_state_create", "dflash_state_free", "dflash_state_ctx_len", "dflash_precompute_ctx_kv",
    "dflash_propose", "dflash_propose_batch", "dflash_propose_noalloc", "dflash_after_verify", "dflash_take_kv", "dflash_install_kv",
    "dflash_free_kv", "dflash_state_read_kv",
    "dflash_read_lm_head_fp8", "dflash_yarn_inv_freq", "dflash_timing_enable", "dflash_timing_read",
    "dflash_last_error",
)
PHASE_LM_HEAD, PHASE_PROPOSE, PHASE_PRECOMPUTE = 0, 1, 2


class DflashError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("num_layers", "hidden", "intermediate", "num_q_heads", "num_kv_heads",
                                         "head_dim", "vocab", "gamma")] + [
        ("mask_token_id", C.c_uint32), ("num_target_layers", C.c_int32), ("target_hidden", C.c_int32),
        ("ctx_window", C.c_int32), ("rope_theta", C.c_float), ("rms_eps", C.c_float),
        ("kv_block_size", C.c_int32), ("kv_pool_blocks", C.c_int32), ("max_batch", C.c_int32),
        ("max_seq_len", C.c_int32), ("weight_dtype", C.c_int), ("lm_head_dtype", C.c_int), ("kv_dtype", C.c_int),
        ("shifted_rows", C.c_int32), ("fp8_weights", C.c_int32), ("lm_act_fp8", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("in_norm", "q", "k", "v", "o", "post_norm", "gate", "up", "down")]


class Weights(C.Structure):
    _fields_ = [("fc", C.c_void_p), ("hidden_norm", C.c_void_p), ("norm", C.c_void_p),
                ("embed_tokens", C.c_void_p), ("lm_head", C.c_void_p), ("lm_head_fp8", C.c_void_p),
                ("lm_head_scale", C.c_void_p), ("kv_scale", C.c_void_p), ("inv_freq", C.c_void_p),
                ("layers", C.POINTER(LayerWeights))]


def library_path():
    return os.path.join(_PKG, "libdflash.so")


_LIB = None


def load_library(path=None):
    """Load libdflash.so and declare the C signatures. Raises when the
    library has not been built: there is no fallback path."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m block_diffusion_draft_03_amd.build`")
    lib = C.CDLL(p)
    vp, i32, i64, u32, u64 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64
    sig = {
        "dflash_build": ([C.POINTER(Config), C.POINTER(Weights), u64, C.POINTER(vp)], C.c_int),
        "dflash_destroy": ([vp], None),
        "dflash_block_gamma": ([vp], C.c_int),
        "dflash_propose_batch_max": ([vp], C.c_int),
        "dflash_state_create": ([vp, i64, vp, i32, C.POINTER(vp)], C.c_int),
        "dflash_state_free": ([vp, vp], C.c_int),
        "dflash_state_ctx_len": ([vp], C.c_int),
        "dflash_precompute_ctx_kv": ([vp, vp, i32, vp, vp, u64], C.c_int),
        "dflash_propose": ([vp, vp, u32, i64, i32, vp, vp, vp, vp, vp, u64], C.c_int),
        "dflash_propose_batch": ([vp, vp, i32, vp, vp, i32, vp, vp, vp, vp, vp, u64], C.c_int),
        "dflash_propose_noalloc": ([vp, vp, u32, i64, i32, vp, vp, vp, vp, vp, u64], C.c_int),
        "dflash_after_verify": ([vp, vp, i32], C.c_int),
        "dflash_take_kv": ([vp, vp, vp, i32, C.POINTER(i32), C.POINTER(i32), C.POINTER(i64)], C.c_int),
        "dflash_install_kv": ([vp, vp, vp, i32, i32, i64], C.c_int),
        "dflash_free_kv": ([vp, vp, i32], C.c_int),
        "dflash_state_read_kv": ([vp, vp, i32, i32, i32, vp, vp, u64], C.c_int),
        "dflash_read_lm_head_fp8": ([vp, vp, vp, u64], C.c_int),
        "dflash_yarn_inv_freq": ([i32, C.c_float, C.c_float, C.c_float, C.c_float, i32, vp], C.c_int),
        "dflash_timing_enable": ([vp, C.c_int], C.c_int),
        "dflash_timing_read": ([vp, i32, C.POINTER(C.c_double), C.POINTER(C.c_int64)], C.c_int),
        "dflash_last_error": ([], C.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    if path is None:
        _LIB = lib
    return lib


def _check(lib, rc):
    if rc < 0:
        raise DflashError(rc, lib.dflash_last_error().decode())
    return rc


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _on(stream):
    """Context in which the call's tensors (outputs and uploaded temporaries)
    are allocated on the stream the library enqueues on: torch's caching
    allocator then hands a freed temporary out again only in that stream's
    order, after the kernels that read it."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def to_device(arr, device="cuda"):
    """numpy array (uint16 = bf16 bits, uint8 = E4M3 codes, f32, i32) ->
    torch device tensor holding the same bytes."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    return torch.from_numpy(a).to(device)


class State:
    def __init__(self, head, handle):
        self.head = head
        self.handle = handle

    @property
    def ctx_len(self):
        return _check(self.head.lib, self.head.lib.dflash_state_ctx_len(self.handle))

    def free(self):
        if self.handle:
            _check(self.head.lib, self.head.lib.dflash_state_free(self.head.handle, self.handle))
            self.handle = None


def yarn_inv_freq(head_dim, rope_theta, factor, beta_fast, beta_slow, original_max_positions):
    """The library's YaRN-corrected RoPE table (f32 [head_dim / 2], host), to
    pass to Head(..., inv_freq=...)."""
    lib = load_library()
    out = np.zeros(head_dim // 2, dtype=np.float32)
    _check(lib, lib.dflash_yarn_inv_freq(int(head_dim), float(rope_theta), float(factor), float(beta_fast),
                                         float(beta_slow), int(original_max_positions),
                                         out.ctypes.data_as(C.c_void_p)))
    return out


class Head:
    """A built draft head. ``weights`` is the dict synth.make_weights returns
    (numpy arrays); they are uploaded, and the borrowed ones kept alive."""

    def __init__(self, geo, weights, kv_pool_blocks=1024, max_batch=1, max_seq_len=8192, stream=None,
                 lm_head_fp8=None, lm_head_scale=None, inv_freq=None, device="cuda"):
        import torch
        self.lib = load_library()
        self.geo = geo
        self.device = device
        self.keep = []
        cfg = Config(num_layers=geo.num_layers, hidden=geo.hidden, intermediate=geo.intermediate,
                     num_q_heads=geo.num_q_heads, num_kv_heads=geo.num_kv_heads, head_dim=geo.head_dim,
                     vocab=geo.vocab, gamma=geo.gamma, mask_token_id=geo.mask_token_id,
                     num_target_layers=geo.num_target_layers, target_hidden=geo.target_hidden,
                     ctx_window=geo.ctx_window, rope_theta=geo.rope_theta, rms_eps=geo.rms_eps,
                     kv_block_size=geo.kv_block, kv_pool_blocks=kv_pool_blocks, max_batch=max_batch,
                     max_seq_len=max_seq_len, weight_dtype=DTYPE[geo.weight_dtype],
                     lm_head_dtype=DTYPE[geo.lm_head_dtype], kv_dtype=DTYPE[geo.kv_dtype],
                     shifted_rows=int(getattr(geo, "shifted_rows", 0)),
                     fp8_weights=int(getattr(geo, "layer_dtype", "bf16") == "fp8"),
                     lm_act_fp8=int(getattr(geo, "lm_act_dtype", "bf16") == "fp8"))
        self.cfg = cfg

        def dev(a):
            t = to_device(a, device)
            self.keep.append(t)
            return _ptr(t)

        layers = (LayerWeights * geo.num_layers)()
        for i, lw in enumerate(weights["layers"]):
            for k in ("in_norm", "q", "k", "v", "o", "post_norm", "gate", "up", "down"):
                setattr(layers[i], k, dev(lw[k]))
        w = Weights()
        w.fc = dev(weights["fc"])
        w.hidden_norm = dev(weights["hidden_norm"])
        w.norm = dev(weights["norm"])
        w.embed_tokens = dev(weights["embed"])
        w.lm_head = dev(weights["lm_head"])
        if lm_head_fp8 is not None:
            w.lm_head_fp8 = dev(lm_head_fp8)
            w.lm_head_scale = dev(np.asarray(lm_head_scale, np.float32))
        kvs = None
        if geo.kv_dtype == "fp8":
            kvs = np.ascontiguousarray(weights["kv_scale"], dtype=np.float32)
            w.kv_scale = kvs.ctypes.data_as(C.c_void_p)
        table = None
        if inv_freq is not None:
            # a host f32 [head_dim / 2] RoPE table (e.g. yarn_inv_freq) replaces the plain theta table
            table = np.ascontiguousarray(inv_freq, dtype=np.float32)
            if table.shape != (geo.head_dim // 2,):
                raise ValueError(f"inv_freq must have head_dim / 2 = {geo.head_dim // 2} entries")
            w.inv_freq = table.ctypes.data_as(C.c_void_p)
        w.layers = layers
        h = C.c_void_p()
        _check(self.lib, self.lib.dflash_build(C.byref(cfg), C.byref(w), _stream_handle(stream), C.byref(h)))
        self.handle = h
        # only the borrowed tensors must outlive the head
        torch.cuda.synchronize()
        self.keep = [t for t in self.keep if t.data_ptr() in (w.embed_tokens, w.lm_head, w.lm_head_fp8,
                                                              w.lm_head_scale)]

    # --- API with the C names' roles ----------------------------------------
    @property
    def gamma(self):
        return _check(self.lib, self.lib.dflash_block_gamma(self.handle))

    @property
    def batch_max(self):
        return _check(self.lib, self.lib.dflash_propose_batch_max(self.handle))

    def state_create(self, budget_tokens=None, block_ids=None):
        budget = INT64_MAX if budget_tokens is None else int(budget_tokens)
        ids = None
        n_ids = 0
        if block_ids is not None:
            ids = np.ascontiguousarray(block_ids, dtype=np.int32)
            n_ids = len(ids)
        h = C.c_void_p()
        _check(self.lib, self.lib.dflash_state_create(self.handle, budget,
                                                      None if ids is None else ids.ctypes.data_as(C.c_void_p),
                                                      n_ids, C.byref(h)))
        return State(self, h)

    def precompute(self, states, n_new, stack, stream=None):
        """Append ctx rows: stack is a device tensor [sum(n_new), T*Ht] (bf16
        bits as int16) or a numpy uint16 array (uploaded)."""
        with _on(stream):
            if isinstance(stack, np.ndarray):
                stack = to_device(stack, self.device)
            arr = (C.c_void_p * len(states))(*[s.handle.value for s in states])
            nn = np.ascontiguousarray(n_new, dtype=np.int32)
            _check(self.lib, self.lib.dflash_precompute_ctx_kv(self.handle, arr, len(states),
                                                               nn.ctypes.data_as(C.c_void_p), _ptr(stack),
                                                               _stream_handle(stream)))
        return stack

    def propose(self, state, last_token, position, num_drafts, bitmask=None, logits=False, stream=None):
        import torch
        g = self.geo.gamma
        with _on(stream):
            ids = torch.empty(g, dtype=torch.int32, device=self.device)
            conf = torch.empty(1, dtype=torch.float32, device=self.device)
            rp = torch.empty(g, dtype=torch.float32, device=self.device)
            lg = torch.empty((g, self.geo.vocab), dtype=torch.float32, device=self.device) if logits else None
            if isinstance(bitmask, np.ndarray):
                bitmask = to_device(bitmask, self.device)
            _check(self.lib, self.lib.dflash_propose(self.handle, state.handle, int(last_token), int(position),
                                                     int(num_drafts), _ptr(bitmask), _ptr(ids), _ptr(conf),
                                                     _ptr(rp), _ptr(lg), _stream_handle(stream)))
        return {"ids": ids, "conf": conf, "row_prob": rp, "logits": lg}

    def propose_noalloc(self, state, last_token, position, num_drafts, bitmask=None, out=None, stream=None):
        """dflash_propose_noalloc: the library allocates nothing; `out` holds
        caller-allocated device tensors ids (int32 [gamma]), conf (f32 [1]),
        row_prob (f32 [gamma] or None) and logits (f32 [gamma, V] or None),
        allocated here when not given; `bitmask` is a device tensor or None."""
        import torch
        g = self.geo.gamma
        with _on(stream):
            if out is None:
                out = {"ids": torch.empty(g, dtype=torch.int32, device=self.device),
                       "conf": torch.empty(1, dtype=torch.float32, device=self.device),
                       "row_prob": torch.empty(g, dtype=torch.float32, device=self.device), "logits": None}
            if isinstance(bitmask, np.ndarray):
                bitmask = to_device(bitmask, self.device)
            _check(self.lib, self.lib.dflash_propose_noalloc(self.handle, state.handle, int(last_token), int(position),
                                                             int(num_drafts), _ptr(bitmask), _ptr(out["ids"]),
                                                             _ptr(out["conf"]), _ptr(out.get("row_prob")),
                                                             _ptr(out.get("logits")), _stream_handle(stream)))
        return out

    def propose_batch(self, states, last_tokens, positions, num_drafts, bitmasks=None, logits=False, stream=None):
        import torch
        n, g = len(states), self.geo.gamma
        with _on(stream):
            ids = torch.empty((n, g), dtype=torch.int32, device=self.device)
            conf = torch.empty(n, dtype=torch.float32, device=self.device)
            rp = torch.empty((n, g), dtype=torch.float32, device=self.device)
            lg = torch.empty((n, g, self.geo.vocab), dtype=torch.float32, device=self.device) if logits else None
            if isinstance(bitmasks, np.ndarray):
                bitmasks = to_device(bitmasks, self.device)
            arr = (C.c_void_p * n)(*[s.handle.value for s in states])
            toks = np.ascontiguousarray(last_tokens, dtype=np.uint32)
            pos = np.ascontiguousarray(positions, dtype=np.int64)
            _check(self.lib, self.lib.dflash_propose_batch(self.handle, arr, n, toks.ctypes.data_as(C.c_void_p),
                                                           pos.ctypes.data_as(C.c_void_p), int(num_drafts),
                                                           _ptr(bitmasks), _ptr(ids), _ptr(conf), _ptr(rp),
                                                           _ptr(lg), _stream_handle(stream)))
        return {"ids": ids, "conf": conf, "row_prob": rp, "logits": lg}

    def after_verify(self, state, num_accepted):
        _check(self.lib, self.lib.dflash_after_verify(self.handle, state.handle, int(num_accepted)))

    def read_kv(self, state, layer, row0, n_rows, stream=None):
        import torch
        geo = self.geo
        dt = torch.uint8 if geo.kv_dtype == "fp8" else torch.int16
        with _on(stream):
            k = torch.empty((n_rows, geo.num_kv_heads, geo.head_dim), dtype=dt, device=self.device)
            v = torch.empty_like(k)
            _check(self.lib, self.lib.dflash_state_read_kv(self.handle, state.handle, layer, row0, n_rows, _ptr(k),
                                                           _ptr(v), _stream_handle(stream)))
        return k, v

    def read_lm_head_fp8(self, stream=None):
        import torch
        with _on(stream):
            codes = torch.empty((self.geo.vocab, self.geo.hidden), dtype=torch.uint8, device=self.device)
            scale = torch.empty(self.geo.vocab, dtype=torch.float32, device=self.device)
            _check(self.lib, self.lib.dflash_read_lm_head_fp8(self.handle, _ptr(codes), _ptr(scale),
                                                              _stream_handle(stream)))
        return codes, scale

    def take_kv(self, state):
        """Move the state's KV blocks out (carry to a later turn): (blocks
        int32 array, rows, last_pair_key), or None when there is nothing to
        carry."""
        n, rows, key = C.c_int32(), C.c_int32(), C.c_int64()
        cap = 1
        while True:
            buf = np.zeros(cap, dtype=np.int32)
            rc = self.lib.dflash_take_kv(self.handle, state.handle, buf.ctypes.data_as(C.c_void_p), cap,
                                         C.byref(n), C.byref(rows), C.byref(key))
            if rc == 0 or n.value <= cap:
                _check(self.lib, rc)
                break
            cap = n.value  # too small: retry with the count the library asked for
        if n.value == 0:
            return None
        return buf[:n.value].copy(), rows.value, key.value

    def install_kv(self, state, blocks, rows, last_pair_key=-1):
        b = np.ascontiguousarray(blocks, dtype=np.int32)
        _check(self.lib, self.lib.dflash_install_kv(self.handle, state.handle, b.ctypes.data_as(C.c_void_p), len(b),
                                                    int(rows), int(last_pair_key)))

    def free_kv(self, blocks):
        b = np.ascontiguousarray(blocks, dtype=np.int32)
        _check(self.lib, self.lib.dflash_free_kv(self.handle, b.ctypes.data_as(C.c_void_p), len(b)))

    def timing_enable(self, on=True):
        _check(self.lib, self.lib.dflash_timing_enable(self.handle, 1 if on else 0))

    def timing_read(self, phase):
        """(total milliseconds, intervals) recorded for a phase since the last read."""
        ms = C.c_double()
        n = C.c_int64()
        _check(self.lib, self.lib.dflash_timing_read(self.handle, int(phase), C.byref(ms), C.byref(n)))
        return ms.value, n.value

    def destroy(self):
        if getattr(self, "handle", None):
            self.lib.dflash_destroy(self.handle)
            self.handle = None
            self.keep = []

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
