"""ctypes wrapper around the CPU oracle (gpt2_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product library.  The oracle
shares no code with the HIP path; both are fed the same seeded input arrays.

Parameter and activation tensors are exposed as numpy views into the C
arenas, so tests can set weights and read any intermediate.
"""
import ctypes
import os

import numpy as np

from .build import LIBS, build

PARAM_NAMES = ["wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw",
               "attprojb", "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb",
               "lnfw", "lnfb"]
ACT_NAMES = ["encoded", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "preatt",
             "att", "attproj", "residual2", "ln2", "ln2_mean", "ln2_rstd", "fch",
             "fch_gelu", "fcproj", "residual3", "lnf", "lnf_mean", "lnf_rstd",
             "logits", "probs", "losses"]

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p


class OracleConfig(ctypes.Structure):
    _fields_ = [("max_seq_len", _int), ("vocab_size", _int),
                ("num_layers", _int), ("num_heads", _int), ("channels", _int),
                ("rope", _int)]


_loaded = {}


def _lib(precision: str):
    if precision in _loaded:
        return _loaded[precision]
    path = LIBS[precision]
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    real = ctypes.c_float if precision == "f32" else ctypes.c_double
    assert lib.oracle_real_size() == ctypes.sizeof(real)
    lib.oracle_param_sizes.restype = _i64
    lib.oracle_param_sizes.argtypes = [ctypes.POINTER(OracleConfig), _vp]
    lib.oracle_act_sizes.restype = _i64
    lib.oracle_act_sizes.argtypes = [ctypes.POINTER(OracleConfig), _int, _int, _vp]
    lib.oracle_create.restype = _vp
    lib.oracle_create.argtypes = [ctypes.POINTER(OracleConfig), _int, _int]
    lib.oracle_destroy.argtypes = [_vp]
    for fn in ("oracle_params", "oracle_grads", "oracle_adam_m", "oracle_adam_v",
               "oracle_acts", "oracle_act_grads"):
        getattr(lib, fn).restype = _vp
        getattr(lib, fn).argtypes = [_vp]
    lib.oracle_num_params.restype = _i64
    lib.oracle_num_params.argtypes = [_vp]
    lib.oracle_num_acts.restype = _i64
    lib.oracle_num_acts.argtypes = [_vp]
    lib.oracle_forward.restype = ctypes.c_double
    lib.oracle_forward.argtypes = [_vp, _vp, _vp]
    lib.oracle_zero_grad.argtypes = [_vp]
    lib.oracle_backward.restype = _int
    lib.oracle_backward.argtypes = [_vp]
    lib.oracle_update.argtypes = [_vp] + [ctypes.c_double] * 5 + [_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [_int]
    lib.oracle_loss_scale_step.restype = _int
    lib.oracle_loss_scale_step.argtypes = [_vp, _vp, _int, _int, ctypes.c_double]
    lib.oracle_sample.restype = _int
    lib.oracle_sample.argtypes = [_vp, _int, ctypes.c_double]
    lib.oracle_generate.restype = _int
    lib.oracle_generate.argtypes = [_vp, _vp, _int, _int, _vp]
    # layer primitives: pointers are passed as void*, sizes as int / int64
    sig = {
        "oracle_encoder_forward": [_vp, _vp, _vp, _vp, _int, _int, _int],
        "oracle_encoder_backward": [_vp, _vp, _vp, _vp, _int, _int, _int],
        "oracle_layernorm_forward": [_vp] * 6 + [_int, _int],
        "oracle_layernorm_backward": [_vp] * 8 + [_int, _int],
        "oracle_matmul_forward": [_vp] * 4 + [_int, _int, _int],
        "oracle_matmul_backward": [_vp] * 6 + [_int, _int, _int],
        "oracle_attention_forward": [_vp] * 4 + [_int] * 4,
        "oracle_attention_backward": [_vp] * 6 + [_int] * 4,
        "oracle_gelu_forward": [_vp, _vp, _i64],
        "oracle_gelu_backward": [_vp, _vp, _vp, _i64],
        "oracle_residual_forward": [_vp, _vp, _vp, _i64],
        "oracle_residual_backward": [_vp, _vp, _vp, _i64],
        "oracle_softmax_forward": [_vp, _vp, _int, _int],
        "oracle_crossentropy_forward": [_vp, _vp, _vp, _int, _int],
        "oracle_crossentropy_softmax_backward": [_vp] * 4 + [_int, _int],
        "oracle_adamw": [_vp] * 4 + [_i64] + [real] * 5 + [_int],
        "oracle_rope_forward": [_vp] + [_int] * 4,
        "oracle_rope_backward": [_vp] + [_int] * 4,
    }
    for name, args in sig.items():
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = None
    lib.real = real
    lib.dtype = np.float32 if precision == "f32" else np.float64
    _loaded[precision] = lib
    return lib


def lib(precision: str = "f32"):
    """The loaded oracle library ("f32" or "f64")."""
    return _lib(precision)


def ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_vp)


def make_config(L, C, NH, V, maxT, rope=0) -> OracleConfig:
    return OracleConfig(max_seq_len=maxT, vocab_size=V, num_layers=L,
                        num_heads=NH, channels=C, rope=int(rope))


def param_sizes(L, C, NH, V, maxT, rope=0):
    cfg = make_config(L, C, NH, V, maxT, rope)
    sizes = np.zeros(16, dtype=np.int64)
    total = _lib("f32").oracle_param_sizes(ctypes.byref(cfg), ptr(sizes))
    return dict(zip(PARAM_NAMES, sizes.tolist())), int(total)


def act_sizes(L, C, NH, V, maxT, B, T):
    cfg = make_config(L, C, NH, V, maxT)
    sizes = np.zeros(23, dtype=np.int64)
    total = _lib("f32").oracle_act_sizes(ctypes.byref(cfg), B, T, ptr(sizes))
    return dict(zip(ACT_NAMES, sizes.tolist())), int(total)


class OracleModel:
    """One GPT-2 with its four parameter arenas and two activation arenas."""

    def __init__(self, L, C, NH, V, maxT, B, T, precision="f32", rope=0):
        self.lib = _lib(precision)
        self.dtype = self.lib.dtype
        self.L, self.C, self.NH, self.V, self.maxT = L, C, NH, V, maxT
        self.B, self.T = B, T
        self._cfg = make_config(L, C, NH, V, maxT, rope)
        self.rope = int(rope)
        h = self.lib.oracle_create(ctypes.byref(self._cfg), B, T)
        if not h:
            raise MemoryError("oracle_create failed (bad config or no memory)")
        self.h = h
        self.num_params = int(self.lib.oracle_num_params(h))
        self.num_acts = int(self.lib.oracle_num_acts(h))
        self.param_sizes, _ = param_sizes(L, C, NH, V, maxT, rope)
        self.act_sizes, _ = act_sizes(L, C, NH, V, maxT, B, T)

        def view(fn, n):
            addr = getattr(self.lib, fn)(h)
            buf = (self.lib.real * n).from_address(addr)
            return np.frombuffer(buf, dtype=self.dtype, count=n)

        self.params = view("oracle_params", self.num_params)
        self.grads = view("oracle_grads", self.num_params)
        self.m = view("oracle_adam_m", self.num_params)
        self.v = view("oracle_adam_v", self.num_params)
        self.acts = view("oracle_acts", self.num_acts)
        self.act_grads = view("oracle_act_grads", self.num_acts)

    def close(self):
        if getattr(self, "h", None):
            self.lib.oracle_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    # --- named tensor views -------------------------------------------------
    def _split(self, arena, sizes, names, name):
        off = 0
        for n in names:
            if n == name:
                return arena[off:off + sizes[n]]
            off += sizes[n]
        raise KeyError(name)

    def param(self, name):
        return self._split(self.params, self.param_sizes, PARAM_NAMES, name)

    def grad(self, name):
        return self._split(self.grads, self.param_sizes, PARAM_NAMES, name)

    def act(self, name):
        return self._split(self.acts, self.act_sizes, ACT_NAMES, name)

    def act_grad(self, name):
        return self._split(self.act_grads, self.act_sizes, ACT_NAMES, name)

    # --- the step -----------------------------------------------------------
    def forward(self, tokens, targets=None) -> float:
        tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        assert tok.size == self.B * self.T
        tgt = None
        if targets is not None:
            tgt = np.ascontiguousarray(targets, dtype=np.int32).reshape(-1)
            assert tgt.size == self.B * self.T
        self._tok, self._tgt = tok, tgt  # keep alive across the call
        return float(self.lib.oracle_forward(
            self.h, ptr(tok), ptr(tgt) if tgt is not None else None))

    def zero_grad(self):
        self.lib.oracle_zero_grad(self.h)

    def backward(self):
        if self.lib.oracle_backward(self.h) != 0:
            raise RuntimeError("oracle backward needs a forward with targets")

    def update(self, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8,
               weight_decay=0.0, step=1):
        self.lib.oracle_update(self.h, lr, beta1, beta2, eps, weight_decay, step)

    def generate(self, prompt, n, coins):
        """B = 1 model: tokens 0..n-1, the prompt then n - len(prompt) draws
        (the model's T positions are run each step; n <= T)."""
        tok = np.zeros(self.T, dtype=np.int32)
        tok[:len(prompt)] = prompt
        c = np.ascontiguousarray(coins, dtype=np.float64)
        if self.lib.oracle_generate(self.h, ptr(tok), len(prompt), n, ptr(c)) != 0:
            raise ValueError("oracle_generate: bad arguments")
        return tok[:n].copy()


def sample(probs, coin, precision="f32"):
    """Inverse-CDF draw from one probability row (oracle_sample)."""
    lb = _lib(precision)
    p = np.ascontiguousarray(probs, dtype=lb.dtype)
    return int(lb.oracle_sample(ptr(p), p.size, float(coin)))


def loss_scale_schedule(scale, found_inf_seq, interval, min_scale=1.0):
    """Runs oracle_loss_scale_step over a sequence of overflow flags; returns
    [(applied, scale after the step)] per step."""
    lb = _lib("f32")
    sc = np.array([scale], dtype=np.float64)
    good = np.zeros(1, dtype=np.int32)
    out = []
    for f in found_inf_seq:
        a = lb.oracle_loss_scale_step(ptr(sc), ptr(good), int(bool(f)), interval, min_scale)
        out.append((bool(a), float(sc[0])))
    return out
