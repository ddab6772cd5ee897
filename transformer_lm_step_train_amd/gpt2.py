"""ctypes binding of libgpt2_hip.so (the C ABI declared in include/gpt2.h).

The functions keep the C names and only marshal arguments.  `Model` is a
small convenience owner of one handle.  PyTorch, when used, only supplies the
device memory (its caching allocator, through the allocator callback) and the
stream; every step of the computation runs in the library's HIP kernels.

Importing this module fails loudly if the library has not been built.
"""
import ctypes
import os

import numpy as np
# torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
# Loading torch first makes the library bind to that one runtime instead of
# pulling a second copy from /opt/rocm into the process.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2_hip.so")

GPT2_OK, GPT2_EINVAL, GPT2_ERANGE, GPT2_ESTATE, GPT2_ENOMEM, GPT2_EDEVICE = 0, -1, -2, -3, -4, -5
GPT2_ECORRUPT = -6
GPT2_FP32, GPT2_BF16_MIXED, GPT2_F16_MIXED = 0, 1, 2
KC_GEMM, KC_ATTENTION, KC_LAYERNORM, KC_SOFTMAX_CE, KC_ADAMW, KC_OTHER = range(6)
KC_NAMES = ["gemm", "attention", "layernorm", "softmax_ce", "adamw", "other"]

PARAM_NAMES = ["wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw",
               "attprojb", "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb",
               "lnfw", "lnfb"]

_c = ctypes
_vp = _c.c_void_p
_i32 = _c.c_int32
_i64 = _c.c_int64


class gpt2_config(_c.Structure):
    _fields_ = [("max_seq_len", _i32), ("vocab_size", _i32), ("num_layers", _i32),
                ("num_heads", _i32), ("channels", _i32), ("batch_size", _i32),
                ("seq_len", _i32), ("precision", _i32), ("rope", _i32),
                ("attn_recompute", _i32)]


ALLOC_FN = _c.CFUNCTYPE(_vp, _c.c_size_t, _vp)
FREE_FN = _c.CFUNCTYPE(None, _vp, _vp)


class gpt2_allocator(_c.Structure):
    _fields_ = [("alloc", ALLOC_FN), ("free", FREE_FN), ("ctx", _vp)]


class GPT2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"gpt2 error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import "
            f"__graft_entry__ as g; g.build()')")
    lib = _c.CDLL(LIB_PATH)
    P = _c.POINTER
    sig = {
        "gpt2_validate_config": (_c.c_int, [P(gpt2_config)]),
        "gpt2_config_num_parameters": (_i64, [P(gpt2_config)]),
        "gpt2_config_param_tensor": (_c.c_int, [P(gpt2_config), _c.c_int,
                                                P(_c.c_char_p), P(_i64), P(_i64)]),
        "gpt2_config_device_bytes": (_i64, [P(gpt2_config)]),
        "gpt2_create": (_c.c_int, [P(gpt2_config), P(gpt2_allocator), _vp, P(_vp)]),
        "gpt2_destroy": (None, [_vp]),
        "gpt2_num_parameters": (_i64, [_vp]),
        "gpt2_param_tensor": (_c.c_int, [_vp, _c.c_int, P(_c.c_char_p), P(_i64), P(_i64)]),
        "gpt2_copy_params": (_c.c_int, [_vp, _vp, _vp]),
        "gpt2_copy_grads": (_c.c_int, [_vp, _vp]),
        "gpt2_copy_opt_state": (_c.c_int, [_vp, _vp, _vp]),
        "gpt2_save_checkpoint": (_c.c_int, [_vp, _c.c_char_p, _i64]),
        "gpt2_load_checkpoint": (_c.c_int, [_vp, _c.c_char_p, P(_i64)]),
        "gpt2_copy_activation": (_c.c_int, [_vp, _c.c_char_p, _c.c_int, _vp, P(_i64)]),
        "gpt2_forward": (_c.c_int, [_vp, _vp, _vp, _c.c_int, _c.c_int, P(_c.c_float)]),
        "gpt2_forward_device": (_c.c_int, [_vp, _vp, _vp, _c.c_int, _c.c_int,
                                           P(_c.c_float)]),
        "gpt2_evaluate": (_c.c_int, [_vp, _vp, _vp, _c.c_int, _c.c_int, P(_c.c_float)]),
        "gpt2_sample": (_c.c_int, [_vp, _c.c_int, _c.c_int, _c.c_float, P(_c.c_int32)]),
        "gpt2_generate": (_c.c_int, [_vp, _vp, _c.c_int, _c.c_int, _vp]),
        "gpt2_loader_open": (_c.c_int, [_c.c_char_p, _c.c_int, _c.c_int, P(_vp)]),
        "gpt2_loader_num_tokens": (_i64, [_vp]),
        "gpt2_loader_num_batches": (_i64, [_vp]),
        "gpt2_loader_next": (_c.c_int, [_vp, _vp, _vp]),
        "gpt2_loader_reset": (_c.c_int, [_vp]),
        "gpt2_loader_close": (None, [_vp]),
        "gpt2_set_loss_scale": (_c.c_int, [_vp, _c.c_float, _c.c_int]),
        "gpt2_get_loss_scale": (_c.c_int, [_vp, P(_c.c_float), P(_c.c_int)]),
        "gpt2_cross_entropy_static": (_c.c_int, [_vp, _i64, _vp, _c.c_int, _c.c_int, _c.c_int,
                                                 _c.c_float, _vp, _vp, _vp]),
        "gpt2_zero_grad": (_c.c_int, [_vp]),
        "gpt2_backward": (_c.c_int, [_vp]),
        "gpt2_update": (_c.c_int, [_vp] + [_c.c_float] * 5 + [_c.c_int]),
        "gpt2_synchronize": (_c.c_int, [_vp]),
        "gpt2_check_guards": (_c.c_int, [_vp]),
        "gpt2_last_error": (_c.c_char_p, []),
        "gpt2_profile": (_c.c_int, [_vp, _c.c_int]),
        "gpt2_profile_read": (_c.c_int, [_vp, _c.c_int, P(_c.c_double), P(_i64),
                                         P(_c.c_double), P(_c.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def gpt2_last_error() -> str:
    return lib.gpt2_last_error().decode()


def _check(rc):
    if rc != GPT2_OK:
        raise GPT2Error(rc, gpt2_last_error())
    return rc


def make_config(L, C, NH, V, maxT, B, T, precision=GPT2_FP32, rope=0,
                attn_recompute=0) -> gpt2_config:
    return gpt2_config(max_seq_len=maxT, vocab_size=V, num_layers=L, num_heads=NH,
                       channels=C, batch_size=B, seq_len=T, precision=precision,
                       rope=int(rope), attn_recompute=int(attn_recompute))


# ---- the C ABI, one function each ------------------------------------------

def gpt2_validate_config(cfg) -> int:
    return lib.gpt2_validate_config(_c.byref(cfg))


def gpt2_config_num_parameters(cfg) -> int:
    return lib.gpt2_config_num_parameters(_c.byref(cfg))


def gpt2_config_param_tensor(cfg, i):
    name, off, n = _c.c_char_p(), _i64(), _i64()
    _check(lib.gpt2_config_param_tensor(_c.byref(cfg), i, _c.byref(name), _c.byref(off),
                                        _c.byref(n)))
    return name.value.decode(), off.value, n.value


def gpt2_save_checkpoint(h, path, step):
    _check(lib.gpt2_save_checkpoint(h, os.fsencode(path), step))


def gpt2_load_checkpoint(h, path) -> int:
    step = _i64()
    _check(lib.gpt2_load_checkpoint(h, os.fsencode(path), _c.byref(step)))
    return step.value


def gpt2_config_device_bytes(cfg) -> int:
    return lib.gpt2_config_device_bytes(_c.byref(cfg))


def gpt2_create(cfg, allocator=None, stream=None):
    h = _vp()
    _check(lib.gpt2_create(_c.byref(cfg), _c.byref(allocator) if allocator else None,
                           stream, _c.byref(h)))
    return h


def gpt2_destroy(h):
    lib.gpt2_destroy(h)


def gpt2_num_parameters(h) -> int:
    return lib.gpt2_num_parameters(h)


def gpt2_param_tensor(h, i):
    name, off, n = _c.c_char_p(), _i64(), _i64()
    _check(lib.gpt2_param_tensor(h, i, _c.byref(name), _c.byref(off), _c.byref(n)))
    return name.value.decode(), off.value, n.value


def _f32(a):
    assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_vp)


def gpt2_copy_params(h, host_dst=None, host_src=None):
    _check(lib.gpt2_copy_params(h, _f32(host_dst) if host_dst is not None else None,
                                _f32(host_src) if host_src is not None else None))


def gpt2_copy_grads(h, host_dst):
    _check(lib.gpt2_copy_grads(h, _f32(host_dst)))


def gpt2_copy_opt_state(h, host_m=None, host_v=None):
    _check(lib.gpt2_copy_opt_state(h, _f32(host_m) if host_m is not None else None,
                                   _f32(host_v) if host_v is not None else None))


def gpt2_copy_activation(h, name, layer=0, host_dst=None) -> int:
    n = _i64()
    _check(lib.gpt2_copy_activation(h, name.encode(), layer,
                                    _f32(host_dst) if host_dst is not None else None,
                                    _c.byref(n)))
    return n.value


def _i32p(a):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_vp)


def gpt2_forward(h, tokens, targets, B, T, want_loss=True):
    loss = _c.c_float(float("nan"))
    _check(lib.gpt2_forward(h, _i32p(tokens), _i32p(targets), B, T,
                            _c.byref(loss) if want_loss else None))
    return loss.value


def gpt2_forward_device(h, tokens_ptr, targets_ptr, B, T, want_loss=True):
    loss = _c.c_float(float("nan"))
    _check(lib.gpt2_forward_device(h, tokens_ptr, targets_ptr, B, T,
                                   _c.byref(loss) if want_loss else None))
    return loss.value


def gpt2_evaluate(h, tokens, targets, B, T):
    loss = _c.c_float(float("nan"))
    _check(lib.gpt2_evaluate(h, _i32p(tokens), _i32p(targets), B, T, _c.byref(loss)))
    return loss.value


def gpt2_cross_entropy_static(logits_ptr, ldv, targets_ptr, N, V, precision, grad_scale,
                              mean_loss_ptr, flag_ptr, stream=None):
    """Device pointers in, device outputs written; nothing allocated."""
    _check(lib.gpt2_cross_entropy_static(logits_ptr, ldv, targets_ptr, N, V, precision,
                                         grad_scale, mean_loss_ptr, flag_ptr, stream))


def gpt2_sample(h, b, t, coin):
    tok = _c.c_int32(-1)
    _check(lib.gpt2_sample(h, b, t, coin, _c.byref(tok)))
    return tok.value


def gpt2_generate(h, tokens, prompt_len, n, coins):
    """tokens: int32 array of length >= n (filled in place from prompt_len);
    coins: float32 array of n - prompt_len uniforms in [0, 1)."""
    assert coins is None or (coins.dtype == np.float32 and coins.flags["C_CONTIGUOUS"])
    _check(lib.gpt2_generate(h, _i32p(tokens), prompt_len, n,
                             None if coins is None else coins.ctypes.data_as(_vp)))


class Loader:
    """Batches of a raw int32 token file (gpt2_loader_*): next() returns
    (tokens, targets) as (B, T) int32 arrays."""

    def __init__(self, path, B, T):
        h = _vp()
        _check(lib.gpt2_loader_open(os.fsencode(path), B, T, _c.byref(h)))
        self.h, self.B, self.T = h, B, T
        self.num_tokens = int(lib.gpt2_loader_num_tokens(h))
        self.num_batches = int(lib.gpt2_loader_num_batches(h))

    def next(self):
        tok = np.empty((self.B, self.T), dtype=np.int32)
        tgt = np.empty((self.B, self.T), dtype=np.int32)
        _check(lib.gpt2_loader_next(self.h, tok.ctypes.data_as(_vp), tgt.ctypes.data_as(_vp)))
        return tok, tgt

    def reset(self):
        _check(lib.gpt2_loader_reset(self.h))

    def close(self):
        if getattr(self, "h", None):
            lib.gpt2_loader_close(self.h)
            self.h = None

    def __del__(self):
        self.close()


def gpt2_zero_grad(h):
    _check(lib.gpt2_zero_grad(h))


def gpt2_backward(h):
    _check(lib.gpt2_backward(h))


def gpt2_update(h, lr, beta1, beta2, eps, weight_decay, step):
    _check(lib.gpt2_update(h, lr, beta1, beta2, eps, weight_decay, step))


def gpt2_synchronize(h):
    _check(lib.gpt2_synchronize(h))


GPT2_PROFILE_ALL = (1 << len(KC_NAMES)) - 1


def gpt2_profile(h, enable):
    """enable: False/0 stops; True times every class; an int is a class mask."""
    mask = GPT2_PROFILE_ALL if enable is True else int(enable)
    _check(lib.gpt2_profile(h, mask))


def gpt2_profile_read(h, kernel_class):
    ms, n, fl, by = _c.c_double(), _i64(), _c.c_double(), _c.c_double()
    _check(lib.gpt2_profile_read(h, kernel_class, _c.byref(ms), _c.byref(n), _c.byref(fl),
                                 _c.byref(by)))
    return dict(ms=ms.value, launches=n.value, flops=fl.value, bytes=by.value)


# ---- convenience owner ------------------------------------------------------

class TorchAllocator:
    """Device memory from torch's caching allocator, on torch's current stream."""

    def __init__(self):
        import torch
        self._torch = torch
        self._alloc = ALLOC_FN(self._do_alloc)
        self._free = FREE_FN(self._do_free)
        self.struct = gpt2_allocator(alloc=self._alloc, free=self._free, ctx=None)

    def _do_alloc(self, nbytes, ctx):
        try:
            return self._torch.cuda.caching_allocator_alloc(int(nbytes))
        except Exception:  # out of memory: report NULL to the library
            return None

    def _do_free(self, ptr, ctx):
        self._torch.cuda.caching_allocator_delete(ptr)


class Model:
    """One model handle.  With torch=True (default) device memory comes from
    torch's caching allocator and work runs on torch's current stream."""

    def __init__(self, L, C, NH, V, maxT, B, T, precision=GPT2_FP32, torch=True, rope=False,
                 attn_recompute=False):
        self.cfg = make_config(L, C, NH, V, maxT, B, T, precision, rope, attn_recompute)
        self.rope = bool(rope)
        self.L, self.C, self.NH, self.V, self.maxT, self.B, self.T = L, C, NH, V, maxT, B, T
        self._allocator = None
        stream = None
        if torch:
            import torch as _t
            self._allocator = TorchAllocator()
            stream = _t.cuda.current_stream().cuda_stream
        self.h = gpt2_create(self.cfg, self._allocator.struct if self._allocator else None,
                             stream)
        self.num_params = gpt2_num_parameters(self.h)
        self.tensors = {}
        for i in range(16):
            name, off, n = gpt2_param_tensor(self.h, i)
            self.tensors[name] = (off, n)

    def close(self):
        if getattr(self, "h", None):
            gpt2_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    def set_params(self, flat):
        flat = np.ascontiguousarray(flat, dtype=np.float32)
        assert flat.size == self.num_params
        gpt2_copy_params(self.h, host_src=flat)

    def params(self):
        out = np.empty(self.num_params, dtype=np.float32)
        gpt2_copy_params(self.h, host_dst=out)
        return out

    def grads(self):
        out = np.empty(self.num_params, dtype=np.float32)
        gpt2_copy_grads(self.h, out)
        return out

    def opt_state(self):
        m = np.empty(self.num_params, dtype=np.float32)
        v = np.empty(self.num_params, dtype=np.float32)
        gpt2_copy_opt_state(self.h, m, v)
        return m, v

    def save_checkpoint(self, path, step):
        """Parameters, AdamW moments and the step counter to one file."""
        gpt2_save_checkpoint(self.h, path, step)

    def load_checkpoint(self, path):
        """Restores a save_checkpoint file; returns its step counter."""
        return gpt2_load_checkpoint(self.h, path)

    def activation(self, name, layer=0):
        n = gpt2_copy_activation(self.h, name, layer)
        out = np.empty(n, dtype=np.float32)
        gpt2_copy_activation(self.h, name, layer, out)
        return out

    def forward(self, tokens, targets=None):
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        B, T = tok.shape
        tgt = None if targets is None else np.ascontiguousarray(targets, dtype=np.int32)
        return gpt2_forward(self.h, tok, tgt, B, T)

    def evaluate(self, tokens, targets):
        """Mean loss without gradient or backward state (the logits stay)."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        B, T = tok.shape
        return gpt2_evaluate(self.h, tok, np.ascontiguousarray(targets, dtype=np.int32), B, T)

    def forward_device(self, tokens, targets=None, want_loss=True):
        """tokens / targets: int32 device tensors of shape (B, T)."""
        B, T = tokens.shape
        return gpt2_forward_device(self.h, tokens.data_ptr(),
                                   None if targets is None else targets.data_ptr(), B, T,
                                   want_loss)

    def sample(self, b, t, coin):
        return gpt2_sample(self.h, b, t, coin)

    def generate(self, prompt, n, coins):
        """Tokens 0..n-1: the prompt, then n - len(prompt) draws."""
        tok = np.zeros(n, dtype=np.int32)
        tok[:len(prompt)] = prompt
        c = np.ascontiguousarray(coins, dtype=np.float32)
        gpt2_generate(self.h, tok, len(prompt), n, c)
        return tok

    def set_loss_scale(self, scale, growth_interval=2000):
        _check(lib.gpt2_set_loss_scale(self.h, scale, growth_interval))

    def loss_scale(self):
        """(scale, last update skipped) of the fp16 model."""
        sc, sk = _c.c_float(0.0), _c.c_int(0)
        _check(lib.gpt2_get_loss_scale(self.h, _c.byref(sc), _c.byref(sk)))
        return sc.value, bool(sk.value)

    def zero_grad(self):
        gpt2_zero_grad(self.h)

    def backward(self):
        gpt2_backward(self.h)

    def update(self, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1):
        gpt2_update(self.h, lr, beta1, beta2, eps, weight_decay, step)

    def synchronize(self):
        gpt2_synchronize(self.h)

    def check_guards(self):
        """Raises GPT2Error (GPT2_ECORRUPT) if a debug guard word changed."""
        _check(lib.gpt2_check_guards(self.h))

    def step(self, tokens, targets, step, **adamw):
        loss = self.forward(tokens, targets)
        self.zero_grad()
        self.backward()
        self.update(step=step, **adamw)
        return loss
