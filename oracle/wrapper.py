"""ctypes wrapper and build step for the CPU oracle (test infrastructure only)."""
import ctypes as ct
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gpt2_oracle.c")
_LIBS = {}


# builds: the double-precision parity reference, a portable float build, and
# the float build for timing on the host it runs on (-march=native, no fast
# math, no contraction: the same arithmetic, vectorised where the compiler may)
BUILDS = {"f64": ("double", []), "f32": ("float", []), "f32n": ("float", ["-march=native"])}


def lib_path(precision="f64"):
    return os.path.join(HERE, f"liboracle_{precision}.so")


def build(force=True, precisions=("f64", "f32")):
    """Compile the oracle builds named in `precisions` (keys of BUILDS)."""
    for prec in precisions:
        real, extra = BUILDS[prec]
        out = lib_path(prec)
        if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
            continue
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
               "-shared", f"-DREAL={real}", "-Wall", "-Wno-unknown-pragmas"] + extra
        tmp = out + ".tmp"
        subprocess.run(cmd + [SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)


class _Cfg(ct.Structure):
    _fields_ = [(n, ct.c_int) for n in ("V", "Vp", "maxT", "C", "L", "NH", "B", "T")]


def load(precision="f64"):
    if precision in _LIBS:
        return _LIBS[precision]
    path = lib_path(precision)
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        build(force=False, precisions=(precision,))
    lib = ct.CDLL(path)
    real = ct.c_double if lib.oracle_real_bytes() == 8 else ct.c_float
    lib._real = real
    P = ct.c_void_p
    R = ct.POINTER(real)
    I = ct.POINTER(ct.c_int)
    D = ct.POINTER(ct.c_double)
    sig = {
        "oracle_create": (P, [ct.POINTER(_Cfg), ct.POINTER(ct.c_float)]),
        "oracle_free": (None, [P]),
        "oracle_num_params": (ct.c_int64, [ct.POINTER(_Cfg)]),
        "oracle_forward": (ct.c_int, [P, I, I, D]),
        "oracle_backward": (ct.c_int, [P]),
        "oracle_update": (None, [P, ct.c_double, ct.c_double, ct.c_double, ct.c_double,
                                 ct.c_double, ct.c_int]),
        "oracle_n_params": (ct.c_int64, [P]),
        "oracle_get_params": (None, [P, D]),
        "oracle_get_grads": (None, [P, D]),
        "oracle_get_m": (None, [P, D]),
        "oracle_get_v": (None, [P, D]),
        "oracle_set_params": (None, [P, D]),
        "oracle_act_size": (ct.c_int64, [P, ct.c_char_p]),
        "oracle_get_act": (ct.c_int, [P, ct.c_char_p, ct.c_int, D]),
        "oracle_fd_grads": (ct.c_int, [ct.POINTER(_Cfg), ct.POINTER(ct.c_float), I, I,
                                       ct.c_double, ct.c_int64, ct.c_int64, D]),
        "oracle_set_threads": (None, [ct.c_int]),
        "oracle_get_threads": (ct.c_int, []),
        "oracle_encoder_forward": (None, [R, I, R, R, ct.c_int, ct.c_int, ct.c_int]),
        "oracle_encoder_backward": (None, [R, R, R, I, ct.c_int, ct.c_int, ct.c_int]),
        "oracle_layernorm_forward": (None, [R, R, R, R, R, R, ct.c_int, ct.c_int]),
        "oracle_layernorm_backward": (None, [R, R, R, R, R, R, R, R, ct.c_int, ct.c_int]),
        "oracle_matmul_forward": (None, [R, R, R, R, ct.c_int, ct.c_int, ct.c_int]),
        "oracle_matmul_backward": (None, [R, R, R, R, R, R, ct.c_int, ct.c_int, ct.c_int]),
        "oracle_attention_forward": (None, [R, R, R, ct.c_int, ct.c_int, ct.c_int, ct.c_int]),
        "oracle_attention_backward": (None, [R, R, R, R, ct.c_int, ct.c_int, ct.c_int,
                                             ct.c_int]),
        "oracle_gelu_forward": (None, [R, R, ct.c_int64]),
        "oracle_gelu_backward": (None, [R, R, R, ct.c_int64]),
        "oracle_residual_forward": (None, [R, R, R, ct.c_int64]),
        "oracle_residual_backward": (None, [R, R, R, ct.c_int64]),
        "oracle_softmax_forward": (None, [R, R, ct.c_int, ct.c_int, ct.c_int]),
        "oracle_crossentropy_forward": (None, [R, R, I, ct.c_int, ct.c_int]),
        "oracle_crossentropy_softmax_backward": (None, [R, R, I, real, ct.c_int, ct.c_int,
                                                        ct.c_int]),
        "oracle_adamw": (None, [R, R, R, R, ct.c_int64, real, real, real, real, real,
                                ct.c_int]),
        "oracle_adamw_scaled": (None, [R, R, R, R, ct.c_int64, real, real, real, real, real,
                                       ct.c_int, real]),
        "oracle_grad_norm": (real, [R, ct.c_int64]),
        "oracle_e4m3_decode": (ct.c_double, [ct.c_int]),
        "oracle_e4m3_encode": (ct.c_int, [ct.c_float]),
        "oracle_fp8_scale": (ct.c_float, [ct.c_float]),
        "oracle_fp8_amax": (ct.c_float, [ct.POINTER(ct.c_float), ct.c_int64]),
        "oracle_fp8_quantize": (None, [ct.POINTER(ct.c_ubyte), ct.POINTER(ct.c_float),
                                       ct.c_int64, ct.c_float]),
        "oracle_fp8_matmul": (None, [D, ct.POINTER(ct.c_ubyte), ct.POINTER(ct.c_ubyte), D,
                                     ct.c_int, ct.c_int, ct.c_int, ct.c_float, ct.c_float]),
        "oracle_lr_schedule": (ct.c_double, [ct.c_double, ct.c_double, ct.c_int, ct.c_int,
                                             ct.c_int]),
        "oracle_update_scheduled": (ct.c_double, [P, ct.c_double, ct.c_double, ct.c_int,
                                                  ct.c_int, ct.c_double, ct.c_double,
                                                  ct.c_double, ct.c_double, ct.c_double,
                                                  ct.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIBS[precision] = lib
    return lib


def real_dtype(lib):
    return np.float64 if lib._real is ct.c_double else np.float32


def ptr(a, ctype):
    """Pointer to a C-contiguous numpy array (None passes through as NULL)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ct.POINTER(ctype))


def cfg_struct(w):
    return _Cfg(w.V, w.Vp, w.max_T, w.C, w.L, w.NH, w.B, w.T)


class Oracle:
    """One oracle model: `forward`, `backward`, `update` as the GPU step has them."""

    def __init__(self, w, params, precision="f64", threads=None):
        self.lib = load(precision)
        if threads:
            self.lib.oracle_set_threads(int(threads))
        self.w = w
        self.cfg = cfg_struct(w)
        params = np.ascontiguousarray(params, dtype=np.float32)
        assert params.size == w.num_params()
        self.h = self.lib.oracle_create(ct.byref(self.cfg), ptr(params, ct.c_float))
        if not self.h:
            raise ValueError("oracle rejected the configuration")
        self.n = self.lib.oracle_n_params(self.h)

    def close(self):
        if self.h:
            self.lib.oracle_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, inputs, targets=None):
        inputs = np.ascontiguousarray(inputs, dtype=np.int32)
        tg = None if targets is None else np.ascontiguousarray(targets, dtype=np.int32)
        loss = ct.c_double(float("nan"))
        rc = self.lib.oracle_forward(self.h, ptr(inputs, ct.c_int), ptr(tg, ct.c_int),
                                     ct.byref(loss))
        if rc != 0:
            raise ValueError("token id outside [0, V)")
        return loss.value if targets is not None else None

    def backward(self):
        if self.lib.oracle_backward(self.h) != 0:
            raise RuntimeError("backward needs a forward with targets")

    def update(self, lr, beta1, beta2, eps, wd, t):
        self.lib.oracle_update(self.h, lr, beta1, beta2, eps, wd, int(t))

    def update_scheduled(self, lr_max, lr_min, warmup, total, beta1, beta2, eps, wd, grad_clip,
                         t):
        """Scheduled (and, with grad_clip > 0, clipped) AdamW step; returns
        the global gradient norm (0 without clipping)."""
        return self.lib.oracle_update_scheduled(self.h, lr_max, lr_min, int(warmup), int(total),
                                                beta1, beta2, eps, wd, grad_clip, int(t))

    def _get(self, fn):
        out = np.empty(self.n, np.float64)
        fn(self.h, ptr(out, ct.c_double))
        return out

    def params(self):
        return self._get(self.lib.oracle_get_params)

    def grads(self):
        return self._get(self.lib.oracle_get_grads)

    def m(self):
        return self._get(self.lib.oracle_get_m)

    def v(self):
        return self._get(self.lib.oracle_get_v)

    def set_params(self, p):
        p = np.ascontiguousarray(p, dtype=np.float64)
        self.lib.oracle_set_params(self.h, ptr(p, ct.c_double))

    def act(self, name, grad=False):
        n = self.lib.oracle_act_size(self.h, name.encode())
        if n < 0:
            raise KeyError(name)
        out = np.empty(n, np.float64)
        if self.lib.oracle_get_act(self.h, name.encode(), int(grad), ptr(out, ct.c_double)):
            raise KeyError(name)
        return out


def fd_grads(w, params, inputs, targets, h=1e-5, start=0, count=None, precision="f64",
             threads=None):
    """Central finite-difference gradient of the mean loss, parameters
    [start, start+count)."""
    lib = load(precision)
    if threads:
        lib.oracle_set_threads(int(threads))
    n = w.num_params()
    count = n - start if count is None else count
    params = np.ascontiguousarray(params, dtype=np.float32)
    inputs = np.ascontiguousarray(inputs, dtype=np.int32)
    targets = np.ascontiguousarray(targets, dtype=np.int32)
    out = np.empty(count, np.float64)
    cfg = cfg_struct(w)
    rc = lib.oracle_fd_grads(ct.byref(cfg), ptr(params, ct.c_float), ptr(inputs, ct.c_int),
                             ptr(targets, ct.c_int), h, start, count, ptr(out, ct.c_double))
    if rc:
        raise ValueError("token id outside [0, V)")
    return out


# ---- FP8 (E4M3) products: the oracle's functions over numpy arrays ----------

def e4m3_decode(codes):
    """Values (float64) of E4M3 codes (any integer array)."""
    lib = load()
    return np.array([lib.oracle_e4m3_decode(int(c)) for c in np.ravel(codes)]).reshape(
        np.shape(codes))


def e4m3_encode(x):
    """E4M3 codes (uint8) of float32 values, one at a time."""
    lib = load()
    x = np.asarray(x, np.float32)
    return np.array([lib.oracle_e4m3_encode(float(v)) for v in np.ravel(x)],
                    np.uint8).reshape(x.shape)


def fp8_amax(x):
    lib = load()
    x = np.ascontiguousarray(x, np.float32).ravel()
    return lib.oracle_fp8_amax(ptr(x, ct.c_float), x.size)


def fp8_scale(amax):
    return load().oracle_fp8_scale(float(amax))


def fp8_quantize(x, s):
    """E4M3(x * s) codes, the product rounded to fp32."""
    lib = load()
    x = np.ascontiguousarray(x, np.float32)
    q = np.empty(x.shape, np.uint8)
    lib.oracle_fp8_quantize(ptr(q, ct.c_ubyte), ptr(x, ct.c_float), x.size, float(s))
    return q


def fp8_matmul(qx, qw, sx, sw, bias=None):
    """(dec(qx) . dec(qw)^T) / (sx sw) + bias, float64 [M, N]."""
    lib = load()
    qx = np.ascontiguousarray(qx, np.uint8)
    qw = np.ascontiguousarray(qw, np.uint8)
    M, K = qx.shape
    N = qw.shape[0]
    assert qw.shape[1] == K
    out = np.empty((M, N), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float64)
    lib.oracle_fp8_matmul(ptr(out, ct.c_double), ptr(qx, ct.c_ubyte), ptr(qw, ct.c_ubyte),
                          ptr(b, ct.c_double), M, N, K, float(sx), float(sw))
    return out


# ---- causal attention on its own ---------------------------------------------

def attention_forward(qkv, NH):
    """The oracle's causal attention of fused (B, T, 3C) activations: out
    (B, T, C) and the probabilities att (B, NH, T, T), float64."""
    lib = load()
    qkv = np.ascontiguousarray(qkv, np.float64)
    B, T, C3 = qkv.shape
    C = C3 // 3
    assert C3 == 3 * C and C % NH == 0
    out = np.empty((B, T, C), np.float64)
    att = np.empty((B, NH, T, T), np.float64)
    lib.oracle_attention_forward(ptr(out, ct.c_double), ptr(att, ct.c_double),
                                 ptr(qkv, ct.c_double), B, T, C, NH)
    return out, att


def attention_backward(qkv, dout, NH):
    """The oracle's attention gradient: dqkv (B, T, 3C) float64 for the
    output gradient dout (B, T, C) of the causal attention of qkv."""
    lib = load()
    qkv = np.ascontiguousarray(qkv, np.float64)
    dout = np.ascontiguousarray(dout, np.float64)
    B, T, C3 = qkv.shape
    C = C3 // 3
    assert dout.shape == (B, T, C)
    _, att = attention_forward(qkv, NH)
    dqkv = np.zeros((B, T, C3), np.float64)
    lib.oracle_attention_backward(ptr(dqkv, ct.c_double), ptr(dout, ct.c_double),
                                  ptr(qkv, ct.c_double), ptr(att, ct.c_double), B, T, C, NH)
    return dqkv
