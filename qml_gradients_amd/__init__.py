"""qml_gradients_amd -- Python binding of the hqml C-ABI library (libhqml.so).

The library runs the whole training step (fused forward passes, the fused
adjoint backward passes and every reduction) in its own gfx950 kernels.  This
module only marshals arguments: it passes device pointers of torch tensors to
the C entry points of ``include/hqml.h``, whose names it keeps.  PyTorch is used
for device memory and streams only.  There is no fallback: if ``libhqml.so`` is
missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhqml.so")

HQML_OK = 0
HQML_ERR_ARG = -1
HQML_ERR_OOM = -2
HQML_ERR_HIP = -3
HQML_ERR_STATE = -4
HQML_ERR_UNSUPPORTED = -5
HQML_STORE_FP32 = 0
HQML_STORE_BF16 = 1
HQML_STORE_FP64 = 2
HQML_COMPUTE_FP32 = 0
HQML_COMPUTE_FP64 = 1
HQML_FUSED = 0
HQML_GATE_BY_GATE = 1
HQML_ENT_CZ = 0
HQML_ENT_CNOT = 1
HQML_K_FWD_PASS, HQML_K_BWD_PASS, HQML_K_SMALL, HQML_K_OTHER, HQML_K_GATE, HQML_K_COUNT = range(6)


class hqml_config(ctypes.Structure):
    _fields_ = [
        ("n_qubits", ctypes.c_int),
        ("n_layers", ctypes.c_int),
        ("max_batch", ctypes.c_int),
        ("storage", ctypes.c_int),
        ("ckpt_block", ctypes.c_int),
        ("device", ctypes.c_int),
        ("stream", ctypes.c_void_p),
        ("fusion", ctypes.c_int),
        ("compute", ctypes.c_int),
        ("obs_mask", ctypes.c_int),
        ("obs_x_mask", ctypes.c_int),
        ("entangler", ctypes.c_int),
    ]


class HqmlError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hqml status {status}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libhqml.so (built by ``python -m qml_gradients_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"hqml library not built: {LIB_PATH} is missing "
                           "(run `python -m qml_gradients_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i = ctypes.c_int
    cfgp = ctypes.POINTER(hqml_config)
    sig = {
        "hqml_workspace_bytes": (ctypes.c_size_t, [cfgp]),
        "hqml_create": (i, [cfgp, ctypes.POINTER(P)]),
        "hqml_destroy": (i, [P]),
        "hqml_forward": (i, [P, i, P, P, P, i]),
        "hqml_backward": (i, [P, P, P]),
        "hqml_train_step": (i, [P, i, P, P, P, P, P, P]),
        "hqml_forward_f64": (i, [P, i, P, P, P, i]),
        "hqml_backward_f64": (i, [P, P, P]),
        "hqml_train_step_f64": (i, [P, i, P, P, P, P, P, P]),
        "hqml_status_str": (ctypes.c_char_p, [i]),
        "hqml_last_error": (ctypes.c_char_p, [P]),
        "hqml_set_timing": (i, [P, i]),
        "hqml_set_overlap": (i, [P, i]),
        "hqml_kernel_times": (i, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong), i]),
        "hqml_plan_info": (i, [P, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i),
                              ctypes.POINTER(ctypes.c_size_t)]),
        "hqml_describe_plan": (ctypes.c_longlong, [cfgp, ctypes.c_char_p, ctypes.c_size_t]),
        "hqml_train_step_noalloc": (i, [cfgp, i, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


EXPORTED = ("hqml_workspace_bytes", "hqml_create", "hqml_destroy", "hqml_forward", "hqml_backward",
            "hqml_train_step", "hqml_forward_f64", "hqml_backward_f64", "hqml_train_step_f64", "hqml_status_str", "hqml_last_error", "hqml_set_timing",
            "hqml_set_overlap", "hqml_kernel_times", "hqml_plan_info", "hqml_describe_plan",
            "hqml_train_step_noalloc")


def make_config(n_qubits, n_layers, max_batch, storage="fp32", ckpt_block=0, device=0, stream=None,
                fusion="fused", obs_mask=0, compute="fp32", obs_x_mask=0, entangler="cz"):
    st = {"fp32": HQML_STORE_FP32, "bf16": HQML_STORE_BF16, "fp64": HQML_STORE_FP64}.get(storage, storage)
    fu = {"fused": HQML_FUSED, "gate_by_gate": HQML_GATE_BY_GATE}.get(fusion, fusion)
    co = {"fp32": HQML_COMPUTE_FP32, "fp64": HQML_COMPUTE_FP64}.get(compute, compute)
    en = {"cz": HQML_ENT_CZ, "cnot": HQML_ENT_CNOT}.get(entangler, entangler)
    return hqml_config(int(n_qubits), int(n_layers), int(max_batch), int(st), int(ckpt_block),
                       int(device), ctypes.c_void_p(stream or 0), int(fu), int(co), int(obs_mask),
                       int(obs_x_mask), int(en))


# ---- the C entry points, same names, argument marshalling only ----

def hqml_workspace_bytes(cfg: hqml_config) -> int:
    return int(load().hqml_workspace_bytes(ctypes.byref(cfg)))


def hqml_describe_plan(cfg: hqml_config) -> str:
    lib = load()
    need = lib.hqml_describe_plan(ctypes.byref(cfg), None, 0)
    if need < 0:
        raise HqmlError(int(need), "invalid configuration")
    buf = ctypes.create_string_buffer(int(need) + 1)
    lib.hqml_describe_plan(ctypes.byref(cfg), buf, len(buf))
    return buf.value.decode()


def hqml_create(cfg: hqml_config) -> ctypes.c_void_p:
    lib = load()
    h = ctypes.c_void_p()
    rc = lib.hqml_create(ctypes.byref(cfg), ctypes.byref(h))
    if rc != HQML_OK:
        raise HqmlError(rc, lib.hqml_last_error(None).decode())
    return h


def _check(ctx, rc):
    if rc != HQML_OK:
        raise HqmlError(rc, load().hqml_last_error(ctx).decode())


def hqml_destroy(ctx) -> None:
    load().hqml_destroy(ctx)


def hqml_forward(ctx, B, x_ptr, theta_ptr, expz_ptr, save_for_backward) -> None:
    _check(ctx, load().hqml_forward(ctx, int(B), x_ptr, theta_ptr, expz_ptr, int(save_for_backward)))


def hqml_backward(ctx, dlde_ptr, grad_ptr) -> None:
    _check(ctx, load().hqml_backward(ctx, dlde_ptr, grad_ptr))


def hqml_train_step(ctx, B, x_ptr, theta_ptr, y_ptr, expz_ptr, loss_ptr, grad_ptr) -> None:
    _check(ctx, load().hqml_train_step(ctx, int(B), x_ptr, theta_ptr, y_ptr, expz_ptr, loss_ptr, grad_ptr))


def hqml_forward_f64(ctx, B, x_ptr, theta_ptr, expz_ptr, save_for_backward) -> None:
    _check(ctx, load().hqml_forward_f64(ctx, int(B), x_ptr, theta_ptr, expz_ptr, int(save_for_backward)))


def hqml_backward_f64(ctx, dlde_ptr, grad_ptr) -> None:
    _check(ctx, load().hqml_backward_f64(ctx, dlde_ptr, grad_ptr))


def hqml_train_step_f64(ctx, B, x_ptr, theta_ptr, y_ptr, expz_ptr, loss_ptr, grad_ptr) -> None:
    _check(ctx, load().hqml_train_step_f64(ctx, int(B), x_ptr, theta_ptr, y_ptr, expz_ptr, loss_ptr, grad_ptr))


def hqml_train_step_noalloc(cfg: hqml_config, B, x_ptr, theta_ptr, y_ptr, expz_ptr, loss_ptr, grad_ptr) -> None:
    lib = load()
    rc = lib.hqml_train_step_noalloc(ctypes.byref(cfg), int(B), x_ptr, theta_ptr, y_ptr, expz_ptr, loss_ptr, grad_ptr)
    if rc != HQML_OK:
        raise HqmlError(rc, lib.hqml_last_error(None).decode())


def hqml_set_timing(ctx, enable: bool) -> None:
    _check(ctx, load().hqml_set_timing(ctx, int(bool(enable))))


def hqml_set_overlap(ctx, chunks: int) -> None:
    _check(ctx, load().hqml_set_overlap(ctx, int(chunks)))


def hqml_kernel_times(ctx, reset: bool = True):
    ms = (ctypes.c_double * HQML_K_COUNT)()
    cnt = (ctypes.c_longlong * HQML_K_COUNT)()
    _check(ctx, load().hqml_kernel_times(ctx, ms, cnt, int(bool(reset))))
    return list(ms), list(cnt)


def hqml_plan_info(ctx):
    f, b, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    sb = ctypes.c_size_t()
    _check(ctx, load().hqml_plan_info(ctx, ctypes.byref(f), ctypes.byref(b), ctypes.byref(t), ctypes.byref(sb)))
    return {"fwd_passes": f.value, "bwd_passes": b.value, "tiles_per_sample": t.value,
            "state_bytes": sb.value}


# ---- convenience wrapper over torch tensors ----

class Context:
    """One hqml context on the current torch device and stream.

    Inputs and outputs are torch CUDA tensors (float32; float64 for a context with
    compute="fp64", through the *_f64 entry points); the library reads and writes
    them in place through their device pointers.
    """

    def __init__(self, n_qubits, n_layers, max_batch, storage="fp32", ckpt_block=0, device=None,
                 stream=None, fusion="fused", obs_mask=0, compute="fp32", obs_x_mask=0, entangler="cz"):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("hqml needs a GPU (torch.cuda.is_available() is False)")
        dev = torch.cuda.current_device() if device is None else int(device)
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        self.torch = torch
        self.device = torch.device("cuda", dev)
        self.n, self.L, self.max_batch = int(n_qubits), int(n_layers), int(max_batch)
        self.cfg = make_config(n_qubits, n_layers, max_batch, storage, ckpt_block, dev, stream, fusion,
                               obs_mask, compute, obs_x_mask, entangler)
        self.f64 = compute == "fp64" or compute == HQML_COMPUTE_FP64
        self.dtype = torch.float64 if self.f64 else torch.float32
        self.handle = hqml_create(self.cfg)
        self.fwd_id = 0          # counts forwards (the saved states belong to the latest one)

    def close(self):
        if self.handle is not None:
            hqml_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _dev(self, a, shape):
        t = self.torch
        a = t.as_tensor(a, dtype=self.dtype, device=self.device).contiguous()
        if tuple(a.shape) != tuple(shape):
            raise ValueError(f"expected shape {tuple(shape)}, got {tuple(a.shape)}")
        return a

    def forward(self, x, theta, save_for_backward=True):
        B = int(x.shape[0])
        x = self._dev(x, (B, self.n))
        theta = self._dev(theta, (self.L, self.n, 3))
        expz = self.torch.empty(B, dtype=self.dtype, device=self.device)
        fwd = hqml_forward_f64 if self.f64 else hqml_forward
        fwd(self.handle, B, x.data_ptr(), theta.data_ptr(), expz.data_ptr(), save_for_backward)
        self.fwd_id += 1
        self._keep = (x, theta)
        return expz

    def backward(self, dlde):
        dlde = self._dev(dlde, (int(dlde.shape[0]),))
        grad = self.torch.empty((self.L, self.n, 3), dtype=self.dtype, device=self.device)
        bwd = hqml_backward_f64 if self.f64 else hqml_backward
        bwd(self.handle, dlde.data_ptr(), grad.data_ptr())
        self._keep_b = dlde
        return grad

    def train_step(self, x, theta, y):
        B = int(x.shape[0])
        x = self._dev(x, (B, self.n))
        theta = self._dev(theta, (self.L, self.n, 3))
        y = self._dev(y, (B,))
        t = self.torch
        expz = t.empty(B, dtype=self.dtype, device=self.device)
        loss = t.empty(1, dtype=self.dtype, device=self.device)
        grad = t.empty((self.L, self.n, 3), dtype=self.dtype, device=self.device)
        step = hqml_train_step_f64 if self.f64 else hqml_train_step
        step(self.handle, B, x.data_ptr(), theta.data_ptr(), y.data_ptr(), expz.data_ptr(), loss.data_ptr(),
             grad.data_ptr())
        self.fwd_id += 1
        self._keep = (x, theta, y)
        return expz, loss, grad

    def set_timing(self, enable=True):
        hqml_set_timing(self.handle, enable)

    def set_overlap(self, chunks):
        hqml_set_overlap(self.handle, chunks)

    def kernel_times(self, reset=True):
        return hqml_kernel_times(self.handle, reset)

    def plan_info(self):
        return hqml_plan_info(self.handle)
