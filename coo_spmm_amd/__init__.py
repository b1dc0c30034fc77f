"""coo_spmm_amd -- MI355X (gfx950) truly sparse COO layer.

A thin ctypes binding of ``libsnack.so`` (the C ABI declared in
``include/snack.h``).  Every function below only marshals arguments: tensors
become device pointers, the current torch stream becomes the hipStream_t, and a
non-OK status becomes ``SnackError``.  All computation runs in the library's
HIP kernels; there is no CPU fallback -- importing this package fails loudly
when the library has not been built.

PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsnack.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m coo_spmm_amd.build` "
                      "(or __graft_entry__.build()); there is no fallback path")

# torch ships its own HIP runtime; loading it before the library makes both use
# that one runtime instance (loaded the other way round, the library's HIP
# calls find no device in a process where torch then initialises the GPU)
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

P = ctypes.c_void_p
i32, i64, u64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double
ST = ctypes.c_int

_SIGS = {
    "snack_status_string": ([ST], ctypes.c_char_p),
    "snack_layer_create": ([i32, i32, i64, P, P, P, u64, P, ctypes.POINTER(P)], ST),
    "snack_layer_destroy": ([P], ST),
    "snack_layer_reserve": ([P, i32], ST),
    "snack_forward": ([P, P, P, i32, P], ST),
    "snack_forward_noalloc": ([P, P, P, i32, P], ST),
    "snack_forward_infer": ([P, P, P, i32, i32, i32, P], ST),
    "snack_forward_chain": ([ctypes.POINTER(P), i32, ctypes.POINTER(i32), P, ctypes.POINTER(P), i32, i32, P], ST),
    "snack_backward": ([P, P, P, P, P, i32, P], ST),
    "snack_backward_sgd": ([P, P, P, P, P, f32, i32, P], ST),
    "snack_train_step_mse": ([P, P, P, P, P, P, P, f32, f32, i32, P], ST),
    "snack_prune_regrow": ([P, i64, P], ST),
    "snack_prune_regrow_grad": ([P, i64, P, P, i32, P], ST),
    "snack_prune_regrow_rows": ([P, i64, i64, i32, P, P, i32, P], ST),
    "snack_layer_shape": ([P, ctypes.POINTER(i32), ctypes.POINTER(i32)], ST),
    "snack_layer_nnz": ([P, ctypes.POINTER(i64)], ST),
    "snack_layer_device_bytes": ([P, ctypes.POINTER(i64)], ST),
    "snack_layer_values": ([P, ctypes.POINTER(P)], ST),
    "snack_layer_values_updated": ([P], ST),
    "snack_layer_export": ([P, P, P, P, P], ST),
    "snack_layer_export_index": ([P, P, P, P, P, P, P], ST),
    "snack_layer_get_epoch": ([P, ctypes.POINTER(u64)], ST),
    "snack_layer_set_epoch": ([P, u64], ST),
    "snack_sgd_step": ([P, P, f32, P], ST),
    "snack_mse_grad": ([P, P, P, i64, f32, P], ST),
    "snack_gelu_fwd": ([P, P, i64, P], ST),
    "snack_gelu_bwd": ([P, P, P, i64, P], ST),
    "snack_profile_enable": ([ctypes.c_int], ST),
    "snack_profile_reset": ([], ST),
    "snack_profile_name": ([ctypes.c_int], ctypes.c_char_p),
    "snack_profile_read": ([ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(f64)], ST),
    "snack_profile_set_tag": ([i64], ST),
    "snack_profile_read_tag": ([ctypes.c_int, i64, ctypes.POINTER(i64), ctypes.POINTER(f64)], ST),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)

OK, ERR_INVALID_ARG, ERR_INDEX_RANGE, ERR_DUPLICATE, ERR_ALLOC, ERR_HIP, ERR_UNSUPPORTED, ERR_WORKSPACE = range(8)


class SnackError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {snack_status_string(code)} (status {code})")


def snack_status_string(code: int) -> str:
    return _lib.snack_status_string(code).decode()


def _check(code: int, where: str):
    if code != OK:
        raise SnackError(code, where)


def _ptr(t):
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, shape, name):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------------------
# Functions with the C names (argument marshalling only)
# ---------------------------------------------------------------------------

def snack_layer_create(M, K, rows, cols, vals, seed=0, stream=None):
    """rows/cols int32 [nnz], vals float32 [nnz] or None: device tensors.  Returns the handle (int)."""
    import torch
    nnz = rows.numel()
    _need(rows, torch.int32, (nnz,), "rows")
    _need(cols, torch.int32, (nnz,), "cols")
    if vals is not None:
        _need(vals, torch.float32, (nnz,), "vals")
    h = P()
    _check(_lib.snack_layer_create(M, K, nnz, _ptr(rows), _ptr(cols), _ptr(vals), seed & (2**64 - 1),
                                   _stream(stream), ctypes.byref(h)), "snack_layer_create")
    return h.value


def snack_layer_destroy(h):
    _check(_lib.snack_layer_destroy(h), "snack_layer_destroy")


def snack_layer_reserve(h, max_batch):
    _check(_lib.snack_layer_reserve(h, max_batch), "snack_layer_reserve")


def snack_forward(h, X, Y, stream=None):
    B = X.shape[0]
    _check(_lib.snack_forward(h, _ptr(X), _ptr(Y), B, _stream(stream)), "snack_forward")


def snack_forward_noalloc(h, X, Y, stream=None):
    B = X.shape[0]
    _check(_lib.snack_forward_noalloc(h, _ptr(X), _ptr(Y), B, _stream(stream)), "snack_forward_noalloc")


ACT_NONE, ACT_GELU = 0, 1
REGROW_RANDOM, REGROW_GRADIENT = 0, 1


def snack_forward_infer(h, X, Y, act=ACT_NONE, bf16_values=False, stream=None):
    B = X.shape[0]
    _check(_lib.snack_forward_infer(h, _ptr(X), _ptr(Y), B, int(act), 1 if bf16_values else 0, _stream(stream)),
           "snack_forward_infer")


def snack_forward_chain(handles, acts, X, Ys, bf16_values=False, stream=None):
    """handles: layer handles; acts: activation codes; Ys: output tensors, one per layer."""
    n = len(handles)
    if len(acts) != n or len(Ys) != n:
        raise ValueError("one activation and one output per layer")
    hs = (P * n)(*handles)
    ac = (i32 * n)(*[int(a) for a in acts])
    ys = (P * n)(*[_ptr(y) for y in Ys])
    _check(_lib.snack_forward_chain(hs, n, ac, _ptr(X), ys, X.shape[0], 1 if bf16_values else 0, _stream(stream)),
           "snack_forward_chain")


def snack_backward(h, X, dY, dX=None, dW=None, stream=None):
    B = dY.shape[0]
    _check(_lib.snack_backward(h, _ptr(X), _ptr(dY), _ptr(dX), _ptr(dW), B, _stream(stream)), "snack_backward")


def snack_backward_sgd(h, X, dY, dX, dW, lr, stream=None):
    B = dY.shape[0]
    _check(_lib.snack_backward_sgd(h, _ptr(X), _ptr(dY), _ptr(dX), _ptr(dW), float(lr), B, _stream(stream)),
           "snack_backward_sgd")


def snack_train_step_mse(h, X, T, Y, dY, dX, dW, scale, lr, stream=None):
    B = X.shape[0]
    _check(_lib.snack_train_step_mse(h, _ptr(X), _ptr(T), _ptr(Y), _ptr(dY), _ptr(dX), _ptr(dW), float(scale),
                                     float(lr), B, _stream(stream)), "snack_train_step_mse")


def snack_prune_regrow(h, n_drop, stream=None):
    _check(_lib.snack_prune_regrow(h, int(n_drop), _stream(stream)), "snack_prune_regrow")


def snack_prune_regrow_grad(h, n_drop, X, dY, stream=None):
    """X [B, K], dY [B, M]: the batch whose dense weight gradient picks the grown cells."""
    B = X.shape[0]
    if dY.shape[0] != B:
        raise ValueError("X and dY must have the same batch")
    _check(_lib.snack_prune_regrow_grad(h, int(n_drop), _ptr(X), _ptr(dY), B, _stream(stream)),
           "snack_prune_regrow_grad")


def snack_prune_regrow_rows(h, drop_num, drop_den, mode, X=None, dY=None, stream=None):
    """Row-local drop / regrow: each row drops floor(n_i * drop_num / drop_den) of its smallest |w| and
    regrows as many inside itself, at random (REGROW_RANDOM) or at the largest |dY^T X| (REGROW_GRADIENT,
    X [B, K], dY [B, M])."""
    B = 0
    if X is not None or dY is not None:
        if X is None or dY is None or dY.shape[0] != X.shape[0]:
            raise ValueError("X and dY must both be given, with the same batch")
        B = X.shape[0]
    _check(_lib.snack_prune_regrow_rows(h, int(drop_num), int(drop_den), int(mode), _ptr(X), _ptr(dY), B,
                                        _stream(stream)), "snack_prune_regrow_rows")


def snack_layer_shape(h):
    m, k = i32(), i32()
    _check(_lib.snack_layer_shape(h, ctypes.byref(m), ctypes.byref(k)), "snack_layer_shape")
    return m.value, k.value


def snack_layer_nnz(h):
    n = i64()
    _check(_lib.snack_layer_nnz(h, ctypes.byref(n)), "snack_layer_nnz")
    return n.value


def snack_layer_device_bytes(h):
    n = i64()
    _check(_lib.snack_layer_device_bytes(h, ctypes.byref(n)), "snack_layer_device_bytes")
    return n.value


def snack_layer_values(h):
    p = P()
    _check(_lib.snack_layer_values(h, ctypes.byref(p)), "snack_layer_values")
    return p.value


def snack_layer_values_updated(h):
    _check(_lib.snack_layer_values_updated(h), "snack_layer_values_updated")


def snack_layer_export(h, rows, cols, vals, stream=None):
    _check(_lib.snack_layer_export(h, _ptr(rows), _ptr(cols), _ptr(vals), _stream(stream)), "snack_layer_export")


def snack_layer_export_index(h, row_ptr, perm, rows_t, col_ptr, vals_t=None, stream=None):
    _check(_lib.snack_layer_export_index(h, _ptr(row_ptr), _ptr(perm), _ptr(rows_t), _ptr(col_ptr), _ptr(vals_t),
                                         _stream(stream)), "snack_layer_export_index")


def snack_layer_get_epoch(h):
    e = u64()
    _check(_lib.snack_layer_get_epoch(h, ctypes.byref(e)), "snack_layer_get_epoch")
    return e.value


def snack_layer_set_epoch(h, epoch):
    _check(_lib.snack_layer_set_epoch(h, epoch), "snack_layer_set_epoch")


def snack_sgd_step(h, dW, lr, stream=None):
    _check(_lib.snack_sgd_step(h, _ptr(dW), float(lr), _stream(stream)), "snack_sgd_step")


def snack_mse_grad(Y, T, dY, scale, stream=None):
    _check(_lib.snack_mse_grad(_ptr(Y), _ptr(T), _ptr(dY), Y.numel(), float(scale), _stream(stream)),
           "snack_mse_grad")


def snack_gelu_fwd(X, Y, stream=None):
    _check(_lib.snack_gelu_fwd(_ptr(X), _ptr(Y), X.numel(), _stream(stream)), "snack_gelu_fwd")


def snack_gelu_bwd(X, dY, dX, stream=None):
    _check(_lib.snack_gelu_bwd(_ptr(X), _ptr(dY), _ptr(dX), X.numel(), _stream(stream)), "snack_gelu_bwd")


def snack_profile_enable(on=True):
    _check(_lib.snack_profile_enable(1 if on else 0), "snack_profile_enable")


def snack_profile_reset():
    _check(_lib.snack_profile_reset(), "snack_profile_reset")


def snack_profile_name(k):
    n = _lib.snack_profile_name(k)
    return None if n is None else n.decode()


def snack_profile_read(k):
    n, ms = i64(), f64()
    _check(_lib.snack_profile_read(k, ctypes.byref(n), ctypes.byref(ms)), "snack_profile_read")
    return n.value, ms.value


def snack_profile_set_tag(tag):
    _check(_lib.snack_profile_set_tag(int(tag)), "snack_profile_set_tag")


def snack_profile_read_tag(k, tag):
    n, ms = i64(), f64()
    _check(_lib.snack_profile_read_tag(k, int(tag), ctypes.byref(n), ctypes.byref(ms)), "snack_profile_read_tag")
    return n.value, ms.value


def profile_class_ids():
    """{kernel class name: id}."""
    out, k = {}, 0
    while True:
        name = snack_profile_name(k)
        if name is None:
            return out
        out[name] = k
        k += 1


def profile_snapshot():
    """{kernel class name: (launches, total ms)} for every class."""
    out, k = {}, 0
    while True:
        name = snack_profile_name(k)
        if name is None:
            return out
        out[name] = snack_profile_read(k)
        k += 1


# ---------------------------------------------------------------------------
# Convenience object over the same calls
# ---------------------------------------------------------------------------

class SnackLayer:
    """Owns one layer handle.  Tensors are torch device tensors."""

    def __init__(self, M, K, rows, cols, vals=None, seed=0, stream=None, max_batch=None):
        """max_batch: also reserve the workspace for batches up to it (create covers up to 64)."""
        self.M, self.K = int(M), int(K)
        self.h = snack_layer_create(self.M, self.K, rows, cols, vals, seed, stream)
        self.nnz = snack_layer_nnz(self.h)
        if max_batch is not None:
            snack_layer_reserve(self.h, int(max_batch))

    def close(self):
        if getattr(self, "h", None):
            snack_layer_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, X, Y=None, stream=None):
        import torch
        if Y is None:
            Y = torch.empty((X.shape[0], self.M), dtype=torch.float32, device=X.device)
        snack_forward(self.h, X, Y, stream)
        return Y

    def backward(self, X, dY, want_dx=True, want_dw=True, dX=None, dW=None, stream=None):
        import torch
        if want_dx and dX is None:
            dX = torch.empty((dY.shape[0], self.K), dtype=torch.float32, device=dY.device)
        if want_dw and dW is None:
            dW = torch.empty((self.nnz,), dtype=torch.float32, device=dY.device)
        snack_backward(self.h, X, dY, dX if want_dx else None, dW if want_dw else None, stream)
        return (dX if want_dx else None), (dW if want_dw else None)

    def backward_sgd(self, X, dY, lr, want_dx=True, dX=None, dW=None, stream=None):
        import torch
        if want_dx and dX is None:
            dX = torch.empty((dY.shape[0], self.K), dtype=torch.float32, device=dY.device)
        if dW is None:
            dW = torch.empty((self.nnz,), dtype=torch.float32, device=dY.device)
        snack_backward_sgd(self.h, X, dY, dX if want_dx else None, dW, lr, stream)
        return (dX if want_dx else None), dW

    def train_step_mse(self, X, T, lr, want_dx=True, scale=None, out=None, stream=None):
        """Forward, MSE gradient (scale defaults to the mean's 2 / (B * M)), backward and SGD step in one
        call; returns (Y, dY, dX, dW).  `out` may supply that tuple of preallocated tensors."""
        import torch
        B = X.shape[0]
        if scale is None:
            scale = 2.0 / (B * self.M)
        if out is None:
            dev = X.device
            out = (torch.empty((B, self.M), dtype=torch.float32, device=dev),
                   torch.empty((B, self.M), dtype=torch.float32, device=dev),
                   torch.empty((B, self.K), dtype=torch.float32, device=dev) if want_dx else None,
                   torch.empty((self.nnz,), dtype=torch.float32, device=dev))
        Y, dY, dX, dW = out
        snack_train_step_mse(self.h, X, T, Y, dY, dX if want_dx else None, dW, scale, lr, stream)
        return Y, dY, (dX if want_dx else None), dW

    def prune_regrow(self, n_drop, stream=None):
        snack_prune_regrow(self.h, n_drop, stream)

    def prune_regrow_grad(self, n_drop, X, dY, stream=None):
        snack_prune_regrow_grad(self.h, n_drop, X, dY, stream)

    def prune_regrow_rows(self, drop_num, drop_den, mode=REGROW_RANDOM, X=None, dY=None, stream=None):
        snack_prune_regrow_rows(self.h, drop_num, drop_den, mode, X, dY, stream)

    def sgd_step(self, dW, lr, stream=None):
        snack_sgd_step(self.h, dW, lr, stream)

    def export(self, device="cuda", stream=None):
        import torch
        r = torch.empty(self.nnz, dtype=torch.int32, device=device)
        c = torch.empty(self.nnz, dtype=torch.int32, device=device)
        v = torch.empty(self.nnz, dtype=torch.float32, device=device)
        snack_layer_export(self.h, r, c, v, stream)
        return r, c, v

    def export_index(self, device="cuda", stream=None, with_values=False):
        import torch
        rp = torch.empty(self.M + 1, dtype=torch.int32, device=device)
        pm = torch.empty(self.nnz, dtype=torch.int32, device=device)
        rt = torch.empty(self.nnz, dtype=torch.int32, device=device)
        cp = torch.empty(self.K + 1, dtype=torch.int32, device=device)
        vt = torch.empty(self.nnz, dtype=torch.float32, device=device)
        ok = self.nnz > 0
        snack_layer_export_index(self.h, rp, pm if ok else None, rt if ok else None, cp,
                                 vt if (ok and with_values) else None, stream)
        if with_values:
            return rp, pm, rt, cp, vt
        return rp, pm, rt, cp

    def values_ptr(self):
        return snack_layer_values(self.h)

    @property
    def epoch(self):
        return snack_layer_get_epoch(self.h)

    @epoch.setter
    def epoch(self, e):
        snack_layer_set_epoch(self.h, e)

    def device_bytes(self):
        return snack_layer_device_bytes(self.h)

    def reserve(self, max_batch):
        snack_layer_reserve(self.h, max_batch)
