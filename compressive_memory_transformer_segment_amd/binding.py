"""Python binding of the C-ABI in ``include/infini_attn.h`` (ctypes).

Argument marshalling only: every step of the layer runs in the HIP library.  Torch is
used for device memory and streams; tensors are passed as raw device pointers together
with the current HIP stream.  There is no fallback: if ``libinfini_attn.so`` is missing
or the call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libinfini_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG_DIR), "include", "infini_attn.h")

UPDATE = {"linear": 0, "delta": 1}
DTYPE = {"bf16": 0, "f32": 1}
TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_OOM, ERR_SCRATCH = 0, -1, -2, -3, -4, -5


class Config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("segment_len", ctypes.c_int32),
        ("update", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("max_window_segments", ctypes.c_int32),
    ]


KERNEL_KINDS = ("key_sums", "state_pass", "chain", "attention", "proj_qkv", "proj_out", "decode", "backward")


class Profile(ctypes.Structure):
    _fields_ = [("total_ms", ctypes.c_double * len(KERNEL_KINDS)), ("launches", ctypes.c_int64 * len(KERNEL_KINDS))]


class InfiniAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} ({status})")
        self.status = status


_lib = None


def exported_names() -> list[str]:
    """Entry points the header declares (used by the load test)."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(infini_attn_[a-z_]+)\s*\(", text)))


def load() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    fp = ctypes.POINTER(ctypes.c_float)
    sig = {
        "infini_attn_create": (ctypes.c_int, [ctypes.POINTER(Config), fp, vp, ctypes.POINTER(vp)]),
        "infini_attn_forward_segment": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp]),
        "infini_attn_forward_stream": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, vp]),
        "infini_attn_forward_stream_ex": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, i64, vp]),
        "infini_attn_forward_stream_local": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, i64, vp]),
        "infini_attn_forward_stream_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, vp]),
        "infini_attn_project_qkv": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i64, i32, vp]),
        "infini_attn_project_out": (ctypes.c_int, [vp, vp, vp, vp, i64, i32, vp]),
        "infini_attn_forward_layer": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, i32, vp]),
        "infini_attn_decode_step": (ctypes.c_int, [vp, vp, vp, vp, vp, vp]),
        "infini_attn_backward": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]),
        "infini_attn_decode_flush": (ctypes.c_int, [vp, vp]),
        "infini_attn_decode_position": (i64, [vp]),
        "infini_attn_reset_state": (ctypes.c_int, [vp, vp]),
        "infini_attn_get_state": (ctypes.c_int, [vp, vp, vp, vp]),
        "infini_attn_set_state": (ctypes.c_int, [vp, vp, vp, vp]),
        "infini_attn_set_beta": (ctypes.c_int, [vp, fp]),
        "infini_attn_device_bytes": (i64, [vp]),
        "infini_attn_window_tokens": (i64, [vp]),
        "infini_attn_destroy": (ctypes.c_int, [vp]),
        "infini_attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "infini_attn_profile_enable": (ctypes.c_int, [vp, ctypes.c_int]),
        "infini_attn_profile_read": (ctypes.c_int, [vp, ctypes.POINTER(Profile)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().infini_attn_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise InfiniAttnError(fn, status, status_string(status))


def _stream_ptr(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _float_array(values) -> ctypes.Array:
    vals = [float(x) for x in values]
    return (ctypes.c_float * len(vals))(*vals)


class InfiniAttention:
    """One Infini-attention layer (per-head part): state M, z and gate on the GPU.

    Q, K, V and outputs are contiguous [B, H, T, d] tensors on the current CUDA (HIP)
    device, dtype bfloat16 (io_dtype="bf16") or float32 ("f32").
    """

    def __init__(self, batch: int, heads: int, head_dim: int, segment_len: int,
                 update: str = "linear", io_dtype: str = "bf16", eps: float = 1e-6,
                 softmax_scale: float = 0.0, beta=None, max_window_segments: int = 0, stream=None):
        self._lib = load()
        self.batch, self.heads, self.head_dim, self.segment_len = batch, heads, head_dim, segment_len
        self.update, self.io_dtype = update, io_dtype
        self.dtype = TORCH_DTYPE[io_dtype]
        cfg = Config(batch, heads, head_dim, segment_len, UPDATE[update], DTYPE[io_dtype],
                     eps, softmax_scale, max_window_segments)
        beta = [0.0] * heads if beta is None else list(beta)
        if len(beta) != heads:
            raise ValueError("beta needs one value per head")
        handle = ctypes.c_void_p()
        _check("infini_attn_create",
               self._lib.infini_attn_create(ctypes.byref(cfg), _float_array(beta), _stream_ptr(stream),
                                            ctypes.byref(handle)))
        self._h = handle

    # ------------------------------------------------------------------ lifecycle
    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            _check("infini_attn_destroy", self._lib.infini_attn_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    # ------------------------------------------------------------------ compute
    def _check_io(self, *tensors):
        for t in tensors:
            if t is None:
                continue
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("tensors must be contiguous and on the GPU")

    def _out_like(self, q, out):
        if out is None:
            out = torch.empty_like(q)
        return out

    def forward_stream(self, q, k, v, out=None, a_mem=None, a_dot=None, stream=None):
        self._check_io(q, k, v, out, a_mem, a_dot)
        out = self._out_like(q, out)
        n = q.shape[2]
        if a_mem is None and a_dot is None:
            st = self._lib.infini_attn_forward_stream(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), n,
                                                      _stream_ptr(stream))
            _check("infini_attn_forward_stream", st)
        else:
            st = self._lib.infini_attn_forward_stream_ex(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                                         _ptr(a_mem), _ptr(a_dot), n, _stream_ptr(stream))
            _check("infini_attn_forward_stream_ex", st)
        return out

    def forward_stream_noalloc(self, q, k, v, out=None, stream=None):
        """forward_stream with the window workspace in the library's static scratch array
        (the call allocates no device memory; ``out`` must then be given by a caller that
        cannot allocate)."""
        self._check_io(q, k, v, out)
        out = self._out_like(q, out)
        st = self._lib.infini_attn_forward_stream_noalloc(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                                          q.shape[2], _stream_ptr(stream))
        _check("infini_attn_forward_stream_noalloc", st)
        return out

    def forward_stream_local(self, q, k, v, q_local=None, k_local=None, out=None, stream=None):
        """Local attention on q_local / k_local (e.g. position-embedded), retrieval and
        memory update on the PE-free q / k.  None means "same as q / k"."""
        self._check_io(q, k, v, q_local, k_local, out)
        out = self._out_like(q, out)
        st = self._lib.infini_attn_forward_stream_local(
            self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(q_local) if q_local is not None else None,
            _ptr(k_local) if k_local is not None else None, _ptr(out), q.shape[2], _stream_ptr(stream))
        _check("infini_attn_forward_stream_local", st)
        return out

    def forward_segment(self, q, k, v, out=None, stream=None):
        self._check_io(q, k, v, out)
        out = self._out_like(q, out)
        st = self._lib.infini_attn_forward_segment(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                                   q.shape[2], _stream_ptr(stream))
        _check("infini_attn_forward_segment", st)
        return out

    # ------------------------------------------------------------------ the layer (Eq. 5, 11)
    def _check_layer_io(self, *tensors):
        self._check_io(*tensors)
        for t in tensors:
            if t is not None and t.dtype != torch.bfloat16:
                raise ValueError("the projections take bfloat16 tensors")

    def project_qkv(self, x, w_qkv, q=None, k=None, v=None, stream=None):
        """x [B, T, d_model], w_qkv [3 H d, d_model] -> Q, K, V [B, H, T, d]."""
        self._check_layer_io(x, w_qkv, q, k, v)
        B, T, dm = x.shape
        shape = (B, self.heads, T, self.head_dim)
        q, k, v = (torch.empty(shape, dtype=x.dtype, device=x.device) if t is None else t for t in (q, k, v))
        st = self._lib.infini_attn_project_qkv(self._h, _ptr(x), _ptr(w_qkv), _ptr(q), _ptr(k), _ptr(v), T, dm,
                                               _stream_ptr(stream))
        _check("infini_attn_project_qkv", st)
        return q, k, v

    def project_out(self, a, w_o, out=None, stream=None):
        """a [B, H, T, d], w_o [d_model, H d] -> O [B, T, d_model]."""
        self._check_layer_io(a, w_o, out)
        B, H, T, d = a.shape
        dm = w_o.shape[0]
        if out is None:
            out = torch.empty((B, T, dm), dtype=a.dtype, device=a.device)
        st = self._lib.infini_attn_project_out(self._h, _ptr(a), _ptr(w_o), _ptr(out), T, dm, _stream_ptr(stream))
        _check("infini_attn_project_out", st)
        return out

    def forward_layer(self, x, w_qkv, w_o, out=None, stream=None):
        """x [B, T, d_model] -> O [B, T, d_model] through the whole layer (Eq. 5 - Eq. 11)."""
        self._check_layer_io(x, w_qkv, w_o, out)
        B, T, dm = x.shape
        if out is None:
            out = torch.empty_like(x)
        st = self._lib.infini_attn_forward_layer(self._h, _ptr(x), _ptr(w_qkv), _ptr(w_o), _ptr(out), T, dm,
                                                 _stream_ptr(stream))
        _check("infini_attn_forward_layer", st)
        return out

    # ------------------------------------------------------------------ decoding
    def decode_step(self, q, k, v, out=None, stream=None):
        """One token per sequence: q, k, v [B, H, d] (or [B, H, 1, d]) -> out of the same shape."""
        self._check_io(q, k, v, out)
        if out is None:
            out = torch.empty_like(q)
        st = self._lib.infini_attn_decode_step(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _stream_ptr(stream))
        _check("infini_attn_decode_step", st)
        return out

    def decode_flush(self, stream=None) -> None:
        _check("infini_attn_decode_flush", self._lib.infini_attn_decode_flush(self._h, _stream_ptr(stream)))

    def decode_position(self) -> int:
        return int(self._lib.infini_attn_decode_position(self._h))

    # ------------------------------------------------------------------ backward
    def backward(self, q, k, v, d_out, m0=None, z0=None, dm_final=None, dz_final=None, want_state_grads=True,
                 stream=None):
        """Gradients of <d_out, O> (+ <dm_final, M_final> + <dz_final, z_final>) for the stream
        q, k, v [B, H, T, d] started from (m0, z0) (zeros when None).  Returns a dict of float32
        tensors dq, dk, dv, dbeta and, with want_state_grads, dm0, dz0."""
        self._check_io(q, k, v, d_out)
        f32 = lambda t: None if t is None else t.to(device="cuda", dtype=torch.float32).contiguous()   # noqa: E731
        m0, z0, dm_final, dz_final = f32(m0), f32(z0), f32(dm_final), f32(dz_final)
        B, H, T, d = q.shape
        res = {n: torch.empty((B, H, T, d), dtype=torch.float32, device=q.device) for n in ("dq", "dk", "dv")}
        res["dbeta"] = torch.empty((H,), dtype=torch.float32, device=q.device)
        if want_state_grads:
            res["dm0"] = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
            res["dz0"] = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
        opt = lambda t: _ptr(t) if t is not None else None   # noqa: E731
        st = self._lib.infini_attn_backward(
            self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(d_out), opt(m0), opt(z0), opt(dm_final), opt(dz_final),
            _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dbeta"]), opt(res.get("dm0")),
            opt(res.get("dz0")), T, _stream_ptr(stream))
        _check("infini_attn_backward", st)
        return res

    # ------------------------------------------------------------------ state
    def reset_state(self, stream=None) -> None:
        _check("infini_attn_reset_state", self._lib.infini_attn_reset_state(self._h, _stream_ptr(stream)))

    def get_state(self, stream=None):
        B, H, d = self.batch, self.heads, self.head_dim
        M = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
        z = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
        _check("infini_attn_get_state",
               self._lib.infini_attn_get_state(self._h, _ptr(M), _ptr(z), _stream_ptr(stream)))
        return M, z

    def set_state(self, M, z, stream=None) -> None:
        """Either part may be None (that part keeps its value)."""
        M = None if M is None else M.to(device="cuda", dtype=torch.float32).contiguous()
        z = None if z is None else z.to(device="cuda", dtype=torch.float32).contiguous()
        _check("infini_attn_set_state",
               self._lib.infini_attn_set_state(self._h, _ptr(M) if M is not None else None,
                                               _ptr(z) if z is not None else None, _stream_ptr(stream)))

    def set_beta(self, beta) -> None:
        _check("infini_attn_set_beta", self._lib.infini_attn_set_beta(self._h, _float_array(beta)))

    def device_bytes(self) -> int:
        return int(self._lib.infini_attn_device_bytes(self._h))

    def window_tokens(self) -> int:
        return int(self._lib.infini_attn_window_tokens(self._h))

    # ------------------------------------------------------------------ measurement
    def profile_enable(self, enable: bool = True) -> None:
        _check("infini_attn_profile_enable", self._lib.infini_attn_profile_enable(self._h, int(enable)))

    def profile_read(self) -> dict:
        """{kernel kind: (total milliseconds, launches)} since the last enable/read."""
        p = Profile()
        _check("infini_attn_profile_read", self._lib.infini_attn_profile_read(self._h, ctypes.byref(p)))
        return {k: (p.total_ms[i], int(p.launches[i])) for i, k in enumerate(KERNEL_KINDS)}
