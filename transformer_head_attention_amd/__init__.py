"""MI355X (gfx950) multi-head attention forward pass: Python binding.

A thin ctypes layer over ``libmha.so``, whose C ABI is declared in
``include/mha.h``. The functions below carry the C names and only marshal
arguments; every step of the computation runs in the library's HIP kernels.
torch is used for device memory and streams only.

There is no fallback: if ``libmha.so`` has not been built, importing this
package raises ImportError.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmha.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(hipcc, gfx950). The multi-head attention path has no CPU fallback.")

# torch ships its own HIP runtime with the same soname (libamdhip64.so.7).
# Loading torch first makes libmha.so bind to that one runtime, so device
# pointers and streams handed over from torch are valid for the library.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

MHA_F32, MHA_BF16 = 0, 1
MHA_OK, MHA_ERR_INVALID_ARG, MHA_ERR_UNSUPPORTED, MHA_ERR_WORKSPACE, MHA_ERR_HIP = range(5)
MHA_NUM_STAGES = 5

MHA_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("mha_create", "mha_create_grouped", "mha_workspace_size", "mha_forward",
            "mha_forward_ex", "mha_forward_noalloc", "mha_destroy",
            "mha_decode_workspace_size", "mha_decode",
            "mha_status_string", "mha_hip_error_string", "mha_profile_begin", "mha_profile_end",
            "mha_stage_name")

_vp, _int, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_lib.mha_create.argtypes = [ctypes.POINTER(_vp), _int, _int, _int]
_lib.mha_create.restype = _int
_lib.mha_create_grouped.argtypes = [ctypes.POINTER(_vp), _int, _int, _int, _int]
_lib.mha_create_grouped.restype = _int
_lib.mha_workspace_size.argtypes = [_vp, _int, _int, _int]
_lib.mha_workspace_size.restype = _sz
_lib.mha_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp,
                             _vp, _vp, _sz, _vp]
_lib.mha_forward.restype = _int


class mha_forward_options(ctypes.Structure):
    _fields_ = [("residual", ctypes.c_int), ("y_bf16", ctypes.c_int),
                ("attn_weights", ctypes.c_void_p), ("average_weights", ctypes.c_int),
                ("gate_w", ctypes.c_void_p), ("gate_b", ctypes.c_void_p),
                ("fp16_overflow", ctypes.c_void_p)]


_lib.mha_forward_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp,
                                _vp, _vp, _sz, ctypes.POINTER(mha_forward_options), _vp]
_lib.mha_forward_ex.restype = _int
_lib.mha_forward_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                                     _vp, _vp, ctypes.POINTER(mha_forward_options), _vp]
_lib.mha_forward_noalloc.restype = _int
_lib.mha_decode_workspace_size.argtypes = [_vp, _int, _int, _int]
_lib.mha_decode_workspace_size.restype = _sz
_lib.mha_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _vp, _vp, _int, _vp, _vp,
                            _vp, _sz, _vp]
_lib.mha_decode.restype = _int
_lib.mha_destroy.argtypes = [_vp]
_lib.mha_destroy.restype = _int
_lib.mha_status_string.argtypes = [_int]
_lib.mha_status_string.restype = ctypes.c_char_p
_lib.mha_hip_error_string.argtypes = []
_lib.mha_hip_error_string.restype = ctypes.c_char_p
_lib.mha_profile_begin.argtypes = [_vp, _int]
_lib.mha_profile_begin.restype = _int
_lib.mha_profile_end.argtypes = [_vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_int)]
_lib.mha_profile_end.restype = _int
_lib.mha_stage_name.argtypes = [_int]
_lib.mha_stage_name.restype = ctypes.c_char_p


class MHAError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {mha_status_string(status)}"
        if status == MHA_ERR_HIP:
            msg += f" ({mha_hip_error_string()})"
        super().__init__(msg)
        self.status = status


def _check(status: int, where: str) -> None:
    if status != MHA_OK:
        raise MHAError(status, where)


# ---- C names ---------------------------------------------------------------

def mha_status_string(status: int) -> str:
    return _lib.mha_status_string(int(status)).decode()


def mha_hip_error_string() -> str:
    return _lib.mha_hip_error_string().decode()


def mha_stage_name(stage: int):
    s = _lib.mha_stage_name(int(stage))
    return None if s is None else s.decode()


def mha_create(d_model: int, num_heads: int, dtype: int):
    """Returns (status, handle); handle is None on error."""
    h = _vp()
    st = _lib.mha_create(ctypes.byref(h), int(d_model), int(num_heads), int(dtype))
    return st, (h.value if st == MHA_OK else None)


def mha_create_grouped(d_model: int, num_heads: int, num_kv_heads: int, dtype: int):
    """Returns (status, handle); handle is None on error."""
    h = _vp()
    st = _lib.mha_create_grouped(ctypes.byref(h), int(d_model), int(num_heads),
                                 int(num_kv_heads), int(dtype))
    return st, (h.value if st == MHA_OK else None)


def mha_workspace_size(handle, B: int, T_q: int, T_k: int) -> int:
    return int(_lib.mha_workspace_size(handle, int(B), int(T_q), int(T_k)))


def mha_forward(handle, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, B, T_q, T_k, causal,
                key_padding_mask, y, workspace, workspace_bytes, stream) -> int:
    """Raw call: every pointer argument is an int device address (or 0/None)."""
    return _lib.mha_forward(handle, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, int(B), int(T_q),
                            int(T_k), int(causal), key_padding_mask, y, workspace,
                            int(workspace_bytes), stream)


def mha_decode_workspace_size(handle, B: int, T_new: int, T_max: int) -> int:
    return int(_lib.mha_decode_workspace_size(handle, int(B), int(T_new), int(T_max)))


def mha_decode(handle, x, w_qkv, b_qkv, w_o, b_o, B, T_new, k_cache, v_cache, T_max, cache_len,
               y, workspace, workspace_bytes, stream) -> int:
    """Raw call: every pointer argument is an int device address (or 0/None)."""
    return _lib.mha_decode(handle, x, w_qkv, b_qkv, w_o, b_o, int(B), int(T_new), k_cache,
                           v_cache, int(T_max), cache_len, y, workspace, int(workspace_bytes),
                           stream)


def mha_forward_ex(handle, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, B, T_q, T_k, causal,
                   key_padding_mask, y, workspace, workspace_bytes, opts, stream) -> int:
    """Raw call; ``opts`` is an mha_forward_options or None."""
    return _lib.mha_forward_ex(handle, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, int(B), int(T_q),
                               int(T_k), int(causal), key_padding_mask, y, workspace,
                               int(workspace_bytes), None if opts is None else ctypes.byref(opts),
                               stream)


def mha_forward_noalloc(handle, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, B, T_q, T_k, causal,
                        key_padding_mask, y, opts, stream) -> int:
    """Raw call; ``opts`` is an mha_forward_options or None. No workspace: the
    library's own per-GPU scratch of MHA_NOALLOC_SCRATCH_BYTES is used."""
    return _lib.mha_forward_noalloc(handle, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, int(B), int(T_q),
                                    int(T_k), int(causal), key_padding_mask, y,
                                    None if opts is None else ctypes.byref(opts), stream)


def mha_destroy(handle) -> int:
    return _lib.mha_destroy(handle)


def mha_profile_begin(handle, max_calls: int) -> int:
    return _lib.mha_profile_begin(handle, int(max_calls))


def mha_profile_end(handle):
    """Returns (status, {stage name: average ms}, n_calls)."""
    arr = (ctypes.c_float * MHA_NUM_STAGES)()
    n = _int(0)
    st = _lib.mha_profile_end(handle, arr, ctypes.byref(n))
    return st, {mha_stage_name(i): float(arr[i]) for i in range(MHA_NUM_STAGES)}, n.value


# ---- torch-tensor convenience wrapper (marshalling only) ---------------------

class MultiHeadAttention:
    """Holds an ``mha_handle_t`` for (d_model, num_heads, dtype) and calls
    ``mha_forward`` on torch CUDA tensors.

    dtype is "bf16" (bf16 inputs/weights, fp32 output) or "fp32".
    num_kv_heads (default num_heads) selects grouped key/value heads; W_QKV
    is then (d_model, d_model + 2 * num_kv_heads * d_k).
    """

    def __init__(self, d_model: int, num_heads: int, dtype: str = "bf16",
                 num_kv_heads: int = None):
        import torch
        self._torch = torch
        self.d_model, self.num_heads = d_model, num_heads
        self.num_kv_heads = num_heads if num_kv_heads is None else num_kv_heads
        self.dtype = dtype
        self._tdtype = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
        st, h = mha_create_grouped(d_model, num_heads, self.num_kv_heads,
                                   MHA_BF16 if dtype == "bf16" else MHA_F32)
        _check(st, "mha_create_grouped")
        self.handle = h
        self._ws = None
        self._uses = []

    def close(self):
        if self.handle is not None:
            mha_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, B: int, T_q: int, T_k: int) -> int:
        return mha_workspace_size(self.handle, B, T_q, T_k)

    def workspace(self, B: int, T_q: int, T_k: int, device):
        n = self.workspace_size(B, T_q, T_k)
        if n == 0:
            raise MHAError(MHA_ERR_INVALID_ARG, "mha_workspace_size")
        if self._ws is None or self._ws.numel() < n or self._ws.device != device:
            self._ws = self._torch.empty(n, dtype=self._torch.uint8, device=device)
        return self._ws

    def _ptr(self, t, dtype=None):
        if t is None:
            return None
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous CUDA tensors")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"expected {dtype}, got {t.dtype}")
        return t.data_ptr()

    def _check_shapes(self, x_q, w_qkv, w_o, b_qkv, b_o, x_kv, key_padding_mask, out,
                      gate_w=None, gate_b=None):
        D = self.d_model
        n_qkv = D + 2 * self.num_kv_heads * (D // self.num_heads)
        B, T_q = x_q.shape[0], x_q.shape[1]
        T_k = T_q if x_kv is None else x_kv.shape[1]
        want = [(x_q, (B, T_q, D)), (w_qkv, (D, n_qkv)), (w_o, (D, D)), (b_qkv, (n_qkv,)),
                (b_o, (D,)), (x_kv, (B, T_k, D)), (key_padding_mask, (B, T_k)),
                (out, (B, T_q, D)), (gate_w, (D, self.num_heads)), (gate_b, (self.num_heads,))]
        for t, shape in want:
            if t is not None and tuple(t.shape) != shape:
                raise ValueError(f"expected shape {shape}, got {tuple(t.shape)}")

    def forward(self, x_q, w_qkv, w_o, b_qkv=None, b_o=None, x_kv=None, causal=False,
                key_padding_mask=None, out=None, workspace=None, stream=None, residual=False,
                y_dtype="fp32", attn_weights=None, average_weights=False, gate_w=None,
                gate_b=None, fp16_overflow=None):
        """Returns y. ``residual`` adds x_q; ``y_dtype`` "bf16" stores y as
        bf16; ``attn_weights`` (a (B, h, T_q, T_k) fp32 tensor, or (B, T_q,
        T_k) with ``average_weights``) receives the softmax weights;
        ``gate_w`` (D, h) and ``gate_b`` (h,) select gated attention;
        ``fp16_overflow`` (an int32 device tensor of one element) is set to 1
        if a value stored in fp16 is not finite (never cleared here)."""
        torch = self._torch
        if x_q.dim() != 3:
            raise ValueError("x_q must be (B, T, D)")
        self._check_shapes(x_q, w_qkv, w_o, b_qkv, b_o, x_kv, key_padding_mask, out, gate_w,
                           gate_b)
        B, T_q, D = x_q.shape
        T_k = T_q if x_kv is None else x_kv.shape[1]
        ydt = {"fp32": torch.float32, "bf16": torch.bfloat16}[y_dtype]
        if out is None:
            out = torch.empty(B, T_q, D, dtype=ydt, device=x_q.device)
        if attn_weights is not None:
            want = (B, T_q, T_k) if average_weights else (B, self.num_heads, T_q, T_k)
            if tuple(attn_weights.shape) != want:
                raise ValueError(f"attn_weights must be {want}")
        if workspace is None:
            workspace = self.workspace(B, T_q, T_k, x_q.device)
        if key_padding_mask is not None and key_padding_mask.dtype != torch.uint8:
            key_padding_mask = key_padding_mask.to(torch.uint8)
        if stream is None:
            stream = torch.cuda.current_stream(x_q.device).cuda_stream
        # buffers allocated here belong to the current stream; when the
        # kernels run on another one they are recorded on it below
        self._uses = [out, workspace, key_padding_mask]
        dt = self._tdtype
        args = (self.handle, self._ptr(x_q, dt), self._ptr(x_kv, dt), self._ptr(w_qkv, dt),
                self._ptr(b_qkv, dt), self._ptr(w_o, dt), self._ptr(b_o, dt), B, T_q, T_k,
                1 if causal else 0, self._ptr(key_padding_mask), self._ptr(out, ydt),
                workspace.data_ptr(), workspace.numel())
        if fp16_overflow is not None and fp16_overflow.numel() != 1:
            raise ValueError("fp16_overflow must hold one int32")
        if (not residual and y_dtype == "fp32" and attn_weights is None and gate_w is None
                and fp16_overflow is None):
            st = mha_forward(*args, stream)
            _check(st, "mha_forward")
        else:
            opts = mha_forward_options(1 if residual else 0, 1 if y_dtype == "bf16" else 0,
                                       self._ptr(attn_weights, torch.float32),
                                       1 if average_weights else 0, self._ptr(gate_w, dt),
                                       self._ptr(gate_b, dt),
                                       self._ptr(fp16_overflow, torch.int32))
            st = mha_forward_ex(*args, opts, stream)
            _check(st, "mha_forward_ex")
        self._record(stream, x_q.device)
        return out

    def _record(self, stream, device):
        """Mark the buffers the call used as in use by `stream` if that is not
        the current stream: the caching allocator then keeps their memory
        until the work queued there has finished, even if they are freed (or
        the cached workspace replaced) on the current stream meanwhile."""
        torch = self._torch
        uses, self._uses = self._uses, []
        if stream == torch.cuda.current_stream(device).cuda_stream:
            return
        ext = torch.cuda.ExternalStream(stream, device=device)
        for t in uses:
            if t is not None:
                t.record_stream(ext)

    __call__ = forward

    def decode(self, x, w_qkv, w_o, k_cache, v_cache, cache_len, b_qkv=None, b_o=None, out=None,
               workspace=None, stream=None):
        """One generation step: x (B, T_new, D) bf16; k_cache, v_cache
        (B, num_kv_heads, T_max, d_k) bf16, rows [len, len + T_new) written;
        cache_len (B,) int32 on the device, not modified. Returns y (B, T_new, D)
        fp32."""
        torch = self._torch
        if x.dim() != 3:
            raise ValueError("x must be (B, T_new, D)")
        B, T_new, D = x.shape
        d_k = D // self.num_heads
        if k_cache.dim() != 4:
            raise ValueError("caches must be (B, num_kv_heads, T_max, d_k)")
        T_max = k_cache.shape[2]
        self._check_shapes(x, w_qkv, w_o, b_qkv, b_o, None, None, out)
        for c in (k_cache, v_cache):
            if tuple(c.shape) != (B, self.num_kv_heads, T_max, d_k):
                raise ValueError(f"cache shape {tuple(c.shape)} != "
                                 f"{(B, self.num_kv_heads, T_max, d_k)}")
        if tuple(cache_len.shape) != (B,) or cache_len.dtype != torch.int32:
            raise ValueError("cache_len must be an int32 tensor of shape (B,)")
        if out is None:
            out = torch.empty(B, T_new, D, dtype=torch.float32, device=x.device)
        n = mha_decode_workspace_size(self.handle, B, T_new, T_max)
        if n == 0:
            raise MHAError(MHA_ERR_INVALID_ARG, "mha_decode_workspace_size")
        if workspace is None:
            if self._ws is None or self._ws.numel() < n or self._ws.device != x.device:
                self._ws = torch.empty(n, dtype=torch.uint8, device=x.device)
            workspace = self._ws
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        self._uses = [out, workspace]
        dt = self._tdtype
        st = mha_decode(self.handle, self._ptr(x, dt), self._ptr(w_qkv, dt), self._ptr(b_qkv, dt),
                        self._ptr(w_o, dt), self._ptr(b_o, dt), B, T_new, self._ptr(k_cache, dt),
                        self._ptr(v_cache, dt), T_max, self._ptr(cache_len, torch.int32),
                        self._ptr(out, torch.float32), workspace.data_ptr(), workspace.numel(),
                        stream)
        _check(st, "mha_decode")
        self._record(stream, x.device)
        return out
