"""Python binding of liblorabwd (the C ABI in include/lorabwd.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks dtype / shape / contiguity, passes their device
pointers and the current HIP stream to the library, and raises LorabwdError
on a non-zero status.  No computation happens here, and there is no
fallback: if the library cannot be loaded every call raises.

Workspaces are torch uint8 tensors cached per (device, stream); the library
itself never allocates.  Calls on one stream share its workspace (they are
ordered by the stream); calls on different streams never share one.  A
workspace that grows is replaced, and the old buffer is kept alive (never
freed), because a HIP graph captured earlier may still write to it.  Under
graph capture the capture stream gets its own workspace, allocated from the
graph's memory pool and likewise kept alive; graphs captured on one stream
share it, so replaying two of them concurrently on different streams races.
"""
import ctypes
import os

__all__ = [
    "LorabwdError", "LayerDesc", "LayerWeights", "LayerSaved", "LoraState", "AdamW",
    "load_library", "lib_path",
    "lorabwd_rmsnorm_backward", "lorabwd_rope_backward", "lorabwd_attn_backward",
    "lorabwd_ffn_backward", "lorabwd_lora_grad_adamw", "lorabwd_layer_backward",
    "lorabwd_attn_workspace_size", "lorabwd_ffn_workspace_size",
    "lorabwd_lora_workspace_size", "lorabwd_layer_workspace_size", "lorabwd_status_string",
    "lorabwd_layer_backward_timed", "lorabwd_layer_backward_noalloc", "KernelRecord",
    "make_desc", "NOALLOC_SCRATCH_BYTES", "lorabwd_pack_ternary", "lorabwd_ternary_packed_bytes",
    "F32", "BF16", "ACT_SWIGLU", "ACT_RELU2",
]

F32, BF16 = 0, 1
ACT_SWIGLU, ACT_RELU2 = 0, 1
EXPORTS = [
    "lorabwd_status_string", "lorabwd_abi_version",
    "lorabwd_rmsnorm_backward", "lorabwd_rope_backward",
    "lorabwd_attn_workspace_size", "lorabwd_attn_backward",
    "lorabwd_ffn_workspace_size", "lorabwd_ffn_backward",
    "lorabwd_lora_workspace_size", "lorabwd_lora_grad_adamw",
    "lorabwd_layer_workspace_size", "lorabwd_layer_backward", "lorabwd_layer_backward_timed",
    "lorabwd_layer_backward_noalloc", "lorabwd_ternary_packed_bytes", "lorabwd_pack_ternary",
    "lorabwd_lm_head_workspace_size", "lorabwd_lm_head_backward", "lorabwd_lm_head_backward_timed",
]
NOALLOC_SCRATCH_BYTES = 16 << 20  # LORABWD_NOALLOC_SCRATCH_BYTES

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path():
    """liblorabwd.so built in-tree, or the build LORABWD_LIB names (the same
    library built differently, e.g. with host sanitizers)."""
    return os.environ.get("LORABWD_LIB") or os.path.join(_HERE, "liblorabwd.so")


class LorabwdError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %d (%s)" % (fn, status, _status_str(status)))


c_i64, c_int, c_float, c_size, c_vp = (ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_size_t, ctypes.c_void_p)


class LayerDesc(ctypes.Structure):
    _fields_ = [("seq", c_i64), ("kv_len", c_i64), ("hidden", c_i64), ("ffn", c_i64),
                ("n_heads", c_i64), ("n_kv_heads", c_i64), ("head_dim", c_i64), ("pos0", c_i64),
                ("act", ctypes.c_int32), ("sub_norms", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32), ("eps", c_float),
                ("rope_base", c_float), ("attn_scale", c_float), ("lora_alpha", c_float),
                ("qk_norm", ctypes.c_int32), ("input_grad", ctypes.c_int32),
                ("weight_format", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("w_o", c_vp), ("w_gate", c_vp), ("w_up", c_vp), ("w_down", c_vp),
                ("gamma_ffn", c_vp), ("gamma_fsub", c_vp), ("gamma_asub", c_vp), ("gamma_q", c_vp),
                ("w_q", c_vp), ("w_k", c_vp), ("w_v", c_vp), ("gamma_attn", c_vp),
                ("gamma_k", c_vp), ("scale_o", c_float), ("scale_gate", c_float),
                ("scale_up", c_float), ("scale_down", c_float)]


class LayerSaved(ctypes.Structure):
    _fields_ = [("attn_input", c_vp), ("resid1", c_vp), ("gate", c_vp), ("up", c_vp),
                ("hidden_pre", c_vp), ("ctx", c_vp), ("P", c_vp), ("K", c_vp), ("V", c_vp),
                ("lora_q_h", c_vp), ("lora_v_h", c_vp), ("q_raw", c_vp), ("x", c_vp), ("q", c_vp),
                ("k_raw", c_vp)]


class KernelRecord(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("alg_bytes", ctypes.c_double),
                ("alg_flops", ctypes.c_double), ("impl_bytes", ctypes.c_double)]


class LoraState(ctypes.Structure):
    _fields_ = [("rank", c_i64), ("A", c_vp), ("B", c_vp), ("m_a", c_vp), ("v_a", c_vp),
                ("m_b", c_vp), ("v_b", c_vp)]


class AdamW(ctypes.Structure):
    _fields_ = [("lr_a", c_float), ("lr_b", c_float), ("beta1", c_float), ("beta2", c_float),
                ("eps", c_float), ("weight_decay", c_float), ("step", ctypes.c_int32)]


_SIGS = {
    "lorabwd_status_string": (ctypes.c_char_p, [c_int]),
    "lorabwd_abi_version": (c_int, []),
    "lorabwd_rmsnorm_backward": (c_int, [c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_float, c_int,
                                         c_int, c_vp]),
    "lorabwd_rope_backward": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_float, c_vp]),
    "lorabwd_attn_workspace_size": (c_size, [c_i64, c_i64, c_i64, c_i64, c_i64, c_int]),
    "lorabwd_attn_backward": (c_int, [c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                                      c_vp, c_vp, c_vp, c_float, c_int, c_int, c_vp, c_size,
                                      c_vp]),
    "lorabwd_ffn_workspace_size": (c_size, [c_i64, c_i64, c_i64, c_int]),
    "lorabwd_ffn_backward": (c_int, [c_i64, c_i64, c_i64, c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_float, c_int, c_vp,
                                     c_size, c_vp]),
    "lorabwd_lora_workspace_size": (c_size, [c_i64, c_i64, c_i64, c_i64]),
    "lorabwd_lora_grad_adamw": (c_int, [c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_float,
                                        c_float, c_float, c_float, c_float, c_float, c_float,
                                        c_int, c_int, c_vp, c_size, c_vp]),
    "lorabwd_lm_head_workspace_size": (c_size, [c_i64, c_i64, c_i64]),
    "lorabwd_lm_head_backward": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                         c_vp, c_vp, c_vp, c_float, c_float, c_float, c_float,
                                         c_float, c_int, c_vp, c_size, c_vp]),
    "lorabwd_lm_head_backward_timed": (c_int, [
        c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_float,
        c_float, c_float, c_float, c_float, c_int, c_vp, c_size, c_vp, ctypes.POINTER(c_vp),
        ctypes.POINTER(KernelRecord), c_int, ctypes.POINTER(c_int)]),
    "lorabwd_layer_workspace_size": (c_size, [ctypes.POINTER(LayerDesc)]),
    "lorabwd_ternary_packed_bytes": (c_size, [c_i64, c_i64]),
    "lorabwd_pack_ternary": (c_int, [c_i64, c_i64, c_vp, c_int, c_vp, c_vp]),
    "lorabwd_layer_backward": (c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                       ctypes.POINTER(LayerSaved), ctypes.POINTER(LoraState),
                                       ctypes.POINTER(LoraState), ctypes.POINTER(AdamW), c_vp,
                                       c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "lorabwd_layer_backward_noalloc": (c_int, [
        ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerSaved),
        ctypes.POINTER(LoraState), ctypes.POINTER(LoraState), ctypes.POINTER(AdamW), c_vp, c_vp,
        c_vp, c_vp, c_vp, c_vp]),
    "lorabwd_layer_backward_timed": (c_int, [
        ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerSaved),
        ctypes.POINTER(LoraState), ctypes.POINTER(LoraState), ctypes.POINTER(AdamW), c_vp, c_vp,
        c_vp, c_vp, c_vp, c_vp, c_size, c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(KernelRecord),
        c_int,
        ctypes.POINTER(c_int)]),
}


def load_library(path=None):
    """Load liblorabwd.so (built in-tree by __graft_entry__.build()).  Raises
    OSError if it is missing: there is no fallback path."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or lib_path()
    if not os.path.exists(p):
        raise OSError("liblorabwd.so not found at %s; build it with "
                      "`python -c 'import __graft_entry__ as g; g.build()'`" % p)
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _LIB = lib
    return lib


def _status_str(status):
    try:
        return load_library().lorabwd_status_string(status).decode()
    except OSError:
        return "?"


def lorabwd_status_string(status):
    return _status_str(status)


def _check(fn, status):
    if status != 0:
        raise LorabwdError(fn, status)


# ---------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dt(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("activation tensors must be float32 or bfloat16, got %s" % t.dtype)


def _need(t, name, dtype=None, shape=None):
    torch = _torch()
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _f32(t, name, shape=None):
    return _need(t, name, _torch().float32, shape)


def _opt(t, name, dtype=None, shape=None):
    return None if t is None else _need(t, name, dtype, shape)


def _stream_obj(stream, device):
    torch = _torch()
    return torch.cuda.current_stream(device) if stream is None else stream


def _stream(stream, device=None):
    return _stream_obj(stream, device).cuda_stream


_WS = {}
_RETIRED = []  # superseded workspaces, kept alive for graphs captured with them


def _workspace(nbytes, device, stream=None):
    """The uint8 device workspace of (device, stream), at least nbytes (grown
    on demand; see the module docstring)."""
    torch = _torch()
    if nbytes == 0:
        return None, 0
    so = _stream_obj(stream, device)
    key = (str(device), so.cuda_stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _RETIRED.append(buf)
        with torch.cuda.stream(so):
            buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf, buf.numel()


# ---------------------------------------------------------------- entry points
def lorabwd_rmsnorm_backward(x, gamma, dy, dx, eps=1e-6, accumulate=False, stream=None):
    rows, n = dy.shape
    _need(x, "x", shape=(rows, n))
    _f32(gamma, "gamma", (n,))
    _f32(dy, "dy")
    _f32(dx, "dx", (rows, n))
    lib = load_library()
    _check("lorabwd_rmsnorm_backward", lib.lorabwd_rmsnorm_backward(
        rows, n, _ptr(x), _ptr(gamma), _ptr(dy), _ptr(dx), eps, int(bool(accumulate)), _dt(x),
        _stream(stream)))
    return dx


def lorabwd_rope_backward(dy, dx, n_heads, head_dim, pos0=0, base=10000.0, stream=None):
    rows = dy.shape[0]
    _f32(dy, "dy", (rows, n_heads * head_dim))
    _f32(dx, "dx", (rows, n_heads * head_dim))
    lib = load_library()
    _check("lorabwd_rope_backward", lib.lorabwd_rope_backward(
        rows, n_heads, head_dim, _ptr(dy), _ptr(dx), pos0, base, _stream(stream)))
    return dx


def lorabwd_ternary_packed_bytes(rows, cols):
    return load_library().lorabwd_ternary_packed_bytes(rows, cols)


def lorabwd_pack_ternary(w, packed=None, stream=None):
    """Packed ternary weights (the format of include/lorabwd.h) of w
    [rows, cols] (float32 or bfloat16), coded by sign: uint8 [rows, cols/4]."""
    rows, cols = w.shape
    _need(w, "w")
    if packed is None:
        packed = _torch().empty((rows, cols // 4), dtype=_torch().uint8, device=w.device)
    _need(packed, "packed", _torch().uint8, (rows, cols // 4))
    lib = load_library()
    _check("lorabwd_pack_ternary", lib.lorabwd_pack_ternary(
        rows, cols, _ptr(w), _dt(w), _ptr(packed), _stream(stream, w.device)))
    return packed


def lorabwd_attn_workspace_size(s_q, s_kv, n_heads, n_kv_heads, head_dim, dtype=F32):
    return load_library().lorabwd_attn_workspace_size(s_q, s_kv, n_heads, n_kv_heads, head_dim,
                                                      dtype)


def lorabwd_attn_backward(dctx, P, K, V, ctx, dq, dv, n_heads, n_kv_heads, head_dim, scale=None,
                          causal=True, stream=None):
    s_q = dctx.shape[0]
    s_kv = K.shape[0]
    _f32(dctx, "dctx", (s_q, n_heads * head_dim))
    dt = _dt(P)
    tdt = P.dtype
    _need(P, "P", tdt, (n_heads, s_q, s_kv))
    _need(K, "K", tdt, (s_kv, n_kv_heads * head_dim))
    _need(V, "V", tdt, (s_kv, n_kv_heads * head_dim))
    _opt(ctx, "ctx", tdt, (s_q, n_heads * head_dim))
    _f32(dq, "dq", (s_q, n_heads * head_dim))
    if dv is not None:
        _f32(dv, "dv", (s_kv, n_kv_heads * head_dim))
    if scale is None:
        scale = head_dim ** -0.5
    lib = load_library()
    need = lib.lorabwd_attn_workspace_size(s_q, s_kv, n_heads, n_kv_heads, head_dim, dt)
    ws, wsb = _workspace(need, dq.device, stream)
    _check("lorabwd_attn_backward", lib.lorabwd_attn_backward(
        s_q, s_kv, n_heads, n_kv_heads, head_dim, _ptr(dctx), _ptr(P), _ptr(K), _ptr(V),
        _ptr(ctx), _ptr(dq), _ptr(dv), scale, int(bool(causal)), dt, _ptr(ws), wsb,
        _stream(stream, dq.device)))
    return dq, dv


def lorabwd_ffn_workspace_size(rows, dim, ffn_dim, dtype=F32):
    return load_library().lorabwd_ffn_workspace_size(rows, dim, ffn_dim, dtype)


def lorabwd_ffn_backward(d_out, w_down, w_gate, w_up, gate, up, resid1, gamma_ffn, d_resid,
                         act=ACT_SWIGLU, hidden_pre=None, gamma_sub=None, eps=1e-6, stream=None):
    rows, dim = d_out.shape
    ffn = gate.shape[1]
    dt = _dt(gate)
    tdt = gate.dtype
    _f32(d_out, "d_out")
    _need(w_down, "w_down", tdt, (dim, ffn))
    _need(w_gate, "w_gate", tdt, (ffn, dim))
    _need(w_up, "w_up", tdt, (ffn, dim))
    _need(gate, "gate", tdt, (rows, ffn))
    _need(up, "up", tdt, (rows, ffn))
    _need(resid1, "resid1", tdt, (rows, dim))
    _opt(hidden_pre, "hidden_pre", tdt, (rows, ffn))
    _opt(gamma_sub, "gamma_sub", _torch().float32, (ffn,))
    _f32(gamma_ffn, "gamma_ffn", (dim,))
    _f32(d_resid, "d_resid", (rows, dim))
    lib = load_library()
    need = lib.lorabwd_ffn_workspace_size(rows, dim, ffn, dt)
    ws, wsb = _workspace(need, d_out.device, stream)
    _check("lorabwd_ffn_backward", lib.lorabwd_ffn_backward(
        rows, dim, ffn, act, _ptr(d_out), _ptr(w_down), _ptr(w_gate), _ptr(w_up), _ptr(gate),
        _ptr(up), _ptr(hidden_pre), _ptr(gamma_sub), _ptr(resid1), _ptr(gamma_ffn),
        _ptr(d_resid), eps, dt, _ptr(ws), wsb, _stream(stream, d_out.device)))
    return d_resid


def lorabwd_lora_workspace_size(rows, in_dim, out_dim, rank):
    return load_library().lorabwd_lora_workspace_size(rows, in_dim, out_dim, rank)


def lorabwd_lora_grad_adamw(dy, x, h, A, B, m_a, v_a, m_b, v_b, alpha, lr_a, lr_b,
                            beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1,
                            grad_a=None, grad_b=None, gnorm_sq=None, stream=None):
    rows, in_dim = x.shape
    rank = A.shape[0]
    out_dim = B.shape[0]
    dt = _dt(x)
    _f32(dy, "dy", (rows, out_dim))
    _need(h, "h", x.dtype, (rows, rank))
    for t, n, s in ((A, "A", (rank, in_dim)), (m_a, "m_a", (rank, in_dim)),
                    (v_a, "v_a", (rank, in_dim)), (B, "B", (out_dim, rank)),
                    (m_b, "m_b", (out_dim, rank)), (v_b, "v_b", (out_dim, rank))):
        _f32(t, n, s)
    if grad_a is not None:
        _f32(grad_a, "grad_a", (rank, in_dim))
    if grad_b is not None:
        _f32(grad_b, "grad_b", (out_dim, rank))
    if gnorm_sq is not None:
        _f32(gnorm_sq, "gnorm_sq", (1,))
    lib = load_library()
    need = lib.lorabwd_lora_workspace_size(rows, in_dim, out_dim, rank)
    ws, wsb = _workspace(need, dy.device, stream)
    _check("lorabwd_lora_grad_adamw", lib.lorabwd_lora_grad_adamw(
        rows, in_dim, out_dim, rank, _ptr(dy), _ptr(x), _ptr(h), _ptr(A), _ptr(B), _ptr(m_a),
        _ptr(v_a), _ptr(m_b), _ptr(v_b), _ptr(grad_a), _ptr(grad_b), _ptr(gnorm_sq), alpha, lr_a,
        lr_b, beta1, beta2, eps, weight_decay, step, dt, _ptr(ws), wsb, _stream(stream, dy.device)))


def lorabwd_lm_head_workspace_size(rows, hidden, vocab):
    return load_library().lorabwd_lm_head_workspace_size(rows, hidden, vocab)


def lorabwd_lm_head_backward(h, logits, labels, W, m, v, grad_hidden, loss, lr, beta1=0.9,
                             beta2=0.999, eps=1e-8, weight_decay=0.01, step=1, grad_w=None,
                             stream=None, timing=None):
    """lm_head backward with AdamW on W (updated in place with m and v):
    grad_hidden [rows, hidden] and loss [1] are written.  h, logits, W, m,
    v float32; labels int32 (a label outside [0, vocab) ignores its row).
    `timing` = (events, records) as for the layer: per-kernel HIP events
    recorded on the call's stream."""
    torch = _torch()
    rows, hidden = h.shape
    vocab = W.shape[0]
    _f32(h, "h", (rows, hidden))
    _f32(logits, "logits", (rows, vocab))
    _need(labels, "labels", torch.int32, (rows,))
    for t, n in ((W, "W"), (m, "m"), (v, "v")):
        _f32(t, n, (vocab, hidden))
    _f32(grad_hidden, "grad_hidden", (rows, hidden))
    _f32(loss, "loss", (1,))
    _opt(grad_w, "grad_w", torch.float32, (vocab, hidden))
    lib = load_library()
    need = lib.lorabwd_lm_head_workspace_size(rows, hidden, vocab)
    ws, wsb = _workspace(need, h.device, stream)
    args = (rows, hidden, vocab, _ptr(h), _ptr(logits), _ptr(labels), _ptr(W), _ptr(m), _ptr(v),
            _ptr(grad_hidden), _ptr(loss), _ptr(grad_w), lr, beta1, beta2, eps, weight_decay,
            step, _ptr(ws), wsb, _stream(stream, h.device))
    if timing is None:
        _check("lorabwd_lm_head_backward", lib.lorabwd_lm_head_backward(*args))
        return None
    events, records = timing
    n = ctypes.c_int(0)
    _check("lorabwd_lm_head_backward_timed", lib.lorabwd_lm_head_backward_timed(
        *args, events, records, len(records), ctypes.byref(n)))
    return n.value


def lorabwd_layer_backward_timed(desc, weights, saved, d_hidden, events, records, **kw):
    return lorabwd_layer_backward(desc, weights, saved, d_hidden, timing=(events, records), **kw)


def lorabwd_layer_workspace_size(desc):
    return load_library().lorabwd_layer_workspace_size(ctypes.byref(desc))


def make_desc(seq, kv_len, hidden, ffn, n_heads, n_kv_heads, head_dim, act=ACT_SWIGLU,
              sub_norms=False, causal=True, dtype=F32, pos0=0, eps=1e-6, rope_base=10000.0,
              attn_scale=None, lora_alpha=0.0, qk_norm=False, input_grad=False,
              weight_format=0):
    return LayerDesc(seq, kv_len, hidden, ffn, n_heads, n_kv_heads, head_dim, pos0, act,
                     int(sub_norms), int(causal), dtype, eps, rope_base,
                     head_dim ** -0.5 if attn_scale is None else attn_scale, lora_alpha,
                     int(qk_norm), int(input_grad), int(weight_format), 0)


def lorabwd_layer_backward_noalloc(desc, weights, saved, d_hidden, **kw):
    """lorabwd_layer_backward on the library's static per-device scratch (no
    workspace is allocated; see include/lorabwd.h for its size limit)."""
    return lorabwd_layer_backward(desc, weights, saved, d_hidden, noalloc=True, **kw)


def lorabwd_layer_backward(desc, weights, saved, d_hidden, q_state=None, v_state=None,
                           adamw=None, dq_pre_out=None, dv_out=None, gnorm_sq=None,
                           stream=None, timing=None, d_out=None, noalloc=False):
    """desc: LayerDesc; weights / saved: dicts of tensors keyed like the C
    structs; q_state / v_state: dicts with A, B, m_a, v_a, m_b, v_b (or None);
    adamw: AdamW or None.  d_hidden receives dH1; it is also the input (the
    gradient of the layer output, updated in place) unless d_out is given.

    timing: None, or (events, records) = (ctypes array of hipEvent_t,
    ctypes array of KernelRecord) to call lorabwd_layer_backward_timed; the
    number of kernels enqueued is then returned.  noalloc: call
    lorabwd_layer_backward_noalloc instead (no timing)."""
    if noalloc and timing is not None:
        raise ValueError("noalloc calls are not timed")
    d = desc
    tdt = _torch().bfloat16 if d.dtype == BF16 else _torch().float32
    S, L, H, I = d.seq, d.kv_len, d.hidden, d.ffn
    qd, kvd = d.n_heads * d.head_dim, d.n_kv_heads * d.head_dim
    _f32(d_hidden, "d_hidden", (S, H))
    if d_out is not None:
        _f32(d_out, "d_out", (S, H))
    wshapes = {"w_o": (H, qd), "w_gate": (I, H), "w_up": (I, H), "w_down": (H, I)}
    for k, s in wshapes.items():
        if d.weight_format == 1:  # packed ternary: uint8 [out, in / 4]
            _need(weights[k], k, _torch().uint8, (s[0], s[1] // 4))
        else:
            _need(weights[k], k, tdt, s)
    _f32(weights["gamma_ffn"], "gamma_ffn", (H,))
    if d.sub_norms:
        _f32(weights["gamma_fsub"], "gamma_fsub", (I,))
        _f32(weights["gamma_asub"], "gamma_asub", (qd,))
    if d.qk_norm:
        _f32(weights["gamma_q"], "gamma_q", (d.head_dim,))
    if d.input_grad:
        for k, s in (("w_q", (qd, H)), ("w_k", (kvd, H)), ("w_v", (kvd, H))):
            _need(weights[k], k, tdt, s)
        _f32(weights["gamma_attn"], "gamma_attn", (H,))
        if d.qk_norm:
            _f32(weights["gamma_k"], "gamma_k", (d.head_dim,))
    sshapes = {"attn_input": (S, H), "resid1": (S, H), "gate": (S, I), "up": (S, I),
               "hidden_pre": (S, I), "ctx": (S, qd), "P": (d.n_heads, S, L), "K": (L, kvd),
               "V": (L, kvd), "q_raw": (S, qd), "x": (S, H), "q": (S, qd), "k_raw": (S, kvd)}
    for k, s in sshapes.items():
        if saved.get(k) is not None:
            _need(saved[k], k, tdt, s)
    w = LayerWeights(*[float(weights.get(k, 1.0)) if t is c_float else _ptr(weights.get(k))
                       for k, t in LayerWeights._fields_])
    a = LayerSaved(*[_ptr(saved.get(k)) for k, _ in LayerSaved._fields_])

    def state(st, out_dim, hkey):
        if st is None:
            return None
        r = st["A"].shape[0]
        for k, s in (("A", (r, H)), ("m_a", (r, H)), ("v_a", (r, H)), ("B", (out_dim, r)),
                     ("m_b", (out_dim, r)), ("v_b", (out_dim, r))):
            _f32(st[k], k, s)
        _need(saved[hkey], hkey, tdt, (S, r))
        return LoraState(r, *[_ptr(st[k]) for k in ("A", "B", "m_a", "v_a", "m_b", "v_b")])

    qs = state(q_state, qd, "lora_q_h")
    vs = state(v_state, kvd, "lora_v_h")
    if dq_pre_out is not None:
        _f32(dq_pre_out, "dq_pre_out", (S, qd))
    if dv_out is not None:
        _f32(dv_out, "dv_out", (L, kvd))
    if gnorm_sq is not None:
        _f32(gnorm_sq, "gnorm_sq", (1,))
    lib = load_library()
    head = (ctypes.byref(d), ctypes.byref(w), ctypes.byref(a),
            ctypes.byref(qs) if qs is not None else None,
            ctypes.byref(vs) if vs is not None else None,
            ctypes.byref(adamw) if adamw is not None else None,
            _ptr(d_out), _ptr(d_hidden), _ptr(dq_pre_out), _ptr(dv_out), _ptr(gnorm_sq))
    if noalloc:
        _check("lorabwd_layer_backward_noalloc", lib.lorabwd_layer_backward_noalloc(
            *head, _stream(stream, d_hidden.device)))
        return d_hidden
    need = lib.lorabwd_layer_workspace_size(ctypes.byref(d))
    ws, wsb = _workspace(need, d_hidden.device, stream)
    args = head + (_ptr(ws), wsb, _stream(stream, d_hidden.device))
    if timing is None:
        _check("lorabwd_layer_backward", lib.lorabwd_layer_backward(*args))
        return d_hidden
    events, records = timing
    n = ctypes.c_int(0)
    _check("lorabwd_layer_backward_timed", lib.lorabwd_layer_backward_timed(
        *args, events, records, len(records), ctypes.byref(n)))
    return n.value
