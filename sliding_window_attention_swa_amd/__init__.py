"""Python binding of libswa.so, the gfx950 sliding-window attention library.

Argument marshalling only: every function checks shapes, dtypes and devices
of torch tensors, then passes raw device pointers and the current HIP stream
to the C ABI declared in include/swa.h.  All arithmetic runs in the HIP
kernels; there is no fallback.  If the library has not been built, every call
raises.

Layouts (contiguous, head-major):
  prefill  q, out [B, Hq, T, d]   k, v [B, Hkv, T, d]
  ring     k_ring, v_ring [B, Hkv, W, d]   k_new, v_new [B, Hkv, d]   pos [B] int32
  decode   q, out [B, Hq, d]
  chunk    q, out [B, Hq, n, d]   k, v [B, Hkv, n, d]   (n new tokens per sequence)
"""

import ctypes
import math
import os

CAUSAL = 0
SYMMETRIC = 1

SWA_F32 = 0
SWA_BF16 = 1

# the in-tree build; no other library is ever loaded
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswa.so")

_lib = None


class SwaError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))


def load():
    """Load libswa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libswa.so not found at %s; build it with "
                           "`python -m sliding_window_attention_swa_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.swa_prefill.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.swa_prefill.restype = i
    lib.swa_prefill_dilated.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.swa_prefill_dilated.restype = i
    lib.swa_prefill_global.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, vp, sz, i, vp]
    lib.swa_prefill_global.restype = i
    lib.swa_prefill_dilated_global.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, vp,
                                               sz, i, vp]
    lib.swa_prefill_dilated_global.restype = i
    lib.swa_cache_append.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.swa_cache_append.restype = i
    lib.swa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.swa_decode.restype = i
    lib.swa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.swa_decode_noalloc.restype = i
    lib.swa_cache_append_chunk.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.swa_cache_append_chunk.restype = i
    lib.swa_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.swa_prefill_chunk.restype = i
    lib.swa_decode_sinks.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.swa_decode_sinks.restype = i
    lib.swa_decode_sinks_workspace_bytes.argtypes = [i, i, i, i]
    lib.swa_decode_sinks_workspace_bytes.restype = sz
    lib.swa_prefill_global_workspace_bytes.argtypes = [i, i, i, i]
    lib.swa_prefill_global_workspace_bytes.restype = sz
    lib.swa_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.swa_decode_workspace_bytes.restype = sz
    lib.swa_calib_mfma_bf16.argtypes = [vp, sz, vp, i, i, vp]
    lib.swa_calib_mfma_bf16.restype = i
    lib.swa_calib_stream_read.argtypes = [vp, sz, vp, i, vp]
    lib.swa_calib_stream_read.restype = i
    lib.swa_calib_vector.argtypes = [i, vp, i, i, vp]
    lib.swa_calib_vector.restype = i
    lib.swa_status_string.argtypes = [i]
    lib.swa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status):
    return load().swa_status_string(int(status)).decode()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _check(t, name, ndim, dtype=None):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))


def _same_device(**tensors):
    """Every tensor of one call on the same device (the C ABI sees only
    pointers and cannot tell)."""
    devs = {t.device for t in tensors.values() if t is not None}
    if len(devs) > 1:
        raise ValueError("tensors on different devices: %s" % ", ".join(
            "%s=%s" % (n, t.device) for n, t in tensors.items() if t is not None))


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _raise(fn, status):
    if status != 0:
        raise SwaError(fn, status)


def prefill(q, k, v, W, mode=CAUSAL, scale=None, out=None, stream=None):
    """Windowed attention over whole sequences; returns `out` [B, Hq, T, d]."""
    import torch
    _check(q, "q", 4)
    _check(k, "k", 4, q.dtype)
    _check(v, "v", 4, q.dtype)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, T, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch q%s k%s v%s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", 4, q.dtype)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _same_device(q=q, k=k, v=v, out=out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = load().swa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), T, int(W),
                            B * Hq, B * Hkv, d, int(mode), float(scale), _dtype_code(q),
                            _stream(stream))
    _raise("swa_prefill", st)
    return out


def prefill_dilated(q, k, v, W, dilation, mode=CAUSAL, scale=None, out=None, stream=None):
    """Windowed attention with keys `dilation` apart in the window; returns
    `out` [B, Hq, T, d].  dilation=1 is `prefill`."""
    import torch
    _check(q, "q", 4)
    _check(k, "k", 4, q.dtype)
    _check(v, "v", 4, q.dtype)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, T, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch q%s k%s v%s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", 4, q.dtype)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _same_device(q=q, k=k, v=v, out=out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = load().swa_prefill_dilated(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), T,
                                    int(W), B * Hq, B * Hkv, d, int(mode), float(scale),
                                    int(dilation), _dtype_code(q), _stream(stream))
    _raise("swa_prefill_dilated", st)
    return out


def prefill_global(q, k, v, W, global_pos, mode=CAUSAL, scale=None, out=None, workspace=None,
                   stream=None, dilation=1):
    """Windowed attention plus global tokens at the positions `global_pos`
    (device int32 [G], strictly increasing): they attend to every key and
    every row attends to them (j <= i when causal).  With dilation > 1 the
    window is the dilated one of `prefill_dilated`.  Returns out [B, Hq, T, d]."""
    import torch
    _check(q, "q", 4)
    _check(k, "k", 4, q.dtype)
    _check(v, "v", 4, q.dtype)
    _check(global_pos, "global_pos", 1, torch.int32)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, T, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch q%s k%s v%s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", 4, q.dtype)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _same_device(q=q, k=k, v=v, global_pos=global_pos, out=out, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    G = global_pos.shape[0]
    if workspace is None:
        workspace = global_workspace(T, B * Hq, G, d, q.device)
    st = load().swa_prefill_dilated_global(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           out.data_ptr(), T, int(W), B * Hq, B * Hkv, d,
                                           int(mode), float(scale), int(dilation),
                                           global_pos.data_ptr() if G else None, G,
                                           workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(),
                                           _dtype_code(q), _stream(stream))
    _raise("swa_prefill_dilated_global", st)
    return out


def cache_append(k_ring, v_ring, pos, k_new, v_new, stream=None):
    """Write k_new/v_new [B, Hkv, d] into slot pos[b] mod W of the rings."""
    import torch
    _check(k_ring, "k_ring", 4)
    _check(v_ring, "v_ring", 4, k_ring.dtype)
    _check(pos, "pos", 1, torch.int32)
    _check(k_new, "k_new", 3, k_ring.dtype)
    _check(v_new, "v_new", 3, k_ring.dtype)
    B, Hkv, W, d = k_ring.shape
    if tuple(v_ring.shape) != tuple(k_ring.shape) or tuple(k_new.shape) != (B, Hkv, d) \
            or tuple(v_new.shape) != (B, Hkv, d) or pos.shape[0] != B:
        raise ValueError("shape mismatch")
    _same_device(k_ring=k_ring, v_ring=v_ring, pos=pos, k_new=k_new, v_new=v_new)
    st = load().swa_cache_append(k_ring.data_ptr(), v_ring.data_ptr(), pos.data_ptr(),
                                 k_new.data_ptr(), v_new.data_ptr(), B, Hkv, W, d,
                                 _dtype_code(k_ring), _stream(stream))
    _raise("swa_cache_append", st)


def decode_workspace_bytes(B, Hq, W, d):
    return int(load().swa_decode_workspace_bytes(int(B), int(Hq), int(W), int(d)))


def decode_workspace(B, Hq, W, d, device="cuda"):
    """A decode workspace (reusable across calls without clearing; 16 bytes
    when the call needs none)."""
    import torch
    return torch.zeros(max(decode_workspace_bytes(B, Hq, W, d), 16), dtype=torch.uint8, device=device)


def global_workspace_bytes(T, Hq, G, d):
    return int(load().swa_prefill_global_workspace_bytes(int(T), int(Hq), int(G), int(d)))


def global_workspace(T, Hq, G, d, device="cuda"):
    """A workspace for prefill_global (Hq with the batch folded in)."""
    import torch
    return torch.zeros(max(global_workspace_bytes(T, Hq, G, d), 16), dtype=torch.uint8, device=device)


def decode(q, k_ring, v_ring, pos, scale=None, out=None, workspace=None, stream=None):
    """One query token per sequence against its ring; returns out [B, Hq, d]."""
    import torch
    _check(q, "q", 3)
    _check(k_ring, "k_ring", 4, q.dtype)
    _check(v_ring, "v_ring", 4, q.dtype)
    _check(pos, "pos", 1, torch.int32)
    B, Hq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    if tuple(k_ring.shape) != (B, Hkv, W, d) or tuple(v_ring.shape) != tuple(k_ring.shape) \
            or pos.shape[0] != B:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", 3, q.dtype)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _same_device(q=q, k_ring=k_ring, v_ring=v_ring, pos=pos, out=out, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(B, Hq, W, d)
    if need == 0:  # one split: the kernel writes out itself and reads no workspace
        ws_ptr, ws_bytes = None, 0
    else:
        if workspace is None:
            workspace = decode_workspace(B, Hq, W, d, q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = load().swa_decode(q.data_ptr(), k_ring.data_ptr(), v_ring.data_ptr(), pos.data_ptr(),
                           out.data_ptr(), B, Hq, Hkv, W, d, float(scale), _dtype_code(q),
                           ws_ptr, ws_bytes, _stream(stream))
    _raise("swa_decode", st)
    return out


def decode_noalloc(q, k_ring, v_ring, pos, scale=None, out=None, stream=None):
    """decode without a workspace: the library's per-GPU scratch holds the
    split partials (calls overlapping on one GPU race); returns out
    [B, Hq, d].  Pass `out` to make the call allocate nothing at all."""
    import torch
    _check(q, "q", 3)
    _check(k_ring, "k_ring", 4, q.dtype)
    _check(v_ring, "v_ring", 4, q.dtype)
    _check(pos, "pos", 1, torch.int32)
    B, Hq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    if tuple(k_ring.shape) != (B, Hkv, W, d) or tuple(v_ring.shape) != tuple(k_ring.shape) \
            or pos.shape[0] != B:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", 3, q.dtype)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _same_device(q=q, k_ring=k_ring, v_ring=v_ring, pos=pos, out=out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = load().swa_decode_noalloc(q.data_ptr(), k_ring.data_ptr(), v_ring.data_ptr(),
                                   pos.data_ptr(), out.data_ptr(), B, Hq, Hkv, W, d, float(scale),
                                   _dtype_code(q), _stream(stream))
    _raise("swa_decode_noalloc", st)
    return out


def cache_append_chunk(k_ring, v_ring, pos, k, v, stream=None):
    """Append n tokens per sequence: k/v [B, Hkv, n, d], token i to slot
    (pos[b] + i) mod W of the rings."""
    import torch
    _check(k_ring, "k_ring", 4)
    _check(v_ring, "v_ring", 4, k_ring.dtype)
    _check(pos, "pos", 1, torch.int32)
    _check(k, "k", 4, k_ring.dtype)
    _check(v, "v", 4, k_ring.dtype)
    B, Hkv, W, d = k_ring.shape
    n = k.shape[2]
    if tuple(v_ring.shape) != tuple(k_ring.shape) or tuple(k.shape) != (B, Hkv, n, d) \
            or tuple(v.shape) != tuple(k.shape) or pos.shape[0] != B:
        raise ValueError("shape mismatch")
    _same_device(k_ring=k_ring, v_ring=v_ring, pos=pos, k=k, v=v)
    st = load().swa_cache_append_chunk(k_ring.data_ptr(), v_ring.data_ptr(), pos.data_ptr(),
                                       k.data_ptr(), v.data_ptr(), B, n, Hkv, W, d,
                                       _dtype_code(k_ring), _stream(stream))
    _raise("swa_cache_append_chunk", st)


def prefill_chunk(q, k, v, k_ring, v_ring, pos, scale=None, out=None, stream=None):
    """Causal attention of a chunk of n new tokens per sequence (positions
    pos[b] .. pos[b]+n-1) over the ring plus the chunk itself; returns out
    [B, Hq, n, d].  Append the chunk to the rings afterwards."""
    import torch
    _check(q, "q", 4)
    _check(k, "k", 4, q.dtype)
    _check(v, "v", 4, q.dtype)
    _check(k_ring, "k_ring", 4, q.dtype)
    _check(v_ring, "v_ring", 4, q.dtype)
    _check(pos, "pos", 1, torch.int32)
    B, Hq, n, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    if tuple(k.shape) != (B, Hkv, n, d) or tuple(v.shape) != tuple(k.shape) \
            or tuple(k_ring.shape) != (B, Hkv, W, d) or tuple(v_ring.shape) != tuple(k_ring.shape) \
            or pos.shape[0] != B:
        raise ValueError("shape mismatch q%s k%s ring%s" % (tuple(q.shape), tuple(k.shape),
                                                          tuple(k_ring.shape)))
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", 4, q.dtype)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _same_device(q=q, k=k, v=v, k_ring=k_ring, v_ring=v_ring, pos=pos, out=out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = load().swa_prefill_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), k_ring.data_ptr(),
                                  v_ring.data_ptr(), pos.data_ptr(), out.data_ptr(), B, n, W, Hq,
                                  Hkv, d, float(scale), _dtype_code(q), _stream(stream))
    _raise("swa_prefill_chunk", st)
    return out


def decode_sinks_workspace(B, Hq, W, d, device="cuda"):
    """A workspace for decode_sinks (reusable across calls without clearing)."""
    import torch
    n = int(load().swa_decode_sinks_workspace_bytes(int(B), int(Hq), int(W), int(d)))
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def decode_sinks(q, k_ring, v_ring, k_sink, v_sink, pos, scale=None, out=None, workspace=None,
                 stream=None):
    """decode with attention sinks: k_sink/v_sink [B, Hkv, S, d] hold the
    first S positions, kept beside the ring; returns out [B, Hq, d]."""
    import torch
    _check(q, "q", 3)
    _check(k_ring, "k_ring", 4, q.dtype)
    _check(v_ring, "v_ring", 4, q.dtype)
    _check(k_sink, "k_sink", 4, q.dtype)
    _check(v_sink, "v_sink", 4, q.dtype)
    _check(pos, "pos", 1, torch.int32)
    B, Hq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    S = k_sink.shape[2]
    if tuple(k_ring.shape) != (B, Hkv, W, d) or tuple(v_ring.shape) != tuple(k_ring.shape) \
            or tuple(k_sink.shape) != (B, Hkv, S, d) or tuple(v_sink.shape) != tuple(k_sink.shape) \
            or pos.shape[0] != B:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", 3, q.dtype)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _same_device(q=q, k_ring=k_ring, v_ring=v_ring, k_sink=k_sink, v_sink=v_sink, pos=pos,
                 out=out, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_sinks_workspace(B, Hq, W, d, q.device)
    st = load().swa_decode_sinks(q.data_ptr(), k_ring.data_ptr(), v_ring.data_ptr(),
                                 k_sink.data_ptr() if S else None, v_sink.data_ptr() if S else None,
                                 S, pos.data_ptr(), out.data_ptr(), B, Hq, Hkv, W, d, float(scale),
                                 _dtype_code(q), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _raise("swa_decode_sinks", st)
    return out


def calib_mfma(operands, sink, n_wg, iters, stream=None):
    """Matrix-core calibration loop (see swa_calib_mfma_bf16): `operands` a
    device bf16 tensor of random values, `sink` a float32 tensor of at least
    n_wg * 256 elements.  Returns the FLOPs it issues."""
    import torch
    _check(operands, "operands", operands.dim(), torch.bfloat16)
    _check(sink, "sink", sink.dim(), torch.float32)
    if sink.numel() < n_wg * 256:
        raise ValueError("sink needs n_wg * 256 elements")
    st = load().swa_calib_mfma_bf16(operands.data_ptr(), operands.numel() * 2, sink.data_ptr(),
                                    int(n_wg), int(iters), _stream(stream))
    _raise("swa_calib_mfma_bf16", st)
    return n_wg * 4 * iters * 16 * 32768


def calib_stream_read(src, sink, n_wg, stream=None):
    """Streaming-read calibration (see swa_calib_stream_read) of the whole of
    the contiguous device tensor `src`; `sink` an int32 tensor of at least
    n_wg * 256 elements.  Returns the bytes it reads."""
    import torch
    _check(src, "src", src.dim())
    _check(sink, "sink", sink.dim(), torch.int32)
    if sink.numel() < n_wg * 256:
        raise ValueError("sink needs n_wg * 256 elements")
    nbytes = src.numel() * src.element_size()
    st = load().swa_calib_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), int(n_wg),
                                      _stream(stream))
    _raise("swa_calib_stream_read", st)
    return nbytes


def calib_vector(op, sink, n_wg, iters, stream=None):
    """Vector-ALU calibration (see swa_calib_vector): op 0 fp32 FMA chains, op
    1 exp2 chains; `sink` a float32 tensor of at least n_wg * 256 elements.
    Returns the wave instructions it issues."""
    import torch
    _check(sink, "sink", sink.dim(), torch.float32)
    if sink.numel() < n_wg * 256:
        raise ValueError("sink needs n_wg * 256 elements")
    st = load().swa_calib_vector(int(op), sink.data_ptr(), int(n_wg), int(iters), _stream(stream))
    _raise("swa_calib_vector", st)
    return n_wg * 4 * iters * 16
