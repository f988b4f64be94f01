"""ctypes binding of liboctopus.so (include/octopus.h).

Argument marshalling only: the functions below turn torch tensors into device
pointers, pass the current HIP stream and raise OctoError on a non-OK status.
Every step of the codec and of attention runs in the library's kernels; there
is no fallback of any kind.  torch provides device memory and streams.

Names follow the C ABI: octo_encode, octo_attend_decode, octo_attend_chunk,
octo_record_sizes, octo_decode_workspace_bytes, octo_chunk_workspace_bytes.
The helper classes Codec and PackedCache hold the codebook values (host
arrays) and allocate the packed streams with torch, and build the descriptor
structs.
"""
import ctypes
import json
import os

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# OCTO_LIB names another build of the same library (the host-sanitized one of
# build.py --sanitize, for the ABI checks under ASan and UBSan).
LIB_PATH = os.environ.get("OCTO_LIB") or os.path.join(PKG, "liboctopus.so")
CODEBOOKS = os.path.join(PKG, "codebooks", "octopus_d{d}.json")

ABI_VERSION = 4
STATUS = ["OCTO_OK", "OCTO_ERR_INVALID_ARGUMENT", "OCTO_ERR_UNSUPPORTED", "OCTO_ERR_ALIGNMENT",
          "OCTO_ERR_CAPACITY", "OCTO_ERR_WORKSPACE_TOO_SMALL", "OCTO_ERR_VERSION", "OCTO_ERR_HIP"]
DTYPE_F32, DTYPE_BF16 = 0, 1
CHUNK_JENSEN_CORRECTION = 1
ROUND_LOCAL3X3, ROUND_SCALAR = 0, 1
LAYOUT_TILE64 = 0


class OctoError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS[status] if 0 <= status < len(STATUS) else status}: {message}")
        self.status = status


class CodecDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("head_dim", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("b_dir", ctypes.c_int32), ("b_nrm", ctypes.c_int32),
                ("rounding", ctypes.c_int32), ("qjl", ctypes.c_int32),
                ("group", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("c_xi", ctypes.c_void_p), ("c_rho", ctypes.c_void_p)]


class CacheView(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("qjl", ctypes.c_void_p), ("gamma_r", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("layout", ctypes.c_int32)]


class StreamSizes(ctypes.Structure):
    _fields_ = [("idx_words", ctypes.c_int32),
                ("qjl_words", ctypes.c_int32), ("n_triplets", ctypes.c_int32),
                ("b_dir", ctypes.c_int32), ("b_nrm", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib():
    """The loaded library.  Raises if it has not been built: nothing runs without it."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m quantized_decode_attention_octo_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.octo_abi_version.restype = ctypes.c_uint32
        L.octo_status_string.restype = ctypes.c_char_p
        L.octo_status_string.argtypes = [ctypes.c_int]
        L.octo_last_error.restype = ctypes.c_char_p
        L.octo_record_sizes.argtypes = [ctypes.POINTER(CodecDesc), ctypes.POINTER(StreamSizes)]
        L.octo_encode.argtypes = [ctypes.POINTER(CodecDesc), _P, ctypes.c_int, _I, _I, _I,
                                  ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(CacheView), _I, _P]
        L.octo_decode_workspace_bytes.argtypes = [ctypes.POINTER(CodecDesc), _I, _I, _I, _I,
                                                  ctypes.POINTER(ctypes.c_size_t)]
        L.octo_attend_decode.argtypes = [ctypes.POINTER(CodecDesc), ctypes.POINTER(CodecDesc),
                                         ctypes.POINTER(CacheView), ctypes.POINTER(CacheView),
                                         _P, ctypes.c_int, _I, _P, _I, ctypes.c_float, _P, _P,
                                         ctypes.c_size_t, _P]
        L.octo_chunk_workspace_bytes.argtypes = [ctypes.POINTER(CodecDesc), _I, _I, _I, _I, _I, _I,
                                                 ctypes.c_uint32, ctypes.POINTER(ctypes.c_size_t)]
        L.octo_attend_chunk.argtypes = [ctypes.POINTER(CodecDesc), ctypes.POINTER(CodecDesc),
                                        ctypes.POINTER(CacheView), ctypes.POINTER(CacheView), _I,
                                        _P, _P, _P, _I, _I, _I, ctypes.c_float, ctypes.c_uint32,
                                        _P, _P, ctypes.c_size_t, _P]
        L.octo_decode_step_workspace_bytes.argtypes = [ctypes.POINTER(CodecDesc), _I, _I, _I, _I,
                                                       ctypes.POINTER(ctypes.c_size_t)]
        L.octo_decode_step.argtypes = [ctypes.POINTER(CodecDesc), ctypes.POINTER(CodecDesc),
                                       ctypes.POINTER(CacheView), ctypes.POINTER(CacheView),
                                       _P, ctypes.c_int, _I, _P, _P, _P, _P, _I, _P, _P, _I,
                                       ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
        L.octo_decode_tokens.argtypes = [ctypes.POINTER(CodecDesc), ctypes.POINTER(CacheView),
                                         _I, _I, _P, _P]
        L.octo_attend_decode_noalloc.argtypes = [ctypes.POINTER(CodecDesc), ctypes.POINTER(CodecDesc),
                                                 ctypes.POINTER(CacheView), ctypes.POINTER(CacheView),
                                                 _P, ctypes.c_int, _I, _P, _I, ctypes.c_float, _P, _P]
        for f in ("octo_record_sizes", "octo_encode", "octo_decode_workspace_bytes",
                  "octo_attend_decode", "octo_chunk_workspace_bytes", "octo_attend_chunk",
                  "octo_decode_step_workspace_bytes", "octo_decode_step", "octo_decode_tokens",
                  "octo_attend_decode_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        if L.octo_abi_version() != ABI_VERSION:
            raise RuntimeError("liboctopus.so ABI version mismatch")
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise OctoError(status, lib().octo_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    """torch's current stream on `device` as a raw handle."""
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _expect(t, name, shape, dtypes, contiguous=True):
    """Raises ValueError unless tensor t has exactly `shape` (None entries
    match any size) and one of `dtypes` and, if asked, is contiguous.  The library sees only pointers, so these checks
    are the only guard against reads and writes past a buffer.  The common
    case (everything right) takes one comparison per property; the messages
    come from the slow path."""
    if type(t) is torch.Tensor and t.dtype in dtypes and (not contiguous or t.is_contiguous()):
        sh = t.shape
        if None in shape:
            if len(sh) == len(shape) and all(e is None or e == n for e, n in zip(shape, sh)):
                return
        elif sh == shape:
            return
    _expect_failed(t, name, shape, dtypes, contiguous)


def _expect_failed(t, name, shape, dtypes, contiguous):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {list(dtypes)}")
    if t.dim() != len(shape) or any(e is not None and e != n for e, n in zip(shape, t.shape)):
        want = tuple("*" if e is None else e for e in shape)
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    # a tensor subclass that passes every check is accepted


def _on_device(device, **tensors):
    """Raises ValueError unless every tensor lives on `device`, a CUDA device
    (checked after the shapes, so that a shape error is named first)."""
    idx = device.index if device.type == "cuda" else -2
    for name, t in tensors.items():
        if t.get_device() != idx:
            if t.device.type != "cuda":
                raise ValueError(f"{name} is on {t.device}; the kernels need device memory")
            raise ValueError(f"{name} is on {t.device}, the cache on {device}")
    if idx == -2:
        raise ValueError(f"the cache is on {device}; the kernels need device memory")


def _same_caches(k_cache, v_cache, k_codec, v_codec):
    if k_cache.device != v_cache.device:
        raise ValueError("the K and V caches live on different devices")
    if (k_cache.B, k_cache.H, k_cache.capacity) != (v_cache.B, v_cache.H, v_cache.capacity):
        raise ValueError("the K and V caches differ in batch, heads or capacity")
    for c, cd, nm in ((k_cache, k_codec, "k_cache"), (v_cache, v_codec, "v_cache")):
        if c.codec_key != cd.key():
            raise ValueError(f"{nm} was allocated for another codec")


F32_BF16 = (torch.float32, torch.bfloat16)
BF16 = (torch.bfloat16,)


def load_codebooks(d=128):
    with open(CODEBOOKS.format(d=d)) as f:
        return json.load(f)


class Codec:
    """A codec descriptor with its fp32 codebook values (host arrays).

    bits: b; the split defaults to the paper's (b+1, b-1) (b_dir, b_nrm).
    The codebook values come from the shipped artifact (Lloyd-Max tables,
    Sec. 3.4 of the OCTOPUS paper).  group = 16 or 32 selects the group-wise
    value codec instead (b-bit codes, E4M3 scales, BF16 zero-points; no
    codebooks)."""

    def __init__(self, bits=3, seed=0, qjl=False, b_dir=None, b_nrm=None,
                 rounding=ROUND_LOCAL3X3, device="cuda", d=128, tables=None, group=0):
        self.group = int(group)
        if self.group:
            self.c_xi = self.c_rho = None
            self.desc = CodecDesc(ABI_VERSION, d, bits, 0, 0, rounding, int(bool(qjl)), self.group,
                                  seed, None, None)
            self.bits, self.b_dir, self.b_nrm, self.seed, self.qjl = bits, 0, 0, seed, bool(qjl)
            self.rounding, self.d, self.device = rounding, d, device
            return
        if b_dir is None:
            b_dir, b_nrm = bits + 1, bits - 1
        art = tables or load_codebooks(d)
        # host arrays: the library reads the values at each call and hands
        # them to the kernels by value
        self.c_xi = np.ascontiguousarray(art["c_xi"][str(b_dir)], dtype=np.float32)
        self.c_rho = np.ascontiguousarray(art["c_rho"][str(b_nrm)], dtype=np.float32)
        self.desc = CodecDesc(ABI_VERSION, d, bits, b_dir, b_nrm, rounding, int(bool(qjl)), 0,
                              seed, self.c_xi.ctypes.data, self.c_rho.ctypes.data)
        self.bits, self.b_dir, self.b_nrm, self.seed, self.qjl = bits, b_dir, b_nrm, seed, bool(qjl)
        self.rounding, self.d, self.device = rounding, d, device

    def sizes(self):
        return octo_record_sizes(self.desc)

    def key(self):
        """What fixes the record layout of a cache: (group, bits, split, QJL)."""
        return (self.group, self.bits if self.group else 0, self.b_dir, self.b_nrm, self.qjl)


class PackedCache:
    """The packed streams of one tensor (K or V) in the tile-64 layout."""

    def __init__(self, codec, B, H, capacity, device="cuda"):
        s = codec.sizes()
        n = B * H * capacity
        i32 = dict(dtype=torch.int32, device=device)
        self.idx = torch.zeros(n * s.idx_words, **i32)
        # the group codec keeps its scales and zero-points in the record
        self.gamma = (None if codec.group else
                      torch.zeros(B, H, capacity, dtype=torch.float32, device=device))
        self.qjl = torch.zeros(n * s.qjl_words, **i32) if codec.qjl else None
        self.gamma_r = torch.zeros(B, H, capacity, dtype=torch.int16, device=device) if codec.qjl else None
        self.B, self.H, self.capacity, self.sizes = B, H, capacity, s
        self.codec_key = codec.key()
        self.device = self.idx.device
        self.view = CacheView(self.idx.data_ptr(), self.gamma.data_ptr() if self.gamma is not None else None,
                              self.qjl.data_ptr() if self.qjl is not None else None,
                              self.gamma_r.data_ptr() if self.gamma_r is not None else None,
                              B, H, capacity, LAYOUT_TILE64)

    def nbytes(self):
        t = [self.idx, self.gamma, self.qjl, self.gamma_r]
        return sum(x.numel() * x.element_size() for x in t if x is not None)

    def to_host(self):
        """Host copies of the streams (numpy) in the layout the oracle reads."""
        out = {"idx": self.idx.cpu().numpy().view("<u4"),
               "B": self.B, "H": self.H, "capacity": self.capacity}
        if self.gamma is not None:
            out["gamma"] = self.gamma.cpu().numpy()
        if self.qjl is not None:
            out["qjl"] = self.qjl.cpu().numpy().view("<u4")
            out["gamma_r"] = self.gamma_r.cpu().numpy().view("<u2")
        return out


# ------------------------------------------------------------------ entry points
def octo_record_sizes(desc):
    out = StreamSizes()
    _check(lib().octo_record_sizes(ctypes.byref(desc), ctypes.byref(out)))
    return out


def octo_encode(codec, x, cache, token_offset=0):
    """Encodes x[B, H, T, d] (fp32 or bf16, any strides with unit last stride)
    into tokens [token_offset, token_offset + T) of `cache`."""
    _expect(x, "x", (cache.B, cache.H, None, codec.d), F32_BF16, contiguous=False)
    if cache.codec_key != codec.key():
        raise ValueError("the cache was allocated for another codec")
    if x.stride(3) != 1 or min(x.stride()) < 0:
        raise ValueError("x needs a unit last stride and non-negative strides")
    _on_device(cache.device, x=x, cache=cache.idx)
    B, H, T, d = x.shape
    strides = (ctypes.c_int64 * 4)(*x.stride())
    dt = DTYPE_F32 if x.dtype == torch.float32 else DTYPE_BF16
    _check(lib().octo_encode(ctypes.byref(codec.desc), _ptr(x), dt, B, H, T, strides,
                             ctypes.byref(cache.view), token_offset, _stream(x.device)))


def octo_decode_tokens(codec, cache, t0, T, out=None):
    """Reconstructed tokens [t0, t0 + T) of every plane: out[B, H, T, d] fp32."""
    if cache.codec_key != codec.key():
        raise ValueError("the cache was allocated for another codec")
    if out is None:
        out = torch.empty(cache.B, cache.H, T, codec.d, dtype=torch.float32, device=cache.device)
    _expect(out, "out", (cache.B, cache.H, T, codec.d), (torch.float32,))
    _on_device(cache.device, out=out, cache=cache.idx)
    _check(lib().octo_decode_tokens(ctypes.byref(codec.desc), ctypes.byref(cache.view), t0, T,
                                    _ptr(out), _stream(out.device)))
    return out


def octo_decode_workspace_bytes(k_codec, B, num_q_heads, kv_heads, max_seq_len):
    n = ctypes.c_size_t()
    _check(lib().octo_decode_workspace_bytes(ctypes.byref(k_codec.desc), B, num_q_heads,
                                             kv_heads, max_seq_len, ctypes.byref(n)))
    return n.value


def _workspace_need(fn, k_codec, *sizes):
    """fn(k_codec, *sizes), remembered per codec: the answer depends only on
    the codec's layout and the sizes, and the query costs a library call."""
    memo = k_codec.__dict__.setdefault("_ws_need", {})
    key = (fn, sizes)
    n = memo.get(key)
    if n is None:
        n = memo[key] = fn(k_codec, *sizes)
    return n


def workspace(nbytes, device):
    """A device buffer with at least nbytes from a 256-byte aligned start."""
    return torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)


def _aligned_ptr(ws):
    p = ws.data_ptr()
    return (p + 255) // 256 * 256


def octo_attend_decode(k_codec, v_codec, k_cache, v_cache, q, seq_lens, max_seq_len=None,
                       softmax_scale=0.0, out=None, ws=None):
    """q[B, H_q, d] (fp32 or bf16, contiguous), seq_lens int32 [B] on the device.
    Returns out[B, H_q, d] fp32."""
    _same_caches(k_cache, v_cache, k_codec, v_codec)
    dev, B = k_cache.device, k_cache.B
    _expect(q, "q", (B, None, k_codec.d), F32_BF16)
    Hq, d = q.shape[1], q.shape[2]
    if Hq % k_cache.H:
        raise ValueError(f"q has {Hq} heads, not a multiple of the {k_cache.H} KV heads")
    _expect(seq_lens, "seq_lens", (B,), (torch.int32,))
    max_seq_len = k_cache.capacity if max_seq_len is None else int(max_seq_len)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    _expect(out, "out", (B, Hq, d), (torch.float32,))
    _on_device(dev, q=q, seq_lens=seq_lens, out=out, k_cache=k_cache.idx, v_cache=v_cache.idx)
    need = _workspace_need(octo_decode_workspace_bytes, k_codec, B, Hq, k_cache.H, max_seq_len)
    if ws is None or ws.numel() < need + 256:
        ws = workspace(need, dev)
    _expect(ws, "ws", (None,), (torch.uint8,))
    if ws.get_device() != q.get_device():
        _on_device(dev, ws=ws)
    dt = DTYPE_F32 if q.dtype == torch.float32 else DTYPE_BF16
    _check(lib().octo_attend_decode(ctypes.byref(k_codec.desc), ctypes.byref(v_codec.desc),
                                    ctypes.byref(k_cache.view), ctypes.byref(v_cache.view),
                                    _ptr(q), dt, Hq, _ptr(seq_lens), max_seq_len,
                                    float(softmax_scale), _ptr(out),
                                    _aligned_ptr(ws), ws.numel() - 256,
                                    _stream(q.device)))
    return out


def octo_attend_decode_noalloc(k_codec, v_codec, k_cache, v_cache, q, seq_lens, max_seq_len=None,
                               softmax_scale=0.0, out=None):
    """octo_attend_decode without a workspace: the library keeps the partials
    in its static per-device scratch (see include/octopus.h; calls on one
    device must not overlap).  Returns out[B, H_q, d] fp32."""
    _same_caches(k_cache, v_cache, k_codec, v_codec)
    dev, B = k_cache.device, k_cache.B
    _expect(q, "q", (B, None, k_codec.d), F32_BF16)
    Hq, d = q.shape[1], q.shape[2]
    if Hq % k_cache.H:
        raise ValueError(f"q has {Hq} heads, not a multiple of the {k_cache.H} KV heads")
    _expect(seq_lens, "seq_lens", (B,), (torch.int32,))
    max_seq_len = k_cache.capacity if max_seq_len is None else int(max_seq_len)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    _expect(out, "out", (B, Hq, d), (torch.float32,))
    _on_device(dev, q=q, seq_lens=seq_lens, out=out, k_cache=k_cache.idx, v_cache=v_cache.idx)
    dt = DTYPE_F32 if q.dtype == torch.float32 else DTYPE_BF16
    _check(lib().octo_attend_decode_noalloc(ctypes.byref(k_codec.desc), ctypes.byref(v_codec.desc),
                                            ctypes.byref(k_cache.view), ctypes.byref(v_cache.view),
                                            _ptr(q), dt, Hq, _ptr(seq_lens), max_seq_len,
                                            float(softmax_scale), _ptr(out), _stream(dev)))
    return out


def octo_decode_step_workspace_bytes(k_codec, B, num_q_heads, kv_heads, max_packed_len):
    n = ctypes.c_size_t()
    _check(lib().octo_decode_step_workspace_bytes(ctypes.byref(k_codec.desc), B, num_q_heads,
                                                  kv_heads, max_packed_len, ctypes.byref(n)))
    return n.value


def octo_decode_step(k_codec, v_codec, k_cache, v_cache, q, k_new, v_new, k_window, v_window,
                     packed_lens, window_lens, max_packed_len=None, softmax_scale=0.0,
                     out=None, ws=None):
    """One decode step with a residual window (see include/octopus.h).
    q[B, H_q, d] (fp32 or bf16), k_new/v_new[B, H_kv, d] bf16, rings
    k_window/v_window[B, H_kv, W, d] bf16, packed_lens/window_lens int32 [B]
    (all on the device; the rings and the lengths are updated in place).
    Returns out[B, H_q, d] fp32."""
    _same_caches(k_cache, v_cache, k_codec, v_codec)
    dev, B, Hkv, D = k_cache.device, k_cache.B, k_cache.H, k_codec.d
    _expect(q, "q", (B, None, D), F32_BF16)
    Hq, d = q.shape[1], q.shape[2]
    if Hq % Hkv:
        raise ValueError(f"q has {Hq} heads, not a multiple of the {Hkv} KV heads")
    _expect(k_new, "k_new", (B, Hkv, D), BF16)
    _expect(v_new, "v_new", (B, Hkv, D), BF16)
    _expect(k_window, "k_window", (B, Hkv, None, D), BF16)
    W = k_window.shape[2]
    _expect(v_window, "v_window", (B, Hkv, W, D), BF16)
    _expect(packed_lens, "packed_lens", (B,), (torch.int32,))
    _expect(window_lens, "window_lens", (B,), (torch.int32,))
    max_packed_len = k_cache.capacity if max_packed_len is None else int(max_packed_len)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    _expect(out, "out", (B, Hq, d), (torch.float32,))
    _on_device(dev, q=q, k_new=k_new, v_new=v_new, k_window=k_window, v_window=v_window,
               packed_lens=packed_lens, window_lens=window_lens, out=out,
               k_cache=k_cache.idx, v_cache=v_cache.idx)
    need = _workspace_need(octo_decode_step_workspace_bytes, k_codec, B, Hq, k_cache.H, max_packed_len)
    if ws is None or ws.numel() < need + 256:
        ws = workspace(need, dev)
    _expect(ws, "ws", (None,), (torch.uint8,))
    if ws.get_device() != q.get_device():
        _on_device(dev, ws=ws)
    dt = DTYPE_F32 if q.dtype == torch.float32 else DTYPE_BF16
    _check(lib().octo_decode_step(ctypes.byref(k_codec.desc), ctypes.byref(v_codec.desc),
                                  ctypes.byref(k_cache.view), ctypes.byref(v_cache.view),
                                  _ptr(q), dt, Hq, _ptr(k_new), _ptr(v_new), _ptr(k_window),
                                  _ptr(v_window), W, _ptr(packed_lens), _ptr(window_lens),
                                  max_packed_len, float(softmax_scale), _ptr(out),
                                  _aligned_ptr(ws), ws.numel() - 256,
                                  _stream(q.device)))
    return out


def octo_chunk_workspace_bytes(k_codec, B, num_q_heads, kv_heads, Tq, cached_tokens, Tc, flags=0):
    n = ctypes.c_size_t()
    _check(lib().octo_chunk_workspace_bytes(ctypes.byref(k_codec.desc), B, num_q_heads,
                                            kv_heads, Tq, cached_tokens, Tc,
                                            ctypes.c_uint32(flags), ctypes.byref(n)))
    return n.value


def octo_attend_chunk(k_codec, v_codec, k_cache, v_cache, cached_tokens, q, k_cur, v_cur,
                      softmax_scale=0.0, out=None, ws=None, correction=False):
    """q[B, H_q, Tq, d], k_cur/v_cur[B, H_kv, Tc, d] (bf16, contiguous).
    correction: the Jensen-bias correction of the cached keys' logits
    (OCTO_CHUNK_JENSEN_CORRECTION; keys in the group codec).
    Returns out[B, H_q, Tq, d] fp32."""
    flags = CHUNK_JENSEN_CORRECTION if correction else 0
    _same_caches(k_cache, v_cache, k_codec, v_codec)
    dev, B, Hkv, D = k_cache.device, k_cache.B, k_cache.H, k_codec.d
    _expect(q, "q", (B, None, None, D), BF16)
    Hq, Tq, d = q.shape[1], q.shape[2], q.shape[3]
    if Hq % Hkv:
        raise ValueError(f"q has {Hq} heads, not a multiple of the {Hkv} KV heads")
    _expect(k_cur, "k_cur", (B, Hkv, None, D), BF16)
    Tc = k_cur.shape[2]
    _expect(v_cur, "v_cur", (B, Hkv, Tc, D), BF16)
    if out is None:
        out = torch.empty(B, Hq, Tq, d, dtype=torch.float32, device=dev)
    _expect(out, "out", (B, Hq, Tq, d), (torch.float32,))
    _on_device(dev, q=q, k_cur=k_cur, v_cur=v_cur, out=out, k_cache=k_cache.idx,
               v_cache=v_cache.idx)
    need = _workspace_need(octo_chunk_workspace_bytes, k_codec, B, Hq, k_cache.H, Tq, cached_tokens, Tc, flags)
    if ws is None or ws.numel() < need + 256:
        ws = workspace(need, dev)
    _expect(ws, "ws", (None,), (torch.uint8,))
    if ws.get_device() != q.get_device():
        _on_device(dev, ws=ws)
    _check(lib().octo_attend_chunk(ctypes.byref(k_codec.desc), ctypes.byref(v_codec.desc),
                                   ctypes.byref(k_cache.view), ctypes.byref(v_cache.view),
                                   cached_tokens, _ptr(q), _ptr(k_cur), _ptr(v_cur), Hq, Tq, Tc,
                                   ctypes.c_float(softmax_scale), ctypes.c_uint32(flags), _ptr(out),
                                   _aligned_ptr(ws), ws.numel() - 256,
                                   _stream(q.device)))
    return out
