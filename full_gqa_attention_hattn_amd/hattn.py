"""Python binding of libhattn (ctypes): argument marshalling only.

Every step of the layer runs in the HIP library; this module turns torch tensors (device
memory) and the current torch stream into the C ABI's pointers and sizes, and raises
HattnError on a non-OK status.  It never computes anything itself and has no fallback: if
the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhattn.so")

HATTN_OK = 0
HATTN_ERR_NULL = 1
HATTN_ERR_SHAPE = 2
HATTN_ERR_UNSUPPORTED = 3
HATTN_ERR_RANGE = 4
HATTN_ERR_ALIGN = 5
HATTN_ERR_WORKSPACE = 6
HATTN_ERR_HIP = 7
HATTN_ERR_SCRATCH = 8
DECODE_NOALLOC_MAX_BYTES = 32 << 20
HATTN_SLIDING = 0
HATTN_FULL = 1
HATTN_ROPE_Q_FUSED = 1
HATTN_KV8_ROPE_K = 1

# Every symbol include/hattn.h declares.
EXPORTS = ("hattn_cfg_preset", "hattn_rope_qk", "hattn_kv_append", "hattn_kv_append_rope",
           "hattn_prefill", "hattn_prefill_ring", "hattn_kv_append_fp8", "hattn_decode_fp8",
           "hattn_decode_fp8_workspace_bytes",
           "hattn_qkv_proj", "hattn_o_proj",
           "hattn_decode_workspace_bytes", "hattn_decode", "hattn_decode_noalloc",
           "hattn_model_layer_kind",
           "hattn_model_kv_bytes", "hattn_model_decode_workspace_bytes", "hattn_model_decode",
           "hattn_model_prefill_workspace_bytes", "hattn_model_prefill",
           "hattn_status_string", "hattn_last_hip_error")


class LayerCfg(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("rot_dim", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


class LayerIO(ctypes.Structure):
    """hattn_layer_io: one layer's device buffers for the whole-model driver."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q", "k", "v", "gate", "k_cache", "v_cache", "out", "lse")]


class HattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.hattn_status_string(status).decode()
        if status == HATTN_ERR_HIP:
            msg += f" (hipError {_lib.hattn_last_hip_error()})"
        super().__init__(f"{where}: {msg} [status {status}]")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it first (__graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
    cfgp = ctypes.POINTER(LayerCfg)
    lib.hattn_cfg_preset.argtypes = [i32, cfgp]
    lib.hattn_cfg_preset.restype = i32
    lib.hattn_rope_qk.argtypes = [cfgp, vp, vp, vp, i32, i32, vp]
    lib.hattn_rope_qk.restype = i32
    lib.hattn_kv_append.argtypes = [cfgp, vp, vp, vp, vp, i32, vp, i32, i32, vp, vp]
    lib.hattn_kv_append.restype = i32
    lib.hattn_kv_append_rope.argtypes = [cfgp, vp, vp, vp, vp, i32, vp, i32, i32, vp, vp]
    lib.hattn_kv_append_rope.restype = i32
    lib.hattn_qkv_proj.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.hattn_qkv_proj.restype = i32
    lib.hattn_o_proj.argtypes = [vp, i32, vp, vp, vp]
    lib.hattn_o_proj.restype = i32
    lib.hattn_kv_append_fp8.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, u32, vp]
    lib.hattn_kv_append_fp8.restype = i32
    lib.hattn_decode_fp8.argtypes = [cfgp, vp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp,
                                     ctypes.c_size_t, u32, vp]
    lib.hattn_decode_fp8.restype = i32
    lib.hattn_decode_fp8_workspace_bytes.argtypes = [cfgp, i32, i32]
    lib.hattn_decode_fp8_workspace_bytes.restype = ctypes.c_size_t
    iop = ctypes.POINTER(LayerIO)
    sz = ctypes.c_size_t
    lib.hattn_model_layer_kind.argtypes = [i32]
    lib.hattn_model_layer_kind.restype = i32
    lib.hattn_model_kv_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.hattn_model_kv_bytes.restype = i32
    lib.hattn_model_decode_workspace_bytes.argtypes = [i32, i32, i32]
    lib.hattn_model_decode_workspace_bytes.restype = sz
    lib.hattn_model_decode.argtypes = [iop, i32, i32, vp, i32, vp, sz, vp]
    lib.hattn_model_decode.restype = i32
    lib.hattn_model_prefill_workspace_bytes.argtypes = [i32, i32, i32]
    lib.hattn_model_prefill_workspace_bytes.restype = sz
    lib.hattn_model_prefill.argtypes = [iop, i32, i32, vp, i32, i32, vp, sz, vp]
    lib.hattn_model_prefill.restype = i32
    lib.hattn_prefill.argtypes = [cfgp, vp, vp, vp, i32, vp, i32, i32, vp, vp, vp, u32, vp]
    lib.hattn_prefill.restype = i32
    lib.hattn_prefill_ring.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, u32, vp]
    lib.hattn_prefill_ring.restype = i32
    lib.hattn_decode_workspace_bytes.argtypes = [cfgp, i32, i32]
    lib.hattn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.hattn_decode.argtypes = [cfgp, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp,
                                 ctypes.c_size_t, u32, vp]
    lib.hattn_decode.restype = i32
    lib.hattn_decode_noalloc.argtypes = [cfgp, vp, vp, vp, i32, vp, i32, vp, vp, vp, u32, vp]
    lib.hattn_decode_noalloc.restype = i32
    lib.hattn_status_string.argtypes = [i32]
    lib.hattn_status_string.restype = ctypes.c_char_p
    lib.hattn_last_hip_error.argtypes = []
    lib.hattn_last_hip_error.restype = i32
    return lib


_lib = _load()


def lib():
    return _lib


def preset(kind) -> LayerCfg:
    k = {"sliding": HATTN_SLIDING, "full": HATTN_FULL}.get(kind, kind)
    cfg = LayerCfg()
    st = _lib.hattn_cfg_preset(int(k), ctypes.byref(cfg))
    if st != HATTN_OK:
        raise HattnError(st, "hattn_cfg_preset")
    return cfg


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("hattn: tensors must be contiguous (the C ABI takes dense layouts)")
    return ctypes.c_void_p(t.data_ptr())


_BF16, _F32, _I32, _U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


class _Args:
    """Marshalling checks of one call's tensor arguments before their pointers cross the C
    ABI, which cannot see sizes or devices.  Each argument is checked for its dtype and its
    shape (None entries match any extent) or element count as it is named; done() then
    requires every named tensor to be GPU-resident and contiguous.  A wrong size would
    reach the kernels as an out-of-bounds device access, so it is a ValueError instead."""

    def __init__(self, where):
        self.where, self.seen = where, []

    def __call__(self, name, t, dtype, shape=None, numel=None, optional=False):
        w = self.where
        if t is None:
            if optional:
                return
            raise ValueError(f"{w}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{w}: {name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise ValueError(f"{w}: {name} must be {dtype}, got {t.dtype}")
        if shape is not None:
            ok = t.dim() == len(shape) and all(e is None or int(d) == e
                                               for d, e in zip(t.shape, shape))
            if not ok:
                want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
                raise ValueError(f"{w}: {name} must have shape {want}, got {list(t.shape)}")
        if numel is not None and t.numel() < numel:
            raise ValueError(f"{w}: {name} holds {t.numel()} elements, needs {numel}")
        self.seen.append((name, t))

    def done(self):
        for name, t in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{self.where}: {name} must be in GPU memory "
                                 f"(got device {t.device})")
            if not t.is_contiguous():
                raise ValueError(f"{self.where}: {name} must be contiguous")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st, where):
    if st != HATTN_OK:
        raise HattnError(st, where)


def rope_qk(cfg: LayerCfg, q, k, pos0, stream=None):
    """In-place RoPE on q [B,S,16,256] and/or k [B,S,4,256] (bf16, device)."""
    a = _Args("rope_qk")
    t = q if q is not None else k
    if t is None:
        raise ValueError("rope_qk: q and k are both None")
    B, S = int(t.shape[0]), int(t.shape[1])
    a("q", q, _BF16, (B, S, 16, 256), optional=True)
    a("k", k, _BF16, (B, S, 4, 256), optional=True)
    a("pos0", pos0, _I32, numel=B)
    a.done()
    _check(_lib.hattn_rope_qk(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(pos0), B, S,
                              _stream(stream)), "hattn_rope_qk")


def _append_args(where, k_new, v_new, k_cache, v_cache, pos0, slots_out):
    a = _Args(where)
    B, n = int(k_new.shape[0]), int(k_new.shape[1])
    a("k_new", k_new, _BF16, (B, n, 4, 256))
    a("v_new", v_new, _BF16, (B, n, 4, 256))
    a("k_cache", k_cache, _BF16, (B, None, 4, 256))
    a("v_cache", v_cache, _BF16, tuple(k_cache.shape))
    a("pos0", pos0, _I32, numel=B)
    a("slots_out", slots_out, _I32, (B, n), optional=True)
    a.done()
    return B, n


def kv_append(cfg: LayerCfg, k_new, v_new, k_cache, v_cache, pos0, slots_out=None, stream=None):
    B, n = _append_args("kv_append", k_new, v_new, k_cache, v_cache, pos0, slots_out)
    _check(_lib.hattn_kv_append(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                _ptr(v_cache), int(k_cache.shape[1]), _ptr(pos0), B, n,
                                _ptr(slots_out), _stream(stream)), "hattn_kv_append")


def kv_append_rope(cfg: LayerCfg, k_new, v_new, k_cache, v_cache, pos0, slots_out=None,
                   stream=None):
    """kv_append with unrotated k_new, rotated by position on the way into the cache."""
    B, n = _append_args("kv_append_rope", k_new, v_new, k_cache, v_cache, pos0, slots_out)
    _check(_lib.hattn_kv_append_rope(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                     _ptr(v_cache), int(k_cache.shape[1]), _ptr(pos0), B, n,
                                     _ptr(slots_out), _stream(stream)), "hattn_kv_append_rope")


def _attn_out_args(a, B, S, gate, out, lse, prefix=""):
    a(prefix + "gate", gate, _BF16, (B, S, 16))
    a(prefix + "out", out, _BF16, (B, S, 16, 256))
    a(prefix + "lse", lse, _F32, (B, S, 16), optional=True)


def prefill(cfg: LayerCfg, q, k_cache, v_cache, pos0, gate, out, lse=None,
            rope_q_fused: bool = True, stream=None):
    a = _Args("prefill")
    B, Sq = int(q.shape[0]), int(q.shape[1])
    a("q", q, _BF16, (B, Sq, 16, 256))
    a("k_cache", k_cache, _BF16, (B, None, 4, 256))
    a("v_cache", v_cache, _BF16, tuple(k_cache.shape))
    a("pos0", pos0, _I32, numel=B)
    _attn_out_args(a, B, Sq, gate, out, lse)
    a.done()
    flags = HATTN_ROPE_Q_FUSED if rope_q_fused else 0
    _check(_lib.hattn_prefill(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              int(k_cache.shape[1]), _ptr(pos0), B, Sq, _ptr(gate), _ptr(out),
                              _ptr(lse), flags, _stream(stream)), "hattn_prefill")


def prefill_ring(cfg: LayerCfg, q, k_new, v_new, k_ring, v_ring, pos0, gate, out, lse=None,
                 rope_q_fused: bool = True, stream=None):
    """Sliding-layer chunk that continues the 512-slot rings k_ring / v_ring [B,512,4,256];
    k_new / v_new [B,Sq,4,256] are the chunk's rotated keys and values."""
    a = _Args("prefill_ring")
    B, Sq = int(q.shape[0]), int(q.shape[1])
    a("q", q, _BF16, (B, Sq, 16, 256))
    a("k_new", k_new, _BF16, (B, Sq, 4, 256))
    a("v_new", v_new, _BF16, (B, Sq, 4, 256))
    a("k_ring", k_ring, _BF16, (B, 512, 4, 256))
    a("v_ring", v_ring, _BF16, (B, 512, 4, 256))
    a("pos0", pos0, _I32, numel=B)
    _attn_out_args(a, B, Sq, gate, out, lse)
    a.done()
    flags = HATTN_ROPE_Q_FUSED if rope_q_fused else 0
    _check(_lib.hattn_prefill_ring(ctypes.byref(cfg), _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_ring), _ptr(v_ring), _ptr(pos0), B, Sq, _ptr(gate),
                                   _ptr(out), _ptr(lse), flags, _stream(stream)),
           "hattn_prefill_ring")


def decode_workspace_bytes(cfg: LayerCfg, B: int, cap: int) -> int:
    return int(_lib.hattn_decode_workspace_bytes(ctypes.byref(cfg), int(B), int(cap)))


def decode(cfg: LayerCfg, q, k_cache, v_cache, pos, gate, out, lse=None, workspace=None,
           rope_q_fused: bool = False, stream=None):
    a = _Args("decode")
    B = int(q.shape[0])
    a("q", q, _BF16, (B, 1, 16, 256))
    a("k_cache", k_cache, _BF16, (B, None, 4, 256))
    a("v_cache", v_cache, _BF16, tuple(k_cache.shape))
    a("pos", pos, _I32, numel=B)
    _attn_out_args(a, B, 1, gate, out, lse)
    a("workspace", workspace, _U8, optional=True)
    a.done()
    cap = int(k_cache.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = HATTN_ROPE_Q_FUSED if rope_q_fused else 0
    _check(_lib.hattn_decode(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache), cap,
                             _ptr(pos), B, _ptr(gate), _ptr(out), _ptr(lse), _ptr(workspace),
                             ws_bytes, flags, _stream(stream)), "hattn_decode")


def decode_noalloc(cfg: LayerCfg, q, k_cache, v_cache, pos, gate, out, lse=None,
                   rope_q_fused: bool = False, stream=None):
    """decode() without a workspace: the library's static per-device scratch holds the
    partials (calls that overlap on one GPU race on it)."""
    a = _Args("decode_noalloc")
    B = int(q.shape[0])
    a("q", q, _BF16, (B, 1, 16, 256))
    a("k_cache", k_cache, _BF16, (B, None, 4, 256))
    a("v_cache", v_cache, _BF16, tuple(k_cache.shape))
    a("pos", pos, _I32, numel=B)
    _attn_out_args(a, B, 1, gate, out, lse)
    a.done()
    flags = HATTN_ROPE_Q_FUSED if rope_q_fused else 0
    _check(_lib.hattn_decode_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     int(k_cache.shape[1]), _ptr(pos), B, _ptr(gate), _ptr(out),
                                     _ptr(lse), flags, _stream(stream)), "hattn_decode_noalloc")


def alloc_workspace(cfg: LayerCfg, B: int, cap: int, device="cuda"):
    n = decode_workspace_bytes(cfg, B, cap)
    return torch.empty(max(16, n), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ whole-model driver --
def model_layer_kind(layer: int) -> str:
    return "full" if _lib.hattn_model_layer_kind(int(layer)) == HATTN_FULL else "sliding"


def model_kv_bytes(n_layers: int, B: int, cap: int):
    """(per-layer KV bytes, total) of the layer schedule."""
    per = (ctypes.c_size_t * n_layers)()
    tot = ctypes.c_size_t(0)
    _check(_lib.hattn_model_kv_bytes(n_layers, B, cap, per, ctypes.byref(tot)),
           "hattn_model_kv_bytes")
    return list(per), int(tot.value)


def _layer_array(where, layers, cap, pos_name, pos, workspace):
    """The LayerIO array of a schedule, after checking every layer's tensors (q / k / v /
    gate / out / lse of one B x S shape, full caches [B, cap, 4, 256], rings
    [B, 512, 4, 256]), the position array and the workspace.  Returns (array, B, S)."""
    if not layers:
        raise ValueError(f"{where}: no layers")
    a = _Args(where)
    B, S = int(layers[0]["q"].shape[0]), int(layers[0]["q"].shape[1])
    for l, L in enumerate(layers):
        rows = 512 if model_layer_kind(l) == "sliding" else cap
        pre = f"layer {l} "
        a(pre + "q", L.get("q"), _BF16, (B, S, 16, 256))
        a(pre + "k", L.get("k"), _BF16, (B, S, 4, 256))
        a(pre + "v", L.get("v"), _BF16, (B, S, 4, 256))
        a(pre + "k_cache", L.get("k_cache"), _BF16, (B, rows, 4, 256))
        a(pre + "v_cache", L.get("v_cache"), _BF16, (B, rows, 4, 256))
        _attn_out_args(a, B, S, L.get("gate"), L.get("out"), L.get("lse"), prefix=pre)
    a(pos_name, pos, _I32, numel=B)
    a("workspace", workspace, _U8, optional=True)   # the library says when one is needed
    a.done()
    arr = (LayerIO * len(layers))()
    for i, L in enumerate(layers):
        for name in ("q", "k", "v", "gate", "k_cache", "v_cache", "out", "lse"):
            p = _ptr(L.get(name))
            setattr(arr[i], name, None if p is None else p.value)
    return arr, B, S


def model_decode_workspace_bytes(n_layers: int, B: int, cap: int) -> int:
    return int(_lib.hattn_model_decode_workspace_bytes(n_layers, B, cap))


def model_prefill_workspace_bytes(n_layers: int, B: int, Sq: int) -> int:
    return int(_lib.hattn_model_prefill_workspace_bytes(n_layers, B, Sq))


def model_decode(layers, cap: int, pos, workspace, stream=None):
    """One decode step of every layer; layers: list of dicts with the LayerIO fields."""
    arr, B, _ = _layer_array("model_decode", layers, cap, "pos", pos, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.hattn_model_decode(arr, len(layers), cap, _ptr(pos), B, _ptr(workspace),
                                   ws_bytes, _stream(stream)),
           "hattn_model_decode")


def model_prefill(layers, cap: int, pos0, workspace, stream=None):
    """One prefill chunk through every layer (chunks in position order)."""
    arr, B, Sq = _layer_array("model_prefill", layers, cap, "pos0", pos0, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.hattn_model_prefill(arr, len(layers), cap, _ptr(pos0), B, Sq, _ptr(workspace),
                                    ws_bytes,
                                    _stream(stream)), "hattn_model_prefill")


# ------------------------------------------------------------------------ 8-bit KV cache --
def _kv8_cache_args(a, B, k_cache, v_cache, k_scale, v_scale):
    a("k_cache", k_cache, _U8, (B, None, 4, 256))
    cap = int(k_cache.shape[1])
    a("v_cache", v_cache, _U8, (B, cap, 4, 256))
    a("k_scale", k_scale, _F32, (B, 4, cap))
    a("v_scale", v_scale, _F32, (B, 4, cap))
    return cap


def kv_append_fp8(cfg: LayerCfg, k_new, v_new, k_cache, v_cache, k_scale, v_scale, pos0,
                  slots_out=None, rope_k: bool = False, stream=None):
    """Quantize and append into an 8-bit cache (uint8 [B,cap,4,256], scales fp32 [B,4,cap])."""
    a = _Args("kv_append_fp8")
    B, n = int(k_new.shape[0]), int(k_new.shape[1])
    a("k_new", k_new, _BF16, (B, n, 4, 256))
    a("v_new", v_new, _BF16, (B, n, 4, 256))
    cap = _kv8_cache_args(a, B, k_cache, v_cache, k_scale, v_scale)
    a("pos0", pos0, _I32, numel=B)
    a("slots_out", slots_out, _I32, (B, n), optional=True)
    a.done()
    _check(_lib.hattn_kv_append_fp8(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                    _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), cap, _ptr(pos0),
                                    B, n, _ptr(slots_out), HATTN_KV8_ROPE_K if rope_k else 0,
                                    _stream(stream)), "hattn_kv_append_fp8")


def alloc_workspace_fp8(cfg: LayerCfg, B: int, cap: int, device="cuda"):
    """Workspace of decode_fp8 (its split-KV partials, for both layer kinds)."""
    n = int(_lib.hattn_decode_fp8_workspace_bytes(ctypes.byref(cfg), int(B), int(cap)))
    return torch.empty(max(16, n), dtype=torch.uint8, device=device)


def decode_fp8(cfg: LayerCfg, q, k_cache, v_cache, k_scale, v_scale, pos, gate, out, lse=None,
               workspace=None, rope_q_fused: bool = False, stream=None):
    a = _Args("decode_fp8")
    B = int(q.shape[0])
    a("q", q, _BF16, (B, 1, 16, 256))
    cap = _kv8_cache_args(a, B, k_cache, v_cache, k_scale, v_scale)
    a("pos", pos, _I32, numel=B)
    _attn_out_args(a, B, 1, gate, out, lse)
    a("workspace", workspace, _U8)
    a.done()
    flags = HATTN_ROPE_Q_FUSED if rope_q_fused else 0
    _check(_lib.hattn_decode_fp8(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(k_scale), _ptr(v_scale), cap, _ptr(pos), B, _ptr(gate),
                                 _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), flags,
                                 _stream(stream)), "hattn_decode_fp8")


# ------------------------------------------------------------------ projections --
def qkv_proj(x, w_qkv, w_gate, q, k, v, gate, stream=None):
    """x [T,2560] -> q [T,16,256], k/v [T,4,256], gate [T,16] (any leading batch dims that
    flatten to T)."""
    a = _Args("qkv_proj")
    if x.shape[-1] != 2560:
        raise ValueError(f"qkv_proj: x must end in the hidden size 2560, got {list(x.shape)}")
    T = int(x.numel() // x.shape[-1])
    a("x", x, _BF16)
    a("w_qkv", w_qkv, _BF16, (6144, 2560))
    a("w_gate", w_gate, _BF16, (16, 2560))
    a("q", q, _BF16, numel=T * 4096)
    a("k", k, _BF16, numel=T * 1024)
    a("v", v, _BF16, numel=T * 1024)
    a("gate", gate, _BF16, numel=T * 16)
    a.done()
    _check(_lib.hattn_qkv_proj(_ptr(x), T, _ptr(w_qkv), _ptr(w_gate), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(gate), _stream(stream)), "hattn_qkv_proj")


def o_proj(attn, w_o, y, stream=None):
    """attn [T,16,256] -> y [T,2560]."""
    a = _Args("o_proj")
    if attn.numel() % 4096:
        raise ValueError(f"o_proj: attn must hold whole 16 x 256 head rows, got {list(attn.shape)}")
    T = int(attn.numel() // 4096)
    a("attn", attn, _BF16)
    a("w_o", w_o, _BF16, (2560, 4096))
    a("y", y, _BF16, numel=T * 2560)
    a.done()
    _check(_lib.hattn_o_proj(_ptr(attn), T, _ptr(w_o), _ptr(y), _stream(stream)), "hattn_o_proj")
