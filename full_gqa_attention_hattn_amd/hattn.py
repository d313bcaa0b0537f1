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
HATTN_SLIDING = 0
HATTN_FULL = 1
HATTN_ROPE_Q_FUSED = 1
HATTN_KV8_ROPE_K = 1

# Every symbol include/hattn.h declares.
EXPORTS = ("hattn_cfg_preset", "hattn_rope_qk", "hattn_kv_append", "hattn_kv_append_rope",
           "hattn_prefill", "hattn_prefill_ring", "hattn_kv_append_fp8", "hattn_decode_fp8",
           "hattn_qkv_proj", "hattn_o_proj",
           "hattn_decode_workspace_bytes", "hattn_decode", "hattn_model_layer_kind",
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


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st, where):
    if st != HATTN_OK:
        raise HattnError(st, where)


def rope_qk(cfg: LayerCfg, q, k, pos0, stream=None):
    """In-place RoPE on q [B,S,16,256] and/or k [B,S,4,256] (bf16, device)."""
    t = q if q is not None else k
    B, S = int(t.shape[0]), int(t.shape[1])
    _check(_lib.hattn_rope_qk(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(pos0), B, S,
                              _stream(stream)), "hattn_rope_qk")


def kv_append(cfg: LayerCfg, k_new, v_new, k_cache, v_cache, pos0, slots_out=None, stream=None):
    B, n = int(k_new.shape[0]), int(k_new.shape[1])
    _check(_lib.hattn_kv_append(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                _ptr(v_cache), int(k_cache.shape[1]), _ptr(pos0), B, n,
                                _ptr(slots_out), _stream(stream)), "hattn_kv_append")


def kv_append_rope(cfg: LayerCfg, k_new, v_new, k_cache, v_cache, pos0, slots_out=None,
                   stream=None):
    """kv_append with unrotated k_new, rotated by position on the way into the cache."""
    B, n = int(k_new.shape[0]), int(k_new.shape[1])
    _check(_lib.hattn_kv_append_rope(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                     _ptr(v_cache), int(k_cache.shape[1]), _ptr(pos0), B, n,
                                     _ptr(slots_out), _stream(stream)), "hattn_kv_append_rope")


def prefill(cfg: LayerCfg, q, k_cache, v_cache, pos0, gate, out, lse=None,
            rope_q_fused: bool = True, stream=None):
    B, Sq = int(q.shape[0]), int(q.shape[1])
    flags = HATTN_ROPE_Q_FUSED if rope_q_fused else 0
    _check(_lib.hattn_prefill(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              int(k_cache.shape[1]), _ptr(pos0), B, Sq, _ptr(gate), _ptr(out),
                              _ptr(lse), flags, _stream(stream)), "hattn_prefill")


def prefill_ring(cfg: LayerCfg, q, k_new, v_new, k_ring, v_ring, pos0, gate, out, lse=None,
                 rope_q_fused: bool = True, stream=None):
    """Sliding-layer chunk that continues the 512-slot rings k_ring / v_ring [B,512,4,256];
    k_new / v_new [B,Sq,4,256] are the chunk's rotated keys and values."""
    B, Sq = int(q.shape[0]), int(q.shape[1])
    flags = HATTN_ROPE_Q_FUSED if rope_q_fused else 0
    _check(_lib.hattn_prefill_ring(ctypes.byref(cfg), _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_ring), _ptr(v_ring), _ptr(pos0), B, Sq, _ptr(gate),
                                   _ptr(out), _ptr(lse), flags, _stream(stream)),
           "hattn_prefill_ring")


def decode_workspace_bytes(cfg: LayerCfg, B: int, cap: int) -> int:
    return int(_lib.hattn_decode_workspace_bytes(ctypes.byref(cfg), int(B), int(cap)))


def decode(cfg: LayerCfg, q, k_cache, v_cache, pos, gate, out, lse=None, workspace=None,
           rope_q_fused: bool = False, stream=None):
    B = int(q.shape[0])
    cap = int(k_cache.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = HATTN_ROPE_Q_FUSED if rope_q_fused else 0
    _check(_lib.hattn_decode(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache), cap,
                             _ptr(pos), B, _ptr(gate), _ptr(out), _ptr(lse), _ptr(workspace),
                             ws_bytes, flags, _stream(stream)), "hattn_decode")


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


def _layer_array(layers):
    arr = (LayerIO * len(layers))()
    for i, L in enumerate(layers):
        for name in ("q", "k", "v", "gate", "k_cache", "v_cache", "out", "lse"):
            t = L.get(name)
            p = _ptr(t)
            setattr(arr[i], name, None if p is None else p.value)
    return arr


def model_decode_workspace_bytes(n_layers: int, B: int, cap: int) -> int:
    return int(_lib.hattn_model_decode_workspace_bytes(n_layers, B, cap))


def model_prefill_workspace_bytes(n_layers: int, B: int, Sq: int) -> int:
    return int(_lib.hattn_model_prefill_workspace_bytes(n_layers, B, Sq))


def model_decode(layers, cap: int, pos, workspace, stream=None):
    """One decode step of every layer; layers: list of dicts with the LayerIO fields."""
    arr = _layer_array(layers)
    B = int(layers[0]["q"].shape[0])
    _check(_lib.hattn_model_decode(arr, len(layers), cap, _ptr(pos), B, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "hattn_model_decode")


def model_prefill(layers, cap: int, pos0, workspace, stream=None):
    """One prefill chunk through every layer (chunks in position order)."""
    arr = _layer_array(layers)
    B, Sq = int(layers[0]["q"].shape[0]), int(layers[0]["q"].shape[1])
    _check(_lib.hattn_model_prefill(arr, len(layers), cap, _ptr(pos0), B, Sq, _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "hattn_model_prefill")


# ------------------------------------------------------------------------ 8-bit KV cache --
def kv_append_fp8(cfg: LayerCfg, k_new, v_new, k_cache, v_cache, k_scale, v_scale, pos0,
                  slots_out=None, rope_k: bool = False, stream=None):
    """Quantize and append into an 8-bit cache (uint8 [B,cap,4,256], scales fp32 [B,4,cap])."""
    B, n = int(k_new.shape[0]), int(k_new.shape[1])
    _check(_lib.hattn_kv_append_fp8(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                    _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                    int(k_cache.shape[1]), _ptr(pos0), B, n, _ptr(slots_out),
                                    HATTN_KV8_ROPE_K if rope_k else 0, _stream(stream)),
           "hattn_kv_append_fp8")


def decode_fp8(cfg: LayerCfg, q, k_cache, v_cache, k_scale, v_scale, pos, gate, out, lse=None,
               workspace=None, rope_q_fused: bool = False, stream=None):
    B = int(q.shape[0])
    cap = int(k_cache.shape[1])
    if workspace is None:
        raise ValueError("decode_fp8 needs a workspace (alloc_workspace)")
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
    T = int(x.numel() // x.shape[-1])
    _check(_lib.hattn_qkv_proj(_ptr(x), T, _ptr(w_qkv), _ptr(w_gate), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(gate), _stream(stream)), "hattn_qkv_proj")


def o_proj(attn, w_o, y, stream=None):
    """attn [T,16,256] -> y [T,2560]."""
    T = int(attn.numel() // 4096)
    _check(_lib.hattn_o_proj(_ptr(attn), T, _ptr(w_o), _ptr(y), _stream(stream)), "hattn_o_proj")
