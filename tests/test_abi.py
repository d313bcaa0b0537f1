"""The C-ABI library loads and exports every symbol include/hattn.h declares, and its host
argument validation returns the documented status codes.  No call here reaches a kernel
launch (every case fails validation first or has an empty size), so this runs without a
GPU."""
import ctypes
import pathlib
import re

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "hattn.h"
LIBPATH = ROOT / "full_gqa_attention_hattn_amd" / "libhattn.so"

pytestmark = pytest.mark.skipif(not LIBPATH.exists(), reason="libhattn.so not built")


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(hattn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def h():
    from full_gqa_attention_hattn_amd import hattn
    return hattn


def test_exports_every_declared_symbol(h):
    decl = declared_functions()
    assert len(decl) >= 8
    assert sorted(h.EXPORTS) == decl
    lib = ctypes.CDLL(str(LIBPATH))
    for name in decl:
        assert hasattr(lib, name), name


def test_header_serves_a_plain_c_caller(tmp_path):
    """include/hattn.h compiles as strict C99 and C++17, and a C program linked against
    libhattn.so gets the documented presets, sizes, schedule, validation codes and status
    strings (tests/c_abi_smoke.c; nothing there touches a GPU)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++17")):
        subprocess.run([gcc if lang == "c" else (shutil.which("g++") or gcc), std, "-Wall",
                        "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", lang,
                        str(HEADER)], check=True)
    exe = tmp_path / "c_abi_smoke"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", str(HEADER.parent), str(ROOT / "tests" / "c_abi_smoke.c"),
                    "-L", str(LIBPATH.parent), "-lhattn", f"-Wl,-rpath,{LIBPATH.parent}",
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_presets(h):
    s, f = h.preset("sliding"), h.preset("full")
    assert (s.kind, s.window, s.rot_dim, s.rope_theta) == (0, 512, 256, 1e4)
    assert (f.kind, f.window, f.rot_dim, f.rope_theta) == (1, 0, 64, 5e6)
    for c in (s, f):
        assert (c.n_q_heads, c.n_kv_heads, c.head_dim, c.softmax_scale) == (16, 4, 256, 0.0625)
    lib = h.lib()
    assert lib.hattn_cfg_preset(7, ctypes.byref(h.LayerCfg())) == h.HATTN_ERR_UNSUPPORTED
    assert lib.hattn_cfg_preset(0, None) == h.HATTN_ERR_NULL


def test_status_strings(h):
    lib = h.lib()
    seen = set()
    for st in range(9):
        s = lib.hattn_status_string(st).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.hattn_status_string(99).decode() == "unknown status"
    assert lib.hattn_last_hip_error() == 0


P = ctypes.c_void_p
A = P(0x10000)          # a 16-byte-aligned stand-in address (never dereferenced)
MIS = P(0x10008)        # 8-byte aligned only


def _cfg(h, preset_kind="full", **kw):
    c = h.preset(preset_kind)
    for k, v in kw.items():
        setattr(c, k, v)
    return ctypes.byref(c)


@pytest.mark.parametrize("field,val", [("n_q_heads", 8), ("n_kv_heads", 8), ("head_dim", 128),
                                       ("window", 256), ("rot_dim", 128), ("rope_theta", 1e6),
                                       ("softmax_scale", 0.1), ("reserved", 1), ("kind", 2)])
def test_unsupported_config(h, field, val):
    lib = h.lib()
    c = _cfg(h, "sliding", **{field: val})
    assert lib.hattn_rope_qk(c, A, A, A, 1, 1, None) == h.HATTN_ERR_UNSUPPORTED
    assert lib.hattn_prefill(c, A, A, A, 8, A, 1, 1, A, A, None, 0, None) == h.HATTN_ERR_UNSUPPORTED
    assert lib.hattn_decode_workspace_bytes(c, 1, 512) == 0


def test_rope_validation(h):
    lib = h.lib()
    c = _cfg(h)
    assert lib.hattn_rope_qk(None, A, A, A, 1, 1, None) == h.HATTN_ERR_NULL
    assert lib.hattn_rope_qk(c, None, None, A, 1, 1, None) == h.HATTN_ERR_NULL
    assert lib.hattn_rope_qk(c, A, None, None, 1, 1, None) == h.HATTN_ERR_NULL
    assert lib.hattn_rope_qk(c, A, None, A, -1, 1, None) == h.HATTN_ERR_SHAPE
    assert lib.hattn_rope_qk(c, MIS, None, A, 1, 1, None) == h.HATTN_ERR_ALIGN
    assert lib.hattn_rope_qk(c, None, MIS, A, 1, 1, None) == h.HATTN_ERR_ALIGN
    assert lib.hattn_rope_qk(c, A, A, P(0x10002), 1, 1, None) == h.HATTN_ERR_ALIGN
    assert lib.hattn_rope_qk(c, A, A, A, 0, 5, None) == h.HATTN_OK       # empty: no launch
    assert lib.hattn_rope_qk(c, A, A, A, 3, 0, None) == h.HATTN_OK
    assert lib.hattn_rope_qk(c, None, None, None, 0, 0, None) == h.HATTN_OK  # empty: no pointers needed


@pytest.mark.parametrize("fn", ["hattn_kv_append", "hattn_kv_append_rope"])
def test_append_validation(h, fn):
    lib = h.lib()
    f, s = _cfg(h, "full"), _cfg(h, "sliding")
    ok = (A, A, A, A)
    lib = type("L", (), {"hattn_kv_append": getattr(lib, fn)})
    assert lib.hattn_kv_append(f, None, A, A, A, 8, A, 1, 1, None, None) == h.HATTN_ERR_NULL
    assert lib.hattn_kv_append(f, *ok, 8, None, 1, 1, None, None) == h.HATTN_ERR_NULL
    assert lib.hattn_kv_append(f, *ok, 0, A, 1, 1, None, None) == h.HATTN_ERR_SHAPE
    assert lib.hattn_kv_append(f, *ok, 8, A, 1, -2, None, None) == h.HATTN_ERR_SHAPE
    assert lib.hattn_kv_append(s, *ok, 511, A, 1, 1, None, None) == h.HATTN_ERR_RANGE
    assert lib.hattn_kv_append(s, *ok, 1024, A, 1, 1, None, None) == h.HATTN_ERR_RANGE
    assert lib.hattn_kv_append(f, A, A, MIS, A, 8, A, 1, 1, None, None) == h.HATTN_ERR_ALIGN
    assert lib.hattn_kv_append(f, *ok, 8, A, 1, 1, P(0x10001), None) == h.HATTN_ERR_ALIGN
    assert lib.hattn_kv_append(s, *ok, 512, A, 0, 1, None, None) == h.HATTN_OK
    assert lib.hattn_kv_append(f, *ok, 8, A, 4, 0, None, None) == h.HATTN_OK


def test_prefill_validation(h):
    lib = h.lib()
    c = _cfg(h, "sliding")
    args = lambda **o: [o.get(k, v) for k, v in (("q", A), ("k", A), ("v", A), ("cap", 64),
                                                   ("pos", A), ("B", 1), ("S", 8), ("g", A),
                                                   ("out", A), ("lse", None), ("flags", 0))]
    for k in ("q", "k", "v", "pos", "g", "out"):
        assert lib.hattn_prefill(c, *args(**{k: None}), None) == h.HATTN_ERR_NULL, k
    assert lib.hattn_prefill(c, *args(S=-1), None) == h.HATTN_ERR_SHAPE
    assert lib.hattn_prefill(c, *args(cap=0), None) == h.HATTN_ERR_SHAPE
    assert lib.hattn_prefill(c, *args(flags=6), None) == h.HATTN_ERR_UNSUPPORTED
    for k in ("q", "k", "v", "out"):
        assert lib.hattn_prefill(c, *args(**{k: MIS}), None) == h.HATTN_ERR_ALIGN, k
    assert lib.hattn_prefill(c, *args(g=P(0x10001)), None) == h.HATTN_ERR_ALIGN
    assert lib.hattn_prefill(c, *args(lse=P(0x10002)), None) == h.HATTN_ERR_ALIGN
    assert lib.hattn_prefill(c, *args(S=0), None) == h.HATTN_OK
    assert lib.hattn_prefill(c, *args(B=0), None) == h.HATTN_OK
    # grid would exceed the 32-bit work-item range
    assert lib.hattn_prefill(c, *args(B=65536, S=1 << 15), None) == h.HATTN_ERR_SHAPE


def test_prefill_ring_validation(h):
    lib = h.lib()
    s, f = _cfg(h, "sliding"), _cfg(h, "full")
    names = ("q", "kn", "vn", "kr", "vr", "pos", "B", "S", "g", "out", "lse", "flags")
    base = dict(q=A, kn=A, vn=A, kr=A, vr=A, pos=A, B=2, S=40, g=A, out=A, lse=None, flags=0)

    def call(cfg=s, **o):
        a = dict(base, **o)
        return lib.hattn_prefill_ring(cfg, *[a[k] for k in names], None)

    assert call(cfg=f) == h.HATTN_ERR_UNSUPPORTED         # ring continuation is sliding-only
    assert call(cfg=None) == h.HATTN_ERR_NULL
    for k in ("q", "kn", "vn", "kr", "vr", "pos", "g", "out"):
        assert call(**{k: None}) == h.HATTN_ERR_NULL, k
        if k not in ("pos", "g"):
            assert call(**{k: MIS}) == h.HATTN_ERR_ALIGN, k
    assert call(g=P(0x10001)) == h.HATTN_ERR_ALIGN
    assert call(pos=P(0x10002)) == h.HATTN_ERR_ALIGN
    assert call(lse=P(0x10002)) == h.HATTN_ERR_ALIGN
    assert call(S=-1) == h.HATTN_ERR_SHAPE
    assert call(B=-1) == h.HATTN_ERR_SHAPE
    assert call(flags=2) == h.HATTN_ERR_UNSUPPORTED
    assert call(B=65536, S=1 << 15) == h.HATTN_ERR_SHAPE
    assert call(S=0, q=None, kn=None) == h.HATTN_OK     # empty: no launch, pointers unread
    assert call(B=0) == h.HATTN_OK


def test_decode_validation_and_workspace(h):
    lib = h.lib()
    f, s = _cfg(h, "full"), _cfg(h, "sliding")
    need = lib.hattn_decode_workspace_bytes(f, 32, 131136)
    assert need > 0 and need % 16 == 0
    # sliding layers: the ring split's partials (8 splits up to B = 8, 4 above; 4 heads x
    # (256 + 2) floats each) and a counter per (sequence, KV head)
    for B, splits in ((1, 8), (2, 8), (8, 8), (9, 4), (32, 4)):
        assert lib.hattn_decode_workspace_bytes(s, B, 512) == \
            B * 4 * splits * 4 * 258 * 4 + B * 4 * 4, B
    assert lib.hattn_decode_workspace_bytes(s, 32, 513) == 0
    assert lib.hattn_decode_workspace_bytes(f, -1, 8) == 0

    def call(cfg=f, q=A, k=A, v=A, cap=131136, pos=A, B=32, g=A, out=A, lse=None, ws=A,
             wsb=need, flags=0):
        return lib.hattn_decode(cfg, q, k, v, cap, pos, B, g, out, lse, ws, wsb, flags, None)

    for kw in ("q", "k", "v", "pos", "g", "out"):
        assert call(**{kw: None}) == h.HATTN_ERR_NULL, kw
    assert call(ws=None) == h.HATTN_ERR_WORKSPACE
    assert call(wsb=need - 1) == h.HATTN_ERR_WORKSPACE
    assert call(ws=MIS) == h.HATTN_ERR_ALIGN
    assert call(cfg=s, cap=131136, wsb=1 << 40) == h.HATTN_ERR_RANGE
    assert call(q=MIS) == h.HATTN_ERR_ALIGN
    assert call(flags=2) == h.HATTN_ERR_UNSUPPORTED
    assert call(B=70000, wsb=1 << 50) == h.HATTN_ERR_SHAPE
    assert call(cap=0) == h.HATTN_ERR_SHAPE
    assert call(B=0) == h.HATTN_OK


def test_decode_fp8_workspace_holds_the_split_for_both_kinds(h):
    """The 8-bit decode splits the keys for both layer kinds (a sliding layer's window of
    the position-indexed cache too), so its workspace is the split-KV partials."""
    lib = h.lib()
    f, s = _cfg(h, "full"), _cfg(h, "sliding")
    for B in (1, 2, 3, 32):
        n = lib.hattn_decode_fp8_workspace_bytes(s, B, 512)
        assert n >= B * 4 * 4 * 258 * 4 and n % (B * 4 * 4 * 258 * 4) == 0, B
    assert lib.hattn_decode_fp8_workspace_bytes(s, 3, 513) == 0
    assert lib.hattn_decode_fp8_workspace_bytes(f, 32, 131136) == \
        lib.hattn_decode_workspace_bytes(f, 32, 131136)


def test_decode_workspace_scales_with_plan(h):
    lib = h.lib()
    f = _cfg(h, "full")
    # partials: B x 4 kv heads x chunks x 4 heads x (256 + 2) floats
    for B, cap in ((1, 1 << 20), (32, 131136), (3, 100)):
        n = lib.hattn_decode_workspace_bytes(f, B, cap)
        per_chunk = B * 4 * 4 * 258 * 4
        assert n % per_chunk == 0 and n >= per_chunk


# ------------------------------------------------------------------ whole-model driver --
def test_model_schedule_and_kv_bytes_match_oracle_and_pages(h):
    import oracle as O
    sched = O.layer_schedule(36)
    assert [h.model_layer_kind(l) for l in range(36)] == sched
    assert h.lib().hattn_model_layer_kind(-1) == -1
    per, total = h.model_kv_bytes(36, 1, 1 << 20)
    assert total == O.kv_cache_bytes(1 << 20)                        # 9 full + 27 rings
    assert total == 9 * 4096 * (1 << 20) + 27 * 4096 * 512
    assert [p == 4096 * (1 << 20) for p in per] == [k == "full" for k in sched]
    _, t32 = h.model_kv_bytes(36, 32, 131073)
    assert t32 == 32 * O.kv_cache_bytes(131073)


def test_model_validation(h):
    lib = h.lib()
    io = (h.LayerIO * 4)()
    for L in io:
        for n in ("q", "k", "v", "gate", "k_cache", "v_cache", "out"):
            setattr(L, n, 0x10000)
    need = lib.hattn_model_decode_workspace_bytes(4, 2, 1024)
    assert need > 0 and lib.hattn_model_decode_workspace_bytes(0, 2, 1024) == 0
    dec = lambda **o: lib.hattn_model_decode(o.get("io", io), o.get("n", 4), o.get("cap", 1024),
                                             o.get("pos", A), o.get("B", 2), o.get("ws", A),
                                             o.get("wsb", need), None)
    assert dec(n=0) == h.HATTN_ERR_SHAPE
    assert dec(cap=511) == h.HATTN_ERR_SHAPE
    assert dec(B=65536) == h.HATTN_ERR_SHAPE          # a grid's y extent; no layer is enqueued
    assert dec(io=None) == h.HATTN_ERR_NULL
    assert dec(pos=None) == h.HATTN_ERR_NULL
    assert dec(ws=None) == h.HATTN_ERR_WORKSPACE
    assert dec(wsb=need - 1) == h.HATTN_ERR_WORKSPACE
    assert dec(ws=MIS) == h.HATTN_ERR_ALIGN
    assert dec(B=0) == h.HATTN_OK
    io[2].v = None
    assert dec() == h.HATTN_ERR_NULL                 # caught before any layer is enqueued
    io[2].v = 0x10008
    assert dec() == h.HATTN_ERR_ALIGN
    io[2].v = 0x10000
    io[3].lse = 0x10002
    assert dec() == h.HATTN_ERR_ALIGN
    io[3].lse = None
    pneed = lib.hattn_model_prefill_workspace_bytes(4, 2, 40)
    assert pneed == 2 * 40 * 4 * 256 * 2
    pre = lambda **o: lib.hattn_model_prefill(io, 4, 1024, o.get("pos", A), 2, o.get("S", 40),
                                              o.get("ws", A), o.get("wsb", pneed), None)
    assert pre(S=-1) == h.HATTN_ERR_SHAPE
    assert lib.hattn_model_prefill(io, 4, 1024, A, 65536, 40, A, pneed, None) == h.HATTN_ERR_SHAPE
    assert pre(S=0) == h.HATTN_OK
    assert pre(pos=None) == h.HATTN_ERR_NULL
    assert pre(wsb=pneed - 16) == h.HATTN_ERR_WORKSPACE
    assert pre(ws=MIS) == h.HATTN_ERR_ALIGN
    assert pre(pos=P(0x10002)) == h.HATTN_ERR_ALIGN


def test_fp8_validation(h):
    lib = h.lib()
    f, s = _cfg(h, "full"), _cfg(h, "sliding")
    app = lambda cfg=f, **o: lib.hattn_kv_append_fp8(
        cfg, o.get("k", A), o.get("v", A), o.get("kc", A), o.get("vc", A), o.get("ks", A),
        o.get("vs", A), o.get("cap", 64), o.get("pos", A), o.get("B", 1), o.get("n", 4),
        o.get("slots", None), o.get("flags", 0), None)
    for k in ("k", "v", "kc", "vc", "ks", "vs", "pos"):
        assert app(**{k: None}) == h.HATTN_ERR_NULL, k
    assert app(kc=MIS) == h.HATTN_ERR_ALIGN
    assert app(ks=P(0x10002)) == h.HATTN_ERR_ALIGN
    assert app(flags=2) == h.HATTN_ERR_UNSUPPORTED
    assert app(cfg=s, cap=64) == h.HATTN_ERR_RANGE
    assert app(n=-1) == h.HATTN_ERR_SHAPE
    assert app(n=0, k=None) == h.HATTN_OK
    need = lib.hattn_decode_workspace_bytes(f, 2, 4096)
    dec = lambda cfg=f, **o: lib.hattn_decode_fp8(
        cfg, o.get("q", A), o.get("kc", A), o.get("vc", A), o.get("ks", A), o.get("vs", A),
        o.get("cap", 4096), o.get("pos", A), o.get("B", 2), o.get("g", A), o.get("out", A),
        None, o.get("ws", A), o.get("wsb", need), o.get("flags", 0), None)
    for k in ("q", "kc", "vc", "ks", "vs", "pos", "g", "out"):
        assert dec(**{k: None}) == h.HATTN_ERR_NULL, k
    assert dec(ws=None) == h.HATTN_ERR_WORKSPACE
    assert dec(wsb=need - 1) == h.HATTN_ERR_WORKSPACE
    assert dec(vc=MIS) == h.HATTN_ERR_ALIGN
    assert dec(flags=4) == h.HATTN_ERR_UNSUPPORTED
    assert dec(cfg=s, cap=4096) == h.HATTN_ERR_RANGE
    assert dec(B=0) == h.HATTN_OK


def test_projection_validation(h):
    lib = h.lib()
    qkv = lambda **o: lib.hattn_qkv_proj(*[o.get(k, A) for k in ("x",)], o.get("T", 8),
                                         *[o.get(k, A) for k in ("w", "wg", "q", "k", "v", "g")], None)
    for k in ("x", "w", "wg", "q", "k", "v", "g"):
        assert qkv(**{k: None}) == h.HATTN_ERR_NULL, k
        assert qkv(**{k: MIS}) == h.HATTN_ERR_ALIGN, k
    assert qkv(T=-1) == h.HATTN_ERR_SHAPE
    assert qkv(T=0, x=None) == h.HATTN_OK
    assert qkv(T=65535 * 128 + 1) == h.HATTN_ERR_SHAPE
    op = lambda **o: lib.hattn_o_proj(o.get("a", A), o.get("T", 8), o.get("w", A), o.get("y", A), None)
    for k in ("a", "w", "y"):
        assert op(**{k: None}) == h.HATTN_ERR_NULL, k
        assert op(**{k: MIS}) == h.HATTN_ERR_ALIGN, k
    assert op(T=-1) == h.HATTN_ERR_SHAPE
    assert op(T=0, a=None) == h.HATTN_OK


# --------------------------------------------------------------- binding marshalling --
def test_binding_rejects_wrong_tensors_before_the_abi(h):
    """The Python binding checks dtype, shape and device of every tensor before its pointer
    crosses the C ABI (which cannot see sizes): a short output, an fp32 cache or a
    host-resident position array is a ValueError, never an out-of-bounds device access.
    Runs on host tensors, so every call below stops in the binding."""
    import torch
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    cfg = h.preset("full")
    B, S, cap = 2, 8, 64
    q = torch.zeros(B, S, 16, 256, dtype=bf)
    K = torch.zeros(B, cap, 4, 256, dtype=bf)
    g = torch.zeros(B, S, 16, dtype=bf)
    out = torch.zeros_like(q)
    lse = torch.zeros(B, S, 16, dtype=f32)
    pos = torch.zeros(B, dtype=i32)

    def raises(fn, *a, match, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*a, **kw)

    # well-formed arguments, but in host memory: the device check fires last
    raises(h.prefill, cfg, q, K, K, pos, g, out, lse, match="GPU memory")
    raises(h.prefill, cfg, q, K.float(), K, pos, g, out, lse, match="k_cache must be torch.bfloat16")
    raises(h.prefill, cfg, q, K, K, pos, g, out[:, :S - 1].contiguous(), lse, match="out must have shape")
    raises(h.prefill, cfg, q, K, K[:, :cap - 1].contiguous(), pos, g, out, lse, match="v_cache must have shape")
    raises(h.prefill, cfg, q, K, K, pos[:1], g, out, lse, match="pos0 holds 1 elements")
    raises(h.prefill, cfg, q, K, K, pos.long(), g, out, lse, match="pos0 must be torch.int32")
    raises(h.prefill, cfg, q, K, K, pos, g, out, lse[..., :15].contiguous(), match="lse must have shape")
    raises(h.decode, cfg, q, K, K, pos, g, out, lse, match="q must have shape")
    qd, gd = q[:, :1].contiguous(), g[:, :1].contiguous()
    raises(h.decode, cfg, qd, K, K, pos, gd, out[:, :1].contiguous(), lse[:, :1].contiguous(),
           torch.zeros(16, dtype=f32), match="workspace must be torch.uint8")
    raises(h.rope_qk, cfg, q, K[:, :S].contiguous(), pos, match="GPU memory")
    raises(h.rope_qk, cfg, q, torch.zeros(B, S, 16, 256, dtype=bf), pos, match="k must have shape")
    kn = torch.zeros(B, S, 4, 256, dtype=bf)
    raises(h.kv_append, cfg, kn, kn, K, K, pos, torch.zeros(B, S - 1, dtype=i32),
           match="slots_out must have shape")
    raises(h.kv_append_fp8, cfg, kn, kn, K, K, lse, lse, pos, match="k_cache must be torch.uint8")
    raises(h.prefill_ring, h.preset("sliding"), q, kn, kn, K, K, pos, g, out,
           match="k_ring must have shape")
    raises(h.o_proj, torch.zeros(3, 100, dtype=bf), torch.zeros(2560, 4096, dtype=bf),
           torch.zeros(3, 2560, dtype=bf), match="whole 16 x 256 head rows")
    raises(h.qkv_proj, torch.zeros(3, 2560, dtype=bf), torch.zeros(6144, 2560, dtype=bf),
           torch.zeros(16, 2560, dtype=bf), torch.zeros(3, 16, 256, dtype=bf),
           torch.zeros(2, 4, 256, dtype=bf), torch.zeros(3, 4, 256, dtype=bf),
           torch.zeros(3, 16, dtype=bf), match="k holds 2048 elements")
    layers = [dict(q=qd, k=kn[:, :1].contiguous(), v=kn[:, :1].contiguous(), gate=gd,
                   k_cache=K, v_cache=K, out=out[:, :1].contiguous(), lse=None)]
    raises(h.model_decode, layers, cap, pos, torch.zeros(16, dtype=torch.uint8),
           match="layer 0 k_cache must have shape")      # layer 0 is sliding: a 512-slot ring


def test_decode_noalloc_validation(h):
    """The allocation-free decode rejects what hattn_decode rejects, with the same codes,
    and a request beyond its static scratch with HATTN_ERR_SCRATCH, all before any launch
    (no GPU needed)."""
    lib = h.lib()
    f, s = _cfg(h, "full"), _cfg(h, "sliding")

    def call(cfg=f, q=A, k=A, v=A, cap=131136, pos=A, B=32, g=A, out=A, lse=None, flags=0):
        return lib.hattn_decode_noalloc(cfg, q, k, v, cap, pos, B, g, out, lse, flags, None)

    for kw in ("q", "k", "v", "pos", "g", "out"):
        assert call(**{kw: None}) == h.HATTN_ERR_NULL, kw
    assert call(q=MIS) == h.HATTN_ERR_ALIGN
    assert call(cfg=s, cap=131136) == h.HATTN_ERR_RANGE
    assert call(flags=2) == h.HATTN_ERR_UNSUPPORTED
    assert call(B=70000) == h.HATTN_ERR_SHAPE
    assert call(cap=0) == h.HATTN_ERR_SHAPE
    assert call(B=0) == h.HATTN_OK
    # beyond the scratch: 3000 sequences of one 1032-float partial per (KV head, q head)
    need = lib.hattn_decode_workspace_bytes(f, 3000, 1 << 20)
    assert need > h.DECODE_NOALLOC_MAX_BYTES
    assert call(B=3000, cap=1 << 20) == h.HATTN_ERR_SCRATCH
    assert "scratch" in lib.hattn_status_string(h.HATTN_ERR_SCRATCH).decode()
    # the largest measured shapes fit
    assert lib.hattn_decode_workspace_bytes(f, 32, 131136) <= h.DECODE_NOALLOC_MAX_BYTES
    assert lib.hattn_decode_workspace_bytes(f, 1, (1 << 20) + 64) <= h.DECODE_NOALLOC_MAX_BYTES
    # sliding layers: 4 ring splits of 4 x 258 floats per (sequence, KV head) and a counter,
    # 66112 bytes a sequence, so 507 sequences fit in 32 MiB and 508 do not
    per_seq = 4 * 4 * 4 * 258 * 4 + 4 * 4
    assert lib.hattn_decode_workspace_bytes(s, 507, 512) == 507 * per_seq <= h.DECODE_NOALLOC_MAX_BYTES
    assert lib.hattn_decode_workspace_bytes(s, 508, 512) > h.DECODE_NOALLOC_MAX_BYTES
    assert call(cfg=s, cap=512, B=508) == h.HATTN_ERR_SCRATCH
