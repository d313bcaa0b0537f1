"""CPU oracle for the Spark-X2.5/X2.6-4B hybrid attention layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it.  It shares no code, header, table or constant generator with the HIP
library; the two meet only in the seeded inputs of ``synth``.

Sources (web pages, cited by title and section):
  [T1] "How a million tokens fit into a 4B model: Spark X2.5's long-context architecture
       and its memory trade-offs" (hotelren.com)
  [T2] "No high-VRAM card needed: a 4B model takes on a million-token context" (163.com)
  [T3] "Spark-X2.6-4B-Base hybrid attention architecture" (lqnn.cn)
  [T4] "Reading Spark-X2.6-4B's config.json: a roadmap to hybrid attention and 1M
       context" (sheratonhq.com)

What it computes, per layer kind (sliding-window or full-causal), for one sequence:
  1. RoPE on Q and K at explicit positions with that kind's base and rotary span.
  2. GQA: query head h reads KV head h // 4 (explicitly, per head).
  3. An explicit boolean visibility mask (causal, plus the 512-token window on sliding).
  4. Scores q.k / 16, masked softmax, P.V.
  5. The per-head sigmoid output gate multiplied into each head's output.
Decode is the same computation with one query row; the ring append is slot = pos mod 512.

Precision: inputs are bf16 values upcast exactly to fp32.  RoPE angles follow the fp32
convention below and cos/sin are evaluated in fp64; the two contractions (Q.K^T and P.V)
run in fp32; softmax exponentials, row sums, the sigmoid and the LSE are fp64.

Every function is pinned by tests/test_oracle_pins.py against closed forms, the pages'
printed constants and figures, a library attention routine, and invariants.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

# --- Layer constants -----------------------------------------------------------------
# [T1] "GQA, fused projection and output gating": 16 query heads share 4 KV heads
# (num_key_value_groups = 4) and head_dim is 256.  [T4] "Model identity" table agrees.
N_Q_HEADS = 16
N_KV_HEADS = 4
HEAD_DIM = 256
# The pages give no softmax scale; head_dim ** -0.5 = 1/16 is taken.
SOFTMAX_SCALE = 1.0 / 16.0
# [T1] "Hybrid attention": sliding layers attend to the most recent 512 tokens.
# [T2] "27 sliding-window layers plus 9 global layers": a token 513 back is invisible,
# so the window holds the current token and the 511 before it.
WINDOW = 512
# [T1] "Per-layer RoPE": full layers use rope_theta 5e6 with partial_rotary_factor 0.25
# (the first 64 of 256 dims rotate, [T3] "Global attention + 5M-base RoPE"); sliding
# layers use rope_theta 1e4 with factor 1.0 (all 256 dims rotate).
N_LAYERS = 36


@dataclass(frozen=True)
class LayerKind:
    name: str
    rope_theta: float
    rot_dim: int          # number of leading dims that rotate
    window: int | None    # None = full causal


SLIDING = LayerKind("sliding", 1.0e4, HEAD_DIM, WINDOW)
FULL = LayerKind("full", 5.0e6, int(HEAD_DIM * 0.25), None)
KINDS = {"sliding": SLIDING, "full": FULL}


def kind_of(kind) -> LayerKind:
    return kind if isinstance(kind, LayerKind) else KINDS[kind]


def layer_schedule(n_layers: int = N_LAYERS) -> list[str]:
    """Layer l is full-causal iff l % 4 == 3: three sliding layers then one full layer,
    repeated, ending on a full layer ([T2] "27 sliding-window layers plus 9 global
    layers"; [T3] "36-layer hybrid layout"; [T1] "Hybrid attention" lists indices
    3, 7, 11, ..., 35)."""
    return ["full" if l % 4 == 3 else "sliding" for l in range(n_layers)]


# --- RoPE ([T1] "Per-layer RoPE"; [T3] "Global attention + 5M-base RoPE") ------------
def rope_inv_freq(theta: float, rot_dim: int) -> torch.Tensor:
    """omega_i = theta ** (-2 i / rot_dim) for i < rot_dim / 2, evaluated in fp64 and
    rounded once to fp32.  The frequencies are built over the rotary span, so a full
    layer's 64 rotating dims get 32 frequencies of base 5e6."""
    i = torch.arange(rot_dim // 2, dtype=torch.float64)
    return torch.pow(torch.tensor(theta, dtype=torch.float64), -2.0 * i / rot_dim).to(torch.float32)


def rope_angles(positions: torch.Tensor, theta: float, rot_dim: int) -> torch.Tensor:
    """Angle of pair i at position p: one fp32 multiply float32(p) * omega_i (exact
    position for p < 2**24).  Returns fp32 [n, rot_dim/2]."""
    pos = positions.to(torch.float32).reshape(-1, 1)
    return pos * rope_inv_freq(theta, rot_dim).reshape(1, -1)


def rope_rotate(x: torch.Tensor, positions: torch.Tensor, kind) -> torch.Tensor:
    """Rotate-half RoPE over the leading rot_dim dims of x [n, H, D] at positions [n].

    Pair (i, i + r/2), i < r/2, turns by angle a_i(p):
        y_i       = x_i * cos a - x_{i+r/2} * sin a
        y_{i+r/2} = x_{i+r/2} * cos a + x_i * sin a
    Dims r..D-1 are returned unchanged.  Computed in fp64 from fp64 cos/sin of the fp32
    angle; returned as fp32."""
    k = kind_of(kind)
    r, half = k.rot_dim, k.rot_dim // 2
    ang = rope_angles(positions, k.rope_theta, r).to(torch.float64)  # [n, half]
    c = torch.cos(ang)[:, None, :]
    s = torch.sin(ang)[:, None, :]
    xf = x.to(torch.float64)
    y = xf.clone()
    a, b = xf[..., :half], xf[..., half:r]
    y[..., :half] = a * c - b * s
    y[..., half:r] = b * c + a * s
    out = y.to(torch.float32)
    out[..., r:] = x[..., r:].to(torch.float32)  # pass-through dims: exact copy
    return out


# --- Visibility ([T1] "Hybrid attention"; [T2] "27 sliding-window layers ...") --------
def visible(q_pos: torch.Tensor, k_pos: torch.Tensor, kind) -> torch.Tensor:
    """Boolean mask [nq, nk]: key at position j is visible to the query at position i
    iff j <= i, and, on sliding layers, i - j <= WINDOW - 1."""
    k = kind_of(kind)
    d = q_pos.reshape(-1, 1).to(torch.int64) - k_pos.reshape(1, -1).to(torch.int64)
    m = d >= 0
    if k.window is not None:
        m &= d <= k.window - 1
    return m


def sigmoid64(g: torch.Tensor) -> torch.Tensor:
    """Headwise output gate sigmoid(g) = 1 / (1 + exp(-g)) in fp64 ([T1] "GQA, fused
    projection and output gating": gate = sigmoid(gate_score.float()); [T3] "GQA,
    head-level gating")."""
    return 1.0 / (1.0 + torch.exp(-g.to(torch.float64)))


# --- Attention core -------------------------------------------------------------------
def attend(q_rot, k_rot, v, gate, q_pos, k_pos, kind, *, row_block: int = 64,
           return_probs: bool = False):
    """Masked GQA attention with the headwise sigmoid gate, for one sequence.

    q_rot [nq, Hq, D], k_rot / v [nk, Hkv, D] (already rotated), gate [nq, Hq] logits,
    q_pos [nq], k_pos [nk] absolute positions.  Query head h uses KV head h // (Hq/Hkv).
    Returns y [nq, Hq, D] fp64, lse [nq, Hq] fp64 (natural log of the row's sum of
    exp(score)), and optionally the probabilities [Hq, nq, nk] fp64.
    Rows are processed in blocks so no nq x nk matrix larger than a block is built.
    """
    nq, hq, _ = q_rot.shape
    hkv = k_rot.shape[1]
    group = hq // hkv
    qf = q_rot.to(torch.float32)
    kf = k_rot.to(torch.float32)
    vf = v.to(torch.float32)
    sig = sigmoid64(gate)
    y = torch.empty(q_rot.shape, dtype=torch.float64)
    lse = torch.empty((nq, hq), dtype=torch.float64)
    probs = torch.empty((hq, nq, k_rot.shape[0]), dtype=torch.float64) if return_probs else None
    for r0 in range(0, nq, row_block):
        r1 = min(nq, r0 + row_block)
        mask = visible(q_pos[r0:r1], k_pos, kind)  # [nb, nk]
        if not bool(mask.any(dim=1).all()):
            raise ValueError("a query row has no visible key")
        for h in range(hq):
            kvh = h // group                      # replicated KV head for this query head
            s = (qf[r0:r1, h, :] @ kf[:, kvh, :].T).to(torch.float64) * SOFTMAX_SCALE
            s = s.masked_fill(~mask, float("-inf"))
            mx = s.max(dim=1, keepdim=True).values
            e = torch.exp(s - mx)
            den = e.sum(dim=1, keepdim=True)
            p = e / den
            o = (p.to(torch.float32) @ vf[:, kvh, :]).to(torch.float64)  # [nb, D]
            y[r0:r1, h, :] = o * sig[r0:r1, h:h + 1]
            lse[r0:r1, h] = (mx + torch.log(den)).squeeze(1)
            if return_probs:
                probs[h, r0:r1] = p
    if return_probs:
        return y, lse, probs
    return y, lse


# --- Layer entry points (the four steps the library exposes) -------------------------
def rope_qk(q, k, pos0: int, kind):
    """Rotate one sequence's q [S, Hq, D] and/or k [S, Hkv, D] (either may be None) at
    positions pos0 .. pos0 + S - 1.  Returns fp32 copies."""
    n = (q if q is not None else k).shape[0]
    pos = torch.arange(n, dtype=torch.int64) + pos0
    return (None if q is None else rope_rotate(q, pos, kind),
            None if k is None else rope_rotate(k, pos, kind))


def append_slots(pos0: int, n: int, kind, cap: int) -> torch.Tensor:
    """Cache slot of each of n appended tokens at positions pos0 ..: the position itself
    on full layers (the cache keeps every token); pos mod WINDOW on sliding layers, whose
    cache keeps only the last 512 tokens ([T2] "The real bottleneck of a million-token
    context": older keys and values are dropped).  -1 marks a token that has no slot."""
    k = kind_of(kind)
    pos = torch.arange(n, dtype=torch.int64) + pos0
    if k.window is None:
        slots = pos.clone()
        slots[(pos < 0) | (pos >= cap)] = -1
    else:
        slots = torch.remainder(pos, k.window)
        slots[pos < 0] = -1
    return slots.to(torch.int32)


def kv_append(k_cache, v_cache, k_new, v_new, pos0: int, kind):
    """Write n tokens into one sequence's cache [cap, Hkv, D] in position order; a later
    token overwrites an earlier one in the same slot.  Returns the int32 slots."""
    slots = append_slots(pos0, k_new.shape[0], kind, k_cache.shape[0])
    for t in range(k_new.shape[0]):
        s = int(slots[t])
        if s >= 0:
            k_cache[s] = k_new[t]
            v_cache[s] = v_new[t]
    return slots


def ring_positions(pos: int, window: int = WINDOW) -> torch.Tensor:
    """Position held by each ring slot after tokens 0..pos were appended in order:
    slot s holds the largest p' <= pos with p' mod window == s, or -1 if none."""
    s = torch.arange(window, dtype=torch.int64)
    held = pos - torch.remainder(pos - s, window)
    held[held < 0] = -1
    return held


def prefill(q, k_cache, v_cache, gate, pos0: int, kind, *, q_rotated: bool = False,
            rows=None, row_block: int = 64):
    """One sequence's prefill.  q [Sq, Hq, D] (unrotated unless q_rotated), gate [Sq, Hq];
    k_cache / v_cache [cap, Hkv, D] hold rotated keys/values indexed by absolute
    position.  Query i sits at pos0 + i and sees keys at positions in its visible set.
    rows: optional 1-D tensor of query indices to evaluate (a sample).
    Returns y [len(rows), Hq, D] fp64 and lse [len(rows), Hq] fp64."""
    sq = q.shape[0]
    idx = torch.arange(sq, dtype=torch.int64) if rows is None else torch.as_tensor(rows, dtype=torch.int64)
    q_pos = idx + pos0
    qs = q[idx]
    q_rot = qs.to(torch.float32) if q_rotated else rope_rotate(qs, q_pos, kind)
    k = kind_of(kind)
    hi = int(q_pos.max()) + 1
    lo = 0 if k.window is None else max(0, int(q_pos.min()) - (k.window - 1))
    k_pos = torch.arange(lo, hi, dtype=torch.int64)
    return attend(q_rot, k_cache[lo:hi], v_cache[lo:hi], gate[idx], q_pos, k_pos, kind,
                  row_block=row_block)


def prefill_ring(q, k_new, v_new, k_ring, v_ring, gate, pos0: int, *,
                 q_rotated: bool = False, rows=None, row_block: int = 64):
    """One sequence's sliding-layer prefill of a chunk that continues a ring cache.
    The chunk's n tokens sit at positions pos0 .. pos0 + n - 1: q [n, Hq, D] (unrotated
    unless q_rotated), gate [n, Hq], and their rotated keys / values k_new, v_new
    [n, Hkv, D].  k_ring / v_ring [WINDOW, Hkv, D] hold the keys / values of positions
    0 .. pos0 - 1 appended in order, so slot s holds ring_positions(pos0 - 1)[s].
    A query at p sees the positions p - 511 .. p: the older ones come from the ring, the
    rest from the chunk.  [T2] "The real bottleneck of a million-token context" (a
    sliding layer keeps only the last 512 tokens' keys and values); [T3] "Sliding window
    512".  Returns y [len(rows), Hq, D] fp64 and lse [len(rows), Hq] fp64."""
    n = q.shape[0]
    idx = torch.arange(n, dtype=torch.int64) if rows is None else torch.as_tensor(rows, dtype=torch.int64)
    q_pos = idx + pos0
    qs = q[idx]
    q_rot = qs.to(torch.float32) if q_rotated else rope_rotate(qs, q_pos, "sliding")
    held = ring_positions(pos0 - 1) if pos0 > 0 else torch.full((WINDOW,), -1, dtype=torch.int64)
    keep = held >= 0
    k_pos = torch.cat([held[keep], torch.arange(n, dtype=torch.int64) + pos0])
    kc = torch.cat([k_ring[keep].to(torch.float32), k_new.to(torch.float32)])
    vc = torch.cat([v_ring[keep].to(torch.float32), v_new.to(torch.float32)])
    return attend(q_rot, kc, vc, gate[idx], q_pos, k_pos, "sliding", row_block=row_block)


def decode(q, k_cache, v_cache, gate, pos: int, kind, *, q_rotated: bool = False):
    """One new token of one sequence at position pos (already appended).  q [Hq, D],
    gate [Hq].  Full layers: the cache holds positions 0..pos at slots 0..pos.  Sliding
    layers: the cache is the WINDOW-slot ring and each slot's position follows from
    ring_positions(pos).  Returns y [Hq, D] fp64, lse [Hq] fp64."""
    k = kind_of(kind)
    q_pos = torch.tensor([pos], dtype=torch.int64)
    q_rot = q[None].to(torch.float32) if q_rotated else rope_rotate(q[None], q_pos, kind)
    if k.window is None:
        k_pos = torch.arange(pos + 1, dtype=torch.int64)
        kc, vc = k_cache[:pos + 1], v_cache[:pos + 1]
    else:
        held = ring_positions(pos, k.window)
        keep = held >= 0
        k_pos, kc, vc = held[keep], k_cache[keep], v_cache[keep]
    y, lse = attend(q_rot, kc, vc, gate[None], q_pos, k_pos, kind)
    return y[0], lse[0]


# --- 8-bit KV cache ---------------------------------------------------------------------
# [T5] §3.2 "Deployment steps and key parameters": to fit a 1M context the deployment
# also quantizes the KV cache (8- or 4-bit), trading some precision for memory.  The
# format here is this library's own: OCP FP8 E4M3 ("e4m3fn": sign, 4 exponent bits with
# bias 7, 3 mantissa bits, subnormals, no infinities, codes 0x7F / 0xFF are NaN, largest
# finite 448) with one fp32 scale per (token, KV head): scale = amax / 448, code =
# e4m3(x / scale) rounded to nearest, ties to even.
E4M3_MAX = 448.0


def e4m3_decode(codes: torch.Tensor) -> torch.Tensor:
    """Value of each uint8 E4M3 code, fp32, from the format's definition."""
    c = codes.to(torch.int64)
    sign = torch.where((c & 0x80) != 0, -1.0, 1.0).to(torch.float64)
    e = (c >> 3) & 0xF
    m = (c & 0x7).to(torch.float64)
    normal = torch.ldexp(1.0 + m / 8.0, (e - 7).to(torch.int32))
    sub = m / 8.0 * 2.0 ** -6
    v = sign * torch.where(e == 0, sub, normal)
    v = torch.where((c & 0x7F) == 0x7F, torch.full_like(v, float("nan")), v)
    return v.to(torch.float32)


_E4M3_POS = None


def _e4m3_positive_table():
    """The 127 non-negative finite codes 0x00..0x7E and their values, ascending."""
    global _E4M3_POS
    if _E4M3_POS is None:
        codes = torch.arange(0, 0x7F, dtype=torch.int64)
        _E4M3_POS = (codes, e4m3_decode(codes).to(torch.float64))
    return _E4M3_POS


def e4m3_encode(x: torch.Tensor) -> torch.Tensor:
    """Nearest E4M3 code of each fp32 value, ties to the even code; |x| > 448 saturates
    to 448 (the quantizer never produces such values; see kv_quantize)."""
    codes, vals = _e4m3_positive_table()
    xf = x.to(torch.float64)
    a = xf.abs().clamp(max=E4M3_MAX).reshape(-1)
    hi = torch.searchsorted(vals, a).clamp(max=len(vals) - 1)   # first value >= a
    lo = (hi - 1).clamp(min=0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    idx = torch.where(pick_hi, hi, lo)
    out = codes[idx]
    neg = (xf.reshape(-1) < 0) | ((xf.reshape(-1) == 0) & torch.signbit(xf.reshape(-1)))
    out = torch.where(neg, out | 0x80, out)
    return out.to(torch.uint8).reshape(x.shape)


def kv_quantize(x: torch.Tensor):
    """Quantize keys or values x [n, Hkv, D] (bf16 or fp32 values) to E4M3 codes with one
    fp32 scale per (token, head): scale = fp32(amax / 448), code = e4m3(fp32(x / scale))
    (0 when the row is all zero).  Returns (codes uint8 [n, Hkv, D], scale fp32 [n, Hkv])."""
    xf = x.to(torch.float32)
    amax = xf.abs().amax(dim=-1)
    scale = amax / torch.tensor(E4M3_MAX, dtype=torch.float32)      # fp32, correctly rounded
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    y = (xf / safe[..., None]).clamp(-E4M3_MAX, E4M3_MAX)
    y = torch.where(scale[..., None] > 0, y, torch.zeros_like(y))
    return e4m3_encode(y), scale


def kv_dequantize(codes: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """codes [n, Hkv, D], scale [n, Hkv] -> fp32 values code_value * scale."""
    return e4m3_decode(codes) * scale[..., None].to(torch.float32)


def decode_kv8(q, k_codes, v_codes, k_scale, v_scale, gate, pos: int, kind, *,
               q_rotated: bool = False):
    """decode() over a cache held as E4M3 codes with per-(token, head) scales: the same
    attention on the dequantized keys and values.  Cache layouts as in decode();
    k_scale / v_scale [cap, Hkv]."""
    return decode(q, kv_dequantize(k_codes, k_scale), kv_dequantize(v_codes, v_scale), gate,
                  pos, kind, q_rotated=q_rotated)


def kv8_bytes_per_token_layer(n_kv_heads: int = N_KV_HEADS, head_dim: int = HEAD_DIM) -> int:
    """K and V codes (1 byte each) plus their two fp32 scales per head."""
    return 2 * n_kv_heads * head_dim + 2 * n_kv_heads * 4


# --- Projections around the layer -----------------------------------------------------
# [T1] "GQA, fused projection and output gating": one linear layer q_k_v_proj of output
# width q_dim + 2 kv_dim replaces three projections, and its output is sliced in that
# order into q, k and v; g_proj gives one gate score per head.  [T4] parameter table:
# hidden_size 2560, 16 x 256 query and 4 x 256 key/value dims; its quantization section
# names the attention output projection o_proj.  Weights use the linear-layer layout
# [out_features, in_features]; no bias (the pages show none).
HIDDEN = 2560
Q_DIM = N_Q_HEADS * HEAD_DIM      # 4096
KV_DIM = N_KV_HEADS * HEAD_DIM    # 1024


def qkv_proj(x, w_qkv, w_g):
    """x [T, 2560]; w_qkv [6144, 2560]; w_g [16, 2560].  Returns fp32 q [T,16,256],
    k [T,4,256], v [T,4,256] (slices of x @ w_qkv^T in that order) and gate logits
    [T,16] = x @ w_g^T.  fp32 products of the bf16 values."""
    xf = x.to(torch.float32)
    qkv = xf @ w_qkv.to(torch.float32).T
    t = x.shape[0]
    q = qkv[:, :Q_DIM].reshape(t, N_Q_HEADS, HEAD_DIM)
    k = qkv[:, Q_DIM:Q_DIM + KV_DIM].reshape(t, N_KV_HEADS, HEAD_DIM)
    v = qkv[:, Q_DIM + KV_DIM:].reshape(t, N_KV_HEADS, HEAD_DIM)
    gate = xf @ w_g.to(torch.float32).T
    return q, k, v, gate


def o_proj(attn, w_o):
    """attn [T, 16, 256] (the gated head outputs, heads concatenated) @ w_o^T with
    w_o [2560, 4096]: [T, 2560] fp32."""
    return attn.reshape(attn.shape[0], -1).to(torch.float32) @ w_o.to(torch.float32).T


# --- KV memory arithmetic ([T1] "Doing the arithmetic first", "Hybrid attention") ----
def kv_bytes_per_token_layer(n_kv_heads: int = N_KV_HEADS, head_dim: int = HEAD_DIM,
                             bytes_per_elem: int = 2) -> int:
    """K and V, each n_kv_heads x head_dim elements of bf16, per token per layer."""
    return 2 * n_kv_heads * head_dim * bytes_per_elem


def kv_cache_bytes(n_tokens: int, schedule=None) -> int:
    """Cache bytes for one sequence of n_tokens over a layer schedule: a full layer keeps
    every token, a sliding layer keeps at most WINDOW tokens."""
    sched = layer_schedule() if schedule is None else schedule
    per = kv_bytes_per_token_layer()
    return sum(per * (n_tokens if s == "full" else min(n_tokens, WINDOW)) for s in sched)


def attention_pairs_prefill(sq: int, pos0: int, kind) -> int:
    """Number of visible (query, key) pairs of one head in a prefill of sq queries at
    positions pos0..pos0+sq-1 (closed form; used to count algorithmic work)."""
    k = kind_of(kind)
    if k.window is None:
        # sum over p = pos0 .. pos0 + sq - 1 of (p + 1)
        return int(sq * pos0 + sq * (sq + 1) // 2)
    # rows at p < window see p + 1 keys, later rows see exactly window keys
    n_short = max(0, min(sq, k.window - pos0))
    short = n_short * pos0 + n_short * (n_short + 1) // 2
    return int(short + (sq - n_short) * k.window)


__all__ = [
    "N_Q_HEADS", "N_KV_HEADS", "HEAD_DIM", "SOFTMAX_SCALE", "WINDOW", "N_LAYERS",
    "LayerKind", "SLIDING", "FULL", "KINDS", "kind_of", "layer_schedule",
    "rope_inv_freq", "rope_angles", "rope_rotate", "visible", "sigmoid64", "attend",
    "rope_qk", "append_slots", "kv_append", "ring_positions", "prefill", "prefill_ring",
    "decode",
    "kv_bytes_per_token_layer", "kv_cache_bytes", "attention_pairs_prefill",
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "kv_quantize", "kv_dequantize", "decode_kv8",
    "kv8_bytes_per_token_layer", "HIDDEN", "Q_DIM", "KV_DIM", "qkv_proj", "o_proj",
]
