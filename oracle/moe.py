"""CPU oracle for the per-token Mixture-of-Experts decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run this module.  The product path (the HIP library and its Python
binding) never imports it, and this module shares no code, table or constant generator with it.

Everything here is the plain definition of what the decode step computes, written for a reader who
checks it against the pages by eye: scalar-clear numpy in float64, library primitives (``np.dot``,
``np.argsort``) used only as whole steps.  The one exception is the 4-bit quantizer: it is an
encoding whose integer decisions must match the device encoder bit for bit, so it takes those
decisions in IEEE fp32 (round-to-nearest-even), the precision the device uses.

Pages cited (by title):
  [G26]  "Gemma 4 26B : Comment faire tourner un LLM en 2 Go de RAM" (lhusser.fr)
  [LEAF] romain.leaflet.pub article on TurboFieldfare (untitled page; sections named below)
  [DAILY] "TurboFieldfare" event page, daily.steinslab.io (2026-07-30)
  [REMIO] "TurboFieldfare exécute Mac Gemma 4 26B dans 2 Go, mais la vitesse du SSD devient le compromis"
  [DEVT] "Een model met 26 miljard parameters uitvoeren in twee gigabyte geheugen op een gewone Mac"

What the pages fix: 128 routed experts of which the router keeps 8 per token and layer, plus one shared
expert used for every token ([DAILY] "L'atout caché des modèles MoE"; [REMIO] "Mac Gemma 4 26B tient en
mémoire..."); routed/shared/attention weights in MLX-style 4-bit affine format and an 8-bit router
([DAILY] "1. Compression par 4"; [REMIO] "L'affirmation des 2 Go..."); the shared branch and the routed
branch are combined ([G26] "Concurrence pour masquer la latence"); a 16-slot least-frequently-used expert
cache per layer ([DAILY] "Cache d'experts"; [DEVT] "Wat is de belangrijkste architectuurtruuc").
What they leave open is taken at its plainest reading; each reading is named where it is used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional, Sequence

import numpy as np

GROUP = 64              # quantization group along the input dimension (reading: MLX's default)
WORD_NIBBLES = 8        # 4-bit codes per uint32 word
SECTION_ALIGN = 256     # byte alignment of each section inside an expert record


# -------------------------------------------------------------------------------------------------
# bf16 helpers (the oracle's own; bf16 is the I/O type of the large configurations)
# -------------------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); result returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


def f64_round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    Done directly from float64 (not via float32) so that the single rounding of the definition is kept:
    the bf16 grid spacing at |x| in [2^e, 2^(e+1)) is 2^(e-7)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    m, e = np.frexp(x[nz])                 # x = m * 2^e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)                # 8 significant bits -> integer part
    out[nz] = np.ldexp(np.rint(scaled), e - 8)   # np.rint rounds half to even
    return out


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    r = f64_round_to_bf16(x).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# -------------------------------------------------------------------------------------------------
# 4-bit affine quantization (the encoding behind "MLX affine 4-bit")
# -------------------------------------------------------------------------------------------------

def quantize_affine_q4(w: np.ndarray, sb_bf16: bool):
    """Encode fp32 weights [N][K] as 4-bit codes with one (scale, bias) pair per group of 64 columns.

    Affine 4-bit weights ([REMIO] "L'affirmation des 2 Go fait de la bande passante SSD la nouvelle
    contrainte"; [DAILY] "1. Compression par 4").  The pages give no formula; reading: plain min-max per
    group, dequantized value = scale * code + bias.
      mn, mx = min and max of the group;  scale = (mx - mn) / 15 in fp32;
      scale, bias = scale and mn rounded to the scale/bias dtype (bf16 RNE, or fp32 as is);
      code = clamp(round_half_even((w - bias) / scale), 0, 15) in fp32 arithmetic; code = 0 if scale == 0.
    Returns codes uint8 [N][K], scale float32 [N][K/64], bias float32 [N][K/64] (values exactly
    representable in the scale/bias dtype).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, kdim = w.shape
    assert kdim % GROUP == 0
    g = w.reshape(n, kdim // GROUP, GROUP)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    scale = (mx - mn) / np.float32(15.0)                 # fp32 subtract, fp32 divide
    bias = mn.copy()
    if sb_bf16:
        scale = f32_round_to_bf16(scale)
        bias = f32_round_to_bf16(bias)
    codes = np.zeros(g.shape, dtype=np.uint8)
    live = scale != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - bias[:, :, None]) / scale[:, :, None]   # fp32 subtract, fp32 divide
    t = np.clip(np.rint(t), 0, 15)
    codes[live] = t[live].astype(np.uint8)
    return codes.reshape(n, kdim), scale.astype(np.float32), bias.astype(np.float32)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack codes [N][K] into uint32 words [N][K/8]: column c sits in word c // 8 at bits 4*(c % 8)
    (low nibble first; reading of the MLX packing order)."""
    n, kdim = codes.shape
    c = codes.astype(np.uint32).reshape(n, kdim // WORD_NIBBLES, WORD_NIBBLES)
    words = np.zeros((n, kdim // WORD_NIBBLES), dtype=np.uint32)
    for p in range(WORD_NIBBLES):
        words |= c[:, :, p] << np.uint32(4 * p)
    return words


def unpack_codes(words: np.ndarray) -> np.ndarray:
    n, nw = words.shape
    out = np.empty((n, nw, WORD_NIBBLES), dtype=np.uint8)
    for p in range(WORD_NIBBLES):
        out[:, :, p] = (words >> np.uint32(4 * p)) & np.uint32(0xF)
    return out.reshape(n, nw * WORD_NIBBLES)


def dequantize(codes: np.ndarray, scale: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """w_hat[r][c] = scale[r][c // 64] * code[r][c] + bias[r][c // 64], in float64."""
    n, kdim = codes.shape
    s = np.repeat(scale.astype(np.float64), GROUP, axis=1)
    b = np.repeat(bias.astype(np.float64), GROUP, axis=1)
    return s * codes.astype(np.float64) + b


# -------------------------------------------------------------------------------------------------
# expert record: one contiguous byte block per expert (the unit the cache copies)
# -------------------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class RecordLayout:
    d: int
    F: int
    sb_bf16: bool
    gate_up_q: int      # byte offsets
    gate_up_sb: int
    down_q: int
    down_sb: int
    total: int


def record_layout(d: int, F: int, sb_bf16: bool) -> RecordLayout:
    """Byte layout of one expert record (hidden size d, FFN width F).

    In order, each section starting on a 256-byte boundary:
      gate_up codes  uint32 [2F][d/8]      rows 0..F-1 are the gate matrix, rows F..2F-1 the up matrix
      gate_up s,b    sbtype [2F][d/64][2]  (scale, bias) pairs
      down codes     uint32 [d][F/8]
      down s,b       sbtype [d][F/64][2]
    sbtype is bf16 or fp32.  The record size is rounded up to 256 bytes."""
    assert d % GROUP == 0 and F % GROUP == 0
    sbw = 2 if sb_bf16 else 4

    def up(x: int) -> int:
        return (x + SECTION_ALIGN - 1) // SECTION_ALIGN * SECTION_ALIGN

    o_guq = 0
    o_gusb = up(o_guq + 2 * F * d // 2)
    o_dq = up(o_gusb + 2 * F * (d // GROUP) * 2 * sbw)
    o_dsb = up(o_dq + d * F // 2)
    total = up(o_dsb + d * (F // GROUP) * 2 * sbw)
    return RecordLayout(d, F, sb_bf16, o_guq, o_gusb, o_dq, o_dsb, total)


def _sb_bytes(scale: np.ndarray, bias: np.ndarray, sb_bf16: bool) -> bytes:
    pair = np.stack([scale.astype(np.float32), bias.astype(np.float32)], axis=-1)   # [N][G][2]
    if sb_bf16:
        return (pair.view(np.uint32) >> np.uint32(16)).astype("<u2").tobytes()
    return pair.astype("<f4").tobytes()


def _sb_parse(buf: np.ndarray, n: int, groups: int, sb_bf16: bool):
    if sb_bf16:
        raw = np.frombuffer(buf, dtype="<u2", count=n * groups * 2).reshape(n, groups, 2)
        vals = (raw.astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        vals = np.frombuffer(buf, dtype="<f4", count=n * groups * 2).reshape(n, groups, 2)
    return vals[:, :, 0].astype(np.float32), vals[:, :, 1].astype(np.float32)


def encode_record(w_gate_up: np.ndarray, w_down: np.ndarray, sb_bf16: bool) -> np.ndarray:
    """Quantize one expert's fp32 weights (gate_up [2F][d], down [d][F]) into its record bytes."""
    twoF, d = w_gate_up.shape
    F = twoF // 2
    assert w_down.shape == (d, F)
    lay = record_layout(d, F, sb_bf16)
    rec = np.zeros(lay.total, dtype=np.uint8)
    qg, sg, bg = quantize_affine_q4(w_gate_up, sb_bf16)
    qd, sd, bd = quantize_affine_q4(w_down, sb_bf16)
    for off, blob in ((lay.gate_up_q, pack_codes(qg).astype("<u4").tobytes()),
                      (lay.gate_up_sb, _sb_bytes(sg, bg, sb_bf16)),
                      (lay.down_q, pack_codes(qd).astype("<u4").tobytes()),
                      (lay.down_sb, _sb_bytes(sd, bd, sb_bf16))):
        rec[off:off + len(blob)] = np.frombuffer(blob, dtype=np.uint8)
    return rec


@dataclasses.dataclass
class DecodedExpert:
    gate_up_codes: np.ndarray   # uint8 [2F][d]
    gate_up_scale: np.ndarray   # f32 [2F][d/64]
    gate_up_bias: np.ndarray
    down_codes: np.ndarray      # uint8 [d][F]
    down_scale: np.ndarray
    down_bias: np.ndarray

    def gate_up(self) -> np.ndarray:
        return dequantize(self.gate_up_codes, self.gate_up_scale, self.gate_up_bias)

    def down(self) -> np.ndarray:
        return dequantize(self.down_codes, self.down_scale, self.down_bias)


def decode_record(rec: np.ndarray, d: int, F: int, sb_bf16: bool) -> DecodedExpert:
    lay = record_layout(d, F, sb_bf16)
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    assert rec.size >= lay.total
    guw = np.frombuffer(rec[lay.gate_up_q:], dtype="<u4", count=2 * F * d // 8).reshape(2 * F, d // 8)
    dw = np.frombuffer(rec[lay.down_q:], dtype="<u4", count=d * F // 8).reshape(d, F // 8)
    gs, gb = _sb_parse(rec[lay.gate_up_sb:], 2 * F, d // GROUP, sb_bf16)
    ds, db = _sb_parse(rec[lay.down_sb:], d, F // GROUP, sb_bf16)
    return DecodedExpert(unpack_codes(guw), gs, gb, unpack_codes(dw), ds, db)


# -------------------------------------------------------------------------------------------------
# router: 8-bit weights, top-k, gate weights
# -------------------------------------------------------------------------------------------------

def router_logits(w_int8: np.ndarray, row_scale: np.ndarray, u: np.ndarray) -> np.ndarray:
    """logit_e = s_e * sum_j W[e, j] * u_j with W int8 [E][d], s fp32 [E]; float64.

    The router keeps 8-bit weights ([G26] "Le pipeline de traitement"; [DAILY] "1. Compression par 4").
    Reading: symmetric int8 with one fp32 scale per expert row, no bias."""
    return row_scale.astype(np.float64) * np.dot(w_int8.astype(np.float64), np.asarray(u, dtype=np.float64))


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """The k experts with the largest logits, ordered by logit descending, equal logits by lower id.

    Top-8 of 128 per token and layer ([DAILY] "L'atout caché des modèles MoE"; [DEVT] "Wat is de
    belangrijkste architectuurtruuc").  Tie order is a reading (the pages do not say)."""
    e = np.arange(logits.size)
    order = np.lexsort((e, -np.asarray(logits, dtype=np.float64)))   # last key is primary
    return order[:k].astype(np.int32)


def gate_weights(logits: np.ndarray, ids: Sequence[int]) -> np.ndarray:
    """Softmax of the logits of the chosen experts (in the order given).

    Reading: the routing weights are the softmax over the k kept logits, which equals the softmax
    over all experts renormalised over the kept ones."""
    z = np.asarray(logits, dtype=np.float64)[np.asarray(ids)]
    e = np.exp(z - z.max())
    return e / e.sum()


# -------------------------------------------------------------------------------------------------
# expert FFN, combine, RMSNorm
# -------------------------------------------------------------------------------------------------

ACT_GELU_TANH = 0
ACT_SILU = 1


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GELU, tanh form (Hendrycks & Gimpel 2016): 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
    Reading: the pages name no activation; Gemma models use this gated GELU."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU / swish: z * sigmoid(z) (offered as the alternative gated activation)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def activation(z: np.ndarray, act: int) -> np.ndarray:
    return gelu_tanh(z) if act == ACT_GELU_TANH else silu(z)


def expert_ffn(ex: DecodedExpert, u: np.ndarray, act: int) -> np.ndarray:
    """y = W_down (act(W_gate u) * (W_up u)) on the dequantized weights, float64.

    The pages compute the selected experts (and the shared one) with quantized matrix-vector kernels
    ([LEAF] "Du code sur-mesure sans dépendance externe"; [DEVT] "Geen afhankelijkheden van llama.cpp en
    MLX"); the gated gate/up -> activation -> down structure is the reading for Gemma-style experts."""
    w_gu = ex.gate_up()
    F = w_gu.shape[0] // 2
    gu = np.dot(w_gu, np.asarray(u, dtype=np.float64))
    h = activation(gu[:F], act) * gu[F:]
    return np.dot(ex.down(), h)


def expert_hidden(ex: DecodedExpert, u: np.ndarray, act: int) -> np.ndarray:
    """h = act(W_gate u) * (W_up u), the FFN's inner activation (float64)."""
    w_gu = ex.gate_up()
    F = w_gu.shape[0] // 2
    gu = np.dot(w_gu, np.asarray(u, dtype=np.float64))
    return activation(gu[:F], act) * gu[F:]


def combine(y_routed: np.ndarray, weights: np.ndarray, y_shared: Optional[np.ndarray],
            residual: Optional[np.ndarray] = None) -> np.ndarray:
    """out = sum_i w_i y_i + y_shared (+ residual), float64 (rounded by the caller).

    The routed outputs and the shared-expert output are merged once the routed experts are in
    ([G26] "Concurrence pour masquer la latence"; [REMIO] "L'affirmation des 2 Go...").  Reading: the
    shared branch is added unweighted; the residual is added in the stacked configuration."""
    out = np.zeros(y_routed.shape[-1], dtype=np.float64)
    for i in range(len(weights)):
        out += float(weights[i]) * y_routed[i]
    if y_shared is not None:
        out += y_shared
    if residual is not None:
        out += np.asarray(residual, dtype=np.float64)
    return out


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """u = x / sqrt(mean(x^2) + eps) * gamma, float64 (the pages list a normalisation kernel; RMSNorm
    before each MoE block is the stacked configuration's reading, eps = 1e-6)."""
    x = np.asarray(x, dtype=np.float64)
    return x / math.sqrt(float(np.mean(x * x)) + eps) * np.asarray(gamma, dtype=np.float64)


# -------------------------------------------------------------------------------------------------
# one MoE layer, and a stack of them
# -------------------------------------------------------------------------------------------------

@dataclasses.dataclass
class OracleLayer:
    """Weights of one MoE layer as the oracle sees them.  ``expert(e)`` returns the record bytes of
    routed expert e (records may be produced lazily)."""
    d: int
    F: int
    S: int
    sb_bf16: bool
    router_w: np.ndarray            # int8 [E][d]
    router_s: np.ndarray            # f32 [E]
    expert: Callable[[int], np.ndarray]
    shared: Optional[np.ndarray]    # record bytes of the shared expert (width S), or None
    gamma: Optional[np.ndarray] = None

    def decoded(self, e: int) -> DecodedExpert:
        return decode_record(self.expert(e), self.d, self.F, self.sb_bf16)

    def decoded_shared(self) -> DecodedExpert:
        return decode_record(self.shared, self.d, self.S, self.sb_bf16)


@dataclasses.dataclass
class LayerResult:
    u: np.ndarray            # expert/router input (float64)
    logits: np.ndarray       # [E]
    ids: np.ndarray          # [k]
    weights: np.ndarray      # [k]
    y_routed: np.ndarray     # [k][d]
    y_shared: Optional[np.ndarray]
    out: np.ndarray          # float64, before output rounding


def moe_layer(layer: OracleLayer, u: np.ndarray, k: int, act: int = ACT_GELU_TANH,
              forced_ids: Optional[Sequence[int]] = None, residual: Optional[np.ndarray] = None) -> LayerResult:
    """One decode step of one MoE block for one token (router -> top-k -> experts -> combine).

    Per token and layer the router picks 8 experts with 8-bit weights, the shared expert runs for
    every token, and the two branches are combined ([G26] "Le pipeline de traitement" and "Concurrence
    pour masquer la latence"; [REMIO] "L'affirmation des 2 Go...").  ``forced_ids`` replaces the
    selection (a routing trace) while the gate weights stay the softmax of the router logits at those ids."""
    u = np.asarray(u, dtype=np.float64)
    logits = router_logits(layer.router_w, layer.router_s, u)
    ids = np.asarray(forced_ids, dtype=np.int32) if forced_ids is not None else select_topk(logits, k)
    w = gate_weights(logits, ids)
    y = np.stack([expert_ffn(layer.decoded(int(e)), u, act) for e in ids])
    ys = expert_ffn(layer.decoded_shared(), u, act) if layer.shared is not None else None
    out = combine(y, w, ys, residual)
    return LayerResult(u, logits, ids, w, y, ys, out)


def dense_moe_layer(layer: OracleLayer, u: np.ndarray, k: int, n_experts: int, act: int = ACT_GELU_TANH) -> np.ndarray:
    """Brute-force form of the same layer: every expert evaluated, multiplied by a dense gate vector
    that is zero outside the top-k.  Used to pin the sparse path."""
    u = np.asarray(u, dtype=np.float64)
    logits = router_logits(layer.router_w, layer.router_s, u)
    order = sorted(range(n_experts), key=lambda e: (-logits[e], e))[:k]
    z = np.array([logits[e] for e in order])
    p = np.exp(z - z.max())
    p /= p.sum()
    gate = np.zeros(n_experts)
    for e, pe in zip(order, p):
        gate[e] = pe
    out = np.zeros(layer.d)
    for e in range(n_experts):
        out += gate[e] * expert_ffn(layer.decoded(e), u, act)
    if layer.shared is not None:
        out += expert_ffn(layer.decoded_shared(), u, act)
    return out


def stack_layer_step(layer: OracleLayer, x_bf16_vals: np.ndarray, k: int, act: int = ACT_GELU_TANH,
                     eps: float = 1e-6, forced_ids: Optional[Sequence[int]] = None):
    """One layer of the stacked configuration: u = bf16(RMSNorm(x)); x_next = bf16(x + MoE(u)).

    Returns (u_bf16 values, LayerResult, x_next bf16 values).  bf16 rounding points: the norm output and
    the layer output (the activations travel as bf16)."""
    gamma = layer.gamma if layer.gamma is not None else np.ones(layer.d)
    u = f64_round_to_bf16(rms_norm(x_bf16_vals, gamma, eps))
    res = moe_layer(layer, u, k, act, forced_ids=forced_ids, residual=x_bf16_vals)
    return u, res, f64_round_to_bf16(res.out)


# -------------------------------------------------------------------------------------------------
# Grouping of a batch's (token, slot) pairs by expert (the batched decode)
# -------------------------------------------------------------------------------------------------

def group_pairs(ids: np.ndarray, n_valid: int):
    """The batch of T tokens routed to k experts each, as groups of pairs that share an expert
    ([G26] "Le pipeline de traitement": a prompt's tokens processed together share each expert's weights).

    Pair p = t*k + i carries the expert ids[t][i].  Reading (the pages give no algorithm): a stable sort of
    the pairs by expert, so pairs of one expert keep ascending pair order; ids outside [0, n_valid) all
    count as one bucket, after every valid expert.  Returns (groups, perm) with perm the sorted pair
    indices and groups the list of (bucket, first index into perm, count) of the non-empty buckets in
    ascending bucket order."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    bucket = np.where((flat >= 0) & (flat < n_valid), flat, n_valid)
    perm = np.argsort(bucket, kind="stable")
    groups = []
    for b in np.unique(bucket):
        members = np.nonzero(bucket[perm] == b)[0]
        groups.append((int(b), int(members[0]), int(len(members))))
    return groups, perm.astype(np.int64)


# -------------------------------------------------------------------------------------------------
# 16-slot LFU expert cache (policy simulation)
# -------------------------------------------------------------------------------------------------

@dataclasses.dataclass
class LfuStep:
    slots: list          # slot index of each requested id, in request order
    hits: int
    misses: int
    loaded: list         # (slot, expert) pairs loaded at this step, in order


class LfuCacheSim:
    """Per-layer least-frequently-used expert cache ([DAILY] "Cache d'experts"; [DEVT] "Wat is de
    belangrijkste architectuurtruuc"; [REMIO] "Mac Gemma 4 26B tient en mémoire...").

    Readings (the pages name only "LFU, 16 slots per layer"):
      * in-cache LFU: a slot's use count starts at 1 when an expert is loaded and is forgotten on eviction;
      * a step first marks every requested expert already resident (count += 1, last use = step), and
        these, with the experts loaded during the step, are pinned until the step ends;
      * each missing expert, in request order, goes to the lowest-numbered empty slot, else evicts the
        unpinned slot with the smallest (count, last use, slot index);
      * the cache starts empty.
    """

    def __init__(self, n_slots: int):
        self.n_slots = n_slots
        self.expert = [-1] * n_slots
        self.count = [0] * n_slots
        self.last = [-1] * n_slots
        self.t = 0

    def step(self, ids: Sequence[int]) -> LfuStep:
        ids = [int(e) for e in ids]
        assert len(set(ids)) == len(ids) and len(ids) <= self.n_slots
        pinned = [False] * self.n_slots
        where = {}
        hits = 0
        for e in ids:
            if e in self.expert:
                s = self.expert.index(e)
                self.count[s] += 1
                self.last[s] = self.t
                pinned[s] = True
                where[e] = s
                hits += 1
        loaded = []
        for e in ids:
            if e in where:
                continue
            empty = [s for s in range(self.n_slots) if self.expert[s] < 0]
            if empty:
                s = empty[0]
            else:
                cand = [s for s in range(self.n_slots) if not pinned[s]]
                s = min(cand, key=lambda j: (self.count[j], self.last[j], j))
            self.expert[s] = e
            self.count[s] = 1
            self.last[s] = self.t
            pinned[s] = True
            where[e] = s
            loaded.append((s, e))
        self.t += 1
        return LfuStep([where[e] for e in ids], hits, len(loaded), loaded)


def lfu_simulate(trace: np.ndarray, n_slots: int):
    """Run one cache per layer over a trace int [T][L][k]; returns slots int32 [T][L][k] and hit counts
    int64 [T][L]."""
    T, L, k = trace.shape
    caches = [LfuCacheSim(n_slots) for _ in range(L)]
    slots = np.zeros((T, L, k), dtype=np.int32)
    hits = np.zeros((T, L), dtype=np.int64)
    for t in range(T):
        for l in range(L):
            st = caches[l].step(trace[t, l])
            slots[t, l] = st.slots
            hits[t, l] = st.hits
    return slots, hits
