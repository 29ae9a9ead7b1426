"""Plain CPU oracle of the SageAttention forward pass (numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product library,
with which it shares no code.

Pages followed (cited by title and section below):

[SA]    "SageAttention: Accurate 8-Bit Attention for Plug-and-Play Inference
        Acceleration" -- paper detail page (arXiv 2410.02367).
[SA2pp] "SageAttention2++: A More Efficient Implementation of SageAttention2"
        -- paper review page (arXiv 2505.21136).

What is computed (the "SAGEAttn-B" kernel, [SA] §3 Algorithm 1, with the
FP8 "8+8" P~V variant of [SA2pp] "三、技术架构"):

1. Smooth K: gamma(K) = K - mean(K), the mean taken over all N tokens per
   channel ([SA] §4 Eq. 6).  Exact under softmax ([SA] §4, the shift-invariance
   argument after Eq. 6).
2. Per-block symmetric INT8 quantisation of Q/sqrt(d) and of gamma(K):
   delta = max|X|/127, X^ = round(X/delta) ([SA] §3 Algorithm 1;
   [SA2pp] "三", core formulas).
3. Tiled attention with an online softmax: S = Q^ K^T * delta_Q * delta_K
   (INT32 product), running max m, running sum l, rescaling of the output by
   exp(m_old - m_new) ([SA] §3 Algorithm 1; §4 Eq. 4-5).
4. P~V in FP16, or in FP8 E4M3 with a static delta_P = 1/448 and a
   per-channel delta_V = colmax|V|/448 ([SA2pp] "三", core formulas; the static
   P~ scale follows from max P~ = 1, [SA] §7 "key implementation details"),
   or in INT8 (the all-INT8 kernel variant of [SA] §3 Figure 5, chosen per
   layer in [SA] §6 step 4): static delta_P = 1/127 ([SA] §7), INT8 V with a
   per-channel delta_V = colmax|V|/127, and the INT8 product P^ V^ of each
   tile dequantised and added to the output as Eq. 4-5 write it
   (O = diag(exp(m_old - m_new)) O_prev + delta_P delta_V P^ V^).
5. O = diag(l)^-1 O ([SA] §3 Algorithm 1).

Optionally (smooth_q), Q is smoothed per block as SageAttention2 does ("SageAttention2"
abstract page: smoothing Q improves the accuracy of the quantised QK^T; the
SageAttention2++ review page, "三", smooths Q and K before quantising).  The
pages give no formula; the reading here (parity pinned by exact constructions
and integer brute force in tests/test_oracle_smooth_q.py):
* per 128-token block, qbar = the block's token mean of Q' = Q/sqrt(d)
  (float32, sequential in token order, one IEEE division by the block's token
  count), Q~ = fp32(Q' - qbar), quantised as any block (a = max|Q~|,
  r = fp32(127/a), codes, delta = fp32(a/127));
* the mean is kept per channel as an integer on a grid 2^8 times finer than
  the codes', w = rne(fp32(qbar r) 2^8), and its product with each key is
  rounded once to the codes' grid: the compensation
  C[t] = rne((w . K^[t]) / 2^8) (exact integer product, ties to even) is one
  integer per query block and key, and S = delta_Q delta_K (Q~^ K^^T + C);
* a block is smoothed only if a > 0 and 127 sum_c |w_c| <= 2^29 (so |C| stays
  at most 2^21, like |Q^ K^^T| <= 127^2 d); any other block is quantised as
  without smoothing (w = 0, C = 0).

Readings where the pages leave a step open (each listed in the design notes):

* Block sizes b_q, b_kv are not given: Q blocks of 128 tokens, K blocks of 64
  tokens, and the online softmax walks K/V in tiles of 64 keys, ascending.
* "Per block" means one scale per (batch, head, token block) over all d
  channels.
* Rounding is round-to-nearest-even; codes are clamped to [-127, 127]
  (the symmetric form delta = max|X|/127; -128 never occurs).
* Quantisation decisions are taken in float32, the precision of the scales:
  the mean is a float32 sum in a fixed order (256-token chunk partials summed
  sequentially, then the partials summed sequentially, then one IEEE
  division by N); K~ = fp32(K - mean); r = fp32(127 / a) with a = max|X|;
  code = rne(fp32(X * r)); delta = fp32(a / 127).  X * (127/a) equals X/delta
  in exact arithmetic; one reciprocal per block is the plain reading.
* Q is scaled by 1/sqrt(d) before quantisation, as Algorithm 1 writes
  psi_Q(Q/sqrt(d)): Q' = fp32(Q * fp32(1/sqrt(d))).
* An all-zero block gets delta = 0 and codes 0.
* Eq. 4-5 prints the rescale factor as exp(m' - m); the factor that makes the
  online softmax exact is exp(m_old - m_new), used here.
* l sums the unquantised P~.
* FP8 uses the static scale delta_P = 1/448, so P^ = E4M3(448 * P~);
  delta_V is per (batch, head, channel) over all N tokens.
* INT8 P~V: P^ = round(127 P~) (nearest even; P~ <= 1, so P^ in [0, 127]);
  V is quantised per (batch, head, channel) over all N tokens like the FP8
  mode's V (the pages give no granularity for this variant's V), with
  r = fp32(127/colmax), code = clamp(rne(fp32(V * r)), -127, 127) and
  delta_V = fp32(colmax/127).
* Causal masking: key j is visible to query i iff j <= i.
* The attention arithmetic after the INT32 product runs in float64 (the
  softmax "stays in full precision", [SA] §4, note under Eq. 4-5).

Parity pins for every function here live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3_decode, e4m3_encode, e4m3_flip_step, fp16_round, int8_flip_step

# ---------------------------------------------------------------------------
# Blocking contract (reading: the pages leave b_q, b_kv open).
Q_BLOCK = 128      # tokens per delta_Q block
K_BLOCK = 64       # tokens per delta_K block
KV_TILE = 64       # keys per online-softmax step
MEAN_CHUNK = 256   # tokens per float32 partial sum of the K column mean

INT8_RANGE = np.float32(127.0)   # symmetric INT8: delta = max|X| / 127
FP8_RANGE = np.float32(448.0)    # E4M3: delta = max|X| / 448
P_STATIC_FP8 = 1.0 / 448.0       # static delta_P, max P~ = 1
LOG2E = 1.4426950408889634       # log2(e), float64
P_STATIC_INT8 = 1.0 / 127.0


def inv_sqrt_d(d: int) -> np.float32:
    """float32(1/sqrt(d)): the softmax temperature folded into Q."""
    return np.float32(1.0 / np.sqrt(np.float64(d)))


# ---------------------------------------------------------------------------
# Smoothing: [SA] §4 Eq. 6, mean(K) = (1/N) sum_t K[t, :].
def column_mean(kf: np.ndarray) -> np.ndarray:
    """Per-(b, h, channel) token mean of K in float32, fixed summation order.

    kf: float32 [B, H, N, d] (exact values of the 16-bit K).
    Returns float32 [B, H, d].

    Order: for each 256-token chunk a partial sum starting at 0.0f, adding
    tokens in increasing order; then the partials in increasing chunk order
    starting at 0.0f; then one IEEE division by N.  The order does not change
    the attention output (any vector subtracted from every key is exact under
    softmax), it only fixes the bits of K^.
    """
    kf = np.asarray(kf, dtype=np.float32)
    B, H, N, d = kf.shape
    nch = -(-N // MEAN_CHUNK)
    pad = nch * MEAN_CHUNK - N
    # Zero padding at the end of the last chunk: adding +0.0 leaves a float32
    # partial sum unchanged, so the padded sums equal the unpadded ones.
    kp = np.concatenate([kf, np.zeros((B, H, pad, d), np.float32)], axis=2) if pad else kf
    kp = kp.reshape(B, H, nch, MEAN_CHUNK, d)
    part = np.zeros((B, H, nch, d), np.float32)
    for t in range(MEAN_CHUNK):
        part = part + kp[:, :, :, t, :]          # float32 + float32 -> float32
    tot = np.zeros((B, H, d), np.float32)
    for j in range(nch):
        tot = tot + part[:, :, j, :]
    return tot / np.float32(N)


# ---------------------------------------------------------------------------
# INT8 per-block quantiser psi: [SA] §3 Algorithm 1 (psi_Q, psi_K);
# [SA2pp] "三" core formulas delta = max|X|/127, X^ = round(X / delta).
def quantize_int8_blocks(x: np.ndarray, block: int):
    """Symmetric per-token-block INT8 quantisation.

    x: float32 [B, H, N, d].  One block = `block` consecutive tokens of one
    (b, h), across all d channels; the last block may be short.
    Returns (codes int8 [B, H, N, d], delta float32 [B, H, ceil(N/block)]).
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nb = -(-N // block)
    pad = nb * block - N
    xp = np.concatenate([x, np.zeros((B, H, pad, d), np.float32)], axis=2) if pad else x
    xb = xp.reshape(B, H, nb, block * d)
    a = np.abs(xb).max(axis=-1)                                   # exact
    with np.errstate(divide="ignore"):
        r = np.where(a > 0, INT8_RANGE / a, np.float32(0.0)).astype(np.float32)
    prod = (xb * r[..., None]).astype(np.float32)                 # one fp32 rounding
    codes = np.clip(np.rint(prod), -127, 127).astype(np.int8)     # RNE
    delta = (a / INT8_RANGE).astype(np.float32)
    codes = codes.reshape(B, H, nb * block, d)[:, :, :N, :]
    return np.ascontiguousarray(codes), delta


SQ_FRAC_BITS = 8     # smooth Q: w is kept on a grid 2^8 times finer than the codes
SQ_LIMIT = 2 ** 29   # smooth-Q guard: 127 * sum_c |w_c| must not exceed it


def q_block_mean(qs: np.ndarray) -> np.ndarray:
    """Per-(b, h, 128-token block, channel) mean of qs (float32 [B,H,N,d]):
    float32 sum starting at 0.0f in increasing token order over the block's
    tokens, then one IEEE division by their count (the last block may be
    short).  Returns float32 [B, H, ceil(N/128), d]."""
    qs = np.asarray(qs, dtype=np.float32)
    B, H, N, d = qs.shape
    nb = -(-N // Q_BLOCK)
    pad = nb * Q_BLOCK - N
    qp = np.concatenate([qs, np.zeros((B, H, pad, d), np.float32)], axis=2) if pad else qs
    qp = qp.reshape(B, H, nb, Q_BLOCK, d)
    acc = np.zeros((B, H, nb, d), np.float32)
    for t in range(Q_BLOCK):
        acc = acc + qp[:, :, :, t, :]            # padding adds +0.0: no change
    cnt = np.minimum(Q_BLOCK, N - Q_BLOCK * np.arange(nb)).astype(np.float32)
    return acc / cnt[None, None, :, None]


def smooth_quantize_q_blocks(qs: np.ndarray):
    """Smoothed per-block INT8 quantisation of Q' (reading in the module
    docstring).  Returns (codes int8 [B,H,N,d], delta float32 [B,H,nb],
    qbar float32 [B,H,nb,d] (0 for blocks left unsmoothed), w int32 [B,H,nb,d],
    smoothed bool [B,H,nb])."""
    qs = np.asarray(qs, dtype=np.float32)
    B, H, N, d = qs.shape
    nb = -(-N // Q_BLOCK)
    pad = nb * Q_BLOCK - N
    qbar = q_block_mean(qs)
    qp = np.concatenate([qs, np.zeros((B, H, pad, d), np.float32)], axis=2) if pad else qs
    qp = qp.reshape(B, H, nb, Q_BLOCK, d)
    valid = (Q_BLOCK * np.arange(nb)[:, None] + np.arange(Q_BLOCK)[None, :]) < N   # [nb, 128]
    qt = np.where(valid[None, None, :, :, None], (qp - qbar[:, :, :, None, :]).astype(np.float32),
                  np.float32(0.0))
    a = np.abs(qt).reshape(B, H, nb, -1).max(axis=-1)
    with np.errstate(divide="ignore"):
        r = np.where(a > 0, INT8_RANGE / a, np.float32(0.0)).astype(np.float32)
    w = np.rint((qbar * r[..., None]).astype(np.float32).astype(np.float64)
                * 2.0 ** SQ_FRAC_BITS).astype(np.int64)
    ok = (a > 0) & (127 * np.abs(w).sum(axis=-1) <= SQ_LIMIT)
    # smoothed blocks
    codes_s = np.clip(np.rint((qt * r[..., None, None]).astype(np.float32)), -127, 127)
    # blocks left unsmoothed: the plain quantiser of Q'
    plain, delta_p = quantize_int8_blocks(qs, Q_BLOCK)
    plain = np.concatenate([plain, np.zeros((B, H, pad, d), np.int8)], axis=2) if pad else plain
    plain = plain.reshape(B, H, nb, Q_BLOCK, d)
    codes = np.where(ok[..., None, None], codes_s, plain).astype(np.int8)
    codes = codes.reshape(B, H, nb * Q_BLOCK, d)[:, :, :N, :]
    delta = np.where(ok, (a / INT8_RANGE).astype(np.float32), delta_p).astype(np.float32)
    w = np.where(ok[..., None], w, 0).astype(np.int32)
    qbar = np.where(ok[..., None], qbar, np.float32(0.0)).astype(np.float32)
    return np.ascontiguousarray(codes), delta, qbar, w, ok


def q_compensation(q_w: np.ndarray, k_i8: np.ndarray) -> np.ndarray:
    """The compensation of smoothed Q blocks, C = rne((w K^^T) / 2^8): int32
    [B, H, nb, N].  The product is exact (a float64 product of integers below
    2^53); the division rounds to nearest, ties to even."""
    p = np.matmul(q_w.astype(np.float64),
                  np.swapaxes(k_i8.astype(np.float64), -1, -2)).astype(np.int64)
    q = p >> SQ_FRAC_BITS                                  # floor
    rem = p - (q << SQ_FRAC_BITS)                          # in [0, 2^8)
    half = 1 << (SQ_FRAC_BITS - 1)
    q = q + ((rem > half) | ((rem == half) & (q & 1 == 1))).astype(np.int64)
    return q.astype(np.int32)


def smooth_quant_qk(qf: np.ndarray, kf: np.ndarray, smooth: bool = True,
                    smooth_q: bool = False):
    """The prepass of [SA] §3 Algorithm 1: smooth K, quantise Q/sqrt(d) and K.

    Returns a dict with k_mean [B,H,d], q_i8, k_i8 [B,H,N,d],
    q_scale [B,H,ceil(N/128)], k_scale [B,H,ceil(N/64)] (float32).  With
    smooth_q, Q is smoothed per block (module docstring) and the dict also
    holds q_mean [B,H,nb,d] float32, q_w [B,H,nb,d] int32, q_smoothed [B,H,nb]
    and q_comp [B,H,nb,N] int32 (w K^^T).
    """
    qf = np.asarray(qf, dtype=np.float32)
    kf = np.asarray(kf, dtype=np.float32)
    d = qf.shape[-1]
    if smooth:
        mean = column_mean(kf)
        ks = (kf - mean[:, :, None, :]).astype(np.float32)
    else:
        mean = np.zeros(kf.shape[:2] + (d,), np.float32)
        ks = kf
    qs = (qf * inv_sqrt_d(d)).astype(np.float32)
    k_i8, k_scale = quantize_int8_blocks(ks, K_BLOCK)
    if not smooth_q:
        q_i8, q_scale = quantize_int8_blocks(qs, Q_BLOCK)
        return dict(k_mean=mean, q_i8=q_i8, k_i8=k_i8, q_scale=q_scale, k_scale=k_scale)
    q_i8, q_scale, q_mean, q_w, ok = smooth_quantize_q_blocks(qs)
    return dict(k_mean=mean, q_i8=q_i8, k_i8=k_i8, q_scale=q_scale, k_scale=k_scale,
                q_mean=q_mean, q_w=q_w, q_smoothed=ok, q_comp=q_compensation(q_w, k_i8))


# ---------------------------------------------------------------------------
# Rotary position embedding ahead of the quantisation.  [SA] §7 (key
# implementation details, item 1): Q and K are quantised right after the RoPE
# computation, in the same kernel, with 1/sqrt(d) folded into Q's
# quantisation.  The pages do not print RoPE itself; the reading here is the
# common "rotate half" form: channel i (< d/2) pairs with channel i + d/2,
# and with c = cos[t, i], s = sin[t, i] of token t
#     y_i       = x_i c - x_{i+d/2} s
#     y_{i+d/2} = x_{i+d/2} c + x_i s,
# each product and each sum rounded to float32 in that order.  The tables are
# inputs (float32 [N, d/2]); smoothing and quantisation then see y.
def rope_rotate_half(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x: float32 [B, H, N, d]; cos, sin: float32 [N, d/2]. Returns float32."""
    x = np.asarray(x, dtype=np.float32)
    h = x.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float32)[None, None]
    sn = np.asarray(sin, dtype=np.float32)[None, None]
    lo, hi = x[..., :h], x[..., h:]
    y = np.empty_like(x)
    y[..., :h] = (lo * c).astype(np.float32) - (hi * sn).astype(np.float32)
    y[..., h:] = (hi * c).astype(np.float32) + (lo * sn).astype(np.float32)
    return y


# ---------------------------------------------------------------------------
# V preparation: FP16 P~V keeps V in FP16 ([SA] §3 Algorithm 1, FP16 matmul);
# FP8 P~V quantises V per channel, delta_V = colmax|V|/448 ([SA2pp] "三");
# INT8 P~V ([SA] §3 Figure 5) quantises V per channel to INT8, delta_V =
# colmax|V|/127 (granularity: reading, as for FP8).
def prep_v(vf: np.ndarray, pv_mode: str):
    """Returns (v_values float64 [B,H,N,d], v_codes, v_scale float32 [B,H,d] or None).

    fp16: v_values = fp16_rne(V); v_codes = the float16 array.
    fp8:  cm = max_t |V[t, c]|; r = fp32(448/cm); codes = E4M3(fp32(V * r));
          v_values = decoded codes; v_scale = fp32(cm / 448).
    int8: cm as for fp8; r = fp32(127/cm); codes = clamp(rne(fp32(V * r)),
          -127, 127) as int8; v_values = the codes; v_scale = fp32(cm / 127).
    """
    vf = np.asarray(vf, dtype=np.float32)
    if pv_mode == "fp16":
        vh = vf.astype(np.float16)
        return vh.astype(np.float64), vh, None
    if pv_mode == "fp8":
        cm = np.abs(vf).max(axis=2)                                      # [B,H,d]
        with np.errstate(divide="ignore"):
            r = np.where(cm > 0, FP8_RANGE / cm, np.float32(0.0)).astype(np.float32)
        prod = (vf * r[:, :, None, :]).astype(np.float32)
        codes = e4m3_encode(prod)
        return e4m3_decode(codes), codes, (cm / FP8_RANGE).astype(np.float32)
    if pv_mode == "int8":
        cm = np.abs(vf).max(axis=2)                                      # [B,H,d]
        with np.errstate(divide="ignore"):
            r = np.where(cm > 0, INT8_RANGE / cm, np.float32(0.0)).astype(np.float32)
        prod = (vf * r[:, :, None, :]).astype(np.float32)
        codes = np.clip(np.rint(prod), -127, 127).astype(np.int8)
        return codes.astype(np.float64), codes, (cm / INT8_RANGE).astype(np.float32)
    raise ValueError(pv_mode)


# ---------------------------------------------------------------------------
def s_int32_tile(q_i8, k_i8, b, h, q0, nq, k0, nk) -> np.ndarray:
    """INT32 S = Q^ K^T on one tile: a float64 GEMM of int8 codes is exact
    (every partial sum is an integer of magnitude <= 127^2 * d < 2^53)."""
    qa = q_i8[b, h, q0:q0 + nq].astype(np.float64)
    ka = k_i8[b, h, k0:k0 + nk].astype(np.float64)
    return (qa @ ka.T).astype(np.int64).astype(np.int32)


def attention(q_op, q_rowscale, k_op, k_keyscale, v_op, v_chanscale, *, causal,
              p_round, rows=None, record=False, p_flip=False, p_codec="fp8", s_add=None):
    """Tiled attention with an online softmax for one (b, h).

    [SA] §3 Algorithm 1 and §4 Eq. 4-5, in float64:
      for each KV tile j (ascending, KV_TILE keys):
        S   = (Q_op K_op^T) * q_rowscale[:, None] * k_keyscale[None, :]
        mask: key > query (causal) -> -inf
        m'  = max(m, rowmax S);  alpha = exp(m - m')
        P~  = exp(S - m')
        l   = alpha * l + rowsum(P~)
        acc = alpha * acc + p_round(P~) @ V_op
        m   = m'
      O = acc / l * v_chanscale[None, :]

    For FP8 P~V, p_round(P~) = E4M3(448 P~)/448 (the static delta_P) and
    v_chanscale = delta_V, so O = sum P^ V^ delta_P delta_V / l.  INT8 P~V
    alike with p_round(P~) = round(127 P~)/127 and the INT8 V codes.

    q_op [R, d], q_rowscale [R], k_op [N, d], k_keyscale [N], v_op [N, d],
    v_chanscale [d]; rows = the query positions of the R rows (default 0..R-1).
    s_add: optional [R, N] addend of the product Q_op K_op^T before scaling
    (the smoothed-Q compensation C of each row's block).
    When `record`, also returns the per-tile P~ row maxima and the final m, l.

    p_flip (quantised P~, reading C-s): also return, per output element, a
    bound on how far O moves if every P~ / delta_P lying within the relative
    error of a float32 evaluation of exp(S - m) from a rounding boundary of
    the P^ codec (p_codec "fp8": E4M3 of 448 P~; "int8": integers of 127 P~)
    rounded to the other side.  The error model: about six float32 roundings
    of numbers of the size of |S| and |m| in log2 units (the scales, the max,
    the argument), with a margin of four, plus that of the exp itself,
        rel = 2^-23 * 4 (|S| + |m|) log2(e) + 2^-21.
    A float value of p_flip replaces the model by that constant relative
    distance.  Returns (O, bound) then.
    """
    q_op = np.asarray(q_op, dtype=np.float64)
    k_op = np.asarray(k_op, dtype=np.float64)
    v_op = np.asarray(v_op, dtype=np.float64)
    R, d = q_op.shape
    N = k_op.shape[0]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    qrs = np.asarray(q_rowscale, dtype=np.float64)[:, None]
    kks = np.asarray(k_keyscale, dtype=np.float64)
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, v_op.shape[1]))
    flip = np.zeros((R, v_op.shape[1]))
    vabs = np.abs(v_op)
    pmax_tiles = []
    for k0 in range(0, N, KV_TILE):
        k1 = min(k0 + KV_TILE, N)
        prod = q_op @ k_op[k0:k1].T
        if s_add is not None:
            prod = prod + np.asarray(s_add[:, k0:k1], dtype=np.float64)
        s = prod * qrs * kks[None, k0:k1]
        if causal:
            keys = np.arange(k0, k1)
            s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
        m_new = np.maximum(m, s.max(axis=1))
        # rows with no visible key yet keep m = -inf; their alpha is irrelevant
        # (l and acc are still 0) and is set to 0 to avoid inf - inf.
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
            p = np.exp(s - m_new[:, None])
        p = np.where(np.isfinite(m_new)[:, None], p, 0.0)
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p_round(p) @ v_op[k0:k1]
        if p_flip is not False:
            if p_flip is True:
                rel = (2.0 ** -23 * 4.0 * (np.abs(np.where(np.isfinite(s), s, 0.0))
                                           + np.abs(np.where(np.isfinite(m_new), m_new, 0.0))[:, None])
                       * LOG2E + 2.0 ** -21)
            else:
                rel = float(p_flip)
            if p_codec == "fp8":
                step = e4m3_flip_step(p * 448.0, rel) * P_STATIC_FP8
            elif p_codec == "int8":
                step = int8_flip_step(p * 127.0, rel) * P_STATIC_INT8
            else:
                raise ValueError(p_codec)
            flip = alpha[:, None] * flip + step @ vabs[k0:k1]
        m = m_new
        if record:
            pmax_tiles.append(p.max(axis=1))
    out = acc / l[:, None] * np.asarray(v_chanscale, dtype=np.float64)[None, :]
    if p_flip is not False:
        return out, flip / l[:, None] * np.abs(np.asarray(v_chanscale, dtype=np.float64))[None, :]
    if record:
        return out, dict(pmax_tiles=np.stack(pmax_tiles, axis=1), m=m, l=l)
    return out


def _p_round_for(pv_mode: str):
    if pv_mode == "fp16":
        return fp16_round
    if pv_mode == "fp8":
        # P^ = E4M3(P~ / delta_P) with the static delta_P = 1/448; the product
        # P^ V^ is dequantised by delta_P here and by delta_V per channel.
        return lambda p: e4m3_decode(e4m3_encode(p * 448.0)) * P_STATIC_FP8
    if pv_mode == "int8":
        # P^ = round(P~ / delta_P) with the static delta_P = 1/127
        return lambda p: np.clip(np.rint(p * 127.0), 0.0, 127.0) * P_STATIC_INT8
    if pv_mode == "none":
        return lambda p: p
    raise ValueError(pv_mode)


def sage_attention(qf, kf, vf, *, causal, pv_mode, quant="int8", smooth=True,
                   rows=None, heads=None, record=False, prep=None, p_flip=False,
                   smooth_q=False):
    """The whole forward pass on float32 inputs [B, H, N, d].

    quant="int8": the method.  quant="none": identity quantiser (Q/sqrt(d) and
    K - mean kept in float64, V unquantised unless pv_mode rounds P~), which
    must reduce to plain softmax attention.
    rows: optional query positions to evaluate (same for every head).
    heads: optional list of (b, h) to evaluate; default all.
    prep: optionally a precomputed smooth_quant_qk dict (quant="int8").
    smooth_q: smooth Q per block (module docstring); the compensation C of
    each row's block is added to the integer product.
    Returns O float64 [B, H, R, d] (R = N or len(rows)); heads not evaluated
    are left NaN.  With `record`, also a dict of per-head intermediates.
    p_flip (pv_mode "fp8" or "int8", quant "int8", not with `record`): also
    returns the per-element bound of `attention` on O's move from rounding
    boundary cases of P^.
    """
    qf = np.asarray(qf, dtype=np.float32)
    kf = np.asarray(kf, dtype=np.float32)
    vf = np.asarray(vf, dtype=np.float32)
    B, H, N, d = qf.shape
    rows_arr = np.arange(N) if rows is None else np.asarray(rows)
    out = np.full((B, H, len(rows_arr), d), np.nan)
    recs = {}
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    if p_flip and (pv_mode not in ("fp8", "int8") or quant != "int8" or record):
        raise ValueError("p_flip needs pv_mode 'fp8' or 'int8', quant='int8' and no record")
    flips = np.full(out.shape, np.nan) if p_flip else None

    if quant == "int8":
        pq = prep if prep is not None else smooth_quant_qk(qf, kf, smooth=smooth,
                                                            smooth_q=smooth_q)
        if pv_mode == "none":
            vvals, vscale = vf.astype(np.float64), None
        else:
            vvals, _, vscale = prep_v(vf, pv_mode)
        for (b, h) in heads:
            q_op = pq["q_i8"][b, h, rows_arr].astype(np.float64)
            s_add = pq["q_comp"][b, h, rows_arr // Q_BLOCK] if "q_comp" in pq else None
            qrs = pq["q_scale"][b, h, rows_arr // Q_BLOCK]
            k_op = pq["k_i8"][b, h].astype(np.float64)
            kks = pq["k_scale"][b, h, np.arange(N) // K_BLOCK]
            vcs = vscale[b, h].astype(np.float64) if vscale is not None else np.ones(d)
            res = attention(q_op, qrs, k_op, kks, vvals[b, h], vcs, causal=causal,
                            p_round=_p_round_for(pv_mode), rows=rows_arr, record=record,
                            p_flip=p_flip, p_codec=pv_mode if p_flip else "fp8",
                            s_add=s_add)
            if record:
                out[b, h], recs[(b, h)] = res
            elif p_flip:
                out[b, h], flips[b, h] = res
            else:
                out[b, h] = res
        if p_flip:
            return out, flips
        return (out, recs) if record else out

    if quant == "none":
        q64 = qf.astype(np.float64) / np.sqrt(np.float64(d))
        k64 = kf.astype(np.float64)
        if smooth:
            k64 = k64 - k64.mean(axis=2, keepdims=True)
        for (b, h) in heads:
            res = attention(q64[b, h, rows_arr], np.ones(len(rows_arr)), k64[b, h],
                            np.ones(N), vf[b, h].astype(np.float64), np.ones(d),
                            causal=causal, p_round=_p_round_for(pv_mode), rows=rows_arr,
                            record=record)
            if record:
                out[b, h], recs[(b, h)] = res
            else:
                out[b, h] = res
        return (out, recs) if record else out
    raise ValueError(quant)


# ---------------------------------------------------------------------------
def brute_attention(qf, kf, vf, *, causal) -> np.ndarray:
    """Textbook softmax(Q K^T / sqrt(d)) V in float64 ([SA] §4 symbol table:
    S = QK^T/sqrt(d), P = softmax(S), O = PV), the whole N x N matrix at once."""
    q = np.asarray(qf, dtype=np.float64)
    k = np.asarray(kf, dtype=np.float64)
    v = np.asarray(vf, dtype=np.float64)
    d = q.shape[-1]
    s = np.einsum("bhnd,bhmd->bhnm", q, k) / np.sqrt(np.float64(d))
    if causal:
        N = q.shape[2]
        s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("bhnm,bhmd->bhnd", p, v)


# ---------------------------------------------------------------------------
# Accuracy metrics named in [SA] §5 Table 2 (CosSim, Relative L1, RMSE); the
# page does not define them, so the usual definitions are used, in float64.
def cos_sim(x, y) -> float:
    x = np.asarray(x, np.float64).ravel()
    y = np.asarray(y, np.float64).ravel()
    return float(x @ y / (np.linalg.norm(x) * np.linalg.norm(y)))


def rel_l1(x, ref) -> float:
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(np.abs(x - ref).sum() / np.abs(ref).sum())


def rmse(x, ref) -> float:
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(np.sqrt(np.mean((x - ref) ** 2)))
