"""Float64 CPU oracle for Multi-head Latent Attention decode.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the HIP path is checked against.  Only the test-suite, the
package smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does.  It imports nothing from the HIP side and shares no
code with it.

Source of truth: the itwiki article "멀티 헤드 잠재 어텐션" (Multi-head latent
attention), section "구조" (Structure):

* "키·값 공동 압축" (joint KV compression): c^KV_t = W^DKV h_t,
  k^C_t = W^UK c^KV_t, v^C_t = W^UV c^KV_t; queries c^Q_t = W^DQ h_t,
  q^C_t = W^UQ c^Q_t.
* "분리 RoPE" (decoupled RoPE): q^R_t = RoPE(W^QR c^Q_t) (one per head),
  k^R_t = RoPE(W^KR h_t) (shared by all heads); q = [q^C; q^R], k = [k^C; k^R];
  o_{t,i} = sum_{j<=t} softmax_j(q^T k / sqrt(d_h + d_h^R)) v^C_{j,i};
  u_t = W^O [o_{t,1}; ...; o_{t,n_h}].
* "행렬 흡수" (matrix absorption): q^T W^UK c = (W^UK^T q)^T c, so the content
  query is moved into latent space and dotted with the cached c^KV; every
  head then uses the same c^KV as key and value ("MQA mode"), and W^UV is
  applied after the weighted latent sum.

The lecture page "MHA · GQA · MQA · MLA" (section "Why Projection Absorption
Helps") states the same absorption identity and the 512 + 64 = 576 values per
token and layer that the cache holds.

Readings where the pages leave a step open (each one is also listed with the
design notes):

* RoPE is the half-split form: pairs (x_k, x_{k+d/2}) are rotated by the
  angle pos * base^(-2k/d), base 10000 (the article's implementation example
  uses this pairing).  Angles are computed in float64.
* Weights are stored [out, in]; W^UK and W^UV are viewed per head as
  [n_h, d_h, d_c] (head i = rows i*d_h .. (i+1)*d_h-1).
* Decode queries: the cache already holds the s_q new tokens; query i of a
  sequence of length L sits at position L - s_q + i and sees keys
  0 .. L - s_q + i (the "j <= t" of the attention equation).
* LSE is the natural log of the sum of exp(scaled score) over visible keys.

Storage decoders (bf16 bits, OCP fp8 e4m3fn codes, the paged fp8 block
layout) are written here from the formats' definitions.

Parity status: every function below is pinned by tests/test_oracle.py
(absorbed vs materialised agreement, closed forms, torch's CPU
scaled_dot_product_attention, complex-number rotation, the cache arithmetic
the pages print).  The fp8 *scheme* (per-token amax/448 scale on e4m3fn
content codes, bf16 RoPE key) is a reading: the pages name only an fp8
content cache beside a bf16 RoPE key, so with respect to the pages it is
parity unpinned -- it is pinned only by self-consistency (the oracle decodes
exactly the codes and scales the GPU reads) and by the e4m3fn format facts.
The low-bit caches (int4 / int2: grouped fp16 scale and minimum, packed
codes) are a reading as well -- the pages name only the bit widths -- and are
parity unpinned with respect to the pages; the decoder is pinned by
hand-written byte fixtures and by the quantisation error bound of a
separately written encoder.
GQLA's GQA path (gqa_decode_rows) is pinned by its algebraic equality with
the MQA-absorb path over the same weights (the page's claim) and by torch's
scaled_dot_product_attention with grouped key/value heads.
The layer's projections (project: c^KV, k^R, c^Q, q^C and the per-head
q^R) are pinned element by element on a tiny layer with explicit sums and
complex-number rotation at non-zero positions.
The cache producer (cache_append) is pinned by an element-by-element
brute force with complex-number rotation, by torch's own bf16 and fp8
casts for its encoders, and by appending a toy layer's tokens and decoding
them to the materialised MHA-mode result.
"""

from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# storage decoders
# --------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): the 16 bits are the top half
    of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn": no infinities) -> float64.

    Layout s.eeee.mmm, exponent bias 7.  e=0 encodes subnormals m/8 * 2^-6;
    e=15, m=7 is NaN; everything else is (1 + m/8) * 2^(e-7).  Max 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = s * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def paged_rows(cache, block_table_row, L, kv_dtype, d_c, d_r, block_size):
    """Logical rows 0..L-1 of one sequence, gathered through its block table.

    Returns (c [L, d_c], k_r [L, d_r]) in float64.  Token j lives in physical
    block table[j // block_size] at slot j % block_size."""
    c = np.empty((L, d_c))
    kr = np.empty((L, d_r))
    for j in range(0, L, block_size):
        n = min(block_size, L - j)
        pb = int(block_table_row[j // block_size])
        blk = cache[pb]
        if kv_dtype == "bf16":
            rows = bf16_to_f64(blk[:n])
            c[j:j + n], kr[j:j + n] = rows[:, :d_c], rows[:, d_c:d_c + d_r]
        elif kv_dtype == "f32":
            rows = np.asarray(blk[:n], dtype=np.float64)
            c[j:j + n], kr[j:j + n] = rows[:, :d_c], rows[:, d_c:d_c + d_r]
        elif kv_dtype == "fp8":
            raw = np.asarray(blk, dtype=np.uint8)
            o1 = block_size * d_c
            o2 = o1 + block_size * d_r * 2
            codes = raw[:o1].reshape(block_size, d_c)[:n]
            kbits = raw[o1:o2].view(np.uint16).reshape(block_size, d_r)[:n]
            scale = raw[o2:o2 + 4 * block_size].view(np.float32)[:n].astype(np.float64)
            c[j:j + n] = e4m3fn_to_f64(codes) * scale[:, None]
            kr[j:j + n] = bf16_to_f64(kbits)
        elif kv_dtype in ("int4", "int2"):
            cb = 4 if kv_dtype == "int4" else 2
            raw = np.asarray(blk, dtype=np.uint8)
            o1 = block_size * d_c * cb // 8
            o2 = o1 + block_size * d_r // 2
            ng = (d_c + d_r) // INT_GROUP
            cc = unpack_codes(raw[:o1].reshape(block_size, -1)[:n], cb)
            rc = unpack_codes(raw[o1:o2].reshape(block_size, -1)[:n], 4)
            prm = raw[o2:o2 + 4 * ng * block_size].view(np.float16).reshape(block_size, ng, 2)[:n]
            prm = prm.astype(np.float64)
            vals = np.concatenate([cc, rc], axis=1).reshape(n, ng, INT_GROUP)
            deq = (vals * prm[..., 0:1] + prm[..., 1:2]).reshape(n, d_c + d_r)
            c[j:j + n], kr[j:j + n] = deq[:, :d_c], deq[:, d_c:]
        else:
            raise ValueError(kv_dtype)
    return c, kr


# Low-bit caches (the QuantMLA review's INT4 content + INT4 RoPE and INT2
# content + INT4 RoPE; the grouping, the asymmetric (scale, min) form and the
# packing are readings): groups of INT_GROUP consecutive values of one token
# share an fp16 scale and an fp16 minimum, value = code * scale + min.
INT_GROUP = 32


def unpack_codes(raw, bits):
    """Little-endian 32-bit words of packed unsigned codes -> codes as float64.

    A word holds 32 / bits consecutive values; value 2k is the bit field at
    k * bits, value 2k + 1 the one at 16 + k * bits."""
    words = np.ascontiguousarray(raw).view("<u4").astype(np.int64)
    per = 32 // bits
    mask = (1 << bits) - 1
    out = np.empty(words.shape + (per,), dtype=np.float64)
    for k in range(per // 2):
        out[..., 2 * k] = (words >> (k * bits)) & mask
        out[..., 2 * k + 1] = (words >> (16 + k * bits)) & mask
    return out.reshape(*words.shape[:-1], -1)


# --------------------------------------------------------------------------
# RoPE (decoupled position part)
# --------------------------------------------------------------------------


def rope(x, pos, base: float = 10000.0):
    """Half-split rotary embedding.  x [..., T, d], pos [T].

    Pair k (k < d/2) is (x_k, x_{k+d/2}); it is rotated by the angle
    pos * base^(-2k/d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# --------------------------------------------------------------------------
# cache arithmetic ("캐시 크기 비교" table of the itwiki article)
# --------------------------------------------------------------------------


def cache_elements_per_token(method: str, n_h=128, d_h=128, n_g=1, d_c=512, d_r=64, layers=1):
    """KV-cache elements per token: MHA 2 n_h d_h l, GQA 2 n_g d_h l,
    MQA 2 d_h l, MLA (d_c + d_h^R) l."""
    if method == "MHA":
        return 2 * n_h * d_h * layers
    if method == "GQA":
        return 2 * n_g * d_h * layers
    if method == "MQA":
        return 2 * d_h * layers
    if method == "MLA":
        return (d_c + d_r) * layers
    raise ValueError(method)


# --------------------------------------------------------------------------
# softmax attention pieces
# --------------------------------------------------------------------------


def _softmax_rows(s):
    """Row softmax of s (masked entries = -inf) and the row log-sum-exp."""
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=-1, keepdims=True)
    return p / z, (m + np.log(z))[..., 0]


def attention_probs(q_lat, q_rope, c, kr, scale, visible):
    """Softmax weights of one query row set over its visible keys.

    q_lat [n, d_c], q_rope [n, d_r], c [L, d_c], kr [L, d_r]; keys 0..visible-1
    are visible.  Returns p [n, visible] and lse [n]."""
    s = (q_lat @ c[:visible].T + q_rope @ kr[:visible].T) * scale
    return _softmax_rows(s)


# --------------------------------------------------------------------------
# O1: MHA mode (materialise k^C and v^C per head)
# --------------------------------------------------------------------------


def project(h, W, pos):
    """The per-token projections of the layer (compression + decoupled RoPE).

    h [B, T, d].  Returns c_kv [B,T,d_c], k_r [B,T,d_r], q_c [B,T,n_h,d_h],
    q_r [B,T,n_h,d_r] (all float64)."""
    dm = W["dims"]
    n_h, d_h, d_r = dm["n_h"], dm["d_h"], dm["d_r"]
    h = np.asarray(h, dtype=np.float64)
    f = lambda name: np.asarray(W[name], dtype=np.float64)
    B, T, _ = h.shape
    c_kv = h @ f("w_dkv").T
    k_r = np.stack([rope(h[b] @ f("w_kr").T, pos) for b in range(B)])
    c_q = h @ f("w_dq").T
    q_c = (c_q @ f("w_uq").T).reshape(B, T, n_h, d_h)
    qr_flat = (c_q @ f("w_qr").T).reshape(B, T, n_h, d_r)
    q_r = np.empty_like(qr_flat)
    for b in range(B):
        for i in range(n_h):
            q_r[b, :, i] = rope(qr_flat[b, :, i], pos)
    return c_kv, k_r, q_c, q_r


def expand_kv(c_kv, w_uk, w_uv, n_h, d_h):
    """Materialise the per-head keys and values from the latent (MHA mode):
    k^C_{t,i} = W^UK_i c^KV_t, v^C_{t,i} = W^UV_i c^KV_t.  c_kv [..., T, d_c];
    weights [n_h*d_h, d_c] ([out, in]).  Returns k_c, v_c [..., T, n_h, d_h]."""
    c = np.asarray(c_kv, dtype=np.float64)
    k_c = (c @ np.asarray(w_uk, dtype=np.float64).T).reshape(*c.shape[:-1], n_h, d_h)
    v_c = (c @ np.asarray(w_uv, dtype=np.float64).T).reshape(*c.shape[:-1], n_h, d_h)
    return k_c, v_c


def mha_attention(q_c, q_r, k_c, k_r, v_c, scale):
    """Causal MHA-mode attention of one sequence (prefill): query t sees keys
    j <= t; head i scores q^C_{t,i}.k^C_{j,i} + q^R_{t,i}.k^R_j (k^R shared by
    all heads), softmax over j, weighted sum of v^C_{j,i}.

    q_c [T, n_h, d_h], q_r [T, n_h, d_r], k_c [T, n_h, d_h], k_r [T, d_r],
    v_c [T, n_h, d_v].  Returns o [T, n_h, d_v] and lse [T, n_h]."""
    q_c, q_r, k_c, k_r, v_c = (np.asarray(a, dtype=np.float64) for a in (q_c, q_r, k_c, k_r, v_c))
    T, n_h = q_c.shape[:2]
    causal = np.tril(np.ones((T, T), dtype=bool))  # key j visible to query t iff j <= t
    o = np.empty((T, n_h, v_c.shape[-1]))
    lse = np.empty((T, n_h))
    for i in range(n_h):
        s = (q_c[:, i] @ k_c[:, i].T + q_r[:, i] @ k_r.T) * scale
        s = np.where(causal, s, -np.inf)
        p, lse[:, i] = _softmax_rows(s)
        o[:, i] = p @ v_c[:, i]
    return o, lse


def mha_mode_layer(h, W, pos):
    """Full layer in MHA mode.

    Returns dict with u [B,T,d] (layer output), o [B,T,n_h,d_h] (per-head
    attention outputs before W^O), lse [B,T,n_h], and the projections."""
    dm = W["dims"]
    n_h, d_h, d_r = dm["n_h"], dm["d_h"], dm["d_r"]
    c_kv, k_r, q_c, q_r = project(h, W, pos)
    B, T = c_kv.shape[:2]
    k_c, v_c = expand_kv(c_kv, W["w_uk"], W["w_uv"], n_h, d_h)
    scale = 1.0 / math.sqrt(d_h + d_r)
    o = np.empty((B, T, n_h, d_h))
    lse = np.empty((B, T, n_h))
    for b in range(B):
        o[b], lse[b] = mha_attention(q_c[b], q_r[b], k_c[b], k_r[b], v_c[b], scale)
    u = o.reshape(B, T, n_h * d_h) @ np.asarray(W["w_o"], dtype=np.float64).T
    return {"u": u, "o": o, "lse": lse, "c_kv": c_kv, "k_r": k_r, "q_c": q_c, "q_r": q_r}


# --------------------------------------------------------------------------
# GQLA: the GQA decode path over a per-group expanded cache
# --------------------------------------------------------------------------
# The GQLA page (abstract) describes weights whose up-projections are shared
# by groups of heads, so the same parameters decode either in MQA-absorb form
# over the latent (as MLA) or in GQA form over a cache expanded per group.
# Reading: n_g groups of n_h / n_g consecutive heads; group g has W^UK_g,
# W^UV_g (rows g*d_h .. of [n_g*d_h, d_c]); the RoPE key stays shared; the
# GQA cache holds k^C_{j,g} = W^UK_g c_j, v^C_{j,g} = W^UV_g c_j and k^R_j.


def gqa_decode_rows(q_c, q_r, k_c, v_c, k_r, scale, n_g):
    """GQA-path decode of one sequence: q_c [s_q, n_h, d_h], q_r [s_q, n_h, d_r],
    k_c / v_c [L, n_g, d_h], k_r [L, d_r].  Head h reads group h // (n_h / n_g);
    query i sits at L - s_q + i and sees keys 0 .. L - s_q + i.
    Returns o [s_q, n_h, d_h] and lse [s_q, n_h]."""
    q_c, q_r, k_c, v_c, k_r = (np.asarray(a, dtype=np.float64) for a in (q_c, q_r, k_c, v_c, k_r))
    s_q, n_h = q_c.shape[:2]
    L = k_c.shape[0]
    hpg = n_h // n_g
    o = np.zeros((s_q, n_h, v_c.shape[-1]))
    lse = np.empty((s_q, n_h))
    for h in range(n_h):
        g = h // hpg
        s = (q_c[:, h] @ k_c[:, g].T + q_r[:, h] @ k_r.T) * scale        # [s_q, L]
        vis = np.arange(L)[None, :] <= (L - s_q + np.arange(s_q))[:, None]
        p, lse[:, h] = _softmax_rows(np.where(vis, s, -np.inf))
        o[:, h] = p @ v_c[:, g]
    return o, lse


def gqa_paged_rows(cache, block_table_row, L, n_g, d_h, d_r, block_size, kv_dtype="bf16"):
    """Logical rows of a paged GQA cache.  Per block of block_size tokens:
    [n_g][block_size][d_h] k^C | [n_g][block_size][d_h] v^C | [block_size][d_r]
    k^R (bf16 bits or fp32).  Returns k_c, v_c [L, n_g, d_h], k_r [L, d_r]."""
    k_c, v_c = np.empty((L, n_g, d_h)), np.empty((L, n_g, d_h))
    k_r = np.empty((L, d_r))
    dec = bf16_to_f64 if kv_dtype == "bf16" else (lambda a: np.asarray(a, dtype=np.float64))
    n1 = n_g * block_size * d_h
    for j in range(0, L, block_size):
        n = min(block_size, L - j)
        blk = dec(np.asarray(cache[int(block_table_row[j // block_size])]).reshape(-1))
        k_c[j:j + n] = blk[:n1].reshape(n_g, block_size, d_h)[:, :n].transpose(1, 0, 2)
        v_c[j:j + n] = blk[n1:2 * n1].reshape(n_g, block_size, d_h)[:, :n].transpose(1, 0, 2)
        k_r[j:j + n] = blk[2 * n1:2 * n1 + block_size * d_r].reshape(block_size, d_r)[:n]
    return k_c, v_c, k_r


def gqla_absorbed_rows(q_c, q_r, c, k_r, w_uk, w_uv, scale, n_g):
    """The MQA-absorb path of the same GQLA weights: head h absorbs its
    group's W^UK into the query, decodes over the latent c [L, d_c], and
    applies its group's W^UV.  Returns o [s_q, n_h, d_h], lse [s_q, n_h]."""
    q_c = np.asarray(q_c, dtype=np.float64)
    s_q, n_h, d_h = q_c.shape
    hpg = n_h // n_g
    w_uk = np.asarray(w_uk, dtype=np.float64).reshape(n_g, d_h, -1)
    w_uv = np.asarray(w_uv, dtype=np.float64).reshape(n_g, d_h, -1)
    grp = np.arange(n_h) // hpg
    q_lat = np.einsum("ihk,hkc->ihc", q_c, w_uk[grp])
    o_lat, lse = mqa_decode_rows(q_lat, q_r, c, k_r, scale)
    return np.einsum("hkc,ihc->ihk", w_uv[grp], o_lat), lse


# --------------------------------------------------------------------------
# absorption, MQA-mode decode, combine, up-projection
# --------------------------------------------------------------------------


def absorb_q(q_c, w_uk, n_h, d_h):
    """q_lat[t,i,:] = W^UK_i^T q^C[t,i,:]; w_uk [n_h*d_h, d_c] ([out, in])."""
    w = np.asarray(w_uk, dtype=np.float64).reshape(n_h, d_h, -1)
    q = np.asarray(q_c, dtype=np.float64)
    return np.einsum("thk,hkc->thc", q, w)


def up_proj_v(o_lat, w_uv, n_h, d_h):
    """o[t,i,:] = W^UV_i o_lat[t,i,:]; w_uv [n_h*d_h, d_c] ([out, in])."""
    w = np.asarray(w_uv, dtype=np.float64).reshape(n_h, d_h, -1)
    return np.einsum("thc,hkc->thk", np.asarray(o_lat, dtype=np.float64), w)


def mqa_decode_rows(q_lat, q_rope, c, kr, scale, key_range=None):
    """MQA-mode decode of one sequence on contiguous latent rows.

    q_lat [s_q, n_h, d_c], q_rope [s_q, n_h, d_r]; c [L, d_c], kr [L, d_r].
    Query i sees keys 0 .. L - s_q + i.  ``key_range`` = (lo, hi) restricts
    the keys to [lo, hi) on top of that (a split-KV partition); a row with no
    visible key gets o = 0 and lse = -inf.

    Returns o_lat [s_q, n_h, d_c] and lse [s_q, n_h]."""
    s_q, n_h, d_c = q_lat.shape
    L = c.shape[0]
    lo, hi = (0, L) if key_range is None else key_range
    o = np.zeros((s_q, n_h, d_c))
    lse = np.full((s_q, n_h), -np.inf)
    for i in range(s_q):
        vis_hi = min(hi, L - s_q + i + 1)
        if vis_hi <= lo:
            continue
        s = (q_lat[i] @ c[lo:vis_hi].T + q_rope[i] @ kr[lo:vis_hi].T) * scale
        p, lse[i] = _softmax_rows(s)
        o[i] = p @ c[lo:vis_hi]
    return o, lse


def combine_lse(o_parts, lse_parts):
    """Merge partial results of disjoint key sets.

    o_parts [S, ..., D] (each normalised over its own keys), lse_parts [S, ...].
    lse = log sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s.  Parts with
    lse = -inf carry no weight; if all are -inf the result is o = 0,
    lse = -inf."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe)
    z = w.sum(axis=0)
    lse = np.where(z > 0, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    o = np.einsum("s...,s...d->...d", w, o_parts) / np.where(z > 0, z, 1.0)[..., None]
    return o, lse


def decode_case_rows(case, b):
    """(q_lat [s_q,n_h,d_c], q_rope [s_q,n_h,d_r], c [L,d_c], kr [L,d_r]) in
    float64 for sequence b of an inputs.DecodeCase-like object."""
    L = int(case.seq_lens[b])
    c, kr = paged_rows(case.cache, case.block_table[b], L, case.kv_dtype,
                       case.d_c, case.d_r, case.block_size)
    dec = bf16_to_f64 if case.q_dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
    return dec(case.q_lat[b]), dec(case.q_rope[b]), c, kr


def mqa_decode_case(case, seqs=None):
    """O2 on a paged case: returns o_lat [B', s_q, n_h, d_c], lse [B', s_q, n_h]
    for the sequences in ``seqs`` (default all)."""
    seqs = range(case.B) if seqs is None else seqs
    outs, lses = [], []
    for b in seqs:
        ql, qr, c, kr = decode_case_rows(case, b)
        o, l = mqa_decode_rows(ql, qr, c, kr, case.softmax_scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def absorbed_layer(h, W, pos):
    """O3: the same layer computed in MQA mode (absorbed), from the same
    projections as mha_mode_layer.  Returns u, o, lse, o_lat."""
    dm = W["dims"]
    n_h, d_h, d_r = dm["n_h"], dm["d_h"], dm["d_r"]
    c_kv, k_r, q_c, q_r = project(h, W, pos)
    B, T = c_kv.shape[:2]
    scale = 1.0 / math.sqrt(d_h + d_r)
    o = np.empty((B, T, n_h, d_h))
    o_lat = np.empty((B, T, n_h, dm["d_c"]))
    lse = np.empty((B, T, n_h))
    for b in range(B):
        q_lat = absorb_q(q_c[b], W["w_uk"], n_h, d_h)           # [T, n_h, d_c]
        # every query row t is a decode step over the first t+1 cache rows
        ol, l = mqa_decode_rows(q_lat, q_r[b], c_kv[b], k_r[b], scale)  # s_q = T
        o_lat[b], lse[b] = ol, l
        o[b] = up_proj_v(ol, W["w_uv"], n_h, d_h)
    u = o.reshape(B, T, n_h * d_h) @ np.asarray(W["w_o"], dtype=np.float64).T
    return {"u": u, "o": o, "lse": lse, "o_lat": o_lat}


# --------------------------------------------------------------------------
# cache producer: compress, rotate, quantise, scatter into pages
# --------------------------------------------------------------------------


def bf16_round_bits(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, round to nearest, ties to even, done
    directly on the float64 value (8 significant bits): x = m * 2^e with
    m in [0.5, 1) keeps round(m * 256) / 256."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.rint(m * 256.0) / 256.0          # numpy rint: half to even
    v = np.ldexp(r, e).astype(np.float32)   # exact: 8 significant bits
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def e4m3fn_encode(x) -> np.ndarray:
    """Nearest OCP e4m3fn code of each value, by comparison against all 254
    finite codes; a tie goes to the code with the even mantissa; magnitudes
    beyond 448 saturate to +-448.  Zero encodes as +0."""
    x = np.asarray(x, dtype=np.float64)
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3fn_to_f64(codes)
    finite = ~np.isnan(vals)
    codes, vals = codes[finite], vals[finite]
    flat = np.clip(x.reshape(-1), -448.0, 448.0)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        d = np.abs(vals - v)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:  # a tie (or +-0): even mantissa, then the positive code
            even = [k for k in best if codes[k] & 1 == 0]
            best = even if even else best
            best = sorted(best, key=lambda k: codes[k] & 0x80)
        out[i] = codes[best[0]]
    return out.reshape(x.shape)


def quantize_token_e4m3(c_row):
    """Per-token fp8 content quantisation: scale = amax / 448 as float32 (1.0
    for an all-zero row), codes = e4m3fn(c / scale).  Returns (codes, scale)."""
    c_row = np.asarray(c_row, dtype=np.float64)
    amax = float(np.max(np.abs(c_row)))
    scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    return e4m3fn_encode(c_row / scale), scale


def cache_append(cache, h, w_dkv, w_kr, pos, slot_mapping, kv_dtype, d_c, d_r, block_size,
                 base: float = 10000.0):
    """The step before decode: for each new token t, c^KV_t = W^DKV h_t and
    k^R_t = RoPE(W^KR h_t, pos_t) (the article's "키·값 공동 압축" and "분리
    RoPE"), stored at physical slot slot_mapping[t] (block = slot // block_size,
    row = slot % block_size); a negative slot skips the token.

    cache: a copy is returned.  Storage: "f32" rows [d_c + d_r] float32,
    "bf16" rows of bf16 bit patterns (round to nearest even), "fp8" blocks
    [block_size x d_c e4m3fn codes | block_size x d_r bf16 | block_size fp32
    scales] with the content quantised per token (quantize_token_e4m3)."""
    h = np.asarray(h, dtype=np.float64)
    c_kv = h @ np.asarray(w_dkv, dtype=np.float64).T
    k_r = rope(h @ np.asarray(w_kr, dtype=np.float64).T, pos, base)
    out = np.array(cache, copy=True)
    for t in range(h.shape[0]):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk, row = slot // block_size, slot % block_size
        if kv_dtype == "f32":
            out[blk, row, :d_c] = c_kv[t]
            out[blk, row, d_c:d_c + d_r] = k_r[t]
        elif kv_dtype == "bf16":
            out[blk, row, :d_c] = bf16_round_bits(c_kv[t])
            out[blk, row, d_c:d_c + d_r] = bf16_round_bits(k_r[t])
        elif kv_dtype == "fp8":
            raw = out[blk]  # uint8 block
            codes, scale = quantize_token_e4m3(c_kv[t])
            raw[row * d_c:(row + 1) * d_c] = codes
            o1 = block_size * d_c
            kr_bits = bf16_round_bits(k_r[t]).view(np.uint8)
            raw[o1 + row * d_r * 2:o1 + (row + 1) * d_r * 2] = kr_bits
            o2 = o1 + block_size * d_r * 2
            raw[o2 + 4 * row:o2 + 4 * row + 4] = np.array([scale], dtype=np.float32).view(np.uint8)
        else:
            raise ValueError(kv_dtype)
    return out
