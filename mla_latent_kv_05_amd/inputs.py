"""Seeded synthetic inputs for absorbed-MLA decode.

This module only *creates* inputs: it draws seeded random numbers, rounds them
to the storage precisions the kernels read (fp32, bf16, OCP fp8 e4m3fn with a
per-token fp32 scale), and lays them out as a paged latent cache with a
shuffled block table.  It holds none of the attention arithmetic; both the
float64 oracle and the HIP path consume what it returns.

Workloads (shapes from DeepSeek-V2/V3 as tabulated on the itwiki "Multi-head
latent attention" page, section "DeepSeek-V2·V3 settings": n_h=128, d_h=128,
d_c=512, d_h^R=64; the toy layer uses the dimensions of that page's
"Implementation" example):

* ``toy_layer``      d=1024, n_h=8, d_h=64, d_c=128, d_cq=256, d_r=32, fp32,
                     T=256 tokens at positions 0..255.
* ``decode_case``    V3-shaped absorbed decode: q_lat ~ N(0, 1/512),
                     q_rope ~ N(0, 1), c^KV and k^R ~ N(0, 1), paged 64-token
                     blocks, bf16 or fp8 content cache.

Random streams: ``numpy.random.Generator(PCG64(seed))``; large tensors are
drawn in float32 (ziggurat) and rounded round-to-nearest-even to bf16.

Storage layouts (shared contract with the C ABI):

* bf16 / fp32 cache: ``[num_blocks, block_size, d_c + d_r]`` row-major, one row
  per token = ``[c^KV | k^R]``.
* fp8 cache: per block ``[block_size*d_c e4m3fn | block_size*d_r bf16 k^R |
  block_size fp32 scale]``, i.e. 644 bytes per token at d_c=512, d_r=64.
* int4 / int2 caches (4-bit or 2-bit content, 4-bit RoPE key): per block
  ``[block_size x content codes | block_size x RoPE codes | block_size x
  (d_c+d_r)/32 (scale, min) fp16 pairs]``; groups of 32 consecutive values of
  one token share a scale and a minimum, value = code * scale + min.  Codes
  are packed in little-endian 32-bit words of 8 (4-bit) or 16 (2-bit)
  consecutive values: value 2k sits at bit k*b, value 2k+1 at bit 16 + k*b.
  360 (int4) or 232 (int2) bytes per token at d_c=512, d_r=64.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 64

# --------------------------------------------------------------------------
# rounding to storage formats (input creation only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as uint16.  NaN stays NaN."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32)
    # finite values cannot wrap in uint32 (max 0xFF7FFFFF + 0x8000); NaNs are fixed below
    with np.errstate(over="ignore"):
        rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_as_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _e4m3fn_positive_table() -> np.ndarray:
    # all non-negative finite e4m3fn values, indexed by their 7-bit code 0..126
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3fn_positive_table()
E4M3_MAX = 448.0


def encode_e4m3fn(x) -> np.ndarray:
    """Encode values as OCP fp8 e4m3fn codes: round to nearest, ties to even
    code (even mantissa), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")  # first code with value >= mag
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    vhi, vlo = _E4M3_POS[hi], _E4M3_POS[lo]
    dhi, dlo = vhi - mag, mag - vlo
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(mag == vhi, hi, code).astype(np.uint8)
    sign = (np.signbit(x) & (code != 0)).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def encode_e4m3fn_fast(x32: np.ndarray) -> np.ndarray:
    """encode_e4m3fn for float32 inputs via torch's round-to-nearest-even cast
    (the two agree bit for bit on float32 values; see tests/test_inputs.py)."""
    import torch
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x32, dtype=np.float32), -E4M3_MAX, E4M3_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_rows_e4m3(c) -> tuple[np.ndarray, np.ndarray]:
    """Per-token fp8 quantisation of content rows ``c`` [..., d_c].

    scale_t = amax_t / 448 in fp32 (1.0 for an all-zero row),
    code = e4m3fn(c / scale_t) with the quotient formed in fp32."""
    c = np.asarray(c, dtype=np.float32)
    amax = np.abs(c).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    codes = encode_e4m3fn_fast(c / scale[..., None])
    return codes, scale


INT_GROUP = 32


def pack_codes(codes, bits: int) -> np.ndarray:
    """Pack unsigned codes [..., n] (n a multiple of 32 / bits * 2) into
    little-endian uint32 words: value 2k of a word at bit k*bits, value 2k+1
    at bit 16 + k*bits.  Returns the bytes [..., n * bits / 8]."""
    c = np.asarray(codes, dtype=np.uint32)
    per = 32 // bits
    w = c.reshape(*c.shape[:-1], -1, per)
    word = np.zeros(w.shape[:-1], dtype=np.uint32)
    for k in range(per // 2):
        word |= w[..., 2 * k] << np.uint32(k * bits)
        word |= w[..., 2 * k + 1] << np.uint32(16 + k * bits)
    return word.view(np.uint8).reshape(*c.shape[:-1], -1)


def quantize_groups(x, bits: int, group: int = INT_GROUP):
    """Asymmetric uniform quantisation of rows x [..., n] in groups of
    ``group`` consecutive values: min m and scale s = (max - min) / (2^bits - 1),
    both rounded to fp16; codes = clip(rint((x - m) / s), 0, 2^bits - 1)
    (0 where s = 0).  Returns (codes uint8 [..., n], params fp16 [..., n/group, 2])."""
    x = np.asarray(x, dtype=np.float64)
    g = x.reshape(*x.shape[:-1], -1, group)
    lo, hi = g.min(axis=-1), g.max(axis=-1)
    qmax = (1 << bits) - 1
    s16 = ((hi - lo) / qmax).astype(np.float16)
    m16 = lo.astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    m = m16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint((g - m) / np.where(s > 0, s, 1.0)), 0.0)
    codes = np.clip(q, 0, qmax).astype(np.uint8).reshape(x.shape)
    return codes, np.stack([s16, m16], axis=-1)


def int_row_bytes(d_c: int, d_r: int, content_bits: int) -> int:
    return d_c * content_bits // 8 + d_r // 2 + (d_c + d_r) // INT_GROUP * 4


def int_blocks(rows, d_c: int, content_bits: int) -> np.ndarray:
    """Rows [n, block_size, d_c + d_r] -> int cache blocks [n, block bytes]."""
    n, bs = rows.shape[:2]
    d_r = rows.shape[-1] - d_c
    cc, cp = quantize_groups(rows[..., :d_c], content_bits)
    rc, rp = quantize_groups(rows[..., d_c:], 4)
    parts = [pack_codes(cc, content_bits).reshape(n, -1), pack_codes(rc, 4).reshape(n, -1),
             np.concatenate([cp, rp], axis=-2).view(np.uint8).reshape(n, -1)]
    return np.concatenate(parts, axis=1)


# --------------------------------------------------------------------------
# toy layer (fp32): d=1024, n_h=8, d_h=64, d_c=128, d_cq=256, d_r=32
# --------------------------------------------------------------------------

TOY_DIMS = dict(d=1024, n_h=8, d_h=64, d_c=128, d_cq=256, d_r=32)


def toy_layer(seed: int = 1, B: int = 1, T: int = 256, dims: dict | None = None,
              dtype=np.float32) -> dict:
    """Weights i.i.d. N(0, 1/fan_in) stored [out, in]; hidden states N(0,1);
    positions 0..T-1.  Values are drawn in float64 and rounded to ``dtype``."""
    dm = dict(TOY_DIMS if dims is None else dims)
    d, n_h, d_h, d_c, d_cq, d_r = (dm[k] for k in ("d", "n_h", "d_h", "d_c", "d_cq", "d_r"))
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = {  # name: (out, in)
        "w_dq": (d_cq, d), "w_uq": (n_h * d_h, d_cq), "w_qr": (n_h * d_r, d_cq),
        "w_dkv": (d_c, d), "w_kr": (d_r, d), "w_uk": (n_h * d_h, d_c),
        "w_uv": (n_h * d_h, d_c), "w_o": (d, n_h * d_h),
    }
    out = {"dims": dm}
    for name, (o, i) in shapes.items():
        out[name] = (rng.standard_normal((o, i)) / math.sqrt(i)).astype(dtype)
    out["h"] = rng.standard_normal((B, T, d)).astype(dtype)
    out["pos"] = np.arange(T, dtype=np.int64)
    return out


# --------------------------------------------------------------------------
# absorbed decode workloads
# --------------------------------------------------------------------------


@dataclass
class DecodeCase:
    B: int
    s_q: int
    n_h: int
    d_c: int
    d_r: int
    d_h: int
    block_size: int
    kv_dtype: str               # "bf16" | "fp8" | "f32" | "int4" | "int2"
    q_dtype: str                # "bf16" | "f32"
    seq_lens: np.ndarray        # [B] int32
    block_table: np.ndarray     # [B, max_blocks] int32 (unused slots = -1 ... or poison)
    cache: np.ndarray           # storage array (uint16 for bf16, uint8 for fp8, float32)
    q_lat: np.ndarray           # [B, s_q, n_h, d_c] storage (uint16 bf16 bits or float32)
    q_rope: np.ndarray          # [B, s_q, n_h, d_r]
    softmax_scale: float
    num_blocks: int
    extra: dict = field(default_factory=dict)

    @property
    def row_bytes(self) -> int:
        if self.kv_dtype == "fp8":
            return self.d_c + 2 * self.d_r + 4
        if self.kv_dtype in ("int4", "int2"):
            return int_row_bytes(self.d_c, self.d_r, 4 if self.kv_dtype == "int4" else 2)
        return (self.d_c + self.d_r) * (2 if self.kv_dtype == "bf16" else 4)

    @property
    def block_bytes(self) -> int:
        return self.row_bytes * self.block_size

    @property
    def latent_bytes(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum()) * self.row_bytes


def _draw(rng, shape, std, kind):
    if kind == "f64":
        return rng.standard_normal(shape) * std
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def make_lengths(kind: str, B: int, rng, L: int | None = None,
                 lo: int = 128, hi: int = 32768) -> np.ndarray:
    if kind == "fixed":
        return np.full(B, L, dtype=np.int32)
    if kind == "loguniform":
        u = rng.uniform(math.log(lo), math.log(hi), size=B)
        return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int32)
    raise ValueError(kind)


def decode_case(seed: int, B: int, seq_lens, s_q: int = 1, n_h: int = 128,
                d_c: int = 512, d_r: int = 64, d_h: int = 128, kv_dtype: str = "bf16",
                q_dtype: str = "bf16", block_size: int = BLOCK, q_lat_std: float | None = None,
                extra_blocks: int = 0, tail_fill: str = "random",
                rope0_shift: list | None = None) -> DecodeCase:
    """Paged absorbed-decode inputs.

    ``seq_lens`` is an int, or an array of per-sequence lengths.  Physical
    block ids are one seeded permutation of 0..num_blocks-1 handed out in
    (sequence, logical block) order.  ``extra_blocks`` adds unreferenced
    physical blocks; ``tail_fill`` = "nan" poisons the unused tail rows of each
    sequence's last block (bf16 / f32 rows; fp8 codes, RoPE keys and scales;
    int4 / int2 group scales and minima) to show they are never read into
    the result.  ``rope0_shift`` (one array of length seq_lens[b] per
    sequence) is added to dimension 0 of each row's k^R before the row is
    encoded: with a query whose RoPE dimension 0 is non-zero it shapes the
    scores along the sequence (steps, ramps) without touching the stream of
    random draws."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.full(B, seq_lens, dtype=np.int32) if np.isscalar(seq_lens) else \
        np.asarray(seq_lens, dtype=np.int32)
    assert lens.shape == (B,) and (lens >= s_q).all()
    nblk = (lens + block_size - 1) // block_size
    max_blocks = int(nblk.max())
    num_blocks = int(nblk.sum()) + extra_blocks
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[k: k + nblk[b]]
        k += nblk[b]
    D = d_c + d_r
    kind = "f32" if (kv_dtype != "f32" and q_dtype != "f32") else "f64"
    # the cache is drawn block-chunk by block-chunk (one continuous random
    # stream) straight into its storage array
    if kv_dtype == "bf16":
        cache = np.empty((num_blocks, block_size, D), dtype=np.uint16)
    elif kv_dtype == "f32":
        cache = np.empty((num_blocks, block_size, D), dtype=np.float32)
    elif kv_dtype == "fp8":
        cache = np.empty((num_blocks, block_size * (d_c + 2 * d_r + 4)), dtype=np.uint8)
    elif kv_dtype in ("int4", "int2"):
        cbits = 4 if kv_dtype == "int4" else 2
        cache = np.empty((num_blocks, block_size * int_row_bytes(d_c, d_r, cbits)), dtype=np.uint8)
    else:
        raise ValueError(kv_dtype)
    shift = None
    if rope0_shift is not None:
        assert len(rope0_shift) == B
        shift = np.zeros((num_blocks, block_size))
        for b in range(B):
            sb = np.asarray(rope0_shift[b], dtype=np.float64)
            assert sb.shape == (lens[b],)
            for j in range(nblk[b]):
                part = sb[j * block_size: (j + 1) * block_size]
                shift[table[b, j], : part.size] = part
    chunk = 32
    for i0 in range(0, num_blocks, chunk):
        i1 = min(num_blocks, i0 + chunk)
        rows = _draw(rng, (i1 - i0, block_size, D), 1.0, kind)
        if shift is not None:
            rows[..., d_c] += shift[i0:i1].astype(rows.dtype)
        if kv_dtype == "bf16":
            cache[i0:i1] = f32_to_bf16_bits(rows)
        elif kv_dtype == "f32":
            cache[i0:i1] = rows
        elif kv_dtype in ("int4", "int2"):
            cache[i0:i1] = int_blocks(rows, d_c, cbits)
        else:
            n = i1 - i0
            codes, scale = quantize_rows_e4m3(rows[..., :d_c])
            kr = f32_to_bf16_bits(rows[..., d_c:])
            o1 = block_size * d_c
            o2 = o1 + block_size * d_r * 2
            cache[i0:i1, :o1] = codes.reshape(n, -1)
            cache[i0:i1, o1:o2] = kr.reshape(n, -1).view(np.uint8).reshape(n, -1)
            cache[i0:i1, o2:] = scale.reshape(n, -1).view(np.uint8).reshape(n, -1)
    if tail_fill == "nan":
        for b in range(B):
            used = lens[b] - (nblk[b] - 1) * block_size
            if used == block_size:
                continue
            pb = table[b, nblk[b] - 1]
            if kv_dtype in ("bf16", "f32"):
                cache[pb, used:] = 0x7FC0 if kv_dtype == "bf16" else np.nan
            elif kv_dtype == "fp8":  # NaN codes (0x7F), NaN bf16 k^R, NaN fp32 scales
                o1 = block_size * d_c
                o2 = o1 + block_size * d_r * 2
                blk = cache[pb]
                blk[used * d_c: o1] = 0x7F
                blk[o1 + used * d_r * 2: o2].view(np.uint16)[:] = 0x7FC0
                blk[o2 + used * 4: o2 + block_size * 4].view(np.float32)[:] = np.nan
            else:  # int4 / int2: NaN fp16 scale and minimum of every group of the tail rows
                cb = 4 if kv_dtype == "int4" else 2
                o2 = block_size * (d_c * cb // 8 + d_r // 2)
                prow = (d_c + d_r) // INT_GROUP * 4
                cache[pb, o2 + used * prow: o2 + block_size * prow].view(np.uint16)[:] = 0x7E00
    if q_lat_std is None:
        q_lat_std = 1.0 / math.sqrt(d_c)
    ql = _draw(rng, (B, s_q, n_h, d_c), q_lat_std, kind)
    qr = _draw(rng, (B, s_q, n_h, d_r), 1.0, kind)
    if q_dtype == "bf16":
        ql, qr = f32_to_bf16_bits(ql), f32_to_bf16_bits(qr)
    else:
        ql, qr = ql.astype(np.float32), qr.astype(np.float32)
    return DecodeCase(B=B, s_q=s_q, n_h=n_h, d_c=d_c, d_r=d_r, d_h=d_h,
                      block_size=block_size, kv_dtype=kv_dtype, q_dtype=q_dtype,
                      seq_lens=lens, block_table=table, cache=cache, q_lat=ql,
                      q_rope=qr, softmax_scale=1.0 / math.sqrt(d_h + d_r),
                      num_blocks=num_blocks)


@dataclass
class GqaCase:
    """Paged GQA-path decode inputs (GQLA's per-group expanded cache)."""
    B: int
    s_q: int
    n_h: int
    n_g: int
    d_h: int
    d_r: int
    block_size: int
    kv_dtype: str               # "bf16" | "f32"
    q_dtype: str
    seq_lens: np.ndarray        # [B] int32
    block_table: np.ndarray     # [B, max_blocks] int32 (-1 unused)
    cache: np.ndarray           # [num_blocks, block elements] (uint16 bf16 bits or float32)
    q_c: np.ndarray             # [B, s_q, n_h, d_h]
    q_r: np.ndarray             # [B, s_q, n_h, d_r]
    softmax_scale: float
    num_blocks: int

    @property
    def row_bytes(self) -> int:
        return (2 * self.n_g * self.d_h + self.d_r) * (2 if self.kv_dtype == "bf16" else 4)

    @property
    def cache_bytes_read(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum()) * self.row_bytes


def gqa_case(seed: int, B: int, seq_lens, s_q: int = 2, n_h: int = 128, n_g: int = 8, d_h: int = 128,
             d_r: int = 64, kv_dtype: str = "bf16", q_dtype: str = "bf16", block_size: int = BLOCK) -> GqaCase:
    """GQA-path inputs: per block of block_size tokens the cache holds
    [n_g][block_size][d_h] k^C | [n_g][block_size][d_h] v^C | [block_size][d_r] k^R.
    k^C, v^C ~ N(0,1) (the per-group expansion of a unit-variance latent with
    fan-in-scaled weights), k^R ~ N(0,1), q^C, q^R ~ N(0,1), so the scores
    scaled by 1/sqrt(d_h + d_r) have unit variance.  Physical blocks are one
    seeded permutation handed out in (sequence, logical block) order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.full(B, seq_lens, dtype=np.int32) if np.isscalar(seq_lens) else np.asarray(seq_lens, dtype=np.int32)
    assert lens.shape == (B,) and (lens >= s_q).all() and n_h % n_g == 0
    nblk = (lens + block_size - 1) // block_size
    num_blocks = int(nblk.sum())
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((B, int(nblk.max())), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[k:k + nblk[b]]
        k += nblk[b]
    E = block_size * (2 * n_g * d_h + d_r)
    kind = "f32" if (kv_dtype != "f32" and q_dtype != "f32") else "f64"
    cache = np.empty((num_blocks, E), dtype=np.uint16 if kv_dtype == "bf16" else np.float32)
    for i0 in range(0, num_blocks, 16):
        i1 = min(num_blocks, i0 + 16)
        vals = _draw(rng, (i1 - i0, E), 1.0, kind)
        cache[i0:i1] = f32_to_bf16_bits(vals) if kv_dtype == "bf16" else vals
    qc = _draw(rng, (B, s_q, n_h, d_h), 1.0, kind)
    qr = _draw(rng, (B, s_q, n_h, d_r), 1.0, kind)
    if q_dtype == "bf16":
        qc, qr = f32_to_bf16_bits(qc), f32_to_bf16_bits(qr)
    else:
        qc, qr = qc.astype(np.float32), qr.astype(np.float32)
    return GqaCase(B=B, s_q=s_q, n_h=n_h, n_g=n_g, d_h=d_h, d_r=d_r, block_size=block_size, kv_dtype=kv_dtype,
                   q_dtype=q_dtype, seq_lens=lens, block_table=table, cache=cache, q_c=qc, q_r=qr,
                   softmax_scale=1.0 / math.sqrt(d_h + d_r), num_blocks=num_blocks)


def projection_weights(seed: int, T_q: int, n_h: int = 128, d_h: int = 128,
                       d_c: int = 512, dtype: str = "bf16") -> dict:
    """Inputs for the query absorption and the W^UV up-projection at V3 shapes.

    q^C ~ N(0,1) [T_q, n_h, d_h]; W^UK ~ N(0, 1/(d_h*d_c)) so that the absorbed
    query has variance 1/d_c like the decode workloads; W^UV ~ N(0, 1/d_c)
    (fan-in d_c); o_lat ~ N(0, 1/64) stands in for a decode output.  Both
    weights are stored [n_h*d_h, d_c] ([out, in])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kind = "f32" if dtype == "bf16" else "f64"
    q_c = _draw(rng, (T_q, n_h, d_h), 1.0, kind)
    w_uk = _draw(rng, (n_h * d_h, d_c), 1.0 / math.sqrt(d_h * d_c), kind)
    w_uv = _draw(rng, (n_h * d_h, d_c), 1.0 / math.sqrt(d_c), kind)
    o_lat = _draw(rng, (T_q, n_h, d_c), 1.0 / 8.0, kind)
    conv = f32_to_bf16_bits if dtype == "bf16" else (lambda a: a.astype(np.float32))
    return {"q_c": conv(q_c), "w_uk": conv(w_uk), "w_uv": conv(w_uv), "o_lat": conv(o_lat),
            "dtype": dtype, "T_q": T_q, "n_h": n_h, "d_h": d_h, "d_c": d_c}


def append_inputs(seed: int, T: int, d: int = 7168, d_c: int = 512, d_r: int = 64, num_blocks: int = 80,
                  block_size: int = 64, dtype: str = "bf16", max_pos: int = 32768, skip_every: int = 0) -> dict:
    """Inputs for the cache producer: hidden states h ~ N(0,1) [T, d]; the
    stacked weight [W^DKV; W^KR] ~ N(0, 1/d) ([out, in], fan-in d); token
    positions uniform in [0, max_pos); each token a distinct physical slot
    (a seeded permutation of the cache's num_blocks*block_size slots), every
    ``skip_every``-th token marked -1 (padding).  ``dtype`` rounds h and W
    (bf16 bits or float32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kind = "f32" if dtype == "bf16" else "f64"
    h = _draw(rng, (T, d), 1.0, kind)
    w = _draw(rng, (d_c + d_r, d), 1.0 / math.sqrt(d), kind)
    pos = rng.integers(0, max_pos, size=T).astype(np.int32)
    slots = rng.permutation(num_blocks * block_size)[:T].astype(np.int32)
    if skip_every:
        slots[::skip_every] = -1
    conv = f32_to_bf16_bits if dtype == "bf16" else (lambda a: a.astype(np.float32))
    return {"h": conv(h), "w": conv(w), "pos": pos, "slots": slots, "T": T, "d": d, "d_c": d_c, "d_r": d_r,
            "num_blocks": num_blocks, "block_size": block_size, "dtype": dtype}


def prefill_inputs(seed: int, T: int, n_h: int = 128, d_h: int = 128, d_r: int = 64, d_c: int = 512,
                   dtype: str = "bf16") -> dict:
    """Inputs of MHA-mode prefill at V3 head shapes, one sequence of T tokens.

    Latent c^KV ~ N(0,1) [T, d_c] (it leaves an RMSNorm) with W^UK, W^UV ~
    N(0, 1/d_c) [n_h*d_h, d_c] ([out, in], fan-in d_c), so the expanded keys
    and values have unit variance; the attention inputs themselves are drawn
    independently: q = [q^C | q^R] ~ N(0,1) [T, n_h, d_h+d_r], k^C, v^C ~
    N(0,1) [T, n_h, d_h], k^R ~ N(0,1) [T, d_r] (RoPE keeps norms).  With
    scale 1/sqrt(d_h+d_r) the scores have unit variance."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kind = "f32" if dtype == "bf16" else "f64"
    out = {"c_kv": _draw(rng, (T, d_c), 1.0, kind),
           "w_uk": _draw(rng, (n_h * d_h, d_c), 1.0 / math.sqrt(d_c), kind),
           "w_uv": _draw(rng, (n_h * d_h, d_c), 1.0 / math.sqrt(d_c), kind),
           "q": _draw(rng, (T, n_h, d_h + d_r), 1.0, kind),
           "k_c": _draw(rng, (T, n_h, d_h), 1.0, kind),
           "v_c": _draw(rng, (T, n_h, d_h), 1.0, kind),
           "k_r": _draw(rng, (T, d_r), 1.0, kind)}
    conv = f32_to_bf16_bits if dtype == "bf16" else (lambda a: a.astype(np.float32))
    out = {k: conv(v) for k, v in out.items()}
    out.update(T=T, n_h=n_h, d_h=d_h, d_r=d_r, d_c=d_c, dtype=dtype, scale=1.0 / math.sqrt(d_h + d_r))
    return out


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

WORKLOADS = {
    "toy_fp32_T256": dict(kind="toy", seed=1),
    "v3_bf16_B64_ctx8192": dict(kind="decode", seed=2, B=64, lens=("fixed", 8192), s_q=1,
                                kv_dtype="bf16"),
    "v3_bf16_B128_ctxlogU128-32768": dict(kind="decode", seed=3, B=128,
                                          lens=("loguniform", None), s_q=1, kv_dtype="bf16"),
    "v3_bf16_B4_ctx131072": dict(kind="decode", seed=4, B=4, lens=("fixed", 131072), s_q=1,
                                 kv_dtype="bf16"),
    "v3_fp8_B64_ctx16384_sq2": dict(kind="decode", seed=5, B=64, lens=("fixed", 16384), s_q=2,
                                    kv_dtype="fp8"),
    "v3_bf16_B64_ctx8192_sq2": dict(kind="decode", seed=8, B=64, lens=("fixed", 8192), s_q=2, kv_dtype="bf16"),
    "v3_int4_B64_ctx8192": dict(kind="decode", seed=6, B=64, lens=("fixed", 8192), s_q=1, kv_dtype="int4"),
    "v3_int2_B64_ctx8192": dict(kind="decode", seed=7, B=64, lens=("fixed", 8192), s_q=1, kv_dtype="int2"),
}


def workload_lengths(name: str, B: int | None = None) -> np.ndarray:
    w = WORKLOADS[name]
    B = w["B"] if B is None else B
    rng = np.random.Generator(np.random.PCG64(w["seed"] + 1000))
    kind, L = w["lens"]
    return make_lengths(kind, B, rng, L)


def workload_case(name: str, B: int | None = None, L: int | None = None, **kw) -> DecodeCase:
    """A decode workload; ``B``/``L`` shrink it for quick tests."""
    w = WORKLOADS[name]
    B = w["B"] if B is None else B
    lens = workload_lengths(name, B)
    if L is not None:
        lens = np.minimum(lens, L).astype(np.int32) if w["lens"][0] != "fixed" else \
            np.full(B, L, dtype=np.int32)
    return decode_case(w["seed"], B, lens, s_q=w["s_q"], kv_dtype=w["kv_dtype"], **kw)
