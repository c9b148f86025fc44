"""Pins for the float64 oracle (CPU only).

Each test ties the oracle to something other than itself: figures the pages
print, closed forms, a textbook library routine (torch's CPU
scaled_dot_product_attention, numpy complex rotation), brute force in 50-digit
arithmetic, and invariants the method guarantees."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_05_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_arithmetic.json")


def _small_decode(seed=0, s_q=2, n_h=4, d_c=16, d_r=8, L=37):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((s_q, n_h, d_c)), rng.standard_normal((s_q, n_h, d_r)),
            rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r)))


# ---------------------------------------------------------------- pages' figures

def test_cache_arithmetic_golden():
    g = json.load(open(GOLDEN))
    for it in g["items"]:
        assert oracle.cache_elements_per_token(it["method"], **it["args"]) == it["elements"], it
    for r in g["ratios"]:
        v = r["num"] / r["den"]
        if "exact" in r:
            assert v == r["exact"]
        else:
            assert abs(v - r["approx"]) <= r["tol"]
    lec = g["bytes_bf16"][0]
    per = lec["per_layer_bytes"]
    assert 2 * oracle.cache_elements_per_token("MHA", n_h=32, d_h=128) == per["MHA"]
    assert 2 * oracle.cache_elements_per_token("GQA", n_g=8, d_h=128) == per["GQA-8"]
    assert 2 * oracle.cache_elements_per_token("MQA", d_h=128) == per["MQA"]
    assert 2 * oracle.cache_elements_per_token("MLA") == per["MLA"]
    assert abs(per["MLA"] / 1024 - lec["mla_approx_kib"]) < 0.05
    chart = g["bytes_bf16"][1]
    for m, kib in chart["kib_per_token"].items():
        el = {"MHA": oracle.cache_elements_per_token("MHA", n_h=32, d_h=128),
              "GQA-8": oracle.cache_elements_per_token("GQA", n_g=8, d_h=128),
              "MLA": oracle.cache_elements_per_token("MLA"),
              "MQA": oracle.cache_elements_per_token("MQA", d_h=128)}[m]
        assert el * 2 * chart["layers"] / 1024 == kib
    for it in g["bytes_bf16"][2:]:
        assert abs(it["elements"] * 2 / 1024 - it["approx_kb"]) <= it["tol_kb"] + 0.5
    s = g["scale"]
    assert abs(1.0 / math.sqrt(s["d_h"] + s["d_r"]) - s["value"]) < 1e-16


def test_storage_row_bytes_match_pages():
    # one bf16 latent row is 576 values = 1152 bytes ("about 1.1 KiB")
    c = inputs.decode_case(0, B=1, seq_lens=64, n_h=4)
    assert c.row_bytes == 1152 and c.d_c + c.d_r == 576
    f = inputs.decode_case(0, B=1, seq_lens=64, n_h=4, kv_dtype="fp8")
    assert f.row_bytes == 512 + 128 + 4


# ---------------------------------------------------------------- absorption (M1)

def _toy_weights(seed, dims):
    return inputs.toy_layer(seed=seed, B=2, T=12, dims=dims, dtype=np.float64)


def test_absorbed_equals_mha_page_example():
    """The article runs both forms in float64 at B=2, T=12 with its example
    dimensions and reports agreement at the 1e-15 level."""
    W = _toy_weights(7, inputs.TOY_DIMS)
    h, pos = W["h"], W["pos"]
    a = oracle.mha_mode_layer(h, W, pos)
    b = oracle.absorbed_layer(h, W, pos)
    assert np.max(np.abs(a["u"] - b["u"])) <= 1e-14 * max(1.0, np.max(np.abs(a["u"])))
    assert np.max(np.abs(a["o"] - b["o"])) <= 1e-14 * np.max(np.abs(a["o"]))
    assert np.max(np.abs(a["lse"] - b["lse"])) <= 1e-13


def test_absorbed_equals_mha_toy_config_T256():
    W = inputs.toy_layer(seed=1, B=1, T=256, dtype=np.float64)
    a = oracle.mha_mode_layer(W["h"], W, W["pos"])
    b = oracle.absorbed_layer(W["h"], W, W["pos"])
    assert np.max(np.abs(a["o"] - b["o"])) <= 1e-13 * np.max(np.abs(a["o"]))
    assert np.max(np.abs(a["u"] - b["u"])) <= 1e-13 * np.max(np.abs(a["u"]))


def test_absorbed_equals_mha_v3_shapes():
    dims = dict(d=512, n_h=128, d_h=128, d_c=512, d_cq=256, d_r=64)
    W = inputs.toy_layer(seed=3, B=1, T=40, dims=dims, dtype=np.float64)
    a = oracle.mha_mode_layer(W["h"], W, W["pos"])
    b = oracle.absorbed_layer(W["h"], W, W["pos"])
    assert np.max(np.abs(a["o"] - b["o"])) <= 1e-13 * np.max(np.abs(a["o"]))


def test_absorption_identity():
    rng = np.random.default_rng(5)
    n_h, d_h, d_c = 8, 16, 32
    w = rng.standard_normal((n_h * d_h, d_c))
    q = rng.standard_normal((3, n_h, d_h))
    cvec = rng.standard_normal(d_c)
    k = (w @ cvec).reshape(n_h, d_h)        # k^C = W^UK c, per head
    lhs = np.einsum("thk,hk->th", q, k)      # q^T k
    rhs = oracle.absorb_q(q, w, n_h, d_h) @ cvec
    assert np.max(np.abs(lhs - rhs)) <= 1e-13 * np.max(np.abs(lhs))


def test_mpmath_bruteforce_tiny():
    """MHA-mode definition evaluated in 50-digit arithmetic on a tiny case
    (materialised keys/values per head) vs the oracle's absorbed decode."""
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    rng = np.random.default_rng(11)
    n_h, d_h, d_c, d_r, L, s_q = 2, 3, 4, 2, 4, 2
    w_uk = rng.standard_normal((n_h * d_h, d_c))
    w_uv = rng.standard_normal((n_h * d_h, d_c))
    q_c = rng.standard_normal((s_q, n_h, d_h))
    q_r = rng.standard_normal((s_q, n_h, d_r))
    c = rng.standard_normal((L, d_c))
    kr = rng.standard_normal((L, d_r))
    scale = 1.0 / math.sqrt(d_h + d_r)
    ql = oracle.absorb_q(q_c, w_uk, n_h, d_h)
    o_lat, lse = oracle.mqa_decode_rows(ql, q_r, c, kr, scale)
    o = oracle.up_proj_v(o_lat, w_uv, n_h, d_h)
    M = lambda a: mp.mpf(float(a))
    for i in range(s_q):
        t = L - s_q + i
        for hh in range(n_h):
            keys = []
            for j in range(t + 1):
                kc = [sum(M(w_uk[hh * d_h + a, b]) * M(c[j, b]) for b in range(d_c)) for a in range(d_h)]
                sc = sum(M(q_c[i, hh, a]) * kc[a] for a in range(d_h)) + \
                    sum(M(q_r[i, hh, a]) * M(kr[j, a]) for a in range(d_r))
                keys.append(sc * M(scale))
            z = sum(mp.e ** s for s in keys)
            assert abs(float(mp.log(z)) - lse[i, hh]) <= 1e-14
            for a in range(d_h):
                val = sum(mp.e ** keys[j] / z *
                          sum(M(w_uv[hh * d_h + a, b]) * M(c[j, b]) for b in range(d_c))
                          for j in range(t + 1))
                assert abs(float(val) - o[i, hh, a]) <= 1e-14 * max(1.0, abs(float(val)))


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("s_q,L", [(1, 1), (1, 37), (2, 2), (2, 37), (3, 70)])
def test_o2_matches_torch_sdpa(s_q, L):
    ql, qr, c, kr = _small_decode(seed=L, s_q=s_q, L=L)
    scale = 1.0 / math.sqrt(24)
    o, lse = oracle.mqa_decode_rows(ql, qr, c, kr, scale)
    q = torch.from_numpy(np.concatenate([ql, qr], -1)).permute(1, 0, 2)[None]   # [1,n_h,s_q,576']
    k = torch.from_numpy(np.concatenate([c, kr], -1))[None, None].expand(1, ql.shape[1], -1, -1)
    v = torch.from_numpy(c)[None, None].expand(1, ql.shape[1], -1, -1)
    pos_q = torch.arange(L - s_q, L)[:, None]
    mask = torch.arange(L)[None, :] <= pos_q                               # j <= t
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-14
    # lse from torch's logsumexp on the same masked scores
    s = (q @ k.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    ref_lse = torch.logsumexp(s, -1)[0].permute(1, 0).numpy()
    assert np.max(np.abs(lse - ref_lse)) <= 1e-13


def test_o1_matches_torch_sdpa_mha_mode():
    """The MHA-mode layer's attention core equals torch's attention with
    d_qk = d_h + d_r and d_v = d_h."""
    W = inputs.toy_layer(seed=4, B=1, T=20, dtype=np.float64)
    out = oracle.mha_mode_layer(W["h"], W, W["pos"])
    dm = W["dims"]
    n_h, d_h = dm["n_h"], dm["d_h"]
    kc = (out["c_kv"][0] @ np.asarray(W["w_uk"]).T).reshape(20, n_h, d_h)
    vc = (out["c_kv"][0] @ np.asarray(W["w_uv"]).T).reshape(20, n_h, d_h)
    q = torch.from_numpy(np.concatenate([out["q_c"][0], out["q_r"][0]], -1)).permute(1, 0, 2)
    kr = np.broadcast_to(out["k_r"][0][:, None, :], (20, n_h, dm["d_r"]))
    k = torch.from_numpy(np.concatenate([kc, kr], -1)).permute(1, 0, 2)
    v = torch.from_numpy(vc).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=True, scale=1 / math.sqrt(d_h + dm["d_r"]))
    assert np.max(np.abs(ref.permute(1, 0, 2).numpy() - out["o"][0])) <= 1e-14


# ---------------------------------------------------------------- closed forms

def test_single_key_returns_that_row():
    ql, qr, c, kr = _small_decode(seed=1, s_q=1, L=1)
    o, lse = oracle.mqa_decode_rows(ql, qr, c, kr, 0.3)
    assert np.array_equal(o[0], np.broadcast_to(c[0], o[0].shape))
    s0 = (np.einsum("hc,c->h", ql[0], c[0]) + np.einsum("hr,r->h", qr[0], kr[0])) * 0.3
    assert np.max(np.abs(lse[0] - s0)) <= 1e-15 * max(1, np.max(np.abs(s0)))


def test_zero_query_is_uniform_mean():
    _, _, c, kr = _small_decode(seed=2, L=29)
    s_q, n_h = 2, 4
    o, lse = oracle.mqa_decode_rows(np.zeros((s_q, n_h, 16)), np.zeros((s_q, n_h, 8)), c, kr, 0.1)
    for i in range(s_q):
        vis = 29 - s_q + i + 1
        assert np.max(np.abs(o[i] - c[:vis].mean(0))) <= 1e-15
        assert np.max(np.abs(lse[i] - math.log(vis))) <= 1e-15


def test_two_keys_sigmoid():
    from scipy.special import expit
    ql, qr, c, kr = _small_decode(seed=3, s_q=1, L=2)
    scale = 0.25
    o, _ = oracle.mqa_decode_rows(ql, qr, c, kr, scale)
    s = (ql[0] @ c.T + qr[0] @ kr.T) * scale
    w0 = expit(s[:, 0] - s[:, 1])
    ref = w0[:, None] * c[0] + (1 - w0)[:, None] * c[1]
    assert np.max(np.abs(o[0] - ref)) <= 1e-15


def test_dominant_key():
    ql, qr, c, kr = _small_decode(seed=4, s_q=1, L=9)
    qr = np.zeros_like(qr)
    ql = np.zeros_like(ql)
    kr = np.zeros_like(kr)
    kr[5, 0] = 1.0
    qr[0, :, 0] = 1e4                    # key 5 scores 1e4*scale above every other
    o, _ = oracle.mqa_decode_rows(ql, qr, c, kr, 1.0)
    assert np.max(np.abs(o[0] - c[5])) <= 1e-12


def test_softmax_rows_sum_to_one():
    ql, qr, c, kr = _small_decode(seed=5, s_q=1, L=50)
    p, _ = oracle.attention_probs(ql[0], qr[0], c, kr, 0.2, 50)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(-1) - 1)) <= 1e-15


def test_causal_rows_differ_only_by_last_keys():
    """s_q=2: the first new token must not see the second (j <= t)."""
    ql, qr, c, kr = _small_decode(seed=6, s_q=2, L=10)
    o, lse = oracle.mqa_decode_rows(ql, qr, c, kr, 0.3)
    o0, l0 = oracle.mqa_decode_rows(ql[:1], qr[:1], c[:9], kr[:9], 0.3)
    assert np.array_equal(o[0], o0[0]) and np.array_equal(lse[0], l0[0])


# ---------------------------------------------------------------- RoPE

def test_rope_is_complex_rotation():
    rng = np.random.default_rng(0)
    d, T = 32, 19
    x = rng.standard_normal((T, d))
    pos = np.arange(T) * 3 + 1
    z = x[:, : d // 2] + 1j * x[:, d // 2:]
    theta = np.power(10000.0, -np.arange(d // 2) * 2.0 / d)
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    ref = np.concatenate([zr.real, zr.imag], -1)
    assert np.max(np.abs(oracle.rope(x, pos) - ref)) <= 1e-13


def test_rope_properties():
    rng = np.random.default_rng(1)
    d = 64
    q, k = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    assert np.array_equal(oracle.rope(q, np.array([0])), q)
    r = oracle.rope(q, np.array([1234]))
    assert abs(np.linalg.norm(r) - np.linalg.norm(q)) <= 1e-12
    # <R_m q, R_n k> depends only on m - n
    def dot(m, n):
        return float((oracle.rope(q, np.array([m])) @ oracle.rope(k, np.array([n])).T)[0, 0])
    assert abs(dot(17, 5) - dot(112, 100)) <= 1e-12
    assert abs(dot(17, 5) - float((oracle.rope(q, np.array([12])) @ k.T)[0, 0])) <= 1e-12


# ---------------------------------------------------------------- split / combine / paging

@pytest.mark.parametrize("cuts", [[0, 37], [0, 1, 37], [0, 10, 20, 30, 37], [0, 36, 36, 37]])
def test_split_combine_equals_unsplit(cuts):
    ql, qr, c, kr = _small_decode(seed=8, s_q=2, L=37)
    full_o, full_l = oracle.mqa_decode_rows(ql, qr, c, kr, 0.2)
    parts = [oracle.mqa_decode_rows(ql, qr, c, kr, 0.2, key_range=(a, b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = oracle.combine_lse([p[0] for p in parts], [p[1] for p in parts])
    assert np.max(np.abs(o - full_o)) <= 1e-14
    assert np.max(np.abs(lse - full_l)) <= 1e-14


def test_combine_all_empty():
    o, lse = oracle.combine_lse(np.zeros((3, 2, 5)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_paging_invariance():
    a = inputs.decode_case(3, B=3, seq_lens=np.array([70, 128, 5]), n_h=4, d_c=16, d_r=8)
    b = inputs.decode_case(3, B=3, seq_lens=np.array([70, 128, 5]), n_h=4, d_c=16, d_r=8)
    # re-permute b's physical blocks
    rng = np.random.default_rng(99)
    perm = rng.permutation(b.num_blocks)
    newc = np.empty_like(b.cache)
    newc[perm] = b.cache
    b.cache = newc
    b.block_table = np.where(b.block_table >= 0, perm[np.maximum(b.block_table, 0)], -1)
    oa, la = oracle.mqa_decode_case(a)
    ob, lb = oracle.mqa_decode_case(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


# ---------------------------------------------------------------- storage formats

def test_e4m3fn_decoder_matches_torch_and_format_facts():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[0x7E] == 448.0 and np.isnan(ours[0x7F]) and ours[0x38] == 1.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0xB8] == -1.0


def test_bf16_decoder_matches_torch():
    bits = np.random.default_rng(0).integers(0, 2 ** 16, size=5000, dtype=np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_fp8_cache_roundtrip_error_bound():
    case = inputs.decode_case(9, B=2, seq_lens=np.array([100, 64]), n_h=4, kv_dtype="fp8")
    rng = np.random.Generator(np.random.PCG64(9))
    rng.permutation(case.num_blocks)
    rows = rng.standard_normal((case.num_blocks, 64, 576), dtype=np.float32)
    for b in range(2):
        L = int(case.seq_lens[b])
        c, kr = oracle.paged_rows(case.cache, case.block_table[b], L, "fp8", 512, 64, 64)
        logical = np.concatenate([rows[case.block_table[b, j]] for j in range((L + 63) // 64)])[:L]
        x = logical[:, :512].astype(np.float64)
        scale = np.abs(x).max(1) / 448.0
        err = np.abs(c - x)
        # e4m3 has 3 mantissa bits: half-ulp relative bound 2^-4 for normals,
        # absolute bound 2^-10 * scale in the subnormal range; plus fp32 scale rounding
        bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
        assert np.all(err <= bound)
        assert np.array_equal(kr, oracle.bf16_to_f64(inputs.f32_to_bf16_bits(logical[:, 512:])))


# ---------------------------------------------------------------- low-bit caches
# Layout (a reading; the QuantMLA review names only INT4 content + INT4 RoPE
# and INT2 content + INT4 RoPE): per block [bs x content codes | bs x RoPE
# codes | bs x groups x (fp16 scale, fp16 min)], groups of 32 values of one
# token, value = code * scale + min; little-endian 32-bit words, value 2k at
# bit k*b and value 2k+1 at bit 16 + k*b.  The fixtures below are written out
# by hand from that description.

_W4_0_7 = "20643175"      # values 0..7      -> word 0x75316420
_W4_8_15 = "a8ecb9fd"     # values 8..15     -> word 0xFDB9ECA8
_W2_0123 = "8888dddd"     # values 0,1,2,3 repeated (2-bit) -> word 0xDDDD8888


def _hexbytes(*parts):
    return np.frombuffer(bytes.fromhex("".join(parts)), dtype=np.uint8)


def test_int4_decoder_hand_fixture():
    # block_size 2, d_c = d_r = 32: token 0 content codes e % 16 with scale 0.5,
    # min -1; RoPE codes all 3 with scale 0.25, min 2; token 1 all codes 0 with
    # scale 0 and mins 1.5 / -0.5
    content = _hexbytes(_W4_0_7, _W4_8_15, _W4_0_7, _W4_8_15) .tolist() + [0] * 16
    rope = _hexbytes("33333333" * 4).tolist() + [0] * 16
    params = _hexbytes("0038" "00bc", "0034" "0040", "0000" "003e", "0000" "00b8").tolist()
    blk = np.array(content + rope + params, dtype=np.uint8)[None]
    c, kr = oracle.paged_rows(blk, [0], 2, "int4", 32, 32, 2)
    e = np.arange(32)
    assert np.array_equal(c[0], -1.0 + 0.5 * (e % 16))
    assert np.array_equal(kr[0], np.full(32, 2.75))
    assert np.array_equal(c[1], np.full(32, 1.5)) and np.array_equal(kr[1], np.full(32, -0.5))


def test_int2_decoder_hand_fixture():
    # block_size 1, d_c = 32 (2-bit codes e % 4, scale 1, min 0), d_r = 32
    # (4-bit codes e % 16, scale 2, min -8)
    blk = _hexbytes(_W2_0123, _W2_0123, _W4_0_7, _W4_8_15, _W4_0_7, _W4_8_15,
                    "003c" "0000", "0040" "00c8")[None]
    c, kr = oracle.paged_rows(blk, [0], 1, "int2", 32, 32, 1)
    e = np.arange(32)
    assert np.array_equal(c[0], (e % 4).astype(float))
    assert np.array_equal(kr[0], -8.0 + 2.0 * (e % 16))


@pytest.mark.parametrize("kv", ["int4", "int2"])
def test_int_cache_roundtrip_error_bound(kv):
    """Inputs' quantiser (written separately) -> oracle decoder: every value is
    within half a step of its group's fp16 scale of the original, plus what the
    fp16 rounding of the scale and minimum can move the grid."""
    case = inputs.decode_case(19, B=2, seq_lens=np.array([90, 40]), n_h=4, kv_dtype=kv)
    rng = np.random.Generator(np.random.PCG64(19))
    rng.permutation(case.num_blocks)
    rows = rng.standard_normal((case.num_blocks, 64, 576), dtype=np.float32).astype(np.float64)
    for b in range(2):
        L = int(case.seq_lens[b])
        c, kr = oracle.paged_rows(case.cache, case.block_table[b], L, kv, 512, 64, 64)
        logical = np.concatenate([rows[case.block_table[b, j]] for j in range((L + 63) // 64)])[:L]
        for got, x, bits in ((c, logical[:, :512], 4 if kv == "int4" else 2), (kr, logical[:, 512:], 4)):
            g = x.reshape(L, -1, 32)
            lo, hi = g.min(-1, keepdims=True), g.max(-1, keepdims=True)
            qmax = (1 << bits) - 1
            s = (hi - lo) / qmax
            s16 = s.astype(np.float16).astype(np.float64)
            m16 = lo.astype(np.float16).astype(np.float64)
            bound = 0.5 * s16 + qmax * np.abs(s16 - s) + np.abs(m16 - lo) + 1e-12
            assert np.all(np.abs(got.reshape(L, -1, 32) - g) <= bound)
            # the decoded values lie on the group's grid m16 + k * s16, k in 0..qmax
            k = (got.reshape(L, -1, 32) - m16) / np.where(s16 > 0, s16, 1.0)
            assert np.all(np.abs(k - np.rint(k)) < 1e-6) and k.min() > -1e-6 and k.max() < qmax + 1e-6


# ---------------------------------------------------------------- cache producer

def test_bf16_encoder_matches_torch_cast():
    # float32 inputs (exact in float64): direct float64 rounding equals torch's
    # float32 -> bfloat16 round-to-nearest-even cast
    x = np.random.default_rng(3).standard_normal(20000).astype(np.float32)
    x = np.concatenate([x, np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(-8, 9, dtype=np.float32)])
    ours = oracle.bf16_round_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3fn_encoder_nearest_ties_saturation():
    vals = oracle.e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
    grid = np.unique(vals[~np.isnan(vals)])
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(3000) * 40, grid, (grid[1:] + grid[:-1]) / 2,
                        [500.0, -1e4, 448.0, -448.0]])
    codes = oracle.e4m3fn_encode(x)
    dec = oracle.e4m3fn_to_f64(codes)
    xc = np.clip(x, -448, 448)
    # nearest grid value (brute force distance)
    dist = np.abs(grid[None, :] - xc[:, None]).min(1)
    assert np.allclose(np.abs(dec - xc), dist, rtol=0, atol=0)
    # representable values round-trip exactly; ties go to the even mantissa
    assert np.array_equal(oracle.e4m3fn_to_f64(oracle.e4m3fn_encode(grid)), grid)
    mid = (grid[1:] + grid[:-1]) / 2
    mc = oracle.e4m3fn_encode(mid)
    assert np.all((mc & 1) == 0)
    # agrees with torch's float32 -> float8_e4m3fn cast (round to nearest even)
    x32 = np.clip(rng.standard_normal(3000).astype(np.float32) * 50, -448, 448)
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_encode(x32.astype(np.float64)), ref)


def test_cache_append_bruteforce_tiny():
    """Element-by-element sums and complex-number rotation on a tiny layer."""
    rng = np.random.default_rng(5)
    T, d, d_c, d_r, bs = 3, 6, 4, 4, 2
    h = rng.standard_normal((T, d))
    wd, wr = rng.standard_normal((d_c, d)), rng.standard_normal((d_r, d))
    pos = np.array([0, 5, 2])
    slots = np.array([3, -1, 0])
    cache = np.full((2, bs, d_c + d_r), 7.0, dtype=np.float32)
    out = oracle.cache_append(cache, h, wd, wr, pos, slots, "f32", d_c, d_r, bs)
    for t in range(T):
        c = [sum(wd[i, k] * h[t, k] for k in range(d)) for i in range(d_c)]
        r = [sum(wr[i, k] * h[t, k] for k in range(d)) for i in range(d_r)]
        z = [complex(r[k], r[k + d_r // 2]) * complex(math.cos(pos[t] * 10000.0 ** (-2 * k / d_r)),
                                                     math.sin(pos[t] * 10000.0 ** (-2 * k / d_r)))
             for k in range(d_r // 2)]
        row = np.array(c + [v.real for v in z] + [v.imag for v in z], dtype=np.float32)
        if slots[t] >= 0:
            assert np.allclose(out[slots[t] // bs, slots[t] % bs], row, rtol=1e-6, atol=1e-6)
    # the skipped token and untouched slots keep their contents
    assert np.all(out[0, 1] == 7.0) and np.all(out[1, 0] == 7.0)


def test_project_bruteforce_tiny():
    """Every output of the layer's projections, recomputed element by element
    on a tiny layer with explicit sums and complex-number rotation (itwiki
    "Multi-head latent attention", "Structure": joint KV compression gives
    c^Q = W^DQ h and q^C = W^UQ c^Q, head i owning rows i*d_h .. (i+1)*d_h-1;
    decoupled RoPE gives q^R_i = RoPE(W^QR_i c^Q) per head and the shared
    k^R = RoPE(W^KR h)).  Fails if W^QR reads h instead of c^Q, if RoPE is
    dropped from either part, if a head's slice is transposed or taken from
    the wrong rows, or if the rotation pairs the wrong elements."""
    rng = np.random.default_rng(21)
    B, T, d, d_cq, n_h, d_h, d_r, d_c = 2, 3, 5, 3, 2, 3, 4, 4
    dims = {"d": d, "n_h": n_h, "d_h": d_h, "d_c": d_c, "d_cq": d_cq, "d_r": d_r}
    W = {"dims": dims}
    for name, (o, i) in {"w_dq": (d_cq, d), "w_uq": (n_h * d_h, d_cq), "w_qr": (n_h * d_r, d_cq),
                         "w_dkv": (d_c, d), "w_kr": (d_r, d)}.items():
        W[name] = rng.standard_normal((o, i))
    h = rng.standard_normal((B, T, d))
    pos = np.array([3, 0, 11])  # non-zero positions (0 is the identity rotation)
    c_kv, k_r, q_c, q_r = oracle.project(h, W, pos)

    def rot(vec, p):  # pair (k, k + n/2) as one complex number, times e^{i p theta_k}
        n = len(vec)
        out = [0.0] * n
        for k in range(n // 2):
            th = p * 10000.0 ** (-2.0 * k / n)
            z = complex(vec[k], vec[k + n // 2]) * complex(math.cos(th), math.sin(th))
            out[k], out[k + n // 2] = z.real, z.imag
        return out

    for b in range(B):
        for t in range(T):
            x = h[b, t]
            cq = [sum(W["w_dq"][m, k] * x[k] for k in range(d)) for m in range(d_cq)]
            ckv = [sum(W["w_dkv"][m, k] * x[k] for k in range(d)) for m in range(d_c)]
            kr = rot([sum(W["w_kr"][m, k] * x[k] for k in range(d)) for m in range(d_r)], pos[t])
            assert np.allclose(c_kv[b, t], ckv, rtol=1e-13, atol=1e-13)
            assert np.allclose(k_r[b, t], kr, rtol=1e-13, atol=1e-13)
            for i in range(n_h):
                qc = [sum(W["w_uq"][i * d_h + j, m] * cq[m] for m in range(d_cq)) for j in range(d_h)]
                qr = rot([sum(W["w_qr"][i * d_r + j, m] * cq[m] for m in range(d_cq)) for j in range(d_r)],
                         pos[t])
                assert np.allclose(q_c[b, t, i], qc, rtol=1e-13, atol=1e-13), (b, t, i)
                assert np.allclose(q_r[b, t, i], qr, rtol=1e-13, atol=1e-13), (b, t, i)
    # the rotation is not the identity here, so the test can see RoPE
    x0 = h[0, 0]
    cq0 = W["w_dq"] @ x0
    assert np.max(np.abs(q_r[0, 0, 1] - W["w_qr"][d_r:2 * d_r] @ cq0)) > 1e-3


def test_cache_append_then_decode_equals_mha_layer():
    """Append the toy layer's 256 tokens to a paged f32 cache through a
    permuted slot mapping, then decode the last token in MQA mode: equals the
    materialised MHA-mode layer output for that token."""
    W = inputs.toy_layer(seed=11, T=256)
    dm = W["dims"]
    n_h, d_h, d_c, d_r = dm["n_h"], dm["d_h"], dm["d_c"], dm["d_r"]
    h, pos = W["h"][0].astype(np.float64), W["pos"]
    bs, T = 64, 256
    perm = np.random.default_rng(12).permutation(T // bs + 2)[: T // bs]  # physical block of logical block j
    slots = perm[pos // bs] * bs + pos % bs
    cache = np.zeros((T // bs + 2, bs, d_c + d_r), dtype=np.float32)
    cache = oracle.cache_append(cache, h, W["w_dkv"], W["w_kr"], pos, slots, "f32", d_c, d_r, bs)
    c, kr = oracle.paged_rows(cache, perm, T, "f32", d_c, d_r, bs)
    ref = oracle.mha_mode_layer(W["h"], W, pos)
    _, _, q_c, q_r = oracle.project(W["h"], W, pos)
    q_lat = oracle.absorb_q(q_c[0, -1:], W["w_uk"], n_h, d_h)
    o_lat, lse = oracle.mqa_decode_rows(q_lat, q_r[0, -1:], c, kr, 1.0 / math.sqrt(d_h + d_r))
    o = oracle.up_proj_v(o_lat, W["w_uv"], n_h, d_h)
    # the cache holds float32-rounded rows: agreement to float32 precision
    assert np.max(np.abs(o[0] - ref["o"][0, -1])) <= 1e-5 * np.max(np.abs(ref["o"][0, -1]))
    assert np.max(np.abs(lse[0] - ref["lse"][0, -1])) <= 1e-5


def test_cache_append_fp8_and_bf16_layouts():
    rng = np.random.default_rng(6)
    T, d, d_c, d_r, bs = 5, 32, 16, 8, 4
    h = rng.standard_normal((T, d))
    wd, wr = rng.standard_normal((d_c, d)) / 5, rng.standard_normal((d_r, d)) / 5
    pos = np.array([3, 100, 7, 0, 4000])
    slots = np.array([5, 0, 11, -1, 2])
    c_ex = h @ wd.T
    r_ex = oracle.rope(h @ wr.T, pos)
    bb = bs * (d_c + 2 * d_r + 4)
    out8 = oracle.cache_append(np.zeros((3, bb), np.uint8), h, wd, wr, pos, slots, "fp8", d_c, d_r, bs)
    out16 = oracle.cache_append(np.zeros((3, bs, d_c + d_r), np.uint16), h, wd, wr, pos, slots, "bf16",
                                d_c, d_r, bs)
    for t in range(T):
        if slots[t] < 0:
            continue
        blk, row = slots[t] // bs, slots[t] % bs
        c8, kr8 = oracle.paged_rows(out8, [blk], bs, "fp8", d_c, d_r, bs)
        scale = np.abs(c_ex[t]).max() / 448.0
        bound = np.maximum(np.abs(c_ex[t]) * 2.0 ** -4, 2.0 ** -10 * scale) * (1 + 1e-6)
        assert np.all(np.abs(c8[row] - c_ex[t]) <= bound)
        assert np.max(np.abs(c8[row])) == pytest.approx(np.abs(c_ex[t]).max(), rel=2 ** -4)
        assert np.all(np.abs(kr8[row] - r_ex[t]) <= np.abs(r_ex[t]) * 2.0 ** -8 + 1e-30)
        c16, kr16 = oracle.paged_rows(out16, [blk], bs, "bf16", d_c, d_r, bs)
        assert np.all(np.abs(c16[row] - c_ex[t]) <= np.abs(c_ex[t]) * 2.0 ** -8)
        assert np.array_equal(kr16[row], kr8[row])
    # the skipped token's would-be rows stay zero
    assert not np.any(out8[0][3 * d_c:4 * d_c])


# ---------------------------------------------------------------- MHA-mode prefill pieces

def test_mha_attention_matches_torch_sdpa_causal():
    """Prefill attention with a RoPE key shared by all heads equals torch's
    causal attention on the concatenated [k^C; k^R] keys."""
    rng = np.random.default_rng(13)
    T, n_h, d_h, d_r = 45, 3, 16, 8
    q_c, q_r = rng.standard_normal((T, n_h, d_h)), rng.standard_normal((T, n_h, d_r))
    k_c, k_r, v_c = rng.standard_normal((T, n_h, d_h)), rng.standard_normal((T, d_r)), rng.standard_normal((T, n_h, 12))
    scale = 0.17
    o, lse = oracle.mha_attention(q_c, q_r, k_c, k_r, v_c, scale)
    q = torch.from_numpy(np.concatenate([q_c, q_r], -1)).permute(1, 0, 2)
    k = torch.from_numpy(np.concatenate([k_c, np.broadcast_to(k_r[:, None], (T, n_h, d_r))], -1)).permute(1, 0, 2)
    v = torch.from_numpy(v_c).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    assert np.max(np.abs(ref.permute(1, 0, 2).numpy() - o)) <= 1e-13
    s = (q @ k.transpose(-1, -2)) * scale
    s = s.masked_fill(~torch.ones(T, T, dtype=torch.bool).tril(), float("-inf"))
    assert np.max(np.abs(torch.logsumexp(s, -1).permute(1, 0).numpy() - lse)) <= 1e-12
    # the first query sees only the first key
    assert np.allclose(o[0], v_c[0], rtol=0, atol=1e-14)


def test_expand_kv_per_head_blocks():
    rng = np.random.default_rng(14)
    T, n_h, d_h, d_c = 7, 3, 4, 5
    c = rng.standard_normal((T, d_c))
    wk, wv = rng.standard_normal((n_h * d_h, d_c)), rng.standard_normal((n_h * d_h, d_c))
    k_c, v_c = oracle.expand_kv(c, wk, wv, n_h, d_h)
    for t in range(T):
        for i in range(n_h):
            for e in range(d_h):
                assert abs(k_c[t, i, e] - sum(wk[i * d_h + e, j] * c[t, j] for j in range(d_c))) <= 1e-12
                assert abs(v_c[t, i, e] - sum(wv[i * d_h + e, j] * c[t, j] for j in range(d_c))) <= 1e-12


# ---------------------------------------------------------------- GQLA GQA path

def _gqla_small(seed=0, s_q=2, n_h=8, n_g=2, d_h=16, d_c=24, d_r=8, L=37):
    rng = np.random.default_rng(seed)
    return dict(q_c=rng.standard_normal((s_q, n_h, d_h)), q_r=rng.standard_normal((s_q, n_h, d_r)),
                c=rng.standard_normal((L, d_c)), k_r=rng.standard_normal((L, d_r)),
                w_uk=rng.standard_normal((n_g * d_h, d_c)) / math.sqrt(d_c),
                w_uv=rng.standard_normal((n_g * d_h, d_c)) / math.sqrt(d_c), n_g=n_g, d_h=d_h,
                scale=1.0 / math.sqrt(d_h + d_r))


@pytest.mark.parametrize("s_q,L,n_g", [(1, 1, 2), (2, 37, 2), (2, 64, 4), (3, 10, 1), (2, 20, 8)])
def test_gqa_path_equals_absorbed_path(s_q, L, n_g):
    """The GQLA page: one set of weights, two algebraically equal decode
    paths.  The GQA path over k^C = W^UK_g c, v^C = W^UV_g c equals the
    MQA-absorb path over the latent, to float64 rounding."""
    X = _gqla_small(seed=L + n_g, s_q=s_q, n_g=n_g, L=L)
    k_c, v_c = oracle.expand_kv(X["c"], X["w_uk"], X["w_uv"], n_g, X["d_h"])
    o1, l1 = oracle.gqa_decode_rows(X["q_c"], X["q_r"], k_c, v_c, X["k_r"], X["scale"], n_g)
    o2, l2 = oracle.gqla_absorbed_rows(X["q_c"], X["q_r"], X["c"], X["k_r"], X["w_uk"], X["w_uv"], X["scale"], n_g)
    assert np.max(np.abs(o1 - o2)) <= 1e-13 * np.max(np.abs(o1))
    assert np.max(np.abs(l1 - l2)) <= 1e-13


@pytest.mark.parametrize("s_q,L", [(1, 5), (2, 37)])
def test_gqa_path_matches_torch_sdpa_grouped(s_q, L):
    X = _gqla_small(seed=3 * L, s_q=s_q, L=L, n_g=2)
    k_c, v_c = oracle.expand_kv(X["c"], X["w_uk"], X["w_uv"], 2, X["d_h"])
    o, lse = oracle.gqa_decode_rows(X["q_c"], X["q_r"], k_c, v_c, X["k_r"], X["scale"], 2)
    q = torch.from_numpy(np.concatenate([X["q_c"], X["q_r"]], -1)).permute(1, 0, 2)[None]       # [1, n_h, s_q, 24]
    kr = np.broadcast_to(X["k_r"][:, None], (L, 2, X["k_r"].shape[1]))
    k = torch.from_numpy(np.ascontiguousarray(np.concatenate([k_c, kr], -1))).permute(1, 0, 2)[None]  # [1, n_g, L, 24]
    v = torch.from_numpy(v_c).permute(1, 0, 2)[None]
    mask = torch.arange(L)[None, :] <= torch.arange(L - s_q, L)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=X["scale"],
                                                           enable_gqa=True)[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-14


def test_gqa_paged_layout_brute_force():
    """gqa_paged_rows against element-by-element placement from the block
    layout [n_g][bs][d_h] k^C | [n_g][bs][d_h] v^C | [bs][d_r] k^R."""
    n_g, d_h, d_r, bs, L = 2, 4, 2, 4, 7
    rng = np.random.default_rng(5)
    kc, vc, kr = rng.standard_normal((L, n_g, d_h)), rng.standard_normal((L, n_g, d_h)), rng.standard_normal((L, d_r))
    table = [1, 0]
    cache = np.full((2, bs * (2 * n_g * d_h + d_r)), np.nan)
    for j in range(L):
        blk, t = table[j // bs], j % bs
        for g in range(n_g):
            for e in range(d_h):
                cache[blk, (g * bs + t) * d_h + e] = kc[j, g, e]
                cache[blk, n_g * bs * d_h + (g * bs + t) * d_h + e] = vc[j, g, e]
        for e in range(d_r):
            cache[blk, 2 * n_g * bs * d_h + t * d_r + e] = kr[j, e]
    a, b, c = oracle.gqa_paged_rows(cache, table, L, n_g, d_h, d_r, bs, kv_dtype="f32")
    assert np.array_equal(a, kc) and np.array_equal(b, vc) and np.array_equal(c, kr)
