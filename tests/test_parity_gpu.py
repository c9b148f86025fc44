"""GPU parity: every C-ABI entry point against the float64 oracle on the same
seeded, rounded inputs (MI355X only)."""

import math

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_05_amd import binding, inputs

from gpu_helpers import (assert_bf16_close, assert_f32_close, assert_lse_close, bf16_dev, case_to_device,
                         f32_dev, run_decode, say)

pytestmark = pytest.mark.gpu

V3 = dict(n_h=128, d_c=512, d_r=64, d_h=128)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()


# ------------------------------------------------------------------ toy layer, fp32

def _toy_paged(rows: np.ndarray, block_size: int, seed: int):
    """Place [T, D] fp32 rows into a shuffled paged cache (test plumbing)."""
    T, D = rows.shape
    nblk = (T + block_size - 1) // block_size
    perm = np.random.default_rng(seed).permutation(nblk)
    cache = np.zeros((nblk, block_size, D), dtype=np.float32)
    for j in range(nblk):
        n = min(block_size, T - j * block_size)
        cache[perm[j], :n] = rows[j * block_size: j * block_size + n]
    return cache, perm.astype(np.int32)[None]


@pytest.mark.parametrize("s_q,block_size,splits", [(1, 64, 0), (1, 64, 3), (16, 64, 0), (4, 32, 2)])
def test_toy_layer_fp32_end_to_end(s_q, block_size, splits):
    """Toy MLA layer (d=1024, n_h=8, d_h=64, d_c=128, d_r=32, T=256, fp32):
    absorb -> paged decode -> up-projection vs the MHA-mode oracle."""
    say(f"toy fp32 s_q={s_q} bs={block_size} splits={splits}")
    W = inputs.toy_layer(seed=1, B=1, T=256)
    dm = W["dims"]
    n_h, d_h, d_c, d_r = dm["n_h"], dm["d_h"], dm["d_c"], dm["d_r"]
    ref = oracle.mha_mode_layer(W["h"], W, W["pos"])
    T = 256
    rows = np.concatenate([ref["c_kv"][0], ref["k_r"][0]], -1).astype(np.float32)
    cache, table = _toy_paged(rows, block_size, seed=11)
    q_c = ref["q_c"][0, T - s_q:].astype(np.float32)                      # [s_q, n_h, d_h]
    q_r = ref["q_r"][0, T - s_q:].astype(np.float32)                      # [s_q, n_h, d_r]
    dev = "cuda"
    q_lat = binding.absorb_q(f32_dev(q_c), f32_dev(W["w_uk"]))             # [s_q, n_h, d_c] fp32
    o_lat, lse = binding.decode(q_lat.view(1, s_q, n_h, d_c), f32_dev(q_r).view(1, s_q, n_h, d_r),
                                f32_dev(cache), torch.from_numpy(table).to(dev),
                                torch.tensor([T], dtype=torch.int32, device=dev), 1.0 / math.sqrt(d_h + d_r),
                                block_size=block_size, out_dtype=torch.float32, num_splits=splits)
    o = binding.up_proj_v(o_lat.view(s_q, n_h, d_c), f32_dev(W["w_uv"]), d_h)
    torch.cuda.synchronize()
    o_ref = ref["o"][0, T - s_q:]
    assert_f32_close(o.cpu().numpy().astype(np.float64), o_ref, "o")
    assert_lse_close(lse.cpu().numpy()[0].astype(np.float64), ref["lse"][0, T - s_q:], "lse", tol=1e-5)
    # absorbed latent output matches the oracle's absorbed form
    o3 = oracle.absorbed_layer(W["h"], W, W["pos"])
    assert_f32_close(o_lat.cpu().numpy()[0].astype(np.float64), o3["o_lat"][0, T - s_q:], "o_lat")


# ------------------------------------------------------------------ V3 shapes, reduced sizes

RAGGED = np.array([1, 31, 32, 33, 63, 64, 65, 127, 1000, 4097], dtype=np.int32)


@pytest.mark.parametrize("force_generic", [False, True])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_v3_bf16_ragged_lengths(force_generic, splits):
    say(f"v3 bf16 ragged generic={force_generic} splits={splits}")
    case = inputs.decode_case(21, B=len(RAGGED), seq_lens=RAGGED, kv_dtype="bf16", tail_fill="nan", **V3)
    g, gl = run_decode(case, num_splits=splits, force_generic=force_generic)
    o, ol = oracle.mqa_decode_case(case)
    assert_bf16_close(g, o, "o_lat")
    assert_lse_close(gl, ol, "lse")


def test_v3_bf16_output_dtype_bf16():
    say("v3 bf16 out bf16")
    case = inputs.decode_case(22, B=4, seq_lens=np.array([700, 64, 5, 2049]), **V3)
    g, gl = run_decode(case, out_dtype=torch.bfloat16)
    o, ol = oracle.mqa_decode_case(case)
    assert_bf16_close(g, o, "o_lat bf16")
    assert_lse_close(gl, ol, "lse")


@pytest.mark.parametrize("s_q", [2, 3, 4])
def test_v3_bf16_multi_token_causal(s_q):
    say(f"v3 bf16 s_q={s_q}")
    lens = np.array([s_q, 40, 64, 65, 300], dtype=np.int32)
    case = inputs.decode_case(23, B=len(lens), seq_lens=lens, s_q=s_q, tail_fill="nan", **V3)
    for splits in (0, 2):
        g, gl = run_decode(case, num_splits=splits)
        o, ol = oracle.mqa_decode_case(case)
        assert_bf16_close(g, o, f"o_lat s_q={s_q} splits={splits}")
        assert_lse_close(gl, ol, "lse")


@pytest.mark.parametrize("force_generic", [False, True])
def test_v3_fp8_cache_sq2(force_generic):
    say(f"v3 fp8 s_q=2 generic={force_generic}")
    lens = np.array([2, 33, 64, 129, 1500], dtype=np.int32)
    case = inputs.decode_case(24, B=len(lens), seq_lens=lens, s_q=2, kv_dtype="fp8", **V3)
    for splits in (0, 3):
        g, gl = run_decode(case, num_splits=splits, force_generic=force_generic)
        o, ol = oracle.mqa_decode_case(case)
        assert_bf16_close(g, o, f"fp8 splits={splits}")
        assert_lse_close(gl, ol, "lse")


@pytest.mark.parametrize("force_generic", [False, True])
@pytest.mark.parametrize("kv", ["int4", "int2"])
@pytest.mark.parametrize("s_q", [1, 2])
def test_v3_int_cache(kv, s_q, force_generic):
    """Low-bit caches (grouped fp16 scale/min, packed codes) against the
    oracle's decoding of the same bytes: the MFMA kernel (values decoded to
    fp16 in LDS, fp16 products with fp32 accumulation) and the portable
    kernel (fp32 values), both at the bf16 output bars and |dlse| <= 1e-3."""
    say(f"v3 {kv} s_q={s_q} generic={force_generic}")
    lens = np.array([2, 33, 64, 129, 1500], dtype=np.int32)
    case = inputs.decode_case(26 + s_q, B=len(lens), seq_lens=lens, s_q=s_q, kv_dtype=kv, **V3)
    o, ol = oracle.mqa_decode_case(case)
    for splits in (0, 3):
        g, gl = run_decode(case, num_splits=splits, force_generic=force_generic)
        assert_bf16_close(g, o, f"{kv} splits={splits}")
        assert_lse_close(gl, ol, "lse")


# Scores that climb in steps along each sequence: RoPE dimension 0 of every
# query is 1 (its other RoPE dimensions are scaled by 1/4) and k^R dimension 0
# of the row at position p holds 84 times the number of step positions <= p
# less the number of steps (the last level is 0), so each step lifts the
# log2-domain score by 84 * log2(e) / sqrt(192) ~ 8.75 while the random parts
# spread it by ~0.3.  Ending at 0 keeps the heavy rows' scores small: the int
# caches' values, rounded to fp16 when decoded, carry a relative error of
# 2^-11 into each score, which at the top level of a staircase that climbs
# from 0 (scores ~28) would alone move the LSE by 1.5e-3.  The running reference max of the
# online softmax then has to move by more than the lazy threshold (2^8) at
# every step past the first subtile, inside units and in their last subtile,
# while the rows before a step keep 1-8 % of the weight (the last step comes
# 30-70 rows before the end): a rescale factor off by 2x moves o_lat by that
# much, and a P.V step applied on the wrong side of a rescale by far more.
STEP_LENS = np.array([4096, 2049, 1500, 700, 300, 129, 3333, 97], dtype=np.int32)
STEP_AT = [[1024, 2048, 3000, 4060], [64, 1000, 2010], [33, 97, 700, 1460], [300, 660],
           [100, 264], [90], [5, 2000, 3300], [60]]


def _stair(n, at):
    """Per position 0..n-1: 84 x (steps at or before it - all steps)."""
    return 84.0 * (np.searchsorted(np.asarray(at), np.arange(n), side="right") - len(at))


def _stepped_case(seed, kv, s_q):
    shift = [_stair(n, at) for n, at in zip(STEP_LENS, STEP_AT)]
    case = inputs.decode_case(seed, B=len(STEP_LENS), seq_lens=STEP_LENS, s_q=s_q, kv_dtype=kv,
                              rope0_shift=shift, **V3)
    qr = inputs.bf16_bits_as_f32(case.q_rope)
    qr[..., 0] = 1.0
    qr[..., 1:] *= 0.25
    case.q_rope = inputs.f32_to_bf16_bits(qr)
    return case


@pytest.mark.parametrize("force_generic", [False, True])
@pytest.mark.parametrize("kv,s_q", [("bf16", 1), ("fp8", 2), ("int4", 1)])
def test_v3_rising_scores_rescale(kv, s_q, force_generic):
    say(f"v3 {kv} s_q={s_q} stepped scores generic={force_generic}")
    case = _stepped_case(31, kv, s_q)
    o, ol = oracle.mqa_decode_case(case)
    for splits in (0, 1, 3):
        g, gl = run_decode(case, num_splits=splits, force_generic=force_generic)
        assert_bf16_close(g, o, f"{kv} stepped splits={splits}")
        assert_lse_close(gl, ol, "lse")


@pytest.mark.parametrize("force_generic", [False, True])
@pytest.mark.parametrize("kv,s_q", [("fp8", 1), ("fp8", 2), ("int4", 1), ("int2", 2)])
def test_v3_low_precision_caches_nan_tails(kv, s_q, force_generic):
    """The unused rows of each sequence's last block hold NaN codes, RoPE keys
    and scales (fp8) or NaN group scales and minima (int4 / int2): nothing of
    them may reach the result, in ragged last subtiles of every length."""
    say(f"v3 {kv} s_q={s_q} nan tails generic={force_generic}")
    lens = np.array([2, 33, 63, 65, 100, 129, 700, 1029], dtype=np.int32)
    case = inputs.decode_case(35 + s_q, B=len(lens), seq_lens=lens, s_q=s_q, kv_dtype=kv, tail_fill="nan", **V3)
    o, ol = oracle.mqa_decode_case(case)
    for splits in (0, 3):
        g, gl = run_decode(case, num_splits=splits, force_generic=force_generic)
        assert_bf16_close(g, o, f"{kv} nan tails splits={splits}")
        assert_lse_close(gl, ol, "lse")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int4"])
def test_v3_zero_queries_closed_form(kv):
    """Zero queries give equal scores: o_lat is the plain mean of the visible
    latent rows and lse = ln(number of visible keys), for every query token
    (a closed form, checked beside the oracle)."""
    say(f"v3 {kv} zero queries")
    lens = np.array([3, 64, 65, 1000, 4097], dtype=np.int32)
    case = inputs.decode_case(39, B=len(lens), seq_lens=lens, s_q=2, kv_dtype=kv, **V3)
    case.q_lat[:] = 0
    case.q_rope[:] = 0
    g, gl = run_decode(case, num_splits=3)
    for b, L in enumerate(lens):
        c, _ = oracle.paged_rows(case.cache, case.block_table[b], int(L), kv, 512, 64, case.block_size)
        for i in range(2):
            n = int(L) - 2 + i + 1  # keys visible to query token i
            assert_bf16_close(g[b, i], np.broadcast_to(c[:n].mean(0), (128, 512)), f"{kv} b={b} i={i}")
            assert np.max(np.abs(gl[b, i] - math.log(n))) <= 1e-3


@pytest.mark.parametrize("seed", range(8))
def test_v3_randomized_configurations(seed):
    """Seeded random configurations at V3 shapes (every cache format with
    both kernels): new tokens per sequence, batch size, log-uniform lengths
    and split count drawn per case, NaN in the unused tail rows, each
    against the oracle."""
    rng = np.random.default_rng(900 + seed)
    kv = ["bf16", "fp8", "int4", "int2"][seed % 4]  # each format with both kernels
    generic = seed >= 4
    s_q = int(rng.integers(1, 4))
    B = int(rng.integers(1, 7))
    lens = np.exp(rng.uniform(np.log(s_q), np.log(5000), size=B)).astype(np.int32)
    lens = np.maximum(lens, s_q)
    splits = int(rng.choice([0, 1, 2, 5]))
    say(f"random v3 seed={seed}: {kv} s_q={s_q} B={B} lens={lens.tolist()} splits={splits} generic={generic}")
    case = inputs.decode_case(950 + seed, B=B, seq_lens=lens, s_q=s_q, kv_dtype=kv, tail_fill="nan", **V3)
    g, gl = run_decode(case, num_splits=splits, force_generic=generic)
    o, ol = oracle.mqa_decode_case(case)
    assert_bf16_close(g, o, f"random seed={seed}")
    assert_lse_close(gl, ol, "lse")


@pytest.mark.parametrize("kv", ["int4", "int2"])
def test_toy_int_cache_fp32_queries(kv):
    """fp32 queries at the toy dimensions (n_h 8, d_c 128, d_r 32): the
    dequantised values are exact in fp32, so the fp32 bar applies."""
    say(f"toy {kv} fp32 queries")
    case = inputs.decode_case(31, B=3, seq_lens=np.array([1, 70, 200]), s_q=1, n_h=8, d_c=128, d_r=32, d_h=64,
                              kv_dtype=kv, q_dtype="f32")
    g, gl = run_decode(case, num_splits=2)
    o, ol = oracle.mqa_decode_case(case)
    assert_f32_close(g, o, f"toy {kv}")
    assert np.max(np.abs(gl - ol)) <= 1e-5


def test_mfma_matches_generic_kernel():
    """The two kernels agree closely with each other (both fp32 accumulation)."""
    say("mfma vs generic")
    case = inputs.decode_case(25, B=3, seq_lens=np.array([333, 2048, 17]), **V3)
    a, al = run_decode(case)
    b, bl = run_decode(case, force_generic=True)
    assert np.abs(a - b).max() <= 2e-3
    assert np.abs(al - bl).max() <= 1e-4


def test_split_count_invariance():
    say("split invariance")
    case = inputs.decode_case(26, B=2, seq_lens=np.array([4096, 1234]), **V3)
    base, bl = run_decode(case, num_splits=1)
    for k in (2, 5, 16, 64):
        g, gl = run_decode(case, num_splits=k)
        assert np.abs(g - base).max() <= 2e-3, k
        assert np.abs(gl - bl).max() <= 1e-4, k


def test_determinism_and_paging_invariance():
    say("determinism + paging")
    case = inputs.decode_case(27, B=3, seq_lens=np.array([900, 64, 3000]), **V3)
    a, al = run_decode(case)
    b, bl = run_decode(case)
    assert np.array_equal(a, b) and np.array_equal(al, bl)
    # same logical rows behind a different physical permutation: bit-identical
    perm = np.random.default_rng(5).permutation(case.num_blocks)
    c2 = inputs.decode_case(27, B=3, seq_lens=np.array([900, 64, 3000]), **V3)
    newc = np.empty_like(c2.cache)
    newc[perm] = c2.cache
    c2.cache = newc
    c2.block_table = np.where(c2.block_table >= 0, perm[np.maximum(c2.block_table, 0)], -1).astype(np.int32)
    c, cl = run_decode(c2)
    assert np.array_equal(a, c) and np.array_equal(al, cl)


def _subbatch(case, rows):
    """The same sequences (cache pages, queries) in another batch: row i of the
    new batch is row rows[i] of `case` (repeats allowed)."""
    import copy
    c = copy.copy(case)
    rows = np.asarray(rows)
    c.B = len(rows)
    c.seq_lens = case.seq_lens[rows].copy()
    nblk = int(((c.seq_lens + case.block_size - 1) // case.block_size).max())
    c.block_table = np.ascontiguousarray(case.block_table[rows, :nblk])
    c.q_lat = np.ascontiguousarray(case.q_lat[rows])
    c.q_rope = np.ascontiguousarray(case.q_rope[rows])
    return c


@pytest.mark.parametrize("splits", [0, 3])
def test_batch_composition_invariance(splits):
    """A sequence's result does not depend on the batch around it (its
    neighbours, its position, the batch size, repeats of it).  With a fixed
    split count every sequence is cut the same way in every batch, so the
    results are bit-identical; automatic planning may cut it differently,
    which changes only the merge's rounding."""
    say(f"batch composition splits={splits}")
    case = inputs.decode_case(31, B=6, seq_lens=np.array([3000, 65, 1, 777, 4096, 130]), **V3)
    base, bl = run_decode(case, num_splits=splits)
    for rows in ([3], [1, 3, 5], [4, 4, 0, 2, 3, 3, 1, 5, 4], [5, 4, 3, 2, 1, 0]):
        g, gl = run_decode(_subbatch(case, rows), num_splits=splits)
        if splits:
            assert np.array_equal(g, base[rows]) and np.array_equal(gl, bl[rows]), rows
        else:
            assert np.abs(g - base[rows]).max() <= 2e-3, rows
            assert np.abs(gl - bl[rows]).max() <= 1e-4, rows


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_long_sequence_many_splits(out_dtype):
    """One long sequence over the whole device: many partitions, merged by the
    one-workgroup-per-row merge (fp32 or bf16 partial rows)."""
    say(f"long sequence 40000 tokens, out {out_dtype}")
    case = inputs.decode_case(28, B=1, seq_lens=np.array([40000]), **V3)
    g, gl = run_decode(case, out_dtype=out_dtype)
    o, ol = oracle.mqa_decode_case(case)
    assert_bf16_close(g, o, "long")
    assert_lse_close(gl, ol, "lse")


def test_more_partitions_than_the_merge_caches():
    """1032 one-page partitions of one sequence: the merge recomputes weights
    instead of caching them in LDS (more than 1024 partitions)."""
    say("1032 partitions")
    case = inputs.decode_case(29, B=1, seq_lens=np.array([66000]), **V3)
    g, gl = run_decode(case, num_splits=1032)
    o, ol = oracle.mqa_decode_case(case)
    assert_bf16_close(g, o, "1032 partitions")
    assert_lse_close(gl, ol, "lse")


# ------------------------------------------------------------------ full workload sizes (sampled)

@pytest.mark.parametrize("name,seqs", [
    ("v3_bf16_B64_ctx8192", [0, 37, 63]),
    ("v3_bf16_B128_ctxlogU128-32768", None),
    ("v3_bf16_B4_ctx131072", [2]),
    ("v3_fp8_B64_ctx16384_sq2", [0, 63]),
    ("v3_bf16_B64_ctx8192_sq2", [3, 61]),
    ("v3_int4_B64_ctx8192", [5, 60]),
    ("v3_int2_B64_ctx8192", [7, 58]),
])
def test_full_size_workloads_sampled(name, seqs):
    """Full workload shape in the automatic split configuration the benchmark
    times; the oracle checks sampled sequences one by one."""
    say(f"full size {name}")
    case = inputs.workload_case(name)
    if seqs is None:  # variable lengths: shortest, longest and a middle one
        order = np.argsort(case.seq_lens)
        seqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    g, gl = run_decode(case, out_dtype=torch.bfloat16)
    o, ol = oracle.mqa_decode_case(case, seqs)
    assert np.all(np.isfinite(g))
    assert_bf16_close(g[seqs], o, name)
    assert_lse_close(gl[seqs], ol, name)


@pytest.mark.parametrize("name,seqs", [
    ("v3_bf16_B64_ctx8192", [0, 33, 63]),
    ("v3_bf16_B128_ctxlogU128-32768", None),
    ("v3_bf16_B4_ctx131072", [1]),
])
def test_decode_step_full_size_sampled(name, seqs):
    """mla_decode_step at full workload sizes with automatic splits, as the
    benchmark times it: absorb + attention + merge/W^UV against the oracle on
    sampled sequences (the 131072-token sequences have 64 partitions each,
    merged in batches by the fused tail)."""
    say(f"decode step full size {name}")
    case = inputs.workload_case(name)
    if seqs is None:  # variable lengths: shortest, longest and a middle one
        order = np.argsort(case.seq_lens)
        seqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    P = inputs.projection_weights(62, T_q=case.B)
    d = case_to_device(case)
    qn = bf16_dev(P["q_c"]).view(case.B, 1, 128, 128)
    o, lse = binding.decode_step(qn, bf16_dev(P["w_uk"]), d["q_rope"], d["kv_cache"], d["block_table"],
                                 d["seq_lens"], bf16_dev(P["w_uv"]), d["softmax_scale"])
    torch.cuda.synchronize()
    g = o.float().cpu().numpy().astype(np.float64).reshape(case.B, 128, 128)
    gl = lse.cpu().numpy().astype(np.float64).reshape(case.B, 1, 128)
    del d
    assert np.all(np.isfinite(g))
    ql = oracle.absorb_q(oracle.bf16_to_f64(P["q_c"]), oracle.bf16_to_f64(P["w_uk"]), 128, 128)
    ql = oracle.bf16_to_f64(oracle.bf16_round_bits(ql))
    for b in seqs:
        _, qr, c, kr = oracle.decode_case_rows(case, b)
        ol, l = oracle.mqa_decode_rows(ql[b][None], qr, c, kr, case.softmax_scale)
        ref = oracle.up_proj_v(ol, oracle.bf16_to_f64(P["w_uv"]), 128, 128)[0]
        assert_bf16_close(g[b], ref, f"step seq {b}")
        assert_lse_close(gl[b], l, f"step lse {b}")


# ------------------------------------------------------------------ combine, projections

@pytest.mark.parametrize("N,S,D", [(1, 1, 4), (37, 5, 512), (256, 64, 512), (5, 3, 132)])
def test_combine_lse(N, S, D):
    say(f"combine N={N} S={S} D={D}")
    rng = np.random.default_rng(N * 1000 + S)
    o = rng.standard_normal((N, S, D)).astype(np.float32)
    l = (rng.standard_normal((N, S)) * 3).astype(np.float32)
    splits = rng.integers(0, S + 1, size=N).astype(np.int32)
    if N > 2:
        l[1, :] = -np.inf          # a row with only empty splits
        l[2, 0] = -np.inf          # one empty split
        splits[1] = S
    for use_splits in (False, True):
        out, lse = binding.combine_lse(f32_dev(o), f32_dev(l),
                                       torch.from_numpy(splits).cuda() if use_splits else None)
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        for n in range(N):
            k = splits[n] if use_splits else S
            if k == 0:
                ro, rl = np.zeros(D), -np.inf
            else:
                ro, rl = oracle.combine_lse(o[n, :k].astype(np.float64), l[n, :k].astype(np.float64))
            assert np.abs(out[n] - ro).max() <= 1e-5 * max(1, np.abs(ro).max()), (n, use_splits)
            if np.isfinite(rl):
                assert abs(lse[n] - rl) <= 1e-5, (n, use_splits)
            else:
                assert np.isneginf(lse[n])


@pytest.mark.parametrize("T", [1, 4, 64, 100])
def test_absorb_and_up_proj_bf16_v3(T):
    say(f"projections bf16 T={T}")
    P = inputs.projection_weights(31 + T, T_q=T)
    qc, wuk, wuv, ol = (bf16_dev(P[k]) for k in ("q_c", "w_uk", "w_uv", "o_lat"))
    q_lat = binding.absorb_q(qc, wuk, out_dtype=torch.float32)
    o = binding.up_proj_v(ol, wuv, 128, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_q = oracle.absorb_q(oracle.bf16_to_f64(P["q_c"]), oracle.bf16_to_f64(P["w_uk"]), 128, 128)
    ref_o = oracle.up_proj_v(oracle.bf16_to_f64(P["o_lat"]), oracle.bf16_to_f64(P["w_uv"]), 128, 128)
    # bf16 inputs, fp32 accumulation over 128 / 512 terms
    assert_f32_close(q_lat.cpu().numpy().astype(np.float64), ref_q, "q_lat", tol=1e-5)
    assert_f32_close(o.cpu().numpy().astype(np.float64), ref_o, "o", tol=1e-5)
    q16 = binding.absorb_q(qc, wuk)            # bf16 output
    torch.cuda.synchronize()
    assert_bf16_close(q16.float().cpu().numpy().astype(np.float64), ref_q, "q_lat bf16")


def test_absorb_strided_tokens():
    """q_nope rows with a token stride larger than n_h*d_h (a slice of a wider buffer)."""
    say("absorb strided")
    P = inputs.projection_weights(41, T_q=5)
    wide = torch.zeros((5, 128 * 128 + 64), dtype=torch.bfloat16, device="cuda")
    wide[:, :128 * 128] = bf16_dev(P["q_c"]).view(5, -1)
    q = wide[:, :128 * 128].view(5, 128, 128)
    out = binding.absorb_q(q, bf16_dev(P["w_uk"]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.absorb_q(oracle.bf16_to_f64(P["q_c"]), oracle.bf16_to_f64(P["w_uk"]), 128, 128)
    assert_f32_close(out.cpu().numpy().astype(np.float64), ref, "strided")


def test_graph_replay_matches_eager():
    """The whole step (absorb, decode, up-projection) captured in a HIP graph:
    every replay, with eager work and synchronisations in between, gives the
    eager results bit for bit (the library issues no memset or allocation)."""
    say("graph replay")
    case = inputs.decode_case(61, B=6, seq_lens=np.array([5000, 64, 777, 3001, 129, 2048]), **V3)
    d = case_to_device(case)
    B, s_q = case.B, case.s_q
    P = inputs.projection_weights(62, T_q=B * s_q)
    qc, wuk, wuv = (bf16_dev(P[k]) for k in ("q_c", "w_uk", "w_uv"))
    q_lat = torch.empty((B * s_q, 128, 512), dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty((B, s_q, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, s_q, 128), dtype=torch.float32, device="cuda")
    o = torch.empty((B * s_q, 128, 128), dtype=torch.bfloat16, device="cuda")
    ws = binding.alloc_workspace(B, s_q, 128, 512, d["block_table"].shape[1])

    def step():
        binding.absorb_q(qc, wuk, out=q_lat)
        binding.decode(q_lat.view(B, s_q, 128, 512), d["q_rope"], d["kv_cache"], d["block_table"], d["seq_lens"],
                       d["softmax_scale"], kv_dtype=d["kv_dtype"], d_r=d["d_r"], out=o_lat, lse=lse, workspace=ws)
        binding.up_proj_v(o_lat.view(B * s_q, 128, 512), wuv, 128, out=o)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q_lat, o_lat, lse, o)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (q_lat, o_lat, lse, o):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip((q_lat, o_lat, lse, o), ref):
            assert torch.equal(t, r), f"replay {rep}"
        step()  # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ cache producer

def _append_gpu(inp, kv_dtype, cache_np):
    if inp["dtype"] == "bf16":
        h, w = bf16_dev(inp["h"]), bf16_dev(inp["w"])
    else:
        h, w = f32_dev(inp["h"]), f32_dev(inp["w"])
    cache = torch.from_numpy(np.ascontiguousarray(cache_np)).cuda()
    kdt = {"bf16": binding.MLA_BF16, "fp8": binding.MLA_FP8_E4M3, "f32": binding.MLA_F32}[kv_dtype]
    binding.cache_append(h, w, torch.from_numpy(inp["pos"]).cuda(), torch.from_numpy(inp["slots"]).cuda(), cache,
                         inp["d_c"], inp["d_r"], inp["block_size"], kv_dtype=kdt)
    torch.cuda.synchronize()
    return cache.cpu().numpy()


def _append_oracle(inp, kv_dtype, cache_np):
    dec = oracle.bf16_to_f64 if inp["dtype"] == "bf16" else (lambda a: np.asarray(a, np.float64))
    h, w = dec(inp["h"]), dec(inp["w"])
    d_c = inp["d_c"]
    return oracle.cache_append(cache_np, h, w[:d_c], w[d_c:], inp["pos"], inp["slots"], kv_dtype, d_c, inp["d_r"],
                               inp["block_size"])


def _exact_rows(inp):
    dec = oracle.bf16_to_f64 if inp["dtype"] == "bf16" else (lambda a: np.asarray(a, np.float64))
    h, w = dec(inp["h"]), dec(inp["w"])
    y = h @ w.T
    d_c = inp["d_c"]
    return y[:, :d_c], oracle.rope(y[:, d_c:], inp["pos"])


@pytest.mark.parametrize("T,skip", [(64, 0), (1, 0), (37, 5), (130, 0), (257, 3)])
def test_cache_append_bf16_v3(T, skip):
    say(f"cache append bf16 T={T}")
    inp = inputs.append_inputs(70 + T, T, skip_every=skip)
    nb, bs, N = inp["num_blocks"], inp["block_size"], 576
    poison = np.full((nb, bs, N), 0x7FC1, dtype=np.uint16)  # NaN bits: untouched rows must keep them
    got = _append_gpu(inp, "bf16", poison)
    ref = _append_oracle(inp, "bf16", poison)
    c_ex, r_ex = _exact_rows(inp)
    written = np.zeros((nb * bs,), dtype=bool)
    for t in range(T):
        sl = inp["slots"][t]
        if sl < 0:
            continue
        written[sl] = True
        row = oracle.bf16_to_f64(got[sl // bs, sl % bs])
        ex = np.concatenate([c_ex[t], r_ex[t]])
        # bf16 storage of an fp32 accumulation: within one bf16 step of the exact row
        assert np.all(np.abs(row - ex) <= np.abs(ex) * 2.0 ** -7 + 1e-6), t
    flat_got, flat_ref = got.reshape(nb * bs, N), ref.reshape(nb * bs, N)
    assert np.array_equal(flat_got[~written], flat_ref[~written])          # untouched rows keep their bits
    same = np.mean(flat_got[written] == flat_ref[written]) if written.any() else 1.0
    assert same >= 0.97                                                    # rounding ties aside, the oracle's bits


@pytest.mark.parametrize("T", [64, 19, 150])
def test_cache_append_fp8_v3(T):
    say(f"cache append fp8 T={T}")
    inp = inputs.append_inputs(90 + T, T, skip_every=7)
    nb, bs, d_c, d_r = inp["num_blocks"], inp["block_size"], 512, 64
    bb = bs * (d_c + 2 * d_r + 4)
    start = np.zeros((nb, bb), dtype=np.uint8)
    got = _append_gpu(inp, "fp8", start)
    ref = _append_oracle(inp, "fp8", start)
    c_ex, r_ex = _exact_rows(inp)
    n_code_diff = 0
    for t in range(T):
        sl = inp["slots"][t]
        if sl < 0:
            continue
        blk, row = sl // bs, sl % bs
        cg, kg = oracle.paged_rows(got, [blk], bs, "fp8", d_c, d_r, bs)
        cr, _ = oracle.paged_rows(ref, [blk], bs, "fp8", d_c, d_r, bs)
        scale = np.abs(c_ex[t]).max() / 448.0
        # within one e4m3 step of the exact content (the fp32 accumulation may
        # move a value across a rounding boundary), and the scale to fp32 precision
        step = np.maximum(np.abs(c_ex[t]) * 2.0 ** -3, 2.0 ** -9 * scale) * (1 + 1e-5)
        assert np.all(np.abs(cg[row] - c_ex[t]) <= step), t
        s_got = got[blk, bs * (d_c + 2 * d_r) + 4 * row: bs * (d_c + 2 * d_r) + 4 * row + 4].view(np.float32)[0]
        assert abs(s_got - scale) <= 1e-5 * scale
        assert np.all(np.abs(kg[row] - r_ex[t]) <= np.abs(r_ex[t]) * 2.0 ** -7 + 1e-6)
        n_code_diff += int(np.sum(got[blk, row * d_c:(row + 1) * d_c] != ref[blk, row * d_c:(row + 1) * d_c]))
    n_written = int(np.sum(inp["slots"] >= 0))
    assert n_code_diff <= 0.01 * n_written * d_c  # the same codes as the oracle except at rounding ties
    written_blocks = set(int(s) // bs for s in inp["slots"] if s >= 0)
    for blk in range(nb):
        if blk not in written_blocks:
            assert not got[blk].any()


def test_cache_append_toy_fp32_generic_then_decode():
    """fp32 toy layer (generic projection kernel): append all 256 tokens, then
    decode the last one on the GPU; equals the oracle's append + decode."""
    say("cache append toy fp32 + decode")
    W = inputs.toy_layer(seed=21, T=256)
    dm = W["dims"]
    d, d_c, d_r, n_h, d_h = dm["d"], dm["d_c"], dm["d_r"], dm["n_h"], dm["d_h"]
    T, bs = 256, 64
    perm = np.random.default_rng(22).permutation(6)[:4].astype(np.int32)
    pos = np.arange(T, dtype=np.int32)
    slots = (perm[pos // bs] * bs + pos % bs).astype(np.int32)
    w = np.concatenate([W["w_dkv"], W["w_kr"]]).astype(np.float32)
    inp = {"h": W["h"][0], "w": w, "pos": pos, "slots": slots, "d_c": d_c, "d_r": d_r, "block_size": bs,
           "dtype": "f32"}
    start = np.zeros((6, bs, d_c + d_r), dtype=np.float32)
    got = _append_gpu(inp, "f32", start)
    ref = _append_oracle(inp, "f32", start)
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    # decode the last token over the GPU-written cache
    _, _, q_c, q_r = oracle.project(W["h"], W, W["pos"])
    q_lat = oracle.absorb_q(q_c[0, -1:], W["w_uk"], n_h, d_h)
    scale = 1.0 / math.sqrt(d_h + d_r)
    o, lse = binding.decode(f32_dev(q_lat[None].astype(np.float32)), f32_dev(q_r[0, -1:][None].astype(np.float32)),
                            torch.from_numpy(got).cuda(), torch.from_numpy(perm[None]).cuda(),
                            torch.tensor([T], dtype=torch.int32).cuda(), scale, d_r=d_r, block_size=bs,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    c, kr = oracle.paged_rows(ref, perm, T, "f32", d_c, d_r, bs)
    o_ref, lse_ref = oracle.mqa_decode_rows(q_lat, q_r[0, -1:], c, kr, scale)
    assert_f32_close(o.cpu().numpy()[0].astype(np.float64), o_ref, "o_lat", tol=1e-5)
    assert np.max(np.abs(lse.cpu().numpy()[0] - lse_ref)) <= 1e-5


# ------------------------------------------------------------------ MHA-mode prefill

def _pf_dev(inp, *keys):
    conv = bf16_dev if inp["dtype"] == "bf16" else f32_dev
    return [conv(inp[k]) for k in keys]


def _pf_dec(inp, *keys):
    dec = oracle.bf16_to_f64 if inp["dtype"] == "bf16" else (lambda a: np.asarray(a, np.float64))
    return [dec(inp[k]) for k in keys]


def _pf_oracle(inp, heads=None):
    q, k_c, v_c, k_r = _pf_dec(inp, "q", "k_c", "v_c", "k_r")
    if heads is not None:
        q, k_c, v_c = q[:, heads], k_c[:, heads], v_c[:, heads]
    d_h = inp["d_h"]
    return oracle.mha_attention(q[..., :d_h], q[..., d_h:], k_c, k_r, v_c, inp["scale"])


@pytest.mark.parametrize("T", [1, 37, 128, 300])
def test_prefill_mha_bf16_v3(T):
    """MFMA kernel (d_h 128, d_r 64, 128 heads) against the oracle: one query
    block, ragged tails, several causal subtiles."""
    say(f"prefill bf16 T={T}")
    inp = inputs.prefill_inputs(110 + T, T)
    q, k_c, k_r, v_c = _pf_dev(inp, "q", "k_c", "k_r", "v_c")
    o, lse = binding.prefill_mha(q, k_c, k_r, v_c, inp["scale"], out_dtype=torch.float32)
    o16, _ = binding.prefill_mha(q, k_c, k_r, v_c, inp["scale"], with_lse=False)
    torch.cuda.synchronize()
    ref_o, ref_lse = _pf_oracle(inp)
    g = o.cpu().numpy().astype(np.float64)
    assert_bf16_close(g, ref_o, f"prefill T={T}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, "prefill lse")
    # bf16 output: the fp32 result rounded once more
    assert_bf16_close(o16.float().cpu().numpy().astype(np.float64), ref_o, "prefill bf16 out")
    if T == 1:  # one visible key: the output is that key's value row (p = 1 up to fp32 rounding)
        v0 = oracle.bf16_to_f64(inp["v_c"])[0]
        assert np.all(np.abs(g[0] - v0) <= 1e-6 * np.abs(v0))


def test_prefill_mha_bf16_rising_scores():
    """Causal prefill with scores that climb in steps along the keys (the
    staircase of the decode test on k^R dimension 0, query RoPE dimension 0
    = 1, the other query dimensions scaled by 1/4): every query block's
    reference max has to move as the key stream enters each new level."""
    say("prefill bf16 stepped scores")
    T, at = 300, [40, 100, 170, 260, 290]
    inp = inputs.prefill_inputs(131, T, n_h=16, d_c=64)
    d_h = inp["d_h"]
    kr = inputs.bf16_bits_as_f32(inp["k_r"])
    kr[:, 0] += _stair(T, at)
    inp["k_r"] = inputs.f32_to_bf16_bits(kr)
    q = inputs.bf16_bits_as_f32(inp["q"]) * np.float32(0.25)
    q[..., d_h] = 1.0
    inp["q"] = inputs.f32_to_bf16_bits(q)
    q_, k_c, k_r, v_c = _pf_dev(inp, "q", "k_c", "k_r", "v_c")
    o, lse = binding.prefill_mha(q_, k_c, k_r, v_c, inp["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_o, ref_lse = _pf_oracle(inp)
    assert_bf16_close(o.cpu().numpy().astype(np.float64), ref_o, "prefill stepped")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, "prefill stepped lse")


@pytest.mark.parametrize("T,n_h", [(200, 3), (129, 9)])
def test_prefill_mha_bf16_head_counts_off_the_xcd_multiple(T, n_h):
    """MFMA kernel with head counts that are not a multiple of the 8 XCDs
    (the grid is padded; the extra workgroups return)."""
    say(f"prefill bf16 T={T} n_h={n_h}")
    inp = inputs.prefill_inputs(120 + n_h, T, n_h=n_h, d_c=64)
    q, k_c, k_r, v_c = _pf_dev(inp, "q", "k_c", "k_r", "v_c")
    o, lse = binding.prefill_mha(q, k_c, k_r, v_c, inp["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_o, ref_lse = _pf_oracle(inp)
    assert_bf16_close(o.cpu().numpy().astype(np.float64), ref_o, f"prefill T={T} n_h={n_h}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, "prefill lse")


def test_prefill_mha_full_size_sampled_heads():
    """4096-token prefill at V3 heads; the oracle checks every query of 3 heads
    (first, middle, last) and the rest is checked to be finite."""
    T = 4096
    say(f"prefill bf16 T={T} sampled heads")
    inp = inputs.prefill_inputs(131, T)
    q, k_c, k_r, v_c = _pf_dev(inp, "q", "k_c", "k_r", "v_c")
    o, lse = binding.prefill_mha(q, k_c, k_r, v_c, inp["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = [0, 77, 127]
    g = o.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g))
    ref_o, ref_lse = _pf_oracle(inp, heads)
    assert_bf16_close(g[:, heads], ref_o, "prefill 4096 sampled")
    assert_lse_close(lse.cpu().numpy().astype(np.float64)[:, heads], ref_lse, "prefill 4096 lse")


@pytest.mark.parametrize("T,n_h,d_h,d_r", [(1, 2, 64, 32), (50, 3, 64, 32), (70, 2, 128, 64), (33, 1, 192, 64)])
def test_prefill_mha_fp32_generic(T, n_h, d_h, d_r):
    """fp32 inputs (portable kernel) at toy and odd head sizes."""
    say(f"prefill fp32 T={T} n_h={n_h} d_h={d_h} d_r={d_r}")
    inp = inputs.prefill_inputs(150 + T, T, n_h=n_h, d_h=d_h, d_r=d_r, d_c=64, dtype="f32")
    q, k_c, k_r, v_c = _pf_dev(inp, "q", "k_c", "k_r", "v_c")
    o, lse = binding.prefill_mha(q, k_c, k_r, v_c, inp["scale"])
    torch.cuda.synchronize()
    ref_o, ref_lse = _pf_oracle(inp)
    assert_f32_close(o.cpu().numpy().astype(np.float64), ref_o, "prefill fp32", tol=1e-5)
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-5


def test_prefill_mfma_matches_generic_on_bf16():
    """Same bf16 inputs through both kernels (the portable one takes a
    misaligned view of the same values)."""
    T = 200
    say("prefill mfma vs generic")
    inp = inputs.prefill_inputs(171, T)
    q, k_c, k_r, v_c = _pf_dev(inp, "q", "k_c", "k_r", "v_c")
    o1, l1 = binding.prefill_mha(q, k_c, k_r, v_c, inp["scale"], out_dtype=torch.float32)
    # shift k_r by one element inside a larger buffer: no longer 16-byte aligned
    buf = torch.empty(k_r.numel() + 1, dtype=k_r.dtype, device=k_r.device)
    buf[1:] = k_r.reshape(-1)
    k_r_mis = buf[1:].view(k_r.shape)
    o2, l2 = binding.prefill_mha(q, k_c, k_r_mis, v_c, inp["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    a, b = o1.cpu().numpy().astype(np.float64), o2.cpu().numpy().astype(np.float64)
    assert_bf16_close(a, b, "mfma vs generic")
    assert np.max(np.abs(l1.cpu().numpy() - l2.cpu().numpy())) <= 1e-3


@pytest.mark.parametrize("T", [1, 45, 300])
def test_expand_kv_bf16_v3(T):
    say(f"expand_kv bf16 T={T}")
    inp = inputs.prefill_inputs(190 + T, T)
    c_kv, w_uk, w_uv = _pf_dev(inp, "c_kv", "w_uk", "w_uv")
    k_c, v_c = binding.expand_kv(c_kv, w_uk, w_uv, 128, out_dtype=torch.float32)
    k16, v16 = binding.expand_kv(c_kv, w_uk, w_uv, 128)
    torch.cuda.synchronize()
    rk, rv = oracle.expand_kv(*_pf_dec(inp, "c_kv", "w_uk", "w_uv"), 128, 128)
    # bf16 inputs, fp32 accumulation over d_c = 512 terms
    assert_f32_close(k_c.cpu().numpy().astype(np.float64), rk, "k_c", tol=1e-5)
    assert_f32_close(v_c.cpu().numpy().astype(np.float64), rv, "v_c", tol=1e-5)
    assert_bf16_close(k16.float().cpu().numpy().astype(np.float64), rk, "k_c bf16")
    assert_bf16_close(v16.float().cpu().numpy().astype(np.float64), rv, "v_c bf16")


@pytest.mark.parametrize("T,n_h,d_c", [(1100, 128, 512), (4500, 16, 64)])
def test_expand_kv_bf16_several_tiles_per_workgroup(T, n_h, d_c):
    """More 256 x 256 output tiles than compute units, so each persistent
    workgroup streams several tiles with its k-slice ring running on across
    tile boundaries; d_c = 64 gives two k slices per tile, fewer than the
    ring's four slots.  T is off the tile (ragged last tile)."""
    say(f"expand_kv bf16 several tiles T={T} n_h={n_h} d_c={d_c}")
    inp = inputs.prefill_inputs(230 + T, T, n_h=n_h, d_c=d_c)
    c_kv, w_uk, w_uv = _pf_dev(inp, "c_kv", "w_uk", "w_uv")
    k_c, v_c = binding.expand_kv(c_kv, w_uk, w_uv, 128, out_dtype=torch.float32)
    k16, v16 = binding.expand_kv(c_kv, w_uk, w_uv, 128)
    torch.cuda.synchronize()
    rk, rv = oracle.expand_kv(*_pf_dec(inp, "c_kv", "w_uk", "w_uv"), n_h, 128)
    assert_f32_close(k_c.cpu().numpy().astype(np.float64), rk, "k_c", tol=1e-5)
    assert_f32_close(v_c.cpu().numpy().astype(np.float64), rv, "v_c", tol=1e-5)
    assert_bf16_close(k16.float().cpu().numpy().astype(np.float64), rk, "k_c bf16")
    assert_bf16_close(v16.float().cpu().numpy().astype(np.float64), rv, "v_c bf16")


def test_expand_kv_bf16_full_size_sampled():
    """The benchmarked size (4096 tokens, 128 heads of 128, d_c = 512) in the
    launch configuration the benchmark times; the oracle computes 96 sampled
    tokens (rows are independent)."""
    T = 4096
    say("expand_kv bf16 T=4096 sampled")
    inp = inputs.prefill_inputs(250, T)
    c_kv, w_uk, w_uv = _pf_dev(inp, "c_kv", "w_uk", "w_uv")
    k16, v16 = binding.expand_kv(c_kv, w_uk, w_uv, 128)
    torch.cuda.synchronize()
    rows = np.sort(np.random.Generator(np.random.PCG64(251)).choice(T, 96, replace=False))
    rows[-1] = T - 1
    c_np, wk_np, wv_np = _pf_dec(inp, "c_kv", "w_uk", "w_uv")
    rk, rv = oracle.expand_kv(c_np[rows], wk_np, wv_np, 128, 128)
    got_k = k16.float().cpu().numpy().astype(np.float64)[rows]
    got_v = v16.float().cpu().numpy().astype(np.float64)[rows]
    assert_bf16_close(got_k, rk, "k_c bf16")
    assert_bf16_close(got_v, rv, "v_c bf16")


def test_expand_kv_bf16_heads_off_the_gemm_tile():
    """n_h * d_h = 192 is not a multiple of the GEMM's 256-row tile: the
    expansion takes the per-head up-projection kernel (shared latent row)."""
    T, n_h, d_h, d_c = 70, 3, 64, 128
    say("expand_kv bf16 small heads")
    inp = inputs.prefill_inputs(211, T, n_h=n_h, d_h=d_h, d_r=32, d_c=d_c)
    c_kv, w_uk, w_uv = _pf_dev(inp, "c_kv", "w_uk", "w_uv")
    k_c, v_c = binding.expand_kv(c_kv, w_uk, w_uv, d_h, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rk, rv = oracle.expand_kv(*_pf_dec(inp, "c_kv", "w_uk", "w_uv"), n_h, d_h)
    assert_f32_close(k_c.cpu().numpy().astype(np.float64), rk, "k_c", tol=1e-5)
    assert_f32_close(v_c.cpu().numpy().astype(np.float64), rv, "v_c", tol=1e-5)


def test_expand_then_prefill_toy_fp32_layer():
    """fp32 toy layer in MHA mode, every step on the GPU: latent -> expand_kv ->
    prefill, against the oracle's MHA-mode layer output o (before W^O)."""
    say("toy fp32 expand + prefill")
    W = inputs.toy_layer(seed=5, B=1, T=256)
    dm = W["dims"]
    n_h, d_h, d_r = dm["n_h"], dm["d_h"], dm["d_r"]
    ref = oracle.mha_mode_layer(W["h"], W, W["pos"])
    c_kv = f32_dev(ref["c_kv"][0])
    k_c, v_c = binding.expand_kv(c_kv, f32_dev(W["w_uk"]), f32_dev(W["w_uv"]), d_h)
    q = f32_dev(np.concatenate([ref["q_c"][0], ref["q_r"][0]], -1))
    o, lse = binding.prefill_mha(q, k_c, v_c=v_c, k_r=f32_dev(ref["k_r"][0]),
                                 softmax_scale=1.0 / math.sqrt(d_h + d_r))
    torch.cuda.synchronize()
    assert_f32_close(o.cpu().numpy().astype(np.float64), ref["o"][0], "toy layer o", tol=1e-5)
    assert np.max(np.abs(lse.cpu().numpy() - ref["lse"][0])) <= 1e-5


# ------------------------------------------------------------------ GQLA GQA path

def _gqa_gpu(case, force_generic=False, out_dtype=torch.float32):
    conv = bf16_dev if case.q_dtype == "bf16" else f32_dev
    cache = bf16_dev(case.cache) if case.kv_dtype == "bf16" else f32_dev(case.cache)
    table = torch.from_numpy(np.maximum(case.block_table, 0).astype(np.int32)).cuda()
    lens = torch.from_numpy(case.seq_lens.astype(np.int32)).cuda()
    o, lse = binding.gqa_decode(conv(case.q_c), conv(case.q_r), cache, table, lens, case.n_g, case.softmax_scale,
                                block_size=case.block_size, out_dtype=out_dtype, force_generic=force_generic)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _gqa_oracle(case, seqs=None):
    dec = oracle.bf16_to_f64 if case.q_dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
    outs, lses = [], []
    for b in (range(case.B) if seqs is None else seqs):
        L = int(case.seq_lens[b])
        k_c, v_c, k_r = oracle.gqa_paged_rows(case.cache, case.block_table[b], L, case.n_g, case.d_h, case.d_r,
                                              case.block_size, case.kv_dtype)
        o, l = oracle.gqa_decode_rows(dec(case.q_c[b]), dec(case.q_r[b]), k_c, v_c, k_r, case.softmax_scale, case.n_g)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("force_generic", [False, True])
@pytest.mark.parametrize("s_q,n_g,lens", [(2, 8, [2, 33, 64, 129, 1500, 300, 7, 4096]),
                                          (1, 4, [1, 95, 2048])])
def test_gqa_decode_bf16_v3(s_q, n_g, lens, force_generic):
    """GQA path at V3 heads (128 heads, d_h 128, d_r 64): 8 groups with two
    new tokens (MTP) and 4 groups with one, ragged lengths; the second case
    has a workgroup count off the multiple of 8 (plain dealing)."""
    say(f"gqa bf16 s_q={s_q} n_g={n_g} generic={force_generic}")
    case = inputs.gqa_case(40 + s_q, B=len(lens), seq_lens=np.array(lens), s_q=s_q, n_g=n_g)
    g, gl = _gqa_gpu(case, force_generic)
    o, ol = _gqa_oracle(case)
    assert_bf16_close(g, o, "gqa o")
    assert_lse_close(gl, ol, "gqa lse")
    g16, _ = _gqa_gpu(case, force_generic, out_dtype=torch.bfloat16)
    assert_bf16_close(g16, o, "gqa o bf16")


@pytest.mark.parametrize("force_generic", [False, True])
def test_gqa_decode_bf16_nan_tails(force_generic):
    """GQA path: the unused rows of each sequence's last block (every group's
    k^C and v^C rows and the shared k^R rows) hold NaN; nothing of them may
    reach the result."""
    say(f"gqa bf16 nan tails generic={force_generic}")
    lens = np.array([2, 33, 63, 65, 130, 1029], dtype=np.int32)
    case = inputs.gqa_case(48, B=len(lens), seq_lens=lens, s_q=2, n_g=8)
    bs, n_g, d_h, d_r = case.block_size, case.n_g, case.d_h, case.d_r
    for b, L in enumerate(lens):
        used = int(L) - (int(L) - 1) // bs * bs
        if used == bs:
            continue
        blk = case.cache[case.block_table[b, (int(L) - 1) // bs]]
        kv = blk[: 2 * n_g * bs * d_h].reshape(2 * n_g, bs, d_h)
        kv[:, used:] = 0x7FC0
        blk[2 * n_g * bs * d_h:].reshape(bs, d_r)[used:] = 0x7FC0
    g, gl = _gqa_gpu(case, force_generic)
    o, ol = _gqa_oracle(case)
    assert_bf16_close(g, o, "gqa nan tails o")
    assert_lse_close(gl, ol, "gqa nan tails lse")


@pytest.mark.parametrize("force_generic", [False, True])
def test_gqa_decode_bf16_rising_scores(force_generic):
    """GQA path with the decode test's stepped scores (k^R dimension 0 of each
    cached row raised by the staircase, query RoPE dimension 0 = 1, the other
    query dimensions scaled by 1/4), two new tokens."""
    say(f"gqa bf16 stepped scores generic={force_generic}")
    case = inputs.gqa_case(47, B=len(STEP_LENS), seq_lens=STEP_LENS, s_q=2, n_g=8)
    bs, off = case.block_size, 2 * case.n_g * case.block_size * case.d_h
    vals = inputs.bf16_bits_as_f32(case.cache)
    for b, (n, at) in enumerate(zip(STEP_LENS, STEP_AT)):
        pos = np.arange(n)
        vals[case.block_table[b, pos // bs], off + (pos % bs) * case.d_r] += _stair(n, at)
    case.cache = inputs.f32_to_bf16_bits(vals)
    case.q_c = inputs.f32_to_bf16_bits(inputs.bf16_bits_as_f32(case.q_c) * np.float32(0.25))
    qr = inputs.bf16_bits_as_f32(case.q_r) * np.float32(0.25)
    qr[..., 0] = 1.0
    case.q_r = inputs.f32_to_bf16_bits(qr)
    g, gl = _gqa_gpu(case, force_generic)
    o, ol = _gqa_oracle(case)
    assert_bf16_close(g, o, "gqa stepped o")
    assert_lse_close(gl, ol, "gqa stepped lse")


@pytest.mark.parametrize("seed", range(4))
def test_gqa_decode_randomized_configurations(seed):
    """GQA path on seeded random configurations: groups and new tokens drawn
    from the MFMA kernel's (16 heads x 2 tokens, 32 x 1, 8 x 4) and other
    combinations (portable kernel), random batch and log-uniform lengths."""
    rng = np.random.default_rng(1100 + seed)
    n_g, s_q = [(8, 2), (4, 1), (16, 4), (8, 1)][seed]
    B = int(rng.integers(1, 7))
    lens = np.maximum(np.exp(rng.uniform(np.log(s_q), np.log(5000), size=B)).astype(np.int32), s_q)
    say(f"random gqa seed={seed}: n_g={n_g} s_q={s_q} B={B} lens={lens.tolist()}")
    case = inputs.gqa_case(1110 + seed, B=B, seq_lens=lens, s_q=s_q, n_g=n_g)
    g, gl = _gqa_gpu(case)
    o, ol = _gqa_oracle(case)
    assert_bf16_close(g, o, f"random gqa seed={seed}")
    assert_lse_close(gl, ol, "lse")


def test_gqa_decode_bf16_four_tokens_of_eight_heads():
    """16 groups of 8 heads with s_q = 4: the MFMA kernel's 32 rows are four
    query tokens of eight heads (causal among the four)."""
    say("gqa bf16 s_q=4 n_g=16")
    case = inputs.gqa_case(43, B=4, seq_lens=np.array([4, 37, 300, 1029]), s_q=4, n_g=16)
    g, gl = _gqa_gpu(case)
    o, ol = _gqa_oracle(case)
    assert_bf16_close(g, o, "gqa s_q=4")
    assert_lse_close(gl, ol, "gqa s_q=4 lse")


def test_gqa_decode_full_size_sampled():
    """16 sequences of 8192 tokens, 8 groups, s_q = 2 (the MFMA kernel's
    launch shape at full length); the oracle checks 3 sequences."""
    say("gqa bf16 B=16 L=8192 sampled")
    case = inputs.gqa_case(44, B=16, seq_lens=8192, s_q=2, n_g=8)
    g, gl = _gqa_gpu(case)
    assert np.all(np.isfinite(g))
    seqs = [0, 7, 15]
    o, ol = _gqa_oracle(case, seqs)
    assert_bf16_close(g[seqs], o, "gqa 8192 sampled")
    assert_lse_close(gl[seqs], ol, "gqa 8192 lse")


def test_gqa_decode_fp32_toy():
    """fp32 toy shapes (8 heads in 2 groups, d_h 64, d_r 32, 16-token blocks):
    the portable kernel to the fp32 bar."""
    say("gqa fp32 toy")
    case = inputs.gqa_case(46, B=3, seq_lens=np.array([2, 40, 77]), s_q=2, n_h=8, n_g=2, d_h=64, d_r=32,
                           kv_dtype="f32", q_dtype="f32", block_size=16)
    g, gl = _gqa_gpu(case)
    o, ol = _gqa_oracle(case)
    assert_f32_close(g, o, "gqa fp32")
    assert np.max(np.abs(gl - ol)) <= 1e-5


def test_gqa_path_equals_absorbed_decode_on_gpu():
    """The same GQLA weights through both GPU paths: expand the latent per
    group (mla_expand_kv), page it, decode on the GQA path; absorb W^UK_g per
    head, decode the latent on the MQA path, apply W^UV_g.  Both agree with
    each other within the bf16 bar."""
    say("gqla two paths on the GPU")
    n_h, n_g, d_h, d_c, d_r, s_q, L = 128, 8, 128, 512, 64, 2, 256
    rng = np.random.Generator(np.random.PCG64(48))
    c = inputs.f32_to_bf16_bits(rng.standard_normal((L, d_c), dtype=np.float32))
    kr = inputs.f32_to_bf16_bits(rng.standard_normal((L, d_r), dtype=np.float32))
    w_uk = inputs.f32_to_bf16_bits(rng.standard_normal((n_g * d_h, d_c), dtype=np.float32) / np.float32(d_c ** 0.5))
    w_uv = inputs.f32_to_bf16_bits(rng.standard_normal((n_g * d_h, d_c), dtype=np.float32) / np.float32(d_c ** 0.5))
    q_c = inputs.f32_to_bf16_bits(rng.standard_normal((1, s_q, n_h, d_h), dtype=np.float32))
    q_r = inputs.f32_to_bf16_bits(rng.standard_normal((1, s_q, n_h, d_r), dtype=np.float32))
    scale = 1.0 / math.sqrt(d_h + d_r)
    # GQA path: expand per group, lay out the pages [n_g][64][d_h] k | [n_g][64][d_h] v | [64][d_r] k^R
    k_c, v_c = binding.expand_kv(bf16_dev(c), bf16_dev(w_uk), bf16_dev(w_uv), d_h)      # [L, n_g, d_h] bf16
    nb = L // 64
    kg = k_c.view(nb, 64, n_g, d_h).permute(0, 2, 1, 3).reshape(nb, -1)
    vg = v_c.view(nb, 64, n_g, d_h).permute(0, 2, 1, 3).reshape(nb, -1)
    cache = torch.cat([kg, vg, bf16_dev(kr).view(nb, -1)], 1).contiguous()
    table = torch.arange(nb, dtype=torch.int32, device="cuda")[None]
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    o_gqa, l_gqa = binding.gqa_decode(bf16_dev(q_c), bf16_dev(q_r), cache, table, lens, n_g, scale,
                                      out_dtype=torch.float32)
    # MQA-absorb path with the group's weights repeated per head
    w_uk_h = bf16_dev(w_uk).view(n_g, 1, d_h, d_c).expand(n_g, n_h // n_g, d_h, d_c).reshape(n_h * d_h, d_c)
    w_uv_h = bf16_dev(w_uv).view(n_g, 1, d_h, d_c).expand(n_g, n_h // n_g, d_h, d_c).reshape(n_h * d_h, d_c)
    q_lat = binding.absorb_q(bf16_dev(q_c).view(s_q, n_h, d_h), w_uk_h.contiguous())
    lat_cache = torch.cat([bf16_dev(c), bf16_dev(kr)], 1).view(nb, 64, d_c + d_r).contiguous()
    o_lat, l_mqa = binding.decode(q_lat.view(1, s_q, n_h, d_c), bf16_dev(q_r), lat_cache, table, lens, scale,
                                  out_dtype=torch.bfloat16)
    o_mqa = binding.up_proj_v(o_lat.view(s_q, n_h, d_c), w_uv_h.contiguous(), d_h, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a = o_gqa.cpu().numpy().astype(np.float64).reshape(s_q, n_h, d_h)
    b = o_mqa.cpu().numpy().astype(np.float64).reshape(s_q, n_h, d_h)
    assert_bf16_close(a, b, "gqa vs absorbed")
    assert np.max(np.abs(l_gqa.cpu().numpy() - l_mqa.cpu().numpy())) <= 0.05


# ------------------------------------------------------------------ fused decode step

@pytest.mark.parametrize("kv,lens,s_q,splits", [("bf16", [2, 33, 64, 129, 1500], 1, 0),
                                                ("bf16", [70, 4096, 9], 2, 3),
                                                ("fp8", [2, 700, 2048], 2, 0),
                                                ("int4", [64, 1000], 1, 1),
                                                ("bf16", [9000, 300], 1, 13)])
def test_decode_step_matches_separate_calls_and_oracle(kv, lens, s_q, splits):
    """mla_decode_step (absorb, attention, merge fused with W^UV) against the
    oracle's absorbed layer on the same rounded inputs, and equal to the three
    separate calls (which also store o_lat in bf16)."""
    say(f"decode step {kv} s_q={s_q} splits={splits}")
    lens = np.array(lens, dtype=np.int32)
    case = inputs.decode_case(60 + s_q, B=len(lens), seq_lens=lens, s_q=s_q, kv_dtype=kv, **V3)
    T_q = case.B * s_q
    P = inputs.projection_weights(61, T_q=T_q)
    d = case_to_device(case)
    qn, wuk, wuv = bf16_dev(P["q_c"]).view(case.B, s_q, 128, 128), bf16_dev(P["w_uk"]), bf16_dev(P["w_uv"])
    o, lse = binding.decode_step(qn, wuk, d["q_rope"], d["kv_cache"], d["block_table"], d["seq_lens"], wuv,
                                 d["softmax_scale"], kv_dtype=d["kv_dtype"], num_splits=splits)
    # the same step through the separate entry points
    q_lat = binding.absorb_q(qn.view(T_q, 128, 128), wuk)
    o_lat, lse2 = binding.decode(q_lat.view(case.B, s_q, 128, 512), d["q_rope"], d["kv_cache"], d["block_table"],
                                 d["seq_lens"], d["softmax_scale"], kv_dtype=d["kv_dtype"], num_splits=splits)
    o2 = binding.up_proj_v(o_lat.view(T_q, 128, 512), wuv, 128)
    torch.cuda.synchronize()
    g = o.float().cpu().numpy().astype(np.float64).reshape(T_q, 128, 128)
    g2 = o2.float().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g - g2)) <= 2e-2 * max(1.0, np.max(np.abs(g2)))
    assert np.max(np.abs(lse.cpu().numpy() - lse2.cpu().numpy())) <= 1e-6
    # oracle: absorbed decode on the bf16-rounded inputs, then W^UV; the step
    # stores q_lat in bf16 (its operand type), so the oracle decodes with the
    # exact q_lat rounded to bf16
    ql = oracle.absorb_q(oracle.bf16_to_f64(P["q_c"]), oracle.bf16_to_f64(P["w_uk"]), 128, 128)
    ql = oracle.bf16_to_f64(oracle.bf16_round_bits(ql)).reshape(case.B, s_q, 128, 512)
    ref_o, ref_l = [], []
    for b in range(case.B):
        _, qr, c, kr = oracle.decode_case_rows(case, b)
        ol, l = oracle.mqa_decode_rows(ql[b], qr, c, kr, case.softmax_scale)
        ref_o.append(oracle.up_proj_v(ol, oracle.bf16_to_f64(P["w_uv"]), 128, 128))
        ref_l.append(l)
    ref_o = np.stack(ref_o).reshape(T_q, 128, 128)
    assert_bf16_close(g, ref_o, f"step {kv}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).reshape(case.B, s_q, 128), np.stack(ref_l), "step lse")


@pytest.mark.parametrize("seed", range(4))
def test_decode_step_randomized_configurations(seed):
    """mla_decode_step on seeded random configurations (cache format, s_q,
    batch, log-uniform lengths, splits) against the oracle's absorbed layer."""
    rng = np.random.default_rng(970 + seed)
    kv = ["bf16", "fp8", "int4", "int2"][seed]
    s_q = int(rng.integers(1, 3))
    B = int(rng.integers(1, 9))
    lens = np.maximum(np.exp(rng.uniform(np.log(s_q), np.log(6000), size=B)).astype(np.int32), s_q)
    splits = int(rng.choice([0, 2, 7]))
    say(f"random step seed={seed}: {kv} s_q={s_q} B={B} lens={lens.tolist()} splits={splits}")
    case = inputs.decode_case(980 + seed, B=B, seq_lens=lens, s_q=s_q, kv_dtype=kv, tail_fill="nan", **V3)
    T_q = B * s_q
    P = inputs.projection_weights(990 + seed, T_q=T_q)
    d = case_to_device(case)
    qn = bf16_dev(P["q_c"]).view(B, s_q, 128, 128)
    o, lse = binding.decode_step(qn, bf16_dev(P["w_uk"]), d["q_rope"], d["kv_cache"], d["block_table"],
                                 d["seq_lens"], bf16_dev(P["w_uv"]), d["softmax_scale"], kv_dtype=d["kv_dtype"],
                                 num_splits=splits)
    torch.cuda.synchronize()
    g = o.float().cpu().numpy().astype(np.float64).reshape(T_q, 128, 128)
    ql = oracle.absorb_q(oracle.bf16_to_f64(P["q_c"]), oracle.bf16_to_f64(P["w_uk"]), 128, 128)
    ql = oracle.bf16_to_f64(oracle.bf16_round_bits(ql)).reshape(B, s_q, 128, 512)
    ref_o, ref_l = [], []
    for b in range(B):
        _, qr, c, kr = oracle.decode_case_rows(case, b)
        ol, l = oracle.mqa_decode_rows(ql[b], qr, c, kr, case.softmax_scale)
        ref_o.append(oracle.up_proj_v(ol, oracle.bf16_to_f64(P["w_uv"]), 128, 128))
        ref_l.append(l)
    assert_bf16_close(g, np.stack(ref_o).reshape(T_q, 128, 128), f"random step seed={seed}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64).reshape(B, s_q, 128), np.stack(ref_l), "lse")


@pytest.mark.parametrize("seed", range(4))
def test_prefill_mha_randomized_shapes(seed):
    """MHA-mode prefill (MFMA kernel) on seeded random lengths and head
    counts against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(1, 700))
    n_h = int(rng.integers(1, 20))
    say(f"random prefill seed={seed}: T={T} n_h={n_h}")
    inp = inputs.prefill_inputs(1010 + seed, T, n_h=n_h, d_c=64)
    q, k_c, k_r, v_c = _pf_dev(inp, "q", "k_c", "k_r", "v_c")
    o, lse = binding.prefill_mha(q, k_c, k_r, v_c, inp["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_o, ref_lse = _pf_oracle(inp)
    assert_bf16_close(o.cpu().numpy().astype(np.float64), ref_o, f"random prefill seed={seed}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, "lse")


@pytest.mark.parametrize("kv,lens,splits", [("bf16", [2, 33, 1500, 4096], 0), ("fp8", [700, 64], 2)])
def test_decode_step_stages_equal_the_whole_step(kv, lens, splits):
    """mla_decode_step_stages run one stage per call (on one workspace, with
    the caller's own events between the calls) gives the bytes of the
    single mla_decode_step call, and the attention stage's events bracket
    that one launch."""
    say(f"decode step stages {kv} splits={splits}")
    lens = np.array(lens, dtype=np.int32)
    case = inputs.decode_case(64, B=len(lens), seq_lens=lens, s_q=1, kv_dtype=kv, **V3)
    P = inputs.projection_weights(65, T_q=case.B)
    d = case_to_device(case)
    qn, wuk, wuv = bf16_dev(P["q_c"]).view(case.B, 1, 128, 128), bf16_dev(P["w_uk"]), bf16_dev(P["w_uv"])
    args = (qn, wuk, d["q_rope"], d["kv_cache"], d["block_table"], d["seq_lens"], wuv, d["softmax_scale"])
    kw = dict(kv_dtype=d["kv_dtype"], num_splits=splits)
    o, lse = binding.decode_step(*args, **kw)
    ws = binding.decode_step_workspace(case.B, 1, 128, 512, d["block_table"].shape[1], splits)
    ws.fill_(0xff)  # nothing carried over from an earlier call
    o2 = torch.full_like(o, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for st in (binding.MLA_STAGE_ABSORB, binding.MLA_STAGE_ATTEND, binding.MLA_STAGE_MERGE):
        if st == binding.MLA_STAGE_ATTEND:
            e0.record()
        binding.decode_step_stages(st, *args, workspace=ws, out=o2, lse=lse2, **kw)
        if st == binding.MLA_STAGE_ATTEND:
            e1.record()
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)
    assert e0.elapsed_time(e1) > 0.0
    # two stages in one call, then the third
    o3 = torch.full_like(o, float("nan"))
    binding.decode_step_stages(binding.MLA_STAGE_ABSORB | binding.MLA_STAGE_ATTEND, *args, workspace=ws, out=o3,
                               lse=lse2, **kw)
    binding.decode_step_stages(binding.MLA_STAGE_MERGE, *args, workspace=ws, out=o3, lse=lse2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o3.view(torch.int16))


def test_decode_step_stages_without_a_plan_stay_in_bounds():
    """The attention and merge stages on a workspace that holds no plan of
    this batch (all bytes 0x7f or 0x80: huge or negative unit counts and
    entries) skip every entry outside the call's shapes: the calls finish,
    and a full step on the same workspace afterwards is correct."""
    say("decode step stages on a workspace without a plan")
    lens = np.array([100, 2000], dtype=np.int32)
    case = inputs.decode_case(66, B=2, seq_lens=lens, s_q=1, **V3)
    P = inputs.projection_weights(67, T_q=case.B)
    d = case_to_device(case)
    qn, wuk, wuv = bf16_dev(P["q_c"]).view(case.B, 1, 128, 128), bf16_dev(P["w_uk"]), bf16_dev(P["w_uv"])
    args = (qn, wuk, d["q_rope"], d["kv_cache"], d["block_table"], d["seq_lens"], wuv, d["softmax_scale"])
    ref, ref_l = binding.decode_step(*args, kv_dtype=d["kv_dtype"])
    ws = binding.decode_step_workspace(case.B, 1, 128, 512, d["block_table"].shape[1], 0)
    out = torch.empty_like(ref)
    for fill in (0x7f, 0x80):
        ws.fill_(fill)
        binding.decode_step_stages(binding.MLA_STAGE_ATTEND | binding.MLA_STAGE_MERGE, *args, workspace=ws,
                                   out=out, kv_dtype=d["kv_dtype"])
        torch.cuda.synchronize()
    binding.decode_step(*args, kv_dtype=d["kv_dtype"], workspace=ws, out=out)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
