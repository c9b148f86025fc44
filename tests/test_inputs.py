"""Seeded input generators: reproducibility, structure, storage rounding."""

import numpy as np
import torch

from mla_latent_kv_05_amd import inputs


def test_seed_reproducible():
    a = inputs.decode_case(5, B=3, seq_lens=np.array([65, 1, 128]), n_h=4)
    b = inputs.decode_case(5, B=3, seq_lens=np.array([65, 1, 128]), n_h=4)
    assert np.array_equal(a.cache, b.cache) and np.array_equal(a.block_table, b.block_table)
    assert np.array_equal(a.q_lat, b.q_lat)


def test_block_table_is_permutation():
    c = inputs.decode_case(1, B=5, seq_lens=np.array([1, 64, 65, 200, 7]), n_h=2, d_c=8, d_r=4)
    nblk = (c.seq_lens + 63) // 64
    used = np.concatenate([c.block_table[b, :nblk[b]] for b in range(5)])
    assert sorted(used.tolist()) == list(range(c.num_blocks))
    for b in range(5):
        assert np.all(c.block_table[b, nblk[b]:] == -1)


def test_loguniform_lengths_in_range():
    lens = inputs.workload_lengths("v3_bf16_B128_ctxlogU128-32768")
    assert lens.shape == (128,) and lens.min() >= 128 and lens.max() <= 32768
    assert np.log(lens).std() > 0.8       # spread over the log range


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 65504.0]   # ties
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_encoder_matches_torch():
    x = np.random.default_rng(1).standard_normal(50000) * 100
    x = np.clip(x, -448, 448)
    x[:6] = [0.0, 2 ** -10, 3 * 2 ** -10, 448.0, -448.0, 2 ** -9 * 1.5]
    ours = inputs.encode_e4m3fn(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch rounds from float32; compare where the float32 value is exact
    exact = x.astype(np.float32).astype(np.float64) == x
    assert np.array_equal(ours[exact], ref[exact])
    # the bulk path used for large caches agrees on every float32 input
    x32 = x.astype(np.float32)
    assert np.array_equal(inputs.encode_e4m3fn_fast(x32), inputs.encode_e4m3fn(x32.astype(np.float64)))


def test_workload_shapes():
    c = inputs.workload_case("v3_bf16_B64_ctx8192", B=2, L=256)
    assert c.cache.shape == (8, 64, 576) and c.cache.dtype == np.uint16
    assert c.q_lat.shape == (2, 1, 128, 512) and c.q_rope.shape == (2, 1, 128, 64)
    f = inputs.workload_case("v3_fp8_B64_ctx16384_sq2", B=2, L=128)
    assert f.cache.shape == (4, 64 * 644) and f.s_q == 2
    assert f.latent_bytes == 2 * 128 * 644


def test_nan_tail_poisons_only_the_unused_rows():
    """tail_fill="nan": every format's unused rows of a sequence's last block
    hold NaN patterns (bf16 rows; fp8 codes, RoPE keys, scales; int group
    scales and minima), while the rows the sequence uses decode to finite
    values."""
    import oracle
    lens = np.array([1, 33, 64, 100], dtype=np.int32)
    bs = inputs.BLOCK
    for kv in ("bf16", "fp8", "int4", "int2"):
        c = inputs.decode_case(41, B=len(lens), seq_lens=lens, kv_dtype=kv, tail_fill="nan",
                               n_h=2, d_c=64, d_r=32, d_h=16)
        for b, L in enumerate(lens):
            ck, kr = oracle.paged_rows(c.cache, c.block_table[b], int(L), kv, 64, 32, bs)
            assert np.isfinite(ck).all() and np.isfinite(kr).all()
            used = int(L) - ((int(L) + bs - 1) // bs - 1) * bs
            blk = c.cache[c.block_table[b, (int(L) - 1) // bs]]
            if used == bs:
                continue
            if kv == "bf16":
                assert (blk[used:] == 0x7FC0).all() and not (blk[:used] == 0x7FC0).all()
            elif kv == "fp8":
                raw = blk.view(np.uint8)
                o1, o2 = bs * 64, bs * 64 + bs * 32 * 2
                assert (raw[used * 64: o1] == 0x7F).all()
                assert (raw[o1 + used * 64: o2].view(np.uint16) == 0x7FC0).all()
                assert np.isnan(raw[o2 + used * 4: o2 + bs * 4].view(np.float32)).all()
                assert np.isfinite(raw[o2: o2 + used * 4].view(np.float32)).all()
            else:
                cb = 4 if kv == "int4" else 2
                o2 = bs * (64 * cb // 8 + 32 // 2)
                prow = (64 + 32) // inputs.INT_GROUP * 4
                prm = blk.view(np.uint8)[o2: o2 + bs * prow].view(np.float16)
                assert np.isnan(prm[used * prow // 2:]).all()
                assert np.isfinite(prm[: used * prow // 2]).all()
