"""The seeded input generator (CPU only): Philox4x32-10 known answers,
bfloat16 rounding, shard consistency and the N(0,1) distribution."""
import numpy as np
import pytest
import torch

import ra_inputs


def test_philox_known_answers():
    # Known-answer vectors published with the Philox4x32-10 reference code
    # (Salmon et al., SC'11, Random123 distribution).
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert ra_inputs.philox4x32_10(ctr, key).tolist() == want


def test_bf16_round_to_nearest_even_matches_torch():
    x = ra_inputs.normal((1, 3, 500, 64), 0, seed=3, dtype="f32", scale=7.0)
    ours = ra_inputs.normal((1, 3, 500, 64), 0, seed=3, dtype="bf16", scale=7.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(ra_inputs.f32_to_bf16(x), ref)
    back = ra_inputs.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_shards_are_slices_of_the_whole_tensor():
    shape = (2, 3, 64, 16)
    full = ra_inputs.normal(shape, 1, seed=9, dtype="bf16")
    n = 4
    for i in range(n):
        striped = ra_inputs.normal(shape, 1, seed=9, dtype="bf16", t0=i, t_stride=n, n_rows=16)
        assert np.array_equal(striped, full[:, :, i::n])
        chunk = ra_inputs.normal(shape, 1, seed=9, dtype="bf16", t0=16 * i, n_rows=16)
        assert np.array_equal(chunk, full[:, :, 16 * i:16 * (i + 1)])
    # different streams and seeds differ
    assert not np.array_equal(full, ra_inputs.normal(shape, 2, seed=9, dtype="bf16"))
    assert not np.array_equal(full, ra_inputs.normal(shape, 1, seed=8, dtype="bf16"))


def test_standard_normal_moments():
    x = ra_inputs.normal((1, 4, 4096, 64), 0, seed=0, dtype="f32").astype(np.float64).ravel()
    n = x.size
    assert abs(x.mean()) < 5 / np.sqrt(n)
    assert abs(x.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    assert abs(np.mean(x ** 3)) < 5 * np.sqrt(15.0 / n)
    assert abs(np.mean(x ** 4) - 3.0) < 5 * np.sqrt(96.0 / n)
    assert abs(np.mean(np.abs(x) < 1.0) - 0.6826894921) < 0.005


def test_sample_rows_are_stratified_and_unique():
    h, t = ra_inputs.sample_rows(4096, 4, 300, heads=8, seed=1)
    pairs = set(zip(h.tolist(), t.tolist()))
    assert len(pairs) == len(h) == 300
    ts = set(t.tolist())
    for b in range(0, 4096, 1024):
        assert b in ts and b + 1023 in ts
    assert np.all((h >= 0) & (h < 8))


def test_sample_rows_exact_count_and_share():
    """Exactly the requested number of distinct rows, also where draws collide
    often (few tokens), and a share's rows lie on its position's tokens."""
    h, t = ra_inputs.sample_rows(64, 4, 500, heads=8, seed=1)
    assert len(set(zip(h.tolist(), t.tolist()))) == len(h) == 500
    with pytest.raises(ValueError):
        ra_inputs.sample_rows(64, 4, 513, heads=8, seed=1)
    for lay in ("striped", "contiguous"):
        h, t = ra_inputs.sample_rows(1 << 20, 32, 4096, heads=32, seed=1, share=31, layout=lay)
        assert len(set(zip(h.tolist(), t.tolist()))) == len(h) == 4096
        if lay == "striped":
            assert np.all(t % 32 == 31) and {31, 31 + 32 * 32767} <= set(t.tolist())
        else:
            assert np.all(t // 32768 == 31) and {31 * 32768, 32 * 32768 - 1} <= set(t.tolist())
    # the draw is seeded
    a = ra_inputs.sample_rows(4096, 4, 300, heads=8, seed=5)
    b = ra_inputs.sample_rows(4096, 4, 300, heads=8, seed=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
