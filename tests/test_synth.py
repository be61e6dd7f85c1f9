"""The seeded input generator (CPU)."""
import numpy as np
import torch

import synth


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 seeded with 0, as produced by the published
    # reference implementation (Vigna, splitmix64.c).
    got = [int(x) for x in synth.splitmix64(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices_agree():
    full = synth.splitmix64(1234, 0, 100)
    assert np.array_equal(full[37:61], synth.splitmix64(1234, 37, 24))
    z = synth.normal_f64(9, 0, 50)
    assert np.array_equal(z[20:40], synth.normal_f64(9, 10, 10))


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 7,
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39, 65504.0,
                                  1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)])
    mine = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(mine),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_normal_statistics_and_determinism():
    a = synth.normal_bf16(77, (4, 300, 128))
    b = synth.normal_bf16(77, (4, 300, 128))
    assert np.array_equal(a, b)
    f = synth.bf16_bits_to_f32(a).astype(np.float64)
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1.0) < 0.01
    assert abs(np.mean(f ** 4) - 3.0) < 0.1          # Gaussian kurtosis
    c = synth.normal_bf16(78, (4, 300, 128))
    assert not np.array_equal(a, c)


def test_multiplier_applied_before_rounding():
    z = synth.normal_f64(5, 0, 8)
    got = synth.bf16_bits_to_f32(synth.normal_bf16(5, (16,), 3.0))
    want = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits((3.0 * z).astype(np.float32)))
    assert np.array_equal(got, want)


def test_workload_catalogue():
    w = synth.WORKLOADS[synth.HEADLINE]
    assert (w.B, w.H_q, w.H_kv, w.N, w.D, w.causal) == (2, 16, 16, 16384, 128, False)
    assert abs(w.flops - 4 * 2 * 16 * 16384 ** 2 * 128) < 1
    c = synth.WORKLOADS["mha_causal_b2_h16_n16384"]
    assert c.flops == w.flops / 2
    assert all(x.H_q % x.H_kv == 0 for x in synth.WORKLOADS.values())
    seeds = [s for x in synth.WORKLOADS.values() for s in (x.seed_base, x.seed_base + 2)]
    assert len(set(seeds)) == len(seeds)


def test_varlen_catalogue():
    """Packed workloads: lengths in range and summing to the token count, distinct
    seeds; the equal-length batch has dense causal B = 8, N = 4096's pair count."""
    seeds = []
    for w in synth.VARLEN_WORKLOADS.values():
        L = w.lengths()
        assert int(L.sum()) == w.total and L.min() >= 1 and L.max() <= w.max_len
        assert (L[:-1] >= w.min_len).all()      # only the last may be cut short
        assert w.cu_seqlens()[-1] == w.total and w.H_q % w.H_kv == 0
        seeds += [w.seed_base, w.seed_base + 3]
    assert len(set(seeds)) == len(seeds)
    eq = synth.VARLEN_WORKLOADS["varlen_causal_equal_h16_8x4096"]
    assert list(eq.lengths()) == [4096] * 8
    assert eq.pairs == 16 * 8 * 4096 * 4097 // 2


def test_e4m3_encoder_matches_torch_and_ties_to_even():
    """f64_to_e4m3 against torch's float8_e4m3fn cast on a dense grid (in range),
    exact midpoints (ties to the even code) and saturation at 448."""
    x = np.concatenate([np.linspace(-448, 448, 400001), np.linspace(-0.02, 0.02, 40001)])
    x = x.astype(np.float32).astype(np.float64)   # torch's cast goes through float32
    got = synth.f64_to_e4m3(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    # midpoints 1.0625 (between 1.0 = 0x38 and 1.125 = 0x39) and 1.1875 (0x39 / 0x3A)
    assert list(synth.f64_to_e4m3(np.array([1.0625, 1.1875, -1.0625]))) == [0x38, 0x3A, 0xB8]
    assert list(synth.f64_to_e4m3(np.array([500.0, -1e9]))) == [0x7E, 0xFE]


def test_e4m3_normals():
    w = synth.FP8_WORKLOADS["fp8_mha_tiny_b1_h2_n256"]
    q8, k8, v8 = w.generate()
    assert q8.dtype == np.uint8 and q8.shape == (1, 2, 256, 128)
    again = synth.normal_e4m3(w.seed_base, q8.shape, w.descale_q)
    assert np.array_equal(q8, again)
    z = synth.normal_f64(w.seed_base, 0, 8)
    assert np.array_equal(q8.reshape(-1)[:16], synth.f64_to_e4m3(z / w.descale_q))
    vals = torch.from_numpy(k8).view(torch.float8_e4m3fn).double().numpy() * w.descale_k
    assert abs(vals.mean()) < 0.02 and abs(vals.std() - 1.0) < 0.02
    assert not np.isnan(vals).any()


def test_sparse_pattern_and_pair_count():
    """Lists are sorted, unique, in range (at or below the diagonal when causal),
    contain the local and global blocks, and pairs() counts the allowed pairs of
    the expanded mask exactly."""
    w = synth.SparseWorkload("t", 1, 2, 2, 300, local=2, n_global=1, n_random=2, causal=True,
                             per_head=True, block=32, seed_base=5)
    nb = -(-300 // 32)
    lists = w.lists()
    assert len(lists) == 2 * nb
    for t, ls in enumerate(lists):
        qb = t % nb
        assert ls == sorted(set(ls)) and all(0 <= x <= qb for x in ls)
        assert qb in ls and 0 in ls and (qb == 0 or qb - 1 in ls)
    m = np.zeros((2, 300, 300), bool)
    for h in range(2):
        for qb in range(nb):
            for kb in lists[h * nb + qb]:
                m[h, qb * 32:(qb + 1) * 32, kb * 32:(kb + 1) * 32] = True
    m &= np.tril(np.ones((300, 300), bool))[None]
    assert w.pairs() == int(m.sum())
    ptr, idx = w.csr()
    assert ptr[0] == 0 and ptr[-1] == idx.size and np.all(np.diff(ptr) >= 0)
