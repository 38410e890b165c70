"""Seeded input generators: layout, determinism and the length/paging recipes."""
import numpy as np
import pytest

import workloads


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 0.0, -0.0], np.float32)])
    ours = workloads.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_tiny_layout():
    t = workloads.tiny(0)
    assert t.q.shape == (192, 2, 64) and t.k.shape == (192, 2, 64)
    np.testing.assert_array_equal(t.cu_q, [0, 37, 101, 102, 192])
    assert t.cu_q.dtype == np.int32
    # values are exactly representable in bf16
    np.testing.assert_array_equal(workloads.bf16_round(t.q), t.q)


def test_seed_determinism():
    a, b = workloads.tiny(3), workloads.tiny(3)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.do, b.do)
    assert not np.array_equal(workloads.tiny(4).q, a.q)


@pytest.mark.parametrize("s", [0.1, 0.5, 0.9])
def test_sparsity_lengths(s):
    rng = np.random.default_rng(0)
    L = workloads.sparsity_lengths(rng, 20000, 1024, s)
    hi = int(np.floor(1024 * (1 - s) * 2))
    assert L.min() >= 1 and L.max() <= min(hi, 1024)
    unclipped_mean = (1 + hi) / 2
    expected = np.mean(np.minimum(np.arange(1, hi + 1), 1024))
    assert abs(L.mean() - expected) < 0.02 * expected
    if s >= 0.5:
        assert abs(L.mean() - unclipped_mean) < 0.02 * unclipped_mean


def test_offsets_monotone():
    cu = workloads.offsets([3, 0, 5])
    np.testing.assert_array_equal(cu, [0, 3, 3, 8])


def test_paged_cache_holds_contiguous_rows():
    inp = workloads.decode(7, [5, 16, 1, 33], heads_q=4, heads_kv=2, head_dim=8, page_size=4)
    assert inp.num_pages == 2 + 4 + 1 + 9
    used = np.concatenate([inp.page_table[b, :-(-L // 4)] for b, L in enumerate(inp.seqlens_k)])
    np.testing.assert_array_equal(np.sort(used), np.arange(inp.num_pages))   # a permutation
    for b, L in enumerate(inp.seqlens_k):
        for t in range(L):
            page, slot = inp.page_table[b, t // 4], t % 4
            np.testing.assert_array_equal(inp.k_cache[page, slot], inp.k[inp.cu_k[b] + t])
            np.testing.assert_array_equal(inp.v_cache[page, slot], inp.v[inp.cu_k[b] + t])
        if L % 4:
            assert np.isnan(inp.k_cache[inp.page_table[b, L // 4], L % 4:]).all()


def test_config_shapes_small():
    g = workloads.gem(0, 0.9)
    assert g.q.shape[1:] == (8, 128) and g.batch == 256 and g.max_len_q <= 1024
    bq = workloads.broadcast_q(0, 0.9, batch=8)
    assert bq.q.shape == (256, 4, 128) and bq.do.shape == (8, 256, 4, 128)


def test_repage_keeps_kv_and_moves_pages():
    a = workloads.decode(3, [10, 1, 33], heads_q=4, heads_kv=2, head_dim=8, page_size=4)
    b = workloads.repage(a, 5, seed=9)
    np.testing.assert_array_equal(a.k, b.k)
    for i, L in enumerate(b.seqlens_k):
        for t in range(L):
            np.testing.assert_array_equal(b.k_cache[b.page_table[i, t // 5], t % 5], b.k[b.cu_k[i] + t])


def test_e4m3_decoding_matches_its_definition():
    """The fp8 caches use OCP e4m3 (float8_e4m3fn): sign, 4 exponent bits with bias 7,
    3 mantissa bits, subnormals m * 2^-9, and only S.1111.111 is NaN (no infinities).
    Every one of the 256 byte values decodes as that definition says."""
    import math
    torch = pytest.importorskip("torch")
    got = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for x in range(256):
        s, e, m = x >> 7, (x >> 3) & 15, x & 7
        if e == 15 and m == 7:
            assert math.isnan(got[x])
            continue
        val = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        assert got[x] == (-val if s else val), x


def test_fp8_decode_inputs_are_exact_dequantisations():
    inp = workloads.decode(3, [5, 40], 8, 2, 64, 16, q_len=2, kv_fp8=True, k_scale=0.5, v_scale=2.0)
    torch = pytest.importorskip("torch")
    kc = torch.from_numpy(inp.k_cache).view(torch.float8_e4m3fn).float().numpy()
    # token 3 of sequence 1 lives in page_table[1][0], slot 3
    page = inp.page_table[1, 0]
    np.testing.assert_array_equal(kc[page, 3] * 0.5, inp.k[inp.cu_k[1] + 3])
    assert np.all(inp.k_cache[inp.page_table[0, 0], 5:] == 0x7F)     # unused slots hold the NaN byte


def test_fp8_qkv_are_exact_dequantisations():
    """fp8_qkv: bytes x scale reproduce the returned values exactly; the default
    scale maps each tensor's amax to 448 (the largest finite e4m3 value)."""
    torch = pytest.importorskip("torch")
    inp = workloads.jagged(5, [7, 30], None, 4, 2, 64, True)
    got, enc = workloads.fp8_qkv(inp)
    for n in ("q", "k", "v"):
        dec = torch.from_numpy(enc[n]).view(torch.float8_e4m3fn).float().numpy() * enc[n + "_scale"]
        np.testing.assert_array_equal(dec, getattr(got, n))
        assert enc[n + "_scale"] == pytest.approx(np.abs(getattr(inp, n)).max() / 448.0)
        assert np.abs(getattr(got, n) - getattr(inp, n)).max() <= np.abs(getattr(inp, n)).max() / 16
    np.testing.assert_array_equal(got.do, inp.do)
    _, enc2 = workloads.fp8_qkv(inp, 0.5, 0.25, 2.0)
    assert (enc2["q_scale"], enc2["k_scale"], enc2["v_scale"]) == (0.5, 0.25, 2.0)
    with pytest.raises(ValueError):
        workloads.fp8_qkv(inp, 1e-3, 1.0, 1.0)        # |q| / scale beyond 448
