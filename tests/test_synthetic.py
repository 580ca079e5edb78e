"""The seeded input generator: determinism and storage-format conversions."""
import numpy as np

from attention_shards_amd import synthetic as syn


def test_deterministic_and_thread_independent(monkeypatch):
    monkeypatch.setattr(syn, "BLOCK", 1000)
    monkeypatch.setenv("TP_SYNTH_THREADS", "1")
    a = syn.normal_tensor(7, 3, (37, 101), 0.02, syn.BF16)
    monkeypatch.setenv("TP_SYNTH_THREADS", "8")
    b = syn.normal_tensor(7, 3, (37, 101), 0.02, syn.BF16)
    assert np.array_equal(a, b)
    c = syn.normal_tensor(7, 4, (37, 101), 0.02, syn.BF16)
    assert not np.array_equal(a, c)


def test_block_definition(monkeypatch):
    monkeypatch.setattr(syn, "BLOCK", 64)
    x = syn.normal_tensor(9, 1, (3, 50), 1.0, syn.F32).ravel()
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(9, spawn_key=(1, 2))))
    assert np.array_equal(x[128:150], g.standard_normal(22, dtype=np.float32))


def test_bf16_round_to_nearest_even():
    bits = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F807FFF,
                     0x3F808001, 0xBF808000, 0x00000001], dtype=np.uint32)
    got = syn.f32_to_bf16_bits(bits.view(np.float32))
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0x3F81, 0xBF80, 0x0000]


def test_bf16_roundtrip_exact():
    x = syn.normal_tensor(3, 0, (1000,), 1.0, syn.BF16)
    f = syn.bf16_bits_to_f32(x)
    assert np.array_equal(syn.f32_to_bf16_bits(f), x)
    assert np.all(np.abs(syn.to_f64(x, syn.BF16)) < 10)


def test_distribution_roughly_right():
    x = syn.to_f64(syn.normal_tensor(5, 1, (1 << 18,), 0.02, syn.BF16), syn.BF16)
    assert abs(x.mean()) < 2e-4
    assert abs(x.std() - 0.02) < 2e-4


def test_sample_rows():
    r = syn.sample_rows(5, 8192, 256)
    assert len(r) == 256 and r[0] == 0 and r[-1] == 8191
    assert len(np.unique(r)) == 256
    assert np.array_equal(r, syn.sample_rows(5, 8192, 256))


def test_held_qkv_shard_layout():
    WQ = np.arange(4 * 8).reshape(4, 8)
    WK = WQ + 100
    WV = WQ + 200
    s = syn.qkv_held_shard(WQ, WK, WV, n_heads=4, head_dim=2, i=1, t=2)
    assert s.shape == (4, 12)
    assert np.array_equal(s[:, 0:4], WQ[:, 4:8])
    assert np.array_equal(s[:, 4:8], WK[:, 4:8])
    assert np.array_equal(s[:, 8:12], WV[:, 4:8])
