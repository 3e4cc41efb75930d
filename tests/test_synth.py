"""Pins of the seeded input generator (CPU)."""
import numpy as np

import synth


def test_splitmix64_published_vectors():
    # SplitMix64 seeded with 0: the first three outputs published with the generator's reference code.
    out = [int(v) for v in synth.draws(0, 0, 3)]
    assert out == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_any_offset():
    s = synth.stream_seed(1, 2, synth.TAG_GATE_UP, 5)
    full = synth.normals_f32(s, 0, 1000)
    part = synth.normals_f32(s, 400, 100)
    assert np.array_equal(full[400:500], part)
    assert np.array_equal(synth.normals_f32(s, 0, 1000, chunk=37), full)


def test_irwin_hall_moments():
    z = synth.normals_f32(synth.stream_seed(0, 0, 0), 0, 400_000).astype(np.float64)
    assert abs(z.mean()) < 0.01
    assert abs(z.std() - 1.0) < 0.01
    # Irwin-Hall(12) has excess kurtosis -1.2/12 = -0.1 and support [-6, 6]
    k = np.mean(z ** 4) / np.mean(z ** 2) ** 2 - 3.0
    assert abs(k + 0.1) < 0.03
    assert np.abs(z).max() <= 6.0


def test_sigma_scaling_is_one_product():
    s = synth.stream_seed(3, 0, 2, 0)
    z = synth.integer_normals(s, 0, 64)
    w = synth.normals_f32(s, 0, 64, 0.02)
    expect = z.astype(np.float32) * np.float32(np.float32(0.02) * np.float32(2.0 ** -16))
    assert np.array_equal(w, expect)


def test_streams_differ():
    a = synth.normals_f32(synth.stream_seed(1, 0, 2, 0), 0, 64)
    b = synth.normals_f32(synth.stream_seed(1, 0, 2, 1), 0, 64)
    c = synth.normals_f32(synth.stream_seed(1, 1, 2, 0), 0, 64)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_bf16_rounding_ties_to_even():
    one = np.float32(1.0)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -(1 + 3 * 2 ** -8)], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert list(got) == [one, 1 + 2 ** -6, one, -(1 + 2 ** -6)]


def test_router_int8_ranges():
    w, s = synth.router_int8(1, 0, 128, 2816)
    assert w.dtype == np.int8 and w.shape == (128, 2816)
    assert w.min() >= -127 and w.max() <= 127
    assert 25 < w.astype(np.float64).std() < 40
    assert s.dtype == np.float32 and np.all(s > 0)
    lo, hi = 0.02 / 32 * 0.75, 0.02 / 32 * 1.25
    assert np.all(s >= lo * (1 - 1e-6)) and np.all(s <= hi)


def test_zipf_trace_distinct_and_distribution():
    tr = synth.zipf_trace(7, 200, 30, 8, 128, 1.1)
    assert tr.shape == (200, 30, 8) and tr.min() >= 0 and tr.max() < 128
    for row in tr.reshape(-1, 8):
        assert len(set(row.tolist())) == 8
    # the first draw of each (token, layer) is a plain Zipf(1.1) sample: chi-square against the pmf
    first = tr[:, :, 0].ravel()
    p = synth.zipf_pmf(128, 1.1)
    obs = np.bincount(first, minlength=128).astype(np.float64)
    exp = p * first.size
    # merge the tail so every bin expects at least 5 samples
    small = np.nonzero(exp < 5)[0]
    cut = int(small[0]) if small.size else exp.size - 1
    o = np.append(obs[:cut], obs[cut:].sum())
    e = np.append(exp[:cut], exp[cut:].sum())
    chi2 = float(((o - e) ** 2 / e).sum())
    dof = o.size - 1
    assert chi2 < dof + 5 * np.sqrt(2 * dof)


def test_configs():
    c = synth.CONFIGS
    assert c["tiny"].d == 256 and c["tiny"].k == 2 and not c["tiny"].sb_bf16
    assert c["layer"].n_experts == 128 and c["layer"].k == 8 and c["layer"].F == 704
    assert c["stack"].n_layers == 30 and c["stack"].n_tokens == 256 and c["stack"].rms_norm
    assert c["batched"].weight_cfg == c["layer"].weight_cfg and c["batched"].n_tokens == 32
    assert c["streamed"].weight_cfg == c["stack"].weight_cfg and c["streamed"].n_slots == 16


def test_host_c_generator_equals_numpy_definition():
    # the C twin (synth_host.c) and the numpy definition draw the same bits, at any offset and thread count
    s = synth.stream_seed(2, 29, synth.TAG_DOWN, 127)
    for start, n, threads in [(0, 1000, 1), (123457, 65537, 0), (3, 1 << 20, 3)]:
        a = synth.normals_f32(s, start, n, 0.02, threads=threads)
        b = synth.normals_f32_numpy(s, start, n, 0.02)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
