"""The seeded input generator: deterministic, slice-stable, right distributions."""
import numpy as np

import synth


def _sm64_seq(seed, n):
    """Sequential SplitMix64 from its published definition (Steele et al.)."""
    out, s = [], seed
    M = (1 << 64) - 1
    for _ in range(n):
        s = (s + 0x9E3779B97F4A7C15) & M
        z = s
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        out.append(z ^ (z >> 31))
    return out


def test_counter_form_equals_sequential_splitmix64():
    k = synth.key(3, 17)
    seq = _sm64_seq(k, 40)
    assert [synth.word(k, i) for i in range(40)] == seq
    # published first output for seed 0 (Vigna's splitmix64 reference)
    assert synth.word(0, 0) == 0xE220A8397B1DCDAF


def test_row_slices_are_stable():
    k = synth.key(1, 0)
    full = synth.q4k_weight(k, 12, 1024)
    part = synth.q4k_weight(k, 5, 1024, row0=4)
    assert np.array_equal(full[4:9], part)


def test_d_dmin_are_normal_halves_in_range():
    w = synth.q4k_weight(synth.key(2, 5), 64, 2048).reshape(-1, 144)
    for off in (0, 2):
        h = (w[:, off].astype(np.uint16) | (w[:, off + 1].astype(np.uint16) << 8))
        v = h.view(np.float16).astype(np.float64)
        assert v.min() >= 1e-4 * (1 - 2 ** -11) and v.max() <= 1e-3 * (1 + 2 ** -11)
        assert ((h >> 10) & 31).min() >= 1          # binary16 normals


def test_half_bits_rne_named_values():
    assert synth.half_bits(1e-4) == int(np.float16(1e-4).view(np.uint16))
    assert synth.half_bits(1e-3) == int(np.float16(1e-3).view(np.uint16))
    rng = np.random.default_rng(0)
    for v in rng.uniform(1e-4, 1e-3, 2000):
        assert synth.half_bits(float(v)) == int(np.float16(v).view(np.uint16))


def test_scale_and_nibble_bytes_look_uniform():
    w = synth.q4k_weight(synth.key(2, 6), 256, 4096).reshape(-1, 144)
    body = w[:, 4:].ravel()
    counts = np.bincount(body, minlength=256)
    exp = body.size / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 400                               # 255 dof, p ~ 1e-7 bound


def test_normals_moments_and_determinism():
    x = synth.normal(synth.key(1, synth.ACT_BASE), 200001)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert np.array_equal(x[:1000], synth.normal(synth.key(1, synth.ACT_BASE), 1000))


def test_q6_k_blocks_counter_layout_and_ranges():
    """Block b of a Q6_K stream is word 27b (d) and words 27b+1 .. 27b+26
    (the 208 bytes before d, little-endian); d is a normal binary16 in
    [1e-4, 1e-3] and the other bytes look uniform."""
    k = synth.key(2, 7)
    w = synth.q6_k_weight(k, 3, 512)                 # 6 blocks
    blocks = w.reshape(-1, 210)
    for b in range(blocks.shape[0]):
        body = b"".join(synth.word(k, 27 * b + 1 + j).to_bytes(8, "little") for j in range(26))
        assert bytes(blocks[b, :208]) == body[:208]
    big = synth.q6_k_weight(synth.key(2, 8), 128, 4096).reshape(-1, 210)
    h = big[:, 208].astype(np.uint16) | (big[:, 209].astype(np.uint16) << 8)
    v = h.view(np.float16).astype(np.float64)
    assert v.min() >= 1e-4 * (1 - 2 ** -11) and v.max() <= 1e-3 * (1 + 2 ** -11)
    counts = np.bincount(big[:, :208].ravel(), minlength=256)
    exp = big[:, :208].size / 256
    assert ((counts - exp) ** 2 / exp).sum() < 400
    assert np.array_equal(synth.q6_k_weight(synth.key(2, 8), 128, 4096).reshape(-1, 210), big)
