"""The input generator against its published definitions (CPU only)."""
import math

import numpy as np
import torch

import synth

M64 = (1 << 64) - 1


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_splitmix64_reference_sequence():
    """Counter-style SplitMix64 equals the sequential generator: state starts at
    the stream key and advances by the golden gamma before each output."""
    seed, stream = 12345, 7
    key = _mix(_mix(seed) ^ ((stream * 0xD1B54A32D192ED03) & M64))
    state = key
    ref = []
    for _ in range(10):
        state = (state + 0x9E3779B97F4A7C15) & M64
        ref.append(_mix(state))
    assert synth.draws(seed, stream, 0, 10).tolist() == ref
    assert synth.draws(seed, stream, 4, 3).tolist() == ref[4:7]


def test_known_splitmix64_outputs():
    """Sequential SplitMix64 seeded with 1234567 (published test sequence)."""
    state = 1234567
    out = []
    for _ in range(3):
        state = (state + 0x9E3779B97F4A7C15) & M64
        out.append(_mix(state))
    assert out == [6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000) * 10, [0.0, -0.0, 1e-40, 3.0e38,
                                                          1.00390625, 1.01171875]])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits_from_float(x), ref)
    back = synth.bf16_to_float(ref)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_normal_moments_and_slices():
    x = synth.bf16_to_float(synth.normal_bf16(9, 1, 0, 1_000_000)).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    part = synth.normal_bf16(9, 1, 1001, 77)
    assert np.array_equal(part, synth.normal_bf16(9, 1, 0, 2000)[1001:1078])


def test_clustered_keys_share_frame_means():
    wl = synth.prefill_32k().with_(seqlens_q=(1024,), seqlens_k=(1024,))
    k = synth.bf16_to_float(wl.k_idx()).astype(np.float64)
    means = k.reshape(4, 256, -1).mean(axis=1)  # per-frame mean vectors
    # frame means ~ N(0, 0.5^2) per channel: their spread is far above noise/16
    assert 0.35 < means.std() < 0.65
    # within a frame, the residual is the unit-variance noise
    resid = k.reshape(4, 256, -1) - means[:, None, :]
    assert abs(resid.std() - 1.0) < 0.03


def test_timestamp_tokens_are_scaled():
    wl = synth.varlen_512k().with_(seqlens_q=(512,), seqlens_k=(512,))
    k = synth.bf16_to_float(wl.k_idx()).astype(np.float64)
    base = wl.with_(ts_tokens=0)
    k0 = synth.bf16_to_float(base.k_idx()).astype(np.float64)
    ts = (np.arange(512) % 256) < 8
    assert np.array_equal(k[~ts], k0[~ts])
    np.testing.assert_allclose(k[ts], 2.0 * k0[ts], rtol=2 ** -7)


def test_varlen_lengths():
    lens = synth.varlen_512k().seqlens_q
    assert sum(lens) == 524288
    assert all(n % 256 == 0 for n in lens)
    assert all(4096 <= n <= 262144 for n in lens[:-1])


def test_integer_workload_ranges():
    wl = synth.prefill_2k_int()
    qi = synth.bf16_to_float(wl.q_idx())
    w = wl.w()
    assert set(np.unique(qi).tolist()) == set(range(-3, 4))
    assert set(np.unique(w).tolist()) == {0.0, 1.0, 2.0, 3.0}
    assert math.isclose(wl.softmax_scale, 0.125)
