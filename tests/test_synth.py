"""Seeded generators: rounding, determinism, mask recipes (no GPU)."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 7,
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, 65504.0, 1e-30], np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(synth.round_bf16(x), want)
    bits = synth.f32_to_bf16_bits(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, tb)


def test_inputs_deterministic_and_per_head():
    cfg = synth.get_config("wan")
    q1, k1, v1 = synth.gen_qkv(cfg, heads=[3, 7])
    q2, k2, v2 = synth.gen_qkv(cfg, heads=[7])
    assert np.array_equal(q1[:, 1], q2[:, 0]) and np.array_equal(v1[:, 1], v2[:, 0])
    qa, ka = synth.gen_qk(cfg, cfg.data_seed, heads=[3])
    assert np.array_equal(qa[:, 0], q1[:, 0]) and np.array_equal(ka[:, 0], k1[:, 0])
    assert np.array_equal(synth.round_bf16(q1), q1), "bf16-exact"
    assert np.all(q1[:, :, cfg.S:] == 0) and np.all(v1[:, :, cfg.S:] == 0), "padding zeroed"
    assert not np.array_equal(q1[:, 0], k1[:, 0])


def test_positional_term():
    pe = synth.positional_term(32768, 32760, 128, (21, 30, 52))
    assert pe.shape == (32768, 128)
    assert np.all(pe[32760:] == 0)
    # token 0: all angles 0 -> sin 0, cos 1
    assert np.allclose(pe[0, 0::2], 0) and np.allclose(pe[0, 1::2], 1)
    # tokens one frame apart share row/col channels
    assert np.array_equal(pe[5, 44:], pe[5 + 1560, 44:])


def _check_csr(cfg, rp, ci):
    assert rp.dtype == np.int32 and ci.dtype == np.int32
    assert len(rp) == cfg.rows + 1 and rp[0] == 0 and rp[-1] == len(ci)
    for r in range(cfg.rows):
        c = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(c) > 0)
        assert len(c) == 0 or (c[0] >= 0 and c[-1] < cfg.nkb_valid)


def test_masks():
    tiny = synth.get_config("tiny")
    rp, ci = synth.csr_for_config(tiny)
    _check_csr(tiny, rp, ci)
    assert len(ci) == 36
    for r in range(8):
        assert r in ci[rp[r]:rp[r + 1]], "diagonal kept"

    mochi = synth.get_config("mochi")
    rp, ci = synth.csr_for_config(mochi)
    _check_csr(mochi, rp, ci)
    assert np.all(np.diff(rp) == 26) and len(ci) == 79872

    wan = synth.get_config("wan")
    rp, ci = synth.csr_for_config(wan)
    _check_csr(wan, rp, ci)
    per_head = np.diff(rp[::wan.nqb])
    assert np.all(per_head >= 0.30 * wan.nqb * wan.nkb)
    assert 0.30 <= len(ci) / (wan.rows * wan.nkb) < 0.34
    a, b = synth.csr_for_config(wan)
    assert np.array_equal(a, rp) and np.array_equal(b, ci), "deterministic"

    imb = synth.get_config("imbalance")
    rp0, ci0 = synth.csr_for_config(imb, 0)
    rp1, ci1 = synth.csr_for_config(imb, 1)
    _check_csr(imb, rp0, ci0)
    assert not np.array_equal(rp0, rp1)
    cnt = np.diff(rp0)
    assert cnt.min() >= 1 and cnt.max() <= 256 and cnt.max() > 4 * cnt.mean() / 2
