"""The seeded input generator: determinism, shapes, rounding, sampled rows."""
import numpy as np
import torch

import workloads as wl


def test_configs_shapes():
    w = wl.WORKLOADS
    assert [w[i].N for i in range(1, 6)] == [256, 32760, 75600, 32760, 75600]
    assert w[5].flops == 4.0 * 2 * 40 * 75600 ** 2 * 128
    for i in range(1, 6):
        assert sum(w[i].split) == w[i].d and all(s % 2 == 0 for s in w[i].split)
    assert w[4].peaky_rows == 328


def test_slices_are_deterministic_and_independent():
    w = wl.WORKLOADS[2]
    a = wl.slice_values(w, "q", 1, 3)
    b = wl.slice_values(w, "q", 1, 3)
    c = wl.slice_values(w, "k", 1, 3)
    assert a.dtype == np.uint16 and a.shape == (w.N, w.d)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_full_matches_slices():
    w = wl.custom(2, 3, (2, 3, 5), 16, (4, 4, 8), seed_id=77)
    f = wl.full(w, "v")
    for b in range(2):
        for h in range(3):
            assert np.array_equal(f[b, h], wl.slice_values(w, "v", b, h))


def test_bf16_rounding_matches_torch_rne():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        # exact ties: low 16 bits 0x8000 with even and odd kept parts
                        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490FDB], dtype=np.uint32).view(np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(wl.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_peaky_rows():
    w = wl.WORKLOADS[4]
    idx = wl.peaky_row_index(w, 0, 5)
    assert idx.size == 328 and np.unique(idx).size == 328
    x = wl.slice_f32(w, "k", 0, 5)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, wl.T_K, 0, 5])))
    base = g.standard_normal((w.N, w.d), dtype=np.float32)
    ratio = np.ones(w.N); ratio[idx] = 8.0
    assert np.array_equal(x, base * ratio[:, None].astype(np.float32))


def test_sample_rows():
    w = wl.WORKLOADS[5]
    r = wl.sample_rows(w, 1, 7)
    assert r.size == 256 and np.unique(r).size == 256
    assert r[0] == 0 and r[-1] == w.N - 1
    assert np.array_equal(r, wl.sample_rows(w, 1, 7))
    assert np.array_equal(wl.sample_rows(wl.WORKLOADS[1], 0, 0), np.arange(256))
