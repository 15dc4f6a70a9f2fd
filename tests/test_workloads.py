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


def test_planted_keys_drive_the_intended_softmax_course():
    """The planted-key inputs of the GPU softmax edge cases do what the
    cases claim, checked on the decoded values: the late keys lift the
    running maximum by more than the exact-step threshold (21 log2 units),
    the largest by enough to overflow exp2(s - m - 20) in fp32 for some rows;
    a first-tile key dominates every later key; tied keys are identical."""
    import oracle
    from tests.test_gpu_parity import EDGE_CASES, EDGE_D, EDGE_N
    q, k, v = wl.planted_keys(EDGE_N, EDGE_D, 2, EDGE_CASES["late_dominant"])
    for h, ((j1, _), (j2, _)) in enumerate(EDGE_CASES["late_dominant"]):
        qd, kd = oracle.decode_bf16(q[0, h]), oracle.decode_bf16(k[0, h])
        s = qd @ kd.T / np.sqrt(EDGE_D) * np.log2(np.e)
        before1 = s[:, :j1 // 64 * 64].max(axis=1)
        assert (s[:, j1] - before1).min() > 21
        assert (s[:, j2] - s[:, j1] - 20).max() > 128  # exp2 overflows for these rows
    q, k, v = wl.planted_keys(EDGE_N, EDGE_D, 2, EDGE_CASES["first_tile_dominant"])
    for h, ((j, _),) in enumerate(EDGE_CASES["first_tile_dominant"]):
        assert j < 64
        qd, kd = oracle.decode_bf16(q[0, h]), oracle.decode_bf16(k[0, h])
        s = qd @ kd.T
        assert (s[:, j] > np.delete(s, j, axis=1).max(axis=1)).all()
    q, k, v = wl.planted_keys(EDGE_N, EDGE_D, 2, EDGE_CASES["ties"])
    for h, plants in enumerate(EDGE_CASES["ties"]):
        rows = [k[0, h, j] for j, _ in plants]
        assert all(np.array_equal(rows[0], r) for r in rows[1:])
