"""The seeded input generator: published known answers and distribution checks."""
import numpy as np
import pytest
import torch

import fixtures as F


@pytest.fixture(scope="module", autouse=True)
def _threads():
    F.set_num_threads(4)


# Known-answer vectors published with the Random123 library for Philox4x32-10
# (Salmon et al., SC'11): counter, key -> output.
PHILOX_KAT = [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    assert list(F.philox4x32_10(ctr, key)) == want


def test_normals_are_standard_normal():
    x = F.normal_rows(7, 0x1234, 0, 400, 4096).ravel().astype(np.float64)
    assert abs(x.mean()) < 4 / np.sqrt(x.size) * 1.5
    assert abs(x.var() - 1) < 0.01
    assert abs((x ** 3).mean()) < 0.02
    assert abs((x ** 4).mean() - 3) < 0.05
    from scipy import stats
    assert stats.kstest(x[:200000], "norm").pvalue > 1e-4


def test_generation_independent_of_thread_count():
    F.set_num_threads(1)
    a = F.expert_blob(F.Q4K, 3, 1, 5, 512, 256)
    x1 = F.activations(3, 1, 7, 512)
    F.set_num_threads(4)
    b = F.expert_blob(F.Q4K, 3, 1, 5, 512, 256)
    x4 = F.activations(3, 1, 7, 512)
    assert np.array_equal(a, b) and np.array_equal(x1, x4)


def test_streams_differ():
    a = F.expert_blob(F.Q8_0, 0, 0, 0, 256, 128)
    b = F.expert_blob(F.Q8_0, 0, 0, 1, 256, 128)
    c = F.expert_blob(F.Q8_0, 0, 1, 0, 256, 128)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_f16_conversion_matches_numpy():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.normal(size=2000) * 10.0 ** rng.integers(-9, 5, size=2000),
                           [0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e-8, 6e-8, 2.98e-8, -3e-5]]).astype(np.float32)
    mine = np.array([F.f32_to_f16_bits(v) for v in vals], dtype=np.uint16)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_conversion_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.normal(size=10000) * 10.0 ** rng.integers(-6, 6, size=10000)).astype(np.float32)
    mine = F.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_logits_have_no_ties():
    lg = F.logits_normal(0, 0, 512, 256)
    for row in lg:
        assert np.unique(row).size == row.size


def test_permutation_is_a_permutation():
    p = F.permutation(5, 2, 128)
    assert sorted(p.tolist()) == list(range(128))


def test_zipf_logits_skew_loads():
    """Gumbel-top-k over Zipf(1.0) log-probabilities: the rank-1 expert is drawn
    far more often than the median one; every draw is a distinct expert."""
    T, E, k = 2048, 128, 8
    lg = F.logits_zipf(0, 0, T, E, 1.0)
    top = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    counts = np.bincount(top.ravel(), minlength=E)
    perm = F.permutation(0, 0, E)
    rank1 = int(np.where(perm == 0)[0][0])
    assert counts[rank1] == counts.max()
    assert counts.max() > 10 * np.median(counts)
    for row in lg:
        assert np.unique(row).size == E
