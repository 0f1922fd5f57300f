"""GPU parity of the streaming vocabulary loss on seeded random problems:
row counts, vocabularies on and off every kernel boundary (the single-read
sub-block splits and the two-pass kernel above 131,072), hidden sizes,
chunk sizes, row lists, dh dtypes, ignored targets, the head gradient and
the logit scale, combined in ways the fixed cases do not pair up.  Each is
checked against the fp64 oracle with the bar of tests/test_gpu_vocab.py."""
import numpy as np
import pytest
import torch

from tests.test_gpu_vocab import _check, _run

pytestmark = pytest.mark.gpu

N_CASES = 16


def _case(i):
    """Parameters of case i, from a generator seeded by i alone."""
    rng = np.random.default_rng(11000 + i)
    V = int(rng.choice([int(rng.integers(2, 2000)), int(rng.integers(2000, 40000)),
                        int(rng.integers(40000, 131073)), int(rng.integers(131073, 150000))]))
    d = 8 * int(rng.integers(1, 33))
    R = int(rng.integers(1, 200))
    row_list = bool(rng.integers(0, 2))
    T = R + (int(rng.integers(0, 100)) if row_list else 0)
    chunk = int(rng.choice([0, int(rng.integers(1, R + 1))]))
    dt = int(rng.integers(0, 2))
    n_ign = int(rng.integers(0, 3))
    ignored = [(int(j), int(rng.choice([-1, V, V + 7]))) for j in rng.choice(R, size=min(n_ign, R), replace=False)]
    head_std = float(rng.choice([1.0, 3.0, 12.0])) / d ** 0.5
    head_grad = bool(rng.integers(0, 2))
    return T, R, V, d, chunk, row_list, dt, ignored, head_std, head_grad


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_bdlm_amd import bdvocab
    bdvocab.lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_vocab(dev, i):
    T, R, V, d, chunk, row_list, dt, ignored, head_std, head_grad = _case(i)
    res = _run(dev, 12000 + i, T, R, V, d, chunk, row_list, dt, ignored=ignored, head_std=head_std,
               head_grad=head_grad)
    _check(res)
    for j, _ in ignored:
        assert res["loss"][j] == 0
