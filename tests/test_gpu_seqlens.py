"""kda_check_seqlens on the device: well-formed packed-sequence boundaries give -1,
and each kind of malformed boundary gives the first index at which it breaks. The
expected values follow from the definition (cu[0] = 0, non-decreasing, cu[N] = T)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()  # fails loudly when the HIP library is missing


def _check(values, total_tokens):
    import torch

    from linear_attention_04_amd import kda

    cu = torch.tensor(np.asarray(values, dtype=np.int32), device="cuda")
    return kda.check_seqlens(cu, total_tokens)


def test_well_formed_boundaries():
    assert _check([0, 16], 16) == -1
    assert _check([0, 0], 0) == -1                  # no tokens at all
    assert _check([0, 5, 5, 40, 100], 100) == -1    # an empty sequence inside the batch
    assert _check([0, 0, 0, 7], 7) == -1


def test_malformed_boundaries():
    assert _check([1, 16], 16) == 0                 # does not start at token 0
    assert _check([0, 10, 9, 16], 16) == 2          # decreasing
    assert _check([0, -5, 16], 16) == 1
    assert _check([0, 10, 12], 16) == 2             # does not end at T
    assert _check([0, 20, 30], 16) == 2             # past T, caught at the end
    assert _check([3, 2, 1], 1) == 0                # the first failure is reported


def test_many_sequences():
    # more boundaries than threads in the checking workgroup
    rng = np.random.default_rng(5)
    lengths = rng.integers(0, 40, size=5000)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    assert _check(cu, T) == -1
    bad = cu.copy()
    bad[4500] = bad[4499] - 1
    bad[3333] = bad[3332] - 1
    assert _check(bad, T) == 3333
    assert _check(cu, T + 1) == 5000
