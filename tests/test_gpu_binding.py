"""The torch wrappers reject badly shaped or typed buffers before anything is
launched: the C ABI sees only pointers, so a short output buffer would be written
past its end. Each check leaves a sentinel buffer, which a launch would overwrite,
untouched."""
import pytest

from linear_attention_04_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()
    w = inputs.custom_workload("binding", 601, heads=2, total_tokens=40, has_initial_state=True)
    x = inputs.generate(w)
    d = gu.upload(x, True, False)
    return torch, kda, d


def _sentinel(torch, shape, dtype=None):
    return torch.full(shape, 7.0, dtype=dtype or torch.float32, device="cuda")


def _untouched(torch, t):
    torch.cuda.synchronize()
    return bool(torch.all(t.float() == 7.0))


def test_initial_state_shape_checked(setup):
    torch, kda, d = setup
    fs = _sentinel(torch, (1, 2, 128, 128))
    bad = torch.zeros((1, 2, 128, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="initial_state"):
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=bad, final_state=fs)
    assert _untouched(torch, fs)


@pytest.mark.parametrize("what", ["shape", "dtype", "noncontiguous"])
def test_out_checked(setup, what):
    torch, kda, d = setup
    fs = _sentinel(torch, (1, 2, 128, 128))
    if what == "shape":
        out = _sentinel(torch, (39, 2, 128), torch.bfloat16)
    elif what == "dtype":
        out = _sentinel(torch, (40, 2, 128))
    else:
        out = _sentinel(torch, (40, 128, 2), torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError, match="out"):
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"], out=out,
                          final_state=fs)
    assert _untouched(torch, fs) and _untouched(torch, out)


def test_final_state_checked(setup):
    torch, kda, d = setup
    out = _sentinel(torch, (40, 2, 128), torch.bfloat16)
    fs = _sentinel(torch, (2, 2, 128, 128))  # N = 1
    with pytest.raises(ValueError, match="final_state"):
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], out=out, final_state=fs)
    assert _untouched(torch, out) and _untouched(torch, fs)


def test_short_workspace_checked(setup):
    torch, kda, d = setup
    out = _sentinel(torch, (40, 2, 128), torch.bfloat16)
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], out=out, workspace=ws)
    assert _untouched(torch, out)


def test_training_forward_outputs_checked(setup):
    torch, kda, d = setup
    fs = _sentinel(torch, (1, 2, 128, 128))
    out = _sentinel(torch, (40, 2, 64), torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        kda.chunk_prefill_for_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], out=out, final_state=fs)
    assert _untouched(torch, fs)


def test_backward_from_saved_needs_the_saved_workspace(setup):
    torch, kda, d = setup
    d_out = torch.zeros_like(d["v"])
    with pytest.raises(ValueError, match="workspace"):
        kda.chunk_prefill_backward_from_saved(d["q"], d["k"], d["v"], d["g"], d["beta"], d_out, None)
    small = torch.empty(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        kda.chunk_prefill_backward_from_saved(d["q"], d["k"], d["v"], d["g"], d["beta"], d_out, small)


def test_inputs_on_another_device_or_shape_rejected(setup):
    torch, kda, d = setup
    with pytest.raises(ValueError):
        kda.chunk_prefill(d["q"], d["k"], d["v"][:, :1], d["g"], d["beta"])
    with pytest.raises(ValueError):
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"].cpu())
