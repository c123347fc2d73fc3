"""kda_chunk_prefill_noalloc (the entry point for callers that cannot allocate) through
the C ABI, against kda_chunk_prefill on the same inputs: bitwise equal, and within
the bf16 bars of the fp64 oracle. Two calls in a row, the second smaller; a single
sequence too large for the fixed buffer (run in segments); a packed batch that fits,
and one that does not (rejected before anything runs)."""
import numpy as np
import pytest

from linear_attention_04_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()
    return kda


def _run_both(kda, w, x, packed, with_s0=True, with_final=True):
    """(out, final) of kda_chunk_prefill_noalloc and of kda_chunk_prefill."""
    torch = gu.torch_mod()
    d = gu.upload(x, w.bf16, packed)
    s0 = d["initial_state"] if with_s0 else None
    dims = kda.make_dims(d["q"], d["v"], d["cu_seqlens"], g=d["g"])
    shape_fs = (dims.num_seqs, dims.num_heads, dims.head_k, dims.head_v)
    res = {}
    for name in ("noalloc", "prefill"):
        out = torch.full(d["v"].shape, 3.0, dtype=d["v"].dtype, device="cuda")
        fs = torch.full(shape_fs, 3.0, dtype=torch.float32, device="cuda") if with_final else None
        p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        stream = torch.cuda.current_stream().cuda_stream
        if name == "noalloc":
            st = kda.kda_chunk_prefill_noalloc(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]),
                                               p(d["cu_seqlens"]), p(s0), p(out), p(fs), dims, stream)
        else:
            ws = kda.workspace_for(dims, "cuda")
            st = kda.kda_chunk_prefill(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]),
                                       p(d["cu_seqlens"]), p(s0), p(out), p(fs), dims, p(ws), ws.numel(), stream)
        assert st == kda.KDA_OK, (name, kda.kda_status_string(st))
        torch.cuda.synchronize()
        res[name] = (out, fs)
    return d, res


def _check(kda, w, x, packed, with_s0=True, with_final=True):
    torch = gu.torch_mod()
    print(f"case {w.name}: H={w.heads} T={w.total_tokens} N={w.num_seqs} gate={w.gate} s0={with_s0} "
          f"final={with_final} workspace={kda.kda_workspace_bytes(_dims(kda, w))} B", flush=True)
    d, res = _run_both(kda, w, x, packed, with_s0, with_final)
    (out_n, fs_n), (out_p, fs_p) = res["noalloc"], res["prefill"]
    assert torch.equal(out_n, out_p), "out differs from kda_chunk_prefill"
    if with_final:
        assert torch.equal(fs_n, fs_p), "final state differs from kda_chunk_prefill"
    xs = dict(x)
    if not with_s0:
        xs["initial_state"] = None
    ro, rs = gu.run_oracle(xs, packed)
    gu.assert_close("out", gu.to_host(out_n), ro, w.bf16)
    if with_final:
        gu.assert_close("final_state", gu.to_host(fs_n), rs, w.bf16)


def _dims(kda, w):
    return kda.KdaDims(w.total_tokens, w.heads, w.head_k, w.head_v, w.num_seqs,
                       kda.KDA_IO_BF16 if w.bf16 else kda.KDA_IO_F32,
                       kda.KDA_GATE_SCALAR if w.gate == "scalar" else kda.KDA_GATE_CHANNEL)


def test_two_calls_second_smaller(lib):
    w1 = inputs.custom_workload("na_first", 701, heads=4, total_tokens=1000, has_initial_state=True)
    _check(lib, w1, inputs.generate(w1), False)
    w2 = inputs.custom_workload("na_second", 702, heads=2, total_tokens=300, has_initial_state=True)
    _check(lib, w2, inputs.generate(w2), False)


def test_one_sequence_in_segments(lib):
    # 48 heads x 8192 tokens need 348 MiB of workspace: seven segments of 85 chunks,
    # the state passed through both carriers in turn
    w = inputs.custom_workload("na_segments", 703, heads=48, total_tokens=8192, has_initial_state=True)
    assert lib.kda_workspace_bytes(_dims(lib, w)) > lib.KDA_NOALLOC_SCRATCH_BYTES
    x = inputs.generate(w)
    _check(lib, w, x, False)
    _check(lib, w, x, False, with_s0=False, with_final=False)


def test_one_sequence_in_segments_scalar_gate_then_smaller(lib):
    w = inputs.custom_workload("na_segments_sg", 704, heads=12, total_tokens=9000, has_initial_state=True,
                               gate="scalar")
    _check(lib, w, inputs.generate(w), False)
    w2 = inputs.custom_workload("na_small", 705, heads=3, total_tokens=77, has_initial_state=True)
    _check(lib, w2, inputs.generate(w2), False)


def test_packed_batch_that_fits(lib):
    w = inputs.custom_workload("na_packed", 706, heads=4, lengths=[100, 17, 0, 333, 16], has_initial_state=True)
    _check(lib, w, inputs.generate(w), True)


def test_fp32_small(lib):
    w = inputs.custom_workload("na_f32", 707, heads=2, total_tokens=70, head_k=32, head_v=32, io_dtype="f32",
                               has_initial_state=True)
    _check(lib, w, inputs.generate(w), False)


@pytest.mark.parametrize("case", ["fits", "segments"])
def test_graph_capture_and_replay(lib, case):
    """The use the entry point exists for: captured once in a HIP graph (it allocates
    nothing, so the capture holds only its kernels) and replayed on new inputs, with
    eager work and synchronisation between replays; every replay equals an eager
    kda_chunk_prefill on the same inputs, bit for bit."""
    torch = gu.torch_mod()
    kda = lib
    H, T = (4, 300) if case == "fits" else (48, 2000)
    mk = lambda seed: inputs.custom_workload(f"na_graph_{case}_{seed}", seed, heads=H, total_tokens=T,  # noqa: E731
                                             has_initial_state=True)
    w = mk(720)
    d = gu.upload(inputs.generate(w), True, False)
    dims = kda.make_dims(d["q"], d["v"], None, g=d["g"])
    assert (kda.kda_workspace_bytes(dims) > kda.KDA_NOALLOC_SCRATCH_BYTES) == (case == "segments")
    out = torch.empty_like(d["v"])
    fs = torch.empty_like(d["initial_state"])
    p = lambda t: t.data_ptr()  # noqa: E731

    def call():
        st = kda.kda_chunk_prefill_noalloc(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), None,
                                           p(d["initial_state"]), p(out), p(fs), dims,
                                           torch.cuda.current_stream().cuda_stream)
        assert st == kda.KDA_OK, kda.kda_status_string(st)

    call()  # eager first: the device's buffer address is looked up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        xr = inputs.generate(mk(721 + rep))
        dr = gu.upload(xr, True, False)
        for name in ("q", "k", "v", "g", "beta", "initial_state"):
            d[name].copy_(dr[name])
        ref_out, ref_fs = gu.run_gpu(dr)  # eager kda_chunk_prefill on its own workspace
        out.zero_()
        fs.zero_()
        graph.replay()
        torch.cuda.synchronize()
        print(f"case {case}: replay {rep}", flush=True)
        assert torch.equal(out, ref_out) and torch.equal(fs, ref_fs), f"replay {rep} differs from the eager call"


def test_packed_batch_too_large_is_rejected(lib):
    torch = gu.torch_mod()
    kda = lib
    # two sequences x 64 heads x 8192 tokens: 486 MiB of workspace, and packed batches
    # are not run in segments. Rejected before anything is launched: the buffers
    # passed here are small sentinels that a launch would overrun.
    dims = kda.KdaDims(8192, 64, 128, 128, 2, kda.KDA_IO_BF16, kda.KDA_GATE_CHANNEL)
    buf = torch.full((1024,), 7.0, dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 4000, 8192], dtype=torch.int32, device="cuda")
    p = buf.data_ptr()
    st = kda.kda_chunk_prefill_noalloc(p, p, p, p, p, cu.data_ptr(), None, p, p, dims,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == kda.KDA_ERR_CAPACITY, kda.kda_status_string(st)
    torch.cuda.synchronize()
    assert bool(torch.all(buf == 7.0))
    # too many heads for even one chunk per segment beside the two state carriers
    dims = kda.KdaDims(64, 4096, 128, 128, 1, kda.KDA_IO_BF16, kda.KDA_GATE_CHANNEL)
    st = kda.kda_chunk_prefill_noalloc(p, p, p, p, p, None, None, p, p, dims,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == kda.KDA_ERR_CAPACITY, kda.kda_status_string(st)
    torch.cuda.synchronize()
    assert bool(torch.all(buf == 7.0))
