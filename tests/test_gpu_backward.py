"""GPU parity of the backward pass (kda_chunk_prefill_backward through the C ABI)
against the fp64 oracle's reverse-mode gradients, at sizes the oracle finishes in
seconds: several chunks and heads, ragged tails, packed sequences with empty ones,
both gate kinds, with and without initial states and final-state gradients."""
import numpy as np
import pytest

import oracle
from linear_attention_04_amd import inputs
from oracle import reference
from tests import gpu_util as gu
from tests import rounding_model

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()  # fails loudly when the HIP library is missing


def _case(name, seed, H, T=None, state=True, gate=0.1, lengths=None, gate_kind="channel"):
    w = inputs.custom_workload(name, seed, heads=H, total_tokens=T, head_k=128, head_v=128, io_dtype="bf16",
                               gate_scale=gate, has_initial_state=state, lengths=lengths, gate=gate_kind)
    x = inputs.generate(w)
    d_out, d_fs = inputs.output_gradients(w)
    return w, x, d_out, d_fs


def _check(w, x, d_out, d_fs, packed, use_dfs=True):
    print(f"case {w.name}: H={w.heads} T={w.total_tokens} N={w.num_seqs} gate={w.gate} "
          f"state={w.has_initial_state} dfs={use_dfs}", flush=True)
    d_fs = d_fs if use_dfs else None
    d = gu.upload_backward(x, d_out, d_fs, packed)
    got = gu.run_gpu_backward(d)
    ref = gu.run_oracle_backward(x, d_out, d_fs, packed)
    model = rounding_model.backward(x if packed else dict(x, cu_seqlens=None), d_out, d_fs)
    for name in GRADS + ("d_initial_state",):
        gu.assert_close_rel(name, gu.to_host(got[name]), ref[name])
        gu.assert_model_band(name, gu.to_host(got[name]), ref[name], model[name])
    return d, got, ref


def test_backward_small_with_intermediates():
    """One sequence, two heads, four chunks; also the workspace's chunk start states
    and end-state gradients against the chunked reference."""
    torch = gu.torch_mod()
    w, x, d_out, d_fs = _case("bwd_small", 101, H=2, T=64)
    d = gu.upload_backward(x, d_out, d_fs, False)
    lay = gu.backward_workspace_layout(w.total_tokens, w.heads, 1)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    got = gu.run_gpu_backward(d, workspace=ws)
    raw = ws.cpu().numpy()
    for h in range(w.heads):
        r = reference.chunked_backward(x["q"][:, h], x["k"][:, h], x["v"][:, h], x["g"][:, h], x["beta"][:, h],
                                       d_out[:, h], x["initial_state"][0, h], d_fs[0, h], intermediates=True)
        for ci in range(4):
            o = (ci * w.heads + h) * 32768  # [chunk][head]
            s0 = gu.decode_state_fragments(raw[lay["off_states"] + o:lay["off_states"] + o + 32768])
            rr = gu.decode_state_fragments(raw[lay["off_dstates"] + o:lay["off_dstates"] + o + 32768])
            gu.assert_close_rel(f"S0[h{h},c{ci}]", s0, r["S0s"][ci])
            gu.assert_close_rel(f"R[h{h},c{ci}]", rr, r["Rs"][ci])
    ref = gu.run_oracle_backward(x, d_out, d_fs, False)
    for name in GRADS:
        gu.assert_close_rel(name, gu.to_host(got[name]), ref[name])
    gu.assert_close_rel("d_initial_state", gu.to_host(got["d_initial_state"]), ref["d_initial_state"])


@pytest.mark.parametrize("T", [1, 15, 16, 17, 100, 333])
def test_backward_lengths(T):
    w, x, d_out, d_fs = _case(f"bwd_t{T}", 110 + T, H=5, T=T)
    _check(w, x, d_out, d_fs, False)


def test_backward_packed_ragged():
    w, x, d_out, d_fs = _case("bwd_packed", 120, H=4, lengths=[1, 15, 16, 17, 47, 0, 64, 100, 3])
    _check(w, x, d_out, d_fs, True)


def test_backward_four_tile_workgroups():
    """72 (sequence, head) pairs: the recomputed forward runs 4-tile recurrent
    workgroups, and the chunk start states it saves feed the token gradients."""
    w, x, d_out, d_fs = _case("bwd_nw4", 132, H=24, lengths=[20, 0, 37])
    _check(w, x, d_out, d_fs, True)


def test_backward_two_and_four_tile_forms_agree_bitwise():
    """As in the forward: the first 64 heads of a 68-head backward (4-tile workgroups in
    both recurrences) equal a 64-head backward of the same inputs (2-tile workgroups)
    bit for bit, every gradient."""
    torch = gu.torch_mod()
    w, x, d_out, d_fs = _case("bwd_forms", 169, H=68, T=150)
    print(f"case {w.name}: H=68 vs 64 heads", flush=True)
    got4 = gu.run_gpu_backward(gu.upload_backward(x, d_out, d_fs, False))
    sub = gu.first_heads(x, 64)
    got2 = gu.run_gpu_backward(gu.upload_backward(sub, np.ascontiguousarray(d_out[:, :64]),
                                                  np.ascontiguousarray(d_fs[:, :64]), False))
    for name in GRADS + ("d_initial_state",):
        assert torch.equal(got4[name][:, :64], got2[name]), name


@pytest.mark.parametrize("case", ["one_sequence", "packed", "four_tile", "scalar_gate"])
def test_training_forward_then_saved_backward_bitwise(case):
    """kda_chunk_prefill_for_backward gives kda_chunk_prefill's out and final state,
    and the reverse pass and token gradients on the workspace it filled give
    kda_chunk_prefill_backward's gradients, all bit for bit."""
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    spec = {"one_sequence": dict(H=5, T=150), "packed": dict(H=3, lengths=[20, 0, 37, 100]),
            "four_tile": dict(H=24, lengths=[20, 0, 37]), "scalar_gate": dict(H=4, T=90, gate_kind="scalar")}[case]
    w, x, d_out, d_fs = _case(f"train_{case}", 170, **spec)
    packed = spec.get("lengths") is not None
    print(f"case {w.name}: H={w.heads} T={w.total_tokens} N={w.num_seqs} gate={w.gate}", flush=True)
    d = gu.upload_backward(x, d_out, d_fs, packed)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    ref_out, ref_fs = kda.chunk_prefill(*args, cu_seqlens=d["cu_seqlens"], initial_state=d["initial_state"])
    out, fs, ws = kda.chunk_prefill_for_backward(*args, cu_seqlens=d["cu_seqlens"],
                                                 initial_state=d["initial_state"])
    got = kda.chunk_prefill_backward_from_saved(*args, d["d_out"], ws, cu_seqlens=d["cu_seqlens"],
                                                d_final_state=d["d_final_state"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(fs, ref_fs)
    ref = gu.run_gpu_backward(d)
    for name in GRADS + ("d_initial_state",):
        assert torch.equal(got[name], ref[name]), name


def test_training_forward_and_saved_backward_without_tokens():
    """T = 0: the training forward's final state is the initial state, and the saved
    backward's initial-state gradient is the final-state gradient."""
    torch = gu.torch_mod()
    from linear_attention_04_amd import kda

    H, N = 2, 3
    s0 = torch.randn((N, H, 128, 128), dtype=torch.float32, device="cuda")
    d_fs = torch.randn((N, H, 128, 128), dtype=torch.float32, device="cuda")
    q = torch.empty((0, H, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((0, H, 128), dtype=torch.float32, device="cuda")
    beta = torch.empty((0, H), dtype=torch.float32, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    out, fs, ws = kda.chunk_prefill_for_backward(q, q, q, g, beta, cu_seqlens=cu, initial_state=s0)
    r = kda.chunk_prefill_backward_from_saved(q, q, q, g, beta, q, ws, cu_seqlens=cu, d_final_state=d_fs)
    torch.cuda.synchronize()
    assert out.numel() == 0
    assert torch.equal(fs, s0)
    assert torch.equal(r["d_initial_state"], d_fs)


def test_backward_recurrent_grid_larger_than_the_gpu():
    """131 heads in two sequences: 528 four-tile workgroups in the recomputed forward,
    1 056 in the reverse recurrence (4-deep rings, several per CU), and odd head groups
    in the token kernels."""
    w, x, d_out, d_fs = _case("bwd_h131", 131, H=131, lengths=[20, 33])
    _check(w, x, d_out, d_fs, True)


def test_backward_more_sequences_than_one_table_block():
    """1 200 packed sequences of 0..12 tokens (the chunk table's carry across blocks)."""
    rng = np.random.default_rng(1200)
    lengths = [int(n) for n in rng.integers(0, 13, size=1200)]
    w, x, d_out, d_fs = _case("bwd_n1200", 1201, H=2, lengths=lengths)
    _check(w, x, d_out, d_fs, True)


def test_backward_scalar_gate():
    w, x, d_out, d_fs = _case("bwd_scalar", 121, H=3, T=150, gate_kind="scalar")
    _check(w, x, d_out, d_fs, False)


def test_backward_scalar_gate_packed():
    w, x, d_out, d_fs = _case("bwd_scalar_packed", 122, H=2, lengths=[40, 0, 77, 16], gate_kind="scalar")
    _check(w, x, d_out, d_fs, True)


def test_backward_no_state_no_final_gradient():
    w, x, d_out, d_fs = _case("bwd_nostate", 123, H=2, T=90, state=False)
    d, got, ref = _check(w, x, d_out, d_fs, False, use_dfs=False)
    # without them the optional output can be skipped, leaving the rest unchanged
    got2 = gu.run_gpu_backward(d, want_d_initial_state=False)
    assert got2["d_initial_state"] is None
    for name in GRADS:
        assert np.array_equal(gu.to_host(got2[name]), gu.to_host(got[name])), name


def test_backward_long_memory_gate():
    w, x, d_out, d_fs = _case("bwd_long_gate", 124, H=2, T=1000, gate=0.02)
    _check(w, x, d_out, d_fs, False)


def test_backward_all_sequences_empty():
    """T = 0: the initial-state gradient is the final-state gradient."""
    torch = gu.torch_mod()
    from linear_attention_04_amd import kda

    H, N = 2, 3
    d_fs = torch.randn((N, H, 128, 128), dtype=torch.float32, device="cuda")
    q = torch.empty((0, H, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((0, H, 128), dtype=torch.float32, device="cuda")
    beta = torch.empty((0, H), dtype=torch.float32, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    r = kda.chunk_prefill_backward(q, q, q, g, beta, q, cu_seqlens=cu, d_final_state=d_fs)
    torch.cuda.synchronize()
    assert torch.equal(r["d_initial_state"], d_fs)


@pytest.mark.parametrize("reverse_first", [False, True], ids=["in_order", "reverse_pass_first"])
def test_backward_stages_equal_one_call(reverse_first):
    """The four stage calls on one workspace give the one-call results bitwise, also
    with the reverse pass enqueued before the recomputed forward (they share no data)."""
    torch = gu.torch_mod()
    from linear_attention_04_amd import kda

    w, x, d_out, d_fs = _case("bwd_stages", 125, H=3, lengths=[33, 0, 70])
    d = gu.upload_backward(x, d_out, d_fs, True)
    one = gu.run_gpu_backward(d)
    dims = kda.make_dims(d["q"], d["v"], d["cu_seqlens"], g=d["g"])
    nbytes = kda.kda_backward_workspace_bytes(dims)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = {n: torch.empty_like(one[n]) for n in one}
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    s = torch.cuda.current_stream().cuda_stream
    assert kda.kda_backward_records(P(d["q"]), P(d["k"]), P(d["g"]), P(d["beta"]), P(d["cu_seqlens"]), dims,
                                    P(ws), nbytes, s) == 0
    def states():
        assert kda.kda_backward_states(P(d["v"]), P(d["cu_seqlens"]), P(d["initial_state"]), dims, P(ws),
                                       nbytes, s) == 0

    def state_grad():
        assert kda.kda_backward_state_grad(P(d["d_out"]), P(d["cu_seqlens"]), P(d["d_final_state"]),
                                           P(out["d_initial_state"]), dims, P(ws), nbytes, s) == 0

    for stage in ((state_grad, states) if reverse_first else (states, state_grad)):
        stage()
    assert kda.kda_backward_token_grad(P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["d_out"]),
                                       P(d["cu_seqlens"]), P(out["dq"]), P(out["dk"]), P(out["dv"]), P(out["dg"]),
                                       P(out["dbeta"]), dims, P(ws), nbytes, s) == 0
    torch.cuda.synchronize()
    for n in one:
        assert torch.equal(out[n], one[n]), n


def test_backward_graph_replay():
    """kda_chunk_prefill_backward (packed sequences) captured once in a HIP graph and
    replayed with new inputs, eager work and synchronisation between replays; every
    replay equals an eager call on fresh buffers, bitwise."""
    torch = gu.torch_mod()
    from linear_attention_04_amd import kda

    lengths = [40, 0, 77, 16]
    w, x, d_out, d_fs = _case("bwd_graph_a", 130, H=3, lengths=lengths)
    d = gu.upload_backward(x, d_out, d_fs, True)
    dims = kda.make_dims(d["q"], d["v"], d["cu_seqlens"], g=d["g"])
    nbytes = kda.kda_backward_workspace_bytes(dims)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    outs = dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["v"]),
                dg=torch.empty_like(d["g"]), dbeta=torch.empty_like(d["beta"]),
                d_initial_state=torch.empty_like(d["initial_state"]))
    P = lambda t: t.data_ptr()  # noqa: E731

    def call():
        st = kda.kda_chunk_prefill_backward(
            P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["cu_seqlens"]), P(d["initial_state"]),
            P(d["d_out"]), P(d["d_final_state"]), P(outs["dq"]), P(outs["dk"]), P(outs["dv"]), P(outs["dg"]),
            P(outs["dbeta"]), P(outs["d_initial_state"]), dims, P(ws), nbytes,
            torch.cuda.current_stream().cuda_stream)
        assert st == 0

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        _, xr, dor, dfr = _case(f"bwd_graph_r{rep}", 131 + rep, H=3, lengths=lengths)
        dr = gu.upload_backward(xr, dor, dfr, True)
        for name in ("q", "k", "v", "g", "beta", "initial_state", "d_out", "d_final_state"):
            d[name].copy_(dr[name])
        ref = gu.run_gpu_backward(dr)  # eager, on fresh buffers and a fresh workspace
        for t in outs.values():
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t, ref[name]), f"replay {rep}: {name} differs from the eager call"
