"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Sizes here finish in seconds on the oracle and span several chunks, several heads
and ragged tails; the full-size workloads are in test_gpu_fullsize.py."""
import numpy as np
import pytest

from linear_attention_04_amd import inputs
from tests import gpu_util as gu
from tests import rounding_model

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()  # fails loudly when the HIP library is missing


def _case(name, seed, H, T=None, K=128, io="bf16", state=False, gate=0.1, lengths=None, gate_kind="channel"):
    w = inputs.custom_workload(name, seed, heads=H, total_tokens=T, head_k=K, head_v=K, io_dtype=io,
                               gate_scale=gate, has_initial_state=state, lengths=lengths, gate=gate_kind)
    return w, inputs.generate(w)


def _check(w, x, packed):
    print(f"case {w.name}: H={w.heads} T={w.total_tokens} K={w.head_k} io={w.io_dtype} N={w.num_seqs}",
          flush=True)
    d = gu.upload(x, w.bf16, packed)
    out, fs = gu.run_gpu(d)
    ro, rs = gu.run_oracle(x, packed)
    gu.assert_close("out", gu.to_host(out), ro, w.bf16)
    gu.assert_close("final_state", gu.to_host(fs), rs, w.bf16)
    if w.bf16 and w.total_tokens > 0:
        mo, mfs = rounding_model.forward(x if packed else dict(x, cu_seqlens=None))
        gu.assert_model_band("out", gu.to_host(out), ro, mo)
        gu.assert_model_band("final_state", gu.to_host(fs), rs, mfs)
    return d, out, fs


def test_tiny_f32_workload():
    w = inputs.WORKLOADS["tiny_f32_h2_t64_d16"]
    _check(w, inputs.generate(w), False)


@pytest.mark.parametrize("K", [16, 32, 64, 128])
def test_f32_ragged(K):
    w, x = _case(f"f32_k{K}", 30 + K, H=3, T=53, K=K, io="f32", state=True)
    _check(w, x, False)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 100, 333])
def test_bf16_lengths(T):
    w, x = _case(f"bf16_t{T}", 40 + T, H=5, T=T, state=True)
    _check(w, x, False)


def test_bf16_zero_state_many_heads():
    w, x = _case("bf16_h9", 7, H=9, T=520)
    _check(w, x, False)


def test_bf16_packed_ragged():
    w, x = _case("bf16_packed", 8, H=4, state=True, lengths=[1, 15, 16, 17, 47, 0, 64, 100, 3])
    _check(w, x, True)


def test_f32_packed():
    w, x = _case("f32_packed", 9, H=2, K=32, io="f32", state=True, lengths=[20, 5, 0, 33])
    _check(w, x, True)


def test_long_gate_workload_shape_small():
    w, x = _case("bf16_long_gate", 11, H=2, T=2000, state=True, gate=0.02)
    _check(w, x, False)


def test_null_initial_state_equals_zeros_bitwise():
    torch = gu.torch_mod()
    w, x = _case("bf16_zero", 12, H=3, T=77)
    d = gu.upload(x, True, False)
    out_a, fs_a = gu.run_gpu(d)
    d["initial_state"] = torch.zeros((1, 3, 128, 128), dtype=torch.float32, device="cuda")
    out_b, fs_b = gu.run_gpu(d)
    assert torch.equal(out_a, out_b) and torch.equal(fs_a, fs_b)


def test_null_final_state_accepted():
    torch = gu.torch_mod()
    w, x = _case("bf16_nofinal", 13, H=2, T=50, state=True)
    d = gu.upload(x, True, False)
    out_a, _ = gu.run_gpu(d)
    out_b, fs_b = gu.run_gpu(d, final_state=None)
    assert fs_b is None and torch.equal(out_a, out_b)


def test_deterministic_bitwise():
    torch = gu.torch_mod()
    w, x = _case("bf16_det", 14, H=6, T=300, state=True)
    d = gu.upload(x, True, False)
    runs = [gu.run_gpu(d) for _ in range(3)]
    for out, fs in runs[1:]:
        assert torch.equal(out, runs[0][0]) and torch.equal(fs, runs[0][1])


def test_packed_equals_separate_calls_bitwise():
    torch = gu.torch_mod()
    lens = [37, 16, 5, 80]
    w, x = _case("bf16_sep", 15, H=3, state=True, lengths=lens)
    cu = x["cu_seqlens"]
    d = gu.upload(x, True, True)
    out, fs = gu.run_gpu(d)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sub = {key: x[key][a:b] for key in ("q", "k", "v", "g", "beta")}
        sub["initial_state"] = x["initial_state"][n:n + 1]
        dn = gu.upload(sub, True, False)
        on, fn = gu.run_gpu(dn)
        assert torch.equal(on, out[a:b]), n
        assert torch.equal(fn[0], fs[n]), n


@pytest.mark.parametrize("cut", [64, 50])
def test_split_and_resume(cut):
    """Running [0, cut) and then [cut, T) from the carried fp32 state matches one
    run: bitwise when the cut is on a chunk boundary, within tolerance otherwise."""
    torch = gu.torch_mod()
    w, x = _case("bf16_split", 16, H=2, T=160, state=True)
    d = gu.upload(x, True, False)
    out, fs = gu.run_gpu(d)
    first = {key: x[key][:cut] for key in ("q", "k", "v", "g", "beta")}
    first["initial_state"] = x["initial_state"]
    o1, f1 = gu.run_gpu(gu.upload(first, True, False))
    second = {key: x[key][cut:] for key in ("q", "k", "v", "g", "beta")}
    d2 = gu.upload(second, True, False)
    d2["initial_state"] = f1
    o2, f2 = gu.run_gpu(d2)
    both = torch.cat([o1, o2])
    if cut % 16 == 0:
        assert torch.equal(both, out) and torch.equal(f2, fs)
    else:
        ro, rs = gu.run_oracle(x, False)
        gu.assert_close("out", gu.to_host(both), ro, True)
        gu.assert_close("final_state", gu.to_host(f2), rs, True)


def test_empty_input_copies_initial_state():
    torch = gu.torch_mod()
    from linear_attention_04_amd import kda

    H = 2
    z = torch.empty((0, H, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((0, H, 128), dtype=torch.float32, device="cuda")
    b = torch.empty((0, H), dtype=torch.float32, device="cuda")
    s0 = torch.randn((1, H, 128, 128), dtype=torch.float32, device="cuda")
    out, fs = kda.chunk_prefill(z, z, z, g, b, initial_state=s0)
    torch.cuda.synchronize()
    assert out.shape == (0, H, 128) and torch.equal(fs, s0)


def test_intra_chunk_intermediates_match_chunked_reference():
    """K1 alone: decode its per-(chunk, head) records and compare with the fp64
    chunked form's T' = T diag(beta), M = P T', W, Q~ = Q+ - P W, K^d and gamma."""
    torch = gu.torch_mod()
    from linear_attention_04_amd import kda
    from oracle import reference

    H, T = 3, 40
    w, x = _case("intra", 21, H=H, T=T)
    d = gu.upload(x, True, False)
    dims = kda.make_dims(d["q"], d["v"])
    ws = kda.workspace_for(dims, "cuda")
    st = kda.kda_intra_chunk(d["q"].data_ptr(), d["k"].data_ptr(), d["g"].data_ptr(), d["beta"].data_ptr(),
                             None, dims, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    n_chunks = (T + 15) // 16
    align = lambda v: (v + 255) // 256 * 256  # noqa: E731
    off = align(4 * 2) + align(4 * n_chunks)
    lane = np.arange(64)
    cl, gl = lane & 15, lane >> 4
    for h in range(H):
        _, _, inter = reference.chunked(x["q"][:, h], x["k"][:, h], x["v"][:, h], x["g"][:, h],
                                        x["beta"][:, h], None, intermediates=True)
        for ci, it in enumerate(inter):
            rec = raw[off + (ci * H + h) * 14848: off + (ci * H + h + 1) * 14848]  # [chunk][head]
            n = it["W"].shape[0]
            beta_c = x["beta"][16 * ci:16 * ci + n, h].astype(np.float64)
            tp_ref = it["T"] * beta_c[None, :]
            m_ref = it["P"] @ tp_ref
            qt_ref = it["Qp"] - it["P"] @ it["W"]

            def bf(u16):
                return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

            # the kernels' key order: row-layout element 8s + u of lane group g is
            # channel 32s + 8g + u; row r of accumulator tile m is key
            # 32(m // 2) + 8(r // 4) + 4(m % 2) + r % 4
            def key_of(m, r):
                return 32 * (m >> 1) + 8 * (r >> 2) + 4 * (m & 1) + (r & 3)

            def dec_rowlayout(base):
                a = bf(rec[base:base + 4096].view(np.uint16).reshape(4, 64, 8))
                out = np.zeros((16, 128))
                for s in range(4):
                    for u in range(8):
                        out[cl, 32 * s + 8 * gl + u] = a[s, :, u]
                return out

            def dec_tile_pairs(base):
                a = bf(rec[base:base + 4096].view(np.uint16).reshape(4, 64, 8))
                out = np.zeros((16, 128))
                for mp in range(4):
                    for u in range(8):
                        m = 2 * mp + (u >> 2)
                        out[4 * gl + (u & 3), key_of(m, cl)] = a[mp, :, u]
                return out

            def dec_hilo(base):
                a = bf(rec[base:base + 1024].view(np.uint16).reshape(64, 8))
                out = np.zeros((16, 16))
                for u in range(4):
                    out[cl, 4 * gl + u] = a[:, u] + a[:, 4 + u]
                return out

            gam = rec[14336:14848].view(np.float32).reshape(4, 32).astype(np.float64)
            gam_full = np.zeros(128)
            for gg in range(4):
                for e in range(32):
                    gam_full[key_of(e >> 2, 4 * gg + (e & 3))] = gam[gg, e]
            got = {"W": dec_rowlayout(0), "QT": dec_rowlayout(4096), "KD": dec_tile_pairs(8192),
                   "TB": dec_hilo(12288), "MM": dec_hilo(13312)}
            ref = {"W": it["W"], "QT": qt_ref, "KD": it["Kd"], "TB": tp_ref, "MM": m_ref}
            for key in got:
                gv, rv = got[key], ref[key]
                pad_rows = gv[n:]
                assert np.all(pad_rows == 0), (key, h, ci)
                if key in ("TB", "MM"):
                    assert np.all(gv[:n, n:] == 0), (key, h, ci)
                    gv, rv = gv[:n, :n], rv
                else:
                    gv = gv[:n]
                max_abs, rel = gu.errors(gv, rv)
                tol = 3e-4 if key in ("TB", "MM") else 6e-3
                assert rel <= tol, (key, h, ci, rel, max_abs)
            assert np.max(np.abs(gam_full / it["gamma"] - 1)) <= 2e-6


@pytest.mark.parametrize("T", [16, 333])
def test_bf16_scalar_gate(T):
    """g [T, H]: one decay per token and head (the scalar-gated delta rule)."""
    w, x = _case(f"bf16_sg_t{T}", 80 + T, H=5, T=T, state=True, gate_kind="scalar")
    _check(w, x, False)


def test_bf16_scalar_gate_packed():
    w, x = _case("bf16_sg_packed", 91, H=4, lengths=(40, 1, 0, 77, 16), state=True, gate_kind="scalar")
    _check(w, x, True)


@pytest.mark.parametrize("K", [16, 128])
def test_f32_scalar_gate(K):
    w, x = _case(f"f32_sg_k{K}", 95 + K, H=3, T=53, K=K, io="f32", state=True, gate_kind="scalar")
    _check(w, x, False)


def test_scalar_gate_equals_broadcast_channel_gate():
    """The scalar-gate kernels must give what the per-channel kernels give for the
    same gate repeated over the channels (both run on the GPU; bf16 io)."""
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    w, x = _case("bf16_sg_vs_cg", 99, H=3, T=200, state=True, gate_kind="scalar")
    d = gu.upload(x, True, False)
    out_s, fs_s = gu.run_gpu(d)
    d["g"] = d["g"][:, :, None].expand(-1, -1, 128).contiguous()
    out_c, fs_c = gu.run_gpu(d)
    gu.assert_close("out", gu.to_host(out_s), gu.to_host(out_c).astype(np.float64), True)
    gu.assert_close("final_state", gu.to_host(fs_s), gu.to_host(fs_c), True)
    assert kda.KDA_GATE_SCALAR == 1


def _fused_vs_split(w, x, packed):
    """The single-kernel ablation runs the same per-wave arithmetic as the two-kernel
    path, so its results must be bitwise equal; the split path is itself checked
    against the oracle."""
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    print(f"case fused {w.name}: H={w.heads} T={w.total_tokens} N={w.num_seqs} gate={w.gate}", flush=True)
    d = gu.upload(x, True, packed)
    out_s, fs_s = gu.run_gpu(d)
    out_f, fs_f = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                                    initial_state=d["initial_state"], fused=True)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_f), "fused out differs from the two-kernel path"
    assert torch.equal(fs_s, fs_f), "fused final state differs from the two-kernel path"


@pytest.mark.parametrize("T", [1, 16, 17, 333])
def test_fused_equals_split_bitwise(T):
    w, x = _case(f"fused_t{T}", 120 + T, H=5, T=T, state=True)
    _fused_vs_split(w, x, False)


def test_fused_packed_ragged_and_scalar_gate():
    w, x = _case("fused_packed", 131, H=4, state=True, lengths=[1, 15, 16, 17, 47, 0, 64, 100, 3])
    _fused_vs_split(w, x, True)
    w, x = _case("fused_sg", 132, H=3, T=200, state=True, gate_kind="scalar")
    _fused_vs_split(w, x, False)


def test_fused_matches_oracle():
    w, x = _case("fused_oracle", 133, H=6, T=300, state=True)
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    d = gu.upload(x, True, False)
    out, fs = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"],
                                fused=True)
    torch.cuda.synchronize()
    ro, rs = gu.run_oracle(x, False)
    gu.assert_close("out", gu.to_host(out), ro, True)
    gu.assert_close("final_state", gu.to_host(fs), rs, True)


@pytest.mark.parametrize("H", [1, 3, 7])
def test_bf16_head_counts_not_multiple_of_four(H):
    """Head counts that leave idle waves in the intra-chunk workgroups and idle
    workgroups in the recurrent grid (rounded up to 8 (sequence, head) pairs)."""
    w, x = _case(f"bf16_h{H}", 140 + H, H=H, T=70, state=True)
    _check(w, x, False)


def test_bf16_four_tile_workgroups():
    """120 (sequence, head) pairs: too many for one 2-tile recurrent workgroup per CU,
    so 4-tile ones (four compute waves sharing one record stream, and a wave that
    stores their outputs from LDS), with ragged and empty packed sequences."""
    w, x = _case("bf16_nw4", 124, H=24, state=True, lengths=[1, 15, 0, 33, 100])
    _check(w, x, True)


def test_bf16_four_tile_staged_output_chunk_counts():
    """The 4-tile form's outputs leave through LDS staging buffers (two, used in turn)
    and a store wave that takes the last chunk's after one extra barrier: sequences of
    one, two, three and four chunks, full and short last chunks, at 144 pairs."""
    w, x = _case("bf16_nw4_stage", 125, H=24, state=True, lengths=[16, 17, 32, 2, 48, 31])
    _check(w, x, True)


@pytest.mark.parametrize("lengths", [None, [37, 150]])
def test_two_and_four_tile_forms_agree_bitwise(lengths):
    """Each head's results depend only on its own inputs, and the intra-chunk kernel
    groups heads in fours either way. So the first 64 (sequence, head) pairs of a batch
    past 64 pairs (4-tile recurrent workgroups) equal the same pairs run alone (2-tile
    workgroups) bit for bit: the two forms share every product, accumulation order and
    rounding."""
    torch = gu.torch_mod()
    H = 68 if lengths is None else 34
    w, x = _case("bf16_forms", 168, H=H, T=200 if lengths is None else None, state=True, lengths=lengths)
    packed = lengths is not None
    n = 64 // w.num_seqs
    print(f"case {w.name}: H={H} vs {n} heads, N={w.num_seqs}", flush=True)
    out4, fs4 = gu.run_gpu(gu.upload(x, True, packed))
    out2, fs2 = gu.run_gpu(gu.upload(gu.first_heads(x, n), True, packed))
    assert torch.equal(out4[:, :n], out2)
    assert torch.equal(fs4[:, :n], fs2)


def test_bf16_recurrent_grid_larger_than_the_gpu():
    """257 heads in two sequences: 514 (sequence, head) pairs, rounded up to 520 in the
    XCD-grouped order, i.e. 1 040 four-tile recurrent workgroups, four rounds of 256 CUs."""
    w, x = _case("bf16_h257", 257, H=257, state=True, lengths=[37, 29])
    _check(w, x, True)


def test_bf16_many_short_sequences():
    """150 packed sequences of 0..40 tokens (many empty or shorter than a chunk)."""
    rng = np.random.default_rng(150)
    lengths = [int(n) for n in rng.integers(0, 41, size=150)]
    lengths[0], lengths[-1] = 0, 0
    w, x = _case("bf16_many", 151, H=3, state=True, lengths=lengths)
    _check(w, x, True)


def test_bf16_more_sequences_than_one_table_block():
    """1 500 packed sequences of 0..20 tokens: the chunk table scans the boundaries in
    blocks of 1 024 sequences and carries the chunk count from one block to the next."""
    rng = np.random.default_rng(1500)
    lengths = [int(n) for n in rng.integers(0, 21, size=1500)]
    w, x = _case("bf16_n1500", 1501, H=2, state=True, lengths=lengths)
    _check(w, x, True)


def test_prefill_graph_replay():
    """kda_chunk_prefill captured once in a HIP graph and replayed with new inputs,
    eager work and synchronisation between replays; every replay equals the eager call."""
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    w, x = _case("graph_a", 160, H=4, T=200, state=True)
    d = gu.upload(x, True, False)
    dims = kda.make_dims(d["q"], d["v"])
    ws = kda.workspace_for(dims, "cuda")
    out = torch.empty_like(d["v"])
    fs = torch.empty_like(d["initial_state"])
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"], out=out,
                      final_state=fs, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"], out=out,
                          final_state=fs, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        _, xr = _case(f"graph_r{rep}", 161 + rep, H=4, T=200, state=True)
        dr = gu.upload(xr, True, False)
        for name in ("q", "k", "v", "g", "beta", "initial_state"):
            d[name].copy_(dr[name])
        ref_out, ref_fs = gu.run_gpu(dr)  # eager, on fresh buffers
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(fs, ref_fs), f"replay {rep} differs from the eager call"
