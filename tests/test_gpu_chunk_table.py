"""The device-built chunk table of a packed batch, bit for bit against its definition:
chunk_off[n] = sum over m < n of ceil(len_m / 16) (chunk_off[N] = the chunk count),
and every chunk slot labelled with its sequence (-1 past the last chunk). Both build
paths: one workgroup (up to 1 024 sequences and 65 536 chunk slots) and the gridded
passes beyond, up to the 2^20-sequence limit of include/kda.h; and a whole prefill at
that limit against the oracle."""
import numpy as np
import pytest

import oracle
from linear_attention_04_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MAX_SEQS = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()  # fails loudly when the HIP library is missing


def _expected(lengths):
    counts = (np.asarray(lengths, np.int64) + 15) // 16
    off = np.concatenate([[0], np.cumsum(counts)])
    T, N = int(np.sum(lengths)), len(lengths)
    max_chunks = (T + 15 * N) // 16
    seq = np.full(max_chunks, -1, np.int64)
    seq[:off[-1]] = np.repeat(np.arange(N), counts)
    return off, seq


def _table(lengths):
    """Build the table on the device (kda_intra_chunk, one head) and read it back
    from the workspace: chunk_off at byte 0, chunk_seq at the next 256-byte boundary."""
    import torch

    from linear_attention_04_amd import kda

    N, T = len(lengths), int(np.sum(lengths))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device="cuda")
    q = torch.zeros((T, 1, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((T, 1, 128), dtype=torch.float32, device="cuda")
    beta = torch.zeros((T, 1), dtype=torch.float32, device="cuda")
    dims = kda.make_dims(q, q, cu, g)
    nb = kda.kda_workspace_bytes(dims)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    st = kda.kda_intra_chunk(q.data_ptr(), q.data_ptr(), g.data_ptr(), beta.data_ptr(), cu.data_ptr(), dims,
                             ws.data_ptr(), nb, s)
    assert st == kda.KDA_OK
    torch.cuda.synchronize()
    max_chunks = (T + 15 * N) // 16
    off_seq = (4 * (N + 1) + 255) // 256 * 256
    off = ws[:4 * (N + 1)].view(torch.int32).cpu().numpy()
    seq = ws[off_seq:off_seq + 4 * max_chunks].view(torch.int32).cpu().numpy()
    return off, seq


@pytest.mark.parametrize("case", ["one_block", "two_blocks", "long_tail", "one_long_sequence", "limit"])
def test_chunk_table_matches_definition(case):
    rng = np.random.default_rng(["one_block", "two_blocks", "long_tail", "one_long_sequence", "limit"].index(case))
    if case == "one_block":          # the one-workgroup path
        lengths = rng.integers(0, 70, size=1000)
    elif case == "two_blocks":       # 1 025 sequences: the gridded passes, two blocks
        lengths = rng.integers(0, 70, size=1025)
    elif case == "long_tail":        # blocks of very different chunk counts, empty ones
        lengths = rng.integers(0, 5, size=9000)
        lengths[::1000] = rng.integers(1000, 5000, size=9)
        lengths[3000:5000] = 0
    elif case == "one_long_sequence":  # one sequence, more than 65 536 chunk slots
        lengths = np.array([16 * 70000 + 9])
    else:                            # the largest batch accepted
        lengths = rng.integers(0, 3, size=MAX_SEQS)
    print(f"case {case}: N={len(lengths)} T={int(np.sum(lengths))}", flush=True)
    off, seq = _table(lengths)
    want_off, want_seq = _expected(lengths)
    assert np.array_equal(off.astype(np.int64), want_off)
    assert np.array_equal(seq.astype(np.int64), want_seq)


def test_prefill_at_the_sequence_limit():
    """2^20 packed sequences of 0 .. 2 tokens, one head: every output row against the
    oracle (no states: 2^20 of them would take 64 GiB)."""
    rng = np.random.default_rng(20)
    lengths = [int(n) for n in rng.integers(0, 3, size=MAX_SEQS)]
    w = inputs.custom_workload("limit_n2e20", 2020, heads=1, lengths=lengths)
    x = inputs.generate(w)
    print(f"case limit: N={w.num_seqs} T={w.total_tokens}", flush=True)
    d = gu.upload(x, True, True)
    out, fs = gu.run_gpu(d, final_state=None)
    assert fs is None
    ro, _ = oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=x["cu_seqlens"],
                           want_state=False)
    gu.assert_close("out", gu.to_host(out), ro, True)
