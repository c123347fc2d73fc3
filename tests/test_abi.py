"""The C ABI without a GPU: libkda.so loads, exports every function include/kda.h
declares, and its host-side logic (sizes, argument checks, status strings) behaves
as documented. Every call here returns before anything is enqueued."""
import ctypes
import os
import re

import pytest

from linear_attention_04_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from linear_attention_04_amd import build

        build.build()
    return kda.load_library()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(kda.EXPORTS)


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert kda.kda_version() >= 200
    for st in (kda.KDA_OK, kda.KDA_ERR_ARG, kda.KDA_ERR_UNSUPPORTED, kda.KDA_ERR_ALIGN,
               kda.KDA_ERR_WORKSPACE, kda.KDA_ERR_LAUNCH, kda.KDA_ERR_CAPACITY):
        s = kda.kda_status_string(st)
        assert isinstance(s, str) and s
    assert kda.kda_status_string(12345)


def dims(T=64, H=2, K=128, V=128, N=1, io=kda.KDA_IO_BF16, gate=kda.KDA_GATE_CHANNEL):
    return kda.KdaDims(T, H, K, V, N, io, gate)


def test_workspace_bytes(lib):
    a = kda.kda_workspace_bytes(dims(T=64))
    b = kda.kda_workspace_bytes(dims(T=6400))
    assert 0 < a < b
    # chunk records grow linearly with the chunk count (16 tokens) and the heads
    assert kda.kda_workspace_bytes(dims(T=6400, H=4)) > b
    assert kda.kda_workspace_bytes(dims(gate=kda.KDA_GATE_SCALAR)) == a
    assert kda.kda_workspace_bytes(dims(io=kda.KDA_IO_F32, K=16, V=16)) > 0
    # invalid or unsupported sizes give 0
    assert kda.kda_workspace_bytes(dims(K=64, V=64)) == 0          # bf16 needs K = V = 128
    assert kda.kda_workspace_bytes(dims(io=kda.KDA_IO_F32, K=16, V=32)) == 0
    assert kda.kda_workspace_bytes(dims(H=0)) == 0
    assert kda.kda_workspace_bytes(dims(T=-1)) == 0
    assert kda.kda_workspace_bytes(dims(gate=7)) == 0
    assert kda.kda_workspace_bytes(dims(io=9)) == 0


def test_size_limits(lib):
    # the largest accepted sizes (include/kda.h): 2^31 - 1 tokens, 2^16 heads, 2^20
    # packed sequences, N * H < 2^25
    assert kda.kda_workspace_bytes(dims(T=(1 << 31) - 1)) > 0
    assert kda.kda_workspace_bytes(dims(H=1 << 16)) > 0
    assert kda.kda_workspace_bytes(dims(N=1 << 20, T=1 << 24, H=1)) > 0
    assert kda.kda_workspace_bytes(dims(N=1 << 20, T=1 << 24, H=31)) > 0
    assert kda.kda_workspace_bytes(dims(N=(1 << 20) - 1, T=1 << 24, H=32)) > 0
    # one past each limit is rejected (no size computation overflows into a small workspace)
    assert kda.kda_workspace_bytes(dims(T=1 << 31)) == 0
    assert kda.kda_workspace_bytes(dims(H=(1 << 16) + 1)) == 0
    assert kda.kda_workspace_bytes(dims(N=(1 << 20) + 1, T=1 << 25, H=1)) == 0
    assert kda.kda_workspace_bytes(dims(N=1 << 20, T=1 << 24, H=32)) == 0       # N * H = 2^25
    assert kda.kda_workspace_bytes(dims(N=0)) == 0
    b = Buf()
    p = b.at()
    big = dims(T=1 << 31)
    assert kda.kda_chunk_prefill(p, p, p, p, p, None, None, p, None, big, p, 1 << 60, None) == kda.KDA_ERR_ARG
    # the workspace for the largest sizes is what the records need, not a wrapped-around value
    per_chunk_head = 14848
    n = kda.kda_workspace_bytes(dims(T=(1 << 31) - 1, H=64))
    assert n >= ((1 << 31) // 16) * 64 * per_chunk_head


class Buf:
    """Host memory standing in for device pointers: the calls below fail their
    checks before anything dereferences them."""

    def __init__(self, n=1 << 16):
        self.raw = ctypes.create_string_buffer(n + 64)
        base = ctypes.addressof(self.raw)
        self.ptr = (base + 63) // 64 * 64

    def at(self, off=0):
        return self.ptr + off


def test_prefill_argument_checks(lib):
    b = Buf()
    p = b.at()
    d = dims()
    ws_need = kda.kda_workspace_bytes(d)
    # missing required pointer
    assert kda.kda_chunk_prefill(None, p, p, p, p, None, None, p, None, d, p, ws_need, None) == kda.KDA_ERR_ARG
    # misaligned pointer
    assert kda.kda_chunk_prefill(b.at(4), p, p, p, p, None, None, p, None, d, p, ws_need, None) == kda.KDA_ERR_ALIGN
    # workspace too small or missing
    assert kda.kda_chunk_prefill(p, p, p, p, p, None, None, p, None, d, p, ws_need - 1, None) == \
        kda.KDA_ERR_WORKSPACE
    assert kda.kda_chunk_prefill(p, p, p, p, p, None, None, p, None, d, None, ws_need, None) == \
        kda.KDA_ERR_WORKSPACE
    # several sequences need cu_seqlens
    d2 = dims(N=2)
    assert kda.kda_chunk_prefill(p, p, p, p, p, None, None, p, None, d2, p, 1 << 40, None) == kda.KDA_ERR_ARG
    # unsupported head size
    assert kda.kda_chunk_prefill(p, p, p, p, p, None, None, p, None, dims(K=64, V=64), p, 1 << 40, None) == \
        kda.KDA_ERR_UNSUPPORTED
    # the two halves check the same way
    assert kda.kda_intra_chunk(None, p, p, p, None, d, p, ws_need, None) == kda.KDA_ERR_ARG
    assert kda.kda_inter_chunk(p, None, None, None, None, d, p, ws_need, None) == kda.KDA_ERR_ARG
    assert kda.kda_inter_chunk(p, None, b.at(8), p, None, d, p, ws_need, None) == kda.KDA_ERR_ALIGN


def test_decode_argument_checks(lib):
    b = Buf()
    p = b.at()
    ok = dims(T=4, N=4)
    # B = 0 is a no-op that succeeds without touching anything
    assert kda.kda_decode_step(None, None, None, None, None, None, None, dims(T=0, N=0), None) == kda.KDA_OK
    assert kda.kda_decode_step(None, p, p, p, p, p, p, ok, None) == kda.KDA_ERR_ARG
    assert kda.kda_decode_step(p, p, p, p, p, b.at(4), p, ok, None) == kda.KDA_ERR_ALIGN
    # one token per sequence
    assert kda.kda_decode_step(p, p, p, p, p, p, p, dims(T=4, N=2), None) == kda.KDA_ERR_ARG
    assert kda.kda_decode_step(p, p, p, p, p, p, p, dims(T=4, N=4, K=64, V=64), None) == kda.KDA_ERR_UNSUPPORTED
    assert kda.kda_decode_step(p, p, p, p, p, p, p, dims(T=4, N=4, gate=3), None) == kda.KDA_ERR_ARG


def test_backward_workspace_bytes(lib):
    from tests import gpu_util as gu

    for T, H, N in ((64, 2, 1), (8192, 64, 1), (300, 5, 7), (0, 3, 2)):
        d = dims(T=T, H=H, N=N)
        assert kda.kda_backward_workspace_bytes(d) == gu.backward_workspace_layout(T, H, N)["total"]
        assert kda.kda_backward_workspace_bytes(d) > kda.kda_workspace_bytes(d)
    # bf16 only; invalid sizes give 0
    assert kda.kda_backward_workspace_bytes(dims(io=kda.KDA_IO_F32, K=16, V=16)) == 0
    assert kda.kda_backward_workspace_bytes(dims(K=64, V=64)) == 0
    assert kda.kda_backward_workspace_bytes(dims(H=0)) == 0


def test_backward_argument_checks(lib):
    b = Buf()
    p = b.at()
    d = dims()
    need = kda.kda_backward_workspace_bytes(d)
    ok = [p] * 5 + [None, None, p, None] + [p] * 5 + [None]
    assert kda.kda_chunk_prefill_backward(*ok, d, p, need - 1, None) == kda.KDA_ERR_WORKSPACE
    bad = list(ok)
    bad[7] = None  # d_out
    assert kda.kda_chunk_prefill_backward(*bad, d, p, need, None) == kda.KDA_ERR_ARG
    bad = list(ok)
    bad[10] = b.at(4)  # dk misaligned
    assert kda.kda_chunk_prefill_backward(*bad, d, p, need, None) == kda.KDA_ERR_ALIGN
    bad = list(ok)
    bad[14] = b.at(8)  # d_initial_state misaligned
    assert kda.kda_chunk_prefill_backward(*bad, d, p, need, None) == kda.KDA_ERR_ALIGN
    assert kda.kda_chunk_prefill_backward(*ok, dims(N=2), p, 1 << 40, None) == kda.KDA_ERR_ARG
    assert kda.kda_chunk_prefill_backward(*ok, dims(io=kda.KDA_IO_F32, K=16, V=16), p, 1 << 40, None) == \
        kda.KDA_ERR_UNSUPPORTED


def test_backward_stage_argument_checks(lib):
    b = Buf()
    p = b.at()
    d = dims()
    need = kda.kda_backward_workspace_bytes(d)
    assert kda.kda_backward_records(None, p, p, p, None, d, p, need, None) == kda.KDA_ERR_ARG
    assert kda.kda_backward_records(p, p, p, p, None, d, p, need - 1, None) == kda.KDA_ERR_WORKSPACE
    assert kda.kda_backward_states(None, None, None, d, p, need, None) == kda.KDA_ERR_ARG
    assert kda.kda_backward_states(p, None, b.at(4), d, p, need, None) == kda.KDA_ERR_ALIGN
    assert kda.kda_backward_state_grad(None, None, None, None, d, p, need, None) == kda.KDA_ERR_ARG
    assert kda.kda_backward_state_grad(p, None, p, b.at(8), d, p, need, None) == kda.KDA_ERR_ALIGN
    assert kda.kda_backward_token_grad(p, p, p, p, p, p, None, p, p, None, p, p, d, p, need, None) == \
        kda.KDA_ERR_ARG
    assert kda.kda_backward_token_grad(*([p] * 6), None, *([p] * 5), dims(K=64, V=64), p, need, None) == \
        kda.KDA_ERR_UNSUPPORTED


def test_training_forward_argument_checks(lib):
    b = Buf()
    p = b.at()
    d = dims()
    need = kda.kda_backward_workspace_bytes(d)
    ok = [p] * 5 + [None, None, p, None]  # q, k, v, g, beta, cu_seqlens, initial_state, out, final_state
    # the forward's own workspace is too small: it fills the backward workspace
    assert kda.kda_chunk_prefill_for_backward(*ok, d, p, kda.kda_workspace_bytes(d), None) == \
        kda.KDA_ERR_WORKSPACE
    assert kda.kda_chunk_prefill_for_backward(*ok, d, p, need - 1, None) == kda.KDA_ERR_WORKSPACE
    bad = list(ok)
    bad[7] = None  # out
    assert kda.kda_chunk_prefill_for_backward(*bad, d, p, need, None) == kda.KDA_ERR_ARG
    bad = list(ok)
    bad[6] = b.at(4)  # initial_state misaligned
    assert kda.kda_chunk_prefill_for_backward(*bad, d, p, need, None) == kda.KDA_ERR_ALIGN
    assert kda.kda_chunk_prefill_for_backward(*ok, dims(N=2), p, 1 << 40, None) == kda.KDA_ERR_ARG
    assert kda.kda_chunk_prefill_for_backward(*ok, dims(io=kda.KDA_IO_F32, K=16, V=16), p, 1 << 40, None) == \
        kda.KDA_ERR_UNSUPPORTED


def test_check_seqlens_argument_checks(lib):
    b = Buf()
    p = b.at()
    assert kda.kda_check_seqlens(None, 1, 16, p, None) == kda.KDA_ERR_ARG
    assert kda.kda_check_seqlens(p, 1, 16, None, None) == kda.KDA_ERR_ARG
    assert kda.kda_check_seqlens(p, 0, 16, p, None) == kda.KDA_ERR_ARG
    assert kda.kda_check_seqlens(p, (1 << 20) + 1, 16, p, None) == kda.KDA_ERR_ARG
    assert kda.kda_check_seqlens(p, 1, -1, p, None) == kda.KDA_ERR_ARG
    assert kda.kda_check_seqlens(p, 1, 1 << 31, p, None) == kda.KDA_ERR_ARG
    # int32 arrays need 4-byte alignment only
    assert kda.kda_check_seqlens(b.at(2), 1, 16, p, None) == kda.KDA_ERR_ALIGN
    assert kda.kda_check_seqlens(p, 1, 16, b.at(6), None) == kda.KDA_ERR_ALIGN


def test_one_library_per_process(lib, tmp_path):
    # without a path, or with the loaded one's, the loaded library comes back; a second
    # copy from another path is refused
    assert kda.load_library() is lib
    assert kda.load_library(os.path.join(ROOT, "linear_attention_04_amd", "..", "linear_attention_04_amd",
                                         "libkda.so")) is lib
    other = tmp_path / "libkda_copy.so"
    other.write_bytes(open(kda.LIB_PATH, "rb").read())
    with pytest.raises(RuntimeError, match="already loaded"):
        kda.load_library(str(other))


def test_library_binds_to_the_hip_runtime_torch_loaded():
    # loaded first thing in a fresh interpreter, the library must not bring a second
    # HIP runtime into the process next to torch's
    import ast
    import subprocess
    import sys

    code = ("from linear_attention_04_amd import kda; kda.load_library(); "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    runtimes = ast.literal_eval(r.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes


def test_noalloc_argument_checks(lib):
    """kda_chunk_prefill_noalloc rejects bad arguments and problems beyond its fixed
    buffer before it looks the buffer up or enqueues anything."""
    f = kda.kda_chunk_prefill_noalloc
    fake = 1 << 20  # an aligned non-NULL address that is never dereferenced
    ptrs = [fake] * 5
    assert f(*ptrs, None, None, fake, None, dims(H=0), None) == kda.KDA_ERR_ARG
    assert f(*ptrs, None, None, fake, None, dims(K=64, V=64), None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*ptrs, None, None, fake, None, dims(N=2), None) == kda.KDA_ERR_ARG  # N > 1 needs cu_seqlens
    assert f(None, *ptrs[1:], None, None, fake, None, dims(), None) == kda.KDA_ERR_ARG
    assert f(fake + 8, *ptrs[1:], None, None, fake, None, dims(), None) == kda.KDA_ERR_ALIGN
    # a packed batch whose workspace exceeds the buffer (2 x 8192 tokens x 64 heads)
    big = dims(T=16384, H=64, N=2)
    assert kda.kda_workspace_bytes(big) > kda.KDA_NOALLOC_SCRATCH_BYTES
    assert f(*ptrs, fake, None, fake, None, big, None) == kda.KDA_ERR_CAPACITY
    # one sequence with so many heads that two fp32 state carriers fill the buffer
    assert f(*ptrs, None, None, fake, None, dims(T=64, H=4096), None) == kda.KDA_ERR_CAPACITY
