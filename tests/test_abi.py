"""The C ABI: the library loads without a GPU, exports what include/ckda.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ckda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ckda_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from gated_delta_rule_sign_amd import ckda
    return ckda.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.ckda_abi_version() == 7
    assert L.ckda_status_string(0) == b"ok"
    for st in range(1, 8):
        assert L.ckda_status_string(st) not in (b"ok", b"unknown status")
    assert L.ckda_status_string(99) == b"unknown status"


P = ctypes.c_void_p
FAKE = P(0x1000)          # never dereferenced: every call below fails validation first


BIG = 1 << 40


def fwd(L, B=1, T=8, H=1, DK=32, DV=32, dt=0, q=FAKE, k=FAKE, v=FAKE, g=FAKE, s=FAKE, beta=FAKE, o=FAKE,
        ws=FAKE, wsb=BIG, gate=0):
    return L.ckda_fwd_chunked(B, T, H, DK, DV, dt, gate, q, k, v, g, s, beta, ctypes.c_float(1.0),
                              None, o, None, None, ws, ctypes.c_size_t(wsb), None)


def test_fwd_rejects_bad_arguments(L):
    assert fwd(L, DK=48) == 4                    # unsupported head size
    assert fwd(L, DV=256) == 4
    assert fwd(L, DK=0) == 2
    assert fwd(L, B=-1) == 2
    assert fwd(L, dt=7) == 3
    assert fwd(L, q=None) == 1
    assert b"'q'" in L.ckda_last_error()
    assert fwd(L, o=None) == 1
    assert fwd(L, T=0, o=None, q=None) != 1      # no tokens: o and q are not needed
    assert fwd(L, g=P(0x1004)) == 4              # misaligned
    assert fwd(L, gate=4) == 4                   # unknown flag bit
    assert fwd(L, gate=0x80000000) == 4          # unknown flag bit
    assert fwd(L, B=0) == 0                      # empty problem: nothing to do
    assert L.ckda_last_error() == b""


def align256(x):
    return (x + 255) // 256 * 256


def seg_bytes(nsslots, H, DK, DV):
    """Segment buffers: start states and zero-start end states (DK x DV each)
    and segment maps (DK x DK), fp32, per segment slot and head."""
    return nsslots * H * (2 * DK * DV + DK * DK) * 4


def bwd_block_bytes(DK, DV):
    """Backward workspace per chunk-head: 9 [64 x DK], 6 [64 x DV], 1 [DK x DV]
    and 10 [64 x 64] fp32 matrices, 3 [DK] and 3 [64] vectors."""
    return 4 * (9 * 64 * DK + 6 * 64 * DV + DK * DV + 10 * 64 * 64 + 3 * DK + 3 * 64)


def test_fwd_workspace(L):
    need = L.ckda_fwd_workspace_bytes(2, 100, 3, 64, 32, 1)
    # one record per (chunk, head): bf16 keeps W, Qh, KbT and M as hi/lo planes
    rec = 2 * (64 * 64 * 2) * 4 + 64 * 4 + 64 * 32 * 4
    # then the segment buffers for segments of 16 chunks: ceil(2/16) per sequence
    assert need == align256(2 * 2 * 3 * rec) + seg_bytes(2 * 1, 3, 64, 32)
    # fp32 records hold every matrix element in 4 bytes too (one fp32 plane)
    assert L.ckda_fwd_workspace_bytes(2, 100, 3, 64, 32, 0) == need
    assert L.ckda_fwd_workspace_bytes(2, 100, 3, 48, 32, 1) == 0       # unsupported head size
    assert L.ckda_fwd_workspace_bytes(2, 0, 3, 64, 32, 1) == 0         # no chunks
    # varlen: ceil(100/64) + 3 chunk slots, ceil(100/1024) + 3 segment slots
    assert L.ckda_fwd_varlen_workspace_bytes(3, 100, 3, 64, 32, 1) == \
        align256((2 + 3) * 3 * rec) + seg_bytes(1 + 3, 3, 64, 32)
    assert fwd(L, ws=None) == 1
    assert b"workspace" in L.ckda_last_error()
    # below the records (fp32, DK = DV = 32: W, Qh, KbT, M, d, u) the call fails
    rec32 = 64 * 32 * 4 * 3 + 64 * 64 * 4 + 32 * 4 + 64 * 32 * 4
    assert fwd(L, wsb=rec32 - 16) == 6
    assert fwd(L, ws=P(0x1008)) == 4             # misaligned workspace


def test_segment_knob(L):
    assert L.ckda_set_segment_chunks(8) == 4     # shorter than 16 chunks
    assert b"16" in L.ckda_last_error()
    for G in (16, 100, -1, 0):
        assert L.ckda_set_segment_chunks(G) == 0


def test_varlen_rejects_bad_cu_seqlens(L):
    def call(cu, N, Tt):
        arr = (ctypes.c_int32 * len(cu))(*cu)
        return L.ckda_fwd_varlen(N, Tt, arr, FAKE, 1, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 ctypes.c_float(1.0), None, FAKE, None, None, FAKE, ctypes.c_size_t(BIG), None)
    assert call([1, 5], 1, 5) == 5              # does not start at 0
    assert call([0, 5, 3], 2, 3) == 5           # decreasing
    assert call([0, 5, 9], 2, 10) == 5          # does not end at T_total
    assert L.ckda_fwd_varlen(2, 4, None, FAKE, 1, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             ctypes.c_float(1.0), None, FAKE, None, None, FAKE, ctypes.c_size_t(BIG), None) == 1


def bwd_varlen(L, cu, N, Tt, DK=32, DV=32, dt=0, ws=FAKE, wsb=BIG, q=FAKE, hc=FAKE):
    arr = None if cu is None else (ctypes.c_int32 * len(cu))(*cu)
    f = ctypes.c_float(1.0)
    return L.ckda_bwd_varlen(N, Tt, arr, FAKE, 1, DK, DV, dt, 0, q, FAKE, FAKE, FAKE, FAKE, FAKE, f, None,
                             hc, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, ctypes.c_size_t(wsb), None)


def test_varlen_backward_boundary(L):
    # chunk slots: ceil(T_total / 64) + N; one workspace block per (slot, head)
    assert L.ckda_varlen_chunk_slots(3, 100) == 2 + 3
    assert L.ckda_varlen_chunk_slots(-1, 100) == 0
    # one backward workspace block per (chunk slot, head), then the segment
    # buffers of the reverse pass (segments of 16 chunks)
    # then room for recomputed checkpoints (one DK x DV state per block)
    one = bwd_block_bytes(64, 32)
    assert L.ckda_bwd_workspace_bytes(1, 64, 1, 64, 32) == \
        align256(one) + align256(64 * 32 * 4) + seg_bytes(1, 1, 64, 32)
    assert L.ckda_bwd_varlen_workspace_bytes(3, 100, 2, 64, 32) == \
        align256((2 + 3) * 2 * one) + align256((2 + 3) * 2 * 64 * 32 * 4) + seg_bytes(1 + 3, 2, 64, 32)
    assert L.ckda_bwd_varlen_workspace_bytes(3, 100, 2, 48, 32) == 0
    assert bwd_varlen(L, [1, 5], 1, 5) == 5                       # does not start at 0
    assert bwd_varlen(L, [0, 5, 3], 2, 3) == 5                    # decreasing
    assert bwd_varlen(L, None, 2, 4) == 1
    assert bwd_varlen(L, [0, 5], 1, 5, DK=96) == 4
    assert bwd_varlen(L, [0, 5], 1, 5, dt=9) == 3
    # no checkpoints: recomputed, which needs room for them beyond the blocks
    assert bwd_varlen(L, [0, 5], 1, 5, hc=None, wsb=2 * bwd_block_bytes(32, 32)) == 6
    assert b"recomputed" in L.ckda_last_error()
    assert bwd_varlen(L, [0, 5], 1, 5, q=P(0x1004)) == 4          # misaligned
    # below the per-chunk blocks (2 chunk slots) the call fails before any launch
    assert bwd_varlen(L, [0, 5], 1, 5, wsb=2 * bwd_block_bytes(32, 32) - 16) == 6
    assert bwd_varlen(L, [0], 0, 0) == 0                          # no documents


def test_decode_and_bwd_reject_bad_arguments(L):
    f = ctypes.c_float(1.0)
    assert L.ckda_decode_step(4, 2, 96, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, FAKE, FAKE, FAKE, None) == 4
    assert L.ckda_decode_step(4, 2, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, None, FAKE, FAKE, None) == 1
    assert L.ckda_decode_step(4, 2, 32, 32, 0, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, FAKE, FAKE, FAKE, None) == 4
    assert b"flags" in L.ckda_last_error()
    assert L.ckda_bwd(1, 8, 1, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, None, None, FAKE, None,
                      FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1   # h_ckpt missing
    assert L.ckda_chunk_prep(1, 8, 1, 100, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 4


def test_size_limits(L):
    """Token-head, chunk-head and state counts must fit the kernels' 32-bit
    chain and token indices; larger problems fail before any pointer is used."""
    f = ctypes.c_float(1.0)
    assert fwd(L, B=1 << 16, T=1 << 16, H=1) == 4            # 2^32 token-heads
    assert b"too large" in L.ckda_last_error()
    assert fwd(L, B=1 << 16, T=0, H=1 << 15) == 4            # 2^31 (sequence, head) states
    assert b"too many heads" in L.ckda_last_error()
    cu = (ctypes.c_int32 * 2)(0, 1 << 30)
    assert L.ckda_fwd_varlen(1, 1 << 30, cu, FAKE, 4, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, None,
                             FAKE, None, None, FAKE, ctypes.c_size_t(BIG), None) == 4
    assert b"too large" in L.ckda_last_error()
    assert L.ckda_decode_step(1 << 20, 1 << 11, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f,
                              FAKE, FAKE, FAKE, None) == 4
    assert b"too many heads" in L.ckda_last_error()
    assert L.ckda_bwd(1 << 16, 1 << 16, 1, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, None, FAKE,
                      FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ctypes.c_size_t(BIG), None) == 4
    assert b"too large" in L.ckda_last_error()
    assert L.ckda_bwd(1 << 16, 0, 1 << 15, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, None, FAKE,
                      FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ctypes.c_size_t(BIG), None) == 4
    assert b"too many heads" in L.ckda_last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from gated_delta_rule_sign_amd import ckda
    monkeypatch.setattr(ckda, "_lib", None)
    monkeypatch.setattr(ckda, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ckda.CkdaError):
        ckda.lib()
