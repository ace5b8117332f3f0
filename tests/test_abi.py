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
    assert L.ckda_abi_version() == 12
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
    assert fwd(L, gate=8) == 4                   # unknown flag bit
    assert fwd(L, gate=0x80000000) == 4          # unknown flag bit
    assert fwd(L, B=0) == 0                      # empty problem: nothing to do
    assert L.ckda_last_error() == b""


def align256(x):
    return (x + 255) // 256 * 256


def seg_bytes(nsslots, H, DK, DV):
    """Segment buffers: start states and zero-start end states (DK x DV each)
    and segment maps (DK x DK), fp32, per segment slot and head."""
    return nsslots * H * (2 * DK * DV + DK * DK) * 4


def bwd_layout(NC, DK, DV):
    """Backward workspace for NC chunk-heads: (bytes without checkpoint room,
    checkpoint room).  Per chunk-head one block of the larger of the reverse
    record (KB [64 x DK], Qh^T and W^T [DK x 64], M^T [64 x 64] at 4 bytes an
    element, d [DK] fp32, a flag word) and the first gradient phase's output
    (dA, dM [64 x 64] and U [64 x DV] at 4 bytes), each padded to 256 bytes;
    then dU [64 x DV], G [max(DK, 64) x DV] and a flag word per chunk-head;
    then the checkpoints [DK x DV], fp32, each region 256-byte aligned."""
    rev = align256(4 * (3 * 64 * DK + 64 * 64) + 4 * DK + 4)
    go = align256(4 * (2 * 64 * 64 + 64 * DV))
    base = (align256(NC * max(rev, go)) + align256(NC * 64 * DV * 4) + align256(NC * max(DK, 64) * DV * 4)
            + align256(NC * 4))
    return base, align256(NC * DK * DV * 4)


def test_fwd_workspace(L):
    need = L.ckda_fwd_workspace_bytes(2, 100, 3, 64, 32, 1)
    # one record per (chunk, head): bf16 keeps W, Qh, KbT and M as hi/lo planes,
    # then d, u and a flag word, padded to a multiple of 256 bytes
    rec = align256(2 * (64 * 64 * 2) * 4 + 64 * 4 + 64 * 32 * 4 + 4)
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
    # below the records (fp32, DK = DV = 32: W, Qh, KbT, M, d, u, flag) the call fails
    rec32 = align256(64 * 32 * 4 * 3 + 64 * 64 * 4 + 32 * 4 + 64 * 32 * 4 + 4)
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
    # per-chunk-head blocks and buffers, room for recomputed checkpoints, then
    # the segment buffers of the reverse pass (segments of 16 chunks)
    assert L.ckda_bwd_workspace_bytes(1, 64, 1, 64, 32) == sum(bwd_layout(1, 64, 32)) + seg_bytes(1, 1, 64, 32)
    assert L.ckda_bwd_workspace_bytes(2, 100, 3, 32, 128) == \
        sum(bwd_layout(2 * 2 * 3, 32, 128)) + seg_bytes(2 * 1, 3, 32, 128)
    assert L.ckda_bwd_varlen_workspace_bytes(3, 100, 2, 64, 32) == \
        sum(bwd_layout((2 + 3) * 2, 64, 32)) + seg_bytes(1 + 3, 2, 64, 32)
    assert L.ckda_bwd_varlen_workspace_bytes(3, 100, 2, 48, 32) == 0
    # with the caller's checkpoints the segment buffers take the checkpoint
    # room's place
    assert L.ckda_bwd_workspace_bytes_given_ckpt(1, 64, 1, 64, 32) == bwd_layout(1, 64, 32)[0] + seg_bytes(1, 1, 64, 32)
    assert L.ckda_bwd_workspace_bytes_given_ckpt(2, 100, 3, 32, 128) == \
        bwd_layout(2 * 2 * 3, 32, 128)[0] + seg_bytes(2 * 1, 3, 32, 128)
    assert L.ckda_bwd_varlen_workspace_bytes_given_ckpt(3, 100, 2, 64, 32) == \
        bwd_layout((2 + 3) * 2, 64, 32)[0] + seg_bytes(1 + 3, 2, 64, 32)
    assert L.ckda_bwd_workspace_bytes_given_ckpt(1, 64, 1, 96, 32) == 0
    assert L.ckda_bwd_varlen_workspace_bytes_given_ckpt(-1, 100, 2, 64, 32) == 0
    # layer_bwd (B=8, T=4096, H=16, d=128): the checkpoint room is 0.54 GB
    full = L.ckda_bwd_workspace_bytes(8, 4096, 16, 128, 128)
    given = L.ckda_bwd_workspace_bytes_given_ckpt(8, 4096, 16, 128, 128)
    assert full - given == bwd_layout(8 * 64 * 16, 128, 128)[1] and given < 2 * 10**9
    assert bwd_varlen(L, [1, 5], 1, 5) == 5                       # does not start at 0
    assert bwd_varlen(L, [0, 5, 3], 2, 3) == 5                    # decreasing
    assert bwd_varlen(L, None, 2, 4) == 1
    assert bwd_varlen(L, [0, 5], 1, 5, DK=96) == 4
    assert bwd_varlen(L, [0, 5], 1, 5, dt=9) == 3
    # no checkpoints: recomputed, which needs room for them beyond the blocks
    assert bwd_varlen(L, [0, 5], 1, 5, hc=None, wsb=bwd_layout(2, 32, 32)[0]) == 6
    assert b"recomputed" in L.ckda_last_error()
    assert bwd_varlen(L, [0, 5], 1, 5, q=P(0x1004)) == 4          # misaligned
    # below the per-chunk blocks (2 chunk slots) the call fails before any launch
    assert bwd_varlen(L, [0, 5], 1, 5, wsb=bwd_layout(2, 32, 32)[0] - 16) == 6
    assert bwd_varlen(L, [0], 0, 0) == 0                          # no documents


def test_decode_and_bwd_reject_bad_arguments(L):
    f = ctypes.c_float(1.0)
    assert L.ckda_decode_step(4, 2, 96, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, FAKE, FAKE, FAKE, None) == 4
    assert L.ckda_decode_step(4, 2, 32, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, None, FAKE, FAKE, None) == 1
    assert L.ckda_decode_step(4, 2, 32, 32, 0, 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, FAKE, FAKE, FAKE, None) == 4
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


def test_outputs_must_not_alias_inputs(L):
    """Overlapping output and input ranges are refused on the host, before
    any launch (the pointers below are never dereferenced)."""
    f = ctypes.c_float(1.0)
    B, T, H, D = 1, 8, 1, 32
    n = B * T * H * D * 4                 # one fp32 token tensor
    base = 0x100000
    q, k, v, g, s, beta = (P(base + i * 0x10000) for i in range(6))
    o = P(base + 6 * 0x10000)
    ws = P(base + 8 * 0x10000)
    wsb = ctypes.c_size_t(0x100000)

    def call(o_=o, q_=q, ws_=ws, ht=None, h0=None):
        return L.ckda_fwd_chunked(B, T, H, D, D, 0, 0, q_, k, v, g, s, beta, f, h0, o_, ht, None, ws_, wsb, None)
    assert call(o_=P(q.value + n - 16)) == 4          # o overlaps the end of q
    assert b"'o'" in L.ckda_last_error() and b"'q'" in L.ckda_last_error()
    assert call(ws_=P(base + 0x10000)) == 4           # workspace over k
    assert call(ht=P(o.value + 64)) == 4              # two outputs overlap
    assert call(h0=P(o.value)) == 4                   # input state over an output
    # decode: o over the in/out state, and sign_prod over q
    st = P(base + 0x40000)
    assert L.ckda_decode_step(1, 1, D, D, 0, 0, q, k, v, g, s, beta, f, st, P(base + 0x50000), P(st.value + 128),
                              None) == 4
    assert L.ckda_decode_step(1, 1, D, D, 0, 0, q, k, v, g, s, beta, f, st, q, o, None) == 4
    # backward: dq over dout
    assert L.ckda_bwd(B, T, H, D, D, 0, 0, q, k, v, g, s, beta, f, None, P(base + 0x60000), P(base + 0x70000), None,
                      P(base + 0x70000), P(base + 0x80000), P(base + 0x90000), P(base + 0xa0000), P(base + 0xb0000),
                      None, P(base + 0x200000), ctypes.c_size_t(1 << 24), None) == 4
    assert b"'dq'" in L.ckda_last_error() and b"'dout'" in L.ckda_last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from gated_delta_rule_sign_amd import ckda
    monkeypatch.setattr(ckda, "_lib", None)
    monkeypatch.setattr(ckda, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ckda.CkdaError):
        ckda.lib()


def test_short_conv_rejects_bad_arguments(L):
    """Host checks of the short convolution: nothing is launched on failure."""
    u = ctypes.c_uint32
    cu = (ctypes.c_int32 * 3)(0, 5, 9)
    def fwd(N=2, T=8, cuh=None, cud=None, C=8, dt=0, flags=0, x=FAKE, y=P(0x20000), so=None, s0=None):
        return L.ckda_short_conv_fwd(N, T, cuh, cud, C, dt, u(flags), x, FAKE, s0, y, so, None)
    assert fwd(C=6) == 4                                   # channels not a multiple of 4
    assert fwd(flags=1) == 4 and fwd(flags=2) == 4          # mixer flags are not conv flags
    assert fwd(dt=7) == 3
    assert fwd(T=9) == 2                                    # 9 tokens do not split into 2 sequences
    assert fwd(N=0, T=8) == 2
    assert fwd(cuh=cu, cud=None, T=9) == 5                  # one copy of cu_seqlens only
    assert fwd(N=2, T=10, cuh=cu, cud=FAKE) == 5            # cu_seqlens[N] != T_total
    assert fwd(x=None) == 1
    assert fwd(x=P(0x1008)) == 4                            # misaligned
    assert fwd(y=FAKE) == 4 and b"overlaps" in L.ckda_last_error()
    assert fwd(T=0, N=0) == 0 and fwd(C=0) == 0             # nothing to do
    # the outgoing window may be the incoming one, but not overlap it otherwise
    assert fwd(N=2, T=0, so=P(0x40000), s0=P(0x40010)) == 4
    # backward: workspace per 64-token run and channel (4 taps, f32)
    assert L.ckda_short_conv_bwd_workspace_bytes(130, 8) == 3 * 8 * 4 * 4
    assert L.ckda_short_conv_bwd_workspace_bytes(130, 6) == 0
    def bwd(ws=P(0x80000), wsb=BIG, C=8, T=8, dx=P(0x30000)):
        return L.ckda_short_conv_bwd(2, T, None, None, C, 0, u(0), FAKE, P(0x50000), None, P(0x60000), dx,
                                     P(0x70000), None, ws, ctypes.c_size_t(wsb), None)
    assert bwd(ws=None) == 1
    assert bwd(wsb=8 * 4 * 4 - 16) == 6
    assert bwd(dx=FAKE) == 4                                # dx over x
    assert bwd(C=10) == 4
    # decode step
    assert L.ckda_short_conv_step(2, 6, 0, u(0), FAKE, FAKE, FAKE, FAKE, None) == 4
    assert L.ckda_short_conv_step(2, 8, 0, u(4), FAKE, FAKE, FAKE, FAKE, None) == 4
    assert L.ckda_short_conv_step(2, 8, 0, u(0), FAKE, FAKE, None, FAKE, None) == 1
    assert L.ckda_short_conv_step(0, 8, 0, u(0), None, None, None, None, None) == 0


def test_backward_with_forward_records_host_checks(L):
    """ckda_bwd_with_records: the forward's checkpoints and its whole record
    area are required, and no output may overlap the kept forward workspace."""
    f = ctypes.c_float(1.0)
    u = ctypes.c_uint32
    # one sequence of 8 tokens, one head, d = 32, fp32: one chunk record
    # (a fp32 record: W, Qh, KbT, M, d, u and the flag word, whole 256-byte lines)
    rec = ((64 * 32 * 3 + 64 * 64 + 32 + 64 * 32) * 4 + 4 + 255) // 256 * 256
    dq, dk, dv, dg, db = (P(0x100000 * (i + 1)) for i in range(5))
    ws = P(0x4000000)
    wsb = L.ckda_bwd_workspace_bytes_given_ckpt(1, 8, 1, 32, 32)
    def call(hc=P(0x900000), fws=P(0xA00000), fwb=BIG, dq_=dq):
        return L.ckda_bwd_with_records(1, 8, 1, 32, 32, 0, u(0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, f, None, hc,
                                       fws, ctypes.c_size_t(fwb), FAKE, None, dq_, dk, dv, dg, db, None, ws,
                                       ctypes.c_size_t(wsb), None)
    assert call(hc=None) == 1 and b"h_ckpt" in L.ckda_last_error()
    assert call(fws=None) == 1
    assert call(fwb=rec - 16) == 6 and b"records" in L.ckda_last_error()
    assert call(fwb=rec, fws=P(0xA00008)) == 4                     # misaligned
    assert call(fwb=rec, dq_=P(0xA00000)) == 4 and b"fwd_workspace" in L.ckda_last_error()
    cu = (ctypes.c_int32 * 2)(0, 8)
    assert L.ckda_bwd_varlen_with_records(1, 8, cu, FAKE, 1, 32, 32, 0, u(0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          f, None, P(0x900000), P(0xA00000), ctypes.c_size_t(16), FAKE, None,
                                          dq, dk, dv, dg, db, None, ws, ctypes.c_size_t(BIG), None) == 6
