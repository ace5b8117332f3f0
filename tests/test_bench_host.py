"""Host logic of bench.py (CPU): the one-GPU guard, the algorithmic byte
counts the roofline is priced on, and the rule that measured traffic is
reported only for the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gated_delta_rule_sign_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _size(dtype):
    return {"bf16": 2, "f32": 4}[dtype]


def test_forward_bytes_per_token_head():
    """Inputs read once and outputs written once, from the workload's own
    shapes and storage types: q, k, v in the input dtype, g fp32 and s int8
    per key channel, beta fp32 per head, o fp32 per value channel."""
    c = I.WORKLOADS["layer_bf16"]
    DK, DV, e = c["DK"], c["DV"], _size(c["dtype"])
    expect = (2 * DK + DV) * e + DK * (np.dtype(np.float32).itemsize + np.dtype(np.int8).itemsize) + 4 + DV * 4
    assert bench.FWD_BYTES_PER_TOKEN_HEAD == expect == 1924
    # head-scalar gate: one g and one s per token-head
    assert bench.FWD_HG_BYTES_PER_TOKEN_HEAD == (2 * DK + DV) * e + 4 + 1 + 4 + DV * 4


def test_decode_bytes_per_head_step():
    """The fp32 state read and written once, the int8 sign product read and
    written once, one token's q, k, v (input dtype), g, s, beta, and o."""
    c = I.WORKLOADS["decode_b256"]
    DK, DV, e = c["DK"], c["DV"], _size(c["dtype"])
    expect = 2 * DK * DV * 4 + 2 * DK * 1 + (2 * DK + DV) * e + DK * 4 + DK * 1 + 4 + DV * 4
    assert bench.DEC_BYTES_PER_HEAD_STEP == expect == 133252


def test_backward_bytes_per_token_head():
    """q, k, v, do (bf16), g, s, beta, the chunk-start checkpoints (one
    DK x DV fp32 state per 64 tokens), and dq, dk, dv, dg, dbeta out."""
    c = I.WORKLOADS["layer_bf16"]
    DK, DV, e = c["DK"], c["DV"], _size(c["dtype"])
    expect = ((2 * DK + 2 * DV) * e + DK * 4 + DK + 4 + DK * DV * 4 // 64
              + (2 * DK + DV + DK) * 4 + 4)
    assert bench.BWD_BYTES_PER_TOKEN_HEAD == expect == 4744


def test_traffic_is_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_FILE))
    for f in rec["sources"]:
        assert os.path.exists(os.path.join(ROOT, "gated_delta_rule_sign_amd", "csrc", f)), f
    got = bench.measured_traffic()
    # either the committed counters match the kernel sources, or bench reports null
    assert got is None or got == float(rec["traffic_bytes_per_call"])
    # a record taken on other sources is never used
    stale = dict(rec, sources_sha256="0" * 64)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic() is None
    # and a missing record gives null as well
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.measured_traffic() is None


def test_decode_traffic_and_mfma_records_follow_the_same_rule(tmp_path, monkeypatch):
    """The decode traffic and the forward's executed matrix-core work come from
    committed counter runs too, and are used only while their sources match."""
    rec = json.load(open(bench.DECODE_TRAFFIC_FILE))
    got = bench.measured_traffic(bench.DECODE_TRAFFIC_FILE)
    assert got is None or got == float(rec["traffic_bytes_per_call"])
    p = tmp_path / "dec.json"
    p.write_text(json.dumps(dict(rec, sources_sha256="0" * 64)))
    assert bench.measured_traffic(str(p)) is None
    m = json.load(open(bench.MFMA_FILE))
    got = bench.measured_mfma()
    assert got is None or got["executed_bf16_flops_per_call"] == m["executed_bf16_flops_per_call"]
    q = tmp_path / "mfma.json"
    q.write_text(json.dumps(dict(m, sources_sha256="0" * 64)))
    monkeypatch.setattr(bench, "MFMA_FILE", str(q))
    assert bench.measured_mfma() is None


def _includes(fname, seen):
    """fname and every local header it includes, transitively."""
    import re
    if fname in seen:
        return seen
    seen.add(fname)
    src = open(os.path.join(ROOT, "gated_delta_rule_sign_amd", "csrc", fname)).read()
    for inc in re.findall(r'#include "([^"/]+)"', src):
        _includes(inc, seen)
    return seen


def test_counter_records_hash_every_source_their_kernels_compile_from(tmp_path):
    """A counter record stays valid only while its kernels are unchanged, so its
    hash must cover every header the kernels' translation units include (the
    forward's chunk kernel body lives in a header of its own)."""
    for path in (bench.TRAFFIC_FILE, bench.MFMA_FILE, bench.DECODE_TRAFFIC_FILE, bench.BWD_TRAFFIC_FILE):
        rec = json.load(open(path))
        listed = set(rec["sources"])
        units = [f for f in rec["sources"] if f.endswith(".hip")]
        assert units, path
        need = set()
        for u in units:
            _includes(u, need)
        assert need <= listed, (os.path.basename(path), sorted(need - listed))
    rec = json.load(open(bench.BWD_TRAFFIC_FILE))
    got = bench.measured_traffic(bench.BWD_TRAFFIC_FILE)
    assert got is None or got == float(rec["traffic_bytes_per_call"])
    p = tmp_path / "bwd.json"
    p.write_text(json.dumps(dict(rec, sources_sha256="0" * 64)))
    assert bench.measured_traffic(str(p)) is None
