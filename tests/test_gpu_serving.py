"""Serving paths on the GPU: a prefill handing its final state to decode
steps (the frame convention: ht in the true frame enters decode as state =
ht, sign_prod = +1), and the forward and decode step captured in a HIP graph
and replayed, every replay checked against eager results with eager work and
synchronisations between the replays."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_prefill_then_decode(dtype, DK, DV):
    """Tokens 0 .. T-1 through the chunked forward, then tokens T .. T+S-1
    one decode step at a time: the outputs and final state equal the oracle
    on the whole sequence."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner(f"prefill then decode {dtype} DK={DK} DV={DV}")
    B, T, S, H = 2, 150, 6, 2
    rng = np.random.default_rng(81)
    tok = I.draw_tokens(rng, (B, T + S), H, DK, DV, dtype)
    h0 = I.draw_state(rng, (B, H, DK, DV), 0.3)
    d = tok_to_dev(tok)
    o_pre, ht, _ = ckda.fwd(**{k: v[:, :T].contiguous() for k, v in d.items()}, scale=0.9, h0=dev_tensor(h0))
    state = ht.clone()
    sp = torch.ones((B, H, DK), dtype=torch.int8, device="cuda:0")
    outs = []
    for t in range(T, T + S):
        step = {k: v[:, t].contiguous() for k, v in d.items()}
        outs.append(host(ckda.decode_step(**step, state=state, sign_prod=sp, scale=0.9)))
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.fwd(**tok.f64(), scale=0.9, h0=h0.astype(np.float64))
    tol = 1e-4 if dtype == "f32" else 2e-3
    assert rel_max(host(o_pre), o_ref[:, :T]) < tol
    assert rel_max(np.stack(outs, axis=1), o_ref[:, T:]) < tol
    true_state = host(sp).astype(np.float64)[..., None] * host(state)
    assert rel_max(true_state, ht_ref) < tol


def test_forward_and_decode_in_a_graph():
    """ckda.fwd and ckda.decode_step with caller-owned buffers, captured in
    one graph; three replays on fresh inputs, each compared with an eager
    call on the same inputs (bitwise: same kernels, same order)."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner("fwd + decode in a HIP graph")
    B, T, H, DK, DV = 2, 200, 2, 128, 128
    ws = torch.empty(ckda.fwd_workspace_bytes(B, T, H, DK, DV, torch.bfloat16), dtype=torch.uint8, device="cuda:0")
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device="cuda:0")
    ht = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda:0")
    od = torch.empty((B, H, DV), dtype=torch.float32, device="cuda:0")

    def draw(seed):
        rng = np.random.default_rng(seed)
        tok = I.draw_tokens(rng, (B, T + 1), H, DK, DV, "bf16")
        return tok_to_dev(tok)

    d = draw(90)
    # caller-owned, contiguous input buffers the graph reads
    pre = {k: v[:, :T].contiguous() for k, v in d.items()}
    last = {k: v[:, T].contiguous() for k, v in d.items()}
    state = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda:0")
    sp = torch.empty((B, H, DK), dtype=torch.int8, device="cuda:0")

    def step():
        ckda.fwd(**pre, o=o, ht=ht, workspace=ws)
        state.copy_(ht)
        sp.fill_(1)
        ckda.decode_step(**last, state=state, sign_prod=sp, o=od)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()   # warm-up outside the capture (kernel attributes, allocator)
    torch.cuda.current_stream().wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        d = draw(91 + rep)
        for k in d:
            pre[k].copy_(d[k][:, :T])
            last[k].copy_(d[k][:, T])
        graph.replay()
        torch.cuda.synchronize()
        got = (host(o), host(ht), host(od), host(state))
        step()   # eager, same buffers and inputs
        torch.cuda.synchronize()
        want = (host(o), host(ht), host(od), host(state))
        for a, b in zip(got, want):
            assert np.array_equal(a, b), rep
        # and eager work in between the replays
        torch.matmul(torch.randn(64, 64, device="cuda:0"), torch.randn(64, 64, device="cuda:0"))
