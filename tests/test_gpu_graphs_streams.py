"""HIP graph capture and concurrent streams.

The library allocates nothing, clears nothing with memset and keeps no state
between calls, so its launches can be captured in a HIP graph (through
torch.cuda.CUDAGraph) and replayed, and independent calls can run on several
streams at once.  Each replay runs on new contents of the captured input
buffers (copied in between replays, with eager work and synchronisations in
between) and must equal an eager call on the same inputs bit for bit (the
kernels are deterministic); calls queued on three streams at once must equal
the same calls made one after another.
"""

import sys

import numpy as np
import pytest

import exact_attention_121_amd as ea
from exact_attention_121_amd.inputs import make_decode_qkv, make_qkv
from parity_util import to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _capture(fn):
    """fn() queued once on a side stream (warm-up), then captured."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _refill(bufs, arrays):
    import torch
    for b, a in zip(bufs, arrays):
        b.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(b.device))


def test_forward_graph_replays():
    import torch
    _say("[graph] forward: B=2 Hq=8 Hkv=2 N=700 d=128 causal")
    q, k, v = to_dev(*make_qkv(2, 8, 2, 700, 128, seed=31))
    o, lse = torch.empty_like(q), torch.empty(2, 8, 700, device=q.device)
    g = _capture(lambda: ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse))
    for i in range(3):
        _refill((q, k, v), make_qkv(2, 8, 2, 700, 128, seed=40 + i))
        g.replay()
        torch.cuda.synchronize()
        ro, rl = ea.attn_fwd(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ro) and torch.equal(lse, rl), f"replay {i}"


def test_decode_graph_replays():
    import torch
    _say("[graph] decode: B=4 Hq=16 Hkv=4 Nq=1 Nk=3000 d=128 (split keys, merge)")
    shape = (4, 16, 4, 1, 3000, 128)
    q, k, v = to_dev(*make_decode_qkv(*shape, seed=51))
    o, lse = torch.empty_like(q), torch.empty(4, 16, 1, device=q.device)
    ws = torch.empty(ea.attn_decode_workspace_size(*shape), dtype=torch.uint8, device=q.device)
    g = _capture(lambda: ea.attn_decode(q, k, v, causal=True, out=o, lse=lse, workspace=ws))
    for i in range(3):
        _refill((q, k, v), make_decode_qkv(*shape, seed=60 + i))
        g.replay()
        torch.cuda.synchronize()
        ro, rl = ea.attn_decode(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ro) and torch.equal(lse, rl), f"replay {i}"


def test_backward_graph_replays():
    import torch
    _say("[graph] backward: B=1 Hq=8 Hkv=2 N=500 d=64 causal")
    q, k, v = to_dev(*make_qkv(1, 8, 2, 500, 64, seed=71))
    do = torch.randn_like(q)
    o, lse = ea.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_size(1, 8, 500, 64), dtype=torch.uint8, device=q.device)
    g = _capture(lambda: ea.attn_bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws))
    for i in range(3):
        _refill((q, k, v), make_qkv(1, 8, 2, 500, 64, seed=80 + i))
        do.copy_(torch.randn_like(do))
        o2, l2 = ea.attn_fwd(q, k, v, causal=True)
        o.copy_(o2)
        lse.copy_(l2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = ea.attn_bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            assert torch.equal(got, want), f"replay {i} {name}"


def test_three_streams_at_once():
    import torch
    _say("[streams] forward, decode and backward queued on three streams at once")
    fq, fk, fv = to_dev(*make_qkv(2, 16, 4, 2000, 128, seed=91))
    dshape = (8, 16, 2, 2, 4000, 64)
    dq_, dk_, dv_ = to_dev(*make_decode_qkv(*dshape, seed=92))
    bq, bk, bv = to_dev(*make_qkv(1, 8, 8, 900, 96, seed=93))
    bdo = torch.randn_like(bq)
    bo, bl = ea.attn_fwd(bq, bk, bv)
    torch.cuda.synchronize()
    # one after another
    r_f = ea.attn_fwd(fq, fk, fv, causal=True)
    r_d = ea.attn_decode(dq_, dk_, dv_)
    r_b = ea.attn_bwd(bq, bk, bv, bo, bl, bdo)
    torch.cuda.synchronize()
    # all at once, twice
    streams = [torch.cuda.Stream() for _ in range(3)]
    for _ in range(2):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(streams[0]):
            c_f = ea.attn_fwd(fq, fk, fv, causal=True)
        with torch.cuda.stream(streams[1]):
            c_d = ea.attn_decode(dq_, dk_, dv_)
        with torch.cuda.stream(streams[2]):
            c_b = ea.attn_bwd(bq, bk, bv, bo, bl, bdo)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(c_f, r_f))
        assert all(torch.equal(a, b) for a, b in zip(c_d, r_d))
        assert all(torch.equal(a, b) for a, b in zip(c_b, r_b))


def test_explicit_stream_without_workspace():
    """stream= a side stream and no workspace: the binding allocates the
    workspace on the current stream, the kernels use it on the side stream
    after the call returns.  A long matrix product queued first keeps the side
    stream busy while a buffer of the same size is allocated and filled on the
    current stream; the results must still match the oracle (and an ordinary
    call bit for bit)."""
    import torch

    from oracle.attention import attention_decode_ref
    from oracle.backward import attention_bwd_ref

    _say("[streams] backward and decode on an explicit side stream, workspace allocated by the binding")
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    qn, kn, vn = make_qkv(1, 4, 2, 300, 64, seed=95)
    don = np.random.default_rng(96).standard_normal(qn.shape, dtype=np.float32).astype(np.float16)
    q, k, v, do = to_dev(qn, kn, vn, don)
    o, lse = ea.attn_fwd(q, k, v, causal=True)
    dshape = (2, 8, 2, 1, 5000, 128)
    dqn, dkn, dvn = make_decode_qkv(*dshape, seed=97)
    dq_in, dk_in, dv_in = to_dev(dqn, dkn, dvn)
    ref_b = ea.attn_bwd(q, k, v, o, lse, do, causal=True)
    ref_d = ea.attn_decode(dq_in, dk_in, dv_in, causal=True)
    big = torch.randn(4096, 4096, device=q.device)
    torch.cuda.synchronize()
    bws = ea.attn_bwd_workspace_size(1, 4, 300, 64)
    dws = ea.attn_decode_workspace_size(*dshape)
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for _ in range(8):
            big = big @ big * 1e-3  # keeps the side stream busy for a while
    got_b = ea.attn_bwd(q, k, v, o, lse, do, causal=True, stream=side)
    got_d = ea.attn_decode(dq_in, dk_in, dv_in, causal=True, stream=side)
    # Same-size allocations on the current stream, filled with NaN bytes.
    junk = [torch.full((n,), 0xFF, dtype=torch.uint8, device=q.device) for n in (bws, dws, bws, dws)]
    torch.cuda.synchronize()
    del junk
    for name, g, r in zip(("dQ", "dK", "dV"), got_b, ref_b):
        assert torch.equal(g, r), f"backward {name} on the side stream differs from the ordinary call"
    assert torch.equal(got_d[0], ref_d[0]) and torch.equal(got_d[1], ref_d[1]), "decode differs"
    refs = attention_bwd_ref(qn, kn, vn, don, float(np.float32(1 / 8)), causal=True)
    for name, g, r in zip(("dQ", "dK", "dV"), got_b, refs):
        err = np.abs(g.cpu().numpy().astype(np.float64) - r)
        assert err.max() <= 1e-2 * np.abs(r).max() and err.mean() <= 2e-3 * np.abs(r).mean(), name
    O_ref, L_ref = attention_decode_ref(dqn, dkn, dvn, float(np.float32(1 / np.sqrt(128))), causal=True)
    err = np.abs(got_d[0].cpu().numpy().astype(np.float64) - O_ref)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
    assert np.abs(got_d[1].cpu().numpy() - L_ref).max() <= 1e-3
