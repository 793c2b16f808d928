"""The HIP path under HIP graph capture: replays give the eager result.

Paged decode (split kernel + merge kernel, with the work counter that the
split kernel resets itself) and causal prefill are captured into one graph
with caller-held outputs and workspace, then replayed several times with
other device work and synchronisations between the replays.  Each replay
must reproduce the eager output bit for bit, and a replay after the query
buffer is overwritten must match an eager call on the new queries.  (The
"GPU Kernel 调度：大模型推理的拐点 2026" page's launch-overhead paragraph:
graph replay replaces per-kernel launches.)
"""
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def afa(cuda):
    import attention_flash_fwd_amd as afa_mod
    from attention_flash_fwd_amd import _lib
    _lib.load()
    return afa_mod


@pytest.mark.parametrize("splits,T", [(8, 1), (2, 1), (16, 4), (4, 16)])
def test_graph_replay_matches_eager(afa, splits, T):
    from attention_flash_fwd_amd import inputs
    say(f"case graph replay: decode B8 mixed lengths, {splits} splits, T{T}; prefill B1 S640 causal")
    dev = "cuda"
    ctx = [700, 1500, 33, 2048, 1, 999, 1600, 64]
    inp = inputs.decode_inputs(ctx, 32, 8, 128, seed=41, device=dev)
    B = len(ctx)
    if T == 1:
        dq = inp.q
        lse_shape = (B, 32)
    else:
        dq = inputs.chunk_queries(B, T, 32, 128, seed=42, device=dev)
        lse_shape = (B, 32, T)
    mb = inp.block_table.shape[1]
    from attention_flash_fwd_amd import _lib
    nbytes = _lib.load().attn_decode_multi_workspace_bytes(B, T, 32, 8, 128, mb, 16, splits)
    ws = torch.empty(int(nbytes), dtype=torch.uint8, device=dev)
    o = torch.empty_like(dq)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    q, k, v = inputs.prefill_inputs(1, 640, 640, 8, 2, 128, seed=43, device=dev)
    po = torch.empty_like(q)
    plse = torch.empty((1, 8, 640), dtype=torch.float32, device=dev)

    def decode(out, lse_out):
        if T == 1:
            afa.decode_paged(dq, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, num_splits=splits,
                             out=out, lse_out=lse_out, workspace=ws)
        else:
            afa.decode_paged_multi(dq, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, num_splits=splits,
                                   out=out, lse_out=lse_out, workspace=ws)

    def step():
        decode(o, lse)
        afa.prefill(q, k, v, causal=True, out=po, lse_out=plse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, po, plse)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    outs = (o, lse, po, plse)
    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("o", "lse", "prefill o", "prefill lse"), outs, ref):
            assert torch.equal(t, r), f"replay {i}: {name} differs from the eager result"

    # The replay reads the buffers it was captured with: new queries in place.
    dq.copy_(torch.flip(dq, dims=[0]))
    q.copy_(-q)
    g.replay()
    torch.cuda.synchronize()
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    decode(o2, lse2)
    po2, plse2 = afa.prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(po, po2) and torch.equal(plse, plse2)
    del g
