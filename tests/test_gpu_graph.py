"""A decode step captured in a HIP graph (positions, quant-scatter of the new
K/V token, decode attention) gives on every replay exactly what the eager calls
give, with eager work and synchronizations between the replays.  None of the
entry points records a memset or allocates, so the whole step is capturable."""
import numpy as np
import pytest
import torch

import quantized_kv_cache_head_amd as kvq
from _gpu import DEV, say

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    B, Hkv, G, S, D = 2, 2, 4, 512, 128
    Hq = Hkv * G
    hist = 300
    say(f"graph step B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} hist={hist}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    K = kvq.Cache.empty(kvq.INT8_TH, B, Hkv, S, D).sentinel_fill()
    V = kvq.Cache.empty(kvq.INT8_TH, B, Hkv, S, D).sentinel_fill()
    x = torch.randn((B, Hkv, hist, D), generator=gen, device=DEV).to(torch.bfloat16)
    kvq.quant_scatter(x, torch.arange(hist, dtype=torch.int32, device=DEV), K)
    kvq.quant_scatter(x.flip(2).contiguous(), torch.arange(hist, dtype=torch.int32, device=DEV), V)
    knew = torch.randn((B, Hkv, 1, D), generator=gen, device=DEV).to(torch.bfloat16)
    vnew = torch.randn((B, Hkv, 1, D), generator=gen, device=DEV).to(torch.bfloat16)
    q = torch.randn((B, Hq, 1, D), generator=gen, device=DEV).to(torch.bfloat16)
    start = torch.tensor([hist], dtype=torch.int32, device=DEV)
    kv_len = torch.tensor([hist + 1], dtype=torch.int32, device=DEV)
    slot = torch.empty(1, dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device=DEV)
    ws = kvq.decode_workspace(B, Hq, Hkv, S, D)

    def step():
        kvq.positions_full(start, 1, S, slot)
        kvq.quant_scatter(knew, slot, K)
        kvq.quant_scatter(vnew, slot, V)
        kvq.sdpa_decode(q, K, V, kv_len=kv_len, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    eager_codes = K.codes.clone()

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

    other_q = torch.randn_like(q)
    for rep in range(4):
        out.fill_(float("nan"))
        # eager work between replays: a decode with another query into a
        # separate output, then a synchronization
        junk = kvq.sdpa_decode(other_q, K, V, kv_len=kv_len)
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}: output differs from the eager step"
        assert torch.equal(K.codes, eager_codes), f"replay {rep}: cache differs"
        assert torch.isfinite(junk.float()).all()
    assert np.isfinite(eager.float().cpu().numpy()).all()


def test_split_prefill_graph_replays_match_eager():
    """The key-split prefill (prefill launch + combine launch, caller
    workspace) captured in a HIP graph: every replay, with eager work and
    synchronizations between replays, equals the eager call bit for bit, also
    after kv_len changes between replays."""
    B, Hkv, G, S, D, Lq = 1, 2, 2, 4096, 128, 32
    Hq = Hkv * G
    say(f"graph split prefill Hq={Hq} Hkv={Hkv} S={S} D={D} Lq={Lq}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(78)
    K = kvq.Cache.empty(kvq.UINT4_TH, B, Hkv, S, D)
    V = kvq.Cache.empty(kvq.UINT4_TH, B, Hkv, S, D)
    x = torch.randn((B, Hkv, S, D), generator=gen, device=DEV).to(torch.bfloat16)
    kvq.quant_scatter(x, torch.arange(S, dtype=torch.int32, device=DEV), K)
    kvq.quant_scatter(x.flip(2).contiguous(), torch.arange(S, dtype=torch.int32, device=DEV), V)
    q = torch.randn((B, Hq, Lq, D), generator=gen, device=DEV).to(torch.bfloat16)
    kv_len = torch.tensor([3000], dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, Lq, D), dtype=torch.float32, device=DEV)
    ws = torch.empty(kvq.sdpa_prefill_split_workspace_bytes(B, Hq, Hkv, Lq, S, D), dtype=torch.uint8, device=DEV)
    assert ws.numel() > 0

    def call():
        kvq.sdpa_prefill_split(q, K, V, kv_len=kv_len, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for n in (3000, 3000, 1800, 4096):
        kv_len.fill_(n)
        call()
        torch.cuda.synchronize()
        eager = out.clone()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay differs at kv_len {n}"
