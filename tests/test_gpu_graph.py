"""Decode steps captured in HIP graphs (pytorch/executorch PR 20351, commit
notes: the position and kv_len stay device tensors so the step can be
captured and replayed).

* A replayed full-context step gives exactly what the eager calls give, with
  eager work and synchronizations between the replays.
* Replayed at successive positions (new inputs and a new device position
  written from the host before each replay), the full-context step leaves
  the same cache bytes as the oracle and an output within the attention
  gate of the oracle's.
* The same for the sink and ring steps with the mask build in the graph
  (positions, K+V quant-scatter, kvq_build_mask, decode with the mask),
  past the cache's capacity: slot, cache positions and mask bit-exact too.
None of the entry points records a memset or allocates, so every step is
capturable."""
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


def _graph_of(fn):
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


@pytest.mark.parametrize("mode", ["positions+scatter", "scatter_kv_full", "append_full"])
def test_full_context_step_graph_vs_oracle(mode):
    """The full-context decode step (positions, K+V quant-scatter, decode; or
    the scatter that derives the slot from the device start position, and
    decode; or the one-launch step kvq_sdpa_decode_append_full) as one
    captured graph, replayed at three successive positions (across a 64-key
    unit boundary):
    before each replay new q / K / V values and the device start position and
    kv_len are written from the host.  After each replay the cache bytes
    equal the oracle's (which takes the same step) and the output is within
    the attention gate of the oracle's attention."""
    import oracle
    import quantized_kv_cache_head_amd.workloads as wl
    from _gpu import assert_cache_equal, check_attention, new_pair
    B, Hkv, G, S, D, hist = 2, 2, 4, 512, 128, 318
    Hq = Hkv * G
    rng = np.random.default_rng(2024)
    (K, hk), (V, hv) = new_pair(kvq.INT8_TH, B, Hkv, S, D), new_pair(kvq.INT8_TH, B, Hkv, S, D)
    slots = np.arange(hist, dtype=np.int32)
    for dc, hc in ((K, hk), (V, hv)):
        x = wl.to_bf16_values(rng.standard_normal((B, Hkv, hist, D)).astype(np.float32))
        kvq.quant_scatter(torch.from_numpy(x).to(torch.bfloat16).to(DEV), torch.from_numpy(slots).to(DEV), dc)
        oracle.quant_scatter(hc, x, slots)
    knew = torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device=DEV)
    vnew = torch.empty_like(knew)
    q = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device=DEV)
    start = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.ones(1, dtype=torch.int32, device=DEV)
    slot = torch.empty(1, dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, 1, D), dtype=torch.float32, device=DEV)
    ws = kvq.decode_workspace(B, Hq, Hkv, S, D)

    def step():
        if mode == "append_full":
            kvq.sdpa_decode_append_full(q, knew, vnew, start, K, V, out=out, workspace=ws)
            return
        if mode == "scatter_kv_full":
            kvq.quant_scatter_kv_full(knew, vnew, start, K, V)
        else:
            kvq.positions_full(start, 1, S, slot)
            kvq.quant_scatter_kv(knew, vnew, slot, K, V)
        kvq.sdpa_decode(q, K, V, kv_len=kv_len, out=out, workspace=ws)

    def load(p):
        vals = [wl.to_bf16_values(rng.standard_normal(shape).astype(np.float32))
                for shape in ((B, Hkv, 1, D), (B, Hkv, 1, D), (B, Hq, 1, D))]
        for t, v in zip((knew, vnew, q), vals):
            t.copy_(torch.from_numpy(v).to(torch.bfloat16))
        start.fill_(p)
        kv_len.fill_(p + 1)
        torch.cuda.synchronize()
        return vals

    # the warm-up run before the capture is a real step at position hist (the
    # oracle takes it too); the replays then continue at hist + 1 .. hist + 3
    kn, vn, qn = load(hist)
    g = _graph_of(step)
    positions = [hist, hist + 1, hist + 2, hist + 3]
    for i, p in enumerate(positions):
        if i:
            kn, vn, qn = load(p)
            say(f"full-context graph replay at position {p}")
            g.replay()
            torch.cuda.synchronize()
        sm, flags = oracle.positions_full(p, 1, S)
        assert flags == 0 and int(sm[0]) == p
        if mode == "positions+scatter":
            assert int(slot.item()) == p
        oracle.quant_scatter(hk, kn, sm)
        oracle.quant_scatter(hv, vn, sm)
        assert_cache_equal(K, hk, f"K after the step at position {p}")
        assert_cache_equal(V, hv, f"V after the step at position {p}")
        check_attention(out, oracle.sdpa(qn, hk, hv, p + 1), f"graph decode at position {p}")


@pytest.mark.parametrize("layout", ["sink", "ring"])
def test_sink_ring_step_graph_with_mask_vs_oracle(layout):
    """The sink / ring decode step with the mask build (positions, K+V
    quant-scatter, kvq_build_mask, decode with the mask) as one captured
    graph, replayed at positions past the cache's capacity: slot, cache
    positions, mask, cache bytes and output against the oracle after every
    replay."""
    import oracle
    import quantized_kv_cache_head_amd.workloads as wl
    from _gpu import assert_cache_equal, check_attention, new_pair
    B, Hkv, G, D = 1, 2, 4, 128
    sink, window = (4, 60) if layout == "sink" else (0, 64)
    S = sink + window
    Hq = Hkv * G
    rng = np.random.default_rng(4242 + sink)
    (K, hk), (V, hv) = new_pair(kvq.INT8_TH, B, Hkv, S, D), new_pair(kvq.INT8_TH, B, Hkv, S, D)
    cp_dev = torch.full((S,), -1, dtype=torch.int32, device=DEV)
    cp_ref = np.full(S, -1, np.int32)
    knew = torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device=DEV)
    vnew = torch.empty_like(knew)
    q = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device=DEV)
    start = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_len = torch.ones(1, dtype=torch.int32, device=DEV)
    slot = torch.empty(1, dtype=torch.int32, device=DEV)
    mask = torch.empty((1, S), dtype=torch.float32, device=DEV)
    out = torch.empty((B, Hq, 1, D), dtype=torch.float32, device=DEV)
    ws = kvq.decode_workspace(B, Hq, Hkv, S, D)

    def positions():
        if sink:
            kvq.positions_with_sink(start, 1, sink, window, slot, cp_dev)
        else:
            kvq.positions_ring(start, 1, window, slot, cp_dev)

    def step():
        positions()
        kvq.quant_scatter_kv(knew, vnew, slot, K, V)
        kvq.build_mask(cp_dev, start, 1, sink, window, mask)
        kvq.sdpa_decode(q, K, V, kv_len=kv_len, mask=mask, out=out, workspace=ws)

    def load(p):
        vals = [wl.to_bf16_values(rng.standard_normal(shape).astype(np.float32))
                for shape in ((B, Hkv, 1, D), (B, Hkv, 1, D), (B, Hq, 1, D))]
        for t, v in zip((knew, vnew, q), vals):
            t.copy_(torch.from_numpy(v).to(torch.bfloat16))
        start.fill_(p)
        kv_len.fill_(min(p + 1, S))
        torch.cuda.synchronize()
        return vals

    def oracle_step(p, kn, vn):
        sm = oracle.positions_sink(p, 1, sink, window, cp_ref)
        oracle.quant_scatter(hk, kn, sm)
        oracle.quant_scatter(hv, vn, sm)
        return sm

    # eager history: positions 0 .. 69 (past the capacity of 64 slots)
    P0 = 70
    for p in range(P0):
        kn, vn, _ = load(p)
        step()
        oracle_step(p, kn, vn)
    torch.cuda.synchronize()
    assert np.array_equal(cp_dev.cpu().numpy(), cp_ref)
    assert_cache_equal(K, hk, f"{layout} history K")
    assert_cache_equal(V, hv, f"{layout} history V")
    # the warm-up run before the capture is a real step at P0 (the oracle
    # takes it too; the capture itself runs nothing); replays continue after it
    kn, vn, qn = load(P0)
    g = _graph_of(step)
    oracle_step(P0, kn, vn)
    for p in (P0 + 1, P0 + 2, P0 + 3):
        kn, vn, qn = load(p)
        say(f"{layout} graph replay at position {p}")
        g.replay()
        torch.cuda.synchronize()
        sm = oracle_step(p, kn, vn)
        assert int(slot.item()) == int(sm[0]), (p, int(slot.item()), int(sm[0]))
        assert np.array_equal(cp_dev.cpu().numpy(), cp_ref), f"cache positions differ at {p}"
        mref = oracle.build_mask(cp_ref, p, 1, sink, window)
        assert np.array_equal(mask.cpu().numpy(), mref), f"mask differs at {p}"
        assert_cache_equal(K, hk, f"{layout} K at {p}")
        assert_cache_equal(V, hv, f"{layout} V at {p}")
        check_attention(out, oracle.sdpa(qn, hk, hv, min(p + 1, S), mask=mref), f"{layout} decode at {p}")
