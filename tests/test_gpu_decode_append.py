"""GPU parity of kvq_sdpa_decode_append_full (the new token's K and V written
into full-context int8 caches and decode attention over them, one launch).

Its definition is the two-call sequence kvq_quant_scatter_kv_full(start_pos)
then kvq_sdpa_decode(kv_len = start_pos + 1); so every case checks, on the
same inputs:
  * the caches after the fused call equal those after the two calls, byte for
    byte, and the oracle's (quant-scatter of the history, then of the token);
  * the output equals the two-call output bit for bit and meets the attention
    tolerance against the fp64 oracle over kv_len = start_pos + 1;
  * the error flags equal the two calls' flags (out-of-range positions).
Positions cover the first slot, both ends of a 64-key unit, the last slot,
and the Llama-3-8B-shaped layer at full size."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, assert_cache_equal, check_attention, dev_input, new_pair, say

pytestmark = pytest.mark.gpu


def clone(c: kvq.Cache) -> kvq.Cache:
    return kvq.Cache(c.qmode, c.B, c.H, c.S, c.D, c.codes.clone(), c.scales.clone(),
                     None if c.zps is None else c.zps.clone())


def history(B, Hkv, S, D, n_fill, rng, check_oracle=True):
    """K and V caches with slots [0, n_fill) written (GPU and oracle), the rest
    sentinel."""
    pairs = []
    for _ in range(2):
        dc, hc = new_pair(kvq.INT8_TH, B, Hkv, S, D)
        if n_fill:
            x = rng.standard_normal((B, Hkv, n_fill, D)).astype(np.float32)
            x[..., rng.choice(D, max(1, D // 32), replace=False)] *= 10
            x = wl.to_bf16_values(x)
            slots = np.broadcast_to(np.arange(n_fill, dtype=np.int32), (B, n_fill)).copy()
            kvq.quant_scatter(dev_input(x, True), torch.from_numpy(slots).to(DEV), dc)
            if check_oracle:
                oracle.quant_scatter(hc, x, slots, parallel=True)
        pairs.append((dc, hc))
    torch.cuda.synchronize()
    if check_oracle:
        for dc, hc in pairs:
            assert_cache_equal(dc, hc, "history")
    return pairs


def one_case(B, Hkv, G, S, D, pos, q_bf16=True, x_bf16=True, out_dtype=torch.bfloat16, seed=0, oracle_check=True):
    say(f"decode append B{B} Hkv{Hkv} G{G} S{S} D{D} start_pos {pos} q_bf16 {q_bf16} x_bf16 {x_bf16} out {out_dtype}")
    rng = np.random.default_rng(seed)
    # slots [0, n_fill) hold history: up to the new slot, every slot when the
    # position is past the cache, and slot 0 when it is negative (the clamped
    # kv_len 1 then reads a written slot)
    n_fill = S if pos >= S else (pos if pos >= 0 else 1)
    (K, hK), (V, hV) = history(B, Hkv, S, D, n_fill, rng, check_oracle=oracle_check)
    q_np = rng.standard_normal((B, Hkv * G, 1, D)).astype(np.float32)
    xk_np = rng.standard_normal((B, Hkv, 1, D)).astype(np.float32)
    xv_np = rng.standard_normal((B, Hkv, 1, D)).astype(np.float32)
    xk_np[..., 3] *= 10
    if q_bf16:
        q_np = wl.to_bf16_values(q_np)
    if x_bf16:
        xk_np, xv_np = wl.to_bf16_values(xk_np), wl.to_bf16_values(xv_np)
    q = dev_input(q_np, q_bf16)
    xk, xv = dev_input(xk_np, x_bf16), dev_input(xv_np, x_bf16)
    sp = torch.tensor([pos], dtype=torch.int32, device=DEV)

    # the two-call definition
    K2, V2 = clone(K), clone(V)
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvq.quant_scatter_kv_full(xk, xv, sp, K2, V2, err_flags=err2)
    kl = torch.tensor([pos + 1], dtype=torch.int32, device=DEV)
    out2 = kvq.sdpa_decode(q, K2, V2, kv_len=kl, out_dtype=out_dtype, err_flags=err2)
    # the fused call
    err1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    out1 = kvq.sdpa_decode_append_full(q, xk, xv, sp, K, V, out_dtype=out_dtype, err_flags=err1)
    torch.cuda.synchronize()

    assert int(err1.item()) == int(err2.item()), (int(err1.item()), int(err2.item()))
    for a, b, what in ((K, K2, "K"), (V, V2, "V")):
        assert torch.equal(a.codes, b.codes), f"{what} codes differ from the two-call sequence"
        assert torch.equal(a.scales.view(torch.int32), b.scales.view(torch.int32)), f"{what} scales differ"
        assert torch.equal(a.zps, b.zps), f"{what} zero points differ"
    iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out1.view(iv), out2.view(iv)), "output differs from the two-call sequence"
    if not oracle_check:
        return int(err1.item())
    if 0 <= pos < S:
        oracle.quant_scatter(hK, xk_np, np.full((B, 1), pos, np.int32))
        oracle.quant_scatter(hV, xv_np, np.full((B, 1), pos, np.int32))
    assert_cache_equal(K, hK, "K after append")
    assert_cache_equal(V, hV, "V after append")
    kv_len = min(max(pos + 1, 1), S)
    check_attention(out1, oracle.sdpa(q_np, hK, hV, kv_len), "append decode")
    return int(err1.item())


@pytest.mark.parametrize("D,G", [(64, 1), (64, 8), (128, 2), (128, 4), (128, 8), (256, 1), (256, 4)])
def test_append_parity_shapes(D, G):
    for pos in (0, 63, 64, 700, 1023):
        assert one_case(2, 2, G, 1024, D, pos, seed=pos + D + G) == 0


@pytest.mark.parametrize("q_bf16,x_bf16,out_dtype", [(False, False, torch.float32), (True, False, torch.float32),
                                                     (False, True, torch.bfloat16)])
def test_append_dtypes(q_bf16, x_bf16, out_dtype):
    assert one_case(3, 4, 4, 2048, 128, 1530, q_bf16, x_bf16, out_dtype, seed=5) == 0


def test_append_positions_out_of_range():
    # nothing written; flags and output as the scatter + decode pair
    assert one_case(2, 2, 4, 256, 128, 256, seed=1) == kvq.FLAG_POS_CAPACITY | kvq.FLAG_KVLEN
    assert one_case(2, 2, 4, 256, 128, 300, seed=2) == kvq.FLAG_POS_CAPACITY | kvq.FLAG_KVLEN
    assert one_case(2, 2, 4, 256, 128, -1, seed=3) == kvq.FLAG_SLOT_RANGE | kvq.FLAG_KVLEN


def test_append_llama8b_layer_full_size():
    # the Llama-3-8B-shaped layer: B 8, 32 / 8 heads, D 128, 8192 slots, the
    # token at position 4095 (kv_len 4096); against the two-call sequence
    # bit for bit (the oracle checks of both calls' kernels at this size are
    # in the workload tests)
    one_case(8, 8, 4, 8192, 128, 4095, seed=11, oracle_check=False)


def test_append_steps_in_a_row():
    """Several steps on the same caches: every token goes where the next
    step's attention finds it."""
    B, Hkv, G, S, D = 2, 2, 4, 512, 128
    rng = np.random.default_rng(17)
    (K, hK), (V, hV) = history(B, Hkv, S, D, 190, rng)
    ws = kvq.decode_workspace(B, Hkv * G, Hkv, S, D, DEV)
    for pos in range(190, 200):
        say(f"append step {pos}")
        q_np = wl.to_bf16_values(rng.standard_normal((B, Hkv * G, 1, D)).astype(np.float32))
        xk_np = wl.to_bf16_values(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32))
        xv_np = wl.to_bf16_values(rng.standard_normal((B, Hkv, 1, D)).astype(np.float32))
        out = kvq.sdpa_decode_append_full(dev_input(q_np, True), dev_input(xk_np, True), dev_input(xv_np, True),
                                          torch.tensor([pos], dtype=torch.int32, device=DEV), K, V,
                                          out_dtype=torch.float32, workspace=ws)
        oracle.quant_scatter(hK, xk_np, np.full((B, 1), pos, np.int32))
        oracle.quant_scatter(hV, xv_np, np.full((B, 1), pos, np.int32))
        check_attention(out, oracle.sdpa(q_np, hK, hV, pos + 1), f"step {pos}")
    assert_cache_equal(K, hK, "K after the steps")
    assert_cache_equal(V, hV, "V after the steps")
