"""The quantize + attention step captured in a HIP graph: every replay gives
the eager step's output bit for bit, with eager steps and synchronizations
between the replays (the benchmark times the step this way)."""
import dataclasses

import pytest
import torch

import workloads
import quantized_attention_smooth_amd as sage

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("v_dtype, gran, causal", [("fp8", "per_warp", False), ("fp16", "per_thread", True)])
def test_step_graph_replays_equal_eager(v_dtype, gran, causal):
    w = dataclasses.replace(workloads.WORKLOADS["b2h8n4096d128"], B=1, Hq=2, Hkv=2, Nq=1000, Nk=1000, v_dtype=v_dtype,
                            gran=gran, causal=causal, pv_accum="fp32" if v_dtype == "fp16" else "fp16+fp32", seed=21)
    print(f"[gpu-case] graph step B1 H2 N1000 d128 V={v_dtype} {gran} causal={causal} seed 21", flush=True)
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    ws_k = torch.empty(sage.workspace_bytes(w.B, w.Hkv, w.Nk, w.d), dtype=torch.uint8, device=dev)
    ws_v = torch.empty_like(ws_k)

    def step():
        qk, qv = sage.sage_quant_qkv(q, k, v, qk_quant_gran=w.gran, smooth_k=True, v_dtype=w.v_dtype,
                                     workspace_k=ws_k, workspace_v=ws_v)
        return sage.sage_attn_fwd(qk, qv, is_causal=w.causal, pv_accum_dtype=w.pv_accum)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        eager = step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = eager.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    torch.cuda.synchronize()
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        again = step()                                  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), eager.view(torch.int16)), f"eager step after replay {i}"
