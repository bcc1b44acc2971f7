"""GPU: the allocation-free entry point (latentmoe_forward_static, the
library's own device scratch as workspace) against latentmoe_forward with a
caller workspace, through the C ABI.  Two calls in a row on one handle, the
second with a smaller batch (the scratch keeps the first call's contents),
must equal the workspace entry point's results bit for bit (same kernels)
and meet the oracle's parity bar."""
import numpy as np
import pytest

import synth
from synth import LayerSpec, workload

from parity_util import check_against_oracle, check_routing_structure, to_f64

pytestmark = pytest.mark.gpu


def _run_both(spec, T, layer, dev, seed):
    import torch
    import mixture_experts_layer_32_amd as pkg
    x_np = synth.make_tokens(spec, T, seed)
    x = pkg.to_device({"x": x_np}, "cuda:0")["x"]
    cw = layer.weights_struct(dev)
    dbg_a = pkg.debug_buffers(spec, T, "cuda:0")
    dbg_b = pkg.debug_buffers(spec, T, "cuda:0")
    act = torch.float32 if spec.act_dtype == "f32" else torch.bfloat16
    out_s = torch.empty((T, spec.d), dtype=act, device="cuda:0")
    layer.forward_static(x, None, out_s, debug=dbg_a, cweights=cw)
    out_w = layer.forward(x, None, debug=dbg_b, cweights=cw)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_w)
    for k in dbg_a:
        assert torch.equal(dbg_a[k], dbg_b[k]), k
    g = {k: v.cpu().numpy() if v.dtype != torch.bfloat16 else to_f64(v) for k, v in dbg_a.items()}
    g["out"] = to_f64(out_s)
    return x_np, g


CASES = {
    "bf16_stream": (LayerSpec(d=512, l=128, m=256, n_experts=32, top_k=4,
                              gating="softmax_topk"), 300, 77),
    "bf16_tiled_std": (LayerSpec(d=256, l=256, m=192, n_experts=8, top_k=2,
                                 gating="softmax_all", has_projections=False), 1000, 333),
    "latent_decode": (workload("latent_decode").spec, 512, 200),
}


@pytest.mark.parametrize("name", list(CASES))
def test_static_scratch_entry_matches_workspace_entry(name):
    import mixture_experts_layer_32_amd as pkg
    spec, T1, T2 = CASES[name]
    layer = pkg.LatentMoELayer(spec)
    assert layer.workspace_size(T1) <= 64 << 20
    w = synth.make_weights(spec, 0)
    dev = pkg.to_device(pkg.pack_gated(w), "cuda:0")
    for T, seed in ((T1, 1), (T2, 2)):     # the second call is smaller
        x_np, g = _run_both(spec, T, layer, dev, seed)
        check_routing_structure(spec, g, T)
        tok = None if T <= 512 and spec.d <= 512 else np.arange(0, T, max(1, T // 40))
        st = check_against_oracle(spec, w, x_np, g, tokens=tok)
        print(name, T, st, flush=True)


def test_static_scratch_refuses_a_batch_beyond_it():
    import torch
    import mixture_experts_layer_32_amd as pkg
    spec = workload("latent_decode").spec
    layer = pkg.LatentMoELayer(spec)
    T = 4096                                   # about 0.4 GB of workspace
    assert layer.workspace_size(T) > 64 << 20
    dev = pkg.to_device(synth.make_weights(spec, 0), "cuda:0")
    x = torch.zeros((T, spec.d), dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty_like(x)
    with pytest.raises(RuntimeError, match="scratch"):
        layer.forward_static(x, dev, out)
