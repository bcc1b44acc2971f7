"""GPU parity on Table 2's 95BT-8BA layer shapes (d 4096, m 2688, S 2) as the
standard MoE and as LatentMoE (l-MoE_eff at alpha 2/4/8, l-MoE_acc at
alpha 4), against the fp64 oracle: the shapes the alpha sweep measures.
Decode batches on sampled tokens, small batches on every token.
"""
import numpy as np
import pytest

import synth
from synth import workload

from parity_util import check_against_oracle, check_routing_structure, run_gpu

pytestmark = pytest.mark.gpu


def _sample_tokens(T, n=40, seed=5):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), np.int64)


@pytest.mark.parametrize("name,T", [("t2_acc_a4", 512), ("t2_eff_a8", 512), ("t2_std", 32),
                                    ("t2_eff_a2", 32), ("t2_eff_a4", 32)])
def test_table2_shapes_match_oracle(name, T):
    spec = workload(name).spec
    w, x = synth.make_weights(spec, 0), synth.make_tokens(spec, T, 0)
    g, layer = run_gpu(spec, w, x)
    print(name, T, "regime", layer.expert_regime(T), flush=True)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g, tokens=_sample_tokens(T) if T > 64 else None)
    print(name, T, st, flush=True)
