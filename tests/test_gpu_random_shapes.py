"""GPU parity of moe_forward on seeded random layer shapes against the fp64
oracle: token counts drawn from 1-4100 and capped so that the oracle
finishes in a second or two (2-600 in this draw: the decode streaming path,
the one-workgroup permutation, the grouped GEMMs, a multi-chunk
permutation), hidden sizes 256-2048, expert widths 128-640, 2-256 experts, k from 1 to 8,
bf16, fp8 (fp32 and UE8M0 block scales) and fp4 experts, row-major and packed
weights.  Router ids and per-expert counts are compared bit for bit, outputs
by the per-row relative L2 error within the dtype's tolerance."""
import random

import numpy as np
import pytest

import oracle
import synthetic
from moe_cases import host, oracle_experts, oracle_route, row_rel_err, run_forward, tol_of

pytestmark = pytest.mark.gpu

_TS = [1, 2, 3, 5, 8, 13, 16, 17, 24, 31, 32, 33, 48, 63, 64, 65, 100, 129, 257, 600, 1000, 2049, 4100]
_ORACLE_FLOPS = 6e9   # per case, so that the oracle finishes in a second or two


def _cases(seed: int, n: int):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        kind = rng.choice(["qwen_prefill", "dsv3_bf16", "dsv3_fp8", "dsv3_fp8_ue8m0", "dsv3_fp4"])
        H = rng.choice([256, 512, 768, 1024, 2048])
        I = rng.choice([128, 256, 384, 512, 640])
        E = rng.choice([2, 4, 8, 16, 60, 64, 100, 128, 160, 256])
        k = rng.randint(1, min(8, E))
        T = rng.choice(_TS)
        T = max(1, min(T, int(_ORACLE_FLOPS / (6 * k * H * I))))
        layout = "packed" if kind == "dsv3_fp4" or rng.random() < 0.7 else "rowmajor"
        out.append((kind, T, H, I, E, k, layout, rng.randint(0, 10000)))
    return out


CASES = _cases(seed=2024, n=40)


@pytest.mark.parametrize("kind,T,H,I,E,k,layout,seed", CASES,
                         ids=["%s-T%d-H%d-I%d-E%d-k%d-%s" % c[:7] for c in CASES])
def test_random_shape(kind, T, H, I, E, k, layout, seed):
    if kind == "dsv3_fp8_ue8m0":
        s = synthetic.spec("dsv3_fp8", T=T, H=H, I=I, E=E, k=k, scale_fmt="ue8m0")
    else:
        s = synthetic.spec(kind, T=T, H=H, I=I, E=E, k=k)
    L = synthetic.make_layer(s, seed=seed, device="cuda")
    hl = host(L)
    out, ids, w, counts = run_forward(s, L, layout=layout)
    ids_o, w_o = oracle_route(s, hl)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(counts.cpu().numpy(), oracle.permute(ids_o, s.E)[0])
    ref = oracle_experts(s, hl).combine(hl["x"], ids_o, w_o)
    err = row_rel_err(out.cpu().float().numpy(), ref)
    print("%s T=%d: max row rel err %.3e (tol %.0e)" % (kind, T, err, tol_of(s)))
    assert err <= tol_of(s)
