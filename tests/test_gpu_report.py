"""Error figures reported as information, beside the parity bar (needs an MI355X).

* the small non-causal case against a reference computed from its fp32 inputs before their
  rounding to bf16 (float64 softmax attention: at lambda = 1e-3 no tile is skipped, so the method
  is dense attention there), next to the error against the bf16-input oracle;
* the output error when the oracle takes its own float64 decisions instead of the GPU's (where a
  near-threshold tile flips, the two outputs differ by that tile's contribution).

Each case prints one JSON line (run with -s to see them); the asserts are loose sanity bounds.
"""
import json
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, err, from_dev_bf16, to_dev

pytestmark = pytest.mark.gpu

sa = pytest.importorskip("sparse_attention_flash_amd")


def _gpu_skip(q, k, v, lam, causal, Br):
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty_like(qd)
    B, Sq, Hq, _ = q.shape
    st = torch.empty((B, Hq, -(-Sq // Br), -(-k.shape[1] // 64)), dtype=torch.uint8,
                     device="cuda")
    sa.sa_skip_softmax_fwd(qd, kd, vd, o, lam, causal=causal, block_q=Br, tile_state=st)
    torch.cuda.synchronize()
    return from_dev_bf16(o), st.cpu().numpy()


def test_small_case_against_fp32_inputs():
    wl = W.WORKLOADS["iid_s256_d64"]
    announce("report: small case vs fp32-input reference")
    q, k, v = wl.generate()
    qf, kf, vf = W.gen_iid_f32(wl.seed, wl.B, wl.S, wl.S, wl.Hq, wl.Hkv, wl.D)
    assert np.array_equal(W.to_bf16_bits(qf), q)           # the same draws
    o, st = _gpu_skip(q, k, v, wl.param("lambda"), False, wl.block_q)
    assert (st == 0).all()
    Q = torch.from_numpy(qf.astype(np.float64)).permute(0, 2, 1, 3)
    K = torch.from_numpy(kf.astype(np.float64)).permute(0, 2, 1, 3)
    V = torch.from_numpy(vf.astype(np.float64)).permute(0, 2, 1, 3)
    ref32 = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=wl.scale)
    ref32 = ref32.permute(0, 2, 1, 3).numpy()
    o_bf, _, _, _ = oracle.skip_softmax(q, k, v, causal=False, block_q=wl.block_q,
                                        block_k=wl.block_k, scale=wl.scale, lam=wl.param("lambda"))
    e32 = err(o, ref32)
    ebf = err(o, o_bf)
    einp = err(o_bf, ref32)
    print(json.dumps({"report": "small_case_fp32_inputs", "gpu_vs_fp32_input_ref":
                      {"max_abs": e32[0], "mean_abs": e32[1]},
                      "gpu_vs_bf16_input_oracle": {"max_abs": ebf[0], "mean_abs": ebf[1]},
                      "bf16_rounding_of_inputs_alone": {"max_abs": einp[0], "mean_abs": einp[1]}}))
    assert e32[0] < 0.1


@pytest.mark.parametrize("case", [("iid_s256_d64", [0.5, 1.0, 1.5, 3.0]),
                                  ("llm_gqa_s1024", [0.5, 1.0, 1.5127145])])
def test_independent_decision_output_error(case):
    name, lams = case
    announce(f"report: independent-decision output error {name}")
    if name == "iid_s256_d64":
        wl = W.WORKLOADS[name]
        q, k, v = wl.generate()
        causal, Br = False, wl.block_q
    else:
        q, k, v = W.gen_llm(2, 1, 1024, 8, 2, 128)
        causal, Br = True, 128
    D = q.shape[-1]
    rows = []
    for lam in lams:
        o, st = _gpu_skip(q, k, v, lam, causal, Br)
        kw = dict(causal=causal, block_q=Br, block_k=64, scale=1 / math.sqrt(D), lam=lam)
        o_ind, _, st_ind, _ = oracle.skip_softmax(q, k, v, mode=0, **kw)
        o_forced, _, _, _ = oracle.skip_softmax(q, k, v, mode=2, state_in=st, **kw)
        vis = st != 2
        rows.append({"lambda": lam, "tiles_visited": int(vis.sum()),
                     "decisions_differing": int((st_ind[vis] != st[vis]).sum()),
                     "max_abs_vs_independent": err(o, o_ind)[0],
                     "mean_abs_vs_independent": err(o, o_ind)[1],
                     "max_abs_vs_forced": err(o, o_forced)[0]})
        assert err(o, o_forced)[0] <= 2e-2
    print(json.dumps({"report": "independent_decision_output_error", "case": name, "rows": rows}))
