"""The comparison byte path of the attention kernel (exponential per score,
then the FP32 -> E4M3 cast; weights="exp_fp8") against the oracle's
exp_cast_codes path: bytes at least 99.9% equal and never more than one code
apart (v_exp_f32 is within 1 ulp of the correctly rounded fp32 weight, and
the logits are fp32), outputs within the same 5e-3 relative L2."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import head64, log, out_rows
from test_gpu_attention import TOL, _compare, check_bytes

pytestmark = pytest.mark.gpu


def _oc():
    import bit_fp8_attention_block_amd as oc
    return oc


@pytest.mark.parametrize("case", ["s1024_h2", "ragged300", "s130"])
def test_exp_path_bytes_match_oracle(case):
    oc = _oc()
    log(f"[exp bytes] case={case}")
    if case == "s1024_h2":
        q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    elif case == "ragged300":
        q, k, v = workloads.make_inputs("s8192_h8", device="cuda", S=300, H=2)
    else:
        q, k, v = workloads.random_qkv(1, 130, 1, seed=4, device="cuda", scale=2.0)
    B, S, H, _ = q.shape
    out = oc.attention(q, k, v, weights="exp_fp8")
    prep = oc.prepare(q, k, v)
    for b in range(B):
        for h in range(H):
            d = check_bytes(q, k, v, prep, b, h, np.arange(S), out=out, weights="exp_cast", label=case)
            # the two byte paths are different maps: about 80% equal, one apart elsewhere
            Mk = d.m_used[:, np.arange(S) // 128]
            other = (d.codes == oracle.expcast_codes(d.x, Mk)).mean()
            log(f"  (b={b},h={h}) equal to ExpCast bytes {other:.3f}")
            assert other < 0.95
            r = oracle.expcast_attention_online(head64(q, b, h), head64(k, b, h), head64(v, b, h), ph=d.ph,
                                                weights="exp_cast", m_trace=d.m_used)
            e = oracle.rel_l2(out_rows(out, b, h, np.arange(S)), r["out"])
            assert e <= TOL, e


@pytest.mark.parametrize("name,rows_per_head,pairs", [
    ("s8192_h8", 256, [(0, 0), (0, 5)]),
    ("s73397_h56", 64, [(0, 0), (0, 55)]),
])
def test_exp_path_output_matches_oracle(name, rows_per_head, pairs):
    oc = _oc()
    w = workloads.WORKLOADS[name]
    log(f"[exp workload] {name}")
    q, k, v = workloads.make_inputs(name, device="cuda")
    out = oc.attention(q, k, v, weights="exp_fp8")
    prep = oc.prepare(q, k, v)
    torch.cuda.synchronize()
    rows = np.array(workloads.sample_rows(w.S, rows_per_head, seed=w.seed))
    _compare(q, k, v, out, pairs, rows, label=name + " exp path", prep=prep, weights="exp_cast")


def test_exp_path_with_repair_matches_oracle():
    oc = _oc()
    log("[exp repair] s8192_h8 at S=2000, budget 0.01")
    q, k, v = workloads.make_inputs("s8192_h8", device="cuda", S=2000, H=2)
    out = oc.attention_v_repair(q, k, v, 0.01, weights="exp_fp8")
    torch.cuda.synchronize()
    prep = oc.prepare_v_repair(q, k, v, 0.01)
    rows = np.arange(0, 2000, 3)
    _compare(q, k, v, out, [(0, 0), (0, 1)], rows, budget=0.01, label="exp path + repair", prep=prep,
             weights="exp_cast")


def test_weights_selection_is_per_call():
    """Switching a plan between the two paths and back gives each path's own
    result, bit for bit."""
    oc = _oc()
    q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    a = oc.attention(q, k, v)
    e = oc.attention(q, k, v, weights="exp_fp8")
    a2 = oc.attention(q, k, v)
    e2 = oc.attention(q, k, v, weights="exp_fp8")
    torch.cuda.synchronize()
    assert torch.equal(a, a2) and torch.equal(e, e2)
    assert not torch.equal(a, e)
