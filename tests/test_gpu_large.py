"""Inputs past 2 GiB per tensor (S=131149, H=72, bf16: 2.42 GB each). The
element and byte offsets of the last heads exceed 2^31, so any 32-bit index
arithmetic on the path (prepare, repair selection and gather, the attention
kernel's tile and row addressing, the output store) would show here as a
wrong or faulting row. Checked against the oracle on sampled rows of the
first and the last head, the ragged tail included."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import _oc, compare, log
from test_gpu_attention import check_bytes

pytestmark = pytest.mark.gpu

S, H = 131072 + 77, 72


@pytest.fixture(scope="module")
def big():
    q, k, v = workloads.random_qkv(1, S, H, seed=71, device="cuda", scale=1.5)
    assert q.numel() * q.element_size() > 2 ** 31
    yield q, k, v
    del q, k, v
    torch.cuda.empty_cache()


def test_inputs_past_2gib_match_oracle(big):
    oc = _oc()
    q, k, v = big
    log(f"[large] S={S} H={H}: {q.numel() * q.element_size() / 1e9:.2f} GB per tensor")
    out = oc.attention(q, k, v)
    prep = oc.prepare(q, k, v)
    torch.cuda.synchronize()
    rows = np.array(workloads.sample_rows(S, 48, seed=5))
    assert rows.max() >= S - 77            # the ragged last key tile's rows
    check_bytes(q, k, v, prep, 0, H - 1, rows, out=out, label=f"S={S} H={H}")
    compare(q, k, v, out, [(0, 0), (0, H - 1)], rows, label=f"S={S} H={H}", prep=prep)
    del prep, out
    torch.cuda.empty_cache()


def test_inputs_past_2gib_with_repair(big):
    oc = _oc()
    q, k, v = big
    budget = 0.005
    log(f"[large] S={S} H={H} repair budget {budget}")
    out = oc.attention_v_repair(q, k, v, budget)
    prep = oc.prepare_v_repair(q, k, v, budget)
    torch.cuda.synchronize()
    rows = np.array(workloads.sample_rows(S, 32, seed=6))
    compare(q, k, v, out, [(0, H - 1)], rows, budget=budget, label=f"S={S} H={H} repair", prep=prep)
    del prep, out
    torch.cuda.empty_cache()
