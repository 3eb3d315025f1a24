"""The seeded input generators: deterministic, per-head reproducible, right structure."""

import numpy as np
import torch

import synth
from synth import WORKLOADS, BY_NAME, make_prefill, prefill_head, boosted_rows, make_decode_q, make_decode_kv


def test_workload_table_shapes():
    w = {x.name: x for x in WORKLOADS}
    assert len(WORKLOADS) == 5
    c1, c2, c3, c4, c5 = WORKLOADS
    assert (c1.B, c1.H, c1.N, c1.d, c1.causal) == (1, 1, 256, 64, False)
    assert (c2.B, c2.H, c2.N, c2.d, c2.causal) == (8, 12, 1024, 64, True)
    assert (c3.B, c3.H, c3.N, c3.d, c3.causal, c3.boost) == (1, 32, 4096, 128, True, 8.0)
    assert (c4.B, c4.H, c4.N, c4.d, c4.causal) == (1, 16, 16384, 128, False)
    assert (c5.B, c5.H, c5.lkv, c5.d, c5.num_splits) == (16, 32, 32768, 128, 64)
    assert c1.scale == 0.125 and c3.scale == float(np.float32(1 / np.sqrt(128)))


def test_prefill_is_deterministic_and_per_head():
    w = WORKLOADS[1].with_(B=2, H=3, N=40)
    q1, k1, v1 = make_prefill(w)
    q2, k2, v2 = make_prefill(w)
    assert q1.dtype == torch.bfloat16 and q1.shape == (2, 3, 40, 64)
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(k1[1, 2], prefill_head(w, "k", 1, 2))
    assert not torch.equal(q1[0, 0], q1[0, 1]) and not torch.equal(q1[0, 0], k1[0, 0])


def test_boost_rows():
    w = BY_NAME["llama3_8b_causal_b1h32n4096d128_kboost"].with_(H=2, N=500)
    rows = boosted_rows(w, 0, 1, 500)
    assert rows.numel() == 5 and len(set(rows.tolist())) == 5
    plain = synth.randn_bf16(synth.seed_for(w, "k", 0, 1), (500, w.d))
    k = prefill_head(w, "k", 0, 1)
    assert torch.equal(k[rows], plain[rows] * 8)          # ×8 is exact in bf16
    mask = torch.ones(500, dtype=torch.bool)
    mask[rows] = False
    assert torch.equal(k[mask], plain[mask])
    assert int(round(0.01 * 4096)) == 41


def test_decode_inputs_cpu():
    w = WORKLOADS[4].with_(B=2, H=2, lkv=33, num_splits=4)
    q = make_decode_q(w)
    k, v = make_decode_kv(w)
    assert q.shape == (2, 2, 1, 128) and k.shape == (2, 2, 33, 128)
    k2, v2 = make_decode_kv(w)
    assert torch.equal(k, k2) and torch.equal(v, v2)


def test_normal_statistics():
    x = synth.randn_bf16(123, (200_000,)).float()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1) < 0.01
