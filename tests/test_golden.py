"""CPU tests against the fixtures under tests/golden/."""
import json
import os

import numpy as np

import oracle
from sparse_mla_amd import workload

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_page_shapes_and_constants():
    """The worked example (decode of position 1000, 1001 cached positions):
    the oracle's outputs have the shapes the pages print, and the workload
    constants are the pages' dimensions."""
    g = _load("page_shapes.json")
    assert workload.H == g["heads"]["value"]
    assert workload.DN + workload.DR == g["qk_head_dim"]["value"]
    assert workload.DR == g["rotary_dims"]["value"]
    assert workload.DC == g["latent_dims"]["value"]
    assert workload.DV == g["value_dims"]["value"]
    assert workload.DQK == g["similarity_in_k"]["value"][2]
    assert abs(workload.SOFTMAX_SCALE - g["qk_head_dim"]["value"] ** -0.5) == 0.0
    w = workload.make("dense_p1000_b1")
    assert w.max_len == g["cached_positions_p1000"]["value"]
    idx = np.arange(w.max_len)[None, :]
    r = oracle.decode(w.q_nope, w.q_pe, w.kv, w.pe, w.wkv_b, w.seq_lens, idx, w.scale,
                      want_weights=True)
    B = 1
    sim = [B] + g["similarity_out"]["value"][1:]
    assert list(r["scores"].shape) == [sim[0], sim[1], sim[3]]           # query axis of size 1 dropped
    assert list(r["weights"].shape) == [B, g["softmax_out"]["value"][1], g["softmax_out"]["value"][3]]
    assert list(r["o_lat"].shape) == [B, g["value_up_in"]["value"][1], g["value_up_in"]["value"][3]]
    assert list(r["out"].shape) == [B, g["value_up_out"]["value"][1], g["value_up_out"]["value"][3]]
    assert np.allclose(r["weights"].sum(-1), 1.0, rtol=0, atol=1e-12)


def test_oracle_regression():
    """The oracle reproduces its committed outputs on a small seeded case."""
    g = _load("oracle_regression.json")
    c = g["case"]
    w = workload.make(c["name"], B=c["B"], L=c["L"], k=c["k"])
    r = oracle.decode(w.q_nope, w.q_pe, w.kv, w.pe, w.wkv_b, w.seq_lens, w.indices, w.scale)
    for b, h, d, v in g["out_samples"]:
        assert abs(r["out"][b, h, d] - v) <= 1e-12 * g["out_abs_max"]
    assert np.allclose(r["lse"], np.array(g["lse"]), rtol=0, atol=1e-12)
