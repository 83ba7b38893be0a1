"""Per-layer rules files: parsing, validation, spans and plans per layer (host only)."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MODEL = os.path.join(GOLDEN, "model_rules.json")


@pytest.fixture(scope="module")
def rules(moa):
    import heterogeneous_sliding_windows_amd.rules as r
    return r


def test_model_file_spans_per_layer(rules):
    rs = rules.load(MODEL)
    assert rs.n_layers == 32 and rs.n_kv_heads == 32
    with open(MODEL) as f:
        doc = json.load(f)
    for n in (1, 100, 4096, 8192, 16384, 65536):
        s = rs.spans(n)
        assert s.shape == (32, 32)
        for layer, entry in enumerate(doc["layers"]):
            assert list(s[layer]) == list(oracle.spans(entry["alpha"], entry["beta"], n)), (n, layer)
    # every layer was drawn to 50 % mean density at N = 8192; layers differ
    dens = rs.spans(8192).mean(axis=1) / 8192
    assert (np.abs(dens - 0.5) <= 0.01).all()
    assert len({tuple(x) for x in rs.spans(8192)}) > 1


def test_roundtrip(rules, tmp_path):
    rs = rules.load(MODEL)
    p = tmp_path / "r.json"
    rules.save(rs, str(p))
    assert rules.load(str(p)) == rs
    assert json.loads(p.read_text()) == json.load(open(MODEL))


@pytest.mark.parametrize("mutate, msg", [
    (lambda d: d.update(format="other"), "format"),
    (lambda d: d.update(version=2), "version"),
    (lambda d: d.update(layers=[]), "layers"),
    (lambda d: d["layers"][3]["alpha"].pop(), "n_kv_heads"),
    (lambda d: d["layers"][0].pop("beta"), "beta"),
    (lambda d: d["layers"][1]["alpha"].__setitem__(0, -64), "alpha"),
    (lambda d: d["layers"][1]["alpha"].__setitem__(0, 1.5), "integers"),
    (lambda d: d["layers"][1]["alpha"].__setitem__(0, "64"), "integers"),
    (lambda d: d["layers"][2]["beta"].__setitem__(5, float("nan")), "beta"),
    (lambda d: d["layers"][2]["beta"].__setitem__(5, -0.25), "beta"),
    (lambda d: d["layers"][2]["beta"].__setitem__(5, True), "numbers"),
    (lambda d: d.update(n_kv_heads=31), "n_kv_heads"),
])
def test_invalid_documents(rules, mutate, msg):
    with open(MODEL) as f:
        doc = json.load(f)
    mutate(doc)
    with pytest.raises(ValueError, match=msg):
        rules.from_dict(doc)


def test_plans_per_layer(rules, moa):
    rs = rules.load(MODEL)
    plans = rs.plans(batch=2, n_q_heads=32, head_dim=128, n_prompt=8192, host_only=True)
    try:
        assert len(plans) == 32
        expect = rs.spans(8192)
        for layer, p in enumerate(plans):
            assert list(p.spans) == list(expect[layer])
            assert p.cache_elems == 2 * sum((int(s) + 31) // 32 * 32 for s in expect[layer]) * 128
    finally:
        for p in plans:
            p.close()
    # per-sequence lengths apply to every layer
    lens = [8192, 3000, 17]
    plans = rs.plans(batch=3, n_q_heads=32, head_dim=128, n_prompt=8192, seq_len=lens,
                     host_only=True)
    try:
        for layer, p in enumerate(plans):
            for b, nb in enumerate(lens):
                assert list(p.seq_spans[b]) == list(rs.spans(nb)[layer])
    finally:
        for p in plans:
            p.close()
