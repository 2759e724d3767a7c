"""The seeded generators: determinism, independence of streams, the stated
distributions, and the residency tables' structure."""
import numpy as np
import scipy.stats

from quantized_routed_expert_rl_amd import synth, workloads


def test_same_seed_same_bytes_and_streams_independent():
    w = workloads.get("tiny")
    a = synth.expert_slot(w, 0, 5)
    assert np.array_equal(a, synth.expert_slot(w, 0, 5))
    assert not np.array_equal(a, synth.expert_slot(w, 0, 6))
    assert not np.array_equal(a, synth.expert_slot(w, 0, 5, seed=1))
    assert np.array_equal(synth.router_weights(w, 0), synth.router_weights(w, 0))
    assert np.array_equal(synth.activations(w, 4, 1), synth.activations(w, 4, 1))
    assert not np.array_equal(synth.activations(w, 4, 1), synth.activations(w, 4, 2))


def test_code_and_scale_uniformity_and_d_range():
    w = workloads.get("decode_1l")
    slot = synth.expert_slot(w, 0, 0)
    lay = synth.plane_offsets(w.hidden * w.width, 2)
    nb = lay["nb"]
    q = slot[lay["q"]:lay["q"] + nb * 64]
    codes = np.concatenate([(q >> s) & 3 for s in (0, 2, 4, 6)])
    chi = scipy.stats.chisquare(np.bincount(codes, minlength=4))
    assert chi.pvalue > 1e-4
    sb = slot[lay["s"]:lay["s"] + nb * 4]
    nib = np.concatenate([sb & 15, sb >> 4])
    assert scipy.stats.chisquare(np.bincount(nib, minlength=16)).pvalue > 1e-4
    d = slot[lay["d"]:lay["d"] + nb * 2].copy().view(np.float16).astype(np.float64)
    assert d.min() >= 0.0099 and d.max() <= 0.0501
    assert abs(d.mean() - 0.03) < 1e-3


def test_normal_moments():
    w = workloads.get("decode_1l")
    W = synth.router_weights(w, 0).astype(np.float64)
    assert abs(W.mean()) < 1e-3 and abs(W.std() - 0.05) < 1e-3
    x = synth.activations(w, 64).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def test_zipf_bias():
    w = workloads.get("decode_48l")
    b = synth.router_bias(w, 3).astype(np.float64)
    ranks = np.round(np.exp(-b / 1.1)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, 513))
    assert synth.router_bias(workloads.get("decode_1l"), 0) is None


def test_residency_tables():
    w = workloads.get("decode_1l")
    t = synth.residency(w)
    assert t.shape == (1, 512) and sorted(t[0].tolist()) == list(range(512))
    w2 = workloads.get("decode_48l")
    t2 = synth.residency(w2)
    assert t2.shape == (48, 512)
    res = t2[t2 >= 0]
    assert res.size == 4608 and sorted(res.tolist()) == list(range(4608))
    w4 = workloads.get("prefill_48l")
    t4 = synth.residency(w4)
    assert sorted(t4.reshape(-1).tolist()) == list(range(48 * 512))


def test_pool_places_each_expert_at_its_slot():
    w = workloads.get("tiny")
    t = synth.residency(w)
    pool = synth.build_pool(w, t)
    for e in (0, 7, 15):
        assert np.array_equal(pool[t[0, e]], synth.expert_slot(w, 0, e))
    part = synth.fill_slots(w, t, 4, 3)
    assert np.array_equal(part, pool[4:7])


def test_real_shapes_match_the_figures_the_notes_print():
    """The real-shape workloads use the layer and chunk shape the notes print
    (tests/golden/layer_shape.txt, each figure with its page and section)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "layer_shape.txt")
    fig = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            name, value = line.split()[:2]
            fig[name] = int(value)
    for name in ("decode_1l", "decode_48l", "decode_48l_hot", "prefill_1l"):
        w = workloads.get(name)
        assert (w.hidden, w.width, w.top_k) == (fig["hidden"], fig["width"], fig["top_k"]), name
    p = workloads.get("prefill_1l")
    assert p.tokens == fig["prefill_chunk"] and p.plan_cap == fig["plan_cap"]
    p48 = workloads.get("prefill_48l")
    assert max(p48.chunks) == fig["prefill_chunk"] and p48.plan_cap == fig["plan_cap"]
