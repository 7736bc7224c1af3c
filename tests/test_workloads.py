"""The seeded input generator (CPU only): determinism, the shared draw of
the decode FP8 layers, and the stated recipe for weights and routing."""
import hashlib

import numpy as np

import moe_workloads as wl


def _digest(L):
    h = hashlib.sha256()
    for key in ("x", "logits", "w13", "w2", "w13_scale", "w2_scale"):
        a = L.get(key)
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes_other_seed_other_bytes():
    a = wl.make_layer(wl.scaled("d", 9, 256, 8, 2, 128, wl.FP8, seed=5))
    b = wl.make_layer(wl.scaled("d", 9, 256, 8, 2, 128, wl.FP8, seed=5))
    c = wl.make_layer(wl.scaled("d", 9, 256, 8, 2, 128, wl.FP8, seed=6))
    assert _digest(a) == _digest(b)
    assert _digest(a) != _digest(c)


def test_decode_fp8_layers_share_one_draw():
    l16 = wl.make_layer(wl.WORKLOADS["decode_fp8_t16"], with_weights=False)
    for T in (1, 4):
        lt = wl.make_layer(wl.WORKLOADS["decode_fp8_t%d" % T], with_weights=False)
        assert np.array_equal(lt["x"], l16["x"][:T])
        assert np.array_equal(lt["logits"], l16["logits"][:T])


def test_fp8_weights_recipe():
    L = wl.make_layer(wl.scaled("w", 4, 256, 3, 2, 128, wl.FP8, seed=2))
    for key, sk in (("w13", "w13_scale"), ("w2", "w2_scale")):
        codes = L[key]
        assert not np.any((codes & 0x7F) == 0x7F)  # no NaN codes
        # every matrix reaches the top code 0x7e (+-448) somewhere: scale = amax/448
        for e in range(codes.shape[0]):
            assert np.max(codes[e] & 0x7F) == 0x7E
        assert np.all(L[sk] > 0)


def test_routing_recipes():
    s = wl.scaled("z", 64, 128, 40, 4, 128, wl.BF16, routing="empty", seed=3)
    L = wl.make_layer(s, with_weights=False)
    dead = np.all(np.isneginf(L["logits"]), axis=0)
    assert dead.sum() == round(0.1 * 40)
    z = wl.make_layer(wl.scaled("z", 64, 128, 40, 4, 128, wl.BF16, routing="zipf", seed=3),
                      with_weights=False)
    u = wl.make_layer(wl.scaled("z", 64, 128, 40, 4, 128, wl.BF16, routing="uniform", seed=3),
                      with_weights=False)
    bias = (z["logits"].astype(np.float64) - u["logits"].astype(np.float64)).mean(axis=0)
    # the bias is -1.1 ln(r) for a permutation r of 1..E
    ranks = np.exp(-bias / 1.1)
    assert np.allclose(np.sort(ranks), np.arange(1, 41), atol=1e-3)


def test_planted_logits_give_the_planted_counts():
    import oracle
    for T, E, k, counts in ((2432, 8, 1, [0, 1, 255, 256, 257, 511, 512, 640]),
                            (4200, 8, 2, [0, 256, 257, 511, 1024, 1280, 2520, 2552]),
                            (5, 4, 4, [5, 5, 5, 5])):
        ids, _ = oracle.topk_gating(wl.planted_logits(T, E, k, counts, seed=3), k)
        assert np.array_equal(np.bincount(ids.ravel(), minlength=E), counts)
        assert all(len(set(r)) == k for r in ids.tolist())
