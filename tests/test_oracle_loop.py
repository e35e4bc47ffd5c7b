"""Composite step loop of the oracle (no GPU).

The loop as a whole is "parity unpinned" beyond its parts: no page prints a numeric
worked example of entropy-bounded acceptance or self-conditioning. These checks pin
what the method and the synthetic driver fix: the canvas converges to the driver's
targets, the budget holds at every step, accepted tokens are the argmax, the stop test
only fires on its two conditions, the commit appends exactly C rows.
"""
import numpy as np

import dg_inputs as di
import oracle as O


def test_tiny_loop_invariants():
    cfg = di.config(0)
    W = di.weights(cfg)
    Kp, Vp = di.prefix_kv(cfg)
    K0 = Kp.copy()
    tgt = di.targets(cfg, 0)
    P, recs = O.run_canvas(W, Kp, Vp, cfg.P0, lambda k: di.hidden(cfg, W["E"], 0, k, tgt),
                           V=cfg.V, C=cfg.C, Hq=cfg.Hq, Hkv=cfg.Hkv, hd=cfg.hd, N=cfg.N,
                           seed=cfg.seed, canvas=0)
    assert P == cfg.P0 + cfg.C
    np.testing.assert_array_equal(Kp[:, :cfg.P0], K0[:, :cfg.P0])
    assert [r["flag"] for r in recs] == [0] * (cfg.N - 1) + [O.STOP_CAP]
    assert (recs[-1]["argmax"] == tgt).all()
    for r in recs:
        acc = r["accept"].astype(bool)
        assert (r["tokens"][acc] == r["argmax"][acc]).all()
        assert r["entropy"][acc].astype(np.float64).sum() <= float(np.float32(0.1))
        assert r["tau"] == O.temperature(r["k"], cfg.N)
        assert r["A"].shape == (cfg.C, cfg.d)
    # entropy falls as the driver sharpens the logits
    means = [float(r["entropy"].mean()) for r in recs]
    assert means[-1] < means[0] / 10
    # the committed block is the last argmax
    Kn = O.from_bf16(Kp[:, cfg.P0:P])
    ref = O.from_bf16(O.to_bf16(O.from_bf16(W["E"][recs[-1]["argmax"]]) @ O.from_bf16(W["Wk"]).T))
    np.testing.assert_array_equal(Kn, ref.reshape(cfg.C, cfg.Hkv, cfg.hd).transpose(1, 0, 2))


def test_loop_stops_early_when_driver_is_confident():
    # a driver that is already sharp: entropies ~0 and a stable argmax -> stop at step 1
    cfg = di.config(0).with_(alpha_max=400.0)
    W = di.weights(cfg)
    Kp, Vp = di.prefix_kv(cfg)
    tgt = di.targets(cfg, 0)
    H = di.f32_to_bf16_bits(200.0 * di.bf16_bits_to_f32(W["E"][tgt]))
    P, recs = O.run_canvas(W, Kp, Vp, cfg.P0, lambda k: H, V=cfg.V, C=cfg.C, Hq=cfg.Hq,
                           Hkv=cfg.Hkv, hd=cfg.hd, N=cfg.N, seed=cfg.seed, canvas=0,
                           with_attn=False)
    assert [r["flag"] for r in recs] == [0, O.STOP_STOP]
    assert recs[0]["n_accept"] == cfg.C
