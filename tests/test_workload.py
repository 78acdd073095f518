"""The seeded input generator: shapes, dtypes, determinism and peaked logits (CPU)."""
import torch

import saga_workload as wl


def test_shapes_and_determinism():
    w = wl.TINY
    a = wl.make_layer(w, 0)
    b = wl.make_layer(w, 0)
    assert a["K"].shape == (1, 1, w.rows, 64) and a["V"].shape == (1, 2, w.rows, 64)
    assert a["q"].shape == (w.steps, 1, 4, 64)
    for k in ("K", "V", "q"):
        assert a[k].dtype == torch.bfloat16 and torch.equal(a[k], b[k])
    c = wl.make_layer(w, 1)
    assert not torch.equal(a["K"], c["K"])


def test_heavy_hitters_make_logits_peaked():
    w = wl.TINY
    x = wl.make_layer(w, 0)
    y = wl.make_layer(w, 0, heavy_hitters=False)
    changed = (x["K"] != y["K"]).any(dim=-1)[0, 0]                   # [rows]
    assert int(changed.sum()) == round(0.01 * w.rows)
    # A shifted key gains ~3|q_0| ~ 3 of logit for the query head it was dealt to.
    s = lambda d: (d["q"][0, 0].float() @ d["K"][0, 0].float().T)    # [hq][rows]
    gain = (s(x) - s(y))[:, changed].max(dim=0).values
    assert gain.min() > 2.0 and gain.max() < 4.5


def test_workload_table():
    assert wl.LLAMA_128K_B16.kv_bytes() == 16 * 16 * 12 * (131072 + 32) * 64 * 2
    assert len(wl.sweep()) == 60
    assert wl.QWEN_128K_B1.gqa(2).h_k == 2
