"""The seeded input generator is deterministic and has the stated shapes."""
import numpy as np

import synth


def test_same_seed_same_bytes():
    w = synth.scaled(synth.WORKLOADS["tiny"], steps=3)
    a, b = synth.draw_run(w), synth.draw_run(w)
    for la, lb in zip(a.layers, b.layers):
        for k in synth.WEIGHT_ORDER:
            assert la[k].tobytes() == lb[k].tobytes()
    assert a.x.tobytes() == b.x.tobytes() and a.s0.tobytes() == b.s0.tobytes()


def test_shapes_and_bf16_inputs():
    w = synth.scaled(synth.WORKLOADS["verify"], n_layers=2, steps=2)
    r = synth.draw_run(w)
    d = w.dims
    assert r.layers[0]["wq"].shape == (d.key_dim, d.d_model)
    assert r.layers[0]["wo"].shape == (d.d_model, d.value_dim)
    assert r.layers[0]["conv_w"].shape == (d.conv_channels, 4)
    assert r.s0.shape == (2, 8, 16, 128, 128)
    assert r.x.shape == (2, 8, 4, 2048)
    assert r.accept.shape == (2, 8) and r.accept.min() >= 1 and r.accept.max() <= 4
    # x is exactly representable in BF16 and matches its bit patterns
    assert np.all((r.x.view(np.uint32) & 0xFFFF) == 0)
    assert np.array_equal((r.x.view(np.uint32) >> 16).astype(np.uint16), r.x_bits)
