"""The seeded synthetic workloads have the shapes and sizes of the pages'
test battery and of the decoder-shaped tensor lists."""
import numpy as np

from bit_companded_adam_amd import workloads as W


def test_battery_shapes_and_seed():
    a, b = W.battery(), W.battery()
    sizes = {k: v.numel() for k, v in a.items()}
    assert sizes == {"normal": 1 << 20, "heavy_tail": 1 << 20, "tiny": 1 << 16,
                     "adam_v_like": 1 << 20, "nonmult32": (1 << 16) + 17,
                     "const_groups": 1 << 12, "with_zeros": 1 << 16}
    for k in a:
        assert a[k].dtype.is_floating_point and (a[k] == b[k]).all()
    z = a["with_zeros"]
    assert 0.28 < float((z == 0).float().mean()) < 0.32
    assert (a["const_groups"] == np.float32(0.37)).all()


def test_split_sweep_structure():
    sw = W.split_sweep(per_exp=1 << 10)
    for width in (24, 32):
        u = sw[width].numpy().view(np.uint32)
        exps = ((u >> 23) & 0xFF).reshape(64, -1)
        assert (exps == np.array(W.SWEEP_EXPONENTS)[:, None]).all()
        neg = (u >> 31).mean()
        assert 0.45 < neg < 0.55


def test_decoder_lists():
    s1 = W.decoder_1b_shapes()
    s8 = W.decoder_8b_shapes()
    assert len(s1) == 199 and len(s8) == 290
    assert sum(W.numel(s) for _, s in s1) == 1_195_991_040
    assert sum(W.numel(s) for _, s in s8) == 8_030_257_152
