"""The oracle's simulated quantization for the error study of "Four Over Six"
sec. 2.2 (Fig. 2), CPU only.

Pins tie the simulation to the already pinned quantizer (with no error
source switched off it must reproduce dequantize(quantize(x)) bit for bit;
the two ends of the threshold sweep must equal the value-HP and the plain
simulation), then check the page's findings as properties of the synthetic
analogue: scale rounding is the minor source of error, the error with
unrounded values is fp32 round-off only, and the error grows fastest when
values around 5 (where FP4 has no grid point between 4 and 6) are rounded.
The stored sweep (tests/golden/error_study_fig2.json, written by
make_error_study.py through the oracle only) must be reproduced."""
import json
import os

import numpy as np
import pytest

import oracle as O
import synthetic as S

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "error_study_fig2.json")


def rel_err(out, x):
    y = S.bf16_bits_to_f32(x).astype(np.float64)
    return float(((out.astype(np.float64) - y) ** 2).sum() / (y * y).sum())


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("wl,shape", [("c1", (256, 1024)), ("c2", (96, 1040))])
def test_simulation_without_switch_is_the_quantizer(wl, shape):
    x = S.gen(wl, *shape)
    q = O.nvfp4_quantize(x, 0)
    d = O.dequantize(0, q["codes"], q["scales"], q["alpha"], *shape)
    sim = O.nvfp4_simulate(x, O.SIM_NVFP4)
    assert np.array_equal(sim.view(np.uint32), d.view(np.uint32))


def test_threshold_ends():
    x = S.gen("c2", 64, 1024)
    none = O.nvfp4_simulate(x, O.SIM_THRESHOLD, 0.0)
    assert np.array_equal(none.view(np.uint32), O.nvfp4_simulate(x, O.SIM_VALUE_HP).view(np.uint32))
    # after E4M3 rounding of the block scale a scaled value is at most
    # 6 * (1 + 2^-4) < 6.5, so every value is rounded
    full = O.nvfp4_simulate(x, O.SIM_THRESHOLD, 6.5)
    assert np.array_equal(full.view(np.uint32), O.nvfp4_simulate(x, O.SIM_NVFP4).view(np.uint32))


def test_value_hp_is_roundoff_only():
    x = S.gen("c4", 64, 2048)
    assert rel_err(O.nvfp4_simulate(x, O.SIM_VALUE_HP), x) < 1e-12


def test_scale_hp_keeps_the_block_max_on_the_grid():
    """With the block scale unrounded, each block's largest value scales to
    6 up to fp32 rounding, so its dequantized value is within 1e-6 relative."""
    x = S.gen("c1", 32, 256)
    out = O.nvfp4_simulate(x, O.SIM_SCALE_HP).reshape(32, 16, 16)
    y = S.bf16_bits_to_f32(x).reshape(32, 16, 16)
    i = np.abs(y).argmax(axis=2)
    ym = np.take_along_axis(y, i[..., None], axis=2)
    om = np.take_along_axis(out, i[..., None], axis=2)
    nz = ym != 0
    assert np.all(np.abs(om[nz] - ym[nz]) <= 1e-6 * np.abs(ym[nz]))


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.nvfp4_simulate(S.gen("c1", 4, 24), O.SIM_NVFP4)
    with pytest.raises(ValueError):
        O.nvfp4_simulate(S.gen("c1", 4, 32), 7)


def test_golden_reproduced_and_findings(golden):
    ws = golden["workloads"]
    # the cheapest workload is recomputed in full; the others spot-checked
    x = S.gen("c1", *ws["c1"]["shape"])
    assert rel_err(O.nvfp4_simulate(x, O.SIM_NVFP4), x) == pytest.approx(ws["c1"]["nvfp4"], rel=1e-12)
    for t, e in ws["c1"]["threshold"]:
        assert rel_err(O.nvfp4_simulate(x, O.SIM_THRESHOLD, t), x) == pytest.approx(e, rel=1e-12,
                                                                                    abs=1e-18)
    for wl, r in ws.items():
        sweep = dict((round(t, 2), e) for t, e in r["threshold"])
        es = [e for _, e in r["threshold"]]
        # cumulative: rounding more values never lowers the error
        assert all(b >= a for a, b in zip(es, es[1:])), wl
        # end points: nothing rounded = value-HP, everything rounded = NVFP4
        assert sweep[0.0] == pytest.approx(r["value_hp"], rel=1e-12, abs=1e-18)
        assert sweep[6.5] == pytest.approx(r["nvfp4"], rel=1e-12)
        # Fig. 2(a): the E4M3 scale is the minor source, FP4 values the major one
        assert 0.5 * r["nvfp4"] < r["scale_hp"] < r["nvfp4"], wl
        assert r["value_hp"] < 1e-9 * r["nvfp4"], wl
        # Fig. 2(b): the error grows fastest where values around 5 get rounded
        assert sweep[5.5] - sweep[4.5] > 2.0 * (sweep[4.5] - sweep[3.5]), wl
        # the premise of 4/6: the adaptive choice lowers the error
        assert r["four_over_six"] < r["nvfp4"], wl
