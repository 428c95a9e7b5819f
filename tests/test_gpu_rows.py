"""GPU parity of NVFP4 with one FP32 scale per row (one read of the input)
against the CPU oracle, bit for bit: codes, E4M3 scales, the per-row FP32
scales and the 4/6 choice, for RTN6, 4/6, SR and RHT16 (the rotation is the
same fp32 butterfly on both sides).  Shapes cover rows held in registers
(one chunk per wave, 1/4/8 blocks per lane), rows swept twice (longer than
8192 values), ragged row lengths, thin and empty tensors, and the full
8192x4096 activation."""
import numpy as np
import pytest

import oracle as O
import synthetic as S

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_reduce_amd as fp4  # noqa: E402

SEED = 0x0123456789ABCDEF
FLAG_SETS = [0, fp4.FOUR_OVER_SIX, fp4.SR, fp4.RHT16, fp4.RHT16 | fp4.SR,
             fp4.RHT16 | fp4.FOUR_OVER_SIX]


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def run_case(x, flags, seed=SEED, ctx=""):
    print("rows case", ctx, x.shape, "flags", flags, flush=True)
    got = fp4.nvfp4_quantize_rows(dev(x), flags, seed=seed, want_choice=True)
    torch.cuda.synchronize()
    want = O.nvfp4_quantize_rows(x, flags, seed=seed)
    keys = ["codes", "scales"] + (["choice"] if flags & fp4.FOUR_OVER_SIX else [])
    for k in keys:
        g, w = got[k].cpu().numpy(), want[k]
        assert g.shape == w.shape, (ctx, k)
        bad = np.argwhere(g != w)
        assert bad.size == 0, "%s flags=%d: %s differs at %d places, first %s: gpu %s oracle %s" % (
            ctx, flags, k, len(bad), bad[:3].tolist(), g[tuple(bad[0])], w[tuple(bad[0])])
    ga = got["alpha"].cpu().numpy()[:x.shape[0]]
    assert np.array_equal(ga, want["alpha"]), ctx
    return got, want


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("wl,shape", [("c1", (40, 1024)), ("c2", (96, 4112)), ("c2", (33, 4096)),
                                      ("c4", (12, 14336)), ("c3", (7, 48))])
def test_rows_parity(wl, shape, flags):
    run_case(S.gen(wl, *shape), flags, ctx=wl)


@pytest.mark.parametrize("flags", [0, fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR])
def test_rows_special_values(flags):
    run_case(S.special_values_tensor(48, 272), flags, ctx="special")


@pytest.mark.parametrize("flags", [fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR])
@pytest.mark.parametrize("rows", [4607, 4609, 9217])
def test_rows_launch_edges(rows, flags):
    """Row counts around the workgroups the workgroup-per-row kernel launches
    for 4096-value rows (three times those resident: 4608 on 256 CUs at six
    per CU): one row each with one workgroup idle, one workgroup taking a
    second row, and every workgroup two or three."""
    run_case(S.gen("c2", rows, 4096), flags, ctx="launch-edge")


def test_rows_edge_shapes():
    run_case(S.gen("c2", 1, 16), fp4.FOUR_OVER_SIX, ctx="one block")
    run_case(S.gen("c2", 3, 16400), fp4.FOUR_OVER_SIX, ctx="three sweeps")
    run_case(S.gen("c2", 5, 8192 + 16), fp4.RHT16 | fp4.SR, ctx="two sweeps, ragged")
    x = S.gen("c2", 8, 64)
    x[3] = 0
    x[5] = 0x8000
    run_case(x, fp4.FOUR_OVER_SIX, ctx="zero rows")
    got = fp4.nvfp4_quantize_rows(torch.zeros((0, 64), dtype=torch.int16, device="cuda"), 0)
    torch.cuda.synchronize()
    assert got["codes"].numel() == 0


def test_rows_full_activation():
    run_case(S.gen("c2"), fp4.FOUR_OVER_SIX, ctx="c2 full")


def test_rows_with_one_amax_match_the_per_tensor_quantizer():
    """Identical rows: the per-row scales equal the tensor scale, so the
    library's two quantizers agree with each other as well."""
    row = S.gen("c2", 1, 4096)
    x = np.ascontiguousarray(np.repeat(row, 64, axis=0))
    a = fp4.nvfp4_quantize_rows(dev(x), fp4.FOUR_OVER_SIX)
    b = fp4.nvfp4_quantize(dev(x), fp4.FOUR_OVER_SIX)
    torch.cuda.synchronize()
    assert torch.equal(a["codes"], b["codes"]) and torch.equal(a["scales"], b["scales"])
    assert torch.all(a["alpha"] == b["alpha"][0])


@pytest.mark.parametrize("flags", [0, fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR])
def test_rows_outside_the_domain_leave_the_others_exact(flags):
    """Rows whose largest magnitude is non-zero but below 2^-64 (bf16
    subnormals; normals near 2^-80) are outside the domain: the call must
    succeed, and every other row (a zero row included) must still equal the
    oracle bit for bit."""
    rng = np.random.default_rng(5)
    x = S.gen("c2", 24, 4096)
    x[5] = (rng.integers(1, 0x80, 4096) | (rng.integers(0, 2, 4096) << 15)).astype(np.uint16)
    x[9] = S.f32_to_bf16_bits((rng.standard_normal(4096) * 2.0 ** -80).astype(np.float32))
    x[13] = 0
    print("rows case out of domain", flags, flush=True)
    got = fp4.nvfp4_quantize_rows(dev(x), flags, seed=SEED, want_choice=True)
    torch.cuda.synchronize()
    want = O.nvfp4_quantize_rows(x, flags, seed=SEED)
    keep = np.setdiff1d(np.arange(24), [5, 9])
    for k in ("codes", "scales") + (("choice",) if flags & fp4.FOUR_OVER_SIX else ()):
        assert np.array_equal(got[k].cpu().numpy()[keep], want[k][keep]), k
    ga = got["alpha"].cpu().numpy()[:24]
    assert np.array_equal(ga, want["alpha"])           # alpha_r = amax_r / (6 C) on every row
