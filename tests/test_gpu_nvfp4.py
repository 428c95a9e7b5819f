"""GPU parity of the NVFP4 1D path against the CPU oracle (bit for bit).

Codes, E4M3 scales, the FP32 tensor scale and the 4/6 choice must match the
oracle exactly for RTN, 4/6 and SR, with and without the 16-point random
Hadamard (both sides run the same fp32 butterfly, so rotated results are
exact too).  Inputs come from the seeded generators; sizes span several
workgroups and a ragged tail; the full workload shapes are checked whole.
"""
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


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def host(t):
    return t.cpu().numpy()


def check_same(got, want, keys, ctx):
    for k in keys:
        g, w = host(got[k]), want[k]
        if g.shape != w.shape:
            raise AssertionError("%s: %s shape %s vs %s" % (ctx, k, g.shape, w.shape))
        bad = np.argwhere(g != w)
        assert bad.size == 0, "%s: %s differs at %d places, first %s: gpu %s oracle %s" % (
            ctx, k, len(bad), bad[:3].tolist(), g[tuple(bad[0])], w[tuple(bad[0])])


def run_case(x, flags, seed=SEED, amax_in=False):
    print("case", x.shape, "flags", flags, "seed", hex(seed), "amax_in", amax_in, flush=True)
    xt = dev(x)
    amax = None
    want_amax = None
    if amax_in:
        want_amax = np.float32(O.tensor_amax(x, flags, seed))
        amax = torch.tensor([want_amax], dtype=torch.float32, device="cuda")
    got = fp4.nvfp4_quantize(xt, flags, seed=seed, amax=amax, want_choice=True)
    torch.cuda.synchronize()
    want = O.nvfp4_quantize(x, flags, seed=seed, amax=want_amax)
    keys = ["codes", "scales"] + (["choice"] if flags & fp4.FOUR_OVER_SIX else [])
    check_same(got, want, keys, "flags=%d shape=%s" % (flags, x.shape))
    assert host(got["alpha"])[0] == want["alpha"]
    return got, want


FLAG_SETS = [0, fp4.FOUR_OVER_SIX, fp4.SR, fp4.RHT16, fp4.RHT16 | fp4.SR,
             fp4.RHT16 | fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.MSEDEN]


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("wl,shape", [("c1", (256, 1024)), ("c2", (96, 4112)),
                                      ("c4", (37, 1008)), ("c3", (5, 16))])
def test_parity_small(wl, shape, flags):
    run_case(S.gen(wl, *shape), flags)


@pytest.mark.parametrize("flags", [0, fp4.FOUR_OVER_SIX, fp4.SR, fp4.RHT16 | fp4.SR,
                                   fp4.RHT16 | fp4.MSEDEN])
def test_parity_special_values(flags):
    run_case(S.special_values_tensor(48, 272), flags)


@pytest.mark.parametrize("flags", [fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR])
def test_parity_amax_given(flags):
    run_case(S.gen("c2", 64, 1024), flags, amax_in=True)


def test_parity_c1_full_with_dequant():
    x = S.gen("c1")
    got, want = run_case(x, 0)
    d = fp4.fp4_dequantize(fp4.FORMAT_NVFP4, got["codes"], got["scales"], got["alpha"], *x.shape)
    dw = O.dequantize(0, want["codes"], want["scales"], want["alpha"], *x.shape)
    assert np.array_equal(host(d), dw)


def test_parity_c2_full():
    run_case(S.gen("c2"), fp4.FOUR_OVER_SIX)


def test_parity_c4_full():
    x = S.gen("c4")
    got, want = run_case(x, fp4.RHT16 | fp4.SR)


def test_parity_c4_full_msed():
    """MS-EDEN on the full gradient: RTN values against the unrounded scale,
    EDEN's factor and one stochastic scale draw per block, bit for bit."""
    run_case(S.gen("c4"), fp4.RHT16 | fp4.MSEDEN)


def test_parity_workloads_at_other_sizes():
    """Row counts that leave partial chunks for the persistent workgroups."""
    for rows in (8193, 9000):
        run_case(S.gen("c2", rows, 4096), fp4.FOUR_OVER_SIX)


@pytest.mark.parametrize("flags", [0, fp4.FOUR_OVER_SIX, fp4.SR])
@pytest.mark.parametrize("shape", [(1000, 4096), (1600, 4112)])
def test_parity_chunk_order(shape, flags):
    """Unrotated shapes whose grid is a multiple of 8, so the workgroups take
    their chunks in the amax pass's XCD order: 1000 chunks (a grid of 1000,
    a chunk count that is not a multiple of 64) and 1607 chunks with a
    partial last one (a grid of 1536 on 256 CUs without SR; with SR every
    chunk gets a workgroup of its own).  Every chunk must be quantized once,
    the SR counter must stay the element index."""
    run_case(S.gen("c2", *shape), flags)


@pytest.mark.parametrize("flags", [fp4.SR, fp4.RHT16 | fp4.SR, fp4.RHT16 | fp4.MSEDEN])
@pytest.mark.parametrize("rows", [3071, 3073, 6145])
def test_parity_launch_edges(rows, flags):
    """Chunk counts (a chunk is 4096 values: one 4096-value row here) around
    the 3072 workgroups the SR and MS-EDEN kernels launch on 256 CUs (twelve
    per CU, four resident): one chunk each with one workgroup idle, one
    workgroup taking a second chunk, and every workgroup two or three."""
    run_case(S.gen("c4", rows, 4096), flags)


@pytest.mark.parametrize("flags", [0, fp4.RHT16, fp4.BLOCK2D])
@pytest.mark.parametrize("shape", [(130, 4096), (16, 16), (4112, 4112), (8208, 4096)])
def test_tensor_amax(shape, flags):
    """Both forms of the amax pass (1D: 512-thread workgroups on 32 KiB
    chunks; 2D and rotated: 1024 threads, 64 KiB), with partial last chunks
    and more chunks than workgroups; the largest magnitude planted in the
    tensor's last element, then elsewhere."""
    x = S.gen("c4", *shape)
    for pos in (x.size - 1, x.size // 3):
        y = x.copy().reshape(-1)
        y[pos] = 0xC2C8                                   # -100.0 in bf16
        y = y.reshape(shape)
        print("amax case", shape, "flags", flags, "pos", pos, flush=True)
        a = fp4.fp4_tensor_amax(dev(y), flags, SEED)
        torch.cuda.synchronize()
        # the oracle's amax takes only the rotation flag (2D tiles change nothing)
        assert host(a)[0] == np.float32(O.tensor_amax(y, flags & fp4.RHT16, SEED))


def test_edge_shapes():
    # one block, one row, empty
    run_case(S.gen("c2", 1, 16), fp4.FOUR_OVER_SIX)
    run_case(S.gen("c2", 1, 4096 + 16), fp4.FOUR_OVER_SIX)
    x = np.zeros((0, 64), np.uint16)
    got = fp4.nvfp4_quantize(torch.zeros((0, 64), dtype=torch.int16, device="cuda"), 0)
    torch.cuda.synchronize()
    assert host(got["alpha"])[0] == 0.0
    # all-zero tensor: alpha 0, codes 0
    run_case(np.zeros((16, 64), np.uint16), fp4.FOUR_OVER_SIX)
    run_case(np.full((16, 64), 0x8000, np.uint16), 0)


def test_deterministic():
    x = dev(S.gen("c4", 256, 2048))
    a = fp4.nvfp4_quantize(x, fp4.RHT16 | fp4.SR, seed=SEED)
    b = fp4.nvfp4_quantize(x, fp4.RHT16 | fp4.SR, seed=SEED)
    c = fp4.nvfp4_quantize(x, fp4.RHT16 | fp4.SR, seed=SEED + 1)
    torch.cuda.synchronize()
    assert torch.equal(a["codes"], b["codes"]) and torch.equal(a["scales"], b["scales"])
    assert not torch.equal(a["codes"], c["codes"])
