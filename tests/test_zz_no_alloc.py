"""GPU check of nvfp4_quantize_noalloc through the C ABI: two calls in a
row (the second on a smaller tensor, so the library's fixed array holds the
first call's partial maxima when it starts) must give exactly what
nvfp4_quantize with a caller workspace gives, and what the oracle gives."""
import ctypes as C

import numpy as np
import pytest

import oracle as O
import synthetic as S

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_reduce_amd as fp4  # noqa: E402


def outputs(rows, cols, flags):
    u8, dev = torch.uint8, "cuda"
    two_d = bool(flags & fp4.BLOCK2D)
    srows = rows // 16 if two_d else rows
    o = dict(codes=torch.full((rows, cols // 2), 0xAB, dtype=u8, device=dev),
             scales=torch.full((srows, cols // 16), 0xAB, dtype=u8, device=dev),
             choice=torch.full((srows, cols // 16), 0xAB, dtype=u8, device=dev),
             alpha=torch.full((1,), -1.0, dtype=torch.float32, device=dev))
    if two_d and flags & fp4.COLWISE:
        o["codes_t"] = torch.full((cols, rows // 2), 0xAB, dtype=u8, device=dev)
        o["scales_t"] = torch.full((cols // 16, rows // 16), 0xAB, dtype=u8, device=dev)
    return o


def call(fn, x, flags, o, extra):
    L = fp4.lib()
    p = lambda k: o[k].data_ptr() if k in o else None
    rows, cols = x.shape
    args = [x.data_ptr(), rows, cols, flags, 0x5EED, None, o["alpha"].data_ptr(), p("codes"),
            p("scales"), p("choice"), p("codes_t"), p("scales_t")]
    rc = getattr(L, fn)(*(args + extra + [torch.cuda.current_stream().cuda_stream]))
    assert rc == 0, (fn, rc, L.fp4_status_str(rc))


CASES = [  # (workload, rows, cols, flags): the second of each pair is smaller
    [("c2", 2048, 4096, fp4.FOUR_OVER_SIX), ("c1", 256, 1024, 0)],
    [("c3", 1024, 2048, fp4.BLOCK2D | fp4.FOUR_OVER_SIX | fp4.COLWISE),
     ("c4", 96, 480, fp4.RHT16 | fp4.SR)],
]


@pytest.mark.parametrize("pair", CASES, ids=["1d", "2d_then_rht_sr"])
def test_noalloc_matches_workspace_entry(pair):
    for wl, rows, cols, flags in pair:
        print("noalloc case", wl, rows, cols, flags, flush=True)
        xn = S.gen(wl, rows, cols)
        x = torch.from_numpy(xn.view(np.int16)).cuda()
        got, ref = outputs(rows, cols, flags), outputs(rows, cols, flags)
        call("nvfp4_quantize_noalloc", x, flags, got, [])
        ws = torch.empty(fp4.fp4_workspace_bytes(rows, cols, flags), dtype=torch.uint8,
                         device="cuda")
        call("nvfp4_quantize", x, flags, ref, [ws.data_ptr(), C.c_size_t(ws.numel())])
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), (wl, k)
        want = O.nvfp4_quantize(xn, flags, seed=0x5EED)
        assert np.array_equal(got["codes"].cpu().numpy(), want["codes"])
        assert np.array_equal(got["scales"].cpu().numpy(), want["scales"])
        assert got["alpha"].cpu().numpy()[0] == want["alpha"]
