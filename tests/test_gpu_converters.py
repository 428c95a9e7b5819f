"""GPU pin of the number-format conversions, through the real kernels.

The quantizers convert on gfx950's own instructions: fp32 -> E2M1 with
nearest-even rounding and saturation at 6, fp32 -> E4M3 with nearest-even
rounding (after a clamp to [0, 448]), E2M1 -> fp32, and power-of-two
scaling by a UE8M0 exponent (a zero exponent meaning 2^-127).  These tests
feed every finite bf16 bit pattern through the kernels in blocks built so
that the scaled values land exactly on the interesting points, and compare
codes, scales, choices and decodes with the oracle bit for bit:

* NVFP4 (RTN, Four Over Six, stochastic rounding, no rotation): each block
  holds an anchor 6 * 2^E (its maximum) and members y with |y| <= 6 * 2^E.
  The caller's amax makes alpha a power of two (6 * 448 * 2^j, or
  6 * 256 * 2^j with Four Over Six), so alpha * Delta is a power of two
  and the scaled values y / 2^E are exact: every E2M1 midpoint 0.25, 0.75,
  1.25, 1.75, 2.5, 3.5, 5 and its bf16 neighbours is reached, for every
  bf16 exponent.  Blocks whose anchor exceeds the caller's amax drive the
  block scale past 448 (saturation) and the scaled values past 6.
* E4M3 block scales: block maxima on every bf16 value in [2^-12, 2^10)
  times 2^j with an amax that makes the encode factor 2^-j, so the
  unrounded scale is that value exactly: every E4M3 midpoint (normal and
  subnormal), its neighbours and saturation above 448.
* MXFP4 without rotation: each 32-value group holds an anchor just below
  2^(e+3) (so its exponent is e) and members down to 2^(e-4), for every e
  the format has, plus groups of bf16 subnormals only (exponent clamped to
  -127, scale code 0) and all-zero groups; both orientations.
* Decodes: every code byte under every E4M3 and UE8M0 scale code.
("Four Over Six" sec. 1 and sec. 2.1, Eq. 1-3; NVIDIA NVFP4 article sec. 1,
sec. 4 and sec. 6.)
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

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE = ALL[((ALL >> 7) & 0xFF) != 0xFF]                 # 65280 patterns
MAG = np.abs(S.bf16_bits_to_f32(FINITE).astype(np.float64))
NZ = MAG > 0
EXP = np.full(FINITE.shape, -1000, np.int64)
EXP[NZ] = np.floor(np.log2(MAG[NZ])).astype(np.int64)
BF16_MAX = float(S.bf16_bits_to_f32(np.array([0x7F7F], np.uint16))[0])


def bits(v):
    """Exact float64 values (bf16-representable) -> bf16 bit patterns."""
    b = S.f32_to_bf16_bits(np.asarray(v, np.float32))
    assert np.array_equal(S.bf16_bits_to_f32(b).astype(np.float64), np.asarray(v, np.float64))
    return b


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def host(t):
    return t.cpu().numpy()


def same(g, w, what):
    g = host(g) if torch.is_tensor(g) else np.asarray(g)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.argwhere(g != w)
    assert bad.size == 0, "%s differs at %d places, first %s: gpu %s oracle %s" % (
        what, len(bad), bad[:3].tolist(), g[tuple(bad[0])], w[tuple(bad[0])])


def pack_blocks(blocks, n, cols):
    """List of n-value blocks (bf16 bits) -> [rows][cols] tensor, padded
    with zero blocks; the anchor (element 0) is rotated to position i % n."""
    per_row = cols // n
    nb = -(-len(blocks) // per_row) * per_row
    out = np.zeros((nb, n), np.uint16)
    for i, b in enumerate(blocks):
        out[i] = np.roll(b, i % n)
    return out.reshape(-1, cols)


def anchored_blocks(anchor_of_E, E_values, n, rng):
    """Blocks of n values: for each E, the anchor anchor_of_E(E) and members
    = every finite pattern with exponent in [E-3, E+2] and magnitude at most
    the anchor's, shuffled, n-1 per block."""
    blocks = []
    for E in E_values:
        a = anchor_of_E(E)
        if a is None:
            continue
        ab = bits([a])[0]
        sel = (EXP >= E - 3) & (EXP <= E + 2) & (MAG <= a)
        mem = rng.permutation(FINITE[sel])
        for i in range(0, len(mem), n - 1):
            chunk = mem[i:i + n - 1]
            blocks.append(np.concatenate([[ab], chunk, np.zeros(n - 1 - len(chunk), np.uint16)]))
    return blocks


def nvfp4_sweep_inputs(j, four_six, rng, lowest=False, highest=False):
    """Blocks for one call with alpha = 2^j (see the module docstring)."""
    def anchor(E):
        a = 6.0 * 2.0 ** E
        return a if a <= BF16_MAX else None
    blocks = anchored_blocks(anchor, range(j - 9, j + 11), 16, rng)
    fill = []
    if lowest:                                   # every smaller pattern (incl. +-0, subnormals)
        fill = list(rng.permutation(FINITE[EXP < j - 12]))
    if highest:                                  # patterns above every anchor: own blocks
        sel = MAG > 6.0 * 2.0 ** (j + 9)
        top = FINITE[sel][np.argsort(MAG[sel], kind="stable")]
        for i in range(0, len(top), 16):
            c = top[i:i + 16]
            blocks.append(np.concatenate([c, np.zeros(16 - len(c), np.uint16)]))
    for i in range(0, len(fill), 15):            # small fillers into existing blocks
        b = blocks[(i // 15) % len(blocks)]
        blocks.append(np.concatenate([[b[0]], fill[i:i + 15],
                                      np.zeros(15 - len(fill[i:i + 15]), np.uint16)]))
    return pack_blocks(blocks, 16, 256)


J_CALLS = list(range(116, -65, -20))             # 116, 96, ..., -64


def run_nvfp4(x, flags, amax, seed=0):
    a = torch.tensor([amax], dtype=torch.float32, device="cuda")
    got = fp4.nvfp4_quantize(dev(x), flags, seed=seed, amax=a, want_choice=True)
    torch.cuda.synchronize()
    want = O.nvfp4_quantize(x, flags, seed=seed, amax=amax)
    for k in ("codes", "scales", "choice"):
        same(got[k], want[k], "%s (flags %d, amax %r)" % (k, flags, amax))
    assert host(got["alpha"])[0] == want["alpha"]
    return want


@pytest.mark.parametrize("mode", ["rtn6", "four_over_six", "sr"])
def test_nvfp4_every_bf16_pattern(mode):
    flags = {"rtn6": 0, "four_over_six": fp4.FOUR_OVER_SIX, "sr": fp4.SR}[mode]
    C = 256.0 if mode == "four_over_six" else 448.0
    rng = np.random.default_rng(7)
    seen = np.zeros(FINITE.shape, bool)
    hits = np.zeros(7, np.int64)
    for j in J_CALLS:
        x = nvfp4_sweep_inputs(j, mode == "four_over_six", rng, lowest=(j == J_CALLS[-1]),
                               highest=(j == J_CALLS[0]))
        seen |= np.isin(FINITE, x)
        print("converter sweep", mode, "j", j, x.shape, flush=True)
        want = run_nvfp4(x, flags, 6.0 * C * 2.0 ** j, seed=0x9E3779B97F4A7C15 + j)
        if mode == "rtn6":                        # scaled values exactly on the midpoints
            t = O.nvfp4_quantize(x, flags, amax=6.0 * C * 2.0 ** j, debug=True)["dbg_t"]
            hits += [(np.abs(t) == b).sum() for b in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)]
    assert seen.all(), "%d bf16 patterns never fed" % int((~seen).sum())
    if mode == "rtn6":
        assert (hits > 0).all(), hits


@pytest.mark.parametrize("mode", ["rtn6", "four_over_six_m6", "four_over_six_m4"])
def test_e4m3_scale_midpoints(mode):
    """Unrounded block scales on every bf16 value of [2^-12, 2^10): all E4M3
    midpoints and their neighbours, subnormal steps, and saturation."""
    flags = 0 if mode == "rtn6" else fp4.FOUR_OVER_SIX
    base = {"rtn6": 448.0, "four_over_six_m6": 256.0, "four_over_six_m4": 384.0}[mode]
    v = np.array([m * 2.0 ** (e - 7) for e in range(-12, 10) for m in range(128, 256)])
    rng = np.random.default_rng(3)
    for j in (0, -30, 40):
        amax = base * 2.0 ** j                   # encode factor 2^-j for the named candidate
        top = v * 2.0 ** j
        f = np.floor(rng.random((len(v), 15)) * 256) / 256
        mem = S.bf16_bits_to_f32(S.f32_to_bf16_bits((top[:, None] * f).astype(np.float32)))
        mem = np.minimum(np.abs(mem), top[:, None].astype(np.float32))
        sgn = rng.random(mem.shape) < 0.5
        memb = S.f32_to_bf16_bits(np.where(sgn, -mem, mem).astype(np.float32))
        blocks = [np.concatenate([[bits([top[i]])[0]], memb[i]]) for i in range(len(v))]
        x = pack_blocks(blocks, 16, 512)
        print("e4m3 sweep", mode, "j", j, x.shape, flush=True)
        run_nvfp4(x, flags, amax)
    # the unrounded scales include every E4M3 midpoint, normal and subnormal
    mids = [(k + 0.5) * 2.0 ** -9 for k in range(8)] + \
        [(8 + m + 0.5) * 2.0 ** (e - 10) for e in range(1, 16) for m in range(8)]
    assert np.isin(np.array(mids), v).all()


def test_nvfp4_caller_amax_below_true_amax():
    """amax_in = half the true amax: block scales saturate at 448 and scaled
    values above 6 saturate (c2-like data)."""
    x = S.gen("c2", 256, 4096)
    true = float(np.abs(S.bf16_bits_to_f32(x)).max())
    for flags in (0, fp4.FOUR_OVER_SIX, fp4.SR):
        want = run_nvfp4(x, flags, 0.5 * true, seed=5)
        assert (want["scales"] == 0x7E).any()


def mx_sweep_tensor(rng):
    """Groups of 32 along rows (see the module docstring), [R][256], R % 32 == 0."""
    def anchor(e):                                # largest bf16 below 2^(e+3): exponent e
        a = 1.9921875 * 2.0 ** (e + 2)
        return a if a <= BF16_MAX and e >= -127 else None
    groups = []
    for e in range(-127, 126):
        a = anchor(e)
        ab = bits([a])[0]
        sel = (EXP >= e - 4) & (EXP <= e + 2) & (MAG <= a)
        mem = rng.permutation(FINITE[sel])
        for i in range(0, len(mem), 31):
            c = mem[i:i + 31]
            groups.append(np.concatenate([[ab], c, np.zeros(31 - len(c), np.uint16)]))
    sel = EXP < -126                              # bf16 subnormals and zeros only
    sub = FINITE[sel][np.argsort(MAG[sel], kind="stable")]
    for i in range(0, len(sub), 32):
        c = sub[i:i + 32]
        groups.append(np.concatenate([c, np.zeros(32 - len(c), np.uint16)]))
    groups.append(np.full(32, 0x8000, np.uint16))  # all -0
    groups.append(np.zeros(32, np.uint16))
    x = pack_blocks(groups, 32, 256)
    pad = (-x.shape[0]) % 32
    return np.concatenate([x, np.zeros((pad, 256), np.uint16)])


def test_mx_every_bf16_pattern_both_orientations():
    rng = np.random.default_rng(11)
    x = mx_sweep_tensor(rng)
    assert np.isin(FINITE, x).all()
    f = fp4.ROWWISE | fp4.COLWISE
    for name, t in (("groups along rows", x), ("groups down columns", np.ascontiguousarray(x.T))):
        print("mx sweep", name, t.shape, flush=True)
        got = fp4.mxfp4_quantize(dev(t), f)
        torch.cuda.synchronize()
        want = O.mxfp4_quantize(t, f)
        for k in want:
            same(got[k], want[k], "%s %s" % (name, k))
    tr = O.mxfp4_quantize(x, fp4.ROWWISE, debug=True)["t_r"]
    for b in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.96875):
        assert (np.abs(tr) == b).any(), b


def test_decode_every_code_and_scale():
    codes = np.arange(256, dtype=np.uint8)
    # NVFP4: [127 scales][256 code bytes] -> one 16-value block = 8 code bytes
    c = np.tile(codes, 127).reshape(127 * 32, 8)
    s = np.repeat(np.arange(127, dtype=np.uint8), 32).reshape(-1, 1)
    for alpha in (1.0, 0.0137, 2.0 ** -20):
        a = torch.tensor([alpha], dtype=torch.float32, device="cuda")
        got = fp4.fp4_dequantize(fp4.FORMAT_NVFP4, torch.from_numpy(c).cuda(),
                                 torch.from_numpy(s).cuda(), a, c.shape[0], 16)
        same(got, O.dequantize(0, c, s, np.float32(alpha), c.shape[0], 16), "nvfp4 decode %r" % alpha)
    # MXFP4: every scale code 0..254 (0 = 2^-127) under every code byte
    c = np.tile(codes, 255 * 16).reshape(255 * 256, 16)
    s = np.repeat(np.arange(255, dtype=np.uint8), 256).reshape(-1, 1)
    got = fp4.fp4_dequantize(fp4.FORMAT_MXFP4, torch.from_numpy(c).cuda(),
                             torch.from_numpy(s).cuda(), None, c.shape[0], 32)
    same(got, O.dequantize(1, c, s, 0.0, c.shape[0], 32), "mx decode")
