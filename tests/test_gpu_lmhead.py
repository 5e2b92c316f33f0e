"""GPU parity of the FP8 LM head against the float64 oracle, through the C ABI.

Quantiser: codes and scales bit-exact (both sides decide in fp32: the scale
amax / 448 and the quotient w / s are fp32 IEEE operations, the rounding to
E4M3 is to nearest even).  Projection: within the fp32 rounding-chain bound of
the kernel's summation (exact products; one token: per lane 16 roundings per
16-byte chunk, a 6-level wave tree, the scale multiply; two or more tokens on
rows a multiple of 256: matrix-core leaves added in K order per wave, the four
waves' sums, the scale multiply)."""
import numpy as np
import pytest

import oracle
from gpu_common import need_gpu, say
from mxfp4_expert_weight_amd import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _logits(torch, x_bits, codes, scales):
    from mxfp4_expert_weight_amd import binding
    M, H = x_bits.shape
    V = codes.shape[0]
    out = torch.full((M, V), float("nan"), dtype=torch.float32, device="cuda")
    binding.moe_lmhead_fp8_logits(_dev(torch, x_bits.view(np.int16)), _dev(torch, codes),
                                  _dev(torch, scales), M, V, H, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _bound(x_bits, codes, scales, H):
    """Rounding-chain bound per logit, chain · u · sum|x w| · s (+ u |ref| at the
    call).  One token, or rows not a multiple of 256: per lane 16 roundings per
    16-byte chunk, a 6-level wave tree, the scale: 16 ceil(H/1024) + 6.  Two or
    more tokens with rows a multiple of 256 (the matrix cores): a 32-product dot
    per leaf (counted as 32 roundings), H/128 leaves per wave added in order,
    the four waves' sums, the scale: 32 + H/128 + 3 + 1."""
    x = oracle.bf16_bits_to_f64(x_bits)
    w = np.abs(oracle.e4m3_decode(codes))
    M = x_bits.shape[0]
    chain = 32 + H // 128 + 4 if M >= 2 and H % 256 == 0 else 16 * -(-H // 1024) + 6
    return (chain * U * (np.abs(x) @ w.T) * scales.astype(np.float64)[None, :]) * 1.01


@pytest.mark.parametrize("V,H", [(300, 2560), (7, 96), (130, 8192), (65, 32)])
def test_quantize_bit_exact(V, H):
    torch = need_gpu()
    from mxfp4_expert_weight_amd import binding
    say(f"lmhead quantize V={V} H={H}")
    s = synth.lmhead_set(1, V, H, seed=V + H)
    w = s.w_bits.copy()
    w[min(3, V - 1)] = 0                                # an all-zero row
    w[0, :4] = [0x8000, 0x0001, 0x8001, 0x3F80]        # -0, the smallest subnormals, 1.0
    codes = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    scales = torch.empty(V, dtype=torch.float32, device="cuda")
    binding.moe_lmhead_fp8_quantize(_dev(torch, w.view(np.int16)), V, H, codes, scales)
    torch.cuda.synchronize()
    want_codes, want_scales = oracle.lmhead_quantize(w)
    got_codes, got_scales = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_scales.view(np.uint32), want_scales.view(np.uint32))
    bad = np.argwhere(got_codes != want_codes)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}: " \
        f"{[hex(got_codes[tuple(b)]) for b in bad[:3]]} vs {[hex(want_codes[tuple(b)]) for b in bad[:3]]}"


def test_projection_decodes_every_code_exactly():
    """Rows holding every finite E4M3 code, one-hot tokens, power-of-two scales:
    each logit is one decoded code times the scale, so it must be exact."""
    torch = need_gpu()
    say("lmhead every code")
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # 254 codes
    H, V, M = 256, 64, 8
    rng = np.random.default_rng(9)
    codes = np.zeros((V, H), dtype=np.uint8)
    for v in range(V):
        codes[v, :254] = rng.permutation(finite)
    scales = (2.0 ** rng.integers(-12, 4, V)).astype(np.float32)
    pos = [0, 1, 2, 31, 64, 127, 200, 253]
    x = np.zeros((M, H), dtype=np.uint16)
    for t, p in enumerate(pos):
        x[t, p] = 0x3F80                                 # 1.0
    got = _logits(torch, x, codes, scales)
    want = oracle.lmhead_logits(x, codes, scales)
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("M,V,H", [(1, 1000, 2560), (4, 777, 2560), (8, 513, 2560), (4, 100, 8192),
                                   (2, 33, 96), (1, 5, 32), (3, 64, 1056), (5, 70, 6528), (6, 40, 5440),
                                   (2, 17, 2560), (7, 31, 4096)])
def test_projection_within_rounding_bound(M, V, H):
    torch = need_gpu()
    say(f"lmhead logits M={M} V={V} H={H}")
    s = synth.lmhead_set(M, V, H, seed=M * 7 + V + H)
    got = _logits(torch, s.x_bits, s.codes, s.scales)
    want = oracle.lmhead_logits(s.x_bits, s.codes, s.scales)
    bound = _bound(s.x_bits, s.codes, s.scales, H) + U * np.abs(want)
    assert np.all(np.abs(got - want) <= bound), float(np.max(np.abs(got - want) / bound))


def test_projection_full_vocabulary_sampled_rows():
    """The Ling head (157,184 x 2,560), one token: the whole logit row from one
    launch, checked on 3,000 sampled vocabulary rows."""
    torch = need_gpu()
    V, H = synth.LMHEAD_VOCAB, synth.LMHEAD_HIDDEN
    say(f"lmhead full size V={V} H={H}")
    s = synth.lmhead_set(1, V, H, seed=2026)
    got = _logits(torch, s.x_bits, s.codes, s.scales)
    assert np.all(np.isfinite(got))
    rows = np.random.default_rng(1).choice(V, 3000, replace=False)
    want = oracle.lmhead_logits(s.x_bits, s.codes[rows], s.scales[rows])
    bound = _bound(s.x_bits, s.codes[rows], s.scales[rows], H) + U * np.abs(want)
    assert np.all(np.abs(got[:, rows] - want) <= bound)


def test_quantize_then_project_matches_bf16_head():
    """End to end on the Ling shape's width: quantise a bf16 head on the GPU,
    project, and compare with the oracle's quantise-then-project (the FP8
    error itself is the oracle's, so the bound is the summation's)."""
    torch = need_gpu()
    from mxfp4_expert_weight_amd import binding
    V, H, M = 2048, 2560, 4
    say("lmhead quantise + project")
    s = synth.lmhead_set(M, V, H, seed=77)
    codes = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    scales = torch.empty(V, dtype=torch.float32, device="cuda")
    binding.moe_lmhead_fp8_quantize(_dev(torch, s.w_bits.view(np.int16)), V, H, codes, scales)
    out = torch.empty((M, V), dtype=torch.float32, device="cuda")
    binding.moe_lmhead_fp8_logits(_dev(torch, s.x_bits.view(np.int16)), codes, scales, M, V, H, out)
    torch.cuda.synchronize()
    c, sc = oracle.lmhead_quantize(s.w_bits)
    want = oracle.lmhead_logits(s.x_bits, c, sc)
    bound = _bound(s.x_bits, c, sc, H) + U * np.abs(want)
    assert np.all(np.abs(out.cpu().numpy() - want) <= bound)
