"""GPU parity of the FP8 variant: fa_quantize_e4m3 and fa_fwd_fp8 against the oracle.

The quantiser must reproduce the oracle's E4M3 codes bit for bit (every
binary16 pattern, a spread of bfloat16 patterns, ragged lengths).  The forward
is compared with the fp64 attention on the quantised Q and K, to the same
tolerances as the 16-bit forward: the scores of E4M3 operands are exact
products summed in fp32, so the result differs from the definition on the
quantised inputs only by the rounding of the accumulations, of P and of O.
"""
import zlib

import numpy as np
import pytest
import torch

import exact_io_aware_65_amd as fa
import fa_inputs as fi
import oracle
from gpu_util import check, device, rand_bits, say, to_np, upload

pytestmark = pytest.mark.gpu


def _quantize_gpu(bits, dtype):
    y = fa.quantize_e4m3(upload(bits, dtype))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_quantize_every_f16_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    say("fa_quantize_e4m3 all binary16 patterns")
    got = _quantize_gpu(bits, "f16")
    x = bits.view(np.float16)
    nan = np.isnan(x)
    ref = oracle.quantize_e4m3(bits[~nan], "f16")
    assert np.array_equal(got[~nan], ref), int(np.sum(got[~nan] != ref))
    assert ((got[nan] & 0x7F) == 0x7F).all()


def test_quantize_bf16_and_ragged_lengths():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 65536, 200003).astype(np.uint16)
    x = oracle.widen(bits, "bf16")
    bits = bits[~np.isnan(x)]
    say("fa_quantize_e4m3 bfloat16")
    assert np.array_equal(_quantize_gpu(bits, "bf16"), oracle.quantize_e4m3(bits, "bf16"))
    for n in (1, 7, 8, 9, 15, 17, 4099):
        b = rand_bits(rng, (n,), "f16", sigma=100.0)
        assert np.array_equal(_quantize_gpu(b, "f16"), oracle.quantize_e4m3(b, "f16")), n


CASES = [
    # B, H, Nq, Nkv, d, causal, dtype
    (1, 2, 64, 64, 128, False, "f16"),
    (1, 2, 130, 130, 128, True, "f16"),
    (2, 1, 100, 257, 64, True, "bf16"),
    (1, 1, 1, 1, 128, False, "f16"),
    (1, 3, 77, 200, 64, False, "f16"),
    (2, 2, 300, 300, 128, True, "bf16"),
    (1, 1, 513, 600, 64, True, "f16"),
    (3, 4, 256, 1024, 128, False, "f16"),
    # enough 256-row tiles for the eight-wave 16x16x128 E4M3 kernel at d = 128
    # (B H ceil(Nq / 256) >= 256): ragged, causal with Nq < Nkv, and no mask
    (2, 128, 300, 330, 128, True, "f16"),
    (4, 64, 128, 700, 128, True, "f16"),
    (1, 256, 257, 200, 128, False, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}q{}k{}d{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6]))
def test_fwd_fp8_small(case):
    B, H, Nq, Nkv, d, causal, dtype = case
    rng = np.random.default_rng(zlib.crc32(("fp8" + repr(case)).encode()))
    q = rand_bits(rng, (B, H, Nq, d), dtype, sigma=1.5)
    k = rand_bits(rng, (B, H, Nkv, d), dtype, sigma=1.5)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    o_ref, lse_ref = oracle.attention_fp8qk(q, k, v, causal=causal, scale=scale, dtype=dtype)
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    say(f"fa_fwd_fp8 {case}")
    o, lse = fa.fwd_fp8(tq, tk, tv, causal=causal, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"fp8 {case}")
    # K given already in E4M3 is the same call
    k8 = fa.quantize_e4m3(tk)
    o2, lse2 = fa.fwd_fp8(tq, k8, tv, causal=causal, scale=scale, out_dtype=torch.float32)
    o16, _ = fa.fwd_fp8(tq, k8, tv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(o16.float(), o.to(o16.dtype).float())


@pytest.mark.parametrize("scale", [0.0, -0.15])
def test_fwd_fp8_scale_values(scale):
    rng = np.random.default_rng(61)
    B, H, Nq, Nkv, d, dtype = 1, 2, 96, 160, 128, "f16"
    q = rand_bits(rng, (B, H, Nq, d), dtype, sigma=1.5)
    k = rand_bits(rng, (B, H, Nkv, d), dtype, sigma=1.5)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    o_ref, lse_ref = oracle.attention_fp8qk(q, k, v, causal=True, scale=scale, dtype=dtype)
    say(f"fa_fwd_fp8 scale={scale}")
    o, lse = fa.fwd_fp8(upload(q, dtype), upload(k, dtype), upload(v, dtype), causal=True, scale=scale,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"fp8 scale={scale}")


def test_fwd_fp8_saturation():
    # values far beyond 448 in Q and K: the kernel's in-register rounding of Q and
    # the quantiser's rounding of K both saturate like the oracle
    rng = np.random.default_rng(67)
    B, H, Nq, Nkv, d, dtype = 1, 1, 64, 96, 64, "bf16"
    q = rand_bits(rng, (B, H, Nq, d), dtype, sigma=1.0)
    k = rand_bits(rng, (B, H, Nkv, d), dtype, sigma=1.0)
    qf = oracle.widen(q, dtype)
    qf[0, 0, :, 0] = 5000.0
    qf[0, 0, :, 1] = -1e30
    kf = oracle.widen(k, dtype)
    kf[0, 0, ::7, 2] = 9000.0
    q = fi.f32_to_bits(qf.astype(np.float32), dtype)
    k = fi.f32_to_bits(kf.astype(np.float32), dtype)
    v = rand_bits(rng, (B, H, Nkv, d), dtype)
    o_ref, lse_ref = oracle.attention_fp8qk(q, k, v, causal=False, scale=1e-4, dtype=dtype)
    say("fa_fwd_fp8 saturation")
    o, lse = fa.fwd_fp8(upload(q, dtype), upload(k, dtype), upload(v, dtype), causal=False, scale=1e-4,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, "fp8 saturation")


def _rows(rng, n, extra):
    return np.unique(np.concatenate([[0, 1, 63, 64, n // 2, n - 2, n - 1], rng.integers(0, n, extra)])).astype(np.int64)


@pytest.mark.parametrize("name,heads", [("prefill_8k_d128", [(0, 3), (0, 31)]),
                                        ("prefill_2k_d64", [(0, 0), (1, 5)]),
                                        ("prefill_16k_d128_bf16", [(0, 9)])])
def test_fwd_fp8_full_size_sampled(name, heads):
    w = fi.WORKLOADS[name]
    say(f"fa_fwd_fp8 {name} full size")
    x = fi.make_inputs(w)
    tq, tk, tv = (upload(x[t], w.dtype) for t in "qkv")
    k8 = fa.quantize_e4m3(tk)
    o, lse = fa.fwd_fp8(tq, k8, tv, causal=w.causal, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any()
    k8n = k8.cpu().numpy()
    rng = np.random.default_rng(3)
    for b, h in heads:
        # the oracle rounds K itself; the GPU quantiser must agree on the whole head
        codes = oracle.quantize_e4m3(x["k"][b, h], w.dtype)
        assert np.array_equal(k8n[b, h], codes), f"quantiser differs from the oracle on head ({b},{h})"
        rows = _rows(rng, w.Nq, 8)
        o_ref, lse_ref = oracle.attention_fp8qk_rows(x["q"][b, h], codes, x["v"][b, h], rows, causal=w.causal,
                                                     scale=w.scale, dtype=w.dtype, k_codes=True)
        check(to_np(o[b, h])[rows], to_np(lse[b, h])[rows], o_ref, lse_ref, w.dtype, f"fp8 {name} head ({b},{h})")
