"""spec_verify_noalloc (include/tsr.h: for callers that cannot allocate) against
spec_verify, through the C ABI: the same kernels on the same inputs, one with
the handle's workspace and one with the library's static device array, must
give identical outputs; two calls in a row, the second smaller, so the second
runs on the array the first left behind."""
import ctypes

import numpy as np
import pytest

from tests.gpu_common import device, gpu_available, to_dev, torch

import token_sampling_row_amd as tsr
from token_sampling_row_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SEED = 0x5EED0004


def case(rng, B, K, V, dtype):
    tgt = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    dft = (tgt[:, :K] + rng.normal(0, 0.8, (B, K, V))).astype(np.float32)
    if dtype == "bf16":
        tgt, dft = wl.f32_to_bf16_bits(tgt), wl.f32_to_bf16_bits(dft)
    xs = rng.integers(0, V, (B, K)).astype(np.int32)
    xs[: B // 2] = np.argmax(tgt[: B // 2, :K].astype(np.float64) if dtype == "f32"
                             else wl.bf16_bits_to_f32(tgt[: B // 2, :K]), axis=-1)
    t = to_dev(tgt.reshape(B * (K + 1), V), dtype).view(B, K + 1, V)
    d = to_dev(dft.reshape(B * K, V), dtype).view(B, K, V)
    return t, d, torch.from_numpy(xs).to(device())


def both(s, t, d, x, prm, step):
    B, K1, _ = t.shape
    ref_t, ref_a = s.spec_verify(t, d, x, prm, step)
    ref_s = torch.full((B,), -7, dtype=torch.int32, device=device())
    s.spec_verify(t, d, x, prm, step, out_status=ref_s)
    got_t = torch.full((B, K1), -9, dtype=torch.int32, device=device())
    got_a = torch.full((B,), -9, dtype=torch.int32, device=device())
    got_s = torch.full((B,), -9, dtype=torch.int32, device=device())
    tsr.spec_verify_noalloc(0, SEED, t, d, x, prm, step, got_t, got_a, got_s)
    torch.cuda.synchronize()
    return (ref_t.cpu().numpy(), ref_a.cpu().numpy(), ref_s.cpu().numpy(),
            got_t.cpu().numpy(), got_a.cpu().numpy(), got_s.cpu().numpy())


def test_noalloc_verify_matches_spec_verify_twice():
    rng = np.random.default_rng(11)
    with tsr.Sampler(0, max_rows=4096, max_vocab=1 << 18, max_k=8, seed=SEED) as s:
        # first call: 64 sequences, K 4, 32000 fp32; second: 16 sequences, K 2, 5000 bf16
        for (B, K, V, dtype) in ((64, 4, 32000, "f32"), (16, 2, 5000, "bf16")):
            t, d, x = case(rng, B, K, V, dtype)
            for step, prm in enumerate([{"temperature": 1.0},
                                        {"temperature": 0.8, "top_k": 40, "top_p": 0.9},
                                        {"temperature": 0.0}]):
                print(f"[case] noalloc B={B} K={K} V={V} {dtype} {prm}", flush=True)
                rt, ra, rs, gt, ga, gs = both(s, t, d, x, prm, step)
                assert np.array_equal(rt, gt) and np.array_equal(ra, ga) and np.array_equal(rs, gs)
                assert (ga >= 0).all() and (ga <= K).all()


def test_noalloc_verify_at_its_vocab_limit():
    """The widest rows the static array serves (65,536 bf16 and 32,768 fp32
    logits: the two-rows-per-workgroup kernel), against spec_verify."""
    rng = np.random.default_rng(12)
    with tsr.Sampler(0, max_rows=64, max_vocab=1 << 17, max_k=4, seed=SEED) as s:
        for (B, K, V, dtype) in ((4, 2, 65536, "bf16"), (4, 3, 32768, "f32")):
            t, d, x = case(rng, B, K, V, dtype)
            for step, prm in enumerate([{"temperature": 1.0}, {"temperature": 0.0}]):
                print(f"[case] noalloc limit B={B} K={K} V={V} {dtype} {prm}", flush=True)
                rt, ra, rs, gt, ga, gs = both(s, t, d, x, prm, step)
                assert np.array_equal(rt, gt) and np.array_equal(ra, ga) and np.array_equal(rs, gs)


def test_noalloc_verify_rejects_sizes_beyond_its_array():
    lib = tsr.load_library()
    p = tsr._Params(1.0, 0, 1.0, 0.0, 0)
    buf = torch.zeros(1 << 16, dtype=torch.int32, device=device())
    ptr = ctypes.c_void_p(buf.data_ptr())
    # 16385 sequences, and 13108 x (4 + 1) = 65540 slots: beyond the static array
    for rows, K in ((16385, 1), (13108, 4)):
        assert lib.spec_verify_noalloc(0, 1, ptr, ptr, 0, ptr, rows, K, 8, ctypes.byref(p), 0, ptr,
                                       ptr, None, None) == 1
    assert lib.spec_verify_noalloc(0, 1, ptr, ptr, 0, ptr, 4, 33, 8, ctypes.byref(p), 0, ptr, ptr,
                                   None, None) == 1                              # K > 32
    assert lib.spec_verify_noalloc(99, 1, ptr, ptr, 0, ptr, 4, 2, 8, ctypes.byref(p), 0, ptr, ptr,
                                   None, None) == 1                              # no such device
    # rows wider than the register-pair path (65,536 bf16 / 32,768 fp32 logits)
    for dtype, vocab in ((1, 65537), (0, 32769)):
        assert lib.spec_verify_noalloc(0, 1, ptr, ptr, dtype, ptr, 4, 2, vocab, ctypes.byref(p), 0,
                                       ptr, ptr, None, None) == 4
    torch.cuda.synchronize()
    assert int(buf.abs().sum()) == 0
