"""Argument errors through the C ABI with a live handle (include/tsr.h, "Argument
errors are returned synchronously and nothing is enqueued"): every entry point
is called with each class of invalid argument; the call must return TSR_EINVAL
(or TSR_EUNSUPPORTED for a size no kernel covers), and outputs prefilled with a
sentinel must be untouched once the stream has drained."""
import ctypes

import numpy as np
import pytest

from tests.gpu_common import device, gpu_available, torch

import token_sampling_row_amd as tsr

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

EINVAL, EUNSUPPORTED = 1, 4
SENTINEL = -7
ROWS, V, K, MAX_ROWS, MAX_K = 4, 1000, 3, 8, 4
BIG_VOCAB = (1 << 23) + 1          # wider than any kernel: TSR_EUNSUPPORTED


def P(temperature=1.0, top_k=0, top_p=1.0, min_p=0.0, mode=0):
    return tsr._Params(temperature, top_k, top_p, min_p, mode)


BAD_PARAMS = [P(temperature=-1.0), P(temperature=float("nan")), P(temperature=float("inf")),
              P(temperature=1e-31), P(top_p=-0.1), P(top_p=float("nan")),
              P(min_p=float("inf")), P(mode=7)]


@pytest.fixture(scope="module")
def env():
    lib = tsr.load_library()
    s = tsr.Sampler(0, max_rows=MAX_ROWS, max_vocab=BIG_VOCAB, max_k=MAX_K, seed=1)
    rng = np.random.default_rng(0)
    e = dict(lib=lib, s=s, h=s._h, dev=device())
    e["x"] = torch.from_numpy(rng.normal(0, 1, (ROWS, V)).astype(np.float32)).to(device())
    e["xb"] = e["x"].to(torch.bfloat16)
    e["tgt"] = torch.from_numpy(rng.normal(0, 1, (ROWS, K + 1, V)).astype(np.float32)).to(device())
    e["dft"] = torch.from_numpy(rng.normal(0, 1, (ROWS, K, V)).astype(np.float32)).to(device())
    e["xs"] = torch.zeros(ROWS, K, dtype=torch.int32, device=device())
    e["mask"] = torch.full((ROWS, (V + 31) // 32), -1, dtype=torch.int32, device=device())
    e["hist"] = torch.zeros(ROWS, 8, dtype=torch.int32, device=device())
    e["big"] = torch.zeros(1 << 20, dtype=torch.uint8, device=device())   # a raw byte buffer
    yield e
    s.close()


def outs(n=ROWS * (K + 1)):
    return torch.full((n,), SENTINEL, dtype=torch.int32, device=device())


def untouched(*ts):
    torch.cuda.synchronize()
    return all(bool((t == SENTINEL).all()) for t in ts)


def vp(t, offset=0):
    return ctypes.c_void_p(t.data_ptr() + offset)


def sample(e, out, x=None, dtype=0, rows=ROWS, vocab=V, stride=V, params=None, off=0):
    x = e["x"] if x is None else x
    p = P() if params is None else params
    return e["lib"].sample_rows(e["h"], vp(x, off), dtype, rows, vocab, stride,
                                ctypes.byref(p), 0, vp(out), None, None)


def test_sample_rows_rejects_each_invalid_argument(env):
    e = env
    out = outs()
    for p in BAD_PARAMS:
        assert sample(e, out, params=p) == EINVAL, (p.temperature, p.top_p, p.min_p)
    assert e["lib"].sample_rows(e["h"], vp(e["x"]), 0, ROWS, V, V, None, 0, vp(out), None,
                                None) == EINVAL                             # no params
    assert e["lib"].sample_rows(e["h"], None, 0, ROWS, V, V, ctypes.byref(P()), 0, vp(out),
                                None, None) == EINVAL                       # no logits
    assert e["lib"].sample_rows(e["h"], vp(e["x"]), 0, ROWS, V, V, ctypes.byref(P()), 0, None,
                                None, None) == EINVAL                       # no output
    assert sample(e, out, dtype=2) == EINVAL                               # unknown dtype
    assert sample(e, out, rows=-1) == EINVAL
    assert sample(e, out, rows=MAX_ROWS + 1) == EINVAL                     # > max_rows
    assert sample(e, out, vocab=0) == EINVAL
    assert sample(e, out, stride=V - 1) == EINVAL                          # stride < vocab
    assert sample(e, out, off=2) == EINVAL                                 # fp32 not 4-aligned
    assert sample(e, out, x=e["xb"], dtype=1, off=1) == EINVAL             # bf16 not 2-aligned
    assert sample(e, out, x=e["big"], dtype=1, rows=0, vocab=BIG_VOCAB,
                  stride=BIG_VOCAB) == EUNSUPPORTED                         # wider than any kernel
    assert untouched(out)


def test_greedy_argmax_rejects_each_invalid_argument(env):
    e = env
    out, st = outs(), outs()
    g = e["lib"].greedy_argmax
    x = vp(e["x"])
    assert g(e["h"], x, 2, ROWS, V, V, vp(out), vp(st), None) == EINVAL
    assert g(e["h"], x, 0, MAX_ROWS + 1, V, V, vp(out), vp(st), None) == EINVAL
    assert g(e["h"], x, 0, ROWS, 0, V, vp(out), vp(st), None) == EINVAL
    assert g(e["h"], x, 0, ROWS, V, V - 1, vp(out), vp(st), None) == EINVAL
    assert g(e["h"], vp(e["x"], 2), 0, ROWS, V, V, vp(out), vp(st), None) == EINVAL
    assert g(e["h"], x, 0, ROWS, V, V, None, vp(st), None) == EINVAL
    assert g(e["h"], vp(e["big"]), 1, 0, BIG_VOCAB, BIG_VOCAB, vp(out), vp(st), None) == \
        EUNSUPPORTED
    assert untouched(out, st)


def test_sample_rows_ex_rejects_each_invalid_constraint(env):
    e = env
    out = outs()
    lp = torch.full((ROWS,), 5.0, dtype=torch.float32, device=device())
    words = (V + 31) // 32

    def call(**kw):
        cs = tsr._Constraints(None, 0, None, 0, 0, 1.0, None)
        for k, v in kw.items():
            setattr(cs, k, v)
        return e["lib"].sample_rows_ex(e["h"], vp(e["x"]), 0, ROWS, V, V, ctypes.byref(cs),
                                       ctypes.byref(P()), 0, vp(out), vp(lp), None, None)

    m, h = e["mask"], e["hist"]
    assert call(allowed=m.data_ptr(), allowed_stride=words - 1) == EINVAL   # stride too short
    assert call(allowed=m.data_ptr() + 2, allowed_stride=words) == EINVAL   # not 4-aligned
    assert call(history=h.data_ptr(), history_len=65, history_stride=65,
                repetition_penalty=1.1) == EINVAL                           # window > 64
    assert call(history=h.data_ptr(), history_len=8, history_stride=7,
                repetition_penalty=1.1) == EINVAL                           # stride < length
    assert call(history=h.data_ptr(), history_len=8, history_stride=8,
                repetition_penalty=0.9) == EINVAL                           # r < 1
    assert call(history=h.data_ptr(), history_len=8, history_stride=8,
                repetition_penalty=float("nan")) == EINVAL
    assert call(history=h.data_ptr() + 2, history_len=8, history_stride=8,
                repetition_penalty=1.1) == EINVAL                           # not 4-aligned
    assert call(history=None, history_len=8, history_stride=8,
                repetition_penalty=1.1) == EINVAL                           # length without ids
    assert call(history_len=-1) == EINVAL
    assert call(row_params=e["big"].data_ptr() + 4) == EINVAL              # misaligned params
    for p in BAD_PARAMS[:3]:
        assert e["lib"].sample_rows_masked(e["h"], vp(e["x"]), 0, ROWS, V, V, vp(m), words,
                                           ctypes.byref(p), 0, vp(out), vp(lp), None,
                                           None) == EINVAL
    assert untouched(out)
    torch.cuda.synchronize()
    assert bool((lp == 5.0).all())


def test_spec_verify_rejects_each_invalid_argument(env):
    e = env
    toks, acc, st = outs(), outs(ROWS), outs(ROWS)
    sv = e["lib"].spec_verify

    def call(tgt=None, dft=None, xs=None, dtype=0, rows=ROWS, k=K, vocab=V, params=None,
             tgt_off=0):
        p = P() if params is None else params
        t = vp(e["tgt"], tgt_off) if tgt is None else tgt
        d = vp(e["dft"]) if dft is None else dft
        x = vp(e["xs"]) if xs is None else xs
        return sv(e["h"], t, d, dtype, x, rows, k, vocab, ctypes.byref(p), 0, vp(toks),
                  vp(acc), vp(st), None)

    for p in BAD_PARAMS:
        assert call(params=p) == EINVAL
    assert call(k=0) == EINVAL                                             # K < 1
    assert call(k=MAX_K + 1) == EINVAL                                     # K > max_k
    assert call(rows=MAX_ROWS + 1) == EINVAL
    assert call(vocab=0) == EINVAL
    assert call(dtype=2) == EINVAL
    assert call(dft=ctypes.c_void_p(0)) == EINVAL                          # T > 0 needs q
    assert call(tgt_off=2) == EINVAL                                       # misaligned
    assert call(xs=ctypes.c_void_p(0)) == EINVAL
    assert call(tgt=vp(e["big"]), dft=vp(e["big"]), rows=0, dtype=1,
                vocab=BIG_VOCAB) == EUNSUPPORTED
    # one past the widest verify rows: 155,648 bf16 and 77,824 fp32 logits
    assert call(tgt=vp(e["big"]), dft=vp(e["big"]), rows=0, dtype=1, vocab=155649) == EUNSUPPORTED
    assert call(tgt=vp(e["big"]), dft=vp(e["big"]), rows=0, dtype=0, vocab=77825) == EUNSUPPORTED
    assert call(tgt=vp(e["big"]), dft=vp(e["big"]), rows=0, dtype=1, vocab=155648) == 0
    assert untouched(toks, acc, st)


def test_tree_verify_rejects_each_invalid_argument(env):
    e = env
    ot, op, acc, st = outs(), outs(), outs(ROWS), outs(ROWS)
    parent = torch.zeros(ROWS, K + 1, dtype=torch.int32, device=device())
    tv = e["lib"].tree_verify

    def call(nodes=K + 1, params=None, dft=None, rows=ROWS, vocab=V, dtype=0):
        p = P() if params is None else params
        d = vp(e["dft"]) if dft is None else dft
        return tv(e["h"], vp(e["tgt"]), d, dtype, vp(parent), vp(e["xs"]), rows, nodes, vocab,
                  ctypes.byref(p), 0, vp(ot), vp(op), vp(acc), vp(st), None)

    assert call(nodes=0) == EINVAL
    assert call(nodes=33) == EINVAL                                        # > 32 nodes
    assert call(nodes=MAX_K + 2) == EINVAL                                 # > max_k + 1
    assert call(params=P(temperature=-2.0)) == EINVAL
    assert call(dft=ctypes.c_void_p(0)) == EINVAL
    assert call(rows=MAX_ROWS + 1) == EINVAL
    assert call(dtype=5) == EINVAL
    assert untouched(ot, op, acc, st)


def test_beam_step_and_philox_reject_invalid_arguments(env):
    e = env
    par, tok, st = outs(), outs(), outs()
    score = torch.full((16,), 3.0, dtype=torch.float64, device=device())
    scores = torch.zeros(MAX_ROWS, dtype=torch.float64, device=device())
    bs = e["lib"].beam_step

    def call(groups=1, beam=4, vocab=V, stride=V, sc=None, dtype=0):
        s_ = vp(scores) if sc is None else sc
        return bs(e["h"], vp(e["x"]), dtype, groups, beam, vocab, stride, s_, vp(par), vp(tok),
                  vp(score), vp(st), None)

    assert call(beam=0) == EINVAL
    assert call(beam=17) == EINVAL                                         # > 16 beams
    assert call(groups=3, beam=4) == EINVAL                                # 12 rows > max_rows
    assert call(groups=-1) == EINVAL
    assert call(stride=V - 1) == EINVAL
    assert call(sc=vp(scores, 4)) == EINVAL                                # scores not 8-aligned
    assert call(sc=ctypes.c_void_p(0)) == EINVAL
    assert call(dtype=3) == EINVAL
    assert e["lib"].sampler_philox(e["h"], vp(e["xs"]), -1, vp(par), None) == EINVAL
    assert untouched(par, tok, st)
    torch.cuda.synchronize()
    assert bool((score == 3.0).all())
