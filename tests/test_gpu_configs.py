"""GPU parity at the full workload shapes, through the same entry point and
launch configuration the benchmark times (lorabwd_layer_backward), against
the float64 oracle on exactly the values the GPU holds.

Bounds (per-tensor max-norm relative error): 1e-4 for float32 inputs, 2e-2
for bf16 inputs; AdamW-updated tensors use the sign-flip allowance described
in tests/harness.py.
"""
import time

import pytest

import synth
from tests import harness as Hn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", ["tiny", "decode", "seq512", "seq2048bf16", "seq512qk", "seq512ig",
                                  "seq2048bf16ig"])
def test_full_size_layer(name):
    cfg = synth.get_config(name)
    t0 = time.time()
    _log("full-size layer %s" % name)
    errs = Hn.layer_parity(cfg, "cuda:0")
    _log("  %s: %.1f s, errors %s" % (name, time.time() - t0,
                                      {k: float("%.3g" % v) for k, v in errs.items()}))
    bad = {k: v for k, v in errs.items() if not v <= Hn.TOL[cfg.dtype]}
    assert not bad, bad


def test_full_size_decode_packed():
    """The decode workload (hidden 2560, ffn 6912, 512-slot cache) on packed
    ternary weights, against the oracle on the dense values."""
    cfg = synth.get_config("decode_packed")
    t0 = time.time()
    errs = Hn.packed_layer_parity(cfg, "cuda:0", check_bytes=False)
    _log("  decode_packed: %.1f s, errors %s" % (time.time() - t0,
                                               {k: float("%.3g" % v) for k, v in errs.items()}))
    bad = {k: v for k, v in errs.items() if not v <= Hn.TOL[cfg.dtype]}
    assert not bad, bad


@pytest.mark.timeout(1500)
def test_stack36_full():
    cfg = synth.get_config("stack36")
    t0 = time.time()
    errs = Hn.stack_parity(cfg, "cuda:0", log=_log)
    _log("  stack36: %.1f s, errors %s" % (time.time() - t0,
                                         {k: float("%.3g" % v) for k, v in errs.items()}))
    bad = {k: v for k, v in errs.items() if not v <= Hn.TOL[cfg.dtype]}
    assert not bad, bad


def test_full_size_lmhead():
    """The lm_head workload (1024 rows, hidden 2560, vocabulary 151936): the
    loss, grad_hidden at sampled rows, and dW's AdamW step at sampled
    vocabulary rows, against the oracle's block-wise form."""
    cfg = synth.get_config("lmhead")
    t0 = time.time()
    errs = Hn.lm_head_parity(cfg, "cuda:0", full=True, log=_log)
    _log("  lmhead: %.1f s, errors %s" % (time.time() - t0,
                                        {k: float("%.3g" % v) for k, v in errs.items()}))
    bad = {k: v for k, v in errs.items() if not v <= Hn.TOL["f32"]}
    assert not bad, bad
