"""The allocation-free layer entry point (lorabwd_layer_backward_noalloc)
against the workspace entry point (lorabwd_layer_backward), through the C
ABI: two calls in a row on the library's static scratch, the second on a
smaller layer, each compared with the workspace entry point on the same
inputs (per-tensor max-norm relative error within the float32 bound; the
kernels are the same and deterministic, so the results are expected to be
bitwise equal as well)."""
import pytest

import synth
from tests import harness as Hn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(cfg, noalloc):
    import layer_backward_pass_amd as lbp
    dl = Hn.DeviceLayer(cfg, 0, DEV)
    d = torch.empty_like(dl.d_out)
    dq = torch.empty(cfg.seq, cfg.q_dim, device=DEV)
    dv = torch.empty(cfg.kv_len, cfg.kv_dim, device=DEV)
    g = torch.zeros(1, device=DEV)
    fn = lbp.lorabwd_layer_backward_noalloc if noalloc else lbp.lorabwd_layer_backward
    fn(dl.desc(), dl.w, dl.saved, d, q_state=dl.lora["q"] if dl.lora else None,
       v_state=dl.lora["v"] if dl.lora else None, adamw=dl.adamw() if dl.lora else None,
       dq_pre_out=dq, dv_out=dv, gnorm_sq=g, d_out=dl.d_out)
    torch.cuda.synchronize()
    out = {"d_hidden": d, "dq_pre": dq, "dv": dv, "gnorm_sq": g}
    if dl.lora:
        for t in ("q", "v"):
            for k in ("A", "B", "m_a", "v_a", "m_b", "v_b"):
                out["%s_%s" % (k, t)] = dl.lora[t][k]
    return {k: Hn.host(v) for k, v in out.items()}


def test_noalloc_matches_workspace_entry_point_twice():
    import layer_backward_pass_amd as lbp
    # one token against a 512-slot cache at hidden 2560 / ffn 6912 (the
    # single-token workload, 3.6 MiB of scratch), then a smaller layer with
    # adapters (16 tokens, hidden 64): the scratch keeps the first call's
    # contents, which the second must not depend on
    cases = [synth.get_config("decode"), synth.get_config("tiny")]
    for cfg in cases:
        need = lbp.lorabwd_layer_workspace_size(Hn.desc_of(cfg))
        assert 0 < need <= lbp.NOALLOC_SCRATCH_BYTES, need
        print("noalloc case", cfg.name, "scratch", need, flush=True)
        ref = _run(cfg, noalloc=False)
        got = _run(cfg, noalloc=True)
        errs = {k: Hn.rel_err(got[k], ref[k]) for k in ref}
        same = all((got[k] == ref[k]).all() for k in ref)
        print("  errors", {k: float("%.3g" % v) for k, v in errs.items()}, "bitwise equal", same,
              flush=True)
        bad = {k: v for k, v in errs.items() if not v <= Hn.TOL[cfg.dtype]}
        assert not bad, bad


def test_noalloc_refuses_a_layer_beyond_the_scratch():
    import layer_backward_pass_amd as lbp
    cfg = synth.get_config("seq512").with_(seq=128, kv_len=128)
    assert lbp.lorabwd_layer_workspace_size(Hn.desc_of(cfg)) > lbp.NOALLOC_SCRATCH_BYTES
    dl = Hn.DeviceLayer(cfg, 0, DEV)
    d = torch.empty_like(dl.d_out)
    with pytest.raises(lbp.LorabwdError) as e:
        lbp.lorabwd_layer_backward_noalloc(dl.desc(), dl.w, dl.saved, d, d_out=dl.d_out)
    assert e.value.status == -5  # LORABWD_ERR_WORKSPACE
