"""GPU parity of the further forms against the fp64 oracle, through the C ABI:
the decay given as d (w = exp(-exp(d))), the Finch-C2 time mixer, and both
together.  Same tolerances as the base form (2e-3 bf16, 1e-5 fp32, normwise
per block)."""
from dataclasses import replace

import numpy as np
import pytest

from synth import make_workload, get_config, f32_to_bf16_bits
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors, gpu_block_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FORMS = [("log", "finch"), ("w", "c2"), ("log", "c2")]
IDS = ["logdecay", "c2", "c2_logdecay"]


def _check(wl, heads=None, g=None, **kw):
    tol = wl.config.tolerance
    log("case %s decay=%s variant=%s B=%d H=%d tokens=%d heads=%s" % (
        wl.config.name, wl.decay, wl.variant, wl.n_seq, wl.u.shape[0], wl.tokens, heads))
    o, s = run_gpu(wl, g, **kw)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(wl, heads)
    err = errors(wl, o, s, o_ref, s_ref, heads)
    eo, es = err
    log("  err o=%.3e state=%.3e (tol %.0e)" % (eo, es, tol))
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= tol and es <= tol, (eo, es)
    # per-row errors (floored denominators) within the same bound: an error
    # confined to a few rows of a long block cannot hide behind its maximum
    assert err.row_o <= tol and err.row_s <= tol, (err.row_o, err.row_s)
    return o, s


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
@pytest.mark.parametrize("T", [1, 63, 65, 1000])
def test_short_sequences(decay, variant, T):
    _check(make_workload(1, T=T, H=4, decay=decay, variant=variant))


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_f32_serial_path(decay, variant):
    wl = make_workload(0, T=300, H=2, B=2, decay=decay, variant=variant)
    wl.state0 = np.random.default_rng(5).normal(0, 0.1, size=(2, 2, 64, 64)).astype(np.float32)
    _check(wl)


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_layer_shape_full_size(decay, variant):
    """T=4096, H=32: every slice against the oracle."""
    _check(make_workload(1, decay=decay, variant=variant))


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_ragged_with_states(decay, variant):
    wl = make_workload(4, lengths=[1024, 3, 0, 2500, 64, 4097], H=4, decay=decay, variant=variant)
    _check(wl)


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_long_sequence_segments_and_chain(decay, variant):
    """20000 tokens, 8 heads, random S_0 (the long-context recipe): split into
    segments; the same sequence as 5 carried-state calls must agree with the
    single call and with the oracle."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(3, T=20000, H=8, decay=decay, variant=variant)
    g = to_gpu(wl)
    o_full, s_full = _check(wl, g=g)
    T = 20000
    cuts = [0, 1, 4000, 4097, 12000, T]
    state = g["state0"].clone()
    o_chain = torch.empty_like(o_full)
    u = None if variant == "c2" else g["u"]
    for a, z in zip(cuts[:-1], cuts[1:]):
        sv = None if g["u2"] is None else g["u2"][:, a:z]
        fw.prefill(g["r"][:, a:z], g["k"][:, a:z], g["v"][:, a:z], g["w"][:, a:z], u, state,
                   o=o_chain[:, a:z], state_out=state, decay=decay, variant=variant,
                   second_value=sv)
    torch.cuda.synchronize()
    e_o = gpu_block_error(o_chain, o_full, (1, 3))
    e_s = gpu_block_error(state, s_full, (2, 3))
    log("  chain vs single call: o=%.3e state=%.3e" % (e_o, e_s))
    assert e_o <= 2e-3 and e_s <= 2e-3
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o_chain, state, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3


def _stiff(T, H, decay, variant):
    """Decays spanning many orders of magnitude inside one chunk (exact
    token-serial path), one head without any decay."""
    wl = make_workload(replace(get_config(1), state_sigma=0.1), T=T, H=H, decay=decay,
                       variant=variant)
    bits = lambda x: f32_to_bf16_bits(np.float32(x)).item()
    w = wl.w
    if decay == "log":
        w[:, 100 % T:180 % T + 1, 1 % H, 5] = bits(4.0)        # w = exp(-e^4) ~ 2e-24
        w[:, (T // 3):(T // 3) + 60, 2 % H, 63] = bits(2.5)     # ~ 5e-6 per token
        w[:, T - 20:T - 10, H - 1, 0] = 0x7F80                  # d = +inf: w = 0
        w[:, :, 0, 17:30] = 0xFF80                              # d = -inf: w = 1
    else:
        w[:, 100 % T:180 % T + 1, 1 % H, 5] = bits(1e-3)
        w[:, (T // 3):(T // 3) + 60, 2 % H, 63] = bits(1e-30)
        w[:, T - 20:T - 10, H - 1, 0] = 0x0001
        w[:, :, 0, 17:30] = bits(1.0)
    return wl


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
@pytest.mark.parametrize("T,H", [(300, 1), (2000, 4)])
def test_stiff_decays(decay, variant, T, H):
    _check(_stiff(T, H, decay, variant))


def test_c2_without_second_value():
    """Finch-C2 with no u' (the pages' ablation without the second value)."""
    wl = make_workload(1, T=700, H=4, variant="c2")
    wl.u2 = None
    g = to_gpu(wl)
    _check(wl, g=g, second_value=None)


def test_c2_second_value_is_additive_on_gpu():
    """o(u') - o(no u') equals u' (fp32 add of the bf16 values), state equal."""
    wl = make_workload(1, T=500, H=4, variant="c2", decay="log")
    g = to_gpu(wl)
    o1, s1 = run_gpu(wl, g)
    o0, s0 = run_gpu(wl, g, second_value=None)
    torch.cuda.synchronize()
    diff = (o1 - o0 - g["u2"].float()).abs().max().item()
    log("  max |o(u') - o(0) - u'| = %.3e" % diff)
    assert diff <= 1e-6 * max(o1.abs().max().item(), 1.0)
    assert torch.equal(s1, s0)
