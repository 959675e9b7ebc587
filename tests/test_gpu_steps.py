"""GPU parity of recurrent generation steps (calls whose sequences have at most
16 tokens, which run the state-streaming step kernel) against the fp64 oracle,
through the C ABI, in every form; and continuity between a pre-fill and the
steps that continue it."""
import numpy as np
import pytest

from synth import make_workload, f32_to_bf16_bits
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors, gpu_block_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FORMS = [("w", "finch"), ("log", "finch"), ("w", "c2"), ("log", "c2")]
IDS = ["finch", "logdecay", "c2", "c2_logdecay"]


def _check(wl, heads=None, g=None, **kw):
    tol = wl.config.tolerance
    log("case %s decay=%s variant=%s B=%d H=%d tokens=%d" % (
        wl.config.name, wl.decay, wl.variant, wl.n_seq, wl.u.shape[0], wl.tokens))
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
@pytest.mark.parametrize("T", [1, 2, 7, 16])
def test_short_steps_with_state(decay, variant, T):
    _check(make_workload(5, T=T, B=3, H=4, decay=decay, variant=variant))


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
@pytest.mark.parametrize("T", [2, 9, 16])
def test_steps_without_initial_state(decay, variant, T):
    """bf16 steps of 2-16 tokens with no initial state (state_in NULL: the
    state starts at zero)."""
    wl = make_workload(1, T=T, B=5, H=3, decay=decay, variant=variant)
    assert wl.state0 is None
    _check(wl)


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
@pytest.mark.parametrize("T", [1, 16])
def test_f32_steps(decay, variant, T):
    wl = make_workload(0, T=T, B=2, H=3, decay=decay, variant=variant)
    wl.state0 = np.random.default_rng(7).normal(0, 0.1, size=(2, 3, 64, 64)).astype(np.float32)
    _check(wl)


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_ragged_steps(decay, variant):
    """Packed short sequences, one of them empty (state passed through)."""
    _check(make_workload(5, lengths=[1, 0, 16, 5, 16, 3], H=4, decay=decay, variant=variant))


@pytest.mark.parametrize("cfg", [5, 6])
@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_step_workloads_full_size(cfg, decay, variant):
    """B=128 sequences x 32 heads, T = 1 and 16: every slice."""
    _check(make_workload(cfg, decay=decay, variant=variant))


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_single_token_ragged_steps(decay, variant):
    """At most one token per sequence (the instantiation without look-ahead),
    some sequences empty: their state passes through unchanged."""
    _check(make_workload(5, lengths=[1, 0, 1, 1, 0, 1, 0], H=4, decay=decay, variant=variant))


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_all_sequences_empty(decay, variant):
    """Packed call without tokens: every state passes through bit for bit."""
    wl = make_workload(5, lengths=[0, 0, 0], H=4, decay=decay, variant=variant)
    log("case all-empty packed decay=%s variant=%s" % (decay, variant))
    o, s = run_gpu(wl)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu().numpy(), wl.state0)


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_stiff_steps(decay, variant):
    """16-token calls in which some items' decay products fall below 2^-96
    (they take the token-serial path inside the matrix-core step kernel),
    next to items without decay and items with a vanishing w."""
    wl = make_workload(5, T=16, B=3, H=4, decay=decay, variant=variant)
    bits = lambda x: f32_to_bf16_bits(np.float32(x)).item()
    w = wl.w
    if decay == "log":
        w[0, 2:10, 1, 5] = bits(4.0)        # w = exp(-e^4) ~ 2e-24 per token
        w[1, 7, 2, 63] = 0x7F80             # d = +inf: w = 0
        w[2, :, 3, 17:30] = 0xFF80          # d = -inf: w = 1
    else:
        w[0, 2:10, 1, 5] = bits(1e-30)
        w[1, 7, 2, 63] = 0x0001             # smallest denormal
        w[2, :, 3, 17:30] = bits(1.0)
    _check(wl)


def test_step_kernel_boundary_16_and_17_tokens():
    """16 tokens take the step kernel, 17 the chunked path: both match."""
    for T in (16, 17):
        _check(make_workload(5, T=T, B=2, H=8))


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_prefill_then_steps_equals_one_prefill(decay, variant):
    """A 4096-token pre-fill followed by 16 one-token steps (carried state)
    equals one pre-fill of all 4112 tokens, and the oracle."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(1, T=4112, H=8, decay=decay, variant=variant)
    g = to_gpu(wl)
    o_full, s_full = run_gpu(wl, g)
    u = None if variant == "c2" else g["u"]
    sv = lambda a, z: None if g["u2"] is None else g["u2"][:, a:z]
    o_pre, state = fw.prefill(g["r"][:, :4096], g["k"][:, :4096], g["v"][:, :4096],
                              g["w"][:, :4096], u, None, decay=decay, variant=variant,
                              second_value=sv(0, 4096))
    outs = [o_pre]
    for t in range(4096, 4112):
        o_t, state = fw.prefill(g["r"][:, t:t + 1], g["k"][:, t:t + 1], g["v"][:, t:t + 1],
                                g["w"][:, t:t + 1], u, state, decay=decay, variant=variant,
                                second_value=sv(t, t + 1))
        outs.append(o_t)
    torch.cuda.synchronize()
    o_chain = torch.cat(outs, dim=1)
    e_o = gpu_block_error(o_chain, o_full, (1, 3))
    e_s = gpu_block_error(state, s_full, (2, 3))
    log("  pre-fill + steps vs one call: o=%.3e state=%.3e" % (e_o, e_s))
    assert e_o <= 2e-3 and e_s <= 2e-3
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o_chain, state, o_ref, s_ref)
    log("  vs oracle: o=%.3e state=%.3e" % (eo, es))
    assert eo <= 2e-3 and es <= 2e-3


def test_step_graph_replays_match_eager():
    """Generation loops replay captured steps: every replay equals eager."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(5, B=16, H=8)
    g = to_gpu(wl)
    o_ref, s_ref = run_gpu(wl, g)
    torch.cuda.synchronize()
    o = torch.empty_like(o_ref)
    st = torch.empty_like(s_ref)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], g["state0"], o=o, state_out=st)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], g["state0"], o=o, state_out=st)
    torch.cuda.synchronize()
    for rep in range(4):
        o.fill_(float("nan"))
        st.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), rep
        assert torch.equal(st, s_ref), rep
