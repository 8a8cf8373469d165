"""Self-decoder gated retention on the GPU against the float64 oracle.

Tolerance.  The kernel takes q, k, v as exact bf16 operands and every fp32
operand of a matrix product (the state, the decayed scores, the gated keys)
as a bf16 high part plus a bf16 low part, which keeps about 17 significant
bits (relative error <= 2^-17 per product); sums are fp32; the decay of a term
is 2^(b_t - b_s) with b an fp32 prefix sum of hardware log2 over at most 32
tokens (relative error a few 1e-7 for gates in [0.5, 1]).  Every error is a
small multiple of the magnitude of the terms it sits on, so the bound is
taken against M, the oracle run on |q|, |k|, |v| and |S0| with the same gates
(the sum of the terms' magnitudes):  |out - oracle| <= 1e-4 M + 1e-6, about
ten times the expected error.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import dev, host, say
from yoco_shared_kv_gather_amd import binding as yb
from yoco_shared_kv_gather_amd import synth

pytestmark = pytest.mark.gpu

REL = 1e-4
ABS = 1e-6


def _to_dev(inp):
    d = dev()
    return dict(q=inp.q.to(d), k=inp.k.to(d), v=inp.v.to(d), gamma=inp.gamma.to(d),
                cu=torch.from_numpy(inp.cu_seqlens).to(d), idx=torch.from_numpy(inp.state_indices).to(d),
                state=inp.state.to(d))


def _oracle_pair(inp, gamma=None, state=None, idx=None, cu=None, rows=None):
    """Oracle outputs and their magnitude bound M for the given rows."""
    q, k, v = host(inp.q), host(inp.k), host(inp.v)
    g = host(inp.gamma) if gamma is None else gamma
    s0 = host(inp.state) if state is None else state
    idx = inp.state_indices if idx is None else idx
    cu = inp.cu_seqlens if cu is None else cu
    if rows is not None:
        q, k, v, g = q[rows], k[rows], v[rows], g[rows]
    ref = oracle.gated_retention(q, k, v, g, cu, s0, idx)
    mag = oracle.gated_retention(np.abs(q), np.abs(k), np.abs(v), g, cu, np.abs(s0), idx)
    return ref, mag


def _close(name, got, ref, mag):
    err = np.abs(got - ref)
    bound = REL * mag + ABS
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"  {name}: max abs err {float(err.max()) if err.size else 0.0:.3e}, worst err/bound {worst:.3f}")
    assert np.all(err <= bound), name


def _run(t, out=None, max_seqlen=0):
    if out is None:
        out = torch.full(t["q"].shape, float("nan"), dtype=torch.float32, device=t["q"].device)
    yb.gated_retention(t["q"], t["k"], t["v"], t["gamma"], t["cu"], t["state"], t["idx"], max_seqlen=max_seqlen,
                       out=out)
    return out


# max_seqlen picks the schedule: 1 the recurrent kernel, <= 2048 one chunkwise
# run per request, 0 (unknown) 2048-row segments in two launches; every
# schedule computes every request in full
PLANS = {"recurrent": 1, "whole": 2048, "segmented": 0}
SHORT = [1, 31, 32, 33, 0, 100, 7, 64, 200]
LONG = [6000, 2048, 2049, 0, 4096, 5, 1, 4200]


@pytest.mark.parametrize("plan", sorted(PLANS))
@pytest.mark.parametrize("lens", [SHORT, LONG], ids=["short", "long"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_retention_matches_oracle(head_dim, lens, plan):
    """Requests of partial, whole and many chunks (short: up to 200 rows;
    long: up to 6000 rows, so up to three segments), some starting from a
    zero state (slot -1), on every schedule; all outputs and every slot
    checked."""
    heads = 3 if lens is SHORT else 2
    say(f"retention: lens {lens}, {heads} heads x {head_dim}, plan {plan}")
    inp = synth.make_retention_inputs(lens, heads, head_dim, zero_state_every=4)
    t = _to_dev(inp)
    out = _run(t, max_seqlen=PLANS[plan])
    torch.cuda.synchronize()
    (ref, new_state), (mag, mag_state) = _oracle_pair(inp)
    _close("outputs", host(out), ref, mag)
    _close("states", host(t["state"]), new_state, mag_state)
    # slots no request names keep their bits
    named = set(int(i) for i, n in zip(inp.state_indices, lens) if i >= 0 and n > 0)
    for s in range(inp.state.shape[0]):
        if s not in named:
            assert torch.equal(t["state"][s].cpu().view(torch.int32), inp.state[s].view(torch.int32)), s


@pytest.mark.parametrize("plan", sorted(PLANS))
@pytest.mark.parametrize("gamma_value", [0.0, 1.0])
def test_retention_gate_edges(gamma_value, plan):
    """gamma = 1 (no forgetting, the state sums every k^T v over 2600 rows,
    two segments) and gamma = 0 (only the current token: o_t = (q_t . k_t)
    v_t), on every schedule."""
    say(f"retention: gamma = {gamma_value}, plan {plan}")
    inp = synth.make_retention_inputs([2600, 5, 1], 2, 128)
    inp.gamma.fill_(gamma_value)
    t = _to_dev(inp)
    out = _run(t, max_seqlen=PLANS[plan])
    torch.cuda.synchronize()
    (ref, new_state), (mag, mag_state) = _oracle_pair(inp)
    _close("outputs", host(out), ref, mag)
    _close("states", host(t["state"]), new_state, mag_state)
    if gamma_value == 0.0:
        q, k, v = host(inp.q), host(inp.k), host(inp.v)
        direct = np.einsum("thd,thd->th", q.astype(np.float64), k)[..., None] * v
        _close("(q.k) v", host(out), direct, np.einsum("thd,thd->th", np.abs(q), np.abs(k))[..., None] * np.abs(v))


def test_retention_split_calls_carry_the_state():
    """A prefill in two calls (the state carried in the slots; the longest
    request two segments in the first call) and then five one-token decode
    steps on the recurrent kernel give the single oracle run's outputs and
    state."""
    lens = np.array([40, 70, 1, 33, 6600], dtype=np.int64)
    steps = 5
    total = lens + steps
    say(f"retention: prefill {list(lens)} in two calls, then {steps} decode steps")
    inp = synth.make_retention_inputs(total, 4, 128)
    (ref, new_state), (mag, mag_state) = _oracle_pair(inp)
    d = dev()
    cu = inp.cu_seqlens
    state = inp.state.to(d)
    idx = torch.from_numpy(inp.state_indices).to(d)
    q, k, v, g = (x.to(d) for x in (inp.q, inp.k, inp.v, inp.gamma))

    def call(row_lists, max_seqlen):
        rows = np.concatenate(row_lists).astype(np.int64)
        c = np.zeros(len(row_lists) + 1, dtype=np.int32)
        c[1:] = np.cumsum([len(r) for r in row_lists])
        ri = torch.from_numpy(rows).to(d)
        o = torch.full((len(rows),) + tuple(q.shape[1:]), float("nan"), dtype=torch.float32, device=d)
        yb.gated_retention(q[ri].contiguous(), k[ri].contiguous(), v[ri].contiguous(), g[ri].contiguous(),
                           torch.from_numpy(c).to(d), state, idx, max_seqlen=max_seqlen, out=o)
        return rows, o

    got = np.full(ref.shape, np.nan)
    first = lens // 3
    for part in ([np.arange(cu[r], cu[r] + first[r]) for r in range(len(lens))],
                 [np.arange(cu[r] + first[r], cu[r] + lens[r]) for r in range(len(lens))]):
        rows, o = call(part, 0)
        got[rows] = host(o)
    for step in range(steps):
        rows, o = call([np.array([cu[r] + lens[r] + step]) for r in range(len(lens))], 1)
        got[rows] = host(o)
    torch.cuda.synchronize()
    _close("outputs", got, ref, mag)
    _close("states", host(state), new_state, mag_state)


@pytest.mark.parametrize("plan", sorted(PLANS))
def test_retention_is_deterministic_and_writes_only_owned_rows(plan):
    """Two calls on the same inputs give the same bits; rows that no request
    owns keep their contents, and empty requests leave their slots alone."""
    say(f"retention: determinism, unowned rows, plan {plan}")
    inp = synth.make_retention_inputs([50, 0, 17, 0, 2090], 2, 128)
    t = _to_dev(inp)
    # rows past the last request: graph padding
    pad = 9
    d = dev()
    for name in ("q", "k", "v"):
        t[name] = torch.cat([t[name], torch.randn((pad,) + tuple(t[name].shape[1:]), device=d).to(t[name].dtype)])
    t["gamma"] = torch.cat([t["gamma"], torch.rand((pad, t["gamma"].shape[1]), device=d)])
    s0 = t["state"].clone()
    out1 = _run(t, max_seqlen=PLANS[plan])
    s1 = t["state"].clone()
    t["state"].copy_(s0)
    out2 = _run(t, max_seqlen=PLANS[plan])
    torch.cuda.synchronize()
    assert torch.equal(out1[:-pad].view(torch.int32), out2[:-pad].view(torch.int32))
    assert torch.equal(s1.view(torch.int32), t["state"].view(torch.int32))
    assert bool(torch.isnan(out1[-pad:]).all())
    for r, n in enumerate(inp.lens):
        if n == 0 and inp.state_indices[r] >= 0:
            s = int(inp.state_indices[r])
            assert torch.equal(s1[s].view(torch.int32), s0[s].view(torch.int32))


def test_retention_full_size_sampled():
    """The mixed step's request mix (16 prefills of 512..16384 rows, 32
    one-token decodes), 24 heads x 128, in one segmented call as the
    benchmark runs it: the longest prefill, a short one and a decode, two
    heads each, against the oracle."""
    lens = synth.retention_lengths("mixed48")
    say(f"retention: full mixed48 mix, {int(lens.sum())} rows, 24 heads x 128")
    inp = synth.make_retention_inputs(lens, 24, 128, device=dev())
    state0 = inp.state.clone()
    t = dict(q=inp.q, k=inp.k, v=inp.v, gamma=inp.gamma, cu=torch.from_numpy(inp.cu_seqlens).to(dev()),
             idx=torch.from_numpy(inp.state_indices).to(dev()), state=inp.state)
    out = torch.empty(inp.q.shape, dtype=torch.float32, device=dev())
    _run(t, out, max_seqlen=int(lens.max()))
    torch.cuda.synchronize()
    order = np.argsort(lens)
    picks = [int(order[-1]), int(next(i for i in order if lens[i] > 1)), int(order[0])]
    cu = inp.cu_seqlens
    for r in picks:
        a, b = int(cu[r]), int(cu[r + 1])
        slot = int(inp.state_indices[r])
        for h in (0, 23):
            sl = lambda x: host(x[a:b, h:h + 1])
            q, k, v, g = sl(inp.q), sl(inp.k), sl(inp.v), host(inp.gamma[a:b, h:h + 1])
            s0 = host(state0[slot:slot + 1, h:h + 1])
            cu1 = np.array([0, b - a])
            ref, st = oracle.gated_retention(q, k, v, g, cu1, s0, np.array([0]))
            mag, mst = oracle.gated_retention(np.abs(q), np.abs(k), np.abs(v), g, cu1, np.abs(s0), np.array([0]))
            _close(f"request {r} ({b - a} rows) head {h} outputs", host(out[a:b, h:h + 1]), ref, mag)
            _close(f"request {r} head {h} state", host(t["state"][slot:slot + 1, h:h + 1]), st, mst)


def test_retention_decode_batch_full_size():
    """64 one-token decodes, 24 heads x 128, on the recurrent kernel as the
    benchmark runs it; every output and state against the oracle."""
    lens = synth.retention_lengths("decode64")
    say("retention: decode64, 24 heads x 128, recurrent kernel")
    inp = synth.make_retention_inputs(lens, 24, 128)
    t = _to_dev(inp)
    out = _run(t, max_seqlen=1)
    torch.cuda.synchronize()
    (ref, new_state), (mag, mag_state) = _oracle_pair(inp)
    _close("outputs", host(out), ref, mag)
    _close("states", host(t["state"]), new_state, mag_state)


def test_retention_in_a_hip_graph():
    """A segmented retention call (two launches, workspace) and a decode call
    on the recurrent kernel, captured in one HIP graph and replayed three
    times with eager work between the replays: every replay gives the eager
    bits (the calls allocate nothing and write no memsets)."""
    say("retention: HIP graph capture, segmented + recurrent")
    d = dev()
    pre = synth.make_retention_inputs([2500, 700, 0, 33], 2, 128, device=d)
    dec = synth.make_retention_inputs([1] * 6, 2, 128, device=d, tag=78)
    ws = torch.empty(max(16, yb.gated_retention_workspace_size(int(pre.lens.sum()), 4, 2, 128, 0)),
                     dtype=torch.uint8, device=d)
    cu_p, idx_p = torch.from_numpy(pre.cu_seqlens).to(d), torch.from_numpy(pre.state_indices).to(d)
    cu_d, idx_d = torch.from_numpy(dec.cu_seqlens).to(d), torch.from_numpy(dec.state_indices).to(d)
    out_p = torch.empty(pre.q.shape, dtype=torch.float32, device=d)
    out_d = torch.empty(dec.q.shape, dtype=torch.float32, device=d)
    sp0, sd0 = pre.state.clone(), dec.state.clone()
    stream = torch.cuda.Stream()

    def step():
        s = torch.cuda.current_stream()
        yb.gated_retention(pre.q, pre.k, pre.v, pre.gamma, cu_p, pre.state, idx_p, max_seqlen=0, out=out_p,
                           workspace=ws, stream=s)
        yb.gated_retention(dec.q, dec.k, dec.v, dec.gamma, cu_d, dec.state, idx_d, max_seqlen=1, out=out_d,
                           stream=s)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    eager = [x.clone() for x in (out_p, out_d, pre.state, dec.state)]
    graph = torch.cuda.CUDAGraph()
    pre.state.copy_(sp0)
    dec.state.copy_(sd0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        step()
    for replay in range(3):
        out_p.fill_(float("nan"))
        out_d.fill_(float("nan"))
        pre.state.copy_(sp0)
        dec.state.copy_(sd0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        owned = int(pre.cu_seqlens[-1])
        for got, want in zip((out_p[:owned], out_d, pre.state, dec.state), (eager[0][:owned], *eager[1:])):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), replay
        # eager work between replays, on the default stream
        yb.gated_retention(dec.q, dec.k, dec.v, dec.gamma, cu_d, dec.state, idx_d, max_seqlen=1)
        torch.cuda.synchronize()
    say("  3 replays identical to the eager calls")


@pytest.mark.parametrize("plan", sorted(PLANS))
def test_retention_without_state_slots(plan):
    """No state tensor rows at all (num_slots = 0): every request starts from
    zeros and nothing is stored, on every schedule."""
    say(f"retention: no state slots, plan {plan}")
    inp = synth.make_retention_inputs([1100, 3, 0, 40], 2, 64)
    d = dev()
    t = _to_dev(inp)
    t["state"] = torch.empty((0, 2, 64, 64), dtype=torch.float32, device=d)
    out = _run(t, max_seqlen=PLANS[plan])
    torch.cuda.synchronize()
    none = -np.ones(len(inp.lens), dtype=np.int64)
    (ref, _), (mag, _) = _oracle_pair(inp, state=np.zeros((1, 2, 64, 64)), idx=none)
    _close("outputs", host(out), ref, mag)
