"""The single-launch path of chain verification (batches whose whole grid fits on the device at
once run as one launch, the pool tasks taking the stats workgroups' partials over through tagged
words) against the separate launches of the statistics and the draw: bit-identical outputs on the
same inputs, and parity with the oracle.  Covers small batches with draft rows (residual and bonus
draws, several pool tasks per sequence), one-hot drafts, the fused n-gram lookup, greedy and
variable-length sequences, invalid device data, repeated calls and graph replays on one workspace
(whose per-sequence run counters give every replay new tags), and a wait that gives up."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import chain_oracle, check_packed, compare_chain, f32, i32, log, logits_to_device

pytestmark = pytest.mark.gpu


def _sv():
    import draft_token_verification_09_amd as sv

    return sv


def _args(inp):
    return (logits_to_device(inp.target, inp.dtype), None if inp.draft is None else logits_to_device(inp.draft, inp.dtype),
            i32(inp.tokens), f32(inp.temperature), f32(inp.u_accept), f32(inp.u_final),
            None if inp.draft_len is None else i32(inp.draft_len))


def _kernels_of(call):
    sv = _sv()
    sv.spec_timing_reset()
    sv.spec_timing_enable(True)
    res = call()
    torch.cuda.synchronize()
    sv.spec_timing_enable(False)
    names = [name for name, _, _ in sv.spec_timing_collect()]
    sv.spec_timing_reset()
    return res, names


def _both(inp, ws=None, nv=4):
    """The default call (which must take the single launch), then the single launch and the
    separate launches with the same chunk size forced (`nv` vectors a lane), checked equal bit
    for bit; returns the default call's result."""
    sv = _sv()
    args = _args(inp)
    res, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True, workspace_buf=ws))
    assert "chain_single" in names, names
    with sv.knob(sv.SPEC_KNOB_CHUNK_VECTORS, nv):
        one, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True, workspace_buf=ws))
        assert "chain_single" in names, names
        with sv.knob(sv.SPEC_KNOB_SINGLE_LAUNCH, 1):
            two, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True, workspace_buf=ws))
            assert "chain_single" not in names, names
    for name in ("tokens", "num_accepted", "probs", "offsets"):
        assert torch.equal(getattr(one, name), getattr(two, name)), name
    total = int(two.offsets[-1])
    assert torch.equal(one.packed[:total], two.packed[:total])
    return res


CASES = {
    "B1_fp32": lambda: synth.chain_config_small_f32(3),
    "B6_fp32_residual": lambda: synth.chain_config_small_f32(4, B=6, V=9000),
    "B8_bf16_high": lambda: synth.chain_config_high_accept_bf16(5, B=8, V=30000),
    "B4_bf16_low_K8": lambda: synth.chain_config_low_accept_bf16(6, B=4, K=8, V=20001),
    "B12_bf16_bonus": lambda: dataclasses.replace(synth.chain_config_high_accept_bf16(7, B=12, K=2, V=40000),
                                                  u_accept=np.full((12, 2), 2.0 ** -24, np.float32)),
    "B16_one_hot": lambda: dataclasses.replace(synth.chain_config_high_accept_bf16(8, B=16, V=32000), draft=None),
    "B5_ragged_unaligned": lambda: synth.chain_inputs(9, B=5, K=3, V=2049, dtype="bf16", target_sigma=2.0,
                                                      draft_sigma=1.5, temperature=0.9),
}


@pytest.mark.parametrize("name", list(CASES))
def test_single_launch_matches_separate_launches_and_oracle(name):
    inp = CASES[name]()
    log(f"[single] {name}: B={inp.B} K={inp.K} V={inp.V} {inp.dtype}")
    g = _both(inp)
    rep = compare_chain(g, chain_oracle(inp), inp)
    log(f"[single]   {rep}")
    assert rep.ok(), rep.failures[:5]
    check_packed(g, inp.B)


def test_greedy_variable_length_and_invalid_sequences():
    inp = synth.chain_config_high_accept_bf16(10, B=10, K=5, V=20000)
    inp.temperature[[1, 4]] = 0.0                      # greedy sequences in a sampled batch
    inp.draft_len = np.array([5, 3, 0, 5, 2, 1, 5, 4, 5, 5], np.int32)
    inp.tokens[6, 2] = 20000                           # out of range
    inp.u_final[7] = 0.0                               # outside (0, 1]
    g = _both(inp)
    n = g.num_accepted.cpu().numpy()
    assert n[6] == -1 and n[7] == -1
    keep = [b for b in range(10) if b not in (6, 7)]
    rep = compare_chain(g, chain_oracle(inp, seqs=keep), inp, seqs=keep)
    assert rep.ok(), rep.failures[:5]


def test_ngram_lookup_in_the_same_launch():
    sv = _sv()
    pr = synth.ngram_prompts(11, B=16, L=3000, V=20000)
    ref_p = oracle.ngram_propose(pr.context, pr.context_len, 1, 4, 5)
    inp = synth.ngram_target_inputs(11, ref_p.draft, ref_p.draft_len, V=20000)
    ctx, cl = i32(pr.context), i32(pr.context_len)
    args = (ctx, cl, 1, 4, logits_to_device(inp.target, "bf16"), f32(inp.temperature), f32(inp.u_accept),
            f32(inp.u_final))
    one, names = _kernels_of(lambda: sv.spec_ngram_verify(*args, want_packed=True))
    assert "chain_single" in names, names
    with sv.knob(sv.SPEC_KNOB_SINGLE_LAUNCH, 1):
        two, names = _kernels_of(lambda: sv.spec_ngram_verify(*args, want_packed=True))
        assert "chain_single" not in names, names
    for name in ("draft_tokens", "draft_len", "match_n"):
        assert torch.equal(getattr(one.proposal, name), getattr(two.proposal, name)), name
    for name in ("tokens", "num_accepted", "probs", "offsets"):
        assert torch.equal(getattr(one.verify, name), getattr(two.verify, name)), name
    assert np.array_equal(one.proposal.draft_tokens.cpu().numpy(), ref_p.draft)
    ref = oracle.verify_chain(inp.target, None, "bf16", ref_p.draft, inp.temperature, inp.u_accept, inp.u_final,
                              draft_len=ref_p.draft_len)
    rep = compare_chain(one.verify, ref, inp)
    assert rep.ok(), rep.failures[:5]


def test_repeated_calls_and_shapes_on_one_dirty_workspace():
    # the run counters and tagged words live in the workspace: junk first, then shapes that
    # alternate, each call checked against the separate launches and the oracle
    sv = _sv()
    shapes = [synth.chain_config_small_f32(12), synth.chain_config_high_accept_bf16(13, B=8, V=30000),
              dataclasses.replace(synth.chain_config_high_accept_bf16(14, B=16, V=32000), draft=None)]
    need = max(sv.spec_verify_chain_workspace_size(i.B, i.K, i.V, 1 if i.dtype == "bf16" else 0) for i in shapes)
    ws = torch.randint(0, 255, (need + 512,), dtype=torch.uint8, device="cuda:0")
    for rnd in range(3):
        for inp in shapes:
            g = _both(inp, ws)
            rep = compare_chain(g, chain_oracle(inp), inp)
            assert rep.ok(), (rnd, inp.name, rep.failures[:5])


def test_graph_replays_get_new_tags():
    # a captured single-launch call replayed with new inputs each time: the launch arguments
    # (and the host's call number) are the same on every replay, the run counters are not
    sv = _sv()
    inps = [synth.chain_config_high_accept_bf16(30 + s, B=6, V=30000) for s in range(3)]
    dev_args = [_args(inp) for inp in inps]
    static = [x.clone() if x is not None else None for x in dev_args[0]]
    B, K1, V = static[0].shape
    out = sv.ChainResult(tokens=torch.empty((B, K1), dtype=torch.int32, device="cuda:0"),
                         num_accepted=torch.empty((B,), dtype=torch.int32, device="cuda:0"),
                         probs=torch.empty((B, K1 - 1, 3), dtype=torch.float32, device="cuda:0"),
                         packed=None, offsets=None)
    ws = torch.empty(sv.spec_verify_chain_workspace_size(B, K1 - 1, V, 1) + 256, dtype=torch.uint8, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sv.spec_verify_chain(*static, out=out, workspace_buf=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.spec_verify_chain(*static, out=out, workspace_buf=ws)
    torch.cuda.synchronize()
    for rep in range(6):
        k = (rep + 1) % 3
        for dst, src in zip(static, dev_args[k]):
            if dst is not None:
                dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"[single] graph replay {rep}: input set {k}")
        rep_ = compare_chain(out, chain_oracle(inps[k]), inps[k])
        assert rep_.ok(), rep_.failures[:5]


def test_wait_that_gives_up_flags_every_sequence():
    # on the single-launch path every pool task waits for the stats workgroups' partials, so with
    # a poll limit of 0 (forced from the host; every workgroup still exits) every sequence is
    # flagged -2 with -1 tokens and zero probabilities by its last task; then the default limit
    # gives the oracle's results on the same workspace
    sv = _sv()
    inp = synth.chain_config_high_accept_bf16(15, B=8, V=30000)
    args = _args(inp)
    with sv.knob(sv.SPEC_KNOB_POLL_LIMIT, 0):
        g = sv.spec_verify_chain(*args, want_packed=True)
        torch.cuda.synchronize()
    assert (g.num_accepted.cpu().numpy() == sv.FLAG_TIMED_OUT).all()
    assert (g.tokens.cpu().numpy() == -1).all() and (g.probs.cpu().numpy() == 0).all()
    assert int(g.offsets[-1]) == 0
    g = sv.spec_verify_chain(*args, want_packed=True)
    torch.cuda.synchronize()
    rep = compare_chain(g, chain_oracle(inp), inp)
    assert rep.ok(), rep.failures[:5]


@pytest.mark.parametrize("name", ["B8_bf16_high", "B12_bf16_bonus", "B16_one_hot", "B1_fp32"])
def test_xcd_local_hand_overs_change_nothing(name):
    # batches of 8 or more: each sequence's workgroups on one XCD (sequence b on XCD b mod 8, the
    # rest of each XCD's share idle) with its hand-overs through that XCD's L2, against
    # agent-scope hand-overs (a smaller batch keeps the spread placement either way)
    sv = _sv()
    inp = CASES[name]()
    args = _args(inp)
    assert sv.spec_get_knob(sv.SPEC_KNOB_XCD_LOCAL) == 1
    local, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True))
    assert names[0] == "chain_single", names
    with sv.knob(sv.SPEC_KNOB_XCD_LOCAL, 0):
        agent, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True))
    assert names[0] == "chain_single", names
    for field in ("tokens", "num_accepted", "probs", "offsets"):
        assert torch.equal(getattr(local, field), getattr(agent, field)), field
    rep = compare_chain(local, chain_oracle(inp), inp)
    log(f"[single] XCD-local {name}: {rep}")
    assert rep.ok(), rep.failures[:5]
