"""The fused path of chain verification (the row statistics and the draws in one launch: each
sequence decided by its last-dispatched stats workgroup, residual draws finished by helper
workgroups at the end of the grid, for batches of at most 2048 helpers) against the separate
launches: bit-identical outputs on the
same inputs, at full benchmark sizes and on ragged, greedy, invalid and one-hot batches, on a
dirty workspace reused across shapes and in graph replays; with hand-overs through one XCD's L2
and through agent-scope stores alike; and the flag of a wait that gives up."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import chain_oracle, check_packed, compare_chain, f32, fused_chunk_vectors, i32, log, logits_to_device

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


def _fused_vs_separate(inp, ws=None):
    """The default call (which must take the fused launch) and the separate launches at the same
    chunk size, checked equal bit for bit; returns the fused result."""
    sv = _sv()
    args = _args(inp)
    one, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True, workspace_buf=ws))
    assert names[0] == "chain_fused", names
    nv = fused_chunk_vectors(inp.B, inp.K, inp.V, inp.dtype, one_hot=inp.draft is None)
    with sv.knob(sv.SPEC_KNOB_SINGLE_LAUNCH, 1), sv.knob(sv.SPEC_KNOB_CHUNK_VECTORS, nv):
        two, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True, workspace_buf=ws))
    assert "chain_stats" in names and "chain_pool" in names, names
    for name in ("tokens", "num_accepted", "probs", "offsets"):
        assert torch.equal(getattr(one, name), getattr(two, name)), name
    total = int(two.offsets[-1])
    assert torch.equal(one.packed[:total], two.packed[:total])
    check_packed(one, inp.B)
    return one


CASES = {
    "headline_B64_K5_V128256": lambda: synth.chain_config_high_accept_bf16(0),
    "low_accept_B96_K8_V152064": lambda: synth.chain_config_low_accept_bf16(1, B=96),
    "ragged_B24_K5_V50000": lambda: synth.chain_config_high_accept_bf16(2, B=24, V=50000),
    "f32_B48_K5_V32000": lambda: synth.chain_config_small_f32(7, B=48),
    "one_hot_B160_K5_V128256": lambda: dataclasses.replace(
        synth.chain_config_high_accept_bf16(21, B=160, V=128256), draft=None),
    "unaligned_B120_K3_V30001": lambda: synth.chain_inputs(9, B=120, K=3, V=30001, dtype="bf16", target_sigma=2.0,
                                                           draft_sigma=1.5, temperature=0.9),
    # a batch that is not a multiple of 8: sequences straddle XCDs, every hand-over at agent scope
    "odd_B37_K4_V64000": lambda: synth.chain_inputs(16, B=37, K=4, V=64000, dtype="bf16", target_sigma=2.0,
                                                    draft_sigma=1.5, temperature=0.8),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_matches_separate_launches(name):
    inp = CASES[name]()
    log(f"[fused] {name}: B={inp.B} K={inp.K} V={inp.V} {inp.dtype}")
    g = _fused_vs_separate(inp)
    n = g.num_accepted.cpu().numpy()
    assert (n >= 0).all()
    # a sample of sequences against the oracle as well
    seqs = sorted(set(range(0, inp.B, max(1, inp.B // 6))) | {inp.B - 1})
    rep = compare_chain(g, chain_oracle(inp, seqs=seqs), inp, seqs=seqs)
    log(f"[fused]   {rep}")
    assert rep.ok(), rep.failures[:5]


@pytest.mark.parametrize("B", [64, 40, 37, 24])
def test_xcd_local_hand_overs_change_nothing(B):
    # batches whose size is a multiple of 8 keep each sequence's workgroups on one XCD and hand
    # over through its L2; the outputs must equal those of agent-scope hand-overs bit for bit
    sv = _sv()
    inp = synth.chain_config_high_accept_bf16(30 + B, B=B, V=128256 if B == 64 else 70000)
    args = _args(inp)
    assert sv.spec_get_knob(sv.SPEC_KNOB_XCD_LOCAL) == 1
    local, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True))
    assert names[0] == "chain_fused", names
    with sv.knob(sv.SPEC_KNOB_XCD_LOCAL, 0):
        agent, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True))
    assert names[0] == "chain_fused", names
    log(f"[fused] XCD-local hand-overs B={B}: mean accepted {local.num_accepted.float().mean().item():.3f}")
    for name in ("tokens", "num_accepted", "probs", "offsets"):
        assert torch.equal(getattr(local, name), getattr(agent, name)), name
    assert (local.num_accepted.cpu().numpy() >= 0).all()
    seqs = [0, B // 3, B - 1]
    rep = compare_chain(local, chain_oracle(inp, seqs=seqs), inp, seqs=seqs)
    assert rep.ok(), rep.failures[:5]


def test_greedy_variable_length_and_invalid_sequences():
    inp = synth.chain_config_high_accept_bf16(10, B=40, K=5, V=60000)
    inp.temperature[[1, 4, 30]] = 0.0
    inp.draft_len = (np.arange(40) % 6).astype(np.int32)
    inp.draft_len[[3, 17]] = [7, -1]                   # out of range: flagged
    inp.tokens[5, 0] = 60000                           # out of range (sequence 5 drafts 5 tokens)
    inp.u_final[7] = 0.0                               # outside (0, 1]
    g = _fused_vs_separate(inp)
    n = g.num_accepted.cpu().numpy()
    for b in (3, 17, 5, 7):
        assert n[b] == -1, (b, n[b])
    keep = [b for b in range(40) if b not in (3, 17, 5, 7)]
    rep = compare_chain(g, chain_oracle(inp, seqs=keep), inp, seqs=keep)
    assert rep.ok(), rep.failures[:5]


def test_dirty_workspace_reused_across_shapes():
    sv = _sv()
    shapes = [synth.chain_config_high_accept_bf16(11, B=32, V=128256),
              synth.chain_config_low_accept_bf16(12, B=20, K=8, V=100000),
              dataclasses.replace(synth.chain_config_high_accept_bf16(13, B=64, V=64000), draft=None)]
    need = max(sv.spec_verify_chain_workspace_size(i.B, i.K, i.V, 1) for i in shapes)
    ws = torch.randint(0, 255, (need + 512,), dtype=torch.uint8, device="cuda:0")
    for rnd in range(2):
        for inp in shapes:
            log(f"[fused] dirty workspace round {rnd}: B={inp.B} K={inp.K} V={inp.V}")
            _fused_vs_separate(inp, ws)


def test_graph_replays_get_new_tags():
    sv = _sv()
    inps = [synth.chain_config_low_accept_bf16(40 + s, B=24, K=6, V=90000) for s in range(3)]
    dev_args = [_args(inp) for inp in inps]
    static = [x.clone() if x is not None else None for x in dev_args[0]]
    B, K1, V = static[0].shape
    out = sv.ChainResult(tokens=torch.empty((B, K1), dtype=torch.int32, device="cuda:0"),
                         num_accepted=torch.empty((B,), dtype=torch.int32, device="cuda:0"),
                         probs=torch.empty((B, K1 - 1, 3), dtype=torch.float32, device="cuda:0"),
                         packed=None, offsets=None)
    ws = torch.empty(sv.spec_verify_chain_workspace_size(B, K1 - 1, V, 1) + 256, dtype=torch.uint8, device="cuda:0")
    refs = []
    nv = fused_chunk_vectors(B, K1 - 1, V, inps[0].dtype)
    for args in dev_args:  # the separate launches' outputs (same chunk size) for every input set
        with sv.knob(sv.SPEC_KNOB_SINGLE_LAUNCH, 1), sv.knob(sv.SPEC_KNOB_CHUNK_VECTORS, nv):
            r = sv.spec_verify_chain(*args)
        torch.cuda.synchronize()
        refs.append(r)
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
        log(f"[fused] graph replay {rep}: input set {k}")
        for name in ("tokens", "num_accepted", "probs"):
            assert torch.equal(getattr(out, name), getattr(refs[k], name)), (rep, name)


def test_wait_that_gives_up_flags_every_sequence():
    # poll limit 0 (forced from the host; every workgroup still exits): each finisher's wait for
    # its sequence's partials gives up at once, so every sequence is flagged -2 with -1 tokens
    # and zero probabilities; then the default limit gives the separate launches' outputs
    sv = _sv()
    inp = synth.chain_config_high_accept_bf16(15, B=32, V=100000)
    args = _args(inp)
    with sv.knob(sv.SPEC_KNOB_POLL_LIMIT, 0):
        g, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True))
    assert names[0] == "chain_fused", names
    assert (g.num_accepted.cpu().numpy() == sv.FLAG_TIMED_OUT).all()
    assert (g.tokens.cpu().numpy() == -1).all() and (g.probs.cpu().numpy() == 0).all()
    assert int(g.offsets[-1]) == 0
    _fused_vs_separate(inp)



def test_phase_stamps_of_the_fused_launch():
    # the fused launch's stamp layout (spec_chain_phase_stamps): 2 words per stats chunk in
    # (sequence, row, chunk) order, 4 per finisher, 7 per helper; with 16-vector chunks forced,
    # C = ceil(V / 32768) and CP = S / 4 helpers a sequence.  Every stamped phase is ordered
    # (start <= end), every finisher records its decision's mode (1 for a residual draw, 2 for a
    # bonus draw) and every helper its start and exit; the outputs are those of an unstamped call
    sv = _sv()
    inp = synth.chain_config_high_accept_bf16(31, B=40, K=5, V=50000)
    args = _args(inp)
    B, K, V = inp.B, inp.K, inp.V
    R, C = 2 * K + 1, -(-V // 32768)
    S = -(-(-(-V // 2048)) // 4) * 4
    CP = S // 4
    G = B * R * C
    buf = torch.full((2 * G + 4 * B + 7 * B * CP,), -1, dtype=torch.int64, device="cuda:0")
    with sv.knob(sv.SPEC_KNOB_CHUNK_VECTORS, 16):
        plain, _ = _kernels_of(lambda: sv.spec_verify_chain(*args))
        sv.spec_chain_phase_stamps(buf)
        try:
            g, names = _kernels_of(lambda: sv.spec_verify_chain(*args))
        finally:
            sv.spec_chain_phase_stamps(None)
    assert names[0] == "chain_fused", names
    for name in ("tokens", "num_accepted", "probs"):
        assert torch.equal(getattr(g, name), getattr(plain, name)), name
    st = buf.cpu().numpy()
    stats = st[: 2 * G].reshape(B, R * C, 2)
    fin = st[2 * G: 2 * G + 4 * B].reshape(B, 4)
    hlp = st[2 * G + 4 * B:].reshape(B, CP, 7)
    n = g.num_accepted.cpu().numpy()
    for b in range(B):
        live = stats[b, :, 0] >= 0
        assert live.sum() >= (K + 1) * C, b  # every target row's chunks at least (draft rows: kb of them)
        assert (stats[b, live, 1] >= stats[b, live, 0]).all(), b
        assert 0 <= fin[b, 0] <= fin[b, 1] <= fin[b, 2], (b, fin[b])
        assert fin[b, 3] == (1 if n[b] < K else 2), (b, fin[b, 3], n[b])
        assert (hlp[b, :, 0] >= 0).all() and (hlp[b, :, 5] >= hlp[b, :, 0]).all(), b
        if n[b] < K:  # a residual draw: every helper located it, one narrowed it
            assert (hlp[b, :, 3] >= hlp[b, :, 1]).all(), b
            owners = (hlp[b, :, 6] & 0xFF) == 1
            assert owners.sum() == 1 and hlp[b, owners, 4][0] >= hlp[b, owners, 3][0], b
            assert ((hlp[b, :, 6] >> 32) == b).all() and (((hlp[b, :, 6] >> 8) & 0xFFFFFF) == np.arange(CP)).all(), b
    log(f"[fused] stamps: {int((n < K).sum())} residual draws, {int((n == K).sum())} bonus draws")


def test_residual_mass_lost_to_rounding_in_the_fused_launch():
    # A rejected draft whose residual max(0, p - q) is zero in both arithmetics, at a batch that
    # runs as the fused launch (hand-overs in one XCD's L2): the last helper finds no mass,
    # re-reads row 0's partials (checking every word's tag) and draws from p_0.  Each row holds
    # 2^17 logits of 0 and four of -50, so every row sum is exactly 2^17 and every p (and q) of a
    # 0 logit exactly 2^-17; the drafted token is a -50 in the target and -49 in the draft, so
    # alpha = 1/e, u = 1 rejects it and q(x) moves no row sum.  u_final stays half a token away
    # from every boundary of p_0's cumulative sum.
    sv = _sv()
    B, K, V = 56, 2, (1 << 17) + 4  # 56 x 33 helpers: one fused launch
    rng = np.random.default_rng(17)
    target = np.zeros((B, K + 1, V), np.float32)
    tokens = np.zeros((B, K), np.int32)
    for b in range(B):
        neg = rng.choice(V, size=4, replace=False)
        target[b, :, neg] = np.float32(-50.0)
        tokens[b] = [int(neg[0]), int(rng.integers(0, V))]
    draft = target[:, :K].copy()
    draft[np.arange(B), 0, tokens[:, 0]] = np.float32(-49.0)
    u_fin = ((rng.integers(0, 1 << 17, B) + 0.5) / float(1 << 17)).astype(np.float32)
    inp = synth.ChainInputs(target=target, draft=draft, dtype="f32", tokens=tokens, draft_len=None,
                            temperature=np.ones((B,), np.float32), u_accept=np.ones((B, K), np.float32),
                            u_final=u_fin, name="lost_residual")
    ref = chain_oracle(inp)
    assert all(s.mode == "residual_zero_fallback" and s.num_accepted == 0 for s in ref.sequences)
    args = _args(inp)
    g, names = _kernels_of(lambda: sv.spec_verify_chain(*args, want_packed=True))
    assert names[0] == "chain_fused", names
    rep = compare_chain(g, ref, inp)
    log(f"[fused] lost residual mass B={B} V={V}: {rep}")
    assert rep.ok(), rep.failures[:5]
    with sv.knob(sv.SPEC_KNOB_XCD_LOCAL, 0):
        h = sv.spec_verify_chain(*args)
    torch.cuda.synchronize()
    for name in ("tokens", "num_accepted", "probs"):
        assert torch.equal(getattr(g, name), getattr(h, name)), name
