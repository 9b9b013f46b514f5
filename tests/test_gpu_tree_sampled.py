"""GPU parity of spec_verify_tree (stochastic tree verification) against the oracle.

Accepted lengths, path nodes and tokens must match the oracle exactly.  The one
exception, as for chains, is a sequence whose walk first differs from the oracle's at a
decision within 1e-5 of its boundary (|u - alpha| for an accept test, the normalised
inverse-CDF gap for the final draw when every accept test agrees): that difference is
counted as a flip, not a failure, and a comparison allows at most a couple of them.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import compare_tree_sampled, dev, f32, i32, log, logits_to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _sv():
    import draft_token_verification_09_amd as sv

    return sv


def run_gpu(x, max_depth=None, workspace_buf=None):
    sv = _sv()
    md = x.max_depth if max_depth is None else max_depth
    r = sv.spec_verify_tree(logits_to_device(x.target, x.dtype), logits_to_device(x.draft, x.dtype), i32(x.parent),
                            i32(x.node_token), f32(x.temperature), f32(x.u_accept), f32(x.u_final), md,
                            workspace_buf=workspace_buf)
    torch.cuda.synchronize()
    return r


def oracle_of(x, max_depth=None, seqs=None):
    md = x.max_depth if max_depth is None else max_depth
    return oracle.verify_tree_sampled(x.target, x.draft, x.dtype, x.parent, x.node_token, x.temperature, x.u_accept,
                                      x.u_final, md, seqs=seqs)


def check(g, ref, x, seqs=None, what=""):
    rep = compare_tree_sampled(g, ref, x, seqs=seqs)
    log(f"[tree_sampled] {x.name}{what}: B={x.B} N1={x.N1} V={x.V}: {rep}")
    assert rep.ok(), rep.failures[:4]
    return rep


def compare(x, max_depth=None, seqs=None):
    g = run_gpu(x, max_depth)
    ref = oracle_of(x, max_depth, seqs)
    check(g, ref, x, seqs)
    return g, ref


def test_golden_b1_rejected_b2_accepted():
    with open(os.path.join(GOLDEN, "tree_sampled_b1_rejected_b2_accepted.json")) as f:
        fx = json.load(f)
    tgt = np.log(np.asarray(fx["target_probs"], dtype=np.float64)).astype(np.float32)[None]
    dft = np.log(np.asarray(fx["draft_probs"], dtype=np.float64)).astype(np.float32)[None]
    x = synth.SampledTreeInputs(target=tgt, draft=dft, dtype="f32", parent=np.asarray([fx["parent"]], np.int32),
                                node_token=np.asarray([fx["node_token"]], np.int32),
                                temperature=np.asarray([fx["temperature"]], np.float32),
                                u_accept=np.asarray([fx["u_accept"]], np.float32),
                                u_final=np.asarray([fx["u_final"]], np.float32), max_depth=fx["max_depth"],
                                name="golden")
    g = run_gpu(x)
    exp = fx["expected"]
    assert int(g.accept_len[0]) == exp["accept_len"]
    assert g.path_nodes[0].cpu().tolist() == exp["path_nodes"]
    assert g.tokens[0].cpu().tolist() == exp["tokens"]


def test_full_size_eagle_trees_bf16():
    # B=32 trees of 60 nodes + root, depth 6, V=128256 bf16 (16 workgroups per sequence)
    compare(synth.tree_sampled_config_bf16(0))


@pytest.mark.parametrize("V,dtype,kind,N1", [
    (1000, "f32", "mixed", 17),      # one slice, ragged
    (33000, "f32", "mixed", 40),     # several slices, ragged tail
    (32001, "bf16", "mixed", 40),    # V * 2 not a multiple of 16: element-wise loads
    (50000, "bf16", "star", 30),     # many siblings: many residual passes
    (20000, "bf16", "chain", 24),    # a deep walk
    (8192 * 5, "bf16", "random", 64),  # slices end exactly at V
])
def test_shapes_and_topologies(V, dtype, kind, N1):
    B = 12
    parent = synth.random_parents(V % 97, B=B, N1=N1, kind=kind)
    x = synth.tree_sampled_inputs(V % 89, B=B, n_nodes=N1 - 1, depth=N1 - 1, V=V, dtype=dtype, parent=parent,
                                  target_sigma=2.0, draft_sigma=1.0, temperature=1.0, peaks=4, peak_shift=4.0,
                                  name=f"{kind}_{dtype}_V{V}")
    compare(x)


def test_low_and_high_temperature():
    for T in (0.3, 2.5):
        x = synth.tree_sampled_inputs(int(T * 10), B=10, n_nodes=30, depth=5, V=24000, dtype="bf16", temperature=T,
                                      name=f"T{T}")
        compare(x)


def test_chain_shaped_trees_match_chain_verification():
    # a chain-shaped tree is spec_verify_chain on the same rows and uniforms
    sv = _sv()
    B, K, V = 16, 5, 40000
    ch = synth.chain_config_high_accept_bf16(3, B=B, K=K, V=V)
    parent = np.tile(np.arange(-1, K, dtype=np.int32), (B, 1))
    draft = np.concatenate([ch.draft, ch.draft[:, :1]], axis=1)  # the leaf's draft row is never read
    x = synth.SampledTreeInputs(target=ch.target, draft=draft, dtype="bf16", parent=parent,
                                node_token=np.concatenate([np.zeros((B, 1), np.int32), ch.tokens], axis=1),
                                temperature=ch.temperature,
                                u_accept=np.concatenate([np.full((B, 1), 0.5, np.float32), ch.u_accept], axis=1),
                                u_final=ch.u_final, max_depth=K, name="chain-shaped")
    g, ref = compare(x)
    c = sv.spec_verify_chain(logits_to_device(ch.target, "bf16"), logits_to_device(ch.draft, "bf16"), i32(ch.tokens),
                             f32(ch.temperature), f32(ch.u_accept), f32(ch.u_final))
    torch.cuda.synchronize()
    same = (c.num_accepted.cpu().numpy() == g.accept_len.cpu().numpy())
    assert (~same).sum() <= 2  # identical except for near-boundary flips of either path
    for b in np.flatnonzero(same):
        n = int(c.num_accepted[b])
        assert c.tokens[b, : n + 1].cpu().tolist() == g.tokens[b, : n + 1].cpu().tolist()


def test_invalid_sequences_are_flagged():
    x = synth.tree_sampled_inputs(5, B=6, n_nodes=12, depth=3, V=3000, dtype="f32", name="invalid")
    x.parent[1, 4] = 7          # parent after child
    x.node_token[2, 3] = 3000   # token out of range
    x.temperature[3] = 0.0      # greedy belongs to spec_verify_tree_greedy
    x.u_accept[4, 5] = 0.0      # uniform outside (0, 1]
    g = run_gpu(x)
    acc = g.accept_len.cpu().numpy()
    assert (acc[1:5] == -1).all()
    assert (g.tokens[1:5].cpu().numpy() == -1).all() and (g.path_nodes[1:5].cpu().numpy() == -1).all()
    compare(x, seqs=[0, 5])


def test_path_longer_than_max_depth_is_flagged():
    # chains that accept everything (draft = target, u small) but max_depth = 2
    B, N1, V = 4, 6, 2000
    parent = np.tile(np.arange(-1, N1 - 1, dtype=np.int32), (B, 1))
    x = synth.tree_sampled_inputs(6, B=B, n_nodes=N1 - 1, depth=N1 - 1, V=V, dtype="f32", parent=parent,
                                  draft_sigma=0.0, name="max_depth")
    x.u_accept[:] = np.float32(2.0**-24)
    g = run_gpu(x, max_depth=2)
    assert (g.accept_len.cpu().numpy() == -1).all()
    compare(x, max_depth=5)


def test_several_launches_and_dirty_workspace():
    # B = 70 sequences of 16 workgroups each need several launches at the default occupancy;
    # the workspace is filled with junk first, then reused by a call of another shape and by
    # a second call of the first: every result is checked against the oracle
    sv = _sv()
    x = synth.tree_sampled_inputs(7, B=70, n_nodes=7, depth=3, V=128256, dtype="bf16", name="B70")
    need = int(sv.lib().spec_verify_tree_workspace_size(70, 8, 128256, 1))
    buf = torch.randint(0, 255, (need + 512,), dtype=torch.uint8, device=dev())
    ref = oracle_of(x)
    check(run_gpu(x, workspace_buf=buf), ref, x, what=" (junk-filled workspace)")
    y = synth.tree_sampled_inputs(8, B=9, n_nodes=20, depth=4, V=9000, dtype="f32", name="reuse")
    check(run_gpu(y, workspace_buf=buf), oracle_of(y), y, what=" (workspace reused)")
    check(run_gpu(x, workspace_buf=buf), ref, x, what=" (workspace reused again)")


def test_prepared_call_matches_plain_call():
    sv = _sv()
    x = synth.tree_sampled_inputs(9, B=8, n_nodes=20, depth=4, V=20000, dtype="bf16", name="prepared")
    args = (logits_to_device(x.target, "bf16"), logits_to_device(x.draft, "bf16"), i32(x.parent), i32(x.node_token),
            f32(x.temperature), f32(x.u_accept), f32(x.u_final), x.max_depth)
    pc = sv.prepare_spec_verify_tree(*args)
    r1 = pc()
    r1 = sv.TreeResult(r1.accept_len.clone(), r1.tokens.clone(), r1.path_nodes.clone(), None)
    r2 = sv.spec_verify_tree(*args)
    torch.cuda.synchronize()
    assert torch.equal(r1.accept_len, r2.accept_len) and torch.equal(r1.tokens, r2.tokens)
    assert torch.equal(r1.path_nodes, r2.path_nodes)


def test_graph_replays_match_eager_calls():
    # the walk's hand-over generation changes on every run, so a captured call replays
    # correctly with new inputs each time
    sv = _sv()
    xs = [synth.tree_sampled_inputs(40 + s, B=6, n_nodes=20, depth=4, V=30000, dtype="bf16", name=f"g{s}")
          for s in range(3)]

    def dev_args(x):
        return [logits_to_device(x.target, "bf16"), logits_to_device(x.draft, "bf16"), i32(x.parent),
                i32(x.node_token), f32(x.temperature), f32(x.u_accept), f32(x.u_final)]

    args = [dev_args(x) for x in xs]
    static = [t.clone() for t in args[0]]
    B, D1 = 6, xs[0].max_depth + 1
    out = sv.TreeResult(torch.empty(B, dtype=torch.int32, device=dev()),
                        torch.empty((B, D1), dtype=torch.int32, device=dev()),
                        torch.empty((B, D1), dtype=torch.int32, device=dev()), None)
    ws = torch.empty(int(sv.lib().spec_verify_tree_workspace_size(B, 21, 30000, 1)) + 256, dtype=torch.uint8,
                     device=dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sv.spec_verify_tree(*static, xs[0].max_depth, out=out, workspace_buf=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.spec_verify_tree(*static, xs[0].max_depth, out=out, workspace_buf=ws)
    torch.cuda.synchronize()
    for rep in range(6):
        k = (rep + 1) % 3
        for dst, src in zip(static, args[k]):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = sv.spec_verify_tree(*args[k], xs[k].max_depth)
        torch.cuda.synchronize()
        log(f"[tree_sampled] graph replay {rep}: input set {k}")
        assert torch.equal(out.accept_len, eager.accept_len)
        assert torch.equal(out.tokens, eager.tokens) and torch.equal(out.path_nodes, eager.path_nodes)


def test_wait_that_gives_up_flags_every_walk():
    # With a poll limit of 0 every hand-over wait gives up before its first poll (forced
    # from the host; every workgroup still exits): each sequence is flagged -2 with -1
    # outputs, written by the sequence's workgroup 0 alone.  Then, with the default limit,
    # the same inputs match the oracle, so a flagged call leaves nothing behind.
    sv = _sv()
    x = synth.tree_sampled_inputs(12, B=10, n_nodes=20, depth=4, V=40000, dtype="bf16", name="poll0")
    with sv.knob(sv.SPEC_KNOB_POLL_LIMIT, 0):
        g = run_gpu(x)
    assert (g.accept_len.cpu().numpy() == sv.FLAG_TIMED_OUT).all()
    assert (g.tokens.cpu().numpy() == -1).all() and (g.path_nodes.cpu().numpy() == -1).all()
    compare(x)


@pytest.mark.parametrize("B", [32, 13])
def test_xcd_local_hand_overs_change_nothing(B):
    # as for the greedy walk: slice exchanges through one XCD's L2 (a launch of a multiple of
    # 8 sequences) and through agent-scope stores give the same walks, which match the oracle
    sv = _sv()
    x = synth.tree_sampled_config_bf16(60 + B) if B == 32 else synth.tree_sampled_inputs(
        61, B=B, n_nodes=30, depth=5, V=128256, dtype="bf16", name="B13")
    assert sv.spec_get_knob(sv.SPEC_KNOB_XCD_LOCAL) == 1
    g = run_gpu(x)
    with sv.knob(sv.SPEC_KNOB_XCD_LOCAL, 0):
        h = run_gpu(x)
    for name in ("accept_len", "tokens", "path_nodes"):
        assert torch.equal(getattr(g, name), getattr(h, name)), name
    seqs = [0, B // 2, B - 1]
    check(g, oracle_of(x, seqs=seqs), x, seqs=seqs, what=" (XCD-local)")
