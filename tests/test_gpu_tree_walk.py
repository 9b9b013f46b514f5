"""GPU parity of greedy tree verification without per-node argmaxes (the walk that reads
only the accepted nodes' rows) against the oracle: accepted length, tokens and path
nodes bit-exact, and equal to the full design (every row's argmax) on the same inputs."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import dev, i32, log, logits_to_device
from test_golden import load_fixtures, tree_rows

pytestmark = pytest.mark.gpu


def _sv():
    import draft_token_verification_09_amd as sv

    return sv


def walk(tr, max_depth=None, want_argmax=False, workspace_buf=None):
    md = tr.max_depth if max_depth is None else max_depth
    r = _sv().spec_verify_tree_greedy(logits_to_device(tr.target, tr.dtype), i32(tr.parent), i32(tr.node_token), md,
                                      want_argmax=want_argmax, workspace_buf=workspace_buf)
    torch.cuda.synchronize()
    return r


def compare(tr, max_depth=None):
    md = tr.max_depth if max_depth is None else max_depth
    log(f"[tree walk] {tr.name} B={tr.B} N1={tr.N1} V={tr.V}")
    g = walk(tr, md)
    ref = oracle.verify_tree_greedy(tr.target, tr.dtype, tr.parent, tr.node_token, md)
    assert g.argmax is None
    assert np.array_equal(g.accept_len.cpu().numpy(), ref.accept_len)
    assert np.array_equal(g.tokens.cpu().numpy(), ref.tokens)
    assert np.array_equal(g.path_nodes.cpu().numpy(), ref.path_nodes)
    full = walk(tr, md, want_argmax=True)
    assert torch.equal(full.accept_len, g.accept_len) and torch.equal(full.tokens, g.tokens)
    assert torch.equal(full.path_nodes, g.path_nodes)
    log(f"[tree walk]   exact; mean accept_len {ref.accept_len.mean():.3f}")
    return g, ref


def test_walk_eagle_full_size():
    compare(synth.tree_config_eagle_bf16(0))


@pytest.mark.parametrize("V", [1000, 77777, 8192 * 4])
def test_walk_ragged_vocab(V):
    compare(synth.tree_inputs(4, B=8, n_nodes=30, depth=5, V=V, dtype="bf16", p_boost=0.9))


def test_walk_fp32_ties():
    tr = synth.tree_inputs(9, B=16, n_nodes=40, depth=4, V=3000, dtype="f32", p_boost=0.9)
    tr.target = np.round(tr.target / 3.0).astype(np.float32)
    compare(tr)


def test_walk_repeated_sibling_tokens():
    # every node's children share one token: when it is the argmax all of them are
    # accepted, the frontier holds several nodes and the deepest, smallest one wins
    tr = synth.tree_inputs(12, B=16, n_nodes=40, depth=5, V=2000, dtype="bf16", p_boost=1.0)
    for b in range(tr.B):
        first = {}
        for i in range(1, tr.N1):
            p = int(tr.parent[b, i])
            first.setdefault(p, int(tr.node_token[b, i]))
            tr.node_token[b, i] = first[p]
    compare(tr)


@pytest.mark.parametrize("kind", ["chain", "star"])
def test_walk_chains_and_stars(kind):
    B, N1, V = 10, 40, 5000
    parent = synth.random_parents(31, B=B, N1=N1, kind=kind)
    tr = synth.tree_inputs(13, B=B, n_nodes=N1 - 1, depth=N1 - 1, V=V, dtype="f32", p_boost=1.0)
    tr.parent = parent
    # make every row's argmax the token of its first child (a chain is accepted to the end)
    for b in range(B):
        kids = {}
        for i in range(1, N1):
            kids.setdefault(int(parent[b, i]), i)
        for u, c in kids.items():
            tr.target[b, u, int(tr.node_token[b, c])] = 50.0
    compare(tr, max_depth=N1 - 1)


@pytest.mark.parametrize("fx", load_fixtures("tree"), ids=lambda f: f["_name"])
def test_walk_golden(fx):
    rows = torch.from_numpy(tree_rows(fx)[None]).to(dev())
    r = _sv().spec_verify_tree_greedy(rows, i32([fx["parent"]]), i32([fx["node_token"]]), fx["max_depth"],
                                      want_argmax=False)
    torch.cuda.synchronize()
    exp = fx["expected"]
    assert int(r.accept_len[0]) == exp["accept_len"]
    assert r.path_nodes[0].cpu().tolist() == exp["path_nodes"]
    assert r.tokens[0].cpu().tolist() == exp["tokens"]


def test_walk_invalid_and_max_depth():
    tr = synth.tree_inputs(3, B=6, n_nodes=12, depth=3, V=500, dtype="bf16", p_boost=1.0)
    tr.parent[1, 4] = 9          # a parent after its child
    tr.node_token[2, 5] = 500    # token out of range
    g = walk(tr)
    assert (g.accept_len.cpu().numpy()[1:3] == -1).all()
    assert (g.tokens[1:3].cpu().numpy() == -1).all() and (g.path_nodes[1:3].cpu().numpy() == -1).all()
    ok = [0, 3, 4, 5]  # the oracle raises on the broken sequences instead of flagging them
    ref = oracle.verify_tree_greedy(tr.target, tr.dtype, tr.parent, tr.node_token, tr.max_depth, seqs=ok)
    assert np.array_equal(g.accept_len.cpu().numpy()[ok], ref.accept_len[ok])
    # max_depth = 1: a deeper accepted path is flagged (the oracle raises for it), others agree
    g1 = walk(tr, max_depth=1)
    for b in ok:
        want = -1 if ref.accept_len[b] >= 2 else int(ref.accept_len[b])
        assert int(g1.accept_len[b]) == want, b


def test_walk_several_launches_dirty_workspace():
    sv = _sv()
    tr = synth.tree_inputs(14, B=70, n_nodes=7, depth=3, V=128256, dtype="bf16", p_boost=0.9)
    need = int(sv.lib().spec_verify_tree_greedy_workspace_size(70, 8, 128256, 1))
    buf = torch.randint(0, 255, (need + 512,), dtype=torch.uint8, device=dev())
    g = walk(tr, workspace_buf=buf)
    ref = oracle.verify_tree_greedy(tr.target, tr.dtype, tr.parent, tr.node_token, tr.max_depth)
    assert np.array_equal(g.tokens.cpu().numpy(), ref.tokens)
    assert np.array_equal(g.path_nodes.cpu().numpy(), ref.path_nodes)


def test_walk_graph_replays_match_eager_calls():
    sv = _sv()
    trs = [synth.tree_inputs(50 + s, B=6, n_nodes=20, depth=4, V=30000, dtype="bf16", p_boost=0.9) for s in range(3)]
    args = [[logits_to_device(t.target, "bf16"), i32(t.parent), i32(t.node_token)] for t in trs]
    static = [t.clone() for t in args[0]]
    B, D1 = 6, trs[0].max_depth + 1
    out = sv.TreeResult(torch.empty(B, dtype=torch.int32, device=dev()),
                        torch.empty((B, D1), dtype=torch.int32, device=dev()),
                        torch.empty((B, D1), dtype=torch.int32, device=dev()), None)
    ws = torch.empty(int(sv.lib().spec_verify_tree_greedy_workspace_size(B, 21, 30000, 1)) + 256,
                     dtype=torch.uint8, device=dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sv.spec_verify_tree_greedy(*static, trs[0].max_depth, want_argmax=False, out=out, workspace_buf=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.spec_verify_tree_greedy(*static, trs[0].max_depth, want_argmax=False, out=out, workspace_buf=ws)
    torch.cuda.synchronize()
    for rep in range(6):
        k = (rep + 1) % 3
        for dst, src in zip(static, args[k]):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.verify_tree_greedy(trs[k].target, "bf16", trs[k].parent, trs[k].node_token, trs[k].max_depth)
        log(f"[tree walk] graph replay {rep}: input set {k}")
        assert np.array_equal(out.tokens.cpu().numpy(), ref.tokens)
        assert np.array_equal(out.path_nodes.cpu().numpy(), ref.path_nodes)


def test_wait_that_gives_up_flags_every_walk():
    # With a poll limit of 0 every hand-over wait of the walk gives up before its first poll
    # (forced from the host; every workgroup still exits): each sequence is flagged -2 by
    # the one workgroup that writes its outputs, with -1 tokens and path nodes.  The design
    # that computes every row's argmax does not hand anything over and is unaffected; with
    # the default limit restored the walk matches the oracle again.
    sv = _sv()
    tr = synth.tree_inputs(11, B=10, n_nodes=20, depth=4, V=40000, dtype="bf16", p_boost=0.9)
    with sv.knob(sv.SPEC_KNOB_POLL_LIMIT, 0):
        g = walk(tr)
        full = walk(tr, want_argmax=True)
    assert (g.accept_len.cpu().numpy() == sv.FLAG_TIMED_OUT).all()
    assert (g.tokens.cpu().numpy() == -1).all() and (g.path_nodes.cpu().numpy() == -1).all()
    ref = oracle.verify_tree_greedy(tr.target, tr.dtype, tr.parent, tr.node_token, tr.max_depth)
    assert np.array_equal(full.accept_len.cpu().numpy(), ref.accept_len)
    assert np.array_equal(full.tokens.cpu().numpy(), ref.tokens)
    compare(tr)


@pytest.mark.parametrize("B", [32, 13])
def test_xcd_local_hand_overs_change_nothing(B):
    # a launch of a multiple of 8 sequences keeps each sequence's workgroups on one XCD and
    # exchanges the slices through its L2; the results must equal those of agent-scope
    # exchanges and the oracle's
    sv = _sv()
    tr = synth.tree_config_eagle_bf16(50 + B) if B == 32 else synth.tree_inputs(
        51, B=B, n_nodes=30, depth=5, V=128256, dtype="bf16", p_boost=0.9)
    assert sv.spec_get_knob(sv.SPEC_KNOB_XCD_LOCAL) == 1
    g = walk(tr)
    with sv.knob(sv.SPEC_KNOB_XCD_LOCAL, 0):
        h = walk(tr)
    for name in ("accept_len", "tokens", "path_nodes"):
        assert torch.equal(getattr(g, name), getattr(h, name)), name
    ref = oracle.verify_tree_greedy(tr.target, tr.dtype, tr.parent, tr.node_token, tr.max_depth)
    assert np.array_equal(g.tokens.cpu().numpy(), ref.tokens)
    assert np.array_equal(g.path_nodes.cpu().numpy(), ref.path_nodes)
    log(f"[tree walk] XCD-local B={B}: exact; mean accept_len {ref.accept_len.mean():.3f}")
