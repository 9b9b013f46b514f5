"""GPU parity of spec_verify_tree_greedy and ngram_propose (+ one-hot verify) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import chain_on_gpu, chain_oracle, compare_chain, i32, log, logits_to_device

pytestmark = pytest.mark.gpu


def _tree_gpu(tr):
    import draft_token_verification_09_amd as sv

    res = sv.spec_verify_tree_greedy(logits_to_device(tr.target, tr.dtype), i32(tr.parent), i32(tr.node_token),
                                     tr.max_depth)
    torch.cuda.synchronize()
    return res


def _tree_compare(tr, seqs=None):
    log(f"[tree] {tr.name} B={tr.B} N1={tr.N1} V={tr.V}")
    g = _tree_gpu(tr)
    ref = oracle.verify_tree_greedy(tr.target, tr.dtype, tr.parent, tr.node_token, tr.max_depth, seqs=seqs)
    idx = list(range(tr.B)) if seqs is None else list(seqs)
    assert np.array_equal(g.argmax.cpu().numpy()[idx], ref.argmax[idx])
    assert np.array_equal(g.accept_len.cpu().numpy()[idx], ref.accept_len[idx])
    assert np.array_equal(g.tokens.cpu().numpy()[idx], ref.tokens[idx])
    assert np.array_equal(g.path_nodes.cpu().numpy()[idx], ref.path_nodes[idx])
    log(f"[tree]   exact on {len(idx)} sequences, mean accept_len {ref.accept_len[idx].mean():.3f}")
    return g, ref


def test_tree_eagle_full_size():
    # B=32 trees of 60 nodes (+ root), depth 6, V=128256 bf16; bit-exact
    _tree_compare(synth.tree_config_eagle_bf16(0))


@pytest.mark.parametrize("V", [1000, 77777])
def test_tree_ragged_vocab(V):
    _tree_compare(synth.tree_inputs(4, B=8, n_nodes=30, depth=5, V=V, dtype="bf16"))


def test_tree_fp32_and_ties():
    # small integer logits produce many tied maxima: the smallest index must win
    tr = synth.tree_inputs(9, B=16, n_nodes=40, depth=4, V=3000, dtype="f32")
    tr.target = np.round(tr.target / 3.0).astype(np.float32)
    _tree_compare(tr)


def test_tree_bf16_ties_and_matches():
    tr = synth.tree_inputs(11, B=16, n_nodes=60, depth=6, V=512, dtype="bf16", p_boost=0.95)
    bits = tr.target.copy()
    bits[:, :, ::3] = bits[:, :, 0:1]  # duplicate values across the row: ties everywhere
    tr.target = bits
    _tree_compare(tr)


# ------------------------------------------------------------------------------ n-gram


def _ngram_gpu(ctx, lens, n_min, n_max, K):
    import draft_token_verification_09_amd as sv

    res = sv.ngram_propose(i32(ctx), i32(lens), n_min, n_max, K)
    torch.cuda.synchronize()
    return res


def _ngram_compare(ctx, lens, n_min, n_max, K):
    g = _ngram_gpu(ctx, lens, n_min, n_max, K)
    ref = oracle.ngram_propose(ctx, lens, n_min, n_max, K)
    assert np.array_equal(g.draft_len.cpu().numpy(), ref.draft_len)
    assert np.array_equal(g.match_n.cpu().numpy(), ref.match_n)
    assert np.array_equal(g.draft_tokens.cpu().numpy(), ref.draft)
    return g, ref


def test_ngram_prompts_full_size():
    pr = synth.ngram_config_prompts(0)
    log("[ngram] prompts B=128 L=4096 V=32000")
    _, ref = _ngram_compare(pr.context, pr.context_len, 1, 4, 5)
    log(f"[ngram]   match_n histogram {np.bincount(ref.match_n, minlength=5).tolist()}")


def test_ngram_random_small_contexts():
    rng = np.random.default_rng(5)
    B, L_max = 200, 64
    ctx = rng.integers(0, 4, (B, L_max)).astype(np.int32)
    lens = rng.integers(1, L_max + 1, B).astype(np.int32)
    for n_min, n_max, K in [(1, 4, 5), (2, 3, 1), (1, 16, 64), (3, 3, 7)]:
        _ngram_compare(ctx, lens, n_min, n_max, K)


def test_ngram_variable_lengths_zipf():
    lens = np.random.default_rng(1).integers(1, 4097, 64).astype(np.int32)
    pr = synth.ngram_prompts(2, B=64, L=4096, V=32000, lengths=lens)
    _ngram_compare(pr.context, pr.context_len, 1, 4, 5)


def test_ngram_multi_tile_contexts():
    # contexts longer than one 4096-token shared-memory tile: lengths around the tile ends,
    # Zipf prompts, and unique-token contexts whose only earlier copy of the suffix is planted
    # across a tile boundary
    lens = np.array([1, 2, 5, 4095, 4096, 4097, 4098, 5000, 8191, 8192, 8193, 8194, 9000, 9999, 10000, 7000],
                    np.int32)
    pr = synth.ngram_prompts(4, B=16, L=10000, V=32000, lengths=lens)
    _ngram_compare(pr.context, pr.context_len, 1, 4, 5)
    starts = [4090, 4092, 4093, 4094, 4095, 4096, 8186, 8189, 8190, 8191, 8192, 100]
    B, L_max = len(starts), 10000
    ctx = np.tile(np.arange(L_max, dtype=np.int32) + 7, (B, 1))
    lens = np.full(B, L_max, np.int32)
    for i, p in enumerate(starts):
        n = 2 + i % 3  # planted copy of the last n tokens, straddling the boundary
        ctx[i, p:p + n] = ctx[i, L_max - n:]
    g, ref = _ngram_compare(ctx, lens, 1, 4, 5)
    assert (ref.match_n >= 2).all()


def test_ngram_invalid_length_flagged():
    ctx = np.zeros((3, 8), np.int32)
    # lengths 0 and 9 (> L_max) are flagged; [0, 0, 0, 0] matches n = 3 at j = 0, leaving one token
    g = _ngram_gpu(ctx, np.array([0, 9, 4], np.int32), 1, 4, 3)
    assert g.draft_len.cpu().tolist() == [0, 0, 1]
    assert g.match_n.cpu().tolist() == [-1, -1, 3]
    assert g.draft_tokens.cpu().tolist() == [[-1, -1, -1], [-1, -1, -1], [0, -1, -1]]


def test_ngram_then_one_hot_verify():
    # propose on the GPU, check against the oracle, then verify the proposals with q one-hot
    pr = synth.ngram_config_prompts(3)
    g, ref = _ngram_compare(pr.context, pr.context_len, 1, 4, 5)
    inp = synth.ngram_target_inputs(3, ref.draft, ref.draft_len, V=32000)
    log(f"[ngram] one-hot verify B={inp.B} K={inp.K} V={inp.V}")
    gpu = chain_on_gpu(inp)
    rep = compare_chain(gpu, chain_oracle(inp), inp)
    log(f"[ngram]   {rep}")
    assert rep.ok(), rep.failures[:5]


def test_ngram_device_outputs_feed_verify_directly():
    # the GPU proposal tensors go straight into spec_verify_chain (no host round trip)
    import draft_token_verification_09_amd as sv

    pr = synth.ngram_config_prompts(4, B=32)
    g = _ngram_gpu(pr.context, pr.context_len, 1, 4, 5)
    drafts = g.draft_tokens.cpu().numpy()
    dlen = g.draft_len.cpu().numpy()
    inp = synth.ngram_target_inputs(4, drafts, dlen, V=32000)
    t = logits_to_device(inp.target, "bf16")
    res = sv.spec_verify_chain(t, None, g.draft_tokens, torch.ones(32, device=t.device),
                               torch.from_numpy(inp.u_accept).to(t.device), torch.from_numpy(inp.u_final).to(t.device),
                               g.draft_len)
    ref = chain_oracle(inp)
    torch.cuda.synchronize()
    rep = compare_chain(res, ref, inp)
    assert rep.ok(), rep.failures[:5]


def test_prepared_tree_and_ngram_match_plain_calls():
    import draft_token_verification_09_amd as sv

    tr = synth.tree_inputs(12, B=8, n_nodes=30, depth=5, V=5000, dtype="bf16")
    t, p, k = logits_to_device(tr.target, "bf16"), i32(tr.parent), i32(tr.node_token)
    plain = sv.spec_verify_tree_greedy(t, p, k, tr.max_depth)
    prep = sv.prepare_spec_verify_tree_greedy(t, p, k, tr.max_depth)
    res = prep()
    res = prep()
    torch.cuda.synchronize()
    for name in ("accept_len", "tokens", "path_nodes", "argmax"):
        assert torch.equal(getattr(plain, name), getattr(res, name)), name
    pr = synth.ngram_config_prompts(5, B=16)
    ctx, cl = i32(pr.context), i32(pr.context_len)
    plain = sv.ngram_propose(ctx, cl, 1, 4, 5)
    res = sv.prepare_ngram_propose(ctx, cl, 1, 4, 5)()
    torch.cuda.synchronize()
    for name in ("draft_tokens", "draft_len", "match_n"):
        assert torch.equal(getattr(plain, name), getattr(res, name)), name
