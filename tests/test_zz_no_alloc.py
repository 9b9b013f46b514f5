"""The allocation-free chain entry point (spec_verify_chain_noalloc) against the entry point
with a workspace (spec_verify_chain): identical outputs on two calls in a row, the second with
a smaller input, both also checked against the oracle.  (The refusal of shapes beyond the
scratch array is a host-side check, tested on the CPU in test_abi.py.)"""

import numpy as np
import pytest
import torch

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


def _out(B, K):
    d = torch.device("cuda:0")
    return _sv().ChainResult(tokens=torch.full((B, K + 1), 7, dtype=torch.int32, device=d),
                             num_accepted=torch.full((B,), 7, dtype=torch.int32, device=d),
                             probs=torch.full((B, K, 3), 7.0, dtype=torch.float32, device=d),
                             packed=torch.full((B * (K + 1),), 7, dtype=torch.int32, device=d),
                             offsets=torch.full((B + 1,), 7, dtype=torch.int32, device=d))


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    sv = _sv()
    first = synth.chain_config_high_accept_bf16(31, B=48, K=5, V=60000)
    second = synth.chain_config_low_accept_bf16(32, B=9, K=3, V=20000)  # smaller: reuses the same array
    for inp in (first, second):
        log(f"[noalloc] B={inp.B} K={inp.K} V={inp.V} {inp.dtype}")
        args = _args(inp)
        got = sv.spec_verify_chain_noalloc(*args, out=_out(inp.B, inp.K))
        want = sv.spec_verify_chain(*args, want_packed=True)
        torch.cuda.synchronize()
        for name in ("tokens", "num_accepted", "probs", "offsets"):
            assert torch.equal(getattr(got, name), getattr(want, name)), name
        total = int(want.offsets[-1])
        assert torch.equal(got.packed[:total], want.packed[:total])
        rep = compare_chain(got, chain_oracle(inp), inp)
        log(f"[noalloc]   {rep}")
        assert rep.ok(), rep.failures[:5]
        check_packed(got, inp.B)



def test_noalloc_falls_back_to_separate_launches_when_one_launch_words_do_not_fit():
    # B=2000, K=32, V=2048 bf16: with the one-launch paths' hand-over words the workspace exceeds
    # the 16 MiB scratch array, without them it fits, so the allocation-free call runs the
    # separate launches while spec_verify_chain (with its own workspace) takes the fused launch;
    # the two give the same outputs bit for bit
    sv = _sv()
    B, K, V = 2000, 32, 2048
    assert sv.spec_verify_chain_workspace_size(B, K, V, 1) > 16 << 20
    inp = synth.chain_inputs(33, B=B, K=K, V=V, dtype="bf16", target_sigma=2.0, draft_sigma=1.0, temperature=1.0)
    log(f"[noalloc] fallback B={B} K={K} V={V}")
    args = _args(inp)
    got = sv.spec_verify_chain_noalloc(*args, out=_out(B, K))
    sv.spec_timing_reset()
    sv.spec_timing_enable(True)
    want = sv.spec_verify_chain(*args, want_packed=True)
    torch.cuda.synchronize()
    sv.spec_timing_enable(False)
    names = [n for n, _, _ in sv.spec_timing_collect()]
    sv.spec_timing_reset()
    assert names[0] == "chain_fused", names
    for name in ("tokens", "num_accepted", "probs", "offsets"):
        assert torch.equal(getattr(got, name), getattr(want, name)), name
    total = int(want.offsets[-1])
    assert torch.equal(got.packed[:total], want.packed[:total])
    seqs = list(range(0, B, 97)) + [B - 1]
    rep = compare_chain(got, chain_oracle(inp, seqs=seqs), inp, seqs=seqs)
    log(f"[noalloc]   {rep}")
    assert rep.ok(), rep.failures[:5]
