"""GPU parity of spec_verify_chain on seeded random shapes.

Each case draws its batch size, draft count, vocabulary size (ragged against every chunk,
piece and segment size the library uses), element type, temperature and logit spreads, and
then, at random, variable draft lengths, one-hot drafts (no draft rows) and greedy
(temperature 0) sequences.  Every sequence of every case is checked against the oracle.
"""

import numpy as np
import pytest

import synth
from gpu_helpers import chain_on_gpu, chain_oracle, check_packed, compare_chain, log

pytestmark = pytest.mark.gpu

VOCABS = [1, 7, 100, 1023, 2047, 2048, 2049, 8191, 8193, 16385, 40000, 65537, 100003, 128256]


def _case(i):
    rng = np.random.default_rng(7000 + i)
    B = int(rng.integers(1, 9))
    K = int(rng.integers(1, 9))
    V = int(rng.choice(VOCABS))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    T = float(rng.choice([0.3, 0.8, 1.0, 2.0]))
    inp = synth.chain_inputs(9000 + i, B=B, K=K, V=V, dtype=dtype, target_sigma=float(rng.choice([1.0, 2.0, 3.0])),
                             draft_sigma=float(rng.choice([0.3, 1.0, 3.0])), temperature=T,
                             peaks=int(rng.choice([0, 0, 5])) if V > 10 else 0, peak_shift=6.0, name=f"random{i}")
    if rng.random() < 0.4:
        inp.draft_len = rng.integers(0, K + 1, B).astype(np.int32)
    if rng.random() < 0.3:
        inp.draft = None  # one-hot drafts: alpha = p(x)
    if rng.random() < 0.3:
        inp.temperature = inp.temperature.copy()
        inp.temperature[rng.random(B) < 0.5] = 0.0  # greedy sequences in the batch
    if rng.random() < 0.2:
        inp.u_accept = np.full_like(inp.u_accept, 2.0 ** -24)  # accept whenever alpha > 0: bonus draws
    return inp


@pytest.mark.parametrize("i", range(64))
def test_random_shape(i):
    inp = _case(i)
    kinds = []
    if inp.draft is None:
        kinds.append("one-hot")
    if inp.draft_len is not None:
        kinds.append("variable lengths")
    if (inp.temperature == 0).any():
        kinds.append(f"{int((inp.temperature == 0).sum())} greedy")
    log(f"[random] case {i}: B={inp.B} K={inp.K} V={inp.V} {inp.dtype} T={float(inp.temperature.max()):.1f} "
        f"{', '.join(kinds)}")
    g = chain_on_gpu(inp)
    rep = compare_chain(g, chain_oracle(inp), inp)
    log(f"[random]   {rep}")
    assert rep.ok(), rep.failures[:5]
    assert rep.sequences == inp.B
    check_packed(g, inp.B)


@pytest.mark.parametrize("i", range(16))
def test_random_batch_of_a_multiple_of_8(i):
    # batches of 8 to 64 sequences: the launch shapes that keep each sequence's workgroups on
    # one XCD (single launch, fused launch, pool kernel) and hand over through its L2; every
    # sequence against the oracle, and the same outputs with agent-scope hand-overs
    import draft_token_verification_09_amd as sv
    import torch

    base = _case(100 + i)
    rng = np.random.default_rng(7100 + i)
    B = 8 * int(rng.integers(1, 9))
    V = int(rng.choice([2049, 8193, 16385, 40000, 65537, 128256]))
    inp = synth.chain_inputs(9100 + i, B=B, K=base.K, V=V, dtype=base.dtype, target_sigma=2.0,
                             draft_sigma=float(rng.choice([0.3, 1.0, 3.0])), temperature=float(base.temperature.max()),
                             name=f"random8x{i}")
    if rng.random() < 0.4:
        inp.draft_len = rng.integers(0, base.K + 1, B).astype(np.int32)
    if rng.random() < 0.3:
        inp.draft = None
    log(f"[random] batch case {i}: B={B} K={inp.K} V={V} {inp.dtype} one-hot={inp.draft is None}")
    g = chain_on_gpu(inp)
    rep = compare_chain(g, chain_oracle(inp), inp)
    log(f"[random]   {rep}")
    assert rep.ok(), rep.failures[:5]
    assert rep.sequences == B
    check_packed(g, B)
    with sv.knob(sv.SPEC_KNOB_XCD_LOCAL, 0):
        h = chain_on_gpu(inp)
    torch.cuda.synchronize()
    for name in ("tokens", "num_accepted", "probs", "offsets"):
        assert torch.equal(getattr(g, name), getattr(h, name)), name
    total = int(g.offsets[-1])
    assert torch.equal(g.packed[:total], h.packed[:total])
