"""GPU parity of spec_verify_chain against the oracle on the seeded workload recipes."""

import os

import numpy as np
import pytest

import synth
from gpu_helpers import chain_on_gpu, chain_oracle, check_packed, compare_chain, log

pytestmark = pytest.mark.gpu


def _run(inp, seqs=None, packed=True):
    log(f"[chain] {inp.name} B={inp.B} K={inp.K} V={inp.V} dtype={inp.dtype}")
    gpu = chain_on_gpu(inp, want_packed=packed)
    ref = chain_oracle(inp, seqs=seqs)
    rep = compare_chain(gpu, ref, inp, seqs=seqs)
    log(f"[chain]   {rep}")
    assert rep.ok(), rep.failures[:5]
    if packed:
        check_packed(gpu, inp.B)
    return gpu, rep


@pytest.mark.parametrize("seed", range(5))
def test_small_fp32_chain(seed):
    # B=1, K=5, V=32000 fp32: target N(0, 2^2), draft = target + N(0, 1), T = 1
    _run(synth.chain_config_small_f32(seed))


def test_small_fp32_recipe_many_sequences():
    gpu, rep = _run(synth.chain_config_small_f32(7, B=48))
    assert rep.exact >= 46


@pytest.mark.parametrize("V", [128256, 50000, 1000])
def test_high_accept_bf16_reduced_batch(V):
    # B=8 of the high-acceptance bf16 recipe; V=50000 and 1000 leave ragged chunk tails
    _run(synth.chain_config_high_accept_bf16(1, B=8, V=V))


def test_high_accept_bf16_full_size():
    # the benchmarked shape: B=64, K=5, V=128256, bf16, T=0.8; every sequence checked
    _, rep = _run(synth.chain_config_high_accept_bf16(0))
    assert rep.sequences == 64


def test_low_accept_bf16_full_size_sampled():
    # B=256, K=8, V=152064, bf16: the GPU runs the whole batch, the oracle checks 48 sequences
    inp = synth.chain_config_low_accept_bf16(0)
    seqs = list(range(0, 256, 16)) + list(range(1, 256, 8))
    _run(inp, seqs=sorted(set(seqs)))


def test_low_accept_bf16_reduced():
    _run(synth.chain_config_low_accept_bf16(3, B=12, K=8, V=20000))


@pytest.mark.parametrize("nv", ["1", "2", "4", "8"])
def test_chunk_sizes_give_identical_decisions(nv, monkeypatch):
    # every chunk size the library may pick agrees with the oracle (and hence with each other)
    monkeypatch.setenv("SPEC_NV", nv)
    _run(synth.chain_config_high_accept_bf16(5, B=6, K=4, V=40000))
    _run(synth.chain_config_small_f32(5, B=6, K=4, V=9000))


def test_repeat_calls_are_bit_identical():
    inp = synth.chain_config_high_accept_bf16(2, B=16, V=60000)
    a = chain_on_gpu(inp)
    b = chain_on_gpu(inp)
    assert np.array_equal(a.tokens.cpu().numpy(), b.tokens.cpu().numpy())
    assert np.array_equal(a.probs.cpu().numpy(), b.probs.cpu().numpy())
    total = int(a.offsets.cpu()[-1])
    assert int(b.offsets.cpu()[-1]) == total
    assert np.array_equal(a.packed.cpu().numpy()[:total], b.packed.cpu().numpy()[:total])
