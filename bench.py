"""Benchmark: batched chain verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu-baseline] [--probe]

One step = one spec_verify_chain call over a batch of B=64 sequences, K=5 drafts,
V=128256 bf16 logits (high-acceptance recipe, T=0.8): the row statistics, accept
tests, first-reject scan, residual/bonus draw and compaction of every sequence.
Inputs are resident in HBM before timing; consecutive steps rotate over several
distinct input sets whose total exceeds twice the 256 MB last-level cache, so
every step streams its logits from HBM.  Before its W warmup calls the headline
workload runs untimed for SETTLE_MS (reported under "settle"), so that the K timed
steps start from the device's steady state.

Prints ONE JSON line (rank 0).  `value` is verified draft positions per second
(B*K per step); `roofline` reports the dominant kernel (chain_fused: the pass that reads
every logit once and the draws, in one launch) against the MI355X HBM peak, with its duration from HIP events
stamped at its own dispatch and completion on its stream (hipExtLaunchKernelGGL), and
against the achievable read rate (pure reads of the same bytes in the same access
shape, timed the same way); `roofline.call` gives the whole call's algorithmic rate, and
`roofline.separate_launches` the same calls with the pass and the draws as separate launches
(the pass alone against the peak: `stats_pass`).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload, on all
the cores of this process's share (worker processes) and on one core.  Secondary
workloads (greedy tree verify, low-acceptance chain, n-gram propose + one-hot verify,
the small fp32 chain) are reported under "other_workloads" unless --quick is given.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# the dominant kernel of a chain call: the fused launch (the pass over every logit and the draws)
# where the call takes it, else the separate statistics pass
ROOF_KERNELS = ("chain_fused", "chain_stats")
LLC_BYTES = 256 * 1024 * 1024


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


STATS_END_MARKER = "// ---------------------------------------------------------------- final draw"


def source_digest(parts) -> str:
    """Digest of the device code a kernel is built from: for each (path, end_marker), the
    file up to the marker line (the whole file when the marker is None)."""
    h = hashlib.sha256()
    for path, marker in parts:
        with open(os.path.join(ROOT, path), "rb") as f:
            text = f.read()
        cut = text.find(marker.encode()) if marker else -1
        h.update(text if cut < 0 else text[:cut])
    return h.hexdigest()[:16]


# the chain_stats kernel: chain.hip up to its draw section, and the shared device helpers; the
# fused kernel: all of chain.hip (it holds the draws too) and the same helpers
KERNEL_SOURCES = {
    "chain_stats": (("draft_token_verification_09_amd/csrc/chain.hip", STATS_END_MARKER),
                    ("draft_token_verification_09_amd/csrc/device_common.h", None)),
    "chain_fused": (("draft_token_verification_09_amd/csrc/chain.hip", None),
                    ("draft_token_verification_09_amd/csrc/device_common.h", None)),
}


def read_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was taken on
    the current kernel source (same digest); otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def sets_needed(bytes_per_set: int) -> int:
    return max(2, -(-2 * LLC_BYTES // bytes_per_set) + 1)


def to_dev(x, dtype, dev):
    import numpy as np
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def chain_device_sets(make, n_sets, dev):
    import numpy as np
    import torch

    sets = []
    host0 = None
    for s in range(n_sets):
        inp = make(s)
        if s == 0:
            host0 = inp
        sets.append(dict(
            t=to_dev(inp.target, inp.dtype, dev),
            d=None if inp.draft is None else to_dev(inp.draft, inp.dtype, dev),
            tok=torch.from_numpy(np.ascontiguousarray(inp.tokens, dtype=np.int32)).to(dev),
            T=torch.from_numpy(inp.temperature).to(dev),
            ua=torch.from_numpy(inp.u_accept).to(dev),
            uf=torch.from_numpy(inp.u_final).to(dev),
            dl=None if inp.draft_len is None else torch.from_numpy(inp.draft_len).to(dev),
        ))
    return sets, host0


def chain_bytes(inp) -> int:
    """Algorithmic bytes of one call: every logit row the method uses read once, plus tokens,
    uniforms, temperatures, draft lengths and the outputs written."""
    import numpy as np

    B, K, V = inp.B, inp.K, inp.V
    es = 2 if inp.dtype == "bf16" else 4
    kb = np.full(B, K) if inp.draft_len is None else np.asarray(inp.draft_len)
    rows = int(np.sum(kb + 1) + (np.sum(kb) if inp.draft is not None else 0))
    small = B * K * 4 * 2 + B * 4 * 2 + (B * 4 if inp.draft_len is not None else 0)
    outs = B * (K + 1) * 4 + B * 4 + B * K * 12
    return rows * V * es + small + outs


def time_calls(call, n_sets, warmup, steps, kernel_timing):
    """Run warmup, then `steps` timed calls rotating over the input sets.  Returns
    (ms per call from events around the whole region, {kernel: (launches, total_ms)})."""
    import torch

    import draft_token_verification_09_amd as sv

    for i in range(warmup):
        call(i % n_sets)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    if kernel_timing:
        sv.spec_timing_reset()
        sv.spec_timing_enable(True)
    torch.cuda.synchronize()
    start.record(stream)
    t_host = time.perf_counter()
    for i in range(steps):
        call((warmup + i) % n_sets)
    t_host = time.perf_counter() - t_host
    stop.record(stream)
    torch.cuda.synchronize()
    time_calls.host_us_per_call = t_host / steps * 1e6
    kernels = {}
    if kernel_timing:
        sv.spec_timing_enable(False)
        for name, launches, ms in sv.spec_timing_collect():
            kernels[name] = (launches, ms)
        sv.spec_timing_reset()
    return start.elapsed_time(stop) / steps, kernels


def time_calls_median(call, n_sets, warmup, steps, passes=3):
    """Median over `passes` timed regions of `steps` calls each (the first after `warmup` calls).
    Used for the secondary workloads, whose latency-bound calls vary with the chip's clock state
    from one region to the next; the headline line times exactly one region."""
    runs = [time_calls(call, n_sets, warmup if i == 0 else 2, steps, False)[0] for i in range(passes)]
    return sorted(runs)[len(runs) // 2]


def bench_chain_workload(make, name, warmup, steps, dev, kernel_timing=True, passes=1, separate=False,
                         settle_ms=0.0):
    """Times `steps` calls of one chain workload (after `warmup`), rotating input sets.  With
    `separate`, the same calls are timed again with the statistics and the draws forced into
    separate launches (SPEC_KNOB_SINGLE_LAUNCH), reported under "separate".  With `settle_ms`,
    the workload first runs untimed for that long (before the warmup calls), so that the timed
    region starts from the device's steady state rather than from the idle state the host-side
    input generation leaves it in."""
    import torch

    import draft_token_verification_09_amd as sv

    probe = make(0)
    per_set = chain_bytes(probe)
    n_sets = sets_needed(per_set)
    progress(f"{name}: generating {n_sets} input sets of {per_set / 1e6:.1f} MB")
    sets, host0 = chain_device_sets(make, n_sets, dev)
    B, K, V = probe.B, probe.K, probe.V
    out = sv.ChainResult(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                         num_accepted=torch.empty((B,), dtype=torch.int32, device=dev),
                         probs=torch.empty((B, K, 3), dtype=torch.float32, device=dev), packed=None, offsets=None)
    code = 1 if probe.dtype == "bf16" else 0
    ws = torch.empty(sv.spec_verify_chain_workspace_size(B, K, V, code) + 256, dtype=torch.uint8, device=dev)

    # one prepared call per input set: arguments are checked and marshalled once, so a step
    # costs the host one foreign call (as in a serving loop that refills fixed buffers)
    prepared = [sv.prepare_spec_verify_chain(s["t"], s["d"], s["tok"], s["T"], s["ua"], s["uf"], s["dl"],
                                             out=out, workspace_buf=ws) for s in sets]

    def call(i):
        prepared[i]()

    settle_calls = 0
    if settle_ms > 0:
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < settle_ms:
            for _ in range(32):
                call(settle_calls % n_sets)
                settle_calls += 1
            torch.cuda.synchronize()
        progress(f"{name}: settled with {settle_calls} untimed calls ({settle_ms:.0f} ms)")
    progress(f"{name}: timing {steps} calls")
    if passes == 1:
        ms, _ = time_calls(call, n_sets, warmup, steps, kernel_timing=False)
    else:
        ms = time_calls_median(call, n_sets, warmup, steps, passes)
    host_us = time_calls.host_us_per_call
    kms = {}
    if kernel_timing:
        _, kms = time_calls(call, n_sets, 2, steps, kernel_timing=True)
    sep = None
    if separate:
        progress(f"{name}: timing {steps} calls as separate launches")
        with sv.knob(sv.SPEC_KNOB_SINGLE_LAUNCH, 1):
            ms_sep, _ = time_calls(call, n_sets, warmup, steps, kernel_timing=False)
            _, kms_sep = time_calls(call, n_sets, 2, steps, kernel_timing=True)
        sep = dict(ms=ms_sep, kernels=kms_sep)
    del sets
    return dict(ms=ms, bytes=per_set, kernels=kms, host=host0, positions=probe.B * probe.K, host_us=host_us,
                steps=steps, separate=sep, settle_calls=settle_calls, settle_ms=settle_ms)


# ---------------------------------------------------------------- CPU baseline (the oracle)
#
# The oracle verifies one sequence at a time.  It is timed in two settings on the host: one
# process on one core, and a pool of worker processes (one per core of this process's CPU
# share, at most CPU_POOL_MAX) that each verify their own sequences of the same input set.
# The pool is forked before the GPU is initialised, with the input set already in memory, so
# the workers share it and never touch the GPU.

CPU_POOL_MAX = 16
_CPU_INPUT = None  # the headline's input set 0, set before the pool forks


def cpu_pool_size() -> int:
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = os.cpu_count() or 1
    return max(1, min(share, CPU_POOL_MAX, int(os.environ.get("OMP_NUM_THREADS", CPU_POOL_MAX))))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_loop(first: int, step: int, budget_s: float):
    """Verify sequences first, first + step, ... of the input set (cycling) for budget_s seconds."""
    import oracle

    inp = _CPU_INPUT
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < budget_s:
        oracle.verify_chain(inp.target, inp.draft, inp.dtype, inp.tokens, inp.temperature, inp.u_accept, inp.u_final,
                            draft_len=inp.draft_len, seqs=[(first + done * step) % inp.B])
        done += 1
    return done, time.perf_counter() - t0


def _oracle_worker(args):
    return _oracle_loop(*args)


def start_cpu_pool(host_inp):
    """Fork the worker pool (before any GPU work) with the input set in memory."""
    import multiprocessing as mp

    global _CPU_INPUT
    _CPU_INPUT = host_inp
    n = cpu_pool_size()
    return mp.get_context("fork").Pool(n), n


def cpu_baseline(pool, workers: int, one_core_s=12.0, pool_s=8.0):
    """The oracle, as it stands, on a bounded sample of sequences of the headline workload."""
    inp = _CPU_INPUT
    done1, dt1 = _oracle_loop(0, 1, one_core_s)
    res = pool.map(_oracle_worker, [(w, workers, pool_s) for w in range(workers)])
    done_all = sum(d for d, _ in res)
    dt_all = max(t for _, t in res)
    shape = f"K={inp.K}, V={inp.V}, {inp.dtype}"
    return dict(
        value=done_all * inp.K / dt_all, unit="positions/s", cores=workers, kind="oracle",
        sample=f"{done_all} sequence verifications in {dt_all:.1f} s by {workers} worker processes, each cycling "
               f"over its own sequences of the {inp.B} of input set 0 ({shape}); float64 NumPy, one thread each",
        cpu_model=cpu_model(), host_cpus=os.cpu_count(),
        one_core=dict(value=done1 * inp.K / dt1, cores=1,
                      sample=f"{done1} sequence verifications cycling over the {inp.B} sequences in {dt1:.1f} s, "
                             f"one process on one thread"))


def other_workloads(warmup, steps, dev):
    import numpy as np
    import torch

    import draft_token_verification_09_amd as sv
    import synth

    out = []
    # chain, low acceptance, B=256 K=8 V=152064 bf16
    r = bench_chain_workload(lambda s: synth.chain_config_low_accept_bf16(s), "chain_B256_K8_V152064_bf16",
                             warmup, steps, dev, passes=3)
    out.append(_entry("chain_verify_B256_K8_V152064_bf16_low_accept", r, r["positions"]))
    # greedy chain (temperature 0): B=64 K=5 V=128256 bf16, target rows only
    def greedy(s):
        inp = synth.chain_config_high_accept_bf16(s)
        inp.draft = None  # a greedy sequence reads no draft row
        inp.temperature = np.zeros_like(inp.temperature)
        return inp

    r = bench_chain_workload(greedy, "chain_greedy_B64_K5_V128256_bf16", warmup, steps, dev, passes=3)
    out.append(_entry("chain_greedy_B64_K5_V128256_bf16", r, r["positions"]))
    # small fp32 chain: latency
    r = bench_chain_workload(lambda s: synth.chain_config_small_f32(s), "chain_B1_K5_V32000_f32", warmup, steps, dev,
                             passes=3)
    out.append(_entry("chain_verify_B1_K5_V32000_f32", r, r["positions"]))

    # greedy tree, B=32 N=60 V=128256 bf16
    tr0 = synth.tree_config_eagle_bf16(0)
    per = tr0.target.nbytes + tr0.parent.nbytes * 2
    n_sets = sets_needed(per)
    progress(f"tree: generating {n_sets} input sets")
    sets = []
    for s in range(n_sets):
        tr = tr0 if s == 0 else synth.tree_config_eagle_bf16(s)
        sets.append((to_dev(tr.target, "bf16", dev), torch.from_numpy(tr.parent).to(dev),
                     torch.from_numpy(tr.node_token).to(dev)))

    # every node's argmax asked for: every row is streamed once
    prepared = [sv.prepare_spec_verify_tree_greedy(t, p, k, 6) for t, p, k in sets]

    def tcall(i):
        prepared[i]()

    ms = time_calls_median(tcall, n_sets, warmup, steps)
    _, kms = time_calls(tcall, n_sets, 2, steps, True)
    torch.cuda.synchronize()
    tree_parents = [p for _, p, _ in sets]
    tree_paths = [(c.result.path_nodes.clone(), c.result.accept_len.clone()) for c in prepared]
    accepted = [c.result.accept_len.cpu().numpy() for c in prepared]
    del prepared
    tb = per + tr0.B * (7 * 3 + 1 + tr0.N1) * 4
    out.append(_entry("tree_greedy_all_argmax_B32_N60_V128256_bf16", dict(ms=ms, bytes=tb, kernels=kms, steps=steps),
                      tr0.B * (tr0.N1 - 1)))
    # the path, its tokens and its nodes only (the workload's outputs): the walk reads the
    # root's row and the accepted nodes' rows
    prepared = [sv.prepare_spec_verify_tree_greedy(t, p, k, 6, want_argmax=False) for t, p, k in sets]
    ms = time_calls_median(tcall, n_sets, warmup, steps)
    _, kms = time_calls(tcall, n_sets, 2, steps, True)
    walked = int(np.mean([int((a + 1).sum()) for a in accepted])) * tr0.V * 2
    r = _entry("tree_greedy_B32_N60_V128256_bf16", dict(ms=ms, bytes=walked, kernels=kms, steps=steps),
               tr0.B * (tr0.N1 - 1))
    r["rows_read_per_call"] = walked // (tr0.V * 2)
    out.append(r)
    del sets, prepared

    # stochastic tree verification, B=32 N=60 V=128256 bf16, T=0.8
    out.append(tree_sampled_workload(warmup, steps, dev))

    # the steps on either side of tree verification, on the same workload's trees
    out += tree_io_workloads(warmup, steps, dev, tree_parents, tree_paths)

    # adaptive gate (host code): decide + observe for a batch of 64 requests over 16 tenants
    out.append(gate_workload())

    # n-gram propose + one-hot verify, B=128 L=4096 K=5 V=32000 bf16
    progress("ngram: generating inputs")
    n_sets = 11
    sets = []
    for s in range(n_sets):
        pr = synth.ngram_config_prompts(s)
        ctx = torch.from_numpy(pr.context).to(dev)
        cl = torch.from_numpy(pr.context_len).to(dev)
        g = sv.ngram_propose(ctx, cl, 1, 4, 5)
        torch.cuda.synchronize()
        inp = synth.ngram_target_inputs(s, g.draft_tokens.cpu().numpy(), g.draft_len.cpu().numpy(), V=32000)
        sets.append(dict(ctx=ctx, cl=cl, t=to_dev(inp.target, "bf16", dev), T=torch.from_numpy(inp.temperature).to(dev),
                         ua=torch.from_numpy(inp.u_accept).to(dev), uf=torch.from_numpy(inp.u_final).to(dev),
                         bytes=chain_bytes(inp) + pr.context.nbytes + pr.context_len.nbytes))

    nb = int(np.mean([s["bytes"] for s in sets]))
    # one call: the lookup runs beside the row statistics of every target row (all K+1 rows are
    # read, since the draft lengths are not known when the streaming starts)
    fused = [sv.prepare_spec_ngram_verify(s["ctx"], s["cl"], 1, 4, s["t"], s["T"], s["ua"], s["uf"]) for s in sets]

    def fcall(i):
        fused[i]()

    ms = time_calls_median(fcall, n_sets, warmup, steps)
    _, kms = time_calls(fcall, n_sets, 2, steps, True)
    r = _entry("ngram_propose_verify_B128_L4096_K5_V32000_bf16", dict(ms=ms, bytes=nb, kernels=kms, steps=steps),
               128 * 5)
    r["call"] = "spec_ngram_verify"
    r["rows_streamed_per_call"] = 128 * 6
    out.append(r)
    del fused
    # the same work as two calls: propose, then verify the proposals in place (the verify reads
    # the propose's outputs and streams only the rows up to each draft length)
    pairs = []
    for s in sets:
        pp = sv.prepare_ngram_propose(s["ctx"], s["cl"], 1, 4, 5)
        pv = sv.prepare_spec_verify_chain(s["t"], None, pp.result.draft_tokens, s["T"], s["ua"], s["uf"],
                                          pp.result.draft_len)
        pairs.append((pp, pv))

    def ncall(i):
        pp, pv = pairs[i]
        pp()
        pv()

    ms = time_calls_median(ncall, n_sets, warmup, steps)
    _, kms = time_calls(ncall, n_sets, 2, steps, True)
    del sets
    r = _entry("ngram_propose_then_verify_B128_L4096_K5_V32000_bf16", dict(ms=ms, bytes=nb, kernels=kms, steps=steps),
               128 * 5)
    r["call"] = "ngram_propose + spec_verify_chain"
    out.append(r)
    return out


def tree_sampled_workload(warmup, steps, dev):
    """Stochastic tree verification on the greedy workload's tree shapes with the
    high-acceptance chain recipe per node.  Algorithmic bytes: the rows the walk needs,
    i.e. the target rows of the root and the accepted nodes and the draft rows of those
    of them that have children."""
    import numpy as np
    import torch

    import draft_token_verification_09_amd as sv
    import synth

    x0 = synth.tree_sampled_config_bf16(0)
    per = x0.target.nbytes + x0.draft.nbytes
    n_sets = sets_needed(per)
    progress(f"tree_sampled: generating {n_sets} input sets")
    prepared, moved = [], []
    for s in range(n_sets):
        x = x0 if s == 0 else synth.tree_sampled_config_bf16(s)
        args = (to_dev(x.target, "bf16", dev), to_dev(x.draft, "bf16", dev), torch.from_numpy(x.parent).to(dev),
                torch.from_numpy(x.node_token).to(dev), torch.from_numpy(x.temperature).to(dev),
                torch.from_numpy(x.u_accept).to(dev), torch.from_numpy(x.u_final).to(dev))
        pc = sv.prepare_spec_verify_tree(*args, x.max_depth)
        r = pc()
        torch.cuda.synchronize()
        rows = 0
        nodes = r.path_nodes.cpu().numpy()
        acc = r.accept_len.cpu().numpy()
        for b in range(x.B):
            visited = [0] + [int(v) for v in nodes[b, : max(0, acc[b])]]
            has_kids = set(int(p) for p in x.parent[b, 1:])
            rows += len(visited) + sum(1 for v in visited if v in has_kids)
        moved.append(rows * x.V * 2)
        prepared.append(pc)
        del x

    def call(i):
        prepared[i]()

    ms = time_calls_median(call, n_sets, warmup, steps)
    _, kms = time_calls(call, n_sets, 2, steps, True)
    r = _entry("tree_sampled_B32_N60_V128256_bf16", dict(ms=ms, bytes=int(np.mean(moved)), kernels=kms, steps=steps),
               x0.B * (x0.N1 - 1))
    r["rows_read_per_call"] = int(np.mean(moved)) // (x0.V * 2)
    del prepared
    torch.cuda.empty_cache()
    return r


def tree_io_workloads(warmup, steps, dev, parents, paths):
    """Tree-attention mask of the B=32 (60 nodes + root) trees, and the commit of each
    verified path's cache entries (`paths`: (path_nodes, accept_len) from verification):
    a 70B-class entry per token, 160 planes (80 layers x K, V) of 8 heads x 128 x bf16 =
    2 KiB, i.e. 320 KiB per token."""
    import numpy as np
    import torch

    import draft_token_verification_09_amd as sv

    out = []
    B, N1 = parents[0].shape
    pm = [sv.prepare_spec_tree_mask(p) for p in parents]

    def mcall(i):
        pm[i]()

    ms = time_calls_median(mcall, len(pm), warmup, steps)
    _, kms = time_calls(mcall, len(pm), 2, steps, True)
    mb = B * N1 * 4 * 2 + B * N1 * N1
    out.append(_entry(f"tree_mask_B{B}_N{N1 - 1}", dict(ms=ms, bytes=mb, kernels=kms, steps=steps), B * (N1 - 1)))

    planes, W, L_cap = 160, 1024, 16
    entry = planes * W * 2
    per_set = int(np.mean([int((a + 1).sum().item()) for _, a in paths])) * entry * 2
    n_sets = sets_needed(per_set)
    progress(f"commit: {n_sets} node buffers of {planes * B * N1 * W * 2 / 1e6:.0f} MB")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    prepared, moved = [], []
    clen = (torch.arange(B, dtype=torch.int32, device=dev) * 3) % (L_cap - 7)
    for s in range(n_sets):
        kv = torch.randint(-32768, 32767, (planes, B, N1, W), dtype=torch.int16, device=dev, generator=gen)
        cache = torch.zeros((planes, B, L_cap, W), dtype=torch.int16, device=dev)
        path, acc = paths[s % len(paths)]
        prepared.append(sv.prepare_spec_commit_path(kv, path, acc, clen, cache))
        moved.append(int((acc + 1).sum().item()) * entry * 2 + B * (path.shape[1] + 3) * 4)

    def ccall(i):
        prepared[i]()

    ms = time_calls_median(ccall, n_sets, warmup, steps)
    _, kms = time_calls(ccall, n_sets, 2, steps, True)
    committed = int(np.mean([int((a + 1).sum().item()) for _, a in paths]))
    r = _entry(f"tree_commit_B{B}_N{N1 - 1}_planes{planes}_entry{entry}",
               dict(ms=ms, bytes=int(np.mean(moved)), kernels=kms, steps=steps), committed)
    r["entries_per_call"] = committed
    del prepared
    # context: a plain contiguous copy of the same bytes, rotating over as many buffer pairs
    half = int(np.mean(moved)) // 2 // 16 * 16
    pairs = [(torch.empty(half, dtype=torch.uint8, device=dev), torch.empty(half, dtype=torch.uint8, device=dev))
             for _ in range(n_sets)]

    def pcall(i):
        sv.spec_probe_copy(*pairs[i])

    pms = time_calls_median(pcall, n_sets, warmup, steps)
    r["plain_copy_same_bytes_us"] = round(pms * 1e3, 3)
    out.append(r)
    del pairs
    torch.cuda.empty_cache()
    return out


def gate_workload(B=64, tenants=16, iters=2000):
    """Host time of one gate decision batch plus one outcome batch (no GPU work)."""
    import numpy as np

    import draft_token_verification_09_amd as sv

    rng = np.random.default_rng(0)
    g = sv.SpecGate()
    keys = rng.integers(0, tenants, size=(iters, B)).astype(np.uint64)
    temps = rng.choice([0.0, 0.5, 0.8], size=(iters, B)).astype(np.float32)
    acc = rng.binomial(5, 0.7, size=(iters, B)).astype(np.int32)
    dl = np.full(B, 5, dtype=np.int32)
    t0 = time.perf_counter()
    for i in range(iters):
        g.decide(keys[i], temps[i])
        g.observe(keys[i], acc[i], dl)
    us = (time.perf_counter() - t0) / iters * 1e6
    return dict(workload=f"gate_decide_observe_B{B}_tenants{tenants}_host", us_per_batch=round(us, 2),
                note="host code through the Python binding; no GPU work")


def _entry(workload, r, positions):
    ms = r["ms"]
    return dict(workload=workload, ms_per_call=round(ms, 5), positions_per_s=round(positions / (ms * 1e-3), 1),
                algorithmic_GBps=round(r["bytes"] / (ms * 1e-3) / 1e9, 1),
                frac_of_hbm_peak=round(r["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                kernels_us_per_call=kernels_per_call(r["kernels"], r.get("steps")))


def kernels_per_call(kernels, steps):
    """{kernel: microseconds per call} (summed over the call's launches of that kernel)."""
    if not steps:
        return {k: round(v[1] / v[0] * 1e3, 2) for k, v in kernels.items()}
    return {k: round(v[1] / steps * 1e3, 3) for k, v in kernels.items()}


MODE_NAMES = {1: "residual", 2: "bonus", 3: "one-hot", 4: "fallback-p", 5: "greedy", 0: "invalid"}


def chain_phases(make, name, warmup, calls, dev, chunk_vectors, pool_segments):
    """Per-phase timeline of chain calls from the library's phase timestamps (device clock,
    100 MHz): for each of `calls` calls (after `warmup`), the stats pass's span and the pool
    kernel's phases, relative to the first stats workgroup's start.  The calls run as separate
    launches (whose stamp layout this reads).  Returns a text summary."""
    import numpy as np
    import torch

    import draft_token_verification_09_amd as sv

    single = sv.spec_get_knob(sv.SPEC_KNOB_SINGLE_LAUNCH)
    sv.spec_set_knob(sv.SPEC_KNOB_SINGLE_LAUNCH, 1)
    probe = make(0)
    per_set = chain_bytes(probe)
    n_sets = sets_needed(per_set)
    sets, _ = chain_device_sets(make, n_sets, dev)
    B, K, V = probe.B, probe.K, probe.V
    if chunk_vectors is None:  # the library's own choice, read back from its chunk rule's inputs
        epv = 8 if probe.dtype == "bf16" else 4
        vec = (V * (2 if probe.dtype == "bf16" else 4)) % 16 == 0
        rows = B * (2 * K + 1 if probe.draft is not None else K + 1)
        chunk_vectors = library_chunk_vectors(rows, V, epv, vec)
    code = 1 if probe.dtype == "bf16" else 0
    ws = torch.empty(sv.spec_verify_chain_workspace_size(B, K, V, code) + 256, dtype=torch.uint8, device=dev)
    prepared = [sv.prepare_spec_verify_chain(s["t"], s["d"], s["tok"], s["T"], s["ua"], s["uf"], s["dl"],
                                             workspace_buf=ws) for s in sets]
    epv = 8 if probe.dtype == "bf16" else 4
    C = -(-V // (chunk_vectors * 256 * epv))
    R = 2 * K + 1 if probe.draft is not None else K + 1
    S = -(-(-(-V // (256 * epv))) // pool_segments) * pool_segments
    G, P = B * R * C, B * (S // pool_segments if probe.draft is not None else 1)
    buf = torch.zeros(2 * G + 6 * P, dtype=torch.int64, device=dev)
    for i in range(warmup):
        prepared[i % n_sets]()
    torch.cuda.synchronize()
    rows = []
    us = 0.01  # microseconds per clock tick
    for i in range(calls):
        buf.fill_(-1)
        torch.cuda.synchronize()
        sv.spec_chain_phase_stamps(buf)
        prepared[(warmup + i) % n_sets]()
        torch.cuda.synchronize()
        sv.spec_chain_phase_stamps(None)
        st = buf.cpu().numpy()
        stats = st[: 2 * G].reshape(G, 2)
        pool = st[2 * G:].reshape(P, 6)
        # every stats workgroup and pool task stamps its start and end (else the layout is not the call's)
        assert (stats != -1).all() and (pool[:, [0, 1, 4, 5]] != -1).all(), "stamp layout does not match the call"
        t0 = stats[:, 0].min()
        r = dict(stats_end=(stats[:, 1].max() - t0) * us, pool_start=(pool[:, 0].min() - t0) * us,
                 decide=np.median(pool[:, 1] - pool[:, 0]) * us,
                 call_end=(pool[:, 4].max() - t0) * us)
        mode = pool[:, 5] & 0xFF
        c = (pool[:, 5] >> 8) & 0xFFFFFF
        res = mode == 1
        last = res & (c == (S // pool_segments if probe.draft is not None else 1) - 1)
        if res.any():
            r["residual_sequences"] = int(last.sum())
            r["published"] = np.median(pool[res, 2] - pool[res, 1]) * us
            r["wait"] = np.median(pool[last, 3] - pool[last, 2]) * us
            r["wait_after_last_published"] = np.median(
                [(pool[last][j, 3] - pool[res & ((pool[:, 5] >> 32) == (pool[last][j, 5] >> 32)), 2].max()) * us
                 for j in range(int(last.sum()))])
            r["narrow"] = np.median(pool[last, 4] - pool[last, 3]) * us
        direct = (mode == 2) | (mode == 3) | (mode == 4)
        first = direct & (c == 0)
        if first.any():
            r["direct_sequences"] = int(first.sum())
            r["direct_select"] = np.median(pool[first, 2] - pool[first, 1]) * us
            r["direct_narrow"] = np.median(pool[first, 4] - pool[first, 2]) * us
        rows.append(r)
    sv.spec_set_knob(sv.SPEC_KNOB_SINGLE_LAUNCH, single)
    del prepared, sets
    torch.cuda.empty_cache()
    keys = ["stats_end", "pool_start", "decide", "published", "wait", "wait_after_last_published", "narrow",
            "direct_select", "direct_narrow", "call_end", "residual_sequences", "direct_sequences"]
    lines = [f"{name}: {calls} calls after {warmup}, medians over the calls (each call: median over its tasks)"]
    for k in keys:
        vals = [r[k] for r in rows if k in r]
        if vals:
            lines.append(f"  {k:28s} {np.median(vals):8.2f}   (min {np.min(vals):.2f}, max {np.max(vals):.2f})")
    return "\n".join(lines)


def chain_phases_single(make, name, warmup, calls, dev):
    """Per-phase timeline of chain calls that run as one launch (the single-launch stamp layout:
    six words per workgroup of the sequences, B x (K+1) x C of them, C from 4-vector chunks):
    medians over the calls of the latest partials published, the median and latest gather, the
    median decision, draw located and end, relative to the first workgroup's start, and the last
    workgroup's end (the call's device time).  Returns a text summary."""
    import numpy as np
    import torch

    import draft_token_verification_09_amd as sv

    sets = []
    probe = make(0)
    for s in range(6):
        inp = probe if s == 0 else make(s)
        t = to_dev(inp.target, inp.dtype, dev)
        d = None if inp.draft is None else to_dev(inp.draft, inp.dtype, dev)
        f = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        sets.append(sv.prepare_spec_verify_chain(t, d, f(inp.tokens), f(inp.temperature), f(inp.u_accept),
                                                 f(inp.u_final)))
    epv = 8 if probe.dtype == "bf16" else 4
    C = -(-probe.V // (4 * 256 * epv))
    nw = probe.B * (probe.K + 1) * C
    buf = torch.full((6 * nw,), -1, dtype=torch.int64, device=dev)
    for i in range(warmup):
        sets[i % len(sets)]()
    torch.cuda.synchronize()
    keys = ["published_last", "gathered_median", "gathered_last", "decided_median", "located_median", "end_last"]
    vals = {k: [] for k in keys}
    for i in range(calls):
        buf.fill_(-1)
        torch.cuda.synchronize()
        sv.spec_chain_phase_stamps(buf)
        sv.spec_timing_reset()
        sv.spec_timing_enable(True)
        sets[(warmup + i) % len(sets)]()
        torch.cuda.synchronize()
        sv.spec_timing_enable(False)
        sv.spec_chain_phase_stamps(None)
        assert "chain_single" in [k for k, _, _ in sv.spec_timing_collect()], "the call did not run as one launch"
        st = buf.cpu().numpy().reshape(nw, 6).astype(np.float64)
        live = st[:, 0] >= 0
        r = (st - st[live, 0].min()) * 0.01  # 100 MHz ticks -> us
        r[st < 0] = np.nan
        vals["published_last"].append(np.nanmax(r[:, 1]))
        vals["gathered_median"].append(np.nanmedian(r[:, 2]))
        vals["gathered_last"].append(np.nanmax(r[:, 2]))
        vals["decided_median"].append(np.nanmedian(r[:, 3]))
        if np.isfinite(r[:, 4]).any():
            vals["located_median"].append(np.nanmedian(r[:, 4]))
        vals["end_last"].append(np.nanmax(r[:, 5]))
    sv.spec_timing_reset()
    lines = [f"{name}: one launch, {nw} workgroups (4-vector chunks, C = {C}); {calls} calls after {warmup}; "
             "us from the first workgroup's start, medians over the calls"]
    for k in keys:
        v = vals[k]
        if v:
            lines.append(f"  {k:28s} {np.median(v):8.2f}   (min {np.min(v):.2f}, max {np.max(v):.2f})")
    return "\n".join(lines)


def chain_phases_fused(make, name, warmup, calls, dev):
    """Per-phase timeline of chain calls that run as the fused launch (its stamp layout: two words
    per stats chunk in sequence/row/chunk order, four per sequence's finisher, seven per helper):
    per call, the pass's end (the last chunk's partials published) and, for the sequence that
    ends last, its own last chunk, its finisher's gather and decision, the last of its helpers to
    see the decision, to publish its masses and to locate the draw, and the draw's end; then the
    medians over the call's residual draws of each step's duration, and the spread of the eight
    XCDs' pass ends, and the last workgroup's exit.  us from the first stats workgroup's start,
    medians over the calls.  Returns
    a text summary."""
    import numpy as np
    import torch

    import draft_token_verification_09_amd as sv

    probe = make(0)
    per_set = chain_bytes(probe)
    n_sets = sets_needed(per_set)
    sets, _ = chain_device_sets(make, n_sets, dev)
    B, K, V = probe.B, probe.K, probe.V
    epv = 8 if probe.dtype == "bf16" else 4
    vec = (V * (2 if probe.dtype == "bf16" else 4)) % 16 == 0
    has_d = probe.draft is not None
    R = 2 * K + 1 if has_d else K + 1  # rows of a sequence in the stats grid
    S = -(-(-(-V // (256 * epv))) // 4) * 4
    CP = S // 4 if has_d else 1
    nv = library_chunk_vectors(B * R, V, epv, vec)
    if nv == 16 and R * -(-V // (8 * 256 * epv)) * 4 <= 512 and B * CP <= 2048:
        nv = 8  # the fused launch streams 32 KiB chunks where its partials fit
    C = -(-V // (nv * 256 * epv))
    G = B * R * C
    code = 1 if probe.dtype == "bf16" else 0
    ws = torch.empty(sv.spec_verify_chain_workspace_size(B, K, V, code) + 256, dtype=torch.uint8, device=dev)
    prepared = [sv.prepare_spec_verify_chain(s["t"], s["d"], s["tok"], s["T"], s["ua"], s["uf"], s["dl"],
                                             workspace_buf=ws) for s in sets]
    buf = torch.zeros(2 * G + 4 * B + 7 * B * CP, dtype=torch.int64, device=dev)
    for i in range(warmup):
        prepared[i % n_sets]()
    torch.cuda.synchronize()
    us = 0.01
    rows = []
    for i in range(calls):
        buf.fill_(-1)
        torch.cuda.synchronize()
        sv.spec_chain_phase_stamps(buf)
        sv.spec_timing_reset()
        sv.spec_timing_enable(True)
        prepared[(warmup + i) % n_sets]()
        torch.cuda.synchronize()
        sv.spec_timing_enable(False)
        sv.spec_chain_phase_stamps(None)
        assert "chain_fused" in [k for k, _, _ in sv.spec_timing_collect()], "the call did not run as the fused launch"
        st = buf.cpu().numpy().astype(np.float64)
        stats = st[: 2 * G].reshape(G, 2)
        fin = st[2 * G: 2 * G + 4 * B].reshape(B, 4)
        hlp = st[2 * G + 4 * B:].reshape(B, CP, 7)
        t0 = stats[stats[:, 0] >= 0, 0].min()
        rel = lambda x: np.where(x >= 0, (x - t0) * us, np.nan)
        s_end = rel(stats[:, 1]).reshape(B, R * C)
        seq_stats_end = np.nanmax(s_end, axis=1)
        f_g, f_d, f_e = rel(fin[:, 0]), rel(fin[:, 1]), rel(fin[:, 2])
        mode = fin[:, 3]
        seen, pub, loc, nar, ext = (rel(hlp[:, :, j]) for j in (1, 2, 3, 4, 5))
        res = mode == 1
        with np.errstate(all="ignore"):
            import warnings
            warnings.simplefilter("ignore", RuntimeWarning)
            seq_end = np.where(res, np.nanmax(nar, axis=1), f_e)
            crit = int(np.nanargmax(seq_end))
            r = dict(pass_end=np.nanmax(s_end), call_end=np.nanmax(seq_end), crit_stats_end=seq_stats_end[crit],
                     crit_gathered=f_g[crit], crit_decided=f_d[crit])
            if res[crit]:
                r.update(crit_seen_last=np.nanmax(seen[crit]), crit_published_last=np.nanmax(pub[crit]),
                         crit_located_last=np.nanmax(loc[crit]))
            r["crit_end"] = seq_end[crit]
            r["last_exit"] = max(np.nanmax(ext), np.nanmax(f_e))
            r["gather"] = np.nanmedian(f_g - seq_stats_end)
            r["decide"] = np.nanmedian(f_d - f_g)
            if res.any():
                sl, pl, ll = np.nanmax(seen[res], axis=1), np.nanmax(pub[res], axis=1), np.nanmax(loc[res], axis=1)
                r["hand_over"] = np.nanmedian(sl - f_d[res])
                r["masses"] = np.nanmedian(pl - sl)
                r["locate"] = np.nanmedian(ll - pl)
                r["narrow"] = np.nanmedian(np.nanmax(nar[res], axis=1) - ll)
                r["residual_sequences"] = int(res.sum())
            if G % 8 == 0:
                xe = [np.nanmax(s_end.reshape(-1)[x * (G // 8):(x + 1) * (G // 8)]) for x in range(8)]
                r["xcd_pass_end_spread"] = max(xe) - min(xe)
        rows.append(r)
    sv.spec_timing_reset()
    del prepared, sets
    torch.cuda.empty_cache()
    keys = ["pass_end", "crit_stats_end", "crit_gathered", "crit_decided", "crit_seen_last", "crit_published_last",
            "crit_located_last", "crit_end", "call_end", "last_exit", "gather", "decide", "hand_over", "masses", "locate", "narrow",
            "residual_sequences", "xcd_pass_end_spread"]
    lines = [f"{name}: fused launch, {G} stats workgroups ({C} chunks a row), {B * CP} helpers; {calls} calls after "
             f"{warmup}; us from the first stats workgroup's start, medians over the calls"]
    for k in keys:
        vals = [r[k] for r in rows if k in r and np.isfinite(r[k])]
        if vals:
            lines.append(f"  {k:28s} {np.median(vals):8.2f}   (min {np.min(vals):.2f}, max {np.max(vals):.2f})")
    return "\n".join(lines)


def library_chunk_vectors(rows, V, epv, vec, max_chunks=16):
    """The chain stats pass's chunk rule (vectors per lane in one chunk), restated for laying out
    the phase timestamps: the largest chunk giving at least 1024 workgroups with at most
    max_chunks chunks a row, else the smallest within that bound but not under 4 vectors."""
    top = 16 if vec and epv == 8 else 8
    pick = 0
    nv = top
    while nv >= 1:
        chunks = -(-V // (nv * 256 * epv))
        if chunks > max_chunks:
            break
        pick = nv
        if rows * chunks >= 1024:
            return nv
        nv //= 2
    return (4 if pick < 4 else pick) if pick else top


def achievable_read(dev, nbytes, warmup, steps):
    """The achievable read rate the streaming pass is compared with: pure reads of the same bytes
    in its access shape (one workgroup per chunk, XCD-blocked, non-temporal 16-byte loads), for
    chunks of 16, 32 and 64 KiB, back to back over rotating buffers that exceed the last-level
    cache, each launch timed by events stamped at its own dispatch and completion (as the
    stats kernel is).  Returns (best GB/s, {chunk KiB: GB/s}, bytes per launch)."""
    import torch

    import draft_token_verification_09_amd as sv

    per = nbytes // 65536 * 65536
    n_sets = sets_needed(per)
    bufs = [torch.empty(per, dtype=torch.uint8, device=dev).random_(0, 255) for _ in range(n_sets)]
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    rates = {}
    for chunk in (16384, 32768, 65536):
        def call(i, chunk=chunk):
            sv.spec_probe_read(bufs[i], out, chunk)

        _, k = time_calls(call, n_sets, warmup, steps, kernel_timing=True)
        launches, ms = k["probe_read"]
        rates[chunk // 1024] = round(per / (ms / launches * 1e-3) / 1e9, 1)
    del bufs
    torch.cuda.empty_cache()
    return max(rates.values()), rates, per


def probe(dev, nbytes=1 << 30):
    """Streaming read and copy probes over `nbytes` (calibration for counters and roofline)."""
    import torch

    import draft_token_verification_09_amd as sv

    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).uniform_()
    dst = torch.empty_like(src)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    for name, fn in (("probe_read", lambda: sv.spec_probe_read(src, out, 65536)),
                     ("probe_copy", lambda: sv.spec_probe_copy(src, dst))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 10
        moved = nbytes * (2 if name == "probe_copy" else 1)
        res[name] = dict(bytes_per_launch=moved, ms=round(ms, 4), GBps=round(moved / (ms * 1e-3) / 1e9, 1))
    return res


# Untimed running of the headline workload before its warmup calls.  The host-side input generation
# leaves the device idle for seconds; measured on one MI355X with 5 warmup and 20 timed calls
# (B=64, K=5, V=128256 bf16): 40.5 us per call from idle, 40.0 after 10-50 ms of pure reads, 39.2
# after 25 ms and 38.9-39.0 after 50 ms of the workload itself, 38.8-39.0 in later regions.
SETTLE_MS = 50.0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # untimed calls before each timed region: about 200 back-to-back calls (10 ms at the headline
    # shape) bring the chip to its sustained clocks; after 20 the headline step still read ~3 % slower
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe", action="store_true", help="also run the streaming read/copy probes")
    ap.add_argument("--phases", metavar="FILE", help="write a per-phase timeline of chain calls (the library's "
                    "phase timestamps) to FILE: the headline, low-acceptance, B=1 fp32 and one-hot workloads as "
                    "separate launches, and small batches as single launches")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the verification path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}); sequences shard across GPUs "
              f"without communication, so run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    import synth

    # the headline's input set 0, generated before any GPU work so that the CPU baseline's
    # worker pool can be forked with it in memory (forking after the GPU is initialised is not)
    progress("generating input set 0 of the headline workload")
    host0 = synth.chain_config_high_accept_bf16(0)
    pool = None
    if not args.no_cpu_baseline:
        pool, workers = start_cpu_pool(host0)

    import torch

    import draft_token_verification_09_amd as sv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sv.lib()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    progress(f"device {torch.cuda.get_device_name(dev)}")

    workload = "chain_verify_B64_K5_V128256_bf16_high_accept"
    head = bench_chain_workload(lambda s: host0 if s == 0 else synth.chain_config_high_accept_bf16(s), workload,
                                args.warmup, args.steps, dev, separate=True, settle_ms=SETTLE_MS)
    ms = head["ms"]
    B, K, V = 64, 5, 128256
    positions = B * K
    logits_bytes = B * (2 * K + 1) * V * 2
    roof_kernel = next((k for k in ROOF_KERNELS if k in head["kernels"]), ROOF_KERNELS[-1])
    launches, kernel_ms = head["kernels"].get(roof_kernel, (1, float("nan")))
    achieved = logits_bytes / (kernel_ms / launches * 1e-3) / 1e9
    traffic = read_traffic(roof_kernel, "B64_K5_V128256_bf16", source_digest(KERNEL_SOURCES[roof_kernel]))
    progress("achievable read rate (pure reads in the stats pass's access shape)")
    achievable, by_chunk, probe_bytes = achievable_read(dev, logits_bytes, args.warmup, args.steps)
    call_bytes = head["bytes"]
    sep = head["separate"]
    s_launches, s_ms = sep["kernels"].get("chain_stats", (1, float("nan")))
    s_achieved = logits_bytes / (s_ms / s_launches * 1e-3) / 1e9

    result = {
        "metric": "verified draft positions/sec and achieved HBM GB/s (% of peak), 1 MI355X",
        "value": round(positions / (ms * 1e-3), 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox): target N(0,3^2) + 20 peaks at +8 per row, draft = target + N(0,0.7^2), "
                "drafts sampled from q, T=0.8",
        "config": {"workload": workload, "B": B, "K": K, "V": V, "temperature": 0.8,
                   "input_sets_rotated": sets_needed(head["bytes"]), "parallelism": "single GPU"},
        "achieved_GBps_step": round(head["bytes"] / (ms * 1e-3) / 1e9, 1),
        "kernels_us_per_call": kernels_per_call(head["kernels"], args.steps),
        "host_issue_us_per_step": round(head["host_us"], 2),
        "settle": {"ms": head["settle_ms"], "calls": head["settle_calls"],
                   "note": "untimed calls of the same workload before the warmup calls, so that the timed region "
                           "starts from the device's steady state"},
        "roofline": {
            "bound": "hbm",
            "kernel": roof_kernel,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": logits_bytes,
            "achievable": achievable,
            "frac_of_achievable": round(achieved / achievable, 4),
            "achievable_probe": {"kernel": "probe_read", "bytes_per_launch": probe_bytes, "GBps_by_chunk_KiB": by_chunk},
            "call": {"achieved": round(call_bytes / (ms * 1e-3) / 1e9, 1),
                     "frac": round(call_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "frac_of_achievable": round(call_bytes / (ms * 1e-3) / 1e9 / achievable, 4),
                     "algorithmic_bytes_per_call": call_bytes},
            # the same calls with the statistics pass and the draws as separate launches: the
            # pass over every logit on its own, and the call it makes
            "separate_launches": {
                "ms_per_step": round(sep["ms"], 5),
                "kernels_us_per_call": kernels_per_call(sep["kernels"], args.steps),
                "stats_pass": {"kernel": "chain_stats", "achieved": round(s_achieved, 1),
                               "frac": round(s_achieved / HBM_PEAK_GBPS, 4),
                               "frac_of_achievable": round(s_achieved / achievable, 4)},
            },
        },
    }
    if pool is not None:
        progress(f"cpu baseline (oracle on a bounded sample, 1 and {workers} cores)")
        result["cpu_baseline"] = cpu_baseline(pool, workers)
        pool.close()
        pool.join()
    if not args.quick:
        result["other_workloads"] = other_workloads(args.warmup, max(20, args.steps // 2), dev)
    if args.probe:
        result["probes"] = probe(dev)
    if args.phases:
        progress("phase timestamps")
        def one_hot(s):
            inp = synth.chain_config_high_accept_bf16(s, B=128, V=32000)
            inp.draft = None
            return inp

        text = ["the default path at the benchmarked shape (one fused launch):",
                chain_phases_fused(lambda s: host0 if s == 0 else synth.chain_config_high_accept_bf16(s), workload,
                                   args.warmup, 20, dev),
                "separate launches (stats pass, then pool kernel):",
                chain_phases(lambda s: host0 if s == 0 else synth.chain_config_high_accept_bf16(s), workload,
                             args.warmup, 20, dev, None, 4),
                chain_phases(lambda s: synth.chain_config_low_accept_bf16(s), "chain_verify_B256_K8_V152064_bf16",
                             args.warmup, 20, dev, None, 4),
                chain_phases(lambda s: synth.chain_config_small_f32(s), "chain_verify_B1_K5_V32000_f32",
                             args.warmup, 20, dev, None, 4),
                chain_phases(one_hot, "chain_verify_one_hot_B128_K5_V32000_bf16", args.warmup, 20, dev, None, 4)]

        def one_hot16(s):
            inp = synth.chain_config_high_accept_bf16(s, B=16, V=32000)
            inp.draft = None
            return inp

        text += ["single launches (the calls' default path at these shapes):",
                 chain_phases_single(lambda s: synth.chain_config_small_f32(s), "chain_verify_B1_K5_V32000_f32",
                                     args.warmup, 20, dev),
                 chain_phases_single(lambda s: synth.chain_config_high_accept_bf16(s, B=8, V=32000),
                                     "chain_verify_B8_K5_V32000_bf16", args.warmup, 20, dev),
                 chain_phases_single(one_hot16, "chain_verify_one_hot_B16_K5_V32000_bf16", args.warmup, 20, dev)]
        with open(args.phases, "w") as f:
            f.write("\n\n".join(text) + "\n")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
