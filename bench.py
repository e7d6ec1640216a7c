"""Benchmark: sparse MLA flash attention decode on one MI355X.

Workload (default): B=64 sequences, S1=2 query tokens each (MTP1), 128 query heads over one
latent KV head, 8192 live cache positions per sequence in a 4096-block paged pool (block 128),
top-k = 2048 distinct positions per token, bf16 cache. All inputs are seeded and synthetic.

A step is one sfa_decode call over one batch. Untimed warm-up calls run first (at least --warmup
calls and at least 1 s of calls, so that the GPU clocks have left their idle state). The timed region then runs
--steps calls back to back. It rotates over --sets independent copies of the inputs; each copy has its own physical
block order, so its pool sits at different addresses and the 256 MB MALL cannot hold the
previous call's rows (cold protocol). Inputs are resident in HBM before timing starts.

Prints one JSON line. Extra fields beyond the contract: the per-launch kernel time, gathered
KV GB/s, TFLOP/s and the roofline object for the attention kernel, plus a CPU baseline: the
fp64 oracle on a bounded token sample of the same workload, on this host's cores.

Algorithmic work per call (fixed by the workload, not by the implementation):
  bytes = sum over valid (token, slot) of 1152 (bf16 row: 1024 nope + 128 rope) or 656 (int8:
          512 + 128 + 16 scale bytes), plus per token Q (n_q*576*2) + out (n_q*512*2) + indices
          (4*topk)
  flop  = sum over valid (token, slot) of 2 * n_q * (576 + 512)
The window workloads on 512-wide rows (rotary channels inside the row) count 1024 (bf16) or 528
(int8: 512 + 16) bytes per row, Q at n_q*512*2 and 2 * n_q * (512 + 512) flop per row.
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
METRIC = "µs/call + gathered-KV GB/s & TFLOP/s vs roofline, B=64 S1=2 topk=2048 decode"

WORKLOADS = {
    "tiny_b1_s1_bf16": ("tiny", "bf16", False),
    "decode_b64_s2_bf16": ("decode_mtp1", "bf16", False),
    "decode_b64_s2_int8": ("decode_mtp1_int8", "int8", False),
    "varlen_b32_s1_bf16": ("varlen_decode", "bf16", False),
    "prefill_b1_s4096_bf16": ("prefill", "bf16", True),
}


def algorithmic_work(inp):
    import numpy as np

    valid = int(np.asarray(inp.valid_counts()).sum())
    row = 1152 if inp.kv_dtype == "bf16" else 656
    per_token = inp.n_q * 576 * 2 + inp.n_q * 512 * 2 + 4 * inp.topk
    nbytes = valid * row + inp.n_tokens * per_token
    flop = valid * 2 * inp.n_q * (576 + 512)
    return valid, nbytes, flop


def permuted_copy(dev, inp, seed):
    """A device copy of the inputs with the physical blocks of the pool permuted (and the block
    table remapped): the same attention problem at different addresses."""
    import torch

    n_pool = inp.num_cache_rows // 128
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(n_pool, generator=g).to(dev["key_rope"].device)
    out = dict(dev)
    for key in ("key_nope", "key_rope", "k_nope_scales"):
        t = dev[key]
        if t is None:
            continue
        blocks = t.view(n_pool, 128, -1)
        moved = torch.empty_like(blocks)
        moved[perm] = blocks
        out[key] = moved.view_as(t)
    out["block_table"] = perm.to(torch.int32)[dev["block_table"].long()].contiguous()
    return out


def traffic_from_profile(kernel_src_hash: str, name: str = "sfa_decode_b64_s2_bf16_traffic.txt"):
    """HBM bytes per launch from a committed rocprofv3 PMC summary under profiles/, if it was taken
    on the same kernel source (its recorded hash matches); otherwise None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_src_hash:
        return None
    return float(m_bytes.group(1))


def mfma_from_profile(kernel_src_hash: str, workload: str):
    """MFMA counters of the attention kernel on `workload` from the committed rocprofv3 summary
    profiles/sfa_attention_mfma_utilisation.txt, if it was taken on the same kernel source."""
    path = os.path.join(ROOT, "profiles", "sfa_attention_mfma_utilisation.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    if not m_hash or m_hash.group(1) != kernel_src_hash:
        return None
    out = {}
    for key in ("mfma_flop_per_launch", "mfma_busy_fraction"):
        m = re.search(re.escape(f"{workload}.{key}") + r":\s*([0-9.eE+]+)", txt)
        if not m:
            return None
        out[key] = float(m.group(1))
    return out


def kernel_source_hash(names=("sfa_kernels.hip", "sfa_internal.h")) -> str:
    """sha256 of the kernel sources with their comments removed, so that a profile stays tied to
    the code it measured across edits of comments only."""
    import hashlib

    h = hashlib.sha256()
    for name in names:
        text = open(os.path.join(ROOT, "mla_sparse_top_amd", "csrc", name)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(text.encode())
    return h.hexdigest()


def cpu_baseline(inp, gpu_out, seconds: float):
    """The fp64 oracle on this host, over as many tokens as fit in `seconds`, scaled to a full
    call. Also compares those tokens with the GPU output."""
    import numpy as np

    import oracle.sfa_oracle as O

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    got = gpu_out.float().cpu().numpy().astype(np.float64).reshape(inp.n_tokens, inp.n_q, 512)
    t0 = time.perf_counter()
    done = 0
    worst = 0.0
    fails = 0
    order = np.random.default_rng(0).permutation(inp.n_tokens)
    checked = 0
    # cycle through the tokens (random order) until the time budget is spent; a token's output is
    # compared with the GPU's on its first visit only
    while done == 0 or time.perf_counter() - t0 < seconds:
        t = int(order[done % inp.n_tokens])
        ref = O.sparse_mla_attention(inp, tokens=[t])[0]
        if done < inp.n_tokens:
            rep = O.allclose_report(got[t], ref)
            worst = max(worst, rep["worst_ratio"])
            fails += rep["fails"]
            checked += 1
        done += 1
    el = time.perf_counter() - t0
    us_per_call = el / done * inp.n_tokens * 1e6
    return {
        "value": round(us_per_call, 1), "unit": "us/call", "cores": cores, "kind": "oracle",
        "blas_threads": blas_threads, "numpy": np.__version__,
        "sample": f"{done} token evaluations ({checked} distinct of {inp.n_tokens}, random order, seed 0) in "
                  f"{el:.1f} s, scaled to one call of {inp.n_tokens} tokens",
        "sample_parity": {"tokens": checked, "fails": fails, "worst_err_over_bound": round(worst, 4)},
    }


def warm_up(step, args, torch):
    """Untimed calls before timing: at least --warmup calls (10 when not given) and, in any case,
    calls for at least --warmup-seconds. From idle the GPU needs time to raise its clocks, so a
    short call count alone would time a GPU that is still clocking up. Returns the number of
    calls made."""
    n_min = 10 if args.warmup is None else args.warmup
    n_warm = 0
    t_w = time.perf_counter()
    while n_warm < n_min or time.perf_counter() - t_w < args.warmup_seconds:
        for _ in range(10):
            step(n_warm)
            n_warm += 1
        torch.cuda.synchronize()
    return n_warm


INDEXER_METRIC = "µs/call (index scores + top-k select) vs roofline, B=64 S1=2 kv=8192 topk=2048 indexer"


def bench_indexer(args):
    """The Lightning Indexer step that produces topk_indices: sfa_indexer_scores then
    sfa_topk_select, on the decode shape (64 sequences x 2 tokens, 8192 live positions, 64
    index heads x 128 dims, top-k 2048). Cold protocol as for attention: --sets copies of the
    index-key pool, each in its own physical block order."""
    import numpy as np
    import torch

    import oracle.indexer_oracle as IO
    from mla_sparse_top_amd import sfa, workloads

    inp = workloads.indexer_decode(seed=args.seed)
    print(f"[bench] generated the indexer inputs, {inp.n_tokens} tokens x {inp.n_positions} positions", file=sys.stderr,
          flush=True)
    dev0 = sfa.indexer_to_device(inp)
    n_pool = inp.num_cache_rows // 128
    sets = [dev0]
    for i in range(1, max(1, args.sets)):
        g = torch.Generator(device="cpu").manual_seed(1000 + i)
        perm = torch.randperm(n_pool, generator=g).to("cuda")
        d = dict(dev0)
        moved = torch.empty_like(dev0["k_index"].view(n_pool, 128, -1))
        moved[perm] = dev0["k_index"].view(n_pool, 128, -1)
        d["k_index"] = moved.view_as(dev0["k_index"])
        d["block_table"] = perm.to(torch.int32)[dev0["block_table"].long()].contiguous()
        sets.append(d)
    T, n_pos, K = inp.n_tokens, inp.n_positions, inp.topk
    scores = [torch.empty((T, n_pos), dtype=torch.float32, device="cuda") for _ in sets]
    outs = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in sets]

    score_calls = [sfa.prepare_indexer_scores(d["q_index"], d["k_index"], d["weights"], d["block_table"],
                                              d["kv_act_seqs"], batch=inp.batch, s1=inp.s1, topk=K, scores=scores[k])
                   for k, d in enumerate(sets)]
    select_calls = [sfa.prepare_topk_select(scores[k], d["kv_act_seqs"], batch=inp.batch, s1=inp.s1, topk=K,
                                            out=outs[k]) for k, d in enumerate(sets)]

    def step(i, ev=None):
        k = i % len(sets)
        score_calls[k]()
        if ev is not None:
            ev.record()
        select_calls[k]()

    n_warm = warm_up(step, args, torch)
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    whole0.record()
    for i in range(args.steps):
        step(i)
    whole1.record()
    torch.cuda.synchronize()
    us_per_call = whole0.elapsed_time(whole1) / args.steps * 1e3
    # per-kernel durations in a second pass, with events around and between the two kernels
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        step(i, ev[i][1])
        ev[i][2].record()
    torch.cuda.synchronize()
    score_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    select_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    same = all(torch.equal(outs[0], o) for o in outs[1:]) and all(torch.equal(scores[0], s) for s in scores[1:])

    src_hash = kernel_source_hash(("indexer_kernels.hip", "indexer_internal.h"))
    live = int(sum(int(inp.kv_act_seqs[t // inp.s1]) for t in range(T)))
    live_keys = int(inp.kv_act_seqs.sum())
    score_bytes = live_keys * 128 * 2 + T * (64 * 128 * 2 + 64 * 4) + T * n_pos * 4
    score_flop = live * (2 * 64 * 128 + 2 * 64)
    gbps = score_bytes / (score_ms * 1e-3) / 1e9
    rec = {
        "metric": INDEXER_METRIC,
        "value": round(us_per_call, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(us_per_call / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp.batch, "s1": inp.s1, "index_heads": inp.n_heads,
                   "index_dim": inp.head_dim, "kv_len": int(inp.kv_act_seqs.max()), "block_size": 128,
                   "topk": K, "cold_sets": len(sets)},
        "scores_kernel_ms_mean": round(score_ms, 5),
        "select_kernel_ms_mean": round(select_ms, 5),
        "algorithmic_bytes_scores": score_bytes,
        "algorithmic_flop_scores": score_flop,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profile(src_hash, "indexer_scores_b64_s2_traffic.txt")},
        "scores_tflops": round(score_flop / (score_ms * 1e-3) / 1e12, 1),
        "rotated_outputs_identical": bool(same),
        "kernel_source_sha256": src_hash,
    }
    if args.cpu_seconds > 0:
        # the oracle (fp64 scores, then the selection) over whole tokens until the budget is spent
        got_sc = scores[(args.steps - 1) % len(sets)].cpu().numpy()
        got_idx = outs[(args.steps - 1) % len(sets)].cpu().numpy()
        q = inp.q_index.reshape(T, inp.n_heads, inp.head_dim)
        order = np.random.default_rng(0).permutation(T)
        t0 = time.perf_counter()
        done, bad = 0, 0
        while done == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            t = int(order[done % T])
            b = t // inp.s1
            ref = IO.indexer_scores(q[t:t + 1], inp.weights[t:t + 1], inp.k_index, inp.block_table[b:b + 1],
                                    inp.kv_act_seqs[b:b + 1], 1, n_pos)
            IO.topk_positions(ref, K)
            if done < T:
                bad += len(IO.check_topk(got_idx[t:t + 1], got_sc[t:t + 1].astype(np.float64), K)["bad"])
            done += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(el / done * T * 1e6, 1), "unit": "us/call", "cores": len(os.sched_getaffinity(0)),
                               "kind": "oracle", "sample": f"{done} token evaluations (scores + selection, random "
                               f"order, seed 0) in {el:.1f} s, scaled to one call of {T} tokens",
                               "selection_rows_checked": min(done, T), "selection_rows_bad": bad}
    print(json.dumps(rec), flush=True)


def bench_decode_step(args):
    """One decode step of one layer at B=64, S1=2, 8K of cache: the cache write of the 128 new
    latent rows (positions 8190 and 8191), the indexer's scores and top-k (2048 of 8192), and
    the sparse attention over the selected rows (bf16 cache). --sets copies of both pools in
    different block orders are rotated. The cache write does not feed the indexer, so it runs on
    a second stream beside it (after the previous step's end); the attention waits for both."""
    import numpy as np
    import torch

    import oracle.cache_oracle as CO
    import oracle.indexer_oracle as IO
    import oracle.sfa_oracle as O
    from mla_sparse_top_amd import sfa, workloads

    lat = workloads.decode_mtp1(seed=args.seed)
    idx_inp = workloads.indexer_decode(seed=args.seed)
    pos = np.tile(np.array([8190, 8191], dtype=np.int32), 64)
    new = workloads.cache_write_generate(batch=64, s1=2, n_pool_blocks=1, max_blocks_per_batch=lat.block_table.shape[1],
                                         kv_dtype="bf16", seed=args.seed, positions=pos, block_table=lat.block_table)
    print("[bench] generated the decode-step inputs", file=sys.stderr, flush=True)
    T, K = lat.n_tokens, lat.topk
    lat0 = sfa.to_device(lat)
    ix0 = sfa.indexer_to_device(idx_inp)
    side = torch.cuda.Stream()  # default priority
    main = torch.cuda.current_stream()
    step_end, cw_done = torch.cuda.Event(), torch.cuda.Event()
    nw = sfa.cache_to_device(new)
    sets = []
    for i in range(max(1, args.sets)):
        if i == 0:
            ld, xd = lat0, ix0
        else:
            ld = permuted_copy(lat0, lat, 1000 + i)
            g = torch.Generator(device="cpu").manual_seed(2000 + i)
            n_pool = idx_inp.num_cache_rows // 128
            perm = torch.randperm(n_pool, generator=g).to("cuda")
            xd = dict(ix0)
            moved = torch.empty_like(ix0["k_index"].view(n_pool, 128, -1))
            moved[perm] = ix0["k_index"].view(n_pool, 128, -1)
            xd["k_index"] = moved.view_as(ix0["k_index"])
            xd["block_table"] = perm.to(torch.int32)[ix0["block_table"].long()].contiguous()
        topk = torch.empty((T, K), dtype=torch.int32, device="cuda")
        out = torch.empty((lat.batch, lat.s1, lat.n_q, 512), dtype=torch.bfloat16, device="cuda")
        cw = sfa.prepare_cache_write(nw["new_nope"], nw["new_rope"], nw["positions"], ld["block_table"], ld["key_nope"],
                                     ld["key_rope"], None, batch=64, s1=2, stream=side)
        ix = sfa.prepare_indexer(xd["q_index"], xd["k_index"], xd["weights"], xd["block_table"], xd["kv_act_seqs"],
                                 batch=64, s1=2, topk=K, out=topk)
        at = sfa.prepare_decode(ld["query_nope"], ld["query_rope"], ld["key_nope"], ld["key_rope"], None, topk,
                                ld["block_table"], ld["kv_act_seqs"], lat.softmax_scale, batch=64, s1=2, out=out)
        sets.append((cw, ix, at, topk, out))
    torch.cuda.synchronize()

    step_end.record(main)

    def step(i):
        cw, ix, at, _, _ = sets[i % len(sets)]
        side.wait_event(step_end)  # the previous step's attention has read the pool
        cw()
        cw_done.record(side)
        ix()
        main.wait_event(cw_done)
        at()
        step_end.record(main)

    n_warm = warm_up(step, args, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    valid, attn_bytes, attn_flop = algorithmic_work(lat)
    idx_bytes = int(idx_inp.kv_act_seqs.sum()) * 256 + T * (64 * 128 * 2 + 64 * 4) + T * idx_inp.n_positions * 4
    cw_bytes = T * (1160 + 1152)
    nbytes = attn_bytes + idx_bytes + cw_bytes
    gbps = nbytes / (us * 1e-6) / 1e9
    rec = {
        "metric": "us/step (cache write + indexer + sparse attention), B=64 S1=2 8K decode",
        "value": round(us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": 64, "s1": 2, "n_q": 128, "index_heads": 64, "topk": K,
                   "kv_len": 8192, "cold_sets": len(sets)},
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    if args.cpu_seconds > 0:
        # one more step on copy 0, then the oracles on sampled tokens: the written cache, the
        # selection (an exact top-k of the kernel's own scores), and the attention over the
        # selected rows of the written cache
        cw, ix, at, topk, out = sets[0]
        cw()
        ix()
        at()
        torch.cuda.synchronize()
        got_idx = topk.cpu().numpy()
        got_sc = ix._keep[0].out.cpu().numpy().astype(np.float64)
        got = out.float().cpu().numpy().astype(np.float64).reshape(T, lat.n_q, 512)
        kn, kr, _ = CO.cache_write(new.new_nope, new.new_rope, new.positions, new.block_table, 2, lat.key_nope,
                                   lat.key_rope)
        q_idx = idx_inp.q_index.reshape(T, idx_inp.n_heads, idx_inp.head_dim)
        order = np.random.default_rng(0).permutation(T)
        t0 = time.perf_counter()
        done, fails, worst, bad_sel = 0, 0, 0.0, 0
        while done == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            t = int(order[done % T])
            b = t // 2
            ref_sc = IO.indexer_scores(q_idx[t:t + 1], idx_inp.weights[t:t + 1], idx_inp.k_index,
                                       idx_inp.block_table[b:b + 1], idx_inp.kv_act_seqs[b:b + 1], 1,
                                       idx_inp.n_positions)
            IO.topk_positions(ref_sc, K)
            rows = O.resolve_rows(got_idx[t:t + 1], lat.block_table[b:b + 1], lat.kv_act_seqs[b:b + 1], 1)[0]
            kn_g, kr_g = O.gather_latents(rows[rows >= 0], kn, kr, None)
            qn = O.bf16_bits_to_f64(lat.query_nope[t * lat.n_q:(t + 1) * lat.n_q])
            qr = O.bf16_bits_to_f64(lat.query_rope[t * lat.n_q:(t + 1) * lat.n_q])
            ref = O.sparse_mla_attention_token(qn, qr, kn_g, kr_g, lat.softmax_scale)
            if done < T:
                rep = O.allclose_report(got[t], ref)
                fails += rep["fails"]
                worst = max(worst, rep["worst_ratio"])
                bad_sel += len(IO.check_topk(got_idx[t:t + 1], got_sc[t:t + 1], K)["bad"])
            done += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(el / done * T * 1e6, 1), "unit": "us/step",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"{done} token evaluations (indexer scores + selection + attention over the "
                               f"written cache, random order, seed 0) in {el:.1f} s, scaled to one step of {T} tokens",
                               "sample_parity": {"tokens": min(done, T), "attention_fails": fails,
                                                 "worst_err_over_bound": round(worst, 4),
                                                 "selection_rows_bad": bad_sel}}
    print(json.dumps(rec), flush=True)


WINDOW_WORKLOADS = {
    "swa_b64_s2_w128_bf16": ("swa_decode", "bf16"),
    "cfa_b64_s2_w128_r128_bf16": ("cfa_decode", "bf16"),
    "scfa_b64_s2_w128_k512_bf16": ("scfa_decode", "bf16"),
    "scfa_b64_s2_w128_k512_int8": ("scfa_decode", "int8"),
    # the same on 512-wide rows, the head size the pages' timing table gives these operators
    "swa_b64_s2_w128_d512_bf16": ("swa_decode_d512", "bf16"),
    "cfa_b64_s2_w128_r128_d512_bf16": ("cfa_decode_d512", "bf16"),
    "scfa_b64_s2_w128_k512_d512_bf16": ("scfa_decode_d512", "bf16"),
    "scfa_b64_s2_w128_k512_d512_int8": ("scfa_decode_d512", "int8"),
}


def bench_window(args):
    """The sliding-window + compressed-cache variants (sfa_window_decode: the sparse attention
    kernel resolving window and compressed slots itself) at the pages' timed shape: 64 sequences
    x 2 query tokens, 8K of original cache, window 128; CFA adds every causal compressed entry
    at compress_ratio 128 (64), SCFA 512 of the 2048 causal entries at compress_ratio 4. --sets copies of the pool in different block orders
    are rotated (both block tables remapped)."""
    import numpy as np
    import torch

    import oracle.sfa_oracle as O
    import oracle.window_oracle as WO
    from mla_sparse_top_amd import sfa, workloads

    fn_name, dtype = WINDOW_WORKLOADS[args.workload]
    inp = getattr(workloads, fn_name)(seed=args.seed, kv_dtype=dtype)
    print(f"[bench] generated {inp.name}", file=sys.stderr, flush=True)
    dev0 = sfa.window_to_device(inp)
    n_pool = inp.num_cache_rows // 128
    sets = [dev0]
    for i in range(1, max(1, args.sets)):
        g = torch.Generator(device="cpu").manual_seed(1000 + i)
        perm = torch.randperm(n_pool, generator=g).to("cuda")
        d = dict(dev0)
        for key in ("key_nope", "key_rope", "k_nope_scales"):
            if dev0[key] is None:
                continue
            blocks = dev0[key].view(n_pool, 128, -1)
            moved = torch.empty_like(blocks)
            moved[perm] = blocks
            d[key] = moved.view_as(dev0[key])
        p32 = perm.to(torch.int32)
        d["block_table_ori"] = p32[dev0["block_table_ori"].long()].contiguous()
        if dev0["block_table_cmp"] is not None:
            d["block_table_cmp"] = p32[dev0["block_table_cmp"].long()].contiguous()
        sets.append(d)
    outs = [torch.empty((inp.batch, inp.s1, inp.n_q, 512), dtype=torch.bfloat16, device="cuda") for _ in sets]
    calls = [sfa.prepare_window_run(inp, d, out=o, num_splits=args.num_splits) for d, o in zip(sets, outs)]
    torch.cuda.synchronize()

    def step(i):
        calls[i % len(calls)]()

    n_warm = warm_up(step, args, torch)
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    whole0.record()
    for i in range(args.steps):
        step(i)
    whole1.record()
    torch.cuda.synchronize()
    us_per_call = whole0.elapsed_time(whole1) / args.steps * 1e3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    launch_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps
    same = all(torch.equal(outs[0], o) for o in outs[1:])

    T = inp.n_tokens
    valid = sum(len(WO.token_rows(t, inp.s1, inp.window, inp.cmp_indices, inp.block_table_ori, inp.block_table_cmp,
                                  inp.ori_len, inp.cmp_len, inp.num_cache_rows)) for t in range(T))
    d_qk = 512 + inp.rope_dim   # score width: 576, or 512 for rows with the rotary channels inside
    row = (512 * 2 if dtype == "bf16" else 512 + 16) + inp.rope_dim * 2
    nbytes = valid * row + T * (inp.n_q * d_qk * 2 + inp.n_q * 512 * 2 + 4 * inp.topk_cmp)
    flop = valid * 2 * inp.n_q * (d_qk + 512)
    gbps = nbytes / (launch_ms * 1e-3) / 1e9
    tflops = flop / (launch_ms * 1e-3) / 1e12
    rec = {
        "metric": f"us/call + GB/s & TFLOP/s vs roofline, {args.workload}",
        "value": round(us_per_call, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(us_per_call / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp.batch, "s1": inp.s1, "n_q": inp.n_q,
                   "head_dim": d_qk, "window": inp.window, "topk_cmp": inp.topk_cmp, "ori_len": int(inp.ori_len.max()),
                   "compress_ratio": (int(inp.ori_len[0]) // int(inp.cmp_len[0])) if inp.topk_cmp else None,
                   "valid_slots": valid, "cold_sets": len(sets)},
        "kernel_ms_mean": round(launch_ms, 5),
        "algorithmic_bytes_per_call": nbytes,
        "algorithmic_flop_per_call": flop,
        "tflops": round(tflops, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profile(kernel_source_hash(), f"{args.workload}_traffic.txt")},
        "rotated_outputs_identical": bool(same),
        "context_pages_one_die_us": {"swa": 65, "cfa": 90, "scfa": 160}[fn_name.split("_")[0]],
    }
    if args.cpu_seconds > 0:
        got = outs[(args.steps - 1) % len(sets)].float().cpu().numpy().astype(np.float64).reshape(T, inp.n_q, 512)
        order = np.random.default_rng(0).permutation(T)
        t0 = time.perf_counter()
        done, fails, worst = 0, 0, 0.0
        while done == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            t = int(order[done % T])
            ref = WO.window_attention(inp, tokens=[t])[0]
            if done < T:
                rep = O.allclose_report(got[t], ref)
                fails += rep["fails"]
                worst = max(worst, rep["worst_ratio"])
            done += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(el / done * T * 1e6, 1), "unit": "us/call",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"{done} token evaluations (random order, seed 0) in {el:.1f} s, scaled to "
                               f"one call of {T} tokens",
                               "sample_parity": {"tokens": min(done, T), "fails": fails,
                                                 "worst_err_over_bound": round(worst, 4)}}
    print(json.dumps(rec), flush=True)


CACHE_WORKLOADS = {
    "cache_write_b64_s8192_int8": ("cache_fill", "int8"),
    "cache_write_b64_s8192_bf16": ("cache_fill", "bf16"),
    "cache_write_b64_s2_int8": ("cache_decode_step", "int8"),
}


def bench_cache_write(args):
    """The cache write (sfa_cache_write): new latent rows into the paged cache, INT8 quantised per
    128-element group or copied as bf16. Default shape: every position of the decode workload's
    cache (64 sequences x 8192 tokens, 524,288 rows). The rows read and written per call (about
    1 GB) already exceed the 256 MB last-level cache; --sets copies are still rotated."""
    import numpy as np
    import torch

    import oracle.cache_oracle as CO
    from mla_sparse_top_amd import sfa, workloads

    fn_name, dtype = CACHE_WORKLOADS[args.workload]
    inp = getattr(workloads, fn_name)(seed=args.seed, kv_dtype=dtype)
    print(f"[bench] generated {inp.name}", file=sys.stderr, flush=True)
    sets = [sfa.cache_to_device(inp) for _ in range(max(1, min(args.sets, 2)))]
    torch.cuda.synchronize()

    calls = [sfa.prepare_cache_write(d["new_nope"], d["new_rope"], d["positions"], d["block_table"], d["key_nope"],
                                     d["key_rope"], d["k_nope_scales"], batch=inp.batch, s1=inp.s1) for d in sets]

    def step(i):
        calls[i % len(sets)]()

    n_warm = warm_up(step, args, torch)
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    whole0.record()
    for i in range(args.steps):
        step(i)
    whole1.record()
    torch.cuda.synchronize()
    us_per_call = whole0.elapsed_time(whole1) / args.steps * 1e3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    launch_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps
    n_w = inp.n_written()
    per_row = (1024 + 128 + 4 + 4) + (512 + 16 + 128 if dtype == "int8" else 1024 + 128)
    nbytes = n_w * per_row
    gbps = nbytes / (launch_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash(("cache_kernels.hip", "cache_internal.h"))
    rec = {
        "metric": f"us/call + GB/s vs HBM roofline, {args.workload}",
        "value": round(us_per_call, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(us_per_call / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp.batch, "s1": inp.s1, "rows_written": n_w,
                   "pool_rows": inp.num_cache_rows, "block_size": 128, "kv_lora_rank": 512, "rope_dim": 64,
                   "quant_group": 128 if dtype == "int8" else None, "cold_sets": len(sets)},
        "kernel_ms_mean": round(launch_ms, 5),
        "algorithmic_bytes_per_call": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profile(src_hash, f"{args.workload}_traffic.txt")},
        "kernel_source_sha256": src_hash,
    }
    if args.cpu_seconds > 0:
        # the oracle over chunks of 4096 tokens (random chunk order) until the budget is spent,
        # scaled to the whole call; each chunk's rows are compared with the GPU's cache
        d = sets[(args.steps - 1) % len(sets)]
        kn = d["key_nope"].cpu()
        kn = kn.numpy() if dtype == "int8" else kn.view(torch.int16).numpy().view(np.uint16)
        kr = d["key_rope"].cpu().view(torch.int16).numpy().view(np.uint16)
        ks = None if d["k_nope_scales"] is None else d["k_nope_scales"].cpu().numpy()
        T = inp.n_tokens
        chunk = min(4096, T)
        n_chunks = (T + chunk - 1) // chunk
        order = np.random.default_rng(0).permutation(n_chunks)
        t0 = time.perf_counter()
        done_tok, bad = 0, 0
        i = 0
        while i == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            c = int(order[i % n_chunks])
            t_lo, t_hi = c * chunk, min(T, (c + 1) * chunk)
            b0 = t_lo // inp.s1
            b1 = (t_hi - 1) // inp.s1 + 1
            sub_pos = inp.positions[t_lo:t_hi]
            # the chunk as its own call: its tokens and the block-table rows of their batches
            # (a chunk holds whole batches, or lies inside one batch)
            assert (t_lo % inp.s1 == 0 and (t_hi - t_lo) % inp.s1 == 0) or b1 - b0 == 1
            rows = CO.target_rows(sub_pos, inp.block_table[b0:b1], inp.s1, inp.num_cache_rows)
            sel = np.nonzero(rows >= 0)[0]
            if dtype == "int8":
                codes, scales = CO.quantize_groups(inp.new_nope[t_lo:t_hi][sel])
                if i < n_chunks:
                    bad += int(np.any(kn[rows[sel]] != codes, axis=1).sum())
                    bad += int(np.any(ks[rows[sel]].view(np.uint32) != scales.view(np.uint32), axis=1).sum())
            elif i < n_chunks:
                bad += int(np.any(kn[rows[sel]] != inp.new_nope[t_lo:t_hi][sel], axis=1).sum())
            if i < n_chunks:
                bad += int(np.any(kr[rows[sel]] != inp.new_rope[t_lo:t_hi][sel], axis=1).sum())
            done_tok += t_hi - t_lo
            i += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(el / done_tok * T * 1e6, 1), "unit": "us/call",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"{done_tok} tokens in chunks of {chunk} (random chunk order, seed 0) in "
                               f"{el:.1f} s, scaled to one call of {T} tokens",
                               "sample_rows_checked": min(done_tok, T), "sample_rows_bad": bad}
    print(json.dumps(rec), flush=True)


COMPRESS_WORKLOADS = {"compress_b64_s2_r4": ("compress_decode", 4),
                      "compress_b64_s2_r4_c128_rot": ("compress_index_decode", 4),
                      "compress_c128a_b64_s2_d512": ("compress_c128a", None)}


def compress_algorithmic_bytes(inp) -> int:
    """Bytes the compressor must move per call: every valid token's kv and score rows; for every
    entry, the state slots not refreshed earlier in the call, its RoPE row, its block-table entry
    and the bf16 row it writes; each refreshed slot's final value; start_pos, ape and gamma."""
    c = inp.channels
    total = inp.batch * 4 + inp.ratio * c * 4 + c * 4
    n_pos = inp.rope_cos.shape[0]
    for b in range(inp.batch):
        p0 = int(inp.start_pos[b])
        s_lo, s_hi = max(0, -p0), min(inp.s1, n_pos - p0)
        n_valid = max(0, s_hi - s_lo)
        total += n_valid * c * 8 + min(inp.ratio, n_valid) * c * 8
        for s in range(s_lo, s_hi):
            if (p0 + s + 1) % inp.ratio == 0:
                total += (inp.ratio - min(inp.ratio, s - s_lo + 1)) * c * 8 + 32 * 8 + 4 + c * 2
    return total


def bench_compress(args):
    """The compressor (sfa_compress): 64 sequences, two new tokens each, ratio 4, every sequence
    closing a window. A call is idempotent on its inputs (it refreshes the same slots with the
    same values), so repeated calls on one input set measure the same work."""
    import numpy as np
    import torch

    import oracle.compress_oracle as CO
    import oracle.sfa_oracle as SO
    from mla_sparse_top_amd import sfa, workloads

    fn_name, ratio = COMPRESS_WORKLOADS[args.workload]
    inp = getattr(workloads, fn_name)(seed=args.seed, **({} if ratio is None else {"ratio": ratio}))
    print(f"[bench] generated {inp.name}", file=sys.stderr, flush=True)
    d = sfa.compress_to_device(inp)
    call = sfa.prepare_compress(inp, d)
    torch.cuda.synchronize()

    def step(i):
        call()

    n_warm = warm_up(step, args, torch)
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    whole0.record()
    for i in range(args.steps):
        step(i)
    whole1.record()
    torch.cuda.synchronize()
    us_per_call = whole0.elapsed_time(whole1) / args.steps * 1e3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    launch_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps
    nbytes = compress_algorithmic_bytes(inp)
    gbps = nbytes / (launch_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash(("compress_kernels.hip", "compress_internal.h"))
    rec = {
        "metric": f"us/call + GB/s vs HBM roofline, {args.workload}",
        "value": round(us_per_call, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(us_per_call / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp.batch, "s1": inp.s1, "ratio": inp.ratio,
                   "channels": inp.channels, "rotate": bool(inp.rotate), "start_pos": int(inp.start_pos[0]),
                   "entries_per_call": inp.batch},
        "kernel_ms_mean": round(launch_ms, 5),
        "algorithmic_bytes_per_call": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profile(src_hash, f"{args.workload}_traffic.txt")},
        "kernel_source_sha256": src_hash,
        # the pages' c128a figure at this shape (ratio 128, one state window, D = 512), on one die
        # of another machine: context only
        "context_pages_one_die_us": 55 if fn_name == "compress_c128a" else None,
    }
    if args.cpu_seconds > 0:
        # the oracle over the whole call, repeated until the budget is spent; its first result is
        # compared with the GPU's pool rows and state
        kn = d["key_nope"].cpu().view(torch.int16).numpy().view(np.uint16)
        kr = None if d["key_rope"] is None else d["key_rope"].cpu().view(torch.int16).numpy().view(np.uint16)
        ks = d["kv_state"].cpu().numpy()
        t0 = time.perf_counter()
        runs, bad = 0, 0
        while runs == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            wks, _, entries = CO.compress(inp)
            if runs == 0:
                bad += int(np.any(ks.view(np.uint32) != wks.view(np.uint32), axis=(1, 2)).sum())
                for _, _, row, y in entries:
                    if row < 0:
                        continue
                    g = (np.concatenate([SO.bf16_bits_to_f64(kn[row]), SO.bf16_bits_to_f64(kr[row])])
                         if kr is not None else SO.bf16_bits_to_f64(kn[row]))
                    bad += int(np.any(np.abs(g - y) > 1e-4 + 5e-3 * np.abs(y)))
            runs += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(el / runs * 1e6, 1), "unit": "us/call",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"the whole call ({inp.batch} sequences) {runs} times in {el:.1f} s",
                               "sample_rows_checked": inp.batch, "sample_rows_bad": bad}
    print(json.dumps(rec), flush=True)


V4_LAYER_WORKLOADS = {"v4_scfa_layer_b64_s2": "v4_scfa_layer_decode", "v4_cfa_layer_b64_s2": "v4_cfa_layer_decode",
                      "v4_swa_layer_b64_s2": "v4_swa_layer_decode"}


def bench_v4_layer(args):
    """One decode step of a DeepSeek-V4 attention layer on 512-wide rows, chained on one stream.
    SCFA layer (ratio 4): the V4 MLA prolog (4 launches), the cache write of the 128 new latent
    rows, the compressor and the index-key compressor, the indexer prolog (on the prolog's cq),
    the Lightning Indexer's scores and top-k over the 2,048 compressed index keys, and SCFA
    (window 128 + the 512 selected entries): 13 launches. CFA layer (ratio 128): the prolog, the
    cache write, the compressor, CFA over every causal entry: 7 launches. SWA layer: the prolog,
    the cache write, SWA: 6 launches. The SCFA step's footprint (~0.5 GB: weights, pools, scores)
    exceeds the 256 MB MALL, so one input set is used for all three.
    In the CFA and SCFA steps the compressors read only the step's projections, so they run on a
    second stream beside the prolog, after the previous step's end (its launches read the rows
    they rewrite); the same stream then waits for the prolog's kv_ready event (kv and cq
    complete) and runs the cache write and the indexer prolog beside the prolog's query
    up-projection. The main stream waits for that stream before the indexer and the attention.
    A one-stream run of the same launches first gives the reference output, which the
    two-stream run must match bit for bit. The SWA step runs on one stream."""
    import numpy as np
    import torch

    import oracle.window_oracle as WO
    from mla_sparse_top_amd import sfa, workloads

    L = getattr(workloads, V4_LAYER_WORKLOADS[args.workload])(seed=args.seed)
    print(f"[bench] generated the V4 {L.kind} layer-step inputs", file=sys.stderr, flush=True)
    pro, win = L.prolog, L.window
    B, S1 = win.batch, win.s1
    T, K = B * S1, L.topk_cmp
    pro_d = sfa.prolog_v4_to_device(pro)
    win_d = sfa.window_to_device(win)
    pos = torch.from_numpy(L.positions).cuda()
    cq = torch.empty((T, pro.q_lora_rank), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((T * pro.n_q, 512), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((T, 512), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, S1, win.n_q, 512), dtype=torch.bfloat16, device="cuda")
    win_d["query_nope"] = q
    side = torch.cuda.Stream()  # default priority
    main = torch.cuda.current_stream()
    kv_ready = torch.cuda.Event()  # recorded by the prolog once kv and cq are complete
    prolog = sfa.prepare_prolog_v4_run(pro, pro_d, out=(q, kv), cq_out=cq, kv_ready=kv_ready)
    # on the side stream: the compressors (they read only the step's projections), then, once the
    # prolog's kv and cq are complete, the cache write (and the indexer prolog); the one-stream
    # reference runs the same launches on the main stream
    comp, comp_one, post, post_one, tail = [], [], [], [], []
    for strm, lst in ((side, post), (None, post_one)):
        lst.append(sfa.prepare_cache_write(kv, None, pos, win_d["block_table_ori"], win_d["key_nope"], None, None,
                                           batch=B, s1=S1, stream=strm))
    bytes_by_stage = {"prolog": prolog_work(pro)[0], "cache_write": T * (1024 + 1024 + 4 + 4)}
    if L.compress_att is not None:
        catt_d = sfa.compress_to_device(L.compress_att)
        catt_d["key_nope"] = win_d["key_nope"]
        comp.append(sfa.prepare_compress(L.compress_att, catt_d, stream=side))
        comp_one.append(sfa.prepare_compress(L.compress_att, catt_d))
        bytes_by_stage["compressors"] = compress_algorithmic_bytes(L.compress_att)
    if L.kind == "scfa":
        cidx_d = sfa.compress_to_device(L.compress_idx)
        ip_d = sfa.indexer_prolog_to_device(L.indexer_prolog)
        ip_d["qr"] = cq
        sel = torch.empty((T, K), dtype=torch.int32, device="cuda")
        win_d["cmp_indices"] = sel
        comp.append(sfa.prepare_compress(L.compress_idx, cidx_d, stream=side))
        comp_one.append(sfa.prepare_compress(L.compress_idx, cidx_d))
        post.append(sfa.prepare_indexer_prolog_run(L.indexer_prolog, ip_d, stream=side))
        post_one.append(sfa.prepare_indexer_prolog_run(L.indexer_prolog, ip_d, out=post[-1].out))
        qi, _, w = post[-1].out
        tail.append(sfa.prepare_indexer(qi, cidx_d["key_nope"], w, win_d["block_table_cmp"], win_d["cmp_len"],
                                        batch=B, s1=S1, topk=K, out=sel))
        n_pos = win.block_table_cmp.shape[1] * 128
        bytes_by_stage["compressors"] += compress_algorithmic_bytes(L.compress_idx)
        bytes_by_stage["indexer_prolog"] = prolog_work(L.indexer_prolog)[0]
        # the live index keys once per batch, the tokens' index queries and weights, the scores
        # written and read back by the selection, the selected positions
        bytes_by_stage["indexer"] = int(win.cmp_len.astype(np.int64).sum()) * 256 + T * (64 * 128 * 2 + 64 * 4) \
            + 2 * T * n_pos * 4 + T * K * 4
    tail.append(sfa.prepare_window_run(win, win_d, out=out))
    # without a compressor (SWA) the cache write alone is too short to pay for the cross-stream
    # waits (measured 113.2 µs on one stream against 118.6 with it on the second), so it stays
    # on the main stream
    use_side = bool(comp)
    calls = [prolog] + comp + (post if use_side else post_one) + tail
    step_end, side_done = torch.cuda.Event(), torch.cuda.Event()
    # the reference: every launch in order on the main stream, from the inputs as generated
    for c in [prolog] + post_one + comp_one + tail:
        c()
    torch.cuda.synchronize()
    ref_out = out.clone()
    step_end.record(main)

    def step(i):
        if not use_side:
            for c in [prolog] + post_one + tail:
                c()
            return
        side.wait_event(step_end)  # the previous step has read every row this step rewrites
        for c in comp:
            c()
        prolog()
        side.wait_event(kv_ready)
        for c in post:
            c()
        side_done.record(side)
        main.wait_event(side_done)
        for c in tail:
            c()
        step_end.record(main)

    n_warm = warm_up(step, args, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    # every step recomputes the same rows from the same inputs, so the output must equal the
    # one-stream reference bit for bit
    two_stream_identical = bool(torch.equal(out.view(torch.int16), ref_out.view(torch.int16)))
    cmp_list = win_d["cmp_indices"].cpu().numpy() if win_d["cmp_indices"] is not None else None
    valid = sum(len(WO.token_rows(t, S1, win.window, cmp_list, win.block_table_ori, win.block_table_cmp, win.ori_len,
                                  win.cmp_len, win.num_cache_rows)) for t in range(T))
    kc = 0 if cmp_list is None else cmp_list.shape[1]
    bytes_by_stage[L.kind] = valid * 1024 + T * (win.n_q * 512 * 2 * 2 + 4 * kc)
    nbytes = sum(bytes_by_stage.values())
    gbps = nbytes / (us * 1e-6) / 1e9
    rec = {
        "metric": f"us/step (V4 {L.kind.upper()} layer), B=64 S1=2 8K decode, D=512",
        "value": round(us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "layer": L.kind, "batch": B, "s1": S1, "n_q": win.n_q,
                   "head_dim": 512, "hidden": pro.hidden, "q_lora_rank": pro.q_lora_rank,
                   "ori_len": int(win.ori_len.max()), "window": win.window,
                   "compress_ratio": {"swa": 1, "cfa": 128, "scfa": 4}[L.kind], "topk_cmp": K,
                   "abi_calls": sum(len(c._calls) for c in calls)},
        "algorithmic_bytes_per_step": nbytes,
        "bytes_by_stage": bytes_by_stage,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None},
        "streams": 2 if use_side else 1,
        "outputs_match_one_stream": two_stream_identical,
    }
    print(json.dumps(rec), flush=True)
    if not two_stream_identical:
        sys.exit("the two-stream layer step differs from the one-stream chain")


PROLOG_WORKLOADS = {"mla_prolog_b64_s2": "prolog_decode", "indexer_prolog_b64_s2": "indexer_prolog_decode",
                    "mla_prolog_v4_b64_s2": "prolog_v4_decode"}


def prolog_work(inp):
    """Bytes and flops the MLA prolog (or the indexer prolog) must move and do per call: every
    weight once, the inputs, the outputs, the positions and the RoPE table rows used; the
    products."""
    rows = len({int(p) for p in inp.positions if 0 <= int(p) < inp.rope_positions})
    if hasattr(inp, "w_idx_qb"):
        t, h, q, n, d = inp.tokens, inp.hidden, inp.q_lora_rank, inp.n_heads, inp.head_dim
        weights = (n * d * q + d * h + 2 * d + n * h) * 2
        nbytes = weights + t * h * 2 + t * q * 2 + t * n * d * 2 + t * d * 2 + t * n * 4 + t * 4 + rows * 32 * 4 * 2
        return nbytes, 2 * t * (q * n * d + h * (d + n))
    if hasattr(inp, "w_uq"):  # the V4 form: 512-wide query heads and latent row, rotary part inside
        t, h, q, n = inp.tokens, inp.hidden, inp.q_lora_rank, inp.n_q
        weights = (q * h + n * 512 * q + 512 * h + q + 512) * 2
        nbytes = weights + t * h * 2 + t * n * 512 * 2 + t * 512 * 2 + t * 4 + rows * 32 * 4 * 2
        return nbytes, 2 * t * (h * (q + 512) + q * n * 512)
    t, h, q, n, dn = inp.tokens, inp.hidden, inp.q_lora_rank, inp.n_q, inp.nope_dim
    weights = (q * h + n * (dn + 64) * q + n * 512 * dn + 576 * h + q + 512) * 2
    nbytes = weights + t * h * 2 + t * n * 576 * 2 + t * 576 * 2 + t * 4 + rows * 32 * 4 * 2
    flop = 2 * t * (h * (q + 576) + q * n * (dn + 64) + n * 512 * dn)
    return nbytes, flop


def bench_prolog(args):
    """The MLA prolog (sfa_mla_prolog) of the decode step: 64 sequences x 2 new tokens, hidden
    7168, query rank 1536, 128 heads. The call streams ~122 MB of weights; it rotates over --sets
    copies of them so that the 256 MB MALL cannot serve the previous call's weights. The V4 form
    (sfa_mla_prolog_v4: hidden 4096, 128 heads of 512 channels) streams ~218 MB; the indexer
    prolog (sfa_indexer_prolog) is timed the same way."""
    import numpy as np
    import torch

    import oracle.prolog_oracle as PO
    from mla_sparse_top_amd import sfa, workloads

    inp = getattr(workloads, PROLOG_WORKLOADS[args.workload])(seed=args.seed)
    print(f"[bench] generated {inp.name}", file=sys.stderr, flush=True)
    indexer = hasattr(inp, "w_idx_qb")
    v4 = hasattr(inp, "w_uq")
    to_dev = sfa.indexer_prolog_to_device if indexer else sfa.prolog_v4_to_device if v4 else sfa.prolog_to_device
    run = sfa.run_indexer_prolog if indexer else sfa.run_prolog_v4 if v4 else sfa.run_prolog
    prep = sfa.prepare_indexer_prolog_run if indexer else sfa.prepare_prolog_v4_run if v4 else sfa.prepare_prolog_run
    d0 = to_dev(inp)
    sets = [d0] + [{k: v.clone() for k, v in d0.items()} for _ in range(1, max(1, args.sets))]
    outs = [tuple(torch.empty_like(o) for o in run(inp, d0)) for _ in sets]
    calls = [prep(inp, sets[k], out=outs[k]) for k in range(len(sets))]
    torch.cuda.synchronize()

    def step(i):
        calls[i % len(sets)]()

    n_warm = warm_up(step, args, torch)
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    whole0.record()
    for i in range(args.steps):
        step(i)
    whole1.record()
    torch.cuda.synchronize()
    us_per_call = whole0.elapsed_time(whole1) / args.steps * 1e3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    launch_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps
    same = all(all(torch.equal(a, b) for a, b in zip(outs[0], o)) for o in outs[1:])
    nbytes, flop = prolog_work(inp)
    gbps = nbytes / (launch_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash(("prolog_kernels.hip", "prolog_internal.h"))
    rec = {
        "metric": f"us/call + GB/s vs HBM roofline, {args.workload}",
        "value": round(us_per_call, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(us_per_call / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": ({"workload": args.workload, "tokens": inp.tokens, "hidden": inp.hidden,
                    "q_lora_rank": inp.q_lora_rank, "n_heads": inp.n_heads, "head_dim": inp.head_dim,
                    "rotate": inp.rotate, "cold_sets": len(sets)} if indexer else
                   {"workload": args.workload, "tokens": inp.tokens, "hidden": inp.hidden,
                    "q_lora_rank": inp.q_lora_rank, "n_q": inp.n_q, "head_dim": 512, "cold_sets": len(sets)}
                   if v4 else
                   {"workload": args.workload, "tokens": inp.tokens, "hidden": inp.hidden,
                    "q_lora_rank": inp.q_lora_rank, "n_q": inp.n_q, "qk_nope_dim": inp.nope_dim,
                    "cold_sets": len(sets)}),
        "kernel_ms_mean": round(launch_ms, 5),
        "algorithmic_bytes_per_call": nbytes,
        "algorithmic_flop_per_call": flop,
        "tflops": round(flop / (launch_ms * 1e-3) / 1e12, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profile(src_hash, f"{args.workload}_traffic.txt")},
        "rotated_outputs_identical": bool(same),
        "kernel_source_sha256": src_hash,
        # the pages' mla_prolog figure at B = 64, S1 = 2 on one die of another machine: context
        "context_pages_one_die_us": 130 if v4 else None,
    }
    if args.cpu_seconds > 0:
        # the oracle over the whole call until the budget is spent; its first result is checked
        # against the GPU's outputs element by element
        got = [PO.bf16_bits_to_f64(o.cpu().view(torch.int16).numpy().view(np.uint16)) if o.dtype == torch.bfloat16
               else o.cpu().numpy().astype(np.float64) for o in outs[0]]
        t0 = time.perf_counter()
        runs, bad = 0, 0
        while runs == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            if indexer:
                want = PO.indexer_prolog(inp.x, inp.qr, inp.w_idx_qb, inp.w_idx_k, inp.ln_gamma_k, inp.ln_beta_k,
                                         inp.w_idx_proj, inp.positions, inp.rope_cos, inp.rope_sin, inp.eps,
                                         inp.n_heads, inp.rotate)
            elif v4:
                want = PO.mla_prolog_v4(inp.x, inp.w_dq, inp.gamma_cq, inp.w_uq, inp.w_dkv, inp.gamma_ckv,
                                        inp.positions, inp.rope_cos, inp.rope_sin, inp.eps, inp.n_q)
            else:
                want = PO.mla_prolog(inp.x, inp.w_dq, inp.gamma_cq, inp.w_uq_qr, inp.w_uk, inp.w_dkv_kr,
                                     inp.gamma_ckv, inp.positions, inp.rope_cos, inp.rope_sin, inp.eps, inp.n_q)
            if runs == 0:
                for g, w in zip(got, want):
                    w = w.reshape(g.shape)
                    bad += int((np.abs(g - w) > 1e-4 + 5e-3 * np.abs(w)).sum())
            runs += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(el / runs * 1e6, 1), "unit": "us/call",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"the whole call ({inp.tokens} tokens) {runs} times in {el:.1f} s",
                               "sample_elements_bad": bad}
    print(json.dumps(rec), flush=True)


def copy_calibration(mib: int, steps: int):
    """A plain copy of a known size: it reads and writes exactly mib MiB per launch, so the HBM
    byte counters read on it give the factor that turns their readings into bytes."""
    import torch

    n = mib * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "steps": steps,
                      "ms_per_copy": round(ms, 5), "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def mfma_probe(workgroups: int = 512, iters: int = 20000):
    """Dense bf16 MFMA throughput this GPU sustains on v_mfma_f32_32x32x16_bf16 (the attention
    kernel's instruction): libsfa_probe.so keeps four independent accumulator chains per wave,
    two waves per SIMD. Context for the published 2.5 PFLOP/s peak, not the attention path."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "mla_sparse_top_amd", "libsfa_probe.so"))
    lib.sfa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sfa_probe_mfma.restype = ctypes.c_int
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(n):
        st = lib.sfa_probe_mfma(workgroups, n, ctypes.c_void_p(out.data_ptr()), stream)
        if st != 0:
            raise RuntimeError(f"sfa_probe_mfma failed: {st}")

    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.5:  # raise the clocks
        launch(iters)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launch(iters)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flop = workgroups * 4 * iters * 4 * 32768
    tflops = flop / (ms * 1e-3) / 1e12
    print(json.dumps({"mfma_probe": "v_mfma_f32_32x32x16_bf16", "workgroups": workgroups, "iters": iters,
                      "ms": round(ms, 4), "tflops": round(tflops, 1),
                      "frac_of_published_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="least number of untimed calls before the timed region (default 10); calls go on "
                         "until --warmup-seconds have also passed, so the GPU clocks have left their idle state")
    ap.add_argument("--warmup-seconds", type=float, default=1.0)
    ap.add_argument("--workload", default="decode_b64_s2_bf16",
                    choices=sorted(WORKLOADS) + ["indexer_b64_s2", "decode_step_b64_s2"] + sorted(CACHE_WORKLOADS)
                    + sorted(WINDOW_WORKLOADS) + sorted(COMPRESS_WORKLOADS) + sorted(PROLOG_WORKLOADS)
                    + sorted(V4_LAYER_WORKLOADS))
    ap.add_argument("--sets", type=int, default=4, help="independent input copies rotated for a cold cache")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle time budget (0 disables)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--num-splits", type=int, default=0,
                    help="attention workloads: top-k partitions per token (0 = the library's automatic choice)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="measure the dense bf16 MFMA throughput (libsfa_probe.so) and exit")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the attention bench, run --steps plain device copies of this many MiB "
                         "(reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the sparse attention path has no "
              f"cross-GPU component.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.mfma_probe:
        mfma_probe()
        return
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib, args.steps)
        return

    if args.workload == "indexer_b64_s2":
        bench_indexer(args)
        return
    if args.workload in CACHE_WORKLOADS:
        bench_cache_write(args)
        return
    if args.workload in WINDOW_WORKLOADS:
        bench_window(args)
        return
    if args.workload in COMPRESS_WORKLOADS:
        bench_compress(args)
        return
    if args.workload in PROLOG_WORKLOADS:
        bench_prolog(args)
        return
    if args.workload in V4_LAYER_WORKLOADS:
        bench_v4_layer(args)
        return
    if args.workload == "decode_step_b64_s2":
        bench_decode_step(args)
        return

    from mla_sparse_top_amd import sfa, workloads

    fn_name, dtype, is_prefill = WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inp = getattr(workloads, fn_name)(seed=args.seed)
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] generated {inp.name} in {gen_s:.1f} s", file=sys.stderr, flush=True)
    dev0 = sfa.to_device(inp, "cuda")
    sets = [dev0] + [permuted_copy(dev0, inp, 1000 + i) for i in range(1, max(1, args.sets))]
    torch.cuda.synchronize()
    outs = [torch.empty((inp.batch, inp.s1, inp.n_q, 512), dtype=torch.bfloat16, device="cuda") for _ in sets]
    valid, nbytes, flop = algorithmic_work(inp)

    # one prepared call per rotated copy: the Python checks and marshalling happen once, each
    # step only enters the C ABI (which validates on the host and queues the kernels)
    calls = [sfa.prepare_run(inp, sets[k], prefill_mode=is_prefill, out=outs[k], num_splits=args.num_splits)
             for k in range(len(sets))]

    def step(i):
        calls[i % len(sets)]()

    # Warm-up. From idle, the GPU takes a while to raise its clocks: measured on the default
    # decode workload, a call takes ~25 us longer after 10 warm-up calls than after 1,000 or more,
    # so the warm-up always lasts --warmup-seconds as well as --warmup calls.
    args.warmup = warm_up(step, args, torch)

    # the timed region: --steps calls back to back between two events on the launch stream
    # (torch's current stream); value comes from it
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    whole0.record()
    for i in range(args.steps):
        step(i)
    whole1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = whole0.elapsed_time(whole1)
    # then the same number of calls, each between its own pair of events: the per-launch kernel
    # duration for the roofline (events between calls would add their own gaps to the region above)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    per_launch_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    mean_launch_ms = sum(per_launch_ms) / len(per_launch_ms)
    median_launch_ms = per_launch_ms[len(per_launch_ms) // 2]
    ms_per_step = total_ms / args.steps
    us_per_call = ms_per_step * 1e3

    # all rotated copies must give bit-identical outputs (block permutation invariance)
    same = all(torch.equal(outs[0], o) for o in outs[1:])

    achieved_gbps = nbytes / (mean_launch_ms * 1e-3) / 1e9
    achieved_tflops = flop / (mean_launch_ms * 1e-3) / 1e12
    src_hash = kernel_source_hash()
    traffic = traffic_from_profile(src_hash, "sfa_decode_b64_s2_bf16_traffic.txt" if args.workload == "decode_b64_s2_bf16"
                                   else f"{args.workload}_traffic.txt")
    if dtype == "bf16" and not is_prefill:
        roofline = {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved_tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic}

    metric = METRIC if args.workload == "decode_b64_s2_bf16" else f"us/call + GB/s & TFLOP/s vs roofline, {args.workload}"
    rec = {
        "metric": metric,
        "value": round(us_per_call, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp.batch, "s1": inp.s1, "n_q": inp.n_q, "n_kv": 1,
                   "topk": inp.topk, "kv_len": int(inp.kv_act_seqs.max()), "block_size": 128,
                   "kv_lora_rank": 512, "rope_dim": 64, "valid_slots": valid, "cold_sets": len(sets)},
        "kernel_ms_mean": round(mean_launch_ms, 5),
        "kernel_ms_median": round(median_launch_ms, 5),
        "gathered_kv_GBps": round(valid * (1152 if dtype == "bf16" else 656) / (mean_launch_ms * 1e-3) / 1e9, 1),
        "algorithmic_bytes_per_call": nbytes,
        "algorithmic_flop_per_call": flop,
        "tflops": round(achieved_tflops, 1),
        "roofline": roofline,
        "rotated_outputs_identical": bool(same),
        "wall_s_timed": round(wall, 3),
        "mfma": None,
        "kernel_source_sha256": src_hash,
    }
    mf = mfma_from_profile(src_hash, args.workload)
    if mf is not None:
        # MFMA unit busy fraction (rocprofv3 counters) and the issued MFMA rate (hi/lo split of P
        # included) against the dense bf16 peak, at this run's kernel time
        issued = mf["mfma_flop_per_launch"] / (mean_launch_ms * 1e-3) / 1e12
        rec["mfma"] = {"busy_fraction": mf["mfma_busy_fraction"], "issued_tflops": round(issued, 1),
                       "issued_frac_of_peak": round(issued / BF16_PEAK_TFLOPS, 4),
                       "source": "profiles/sfa_attention_mfma_utilisation.txt"}
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(inp, outs[(args.steps - 1) % len(sets)], args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
