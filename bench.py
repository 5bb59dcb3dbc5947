#!/usr/bin/env python3
"""Benchmark of one MLA decode step on one MI355X.

A step is the whole hot path over one batch: query absorption, append of the
B*Q new cache rows, split-KV decode, log-sum-exp combine, value
up-projection (three library calls: absorption + append and combine +
up-projection each run as one fused call; --unfused runs five). The default workload is the DeepSeek-V2-Lite layer shape at
32K context (B = 8 sequences of 32,768 tokens, 16 heads, 512 + 64 latent
row). Inputs are seeded synthetic tensors already resident in HBM when the
timed region starts. One cache per layer is rotated (27 layers, as V2-Lite
has) so every step reads its latent cache from HBM rather than from the
256 MB Infinity Cache.

Prints one JSON line. value = latent-cache bytes read per step / step time
(GB/s); the decode kernel's own rate against the 8 TB/s HBM peak is in
"roofline"; the fp64 oracle timed on the host cores is in "cpu_baseline".
A sparse-read workload (v2lite_32k_dsa) adds the indexer-key append, the
index scores and the top-k selection to the step, and its decode reads only
the selected rows: value = (indexer keys + selected latent rows) per step
time, and "roofline" is the indexer pass, the step's dominant kernel.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--graph]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode latent-cache GB/s (% of HBM peak) + decode tokens/s, V2-Lite 32K"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
LAYERS = {"v2lite_32k": 27, "v2lite_paged_varlen": 27, "v2_h128_8k": 4, "v2_h128_1m_q4": 2,
          "v2lite_32k_tree8": 27, "v2lite_32k_q8": 27, "v2lite_32k_q4": 27, "v2lite_32k_dsa": 27,
          "v2lite_prefill_32k_c4k": 2, "tiny_f32": 4}
PREFILL_MIN_Q = 64             # q_len from which a step is a prefill chunk
CSRC = os.path.join(ROOT, "mla_latent_kv_03_amd", "csrc")
# decode kernel name (mla_decode_kernel_name) -> (kernel symbol, the sources that define it)
DECODE_KERNELS = {
    "mfma_rows16": ("decode_rows16_kernel", ["mla_decode_common.h", "mla_decode_rows16.hip"]),
    "mfma_ws": ("decode_ws_kernel", ["mla_decode_common.h", "mla_decode_ws.hip"]),
    "generic": ("decode_generic_kernel", ["mla_kernels.hip"]),
    "mfma_q8": ("decode_q8_kernel<8>", ["mla_decode_common.h", "mla_q8.hip"]),
    "mfma_q4": ("decode_q8_kernel<4>", ["mla_decode_common.h", "mla_q8.hip"]),
    # sparse read: the indexer pass is the step's dominant kernel
    "index_scores_mfma": ("index_scores_mfma_kernel<false>", ["mla_decode_common.h", "mla_sparse.hip"]),
    # prefill chunk in the unabsorbed form: one library call, three launches
    "prefill_unabsorbed": ("prefill_expand_kernel + prefill_query_kernel + prefill_attn_kernel",
                           ["mla_decode_common.h", "mla_prefill.hip"]),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="v2lite_32k")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--split-chunk", type=int, default=0,
                    help="fixed partition size in tokens (-1: per-sequence plan; 0: the workload's)")
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--graph", action="store_true", help="replay each layer's step as a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-form", choices=["auto", "absorbed", "unabsorbed"], default="auto",
                    help="prefill chunks (q_len >= 64): the form the step takes (auto: the "
                         "library's choice, mla_prefill_form)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as five library calls instead of three")
    ap.add_argument("--no-stream-read", action="store_true",
                    help="skip the plain streaming-read reference (achievable HBM read rate)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def src_hash(names):
    """sha256[:16] over the given sources (concatenated, in order)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(wl_name, kernel_src_hash):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    only if it was taken on the current decode kernel source."""
    p = os.path.join(ROOT, "profiles", f"decode_{wl_name}_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("decode_src_sha256_16") != kernel_src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def visible_pairs(wl, inp):
    """(query, cached token) pairs the attention scores: query j of sequence b
    sees tokens 0 .. L_b - Q + j (a drafted tree sees no more than that)."""
    Q = wl.q_len
    return sum(Q * (int(L) - Q) + Q * (Q + 1) // 2 for L in inp.seq_lens)


def cpu_threads():
    """(threads the oracle's BLAS calls run on, host CPU counts): the oracle
    is NumPy, whose matrix products use the BLAS thread pool and whose other
    operations run on one thread."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = os.cpu_count() or 1
    return int(min(blas, aff)), {"host_cpus": os.cpu_count(), "affinity_cpus": aff,
                                 "blas_threads": int(blas)}


def cpu_baseline_prefill(wl, inp, flops_step, bytes_step, n_queries=8):
    """Prefill chunk: the oracle on sampled queries of the chunk (each one a
    one-token decode over the tokens it sees, head 0 only), scaled by the
    share of the step's algorithmic work they represent."""
    import numpy as np
    import oracle
    threads, host = cpu_threads()
    L, Q = int(inp.seq_lens[0]), wl.q_len
    P = L - Q
    js = [int(x) for x in np.linspace(0, Q - 1, n_queries)]
    c, kr = inp.seq(0)
    t = time.perf_counter()
    for j in js:
        oracle.attend_sequence(c[:P + j + 1], kr[:P + j + 1], inp.q_nope[0][j:j + 1][:, :1],
                               inp.q_rope[0][j:j + 1][:, :1], inp.w_uk[:1], inp.w_uv[:1],
                               wl.softmax_scale, wl.rope_base)
    dt = time.perf_counter() - t
    flops = sum(P + j + 1 for j in js) * (2 * wl.dim + 2 * wl.kv_rank)
    share = flops / flops_step
    return {"value": round(bytes_step * share / dt / 1e9, 6), "unit": "GB/s",
            "cores": int(threads), **host, "kind": "oracle",
            "sample": f"{len(js)} of {Q} queries of sequence 0 (each a one-token decode over the "
                      f"tokens it sees), head 0 of {wl.heads}, {dt:.1f} s; fp64 unabsorbed NumPy "
                      f"oracle; scaled by the sample's share {share:.2e} of the step's "
                      f"algorithmic flops",
            "seconds": round(dt, 2),
            "prefill_tokens_per_s": round(wl.batch * Q * share / dt, 6)}


def cpu_baseline(wl, inp, budget_flops=2.4e12):
    """Time the fp64 oracle on the host cores over a bounded sample of the workload.

    The sample is the first sequences (and, when one sequence with every head
    is over budget, the first heads) such that the oracle's work is about
    ``budget_flops`` (roughly 10-20 s). The rate is scaled to the metric's
    unit: latent-cache bytes processed per second, counting a sequence's bytes
    in proportion to the heads sampled.
    """
    import oracle
    threads, host = cpu_threads()
    per_tok_head = 2 * wl.kv_rank * (wl.nope_dim + wl.v_dim) + 4 * (wl.nope_dim + wl.rope_dim)
    heads = wl.heads
    seq_cost = lambda b, h: int(inp.seq_lens[b]) * h * wl.q_len * per_tok_head  # noqa: E731
    if seq_cost(0, heads) > budget_flops:
        heads = max(1, min(heads, int(budget_flops // seq_cost(0, 1))))
    seqs, spent = [], 0
    for b in range(wl.batch):
        if seqs and spent + seq_cost(b, heads) > budget_flops:
            break
        seqs.append(b)
        spent += seq_cost(b, heads)
    sparse = wl.index_topk > 0
    if sparse:  # indexer scores + selection of every sequence of the sample, then attention
        ref = lambda x, heads, seqs: oracle.mla_decode_ref_sparse(  # noqa: E731
            x, sparse_selection(x, seqs), heads=heads, seqs=seqs)
    else:
        bits = {"q8": 8, "q4": 4}.get(wl.cache)
        ref = ((lambda x, heads, seqs: oracle.mla_decode_ref_q8(x, heads=heads, seqs=seqs,
                                                                bits=bits))
               if bits else oracle.mla_decode_ref)
    t = time.perf_counter()
    ref(inp, heads=list(range(heads)), seqs=seqs)
    dt = time.perf_counter() - t
    tokens = sum(int(inp.seq_lens[b]) for b in seqs)
    if sparse:  # indexer keys of every token + the selected latent rows
        sel = sum(min(wl.index_topk, int(inp.seq_lens[b]) - wl.q_len + j + 1)
                  for b in seqs for j in range(wl.q_len))
        nbytes = (tokens * wl.index_dim * wl.elem_bytes
                  + sel * wl.cache_row_bytes * heads / wl.heads)
    else:
        nbytes = tokens * wl.cache_row_bytes * heads / wl.heads
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            **host, "kind": "oracle",
            "sample": f"{len(seqs)} of {wl.batch} sequences ({tokens} cached tokens), "
                      f"{heads} of {wl.heads} heads, {dt:.1f} s; fp64 unabsorbed NumPy oracle"
                      f"{' (rows coded to 8 bits first)' if wl.cache == 'q8' else ''}"
                      f"{' (rows coded to 4 bits first)' if wl.cache == 'q4' else ''}"
                      f"{' (indexer scores and top-k selection first)' if sparse else ''}; "
                      f"bytes counted x {heads}/{wl.heads}",
            "seconds": round(dt, 2),
            "decode_tokens_per_s": round(len(seqs) * wl.q_len * heads / wl.heads / dt, 4)}


def sparse_selection(inp, seqs):
    """The oracle's selection for the sampled sequences only (others empty)."""
    import oracle
    wl = inp.wl
    out = []
    for b in range(wl.batch):
        if b not in seqs:
            out.append([[] for _ in range(wl.q_len)])
            continue
        L = int(inp.seq_lens[b])
        sc = oracle.indexer_scores(inp.q_idx[b], inp.w_idx[b], inp.seq_index_keys(b))
        out.append([oracle.topk_tokens(sc[j], wl.index_topk, L - wl.q_len + j + 1)
                    for j in range(wl.q_len)])
    return out


def stream_read_rate(torch, mla, stream, nbytes=4 << 30, reps=10):
    """GB/s of a plain coalesced read of a 4 GiB buffer (each block one
    contiguous chunk, 16-byte non-temporal loads, mla_stream_read): what a
    stream with no arithmetic reaches on this device, for context beside the
    decode kernel's fraction of the 8 TB/s peak. Best over a few grid sizes;
    HIP events on the launch stream."""
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    best = None
    for blocks in (512, 1024, 2048, 4096):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        mla.stream_read(buf, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            mla.stream_read(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        gbs = nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, blocks)
    del buf
    return {"gbs": round(best[0], 1), "pct_of_peak": round(100 * best[0] / HBM_PEAK_GBS, 2),
            "bytes": nbytes, "blocks": best[1], "threads_per_block": 256,
            "kernel": "stream_read_kernel (one contiguous chunk per block, 16-byte non-temporal "
                      "loads)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note, not an implementation)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workload
    import mla_latent_kv_03_amd as mla
    from mla_latent_kv_03_amd.pipeline import (DecodeStep, fill_cache, fill_cache_q8,
                                               fill_index_cache, upload)

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    mla.lib()
    wl = workload.WORKLOADS[args.workload]
    if args.split_chunk < 0:
        wl = wl.replace(split_chunk=0)
    elif args.split_chunk > 0:
        wl = wl.replace(split_chunk=args.split_chunk,
                        num_splits=-(-wl.max_seq_len // args.split_chunk))
    if args.num_splits:
        wl = wl.replace(num_splits=args.num_splits)
    n_layers = args.layers or LAYERS.get(wl.name, 2)
    cfg = mla.Config.from_workload(wl)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    t_setup = time.perf_counter()
    inp = workload.make(wl, 0)
    B, Q, H = wl.batch, wl.q_len, wl.heads

    # ---- device state: one cache pool per layer (same bytes, distinct addresses)
    pt = upload(inp.page_table, torch.int32)
    seq_lens = upload(inp.seq_lens, torch.int32)
    bits = {"q8": 8, "q4": 4}.get(wl.cache, 0)
    q8 = bits != 0
    if q8:  # 8- or 4-bit rows: codes plus (min, step) pairs
        pool0 = torch.full((inp.num_pages, wl.page_size, wl.cache_row_bytes), 255,
                           dtype=torch.uint8, device="cuda")
    else:
        pool0 = torch.full((inp.num_pages, wl.page_size, wl.dim), float("nan"), dtype=dt,
                           device="cuda")
    si = np.concatenate([np.full(int(L), b, np.int32) for b, L in enumerate(inp.seq_lens)])
    pos = np.concatenate([np.arange(int(L), dtype=np.int32) for L in inp.seq_lens])
    if q8:
        fill_cache_q8(cfg, pool0, pt, upload(inp.c, dt), upload(inp.k_rope, dt),
                      upload(si, torch.int32), upload(pos, torch.int32), bits=bits)
    else:
        fill_cache(cfg, pool0, pt, upload(inp.c, dt), upload(inp.k_rope, dt),
                   upload(si, torch.int32), upload(pos, torch.int32))
    q_nope, q_rope = upload(inp.q_nope, dt), upload(inp.q_rope, dt)
    w_uk, w_uv = upload(inp.w_uk, dt), upload(inp.w_uv, dt)
    rows = np.concatenate([inp.offsets[b] + np.arange(int(L) - Q, int(L))
                           for b, L in enumerate(inp.seq_lens)])
    c_new, k_new = upload(inp.c[rows], dt), upload(inp.k_rope[rows], dt)
    sparse = wl.index_topk > 0
    if sparse:  # indexer keys: one pool per layer, like the latent cache
        ipool0 = torch.full((inp.num_pages, wl.page_size, wl.index_dim), float("nan"), dtype=dt,
                            device="cuda")
        fill_index_cache(cfg, ipool0, pt, upload(inp.k_idx, dt), upload(si, torch.int32),
                         upload(pos, torch.int32))
        ipools = [ipool0] + [ipool0.clone() for _ in range(n_layers - 1)]
        q_idx, w_idx = upload(inp.q_idx, dt), upload(inp.w_idx, torch.float32)
        k_idx_new = upload(inp.k_idx[rows], dt)
    st = DecodeStep(cfg, B, Q, wl.num_splits, inp.seq_lens, split_chunk=wl.split_chunk,
                    tree_parents=inp.parents, cache_bits=bits, index_topk=wl.index_topk)
    # the drafted rows at their positions (a tree's keys sit at prefix + depth;
    # the fill rotated every key at its slot), then one copy per layer
    st.append(c_new, k_new, pt, pool0)
    pools = [pool0] + [pool0.clone() for _ in range(n_layers - 1)]
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    stream = torch.cuda.current_stream()

    # prefill chunk: the absorbed form (the decode calls with q_len = C) or the
    # unabsorbed one (append the chunk, then mla_prefill_unabsorbed per sequence)
    prefill = Q >= PREFILL_MIN_Q
    form = None
    if prefill:
        form = (mla.prefill_form(cfg, Q, int(inp.seq_lens.max())) if args.prefill_form == "auto"
                else args.prefill_form)
        un_ok = mla.prefill_form(cfg, 4096, 4096) == "unabsorbed"  # the form is supported
        if un_ok:
            ws_u = [torch.empty(mla.prefill_workspace_bytes(cfg, int(L), Q), dtype=torch.uint8,
                                device="cuda") for L in inp.seq_lens]
            out_u = torch.empty((B, Q, H, wl.v_dim), dtype=dt, device="cuda")
            lse_u = torch.empty((B, Q, H), dtype=torch.float32, device="cuda")
            qn_b = [q_nope[b].contiguous() for b in range(B)]
            qr_b = [q_rope[b].contiguous() for b in range(B)]

        def unabsorbed_call(pool):
            for b in range(B):
                mla.prefill_unabsorbed(cfg, qn_b[b], qr_b[b], w_uk, w_uv, pool, pt[b],
                                       int(inp.seq_lens[b]), ws_u[b], out_u[b], lse_u[b])

    def unabsorbed_step(layer):
        pool = pools[layer % n_layers]
        st.append(c_new, k_new, pt, pool)
        unabsorbed_call(pool)

    def absorbed_step(layer):
        pool = pools[layer % n_layers]
        if args.unfused:
            st.absorb(q_nope, q_rope, w_uk)
            st.append(c_new, k_new, pt, pool)
        elif sparse:  # the indexer keys go in the same launch
            mla.absorb_append_index(cfg, q_nope, q_rope, st.qpos, w_uk, st.q_full, c_new, k_new,
                                    st.seq_idx, st.slot, pt, pool, k_idx_new,
                                    ipools[layer % n_layers])
        else:
            st.absorb_append(q_nope, q_rope, w_uk, c_new, k_new, pt, pool)
        if sparse:
            ipool = ipools[layer % n_layers]
            if args.unfused:
                st.index_append(k_idx_new, pt, ipool)
            if args.unfused:
                st.index_scores(q_idx, w_idx, ipool, pt, seq_lens)
                st.select(seq_lens)
            else:
                st.index_select(q_idx, w_idx, ipool, pt, seq_lens)
        st.decode(pool, pt, seq_lens)
        if args.unfused:
            st.combine()
            st.up_project(w_uv)
        else:
            st.combine_up_project(w_uv)

    one_step = unabsorbed_step if form == "unabsorbed" else absorbed_step

    graphs = None
    if args.graph:
        for layer in range(n_layers):
            one_step(layer)
        torch.cuda.synchronize()
        graphs = []
        for layer in range(n_layers):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_step(layer)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(layer):
        if graphs is not None:
            graphs[layer % n_layers].replay()
        else:
            one_step(layer)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        run(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # ---- prefill: the step in both forms (the other one after the timed
    # region), and the unabsorbed call alone back to back
    forms = None
    if prefill and un_ok:
        def time_steps(fn, k):
            torch.cuda.synchronize()
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(k):
                fn(i)
            b_.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b_) / k
        kf = max(3, min(args.steps, 20))
        other = absorbed_step if form == "unabsorbed" else unabsorbed_step
        other(0)
        ms_other = time_steps(other, kf)
        for i in range(n_layers):  # every layer cache holds the chunk
            st.append(c_new, k_new, pt, pools[i])
        un_call_ms = time_steps(lambda i: unabsorbed_call(pools[i % n_layers]), kf)
        forms = {"picked": form,
                 "absorbed_step_us": round(1e3 * (ms_step if form != "unabsorbed" else ms_other), 1),
                 "unabsorbed_step_us": round(1e3 * (ms_step if form == "unabsorbed" else ms_other), 1),
                 "unabsorbed_call_us": round(1e3 * un_call_ms, 1)}

    # ---- average duration of the decode kernel: kd launches back to back on
    # the launch stream (rotating the layer caches as the step does), between
    # two HIP events; launch-to-launch, so the gap between kernels is included
    kd = max(20, min(args.steps, 200))
    for i in range(n_layers):  # absorb + append once per layer cache (inputs of the decode)
        st.absorb_append(q_nope, q_rope, w_uk, c_new, k_new, pt, pools[i])
    torch.cuda.synchronize()
    eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eb0.record(stream)
    for i in range(kd):
        if sparse:  # the dominant kernel of a sparse step: the indexer pass
            st.index_scores(q_idx, w_idx, ipools[i % n_layers], pt, seq_lens)
        else:
            st.decode(pools[i % n_layers], pt, seq_lens)
    eb1.record(stream)
    torch.cuda.synchronize()
    decode_ms = eb0.elapsed_time(eb1) / kd
    sparse_calls = None
    if sparse:  # per-call events around the selection and the gather decode
        se = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(kd)]
        for i in range(kd):
            st.index_scores(q_idx, w_idx, ipools[i % n_layers], pt, seq_lens)
            se[i][0].record(stream)
            st.select(seq_lens)
            se[i][1].record(stream)
            st.decode(pools[i % n_layers], pt, seq_lens)
            se[i][2].record(stream)
        torch.cuda.synchronize()
        tk = sorted(a.elapsed_time(b) for a, b, _ in se)
        sd = sorted(b.elapsed_time(c) for _, b, c in se)
        sparse_calls = {"topk_median_us": round(tk[len(tk) // 2] * 1e3, 2),
                        "sparse_decode_median_us": round(sd[len(sd) // 2] * 1e3, 2),
                        "sparse_decode_kernel": mla.decode_sparse_kernel_kind(
                            cfg, wl.index_topk, wl.num_splits)}

    # ---- per-call durations of the decode kernel and of decode + combine:
    # HIP events around each call of a third pass (there the merge and the
    # up-projection run as separate calls); each sample also holds one event
    # record, so these read a little above the back-to-back average
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(kd)]
    torch.cuda.synchronize()
    for i in range(kd):
        pool = pools[i % n_layers]
        st.absorb_append(q_nope, q_rope, w_uk, c_new, k_new, pt, pool)
        evs[i][0].record(stream)
        st.decode(pool, pt, seq_lens)  # (sparse: over the last selection)
        evs[i][1].record(stream)
        st.combine()
        evs[i][2].record(stream)
        st.up_project(w_uv)
    torch.cuda.synchronize()
    d_ms = sorted(a.elapsed_time(b) for a, b, _ in evs)
    dc_ms = sorted(a.elapsed_time(c) for a, _, c in evs)
    decode_call_avg = sum(d_ms) / len(d_ms)
    decode_med = d_ms[len(d_ms) // 2]
    dc_med = dc_ms[len(dc_ms) // 2]
    if form == "unabsorbed":  # the picked form's call (no split partials to merge)
        decode_call_avg = decode_med = dc_med = un_call_ms

    # ---- algorithmic work
    total_tokens = int(inp.seq_lens.astype(np.int64).sum())
    if sparse:
        # a sparse step reads every indexer key and the selected latent rows;
        # the indexer pass (the timed kernel) reads the keys
        sel_rows = sum(min(wl.index_topk, int(L) - Q + j + 1)
                       for L in inp.seq_lens for j in range(Q))
        kernel_bytes = total_tokens * wl.index_dim * wl.elem_bytes
        step_bytes = kernel_bytes + sel_rows * wl.cache_row_bytes
        flops = total_tokens * Q * 2 * wl.index_heads * wl.index_dim
        kernel = "index_scores_mfma"
    else:
        kernel_bytes = step_bytes = total_tokens * wl.cache_row_bytes  # read once per step
        # every (query row, visible token) pair: 2 * D for the score, 2 * d_c for P.V
        flops = visible_pairs(wl, inp) * H * (2 * wl.dim + 2 * wl.kv_rank)
        kernel = {8: "mfma_q8", 4: "mfma_q4"}[bits] if q8 else mla.decode_kernel_kind(cfg, Q)
    if form == "unabsorbed":
        # the picked form's work: the expansion of every cached token (2 x 512
        # x 256 flops per token and head) and the per-head attention (2 x 192
        # + 2 x 128 per visible pair), timed as one library call (3 launches)
        flops = (visible_pairs(wl, inp) * H * (2 * (wl.nope_dim + wl.rope_dim) + 2 * wl.v_dim)
                 + total_tokens * H * 2 * wl.kv_rank * (wl.nope_dim + wl.v_dim))
        kernel = "prefill_unabsorbed"
    cache_bytes = kernel_bytes
    gbs_step = step_bytes / (ms_step * 1e-3) / 1e9
    if form == "unabsorbed":
        decode_ms = un_call_ms
    gbs_decode = cache_bytes / (decode_ms * 1e-3) / 1e9
    tflops_decode = flops / (decode_ms * 1e-3) / 1e12
    ai = flops / cache_bytes
    bound = "hbm" if ai < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    ksym, ksrc = DECODE_KERNELS[kernel]
    khash = src_hash(ksrc)
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs_decode, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs_decode / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops_decode, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops_decode / BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = traffic_from_profile(wl.name, khash)
    roof["kernel"] = ksym
    roof["algorithmic_bytes_per_launch"] = cache_bytes
    roof["algorithmic_flops_per_launch"] = flops
    roof["avg_launch_us"] = round(decode_ms * 1e3, 2)
    roof["launches_timed"] = kd
    roof["per_call_avg_us"] = round(decode_call_avg * 1e3, 2)
    roof["per_call_median_us"] = round(decode_med * 1e3, 2)

    out = {
        "metric": METRIC,
        "value": round(gbs_step, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic: seeded N(0,1) latents/keys/queries, N(0,1/d_c) weights"
                + ("; indexer queries/keys N(0,1), head weights N(0,1/H_I)" if sparse else ""),
        "config": {"workload": wl.name, "batch": B, "q_len": Q, "heads": H,
                   "seq_len": wl.seq_len if wl.seq_len else list(wl.len_range),
                   "total_cached_tokens": total_tokens, "kv_rank": wl.kv_rank,
                   "rope_dim": wl.rope_dim, "page_size": wl.page_size,
                   "paged": wl.paged, "num_splits": wl.num_splits,
                   "split_chunk": wl.split_chunk,
                   "layer_caches_rotated": n_layers, "hip_graph": bool(args.graph),
                   "library_calls_per_step": (5 if args.unfused else 3) +
                                             ((3 if args.unfused else 1) if sparse else 0),
                   "drafted_tree": None if wl.tree is None else list(wl.tree),
                   "cache_format": wl.cache, "cache_bytes_per_token": wl.cache_row_bytes,
                   "decode_kernel": kernel,
                   "index_topk": wl.index_topk or None,
                   "indexer": ([wl.index_heads, wl.index_dim] if sparse else None)},
        "pct_hbm_peak": round(100 * gbs_step / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(B * Q / (ms_step * 1e-3), 1),
        "decode_gbs": round(gbs_decode, 1),
        "decode_combine_gbs": round(cache_bytes / (dc_med * 1e-3) / 1e9, 1),
        "decode_tflops": round(tflops_decode, 2),
        "mfma_pct": round(100 * tflops_decode / BF16_PEAK_TFLOPS, 2),
        "roofline": roof,
        "setup_s": round(t_setup, 1),
        "decode_src_sha256_16": khash,
    }
    if sparse:
        out["sparse"] = dict(sparse_calls, selected_rows_per_step=sel_rows,
                             step_bytes=step_bytes,
                             dense_equivalent_cache_bytes=total_tokens * wl.cache_row_bytes)
    if Q >= PREFILL_MIN_Q:
        out["prefill_tokens_per_s"] = round(B * Q / (ms_step * 1e-3), 1)
        out["prefill_step_tflops"] = round(flops / (ms_step * 1e-3) / 1e12, 2)
        out["prefill_forms"] = forms
    elif wl.name.startswith("v2lite"):
        out["v2lite_attention_tokens_per_s_27_layers"] = round(B / (27 * ms_step * 1e-3), 1)
    props = torch.cuda.get_device_properties(0)
    out["device"] = {"name": props.name, "compute_units": props.multi_processor_count,
                     "gcn_arch": getattr(props, "gcnArchName", "")}
    if not args.no_stream_read:
        out["hbm_stream_read"] = stream_read_rate(torch, mla, stream)
    if args.calibrate_copy:
        # a plain copy of known size, for scaling the HBM byte counters
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = src.numel() * 4
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_prefill(wl, inp, flops, cache_bytes)
                               if Q >= PREFILL_MIN_Q else cpu_baseline(wl, inp))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
