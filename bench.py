"""Benchmark of the CSA2 decode hot path on one MI355X.

A step is one Full-layer decode call (csa2_sparse_attn_decode: indexer scan,
exact top-512, FP4 gather + dequant, 64-head attention over the selection
plus the 128-row window) for every sequence of the 64K-context workload
(32 sequences x 32,768 MXFP4/FP4 entries).  Inputs are resident in HBM
before timing; the caches are replicated and rotated so the 256 MB
last-level cache cannot serve one call's data to the next (each call reads
~83 MB; 8 replicas put >= 512 MB between two uses of one replica).

Prints ONE JSON line.  `python bench.py --gpus N --steps K --warmup W`.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "indexer_encoder-full-64k_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--query", choices=("bf16", "mxfp4"), default="bf16",
                    help="indexer query format of the headline step (the "
                         "other is reported under variants)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="counter-collection run: plain indexer launches on "
                         "rotated cache replicas, then a float32 copy kernel "
                         "of known size (read 256 MiB, write 256 MiB) to "
                         "calibrate FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def n_blocks(wl):
    return -(-wl.n // wl.pool[1]) if wl.pool else 0


def query_bytes(query):
    """Indexer query bytes per sequence: 32 x 128 bf16, or the 32 heads as
    MXFP4 (64 code + 4 scale bytes each)."""
    return 32 * 68 if query == "mxfp4" else 32 * 128 * 2


def algorithmic_bytes(wl, query="bf16"):
    """Bytes the method must move for one query through a Full layer:
    the indexer keys scanned (68 n; hierarchically 256 per bf16 block key
    plus 68 per pool member), 288 k (chosen main entries), 512 n_swa
    (window), the indexer query (8192 bf16 or 2176 MXFP4) + 128 (head
    weights), 65536 (bf16 query), 65536 (bf16 output) and 4 k (top-k ids
    written)."""
    scan = (256 * n_blocks(wl) + 68 * wl.pool[0] * wl.pool[1] if wl.pool
            else 68 * wl.n)
    return (scan + 288 * wl.k + 512 * wl.n_swa + query_bytes(query) + 128
            + 65536 + 65536 + 4 * wl.k)


def indexer_bytes(wl, query="bf16"):
    """Algorithmic bytes of one launch of the scan kernel the roofline is
    quoted on: the MXFP4 keys of every visible entry (hierarchically: the
    bf16 block keys of every block) plus the per-sequence query and
    weights."""
    per = 256 * n_blocks(wl) if wl.pool else 68 * wl.n
    return wl.B * (per + query_bytes(query) + 128)


def source_hash():
    h = hashlib.sha256()
    for f in ("indexer.hip", "common.h"):
        with open(os.path.join(ROOT, "fp4_kv_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(query):
    """HBM bytes per indexer launch (the scan with a bf16 or an MXFP4 query)
    from the committed rocprofv3 counter summary, or None when it is absent
    or the kernel changed since."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    if prof.get("source_hash") != source_hash():
        return None
    return prof.get("kernels", {}).get(query, {}).get("hbm_bytes_per_launch")


def replicate(st, R):
    """R independent copies of the caches (same contents); each entry of
    `planes` is (main codes, main scales, idx codes, idx scales, block keys
    or None)."""
    import torch
    from fp4_kv_cache_amd import csa2
    reps = [st.cache]
    planes = [(st.main_codes, st.main_scales, st.idx_codes, st.idx_scales,
               st.block_keys)]
    for _ in range(R - 1):
        t = (st.main_codes.clone(), st.main_scales.clone(),
             st.idx_codes.clone(), st.idx_scales.clone(),
             None if st.block_keys is None else st.block_keys.clone())
        planes.append(t)
        reps.append(csa2.cache_desc(*t[:4], st.n_entries, block_keys=t[4]))
    torch.cuda.synchronize()
    return reps, planes


def time_steps(step, args, R, out, ids):
    """Eager and HIP-graph time per step of `step(i)` (i picks the cache
    replica).  The graph holds one step per replica (R steps) and is
    replayed until at least K steps have run; a replay must reproduce the
    eager result bit for bit.  After the timed region, further replays are
    timed one by one with events for the spread (p10 / p50 / p90 of the time
    per step within a replay)."""
    import numpy as np
    import torch
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t0) / args.steps
    if args.no_graph:
        return eager_s, None, args.steps, None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(R):
            step(r)          # warm the capture path on this stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            step(r)
    reps_needed = max(1, math.ceil(args.steps / R))
    steps_run = reps_needed * R
    for _ in range(max(1, args.warmup // R)):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps_needed):
        g.replay()
    torch.cuda.synchronize()
    graph_s = (time.perf_counter() - t0) / steps_run
    per_step = []
    for _ in range(max(10, min(reps_needed, 50))):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        per_step.append(e0.elapsed_time(e1) * 1e3 / R)
    spread = {f"p{q}": float(np.percentile(per_step, q)) for q in (10, 50, 90)}
    spread.update(replays=len(per_step), steps_per_replay=R)
    step(R - 1)
    torch.cuda.synchronize()
    e_out, e_ids = out.clone(), ids.clone()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), e_out.view(torch.int16))
    assert torch.equal(ids, e_ids)
    del g
    return eager_s, graph_s, steps_run, spread


def run_gpu(args, wl):
    import torch
    from fp4_kv_cache_amd import csa2, workload

    dev = "cuda:0"
    st = workload.build(wl, dev)
    per_call = wl.B * algorithmic_bytes(wl)
    R = args.replicas or max(1, math.ceil(2 * 256e6 / per_call) + 1)
    reps, planes = replicate(st, R)
    k = wl.k
    out = torch.empty((wl.B, 64, 512), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((wl.B, k), dtype=torch.int32, device=dev)
    ws = csa2.workspace(csa2.workspace_size(csa2.OP_DECODE, wl.B, wl.n, k,
                                            wl.pool), dev)
    # The MXFP4 indexer query (V4's FP4 indexer query): an input of the
    # layer call like the bf16 one, packed once outside the timed steps.
    qc, qs = csa2.pack_query_fp4(st.q_idx)

    def step_bf16(i):
        csa2.sparse_attn_decode(reps[i % R], st.q_idx, st.w, st.q[0],
                                st.swa[0], st.n_swa, k, st.scale,
                                pool=wl.pool, out=out, topk_out=ids, ws=ws)

    def step_mxfp4(i):
        csa2.sparse_attn_decode_fp4q(reps[i % R], qc, qs, st.w, st.q[0],
                                     st.swa[0], st.n_swa, k, st.scale,
                                     pool=wl.pool, out=out, topk_out=ids,
                                     ws=ws)

    # The V4 attention details on the same step: per-head sink logits and
    # the partial-RoPE output de-rotation at each sequence's position.
    g_sink = torch.linspace(-2.0, 2.0, 64, device=dev)
    g_pos = torch.full((wl.B,), wl.ctx - 1, dtype=torch.int32, device=dev)

    def step_epilogue(i):
        csa2.sparse_attn_decode(reps[i % R], st.q_idx, st.w, st.q[0],
                                st.swa[0], st.n_swa, k, st.scale,
                                pool=wl.pool, out=out, topk_out=ids, ws=ws,
                                sink=g_sink, pos=g_pos)

    steps = {"bf16": step_bf16, "mxfp4": step_mxfp4,
             "sink_rope": step_epilogue}
    if not wl.pool:
        # The pages' hierarchical decoder group on the same caches: the first
        # Full layer also emitting the max-of-fine-scores pool (2,048 blocks
        # of 8), and a Reindex layer scoring only that pool with its own
        # indexer query.
        from fp4_kv_cache_amd import inputs
        group_pool = (2048, 8)
        pool_ids = torch.empty((wl.B, group_pool[0] * group_pool[1]),
                               dtype=torch.int32, device=dev)
        ws_fp = csa2.workspace(csa2.load().csa2_workspace_size(
            csa2.OP_FULL_POOL, wl.B, wl.n, k,
            csa2.ctypes.byref(csa2.PoolOpts(*group_pool))), dev)
        ws_ri = csa2.workspace(csa2.load().csa2_workspace_size(
            csa2.OP_REINDEX, wl.B, pool_ids.shape[1], k, None), dev)
        qi1, w1 = (torch.stack(t).contiguous() for t in zip(*[
            inputs.index_query(wl, b, dev, layer=1) for b in range(wl.B)]))

        def step_full_pool(i):
            csa2.full_pool_decode(reps[i % R], st.q_idx, st.w, st.q[0],
                                  st.swa[0], st.n_swa, k, st.scale,
                                  pool=group_pool, out=out, topk_out=ids,
                                  pool_out=pool_ids, ws=ws_fp)

        def step_reindex(i):
            csa2.reindex_decode(reps[i % R], pool_ids, qi1, w1, st.q[0],
                                st.swa[0], st.n_swa, k, st.scale, out=out,
                                topk_out=ids, ws=ws_ri)

        steps["full_pool"] = step_full_pool
        steps["reindex"] = step_reindex
    # The write path at decode: one new entry per sequence from the m newest
    # tokens' hidden states (d = 7168, the pages' model width), appended to
    # caches of its own (the timed steps' caches stay as they are).
    from fp4_kv_cache_amd import inputs as inp
    cm, cd = wl.m, 7168
    c_h = inp.hidden_states(900, wl.B, cm, cd, dev)
    c_w = inp.compressor_weights(900, cd, dev)
    c_rows = torch.zeros((wl.B,), dtype=torch.int32, device=dev)
    c_slot = torch.zeros((wl.B,), dtype=torch.int32, device=dev)
    c_bufs = [torch.zeros(sh, dtype=torch.uint8, device=dev)
              for sh in ((wl.B, 1, 256), (wl.B, 1, 32), (wl.B, 1, 64),
                         (wl.B, 1, 4), (wl.B, 128, 512))]
    c_ws = csa2.workspace(csa2.load().csa2_workspace_size(
        csa2.OP_COMPRESS, wl.B, cm, cd, None), dev)

    def step_compress(i):
        csa2.compress_append(c_h, *c_w, c_rows, *c_bufs[:4], swa=c_bufs[4],
                             swa_slot=c_slot, ws=c_ws)

    steps["compress"] = step_compress
    compress_bytes = (2 * 512 * cd * 2 + 128 * 512 * 2 + wl.B * cm * cd * 2
                      + wl.B * (288 + 68 + cm * 512))
    timing = {q: time_steps(fn, args, R, out, ids) for q, fn in steps.items()}

    # -- per-kernel durations with HIP events on the launch stream: the same
    # kernels through the component calls, M back-to-back launches of one
    # kernel queued behind a spin kernel (so host enqueue time is hidden),
    # rotated over the replicas.
    # The scan kernel: the MXFP4 indexer over every entry, or, for the
    # hierarchical workload, the bf16 block-key scan (its top-k keeps
    # n_keep blocks expanded by the block size).
    if wl.pool:
        ld = n_blocks(wl)
        nvalid = torch.full((wl.B,), ld, dtype=torch.int32, device=dev)
        tk_k, tk_block = min(wl.pool[0], ld), wl.pool[1]
    else:
        ld, nvalid, tk_k, tk_block = wl.n, st.n_entries, k, 1
    scores = torch.empty((wl.B, ld), dtype=torch.float32, device=dev)
    tk_out = torch.empty((wl.B, tk_k * tk_block), dtype=torch.int32, device=dev)
    tk_ws = csa2.workspace(csa2.workspace_size(csa2.OP_TOPK, wl.B, ld, tk_k), dev)
    at_ws = csa2.workspace(csa2.workspace_size(csa2.OP_REUSE, wl.B, wl.n, k), dev)

    def k_idx(r, query="bf16"):
        pl = planes[r]
        kf, kc, ks = ((csa2.KEYS_BF16, pl[4], None) if wl.pool
                      else (csa2.KEYS_MXFP4, pl[2], pl[3]))
        if query == "mxfp4":
            csa2.indexer_score_fp4q(kf, kc, ks, nvalid, qc, qs, st.w,
                                    out=scores)
        else:
            csa2.indexer_score(kf, kc, ks, nvalid, st.q_idx, st.w, out=scores)

    def k_topk(r):
        csa2.topk(scores, tk_k, n_valid=nvalid, block=tk_block,
                  limit=st.n_entries if wl.pool else None, out=tk_out,
                  ws=tk_ws)

    def k_attn(r):
        csa2.reuse_attn(planes[r][0], planes[r][1], ids, st.q[0],
                        st.swa[0], st.n_swa, st.scale, out=out, ws=at_ws)

    def timed(fn, M):
        for r in range(R):
            fn(r)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(200_000_000)
        e0.record()
        for i in range(M):
            fn(i % R)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / M

    M = max(8, min(args.steps, 200))
    k_idx(0)
    t_idx = {"bf16": timed(k_idx, M),
             "mxfp4": timed(lambda r: k_idx(r, "mxfp4"), M)}
    t_tk = timed(k_topk, M)
    t_at = timed(k_attn, M)
    return dict(timing=timing, t_idx=t_idx, t_topk=t_tk, t_attn=t_at,
                replicas=R, st=st, compress=(cm, cd, compress_bytes))


COPY_ELEMS = 64 << 20          # float32 elements of the calibration copy


def run_pmc_pass(args, wl):
    """Launch sequence for rocprofv3 --pmc: M plain indexer launches with
    the bf16 query, then M with the MXFP4 query (the roofline kernels, same
    arguments as the timed ones), then 4 copies
    y = x * 1 over COPY_ELEMS float32 (a kernel whose HBM bytes are known:
    4 * COPY_ELEMS read and written), then M eager decode steps with the
    bf16 query (the counters of the attention, select and merge kernels)."""
    import torch
    from fp4_kv_cache_amd import csa2, workload

    dev = "cuda:0"
    st = workload.build(wl, dev)
    per_call = wl.B * algorithmic_bytes(wl)
    R = args.replicas or max(1, math.ceil(2 * 256e6 / per_call) + 1)
    reps, planes = replicate(st, R)
    scores = torch.empty((wl.B, wl.n), dtype=torch.float32, device=dev)
    qc, qs = csa2.pack_query_fp4(st.q_idx)
    M = max(8, min(args.steps, 64))
    for i in range(M):
        pl = planes[i % R]
        csa2.indexer_score(csa2.KEYS_MXFP4, pl[2], pl[3], st.n_entries,
                           st.q_idx, st.w, out=scores)
    for i in range(M):
        pl = planes[i % R]
        csa2.indexer_score_fp4q(csa2.KEYS_MXFP4, pl[2], pl[3], st.n_entries,
                                qc, qs, st.w, out=scores)
    torch.cuda.synchronize()
    x = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(4):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    del x, y
    if not wl.pool:
        out = torch.empty((wl.B, 64, 512), dtype=torch.bfloat16, device=dev)
        ids = torch.empty((wl.B, wl.k), dtype=torch.int32, device=dev)
        ws = csa2.workspace(csa2.workspace_size(csa2.OP_DECODE, wl.B, wl.n,
                                                wl.k, None), dev)
        for i in range(M):
            csa2.sparse_attn_decode(reps[i % R], st.q_idx, st.w, st.q[0],
                                    st.swa[0], st.n_swa, wl.k, st.scale,
                                    out=out, topk_out=ids, ws=ws)
        torch.cuda.synchronize()
    print(json.dumps({"pmc_pass": True, "indexer_launches": M,
                      "decode_steps": 0 if wl.pool else M,
                      "indexer_algorithmic_bytes": {
                          q: indexer_bytes(wl, q) for q in ("bf16", "mxfp4")},
                      "copy_bytes_each_way": 4 * COPY_ELEMS}))


def run_cpu(wl, budget_s):
    """The oracle as it stands, on a bounded sample of the same workload:
    whole sequences (indexer over all entries, exact top-k, gather and
    attention) until ~budget_s of work; packing is not timed."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from fp4_kv_cache_amd import inputs
    from oracle import csa2 as O

    cores = len(os.sched_getaffinity(0))
    dev = "cuda:0" if torch.cuda.is_available() else "cpu"
    bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    done, spent = 0, 0.0
    with threadpool_limits(limits=cores):
        for b in range(wl.B):
            ic, isc = O.pack_idx(inputs.idx_latents(wl, b, 0, wl.n, dev).cpu().numpy())
            qi, w = inputs.index_query(wl, b, dev)
            q = bits(inputs.attn_query(wl, b, 0, dev))
            sw = O.pack_swa(inputs.window_latents(wl, b, 0, dev).cpu().numpy())
            qi, w = bits(qi), w.cpu().numpy()
            # Packing is the write path (untimed); only the main rows this
            # query will read need packing, found by an untimed oracle pass.
            if wl.pool:
                bk = O.block_keys(ic, isc, wl.n, wl.pool[1])
                sel = O.hier_layer(np.zeros((wl.n, 256), np.uint8),
                                   np.zeros((wl.n, 32), np.uint8), ic, isc, bk,
                                   wl.n, qi, w, q, sw, wl.n_swa, wl.k, 1.0,
                                   n_keep=wl.pool[0], block=wl.pool[1])[0]
            else:
                sel = O.topk(O.indexer_scores(qi, w, O.unpack_idx(ic, isc)),
                             wl.k)
            sel = sel[sel >= 0]
            lat = inputs.main_latents(wl, b, 0, wl.n, dev)[
                torch.from_numpy(sel).to(dev)].cpu().numpy()
            mc = np.zeros((wl.n, 256), np.uint8)
            ms = np.zeros((wl.n, 32), np.uint8)
            mc[sel], ms[sel] = O.pack_main(lat)
            scale = float(np.float32(1 / math.sqrt(512)))
            t0 = time.perf_counter()
            if wl.pool:
                O.hier_layer(mc, ms, ic, isc, bk, wl.n, qi, w, q, sw,
                             wl.n_swa, wl.k, scale, n_keep=wl.pool[0],
                             block=wl.pool[1])
            else:
                O.full_layer(mc, ms, ic, isc, wl.n, qi, w, q, sw, wl.n_swa,
                             wl.k, scale)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget_s:
                break
    return dict(value=done / spent, unit="query-tokens/s", cores=cores,
                kind="oracle",
                sample=f"{done} of {wl.B} sequences of {wl.name} "
                       f"({'hierarchical' if wl.pool else 'full'} layer each, {spent:.1f} s, float64 NumPy, "
                       f"BLAS threads={cores}, cpu={platform.processor() or 'x86_64'})")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (got --gpus "
              f"{args.gpus}); the decode is not sharded across GPUs",
              file=sys.stderr)
        sys.exit(2)
    from fp4_kv_cache_amd.inputs import WORKLOADS
    wl = WORKLOADS[args.workload]
    if args.pmc_pass:
        run_pmc_pass(args, wl)
        return
    g = run_gpu(args, wl)
    scan_name = ("indexer_kernel<1, *, Q> (bf16 block-key scan)" if wl.pool
                 else "indexer_kernel<0, *, Q> (MXFP4 scan)")

    def summary(query):
        eager_s, graph_s, steps_run, spread = g["timing"][query]
        step_s = graph_s if graph_s is not None else eager_s
        idx_alg = indexer_bytes(wl, query)
        achieved = idx_alg / g["t_idx"][query] / 1e9
        per_call = wl.B * algorithmic_bytes(wl, query)
        qf = "true" if query == "mxfp4" else "false"
        return dict(
            step_s=step_s, eager_s=eager_s, graph_s=graph_s,
            steps_run=steps_run, per_call=per_call, spread=spread,
            roofline={"bound": "hbm", "achieved": achieved,
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": achieved / HBM_PEAK_GBS,
                      "traffic": (traffic_from_profile(query)
                                  if args.workload == 1 else None),
                      "kernel": scan_name.replace("Q", qf),
                      "algorithmic_bytes_per_launch": idx_alg,
                      "avg_launch_us": g["t_idx"][query] * 1e6})

    head = summary(args.query)
    other = "mxfp4" if args.query == "bf16" else "bf16"
    alt = summary(other)
    step_s = head["step_s"]
    line = {
        "metric": "CSA2 decode query-tokens/s per layer at 64K ctx; "
                  "achieved HBM GB/s vs peak",
        "value": wl.B / step_s,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": head["steps_run"],
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents packed to FP4/MXFP4/E4M3)",
        "config": {"workload": wl.name, "global_batch": wl.B,
                   "entries_per_seq": wl.n, "context": wl.ctx, "m": wl.m,
                   "k": wl.k, "n_swa": wl.n_swa, "heads": 64,
                   "head_dim": 512, "indexer": "32 heads x 128, MXFP4 keys",
                   "indexer_query": args.query,
                   "pool": list(wl.pool) if wl.pool else None,
                   "cache_replicas": g["replicas"],
                   "launch": "hip-graph" if head["graph_s"] else "eager"},
        "roofline": head["roofline"],
        "step_hbm": {"algorithmic_bytes": head["per_call"],
                     "achieved_GBs": head["per_call"] / step_s / 1e9,
                     "frac": head["per_call"] / step_s / 1e9 / HBM_PEAK_GBS},
        "kernels_us": {"indexer": g["t_idx"][args.query] * 1e6,
                       "topk": g["t_topk"] * 1e6,
                       "attention": g["t_attn"] * 1e6},
        "eager_ms_per_step": head["eager_s"] * 1e3,
        "graph_step_us_spread": head["spread"],
        "variants": {f"indexer_query_{other}": {
            "value": wl.B / alt["step_s"], "ms_per_step": alt["step_s"] * 1e3,
            "roofline": alt["roofline"]}},
    }
    ep = g["timing"]["sink_rope"]
    ep_s = ep[1] if ep[1] is not None else ep[0]
    line["variants"]["attn_sink_rope"] = {
        "value": wl.B / ep_s, "ms_per_step": ep_s * 1e3,
        "what": "the headline step with per-head sink logits and the "
                "partial-RoPE output de-rotation (csa2_sparse_attn_decode_ex)"}
    cp = g["timing"]["compress"]
    cp_s = cp[1] if cp[1] is not None else cp[0]
    cm, cd, cbytes = g["compress"]
    line["variants"]["compress_append"] = {
        "value": wl.B / cp_s, "ms_per_step": cp_s * 1e3, "m": cm, "d": cd,
        "algorithmic_bytes": cbytes,
        "achieved_GBs": cbytes / cp_s / 1e9,
        "what": "csa2_compress_append: one new entry per sequence (C, Z "
                "projections, softmax pooling, K^I, FP4/MXFP4/E4M3 append)"}
    if "full_pool" in g["timing"]:
        fp, ri = (g["timing"][x] for x in ("full_pool", "reindex"))
        fp_s = fp[1] if fp[1] is not None else fp[0]
        ri_s = ri[1] if ri[1] is not None else ri[0]
        line["variants"]["decoder_group_pool"] = {
            "pool": [2048, 8],
            "full_pool_layer": {"value": wl.B / fp_s, "ms_per_step": fp_s * 1e3},
            "reindex_layer": {"value": wl.B / ri_s, "ms_per_step": ri_s * 1e3,
                              "scored_entries_per_seq": 2048 * 8},
            "unit": "query-tokens/s"}
    if not args.no_cpu:
        cpu = run_cpu(wl, args.cpu_seconds)
        line["cpu_baseline"] = cpu
    print(json.dumps(line))


if __name__ == "__main__":
    main()
