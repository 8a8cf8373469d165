"""Benchmark of one YOCO cross-decoder step on one MI355X.

A step is one pass of the whole hot path over one batch: yoco_kv_append of the
step's new tokens into the shared cache, yoco_gather_last of each request's
last row, then the L cross layers in order, each one yoco_cross_attn over the
same cache (layer l walks its work items in reverse when l is odd, so a layer
starts where the previous one ended in the last-level cache).

Default workload: decode32x32k -- 32 decoding requests at 32768 tokens of
context each, bf16 cache of 8 KV heads x 128 dims in blocks of 16 (0.1% of key
vectors scaled by 20), 16 cross layers of 32 query heads, hidden 3072; the
largest single-GPU workload and the long-context case.  Inputs are synthetic
and seeded and sit in HBM before timing starts.  Between steps a 1 GiB buffer
is read so the L2s and the 256 MB last-level cache start cold each step (other
model work would evict them); that read is outside the step's events.

The CPU baseline runs the float64 oracle on the host's cores: worker
processes (started before the GPU is touched, one BLAS thread each) each own
a share of the (request, KV head) groups, hold those groups' K/V rows, and
compute every layer's attention for them.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "cross-attn decode tokens/s & achieved HBM GB/s (% of 8 TB/s) on 1 MI355X"
HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=3, help="synthetic workload id (1-5); 3 = decode32x32k")
    p.add_argument("--partition-tokens", type=int, default=0, help="0 = library default")
    p.add_argument("--query-rows", type=int, default=1, help="query rows per request (decode workloads 2, 3, 5)")
    p.add_argument("--window", type=int, default=0, help="sliding window of every cross layer in tokens (0 = none)")
    p.add_argument("--fp8", action="store_true", help="8-bit shared cache (FP8 E4M3 codes, per-row scales)")
    p.add_argument("--retention", choices=["mixed48", "decode64"], default=None,
                   help="time the self-decoder's gated retention instead (16 layers, 24 heads x 128) over the "
                        "mixed step's rows or 64 decode tokens")
    p.add_argument("--no-flush", action="store_true", help="keep the last-level cache warm between steps")
    p.add_argument("--vector-kernel", action="store_true",
                   help="run the vector-ALU attention kernel where the matrix-core kernel is the default "
                        "(YOCO_FLAG_VECTOR_KERNEL; for comparison)")
    p.add_argument("--no-alternate", action="store_true",
                   help="every cross layer walks its work items in the same order (no last-level-cache reuse "
                        "between consecutive layers; for comparison)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle baseline")
    p.add_argument("--cpu-workers", type=int, default=0,
                   help="worker processes of the CPU baseline (0 = the usable host cores, at most 16)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--seed", type=int, default=2024)
    p.add_argument("--append-reference", action="store_true",
                   help="only time yoco_kv_append of the workload's step against torch.mm (the vendor GEMM library) "
                        "on the same [tokens x hidden] x [hidden x 2*Hkv*D] bf16 product")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB mebibytes (reference for HBM byte counters)")
    return p.parse_args()


MFMA_BF16_PEAK_TFLOPS = 2500.0


def append_reference(args):
    """yoco_kv_append of the step's tokens (RMSNorm, the fused K/V projection,
    the scatter into the cache) against a plain torch.mm of the same shape
    (no normalisation, no scatter): both timed with events over 10 calls after
    3 warm-up calls, the last-level cache flushed by a 1 GiB read before
    each call."""
    import torch

    from yoco_shared_kv_gather_amd import binding as yb
    from yoco_shared_kv_gather_amd import synth

    dev = torch.device("cuda", 0)
    meta = synth.make_metadata(args.workload, "full", args.seed)
    geom = meta.geom
    k, v = synth.make_cache(meta, dev, args.seed)
    x, w_rms, w_k, w_v = synth.make_append_inputs(meta, dev, args.seed)
    slots = torch.from_numpy(meta.slot_mapping).to(dev)
    code = yb.DTYPE_BF16 if geom.dtype == "bf16" else yb.DTYPE_F32
    ws = torch.zeros(max(16, yb.kv_append_workspace_size(code, geom.hidden, geom.num_kv_heads, geom.head_dim)),
                     dtype=torch.uint8, device=dev)
    w_t = torch.cat([w_k, w_v], 0).t().contiguous()            # [hidden][2*Hkv*D]
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(3):
            flush.sum(dtype=torch.int64)
            fn()
        times = []
        for _ in range(10):
            flush.sum(dtype=torch.int64)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        return float(np.mean(times))

    ours = timed(lambda: yb.kv_append(x, w_rms, 1e-6, w_k, w_v, slots, k, v, workspace=ws, stream=stream))
    ref = timed(lambda: torch.mm(x, w_t))
    flops = 2.0 * meta.num_tokens * geom.hidden * 2 * geom.num_kv_heads * geom.head_dim
    out = {"workload": geom.name, "tokens": meta.num_tokens, "hidden": geom.hidden,
           "features": 2 * geom.num_kv_heads * geom.head_dim, "tflop": round(flops / 1e12, 4),
           "yoco_kv_append_us": round(ours, 2), "yoco_kv_append_tflops": round(flops / ours / 1e6, 1),
           "yoco_kv_append_frac_of_2.5pf": round(flops / ours / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
           "torch_mm_us": round(ref, 2), "torch_mm_tflops": round(flops / ref / 1e6, 1),
           "torch_mm_frac_of_2.5pf": round(flops / ref / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}
    print(json.dumps(out), flush=True)


def copy_calibration(mib):
    """A plain copy of known size: reads and writes mib MiB once per launch.
    Its FETCH_SIZE/WRITE_SIZE counter readings scale the counters of the
    hot-path kernels to bytes."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host's cores
# ---------------------------------------------------------------------------

def host_cores():
    """(os.cpu_count(), usable cores from the affinity mask)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return os.cpu_count() or 1, usable


def _oracle_worker(conn):
    """Worker process of the CPU baseline: holds the K/V rows (or retention
    slices) of its share of the groups and runs the oracle on them when asked.
    One BLAS thread per worker: the workers are the parallelism."""
    import threadpoolctl

    threadpoolctl.threadpool_limits(limits=1)
    import oracle

    groups = {}
    while True:
        msg = conn.recv()
        kind = msg[0]
        if kind == "stop":
            break
        if kind == "load":
            groups[msg[1]] = msg[2]
            conn.send(None)
        elif kind == "attn":
            # msg[1]: list of (group key, q rows [Q][G][D]); msg[2]: (scale, window, varlen)
            scale, window, varlen = msg[2]
            t0 = time.perf_counter()
            for key, qg in msg[1]:
                n, nb, kc, vc = groups[key]
                table = np.arange(max(nb, 1))[None, :]
                if varlen:
                    oracle.cross_attention_varlen(qg, kc, vc, table, np.array([n]), np.array([0, qg.shape[0]]),
                                                  scale, window)
                else:
                    oracle.cross_attention(qg, kc, vc, table, np.array([n]), scale)
            conn.send(time.perf_counter() - t0)
        elif kind == "retention":
            # msg[1]: group keys in order; msg[2]: seconds; each group is one (request, head) slice
            budget = msg[2]
            t0 = time.perf_counter()
            done = 0
            for key in msg[1]:
                q, k, v, g, s, idx = groups[key]
                oracle.gated_retention(q, k, v, g, np.array([0, q.shape[0]]), s, np.array([idx]))
                done += q.shape[0]
                if time.perf_counter() - t0 > budget:
                    break
            conn.send((done, time.perf_counter() - t0))


class OraclePool:
    """Worker processes for the CPU baseline.  They are forked before the
    process touches the GPU (a fork after HIP is initialised is not safe) and
    get their data through pipes during set-up, outside any timing."""

    def __init__(self, workers):
        import multiprocessing

        ctx = multiprocessing.get_context("fork")
        self.conns, self.procs = [], []
        for _ in range(workers):
            parent, child = ctx.Pipe()
            proc = ctx.Process(target=_oracle_worker, args=(child,), daemon=True)
            proc.start()
            child.close()
            self.conns.append(parent)
            self.procs.append(proc)

    @property
    def size(self):
        return len(self.conns)

    def load(self, worker, key, value):
        self.conns[worker].send(("load", key, value))
        self.conns[worker].recv()

    def run(self, per_worker, kind, arg):
        """Send every worker its share at once, wait for all; returns the
        replies (workers with an empty share are not asked)."""
        busy = [w for w in range(self.size) if per_worker[w]]
        for w in busy:
            self.conns[w].send((kind, per_worker[w], arg))
        return [self.conns[w].recv() for w in busy]

    def close(self):
        for c in self.conns:
            try:
                c.send(("stop",))
            except (BrokenPipeError, OSError):
                pass
        for p in self.procs:
            p.join(timeout=10)


def start_cpu_pool(args):
    """The CPU baseline's workers: one per usable core, at most 16 (about one
    GPU's share of a multi-GPU host's CPUs)."""
    if args.no_cpu_baseline:
        return None
    _, usable = host_cores()
    workers = args.cpu_workers if args.cpu_workers > 0 else min(usable, 16)
    return OraclePool(max(1, workers))


def _balance(sizes, workers):
    """Assign items (largest first) to the least loaded worker."""
    order = sorted(range(len(sizes)), key=lambda i: -sizes[i])
    load = [0] * workers
    share = [[] for _ in range(workers)]
    for i in order:
        w = min(range(workers), key=lambda j: load[j])
        share[w].append(i)
        load[w] += sizes[i]
    return share


def cpu_baseline(pool, meta, k, v, q, x, w_rms, w_k, w_v, budget_s, rows_per_req=1, window=0, ks=None, vs=None):
    """Time the float64 oracle on the host's cores on a bounded sample of the
    same step: the append and gather of all scheduled tokens (BLAS threads =
    the pool's size), then whole cross layers over every (request, KV head)
    group, spread over the worker processes, until the time budget is spent;
    the per-layer time is scaled to all L layers.  For the tiny and decode64
    workloads the same layer is also run on one thread."""
    import threadpoolctl
    import torch

    import oracle

    geom = meta.geom
    scale = 1.0 / math.sqrt(geom.head_dim)
    bs = geom.block_size
    hkv = geom.num_kv_heads
    group = geom.num_q_heads // hkv
    Q = rows_per_req
    varlen = Q > 1 or window > 0 or ks is not None
    cpu_count, usable = host_cores()
    workers = pool.size
    single = meta.config_id in (1, 2)
    w_host = (w_rms.float().cpu().numpy(), w_k.float().cpu().numpy(), w_v.float().cpu().numpy())
    x_host = x.float().cpu().numpy()
    # an 8-bit cache holds code * scale: the codes' values from the oracle's
    # decoder, once for all 256 codes (set-up, outside the timing)
    code_value = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)) if ks is not None else None
    keys = [(r, g) for r in range(meta.num_reqs) for g in range(hkv)]
    sizes = [max(int(meta.seq_lens[r]), 1) for r, _ in keys]
    share = _balance(sizes, workers)
    owner = {}
    for w, items in enumerate(share):
        for i in items:
            owner[keys[i]] = w
    kept = {}
    log(f"cpu baseline: handing {meta.num_reqs} requests' contexts ({len(keys)} groups) to {workers} workers")
    for r in range(meta.num_reqs):
        n = int(meta.seq_lens[r])
        nb = -(-n // bs)
        blocks = torch.from_numpy(meta.block_table[r, :max(nb, 1)].astype(np.int64)).to(k.device)
        if ks is not None:
            kc = code_value[k.index_select(0, blocks).cpu().numpy()] * \
                ks.index_select(0, blocks).cpu().numpy().astype(np.float64)[..., None]
            vc = code_value[v.index_select(0, blocks).cpu().numpy()] * \
                vs.index_select(0, blocks).cpu().numpy().astype(np.float64)[..., None]
        else:
            kc = k.index_select(0, blocks).float().cpu().numpy()
            vc = v.index_select(0, blocks).float().cpu().numpy()
        for g in range(hkv):
            item = (n, nb, np.ascontiguousarray(kc[:, g:g + 1]), np.ascontiguousarray(vc[:, g:g + 1]))
            pool.load(owner[(r, g)], (r, g), item)
            if single:
                kept[(r, g)] = item
        del kc, vc

    def append_gather():
        """Seconds of the step's append and gather (the 8-bit append's
        quantizer runs element by element in Python: a sample of at most 256
        tokens, scaled to all of them)."""
        t0 = time.perf_counter()
        append_scale = 1.0
        if ks is not None:
            n_s = min(meta.num_tokens, 256)
            oracle.kv_append_fp8(x_host[:n_s], w_host[0], 1e-6, w_host[1], w_host[2], meta.slot_mapping[:n_s],
                                 geom.num_kv_heads, geom.head_dim)
            append_scale = meta.num_tokens / max(n_s, 1)
        else:
            oracle.kv_project(x_host, w_host[0], 1e-6, w_host[1], w_host[2], geom.num_kv_heads, geom.head_dim)
        t_append = (time.perf_counter() - t0) * append_scale
        t0 = time.perf_counter()
        if Q > 1:
            idx = np.arange(meta.num_tokens)
            oracle.cross_metadata(idx, meta.cu_seqlens)
            oracle.gather_rows(x_host, idx)
        else:
            oracle.gather_last(x_host, meta.cu_seqlens)
        return t_append + time.perf_counter() - t0

    with threadpoolctl.threadpool_limits(limits=workers):
        t_other = append_gather()
    log(f"cpu baseline: append + gather {t_other:.1f} s; timing cross layers on {workers} workers")

    def layer_tasks(layer):
        qh = q[layer].float().cpu().numpy()
        per_worker = [[] for _ in range(workers)]
        for (r, g), w in owner.items():
            per_worker[w].append(((r, g), np.ascontiguousarray(qh[r * Q:(r + 1) * Q, g * group:(g + 1) * group])))
        return per_worker

    layers = 0
    t_attn = 0.0
    busiest = 0.0
    while layers < geom.num_layers and (layers == 0 or t_other + t_attn < budget_s):
        tasks = layer_tasks(layers)
        t1 = time.perf_counter()
        replies = pool.run(tasks, "attn", (scale, window, varlen))
        t_attn += time.perf_counter() - t1
        busiest = max(busiest, max(replies))
        layers += 1
    step_s = t_other + geom.num_layers * t_attn / layers
    used = sum(1 for items in share if items)
    result = {
        "value": round(meta.num_reqs * Q / step_s, 3),
        "unit": "tokens/s",
        "cores": used,
        "kind": "oracle",
        "cpu_count": cpu_count,
        "usable_cores": usable,
        "worker_processes": used,
        "blas_threads_per_worker": 1,
        "blas_threads_append": workers,
        "sample": (f"append + gather of all {meta.num_tokens} tokens"
                   + (f" (8-bit append timed on {min(meta.num_tokens, 256)} tokens and scaled)" if ks is not None
                      else "")
                   + f", then {layers} of {geom.num_layers} cross layers over all {len(keys)} (request, KV head) "
                   f"groups spread over {used} worker processes ({t_other + t_attn:.1f} s wall, float64 numpy); "
                   f"per-layer wall time scaled to {geom.num_layers} layers"),
    }
    if single:
        with threadpoolctl.threadpool_limits(limits=1):
            t_other1 = append_gather()
            qh = q[0].float().cpu().numpy()
            t0 = time.perf_counter()
            for (r, g), (n, nb, kc, vc) in kept.items():
                qg = qh[r * Q:(r + 1) * Q, g * group:(g + 1) * group]
                table = np.arange(max(nb, 1))[None, :]
                if varlen:
                    oracle.cross_attention_varlen(qg, kc, vc, table, np.array([n]), np.array([0, Q]), scale, window)
                else:
                    oracle.cross_attention(qg, kc, vc, table, np.array([n]), scale)
            t_layer1 = time.perf_counter() - t0
        result["single_thread_value"] = round(meta.num_reqs * Q / (t_other1 + geom.num_layers * t_layer1), 3)
        result["single_thread_sample"] = "the same append + gather and one cross layer on one thread, scaled to L"
    return result


def quantize_cache(meta, k, v, yb, torch):
    """The workload's bf16 cache rows, quantized into an FP8 cache with the
    library's own scatter (free blocks and tail slots keep NaN codes/scales)."""
    bs = meta.geom.block_size
    dev = k.device
    live = torch.from_numpy(synth_live(meta)).to(dev)
    slots = torch.nonzero(live.reshape(-1)).reshape(-1).to(torch.int32)
    kc = torch.full(k.shape, 0x7F, dtype=torch.uint8, device=dev)
    vc = torch.full(v.shape, 0x7F, dtype=torch.uint8, device=dev)
    ks = torch.full(k.shape[:-1], float("nan"), dtype=torch.float32, device=dev)
    vs = torch.full(v.shape[:-1], float("nan"), dtype=torch.float32, device=dev)
    step = 1 << 18
    for s0 in range(0, slots.numel(), step):
        sl = slots[s0:s0 + step]
        blk, off = (sl // bs).long(), (sl % bs).long()
        rk = k[blk, :, off].contiguous()
        rv = v[blk, :, off].contiguous()
        yb.kv_scatter(rk, rv, sl.contiguous(), kc, vc, ks, vs)
    torch.cuda.synchronize()
    return kc, vc, ks, vs


def synth_live(meta):
    from yoco_shared_kv_gather_amd import synth
    return synth.live_slot_mask(meta)


RETENTION_HEADS, RETENTION_DIM, RETENTION_LAYERS = 24, 128, 16


def retention_cpu_baseline(pool, layer, budget_s):
    """The float64 oracle's recurrence on (request, head) slices of one layer,
    spread over the worker processes (longest first on each), until the
    budget is spent; rows x heads per second, scaled to the whole pass."""
    lens = layer["lens"]
    cu = layer["cu"]
    keys = [(int(r), h) for r in np.argsort(-lens, kind="stable") if lens[r] > 0 for h in range(RETENTION_HEADS)]
    share = _balance([int(lens[r]) for r, _ in keys], pool.size)
    per_worker = []
    for w, items in enumerate(share):
        mine = []
        for i in items:
            r, h = keys[i]
            a, b = int(cu[r]), int(cu[r + 1])
            sl = lambda x: np.ascontiguousarray(x[a:b, h:h + 1])
            pool.load(w, (r, h), (sl(layer["q"]), sl(layer["k"]), sl(layer["v"]), sl(layer["g"]),
                                  np.ascontiguousarray(layer["s"][:, h:h + 1]), int(layer["idx"][r])))
            mine.append((r, h))
        per_worker.append(mine)
    t0 = time.perf_counter()
    replies = pool.run(per_worker, "retention", budget_s)
    elapsed = time.perf_counter() - t0
    done = sum(d for d, _ in replies)
    rate = done / elapsed                                 # rows x heads per second
    tokens_per_s = rate / (RETENTION_HEADS * RETENTION_LAYERS)
    cpu_count, usable = host_cores()
    log(f"CPU oracle: {done} row-heads in {elapsed:.1f} s on {len(replies)} workers")
    return {"value": round(tokens_per_s, 3), "unit": "tokens/s", "cores": len(replies), "kind": "oracle",
            "cpu_count": cpu_count, "usable_cores": usable, "worker_processes": len(replies),
            "blas_threads_per_worker": 1,
            "sample": f"the float64 recurrence on {done} (row, head) pairs of one layer ((request, head) slices "
                      f"longest first on {len(replies)} worker processes, {elapsed:.1f} s wall), scaled to "
                      f"{RETENTION_HEADS} heads x {RETENTION_LAYERS} layers"}


def bench_retention(args, pool):
    """One self-decoder pass: RETENTION_LAYERS gated-retention layers in order,
    each over the same rows with its own q, k, v, gates and state slots."""
    import torch

    from yoco_shared_kv_gather_amd import binding as yb
    from yoco_shared_kv_gather_amd import bytes_model as bm
    from yoco_shared_kv_gather_amd import profiling
    from yoco_shared_kv_gather_amd import synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    yb.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    H, D, L = RETENTION_HEADS, RETENTION_DIM, RETENTION_LAYERS
    lens = synth.retention_lengths(args.retention, args.seed)
    rows = int(lens.sum())
    log(f"retention workload {args.retention}: {len(lens)} requests, {rows} rows, {L} layers x {H} heads x {D}")
    layers = [synth.make_retention_inputs(lens, H, D, dev, seed=args.seed, tag=100 + l) for l in range(L)]
    cu = torch.from_numpy(layers[0].cu_seqlens).to(dev)
    idx = [torch.from_numpy(x.state_indices).to(dev) for x in layers]
    outs = [torch.empty((rows, H, D), dtype=torch.float32, device=dev) for _ in range(L)]
    max_seqlen = int(lens.max())
    ws = torch.empty(max(16, yb.gated_retention_workspace_size(rows, len(lens), H, D, max_seqlen)), dtype=torch.uint8,
                     device=dev)
    host_layer = None
    if not args.no_cpu_baseline:
        x = layers[0]
        host_layer = dict(lens=lens, cu=x.cu_seqlens, idx=x.state_indices, q=x.q.float().cpu().numpy(),
                          k=x.k.float().cpu().numpy(), v=x.v.float().cpu().numpy(), g=x.gamma.cpu().numpy(),
                          s=x.state.cpu().numpy())
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        for l in range(L):
            x = layers[l]
            yb.gated_retention(x.q, x.k, x.v, x.gamma, cu, x.state, idx[l], max_seqlen=max_seqlen, out=outs[l],
                               workspace=ws, stream=stream)

    for _ in range(args.warmup):
        if not args.no_flush:
            flush.sum(dtype=torch.int64)
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        if not args.no_flush:
            flush.sum(dtype=torch.int64)
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_per_step = float(step_ms.mean())
    call_us = ms_per_step * 1e3 / L
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (events), {call_us:.1f} us per layer")
    layer_bytes = bm.retention_layer_bytes(lens, layers[0].state_indices, H, D)
    layer_flops = bm.retention_layer_flops(lens, H, D)
    achieved = layer_bytes / (call_us * 1e-6) / 1e9
    # the schedule the library picks from max_seqlen: the recurrent kernel for
    # decode batches, one chunkwise run per request up to 1024 rows, else a
    # state pass over the segments of long requests and a full pass
    if max_seqlen == 1:
        kernels = [f"gated_retention_decode_kernel<{D}>"]
    elif max_seqlen <= 1024:
        kernels = [f"gated_retention_kernel<{D}, 0>"]
    else:
        kernels = [f"gated_retention_kernel<{D}, 1>", f"gated_retention_kernel<{D}, 2>"]
    kernel = " + ".join(kernels)
    variant = f"retention_{args.retention}"
    measured = profiling.measured_traffic(f"gated_retention_{args.retention}", kernels)
    traffic = profile_us = None
    if measured is not None:
        traffic = round(measured["read_bytes"] + measured["write_bytes"])
        profile_us = round(measured["kernel_us"], 2)
    result = {
        "metric": METRIC,
        "value": round(rows / (ms_per_step * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 q/k/v, fp32 state and outputs",
        "data": "synthetic",
        "config": {
            "workload": variant,
            "num_reqs": int(len(lens)),
            "rows": rows,
            "longest_request_rows": int(lens.max()),
            "num_layers": L,
            "num_heads": H,
            "head_dim": D,
            "chunk_tokens": 32,
            "segment_rows": 1024,
            "max_seqlen": max_seqlen,
            "llc_flushed_between_steps": not args.no_flush,
            "parallelism": "single GPU",
        },
        "wall_ms_per_step": round(1e3 * wall / args.steps, 4),
        "mfma_tflops_recurrence": round(layer_flops / (call_us * 1e-6) / 1e12, 2),
        "roofline": {
            "kernel": f"yoco_gated_retention: {kernel}",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": layer_bytes,
            "avg_launch_us": round(call_us, 2),
            "profile_kernel_us": profile_us,
        },
    }
    if host_layer is not None:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = retention_cpu_baseline(pool, host_layer, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.append_reference:
        append_reference(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    # the CPU baseline's workers are forked here, before anything touches the GPU
    pool = start_cpu_pool(args)
    try:
        if args.retention:
            bench_retention(args, pool)
        else:
            bench_cross(args, pool)
    finally:
        if pool is not None:
            pool.close()


def bench_cross(args, pool):
    """One cross-decoder step of the chosen workload (module docstring)."""

    import torch

    from yoco_shared_kv_gather_amd import binding as yb
    from yoco_shared_kv_gather_amd import bytes_model as bm
    from yoco_shared_kv_gather_amd import profiling
    from yoco_shared_kv_gather_amd import synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    yb.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    meta = synth.make_metadata(args.workload, "full", args.seed)
    Q, W = args.query_rows, args.window
    varlen = Q > 1 or W > 0 or args.fp8
    if Q > 1:
        if args.workload not in (2, 3, 5):
            log("--query-rows applies to the decode workloads 2, 3 and 5")
            sys.exit(2)
        meta = synth.with_query_rows(meta, Q)
    geom = meta.geom
    R = meta.num_reqs
    num_rows = R * Q
    log(f"workload {geom.name}: {R} requests, {int(meta.seq_lens.sum())} context tokens, "
        f"{geom.num_layers} layers, {Q} query rows per request, window {W}")
    k, v = synth.make_cache(meta, dev, args.seed)
    ks = vs = None
    if args.fp8:
        if geom.dtype != "bf16":
            log("--fp8 needs a bf16 workload")
            sys.exit(2)
        k, v, ks, vs = quantize_cache(meta, k, v, yb, torch)
    q = synth.make_queries(meta, dev, args.seed, rows=num_rows)
    x, w_rms, w_k, w_v = synth.make_append_inputs(meta, dev, args.seed)
    table = torch.from_numpy(meta.block_table).to(dev)
    seq = torch.from_numpy(meta.seq_lens).to(dev)
    cu = torch.from_numpy(meta.cu_seqlens).to(dev)
    slots = torch.from_numpy(meta.slot_mapping).to(dev)
    code = yb.DTYPE_BF16 if geom.dtype == "bf16" else yb.DTYPE_F32
    attn_dtype = yb.DTYPE_FP8_E4M3 if args.fp8 else code
    part, piece, tail, nparts = yb.cross_attn_partition_split(R, geom.num_kv_heads, geom.head_dim, meta.max_seq_len,
                                                              geom.block_size, args.partition_tokens, attn_dtype,
                                                              Q if varlen else 1, W,
                                                              yb.FLAG_VECTOR_KERNEL if args.vector_kernel else 0)
    if varlen:
        ws_bytes = yb.cross_attn_varlen_workspace_size(num_rows, R, geom.num_q_heads, geom.num_kv_heads,
                                                       geom.head_dim, meta.max_seq_len, Q, W, geom.block_size,
                                                       args.partition_tokens)
    else:
        ws_bytes = yb.cross_attn_workspace_size(R, geom.num_q_heads, geom.num_kv_heads, geom.head_dim,
                                                meta.max_seq_len, geom.block_size, args.partition_tokens)
    ws = torch.zeros(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    if args.fp8:
        ws_append_bytes = yb.kv_append_fp8_workspace_size(code, meta.num_tokens, geom.hidden, geom.num_kv_heads,
                                                          geom.head_dim)
    else:
        ws_append_bytes = yb.kv_append_workspace_size(code, geom.hidden, geom.num_kv_heads, geom.head_dim)
    ws_append = torch.zeros(max(16, ws_append_bytes), dtype=torch.uint8, device=dev)
    outs = torch.empty((geom.num_layers, num_rows, geom.num_q_heads, geom.head_dim), dtype=torch.float32, device=dev)
    rows = torch.empty((num_rows, geom.hidden), dtype=x.dtype, device=dev)
    rows_idx = torch.empty(R, dtype=torch.int32, device=dev)
    logits_idx = torch.arange(num_rows, dtype=torch.int32, device=dev)     # every scheduled row is verified
    cross_qsl = torch.empty(R + 1, dtype=torch.int32, device=dev)
    cross_max = torch.empty(1, dtype=torch.int32, device=dev)
    # Between steps, read 1 GiB of other memory: that evicts the cache from the
    # L2s and the last-level cache without leaving dirty lines behind (a fill
    # would, and writing them back would slow the first kernel of the step).
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    L = geom.num_layers

    def order(layer):
        """Work order of a layer: odd layers reversed, so each layer starts on
        the blocks the previous one read last (unless --no-alternate)."""
        force = yb.FLAG_VECTOR_KERNEL if args.vector_kernel else 0
        return force | (0 if args.no_alternate else (layer & 1) * yb.FLAG_REVERSE_ORDER)

    def step(ev_layers_start=None):
        if args.fp8:
            yb.kv_append_fp8(x, w_rms, 1e-6, w_k, w_v, slots, k, v, ks, vs, workspace=ws_append, stream=stream)
        else:
            yb.kv_append(x, w_rms, 1e-6, w_k, w_v, slots, k, v, workspace=ws_append, stream=stream)
        if Q > 1:
            yb.gather_logits(x, logits_idx, cu, out=rows, out_query_start_loc=cross_qsl, out_max_query_len=cross_max,
                             stream=stream)
        else:
            yb.gather_last(x, cu, out=rows[:R], out_index=rows_idx, stream=stream)
        if ev_layers_start is not None:
            ev_layers_start.record(stream)
        for l in range(L):
            if varlen:
                yb.cross_attn_varlen(q[l], k, v, table, seq, meta.max_seq_len,
                                     query_start_loc=cross_qsl if Q > 1 else None, max_query_len=Q, window=W,
                                     partition_tokens=args.partition_tokens, flags=order(l), out=outs[l],
                                     workspace=ws, stream=stream, k_scale=ks, v_scale=vs)
            else:
                yb.cross_attn(q[l], k, v, table, seq, meta.max_seq_len, partition_tokens=args.partition_tokens,
                              flags=order(l), out=outs[l], workspace=ws, stream=stream)

    for i in range(args.warmup):
        if not args.no_flush:
            flush.sum(dtype=torch.int64)
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); partition_tokens {part} (last {tail} tokens in pieces of {piece}), "
        f"at most {nparts} partitions per request")

    # Three events per step: step start, start of the cross layers, step end
    # (an event between every layer would add its own gap to every call).
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if not args.no_flush:
            flush.sum(dtype=torch.int64)
        ev[i][0].record(stream)
        step(ev[i][1])
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(c) for a, _, c in ev])
    layer_ms = np.array([b.elapsed_time(c) / L for _, b, c in ev])    # average call, inter-layer gaps included
    head_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])         # the step's append + gather
    ms_per_step = float(step_ms.mean())
    tokens_per_s = num_rows / (ms_per_step * 1e-3)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (events), wall {1e3 * wall / args.steps:.3f} ms/step")

    cache_bytes = 1 if args.fp8 else geom.elem_bytes
    layer_bytes = bm.attn_layer_bytes(meta.seq_lens, geom.num_q_heads, geom.num_kv_heads, geom.head_dim,
                                      geom.block_size, cache_bytes, query_lens=meta.query_lens if Q > 1 else None,
                                      window=W, q_bytes=geom.elem_bytes, scale_bytes=8 if args.fp8 else 0)
    written = int((meta.slot_mapping >= 0).sum())
    step_bytes = (L * layer_bytes
                  + bm.append_bytes(meta.num_tokens, geom.hidden, geom.num_kv_heads, geom.head_dim, geom.elem_bytes,
                                    written)
                  - (written * 2 * geom.num_kv_heads * geom.head_dim * (geom.elem_bytes - 1) if args.fp8 else 0)
                  + bm.gather_bytes(num_rows, geom.hidden * geom.elem_bytes))
    attn_us = float(layer_ms.mean()) * 1e3
    achieved = layer_bytes / (attn_us * 1e-6) / 1e9
    group = geom.num_q_heads // geom.num_kv_heads
    # the kernel the library picks for this call
    mfma = yb.cross_attn_kernel(R, geom.num_kv_heads, geom.head_dim, meta.max_seq_len, geom.block_size,
                                args.partition_tokens, attn_dtype, Q, W,
                                yb.FLAG_VECTOR_KERNEL if args.vector_kernel else 0) == "matrix"
    rows_per_item = 0 if Q == 1 else (16 if mfma else 8) // group
    elem_type = 2 if args.fp8 else (1 if geom.dtype == "bf16" else 0)
    kname = "cross_attn_mfma_kernel" if mfma else "cross_attn_kernel"
    attn_kernel = f"{kname}<{elem_type}, {geom.head_dim}, {group}, {rows_per_item}>"
    merge_split = 1
    triples = R * Q * geom.num_q_heads
    while merge_split < 8 and triples * merge_split < 512 and geom.head_dim // 4 // (merge_split * 2) >= 8:
        merge_split *= 2
    merge_kernel = f"cross_attn_merge_kernel<{geom.head_dim}, {merge_split}>"
    variant = geom.name + (f"_q{Q}" if Q > 1 else "") + (f"_w{W}" if W > 0 else "") + ("_fp8" if args.fp8 else "")
    measured = profiling.measured_traffic(f"cross_attn_{variant}", [attn_kernel, merge_kernel] if nparts > 1 else [attn_kernel])
    traffic = None
    profile_us = None
    if measured is not None:
        traffic = round(measured["read_bytes"] + measured["write_bytes"])
        profile_us = round(measured["kernel_us"], 2)
        log(f"HBM traffic per call from {measured['profile']}: {traffic / 1e6:.1f} MB "
            f"(algorithmic {layer_bytes / 1e6:.1f} MB)")
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 cache, bf16 queries" if args.fp8 else geom.dtype,
        "data": "synthetic",
        "config": {
            "workload": variant,
            "num_reqs": R,
            "query_rows_per_request": Q,
            "window": W,
            "context_tokens": int(meta.seq_lens.sum()),
            "num_layers": L,
            "num_q_heads": geom.num_q_heads,
            "num_kv_heads": geom.num_kv_heads,
            "head_dim": geom.head_dim,
            "block_size": geom.block_size,
            "hidden": geom.hidden,
            "partition_tokens": part,
            "partitions_per_request": nparts,
            "piece_tokens": piece,
            "tail_tokens": tail,
            "llc_flushed_between_steps": not args.no_flush,
            "alternating_layer_order": not args.no_alternate,
            "parallelism": "single GPU",
        },
        "append_gather_us": round(float(head_ms.mean()) * 1e3, 2),
        "append_tflops": round(2.0 * meta.num_tokens * geom.hidden * 2 * geom.num_kv_heads * geom.head_dim /
                               (float(head_ms.mean()) * 1e-3) / 1e12, 2),
        "step_hbm_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "wall_ms_per_step": round(1e3 * wall / args.steps, 4),
        "roofline": {
            "kernel": f"{'yoco_cross_attn_varlen' if varlen else 'yoco_cross_attn'}: {attn_kernel} + {merge_kernel}",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": layer_bytes,
            "avg_launch_us": round(attn_us, 2),
            # the same kernels' summed average durations in the committed
            # rocprofv3 trace (avg_launch_us is the span of the L serial
            # calls over L, so it also holds the gaps between the kernels)
            "profile_kernel_us": profile_us,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(pool, meta, k, v, q, x, w_rms, w_k, w_v, args.cpu_seconds, Q, W, ks, vs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
