"""Decode benchmark of the tile-synchronized decoder on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b_b1]

A step is one teacher-forced decode step of the whole model for the workload's
batch: embedding, every decoder layer (one megakernel launch), the LM head and
the argmax.  The default workload is the largest single-GPU one: the
Llama-3-8B-shaped bf16 model at batch 1, decoding from a 4096-token cache.  The
Llama-3-1B-shaped batch-1 workload runs after it and is reported under
"extra".  Inputs (random-init weights, KV cache, token ids) are seeded and
synthetic and are resident in HBM before timing.

Prints one JSON line: the megakernel's tokens/s as `value`, the kernel-per-op
modes (eager, and the library's HIP-graph mode), the multi-stream mode (one
kernel per segment on S streams, synchronised on tiles) and the persistent
multi-step mode (all timed steps in one launch, LM head and argmax inside it)
beside it, the dominant
kernel's roofline (algorithmic bytes per launch over its event-timed average
duration, against 8 TB/s) and the CPU oracle run on float32 weights, timed on a
bounded sample on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(m) -> int:
    """Weight bytes of one decoder layer (matrices + fp32 gains)."""
    wb = 2 if m.dtype == "bf16" else 4
    mats = m.qkv_cols * m.hidden + m.hidden * m.attn_cols + 3 * m.ffn * m.hidden
    gains = 2 * m.hidden + (2 * m.head_dim if m.qk_norm else 0)
    return mats * wb + gains * 4


def megakernel_bytes(m, ctx) -> int:
    """Algorithmic HBM bytes of one megakernel launch: every layer's weights
    once, the embedding rows, the cached keys/values read and the new ones written."""
    kvb = 2 if m.dtype == "bf16" else 4
    wb = 2 if m.dtype == "bf16" else 4
    B = len(ctx)
    kv_read = m.n_layers * sum(ctx) * m.n_kv_heads * m.head_dim * 2 * kvb
    kv_write = m.n_layers * B * m.n_kv_heads * m.head_dim * 2 * kvb
    emb = B * m.hidden * wb if m.has_embed else 0
    return m.n_layers * layer_bytes(m) + emb + kv_read + kv_write


def prefill_flops(m, S) -> int:
    """Matrix FLOPs of a causal prefill of S tokens: the layer GEMMs, the causal
    attention products (QK^T and PV over keys 0..i), and the LM head on the last row."""
    mats = m.qkv_cols * m.hidden + m.hidden * m.attn_cols + 3 * m.ffn * m.hidden
    attn = 4 * m.n_q_heads * m.head_dim * S * (S + 1) // 2
    return m.n_layers * (2 * S * mats + attn) + (2 * m.vocab * m.hidden if m.has_lm_head else 0)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def lm_head_bytes(m, B) -> int:
    wb = 2 if m.dtype == "bf16" else 4
    return m.vocab * m.hidden * wb + m.hidden * 4 + 4 * B * m.vocab if m.has_lm_head else 0


def cpu_model_name() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, raw_layers, raw_global, Kh, Vh, budget_s: float = 20.0) -> dict:
    """The oracle's decode step run on float32 weights (numpy and its BLAS),
    step by step, on the host's cores, over a bounded number of steps."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    from oracle import numerics as N
    import workloads as W
    m, r = wl.model, wl.run
    t0 = time.time()
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        layers = list(ex.map(lambda raw: N.prepare_layer(raw, np.float32), raw_layers))
    model = N.Model(m, layers, **{k: N.widen(v, np.float32) for k, v in raw_global.items()})
    K, V = Kh.copy(), Vh.copy()
    tokens = W.gen.decode_tokens(m, r) if m.has_embed else None
    x0 = None if m.has_embed else W.gen.input_rows(m, r)
    prep = time.time() - t0
    steps, spent = 0, 0.0
    while steps < r.steps and (steps == 0 or spent + spent / steps <= budget_s):
        ctx = [p + steps for p in r.ctx0]
        t1 = time.time()
        if m.has_embed:
            N.decode_step(model, K, V, ctx, tokens=tokens[steps])
        else:
            N.decode_step(model, K, V, ctx, x0=x0[steps])
        spent += time.time() - t1
        steps += 1
    cores = len(os.sched_getaffinity(0))
    threads = os.environ.get("OMP_NUM_THREADS", str(cores))
    return {"value": round(r.batch * steps / spent, 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{steps} teacher-forced decode steps of {wl.name} (batch {r.batch}), the oracle's "
                      f"decode step on float32 weights (numpy; BLAS threads {threads}) on {cores} host cores "
                      f"of a {cpu_model_name()}; weights widened to float32 before timing ({prep:.0f} s)",
            "cpu_model": cpu_model_name(), "ms_per_step": round(1e3 * spent / steps, 2)}


def run_workload(wl, args, modes, with_prefill=True):
    """Generate and upload one workload's inputs, then time its decode steps in
    each mode (and its prefill when it has one).  Returns the results and the
    host arrays the CPU baseline reuses."""
    import torch
    import tile_synchronized_decoder_amd as T
    from tile_synchronized_decoder_amd import device as D
    import workloads as W

    import dataclasses
    m, r = wl.model, wl.run
    K_steps = min(args.steps, r.steps)
    t0 = time.time()
    raw_layers = W.gen.all_layer_weights(m, r.seed, threads=16)
    raw_global = W.gen.global_weights(m, r.seed)
    Kh, Vh = W.gen.kv_cache(m, r, threads=16)
    tokens = W.gen.decode_tokens(m, r)
    log(f"[bench] {wl.name}: inputs generated in {time.time() - t0:.1f} s")
    q = T.mk_build_queue(T.make_config(m), T.make_plan(wl.plan, T.MK_DECODE, r.batch, r.ctx_max))
    dq = D.upload_queue(q)
    dm = D.upload_weights(raw_layers, raw_global)
    dkv = D.upload_kv(Kh, Vh)
    ws = D.workspace(q)
    B = r.batch
    prefill_res = None
    if r.prefill_len and with_prefill:
        # causal prefill of the prompt into the (empty) cache, timed per call in both modes;
        # the decode steps below continue from the cache the last call wrote
        S = r.prefill_len
        qp = T.mk_build_queue(T.make_config(m), T.make_plan(wl.plan.for_prefill(), T.MK_PREFILL, S, r.ctx_max))
        dqp, wsp = D.upload_queue(qp), D.workspace(qp)
        ptok = torch.from_numpy(W.gen.prefill_tokens(m, r)).cuda()
        plg = torch.empty((m.vocab,), dtype=torch.float32, device="cuda")
        pnx = torch.empty((1,), dtype=torch.int32, device="cuda")
        prefill_res = {"tokens": S, "flops": prefill_flops(m, S), "modes": {},
                       "lo_parts_mask": int(T.mk_get_option(T.MK_OPT_PREFILL_LO))}
        for name in ("mega", "kpo"):
            mode = T.MK_MEGAKERNEL if name == "mega" else T.MK_KERNEL_PER_OP
            for _ in range(2):
                T.mk_prefill(qp, dqp, dm.w, dkv.kv, ptok, S, 0, wsp, plg, pnx, mode)
            torch.cuda.synchronize()
            n_runs = 5
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(torch.cuda.current_stream())
            for _ in range(n_runs):
                T.mk_prefill(qp, dqp, dm.w, dkv.kv, ptok, S, 0, wsp, plg, pnx, mode)
            e1.record(torch.cuda.current_stream())
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n_runs
            err = T.mk_device_error(qp, wsp)
            assert err.code == 0, f"device error {err.code} in prefill mode {name}"
            tf = prefill_res["flops"] / (ms * 1e-3) / 1e12
            prefill_res["modes"][name] = {"ms": round(ms, 4), "tokens_per_s": round(S / (ms * 1e-3), 1),
                                          "tflops": round(tf, 1)}
            log(f"[bench] prefill {name}: {ms:.3f} ms, {tf:.1f} TFLOP/s")
        best = prefill_res["modes"]["mega"]["tflops"]
        prefill_res["roofline"] = {"bound": "mfma", "achieved": best, "peak": MFMA_BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(best / MFMA_BF16_PEAK_TFLOPS, 4),
                                   "traffic": None}
        del wsp
    # input rows: token ids, or for a model without an embedding its given rows [steps, B, H]
    tok_all = torch.from_numpy(tokens.astype(np.int32)).cuda() if m.has_embed else None
    x0_all = None if m.has_embed else torch.from_numpy(W.gen.input_rows(m, r)).cuda()
    x0_buf = None if m.has_embed else torch.empty_like(x0_all[0])
    ctx_all = torch.tensor([[p + t for p in r.ctx0] for t in range(r.steps)], dtype=torch.int32,
                           device="cuda")
    logits = torch.empty((B, m.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty((B,), dtype=torch.int32, device="cuda")
    tok_buf = torch.empty((B,), dtype=torch.int32, device="cuda")
    ctx_buf = torch.empty((B,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: {q.nbytes(T.MK_PART_INSTR) // 32} instructions, queue "
        f"{q.nbytes(T.MK_PART_DEVICE) / 1e6:.2f} MB, workspace {ws.numel() / 1e6:.1f} MB")

    def set_inputs(t):
        if m.has_embed:
            tok_buf.copy_(tok_all[t % r.steps])
        else:
            x0_buf.copy_(x0_all[t % r.steps])
        ctx_buf.copy_(ctx_all[t % r.steps])

    def step(t, mode, marks=None):
        set_inputs(t)
        if mode == T.MK_KERNEL_PER_OP_GRAPH:
            # the library replays one HIP graph of the per-op launches and the LM head
            T.mk_decode_step(q, dq, dm.w, dkv.kv, tok_buf if m.has_embed else None, x0_buf, ctx_buf, B, ws,
                             logits if m.has_lm_head else None, nxt if m.has_lm_head else None, mode)
            return
        T.mk_decode_step(q, dq, dm.w, dkv.kv, tok_buf if m.has_embed else None, x0_buf, ctx_buf, B, ws, None,
                         None, mode)
        if marks is not None:
            marks.append(torch.cuda.Event(enable_timing=True))
            marks[-1].record(stream)
        if m.has_lm_head:
            T.mk_lm_head(q, dm.w, ws, logits, nxt)

    if args.copy_calibration:
        src = torch.ones(args.copy_calibration * 2 ** 20 // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {args.copy_calibration} MiB")
        del src, dst

    mode_of = {"mega": T.MK_MEGAKERNEL, "kpo": T.MK_KERNEL_PER_OP, "kpo_graph": T.MK_KERNEL_PER_OP_GRAPH}
    results = {}
    for name in modes:
        if name == "loop":
            # persistent multi-step decode: all K timed steps in one launch of a loop queue,
            # the LM head and argmax inside it (teacher-forced with the same token ids)
            if not (m.has_embed and m.has_lm_head and m.dtype == "bf16"):
                continue
            ql = T.mk_build_queue(T.make_config(m), T.make_plan(dataclasses.replace(wl.plan, loop=1, attn_pop=0), T.MK_DECODE,
                                                                r.batch, r.ctx_max))
            dql, wsl = D.upload_queue(ql), D.workspace(ql)
            lg_all = torch.empty((K_steps, B, m.vocab), dtype=torch.float32, device="cuda")
            nx_all = torch.empty((K_steps, B), dtype=torch.int32, device="cuda")
            toks, ctx0 = tok_all[:K_steps].contiguous(), ctx_all[0].clone()

            def run_loop(k):
                T.mk_decode_loop(ql, dql, dm.w, dkv.kv, toks, ctx0, B, k, 0, wsl, lg_all, nx_all)

            run_loop(min(max(args.warmup, 1), K_steps))
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            w0 = time.perf_counter()
            e0.record(stream)
            run_loop(K_steps)
            e1.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - w0
            total_ms = e0.elapsed_time(e1)
            err = T.mk_device_error(ql, wsl)
            assert err.code == 0, f"device error {err.code} in the multi-step loop"
            results[name] = {"ms_per_step": total_ms / K_steps, "tokens_per_s": B * K_steps / (total_ms / 1e3),
                             "steps_per_launch": K_steps, "host_wall_tokens_per_s": B * K_steps / wall}
            log(f"[bench] {wl.name} loop: {total_ms / K_steps:.4f} ms/step ({K_steps} steps in one launch)")
            del wsl, lg_all
            continue
        T.mk_set_option(T.MK_OPT_MEGAKERNELS, 1)
        if name.startswith("ms"):
            # multi-stream mode: one kernel per segment on `streams` internal streams, tile waits
            T.mk_set_option(T.MK_OPT_STREAMS, int(name[2:]))
            mode = T.MK_MULTI_STREAM
        elif name.startswith("mega") and name != "mega":
            # a composition of megakernels: `megaK` cuts each step into K launches at layer
            # boundaries
            T.mk_set_option(T.MK_OPT_MEGAKERNELS, int(name[4:]))
            mode = T.MK_MEGAKERNEL
        else:
            mode = mode_of[name]
        composition = name.startswith("mega") and name != "mega"
        try:
            for t in range(max(args.warmup, 1 if composition else 0)):
                step(t, mode)
        except T.MkError as e:
            # a composition the library refuses for this plan (shared sub-queues, more
            # launches than layers) is left out of the line
            if not (composition and e.status == T.MK_ENOTSUP):
                raise
            T.mk_set_option(T.MK_OPT_MEGAKERNELS, 1)
            log(f"[bench] {wl.name} {name}: refused ({e})")
            continue
        torch.cuda.synchronize()
        # timed region: K steps, events on the launch stream before each step and after
        # the decoder layers of each step (the megakernel / per-op launches end there)
        starts, mids = [], []
        ev_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        # host time to enqueue one step: the least over the steps (a call that finds
        # the device queue full blocks, which only adds)
        host = []
        for t in range(K_steps):
            starts.append(torch.cuda.Event(enable_timing=True))
            starts[-1].record(stream)
            h0 = time.perf_counter()
            step(t, mode, mids)
            host.append(time.perf_counter() - h0)
        ev_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        total_ms = starts[0].elapsed_time(ev_end)
        per_step = [starts[i].elapsed_time(starts[i + 1]) for i in range(K_steps - 1)]
        per_step.append(starts[-1].elapsed_time(ev_end))
        res = {"ms_per_step": total_ms / K_steps, "tokens_per_s": B * K_steps / (total_ms / 1e3),
               "p50_ms": float(np.percentile(per_step, 50)), "p95_ms": float(np.percentile(per_step, 95)),
               "host_wall_tokens_per_s": B * K_steps / wall, "host_enqueue_us": 1e6 * min(host)}
        if mids:
            layers_ms = [starts[i].elapsed_time(mids[i]) for i in range(K_steps)]
            res["layers_ms"] = float(np.mean(layers_ms))           # reset + megakernel (or per-op launches)
            res["lm_head_ms"] = res["ms_per_step"] - res["layers_ms"]
        results[name] = res
        err = T.mk_device_error(q, ws)
        assert err.code == 0, f"device error {err.code} in mode {name}"
        T.mk_set_option(T.MK_OPT_MEGAKERNELS, 1)
        log(f"[bench] {wl.name} {name}: {res['ms_per_step']:.4f} ms/step, {res['tokens_per_s']:.1f} tok/s")

    mega = results.get("mega", next(iter(results.values())))
    ctx_mid = [p + K_steps // 2 for p in r.ctx0]
    mbytes = megakernel_bytes(m, ctx_mid)
    step_bytes = mbytes + lm_head_bytes(m, B)
    out = {"workload": wl, "steps": K_steps, "results": results, "prefill": prefill_res,
           "instructions": q.nbytes(T.MK_PART_INSTR) // 32,
           "step_hbm_gbs": step_bytes / (mega["ms_per_step"] * 1e-3) / 1e9}
    if "layers_ms" in mega:
        from tile_synchronized_decoder_amd.profiling import read_traffic
        ach = mbytes / (mega["layers_ms"] * 1e-3) / 1e9
        # HBM bytes per launch counted by FETCH_SIZE / WRITE_SIZE in a separate profiled run of
        # this workload (null when the kernel sources changed since)
        traffic = read_traffic(os.path.join(ROOT, "profiles", f"mk_interp_{wl.name}_traffic.md"))
        out["roofline"] = {"bound": "hbm", "kernel": "mk_interp (decoder layers, one launch per step)",
                           "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                           "algorithmic_bytes_per_launch": mbytes}
    kpos = [v["ms_per_step"] for k, v in results.items() if k.startswith("kpo")]
    if "loop" in results and "mega" in results:
        out["loop_speedup_vs_mega"] = round(mega["ms_per_step"] / results["loop"]["ms_per_step"], 4)
    if kpos and "mega" in results:
        out["speedup"] = round(min(kpos) / mega["ms_per_step"], 4)
    mss = [v["ms_per_step"] for k, v in results.items() if k.startswith("ms")]
    if mss and "mega" in results:
        out["ms_speedup"] = round(min(mss) / mega["ms_per_step"], 4)
    out["host"] = (raw_layers, raw_global, Kh, Vh)
    del dm, dkv, ws
    torch.cuda.empty_cache()
    return out


def _rounded(results):
    return {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
            for k, v in results.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama8b_b1")
    ap.add_argument("--extra", default="llama1b_b1",
                    help="comma-separated workloads also timed and reported under 'extra' ('' for none)")
    ap.add_argument("--workers-per-cu", type=int, default=1)
    ap.add_argument("--queues", type=int, default=0, help="sub-queues (0: the workload's plan)")
    ap.add_argument("--tiles", default="", help="override tile widths, e.g. tq=16,to=8,tf=16,td=8,kb=256")
    ap.add_argument("--gemv-pipe", type=int, default=0,
                    help="decode GEMV weight issue: 0 or 1 pipelined (default), 2 compiler-ordered")
    ap.add_argument("--prefill-lo", type=int, default=None,
                    help="prefill GEMMs taking both bf16 parts of their activations, a mask (1 QKV, 2 O, "
                         "4 gate/up, 8 down; default: the library's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--modes", default="mega,kpo,kpo_graph,loop,ms2,ms4,mega2,mega4",
                    help="mega, kpo, kpo_graph, loop, msS: the multi-stream mode on S streams, and "
                         "megaK: a composition of K megakernels per step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the modes, copy MIB MiB device to device three times: a plain copy "
                         "kernel of known size that hardware byte counters can be scaled by")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only (no collectives or sharding are built); "
                                   "--gpus must be 1"}))
        sys.exit(2)

    import dataclasses
    import torch
    import tile_synchronized_decoder_amd as T
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    if args.queues:
        wl = dataclasses.replace(wl, plan=dataclasses.replace(wl.plan, n_queues=args.queues))
    if args.tiles:
        kv = {k: int(v) for k, v in (p.split("=") for p in args.tiles.split(","))}
        wl = dataclasses.replace(wl, plan=dataclasses.replace(wl.plan, **kv))
    m, r = wl.model, wl.run
    torch.cuda.set_device(0)
    T.mk_set_option(T.MK_OPT_WORKERS_PER_CU, args.workers_per_cu)
    T.mk_set_option(T.MK_OPT_GEMV_PIPE, args.gemv_pipe)
    if args.prefill_lo is not None:
        T.mk_set_option(T.MK_OPT_PREFILL_LO, args.prefill_lo)
    modes = args.modes.split(",")

    head = run_workload(wl, args, modes)
    res = head["results"]
    mega = res.get("mega", next(iter(res.values())))
    B = r.batch
    line = {
        "metric": "decode tokens/s + step latency vs kernel-per-op; HBM GB/s as % of peak",
        "value": round(mega["tokens_per_s"], 2), "unit": "tokens/s", "n_gpus": 1, "steps": head["steps"],
        "warmup": args.warmup, "ms_per_step": round(mega["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "storage": m.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.describe}", "batch": B, "context": f"{r.ctx0[0]}+",
                   "layers": m.n_layers, "hidden": m.hidden, "vocab": m.vocab,
                   "instructions_per_step": head["instructions"],
                   "workers_per_cu": args.workers_per_cu, "n_queues": wl.plan.n_queues,
                   "tiles": {k: getattr(wl.plan, k) for k in ("tq", "to", "tf", "td", "kb")}},
        "step_hbm_gbs": round(head["step_hbm_gbs"], 1),
        "step_hbm_frac": round(head["step_hbm_gbs"] / HBM_PEAK_GBS, 4),
        "modes": _rounded(res),
        "roofline": head.get("roofline"),
    }
    if head["prefill"] is not None:
        line["prefill"] = head["prefill"]
    if "speedup" in head:
        line["megakernel_speedup_vs_best_kpo"] = head["speedup"]
    if "loop_speedup_vs_mega" in head:
        line["loop_speedup_vs_mega"] = head["loop_speedup_vs_mega"]
    if "ms_speedup" in head:
        line["megakernel_speedup_vs_best_multi_stream"] = head["ms_speedup"]
    host = head.pop("host")
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        line["cpu_baseline"] = cpu_baseline(wl, *host, budget_s=args.cpu_budget)
    del host, head
    extra = {}
    for name in [n for n in args.extra.split(",") if n and n != wl.name]:
        ex = run_workload(W.WORKLOADS[name], args, modes, with_prefill=False)
        ex.pop("host")
        extra[name] = {"describe": ex["workload"].describe, "steps": ex["steps"],
                       "modes": _rounded(ex["results"]), "roofline": ex.get("roofline"),
                       "step_hbm_frac": round(ex["step_hbm_gbs"] / HBM_PEAK_GBS, 4),
                       "megakernel_speedup_vs_best_kpo": ex.get("speedup"),
                       "loop_speedup_vs_mega": ex.get("loop_speedup_vs_mega"),
                       "megakernel_speedup_vs_best_multi_stream": ex.get("ms_speedup")}
    if extra:
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
