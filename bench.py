"""Benchmark of the MoE expert layer on one MI355X.

A step is one pass of the whole layer path (route -> align -> expert FFN with
combine) over every layer of a workload, on one stream (captured as a HIP
graph unless --eager). Inputs are synthetic (gen/) and resident in HBM before
the timed region. Prints one JSON line.

Default run: the headline workload is the decode-regime layer stack, T=32
tokens through 40 layers of H=2048, I=512, E=256, top-8, each with its own
102-slot FP8 pool (grown to hold every routed expert when more are needed).
The same line carries one record per other workload ("records"): the other
decode stacks (T=8; the larger-expert stack at T=32; the mixed FP8/int4
stack at T=8) and the batched layers (16384 accumulated tokens; 4096 tokens
of the larger-expert stack; 8192 tokens of the mixed stack). Each record has
its layer time, layer-level HBM and FP8-matrix fractions, the roofline of
its dominant kernel and the oracle's CPU baseline. The roofline is the FP8
matrix peak for the 16384-token layer (a dense contraction) and HBM
bandwidth for every other workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0

# (config, tokens): the headline first, then the other records of the default run
DEFAULT_RUN = [("C1", 32), ("C1", 8), ("C3", 32), ("C4", 8), ("C2", 16384), ("C3", 4096), ("C4", 8192)]
MFMA_BOUND = {("C2", 16384)}          # dense contraction: FP8 matrix roofline; everything else: HBM


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None, help="measure one workload only (default: every workload)")
    ap.add_argument("--tokens", type=int, default=None, help="tokens per layer (with --config)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--act", choices=["auto", "bf16", "fp8"], default="auto")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--calls", choices=("layer", "split"), default="layer",
                    help="layer: one moe_layer call per layer; split: moe_route_align then moe_expert_ffn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pager", action="store_true", help="leave out the slot-miss path records")
    ap.add_argument("--pager-only", action="store_true", help="only the slot-miss path records")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time budget of the headline workload")
    ap.add_argument("--cpu-seconds-records", type=float, default=5.0, help="... of each other record")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device-to-device copies of MIB MiB (to scale HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources a kernel's byte counters depend on: counters taken for one
# version of these files say nothing about another
KERNEL_SOURCES = {
    "gemm1_stream": ("ffn_stream.hip", "moe_common.h"),
    "gemm2_stream": ("ffn_stream.hip", "moe_common.h"),
    "combine": ("ffn_stream.hip",),
    "gemm1_fp8": ("ffn_mfma.hip", "moe_common.h"),
    "gemm2_fp8": ("ffn_mfma.hip", "moe_common.h"),
    "gemm1_tile": ("ffn_int4.hip", "ffn_grouped.hip", "moe_common.h"),
    "gemm2_tile": ("ffn_int4.hip", "ffn_grouped.hip", "moe_common.h"),
}


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "moe_expert_layer_topk_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def host_info():
    """CPU model and BLAS build of the host the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')} ({b.get('openblas configuration', '').strip()})"
    except Exception:
        pass
    return model, blas


def measure(args, name, T, L, cpu_seconds, mfma_bound):
    import torch
    import moe_expert_layer_topk_amd as moe
    from gen import CONFIGS, make_layer, make_bank
    from harness import device_pool, device_inputs, bank_on_device, oracle_layer

    cfg = CONFIGS[name]
    act = {"bf16": moe.ACT_BF16, "fp8": moe.ACT_FP8_G128_POW2}.get(args.act)
    if act is None:
        act = moe.ACT_BF16 if T <= 64 else moe.ACT_FP8_G128_POW2
    bm = args.block_m or (16 if act == moe.ACT_BF16 else 128)
    dev = torch.device("cuda:0")
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k

    t0 = time.time()
    bank = make_bank(cfg)
    bdev = bank_on_device(bank, dev)
    layers = []
    for l in range(L):
        li = make_layer(cfg, T, l)
        pool = device_pool(li, bank, dev, bdev)
        x, logits, soe, mask = device_inputs(li, dev)
        cap = moe.align_capacity(T, k, E, bm)
        buf = dict(ids=torch.empty((T, k), dtype=torch.int32, device=dev),
                   w=torch.empty((T, k), dtype=torch.float32, device=dev),
                   err=torch.zeros(2, dtype=torch.int32, device=dev),
                   al=dict(sorted_pair=torch.empty(cap, dtype=torch.int32, device=dev),
                           block_slot=torch.empty(cap // bm, dtype=torch.int32, device=dev),
                           counts=torch.empty(E, dtype=torch.int32, device=dev),
                           seg_offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
                           n_padded=torch.empty(1, dtype=torch.int32, device=dev)),
                   aws=torch.empty(max(1, moe.route_align_workspace_bytes(T, k, E, bm)), dtype=torch.uint8,
                                   device=dev),
                   fws=torch.empty(max(1, moe.ffn_workspace_bytes(T, k, E, H, I, bm, act)), dtype=torch.uint8,
                                   device=dev) if args.calls == "split" else None,
                   lws=torch.empty(max(1, moe.layer_workspace_bytes(T, k, E, H, I, bm, act)), dtype=torch.uint8,
                                   device=dev) if args.calls == "layer" else None,
                   out=torch.empty((T, H), dtype=torch.bfloat16, device=dev))
        layers.append((li, pool, x, logits, soe, mask, buf))
    del bdev
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name} T={T} layers={L} act={act} block_m={bm}: inputs ready in {time.time() - t0:.1f}s")

    def run_layer(entry, stream):
        li, pool, x, logits, soe, mask, b = entry
        if args.calls == "layer":
            moe.layer_call(pool, x, logits, k, soe, bm, act, mask=mask, ids=b["ids"], w=b["w"], aligned=b["al"],
                           err=b["err"], out=b["out"], ws=b["lws"], stream=stream)
            return
        moe.route_align(logits, k, bm, soe, mask=mask, ids=b["ids"], w=b["w"], out=b["al"], err=b["err"],
                        ws=b["aws"] if b["aws"].numel() > 1 else None, stream=stream)
        moe.expert_ffn(pool, x, k, E, b["w"], b["al"], bm, act, out=b["out"], ws=b["fws"], stream=stream)

    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)

    def step():
        for entry in layers:
            run_layer(entry, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    # ---- timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    tok_s = T * L / (ms_step / 1e3)          # expert-layer tokens per second
    log(f"[bench] {ms_step:.4f} ms/step, {ms_step / L * 1e3:.2f} us/layer (wall {wall:.3f}s)")

    # ---- per-kernel durations with the library's event tracing (HIP events
    # the dispatches stamp on the launch stream), same steps launched eagerly
    moe.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = moe.profile_read()
    moe.profile_enable(False)
    log("[bench] kernels: " + ", ".join(f"{n}: {c} x {ms / c * 1e3:.2f} us" for n, (c, ms) in prof.items()))

    # ---- algorithmic work per layer (distinct routed experts' slot bytes, not padding)
    w13_bytes = {0: 2 * I * H + 8 * I, 1: I * H + 2 * I * (H // 128) * 4}
    w2_bytes = {0: H * I + 4 * H, 1: H * I // 2 + H * (I // 128) * 4}
    NP = T * k
    tot_bytes = tot_flops = 0
    kern_bytes = {}          # per kernel, summed over layers
    kern_flops = {}
    distinct, fmt_hist = [], {"fp8": 0, "int4": 0}
    for li, pool, x, logits, soe, mask, b in layers:
        ids = b["ids"].cpu().numpy()
        used, cnt = np.unique(ids[ids >= 0], return_counts=True)
        distinct.append(used.size)
        fm = li.expert_fmt[used].astype(int)
        fmt_hist["fp8"] += int((fm == 0).sum())
        fmt_hist["int4"] += int((fm == 1).sum())
        w13 = sum(w13_bytes[f] for f in fm)
        w2 = sum(w2_bytes[f] for f in fm)
        w13_fp8 = sum(w13_bytes[0] for f in fm if f == 0)
        w2_fp8 = sum(w2_bytes[0] for f in fm if f == 0)
        np_fp8 = int(cnt[fm == 0].sum())
        tot_bytes += w13 + w2 + T * H * 2 + T * E * 4 + T * H * 2 + NP * 16
        tot_flops += 6 * NP * H * I

        def add(d, key, v):
            d[key] = d.get(key, 0) + v
        # decode kernels: weights of every routed expert + token rows + h rows
        add(kern_bytes, "gemm1_stream", w13 + T * H * 2 + NP * I * 2)
        add(kern_bytes, "gemm2_stream", w2 + NP * I * 2 + NP * H * 4)
        # batched FP8 matrix-core kernels: FP8-slot experts' weights, activation codes, h codes
        add(kern_bytes, "gemm1_fp8", w13_fp8 + T * H + np_fp8 * I)
        add(kern_bytes, "gemm2_fp8", w2_fp8 + np_fp8 * I + np_fp8 * H * 2)
        add(kern_bytes, "gemm1_tile", (w13 - w13_fp8) + (NP - np_fp8) * (H + I))
        add(kern_bytes, "gemm2_tile", (w2 - w2_fp8) + (NP - np_fp8) * (I + H * 2))
        add(kern_bytes, "combine", NP * H * (4 if act == moe.ACT_BF16 else 2) + T * H * 2)
        add(kern_flops, "gemm1_fp8", 4 * np_fp8 * H * I)
        add(kern_flops, "gemm2_fp8", 2 * np_fp8 * H * I)
    layer_s = ms_step / 1e3 / L
    hbm_frac_layer = tot_bytes / L / layer_s / (HBM_PEAK_GBS * 1e9)
    mfma_frac_layer = tot_flops / L / layer_s / (FP8_PEAK_TFLOPS * 1e12)

    # dominant kernel: the one with the most time per step
    dom = max(prof, key=lambda n: prof[n][1])
    n_launch, ms = prof[dom]
    per_launch_s = ms / n_launch / 1e3
    launches_per_step = n_launch / args.steps
    if mfma_bound:
        work = kern_flops.get(dom, 0) / launches_per_step
        achieved = work / per_launch_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / FP8_PEAK_TFLOPS, 4))
    else:
        work = kern_bytes.get(dom, 0) / launches_per_step
        achieved = work / per_launch_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
    roof["kernel"] = dom
    roof["avg_us"] = round(per_launch_s * 1e6, 3)
    roof["work_per_launch"] = int(work)
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        rec = json.load(open(tpath)).get(f"{cfg.name}-T{T}-{dom}")
        if rec and rec.get("source_hash") == source_hash(*KERNEL_SOURCES.get(dom, ("ffn_stream.hip",))):
            traffic = rec.get("bytes_per_launch")
    roof["traffic"] = traffic
    roof["layer_frac"] = round(mfma_frac_layer if mfma_bound else hbm_frac_layer, 4)

    # ---- CPU baseline: the oracle on a bounded sample of the same layers
    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # noqa: F401
        threads = len(os.sched_getaffinity(0))
        if T <= 64:
            # decode sizes: whole layers, as many as fit in the time budget
            done_tok, t_cpu, n_layers = 0, 0.0, 0
            for li, *_ in layers:
                c0 = time.perf_counter()
                oracle_layer(li, bank, bm, act)
                t_cpu += time.perf_counter() - c0
                done_tok += T
                n_layers += 1
                if t_cpu >= cpu_seconds:
                    break
            what = f"{n_layers} of {L} layers, all {T} tokens each"
        else:
            # batched sizes: the FFN of a token subset of the first layer (route and
            # align on all tokens, every routed expert dequantized), the subset
            # growing 4x until one run takes about a third of the budget
            li = layers[0][0]
            n = 16
            while True:
                sub = np.arange(min(T, n))
                c0 = time.perf_counter()
                oracle_layer(li, bank, bm, act, token_subset=sub)
                t_cpu = time.perf_counter() - c0
                if t_cpu >= cpu_seconds / 3 or n >= T:
                    break
                n *= 4
            done_tok = sub.size
            what = f"layer 0, FFN of {sub.size} of {T} tokens (route and align on all {T})"
        model, blas = host_info()
        cpu = dict(value=round(done_tok / t_cpu, 3), unit="tokens/s", cores=threads, kind="oracle",
                   sample=f"{what}; fp64 NumPy incl. slot dequant; {t_cpu:.1f}s", cpu_model=model, blas=blas)
        log(f"[bench] cpu oracle {cpu['value']} tokens/s over {t_cpu:.1f}s")

    rec = dict(
        workload=f"{cfg.name}: T={T} tokens x {L} layers, H={H}, I={I}, E={E}, top-{k}, "
                 f"{'per-layer slot pools' if cfg.slots and T < cfg.resident_all_at else 'all experts resident'}, "
                 f"{'FP8 + int4' if cfg.int4_frac else 'FP8'} slots",
        value=round(tok_s, 1), ms_per_step=round(ms_step, 5), tokens_per_layer=T, layers=L, block_m=bm,
        act_mode="bf16" if act == moe.ACT_BF16 else "fp8_g128_pow2", graph=graph is not None,
        distinct_experts_per_layer=round(float(np.mean(distinct)), 1),
        slot_formats_routed=fmt_hist,
        layer_us=round(layer_s * 1e6, 3), layer_hbm_frac=round(hbm_frac_layer, 4),
        layer_mfma_frac=round(mfma_frac_layer, 4), layer_tflops=round(tot_flops / L / layer_s / 1e12, 2),
        kernels_us={n: round(m / c * 1e3, 3) for n, (c, m) in prof.items()},
        roofline=roof, cpu_baseline=cpu, dtype="bf16" if act == moe.ACT_BF16 else "fp8")
    # free this workload's device memory before the next one
    del layers, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def measure_pager(args, name="C1", T=8, L=40, steps=8, n_slots=102, packed=False):
    """The slot-miss path over a decode loop: each layer's VRAM pool holds
    n_slots experts, every expert sits in page-locked host RAM, each step
    brings new tokens (the layer's gate and reuse prior fixed). Per layer and
    step: route, read the ids back, plan with the pager, fill the misses on a
    copy stream while the resident experts' pass runs, then the filled
    experts' pass. Step 0 starts from empty pools; the timed steps are 1...
    packed: the host bank holds the slots packed (per-row Huffman codes of
    the FP8 exponents); each fill copies the packed bytes to a staging buffer
    and expands them into the slot on the copy stream."""
    import torch
    import moe_expert_layer_topk_amd as moe
    from gen import CONFIGS, make_bank, step_tokens

    cfg = CONFIGS[name]
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    dev = torch.device("cuda:0")
    t0 = time.time()
    bank = make_bank(cfg)
    host = torch.from_numpy(bank.materialize(0)).pin_memory()
    host_fmt = torch.zeros(E, dtype=torch.uint8).pin_memory()
    if packed:
        pk = [moe.fp8_pack(host[e].numpy(), H, I) for e in range(E)]
        p_sizes = np.array([p.size for p in pk], dtype=np.uint64)
        p_offsets = np.concatenate([[0], np.cumsum(p_sizes)[:-1]]).astype(np.uint64)
        host_packed = torch.from_numpy(np.concatenate(pk)).pin_memory()
        staging = torch.empty(int(n_slots * (int(p_sizes.max()) + 16)), dtype=torch.uint8, device=dev)
        pack_ratio = float(p_sizes.sum()) / (E * bank.stride)
    pools = [moe.SlotPool(torch.zeros((n_slots, bank.stride), dtype=torch.uint8, device=dev),
                          torch.zeros(n_slots, dtype=torch.uint8, device=dev), H, I) for _ in range(L)]
    inputs = []
    for st in range(steps):
        row = []
        for l in range(L):
            xb, lg = step_tokens(cfg, T, l, st)
            row.append((torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16),
                        torch.from_numpy(lg).to(dev)))
        inputs.append(row)
    pager = moe.Pager(L, E, n_slots)
    ws = torch.empty(moe.ffn_workspace_bytes(T, k, E, H, I, 16, 0), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ids_h = torch.empty((T, k), dtype=torch.int32).pin_memory()
    t1h = torch.empty(E, dtype=torch.int32).pin_memory()
    t2h = torch.empty(E, dtype=torch.int32).pin_memory()
    t1d = torch.empty(E, dtype=torch.int32, device=dev)
    t2d = torch.empty(E, dtype=torch.int32, device=dev)
    comp = torch.cuda.Stream()
    copy = torch.cuda.Stream()
    torch.cuda.set_stream(comp)
    torch.cuda.synchronize()
    log(f"[bench] pager {name} T={T} layers={L} slots={n_slots}: inputs ready in {time.time() - t0:.1f}s")
    stats = dict(bytes=0, slot_bytes=0, fill_ms=0.0, misses=0, hits=0)

    def run_step(st, timed):
        for l in range(L):
            x, logits = inputs[st][l]
            ids, w, _ = moe.route(logits, k, stream=comp)
            ids_h.copy_(ids, non_blocking=True)
            comp.synchronize()
            table, fe, fs = pager.plan(l, ids_h.numpy())
            miss = np.zeros(E, bool)
            miss[fe] = True
            t1h.numpy()[:] = np.where(miss, moe.SLOT_DEFERRED, table)
            t2h.numpy()[:] = np.where(miss, table, moe.SLOT_DEFERRED)
            copy.wait_stream(comp)                       # earlier kernels may still read the victim slots
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(copy)
            if packed:
                moe.pager_fill_packed(pools[l], host_packed, p_offsets, p_sizes, fe, fs, staging, copy)
            else:
                moe.pager_fill(pools[l], host, host_fmt, fe, fs, copy)
            c1.record(copy)
            t1d.copy_(t1h, non_blocking=True)
            t2d.copy_(t2h, non_blocking=True)
            a1 = moe.align(ids, E, 16, t1d, stream=comp)
            moe.expert_ffn_pass(pools[l], x, k, E, w, a1, 16, 0, False, out, ws, stream=comp)
            comp.wait_event(c1)
            a2 = moe.align(ids, E, 16, t2d, stream=comp)
            moe.expert_ffn_pass(pools[l], x, k, E, w, a2, 16, 0, True, out, ws, stream=comp)
            if timed:
                c1.synchronize()
                stats["fill_ms"] += c0.elapsed_time(c1)
                stats["bytes"] += int(p_sizes[fe].sum()) if packed else int(fe.size) * bank.stride
                stats["misses"] += int(fe.size)
                stats["slot_bytes"] += int(fe.size) * bank.stride
                stats["hits"] += int(len(set(ids_h.numpy().reshape(-1).tolist())) - fe.size)

    run_step(0, False)                                   # cold pools
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for st in range(1, steps):
        run_step(st, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    n = (steps - 1) * L
    layer_us = wall / n * 1e6
    rec = dict(
        workload=f"{name} slot-miss path: T={T} tokens x {L} layers, {n_slots} VRAM slots per layer, all {E} experts "
                 f"in page-locked host RAM{' packed (per-row Huffman-coded FP8 exponents)' if packed else ''}, "
                 f"new tokens every step",
        value=round(T * n / wall, 1), tokens_per_layer=T, layers=L, steps_timed=steps - 1, vram_slots=n_slots,
        layer_us=round(layer_us, 2), hit_rate=round(stats["hits"] / max(1, stats["hits"] + stats["misses"]), 4),
        misses_per_layer_step=round(stats["misses"] / n, 2),
        h2d_GBps=round(stats["bytes"] / max(1e-9, stats["fill_ms"] / 1e3) / 1e9, 2),
        h2d_bytes_per_layer_step=int(stats["bytes"] / n),
        slot_GBps_delivered=round(stats["slot_bytes"] / max(1e-9, stats["fill_ms"] / 1e3) / 1e9, 2),
        fill_us_per_layer_step=round(stats["fill_ms"] / n * 1e3, 2),
        host_bank_ratio=round(pack_ratio, 4) if packed else 1.0,
        note="per layer: route, ids read back, LRU plan on the host, misses copied on a copy stream while "
             "the resident experts' pass runs, then the filled experts' pass; wall-clock over the timed steps")
    log(f"[bench] pager: {layer_us:.1f} us/layer, hit rate {rec['hit_rate']}, {rec['h2d_GBps']} GB/s H2D")
    del pools, host
    if packed:
        del staging, host_packed
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer runs unsharded on one MI355X); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 5}))
        return
    from gen import CONFIGS

    if args.pager_only:
        print(json.dumps({"records": [measure_pager(args), measure_pager(args, packed=True)]}), flush=True)
        return
    if args.config:
        cfg = CONFIGS[args.config]
        T = args.tokens or (max(t for t in cfg.Ts if t <= 64) if min(cfg.Ts) <= 64 else cfg.Ts[0])
        runs = [(args.config, T)]
    else:
        runs = DEFAULT_RUN
    recs = []
    for i, (name, T) in enumerate(runs):
        L = args.layers or CONFIGS[name].layers
        recs.append(measure(args, name, T, L, args.cpu_seconds if i == 0 else args.cpu_seconds_records,
                            (name, T) in MFMA_BOUND))
    if not args.config and not args.no_pager:
        recs.append(measure_pager(args))
        recs.append(measure_pager(args, packed=True))
    head = recs[0]
    res = {
        "metric": "MoE expert-layer tokens/s (layer tokens per second over the layer stack)",
        "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic",
        "config": {k: v for k, v in head.items() if k not in ("value", "ms_per_step", "roofline", "cpu_baseline",
                                                              "dtype")},
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "records": recs[1:],
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
