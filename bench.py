"""Benchmark: DDTree verification rounds per second on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload C4]

A step is one whole verification round for every sequence of the workload:
ddt_topk -> ddt_build_tree -> ddt_tree_mask -> ddt_tree_attention -> ddt_tree_walk,
on inputs already resident in HBM, replayed from HIP graphs.  Enough copies of the
inputs are rotated that the working set exceeds the 256 MB Infinity Cache.  The
default workload is the largest one: 32 sequences with 16K-32K prefixes, V = 128256,
Hq = 64, Hkv = 8, D = 128, bf16.

Prints one JSON line: rounds/s, the attention main kernel's roofline (HIP events
attached to its dispatches), the whole attention step (main kernel and split merge)
next to it, the fused verifier epilogue (LM head + arg-max per node, on the same
trees) with its own roofline, and the CPU oracle's rate on a bounded sample of the
same workload, timed on this host's cores.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from ddt_synthetic import configs, gen  # noqa: E402

METRIC = "verify rounds/sec (build+tree attn+walk); tree-attn HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFS = 2500.0
F32_PEAK_TFS = 157.3
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attempts_for(cfg):
    """Draft attempts that pass the near-tie rule, from the committed table."""
    path = os.path.join(ROOT, "tests", "golden", "attempts.json")
    key = "C3" if cfg.name.startswith("C3-") else cfg.name
    try:
        with open(path) as f:
            t = json.load(f).get(key)
        if t and len(t) >= cfg.S:
            return list(t[:cfg.S])
    except OSError:
        pass
    return [0] * cfg.S


def describe(cfg):
    P = f"{cfg.prefix[0]}" if cfg.prefix[0] == cfg.prefix[1] else f"U[{cfg.prefix[0]},{cfg.prefix[1]}]"
    return (f"{cfg.name}: {cfg.S} seq, L={cfg.L}, V={cfg.V}, K={cfg.K}, B={cfg.B}, prefix {P}, "
            f"Hq={cfg.Hq}, Hkv={cfg.Hkv}, D={cfg.D}, {cfg.dtype}")


def attention_cost(cfg, prefix_lens):
    """Algorithmic HBM bytes and flops of one tree-attention call: every prefix K/V
    row read once per KV head, the tree K/V, Q and the mask read once, the output O
    written once.  Flops are QK^T and PV over the prefix (the ancestors add at most
    L + 1 keys per row; the prefix dominates)."""
    e = 2 if cfg.dtype == "bf16" else 4
    N, W = cfg.N, cfg.W
    P = int(np.sum(prefix_lens))
    kv = P * cfg.Hkv * cfg.D * e * 2
    tree = cfg.S * N * cfg.Hkv * cfg.D * e * 2
    q = cfg.S * N * cfg.Hq * cfg.D * e
    o = cfg.S * N * cfg.Hq * cfg.D * e
    mask = cfg.S * N * W * 4
    flops = 4.0 * N * cfg.Hq * cfg.D * P
    return kv + tree + q + o + mask, flops


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def attention_kernel(cfg):
    if cfg.dtype != "bf16":
        return "attn_f32"
    return "attn_d128" if cfg.D == 128 else "attn_partial_bf16"


CSRC = os.path.join(ROOT, "block_diffusion_draft_position_amd", "csrc")
TRAFFIC = {  # kernel -> (committed rocprofv3 summary, the source it was taken on)
    "attention": (os.path.join(ROOT, "profiles", "attn_hbm_traffic.txt"), os.path.join(CSRC, "tree_attention.hip")),
    "epilogue": (os.path.join(ROOT, "profiles", "lm_head_hbm_traffic.txt"), os.path.join(CSRC, "lm_head.hip")),
}


def measured_traffic(workload, kernel="attention"):
    """HBM bytes per launch of the kernel, from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, if it was taken on the current kernel source."""
    import hashlib
    path, source = TRAFFIC[kernel]
    try:
        with open(path) as f:
            lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
        with open(source, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    recorded = {l[1] for l in lines if l[0] == "source_sha256"}
    if sha not in recorded:
        return None
    for l in lines:
        if l[0] == "workload" and l[1] == workload:
            kv = dict(zip(l[2::2], l[3::2]))
            return float(kv["traffic_bytes"])
    return None


def epilogue_bench(cfg, b, rnd, dev, up, workers, calls=20):
    """The fused verifier epilogue on this workload's trees (the ones the timed rounds
    build): final hidden states [S, N, Hq*D] that plant each node's synthetic target
    token, an N(0, 1/d) LM-head weight [V, Hq*D], bf16.  Timed with HIP events attached
    to the tile kernel's dispatches over eager calls; the walk from its tokens is
    checked against the round's walk over the target logits."""
    import torch
    import block_diffusion_draft_position_amd as ddt
    d = gen.d_model(cfg)
    t0 = time.time()
    W = gen.lm_head_weight(cfg, workers=workers)
    tree = {k: rnd.tree[k].cpu().numpy() for k in ("tree_tok", "parent", "num_nodes")}
    H = gen.tree_hidden_states(cfg, b, tree, W, workers=workers)
    log(f"[bench] epilogue inputs ready in {time.time() - t0:.1f}s")
    Wd, Hd = up(W), up(H)
    del W, H
    nn = rnd.tree["num_nodes"]
    tok = torch.empty(cfg.S, cfg.N, dtype=torch.int32, device=dev)
    mx = torch.empty(cfg.S, cfg.N, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, ddt.load().ddt_lm_head_argmax_workspace_size(cfg.S, cfg.B, cfg.V, d)),
                     dtype=torch.uint8, device=dev)
    for _ in range(3):
        ddt.ddt_lm_head_argmax(Hd, Wd, nn, tok, mx, ws)
    torch.cuda.synchronize()
    ddt.lm_head_profiling(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(calls):
        ddt.ddt_lm_head_argmax(Hd, Wd, nn, tok, mx, ws)
    stop.record()
    torch.cuda.synchronize()
    tiles_ms, n = ddt.lm_head_timing()
    ddt.lm_head_profiling(False)
    call_s = start.elapsed_time(stop) / calls / 1e3
    tiles_s = tiles_ms / max(n, 1) / 1e3
    w = ddt.ddt_tree_walk_tokens(rnd.tree["tree_tok"], rnd.tree["parent"], nn, tok, cfg.L)
    torch.cuda.synchronize()
    same = all(torch.equal(w[k], rnd.walk[k]) for k in ("accept_len", "acc_nodes", "acc_tok", "bonus"))
    M = cfg.S * cfg.N
    flops = 2.0 * M * cfg.V * d
    wbytes = cfg.V * d * 2 + M * d * 2 + M * 8
    ridge = BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / wbytes >= ridge:
        roof = {"bound": "mfma", "achieved": flops / tiles_s / 1e12, "peak": BF16_PEAK_TFS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": wbytes / tiles_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(cfg.name, "epilogue")
    return {"kernel": "lm_head_tiles", "rows": M, "d_model": d, "vocab": cfg.V,
            "kernel_us": tiles_s * 1e6, "call_us": call_s * 1e6, "launches_timed": n,
            "roofline": roof, "flops_per_launch": flops, "bytes_per_launch": wbytes,
            "logits_round_trip_avoided_bytes": 2 * M * cfg.V * 4,
            "walk_matches_logits_walk": bool(same),
            "timing": "HIP events attached to the tile kernel's dispatches; call_us adds the "
                      "per-node reduce (torch events around the eager calls)"}


def cpu_baseline(cfg, b, att, budget_s=12.0):
    """The oracle as it stands on a bounded sample of the workload, scaled to
    rounds/s: steps 1-3 and the walk for one sequence, attention for a sample of that
    sequence's rows; the rest is extrapolated linearly.  Its numpy BLAS calls may use
    every core this process may run on; its Python loops run on one."""
    from threadpoolctl import threadpool_limits

    import oracle
    scale = 1.0 / math.sqrt(cfg.D)
    s = 0
    cores = host_cores()
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
        tree = oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B)
        nn = int(tree["num_nodes"])
        mask = oracle.tree_mask(tree["parent"], nn, cfg.N)
        t_steps = time.perf_counter() - t0
        # the target's logits at the tree are an input of the walk (synthesised, untimed)
        tl = gen.target_logits(cfg, s, att[s], tree["tree_tok"], tree["parent"], nn, b["chain"][s], b["keep"][s])
        t0 = time.perf_counter()
        oracle.tree_walk(tree["tree_tok"], tree["parent"], nn, tl, cfg.L)
        t_steps += time.perf_counter() - t0
        p0, p1 = int(b["cu_prefix"][s]), int(b["cu_prefix"][s + 1])
        w = oracle.round.widen
        q, kp, vp = w(b["q"][s]), w(b["k_cache"][p0:p1]), w(b["v_cache"][p0:p1])
        kt, vt = w(b["k_tree"][s]), w(b["v_tree"][s])
        rows_all = [(n, h) for n in range(nn) for h in range(cfg.Hq)]
        order = np.random.default_rng(0).permutation(len(rows_all))
        done, t_att = 0, 0.0
        while done < len(rows_all) and t_att < budget_s:
            chunk = [rows_all[i] for i in order[done:done + 32]]
            ta = time.perf_counter()
            oracle.tree_attention(q, kp, vp, kt, vt, mask, nn, scale, rows=chunk)
            t_att += time.perf_counter() - ta
            done += len(chunk)
    total_rows = cfg.S * cfg.N * cfg.Hq
    per_round = cfg.S * t_steps + t_att / done * total_rows
    return {"value": 1.0 / per_round, "unit": "rounds/s", "cores": cores, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": (f"sequence 0 of {cfg.S}: top-K, tree, mask and walk in full, tree attention "
                       f"for {done} of its {nn * cfg.Hq} (node, head) rows; scaled linearly to "
                       f"{cfg.S} sequences x {total_rows // cfg.S} rows; fp64 numpy with BLAS on "
                       f"{cores} threads (Python loops on one), {per_round:.3g} s per round")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="C4", help="one of " + ", ".join(sorted(configs.CONFIGS)))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0 = auto)")
    ap.add_argument("--no-epilogue", action="store_true", help="skip the fused LM-head epilogue")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verification round is data-parallel across sequences and needs no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_diffusion_draft_position_amd as ddt

    cfg = configs.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ddt.load()
    att = attempts_for(cfg)
    log(f"[bench] generating {describe(cfg)}")
    t0 = time.time()
    workers = min(16, host_cores())
    b = gen.batch(cfg, att, workers=workers)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    def up(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    base = {k: up(b[k]) for k in ("draft_logits", "q", "k_cache", "v_cache", "k_tree", "v_tree", "cu_prefix")}
    base["bonus"] = up(b["bonus"].astype(np.int32))
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = ddt.Shape(S=cfg.S, L=cfg.L, V=cfg.V, K=cfg.K, B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D,
                      dtype=tdt, max_prefix=int(np.max(b["prefix_lens"])))
    rnd = ddt.VerifyRound(shape, dev)
    # the target logits are evaluated at the tree this library builds
    rnd.draft_tree(base["draft_logits"], base["bonus"], base["cu_prefix"])
    torch.cuda.synchronize()
    tt, par, nn = (rnd.tree[k].cpu().numpy() for k in ("tree_tok", "parent", "num_nodes"))
    tl = np.zeros((cfg.S, cfg.N, cfg.V), dtype=np.float32)

    def target_of(s):
        gen.target_logits(cfg, s, att[s], tt[s], par[s], int(nn[s]), b["chain"][s], b["keep"][s], out=tl[s])

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(target_of, range(cfg.S)))
    base["target"] = up(tl)
    del tl
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    ncopies = args.copies or max(1, min(64, math.ceil(2 * MALL_BYTES / per_copy)))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(ncopies - 1)]
    log(f"[bench] {ncopies} input copies of {per_copy / 2**20:.1f} MiB")

    def step(c):
        rnd(c["draft_logits"], c["bonus"], c["q"], c["k_cache"], c["v_cache"], c["cu_prefix"],
            c["k_tree"], c["v_tree"], c["target"])

    for i in range(max(2, args.warmup)):
        step(copies[i % ncopies])
    torch.cuda.synchronize()
    graphs = []
    if not args.no_graph:
        for c in copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % ncopies].replay()
        run = lambda i: graphs[i % ncopies].replay()
    else:
        run = lambda i: step(copies[i % ncopies])
    # ---- timed region: whole rounds
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        run(i)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    # ---- the attention kernel alone: HIP events that the library records around it on
    # its stream, over the same rounds launched eagerly (events inside graphs cannot be
    # read back on this runtime)
    ddt.attention_profiling(True)
    nprof = min(args.steps, max(ncopies, 100))
    for i in range(nprof):
        step(copies[i % ncopies])
    torch.cuda.synchronize()
    attn_ms, step_ms, attn_n = ddt.attention_timing()
    ddt.attention_profiling(False)
    del graphs
    acc = rnd.walk["accept_len"].float().mean().item()
    rounds_s = args.steps / (ms / 1e3)
    bytes_, flops = attention_cost(cfg, b["prefix_lens"])
    attn_s = attn_ms / max(attn_n, 1) / 1e3
    R = cfg.N * (cfg.Hq // cfg.Hkv)
    ridge = (BF16_PEAK_TFS if cfg.dtype == "bf16" else F32_PEAK_TFS) * 1e12 / (HBM_PEAK_GBS * 1e9)
    intensity = flops / bytes_
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": bytes_ / attn_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        peak = BF16_PEAK_TFS if cfg.dtype == "bf16" else F32_PEAK_TFS
        roof = {"bound": "mfma", "achieved": flops / attn_s / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(cfg.name)
    step_s = step_ms / max(attn_n, 1) / 1e3
    step_ach = (bytes_ / step_s / 1e9) if roof["bound"] == "hbm" else (flops / step_s / 1e12)
    roof["kernel"] = attention_kernel(cfg)
    roof["kernel_us"] = attn_s * 1e6
    roof["launches_timed"] = attn_n
    roof["timing"] = ("HIP events attached to each dispatch of the kernel (hipExtLaunchKernelGGL) "
                      "on its stream, eager rounds right after the timed graph replays")
    roof["bytes_per_launch"] = bytes_
    roof["flops_per_launch"] = flops
    out = {
        "metric": METRIC, "value": rounds_s, "unit": "rounds/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": describe(cfg), "sequences": cfg.S, "draft_positions": cfg.L,
                   "vocab": cfg.V, "top_k": cfg.K, "node_budget": cfg.B,
                   "prefix_tokens": int(np.sum(b["prefix_lens"])), "q_heads": cfg.Hq,
                   "kv_heads": cfg.Hkv, "head_dim": cfg.D, "rows_per_kv_head": R,
                   "input_copies": ncopies, "graph_replay": not args.no_graph,
                   "walk": {ddt.WALK_SCAN: "row scan", ddt.WALK_PATH: "path walk",
                            ddt.WALK_HYBRID: "hybrid"}[ddt.walk_mode(cfg.S, cfg.B, cfg.L, cfg.V)]},
        "roofline": roof,
        "attention_step": {"kernels": [roof["kernel"], "attn_combine"] if cfg.dtype == "bf16" else [roof["kernel"]],
                           "us": step_s * 1e6, "achieved": step_ach, "unit": roof["unit"],
                           "frac": step_ach / roof["peak"],
                           "timing": "main kernel start to split-merge end, HIP events attached to "
                                     "the two dispatches, same eager rounds"},
        "accept_len_mean": acc,
    }
    if not args.no_epilogue and cfg.dtype == "bf16":
        log("[bench] fused verifier epilogue")
        del copies
        out["epilogue"] = epilogue_bench(cfg, b, rnd, dev, up, workers)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(cfg, b, att)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
