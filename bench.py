"""Benchmark of the fused shared-QK LSH-attention forward pass on one MI355X.

A step is one call of reformer_lsh_attn_fwd over one batch of synthetic input
(hash -> sort -> chunked attention -> unsort/combine, all heads).  Inputs,
workspace and outputs are resident in HBM before timing starts.  Prints one
JSON line on stdout; diagnostics go to stderr.

Timing: after the warmup, K steps with a hipEvent between every two kernels give
the per-kernel breakdown and name the dominant kernel; then the K timed steps
(the reported value) record events around that kernel only, since each event
record adds a few microseconds in front of the kernel after it.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_seq_64k]
                  [--attend none|same_bucket|dedup|both]

--attend times an attended-set variant (reformer_lsh_attn_fwd_ex) instead of
the method as described; such a line names the variant in its config and
carries no cpu_baseline leg.  --backward times a training step of the layer
instead: the fused forward that keeps its permutation and per-round lse
(reformer_lsh_attn_fwd_train) followed by lsh_attn_bwd, with seeded output
gradients; its line has "pass": "fwd+bwd" in its config.  --block times one
reversible Reformer block around the attention (reformer_block_fwd: LayerNorm,
projections, the attention, output projection, LayerNorm, chunked GELU
feed-forward) on the workload's sequence with dim = 64 heads; per stage.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LSH-attn fwd tokens/sec at L=64K, 8 hashes; % HBM / MFMA roofline"
METRIC_TRAIN = "LSH-attn fwd+bwd (training step) tokens/sec at L=64K, 8 hashes; % HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 MFMA / packed vector
TOP_CLOCK_MHZ = 2400         # MI355X top engine clock (the published peaks' clock)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


ATTEND = {"none": (False, False), "same_bucket": (True, False), "dedup": (False, True), "both": (True, True)}


def algorithmic_work(B, H, L, D, n_b, n_h, es, same_bucket=False, dedup=False):
    """Per-launch algorithmic bytes and flops of each kernel: what the method
    must read and write (each input once, each output once), not what a kernel
    happens to move."""
    th = B * H * L            # token-heads
    tr = th * n_h             # token-rounds
    # variants: the slot's bucket (same-bucket), every round's unsort index (set union)
    extra = 4 * tr * (int(same_bucket) + int(dedup))
    half = n_b // 2
    return {
        "prep": {"bytes": 2 * n_h * D * half * es, "flops": 0},
        # per token-head: its row read, one bucket id per round written; D * n_b * n_h flop
        # (the n_b/2 dot products of [xR; -xR], 2 flop per multiply-add)
        "hash": {"bytes": th * (D * es + 4 * n_h), "flops": 2 * th * D * half * n_h},
        "fixup": {"bytes": 0, "flops": 0},
        # the sort as a whole reads each bucket id and writes the sorted and unsort
        # indices: 12 B per token-round, split as the two launches touch them
        "sort_hist": {"bytes": tr * 4, "flops": 0},
        "sort_scatter": {"bytes": tr * 8, "flops": 0},
        # per token-round: its sorted index, its output row and lse; the QK and V rows
        # are compulsory once per token-head (2 D es / n_h per token-round).  A kernel
        # whose rounds each gather their rows from beyond the caches moves
        # 2 D es per token-round instead (gathered_bytes below).
        "chunk_attn": {"bytes": tr * (4 + D * es + 4) + th * 2 * D * es + extra, "flops": tr * 4 * D * 128,
                       "gathered_bytes": tr * (4 + 3 * D * es + 4) + extra},
        # per token-head: n_h rows + lse + undo index read, one output row + LSE written
        "combine": {"bytes": th * (n_h * (D * es + 8) + D * es + 4), "flops": 0},
        # backward: per token x, out, dout rows and dLSE read, key scales written; per slot
        # its undo index and lse read, its combine weights written
        "bwd_prep": {"bytes": th * (3 * D * es + 12) + tr * 16, "flops": 0},
        # per slot: index, gathered x, v and dout rows, lse, weights, key scales read;
        # its dx and dv rows written.  flops: S, dP, dV, dK, dQ over its 128 keys
        "attn_bwd": {"bytes": tr * (5 * D * es + 24), "flops": tr * 128 * 10 * D},
        # per token: its n_h slots' dx and dv rows (and undo indices) read, dx and dv written
        "bwd_reduce": {"bytes": tr * (4 + 2 * D * es) + th * 2 * D * es, "flops": 0},
    }


def block_work(B, L, H, n_b, n_h, es=2):
    """Algorithmic bytes and flops of each block stage: activations read and
    written once ([B L dim] bf16), weights read once; the feed-forward's hidden
    activation stays out of the count (a fused design never writes it); the
    attention stage is the sum of its kernels."""
    M, dim = B * L, 64 * H
    act = M * dim * es
    att = algorithmic_work(B, H, L, 64, n_b, n_h, es)
    att_b = sum(v["bytes"] for k, v in att.items() if not k.startswith(("bwd", "attn_bwd")))
    att_f = sum(v["flops"] for k, v in att.items() if not k.startswith(("bwd", "attn_bwd")))
    return {
        "ln1": {"bytes": 2 * act, "flops": 0},
        "qkv_proj": {"bytes": 3 * act + 2 * dim * dim * es, "flops": 2 * 2 * M * dim * dim},
        "attention": {"bytes": att_b, "flops": att_f},
        "out_proj": {"bytes": 3 * act + dim * dim * es, "flops": 2 * M * dim * dim},
        "ln2": {"bytes": 2 * act, "flops": 0},
        "ffn": {"bytes": 3 * act + 8 * dim * dim * es, "flops": 2 * 2 * M * dim * 4 * dim},
    }


def measured_traffic(workload: str, kernel: str, attend: str = "none"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record (profiles/traffic_<workload>[_<attend>].json, "train" for the
    training step), or None when there is no record or the kernel's source has
    changed since it was taken."""
    from lsh_attention_amd.prof_summary import source_sha256
    tag = workload if attend == "none" else f"{workload}_{attend}"
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(kernel)
    if rec is None or rec.get("source_sha256") != source_sha256(kernel):
        return None
    return rec["traffic_bytes"]


def hbm_copy_gbs(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Achievable HBM bandwidth: read + write bytes of a plain 1 GiB device copy
    per second (reported beside the datasheet peak, not instead of it)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    del src, dst
    return 2.0 * nbytes * reps / (ms * 1e-3) / 1e9


SMALL_WORKLOADS = ("single_head_fp32", "mlm_small_512", "causal_lm_4k")


def _oracle_problem(args):
    """One (batch, head) problem through the oracle, in a worker process with a
    one-thread BLAS (so that the worker count is the core count)."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    x, v, rot, n_b, n_h, C, causal = args
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.forward_problem(x, v, rot, n_b, n_h, C, causal)
        return time.perf_counter() - t0


def _warm_worker(_):
    """Imports the oracle in a worker and holds it briefly, so that every worker
    has started and imported before the timed run."""
    import oracle  # noqa: F401
    time.sleep(0.5)
    return 0


def _one_thread_env():
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"


def cpu_baseline(inp, min_seconds: float = 10.0, max_workers: int = 16):
    """The oracle, untouched, timed on the host: whole (batch, head) problems of
    the workload at full length, spread over worker processes (one problem per
    worker at a time, one BLAS thread each), submitted until at least
    `min_seconds` of wall time have passed or every problem is done.  A run
    that finishes within 10 s is repeated three times and the median taken.
    tokens/s = B*L * problems_done / (B*H * wall)."""
    from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait
    from multiprocessing import get_context

    import numpy as np
    w = inp.workload
    B, H, L, _ = inp.qk.values.shape
    rot = None if inp.rot is None else inp.rot.values.astype(np.float64)
    n_prob = B * H
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    workers = max(1, min(max_workers, avail, n_prob))

    def job(k):
        b, h = divmod(k, H)
        return (inp.qk.values[b, h].astype(np.float64), inp.v.values[b, h].astype(np.float64), rot,
                w.n_buckets, inp.n_hashes, w.chunk_len, w.causal)

    runs = []
    with ProcessPoolExecutor(workers, mp_context=get_context("spawn"), initializer=_one_thread_env) as ex:
        list(ex.map(_warm_worker, range(workers)))  # every worker started and importing before timing
        while True:
            t0 = time.perf_counter()
            pending, nxt, done = set(), 0, 0
            while nxt < n_prob and len(pending) < workers:
                pending.add(ex.submit(_oracle_problem, job(nxt)))
                nxt += 1
            while pending:
                fin, pending = wait(pending, return_when=FIRST_COMPLETED)
                done += len(fin)
                if nxt < n_prob and time.perf_counter() - t0 < min_seconds:
                    for _ in fin:
                        if nxt < n_prob:
                            pending.add(ex.submit(_oracle_problem, job(nxt)))
                            nxt += 1
            runs.append((time.perf_counter() - t0, done))
            if len(runs) == 3 or runs[0][0] > min_seconds:
                break
    rates = sorted(B * L * d / (n_prob * t) for t, d in runs)
    med = rates[len(rates) // 2]
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    t_med, d_med = next((t, d) for t, d in runs if B * L * d / (n_prob * t) == med)
    return {"value": round(med, 1), "unit": "tokens/s", "cores": workers, "kind": "oracle", "cpu_model": cpu,
            "sample": f"{d_med} of {n_prob} (batch, head) problems at full L={L}, all {inp.n_hashes} rounds, "
                      f"float64 numpy oracle in {workers} worker processes with one BLAS thread each, "
                      f"{t_med:.2f} s wall; median of {len(runs)} run(s); "
                      f"tokens/s = B*L*problems / (B*H*wall)",
            "seconds": round(t_med, 3), "runs": [round(B * L * d / (n_prob * t), 1) for t, d in runs]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_seq_64k")
    ap.add_argument("--n-hashes", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attend", choices=sorted(ATTEND), default="none",
                    help="attended-set variant: same-bucket mask, set-union correction, or both")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step (forward keeping its state, then the backward pass)")
    ap.add_argument("--block", action="store_true",
                    help="time one reversible block (attention sublayer + chunked feed-forward)")
    ap.add_argument("--chunk-rows", type=int, default=16384, help="feed-forward row chunk of --block")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device-to-device copy of this many MiB "
                         "(a reference kernel of known traffic for hardware byte counters; the run then "
                         "skips its own bandwidth copy)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs each problem on one GPU and has no "
              "multi-GPU sharding (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lsh_attention_amd import binding as bd
    from lsh_attention_amd import inputs as I

    if args.block:
        return bench_block(args)
    inp = I.make_inputs(args.workload, n_hashes=args.n_hashes)
    w = inp.workload
    B, H, L, D = inp.qk.values.shape
    n_h, n_b = inp.n_hashes, w.n_buckets
    es = 2 if w.dtype == "bf16" else 4
    same_bucket, dedup = ATTEND[args.attend]
    log(f"workload {w.name}: B{B} H{H} L{L} D{D} n_b{n_b} n_h{n_h} causal={w.causal} {w.dtype} "
        f"attend={args.attend}; sha256(qk)={inp.meta['qk_sha256'][:16]}")

    def dev(t):
        if t is None:
            return None
        if t.bits is not None:
            return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(t.values)).cuda()

    qk, v, rot = dev(inp.qk), dev(inp.v), dev(inp.rot)
    dt = bd.LSH_BF16 if w.dtype == "bf16" else bd.LSH_F32
    ws = torch.empty(bd.fwd_workspace_bytes(B, H, L, D, n_b, n_h, 64, dt), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qk)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")

    if args.backward and args.attend != "none":
        raise SystemExit("--backward covers the method as described (no --attend)")
    names = list(bd.KERNEL_NAMES)
    if args.backward:
        n_slots = n_h * L
        sidx = torch.empty((B, H, n_slots), dtype=torch.int32, device="cuda")
        undo = torch.empty((B, H, n_h, L), dtype=torch.int32, device="cuda")
        lse_s = torch.empty((B, H, n_slots), dtype=torch.float32, device="cuda")
        dout = dev(I.gaussian(4242, (B, H, L, D), w.dtype))
        dlse = dev(I.gaussian(4243, (B, H, L), "f32"))
        dqk, dv = torch.empty_like(qk), torch.empty_like(v)
        bws = torch.empty(bd.bwd_workspace_bytes(B, H, L, D, n_h, 64, dt), dtype=torch.uint8, device="cuda")
        names += bd.BWD_KERNEL_NAMES

    def step(events=None):
        if args.backward:
            bd.reformer_lsh_attn_fwd_train(qk, v, rot, n_b, n_h, 64, w.causal, out=out, lse=lse, sorted_idx=sidx,
                                           undo_idx=undo, lse_sorted=lse_s, workspace=ws,
                                           stage_events=None if events is None else events[0])
            bd.lsh_attn_bwd(qk, v, sidx, undo, lse_s, out, dout, dlse, n_h, 64, w.causal, dqk=dqk, dv=dv,
                            workspace=bws, stage_events=None if events is None else events[1])
        else:
            bd.reformer_lsh_attn_fwd(qk, v, rot, n_b, n_h, 64, w.causal, out=out, lse=lse, workspace=ws,
                                     stage_events=None if events is None else events[0], same_bucket=same_bucket,
                                     dedup=dedup)

    for _ in range(args.warmup):
        step()
    n_fwd = len(bd.KERNEL_NAMES)

    def run(events):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(events[k])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # Per-kernel breakdown: K steps with an event between every two kernels.  Each
    # event record adds a few microseconds in front of the next kernel, so these
    # steps are not the timed ones.
    events = [(bd.EventSet(), bd.EventSet(bd.BWD_N_EVENTS) if args.backward else None) for _ in range(args.steps)]
    breakdown_s = run(events)
    per_kernel = np.array([e[0].durations_ms() + (e[1].durations_ms() if e[1] else []) for e in events])
    for e in events:
        e[0].close()
        if e[1]:
            e[1].close()
    dom_i = int(np.argmax(per_kernel.mean(axis=0)))
    log(f"{args.steps} steps with every kernel bracketed by events: {breakdown_s * 1e3 / args.steps:.4f} ms/step")

    # Timed region: K steps with events around the dominant kernel only, for its
    # live launch duration.
    if dom_i < n_fwd:
        events = [(bd.EventSet(only=(dom_i, dom_i + 1)), None) for _ in range(args.steps)]
        dur = lambda e: e[0].elapsed_ms(dom_i, dom_i + 1)
    else:
        j = dom_i - n_fwd
        events = [(None, bd.EventSet(bd.BWD_N_EVENTS, only=(j, j + 1))) for _ in range(args.steps)]
        dur = lambda e: e[1].elapsed_ms(j, j + 1)

    elapsed = run(events)
    dom_ms = float(np.mean([dur(e) for e in events]))
    for e in events:
        for x in e:
            if x is not None:
                x.close()
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = B * L
    value = tokens / (elapsed / args.steps)
    log(f"{args.steps} timed steps: {ms_per_step:.4f} ms/step wall (events around {names[dom_i]} only: "
        f"{dom_ms * 1e3:.2f} us)")
    # near-ties of the hash argmax in the last step: decisions fp32 could not
    # certify, re-decided from float64 sums
    uncertified = bd.hash_uncertified(ws, B, H, L, n_b, n_h, qk.dtype)
    n_decisions = B * H * n_h * L
    log(f"hash: {uncertified} of {n_decisions} token-rounds re-decided in float64 ({uncertified / n_decisions:.2e})")

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # A counter run's copy probe must be the run's only device copy.
    copy_gbs = None if args.copy_probe_mib else hbm_copy_gbs()
    if copy_gbs is not None:
        log(f"plain device copy: {copy_gbs:.0f} GB/s (read + write), {copy_gbs / HBM_PEAK_GBS:.3f} of the HBM peak")
    # The shader clock under load, beside fractions that use the published peaks
    # (which assume the 2400 MHz top clock).
    clock_mhz = None if args.copy_probe_mib else bd.measure_clock_mhz(200)
    if clock_mhz is not None:
        log(f"shader clock under a full-chip FMA spin: {clock_mhz:.0f} MHz (top {TOP_CLOCK_MHZ})")

    work = algorithmic_work(B, H, L, D, n_b, n_h, es, same_bucket, dedup)
    peak_flops = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS

    def rates(wk, us):
        ent = {"us": round(us, 2)}
        if us > 0 and wk["bytes"]:
            ent["GBps"] = round(wk["bytes"] / (us * 1e-6) / 1e9, 1)
            ent["hbm_frac"] = round(ent["GBps"] / HBM_PEAK_GBS, 4)
        if us > 0 and wk.get("gathered_bytes"):
            ent["gathered_GBps"] = round(wk["gathered_bytes"] / (us * 1e-6) / 1e9, 1)
        if us > 0 and wk["flops"]:
            ent["TFLOPs"] = round(wk["flops"] / (us * 1e-6) / 1e12, 1)
            ent["mfma_frac"] = round(ent["TFLOPs"] / peak_flops, 4)
        return ent

    kernels = {}
    for i, name in enumerate(names):
        # the dominant kernel's time is the timed steps' own; the others come from
        # the breakdown steps
        kernels[name] = rates(work[name], (dom_ms if i == dom_i else float(np.mean(per_kernel[:, i]))) * 1e3)
        log(f"  {name:13s} {kernels[name]['us']:9.2f} us  "
            f"{json.dumps({k: x for k, x in kernels[name].items() if k != 'us'})}")
    # the sort as one step (its launches together): 12 B per token-round
    if "sort_hist" in kernels and "sort_scatter" in kernels:
        sort_wk = {"bytes": work["sort_hist"]["bytes"] + work["sort_scatter"]["bytes"], "flops": 0}
        sort_ent = rates(sort_wk, kernels["sort_hist"]["us"] + kernels["sort_scatter"]["us"])
        log(f"  {'sort (both)':13s} {sort_ent['us']:9.2f} us  {json.dumps({k: x for k, x in sort_ent.items() if k != 'us'})}")
    else:
        sort_ent = None
    dom = names[dom_i]
    d_us = kernels[dom]["us"]
    wk = work[dom]
    # The binding roofline of the dominant kernel: compute if its flops take longer
    # at peak than its algorithmic bytes at peak bandwidth.
    if wk["flops"] / (peak_flops * 1e12) > wk["bytes"] / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(wk["flops"] / (d_us * 1e-6) / 1e12, 2), "peak": peak_flops,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(wk["bytes"] / (d_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["traffic"] = measured_traffic(w.name, dom, "train" if args.backward else args.attend)
    roof["algorithmic_bytes"] = wk["bytes"]
    if roof["traffic"] is not None:
        roof["traffic_over_algorithmic"] = round(roof["traffic"] / wk["bytes"], 3)
    if "hbm_frac" in kernels[dom]:
        roof["hbm_frac"] = kernels[dom]["hbm_frac"]
    if "mfma_frac" in kernels[dom]:
        roof["mfma_frac"] = kernels[dom]["mfma_frac"]

    # Each step against the roofline its target is stated on: chunk attention
    # against bf16 (fp32) MFMA peak, sort and unsort+combine against HBM peak,
    # the hash against whichever of MFMA and HBM binds its algorithmic work.
    stage_roof = {}
    if not args.backward:
        hk, hw = kernels.get("hash"), work["hash"]
        if hk:
            hb = "mfma" if hw["flops"] / (peak_flops * 1e12) > hw["bytes"] / (HBM_PEAK_GBS * 1e9) else "hbm"
            stage_roof["hash"] = {"measure": hb, "frac": hk["mfma_frac" if hb == "mfma" else "hbm_frac"],
                                  "hbm_frac": hk.get("hbm_frac"), "target": None if hb == "mfma" else 0.5}
        if sort_ent:
            stage_roof["sort"] = {"measure": "hbm", "frac": sort_ent.get("hbm_frac"), "us": sort_ent["us"],
                                  "target": 0.5}
        if "chunk_attn" in kernels:
            ck = kernels["chunk_attn"]
            stage_roof["chunk_attn"] = {"measure": "mfma", "frac": ck.get("mfma_frac"),
                                        "hbm_frac": ck.get("hbm_frac"), "target": 0.4}
        if "combine" in kernels:
            stage_roof["unsort_combine"] = {"measure": "hbm", "frac": kernels["combine"].get("hbm_frac"),
                                            "target": 0.5}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "seq_len": L, "d_head": D, "n_buckets": n_b,
                   "n_hashes": n_h, "chunk_len": 64, "causal": w.causal},
        "roofline": roof,
        "stage_roofline": stage_roof,
        "kernels": kernels,
        "kernel_timing": {
            "breakdown_ms_per_step": round(breakdown_s * 1e3 / args.steps, 4),
            "what": "each kernel's us from K extra steps with events between all kernels; the dominant kernel's "
                    "from the timed steps, whose only events bracket it"},
        "token_head_rounds_per_s": round(n_decisions / (elapsed / args.steps), 1),
        "hash_uncertified": {"token_rounds": uncertified, "of": n_decisions},
        "clock": None if clock_mhz is None else {
            "mhz": round(clock_mhz, 1), "top_mhz": TOP_CLOCK_MHZ,
            "what": "shader cycles per real-time tick over a 200 us full-chip FMA spin right after the timed steps"},
        "hbm_copy": None if copy_gbs is None else {
            "GBps": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
            "what": "1 GiB device-to-device copy, read + write bytes"},
    }
    if args.attend != "none":
        result["config"]["attend"] = args.attend
    if args.backward:
        result["metric"] = METRIC_TRAIN
        result["config"]["pass"] = "fwd+bwd"
    if not args.no_cpu_baseline and args.attend == "none" and not args.backward:
        log("timing the oracle on the host (cpu_baseline leg)")
        result["cpu_baseline"] = cpu_baseline(inp)
        log(f"  oracle: {result['cpu_baseline']['value']} tokens/s on {result['cpu_baseline']['cores']} cores")
    print(json.dumps(result), flush=True)


def bench_block(args):
    import numpy as np
    import torch

    from lsh_attention_amd import binding as bd
    from lsh_attention_amd import inputs as I

    bi = I.make_block_inputs(args.workload, n_hashes=args.n_hashes)
    w = bi.workload
    B, L, dim = bi.x1.values.shape
    H, n_h, n_b = dim // 64, bi.n_hashes, w.n_buckets
    log(f"block {w.name}: B{B} L{L} dim{dim} heads{H} n_b{n_b} n_h{n_h} causal={w.causal} bf16 "
        f"chunk_rows={args.chunk_rows}")

    def dev(t):
        if t is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).cuda()

    x1, x2, rot = dev(bi.x1), dev(bi.x2), dev(bi.rot)
    P = {k: dev(t) for k, t in bi.params.items()}
    y1, y2 = torch.empty_like(x1), torch.empty_like(x2)
    ws = torch.empty(bd.block_workspace_bytes(B, L, H, n_b, n_h, 64, args.chunk_rows), dtype=torch.uint8,
                     device="cuda")

    def step(ev=None):
        bd.reformer_block_fwd(x1, x2, rot, P, n_b, n_h, w.causal, chunk_rows=args.chunk_rows, y1=y1, y2=y2,
                              workspace=ws, stage_events=ev)

    for _ in range(args.warmup):
        step()

    def run(events):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(events[k])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # per-stage breakdown (events between all stages), then the timed steps with
    # events around the dominant stage only, as for the forward
    events = [bd.EventSet(bd.BLOCK_N_EVENTS) for _ in range(args.steps)]
    breakdown_s = run(events)
    per = np.array([e.durations_ms() for e in events])
    for e in events:
        e.close()
    dom_i = int(np.argmax(per.mean(axis=0)))
    events = [bd.EventSet(bd.BLOCK_N_EVENTS, only=(dom_i, dom_i + 1)) for _ in range(args.steps)]
    elapsed = run(events)
    dom_ms = float(np.mean([e.elapsed_ms(dom_i, dom_i + 1) for e in events]))
    for e in events:
        e.close()
    ms = elapsed * 1e3 / args.steps
    log(f"{args.steps} steps with events between all stages: {breakdown_s * 1e3 / args.steps:.4f} ms/step; "
        f"{args.steps} timed steps: {ms:.4f} ms/step wall")
    work = block_work(B, L, H, n_b, n_h)
    stages = {}
    for i, name in enumerate(bd.BLOCK_STAGE_NAMES):
        us = (dom_ms if i == dom_i else float(np.mean(per[:, i]))) * 1e3
        wk = work[name]
        ent = {"us": round(us, 2)}
        if wk["bytes"]:
            ent["GBps"] = round(wk["bytes"] / (us * 1e-6) / 1e9, 1)
            ent["hbm_frac"] = round(ent["GBps"] / HBM_PEAK_GBS, 4)
        if wk["flops"]:
            ent["TFLOPs"] = round(wk["flops"] / (us * 1e-6) / 1e12, 1)
            ent["mfma_frac"] = round(ent["TFLOPs"] / BF16_PEAK_TFLOPS, 4)
        stages[name] = ent
        log(f"  {name:10s} {us:9.2f} us  {json.dumps({k: x for k, x in ent.items() if k != 'us'})}")
    dom = bd.BLOCK_STAGE_NAMES[dom_i]
    wk, d_us = work[dom], stages[dom]["us"]
    if wk["flops"] / (BF16_PEAK_TFLOPS * 1e12) > wk["bytes"] / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(wk["flops"] / (d_us * 1e-6) / 1e12, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(wk["bytes"] / (d_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["traffic"] = None
    result = {
        "metric": "Reformer block fwd (LSH attention + chunked FFN) tokens/sec at L=64K, 8 hashes",
        "value": round(B * L / (elapsed / args.steps), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "pass": "block", "batch": B, "seq_len": L, "dim": dim, "heads": H,
                   "n_buckets": n_b, "n_hashes": n_h, "chunk_len": 64, "causal": w.causal,
                   "ffn_chunk_rows": args.chunk_rows},
        "roofline": roof, "stages": stages,
        "stage_timing": {
            "breakdown_ms_per_step": round(breakdown_s * 1e3 / args.steps, 4),
            "what": "each stage's us from K extra steps with events between all stages; the dominant stage's "
                    "from the timed steps, whose only events bracket it"},
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
