"""Medusa tree-decode step throughput on one MI355X.

One step = the whole hot path on one batch of seeded synthetic input, inputs
resident in HBM: heads (residual block + vocabulary projection + per-head
top-k) -> candidate tree -> tree attention over the KV cache -> target argmax,
greedy acceptance and KV compaction. Default workload: 70B-shaped heads at
batch 1 (d = 8,192, V = 128,256, 4 heads in bf16 = 8.94 GB of weights, top-k
(10, 4, 2, 1), 64-node tree, GQA 64/8 heads of 128, 4,096 cached positions).
Other workloads (--workload) are secondary measurements: the batch-8 step
whose heads run over all 512 tree nodes on the matrix cores, the Hydra step
(four sequential head levels), the 8B-shaped step, the top-1 chain, the
70B-shaped step with one vocabulary projection shared by the four heads, the
70B-shaped step verified from the target's hidden states through its LM head
with a fused argmax (no logits in memory), and the 70B-shaped step sampled at
temperature 1: drafts drawn from the heads' distributions and verified by
rejection sampling ("70b_sampled"), or top-k drafts under typical acceptance
("70b_typical").

Prints one JSON line: steps/s over K steps timed with nothing between them
but the steps, the roofline of the dominant kernel (the vocabulary
projection + top-k, timed with HIP events that the library records around
that kernel on the stream it runs on, over a second pass of K steps) and the
CPU oracle's own throughput on the same inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PMC_FILE = os.path.join(ROOT, "profiles", "heads_fused_70b_pmc.json")


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def file_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed steps before timing (default: as many as take 0.5 s; the clocks take a few "
                         "hundred milliseconds of load to settle)")
    ap.add_argument("--workload", default="70b",
                    choices=["70b", "70b_chain", "8b", "tiny", "70b_b8", "hydra_b4", "70b_shared", "70b_lmhead",
                             "70b_sampled", "70b_typical"])
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated per step (0: enough that the non-weight bytes exceed twice the 256 MB "
                         "Infinity Cache, at most 16)")
    ap.add_argument("--cpu-steps", type=int, default=11,
                    help="oracle steps timed for the CPU baseline, one per input set (0: skip); the default takes every "
                         "set of the 70B-shaped workload, ~5 s on 16 host threads plus ~6 s for one step on one thread")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (scale factor for HBM counters)")
    ap.add_argument("--operand-order", default="auto", choices=["auto", "on", "off"],
                    help="also keep operand-order copies of the vocabulary matrices for the few-row matrix-core "
                         "kernels (auto: bf16 Hydra levels, LM-head verification and the shared projection, where "
                         "2 to 128 projection columns meet them)")
    ap.add_argument("--tile-norms", default="auto", choices=["auto", "on", "off"],
                    help="also keep the vocabulary matrices' tile norms (md_vocab_tile_norms), which the many-row "
                         "certified pass then reads instead of computing (auto: bf16 heads over more than 128 rows)")
    ap.add_argument("--seed", type=int, default=70)
    ap.add_argument("--cpu-1thread", type=int, default=1, help="also time one oracle step on one thread (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch

    import medusa_draft_heads_amd as md
    import oracle
    from synth.workloads import ALL, plant, plant_hidden, step_inputs, weights

    wl = ALL[args.workload]
    hydra = wl.kind == "hydra"
    topo = wl.topology()
    depth = max(len(p) for p in topo.paths)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t0 = time.time()
    w = weights(wl, args.seed)
    log("weights generated (%.1f s)" % (time.time() - t0))
    wd = {k: to_dev(v) for k, v in w.items()}
    torch.cuda.synchronize()
    log("weights on the GPU (%.1f GB)" % (sum(v.numel() * v.element_size() for v in wd.values()) / 1e9))

    # Input sets. Each set's verification logits are planted from the oracle's
    # own tree tokens; the oracle's step on the first --cpu-steps sets is the
    # CPU baseline. With heads over many rows the oracle runs the rows that
    # build the trees and its per-row time is scaled to all rows.
    sets, cpu_times, acc_oracle, oracle_margin = [], [], [], []
    threads = oracle.threads()
    sample_note = ""
    if args.sets <= 0:  # rotate past the 256 MB Infinity Cache: non-weight bytes >= 2 x 256 MB
        per_set = sum(v.nbytes for v in step_inputs(wl, args.seed, step=0).values())
        args.sets = int(min(16, max(2, -(-2 * (256 << 20) // per_set))))
        log("%d input sets of %.1f MB" % (args.sets, per_set / 1e6))

    def oracle_tree(x):
        """The oracle's heads and tree tokens for one input set, and their time."""
        nonlocal sample_note
        ta = time.perf_counter()
        heads = None
        if hydra:
            hy = oracle.hydra_expand(w["W"], w["b"], w["U"], w["E"], x["h"], topo.parent, topo.rank, wl.topk,
                                     x["root_tok"], x["lens"])
            margin = min(float(np.min(lvl["margin"])) for lvl in hy["levels"])
            return hy["tree_tok"], {"margin": margin}, time.perf_counter() - ta
        if wl.verify == "sampled":  # one row per request: the heads' logits, then the drafts drawn from them
            heads = oracle.heads_medusa(w["W"], w["b"], w["U"], x["h"], [1] * wl.K, want_logits=True)
            dr = oracle.draft_sample(heads["logits"], x["draft_words"], wl.topk, wl.temperature)
            tok, _ = oracle.tree_tokens_medusa(topo.parent, topo.rank, dr["tok"], x["src_row"], x["root_tok"],
                                               x["lens"])
            heads["margin"] = dr["margin"]
            return tok, heads, time.perf_counter() - ta
        rows = sorted(set(int(r) for r in x["src_row"]))
        heads = oracle.heads_medusa(w["W"], w["b"], w["U"], x["h"], wl.topk, rows=rows)
        full = np.full((wl.M, wl.K, wl.kmax), -1, np.int32)
        for j, r in enumerate(rows):
            full[r] = heads["idx"][j]
        tok, _ = oracle.tree_tokens_medusa(topo.parent, topo.rank, full, x["src_row"], x["root_tok"], x["lens"])
        if wl.M != len(rows):
            sample_note = " (heads timed on the %d rows that build the trees, scaled to all %d rows)" % (
                len(rows), wl.M)
        return tok, heads, (time.perf_counter() - ta) * (wl.M / len(rows))

    def oracle_rest(x, tok, heads, logits):
        """The rest of the oracle's step (attention, verification, acceptance, compaction), and its time."""
        tc = time.perf_counter()
        oracle.tree_attention(topo.parent, x["q"], x["Kc"], x["Vc"], x["lens"])
        vmargin = np.inf
        if wl.target_head:
            tstar, _, tm = oracle.target_argmax(x["Ht"].reshape(wl.B * topo.n, wl.d), w["Wt"])
            tstar, vmargin = tstar.reshape(wl.B, topo.n), float(np.min(tm))
        elif wl.verify == "sampled":  # the token after every node the walk passes through
            vs = oracle.verify_sampled(topo.parent, tok, logits, heads["logits"], wl.temperature, x["u_words"],
                                       x["g_words"])
            tstar, vmargin = vs["chosen"], float(np.min(vs["margin"]))
        elif wl.verify == "typical":
            ty = oracle.typical_accept(topo.parent, tok, logits, wl.temperature, wl.eps, wl.delta, x["g_words"])
            tstar, vmargin = ty["chosen"], float(np.min(ty["margin"]))
        else:
            tstar = oracle.argmax(logits)
        r = oracle.accept(topo.parent, wl.K, tok, tstar, x["lens"])
        oracle.compact(x["Kc"], x["Vc"], x["lens"], r["accept_len"], r["path"], wl.K)
        r["margin"] = min(vmargin, float(np.min(heads["margin"])) if heads is not None else np.inf)
        return r, time.perf_counter() - tc

    first = None
    for s in range(args.sets):
        x = step_inputs(wl, args.seed, step=s)
        tok, heads, heads_time = oracle_tree(x)
        if wl.target_head:  # verification through the target's LM head: plant its hidden states
            plant_hidden(x["Ht"], w["Wt"], topo, tok, wl.a, seed=args.seed, step=s)
            logits = None
        elif wl.verify == "greedy":
            logits = plant(x["logits"], topo, tok, wl.a, seed=args.seed, step=s)
        else:  # sampled decoding: the target's logits as drawn, N(0, 1)
            logits = x["logits"]
        if s < args.cpu_steps:
            r, rest_time = oracle_rest(x, tok, heads, logits)
            cpu_times.append(heads_time + rest_time)
            acc_oracle.append([int(v) for v in r["accept_len"]])
            oracle_margin.append(r["margin"])
            log("oracle step %d: %.2f s (accept_len %s)" % (s, cpu_times[-1], acc_oracle[-1]))
            if first is None:
                first = x
        xd = {k: to_dev(v) for k, v in x.items() if k != "logits"}
        if not wl.target_head:
            xd["logits"] = to_dev(logits)
        xd["lens0"] = xd["lens"].clone()
        sets.append(xd)
    torch.cuda.synchronize()
    log("%d input sets on the GPU" % len(sets))
    cpu_1thread = None
    if first is not None and args.cpu_1thread:  # the same oracle step on one thread
        oracle.set_threads(1)
        tok1, heads1, t1 = oracle_tree(first)
        _, t2 = oracle_rest(first, tok1, heads1, first.get("logits"))  # the logits were planted in place
        oracle.set_threads(threads)
        cpu_1thread = t1 + t2
        log("oracle step on 1 thread: %.2f s" % cpu_1thread)

    kind = md.MD_HEADS_HYDRA if hydra else (md.MD_HEADS_MEDUSA_SHARED if wl.shared_u else md.MD_HEADS_MEDUSA)
    cfg = md.StepConfig(kind=kind,
                        dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32, B=wl.B,
                        M=wl.B if hydra else wl.M, d=wl.d, V=wl.V, K=wl.K, k_per_head=wl.topk, parent=topo.parent,
                        rank=topo.rank, Hq=wl.Hq, Hkv=wl.Hkv, hd=wl.hd, Lcap=wl.Lcap, max_len=wl.L_max,
                        target_head=wl.target_head, verify=wl.verify, temperature=wl.temperature, eps=wl.eps,
                        delta=wl.delta)
    step = md.MedusaStep(cfg)
    use_op = args.operand_order == "on" or (args.operand_order == "auto" and wl.dtype == "bf16"
                                             and (hydra or wl.target_head or wl.shared_u))
    if use_op:  # made once with the weights, outside every timed region
        wd.update(step.operand_order_weights(wd))
        torch.cuda.synchronize()
        log("operand-order copies: %s" % ", ".join(k for k in ("U_op", "W_op", "Wt_op") if k in wd))
    use_tn = args.tile_norms == "on" or (args.tile_norms == "auto" and wl.dtype == "bf16" and not hydra
                                          and wl.M * (wl.K if wl.shared_u else 1) > 128)
    if use_tn:  # made once with the weights, outside every timed region
        wd.update(step.tile_norm_weights(wd))
        torch.cuda.synchronize()
        log("tile norms of U: %d floats" % wd["U_norms"].numel())
    stream = torch.cuda.current_stream()
    calls = depth if hydra else 1  # heads calls per step, each with its own event pair
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
          for _ in range(args.steps)]
    lm_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)] if (wl.target_head or wl.verify != "greedy") else None
    for pairs in ev + ([lm_ev] if lm_ev else []):  # materialise the underlying hipEvent_t handles
        for a, b in pairs:
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()

    # every step starts from its set's cached lengths: each step gets its own
    # copy of them (the step grows them)

    def one_step(i: int, pairs=None, lm=None, lens=None):
        xd = dict(sets[i % len(sets)])
        xd["lens"] = lens
        for lvl in range(calls):
            if pairs is not None:
                md.md_set_vocab_timing_events(pairs[lvl][0].cuda_event, pairs[lvl][1].cuda_event)
            if hydra:
                step.heads(xd["h"], wd["W"], wd["b"], wd["U"], E=wd["E"], root_tok=xd["root_tok"], level=lvl + 1,
                           U_op=wd.get("U_op"), W_op=wd.get("W_op"))
                step.build(None, xd["root_tok"], xd["lens"], level=lvl + 1)
            elif wl.verify == "sampled":
                step.heads_logits(xd["h"], wd["W"], wd["b"], wd["U"])
            else:
                step.heads(xd["h"], wd["W"], wd["b"], wd["U"], U_op=wd.get("U_op"), U_norms=wd.get("U_norms"),
                           W_op=wd.get("W_op"))
            if pairs is not None:
                md.md_set_vocab_timing_events(None, None)
        if wl.verify == "sampled":
            step.draft(xd["draft_words"])
        if not hydra:
            step.build(xd["src_row"], xd["root_tok"], xd["lens"])
        step.attention(xd["q"], xd["Kc"], xd["Vc"], xd["lens"])
        if lm is not None:
            lm[0].record(stream)
        if wl.target_head:
            step.verify(xd["Ht"], wd["Wt"], wd.get("Wt_op"))
            if lm is not None:
                lm[1].record(stream)
            step.accept_tokens(xd["Kc"], xd["Vc"], xd["lens"])
        elif wl.verify == "sampled":
            step.verify_sampled(xd["logits"], xd["u_words"], xd["g_words"], xd["Kc"], xd["Vc"], xd["lens"])
        elif wl.verify == "typical":
            step.accept_typical(xd["logits"], xd["g_words"], xd["Kc"], xd["Vc"], xd["lens"])
        else:
            step.accept(xd["logits"], xd["Kc"], xd["Vc"], xd["lens"])
        if lm is not None and not wl.target_head:
            lm[1].record(stream)

    # outside every timed region: one step on every input set the oracle ran,
    # its accepted lengths against the oracle's (bit for bit; a difference is
    # allowed only where the oracle saw a decision within tau of a tie)
    acc_gpu, acc_check = [], []
    for i in range(len(acc_oracle)):
        one_step(i, lens=sets[i]["lens0"].clone())
        acc_gpu.append([int(v) for v in step.accept_len.cpu().numpy()])
        if acc_gpu[-1] == acc_oracle[i]:
            acc_check.append("equal")
        elif oracle_margin[i] <= 1e-4:
            acc_check.append("near tie (oracle margin %.2g)" % oracle_margin[i])
        else:
            acc_check.append("DIFFERENT")
    mismatch = [i for i, c in enumerate(acc_check) if c == "DIFFERENT"]
    log("accepted lengths, GPU vs oracle, %d input sets: %s" % (len(acc_gpu), "all equal" if all(
        c == "equal" for c in acc_check) else acc_check))
    # warm-up: a fixed count, or by default steps until 0.5 s have passed (with
    # 10 warm-up steps the first ~100 timed steps of the Hydra workload ran
    # 1.03 ms against 0.91 ms once the clocks had settled); each step gets a
    # fresh copy of its set's lengths
    n_warm = 0
    t_warm = time.perf_counter()
    while (n_warm < args.warmup) if args.warmup >= 0 else (time.perf_counter() - t_warm < 0.5):
        for _ in range(1 if args.warmup >= 0 else 10):
            one_step(n_warm, lens=sets[n_warm % len(sets)]["lens0"].clone())
            n_warm += 1
        if args.warmup < 0:
            torch.cuda.synchronize()
    args.warmup = n_warm
    # every timed step's own copy of its set's lengths, made before timing
    lens_bank = [sets[(n_warm + i) % len(sets)]["lens0"].clone() for i in range(2 * args.steps)]
    torch.cuda.synchronize()
    # the timed steps: nothing but the steps between the two events (a HIP
    # event recorded between two kernels costs ~6 us of GPU time here)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        one_step(args.warmup + i, lens=lens_bank[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    # the same number of steps again, now with HIP events around the vocabulary
    # kernel (recorded by the library on its stream) and the verification, and
    # one at every step boundary for the distribution of step times
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    bounds[0].record(stream)
    for i in range(args.steps):
        one_step(args.warmup + args.steps + i, ev[i], lm_ev[i] if lm_ev else None, lens=lens_bank[args.steps + i])
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)])
    vocab_ms = sum(a.elapsed_time(b) for pairs in ev for a, b in pairs) / args.steps
    acc_len = step.accept_len.cpu().numpy().tolist()

    # attainable HBM read bandwidth on this GPU: the library's plain streaming-read probe over 4 GiB
    probe_buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(md.md_hbm_read_probe_blocks(), dtype=torch.int32, device=dev)
    for _ in range(2):
        md.md_hbm_read_probe(probe_buf, probe_buf.numel(), sink)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for _ in range(10):
        md.md_hbm_read_probe(probe_buf, probe_buf.numel(), sink)
    p1.record(stream)
    torch.cuda.synchronize()
    stream_gbs = probe_buf.numel() * 10 / (p0.elapsed_time(p1) * 1e-3) / 1e9
    del probe_buf

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")

    esz = 2 if wl.dtype == "bf16" else 4
    # heads rows per step: Medusa M; Hydra the parents of every level of every request
    if hydra:
        head_rows = [wl.B * len(oracle.hydra_rows(topo.parent, lvl)) for lvl in range(1, depth + 1)]
    else:
        head_rows = [wl.M] * wl.K
    # U bytes read per step: one matrix per head (per level for Hydra), or one shared by the heads
    u_reads = depth if hydra else (1 if wl.shared_u else wl.K)
    vocab_bytes = u_reads * wl.V * wl.d * esz
    vocab_bytes += sum(head_rows) * wl.d * 4
    if wl.verify == "sampled":  # the logits kernel writes every logit
        vocab_bytes += sum(head_rows) * wl.V * 4
    vocab_flops = 2.0 * wl.V * wl.d * sum(head_rows)  # algorithmic multiply-adds of the projections
    kernel = "vocabulary projection + per-head top-k"
    # one bf16 row through per-head projections: residual blocks, projections, top-k and merge in
    # one launch, which then reads W and b as well (and h, not h')
    fused = (not hydra and wl.verify != "sampled"
             and md.md_heads_fused(kind, 1 if wl.dtype == "bf16" else 0, wl.M, wl.d, wl.K))
    if fused:
        vocab_bytes = md.md_heads_weight_bytes(kind, 1, wl.d, wl.V, wl.K) + wl.M * wl.d * 2
    mfma_rows = min(head_rows) >= 8 and wl.dtype == "bf16"
    if mfma_rows:
        achieved = vocab_flops / (vocab_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                    "kernel": "k_vocab_mfma_cert (%s; one bf16 product per term, the candidates that a "
                              "Cauchy-Schwarz bound cannot exclude re-scored in float32 by k_rescore)" % kernel,
                    "kernel_ms": round(vocab_ms, 4), "flops_per_step": vocab_flops}
    else:
        achieved = vocab_bytes / (vocab_ms * 1e-3) / 1e9
        traffic = None
        if os.path.exists(PMC_FILE):
            with open(PMC_FILE) as f:
                pmc = json.load(f)
            if pmc.get("heads_hip_sha256") == file_sha(os.path.join(ROOT, "medusa_draft_heads_amd", "csrc",
                                                                     "heads.hip")) \
                    and pmc.get("workload") == args.workload:
                traffic = pmc.get("hbm_bytes_per_launch")
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "kernel": ("vocabulary kernels of the 4 levels" if hydra else
                               "k_heads_fused (residual blocks + vocabulary projections + per-head top-k + their "
                               "merge, one launch)" if fused else
                               "k_vocab_topk<..., LOGITS> (vocabulary projection writing every logit)"
                               if wl.verify == "sampled" else
                               "k_vocab_topk (%s%s)" % (kernel, "; one U for the %d heads" % wl.K if wl.shared_u
                                                        else "")),
                    "kernel_ms": round(vocab_ms, 4), "bytes_per_launch": vocab_bytes,
                    "stream_read_GBps": round(stream_gbs, 1), "frac_of_stream_read": round(achieved / stream_gbs, 4)}
    # verification input: the logits, or the hidden states plus the LM head through the fused argmax
    verify_bytes = (wl.V * wl.d * esz + wl.B * wl.N * wl.d * esz) if wl.target_head else wl.B * wl.N * wl.V * 4
    if wl.verify == "sampled":  # head logits written and read back, the draft words, the final draw's words
        verify_bytes += 2 * wl.M * wl.K * wl.V * 4 + wl.M * wl.K * wl.V * 4 + wl.B * wl.V * 4
    elif wl.verify == "typical":
        verify_bytes += wl.B * wl.V * 4
    step_bytes = (md.md_heads_weight_bytes(kind, 1 if esz == 2 else 0, wl.d, wl.V, wl.K)
                  + 2 * wl.B * wl.Hkv * (wl.L_max + wl.N) * wl.hd * esz  # K and V of prefix + tree (upper bound)
                  + 2 * wl.B * wl.N * wl.Hq * wl.hd * esz  # q in, attention out
                  + verify_bytes)
    lm_head = verification = None
    if lm_ev and not wl.target_head:
        vms = sum(a.elapsed_time(b) for a, b in lm_ev) / args.steps
        verification = {"kernels": "rejection-sampling walk + acceptance and compaction (md_tree_verify_sampled)"
                        if wl.verify == "sampled" else
                        "row statistics + typical acceptance + acceptance and compaction (md_tree_accept_typical)",
                        "ms": round(vms, 4), "temperature": wl.temperature}
        if wl.verify == "typical":
            verification.update({"eps": wl.eps, "delta": wl.delta})
    elif lm_ev:
        lm_ms = sum(a.elapsed_time(b) for a, b in lm_ev) / args.steps
        lm_gbs = verify_bytes / (lm_ms * 1e-3) / 1e9
        lm_head = {"kernels": "target LM head + fused argmax (md_target_argmax)", "ms": round(lm_ms, 4),
                   "bytes": verify_bytes, "GBps": round(lm_gbs, 1), "frac": round(lm_gbs / PEAK_HBM_GBS, 4),
                   "flops": 2.0 * wl.B * wl.N * wl.V * wl.d}
    cpu = None
    if cpu_times:
        cpu = {"value": round(1.0 / float(np.median(cpu_times)), 4), "unit": "steps/s", "cores": threads,
               "kind": "oracle",
               "sample": "%d whole oracle steps (heads, tree, attention, argmax, accept, compaction) on the same "
                         "seeded inputs, median%s" % (len(cpu_times), sample_note),
               "cpu_model": cpu_model()}
        if cpu_1thread:
            cpu["value_1_thread"] = round(1.0 / cpu_1thread, 4)
    E = 1.0
    run = 1.0
    for ai in wl.a:
        run *= ai
        E += run
    out = {
        "metric": "Medusa tree-decode steps/s at 70B-shaped heads, batch 1; achieved HBM GB/s % peak",
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_distribution": {"median": round(float(np.median(per_step)), 4),
                                 "p10": round(float(np.percentile(per_step, 10)), 4),
                                 "p90": round(float(np.percentile(per_step, 90)), 4),
                                 "pass": "the instrumented pass: every step also records its boundary event and the "
                                         "kernel events (~6 us of GPU time each)"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded Philox inputs, random-init heads of the workload's shape)",
        "config": {"workload": wl.name, "batch": wl.B, "d": wl.d, "V": wl.V, "heads": wl.K, "topk": list(wl.topk),
                   "tree_nodes": wl.N, "heads_rows_per_step": sum(head_rows), "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "head_dim": wl.hd, "L": wl.L_max, "input_sets": len(sets),
                   "weights_layout": "row-major + operand-order copy" if use_op else "row-major",
                   "tile_norms": bool(use_tn)},
        "roofline": roofline,
        "step_hbm": {"bytes_per_step": step_bytes, "GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "stream_read_GBps": round(stream_gbs, 1),
        "acceptance": {"last_step_accept_len": acc_len, "gpu_accept_len": acc_gpu, "oracle_accept_len": acc_oracle,
                       "gpu_vs_oracle": "equal on all %d input sets" % len(acc_gpu)
                       if all(c == "equal" for c in acc_check) else acc_check,
                       "E_closed_form": round(E, 4)},
        "cpu_baseline": cpu,
    }
    if lm_head:
        out["lm_head"] = lm_head
    if verification:
        out["verification"] = verification
        out["acceptance"].pop("E_closed_form")
    print(json.dumps(out), flush=True)
    if mismatch:
        log("GPU accepted lengths differ from the oracle's on input sets %s" % mismatch)
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
