"""Benchmark of the verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --workload full-model|sweep|masked-head|filtered|drafter|rounds

One step is one verify pass of the large-vocabulary workload: bf16 LM head
W[262144, 1536] (about 805 MB), final hidden states [B=1, gamma+1=5, 1536],
gamma = 4 drafts with a bf16 draft distribution q, temperature 1: logits of
all five slots, vocab-wide softmax statistics, the min(1, p/q) acceptance
test, the residual/bonus resample and the commit of n_accepted / tokens.
Inputs are seeded synthetic arrays resident in HBM before timing starts; step i
verifies one of eight input sets at its own positions (pos0 + 11 i), so
acceptance and the random draws vary from step to step.

Prints one JSON line: the metric is committed (verified) tokens per second,
sum over steps of (n_accepted + 1) divided by the timed wall time between two
device synchronisations.  ``roofline`` reports the fused verify kernel (the
whole step is one launch): algorithmic bytes per launch (W once, the hidden
states, the q row of a rejected step) over its average duration measured with
HIP events on the stream the library launches it on (one event pair around the
timed loop, so launch gaps are included), against the 8 TB/s HBM peak.
``config`` also carries:
- the acceptance per slot and the mean committed tokens of the timed steps;
- the greedy rule (T = 0) on the same table;
- the d = 4096 head's B = 1, gamma = 4 point;
- the settle phase: before tuning and timing, the sampling step runs untimed for
  --settle-seconds (5 s by default), since the device's clocks ramp with load.
``cpu_baseline`` times the CPU oracle (float64 numpy) on a bounded sample of
the same workload: three warm-up steps, then the median of the timed ones.  It
reports the core counts, a spot check of the oracle against the GPU's decisions,
and the pages' closed form for the expected committed tokens from the
measured alpha = sum_v min(p, q) per slot.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "verified tokens/s + verify-step HBM GB/s (% of MI355X peak), γ=4, V=262144"
HBM_PEAK_GBS = 8000.0
N_SETS = 8
POS_STRIDE = 11            # positions between consecutive timed steps (more than gamma + 1)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-seconds", type=float, default=5.0,
                    help="run the workload's step untimed for this long before the tuning, the warm-up and "
                         "the timed region (the device's clocks ramp with load; sweep: before its first point)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB five times (a plain copy kernel of known "
                         "size, used to scale the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--workload", choices=("large-vocab", "full-model", "masked-head", "filtered", "drafter",
                                           "rounds", "sweep"),
                    default="large-vocab",
                    help="large-vocab (default, the headline metric), full-model (the 32-layer decoder verify), "
                         "masked-head (the drafter's centroid-masked LM head), filtered (the large-vocab step "
                         "with top_k 64 / top_p 0.95 applied alike to the target), drafter (the MTP drafter's "
                         "gamma = 4 draft steps), rounds (draft, per-sequence padding, verify and the heuristic "
                         "schedule, on the device) or sweep (the batch x gamma sweep over the d = 4096 head: "
                         "B in {1, 4, 16, 64} x gamma in {2, 4, 8}, T = 1 sampling)")
    ap.add_argument("--rows", type=int, default=1, help="masked-head: hidden states per call")
    ap.add_argument("--graph", action="store_true",
                    help="drafter, full-model: capture one call into a HIP graph (torch.cuda.graph on the launch "
                         "stream) and time its replays instead of eager calls")
    ap.add_argument("--traffic-summary", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                                              "k_head_vocab262144_d1536_B1_traffic.md"))
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (got --gpus {args.gpus}); "
              "multi-GPU sharding of the verify step is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    import torch
    import accept_step_amd as sv
    import workloads

    if args.workload == "full-model":
        return full_model(args, torch, sv)
    if args.workload == "masked-head":
        return masked_head(args, torch, sv, workloads)
    if args.workload == "filtered":
        return filtered(args, torch, sv, workloads)
    if args.workload == "drafter":
        return drafter(args, torch, sv, workloads)
    if args.workload == "rounds":
        return rounds_bench(args, torch, sv, workloads)
    if args.workload == "sweep":
        return sweep(args, torch, sv)
    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs (resident in HBM before timing): the large-vocab workload at T = 1 (the
    # headline) and T = 0, eight independent input sets each over one table
    B, gamma, T = 1, 4, 1.0
    V, d = 262144, 1536
    cases, cases0, w = [], [], None
    for s_ in range(N_SETS):
        cs = workloads.lm_head_case(V, d, B, gamma, T, 1.0, 3, w=w, pos0=7 * s_, variant=s_)
        w = cs.w
        cases.append(cs)
        cases0.append(workloads.lm_head_case(V, d, B, gamma, 0.0, 1.0, 3, w=w, pos0=7 * s_, variant=s_))
    W = to_dev_bf16(w)
    model = sv.lm_head_model(W)
    sets = [(to_dev_bf16(cs.h), torch.from_numpy(cs.draft.astype(np.int32)).to(dev), to_dev_bf16(cs.q))
            for cs in cases]
    # step i verifies at positions pos0 + POS_STRIDE * i, so every step draws its own
    # acceptance uniforms and noise (as consecutive rounds of one sequence would)
    pos_all = torch.from_numpy(np.stack([cases[i % N_SETS].pos0 + POS_STRIDE * i
                                         for i in range(max(args.steps, args.warmup))])).to(dev)
    sets0 = [(to_dev_bf16(cs.h), torch.from_numpy(cs.draft.astype(np.int32)).to(dev)) for cs in cases0]
    K, Wm = args.steps, args.warmup
    n_out = torch.empty((K, B), dtype=torch.int32, device=dev)
    t_out = torch.empty((K, B, gamma + 1), dtype=torch.int32, device=dev)
    ws = sv.Workspace()
    seed = cases[0].seed

    # ---- settle.  The device's clocks follow its load: after minutes of light work (a
    # test run) the first seconds of this step ran about 3.5 % slower (133.3, 131.7, then
    # 128.6 us per launch at two-second intervals, steady after), while a device that
    # had been idle ran at full speed at once.  The same sampling step therefore runs
    # untimed for --settle-seconds before the tuning, the warm-up and the timed region.
    settle_steps = 0
    t_settle = time.perf_counter() + max(args.settle_seconds, 0.0)
    while time.perf_counter() < t_settle:
        for _ in range(50):
            h, dr, q = sets[settle_steps % N_SETS]
            sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, h, B, gamma, dr, q, T, seed,
                                  pos_all[settle_steps % len(pos_all)], ws=ws)
            settle_steps += 1
        torch.cuda.synchronize()

    # the fused step's load grouping for this device (a setup call; same bits either way)
    tuned = sv.tune_verify(model, B, gamma)

    def step(i, out=None):
        h, dr, q = sets[i % N_SETS]
        return sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, h, B, gamma, dr, q, T, seed, pos_all[i], out=out, ws=ws)

    def step0(i, out=None):
        h, dr = sets0[i % N_SETS]
        return sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, h, B, gamma, dr, out=out, ws=ws)

    if args.calibration_copy_mib:
        src = torch.empty(args.calibration_copy_mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- timed region.  One pair of HIP events on the stream the library launches on
    # (torch's current stream) brackets the K launches: at this batch a step is one
    # launch of the fused kernel, so the event time over K is that kernel's average
    # duration per launch, launch gaps included (an upper bound on its own duration).
    # Events around every launch would cost the GPU ~7 us per step on this system.
    stream = torch.cuda.current_stream()

    def timed(fn, steps, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            fn(i, out=(n_out[i], t_out[i]))
        ev1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, ev0.elapsed_time(ev1)

    elapsed, gemm_ms = timed(step, K, Wm)
    gemm_n = K
    n_host = n_out.to(torch.int64).cpu()
    tok_host = t_out.cpu().numpy()
    require_valid(n_host, "large-vocab")
    committed = int((n_host + 1).sum().item())
    value = committed / elapsed
    ms_per_step = elapsed / K * 1e3
    gemm_avg_s = gemm_ms / max(gemm_n, 1) * 1e-3
    # algorithmic bytes of one step: W once, the hidden states, and the q row of each
    # rejected sequence (the residual draw); the q gathers at the drafts are negligible
    rejected = int((n_host < gamma).sum().item())
    algo_bytes = V * d * 2 + B * (gamma + 1) * d * 2 + rejected * V * 2 / K
    achieved = algo_bytes / gemm_avg_s / 1e9
    traffic = committed_traffic(args.traffic_summary, root)
    # acceptance of the timed steps: per slot, the rate of acceptance given the slot was
    # reached, and the mean committed tokens per step
    nn = n_host.numpy().reshape(-1)
    alpha = [float((nn > i).sum() / max((nn >= i).sum(), 1)) for i in range(gamma)]

    # ---- the greedy rule (T = 0) on the same table.  The host work above leaves the
    # device idle for a moment, and without a settle phase the first ~60 greedy launches
    # ran at 130-153 us before coming down to 117-120
    n_h1, tok_h1 = n_host.clone(), tok_host.copy()
    settle0 = settle(torch, step0, args.settle_seconds)
    el0, ms0 = timed(step0, K, Wm)
    n0_host = n_out.to(torch.int64).cpu()
    require_valid(n0_host, "large-vocab T=0")
    us0 = ms0 / K * 1e3
    algo0 = V * d * 2 + B * (gamma + 1) * d * 2

    # ---- configuration 4's B = 1, gamma = 4 point (d = 4096, 2,147,483,648 bytes of W)
    c4 = workloads.batch_sweep(B=1, gamma=4)
    model4 = sv.lm_head_model(to_dev_bf16(c4.w))
    set4 = (to_dev_bf16(c4.h), torch.from_numpy(c4.draft.astype(np.int32)).to(dev), to_dev_bf16(c4.q),
            torch.from_numpy(c4.pos0).to(dev))
    del c4

    def step4(i, out=None):
        h, dr, q, p0 = set4
        return sv.spec_verify_sample(model4, sv.SV_IN_HIDDEN, h, 1, 4, dr, q, 1.0, seed + 1, p0, out=out, ws=ws)

    # the table's generation left the device idle: settle again before tuning and timing
    settle4 = settle(torch, step4, args.settle_seconds)
    tuned4 = sv.tune_verify(model4, 1, 4)

    K4 = max(1, K // 2)
    el4, ms4 = timed(step4, K4, max(2, Wm // 2))
    n4 = n_out[:K4].to(torch.int64).cpu()
    require_valid(n4, "config-4 B=1")
    us4 = ms4 / K4 * 1e3
    algo4 = 262144 * 4096 * 2 + 5 * 4096 * 2 + int((n4 < 4).sum().item()) * 262144 * 2 / K4
    del model4, set4

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "large-vocab verify: bf16 LM head V=262144 d=1536, B=1, gamma=4, T=1.0 sampling "
                               "(min(1,p/q) accept, residual/bonus resample)",
                   "B": B, "gamma": gamma, "V": V, "d": d, "temperature": T,
                   "committed_tokens": committed, "candidate_positions_per_s": round(B * (gamma + 1) * K / elapsed, 1),
                   "verify_steps_per_s": round(K / elapsed, 1),
                   "step_hbm_gbs": round(algo_bytes / (elapsed / K) / 1e9, 1),
                   "step_frac_of_peak": round(algo_bytes / (elapsed / K) / 1e9 / HBM_PEAK_GBS, 4),
                   "fused_step_item_size": tuned,
                   "settle": {"seconds": args.settle_seconds, "untimed_steps": settle_steps},
                   "acceptance_per_slot": [round(a_, 4) for a_ in alpha],
                   "mean_committed_per_step": round(float((nn + 1).mean()), 4),
                   "greedy_T0": {"settle_untimed_calls": settle0, "us_per_step": round(us0, 2),
                                 "verified_tokens_per_s": round(
                       int((n0_host + 1).sum().item()) / el0, 1),
                       "step_hbm_gbs": round(algo0 / (us0 * 1e-6) / 1e9, 1),
                       "step_frac_of_peak": round(algo0 / (us0 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
                   "config4_B1_gamma4_T1": {"workload": "bf16 LM head V=262144 d=4096, B=1, gamma=4, T=1.0",
                                            "fused_step_item_size": tuned4, "settle_untimed_calls": settle4,
                                            "us_per_step": round(us4, 2),
                                            "step_hbm_gbs": round(algo4 / (us4 * 1e-6) / 1e9, 1),
                                            "step_frac_of_peak": round(algo4 / (us4 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}},
        "roofline": {"bound": "hbm", "kernel": "k_head (fused verify step: LM-head product, row statistics, "
                                                "acceptance, residual/bonus draw, commit)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(algo_bytes), "avg_launch_us": round(gemm_avg_s * 1e6, 2),
                     "timing": "HIP events around the timed loop on the launch stream (duration per launch, gaps included)",
                     "launches": gemm_n},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cases, args.cpu_seconds, elapsed / K, n_h1.numpy(), tok_h1)
        # the pages' alpha = sum_v min(p, q) per slot over the sampled steps, and the
        # expected committed tokens 1 + sum_k prod_{i<k} alpha_i ([Infra-ch8] "how the
        # benefit is computed"), beside the measured mean of the timed steps
        out["config"]["alpha_sum_min_pq_per_slot"] = out["cpu_baseline"].pop("alpha_per_slot")
        out["config"]["expected_committed_closed_form"] = out["cpu_baseline"].pop("expected_committed")
    print(json.dumps(out), flush=True)


def sweep(args, torch, sv):
    """The batch x gamma sweep: bf16 LM head W[262144, 4096] (2,147,483,648 bytes),
    B in {1, 4, 16, 64} x gamma in {2, 4, 8} (M = B (gamma + 1) from 3 to 576 rows),
    T = 1 sampling.  W, the hidden states N(0, 1) and the draft distributions are drawn
    on the GPU from a seeded generator: q = softmax(l + N(0, 1)) of the true logits l
    (bf16 product in torch), drafts drawn from q.  Per point: microseconds per verify
    step (HIP events around the timed launches on the launch stream), the step's
    algorithmic bytes (W once, the hidden states, the q rows of rejected sequences) per
    second against the 8 TB/s HBM peak, and MFMA utilisation 2 M V d / t against the
    2.5 PFLOP/s dense bf16 peak.  The points below M ~ 300 are bound by HBM, the largest
    by the matrix cores."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    V, d, T = 262144, 4096, 1.0
    gen = torch.Generator(device=dev)
    gen.manual_seed(4004)
    W = (torch.randn((V, d), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    model = sv.lm_head_model(W)
    ws = sv.Workspace()
    stream = torch.cuda.current_stream()
    K = max(2, min(args.steps, 50))
    points = []
    for B in (1, 4, 16, 64):
        for gamma in (2, 4, 8):
            M = B * (gamma + 1)
            h = torch.randn((B, gamma + 1, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            lt = (h[:, :gamma].reshape(-1, d) @ W.t()).float()
            lt += torch.randn(lt.shape, generator=gen, device=dev, dtype=torch.float32)
            q32 = torch.softmax(lt / T, dim=-1)
            draft = torch.multinomial(q32, 1, generator=gen).view(B, gamma).to(torch.int32)
            q = q32.to(torch.bfloat16).view(B, gamma, V)
            del lt, q32
            pos = torch.arange(0, 11 * (K + 4), 11, device=dev, dtype=torch.int64)[:, None].expand(-1, B).contiguous()
            n_out = torch.empty((K, B), dtype=torch.int32, device=dev)
            t_out = torch.empty((K, B, gamma + 1), dtype=torch.int32, device=dev)

            def step(i, out=None):
                return sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, h, B, gamma, draft, q, T, 77, pos[i], out=out,
                                             ws=ws)
            if not points:          # the first point brings the clocks up; the rest follow under load
                settled = settle(torch, lambda i: step(i % K), args.settle_seconds)
            for i in range(3):
                step(i)
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for i in range(K):
                step(i, out=(n_out[i], t_out[i]))
            ev1.record(stream)
            torch.cuda.synchronize()
            us = ev0.elapsed_time(ev1) / K * 1e3
            n_host = n_out.to(torch.int64).cpu()
            require_valid(n_host, f"sweep B={B} gamma={gamma}")
            rejected = int((n_host < gamma).sum().item()) / K
            algo = V * d * 2 + M * d * 2 + rejected * V * 2
            gbs = algo / (us * 1e-6) / 1e9
            tflops = 2.0 * M * V * d / (us * 1e-6) / 1e12
            points.append({"B": B, "gamma": gamma, "M": M, "us_per_step": round(us, 2),
                           "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                           "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / 2500.0, 4),
                           "mean_accepted": round(float(n_host.float().mean()), 3)})
            print(f"# sweep B={B} gamma={gamma} M={M}: {us:.1f} us, {gbs:.0f} GB/s, {tflops:.0f} TFLOP/s",
                  file=sys.stderr, flush=True)
            del h, q, draft, pos, n_out, t_out
    worst = min(points, key=lambda p_: max(p_["hbm_frac"], p_["mfma_frac"]))
    out = {
        "metric": "verify-step time over the batch x gamma sweep (HBM GB/s below the crossover, MFMA use above)",
        "value": round(sum(p_["us_per_step"] for p_ in points), 1),
        "unit": "us (sum of the 12 points' step times)",
        "n_gpus": 1, "steps": K, "warmup": 3, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "batch x gamma sweep: bf16 LM head V=262144 d=4096, T=1 sampling",
                   "points": points,
                   "furthest_from_its_roof": {k_: worst[k_] for k_ in ("B", "gamma", "M")}},
    }
    out["config"]["settle"] = {"seconds": args.settle_seconds, "untimed_calls": settled}
    print(json.dumps(out), flush=True)


def full_model(args, torch, sv):
    """The full-model verify: a 32-layer decoder (d 4096, 32 heads x 128, FFN 11008,
    vocabulary 32000, bf16 weights N(0, 0.02), norm gains 1), a KV cache of 2048
    positions, B = 1, gamma = 4, T = 1 sampling with a uniform draft distribution.
    Weights and cache are drawn on the GPU from a seeded generator.  One step = embed,
    32 layers, final norm, LM head, rule, draw, commit; the cache length is reset to
    2048 before each step so every step does the same work."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, d, H, hd, ff, V, C, B, gamma, T = 32, 4096, 32, 128, 11008, 32000, 2048, 1, 4, 1.0
    gen = torch.Generator(device=dev)
    gen.manual_seed(1005)

    def normal(shape, std):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)

    ones = torch.ones(d, dtype=torch.bfloat16, device=dev)
    layers = []
    for _ in range(L):
        layers.append({"attn_norm": ones, "wq": normal((H * hd, d), 0.02), "wk": normal((H * hd, d), 0.02),
                       "wv": normal((H * hd, d), 0.02), "wo": normal((d, H * hd), 0.02), "ffn_norm": ones,
                       "w_gate": normal((ff, d), 0.02), "w_up": normal((ff, d), 0.02), "w_down": normal((d, ff), 0.02)})
    embed, lm_head = normal((V, d), 0.02), normal((V, d), 0.02)
    model = sv.decoder_model(embed, layers, ones, lm_head, H, hd)
    max_len = C + gamma + 1
    kc = torch.zeros((L, B, H, max_len, hd), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    kc[:, :, :, :C] = normal((L, B, H, C, hd), 1.0)
    vc[:, :, :, :C] = normal((L, B, H, C, hd), 1.0)
    length = torch.full((B,), C, dtype=torch.int32, device=dev)
    kv = sv.KVCache(kc, vc, length)
    tokens = torch.randint(0, V, (B, gamma + 1), generator=gen, device=dev, dtype=torch.int32)
    q = torch.full((B, gamma, V), 1.0 / V, dtype=torch.float32, device=dev)
    pos0 = torch.full((B,), C, dtype=torch.int64, device=dev)
    ws = sv.Workspace()
    K, Wm = max(1, args.steps // 10), max(1, args.warmup // 4)
    n_out = torch.empty((K, B), dtype=torch.int32, device=dev)
    t_out = torch.empty((K, B, gamma + 1), dtype=torch.int32, device=dev)

    def step(out):
        length.fill_(C)
        return sv.spec_verify_sample(model, sv.SV_IN_TOKENS, tokens, B, gamma, None, q, T, 0x5EED0005, pos0, kv=kv,
                                     out=out, ws=ws)

    settled = settle(torch, lambda i: step(None), args.settle_seconds)
    for _ in range(Wm):
        step(None)
    torch.cuda.synchronize()
    graph = capture_graph(torch, lambda: step((n_out[0], t_out[0]))) if args.graph else None
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        if graph is not None:
            graph.replay()          # same inputs every step: the outputs of step 0 stand for all
        else:
            step((n_out[i], t_out[i]))
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / K
    if graph is not None:
        n_out[1:] = n_out[0]
    # per-part split from a separate run with per-launch events (decoder layers / LM-head step)
    sv.timing_enable(0b011)
    for _ in range(3):
        step(None)
    dec_ms, dec_n = sv.timing_read(1)
    head_ms, head_n = sv.timing_read(0)
    sv.timing_enable(0)
    weight_bytes = L * (4 * H * hd * d + 3 * ff * d) * 2
    kv_read = 2 * L * B * H * C * hd * 2
    kv_write = 2 * L * B * H * (gamma + 1) * hd * 2
    with_kv = weight_bytes + V * d * 2 + kv_read + kv_write + B * (gamma + 1) * d * 2
    params_bytes = weight_bytes + 2 * V * d * 2          # the 6.74B parameters incl. the embedding table
    require_valid(n_out.to(torch.int64).cpu(), "full-model")
    committed = int((n_out.to(torch.int64) + 1).sum().item())
    out = {
        "metric": "full-model verify step latency (ms/step) and HBM GB/s",
        "value": round(ms, 4), "unit": "ms/step", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full-model verify: 32-layer decoder d=4096, 32x128 heads, FFN 11008, V=32000, "
                               "KV cache 2048, B=1, gamma=4, T=1.0 sampling",
                   "launch": "HIP graph replay" if args.graph else "eager calls",
                   "verified_tokens_per_s": round(committed / elapsed, 1),
                   "bytes_weights_lm_head_kv": with_kv, "gbs_weights_lm_head_kv": round(with_kv / (ms * 1e-3) / 1e9, 1),
                   "frac_of_peak": round(with_kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "bytes_params": params_bytes, "gbs_params": round(params_bytes / (ms * 1e-3) / 1e9, 1),
                   "decoder_ms": round(dec_ms / max(dec_n, 1), 4), "lm_head_step_ms": round(head_ms / max(head_n, 1), 4)},
    }
    out["config"]["settle"] = {"seconds": args.settle_seconds, "untimed_calls": settled}
    print(json.dumps(out), flush=True)


def masked_head(args, torch, sv, workloads):
    """The drafter's centroid-masked LM head: V = 262144 token embeddings (d = 1536) in
    2048 clusters of 128, 32 clusters kept, ``--rows`` hidden states per call.  One step
    = one call (cluster scores, selection, member-token logits).  Algorithmic bytes: the
    cluster table once plus the kept clusters' rows of the token table per hidden state."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    V, d, C, top_k, M = 262144, 1536, 2048, 32, args.rows
    case = workloads.masked_head_case(V=V, d=d, C=C, M=M, top_k=top_k)

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    head = sv.masked_head(to_dev_bf16(case.w), to_dev_bf16(case.centroids))
    hs = [to_dev_bf16(workloads.normal_bf16((M, d), 1.0, 77, (M, i))) for i in range(8)]
    cs = V // C
    sel = torch.empty((M, top_k), dtype=torch.int32, device=dev)
    logits = torch.empty((M, top_k * cs), dtype=torch.float32, device=dev)
    ws = sv.Workspace()
    K, Wm = args.steps, args.warmup
    settled = settle(torch, lambda i: sv.draft_masked_logits(head, hs[i % 8], top_k, clusters=sel, logits=logits,
                                                             ws=ws), args.settle_seconds)
    for i in range(Wm):
        sv.draft_masked_logits(head, hs[i % 8], top_k, clusters=sel, logits=logits, ws=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        sv.draft_masked_logits(head, hs[i % 8], top_k, clusters=sel, logits=logits, ws=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = ev0.elapsed_time(ev1) / K * 1e3
    algo = C * d * 2 + M * top_k * cs * d * 2 + M * d * 2
    out = {
        "metric": "drafter masked LM-head latency (us/call) and HBM GB/s",
        "value": round(us, 2), "unit": "us/call", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"centroid-masked LM head: V={V} d={d}, {C} clusters of {cs}, top {top_k} kept, "
                               f"{M} hidden state(s) per call",
                   "scored_tokens_per_row": top_k * cs, "algorithmic_bytes": algo,
                   "gbs": round(algo / (us * 1e-6) / 1e9, 1),
                   "frac_of_peak": round(algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "full_head_bytes": V * d * 2, "full_head_us_at_peak": round(V * d * 2 / (HBM_PEAK_GBS * 1e3), 2)},
    }
    out["config"]["settle"] = {"seconds": args.settle_seconds, "untimed_calls": settled}
    print(json.dumps(out), flush=True)


def filtered(args, torch, sv, workloads):
    """The large-vocabulary step with the deployment's sampling filters (top_k 64,
    top_p 0.95, T = 1) applied to the target as the drafter applied them: the LM-head
    product (logits to the workspace), the top-k of every 4096-logit chunk, the per-row
    top-k with the top-p cut, and the rule.  B = 1, gamma = 4, V = 262144, d = 1536.
    q is the drafter's unfiltered distribution of the large-vocab workload (the rule
    uses q as given; only its values at the drafts and the kept tokens are read), so
    acceptance is lower than with a filtering drafter; the step's cost does not depend
    on it.  The value is microseconds per step from HIP events around the timed loop."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, gamma, T, top_k, top_p, V, d = 1, 4, 1.0, 64, 0.95, 262144, 1536

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    cases, w = [], None
    for s_ in range(N_SETS):
        cs = workloads.lm_head_case(V, d, B, gamma, T, 1.0, 3, w=w, pos0=7 * s_, variant=s_)
        w = cs.w
        cases.append(cs)
    model = sv.lm_head_model(to_dev_bf16(w))
    sets = [(to_dev_bf16(cs.h), torch.from_numpy(cs.draft.astype(np.int32)).to(dev), to_dev_bf16(cs.q),
             torch.from_numpy(cs.pos0).to(dev)) for cs in cases]
    K, Wm = args.steps, args.warmup
    n_out = torch.empty((K, B), dtype=torch.int32, device=dev)
    t_out = torch.empty((K, B, gamma + 1), dtype=torch.int32, device=dev)
    ws = sv.Workspace()

    def step(i, out=None):
        h, dr, q, p0 = sets[i % N_SETS]
        return sv.spec_verify_sample_filtered(model, sv.SV_IN_HIDDEN, h, B, gamma, dr, q, T, top_k, top_p,
                                              cases[0].seed, p0, out=out, ws=ws)

    settled = settle(torch, lambda i: step(i % K), args.settle_seconds)
    for i in range(Wm):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        step(i, out=(n_out[i], t_out[i]))
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = ev0.elapsed_time(ev1) / K * 1e3
    n_host = n_out.to(torch.int64).cpu()
    require_valid(n_host, "filtered")
    committed = int((n_host + 1).sum().item())
    algo = V * d * 2 + B * (gamma + 1) * d * 2
    out = {
        "metric": "filtered verify-step latency (us/step), top_k 64 / top_p 0.95, gamma=4, V=262144",
        "value": round(us, 2), "unit": "us/step", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"large-vocab verify with aligned filters: bf16 LM head V={V} d={d}, B={B}, "
                               f"gamma={gamma}, T={T}, top_k={top_k}, top_p={top_p}",
                   "committed_tokens": committed, "verified_tokens_per_s": round(committed / elapsed, 1),
                   "step_hbm_gbs": round(algo / (us * 1e-6) / 1e9, 1),
                   "step_frac_of_peak": round(algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    out["config"]["settle"] = {"seconds": args.settle_seconds, "untimed_calls": settled}
    print(json.dumps(out), flush=True)


def drafter(args, torch, sv, workloads):
    """The MTP drafter's draft round: gamma = 4 steps for B = ``--rows`` sequences of a
    random-init drafter of the E2B shapes (V = 262144 shared token table, D = 1536,
    H = 256, four layers of 4 x 128 query heads reading 2048 cached positions, d_ff 2048,
    2048 clusters with 32 kept), T = 1, q in bf16.  The value is microseconds per round
    from HIP events around the timed loop.  Algorithmic bytes per step: the drafter's
    weights, the cluster table, the kept clusters' token rows and the cached keys and
    values each layer reads, once."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, gamma, T = args.rows, 4, 1.0
    c = workloads.drafter_case(B=B, length=2048, max_len=2048)

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    layers = [{k: to_dev_bf16(L[k]) for k in sv.DRAFTER_LAYER_KEYS} for L in c.layers]
    dr = sv.drafter(to_dev_bf16(c.embed), to_dev_bf16(c.pre_proj), layers, to_dev_bf16(c.final_norm),
                    to_dev_bf16(c.post_proj), c.n_heads, c.head_dim, centroids=to_dev_bf16(c.centroids),
                    top_k_clusters=c.top_k)
    cache = {}
    ks = [cache.setdefault(id(a), to_dev_bf16(a)) for a in c.kv_k]
    vs = [cache.setdefault(id(a), to_dev_bf16(a)) for a in c.kv_v]
    kv = sv.shared_kv(ks, vs, torch.from_numpy(c.length.astype(np.int32)).to(dev))
    tok = torch.from_numpy(c.last_token.astype(np.int32)).to(dev)
    hid = to_dev_bf16(c.h_target)
    draft = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    q = torch.empty((B, gamma, c.vocab), dtype=torch.bfloat16, device=dev)
    ws = sv.Workspace()
    K, Wm = args.steps, args.warmup
    settled = settle(torch, lambda i: sv.mtp_draft(dr, kv, tok, hid, gamma, T, 1234 + i, draft=draft, q=q, ws=ws),
                     args.settle_seconds)
    for i in range(Wm):
        sv.mtp_draft(dr, kv, tok, hid, gamma, T, 1234 + i, draft=draft, q=q, ws=ws)
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        graph = capture_graph(torch, lambda: sv.mtp_draft(dr, kv, tok, hid, gamma, T, 99, draft=draft, q=q, ws=ws))
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        if graph is not None:
            graph.replay()
        else:
            sv.mtp_draft(dr, kv, tok, hid, gamma, T, 99 + i, draft=draft, q=q, ws=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = ev0.elapsed_time(ev1) / K * 1e3
    if int((draft < 0).sum().item()):
        print("bench.py: the drafter returned invalid drafts; no result reported", file=sys.stderr)
        sys.exit(3)
    H, D, ff, HQ, L, C, cs = c.hidden, c.d_model, c.d_ff, c.n_heads * c.head_dim, len(c.layers), 2048, c.vocab // 2048
    weights = 2 * (H * 2 * D + L * (2 * H * HQ + 3 * H * ff) + D * H)
    head = 2 * (C * D + B * c.top_k * cs * D)
    kvb = 2 * 2 * L * B * 2048 * HQ
    algo = weights + head + kvb
    out = {
        "metric": "MTP draft round latency (us per gamma=4 steps) and HBM GB/s",
        "value": round(us, 2), "unit": "us/round", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"MTP drafter draft round: V={c.vocab} shared table, D={D}, H={H}, {L} Q-only layers "
                               f"of {c.n_heads}x{c.head_dim} over 2048 cached positions, d_ff={ff}, masked head "
                               f"{C} clusters top {c.top_k}, B={B}, gamma={gamma}, T={T}, q bf16",
                   "launch": "HIP graph replay" if args.graph else "eager calls",
                   "us_per_draft_step": round(us / gamma, 2), "algorithmic_bytes_per_step": algo,
                   "step_gbs": round(algo / (us / gamma * 1e-6) / 1e9, 1),
                   "step_frac_of_peak": round(algo / (us / gamma * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    out["config"]["settle"] = {"seconds": args.settle_seconds, "untimed_calls": settled}
    print(json.dumps(out), flush=True)


def rounds_bench(args, torch, sv, workloads):
    """Device-resident speculative rounds at gamma_max = 6 for B = ``--rows`` sequences:
    the MTP drafter of the drafter workload drafts 6 tokens, round_pad_drafts pads each
    sequence to its current draft length, the large-vocab verify (V = 262144, d = 1536,
    T = 1) checks the padded batch, and round_update_gamma applies the heuristic
    schedule; nothing returns to the host between rounds.  The target's hidden states
    are synthetic (no trained target), so acceptance is low and the schedule mostly
    shortens the drafts; the timing of the round's kernels is what this measures."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, G, T = args.rows, 6, 1.0
    c = workloads.drafter_case(B=B, length=2048, max_len=2048)

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    emb = to_dev_bf16(c.embed)
    layers = [{k: to_dev_bf16(L[k]) for k in sv.DRAFTER_LAYER_KEYS} for L in c.layers]
    dr = sv.drafter(emb, to_dev_bf16(c.pre_proj), layers, to_dev_bf16(c.final_norm), to_dev_bf16(c.post_proj),
                    c.n_heads, c.head_dim, centroids=to_dev_bf16(c.centroids), top_k_clusters=c.top_k)
    cache = {}
    ks = [cache.setdefault(id(a), to_dev_bf16(a)) for a in c.kv_k]
    vs = [cache.setdefault(id(a), to_dev_bf16(a)) for a in c.kv_v]
    kv = sv.shared_kv(ks, vs, torch.from_numpy(c.length.astype(np.int32)).to(dev))
    model = sv.lm_head_model(emb)                  # the target's head: the shared token table
    tok = torch.from_numpy(c.last_token.astype(np.int32)).to(dev)
    hid = to_dev_bf16(c.h_target)
    hs = [to_dev_bf16(workloads.normal_bf16((B, G + 1, c.d_model), 1.0, 55, (i, B))) for i in range(4)]
    pos0 = torch.from_numpy(c.length.astype(np.int64)).to(dev)
    gamma_b = torch.full((B,), 4, dtype=torch.int32, device=dev)
    draft = torch.empty((B, G), dtype=torch.int32, device=dev)
    q = torch.empty((B, G, c.vocab), dtype=torch.bfloat16, device=dev)
    K, Wm = args.steps, args.warmup
    n_all = torch.empty((K, B), dtype=torch.int32, device=dev)
    g_all = torch.empty((K, B), dtype=torch.int32, device=dev)
    t_out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    wsd, wsp, wsv = sv.Workspace(), sv.Workspace(), sv.Workspace()

    def one(i, n_out):
        sv.mtp_draft(dr, kv, tok, hid, G, T, 7 + i, draft=draft, q=q, ws=wsd)
        sv.round_pad_drafts(gamma_b, draft, q, ws=wsp)
        sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, hs[i % 4], B, G, draft, q, T, 99, pos0, out=(n_out, t_out),
                              ws=wsv)
        sv.round_update_gamma(n_out, gamma_b, 1, G)

    settled = settle(torch, lambda i: one(i, n_all[0]), args.settle_seconds)
    for i in range(Wm):
        one(i, n_all[0])
    torch.cuda.synchronize()
    gamma_b.fill_(4)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        g_all[i].copy_(gamma_b)
        one(i, n_all[i])
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = ev0.elapsed_time(ev1) / K * 1e3
    n_host = n_all.to(torch.int64).cpu()
    require_valid(n_host, "rounds")
    committed = int((n_host + 1).sum().item())
    out = {
        "metric": "device-resident speculative round latency (us per round: draft, pad, verify, schedule)",
        "value": round(us, 2), "unit": "us/round", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"rounds: MTP drafter (masked head) drafting {G}, per-sequence padding, large-vocab "
                               f"verify V={c.vocab} d={c.d_model} T={T}, heuristic schedule in [1, {G}], B={B}",
                   "committed_tokens": committed, "mean_gamma": round(float(g_all.float().mean().item()), 3),
                   "note": "synthetic target hidden states: acceptance is not meaningful"},
    }
    out["config"]["settle"] = {"seconds": args.settle_seconds, "untimed_calls": settled}
    print(json.dumps(out), flush=True)


def settle(torch, fn, seconds):
    """Call fn(i) untimed until ``seconds`` have passed, synchronising every eight calls
    (the device's clocks ramp with load; see main).  Returns the number of calls."""
    n = 0
    t_end = time.perf_counter() + max(seconds, 0.0)
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def capture_graph(torch, fn):
    """One eager warm-up call of ``fn`` on a side stream, then ``fn`` captured into a
    HIP graph.  Seeds and sizes become constants of the graph; lengths, positions and
    tokens stay device data, read at every replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def require_valid(n_host, what):
    """Every timed step must have produced a valid result (n_accepted >= 0): a step the
    library reports invalid did not run the whole path, so its time is not a measurement."""
    bad = int((n_host < 0).sum().item())
    if bad:
        print(f"bench.py: {bad} of {n_host.numel()} sequences in the timed {what} steps came back invalid "
              "(n_accepted = -1); no measurement is reported", file=sys.stderr)
        sys.exit(3)


def committed_traffic(path, root):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary, or
    None when the summary is missing or was taken on different kernel sources."""
    vals = {}
    try:
        for line in open(path):
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "kernel_source_hash"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    except OSError:
        return None
    if vals.get("kernel_source_hash") != kernel_source_hash(root):
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def kernel_source_hash(root):
    import hashlib
    h = hashlib.sha256()
    for f in ("sv_head.hpp", "sv_accept.hpp", "sv_gemm.hpp", "sv_device.hpp"):
        h.update(open(os.path.join(root, "accept_step_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(cases, budget_s, gpu_step_s, gpu_n, gpu_tok):
    """The oracle as it stands, on a bounded sample of the same workload: whole verify
    steps (float64 logits from the bf16 table, then the sampling rule) of the timed
    steps' input sets.  The method of [Self-spec] 5.1: three warm-up steps, then the
    median of at least five timed steps (more while the budget lasts).  Each oracle step
    is also compared with the GPU's output for the same input set (``gpu_n``/``gpu_tok``
    of the timed steps): the mismatches not flagged by the oracle must be zero."""
    from oracle import bf16 as obf16
    from oracle import rules
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = os.cpu_count() or 1
    checked = {"compared": 0, "mismatched": 0, "flagged": 0, "unflagged_mismatches": 0}
    alphas = []

    def one(j):
        cs = cases[j % len(cases)]
        h = obf16.bf16_to_f64(cs.h)
        V = cs.w.shape[0]
        logits = np.empty(h.shape[:-1] + (V,))
        for v0 in range(0, V, 32768):
            logits[..., v0:v0 + 32768] = rules.lm_head_logits(h, obf16.bf16_to_f64(cs.w[v0:v0 + 32768]))
        qf = (cs.q.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        n, tok, fl = rules.verify_sample(logits, cs.draft, qf, cs.temperature, cs.seed, cs.pos0 + POS_STRIDE * j)
        p = rules.target_probs(rules.f32_logits(logits[:, :-1]), cs.temperature).astype(np.float64)
        alphas.append(np.minimum(p, qf).sum(axis=-1).mean(axis=0))
        if j < len(gpu_n):
            same = (gpu_n[j] == n) & np.all(gpu_tok[j] == tok, axis=1)
            checked["compared"] += len(n)
            checked["mismatched"] += int((~same).sum())
            checked["flagged"] += int(fl.sum())
            checked["unflagged_mismatches"] += int((~same & ~fl).sum())
        return int((n + 1).sum())

    for j in range(3):
        one(j)
    times, committed, j = [], 0, 3
    t_start = time.perf_counter()
    while len(times) < 5 or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        committed += one(j)
        times.append(time.perf_counter() - t0)
        j += 1
        if len(times) >= 200:
            break
    med = float(np.median(times))
    per_step_tokens = committed / len(times)
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = os.cpu_count() or 1
    a_ = np.mean(alphas, axis=0)
    expected = 1.0 + sum(float(np.prod(a_[:k])) for k in range(1, len(a_) + 1))
    return {"value": round(per_step_tokens / med, 3), "unit": "verified tokens/s", "cores": int(blas),
            "alpha_per_slot": [round(float(x), 4) for x in a_], "expected_committed": round(expected, 4),
            "kind": "oracle", "os_cpu_count": os.cpu_count(), "sched_affinity": affinity,
            "sample": f"{len(times)} whole verify steps of the same workload timed after 3 warm-ups (float64 numpy "
                      f"oracle, bf16 table converted per 32768-row chunk inside the timed region); value = mean "
                      f"committed tokens per step / median step time",
            "ms_per_step_median": round(med * 1e3, 1), "gpu_speedup": round(med / gpu_step_s, 1),
            "parity_spot_check": checked}


if __name__ == "__main__":
    main()
