"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one chunkwise prefill pass -- gate, intra-chunk and inter-chunk
stages, all in libkda's HIP kernels -- over the million-token synthetic
workload: B=1, H=32, T=1,048,576, d_k=d_v=128, bf16 q/k/v/z, fp32
beta/A/state, g_min=-5.  kda_chunk_prefill runs it as a scan over 8 segments
(two state-only map passes, the scan, a full pass).  Inputs (34 GiB) are
resident in HBM before timing and far larger than the last-level cache, so
every step streams them from HBM.

Prints ONE JSON line: the prefill tokens/s as ``value`` with a ``roofline``
object for the pass; ``mid`` (B1 H32 T4096) and ``batched`` (B8 H32 T32768,
carried state) prefill objects with their own rooflines (cold inputs:
the steps cycle through copies); ``decode`` (B=256, 1,000 back-to-back
in-place steps), ``decode_paged`` (states in a slot-addressed pool),
``verify`` (T drafted tokens per sequence from a live state) and
``backward`` (gradients of the mid prefill) objects; and the fp64 CPU oracle
timed on the host's cores on the first 16,384 tokens of the million-token
sequence (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
CHUNK = 16


def prefill_alg_bytes(B, T, H, d, es=2, with_s0=False):
    """q, k, v, z, o (es bytes each) + beta (fp32) per token-head, S_T (and S0)."""
    per_tok = (4 * d + d) * es + 4
    return B * T * H * per_tok + B * H * d * d * 4 * (2 if with_s0 else 1)


def prefill_alg_flops(B, T, H, d):
    """Chunk-form flops (triangular-aware), summed over chunks of 16 (last short)."""
    total = 0
    n_full, rem = divmod(T, CHUNK)
    for C, n in ((CHUNK, n_full), (rem, 1 if rem else 0)):
        per = (6 * C * d * d + C * (C - 1) * d + C * (C + 1) * d + C * (C - 1) * 2 * d
               + C * (C + 1) * d + d * d)
        total += per * n
    return total * B * H


def verify_alg_bytes(B, H, d, T, es=2):
    """S read + S_out written (fp32) once, and per token q, k, v, z, o in the
    input dtype and beta fp32."""
    return B * H * (2 * d * d * 4 + T * (5 * d * es + 4))


def backward_alg_bytes(B, T, H, d, es=2):
    """Per token-head: q, k, v, z, dO read and dq, dk, dv, dz written (es
    bytes each), beta read and dbeta written (fp32); per (b, h): dS_T read and
    dS0 written (fp32)."""
    return B * T * H * (9 * d * es + 8) + B * H * d * d * 4 * 2


def decode_alg_bytes(B, H, d, es=2):
    """S read + write (fp32) + q, k, v, z, o (es) + beta per (b, h)."""
    return B * H * (2 * d * d * 4 + 5 * d * es + 4)


def measured_traffic(key):
    """HBM bytes per launch (or pass) recorded under profiles/traffic.json
    (calibrated FETCH_SIZE + WRITE_SIZE), or None if the record is missing or
    the kernel sources it was taken on have changed since."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["records"][key]
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, s), "rb").read()
                                    for s in rec["sources"])).hexdigest()[:16]
        return rec["bytes"] if h == rec["sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def measured_record(key):
    """A figure recorded under profiles/traffic.json (e.g. an MFMA-busy
    fraction from counters), or None if it is missing or the kernel sources
    it was taken on have changed since."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["records"][key]
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, s), "rb").read()
                                    for s in rec["sources"])).hexdigest()[:16]
        return rec["value"] if h == rec["sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_prefill(kda, torch, workload, stream, dev, steps, warmup, segments=1, rotate=False,
                 flush=False, g_min=None):
    """Times `steps` prefill passes of one workload (after `warmup` untimed
    ones) with HIP events on `stream`; g_min overrides the workload's.
    Returns (result dict, inputs)."""
    from linear_attention_recurrence_05_amd.inputs import PREFILL_CONFIGS, config_inputs
    cfg_index = WORKLOADS[workload]
    cfg = PREFILL_CONFIGS[cfg_index]
    B, T, H, d = cfg.B, cfg.T, cfg.H, cfg.dk
    x = config_inputs(cfg_index, dev)
    if g_min is not None:
        x["g_min"] = g_min
    o = torch.empty(B, T, H, d, dtype=cfg.dtype, device=dev)
    ST = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
    if segments > 1:
        nb = kda.kda_chunk_prefill_segmented_workspace_bytes(B, T, H, d, d, segments, cfg.dtype)
    else:
        nb = kda.kda_chunk_prefill_workspace_bytes(B, T, H, d, d, cfg.dtype)
    # segments the plain prefill entry point chooses by itself (1: direct plan)
    auto_seg = 1 if segments > 1 else kda.kda_chunk_prefill_segments(B, T, H, d, d, cfg.dtype)
    n_seg = segments if segments > 1 else auto_seg
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    # Cold inputs.  A workload much larger than the 256 MB last-level cache
    # streams from HBM by itself; a small one cycles through copies of its
    # inputs so that a step's inputs were last touched more than 1 GiB of
    # other traffic ago.
    in_bytes = sum(t.numel() * t.element_size() for t in x.values() if torch.is_tensor(t))
    n_rot = min(8, 1 + -(-(1 << 30) // in_bytes)) if rotate else 1
    xs = [x] + [{kk: (vv.clone() if torch.is_tensor(vv) else vv) for kk, vv in x.items()}
                for _ in range(n_rot - 1)]

    def step(i):
        xi = xs[i % n_rot]
        if segments > 1:
            kda.kda_chunk_prefill_segmented(xi["q"], xi["k"], xi["v"], xi["z"], xi["beta"],
                                            xi["A"], xi["g_min"], xi["S0"], o, ST, segments,
                                            ws, stream)
        else:
            kda.kda_chunk_prefill(xi["q"], xi["k"], xi["v"], xi["z"], xi["beta"], xi["A"],
                                  xi["g_min"], xi["S0"], o, ST, ws, stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        step(warmup + i)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    ms = sum(times_ms) / len(times_ms)
    res = {"ms_per_step": ms, "ms_per_step_median": times_ms[len(times_ms) // 2],
           "wall_s_timed_region": wall}
    if rotate:
        res["cold_inputs"] = (f"steps cycle through {n_rot} copies of the inputs "
                              f"({in_bytes / 2**20:.0f} MiB each)")
    else:
        res["cold_inputs"] = (f"inputs of {in_bytes / 2**30:.1f} GiB, far beyond the 256 MB "
                              "last-level cache: every step streams them from HBM")
    if flush:
        # the same steps, each after a 1 GiB write flush, and back to back
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        fl_ms = []
        for i in range(steps):
            buf.zero_()
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            f0.record(stream)
            step(0)
            f1.record(stream)
            torch.cuda.synchronize()
            fl_ms.append(f0.elapsed_time(f1))
        del buf
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for _ in range(steps):
            step(0)
        w1.record(stream)
        torch.cuda.synchronize()
        res["ms_per_step_after_write_flush"] = sum(fl_ms) / len(fl_ms)
        res["ms_per_step_warm"] = w0.elapsed_time(w1) / steps

    direct = kda.kda_chunk_prefill_plan(B, T, H, d, d, cfg.dtype)
    plan = (f"segment scan over {segments} segments" if segments > 1
            else f"segment scan over {auto_seg} segments (chosen by kda_chunk_prefill)"
            if auto_seg > 1 else direct)
    alg_b = prefill_alg_bytes(B, T, H, d, with_s0=x["S0"] is not None)
    alg_f = prefill_alg_flops(B, T, H, d)
    gbs = alg_b / (ms * 1e-3) / 1e9
    tflops = alg_f / (ms * 1e-3) / 1e12
    key = f"prefill_{workload}_pass" if g_min is None else f"prefill_{workload}_gmin{g_min:g}_pass"
    kernel = ("segment-scan prefill pass (seg_fill_kernel, the state-only fused_kernel map pass, "
              "the zero-start fused_kernel pass, segscan_kernel, the fused_kernel redo)" if n_seg > 1
              else "prefill pass (ring_flags_init + pair_ring_kernel)" if direct == "ring"
              else "prefill pass (pair_intra_kernel + pair_roles_kernel)" if direct == "split"
              else "prefill pass (fused_kernel)")
    kind = ("segscan" if n_seg > 1 else "ring" if direct == "ring" else "split" if direct == "split"
            else "fused")
    tkey = f"{key}_bytes_{kind}"
    res.update({
        "value": B * T / (ms * 1e-3), "unit": "tokens/s",
        "config": {"workload": f"{cfg.name}_prefill_B{B}_H{H}_T{T}_d{d}_bf16", "B": B, "T": T,
                   "H": H, "d_k": d, "d_v": d, "chunk": CHUNK, "g_min": x["g_min"],
                   "S0": "zeros" if x["S0"] is None else "N(0, 0.01)",
                   "parallelism": "single GPU", "plan": plan, "workspace_bytes": nb},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(tkey),
                     "traffic_unit": "bytes per pass", "kernel": kernel,
                     "alg_bytes_per_step": alg_b,
                     "mfma_tflops": tflops, "mfma_frac": tflops / BF16_PEAK_TFLOPS,
                     "alg_flops_per_step": alg_f,
                     "mfma_busy": measured_record(f"{key}_mfma_busy")},
    })
    del o, ST, ws, xs
    return res, x


WORKLOADS = {"mid": 1, "batched": 2, "long": 3}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="time only the headline workload (no mid/batched sub-objects)")
    ap.add_argument("--verify-tokens", type=int, default=4,
                    help="drafted tokens per sequence in the verify-step measurement (1..16)")
    ap.add_argument("--workload", choices=list(WORKLOADS), default="long",
                    help="headline prefill workload: long = B1 H32 T1048576 (one million-token "
                         "sequence, the default), mid = B1 H32 T4096, batched = B8 H32 T32768 "
                         "with a carried state")
    ap.add_argument("--segments", type=int, default=1,
                    help="prefill by a scan over this many segments of each sequence "
                         "(kda_chunk_prefill_segmented); 1 = the plan kda_chunk_prefill chooses")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--plan", default=None,
                    help="force the prefill plan (sets KDA_PREFILL_PLAN: split | fused:<ncol>)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 1 GiB device-to-device copies (the reference kernel that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.plan:
        os.environ["KDA_PREFILL_PLAN"] = args.plan
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA units (b, h) are independent and shard "
              "without communication, so run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_recurrence_05_amd as kda
    from linear_attention_recurrence_05_amd.inputs import (DECODE_CONFIG, PREFILL_CONFIGS,
                                                            decode_state, decode_step_inputs,
                                                            prefill_inputs)

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "copies": 3}), flush=True)
        return
    kda.lib()
    stream = torch.cuda.current_stream()
    small = args.workload != "long"
    head, x = time_prefill(kda, torch, args.workload, stream, dev, args.steps, args.warmup,
                           segments=args.segments, rotate=small, flush=small)
    cfg = PREFILL_CONFIGS[WORKLOADS[args.workload]]
    B, T, H, d = cfg.B, cfg.T, cfg.H, cfg.dk
    tokens = B * T
    ms = head["ms_per_step"]
    line = {
        "metric": "KDA prefill tokens/s (decode steps/s in 'decode'); % of MFMA/HBM roofline",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1); v,z N(0,1); beta=sigmoid(N(0,1)); A~U(-1,1))",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    for kk in ("ms_per_step_median", "ms_per_step_warm", "ms_per_step_after_write_flush",
               "cold_inputs", "wall_s_timed_region"):
        if kk in head:
            line[kk] = head[kk]
    cpu_x = None
    if args.workload == "long" and not args.no_cpu_baseline:
        # the oracle's sample: the first 16,384 tokens of the same sequence
        P = 16384
        cpu_x = {kk: (vv[:, :P].cpu() if kk in ("q", "k", "v", "z", "beta") else
                      vv.cpu() if hasattr(vv, "cpu") else vv) for kk, vv in x.items()}
    del x
    torch.cuda.empty_cache()

    if not args.no_sub and args.workload == "long" and args.segments == 1:
        # the same sequence with slow decay (g_min = -0.05): no segment's map
        # vanishes, so the segment scan runs its map pass in full and redoes
        # every segment from its scanned start state
        r, xw = time_prefill(kda, torch, "long", stream, dev, 3, 1, g_min=-0.05)
        del xw
        torch.cuda.empty_cache()
        r["metric"] = "KDA prefill tokens/s, slow decay (g_min = -0.05)"
        line["long_slow_decay"] = r

    if not args.no_sub:
        for wl in ("mid", "batched"):
            if wl == args.workload:
                continue
            r, xw = time_prefill(kda, torch, wl, stream, dev, max(5, min(args.steps, 20)),
                                 args.warmup, rotate=True)
            del xw
            torch.cuda.empty_cache()
            r["metric"] = "KDA prefill tokens/s"
            line[wl] = r

    if not args.no_decode:
        c = DECODE_CONFIG
        gen, A, S = decode_state(c.B, c.H, c.dk, c.dv, seed=c.seed, s0_std=c.s0_std, device=dev)
        n = args.decode_steps
        stg = decode_step_inputs(gen, c.B, c.H, c.dk, c.dv, c.dtype, dev, steps=n)
        od = torch.empty(c.B, c.H, c.dv, dtype=c.dtype, device=dev)
        S_save = S.clone()

        def run_decode():
            for i in range(n):
                kda.kda_decode_step(stg["q"][i], stg["k"][i], stg["v"][i], stg["z"][i],
                                    stg["beta"][i], A, -5.0, S, od, stream)

        run_decode()   # warm-up pass
        reps = []
        for _ in range(3):
            S.copy_(S_save)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_decode()
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1))
        dms = sorted(reps)[1] / n
        db = decode_alg_bytes(c.B, c.H, c.dk)
        dgbs = db / (dms * 1e-3) / 1e9
        # practical ceiling: a device copy of the same 512 MiB state (read
        # once, written once), the same byte count as a decode step's state
        cps = []
        for _ in range(5):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            S_save.copy_(S)
            e1.record(stream)
            torch.cuda.synchronize()
            cps.append(e0.elapsed_time(e1))
        copy_gbs = 2 * S.numel() * 4 / (sorted(cps)[2] * 1e-3) / 1e9
        line["decode"] = {
            "metric": "KDA decode steps/s", "value": 1e3 / dms, "unit": "steps/s",
            "ms_per_step": dms, "steps": n, "repetitions": 3,
            "config": {"workload": "decode_B256_H32_d128_bf16_state_fp32", "B": c.B, "H": c.H,
                       "d_k": c.dk, "d_v": c.dv},
            "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dgbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_B256_H32_d128_bf16_step_bytes"),
                         "traffic_unit": "bytes per step",
                         "kernel": "decode_kernel", "alg_bytes_per_step": db,
                         "copy_ceiling_gbs": copy_gbs, "frac_of_copy": dgbs / copy_gbs},
        }
        del stg, S, S_save

        # the same decode with the states in a pool of 2 B slots, addressed by
        # a shuffled slot table (the serving layout)
        n_slots = 2 * c.B
        gen, A, _ = decode_state(1, c.H, c.dk, c.dv, seed=c.seed, s0_std=c.s0_std, device=dev)
        pool = torch.randn(n_slots, c.H, c.dk, c.dv, device=dev) * float(c.s0_std)
        slots = torch.randperm(n_slots, device=dev)[:c.B].to(torch.int32)
        n_p = min(200, n)
        stg = decode_step_inputs(gen, c.B, c.H, c.dk, c.dv, c.dtype, dev, steps=n_p)

        def run_paged():
            for i in range(n_p):
                kda.kda_decode_step_paged(stg["q"][i], stg["k"][i], stg["v"][i], stg["z"][i],
                                          stg["beta"][i], A, -5.0, pool, slots, od, stream)

        run_paged()
        reps = []
        for _ in range(3):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_paged()
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1))
        pms = sorted(reps)[1] / n_p
        pgbs = db / (pms * 1e-3) / 1e9
        line["decode_paged"] = {
            "metric": "KDA decode steps/s, states in a slot-addressed pool", "value": 1e3 / pms,
            "unit": "steps/s", "ms_per_step": pms, "steps": n_p, "repetitions": 3,
            "config": {"workload": f"decode_paged_B{c.B}_H{c.H}_d{c.dk}_bf16_pool{n_slots}",
                       "B": c.B, "H": c.H, "d_k": c.dk, "d_v": c.dv, "n_slots": n_slots},
            "roofline": {"bound": "hbm", "achieved": pgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": pgbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_B256_H32_d128_bf16_step_bytes"),
                         "traffic_unit": "bytes per step (the same kernel as dense decode)",
                         "kernel": "decode_kernel (paged)", "alg_bytes_per_step": db},
        }
        del stg, pool

        # multi-token verify step: T drafted tokens per sequence from the live
        # state, the state after them to a separate buffer (the snapshot stays)
        T_v = args.verify_tokens
        gen, A, S = decode_state(c.B, c.H, c.dk, c.dv, seed=c.seed, s0_std=c.s0_std, device=dev)
        xv = prefill_inputs(c.B, T_v, c.H, c.dk, c.dv, c.dtype, seed=c.seed + 1, device=dev)
        ov = torch.empty(c.B, T_v, c.H, c.dv, dtype=c.dtype, device=dev)
        S_out = torch.empty_like(S)

        def run_verify(src, dst):
            kda.kda_decode_tokens(xv["q"], xv["k"], xv["v"], xv["z"], xv["beta"], A, -5.0, src,
                                  dst, ov, stream)

        # V_STEPS steps back to back, as decode steps run: each step reads the
        # state the previous one wrote (the two buffers alternate), so every
        # step streams 512 MiB in and 512 MiB out
        V_STEPS = 20
        run_verify(S, S_out)
        reps = []
        for _ in range(5):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(V_STEPS):
                run_verify(S, S_out) if i % 2 == 0 else run_verify(S_out, S)
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / V_STEPS)
        vms = sorted(reps)[2]
        vb = verify_alg_bytes(c.B, c.H, c.dk, T_v)
        vgbs = vb / (vms * 1e-3) / 1e9
        line["verify"] = {
            "metric": "KDA multi-token verify steps/s (T drafted tokens per sequence per step)",
            "value": 1e3 / vms, "unit": "steps/s", "ms_per_step": vms, "tokens_per_step": T_v,
            "steps": V_STEPS, "repetitions": 5,
            "config": {"workload": f"verify_B{c.B}_H{c.H}_T{T_v}_d{c.dk}_bf16_state_fp32",
                       "B": c.B, "H": c.H, "T": T_v, "d_k": c.dk, "d_v": c.dv},
            "roofline": {"bound": "hbm", "achieved": vgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": vgbs / HBM_PEAK_GBS,
                         "traffic": (measured_traffic(f"verify_B{c.B}_H{c.H}_T{T_v}_d{c.dk}_bf16_step_bytes")
                                     if T_v == 4 else None),
                         "traffic_unit": "bytes per step",
                         "kernel": "tokens_kernel", "alg_bytes_per_step": vb},
        }
        del S, S_out, xv

    if not args.no_backward:
        # gradients of the mid workload's prefill (dO ~ N(0, 1), dS_T ~ N(0, 1))
        from linear_attention_recurrence_05_amd.inputs import backward_grads, config_inputs
        cm = PREFILL_CONFIGS[1]
        Bm, Tm, Hm, dm = cm.B, cm.T, cm.H, cm.dk
        xm = config_inputs(1, dev)
        gr = backward_grads(Bm, Tm, Hm, dm, dm, cm.dtype, seed=1, device=dev)
        gq = [torch.empty_like(xm[n]) for n in ("q", "k", "v", "z")]
        gb = torch.empty(Bm, Tm, Hm, dtype=torch.float32, device=dev)
        gA = torch.empty(Hm, dtype=torch.float32, device=dev)
        gS0 = torch.empty(Bm, Hm, dm, dm, dtype=torch.float32, device=dev)
        nbw = kda.kda_chunk_backward_workspace_bytes(Bm, Tm, Hm, dm, dm, cm.dtype)
        wsb = torch.empty(nbw, dtype=torch.uint8, device=dev)

        def run_bwd():
            kda.kda_chunk_backward(xm["q"], xm["k"], xm["v"], xm["z"], xm["beta"], xm["A"],
                                   xm["g_min"], xm["S0"], gr["dO"], gr["dST"], *gq, gb, gA, gS0,
                                   wsb, stream)

        run_bwd()
        reps = []
        for _ in range(args.backward_steps):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_bwd()
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1))
        bms = sorted(reps)[len(reps) // 2]
        bb = backward_alg_bytes(Bm, Tm, Hm, dm)
        bgbs = bb / (bms * 1e-3) / 1e9
        line["backward"] = {
            "metric": "KDA prefill-backward tokens/s",
            "value": Bm * Tm / (bms * 1e-3), "unit": "tokens/s", "ms_per_step": bms,
            "repetitions": args.backward_steps,
            "config": {"workload": f"backward_B{Bm}_H{Hm}_T{Tm}_d{dm}_bf16", "B": Bm, "T": Tm,
                       "H": Hm, "d_k": dm, "d_v": dm, "workspace_bytes": nbw},
            "roofline": {"bound": "hbm", "achieved": bgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bgbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("backward_mid_pass_bytes"),
                         "traffic_unit": "bytes per pass",
                         "kernel": "backward pass (all its launches)",
                         "alg_bytes_per_step": bb,
                         "mfma_busy": measured_record("backward_mid_pass_mfma_busy")},
        }
        del wsb, gq, gS0, xm, gr

    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        if cpu_x is not None:
            xc, what = cpu_x, (f"the first {cpu_x['q'].shape[1]:,} tokens of the same "
                               f"{T:,}-token sequence, all {H} heads")
        else:
            from linear_attention_recurrence_05_amd.inputs import config_inputs
            xc = {kk: (vv.cpu() if hasattr(vv, "cpu") else vv)
                  for kk, vv in config_inputs(WORKLOADS[args.workload], "cpu").items()}
            what = f"the whole workload (B={B}, T={T}, H={H}, d={d})"
        n_tok = xc["q"].shape[0] * xc["q"].shape[1]
        reps, t0 = 0, time.perf_counter()
        while True:   # repeated until about 10 s of CPU work
            oracle.prefill(xc["q"], xc["k"], xc["v"], xc["z"], xc["beta"], xc["A"], xc["g_min"],
                           xc["S0"], nthreads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or reps >= 200:
                break
        units = xc["q"].shape[0] * xc["q"].shape[2]
        line["cpu_baseline"] = {
            "value": reps * n_tok / dt, "unit": "tokens/s", "cores": min(threads, units),
            "kind": "oracle",
            "sample": f"{what}, {reps} times: fp64 token-by-token recurrence, OpenMP over the "
                      f"{units} heads, {threads} threads available",
            "cpu_model": cpu_model(),
            "seconds": dt,
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
