"""Bench of the MALA hot path on one MI355X.

One step = forward + backward of the 128K training shape (B=1, H=4 of a
32-head layer, L=131072, d=128, bf16, 128x64 tiles) followed by split-KV
decode of the 128K decode shape (B=16, 32 query / 8 KV heads, Lk=131073,
split 4096, 64-key tiles), all at the same tau (default 1).  Inputs are the
seeded planted-structure synthetic inputs, resident in HBM before timing.

Printed: one JSON line.  `value` is dense-equivalent TFLOP/s of the whole
step (FlashAttention causal convention: fwd 2*B*H*L^2*d, bwd 2.5x fwd,
decode 4*B*Hq*Lk*d) at tau; the same library at tau=0 (full attention) is
timed beside it.  `roofline` covers the kernel that takes most of the step;
`cpu_baseline` times the fp64 CPU oracle on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dev_bf16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def legal_tiles(L, bq, bk):
    nqb = -(-L // bq)
    return sum((min(b * bq + bq, L) - 1) // bk + 1 for b in range(nqb))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tau", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tau0", action="store_true", help="skip the tau=0 comparison run")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 32K tau sweep")
    ap.add_argument("--no-matched-work", action="store_true", help="skip the 8K matched-work measurement")
    ap.add_argument("--fidelity", action="store_true",
                    help="only run the tau=1 fidelity sweep from 1K to 32K (slots per query, omitted mass, "
                         "rel-L2 of O against exact attention, per-row errors of O/dQ/dK/dV against tau=0) and "
                         "print it as one JSON line")
    ap.add_argument("--matched-work", action="store_true",
                    help="only run the 8K matched-work study (MALA vs the reference-mass and position-only "
                         "policies at the same tile count) and print it as one JSON line")
    ap.add_argument("--cpu-sample-blocks", type=int, default=0,
                    help="query blocks in the CPU-oracle sample (0: three per OpenMP thread, at most 48)")
    ap.add_argument("--micro", action="store_true",
                    help="only run the ceiling microbenchmarks (MFMA, LDS, transposed LDS, HBM)")
    ap.add_argument("--profile-op", choices=("fwd", "bwd", "decode"),
                    help="only run one operation on --workload, --iters times after one warmup call, and print "
                         "its mean time per kernel (a short program for rocprofv3 counter passes)")
    ap.add_argument("--workload", default="sweep32k", help="workload of --profile-op (see synth.configs)")
    ap.add_argument("--iters", type=int, default=2, help="timed calls of --profile-op")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter calibration)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="no GPU: NAME WORKLOAD TAU DIR... -- per-kernel means of the rocprofv3 --pmc csv dirs "
                         "(one pass each, made with --profile-op on WORKLOAD at TAU) into profiles/NAME.md")
    ap.add_argument("--summarize-profiles", nargs=5, metavar=("TRACE", "FETCH", "WRITE", "CFETCH", "CWRITE"),
                    help="no GPU: turn rocprofv3 csv output dirs (kernel trace of this bench; FETCH_SIZE and "
                         "WRITE_SIZE passes of a short bench run; the same two passes of --copy-calibration) "
                         "into profiles/*.md and profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.micro:
        print(json.dumps(micro(torch)))
        return

    if args.profile_op:
        from mass_gated_sparse_amd import ops
        print(json.dumps(profile_op(torch, ops, args.profile_op, args.workload, args.tau, args.iters)))
        return
    if args.fidelity:
        from mass_gated_sparse_amd import ops
        print(json.dumps({fam: fidelity_sweep(torch, ops, fam) for fam in ("planted", "diffuse")}))
        return
    if args.matched_work:
        from mass_gated_sparse_amd import ops
        print(json.dumps(matched_work_8k(torch, ops, args.steps)))
        return

    if args.copy_calibration:
        n = 1 << 28  # 256 Mi bf16 elements = 512 MiB read + 512 MiB written
        a = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "launches": 3}))
        return

    from mass_gated_sparse_amd import ops
    from synth import WORKLOADS, decode_inputs, prefill_inputs
    from synth import sharpness

    wx, wd = WORKLOADS["train128k"], WORKLOADS["decode128k"]
    t0 = time.time()
    xp = prefill_inputs(wx)
    q, k, v, do = (dev_bf16(torch, xp[n]) for n in ("q", "k", "v", "do"))
    log(f"prefill inputs {q.shape} ready in {time.time() - t0:.1f}s")
    t0 = time.time()
    xd = decode_inputs(wd, threads=16)
    qd, kc, vc = (dev_bf16(torch, xd[n]) for n in ("q", "k", "v"))
    xd0 = {"q": xd["q"][:1].copy(), "k": xd["k"][:1, :2].copy(), "v": xd["v"][:1, :2].copy()}
    del xd
    log(f"decode inputs {tuple(kc.shape)} ready in {time.time() - t0:.1f}s")

    B, H, L, d = q.shape
    Bd, Hq, Lk = wd.B, wd.H, wd.L
    split = wd.split_keys
    tile = (wx.bq, wx.bk)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_b = ops.bwd_workspace(q, tile)
    od = torch.empty_like(qd)
    lsed = torch.empty(Bd, Hq, dtype=torch.float32, device="cuda")
    ws_d = ops.decode_workspace(Bd, Hq, wd.Hkv, Lk, d, split, qd.device)

    # ---- kept-tile statistics (untimed; stats-enabled launches)
    def stats_pass(tau):
        st = ops.prefill_stats_buffers(B, H, L, tile, q.device, dkdv=False)
        ops.fwd_into(q, k, v, o, lse, tau, tile, stats=st)
        fk = int(st["kept"].sum())
        stb = ops.prefill_stats_buffers(B, H, L, tile, q.device, dkdv=False)
        ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws_b, tile, stats=stb)
        bk_ = int(stb["kept"].sum())
        std = ops.decode_stats_buffers(Bd, wd.Hkv, Lk, split, wd.bk, qd.device)
        ops.decode_into(qd, kc, vc, Lk, od, lsed, tau, ws_d, split, wd.bk, stats=std)
        dkp, dlg = int(std["kept"].sum()), int(std["legal"].sum())
        torch.cuda.synchronize()
        # per (sequence, head): its sharpness multiplier c_h and kept fractions
        per_head = [{"b": b_, "h": h_, "c_h": sharpness(wx, b_, h_),
                     "fwd": int(st["kept"][b_, h_].sum()) / legal_tiles(L, *tile),
                     "bwd": int(stb["kept"][b_, h_].sum()) / legal_tiles(L, *tile)}
                    for b_ in range(B) for h_ in range(H)]
        return fk, bk_, dkp, dlg, per_head

    n_legal = B * H * legal_tiles(L, *tile)

    # ---- timed steps: each kernel is bracketed by events that the library
    # records on the stream it launches on (mala_stats.events)
    def run(tau, steps, warmup):
        for _ in range(warmup):
            ops.fwd_into(q, k, v, o, lse, tau, tile)
            ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws_b, tile)
            ops.decode_into(qd, kc, vc, Lk, od, lsed, tau, ws_d, split, wd.bk)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(steps)]
        t_start = time.perf_counter()
        for e in evs:
            ops.fwd_into(q, k, v, o, lse, tau, tile, stats={"events": e[0:2]})
            ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws_b, tile, stats={"events": e[2:6]})
            ops.decode_into(qd, kc, vc, Lk, od, lsed, tau, ws_d, split, wd.bk, stats={"events": e[6:8]})
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t_start) * 1e3 / steps

        def avg(a, b):  # per-kernel time: median over the timed steps
            return float(np.median([e[a].elapsed_time(e[b]) for e in evs]))
        ms = {"fwd": avg(0, 1), "bwd": avg(2, 5), "bwd_prep": avg(2, 3), "dq": avg(3, 4), "dkdv": avg(4, 5),
              "dec": avg(6, 7)}
        return wall, ms

    dense_fwd = 2.0 * B * H * L * L * d
    dense_bwd = 2.5 * dense_fwd
    dense_dec = 4.0 * Bd * Hq * Lk * d
    dense_step = dense_fwd + dense_bwd + dense_dec

    fk, bk_, dkp, dlg, per_head = stats_pass(args.tau)
    log(f"tau={args.tau}: fwd kept {fk}/{n_legal}, bwd kept {bk_}/{n_legal}, decode kept {dkp}/{dlg}")
    wall, ms = run(args.tau, args.steps, args.warmup)
    log(f"tau={args.tau}: step {wall:.2f} ms  fwd {ms['fwd']:.2f}  bwd {ms['bwd']:.2f} (dK/dV {ms['dkdv']:.2f}, "
        f"dQ {ms['dq']:.2f})  decode {ms['dec']:.3f}")
    out_tau0 = None
    if not args.no_tau0 and args.tau != 0.0:
        wall0, ms0 = run(0.0, args.steps, args.warmup)
        log(f"tau=0: step {wall0:.2f} ms  fwd {ms0['fwd']:.2f}  bwd {ms0['bwd']:.2f} (dK/dV {ms0['dkdv']:.2f}, "
            f"dQ {ms0['dq']:.2f})  decode {ms0['dec']:.3f}")
        out_tau0 = {"ms_per_step": wall0, "fwd_ms": ms0["fwd"], "bwd_ms": ms0["bwd"], "decode_ms": ms0["dec"],
                    "dkdv_ms": ms0["dkdv"], "dq_ms": ms0["dq"],
                    "speedup_fwd": ms0["fwd"] / ms["fwd"], "speedup_bwd": ms0["bwd"] / ms["bwd"],
                    "speedup_decode": ms0["dec"] / ms["dec"], "speedup_step": wall0 / wall}

    # ---- QK rate and vote overhead (forward and backward on the same inputs):
    # at tau=+inf only the forced tiles keep, so the forward is QK + vote on
    # every legal tile; tau=1e-30 votes on every tile but keeps all of them.
    tile_flop = 2.0 * tile[0] * tile[1] * d
    extra = None
    if not args.no_tau0:
        ms_inf = kernel_times(torch, ops, q, k, v, o, lse, do, dq, dk, dv, ws_b, tile, float("inf"), args.steps)
        st = ops.prefill_stats_buffers(B, H, L, tile, q.device, dkdv=False)
        ops.fwd_into(q, k, v, o, lse, float("inf"), tile, stats=st)
        torch.cuda.synchronize()
        fk_inf = int(st["kept"].sum())
        qk_flop = tile_flop * (n_legal + fk_inf)
        ms_vote = kernel_times(torch, ops, q, k, v, o, lse, do, dq, dk, dv, ws_b, tile, 1e-30, args.steps)
        extra = {
            "qk_rate": {"tau": "inf", "fwd_ms": ms_inf["fwd"], "kept_tiles": fk_inf, "legal_tiles": n_legal,
                        "executed_tflop": qk_flop / 1e12,
                        "tflops": qk_flop / (ms_inf["fwd"] * 1e-3) / 1e12,
                        "frac_of_peak": qk_flop / (ms_inf["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "note": "QK on every legal tile + vote; PV only on the forced tiles"},
            "vote_overhead": {"tau": 1e-30, "fwd_ms": ms_vote["fwd"], "dq_ms": ms_vote["dq"],
                              "dkdv_ms": ms_vote["dkdv"],
                              "fwd_vs_tau0": ms_vote["fwd"] / out_tau0["fwd_ms"] if out_tau0 else None,
                              "dq_vs_tau0": ms_vote["dq"] / out_tau0["dq_ms"] if out_tau0 else None,
                              "dkdv_vs_tau0": ms_vote["dkdv"] / out_tau0["dkdv_ms"] if out_tau0 else None,
                              "note": "every tile voted on and kept; ratio to the tau=0 kernels (ungated dQ and dK/dV; the tau=0 forward without statistics runs the gated kernel, whose thresholds are then -inf)"},
        }
        log(f"tau=inf fwd {ms_inf['fwd']:.2f} ms (QK rate {extra['qk_rate']['tflops']:.0f} TFLOP/s); "
            f"tau=1e-30 fwd {ms_vote['fwd']:.2f} dQ {ms_vote['dq']:.2f} dK/dV {ms_vote['dkdv']:.2f}")

    # ---- rooflines: algorithmic work per launch / live average launch duration
    per_tile = f"2*{tile[0]}*{tile[1]}*{d} FLOP per tile product"
    traffic = load_traffic()
    kern = {
        "fwd_bf16_d128": (ms["fwd"], tile_flop * (n_legal + fk), "mfma",
                          f"QK on every legal tile + PV on each kept tile; {per_tile}"),
        "bwd_dkdv_pair_bf16_d128": (ms["dkdv"], tile_flop * 4 * bk_, "mfma",
                                    f"S, dP, dV, dK on each kept tile (the dQ pass decides; this pass visits "
                                    f"kept tiles only); {per_tile}"),
        "bwd_dq_bf16_d128": (ms["dq"], tile_flop * (n_legal + 2 * bk_), "mfma",
                             f"S on every legal tile + dP, dQ on each kept tile; {per_tile}"),
        "decode_split_bf16_d128": (ms["dec"], Bd * wd.Hkv * Lk * d * 2 * (1.0 + dkp / dlg), "hbm",
                                   "256 B of K per cached key always + 256 B of V per key of a kept tile"),
    }
    rooflines = {}
    for name, (t_ms, work, bound, per_unit) in kern.items():
        if bound == "mfma":
            ach, peak, unit = work / (t_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = work / (t_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
        rooflines[name] = {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
                           "traffic": traffic.get(name), "kernel": name, "ms": t_ms,
                           "work_per_launch": work, "per_unit": per_unit}
    roofline = rooflines[max(rooflines, key=lambda n: rooflines[n]["ms"])]

    dec_var = None if args.no_tau0 else decode_variants_128k(torch, ops, qd, kc, vc, od, lsed, ws_d, wd, args.tau,
                                                                args.steps)
    chunk = None if args.no_tau0 else chunked_prefill(torch, ops, q, k, v, args.tau, args.steps)
    sweep = None if args.no_sweep else sweep32k(torch, ops, args.steps, args.warmup)
    gqa = None if args.no_sweep else gqa_8k(torch, ops, args.tau, args.steps)
    matched = None if args.no_matched_work else matched_work_8k(torch, ops, args.steps)

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        nb = args.cpu_sample_blocks or 3 * min(16, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
        cpu = cpu_baseline(wx, wd, xp, xd0, nb, args.tau)
        log(f"cpu baseline took {time.time() - t0:.1f}s")

    res = {
        "metric": "fwd/bwd/decode ms + dense-equiv TFLOP/s at 128K, tau=1 vs tau=0; % tiles kept",
        "value": dense_step / (wall * 1e-3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent, fwd+bwd+decode step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded planted sink+local+retrieval inputs)",
        "config": {"workload": "train128k fwd+bwd (B1 H4 L131072 d128, 128x64 tiles) + decode128k "
                               "(B16 Hq32 Hkv8 Lk131073 d128, split 4096, 64-key tiles)",
                   "tau": args.tau, "global_batch": B, "seq_len": L, "parallelism": "none (one GPU's 4-head share)"},
        "fwd_ms": ms["fwd"], "bwd_ms": ms["bwd"], "decode_ms": ms["dec"],
        "bwd_kernels_ms": {"prep": ms["bwd_prep"], "dkdv": ms["dkdv"], "dq": ms["dq"]},
        "fwd_dense_tflops": dense_fwd / (ms["fwd"] * 1e-3) / 1e12,
        "bwd_dense_tflops": dense_bwd / (ms["bwd"] * 1e-3) / 1e12,
        "decode_dense_tflops": dense_dec / (ms["dec"] * 1e-3) / 1e12,
        "kept_frac": {"fwd": fk / n_legal, "bwd": bk_ / n_legal, "decode": dkp / dlg},
        "kept_frac_per_head": per_head,
        "tau0": out_tau0,
        "qk_rate": extra["qk_rate"] if extra else None,
        "vote_overhead": extra["vote_overhead"] if extra else None,
        "roofline": roofline,
        "kernel_rooflines": rooflines,
        "sweep32k": sweep,
        "matched_work_8k": matched,
        "decode_variants": dec_var,
        "chunked_prefill": chunk,
        "gqa8k": gqa,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


def kernel_times(torch, ops, q, k, v, o, lse, do, dq, dk, dv, ws, tile, tau, steps):
    """Mean per-kernel ms of forward and backward at tau (events recorded by the
    library around each kernel), after one untimed warmup."""
    ops.fwd_into(q, k, v, o, lse, tau, tile)
    ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws, tile)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for e in evs:
        ops.fwd_into(q, k, v, o, lse, tau, tile, stats={"events": e[0:2]})
        ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws, tile, stats={"events": e[2:6]})
    torch.cuda.synchronize()

    def avg(a, b):  # median over the calls
        return float(np.median([e[a].elapsed_time(e[b]) for e in evs]))
    return {"fwd": avg(0, 1), "dq": avg(3, 4), "dkdv": avg(4, 5)}


# kernel -> (instantiation timed by the bench at tau > 0, source files it is built from)
PROFILED = {
    "fwd_bf16_d128": ("fwd_bf16_d128<true, false>", ["mala_fwd.hip"]),
    "bwd_dkdv_pair_bf16_d128": ("bwd_dkdv_pair_bf16_d128<true>", ["mala_bwd.hip"]),
    "bwd_dq_bf16_d128": ("bwd_dq_bf16_d128<true, false>", ["mala_bwd.hip"]),
    "decode_split_bf16_d128": ("decode_split_bf16_d128<true, false, false, false>", ["mala_decode.hip"]),
}
COMMON_SOURCES = ["mala_device.hpp", "mala_kernels.hpp"]
CSRC = "mass_gated_sparse_amd/csrc"


def sources_sha1(files):
    import hashlib
    h = hashlib.sha1()
    for f in files + COMMON_SOURCES:
        with open(os.path.join(ROOT, CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def _counter_per_dispatch(d, counter):
    """{kernel name: [value per dispatch]} from a rocprofv3 --pmc csv dir (values summed over
    the counter's instances within a dispatch)."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (_, name), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def summarize_counters(name, workload, tau, *dirs):
    """profiles/<name>.md: per kernel, the mean per dispatch of every SQ
    counter found in the --pmc csv dirs, plus derived fractions:
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES),
    LDS active = SQ_LDS_IDX_ACTIVE / SQ_BUSY_CU_CYCLES, wave time waiting =
    SQ_WAIT_ANY / SQ_WAVE_CYCLES, LDS-instruction waits = SQ_WAIT_INST_LDS /
    SQ_WAVE_CYCLES."""
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    passes = []
    for d in dirs:
        names, per = {}, collections.defaultdict(float)
        counters = set()
        for r in _csv_rows(d, "counter_collection.csv"):
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per[key] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"].split("(")[0].replace("void ", "")
            counters.add(r["Counter_Name"])
        passes.append(sorted(counters))
        for (disp, cn), v in per.items():
            vals[names[disp]][cn].append(v)
    from synth import WORKLOADS
    op = "decode" if WORKLOADS[workload].kind == "decode" else "<fwd|bwd>"
    lines = [f"# Hardware counters per dispatch: {workload}, tau={tau}", "",
             "Commands (from the repository root, on one MI355X; one rocprofv3 pass per counter set):", ""]
    for cs in dict.fromkeys(tuple(c) for c in passes):
        lines.append(f"    cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {' '.join(cs)} --output-format csv "
                     f"-d <dir> -o run -- python3 <repo>/bench.py --profile-op {op} "
                     f"--workload {workload} --tau {tau} --iters 1")
    lines += ["", "Derived: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES); LDS active = "
              "SQ_LDS_IDX_ACTIVE / SQ_BUSY_CU_CYCLES; waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES; LDS waits = "
              "SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES.", ""]
    for kern, cs in vals.items():
        if not kern.startswith("mala::"):
            continue
        m = {cn: float(np.mean(v)) for cn, v in cs.items()}
        lines += [f"## `{kern}`", "", "| counter | mean per dispatch |", "|---|---:|"]
        lines += [f"| {cn} | {v:.4g} |" for cn, v in sorted(m.items())]
        der = []
        if m.get("SQ_BUSY_CU_CYCLES"):
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                der.append(f"MFMA busy {100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * m['SQ_BUSY_CU_CYCLES']):.0f}%")
            if "SQ_LDS_IDX_ACTIVE" in m:
                der.append(f"LDS active {100 * m['SQ_LDS_IDX_ACTIVE'] / m['SQ_BUSY_CU_CYCLES']:.0f}%")
        if m.get("SQ_WAVE_CYCLES"):
            if "SQ_WAIT_ANY" in m:
                der.append(f"waiting {100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.0f}%")
            if "SQ_WAIT_INST_LDS" in m:
                der.append(f"LDS waits {100 * m['SQ_WAIT_INST_LDS'] / m['SQ_WAVE_CYCLES']:.0f}%")
        if "SQ_LDS_BANK_CONFLICT" in m:
            der.append(f"LDS bank conflicts {m['SQ_LDS_BANK_CONFLICT']:.0f}")
        lines += ["", "Derived: " + "; ".join(der) + ".", ""]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_profiles(trace_dir, fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    # kernel-time summary of the bench command
    rows = _csv_rows(trace_dir, "kernel_stats.csv")
    lines = ["# Kernel time: bench.py, 128K training step + 128K decode", "",
             "Command (from the repository root, on one MI355X):", "",
             "    cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats "
             "--output-format csv -d <dir> -o run -- python3 <repo>/bench.py --steps 3 --warmup 1 "
             "--no-tau0 --no-sweep --no-matched-work --no-cpu-baseline", "",
             "Runs at tau=1 only: every launch of an instantiation below is a tau=1 launch (the "
             "statistics pass uses the separate `<..., true>` instantiations; warmup and timed steps "
             "are included).", "",
             "| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---:|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    with open(os.path.join(prof, "kernel_trace_train128k_decode128k.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    # HBM traffic: counters scaled by what they read for a copy of known size
    cal = {}
    for cdir, counter in ((cfetch_dir, "FETCH_SIZE"), (cwrite_dir, "WRITE_SIZE")):
        vals = _counter_per_dispatch(cdir, counter)
        big = max((v for vs in vals.values() for v in vs))
        cal[counter] = (1 << 29) / (big * 1024.0)  # 512 MiB read and written per copy launch
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    rec = {"unit": "bytes per launch", "calibration": {
        "copy_bytes": 1 << 29, "fetch_factor": cal["FETCH_SIZE"], "write_factor": cal["WRITE_SIZE"],
        "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o run -- "
                   "python3 bench.py --copy-calibration"},
        "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o run -- python3 "
                   "bench.py --steps 1 --warmup 0 --no-tau0 --no-sweep --no-matched-work --no-cpu-baseline",
        "kernels": {}}
    md = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated)", "",
          f"Commands: `{rec['command']}`; calibration: `{rec['calibration']['command']}` "
          "(torch copy of 512 MiB bf16).", "",
          f"Calibration factors (bytes per counter KiB / 1024): fetch {cal['FETCH_SIZE']:.4f}, "
          f"write {cal['WRITE_SIZE']:.4f}.", "",
          "| kernel | dispatches | FETCH KiB | WRITE KiB | scaled GB per launch |", "|---|---:|---:|---:|---:|"]
    for kname, (inst, srcs) in PROFILED.items():
        fv = [v for n, vs in fetch.items() if inst in n for v in vs]
        wv = [v for n, vs in write.items() if inst in n for v in vs]
        if not fv or not wv:
            continue
        fk, wk = float(np.mean(fv)), float(np.mean(wv))
        b = fk * 1024 * cal["FETCH_SIZE"] + wk * 1024 * cal["WRITE_SIZE"]
        rec["kernels"][kname] = {"instantiation": inst, "dispatches": len(fv), "fetch_kib": fk, "write_kib": wk,
                                 "bytes_per_launch": b, "sources": [f"{CSRC}/{x}" for x in srcs + COMMON_SOURCES],
                                 "sources_sha1": sources_sha1(srcs)}
        md.append(f"| `{inst}` | {len(fv)} | {fk:.0f} | {wk:.0f} | {b / 1e9:.3f} |")
    with open(os.path.join(prof, "hbm_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    with open(os.path.join(prof, "hbm_traffic_train128k_decode128k.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(rec["kernels"], indent=1))


def load_traffic():
    """Measured HBM bytes per launch of each kernel from profiles/hbm_traffic.json.
    An entry is used only while the sha1 of the kernel's sources still equals
    the one recorded with the counters: once a kernel has changed, its traffic
    is unknown (None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    out = {}
    for name, r in rec.get("kernels", {}).items():
        if name in PROFILED and sources_sha1(PROFILED[name][1]) == r["sources_sha1"]:
            out[name] = r["bytes_per_launch"]
    return out


def micro(torch):
    """Measured ceilings on this GPU: dense bf16 MFMA (32x32x16, 8 independent
    chains per wave), LDS read bandwidth (16-byte reads, conflict-free) and the
    transposing 8-byte LDS reads, the hardware exp2 rate (8 independent chains
    per thread), HBM streaming reads (8 GiB)."""
    import ctypes
    from mass_gated_sparse_amd.build import ubench_path
    lib = ctypes.CDLL(ubench_path())
    vp = ctypes.c_void_p
    dev = torch.cuda.get_device_properties(0)
    cus = dev.multi_processor_count
    st = vp(torch.cuda.current_stream().cuda_stream)
    out = torch.empty(1 << 22, dtype=torch.int32, device="cuda")
    seed = torch.randint(0, 1 << 16, (256,), dtype=torch.int32, device="cuda")

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    res = {"cus": cus}
    blocks = cus * 8
    it = 2000
    t = timed(lambda: lib.ubench_mfma(vp(seed.data_ptr()), vp(out.data_ptr()), blocks, it, st))
    res["mfma_bf16_tflops"] = blocks * 4 * it * 8 * 32768 / t / 1e12
    it = 4000
    t = timed(lambda: lib.ubench_lds(vp(out.data_ptr()), cus * 2, it, st))
    res["lds_read_bytes_per_clk_per_cu_at_2p4ghz"] = cus * 2 * 4 * it * 8 * 1024 / t / cus / 2.4e9
    res["lds_read_tbs"] = cus * 2 * 4 * it * 8 * 1024 / t / 1e12
    t = timed(lambda: lib.ubench_lds_tr(vp(out.data_ptr()), cus * 2, it, st))
    res["lds_tr_read_bytes_per_clk_per_cu_at_2p4ghz"] = cus * 2 * 4 * it * 4 * 1024 / t / cus / 2.4e9
    it = 4000
    t = timed(lambda: lib.ubench_exp(vp(seed.data_ptr()), vp(out.data_ptr()), cus * 8, it, st))
    res["exp2_per_clk_per_cu_at_2p4ghz"] = cus * 8 * 256 * it * 8 / t / cus / 2.4e9
    res["exp2_gops"] = cus * 8 * 256 * it * 8 / t / 1e9
    n16 = (8 << 30) // 16
    buf = torch.empty(n16 * 4, dtype=torch.int32, device="cuda").fill_(1)
    t = timed(lambda: lib.ubench_hbm(vp(buf.data_ptr()), ctypes.c_long(n16), vp(out.data_ptr()), cus * 16, st))
    res["hbm_read_gbs_one_load_per_thread"] = n16 * 16 / t / 1e9
    # several independent loads in flight per thread; the best of a small sweep
    # of loads per thread and workgroups per CU is the streaming ceiling
    sweep = {}
    for unroll in (4, 8):
        for per_cu in (4, 8, 16):
            blocks = cus * per_cu
            if n16 % (unroll * blocks * 256) or blocks * 256 > out.numel():
                continue
            t = timed(lambda: lib.ubench_hbm_unroll(vp(buf.data_ptr()), ctypes.c_long(n16), vp(out.data_ptr()),
                                                    blocks, unroll, st))
            sweep[f"unroll{unroll}_wg{per_cu}_per_cu"] = n16 * 16 / t / 1e9
    res["hbm_read_sweep_gbs"] = sweep
    res["hbm_read_gbs"] = max([res["hbm_read_gbs_one_load_per_thread"], *sweep.values()])
    return res


# timed repetitions and warm-up calls of the 32K sweep configurations (at
# least; --steps / --warmup raise them): the first few calls of a
# configuration in a process can read several percent slow
SMALL_REPS = 10
SMALL_WARMUP = 10


def sweep32k(torch, ops, steps, warmup):
    """32K tau sweep (B1 H8 L32768 d128 bf16): fwd/bwd ms, dense-equivalent
    TFLOP/s and kept-tile fractions at tau in {0, 0.5, 1, 2}, for the planted
    family (c_h ~ U[0.5, 2]), the planted family with c = 1 on every head,
    and the diffuse family."""
    from synth import WORKLOADS, prefill_inputs
    w = WORKLOADS["sweep32k"]
    tile = (w.bq, w.bk)
    out = {}
    for family in ("planted", "planted_c1", "diffuse"):
        x = prefill_inputs(w, family=family)
        q, k, v, do = (dev_bf16(torch, x[n]) for n in ("q", "k", "v", "do"))
        del x
        B, H, L, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = ops.bwd_workspace(q, tile)
        n_legal = B * H * legal_tiles(L, *tile)
        dense_fwd = 2.0 * B * H * L * L * d
        res = {}
        for tau in w.taus:  # decisions and kept fractions
            st = ops.prefill_stats_buffers(B, H, L, tile, q.device)
            ops.fwd_into(q, k, v, o, lse, tau, tile, stats=st)
            stb = ops.prefill_stats_buffers(B, H, L, tile, q.device)
            ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws, tile, stats=stb)
            torch.cuda.synchronize()
            res[str(tau)] = {"kept_fwd": int(st["kept"].sum()) / n_legal, "kept_bwd": int(stb["kept"].sum()) / n_legal}
        # timing interleaved over tau (every repetition visits every tau), so
        # drift during the sweep lands on all of them alike
        for _ in range(max(SMALL_WARMUP, warmup)):
            for tau in w.taus:
                ops.fwd_into(q, k, v, o, lse, tau, tile)
                ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws, tile)
        times = {tau: ([], []) for tau in w.taus}
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for _ in range(max(SMALL_REPS, steps)):
            for tau in w.taus:
                ev[0].record()
                ops.fwd_into(q, k, v, o, lse, tau, tile)
                ev[1].record()
                ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws, tile)
                ev[2].record()
                torch.cuda.synchronize()
                times[tau][0].append(ev[0].elapsed_time(ev[1]))
                times[tau][1].append(ev[1].elapsed_time(ev[2]))
        for tau in w.taus:
            tf, tb = float(np.median(times[tau][0])), float(np.median(times[tau][1]))  # medians over the repetitions
            res[str(tau)].update({"fwd_ms": tf, "bwd_ms": tb, "fwd_dense_tflops": dense_fwd / tf / 1e9,
                                  "bwd_dense_tflops": 2.5 * dense_fwd / tb / 1e9})
        for tau in w.taus:
            if tau != 0.0:
                r = res[str(tau)]
                r["speedup_fwd_vs_tau0"] = res["0.0"]["fwd_ms"] / r["fwd_ms"]
                r["speedup_bwd_vs_tau0"] = res["0.0"]["bwd_ms"] / r["bwd_ms"]
        out[family] = res
        log(f"sweep32k {family}: " + ", ".join(f"tau={t}: fwd {r['fwd_ms']:.2f} bwd {r['bwd_ms']:.2f} "
                                              f"kept {r['kept_fwd']:.3f}/{r['kept_bwd']:.3f}" for t, r in res.items()))
        del q, k, v, do, o, dq, dk, dv
    return out


def profile_op(torch, ops, op, workload, tau, iters):
    """One operation of the path on a named workload: one warmup call, then
    `iters` calls with the library's events around each kernel; mean ms per
    kernel."""
    from synth import WORKLOADS, decode_inputs, prefill_inputs
    w = WORKLOADS[workload]
    if (op == "decode") != (w.kind == "decode"):
        raise SystemExit(f"--profile-op {op} needs a {'decode' if op == 'decode' else 'prefill'} workload")
    if w.kind == "prefill":
        x = prefill_inputs(w)
        q, k, v, do = (dev_bf16(torch, x[n]) for n in ("q", "k", "v", "do"))
        tile = (w.bq, w.bk)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        ops.fwd_into(q, k, v, o, lse, tau, tile)
        if op == "fwd":
            names = ("fwd",)

            def call(e):
                ops.fwd_into(q, k, v, o, lse, tau, tile, stats={"events": e})
        else:
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = ops.bwd_workspace(q, tile)
            names = ("bwd_prep", "dq", "dkdv")

            def call(e):
                ops.bwd_into(q, k, v, o, lse, do, dq, dk, dv, tau, ws, tile, stats={"events": e})
    else:
        x = decode_inputs(w, threads=16)
        q, kc, vc = (dev_bf16(torch, x[n]) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        ws = ops.decode_workspace(w.B, w.H, w.Hkv, w.L, w.d, w.split_keys, q.device)
        names = ("decode",)

        def call(e):
            ops.decode_into(q, kc, vc, w.L, o, lse, tau, ws, w.split_keys, w.bk, stats={"events": e})
    n = len(names) + 1
    call([torch.cuda.Event(enable_timing=True) for _ in range(n)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(iters)]
    for e in evs:
        call(e)
    torch.cuda.synchronize()
    return {"op": op, "workload": workload, "tau": tau, "iters": iters,
            "ms": {nm: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, nm in enumerate(names)}}


def decode_variants_128k(torch, ops, qd, kc, vc, od, lsed, ws, wd, tau, steps, warmup=3):
    """Every decode variant on the decode128k shape, timed back to back in
    this function after warm-up calls of each: plain and seeded partitions
    (mala_decode, mala_decode_seeded), each with the whole KV group voting
    (rows_per_vote = G) and with one vote per query head (rows_per_vote = 1)
    at tau, and both at tau = 0.  Per variant: ms per call (the library's
    events around its launches), the fraction of (vote group, tile) pairs
    kept, the fraction of tiles whose V is read (a tile is read when a vote
    group of its KV head keeps it) and the algorithmic HBM rate (K always, V
    of the read tiles)."""
    Lk, split, bk, G = wd.L, wd.split_keys, wd.bk, wd.group
    out = {"workload": "decode128k (B16 Hq32 Hkv8 Lk131073 d128, split 4096); seeded partitions are counted "
                       "back from the newest tile",
           "note": "timed back to back, 3 warm-up calls per variant; the step's own decode runs between the "
                   "backward and the next forward"}

    def one(seeded, rpv, t):
        vg = G // rpv
        kw = dict(seeded=seeded, rows_per_vote=rpv)
        st = ops.decode_stats_buffers(wd.B, wd.Hkv, Lk, split, bk, qd.device, vote_groups=vg)
        ops.decode_into(qd, kc, vc, Lk, od, lsed, t, ws, split, bk, stats=st, **kw)
        torch.cuda.synchronize()
        kept, legal = int(st["kept"].sum()), int(st["legal"].sum())
        bits = st["keep_bits"].cpu().numpy().astype(np.uint32)  # [B, Hkv * vg, nsplit, words]
        union = np.bitwise_or.reduce(bits.reshape(wd.B, wd.Hkv, vg, *bits.shape[2:]), axis=2)
        v_frac = int(sum(bin(int(x)).count("1") for x in union.ravel())) / (legal // vg)
        for _ in range(warmup):
            ops.decode_into(qd, kc, vc, Lk, od, lsed, t, ws, split, bk, **kw)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in evs:
            ops.decode_into(qd, kc, vc, Lk, od, lsed, t, ws, split, bk, stats={"events": e}, **kw)
        torch.cuda.synchronize()
        ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
        nbytes = wd.B * wd.Hkv * Lk * wd.d * 2 * (1.0 + v_frac)
        return {"ms": ms, "kept_frac_vote_tiles": kept / legal, "v_read_frac": v_frac,
                "algorithmic_GBps": nbytes / (ms * 1e-3) / 1e9}

    for seeded in (False, True):
        name = "seeded" if seeded else "plain"
        for rpv in (G, 1):
            out[f"{name}, tau={tau}, rows_per_vote={rpv}"] = one(seeded, rpv, tau)
        out[f"{name}, tau=0.0"] = one(seeded, G, 0.0)
    grp = f"rows_per_vote={G}"
    out["seeded_vs_plain"] = out[f"plain, tau={tau}, {grp}"]["ms"] / out[f"seeded, tau={tau}, {grp}"]["ms"]
    out["seeded_vs_tau0"] = out["plain, tau=0.0"]["ms"] / out[f"seeded, tau={tau}, {grp}"]["ms"]
    out["plain_vs_tau0"] = out["plain, tau=0.0"]["ms"] / out[f"plain, tau={tau}, {grp}"]["ms"]
    log("decode variants: " + json.dumps(out))
    return out


def chunked_prefill(torch, ops, q, k, v, tau, steps, Lq=16384):
    """Chunked prefill on the 128K training shape: the last Lq query rows
    (key offset P = L - Lq) against the K/V cache holding all L keys, at tau
    and at tau=0.  Dense-equivalent FLOPs: 4*d per visible (row, key) pair."""
    B, H, L, d = q.shape
    P = L - Lq
    qc = q[:, :, P:].contiguous()
    tile = (128, 64)
    out = {"workload": f"train128k shape, last {Lq} rows at key offset {P} against the {L}-key cache"}
    pairs = B * H * (Lq * P + Lq * (Lq + 1) / 2)
    for t in (tau, 0.0):
        o, lse, st = ops.fwd_chunk(qc, k, v, P, t, stats=True)
        torch.cuda.synchronize()
        kept, legal = int(st["kept"].sum()), int(st["legal"].sum())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ops.fwd_chunk_into(qc, k, v, P, o, lse, t, tile)
        e0.record()
        for _ in range(steps):
            ops.fwd_chunk_into(qc, k, v, P, o, lse, t, tile)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[f"tau={t}"] = {"ms": ms, "kept_frac": kept / legal, "dense_equiv_tflops": 4.0 * d * pairs / ms / 1e9}
    log(f"chunked prefill: " + json.dumps(out))
    return out


def gqa_8k(torch, ops, tau, steps):
    """Grouped K/V heads: B1, 8 query heads over 2 K/V heads, L=8192, d=128,
    planted inputs; forward and backward ms at tau and at tau=0."""
    from synth import WORKLOADS, prefill_inputs
    w = WORKLOADS["gqa8k"]
    x = prefill_inputs(w)
    q, k, v, do = (dev_bf16(torch, x[n]) for n in ("q", "k", "v", "do"))
    del x
    tile = (w.bq, w.bk)
    o, lse = ops.fwd(q, k, v, tau)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = ops.bwd_workspace(q, tile)
    out = {"workload": "gqa8k (B1 H8 Hkv2 L8192 d128 bf16, 128x64 tiles, planted)"}
    for t in (tau, 0.0):
        ms = kernel_times(torch, ops, q, k, v, o, lse, do, dq, dk, dv, ws, tile, t, max(SMALL_REPS, steps))
        st = ops.prefill_stats_buffers(*q.shape[:3], tile, q.device)
        ops.fwd_into(q, k, v, o, lse, t, tile, stats=st)
        torch.cuda.synchronize()
        out[f"tau={t}"] = dict(ms, kept_frac_fwd=int(st["kept"].sum()) / int(st["legal"].sum()))
    log("gqa8k: " + json.dumps(out))
    return out


def exact_row_stats(qh, kh, vh, keep, blocks, bq, bk, scale, o_gpu=None):
    """Against exact causal softmax attention (fp64, numpy; a measurement, not
    the oracle): for every row of the given query blocks of one head, the
    probability mass of its visible keys in tiles the forward skipped, and the
    number of its visible keys in kept tiles (post-score slots).  With o_gpu
    (the GPU output rows of those blocks) also sum |O - O*|^2 and |O*|^2.
    qh, kh, vh: [L, d] fp64; keep: [nqb, ntiles] forward decisions."""
    L = kh.shape[0]
    omitted, slots, err2, ref2 = [], [], 0.0, 0.0
    cols = np.arange(L)
    for qb in blocks:
        rows = np.arange(qb * bq, min(qb * bq + bq, L))
        s = (qh[rows] @ kh.T) * scale
        vis = cols[None, :] <= rows[:, None]
        s = np.where(vis, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        kt = keep[qb][cols // bk][None, :] & vis
        omitted.append((p * (vis & ~kt)).sum(axis=1))
        slots.append(kt.sum(axis=1))
        if o_gpu is not None:
            ref = p @ vh
            err2 += float(((o_gpu[rows - qb * bq + blocks.index(qb) * bq] - ref) ** 2).sum())
            ref2 += float((ref ** 2).sum())
    return np.concatenate(omitted), np.concatenate(slots), err2, ref2


def _jmax(qb, bq, bk, L):
    return (min(qb * bq + bq, L) - 1) // bk


def position_window(blocks, bq, bk, L, heads, target_tiles):
    """Window w (in key tiles) of the position-only policy -- the sink tile 0
    plus the w tiles ending at the block's diagonal -- whose tile count over
    the sampled blocks of all heads is closest to target_tiles."""
    def count(w):
        return heads * sum(min(_jmax(b, bq, bk, L) + 1, w + 1) for b in blocks)
    return min(range(1, _jmax(blocks[-1], bq, bk, L) + 2), key=lambda w: (abs(count(w) - target_tiles), w)), count


def policy_fidelity(qh, kh, vh, keep_h, blocks, bq, bk, scale, window, o_gpu=None):
    """One head of the matched-work study, against exact causal softmax
    attention (fp64, numpy; a measurement, not the oracle).

    Policies, each a set of (query block, key tile) pairs over the sampled
    blocks: "mala" (the forward's decisions), "reference_mass" (the tiles of
    largest exact probability mass, as many as MALA kept on this head: the
    per-instance optimum of mean omitted mass at that tile budget) and
    "position_only" (tile 0 plus the `window` tiles ending at the diagonal).
    Per row: omitted mass (exact mass of visible keys outside the policy),
    slots (visible keys inside it) and the relative L2 error of the policy's
    output, softmax renormalized over its keys, against exact attention;
    with o_gpu (GPU rows of the sampled blocks, in order) also the GPU
    output's per-row relative error."""
    L = kh.shape[0]
    cols = np.arange(L)
    probs, vis_l, mass = [], [], []
    for qb in blocks:
        rows = np.arange(qb * bq, min(qb * bq + bq, L))
        s = (qh[rows] @ kh.T) * scale
        vis = cols[None, :] <= rows[:, None]
        s = np.where(vis, s, -np.inf)
        pr = np.exp(s - s.max(axis=1, keepdims=True))
        pr /= pr.sum(axis=1, keepdims=True)
        probs.append(pr)
        vis_l.append(vis)
        nt = _jmax(qb, bq, bk, L) + 1
        mass.append(np.array([pr[:, t * bk:(t + 1) * bk].sum() for t in range(nt)]))
    # tile sets
    sets = {"mala": [keep_h[qb][: _jmax(qb, bq, bk, L) + 1].astype(bool) for qb in blocks]}
    budget = int(sum(m.sum() for m in sets["mala"]))
    cand = sorted(((-m[t], i, t) for i, m in enumerate(mass) for t in range(len(m))))
    ref = [np.zeros(len(m), bool) for m in mass]
    for _, i, t in cand[:budget]:
        ref[i][t] = True
    sets["reference_mass"] = ref
    pos = []
    for qb in blocks:
        jm = _jmax(qb, bq, bk, L)
        m = np.zeros(jm + 1, bool)
        m[0] = True
        m[max(0, jm - window + 1):] = True
        pos.append(m)
    sets["position_only"] = pos
    out = {}
    for name, tiles in sets.items():
        om, sl, rel = [], [], []
        for i, qb in enumerate(blocks):
            kt = np.zeros(L, bool)
            kt[: len(tiles[i]) * bk] = np.repeat(tiles[i], bk)[:L]
            sel = vis_l[i] & kt[None, :]
            pm = probs[i] * sel
            om.append(1.0 - pm.sum(axis=1))
            sl.append(sel.sum(axis=1))
            exact = probs[i] @ vh
            z = pm.sum(axis=1, keepdims=True)
            o_pol = np.where(z > 0, (pm @ vh) / np.where(z > 0, z, 1.0), 0.0)
            rel.append(np.linalg.norm(o_pol - exact, axis=1) / np.linalg.norm(exact, axis=1))
        out[name] = {"tiles": int(sum(t.sum() for t in tiles)), "omitted": np.concatenate(om),
                     "slots": np.concatenate(sl), "rel": np.concatenate(rel)}
    if o_gpu is not None:
        rel = []
        for i, qb in enumerate(blocks):
            exact = probs[i] @ vh
            n = exact.shape[0]
            rel.append(np.linalg.norm(o_gpu[i * bq: i * bq + n] - exact, axis=1) / np.linalg.norm(exact, axis=1))
        out["mala"]["rel_gpu"] = np.concatenate(rel)
    return out


def matched_work_8k(torch, ops, steps):
    """The 8K matched-work shape (B1 H16 L8192 d128, bf16, 128x64 tiles, tau=1,
    planted inputs with per-head sharpness c_h ~ U[0.5, 2]): GPU fwd/bwd ms and
    kept-tile fractions, and -- on every 8th query block of every head -- the
    matched-work comparison of MALA's forward decisions with the per-instance
    reference-mass policy and the position-only policy at the same number of
    tiles (mean omitted probability mass, post-score slots per query and mean
    per-row relative output error against exact attention)."""
    from synth import WORKLOADS, prefill_inputs, to_f64
    w = WORKLOADS["mw8k"]
    tile, tau = (w.bq, w.bk), 1.0
    x = prefill_inputs(w)
    q, k, v, do = (dev_bf16(torch, x[n]) for n in ("q", "k", "v", "do"))
    B, H, L, d = q.shape
    o, lse, st = ops.fwd(q, k, v, tau, tile=tile, stats=True)
    dq, dk, dv, stb = ops.bwd(q, k, v, o, lse, do, tau, tile=tile, stats=True)
    torch.cuda.synchronize()
    n_legal = B * H * legal_tiles(L, *tile)
    ws = ops.bwd_workspace(q, tile)
    ms = kernel_times(torch, ops, q, k, v, o, lse, do, dq, dk, dv, ws, tile, tau, max(SMALL_REPS, steps))
    nt = -(-L // w.bk)
    keep = ops.bits_to_keep(st["keep_bits"], nt)[0]
    og = o.float().cpu().numpy()[0]
    blocks = list(range(0, -(-L // w.bq), 8))
    scale = 1.0 / np.sqrt(d)
    mala_tiles = int(sum(keep[h][b][: _jmax(b, w.bq, w.bk, L) + 1].sum() for h in range(H) for b in blocks))
    window, count = position_window(blocks, w.bq, w.bk, L, H, mala_tiles)
    acc = {}
    t0 = time.time()
    rows = np.concatenate([np.arange(b * w.bq, min(b * w.bq + w.bq, L)) for b in blocks])
    for h in range(H):
        qh, kh, vh = (to_f64(x[n][0, h], "bf16") for n in ("q", "k", "v"))
        r = policy_fidelity(qh, kh, vh, keep[h], blocks, w.bq, w.bk, scale, window, og[h][rows])
        for name, dct in r.items():
            a = acc.setdefault(name, {})
            for key, val in dct.items():
                a[key] = a.get(key, 0) + val if key == "tiles" else np.concatenate([a.get(key, np.zeros(0)), val])
    log(f"matched-work 8K: exact-attention sample took {time.time() - t0:.1f}s")
    policies = {}
    for name, a in acc.items():
        policies[name] = {"tiles": int(a["tiles"]), "mean_omitted_mass_pct": 100.0 * float(a["omitted"].mean()),
                          "max_omitted_mass_pct": 100.0 * float(a["omitted"].max()),
                          "slots_per_query": float(a["slots"].mean()),
                          "mean_rel_l2_O_pct": 100.0 * float(a["rel"].mean())}
    policies["mala"]["mean_rel_l2_O_gpu_pct"] = 100.0 * float(acc["mala"]["rel_gpu"].mean())
    policies["position_only"]["window_tiles"] = window
    log("matched-work 8K policies: " + json.dumps(policies))
    return {"workload": "mw8k (B1 H16 L8192 d128 bf16, 128x64 tiles, planted, c_h~U[0.5,2])", "tau": tau,
            "fwd_ms": ms["fwd"], "dq_ms": ms["dq"], "dkdv_ms": ms["dkdv"],
            "kept_frac_fwd": int(st["kept"].sum()) / n_legal, "kept_frac_bwd": int(stb["kept"].sum()) / n_legal,
            "mean_omitted_mass_pct": policies["mala"]["mean_omitted_mass_pct"],
            "max_omitted_mass_pct": policies["mala"]["max_omitted_mass_pct"],
            "omitted_mass_bound_pct": 100.0 * tau / (1.0 + tau),
            "slots_per_query": policies["mala"]["slots_per_query"],
            "policies": policies,
            "sample": f"every 8th query block ({len(blocks)} of {-(-L // w.bq)}) of all {H} heads",
            "note": "omitted mass = exact softmax mass of a row's visible keys outside the policy's tiles; "
                    "slots = the row's visible keys inside them; a policy's output renormalizes the softmax over "
                    "its keys (fp64), mala's GPU output also includes bf16 rounding; reference_mass = top exact-mass "
                    "tiles of each head at MALA's tile count there; position_only = tile 0 plus a window of "
                    "window_tiles tiles ending at the diagonal, window chosen so the total tile count is closest "
                    "to MALA's"}


def mean_row_rel(torch, a, ref):
    """Mean over rows (last axis = features) of |a - ref| / |ref|, rows with
    ref = 0 left out; computed in fp32 on the device."""
    a, ref = a.float(), ref.float()
    n, r = (a - ref).norm(dim=-1), ref.norm(dim=-1)
    m = r > 0
    return float((n[m] / r[m]).mean())


def mean_head_rel(torch, a, ref):
    """Mean over (batch, head) of the whole-head relative L2 error
    |a - ref|_F / |ref|_F, in fp32 on the device."""
    a, ref = a.float().flatten(2), ref.float().flatten(2)
    return float(((a - ref).norm(dim=-1) / ref.norm(dim=-1)).mean())


def fidelity_sweep(torch, ops, family="planted"):
    """tau=1 from 1K to 32K on the planted family of the 32K sweep shape
    (H=8, d=128, bf16, 128x64 tiles): kept-tile fraction, post-score slots
    per query, omitted mass and rel-L2 of O against exact attention on every
    query block of L <= 4K and a sample of 16 blocks per head beyond; and,
    over every row, the mean per-row relative L2 error of O, dQ, dK and dV
    against the same kernels ungated (tau=0: full attention, the reference
    operator), both in bf16."""
    from synth import WORKLOADS, prefill_inputs, to_f64
    w = WORKLOADS["sweep32k"]
    tile, tau = (w.bq, w.bk), 1.0
    out = {}
    for L in (1024, 2048, 4096, 8192, 16384, 32768):
        x = prefill_inputs(w, L=L, family=family)
        q, k, v, do = (dev_bf16(torch, x[n]) for n in ("q", "k", "v", "do"))
        B, H, _, d = q.shape
        o, lse, st = ops.fwd(q, k, v, tau, tile=tile, stats=True)
        grads = ops.bwd(q, k, v, o, lse, do, tau, tile=tile)
        o0, lse0 = ops.fwd(q, k, v, 0.0, tile=tile)
        grads0 = ops.bwd(q, k, v, o0, lse0, do, 0.0, tile=tile)
        pairs = list(zip(("O", "dQ", "dK", "dV"), (o,) + tuple(grads), (o0,) + tuple(grads0)))
        rel_vs_full = {n: 100.0 * mean_row_rel(torch, a, b) for n, a, b in pairs}
        head_vs_full = {n: 100.0 * mean_head_rel(torch, a, b) for n, a, b in pairs}
        del grads, grads0, o0, lse0, do
        torch.cuda.synchronize()
        nqb, nt = -(-L // w.bq), -(-L // w.bk)
        keep = ops.bits_to_keep(st["keep_bits"], nt)[0]
        og = o.float().cpu().numpy()[0]
        blocks = list(range(nqb)) if nqb <= 32 else sorted(set(np.linspace(0, nqb - 1, 16).astype(int).tolist()))
        om, sl, e2, r2 = [], [], 0.0, 0.0
        for h in range(H):
            qh, kh, vh = (to_f64(x[n][0, h], "bf16") for n in ("q", "k", "v"))
            rows = np.concatenate([np.arange(b * w.bq, min(b * w.bq + w.bq, L)) for b in blocks])
            a, b_, e, r = exact_row_stats(qh, kh, vh, keep[h], blocks, w.bq, w.bk, 1.0 / np.sqrt(d), og[h][rows])
            om.append(a)
            sl.append(b_)
            e2 += e
            r2 += r
        om, sl = np.concatenate(om), np.concatenate(sl)
        out[str(L)] = {"kept_frac_fwd": int(st["kept"].sum()) / (B * H * legal_tiles(L, *tile)),
                       "slots_per_query": float(sl.mean()), "mean_omitted_mass_pct": 100.0 * float(om.mean()),
                       "rel_l2_O_vs_exact": float(np.sqrt(e2 / r2)),
                       "mean_row_rel_l2_vs_full_pct": rel_vs_full,
                       "mean_head_rel_l2_vs_full_pct": head_vs_full,
                       "sample_blocks_per_head": len(blocks)}
        log(f"fidelity {family} L={L}: " + json.dumps(out[str(L)]))
    return {"fidelity": out, "tau": tau, "workload": f"sweep32k shape (H8 d128 bf16, 128x64 tiles), {family} family",
            "note": "slots = a row's visible keys in kept tiles; omitted mass against exact softmax; "
                    "mean_row_rel_l2_vs_full_pct: per-row relative L2 of the tau=1 outputs against the tau=0 "
                    "(ungated) outputs of the same kernels, mean over all rows (key rows for dK, dV); "
                    "mean_head_rel_l2_vs_full_pct: the same comparison over each whole head, mean over heads"}


def cpu_baseline(wx, wd, xp, xd0, nblocks, tau):
    """fp64 CPU oracle on a bounded sample of the same step.

    Sample: head 0 of the 128K prefill, rows of its last `nblocks` query
    blocks (full-length rows): forward of those rows, dQ of those rows, dK/dV
    of the 2*nblocks key tiles whose contributing rows all lie in that range;
    plus decode of two (sequence, KV head) units of the decode shape.  FLOPs
    are the dense-equivalent work the oracle executes on the sample (every
    legal (row, key) pair counted as kept): 4d per pair forward, 6d per pair
    in the dQ pass (S, dP, dQ), 8d per pair in the dK/dV pass (S, dP, dK,
    dV), 4d per (row, key) in decode."""
    import oracle
    from synth import to_f64

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    L, d, bq, bk = wx.L, wx.d, wx.bq, wx.bk
    nqb = -(-L // bq)
    qbs = list(range(nqb - nblocks, nqb))
    r0 = qbs[0] * bq
    kts = list(range(r0 // bk, -(-L // bk)))
    qf, kf, vf, dof = (to_f64(xp[n][:, :1], "bf16") for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    o, lse, keep, _ = oracle.fwd(qf, kf, vf, tau, bq, bk, qblocks=qbs)
    oracle.bwd(qf, kf, vf, np.nan_to_num(o), np.nan_to_num(lse), dof, tau, bq, bk, qblocks=qbs, ktiles=kts)
    t_pre = time.perf_counter() - t0
    t1 = time.perf_counter()
    oracle.decode(to_f64(xd0["q"], "bf16"), xd0["k"], xd0["v"], wd.L, tau, wd.split_keys, wd.bk,
                  units=[(0, 0), (0, 1)])
    t_dec = time.perf_counter() - t1
    pairs_rows = sum(i + 1 for i in range(r0, L))
    pairs_keys = sum(L - j for j in range(kts[0] * bk, L))
    flops = 4.0 * d * pairs_rows + 6.0 * d * pairs_rows + 8.0 * d * pairs_keys + 2 * wd.group * 4.0 * wd.L * d
    total = t_pre + t_dec
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
    except OSError:
        pass
    return {"value": flops / total / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": threads,
            "cpu_model": cpu_model, "kind": "oracle", "seconds": round(total, 2),
            "sample": f"head 0 of train128k, last {nblocks} query blocks (rows {r0}..{L - 1}): fwd, dQ of those "
                      f"rows, dK/dV of key tiles {kts[0]}..{kts[-1]}; decode128k units (b0,g0),(b0,g1); "
                      f"tau={tau}; dense-equivalent FLOPs executed by the oracle"}


if __name__ == "__main__":
    main()
