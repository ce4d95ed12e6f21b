"""Throughput of one fwd+bwd iteration of the tile rasterizer on one MI355X.

A step is one pass of the whole hot path for one camera: gs_project -> gs_bin_and_sort ->
gs_rasterize_fwd_l1 (the blend, with the L1 gradient against the camera's target image formed as
each pixel is finished; on the workloads whose loss is 0.8 L1 + 0.2 (1 - SSIM),
gs_rasterize_fwd -> gs_loss_l1_ssim) ->
gs_rasterize_bwd (with --optimizer, then gs_adam_step). Steps cycle through the workload's cameras; all inputs (Gaussians, cameras,
target images) are resident in HBM before the timed region. The default workload is the
30,000-Gaussian distillation student at 1280x720 over 60 ring cameras, with target images
rendered once (by the forward path) from a seeded 300,000-Gaussian teacher.

Camera iterations are independent (the Gaussians are only read), so by default four run at once,
each on its own HIP stream with its own buffers: at this size every kernel of one iteration is
short and latency-bound, and the concurrent iterations fill the GPU. The same steps run again one
at a time afterwards ("single_stream" in the output). --optimizer runs one stream (every Adam step
changes what the next iteration reads).

Prints one JSON line: the iterations/s metric, Mpix/s and sorted pairs/s, per-kernel times from
HIP events recorded by the library on the stream it launches on (a second pass over the same
steps, right after the timed one), the roofline of the dominant kernel and the CPU oracle timed
on a bounded sample of the same workload.
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

# MI355X figures used for rooflines (public specs): HBM3E 8 TB/s; 256 CUs x 4 SIMD x 16 lanes at
# 2.4 GHz issue 39.3e12 non-packed fp32 VALU lane-operations per second (157.3 TFLOP/s counts
# packed FMAs as 4 flops per lane-cycle).
HBM_PEAK_GBS = 8000.0
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12

# VALU lane-operations per (pixel, splat) evaluation that the roofline counts: the blend's is
# the algorithmic count of a front-to-back step (evaluation, alpha, transmittance test and
# update, three colour sums: 27); the backward's that of a (pixel, entry) walked back
# (evaluation, T recovery, dL/dalpha and the nine gradient pieces: 60). Beside them, the loop
# bodies' counts in the gfx950 ISA of the built library (52 VALU ops per two splats in the
# blend; 126 in the backward, the wave reduction included).
VALU_PER_EVAL = {"blend": 27.0, "rbwd": 60.0}
VALU_PER_EVAL_ISA = {"blend": 26.0, "rbwd": 63.0}
# the binning kernels, and among them those that move keys (the radix passes and the emission
# fused with the first pair pass)
BIN_KERNELS = ("small_local", "small_merge", "bin_prep", "hist_reduce", "depth_sort_pass", "scan", "emit_sort",
               "pair_sort_pass")
SORT_KERNELS = ("small_local", "small_merge", "depth_sort_pass", "emit_sort", "pair_sort_pass")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="distill_30k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--streams", type=int, default=4,
                    help="camera iterations in flight at once, each on its own HIP stream with its own buffers "
                         "(1 with --optimizer, whose updates every iteration must see)")
    ap.add_argument("--backward", choices=("auto", "atomic", "deterministic"), default="auto",
                    help="gs_rasterize_bwd (fp32 atomics) or gs_rasterize_bwd_deterministic (per-pair records, "
                         "bitwise reproducible); auto: the deterministic one up to 4M pairs per camera, where "
                         "concurrent iterations run it faster (no contended global atomics), else the atomic one")
    ap.add_argument("--deterministic", action="store_true", help="same as --backward deterministic")
    ap.add_argument("--tile-lists", choices=("rect", "tight"), default="rect",
                    help="rect: every tile of a splat's rectangle; tight: only the tiles its ellipse reaches "
                         "(camera option tight_tiles: fewer pairs, the same image)")
    ap.add_argument("--optimizer", action="store_true",
                    help="a training step: each step also takes an Adam step on the raw parameters")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the timed steps, copy a buffer of this many MiB 5 times (a plain copy "
                         "kernel of known size, to scale HBM byte counters)")
    return ap.parse_args()


def kernel_bytes(name, stats):
    """Algorithmic HBM bytes of one launch of a binning kernel."""
    P, N = stats["pairs"], stats["n"]
    return {
        # small frames: depth, tile count, mean and radii in (24 B), the rectangle record and the
        # block-sorted key, id and count prefix out (28 B) per Gaussian
        "small_local": 52.0 * N,
        # the sorted keys, ids, count prefixes and rectangle records in (28 B), the depth-ordered
        # record out (16 B) per Gaussian
        "small_merge": 44.0 * N,
        "bin_prep": 48.0 * N,
        # the first depth pass sorts all N keys and drops the culled ones, the other three sort the
        # visible ones (per launch: the mean of the four passes)
        "depth_sort_pass": (16.0 * N + 3 * 16.0 * stats["visible"]) / 4.0,
        "scan": 40.0 * stats["visible"],
        # the emission fused with the first pair pass: depth-ordered records in, pairs out
        # (the final pass when it is the only one: 64-bit keys, ids and the depth gather)
        "emit_sort": 16.0 * stats["visible"] + (16.0 if stats["pair_passes"] == 0 else 8.0) * P,
        # the other pair passes: 8 B in and 8 B out per pair; the final one writes 12 B and
        # gathers 4 B of depth
        "pair_sort_pass": (16.0 * P + 8.0 * P / max(1, stats["pair_passes"])) if stats["pair_passes"] else 0.0,
        "project": stats["project_bytes"],
        "loss_l1": 12.0 * stats["pixels"] * 3,
        # two passes: 24 B in, 36 B of partials out; 36 B of partials and 24 B in, 12 B out
        "loss_ssim": (24.0 + 36.0 + 36.0 + 24.0 + 12.0) * stats["pixels"],
    }.get(name)


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current source of that kernel and on this workload; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except ValueError:
        return None
    if not rec or rec.get("workload") != workload:
        return None
    src = os.path.join(ROOT, "gaussian_splatting_tile_gs_amd", "csrc", rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["sha256"]:
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(wl, scene, cams_d, target_of, seconds):
    """The oracle on the host cores: projection of all N, dense render + backward (sparse L1 loss on
    the rendered pixels), chain rule to raw parameters. The pixel sample of camera 0 grows until it
    takes about half the time budget; once it is the whole frame, further cameras' full frames are
    added until about 0.7 of the budget is spent. A partial frame is scaled to the full frame."""
    import oracle
    from gaussian_splatting_tile_gs_amd import synth

    W, H = wl.width, wl.height

    fragile = {}

    def one(ci, npix):
        cam = cams_d[ci]
        pix = synth.sample_pixels(W, H, npix, seed=1)
        tgt = target_of(ci)
        t0 = time.perf_counter()
        proj = oracle.project(scene, cam)
        t1 = time.perf_counter()
        fwd = oracle.render(proj, cam, pixels=pix)
        dimg = np.sign(fwd["image"] - tgt[pix[:, 0], pix[:, 1]]) / (3.0 * W * H)
        g2d, _ = oracle.render_backward(proj, cam, dimg, pixels=pix)
        t3 = time.perf_counter()
        oracle.project_backward(scene, cam, g2d)
        t4 = time.perf_counter()
        fragile[ci] = (int(npix), int(np.count_nonzero(fwd["fragile"])))
        return t4 - t0, (t1 - t0) + (t4 - t3) + (t3 - t1) / npix * W * H

    # one core: a pixel sample of camera 0 grown to about a sixth of the budget
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    npix1 = 256
    while True:
        total1, frame1 = one(0, npix1)
        if total1 >= seconds / 6.0 or npix1 >= W * H:
            break
        npix1 = min(W * H, int(npix1 * max(2.0, 0.8 * seconds / 6.0 / max(total1, 1e-3))))
    oracle.set_num_threads(threads)

    npix = 1024
    while True:
        total, frame = one(0, npix)
        if total >= 0.5 * seconds or npix >= W * H:
            break
        npix = min(W * H, int(npix * max(2.0, 0.7 * seconds / max(total, 1e-3))))
    frames, measured = [frame], total
    if npix >= W * H:
        while measured < 0.7 * seconds and len(frames) < len(cams_d):
            total, frame = one(len(frames), W * H)
            frames.append(frame)
            measured += total
        sample = (f"full frames of cameras 0-{len(frames) - 1} of {wl.name}: projection of all "
                  f"{scene['means'].shape[0]} Gaussians, dense render + backward of all {W * H} pixels "
                  f"(L1 loss), chain rule (measured {measured:.1f} s)")
    else:
        sample = (f"camera 0 of {wl.name}: projection of all {scene['means'].shape[0]} Gaussians, dense "
                  f"render + backward on {npix} seeded pixels of {W * H} (sparse L1 loss), chain rule; "
                  f"per-pixel time scaled to the full frame (measured {measured:.1f} s)")
    frame_s = sum(frames) / len(frames)
    npx0, nfrag0 = fragile[0]
    return {"value": 1.0 / frame_s, "unit": "iterations/s", "cores": threads, "kind": "oracle",
            "sample": sample, "measured_seconds": round(measured, 3), "frame_seconds": round(frame_s, 3),
            "one_core": {"value": 1.0 / frame1, "unit": "iterations/s", "cores": 1,
                         "sample": f"camera 0 of {wl.name}: {npix1} seeded pixels of {W * H}, per-pixel time scaled "
                                   f"to the full frame (measured {total1:.1f} s)"},
            "fragile_pixels": {"camera": 0, "pixels": npx0, "fragile": nfrag0}}


def adam_roofline(gs, torch, params, grads, wl, launches=50):
    """The Adam kernel on copies of the parameters: 16 B read (p, g, m, v) and 12 B written
    (p, m, v) per value, against its average launch time from the library's HIP events."""
    p = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in params.items()}
    F = gs.gs_adam_state_floats(wl.n, wl.sh_degree)
    m = torch.zeros(F, device="cuda")
    v = torch.zeros(F, device="cuda")
    cfg = gs.adam_config()
    gs.gs_adam_step(wl.n, wl.sh_degree, 1, cfg, p, grads, m, v)
    torch.cuda.synchronize()
    gs.gs_timing_enable(True)
    for t in range(launches):
        gs.gs_adam_step(wl.n, wl.sh_degree, t + 2, cfg, p, grads, m, v)
    torch.cuda.synchronize()
    recs = [ms for name, ms in gs.gs_timing_collect(1 << 12) if name == "adam"]
    gs.gs_timing_enable(False)
    avg_s = sum(recs) / len(recs) / 1e3
    b = 28.0 * wl.n * (11 + 3 * (wl.sh_degree + 1) ** 2)  # the values, not the state's padding
    return {"kernel": "adam", "bound": "hbm", "bytes_per_launch": b, "avg_us": avg_s * 1e6,
            "achieved": b / avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": b / avg_s / 1e9 / HBM_PEAK_GBS}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: bench.py --gpus N with N > 1 is not supported"}))
        sys.exit(2)
    import torch

    from gaussian_splatting_tile_gs_amd import gs, synth

    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    scene = synth.make_scene(wl)
    cams_d = [dict(c, tight_tiles=args.tile_lists == "tight") for c in synth.make_cameras(wl)]
    cams = [gs.make_camera(c) for c in cams_d]
    W, H = wl.width, wl.height
    params = gs.scene_to_device(scene)

    # targets: the teacher rendered by the forward path, once, resident in HBM
    teacher = synth.make_teacher(wl)
    tparams = gs.scene_to_device(teacher)
    tpipe = gs.Pipeline(tparams, W, H, pair_capacity=1 << 20)
    targets = torch.empty(len(cams), H, W, 3, device="cuda")
    for i, cam in enumerate(cams):
        tpipe.project(cam)
        tpipe.bin(cam)
        tpipe.forward(cam, checkpoints=False)
        targets[i].copy_(tpipe.image)
    del tpipe, tparams
    torch.cuda.synchronize()
    log(f"{wl.name}: {len(cams)} target images rendered from the {teacher['means'].shape[0]}-Gaussian teacher")

    nstreams = 1 if args.optimizer else max(1, args.streams)

    def make_pipe():
        p = gs.Pipeline(params, W, H, pair_capacity=1 << 16)
        # the workload's loss: L1, or 0.8 L1 + 0.2 (1 - SSIM) (gs_loss_l1_ssim)
        p.ssim_lambda = 0.2 if wl.loss == "l1_dssim" else 0.0
        return p

    pipe = make_pipe()
    pairs = []
    for cam in cams:  # size the pair buffers for every camera
        pipe.project(cam)
        pairs.append(pipe.bin(cam))
    need = max(pairs)
    # with the optimizer the scene drifts, so leave more room
    cap = int(need * (1.5 if args.optimizer else 1.1)) + 1024
    pipe.reserve_pairs(cap)
    # concurrent camera iterations: their own buffers (pairs, images, workspaces, gradients) and
    # streams (default priority); the Gaussians are shared read-only
    backward = "deterministic" if args.deterministic else args.backward
    if backward == "auto":
        backward = "deterministic" if need <= 4_000_000 else "atomic"
    pipe.deterministic = backward == "deterministic"
    pipes = [pipe] + [make_pipe() for _ in range(nstreams - 1)]
    for p in pipes:
        p.deterministic = pipe.deterministic
    for p in pipes[1:]:
        p.reserve_pairs(cap)
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
    ncam = len(cams)
    adam_cfg = gs.adam_config()

    def step(i, k=0):
        # no host wait anywhere in a step: the pair buffers already hold every camera's pairs
        c = i % ncam
        p, st = pipes[k], streams[k]
        with torch.cuda.stream(st):
            if wl.backward:
                p.iteration(cams[c], targets[c], stream=st, wait=False)
                if args.optimizer:
                    p.adam_step(adam_cfg, stream=st)
            else:
                p.project(cams[c], stream=st)
                p.bin(cams[c], stream=st, wait=False)
                p.forward(cams[c], stream=st, checkpoints=False)  # a render: no backward follows

    issue = {}

    def timed(nsteps, first, k_streams):
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for i in range(nsteps):
            step(first + i, i % k_streams)
        issue[k_streams] = time.perf_counter() - ta  # the host's time to enqueue the steps
        torch.cuda.synchronize()
        return time.perf_counter() - ta

    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 18, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i, i % nstreams)
    elapsed = timed(args.steps, args.warmup, nstreams)
    its = args.steps / elapsed
    log(f"timed {args.steps} steps on {nstreams} stream(s): {1e3 * elapsed / args.steps:.4f} ms/step "
        f"(host enqueue {1e3 * issue[nstreams] / args.steps:.4f} ms/step)")
    if args.optimizer:
        # the scene moved: every camera's pairs must still fit the buffers the steps ran with
        P_last = int(pipe.num_pairs_dev.item())
        assert P_last <= pipe.capacity, "pair buffers overflowed"
        steps_pairs = args.steps * P_last
    else:
        for k, p in enumerate(pipes):
            ks = [i for i in range(args.steps) if i % nstreams == k]
            if ks:
                last = (args.warmup + ks[-1]) % ncam
                assert int(p.num_pairs_dev.item()) == pairs[last] <= p.capacity, "pair count changed between runs"
        steps_pairs = sum(pairs[(args.warmup + i) % ncam] for i in range(args.steps))
    # the same steps one at a time (one stream): the latency-bound rate of a single camera
    single = None
    if nstreams > 1:
        e1 = timed(args.steps, args.warmup, 1)
        single = {"value": args.steps / e1, "ms_per_step": 1e3 * e1 / args.steps,
                  "host_enqueue_ms_per_step": 1e3 * issue[1] / args.steps}
        log(f"one stream: {1e3 * e1 / args.steps:.4f} ms/step (host enqueue {1e3 * issue[1] / args.steps:.4f})")

    result = {
        "metric": "fwd+bwd iterations/sec and Mpix/s at 30k Gaussians 1280x720; sorted pairs/sec"
                  + (" (training steps: fwd+bwd+Adam)" if args.optimizer else ""),
        "value": its, "unit": "iterations/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps, "higher_is_better": True, "scaling": "weak",
        # the host's time to enqueue a step (no host wait in a step): at or near ms_per_step the
        # rate is set by the launching thread, not the GPU
        "host_enqueue_ms_per_step": 1e3 * issue[nstreams] / args.steps,
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "mpix_per_s": its * W * H / 1e6, "sorted_pairs_per_s": None,
        # pairs of the timed steps per second of the whole timed region (not of the sort alone)
        "pairs_per_s_end_to_end": steps_pairs / elapsed,
        "config": {"workload": wl.name, "gaussians": wl.n, "width": W, "height": H, "cameras": ncam,
                   "loss": "0.8 L1 + 0.2 (1 - SSIM)" if pipe.ssim_lambda > 0 else "L1 (gradient formed in the blend)",
                   "concurrent_cameras": nstreams, "backward": backward, "tile_lists": args.tile_lists,
                   "sh_degree": wl.sh_degree, "teacher_gaussians": int(teacher["means"].shape[0]),
                   "mean_pairs_per_camera": float(np.mean(pairs)), "parallelism": "single GPU"},
    }

    result["single_stream"] = single
    if not args.no_kernel_timing:
        # per-kernel HIP events (recorded by the library on the stream it launches on) over a
        # second pass of the same steps; then an untimed pass with the evaluation counters on
        nprof = min(args.steps, 4 * ncam)
        gs.gs_timing_enable(True)
        for i in range(nprof):
            step(args.warmup + i)
        torch.cuda.synchronize()
        recs = gs.gs_timing_collect(1 << 16)
        gs.gs_timing_enable(False)
        evals_f = torch.zeros(1, device="cuda", dtype=torch.int64)
        evals_b = torch.zeros(1, device="cuda", dtype=torch.int64)
        for i in range(nprof):
            c = (args.warmup + i) % ncam
            pipe.project(cams[c])
            pipe.bin(cams[c], wait=False)
            fused = wl.backward and pipe.ssim_lambda == 0.0  # the L1 gradient formed in the blend
            pipe.forward(cams[c], eval_count=evals_f, checkpoints=None if wl.backward else False,
                         l1_target=targets[c] if fused else None)
            if wl.backward:
                if not fused:
                    pipe.loss_l1(targets[c])
                pipe.backward(cams[c], eval_count=evals_b)
        torch.cuda.synchronize()
        per = {}
        for name, ms in recs:
            d = per.setdefault(name, [0.0, 0])
            d[0] += ms
            d[1] += 1
        visible = int((pipe.proj.tiles_touched > 0).sum().item())
        K = (wl.sh_degree + 1) ** 2
        stats = {"pairs": float(np.mean(pairs)), "n": wl.n, "visible": visible, "pixels": W * H,
                 "pair_passes": per.get("pair_sort_pass", [0, 0])[1] // max(1, per.get("emit_sort", [0, 1])[1]),
                 "project_bytes": wl.n * (4 * (3 + 3 + 4 + 1 + 3 * K) + 52)}
        kernels = {}
        for name, (tot, cnt) in sorted(per.items(), key=lambda kv: -kv[1][0]):
            kernels[name] = {"launches": cnt, "avg_us": 1e3 * tot / cnt, "share": tot / sum(v[0] for v in per.values())}
        result["kernels"] = kernels
        dom = max(per.items(), key=lambda kv: kv[1][0])[0]
        tot, cnt = per[dom]
        avg_s = tot / cnt / 1e3
        if dom in VALU_PER_EVAL:
            evals = (evals_f if dom == "blend" else evals_b).item() / cnt
            ops = evals * VALU_PER_EVAL[dom]
            achieved = ops / avg_s / 1e12
            isa = evals * VALU_PER_EVAL_ISA[dom] / avg_s / 1e12
            roof = {"bound": "alu", "achieved": achieved, "peak": VALU_PEAK_TOPS, "unit": "TOP/s",
                    "frac": achieved / VALU_PEAK_TOPS, "traffic": traffic_for(dom, wl.name), "kernel": dom,
                    "evals_per_launch": evals, "valu_per_eval": VALU_PER_EVAL[dom],
                    "valu_per_eval_isa": VALU_PER_EVAL_ISA[dom], "frac_isa": isa / VALU_PEAK_TOPS,
                    "avg_us": avg_s * 1e6}
        else:
            b = kernel_bytes(dom, stats) or 0.0
            achieved = b / avg_s / 1e9
            roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(dom, wl.name), "kernel": dom,
                    "bytes_per_launch": b, "avg_us": avg_s * 1e6}
        result["roofline"] = roof
        bin_s = sum(per[k][0] for k in BIN_KERNELS if k in per) / 1e3 / nprof
        bin_b = sum((kernel_bytes(k, stats) or 0.0) * per[k][1] for k in BIN_KERNELS if k in per) / nprof
        sort_s = sum(per[k][0] for k in SORT_KERNELS if k in per) / 1e3 / nprof
        # sorted pairs per second of the sort kernels' time and of the whole binning's
        result["sorted_pairs_per_s"] = stats["pairs"] / sort_s if sort_s > 0 else None
        result["sorted_pairs_per_s_bin_sort"] = stats["pairs"] / bin_s if bin_s > 0 else None
        result["sort_kernels"] = [k for k in SORT_KERNELS if k in per]
        # the same time against the bytes a stable 64-bit (tile | depth) key sort with a separate
        # count/emit/range would move (172 B per pair + 32 B per Gaussian): what a design that
        # sorts the full keys would have to stream to finish in this time
        ref_b = 172.0 * stats["pairs"] + 32.0 * wl.n
        result["bin_sort"] = {"kernel_us_per_step": bin_s * 1e6, "bytes_per_step": bin_b,
                              "gbs": bin_b / bin_s / 1e9 if bin_s > 0 else None,
                              "frac_hbm": (bin_b / bin_s / 1e9) / HBM_PEAK_GBS if bin_s > 0 else None,
                              "key_sort_bytes_per_step": ref_b,
                              "key_sort_equiv_frac_hbm": (ref_b / bin_s / 1e9) / HBM_PEAK_GBS if bin_s > 0 else None}
        result["evals_per_step"] = {"fwd": evals_f.item() / nprof, "bwd": evals_b.item() / nprof}
        result["optimizer"] = adam_roofline(gs, torch, params, pipe.grads, wl)

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a pixel sample")
        cb = cpu_baseline(wl, scene, cams_d, lambda i: targets[i].cpu().numpy().astype(np.float64),
                          args.cpu_seconds)
        # the oracle's fragile pixels (a skip/stop decision within fp32 rounding of its threshold)
        # on the sample of camera 0 it rendered
        result["fragile_pixels"] = cb.pop("fragile_pixels")
        result["cpu_baseline"] = cb
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
