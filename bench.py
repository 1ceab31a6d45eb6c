#!/usr/bin/env python3
"""Benchmark of the VBM stencil pipeline on one MI355X.

Workload: the sphere shell of radius 185 and half thickness 1.5
(1,290,538 active voxels, 11,255 leaves), interleaved fp32 sidecar with
C = 16 channels, BlockWidth 128.  One step is one launch of the fused cached
streaming 27-tap box filter: per slot decode, LDS neighbour-leaf table,
streamed taps, gather-accumulate of 16 channels.

The timed region holds exactly --steps launches back to back on the current
stream, bracketed by torch.cuda.synchronize() and HIP events, after --warmup
untimed launches; before those, about 0.1 s of untimed launches bring the GPU
from the idle clocks of the host-side set-up to steady state.  Inputs are
resident in HBM; to keep the 256 MB Infinity Cache from serving repeated
launches, successive steps rotate over several sidecar/output buffer sets
whose total size exceeds three times the cache.

Printed (stdout, one JSON line): value = active-voxel*channels per second,
the roofline object for this kernel (algorithmic bytes per launch / mean
launch time vs 8 TB/s), the CPU oracle baseline on the host (with the host's
CPU model and thread counts), the decode metric (select-based decode at
BlockWidth 128, ms), the noisy narrow band (cached streaming box, W512, C=16;
skipped with --no-band) and extra measurements (other resolvers, channel
counts, widths, the decode, the Laplacian) under "extra".  Progress goes to
stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
PROFILE = os.path.join(ROOT, "profiles", "box_cached_streaming_cfg_shell_C16_W128.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def alg_bytes_filter(n_active, n_leaves, n_blocks, width, channels):
    """Bytes a filter pass must move: own sidecar row read once, own output row
    written once, leaf records (mask 64 + prefix 8 + first 8 + origin 12 B) and
    block metadata (firstLeafID 4 B + jumpMap W/8 B)."""
    return 8 * channels * n_active + 92 * n_leaves + (4 + width // 8) * n_blocks


def alg_bytes_decode(n_active, n_leaves, n_blocks, width):
    """Decode: 6 B written per slot (u32 + u16), leaf mask/prefix/first (80 B),
    block metadata."""
    return 6 * n_blocks * width + 80 * n_leaves + (4 + width // 8) * n_blocks


def host_cpu():
    """Model string of the host CPU and the thread counts the machine reports."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"model": model, "hardware_concurrency": os.cpu_count(), "usable_cpus": usable}


def kernel_sources_sha256():
    """Hash of the kernel sources; the HBM counters in profiles/ are valid only for this hash."""
    import hashlib
    h = hashlib.sha256()
    for f in ("vbm_device.hpp", "vbm_division.hpp", "vbm_kernels.hip"):
        with open(os.path.join(ROOT, "nanovdb_stencil_filtering_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(path=PROFILE):
    """HBM bytes per launch of the headline kernel from the rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    summarised in profiles/ (already scaled by the copy calibration), or None when the summary is
    missing or was taken on other kernel sources."""
    try:
        with open(path) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines() if ": " in line)
    except OSError:
        return None
    if kv.get("sources_sha256", "").strip() != kernel_sources_sha256():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"].split()[0])
    except (KeyError, ValueError):
        return None


def headline_kernel(channels):
    """Name of the kernel vbm_box_filter launches for the cached streaming box at these channels."""
    if channels in (8, 16):
        return "k_box_cached_split<%d, true, Sidecar>" % channels
    return "k_box_cached<%d, %s, true, Sidecar>" % (channels, "true" if channels % 4 == 0 else "false")


def time_builds(coords, log2w, reps, dev):
    """Wall-clock seconds (median of reps) of the host build (vbm_build, C++ on one
    host core) and of the device-side build (plan + fill, coordinates already in
    device memory, workspace and blob allocated beforehand), and the device blob's
    equality with the host's."""
    import ctypes
    import numpy as np
    import torch
    from nanovdb_stencil_filtering_amd import vbm
    lib = vbm.load_library()
    host_t = []
    for _ in range(reps):
        t0 = time.perf_counter()
        hdr, host_blob = vbm.build_host(coords, log2w)
        host_t.append(time.perf_counter() - t0)
    c = torch.from_numpy(np.ascontiguousarray(coords, np.int32)).to(dev)
    n = c.shape[0]
    need = ctypes.c_uint64()
    assert lib.vbm_build_device_workspace(n, ctypes.byref(need)) == 0
    ws = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    blob = torch.empty(int(hdr.blob_bytes), dtype=torch.uint8, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dev_t = []
    for _ in range(reps + 1):  # the first call warms up (code objects, allocator)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h2 = vbm.GridHeader()
        assert lib.vbm_build_device_plan(ctypes.c_void_p(c.data_ptr()), n, log2w, ctypes.c_void_p(ws.data_ptr()),
                                         need.value, ctypes.byref(h2), st) == 0
        assert lib.vbm_build_device_fill(ctypes.byref(h2), n, ctypes.c_void_p(ws.data_ptr()), need.value,
                                         ctypes.c_void_p(blob.data_ptr()), st) == 0
        torch.cuda.synchronize()
        dev_t.append(time.perf_counter() - t0)
    same = bytes(h2) == bytes(hdr) and bool(np.array_equal(blob.cpu().numpy(), host_blob))
    med = lambda v: sorted(v)[len(v) // 2]
    return {"host_ms": round(1e3 * med(host_t), 3), "device_ms": round(1e3 * med(dev_t[1:]), 3),
            "speedup": round(med(host_t) / med(dev_t[1:]), 1), "n_coords": int(n), "blob_identical": same,
            "workspace_bytes": int(need.value)}


def settle(fn, n_sets, seconds):
    """Untimed launches of fn for about `seconds` of wall time, then a sync: after
    the host-side set-up the GPU sits at its idle clocks, and a handful of warmup
    launches does not bring it to steady state (the first timed region then reads
    4-5 % slow against the same kernel timed later in the run)."""
    import torch
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < seconds:
        fn(k % n_sets)
        k += 1
    torch.cuda.synchronize()
    return k


def time_launches(fn, n_sets, steps, warmup):
    """Mean ms per launch of fn(k) for k = 0..steps-1 over rotating buffer sets."""
    import torch
    for k in range(warmup):
        fn(k % n_sets)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(steps):
        fn(k % n_sets)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_graph(fn, n_sets, steps, warmup):
    """Mean ms per launch of fn(k), k = 0..steps-1, captured once into a HIP graph and
    replayed: for kernels shorter than a Python launch, timing eager launches would
    measure the host.  Returns (ms, graph) so the caller can check a replay's output."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for k in range(warmup):
            fn(k % n_sets)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(steps):
            fn(k % n_sets)
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, graph


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--channels", type=int, default=16)
    ap.add_argument("--log2w", type=int, default=7)
    ap.add_argument("--no-extra", action="store_true", help="only the headline kernel")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="", help="profile mode: run only this variant (box_cs, box_c, box_s, box_p, "
                                               "weno_cs, decode, decode_sweep) and exit")
    ap.add_argument("--no-band", action="store_true",
                    help="skip the ~27M-voxel noisy narrow band (cached streaming box, W512, C=16; "
                         "about a minute of set-up), which is timed by default")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="profile mode: time a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library drives a single device, and a sharded run "
              "(contiguous block ranges per GPU plus a halo exchange) is not implemented; --gpus %d is "
              "not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from nanovdb_stencil_filtering_amd import inputs, vbm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        n = args.calib_copy << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        ms = time_launches(lambda k: dst.copy_(src), 1, args.steps, args.warmup)
        log("calib-copy %d MiB: %.4f ms/copy, %.1f GB/s (read+write)" % (args.calib_copy, ms, 2 * n * 4 / ms / 1e6))
        return
    vbm.load_library()
    C = args.channels
    log("bench: generating cfg-shell")
    coords = inputs.shell_coords(**inputs.CFG_SHELL)
    grids = {w: vbm.build(coords, w, device=dev) for w in sorted({args.log2w, 6, 7, 8, 9})}
    g = grids[args.log2w]
    N, L, nb, W = g.n_active, g.n_leaves, g.n_blocks, g.width
    log("bench: N=%d leaves=%d blocks=%d W=%d C=%d" % (N, L, nb, W, C))

    def make_sets(channels):
        sc = torch.from_numpy(inputs.sidecar(2, N, channels)).to(dev)
        per_set = 2 * sc.numel() * 4
        n_sets = max(2, -(-3 * MALL_BYTES // per_set))
        scs = [sc] + [sc.clone() for _ in range(n_sets - 1)]
        outs = [torch.empty_like(sc) for _ in range(n_sets)]
        return scs, outs, n_sets

    scs, outs, n_sets = make_sets(C)
    flags_cs = vbm.CACHED | vbm.STREAMING

    def box_step(grid, flags, scs_, outs_):
        return lambda k: vbm.box_filter(grid, scs_[k], flags, out=outs_[k])

    if args.only:
        # profiling mode: one variant, plain launches, no CPU leg
        variants = {"box_cs": flags_cs, "box_c": vbm.CACHED, "box_s": vbm.STREAMING, "box_p": 0}
        if args.only in ("decode", "decode_sweep"):
            fn = lambda k: vbm.decode(g, sweep=args.only == "decode_sweep")
        elif args.only == "weno_cs":
            fn = lambda k: vbm.weno_filter(g, scs[k], flags_cs, out=outs[k])
        else:
            fn = box_step(g, variants[args.only], scs, outs)
        settle(fn, n_sets, 0.1)
        ms = time_launches(fn, n_sets, args.steps, args.warmup)
        log("only %s: %.4f ms/launch" % (args.only, ms))
        return

    # sanity: the headline variant equals the plain materialised one, bit for bit
    a = vbm.box_filter(g, scs[0], flags_cs)
    b = vbm.box_filter(g, scs[0], 0)
    torch.cuda.synchronize()
    if not torch.equal(a.view(torch.int32), b.view(torch.int32)):
        raise SystemExit("bench: cached streaming and plain materialised outputs differ")

    log("bench: timing %d steps (warmup %d), %d rotating buffer sets" % (args.steps, args.warmup, n_sets))
    torch.cuda.synchronize()
    settled = settle(box_step(g, flags_cs, scs, outs), n_sets, 0.1)
    log("bench: %d untimed launches to bring the GPU to steady clocks" % settled)
    ms = time_launches(box_step(g, flags_cs, scs, outs), n_sets, args.steps, args.warmup)
    value = N * C / (ms * 1e-3)
    ab = alg_bytes_filter(N, L, nb, W, C)
    achieved = ab / (ms * 1e-3) / 1e9
    log("bench: headline %.4f ms/step, %.3e voxel*ch/s, %.1f GB/s" % (ms, value, achieved))
    # the same launches one by one, each between its own pair of events (after the timed
    # region): median and min per launch beside the mean above
    fn = box_step(g, flags_cs, scs, outs)
    pairs = []
    for k in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(k % n_sets)
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in pairs)
    per_launch = {"median": round(per[len(per) // 2], 5), "min": round(per[0], 5), "max": round(per[-1], 5)}
    log("bench: per launch median %.4f min %.4f max %.4f ms" % (per_launch["median"], per_launch["min"],
                                                                   per_launch["max"]))

    extra = {"headline_per_launch_ms": per_launch}
    if not args.no_extra:
        def rec(name, ms_, bytes_, n_work=None):
            d = {"ms": round(ms_, 5), "GBps": round(bytes_ / (ms_ * 1e-3) / 1e9, 1),
                 "hbm_frac": round(bytes_ / (ms_ * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if n_work is not None:
                d["voxel_ch_per_s"] = float("%.4e" % (n_work / (ms_ * 1e-3)))
            extra[name] = d
            log("  %-34s %.4f ms  %7.1f GB/s" % (name, ms_, d["GBps"]))

        names = {0: "plain_materialised", vbm.STREAMING: "plain_streaming", vbm.CACHED: "cached_materialised",
                 flags_cs: "cached_streaming"}
        for ch in sorted({1, 3, 8, 16}):
            s_, o_, ns_ = (scs, outs, n_sets) if ch == C else make_sets(ch)
            for w in (7, 9):
                gw = grids[w]
                for fl, nm in names.items():
                    t = time_launches(box_step(gw, fl, s_, o_), ns_, 20, 5)
                    rec("box_%s_W%d_C%d" % (nm, gw.width, ch), t,
                        alg_bytes_filter(N, L, gw.n_blocks, gw.width, ch), N * ch)
            # the 7-direction consumers at every BlockWidth: Laplacian and cross sum, tree
            # walk vs Cached, materialised vs streamed; the 19-tap axis sum at W128/W512
            for w in (6, 7, 8, 9):
                gw = grids[w]
                if ch in (1, 8):
                    ab_w = alg_bytes_filter(N, L, gw.n_blocks, gw.width, ch)
                    for op, opn in ((vbm.OP_LAPLACIAN, "laplacian"), (0, "cross_sum")):
                        for fl, nm in names.items():
                            t = time_launches(lambda k: vbm.cross_filter(gw, s_[k], fl | op, out=o_[k]), ns_, 20, 5)
                            rec("%s_%s_W%d_C%d" % (opn, nm, gw.width, ch), t, ab_w, N * ch)
                    if w in (7, 9):
                        for fl, nm in names.items():
                            t = time_launches(lambda k: vbm.axis_filter(gw, s_[k], fl, out=o_[k]), ns_, 20, 5)
                            rec("axis19_%s_W%d_C%d" % (nm, gw.width, ch), t, ab_w, N * ch)
                        # the WENO consumer of the same 19 taps (fifth-order WENO |grad u|^2)
                        for fl, nm in names.items():
                            t = time_launches(lambda k: vbm.weno_filter(gw, s_[k], fl, out=o_[k]), ns_, 20, 5)
                            rec("weno19_%s_W%d_C%d" % (nm, gw.width, ch), t, ab_w, N * ch)
            if ch != C:
                del s_, o_
        # the pages' resolver table, on the shell that reproduces their grid (R=160, h=2:
        # 1,288,594 voxels, 9,140 leaves): the six resolvers at C=1 and C=8, W128 and W512,
        # as speedups over the tree-walk materialised box (their baseline)
        pcoords = inputs.shell_coords(**inputs.PAGES_SHELL)
        pgrids = {w: vbm.build(pcoords, w, device=dev) for w in (7, 9)}
        Np = pgrids[7].n_active
        six = (("computeBoxStencil", "box", 0), ("forEachBoxStencil", "box", vbm.STREAMING),
               ("computeBoxStencilCached", "box", vbm.CACHED), ("forEachBoxStencilCached", "box", flags_cs),
               ("computeCrossStencil", "cross", 0), ("computeCrossStencilCached", "cross", vbm.CACHED))
        pages_table = {}
        for ch in (1, 8):
            psc = torch.from_numpy(inputs.sidecar(2, Np, ch)).to(dev)
            pn = max(2, -(-3 * MALL_BYTES // (2 * psc.numel() * 4)))
            ps = [psc] + [psc.clone() for _ in range(pn - 1)]
            po = [torch.empty_like(psc) for _ in range(pn)]
            for w in (7, 9):
                gw = pgrids[w]
                row = {}
                for name, op, fl in six:
                    if op == "box":
                        t = time_launches(lambda k: vbm.box_filter(gw, ps[k], fl, out=po[k]), pn, 30, 8)
                    else:
                        t = time_launches(lambda k: vbm.cross_filter(gw, ps[k], fl | vbm.OP_SUM, out=po[k]), pn, 30, 8)
                    row[name] = t
                base = row["computeBoxStencil"]
                for name, t in row.items():
                    pages_table["%s_W%d_C%d" % (name, gw.width, ch)] = {"ms": round(t, 5), "x": round(base / t, 2)}
                    log("  pages-shell %-26s W%d C%d %.4f ms  %.2fx" % (name, gw.width, ch, t, base / t))
            del ps, po, psc
        extra["pages_shell_resolvers"] = pages_table
        # hot-cache figure (single buffer set; the Infinity Cache may serve it)
        t = time_launches(box_step(g, flags_cs, scs[:1], outs[:1]), 1, 20, 5)
        rec("box_cached_streaming_W%d_C%d_hot" % (W, C), t, ab, N * C)
        # the same launch with the sidecar rows reached by 64-bit addresses (the path a
        # sidecar of 4 GiB or more takes by itself): one row per work-item, no prefetch
        t = time_launches(box_step(g, flags_cs | vbm.WIDE_ROWS, scs, outs), n_sets, 20, 5)
        rec("box_cached_streaming_W%d_C%d_wide_rows" % (W, C), t, ab, N * C)
        for ch in (1, 8):
            scw, outw, nw = make_sets(ch)
            abw = alg_bytes_filter(N, L, nb, W, ch)
            t = time_launches(box_step(g, flags_cs | vbm.WIDE_ROWS, scw, outw), nw, 20, 5)
            rec("box_cached_streaming_W%d_C%d_wide_rows" % (W, ch), t, abw, N * ch)
            del scw, outw
        # device-side metadata build (leaf directories, leafFirst, block metadata)
        # (short kernels: timed by replaying a captured graph, see time_graph)
        lib = vbm.load_library()
        import ctypes
        for w in (7, 9):
            gw = grids[w]
            total = torch.zeros(1, dtype=torch.int64, device=dev)

            def meta(k, gw=gw, total=total):
                rc = lib.vbm_build_metadata(ctypes.byref(gw.hdr), ctypes.c_void_p(gw.blob.data_ptr()),
                                            ctypes.c_void_p(total.data_ptr()),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                assert rc == 0
            blob0 = gw.blob.clone()
            t, _ = time_graph(meta, 1, 20, 5)
            assert torch.equal(gw.blob, blob0) and int(total.item()) == N, "metadata replay changed the grid"
            rec("build_metadata_W%d" % gw.width, t, 2 * 80 * L + (4 + gw.width // 8) * gw.n_blocks)
        # grid build from coordinates: host (vbm_build) vs device (vbm_build_device_plan + _fill)
        extra["build_cfg_shell_W128"] = time_builds(coords, 7, 3, dev)
        log("  build cfg-shell W128: host %.1f ms, device %.2f ms" % (extra["build_cfg_shell_W128"]["host_ms"],
                                                                     extra["build_cfg_shell_W128"]["device_ms"]))
        # decode: select-based vs the sweep it replaced, every width (the pages' A/B), on the
        # cfg-shell and on the decode-stress topology (20,000 leaves, occupancy 2-100 %)
        stress = inputs.leaf_bernoulli_coords(4, **inputs.STRESS)
        decode_grids = [("", grids[w], N, L) for w in (6, 7, 8, 9)]
        for w in (6, 7, 8, 9):
            gs = vbm.build(stress, w, device=dev)
            decode_grids.append(("_stress", gs, gs.n_active, gs.n_leaves))
        for tag, gw, N_, L_ in decode_grids:
            lo = [torch.empty(gw.n_slots, dtype=torch.int32, device=dev) for _ in range(4)]
            oo = [torch.empty(gw.n_slots, dtype=torch.int16, device=dev) for _ in range(4)]
            for fn, nm in ((lib.vbm_decode, "decode"), (lib.vbm_decode_sweep, "decode_sweep")):
                def dec(k, gw=gw, lo=lo, oo=oo, fn=fn):
                    rc = fn(ctypes.byref(gw.hdr), ctypes.c_void_p(gw.blob.data_ptr()),
                            ctypes.c_void_p(lo[k].data_ptr()), ctypes.c_void_p(oo[k].data_ptr()),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                    assert rc == 0
                t, _ = time_graph(dec, 4, 50, 15)
                ref_leaf, ref_off = vbm.decode(gw, sweep=(nm == "decode_sweep"))
                assert all(torch.equal(lo[k], ref_leaf.view(torch.int32)) and
                           torch.equal(oo[k], ref_off.view(torch.int16)) for k in range(4)), nm
                rec("%s%s_W%d" % (nm, tag, gw.width), t, alg_bytes_decode(N_, L_, gw.n_blocks, gw.width))

    traffic = counted_traffic() if (C == 16 and W == 128) else None

    # the pages' decode metric: ms of the select-based decode at BlockWidth 128 on the
    # cfg-shell (graph-replayed: the kernel is shorter than an eager Python launch)
    decode_ms = extra.get("decode_W128", {}).get("ms")
    if decode_ms is None:
        import ctypes
        lib = vbm.load_library()
        g7 = grids[7]
        lo = [torch.empty(g7.n_slots, dtype=torch.int32, device=dev) for _ in range(4)]
        oo = [torch.empty(g7.n_slots, dtype=torch.int16, device=dev) for _ in range(4)]

        def dec(k):
            rc = lib.vbm_decode(ctypes.byref(g7.hdr), ctypes.c_void_p(g7.blob.data_ptr()),
                                ctypes.c_void_p(lo[k].data_ptr()), ctypes.c_void_p(oo[k].data_ptr()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert rc == 0
        decode_ms = round(time_graph(dec, 4, 50, 15)[0], 5)

    band = None
    if not args.no_band:
        # configuration 5: noisy narrow band, W512, C=16 (a measurement, not the headline)
        del scs, outs
        log("bench: generating the narrow band")
        band = inputs.band_coords(5, **inputs.BAND)
        band_build = time_builds(band, 9, 1, dev)
        log("  build band W512: host %.1f ms, device %.2f ms" % (band_build["host_ms"], band_build["device_ms"]))
        gb = vbm.build(band, 9, device=dev)
        Nb = gb.n_active
        log("bench: band N=%d leaves=%d blocks=%d" % (Nb, gb.n_leaves, gb.n_blocks))
        scb = torch.empty((Nb + 1, 16), dtype=torch.float32, device=dev)
        step = 1 << 22
        for a in range(0, Nb + 1, step):
            b = min(Nb + 1, a + step)
            scb[a:b] = torch.from_numpy(inputs.sidecar_rows(6, a, b, 16)).to(dev)
        outb = torch.empty_like(scb)
        # the band's sidecar and output (1.7 GB each) exceed the Infinity Cache several times
        # over, so one buffer set already reaches every launch from HBM
        tb = time_launches(lambda k: vbm.box_filter(gb, scb, flags_cs, out=outb), 1, 10, 3)
        abb = alg_bytes_filter(Nb, gb.n_leaves, gb.n_blocks, gb.width, 16)
        band = {
            "ms": round(tb, 4), "GBps": round(abb / (tb * 1e-3) / 1e9, 1),
            "hbm_frac": round(abb / (tb * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "voxel_ch_per_s": float("%.4e" % (Nb * 16 / (tb * 1e-3))), "n_active": Nb, "n_leaves": gb.n_leaves,
            "kernel": headline_kernel(16), "alg_bytes_per_launch": abb, "build": band_build}
        extra["band_box_cached_streaming_W512_C16"] = band
        log("  band box cached streaming W512 C16: %.4f ms, %.1f GB/s" % (tb, abb / (tb * 1e-3) / 1e9))
        del scb, outb, gb

    cpu = None
    if not args.no_cpu:
        import numpy as np
        import oracle
        log("bench: CPU oracle baseline")
        ref = oracle.OracleGrid(coords)
        sc_host = inputs.sidecar(2, N, C)
        reps, t_cpu = 0, 0.0
        while t_cpu < 10.0 and reps < 20:
            t0 = time.perf_counter()
            ref.box(sc_host)
            t_cpu += time.perf_counter() - t0
            reps += 1
        cpu = {"value": float("%.4e" % (N * C * reps / t_cpu)), "unit": "active-voxel*channels/s", "cores": 1,
               "kind": "oracle",
               "sample": "whole cfg-shell box filter (C=%d, N=%d), %d passes, %.1f s, single thread" %
                         (C, N, reps, t_cpu),
               "host": host_cpu()}
        log("bench: oracle %.3e voxel*ch/s" % cpu["value"])
        # the same oracle function over disjoint index ranges on every usable host
        # core (ctypes releases the GIL inside the oracle's C calls); reported
        # beside the single-thread baseline, which stays the stated one
        from concurrent.futures import ThreadPoolExecutor
        n_thr = cpu["host"]["usable_cpus"] or 1
        bounds = [1 + (N * k) // n_thr for k in range(n_thr + 1)]
        chunks = [np.arange(bounds[k], bounds[k + 1], dtype=np.uint64) for k in range(n_thr)]
        with ThreadPoolExecutor(n_thr) as pool:
            reps_mt, t_mt = 0, 0.0
            while t_mt < 5.0 and reps_mt < 50:
                t0 = time.perf_counter()
                list(pool.map(lambda ix: ref.box(sc_host, ix), chunks))
                t_mt += time.perf_counter() - t0
                reps_mt += 1
        cpu["all_cores"] = {"value": float("%.4e" % (N * C * reps_mt / t_mt)), "cores": n_thr,
                            "sample": "the same whole-grid pass split into %d disjoint index ranges, one "
                                      "thread each, %d passes, %.1f s" % (n_thr, reps_mt, t_mt)}
        log("bench: oracle on %d threads %.3e voxel*ch/s" % (n_thr, cpu["all_cores"]["value"]))
        # the same single-thread oracle on the other measured steps (reported beside the
        # GPU figures under extra, never a target)

        def oracle_rate(fn, work, unit, min_s=1.0):
            n, t = 0, 0.0
            while t < min_s:
                t0 = time.perf_counter()
                fn()
                t += time.perf_counter() - t0
                n += 1
            return {"value": float("%.4e" % (work * n / t)), "unit": unit, "cores": 1, "kind": "oracle",
                    "passes": n, "seconds": round(t, 2)}
        cpu_more = {}
        for ch in (1, 8):
            sc_c = inputs.sidecar(3, N, ch)
            cpu_more["box_C%d" % ch] = oracle_rate(lambda: ref.box(sc_c), N * ch, "active-voxel*channels/s")
            cpu_more["laplacian_C%d" % ch] = oracle_rate(lambda: ref.cross(sc_c, "laplacian"), N * ch,
                                                         "active-voxel*channels/s")
            cpu_more["cross_sum_C%d" % ch] = oracle_rate(lambda: ref.cross(sc_c, "sum"), N * ch,
                                                         "active-voxel*channels/s")
            cpu_more["axis19_C%d" % ch] = oracle_rate(lambda: ref.axis(sc_c), N * ch, "active-voxel*channels/s")
            cpu_more["weno19_C%d" % ch] = oracle_rate(lambda: ref.weno(sc_c), N * ch, "active-voxel*channels/s")
        # the leaf / block metadata by their plain definitions (leaves, prefix
        # directories, leafFirst, firstLeafID, jumpMap)
        cpu_more["metadata_W128"] = oracle_rate(lambda: (ref.leaves(), ref.blocks(7)), L, "leaves/s")
        cpu_more["metadata_W128"]["sample"] = ("leaf masks and prefix directories from the voxel list, then "
                                               "firstLeafID and jumpMap per block (leafFirst comes with the "
                                               "oracle's grid)")
        cpu_more["decode_W128"] = oracle_rate(lambda: ref.decode(7), -(-N // 128) * 128, "slots/s")
        ref_stress = oracle.OracleGrid(inputs.leaf_bernoulli_coords(4, **inputs.STRESS))
        n_stress_slots = -(-ref_stress.n_active // 128) * 128
        cpu_more["decode_stress_W128"] = oracle_rate(lambda: ref_stress.decode(7), n_stress_slots, "slots/s")
        for k, v in cpu_more.items():
            log("bench: oracle %-20s %.3e %s" % (k, v["value"], v["unit"]))
        extra["cpu_oracle"] = cpu_more

    out = {
        "metric": "box-filter active-voxel*channels/s (cached streaming 27-tap box, C=%d)" % C,
        "value": float("%.6e" % value),
        "unit": "active-voxel*channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "sphere shell R=185 |d|<=1.5, N=%d, leaves=%d, BlockWidth %d, C=%d fp32 sidecar, "
                               "cached streaming box filter" % (N, L, W, C),
                   "n_active": N, "n_leaves": L, "block_width": W, "channels": C,
                   "buffer_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": ab, "kernel": headline_kernel(C)},
        "cpu_baseline": cpu,
        "decode_ms_W128": decode_ms,
        "band": band,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
