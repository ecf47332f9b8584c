"""Benchmark of the looped weight-shared transformer forward pass on one MI355X.

Timed step: one tl_prefill of 128 uniform token ids through the 407M-shaped
model (d 2048, 16 x 128 heads, ffn 5632, 2 pre-blocks + the shared loop block
at L = 8, INT4 group-128 weights, FP16 KV) with no logits materialised -- the
benchmark shape of the "Performance and Memory" page ("Benchmark Shape
Matters": seq_len 128, loops 8, no logits). `value` is prefill tokens/s.

Also reported (same JSON line):
  decode   -- cached greedy decode at L = 8 after a 256-token prompt, 128 steps,
              each step's argmax fed to the next on the device; ms/token.
  roofline -- the dominant prefill kernel (W4A16 MFMA GEMM) against the fp16
              MFMA peak; roofline_decode -- the W4 decode GEMV against HBM.
              Per-launch durations come from HIP event pairs the library
              attaches to every launch's own dispatch (tl_profile_begin/end)
              during a separate pass over the same steps.
  kernels  -- the W4 GEMV (M = 1, cold and warm weights) and the W4A16 GEMM
              (M = 1024) alone, at the loop block's four linear shapes.
  cpu_baseline -- the CPU oracle timed on this host on a bounded sample of
              the same prefill step (reported, not a target).
  decode graph replay, host enqueue time, self-speculative decode, store-h
              (FP16 and INT8 h), the FP16-body comparator, the empty-kernel
              dispatch floor, and the other 407M workloads (prefill seq 1024
              at L = 16 / 32; INT8-KV decode at context 2048, one lane and
              three lanes at L = 4 / 16 / 32), and the page's two comparison
              tables at L = 8 (W4 against FP16-body prefill at seq 128-1024;
              FP16 against INT8 KV decode at context 256 / 1024 / 2048), each
              skippable (--no-*).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Profiling helpers (no timed step): --pmc-kernels (single-kernel launches for
counter runs), --summarize-trace CSV / --summarize-pmc DIR... (per-kernel
tables, windowed with --trace-until / --trace-since), --ingest-pmc FETCH WRITE
(writes profiles/traffic.json), --cpu-configs (oracle on the other workloads).
"""
from __future__ import annotations

import argparse
import hashlib
import importlib.util
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tok/s + decode ms/token, 407M-shape W4 loop L=8; % HBM/MFMA peak"
PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def _build_mod():
    """looped_weight_shared_amd/build.py, loaded without importing the package."""
    spec = importlib.util.spec_from_file_location(
        "_tl_build", os.path.join(ROOT, "looped_weight_shared_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _ensure_built():
    """Builds libtl.so when it is missing or older than its sources."""
    _build_mod().ensure_current()


def _src_hash(*names):
    """Hash of the named kernel sources and of the per-source compiler flags
    they are built with (a counter entry is only current for both)."""
    dev_flags = _build_mod().DEVICE_FLAGS
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "looped_weight_shared_amd", "csrc", n), "rb") as f:
            h.update(f.read())
        if n in dev_flags:
            h.update(" ".join(dev_flags[n]).encode())
    return h.hexdigest()[:16]


GEMM_SRC = ["w4mm.hip", "w4_epi.h", "tl_device.h"]
GEMV_SRC = ["w4gemv.hip", "w4_epi.h", "tl_device.h"]


def _kernel_src(kernel_key):
    """The sources a counter entry was taken on: the prefill GEMM's or the decode GEMV's."""
    return GEMV_SRC if kernel_key.startswith("gemv") else GEMM_SRC


def _traffic(kernel_key, src_files, launches_bytes_expected=None):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters, if
    they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != _src_hash(*src_files):
        return None
    return ent.get("bytes_per_launch")


def _traffic_sum(keys):
    """Sum of the counters' bytes per launch over several kernels (None unless all are current)."""
    v = [_traffic(k, GEMV_SRC) for k in keys]
    return None if any(x is None for x in v) else sum(v)


def _pmc_dispatches(d, counter):
    """(kernel name, grid size, value) per dispatch from a rocprofv3 --pmc CSV directory."""
    import csv
    import glob
    out = []
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def ingest_pmc(fetch_dir, write_dir, copy_mib, kfetch_dir=None, kwrite_dir=None):
    """Writes profiles/traffic.json from two rocprofv3 --pmc runs of
    `bench.py --steps 3 --warmup 1 --no-cpu --no-spec --no-storeh --no-fp16body --no-kernels --no-configs
    --no-tables --decode-steps 4 --copy-mib <copy_mib>`, one with FETCH_SIZE, one with WRITE_SIZE (KiB per
    dispatch), and optionally two of `bench.py --pmc-kernels` (the cold M = 1 GEMVs). Each counter
    is scaled by what it reads for the plain device copy of copy_mib MiB in the same run."""
    copy_bytes = copy_mib * 2**20
    data = _ingest_runs(fetch_dir, write_dir, copy_bytes, _forward_kernels())
    run = ("bench.py --steps 3 --warmup 1 --no-cpu --no-spec --no-storeh --no-fp16body --no-kernels --no-configs "
           "--no-tables --decode-steps 4 --copy-mib %d" % copy_mib)
    cmds = ["export TMPDIR=/tmp; timeout -s KILL 150 rocprofv3 --pmc FETCH_SIZE -d %s -o run -f csv -- python -u %s"
            % (fetch_dir, run),
            "export TMPDIR=/tmp; timeout -s KILL 150 rocprofv3 --pmc WRITE_SIZE -d %s -o run -f csv -- python -u %s"
            % (write_dir, run)]
    ing = "python bench.py --ingest-pmc %s %s --copy-mib %d" % (fetch_dir, write_dir, copy_mib)
    if kfetch_dir and kwrite_dir:
        data.update(_ingest_runs(kfetch_dir, kwrite_dir, 256 * 2**20, _cold_gemv_kernels()))
        cmds += ["export TMPDIR=/tmp; timeout -s KILL 150 rocprofv3 --pmc %s -d %s -o run -f csv -- python -u "
                 "bench.py --pmc-kernels" % (c, d) for c, d in (("FETCH_SIZE", kfetch_dir), ("WRITE_SIZE", kwrite_dir))]
        ing += " --ingest-pmc-kernels %s %s" % (kfetch_dir, kwrite_dir)
    out = {"commands": cmds + [ing],
           "note": "per-dispatch KiB counters x 1024 x (copy bytes / the counter's reading for the plain device copy "
                   "of the same run); bytes_per_launch = scaled FETCH_SIZE + scaled WRITE_SIZE, averaged over the "
                   "kernel's dispatches"}
    out.update(data)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fo:
        json.dump(out, fo, indent=1)
    print(json.dumps(out, indent=1))


def _forward_kernels():
    d, f = 2048, 5632
    return {
        # dominant prefill kernel: the gate/up GEMM at M=128, 32x128 tiles: 88 column blocks x 4
        # row tiles = 352 blocks of 256 threads (the 256-token prompt's instance has 704)
        "gemm_gate_up": (lambda n, g: "w4_gemm_kernel<2, 2, false, 2>" in n and g == 352 * 256,
                         tl_packed_bytes(2 * f, d) + 128 * d * 2 + 128 * f * 2),
        # decode gate/up GEMV: the only two-n-block GEMV (fused RMSNorm, one row)
        "gemv_gate_up": (lambda n, g: "w4_gemv_kernel<2, 1, 1, 2, 1, false>" in n,
                         tl_packed_bytes(2 * f, d) + d * 4 + f * 2),
    }


def _gemv_a16_template(K, M=1):
    """Template of the fp16-input W4 GEMV the library launches for K (groups requested per wave:
    2, 6 or 8 for up to 16, 48 or 64 groups; fp16 chunks per thread rounded up to a power of 2)."""
    G = (K + 127) // 128
    gi = 2 if G <= 16 else (6 if G <= 48 else 8)
    apt_raw = -(-(M * (K // 8)) // 512)
    apt = next(a for a in (1, 2, 4, 8, 16) if apt_raw <= a)
    return f"w4_gemv_kernel<1, 0, 1, {gi}, {apt}, false>"


def _cold_gemv_kernels():
    """The M = 1 GEMVs of `bench.py --pmc-kernels` (fp16 A row in, fp32 C row out), one entry per
    loop-block linear, told apart by template and grid (512 threads, N / 16 blocks)."""
    out = {}
    for name, (N, K) in PMC_SHAPES.items():
        tmpl = _gemv_a16_template(K)
        out["gemv_cold_" + name] = ((lambda t, g0: (lambda n, g: t in n and g == g0))(tmpl, (N // 16) * 512),
                                    tl_packed_bytes(N, K) + K * 2 + N * 4)
    return out


def _ingest_runs(fetch_dir, write_dir, copy_bytes, kernels):
    fetch = _pmc_dispatches(fetch_dir, "FETCH_SIZE")
    write = _pmc_dispatches(write_dir, "WRITE_SIZE")

    def pick(rows, pred):
        v = [x[2] * 1024 for x in rows if pred(x[0], x[1])]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    def is_copy(name, grid):
        return "copyBuffer" in name or "copy_kernel" in name or "CopyKernel" in name
    cf, _ = pick([x for x in fetch if is_copy(x[0], x[1])][-1:], lambda n, g: True)
    cw, _ = pick([x for x in write if is_copy(x[0], x[1])][-1:], lambda n, g: True)
    if not cf or not cw:
        raise SystemExit("no copy-kernel dispatch found in the counter runs")
    kf, kw = copy_bytes / cf, copy_bytes / cw
    data = {}
    for key, (pred, algo) in kernels.items():
        fb, nf = pick(fetch, pred)
        wb, nw = pick(write, pred)
        if fb is None or wb is None:
            continue
        data[key] = {"source_hash": _src_hash(*_kernel_src(key)),
                     "bytes_per_launch": round(fb * kf + wb * kw),
                     "fetch_bytes_per_launch": round(fb * kf), "write_bytes_per_launch": round(wb * kw),
                     "algorithmic_bytes_per_launch": algo, "dispatches": [nf, nw],
                     "copy_calibration": {"bytes": copy_bytes, "fetch_factor": round(kf, 4),
                                          "write_factor": round(kw, 4)}}
    return data


def tl_packed_bytes(N, K):
    """Packed bytes of an N x K W4 linear: 1 KiB per 16x128 tile plus 32 B of scales."""
    return (N // 16) * ((K + 127) // 128) * 1056


def _layer_flops(s, M):
    """Algorithmic flop of one effective layer over M prompt rows: the four
    W4 GEMMs (2*M*N*K) and causal attention (4*H*hd*M(M+1)/2)."""
    d, f = s.d_model, s.ffn_dim
    gemm = 2 * M * (3 * d * d + d * d + 2 * f * d + d * f)
    return gemm + 4 * s.n_heads * s.head_dim * M * (M + 1) // 2


def other_configs(s, w, tl, Model, torch, synth, stream, only=None):
    """The 407M workloads besides the headline one: seq-1024 prefill at L=16
    and 32 (tokens/s against the MFMA roofline), and cached greedy decode at
    context 2048 with an INT8 KV cache (prompt 1920 + 128 steps), one lane at
    L=8 and three lanes at L=4/16/32 decoded together (against the HBM
    roofline of their algorithmic bytes)."""
    res = {}

    def timed(fn, reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    M = 1024
    t1024 = torch.from_numpy(synth.make_tokens(s.vocab, M, seed=0)).cuda()
    for Lx in (16, 32):
        if only and f"prefill_seq{M}_L{Lx}" not in only:
            continue
        mx = Model(w, max_seq=2048, max_loops=Lx, n_lanes=1, kv_dtype=tl.TL_KV_FP16, max_tokens=M)
        mx.set_loops(0, Lx)

        def step():
            mx.reset(0)
            mx.prefill(t1024)
        for _ in range(2):
            step()
        ms = timed(step, 5)
        flop = _layer_flops(s, M) * (s.n_pre + Lx)
        roof_us = flop / (PEAK_F16_TFLOPS * 1e12) * 1e6
        tl.tl_profile_begin(mx.ctx, 100000)
        for _ in range(2):
            step()
        prof = tl.tl_profile_end(mx.ctx)
        res[f"prefill_seq{M}_L{Lx}"] = {"ms_per_step": round(ms, 3), "tokens_per_s": round(M / ms * 1e3, 1),
                                        "gflop": round(flop / 1e9, 1), "mfma_roofline_us": round(roof_us, 1),
                                        "frac": round(roof_us / (ms * 1e3), 4),
                                        "kernels_us": {k: round(v / n * 1e3, 2) for k, (n, v) in prof.items() if n}}
        print(f"[bench] prefill seq {M} L={Lx}: {ms:.3f} ms/step, {M / ms * 1e3:,.0f} tok/s "
              f"({roof_us / (ms * 1e3):.1%} of the MFMA roofline)", file=sys.stderr, flush=True)
        mx.close()

    P, D = 1920, 128
    wbytes = (tl.tl_qlinear_packed_bytes(3 * s.d_model, s.d_model) + tl.tl_qlinear_packed_bytes(s.d_model, s.d_model)
              + tl.tl_qlinear_packed_bytes(2 * s.ffn_dim, s.d_model)
              + tl.tl_qlinear_packed_bytes(s.d_model, s.ffn_dim))
    kv_per_tok = 2 * s.n_heads * (s.head_dim + 2)  # INT8 K and V rows plus their fp16 scales, one layer
    for name, loops in (("decode_int8_ctx2048_L8", [8]), ("decode_int8_ctx2048_3lanes_L4_16_32", [4, 16, 32])):
        if only and name not in only:
            continue
        nl = len(loops)
        mi = Model(w, max_seq=2048, max_loops=max(loops), n_lanes=nl, kv_dtype=tl.TL_KV_INT8, max_tokens=P)
        bufs = [torch.zeros(nl, dtype=torch.int32, device="cuda") for _ in range(2)]

        def prime():
            for lane, Lx in enumerate(loops):
                mi.reset(lane)
                mi.set_loops(lane, Lx)
                pt = torch.from_numpy(synth.make_tokens(s.vocab, P, seed=0, lane=lane)).cuda()
                mi.prefill(pt, lane=lane, next_tok=bufs[0][lane:lane + 1])
        prime()
        for t in range(4):
            mi.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
        prime()
        it = iter(range(D))

        def dstep():
            t = next(it)
            mi.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
        ms = timed(dstep, D)
        # lanes decoded together share each layer's weight read (the deepest
        # lane sets the layer count) and the head read; K/V are per lane
        algo = (wbytes * (s.n_pre + max(loops)) + s.vocab * s.d_model * 2
                + sum(kv_per_tok * (s.n_pre + Lx) * (P + D // 2) for Lx in loops))
        roof_us = algo / (PEAK_HBM_GBS * 1e9) * 1e6
        prime()
        tl.tl_profile_begin(mi.ctx, 100000)
        for t in range(32):
            mi.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
        prof = tl.tl_profile_end(mi.ctx)
        res[name] = {"ms_per_step": round(ms, 4), "lanes": nl, "loops": loops, "context": P + D, "graph_replayed": False,
                     "algorithmic_bytes_per_step": int(algo), "hbm_roofline_us": round(roof_us, 1),
                     "frac": round(roof_us / (ms * 1e3), 4),
                     "kernels_us": {k: round(v / n * 1e3, 2) for k, (n, v) in prof.items() if n}}
        print(f"[bench] {name}: {ms:.4f} ms/step ({roof_us / (ms * 1e3):.1%} of the HBM roofline)",
              file=sys.stderr, flush=True)
        mi.close()
    return res


def pages_tables(s, w, tl, Model, torch, synth, stream):
    """The two comparisons the "Performance and Memory" page tabulates, at
    L = 8 on the 407M shape: (1) prefill of the INT4 loop block against the
    FP16 body (block weights dequantized once to fp16) at seq 128, 256, 512
    and 1024, no logits ("FP16 body cache" table); (2) cached decode with an
    FP16 KV cache against INT8 KV at contexts 256, 1024 and 2048 ("KV cache
    INT8" table): a prompt of N - 32 tokens, then 32 timed greedy steps up to
    context N. Synthetic weights and ids; the pages' rows are H100 numbers
    of a trained checkpoint, context only."""
    res = {"prefill_w4_vs_fp16_body_L8": {}, "decode_fp16_vs_int8_kv_L8": {}}
    L = 8

    def timed(fn, reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    mods = {body: Model(w, max_seq=2048, max_loops=L, n_lanes=1, kv_dtype=tl.TL_KV_FP16, max_tokens=1024,
                        fp16_body=(body == "fp16_body")) for body in ("w4", "fp16_body")}
    for mx in mods.values():
        mx.set_loops(0, L)
    for n in (128, 256, 512, 1024):
        toks = torch.from_numpy(synth.make_tokens(s.vocab, n, seed=0)).cuda()
        row = {}
        for body, mx in mods.items():
            def step():
                mx.reset(0)
                mx.prefill(toks)
            for _ in range(2):
                step()
            ms = timed(step, 5)
            row[f"{body}_ms"] = round(ms, 4)
            row[f"{body}_tok_s"] = round(n / ms * 1e3, 1)
        row["w4_speedup_over_fp16_body"] = round(row["fp16_body_ms"] / row["w4_ms"], 3)
        res["prefill_w4_vs_fp16_body_L8"][f"seq{n}"] = row
        print(f"[bench] prefill seq {n} L=8: W4 {row['w4_ms']:.3f} ms, FP16 body {row['fp16_body_ms']:.3f} ms",
              file=sys.stderr, flush=True)
    for mx in mods.values():
        mx.close()

    D = 32
    for kvname, kvd in (("fp16", tl.TL_KV_FP16), ("int8", tl.TL_KV_INT8)):
        mk = Model(w, max_seq=2048, max_loops=L, n_lanes=1, kv_dtype=kvd, max_tokens=2048 - D)
        mk.set_loops(0, L)
        bufs = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]
        for n in (256, 1024, 2048):
            pt = torch.from_numpy(synth.make_tokens(s.vocab, n - D, seed=0)).cuda()

            def prime():
                mk.reset(0)
                mk.prefill(pt, next_tok=bufs[0])
            prime()
            for t in range(4):
                mk.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
            prime()
            it = iter(range(D))

            def dstep():
                t = next(it)
                mk.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
            ms = timed(dstep, D)
            res["decode_fp16_vs_int8_kv_L8"].setdefault(f"ctx{n}", {})[f"{kvname}_kv_ms_per_token"] = round(ms, 4)
        mk.close()
    for n in (256, 1024, 2048):
        row = res["decode_fp16_vs_int8_kv_L8"][f"ctx{n}"]
        row["int8_over_fp16"] = round(row["int8_kv_ms_per_token"] / row["fp16_kv_ms_per_token"], 3)
        print(f"[bench] decode to context {n} L=8: FP16 KV {row['fp16_kv_ms_per_token']:.4f}, "
              f"INT8 KV {row['int8_kv_ms_per_token']:.4f} ms/token", file=sys.stderr, flush=True)
    return res


def host_info():
    """CPU model name (from /proc/cpuinfo) and the BLAS NumPy calls."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "logical_cpus": os.cpu_count()}


def cpu_configs(s, w, synth):
    """The float64 oracle on the other workloads, each on a bounded sample:
    cfg2 decode (8 cached steps after the 256-token prompt, L=8), seq-1024
    prefill at L=16 and L=32 (one run each), INT8-KV decode at context
    1920 + (one prefill of 1920 tokens, then 4 cached steps; L=8), and the
    three-lane step (the L=4/16/32 lanes' decode steps at context 1920 after
    each lane's prefill, 2 steps). Prefill time is reported beside the
    per-step figures."""
    import numpy as np
    import oracle
    om = oracle.OracleModel(w)
    res = {}
    tic = time.perf_counter

    def greedy_steps(prompt, L, steps, kv_int8):
        c = oracle.Cache(s, len(prompt) + steps + 1, kv_int8=kv_int8)
        t0 = tic()
        r = oracle.forward(om, prompt, L, cache=c)
        tp = tic() - t0
        tok = int(np.argmax(r["logits"]))
        t0 = tic()
        for _ in range(steps):
            lg, _ = oracle.decode_step(om, c, tok, L)
            tok = int(np.argmax(lg))
        return tp, (tic() - t0) / steps

    tp, td = greedy_steps(synth.make_tokens(s.vocab, 256, seed=0), 8, 8, False)
    res["decode_prompt256_L8_fp16kv"] = {"ms_per_token": round(td * 1e3, 1), "prefill_s": round(tp, 2),
                                         "sample": "8 cached greedy steps after the 256-token prompt"}
    print(f"[bench] oracle decode prompt 256 L=8: {td * 1e3:.1f} ms/token", file=sys.stderr, flush=True)
    t1024 = synth.make_tokens(s.vocab, 1024, seed=0)
    for Lx in (16, 32):
        t0 = tic()
        oracle.forward(om, t1024, Lx, logits=None)
        dt = tic() - t0
        res[f"prefill_seq1024_L{Lx}"] = {"tokens_per_s": round(1024 / dt, 1), "seconds": round(dt, 2)}
        print(f"[bench] oracle prefill seq 1024 L={Lx}: {1024 / dt:.1f} tok/s", file=sys.stderr, flush=True)
    p1920 = synth.make_tokens(s.vocab, 1920, seed=0)
    tp, td = greedy_steps(p1920, 8, 4, True)
    res["decode_int8_ctx1920_L8"] = {"ms_per_token": round(td * 1e3, 1), "prefill_s": round(tp, 2),
                                     "sample": "4 cached greedy steps after the 1920-token prompt"}
    print(f"[bench] oracle INT8 decode ctx 1920 L=8: {td * 1e3:.1f} ms/token", file=sys.stderr, flush=True)
    step = pre = 0.0
    for lane, Lx in enumerate((4, 16, 32)):
        tp, td = greedy_steps(synth.make_tokens(s.vocab, 1920, seed=0, lane=lane), Lx, 2, True)
        step += td
        pre += tp
    res["decode_int8_ctx1920_3lanes_L4_16_32"] = {"ms_per_step": round(step * 1e3, 1), "prefill_s": round(pre, 2),
                                                  "sample": "2 cached greedy steps per lane after its 1920-token "
                                                            "prompt; a step is one token on each lane"}
    print(f"[bench] oracle INT8 3-lane step: {step * 1e3:.1f} ms", file=sys.stderr, flush=True)
    res.update(host_info())
    return res


def kernel_leg(s, tl, torch, stream):
    """Single-kernel rates through tl_w4_linear at the loop block's four
    linear shapes (QKV, O, gate/up, down of the 407M shape): the W4 GEMV at
    M = 1 against HBM, with the weights cold -- the packed matrix replicated
    until the copies exceed 320 MB (more than the 256 MB Infinity Cache) and
    the launches cycling through them -- and warm (one copy re-read, as the
    loop's later iterations see it); and the W4A16 GEMM at M = 1024 (the
    seq-1024 prefill's shape) against the fp16 MFMA peak. A run of launches
    is captured once as a HIP graph (no memset nodes: each call is a single
    kernel) and replayed, so the host's call overhead does not pace the GPU;
    the figure is the replay's event time divided by its launches, per-dispatch
    gap included."""
    d, f = s.d_model, s.ffn_dim
    shapes = {"qkv": (3 * d, d), "o": (d, d), "gate_up": (2 * f, d), "down": (d, f)}
    g = torch.Generator(device="cpu").manual_seed(0)
    res = {}

    def per_launch_us(calls):
        tl.lib.tl_w4_linear(*calls[0], None)  # eager first call (one-time kernel attributes)
        torch.cuda.synchronize()
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            cs = torch.cuda.current_stream().cuda_stream
            for c in calls:
                if tl.lib.tl_w4_linear(*c, cs) != 0:
                    raise RuntimeError(tl.tl_last_error())
        cur = torch.cuda.current_stream()
        for _ in range(2):
            gph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 4
        e0.record(cur)
        for _ in range(reps):
            gph.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        del gph
        return e0.elapsed_time(e1) * 1e3 / (reps * len(calls))

    for name, (N, K) in shapes.items():
        qw = torch.randint(-2**31, 2**31 - 1, (N, K // 8), generator=g, dtype=torch.int32).cuda()
        sc = (torch.rand((N, (K + 127) // 128), generator=g) * 0.002 + 0.002).half().cuda()
        nb = tl.tl_qlinear_packed_bytes(N, K)
        ncopy = -(-320 * 2**20 // nb)
        packed = torch.empty((ncopy, -(-nb // 256) * 256), dtype=torch.uint8, device="cuda")
        tl.tl_qlinear_pack(qw, sc, N, K, packed[0])
        packed[1:].copy_(packed[0].expand(ncopy - 1, -1))
        torch.cuda.synchronize()
        del qw, sc
        ptrs = [packed[i].data_ptr() for i in range(ncopy)]
        r = {"N": N, "K": K, "packed_bytes": nb}
        for M in (1, 1024):
            A = (torch.randn((M, K), generator=g) * 0.5).half().cuda()
            C = torch.empty((M, N), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(tl.tl_w4_linear_ws_bytes(N, K, M), 256), dtype=torch.uint8, device="cuda")

            def calls(n, copies):
                return [(ptrs[i % copies], N, K, A.data_ptr(), M, C.data_ptr(), ws.data_ptr()) for i in range(n)]
            if M == 1:
                algo = nb + K * 2 + N * 4
                cold = per_launch_us(calls(ncopy, ncopy))
                warm = per_launch_us(calls(64, 1))
                r["gemv_m1"] = {"algorithmic_bytes": algo, "cold_us": round(cold, 3), "warm_us": round(warm, 3),
                                "cold_GBps": round(algo / cold / 1e3, 1), "warm_GBps": round(algo / warm / 1e3, 1),
                                "cold_frac_hbm": round(algo / cold / 1e3 / PEAK_HBM_GBS, 4), "copies": ncopy}
            else:
                flop = 2 * M * N * K
                t = per_launch_us(calls(16, ncopy))
                r["gemm_m1024"] = {"gflop": round(flop / 1e9, 2), "us": round(t, 2),
                                   "TFLOPs": round(flop / t / 1e6, 1),
                                   "frac_mfma": round(flop / t / 1e6 / PEAK_F16_TFLOPS, 4)}
            del A, C, ws
        del packed
        torch.cuda.empty_cache()
        res[name] = r
        print(f"[bench] kernel {name} N={N} K={K}: GEMV cold {r['gemv_m1']['cold_us']} us "
              f"({r['gemv_m1']['cold_GBps']} GB/s), warm {r['gemv_m1']['warm_us']} us; GEMM M=1024 "
              f"{r['gemm_m1024']['us']} us ({r['gemm_m1024']['TFLOPs']} TFLOP/s)", file=sys.stderr, flush=True)
    return res


PMC_SHAPES = {"qkv": (6144, 2048), "o": (2048, 2048), "gate_up": (11264, 2048), "down": (2048, 5632)}


def pmc_kernels(tl, torch):
    """Eager launches for counter runs, each launch a dispatch of its own: per
    loop-block linear shape, 4 W4A16 GEMMs at M = 1024 and 8 W4 GEMVs at M = 1
    cycling through copies of the packed matrix that together exceed 320 MB
    (cold weights); then 200 empty kernels and one plain 256 MiB device copy
    (the calibration of the FETCH_SIZE / WRITE_SIZE counters)."""
    g = torch.Generator(device="cpu").manual_seed(0)
    for name, (N, K) in PMC_SHAPES.items():
        qw = torch.randint(-2**31, 2**31 - 1, (N, K // 8), generator=g, dtype=torch.int32).cuda()
        sc = (torch.rand((N, (K + 127) // 128), generator=g) * 0.002 + 0.002).half().cuda()
        nb = tl.tl_qlinear_packed_bytes(N, K)
        ncopy = -(-320 * 2**20 // nb)
        packed = torch.empty((ncopy, -(-nb // 256) * 256), dtype=torch.uint8, device="cuda")
        tl.tl_qlinear_pack(qw, sc, N, K, packed[0])
        packed[1:].copy_(packed[0].expand(ncopy - 1, -1))
        for M, reps in ((1024, 4), (1, 8)):
            A = (torch.randn((M, K), generator=g) * 0.5).half().cuda()
            C = torch.empty((M, N), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(tl.tl_w4_linear_ws_bytes(N, K, M), 256), dtype=torch.uint8, device="cuda")
            for i in range(reps):
                tl.tl_w4_linear(packed[(i * 7) % ncopy], N, K, A, M, C, ws)
            torch.cuda.synchronize()
        print(f"[pmc] {name} N={N} K={K}: GEMM M=1024 x4, GEMV M=1 x8 over {ncopy} copies", file=sys.stderr,
              flush=True)
        del packed
        torch.cuda.empty_cache()
    tl.tl_launch_empty(200)
    src = torch.ones(256 * 2**18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def _kernel_name(full):
    """Kernel name without its argument list (and without an anonymous
    namespace's parenthesised prefix)."""
    full = full.replace("(anonymous namespace)::", "")
    return full.split("(")[0]


def _dims(r, field):
    """Total threads of a grid or workgroup from per-axis (or total) CSV columns."""
    if field + "_X" in r:
        return int(r[field + "_X"]) * int(r.get(field + "_Y") or 1) * int(r.get(field + "_Z") or 1)
    return int(r.get(field) or 0)


def summarize_pmc(dirs, until=None, since=None):
    """Per kernel (name, grid) averages of every counter found in the given
    rocprofv3 --pmc output directories (CSV), one line per kernel. `until` and
    `since` window each run's dispatches as in summarize_trace."""
    import collections
    import csv
    import glob
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn) as f:
                rows = list(csv.DictReader(f))
            mark = until or since
            if mark:
                cut = min((int(r["Dispatch_Id"]) for r in rows if mark in r["Kernel_Name"]), default=1 << 62)
                rows = [r for r in rows if (int(r["Dispatch_Id"]) < cut) == bool(until)]
            if rows:
                for r in rows:
                    key = (_kernel_name(r["Kernel_Name"])[:60], int(r["Grid_Size"]))
                    acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for v in acc.values() for c in v})
    print("kernel".ljust(62) + "grid".rjust(10) + "    n" + "".join(c[:24].rjust(26) for c in names))
    for (k, grid), v in sorted(acc.items(), key=lambda kv: kv[0]):
        n = max(len(x) for x in v.values())
        print(k.ljust(62) + str(grid).rjust(10) + f"{n:5d}" +
              "".join((f"{sum(v[c]) / len(v[c]):26.1f}" if v.get(c) else " " * 26) for c in names))


def summarize_trace(csv_path, until=None, since=None):
    """Per (kernel, grid) call count and average / median / min duration (us)
    from a rocprofv3 --kernel-trace CSV, in descending total time. With
    `until` (`since`), only the dispatches that start before (at or after) the
    first dispatch whose kernel name contains that text are counted."""
    import collections
    import csv
    import statistics
    d = collections.defaultdict(list)
    meta = {}
    with open(csv_path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    mark = until or since
    if mark:
        cut = next((i for i, r in enumerate(rows) if mark in r["Kernel_Name"]), len(rows))
        rows = rows[:cut] if until else rows[cut:]
    if rows:
        for r in rows:
            name = _kernel_name(r["Kernel_Name"])
            grid = _dims(r, "Grid_Size")
            wg = _dims(r, "Workgroup_Size")
            key = (name, grid)
            d[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            meta[key] = (wg, r.get("LDS_Block_Size", r.get("Lds_Size", "")), r.get("VGPR_Count", r.get("Arch_VGPR_Count", "")))
    tot = sum(sum(v) for v in d.values()) or 1.0
    print(" calls   avg_us   med_us   min_us   %time   blocks   wg  lds_B vgpr  kernel")
    for key, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        wg, lds, vg = meta[key]
        blocks = key[1] // wg if wg else key[1]
        print(f"{len(v):6d} {sum(v) / len(v):8.2f} {statistics.median(v):8.2f} {min(v):8.2f} "
              f"{100 * sum(v) / tot:7.2f} {blocks:8d} {wg:4d} {lds:>6} {vg:>4}  {key[0][:90]}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--prompt", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-spec", action="store_true", help="skip the self-speculative decode leg")
    ap.add_argument("--no-storeh", action="store_true", help="skip the store-h legs (TL_KV_H16, TL_KV_H8)")
    ap.add_argument("--no-fp16body", action="store_true", help="skip the FP16-body leg")
    ap.add_argument("--no-kernels", action="store_true",
                    help="skip the single-kernel leg (cold W4 GEMV and M=1024 GEMM at the loop block's shapes)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other 407M workloads (seq-1024 prefill at L=16/32; INT8 KV decode at "
                         "context 2048, one lane at L=8 and three lanes at L=4/16/32)")
    ap.add_argument("--no-tables", action="store_true",
                    help="skip the pages' comparison tables (W4 vs FP16-body prefill at seq 128-1024; FP16 vs "
                         "INT8 KV decode at context 256/1024/2048)")
    ap.add_argument("--configs", metavar="NAMES",
                    help="comma-separated subset of the other workloads (prefill_seq1024_L16, prefill_seq1024_L32, "
                         "decode_int8_ctx2048_L8, decode_int8_ctx2048_3lanes_L4_16_32)")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="also time the CPU oracle on those workloads (bounded samples; about two minutes)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="finish with one plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit (no GPU)")
    ap.add_argument("--ingest-pmc-kernels", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="with --ingest-pmc: also the cold M = 1 GEMVs from two --pmc-kernels counter runs")
    ap.add_argument("--pmc-kernels", action="store_true",
                    help="only launch the single kernels for counter runs (GEMM M=1024, cold GEMV M=1, empty "
                         "kernels) and exit")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print per-kernel averages of the counters in rocprofv3 --pmc output dirs and exit (no GPU)")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print per-kernel durations from a rocprofv3 --kernel-trace CSV and exit (no GPU)")
    ap.add_argument("--trace-until", metavar="NAME",
                    help="with --summarize-trace/--summarize-pmc: only dispatches before the first one of a "
                         "kernel whose name contains NAME")
    ap.add_argument("--trace-since", metavar="NAME",
                    help="with --summarize-trace/--summarize-pmc: only dispatches from the first one of a "
                         "kernel whose name contains NAME on")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.trace_until, args.trace_since)
        return
    if args.ingest_pmc:
        kp = args.ingest_pmc_kernels or (None, None)
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.copy_mib or 256, kp[0], kp[1])
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.trace_until, args.trace_since)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path; the forward pass would shard across GPUs by lanes (data parallel).",
              file=sys.stderr)
        sys.exit(2)

    _ensure_built()
    import numpy as np
    import torch

    import synth
    import looped_weight_shared_amd as tl
    from looped_weight_shared_amd import model as mod
    from looped_weight_shared_amd.model import Model

    torch.cuda.set_device(0)
    if args.pmc_kernels:
        pmc_kernels(tl, torch)
        return
    s = synth.SHAPES["m407"]
    L, SEQ = 8, 128
    t0 = time.time()
    w = synth.make_weights(s, seed=0)
    print(f"[bench] synthetic 407M-shape weights in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    m = Model(w, max_seq=2048, max_loops=L, n_lanes=1, kv_dtype=tl.TL_KV_FP16,
              max_tokens=max(SEQ, args.prompt))
    m.set_loops(0, L)
    toks = torch.from_numpy(synth.make_tokens(s.vocab, SEQ, seed=0)).cuda()
    stream = torch.cuda.current_stream()

    def prefill_step():
        m.reset(0)               # host-only: the lane is empty again
        m.prefill(toks)          # no hidden, no logits

    # ---------------------------------------------------------------- prefill leg
    for _ in range(args.warmup):
        prefill_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        prefill_step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    tok_s = SEQ / (ms_step / 1e3)
    print(f"[bench] prefill seq {SEQ} L={L}: {ms_step:.3f} ms/step, {tok_s:,.0f} tok/s",
          file=sys.stderr, flush=True)

    # per-kernel durations over the same steps (HIP events around every launch)
    tl.tl_profile_begin(m.ctx, 200000)
    for _ in range(args.steps):
        prefill_step()
    prof = tl.tl_profile_end(m.ctx)
    kern_prefill = {k: (n, ms / n * 1e3) for k, (n, ms) in prof.items() if n}
    d, f = s.d_model, s.ffn_dim
    flops = {"qkv": 2 * SEQ * 3 * d * d, "o": 2 * SEQ * d * d, "gate_up": 2 * SEQ * 2 * f * d,
             "down": 2 * SEQ * d * f}
    gemm_kinds = [k for k in flops if k in kern_prefill]
    dom = max(gemm_kinds, key=lambda k: kern_prefill[k][0] * kern_prefill[k][1])
    avg_us = kern_prefill[dom][1]
    achieved = flops[dom] / (avg_us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                "traffic": _traffic("gemm_" + dom, GEMM_SRC),
                "kernel": f"w4_gemm_kernel ({dom}: M={SEQ} N={2 * f if dom == 'gate_up' else (3 * d if dom == 'qkv' else d)} "
                          f"K={f if dom == 'down' else d})",
                "flop_per_launch": flops[dom], "avg_launch_us": round(avg_us, 3)}

    out = {"metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic",
           "config": {"workload": "407M-shape looped transformer prefill, seq 128, L=8 (2 pre + 1 loop "
                                  "block, 10 effective layers), W4 g128 weights, FP16 KV, no logits",
                      "global_batch": 1, "seq_len": SEQ, "loops": L, "parallelism": "none (1 GPU)"},
           "roofline": roofline,
           "kernels_prefill_us": {k: round(v[1], 3) for k, v in kern_prefill.items()}}

    # ---------------------------------------------------------------- decode leg
    if not args.no_decode:
        P, D = args.prompt, args.decode_steps
        ptoks = torch.from_numpy(synth.make_tokens(s.vocab, P, seed=0)).cuda()
        nx = torch.zeros(1, dtype=torch.int32, device="cuda")
        bufs = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]

        def decode_run(steps, timed):
            m.reset(0)
            m.prefill(ptoks, next_tok=bufs[0])
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record(stream)
            for t in range(steps):
                m.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
            ev[1].record(stream)
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1])

        def host_enqueue_ms():
            # host time to enqueue one step (the calls return before the GPU is done)
            m.reset(0)
            m.prefill(ptoks, next_tok=bufs[0])
            torch.cuda.synchronize()
            h0 = time.perf_counter()
            for t in range(D):
                m.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
            h = (time.perf_counter() - h0) * 1e3 / D
            torch.cuda.synchronize()
            return h

        decode_run(8, False)                       # warm-up
        ms_tok = decode_run(D, True) / D
        host_ms = host_enqueue_ms()
        # the same steps replayed from captured graphs (one per shape and
        # token buffer; the part count changes every 128 keys): the host
        # enqueues ~5x faster, the GPU time is a few percent higher
        m.set_graphs(2)
        decode_run(8, False)
        ms_graph = decode_run(D, True) / D
        host_graph = host_enqueue_ms()
        m.set_graphs(0)
        print(f"[bench] decode L={L} prompt {P} + {D} steps: {ms_tok:.4f} ms/token (host enqueue {host_ms:.4f} "
              f"ms/step); graph-replayed {ms_graph:.4f} ms/token (host enqueue {host_graph:.4f} ms/step)",
              file=sys.stderr, flush=True)
        # profiled pass
        m.reset(0)
        m.prefill(ptoks, next_tok=bufs[0])
        tl.tl_profile_begin(m.ctx, 200000)
        for t in range(D):
            m.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
        dprof = tl.tl_profile_end(m.ctx)
        kern_dec = {k: (n, ms_ / n * 1e3) for k, (n, ms_) in dprof.items() if n}
        wbytes = {"qkv": tl.tl_qlinear_packed_bytes(3 * d, d), "o": tl.tl_qlinear_packed_bytes(d, d),
                  "gate_up": tl.tl_qlinear_packed_bytes(2 * f, d), "down": tl.tl_qlinear_packed_bytes(d, f)}
        gb = {k: wbytes[k] / (kern_dec[k][1] * 1e-6) / 1e9 for k in wbytes if k in kern_dec}
        dk = "gate_up"
        rd = {"bound": "hbm", "achieved": round(gb[dk], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": round(gb[dk] / PEAK_HBM_GBS, 4),
              "traffic": _traffic("gemv_" + dk, GEMV_SRC),
              "kernel": "w4_gemv_kernel (gate_up: M=1 N=11264 K=2048)",
              "bytes_per_launch": wbytes[dk], "avg_launch_us": round(kern_dec[dk][1], 3),
              "note": "weights of the loop block are re-read every iteration; iterations after the "
                      "first can be served from the 256 MB Infinity Cache, so this is an in-situ rate"}
        algo = (sum(wbytes.values()) * (s.n_pre + L) + s.vocab * d * 2
                + 2 * 2 * s.n_heads * s.head_dim * (s.n_pre + L) * (P + D / 2))
        out["decode"] = {"ms_per_token": round(ms_tok, 4), "prompt": P, "steps": D, "loops": L,
                         "kv": "fp16", "graph_replayed": False, "host_enqueue_ms_per_step": round(host_ms, 4),
                         "graph_replayed_ms_per_token": round(ms_graph, 4),
                         "graph_replayed_host_enqueue_ms_per_step": round(host_graph, 4),
                         "algorithmic_bytes_per_token": int(algo),
                         "hbm_roofline_ms_per_token": round(algo / (PEAK_HBM_GBS * 1e9) * 1e3, 4),
                         "frac_of_hbm_roofline": round(algo / (PEAK_HBM_GBS * 1e9) * 1e3 / ms_tok, 4),
                         "kernels_us": {k: round(v[1], 3) for k, v in kern_dec.items()},
                         "gemv_GBps": {k: round(v, 1) for k, v in gb.items()}}
        out["roofline_decode"] = rd

        # ------------------------------------------------------------ self-speculative decode
        # same prompt and depth; drafts at L=2 ("Current Status" page: L=2
        # draft, L=8 verify). Wall clock (the call synchronises once per round).
        spec = {}
        for kd in (() if args.no_spec else (2, 4, 7)):
            m.reset(0)
            m.prefill(ptoks, next_tok=bufs[0])
            torch.cuda.synchronize()
            t_first = int(bufs[0].item())
            m.spec_decode(t_first, 8, draft_loops=2, k_draft=kd)      # warm-up
            m.reset(0)
            m.prefill(ptoks, next_tok=bufs[0])
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            _, st = m.spec_decode(t_first, D, draft_loops=2, k_draft=kd)
            dt = time.perf_counter() - t0
            spec[f"k{kd}"] = {"ms_per_token": round(dt * 1e3 / D, 4), "rounds": st.rounds,
                              "drafted": st.drafted, "accepted": st.accepted,
                              "speedup_vs_plain": round(ms_tok / (dt * 1e3 / D), 3)}
            print(f"[bench] spec decode draft L=2 verify L={L} k={kd}: {dt * 1e3 / D:.4f} ms/token, "
                  f"accepted {st.accepted}/{st.drafted}", file=sys.stderr, flush=True)
        # ------------------------------------------------------------ store-h cache
        # same prompt/steps with h kept per position (FP16, or INT8 per
        # 128-element group) and K/V rebuilt per layer
        if not args.no_storeh:
            kvb = {k: tl.tl_kv_layer_bytes(mod.make_config(s, 2048, L, kv_dtype=v))
                   for k, v in (("fp16", tl.TL_KV_FP16), ("h16", tl.TL_KV_H16), ("h8", tl.TL_KV_H8))}
            out["store_h"] = {"kv_bytes_per_lane_layer": kvb,
                              "note": "h16 prefill bit-identical to FP16 K/V; decode rebuilds K/V of the "
                                      "context every layer (h8: from fp16(q*s) of the INT8 rows)"}
            for name, kvd in (("h16", tl.TL_KV_H16), ("h8", tl.TL_KV_H8)):
                mh = Model(w, max_seq=2048, max_loops=L, n_lanes=1, kv_dtype=kvd,
                           max_tokens=max(SEQ, args.prompt))
                mh.set_loops(0, L)

                def prefill_h():
                    mh.reset(0)
                    mh.prefill(toks)
                for _ in range(3):
                    prefill_h()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(10):
                    prefill_h()
                e1.record(stream)
                torch.cuda.synchronize()
                ms_pre_h = e0.elapsed_time(e1) / 10
                mh.reset(0)
                mh.prefill(ptoks, next_tok=bufs[0])
                torch.cuda.synchronize()
                e0.record(stream)
                for t in range(D):
                    mh.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
                e1.record(stream)
                torch.cuda.synchronize()
                ms_tok_h = e0.elapsed_time(e1) / D
                mh.close()
                out["store_h"][name] = {"kv_saving": round(1 - kvb[name] / kvb["fp16"], 3),
                                        "prefill_ms_seq128": round(ms_pre_h, 4),
                                        "decode_ms_per_token": round(ms_tok_h, 4)}
                print(f"[bench] store-h {name}: prefill {ms_pre_h:.3f} ms/step, decode {ms_tok_h:.4f} ms/token, "
                      f"KV bytes {kvb[name]} vs {kvb['fp16']}", file=sys.stderr, flush=True)

        # ------------------------------------------------------------ FP16 body
        # the same steps with the block weights dequantized once to fp16
        if not args.no_fp16body:
            mf = Model(w, max_seq=2048, max_loops=L, n_lanes=1, kv_dtype=tl.TL_KV_FP16,
                       max_tokens=max(SEQ, args.prompt), fp16_body=True)
            mf.set_loops(0, L)

            def prefill_f():
                mf.reset(0)
                mf.prefill(toks)
            for _ in range(3):
                prefill_f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                prefill_f()
            e1.record(stream)
            torch.cuda.synchronize()
            ms_pre_f = e0.elapsed_time(e1) / 20
            mf.reset(0)
            mf.prefill(ptoks, next_tok=bufs[0])
            torch.cuda.synchronize()
            e0.record(stream)
            for t in range(D):
                mf.decode_step(bufs[t % 2], next_tok=bufs[(t + 1) % 2])
            e1.record(stream)
            torch.cuda.synchronize()
            ms_tok_f = e0.elapsed_time(e1) / D
            wsb = {k: tl.tl_weights_ws_bytes(mod.make_config(s, 2048, L, fp16_body=v)) for k, v in (("w4", 0), ("fp16", 1))}
            mf.close()
            out["fp16_body"] = {"weights_ws_bytes": wsb, "prefill_ms_seq128": round(ms_pre_f, 4),
                                "prefill_speedup_w4_over_fp16": round(ms_pre_f / ms_step, 3),
                                "decode_ms_per_token": round(ms_tok_f, 4),
                                "decode_speedup_w4_over_fp16": round(ms_tok_f / ms_tok, 3)}
            print(f"[bench] FP16 body: prefill {ms_pre_f:.3f} ms/step, decode {ms_tok_f:.4f} ms/token, "
                  f"weights {wsb['fp16']} vs {wsb['w4']} B", file=sys.stderr, flush=True)

        if spec:
            out["spec_decode"] = {"draft_loops": 2, "verify_loops": L, "prompt": P, "tokens": D,
                                  "note": "greedy; acceptance is a property of the weights (synthetic here)",
                                  **spec}

    # ---------------------------------------------------------------- single kernels
    if not args.no_kernels:
        out["kernels"] = kernel_leg(s, tl, torch, stream)
        # per-dispatch floor: back-to-back empty kernels, eager (event time / count)
        tl.tl_launch_empty(100)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        tl.tl_launch_empty(2000)
        e1.record(stream)
        torch.cuda.synchronize()
        out["dispatch_floor_us"] = round(e0.elapsed_time(e1) * 1e3 / 2000, 3)
        print(f"[bench] empty kernels back to back: {out['dispatch_floor_us']} us each", file=sys.stderr,
              flush=True)

    # ---------------------------------------------------------------- other workloads
    if not args.no_configs:
        out["other_configs"] = other_configs(s, w, tl, Model, torch, synth, stream,
                                             args.configs.split(",") if args.configs else None)

    if not args.no_tables:
        out["pages_tables"] = pages_tables(s, w, tl, Model, torch, synth, stream)

    # ---------------------------------------------------------------- decode roofline
    # headline: the four loop-block GEMVs with cold weights (kernel leg), their
    # algorithmic bytes summed over their summed launch times; the in-situ
    # gate/up rate (weights possibly served by the Infinity Cache) is context
    if "decode" in out:
        rd = out["roofline_decode"]
        if "kernels" in out:
            kl = out["kernels"]
            byts = sum(kl[k]["gemv_m1"]["algorithmic_bytes"] for k in kl)
            us = sum(kl[k]["gemv_m1"]["cold_us"] for k in kl)
            agg = byts / us / 1e3
            out["roofline_decode"] = {
                "bound": "hbm", "achieved": round(agg, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(agg / PEAK_HBM_GBS, 4), "traffic": _traffic_sum(["gemv_cold_" + k for k in kl]),
                "kernel": "w4_gemv_kernel, M=1, cold weights: QKV + O + gate/up + down of the loop block "
                          "(bytes summed over summed launch times)",
                "bytes_per_launch": {k: kl[k]["gemv_m1"]["algorithmic_bytes"] for k in kl},
                "avg_launch_us": {k: kl[k]["gemv_m1"]["cold_us"] for k in kl},
                "in_situ": rd}

    # ---------------------------------------------------------------- CPU oracle on the other workloads
    if args.cpu_configs:
        out["cpu_configs"] = cpu_configs(s, w, synth)

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
        except Exception:
            cores = os.cpu_count()
        om = oracle.OracleModel(w)
        ptok = synth.make_tokens(s.vocab, SEQ, seed=0)
        n, t_start = 0, time.perf_counter()
        while True:
            oracle.forward(om, ptok, L, logits=None)
            n += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or n >= 50:
                break
        out["cpu_baseline"] = {"value": round(SEQ * n / el, 2), "unit": "tokens/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"{n} x float64 oracle prefill of the same 128-token L=8 step "
                                         f"({el:.1f} s; weight dequantization not timed)",
                               **host_info()}
    if args.copy_mib:
        src = torch.ones(args.copy_mib * 2**18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
