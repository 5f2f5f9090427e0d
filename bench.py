#!/usr/bin/env python3
"""Decode-step benchmark of the TurboQuant KV-cache path on one MI355X.

One step = append-encode of the newest tokens + one decode-attention step
over the whole packed context, as one fused launch
(tq_append_chunk_attend_decode; the same work as the two calls
tq_encode_kv + tq_attend_decode, also timed, as `step_two_calls_us`). The
default workload is the long-context decode: batch 1, 32 query / 8 KV heads,
d = 128, 524288-token context, 3-bit keys / 4-bit values with fp16 norms,
4096 tokens appended per step, bf16 N(0,1) inputs.

The K timed steps run twice: as replays of a HIP graph of the step (one
graph launch per step, so that the host's per-call Python and argument
set-up cannot starve the GPU) and as two eager launches per step; the step
time is the faster of the two (`config.launch` names it; `step_graph_us`
and `step_eager_us` hold both). Decode and
encode rates are measured on back-to-back launches bracketed by one pair of
HIP events on the launch stream (no per-call markers inside the timed
region).

Prints ONE JSON line on stdout (progress goes to stderr):
  value         KV-tokens/s of the whole step (B * N / step time)
  roofline      the decode kernel's algorithmic bytes per launch / its average
                launch duration, against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle on the host cores, one process per
                (batch, KV head) unit, the step's append encode and decode
  other_workloads  decode rate and roofline of the two other 128k+ contexts
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP16_DENSE_PEAK_TFLOPS = 2500.0
METRIC = "packed decode-attention KV-tokens/s and achieved HBM GB/s as % of peak"
DECODE_KERNEL = "k_decode_mx"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "decode_attention_seeded_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def profile_summary(name):
    """A committed profile summary (JSON under profiles/) if it was taken on
    the current kernel sources, else None."""
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    return t if t.get("source_hash") == source_hash() else None


def alg_bytes_of(tq, cfg, w, q):
    """Algorithmic bytes of one decode call: every packed plane over the
    context, the queries in and the fp32 outputs."""
    cache_bytes, _ = tq.tq_cache_bytes(cfg, w.B, w.Hkv, w.N)
    return cache_bytes + q.numel() * q.element_size() + w.B * w.Hq * w.d * 4


def to_dev(torch, raw, in_dtype):
    import numpy as np
    if in_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(raw)).cuda()


def timed(torch, fn, n, warm=3):
    """Average microseconds of fn() over n back-to-back calls (one event pair
    around the loop, on the current stream)."""
    for _ in range(warm):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


# --------------------------------------------------------------------------
# CPU oracle baseline: one spawned process per (batch, KV head) unit.
# --------------------------------------------------------------------------

_BARRIER = None


def _cpu_init(barrier):
    global _BARRIER
    _BARRIER = barrier


def _cpu_unit(job):
    """Worker: the oracle's encode of one unit's context (set-up, untimed),
    then the step for that unit (append encode of the newest tokens, decode
    of its G query heads over the whole context), timed. With a barrier the
    units start their timed phase together."""
    wid, b, h, threads = job
    os.environ["OMP_NUM_THREADS"] = str(threads)
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(threads)
    except Exception:
        pass
    import oracle as o
    import seeded_inputs as si
    w = si.WORKLOADS[wid]
    A = w.append or 0
    _, fk = si.kv_rows(w, si.T_K, b, h, 0, w.N)
    _, fv = si.kv_rows(w, si.T_V, b, h, 0, w.N)
    fk = fk.astype(np.float64)[None, None]
    fv = fv.astype(np.float64)[None, None]
    kw = dict(seed=w.seed, bits_k=w.bits_k, bits_v=w.bits_v, norm_dtype=w.norm_dtype,
              qjl=w.qjl, qjl_seed=w.qjl_seed)
    t0 = time.perf_counter()
    cache = o.encode_kv(fk[:, :, :w.N - A], fv[:, :, :w.N - A], **kw)
    for key in ("k_enc", "v_enc", "k_qjl"):     # the encode's intermediates
        cache.pop(key, None)
    setup = time.perf_counter() - t0
    _, qf = si.queries(w)
    q = qf[b:b + 1, h * w.G:(h + 1) * w.G].astype(np.float64)
    if _BARRIER is not None:
        _BARRIER.wait()
    t0 = time.perf_counter()
    if A:
        app = o.encode_kv(fk[:, :, w.N - A:], fv[:, :, w.N - A:], **kw)
        for key in ("kc", "vc", "kn", "vn", "kq", "kr"):
            if key in cache:
                cache[key] = np.concatenate([cache[key], app[key]], axis=2)
    o.attend(q, cache, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k, bits_v=w.bits_v, Hkv=1,
             qjl=w.qjl, qjl_seed=w.qjl_seed)
    step = time.perf_counter() - t0
    return setup, step


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family, model and
    stepping numbers (virtual machines often report a generic name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                      # the first processor is enough
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(w, max_units):
    """The oracle (NumPy fp64, as it stands) on the host's cores: one spawned
    process per (batch, KV head) unit, each unit's share of the step run on
    its whole context; the units run side by side and start their timed
    phase together (a barrier after each unit's set-up). Covers min(units,
    max_units) units and scales by units / covered."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)][:max_units]
    procs = min(len(units), cores)
    threads = max(1, cores // procs)
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(procs) if len(units) == procs else None
    t0 = time.perf_counter()
    with ctx.Pool(procs, initializer=_cpu_init, initargs=(barrier,)) as pool:
        res = pool.map(_cpu_unit, [(w.wid, b, h, threads) for b, h in units], chunksize=1)
    wall = time.perf_counter() - t0
    rounds = (len(units) + procs - 1) // procs
    step_s = max(r[1] for r in res) * rounds * (w.B * w.Hkv) / len(units)
    return {
        "value": w.B * w.N / step_s,
        "unit": "KV-tokens/s",
        "cores": cores,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "processes": procs,
        "threads_per_process": threads,
        "sample": (f"{len(units)} of {w.B * w.Hkv} (batch, KV head) units, one process each "
                   f"({procs} side by side, {threads} BLAS thread(s) each): "
                   f"{w.append or 0}-token append encode and decode of {w.G} query heads over "
                   f"all {w.N} tokens; slowest unit {max(r[1] for r in res):.2f} s, scaled by "
                   f"units/processes to the whole step ({step_s:.2f} s); encoding each "
                   f"unit's cache first took up to {max(r[0] for r in res):.1f} s (not part of "
                   f"the step); {wall:.0f} s wall"),
    }


# --------------------------------------------------------------------------
# Decode of one workload: encode, back-to-back and cold decode calls.
# --------------------------------------------------------------------------

def decode_record(torch, tq, si, w, n_calls, flush, fsink):
    k_host = si.kv_full(w, si.T_K)
    v_host = si.kv_full(w, si.T_V)
    q_raw, _ = si.queries(w)
    K, V, q = (to_dev(torch, k_host, w.in_dtype), to_dev(torch, v_host, w.in_dtype),
               to_dev(torch, q_raw, w.in_dtype))
    del k_host, v_host
    cfg = tq.Config(d=w.d, bits_k=w.bits_k, bits_v=w.bits_v, norm_dtype=w.norm_dtype,
                    qjl=w.qjl, seed=w.seed, qjl_seed=w.qjl_seed)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_encode_kv(cfg, K[:, :, :1].contiguous(), V[:, :, :1].contiguous(), 0, cache)
    torch.cuda.synchronize()
    enc_us = timed(torch, lambda: tq.tq_encode_kv(cfg, K, V, 0, cache), 3, warm=1)
    in_bytes = (K.numel() + V.numel()) * K.element_size()
    out_bytes = tq.tq_cache_bytes(cfg, w.B, w.Hkv, w.N)[0]
    del K, V
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))
    dec = lambda: tq.tq_attend_decode(cfg, q, cache, w.N, out, ws)
    # the inputs are generated on the host for seconds while the GPU idles:
    # 200 untimed calls (about 20 ms) bring its clocks back before timing
    us = timed(torch, dec, n_calls, warm=200)
    cold = []
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(10):
        tq.tq_read_probe(flush, fsink)
        c0, c1 = ev(), ev()
        c0.record()
        dec()
        c1.record()
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1) * 1e3)
    import numpy as np
    alg = alg_bytes_of(tq, cfg, w, q)
    bf16_kv = 2 * w.B * w.Hkv * w.N * w.d * 2
    rec = {
        "workload": w.name,
        "decode_call_us": round(us, 2),
        "decode_call_cold_median_us": round(float(np.median(cold)), 2),
        "kv_tokens_per_s": round(w.B * w.N / (us * 1e-6), 1),
        "algorithmic_bytes": alg,
        "achieved_gbps": round(alg / us / 1e3, 1),
        "frac_of_hbm_peak": round(alg / us / 1e3 / HBM_PEAK_GBPS, 4),
        "splits": tq.tq_num_splits(cfg, w.B, w.Hq, w.Hkv, w.N),
        "kv_bytes_vs_bf16": round(out_bytes / bf16_kv, 4),
        "encode": {"tokens": w.N, "us": round(enc_us, 1), "bytes_in": in_bytes,
                   "bytes_out": out_bytes,
                   "frac_of_hbm_peak": round((in_bytes + out_bytes) / enc_us / 1e3 /
                                             HBM_PEAK_GBPS, 4)},
    }
    del cache, ws, out, q
    return rec


def _exact_attention(q, k, v, G, scale):
    """softmax(scale q K^T) V in float64 from the rounded inputs [B][H][n][d]."""
    import numpy as np
    heads = np.arange(q.shape[1]) // G
    s = scale * np.einsum("bhd,bhtd->bht", q, k[:, heads])
    s -= s.max(-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(-1, keepdims=True)
    return np.einsum("bht,bhtd->bhd", p, v[:, heads])


def accuracy_report(torch, tq, si):
    """The method's accuracy on the GPU's own outputs (small seeded cases).

    p13: relative L2 error of the decode output against unquantized fp64
    attention softmax(q K^T / sqrt(d)) V, per format, iid and correlated
    queries (README, "Measured results"). qjl_score_bias: mean error of the
    score difference s_j - s_other over two-token contexts with queries
    correlated to token j, MSE-only against QJL-corrected (README, "The 1-bit
    QJL residual"); the kernel's score difference is read back from its
    output o = p0 v0 + (1 - p0) v1, with v0 and v1 the dequantized values
    (one-token decodes of the same codes).
    """
    import numpy as np
    def run(w, q_raw, n_ctx, scale=0.0, swap=False):
        cfg = tq.Config(d=w.d, bits_k=w.bits_k, bits_v=w.bits_v, norm_dtype=w.norm_dtype,
                        qjl=w.qjl, seed=w.seed, qjl_seed=w.qjl_seed)
        kr, vr = si.kv_full(w, si.T_K), si.kv_full(w, si.T_V)
        if swap:
            kr, vr = kr[:, :, ::-1].copy(), vr[:, :, ::-1].copy()
        cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
        tq.tq_encode_kv(cfg, to_dev(torch, kr, w.in_dtype), to_dev(torch, vr, w.in_dtype), 0,
                        cache)
        out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
        ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, n_ctx))
        tq.tq_attend_decode(cfg, to_dev(torch, q_raw, w.in_dtype), cache, n_ctx, out, ws,
                            scale=scale)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    f64 = lambda raw, w: (si.bf16_bits_to_f32(raw) if w.in_dtype == "bf16"
                          else raw.astype(np.float32)).astype(np.float64)
    p13 = {}
    for structure in ("iid", "correlated"):
        rows = {}
        for bk, bv in ((2, 2), (3, 3), (4, 4), (3, 4)):
            for qjl in (False, True):
                w = si.small_workload(B=1, Hq=32, Hkv=8, d=128, N=4096, bits_k=bk, bits_v=bv,
                                      norm_dtype="f16", qjl=qjl, in_dtype="bf16",
                                      structure=structure, wid=301)
                q_raw, qf = si.queries(w)
                got = run(w, q_raw, w.N)
                ref = _exact_attention(qf.astype(np.float64), f64(si.kv_full(w, si.T_K), w),
                                       f64(si.kv_full(w, si.T_V), w), w.G, 1 / math.sqrt(w.d))
                e = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
                rows[f"K{bk}{'+QJL' if qjl else ''}/V{bv}"] = {
                    "mean": round(float(e.mean()), 5), "max": round(float(e.max()), 5)}
        p13[f"{structure}_queries"] = rows
    bias = {}
    scale = 1.0 / 128
    for qjl in (False, True):
        w = si.small_workload(B=64, Hq=32, Hkv=8, d=128, N=2, bits_k=3, bits_v=4,
                              norm_dtype="f16", qjl=qjl, in_dtype="bf16",
                              structure="correlated", wid=300)
        q_raw, qf = si.queries(w)
        o2 = run(w, q_raw, 2, scale)
        v0 = run(w, q_raw, 1, scale)
        v1 = run(w, q_raw, 1, scale, swap=True)
        dv = v0 - v1
        p0 = np.clip(((o2 - v1) * dv).sum(-1) / (dv * dv).sum(-1), 1e-9, 1 - 1e-9)
        heads = np.arange(w.Hq) // w.G
        s = scale * np.einsum("bhd,bhtd->bht", qf.astype(np.float64),
                              f64(si.kv_full(w, si.T_K), w)[:, heads])
        sign = np.where(si.correlated_tokens(w) == 0, 1.0, -1.0)
        err = (np.log(p0 / (1 - p0)) - (s[..., 0] - s[..., 1])) * sign
        bias["qjl" if qjl else "mse_only"] = round(float(err.mean()), 5)
        bias[("qjl" if qjl else "mse_only") + "_sem"] = round(
            float(err.std() / math.sqrt(err.size)), 5)
        bias["mean_true_difference"] = round(float(((s[..., 0] - s[..., 1]) * sign).mean()), 5)
        bias["pairs"] = int(err.size)
    bias["format"] = "K3/V4 (+QJL), d 128, scale 1/128, q = 0.8 k_j + 0.6 eps"
    return {"p13_rel_l2_error_vs_fp64_attention": p13, "qjl_score_bias": bias}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-affine", action="store_true")
    ap.add_argument("--no-accuracy", action="store_true",
                    help="skip the accuracy report (P13 errors, QJL score bias)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the decode records of the other 128k+ workloads")
    ap.add_argument("--cpu-units", type=int, default=8,
                    help="(batch, KV head) units the CPU oracle runs (scaled to all)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="copy a buffer of this many MiB once before timing (a kernel of "
                         "known traffic, for calibrating HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_seeded_amd as tq
    import seeded_inputs as si

    w = si.WORKLOADS[args.workload]
    A = w.append if w.append else 0
    log(f"workload {w.wid}: {w.name}")
    torch.cuda.set_device(0)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # ---------------- inputs (seeded, host-generated, uploaded once)
    t0 = time.time()
    k_host = si.kv_full(w, si.T_K)
    v_host = si.kv_full(w, si.T_V)
    q_raw, _ = si.queries(w)
    log(f"generated inputs in {time.time() - t0:.1f} s")
    K, V = to_dev(torch, k_host, w.in_dtype), to_dev(torch, v_host, w.in_dtype)
    q = to_dev(torch, q_raw, w.in_dtype)
    del k_host, v_host

    cfg = tq.Config(d=w.d, bits_k=w.bits_k, bits_v=w.bits_v, norm_dtype=w.norm_dtype,
                    qjl=w.qjl, seed=w.seed, qjl_seed=w.qjl_seed)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    n_bulk = w.N - A
    k_bulk, v_bulk = K[:, :, :n_bulk].contiguous(), V[:, :, :n_bulk].contiguous()
    k_app, v_app = K[:, :, n_bulk:].contiguous(), V[:, :, n_bulk:].contiguous()
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    splits = tq.tq_num_splits(cfg, w.B, w.Hq, w.Hkv, w.N)
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))

    # bulk encode (after a one-token encode that loads the code object): 20
    # back-to-back calls after 10 untimed ones, which let the clocks settle
    # (the first calls after an idle GPU run up to 30% slower)
    tq.tq_encode_kv(cfg, k_bulk[:, :, :1].contiguous(), v_bulk[:, :, :1].contiguous(), 0, cache)
    torch.cuda.synchronize()
    bulk_us = timed(torch, lambda: tq.tq_encode_kv(cfg, k_bulk, v_bulk, 0, cache), 20, warm=10)
    bulk_in = (k_bulk.numel() + v_bulk.numel()) * k_bulk.element_size()
    bulk_out = tq.tq_cache_bytes(cfg, w.B, w.Hkv, n_bulk)[0]
    del k_bulk, v_bulk
    log(f"bulk encode of {n_bulk} tokens x {w.B * w.Hkv} heads: {bulk_us:.1f} us "
        f"({(bulk_in + bulk_out) / bulk_us / 1e3:.0f} GB/s in + out)")

    # the step: one launch that appends the chunk and attends (every split
    # encodes its share of the new rows, then decodes its old and new
    # tokens); the same work as two calls, timed as step_two_calls_us
    def step():
        if A:
            tq.tq_append_chunk_attend_decode(cfg, k_app, v_app, q, cache, w.N, out, ws)
        else:
            tq.tq_attend_decode(cfg, q, cache, w.N, out, ws)

    def step_two_calls():
        if A:
            tq.tq_encode_kv(cfg, k_app, v_app, n_bulk, cache)
        tq.tq_attend_decode(cfg, q, cache, w.N, out, ws)

    if args.copy_probe_mb:
        src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {args.copy_probe_mb} MiB read + written")

    # ---------------- the step as a HIP graph (one launch per step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    ref_out = out.clone()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; timing {args.steps} steps (graph replays)")
    s0, s1 = ev(), ev()
    torch.cuda.synchronize()
    s0.record()
    for _ in range(args.steps):
        graph.replay()
    s1.record()
    torch.cuda.synchronize()
    graph_us = s0.elapsed_time(s1) * 1e3 / args.steps
    replay_equal = bool(torch.equal(out, ref_out))
    # the same K steps launched eagerly (two launches each, W warm-up steps
    # first); the step's time is the faster of the two launch modes (a
    # replay's fixed cost on this stack can exceed two kernel launches)
    step_eager_us = timed(torch, step, args.steps, warm=args.warmup)
    graph_faster = graph_us <= step_eager_us
    ms_per_step = min(graph_us, step_eager_us) / 1e3
    fused_desc = ("one tq_append_chunk_attend_decode launch per step" if A else
                  "one tq_attend_decode launch per step")
    launch_mode = (f"{fused_desc}, captured as a HIP graph (one replay per step)"
                   if graph_faster else f"{fused_desc}, launched directly (faster here than "
                   "one HIP-graph replay)")
    step_two_us = timed(torch, step_two_calls, args.steps, warm=args.warmup)
    log(f"step {graph_us:.1f} us (graph), {step_eager_us:.1f} us eager; graph output "
        f"equals the eager step: {replay_equal}; as two calls (encode, decode) "
        f"{step_two_us:.1f} us")

    # ---------------- decode alone: back-to-back launches
    alg_bytes = alg_bytes_of(tq, cfg, w, q)
    n_dec = max(args.steps, 50)
    dec_us = timed(torch, lambda: tq.tq_attend_decode(cfg, q, cache, w.N, out, ws), n_dec)
    achieved = alg_bytes / dec_us / 1e3
    log(f"decode call {dec_us:.2f} us over {n_dec} back-to-back calls = {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBPS:.3f} of peak)")

    # streaming-read probe over as many bytes as one decode call reads, and
    # decode calls after a 1 GiB read has evicted the 256 MB last-level cache
    probe_bytes = (alg_bytes + 15) // 16 * 16
    pbuf = torch.empty(probe_bytes, dtype=torch.uint8, device="cuda")
    pbuf.random_(0, 255)
    sink = tq.tq_read_probe(pbuf)
    probe_us = timed(torch, lambda: tq.tq_read_probe(pbuf, sink), 20)
    probe_gbps = probe_bytes / probe_us / 1e3
    del pbuf
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    fsink = tq.tq_read_probe(flush)
    cold_us = []
    for _ in range(20):
        tq.tq_read_probe(flush, fsink)
        c0, c1 = ev(), ev()
        c0.record()
        tq.tq_attend_decode(cfg, q, cache, w.N, out, ws)
        c1.record()
        torch.cuda.synchronize()
        cold_us.append(c0.elapsed_time(c1) * 1e3)
    log(f"read probe {probe_gbps:.1f} GB/s over {probe_bytes} B; cold decode median "
        f"{np.median(cold_us):.1f} us")

    # append-encode alone
    enc_us = None
    if A:
        enc_us = timed(torch, lambda: tq.tq_encode_kv(cfg, k_app, v_app, n_bulk, cache), 20)

    # single-token generation step (append token N-1, attend over N): the
    # fused entry point against the two calls it replaces, on the same cache
    k1, v1 = K[:, :, w.N - 1:].contiguous(), V[:, :, w.N - 1:].contiguous()

    def two_calls():
        tq.tq_encode_kv(cfg, k1, v1, w.N - 1, cache)
        tq.tq_attend_decode(cfg, q, cache, w.N, out, ws)

    def fused():
        tq.tq_append_attend_decode(cfg, k1, v1, q, cache, w.N, out, ws)

    # four interleaved rounds of 100 calls each, the median round of each
    # (one round each was at the mercy of the clocks after the cold-cache
    # measurements above)
    rounds = {"two": [], "fused": []}
    for _ in range(4):
        rounds["two"].append(timed(torch, two_calls, 100, warm=10))
        rounds["fused"].append(timed(torch, fused, 100, warm=10))
    single = {
        "two_calls_us": round(float(np.median(rounds["two"])), 2),
        "fused_us": round(float(np.median(rounds["fused"])), 2),
        "measured": "median of 4 interleaved rounds of 100 back-to-back calls",
    }
    log(f"single-token step: encode + decode {single['two_calls_us']} us, "
        f"fused {single['fused_us']} us")

    # causal prefill of a chunk at the end of the context (the appended
    # chunk, else the last 1024 tokens) over the packed cache, on the
    # matrix cores; algorithmic flops = 4 d per (query row, visible token)
    prefill = None
    if not args.no_prefill:
        nq = A if A else min(1024, w.N)
        qc_raw, _ = si.chunk_queries(w, nq)
        qc = to_dev(torch, qc_raw, w.in_dtype)
        pout = torch.empty((w.B, w.Hq, nq, w.d), dtype=torch.float32, device="cuda")
        pus = timed(torch, lambda: tq.tq_attend_prefill(cfg, qc, cache, w.N, pout), 3, warm=1)
        visible = nq * (w.N - nq) + nq * (nq + 1) // 2
        flops = 4 * w.d * w.B * w.Hq * visible
        tflops = flops / (pus * 1e-6) / 1e12
        prefill = {"chunk_tokens": nq, "context": w.N, "ms": round(pus / 1e3, 3),
                   "tflops": round(tflops, 1),
                   "frac_of_fp16_dense_peak": round(tflops / FP16_DENSE_PEAK_TFLOPS, 4),
                   "flops": flops}
        del qc, pout
        log(f"prefill of {nq} tokens over {w.N}: {pus / 1e3:.2f} ms, {tflops:.1f} TFLOP/s")

    # the group-affine variant (group 64, fp16 scale and bias, rotated keys)
    # at 4 bits, the README's iso-byte comparison format, on the same K/V
    # and query; bytes = its six planes over N tokens plus q in and out
    affine = None
    if not args.no_affine:
        acfg = tq.AffineConfig(d=w.d, bits_k=4, bits_v=4, group=64, seed=w.seed)
        acache = tq.AffineCache(acfg, w.B, w.Hkv, w.N)
        tq.tq_affine_encode_kv(acfg, K, V, 0, acache)
        aws = tq.workspace(tq.tq_affine_workspace_bytes(acfg, w.B, w.Hq, w.Hkv, w.N))
        aout = torch.empty_like(out)
        aus = timed(torch, lambda: tq.tq_affine_attend_decode(acfg, q, acache, w.N, aout, aws),
                    20)
        abytes = acache.nbytes() + q.numel() * q.element_size() + aout.numel() * 4
        affine = {"format": "K4/V4 group-64 affine, fp16 scale and bias, rotated keys",
                  "us_per_call": round(aus, 2),
                  "kv_tokens_per_s": round(w.B * w.N / (aus * 1e-6), 1),
                  "algorithmic_bytes": abytes,
                  "gbps": round(abytes / aus / 1e3, 1),
                  "frac_of_hbm_peak": round(abytes / aus / 1e3 / HBM_PEAK_GBPS, 4),
                  "finite": bool(torch.isfinite(aout).all())}
        del acache, aws, aout
        log(f"affine K4V4 decode: {aus:.1f} us/call, {affine['gbps']} GB/s")

    # dense bf16 decode on the same GPU (same split-K skeleton, bf16 rows)
    qbytes = q.numel() * q.element_size()
    dense = None
    if not args.no_dense and w.in_dtype == "bf16":
        dws = tq.workspace(tq.tq_dense_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N))
        dout = torch.empty_like(out)
        dus = timed(torch, lambda: tq.tq_dense_decode_bf16(q, K, V, dout, dws), 20)
        dbytes = 2 * K.numel() * 2 + qbytes + out.numel() * 4
        dgbps = dbytes / dus / 1e3
        probe_bound_us = dbytes / probe_gbps / 1e3
        dense = {"decode_us": round(dus, 2), "achieved_gbps": round(dgbps, 1),
                 "frac_of_hbm_peak": round(dgbps / HBM_PEAK_GBPS, 4),
                 "frac_of_read_probe": round(dgbps / probe_gbps, 4),
                 "packed_speedup": round(dus / dec_us, 3),
                 "read_probe_bound_us": round(probe_bound_us, 2),
                 "packed_speedup_vs_probe_bound_dense": round(probe_bound_us / dec_us, 3),
                 "ideal_byte_ratio": round(dbytes / alg_bytes, 3)}
        log(f"dense bf16 decode {dus:.1f} us ({dgbps:.1f} GB/s, {dgbps / probe_gbps:.2f} of the "
            f"read probe); at the probe rate it would take {probe_bound_us:.1f} us")
    # other fractional splits on the same K/V and query: K3/V3 and the
    # 2.5-bit K2/V3, on the same matrix-core kernel
    formats = None
    if not args.no_others and args.workload == 4:
        formats = {}
        for bk, bv in ((3, 3), (2, 3)):
            fcfg = tq.Config(d=w.d, bits_k=bk, bits_v=bv, norm_dtype=w.norm_dtype, qjl=False,
                             seed=w.seed)
            fcache = tq.PackedCache(fcfg, w.B, w.Hkv, w.N)
            tq.tq_encode_kv(fcfg, K, V, 0, fcache)
            fws = tq.workspace(tq.tq_workspace_bytes(fcfg, w.B, w.Hq, w.Hkv, w.N))
            fout = torch.empty_like(out)
            fus = timed(torch, lambda: tq.tq_attend_decode(fcfg, q, fcache, w.N, fout, fws), 50)
            fb = tq.tq_cache_bytes(fcfg, w.B, w.Hkv, w.N)[0] + qbytes + fout.numel() * 4
            formats[f"K{bk}/V{bv}"] = {
                "decode_call_us": round(fus, 2), "algorithmic_bytes": fb,
                "achieved_gbps": round(fb / fus / 1e3, 1),
                "frac_of_hbm_peak": round(fb / fus / 1e3 / HBM_PEAK_GBPS, 4),
                "kernel": "k_decode_mx (matrix cores)",
                "kv_bytes_vs_bf16": round(tq.tq_cache_bytes(fcfg, w.B, w.Hkv, w.N)[0] /
                                          (2 * K.numel() * 2), 4)}
            del fcache, fws, fout
            log(f"K{bk}/V{bv} decode over {w.N} tokens: {fus:.1f} us "
                f"({formats[f'K{bk}/V{bv}']['frac_of_hbm_peak']} of peak)")
    # the headline format on the vector-ALU decode kernel (no matrix cores)
    valu = None
    if not args.no_others and args.workload == 4:
        os.environ["TQ_DECODE_VALU"] = "1"
        try:
            vws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))
            vout = torch.empty_like(out)
            vus = timed(torch, lambda: tq.tq_attend_decode(cfg, q, cache, w.N, vout, vws), 30)
            valu = {"decode_call_us": round(vus, 2),
                    "frac_of_hbm_peak": round(alg_bytes / vus / 1e3 / HBM_PEAK_GBPS, 4),
                    "kernel": "k_decode_pk (TQ_DECODE_VALU=1)",
                    "max_abs_diff_vs_matrix_core": float((vout - out).abs().max())}
            del vws, vout
        finally:
            del os.environ["TQ_DECODE_VALU"]
        log(f"VALU decode kernel: {valu['decode_call_us']} us ({valu['frac_of_hbm_peak']} of peak)")
    del K, V

    # the other two 128k+ contexts (outlier keys d 256 K2/V2; QJL K3/V4)
    others = None
    if not args.no_others and args.workload == 4:
        del cache, ws
        others = {}
        for wid in (3, 5):
            log(f"workload {wid}: {si.WORKLOADS[wid].name}")
            rec = decode_record(torch, tq, si, si.WORKLOADS[wid], 100, flush, fsink)
            others[str(wid)] = rec
            log(f"  decode {rec['decode_call_us']} us = {rec['achieved_gbps']} GB/s "
                f"({rec['frac_of_hbm_peak']} of peak); cold median "
                f"{rec['decode_call_cold_median_us']} us")
    del flush

    accuracy = None
    if not args.no_accuracy:
        accuracy = accuracy_report(torch, tq, si)
        log(f"accuracy: QJL score bias {accuracy['qjl_score_bias']}")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the host cores")
        cpu = cpu_baseline(w, args.cpu_units)
        log(f"oracle: {cpu['value']:.3e} KV-tokens/s ({cpu['sample']})")

    trace = profile_summary("decode_long_context_kernel_trace.json") \
        if args.workload == 4 else None
    traffic = profile_summary(f"decode_hbm_traffic_workload{w.wid}.json")
    kernel_us = trace.get("kernel_avg_us") if trace else None
    bf16_kv = 2 * w.B * w.Hkv * w.N * w.d * 2
    fp16_kv = bf16_kv
    cache_bytes = tq.tq_cache_bytes(cfg, w.B, w.Hkv, w.N)[0]
    cfg_desc = {
        "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
        "context": w.N, "bits_k": w.bits_k, "bits_v": w.bits_v, "norms": w.norm_dtype,
        "qjl": w.qjl, "append_tokens_per_step": A, "inputs": f"{w.in_dtype} seeded synthetic",
        "splits": splits, "launch": launch_mode,
    }
    rec = {
        "metric": METRIC,
        "value": round(w.B * w.N / (ms_per_step * 1e-3), 1),
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 operands, f32 accumulate",
        "dtype_note": ("decode products on fp16 operands (rotated query, scaled centroids, "
                       "softmax weight times value norm) with fp32 accumulation; encode in fp64"),
        "data": "synthetic",
        "config": cfg_desc,
        "roofline": {
            "bound": "hbm",
            "kernel": DECODE_KERNEL,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic.get("hbm_bytes_per_launch") if traffic else None,
            "bytes_per_launch": alg_bytes,
            "launch_us": round(dec_us, 2),
            "measured": f"{n_dec} back-to-back launches between two HIP events",
            "kernel_trace_avg_us": kernel_us,
            "frac_kernel_trace": (round(alg_bytes / kernel_us / 1e3 / HBM_PEAK_GBPS, 4)
                                  if kernel_us else None),
            # in the committed traced run: the traced back-to-back calls and
            # this script's HIP-event time of the same calls
            "trace_back_to_back_us": trace.get("back_to_back_run_mean_us") if trace else None,
            "trace_run_launch_us": (trace.get("bench_live_launch_us_in_traced_run")
                                    if trace else None),
            "frac_of_read_probe": round(achieved / probe_gbps, 4),
        },
        "cpu_baseline": cpu,
        "decode_call_us": round(dec_us, 2),
        "decode_kv_tokens_per_s": round(w.B * w.N / (dec_us * 1e-6), 1),
        "decode_call_cold_us": {
            "note": "each call after a 1 GiB streaming read (last-level cache evicted)",
            "p10": round(float(np.percentile(cold_us, 10)), 2),
            "median": round(float(np.median(cold_us)), 2),
            "p90": round(float(np.percentile(cold_us, 90)), 2)},
        "step_eager_us": round(step_eager_us, 2),
        "step_graph_us": round(graph_us, 2),
        "step_two_calls_us": round(step_two_us, 2),
        "graph_replay_equals_eager": replay_equal,
        "read_probe": {"bytes": probe_bytes, "us": round(probe_us, 2),
                       "gbps": round(probe_gbps, 1)},
        "kv_cache": {"packed_bytes": cache_bytes, "bf16_bytes": bf16_kv,
                     "reduction_vs_bf16": round(1 - cache_bytes / bf16_kv, 4),
                     "reduction_vs_fp16": round(1 - cache_bytes / fp16_kv, 4)},
        "append_encode_us": round(enc_us, 2) if enc_us else None,
        "bulk_encode": {"tokens": n_bulk, "us": round(bulk_us, 1), "bytes_in": bulk_in,
                        "bytes_out": bulk_out,
                        "gbps": round((bulk_in + bulk_out) / bulk_us / 1e3, 1),
                        "frac_of_hbm_peak": round((bulk_in + bulk_out) / bulk_us / 1e3 /
                                                  HBM_PEAK_GBPS, 4)},
        "single_token_step": single,
        "algorithmic_bytes_per_decode": alg_bytes,
        "dense_bf16": dense,
        "prefill": prefill,
        "affine": affine,
        "other_workloads": others,
        "other_formats_same_context": formats,
        "valu_decode_kernel": valu,
        "accuracy": accuracy,
        "source_hash": source_hash(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
