#!/usr/bin/env python3
"""Decode-step benchmark of the TurboQuant KV-cache path on one MI355X.

One step = append-encode of the newest tokens + one decode-attention step
over the whole packed context (the two calls a generation step makes). The
default workload is the long-context decode: batch 1, 32 query / 8 KV heads,
d = 128, 524288-token context, 3-bit keys / 4-bit values with fp16 norms,
4096 tokens appended per step, bf16 N(0,1) inputs.

Prints ONE JSON line on stdout (progress goes to stderr):
  value     KV-tokens/s of the whole step (B * N / step time)
  roofline  the decode call's algorithmic bytes / its measured duration
            against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle timed on a bounded sample, scaled
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
METRIC = "packed decode-attention KV-tokens/s and achieved HBM GB/s as % of peak"


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


def traffic_from_profile(wid):
    """HBM bytes per decode launch from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"decode_hbm_traffic_workload{wid}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def alg_bytes_of(tq, cfg, w, q):
    """Algorithmic bytes of one decode call: every packed plane over the
    context, the queries in and the fp32 outputs."""
    cache_bytes, _ = tq.tq_cache_bytes(cfg, w.B, w.Hkv, w.N)
    return cache_bytes + q.numel() * q.element_size() + w.B * w.Hq * w.d * 4


def to_dev_bf16(torch, raw):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()


def cpu_baseline(w, sample_tokens):
    """The oracle (NumPy fp64, as it stands) on a bounded sample of the same
    step: the append-encode of the newest tokens for one KV head and the
    decode of that KV head's query heads over `sample_tokens` tokens; both
    scaled linearly to the whole step."""
    import numpy as np
    import oracle as o
    import seeded_inputs as si
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    n = min(sample_tokens, w.N) if sample_tokens > 0 else w.N
    A = min(w.append or 4096, n)
    _, fk = si.kv_rows(w, si.T_K, 0, 0, 0, n)
    _, fv = si.kv_rows(w, si.T_V, 0, 0, 0, n)
    fk = fk.astype(np.float64)[None, None]
    fv = fv.astype(np.float64)[None, None]
    kw = dict(seed=w.seed, bits_k=w.bits_k, bits_v=w.bits_v, norm_dtype=w.norm_dtype,
              qjl=w.qjl, qjl_seed=w.qjl_seed)
    t0 = time.perf_counter()
    cache = o.encode_kv(fk, fv, **kw)                      # setup, untimed
    t_setup = time.perf_counter() - t0
    t0 = time.perf_counter()
    o.encode_kv(fk[:, :, n - A:], fv[:, :, n - A:], **kw)  # the step's append
    t_enc = time.perf_counter() - t0
    _, qf = si.queries(w)
    q = qf[:1, :w.G].astype(np.float64)
    t0 = time.perf_counter()
    o.attend(q, cache, n, d=w.d, seed=w.seed, bits_k=w.bits_k, bits_v=w.bits_v, Hkv=1,
             qjl=w.qjl, qjl_seed=w.qjl_seed)
    t_dec = time.perf_counter() - t0
    units = w.B * w.Hkv
    step_s = t_enc * units * (w.append or A) / A + t_dec * units * w.N / n
    return {
        "value": w.B * w.N / step_s,
        "unit": "KV-tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"1 of {units} KV heads: {A}-token append encode ({t_enc:.2f} s) and "
                   f"decode of {w.G} query heads over {n} of {w.N} tokens ({t_dec:.2f} s), "
                   f"scaled linearly to the full step ({step_s:.1f} s); encoding the "
                   f"sample's cache first took {t_setup:.1f} s (not part of the step)"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-affine", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="context tokens of the CPU-oracle sample (0: the whole context "
                         "of one KV head)")
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

    # ---------------- inputs (seeded, host-generated, uploaded once)
    t0 = time.time()
    k_host = si.kv_full(w, si.T_K)
    v_host = si.kv_full(w, si.T_V)
    q_raw, _ = si.queries(w)
    log(f"generated inputs in {time.time() - t0:.1f} s")
    if w.in_dtype == "bf16":
        K, V, q = to_dev_bf16(torch, k_host), to_dev_bf16(torch, v_host), to_dev_bf16(torch, q_raw)
    else:
        K = torch.from_numpy(k_host).cuda()
        V = torch.from_numpy(v_host).cuda()
        q = torch.from_numpy(q_raw).cuda()
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

    ev = lambda: torch.cuda.Event(enable_timing=True)
    # one-token encode first, so the timed bulk encode excludes code-object
    # loading and the host's one-time codebook set-up
    tq.tq_encode_kv(cfg, k_bulk[:, :, :1].contiguous(), v_bulk[:, :, :1].contiguous(), 0, cache)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    tq.tq_encode_kv(cfg, k_bulk, v_bulk, 0, cache)
    e1.record()
    torch.cuda.synchronize()
    bulk_ms = e0.elapsed_time(e1)
    del k_bulk, v_bulk
    log(f"bulk encode of {n_bulk} tokens x {w.B * w.Hkv} heads: {bulk_ms:.3f} ms")

    def step(dec_events=None):
        if A:
            tq.tq_encode_kv(cfg, k_app, v_app, n_bulk, cache)
        if dec_events:
            dec_events[0].record()
        tq.tq_attend_decode(cfg, q, cache, w.N, out, ws)
        if dec_events:
            dec_events[1].record()

    if args.copy_probe_mb:
        src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {args.copy_probe_mb} MiB read + written")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; timing {args.steps} steps")

    dec_ev = [(ev(), ev()) for _ in range(args.steps)]
    s0, s1 = ev(), ev()
    torch.cuda.synchronize()
    s0.record()
    for i in range(args.steps):
        step(dec_ev[i])
    s1.record()
    torch.cuda.synchronize()
    total_ms = s0.elapsed_time(s1)
    ms_per_step = total_ms / args.steps
    dec_us = [a.elapsed_time(b) * 1e3 for a, b in dec_ev]
    dec_avg_us = float(np.mean(dec_us))
    log(f"step {ms_per_step * 1e3:.1f} us; decode call avg {dec_avg_us:.1f} us "
        f"(p10 {np.percentile(dec_us, 10):.1f}, p90 {np.percentile(dec_us, 90):.1f})")

    # streaming-read probe over as many bytes as one decode call reads, and
    # decode calls after a 1 GiB read has evicted the 256 MB last-level cache
    probe_bytes = (alg_bytes_of(tq, cfg, w, q) + 15) // 16 * 16
    pbuf = torch.empty(probe_bytes, dtype=torch.uint8, device="cuda")
    sink = tq.tq_read_probe(pbuf)
    a, b = ev(), ev()
    torch.cuda.synchronize()
    a.record()
    for _ in range(20):
        tq.tq_read_probe(pbuf, sink)
    b.record()
    torch.cuda.synchronize()
    probe_us = a.elapsed_time(b) * 1e3 / 20
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
    del flush
    log(f"read probe {probe_bytes / probe_us / 1e3:.1f} GB/s over {probe_bytes} B; cold decode "
        f"median {np.median(cold_us):.1f} us")

    # append-encode alone
    enc_us = None
    if A:
        a, b = ev(), ev()
        a.record()
        for _ in range(20):
            tq.tq_encode_kv(cfg, k_app, v_app, n_bulk, cache)
        b.record()
        torch.cuda.synchronize()
        enc_us = a.elapsed_time(b) * 1e3 / 20

    # single-token generation step (append token N-1, attend over N): the
    # fused entry point against the two calls it replaces, on the same cache
    k1, v1 = K[:, :, w.N - 1:].contiguous(), V[:, :, w.N - 1:].contiguous()

    def time_calls(fn, n=20):
        for _ in range(3):
            fn()
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    def two_calls():
        tq.tq_encode_kv(cfg, k1, v1, w.N - 1, cache)
        tq.tq_attend_decode(cfg, q, cache, w.N, out, ws)

    single = {
        "two_calls_us": round(time_calls(two_calls), 2),
        "fused_us": round(time_calls(
            lambda: tq.tq_append_attend_decode(cfg, k1, v1, q, cache, w.N, out, ws)), 2),
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
        qc = to_dev_bf16(torch, qc_raw) if w.in_dtype == "bf16" else \
            torch.from_numpy(qc_raw).cuda()
        pout = torch.empty((w.B, w.Hq, nq, w.d), dtype=torch.float32, device="cuda")
        tq.tq_attend_prefill(cfg, qc, cache, w.N, pout)
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for _ in range(3):
            tq.tq_attend_prefill(cfg, qc, cache, w.N, pout)
        b.record()
        torch.cuda.synchronize()
        pms = a.elapsed_time(b) / 3
        visible = nq * (w.N - nq) + nq * (nq + 1) // 2
        flops = 4 * w.d * w.B * w.Hq * visible
        prefill = {"chunk_tokens": nq, "context": w.N, "ms": round(pms, 3),
                   "tflops": round(flops / (pms * 1e-3) / 1e12, 1),
                   "frac_of_fp16_dense_peak": round(flops / (pms * 1e-3) / 2.5e15, 4),
                   "flops": flops}
        del qc, pout
        log(f"prefill of {nq} tokens over {w.N}: {pms:.2f} ms, {prefill['tflops']} TFLOP/s")

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
        for _ in range(3):
            tq.tq_affine_attend_decode(acfg, q, acache, w.N, aout, aws)
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for _ in range(20):
            tq.tq_affine_attend_decode(acfg, q, acache, w.N, aout, aws)
        b.record()
        torch.cuda.synchronize()
        aus = a.elapsed_time(b) / 20 * 1e3
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

    # algorithmic bytes of one decode call: every packed plane over N tokens,
    # plus q in and out
    alg_bytes = alg_bytes_of(tq, cfg, w, q)
    qbytes = q.numel() * q.element_size()
    achieved = alg_bytes / (dec_avg_us * 1e-6) / 1e9
    traffic = traffic_from_profile(w.wid)

    # dense bf16 decode on the same GPU (same split-K skeleton, bf16 rows)
    dense = None
    if not args.no_dense and w.in_dtype == "bf16":
        dws = tq.workspace(tq.tq_dense_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N))
        dout = torch.empty_like(out)
        for _ in range(3):
            tq.tq_dense_decode_bf16(q, K, V, dout, dws)
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for _ in range(20):
            tq.tq_dense_decode_bf16(q, K, V, dout, dws)
        b.record()
        torch.cuda.synchronize()
        dus = a.elapsed_time(b) * 1e3 / 20
        dbytes = 2 * K.numel() * 2 + qbytes + out.numel() * 4
        dense = {"decode_us": round(dus, 2), "achieved_gbps": round(dbytes / dus / 1e3, 1),
                 "packed_speedup": round(dus / dec_avg_us, 3)}
        log(f"dense bf16 decode {dus:.1f} us ({dense['achieved_gbps']} GB/s)")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, args.cpu_sample_tokens)
        log(f"oracle: {cpu['value']:.3e} KV-tokens/s ({cpu['sample']})")

    cfg_desc = {
        "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
        "context": w.N, "bits_k": w.bits_k, "bits_v": w.bits_v, "norms": w.norm_dtype,
        "qjl": w.qjl, "append_tokens_per_step": A, "inputs": f"{w.in_dtype} seeded synthetic",
        "splits": splits,
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
        "dtype": "f32",
        "data": "synthetic",
        "config": cfg_desc,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "decode_call_us": round(dec_avg_us, 2),
        "decode_call_percentiles_us": {
            "p10": round(float(np.percentile(dec_us, 10)), 2),
            "median": round(float(np.median(dec_us)), 2),
            "p90": round(float(np.percentile(dec_us, 90)), 2)},
        "decode_call_cold_us": {
            "note": "each call after a 1 GiB streaming read (last-level cache evicted)",
            "p10": round(float(np.percentile(cold_us, 10)), 2),
            "median": round(float(np.median(cold_us)), 2),
            "p90": round(float(np.percentile(cold_us, 90)), 2)},
        "read_probe": {
            "bytes": probe_bytes, "us": round(probe_us, 2),
            "gbps": round(probe_bytes / probe_us / 1e3, 1),
            "decode_frac_of_probe": round(achieved / (probe_bytes / probe_us / 1e3), 4)},
        "decode_kv_tokens_per_s": round(w.B * w.N / (dec_avg_us * 1e-6), 1),
        "append_encode_us": round(enc_us, 2) if enc_us else None,
        "single_token_step": single,
        "bulk_encode_ms": round(bulk_ms, 3),
        "algorithmic_bytes_per_decode": alg_bytes,
        "dense_bf16": dense,
        "prefill": prefill,
        "affine": affine,
        "source_hash": source_hash(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
