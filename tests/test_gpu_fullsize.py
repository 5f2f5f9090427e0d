"""Full-size GPU parity for the five decode workloads, in the launch
configuration bench.py times (default split count; for the long-context
workload bulk encode followed by the 4096-token append).

The oracle cannot redo whole contexts element by element, so it checks
* the packed codes, norms and QJL bits of a random sample of rows, and
* the attention output over the FULL context of every query head of two KV
  heads (the first of batch 0, the last of the last batch), from the
  oracle's own streamed encode of each KV head (blocks of 65536 tokens,
  rotated frame, exact log-sum-exp merge).
Bars as in test_gpu_parity.py."""

import numpy as np
import pytest

import oracle as o
import seeded_inputs as si
from gpu_helpers import TOL, config_of, log, rel_err, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def _encode_full(w):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    cfg = config_of(w)
    k_host = si.kv_full(w, si.T_K)
    v_host = si.kv_full(w, si.T_V)
    K, V = to_device(k_host, w.in_dtype), to_device(v_host, w.in_dtype)
    del k_host, v_host
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    n_bulk = w.N - w.append
    if w.append:
        tq.tq_encode_kv(cfg, K[:, :, :n_bulk].contiguous(), V[:, :, :n_bulk].contiguous(), 0,
                        cache)
        tq.tq_encode_kv(cfg, K[:, :, n_bulk:].contiguous(), V[:, :, n_bulk:].contiguous(),
                        n_bulk, cache)
    else:
        tq.tq_encode_kv(cfg, K, V, 0, cache)
    torch.cuda.synchronize()
    del K, V
    return cfg, cache


def _check_sampled_rows(w, cache, groups=8, per_group=128):
    """Codes/norms/sketch of random rows from a few (b, kv-head, block)
    groups (each block is generated once), including the first and last
    token of the context and, with an append, both sides of its start."""
    torch = torch_cuda()
    rng = np.random.default_rng(w.wid)
    nblk = (w.N + si.BLOCK - 1) // si.BLOCK
    picks = {(0, 0, 0), (w.B - 1, w.Hkv - 1, nblk - 1)}
    while len(picks) < min(groups, w.B * w.Hkv * nblk):
        picks.add((int(rng.integers(0, w.B)), int(rng.integers(0, w.Hkv)),
                   int(rng.integers(0, nblk))))
    bs, hs, ts, fk, fv = [], [], [], [], []
    for b, h, blk in sorted(picks):
        t0, t1 = blk * si.BLOCK, min(w.N, (blk + 1) * si.BLOCK)
        _, k = si.kv_rows(w, si.T_K, b, h, t0, t1)
        _, v = si.kv_rows(w, si.T_V, b, h, t0, t1)
        sel = rng.integers(0, t1 - t0, per_group)
        sel[:2] = [0, t1 - t0 - 1]
        if w.append and t0 <= w.N - w.append < t1:
            sel[2:4] = [w.N - w.append - 1 - t0, w.N - w.append - t0]
        bs += [b] * per_group
        hs += [h] * per_group
        ts += list(t0 + sel)
        fk.append(k[sel])
        fv.append(v[sel])
    fk = np.concatenate(fk).astype(np.float64)
    fv = np.concatenate(fv).astype(np.float64)
    ref = o.encode_kv(fk, fv, seed=w.seed, bits_k=w.bits_k, bits_v=w.bits_v,
                      norm_dtype=w.norm_dtype, qjl=w.qjl, qjl_seed=w.qjl_seed)
    idx = tuple(torch.as_tensor(np.asarray(x, dtype=np.int64), device="cuda")
                for x in (bs, hs, ts))
    counts = {}
    for side, bits in (("k", w.bits_k), ("v", w.bits_v)):
        enc = ref[f"{side}_enc"]
        got = o.unpack_codes(getattr(cache, f"{side}c")[idx].cpu().numpy(), bits, w.d)
        _, thr = o.lloyd_max(bits)
        bnd = o.boundary_mask(enc["z"], thr)
        assert not ((got != enc["codes"]) & ~bnd).any(), f"{side} codes differ"
        gn = getattr(cache, f"{side}n")[idx].float().cpu().numpy().astype(np.float64)
        amb = o.norm_ambiguous(enc["norm_exact"], w.norm_dtype)
        assert not ((gn != enc["norm"]) & ~amb).any(), f"{side} norms differ"
        counts[side] = int(bnd.sum())
    if w.qjl:
        sk = ref["k_qjl"]
        got = o.unpack_signs(cache.kq[idx].cpu().numpy(), w.d)
        bnd = o.qjl_boundary_mask(sk["w"], sk["rnorm_exact"])
        assert not ((got != sk["bits"]) & ~bnd).any(), "qjl bits differ"
        gr = cache.kr[idx].float().cpu().numpy().astype(np.float64)
        amb = o.norm_ambiguous(sk["rnorm_exact"], "f16")
        assert not ((gr != sk["rnorm"]) & ~amb).any(), "qjl norms differ"
    return counts


def _oracle_heads(w, qf, heads):
    """Oracle attention of the query heads [(b, h)] over the full context
    (one streamed pass per KV head)."""

    def block(bb, gg, t0, t1):
        _, fk = si.kv_rows(w, si.T_K, bb, gg, t0, t1)
        _, fv = si.kv_rows(w, si.T_V, bb, gg, t0, t1)
        ek = o.encode_vectors(fk.astype(np.float64), w.seed, w.bits_k, w.norm_dtype)
        ev = o.encode_vectors(fv.astype(np.float64), w.seed, w.bits_v, w.norm_dtype)
        blk = {"kcodes": ek["codes"], "kn": ek["norm"], "vcodes": ev["codes"], "vn": ev["norm"]}
        if w.qjl:
            sk = o.qjl_from_encoding(ek, w.bits_k, w.qjl_seed)
            blk["ksig"] = sk["bits"]
            blk["kr"] = sk["rnorm"]
        return blk

    return o.attend_rotated_blocked(qf.astype(np.float64), block, w.N, B=w.B, Hq=w.Hq,
                                    Hkv=w.Hkv, d=w.d, seed=w.seed, bits_k=w.bits_k,
                                    bits_v=w.bits_v, qjl=w.qjl, qjl_seed=w.qjl_seed,
                                    heads=heads)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_full_size_workload(wid):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.WORKLOADS[wid]
    log(f"workload {wid}: {w.name}")
    cfg, cache = _encode_full(w)
    counts = _check_sampled_rows(w, cache)
    log(f"  sampled rows: codes/norms exact off boundaries; boundary coords {counts}")
    qraw, qf = si.queries(w)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))
    tq.tq_attend_decode(cfg, to_device(qraw, w.in_dtype), cache, w.N, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    # every query head of KV head 0 of batch 0 and of the last KV head of the
    # last batch (one oracle pass per KV head)
    heads = sorted({(0, h) for h in range(w.G)} |
                   {(w.B - 1, h) for h in range(w.Hq - w.G, w.Hq)})
    want = _oracle_heads(w, qf, heads)
    worst = 0.0
    for b, h in heads:
        err, _ = rel_err(got[b, h][None], want[b, h][None])
        log(f"  head (b={b}, h={h}): max relative error {err:.3e}")
        worst = max(worst, err)
    assert worst <= TOL


@pytest.mark.timeout(300)
def test_full_size_prefill_sampled_rows():
    """The causal prefill bench.py times: the 4096 appended tokens of the
    long-context workload attend over its 524288-token cache. Sampled query
    rows (chunk start, middle and end) against the oracle's streamed attention over each
    row's own prefix. Every query head of KV head 0 and of the last KV head
    at each sampled row."""
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.WORKLOADS[4]
    n_q = w.append
    log(f"prefill: {n_q} chunk tokens over {w.name}")
    cfg, cache = _encode_full(w)
    qraw, qf = si.chunk_queries(w, n_q)
    out = torch.empty((w.B, w.Hq, n_q, w.d), dtype=torch.float32, device="cuda")
    tq.tq_attend_prefill(cfg, to_device(qraw, w.in_dtype), cache, w.N, out)
    torch.cuda.synchronize()
    memo = {}

    def block(bb, gg, t0, t1):
        base = t0 - t0 % si.BLOCK
        key = (bb, gg, base)
        if key not in memo:
            end = min(w.N, base + si.BLOCK)
            _, fk = si.kv_rows(w, si.T_K, bb, gg, base, end)
            _, fv = si.kv_rows(w, si.T_V, bb, gg, base, end)
            ek = o.encode_vectors(fk.astype(np.float64), w.seed, w.bits_k, w.norm_dtype)
            ev = o.encode_vectors(fv.astype(np.float64), w.seed, w.bits_v, w.norm_dtype)
            memo[key] = {"kcodes": ek["codes"], "kn": ek["norm"], "vcodes": ev["codes"],
                         "vn": ev["norm"]}
        full = memo[key]
        return {k: v[t0 - base:t1 - base] for k, v in full.items()}

    hs_all = list(range(w.G)) + list(range(w.Hq - w.G, w.Hq))
    samples = [(0, hs_all), (n_q // 2 - 1, hs_all), (n_q - 1, hs_all)]
    worst = 0.0
    for i, hs in samples:
        n_ctx = w.N - n_q + i + 1
        want = o.attend_rotated_blocked(qf[:, :, i].astype(np.float64), block, n_ctx, B=w.B,
                                        Hq=w.Hq, Hkv=w.Hkv, d=w.d, seed=w.seed, bits_k=w.bits_k,
                                        bits_v=w.bits_v, heads=[(0, h) for h in hs])
        for h in hs:
            got = out[0, h, i].cpu().numpy().astype(np.float64)
            assert np.isfinite(got).all()
            err, _ = rel_err(got[None], want[0, h][None])
            log(f"  query {i} (position {n_ctx - 1}), head {h}: max relative error {err:.3e}")
            worst = max(worst, err)
    assert worst <= TOL


@pytest.mark.timeout(300)
def test_full_size_chunk_append_step():
    """The long-context step as one call: tq_append_chunk_attend_decode of the
    4096 newest tokens onto the bulk-encoded 520192 (default split count).
    The appended rows are sampled against the oracle, the output of every
    query head of two KV heads against the oracle over the full context, and
    the whole output against tq_attend_decode on the resulting cache."""
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.WORKLOADS[4]
    cfg = config_of(w)
    k_host = si.kv_full(w, si.T_K)
    v_host = si.kv_full(w, si.T_V)
    K, V = to_device(k_host, w.in_dtype), to_device(v_host, w.in_dtype)
    del k_host, v_host
    n_bulk = w.N - w.append
    log(f"chunk step: {w.append} tokens appended onto {n_bulk} ({w.name})")
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_encode_kv(cfg, K[:, :, :n_bulk].contiguous(), V[:, :, :n_bulk].contiguous(), 0, cache)
    kc, vc = K[:, :, n_bulk:].contiguous(), V[:, :, n_bulk:].contiguous()
    del K, V
    qraw, qf = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))
    tq.tq_append_chunk_attend_decode(cfg, kc, vc, q, cache, w.N, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    counts = _check_sampled_rows(w, cache)
    log(f"  sampled rows: codes/norms exact off boundaries; boundary coords {counts}")
    out2 = torch.empty_like(out)
    tq.tq_attend_decode(cfg, q, cache, w.N, out2, ws)
    torch.cuda.synchronize()
    diff, _ = rel_err(got, out2.cpu().numpy().astype(np.float64))
    log(f"  against tq_attend_decode on the same cache: {diff:.2e}")
    assert diff <= TOL
    heads = sorted({(0, h) for h in range(w.G)} |
                   {(w.B - 1, h) for h in range(w.Hq - w.G, w.Hq)})
    want = _oracle_heads(w, qf, heads)
    worst = max(rel_err(got[b, h][None], want[b, h][None])[0] for b, h in heads)
    log(f"  worst head against the oracle: {worst:.3e}")
    assert worst <= TOL
