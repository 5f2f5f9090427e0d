"""Accuracy of the method measured on the HIP path's own outputs.

* Score bias with and without the QJL residual sketch (mlx-turboquant README,
  "The 1-bit QJL residual (unbiased inner-product estimator)": the MSE-only
  inner product is biased, the sketch removes the bias in expectation). With a
  context of two tokens the decode output is o = p0 v0 + (1 - p0) v1 with the
  dequantized values v0, v1, so o reveals p0 and with it the score difference
  s0 - s1 that the kernel used. Queries are the correlated-query recipe
  (q = 0.8 k_j + 0.6 eps), so s_j - s_other carries the bias of the
  correlated pair. Per pair, the GPU's recovered difference must equal the
  oracle's (the same recovery applied to the oracle's attention output); over
  all pairs, the QJL-corrected mean bias must be smaller in magnitude than
  the MSE-only one, and the MSE-only bias must be negative (the quantized key
  is shorter along the query's direction).
* The decode output's error against unquantized fp64 attention
  softmax(q K^T / sqrt(d)) V per bit width, with and without the sketch
  (README, "Measured results": rotated 4-bit KV stays close to unquantized
  attention). This is reported, not asserted, apart from a sanity ordering
  (more bits, smaller error).
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle as o
import seeded_inputs as si
from gpu_helpers import (config_of, gpu_decode, gpu_encode, kv_host, log, oracle_encode,
                         to_device, torch_cuda)

pytestmark = pytest.mark.gpu


def _log_odds(out, v0, v1):
    """p0 of o = p0 v0 + (1 - p0) v1 by least squares, as log(p0 / (1 - p0))."""
    dv = v0 - v1
    p0 = ((out - v1) * dv).sum(-1) / (dv * dv).sum(-1)
    p0 = np.clip(p0, 1e-9, 1 - 1e-9)
    return np.log(p0 / (1 - p0))


def _pair_workload(qjl: bool):
    return si.small_workload(B=64, Hq=32, Hkv=8, d=128, N=2, bits_k=3, bits_v=4,
                             norm_dtype="f16", qjl=qjl, in_dtype="bf16",
                             structure="correlated", wid=300)


def _pair_log_odds(w, scale):
    """(GPU log-odds, oracle log-odds, exact log-odds, correlated token j),
    all oriented towards token j: s_j - s_other."""
    torch_cuda()
    qraw, qf = si.queries(w)
    _, _, fk, fv = kv_host(w, 0, w.N)
    cfg, cache = gpu_encode(w)
    got = gpu_decode(w, cfg, cache, to_device(qraw, w.in_dtype), w.N, scale=scale)
    ref = oracle_encode(w)
    want = o.attend_dense(qf.astype(np.float64), ref, d=w.d, seed=w.seed, bits_k=w.bits_k,
                          bits_v=w.bits_v, Hkv=w.Hkv, scale=scale, qjl=w.qjl,
                          qjl_seed=w.qjl_seed)
    vc = ref["v_enc"]["codes"]
    vhat = o.rht_inverse(o.dequant_rot(vc, ref["vn"], w.bits_v), w.seed)   # [B][Hkv][2][d]
    heads = np.arange(w.Hq) // w.G
    v0, v1 = vhat[:, heads, 0], vhat[:, heads, 1]                       # [B][Hq][d]
    lg, lo = _log_odds(got, v0, v1), _log_odds(want, v0, v1)
    q = qf.astype(np.float64)
    s = scale * np.einsum("bhd,bhtd->bht", q, fk[:, heads])             # exact scores
    lt = s[..., 0] - s[..., 1]
    j = si.correlated_tokens(w)
    sign = np.where(j == 0, 1.0, -1.0)
    return lg * sign, lo * sign, lt * sign


def test_qjl_removes_the_score_bias_on_gpu_outputs():
    scale = 1.0 / 128          # scores of order 1, so both weights are measurable
    res = {}
    for qjl in (False, True):
        w = _pair_workload(qjl)
        lg, lo, lt = _pair_log_odds(w, scale)
        # the kernel's score difference is the oracle's (fp16 operands and
        # weights: a few 1e-3 per pair)
        assert np.abs(lg - lo).max() < 2e-2, np.abs(lg - lo).max()
        res[qjl] = dict(bias_gpu=float((lg - lt).mean()), bias_oracle=float((lo - lt).mean()),
                        sem=float((lg - lt).std() / math.sqrt(lg.size)),
                        mean_true=float(lt.mean()), pairs=int(lg.size))
        assert abs(res[qjl]["bias_gpu"] - res[qjl]["bias_oracle"]) < 2e-3
    mse, q = res[False], res[True]
    log(f"score bias on {mse['pairs']} correlated pairs (log-odds units, scale 1/128, "
        f"mean true difference {mse['mean_true']:.4f}): "
        f"MSE-only {mse['bias_gpu']:+.5f} +- {mse['sem']:.5f} "
        f"(oracle {mse['bias_oracle']:+.5f}), "
        f"with QJL {q['bias_gpu']:+.5f} +- {q['sem']:.5f} (oracle {q['bias_oracle']:+.5f})")
    assert mse["bias_gpu"] < 0
    assert abs(q["bias_gpu"]) < abs(mse["bias_gpu"])


P13_FORMATS = [(2, 2), (3, 3), (4, 4), (3, 4)]


def _exact_attention(qf, fk, fv, G):
    """softmax(q K^T / sqrt(d)) V in float64 from the (rounded) inputs."""
    B, Hq, d = qf.shape
    heads = np.arange(Hq) // G
    q = qf.astype(np.float64)
    s = np.einsum("bhd,bhtd->bht", q, fk[:, heads]) / math.sqrt(d)
    s -= s.max(-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(-1, keepdims=True)
    return np.einsum("bht,bhtd->bhd", p, fv[:, heads])


@pytest.mark.parametrize("structure", ["iid", "correlated"])
def test_decode_error_against_unquantized_attention(structure):
    torch_cuda()
    rows = []
    errs = {}
    for bk, bv in P13_FORMATS:
        for qjl in (False, True):
            w = si.small_workload(B=1, Hq=32, Hkv=8, d=128, N=4096, bits_k=bk, bits_v=bv,
                                  norm_dtype="f16", qjl=qjl, in_dtype="bf16",
                                  structure=structure, wid=301)
            qraw, qf = si.queries(w)
            _, _, fk, fv = kv_host(w, 0, w.N)
            cfg, cache = gpu_encode(w)
            got = gpu_decode(w, cfg, cache, to_device(qraw, w.in_dtype), w.N)
            ref = _exact_attention(qf, fk, fv, w.G)
            e = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
            assert np.isfinite(e).all()
            errs[(bk, bv, qjl)] = float(e.mean())
            rows.append(f"K{bk}{'+QJL' if qjl else ''}/V{bv}: mean {e.mean():.4f} max {e.max():.4f}")
    log(f"relative L2 error of the decode output vs fp64 attention ({structure} queries, "
        f"N=4096, d=128): " + "; ".join(rows))
    for qjl in (False, True):
        assert errs[(4, 4, qjl)] < errs[(3, 3, qjl)] < errs[(2, 2, qjl)]
