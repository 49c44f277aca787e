"""Precision of the QK stage: the forward's bf16 path against the scaled fp8
MFMA with the q hi/lo split that the FlyDSL page builds its QK on (module
docstring, "QK:"), measured through sparse_mla_qk_probe against fp64 scores.

Two record sets of 2,048 records each, made by the workload recipes: latent
N(0, 1) (the decode workloads) and latent N(0, 4) with 1 % of values +-1000
(the ragged workload).  q: 16 heads of bf16 N(0, 1).  The figure that
matters for parity is the logit error sigma * |s_gpu - s_exact| (sigma =
1/sqrt(576)): lse moves by at most the largest logit error, and lse must stay
within 1e-3.

Modes (see include/smla.h): 0 the forward's path (K decoded exactly to bf16,
bf16 MFMA); 1 the scaled fp8 MFMA with q = s (hi + lo / 32); 2 hi only; 3 q =
s (hi + lo / 16).  Modes 2 and 3 are also compared with fp64 scores of their
own quantised q, which isolates the MFMA's accumulation from the rounding of
q.  The test pins what the choice of the bf16 path rests on; it prints every
figure.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
SIGMA = float(np.float32(1.0 / np.sqrt(576.0)))
LSE_TOL = 1e-3
N = 2048


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def record_set(name):
    kw = dict(latent_std=2.0, outlier_p=0.01, outlier_mag=1000.0) if name == "outliers" else {}
    return synth.build_workload(f"qk_{name}", 1, 16, N, lambda g, r, m: np.arange(N), seed=91,
                                device="cuda", **kw)


def quantised_q(qf: np.ndarray, lo_factor):
    """q [16, 576] f64 -> the q the hi/lo split represents (latent dims; rope
    unchanged): per head and 128-dim block, s = the smallest power of two with
    amax / s <= 448, hi = e4m3(q / s), lo = e4m3(f (q / s - hi)), q' = s (hi +
    lo / f); lo_factor None: hi only.  e4m3 rounding by torch's float8_e4m3fn
    cast (round to nearest even)."""
    out = qf.copy()
    for h in range(16):
        for b in range(4):
            x = qf[h, 128 * b:128 * (b + 1)]
            amax = np.abs(x).max()
            m, e = np.frexp(amax / 448.0)
            s = np.ldexp(1.0, int(e) - (1 if m == 0.5 else 0)) if amax > 0 else 1.0
            y = x / s
            hi = torch.from_numpy(y).to(torch.float8_e4m3fn).double().numpy()
            val = hi
            if lo_factor is not None:
                lo = torch.from_numpy(lo_factor * (y - hi)).to(torch.float8_e4m3fn).double().numpy()
                val = hi + lo / lo_factor
            out[h, 128 * b:128 * (b + 1)] = s * val
    return out


@pytest.fixture(scope="module")
def measured():
    from sparse_mla_decode_fp8_amd import binding as b
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    res = {}
    for name in ("normal", "outliers"):
        w = record_set(name)
        K = oracle.decode_records(w.kv.cpu().numpy())                        # [N, 576] f64
        qb = w.q[0].contiguous()
        Qf = oracle.bf16_bits_to_f64(qb.cpu().view(torch.int16).numpy().view(np.uint16))   # [16, 576]
        exact = K @ Qf.T
        absdot = np.abs(K) @ np.abs(Qf).T                                     # sum |k_i q_i|
        rows = torch.arange(N, dtype=torch.int32, device=DEV)
        for mode in (0, 1, 2, 3):
            s = b.qk_probe(qb, w.kv, rows, mode).double().cpu().numpy()
            torch.cuda.synchronize()
            res[(name, mode, "exact")] = SIGMA * np.abs(s - exact).max()
            if mode == 0:
                res[(name, 0, "bound")] = (SIGMA * (np.abs(s - exact) / (576 * 2.0 ** -24 * absdot + 1e-30))).max()
            if mode in (2, 3):
                qq = quantised_q(Qf, None if mode == 2 else 16.0)
                ref = K @ qq.T
                prod = np.abs(K[:, :512]) @ np.abs(qq[:, :512]).T
                res[(name, mode, "own_q")] = SIGMA * np.abs(s - ref).max()
                res[(name, mode, "rel")] = (np.abs(s - ref) / prod).max()
        res[(name, "max_logit")] = SIGMA * np.abs(exact).max()
        for mode in (0, 1, 2, 3):
            note(f"{name}: mode {mode}: max logit error vs exact q {res[(name, mode, 'exact')]:.3e}"
                 + (f"; vs its own quantised q {res[(name, mode, 'own_q')]:.3e}"
                    f" ({res[(name, mode, 'rel')]:.2e} of sum |k q|)" if mode in (2, 3) else "")
                 + f"  (max |logit| {res[(name, 'max_logit')]:.1f})")
    return res


def test_forward_qk_is_f32_accurate(measured):
    # the forward's path: exact bf16 products, f32 accumulation: within the
    # summation bound n u sum |k q| (n = 576, u = 2^-24), and well inside the
    # lse tolerance even where logits reach hundreds
    for name in ("normal", "outliers"):
        assert measured[(name, 0, "bound")] <= 1.0, name
        assert measured[(name, 0, "exact")] <= LSE_TOL / 4, name


def test_page_lo_factor_overflows_e4m3(measured):
    # lo = 32 x the residual: a hi in e4m3's top binade [256, 448] has a step
    # of 32, so its residual reaches 16 and 32 x 16 = 512 is past e4m3's 448;
    # such q elements occur in every set and the conversion gives NaN codes
    for name in ("normal", "outliers"):
        assert not (measured[(name, 1, "exact")] <= LSE_TOL), name  # NaN


def test_scaled_fp8_qk_misses_the_lse_tolerance_on_outliers(measured):
    # with the 16 x residual the split is fine on N(0, 1) records ...
    assert measured[("normal", 3, "exact")] <= LSE_TOL
    # ... but on the outlier records it moves some logit by more than the lse
    # tolerance, which is why the forward keeps the bf16 path
    assert measured[("outliers", 3, "exact")] > LSE_TOL
    # and the cause is the MFMA's accumulation, not the rounding of q: against
    # fp64 scores of the same quantised q the error is the same
    assert measured[("outliers", 3, "own_q")] > LSE_TOL
    assert measured[("outliers", 3, "own_q")] >= 0.9 * measured[("outliers", 3, "exact")]
    # the hi part alone is far off everywhere
    assert measured[("normal", 2, "exact")] > LSE_TOL
