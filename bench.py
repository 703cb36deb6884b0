"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs fwd,bwd,decode]
                    [--no-cpu-baseline] [--aux] [--calib-copy]
    python bench.py --write-traffic FETCH_CSV WRITE_CSV

One step runs the whole path once, each leg on its own synthetic workload with
inputs already resident in HBM:

  fwd     causal GQA forward, B1 Hq32 Hkv8 N16384 D128, bf16, LSE saved
  bwd     causal recompute backward, B2 H16 N4096 D128, bf16 (per-row statistics,
          dK/dV key-tile kernel, dQ query-tile kernel; no atomics); O and LSE come
          from fa_fwd on the same inputs before timing
  decode  split-KV decode, 64 sequences x 1 token, Hq32 Hkv8 D128, bf16 cache,
          lengths U[1024, 32768] (seed 0), chunks of 2048 + merge

--aux also times, outside the step: the B4 H16 N2048 D128 forwards (non-causal and
causal), the forward and backward workloads with dropout p = 0.1, the long forward with E4M3
Q and K (and the quantisation passes), the GQA backward at B1 Hq32 Hkv8 N16384 D128 causal, a packed variable-length causal forward (32 sequences of U[256, 4096] rows,
Hq32 Hkv8 D128) and the decode workload read from page pools of 16 and of 256 rows
in random page order through a block table.

Throughput counts only matmul FLOPs over the (query, key) pairs that exist:
4*D per pair for the forward and the decode (QK^T and PV), 10*D per pair for the
backward (five products, one of them the recompute of S).  Decode bandwidth counts
each valid cached K/V byte once plus q and O.

Outside the step (not in `value`), the bench also times the two short forwards,
B4 H16 N2048 D128 bf16 non-causal and causal, and the fp32 forward B1 H2 N256 D64.
That last kernel takes about as long as the binding's host cost per call, so its line
gives the eager time as `eager_ms` and, as `ms`, the GPU time per call of 200 calls
captured into one HIP graph.

Prints one JSON line.  The CPU baseline times the fp64 oracle on bounded samples of
each leg's workload (whole query heads, (batch, head) slices, sequences) on the host
cores and reports the step-level rate those samples imply.  The same oracle results
are compared with the GPU's outputs of one untimed call per leg made after the timed
steps (`parity`: forward O max-abs <= 1e-2 plus half a bf16 ulp of the reference and
LSE <= 1e-3, backward relative L2 <= 2e-2 per tensor and slice, decode as the forward;
the short forwards are checked on two whole (batch, head) slices each); the run exits
with status 3 if any sample fails.  `value` is the credited matmul FLOPs of the three
legs (the decode's Q K^T and P V included, at 4*D per cached key and query head) over
the step time.  `roofline`
describes the forward kernel (the largest share of the step): achieved = credited
FLOPs / mean HIP-event duration of its launch; `traffic` = HBM bytes per launch from
the committed counter summary (FETCH_SIZE and WRITE_SIZE scaled by their readings
for a plain copy), null once the kernel sources no longer match it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import re
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import io_aware_tiled_10_amd as fa  # noqa: E402
from io_aware_tiled_10_amd import inputs  # noqa: E402

METRIC = "attention fwd/bwd TFLOP/s & % bf16 MFMA peak; split-KV decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
DEV = "cuda:0"

FWD_CFG = dict(B=1, Hq=32, Hkv=8, N=16384, D=128, causal=True)
BWD_CFG = dict(B=2, H=16, N=4096, D=128, causal=True)
DEC_CFG = dict(Bs=64, Hq=32, Hkv=8, D=128, lo=1024, hi=32768, split=2048, lmax=32768)
# timed outside the step by default: the short forwards and the fp32 forward
SHORT_CFGS = {"fwd_b4h16n2048_noncausal": dict(B=4, Hq=16, Hkv=16, N=2048, D=128, causal=False),
              "fwd_b4h16n2048_causal": dict(B=4, Hq=16, Hkv=16, N=2048, D=128, causal=True),
              "fwd_f32_b1h2n256d64": dict(B=1, Hq=2, Hkv=2, N=256, D=64, causal=False, dtype="fp32")}
TOL_O, TOL_LSE, TOL_GRAD = 1e-2, 1e-3, 2e-2
# packed variable-length prefill: 32 sequences of U[256, 4096] rows (seed 0), causal GQA
VARLEN_CFG = dict(B=32, lo=256, hi=4096, Hq=32, Hkv=8, D=128, causal=True)
# GQA backward at the long-sequence forward's shape
BWD_GQA_CFG = dict(B=1, Hq=32, Hkv=8, N=16384, D=128, causal=True)
# the decode workload's cache scattered over pages of 16 and of 256 rows, random page order
PAGED_SIZES = (16, 256)

CSRC = os.path.join(ROOT, "io_aware_tiled_10_amd", "csrc")
# sources the forward kernel's machine code depends on
FWD_KERNEL_SRCS = [os.path.join(CSRC, f) for f in ("fa_fwd.hip", "fa_common.h", "fa_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_b1h32kv8n16384d128_causal_hbm_traffic.md")
FWD_GRID_THREADS = 1048576  # workgroups x threads of the timed forward launch (rocprofv3 Grid_Size)
COPY_BYTES = 256 << 20      # the --calib-copy transfer


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pairs(nq: int, nk: int, causal: bool) -> int:
    """Number of (query, key) pairs that exist; causal: j <= i + (nk - nq)."""
    if not causal:
        return nq * nk
    return int(np.clip(np.arange(nq, dtype=np.int64) + (nk - nq) + 1, 0, nk).sum())


def bf16_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x).to(DEV).to(torch.bfloat16)


# ------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------

class FwdLeg:
    def __init__(self, cfg, seed=0):
        self.cfg = cfg
        dt = cfg.get("dtype", "bf16")
        x = inputs.attention_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["N"], cfg["D"], dt, seed)
        self.x = x
        dev = bf16_dev if dt == "bf16" else (lambda a: torch.from_numpy(a).to(DEV))
        self.q, self.k, self.v = dev(x.q), dev(x.k), dev(x.v)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=DEV)
        self.flops = 4 * cfg["D"] * pairs(cfg["N"], cfg["N"], cfg["causal"]) * cfg["B"] * cfg["Hq"]

    def run(self):
        fa.fwd(self.q, self.k, self.v, causal=self.cfg["causal"], out=self.o, lse_out=self.lse)


class BwdLeg:
    def __init__(self, cfg, seed=0):
        self.cfg = cfg
        B, H, N, D = cfg["B"], cfg.get("Hq", cfg.get("H")), cfg["N"], cfg["D"]
        Hkv = cfg.get("Hkv", H)
        x = inputs.attention_inputs(B, H, Hkv, N, N, D, "bf16", seed, with_grad=True)
        self.q, self.k, self.v, self.do = bf16_dev(x.q), bf16_dev(x.k), bf16_dev(x.v), bf16_dev(x.do)
        self.o, self.lse = fa.fwd(self.q, self.k, self.v, causal=cfg["causal"])
        self.grads = (torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v))
        need = fa.binding.bwd_workspace_bytes(self.q, self.k, self.v)
        self.ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        self.flops = 10 * D * pairs(N, N, cfg["causal"]) * B * H

    def run(self):
        fa.bwd(self.q, self.k, self.v, self.o, self.do, self.lse, causal=self.cfg["causal"],
               workspace=self.ws, grads=self.grads)


class DecodeLeg:
    def __init__(self, cfg, seed=0):
        self.cfg = cfg
        d = inputs.decode_inputs(cfg["Bs"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["lo"], cfg["hi"], seed)
        self.lens = d.seq_lens
        shape = (cfg["Bs"], cfg["Hkv"], cfg["lmax"], cfg["D"])
        self.kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        self.vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)

        def fill(s):
            kb, vb = d.kv_bits(s)
            return s, kb, vb

        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
            for s, kb, vb in ex.map(fill, range(cfg["Bs"])):
                L = int(self.lens[s])
                self.kc[s, :, :L] = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV)
                self.vc[s, :, :L] = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV)
        self.q = bf16_dev(d.q)
        self.sl = torch.tensor(self.lens, dtype=torch.int32, device=DEV)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device=DEV)
        a = fa.binding.decode_args(self.q, self.kc, self.vc, self.sl, self.o, self.lse, cfg["lmax"],
                                   cfg["split"], None)
        import ctypes
        self.ws = torch.empty(fa.lib().fa_decode_workspace_bytes(ctypes.byref(a)), dtype=torch.uint8,
                              device=DEV)
        tot = int(self.lens.sum())
        D, Hq, Hkv = cfg["D"], cfg["Hq"], cfg["Hkv"]
        self.flops = 4 * D * tot * Hq
        self.bytes = 2 * Hkv * D * 2 * tot + cfg["Bs"] * Hq * D * 2 * 2 + cfg["Bs"] * Hq * 4

    def run(self):
        fa.decode(self.q, self.kc, self.vc, self.sl, max_len=self.cfg["lmax"], split_len=self.cfg["split"],
                  workspace=self.ws, out=self.o, lse_out=self.lse)


class FwdFp8Leg:
    """The long causal GQA forward with Q and K quantised to E4M3 (per-64-row steps)."""

    def __init__(self, cfg, seed=0):
        self.cfg = cfg
        x = inputs.attention_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["N"], cfg["D"], "bf16", seed)
        self.q, self.k, self.v = bf16_dev(x.q), bf16_dev(x.k), bf16_dev(x.v)
        self.q8, self.qs = fa.quantize_fp8(self.q)
        self.k8, self.ks = fa.quantize_fp8(self.k)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=DEV)
        self.flops = 4 * cfg["D"] * pairs(cfg["N"], cfg["N"], cfg["causal"]) * cfg["B"] * cfg["Hq"]

    def run(self):
        fa.fwd_fp8(self.q8, self.qs, self.k8, self.ks, self.v, causal=self.cfg["causal"], out=self.o,
                   lse_out=self.lse)

    def quantize(self):
        fa.quantize_fp8(self.q, out=self.q8, scales_out=self.qs)
        fa.quantize_fp8(self.k, out=self.k8, scales_out=self.ks)


class DropoutLegs:
    """The forward and backward workloads with dropout p = 0.1 on P (Philox mask)."""
    P_DROP, SEED = 0.1, 0x5EED

    def __init__(self, fwd: FwdLeg, bwd: BwdLeg):
        self.f, self.b = fwd, bwd
        self.o, self.lse = fa.fwd_dropout(bwd.q, bwd.k, bwd.v, self.P_DROP, self.SEED, causal=bwd.cfg["causal"])

    def run_fwd(self):
        f = self.f
        fa.fwd_dropout(f.q, f.k, f.v, self.P_DROP, self.SEED, causal=f.cfg["causal"], out=f.o, lse_out=f.lse)

    def run_bwd(self):
        b = self.b
        fa.bwd_dropout(b.q, b.k, b.v, self.o, b.do, self.lse, self.P_DROP, self.SEED, causal=b.cfg["causal"],
                       workspace=b.ws, grads=b.grads)


class DecodePagedLeg:
    """The decode workload read through a block table from a randomly ordered page pool."""

    def __init__(self, dec: DecodeLeg, page: int, seed=0):
        self.dec = dec
        self.kp, self.vp, self.table = inputs.paged_pools_torch(dec.kc, dec.vc, dec.lens, page, seed)
        self.max_len = int(dec.lens.max())
        a = fa.binding.decode_paged_args(dec.q, self.kp, self.vp, self.table, dec.sl, dec.o, dec.lse,
                                         page, self.max_len, dec.cfg["split"], None)
        import ctypes
        self.ws = torch.empty(fa.lib().fa_decode_paged_workspace_bytes(ctypes.byref(a)),
                              dtype=torch.uint8, device=DEV)
        self.flops = dec.flops
        # cached K/V once, q, O, LSE, plus the block-table entries that are read
        self.bytes = dec.bytes + 4 * sum((int(L) + page - 1) // page for L in dec.lens)

    def run(self):
        d = self.dec
        fa.decode_paged(d.q, self.kp, self.vp, self.table, d.sl, max_len=self.max_len,
                        split_len=d.cfg["split"], workspace=self.ws, out=d.o, lse_out=d.lse)


class FwdVarlenLeg:
    """Packed variable-length causal forward (prefill of a ragged batch)."""

    def __init__(self, cfg, seed=0):
        self.cfg = cfg
        lens = [int(x) for x in inputs.ragged_lengths(cfg["B"], cfg["lo"], cfg["hi"], seed)]
        x = inputs.varlen_inputs(lens, lens, cfg["Hq"], cfg["Hkv"], cfg["D"], "bf16", seed)
        self.q, self.k, self.v = bf16_dev(x.q), bf16_dev(x.k), bf16_dev(x.v)
        self.cu = torch.from_numpy(x.cu_q).to(DEV)
        self.max_len = max(lens)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((cfg["Hq"], self.q.shape[0]), dtype=torch.float32, device=DEV)
        self.flops = 4 * cfg["D"] * cfg["Hq"] * sum(pairs(n, n, cfg["causal"]) for n in lens)
        self.tokens = sum(lens)

    def run(self):
        fa.fwd_varlen(self.q, self.k, self.v, self.cu, self.cu, self.max_len, causal=self.cfg["causal"],
                      out=self.o, lse_out=self.lse)


def time_graph(leg, reps=200):
    """Mean GPU time of one call of `leg` with the host's launch cost removed: `reps` calls
    captured into one HIP graph (the entry points launch kernels only), replayed once after
    a warm-up replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first calls outside the capture
        for _ in range(3):
            leg.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            leg.run()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / reps


def time_aux(leg, stream, reps=20):
    for _ in range(3):
        leg.run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        leg.run()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


# ------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on bounded samples of each leg's workload
# ------------------------------------------------------------------------------------

def _host_cpu():
    """Host threads the oracle's BLAS uses, cores this process may run on, CPU model."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except OSError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    model = ""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = {}
        for ln in out.splitlines():
            if ":" in ln:
                k, v = ln.split(":", 1)
                f.setdefault(k.strip(), v.strip())
        model = f.get("Model name", "")
        # a virtualised host may report only the vendor line: add the CPUID family, model
        # and stepping, which name the part
        ids = [f"{k.lower()} {f[k]}" for k in ("CPU family", "Model", "Stepping") if f.get(k)]
        if model and ids:
            model = f"{model} ({', '.join(ids)})"
    except Exception:  # pragma: no cover
        pass
    if not model:
        try:
            for ln in open("/proc/cpuinfo"):
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
        except OSError:  # pragma: no cover
            pass
    return int(blas), int(affinity), model


def _half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 2.0 ** -134)


class _Parity:
    """Running worst errors of one leg's samples against the oracle."""

    def __init__(self, kind: str):
        self.kind, self.n, self.ok = kind, 0, True
        self.worst = {}

    def _max(self, k, v):
        self.worst[k] = max(self.worst.get(k, 0.0), float(v))

    def fwd(self, o, lse, o_ref, lse_ref, o_bf16: bool):
        self.n += 1
        finite = bool(np.all(np.isfinite(o)))
        err = np.abs(o - o_ref)
        excess = float((err - (TOL_O + (_half_ulp_bf16(o_ref) if o_bf16 else 0.0))).max())
        # a row with no visible key has LSE -inf on both sides; -inf must meet -inf
        lse, lse_ref = np.asarray(lse, np.float64), np.asarray(lse_ref, np.float64)
        both = np.isneginf(lse) & np.isneginf(lse_ref)
        finite &= bool(np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)) and np.all(np.isfinite(lse[~both])))
        diff = np.zeros_like(lse)
        diff[~both] = lse[~both] - lse_ref[~both]
        el = float(np.abs(diff).max()) if lse.size else 0.0
        self._max("o_max_abs", err.max())
        self._max("lse_max_abs", el)
        self.worst["o_bound_excess"] = max(self.worst.get("o_bound_excess", -1.0), excess)
        self.ok &= finite and excess <= 0 and el <= TOL_LSE

    def grads(self, got, ref):
        self.n += 1
        for nm, g, r in zip(("dq", "dk", "dv"), got, ref):
            g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
            e = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
            self._max(f"{nm}_rel_l2", e)
            self.ok &= bool(np.all(np.isfinite(g))) and e <= TOL_GRAD

    def record(self, samples: str):
        return {"samples": samples, "checked": self.n,
                **{k: float(f"{v:.4g}") for k, v in self.worst.items()}, "pass": bool(self.ok and self.n > 0)}


def cpu_baseline(gpu=None, budgets=(9.0, 4.0, 3.0)):
    """The fp64 oracle timed on the host cores, leg by leg, on bounded samples of the
    step's own workloads: whole query heads of the forward, whole (batch, head) slices
    of the backward, whole sequences of the decode (each until its time budget in
    seconds runs out; input generation is not timed).  `value` is the step's credited
    FLOPs over the time the oracle would take for the whole step at those rates.

    ``gpu``: host copies of the GPU's outputs for the same workloads (one untimed call
    per leg after the timed steps); each oracle result is then also compared with them
    (outside the timed calls).  Returns (baseline record, parity record or None)."""
    import oracle

    rates, samples = {}, {}
    par = {k: _Parity(k) for k in ("fwd", "bwd", "decode")} if gpu is not None else None
    # forward: query heads of B1 Hq32 Hkv8 N16384 D128 causal
    cfg = FWD_CFG
    x = inputs.attention_inputs(1, cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["N"], cfg["D"], "bf16", 0)
    G = cfg["Hq"] // cfg["Hkv"]
    per_head = 4 * cfg["D"] * pairs(cfg["N"], cfg["N"], cfg["causal"])
    step_flops = {"fwd": per_head * cfg["Hq"]}
    done, el = 0, 0.0
    # heads spread over the KV groups: 0, 31, 9, 22, ... (every group within the first 8)
    order = [0, 31, 9, 22, 5, 18, 27, 14] + [h for h in range(32) if h not in (0, 31, 9, 22, 5, 18, 27, 14)]
    while done < cfg["Hq"] and el < budgets[0]:
        h = order[done]
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attn_fwd(x.q[:, h:h + 1], x.k[:, h // G:h // G + 1], x.v[:, h // G:h // G + 1],
                                         None, True)
        el += time.perf_counter() - t0
        done += 1
        if par is not None:
            par["fwd"].fwd(gpu["fwd_o"][:, h:h + 1], gpu["fwd_lse"][:, h:h + 1], o_ref, lse_ref, True)
    rates["fwd"] = per_head * done / el
    samples["fwd"] = f"{done} of 32 query heads, all rows ({done * per_head / 1e9:.1f} GFLOP, {el:.1f} s)"
    del x
    # backward: (batch, head) slices of B2 H16 N4096 D128 causal
    cfg = BWD_CFG
    B, H, N, D = cfg["B"], cfg["H"], cfg["N"], cfg["D"]
    x = inputs.attention_inputs(B, H, H, N, N, D, "bf16", 0, with_grad=True)
    per_head = 10 * D * pairs(N, N, cfg["causal"])
    step_flops["bwd"] = per_head * B * H
    done, el = 0, 0.0
    while done < B * H and el < budgets[1]:
        b, h = divmod((13 * done) % (B * H), H)  # a fixed permutation of the slices
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        ref = oracle.attn_bwd(x.q[sl], x.k[sl], x.v[sl], x.do[sl], None, True)
        el += time.perf_counter() - t0
        done += 1
        if par is not None:
            par["bwd"].grads([gpu[f"bwd_{n}"][sl] for n in ("dq", "dk", "dv")], ref[:3])
    rates["bwd"] = per_head * done / el
    samples["bwd"] = f"{done} of {B * H} (batch, head) slices ({done * per_head / 1e9:.1f} GFLOP, {el:.1f} s)"
    del x
    # decode: whole sequences of the 64-sequence workload
    cfg = DEC_CFG
    d = inputs.decode_inputs(cfg["Bs"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["lo"], cfg["hi"], 0)
    fl_per_key = 4 * cfg["D"] * cfg["Hq"]
    step_flops["decode"] = fl_per_key * int(d.seq_lens.sum())
    done, keys, el = 0, 0, 0.0
    while done < cfg["Bs"] and el < budgets[2]:
        k, v = d.kv(done)
        L = int(d.seq_lens[done])
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attn_decode(d.q[done:done + 1], k[None], v[None], [L])
        el += time.perf_counter() - t0
        if par is not None:
            par["decode"].fwd(gpu["dec_o"][done:done + 1], gpu["dec_lse"][done:done + 1], o_ref, lse_ref, True)
        done, keys = done + 1, keys + L
    rates["decode"] = fl_per_key * keys / el
    samples["decode"] = (f"{done} of 64 sequences ({keys} cached positions, "
                         f"{2 * cfg['Hkv'] * cfg['D'] * 2 * keys / el / 1e9:.2f} GB/s of K/V, {el:.1f} s)")

    blas, affinity, cpu_model = _host_cpu()
    t_step = sum(step_flops[k] / rates[k] for k in step_flops)
    base = {"value": round(sum(step_flops.values()) / t_step / 1e12, 6), "unit": "TFLOP/s",
            "cores": blas, "kind": "oracle", "blas_threads": blas, "affinity_cores": affinity,
            "cpu_model": cpu_model,
            "legs_tflops": {k: round(r / 1e12, 6) for k, r in rates.items()},
            "est_s_per_step": round(t_step, 1),
            "sample": "fp64 numpy oracle on the step's workloads, timed per leg on bounded samples: "
                      + "; ".join(f"{k}: {v}" for k, v in samples.items())}
    parity = None
    if par is not None:
        parity = {k: par[k].record(samples[k]) for k in par}
        if "short" in gpu:
            ps = _Parity("short")
            for name, (leg, o, lse) in gpu["short"].items():
                cfg = leg.cfg
                for b, h in ((0, 0), (cfg["B"] - 1, cfg["Hq"] - 1)):
                    sl = (slice(b, b + 1), slice(h, h + 1))
                    o_ref, lse_ref = oracle.attn_fwd(leg.x.q[sl], leg.x.k[sl], leg.x.v[sl], None, cfg["causal"])
                    ps.fwd(o[sl], lse[sl], o_ref, lse_ref, cfg.get("dtype", "bf16") == "bf16")
            parity["short_fwd"] = ps.record("two whole (batch, head) slices of each of " + ", ".join(gpu["short"]))
        parity["tolerances"] = {"o_max_abs": f"{TOL_O} (+ half a bf16 ulp of the reference for bf16 O)",
                                "lse_max_abs": TOL_LSE, "grad_rel_l2": TOL_GRAD}
        parity["pass"] = all(v["pass"] for k, v in parity.items() if isinstance(v, dict) and "pass" in v)
    return base, parity


def mfma_ceiling(pattern: int, seconds: float = 1.0) -> float:
    """TFLOP/s of libfa_ceiling's register-resident bf16 MFMA loop (the forward's
    occupancy: 8-wave workgroups, one per compute unit, four launches per timing)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "io_aware_tiled_10_amd", "libfa_ceiling.so"))
    lib.fa_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_ceiling_mfma_flops.restype = ctypes.c_double
    lib.fa_ceiling_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    wgs = torch.cuda.get_device_properties(DEV).multi_processor_count
    out = torch.empty(wgs * 512, dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream

    def run(iters, n=1):
        for _ in range(n):
            if lib.fa_ceiling_mfma(ctypes.c_void_p(out.data_ptr()), wgs, iters, pattern, ctypes.c_void_p(stream)):
                raise RuntimeError("fa_ceiling_mfma failed")

    def timed(iters, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        run(iters, n)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    iters = 2000
    run(iters)
    t = timed(iters, 1)
    iters = max(1, int(iters * seconds / 4 / max(t, 1e-6)))  # four launches of ~seconds / 4
    run(iters)
    t = timed(iters, 4)
    return 4 * lib.fa_ceiling_mfma_flops(wgs, iters) / t / 1e12


def stream_ceiling(gib: int = 4, wgs_per_cu: int = 4) -> float:
    """GB/s of libfa_ceiling's plain streaming read of `gib` GiB (each byte read once,
    16-byte non-temporal loads, eight in flight per thread): the HBM read rate a kernel
    that reads its bytes once, as the decode does, can reach."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "io_aware_tiled_10_amd", "libfa_ceiling.so"))
    lib.fa_ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    wgs = wgs_per_cu * torch.cuda.get_device_properties(DEV).multi_processor_count
    nbytes = ((gib << 30) // (32768 * wgs)) * 32768 * wgs
    src = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.empty(wgs * 256, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        if lib.fa_ceiling_stream(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()), wgs,
                                 ctypes.c_void_p(stream)):
            raise RuntimeError("fa_ceiling_stream failed")

    for _ in range(2):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        run()
    e1.record()
    torch.cuda.synchronize()
    del src, out
    return nbytes / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9


def ceilings():
    """Achievable rates on this GPU for the same data statistics, for context: the
    matrix cores alone on register-resident operands (random-like and all-ones), a
    library bf16 GEMM (hipBLASLt via torch.matmul, 8192^3) on N(0,1) data and on all-ones
    data (the sustained clock depends on the data), a 2 GiB device-to-device copy, and a
    plain streaming read of 4 GiB."""
    res = {}
    res["mfma_loop_bf16_random_tflops"] = round(mfma_ceiling(0), 1)
    res["mfma_loop_bf16_ones_tflops"] = round(mfma_ceiling(1), 1)
    n = 8192
    g = torch.Generator(device=DEV).manual_seed(0)
    for name, fill in (("random", None), ("ones", 1.0)):
        a = torch.randn(n, n, device=DEV, generator=g).to(torch.bfloat16) if fill is None else \
            torch.full((n, n), fill, dtype=torch.bfloat16, device=DEV)
        b = torch.randn(n, n, device=DEV, generator=g).to(torch.bfloat16) if fill is None else a.clone()
        c = torch.empty(n, n, dtype=torch.bfloat16, device=DEV)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        it = 40  # ~1 s of sustained MFMA work
        for _ in range(it):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / it
        res[f"gemm_bf16_8192_{name}_tflops"] = round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    x = torch.ones(1 << 30, dtype=torch.bfloat16, device=DEV)  # 2 GiB
    y = torch.empty_like(x)
    y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    res["device_copy_2gib_read_plus_write_gbs"] = round(2 * x.numel() * 2 / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9, 1)
    del x, y
    res["stream_read_4gib_gbs"] = round(stream_ceiling(), 1)
    return res


def _gpu_clock_info():
    """The graphics clock range and power cap the GPU reports (amd-smi, rocm-smi; read
    once, in child processes), or None where a tool is missing.  The clock is not locked
    on these parts: it floats under the power cap, which is why rates move from box to box."""
    import subprocess
    info = {}
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout)
        gpus = data["gpu_data"] if isinstance(data, dict) else data
        clk = gpus[0]["clock"]
        gfx = [v for k, v in clk.items() if k.startswith("gfx")]
        info["gfx_clk_max_mhz"] = gfx[0]["max_clk"]["value"]
        info["gfx_clk_min_mhz"] = gfx[0]["min_clk"]["value"]
        info["gfx_clk_locked"] = gfx[0].get("clk_locked")
    except Exception:  # pragma: no cover - tool missing or output changed
        pass
    try:
        r = subprocess.run(["rocm-smi", "--showmaxpower", "--json"], capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout[r.stdout.index("{"):])
        card = next(iter(data.values()))
        info["power_cap_w"] = float(next(v for k, v in card.items() if "Power" in k))
    except Exception:  # pragma: no cover
        pass
    return info or None


def _code_only(text: str) -> str:
    """The source with comments and blank lines removed, so that a change to comments
    alone does not retire a counter summary taken on the same machine code."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def sources_sha256(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(_code_only(open(p, encoding="utf-8").read()).encode())
    return h.hexdigest()


def traffic_for(paths, summary: str):
    """HBM bytes per launch from the committed counter summary, if the kernel is unchanged."""
    if not os.path.exists(summary):
        return None
    fields = {}
    for line in open(summary):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel sources sha256") != sources_sha256(paths):
        return None
    return int(fields["HBM bytes per launch"])


def write_traffic_summary(fetch_csv: str, write_csv: str, out: str) -> None:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; with --calib-copy) into the
    committed summary.  Each counter is scaled by what it reads for the plain 256 MiB copy."""
    import csv

    def per_kernel(path, counter):
        fwd, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            # the bf16 forward: out_dtype bf16, no E4M3, no dropout
            if ("fwd_bf16_kernel<128, false, false, false>" in name
                    and int(r["Grid_Size"]) == FWD_GRID_THREADS):
                fwd.append(v)
            if "copyBuffer" in r["Kernel_Name"] and v > 0.25 * COPY_BYTES / 1024:
                copy.append(v)
        if not fwd or not copy:
            raise SystemExit(f"{path}: no forward or calibration-copy dispatch with {counter}")
        return float(np.mean(fwd)), float(np.mean(copy))

    f_fwd, f_copy = per_kernel(fetch_csv, "FETCH_SIZE")
    w_fwd, w_copy = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = COPY_BYTES / 1024 / f_copy, COPY_BYTES / 1024 / w_copy
    total = int(round((f_fwd * f_scale + w_fwd * w_scale) * 1024))
    algo = 337_641_472  # Q, K, V, O (bf16) and LSE (fp32) of the workload, read/written once
    with open(out, "w") as fh:
        fh.write("# HBM traffic of fwd_bf16_kernel<128>, B1 Hq32 Hkv8 N16384 D128 causal\n\n")
        fh.write("Commands (MI355X, repository root; one counter per run):\n\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            fh.write(f"    rocprofv3 --pmc {c} --output-format csv -d gpurun_out/<dir> -o run -- "
                     "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --calib-copy\n")
        fh.write("\nThe counters are scaled by their reading for the plain 256 MiB device copy that "
                 "`--calib-copy` runs in the same process (a copy kernel reads and writes exactly "
                 "268,435,456 bytes).\n\n")
        fh.write(f"- FETCH_SIZE KiB per forward launch: {f_fwd:.1f}\n")
        fh.write(f"- FETCH_SIZE KiB of the copy: {f_copy:.1f} (scale {f_scale:.4f})\n")
        fh.write(f"- WRITE_SIZE KiB per forward launch: {w_fwd:.1f}\n")
        fh.write(f"- WRITE_SIZE KiB of the copy: {w_copy:.1f} (scale {w_scale:.4f})\n")
        fh.write(f"- HBM bytes per launch: {total}\n")
        fh.write(f"- algorithmic bytes per launch: {algo} (ratio {total / algo:.2f})\n")
        fh.write(f"- kernel sources sha256: `{sources_sha256(FWD_KERNEL_SRCS)}`\n")
        fh.write("\nbench.py reports `roofline.traffic` from the HBM-bytes line only while the kernel "
                 "sources, comments and blank lines aside, hash to the value above.\n")
    print(f"wrote {out}: {total} bytes per launch", file=sys.stderr)


# ------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64,
                    help="timed steps (64 steps of the default legs take about 0.2 s)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="fwd,bwd,decode")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle on the host (and with it the parity check)")
    ap.add_argument("--no-short", action="store_true",
                    help="skip the short forwards timed outside the step")
    ap.add_argument("--aux", action="store_true",
                    help="also time dropout, the FP8 forward, the GQA backward, the packed "
                         "variable-length forward and the paged-cache decode (outside the step)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--ceilings", action="store_true",
                    help="also measure a library bf16 GEMM and a streaming read (context only)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM-traffic summary from two rocprofv3 counter CSVs and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic_summary(args.write_traffic[0], args.write_traffic[1], TRAFFIC_FILE)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward would shard over heads with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if not fa.device_supported(0):
        print("cuda:0 is not gfx950", file=sys.stderr)
        sys.exit(1)

    legs_wanted = [s for s in args.legs.split(",") if s]
    log("setting up inputs ...")
    legs = {}
    if "fwd" in legs_wanted:
        legs["fwd"] = FwdLeg(FWD_CFG)
    if "bwd" in legs_wanted:
        legs["bwd"] = BwdLeg(BWD_CFG)
    if "decode" in legs_wanted:
        legs["decode"] = DecodeLeg(DEC_CFG)
    torch.cuda.synchronize()
    log("inputs resident; warmup")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for leg in legs.values():
            leg.run()
    torch.cuda.synchronize()

    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in legs}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        for n, leg in legs.items():
            ev[n][i][0].record(stream)
            leg.run()
            ev[n][i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    leg_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in legs}
    log(f"timed {args.steps} steps: {total_ms:.2f} ms (host wall {wall * 1e3:.2f} ms)")

    out_legs = {}
    flops = 0
    for n, leg in legs.items():
        ms = leg_ms[n]
        tf = leg.flops / (ms * 1e-3) / 1e12
        flops += leg.flops
        per_step = sorted(a.elapsed_time(b) for a, b in ev[n])
        rec = {"ms": round(ms, 4), "median_ms": round(float(np.median(per_step)), 4),
               "min_ms": round(per_step[0], 4), "tflops": round(tf, 2),
               "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        if n == "decode":
            gbs = leg.bytes / (ms * 1e-3) / 1e9
            rec.update({"hbm_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes": int(leg.bytes)})
        out_legs[n] = rec

    # one untimed call per leg; host copies of its outputs for the parity check
    gpu_out = {}
    if not args.no_cpu_baseline:
        for n, leg in legs.items():
            leg.run()
        torch.cuda.synchronize()
        host = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
        if "fwd" in legs:
            gpu_out["fwd_o"], gpu_out["fwd_lse"] = host(legs["fwd"].o), host(legs["fwd"].lse)
        if "bwd" in legs:
            for nm, t in zip(("dq", "dk", "dv"), legs["bwd"].grads):
                gpu_out[f"bwd_{nm}"] = host(t)
        if "decode" in legs:
            gpu_out["dec_o"], gpu_out["dec_lse"] = host(legs["decode"].o), host(legs["decode"].lse)

    def flops_rec(leg, ms):
        tf = leg.flops / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "tflops": round(tf, 2), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                "in_step": False}

    if not args.no_short:
        short = {}
        for name, cfg in SHORT_CFGS.items():
            leg = FwdLeg(cfg)
            out_legs[name] = flops_rec(leg, time_aux(leg, stream, reps=20 if cfg["N"] > 1024 else 200))
            if cfg["N"] <= 1024:
                # the binding's host cost per call (about 15 us) is as long as this kernel, so
                # the eager figure above is bound by the host: report the GPU time per call of
                # a graph of the calls as `ms`, and the eager figure beside it
                out_legs[name]["eager_ms"] = out_legs[name]["ms"]
                gr = flops_rec(leg, time_graph(leg))
                out_legs[name].update(ms=gr["ms"], tflops=gr["tflops"], frac_bf16_peak=gr["frac_bf16_peak"],
                                      timing="one HIP graph of 200 calls, replayed")
            leg.run()  # untimed call for the parity check
            torch.cuda.synchronize()
            short[name] = (leg, leg.o.detach().float().cpu().numpy().astype(np.float64),
                           leg.lse.detach().cpu().numpy().astype(np.float64))
            leg.q = leg.k = leg.v = leg.o = None
        if not args.no_cpu_baseline:
            gpu_out["short"] = short

    if args.aux:
        fl = legs["fwd"] if "fwd" in legs else FwdLeg(FWD_CFG)
        bl = legs["bwd"] if "bwd" in legs else BwdLeg(BWD_CFG)
        dl = DropoutLegs(fl, bl)

        class _F:
            run = dl.run_fwd

        class _B:
            run = dl.run_bwd
        _F.flops, _B.flops = fl.flops, bl.flops
        out_legs["fwd_dropout_p0.1"] = flops_rec(_F, time_aux(_F, stream))
        out_legs["bwd_dropout_p0.1"] = flops_rec(_B, time_aux(_B, stream))
        del dl
        leg = FwdFp8Leg(FWD_CFG)
        rec = flops_rec(leg, time_aux(leg, stream))

        class _Q:  # the two quantisation passes for Q and K, timed alone
            run = leg.quantize
        rec["quantize_q_k_ms"] = round(time_aux(_Q, stream), 4)
        out_legs["fwd_fp8qk_b1h32kv8n16384_causal"] = rec
        del leg
        leg = BwdLeg(BWD_GQA_CFG)
        out_legs["bwd_gqa_b1h32kv8n16384_causal"] = flops_rec(leg, time_aux(leg, stream, reps=5))
        del leg
        leg = FwdVarlenLeg(VARLEN_CFG)
        out_legs["fwd_varlen_32seqs_u256_4096_causal"] = dict(flops_rec(leg, time_aux(leg, stream)),
                                                               tokens=leg.tokens)
        del leg
        dec = legs["decode"] if "decode" in legs else DecodeLeg(DEC_CFG)
        for page in PAGED_SIZES:
            leg = DecodePagedLeg(dec, page)
            ms = time_aux(leg, stream)
            gbs = leg.bytes / (ms * 1e-3) / 1e9
            out_legs[f"decode_paged_p{page}"] = {"ms": round(ms, 4), "hbm_gbs": round(gbs, 1),
                                                 "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                                                 "algorithmic_bytes": int(leg.bytes), "in_step": False}
            del leg

    if args.calib_copy:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=DEV).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst

    value = flops / (ms_per_step * 1e-3) / 1e12
    roofline = None
    if "fwd" in legs:
        ach = legs["fwd"].flops / (leg_ms["fwd"] * 1e-3) / 1e12
        roofline = {"kernel": "fwd_bf16_kernel<128> (one launch per fa_fwd call)", "bound": "mfma",
                    "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_for(FWD_KERNEL_SRCS, TRAFFIC_FILE)}
    ceil = None
    if args.ceilings:
        log("measuring library GEMM / streaming-read ceilings ...")
        ceil = ceilings()
    cpu = parity = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host and checking the GPU outputs against it ...")
        cpu, parity = cpu_baseline(gpu_out if legs else None)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one step = fwd B1 Hq32 Hkv8 N16384 D128 causal + bwd B2 H16 N4096 D128 "
                               "causal + split-KV decode 64 seqs Hq32 Hkv8 D128 L~U[1024,32768] split 2048",
                   "legs": list(legs), "seed": 0, "global_batch": None, "parallelism": "single GPU",
                   "value": "credited matmul FLOPs of the step's three legs (4*D per visible pair forward, "
                            "10*D backward, 4*D per cached key and query head decode) / step time; the "
                            "per-leg rates and fractions of peak are under legs"},
        "legs": out_legs,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if ceil is not None:
        line["ceilings"] = ceil
    props = torch.cuda.get_device_properties(0)
    line["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                      "hip_runtime": getattr(torch.version, "hip", None), "cus": props.multi_processor_count,
                      "clocks": _gpu_clock_info()}
    print(json.dumps(line), flush=True)
    if parity is not None and not parity["pass"]:
        log("parity check FAILED: " + json.dumps(parity))
        sys.exit(3)


if __name__ == "__main__":
    main()
