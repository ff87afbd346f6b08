#!/usr/bin/env python3
"""Throughput of THD varlen attention forward + backward on one MI355X.

Workload (the headline configuration): 65536 packed tokens, 16 sequences
with lengths drawn uniform in [256, 8192] (seed 0) and padded to multiples of
64, hq=64, hkv=8, d=128, bf16, padding_causal, deterministic backward.
A step is one forward (scheduler, forward kernel, zero fill) plus one
backward (scheduler, Delta, dQ, dK/dV, zero fills) over the whole batch,
with inputs, outputs and workspace resident in HBM.

FLOP model of the metric: F_fwd = 4*d*hq*sum(Lq*Lkv)/2 (causal) on real
lengths, F_bwd = 2.5*F_fwd; value = (F_fwd + F_bwd) / time per step.

Prints ONE JSON line.  Besides the metric it carries
  stages_ms    -- per-stage times of a few instrumented steps run after the
                  warmup, outside the timed region (a HIP event at every
                  stage boundary costs ~1% of a step);
  split        -- the forward alone and the backward alone from those steps
                  (their stages summed), in ms and TFLOP/s by the FLOP model;
  roofline     -- the dominant kernel's algorithmic FLOP/s (from the two HIP
                  events recorded around its launches in the timed region,
                  the only events the timed steps record) against
                  the dense bf16 MFMA peak, and its HBM traffic from the
                  committed rocprofv3 counter summary when that summary was
                  taken on the current kernel source (else null);
  cpu_baseline -- the fp64 CPU oracle timed on a bounded sample of the same
                  workload (rank 0, N=1 only).

Options: --gpus N (only 1 is supported: the library runs on one GPU),
--steps K, --warmup W, --no-cpu-baseline, --copy-calibration (adds a plain
1 GiB device copy after the timed region, used to scale rocprofv3's
FETCH_SIZE / WRITE_SIZE counters to bytes), --smi (samples board power and
graphics clocks with amd-smi during the timed steps; give enough --steps for
a few seconds), --workload NAME:
  throughput_65k        the headline configuration above (default)
  sbhd_65k              sbhd [4096, 16, 64, 128] bf16 padding_causal, read in
                        place by the batched entry points (same FLOP model)
  chunks4_65k           the headline sequences with every sequence's keys in 4
                        chunks of consecutive positions, run through the
                        chunked entry points (partial forwards merged, chunk
                        backwards from the merged O/LSE, dQ accumulated)
  fp8_65k               the headline sequences with q, k, v as E4M3 codes and
                        per-tensor descales; the step is the FP8-input forward
  fp8_train_65k         the fp8_65k inputs; the step is the FP8-input forward
                        and backward (gradients in bf16)
  dropout_65k           the headline workload with dropout p = 0.1 (Philox keep
                        mask) in the forward and the backward
  d64_65k, d256_65k     the headline sequences at head dim 64 / 256 (hq 64,
                        hkv 8, bf16, causal)
  mqa_65k               the headline sequences with one KV head (hq 64, d 128)
  chunked_bottom_right  THD query chunks of 2048 tokens (the last tokens of
                        each context) against contexts U[2048, 8192] (65536
                        key tokens), bottom-right causal; FLOPs counted on
                        the exact number of visible (query, key) pairs
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
MFMA_PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E, published
METRIC = "fwd+bwd TFLOP/s (THD bf16 padding_causal, hq64/hkv8/d128) + % MFMA peak"
PROFILES = os.path.join(ROOT, "profiles")

WORKLOADS = {
    "throughput_65k": dict(
        layout="thd", metric=METRIC,
        desc="throughput_65k: 65536 packed tokens, 16 sequences, lengths U[256,8192] seed 0 "
             "padded to 64, hq=64 hkv=8 d=128, bf16, padding_causal, fwd+bwd"),
    "sbhd_65k": dict(
        layout="sbhd",
        metric="fwd+bwd TFLOP/s (sbhd bf16 padding_causal, hq64/hkv8/d128) + % MFMA peak",
        desc="sbhd_65k: sbhd [4096, 16, 64, 128] read in place, 16 full sequences, hq=64 "
             "hkv=8 d=128, bf16, padding_causal, fwd+bwd"),
    "chunks4_65k": dict(
        layout="chunks", chunks=4, case="throughput_65k",
        metric="fwd+bwd TFLOP/s (THD bf16 padding_causal over 4 key chunks + merge, "
               "hq64/hkv8/d128) + % MFMA peak",
        desc="chunks4_65k: the throughput_65k sequences with every sequence's keys in 4 chunks "
             "of consecutive positions; per step 4 chunk forwards + 3 (O, LSE) merges, then 4 "
             "chunk backwards from the merged O/LSE with dQ accumulated; same FLOP model"),
    "dropout_65k": dict(
        layout="thd", case="throughput_65k", dropout=(0.1, 0x5EED, 0),
        metric="fwd+bwd TFLOP/s (THD bf16 padding_causal, dropout 0.1, hq64/hkv8/d128) "
               "+ % MFMA peak",
        desc="dropout_65k: the throughput_65k workload with dropout p = 0.1 (Philox keep mask, "
             "seed 0x5EED, offset 0) in the forward and the backward; same FLOP model"),
    "fp8_65k": dict(
        layout="fp8", case="throughput_65k", fwd_only=True, dtype="e4m3/bf16",
        # the forward's S products run on the E4M3 MFMA, its PV products on bf16:
        # half of F_fwd at each peak
        peak=1.0 / (0.5 / MFMA_PEAK_FP8_TFLOPS + 0.5 / MFMA_PEAK_BF16_TFLOPS),
        metric="fwd TFLOP/s (THD FP8 E4M3 inputs, bf16 out, padding_causal, hq64/hkv8/d128) "
               "+ % MFMA peak",
        desc="fp8_65k: the throughput_65k sequences with q, k, v quantised to E4M3 (per-tensor "
             "descale = amax / 448); one step = the FP8-input forward (decode of V + forward); "
             "FLOPs = F_fwd"),
    "fp8_train_65k": dict(
        layout="fp8", case="throughput_65k", dtype="e4m3/bf16",
        peak=1.0 / (0.5 / MFMA_PEAK_FP8_TFLOPS + 0.5 / MFMA_PEAK_BF16_TFLOPS),
        metric="fwd+bwd TFLOP/s (THD FP8 E4M3 inputs, bf16 out and gradients, padding_causal, "
               "hq64/hkv8/d128) + % MFMA peak",
        desc="fp8_train_65k: the fp8_65k inputs; one step = the FP8-input forward and the "
             "FP8-input backward (q, k, v decoded exactly, 16-bit backward products, gradients "
             "in bf16 with respect to the descaled inputs); FLOPs = F_fwd + F_bwd"),
    "d64_65k": dict(
        layout="thd",
        metric="fwd+bwd TFLOP/s (THD bf16 padding_causal, hq64/hkv8/d64) + % MFMA peak",
        desc="d64_65k: the throughput_65k sequences at head dim 64 (hq=64 hkv=8), bf16, "
             "padding_causal, fwd+bwd; same FLOP model"),
    "d256_65k": dict(
        layout="thd",
        metric="fwd+bwd TFLOP/s (THD bf16 padding_causal, hq64/hkv8/d256) + % MFMA peak",
        desc="d256_65k: the throughput_65k sequences at head dim 256 (hq=64 hkv=8), bf16, "
             "padding_causal, fwd+bwd; same FLOP model"),
    "mqa_65k": dict(
        layout="thd",
        metric="fwd+bwd TFLOP/s (THD bf16 padding_causal, hq64/hkv1/d128) + % MFMA peak",
        desc="mqa_65k: the throughput_65k sequences with one KV head for 64 query heads, d=128, "
             "bf16, padding_causal, fwd+bwd; same FLOP model"),
    "chunked_bottom_right": dict(
        layout="thd",
        metric="fwd+bwd TFLOP/s (THD bf16 padding_causal_bottom_right, query chunks, "
               "hq64/hkv8/d128) + % MFMA peak",
        desc="chunked_bottom_right: 14 contexts U[2048,8192] seed 0 padded to 64 (65536 key "
             "tokens), queries = last 2048 tokens of each, hq=64 hkv=8 d=128, bf16, "
             "bottom-right causal, fwd+bwd; FLOPs on exact visible pairs"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def read_traffic(stage: str):
    """HBM bytes per launch of `stage` from profiles/<stage>_throughput_65k_pmc.txt,
    or None when absent or taken on other kernel source."""
    path = os.path.join(PROFILES, f"{stage}_throughput_65k_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_0-9]+)\s*=\s*(\S+)\s*$", line)
        if m:
            kv[m.group(1)] = m.group(2)
    from bwd_thd_varlen_amd.rocprof_summary import source_hash
    if kv.get("kernel_source_sha256") != source_hash(stage):
        log(f"[bench] {path}: taken on other kernel source -> traffic null")
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def visible_pairs(lq: int, lk: int, causal) -> float:
    """(query, key) pairs a FLOP model counts for one sequence: Lq*Lk, halved
    for the top-left causal triangle (the headline metric's model), and the
    exact count of pairs with key <= query + Lk - Lq for bottom-right."""
    if causal == "bottom_right":
        return float(sum(max(0, min(lk, i + lk - lq + 1)) for i in range(lq)))
    return lq * lk / 2.0 if causal else float(lq * lk)


class SmiSampler:
    """Board power and graphics clocks, sampled with ``amd-smi metric -p -c``
    from a host thread while the timed steps run (``--smi``): shows whether
    the chip holds its nominal clock or sits at its power limit."""

    def __init__(self, gpu: int = 0):
        import threading
        self.gpu, self.samples, self._stop = gpu, [], threading.Event()
        self._th = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import subprocess
        while not self._stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", str(self.gpu), "-p", "-c"],
                                   capture_output=True, text=True, timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            pw = re.search(r"SOCKET_POWER:\s*(\d+)", r.stdout)
            clk = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+) MHz", r.stdout)]
            if pw and clk:
                self.samples.append((int(pw.group(1)), sum(clk) / len(clk)))

    def __enter__(self):
        self._th.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._th.join()

    def summary(self):
        # the first sample may precede the load
        s = self.samples[1:] or self.samples
        if not s:
            return None
        return {"power_w": round(sum(p for p, _ in s) / len(s), 1),
                "gfx_clock_mhz": round(sum(c for _, c in s) / len(s), 1),
                "samples": len(s), "source": "amd-smi metric -p -c during the timed steps"}


def cpu_model(path: str = "/proc/cpuinfo") -> str:
    """The host CPU's model name (/proc/cpuinfo) with its family / model /
    stepping numbers (which identify the part where a virtual machine reports
    only a generic name) and the logical CPU count."""
    fields = {}
    names = 0
    try:
        for line in open(path):
            key, _, val = line.partition(":")
            key = key.strip()
            if key == "model name":
                names += 1
            if key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                fields[key] = val.strip()
    except OSError:
        pass
    if "model name" not in fields:
        return "unknown"
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{fields['model name']} ({ids + '; ' if ids else ''}{names} logical CPUs)"


def cpu_baseline(case, budget_s: float = 12.0, dropout=None, fwd_only=False):
    """The fp64 oracle, as it stands, on (sequence, KV group) units of the same
    workload: the sequences closest to 2400 query tokens first, KV groups 0,
    1, ... of each, until `budget_s` of CPU work has been spent."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    real = np.diff(case.cu_seqlens_q)
    real_k = np.diff(case.cu_seqlens_kv)
    G = case.hq // case.hkv
    f64 = lambda t: t.to(torch.float64).numpy()
    flops, spent, units = 0.0, 0.0, []
    for b in np.argsort(np.abs(real - 2400), kind="stable"):
        L, oq = int(real[b]), int(case.cu_seqlens_q_padded[b])
        Lk, ok = int(real_k[b]), int(case.cu_seqlens_kv_padded[b])
        for g in range(case.hkv):
            q = f64(case.q[oq:oq + L, g * G:(g + 1) * G])
            k = f64(case.k[ok:ok + Lk, g:g + 1])
            v = f64(case.v[ok:ok + Lk, g:g + 1])
            do = f64(case.dout[oq:oq + L, g * G:(g + 1) * G])
            t0 = time.perf_counter()
            keep, kscale = None, 1.0
            if dropout is not None:
                from oracle.philox import dropout_threshold, keep_mask
                t = dropout_threshold(dropout[0])
                keep = np.stack([keep_mask(L, Lk, int(b), h, case.hq, dropout[1], dropout[2], t)
                                 for h in range(g * G, (g + 1) * G)])
                kscale = 256.0 / (256.0 - t)
            oracle.attn_fwd_seq(q, k, v, case.scale, case.causal, keep=keep, keep_scale=kscale)
            if not fwd_only:
                oracle.attn_bwd_seq(q, k, v, do, case.scale, case.causal, keep=keep,
                                    keep_scale=kscale)
            spent += time.perf_counter() - t0
            flops += (1.0 if fwd_only else 3.5) * 4.0 * case.d * G * visible_pairs(L, Lk, case.causal)
            units.append((int(b), L))
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    seqs = sorted({u for u in units})
    desc = ", ".join(f"sequence {b} (L={L}) x {sum(1 for u in units if u[0] == b)} KV group(s)"
                     for b, L in seqs)
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": (f"fp64 numpy oracle {'fwd' if fwd_only else 'fwd+bwd'} of {desc} ({G} query "
                       f"heads per group) of the "
                       f"same workload, {spent:.1f} s; FLOPs by the workload's pair model")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--smi", action="store_true",
                    help="sample board power and clocks (amd-smi) during the timed steps")
    ap.add_argument("--workload", default="throughput_65k", choices=sorted(WORKLOADS))
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the library runs on one GPU only (got --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the per-GPU kernel is measured with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bwd_thd_varlen_amd as A
    import workloads

    A.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    log(f"[bench] generating the {args.workload} workload")
    case = getattr(workloads, wl.get("case", args.workload))()
    pairs = sum(visible_pairs(int(a), int(b_), case.causal)
                for a, b_ in zip(np.diff(case.cu_seqlens_q), np.diff(case.cu_seqlens_kv)))
    f_fwd = 4.0 * case.d * case.hq * pairs
    f_bwd = 0.0 if wl.get("fwd_only") else 2.5 * f_fwd
    q, k, v, do = (t.to(dev) for t in (case.q, case.k, case.v, case.dout))
    cu = lambda a: torch.as_tensor(a, dtype=torch.int32, device=dev)
    cq, ck = cu(case.cu_seqlens_q), cu(case.cu_seqlens_kv)
    cqp, ckp = cu(case.cu_seqlens_q_padded), cu(case.cu_seqlens_kv_padded)
    if wl["layout"] == "sbhd":
        # the THD rows b*S + i laid out as sbhd [S, B, h, d] (outside the timed region)
        S, B = case.max_seqlen_q, case.batch
        sb = lambda t: t.view(B, S, *t.shape[1:]).transpose(0, 1).contiguous()
        q, k, v, do = sb(q), sb(k), sb(v), sb(do)
    out, dq, dk, dv = (torch.empty_like(t) for t in (q, q, k, v))
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    tq, tk = case.q.shape[0], case.k.shape[0]
    ws = torch.empty(A.workspace_size(case.batch, tq, tk, case.hq, case.hkv, case.d),
                     dtype=torch.uint8, device=dev)

    # a step is n_fwd forward calls and n_bwd backward calls, each with its
    # own stage events (the chunked workload also times its merges)
    n_fwd = n_bwd = 1
    merge_ev = None
    if wl["layout"] == "sbhd":
        bkw = dict(layout="sbhd", cu_seqlens_q=cq, cu_seqlens_kv=ck,
                   attn_mask_type=case.mask_type, softmax_scale=case.scale, workspace=ws)

        def step(ev_f=(None,), ev_b=(None,), ev_m=None):
            A.fwd_batched(q, k, v, out=out, lse=lse, events=ev_f[0], **bkw)
            A.bwd_batched(q, k, v, out, do, lse, dq=dq, dk=dk, dv=dv, events=ev_b[0], **bkw)
    elif wl["layout"] == "fp8":
        def quant(t):
            s_ = float(t.float().abs().max()) / 448.0
            return (t.float() / s_).to(torch.float8_e4m3fn), s_
        (q8, sq), (k8, sk), (v8, sv) = quant(q), quant(k), quant(v)
        ws8 = torch.empty(A.fp8_workspace_size(case.batch, q.shape[0], k.shape[0], case.hq,
                                               case.hkv, case.d), dtype=torch.uint8, device=dev)
        n_fwd, n_bwd = 1, 0 if wl.get("fwd_only") else 1
        fkw = dict(cu_seqlens_q_padded=cqp, cu_seqlens_kv_padded=ckp,
                   attn_mask_type=case.mask_type, softmax_scale=case.scale, workspace=ws8)

        def step(ev_f=(None,), ev_b=(None,) * n_bwd, ev_m=None):
            A.fwd_fp8(q8, k8, v8, sq, sk, sv, cq, ck, out=out, lse=lse, events=ev_f[0], **fkw)
            if n_bwd:
                A.bwd_fp8(q8, k8, v8, sq, sk, sv, out, do, lse, cq, ck, dq=dq, dk=dk, dv=dv,
                          events=ev_b[0], **fkw)
    elif wl["layout"] == "chunks":
        # every sequence's keys in C chunks of consecutive positions (outside
        # the timed region: gathered into THD chunk tensors)
        C = wl["chunks"]
        real, offs = np.diff(case.cu_seqlens_kv), case.cu_seqlens_kv_padded[:-1]
        chunks = []
        for c in range(C):
            a, e = real * c // C, real * (c + 1) // C
            rows = np.concatenate([np.arange(o + x, o + y) for o, x, y in zip(offs, a, e)])
            idx = torch.as_tensor(rows, dtype=torch.long, device=dev)
            kc, vc = k.index_select(0, idx).contiguous(), v.index_select(0, idx).contiguous()
            chunks.append(dict(k=kc, v=vc, cu=cu(np.concatenate([[0], np.cumsum(e - a)])),
                               pos=cu(a), dk=torch.empty_like(kc), dv=torch.empty_like(vc)))
        o_part, l_part = torch.empty_like(out), torch.empty_like(lse)
        # one workspace for every chunk call, of the largest size they ask for
        # (fewer key tokens per call can mean partial dK/dV planes)
        need = max(A.workspace_size(case.batch, tq, int(ch["k"].shape[0]), case.hq, case.hkv, case.d)
                   for ch in chunks)
        if need > ws.numel():
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        n_fwd = n_bwd = C
        merge_ev = True
        ckw = dict(cu_seqlens_q_padded=cqp, attn_mask_type=case.mask_type,
                   softmax_scale=case.scale, workspace=ws)

        def step(ev_f=(None,) * C, ev_b=(None,) * C, ev_m=None):
            for c, ch in enumerate(chunks):
                o_c, l_c = (out, lse) if c == 0 else (o_part, l_part)
                A.fwd_chunk(q, ch["k"], ch["v"], cq, ch["cu"], kv_pos0=ch["pos"], out=o_c,
                            lse=l_c, events=ev_f[c], **ckw)
                if c > 0:
                    if ev_m is not None:
                        ev_m[c - 1][0].record()
                    A.merge(out, lse, o_part, l_part)
                    if ev_m is not None:
                        ev_m[c - 1][1].record()
            for c, ch in enumerate(chunks):
                A.bwd_chunk(q, ch["k"], ch["v"], out, do, lse, cq, ch["cu"], kv_pos0=ch["pos"],
                            dq=dq, dk=ch["dk"], dv=ch["dv"],
                            accumulate={"dq"} if c > 0 else False, events=ev_b[c], **ckw)
    else:
        kw = dict(cu_seqlens_q_padded=cqp, cu_seqlens_kv_padded=ckp,
                  max_seqlen_q=case.max_seqlen_q, max_seqlen_kv=case.max_seqlen_kv,
                  attn_mask_type=case.mask_type, softmax_scale=case.scale, workspace=ws)
        if "dropout" in wl:
            p_, seed_, off_ = wl["dropout"]
            kw.update(dropout_p=p_, rng_seed=seed_, rng_offset=off_)

        def step(ev_f=(None,), ev_b=(None,), ev_m=None):
            A.fwd(q, k, v, cq, ck, out=out, lse=lse, events=ev_f[0], **kw)
            A.bwd(q, k, v, out, do, lse, cq, ck, dq=dq, dk=dk, dv=dv, events=ev_b[0], **kw)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fwd_stage_names = A.FP8_FWD_STAGES if wl["layout"] == "fp8" else A.FWD_STAGES
    bwd_stage_names = A.FP8_BWD_STAGES if wl["layout"] == "fp8" else A.BWD_STAGES

    def events(only=None):
        """Stage events of one step: every stage boundary (only=None), or just
        the two events around stage `only` = ("fwd" | "bwd", index) of each call."""
        f_only = only[1] if only and only[0] == "fwd" else None
        b_only = only[1] if only and only[0] == "bwd" else None
        ef = [A.StageEvents(len(fwd_stage_names) + 1, f_only) if only is None or f_only is not None
              else None for _ in range(n_fwd)]
        eb = [A.StageEvents(len(bwd_stage_names) + 1, b_only) if only is None or b_only is not None
              else None for _ in range(n_bwd)]
        em = ([(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_fwd - 1)] if merge_ev and only is None else None)
        return ef, eb, em

    def stage_sums(ef, eb, em):
        """Each stage's time summed over one step's calls (stages not timed: absent)."""
        tot = {}
        for e in ef:
            for name, ms in zip(("fwd." + s_ for s_ in fwd_stage_names), e.stage_ms() if e else []):
                if ms is not None:
                    tot[name] = tot.get(name, 0.0) + ms
        for e in eb:
            for name, ms in zip(("bwd." + s_ for s_ in bwd_stage_names), e.stage_ms() if e else []):
                if ms is not None:
                    tot[name] = tot.get(name, 0.0) + ms
        if em:
            tot["fwd.merge"] = sum(a.elapsed_time(b_) for a, b_ in em)
        return tot

    # Per-stage breakdown from an instrumented pass outside the timed region
    # (a HIP event at every stage boundary costs ~1% of a step).
    n_probe = max(1, min(5, args.steps))
    probe = [events() for _ in range(n_probe)]
    for ef, eb, em in probe:
        step(ef, eb, em)
    torch.cuda.synchronize()
    stage_ms = {}
    for ef, eb, em in probe:
        for name, ms in stage_sums(ef, eb, em).items():
            stage_ms.setdefault(name, []).append(ms)
    avg = {k_: sum(v_) / len(v_) for k_, v_ in stage_ms.items()}
    log(f"[bench] per-stage average ms ({n_probe} instrumented steps): " +
        ", ".join(f"{k_}={v_:.3f}" for k_, v_ in avg.items()))

    # algorithmic work per step of each compute kernel (GEMM FLOPs it must
    # do), over its time per step (one launch, or the sum of a step's launches)
    work = {"fwd.fwd": ("fwd", f_fwd),            # S = QK^T, O = PV
            "bwd.dkdv": ("dkdv", 2.0 * f_fwd),    # S, dP, dV = P^T dO, dK = dS^T Q
            "bwd.dq": ("dq", 1.5 * f_fwd)}        # S, dP (recomputed), dQ = dS K
    work = {k_: w_ for k_, w_ in work.items() if k_ in avg}
    dom = max(work, key=lambda s_: avg[s_])
    kname, flops = work[dom]
    side, sname = dom.split(".")
    dom_only = (side, (fwd_stage_names if side == "fwd" else bwd_stage_names).index(sname))

    # The timed region: K steps; the only events recorded are the two around
    # the dominant kernel of each call, for its live launch time.
    evs = [events(dom_only) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    smi = SmiSampler() if args.smi else None
    if smi:
        smi.__enter__()
    t0 = time.perf_counter()
    for ef, eb, em in evs:
        step(ef, eb, em)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if smi:
        smi.__exit__(None, None, None)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    dom_ms = sum(stage_sums(*e)[dom] for e in evs) / len(evs)
    log(f"[bench] {dom} in the timed steps: {dom_ms:.3f} ms per step")

    # forward alone and backward alone (their stages summed, instrumented pass)
    fwd_ms = sum(v_ for k_, v_ in avg.items() if k_.startswith("fwd."))
    bwd_ms = sum(v_ for k_, v_ in avg.items() if k_.startswith("bwd."))
    split = {"fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2)}
    if bwd_ms > 0:
        split.update({"bwd_ms": round(bwd_ms, 4),
                      "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2)})

    achieved = flops / (dom_ms * 1e-3) / 1e12
    # the FP8 forward mixes E4M3 and bf16 products; every other kernel is bf16
    peak = wl.get("peak", MFMA_PEAK_BF16_TFLOPS) if dom == "fwd.fwd" else MFMA_PEAK_BF16_TFLOPS
    n_calls = n_bwd if side == "bwd" else n_fwd
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                # counter summaries are taken on the headline workload only
                "traffic": read_traffic(kname) if args.workload == "throughput_65k" else None,
                "kernel": kname,
                "avg_launch_ms": round(dom_ms / n_calls, 4),
                "launches_per_step": n_calls}

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device copies done")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(case, dropout=wl.get("dropout"), fwd_only=bool(wl.get("fwd_only")))

    rec = {
        "metric": wl["metric"], "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.get("dtype", "bf16"),
        "data": "synthetic",
        "config": {"workload": wl["desc"],
                   "tokens_q": int(tq), "tokens_kv": int(tk), "sequences": case.batch,
                   "hq": case.hq, "hkv": case.hkv, "d": case.d,
                   "max_seqlen_q": case.max_seqlen_q, "max_seqlen_kv": case.max_seqlen_kv,
                   "flops_per_step": f_fwd + f_bwd},
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        # from the instrumented steps after the warmup (outside the timed region)
        "stages_ms": {k_: round(v_, 4) for k_, v_ in avg.items()},
        "split": split,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if smi:
        rec["board"] = smi.summary()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
