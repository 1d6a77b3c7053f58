"""Benchmark of the varlen gated delta-rule hot path on one MI355X.

A step is one pass of the whole path over one batch of seeded synthetic input, with inputs resident
in HBM: the varlen causal conv1d (its window carried to the next step) followed by the gated delta-rule
recurrence (state updated in place).  The default workload is the decode step (B=256 sequences x 1
token, HQ=16, H=32, K=V=128, bf16, fp32 state) as one gdn_decode_step launch, the new conv window
written to a second buffer that swaps with the first every step (--two-call runs gdn_conv1d_varlen
then gdn_scan_varlen on its DECODE path instead; "also" compares the forms at several batch sizes).
The prefill workload (B=8, lengths ~ U[512, 4096]) and the long single sequence (N=65536, H=16) are
measured too and reported in "also", with the arithmetic roofline of the path they take, and so is a
speculative verification step (B=256 x 5 tokens) with and without the capture of 4 tokens per
sequence, both steps with one decay per key channel instead of one per head, and the recurrence
reading separate padded q/k/v buffers instead of the packed row.

Prints ONE JSON line.  The dominant kernel (the fused step, or the recurrence in the two-call form)
is timed with HIP events on the stream it is launched on; its algorithmic bytes per launch are the
fp32 state read and written, the token streams it must read (q, k, v, a, b) and write (out), and
for the fused step also the carried conv window read and written and the conv weights.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
SCAN_SOURCES = ["gated_delta_rule_varlen_amd/csrc/gdn_scan.hip", "gated_delta_rule_varlen_amd/csrc/gdn_device.hpp"]
STEP_SOURCES = ["gated_delta_rule_varlen_amd/csrc/gdn_decode.hip", "gated_delta_rule_varlen_amd/csrc/gdn_device.hpp"]
CHUNK_SOURCES = ["gated_delta_rule_varlen_amd/csrc/gdn_chunk.hpp", "gated_delta_rule_varlen_amd/csrc/gdn_device.hpp"]


def sizeof(dt: str) -> int:
    return 4 if dt == "f32" else 2


def scan_bytes(w) -> int:
    """Algorithmic HBM bytes of one recurrence launch: state in + out (fp32), token rows
    [q|k|v] and the two gate inputs read, outputs written."""
    state = 2 * w.B * w.H * w.V * w.K * 4
    tokens = w.N * (w.C * sizeof(w.io) + 2 * w.H * sizeof(w.gate_dtype)) + w.N * w.H * w.V * sizeof(w.io)
    return state + tokens


def capsule_bytes(w, cap: int) -> int:
    """Bytes of the fp32 capture capsule the recurrence writes: cap slots of (H decays, HQ*K keys,
    H*V written values) per sequence."""
    return w.B * cap * (w.H + w.HQ * w.K + w.H * w.V) * 4


def step_bytes(w) -> int:
    """Algorithmic HBM bytes of one fused decode step (gdn_decode_step): the recurrence's bytes with
    the raw token rows in place of the conv output, plus the carried window read and written and the
    conv weights and bias read once."""
    window = 2 * w.B * w.C * w.L * sizeof(w.conv_state_dtype)
    params = w.C * w.W * sizeof(w.io) + (w.C * sizeof(w.io) if w.conv_bias is not None else 0)
    return scan_bytes(w) + window + params


def src_digest(sources=SCAN_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(record: str, sources=SCAN_SOURCES):
    """HBM bytes per launch from committed rocprofv3 counter runs, only while the kernel source is
    unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{record}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("src_digest") != src_digest(sources):
        return None
    return rec.get("bytes_per_launch")


class Path:
    """Device-resident inputs of one workload and one step of the hot path."""

    def __init__(self, w, torch, path: str, fused_step: bool = False, cap: int = 0, gate_per_key: bool = False,
                 window_in_place: bool = False):
        import gated_delta_rule_varlen_amd as gdn

        self.gdn, self.torch, self.w, self.path, self.fused_step, self.cap = gdn, torch, w, path, fused_step, cap
        self.window_in_place = window_in_place
        self.gate_per_key = gate_per_key
        dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

        def dev(a, d):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            t = torch.from_numpy(a if d == "f32" else a.view(np.int16)).cuda()
            return t if d == "f32" else t.view(dt[d])

        self.x = dev(w.x, w.io)
        self.conv_w = dev(w.conv_w, w.io)
        self.conv_b = dev(w.conv_bias, w.io)
        self.conv_state = dev(w.conv_state, w.conv_state_dtype)
        if self.conv_state is None and w.L > 0:
            self.conv_state = torch.zeros((w.B, w.C, w.L), dtype=dt[w.conv_state_dtype], device="cuda")
        self.offsets = torch.from_numpy(w.offsets).cuda()
        self.a, self.b = dev(w.a, w.gate_dtype), dev(w.b, w.gate_dtype)
        if gate_per_key:
            # one decay input per key channel, drawn like the per-head ones
            rng = np.random.default_rng(7)
            a_pk = rng.standard_normal((w.N, w.H, w.K), dtype=np.float32)
            self.a = torch.from_numpy(a_pk).cuda().to(self.b.dtype if self.b is not None else torch.float32)
        self.A_log, self.dt_bias = dev(w.A_log, "f32"), dev(w.dt_bias, "f32")
        self.state = dev(w.state, "f32")
        if self.state is None:
            self.state = torch.zeros((w.B, w.H, w.V, w.K), dtype=torch.float32, device="cuda")
        # the fused step writes the new window into a second buffer and the two swap every step
        # (with an in-place window it takes its key-head form, which is slower at large batches)
        self.conv_state_next = (self.conv_state.clone() if fused_step and not window_in_place
                                and self.conv_state is not None else self.conv_state)
        self.y = torch.empty_like(self.x)
        self.out = torch.empty((w.N, w.H, w.V), dtype=self.x.dtype, device="cuda")
        if cap > 0:
            # speculative decoding: record every token up to the capacity
            self.counts = torch.full((w.B,), cap, dtype=torch.int32, device="cuda")
            self.updates = torch.empty((w.B, cap, w.C), dtype=self.x.dtype, device="cuda")
            self.capsule = torch.empty((w.B, capsule_bytes(w, cap) // (4 * w.B)), dtype=torch.float32,
                                       device="cuda")

    def step(self, ev=None):
        w, gdn = self.w, self.gdn
        if self.fused_step:
            # conv and recurrence in one launch; window and state updated in place
            if ev is not None:
                ev[0].record()
            gdn.decode_step(self.x, self.conv_w, self.offsets, HQ=w.HQ, H=w.H, K=w.K, V=w.V, bias=self.conv_b,
                            conv_state_in=self.conv_state, conv_state_out=self.conv_state_next, dilation=w.D,
                            silu=w.silu, a=self.a, b=self.b, A_log=self.A_log, dt_bias=self.dt_bias,
                            state_in=self.state, state_out=self.state, l2norm=w.l2norm, softplus=w.softplus,
                            sigmoid=w.sigmoid, out=self.out)
            if ev is not None:
                ev[1].record()
            self.conv_state, self.conv_state_next = self.conv_state_next, self.conv_state
            return "decode_step"
        scan_kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=self.a, b=self.b, A_log=self.A_log, dt_bias=self.dt_bias,
                       state_in=self.state, l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid, path=self.path,
                       out=self.out, state_out=self.state)
        if self.gate_per_key:
            scan_kw["gate_per_key"] = True
        if self.cap > 0:
            gdn.conv1d_varlen_capture(self.x, self.conv_w, self.offsets, cap=self.cap, counts=self.counts,
                                      updates=self.updates, bias=self.conv_b, state_in=self.conv_state,
                                      dilation=w.D, silu=w.silu, y=self.y, state_out=self.conv_state)
            if ev is not None:
                ev[0].record()
            _, _, _, used = gdn.scan_varlen_capture(self.y, self.offsets, cap=self.cap, counts=self.counts,
                                                    capsule=self.capsule, **scan_kw)
            if ev is not None:
                ev[1].record()
            return used
        gdn.conv1d_varlen(self.x, self.conv_w, self.offsets, bias=self.conv_b, state_in=self.conv_state,
                          dilation=w.D, silu=w.silu, y=self.y, state_out=self.conv_state)
        if ev is not None:
            ev[0].record()
        _, _, used = gdn.scan_varlen(self.y, self.offsets, **scan_kw)
        if ev is not None:
            ev[1].record()
        return used


EV_EVERY = 8


def time_path(p: "Path", steps: int, warmup: int, ev_every: int = EV_EVERY):
    torch = p.torch
    for _ in range(warmup):
        used = p.step()
    torch.cuda.synchronize()
    # the recurrence launch is bracketed by events on every ev_every-th step of the timed region
    # (events on every step add a few microseconds to each short step; long steps take them on
    # every step)
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in range(0, steps, ev_every)}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        used = p.step(evs.get(i))
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    scan_ms = float(np.mean([a.elapsed_time(b) for a, b in evs.values()]))
    return total_ms / steps, scan_ms, used, wall


def roofline(w, scan_ms: float, workload: str, kernel: str = "scan_kernel", fused_step: bool = False,
             sources=SCAN_SOURCES):
    nbytes = step_bytes(w) if fused_step else scan_bytes(w)
    traffic = measured_traffic(f"{workload}_step", STEP_SOURCES) if fused_step else measured_traffic(workload, sources)
    achieved = nbytes / (scan_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": kernel, "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_us": round(scan_ms * 1e3, 2)}


MFMA_BF16_PEAK_TFS = 2500.0      # MI355X dense bf16 matrix peak, published
VALU_FP32_PUBLISHED_TFS = 157.3  # MI355X fp32 vector peak, published (packed fp32 FMA)
VALU_FP32_PEAK_TFS = 78.6        # 256 CUs x 64 fp32 FMA lanes per clock x 2 flops x 2.4 GHz, non-packed FMA


def compute_roofline(w, scan_ms: float, used: str):
    """Arithmetic side of one recurrence launch.  The chunked form's dense contractions per token and
    value head are 2C(3K + 2V) + 6KV flops (C = 64 tokens per chunk), on bf16 matrix cores; the
    token-sequential form does 7KV fp32 flops per token and value head on the vector ALUs (packed
    fp32 is not used, so the peak is the non-packed one)."""
    if used == "chunk":
        flops = (2 * 64 * (3 * w.K + 2 * w.V) + 6 * w.K * w.V) * w.H * w.N
        bound, peak = "mfma", MFMA_BF16_PEAK_TFS
    else:
        flops = 7 * w.K * w.V * w.H * w.N
        bound, peak = "alu", VALU_FP32_PEAK_TFS
    tfs = flops / (scan_ms * 1e-3) / 1e12
    rec = {"bound": bound, "achieved": round(tfs, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(tfs / peak, 4),
           "flops_per_launch": flops}
    if bound == "alu":  # the published fp32 vector peak counts packed FMAs, which this path does not use
        rec["published_peak"] = VALU_FP32_PUBLISHED_TFS
        rec["frac_of_published"] = round(tfs / VALU_FP32_PUBLISHED_TFS, 4)
    return rec


def secondary(torch, wl, steps: int, warmup: int, record: str):
    """One more workload, measured the same way (chunked path when eligible).  The counter traffic of
    a chunked call is the sum over its kernels (index, tmat, summary, combine, main)."""
    pp = Path(wl, torch, "auto")
    pms, pscan_ms, pused, _ = time_path(pp, steps, warmup, ev_every=1)
    rec = {"workload": wl.name, "N": wl.N, "path": pused, "tokens_per_s": round(wl.N / (pms * 1e-3), 1),
           "ms_per_step": round(pms, 4), "scan_ms": round(pscan_ms, 4),
           "roofline": roofline(wl, pscan_ms, record if pused == "chunk" else "none",
                                "gdn_scan_varlen call (all its kernels)", sources=CHUNK_SOURCES),
           "compute_roofline": compute_roofline(wl, pscan_ms, pused)}
    del pp
    torch.cuda.empty_cache()
    return rec


def fused_comparison(torch, batches=(1, 8, 256), steps: int = 100):
    """Whole decode steps (HQ=16, H=32, K=V=128, bf16) as one gdn_decode_step launch (new window in a
    second buffer, and in place) and as two launches, at several batch sizes: microseconds per
    step, launch cost included (best of 3)."""
    import workloads

    res = {}
    for B in batches:
        w = workloads.make(name=f"decode_b{B}", seed=102, lengths=[1] * B, HQ=16, H=32, K=128, V=128, W=4, D=1,
                           io="bf16", conv_state_dtype="f32", conv_state_std=1.0, state_std=0.1)
        rec = {}
        for name, fused, inplace in (("two_call_us", False, True), ("fused_us", True, False),
                                     ("fused_window_in_place_us", True, True)):
            p = Path(w, torch, "decode", fused_step=fused, window_in_place=inplace)
            rec[name] = round(min(time_path(p, steps, 10)[0] for _ in range(3)) * 1e3, 2)
            del p
        res[f"B{B}"] = rec
    torch.cuda.empty_cache()
    return res


def verify_comparison(torch, steps: int = 50, cap: int = 4):
    """The speculative verification step (B=256 x 5 tokens, HQ=16, H=32, K=V=128, bf16) on the DECODE
    and SEQ paths, without and with capture of cap tokens per sequence: microseconds per whole step
    (best of 3) and the recurrence launch against HBM (its algorithmic bytes include the capsule)."""
    import workloads

    w = workloads.spec_verify()
    res = {"workload": w.name, "cap": cap}
    for path in ("decode", "seq"):
        for c in (0, cap):
            p = Path(w, torch, path, cap=c)
            best = min((time_path(p, steps, 5) for _ in range(3)), key=lambda r: r[0])
            ms, scan_ms, used, _ = best
            nbytes = scan_bytes(w) + (capsule_bytes(w, c) if c else 0)
            gbs = nbytes / (scan_ms * 1e-3) / 1e9
            res[f"{path}_{'capture' if c else 'plain'}"] = {
                "path": used, "step_us": round(ms * 1e3, 2), "tokens_per_s": round(w.N / (ms * 1e-3), 1),
                "scan_us": round(scan_ms * 1e3, 2), "scan_bytes": nbytes, "scan_gbs": round(gbs, 1),
                "scan_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
            del p
    torch.cuda.empty_cache()
    return res


def per_key_comparison(torch, steps: int = 50):
    """The decode step (B=256) and the verification step (B=256 x 5 tokens) with one decay per head
    and with one decay per key channel ([N, H, K] decay input): microseconds per whole step (best of
    3) and the recurrence launch against HBM (the per-key form also reads the [N, H, K] decays)."""
    import workloads

    res = {}
    for w in (workloads.decode_step(), workloads.spec_verify()):
        for pk in (False, True):
            p = Path(w, torch, "auto", gate_per_key=pk)
            ms, scan_ms, used, _ = min((time_path(p, steps, 5) for _ in range(3)), key=lambda r: r[0])
            nbytes = scan_bytes(w) + (w.N * w.H * (w.K - 1) * sizeof(w.gate_dtype) if pk else 0)
            gbs = nbytes / (scan_ms * 1e-3) / 1e9
            res[f"{w.name}_{'per_key' if pk else 'per_head'}"] = {
                "path": used, "step_us": round(ms * 1e3, 2), "scan_us": round(scan_ms * 1e3, 2),
                "scan_gbs": round(gbs, 1), "scan_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
            del p
    torch.cuda.empty_cache()
    return res


def prepare_bytes(w) -> int:
    """Algorithmic HBM bytes of one gdn_prepare_qk_gates launch: the q and k rows and the two gate
    inputs read, the fp32 normalised q/k planes and the g/beta planes written."""
    reads = w.N * (2 * w.HQ * w.K * sizeof(w.io) + 2 * w.H * sizeof(w.gate_dtype))
    writes = w.N * (2 * w.HQ * w.K + 2 * w.H) * 4
    return reads + writes


def prepare_measurement(torch, steps: int = 50):
    """gdn_prepare_qk_gates alone on the prefill and decode workloads: mean microseconds per launch
    (HIP events on the launch stream, best of 3) against the HBM roofline of its algorithmic bytes."""
    import gated_delta_rule_varlen_amd as gdn
    import workloads

    res = {}
    for w in (workloads.varlen_prefill(), workloads.decode_step()):
        p = Path(w, torch, "auto")
        kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=p.a, b=p.b, A_log=p.A_log, dt_bias=p.dt_bias,
                  l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid)
        qk, gb = gdn.prepare_qk_gates(p.x, **kw)
        best = None
        for _ in range(3):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for _ in range(10):
                gdn.prepare_qk_gates(p.x, qk_out=qk, gb_out=gb, **kw)
            for a, b in evs:
                a.record()
                gdn.prepare_qk_gates(p.x, qk_out=qk, gb_out=gb, **kw)
                b.record()
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
            best = us if best is None else min(best, us)
        nbytes = prepare_bytes(w)
        gbs = nbytes / (best * 1e-6) / 1e9
        res[w.name] = {"us": round(best, 2), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
                       "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del p, qk, gb
    torch.cuda.empty_cache()
    return res


def cache_flushed(torch, steps: int = 50, flush_mb: int = 512):
    """The recurrence of the decode, prefill and edge workloads timed with a flush_mb buffer written
    between steps, so that nothing the previous step touched can still sit in the 256 MB memory-side
    cache: mean microseconds per recurrence launch (HIP events on the launch stream, the flush
    outside the pair) next to the back-to-back figure from the same setup, and the flushed launch
    against the HBM roofline of its algorithmic bytes."""
    import workloads

    res = {}
    scratch = torch.empty(flush_mb << 20, dtype=torch.uint8, device="cuda")
    for w in (workloads.decode_step(), workloads.varlen_prefill(), workloads.edge_fp16()):
        p = Path(w, torch, "auto")
        for _ in range(10):
            used = p.step()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            scratch.fill_(i & 0xFF)
            p.step(evs[i])
        torch.cuda.synchronize()
        flushed = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        _, back_to_back, _, _ = time_path(p, steps, 5)
        del p
        gbs = scan_bytes(w) / (flushed * 1e-3) / 1e9
        res[w.name] = {"path": used, "flush_mb": flush_mb, "scan_us_flushed": round(flushed * 1e3, 2),
                       "scan_us_back_to_back": round(back_to_back * 1e3, 2), "scan_gbs_flushed": round(gbs, 1),
                       "scan_hbm_frac_flushed": round(gbs / HBM_PEAK_GBS, 4)}
    del scratch
    torch.cuda.empty_cache()
    return res


def strided_comparison(torch, steps: int = 20):
    """The recurrence on the decode (DECODE) and prefill (CHUNK) workloads reading the packed
    [q | k | v] row and reading three separate buffers with padded rows (row strides HQ*K + 64,
    HQ*K + 64, H*V + 64): microseconds per launch (HIP events, best of 3)."""
    import gated_delta_rule_varlen_amd as gdn
    import workloads

    res = {}
    for w in (workloads.decode_step(), workloads.varlen_prefill()):
        p = Path(w, torch, "auto")
        HQK, HV = w.HQ * w.K, w.H * w.V
        x = p.x
        sep = []
        for lo, width in ((0, HQK), (HQK, HQK), (2 * HQK, HV)):
            buf = torch.empty((w.N, width + 64), dtype=x.dtype, device="cuda")
            buf[:, :width] = x[:, lo:lo + width]
            sep.append(buf[:, :width])
        kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=p.a, b=p.b, A_log=p.A_log, dt_bias=p.dt_bias, state_in=p.state,
                  l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid, out=p.out, state_out=p.state)
        ws_n = gdn.scan_workspace_bytes(x, w.B, HQ=w.HQ, H=w.H, K=w.K, V=w.V)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
        runs = {"packed": lambda: gdn.scan_varlen(x, p.offsets, workspace=ws, **kw)[2],
                "strided": lambda: gdn.scan_varlen_strided(*sep, p.offsets, workspace=ws, **kw)[2]}
        rec = {}
        for name, fn in runs.items():
            best = None
            for _ in range(3):
                for _ in range(3):
                    used = fn()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / steps
                best = us if best is None else min(best, us)
            rec[name] = {"path": used, "us": round(best, 2)}
        res[w.name] = rec
        del p, sep, ws
    torch.cuda.empty_cache()
    return res


def mixed_comparison(torch, steps: int = 10):
    """A serving batch of 255 single tokens and one 4096-token prefill (HQ=16, H=32, K=V=128, bf16):
    the recurrence call on AUTO and on each forced path, microseconds per call with the workspace
    allocated once (best of 3), and AUTO's time over the fastest forced path's."""
    import workloads

    w = workloads.mixed_batch()
    p = Path(w, torch, "auto")
    gdn = p.gdn
    n = gdn.scan_workspace_bytes(p.y, w.B, HQ=w.HQ, H=w.H, K=w.K, V=w.V)
    ws = torch.empty(max(int(n), 1), dtype=torch.uint8, device="cuda")
    p.step()  # the conv output feeds the recurrence
    torch.cuda.synchronize()
    rec = {"workload": w.name, "N": w.N}
    for path in ("auto", "decode", "seq", "chunk"):
        kw = dict(HQ=w.HQ, H=w.H, K=w.K, V=w.V, a=p.a, b=p.b, A_log=p.A_log, dt_bias=p.dt_bias, state_in=p.state,
                  path=path, out=p.out, state_out=p.state, workspace=ws)
        _, _, used = gdn.scan_varlen(p.y, p.offsets, **kw)
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                gdn.scan_varlen(p.y, p.offsets, **kw)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            best = us if best is None else min(best, us)
        rec[path] = {"path": used, "us": round(best, 1), "tokens_per_s": round(w.N / (best * 1e-6), 1)}
    fastest = min(rec[q]["us"] for q in ("decode", "seq", "chunk"))
    rec["auto_over_fastest_forced"] = round(rec["auto"]["us"] / fastest, 3)
    del p, ws
    torch.cuda.empty_cache()
    return rec


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle (conv + scan, fp64, OpenMP) on a bounded sample of the same workload: its first P
    sequences as one batched call (P doubled while a call stays short, up to the whole batch),
    repeated for about budget_s / 2 seconds, once on one thread and once on the default thread
    count (all the host cores the process is given)."""
    import oracle

    def sample(P):
        s, e = 0, int(w.offsets[P])
        off = np.ascontiguousarray(w.offsets[:P + 1])
        return dict(x=np.ascontiguousarray(w.x[s:e]), qkv=np.ascontiguousarray(w.qkv[s:e]), off=off,
                    a=None if w.a is None else np.ascontiguousarray(w.a[s:e]),
                    b=None if w.b is None else np.ascontiguousarray(w.b[s:e]),
                    cst=None if w.conv_state is None else np.ascontiguousarray(w.conv_state[:P]),
                    st=None if w.state is None else np.ascontiguousarray(w.state[:P]), tokens=e - s)

    def call(d):
        oracle.conv(d["x"], w.conv_w, d["off"], W=w.W, D=w.D, x_dtype=w.io, bias=w.conv_bias, state_in=d["cst"],
                    state_dtype=w.conv_state_dtype, silu=w.silu)
        oracle.scan(d["qkv"], d["off"], HQ=w.HQ, H=w.H, K=w.K, V=w.V, qkv_dtype=w.io, gate_dtype=w.gate_dtype,
                    a=d["a"], b=d["b"], A_log=w.A_log, dt_bias=w.dt_bias, state_in=d["st"], l2norm=w.l2norm,
                    softplus=w.softplus, sigmoid=w.sigmoid)

    def run(n_threads):
        oracle.set_threads(n_threads)
        used = oracle.threads()
        P = 1
        while True:
            d = sample(P)
            t0 = time.perf_counter()
            call(d)
            dt = time.perf_counter() - t0
            if P >= w.B or dt >= budget_s / 8:
                break
            P = min(w.B, 2 * P)
        calls, total = 1, dt
        while total < budget_s / 2 and calls < 1000:
            t0 = time.perf_counter()
            call(d)
            total += time.perf_counter() - t0
            calls += 1
        return {"value": round(d["tokens"] * calls / total, 2), "cores": used,
                "sample": f"the first {P} of {w.B} sequences ({d['tokens']} tokens) as one call, {calls} calls, "
                          f"{total:.1f} s"}

    default = oracle.threads()
    one = run(1)
    full = run(default)
    oracle.set_threads(default)
    return {"value": full["value"], "unit": "tokens/s", "cores": full["cores"], "kind": "oracle",
            "sample": full["sample"] + "; conv + scan in fp64",
            "one_thread": {"value": one["value"], "unit": "tokens/s", "cores": 1, "sample": one["sample"]},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def copy_calibration(torch, steps: int, warmup: int):
    """A plain streaming copy of 1 GiB (1 GiB read + 1 GiB written per launch) through an elementwise
    kernel, dst = src * 1: the rate a read-once/write-once kernel reaches on this device.  (The
    runtime's own device-to-device copy, torch's copy_, measured about 20% slower.)"""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        torch.mul(src, 1.0, out=dst)
        b.record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    nbytes = 2 * 4 * n
    return {"copy_bytes_per_launch": nbytes, "avg_launch_us": round(us, 2), "gb_per_s": round(nbytes / (us * 1e-6) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "long", "edge_fp16", "tiny_fp32", "verify", "mixed"])
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "seq", "chunk"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="skip the secondary prefill measurement")
    ap.add_argument("--two-call", action="store_true",
                    help="decode: run the step as gdn_conv1d_varlen + gdn_scan_varlen instead of one "
                         "gdn_decode_step launch (the default, faster at every batch size measured)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain 1 GiB device-to-device copy (reference for HBM counters and achievable bandwidth)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards with no exchange across sequences or key-head groups; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        print(json.dumps(copy_calibration(torch, args.steps, args.warmup)), flush=True)
        return
    w = workloads.NAMED[args.workload]()
    # a decode step (at most one token per sequence) can run as one fused launch
    fused = (not args.two_call and args.workload == "decode" and args.path in ("auto", "decode")
             and int(np.max(np.diff(w.offsets))) <= 1)
    p = Path(w, torch, args.path, fused_step=fused)
    ms, scan_ms, used, _ = time_path(p, args.steps, args.warmup)
    tokens_per_s = w.N / (ms * 1e-3)
    line = {
        "metric": "gated-delta varlen scan tokens/s + achieved HBM GB/s (decode & prefill)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 I/O, f32 state and arithmetic" if w.io == "bf16" else w.io,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "HQ": w.HQ, "H": w.H, "K": w.K, "V": w.V,
                   "conv_W": w.W, "conv_D": w.D, "path": used, "parallelism": "single GPU"},
        "roofline": roofline(w, scan_ms, args.workload, "decode_col_kernel (conv + recurrence)" if fused else "scan_kernel",
                             fused_step=fused),
    }
    if used not in ("decode", "decode_step"):
        line["compute_roofline"] = compute_roofline(w, scan_ms, used)
    # the achievable HBM rate on this machine: a plain 1 GiB device copy, timed the same way
    cp = copy_calibration(torch, 20, 5)
    line["roofline"]["measured_copy_gb_per_s"] = cp["gb_per_s"]
    line["roofline"]["frac_of_measured_copy"] = round(line["roofline"]["achieved"] / cp["gb_per_s"], 4)
    if not args.no_also and args.workload == "decode":
        del p
        torch.cuda.empty_cache()
        # warmups long enough for the clocks to settle (a 2-step warmup reads ~15% slow)
        line["also"] = {"prefill": secondary(torch, workloads.varlen_prefill(), max(3, args.steps // 10), 20, "prefill"),
                        "long": secondary(torch, workloads.long_single(), 10, 10, "long"),
                        "decode_step_fused_vs_two_call": fused_comparison(torch),
                        "speculative_verify_capture": verify_comparison(torch),
                        "mixed_batch": mixed_comparison(torch),
                        "per_key_decay": per_key_comparison(torch),
                        "strided_qkv": strided_comparison(torch),
                        "cache_flushed": cache_flushed(torch),
                        "prepare": prepare_measurement(torch)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
