"""Benchmark: one ring rank's share of causal attention on one MI355X.

A step is one pass of the whole path for the rank under study: the layout
permutation of its query chunk and of every K/V chunk out of global order
(ra_layout_permute), the accumulator start state, one ra_step_fwd per chunk
in ring order, ra_finalize, and -- for the workloads that have one -- the
backward ring (ra_bwd_delta + one ra_step_bwd per chunk). Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts.

The rank permutes its own Q, K and V chunks on the launch stream. The K/V
chunks of the other ranks -- in a real ring each permuted by its owner at the
same time and then received -- are permuted on a second stream (default
priority), each while the step before the one that uses it runs; each step
waits for its chunk's event. --serial-permute runs every permutation on the launch
stream before the first step instead.

Prints one JSON line. `value` is causal-effective TFLOP/s of the whole step
(forward 4*D FLOP per visible (query, key) pair per query head, backward
10*D), from the mean step time of the timed region; `breakdown` also gives
the median of the per-step times (HIP events on the launch stream).
`roofline` is the dominant kernel timed live with HIP events on the stream it
runs on: the forward step kernel (ra_step_fwd), or for the workloads with a
backward the backward step (ra_step_bwd, its two kernels), whose time
dominates there. It also carries the step's algorithmic HBM bytes per launch
and the rate they imply. `cpu_baseline` is the fp64 oracle timed on a bounded
sample of the same workload on the host cores. `breakdown` adds the layout
permutation's rate, the backward at 8*D per pair (without the recomputed S)
next to the 10*D figure, the shader clock and socket power read from the
device over untimed steps run after the timed region (with the peak scaled to
the clock, the power cap, and the fraction of the window in which the package
power limit was holding the clock down), and the rotary position embedding of
the rank's K chunks, timed after the step as a separate pass.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import seeded_inputs as si  # noqa: E402
from ring_attention_ra_amd import _lib, configs, ring  # noqa: E402

PEAK_HBM_TBS = 8.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, 2.4 GHz
PEAK_HBM_GBS = 8000.0
PEAK_CLOCK_MHZ = 2400.0  # the clock the bf16 peak is quoted at


class ClockReader:
    """Reads the GPU's shader clock (MHz, mean over the XCDs) from the
    device's metrics table through amdsmi; None when amdsmi is missing or
    refuses."""

    def __init__(self):
        self._api = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if len(handles) == 1 or (bus is not None and int(bdf.split(":")[1], 16) == int(bus)):
                    self._handle = h
                    self._api = amdsmi
        except Exception:  # noqa: BLE001 - the clock is optional
            self._api = None

    def read(self):
        """(shader clock MHz, socket power W or None), or None."""
        if self._api is None:
            return None
        try:
            m = self._api.amdsmi_get_gpu_metrics_info(self._handle)
        except Exception:  # noqa: BLE001
            return None
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and 0 < c < 10000]
        if clks:
            mhz = sum(clks) / len(clks)
        else:
            c = m.get("current_gfxclk")
            if not (isinstance(c, int) and 0 < c < 10000):
                return None
            mhz = float(c)
        pw = m.get("current_socket_power")
        return mhz, (float(pw) if isinstance(pw, int) and 0 < pw < 100000 else None)

    def power_cap_w(self):
        if self._api is None:
            return None
        try:
            cap = self._api.amdsmi_get_power_cap_info(self._handle).get("power_cap")
        except Exception:  # noqa: BLE001
            return None
        return cap / 1e6 if isinstance(cap, int) and cap > 0 else None

    def ppt_counters(self):
        """(accumulation counter, of which with the package power limit
        active), from the device's violation status; None if unavailable."""
        if self._api is None:
            return None
        try:
            v = self._api.amdsmi_get_violation_status(self._handle)
        except Exception:  # noqa: BLE001
            return None
        acc, ppt = v.get("acc_counter"), v.get("acc_ppt_pwr")
        return (acc, ppt) if isinstance(acc, int) and isinstance(ppt, int) else None


def clock_window(step, reader, seconds, ms_per_step, settle=1.0):
    """The shader clock and socket power under the same load: after the timed
    region, run untimed steps for about `seconds`, keeping two steps in
    flight, and read the clock and power after each. The device's metrics
    table refreshes only now and then, so readings from the first `settle`
    seconds (which may still describe the idle gap before the window) are
    dropped; the clock is averaged over the distinct readings left, the power
    over all of them. The package power limit's active fraction comes from the
    violation counters read at `settle` and at the end."""
    if reader.read() is None:
        return None
    n = max(20, int(seconds * 1e3 / max(ms_per_step, 1e-3)))
    done = []
    samples = []
    ppt0 = None
    t0 = time.perf_counter()
    for i in range(n):
        step(False)
        ev = torch.cuda.Event()
        ev.record()
        done.append(ev)
        if i >= 2:
            done[i - 2].synchronize()
            if time.perf_counter() - t0 >= settle:
                if ppt0 is None:
                    ppt0 = reader.ppt_counters()
                v = reader.read()
                if v is not None:
                    samples.append(v)
    ppt1 = reader.ppt_counters()
    torch.cuda.synchronize()
    if not samples:
        return None
    distinct = [v for k, v in enumerate(samples) if k == 0 or v != samples[k - 1]]
    mhz = [v[0] for v in distinct]
    watts = [v[1] for v in samples if v[1] is not None]
    out = {"gfx_mhz_mean": round(statistics.fmean(mhz), 1), "gfx_mhz_min": round(min(mhz), 1),
           "gfx_mhz_max": round(max(mhz), 1), "readings": len(distinct), "window_steps": n,
           "source": "amdsmi gpu metrics (current_gfxclks, current_socket_power) and violation status, "
                     f"untimed steps after the timed region, readings after the first {settle:g} s"}
    if watts:
        out["socket_power_w_mean"] = round(statistics.fmean(watts), 1)
        out["socket_power_w_max"] = round(max(watts), 1)
        out["power_cap_w"] = reader.power_cap_w()
    if ppt0 and ppt1 and ppt1[0] > ppt0[0]:
        out["power_limit_active_frac"] = round((ppt1[1] - ppt0[1]) / (ppt1[0] - ppt0[0]), 3)
    return out


def kernel_source_sha256(source):
    """sha256 of a kernel source file followed by the shared tile header it includes."""
    h = hashlib.sha256()
    for name in (source, "tile_common.h"):
        with open(os.path.join(ROOT, "ring_attention_ra_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def visible_pairs_per_chunk(w, pos_cpu):
    """Visible (query, key) pairs per head for each ring step of the rank."""
    qp = pos_cpu[w.rank]
    out = []
    for s in ring.ring_schedule(w.n_ranks, w.rank):
        kp = pos_cpu[s]
        if w.causal:
            out.append(int(torch.searchsorted(kp, qp, right=True).sum()))
        else:
            out.append(int(qp.numel() * kp.numel()))
    return out


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=str(configs.HEADLINE.index),
                    help="workload index (1-6) or name; default: the 128K zig-zag share")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the clock reading window after the timed region")
    ap.add_argument("--serial-permute", action="store_true",
                    help="permute every K/V chunk on the launch stream before the first step")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="query rows in the CPU-baseline sample")
    ap.add_argument("--cpu-heads", type=int, default=6, help="heads in the CPU-baseline sample")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "step_kernel_traffic.json"),
                    help="JSON records of counter-measured HBM bytes per launch of a step kernel; a record is "
                         "used only when it was taken on this workload and on the current kernel source")
    return ap.parse_args()


def cpu_baseline(w, q, k, v, rows_n, heads_n):
    """Time the fp64 oracle on a bounded sample: `heads_n` heads x `rows_n`
    query rows spread evenly over the rank's chunk, all their visible keys."""
    import numpy as np

    import oracle

    g = w.heads_q // w.heads_kv
    heads = sorted({int(x) for x in np.linspace(0, w.heads_q - 1, heads_n).round()})
    rows = np.unique(np.linspace(0, w.chunk - 1, rows_n).round().astype(np.int64))

    def host(t, hs):
        out = np.zeros(tuple(t.shape), dtype=np.float32)
        for h in sorted(set(hs)):
            out[:, h] = t[:, h].float().cpu().numpy()
        return out

    qh, kh, vh = host(q, heads), host(k, [h // g for h in heads]), host(v, [h // g for h in heads])
    slopes = oracle.alibi_slopes(w.heads_q) if w.alibi else None
    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.attention_rank_share(qh, kh, vh, w.n_ranks, w.rank, w.layout, w.causal, w.scale, slopes,
                                rows=rows, heads=heads, threads=threads)
    dt = time.perf_counter() - t0
    pos = oracle.rank_positions(w.seq_len, w.n_ranks, w.rank, w.layout)[rows]
    pairs = int((pos + 1).sum()) if w.causal else rows.size * w.seq_len
    flops = 4.0 * w.head_dim * pairs * len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle forward, {len(heads)} heads x {rows.size} query rows spread over the "
                      f"rank's {w.chunk}-row chunk ({pairs * len(heads)} visible pairs, {dt:.1f} s)",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one rank's share on ONE GPU; --gpus {args.gpus} is not supported "
              "(the ring is simulated on a single device)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    _lib.lib()
    w = configs.get(int(args.workload)) if args.workload.isdigit() else configs.get(args.workload)
    dev = torch.device("cuda:0")
    dt = si.torch_dtype(w.dtype)
    b, hq, hkv, d, s, n, c = w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seq_len, w.n_ranks, w.chunk

    # ---- inputs, resident in HBM ----
    q_g = si.normal((b, hq, s, d), si.seed_for(w.index, si.Q_STREAM), w.std, w.dtype, dev)
    k_g = si.normal((b, hkv, s, d), si.seed_for(w.index, si.K_STREAM), w.std, w.dtype, dev)
    v_g = si.normal((b, hkv, s, d), si.seed_for(w.index, si.V_STREAM), w.std, w.dtype, dev)
    d_o = si.normal((b, hq, c, d), si.seed_for(w.index, si.DO_STREAM), 1.0, w.dtype, dev) if w.backward else None
    slopes = ring.alibi_slopes(hq, dev) if w.alibi else None

    # ---- buffers, allocated once ----
    q_loc = torch.empty((b, hq, c, d), dtype=dt, device=dev)
    k_ch = torch.empty((n, b, hkv, c, d), dtype=dt, device=dev)
    v_ch = torch.empty_like(k_ch)
    pos = torch.empty((n, c), dtype=torch.int32, device=dev)
    dims = _lib.make_dims(b, hq, hkv, d, c, c, dt)
    o_acc = torch.empty((b, hq, c, d), dtype=torch.float32, device=dev)
    m = torch.empty((b, hq, c), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    o = torch.empty((b, hq, c, d), dtype=dt, device=dev)
    lse = torch.empty_like(m)
    if w.backward:
        delta = torch.empty_like(m)
        dq = torch.empty((b, hq, c, d), dtype=torch.float32, device=dev)
        dk = torch.empty((n, b, hkv, c, d), dtype=torch.float32, device=dev)
        dv = torch.empty_like(dk)
    sched = ring.ring_schedule(n, w.rank)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=dev)  # default priority

    # Every library call of a step is checked and marshalled once here
    # (_lib.bind); the loop then only re-issues the calls, so that on the
    # short chunks the host keeps ahead of the GPU.
    bind = _lib.bind
    perm_own = [bind(_lib.ra_layout_permute, q_g, q_loc, None, b * hq, s, d, n, w.layout, rank=w.rank)]
    if args.serial_permute:
        perm_own += [bind(_lib.ra_layout_permute, k_g, k_ch, pos, b * hkv, s, d, n, w.layout, rank=-1),
                     bind(_lib.ra_layout_permute, v_g, v_ch, None, b * hkv, s, d, n, w.layout, rank=-1)]
    else:
        perm_own += [bind(_lib.ra_layout_permute, k_g, k_ch[w.rank], pos[w.rank], b * hkv, s, d, n, w.layout,
                          rank=w.rank),
                     bind(_lib.ra_layout_permute, v_g, v_ch[w.rank], None, b * hkv, s, d, n, w.layout,
                          rank=w.rank)]
    # The next chunk in ring order is permuted on the side stream while a
    # step runs, the way it would arrive during it.
    perm_side = {nxt: [bind(_lib.ra_layout_permute, k_g, k_ch[nxt], pos[nxt], b * hkv, s, d, n, w.layout,
                            rank=nxt, stream=side),
                       bind(_lib.ra_layout_permute, v_g, v_ch[nxt], None, b * hkv, s, d, n, w.layout, rank=nxt,
                            stream=side)]
                 for nxt in sched[1:]}
    init_call = bind(_lib.ra_state_init, dims, o_acc, m, l)
    fwd_calls = [bind(_lib.ra_step_fwd, dims, q_loc, k_ch[src], v_ch[src], pos[w.rank], pos[src], w.causal,
                      w.scale, slopes, o_acc, m, l) for src in sched]
    fin_call = bind(_lib.ra_finalize, dims, o_acc, m, l, o, lse)
    if w.backward:
        delta_call = bind(_lib.ra_bwd_delta, dims, o, d_o, delta)
        bwd_calls = [bind(_lib.ra_step_bwd, dims, q_loc, k_ch[src], v_ch[src], pos[w.rank], pos[src], w.causal,
                          w.scale, slopes, d_o, lse, delta, dq, dk[src], dv[src]) for src in sched]
    # Events that only order the two streams, reused every step.
    go = [torch.cuda.Event() for _ in sched]
    ready = [torch.cuda.Event() for _ in sched]

    fwd_events, bwd_events, perm_events, side_events, step_events = [], [], [], [], []
    pool = []  # timing events, created before the timed steps

    def ev(on=None):
        e = pool.pop() if pool else torch.cuda.Event(enable_timing=True)
        e.record(stream if on is None else on)
        return e

    def step(timed):
        if timed:
            step_events.append(ev())
            perm_events.append(ev())
        for call in perm_own:
            call()
        if timed:
            perm_events.append(ev())
        init_call()
        for j in range(n):
            if j > 0 and not args.serial_permute:
                stream.wait_event(ready[j])
            if not args.serial_permute and j + 1 < n:
                # It starts once every earlier use of its buffers (all on the
                # launch stream) is behind it.
                go[j + 1].record(stream)
                side.wait_event(go[j + 1])
                if timed:
                    side_events.append(ev(side))
                for call in perm_side[sched[j + 1]]:
                    call()
                ready[j + 1].record(side)
                if timed:
                    side_events.append(ev(side))
            if timed:
                fwd_events.append(ev())
            fwd_calls[j]()
            if timed:
                fwd_events.append(ev())
        fin_call()
        if w.backward:
            delta_call()
            dq.zero_()
            dk.zero_()
            dv.zero_()
            for j in range(n):
                if timed:
                    bwd_events.append(ev())
                bwd_calls[j]()
                if timed:
                    bwd_events.append(ev())
        if timed:
            step_events.append(ev())

    for _ in range(args.warmup):
        step(False)
    per_step = 4 + 2 * n + (2 * (n - 1) if not args.serial_permute else 0) + (2 * n if w.backward else 0)
    pool.extend(torch.cuda.Event(enable_timing=True) for _ in range(per_step * args.steps))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    clk = None if args.no_clock else clock_window(step, ClockReader(), 3.0, ms_per_step)

    pairs = visible_pairs_per_chunk(w, pos.cpu())
    fwd_flops = 4.0 * d * hq * b * sum(pairs)
    bwd_flops = 10.0 * d * hq * b * sum(pairs) if w.backward else 0.0
    step_flops = fwd_flops + bwd_flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    def pair_ms(evs):
        return [evs[i].elapsed_time(evs[i + 1]) for i in range(0, len(evs), 2)]

    step_ms = pair_ms(step_events)
    median_ms = statistics.median(step_ms)
    fwd_ms = pair_ms(fwd_events)
    fwd_launch_ms = sum(fwd_ms) / len(fwd_ms)
    fwd_total_ms = sum(fwd_ms) / args.steps
    fwd_tflops = fwd_flops / (fwd_total_ms * 1e-3) / 1e12
    perm_ms = sum(pair_ms(perm_events)) / args.steps
    esz = q_loc.element_size()
    if args.serial_permute:
        perm_bytes = 2.0 * (q_loc.numel() + k_ch.numel() + v_ch.numel()) * esz + pos.numel() * 4
    else:
        perm_bytes = 2.0 * (q_loc.numel() + k_ch[0].numel() + v_ch[0].numel()) * esz + pos[0].numel() * 4
        side_ms = sum(pair_ms(side_events)) / args.steps
        side_bytes = 2.0 * (n - 1) * (k_ch[0].numel() + v_ch[0].numel()) * esz + (n - 1) * pos[0].numel() * 4

    # Algorithmic HBM bytes of one forward step through the step API: a step
    # with a visible pair reads Q and the K/V chunk, and reads and writes the
    # fp32 state (o_acc, m, l); a fully masked step moves nothing.
    q_bytes = b * hq * c * d * esz
    kv_bytes = 2 * b * hkv * c * d * esz
    state_bytes = 2 * (b * hq * c * d * 4 + 2 * b * hq * c * 4)
    fwd_alg_bytes = sum(q_bytes + kv_bytes + state_bytes for p_ in pairs if p_ > 0) / n

    def traffic_for(kernel, source):
        """Counter-measured bytes per launch, if a record matches the workload
        and the kernel source as it is now."""
        if not (args.traffic and os.path.exists(args.traffic)):
            return None
        with open(args.traffic) as f:
            recs = json.load(f).get("records", [])
        sha = kernel_source_sha256(source)
        for rec in recs:
            if rec.get("kernel") == kernel and rec.get("workload") == w.name and \
                    rec.get("kernel_source_sha256") == sha:
                return rec.get("bytes_per_launch")
        return None

    extra = {
        "median_ms_per_step": round(median_ms, 4),
        "value_at_median": round(step_flops / (median_ms * 1e-3) / 1e12, 3),
        "step_kernel_tflops": round(fwd_tflops, 2),
        "step_kernel_frac_of_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "step_kernel_ms_per_step": round(fwd_total_ms, 4),
        "step_kernel_launch_ms": round(fwd_launch_ms, 4),
        "step_kernel_alg_bytes_per_launch": int(fwd_alg_bytes),
        "step_kernel_hbm_gbs": round(fwd_alg_bytes / (fwd_launch_ms * 1e-3) / 1e9, 1),
        "step_kernel_frac_of_hbm": round(fwd_alg_bytes / (fwd_launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "permute_ms_per_step": round(perm_ms, 4),
        "permute_gbs": round(perm_bytes / (perm_ms * 1e-3) / 1e9, 1),
        "permute_scope": "every chunk, launch stream" if args.serial_permute else "own Q/K/V chunks, launch stream",
        "visible_pairs_per_head": sum(pairs),
        "fwd_flop_per_step": fwd_flops,
    }
    if clk:
        peak_clk = PEAK_BF16_TFLOPS * clk["gfx_mhz_mean"] / PEAK_CLOCK_MHZ
        clk["bf16_peak_at_clock_tflops"] = round(peak_clk, 1)
        clk["value_frac_of_peak_at_clock"] = round(value / peak_clk, 4)
    extra["clock"] = clk
    if not args.serial_permute:
        # The other ranks' chunks on the side stream, one per step, each
        # overlapped with a step (so not a rate of its own).
        extra["permute_other_ranks"] = {"stream": "side, overlapped with the steps",
                                        "ms_per_step": round(side_ms, 4),
                                        "gbs_while_overlapped": round(side_bytes / (side_ms * 1e-3) / 1e9, 1)}
    # Rotary position embedding of the rank's K chunks (every chunk by its own
    # global positions), out of place, as a separate HBM-bound pass: not part
    # of the step above, timed after it with HIP events on the same stream.
    k_rot = torch.empty_like(k_ch)
    rope_ev = []
    for it in range(4):
        if it == 1:
            rope_ev.append(torch.cuda.Event(enable_timing=True))
            rope_ev[-1].record()
        for s_ in range(n):
            _lib.ra_rope(k_ch[s_], k_rot[s_], pos[s_])
    rope_ev.append(torch.cuda.Event(enable_timing=True))
    rope_ev[-1].record()
    torch.cuda.synchronize()
    rope_ms = rope_ev[0].elapsed_time(rope_ev[1]) / 3
    rope_bytes = 2.0 * k_ch.numel() * k_ch.element_size() + pos.numel() * 4
    del k_rot
    extra["rope"] = {"kernel": "rope_kernel (ra_rope)", "tensor": "K chunks [N,B,Hkv,C,D]", "ms": round(rope_ms, 4),
                     "gbs": round(rope_bytes / (rope_ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm": round(rope_bytes / (rope_ms * 1e-3) / 1e12 / PEAK_HBM_TBS, 4)}

    roofline = {
        "bound": "mfma",
        "achieved": round((fwd_flops / n) / (fwd_launch_ms * 1e-3) / 1e12, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": None,
        "traffic": traffic_for("fwd_bf16_kernel", "fwd_bf16.hip"),
        "kernel": "fwd_bf16_kernel (ra_step_fwd)",
        "launch_ms": round(fwd_launch_ms, 4),
        "flop_per_launch": fwd_flops / n,
        "alg_bytes_per_launch": int(fwd_alg_bytes),
    }
    if w.backward:
        bwd_ms = pair_ms(bwd_events)
        bwd_total_ms = sum(bwd_ms) / args.steps
        bwd_launch_ms = sum(bwd_ms) / len(bwd_ms)
        extra["bwd_kernel_ms_per_step"] = round(bwd_total_ms, 4)
        extra["bwd_kernel_tflops"] = round(bwd_flops / (bwd_total_ms * 1e-3) / 1e12, 2)
        # The same time counted without the recomputed S (8*D per visible pair).
        extra["bwd_kernel_tflops_8d"] = round(0.8 * bwd_flops / (bwd_total_ms * 1e-3) / 1e12, 2)
        extra["bwd_flop_per_step"] = bwd_flops
        extra["fwd_roofline"] = dict(roofline, frac=round(roofline["achieved"] / PEAK_BF16_TFLOPS, 4))
        # The backward step dominates the time here: it is the roofline kernel.
        roofline = {
            "bound": "mfma",
            "achieved": round((bwd_flops / n) / (bwd_launch_ms * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": None,
            "traffic": traffic_for("bwd_step (bwd_dkdv_kernel + bwd_dq_kernel)", "bwd_bf16.hip"),
            "kernel": "bwd_dkdv_kernel + bwd_dq_kernel (ra_step_bwd)",
            "launch_ms": round(bwd_launch_ms, 4),
            "flop_per_launch": bwd_flops / n,
        }
    roofline["frac"] = round(roofline["achieved"] / PEAK_BF16_TFLOPS, 4)

    result = {
        "metric": "causal attention TFLOP/s per ring-rank share + % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0, std^2) inputs, see seeded_inputs.py)",
        "config": w.describe(),
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "breakdown": extra,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, q_g, k_g, v_g, args.cpu_rows, args.cpu_heads)
        cb["value"] = round(cb["value"], 5)
        cb.pop("seconds")
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
