"""Benchmark of the FlashAttention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-s SECONDS] [--workload NAME]
                    [--no-cpu] [--no-probe]

Workloads (one step = one call over the whole batch, inputs resident in HBM before timing):

    headline          forward, B=4 H=16 N=4096 d=64 bf16 (the default line)
    headline_f16      the same in fp16
    headline_literal  the headline with the literal recurrence: exact running max, l and acc
                      rescaled by exp(m_old - m_new) whenever the maximum grows
    long_seq          forward, B=1 H=32 N=16384 d=128 bf16, K x3
    causal            the headline shape under the causal mask (4*d flops per visible pair)
    single_head       forward, B=H=1 N=256 d=64 fp32 (latency-bound; reported in microseconds)
    one_query         one query of d=64 against 4096 keys, fp32 (microseconds)
    batched_queries   4096 queries sharing those 4096 keys, fp32 (TFLOP/s against the fp32 peak)
    decode, decode_lse, gqa_decode
                      split-KV decode (16 ranges) + merge; (m, l, o) or (lse, o) states; GB/s
    bwd, bwd_causal, bwd_d128
                      fa_bwd at the headline shape / under the mask / at d=128 (10*d flops per pair)

Before the W warm-up steps, steps run back to back for --prewarm-s seconds (reported under
"prewarm"): the GPU's clock ramps up under sustained load, and a short run would otherwise time a
cold chip. The shader clock (amdsmi) is sampled around the timed region. After the timed region the
two probes of include/fa_probe.h measure the matrix-core and HBM-read ceilings of the same GPU in the
same process ("probe"; roofline.frac_of_probe). The cpu_baseline leg times the fp64 oracle on a
bounded sample of the same inputs in a pool of worker processes on the host's cores.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
FP32_VECTOR_PEAK_TFLOPS = 157.3  # published fp32 vector peak (counts packed fp32 FMAs)
MFMA_F32_PEAK_TFLOPS = 157.3    # published dense fp32 matrix-core peak
EVENT_STRIDE_MIN = 4            # kernel launch timed by an event pair in at most every 4th timed step,
EVENT_SAMPLES = 16              # and in about 16 steps of a longer timed region
HBM_PEAK_GBS = 8000.0
METRIC = "FA fwd TFLOP/s (4*B*H*N^2*d) at N=4096,d=64 bf16; % of MFMA peak"

FWD_WORKLOADS = ("headline", "headline_f16", "headline_literal", "long_seq", "causal", "single_head", "one_query",
                 "batched_queries")
DECODE_WORKLOADS = ("decode", "decode_lse", "gqa_decode")
BWD_WORKLOADS = ("bwd", "bwd_causal", "bwd_d128")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--prewarm-s", type=float, default=2.0,
                   help="seconds of back-to-back steps before the warm-up steps (clock ramp); 0 to skip")
    p.add_argument("--workload", default="headline", choices=FWD_WORKLOADS + DECODE_WORKLOADS + BWD_WORKLOADS)
    p.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    p.add_argument("--no-probe", action="store_true", help="skip the matrix-core and HBM probes")
    p.add_argument("--cpu-budget-s", type=float, default=20.0, help="wall-time budget of the cpu_baseline leg")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="before warm-up, run one plain device copy of MIB MiB (reads MIB, writes MIB): the "
                        "reference dispatch that scales the HBM byte counters of a profiling run")
    return p.parse_args()


# ---------------------------------------------------------------------------
# evidence records
# ---------------------------------------------------------------------------

def device_code_hash(*names):
    """Hash of the device code a kernel is built from: the named sources plus the internal headers, with
    comments and blank space removed, so that a comment-only edit keeps the hash and any code edit changes it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "flashattention_forward_02_amd", "csrc")
    for n in tuple(names) + ("fa_internal.h", "mfma_common.h"):
        text = open(os.path.join(csrc, n), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(n.encode() + b"\0" + text.encode() + b"\0")
    return h.hexdigest()[:16]


def traffic_for(kernel_key, src_hash):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was taken on this exact device code."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    if not rec or rec.get("device_code_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


class GfxClock:
    """Current shader (GFX) clock of the GPU behind cuda:0, read through amdsmi; None when unavailable."""

    def __init__(self, torch):
        self.h = None
        self.err = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            want = None
            try:
                pr = torch.cuda.get_device_properties(0)
                want = (int(getattr(pr, "pci_domain_id", 0)), int(pr.pci_bus_id), int(pr.pci_device_id))
            except Exception:
                pass
            for hd in handles:
                if want is None:
                    break
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(hd)        # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.h = hd
            if self.h is None and len(handles) == 1:
                self.h = handles[0]
            self.amdsmi = amdsmi
        except Exception as e:  # no amdsmi, no permission: the figure is reported as null
            self.err = repr(e)[:200]

    def read(self):
        if self.h is None:
            return None
        try:
            return int(self.amdsmi.amdsmi_get_clock_info(self.h, self.amdsmi.AmdSmiClkType.GFX)["clk"])
        except Exception:
            return None


def cpu_model():
    try:
        out = os.popen("lscpu 2>/dev/null").read()
        for ln in out.splitlines():
            if ln.startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


# ---------------------------------------------------------------------------
# cpu_baseline: the fp64 oracle in a pool of worker processes
# ---------------------------------------------------------------------------

def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)           # one BLAS thread per worker process
    global _ORACLE
    import oracle as _o
    _ORACLE = _o


def _oracle_task(task):
    """One task of the cpu_baseline leg: oracle rows r0..r1 of one head (forward) or one whole head (backward)."""
    import numpy as np
    kind, key, arrays, scale, causal = task
    t0 = time.perf_counter()
    if kind == "fwd":
        q, k, v, r0, Nq = arrays
        last = None
        if causal:
            last = _ORACLE.causal_last_key(np.arange(r0, r0 + q.shape[0]), Nq, k.shape[0])
        ref = _ORACLE.attention_rows_fp64(q, k, v, scale, last_key=last)[0]
    else:
        q, k, v, do = arrays
        ref = _ORACLE.attention_backward_fp64(q[None, None], k[None, None], v[None, None], do[None, None], scale,
                                              causal=causal)[:3]
    return key, ref, time.perf_counter() - t0


def cpu_baseline(tasks, flops_of, budget_s, compare):
    """Run oracle tasks in a pool of worker processes for about ``budget_s`` seconds of wall time (after the
    workers start): at most two tasks per worker are in flight, no task is submitted once the budget is spent,
    and the tasks in flight are finished. Returns (cpu_baseline record, parity record)."""
    import multiprocessing as mp
    from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait
    workers = max(1, min(len(os.sched_getaffinity(0)), 16))
    # spawn: fresh interpreters, nothing of this process's GPU state is inherited
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"), initializer=_worker_init) as ex:
        list(ex.map(abs, range(workers)))      # workers up and the oracle imported before the clock starts
        t0 = time.perf_counter()
        done, flops, errs, nxt, pending, last_note = 0, 0.0, [], 0, set(), t0
        while nxt < len(tasks) or pending:
            while nxt < len(tasks) and len(pending) < 2 * workers and time.perf_counter() - t0 < budget_s:
                pending.add(ex.submit(_oracle_task, tasks[nxt]))
                nxt += 1
            if not pending:
                break
            finished, pending = wait(pending, return_when=FIRST_COMPLETED)
            for fu in finished:
                key, ref, _ = fu.result()
                done += 1
                flops += flops_of(key)
                errs.extend(compare(key, ref))
            if time.perf_counter() - last_note > 5.0:
                last_note = time.perf_counter()
                print(f"cpu_baseline: {done} of {len(tasks)} tasks, {last_note - t0:.1f} s", file=sys.stderr, flush=True)
        dt = time.perf_counter() - t0
    max_abs = max(e[0] for e in errs)
    rel = (sum(e[1] ** 2 for e in errs) ** 0.5) / max(sum(e[2] ** 2 for e in errs) ** 0.5, 1e-300)
    return ({"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "cpu_model": cpu_model(),
             "host_cpus": os.cpu_count(), "kind": "oracle", "wall_s": dt, "tasks_done": done,
             "tasks_total": len(tasks)},
            {"max_abs": max_abs, "rel_l2": rel, "tasks_checked": done})


def fwd_oracle_tasks(w, q, k, v, rows_per_task):
    import seeded_inputs as si
    tasks = []
    for b in range(w.B):
        for h in range(w.H):
            hk = h // (w.H // w.kv_heads)
            kh, vh = si.torch_to_f64(k[b, hk]), si.torch_to_f64(v[b, hk])
            qh = si.torch_to_f64(q[b, h])
            for r0 in range(0, w.Nq, rows_per_task):
                r1 = min(w.Nq, r0 + rows_per_task)
                tasks.append(("fwd", (b, h, r0, r1), (qh[r0:r1], kh, vh, r0, w.Nq), w.scale, w.causal))
    return tasks


def err_triplet(got, ref):
    import numpy as np
    return (float(np.max(np.abs(got - ref))), float(np.linalg.norm(got - ref)), float(np.linalg.norm(ref)))


# ---------------------------------------------------------------------------
# probes
# ---------------------------------------------------------------------------

def run_probes(torch, fa, stream):
    """Matrix-core and HBM-read ceilings of this GPU (include/fa_probe.h), best of 5 timed launches each."""
    res = {}
    flops, out = fa.probe_mfma_bf16(nblocks=2048, iters=1024)
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fa.probe_mfma_bf16(nblocks=2048, iters=1024, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    res["mfma_bf16_tflops"] = flops / (best * 1e-3) / 1e12
    flops, out = fa.probe_mfma_f32(nblocks=2048, iters=256)
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fa.probe_mfma_f32(nblocks=2048, iters=256, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    res["mfma_f32_tflops"] = flops / (best * 1e-3) / 1e12
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    rout = torch.empty(1024 * 256, dtype=torch.int32, device="cuda")
    nbytes = fa.probe_hbm_read(buf, nblocks=1024, out=rout)
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fa.probe_hbm_read(buf, nblocks=1024, out=rout)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    res["hbm_read_gbs"] = nbytes / (best * 1e-3) / 1e9
    res["what"] = ("fa_probe_mfma_bf16 (2048 workgroups x 4 waves x 1024 x 8 MFMAs 32x32x16), fa_probe_mfma_f32 "
                   "(2048 x 4 waves x 256 x 8 MFMAs 16x16x4 fp32) and fa_probe_hbm_read (4 GiB in 1024 contiguous 4 MiB chunks, nontemporal 16-byte loads), "
                   "best of 5 launches each")
    del buf
    return res


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def time_split_one_query(torch, fa, q, k, v, o_ref, scale, stream, S=16, calls=200):
    """The single query the split-KV way: S key ranges on S workgroups, then the merge.

    fa_fwd keeps one row on one workgroup (it takes no workspace), so its time is set by one compute
    unit's load rate; the decoding demo's blocks of 256 keys as 16 ranges spread the row over 16."""
    part_lse = torch.empty((S,) + tuple(q.shape[:3]), device=q.device, dtype=torch.float32)
    part_o = torch.empty((S,) + tuple(q.shape), device=q.device, dtype=torch.float32)
    o = torch.empty_like(o_ref)

    def call():
        fa.fwd_split_lse(q, k, v, S, scale=scale, workspace=(part_lse, part_o))
        fa.merge_lse(part_lse, part_o, out=o, return_lse=False)

    for _ in range(50):
        call()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / calls * 1e3)
    return {"us_per_call": best, "num_splits": S, "max_abs_diff_vs_fa_fwd": (o - o_ref).abs().max().item(),
            "what": f"fa_fwd_split_lse over {S} key ranges of {k.shape[2] // S} keys, then "
                    f"fa_merge_lse; best of 3 runs of {calls} back-to-back calls"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only; multi-GPU runs are not implemented "
                                   "(heads shard across GPUs with no exchange)"}))
        sys.exit(2)
    wname = args.workload
    if wname == "headline_literal":
        # rescale l and acc by 2^(m_ref_old - m_ref_new) whenever the running maximum grows (read once, at the
        # library's first call)
        os.environ["FA_RESCALE_THRESHOLD"] = "0"

    import torch
    import flashattention_forward_02_amd as fa
    import seeded_inputs as si

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = {"headline": si.HEADLINE_BF16, "headline_f16": si.HEADLINE_F16, "headline_literal": si.HEADLINE_BF16,
          "long_seq": si.LONG_SEQ_BF16, "causal": si.CAUSAL_BF16, "single_head": si.SINGLE_HEAD_FP32,
          "one_query": si.ONE_QUERY_LONG_KEYS, "batched_queries": si.BATCHED_QUERIES_LONG_KEYS,
          "decode": si.DECODE_BF16, "decode_lse": si.DECODE_BF16, "gqa_decode": si.GQA_DECODE_BF16,
          "bwd": si.BWD_BF16, "bwd_causal": si.BWD_CAUSAL_BF16, "bwd_d128": si.BWD_D128_BF16}[wname]
    is_bwd = wname in BWD_WORKLOADS
    is_decode = wname in DECODE_WORKLOADS
    lse_form = wname == "decode_lse"
    clock = GfxClock(torch)

    if is_decode:
        q, k, v = si.decode_inputs_device(wl, dev)
    else:
        if wname == "single_head":
            qh, kh, vh = si.single_head_fp32()
        elif wname in ("one_query", "batched_queries"):
            qh, kh, vh = si.one_query_long_keys(batched=wname == "batched_queries")
        else:
            qh, kh, vh = si.workload_inputs(wl)
        q, k, v = qh.to_torch(dev), kh.to_torch(dev), vh.to_torch(dev)
        del qh, kh, vh
        if is_bwd:
            dout = si.grad_output(wl).to_torch(dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        n_el = args.copy_calibration * 2 ** 20 // 4
        src = torch.ones(n_el, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if is_decode:
        S = wl.num_splits
        pm = torch.empty((S, wl.B, wl.H, wl.Nq), device=dev, dtype=torch.float32)
        pl = torch.empty_like(pm)
        po = torch.empty((S, wl.B, wl.H, wl.Nq, wl.d), device=dev, dtype=torch.float32)
        o = torch.empty((wl.B, wl.H, wl.Nq, wl.d), device=dev, dtype=torch.float32)
        order = si.merge_order(wl.seed, S)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            if lse_form:
                fa.fwd_split_lse(q, k, v, S, scale=wl.scale, workspace=(pm, po))
            else:
                fa.fwd_split(q, k, v, S, scale=wl.scale, workspace=(pm, pl, po))
            if ev is not None:
                ev[1].record(stream)
            if lse_form:
                fa.merge_lse(pm, po, order=order, out=o, return_lse=False)
            else:
                fa.merge_states(pm, pl, po, order=order, out=o)
    elif is_bwd:
        o, lse = fa.fwd_lse(q, k, v, scale=wl.scale, causal=wl.causal)
        grads = (torch.empty((wl.B, wl.H, wl.Nq, wl.d), device=dev, dtype=torch.float32),
                 torch.empty(k.shape, device=dev, dtype=torch.float32),
                 torch.empty(k.shape, device=dev, dtype=torch.float32),
                 torch.empty((wl.B, wl.H, wl.Nq), device=dev, dtype=torch.float32))

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            fa.bwd(q, k, v, o, dout, lse, scale=wl.scale, causal=wl.causal, out=grads)
            if ev is not None:
                ev[1].record(stream)
    else:
        o = torch.empty((wl.B, wl.H, wl.Nq, wl.d), device=dev, dtype=torch.float32)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            fa.fwd(q, k, v, scale=wl.scale, out=o, causal=wl.causal)
            if ev is not None:
                ev[1].record(stream)

    # pre-warm: back-to-back steps for a fixed wall time (the clock ramps up under load)
    clk_idle = clock.read()
    prewarm_steps, clk_prewarm = 0, []
    t_pw = time.perf_counter()
    if args.prewarm_s > 0:
        step()
        torch.cuda.synchronize()
        while time.perf_counter() - t_pw < args.prewarm_s:
            for _ in range(8):
                step()
            prewarm_steps += 8
            torch.cuda.synchronize()
            if prewarm_steps % 256 == 0:
                clk_prewarm.append(clock.read())
        prewarm_steps += 1
    prewarm_wall = time.perf_counter() - t_pw

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    clk_before = clock.read()

    # timed region: exactly K steps, synchronised on both sides
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    # an event pair around the dominant kernel's launch in every stride-th step of the timed region:
    # its average launch duration. A timed event pair costs the stream several microseconds: in every
    # step it lengthened the 9 us single-head steps by 80 %, in every 4th by 15 %, in every 12th by 4 %.
    stride = max(EVENT_STRIDE_MIN, args.steps // EVENT_SAMPLES)
    sampled = list(range(0, args.steps, stride))
    kev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record(stream)
    for i in range(args.steps):
        step(kev.get(i))
    ev_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clk_after = clock.read()
    gpu_ms = ev_start.elapsed_time(ev_end)
    ms_per_step = gpu_ms / args.steps
    launch_ms = sorted(a.elapsed_time(b) for a, b in kev.values())
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    launch_stats = {"avg_launch_ms": avg_launch_ms, "median_launch_ms": launch_ms[len(launch_ms) // 2],
                    "min_launch_ms": launch_ms[0], "launches_timed": len(launch_ms),
                    "launch_sampling": f"every {stride}th step of the timed region"}

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16", "data": "synthetic (seeded N(0,1) draws, see seeded_inputs)"}
    if wl.dtype != "bf16":
        result["dtype"] = {"f16": "fp16", "f32": "fp32"}[wl.dtype]
    if is_decode:
        split_ms = avg_launch_ms
        kv_bytes = 2.0 * wl.B * wl.kv_heads * wl.Nk * wl.d * 2
        state_vals = wl.d + (1 if lse_form else 2)           # (lse, o) or (m, l, o) per row and range
        alg_bytes = kv_bytes + wl.B * wl.H * wl.d * 2 + wl.num_splits * wl.B * wl.H * state_vals * 4
        step_bytes = alg_bytes + wl.num_splits * wl.B * wl.H * state_vals * 4 + wl.B * wl.H * wl.d * 4
        result.update({"metric": "split-KV decode HBM GB/s (K+V bytes / step time)" +
                                 (", partial states in the (lse, o) form" if lse_form else ""), "unit": "GB/s",
                       "value": kv_bytes / (ms_per_step * 1e-3) / 1e9,
                       "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "H_kv": wl.kv_heads, "Nq": wl.Nq,
                                  "Nk": wl.Nk, "d": wl.d, "num_splits": wl.num_splits,
                                  "merge_order": f"default_rng({wl.seed}).permutation({wl.num_splits})"}})
        achieved = alg_bytes / (split_ms * 1e-3) / 1e9
        kname = "decode_rows_kernel (split)" if wname == "gqa_decode" else "decode_kernel (split)"
        result["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": achieved,
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                              **launch_stats, "traffic": traffic_for(wname, device_code_hash("decode.hip"))}
        result["step_bytes"] = step_bytes
    elif is_bwd:
        flops = 2.5 * wl.flops   # 10*d per visible pair: the products S, dP, dV, dK, dQ
        shape = f"N={wl.Nq},d={wl.d} bf16"
        metric = f"FA bwd TFLOP/s (10*B*H*N^2*d: the products S, dP, dV, dK, dQ) at {shape}; % of MFMA peak"
        if wl.causal:
            metric = (f"FA bwd causal TFLOP/s (10*d per visible query-key pair, B*H*N(N+1)/2 pairs) at {shape}; "
                      "% of MFMA peak")
        result.update({"metric": metric, "unit": "TFLOP/s",
                       "value": flops / (ms_per_step * 1e-3) / 1e12,
                       "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.Nq, "d": wl.d,
                                  "causal": wl.causal, "grad_dtype": "fp32"}})
        achieved = flops / (avg_launch_ms * 1e-3) / 1e12
        kname = "fa_bwd (bwd_dq_pp + bwd_dkdv_pp)" if wl.d == 64 else "fa_bwd (bwd_delta + bwd_dq + bwd_dkdv16)"
        result["roofline"] = {"bound": "mfma", "kernel": kname, "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, **launch_stats,
                              "traffic": traffic_for(wname, device_code_hash("bwd.hip"))}
    else:
        flops = wl.flops
        tflops = flops / (ms_per_step * 1e-3) / 1e12
        achieved = flops / (avg_launch_ms * 1e-3) / 1e12
        cfg = {"workload": wl.name, "B": wl.B, "H": wl.H, "Nq": wl.Nq, "Nk": wl.Nk, "d": wl.d, "causal": wl.causal,
               "out_dtype": "fp32"}
        if wname in ("single_head", "one_query"):
            # latency-bound correctness shapes: the figure is the time per call
            what = ("B=H=1,N=256,d=64 fp32" if wname == "single_head"
                    else "one query, Nk=4096, d=64 fp32, keys in blocks of 256 in the pages' demo")
            result.update({"metric": f"FA fwd microseconds per call at {what}", "unit": "us",
                           "value": ms_per_step * 1e3, "higher_is_better": False, "config": cfg,
                           "tflops": tflops})
            # both run on fwd_f32_rows_kernel (one workgroup per query row: 256 rows of one head at
            # d = 64 is a launch it takes too)
            result["roofline"] = {"bound": "alu", "kernel": "fwd_f32_rows_kernel", "achieved": achieved,
                                  "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": achieved / FP32_VECTOR_PEAK_TFLOPS, **launch_stats, "traffic": None}
            if wname == "one_query":
                result["split_path"] = time_split_one_query(torch, fa, q, k, v, o, wl.scale, stream)
        elif wname == "batched_queries":
            result.update({"metric": "FA fwd TFLOP/s (4*Nq*Nk*d) at 4096 queries sharing Nk=4096 keys, d=64 fp32; "
                                     "% of the fp32 matrix-core peak", "unit": "TFLOP/s", "value": tflops, "config": cfg})
            result["roofline"] = {"bound": "mfma", "kernel": "fwd_f32_mfma_kernel", "achieved": achieved,
                                  "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": achieved / MFMA_F32_PEAK_TFLOPS, **launch_stats, "traffic": None}
        else:
            if wname == "long_seq":
                result["metric"] = "FA fwd TFLOP/s (4*B*H*N^2*d) at N=16384,d=128 bf16, K x3; % of MFMA peak"
            if wname == "headline_f16":
                result["metric"] = "FA fwd TFLOP/s (4*B*H*N^2*d) at N=4096,d=64 fp16; % of MFMA peak"
            if wname == "headline_literal":
                result["metric"] = ("FA fwd TFLOP/s (4*B*H*N^2*d) at N=4096,d=64 bf16, literal recurrence (exact "
                                    "running max, rescale on every increase); % of MFMA peak")
            if wname == "causal":
                result["metric"] = ("FA fwd causal TFLOP/s (4*d per visible query-key pair, B*H*N(N+1)/2 pairs) "
                                    "at N=4096,d=64 bf16; % of MFMA peak")
            result.update({"unit": "TFLOP/s", "value": tflops, "config": cfg})
            result["roofline"] = {"bound": "mfma", "kernel": "fwd_mfma_kernel", "achieved": achieved,
                                  "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": achieved / MFMA_BF16_PEAK_TFLOPS, **launch_stats,
                                  "traffic": traffic_for(wname, device_code_hash("fwd_mfma.hip"))}
    result["prewarm"] = {"seconds": prewarm_wall, "steps": prewarm_steps}
    result["sclk_mhz"] = {"idle": clk_idle, "prewarm": clk_prewarm[-8:], "before_timed": clk_before,
                          "after_timed": clk_after, "source": "amdsmi GFX clock" if clock.h is not None
                          else f"unavailable ({clock.err})"}
    result["wall_s_timed"] = wall

    if not args.no_probe:
        probe = run_probes(torch, fa, stream)
        result["probe"] = probe
        rf = result["roofline"]
        if rf["bound"] == "mfma":
            key = "mfma_f32_tflops" if rf["peak"] == MFMA_F32_PEAK_TFLOPS and wl.dtype == "f32" else "mfma_bf16_tflops"
            rf["frac_of_probe"] = rf["achieved"] / probe[key]
        elif rf["bound"] == "hbm":
            rf["frac_of_probe"] = rf["achieved"] / probe["hbm_read_gbs"]

    if not args.no_cpu and not is_decode:
        torch.cuda.synchronize()
        if is_bwd:
            qs, ks, vs, ds = (si.torch_to_f64(x) for x in (q, k, v, dout))
            gs = [si.torch_to_f64(g) for g in grads[:3]]
            tasks = [("bwd", (b, h), (qs[b, h], ks[b, h], vs[b, h], ds[b, h]), wl.scale, wl.causal)
                     for b in range(wl.B) for h in range(wl.H)]
            per_head = 10.0 * wl.visible_pairs * wl.d

            def compare(key, ref):
                b, h = key
                return [err_triplet(g[b, h], r[0, 0]) for g, r in zip(gs, ref)]

            base, check = cpu_baseline(tasks, lambda key: per_head, args.cpu_budget_s, compare)
            base["sample"] = (f"{check['tasks_checked']} of {len(tasks)} heads (dQ, dK, dV of all {wl.Nq} rows) of "
                              f"the same inputs, fp64 numpy, one head per task")
        else:
            rows = 1024 if wl.Nq * wl.Nk >= 4096 * 4096 else wl.Nq
            tasks = fwd_oracle_tasks(wl, q, k, v, rows)
            og = si.torch_to_f64(o)

            def pairs(key):
                b, h, r0, r1 = key
                if not wl.causal:
                    return float(r1 - r0) * wl.Nk
                off = wl.Nk - wl.Nq
                return float(sum(min(wl.Nk, i + off + 1) for i in range(r0, r1)))

            def compare(key, ref):
                b, h, r0, r1 = key
                return [err_triplet(og[b, h, r0:r1], ref)]

            base, check = cpu_baseline(tasks, lambda key: 4.0 * wl.d * pairs(key), args.cpu_budget_s, compare)
            base["sample"] = (f"{check['tasks_checked']} of {len(tasks)} tasks of {rows} query rows of one head "
                              f"each, the same inputs, fp64 numpy")
        result["cpu_baseline"] = base
        result["parity_sample"] = check
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
