"""Benchmark of the paged-attention hot path on one MI355X.

Step = one pa_forward call (persistent attention kernel that plans the call
itself + split merge) over one batch of synthetic Llama-3.1-8B-shaped decode
requests: 64 sequences, context lengths uniform in [500, 8192], 32 query / 8
KV heads, head dim 128, page size 16, bf16, pages in random physical order.
Inputs are resident in HBM before the timed region.

Printed (one JSON line): decode HBM GB/s of the whole step (algorithmic bytes
/ step time), the roofline entry of the attention kernel timed alone with HIP
events recorded by the library around that launch, the prefill half of the
metric (TFLOP/s of the Qwen3-235B-shaped prefill + extend requests of the
mixed batch, same method), one entry per other measured case (split-KV long
contexts, the mixed batch and its decode share, MLA decode, chunked extend,
small decode cases) with its roofline fraction, and the fp64 CPU oracle timed
on the host.
"""
import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn HBM GB/s (% of peak) + prefill attn TFLOP/s (% MFMA peak), 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
CSRC = os.path.join(ROOT, "paged_attention_kv_pa_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_times.json")
MALL_GUARD_BYTES = 512 << 20   # 2x the 256 MB last-level cache


def source_sha256():
    """sha256 over the HIP sources (names and contents) of the library."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


class HipEvents:
    """Raw hipEvent_t pairs (the library records them on its own launch stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0
            assert self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a, b))

    def elapsed_ms(self, i):
        t = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(t), self.pairs[i][0], self.pairs[i][1])
        assert rc == 0, rc
        return float(t.value)

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


def time_steps(call, steps, warmup, lib):
    """Run `call` warmup + steps times, then `steps` more times.

    Returns (ms per step, mean attention-kernel ms).  The step time comes from
    the first timed run, made exactly as a caller would make the calls.  The
    kernel time comes from the second, in which the library records a HIP event
    pair on its stream right around every attention-kernel launch; those
    markers widen the gaps between the launches of a step, so they stay out of
    the step timing.
    """
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    ev = HipEvents(steps)
    for i in range(steps):
        lib.pa_set_kernel_events(ev.pairs[i][0], ev.pairs[i][1])
        call()
    lib.pa_set_kernel_events(None, None)
    torch.cuda.synchronize()
    kern_ms = sum(ev.elapsed_ms(i) for i in range(steps)) / steps
    ev.close()
    return step_ms, kern_ms


def committed_entry(path, kernel_name, sha):
    """Entry of a committed profile summary, if taken on the current sources."""
    try:
        with open(path) as f:
            e = json.load(f).get(kernel_name)
        if e and e.get("source_sha256") == sha:
            return e
    except (OSError, ValueError):
        pass
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(b, nbytes):
    import oracle
    h = b.to("cpu")
    threads = oracle.max_threads()
    t = time.perf_counter()
    reps = 0
    while True:
        oracle.attention(h.q, h.k_cache, h.v_cache, h.block_table, h.seq_lens, h.query_start_loc,
                         h.scale, h.num_kv_heads, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t
        if el >= 10.0 or reps >= 1000:
            break
    per = el / reps
    return {"value": round(nbytes / per / 1e9, 3), "unit": "GB/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "the whole timed batch (64 decode requests), %d pass(es), %.2f s each" % (reps, per)}


def roof(nbytes, flops, ms, new_tokens, copy_gbs):
    """Rates of one case: HBM GB/s and TFLOP/s against the peaks, tokens/s, and the
    roofline fraction t_roof / t with t_roof = max(bytes / 8 TB/s, flops / 2.5 PF)."""
    s = ms * 1e-3
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    r = {"ms": round(ms, 4), "gbs": round(nbytes / s / 1e9, 1),
         "hbm_frac": round(nbytes / s / 1e9 / HBM_PEAK_GBS, 4),
         "tflops": round(flops / s / 1e12, 2),
         "mfma_frac": round(flops / s / 1e12 / BF16_PEAK_TFLOPS, 4),
         "tokens_per_s": round(new_tokens / s, 1), "t_roof_over_t": round(t_roof / s, 4)}
    if copy_gbs:
        r["frac_of_copy_bw"] = round(nbytes / s / 1e9 / copy_gbs, 4)
    return r


def copy_bandwidth(torch, dev, steps=10, n=1 << 30):
    """Read + write GB/s of a plain n-byte device-to-device copy (HBM reference)."""
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del src, dst
    return ms, 2 * n / (ms * 1e-3) / 1e9


def kv_copies(b, min_bytes=MALL_GUARD_BYTES):
    """The batch's K / V pools plus clones, enough that cycling through them reads
    more than min_bytes of KV no earlier call of the cycle touched."""
    one = b.k_cache.numel() * b.k_cache.element_size()
    if b.v_cache is not b.k_cache:
        one += b.v_cache.numel() * b.v_cache.element_size()
    n = max(1, math.ceil(min_bytes / max(one, 1)) + (1 if one < min_bytes else 0))
    ks, vs = [b.k_cache], [b.v_cache]
    for _ in range(n - 1):
        kc = b.k_cache.clone()
        ks.append(kc)
        vs.append(kc if b.v_cache is b.k_cache else b.v_cache.clone())
    return ks, vs


def small_decode_cases(torch, pa, workload, dev, args, copy_gbs, layers=32):
    """Per-call time of the small Llama decode cases, replayed from a graph of
    `layers` pa_forward calls that each read their own KV-cache copy."""
    res = []
    for case, name in ((0, "B1 L500"), (1, "B64 L500"), (2, "B1 L~U[500,8192]")):
        b = workload.llama_decode(case, device=dev)
        T, Hq = b.num_tokens, b.num_q_heads
        maxL, maxq = max(b.seq_lens_list), max(b.q_lens)
        kcs = [b.k_cache] + [b.k_cache.clone() for _ in range(layers - 1)]
        vcs = [b.v_cache] + [b.v_cache.clone() for _ in range(layers - 1)]
        outs = [torch.empty(T, Hq, b.head_dim_v, dtype=b.dtype, device=dev) for _ in range(layers)]
        dims = pa.make_dims(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, T,
                            max_seq_len=maxL, max_q_len=maxq)
        ws = torch.empty(pa.pa_workspace_size(dims), dtype=torch.uint8, device=dev)

        def step():
            for i in range(layers):
                pa.pa_forward(b.q, kcs[i], vcs[i], b.block_table, b.seq_lens, b.query_start_loc,
                              b.scale, out=outs[i], workspace=ws, max_seq_len=maxL, max_q_len=maxq)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(5, args.steps // 3)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per_call_ms = e0.elapsed_time(e1) / reps / layers
        r = {"case": name, "us_per_call": round(per_call_ms * 1e3, 2)}
        r.update(roof(workload.algorithmic_bytes(b), workload.algorithmic_flops(b), per_call_ms,
                      b.num_tokens, copy_gbs))
        # below 256 MB a replay's KV fits in the last-level cache
        r["kv_bytes_per_replay"] = 2 * b.k_cache.numel() * b.k_cache.element_size() * layers
        res.append(r)
        del graph, kcs, vcs, outs, ws
    return {"workload": "Llama-3.1-8B-shaped decode, small cases; each a graph of %d pa_forward "
                        "calls over %d distinct KV-cache copies, time per call" % (layers, layers),
            "cases": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip every case but the headline decode step")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the small decode cases (their graph replays would dominate "
                         "per-kernel profiler averages)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only time a plain 2 GiB device-to-device copy (HBM reference and the "
                         "byte-counter calibration kernel)")
    ap.add_argument("--gather-calibration", action="store_true",
                    help="only run a gather of 131072 random 4 KiB rows of a 1 GiB pool (a second "
                         "byte-counter calibration with the decode kernel's access pattern: "
                         "scattered 4 KiB blocks, one K or V page of one KV head)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_attention_kv_pa_amd as pa
    from paged_attention_kv_pa_amd import workload

    if not os.path.exists(pa.library_path()):
        from paged_attention_kv_pa_amd import build as pbuild
        pbuild.build()
    lib = pa.library()
    lib.pa_set_kernel_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.pa_set_kernel_events.restype = ctypes.c_int32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        ms, gbs = copy_bandwidth(torch, dev, steps=args.steps, n=2 << 30)
        n = 2 << 30
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                          "read_plus_write_GBs": round(gbs, 1)}), flush=True)
        return
    if args.gather_calibration:
        row_bytes, rows = 4096, (1 << 30) // 4096
        pool = torch.empty(rows, row_bytes // 2, dtype=torch.bfloat16, device=dev).fill_(1)
        gen = torch.Generator(device="cpu").manual_seed(7)
        idx = torch.randperm(rows, generator=gen)[: rows // 2].to(dev)
        gout = torch.empty(rows // 2, row_bytes // 2, dtype=torch.bfloat16, device=dev)
        for _ in range(max(args.steps, 1)):
            torch.index_select(pool, 0, idx, out=gout)
        torch.cuda.synchronize()
        print(json.dumps({"gather_rows": rows // 2, "row_bytes": row_bytes,
                          "bytes_read": rows // 2 * row_bytes + idx.numel() * idx.element_size(),
                          "bytes_written": rows // 2 * row_bytes}), flush=True)
        return
    sha = source_sha256()
    copy_ms, copy_gbs = copy_bandwidth(torch, dev)

    # ---- decode: Llama-3.1-8B shapes, B = 64, L ~ U[500, 8192]
    b = workload.llama_decode(3, device=dev)
    T, Hq = b.num_tokens, b.num_q_heads
    out = torch.empty(T, Hq, b.head_dim_v, dtype=b.dtype, device=dev)
    lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    maxL, maxq = max(b.seq_lens_list), max(b.q_lens)
    dims = pa.make_dims(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, T,
                        max_seq_len=maxL, max_q_len=maxq)
    ws = torch.empty(pa.pa_workspace_size(dims), dtype=torch.uint8, device=dev)

    def step():
        pa.pa_forward(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.query_start_loc,
                      b.scale, out=out, lse=lse, workspace=ws, max_seq_len=maxL, max_q_len=maxq)

    step_ms, kern_ms = time_steps(step, args.steps, args.warmup, lib)
    nbytes = workload.algorithmic_bytes(b)
    value = nbytes / (step_ms * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    kname = "mha_forward_kernel<128, decode>"
    tr = committed_entry(TRAFFIC_FILE, kname, sha)
    tt = committed_entry(TRACE_FILE, kname, sha)
    rl = {"kernel": "mha_forward_kernel<128, decode-only>", "bound": "hbm",
          "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
          "frac": round(achieved / HBM_PEAK_GBS, 4), "kernel_ms": round(kern_ms, 5),
          "traffic": tr.get("bytes_per_launch") if tr else None,
          "frac_of_copy_bw": round(achieved / copy_gbs, 4)}
    if tt:
        # the same kernel's mean duration in the committed rocprofv3 trace of this source
        rl["trace_kernel_ms"] = round(tt["avg_us"] * 1e-3, 5)
        rl["trace_frac"] = round(nbytes / (tt["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped paged decode", "batch": 64,
                   "context": "uniform [500, 8192]", "q_heads": 32, "kv_heads": 8,
                   "head_dim": 128, "page_size": 16, "total_keys": int(sum(b.seq_lens_list)),
                   "algorithmic_bytes": nbytes},
        "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": rl,
        "copy_reference": {"workload": "1 GiB device-to-device copy", "ms": round(copy_ms, 4),
                           "read_plus_write_gbs": round(copy_gbs, 1)},
        "step": roof(nbytes, workload.algorithmic_flops(b), step_ms, T, copy_gbs),
        "source_sha256": sha,
    }
    del ws, out, lse
    b_host_needed = not args.no_cpu_baseline

    if not args.no_extra and not args.no_small:
        result["small_decode"] = small_decode_cases(torch, pa, workload, dev, args, copy_gbs)

    def timed_forward(m, steps, mask=None, warmup=2, pools=None):
        """pa_forward (or pa_forward_masked) over batch m; pools: K / V copies cycled
        through call by call."""
        Tm = m.num_tokens
        mo = torch.empty(Tm, m.num_q_heads, m.head_dim_v, dtype=m.dtype, device=dev)
        mmaxL, mmaxq = max(m.seq_lens_list), max(m.q_lens)
        mdims = pa.make_dims(m.q, m.k_cache, m.v_cache, m.block_table, m.seq_lens, Tm,
                             max_seq_len=mmaxL, max_q_len=mmaxq)
        mws = torch.empty(pa.pa_workspace_size(mdims), dtype=torch.uint8, device=dev)
        ks, vs = pools if pools is not None else ([m.k_cache], [m.v_cache])
        it = [0]

        def pstep():
            i = it[0] % len(ks)
            it[0] += 1
            if mask is None:
                pa.pa_forward(m.q, ks[i], vs[i], m.block_table, m.seq_lens, m.query_start_loc,
                              m.scale, out=mo, workspace=mws, max_seq_len=mmaxL, max_q_len=mmaxq)
            else:
                pa.pa_forward_masked(m.q, ks[i], vs[i], m.block_table, m.seq_lens,
                                     m.query_start_loc, m.scale, mask, out=mo, workspace=mws,
                                     max_seq_len=mmaxL, max_q_len=mmaxq)

        return time_steps(pstep, steps, warmup, lib)

    # ---- prefill half of the metric: the prefill + extend requests of the Qwen3-235B
    # mixed batch (requests 48..63); the decode share (requests 0..47); the whole batch
    if not args.no_prefill and not args.no_extra:
        full = workload.qwen3_mixed(0, device=dev)
        psteps = max(3, args.steps // 3)
        pre = workload.sub_batch(full, range(48, 64))
        p_step_ms, p_kern_ms = timed_forward(pre, psteps)
        flops = workload.algorithmic_flops(pre)
        tf = flops / (p_kern_ms * 1e-3) / 1e12
        result["prefill"] = {
            "workload": "Qwen3-235B-shaped mixed batch, its 8 extend (q~U[256,2048] on "
                        "c~U[4096,32768]) + 8 prefill (q~U[512,8192]) requests; 64/4 heads, "
                        "d=128, page 16, causal",
            "value": round(tf, 2), "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS,
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "kernel_ms": round(p_kern_ms, 4),
            "ms_per_step": round(p_step_ms, 4), "algorithmic_flops": flops, "steps": psteps,
            "step": roof(workload.algorithmic_bytes(pre), flops, p_step_ms, pre.num_tokens,
                         copy_gbs)}
        # the same sub-batch under the full mask (every new token sees all keys of its
        # request, as in encoder or cross-attention): pairs = q_b * L_b per request
        f_step_ms, f_kern_ms = timed_forward(pre, psteps, mask=pa.PA_MASK_FULL)
        fflops = sum(4 * q * L * pre.num_q_heads * pre.head_dim_qk
                     for q, L in zip(pre.q_lens, pre.seq_lens_list))
        ftf = fflops / (f_kern_ms * 1e-3) / 1e12
        result["prefill_full_mask"] = {
            "workload": "the prefill + extend sub-batch above through pa_forward_masked with "
                        "PA_MASK_FULL (no causal mask)",
            "value": round(ftf, 2), "unit": "TFLOP/s", "frac": round(ftf / BF16_PEAK_TFLOPS, 4),
            "kernel_ms": round(f_kern_ms, 4), "ms_per_step": round(f_step_ms, 4),
            "algorithmic_flops": fflops}
        # the decode share: 48 requests, L ~ U[1K, 16K], G = 16 (one MFMA tile of rows)
        dsub = workload.sub_batch(full, range(0, 48))
        dpools = kv_copies(dsub)
        d_step_ms, d_kern_ms = timed_forward(dsub, max(10, args.steps // 2), pools=dpools,
                                             warmup=len(dpools[0]))
        dbytes = workload.algorithmic_bytes(dsub)
        result["mixed_decode_share"] = {
            "workload": "the 48 decode requests of the Qwen3-235B mixed batch (64/4 heads, "
                        "L~U[1024,16384]) in one pa_forward call; %d KV pool copies cycled "
                        "(more than 512 MB of fresh KV per call)" % len(dpools[0]),
            "algorithmic_bytes": dbytes, "kernel_frac": round(
                dbytes / (d_kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_ms": round(d_kern_ms, 4),
            "step": roof(dbytes, workload.algorithmic_flops(dsub), d_step_ms, dsub.num_tokens,
                         copy_gbs)}
        del dpools, dsub
        # MLA prefill / extend on the uncompressed representation (DeepSeek-R1 shapes,
        # 128 heads, query / key 192, value 128), same extend / prefill length mix
        nab = workload.deepseek_mha_prefill(0, device=dev)
        n_step_ms, n_kern_ms = timed_forward(nab, psteps)
        nflops = workload.algorithmic_flops(nab)
        ntf = nflops / (n_kern_ms * 1e-3) / 1e12
        result["mla_prefill_non_absorbed"] = {
            "workload": "DeepSeek-R1-shaped MLA prefill + extend run non-absorbed: 8 extend "
                        "(q~U[256,2048] on c~U[4096,32768]) + 8 prefill (q~U[512,8192]) "
                        "requests, 128 heads, query/key 192, value 128, page 64, causal",
            "value": round(ntf, 2), "unit": "TFLOP/s", "frac": round(ntf / BF16_PEAK_TFLOPS, 4),
            "kernel_ms": round(n_kern_ms, 4), "ms_per_step": round(n_step_ms, 4),
            "algorithmic_flops": nflops,
            "step": roof(workload.algorithmic_bytes(nab), nflops, n_step_ms, nab.num_tokens,
                         copy_gbs)}
        del nab
        # the same prefill + extend sub-batch with the ALiBi-sqrt bias (standard slopes)
        al = torch.tensor(workload.alibi_slopes(pre.num_q_heads), dtype=torch.float32, device=dev)
        a_mo = torch.empty(pre.num_tokens, pre.num_q_heads, pre.head_dim_v, dtype=pre.dtype,
                           device=dev)
        a_dims = pa.make_dims(pre.q, pre.k_cache, pre.v_cache, pre.block_table, pre.seq_lens,
                              pre.num_tokens, max_seq_len=max(pre.seq_lens_list),
                              max_q_len=max(pre.q_lens))
        a_ws = torch.empty(pa.pa_workspace_size(a_dims), dtype=torch.uint8, device=dev)

        def astep():
            pa.pa_forward_masked(pre.q, pre.k_cache, pre.v_cache, pre.block_table, pre.seq_lens,
                                 pre.query_start_loc, pre.scale, pa.PA_MASK_CAUSAL, out=a_mo,
                                 workspace=a_ws, max_seq_len=max(pre.seq_lens_list),
                                 max_q_len=max(pre.q_lens), alibi_slopes=al,
                                 alibi_mode=pa.PA_ALIBI_SQRT)

        a_step_ms, a_kern_ms = time_steps(astep, psteps, 2, lib)
        atf = flops / (a_kern_ms * 1e-3) / 1e12
        result["prefill_alibi_sqrt"] = {
            "workload": "the prefill + extend sub-batch above through pa_forward_masked with the "
                        "ALiBi-sqrt bias (slopes 2^(-8(h+1)/64))",
            "value": round(atf, 2), "unit": "TFLOP/s", "frac": round(atf / BF16_PEAK_TFLOPS, 4),
            "kernel_ms": round(a_kern_ms, 4), "ms_per_step": round(a_step_ms, 4)}
        del a_mo, a_ws, al
        m_step_ms, m_kern_ms = timed_forward(full, psteps)
        result["mixed_batch"] = {
            "workload": "Qwen3-235B-shaped mixed batch, all 64 requests [48 decode : 8 extend : "
                        "8 prefill] in one pa_forward call",
            "ms_per_step": round(m_step_ms, 4), "kernel_ms": round(m_kern_ms, 4),
            "new_tokens_per_s": round(full.num_tokens / (m_step_ms * 1e-3), 1),
            "step": roof(workload.algorithmic_bytes(full), workload.algorithmic_flops(full),
                         m_step_ms, full.num_tokens, copy_gbs)}
        # the whole mixed batch plus one extend of 256 new tokens on 131072 cached
        # ones, which pa_forward's planner cuts into 32K-key chunks inside the batch
        lx = workload.qwen3_mixed_with_long_extend(0, device=dev)
        x_step_ms, x_kern_ms = timed_forward(lx, psteps)
        result["mixed_batch_with_long_extend"] = {
            "workload": "the Qwen3-235B-shaped mixed batch above plus one extend of 256 new "
                        "tokens on 131072 cached tokens (cut into 32K-key chunks by the planner) "
                        "in one pa_forward call",
            "ms_per_step": round(x_step_ms, 4), "kernel_ms": round(x_kern_ms, 4),
            "step": roof(workload.algorithmic_bytes(lx), workload.algorithmic_flops(lx),
                         x_step_ms, lx.num_tokens, copy_gbs)}
        del lx, full, pre

    if not args.no_extra:
        xsteps = max(10, args.steps // 2)
        # ---- long-context split-KV decode, Llama-3.1-8B heads: B 1 / 4 / 16 with
        # L ~ U[32K, 128K], and B 1 at L = 32768 and 131072; pa_decode_split with S
        # partitions + pa_merge_lse, and the same batch through pa_forward (which
        # splits the keys itself)
        cases = []
        for batch, S, lengths, name in ((1, 64, None, "B1 L~U[32768,131072] S64"),
                                        (4, 32, None, "B4 L~U[32768,131072] S32"),
                                        (16, 16, None, "B16 L~U[32768,131072] S16"),
                                        (1, 64, [32768], "B1 L32768 S64"),
                                        (1, 64, [131072], "B1 L131072 S64")):
            lb = workload.llama_long(batch=batch, lengths=lengths, device=dev)
            B = lb.num_seqs
            pools = kv_copies(lb)
            po = torch.empty(B, lb.num_q_heads, S, lb.head_dim_v, dtype=torch.float32, device=dev)
            pl = torch.empty(B, lb.num_q_heads, S, dtype=torch.float32, device=dev)
            lo = torch.empty(B, lb.num_q_heads, lb.head_dim_v, dtype=lb.dtype, device=dev)
            it = [0]

            def sstep():
                i = it[0] % len(pools[0])
                it[0] += 1
                pa.pa_decode_split(lb.q, pools[0][i], pools[1][i], lb.block_table, lb.seq_lens,
                                   lb.scale, S, part_out=po, part_lse=pl,
                                   max_seq_len=max(lb.seq_lens_list))
                pa.pa_merge_lse(po, pl, out=lo)

            s_step_ms, s_kern_ms = time_steps(sstep, xsteps, len(pools[0]), lib)
            f_step_ms, _ = timed_forward(lb, xsteps, pools=pools, warmup=len(pools[0]))
            sbytes = workload.algorithmic_bytes(lb)
            sflops = workload.algorithmic_flops(lb)
            cases.append({"case": name, "keys": int(sum(lb.seq_lens_list)),
                          "kv_pool_copies": len(pools[0]), "algorithmic_bytes": sbytes,
                          "split_kernel_ms": round(s_kern_ms, 4),
                          "split_kernel_frac": round(sbytes / (s_kern_ms * 1e-3) / 1e9 /
                                                     HBM_PEAK_GBS, 4),
                          "split_plus_merge": roof(sbytes, sflops, s_step_ms, B, copy_gbs),
                          "pa_forward": roof(sbytes, sflops, f_step_ms, B, copy_gbs)})
            del lb, pools, po, pl, lo
        b16 = cases[2]
        result["split_kv"] = {
            "workload": "Llama-3.1-8B-shaped long-context decode (32/8 heads, d=128, page 16); "
                        "pa_decode_split + pa_merge_lse, and pa_forward; KV pools cycled so "
                        "that every call reads more than 512 MB of fresh KV",
            "hbm_gbs": b16["split_plus_merge"]["gbs"],
            "frac": b16["split_kernel_frac"], "cases": cases}
        # ---- absorbed MLA decode: 64 sequences, 128 heads, latent 576 / 512, L ~ U[1K, 32K]
        mb = workload.deepseek_mla(0, device=dev)
        mout = torch.empty(mb.num_seqs, mb.num_q_heads, 512, dtype=mb.dtype, device=dev)
        mdims = pa.make_dims(mb.q, mb.k_cache, mb.k_cache, mb.block_table, mb.seq_lens,
                             mb.num_seqs, layout="mla", max_seq_len=max(mb.seq_lens_list),
                             max_q_len=1)
        mws = torch.empty(max(1, pa.mla_workspace_size(mdims, 0)), dtype=torch.uint8, device=dev)

        def mstep():
            pa.mla_decode(mb.q, mb.k_cache, mb.block_table, mb.seq_lens, mb.scale, out=mout,
                          workspace=mws, max_seq_len=max(mb.seq_lens_list))

        m_step_ms, m_kern_ms = time_steps(mstep, xsteps, 5, lib)
        mbytes = workload.algorithmic_bytes(mb)
        mflops = workload.algorithmic_flops(mb)
        mtt = committed_entry(TRACE_FILE, "mla_balanced_kernel", sha)
        result["mla"] = {
            "workload": "DeepSeek-R1-shaped absorbed MLA decode, 64 sequences, 128 heads, "
                        "latent 576 (value 512), page 64, L~U[1024,32768]",
            "hbm_gbs": round(mbytes / (m_step_ms * 1e-3) / 1e9, 2),
            "kernel_gbs": round(mbytes / (m_kern_ms * 1e-3) / 1e9, 2),
            "frac": round(mbytes / (m_kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_tflops": round(mflops / (m_kern_ms * 1e-3) / 1e12, 2),
            "ms_per_step": round(m_step_ms, 4), "kernel_ms": round(m_kern_ms, 4),
            "algorithmic_bytes": mbytes, "algorithmic_flops": mflops,
            "trace_frac": (round(mbytes / (mtt["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                           if mtt else None),
            "step": roof(mbytes, mflops, m_step_ms, mb.num_seqs, copy_gbs)}
        del mb, mout, mws
        # ---- chunked-context extend: 256 new tokens on 131072 cached tokens in 8 chunks (one
        # work item per compute unit), against the same request in one pa_forward call
        cb = workload.llama_long_extend(0, device=dev)
        cL, cq = max(cb.seq_lens_list), max(cb.q_lens)
        C = ((cL + 7) // 8 + 63) // 64 * 64
        cS = (cL + C - 1) // C
        cpo = torch.empty(cb.num_tokens, cb.num_q_heads, cS, cb.head_dim_v, dtype=torch.float32,
                          device=dev)
        cpl = torch.empty(cb.num_tokens, cb.num_q_heads, cS, dtype=torch.float32, device=dev)
        cout = torch.empty(cb.num_tokens, cb.num_q_heads, cb.head_dim_v, dtype=cb.dtype, device=dev)
        cdims = pa.make_dims(cb.q, cb.k_cache, cb.v_cache, cb.block_table, cb.seq_lens,
                             cb.num_tokens, max_seq_len=cL, max_q_len=cq)
        cws = torch.empty(max(1, pa.pa_workspace_size(cdims)), dtype=torch.uint8, device=dev)

        def cstep():
            pa.pa_forward_chunked(cb.q, cb.k_cache, cb.v_cache, cb.block_table, cb.seq_lens,
                                  cb.query_start_loc, cb.scale, C, num_chunks=cS, part_out=cpo,
                                  part_lse=cpl, max_seq_len=cL, max_q_len=cq)
            pa.pa_merge_lse(cpo, cpl, out=cout)

        def fstep():
            pa.pa_forward(cb.q, cb.k_cache, cb.v_cache, cb.block_table, cb.seq_lens,
                          cb.query_start_loc, cb.scale, out=cout, workspace=cws, max_seq_len=cL,
                          max_q_len=cq)

        c_step_ms, c_kern_ms = time_steps(cstep, xsteps, 3, lib)
        f_step_ms, f_kern_ms = time_steps(fstep, xsteps, 3, lib)
        cflops = workload.algorithmic_flops(cb)
        cbytes = workload.algorithmic_bytes(cb)
        result["chunked_extend"] = {
            "workload": "Llama-3.1-8B-shaped extend, 256 new tokens on 131072 cached tokens, "
                        "page 16: pa_forward_chunked (8 chunks) + pa_merge_lse, and the "
                        "same request through pa_forward (which runs such calls as chunks too)",
            "chunk_keys": C, "chunks": cS,
            "tflops": round(cflops / (c_step_ms * 1e-3) / 1e12, 2),
            "frac": round(cflops / (c_step_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "ms_per_step": round(c_step_ms, 4), "kernel_ms": round(c_kern_ms, 4),
            "pa_forward_ms_per_step": round(f_step_ms, 4),
            "pa_forward_tflops": round(cflops / (f_step_ms * 1e-3) / 1e12, 2),
            "algorithmic_flops": cflops,
            "step": roof(cbytes, cflops, c_step_ms, cb.num_tokens, copy_gbs),
            "pa_forward_step": roof(cbytes, cflops, f_step_ms, cb.num_tokens, copy_gbs)}
        del cb, cpo, cpl, cout, cws

    if b_host_needed:
        result["cpu_baseline"] = cpu_baseline(b, nbytes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
