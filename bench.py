"""Benchmark of the exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads all|main|decode|...]

A step is one pass of the hot path over one batch of synthetic input: one
sdpa_fwd call on the causal bf16 workload B=4, H=16, L=S=2048, E=128 (the
headline configuration).  The JSON line reports its attention TFLOP/s with
the matrix-core roofline of the prefill kernel, the CPU oracle timed on the
host cores on a bounded sample of the same workload, and (under "secondary")
the other workloads: split-KV GQA decode in GB/s against the HBM roofline
(dense, and with the cache in 64-key pages of a shuffled pool),
the GPT-NeoX-shaped E=96 variants, packed variable-length fp16, the
single-head fp32 case and the backward of the headline workload (5 products
per kept pair: 10 E flops).

Algorithmic work (what the method must do, not what a kernel happens to do):
flops = (2E + 2Ev) x kept (query, key) pairs; bytes = Q + K + V + O + lse
(+ the float mask over the kept region when one is read), K/V counted once per
key/value head.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # dense bf16/fp16 matrix peak: 256 CUs x 2.4 GHz x 4096 flop/clk
PEAK_FP32_TFLOPS = 157.3    # fp32 matrix peak (the fp32 path runs on the vector ALUs)
PEAK_HBM_GBS = 8000.0       # HBM3E
METRIC = "attn fwd TFLOP/s (% MFMA peak) prefill; GB/s (% HBM peak) split-KV decode"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["prefill_pp.h", "prefill_mfma.h", "device_utils.h", "attn_common.h", "decode.hip"]


def kernel_source_hash():
    """Hash of the kernel sources with comments and blank lines removed, so that
    the stored counter results stay tied to the code, not to its prose."""
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "transformer_attention_04_amd", "csrc", name)) as f:
            text = re.sub(r"//[^\n]*", "", f.read())
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def causal_pairs(L, S):
    """Kept (i, j) pairs with j <= i for one head."""
    return sum(min(i + 1, S) for i in range(L))


def flops_prefill(B, H, L, S, E, causal):
    pairs = causal_pairs(L, S) if causal else L * S
    return 4 * E * pairs * B * H, pairs


def time_launches(fn, steps, warmup):
    """Run fn warmup times, then time `steps` back-to-back calls: wall time
    between two synchronizes, and GPU time from one pair of events recorded on
    torch's current stream (the stream the kernels are launched on) around the
    whole timed region.  Returns (wall seconds, [GPU ms per call])."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) / steps]


def load_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if the kernels are unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def _cpu_info():
    """(model name from /proc/cpuinfo, cores this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def oracle_timing(calls, work, unit, sample):
    """The float64 oracle on the host cores: one warm-up call, then the whole sample
    (``calls``, a list of thunks) timed 3 times; the median gives ``work`` / s in ``unit``."""
    from threadpoolctl import threadpool_limits
    model, cores = _cpu_info()
    with threadpool_limits(limits=cores):
        calls[0]()
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            for c in calls:
                c()
            times.append(time.perf_counter() - t0)
    med = sorted(times)[1]
    return {"value": round(work / med, 6), "unit": unit, "cores": cores, "cpu": model, "kind": "oracle",
            "median_of": 3, "seconds": round(med, 3), "sample": sample}


def cpu_baseline(n_heads=64):
    """The float64 oracle on whole heads of the headline workload (median of 3 passes;
    by default all 64 heads, i.e. the whole workload: ~7 s a pass on 16 cores)."""
    from oracle import sdpa_oracle as O
    from transformer_attention_04_amd import inputs
    q, k, v = inputs.workload_inputs("bf16_causal_e128")
    B, H, L, E = q.shape
    per_head_flops = flops_prefill(1, 1, L, L, E, True)[0]
    heads = [(i // H, i % H) for i in range(min(n_heads, B * H))]
    calls = [lambda b=b, h=h: O.sdpa(q[b, h], k[b, h], v[b, h], is_causal=True) for b, h in heads]
    return oracle_timing(calls, per_head_flops * len(heads) / 1e12, "TFLOP/s",
                         f"{len(heads)} of {B * H} heads (causal, L=S={L}, E={E}), float64 numpy")


def cpu_secondary():
    """The oracle beside the secondary workloads, each on a bounded sample (median of 3)."""
    from oracle import sdpa_oracle as O
    from transformer_attention_04_amd import inputs
    res = {}
    q, k, v = inputs.workload_inputs("bf16_neox_e96")
    f = flops_prefill(1, 1, 2048, 2048, 96, True)[0]
    calls = [lambda h=h: O.sdpa(q[0, h], k[0, h], v[0, h], is_causal=True) for h in range(4)]
    res["bf16_neox_e96"] = oracle_timing(calls, 4 * f / 1e12, "TFLOP/s", "4 of 128 heads, scale 1/sqrt(96)")
    bias = inputs.alibi_causal_bias(64, 2048, 2048).numpy()
    calls = [lambda h=h: O.sdpa(q[0, h], k[0, h], v[0, h], attn_mask=bias[h], is_causal=True) for h in range(4)]
    res["bf16_neox_e96 alibi+causal"] = oracle_timing(calls, 4 * f / 1e12, "TFLOP/s", "4 of 128 heads")
    del q, k, v, bias
    w = inputs.WORKLOADS["fp16_varlen_e64"]
    lengths = inputs.segment_lengths(seed=w["len_seed"])[:8]
    qv, kv, vv, cu = inputs.varlen_inputs(lengths, 8, 8, 64, "fp16", seed=w["seed"])
    cu8 = cu.numpy()
    fl = sum(4 * 64 * l * (l + 1) // 2 for l in lengths) * 8
    res["fp16_varlen_e64"] = oracle_timing([lambda: O.sdpa_varlen(qv[0], kv[0], vv[0], cu8, is_causal=True)],
                                           fl / 1e12, "TFLOP/s", f"the first 8 of the 32 segments ({sum(lengths)} "
                                           "tokens, 8 heads)")
    q, k, v = inputs.workload_inputs("fp32_single_head")
    res["fp32_single_head"] = oracle_timing([lambda: O.sdpa(q, k, v)], 1.0, "calls/s", "the whole workload")
    # decode: 2 sequences of the workload's shape (32768 keys, Hq=32 over Hkv=8, E=128, bf16 values)
    q, k, v = inputs.randn_qkv((2, 32, 1, 128), (2, 8, 32768, 128), (2, 8, 32768, 128), "bf16", seed=0)
    groups = [(b, g) for b in range(2) for g in range(8)]
    nbytes = len(groups) * (2 * 2 * 32768 * 128 + 2 * 2 * 4 * 128)
    calls = [lambda b=b, g=g: O.sdpa(q[b, 4 * g:4 * g + 4], k[b, g:g + 1], v[b, g:g + 1]) for b, g in groups]
    res["bf16_gqa_decode"] = oracle_timing(calls, nbytes / 1e9, "GB/s",
                                           "16 key/value-head groups of the same shape (2 sequences, seed 0)")
    return res


def bench_prefill(name, steps, warmup, scale=None, mask=None, device="cuda"):
    import torch
    from transformer_attention_04_amd import inputs
    from transformer_attention_04_amd import sdpa as S
    w = inputs.WORKLOADS[name]
    q, k, v = (t.to(device) for t in inputs.workload_inputs(name))
    md = mask.to(device) if mask is not None else None
    fn = S.PreparedSdpaFwd(q, k, v, attn_mask=md, is_causal=w["causal"], scale=scale)
    wall, per = time_launches(fn, steps, warmup)
    flops, pairs = flops_prefill(w["B"], w["Hq"], w["L"], w["S"], w["E"], w["causal"])
    kern_ms = sum(per) / len(per)
    res = {"ms_per_step": wall * 1e3 / steps, "kernel_ms": kern_ms, "flops": flops,
           "tflops": flops / (wall / steps) / 1e12, "kernel_tflops": flops / (kern_ms * 1e-3) / 1e12}
    if mask is not None:
        qkvo = 2 * (q.numel() + k.numel() + v.numel() + q.numel())
        mbytes = 4 * pairs * w["Hq"] * (1 if mask.dim() == 3 else w["B"])
        res["bytes"] = qkvo + 4 * q.numel() // w["E"] + mbytes
        res["gbs"] = res["bytes"] / (kern_ms * 1e-3) / 1e9
    return res


def bench_boolmask(steps, warmup, device="cuda"):
    """The headline shape (bf16, B=4, H=16, L=S=2048, E=128), causal and a bool
    mask (L, S) shared by batch and heads keeping each key with probability 0.9
    (seed 21): contiguous (eight-wave kernel), and for comparison as views with
    row strides S + 8 (four-wave kernel: rows not in whole 16-byte chunks) and
    S + 16 (eight-wave kernel)."""
    import torch
    from transformer_attention_04_amd import inputs
    from transformer_attention_04_amd import sdpa as S
    w = inputs.WORKLOADS["bf16_causal_e128"]
    q, k, v = (t.to(device) for t in inputs.workload_inputs("bf16_causal_e128"))
    L, Sk = w["L"], w["S"]
    m = torch.rand((1, 1, L, Sk), generator=torch.Generator().manual_seed(21)) < 0.9
    kept = int((m[0, 0] & torch.ones(L, Sk, dtype=torch.bool).tril()).sum())
    flops = 4 * w["E"] * kept * w["B"] * w["Hq"]
    res = {"flops": flops, "kept_pairs_per_head": kept}
    for tag, pad in (("contiguous", 0), ("four_wave_stride_s8", 8), ("eight_wave_stride_s16", 16)):
        wide = torch.zeros((1, 1, L, Sk + pad), dtype=torch.bool)
        wide[..., :Sk] = m
        mm = wide.to(device)[..., :Sk]
        fn = S.PreparedSdpaFwd(q, k, v, attn_mask=mm, is_causal=True)
        wall, per = time_launches(fn, steps, warmup)
        kern_ms = sum(per) / len(per)
        res[tag] = {"kernel_ms": kern_ms, "kernel_tflops": flops / (kern_ms * 1e-3) / 1e12}
    return res


def bench_decode(steps, warmup, device="cuda"):
    import torch
    from transformer_attention_04_amd import inputs
    from transformer_attention_04_amd import sdpa as S
    q, k, v = (t.to(device) for t in inputs.workload_inputs("bf16_gqa_decode"))
    fn = S.PreparedSdpaFwd(q, k, v, enable_gqa=True)
    nws = 0 if fn.workspace is None else fn.workspace.numel()
    wall, per = time_launches(fn, steps, warmup)
    nbytes = 2 * (q.numel() + k.numel() + v.numel() + fn.out.numel()) + 4 * fn.lse.numel()
    kern_ms = sum(per) / len(per)
    return {"ms_per_step": wall * 1e3 / steps, "kernel_ms": kern_ms, "bytes": nbytes,
            "gbs": nbytes / (kern_ms * 1e-3) / 1e9, "frac_hbm": nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "workspace_bytes": nws}


def bench_paged(steps, warmup, device="cuda", page=64):
    """The decode workload with its cache in 64-key pages of a shuffled pool,
    read through a block table (sdpa_fwd_paged)."""
    import torch
    from transformer_attention_04_amd import inputs
    from transformer_attention_04_amd import sdpa as S
    q, k, v = (t.to(device) for t in inputs.workload_inputs("bf16_gqa_decode"))
    B, Hkv, Sk, E = k.shape
    nb = Sk // page
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(B * nb, generator=g).to(device)
    def pool(x):  # page j of sequence b goes to slot perm[b * nb + j]
        pages = x.reshape(B, Hkv, nb, page, E).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, page, E)
        out = torch.empty_like(pages)
        out[perm] = pages
        return out
    kc, vc = pool(k), pool(v)
    del k, v
    bt = perm.reshape(B, nb).to(torch.int32)
    lens = torch.full((B,), Sk, dtype=torch.int32, device=device)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=device)
    fn = lambda: S.sdpa_fwd_paged(q, kc, vc, bt, lens, max_seq_len=Sk, enable_gqa=True, workspace=ws)
    wall, per = time_launches(fn, steps, warmup)
    out_numel = q.numel()
    nbytes = 2 * (q.numel() + kc.numel() + vc.numel() + out_numel) + 4 * (q.numel() // E)
    kern_ms = sum(per) / len(per)
    return {"ms_per_step": wall * 1e3 / steps, "kernel_ms": kern_ms, "bytes": nbytes,
            "gbs": nbytes / (kern_ms * 1e-3) / 1e9, "frac_hbm": nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


CHUNKED = dict(B=8, Hq=32, Hkv=8, E=128, L=512, S=4096, page=64, seed=11)


def bench_chunked(steps, warmup, device="cuda", packed=False):
    """Chunked prefill against a paged cache: 8 sequences of 4096 cached keys
    (bf16, 64-key pages in a shuffled pool) whose last 512 positions are the new
    rows, Hq=32 over Hkv=8, E=128, causal aligned bottom-right.  packed: the
    same rows packed token-major and passed with cu_seqlens_q
    (sdpa_fwd_paged_varlen, the serving-batch form)."""
    import torch
    from transformer_attention_04_amd import inputs
    from transformer_attention_04_amd import sdpa as S
    c = CHUNKED
    nb = c["S"] // c["page"]
    n_pages = c["B"] * nb
    q, kc, vc = (t.to(device) for t in inputs.randn_qkv(
        (c["B"], c["Hq"], c["L"], c["E"]), (n_pages, c["Hkv"], c["page"], c["E"]),
        (n_pages, c["Hkv"], c["page"], c["E"]), "bf16", seed=c["seed"]))
    g = torch.Generator().manual_seed(c["seed"] + 1)
    bt = torch.randperm(n_pages, generator=g).reshape(c["B"], nb).to(torch.int32).to(device)
    lens = torch.full((c["B"],), c["S"], dtype=torch.int32, device=device)
    if packed:
        qp = q.permute(0, 2, 1, 3).reshape(c["B"] * c["L"], c["Hq"], c["E"]).contiguous()
        cu = torch.arange(0, c["B"] + 1, dtype=torch.int32, device=device) * c["L"]
        fn = lambda: S.sdpa_fwd_paged_varlen(qp, cu, kc, vc, bt, lens, max_seqlen_q=c["L"], max_seq_len=c["S"],
                                             is_causal=True, enable_gqa=True)
    else:
        fn = lambda: S.sdpa_fwd_paged(q, kc, vc, bt, lens, max_seq_len=c["S"], is_causal=True, enable_gqa=True)
    wall, per = time_launches(fn, steps, warmup)
    L, Sk = c["L"], c["S"]
    pairs = L * (Sk - L) + L * (L + 1) // 2
    flops = 4 * c["E"] * pairs * c["B"] * c["Hq"]
    kern_ms = sum(per) / len(per)
    return {"ms_per_step": wall * 1e3 / steps, "kernel_ms": kern_ms, "flops": flops,
            "kernel_tflops": flops / (kern_ms * 1e-3) / 1e12}


def bench_varlen(steps, warmup, device="cuda"):
    from transformer_attention_04_amd import inputs
    from transformer_attention_04_amd import sdpa as S
    w = inputs.WORKLOADS["fp16_varlen_e64"]
    lengths = inputs.segment_lengths(seed=w["len_seed"])
    q, k, v, cu = (t.to(device) for t in inputs.varlen_inputs(lengths, w["Hq"], w["Hkv"], w["E"], "fp16",
                                                                seed=w["seed"]))
    mx = max(lengths)
    fn = lambda: S.sdpa_fwd_varlen(q, k, v, cu, max_seqlen_q=mx, max_seqlen_k=mx, is_causal=True)
    wall, per = time_launches(fn, steps, warmup)
    pairs = sum(l * (l + 1) // 2 for l in lengths)
    flops = 4 * w["E"] * pairs * w["Hq"]
    kern_ms = sum(per) / len(per)
    return {"ms_per_step": wall * 1e3 / steps, "kernel_ms": kern_ms, "flops": flops,
            "kernel_tflops": flops / (kern_ms * 1e-3) / 1e12, "total_tokens": sum(lengths)}


def bench_backward(steps, warmup, device="cuda"):
    """Gradients of the headline workload (sdpa_bwd with the full workspace: the
    D = dO . O pass, the dK/dV kernel, which stores dS^T, and the dQ kernel
    that reads it) for an N(0,1) output gradient (seed 99)."""
    import torch
    from transformer_attention_04_amd import inputs
    from transformer_attention_04_amd import sdpa as S
    w = inputs.WORKLOADS["bf16_causal_e128"]
    q, k, v = (t.to(device) for t in inputs.workload_inputs("bf16_causal_e128"))
    g = inputs.randn_qkv(tuple(q.shape), (1, 1, 1, w["E"]), (1, 1, 1, w["E"]), "bf16", seed=99)[0].to(device)
    out, lse = S.sdpa_fwd(q, k, v, is_causal=True)
    ws = torch.empty(S.sdpa_bwd_workspace_size(q, k, v), dtype=torch.uint8, device=device)
    fn = lambda: S.sdpa_bwd(q, k, v, out, lse, g, is_causal=True, workspace=ws)
    wall, per = time_launches(fn, steps, warmup)
    pairs = w["L"] * (w["L"] + 1) // 2
    # five products per kept pair: S, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q
    flops = 10 * w["E"] * pairs * w["B"] * w["Hq"]
    kern_ms = sum(per) / len(per)
    return {"ms_per_step": wall * 1e3 / steps, "kernel_ms": kern_ms, "flops": flops,
            "kernel_tflops": flops / (kern_ms * 1e-3) / 1e12}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workloads", default="all",
                    help="all | main | decode | paged | chunked | boolmask | neox | varlen | fp32 | bwd | copy "
                         "(comma separated)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    from transformer_attention_04_amd import sdpa as S
    from transformer_attention_04_amd import inputs
    S.load_library()
    sel = set(a.workloads.split(","))
    run_all = "all" in sel

    secondary = {}
    main_res = None
    if run_all or "main" in sel:
        main_res = bench_prefill("bf16_causal_e128", a.steps, a.warmup)
        print(f"# bf16_causal_e128: {main_res['kernel_ms'] * 1e3:.1f} us/launch, "
              f"{main_res['kernel_tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    # Warm-up calls of each secondary line: enough for the clocks to settle
    # after the host-side set-up between lines (a 1 GiB mask upload, say); with
    # 5, the first timed calls of the ALiBi and backward lines ran 10-15% slow.
    sw = max(5, min(a.warmup, 40))
    if run_all or "decode" in sel:
        d = bench_decode(max(5, a.steps // 2), sw)
        secondary["bf16_gqa_decode"] = {"metric": "GB/s", "value": round(d["gbs"], 1),
                                        "frac_hbm_peak": round(d["frac_hbm"], 4),
                                        "kernel_us": round(d["kernel_ms"] * 1e3, 1),
                                        "bytes_per_call": d["bytes"],
                                        "traffic": load_traffic("decode_split_kernel"),
                                        "kernels": "decode_split_kernel + decode_merge_kernel"}
        print(f"# bf16_gqa_decode: {d['kernel_ms'] * 1e3:.1f} us, {d['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    if run_all or "paged" in sel:
        d = bench_paged(max(5, a.steps // 2), sw)
        secondary["bf16_gqa_decode paged"] = {"metric": "GB/s", "value": round(d["gbs"], 1),
                                              "frac_hbm_peak": round(d["frac_hbm"], 4),
                                              "kernel_us": round(d["kernel_ms"] * 1e3, 1),
                                              "bytes_per_call": d["bytes"], "page_size": 64,
                                              "kernels": "decode_split_kernel (paged) + decode_merge_kernel"}
        print(f"# bf16_gqa_decode paged: {d['kernel_ms'] * 1e3:.1f} us, {d['gbs']:.0f} GB/s", file=sys.stderr,
              flush=True)
    if run_all or "chunked" in sel:
        r = bench_chunked(max(5, a.steps // 4), sw)
        secondary["bf16 chunked prefill paged"] = {
            "metric": "TFLOP/s", "value": round(r["kernel_tflops"], 1),
            "frac_mfma_peak": round(r["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "kernel_us": round(r["kernel_ms"] * 1e3, 1), "flop_per_call": r["flops"],
            "shape": "B=8 Hq=32 Hkv=8 E=128, 512 new rows on 4096 cached keys, 64-key pages, causal",
            "kernels": "prefill_pp_kernel (paged)"}
        print(f"# chunked prefill paged: {r['kernel_ms'] * 1e3:.1f} us, {r['kernel_tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        r = bench_chunked(max(5, a.steps // 4), sw, packed=True)
        secondary["bf16 chunked prefill paged, packed rows"] = {
            "metric": "TFLOP/s", "value": round(r["kernel_tflops"], 1),
            "frac_mfma_peak": round(r["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "kernel_us": round(r["kernel_ms"] * 1e3, 1), "flop_per_call": r["flops"],
            "shape": "the same rows packed token-major with cu_seqlens_q (sdpa_fwd_paged_varlen)",
            "kernels": "prefill_pp_kernel (paged, packed rows)"}
        print(f"# chunked prefill paged, packed rows: {r['kernel_ms'] * 1e3:.1f} us, "
              f"{r['kernel_tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if run_all or "boolmask" in sel:
        r = bench_boolmask(max(5, a.steps // 4), sw)
        secondary["bf16_causal_e128 + bool mask"] = {
            "metric": "TFLOP/s", "value": round(r["contiguous"]["kernel_tflops"], 1),
            "frac_mfma_peak": round(r["contiguous"]["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "kernel_us": round(r["contiguous"]["kernel_ms"] * 1e3, 1), "flop_per_call": r["flops"],
            "four_wave_kernel_us_row_stride_s8": round(r["four_wave_stride_s8"]["kernel_ms"] * 1e3, 1),
            "eight_wave_kernel_us_row_stride_s16": round(r["eight_wave_stride_s16"]["kernel_ms"] * 1e3, 1),
            "mask": "(1, 1, 2048, 2048) bool, keep probability 0.9, seed 21, with is_causal",
            "kernels": "prefill_pp_kernel<BF16,128,causal,bool>"}
        print(f"# bool mask: contiguous (eight-wave) {r['contiguous']['kernel_ms'] * 1e3:.1f} us, "
              f"stride S+8 (four-wave) {r['four_wave_stride_s8']['kernel_ms'] * 1e3:.1f} us, "
              f"stride S+16 (eight-wave) {r['eight_wave_stride_s16']['kernel_ms'] * 1e3:.1f} us",
              file=sys.stderr, flush=True)
    if run_all or "neox" in sel:
        for tag, sc in (("1/sqrt96", None), ("1/96", 1 / 96), ("1.0", 1.0)):
            r = bench_prefill("bf16_neox_e96", max(5, a.steps // 2), sw, scale=sc)
            secondary[f"bf16_neox_e96 scale={tag}"] = {
                "metric": "TFLOP/s", "value": round(r["kernel_tflops"], 1),
                "frac_mfma_peak": round(r["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                "kernel_us": round(r["kernel_ms"] * 1e3, 1)}
        bias = inputs.alibi_causal_bias(64, 2048, 2048)
        r = bench_prefill("bf16_neox_e96", max(5, a.steps // 2), sw, mask=bias)
        secondary["bf16_neox_e96 alibi+causal"] = {
            "metric": "TFLOP/s", "value": round(r["kernel_tflops"], 1),
            "frac_mfma_peak": round(r["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "gbs": round(r["gbs"], 1), "kernel_us": round(r["kernel_ms"] * 1e3, 1)}
        del bias
    if run_all or "varlen" in sel:
        r = bench_varlen(max(5, a.steps // 2), sw)
        secondary["fp16_varlen_e64"] = {"metric": "TFLOP/s", "value": round(r["kernel_tflops"], 1),
                                        "frac_mfma_peak": round(r["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                                        "kernel_us": round(r["kernel_ms"] * 1e3, 1)}
    if run_all or "fp32" in sel:
        r = bench_prefill("fp32_single_head", max(5, a.steps // 2), sw)
        secondary["fp32_single_head"] = {"metric": "us per call", "value": round(r["kernel_ms"] * 1e3, 2),
                                         "tflops": round(r["kernel_tflops"], 3)}

    if run_all or "bwd" in sel:
        r = bench_backward(max(5, a.steps // 4), sw)
        secondary["bf16_causal_e128 backward"] = {
            "metric": "TFLOP/s", "value": round(r["kernel_tflops"], 1),
            "frac_mfma_peak": round(r["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "call_us": round(r["kernel_ms"] * 1e3, 1), "flop_per_call": r["flops"],
            "kernels": "bwd_dsum_kernel + bwd_dkdv_kernel (storing dS^T) + bwd_dq_ds_kernel"}
        print(f"# bf16_causal_e128 backward: {r['kernel_ms'] * 1e3:.1f} us/call, "
              f"{r['kernel_tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)

    if "copy" in sel:
        # calibration for the HBM byte counters: a plain device copy of a known size
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        secondary["copy_calibration"] = {"bytes_read_per_copy": src.numel(), "bytes_written_per_copy": dst.numel(),
                                         "copies": 4}
    if main_res is None:
        print(json.dumps({"secondary": secondary}))
        return 0
    w = inputs.WORKLOADS["bf16_causal_e128"]
    achieved = main_res["kernel_tflops"]
    line = {
        "metric": METRIC,
        "value": round(main_res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Q, K, V i.i.d. N(0,1) (seed 0) rounded to bf16",
        "config": {"workload": "bf16_causal_e128", "B": w["B"], "H": w["Hq"], "L": w["L"], "S": w["S"],
                   "E": w["E"], "is_causal": True, "scale": "1/sqrt(128)", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic("prefill_pp_kernel"),
                     "kernel": "prefill_pp_kernel<BF16,128,causal>",
                     "flop_per_launch": main_res["flops"]},
        "cpu_baseline": None if a.no_cpu_baseline else cpu_baseline(),
        "secondary": secondary,
    }
    if not a.no_cpu_baseline and run_all:
        cpu = cpu_secondary()
        beside = {"bf16_neox_e96 scale=1/sqrt96": "bf16_neox_e96", "bf16_neox_e96 alibi+causal":
                  "bf16_neox_e96 alibi+causal", "fp16_varlen_e64": "fp16_varlen_e64",
                  "fp32_single_head": "fp32_single_head", "bf16_gqa_decode": "bf16_gqa_decode",
                  "bf16_gqa_decode paged": "bf16_gqa_decode"}
        for name, key in beside.items():
            if name in secondary:
                secondary[name]["cpu_oracle"] = cpu[key]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
