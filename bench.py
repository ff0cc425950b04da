"""Benchmark of the paged decode step on one MI355X.

Workload (one "step" = one pass of the whole decode path over one batch): the GQA decode
batch -- 256 sequences, 64 query / 8 KV heads, head_dim 128, bf16 cache, 16-token blocks at
seeded random physical placement, context lengths log-normal (median 512, sigma 1) clipped to
[16, 4096]. Each step stores one new token per sequence and decodes all sequences with
``paged_attn_decode_append`` (the append fused into the decode). Inputs are resident in HBM
before timing starts. ``--workload mha`` / ``long`` put the multi-head fp16 batch or the
long-context batch in the headline loop instead (for profiling those configs on their own).

Prints ONE JSON line. ``value`` is KV bytes per step (2 * sum(L) * H_kv * d * sizeof, each KV
head once) divided by the measured step time: K steps launched back to back, wall clock
around them, the library's own timing off (the same step captured in a HIP graph and replayed
is reported under ``graph_replay``). ``roofline`` reports the decode kernel: the same KV bytes
divided by that kernel's average duration, from hipEvents the library records on the launch
stream around every launch of a dedicated loop of ``--kernel-launches`` steps (100 by
default, whatever ``--steps`` is), against the 8 TB/s HBM peak. ``cpu_baseline`` times the CPU oracle (fp64, one
thread) on the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak of MI355X
KERNEL_LAUNCHES = 100
# untimed steps before any timing: the first ~60 decode launches of a process run 176-182 us and
# later ones settle at ~165 us (rocprofv3 kernel traces), so the device is brought to that state
DEVICE_WARMUP_STEPS = 100
METRIC = "paged decode attention KV GB/s (fraction of HBM peak) and seq-steps/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_mfma_gqa256_b16_traffic.json")
KERNEL_SOURCES = ["paged_kv_cache_127_amd/csrc/decode_mfma.hip",
                  "paged_kv_cache_127_amd/csrc/device_common.h",
                  "paged_kv_cache_127_amd/csrc/mfma_common.h",
                  "paged_kv_cache_127_amd/csrc/schedule.h"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(block_size: int, workers: int):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on the
    current kernel source and the same launch configuration; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    if t.get("block_size") != block_size or t.get("num_workers") != workers:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(batch, steps: int):
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for _ in range(steps):
            oracle.paged_decode(batch.q, batch.k_pool, batch.v_pool, batch.tables, batch.lengths,
                                batch.block_size)
        dt = time.perf_counter() - t0
    per_step = dt / steps
    return {
        "value": round(batch.kv_bytes / per_step / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"the full batch ({batch.num_seqs} sequences, sum L = {int(batch.lengths.sum())}), "
                   f"{steps} decode steps, numpy fp64 with one BLAS thread"),
        "seq_steps_per_s": round(batch.num_seqs / per_step, 2),
        "seconds": round(dt, 2),
    }


def _kernel_times(pkv, torch, launch, names, launches: int):
    """({kernel name: mean us}, step p50 us) of `launch` (one call sequence): the step from
    torch events around every call with the library's own timing off, then the kernels from
    hipEvents around every launch of each library kernel in a second run. 60 untimed calls
    first: launches over freshly allocated pools run a few percent slower for their first
    few dozen calls."""
    for _ in range(60):
        launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    for a, b_ in ev:
        a.record()
        launch()
        b_.record()
    torch.cuda.synchronize()
    steps = sorted(a.elapsed_time(b_) * 1e3 for a, b_ in ev)
    pkv.timing_enable(True, every=1)
    for _ in range(launches):
        launch()
    torch.cuda.synchronize()
    out = {}
    for name in names:
        ms, n = pkv.timing_query(name)
        out[name] = ms / n * 1e3 if n else 0.0
    pkv.timing_enable(False)
    return out, steps[len(steps) // 2]


def _decode_timing(pkv, torch, launch, launches: int):
    """(decode us, merge us, append us, copy us, step p50 us) of `launch` (see _kernel_times)."""
    names = ("decode_partial", "splitk_reduce", "append", "cow")
    kt, step = _kernel_times(pkv, torch, launch, names, launches)
    return [kt[n] for n in names] + [step]


def kernel_loop(pkv, torch, launch, names, launches: int):
    """{kernel name: (mean us, launches timed)} over `launches` calls of `launch`, from the
    hipEvents the library records on the launch stream around every launch of each kernel."""
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    pkv.timing_enable(True, every=1)
    for _ in range(launches):
        launch()
    torch.cuda.synchronize()
    out = {}
    for name in names:
        ms, n = pkv.timing_query(name)
        out[name] = (ms / n * 1e3 if n else 0.0, n)
    pkv.timing_enable(False)
    return out


def other_configs(pkv, W, torch, dev: str, workers: int, launches: int = 50):
    """Figures on the other batch configs: decode-kernel roofline for the HBM-bound ones (GQA
    at block size 32, multi-head fp16, long contexts with their 8-token append per step),
    logical GB/s for the shared-prefix batch (cache-assisted, no HBM claim), and latencies for
    the tiny and copy-on-write configs (no roofline claim). Kernel durations from hipEvents
    around every launch; step p50 from events around every call."""
    import numpy as np
    res = {}

    def stage(b):
        t = dict(q=b.q.to(dev), kp=b.k_pool.to(dev), vp=b.v_pool.to(dev),
                 tab=torch.from_numpy(b.tables).to(dev), lens=torch.from_numpy(b.lengths).to(dev))
        S, Hq, d = b.q.shape
        t["out"] = torch.empty(S, Hq, d, dtype=torch.float32, device=dev)
        t["ws"] = pkv.decode_workspace(S, Hq, b.num_kv_heads, d, workers, dev)
        t["mx"] = int(b.lengths.max())
        return t

    def decode_call(t, tab=None, lens=None, mx=None):
        pkv.paged_attn_decode(t["out"], t["q"], t["kp"], t["vp"], t["tab"] if tab is None else tab,
                              t["lens"] if lens is None else lens, t["mx"] if mx is None else mx,
                              num_workers=workers, workspace=t["ws"])

    def hbm_entry(desc, b, dus, mus, aus, step):
        gbs = b.kv_bytes / (dus * 1e-6) / 1e9
        e = {"workload": desc, "kv_bytes": b.kv_bytes, "decode_us": round(dus, 2),
             "merge_us": round(mus, 2), "achieved_gbs": round(gbs, 1),
             "frac": round(gbs / HBM_PEAK_GBS, 4), "step_p50_us": round(step, 2),
             "step_gbs": round(b.kv_bytes / (step * 1e-6) / 1e9, 1)}
        if aus:
            e["append_us"] = round(aus, 2)
        return e

    # GQA batch at block size 32
    b = W.config3(32)
    t = stage(b)
    dus, mus, aus, cus, step = _decode_timing(pkv, torch, lambda: decode_call(t), launches)
    res["gqa256_b32"] = hbm_entry("GQA decode batch at block size 32 (as above), decode + merge",
                                  b, dus, mus, 0, step)
    del t
    # multi-head fp16 batch
    b = W.config2()
    t = stage(b)
    dus, mus, aus, cus, step = _decode_timing(pkv, torch, lambda: decode_call(t), launches)
    res["mha64_fp16"] = hbm_entry("MHA decode batch: 64 sequences, 32/32 heads, head_dim 128, "
                                  "fp16, block size 16, lengths uniform in [128, 2048]; decode + "
                                  "merge", b, dus, mus, 0, step)
    del t
    # long contexts: one 8-token append (the current token of each sequence, rewritten) + decode
    b = W.config5(steps=1)
    t = stage(b)
    kn, vn = (x.to(dev) for x in W.new_tokens(b.seed, 1, b.num_seqs, b.num_kv_heads,
                                              b.head_dim, b.dtype))

    def long_step():
        pkv.paged_attn_decode_append(t["out"], t["q"], t["kp"], t["vp"], kn, vn, t["tab"],
                                     t["lens"], t["mx"], num_workers=workers, workspace=t["ws"])
    dus, mus, aus, cus, step = _decode_timing(pkv, torch, long_step, launches)
    res["long8_bf16"] = hbm_entry("long contexts: 8 sequences, 64/8 heads, head_dim 128, bf16, "
                                  "block size 16, lengths uniform in [16384, 32768]; step = "
                                  "decode with the 8-token append fused in + merge", b, dus, mus,
                                  aus, step)
    # the engine's table-row upload per step (pinned host rows -> device, on the same stream)
    host_tab = torch.from_numpy(b.tables).pin_memory()

    def long_step_upload():
        t["tab"].copy_(host_tab, non_blocking=True)
        long_step()
    _, _, _, _, step_up = _decode_timing(pkv, torch, long_step_upload, launches)
    res["long8_bf16"]["step_with_table_upload_p50_us"] = round(step_up, 2)
    del t
    # shared prefix: 128 sequences over one 800-token prefix (logical bytes; the prefix blocks
    # are re-read by every sharer, so caches serve most of them), plain decode and the
    # shared-prefix call; then the same over 4096- and 8192-token prefixes
    for P, key in ((800, "shared_prefix128"), (4096, "shared_prefix128_p4096"),
                   (8192, "shared_prefix128_p8192")):
        b = W.config4a(prefix_len=P)
        t = stage(b)
        dus, mus, aus, cus, step = _decode_timing(pkv, torch, lambda: decode_call(t), launches)
        S, Hq, d = b.q.shape
        pre = t["tab"][0, :P // b.block_size].contiguous()
        ws_sp = pkv.shared_prefix_workspace(S, Hq, b.num_kv_heads, d, P, workers, dev)

        def sp_call():
            pkv.paged_attn_decode_shared_prefix(t["out"], t["q"], t["kp"], t["vp"], pre, P,
                                                t["tab"], t["lens"], t["mx"],
                                                num_workers=workers, workspace=ws_sp)
        kt, sp_step = _kernel_times(pkv, torch, sp_call, ("prefix_states", "decode_partial",
                                                           "splitk_reduce"), launches)
        unique = 2 * (P + int(b.lengths.sum()) - S * P) * b.num_kv_heads * d * 2
        res[key] = {
            "workload": f"shared prefix: 128 sequences, {P}-token shared prefix + U{{1..512}} "
                        "private tokens, 64/8 heads, head_dim 128, bf16, block size 16",
            "logical_kv_bytes": b.kv_bytes, "unique_kv_bytes": unique,
            "decode_us": round(dus, 2), "merge_us": round(mus, 2),
            "logical_gbs": round(b.kv_bytes / (dus * 1e-6) / 1e9, 1), "cache_assisted": True,
            "step_p50_us": round(step, 2),
            "shared_prefix_call": {
                "what": "paged_attn_decode_shared_prefix on the same batch: prefix states of "
                        "all sharers' rows (prefix read once), decode over the suffixes, merge",
                "kernel_us": {k: round(v, 2) for k, v in kt.items()},
                "step_p50_us": round(sp_step, 2),
                "logical_gbs": round(b.kv_bytes / (sp_step * 1e-6) / 1e9, 1),
                "speedup_vs_plain_step": round(step / sp_step, 3)}}
        # the prefix pass against the dense bf16 matrix peak: 4 * S * H_q * d * P flops
        pf = 4 * S * Hq * d * P / (kt["prefix_states"] * 1e-6) / 1e12
        res[key]["shared_prefix_call"]["prefix_states_roofline"] = {
            "bound": "mfma", "achieved": round(pf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(pf / MFMA_BF16_PEAK_TFLOPS, 4)}
        del t, ws_sp
    # copy-on-write pairs: copy 8 slots of each pair's shared partial block, append B's token,
    # decode all 128 sequences (the copy and append rewrite the same slots every call)
    b = W.config4b()
    t = stage(b)
    free = W.config4b_free_blocks(b)
    npairs = b.num_seqs // 2
    tab2 = b.tables.copy()
    src, dst = [], []
    for i in range(npairs):
        src.append(int(b.tables[2 * i + 1][1]))
        dst.append(free[i])
        tab2[2 * i + 1][1] = free[i]
    as_dev = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
    dsrc, ddst, dn = as_dev(src), as_dev(dst), as_dev([8] * npairs)
    dtab2 = torch.from_numpy(tab2).to(dev)
    lens2 = torch.from_numpy(np.tile(np.array([24, 25], np.int32), npairs)).to(dev)
    kn, vn = (x.to(dev) for x in W.new_tokens(b.seed, 1, npairs, b.num_kv_heads, b.head_dim,
                                              b.dtype))
    bsid, bpos = as_dev(list(range(1, 2 * npairs, 2))), as_dev([24] * npairs)

    def cow_step():
        pkv.cow_block_copy(t["kp"], t["vp"], dsrc, ddst, dn)
        pkv.kv_cache_append(t["kp"], t["vp"], kn, vn, bsid, bpos, dtab2)
        decode_call(t, tab=dtab2, lens=lens2, mx=25)
    dus, mus, aus, cus, step = _decode_timing(pkv, torch, cow_step, launches)
    res["cow_pairs64"] = {
        "workload": "copy-on-write: 64 pairs sharing 24 tokens; per call copy 8 slots of each "
                    "shared partial block, append B's token, decode 128 sequences",
        "copy_us": round(cus, 2), "append_us": round(aus, 2), "decode_us": round(dus, 2),
        "merge_us": round(mus, 2), "step_p50_us": round(step, 2), "roofline": None}
    del t
    # tiny: the pages' three requests (25, 47, 12 tokens), fp32
    b = W.config1()
    t = stage(b)
    dus, mus, aus, cus, step = _decode_timing(pkv, torch, lambda: decode_call(t), launches)
    res["tiny3_fp32"] = {"workload": "tiny: 3 sequences of 25, 47, 12 tokens, 4/4 heads, head_dim "
                                     "64, fp32, block size 16", "decode_us": round(dus, 2),
                         "merge_us": round(mus, 2), "step_p50_us": round(step, 2),
                         "roofline": None}
    del t
    torch.cuda.empty_cache()
    for k, v in res.items():
        print(f"bench: {k} decode {v['decode_us']} us step p50 {v['step_p50_us']} us",
              file=sys.stderr, flush=True)
    return res


def swap_figures(pkv, W, torch, dev: str, preempt: int = 32, launches: int = 10):
    """Preemption of the first `preempt` sequences of the GQA batch (block size 16): every block
    they hold goes to pinned host memory in one kv_swap_out and comes back into other free
    device blocks in one kv_swap_in. Kernel durations from hipEvents around every launch. The
    host-link ceiling is a plain DMA copy (torch copy_, i.e. hipMemcpyAsync) of the same bytes
    between one contiguous device buffer and pinned host memory, each direction."""
    b = W.config3(16)
    kp, vp = b.k_pool.to(dev), b.v_pool.to(dev)
    blocks = [int(x) for s in range(preempt) for x in b.tables[s] if x >= 0]
    n = len(blocks)
    used = set(int(x) for x in b.tables.ravel() if x >= 0)
    free = [x for x in range(b.num_blocks) if x not in used][:n]
    if len(free) < n:
        raise RuntimeError("pool too small for the swap-in destinations")
    shape = (n,) + tuple(kp.shape[1:])
    hk = torch.empty(shape, dtype=kp.dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=kp.dtype, pin_memory=True)
    ids = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
    dev_ids, host_ids, back_ids = ids(blocks), ids(list(range(n))), ids(free)

    def kernel_us(name, fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        pkv.timing_enable(True, every=1)
        for _ in range(launches):
            fn()
        torch.cuda.synchronize()
        ms, cnt = pkv.timing_query(name)
        pkv.timing_enable(False)
        return ms / cnt * 1e3

    out_us = kernel_us("swap_out", lambda: pkv.kv_swap_out(kp, vp, hk, hv, dev_ids, host_ids))
    in_us = kernel_us("swap_in", lambda: pkv.kv_swap_in(kp, vp, hk, hv, host_ids, back_ids))
    torch.cuda.synchronize()
    # the GQA decode alone, then with swap-outs running on a second stream meanwhile
    q, tab, lens = b.q.to(dev), torch.from_numpy(b.tables).to(dev), torch.from_numpy(b.lengths).to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = pkv.decode_workspace(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, 0, dev)
    dec = lambda: pkv.paged_attn_decode(out, q, kp, vp, tab, lens, int(b.lengths.max()),
                                        workspace=ws)
    dec_alone = kernel_us("decode_partial", dec)
    s2 = torch.cuda.Stream()
    pkv.timing_enable(True, every=1)
    for _ in range(3):
        pkv.kv_swap_out(kp, vp, hk, hv, dev_ids, host_ids, stream=s2)
    for _ in range(20):      # about 4 ms of decode against 5 ms of swap-out
        dec()
    torch.cuda.synchronize()
    dms, dn = pkv.timing_query("decode_partial")
    sms, sn = pkv.timing_query("swap_out")
    pkv.timing_enable(False)
    # the copy-engine variant (host run 0..n-1): call time from torch events on its stream, and
    # the decode with copy-engine swap-outs on the second stream meanwhile
    staging = pkv.swap_staging(n, kp)

    def call_us(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(launches)]
        for a, e in ev:
            a.record()
            fn()
            e.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(e) * 1e3 for a, e in ev)
        return t[len(t) // 2]

    dma_out_us = call_us(lambda: pkv.kv_swap_out_dma(kp, vp, hk, hv, dev_ids, 0, staging))
    dma_in_us = call_us(lambda: pkv.kv_swap_in_dma(kp, vp, hk, hv, 0, back_ids, staging))
    pkv.timing_enable(True, every=1)
    for _ in range(3):
        pkv.kv_swap_out_dma(kp, vp, hk, hv, dev_ids, 0, staging, stream=s2)
    for _ in range(20):
        dec()
    torch.cuda.synchronize()
    dms2, dn2 = pkv.timing_query("decode_partial")
    pkv.timing_enable(False)
    dma_moved = (torch.equal(hk[n - 1].view(torch.int16), b.k_pool[blocks[-1]].view(torch.int16))
                 and torch.equal(kp[free[0]].cpu().view(torch.int16),
                                 b.k_pool[blocks[0]].view(torch.int16)))
    del q, tab, lens, out, ws, staging
    moved = (torch.equal(hk[0].view(torch.int16), b.k_pool[blocks[0]].view(torch.int16)) and
             torch.equal(kp[free[-1]].cpu().view(torch.int16),
                         b.k_pool[blocks[-1]].view(torch.int16)))
    nbytes = 2 * hk.numel() * hk.element_size()
    del kp, vp
    dbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)

    def dma_us(dst, src):
        for _ in range(2):
            dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(launches)]
        for a, e in ev:
            a.record()
            dst.copy_(src, non_blocking=True)
            e.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(e) * 1e3 for a, e in ev)
        return t[len(t) // 2]

    d2h_us, h2d_us = dma_us(hbuf, dbuf), dma_us(dbuf, hbuf)
    del dbuf, hbuf
    torch.cuda.empty_cache()
    gbs = lambda us: round(nbytes / (us * 1e-6) / 1e9, 2)
    res = {
        "workload": f"preempt the first {preempt} sequences of the GQA decode batch (block size "
                    f"16): {n} blocks of 8 heads x 16 slots x 128 bf16, keys and values, out to "
                    "pinned host memory in one call and back into other free blocks in one call",
        "blocks": n, "bytes": nbytes, "data_checked": bool(moved),
        "swap_out_us": round(out_us, 2), "swap_out_gbs": gbs(out_us),
        "swap_in_us": round(in_us, 2), "swap_in_gbs": gbs(in_us),
        "dma_d2h_us": round(d2h_us, 2), "dma_d2h_gbs": gbs(d2h_us),
        "dma_h2d_us": round(h2d_us, 2), "dma_h2d_gbs": gbs(h2d_us),
        "out_frac_of_dma": round(d2h_us / out_us, 4), "in_frac_of_dma": round(h2d_us / in_us, 4),
        "bound": "host link (ceiling: contiguous DMA copy of the same bytes)",
        "overlap": {"what": "swap-outs on a second stream while the GQA decode (plain call) runs",
                    "decode_us_alone": round(dec_alone, 2),
                    "decode_us_during_swap": round(dms / dn * 1e3, 2),
                    "swap_out_gbs_during_decode": gbs(sms / sn * 1e3)},
        "copy_engine": {"what": "kv_swap_out_dma / kv_swap_in_dma of the same blocks (gather or "
                                "scatter through a device staging buffer, one DMA copy per "
                                "pool); call time from torch events",
                        "data_checked": bool(dma_moved),
                        "swap_out_us": round(dma_out_us, 2), "swap_out_gbs": gbs(dma_out_us),
                        "swap_in_us": round(dma_in_us, 2), "swap_in_gbs": gbs(dma_in_us),
                        "decode_us_during_swap": round(dms2 / dn2 * 1e3, 2)},
    }
    print(f"bench: swap out {res['swap_out_gbs']} GB/s in {res['swap_in_gbs']} GB/s "
          f"(DMA {res['dma_d2h_gbs']} / {res['dma_h2d_gbs']}); copy-engine swap out "
          f"{res['copy_engine']['swap_out_gbs']} in {res['copy_engine']['swap_in_gbs']} GB/s, "
          f"decode meanwhile {res['copy_engine']['decode_us_during_swap']} us",
          file=sys.stderr, flush=True)
    return res


def extend_figures(pkv, W, torch, dev: str, launches: int = 20):
    """Extend (multi-query, causal) attention: (1) speculative verification on the GQA batch --
    each sequence's last 4 stored tokens are the new ones -- against the plain decode of the
    same batch; (2) a prefill chunk: 8 sequences of 1024..4096 tokens whose last 256 are new.
    Kernel durations from hipEvents around every launch, call p50 from torch events."""
    import numpy as np
    res = {}

    def run(b, new, seed, key, desc, bound):
        q, start = W.extend_queries(b, new, seed=seed)
        qd, sd = q.to(dev), torch.from_numpy(start).to(dev)
        kp, vp = b.k_pool.to(dev), b.v_pool.to(dev)
        tab, lens = torch.from_numpy(b.tables).to(dev), torch.from_numpy(b.lengths).to(dev)
        mx, maxq = int(b.lengths.max()), int(np.max(new))
        out = torch.empty(qd.shape, dtype=torch.float32, device=dev)
        ws = pkv.extend_workspace(b.num_seqs, qd.shape[0], b.num_q_heads, b.num_kv_heads,
                                  b.head_dim, maxq, mx, dev)

        def call():
            pkv.paged_attn_extend(out, qd, sd, maxq, kp, vp, tab, lens, mx, workspace=ws)
        kt, step = _kernel_times(pkv, torch, call, ("extend_states", "extend_finish"), launches)
        # causal work: row (s, t, h) attends L_s - n_s + t + 1 positions
        att = sum(int(n) * (2 * int(L) - int(n) + 1) // 2 for L, n in zip(b.lengths, new))
        flops = 4 * att * b.num_q_heads * b.head_dim
        r = {"workload": desc, "query_tokens": int(np.sum(new)), "kv_bytes": b.kv_bytes,
             "kernel_us": {k: round(v, 2) for k, v in kt.items()},
             "step_p50_us": round(step, 2),
             "kv_gbs": round(b.kv_bytes / (step * 1e-6) / 1e9, 1),
             "tflops": round(flops / (step * 1e-6) / 1e12, 2)}
        # the kernels' own time against the bound of the run: context bytes against the HBM
        # peak for short runs, causal-attention flops against the dense bf16 matrix peak for
        # prefill chunks
        kus = sum(kt.values())
        if bound == "hbm":
            a = b.kv_bytes / (kus * 1e-6) / 1e9
            r["roofline"] = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4)}
        else:
            a = flops / (kus * 1e-6) / 1e12
            r["roofline"] = {"bound": "mfma", "achieved": round(a, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4)}
        del kp, vp, out, ws
        return r

    b = W.config3(16)
    new = np.minimum(4, b.lengths)
    res["spec_verify4_gqa256"] = run(b, new, 71, "spec", "speculative verification: the GQA "
                                     "decode batch (256 sequences, 64/8 heads, d 128, bf16, B "
                                     "16), the last 4 stored tokens of each sequence as new "
                                     "query tokens (1,024 rows per KV head)", "hbm")
    b = W.small_batch(W.rng_for(W.SEED_BASE + 9, 0).integers(1024, 4096, size=8, endpoint=True),
                      64, 8, 128, 16, torch.bfloat16, seed=W.SEED_BASE + 9)
    new = np.full(8, 256)
    res["prefill_chunk256_x8"] = run(b, new, 72, "prefill", "prefill chunk: 8 sequences of "
                                     "1024..4096 stored tokens (64/8 heads, d 128, bf16, B 16), "
                                     "the last 256 of each new (2,048 query tokens)", "mfma")
    torch.cuda.empty_cache()
    for k, v in res.items():
        print(f"bench: {k} step p50 {v['step_p50_us']} us, {v['tflops']} TFLOP/s",
              file=sys.stderr, flush=True)
    return res


def prefix_index_figures(pkv, requests: int = 500):
    """The host prefix index on the shared system prompt of "KV Cache Optimization and
    Management" (Worked Example 2): 500 requests of a 380-token prompt + a 90-token question,
    block size 16. Each request matches, allocates the rest, inserts its blocks and finishes;
    reported: blocks held with and without sharing, host microseconds per request in match and
    insert (through the Python binding)."""
    import numpy as np
    rng = np.random.default_rng(2024)
    B = 16
    prompt = rng.integers(0, 50000, 380).tolist()
    pool = pkv.BlockPool(40000)
    idx = pkv.PrefixIndex(pool, B)
    t_index = 0.0
    matched = 0
    for _ in range(requests):
        toks = prompt + rng.integers(0, 50000, 90).tolist()
        t0 = time.perf_counter()
        got = idx.match(toks)
        t_index += time.perf_counter() - t0
        matched += len(got)
        mine = got + [pool.alloc() for _ in range(-(-len(toks) // B) - len(got))]
        t0 = time.perf_counter()
        idx.insert(toks, mine)
        t_index += time.perf_counter() - t0
        for b in mine:                 # the request finishes; the index keeps its blocks
            pool.decref(b)
    us = t_index * 1e6 / requests
    held = idx.size()
    per_request = -(-470 // B)
    return {"workload": f"{requests} requests: 380-token shared prompt + 90-token question, "
                        "block size 16 (match, allocate, insert, finish per request)",
            "blocks_held": held, "blocks_without_sharing": per_request * requests,
            "shared_blocks_matched_per_request": round(matched / max(requests - 1, 1), 2),
            "host_us_per_request_match_and_insert": round(us, 2)}


def mfma_probe(pkv, torch, dev: str, iters: int = 4000, launches: int = 5):
    """What 16x16x32 bf16 MFMAs sustain here (the library's probe), with one, two and four
    wavefronts per SIMD (1, 2 and 4 workgroups of 4 wavefronts per CU)."""
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    res = {}
    for per_cu in (1, 2, 4):
        wgs = cus * per_cu
        pkv.mfma_rate_probe(wgs, 10, sink)
        torch.cuda.synchronize()
        pkv.timing_enable(True, every=1)
        for _ in range(launches):
            pkv.mfma_rate_probe(wgs, iters, sink)
        torch.cuda.synchronize()
        ms, n = pkv.timing_query("mfma_rate")
        pkv.timing_enable(False)
        flops = wgs * 4 * iters * 8 * 16384
        res[f"waves_per_simd_{per_cu}_tflops"] = round(flops / (ms / n * 1e-3) / 1e12, 1)
    return res


def stream_probe(pkv, torch, dev: str, gib: int = 2, launches: int = 20):
    """Plain streaming-read bandwidth of this device (the library's probe kernel)."""
    buf = torch.ones((gib << 30) // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        pkv.stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    pkv.timing_enable(True, every=1)
    for _ in range(launches):
        pkv.stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    ms, n = pkv.timing_query("stream_read")
    pkv.timing_enable(False)
    nbytes = buf.numel() * 4
    del buf
    torch.cuda.empty_cache()
    us = ms / n * 1e3
    return {"bytes": nbytes, "us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def cpu_baseline_multi(block_size: int, steps: int = 3):
    """The oracle over a process pool (one worker per host core this process may use, at most
    16), run in a child interpreter that never touches the GPU: same batch, same oracle,
    sequences split across the workers. The workers see the batch as NumPy arrays (the 16-bit
    values widened to fp32, exactly) and use no torch, so nothing threaded is forked."""
    import subprocess
    code = (
        "import os, sys, time, json\n"
        "os.environ['OMP_NUM_THREADS'] = os.environ['OPENBLAS_NUM_THREADS'] = '1'\n"
        "sys.path.insert(0, %r)\n"
        "import numpy as np, multiprocessing as mp, torch\n"
        "import workloads as W, oracle\n"
        "b = W.config3(%d)\n"
        "q, kp, vp = (x.float().numpy() for x in (b.q, b.k_pool, b.v_pool))\n"
        "tables, lengths, B, kvb, S = b.tables, b.lengths, b.block_size, b.kv_bytes, b.num_seqs\n"
        "del b\n"
        "def run(seqs):\n"
        "    oracle.paged_decode(q, kp, vp, tables, lengths, B, seqs=seqs)\n"
        "    return len(seqs)\n"
        "n = min(16, len(os.sched_getaffinity(0)))\n"
        "parts = [list(range(i, S, n)) for i in range(n)]\n"
        "print('cpu baseline: %%d processes' %% n, file=sys.stderr, flush=True)\n"
        "with mp.get_context('fork').Pool(n) as pool:\n"
        "    pool.map_async(run, parts).get(timeout=120)\n"
        "    t = time.perf_counter()\n"
        "    for _ in range(%d):\n"
        "        pool.map_async(run, parts).get(timeout=120)\n"
        "        print('cpu baseline: step done', file=sys.stderr, flush=True)\n"
        "    dt = (time.perf_counter() - t) / %d\n"
        "print(json.dumps({'cores': n, 'step_s': dt, 'kv_bytes': kvb, 'S': S}))\n"
    ) % (ROOT, block_size, steps, steps)
    try:
        r = subprocess.run([sys.executable, "-c", code], stdout=subprocess.PIPE, text=True,
                           timeout=400)
    except subprocess.TimeoutExpired:
        return {"error": "timed out"}
    if r.returncode != 0 or not r.stdout.strip():
        return {"error": f"exit status {r.returncode}"}
    d = json.loads(r.stdout.strip().splitlines()[-1])
    return {"value": round(d["kv_bytes"] / d["step_s"] / 1e9, 4), "unit": "GB/s",
            "cores": d["cores"], "kind": "oracle",
            "sample": f"the full batch, {steps} decode steps after one warm-up, sequences split "
                      f"over a pool of {d['cores']} processes (one BLAS thread each)",
            "seq_steps_per_s": round(d["S"] / d["step_s"], 2)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def headline_workload(name, block_size, W, torch, dev):
    """The batch, the step and its description for the workload the JSON line reports.

    gqa (default): the GQA decode batch at ``block_size``; a step appends one new token per
    sequence (it rewrites the current token's slot, so the batch is the same every step) and
    decodes all sequences with ``paged_attn_decode_append``. mha: the multi-head fp16 batch,
    a plain decode per step. long: the long-context batch, one appended token per sequence
    fused into the decode. The last two exist so that each HBM-bound config can be profiled
    on its own; the default line is the GQA batch."""
    if name == "gqa":
        b = W.config3(block_size)
        desc = (f"GQA decode batch: {b.num_seqs} sequences, {b.num_q_heads} query / "
                f"{b.num_kv_heads} KV heads, head_dim {b.head_dim}, bf16 cache, block size "
                f"{block_size}, log-normal context lengths (median 512, sigma 1, clipped to "
                "[16, 4096]), seeded random block placement in a 1.25x pool; one appended "
                "token per sequence per step (paged_attn_decode_append: append fused into the "
                "decode kernel)")
        append = True
    elif name == "mha":
        b = W.config2()
        desc = ("MHA decode batch: 64 sequences, 32 query / 32 KV heads, head_dim 128, fp16 "
                "cache, block size 16, context lengths uniform in [128, 2048], seeded random "
                "block placement in a 1.25x pool; one decode per step (paged_attn_decode)")
        append = False
    else:
        b = W.config5(steps=1)
        desc = ("long contexts: 8 sequences, 64 query / 8 KV heads, head_dim 128, bf16 cache, "
                "block size 16, context lengths uniform in [16384, 32768]; one appended token "
                "per sequence per step (paged_attn_decode_append)")
        append = True
    return b, desc, append


def row_state_line(args, pkv, W, torch, dev):
    """One JSON line for a row-state call alone (for profiling the matrix-core kernel):
    prefix800 / prefix4096 / prefix8192 -- paged_attn_decode_shared_prefix on 128 sequences over
    an 800-, 4096- or 8192-token shared prefix (the prefix-state kernel, the suffix decode and
    the merge);
    prefill -- paged_attn_extend of a 256-token chunk on 8 sequences of 1024..4096 tokens;
    verify -- paged_attn_extend of the last 4 tokens of every sequence of the GQA batch.
    ``value`` is the call's causal-attention rate in TFLOP/s (prefix: the prefix-state kernel's
    flops over the whole call)."""
    import numpy as np
    if args.workload.startswith("prefix"):
        P = int(args.workload[6:])
        b = W.config4a(prefix_len=P)
        S, Hq, d = b.q.shape
        q, kp, vp = b.q.to(dev), b.k_pool.to(dev), b.v_pool.to(dev)
        tab, lens = torch.from_numpy(b.tables).to(dev), torch.from_numpy(b.lengths).to(dev)
        mx = int(b.lengths.max())
        out = torch.empty(S, Hq, d, dtype=torch.float32, device=dev)
        pre = tab[0, :P // b.block_size].contiguous()
        ws = pkv.shared_prefix_workspace(S, Hq, b.num_kv_heads, d, P, args.workers, dev)

        def call():
            pkv.paged_attn_decode_shared_prefix(out, q, kp, vp, pre, P, tab, lens, mx,
                                                num_workers=args.workers, workspace=ws)
        kname = "prefix_states"
        flops = 4 * S * Hq * d * P
        desc = (f"shared prefix: 128 sequences, {P}-token shared prefix + U{{1..512}} private "
                "tokens, 64/8 heads, head_dim 128, bf16, block size 16; one "
                "paged_attn_decode_shared_prefix call per step")
    else:
        if args.workload == "prefill":
            b = W.small_batch(W.rng_for(W.SEED_BASE + 9, 0).integers(1024, 4096, size=8,
                                                                    endpoint=True),
                              64, 8, 128, 16, torch.bfloat16, seed=W.SEED_BASE + 9)
            new = np.full(8, 256)
            seed, desc = 72, ("prefill chunk: 8 sequences of 1024..4096 stored tokens (64/8 heads, "
                              "d 128, bf16, B 16), the last 256 of each new; one paged_attn_extend "
                              "call per step")
        else:
            b = W.config3(16)
            new = np.minimum(4, b.lengths)
            seed, desc = 71, ("speculative verification: the GQA decode batch, the last 4 stored "
                              "tokens of each sequence as new query tokens; one paged_attn_extend "
                              "call per step")
        qn, start = W.extend_queries(b, new, seed=seed)
        qd, sd = qn.to(dev), torch.from_numpy(start).to(dev)
        kp, vp = b.k_pool.to(dev), b.v_pool.to(dev)
        tab, lens = torch.from_numpy(b.tables).to(dev), torch.from_numpy(b.lengths).to(dev)
        mx, maxq = int(b.lengths.max()), int(np.max(new))
        out = torch.empty(qd.shape, dtype=torch.float32, device=dev)
        ws = pkv.extend_workspace(b.num_seqs, qd.shape[0], b.num_q_heads, b.num_kv_heads,
                                  b.head_dim, maxq, mx, dev)

        def call():
            pkv.paged_attn_extend(out, qd, sd, maxq, kp, vp, tab, lens, mx, workspace=ws)
        kname = "extend_states"
        att = sum(int(n) * (2 * int(L) - int(n) + 1) // 2 for L, n in zip(b.lengths, new))
        flops = 4 * att * b.num_q_heads * b.head_dim
    for _ in range(DEVICE_WARMUP_STEPS):
        call()
    torch.cuda.synchronize()
    kt = kernel_loop(pkv, torch, call, (kname,), args.kernel_launches)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kus = kt[kname][0]
    print(json.dumps({
        "metric": "row-state call time (matrix-core kernel)", "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": desc, "flops_per_step": flops},
        "kernel": {"name": kname, "avg_us": round(kus, 3), "launches": kt[kname][1],
                   "tflops": round(flops / (kus * 1e-6) / 1e12, 2),
                   "frac_of_dense_bf16_peak": round(flops / (kus * 1e-6) / 2.5e15, 4)}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa",
                    choices=("gqa", "mha", "long", "prefix800", "prefix4096", "prefix8192",
                             "prefill", "verify"),
                    help="batch of the headline line (gqa by default; prefix*, prefill and verify "
                         "run the matrix-core row-state calls alone, for profiling them)")
    ap.add_argument("--block-size", type=int, default=16, choices=(16, 32))
    ap.add_argument("--workers", type=int, default=0, help="decode wavefronts (0 = automatic)")
    ap.add_argument("--kernel-launches", type=int, default=KERNEL_LAUNCHES,
                    help="launches in the dedicated kernel-timing loop")
    ap.add_argument("--cpu-steps", type=int, default=15,
                    help="decode steps of the CPU oracle (about 0.7 s each on one core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the figures on the other batch configs and the read probe")
    ap.add_argument("--no-graph-replay", action="store_true",
                    help="skip the HIP-graph replay comparison (counter runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_127_amd as pkv
    import workloads as W

    dev = "cuda:0"
    if args.workload in ("prefix800", "prefix4096", "prefix8192", "prefill", "verify"):
        row_state_line(args, pkv, W, torch, dev)
        return
    t_gen = time.perf_counter()
    b, desc, fused_append = headline_workload(args.workload, args.block_size, W, torch, dev)
    S, Hq, Hkv, d = b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim
    q = b.q.to(dev)
    k_pool = b.k_pool.to(dev)
    v_pool = b.v_pool.to(dev)
    tables = torch.from_numpy(b.tables).to(dev)
    lens = torch.from_numpy(b.lengths).to(dev)
    max_ctx = int(b.lengths.max())
    out = torch.empty(S, Hq, d, dtype=torch.float32, device=dev)
    ws = pkv.decode_workspace(S, Hq, Hkv, d, args.workers, dev)
    k_new, v_new = (x.to(dev) for x in W.new_tokens(b.seed, 1, S, Hkv, d, b.dtype))
    seq_ids = torch.arange(S, dtype=torch.int32, device=dev)
    positions = (lens - 1).to(torch.int32)
    gen_s = time.perf_counter() - t_gen
    dtype_name = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[b.dtype]

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # One decode step over the whole batch (see headline_workload). The same work as two calls
    # (kv_cache_append, then paged_attn_decode) is timed afterwards for comparison.
    def step():
        if fused_append:
            pkv.paged_attn_decode_append(out, q, k_pool, v_pool, k_new, v_new, tables, lens,
                                         max_ctx, num_workers=args.workers, workspace=ws)
        else:
            pkv.paged_attn_decode(out, q, k_pool, v_pool, tables, lens, max_ctx,
                                  num_workers=args.workers, workspace=ws)

    def step_two_calls():
        pkv.kv_cache_append(k_pool, v_pool, k_new, v_new, seq_ids, positions, tables)
        pkv.paged_attn_decode(out, q, k_pool, v_pool, tables, lens, max_ctx,
                              num_workers=args.workers, workspace=ws)

    # the device to its steady state first (untimed), then the kernel durations: a dedicated
    # loop of its own (independent of --steps), hipEvents stamped with each launch's own start
    # and end by the library, on the launch stream
    for _ in range(DEVICE_WARMUP_STEPS):
        step()
    torch.cuda.synchronize()
    kt = kernel_loop(pkv, torch, step, ("decode_partial", "splitk_reduce"), args.kernel_launches)
    kern_avg_us, kernel_n = kt["decode_partial"]
    reduce_us, _ = kt["splitk_reduce"]

    pkv.timing_enable(False)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # headline: K steps back to back, launched eagerly through the Python binding, the
    # library's own timing off, wall clock around them
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # the same step captured once in a HIP graph and replayed K times (for comparison: on this
    # ROCm release graph replays of this step run slower than eager launches)
    graph_ms = None
    if not args.no_graph_replay:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del graph

    kv_bytes = b.kv_bytes
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (kern_avg_us * 1e-6) / 1e9
    is_valu = Hq == Hkv or b.dtype == torch.float32
    kname = "decode_partial_valu" if is_valu else "decode_partial_mfma"
    traffic = measured_traffic(args.block_size, args.workers) if args.workload == "gqa" else None

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
        "config": {
            "workload": desc,
            "num_seqs": S,
            "sum_context_tokens": int(b.lengths.sum()),
            "block_size": b.block_size,
            "num_workers": args.workers or "auto",
            "kv_bytes_per_step": kv_bytes,
        },
        "step_launch": "eager calls through the Python binding, back to back",
        "graph_replay": None if graph_ms is None else {
            "what": "the same step captured in a HIP graph, K replays back to back",
            "ms_per_step": round(graph_ms, 5),
            "value": round(kv_bytes / (graph_ms * 1e-3) / 1e9, 2)},
        "seq_steps_per_s": round(S / (ms_per_step * 1e-3), 1),
        "hbm_fraction_of_step": round(value / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_kernel_us": round(kern_avg_us, 3),
            "timed_launches": kernel_n,
            "timing": (f"hipEvents stamped with the kernel's own start and end "
                       f"(hipExtLaunchKernelGGL) for each of {kernel_n} launches in a dedicated loop, "
                       f"after {DEVICE_WARMUP_STEPS} untimed steps and before the warm-up and timed "
                       "steps; the headline steps ran with the library's timing off"),
        },
        "other_kernels_avg_us": {"splitk_reduce": round(reduce_us, 3)},
        "setup_s": round(gen_s, 2),
    }
    if args.workload == "gqa":
        for _ in range(args.warmup):
            step_two_calls()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            step_two_calls()
        torch.cuda.synchronize()
        two_ms = (time.perf_counter() - t2) * 1e3 / args.steps
        kt2 = kernel_loop(pkv, torch, step_two_calls, ("decode_partial", "append"),
                          max(20, args.kernel_launches // 4))
        result["two_calls"] = {
            "what": "the same step as kv_cache_append + paged_attn_decode",
            "ms_per_step": round(two_ms, 5),
            "value": round(kv_bytes / (two_ms * 1e-3) / 1e9, 2),
            "decode_kernel_us": round(kt2["decode_partial"][0], 3),
            "append_kernel_us": round(kt2["append"][0], 3),
        }
    # step-time spread: torch events around every step (on the stream the library launches on)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(100)]
    for a, e in ev:
        a.record()
        step()
        e.record()
    torch.cuda.synchronize()
    st_us = sorted(a.elapsed_time(e) * 1e3 for a, e in ev)
    result["step_us_percentiles"] = {"p10": round(st_us[10], 2), "p50": round(st_us[50], 2),
                                     "p90": round(st_us[90], 2), "steps": len(st_us),
                                     "what": "torch events around each of 100 eager steps"}
    print(f"bench: step {ms_per_step * 1e3:.1f} us, decode kernel {kern_avg_us:.1f} us "
          f"({achieved / HBM_PEAK_GBS:.3f} of peak)", file=sys.stderr, flush=True)
    if not args.no_other_configs and args.workload == "gqa":
        del k_pool, v_pool, q, out, ws
        torch.cuda.empty_cache()
        probe = stream_probe(pkv, torch, dev)
        probe["decode_frac_of_probe"] = round(achieved / probe["gbs"], 4)
        result["read_probe"] = probe
        result["mfma_probe"] = mfma_probe(pkv, torch, dev)
        result["other_configs"] = other_configs(pkv, W, torch, dev, args.workers)
        result["swap"] = swap_figures(pkv, W, torch, dev)
        result["extend"] = extend_figures(pkv, W, torch, dev)
        result["prefix_index"] = prefix_index_figures(pkv)
    if not args.no_cpu_baseline and args.workload == "gqa":
        print("bench: oracle on one core", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(b, args.cpu_steps)
        print("bench: oracle on a process pool", file=sys.stderr, flush=True)
        result["cpu_baseline"]["cpu_model"] = cpu_model()
        result["cpu_baseline_multi"] = cpu_baseline_multi(args.block_size)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
