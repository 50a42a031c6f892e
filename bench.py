#!/usr/bin/env python3
"""Benchmark of the shared-KV attention path on one MI355X.

A step is one decode step of the 8-decoder Qwen3-8B-shaped agentic workload
over all 36 layers: for every layer, one shared_kv_decode_append call writes
the step's token K/V of every session into its page (the frozen base model's
cache store) and runs the N=8 decoders x 4 GQA heads of every KV head over the
shared pages, that token included.  `value` is the decode's algorithmic bytes per second over whole
steps.  Extend (partial prefill of 512 new tokens on 8K cached prefixes,
16 sessions) is timed alongside and reported as TFLOP/s under "extend".

Prints ONE JSON line.  Inputs are seeded synthetic tensors already resident in
HBM when timing starts.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
DECODE_WORKLOAD = "qwen3_8b_n8"
EXTEND_WORKLOAD = "extend_8k_512"
PRIVATE_WORKLOAD = "qwen3_8b_n8_private"
HANDOFF_WORKLOAD = "handoff_8k"
CASCADE_WORKLOAD = "qwen3_8b_n8_cascade"
LAYER_GROUP_WORKLOAD = "llama8b_layer_group"
# the other decode workloads, one layer each: Llama-3.1-8B-shaped (N=4, 1K-8K tokens) and
# Qwen3-14B-shaped long context (N=2, truncated log-normal lengths, mean 27K)
CONFIG_DECODE_WORKLOADS = ("llama8b_n4", "qwen3_14b_long")
# pool replicas a one-layer workload rotates over, so that no call finds its KV (or q, or
# chunk rows) in the 256 MB infinity cache left there by the call before
REPLICAS = 4


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--extend-calls", type=int, default=40)
    ap.add_argument("--extend-warmup", type=int, default=50)
    ap.add_argument("--private-calls", type=int, default=20)
    ap.add_argument("--no-private", action="store_true", help="skip the private-suffix decode section")
    ap.add_argument("--no-handoff", action="store_true", help="skip the page handoff section")
    ap.add_argument("--no-cascade", action="store_true", help="skip the shared-prefix cascade section")
    ap.add_argument("--no-layer-group", action="store_true", help="skip the layer-group recompute section")
    ap.add_argument("--layer-group-calls", type=int, default=8)
    ap.add_argument("--no-decode-configs", action="store_true",
                    help="skip the llama8b_n4 and qwen3_14b_long decode sections")
    ap.add_argument("--config-groups", type=int, default=40,
                    help="timed groups of back-to-back calls per decode workload section")
    ap.add_argument("--config-group-calls", type=int, default=5, help="calls per timed group")
    ap.add_argument("--only", default=None,
                    help="run one section alone and print its JSON (counter runs): a name in "
                         "CONFIG_DECODE_WORKLOADS, or 'extend'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=None,
                    help="decode layers per step (default: the workload's 36; fewer only for counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 1 GiB device-to-device copy before timing (scale for HBM byte counters)")
    return ap.parse_args()


DECODE_SOURCES = ["cross_model_shared_amd/csrc/decode.hip", "cross_model_shared_amd/csrc/attn_core.h",
                  "cross_model_shared_amd/csrc/kvs_device.h"]
PMC_SUMMARY = "profiles/decode_qwen3_8b_n8_hbm_counters.md"
CONFIG_PMC_SUMMARY = "profiles/decode_{}_hbm_counters.md"
EXTEND_SOURCES = ["cross_model_shared_amd/csrc/extend.hip", "cross_model_shared_amd/csrc/kvs_device.h"]
EXTEND_PMC_SUMMARY = "profiles/extend_8k_512_counters.md"


def kernel_source_hash(paths):
    """Hash of the kernel sources' code: line comments and blank lines do not count,
    so editing a comment does not retire the counter figures taken on the code."""
    import hashlib
    import re

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def summary_values(path, sources):
    """The "Values read by bench.py" fields of a committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, path)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return fields


def measured_traffic(summary=PMC_SUMMARY):
    """HBM bytes per decode launch from a committed counter summary (None if stale)."""
    fields = summary_values(summary, DECODE_SOURCES)
    try:
        return float(fields["hbm_bytes_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def extend_counters():
    """Counter figures of one extend_8k_512 dispatch from the committed summary (None if stale)."""
    fields = summary_values(EXTEND_PMC_SUMMARY, EXTEND_SOURCES)
    if not fields:
        return None
    try:
        return {"hbm_bytes": float(fields["hbm_bytes_per_launch"]),
                "mfma_flop_executed": float(fields["mfma_flop_per_launch"]),
                "mfma_busy_frac": float(fields["mfma_busy_frac"])}
    except (KeyError, ValueError):
        return None


def calibrate_copy():
    """A plain 1 GiB copy: its FETCH_SIZE / WRITE_SIZE readings give the counters' scale."""
    import torch

    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[bench] calibration copy: 3 x 1 GiB device-to-device")
    del src, dst


def decode_bytes(lens, B, N, Hq, Hkv, D):
    """Algorithmic bytes of one decode call: valid KV + q + out + block table + lengths."""
    kv = sum(lens) * Hkv * D * 2 * 2
    qo = 2 * B * N * Hq * D * 2
    bt = 4 * sum((L + 15) // 16 for L in lens)
    return kv + qo + bt + 4 * B


def private_decode_bytes(lens, priv, B, N, Hq, Hkv, D):
    """Algorithmic bytes of one shared_kv_decode_private call: the shared KV once, every
    private KV once, q + out, both block tables and all lengths."""
    kv = (sum(lens) + sum(priv)) * Hkv * D * 2 * 2
    qo = 2 * B * N * Hq * D * 2
    bt = 4 * (sum((L + 15) // 16 for L in lens) + sum((U + 15) // 16 for U in priv))
    return kv + qo + bt + 4 * (B + B * N)


def append_bytes(tokens, Hkv, D):
    return tokens * Hkv * D * 2 * 2 * 2     # read k/v rows, write them


def extend_flops(prefix, new, Hq, D):
    return 4 * D * Hq * sum(c * p + c * (c + 1) // 2 for p, c in zip(prefix, new))


class EventTimer:
    """Sums HIP-event durations of the bracketed calls on the current stream."""

    def __init__(self):
        self.pairs = []

    def start(self):
        import torch

        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        import torch

        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else float("nan")

    def all_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def setup_decode(wl, layers):
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens = wl.lens
    bt, num_pages = W.build_block_table(lens, wl.seed)
    pool = binding.Pool(layers, num_pages, Hkv, D)
    dev = dict(bt=torch.from_numpy(bt).cuda(), lens=torch.tensor(lens, dtype=torch.int32, device="cuda"),
               zeros=torch.zeros(B, dtype=torch.int32, device="cuda"))
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    dev["cu_all"] = torch.from_numpy(cu.astype(np.int32)).cuda()
    total = int(cu[-1])
    maxL = max(lens)
    t0 = time.perf_counter()
    for layer in range(layers):
        k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 10, layer)).view(total, Hkv, D)
        v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 11, layer)).view(total, Hkv, D)
        binding.append(pool, layer, k, v, dev["cu_all"], dev["bt"], dev["zeros"], max_new=maxL,
                       max_seq_len=maxL)
        del k, v
    torch.cuda.synchronize()
    log(f"[bench] pool filled: {layers} layers x {num_pages} pages = {pool.nbytes / 1e9:.1f} GB "
        f"in {time.perf_counter() - t0:.1f}s")
    q = [W.device_normal_bf16(B * N * Hq * D, wl.std, W.mix_seed(wl.seed, 12, l)).view(B, N, Hq, D)
         for l in range(layers)]
    tok_k = [W.device_normal_bf16(B * Hkv * D, wl.std, W.mix_seed(wl.seed, 13, l)).view(B, Hkv, D)
             for l in range(layers)]
    tok_v = [W.device_normal_bf16(B * Hkv * D, wl.std, W.mix_seed(wl.seed, 14, l)).view(B, Hkv, D)
             for l in range(layers)]
    out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(binding.decode_workspace_bytes(B, N, Hq, Hkv, D, maxL), dtype=torch.uint8, device="cuda")
    return dict(pool=pool, dev=dev, q=q, tok_k=tok_k, tok_v=tok_v, out=out, ws=ws, maxL=maxL,
                num_pages=num_pages, bt=bt)


# Layers per step whose decode call is bracketed by HIP events.  A timing event
# costs the stream about 3 us, so bracketing all 36 calls would slow the step it
# measures by about 1%; four spread layers per step, rotated from step to step,
# sample every layer over the timed steps.
TIMED_LAYERS_PER_STEP = 4


def timed_layers(step, layers):
    every = max(1, layers // TIMED_LAYERS_PER_STEP)
    return {(step + every * j) % layers for j in range(min(TIMED_LAYERS_PER_STEP, layers))}


def decode_step(wl, st, layers, timer=None, timed=()):
    from cross_model_shared_amd import binding

    d = st["dev"]
    for layer in range(layers):
        e0 = timer.start() if timer and layer in timed else None
        binding.decode_append(st["pool"], layer, st["tok_k"][layer], st["tok_v"][layer], st["q"][layer], st["out"],
                              d["bt"], d["lens"], st["maxL"], wl.scale, st["ws"])
        if e0 is not None:
            timer.stop(e0)


def setup_extend(wl):
    """REPLICAS layers of one pool, each holding every session's cached prefix, and a chunk
    (q, k, v) per replica: call i extends layer i % REPLICAS with chunk i % REPLICAS."""
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    B, Hq, Hkv, D = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    full = wl.total_lens()
    bt, num_pages = W.build_block_table(full, wl.seed)
    pool = binding.Pool(REPLICAS, num_pages, Hkv, D)
    btd = torch.from_numpy(bt).cuda()
    P = sum(wl.prefix)
    cu_p = torch.tensor(np.concatenate([[0], np.cumsum(wl.prefix)]), dtype=torch.int32, device="cuda")
    for r in range(REPLICAS):
        kp = W.device_normal_bf16(P * Hkv * D, wl.std, W.mix_seed(wl.seed, 20, r)).view(P, Hkv, D)
        vp = W.device_normal_bf16(P * Hkv * D, wl.std, W.mix_seed(wl.seed, 21, r)).view(P, Hkv, D)
        binding.append(pool, r, kp, vp, cu_p, btd, torch.zeros(B, dtype=torch.int32, device="cuda"),
                       max_new=max(wl.prefix), max_seq_len=max(full))
        del kp, vp
    T = sum(wl.new)
    q = [W.device_normal_bf16(T * Hq * D, wl.std, W.mix_seed(wl.seed, 22, r)).view(T, Hq, D) for r in range(REPLICAS)]
    kn = [W.device_normal_bf16(T * Hkv * D, wl.std, W.mix_seed(wl.seed, 23, r)).view(T, Hkv, D) for r in range(REPLICAS)]
    vn = [W.device_normal_bf16(T * Hkv * D, wl.std, W.mix_seed(wl.seed, 24, r)).view(T, Hkv, D) for r in range(REPLICAS)]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(wl.new)]), dtype=torch.int32, device="cuda")
    out = [torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(REPLICAS)]
    pre = torch.tensor(wl.prefix, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    return dict(pool=pool, bt=btd, q=q, kn=kn, vn=vn, cu=cu, out=out, pre=pre, max_new=max(wl.new),
                msl=max(full))


def extend_call(wl, st, i=0):
    from cross_model_shared_amd import binding

    r = i % REPLICAS
    binding.extend(st["pool"], r, st["q"][r], st["kn"][r], st["vn"][r], st["out"][r], st["cu"], st["bt"], st["pre"],
                   st["max_new"], st["msl"], wl.scale)


def fill_pool_layer(pool, layer, wl, lens, bt_dev, stream_key):
    """Seeded N(0, std) K/V for every session's tokens, written into one pool layer with
    kv_pool_append (device draws; the oracle checks such pools in the full-size tests)."""
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    B, Hkv, D = len(lens), wl.num_kv_heads, wl.head_dim
    total = int(sum(lens))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, stream_key, layer)).view(total, Hkv, D)
    v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, stream_key + 1, layer)).view(total, Hkv, D)
    binding.append(pool, layer, k, v, cu, bt_dev, torch.zeros(B, dtype=torch.int32, device="cuda"),
                   max_new=max(max(lens), 1), max_seq_len=max(max(lens), 1))
    del k, v


def grouped_call_ms(fn, groups, per_group, warmup=20):
    """Per-call times of `fn(i)` run back to back: `groups` groups of `per_group` calls, one
    pair of HIP events (on the current stream) around each group.  Returns the per-call
    time of every group (group time / per_group), in ms."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t = EventTimer()
    i = 0
    for _ in range(groups):
        e = t.start()
        for _ in range(per_group):
            fn(i)
            i += 1
        t.stop(e)
    torch.cuda.synchronize()
    return [ms / per_group for ms in t.all_ms()]


def decode_config_section(name, groups, per_group):
    """shared_kv_decode on one layer of a decode workload, rotating over REPLICAS pool
    replicas (layers of one pool, each with its own queries); plus time(N)/time(1) at
    fixed KV (one decoder's queries over the same pages)."""
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    wl = W.make_workload(name)
    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens = wl.lens
    bt, num_pages = W.build_block_table(lens, wl.seed)
    pool = binding.Pool(REPLICAS, num_pages, Hkv, D)
    d_bt = torch.from_numpy(bt).cuda()
    d_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for r in range(REPLICAS):
        fill_pool_layer(pool, r, wl, lens, d_bt, 10)
    q = [W.device_normal_bf16(B * N * Hq * D, wl.std, W.mix_seed(wl.seed, 12, r)).view(B, N, Hq, D)
         for r in range(REPLICAS)]
    q1 = [x[:, :1].contiguous() for x in q]
    out, out1 = torch.empty_like(q[0]), torch.empty_like(q1[0])
    maxL = max(lens)
    ws = binding.decode_workspace(B, N, Hq, Hkv, D, maxL)
    ws1 = binding.decode_workspace(B, 1, Hq, Hkv, D, maxL)
    torch.cuda.synchronize()

    def call(i):
        binding.decode(pool, i % REPLICAS, q[i % REPLICAS], out, d_bt, d_lens, maxL, wl.scale, ws)

    def call1(i):
        binding.decode(pool, i % REPLICAS, q1[i % REPLICAS], out1, d_bt, d_lens, maxL, wl.scale, ws1)

    per = grouped_call_ms(call, groups, per_group)
    per1 = grouped_call_ms(call1, groups, per_group)
    ms, ms1 = float(np.median(per)), float(np.median(per1))
    nbytes = decode_bytes(lens, B, N, Hq, Hkv, D)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] {name} decode call {ms * 1e3:.1f} us ({gbs:.0f} GB/s), N=1 {ms1 * 1e3:.1f} us")
    res = {
        "workload": f"{name}: one layer, B={B} sessions, N={N} decoders, {Hq} q / {Hkv} KV heads, D={D}, page 16, "
                    f"lengths {'log-uniform [1024, 8192]' if name == 'llama8b_n4' else 'truncated log-normal mean 27K in [4096, 131072]'} "
                    f"(sum {sum(lens)}, max {maxL}); shared_kv_decode rotating over {REPLICAS} pool replicas",
        "value": round(gbs, 1), "unit": "GB/s", "ms_per_call": round(ms, 5), "bytes_per_call": nbytes,
        "ms_per_call_p10_p50_p90": [round(float(np.percentile(per, x)), 5) for x in (10, 50, 90)],
        "calls": groups * per_group,
        "timing": f"{groups} groups of {per_group} back-to-back calls, HIP events around each group",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(CONFIG_PMC_SUMMARY.format(name))},
        "decoder_concat": {f"time_N{N}_over_N1": round(ms / ms1, 3), f"ms_N{N}": round(ms, 5),
                           "ms_N1": round(ms1, 5)},
    }
    del pool, q, q1
    torch.cuda.empty_cache()
    return res


def private_section(calls):
    """shared_kv_decode_private on the private-suffix workload, one layer."""
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    wl = W.make_workload(PRIVATE_WORKLOAD)
    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    bt, pbt, num_pages = W.build_private_tables(wl.lens, wl.priv, wl.seed)
    pool = binding.Pool(1, num_pages, Hkv, D)
    zero_b = torch.zeros(B * N, dtype=torch.int32, device="cuda")
    for i, (table, lens) in enumerate(((bt, wl.lens), (pbt, wl.priv))):
        total = sum(lens)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
        k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 30 + 2 * i)).view(total, Hkv, D)
        v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 31 + 2 * i)).view(total, Hkv, D)
        binding.append(pool, 0, k, v, cu, torch.from_numpy(table).cuda(), zero_b[:len(lens)],
                       max_new=max(lens), max_seq_len=max(lens))
        del k, v
    q = W.device_normal_bf16(B * N * Hq * D, wl.std, W.mix_seed(wl.seed, 34)).view(B, N, Hq, D)
    out = torch.empty_like(q)
    maxL, maxU = max(wl.lens), max(wl.priv)
    ws = torch.zeros(binding.decode_workspace_bytes(B, N, Hq, Hkv, D, maxL), dtype=torch.uint8, device="cuda")
    d_bt, d_pbt = torch.from_numpy(bt).cuda(), torch.from_numpy(pbt).cuda()
    d_lens = torch.tensor(wl.lens, dtype=torch.int32, device="cuda")
    d_priv = torch.tensor(wl.priv, dtype=torch.int32, device="cuda")

    def call():
        binding.decode_private(pool, 0, q, out, d_bt, d_lens, d_pbt, d_priv, maxL, maxU, wl.scale, ws)

    for _ in range(30):                              # about 25 ms of calls: the clock settles first
        call()
    torch.cuda.synchronize()
    t = EventTimer()
    for _ in range(calls):
        e = t.start()
        call()
        t.stop(e)
    torch.cuda.synchronize()
    ms = float(np.median(t.all_ms()))
    nbytes = private_decode_bytes(wl.lens, wl.priv, B, N, Hq, Hkv, D)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] private-suffix decode call {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    shared_gb = sum(wl.lens) * Hkv * D * 4 / 1e9
    priv_gb = sum(wl.priv) * Hkv * D * 4 / 1e9
    res = {
        "workload": f"{PRIVATE_WORKLOAD}: the {DECODE_WORKLOAD} sessions (shared prefixes, sum {sum(wl.lens)}) "
                    f"plus a private suffix per decoder (U[0,2048], sum {sum(wl.priv)}), one layer, "
                    f"shared_kv_decode_private",
        "value": round(gbs, 1), "unit": "GB/s", "ms_per_call": round(ms, 5), "bytes_per_call": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "footprint": {"shared_plus_private_GB": round(shared_gb + priv_gb, 3),
                      "n_full_copies_GB": round(N * shared_gb + priv_gb, 3)},
    }
    del pool
    torch.cuda.empty_cache()
    return res


def cascade_section(calls):
    """shared_kv_decode_cascade against shared_kv_decode on sessions that share prefix pages."""
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    wl = W.make_workload(CASCADE_WORKLOAD)
    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    bt, lens, gid, pref, num_pages = W.build_prefix_groups(wl.groups, wl.seed)
    pool = binding.Pool(1, num_pages, Hkv, D)
    d_bt = torch.from_numpy(bt).cuda()
    # the pages hold seeded values: each group's prefix written once, then every session's own tokens
    own = [L - pre for pre, ls in wl.groups for L in ls]
    first_rows = [b for b in range(B) if b == 0 or gid[b] != gid[b - 1]]
    pre_tok = [wl.groups[gid[b]][0] for b in first_rows]
    for i, (rows, lengths, before) in enumerate(((first_rows, pre_tok, [0] * len(first_rows)),
                                                 (list(range(B)), own, [int(p) * 16 for p in pref]))):
        total = sum(lengths)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).cuda()
        k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 50 + 2 * i)).view(total, Hkv, D)
        v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 51 + 2 * i)).view(total, Hkv, D)
        binding.append(pool, 0, k, v, cu, d_bt[rows].contiguous(),
                       torch.tensor(before, dtype=torch.int32, device="cuda"), max_new=max(max(lengths), 1),
                       max_seq_len=max(lens))
        del k, v
    q = W.device_normal_bf16(B * N * Hq * D, wl.std, W.mix_seed(wl.seed, 54)).view(B, N, Hq, D)
    out = torch.empty_like(q)
    maxL = max(lens)
    ws = torch.zeros(binding.decode_workspace_bytes(B, N, Hq, Hkv, D, maxL), dtype=torch.uint8, device="cuda")
    d_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    d_gid, d_pref = torch.from_numpy(gid).cuda(), torch.from_numpy(pref).cuda()

    def cascade():
        binding.decode_cascade(pool, 0, q, out, d_bt, d_lens, d_gid, d_pref, maxL, wl.scale, ws)

    def plain():
        binding.decode(pool, 0, q, out, d_bt, d_lens, maxL, wl.scale, ws)

    # the two entry points alternate, each call between its own events, after a warm-up long
    # enough (about 25 ms of calls) that the first timed calls run at the settled clock
    for _ in range(30):
        cascade()
        plain()
    torch.cuda.synchronize()
    tc, tp = EventTimer(), EventTimer()
    for _ in range(calls):
        for fn, t in ((cascade, tc), (plain, tp)):
            e = t.start()
            fn()
            t.stop(e)
    torch.cuda.synchronize()
    ms_c, ms_p = float(np.median(tc.all_ms())), float(np.median(tp.all_ms()))
    # unique KV bytes: every group's prefix once (units of 64 / (N G) = 2 sessions hold whole pairs here)
    uniq_tokens = sum(pre + sum(L - pre for L in ls) for pre, ls in wl.groups)
    nbytes = uniq_tokens * Hkv * D * 4 + 2 * B * N * Hq * D * 2 + 4 * (num_pages + 3 * B)
    gbs = nbytes / (ms_c * 1e-3) / 1e9
    res = {
        "workload": f"{CASCADE_WORKLOAD}: 64 sessions in 32 pairs sharing 4K-8K-token prefix pages, own 0-8K "
                    f"tokens each (sum of session lengths {sum(lens)}, unique tokens {uniq_tokens}), N=8, one layer",
        "value": round(gbs, 1), "unit": "GB/s (unique KV bytes)", "ms_per_call": round(ms_c, 5),
        "bytes_per_call": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "shared_kv_decode_ms_same_tables": round(ms_p, 5), "speedup": round(ms_p / ms_c, 3),
    }
    log(f"[bench] cascade decode {ms_c * 1e3:.1f} us ({gbs:.0f} GB/s unique), plain {ms_p * 1e3:.1f} us")
    del pool
    torch.cuda.empty_cache()
    return res


def layer_group_section(calls):
    """partial_prefill_layers over a 4-layer group (full prompts, no cached prefix) against one
    partial_prefill_extend per layer, on the same inputs."""
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    wl = W.make_workload(LAYER_GROUP_WORKLOAD)
    B, Hq, Hkv, D = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lb, nl = wl.layer_group
    full = wl.total_lens()
    bt, num_pages = W.build_block_table(full, wl.seed)
    pool = binding.Pool(wl.num_layers, num_pages, Hkv, D)
    btd = torch.from_numpy(bt).cuda()
    T = sum(wl.new)
    q = W.device_normal_bf16(nl * T * Hq * D, wl.std, W.mix_seed(wl.seed, 70)).view(nl, T, Hq, D)
    kn = W.device_normal_bf16(nl * T * Hkv * D, wl.std, W.mix_seed(wl.seed, 71)).view(nl, T, Hkv, D)
    vn = W.device_normal_bf16(nl * T * Hkv * D, wl.std, W.mix_seed(wl.seed, 72)).view(nl, T, Hkv, D)
    out = torch.empty_like(q)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(wl.new)]), dtype=torch.int32, device="cuda")
    pre = torch.tensor(wl.prefix, dtype=torch.int32, device="cuda")
    mx, msl = max(wl.new), max(full)

    def group():
        binding.extend_layers(pool, lb, q, kn, vn, out, cu, btd, pre, mx, msl, wl.scale)

    def per_layer():
        for i in range(nl):
            binding.extend(pool, lb + i, q[i], kn[i], vn[i], out[i], cu, btd, pre, mx, msl, wl.scale)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t = EventTimer()
        for _ in range(calls):
            e = t.start()
            fn()
            t.stop(e)
        torch.cuda.synchronize()
        return float(np.median(t.all_ms()))

    ms_g = timed(group)
    ms_l = timed(per_layer)
    flops = nl * extend_flops(wl.prefix, wl.new, Hq, D)
    tf = flops / (ms_g * 1e-3) / 1e12
    res = {
        "workload": f"{LAYER_GROUP_WORKLOAD}: layers [{lb}, {lb + nl}) of a {wl.num_layers}-layer pool recomputed "
                    f"for {B} prompts of {wl.new[0]} tokens (no cached prefix), 32 q / 8 KV heads, D={D}",
        "value": round(tf, 1), "unit": "TFLOP/s", "ms_per_call": round(ms_g, 4), "flops_per_call": flops,
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)},
        "per_layer_calls_ms": round(ms_l, 4), "speedup_over_per_layer_calls": round(ms_l / ms_g, 3),
    }
    log(f"[bench] layer group {ms_g:.3f} ms ({tf:.1f} TFLOP/s), {nl} per-layer calls {ms_l:.3f} ms")
    del pool, q, kn, vn, out
    torch.cuda.empty_cache()
    return res


def handoff_section(reps):
    """kv_pages_pack / kv_pages_unpack of every page of the handoff workload (all 36 layers) and
    kv_pool_fetch of its rows (all layers); HBM bytes = what is read + what is written."""
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    wl = W.make_workload(HANDOFF_WORKLOAD)
    B, Hkv, D, layers = wl.batch, wl.num_kv_heads, wl.head_dim, wl.num_layers
    bt, num_pages = W.build_block_table(wl.lens, wl.seed)
    src = binding.Pool(layers, num_pages, Hkv, D)
    total = sum(wl.lens)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(wl.lens)]).astype(np.int32)).cuda()
    d_bt = torch.from_numpy(bt).cuda()
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    for layer in range(layers):
        k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 40, layer)).view(total, Hkv, D)
        v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 41, layer)).view(total, Hkv, D)
        binding.append(src, layer, k, v, cu, d_bt, zeros, max_new=max(wl.lens), max_seq_len=max(wl.lens))
        del k, v
    ids = torch.from_numpy(np.concatenate([bt[b, :(L + 15) // 16] for b, L in enumerate(wl.lens)])).cuda()
    n = ids.numel()
    buf = torch.empty(binding.pages_buffer_bytes(src, layers, n), dtype=torch.uint8, device="cuda")
    dst = binding.Pool(layers, n, Hkv, D)
    dst_ids = torch.randperm(n, generator=torch.Generator().manual_seed(wl.seed)).to(torch.int32).cuda()
    k_out = torch.empty((total, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v_out = torch.empty_like(k_out)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t = EventTimer()
        for _ in range(reps):
            e = t.start()
            fn()
            t.stop(e)
        torch.cuda.synchronize()
        return float(np.median(t.all_ms()))

    ms_pack = timed(lambda: binding.pack(src, 0, layers, ids, buf))
    ms_unpack = timed(lambda: binding.unpack(dst, 0, layers, dst_ids, buf))
    d_lens = torch.tensor(wl.lens, dtype=torch.int32, device="cuda")
    ms_fetch = timed(lambda: [binding.fetch(src, l, d_bt, d_lens, cu, max(wl.lens), k_out, v_out)
                              for l in range(layers)])
    moved = buf.numel()                              # bytes of tiles moved by pack or unpack
    fetched = 2 * total * Hkv * D * 2 * layers       # K and V rows of every layer
    res = {
        "workload": f"{HANDOFF_WORKLOAD}: {B} sessions x {wl.lens[0]} tokens, 8 KV heads, D=128, {layers} layers "
                    f"({n} pages, {moved / 1e9:.2f} GB of tiles)",
        "pack": {"ms": round(ms_pack, 4), "GBps": round(2 * moved / (ms_pack * 1e-3) / 1e9, 1),
                 "frac": round(2 * moved / (ms_pack * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "unpack": {"ms": round(ms_unpack, 4), "GBps": round(2 * moved / (ms_unpack * 1e-3) / 1e9, 1),
                   "frac": round(2 * moved / (ms_unpack * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "fetch_all_layers": {"ms": round(ms_fetch, 4), "GBps": round(2 * fetched / (ms_fetch * 1e-3) / 1e9, 1),
                             "frac": round(2 * fetched / (ms_fetch * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "unit": "GB/s (read + written)",
    }
    log(f"[bench] handoff pack {res['pack']['GBps']} GB/s, unpack {res['unpack']['GBps']} GB/s, "
        f"fetch {res['fetch_all_layers']['GBps']} GB/s")
    del src, dst, buf
    torch.cuda.empty_cache()
    return res


def cpu_host():
    """Host cores this process may use, the BLAS threads NumPy runs, and the CPU model."""
    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cores": len(os.sched_getaffinity(0)), "blas_threads": blas_threads, "cpu_model": cpu_model}


def cpu_decode_baseline(wl, q, kv_key=(10, 11), layer=0):
    """The CPU oracle's decode (gather through the pages + float64 softmax), untuned, on every
    session of one layer of a decode workload: the layer's seeded K/V (the bench's own device
    draws, copied to the host) appended into a per-session page image by the oracle (untimed),
    then oracle.decode timed per session.  q: the layer's queries, host uint16 bits."""
    import torch

    import oracle
    from cross_model_shared_amd import workload as W

    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens = wl.lens
    cu = np.concatenate([[0], np.cumsum(lens)])
    total = int(cu[-1])
    k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, kv_key[0], layer)).view(total, Hkv, D)
    v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, kv_key[1], layer)).view(total, Hkv, D)
    spent, done_bytes = 0.0, 0
    for b in range(B):
        L = lens[b]
        kb = k[cu[b]:cu[b + 1]].view(torch.int16).cpu().numpy().view(np.uint16)
        vb = v[cu[b]:cu[b + 1]].view(torch.int16).cpu().numpy().view(np.uint16)
        npg = (L + 15) // 16
        shape = oracle.PoolShape(1, npg, Hkv, D)
        bt = np.arange(npg, dtype=np.int32)[None]
        img = oracle.append(np.zeros(shape.elems, np.uint16), shape, 0, kb, vb, [0, L], bt, [0])
        t0 = time.perf_counter()
        oracle.decode(img, shape, 0, q[b:b + 1], bt, [L], wl.scale)
        spent += time.perf_counter() - t0
        done_bytes += decode_bytes([L], 1, N, Hq, Hkv, D)
    del k, v
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "kind": "oracle", "seconds": round(spent, 2),
            "sample": f"{wl.name}: float64 oracle decode (gather + softmax) of all {B} sessions of one layer "
                      f"({total} tokens), all {N} decoders x {Hq} heads; {spent:.1f}s CPU time", **cpu_host()}


def cpu_extend_baseline(ew, sessions=1):
    """The CPU oracle's partial prefill (append + float64 causal attention), untuned, on the
    first `sessions` sessions of the extend workload (the bench's seeded device draws for
    replica 0, copied to the host); TFLOP/s of the algorithmic flops of those sessions."""
    import torch

    import oracle
    from cross_model_shared_amd import workload as W

    Hq, Hkv, D = ew.num_q_heads, ew.num_kv_heads, ew.head_dim
    P, T = sum(ew.prefix), sum(ew.new)
    host = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    kp = host(W.device_normal_bf16(P * Hkv * D, ew.std, W.mix_seed(ew.seed, 20, 0)).view(P, Hkv, D))
    vp = host(W.device_normal_bf16(P * Hkv * D, ew.std, W.mix_seed(ew.seed, 21, 0)).view(P, Hkv, D))
    q = host(W.device_normal_bf16(T * Hq * D, ew.std, W.mix_seed(ew.seed, 22, 0)).view(T, Hq, D))
    kn = host(W.device_normal_bf16(T * Hkv * D, ew.std, W.mix_seed(ew.seed, 23, 0)).view(T, Hkv, D))
    vn = host(W.device_normal_bf16(T * Hkv * D, ew.std, W.mix_seed(ew.seed, 24, 0)).view(T, Hkv, D))
    cup = np.concatenate([[0], np.cumsum(ew.prefix)])
    cun = np.concatenate([[0], np.cumsum(ew.new)])
    spent, flops = 0.0, 0
    for b in range(sessions):
        Pb, Cb = ew.prefix[b], ew.new[b]
        npg = (Pb + Cb + 15) // 16
        shape = oracle.PoolShape(1, npg, Hkv, D)
        bt = np.arange(npg, dtype=np.int32)[None]
        img = oracle.append(np.zeros(shape.elems, np.uint16), shape, 0, kp[cup[b]:cup[b + 1]], vp[cup[b]:cup[b + 1]],
                            [0, Pb], bt, [0])
        t0 = time.perf_counter()
        oracle.extend(img, shape, 0, q[cun[b]:cun[b + 1]], kn[cun[b]:cun[b + 1]], vn[cun[b]:cun[b + 1]], [0, Cb], bt,
                      [Pb], ew.scale)
        spent += time.perf_counter() - t0
        flops += extend_flops([Pb], [Cb], Hq, D)
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle", "seconds": round(spent, 2),
            "sample": f"{ew.name}: float64 oracle partial prefill (append + causal attention) of {sessions} of "
                      f"{ew.batch} sessions ({ew.prefix[0]} cached + {ew.new[0]} new tokens, {Hq} heads); the "
                      f"whole batch would take about {ew.batch // sessions}x as long (extrapolated, not run); "
                      f"{spent:.1f}s CPU time", **cpu_host()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path runs on a "
              f"single MI355X; sharding it over several GPUs is designed, not built)", file=sys.stderr)
        sys.exit(2)
    import torch

    from cross_model_shared_amd import binding
    from cross_model_shared_amd import workload as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    if args.calibrate_copy:
        calibrate_copy()
    if args.only:  # one section alone (counter runs): its dispatches are the run's only ones of its kernel
        if args.only in CONFIG_DECODE_WORKLOADS:
            res = decode_config_section(args.only, args.config_groups, args.config_group_calls)
        elif args.only == "extend":
            ew = W.make_workload(EXTEND_WORKLOAD)
            es = setup_extend(ew)
            for i in range(args.extend_calls):
                extend_call(ew, es, i)
            torch.cuda.synchronize()
            res = {"workload": EXTEND_WORKLOAD, "calls": args.extend_calls}
        else:
            print(f"--only {args.only}: unknown section", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"only": args.only, **res}), flush=True)
        return
    wl = W.make_workload(DECODE_WORKLOAD)
    layers = args.layers or wl.num_layers
    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    st = setup_decode(wl, layers)
    # one shared_kv_decode_append call: the decode's bytes plus the step's token rows read and written
    per_call = decode_bytes(wl.lens, B, N, Hq, Hkv, D) + append_bytes(B, Hkv, D)
    step_bytes = layers * per_call

    for _ in range(args.warmup):
        decode_step(wl, st, layers)
    torch.cuda.synchronize()
    timer = EventTimer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        decode_step(wl, st, layers, timer, timed_layers(k, layers))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9
    call_ms = timer.mean_ms()
    achieved = per_call / (call_ms * 1e-3) / 1e9
    log(f"[bench] decode step {ms_step:.3f} ms ({layers} layers), decode call {call_ms * 1e3:.1f} us, "
        f"{achieved:.0f} GB/s")

    # time(N) / time(1) at fixed KV: one decoder's queries only (ICaRus Key design 3 claim)
    q1 = st["q"][0][:, :1].contiguous()
    out1 = torch.empty_like(q1)
    ws1 = torch.zeros(binding.decode_workspace_bytes(B, 1, Hq, Hkv, D, st["maxL"]), dtype=torch.uint8,
                      device="cuda")
    t1, tN = EventTimer(), EventTimer()
    for i in range(12):
        e = t1.start()
        binding.decode(st["pool"], i % layers, q1, out1, st["dev"]["bt"], st["dev"]["lens"], st["maxL"],
                       wl.scale, ws1)
        t1.stop(e)
        e = tN.start()
        binding.decode(st["pool"], (i + 5) % layers, st["q"][0], st["out"], st["dev"]["bt"], st["dev"]["lens"],
                       st["maxL"], wl.scale, st["ws"])
        tN.stop(e)
    torch.cuda.synchronize()
    n1_ms = float(np.median(t1.all_ms()[2:]))
    nN_ms = float(np.median(tN.all_ms()[2:]))

    # layer 0's queries for the CPU baseline, which runs after the GPU sections
    # (twelve seconds of an idle GPU would let its clocks drop before the extend timing)
    q0_host = st["q"][0].view(torch.int16).cpu().numpy().view(np.uint16)
    pool_gb = st["pool"].nbytes / 1e9
    del st
    torch.cuda.empty_cache()

    # ---- extend ----
    ew = W.make_workload(EXTEND_WORKLOAD)
    es = setup_extend(ew)
    for i in range(args.extend_warmup):  # ~1 ms each: brings the clocks to their steady state
        extend_call(ew, es, i)
    torch.cuda.synchronize()
    et = EventTimer()
    for i in range(args.extend_calls):
        e = et.start()
        extend_call(ew, es, i)
        et.stop(e)
    torch.cuda.synchronize()
    ext_ms = float(np.median(et.all_ms()))
    ext_p = [round(float(np.percentile(et.all_ms(), x)), 5) for x in (10, 50, 90)]
    del es
    torch.cuda.empty_cache()
    flops = extend_flops(ew.prefix, ew.new, ew.num_q_heads, ew.head_dim)
    ext_tflops = flops / (ext_ms * 1e-3) / 1e12
    log(f"[bench] extend call {ext_ms:.3f} ms, {ext_tflops:.1f} TFLOP/s")

    configs = {} if args.no_decode_configs else {
        name: decode_config_section(name, args.config_groups, args.config_group_calls)
        for name in CONFIG_DECODE_WORKLOADS}
    private = None if args.no_private else private_section(args.private_calls)
    handoff = None if args.no_handoff else handoff_section(10)
    cascade = None if args.no_cascade else cascade_section(20)
    layer_group = None if args.no_layer_group else layer_group_section(args.layer_group_calls)

    cpu, cpus = None, None
    if not args.no_cpu_baseline:
        cpu = cpu_decode_baseline(wl, q0_host)
        cpu["sample"] += f"; the {layers}-layer step would take {layers}x as long (extrapolated, not run)"
        log(f"[bench] cpu baseline {wl.name} {cpu['value']} GB/s ({cpu['seconds']}s)")
        cpus = {}
        if not args.no_decode_configs:
            for name in CONFIG_DECODE_WORKLOADS:
                cw_ = W.make_workload(name)
                qc = W.device_normal_bf16(cw_.batch * cw_.num_decoders * cw_.num_q_heads * cw_.head_dim, cw_.std,
                                          W.mix_seed(cw_.seed, 12, 0))
                qc = qc.view(torch.int16).cpu().numpy().view(np.uint16).reshape(
                    cw_.batch, cw_.num_decoders, cw_.num_q_heads, cw_.head_dim)
                cpus[name] = cpu_decode_baseline(cw_, qc)
                log(f"[bench] cpu baseline {name} {cpus[name]['value']} GB/s ({cpus[name]['seconds']}s)")
        cpus[EXTEND_WORKLOAD] = cpu_extend_baseline(ew, 1)
        log(f"[bench] cpu baseline {EXTEND_WORKLOAD} {cpus[EXTEND_WORKLOAD]['value']} TFLOP/s "
            f"({cpus[EXTEND_WORKLOAD]['seconds']}s)")

    res = {
        "metric": "shared-KV decode attn KV GB/s (% HBM peak) at N=8 decoders; extend TFLOP/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{DECODE_WORKLOAD}: Qwen3-8B-shaped 8-decoder agentic decode step, {layers} layers "
                        f"(shared_kv_decode_append per layer: the step's token written and attended), B={B} sessions, N={N}, "
                        f"32 q / 8 KV heads, D=128, page 16, lengths U[4096,16384] (sum {sum(wl.lens)})",
            "batch": B, "num_decoders": N, "layers": layers, "context_tokens": sum(wl.lens),
            "step_algorithmic_bytes": step_bytes, "decode_bytes_per_layer": per_call,
        },
        "roofline": {
            "bound": "hbm", "kernel": "shared_kv_decode_append (per-layer call)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
            "launch_ms": round(call_ms, 5),
            "launch_ms_p10_p50_p90": [round(float(np.percentile(timer.all_ms(), x)), 5) for x in (10, 50, 90)],
            "launches": len(timer.all_ms()),
        },
        "cpu_baseline": cpu,
        "cpu_baselines_other": cpus,
        "decoder_concat": {"time_N8_over_N1": round(nN_ms / n1_ms, 3), "ms_N8": round(nN_ms, 4),
                           "ms_N1": round(n1_ms, 4)},
        "footprint": {"pool_GB": round(pool_gb, 2), "n_private_copies_GB": round(pool_gb * N, 2),
                      "ratio": N},
        "decode_configs": configs,
        "private": private,
        "handoff": handoff,
        "cascade": cascade,
        "layer_group": layer_group,
        "extend": {
            "workload": f"{EXTEND_WORKLOAD}: B=16, cached prefix 8192 + 512 new tokens, 32 q / 8 KV heads, "
                        f"D=128 (partial_prefill_extend = append chunk + causal attention)",
            "value": round(ext_tflops, 2), "unit": "TFLOP/s", "ms_per_call": round(ext_ms, 4),
            "ms_per_call_p10_p50_p90": ext_p, "calls": args.extend_calls,
            "timing": f"HIP events around each call; calls rotate over {REPLICAS} pool replicas and chunks",
            "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(ext_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ext_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         # rocprofv3 counters of one dispatch (HBM bytes, matrix-core flop executed
                         # and pipe-busy fraction), from the committed summary; null if stale
                         "counters": extend_counters()},
        },
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
