#!/usr/bin/env python3
"""Decode-step benchmark of the DSA hot path on one MI355X.

Workload: long-context decode, batch 8, 131072 cached tokens per sequence,
64 indexer heads (d=128), Top-K 2048, 128 SFA heads over a 576/512 MLA
latent cache (FP8 latent with per-128 tile scales + bf16 rope), 64-token
pages under a shuffled block table; seeded synthetic N(0,1) data.

One step = the whole hot path for one decode token of each sequence:
  dsa_decode_prolog (in one launch: mxfp8_quant of the indexer q, the new
  indexer k into the K cache, kv_fp8_quant_paged_write of the new KV row)
  -> dsa_indexer_topk -> dsa_sparse_attn
(--separate-prolog runs the three quantisations as three launches instead;
--graph captures the step once per cache replica in a HIP graph and times
graph replays instead of eager launches).
Caches are replicated (default 4 replicas, about 3.3 GB) and rotated per step
so that the 256 MB Infinity Cache cannot serve one step's reads from the
previous step.

Timing: W untimed steps, then exactly K steps between two device
synchronisations (no event inside the loop: an event recorded between two
launches drains the queue and adds several microseconds).  Per-entry-point
durations come from two further timed regions on the launch stream: K
back-to-back dsa_indexer_topk calls, then K back-to-back dsa_sparse_attn
calls, each bracketed by HIP events; the indexer's average is the roofline
duration.  `traffic` is filled from the committed FETCH_SIZE/WRITE_SIZE
summary when it was taken on the current indexer source.

Prints one JSON line.  `value` is query tokens/s (rows * steps / seconds;
for decode one row per sequence).  --config prefill_chunk_8k_of_128k times
the chunked-prefill step instead (8192 query rows of one sequence through
dsa_indexer_topk_seq), whose roofline is the MFMA one of its longer entry
point; `mfma_rooflines` gives both entry points' scaled-MFMA rates.
--config decode_mtp4_128k_b8 times multi-query decode (4 query tokens per
sequence, as in the verification of drafted tokens) through
dsa_indexer_topk_mq, which reads each sequence's K once for its 4 rows; its
roofline counts those bytes once per sequence.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LI+SFA decode tokens/s and achieved HBM GB/s at 128K ctx, batch 8, 1 GPU"
METRIC_MQ = ("LI+SFA multi-query decode query tokens/s and achieved HBM GB/s at 128K ctx, "
             "batch 8 x 4 query tokens, 1 GPU")
METRIC_PREFILL = "LI+SFA chunked-prefill query tokens/s and MFMA utilisation, 8K rows of a 128K context, 1 GPU"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFS = 5000.0          # dense fp8 MFMA
BF16_PEAK_TFS = 2500.0         # dense bf16 / fp16 MFMA
IDX_BYTES_PER_TOKEN = 132      # 128 E4M3 + 4 E8M0 per history token (one query row)
SFA_BYTES_PER_ENTRY = 656      # one latent record per selected position


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--config", default="decode_128k_b8")
    ap.add_argument("--cpu-rows", type=int, default=8, help="oracle rows timed for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-prolog", action="store_true",
                    help="quantise q, k and kv with three launches instead of dsa_decode_prolog")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step once per cache replica in a HIP graph and time graph replays")
    ap.add_argument("--profile-steps", action="store_true",
                    help="only warm up and run the timed steps (for profiler runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES between two device buffers (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DSA decode path here has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.graph and args.separate_prolog:
        print("--graph captures the fused prolog; drop --separate-prolog", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    from sparse_attention_decode_topk_amd import ops, synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = synth.config(args.config)
    t_gen = time.perf_counter()
    inp = synth.make(cfg)
    t_gen = time.perf_counter() - t_gen
    B = cfg.batch
    R = len(inp["row_seq"])
    H_I, H, K = cfg.h_index, cfg.h_attn, cfg.topk
    npages = int(inp["total_pages"])
    lens = inp["seq_lens"].astype(np.int64)
    starts = inp["seq_starts"]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- resident inputs ---------------------------------------------------
    block_table = torch.from_numpy(inp["block_table"]).to(dev)
    row_seq = torch.from_numpy(inp["row_seq"]).to(dev)
    row_pos = torch.from_numpy(inp["row_pos"]).to(dev)
    q_idx = bf16(inp["q_idx"])
    w = torch.from_numpy(inp["w"]).to(dev)
    q_sfa = bf16(inp["q_sfa"])
    # the token of every query row (decode: the last token of its sequence;
    # chunked prefill: the chunk's tokens), written into the caches by the prolog
    new_tok = starts[inp["row_seq"]].astype(np.int64) + inp["row_pos"].astype(np.int64)
    k_new = bf16(inp["k_idx"][new_tok])
    kv_new = bf16(inp["kv"][new_tok])
    slots_new = torch.from_numpy(inp["slot_mapping"][new_tok]).to(dev)
    # rows of one sequence (a prefill chunk) take the row-tiled indexer entry
    one_seq = len(np.unique(inp["row_seq"])) == 1 and R > B
    # several query rows per sequence (multi-query decode) take the entry
    # point that reads each sequence's K once for its group of rows
    mq = cfg.q_per_seq if (not one_seq and cfg.q_per_seq > 1) else 0
    k0 = torch.zeros((npages, ops.K_PAGE_BYTES), dtype=torch.uint8, device=dev)
    kv0 = torch.zeros((npages, ops.KV_PAGE_BYTES), dtype=torch.uint8, device=dev)
    slots_all = torch.from_numpy(inp["slot_mapping"]).to(dev)
    ops.mxfp8_quant_paged(bf16(inp["k_idx"]), slots_all, k0)
    ops.kv_fp8_quant_paged_write(bf16(inp["kv"]), slots_all, kv0)
    torch.cuda.synchronize()
    k_pools = [k0] + [k0.clone() for _ in range(args.replicas - 1)]
    kv_pools = [kv0] + [kv0.clone() for _ in range(args.replicas - 1)]
    q_fp8 = torch.empty((R, H_I, 128), dtype=torch.uint8, device=dev)
    q_e8 = torch.empty((R, H_I, 4), dtype=torch.uint8, device=dev)
    out_idx = torch.empty((R, K), dtype=torch.int32, device=dev)
    out_sc = torch.empty((R, K), dtype=torch.float32, device=dev)
    out = torch.empty((R, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    if one_seq:
        bt_row = block_table[int(inp["row_seq"][0])].contiguous()
        ws_i = ops.indexer_seq_workspace(R, bt_row.numel(), H_I, K, dev)
    else:
        ws_i = ops.indexer_workspace(R, block_table.shape[1], H_I, K, dev)
    ws_s = ops.sparse_attn_workspace(R, H, K, dev)
    torch.cuda.synchronize()

    # ---- raw C calls with prebuilt arguments (no per-call marshalling) -----
    L = ops.lib()
    P = ctypes.c_void_p
    ptr = lambda t: P(t.data_ptr())
    stream = P(torch.cuda.current_stream().cuda_stream)
    steps_args = []
    for j in range(args.replicas):
        steps_args.append(dict(
            qq=(ptr(q_idx), R * H_I, 128, ptr(q_fp8), ptr(q_e8), None, None, 0, stream),
            kq=(ptr(k_new), R, 128, None, None, ptr(k_pools[j]), ptr(slots_new), npages, stream),
            kvq=(ptr(kv_new), R, ptr(slots_new), ptr(kv_pools[j]), npages, stream),
            pro=(ptr(q_idx), R * H_I, 128, ptr(q_fp8), ptr(q_e8), ptr(k_new), ptr(kv_new), R,
                 ptr(slots_new), ptr(k_pools[j]), ptr(kv_pools[j]), npages, stream),
            idx=((ptr(q_fp8), ptr(q_e8), ptr(w), ptr(k_pools[j]), npages, ptr(bt_row),
                  bt_row.numel(), ptr(row_pos), R, H_I, K, ptr(out_idx), ptr(out_sc), ptr(ws_i),
                  ws_i.numel(), stream) if one_seq else
                 (ptr(q_fp8), ptr(q_e8), ptr(w), ptr(k_pools[j]), npages, ptr(block_table),
                  block_table.shape[1], ptr(row_seq), ptr(row_pos), R, mq, H_I, K, ptr(out_idx),
                  ptr(out_sc), ptr(ws_i), ws_i.numel(), stream) if mq else
                 (ptr(q_fp8), ptr(q_e8), ptr(w), ptr(k_pools[j]), npages, ptr(block_table),
                  block_table.shape[1], ptr(row_seq), ptr(row_pos), R, H_I, K, ptr(out_idx),
                  ptr(out_sc), ptr(ws_i), ws_i.numel(), stream)),
            sfa=(ptr(q_sfa), ptr(kv_pools[j]), npages, ptr(block_table), block_table.shape[1],
                 ptr(row_seq), ptr(out_idx), R, H, K, ctypes.c_float(ops.DEFAULT_SCALE),
                 ptr(out), ptr(lse), ptr(ws_s), ws_s.numel(), stream)))

    indexer_call = (L.dsa_indexer_topk_seq if one_seq else
                    L.dsa_indexer_topk_mq if mq else L.dsa_indexer_topk)

    def step(i):
        a = steps_args[i % args.replicas]
        if args.separate_prolog:
            st = L.mxfp8_quant(*a["qq"]) | L.mxfp8_quant(*a["kq"]) | L.kv_fp8_quant_paged_write(*a["kvq"])
        else:
            st = L.dsa_decode_prolog(*a["pro"])
        st |= indexer_call(*a["idx"])
        st |= L.dsa_sparse_attn(*a["sfa"])
        if st:
            raise RuntimeError(f"library call failed (status bits {st})")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    run_step = step
    if args.graph:
        # one graph per replica, its launches recorded on a capture stream
        cap = torch.cuda.Stream()
        cap_h = P(cap.cuda_stream)
        graphs = []
        for j in range(args.replicas):
            aj = {k: tuple(cap_h if x is stream else x for x in v) for k, v in steps_args[j].items()}
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                st = L.dsa_decode_prolog(*aj["pro"]) | indexer_call(*aj["idx"]) | L.dsa_sparse_attn(*aj["sfa"])
            if st:
                raise RuntimeError(f"library call failed during capture (status bits {st})")
            graphs.append(g)
        torch.cuda.synchronize()
        run_step = lambda i: graphs[i % args.replicas].replay()
        for i in range(args.warmup):
            run_step(i)
        torch.cuda.synchronize()
    K_steps = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K_steps):
        run_step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if args.profile_steps:
        print(json.dumps({"profile_steps": K_steps, "seconds": elapsed}))
        return

    # per-entry-point durations: K back-to-back calls between two events
    def timed_calls(fn, key):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(K_steps):
            if fn(*steps_args[i % args.replicas][key]):
                raise RuntimeError(f"{key} call failed")
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / K_steps

    idx_avg = timed_calls(indexer_call, "idx")
    sfa_avg = timed_calls(L.dsa_sparse_attn, "sfa")
    ms_per_step = elapsed * 1e3 / K_steps
    tokens_per_s = R * K_steps / elapsed   # query tokens (decode: one per sequence)

    hist_tokens = int((inp["row_pos"].astype(np.int64) + 1).sum())
    if mq:
        # K is read once per group of a sequence's rows: its longest history
        groups = (inp["row_pos"].astype(np.int64) + 1).reshape(-1, mq).max(axis=1)
        idx_bytes = int(groups.sum()) * IDX_BYTES_PER_TOKEN
    else:
        idx_bytes = hist_tokens * IDX_BYTES_PER_TOKEN
    sel = out_idx.cpu().numpy()
    n_sel = int((sel >= 0).sum())
    sfa_bytes = n_sel * SFA_BYTES_PER_ENTRY
    step_bytes = idx_bytes + sfa_bytes
    achieved = idx_bytes / (idx_avg * 1e-3) / 1e9
    # scaled-MFMA work: the indexer's q.k contraction and the attention's
    # logits and P.V products
    idx_flop = hist_tokens * H_I * 128 * 2
    sfa_flop = n_sel * H * (576 + 512) * 2
    idx_tf = idx_flop / (idx_avg * 1e-3) / 1e12
    sfa_tf = sfa_flop / (sfa_avg * 1e-3) / 1e12
    err_word = int(ws_i[8:12].view(torch.int32).item())
    traffic = measured_traffic(cfg.name)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_rows)

    idx_name = ("dsa_indexer_topk_seq" if one_seq else
                "dsa_indexer_topk_mq" if mq else "dsa_indexer_topk")
    mfma = {idx_name: {"achieved": round(idx_tf, 1), "peak": FP8_PEAK_TFS, "unit": "TFLOP/s",
                       "frac": round(idx_tf / FP8_PEAK_TFS, 4), "flop": idx_flop,
                       "dtype": "fp8 e4m3 x e4m3, E8M0 block scales"},
            "dsa_sparse_attn": {"achieved": round(sfa_tf, 1), "peak": BF16_PEAK_TFS, "unit": "TFLOP/s",
                                "frac": round(sfa_tf / BF16_PEAK_TFS, 4), "flop": sfa_flop,
                                "dtype": "bf16 logits, f16 P.V"}}
    if one_seq:
        # a prefill chunk is MFMA-bound: the longer of the two entry points
        kname = idx_name if idx_avg >= sfa_avg else "dsa_sparse_attn"
        m = mfma[kname]
        roofline = {"bound": "mfma", "kernel": kname, "achieved": m["achieved"], "peak": m["peak"],
                    "unit": "TFLOP/s", "frac": m["frac"], "traffic": None, "flop": m["flop"]}
    else:
        roofline = {"bound": "hbm", "kernel": idx_name, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "algorithmic_bytes": idx_bytes}
    rec = {
        "metric": METRIC_PREFILL if one_seq else METRIC_MQ if mq else METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 inputs; indexer fp8 MFMA with E8M0 block scales, SFA bf16/f16 MFMA; fp32 accumulate",
        "data": "synthetic (seeded N(0,1), bf16-rounded, MXFP8/FP8-quantised on device)",
        "config": {"workload": cfg.name, "batch": B, "context": int(lens.max()), "query_rows": R,
                   "h_index": H_I, "h_attn": H, "topk": K, "page_tokens": 64,
                   "cache_replicas_rotated": args.replicas, "parallelism": "single GPU",
                   "prolog": "three launches" if args.separate_prolog else "dsa_decode_prolog (one launch)",
                   "launch": "hipGraph replay per step" if args.graph else "eager launches"},
        "hbm_gbs_step": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "algorithmic_bytes_step": step_bytes,
        "kernel_ms": {idx_name: round(idx_avg, 5),
                      "dsa_sparse_attn": round(sfa_avg, 5)},
        "roofline": roofline,
        "mfma_rooflines": mfma,
        "cpu_baseline": cpu,
        "indexer_error_word": err_word,
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(rec))


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "dsa_indexer_topk_decode_128k_b8_traffic.txt")
INDEXER_SOURCE = os.path.join(ROOT, "sparse_attention_decode_topk_amd", "csrc", "indexer.hip")


def measured_traffic(workload):
    """HBM bytes per dsa_indexer_topk call from the committed counter summary
    (calibrated FETCH_SIZE + WRITE_SIZE), or None when the summary is missing,
    for another workload, or was taken on a different indexer source."""
    import hashlib
    try:
        fields = {}
        with open(TRAFFIC_SUMMARY) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        with open(INDEXER_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if fields.get("indexer_source_sha256") != sha or fields.get("workload") != workload:
            return None
        return int(fields["traffic_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        return None


def copy_probe(nbytes):
    """One elementwise kernel that reads nbytes and writes nbytes (b = 2a):
    the reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    torch.cuda.set_device(0)
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.mul(a, 2.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}))


def cpu_baseline(inp, rows):
    """The fp64 oracle (as it stands) on the first `rows` decode rows of the
    same inputs: indexer scores, Top-K and sparse attention per row."""
    import numpy as np

    from oracle.pipeline import Oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    o = Oracle(inp)
    t0 = time.perf_counter()
    for r in range(rows):
        res = o.topk(r)
        o.sfa(r, res["idx"])
    dt = time.perf_counter() - t0
    return {"value": round(rows / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {len(inp['row_seq'])} query rows (indexer+Top-K+SFA per row, "
                      f"fp64 numpy), {dt:.1f} s"}


if __name__ == "__main__":
    main()
