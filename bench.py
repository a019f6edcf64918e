#!/usr/bin/env python3
"""Benchmark of exact full-request tokenization on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the whole GPU path (UTF-8 decode and classification, automaton scan and piece
starts, length-binned BPE, ID compaction, per-document offsets) over one batch: the batch of 64 agent
transcripts with log-uniform lengths between 1e4 and 1e6 characters (18,448,209 bytes, cl100k-style
rules, 131,072 merges).  Inputs are resident in device memory before the timed region starts.

Prints ONE JSON line:
  value        scanned GB/s of the batch = input bytes x K / wall time of K back-to-back steps
  latency_ms   p50 / p90 wall-clock latency of single requests, device-resident input, including the
               final device-to-host read of the token count (configs 1, 2, 3, 5); the 1M-character
               multilingual request is the "p50 ms per 1M-char request"; graph_p50 / graph_p90: the
               same request replayed through a captured HIP graph of the kernel chain (toktier_plan)
  value_two_in_flight  the same steps alternating between two streams (two batches in flight, each
               with its own workspace and outputs)
  path_alg_frac_of_hbm  the headline roofline figure: the path's algorithmic bytes (input, 4 B per
               token ID, document offsets in and out) per step / the step time / 8 TB/s
  roofline     the dominant kernel (longest average duration, HIP events recorded around each launch
               on its stream inside the timed steps): its bound as the instruction counters of
               profiles/ show it ("alu": VALU issue, against 614.4 G wavefront instructions/s), the
               committed per-launch counts over the live duration; its own algorithmic bytes and
               their fraction of 8 TB/s beside; kernels: every kernel's duration and own bytes
  repair_ms    incremental repair (toktier_repair_append, records repaired in place): wall-clock ms per
               append, host text in and host records out, on one agent session of 100K / 1M / 4.4M
               characters with 1,400-character appends, and on the 1M session with 1K / 10K / 100K
               appends; the first append apart, p50 / p90 over the next 24; each session's records
               are checked against a fresh GPU encode of its whole text
  cpu_baseline the CPU oracle (serial pre-tokenizer + priority-queue BPE, one document per worker
               process) timed on this host's available cores over a bounded sample of the same batch,
               and single-core on each single-request configuration; the same run checks the GPU
               output against the oracle bit for bit ("bit_exact")
"""
import argparse
import hashlib
import json
import multiprocessing as mp
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import textgen  # noqa: E402

METRIC = "full-tokenize scanned GB/s (batched) + p50 ms per 1M-char request, bit-exact IDs"
HBM_PEAK_GBS = 8000.0
MAIN = "c4_batch64"
LATENCY = ("c1_ec4k", "c2_at100k", "c3_mix1m", "c5_adv4m4")

# incremental repair: appends to one agent session (a single 4.4M-character transcript stream; A is
# its first N characters, each append the next slice), host bytes in, host records out
REPAIR_CONTEXTS = (100_000, 1_000_000, 4_400_000)   # characters of A
REPAIR_APPEND = 1_400                                # the median append of the interactive traces
REPAIR_SWEEP = (1_000, 10_000, 100_000)              # append sizes on the 1M-character session
REPAIR_SAMPLES = 24                                  # steady-state appends per shape, after a first one

VALU_PEAK = 256 * 4 * 2.4e9 / 4 / 1e9   # G wavefront instructions/s: 256 CUs x 4 SIMDs, 4 cycles per wave64 op


def own_bytes(n, D, P, T, M, Bm, Tm):
    """Algorithmic bytes each kernel moves itself: n input bytes, D documents, P pieces, T tokens, M
    pieces left for BPE (Bm of their bytes, Tm of their tokens)."""
    return {
        "summary": 8 * (D + 1),
        "pieces": n + 4 * P + 8 * (D + 1),                       # input in, piece starts out
        "giant_seams": 0, "bpe_giant": 0,                         # no piece over 4096 bytes here
        "tiles": n + 4 * (P + 1) + 4 * P + 4 * M,                 # input and starts in, results and lists out
        "bpe": Bm + 4 * M + 8 * M + 4 * M + 4 * Tm,               # bytes, list, starts in; results out
        "emit": 4 * P + 4 * P + 4 * Tm + 4 * T + 16 * (D + 1),   # results, starts, BPE IDs in; IDs out
    }


def token_lengths(merges):
    """Byte length of every token ID of a merge list (256 single bytes, then one per merge)."""
    m = np.asarray(merges, dtype=np.int64).reshape(-1, 2)
    ln = np.ones(256 + m.shape[0], dtype=np.int64)
    for r, (a, b) in enumerate(m.tolist()):
        ln[256 + r] = ln[a] + ln[b]
    return ln


def _log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------------
# CPU baseline leg (the oracle).  Runs before the GPU is touched, so the worker pool can fork.

_MERGES_CACHE = {}
_DOCS = []


def _oracle_doc(args):
    """Encode one document with the oracle; returns (ids or None, seconds)."""
    fam, voc, i, keep = args
    import oracle
    if voc not in _MERGES_CACHE:
        _MERGES_CACHE[voc] = oracle.Merges(textgen.load_vocab(voc)[0])
    doc = _DOCS[i] if i >= 0 else b"warm"
    t0 = time.perf_counter()
    ids, _ = oracle.encode_batch(fam, _MERGES_CACHE[voc], doc)
    return (ids if keep else None), time.perf_counter() - t0


def cpu_baseline(fam, voc, data, offs, target_s, workers):
    import oracle
    oracle.lib()
    _DOCS[:] = [data[int(offs[i]):int(offs[i + 1])].tobytes() for i in range(offs.size - 1)]
    order = sorted(range(len(_DOCS)), key=lambda i: -len(_DOCS[i]))      # longest first
    ctx = mp.get_context("fork")                                         # the GPU is not touched yet
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_doc, [(fam, voc, -1, False)] * workers)
        t0 = time.perf_counter()
        first = pool.map(_oracle_doc, [(fam, voc, i, True) for i in order], chunksize=1)
        one_pass = time.perf_counter() - t0
        cpu_s = sum(t for _, t in first)
        reps = max(0, int(np.ceil(target_s / max(cpu_s, 1e-3))) - 1)
        t1 = time.perf_counter()
        for _ in range(reps):
            pool.map(_oracle_doc, [(fam, voc, i, False) for i in order], chunksize=1)
        more = time.perf_counter() - t1
    wall = one_pass + more
    passes = reps + 1
    by_doc = [None] * len(_DOCS)
    for i, (ids, _) in zip(order, first):
        by_doc[i] = ids
    oo = np.zeros(len(by_doc) + 1, dtype=np.uint64)
    oo[1:] = np.cumsum([x.size for x in by_doc])
    gbs = data.size * passes / wall / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{passes} passes over the {len(by_doc)}-document batch ({data.size} bytes each), "
                      f"one document per task, longest first, on {workers} worker processes; "
                      f"{cpu_s * passes:.1f} s of CPU work inside the oracle",
            "cpu_seconds": round(cpu_s * passes, 2)}, (np.concatenate(by_doc), oo)


def oracle_latency(fam, voc, data, offs, reps=5):
    import oracle
    merges, _ = textgen.load_vocab(voc)
    m = oracle.Merges(merges)
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.encode_batch(fam, m, data, offs)
        ts.append((time.perf_counter() - t0) * 1e3)
    return statistics.median(ts)


def repair_latency(tt):
    """Wall-clock latency of toktier_repair_append through RepairSession (records repaired in place),
    per (context, append) shape: the first append apart, then REPAIR_SAMPLES appends; the session's
    records are then checked against a fresh GPU encode of its whole text."""
    fam, voc, _ = textgen.WORKLOADS["c2_at100k"]
    merges, ff = textgen.load_vocab(voc)
    tok = tt.Tokenizer(merges, ff, device="cuda:0")
    need = max(max(REPAIR_CONTEXTS) + (REPAIR_SAMPLES + 1) * REPAIR_APPEND,
               1_000_000 + (REPAIR_SAMPLES + 1) * max(REPAIR_SWEEP))
    raw = textgen.agent_transcript(9, need).encode()   # ASCII: characters = bytes
    res = {}
    shapes = [(n, REPAIR_APPEND) for n in REPAIR_CONTEXTS] + [(1_000_000, d) for d in REPAIR_SWEEP
                                                             if d != REPAIR_APPEND]
    for n_a, delta in shapes:
        sess = tt.RepairSession(tok, raw[:n_a])
        ts, spliced, attempts = [], 0, 0
        for k in range(REPAIR_SAMPLES + 1):
            b = raw[n_a + k * delta: n_a + (k + 1) * delta]
            t0 = time.perf_counter()
            info = sess.append(b)
            ts.append((time.perf_counter() - t0) * 1e3)
            spliced += info["spliced"]
            attempts += info["attempts"]
        end = n_a + (REPAIR_SAMPLES + 1) * delta
        ids, _, spans = tok.encode(raw[:end], spans=True)
        first, st = ts[0], sorted(ts[1:])
        res[f"ctx{n_a}_add{delta}"] = {
            "context_chars": n_a, "append_chars": delta, "first_ms": round(first, 4),
            "p50": round(statistics.median(st), 4), "p90": round(st[int(0.9 * (len(st) - 1))], 4),
            "samples": len(st), "spliced": spliced, "windows_encoded": attempts,
            "same_as_full_encode": bool(np.array_equal(sess.ids, ids) and np.array_equal(sess.spans, spans))}
        _log("repair", n_a, delta, res[f"ctx{n_a}_add{delta}"])
    return res


# ---------------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--latency-reps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-two-streams", action="store_true",
                    help="skip the two-batches-in-flight leg (so that a profiler sees no overlapping launches)")
    ap.add_argument("--no-latency", action="store_true",
                    help="skip the single-request latency leg (so that a profiler sees only batch launches)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the design for several GPUs is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)

    t_start = time.time()
    _log("generating workloads")
    work = {name: textgen.workload(name) for name in (MAIN,) + (() if args.no_latency else LATENCY)}
    fam, voc, data, offs = work[MAIN]

    cpu = None
    oracle_ref = {}
    if not args.no_cpu_baseline:
        # every core this process may run on, within the host's share for one GPU when the
        # environment states it (OMP_NUM_THREADS)
        affinity = len(os.sched_getaffinity(0))
        share = int(os.environ.get("OMP_NUM_THREADS") or affinity)
        workers = max(1, min(affinity, share))
        _log(f"cpu baseline: oracle on {workers} workers")
        cpu, oracle_ref[MAIN] = cpu_baseline(fam, voc, data, offs, args.cpu_seconds, workers)
        cpu["affinity_cores"] = affinity
        cpu["os_cpu_count"] = os.cpu_count()
        import oracle
        single = {}
        for name in (() if args.no_latency else LATENCY):
            f2, v2, d2, o2 = work[name]
            merges, _ = textgen.load_vocab(v2)
            oracle_ref[name] = oracle.encode_batch(f2, merges, d2, o2)
            reps = 20 if d2.size < 50_000 else (7 if d2.size < 2_000_000 else 3)
            single[name] = round(oracle_latency(f2, v2, d2, o2, reps), 3)
        if single:
            cpu["p50_ms_single_core"] = single
            cpu["p50_ms_1m_char_request_single_core"] = single["c3_mix1m"]

    import torch
    import exact_bpe_tokenization_amd as tt
    torch.cuda.init()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- batched throughput on the main workload ----
    merges, f = textgen.load_vocab(voc)
    tok = tt.Tokenizer(merges, f, device="cuda:0")
    d_data = torch.from_numpy(data).to(dev)
    d_offs = torch.from_numpy(offs.astype(np.int64)).to(dev)
    n, D = data.size, offs.size - 1
    tok._buffers(n, D)
    ws = tok.workspace[: tt.toktier_workspace_bytes(n, D)]
    out_ids, out_offs = tok.out_ids[:n], tok.out_offsets[: D + 1]

    def step(sync):
        return tt.toktier_encode_batch(tok.vocab, d_data, d_offs, out_ids, out_offs, ws, sync=sync)

    # warmup: the first step waits for its count (and reports any input error), the others run back
    # to back up to the timed steps (an idle gap -- a readback, a sleep -- before them lets the chip
    # slow down and costs the next steps several microseconds each)
    _log("warmup")
    step(True)
    for _ in range(args.warmup - 1):
        step(False)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gbs = n / (wall / args.steps) / 1e9
    _log("timed steps done")
    # every step encodes the whole batch again: the last step's outputs are the ones checked
    n_tok = n_tokens = tt.toktier_last_status(ws)
    gpu_ids = out_ids[:n_tok].cpu().numpy().view(np.uint32).copy()
    gpu_oo = out_offs.cpu().numpy().astype(np.uint64)

    # ---- the same steps with two batches in flight: alternate steps on two streams, each with its
    # own workspace and outputs (every step still encodes the whole batch) ----
    gbs_two, two_exact = None, None
    if not args.no_two_streams:
        s2 = [torch.cuda.Stream(device=dev) for _ in range(2)]
        bufs2 = [(ws, out_ids, out_offs), (torch.empty_like(ws), torch.empty_like(out_ids), torch.empty_like(out_offs))]
        for _ in range(max(1, args.warmup)):   # warm the second set of buffers too
            for k in range(2):
                tt.toktier_encode_batch(tok.vocab, d_data, d_offs, bufs2[k][1], bufs2[k][2], bufs2[k][0], stream=s2[k],
                                        sync=False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            w2, i2, o2 = bufs2[i % 2]
            tt.toktier_encode_batch(tok.vocab, d_data, d_offs, i2, o2, w2, stream=s2[i % 2], sync=False)
        torch.cuda.synchronize()
        wall2 = time.perf_counter() - t0
        gbs_two = round(n / (wall2 / args.steps) / 1e9, 4)
        two_exact = all(np.array_equal(b[1][:n_tok].cpu().numpy().view(np.uint32), gpu_ids) for b in bufs2)
        del bufs2

    # ---- per-kernel durations from HIP events around each launch, same steps ----
    _log("timed steps with per-kernel events")
    nk = len(tt.KERNELS)
    ev = tt.HipEvents(2 * nk * args.steps)
    torch.cuda.synchronize()
    for s in range(args.steps):
        b = ev.handles[2 * nk * s: 2 * nk * s + nk]
        a = ev.handles[2 * nk * s + nk: 2 * nk * (s + 1)]
        tt.toktier_encode_batch_timed(tok.vocab, d_data, d_offs, out_ids, out_offs, ws, b, a, sync=False)
    torch.cuda.synchronize()
    kms = {}
    for k, name in enumerate(tt.KERNELS):
        xs = [ev.elapsed_ms(ev.handles[2 * nk * s + k], ev.handles[2 * nk * s + nk + k]) for s in range(args.steps)]
        kms[name] = statistics.mean(xs)
    dominant = max(kms, key=kms.get)

    # the path's algorithmic bytes, and each kernel's own (from the GPU split and the piece results)
    starts = tok.pretokenize(data.tobytes(), offs)
    plen = np.diff(starts.astype(np.int64))
    P = int(plen.size)
    ref_ids = gpu_ids
    # tokens per piece from the IDs' byte lengths (the IDs spell the pieces in order)
    tl = token_lengths(merges)[ref_ids]
    ends = np.cumsum(tl)
    ntok_piece = np.diff(np.concatenate([[0], np.searchsorted(ends, starts[1:].astype(np.int64), side="right")]))
    multi = ntok_piece > 1
    M = int(multi.sum())
    Bm, Tm = int(plen[multi].sum()), int(ntok_piece[multi].sum())
    own = own_bytes(n, D, P, int(n_tokens), M, Bm, Tm)
    path_bytes = n + 4 * n_tokens + 16 * (D + 1)
    path_alg = path_bytes / (wall / args.steps) / 1e9
    kernels = {k: {"ms": round(kms[k], 5), "own_alg_bytes": int(own.get(k, 0)),
                   "own_hbm_frac": round(own.get(k, 0) / (kms[k] * 1e-3) / 1e9 / HBM_PEAK_GBS, 5)} for k in kms}
    traffic = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{dominant}_{MAIN}.json")
    if os.path.exists(tf):
        rec = json.load(open(tf))
        src = open(os.path.join(ROOT, "exact_bpe_tokenization_amd", "csrc", rec["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest() == rec["source_sha256"]:
            traffic = rec["bytes_per_launch"]
    valu = None
    cf = os.path.join(ROOT, "profiles", f"counters_{MAIN}.json")
    if os.path.exists(cf):
        rec = json.load(open(cf)).get(dominant)
        if rec:
            src = open(os.path.join(ROOT, "exact_bpe_tokenization_amd", "csrc", rec["source"]), "rb").read()
            if hashlib.sha256(src).hexdigest() == rec["source_sha256"]:
                valu = rec["SQ_INSTS_VALU"]
    own_gbs = own[dominant] / (kms[dominant] * 1e-3) / 1e9
    # the bound the counters point at: VALU issue against its peak, or the measured HBM traffic
    # against 8 TB/s, whichever the kernel uses more of (without counters for this source: HBM)
    valu_frac = valu / (kms[dominant] * 1e-3) / 1e9 / VALU_PEAK if valu is not None else None
    traffic_frac = traffic / (kms[dominant] * 1e-3) / 1e9 / HBM_PEAK_GBS if traffic is not None else None
    if valu_frac is not None and (traffic_frac is None or valu_frac >= traffic_frac):
        achieved = valu / (kms[dominant] * 1e-3) / 1e9
        roofline = {"bound": "alu", "achieved": round(achieved, 3), "peak": VALU_PEAK,
                    "unit": "G VALU wavefront instructions/s", "frac": round(achieved / VALU_PEAK, 5)}
    else:   # the kernel's own algorithmic bytes against HBM
        roofline = {"bound": "hbm", "achieved": round(own_gbs, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(own_gbs / HBM_PEAK_GBS, 6)}
    roofline["valu_issue_frac"] = round(valu_frac, 5) if valu_frac is not None else None
    roofline["traffic_hbm_frac"] = round(traffic_frac, 5) if traffic_frac is not None else None
    roofline.update({"traffic": traffic, "kernel": dominant, "kernel_ms": round(kms[dominant], 5),
                     "valu_insts_per_launch": valu, "own_alg_bytes_per_launch": int(own[dominant]),
                     "own_hbm_gbs": round(own_gbs, 3), "own_hbm_frac": round(own_gbs / HBM_PEAK_GBS, 6),
                     "path_alg_frac_of_hbm": round(path_alg / HBM_PEAK_GBS, 6)})

    # ---- single-request latency ----
    latency = {}
    exact = {}
    kms_c3 = None
    if two_exact is not None:
        exact[MAIN + "_two_in_flight_same_ids"] = bool(two_exact)
    if oracle_ref:
        exact[MAIN] = bool(np.array_equal(gpu_ids, oracle_ref[MAIN][0]) and np.array_equal(gpu_oo, oracle_ref[MAIN][1]))
    for name in (() if args.no_latency else LATENCY):
        f2, v2, d2, o2 = work[name]
        m2, ff = textgen.load_vocab(v2)
        t2 = tok if v2 == voc else tt.Tokenizer(m2, ff, device="cuda:0")
        dd = torch.from_numpy(d2).to(dev)
        do = torch.from_numpy(o2.astype(np.int64)).to(dev)
        for _ in range(3):
            ids_v, oo_v, nt = t2.encode_device(dd, do)
        if name in oracle_ref:
            exact[name] = bool(np.array_equal(ids_v[:nt].cpu().numpy().view(np.uint32), oracle_ref[name][0]) and
                               np.array_equal(oo_v.cpu().numpy().astype(np.uint64), oracle_ref[name][1]))
        reps = args.latency_reps if d2.size < 2_000_000 else max(5, args.latency_reps // 3)
        # per-kernel durations of the request (HIP events on the library's stream)
        nd3 = o2.size - 1
        ws3 = t2.workspace[: tt.toktier_workspace_bytes(d2.size, nd3)]
        ev3 = tt.HipEvents(2 * nk * 20)
        torch.cuda.synchronize()
        for s3 in range(20):
            b3 = ev3.handles[2 * nk * s3: 2 * nk * s3 + nk]
            a3 = ev3.handles[2 * nk * s3 + nk: 2 * nk * (s3 + 1)]
            tt.toktier_encode_batch_timed(t2.vocab, dd, do, t2.out_ids[:max(d2.size, 1)], t2.out_offsets[:nd3 + 1],
                                          ws3, b3, a3, sync=False)
        torch.cuda.synchronize()
        kms_req = {kn: round(statistics.mean(ev3.elapsed_ms(ev3.handles[2 * nk * s3 + k], ev3.handles[2 * nk * s3 + nk + k])
                                             for s3 in range(20)), 5) for k, kn in enumerate(tt.KERNELS)}
        del ev3
        ts = []
        torch.cuda.synchronize()
        for _ in range(reps):
            t0 = time.perf_counter()
            t2.encode_device(dd, do)
            ts.append((time.perf_counter() - t0) * 1e3)
        ts.sort()
        chars = len(d2.tobytes().decode("utf-8"))
        latency[name] = {"p50": round(statistics.median(ts), 4), "p90": round(ts[int(0.9 * (len(ts) - 1))], 4),
                         "bytes": int(d2.size), "chars": chars, "reps": reps,
                         "scanned_gbs_p50": round(d2.size / (statistics.median(ts) * 1e-3) / 1e9, 3),
                         "kernel_ms": kms_req}
        if name == "c3_mix1m":
            kms_c3 = kms_req
        # the same request replayed through a captured HIP graph of the kernel chain (a plan bound to
        # these buffers; every replay recomputes everything from the input buffer)
        nd2 = o2.size - 1
        plan = tt.Plan(t2.vocab, dd, do, t2.out_ids[:max(d2.size, 1)], t2.out_offsets[:nd2 + 1],
                       t2.workspace[: tt.toktier_workspace_bytes(d2.size, nd2)])
        for _ in range(3):
            nt = plan.launch()
        if name in oracle_ref:
            exact[name + "_graph"] = bool(
                np.array_equal(t2.out_ids[:nt].cpu().numpy().view(np.uint32), oracle_ref[name][0]) and
                np.array_equal(t2.out_offsets[:nd2 + 1].cpu().numpy().astype(np.uint64), oracle_ref[name][1]))
        gs = []
        torch.cuda.synchronize()
        for _ in range(reps):
            t0 = time.perf_counter()
            plan.launch()
            gs.append((time.perf_counter() - t0) * 1e3)
        del plan
        gs.sort()
        latency[name]["graph_p50"] = round(statistics.median(gs), 4)
        latency[name]["graph_p90"] = round(gs[int(0.9 * (len(gs) - 1))], 4)

    # ---- incremental repair of appends to one session ----
    repair = None if args.no_latency else repair_latency(tt)

    if args.calibrate_copy_mib:
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC, "value": round(gbs, 4), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "c4_batch64: 64 synthetic agent transcripts, lengths 10^U(4,6) chars, "
                               f"{n} bytes, cl100k-style rules, 131,072-merge vocabulary",
                   "bytes": int(n), "docs": int(D), "tokens": int(n_tokens), "family": fam,
                   "input_sha256": textgen.sha256(data.tobytes())},
        "value_two_in_flight": gbs_two,
        "p50_ms_per_1m_char_request": latency["c3_mix1m"]["p50"] if latency else None,
        "p50_ms_per_1m_char_request_graph": latency["c3_mix1m"]["graph_p50"] if latency else None,
        "latency_ms": latency,
        "path_alg_frac_of_hbm": round(path_alg / HBM_PEAK_GBS, 6),
        "path_alg_gbs": round(path_alg, 3),
        "path_alg_bytes_per_step": int(path_bytes),
        "kernel_ms": {k: round(v, 5) for k, v in kms.items()},
        "kernels": kernels,
        "kernel_ms_c3_mix1m": kms_c3,
        "repair_ms": repair,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "bit_exact": exact if exact else None,
        "bench_seconds": round(time.time() - t_start, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
