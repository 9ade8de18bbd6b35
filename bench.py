"""Benchmark: E2B-like Q4_0 prompt prefill on one MI355X.

One step = one ppx_prefill call from an empty cache (all ubatches, the
pruned single-row phase and the head), inputs resident in HBM.  Prints one
JSON line.  The metric is prefill tokens/s.  `roofline` reports the dominant
kernel, the gate|up GEMM of the row-batched layers (the largest single
contraction of a layer), against the dense fp16 MFMA peak: its algorithmic
FLOP per launch over its average launch time, from HIP events on the stream
it runs on around back-to-back launches of the same kernel, shape and
epilogue through ppx_op_gemm_glu (per-launch events inside a prefill add
their own overhead; that figure is given beside it).  `phases` gives the
whole GEMM phase, the attention phase (MFMA) and the single-row phase (HBM)
from events around every launch in a separate, identical prefill pass.  `traffic` is read from the
committed counter summary when it was taken on the current kernel source.
`cpu_baseline` times the fp64 oracle on a bounded sample.  Beside the main
line: `other_lengths`, `decode`, `prefix_reuse`, `multi_sequence` (k prompts
in one call with split caches and with one unified cache, against k calls),
`server_unified_vs_slots` (one long prompt as the only sequence of a unified
cache, where the predicate prunes, against four configured slots, where it
does not) and `config_table` (E2B-like and E4B-like at 2048 tokens and the
no-sharing control at 8192, pruned and unpruned; --table for the full set).

--pmc-pass runs the roofline's gate|up launches, an LDS-DMA read and a plain
device copy of known sizes and exits: the command under which the HBM
counters are collected.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="e2b")
    ap.add_argument("--n", type=int, default=2048, help="prompt tokens")
    ap.add_argument("--ubatch", type=int, default=0, help="0 = the config's ubatch")
    ap.add_argument("--prune", default="auto", choices=["auto", "on", "off"])
    ap.add_argument("--extra-n", default="512,8192", help="other prompt lengths to report (comma list, '' = none)")
    ap.add_argument("--decode", type=int, default=32, help="tokens decoded after the main prompt (0 = none)")
    ap.add_argument("--no-reuse", dest="reuse", action="store_false",
                    help="skip the token-verified prefix-reuse timing")
    ap.add_argument("--multi", default="16x128,8x256,4x512",
                    help="multi-sequence prefills to report, KxN = K prompts of N tokens ('' = none)")
    ap.add_argument("--server-n", type=int, default=13789,
                    help="one-prompt server case: unified cache, one sequence vs four slots (0 = skip)")
    ap.add_argument("--table", action="store_true",
                    help="time every config's full shapes, pruned and unpruned (builds 3 more models)")
    ap.add_argument("--no-matrix", dest="matrix", action="store_false",
                    help="skip the default config matrix (E2B-like and E4B-like at 2048 tokens and the "
                         "no-sharing control at 8192, each pruned and unpruned)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="prompt tokens of the oracle sample (0 = all)")
    ap.add_argument("--pmc-pass", action="store_true", help="the roofline's gate|up launches and two calibration passes, then exit")
    ap.add_argument("--pmc-attn", action="store_true",
                    help="prefill attention launches (M = ubatch rows at the end of an 8192-token context), then exit")
    return ap.parse_args()


# Sources of the GEMM kernel; counter-derived traffic is reported only while they are unchanged.
GEMM_SOURCES = ("prompt_prefill_cross_amd/csrc/gemm.hip", "prompt_prefill_cross_amd/csrc/ppx_dev.h")
TRAFFIC_FILE = "profiles/k_q4gemm_gate_up_e2b2048_traffic.txt"
COPY_CAL_BYTES = 1 << 29  # write calibration: a copy of 512 MiB (read and written once)
STREAM_CAL_BYTES = 1 << 29  # fetch calibration: 512 MiB read through LDS DMA


def gemm_source_sha():
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic():
    """Bytes per launch from the counter summary, or None when it is missing
    or was taken on another version of the kernel."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != gemm_source_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed_steps(mm, kv, toks, ub, prune, steps, warmup):
    import torch
    logits = torch.empty(mm.info["n_vocab"], dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        kv.clear()
        mm.prefill(toks, kv, n_ubatch=ub, prune=prune, logits=logits)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(steps):
        kv.clear()
        t0.record()
        mm.prefill(toks, kv, n_ubatch=ub, prune=prune, logits=logits)
        t1.record()
        t1.synchronize()
        times.append(t0.elapsed_time(t1))
    torch.cuda.synchronize()
    return np.array(times), logits


def phase_pass(ppx, mm, kv, toks, ub, prune, reps=3):
    tm_sum = None
    for _ in range(reps):
        t = ppx.Timing()
        kv.clear()
        mm.prefill(toks, kv, n_ubatch=ub, prune=prune, timing=t)
        d = t.as_dict()
        if tm_sum is None:
            tm_sum = d
        else:
            for k in d["ms"]:
                tm_sum["ms"][k] += d["ms"][k]
            tm_sum["glu_ms"] += d["glu_ms"]
    for k in tm_sum["ms"]:
        tm_sum["ms"][k] /= reps
    tm_sum["glu_ms"] /= reps
    return tm_sum


def glu_operands(mm, ub):
    """Inputs of the roofline's gate|up launches: a seeded tiled fp16 A of ub
    rows and the output h."""
    import torch
    I = mm.info
    g = torch.Generator(device="cuda").manual_seed(7)
    a = mm.tile(torch.randn((ub, I["d_model"]), generator=g, device="cuda").to(torch.float16))
    h = torch.empty(((ub + 15) // 16 * 16) * I["n_ff"], dtype=torch.float16, device="cuda")
    return a, h


def glu_kernel_us(mm, ub, reps=50, warmup=5):
    """Average duration of the gate|up GEMM (layer 0's weights, ub rows)."""
    import torch
    a, h = glu_operands(mm, ub)
    for _ in range(warmup):
        mm.op_gemm_glu("blk.0.ffn_gate", a, M=ub, out=h, raw=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        mm.op_gemm_glu("blk.0.ffn_gate", a, M=ub, out=h, raw=True)
    t1.record()
    t1.synchronize()
    return t0.elapsed_time(t1) * 1e3 / reps, reps


def decode_bytes(I, pos):
    """HBM bytes one decode step at position pos reads: every layer's Q4_0
    weights, the head, its per-layer embedding row and the K/V of positions
    0..pos of each layer's cache."""
    q4 = lambda n, k: n * k * 18 / 32
    d, qd, kvd, F, E = I["d_model"], I["n_head"] * I["head_dim"], I["kv_dim"], I["n_ff"], I["ple_dim"]
    per = q4(qd, d) + q4(d, qd) + q4(2 * F, d) + q4(d, F) + (q4(E, d) + q4(d, E) if E else 0)
    b = I["n_layer"] * (per + (pos + 1) * kvd * 2 * 2) + I["n_layer_kv_from_start"] * q4(2 * kvd, d)
    return b + q4(I["n_vocab"], d) + I["n_layer"] * E * 18 / 32


def decode_pass(mm, kv, toks, ub, n_dec, warmup=2):
    """Prefill toks[:-n_dec-warmup], then time n_dec single-token decode steps."""
    import torch
    n0 = len(toks) - n_dec - warmup
    logits = torch.empty(mm.info["n_vocab"], dtype=torch.float32, device="cuda")
    kv.clear()
    mm.prefill(toks[:n0], kv, n_ubatch=ub, logits=logits)
    for i in range(warmup):
        mm.decode(int(toks[n0 + i]), kv, logits=logits)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    p0 = kv.n_pos
    t0.record()
    for i in range(n_dec):
        mm.decode(int(toks[p0 + i]), kv, logits=logits)
    t1.record()
    t1.synchronize()
    ms = t0.elapsed_time(t1) / n_dec
    byts = float(np.mean([decode_bytes(mm.info, p0 + i) for i in range(n_dec)]))
    return {"after_prompt": p0, "tokens": n_dec, "ms_per_token": ms, "tokens_per_s": 1e3 / ms,
            "hbm_bytes_per_token": byts, "gbs": byts / (ms * 1e-3) / 1e9,
            "frac_hbm": byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def prefix_reuse_pass(mm, kv, toks, ub, keep, reps=3):
    """Token-verified prefix reuse: a snapshot of the prompt, then a prompt
    that shares its first `keep` tokens; times loading that prefix (file read
    and upload) plus the prefill of the rest, against the full prefill."""
    import tempfile
    import torch
    V = mm.info["n_vocab"]
    n = len(toks)
    new = np.concatenate([toks[:keep], (toks[keep:] + 1) % V]).astype(np.int32)
    logits = torch.empty(V, dtype=torch.float32, device="cuda")
    kv.clear()
    mm.prefill(toks, kv, n_ubatch=ub, logits=logits)
    with tempfile.TemporaryDirectory() as d:
        snap = os.path.join(d, "prefix.kvc")
        kv.save_tokens(snap, toks)
        loads, rests = [], []
        for _ in range(reps):
            kv.clear()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            L = kv.load_prefix(snap, new)
            t1 = time.perf_counter()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            mm.prefill(new[L:], kv, n_ubatch=ub, logits=logits)
            e1.record()
            e1.synchronize()
            loads.append((t1 - t0) * 1e3)
            rests.append(e0.elapsed_time(e1))
        size = os.path.getsize(snap)
    return {"prompt": n, "reused": int(L), "snapshot_bytes": size, "load_ms": float(np.median(loads)),
            "prefill_rest_ms": float(np.median(rests)),
            "total_ms": float(np.median(loads) + np.median(rests))}


def multi_pass(ppx, mm, cfg, ub, shapes, reps=5):
    """k prompts of n tokens in one ppx_prefill_multi call (one cache per
    sequence: split), in one ppx_prefill_unified call (one buffer for all
    sequences), and run one ppx_prefill after another (same stream, one timed
    region each way)."""
    import torch
    import synth
    V = mm.info["n_vocab"]
    out = {}
    for k, n in shapes:
        base = synth.prompt(cfg, k * n)
        prompts = [base[i * n:(i + 1) * n] for i in range(k)]
        kvs = [ppx.KVCache(mm, n) for _ in range(k)]
        ucache = ppx.UnifiedCache(mm, k * ((n + 63) // 64 * 64), k)
        lg_multi = torch.empty((k, V), dtype=torch.float32, device="cuda")
        lg_one = torch.empty(V, dtype=torch.float32, device="cuda")

        def run_multi():
            for kv in kvs:
                kv.clear()
            mm.prefill_multi(prompts, kvs, n_ubatch=ub, logits=lg_multi)

        def run_unified():
            for sid in range(k):
                ucache.seq_rm(sid)
            mm.prefill_unified(prompts, list(range(k)), ucache, n_ubatch=ub, logits=lg_multi)

        def run_single():
            for kv, t in zip(kvs, prompts):
                kv.clear()
                mm.prefill(t, kv, n_ubatch=ub, logits=lg_one)

        res = {}
        for name, fn in (("multi", run_multi), ("unified", run_unified), ("one_by_one", run_single)):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
            res[name] = float(np.median(ts))
        out[f"{k}x{n}"] = {"sequences": k, "tokens_each": n, "multi_ms": res["multi"],
                           "unified_ms": res["unified"], "one_by_one_ms": res["one_by_one"],
                           "multi_tokens_per_s": k * n / res["multi"] * 1e3,
                           "unified_tokens_per_s": k * n / res["unified"] * 1e3,
                           "one_by_one_tokens_per_s": k * n / res["one_by_one"] * 1e3}
        del kvs, ucache
    return out


def server_pass(ppx, mm, cfg, ub, n, reps=3):
    """The server case of the llama.cpp Gemma 4 prefill page (section 5): one
    long prompt (13,789 tokens there) into a unified cache as the only
    sequence, where the predicate prunes, against the same prompt with
    several sequence slots configured (n_seq_max 4), where the predicate's
    single-sequence clause keeps every row through every layer; and the same
    prompt through ppx_prefill into a cache of its own."""
    import torch
    import synth
    toks = synth.prompt(cfg, n)
    ucache = ppx.UnifiedCache(mm, (n + 63) // 64 * 64, 4)
    lg = torch.empty((1, mm.info["n_vocab"]), dtype=torch.float32, device="cuda")
    flags = np.zeros(mm.info["n_layer"] + 1, np.uint8)
    slots_prune = ppx.prune_predicate(mm.info["n_layer"], mm.info["n_layer_kv_from_start"], 0, 4, flags)
    kv = ppx.KVCache(mm, n)
    res = {}

    def unified(prune):
        ucache.seq_rm(0)
        mm.prefill_unified([toks], [0], ucache, n_ubatch=ub, prune=prune, logits=lg)

    def own_cache():
        kv.clear()
        mm.prefill(toks, kv, n_ubatch=ub, logits=lg[0])

    for name, fn in (("one_sequence", lambda: unified("auto")),
                     ("four_slots", lambda: unified("auto" if slots_prune else "off")),
                     ("own_cache", own_cache)):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[name] = float(np.median(ts))
    del ucache, kv
    torch.cuda.synchronize()
    return {"prompt": n, "unified_one_sequence_ms": res["one_sequence"],
            "single_sequence_cache_ms": res["own_cache"],
            "four_slots_predicate_prunes": bool(slots_prune), "four_slots_ms": res["four_slots"],
            "one_sequence_tokens_per_s": n / res["one_sequence"] * 1e3,
            "four_slots_tokens_per_s": n / res["four_slots"] * 1e3,
            "ratio": res["four_slots"] / res["one_sequence"]}


FULL_TABLE = [("e2b", (512, 2048, 8192), ("auto", "off")), ("e4b", (512, 2048, 8192), ("auto", "off")),
              ("e2b_long", (16384, 32768), ("auto",)), ("e2b_ctrl", (8192,), ("auto", "off"))]
MATRIX = [("e2b", (2048,), ("auto", "off")), ("e4b", (2048,), ("auto", "off")), ("e2b_ctrl", (8192,), ("auto", "off"))]


def table_pass(ppx, main_cfg, main_model, plan):
    """Configs of the plan [(config, prompt lengths, prune modes)], each from
    an empty cache: by default E2B-like and E4B-like at 2048 tokens and the
    no-sharing control at 8192 (pruned vs unpruned should time the same
    there), pruned and unpruned; --table adds 512 and 8192 tokens and the long
    E2B-like prompts (16384, 32768; ubatch 1024).  5 timed runs after 2
    warm-ups each, and one per-launch timing pass for the phase fractions."""
    import torch
    import synth
    rows = []
    for name, lens, prunes in plan:
        cfg = synth.CONFIGS[name]
        ub = cfg.n_ubatch
        if name == main_cfg.name:
            mm = main_model
        else:
            mm = ppx.Model(synth.build_model(cfg))
        kv = ppx.KVCache(mm, max(lens))
        for n in lens:
            toks = synth.prompt(cfg, n)
            for pr in prunes:
                times, _ = timed_steps(mm, kv, toks, ub, pr, 5, 2)
                ph = phase_pass(ppx, mm, kv, toks, ub, pr, reps=1)
                med = float(np.median(times))
                gemm = ph["gemm_flop"] / (ph["ms"]["gemm"] * 1e-3) / 1e12 if ph["ms"]["gemm"] else 0.0
                attn = ph["attn_flop"] / (ph["ms"]["attn"] * 1e-3) / 1e12 if ph["ms"]["attn"] else 0.0
                row = ph["row_bytes"] / (ph["ms"]["row"] * 1e-3) / 1e9 if ph["ms"]["row"] else 0.0
                rows.append({"config": name, "n": n, "prune": pr, "ubatch": ub, "ms_median": med,
                             "tokens_per_s": n / med * 1e3, "gemm_frac_mfma": gemm / PEAK_FP16_TFLOPS,
                             "attn_frac_mfma": attn / PEAK_FP16_TFLOPS, "row_frac_hbm": row / PEAK_HBM_GBS,
                             "phases_ms": ph["ms"]})
                print(f"# table {name} n={n} prune={pr}: {med:.2f} ms, {n / med * 1e3:.0f} tok/s, GEMM phase "
                      f"{gemm / PEAK_FP16_TFLOPS:.2f} / attention {attn / PEAK_FP16_TFLOPS:.2f} of MFMA peak",
                      file=sys.stderr, flush=True)
        del kv
        if mm is not main_model:
            mm.close()
            del mm
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return rows


def pmc_pass(ppx, mm, ub, glu_launches=20):
    """The dispatches the traffic counters are read on: the gate|up GEMM
    exactly as the roofline times it (layer 0's weights, ub rows), then a read
    of STREAM_CAL_BYTES through the same LDS DMA its producer waves use
    (FETCH_SIZE calibration: known bytes, the GEMM's load instruction), then
    a plain device copy of COPY_CAL_BYTES (WRITE_SIZE calibration)."""
    import torch
    a, h = glu_operands(mm, ub)
    for _ in range(glu_launches):
        mm.op_gemm_glu("blk.0.ffn_gate", a, M=ub, out=h, raw=True)
    buf = torch.ones(STREAM_CAL_BYTES // 4, dtype=torch.int32, device="cuda")
    ppx.stream_read(buf)
    del buf
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# pmc pass done: {glu_launches} gate|up launches (M={ub}), one {STREAM_CAL_BYTES} B LDS-DMA read, "
          f"one {COPY_CAL_BYTES} B copy", flush=True)


def pmc_attn(mm, ub, ctx=8192, launches=10):
    """The dispatches the attention counters are read on: ub query rows at
    positions ctx - ub .. ctx - 1 against ctx keys (seeded fp16 q, K, V of
    the model's head shape), through ppx_op_attention."""
    import torch
    I = mm.info
    g = torch.Generator(device="cuda").manual_seed(11)
    q = torch.randn((ub, I["n_head"], I["head_dim"]), generator=g, device="cuda").to(torch.float16)
    k = torch.randn((ctx, I["n_kv_head"], I["head_dim"]), generator=g, device="cuda").to(torch.float16)
    v = torch.randn((ctx, I["n_kv_head"], I["head_dim"]), generator=g, device="cuda").to(torch.float16)
    for _ in range(launches):
        mm.op_attention(q, k, v, ctx - ub)
    torch.cuda.synchronize()
    flop = 4.0 * I["n_head"] * I["head_dim"] * sum(ctx - ub + t + 1 for t in range(ub))
    print(f"# pmc attention pass done: {launches} launches, M={ub} at position {ctx - ub}, "
          f"{flop:.4g} FLOP per launch", flush=True)


def cpu_baseline(cfg, buf, toks, sample):
    import oracle
    m = oracle.parse_model(buf)
    kv = oracle.KVState(m, sample)
    t = time.perf_counter()
    oracle.prefill(m, kv, toks[:sample], prune=True)
    dt = time.perf_counter() - t
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": sample / dt, "unit": "tokens/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle, first {sample} tokens of the same {cfg} prompt, pruned, "
                      f"empty cache; {dt:.1f} s"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this engine runs on one GPU; --gpus {a.gpus} is not supported "
              "(multi-GPU sharding is design-only)", file=sys.stderr)
        sys.exit(2)
    import torch
    import prompt_prefill_cross_amd as ppx
    import synth

    cfg = synth.CONFIGS[a.config]
    ub = a.ubatch or cfg.n_ubatch
    buf = synth.build_model(cfg)
    mm = ppx.Model(buf)
    lens = [a.n] + [int(x) for x in a.extra_n.split(",") if x.strip() and int(x) != a.n]
    n_ctx = max(max(lens), a.n + a.decode + 2)
    kv = ppx.KVCache(mm, n_ctx)
    mm.workspace(ub, n_ctx)

    if a.pmc_pass:
        pmc_pass(ppx, mm, ub)
        return
    if a.pmc_attn:
        pmc_attn(mm, ub)
        return

    results = {}
    for n in lens:
        toks = synth.prompt(cfg, n)
        steps = a.steps if n == a.n else max(3, a.steps // 2)
        times, _ = timed_steps(mm, kv, toks, ub, a.prune, steps, a.warmup if n == a.n else 1)
        ph = phase_pass(ppx, mm, kv, toks, ub, a.prune)
        results[n] = (times, ph)
        print(f"# n={n}: {np.median(times):.3f} ms median, {n / np.median(times) * 1e3:.0f} tok/s; "
              f"phases ms {ph['ms']}", file=sys.stderr, flush=True)

    reuse = prefix_reuse_pass(mm, kv, synth.prompt(cfg, a.n), ub, a.n * 3 // 4) if a.reuse else None
    if reuse:
        print(f"# prefix reuse: {reuse['reused']} of {reuse['prompt']} cached; load {reuse['load_ms']:.1f} ms + "
              f"prefill {reuse['prefill_rest_ms']:.2f} ms", file=sys.stderr, flush=True)
    multi = None
    if a.multi.strip():
        shapes = [tuple(int(v) for v in x.split("x")) for x in a.multi.split(",") if x.strip()]
        multi = multi_pass(ppx, mm, cfg, ub, shapes)
        for key, r in multi.items():
            print(f"# multi {key}: split {r['multi_ms']:.2f} ms ({r['multi_tokens_per_s']:.0f} tok/s), unified "
                  f"{r['unified_ms']:.2f} ms, one by one {r['one_by_one_ms']:.2f} ms "
                  f"({r['one_by_one_tokens_per_s']:.0f} tok/s)", file=sys.stderr, flush=True)
    server = None
    if a.server_n:
        server = server_pass(ppx, mm, cfg, ub, a.server_n)
        print(f"# server prompt {a.server_n}: unified, one sequence {server['unified_one_sequence_ms']:.1f} ms; "
              f"four slots {server['four_slots_ms']:.1f} ms; ratio {server['ratio']:.2f}; own cache "
              f"{server['single_sequence_cache_ms']:.1f} ms", file=sys.stderr,
              flush=True)
    dec = None
    if a.decode:
        dec = decode_pass(mm, kv, synth.prompt(cfg, a.n + a.decode + 2), ub, a.decode)
        print(f"# decode after {dec['after_prompt']}: {dec['ms_per_token']:.3f} ms/token, "
              f"{dec['gbs']:.0f} GB/s", file=sys.stderr, flush=True)

    table = None
    if a.table or a.matrix:
        table = table_pass(ppx, cfg, mm, FULL_TABLE if a.table else MATRIX)
    times, ph = results[a.n]
    glu_us, glu_reps = glu_kernel_us(mm, ub)
    ms = float(np.mean(times))
    gemm_tflops = ph["gemm_flop"] / (ph["ms"]["gemm"] * 1e-3) / 1e12 if ph["ms"]["gemm"] else 0.0
    attn_tflops = ph["attn_flop"] / (ph["ms"]["attn"] * 1e-3) / 1e12 if ph["ms"]["attn"] else 0.0
    row_gbs = ph["row_bytes"] / (ph["ms"]["row"] * 1e-3) / 1e9 if ph["ms"]["row"] else 0.0
    glu_flop = 2.0 * ub * (2 * cfg.n_ff) * cfg.d_model
    glu_tflops = glu_flop / (glu_us * 1e-6) / 1e12
    # inside the prefill the gate|up launches cover every ubatch in flight at once
    glu_in_tflops = ph["glu_flop"] / (ph["glu_ms"] * 1e-3) / 1e12 if ph["glu_ms"] else 0.0
    out = {
        "metric": "prefill tokens/sec at 512/2048/8192 prompt (E2B-like Q4_0), % MFMA peak",
        "value": a.n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA (fp32 accumulate), Q4_0 weights, fp16 KV",
        "data": "synthetic: seeded random Q4_0 weights and uniform-random token ids",
        "config": {"workload": f"{cfg.name} prefill, {a.n}-token prompt, empty cache",
                   "model": f"{cfg.name}: {cfg.n_layer} layers ({cfg.n_layer_kv_from_start} own KV), d {cfg.d_model}, "
                            f"{cfg.n_head}x{cfg.head_dim} heads, {cfg.n_kv_head} KV head(s), FFN {cfg.n_ff}, "
                            f"vocab {cfg.n_vocab}, PLE {cfg.ple_dim}",
                   "global_batch": 1, "seq_len": a.n, "ubatch": ub, "prune": a.prune, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": f"k_q4gemm_p gate|up + GLU epilogue, M={ub} N={2 * cfg.n_ff} "
                                                  f"K={cfg.d_model}",
                     "achieved": glu_tflops, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": glu_tflops / PEAK_FP16_TFLOPS, "traffic": stored_traffic(),
                     "flop_per_launch": glu_flop, "avg_launch_us": glu_us, "timed_launches": glu_reps,
                     "in_prefill_launches": ph["glu_launches"],
                     "in_prefill_units": round(ph["glu_flop"] / glu_flop, 3),
                     "in_prefill_tflops_with_event_overhead": glu_in_tflops,
                     "in_prefill_frac_with_event_overhead": glu_in_tflops / PEAK_FP16_TFLOPS},
        "phases": {"ms": ph["ms"], "launches": ph["launches"],
                   "gemm_tflops": gemm_tflops, "gemm_frac_mfma": gemm_tflops / PEAK_FP16_TFLOPS,
                   "attn_tflops": attn_tflops, "attn_frac_mfma": attn_tflops / PEAK_FP16_TFLOPS,
                   "row_gbs": row_gbs, "row_frac_hbm": row_gbs / PEAK_HBM_GBS,
                   "gemm_flop": ph["gemm_flop"], "attn_flop": ph["attn_flop"], "row_bytes": ph["row_bytes"]},
        "other_lengths": {str(n): {"ms_median": float(np.median(t)), "tokens_per_s": n / float(np.median(t)) * 1e3}
                          for n, (t, _) in results.items()},
        "decode": dec,
        "prefix_reuse": reuse,
        "multi_sequence": multi,
        "server_unified_vs_slots": server,
        "config_table": table,
        "ms_median": float(np.median(times)),
        "ms_std": float(np.std(times)),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg.name, buf, synth.prompt(cfg, a.n), a.cpu_sample or a.n)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
