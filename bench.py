"""Throughput of one EAGLE-3 speculative step (draft tree + verify + accept +
compact) on one MI355X, on the LLaMA-3.1-8B-shaped workload with seeded
random weights.

Prints ONE JSON line: verified tree tokens/s (= batch * (n_nodes + 1) per step),
ms per step, the roofline of the dominant kernel (the 64-row MFMA GEMM that
streams the verify weights) from HIP events on the library's stream, the verify
pass as a whole against the same peaks (verify_pass: all of its kernels), and
the CPU oracle timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
BF16_PEAK = 2.5e15         # MI355X dense bf16 MFMA, flop/s


def max_seq_for(w, steps):
    return w.prompt_len + (steps + 2) * (w.depth + 1) + w.rows + (w.depth - 1) * w.topk + 64


def run_gpu(w, steps, warmup):
    """Timed region: `steps` replays of the captured step graph (after `warmup`
    replays).  Then `steps` eager steps with a HIP event pair around every GEMM
    and attention launch on the library's stream give per-kernel durations."""
    import torch

    from speculative_decoding_step_amd import binding as B
    from speculative_decoding_step_amd import configs
    from speculative_decoding_step_amd.engine import Engine, Spec

    t0 = time.time()
    prompts = [p for p in configs.prompts_np(w)]
    eng = Engine(w.shape, Spec.of(w), w.batch, max_seq_for(w, 2 * (steps + warmup)), w.target_seed, w.head_seed,
                 prefill_chunk=512, block_size=w.block_size, page_seed=w.cid)
    print(f"[bench] weights + context ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    if eng.sampling:                             # seeded uniforms, fixed across the replays
        from speculative_decoding_step_amd import synth
        K = w.depth
        eng.prefill(prompts, synth.uniform24_t(5000, "u_root", w.batch, "cuda"))
        na = eng.n_u_accept
        eng.set_uniforms(synth.uniform24_t(5000, "u_draft", w.batch * K, "cuda").view(w.batch, K),
                         synth.uniform24_t(5000, "u_accept", w.batch * na, "cuda").view(w.batch, na))
    else:
        eng.prefill(prompts)
    torch.cuda.synchronize()
    print(f"[bench] prefill done in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    eng.step()                                   # one eager step, then capture
    eng.capture()
    for _ in range(warmup):
        eng.replay()
    torch.cuda.synchronize()
    print("[bench] graph captured, warmup done", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(steps):
        eng.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    print(f"[bench] timed {steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    # the verify pass alone as its own graph (its replays rewrite the same tree rows: idempotent)
    gv = eng.capture_call(eng.verify)
    for _ in range(warmup):
        gv.replay()
    st = torch.cuda.current_stream()
    va, vb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    va.record(st)
    for _ in range(steps):
        gv.replay()
    vb.record(st)
    torch.cuda.synchronize()
    verify_ms = va.elapsed_time(vb) / steps
    del gv
    B.eagle3_profile(eng.ctx, True)
    # eager steps with an event pair around each of the four calls (the library launches on this stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(st)
        eng.draft()
        ev[i][1].record(st)
        eng.verify()
        ev[i][2].record(st)
        eng.accept()
        ev[i][3].record(st)
        eng.compact()
        ev[i][4].record(st)
        eng.step_idx += 1
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    phases = {name: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / steps
              for j, name in enumerate(("draft", "verify", "accept", "compact"))}
    phases["verify_graph"] = verify_ms
    prof = {k: B.eagle3_profile_read(eng.ctx, k)
            for k in (B.PROF_GEMM_M64, B.PROF_GEMM_M16, B.PROF_ATTN, B.PROF_GEMM_BIG)}
    B.eagle3_profile(eng.ctx, False)
    status = eng.device_status()
    if status:
        raise RuntimeError(f"device status flags {status:#x}")
    eng.close()
    return ms, eager_ms, prof, phases


def _slice_weights(w, n_layers):
    """float64 weights of the first n_layers target layers plus the head, seeded as
    on the GPU.  The torch twin of the seeded generator (integer-only, so its
    values equal the numpy generator's bit for bit) runs on the GPU when there
    is one, and the values are copied to host memory."""
    import numpy as np
    import torch

    from speculative_decoding_step_amd import configs, synth

    ms = w.shape
    sms = configs.ModelShape(n_layers, ms.d, ms.n_heads, ms.n_kv_heads, ms.head_dim, ms.ffn, ms.vocab,
                             ms.rope_theta, (0, 0, n_layers - 1), ms.dtype)

    def gen(seed, name, shape, kind):
        if kind == "norm":
            return np.ones(shape)
        dev = "cuda" if torch.cuda.is_available() else "cpu"
        return synth.normal_t(seed, name, shape, dev, 0.02, ms.dtype, chunk=1 << 25).cpu().to(torch.float64).numpy()

    W = {"layers": [dict() for _ in range(n_layers)]}
    for name, shape, kind in configs.target_tensor_specs(sms):
        if name[0] == "l" and name[1].isdigit():
            l, key = name[1:].split(".", 1)
            W["layers"][int(l)][key] = gen(w.target_seed, name, shape, kind)
        else:
            W[name] = gen(w.target_seed, name, shape, kind)
    H = {name[2:]: gen(w.head_seed, name, shape, kind) for name, shape, kind in configs.head_tensor_specs(sms)}
    return sms, W, H


def cpu_baseline(w):
    """The oracle (float64 numpy) on a bounded sample of the same step.

    Sample: the tree-verify target pass over the step's rows on 1-layer and
    2-layer slices of the workload's model (committed KV of prompt_len positions,
    seeded), giving the per-layer and LM-head costs, plus the oracle's whole
    draft stage (catch-up row, depth-D expansion, full-vocabulary head) on a
    short committed draft context.  Each piece is timed REPS times and its
    median is used (about 10 s of CPU work in all); step time = 32 layers +
    LM head + draft.
    """
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.llama import KVCache, Shape, target_forward
    from oracle.step import OracleSequence, SpecConfig
    from oracle.tree import tree_mask
    from speculative_decoding_step_amd import synth

    ms = w.shape
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    t_gen = time.time()
    sms, W, H = _slice_weights(w, 2)
    t_gen = time.time() - t_gen
    rng = np.random.default_rng(0)
    P, n = w.prompt_len, w.rows
    parents = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
    dep = [0] * n
    for i in range(1, n):
        dep[i] = dep[parents[i]] + 1
    m = tree_mask(parents)
    vis = [list(np.nonzero(m[i])[0]) for i in range(n)]
    toks = synth.tokens_np(1, "cpu_tree", n, ms.vocab)
    cache = KVCache(2, P + 1, ms.n_kv_heads, ms.head_dim)
    for l in range(2):
        cache.k[l][:P] = synth.normal_np(7, f"k{l}", (P, ms.n_kv_heads, ms.head_dim), 1.0, "bf16")
        cache.v[l][:P] = synth.normal_np(7, f"v{l}", (P, ms.n_kv_heads, ms.head_dim), 1.0, "bf16")
    cache.length = P
    REPS = 5
    samples = {1: [], 2: [], "draft": []}
    shp2 = Shape(2, ms.d, ms.n_heads, ms.n_kv_heads, ms.head_dim, ms.ffn, ms.vocab, ms.rope_theta, ms.eps,
                 ms.dtype, (0, 0, 1))
    spec = SpecConfig(w.mode, w.depth, w.topk, w.n_nodes, w.temperature)
    u_draft = synth.uniform24_np(10, "cpu_u_draft", w.depth + 1)  # the sampled chain's draws (seeded)
    Pd = 32
    dk = synth.normal_np(8, "dk", (Pd - 1, ms.n_kv_heads, ms.head_dim), 1.0, "bf16")
    dv = synth.normal_np(8, "dv", (Pd - 1, ms.n_kv_heads, ms.head_dim), 1.0, "bf16")
    aux = synth.normal_np(9, "aux", (1, 3 * ms.d), 1.0, "bf16").astype(np.float64)
    for _ in range(REPS):
        for L in (1, 2):
            shp = Shape(L, ms.d, ms.n_heads, ms.n_kv_heads, ms.head_dim, ms.ffn, ms.vocab, ms.rope_theta, ms.eps,
                        ms.dtype, (0, 0, 0))
            t0 = time.perf_counter()
            target_forward(W, shp, cache, toks, P + np.array(dep), vis)
            samples[L].append(time.perf_counter() - t0)
        seq = OracleSequence(W, H, shp2, spec, Pd + 2 * n + w.depth * w.topk)  # fresh state for each repeat
        seq.cache.length = Pd
        seq.dcache.k[0][:Pd - 1] = dk
        seq.dcache.v[0][:Pd - 1] = dv
        seq.dcache.length = Pd - 1
        seq.aux_new = aux
        seq.next_tok = [int(toks[0])]
        seq.root = int(toks[0])
        t0 = time.perf_counter()
        seq.draft_tree(u_draft)
        samples["draft"].append(time.perf_counter() - t0)
    times = {k: float(np.median(v)) for k, v in samples.items()}
    t_layer = times[2] - times[1]
    t_head = max(times[1] - t_layer, 0.0)
    t_step = ms.n_layers * t_layer + t_head + times["draft"]
    work = sum(sum(v) for v in samples.values())
    return {"value": round(w.batch * w.rows / t_step, 3), "unit": "verified tree tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"float64 numpy oracle, batch 1: tree verify of {n} rows over {P} committed positions on "
                       f"1- and 2-layer slices of the {w.name} model ({times[1]:.1f}s, {times[2]:.1f}s) and the draft "
                       f"stage ({times['draft']:.1f}s), medians of {REPS} repeats; step = {ms.n_layers} x layer ({t_layer:.2f}s) + LM head "
                       f"({t_head:.2f}s) + draft = {t_step:.1f}s; {work:.0f}s of CPU work "
                       f"(+{t_gen:.0f}s generating the slice's seeded weights)")}


KERNEL_NAMES = {
    0: "k_gemm_bf16<4,*,*> (64-row MFMA weight-streaming GEMMs, packed weights)",
    1: "k_gemm_bf16<1,2,4,*> (16-row MFMA weight-streaming GEMMs, packed weights)",
    3: "k_gemm_bf16_big (128x256-tile MFMA GEMM)",
}


def step_bytes(w):
    """Algorithmic HBM bytes of one step: every weight the step's passes read
    (target layers + LM head once; draft FC once; draft layer + draft LM head per
    draft forward, depth forwards per step) plus the K/V the attention reads."""
    import numpy as np

    from speculative_decoding_step_amd import configs

    s = w.shape
    e = 2 if s.dtype == "bf16" else 4
    q, kv = s.n_heads * s.head_dim, s.n_kv_heads * s.head_dim
    tgt_layer = s.d * q + 2 * s.d * kv + q * s.d + 3 * s.d * s.ffn
    drf_layer = 2 * s.d * q + 2 * 2 * s.d * kv + q * s.d + 3 * s.d * s.ffn
    lm = s.vocab * s.d
    dlm = (s.draft_vocab or s.vocab) * s.d  # the draft's head: its own reduced one, or the shared target head
    weights = s.n_layers * tgt_layer + lm + 3 * s.d * s.d + w.depth * (drf_layer + dlm)
    ctx = float(np.sum(configs.prompt_lengths(w)))
    kv_bytes = 2 * kv * e * (s.n_layers * (ctx + w.batch * w.rows) + w.depth * ctx)
    return weights * e + kv_bytes


def verify_work(w):
    """Algorithmic work of one verify pass: HBM bytes (every target weight and the
    LM head once, the committed K/V the attention reads, the tree rows' K/V and
    aux rows written) and the GEMM flops (2 x rows x weight elements)."""
    import numpy as np

    from speculative_decoding_step_amd import configs

    s = w.shape
    e = 2 if s.dtype == "bf16" else 4
    q, kv = s.n_heads * s.head_dim, s.n_kv_heads * s.head_dim
    params = s.n_layers * (s.d * q + 2 * s.d * kv + q * s.d + 3 * s.d * s.ffn) + s.vocab * s.d
    ctx = float(np.sum(configs.prompt_lengths(w)))
    rows = w.batch * w.rows
    nbytes = params * e + 2 * kv * e * s.n_layers * (ctx + rows) + rows * 3 * s.d * e
    return nbytes, 2.0 * rows * params


def verify_pass(w, phases):
    """The verify pass as a whole (every kernel of eagle3_verify_tree: GEMMs,
    attention and its merge, norms, RoPE/KV writes, top-2), timed as its own
    graph replayed back to back: algorithmic bytes against the HBM peak, and
    GEMM flops against the bf16 MFMA peak.  phases_ms: the four calls of the
    eager profiled steps (host launch gaps included) and the verify graph."""
    nbytes, flops = verify_work(w)
    t = phases["verify_graph"] / 1e3
    return {"ms": round(phases["verify_graph"], 4), "algorithmic_bytes": round(nbytes), "gemm_flops": round(flops),
            "hbm_gbps": round(nbytes / t / 1e9, 1), "hbm_frac": round(nbytes / t / HBM_PEAK, 4),
            "mfma_tflops": round(flops / t / 1e12, 1), "mfma_frac": round(flops / t / BF16_PEAK, 4),
            "phases_ms": {k: round(v, 4) for k, v in phases.items()}}


def roofline(w, prof, steps):
    """Roofline of the dominant kernel (largest total time among the GEMM kinds):
    HBM-bound weight streaming for the skinny kernels, MFMA-bound for the
    large-M kernel.  achieved = algorithmic bytes (or flops) / event time."""
    kinds = [k for k in (0, 1, 3) if prof[k][0] > 0]
    k = max(kinds, key=lambda x: prof[x][1])
    n, t_ms, by, fl = prof[k]
    if k == 3:
        achieved = fl / (t_ms / 1e3)
        out = {"bound": "mfma", "achieved": round(achieved / 1e12, 1), "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s",
               "frac": round(achieved / BF16_PEAK, 4)}
    else:
        achieved = by / (t_ms / 1e3)
        out = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
               "frac": round(achieved / HBM_PEAK, 4)}
    out["traffic"] = measured_traffic(w, k)
    out.update({"kernel": KERNEL_NAMES[k], "launches_per_step": n / steps, "kernel_ms_per_step": round(t_ms / steps, 4),
                "algorithmic_bytes_per_launch": round(by / n), "flops_per_launch": round(fl / n)})
    return out


def _kernel_source_digest(kind):
    """Digest of the source file that holds the kernel of this kind."""
    import hashlib

    name = "k_gemm_big.hip" if kind == 3 else "k_gemm.hip"
    path = os.path.join(ROOT, "speculative_decoding_step_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(w, kind):
    """HBM bytes per launch of the dominant kernel from the counter summary in
    profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by the copy calibration),
    or None when there is none for this workload or the kernel source changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_kind") != kind or t.get("source_digest") != _kernel_source_digest(kind):
        return None
    return t["bytes_per_launch"]


def traffic_from_counters(workload, kind, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, mib, last=0):
    """Writes profiles/traffic_<workload>.json from rocprofv3 --pmc FETCH_SIZE and
    WRITE_SIZE runs of bench.py and of --copy-probe MIB (the copy kernel reads
    and writes MIB MiB per dispatch: its counters give the scale factors).
    last > 0 keeps only the kernel's last `last` dispatches (the profiled eager
    steps that end a bench run, not the prefill's launches of the same kernel)."""
    import csv

    # kernel-name prefixes: the 64-row kernels (plain and fused gate/up), the 16-row ones, the large-M one
    names = {0: "k_gemm_bf16<4, ", 1: "k_gemm_bf16<1, ", 3: "k_gemm_bf16_big"}

    def per_dispatch(path, needle, keep=0):
        rows = [r for r in csv.DictReader(open(path)) if needle in r["Kernel_Name"]]
        if rows and "Dispatch_Id" in rows[0]:
            rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        vals = [float(r["Counter_Value"]) * 1024.0 for r in rows]
        return vals[-keep:] if keep else vals

    nbytes = mib << 20
    f_copy = per_dispatch(copy_fetch_csv, "copyBuffer")
    w_copy = per_dispatch(copy_write_csv, "copyBuffer")
    f_scale = nbytes / (sum(f_copy) / len(f_copy))
    w_scale = nbytes / (sum(w_copy) / len(w_copy))
    fv = per_dispatch(fetch_csv, names[kind], last)
    wv = per_dispatch(write_csv, names[kind], last)
    per_launch = sum(fv) / len(fv) * f_scale + sum(wv) / len(wv) * w_scale
    out = {"workload": workload, "kernel_kind": kind, "kernel": names[kind], "source_digest": _kernel_source_digest(kind),
           "bytes_per_launch": round(per_launch), "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "dispatches": [len(fv), len(wv)]}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def copy_probe(mib):
    """Five copies of a MIB-MiB device buffer into another: each dispatch reads and
    writes exactly mib * 2^20 bytes."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_dispatch": n, "dispatches": 5}), flush=True)


def ttt_cpu_baseline(T, S, Hq, Hkv, hd, n_sample=2048):
    """The oracle's training-time-test attention (float64 numpy) on n_sample evenly spaced
    positions of the same call (their mean causal length is the call's; at the default
    T 2048 every position, ~10 s), timed once; positions/s = n_sample / time."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.ttt import ttt_attention
    from speculative_decoding_step_amd import synth

    cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    args = [synth.normal_np(9, n, shp, 1.0, "bf16").astype(np.float64)
            for n, shp in (("q", (T, Hq, hd)), ("k0", (Hkv, T, hd)), ("v0", (Hkv, T, hd)),
                           ("ks", (S, Hkv, T, hd)), ("vs", (S, Hkv, T, hd)))]
    pos = sorted(set(int(x) for x in np.linspace(0, T - 1, min(n_sample, T))))
    t0 = time.perf_counter()
    ttt_attention(*args, positions=pos)
    t = time.perf_counter() - t0
    return {"value": round(len(pos) / t, 2), "unit": "positions/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 numpy oracle: {len(pos)} evenly spaced positions of the same call "
                      f"(T {T}, S {S}, {Hq}/{Hkv} heads x {hd}), {t:.1f}s"}


def ttt_bench(steps, warmup, T=2048, S=7, Hq=32, Hkv=8, hd=128, cpu=True):
    """Training-time-test attention at the 8B draft layer's head layout (T positions,
    S simulated steps, bf16, seeded N(0, 1) inputs resident on the device).  One step
    = one eagle3_ttt_attention call.  Roofline: MFMA against the bf16 peak, with the
    algorithmic flops of the causal QK and PV products plus the diagonal terms."""
    import torch

    from speculative_decoding_step_amd import binding as B
    from speculative_decoding_step_amd import synth

    dev = "cuda"
    ten = {n: synth.normal_t(9, n, shp, dev, 1.0, "bf16")
           for n, shp in (("q", (T, Hq, hd)), ("k0", (Hkv, T, hd)), ("v0", (Hkv, T, hd)),
                          ("ks", (S, Hkv, T, hd)), ("vs", (S, Hkv, T, hd)))}
    out = torch.empty(T, Hq, hd, dtype=torch.bfloat16, device=dev)
    wsb = B.eagle3_ttt_workspace_bytes(T, Hq, hd)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()

    def call():
        B.eagle3_ttt_attention(B.BF16, T, S, Hq, Hkv, hd, ten["q"].data_ptr(), ten["k0"].data_ptr(),
                               ten["v0"].data_ptr(), ten["ks"].data_ptr(), ten["vs"].data_ptr(), out.data_ptr(),
                               ws.data_ptr(), wsb, st.cuda_stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(steps):
        call()
    b.record(st)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    flops = 4.0 * Hq * hd * (T * (T + 1) / 2 + T * S)
    nbytes = 2.0 * (2 * T * Hq * hd + 2 * (1 + S) * Hkv * T * hd)  # q, out, and every step's K and V
    achieved = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "training-time-test attention positions/s", "value": round(T / (ms * 1e-3), 1),
        "unit": "positions/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) q, k, v", "config": {"workload": "ttt_attn_8b", "positions": T,
                                                                "simulated_steps": S, "q_heads": Hq,
                                                                "kv_heads": Hkv, "head_dim": hd},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(achieved / 2500.0, 4), "traffic": None, "algorithmic_bytes": nbytes,
                     "hbm_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)},
        "cpu_baseline": ttt_cpu_baseline(T, S, Hq, Hkv, hd) if cpu else None}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_tree_b1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the reference point that "
                         "scales the HBM byte counters of a profiler run) and exit")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="only write profiles/traffic_<workload>.json from the counter CSVs of a bench run and a "
                         "--copy-probe run, then exit")
    ap.add_argument("--traffic-kind", type=int, default=0, help="kernel kind for --traffic-from (0, 1 or 3)")
    ap.add_argument("--traffic-mib", type=int, default=1024, help="copy size of the --copy-probe run, MiB")
    ap.add_argument("--traffic-last", type=int, default=0,
                    help="for --traffic-from: use only the kernel's last N dispatches (the profiled steps)")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from_counters(args.workload, args.traffic_kind, *args.traffic_from, args.traffic_mib,
                              args.traffic_last)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the step shards by sequence "
              "with no exchange; run one process per GPU). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "ttt_attn_8b":
        ttt_bench(args.steps, args.warmup, cpu=not args.no_cpu_baseline)
        return
    from speculative_decoding_step_amd import configs

    w = configs.WORKLOADS[args.workload]
    ms, eager_ms, prof, phases = run_gpu(w, args.steps, args.warmup)
    rows = w.batch * w.rows
    line = {
        "metric": "verified tree tokens/s",
        "value": round(rows / (ms / 1e3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "eager_ms_per_step": round(eager_ms, 4),
        "us_per_step": round(ms * 1e3, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.shape.dtype,
        "data": "synthetic: seeded N(0,0.02) weights, uniform prompt ids",
        "config": {"workload": w.name, "batch": w.batch, "prompt_len": w.prompt_len, "tree_depth": w.depth,
                   "topk": w.topk, "tree_nodes": w.n_nodes, "rows_per_step": rows,
                   "kv_block_size": w.block_size or None},
        "roofline": roofline(w, prof, args.steps),
        "verify_pass": verify_pass(w, phases),
        "hbm_gbps_step": round(step_bytes(w) / (ms / 1e3) / 1e9, 1),
        "cpu_baseline": None,
    }
    vp = line["verify_pass"]
    line["roofline"]["verify_pass_frac"] = vp["mfma_frac"] if line["roofline"]["bound"] == "mfma" else vp["hbm_frac"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
