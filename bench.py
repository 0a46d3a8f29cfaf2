"""Benchmark of the GDN mixer core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-layer]
                    [--no-spec] [--no-gqa] [--no-cpu]

Headline workload (N=1): one decode step of 64 requests at full shapes (16 key /
48 value heads, d = 128, fp32 state [64,48,128,128]): conv update -> recurrence
-> gated norm in one launch (gdn_decode_fused), with every input already
resident in HBM; the same step as three launches (conv1d_update ->
decode_step -> gated_norm) is timed beside it.  `value`
is the state bytes each step reads and writes (2 x 64 x 3 MiB) divided by the
measured step time.  A prefill leg (single 4096-token sequence; 16-request
packed varlen batch) reports tokens/s in the same run, a speculative-verify leg
times 64 requests x 4 tokens with per-position state slots, a GQA leg times the
full-attention layers' decode core (64 requests over a paged KV cache of about
131k positions, bf16 and fp8 e4m3), a layer leg times the
whole layer block on the mixed 8 x 2048 + 256 batch at hidden 5120, and the
fp64 CPU oracle is timed on a bounded sample on the host cores.

Prints ONE JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("GDN prefill tokens/s + decode state GB/s vs HBM peak "
          "(48×128×128 fp32 state)")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
NORM_EPS = 1e-6
L2_EPS = 1e-6


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-varlen", action="store_true")
    p.add_argument("--no-layer", action="store_true")
    p.add_argument("--layer-steps", type=int, default=5)
    p.add_argument("--no-spec", action="store_true")
    p.add_argument("--spec-steps", type=int, default=20)
    p.add_argument("--no-gqa", action="store_true")
    p.add_argument("--gqa-steps", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-ref-mib", type=int, default=0,
                   help="after the benchmark, run plain device copies of this many MiB "
                        "(a known-size reference for the HBM byte counters)")
    return p.parse_args()


def source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, source):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/<kernel>_traffic.txt: FETCH_SIZE and WRITE_SIZE scaled by
    a plain copy's reading), or None when that summary is missing or was taken
    on a different version of the kernel's source file."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    src = os.path.join(ROOT, "hybrid_linear_attention_amd", "csrc", source)
    if vals.get("source") != source or source_digest(src) != vals.get("source_sha256_16"):
        return None
    return int(float(vals["hbm_bytes_per_launch"]))


def step_counters(name):
    """Counter summary of a multi-kernel step (profiles/<name>_counters.txt:
    per-kernel HBM bytes from FETCH_SIZE / WRITE_SIZE scaled by a plain copy's
    reading, MFMA busy cycles and issued MFMA flops), or None when it is missing
    or any source file it names has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.txt")
    if not os.path.exists(path):
        return None
    vals, kernels = {}, []
    with open(path) as f:
        for line in f:
            if line.startswith("#"):
                continue
            if line.startswith("kernel:"):
                kernels.append(line.split()[1])
                continue
            if line.startswith("source_sha256_16 "):
                src, digest = line[len("source_sha256_16 "):].split(":")
                if source_digest(os.path.join(ROOT, "hybrid_linear_attention_amd", "csrc",
                                              src.strip())) != digest.strip():
                    return None
                continue
            if ":" in line:
                key, val = line.split(":", 1)
                vals[key.strip()] = float(val.strip())
    vals["kernels"] = kernels
    return vals


def gemm_counters():
    """MFMA-busy share and calibrated HBM bytes of the layer's two GEMMs from
    profiles/layer_gemm_counters.txt, or None when it is missing or gemm.hip has
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "layer_gemm_counters.txt")
    if not os.path.exists(path):
        return None
    out, cur = {}, None
    with open(path) as f:
        for line in f:
            if line.startswith("gemm:"):
                cur = "in_proj" if "in-projection" in line else "out_proj"
            elif line.startswith("  mfma_busy") and cur:
                out[cur + "_mfma_busy"] = float(line.split()[1])
            elif line.startswith("  fetch_bytes") and cur:
                t = line.split()
                out[cur + "_hbm_bytes"] = int(float(t[1]) + float(t[3]))
            elif line.startswith("source_sha256_16 "):
                src, digest = line[len("source_sha256_16 "):].split(":")
                if source_digest(os.path.join(ROOT, "hybrid_linear_attention_amd", "csrc",
                                              src.strip())) != digest.strip():
                    return None
    out["counters"] = "profiles/layer_gemm_counters.txt"
    return out


def fused_decode_bytes(d, R, act_bytes=2, y_bytes=2, state_bytes=4):
    """Algorithmic HBM bytes of one gdn_decode_fused launch: the state read and
    written once; the token's conv inputs, z and gates read once; its conv
    history read and written once; y written once (413,413,376 B at 64
    requests, full shapes, bf16 activations, fp32 state; 212,086,784 B with a
    bf16 state)."""
    Hv, D = d.num_v_heads, d.head_dim_v
    C = 2 * d.num_k_heads * d.head_dim_k + Hv * D
    state = 2 * R * Hv * D * d.head_dim_k * state_bytes
    io = R * (C * act_bytes + 2 * C * (d.conv_taps - 1) * act_bytes + Hv * D * act_bytes
              + 2 * Hv * act_bytes + Hv * D * y_bytes)
    return state + io


def decode_bytes(d, R, act_bytes=4, o_bytes=4):
    """Algorithmic HBM bytes of one decode_step launch: the state read and
    written once, q/k/v/a/b read once, o written once."""
    D = d.head_dim_k
    state = 2 * R * d.num_v_heads * D * D * 4
    qkv = R * (2 * d.num_k_heads + d.num_v_heads) * D * act_bytes
    gates = 2 * R * d.num_v_heads * 2
    o = R * d.num_v_heads * D * o_bytes
    return state, state + qkv + gates + o


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from hybrid_linear_attention_amd import gdn
    from hybrid_linear_attention_amd.workloads import decode_r64, prefill_4096, prefill_varlen16

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gdn.lib()
    dev = "cuda"
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------------ decode
    case = decode_r64()
    d = case.dims
    R = case.num_reqs
    D = d.head_dim_k
    x = case.x_qkv.to(dev)
    conv_w = case.conv_w.to(dev)
    # Three layers' worth of caches, used in turn: a model's GDN layers each own
    # a state pool, so a layer's state is never still resident in the 256 MB
    # memory-side cache when its next decode step comes round.
    n_rot = 3
    conv_pools = [case.conv_pool.to(dev) for _ in range(n_rot)]
    states = [case.state_pool.to(dev) for _ in range(n_rot)]
    qsl = case.qsl.to(dev)
    slots = case.slot_ids.to(dev)
    hinit = case.has_initial.to(dev)
    a, b, z, gamma = case.a.to(dev), case.b.to(dev), case.z.to(dev), case.gamma.to(dev)
    q = torch.empty((R, d.num_k_heads, D), device=dev)
    k = torch.empty_like(q)
    v = torch.empty((R, d.num_v_heads, D), device=dev)
    o = torch.empty((R, d.num_v_heads, D), device=dev)
    y = torch.empty((R, d.num_v_heads * D), dtype=torch.bfloat16, device=dev)

    sh = stream.cuda_stream  # raw hipStream_t, passed to every call
    it_count = [0]

    def three_launch_step(ev=None):
        conv_pool = conv_pools[it_count[0] % n_rot]
        state = states[it_count[0] % n_rot]
        it_count[0] += 1
        if ev:
            ev[0].record(stream)
        gdn.gdn_conv1d_update(d, x, conv_w, conv_pool, qsl, slots, hinit, q, k, v, l2_eps=L2_EPS,
                              stream=sh)
        if ev:
            ev[1].record(stream)
        gdn.gdn_decode_step(d, q, k, v, a, b, state, slots, o, stream=sh)
        if ev:
            ev[2].record(stream)
        gdn.gdn_gated_norm(d, o, z, gamma, y, eps=NORM_EPS, stream=sh)
        if ev:
            ev[3].record(stream)

    def fused_step(ev=None):
        conv_pool = conv_pools[it_count[0] % n_rot]
        state = states[it_count[0] % n_rot]
        it_count[0] += 1
        gdn.gdn_decode_fused(d, x, z, a, b, conv_w, gamma, conv_pool, state, slots, y,
                             l2_eps=L2_EPS, norm_eps=NORM_EPS, stream=sh)

    def timed(step):
        """K back-to-back steps after W warm-up steps: wall-clock ms per step, and
        the stream's own time per step from one event pair around the region."""
        for _ in range(args.warmup):
            step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / args.steps
        return wall, e0.elapsed_time(e1) / args.steps

    ms_three, gpu_three = timed(three_launch_step)
    ms_step, gpu_fused = timed(fused_step)
    # per-launch breakdown of the three-launch step (events between launches add a
    # few microseconds each, so this pass is separate from the timed ones)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        three_launch_step(e)
    torch.cuda.synchronize()
    kern_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
               for i, n in enumerate(("conv", "decode", "norm"))}
    kern_ms["fused"] = gpu_fused
    state_bytes, dec_bytes = decode_bytes(d, R)
    step_bytes = fused_decode_bytes(d, R)
    value = state_bytes / (ms_step * 1e-3) / 1e9
    achieved = step_bytes / (gpu_fused * 1e-3) / 1e9
    achieved_dec = dec_bytes / (kern_ms["decode"] * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode_r64: 64 requests x 1 token; 16 key / 48 value heads; "
                        "d_k = d_v = 128; fp32 state [64,48,128,128]; bf16 inputs",
            "step": "gdn_decode_fused (conv update + recurrence + gated norm, one launch)",
            "state_bytes_per_step": state_bytes,
            "state_pools_rotated": n_rot,
        },
        "kernel_ms": {n: round(t, 4) for n, t in kern_ms.items()},
        "roofline": {
            "kernel": "decode_fused_kernel (gdn_decode_fused)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": step_bytes,
            "traffic": measured_traffic("decode_fused_kernel", "decode_fused.hip"),
        },
        "three_launch": {
            "step": "gdn_conv1d_update + gdn_decode_step + gdn_gated_norm",
            "ms_per_step": round(ms_three, 4),
            "gpu_ms_per_step": round(gpu_three, 4),
            "value": round(state_bytes / (ms_three * 1e-3) / 1e9, 2),
            "decode_kernel_roofline": {
                "achieved": round(achieved_dec, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_dec / HBM_PEAK_GBS, 4), "bytes_per_launch": dec_bytes,
                "traffic": measured_traffic("decode_kernel", "decode.hip"),
            },
        },
    }
    # the same step with the state stored in bf16 (the state-dtype variant)
    states16 = [st.to(torch.bfloat16) for st in states]
    it_count[0] = 0

    def fused_step_bf16():
        i = it_count[0] % n_rot
        it_count[0] += 1
        gdn.gdn_decode_fused(d, x, z, a, b, conv_w, gamma, conv_pools[i], states16[i], slots, y,
                             l2_eps=L2_EPS, norm_eps=NORM_EPS, stream=sh)

    ms16, gpu16 = timed(fused_step_bf16)
    b16 = fused_decode_bytes(d, R, state_bytes=2)
    a16 = b16 / (gpu16 * 1e-3) / 1e9
    result["decode_bf16_state"] = {
        "step": "gdn_decode_fused with a bf16 state [64,48,128,128] (widened on load, "
                "rounded once on store)",
        "ms_per_step": round(ms16, 4),
        "gpu_ms_per_step": round(gpu16, 4),
        "state_gbs": round(state_bytes / 2 / (ms16 * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "decode_fused_kernel (bf16 state)", "bound": "hbm",
                     "achieved": round(a16, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(a16 / HBM_PEAK_GBS, 4), "bytes_per_launch": b16,
                     "traffic": measured_traffic("decode_fused_kernel_bf16_state", "decode_fused.hip")},
    }
    del states, conv_pools, states16
    torch.cuda.empty_cache()

    # ----------------------------------------------------------------- prefill
    if not args.no_prefill:
        legs = [("prefill_4096", prefill_4096)]
        if not args.no_varlen:
            legs.append(("prefill_varlen16", prefill_varlen16))
        pre = {}
        for name, make in legs:
            c = make()
            pre[name] = bench_prefill(c, args.prefill_steps, dev, stream, torch, gdn, np, name=name)
            if name == "prefill_varlen16":
                # the same step keeping a prefix-cache snapshot every 512 tokens
                pre[name]["with_snapshots"] = bench_prefill(c, args.prefill_steps, dev, stream,
                                                            torch, gdn, np, snap_interval=512)
            if not args.no_cpu:
                pre[name]["cpu_baseline"] = (cpu_prefill_baseline(c, 4096, 1024) if c.num_reqs == 1
                                             else cpu_prefill_baseline(c, 512, 64))
            del c
            torch.cuda.empty_cache()
        result["prefill"] = pre

    # ------------------------------------------------------ speculative verify
    if not args.no_spec:
        result["spec_verify"] = bench_spec(args.spec_steps, args.warmup, dev, stream, torch, gdn)
        torch.cuda.empty_cache()

    # ------------------------------------------------- GQA layer decode core
    if not args.no_gqa:
        from hybrid_linear_attention_amd import gqa
        result["gqa_decode"] = bench_gqa(args.gqa_steps, args.warmup, dev, stream, torch, gqa)
        torch.cuda.empty_cache()
        result["gqa_decode_fp8"] = bench_gqa(args.gqa_steps, args.warmup, dev, stream, torch, gqa, fp8=True)
        torch.cuda.empty_cache()

    # ------------------------------------------------------------- layer block
    if not args.no_layer:
        result["layer"] = bench_layer(args.layer_steps, dev, stream, torch, np)
        torch.cuda.empty_cache()
        if not args.no_cpu:
            result["layer"]["cpu_baseline"] = cpu_layer_baseline()

    # --------------------------------------- measured HBM reference rates
    result["hbm_reference"] = hbm_reference(torch, dev)

    # ------------------------------------------------------------ CPU baseline
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)

    if args.copy_ref_mib > 0:
        # a plain elementwise kernel of known size: reads n*4 bytes, writes n*4
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        result["copy_ref_bytes"] = {"read": n * 4, "write": n * 4, "launches": 3}

    print(json.dumps(result), flush=True)


def prefill_flops(d, T, chunk=32):
    """Algorithmic flops of the chunkwise gated delta rule over T tokens at
    chunk length C: per token and value head 6 d_k d_v (K S0^T, Q S0^T and the
    state update) + C (2 d_k + 4 d_v) (the triangular solve applied to V and K,
    and P Delta) + C^2 / 3 (forming T), plus per key head 4 C d_k (K K^T and
    Q K^T).  6.16 MFLOP per token at 16/48 heads, d = 128, C = 32 (the
    chunk length the prefill kernels use)."""
    Dk, Dv = d.head_dim_k, d.head_dim_v
    per_tok = (d.num_v_heads * (6 * Dk * Dv + chunk * (2 * Dk + 4 * Dv) + chunk * chunk / 3)
               + d.num_k_heads * 4 * chunk * Dk)
    return float(per_tok * T)


def prefill_bytes(d, T, nreq, n_init, act_bytes=4, gate_bytes=2, o_bytes=4):
    """Algorithmic HBM bytes of one gdn_prefill_varlen launch: q, k, v and the
    two gate rows read once, o written once, each request's state written once
    (and read once where it has an initial state)."""
    per_tok = (act_bytes * (2 * d.num_k_heads * d.head_dim_k + d.num_v_heads * d.head_dim_v)
               + 2 * gate_bytes * d.num_v_heads + o_bytes * d.num_v_heads * d.head_dim_v)
    state = d.num_v_heads * d.head_dim_v * d.head_dim_k * 4
    return per_tok * T + state * (nreq + n_init)


def bench_layer(steps, dev, stream, torch, np):
    """The full layer block on the mixed batch (8 x 2048 prefill tokens + 256
    decode tokens, hidden 5120): RMSNorm -> in-projection -> gdn_prefill_fused
    (prefill requests) and gdn_decode_fused (decode requests) -> out-projection +
    residual, with every launch timed by events on the stream."""
    from hybrid_linear_attention_amd.layer import GdnLayer, stack_weights
    from hybrid_linear_attention_amd.workloads import layer_mixed

    case = layer_mixed()
    core = case.core
    d = core.dims
    T = int(core.qsl[-1])
    T_pf = case.num_prefill * case.prefill_len
    w = stack_weights(d, case.W_qkvz, case.W_ba, case.W_o, core.conv_w, case.gamma_in,
                      core.gamma, device=dev)
    layer = GdnLayer(d, w, T, case.num_prefill, T_pf, case.num_decode, NORM_EPS, L2_EPS,
                     device=dev)
    X = case.X.to(dev)
    pool, state = core.conv_pool.to(dev), core.state_pool.to(dev)
    qsl, slots, hinit = core.qsl.to(dev), core.slot_ids.to(dev), core.has_initial.to(dev)
    del case
    stages = layer.stages(X, pool, state, qsl, slots, hinit)
    names = [n for n, _ in stages]
    per, tot = {n: [] for n in names}, []
    # every step enqueued before the one synchronisation, so that no step's events
    # also time the host launching onto an idle GPU
    evs = []
    for it in range(steps + 1):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
        ev[0].record(stream)
        for i, (_, fn) in enumerate(stages):
            fn()
            ev[i + 1].record(stream)
        evs.append(ev)
    torch.cuda.synchronize()
    for ev in evs[1:]:  # the first step is warm-up
        for i, n in enumerate(names):
            per[n].append(ev[i].elapsed_time(ev[i + 1]))
        tot.append(ev[0].elapsed_time(ev[-1]))
    med = {n: float(np.median(v)) for n, v in per.items()}
    ms = float(np.median(tot))
    hidden = X.shape[1]
    n_in = w.W_in.shape[0]
    f_in = 2.0 * T * hidden * n_in
    f_out = 2.0 * T * w.W_out.shape[1] * hidden
    out = {
        "workload": f"layer_mixed: {T} tokens = 8 x 2048 prefill + 256 decode, hidden {hidden}",
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "stage_ms": {n: round(v, 4) for n, v in med.items()},
        "in_proj_tflops": round(f_in / (med["in_proj"] * 1e-3) / 1e12, 1),
        "out_proj_tflops": round(f_out / (med["out_proj"] * 1e-3) / 1e12, 1),
        "gemm_counters": gemm_counters(),
    }
    del layer, w, X, pool, state
    return out


def fused_prefill_bytes(d, T, nreq, n_init, act_bytes=2, y_bytes=2):
    """Algorithmic HBM bytes of one gdn_prefill_fused call: each token's conv
    inputs, z and gates read once and its y written once; each request's state
    written once (read once where it has an initial state) and its conv history
    read and written once."""
    Hv, D = d.num_v_heads, d.head_dim_v
    C = 2 * d.num_k_heads * d.head_dim_k + Hv * D
    per_tok = act_bytes * (C + Hv * D + 2 * Hv) + y_bytes * Hv * D
    state = Hv * D * d.head_dim_k * 4
    hist = 2 * C * (d.conv_taps - 1) * act_bytes
    return per_tok * T + state * (nreq + n_init) + hist * nreq


def cnt_kernels(name):
    """The kernels a step's counter summary lists, in dispatch order ([] when
    there is no current summary)."""
    cnt = step_counters(name)
    return cnt["kernels"] if cnt else []


def bench_prefill(c, steps, dev, stream, torch, gdn, np, snap_interval=0, name=None):
    """One prefill step (gdn_prefill_fused: conv update -> recurrence -> gated
    norm) over one packed batch.  State and history are re-seeded from device
    copies before every step, outside the timed events.  With snap_interval,
    the step also keeps a prefix-cache snapshot every snap_interval tokens, in
    slots appended to the pools."""
    d = c.dims
    T = c.num_tokens
    x, conv_w = c.x_qkv.to(dev), c.conv_w.to(dev)
    snaps, nsnap = None, 0
    if snap_interval:
        lens = np.diff(c.qsl.numpy())
        max_snaps = int(lens.max() // snap_interval)
        nsnap = int(sum(min(L // snap_interval, max_snaps) for L in lens))
        base = c.num_slots
        snaps = (base + torch.arange(c.num_reqs * max_snaps, dtype=torch.int32)).reshape(
            c.num_reqs, max_snaps).to(dev)
        extra = c.num_reqs * max_snaps
        pool0 = torch.cat([c.conv_pool, torch.zeros((extra,) + tuple(c.conv_pool.shape[1:]),
                                                    dtype=c.conv_pool.dtype)]).to(dev)
        state0 = torch.cat([c.state_pool, torch.zeros((extra,) + tuple(c.state_pool.shape[1:]),
                                                      dtype=c.state_pool.dtype)]).to(dev)
    else:
        pool0, state0 = c.conv_pool.to(dev), c.state_pool.to(dev)
    pool, state = pool0.clone(), state0.clone()
    qsl, slots, hinit = c.qsl.to(dev), c.slot_ids.to(dev), c.has_initial.to(dev)
    a, b, z, gamma = c.a.to(dev), c.b.to(dev), c.z.to(dev), c.gamma.to(dev)
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gdn.gdn_prefill_fused_workspace_bytes(d, T, c.num_reqs), dtype=torch.uint8,
                     device=dev)
    sh = stream.cuda_stream
    # every step (re-seed copies, then the timed call) is enqueued before the one
    # synchronisation: the events time the call's kernels, not the host launching
    # them onto an idle GPU
    evs = []
    for it in range(steps + 1):
        pool.copy_(pool0)
        state.copy_(state0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gdn.gdn_prefill_fused(d, x, z, a, b, conv_w, gamma, pool, state, qsl, slots, hinit, y, ws,
                              l2_eps=L2_EPS, norm_eps=NORM_EPS, snap_slot_ids=snaps,
                              snap_interval=snap_interval, stream=sh)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    times = [e0.elapsed_time(e1) for e0, e1 in evs[1:]]  # the first step is warm-up
    ms = float(np.median(times))
    if snap_interval:
        return {"snap_interval": snap_interval, "snapshots": nsnap, "ms_per_step": round(ms, 4),
                "tokens_per_s": round(T / (ms * 1e-3), 1)}
    flops = prefill_flops(d, T)
    nbytes = fused_prefill_bytes(d, T, c.num_reqs, int(c.has_initial.sum()))
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the binding resource is the one whose peak needs longer for this work
    hbm_bound = nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (BF16_PEAK_TFLOPS * 1e12)
    # the launches of the step, as its counter summary lists them
    roof = {"kernel": "prefill step (gdn_prefill_fused: " + (
        ", ".join(k.split("<")[0] for k in cnt_kernels(name)) if name and cnt_kernels(name) else
        "prep, chain, gated norm") + ")"}
    if hbm_bound:
        roof.update(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        roof.update(bound="mfma", achieved=round(tflops, 2), peak=BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(tflops / BF16_PEAK_TFLOPS, 4))
    cnt = step_counters(name) if name else None
    roof.update(bytes_per_launch=nbytes, flops_per_launch=flops,
                traffic=int(cnt["hbm_bytes_per_step"]) if cnt else None,
                mfma_tflops=round(tflops, 2),
                mfma_util_algorithmic=round(tflops / BF16_PEAK_TFLOPS, 4))
    if cnt:
        # from the counters: the MFMA work the step issues (bf16x3: three products
        # per algorithmic one) over the step time, and the chain kernel's MFMA-busy
        # share of its own cycles
        issued = cnt["mfma_bf16_flops_issued_per_step"] / (ms * 1e-3) / 1e12
        roof.update(traffic_per_token=int(cnt["hbm_bytes_per_token"]),
                    mfma_issued_tflops=round(issued, 1),
                    mfma_issued_util=round(issued / BF16_PEAK_TFLOPS, 4),
                    chain_mfma_busy=cnt["chain_mfma_busy"],
                    counters=f"profiles/{name}_counters.txt")
    return {
        "roofline": roof,
        "tokens": T,
        "requests": c.num_reqs,
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
    }


def spec_bytes(d, R, n, act_bytes=2, y_bytes=2):
    """Algorithmic HBM bytes of one gdn_spec_verify launch over R requests of n
    tokens: each request's state read once and written once per token; its conv
    history read once and written once per token; every token's conv inputs, z
    and gates read once and its y written once (1,037,877,248 B at 64 x 4, full
    shapes, bf16 activations)."""
    Hv, D = d.num_v_heads, d.head_dim_v
    C = 2 * d.num_k_heads * d.head_dim_k + Hv * D
    state = R * (1 + n) * Hv * D * d.head_dim_k * 4
    hist = R * (1 + n) * C * (d.conv_taps - 1) * act_bytes
    tok = R * n * (C * act_bytes + Hv * D * act_bytes + 2 * Hv * act_bytes + Hv * D * y_bytes)
    return state, state + hist + tok


def bench_spec(steps, warmup, dev, stream, torch, gdn):
    """gdn_spec_verify on 64 requests x 4 tokens (the last accepted token and 3
    drafts) at full shapes: K back-to-back launches between one event pair, three
    pools used in turn so that no state is still in the memory-side cache."""
    from hybrid_linear_attention_amd.workloads import spec_verify_r64

    c = spec_verify_r64()
    d = c.dims
    R, T = c.num_reqs, c.num_tokens
    n = T // R
    n_rot = 3
    pools = [c.conv_pool.to(dev) for _ in range(n_rot)]
    states = [c.state_pool.to(dev) for _ in range(n_rot)]
    x, z, a, b = c.x_qkv.to(dev), c.z.to(dev), c.a.to(dev), c.b.to(dev)
    conv_w, gamma = c.conv_w.to(dev), c.gamma.to(dev)
    qsl, slots, spec = c.qsl.to(dev), c.slot_ids.to(dev), c.meta["spec_slots"].to(dev)
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=torch.bfloat16, device=dev)
    sh = stream.cuda_stream
    it = [0]

    def step():
        i = it[0] % n_rot
        it[0] += 1
        gdn.gdn_spec_verify(d, x, z, a, b, conv_w, gamma, pools[i], states[i], qsl, slots, spec,
                            y, l2_eps=L2_EPS, norm_eps=NORM_EPS, stream=sh)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    gpu = e0.elapsed_time(e1) / steps
    state_b, nbytes = spec_bytes(d, R, n)
    achieved = nbytes / (gpu * 1e-3) / 1e9
    del pools, states
    return {
        "workload": f"spec_verify_r64: {R} requests x {n} tokens (1 accepted + {n - 1} drafts), "
                    "16/48 heads, d = 128, state and history kept after every token",
        "ms_per_step": round(wall, 4),
        "gpu_ms_per_step": round(gpu, 4),
        "tokens_per_s": round(T / (wall * 1e-3), 1),
        "state_gbs": round(state_b / (wall * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "spec_verify_kernel (gdn_spec_verify)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
                     "traffic": measured_traffic("spec_verify_kernel", "spec_verify.hip")},
    }


def gqa_bytes(c, act_bytes=2, y_bytes=2):
    """Algorithmic HBM bytes of one gqa_decode_paged call: every cached position
    of every request read once per key/value head as K and V (the new token's
    included), the new token's q, gate, k and v read once, its rotated k and v
    written into the cache once, y written once."""
    d = c.dims
    R, Hq, Hkv, D = c.num_reqs, d.num_q_heads, d.num_kv_heads, d.head_dim
    eb = c.k_cache.element_size()   # 2 (bf16) or 1 (e4m3 codes)
    kv = int(c.context_lens.sum()) * Hkv * D * eb * 2
    tok = R * (2 * Hq * D + 2 * Hkv * D) * act_bytes + R * 2 * Hkv * D * eb + R * Hq * D * y_bytes
    return kv, kv + tok


def bench_gqa(steps, warmup, dev, stream, torch, gqa, fp8=False):
    """gqa_decode_paged on 64 requests with 1024-3072 cached positions (pages of
    16), bf16 or e4m3 K/V: K back-to-back calls between one event pair, two
    cache copies used in turn so that no K/V is still in the memory-side cache
    from the call before."""
    from hybrid_linear_attention_amd.workloads import gqa_decode_r64, gqa_decode_r64_fp8

    c = gqa_decode_r64_fp8() if fp8 else gqa_decode_r64()
    d = c.dims
    R = c.num_reqs
    n_rot = 2
    kcs = [c.k_cache.to(dev) for _ in range(n_rot)]
    vcs = [c.v_cache.to(dev) for _ in range(n_rot)]
    q, gate, k, v = c.q.to(dev), c.gate.to(dev), c.k.to(dev), c.v.to(dev)
    bt, lens = c.block_tables.to(dev), c.context_lens.to(dev)
    y = torch.empty((R, d.num_q_heads * d.head_dim), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(d, R, c.max_context_len), dtype=torch.uint8,
                     device=dev)
    sh = stream.cuda_stream
    it = [0]

    def step():
        i = it[0] % n_rot
        it[0] += 1
        gqa.gqa_decode_paged(d, q, gate, k, v, kcs[i], vcs[i], bt, lens, c.page_size,
                             c.max_context_len, y, ws, rope_theta=c.rope_theta, k_scale=c.k_scale,
                             v_scale=c.v_scale, stream=sh)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    gpu = e0.elapsed_time(e1) / steps
    kv_b, nbytes = gqa_bytes(c)
    achieved = nbytes / (gpu * 1e-3) / 1e9
    ctx = int(c.context_lens.sum())
    del kcs, vcs
    return {
        "workload": f"gqa_decode_r64: {R} requests, {ctx} cached positions "
                    f"({int(c.context_lens.min())}-{int(c.context_lens.max())} each), pages of "
                    f"{c.page_size}, 24 query / 4 kv heads x 256, RoPE on 64 dims, "
                    + ("fp8 e4m3 K/V (scales 1)" if fp8 else "bf16 K/V"),
        "ms_per_step": round(wall, 4),
        "gpu_ms_per_step": round(gpu, 4),
        "tokens_per_s": round(R / (wall * 1e-3), 1),
        "kv_gbs": round(kv_b / (gpu * 1e-3) / 1e9, 1),
        # call level (two launches between the events); the counters are the
        # attention kernel's alone, which moves all but ~3 MB of the call's bytes
        # (the combine's partials and y are not in `traffic`)
        "roofline": {"kernel": "gqa_decode_paged (attn_split with RoPE and append, combine)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
                     "traffic": measured_traffic(
                         "gqa_attn_split_kernel_fp8" if fp8 else "gqa_attn_split_kernel", "gqa_decode.hip"),
                     "traffic_kernel": "gqa_attn_split_kernel",
                     "attn_split_kernel_kv_bytes": kv_b},
    }


def hbm_reference(torch, dev, mib=1024, reps=10):
    """What plain torch kernels reach on this machine beside the 8 TB/s peak: a
    device-to-device copy (reads and writes `mib` MiB) and a sum (reads them)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    out = {}
    for name, fn, nbytes in (("torch_copy_gbs", lambda: dst.copy_(src), 2 * n * 4),
                             ("torch_sum_read_gbs", lambda: src.sum(), n * 4)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    out["bytes"] = mib * (1 << 20)
    return out


def cpu_baseline(case, seconds):
    """The fp64 oracle (conv1d_update -> decode_step -> gated_norm) on the same
    decode workload, repeated until ~`seconds` of CPU time have passed."""
    import oracle
    import numpy as np

    d = case.dims

    def f64(t):
        return t.double().numpy()

    x, w, hist = f64(case.x_qkv), f64(case.conv_w), f64(case.conv_pool)
    st = f64(case.state_pool)
    a, b, z, g = f64(case.a), f64(case.b), f64(case.z), f64(case.gamma)
    qsl, slots, hi = case.qsl.numpy(), case.slot_ids.numpy(), case.has_initial.numpy()
    def sample(secs):
        nonlocal hist, st
        reps = 0
        t0 = time.perf_counter()
        while True:
            qq, kk, vv, hist = oracle.conv1d_update(x, w, hist, qsl, slots, hi, d.num_k_heads,
                                                    d.num_v_heads, d.head_dim_k, d.head_dim_v, L2_EPS)
            o, st = oracle.decode_step(qq, kk, vv, a, b, st, slots)
            oracle.gated_norm(o, z, g, NORM_EPS)
            reps += 1
            el = time.perf_counter() - t0
            if el >= secs:
                return reps, el

    threads = oracle.num_threads()
    reps, el = sample(seconds)
    oracle.set_num_threads(1)               # the same step on one thread, a shorter sample
    reps1, el1 = sample(max(2.0, seconds / 4))
    oracle.set_num_threads(threads)
    state_bytes = 2 * case.num_reqs * d.num_v_heads * d.head_dim_k * d.head_dim_v * 4
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": round(state_bytes * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{reps} full decode steps of the same 64-request workload "
                  f"(conv + recurrence + gated norm, fp64) in {el:.1f} s; "
                  f"state bytes counted as fp32, as on the GPU",
        "ms_per_step": round(el * 1e3 / reps, 2),
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model,
        "one_thread": {"value": round(state_bytes * reps1 / el1 / 1e9, 4), "unit": "GB/s",
                       "ms_per_step": round(el1 * 1e3 / reps1, 2), "steps": reps1},
    }


def _cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return model


def _sub_batch(c, take):
    """Rows of the first take[r] tokens of every request, with their qsl."""
    import numpy as np
    qsl = c.qsl.numpy()
    rows, lens = [], []
    for r in range(c.num_reqs):
        n = int(min(take[r], qsl[r + 1] - qsl[r]))
        rows.append(np.arange(qsl[r], qsl[r] + n))
        lens.append(n)
    return np.concatenate(rows), np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _oracle_core(c, rows, sub_qsl):
    """conv1d_update -> gated_delta_rule -> gated_norm, fp64, on the given rows
    (the whole step of gdn_prefill_fused); returns seconds."""
    import oracle
    d = c.dims
    slots, hi = c.slot_ids.numpy(), c.has_initial.numpy()
    x = c.x_qkv[rows].double().numpy()
    a, b = c.a[rows].double().numpy(), c.b[rows].double().numpy()
    z = c.z[rows].double().numpy()
    hist, st = c.conv_pool.double().numpy(), c.state_pool.double().numpy()
    w, g = c.conv_w.double().numpy(), c.gamma.double().numpy()
    t0 = time.perf_counter()
    q, k, v, _ = oracle.conv1d_update(x, w, hist, sub_qsl, slots, hi, d.num_k_heads, d.num_v_heads,
                                      d.head_dim_k, d.head_dim_v, L2_EPS)
    o, _ = oracle.gated_delta_rule(q, k, v, a, b, st, sub_qsl, slots, hi)
    oracle.gated_norm(o, z, g, NORM_EPS)
    return time.perf_counter() - t0


def cpu_prefill_baseline(c, per_req, per_req_one):
    """The fp64 oracle of one prefill step (conv update, recurrence, gated norm)
    on a bounded sample of the same workload: every request cut to its first
    per_req tokens, all heads, on all the host threads; and every request cut to
    per_req_one tokens on one thread.  Tokens/s over the sample."""
    import oracle
    rows, sq = _sub_batch(c, [per_req] * c.num_reqs)
    el = _oracle_core(c, rows, sq)
    rows1, sq1 = _sub_batch(c, [per_req_one] * c.num_reqs)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    el1 = _oracle_core(c, rows1, sq1)
    oracle.set_num_threads(threads)
    return {"value": round(len(rows) / el, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} tokens (each of the {c.num_reqs} requests cut to its first "
                      f"{per_req}), all 48 heads, conv + recurrence + gated norm in fp64: {el:.2f} s",
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_info(),
            "one_thread": {"value": round(len(rows1) / el1, 1), "unit": "tokens/s",
                           "sample": f"{len(rows1)} tokens (first {per_req_one} of each request): "
                                     f"{el1:.2f} s"}}


def cpu_layer_baseline(n_prefill_tokens=2048, n_decode=64):
    """The fp64 oracle of the layer block (RMSNorm, in-projection by numpy fp64
    matmul, conv, recurrence, gated norm, out-projection + residual) on a
    sub-batch of the mixed workload: the first prefill request (its first
    n_prefill_tokens tokens) and the first n_decode decode requests, per stage."""
    import numpy as np
    import oracle
    from hybrid_linear_attention_amd.workloads import layer_mixed
    case = layer_mixed()
    core = case.core
    d = core.dims
    qsl = core.qsl.numpy()
    reqs = [0] + list(range(case.num_prefill, case.num_prefill + n_decode))
    take = {0: n_prefill_tokens}
    rows = np.concatenate([np.arange(qsl[r], qsl[r] + min(take.get(r, 1), qsl[r + 1] - qsl[r]))
                           for r in reqs])
    lens = [min(take.get(r, 1), int(qsl[r + 1] - qsl[r])) for r in reqs]
    sq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = core.slot_ids.numpy()[reqs]
    hi = core.has_initial.numpy()[reqs]
    X = case.X[torch_rows(rows)].double().numpy()
    W_in = np.concatenate([case.W_qkvz.double().numpy(), case.W_ba.double().numpy()], axis=1)
    W_o = case.W_o.double().numpy()
    Hk, Hv, D = d.num_k_heads, d.num_v_heads, d.head_dim_k
    cq = 2 * Hk * D + Hv * D
    T = len(rows)
    st = {}
    t = time.perf_counter()
    U = oracle.rmsnorm(X, case.gamma_in.double().numpy(), NORM_EPS)
    st["rmsnorm"] = time.perf_counter() - t
    t = time.perf_counter()
    P = oracle.linear(U, W_in)
    st["in_proj"] = time.perf_counter() - t
    t = time.perf_counter()
    q, k, v, _ = oracle.conv1d_update(P[:, :cq], core.conv_w.double().numpy(),
                                      core.conv_pool.double().numpy()[slots], sq,
                                      np.arange(len(reqs), dtype=np.int32), hi, Hk, Hv, D, D, L2_EPS)
    o, _ = oracle.gated_delta_rule(q, k, v, P[:, cq + Hv * D + Hv:], P[:, cq + Hv * D:cq + Hv * D + Hv],
                                   core.state_pool.double().numpy()[slots], sq,
                                   np.arange(len(reqs), dtype=np.int32), hi)
    y = oracle.gated_norm(o, P[:, cq:cq + Hv * D].reshape(T, Hv, D), core.gamma.double().numpy(),
                          NORM_EPS)
    st["core"] = time.perf_counter() - t
    t = time.perf_counter()
    oracle.residual_add(X, oracle.linear(y, W_o))
    st["out_proj"] = time.perf_counter() - t
    total = sum(st.values())
    return {"value": round(T / total, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{T} tokens: the first {n_prefill_tokens} of prefill request 0 and {n_decode} "
                      f"decode requests, the whole layer block in fp64 (numpy BLAS for the "
                      f"projections): {total:.2f} s",
            "stage_s": {k_: round(v_, 3) for k_, v_ in st.items()},
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_info()}


def torch_rows(rows):
    import torch
    return torch.from_numpy(rows)


if __name__ == "__main__":
    main()
