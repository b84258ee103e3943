"""Training-step throughput of libgptstep on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload d20]
                    [--precision bf16|fp8] [--normuon] [--no-cpu-baseline]

One step = gpt_step_fwd + gpt_step_bwd + muon_update on the three groups of
block matrices (the q/k/v/o matrices, the MLP input matrices, the MLP output
matrices) + adamw_update on the embedding and the head, on synthetic inputs
already resident in HBM: uniform token ids and
N(0, 1/fan_in) weights from the seeded generators.  W untimed warm-up steps,
then K timed steps between two synchronised events on the launch stream.
Prints one JSON line.

MFU counts algorithmic FLOPs only: 6 (12 L d^2 + V d) per token for the
matrix products, 6 L d T per token for the causal half of attention, plus
5 Newton-Schulz iterations of (4 l s^2 + 2 s^3) per block matrix; recomputed
scores and logits are not counted.  Peak: MI355X dense bf16 MFMA,
2.5166 PFLOP/s.  Also reported: mfu_model (forward + backward time only),
mfu_palm (the PaLM convention: 6 (12 L d^2 + V d) + 12 L d T per token, the
whole attention square, over the step time), and the same MFU against the
matrix-core rate an MFMA-only probe sustains in the same run
(mfu_vs_achievable_peak).

The default bf16 run also times the fp8 step (--precision fp8) right after,
on the same resident token ids and the same initial weights and optimizer
state: fp8_ms_per_step, fp8_speedup = bf16 / fp8 step time, and the fp8 MFU
against the mixed peak (block products at the fp8 peak, the rest at bf16).
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2516.6e12   # dense MFMA FLOP/s
PEAK_FP8 = 5033.2e12
NS5 = [(15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)] * 5
METRIC = "training tokens/sec + MFU (% of MFMA peak), depth-20 GPT, 1 MI355X"


class Model:
    """Shapes of one configuration: depth-derived widths, the key/value head
    count and the per-layer attention windows."""

    def __init__(self, depth, V, T, B, n_kv_head=0, window=0, pattern=""):
        self.L, self.V, self.T, self.B = depth, V, T, B
        self.d = 64 * depth
        self.H = self.d // 128
        self.Hkv = n_kv_head or self.H
        self.dkv = 128 * self.Hkv
        self.hid = 4 * self.d
        self.N = B * T
        self.n_kv_head, self.window, self.pattern = n_kv_head, window, pattern
        # left window of each layer (None: full causal); pattern letters repeat over the depth
        self.windows = [window if (window > 0 and pattern and pattern[l % len(pattern)] == "S") else None
                        for l in range(depth)]

    def pairs(self, w):
        """Query-key pairs of one sequence and head, the diagonal counted half
        (T^2/2 for a full causal layer)."""
        T = self.T
        if w is None or w >= T - 1:
            return T * T / 2.0
        i = np.arange(T)
        return float(np.minimum(i + 1, w + 1).sum()) - T / 2.0

    def block_mats(self, offs):
        """(offset, rows, cols) of every block matrix in packed order."""
        L, d, dkv, hid = self.L, self.d, self.dkv, self.hid
        mats = []
        for l in range(L):
            q, k, v, o = offs[1 + 4 * l: 5 + 4 * l]
            mats += [(q, d, d), (k, dkv, d), (v, dkv, d), (o, d, d)]
        mats += [(offs[1 + 4 * L + l], hid, d) for l in range(L)]
        mats += [(offs[1 + 5 * L + l], d, hid) for l in range(L)]
        return mats

    def block_shapes(self):
        """(rows, cols) of every block matrix (offsets not needed)."""
        d, dkv, hid = self.d, self.dkv, self.hid
        return [(d, d), (dkv, d), (dkv, d), (d, d)] * self.L + [(hid, d)] * self.L + [(d, hid)] * self.L

    def attn_flops(self):
        """Algorithmic attention FLOPs of one forward over all layers (QK^T and
        PV over the visible pairs)."""
        return sum(2.0 * self.B * self.H * self.pairs(w) * 128 * 2 for w in self.windows)


def alg_flops(m):
    """(model FLOPs of one forward+backward, Newton-Schulz FLOPs of one
    optimizer step)."""
    d, dkv, N = m.d, m.dkv, m.N
    per_layer = d * (d + 2 * dkv) + d * d + 8 * d * d
    f_model = 6 * (m.L * per_layer + m.V * d) * N + 3 * m.attn_flops()
    f_ns = 0
    for rows, cols in m.block_shapes():
        l, s_ = max(rows, cols), min(rows, cols)
        f_ns += 5 * (4 * l * s_ * s_ + 2 * s_ ** 3)
    return f_model, f_ns


def palm_flops(m):
    """Model FLOPs of one forward+backward in the PaLM convention: 6 per
    parameter-token for the matrices (embedding included, as above) and
    12 L d T per token for attention over the whole T x T square."""
    d, dkv, N = m.d, m.dkv, m.N
    per_layer = d * (d + 2 * dkv) + d * d + 8 * d * d
    return 6.0 * (m.L * per_layer + m.V * d) * N + 12.0 * m.L * d * m.T * N


def muon_runs(mats):
    """Runs of adjacent same-shape matrices, each one muon_update call:
    (start, count, rows, cols)."""
    runs = []
    for off, rows, cols in mats:
        if runs:
            st, cnt, r, c = runs[-1]
            if (r, c) == (rows, cols) and st + cnt * r * c == off:
                runs[-1] = (st, cnt + 1, r, c)
                continue
        runs.append((off, 1, rows, cols))
    return runs


def kernel_flops(name, m):
    """Algorithmic FLOPs of one launch of a kernel category, averaged over the
    layers (None: not a contraction)."""
    d, dkv, hid, N = m.d, m.dkv, m.hid, m.N
    attn = m.attn_flops() / m.L
    table = {
        "gemm_qkv_rope_fwd": 2.0 * N * (d + 2 * dkv) * d, "gemm_o_fwd": 2.0 * N * d * d,
        "gemm_fc_relu2_fwd": 2.0 * N * hid * d, "gemm_proj_fwd": 2.0 * N * d * hid,
        "gemm_ce_fwd": 2.0 * N * m.V * d, "attn_fwd": attn,
        # backward: dV, dP, dK in the dK/dV kernel, dQ in the dQ kernel (recomputed
        # scores and the dQ kernel's second dP are not counted)
        "attn_bwd_dkdv": 1.5 * attn, "attn_bwd_dq": 0.5 * attn,
        "gemm_proj_dgrad": 2.0 * N * d * hid, "gemm_proj_wgrad": 2.0 * N * d * hid,
        "gemm_fc_dgrad": 2.0 * N * d * hid, "gemm_fc_wgrad": 2.0 * N * d * hid,
        "gemm_o_dgrad": 2.0 * N * d * d, "gemm_o_wgrad": 2.0 * N * d * d,
        "gemm_qkv_dgrad": 2.0 * N * (d + 2 * dkv) * d, "gemm_qkv_wgrad": 2.0 * N * (d + 2 * dkv) * d,
    }
    return table.get(name)


BLOCK_GEMMS = {"gemm_qkv_rope_fwd", "gemm_o_fwd", "gemm_fc_relu2_fwd", "gemm_proj_fwd", "gemm_proj_dgrad",
               "gemm_proj_wgrad", "gemm_fc_dgrad", "gemm_fc_wgrad", "gemm_o_dgrad", "gemm_o_wgrad",
               "gemm_qkv_dgrad", "gemm_qkv_wgrad"}


def block_gemm_flops(m):
    """FLOPs of the four block products per layer, forward and backward."""
    d, dkv = m.d, m.dkv
    return 6.0 * m.L * (d * (d + 2 * dkv) + 9 * d * d) * m.N


def measured_traffic(category):
    """HBM bytes per launch of a kernel category from the committed rocprofv3
    counter summary (profiles/traffic.json), or None when there is none or the
    kernel's source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(category)
        if rec is None:
            return None
        sha = hashlib.sha256(open(os.path.join(ROOT, rec["source"]), "rb").read()).hexdigest()
        return rec["hbm_bytes_per_launch"] if sha == rec["source_sha256"] else None
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(wl, m, seed_ids, seed_w):
    """The oracle (numpy, as it stands) on a bounded sample of the workload:
    one sequence's forward+backward in float32 and one Newton-Schulz per block
    matrix shape (float64), scaled to a full step."""
    from gpt_transformer_step_amd import inputs
    from oracle import model as om
    from oracle import muon as omu
    from oracle import precision
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    dims = inputs.Dims.from_depth(m.L, m.V, m.n_kv_head)
    cfg = om.Config.from_depth(m.L, m.V, m.n_kv_head, m.window, m.pattern or "L")
    master = inputs.master_weights(dims, seed_w)
    P = {k: v for k, v in inputs.unpack(dims, precision.round_bf16(master)).items()}
    ids = inputs.token_ids(m.B, m.T, m.V, seed_ids)[:1]
    t0 = time.perf_counter()
    om.forward_backward(P, ids, cfg, dtype=np.float32)
    t_seq = time.perf_counter() - t0
    t_ns = 0.0
    g = np.random.default_rng(0)
    counts = {}
    for shp in m.block_shapes():
        counts[shp] = counts.get(shp, 0) + 1
    for (rows, cols), count in counts.items():
        G = g.standard_normal((rows, cols)).astype(np.float32)
        t0 = time.perf_counter()
        omu.newton_schulz(G, NS5)
        t_ns += count * (time.perf_counter() - t0)
    step_s = m.B * t_seq + t_ns
    return {"value": m.B * m.T / step_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"{wl}: forward+backward of 1 of {m.B} sequences (float32, {t_seq:.1f} s) and one "
                       f"Newton-Schulz per block-matrix shape (float64); scaled to a full step "
                       f"({step_s:.0f} s)")}


def ns_standalone(args):
    """Newton-Schulz alone: normalisation, 5 iterations of A = X^T X,
    B = b A + c A A, X = a X + X B, and the copy-out, on one matrix."""
    import torch
    from gpt_transformer_step_amd import binding as Bd
    from gpt_transformer_step_amd import inputs
    dev = torch.device("cuda:0")
    res = {}
    for rows, cols in ((1664, 6656), (1664, 1664)):
        G = torch.from_numpy(inputs.normal_matrix(rows, cols, inputs.SEED_NS)[0]).to(dev)
        O = torch.empty_like(G)
        ws = torch.empty(Bd.muon_workspace_size(1, rows, cols), dtype=torch.uint8, device=dev)
        for _ in range(max(1, args.warmup)):
            Bd.muon_update(G, NS5, ws, O_out=O)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            Bd.muon_update(G, NS5, ws, O_out=O)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        s_, l_ = min(rows, cols), max(rows, cols)
        flops = 5 * (4 * l_ * s_ * s_ + 2 * s_ ** 3)
        res[f"{rows}x{cols}"] = {"ms": ms, "tflops": flops / ms / 1e9, "frac": flops / (ms * 1e-3) / PEAK_BF16,
                                 "flops": flops}
    tot_ms = sum(r["ms"] for r in res.values())
    tot_fl = sum(r["flops"] for r in res.values())
    print(json.dumps({"metric": "Newton-Schulz standalone, 5 iterations (TFLOP/s)", "value": tot_fl / tot_ms / 1e9,
                      "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "higher_is_better": True, "dtype": "bf16", "data": "synthetic: N(0,1) fp32 (seeded PCG64)",
                      "config": {"workload": "ns-standalone", "shapes": list(res)}, "per_shape": res}), flush=True)


def achievable_peak():
    """Dense bf16 matrix-core rate an MFMA-only probe sustains (FLOP/s): one
    workgroup of 4 waves per SIMD slot pair on every CU, timed with events."""
    import torch
    from gpt_transformer_step_amd import binding as Bd
    blocks, iters = 256 * 8, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    Bd.probe_mfma(0, blocks, 64, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = Bd.probe_mfma(0, blocks, iters, out)
    e1.record()
    torch.cuda.synchronize()
    return flops / (e0.elapsed_time(e1) * 1e-3)


def run_precision(args, m, prec, master0, ids, dims, profile):
    """Warm-up, (optionally) the per-category pass, then the timed steps of one
    precision, from the initial weights master0 and zero optimizer state."""
    import torch
    from gpt_transformer_step_amd import binding as Bd
    depth, V, T, B = m.L, m.V, m.T, m.B
    dev = master0.device
    sh = Bd.shape(depth, V, T, B, prec, n_kv_head=args.n_kv_head, window=args.window, pattern=args.pattern,
                  features=args.features)
    n = Bd.param_count(sh)
    assert n == master0.numel()
    master = master0.clone()
    bf16 = torch.empty(n, dtype=torch.bfloat16, device=dev)
    Bd.cast_bf16(master, bf16)
    grad = torch.zeros(n, dtype=torch.float32, device=dev)
    ws = torch.empty(Bd.workspace_size(sh), dtype=torch.uint8, device=dev)
    params = Bd.make_params(master, bf16, grad)
    loss = torch.zeros(1, dtype=torch.float32, device=dev)
    offs = Bd.param_layout(sh)
    # one muon_update per run of adjacent same-shape block matrices: the three
    # groups (q/k/v/o, MLP in, MLP out) when every head has its own key/value
    # head; with grouped heads wq/wo and wk/wv pairs differ in shape
    groups = []
    for st, count, rows, cols in muon_runs(m.block_mats(offs)):
        size = count * rows * cols
        groups.append(dict(count=count, rows=rows, cols=cols, start=st,
                           M=torch.zeros(size, dtype=torch.float32, device=dev),
                           V=torch.zeros(count * rows, dtype=torch.float32, device=dev) if args.normuon else None,
                           ws=torch.empty(Bd.muon_workspace_size(count, rows, cols), dtype=torch.uint8,
                                          device=dev)))

    # AdamW for the embedding and the head (the two [V, d] tables) and, with the
    # record-model features, for everything after the head (value-embedding
    # tables, their gates and the scalars)
    d = m.d
    lm = offs[1 + 6 * depth]
    ranges = [(offs[0], V * d), (lm, V * d)]
    if args.features:
        ranges.append((lm + V * d, n - (lm + V * d)))
    adam = []
    for start, size in ranges:
        adam.append(dict(start=start, size=size, M=torch.zeros(size, dtype=torch.float32, device=dev),
                         V=torch.zeros(size, dtype=torch.float32, device=dev)))
    step_count = [0]

    def step():
        Bd.step_fwd(sh, params, ids, loss, ws)
        Bd.step_bwd(sh, params, ids, ws)
        step_count[0] += 1
        for ad in adam:
            st, size = ad["start"], ad["size"]
            Bd.adamw_update(master[st:st + size], grad[st:st + size], ad["M"], ad["V"], step_count[0], lr=0.004,
                            beta1=0.8, beta2=0.95, eps=1e-10, weight_decay=0.0, W_bf16=bf16[st:st + size])
        for gr in groups:
            st, size = gr["start"], gr["count"] * gr["rows"] * gr["cols"]
            view = (gr["count"], gr["rows"], gr["cols"])
            if args.normuon:
                Bd.normuon_update(grad[st:st + size].view(view), NS5, gr["ws"], gr["V"],
                                  W=master[st:st + size].view(view), W_bf16=bf16[st:st + size].view(view),
                                  M=gr["M"], lr=0.02, momentum=0.95, weight_decay=0.0, beta2=0.95, eps=1e-8)
            else:
                Bd.muon_update(grad[st:st + size].view(view), NS5, gr["ws"], W=master[st:st + size].view(view),
                               W_bf16=bf16[st:st + size].view(view), M=gr["M"], lr=0.02, momentum=0.95,
                               weight_decay=0.0)

    tag = "fp8" if prec == Bd.PREC_FP8 else "bf16"
    print(f"bench: inputs resident ({args.workload}, {tag}); warm-up", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    first_loss = float(loss.item())
    out = dict(first_loss=first_loss, breakdown=None, dom=None, dom_ms=None, dom_cnt=None)
    if profile:
        print("bench: warm-up done; per-category pass", file=sys.stderr, flush=True)
        # per-kernel-category pass (untimed) to find the dominant kernel
        cats = Bd.profile_categories()
        Bd.profile_reset()
        Bd.profile_enable((1 << len(cats)) - 1)
        step()
        torch.cuda.synchronize()
        breakdown = {}
        for i, c in enumerate(cats):
            t, cnt = Bd.profile_read(i)
            if cnt:
                breakdown[c] = (t, cnt)
        Bd.profile_enable(0)
        Bd.profile_reset()
        contractions = {c: v for c, v in breakdown.items() if kernel_flops(c, m)}
        dom = max(contractions, key=lambda c: contractions[c][0])
        dom_idx = cats.index(dom)
        print(f"bench: dominant contraction {dom}; timed steps", file=sys.stderr, flush=True)
        # the dominant kernel bracketed by HIP events on its launch stream
        Bd.profile_enable(1 << dom_idx)
        out.update(breakdown=breakdown, dom=dom)
    # timed region: K steps between two events on the launch stream
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    out["ms"] = e0.elapsed_time(e1) / args.steps
    if profile:
        dom_ms, dom_cnt = Bd.profile_read(dom_idx)
        Bd.profile_enable(0)
        Bd.profile_reset()
        out.update(dom_ms=dom_ms, dom_cnt=dom_cnt)
    out["last_loss"] = float(loss.item())
    print(f"bench: {tag} {out['ms']:.2f} ms per step", file=sys.stderr, flush=True)
    del ws, groups, adam, grad, bf16, master
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="d20", choices=["d2", "d12", "d20", "d26"])
    ap.add_argument("--precision", default="bf16", choices=["bf16", "fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 step timed after the bf16 one")
    ap.add_argument("--normuon", action="store_true",
                    help="NorMuon per-neuron rescale after Newton-Schulz (normuon_update)")
    ap.add_argument("--n-kv-head", type=int, default=0, help="key/value heads (0: one per query head)")
    ap.add_argument("--window", type=int, default=0, help="left window of the short ('S') layers")
    ap.add_argument("--pattern", default="", help="layer pattern of S (windowed) / L (full) letters, e.g. SSSL")
    ap.add_argument("--features", default="",
                    help="record-model features: v (value embeddings), s (smear), r (residual scalars), b (backout)")
    ap.add_argument("--breakdown", action="store_true", help="print per-kernel times to stderr")
    ap.add_argument("--ns-standalone", action="store_true",
                    help="only time Newton-Schulz (5 iterations, muon_update with no momentum and no apply) on "
                         "N(0,1) 1664x6656 and 1664x1664 matrices and print one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES three times and exit (the reference "
                         "for scaling the HBM byte counters of a profiler)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "copies": 3}), flush=True)
        return
    if args.ns_standalone:
        ns_standalone(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the step runs on a "
              f"single MI355X with no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    from gpt_transformer_step_amd import binding as Bd
    from gpt_transformer_step_amd import inputs

    wl = inputs.WORKLOADS[args.workload]
    depth, T, B = wl["depth"], wl["seq_len"], wl["batch"]
    V = 32768
    m = Model(depth, V, T, B, args.n_kv_head, args.window, args.pattern)
    d, H = m.d, m.H
    prec = Bd.PREC_FP8 if args.precision == "fp8" else Bd.PREC_BF16
    dev = torch.device("cuda:0")
    dims = inputs.Dims.from_depth(depth, V, args.n_kv_head, features=args.features)
    master0 = torch.from_numpy(inputs.master_weights(dims, inputs.SEED_W)).to(dev)
    ids = torch.from_numpy(inputs.token_ids(B, T, V, inputs.SEED_IDS)).to(dev)
    ach_peak = achievable_peak()

    res = run_precision(args, m, prec, master0, ids, dims, profile=True)
    fp8_res = None
    if prec == Bd.PREC_BF16 and not args.no_fp8 and not args.features:
        print("bench: fp8 step on the same inputs", file=sys.stderr, flush=True)
        fp8_res = run_precision(args, m, Bd.PREC_FP8, master0, ids, dims, profile=False)
    ms, first_loss, last_loss = res["ms"], res["first_loss"], res["last_loss"]
    breakdown, dom, dom_ms, dom_cnt = res["breakdown"], res["dom"], res["dom_ms"], res["dom_cnt"]

    f_model, f_ns = alg_flops(m)
    tok = B * T
    step_s = ms / 1e3
    fwd_bwd_ms = sum(v[0] for k, v in breakdown.items()
                     if not k.startswith("ns_") and k not in ("muon_elementwise", "adamw"))
    kf = kernel_flops(dom, m)
    avg_launch_s = dom_ms / dom_cnt / 1e3
    achieved = kf / avg_launch_s / 1e12
    fp8 = prec == Bd.PREC_FP8
    peak = (PEAK_FP8 if (fp8 and dom in BLOCK_GEMMS) else PEAK_BF16) / 1e12
    # fp8: the block products run against the fp8 peak, everything else against bf16
    f_block = block_gemm_flops(m) if fp8 else 0.0
    t_ideal = f_block / PEAK_FP8 + (f_model + f_ns - f_block) / PEAK_BF16
    out = {
        "metric": METRIC,
        "value": tok / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if prec == Bd.PREC_BF16 else "fp8-e4m3/e5m2 block GEMMs, bf16 rest",
        "data": "synthetic: uniform token ids, N(0,1/fan_in) weights (seeded PCG64)",
        "config": {"workload": args.workload, "depth": depth, "d_model": d, "n_head": H,
                   "n_kv_head": m.Hkv, "window": args.window, "pattern": args.pattern or "L",
                   "features": args.features or "none", "seq_len": T,
                   "micro_batch": B, "vocab": V, "tokens_per_step": tok, "parallelism": "single GPU",
                   "optimizer": ("NorMuon" if args.normuon else "Muon") +
                                " (5 Newton-Schulz iterations) on all block matrices, AdamW on embedding and head" +
                                (" and the record-model tensors" if args.features else "")},
        "mfu": (f_model + f_ns) / step_s / PEAK_BF16,
        "mfu_vs_achievable_peak": (f_model + f_ns) / step_s / ach_peak,
        "achievable_peak_tflops": ach_peak / 1e12,
        "mfu_palm": palm_flops(m) / step_s / PEAK_BF16,
        "mfu_vs_mixed_peak": t_ideal / step_s if fp8 else None,
        "mfu_model": f_model / (fwd_bwd_ms / 1e3) / PEAK_BF16 if fwd_bwd_ms else None,
        "tflops": (f_model + f_ns) / step_s / 1e12,
        "loss": [first_loss, last_loss],
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": measured_traffic(dom),
                     "flops_per_launch": kf, "avg_launch_ms": avg_launch_s * 1e3,
                     "launches": dom_cnt},
        "breakdown_ms_per_step": {k: round(v[0], 3) for k, v in sorted(breakdown.items(), key=lambda kv: -kv[1][0])},
    }
    if fp8_res is not None:
        f_block = block_gemm_flops(m)
        t8_ideal = f_block / PEAK_FP8 + (f_model + f_ns - f_block) / PEAK_BF16
        out.update({"fp8_ms_per_step": fp8_res["ms"], "fp8_tokens_per_s": tok / (fp8_res["ms"] / 1e3),
                    "fp8_speedup": ms / fp8_res["ms"], "fp8_mfu_vs_mixed_peak": t8_ideal / (fp8_res["ms"] / 1e3),
                    "fp8_loss": [fp8_res["first_loss"], fp8_res["last_loss"]]})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, m, inputs.SEED_IDS, inputs.SEED_W)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
