"""Benchmark of the MI355X MoE decode layer: MoE-layer decode us/layer and
achieved HBM GB/s, W4A16 (NVFP4 weights, bf16 activations), batch 1 and 8.

Headline workload (value): the 47 MoE layers of the Flint-shaped model
(hidden 2048, 256 routed experts + 1 shared, sigmoid top-6, expert
intermediate 512; distinct seeded NVFP4 weights per layer, 21.4 GB resident
in HBM) run as a chained residual stream at batch 1,

    x_{l+1} = x_l + layer_l(rmsnorm_l(x_l)),

so each layer's routing depends on the previous layer's output, in one
launch per pass (moe_decode_chain_forward) replayed from a HIP graph.  One
step = one pass over the 47 layers.  A pass touches 631 MB, more than the
256 MiB last-level cache, so the weights stream from HBM every step.

value = algorithmic bytes per pass / time per pass, in GB/s: per layer the
selected experts' packed weights (codes + block scales + tensor scales), the
shared expert, the router, the norm weight, x and y; the untouched experts
are not counted.  Beside it: the same layers as independent layers on one x
(one stacked launch), as one launch per layer (plain, and chained through
the fused RMSNorm/residual entry point), batch 8, BF16 weights (W16A16), the
8,192-token prefill layer, the dense GEMVs and the other MoE shapes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, I, E, K = 2048, 512, 256, 6
NVFP4_EXPERT_BYTES = 3 * (H * I // 2 + H * I // 16 + 4)        # 1,769,484
BF16_EXPERT_BYTES = 3 * H * I * 2                               # 6,291,456
ROUTER_BYTES = E * H * 2                                        # 1,048,576
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 matrix-core peak (published)
PREFILL_T = 8192


def prefill_flop(T: int) -> float:
    """Algorithmic prefill FLOP: 7 experts per token x (gate, up, down) + router."""
    return 2.0 * T * 7 * 3 * I * H + 2.0 * T * E * H


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(record: str, layers: int | None = None) -> float | None:
    """HBM bytes per launch of a batch-1 decode kernel from a committed
    rocprofv3 counter record (profiles/<record>.json), if that kernel's
    sources are unchanged since the counters were taken and (stack) the
    record covers the same number of layers; else None."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", record + ".json")))
        if source_hash() != rec.get("source_sha256_16"):
            return None
        if layers is not None and rec.get("layers") != layers:
            return None
    except OSError:
        return None
    return float(rec["traffic_bytes_per_launch"])


def source_hash() -> str:
    """First 16 hex of SHA-256 over the single-launch decode kernels' code
    (decode_layer.h + common.h, comments and blank space removed, so comment
    edits keep it)."""
    import hashlib
    import re
    text = "".join(open(os.path.join(ROOT, "moe_decode_sigmoid_amd", "csrc", f)).read()
                   for f in ("decode_layer.h", "common.h"))
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def write_traffic_record(dec_fetch: str, dec_write: str, copy_fetch: str, copy_write: str,
                         layers: int) -> int:
    """Per-launch HBM bytes of the batch-1 decode kernels (one layer per launch,
    the stack of `layers` independent layers and the chained stack of `layers`
    layers in one launch) from counter runs of `bench.py --workload decode
    --layers <layers>`, each counter scaled by what it reads for a plain 1 GiB
    copy.  Algorithmic bytes: 7 experts per layer (batch 1 reads 6 routed
    experts and the shared one)."""
    import csv

    def mean_kib(path, kernel_part, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if kernel_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        assert vals, f"no {counter} rows for {kernel_part} in {path}"
        return sum(vals.values()) / len(vals), len(vals)

    f_cp, _ = mean_kib(copy_fetch, "copyBuffer", "FETCH_SIZE")
    w_cp, _ = mean_kib(copy_write, "copyBuffer", "WRITE_SIZE")
    gib_kib = float(1 << 20)
    fs, wsc = gib_kib / f_cp, gib_kib / w_cp
    for kname, label, record, n in [
            ("k_decode_fused<1, 0, false, false, 1, false>", "k_decode_fused<1, nvfp4>",
             "k_decode_fused_b1_traffic", 1),
            ("k_decode_stack<1, 0>", f"k_decode_stack<1, nvfp4> ({layers} layers)",
             "k_decode_stack_b1_traffic", layers),
            ("k_decode_chain<1, 0, true>", f"k_decode_chain<1, nvfp4, rmsnorm> ({layers} layers)",
             "k_decode_chain_b1_traffic", layers)]:
        f_dec, nf = mean_kib(dec_fetch, kname, "FETCH_SIZE")
        w_dec, nw = mean_kib(dec_write, kname, "WRITE_SIZE")
        rec = {"kernel": label, "source_sha256_16": source_hash(), "layers": n,
               "fetch_kib_per_launch": f_dec, "write_kib_per_launch": w_dec,
               "dispatches_sampled": [nf, nw], "copy_fetch_kib_per_gib": f_cp,
               "copy_write_kib_per_gib": w_cp, "fetch_scale": fs, "write_scale": wsc,
               "traffic_bytes_per_launch": (f_dec * fs + w_dec * wsc) * 1024,
               "algorithmic_bytes_per_launch": n * layer_bytes(7, 1, "nvfp4",
                                                               norm="chain" in record)}
        with open(os.path.join(ROOT, "profiles", record + ".json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec))
    return 0


def layer_bytes(n_experts_read: int, B: int, fmt: str, norm: bool = False) -> int:
    """Algorithmic HBM bytes of one decode layer: the experts it reads, the
    router, x in and y out (and the RMSNorm weight when the norm is fused)."""
    per = NVFP4_EXPERT_BYTES if fmt == "nvfp4" else BF16_EXPERT_BYTES
    return n_experts_read * per + ROUTER_BYTES + 2 * B * H * 2 + (2 * H if norm else 0)


# the non-expert projections of one attention block: fused q/k/v (32 query + 2 x 4
# key/value heads of 128 over hidden 2048) and the output projection
DENSE_SHAPES = {"qkv_proj": (5120, 2048), "o_proj": (2048, 4096)}


def dense_bytes(N: int, K: int, B: int) -> int:
    """HBM bytes one GEMV must move: codes + E4M3 scales + global, x in, y out."""
    return N * K // 2 + N * K // 16 + 4 + 2 * B * K + 2 * B * N


def run_dense(args, moe, testgen, torch, dev) -> dict:
    """Each projection at batch 1 and 8: one graph of `layers` launches over as
    many weight copies (so no launch finds its weights in cache), timed by HIP
    events around the replays."""
    out = {}
    for name, (N, K) in DENSE_SHAPES.items():
        codes, scales, glob = testgen.make_dense(args.seed, 0, 90 + len(out), N, K)
        c0, s0 = torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev)
        ws = [(c0.clone(), s0.clone()) for _ in range(args.layers)]
        g0 = torch.tensor([glob], dtype=torch.float32, device=dev)
        del c0, s0
        for B in (1, 8):
            x = moe.device.to_device_bf16(testgen.make_x(args.seed, B, K), dev)
            y = torch.empty((args.layers, B, N), dtype=torch.bfloat16, device=dev)
            for l, (c, sc) in enumerate(ws):
                moe.moe_nvfp4_gemv(x, c, sc, g0, y[l])
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for l, (c, sc) in enumerate(ws):
                    moe.moe_nvfp4_gemv(x, c, sc, g0, y[l])
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000 / (args.steps * args.layers)
            nb = dense_bytes(N, K, B)
            out[f"{name}_b{B}"] = dict(N=N, K=K, B=B, us_per_launch=round(us, 3),
                                       bytes_per_launch=nb, gbps=round(nb / (us * 1e-6) / 1e9, 1))
            log(f"dense {name} [{N}x{K}] B={B}: {us:.2f} us, {nb / (us * 1e-6) / 1e9:.0f} GB/s")
            del g
        del ws
    return out


# other MoE shapes of the pages (the general decode path); hidden and expert
# intermediate sizes are Flint's (the pages give none for these models)
GENERAL_SHAPES = {
    "inkling2small_384x8_mxfp8": (2048, 512, 384, 8, 0, "mxfp8"),
    "inkling_256x6_2shared_nvfp4": (2048, 512, 256, 6, 2, "nvfp4"),
    "flint_w4a4_four_over_six": (2048, 512, 256, 6, 1, "nvfp4_a4"),
}


def expert_bytes(H: int, I: int, fmt: str) -> int:
    """Bytes of one expert (gate, up, down) as the kernels read them."""
    m = H * I
    if fmt in ("nvfp4", "nvfp4_a4"):
        return 3 * (m // 2 + m // 16 + 4)
    if fmt == "mxfp8":
        return 3 * (m + m // 32)
    return 3 * 2 * m


def run_general(args, moe, testgen, torch, dev, copies: int = 16) -> dict:
    """Each shape at batch 1 and 8: one host layer, `copies` device copies (a
    pass touches more than the last-level cache), one graph of `copies`
    launches per step, HIP events around the replays."""
    out = {}
    for name, (H, I, E, K, NS, fmt) in GENERAL_SHAPES.items():
        host = testgen.make_layer(args.seed, 0, "nvfp4" if fmt == "nvfp4_a4" else fmt, H, I, E, K,
                                  n_shared=NS)
        d0 = moe.DeviceLayer.from_host(host, dev)
        del host

        def clone(dx):
            if dx is None:
                return None
            return moe.device.DeviceExperts(
                dx.fmt, dx.n, dx.w13.clone(), dx.w2.clone(),
                None if dx.w13_scale is None else dx.w13_scale.clone(),
                None if dx.w2_scale is None else dx.w2_scale.clone(),
                None if dx.glob is None else dx.glob.clone())
        ls = [d0] + [moe.device.DeviceLayer(d0.fmt, d0.router.clone(), clone(d0.routed),
                                            clone(d0.shared)) for _ in range(copies - 1)]
        S = moe.shape(moe._fmt(fmt), hidden=H, inter=I, n_experts=E, top_k=K, n_shared=NS)
        for B in (1, 8):
            x = moe.device.to_device_bf16(testgen.make_x(args.seed, B, H), dev)
            y = torch.empty((copies, B, H), dtype=torch.bfloat16, device=dev)
            ids = torch.empty((B, K), dtype=torch.int32, device=dev)
            ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, S=S), dev)
            moe.moe_decode_forward(x, ls[0].router, ls[0].routed, ls[0].shared, y[0], ws, ids,
                                   S=S)
            torch.cuda.synchronize()
            n_read = len(set(ids.cpu().numpy().ravel().tolist())) + NS
            nb = n_read * expert_bytes(H, I, fmt) + E * H * 2 + 2 * 2 * B * H
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for l, d in enumerate(ls):
                    moe.moe_decode_forward(x, d.router, d.routed, d.shared, y[l], ws, S=S)
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000 / (args.steps * copies)
            out[f"{name}_b{B}"] = dict(H=H, I=I, E=E, top_k=K, n_shared=NS, fmt=fmt, B=B,
                                       experts_read=n_read, bytes_per_call=nb,
                                       us_per_layer=round(us, 3),
                                       gbps=round(nb / (us * 1e-6) / 1e9, 1))
            log(f"general {name} B={B}: {us:.2f} us/layer, {nb / (us * 1e-6) / 1e9:.0f} GB/s")
            del g
        del ls, d0
        torch.cuda.empty_cache()
    return out


def time_graph(fn, steps: int, warmup: int, torch) -> tuple[dict, object]:
    """Capture fn in a HIP graph and time its replays on the current stream:
    mean over `steps` back-to-back replays (HIP events around them, with a
    synchronize on both sides), then p10 / median / p90 of `steps` replays
    each bracketed by its own events."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    return dict(ms=ms, p10=float(np.percentile(per, 10)), p50=float(np.median(per)),
                p90=float(np.percentile(per, 90))), g


def rate(d: dict, nbytes: int, L: int) -> dict:
    """us per layer and GB/s (algorithmic bytes) of a timing dict of passes of L layers."""
    return dict(us_per_layer=d["ms"] * 1000 / L,
                us_per_layer_p10_p50_p90=[d["p10"] * 1000 / L, d["p50"] * 1000 / L,
                                          d["p90"] * 1000 / L],
                ms_per_pass=d["ms"], bytes_per_pass=int(nbytes),
                gbps=nbytes / (d["ms"] * 1e-3) / 1e9,
                frac_of_hbm_peak=nbytes / (d["ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=47)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--no-batch8", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate host time per oracle baseline leg (0 = skip)")
    ap.add_argument("--workload", default="all",
                    choices=["all", "decode", "prefill", "dense", "general", "bf16", "copy"],
                    help="decode = the 47-layer NVFP4 stacks only; prefill = the 8192-token "
                         "layer only; dense = the NVFP4 attention-projection GEMVs only; "
                         "general = the other MoE shapes (general decode path) only; bf16 = the "
                         "W16A16 layers only; copy = a plain 1 GiB device copy (reference for "
                         "the traffic counters)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--traffic-record", nargs=4, metavar="CSV",
                    help="no GPU work: read four rocprofv3 counter_collection.csv files "
                         "(decode FETCH_SIZE, decode WRITE_SIZE, copy FETCH_SIZE, copy "
                         "WRITE_SIZE; the decode runs with the same --layers) and write "
                         "profiles/k_decode_{fused,stack,chain}_b1_traffic.json")
    args = ap.parse_args()
    if args.traffic_record:
        return write_traffic_record(*args.traffic_record, args.layers)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: this MoE decode layer runs on one GPU (tensor/expert sharding is "
              f"described in DESIGN.md but not built); --gpus {max(args.gpus, world)} is not "
              f"supported", file=sys.stderr)
        return 2

    import torch
    import moe_decode_sigmoid_amd as moe
    import testgen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = "cuda:0"
    if args.workload == "copy":
        nbytes = 1 << 30
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "copies": 3}))
        return 0
    if args.workload == "dense":
        print(json.dumps({"dense_gemv": run_dense(args, moe, testgen, torch, dev)}), flush=True)
        return 0
    if args.workload == "general":
        print(json.dumps({"general_shapes": run_general(args, moe, testgen, torch, dev)}),
              flush=True)
        return 0
    if args.workload == "bf16":
        print(json.dumps({"bf16_w16a16": run_bf16(args, moe, testgen, torch, dev)}), flush=True)
        return 0
    L = 1 if args.workload == "prefill" else args.layers

    # ---------------------------------------------------------------- weights
    t0 = time.time()
    layers = []
    host0 = None
    for l in range(L):
        hl = testgen.make_layer(args.seed, l, "nvfp4")
        layers.append(moe.DeviceLayer.from_host(hl, dev))
        if l == 0:
            host0 = hl
        del hl
        if l % 8 == 7 or l == L - 1:
            log(f"layer {l + 1}/{L} generated and resident ({time.time() - t0:.1f} s)")

    def nbytes(t):
        return 0 if t is None else t.numel() * t.element_size()
    resident = sum(nbytes(d.router) + sum(nbytes(getattr(s, f)) for s in (d.routed, d.shared)
                                          for f in ("w13", "w2", "w13_scale", "w2_scale", "glob"))
                   for d in layers)
    table = moe.layer_table(layers, dev)
    norm_w = moe.device.to_device_bf16(testgen.make_x(args.seed + 7, L), dev)   # [L, H]
    EPS = 1e-5

    def run_decode(B: int) -> dict:
        """The L layers at batch B five ways, each one HIP-graph replay per pass:
        chain (one launch, residual stream with RMSNorm), chain without the norm,
        stack (one launch, independent layers on one x), per-layer launches of
        the plain layer, per-layer launches chained through the fused entry."""
        x = moe.device.to_device_bf16(testgen.make_x(args.seed, B), dev)
        ws = moe.alloc_workspace(moe.moe_workspace_bytes(B), dev)
        out = torch.empty((L, B, H), dtype=torch.bfloat16, device=dev)
        ref = torch.empty_like(out)
        ids = torch.empty((L, B, K), dtype=torch.int32, device=dev)
        ids_r = torch.empty_like(ids)

        def chain(norm=True, with_ids=False):
            moe.moe_decode_chain_forward(x, table, out, ws, norm_w=norm_w if norm else None,
                                         eps=EPS, ids_out=ids if with_ids else None, B=B)

        def stack(with_ids=False):
            moe.moe_decode_stack_forward(x, table, out, ws, ids if with_ids else None, B=B)

        def per_layer(with_ids=False):
            for l, d in enumerate(layers):
                moe.moe_decode_forward(x, d.router, d.routed, d.shared, ref[l], ws,
                                       ids_r[l] if with_ids else None, None, B=B)

        def per_layer_chain(with_ids=False):
            cur = x
            for l, d in enumerate(layers):
                moe.moe_decode_forward_ex(cur, d.router, d.routed, d.shared, ref[l], ws,
                                          norm_w=norm_w[l], eps=EPS, residual=cur,
                                          ids_out=ids_r[l] if with_ids else None, B=B)
                cur = ref[l]

        def pass_bytes(ids_t, norm):
            h = ids_t.cpu().numpy()
            n_read = [len(set(h[l].ravel().tolist())) + 1 for l in range(L)]
            return sum(layer_bytes(n, B, "nvfp4", norm) for n in n_read), float(np.mean(n_read))

        res = {"B": B}
        # chained residual stream: the one launch and L fused per-layer launches
        chain(True, True)
        per_layer_chain(True)
        torch.cuda.synchronize()
        same_chain = bool(torch.equal(out, ref)) and bool(torch.equal(ids, ids_r))
        nb_chain, e_chain = pass_bytes(ids, True)
        t, g = time_graph(lambda: chain(True), args.steps, args.warmup, torch)
        ref.copy_(out)
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        res["chain"] = dict(rate(t, nb_chain, L), experts_read_mean=e_chain,
                            equals_per_layer_fused_calls=same_chain,
                            graph_matches_eager=bool(torch.equal(out, ref)))
        del g
        t, g = time_graph(lambda: per_layer_chain(), args.steps, args.warmup, torch)
        res["per_layer_chain"] = rate(t, nb_chain, L)
        del g
        chain(False, True)
        torch.cuda.synchronize()
        nb_c0, e_c0 = pass_bytes(ids, False)
        t, g = time_graph(lambda: chain(False), args.steps, args.warmup, torch)
        res["chain_no_norm"] = dict(rate(t, nb_c0, L), experts_read_mean=e_c0)
        del g
        # independent layers on one x: the one launch and L plain launches
        stack(True)
        per_layer(True)
        torch.cuda.synchronize()
        same_stack = bool(torch.equal(out, ref)) and bool(torch.equal(ids, ids_r))
        nb_st, e_st = pass_bytes(ids, False)
        t, g = time_graph(lambda: stack(), args.steps, args.warmup, torch)
        res["stack"] = dict(rate(t, nb_st, L), experts_read_mean=e_st,
                            equals_per_layer_calls=same_stack)
        del g
        t, g = time_graph(lambda: per_layer(), args.steps, args.warmup, torch)
        res["per_layer"] = rate(t, nb_st, L)
        del g
        # single eager launches timed by the kernel's own start / end events
        st = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * L)]
        for l, d in enumerate(layers):
            moe.moe_decode_forward_timed(x, d.router, d.routed, d.shared, ref[l], ws, ev[2 * l],
                                         ev[2 * l + 1], B=B, stream=st)
        torch.cuda.synchronize()
        res["per_layer"]["kernel_us_mean_eager"] = float(np.mean(
            [ev[2 * l].elapsed_time(ev[2 * l + 1]) for l in range(L)])) * 1000
        status = torch.full((1,), -1, dtype=torch.int32, device=dev)
        moe.moe_workspace_status(ws, status)
        torch.cuda.synchronize()
        res["wait_status"] = int(status.item())
        return res

    def run_prefill() -> dict:
        T = PREFILL_T
        d = layers[0]
        x = moe.device.to_device_bf16(testgen.make_x(args.seed + 1000, T), dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ws = moe.alloc_workspace(moe.moe_workspace_bytes(T, prefill=True), dev)
        nw = moe.device.to_device_bf16(testgen.make_x(args.seed + 7, 1)[0], dev)
        res = moe.device.to_device_bf16(testgen.make_x(args.seed + 1001, T), dev)
        t, g = time_graph(lambda: moe.moe_prefill_forward(x, d.router, d.routed, d.shared, out, ws,
                                                          T=T), args.prefill_steps, 2, torch)
        del g
        ms = t["ms"]
        tf = prefill_flop(T) / (ms * 1e-3) / 1e12
        tn, g = time_graph(lambda: moe.moe_prefill_forward_ex(
            x, d.router, d.routed, d.shared, out, ws, norm_w=nw, eps=EPS, residual=res, T=T),
            args.prefill_steps, 2, torch)
        del g
        return dict(tokens=T, ms_per_layer=ms, ms_p10_p50_p90=[t["p10"], t["p50"], t["p90"]],
                    tflops=tf, mfma_util=tf / PEAK_BF16_TFLOPS, flop=prefill_flop(T),
                    ms_per_layer_fused_norm_residual=tn["ms"])

    r1 = r8 = rp = rd = rg = rb = None
    if args.workload in ("all", "decode"):
        r1 = run_decode(1)
        for k in ("chain", "chain_no_norm", "per_layer_chain", "stack", "per_layer"):
            log(f"B=1 {k}: {r1[k]['us_per_layer']:.2f} us/layer, {r1[k]['gbps']:.0f} GB/s")
        if not args.no_batch8:
            r8 = run_decode(8)
            for k in ("chain", "chain_no_norm", "per_layer_chain", "stack", "per_layer"):
                log(f"B=8 {k}: {r8[k]['us_per_layer']:.2f} us/layer, {r8[k]['gbps']:.0f} GB/s")
    if args.workload in ("all", "prefill"):
        rp = run_prefill()
        log(f"prefill {rp['tokens']} tokens: {rp['ms_per_layer']:.3f} ms/layer, "
            f"{rp['tflops']:.0f} TFLOP/s ({100 * rp['mfma_util']:.1f}% of bf16 peak)")
    if args.workload == "all":
        rb = run_bf16(args, moe, testgen, torch, dev)
        rd = run_dense(args, moe, testgen, torch, dev)
        rg = run_general(args, moe, testgen, torch, dev)
    if r1 is None:
        print(json.dumps({"prefill": rp}), flush=True)
        return 0

    # ---------------------------------------------------------------- CPU baseline
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args, host0, testgen)

    # The timed region is one HIP-graph replay per step holding the whole
    # L-layer chained pass as ONE launch of the chained kernel: the HIP-event
    # time per replay is that kernel's average launch duration.
    ch = r1["chain"]
    roof = {"bound": "hbm",
            "kernel": f"k_decode_chain<1, nvfp4, rmsnorm> (one launch per {L}-layer pass)",
            "achieved": ch["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ch["gbps"] / PEAK_HBM_GBS,
            "traffic": measured_traffic("k_decode_chain_b1_traffic", L),
            "per_launch_bytes": ch["bytes_per_pass"], "launch_us": ch["ms_per_pass"] * 1000,
            "timing": f"HIP events around {args.steps} graph replays of one launch each "
                      f"(p10/p50/p90 of single replays in batch1.chain)"}
    res = {
        "metric": "MoE-layer decode µs/layer + achieved HBM GB/s (W4A16, batch 1 and 8)",
        "value": round(ch["gbps"], 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ch["ms_per_pass"], 4),
        "us_per_layer": round(ch["us_per_layer"], 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4-w/bf16-a, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights packed to NVFP4)",
        "config": {"workload": f"{L}-layer Flint-shaped MoE decode stack, batch 1, nvfp4, "
                               f"chained residual stream x_(l+1) = x_l + MoE_l(RMSNorm_l(x_l)), "
                               f"one HIP graph per pass holding one launch, weights cold (pass "
                               f"> last-level cache)",
                   "hidden": H, "inter": I, "experts": E, "top_k": K, "shared": 1,
                   "layers": L, "batch": 1, "weight_format": "nvfp4",
                   "resident_weight_bytes": int(resident)},
        "batch1": r1, "batch8": r8, "bf16_w16a16": rb, "prefill": rp, "dense_gemv": rd,
        "general_shapes": rg, "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


def run_bf16(args, moe, testgen, torch, dev, n_layers: int = 8) -> dict:
    """The W16A16 layer (bf16 expert weights, config 3) at batch 1 and 8: 8
    distinct layers (a pass reads more than the last-level cache), as one
    stacked launch and as one launch per layer, HIP graphs."""
    t0 = time.time()
    layers = [moe.DeviceLayer.from_host(testgen.make_layer(args.seed, l, "bf16"), dev)
              for l in range(n_layers)]
    log(f"bf16: {n_layers} layers generated and resident ({time.time() - t0:.1f} s)")
    table = moe.layer_table(layers, dev)
    S = moe.shape(moe.MOE_W_BF16)
    out = {}
    for B in (1, 8):
        x = moe.device.to_device_bf16(testgen.make_x(args.seed, B), dev)
        ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, fmt="bf16"), dev)
        y = torch.empty((n_layers, B, H), dtype=torch.bfloat16, device=dev)
        ids = torch.empty((n_layers, B, K), dtype=torch.int32, device=dev)
        moe.moe_decode_stack_forward(x, table, y, ws, ids, S=S, B=B)
        torch.cuda.synchronize()
        h = ids.cpu().numpy()
        nb = sum(layer_bytes(len(set(h[l].ravel().tolist())) + 1, B, "bf16")
                 for l in range(n_layers))

        def per_layer():
            for l, d in enumerate(layers):
                moe.moe_decode_forward(x, d.router, d.routed, d.shared, y[l], ws, S=S, B=B)
        t, g = time_graph(lambda: moe.moe_decode_stack_forward(x, table, y, ws, S=S, B=B),
                          args.steps, args.warmup, torch)
        del g
        tp, g = time_graph(per_layer, args.steps, args.warmup, torch)
        del g
        out[f"b{B}"] = dict(B=B, stack=rate(t, nb, n_layers), per_layer=rate(tp, nb, n_layers))
        log(f"bf16 B={B}: stack {out[f'b{B}']['stack']['us_per_layer']:.2f} us/layer "
            f"({out[f'b{B}']['stack']['gbps']:.0f} GB/s), per layer "
            f"{out[f'b{B}']['per_layer']['us_per_layer']:.2f} us")
    del layers
    torch.cuda.empty_cache()
    return out


def cpu_baseline(args, host0, testgen) -> dict:
    """The fp64 C oracle on the host cores, each leg bounded by --cpu-seconds:
    the batch-1 layer (layer 0, from packed weights, its dequant of the 7
    experts read included) on one thread and on all threads, and the
    8,192-token prefill layer extrapolated from 512 tokens on all threads."""
    import oracle
    nthreads = oracle.num_threads()
    x1 = testgen.make_x(args.seed, 1)

    def timed(fn, budget):
        reps, t_start = 0, time.time()
        while True:
            fn()
            reps += 1
            if time.time() - t_start >= budget:
                break
        return (time.time() - t_start) / reps, reps
    oracle.set_num_threads(1)
    st_s, st_reps = timed(lambda: oracle.forward_layer(x1, host0), args.cpu_seconds / 3)
    oracle.set_num_threads(nthreads)
    mt_s, mt_reps = timed(lambda: oracle.forward_layer(x1, host0), args.cpu_seconds / 3)
    xp = testgen.make_x(args.seed + 1000, 512)
    t0 = time.time()
    oracle.forward_layer(xp, host0)
    pf_512 = time.time() - t0
    nb = layer_bytes(7, 1, "nvfp4")
    log(f"oracle: {st_s * 1e6:.0f} us/layer on 1 thread, {mt_s * 1e6:.0f} us on {nthreads}; "
        f"prefill 512 tokens {pf_512:.2f} s")
    return {"value": nb / mt_s / 1e9, "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "us_per_layer_all_threads": mt_s * 1e6, "us_per_layer_one_thread": st_s * 1e6,
            "gbps_one_thread": nb / st_s / 1e9,
            "prefill_8192_ms_extrapolated": pf_512 * 16 * 1e3,
            "sample": f"fp64 C oracle, batch-1 forward of layer 0 (from packed weights, incl. "
                      f"its dequant of the 7 experts read): {mt_reps} reps on {nthreads} OpenMP "
                      f"threads and {st_reps} reps on 1 thread; prefill: 512 of the 8,192 tokens "
                      f"on {nthreads} threads, x16 (extrapolated)"}


if __name__ == "__main__":
    sys.exit(main())
