#!/usr/bin/env python3
"""Throughput of the hyper-connection residual-stream layer on one GPU.

A step is one pass of the whole layer path over one batch of synthetic
input: for the default workload, the 8-layer xHC chain at N=16 streams,
k=4 active (m=2 fixed), C=4096, batch 2 x seq 8192, bf16, layers
alternating attention-type (K_r=1) and MLP-type (causal convolutions
{4,8,12} + Gram-Schmidt, K_r=4), the state carried in place from layer to
layer.  The chain runs through the chained C-ABI calls (xhc_route once,
then xhc_pre_chained + xhc_post_chained per layer: each layer's routing is
accumulated while the layer before it runs); --api single times xhc_pre +
xhc_post per layer instead.  The sublayer F is a given tensor per layer (its
cost is not part of the layer).

Prints ONE JSON line.  ``value`` is tokens/s per layer (tokens x layers /
elapsed); ``hbm`` gives the algorithmic bytes moved (state read/write
counted once per the byte model below) as GB/s and as a fraction of the
MI355X peak of 8 TB/s.  ``roofline`` covers the call that dominates the
step, timed with HIP events on the stream the kernels are launched on; its
``traffic`` is the measured HBM bytes per launch from the committed counter
summary, while the kernel sources are the ones it was measured on.
``cpu_baseline`` times the float64 oracle on a bounded sample of the same
workload on the host cores.

Byte model per token and layer (C-element units, state dtype): pre reads
the N streams and writes the sublayer input (N + 1); post reads F's output
and the k active rows and writes the k rows back (1 + 2k).  Weights (a few
MiB per layer) and per-token coefficients (< 1%) are not counted.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    # name: (kind, N, k, m, C, B, S, layer kinds)
    "xhc_chain_n16k4_c4096": ("xhc", 16, 4, 2, 4096, 2, 8192, "AMAMAMAM"),
    "xhc_mlp_n16k4_c2048": ("xhc", 16, 4, 2, 2048, 4, 4096, "M"),
    "mhc_n4_c4096": ("mhc", 4, 4, 0, 4096, 4, 4096, "D"),
    "mhc_n16_c4096": ("mhc", 16, 16, 0, 4096, 4, 4096, "D"),
    # xHC-Flash: 4 blocks, each an attention + MLP pair sharing one routing
    "xhcf_chain_n16k4_c4096": ("xhcf", 16, 4, 2, 4096, 2, 8192, "AMAMAMAM"),
    # xHC-Flash-4sub: 2 groups of two blocks sharing one routing
    "xhcf4_chain_n16k4_c4096": ("xhcf4", 16, 4, 2, 4096, 2, 8192, "AMAMAMAM"),
    # single-token decode: 256 sequences, one new token each, 8 sublayers
    "xhc_decode_n16k4_c4096": ("xhcd", 16, 4, 2, 4096, 256, 1, "AMAMAMAM"),
    # backward of an MLP-type and an attention-type sublayer (the gradients of
    # xhc_pre + xhc_post), the state gradient carried from the one to the other
    "xhc_bwd_n16k4_c4096": ("xhcb", 16, 4, 2, 4096, 2, 8192, "AM"),
}
DEFAULT = "xhc_chain_n16k4_c4096"
SEED = {"xhc_chain_n16k4_c4096": 3, "xhc_mlp_n16k4_c2048": 2, "mhc_n4_c4096": 1, "mhc_n16_c4096": 4,
        "xhcf_chain_n16k4_c4096": 3, "xhc_decode_n16k4_c4096": 5, "xhcf4_chain_n16k4_c4096": 3,
        "xhc_bwd_n16k4_c4096": 6}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_configs(name):
    from stream_residual_mixing_amd.binding import Config
    kind, N, k, m, C, B, S, kinds = WORKLOADS[name]
    cfgs = []
    for lk in kinds:
        if kind == "mhc":
            cfgs.append(Config(N=N, C=C, B=B, S=S, dtype="bf16"))
        else:
            cfgs.append(Config(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=3 if lk == "M" else 0, dtype="bf16"))
    return kind, cfgs, kinds


def flash_bytes_per_token(cfg, esz=2):
    """Algorithmic bytes per token of one xHC-Flash block's three calls, in
    the pages' design of two full-state passes per block: pre reads the state
    for the projection and again for both readouts and writes the two inputs
    (2N + 2); mid reads the attention output, the k active rows and the MLP
    base readout and writes both back (1 + k + 1, k + 1); post is full xHC's
    (1 + 2k).  The active-row projections (k rows, twice) are not counted."""
    N, k, C = cfg.N, cfg.k, cfg.C
    return (2 * N + 2) * C * esz, (2 * k + 3) * C * esz, (1 + 2 * k) * C * esz


def flash4_bytes_per_token(cfg, esz=2):
    """Algorithmic bytes per token of an xHC-Flash-4sub group's five calls, in
    the pages' design of two full-state passes per group: pre reads the state
    twice and writes the first input and three non-active bases (2N + 4);
    each intermediate post writes its sublayer (1 + 2k) and forms the next
    input from its base and the k active rows (1 + k + 1); the last post is
    full xHC's (1 + 2k).  The active-map projections share the input's read
    of the k rows."""
    N, k, C = cfg.N, cfg.k, cfg.C
    mid = (1 + 2 * k + 2 + k) * C * esz
    return (2 * N + 4) * C * esz, mid, mid, mid, (1 + 2 * k) * C * esz


def bwd_bytes_per_token(cfg, esz=2):
    """Algorithmic bytes per token of the backward's two calls.  Application
    half: read the state (N rows, for the H_pre and H_res gradients), the new
    state's gradient on the k active rows, d_inp and out; write d_out:
    N + k + 3.  Generation half: read the state (the norms and projections),
    the new state's gradient on the N - k other rows and d_inp; write the
    state gradient: 3N - k + 1.  Intermediates (the gathered active rows,
    the active rows' float gradient, the basis gradient, the partial weight
    gradients) are not counted."""
    N, k, C = cfg.N, cfg.k, cfg.C
    return (N + k + 3) * C * esz, (3 * N - k + 1) * C * esz


def bytes_per_token(kind, cfg, esz=2):
    """Algorithmic bytes per token of (pre, post).  Decode: the MLP-type
    write also reads the 11 earlier outputs from the ring and stores the new
    one (11 + 1 more).  Backward: (application half, generation half)."""
    if kind == "xhcb":
        return bwd_bytes_per_token(cfg, esz)
    if kind == "xhcd":
        extra = 12 if cfg.K_r == 4 else 0
        return (cfg.N + 1) * cfg.C * esz, (1 + 2 * cfg.k + extra) * cfg.C * esz
    if kind == "xhcf":
        # a block is two sublayers: half of its bytes per sublayer
        return sum(flash_bytes_per_token(cfg, esz)) // 2, 0
    if kind == "xhcf4":
        return sum(flash4_bytes_per_token(cfg, esz)) // 4, 0
    if kind == "mhc":
        return (cfg.N + 1) * cfg.C * esz, (1 + 2 * cfg.N) * cfg.C * esz
    return (cfg.N + 1) * cfg.C * esz, (1 + 2 * cfg.k) * cfg.C * esz


def flops_per_token(kind, cfg):
    if kind == "xhcb":   # the projections recomputed, and their transposes for dX and dW
        return 3 * (2 * cfg.N * cfg.C * 2 * cfg.N + 2 * cfg.k * cfg.C * (cfg.k * cfg.k + cfg.k * cfg.K_r))
    if kind == "xhcf4":   # per sublayer: a quarter of a group's projections
        N, k, C, KR = cfg.N, cfg.k, cfg.C, 4
        return (2 * N * C * 5 * N + 2 * k * C * (k + k * KR + k + k * k + k * KR)) // 4
    if kind == "xhcf":   # per sublayer: half of a block's three projections
        N, k, C = cfg.N, cfg.k, cfg.C
        return (2 * N * C * 3 * N + 2 * k * C * k + 2 * k * C * (k * k + 4 * k)) // 2
    if kind == "mhc":
        return 2 * cfg.N * cfg.C * (2 * cfg.N + cfg.N * cfg.N)
    return 2 * cfg.N * cfg.C * 2 * cfg.N + 2 * cfg.k * cfg.C * (cfg.k * cfg.k + cfg.k * cfg.K_r)


def make_inputs(name, kind, cfgs, kinds):
    """Seeded synthetic inputs (CPU) moved to the GPU."""
    import torch
    from stream_residual_mixing_amd import synth
    from stream_residual_mixing_amd.binding import weights_to_device
    seed = SEED[name]
    c0 = cfgs[0]
    t = time.time()
    X = synth.state(seed, c0.T, c0.N, c0.C, "bf16").to("cuda")
    outs, ws_ = [], []
    for l, cfg in enumerate(cfgs):
        outs.append(synth.sublayer_out(seed, l, cfg.B, cfg.S, cfg.C, "bf16").to("cuda"))
        if kind == "xhcf4":
            if l % 4 == 0:
                from stream_residual_mixing_amd.binding import flash4_weights_to_device
                ws_.append(flash4_weights_to_device(synth.xhcf4_group_weights(seed, l // 4, cfg.N, cfg.k, cfg.C, 4,
                                                                               "bf16")))
            continue
        if kind == "xhcf":
            if l % 2 == 0:
                from stream_residual_mixing_amd.binding import flash_weights_to_device
                ws_.append(flash_weights_to_device(synth.xhcf_block_weights(seed, l // 2, cfg.N, cfg.k, cfg.C, 4,
                                                                            "bf16")))
            continue
        if kind == "mhc":
            wd = synth.mhc_layer_weights(seed, l, cfg.N, cfg.C, "bf16")
        else:
            wd = synth.xhc_layer_weights(seed, l, cfg.N, cfg.k, cfg.C, cfg.K_r, "bf16")
        ws_.append(weights_to_device(wd))
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t:.1f} s (X {tuple(X.shape)} {X.dtype})")
    return X, outs, ws_


def default_api(name):
    kind, _, _, _, _, _, _, kinds = WORKLOADS[name]
    if kind == "xhcf":
        return "flash"
    if kind == "xhcd":
        return "decode"
    if kind == "xhcf4":
        return "flash4"
    if kind == "xhcb":
        return "backward"
    return "chained" if kind == "xhc" and len(kinds) > 1 else "single"


def run_gpu(name, steps, warmup, api):
    import torch
    from stream_residual_mixing_amd import binding
    from stream_residual_mixing_amd.binding import Config
    kind, cfgs, kinds = layer_configs(name)
    lib = binding.load()
    X, outs, weights = make_inputs(name, kind, cfgs, kinds)
    c0 = cfgs[0]
    T = c0.T
    inp = torch.empty((T, c0.C), dtype=torch.bfloat16, device="cuda")
    mhc = kind == "mhc"
    big = max(cfgs, key=lambda c: lib.workspace_bytes(c, mhc))
    stream = torch.cuda.current_stream()
    calls = []   # (name, bytes per token, launch function), in step order
    b_pre, b_post = bytes_per_token(kind, c0)
    if kind == "xhcf":
        fcfg = Config(N=c0.N, k=c0.k, m=c0.m, C=c0.C, B=c0.B, S=c0.S, n_convs=3, dtype="bf16")
        ws = lib.flash_workspace(fcfg)
        inp_m = torch.empty_like(inp)
        bp, bm, bq = flash_bytes_per_token(fcfg)
        for b in range(len(cfgs) // 2):
            w = weights[b]
            calls.append(("xhcf_pre", bp, lambda w=w: lib.xhcf_pre(fcfg, w, X, inp, inp_m, ws, stream)))
            calls.append(("xhcf_mid", bm, lambda w=w, b=b: lib.xhcf_mid(fcfg, w, X, outs[2 * b], inp_m, ws, stream)))
            calls.append(("xhcf_post", bq, lambda w=w, b=b: lib.xhcf_post(fcfg, w, X, outs[2 * b + 1], ws, stream)))
    elif kind == "xhcf4":
        fcfg = Config(N=c0.N, k=c0.k, m=c0.m, C=c0.C, B=c0.B, S=c0.S, n_convs=3, dtype="bf16")
        ws = lib.flash4_workspace(fcfg)
        bases = torch.empty((3, T, c0.C), dtype=torch.bfloat16, device="cuda")
        fb = flash4_bytes_per_token(fcfg)
        for g in range(len(cfgs) // 4):
            w = weights[g]
            calls.append(("xhcf4_pre", fb[0], lambda w=w: lib.xhcf4_pre(fcfg, w, X, inp, bases, ws, stream)))
            for q in range(1, 5):
                calls.append((f"xhcf4_post{q}", fb[q], lambda w=w, g=g, q=q: lib.xhcf4_post(
                    fcfg, w, q, X, outs[4 * g + q - 1], bases, inp, ws, stream)))
    elif kind == "xhcb":
        # the maps of each layer, left by xhc_pre, stay in that layer's workspace
        wss = [lib.workspace(cfg) for cfg in cfgs]
        for l, cfg in enumerate(cfgs):
            lib.xhc_pre(cfg, weights[l], X, inp, wss[l], stream)
        bws = lib.backward_workspace(max(cfgs, key=lib.backward_workspace_bytes))
        g0 = torch.empty_like(X).normal_()
        gbuf = [torch.empty_like(X), torch.empty_like(X)]
        d_inp = torch.empty_like(inp).normal_()
        d_out = torch.empty_like(inp)
        d_conv = torch.empty((24, c0.C), dtype=torch.float32, device="cuda")
        grads = [lib.grads(cfg) for cfg in cfgs]
        src = g0
        for j, l in enumerate(reversed(range(len(cfgs)))):
            cfg, lk = cfgs[l], kinds[l]
            dst = gbuf[j % 2]
            bp, bq = bytes_per_token(kind, cfg)
            calls.append((f"xhc_post_backward_{lk}", bp, lambda cfg=cfg, l=l, s_=src: lib.xhc_post_backward(
                cfg, weights[l], X, outs[l].reshape(cfg.T, cfg.C), d_inp, s_, d_out,
                d_conv if cfg.K_r == 4 else None, wss[l], bws, stream)))
            calls.append((f"xhc_pre_backward_{lk}", bq, lambda cfg=cfg, l=l, s_=src, d_=dst: lib.xhc_pre_backward(
                cfg, weights[l], X, d_inp, s_, d_, grads[l], wss[l], bws, stream)))
            src = dst
    elif kind == "xhcd":
        ws = lib.workspace(big)
        ring = torch.zeros((c0.B, 12, c0.C), dtype=torch.bfloat16, device="cuda")
        steps_t = torch.full((c0.B,), 100, dtype=torch.int32, device="cuda")
        for l, (cfg, lk) in enumerate(zip(cfgs, kinds)):
            bp, bq = bytes_per_token(kind, cfg)
            calls.append((f"xhc_pre_{lk}", bp, lambda cfg=cfg, l=l: lib.xhc_pre(cfg, weights[l], X, inp, ws, stream)))
            if lk == "M":
                calls.append((f"xhc_post_decode_{lk}", bq, lambda cfg=cfg, l=l: lib.xhc_post_decode(
                    cfg, weights[l], X, outs[l].reshape(cfg.T, cfg.C), ring, steps_t, ws, stream)))
            else:
                calls.append((f"xhc_post_{lk}", bq, lambda cfg=cfg, l=l: lib.xhc_post(cfg, weights[l], X, outs[l], ws,
                                                                                      stream)))
    elif api == "chained":
        wsp = [lib.workspace(big), lib.workspace(big)]
        calls.append(("xhc_route", c0.N * c0.C * 2, lambda: lib.xhc_route(cfgs[0], weights[0], X, wsp[0], stream)))
        for l, (cfg, lk) in enumerate(zip(cfgs, kinds)):
            nx = l + 1 < len(cfgs)
            cn, wn, wsn = (cfgs[l + 1], weights[l + 1], wsp[(l + 1) % 2]) if nx else (None, None, None)
            ws = wsp[l % 2]
            calls.append((f"xhc_pre_chained_{lk}", b_pre,
                          lambda cfg=cfg, l=l, cn=cn, wn=wn, ws=ws, wsn=wsn:
                          lib.xhc_pre_chained(cfg, weights[l], cn, wn, X, inp, ws, wsn, stream)))
            calls.append((f"xhc_post_chained_{lk}", b_post,
                          lambda cfg=cfg, l=l, cn=cn, wn=wn, ws=ws, wsn=wsn:
                          lib.xhc_post_chained(cfg, weights[l], cn, wn, X, outs[l], ws, wsn, stream)))
    else:
        ws = lib.workspace(big, mhc)
        pre = lib.mhc_pre if mhc else lib.xhc_pre
        post = lib.mhc_post if mhc else lib.xhc_post
        p = "mhc" if mhc else "xhc"
        for l, (cfg, lk) in enumerate(zip(cfgs, kinds)):
            calls.append((f"{p}_pre_{lk}", b_pre, lambda cfg=cfg, l=l: pre(cfg, weights[l], X, inp, ws, stream)))
            calls.append((f"{p}_post_{lk}", b_post, lambda cfg=cfg, l=l: post(cfg, weights[l], X, outs[l], ws, stream)))

    def step(evs=None):
        for j, (_, _, fn) in enumerate(calls):
            if evs is not None:
                evs[j].record(stream)
            fn()
        if evs is not None:
            evs[len(calls)].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs_all = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    log(f"timing {steps} steps of {len(cfgs)} layers ({name}, {api} calls)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(evs_all[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    per_call = {}
    for s in range(steps):
        e = evs_all[s]
        for j, (cname, _, _) in enumerate(calls):
            per_call.setdefault(cname, []).append(e[j].elapsed_time(e[j + 1]) * 1e-3)
    call_bytes = {cname: bpt * T for cname, bpt, _ in calls}
    return dict(kind=kind, cfgs=cfgs, kinds=kinds, elapsed=elapsed, per_call=per_call, T=T, call_bytes=call_bytes)


def cpu_baseline(name, tokens=256):
    """The oracle on the first `tokens` tokens of batch item 0, one layer of
    each kind in the workload; tokens/s per layer."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import cases as K
    from stream_residual_mixing_amd import synth
    from stream_residual_mixing_amd.binding import Config
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = os.cpu_count() or 1
    kind, cfgs, kinds = layer_configs(name)
    seed = SEED[name]
    done = {}
    total_t, total_tok = 0.0, 0
    for l, (cfg, lk) in enumerate(zip(cfgs, kinds)):
        if lk in done:
            continue
        sub = Config(N=cfg.N, k=cfg.k, m=cfg.m, C=cfg.C, B=1, S=tokens, n_convs=cfg.n_convs, dtype="bf16")
        X = K.f64(synth.state_rows(seed, range(tokens), cfg.N, cfg.C, "bf16"))
        out = K.f64(synth.out_rows(seed, l, range(tokens), cfg.C, "bf16")).reshape(1, tokens, cfg.C)
        if kind == "xhcf4":
            # one group: all four sublayers
            ow = K.flash4_oracle_weights(synth.xhcf4_group_weights(seed, 0, cfg.N, cfg.k, cfg.C, 4, "bf16"))
            outs = [K.f64(synth.out_rows(seed, q, range(tokens), cfg.C, "bf16")).reshape(1, tokens, cfg.C)
                    for q in range(4)]
            sub.n_convs = 3
            t = time.perf_counter()
            K.oracle_flash4(sub, X, outs, ow)
            dt = time.perf_counter() - t
            done["A"] = done["M"] = dt / 4
            total_t += dt
            total_tok += 4 * tokens
            break
        if kind == "xhcf":
            # one block: both sublayers of the pair
            ow = K.flash_oracle_weights(synth.xhcf_block_weights(seed, 0, cfg.N, cfg.k, cfg.C, 4, "bf16"))
            outm = K.f64(synth.out_rows(seed, 1, range(tokens), cfg.C, "bf16")).reshape(1, tokens, cfg.C)
            sub.n_convs = 3
            t = time.perf_counter()
            K.oracle_flash(sub, X, out, outm, ow)
            dt = time.perf_counter() - t
            done["A"] = done["M"] = dt / 2
            total_t += dt
            total_tok += 2 * tokens
            break
        if kind == "xhcb":
            from oracle import hc_grad as G
            from oracle import hc_oracle as O
            ow = K.oracle_weights(synth.xhc_layer_weights(seed, l, cfg.N, cfg.k, cfg.C, cfg.K_r, "bf16"))
            r = np.random.default_rng([seed, 99, l])
            d_inp, d_X = r.standard_normal((tokens, cfg.C)), r.standard_normal((tokens, cfg.N, cfg.C))
            alpha = (ow["alpha_pre"], ow["alpha_res"], ow["alpha_post"])
            t = time.perf_counter()
            pre = O.xhc_pre(X, ow["w_full"], ow["w_act"], cfg.m, cfg.k, cfg.K_r, alpha, ow["b_pre"], ow["b_res"],
                            ow["b_post"], iters=cfg.iters)
            ga = G.xhc_apply_grads(X, out, pre["I"], pre["p"], pre["h_pre"], pre["h_res"], pre["h_post"],
                                   ow["conv"], d_inp, d_X)
            G.xhc_gen_grads(X, ow["w_full"], ow["w_act"], cfg.m, cfg.k, cfg.K_r, alpha, ow["b_pre"], ow["b_res"],
                            ow["b_post"], pre["I"], ga["h_pre"], ga["h_res"], ga["h_post"], ga["p"],
                            iters=cfg.iters)
        elif kind == "mhc":
            ow = K.oracle_weights(synth.mhc_layer_weights(seed, l, cfg.N, cfg.C, "bf16"))
            t = time.perf_counter()
            K.oracle_mhc(sub, X, out, ow)
        else:
            ow = K.oracle_weights(synth.xhc_layer_weights(seed, l, cfg.N, cfg.k, cfg.C, cfg.K_r, "bf16"))
            t = time.perf_counter()
            K.oracle_xhc(sub, X, out, ow)
        dt = time.perf_counter() - t
        done[lk] = dt
        total_t += dt
        total_tok += tokens
    kinds_s = "+".join({"A": "attention", "M": "MLP", "D": "dense"}[k] for k in done)
    if kind == "xhcb":
        kinds_s += " backward (maps, both gradient halves; PyTorch CPU autograd in float64)"
    if kind == "xhcf":
        kinds_s = "xHC-Flash block (attention + MLP)"
    if kind == "xhcf4":
        kinds_s = "xHC-Flash-4sub group (attention, MLP, attention, MLP)"
    return dict(value=total_tok / total_t, unit="tokens/s per layer", cores=int(cores), kind="oracle",
                sample=f"first {tokens} tokens of batch item 0, one {kinds_s} layer each, float64 NumPy")


# ----------------------------------------------------------------- traffic
# Measured HBM bytes per call come from two rocprofv3 counter runs of this
# script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) and the same two
# counters read for a plain 1 GiB device copy (--copy-probe), whose true bytes
# are known: each counter is scaled by (true bytes / counter) of the copy.
# --traffic-summary turns those runs into profiles/<workload>_traffic.json,
# stamped with a hash of the kernel sources; a later run reports the traffic
# only while the sources still hash the same.
CSRC = os.path.join(ROOT, "stream_residual_mixing_amd", "csrc")


def sources_hash():
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"{workload}_traffic.json")


def _pmc_rows(d):
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = list(csv.DictReader(open(f[0])))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]


def _attention_post_pass(name):
    """The persistent post pass that writes an attention-type sublayer
    (register- or LDS-staged; its last template argument, the write kind,
    is 1)."""
    import re
    m = re.search(r"xhc_post_[ps]_kernel<[^>]*,\s*(\d+)>", name)
    return bool(m) and m.group(1) == "1"


def _split_calls(rows, single=False):
    """Group this library's dispatches of one step into calls, in order: a
    call starts at a weight-packing kernel (xHC or mHC), at the Gram kernel, at an apply
    kernel not preceded by the Gram kernel, at the persistent post pass that
    also writes (the chained attention-type post call), or at the mHC write.
    With per-sublayer calls (single), a weight-packing kernel right after the
    routing finalize continues the call: a large xhc_pre runs the routing
    pass and then the pre pass, each with its own packing."""
    calls, prev = [], ""
    for name, v in rows:
        if "xhc::" not in name:
            continue
        cont = single and "xhc_prep_kernel" in name and "xhc_route_fin_kernel" in prev
        start = (("xhc_prep_kernel" in name and not cont) or "pack_b_kernel" in name or "xhc_gram_kernel" in name
                 or ("xhc_apply_kernel" in name and "xhc_gram_kernel" not in prev)
                 or _attention_post_pass(name) or "mhc_post_kernel" in name)
        if start or not calls:
            calls.append([])
        calls[-1].append((name, v))
        prev = name
    return calls


_FORWARD_PRE_KERNELS = ("xhc_pre_fused_kernel", "xhc_prep_kernel", "xhc_proj_s_kernel", "xhc_proj_p_kernel",
                        "xhc_route_fin_kernel", "xhc_pre_chained_s_kernel", "xhc_pre_chained_kernel",
                        "xhc_act_fin_kernel")


def _split_backward_calls(rows):
    """Backward workload: skip the set-up (xhc_pre of each sublayer, by any
    of its kernels); a call starts at an application kernel
    (xhc_post_backward) or at the first weight-packing kernel of a run of
    them (xhc_pre_backward)."""
    calls, prev = [], ""
    for name, v in rows:
        if "xhc::" not in name or any(k in name for k in _FORWARD_PRE_KERNELS):
            continue
        start = "bwd_apply_kernel" in name or ("pack_b_kernel" in name and "pack_b_kernel" not in prev)
        if start or not calls:
            calls.append([])
        calls[-1].append((name, v))
        prev = name
    return calls


def traffic_summary(workload, pmcdir):
    """Writes profiles/<workload>_traffic.json from the four counter runs
    under pmcdir (chain_fetch, chain_write, copy_fetch, copy_write; for the
    backward workload the first two hold its runs)."""
    copy_bytes = 1 << 30
    scale = {}
    for c, sub in (("FETCH_SIZE", "copy_fetch"), ("WRITE_SIZE", "copy_write")):
        vals = [v for n, v in _pmc_rows(os.path.join(pmcdir, sub)) if "copyBuffer" in n and v > 1e5]
        scale[c] = copy_bytes / (sum(vals) / len(vals) * 1024)
    kind, cfgs, kinds = layer_configs(workload)
    api = default_api(workload)
    if kind == "xhcb":
        split = _split_backward_calls
    else:
        def split(rows):
            return _split_calls(rows, single=(api == "single"))
    fetch = split(_pmc_rows(os.path.join(pmcdir, "chain_fetch")))
    write = split(_pmc_rows(os.path.join(pmcdir, "chain_write")))
    if kind == "xhcb":
        names = [f"{p}_{lk}" for lk in reversed(kinds) for p in ("xhc_post_backward", "xhc_pre_backward")]
    elif kind == "xhc" and api == "single":
        names = [f"{p}_{lk}" for lk in kinds for p in ("xhc_pre", "xhc_post")]
    else:
        names = (["xhc_route"] if kind == "xhc" else []) + [
            f"{p}_{lk}" for lk in kinds for p in (("xhc_pre_chained", "xhc_post_chained") if kind == "xhc"
                                                  else ("mhc_pre", "mhc_post"))]
    if len(fetch) != len(names) or len(write) != len(names):
        raise SystemExit(f"found {len(fetch)} / {len(write)} calls, expected {len(names)}")
    per = {}
    for name, fc, wc in zip(names, fetch, write):
        fb = sum(v for _, v in fc) * 1024 * scale["FETCH_SIZE"]
        wb = sum(v for _, v in wc) * 1024 * scale["WRITE_SIZE"]
        per.setdefault(name, []).append((fb, wb, [n.replace("(anonymous namespace)::", "").split("(")[0]
                                                  for n, _ in fc]))
    out = {"workload": workload, "sources_sha256": sources_hash(), "copy_scale": scale, "calls": {}}
    for name, lst in per.items():
        out["calls"][name] = {"fetch_bytes": sum(x[0] for x in lst) / len(lst),
                              "write_bytes": sum(x[1] for x in lst) / len(lst), "kernels": lst[0][2]}
    with open(traffic_path(workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def measured_traffic(workload, call):
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != sources_hash() or call not in t.get("calls", {}):
        return None
    c = t["calls"][call]
    return round(c["fetch_bytes"] + c["write_bytes"])


def copy_probe(nbytes=1 << 30, reps=10):
    """A plain device-to-device copy of known size: the reference that scales
    the hardware byte counters, and the achievable-bandwidth yardstick."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    dt = a.elapsed_time(b) * 1e-3 / reps
    print(json.dumps({"copy_probe_bytes": nbytes, "read_plus_write_GBps": round(2 * nbytes / dt / 1e9, 1),
                      "avg_us": round(dt * 1e6, 2)}), flush=True)


def read_probe(nbytes=2 << 30, reps=10):
    """Read-only streams over a state-sized buffer (2 GiB, the chain's state):
    16-byte loads spread over the device with the default cache policy and
    with non-temporal loads (libxhc's xhc_probe_read), next to the copy
    probe.  The achievable rates the layer's kernels are compared with."""
    import torch
    from stream_residual_mixing_amd import binding
    lib = binding.load()
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {"read_probe_bytes": nbytes}
    for mode, name in ((0, "read_GBps"), (1, "read_nontemporal_GBps")):
        for _ in range(3):
            lib.probe_read(src, sink, mode, stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            lib.probe_read(src, sink, mode, stream)
        b.record(stream)
        torch.cuda.synchronize()
        dt = a.elapsed_time(b) * 1e-3 / reps
        res[name] = round(nbytes / dt / 1e9, 1)
        res[name.replace("GBps", "avg_us")] = round(dt * 1e6, 2)
    print(json.dumps(res), flush=True)
    copy_probe()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=256)
    ap.add_argument("--copy-probe", action="store_true", help="time a 1 GiB device copy and exit")
    ap.add_argument("--read-probe", action="store_true",
                    help="time read-only streams over a 2 GiB buffer (and the copy probe) and exit")
    ap.add_argument("--traffic-summary", metavar="PMCDIR", default=None,
                    help="write profiles/<workload>_traffic.json from rocprofv3 counter runs and exit")
    ap.add_argument("--api", choices=("chained", "single", "flash", "flash4", "decode", "backward"), default=None,
                    help="xHC calls: chained (routing of layer l+1 prepared during layer l; default for "
                         "multi-layer workloads) or single (xhc_pre / xhc_post per layer)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.workload, args.traffic_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the layer has no multi-GPU path in this library "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    if args.read_probe:
        read_probe()
        return
    api = args.api or default_api(args.workload)
    r = run_gpu(args.workload, args.steps, args.warmup, api)
    kind, cfgs, kinds, T = r["kind"], r["cfgs"], r["kinds"], r["T"]
    L = len(cfgs)
    ms_per_step = r["elapsed"] / args.steps * 1e3
    value = T * L * args.steps / r["elapsed"]
    # algorithmic bytes: the method's byte model, whatever the calls move
    step_bytes = 0
    for cfg, lk in zip(cfgs, kinds):
        b_pre, b_post = bytes_per_token(kind, cfg)
        step_bytes += T * (b_pre + b_post)
    call_bytes = r["call_bytes"]
    hbm_gbps = step_bytes * args.steps / r["elapsed"] / 1e9
    calls = {}
    for name, ts in r["per_call"].items():
        avg = sum(ts) / len(ts)
        calls[name] = dict(avg_us=round(avg * 1e6, 2), share=None,
                           GBps=round(call_bytes[name] / avg / 1e9, 1))
    tot = sum(sum(ts) for ts in r["per_call"].values())
    for name, ts in r["per_call"].items():
        calls[name]["share"] = round(sum(ts) / tot, 3)
    dom = max(r["per_call"], key=lambda n: sum(r["per_call"][n]))
    dom_avg = sum(r["per_call"][dom]) / len(r["per_call"][dom])
    achieved = call_bytes[dom] / dom_avg / 1e9
    c0 = cfgs[0]
    res = {
        "metric": "xHC layer tokens/s + HBM GB/s (% of peak), N=16 k=4 C=4096, 1 MI355X"
        if args.workload == DEFAULT else f"{args.workload} layer tokens/s",
        "value": round(value, 1),
        "unit": "tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "kind": kind, "api": api, "N": c0.N,
                   "k": c0.k if kind in ("xhc", "xhcf", "xhcf4", "xhcd", "xhcb") else c0.N,
                   "m": c0.m, "C": c0.C, "batch": c0.B, "seq": c0.S, "tokens": T, "layers": kinds,
                   "sinkhorn_iters": c0.iters},
        "hbm": {"GBps": round(hbm_gbps, 1), "frac_of_peak": round(hbm_gbps / HBM_PEAK_GBPS, 4),
                "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.workload, dom) if api == default_api(args.workload) else None,
                     "kernel": dom,
                     "bytes_per_launch": call_bytes[dom], "avg_us": round(dom_avg * 1e6, 2)},
        "calls": calls,
        "mfma": {"flop_per_token_layer": [flops_per_token(kind, c) for c in cfgs][:2],
                 "peak_TFLOPs_bf16": MFMA_BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a CPU sample")
        res["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
