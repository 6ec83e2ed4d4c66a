"""Benchmark of the W8A8 INT8 linear-layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-rows] [--no-cpu]

Headline step (the DeepSeek-V3 dense MLP at M = 4096 tokens, channel-wise
scheme, inputs resident in HBM):
    quant_act_token(x[4096, 7168])  -> gemm_w8a8_channel(gate_up: K=7168 -> N=36864)
    quant_act_token(h[4096, 18432]) -> gemm_w8a8_channel(down:    K=18432 -> N=7168)
The intermediate h is a separate synthetic input (the SiLU-and-multiply
between the two GEMMs is not part of the method).  Two weight sets alternate
between steps.  value = int8 GEMM operations of the step / step time, in TOPS.

Also reported (unless --no-rows): every other row of the path at its own
shapes - block-wise GEMMs and quantisers at M = 4096, channel-wise at
M = 128 and 1024, decode (M = 1..64) block-wise and W8A16 GEMMs in GB/s over
weight copies rotated through more than 1 GB so the 256 MB Infinity Cache
cannot serve repeats, the grouped MoE GEMMs, and the FP8 requantisation.

roofline: the dominant kernel (the gate_up channel GEMM), timed with HIP
events on the stream it runs on, against the dense int8 MFMA peak of 5.0 POP/s.
clock: the GFX clocks and socket power that amd-smi reports while the gate_up
GEMM runs back to back for about two seconds (the MFMA peak assumes 2.4 GHz).
cpu_baseline: the CPU oracle (numpy) on a bounded sample of the same step.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0       # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, 8 TB/s
M_HEAD = 4096
GATE_UP = (7168, 36864)       # (K, N)
DOWN = (18432, 7168)

# traffic of the dominant kernel from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE,
# scaled by the same counters' reading for a copy kernel of known size; None
# until counters have been taken for the current kernel.
TRAFFIC_GATE_UP_BYTES = 1.889e9   # rocprofv3 FETCH_SIZE x2.000 + WRITE_SIZE x1.000 (copy-calibrated), per launch of the current kernel


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-rows", action="store_true", help="headline step only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rows-reps", type=int, default=20)
    ap.add_argument("--rows-only", default="",
                    help="comma list of row groups to run: quant,tile,decode,w8a16,moe (default all)")
    ap.add_argument("--no-clock", action="store_true", help="skip the amd-smi clock window")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times): the reference kernel of known "
                         "size for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_calls(fn, n_rot, reps, warm=3):
    """Average ms per call of fn(i) over reps calls, i cycling over n_rot buffers."""
    import torch
    for i in range(warm):
        fn(i % n_rot)
    torch.cuda.synchronize()
    a, b = _events()
    a.record()
    for i in range(reps):
        fn(i % n_rot)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def headline(args):
    import torch
    import synth
    import w8a8_int8_quantized_amd as w8

    dev = torch.device("cuda:0")
    seed = synth.SEEDS["channel"]
    (Kg, Ng), (Kd, Nd) = GATE_UP, DOWN
    x = synth.activations(M_HEAD, Kg, seed=seed, device=dev)
    h = synth.activations(M_HEAD, Kd, seed=seed + 10, device=dev)
    sets = []
    for s in range(2):
        wg = synth.weights(Ng, Kg, seed=seed + 20 + s, device=dev)
        wd = synth.weights(Nd, Kd, seed=seed + 30 + s, device=dev)
        sets.append((w8.quant_weight_channel(wg), w8.quant_weight_channel(wd)))
        del wg, wd
    qx = (torch.empty(M_HEAD, Kg, dtype=torch.int8, device=dev), torch.empty(M_HEAD, dtype=torch.float32, device=dev))
    qh = (torch.empty(M_HEAD, Kd, dtype=torch.int8, device=dev), torch.empty(M_HEAD, dtype=torch.float32, device=dev))
    yg = torch.empty(M_HEAD, Ng, dtype=torch.bfloat16, device=dev)
    yd = torch.empty(M_HEAD, Nd, dtype=torch.bfloat16, device=dev)
    ev = []

    def step(i, record=False):
        (wg_q, wg_s), (wd_q, wd_s) = sets[i % 2]
        w8.quant_act_token(x, out=qx)
        if record:
            a, b = _events()
            a.record()
        w8.gemm_w8a8_channel(qx[0], qx[1], wg_q, wg_s, out=yg)
        if record:
            b.record()
            ev.append((a, b))
        w8.quant_act_token(h, out=qh)
        w8.gemm_w8a8_channel(qh[0], qh[1], wd_q, wd_s, out=yd)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, record=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    ops = 2.0 * M_HEAD * (Ng * Kg + Nd * Kd)
    tops = ops / (ms * 1e-3) / 1e12
    k_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    k_tops = 2.0 * M_HEAD * Ng * Kg / (k_ms * 1e-3) / 1e12
    # per-kernel split of one step (events around each call)
    parts = {}
    for name, fn in (("quant_act_token_x", lambda i: w8.quant_act_token(x, out=qx)),
                     ("gemm_channel_gate_up", lambda i: w8.gemm_w8a8_channel(qx[0], qx[1], sets[i][0][0], sets[i][0][1], out=yg)),
                     ("quant_act_token_h", lambda i: w8.quant_act_token(h, out=qh)),
                     ("gemm_channel_down", lambda i: w8.gemm_w8a8_channel(qh[0], qh[1], sets[i][1][0], sets[i][1][1], out=yd))):
        parts[name] = round(time_calls(fn, 2, 10), 4)
    del sets
    torch.cuda.empty_cache()
    return ms, tops, k_ms, k_tops, parts


def _smi_sample():
    """GFX clocks (MHz, one per XCD) and socket power (W) from amd-smi."""
    import re
    import shutil
    import subprocess
    exe = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if exe is None:
        return None
    try:
        txt = subprocess.run([exe, "metric", "-g", "0", "-c", "-p"], capture_output=True, text=True,
                             timeout=20).stdout
    except Exception:                                           # pragma: no cover
        return None
    clocks, power, in_gfx = [], None, False
    for line in txt.splitlines():
        t = line.strip()
        if re.match(r"GFX_\d+:", t):
            in_gfx = True
        elif re.match(r"[A-Z]+_\d+:", t) or t.startswith("MEM"):
            in_gfx = False
        m = re.match(r"CLK:\s*(\d+)\s*MHz", t)
        if m and in_gfx:
            clocks.append(int(m.group(1)))
        m = re.match(r"SOCKET_POWER:\s*(\d+)", t)
        if m:
            power = int(m.group(1))
    return (clocks, power) if clocks else None


def clock_window(seconds=4.0):
    """The gate_up GEMM back to back for about `seconds` while a thread
    samples amd-smi three times inside that window: mean GFX clock, socket
    power, and the GEMM's rate in the same window."""
    import threading
    import torch
    import synth
    import w8a8_int8_quantized_amd as w8
    dev = torch.device("cuda:0")
    (K, N) = GATE_UP
    qa = w8.quant_act_token(synth.activations(M_HEAD, K, seed=synth.SEEDS["channel"], device=dev))
    wq = w8.quant_act_token(synth.weights(N, K, seed=synth.SEEDS["channel"] + 20, device=dev))
    y = torch.empty(M_HEAD, N, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        w8.gemm_w8a8_channel(qa[0], qa[1], wq[0], wq[1], out=y)
    torch.cuda.synchronize()
    a, b = _events()
    a.record()
    w8.gemm_w8a8_channel(qa[0], qa[1], wq[0], wq[1], out=y)
    b.record()
    torch.cuda.synchronize()
    n = max(1, int(seconds / max(a.elapsed_time(b) * 1e-3, 1e-4)))
    samples = []

    def sampler():
        time.sleep(0.5)
        for _ in range(3):
            r = _smi_sample()
            if r is not None:
                samples.append(r)
            time.sleep(0.3)

    th = threading.Thread(target=sampler)
    th.start()
    a.record()
    for _ in range(n):
        w8.gemm_w8a8_channel(qa[0], qa[1], wq[0], wq[1], out=y)
    b.record()
    th.join()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    del qa, wq, y
    torch.cuda.empty_cache()
    out = {"gate_up_ms": round(ms, 4), "gate_up_tops": round(2.0 * M_HEAD * N * K / ms / 1e9, 1),
           "window_s": round(ms * n / 1e3, 2)}
    if not samples:
        out["source"] = "amd-smi unavailable"
        return out
    clocks = [c for cl, _ in samples for c in cl]
    powers = [p for _, p in samples if p is not None]
    out.update({"source": "amd-smi metric -c -p, 3 samples while the gate_up GEMM runs back to back",
                "gfx_mhz_mean": round(sum(clocks) / len(clocks)), "gfx_mhz_min": min(clocks),
                "gfx_mhz_max": max(clocks),
                "socket_power_w": round(sum(powers) / len(powers)) if powers else None})
    return out


def rows(args):
    """Every other row of the path at its own shapes."""
    import torch
    import synth
    import w8a8_int8_quantized_amd as w8

    dev = torch.device("cuda:0")
    R = args.rows_reps
    out = {}

    def gemm_entry(ms, M, N, K, wbytes):
        ops = 2.0 * M * N * K
        byts = wbytes + M * K + 2 * M * N
        return {"ms": round(ms, 4), "TOPS": round(ops / ms / 1e9, 1),
                "mfma_frac": round(ops / ms / 1e9 / PEAK_INT8_TOPS, 3),
                "GBps": round(byts / ms / 1e6, 1), "hbm_frac": round(byts / ms / 1e6 / PEAK_HBM_GBS, 3)}

    groups = args.rows_only.split(",") if args.rows_only else None

    def want(g):
        return groups is None or g in groups

    if want("quant"):
        # --- quantisers at M = 4096, K = 7168 (bytes: 2 in + 1 out + scales),
        # 12 input and output copies (1.06 GB) rotated
        NQ = 12
        xs = [synth.activations(4096, 7168, seed=2 + i, device=dev) for i in range(NQ)]
        qs = [torch.empty(4096, 7168, dtype=torch.int8, device=dev) for _ in range(NQ)]
        sg = [torch.empty(4096, 56, dtype=torch.float32, device=dev) for _ in range(NQ)]
        st_ = [torch.empty(4096, dtype=torch.float32, device=dev) for _ in range(NQ)]
        ms = time_calls(lambda i: w8.quant_act_group(xs[i], out=(qs[i], sg[i])), NQ, R)
        b = 4096 * 7168 * 3 + 4096 * 56 * 4
        out["quant_act_group_4096x7168"] = {"ms": round(ms, 4), "GBps": round(b / ms / 1e6, 1),
                                            "hbm_frac": round(b / ms / 1e6 / PEAK_HBM_GBS, 3)}
        ms = time_calls(lambda i: w8.quant_act_token(xs[i], out=(qs[i], st_[i])), NQ, R)
        b = 4096 * 7168 * 3 + 4096 * 4
        out["quant_act_token_4096x7168"] = {"ms": round(ms, 4), "GBps": round(b / ms / 1e6, 1),
                                            "hbm_frac": round(b / ms / 1e6 / PEAK_HBM_GBS, 3)}
        del xs, qs, sg, st_
        torch.cuda.empty_cache()

    if want("tile"):
        # --- block-wise at M = 4096 (DeepSeek-V3 shapes), weights FP8 -> requantised
        qa_cache = {}
        for name in ("gate_up", "down", "q_a", "q_b", "kv_a"):
            K, N = synth.SHAPES[name]
            codes, si = synth.fp8_weights(N, K, seed=synth.SEEDS["block"], device=dev)
            if name == "gate_up":
                # two sets of codes and outputs rotated (2 x 529 MB of traffic per pair of calls)
                codes2 = [codes, synth.fp8_weights(N, K, seed=synth.SEEDS["block"] + 50, device=dev)[0]]
                outs2 = [(torch.empty(N, K, dtype=torch.int8, device=dev),
                          torch.empty((N + 127) // 128, K // 128, dtype=torch.float32, device=dev)) for _ in range(2)]
                ms = time_calls(lambda i: w8.requant_fp8_to_int8_block(codes2[i], si, out=outs2[i]), 2, 6)
                b = N * K * 2
                out["requant_fp8_block_gate_up"] = {"ms": round(ms, 4), "GBps": round(b / ms / 1e6, 1),
                                                    "hbm_frac": round(b / ms / 1e6 / PEAK_HBM_GBS, 3)}
                del codes2, outs2
            wq, ws = w8.requant_fp8_to_int8_block(codes, si)
            del codes
            if K not in qa_cache:
                xa = synth.activations(4096, K, seed=synth.SEEDS["block"] + 1, device=dev)
                qa_cache[K] = w8.quant_act_group(xa)
                del xa
            qa, sa = qa_cache[K]
            y = torch.empty(4096, N, dtype=torch.bfloat16, device=dev)
            ms = time_calls(lambda i: w8.gemm_w8a8_block(qa, sa, wq, ws, out=y), 1, max(5, R // 2))
            out[f"gemm_block_m4096_{name}"] = gemm_entry(ms, 4096, N, K, N * K)
            if name == "gate_up":
                # the next layer's group quantisation fused into the epilogue,
                # against the GEMM (bf16) followed by quant_act_group
                qo = (torch.empty(4096, N, dtype=torch.int8, device=dev),
                      torch.empty(4096, N // 128, dtype=torch.float32, device=dev))
                ms_f = time_calls(lambda i: w8.gemm_w8a8_block_quant(qa, sa, wq, ws, out=qo), 1, max(5, R // 2))
                ms_u = time_calls(lambda i: (w8.gemm_w8a8_block(qa, sa, wq, ws, out=y), w8.quant_act_group(y, out=qo)),
                                  1, max(5, R // 2))
                out["fused_block_quant_m4096_gate_up"] = {"ms": round(ms_f, 4), "unfused_ms": round(ms_u, 4),
                                                          "TOPS": round(2.0 * 4096 * N * K / ms_f / 1e9, 1)}
                del qo
            if name in ("gate_up", "down"):
                qt = w8.quant_act_token(synth.activations(4096, K, seed=5, device=dev))
                # weight copies rotated through more than 1 GB (4 of gate_up's
                # 264 MB, 8 of down's 132 MB): the M = 128 rows are HBM-bound
                nrot = 4 if name == "gate_up" else 8
                wcs = [w8.quant_act_token(synth.weights(N, K, seed=6 + i, device=dev)) for i in range(nrot)]
                ms = time_calls(lambda i: w8.gemm_w8a8_channel(qt[0], qt[1], wcs[i][0], wcs[i][1], out=y), nrot,
                                max(5, R // 2))
                out[f"gemm_channel_m4096_{name}"] = gemm_entry(ms, 4096, N, K, N * K)
                for M in (128, 1024):
                    yq = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
                    a0, a1 = qt[0][:M].contiguous(), qt[1][:M].contiguous()
                    ms = time_calls(lambda i: w8.gemm_w8a8_channel(a0, a1, wcs[i][0], wcs[i][1], out=yq), nrot, R)
                    out[f"gemm_channel_m{M}_{name}"] = gemm_entry(ms, M, N, K, N * K)
                del wcs, qt
            del wq, ws, y
        del qa_cache
        torch.cuda.empty_cache()

    if want("decode"):
        # --- decode block-wise: M in {1, 8, 32, 64}, K = 7168, N = 36864, 4 weight copies (1.06 GB)
        K, N = GATE_UP
        wsets = []
        for s in range(4):
            w = synth.weights(N, K, seed=synth.SEEDS["decode"] + s, device=dev)
            wsets.append(w8.quant_weight_block(w))
            del w
        for M in (1, 8, 32, 64):
            qa, sa = w8.quant_act_group(synth.activations(M, K, seed=M, device=dev))
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            ms = time_calls(lambda i: w8.gemm_w8a8_block(qa, sa, wsets[i][0], wsets[i][1], out=y), 4, R)
            e = gemm_entry(ms, M, N, K, N * K + 4 * ((N + 127) // 128) * (K // 128))
            out[f"decode_block_m{M}"] = e
            # the one-call linear layer: bf16 activations quantised online, then the same GEMM
            xb = synth.activations(M, K, seed=M, device=dev)
            wsp = torch.empty(w8.linear_workspace_bytes(w8.W8_SCHEME_BLOCK, M, K), dtype=torch.uint8, device=dev)
            ms = time_calls(lambda i: w8.linear_w8a8_block(xb, wsets[i][0], wsets[i][1], out=y, workspace=wsp), 4, R)
            out[f"decode_linear_block_m{M}"] = gemm_entry(ms, M, N, K, N * K + 4 * ((N + 127) // 128) * (K // 128))
            # the output quantised for the next layer: fused, and GEMM + quant_act_group
            qo = (torch.empty(M, N, dtype=torch.int8, device=dev), torch.empty(M, N // 128, dtype=torch.float32, device=dev))
            ms_f = time_calls(lambda i: w8.gemm_w8a8_block_quant(qa, sa, wsets[i][0], wsets[i][1], out=qo), 4, R)
            ms_u = time_calls(lambda i: (w8.gemm_w8a8_block(qa, sa, wsets[i][0], wsets[i][1], out=y),
                                         w8.quant_act_group(y, out=qo)), 4, R)
            e = gemm_entry(ms_f, M, N, K, N * K + 4 * ((N + 127) // 128) * (K // 128))
            e["unfused_ms"] = round(ms_u, 4)
            out[f"decode_fused_block_quant_m{M}"] = e
        del wsets
        torch.cuda.empty_cache()
        # --- the down projection of the same MLP at decode (K = 18432, N = 7168: the
        # split-K decode kernel, N giving no balanced shared grid), 8 weight copies (1.06 GB)
        K, N = DOWN
        wsets = []
        for s in range(8):
            w = synth.weights(N, K, seed=synth.SEEDS["decode"] + 10 + s, device=dev)
            wsets.append(w8.quant_weight_block(w))
            del w
        for M in (1, 8, 32, 64):
            qa, sa = w8.quant_act_group(synth.activations(M, K, seed=M + 100, device=dev))
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            ms = time_calls(lambda i: w8.gemm_w8a8_block(qa, sa, wsets[i][0], wsets[i][1], out=y), 8, R)
            out[f"decode_block_down_m{M}"] = gemm_entry(ms, M, N, K, N * K + 4 * ((N + 127) // 128) * (K // 128))
        del wsets
        torch.cuda.empty_cache()

    if want("asym"):
        # --- asymmetric per-tensor activations: quantiser (two passes over x;
        # algorithmic bytes 2 in + 1 out per element) and the GEMM at 4096 rows
        # and one row, gate_up shape, per-channel weights
        K, N = GATE_UP
        xs = [synth.activations(4096, K, seed=7 + i, device=dev) for i in range(12)]
        ms = time_calls(lambda i: w8.quant_act_asym(xs[i]), 12, R)
        x = xs[0]
        del xs[1:]
        b = 4096 * K * 3
        out["quant_act_asym_4096x7168"] = {"ms": round(ms, 4), "GBps": round(b / ms / 1e6, 1),
                                           "hbm_frac": round(b / ms / 1e6 / PEAK_HBM_GBS, 3)}
        qa, prm = w8.quant_act_asym(x)
        # four weight copies (1.06 GB) rotated: the one-row GEMM is HBM-bound
        wts = []
        for i in range(4):
            wq, wsc = w8.quant_act_token(synth.weights(N, K, seed=8 + i, device=dev))
            wts.append((wq, wsc, w8.weight_row_sums(wq)))
        y = torch.empty(4096, N, dtype=torch.bfloat16, device=dev)
        ms = time_calls(lambda i: w8.gemm_w8a8_asym(qa, prm, *wts[i], out=y), 4, max(5, R // 2))
        out["gemm_asym_m4096_gate_up"] = gemm_entry(ms, 4096, N, K, N * K)
        y1 = torch.empty(1, N, dtype=torch.bfloat16, device=dev)
        a1 = qa[:1].contiguous()
        ms = time_calls(lambda i: w8.gemm_w8a8_asym(a1, prm, *wts[i], out=y1), 4, R)
        out["decode_asym_m1_gate_up"] = gemm_entry(ms, 1, N, K, N * K + 8 * N)
        del x, qa, wts, y
        torch.cuda.empty_cache()

    if want("w8a16"):
        # --- decode W8A16: Qwen3-8B-shaped linears, 20 weight copies (> 1 GB)
        for name in ("w8a16_qkv", "w8a16_down"):
            K, N = synth.SHAPES[name]
            ws_ = []
            for s in range(20):
                w = synth.weights(N, K, seed=40 + s, device=dev, dtype=torch.float16)
                ws_.append(w8.quant_act_group(w))
                del w
            for M in (1, 8, 32, 64):
                xx = synth.activations(M, K, seed=M, device=dev, dtype=torch.float16)
                y = torch.empty(M, N, dtype=torch.float16, device=dev)
                ms = time_calls(lambda i: w8.gemm_w8a16_group(xx, ws_[i][0], ws_[i][1], out=y), 20, R)
                byts = N * K + 4 * N * (K // 128) + 2 * M * K + 2 * M * N
                out[f"decode_w8a16_{name}_m{M}"] = {"ms": round(ms, 4), "GBps": round(byts / ms / 1e6, 1),
                                                    "hbm_frac": round(byts / ms / 1e6 / PEAK_HBM_GBS, 3)}
            del ws_
        torch.cuda.empty_cache()
        # --- decode W4A16: the same linears with INT4 group-wise weights
        # (packed two per byte), 40 weight copies (> 1 GB)
        for name in ("w8a16_qkv", "w8a16_down"):
            K, N = synth.SHAPES[name]
            ws_ = []
            for s in range(40):
                w = synth.weights(N, K, seed=40 + s, device=dev, dtype=torch.float16)
                ws_.append(w8.quant_weight_int4_group(w))
                del w
            for M in (1, 8, 32, 64):
                xx = synth.activations(M, K, seed=M, device=dev, dtype=torch.float16)
                y = torch.empty(M, N, dtype=torch.float16, device=dev)
                ms = time_calls(lambda i: w8.gemm_w4a16_group(xx, ws_[i][0], ws_[i][1], out=y), 40, R)
                byts = N * K // 2 + 4 * N * (K // 128) + 2 * M * K + 2 * M * N
                short = name.replace("w8a16_", "")
                out[f"decode_w4a16_{short}_m{M}"] = {"ms": round(ms, 4), "GBps": round(byts / ms / 1e6, 1),
                                                     "hbm_frac": round(byts / ms / 1e6 / PEAK_HBM_GBS, 3)}
            del ws_
        torch.cuda.empty_cache()

    if want("moe"):
        # --- MoE: 256 experts, top-8 of 4096 tokens
        E, T, TOPK = 256, 4096, 8
        logits = synth.router_logits(T, E, seed=synth.SEEDS["moe"], device=dev)
        rows_, _, offs = synth.route_topk(logits, TOPK)
        P = rows_.numel()
        for name in ("moe_gate_up", "moe_down"):
            K, N = synth.SHAPES[name]
            NB, KB = (N + 127) // 128, K // 128
            Wq = torch.empty(E, N, K, dtype=torch.int8, device=dev)
            Ws = torch.empty(E, NB, KB, dtype=torch.float32, device=dev)
            for e0 in range(0, E, 32):
                w = synth.weights(32 * N, K, seed=100 + e0, device=dev)
                q, s = w8.quant_weight_block(w)
                Wq[e0:e0 + 32] = q.view(32, N, K)
                Ws[e0:e0 + 32] = s.view(32, NB, KB)
                del w, q, s
            if name == "moe_gate_up":
                xt = synth.activations(T, K, seed=7, device=dev)
                qa, sa = w8.quant_act_group(xt[rows_].contiguous())
                del xt
            else:
                qa, sa = w8.quant_act_group(synth.activations(P, K, seed=8, device=dev))
            y = torch.empty(P, N, dtype=torch.bfloat16, device=dev)
            ms = time_calls(lambda i: w8.gemm_w8a8_block_grouped(qa, sa, Wq, Ws, offs, out=y), 1, 5, warm=1)
            ops = 2.0 * P * N * K
            byts = E * N * K + P * K + 2 * P * N
            out[f"gemm_block_grouped_{name}"] = {"ms": round(ms, 4), "TOPS": round(ops / ms / 1e9, 1),
                                                 "GBps": round(byts / ms / 1e6, 1),
                                                 "hbm_frac": round(byts / ms / 1e6 / PEAK_HBM_GBS, 3)}
            if name == "moe_gate_up":
                qo = (torch.empty(P, N, dtype=torch.int8, device=dev), torch.empty(P, N // 128, dtype=torch.float32,
                                                                                 device=dev))
                ms_f = time_calls(lambda i: w8.gemm_w8a8_block_grouped_quant(qa, sa, Wq, Ws, offs, out=qo), 1, 5, warm=1)
                ms_u = time_calls(lambda i: (w8.gemm_w8a8_block_grouped(qa, sa, Wq, Ws, offs, out=y),
                                             w8.quant_act_group(y, out=qo)), 1, 5, warm=1)
                out["fused_grouped_quant_moe_gate_up"] = {"ms": round(ms_f, 4), "unfused_ms": round(ms_u, 4),
                                                          "hbm_frac": round(byts / ms_f / 1e6 / PEAK_HBM_GBS, 3)}
                del qo
            del Wq, Ws, qa, sa, y
            torch.cuda.empty_cache()
    return out


def cpu_baseline():
    """The CPU oracle as it stands on the headline step itself (all 4096
    tokens, all output channels), median of 5 runs: about 15-20 s of CPU
    work on the host's threads."""
    import numpy as np
    import synth
    from oracle import gemm as ogemm, quant as oquant
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info())
    except Exception:                                           # pragma: no cover
        cores = os.cpu_count()
    Ms = 4096
    (Kg, Ng), (Kd, Nd) = GATE_UP, DOWN
    Ngs, Nds = Ng, Nd
    seed = synth.SEEDS["channel"]
    x = synth.to_numpy(synth.activations(Ms, Kg, seed=seed))
    h = synth.to_numpy(synth.activations(Ms, Kd, seed=seed + 10))
    wg = oquant.quant_act_token(synth.to_numpy(synth.weights(Ngs, Kg, seed=seed + 20)))
    wd = oquant.quant_act_token(synth.to_numpy(synth.weights(Nds, Kd, seed=seed + 30)))
    times = []
    for _ in range(5):
        t0 = time.perf_counter()
        qa, sa = oquant.quant_act_token(x)
        ogemm.gemm_channel(qa, sa, wg[0], wg[1])
        qh, sh = oquant.quant_act_token(h)
        ogemm.gemm_channel(qh, sh, wd[0], wd[1])
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    ops = 2.0 * Ms * (Ngs * Kg + Nds * Kd)
    return {"value": round(ops / t / 1e12, 4), "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"the full channel-wise MLP step ({Ms} tokens, gate_up N={Ngs}, down N={Nds}); "
                      f"median of 5 runs of {t:.2f} s",
            "seconds": round(t, 3), "cpu_model": _cpu_model(), "tiny": _oracle_tiny()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:                                             # pragma: no cover
        pass
    return "unknown"


def _oracle_tiny():
    """The oracle on the tiny block-wise case (16 tokens, K = 256 -> N = 256:
    group quantisation, tile quantisation of the weights, block-wise GEMM),
    median of 5 wall-clock runs in ms, with all BLAS threads and with one."""
    import numpy as np
    import synth
    from oracle import gemm as ogemm, quant as oquant
    x = synth.to_numpy(synth.activations(16, 256, seed=0, outlier_frac=0.01, outlier_factor=20.0))
    w = synth.to_numpy(synth.weights(256, 256, seed=1))

    def once():
        t0 = time.perf_counter()
        qa, sa = oquant.quant_act_group(x)
        qw, sw = oquant.quant_weight_block(w)
        ogemm.gemm_block(qa, sa, qw, sw)
        return (time.perf_counter() - t0) * 1e3

    out = {"workload": "M=16, K=256, N=256 block-wise (quantisers + GEMM)",
           "ms_all_threads": round(float(np.median([once() for _ in range(5)])), 3)}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            out["ms_1_thread"] = round(float(np.median([once() for _ in range(5)])), 3)
    except Exception:                                           # pragma: no cover
        out["ms_1_thread"] = None
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": src.numel() * 4}))
        return
    print(f"[bench] headline: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    ms, tops, k_ms, k_tops, parts = headline(args)
    print(f"[bench] headline {ms:.3f} ms/step, {tops:.1f} TOPS; gate_up kernel {k_ms:.3f} ms", file=sys.stderr,
          flush=True)
    clock = None
    if not args.no_clock:
        print("[bench] clock window", file=sys.stderr, flush=True)
        clock = clock_window()
    extra = {}
    if not args.no_rows:
        print("[bench] rows", file=sys.stderr, flush=True)
        extra = rows(args)
    cpu = None
    if not args.no_cpu:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    Kg, Ng = GATE_UP
    traffic = TRAFFIC_GATE_UP_BYTES
    line = {
        "metric": "int8 GEMM TOPS and % of MI355X int8 peak (M=4096); decode GB/s % HBM",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "DeepSeek-V3 dense MLP, channel-wise W8A8: per-token quant + gate_up "
                               "(K=7168 -> N=36864) + per-token quant + down (K=18432 -> N=7168)",
                   "M": M_HEAD, "gate_up": [Kg, Ng], "down": list(DOWN), "out_dtype": "bf16",
                   "parallelism": "1 GPU"},
        "roofline": {"bound": "mfma", "achieved": round(k_tops, 1), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                     "frac": round(k_tops / PEAK_INT8_TOPS, 4), "traffic": traffic,
                     "kernel": "gemm_w8a8_channel gate_up M=4096", "kernel_ms": round(k_ms, 4),
                     "peak_note": "dense int8 MFMA, 5.0 POP/s at 2.4 GHz (int8 ops, not flops)"},
        "clock": clock,
        "cpu_baseline": cpu,
        "step_parts_ms": parts,
        "rows": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
