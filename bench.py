"""Benchmark of the MXFP8 hot path on one MI355X (gfx950).

One step is one pass of the whole hot path over one Qwen3 layer's worth of
synthetic input ("End-to-End MXFP8 Reinforcement Learning on Blackwell":
Figure 1 for the path, Table 2 for the models and token counts, Table 7 for
the ~4.5k-token dense break-even that sets M = 4608):

  1. weight sync of a Qwen3-8B decoder layer: row-wise and column-wise MXFP8
     quantization of q, k, v, o, gate, up, down, plus scale rearrangement;
  2. dense forward at 4608 tokens: quantize X_h, X_i row-wise, rearrange,
     GEMMs qkv / o / gate_up / down against the row-wise weights of step 1;
  3. dense backward of gate_up at 12288 tokens: dY row-wise and column-wise,
     X column-wise; dgrad = dY . W (column-wise weights of step 1) and
     wgrad = dY^T . X;
  4. Qwen3-30B-A3B MoE layer: 20480 tokens x top-8 = 163840 routed rows over
     128 experts with Zipf(1.1) loads; expert weights quantized in both
     orientations (one dual pass over all experts); dispatch (rows sorted by
     expert, gathered and quantized), grouped gate_up, SwiGLU fused with the
     quantization of its output, grouped down, weighted combine;
  5. the same MoE layer's expert backward (Table 8's update_actor): per
     projection, dY row-wise for the data gradient dX = dY . W_g (grouped over
     rows, column-wise expert weights of step 4), dY and the forward input
     column-wise per expert into 256-aligned column ranges for the weight
     gradient dW_g = dY_g^T X_g (grouped over each expert's token range).  The
     forward input of down is step 4's SwiGLU output; that of gate_up, the
     expert-sorted BF16 rows, and the two dY are synthetic of their shapes.

Inputs are drawn once on the device (seeded, same distributions as the
parity tests' CPU draws) and stay resident in HBM; the timed region holds
only the library's kernels.  Prints ONE JSON line.
"""
import argparse
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, 8 TB/s
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 / MXFP8 matrix peak, 5.0 PFLOP/s
QUANT_BYTES_PER_ELEMENT = 2 + 1 + 1 / 32  # BF16 in, E4M3 out, E8M0 per 32
DUAL_BYTES_PER_ELEMENT = 2 + 2 * (1 + 1 / 32)  # one BF16 read, both orientations out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager launches only (no HIP graph replay of the step)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES between two device buffers (a plain copy of known "
                         "size, for scaling the HBM byte counters) and exit")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only time plain device copies and reads of 1 GiB (what this GPU's HBM "
                         "delivers to simple streaming kernels) and exit")
    ap.add_argument("--library-compare", type=int, default=0, metavar="CALLS",
                    help="only run the 12288x4096x24576 product (the dense data gradient) CALLS "
                         "times back to back with this library's MX GEMM and with torch's "
                         "hipBLASLt FP8 GEMM (per-tensor scales, no block scales), twice each, "
                         "print per-call times and exit (context for the matrix-core counters)")
    return ap.parse_args()


def library_compare(torch, mx, calls):
    """Back-to-back sequences of one dense product, this library's MX GEMM and
    hipBLASLt's per-tensor-scaled FP8 GEMM (torch._scaled_mm) on the same E4M3
    codes, alternating ours, hipBLASLt, ours, hipBLASLt; per sequence the
    per-call times (HIP events) and the median of its second half, after the
    clock has settled."""
    M, N, K = 12288, 4096, 24576
    g = torch.Generator(device="cuda").manual_seed(0)

    def operand(rows, std):
        x = (torch.randn(rows, K, device="cuda", generator=g) * std).to(torch.bfloat16)
        q, s = mx.mx_quantize_rowwise(x)
        return q, mx.mx_scale_swizzle(s)

    a, sa = operand(M, 1.0)
    b, sb = operand(N, 0.02)
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, mx.mx_gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda")
    a8, b8 = a.view(torch.float8_e4m3fn), b.view(torch.float8_e4m3fn)
    one = torch.ones((), device="cuda")
    fns = {"mx_gemm (MX block scales)": lambda: mx.mx_gemm(a, sa, b, sb, c=c, workspace=ws),
           "hipBLASLt torch._scaled_mm (per-tensor scales)":
               lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)}
    out = []
    for name in list(fns) * 2:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(calls):
            fns[name]()
            ev[i + 1].record()
        torch.cuda.synchronize()
        t = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(calls)]
        half = sorted(t[calls // 2:])
        med = half[len(half) // 2]
        out.append({"kernel": name, "us": [round(x, 1) for x in t], "median_second_half_us": round(med, 1),
                    "frac_of_5PF": round(2 * M * N * K / (med * 1e-6) / 5e15, 3)})
    return {"product": f"{M}x{N}x{K}", "sequences": out}


def hbm_probe(torch):
    """Best-of-10 bandwidth of plain streaming kernels over 1 GiB buffers:
    the runtime's device-to-device copy, an elementwise copy (torch's vectorized
    kernel) and a read-only reduction; read + written bytes / time."""
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    out = {}
    cases = (("runtime device copy", lambda: b.copy_(a), 2 * n),
             ("elementwise copy (x * 1)", lambda: torch.mul(a, 1.0, out=b), 2 * n),
             ("read-only reduction (sum)", lambda: a.sum(), n))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, fn, traffic in cases:
        best = float("inf")
        for _ in range(11):
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        out[name] = {"us": round(best * 1e3, 1), "GB/s": round(traffic / (best * 1e-3) / 1e9, 1)}
    return out


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_hbm_traffic_qwen3_layer.md")
GEMM_SOURCE = os.path.join(ROOT, "mxfp8_block_scaled_08_amd", "csrc", "mx_gemm.hip")


def measured_traffic():
    """HBM bytes per dense-GEMM launch from the committed counter summary, or
    None when the summary is missing or was taken on another kernel source
    (the summary records the source's SHA-256)."""
    import hashlib
    try:
        text = open(TRAFFIC_SUMMARY).read()
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source sha256") != src:
        return None
    try:
        return int(fields["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events around launches on the current stream, summed per category."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.totals = {}
        self.counts = {}

    def __call__(self, cat, fn, *a, **kw):
        t = self.torch
        s = t.cuda.Event(enable_timing=True)
        e = t.cuda.Event(enable_timing=True)
        s.record()
        out = fn(*a, **kw)
        e.record()
        self.pending.append((cat, s, e))
        return out

    def collect(self):
        for cat, s, e in self.pending:
            self.totals[cat] = self.totals.get(cat, 0.0) + s.elapsed_time(e)
            self.counts[cat] = self.counts.get(cat, 0) + 1
        self.pending = []


def build_workload(mx, torch, mxsynth):
    dev = "cuda"
    W = mxsynth.weight_sync(device=dev)
    xh, xi = mxsynth.dense_fwd_activations(device=dev)
    dy, xb = mxsynth.dense_bwd_inputs(device=dev)
    rows_per, a_gu, a_dn, w_gu, w_dn = mxsynth.moe_inputs(device=dev)
    del a_gu, a_dn  # the MoE pass starts from x_tok and the SwiGLU output instead
    dy_gu, dy_dn = mxsynth.moe_bwd_grads(device=dev)
    off = torch.from_numpy(mxsynth.offsets_from_rows(rows_per)).to(dev)
    ids, rw = mxsynth.moe_routing()
    x_tok = mxsynth.normal_bf16((ids.shape[0], w_gu.shape[2]), 1.0, 5300, device=dev)
    ids = torch.from_numpy(ids).to(dev).contiguous()
    rw = torch.from_numpy(rw).to(dev).contiguous()
    u8 = dict(dtype=torch.uint8, device=dev)
    swz = mx.mx_scale_swizzled_bytes

    o = {}
    # weight sync outputs: row-wise into the fused forward operands, column-wise
    # into the fused backward operand of gate_up
    o["qkv_q"] = torch.empty(6144, 4096, **u8)
    o["o_q"] = torch.empty(4096, 4096, **u8)
    o["gu_q"] = torch.empty(24576, 4096, **u8)
    o["dn_q"] = torch.empty(4096, 12288, **u8)
    o["guT_q"] = torch.empty(4096, 24576, **u8)
    o["colT"] = {n: torch.empty(W[n].shape[1], W[n].shape[0], **u8)
                 for n in ("q", "k", "v", "o", "down")}
    for name, (r, c) in (("qkv", (6144, 4096)), ("o", (4096, 4096)), ("gu", (24576, 4096)),
                         ("dn", (4096, 12288)), ("guT", (4096, 24576))):
        o[name + "_swz"] = torch.empty(swz(r, c // 32), **u8)
    o["colT_swz"] = {n: torch.empty(swz(W[n].shape[1], W[n].shape[0] // 32), **u8)
                     for n in o["colT"]}
    # activations
    for name, x in (("xh", xh), ("xi", xi)):
        o[name + "_q"] = torch.empty(x.shape, **u8)
        o[name + "_swz"] = torch.empty(swz(x.shape[0], x.shape[1] // 32), **u8)
    o["dy_q"] = torch.empty(12288, 24576, **u8)
    o["dy_swz"] = torch.empty(swz(12288, 768), **u8)
    o["dyT_q"] = torch.empty(24576, 12288, **u8)
    o["dyT_swz"] = torch.empty(swz(24576, 384), **u8)
    o["xT_q"] = torch.empty(4096, 12288, **u8)
    o["xT_swz"] = torch.empty(swz(4096, 384), **u8)
    M = int(off[-1].item())
    G = w_gu.shape[0]
    k_cap = mx.mx_grouped_k_capacity(M, G)
    for name, w in (("mgu", w_gu), ("mdn", w_dn)):
        G, N, K = w.shape
        # expert weights, both orientations: [G][N][K] and [G][K][N], scales
        # rearranged per expert, back to back
        o[name + "_wq"] = torch.empty(G, N, K, **u8)
        o[name + "_wswz"] = torch.empty(G * swz(N, K // 32), **u8)
        o[name + "_wqt"] = torch.empty(G, K, N, **u8)
        o[name + "_wstswz"] = torch.empty(G * swz(K, N // 32), **u8)
        # backward: dY [M][N] row-wise (data gradient), dY and the forward
        # input column-wise per expert (weight gradient)
        o[name + "_dyq"] = torch.empty(M, N, **u8)
        o[name + "_dyswz"] = torch.empty(swz(M, N // 32), **u8)
        o[name + "_dyT"] = torch.empty(N, k_cap, **u8)
        o[name + "_dyTswz"] = torch.empty(swz(N, k_cap // 32), **u8)
        o[name + "_xT"] = torch.empty(K, k_cap, **u8)
        o[name + "_xTswz"] = torch.empty(swz(K, k_cap // 32), **u8)
        o[name + "_pad"] = torch.empty(G + 1, dtype=torch.int64, device=dev)
        o[name + "_pad2"] = torch.empty(G + 1, dtype=torch.int64, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    o["C_qkv"] = torch.empty(4608, 6144, **bf)
    o["C_o"] = torch.empty(4608, 4096, **bf)
    o["C_gu"] = torch.empty(4608, 24576, **bf)
    o["C_dn"] = torch.empty(4608, 4096, **bf)
    o["C_dgrad"] = torch.empty(12288, 4096, **bf)
    o["C_wgrad"] = torch.empty(24576, 4096, **bf)
    o["C_mgu"] = torch.empty(M, 1536, **bf)
    o["C_mdn"] = torch.empty(M, 2048, **bf)
    o["dX_mgu"] = torch.empty(M, 2048, **bf)
    o["dX_mdn"] = torch.empty(M, 768, **bf)
    o["dW_mgu"] = torch.empty(G, 1536, 2048, **bf)
    o["dW_mdn"] = torch.empty(G, 2048, 768, **bf)
    # MoE forward through dispatch, SwiGLU and combine
    n_assign = ids.numel()
    o["moff"] = torch.empty(G + 1, dtype=torch.int64, device=dev)
    o["xq"] = torch.empty(M, 2048, **u8)                 # dispatched rows, quantized
    o["xswz"] = torch.empty(swz(M, 2048 // 32), **u8)
    o["msrc"] = torch.empty(n_assign, dtype=torch.int32, device=dev)
    o["mslot"] = torch.empty(n_assign, dtype=torch.int32, device=dev)
    o["hq"] = torch.empty(M, 768, **u8)
    o["hswz"] = torch.empty(swz(M, 768 // 32), **u8)
    o["moe_out"] = torch.empty(ids.shape[0], 2048, **bf)
    # one scratch buffer for every call that takes a workspace (split-tail
    # GEMMs, the dispatch's chunk counts, the weight gradients' tile counter):
    # the step runs on one stream, so the calls never overlap in time
    gemm_ws = max(mx.mx_gemm_workspace_bytes(m, n, k) for m, n, k in
                  ((4608, 6144, 4096), (4608, 4096, 4096), (4608, 24576, 4096), (4608, 4096, 12288),
                   (12288, 4096, 24576), (24576, 4096, 12288)))
    o["ws"] = torch.empty(max(gemm_ws, mx.mx_moe_dispatch_workspace_bytes(ids.shape[0], ids.shape[1], G),
                              mx.mx_grouped_gemm_wgrad_workspace_bytes()), **u8)
    assert n_assign == M
    inputs = dict(W=W, xh=xh, xi=xi, dy=dy, x=xb, off=off,
                  w_gu=w_gu, w_dn=w_dn, dy_gu=dy_gu, dy_dn=dy_dn, M=M, k_cap=k_cap,
                  x_tok=x_tok, ids=ids, rw=rw)
    return inputs, o


def step(mx, I, o, T):
    """One pass of the hot path; T(category, fn, ...) times each launch."""
    W = I["W"]
    # 1. weight sync: both orientations of every weight in one pass each, the
    #    row-wise codes into the fused forward operands (q, k, v stacked; gate,
    #    up stacked) and the column-wise ones into the backward operands (gate
    #    and up side by side along K), scales straight into the GEMM layout
    dq = mx.mx_quantize_dual
    t16 = 4096 // 256  # rearranged tiles per row of a K = 4096 operand
    jobs = []
    for name, r0, r1 in (("q", 0, 4096), ("k", 4096, 5120), ("v", 5120, 6144)):
        jobs.append(dict(x=W[name], q=o["qkv_q"][r0:r1], s_swz=o["qkv_swz"][(r0 // 32) * t16 * 256:],
                         s_tiles=t16, qt=o["colT"][name], st_swz=o["colT_swz"][name]))
    jobs.append(dict(x=W["o"], q=o["o_q"], s_swz=o["o_swz"], qt=o["colT"]["o"],
                     st_swz=o["colT_swz"]["o"]))
    for name, r0, r1 in (("gate", 0, 12288), ("up", 12288, 24576)):
        jobs.append(dict(x=W[name], q=o["gu_q"][r0:r1], s_swz=o["gu_swz"][(r0 // 32) * t16 * 256:],
                         s_tiles=t16, qt=o["guT_q"][:, r0:r1],
                         st_swz=o["guT_swz"][(r0 // 256) * 256:], st_tiles=24576 // 256))
    jobs.append(dict(x=W["down"], q=o["dn_q"], s_swz=o["dn_swz"], qt=o["colT"]["down"],
                     st_swz=o["colT_swz"]["down"]))
    T("quant_dual", mx.mx_quantize_dual_batch, jobs)
    # 2. dense forward, M = 4608: both activations in one launch
    T("quant_row", mx.mx_quantize_rowwise_swz_batch,
      [dict(x=I[name], q=o[name + "_q"], s_swz=o[name + "_swz"]) for name in ("xh", "xi")])
    g = mx.mx_gemm
    T("gemm", g, o["xh_q"], o["xh_swz"], o["qkv_q"], o["qkv_swz"], c=o["C_qkv"], workspace=o["ws"])
    T("gemm", g, o["xh_q"], o["xh_swz"], o["o_q"], o["o_swz"], c=o["C_o"], workspace=o["ws"])
    T("gemm", g, o["xh_q"], o["xh_swz"], o["gu_q"], o["gu_swz"], c=o["C_gu"], workspace=o["ws"])
    T("gemm", g, o["xi_q"], o["xi_swz"], o["dn_q"], o["dn_swz"], c=o["C_dn"], workspace=o["ws"])
    # 3. dense backward of gate_up, 12288 tokens
    T("quant_dual", dq, I["dy"], q=o["dy_q"], s_swz=o["dy_swz"], qt=o["dyT_q"],
      st_swz=o["dyT_swz"])
    T("quant_col", mx.mx_quantize_colwise_swz, I["x"], qt=o["xT_q"], st_swz=o["xT_swz"])
    T("gemm", g, o["dy_q"], o["dy_swz"], o["guT_q"], o["guT_swz"], c=o["C_dgrad"], workspace=o["ws"])
    T("gemm", g, o["dyT_q"], o["dyT_swz"], o["xT_q"], o["xT_swz"], c=o["C_wgrad"], workspace=o["ws"])
    # 4. MoE layer: expert weights in both orientations, dispatch, gate_up,
    #    SwiGLU + quantize, down, combine
    for name, w in (("mgu", I["w_gu"]), ("mdn", I["w_dn"])):
        T("quant_dual", mx.mx_quantize_dual_experts, w, q=o[name + "_wq"], s_swz=o[name + "_wswz"],
          qt=o[name + "_wqt"], st_swz=o[name + "_wstswz"])
    # the dispatched rows quantized row-wise (gate_up's A) and per expert
    # column-wise (gate_up's weight-gradient operand) from one gather
    T("moe_dispatch", mx.mx_moe_dispatch_dual_grouped, I["x_tok"], I["ids"], I["w_gu"].shape[0],
      k_cap=I["k_cap"], offsets=o["moff"], src=o["msrc"], slot=o["mslot"], q=o["xq"], s_swz=o["xswz"],
      pad_offsets=o["mgu_pad2"], qt=o["mgu_xT"], st_swz=o["mgu_xTswz"], workspace=o["ws"])
    T("grouped_gemm", mx.mx_grouped_gemm, o["moff"], o["xq"], o["xswz"], o["mgu_wq"],
      o["mgu_wswz"], c=o["C_mgu"])
    # h = SwiGLU(gate, up) quantized row-wise (the down projection's A) and per
    # expert column-wise (its weight gradient's operand) from one read; h
    # itself is never written
    T("swiglu", mx.mx_swiglu_quantize_dual_grouped, o["C_mgu"], o["moff"], k_cap=I["k_cap"], q=o["hq"],
      s_swz=o["hswz"], qt=o["mdn_xT"], st_swz=o["mdn_xTswz"], pad_offsets=o["mdn_pad2"])
    T("grouped_gemm", mx.mx_grouped_gemm, o["moff"], o["hq"], o["hswz"], o["mdn_wq"],
      o["mdn_wswz"], c=o["C_mdn"])
    T("moe_combine", mx.mx_moe_combine, o["C_mdn"], o["mslot"], I["rw"], out=o["moe_out"])
    # 5. MoE expert backward: data gradient grouped over rows, weight gradient
    #    grouped over each expert's token range
    k_cap = I["k_cap"]
    for name, dyp in (("mgu", I["dy_gu"]), ("mdn", I["dy_dn"])):
        # dY row-wise (data gradient) and per expert column-wise (weight
        # gradient) from one read
        T("quant_dual_grouped", mx.mx_quantize_dual_grouped, dyp, I["off"], k_cap=k_cap,
          q=o[name + "_dyq"], s_swz=o[name + "_dyswz"], qt=o[name + "_dyT"], st_swz=o[name + "_dyTswz"],
          pad_offsets=o[name + "_pad"])
        T("grouped_gemm", mx.mx_grouped_gemm, I["off"], o[name + "_dyq"], o[name + "_dyswz"],
          o[name + "_wqt"], o[name + "_wstswz"], c=o["dX_" + name])
        # the weight gradient's other operand (X for gate_up, h for down) was
        # quantized per expert column-wise in the forward (dispatch, SwiGLU)
        T("grouped_wgrad", mx.mx_grouped_gemm_wgrad, o[name + "_pad"], o[name + "_dyT"],
          o[name + "_dyTswz"], o[name + "_xT"], o[name + "_xTswz"], c=o["dW_" + name], workspace=o["ws"])


def work_per_step(I):
    """Algorithmic work of one step: elements quantized per orientation (those
    quantized in both orientations by one dual pass counted in each), GEMM
    FLOPs (dense and grouped)."""
    W = I["W"]
    dual_el = sum(w.numel() for w in W.values())                 # weight sync, both
    dual_el += I["dy"].numel()                                   # dgrad + wgrad operand
    dual_el += I["w_gu"].numel() + I["w_dn"].numel()             # MoE expert weights
    row_el = dual_el + I["xh"].numel() + I["xi"].numel()         # + forward activations
    col_el = dual_el + I["x"].numel()                            # + wgrad activation operand
    # per-expert column-wise operands of the MoE weight gradients
    # per-expert column-wise operands of the MoE weight gradients: the
    # dispatched rows (2048 columns) and the SwiGLU output (768), both
    # quantized in the forward passes from rows they already read
    colg_el = I["M"] * (2048 + 768)
    colg_gu_el = 0
    # MoE output gradients: row-wise and per-expert column-wise from one read
    dualg_el = I["dy_gu"].numel() + I["dy_dn"].numel()
    M = I["M"]
    dense = (2 * 4608 * 6144 * 4096 + 2 * 4608 * 4096 * 4096 + 2 * 4608 * 24576 * 4096
             + 2 * 4608 * 4096 * 12288 + 2 * 12288 * 4096 * 24576 + 2 * 24576 * 4096 * 12288)
    grouped = 2 * (2 * M * 1536 * 2048 + 2 * M * 2048 * 768)   # forward + data gradient
    wgrad = 2 * M * 1536 * 2048 + 2 * M * 2048 * 768
    disp_el = M * 2048           # routed rows quantized and written
    # dispatch traffic: each token row read once (the gathers of its other
    # routed copies hit in cache), every routed row written row-wise and the
    # per-expert column-wise operand written (codes + scales), the routing ids
    # read and the slot / source-token indices written
    disp_bytes = (I["x_tok"].numel() * 2 + disp_el * (1 + 1 / 32)
                  + 2048 * I["k_cap"] * (1 + 1 / 32)   # the per-expert column-wise operand
                  + I["ids"].numel() * 4 * 3)
    swiglu_el = M * 768          # SwiGLU outputs, quantized
    comb_el = I["x_tok"].numel()  # combined outputs
    return dict(row_el=row_el, col_el=col_el, dual_el=dual_el, colg_el=colg_el, colg_gu_el=colg_gu_el,
                dualg_el=dualg_el,
                dense=dense,
                grouped=grouped, wgrad=wgrad, disp_el=disp_el, disp_bytes=disp_bytes, swiglu_el=swiglu_el,
                comb_el=comb_el, topk=I["ids"].shape[1])


# outputs compared between the eager step and a graph replay (every output of
# the step is deterministic; these cover each kind of launch)
GRAPH_CHECK = ("qkv_q", "qkv_swz", "guT_q", "xh_q", "xh_swz", "C_qkv", "C_dn", "C_dgrad", "C_wgrad",
               "moff", "xq", "C_mgu", "hq", "C_mdn", "moe_out", "dX_mgu", "dW_mgu", "dW_mdn",
               "mgu_wqt")


def graph_replay(torch, mx, I, o, noop, steps):
    """Capture one step into a HIP graph on the current (side) stream, check a
    replay byte-equal to the eager step's outputs, and time `steps` replays."""
    torch.cuda.synchronize()
    ref = {k: o[k].clone() for k in GRAPH_CHECK}
    g = torch.cuda.CUDAGraph()
    try:
        with torch.cuda.graph(g, stream=torch.cuda.current_stream()):
            step(mx, I, o, noop)
    except RuntimeError as e:  # report the eager timing instead
        torch.cuda.synchronize()
        return {"error": str(e)[:200], "bytes_equal_to_eager": False}
    for k in GRAPH_CHECK:
        o[k].view(torch.uint8).fill_(0xA5)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    equal = all(torch.equal(o[k].view(torch.uint8), ref[k].view(torch.uint8)) for k in GRAPH_CHECK)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return {"ms_per_step": round(start.elapsed_time(end) / steps, 4), "replays": steps,
            "bytes_equal_to_eager": bool(equal), "checked_outputs": len(GRAPH_CHECK)}


def cpu_baseline(torch, mxsynth, row_el, col_el, flops):
    """The CPU oracle (plain C, as it stands) on a bounded sample of the same
    workload, extrapolated to the step's work in the metric's unit: on all the
    host's usable cores (the sample split by rows over threads; the C calls
    release the GIL), and on one thread beside it."""
    import concurrent.futures as cf

    import numpy as np
    import oracle

    threads = min(len(os.sched_getaffinity(0)), 16)
    t0 = time.perf_counter()
    w = mxsynth.normal_bf16((1024, 4096), 0.02, 2004, 0.001, 20.0)
    wb = mxsynth.bits(w)
    xh = mxsynth.channel_outliers_bf16(64, 4096, 1.0, 3000, 0.005, 50.0)
    qa, sa = oracle.quantize_rowwise(mxsynth.bits(xh))
    qb, sb = oracle.quantize_rowwise(mxsynth.bits(
        mxsynth.normal_bf16((512, 4096), 0.02, 2000, 0.001, 20.0)))
    rows = np.repeat(np.arange(64), 512)
    cols = np.tile(np.arange(512), 64)

    def rates(n_threads, q_secs, g_secs):
        q_parts = np.array_split(np.arange(wb.shape[0]), n_threads)

        def quant(idx):
            part = np.ascontiguousarray(wb[idx[0]:idx[-1] + 1])
            oracle.quantize_rowwise(part)
            oracle.quantize_colwise(part)

        g_parts = np.array_split(np.arange(rows.size), n_threads)

        def gemm(idx):
            oracle.gemm_sampled(rows[idx], cols[idx], qa, sa, qb, sb)

        with cf.ThreadPoolExecutor(max_workers=n_threads) as ex:
            t, n_q = time.perf_counter(), 0
            while time.perf_counter() - t < q_secs:
                list(ex.map(quant, q_parts))
                n_q += 1
            q_time = time.perf_counter() - t
            t, n_g = time.perf_counter(), 0
            while time.perf_counter() - t < g_secs:
                list(ex.map(gemm, g_parts))
                n_g += 1
            g_time = time.perf_counter() - t
        q_rate = n_q * wb.size / q_time * 2          # element-orientations per second
        g_rate = n_g * 2 * rows.size * 4096 / g_time  # FLOP/s
        step_s = (row_el + col_el) / q_rate + flops / g_rate
        return q_rate, g_rate, step_s, n_q, n_g, q_time, g_time

    def record(n_threads, q_secs, g_secs):
        q_rate, g_rate, step_s, n_q, n_g, q_time, g_time = rates(n_threads, q_secs, g_secs)
        return {
            "value": flops / step_s / 1e12,
            "unit": "TFLOP/s",
            "cores": n_threads,
            "kind": "oracle",
            "sample": (f"row+column quantize of a 1024x4096 weight ({n_q} passes, {q_time:.1f} s: "
                       f"{q_rate / 1e6:.1f} M element-orientations/s) and FP64 GEMM of a 64x512x4096 "
                       f"slice of the forward qkv product ({n_g} passes, {g_time:.1f} s: "
                       f"{g_rate / 1e9:.3f} GFLOP/s), {n_threads} thread(s); step time extrapolated to "
                       f"the full step ({step_s:.0f} s)"),
        }

    result = record(threads, 3.0, 5.0)
    result["single_thread"] = record(1, 3.0, 5.0)
    result["wall_s"] = round(time.perf_counter() - t0, 1)
    result["host_cpu"] = platform.processor() or platform.machine()
    result["host_nproc"] = os.cpu_count()
    result["host_usable_cores"] = len(os.sched_getaffinity(0))
    return result


def _ulp_bf16(y):
    import numpy as np
    a = np.abs(y)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -126)
    return np.where(a > 0, np.ldexp(1.0, (e - 7).astype(int)), 2.0 ** -133)


def oracle_parity(torch, mx, mxsynth, I, o):
    """GEMM outputs of the timed step against the CPU oracle on bounded
    samples (256 entries per product, every product of the step), and the
    Tiny workload (128x256x256) in full: how many meet the stated bar
    |C - C_ref| <= 1e-5 (|A||B|)_ij + 1 BF16 ulp, and the largest error beyond
    the ulp allowance relative to (|A||B|)_ij.  The oracle sees the GPU's
    quantized operands (their bytes are checked against the oracle by the
    test suite)."""
    import numpy as np
    import oracle

    rng = np.random.default_rng(77)

    def host(t):
        return t.cpu().numpy()

    def unswz(buf, rows, kb):
        return oracle.scale_unswizzle(host(buf), rows, kb)

    def stats(got, ref, bnd):
        err = np.abs(got - ref)
        net = np.maximum(err - _ulp_bf16(ref), 0.0) / np.where(bnd > 0, bnd, np.inf)
        return {"n": int(got.size), "within_stated": int((err <= 1e-5 * bnd + _ulp_bf16(ref)).sum()),
                "max_err_over_bnd": float(net.max())}

    def pairs(C, r, c, qa_rows, sa_rows, qb_rows, sb_rows):
        n = len(r)
        ref, bnd = oracle.gemm_sampled(np.arange(n), np.arange(n), qa_rows, sa_rows, qb_rows, sb_rows)
        got = C[torch.from_numpy(np.asarray(r)).cuda(), torch.from_numpy(np.asarray(c)).cuda()]
        return stats(got.float().cpu().numpy().astype(np.float64), ref, bnd)

    out = {}
    # Tiny: A[128x256] row-wise, B[256x256] column-wise, BF16 out, every output
    A, B = mxsynth.tiny()
    qa, sa = mx.mx_quantize_rowwise(A.cuda())
    qbt, sbt = mx.mx_quantize_colwise(B.cuda())
    C = mx.mx_gemm(qa, mx.mx_scale_swizzle(sa), qbt, mx.mx_scale_swizzle(sbt))
    ref, bnd = oracle.gemm(host(qa), host(sa), host(qbt), host(sbt))
    out["tiny"] = stats(C.float().cpu().numpy().astype(np.float64), ref, bnd)
    # dense products of the step
    dense = {"qkv": ("xh", "qkv", "C_qkv"), "o": ("xh", "o", "C_o"), "gate_up": ("xh", "gu", "C_gu"),
             "down": ("xi", "dn", "C_dn"), "dgrad": ("dy", "guT", "C_dgrad"), "wgrad": ("dyT", "xT", "C_wgrad")}
    for name, (an, bn, cn) in dense.items():
        a_q, b_q, C = o[an + "_q"], o[bn + "_q"], o[cn]
        M, K = a_q.shape
        N = b_q.shape[0]
        r, c = rng.integers(0, M, 256), rng.integers(0, N, 256)
        sa_, sb_ = unswz(o[an + "_swz"], M, K // 32), unswz(o[bn + "_swz"], N, K // 32)
        out[name] = pairs(C, r, c, host(a_q[torch.from_numpy(r).cuda()]), sa_[r],
                          host(b_q[torch.from_numpy(c).cuda()]), sb_[c])
    # row-grouped MoE products: forward gate_up / down, data gradients
    G = I["w_gu"].shape[0]
    grouped = {"moe_gate_up": ("moff", "xq", "xswz", "mgu_wq", "mgu_wswz", "C_mgu"),
               "moe_down": ("moff", "hq", "hswz", "mdn_wq", "mdn_wswz", "C_mdn"),
               "moe_dgrad_gate_up": (None, "mgu_dyq", "mgu_dyswz", "mgu_wqt", "mgu_wstswz", "dX_mgu"),
               "moe_dgrad_down": (None, "mdn_dyq", "mdn_dyswz", "mdn_wqt", "mdn_wstswz", "dX_mdn")}
    for name, (offn, an, asn, bn, bsn, cn) in grouped.items():
        off = host(o[offn]) if offn else host(I["off"])
        a_q, C = o[an], o[cn]
        K = a_q.shape[1]
        Gb, N, Kb = o[bn].shape
        assert Gb == G and Kb == K
        r = rng.integers(0, int(off[-1]), 256)
        c = rng.integers(0, N, 256)
        g = np.searchsorted(off, r, side="right") - 1
        sa_ = unswz(o[asn], a_q.shape[0], K // 32)
        per = mx.mx_scale_swizzled_bytes(N, K // 32)
        bsw = host(o[bsn]).reshape(G, per)
        sb_ = np.stack([oracle.scale_unswizzle(bsw[gi], N, K // 32)[ci] for gi, ci in zip(g, c)])
        qb_rows = host(o[bn][torch.from_numpy(g).cuda(), torch.from_numpy(c).cuda()])
        out[name] = pairs(C, r, c, host(a_q[torch.from_numpy(r).cuda()]), sa_[r], qb_rows, sb_)
    # K-grouped MoE weight gradients: C_g over expert g's column range
    for name, (an, bn, cn) in {"moe_wgrad_gate_up": ("mgu_dyT", "mgu_xT", "dW_mgu"),
                               "moe_wgrad_down": ("mdn_dyT", "mdn_xT", "dW_mdn")}.items():
        pad = host(o[an.split("_")[0] + "_pad"])
        a_q, b_q, C = o[an], o[bn], o[cn]
        Mw, kc = a_q.shape
        Nw = b_q.shape[0]
        g = rng.integers(0, G, 256)
        i, j = rng.integers(0, Mw, 256), rng.integers(0, Nw, 256)
        sa_, sb_ = unswz(o[an + "swz"], Mw, kc // 32), unswz(o[bn + "swz"], Nw, kc // 32)
        qa_h, qb_h = host(a_q[torch.from_numpy(i).cuda()]), host(b_q[torch.from_numpy(j).cuda()])
        refs, bnds = [], []
        for e in range(256):
            lo, hi = int(pad[g[e]]), int(pad[g[e] + 1])
            rf, bd = oracle.gemm_sampled(np.zeros(1, np.int64), np.zeros(1, np.int64),
                                         np.ascontiguousarray(qa_h[e:e + 1, lo:hi]),
                                         np.ascontiguousarray(sa_[i[e]:i[e] + 1, lo // 32:hi // 32]),
                                         np.ascontiguousarray(qb_h[e:e + 1, lo:hi]),
                                         np.ascontiguousarray(sb_[j[e]:j[e] + 1, lo // 32:hi // 32]))
            refs.append(rf[0])
            bnds.append(bd[0])
        got = C[torch.from_numpy(g).cuda(), torch.from_numpy(i).cuda(), torch.from_numpy(j).cuda()]
        out[name] = stats(got.float().cpu().numpy().astype(np.float64), np.array(refs), np.array(bnds))
    groups = {"tiny": ["tiny"], "dense_fwd_m4608": ["qkv", "o", "gate_up", "down"],
              "dense_bwd_gate_up": ["dgrad", "wgrad"],
              "moe_qwen3_30b_a3b": [k for k in out if k.startswith("moe_")]}
    per_config = {}
    for cfg, keys in groups.items():
        per_config[cfg] = {"n": sum(out[k]["n"] for k in keys),
                           "within_stated": sum(out[k]["within_stated"] for k in keys),
                           "max_err_over_bnd": max(out[k]["max_err_over_bnd"] for k in keys)}
    return {"bar": "|C - C_ref| <= 1e-5 (|A||B|)_ij + 1 BF16 ulp of C_ref (BF16 out)",
            "per_config": per_config, "per_product": out}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the MXFP8 hot "
              "path here is a single-GPU library with no collectives", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        torch.cuda.set_device(0)
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return
    if args.hbm_probe:
        torch.cuda.set_device(0)
        print(json.dumps({"hbm_probe_1GiB": hbm_probe(torch)}))
        return
    if args.library_compare:
        import mxfp8_block_scaled_08_amd as mx
        mx.load()
        torch.cuda.set_device(0)
        print(json.dumps({"library_compare": library_compare(torch, mx, args.library_compare)}))
        return

    import mxfp8_block_scaled_08_amd as mx
    import mxsynth

    mx.load()
    torch.cuda.set_device(0)
    I, o = build_workload(mx, torch, mxsynth)
    torch.cuda.synchronize()
    # everything runs on one side stream (the step's calls share one
    # workspace, so they must not overlap in time)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    stream_ctx = torch.cuda.stream(stream)
    stream_ctx.__enter__()

    noop = lambda cat, fn, *a, **kw: fn(*a, **kw)
    for _ in range(args.warmup):
        step(mx, I, o, noop)
    torch.cuda.synchronize()

    T = Timer(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step(mx, I, o, T)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    T.collect()
    gpu_ms = start.elapsed_time(end)
    ms_per_step_eager = gpu_ms / args.steps
    ms_per_step = ms_per_step_eager
    graph = None if args.no_graph else graph_replay(torch, mx, I, o, noop, args.steps)
    if graph is not None and graph["bytes_equal_to_eager"]:
        ms_per_step = graph["ms_per_step"]

    w = work_per_step(I)
    row_el, col_el, dual_el, colg_el = w["row_el"], w["col_el"], w["dual_el"], w["colg_el"]
    dualg_el = w["dualg_el"]
    dense, grouped, wgrad = w["dense"], w["grouped"], w["wgrad"]
    flops = dense + grouped + wgrad
    K = args.steps
    row_only, col_only = row_el - dual_el, col_el - dual_el
    q_bytes = ((row_only + col_only + w["colg_gu_el"]) * QUANT_BYTES_PER_ELEMENT
               + (dual_el + dualg_el) * DUAL_BYTES_PER_ELEMENT)
    qt = (T.totals.get("quant_row", 0) + T.totals.get("quant_col", 0)
          + T.totals.get("quant_dual", 0) + T.totals.get("quant_col_grouped", 0)
          + T.totals.get("quant_dual_grouped", 0)) / K  # ms
    gemm_ms = T.totals["gemm"] / K
    ggemm_ms = T.totals["grouped_gemm"] / K
    wg_ms = T.totals["grouped_wgrad"] / K
    ops = {
        "quantize_rowwise": {"ms": T.totals["quant_row"] / K,
                             "GB/s": row_only * QUANT_BYTES_PER_ELEMENT / (T.totals["quant_row"] / K) / 1e6},
        "quantize_colwise": {"ms": T.totals["quant_col"] / K,
                             "GB/s": col_only * QUANT_BYTES_PER_ELEMENT / (T.totals["quant_col"] / K) / 1e6},
        "quantize_dual": {"ms": T.totals["quant_dual"] / K,
                          "GB/s": dual_el * DUAL_BYTES_PER_ELEMENT / (T.totals["quant_dual"] / K) / 1e6},
        "scale_swizzle": {"launches": T.counts.get("swizzle", 0) // K},
        "moe_dispatch": {
            "ms": T.totals["moe_dispatch"] / K,
            "GB/s": w["disp_bytes"] / (T.totals["moe_dispatch"] / K) / 1e6},
        "swiglu_quantize": {
            "ms": T.totals["swiglu"] / K,
            # gate and up read (4 B), h quantized in both orientations
            "GB/s": w["swiglu_el"] * (4 + 2 * (QUANT_BYTES_PER_ELEMENT - 2)) / (T.totals["swiglu"] / K) / 1e6},
        "moe_combine": {
            "ms": T.totals["moe_combine"] / K,
            "GB/s": w["comb_el"] * (2 * w["topk"] + 2) / (T.totals["moe_combine"] / K) / 1e6},
        "quantize_dual_grouped": {
            "ms": T.totals["quant_dual_grouped"] / K,
            "GB/s": dualg_el * DUAL_BYTES_PER_ELEMENT / (T.totals["quant_dual_grouped"] / K) / 1e6},
        "dense_gemm": {"ms": gemm_ms, "TFLOP/s": dense / gemm_ms / 1e9},
        "grouped_gemm": {"ms": ggemm_ms, "TFLOP/s": grouped / ggemm_ms / 1e9},
        "grouped_wgrad": {"ms": wg_ms, "TFLOP/s": wgrad / wg_ms / 1e9},
    }
    for k, v in ops.items():
        if "GB/s" in v:
            v["frac_hbm_peak"] = v["GB/s"] / HBM_PEAK_GBPS
        if "TFLOP/s" in v:
            v["frac_mfma_peak"] = v["TFLOP/s"] / MFMA_FP8_PEAK_TFLOPS
        for kk in list(v):
            if isinstance(v[kk], float):
                v[kk] = round(v[kk], 4)
    dense_tflops = dense / gemm_ms / 1e9
    result = {
        "metric": "MXFP8 GEMM TFLOP/s + quantize GB/s vs MI355X peaks, Qwen3 layer shapes",
        "value": round(flops / ms_per_step / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_eager": round(ms_per_step_eager, 4),
        "timing": ("HIP graph replay of the step (one capture, replayed; outputs checked byte-equal "
                   "to the eager step)" if ms_per_step != ms_per_step_eager else "eager launches"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3 (E8M0 block scales, FP32 accumulate, BF16 out)",
        "data": "synthetic (seeded device draws; Qwen3-8B / Qwen3-30B-A3B layer shapes)",
        "config": {
            "workload": ("qwen3-layer-pass: weight-sync row+column MXFP8 quantize of one "
                         "Qwen3-8B layer (one dual pass per weight); dense fwd M=4608 (qkv, o, gate_up, down); dense bwd "
                         "gate_up dgrad 12288x4096x24576 + wgrad 24576x4096x12288; Qwen3-30B-A3B "
                         "MoE grouped gate_up/down, 163840 rows, 128 experts, Zipf(1.1), forward "
                         "and expert backward (data gradient grouped over rows, weight gradient "
                         "grouped over each expert's token range)"),
            "gemm_flop_per_step": flops,
            "quantized_elements_per_step": row_el + col_el + colg_el + 2 * dualg_el,
            "parallelism": "single GPU",
        },
        "value_definition": "total GEMM FLOP of the step / wall time of the whole step "
                            "(quantize, rearrangement and GEMMs, HIP events)",
        "quantize_GBps": round(q_bytes / qt / 1e6, 1),
        "quantize_frac_hbm_peak": round(q_bytes / qt / 1e6 / HBM_PEAK_GBPS, 4),
        "gemm_TFLOPs": round(flops / (gemm_ms + ggemm_ms + wg_ms) / 1e9, 1),
        "gemm_frac_mfma_peak": round(flops / (gemm_ms + ggemm_ms + wg_ms) / 1e9
                                     / MFMA_FP8_PEAK_TFLOPS, 4),
        "ops": ops,
        "roofline": {
            "kernel": "mx_gemm_kernel<dense, BF16 out>",
            "bound": "mfma",
            "achieved": round(dense_tflops, 1),
            "peak": MFMA_FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dense_tflops / MFMA_FP8_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(),
            "launches_per_step": T.counts["gemm"] // K,
            "avg_launch_ms": round(gemm_ms / (T.counts["gemm"] // K), 4),
        },
        "wall_s_timed_region": round(wall, 3),
    }
    if graph is not None:
        result["graph"] = graph
    if not args.no_cpu_baseline:
        # the CPU-oracle leg: the oracle's speed on the host, and the step's
        # GEMM outputs against it
        result["cpu_baseline"] = cpu_baseline(torch, mxsynth, row_el + dualg_el, col_el + colg_el + dualg_el,
                                              flops)
        result["parity_vs_oracle"] = oracle_parity(torch, mx, mxsynth, I, o)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
