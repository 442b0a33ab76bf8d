"""Benchmark of the MoE FP8 training hot path on one MI355X.

One step = one pass of every hot-path operation over one batch of synthetic input resident in
HBM:
  X         both FP8 layouts of X in one call: rowwise (the forward's A operand) and the
            token-grouped transposed colwise copy (the weight gradient's A operand)
  forward   per-expert colwise quant of W (transposed), M-grouped FP8 GEMM
  backward  colwise-grouped transposed quant of dY, K-grouped FP8 weight-gradient GEMM
  MXFP8     MX rowwise quant of X, MX colwise quant of W, MX grouped GEMM (forward)
  (a configuration without the backward quantizes X rowwise only)
Next rows, timed in passes of their own after the step and reported under "next_rows":
  the two single-layout quantizations of X (rowwise, transposed colwise) that the dual call
  replaces, and both layouts of dY in one call;
  rowwise quant of routed rows gathered in expert order from 2048 token rows (top-8);
  rowwise quant of dY and of W along N, M-grouped FP8 data-gradient GEMM (dX = dY W^T);
  MX colwise quant of X and dY along tokens, MX K-grouped weight-gradient GEMM.
Default workload: the DeepSeek-V3-shaped local expert slice (32 experts, hidden 7168,
intermediate 2048, 16384 routed token rows, Zipf(1.1) group sizes), e4m3fn.

Timing: W untimed warm-up steps, then exactly K timed steps between device synchronisations
(the step time and `value`); every operation is bracketed with HIP events on the stream it runs
on, giving per-launch warm averages (us_warm).  Each operation is then timed again K times with
a 1 GiB cache flush before every launch (us, the median: inputs come from HBM, not from the
L2s or the 256 MB last-level cache).  The JSON line reports whole-step throughput (algorithmic
GEMM flops of the step per second of step time, quantization time included), per-op flushed
and warm times with GB/s or TFLOP/s and % of peak, the same for the other configurations
(tiny in e4m3fnuz, the dense Llama3-8B FFN GEMM, DeepSeek-MoE-16B experts, the DeepSeek-V3
slice in e4m3fnuz), a roofline entry for the step kernel that takes the most time, and the CPU
oracle timed on the host at all threads and at one thread.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quantize GB/s (% HBM peak) + FP8 grouped GEMM TFLOP/s (% MFMA peak)"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 (and MXFP8) matrix throughput

WORKLOADS = {
    # name: (workloads-module config, format, ops)
    "dsv3": ("dsv3_bwd", 1, ("fwd", "gather", "wgrad", "dgrad", "mx", "mxwgrad")),
    "dense": ("dense", 1, ("fwd",)),
    "moe16b": ("moe16b", 1, ("fwd",)),
    "tiny": ("tiny", 0, ("fwd", "wgrad")),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the further configurations timed after the headline workload")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy 4 times (reference for the HBM "
                         "byte counters) and exit")
    return ap.parse_args()


def copy_calibration(torch):
    """A plain device-to-device copy of known size: FETCH_SIZE / WRITE_SIZE of its dispatches
    give the counters' bytes per algorithmic byte."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 4}), flush=True)


def make_inputs(name, torch, dev, fmt=None, ops=None):
    """Device-resident synthetic inputs.  Group offsets come from the seeded numpy recipe of the
    workloads module; the bf16 tensors are drawn on the device with a seeded generator (same
    distributions as the recipe: X, dY ~ N(0,1), W ~ N(0, 0.02); the tiny workload adds 1% x50
    outliers).  fmt / ops override the workload's encoding and operation list."""
    import workloads
    cfg_name, fmt0, ops0 = WORKLOADS[name]
    fmt = fmt0 if fmt is None else fmt
    ops = ops0 if ops is None else ops
    cfg = workloads.CONFIGS[cfg_name]
    M, K, N, E = cfg["M"], cfg["K"], cfg["N"], cfg["E"]
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    if cfg_name == "dense":
        offsets = np.array([M], np.int32)
    elif cfg_name == "moe16b":
        offsets = workloads.routed_offsets_topk(rng, cfg["tokens"], E, cfg["topk"])
    elif cfg_name == "tiny":
        offsets = workloads.random_offsets(rng, M, E)
    else:
        offsets = workloads.multinomial_offsets(rng, M, E)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(cfg["seed"]))
    x = torch.randn((M, K), generator=gen, device=dev, dtype=torch.float32)
    if cfg_name == "tiny":
        mask = torch.rand((M, K), generator=gen, device=dev) < 0.01
        x = torch.where(mask, x * 50.0, x)
    x = x.to(torch.bfloat16)
    w = (torch.randn((E * K, N), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(
        torch.bfloat16)
    dy = None
    if "wgrad" in ops or "dgrad" in ops or "mxwgrad" in ops:
        dy = torch.randn((M, N), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return dict(M=M, K=K, N=N, E=E, fmt=fmt, ops=ops, x=x, w=w, dy=dy,
                offsets=torch.tensor(offsets, dtype=torch.int32, device=dev),
                offsets_np=offsets, cfg_name=cfg_name)


class Step:
    """Pre-allocated outputs/workspaces and the per-operation launch sequence."""

    def __init__(self, fq, torch, d):
        self.fq, self.torch, self.d = fq, torch, d
        dev = d["x"].device
        M, K, N, E = d["M"], d["K"], d["N"], d["E"]
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=dev)
        self.off_w = torch.tensor(np.arange(1, E + 1, dtype=np.int32) * K, device=dev)
        G = d["offsets"].numel()
        ldm = -(-M // 16) * 16  # 16-byte aligned token rows for the transposed operands
        self.buf = dict(
            xq=e(M, K), sx=e(M, dt=f32), wqt=e(N, E * K), sw=e(E, N, dt=f32), y=e(M, N, dt=bf),
            ws_w=e(max(256, fq.fp8_quant_colwise_grouped_workspace_size(E * K, N, E))),
            gws=e(fq.fp8_grouped_gemm_workspace_size(0, M, N, K, int(d["offsets"].numel()))),
        )
        if "wgrad" in d["ops"]:
            self.buf.update(
                xqt=e(K, ldm), sxg=e(G, K, dt=f32), dyqt=e(N, ldm), sdyg=e(G, N, dt=f32),
                dw=e(G, K, N, dt=bf),
                ws_x=e(max(256, fq.fp8_quant_colwise_grouped_workspace_size(M, K, G))),
                ws_dy=e(max(256, fq.fp8_quant_colwise_grouped_workspace_size(M, N, G))),
                # both layouts of X and of dY in one call each (rowwise + transposed)
                dxq=e(M, K), dxs=e(M, dt=f32), dyq2=e(M, N), dys2=e(M, dt=f32),
                ws_dual=e(max(256, fq.fp8_quant_dual_grouped_workspace_size(M, K, G),
                                      fq.fp8_quant_dual_grouped_workspace_size(M, N, G))))
        if "gather" in d["ops"]:
            # dispatch in expert order: 2048 tokens x top-8 over 32 experts (seeded Zipf routing)
            import workloads
            _, gidx = workloads.routed_rows_topk(np.random.Generator(np.random.PCG64(6)),
                                                 M // 8, E, 8)
            self.gidx = torch.tensor(gidx, device=dev)
            self.buf.update(gq=e(M, K), gs=e(M, dt=f32))
        if "dgrad" in d["ops"]:
            # data gradient: dY and W quantized rowwise along N (the contraction), dX bf16 [M, K]
            self.buf.update(dyq=e(M, N), sdyr=e(M, dt=f32), wqn=e(E * K, N), swk=e(E * K, dt=f32),
                            dx=e(M, K, dt=bf))
            # both weight layouts in one call (quantized once per optimizer step)
            self.buf.update(dwr=e(E * K, N), dwrs=e(E * K, dt=f32), dwt=e(N, E * K),
                            dwts=e(E, N, dt=f32),
                            ws_wdual=e(max(256, fq.fp8_quant_weights_dual_workspace_size(E, K, N))))
        if "mx" in d["ops"]:
            self.buf.update(mxq=e(M, K), mxe=e(M, K // 32), mxwt=e(N, E * K),
                            mxwe=e(N, E * K // 32), ymx=e(M, N, dt=bf))
        if "mxwgrad" in d["ops"]:
            # MX backward: X and dY quantized along tokens in 32-token blocks (M % 32 == 0)
            self.buf.update(mxxt=e(K, M), mxxe=e(K, M // 32), mxdyt=e(N, M),
                            mxdye=e(N, M // 32), mxdw=e(G, K, N, dt=bf))
        self.ldm = ldm
        self.flops = {}
        self.bytes = {}
        self.units = {}
        tot_m = M
        # GEMMs' algorithmic HBM bytes: each operand byte read once, the bf16 output written once
        self.gemm_bytes = {}
        self.flops["gemm_fwd"] = 2.0 * tot_m * N * K
        self.gemm_bytes["gemm_fwd"] = M * K + E * N * K + M * N * 2 + M * 4 + E * N * 4
        self.bytes["quant_rowwise_x"] = M * K * 3 + M * 4
        self.bytes["quant_colwise_w"] = E * K * N * 3 + E * N * 4
        if "wgrad" in d["ops"]:
            self.flops["gemm_wgrad"] = 2.0 * M * N * K
            self.gemm_bytes["gemm_wgrad"] = K * M + N * M + G * K * N * 2 + G * K * 4 + G * N * 4
            self.bytes["quant_colwise_xT"] = M * K * 3 + G * K * 4
            self.bytes["quant_colwise_dyT"] = M * N * 3 + G * N * 4
            # algorithmic: read once, both FP8 layouts written, both scale sets
            self.bytes["quant_dual_x"] = M * K * 4 + M * 4 + G * K * 4
            self.bytes["quant_dual_dy"] = M * N * 4 + M * 4 + G * N * 4
        if "mxwgrad" in d["ops"]:
            self.flops["gemm_mx_wgrad"] = 2.0 * M * N * K
            self.gemm_bytes["gemm_mx_wgrad"] = (K * M + N * M + G * K * N * 2 + K * M // 32
                                                + N * M // 32)
            self.bytes["mx_quant_colwise_xT"] = M * K * 3 + M * K // 32
            self.bytes["mx_quant_colwise_dyT"] = M * N * 3 + M * N // 32
        if "gather" in d["ops"]:
            # minimum traffic: each token row read once, every routed row written, index, scales
            self.bytes["quant_rowwise_gather_x"] = (M // 8) * K * 2 + M * K + M * 4 + M * 4
        if "dgrad" in d["ops"]:
            self.flops["gemm_dgrad"] = 2.0 * M * N * K
            self.gemm_bytes["gemm_dgrad"] = M * N + E * K * N + M * K * 2 + M * 4 + E * K * 4
            self.bytes["quant_rowwise_dy"] = M * N * 3 + M * 4
            self.bytes["quant_rowwise_w"] = E * K * N * 3 + E * K * 4
            # algorithmic: W read once, both FP8 layouts written, both scale sets
            self.bytes["quant_weights_dual"] = E * K * N * 4 + E * K * 4 + E * N * 4
        if "mx" in d["ops"]:
            self.flops["gemm_mx"] = 2.0 * M * N * K
            self.gemm_bytes["gemm_mx"] = (M * K + E * N * K + M * N * 2 + M * K // 32
                                          + E * N * K // 32)
            self.bytes["mx_quant_rowwise_x"] = M * K * 3 + M * K // 32
            self.bytes["mx_quant_colwise_w"] = E * K * N * 3 + E * K * N // 32

    def ops(self):
        fq, d, b = self.fq, self.d, self.buf
        M, K, N, E, fmt = d["M"], d["K"], d["N"], d["E"], d["fmt"]
        q_rows_x = ("quant_rowwise_x", lambda: fq.fp8_quant_rowwise(d["x"], fmt, q=b["xq"],
                                                                    scales=b["sx"]))
        # with the backward in the step, X's two layouts come from one call (bit-identical to
        # the rowwise and the transposed colwise calls, which are timed among the next rows)
        dual_x = ("quant_dual_x", lambda: fq.fp8_quant_dual_grouped(
            d["x"], d["offsets"], fmt, q=b["xq"], s_rows=b["sx"], q_t=b["xqt"][:, :M],
            s_cols=b["sxg"], workspace=b["ws_dual"]))
        seq = [
            dual_x if "wgrad" in d["ops"] else q_rows_x,
            ("quant_colwise_w", lambda: fq.fp8_quant_colwise_grouped(
                d["w"], self.off_w, fmt, q_t=b["wqt"], scales=b["sw"].view(E, N),
                workspace=b["ws_w"])),
            ("gemm_fwd", lambda: fq.fp8_grouped_gemm(
                fq.GEMM_FWD_MGROUPED, fmt, b["xq"], b["sx"], b["wqt"], b["sw"], d["offsets"],
                M, N, K, ldb=E * K, b_group_stride=K, c=b["y"], workspace=b["gws"])),
        ]
        # rows beyond the hot-path step (gathered dispatch quant, data gradient, MX backward):
        # timed in passes of their own after the step
        extra = []
        if "gather" in d["ops"]:
            extra += [("quant_rowwise_gather_x", lambda: fq.fp8_quant_rowwise_gather(
                d["x"][: M // 8], self.gidx, fmt, q=b["gq"], scales=b["gs"]))]
        if "wgrad" in d["ops"]:
            seq += [
                ("quant_colwise_dyT", lambda: fq.fp8_quant_colwise_grouped(
                    d["dy"], d["offsets"], fmt, q_t=b["dyqt"][:, :M], scales=b["sdyg"],
                    workspace=b["ws_dy"])),
                ("gemm_wgrad", lambda: fq.fp8_grouped_gemm(
                    fq.GEMM_WGRAD_KGROUPED, fmt, b["xqt"], b["sxg"], b["dyqt"], b["sdyg"],
                    d["offsets"], M, N, K, ldb=self.ldm, c=b["dw"], workspace=b["gws"])),
            ]
        if "wgrad" in d["ops"]:
            # X's single-layout calls (the step uses the dual call); both layouts of dY at once,
            # for the data gradient and the weight gradient
            extra += [
                q_rows_x,
                ("quant_colwise_xT", lambda: fq.fp8_quant_colwise_grouped(
                    d["x"], d["offsets"], fmt, q_t=b["xqt"][:, :M], scales=b["sxg"],
                    workspace=b["ws_x"])),
                ("quant_dual_dy", lambda: fq.fp8_quant_dual_grouped(
                    d["dy"], d["offsets"], fmt, q=b["dyq2"], s_rows=b["dys2"],
                    q_t=b["dyqt"][:, :M], s_cols=b["sdyg"], workspace=b["ws_dual"])),
            ]
        if "dgrad" in d["ops"]:
            # dX[m, k] = sum_n dY[m, n] W_g[k, n]: the forward mode with W's [K, N] rows of expert
            # g as the per-group B operand (contraction over N)
            extra += [
                ("quant_rowwise_dy", lambda: fq.fp8_quant_rowwise(d["dy"], fmt, q=b["dyq"],
                                                                  scales=b["sdyr"])),
                ("quant_rowwise_w", lambda: fq.fp8_quant_rowwise(d["w"], fmt, q=b["wqn"],
                                                                 scales=b["swk"])),
                ("gemm_dgrad", lambda: fq.fp8_grouped_gemm(
                    fq.GEMM_FWD_MGROUPED, fmt, b["dyq"], b["sdyr"], b["wqn"], b["swk"],
                    d["offsets"], M, K, N, ldb=N, b_group_stride=K * N, c=b["dx"],
                    workspace=b["gws"])),
                ("quant_weights_dual", lambda: fq.fp8_quant_weights_dual(
                    d["w"], E, fmt, q_rows=b["dwr"], s_rows=b["dwrs"], q_t=b["dwt"],
                    s_cols=b["dwts"], workspace=b["ws_wdual"])),
            ]
        if "mx" in d["ops"]:
            seq += [
                ("mx_quant_rowwise_x", lambda: fq.fp8_mx_quant_rowwise(d["x"], q=b["mxq"],
                                                                      e8m0=b["mxe"])),
                ("mx_quant_colwise_w", lambda: fq.fp8_mx_quant_colwise(d["w"], q_t=b["mxwt"],
                                                                      e8m0=b["mxwe"])),
                ("gemm_mx", lambda: fq.fp8_mx_grouped_gemm(
                    b["mxq"], b["mxe"], b["mxwt"], b["mxwe"], d["offsets"], M, N, K,
                    ldb=E * K, b_group_stride=K, ld_sb=E * K // 32, sb_group_stride=K // 32,
                    c=b["ymx"], workspace=b["gws"])),
            ]
        if "mxwgrad" in d["ops"]:
            extra += [
                ("mx_quant_colwise_xT", lambda: fq.fp8_mx_quant_colwise(
                    d["x"], q_t=b["mxxt"], e8m0=b["mxxe"])),
                ("mx_quant_colwise_dyT", lambda: fq.fp8_mx_quant_colwise(
                    d["dy"], q_t=b["mxdyt"], e8m0=b["mxdye"])),
                ("gemm_mx_wgrad", lambda: fq.fp8_mx_grouped_gemm_wgrad(
                    b["mxxt"], b["mxxe"], b["mxdyt"], b["mxdye"], d["offsets"], M, N, K,
                    c=b["mxdw"], workspace=b["gws"])),
            ]
        return seq, extra


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, seconds):
    """The oracle (never tuned) on the host, at all its threads and at one thread:
      - forward grouped GEMM rows of the workload's shapes (N x K), on a row sample sized to
        roughly `seconds` of work (all threads) or a quarter of it (one thread);
      - rowwise quantization of a full-size [M, N] gradient matrix (dY's shape) at both thread
        counts, and of the full [M, K] activations at all threads."""
    import oracle
    import workloads
    M, K, N, fmt = d["M"], d["K"], d["N"], d["fmt"]
    all_threads = oracle.num_threads()
    xs = workloads.make_matrix(1234, 1024, K, 1.0, 0.0)
    ws = workloads.make_matrix(1235, K, N, 0.02)
    qa, sa = oracle.quant_rowwise(xs, fmt)
    qbt, sb = oracle.quant_colwise_grouped(ws, np.array([K], np.int32), fmt)
    off = np.array([qa.shape[0]], np.int32)

    def gemm_rate(threads, budget):
        oracle.set_num_threads(threads)
        # calibrate on as many rows as threads (fewer would leave threads idle), then a sample
        # sized to the budget
        ncal = max(2, min(1024, threads))
        t0 = time.perf_counter()
        oracle.gemm_fwd_rows(fmt, qa, sa, qbt, K, 0, sb, off, N, K, np.arange(ncal))
        tcal = time.perf_counter() - t0
        nrows = int(max(2, min(1024, ncal * budget / max(tcal, 1e-6))))
        t0 = time.perf_counter()
        oracle.gemm_fwd_rows(fmt, qa, sa, qbt, K, 0, sb, off, N, K, np.arange(nrows))
        tg = time.perf_counter() - t0
        return 2.0 * nrows * N * K / tg / 1e12, nrows, tg

    def quant_rate(threads, rows, cols):
        oracle.set_num_threads(threads)
        x = workloads.make_matrix(1236, rows, cols, 1.0, 0.0)
        t0 = time.perf_counter()
        oracle.quant_rowwise(x, fmt)
        tq = time.perf_counter() - t0
        return rows * cols * 3 / tq / 1e9, tq

    try:
        tf_all, rows_all, tg_all = gemm_rate(all_threads, seconds)
        tf_one, rows_one, tg_one = gemm_rate(1, seconds / 4)
        qdy_all, _ = quant_rate(all_threads, M, N)
        qdy_one, tq_one = quant_rate(1, M, N)
        qx_all, _ = quant_rate(all_threads, M, K)
    finally:
        oracle.set_num_threads(all_threads)
    return dict(
        value=tf_all, unit="TFLOP/s", cores=all_threads, kind="oracle",
        sample=(f"forward grouped GEMM rows at N={N}, K={K}: {rows_all} rows at {all_threads} "
                f"threads ({tg_all:.1f} s), {rows_one} rows at 1 thread ({tg_one:.1f} s); rowwise "
                f"quant of the full {M}x{N} and {M}x{K} bf16 matrices"),
        value_1thread=tf_one, cpu_model=cpu_model(), nproc=os.cpu_count(),
        omp_num_threads=os.environ.get("OMP_NUM_THREADS"),
        quant_GBps={f"{M}x{N}": {"threads_all": round(qdy_all, 4), "threads_1": round(qdy_one, 4)},
                    f"{M}x{K}": {"threads_all": round(qx_all, 4)}})


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_dsv3_step.md")


def source_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE/WRITE_SIZE summary, or
    None when there is none or the kernel's source changed since the counters were taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    blk = text.split("```json", 1)
    if len(blk) < 2:
        return None
    rec = json.loads(blk[1].split("```", 1)[0])
    src = ["fp8_quantization_grouped_amd/csrc/grouped_gemm.hip",
           "fp8_quantization_grouped_amd/csrc/common.hpp"]
    if rec.get("kernel") != kernel or rec.get("source_sha256_16") != source_hash(src):
        return None
    return int(rec["traffic_bytes"])


def time_passes(torch, seq, warmup, steps):
    """Average per-op milliseconds over `steps` passes of `seq` after `warmup` passes, each op
    bracketed by HIP events on the stream it runs on (warm: inputs may sit in the caches)."""
    if not seq:
        return {}
    for _ in range(warmup):
        for _, fn in seq:
            fn()
    torch.cuda.synchronize()
    evs = {name: [] for name, _ in seq}
    for _ in range(steps):
        for name, fn in seq:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs[name].append((a, b))
    torch.cuda.synchronize()
    return {n: float(np.mean([a.elapsed_time(b) for a, b in v])) for n, v in evs.items()}


class Flush:
    """Writes a 1 GiB buffer: evicts the 8 L2s (4 MB each) and the 256 MB last-level cache, so
    that the next kernel reads its inputs from HBM."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        self.v = 0

    def __call__(self):
        self.v ^= 1
        self.buf.fill_(self.v)


def time_flushed(torch, seq, steps, flush):
    """Median per-op milliseconds over `steps` launches, each launch preceded by a cache flush
    (outside its events)."""
    if not seq:
        return {}
    evs = {name: [] for name, _ in seq}
    for _ in range(steps):
        for name, fn in seq:
            flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs[name].append((a, b))
    torch.cuda.synchronize()
    return {n: float(np.median([a.elapsed_time(b) for a, b in v])) for n, v in evs.items()}


def entry(st, n, ms, ms_warm=None):
    """Per-op record: flushed microseconds and their throughput (% of peak); warm beside."""
    ent = {"us": round(ms * 1e3, 2)}
    if ms_warm is not None:
        ent["us_warm"] = round(ms_warm * 1e3, 2)
    if n in st.flops:
        tf = st.flops[n] / (ms * 1e-3) / 1e12
        ent.update(TFLOPs=round(tf, 1), frac_mfma_peak=round(tf / FP8_PEAK_TFLOPS, 4))
        gb = st.gemm_bytes[n] / (ms * 1e-3) / 1e9
        ent.update(GBps=round(gb, 1), frac_hbm_peak=round(gb / HBM_PEAK_GBPS, 4))
    if n in st.bytes:
        gb = st.bytes[n] / (ms * 1e-3) / 1e9
        ent.update(GBps=round(gb, 1), frac_hbm_peak=round(gb / HBM_PEAK_GBPS, 4))
    return ent


# Further configurations timed after the headline workload (per-op flushed and warm times):
# name -> (workload, format, ops)
EXTRA_CONFIGS = {
    "tiny_e4m3fnuz": ("tiny", 0, ("fwd", "wgrad")),
    "dense_llama3_8b_ffn": ("dense", 1, ("fwd",)),
    "moe16b": ("moe16b", 1, ("fwd",)),
    "dsv3_e4m3fnuz": ("dsv3", 0, ("fwd", "wgrad")),
}


def run_config(fq, torch, dev, name, fmt, ops, warmup, steps, flush):
    d = make_inputs(name, torch, dev, fmt=fmt, ops=ops)
    st = Step(fq, torch, d)
    seq, extra = st.ops()
    seq = seq + extra
    warm = time_passes(torch, seq, warmup, steps)
    cold = time_flushed(torch, seq, steps, flush)
    out = {n: entry(st, n, cold[n], warm[n]) for n in cold}
    del st, d
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): this path has no "
              "multi-GPU mode (under expert parallelism each GPU runs this same path on its own "
              "experts' token rows).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import fp8_quantization_grouped_amd as fq
    fq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = make_inputs(args.workload, torch, dev)
    st = Step(fq, torch, d)
    seq, extra = st.ops()
    for _ in range(args.warmup):
        for _, fn in seq:
            fn()
    torch.cuda.synchronize()
    evs = {name: [] for name, _ in seq}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for _ in range(args.steps):
        for name, fn in seq:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs[name].append((a, b))
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    warm_op = {n: float(np.mean([a.elapsed_time(b) for a, b in v])) for n, v in evs.items()}
    warm_extra = time_passes(torch, extra, args.warmup, args.steps)
    flush = Flush(torch, dev)
    cold_op = time_flushed(torch, seq, args.steps, flush)
    cold_extra = time_flushed(torch, extra, args.steps, flush)

    kernels = {n: entry(st, n, cold_op[n], warm_op[n]) for n in cold_op}
    next_rows = {n: entry(st, n, cold_extra[n], warm_extra[n]) for n in cold_extra}
    gemm_ms = sum(cold_op[n] for n in cold_op if n in st.flops)
    quant_ms = sum(cold_op[n] for n in cold_op if n in st.bytes)
    total_flops = sum(st.flops[n] for n in cold_op if n in st.flops)
    total_bytes = sum(st.bytes[n] for n in cold_op if n in st.bytes)
    value = total_flops / (ms_step * 1e-3) / 1e12

    dom = max(cold_op, key=cold_op.get)
    # a GEMM is bound by whichever peak gives the longer ideal time: the weight-gradient GEMM's
    # bf16 output (groups x K x N) makes it HBM-bound on these shapes
    gemm_hbm_bound = (dom in st.flops and st.gemm_bytes[dom] / (HBM_PEAK_GBPS * 1e9)
                      > st.flops[dom] / (FP8_PEAK_TFLOPS * 1e12))
    if dom in st.flops and not gemm_hbm_bound:
        ach = st.flops[dom] / (cold_op[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / FP8_PEAK_TFLOPS, 4)}
    else:
        nbytes = st.gemm_bytes[dom] if dom in st.flops else st.bytes[dom]
        ach = nbytes / (cold_op[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4)}
    roof["kernel"] = dom
    roof["timing"] = "median of flushed launches"
    roof["traffic"] = measured_traffic(dom)

    configs = {}
    if args.workload == "dsv3" and not args.no_configs:
        del st, seq, extra
        torch.cuda.empty_cache()
        for cname, (wl, cfmt, cops) in EXTRA_CONFIGS.items():
            configs[cname] = run_config(fq, torch, dev, wl, cfmt, cops, args.warmup,
                                        max(5, args.steps // 2), flush)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(d, args.cpu_seconds)

    cfg = {"workload": {
        "dsv3": "DeepSeek-V3-shaped local expert slice: 32 experts, hidden 7168, intermediate "
                "2048, 16384 routed token rows (Zipf 1.1 group sizes); step: FP8 forward + "
                "weight-gradient + MXFP8 forward; next_rows: rowwise quant gathered in expert "
                "order from 2048 tokens x top-8, data gradient, MXFP8 weight gradient",
        "dense": "Llama3-8B-style FFN GEMM: M=8192, K=4096, N=14336, G=1; FP8 forward",
        "moe16b": "DeepSeek-MoE-16B-shaped experts: 64 experts, K=2048, N=1408, 49152 routed "
                  "rows (top-6, Zipf 1.1); FP8 forward",
        "tiny": "4 experts, K=256, N=512, 1024 token rows; e4m3fnuz forward + weight-gradient",
    }[args.workload], "M": d["M"], "K": d["K"], "N": d["N"], "experts": d["E"],
        "fp8_format": "e4m3fn" if d["fmt"] == 1 else "e4m3fnuz"}
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3fn x fp8e4m3fn -> fp32 acc" if d["fmt"] == 1 else
                 "fp8e4m3fnuz -> fp32 acc",
        "data": "synthetic (seeded; device-drawn N(0,1) activations/gradients, N(0,0.02) "
                "weights; Zipf-routed group offsets)",
        "config": cfg,
        "timing": "per-op us: median of launches each preceded by a 1 GiB cache flush; us_warm: "
                  "mean inside the timed steps",
        "quantize_GBps": round(total_bytes / (quant_ms * 1e-3) / 1e9, 1),
        "quantize_frac_hbm_peak": round(total_bytes / (quant_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "gemm_TFLOPs": round(total_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "gemm_frac_mfma_peak": round(total_flops / (gemm_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
        "kernels": kernels,
        "next_rows": next_rows,
        "configs": configs,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
