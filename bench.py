"""Benchmark of the w8a8 scaled-GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

One step is one pass of the hot path over one batch of synthetic input,
captured in a HIP graph and replayed (the library allocates and synchronises
nothing, so a whole step captures). Workloads:

  decode  (default) fp8 e4m3 decode GEMMs of the four Llama-3-8B linear
          layers (QKV 6144x4096, O 4096x4096, gate_up 28672x4096, down
          4096x14336) at M = 1, 16, 64: for each, dynamic per-token fp8
          quantisation of the bf16 activations, then the scaled GEMM with
          per-channel fp8 weights, bf16 out (at M = 1 both in one kernel,
          w8a8_quant_scaled_mm).
  prefill the same layers at M = 512, 2048, 8192 with a static per-tensor
          activation scale (calibrated on a seeded [512, K] batch), bf16 out.
  int8    Llama-3-70B layers (QKV 10240x8192, O 8192x8192, gate_up
          57344x8192, down 8192x28672) at M = 1, 64, 4096: per-token int8
          activations, per-channel int8 weights, int32 accumulate, bf16 out.
  kv      scaled fp8 KV cache: per-tensor dynamic quant + dequant of 32
          layers of K and V [32768, 8, 128] bf16, plus the standalone
          per-token fp8 quantisation of [8192, 4096] bf16.
  attn    decode attention over each of 32 layers' fp8 KV caches [32768,
          8, 128] (16 sequences of uneven length, 32 query heads over 8 KV
          heads), K and V dequantised with their scales as they are read.

Weights are quantised once before timing (offline preparation). Every
(M, layer) GEMM has its own weight copy, so one step streams 0.65 GB (decode)
and the 256 MB last-level cache holds no weight from one use to the next.

Prints one JSON line: the workload's throughput, a roofline entry for the
scaled-product kernel (KV: the quant call) that takes the most time per step
(the step's launches of that kernel captured alone and replayed, timed with HIP
events on the launch stream), the same figures for every kernel, and the CPU
oracle timed on a bounded sample of the same workload. The roofline's `traffic` is the HBM traffic per launch from
the rocprofv3 FETCH_SIZE / WRITE_SIZE record under profiles/, when that record
was taken from the current kernel sources (else null). `clock` is the graphics
clock (amdsmi) while the roofline kernel's launches replay back to back; an
MFMA-bound roofline entry is also given against the peak scaled to that clock
(`peak_at_clock`, `frac_at_clock`).

    python bench.py --copy-calibration

runs only a plain device copy of 256 MiB, four times: the FETCH_SIZE and
WRITE_SIZE counters read for it calibrate those of the kernels.
"""
from __future__ import annotations

import argparse
import json
import re
import os
import sys
import threading
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import int8_scaled_gemm_amd as w8  # noqa: E402
import workloads  # noqa: E402

METRIC = "scaled_mm TFLOP/s (fp8/int8) at Llama-3-8B shapes; % of MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "int8": 5000.0}
SPEC_GFX_MHZ = 2400.0  # the clock the published matrix-core peaks are quoted at


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# Workloads: each builds device buffers and returns a list of launches. A
# launch is (kind, fn, units) where fn() enqueues one library call, kind
# names the kernel family, and units are its algorithmic flops and bytes.
# --------------------------------------------------------------------------
class Launch:
    """One library call of a step: call(*args). `kernel` names the kernel
    configuration it runs (several calls of one step can share it); `flops`
    and `nbytes` are its algorithmic work: 2*M*N*K, and every operand, scale
    and output byte read or written once."""

    def __init__(self, kind, call, args, flops, nbytes, label, kernel):
        self.kind, self.call, self.args = kind, call, tuple(args)
        self.flops, self.nbytes, self.label, self.kernel = flops, nbytes, label, kernel

    def fn(self):
        return self.call(*self.args)

    def copy(self):
        """The same call on its own copies of every device buffer (for timing
        a kernel over more distinct bytes than the last-level cache holds)."""
        args = [a.clone() if isinstance(a, torch.Tensor) else a for a in self.args]
        return Launch(self.kind, self.call, args, self.flops, self.nbytes, self.label, self.kernel)


def _gemm_bytes(M, N, K, n_sa, n_sb, out_bytes=2):
    return M * K + N * K + 4 * n_sa + 4 * n_sb + out_bytes * M * N


def _quant_call(qtype, x, q, s):
    return w8.w8a8_quant_per_token(x, qtype, q=q, scales=s)


def _azp_quant_call(x, q, s, z):
    return w8.w8a8_quant_per_token_azp(x, q=q, scales=s, azp=z)


def _static_quant_call(qtype, x, q, s):
    return w8.w8a8_quant_per_tensor(x, qtype, scale=s, q=q)


def _mm_call(otype, q, wq, s, wsc, out, ws):
    return w8.w8a8_scaled_mm(q, wq.t(), s, wsc, otype, out=out, workspace=ws)


def _mm_azp_call(otype, q, wq, s, z, cs, wsc, out):
    return w8.w8a8_scaled_mm_azp(q, wq.t(), s, z, cs, wsc, otype, out=out)


def _fused_call(qtype, otype, x, wq, wsc, out, q, s):
    return w8.w8a8_quant_scaled_mm(x, wq.t(), wsc, qtype, otype, out=out, q=q, a_scales=s)


def build_gemm_workload(layers, Ms, qtype, act_scheme, dev, otype=torch.bfloat16):
    launches, keep = [], []
    code_dtype = torch.float8_e4m3fn if qtype == "fp8" else torch.int8
    # one workspace for the step's split-K problems (they run one after another)
    ws_bytes = max(w8.w8a8_scaled_mm_workspace_size(M, N, K) for M in Ms for _, N, K in layers)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    keep.append(ws)
    seed = 1000
    for M in Ms:
        for name, N, K in layers:
            seed += 1
            w = workloads.weights(N, K, seed=seed, device=dev)
            wq, wsc = w8.w8a8_quant_per_token(w, qtype)   # offline: per-channel weights
            del w
            x = workloads.activations(M, K, seed=seed + 500, device=dev)
            q = torch.empty((M, K), dtype=code_dtype, device=dev)
            out = torch.empty((M, N), dtype=otype, device=dev)
            cs = z = None
            if act_scheme == "azp":  # asymmetric per-token int8, weight code sums offline
                s = torch.empty(M, dtype=torch.float32, device=dev)
                z = torch.empty(M, dtype=torch.int32, device=dev)
                cs = w8.w8a8_colsum(wq)
                qcall, qargs = _azp_quant_call, (x, q, s, z)
                n_sa = M
                qbytes = 3 * M * K + 8 * M
            elif act_scheme == "per_token":
                s = torch.empty(M, dtype=torch.float32, device=dev)
                qcall, qargs = _quant_call, (qtype, x, q, s)
                n_sa = M
                qbytes = 3 * M * K + 4 * M
            else:  # static per-tensor scale from a seeded calibration batch
                calib = workloads.activations(workloads.CALIBRATION_ROWS, K,
                                              seed=workloads.CALIBRATION_SEED, device=dev)
                _, s = w8.w8a8_quant_per_tensor(calib, qtype, dynamic=True)
                del calib
                qcall, qargs = _static_quant_call, (qtype, x, q, s)
                n_sa = 1
                qbytes = 3 * M * K + 4
            mcall, margs = _mm_call, (otype, q, wq, s, wsc, out, ws)
            if act_scheme == "azp":
                mcall, margs = _mm_azp_call, (otype, q, wq, s, z, cs, wsc, out)
            fused = (act_scheme == "per_token"
                     and w8.w8a8_quant_scaled_mm_kernel(M, N, K) == "gemm_dynq_kernel")
            obytes = torch.tensor([], dtype=otype).element_size()
            if fused:  # one kernel quantises the token and runs the product
                launches.append(Launch("gemm", _fused_call, (qtype, otype, x, wq, wsc, out, q, s),
                                       2 * M * N * K,
                                       _gemm_bytes(M, N, K, n_sa, N, obytes) + qbytes - M * K,
                                       f"quant+gemm M={M} {name} {N}x{K}", "gemm_dynq_kernel"))
            else:
                qkern = {"per_token": "quant_rows_kernel", "azp": "quant_rows_azp_kernel"}.get(
                    act_scheme, "quant_tensor_kernel")
                launches.append(Launch("quant", qcall, qargs, 0, qbytes, f"quant M={M} {name}", qkern))
                extra = 4 * M + 4 * N if act_scheme == "azp" else 0  # zero points, code sums
                launches.append(Launch("gemm", mcall, margs, 2 * M * N * K,
                                       _gemm_bytes(M, N, K, n_sa, N, obytes) + extra,
                                       f"gemm M={M} {name} {N}x{K}",
                                       w8.w8a8_scaled_mm_kernel(M, N, K, workspace=act_scheme != "azp")))
            keep += [wq, wsc, x, q, s, out] + ([z, cs] if act_scheme == "azp" else [])
    return launches, keep


# A dynamic per-tensor quantisation is one library call of three kernels: the
# absmax pass (partial maxima), the quantisation, and the scale plus the last
# few KB of codes.
KV_QUANT_KERNELS = "absmax_kernel+quant_tensor_kernel+finish_tail_kernel"


def _kv_quant_call(x, q, s):
    return w8.kv_fp8_scaled_quant(x, scale=s, q=q)


def _kv_dequant_call(q, s, y):
    return w8.kv_fp8_scaled_dequant(q, s, out=y)


def build_kv_workload(dev, layers=workloads.KV_LAYERS):
    launches, keep = [], []
    n = 1
    for d in workloads.KV_SHAPE:
        n *= d
    for layer in range(layers):
        for which in ("k", "v"):
            x = workloads.kv_tensor(layer, which, device=dev)
            q = torch.empty(workloads.KV_SHAPE, dtype=torch.float8_e4m3fn, device=dev)
            s = torch.empty(1, dtype=torch.float32, device=dev)
            y = torch.empty(workloads.KV_SHAPE, dtype=torch.bfloat16, device=dev)
            launches.append(Launch("kv_quant", _kv_quant_call, (x, q, s),
                                   0, 2 * n + n + 2 * n, f"kv quant L{layer}{which}",
                                   KV_QUANT_KERNELS))
            launches.append(Launch("kv_dequant", _kv_dequant_call, (q, s, y),
                                   0, n + 2 * n, f"kv dequant L{layer}{which}",
                                   "kv_dequant_kernel"))
            keep += [x, q, s, y]
    M, K = workloads.PER_TOKEN_STANDALONE
    x = workloads.activations(M, K, seed=0, device=dev)
    q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    s = torch.empty(M, dtype=torch.float32, device=dev)
    launches.append(Launch("quant", _quant_call, ("fp8", x, q, s),
                           0, 3 * M * K + 4 * M, "per-token quant 8192x4096",
                           "quant_rows_kernel"))
    keep += [x, q, s]
    return launches, keep


def shard_scales(S: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.rand(S, generator=g) * 3.8e-3 + 2e-4


def _expand_call(s, rows, sb):
    return w8.w8a8_expand_shard_scales(s, rows, out=sb)


def _requant_call(w, rows, s, out, sh):
    return w8.w8a8_requant_shared_scale(w, rows, s, out=out, shared_scale=sh)


def build_merge_workload(dev):
    """Merged QKV / gate_up weights: the per-shard scales expanded to
    per-channel scales, and the codes rescaled to one shared scale."""
    launches, keep = [], []
    for i, (name, rows, K, qtype) in enumerate(workloads.MERGED_LAYERS):
        N, S = sum(rows), len(rows)
        w = workloads.random_codes((N, K), qtype, seed=40 + i, device=dev).view(
            torch.float8_e4m3fn if qtype == "fp8" else torch.int8)
        s = shard_scales(S, 50 + i).to(dev)
        sb = torch.empty(N, dtype=torch.float32, device=dev)
        out = torch.empty_like(w)
        sh = torch.empty(1, dtype=torch.float32, device=dev)
        launches.append(Launch("merge_expand", _expand_call, (s, rows, sb),
                               0, 4 * S + 4 * N, f"expand {name}", "expand_shard_scales_kernel"))
        launches.append(Launch("merge_requant", _requant_call, (w, rows, s, out, sh),
                               0, 2 * N * K + 4 * S + 4, f"requant {name}", "requant_shared_kernel"))
        keep += [w, s, sb, out, sh]
    return launches, keep


ATTN_KERNELS = "attn_split_kernel+attn_combine_kernel"


def _attn_call(q, kc, vc, starts, max_len, ks, vs, out, ws):
    return w8.kv_fp8_decode_attention(q, kc, vc, starts, max_len, ks, vs, out=out, workspace=ws)


def _paged_attn_call(q, kc, vc, tables, lens, max_len, ks, vs, out, ws):
    return w8.kv_fp8_paged_decode_attention(q, kc, vc, tables, lens, max_len, ks, vs, out=out,
                                            workspace=ws)


PAGE_ROWS = 16  # rows per cache block of the paged layout


def paged_layout(starts, block_size=PAGE_ROWS, seed=7):
    """Block tables of the attention workload's sequences in a paged cache:
    each sequence's rows cut into blocks of block_size rows (the last one
    padded), the blocks placed in a seeded shuffled order. Returns the
    tables [B, max blocks] (-1 past each sequence), the lengths, the block
    count, and for every physical block the contiguous row its rows start at
    (-1 for none)."""
    lens = (starts[1:] - starts[:-1]).to(torch.int32)
    nb = [-(-int(L) // block_size) for L in lens]
    nblk = sum(nb)
    perm = torch.randperm(nblk, generator=torch.Generator().manual_seed(seed))
    tables = torch.full((len(nb), max(nb)), -1, dtype=torch.int32)
    src = torch.full((nblk,), -1, dtype=torch.int64)
    used = 0
    for b, n in enumerate(nb):
        for j in range(n):
            blk = int(perm[used])
            used += 1
            tables[b, j] = blk
            src[blk] = int(starts[b]) + j * block_size
    return tables, lens, nblk, src


def build_attn_workload(dev, layers=workloads.KV_LAYERS, paged=False):
    """Decode attention of one query token per sequence over each layer's
    fp8 KV cache: the layer's K and V [32768, 8, 128] quantised offline
    (kv_fp8_scaled_quant, not timed), 16 sequences of uneven length, 32
    query heads over 8 KV heads. Each layer reads its own cache."""
    launches, keep = [], []
    hq, hkv, d = workloads.ATTN_HEADS
    starts = workloads.attention_seq_starts()
    if paged:
        tables, lens, nblk, src = paged_layout(starts)
        tables_d, lens_d = tables.to(dev), lens.to(dev)
        # physical row r of the paged cache holds contiguous row gather[r] (or zeros)
        offs = torch.arange(PAGE_ROWS).repeat(nblk)
        base = src.repeat_interleave(PAGE_ROWS)
        gather = torch.where(base >= 0, base + offs, torch.full_like(base, -1))
        seq_end = torch.zeros_like(gather)
        for b in range(len(lens)):
            for j in range(tables.shape[1]):
                blk = int(tables[b, j])
                if blk >= 0:
                    seq_end[blk * PAGE_ROWS:(blk + 1) * PAGE_ROWS] = int(starts[b + 1])
        gather = torch.where((gather >= 0) & (gather < seq_end), gather, torch.full_like(gather, -1)).to(dev)
        keep += [tables_d, lens_d, gather]
    B = starts.numel() - 1
    max_len = int((starts[1:] - starts[:-1]).max())
    rows = workloads.KV_SHAPE[0]
    starts_d = starts.to(dev)
    ws = torch.empty(w8.kv_fp8_attention_workspace_size(B, hq, hkv, max_len), dtype=torch.uint8,
                     device=dev)
    keep += [starts_d, ws]
    for layer in range(layers):
        cache = []
        for which in ("k", "v"):
            x = workloads.kv_tensor(layer, which, device=dev)
            q8, sc = w8.kv_fp8_scaled_quant(x)
            del x
            if paged:  # the same rows, blocks of 16 in shuffled places (padding rows zero)
                flat = q8.view(torch.uint8).reshape(q8.shape[0], -1)
                pg = torch.zeros((gather.numel(), flat.shape[1]), dtype=torch.uint8, device=dev)
                ok = gather >= 0
                pg[ok] = flat[gather[ok]]
                q8 = pg.reshape(nblk, PAGE_ROWS, hkv, d)
                del flat
            cache += [q8.view(torch.uint8), sc]
        kc, ks, vc, vs = cache
        q = workloads.attention_queries(B, hq, d, seed=200 + layer, device=dev)
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
        nbytes = 2 * rows * hkv * d + 2 * 2 * B * hq * d + 4 * (B + 1) + 8
        if paged:
            nbytes += 4 * tables.numel()
            launches.append(Launch("attn", _paged_attn_call,
                                   (q, kc, vc, tables_d, lens_d, max_len, ks, vs, out, ws),
                                   4 * rows * hq * d, nbytes, f"paged attention L{layer}", ATTN_KERNELS))
        else:
            launches.append(Launch("attn", _attn_call, (q, kc, vc, starts_d, max_len, ks, vs, out, ws),
                                   4 * rows * hq * d, nbytes, f"attention L{layer}", ATTN_KERNELS))
        keep += [kc, ks, vc, vs, q, out]
    return launches, keep


WORKLOADS = {
    "decode": dict(desc="fp8 e4m3 decode GEMMs, Llama-3-8B QKV/O/gate_up/down at M=1,16,64: "
                        "dynamic per-token activation quant + scaled_mm, per-channel weights, "
                        "bf16 out",
                   layers=workloads.LLAMA3_8B_LAYERS, Ms=workloads.FP8_DECODE_M, qtype="fp8",
                   act="per_token", cpu_n_frac=1),
    "prefill": dict(desc="fp8 e4m3 prefill GEMMs, Llama-3-8B QKV/O/gate_up/down at "
                         "M=512,2048,8192: static per-tensor activation quant + scaled_mm, "
                         "per-channel weights, bf16 out",
                    layers=workloads.LLAMA3_8B_LAYERS, Ms=workloads.FP8_PREFILL_M, qtype="fp8",
                    act="per_tensor_static", cpu_n_frac=2),
    "int8": dict(desc="int8 w8a8 GEMMs, Llama-3-70B unsharded QKV/O/gate_up/down at "
                      "M=1,64,4096: per-token int8 activations + scaled_mm, per-channel int8 "
                      "weights, int32 accumulate, bf16 out",
                 layers=workloads.LLAMA3_70B_LAYERS, Ms=workloads.INT8_70B_M, qtype="int8",
                 act="per_token", cpu_n_frac=1),
    "int8_azp": dict(desc="int8 w8a8 GEMMs with asymmetric activations, Llama-3-70B unsharded "
                          "QKV/O/gate_up/down at M=1,64,4096: per-token int8 scale + zero point, "
                          "per-channel int8 weights with precomputed code sums, zero-point term "
                          "fused in the epilogue, bf16 out",
                     layers=workloads.LLAMA3_70B_LAYERS, Ms=workloads.INT8_70B_M, qtype="int8",
                     act="azp", cpu_n_frac=1),
    "kv": dict(desc="scaled fp8 KV cache: per-tensor dynamic quant + dequant of 32 layers of "
                    "K and V [32768,8,128] bf16, plus per-token fp8 quant of [8192,4096]",
               ),
    "attn": dict(desc="decode attention over the scaled fp8 KV cache: 32 layers, each one query "
                      "token for 16 sequences of uneven length (32768 cache rows), 32 query heads "
                      "over 8 KV heads, head dim 128, K and V dequantised with their per-tensor "
                      "scales as they are read, bf16 out"),
    "attn_paged": dict(desc="decode attention over the scaled fp8 KV cache in a paged layout: the attn "
                            "workload's 32 layers with each sequence's rows in blocks of 16 placed in a "
                            "shuffled order and found through per-sequence block tables"),
    "merge": dict(desc="merged-layer weight scales: per-shard scales of the merged QKV and "
                       "gate_up weights (Llama-3-8B fp8, Llama-3-70B int8) expanded to "
                       "per-channel scales, and the codes rescaled to one shared scale"),
}


# --------------------------------------------------------------------------
def capture(launches, stream):
    """Capture the launches, in order, into one graph on `stream`."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for L in launches:
                L.fn()
    return g


def time_graph(g, stream, reps):
    """Average milliseconds of one replay over `reps` back-to-back replays,
    from HIP events recorded on `stream` (the caller makes it current), and
    the wall time of the loop."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps, time.perf_counter() - t0


def gfx_clock_reader():
    """A function returning (refresh counter, graphics clocks in MHz, one per
    XCD) of the GPU torch sees as device 0, from the power management
    metrics table read through amdsmi, and a function that closes amdsmi;
    None where amdsmi or the device is not available."""
    try:
        import amdsmi
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
    except Exception:
        return None
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
        pick = [h for h in handles
                if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == int(bus)]
        h = pick[0] if pick else (handles[0] if len(handles) == 1 else None)
        if h is None:
            amdsmi.amdsmi_shut_down()
            return None

        def read():
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            clks = m.get("current_gfxclks")
            clks = clks if isinstance(clks, list) else [m.get("current_gfxclk")]
            return (m.get("system_clock_counter"),
                    [float(c) for c in clks if isinstance(c, (int, float)) and 0 < c < 10000])
        read()
        return read, amdsmi.amdsmi_shut_down
    except Exception:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass
        return None


def clock_under_load(g, stream, replay_s, seconds=2.5, settle_s=0.3, period_s=0.02):
    """Graphics clock while graph `g` replays back to back for `seconds`.
    The metrics table behind it is refreshed about once a second, so the
    reading is the mean over the XCDs of each distinct refresh first seen at
    least `settle_s` after the load started. None without amdsmi or without
    such a refresh."""
    rc = gfx_clock_reader()
    if rc is None:
        return None
    read, close = rc
    refreshes, seen, stop = [], set(), threading.Event()
    t_start = time.perf_counter()

    def poll():
        while not stop.is_set():
            try:
                counter, clks = read()
            except Exception:
                return
            if counter not in seen:
                seen.add(counter)
                if clks and time.perf_counter() - t_start >= settle_s:
                    refreshes.append(sum(clks) / len(clks))
            time.sleep(period_s)

    seen.add(read()[0])  # the table as it stood before the load
    batch = max(1, int(0.02 / max(replay_s, 1e-6)))  # about 20 ms of replays per batch
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    try:
        while time.perf_counter() - t_start < seconds:
            for _ in range(batch):
                g.replay()
            stream.synchronize()
    finally:
        stop.set()
        th.join()
        close()
    if not refreshes:
        return None
    return {"gfx_mhz_mean": round(sum(refreshes) / len(refreshes), 1),
            "gfx_mhz_min": round(min(refreshes), 1), "gfx_mhz_max": round(max(refreshes), 1),
            "refreshes": len(refreshes), "spec_mhz": SPEC_GFX_MHZ,
            "source": "amdsmi gpu metrics current_gfxclks (mean over the XCDs), each refresh of the "
                      "table (about 1 per second) taken from %.1f s after the roofline kernel's "
                      "launches began replaying back to back, over %.1f s" % (settle_s, seconds)}


def source_digest(kernel):
    """sha256 over the sources that define `kernel` ("a+b" for a call of
    several kernels): the host code and shared headers, and each source file
    that defines one of its kernels. A PMC traffic record taken from other
    sources no longer describes the kernel."""
    import hashlib
    csrc = os.path.join(ROOT, "int8_scaled_gemm_amd", "csrc")
    names = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp", ".cpp")))
    texts = {}
    for f in names:
        with open(os.path.join(csrc, f), "rb") as fh:
            texts[f] = fh.read()
    parts = [k.split("<")[0].encode() for k in kernel.split("+")]
    used = [f for f in names if not f.endswith(".hip")
            or any(re.search(rb"void\s+" + re.escape(k) + rb"\s*\(", texts[f]) for k in parts)]
    h = hashlib.sha256()
    for f in used:
        h.update(f.encode() + b"\0" + texts[f])
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` in `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE record (calibrated on a plain copy),
    or None when there is none for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    digest = source_digest(kernel)
    for e in rec.get("entries", []):
        if e.get("kernel") == kernel and e.get("workload") == workload \
                and e.get("source_sha256") == digest:
            return e.get("hbm_bytes_per_launch")
    return None


def roofline(name, k, spec, workload):
    """Roofline entry of one kernel: algorithmic bytes (or flops) per launch
    over its average launch time."""
    tile = name.startswith("gemm_tile_kernel")
    if tile:
        achieved = k["flops"] / k["avg_s"] / 1e12
        peak = MFMA_PEAK_TFLOPS[spec["qtype"]]
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s"}
    else:
        achieved = k["nbytes"] / k["avg_s"] / 1e9
        peak = HBM_PEAK_GBS
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s"}
    traffic = recorded_traffic(name, workload)
    roof.update(frac=round(achieved / peak, 4),
                traffic=None if traffic is None else round(traffic),
                kernel=name, launches_per_step=k["launches"],
                avg_launch_us=round(k["avg_s"] * 1e6, 3),
                algorithmic_bytes_per_launch=round(k["nbytes"]),
                algorithmic_flops_per_launch=round(k["flops"]),
                rotated_bytes=round(k["rotated_bytes"]), copies=k["copies"],
                timing="the step's launches of this kernel captured alone (with copies on their "
                       "own buffers up to >= 512 MiB of distinct bytes), replayed, HIP events on "
                       "the launch stream")
    return roof


def cpu_baseline(spec, launches_meta, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    cores = oracle.num_threads()
    if spec is WORKLOADS["merge"]:   # the oracle's requantisation of the 8B merged weights
        dt, nbytes, done = 0.0, 0, 0
        for i, (name, rows, K, qtype) in enumerate(workloads.MERGED_LAYERS):
            w = workloads.random_codes((sum(rows), K), qtype, seed=40 + i).numpy()
            s = shard_scales(len(rows), 50 + i).numpy()
            t0 = time.perf_counter()
            oracle.expand_shard_scales(s, rows)
            oracle.requant_shared_scale(w, qtype, rows, s)
            dt += time.perf_counter() - t0
            nbytes += 2 * w.size + 4 * sum(rows)
            done += 1
            if dt > budget_s:
                break
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
                "kind": "oracle",
                "sample": f"expansion + requantisation of {done} of the step's "
                          f"{len(workloads.MERGED_LAYERS)} merged weights ({dt:.1f} s)"}
    if spec is WORKLOADS["attn"] or spec is WORKLOADS["attn_paged"]:   # attention over whole layers
        paged = spec is WORKLOADS["attn_paged"]
        hq, hkv, d = workloads.ATTN_HEADS
        st = workloads.attention_seq_starts()
        starts = st.numpy()
        B = starts.size - 1
        if paged:
            tables, lens, nblk, src = paged_layout(st)
            tables, lens = tables.numpy(), lens.numpy()
        dt, nbytes, done = 0.0, 0, 0
        for layer in range(4):   # drawing and quantising a layer's cache costs more than its attention
            codes = []
            for which in ("k", "v"):   # the offline quantisation is not timed
                xh = workloads.as_u16(workloads.kv_tensor(layer, which)).reshape(-1)
                c, sc = oracle.kv_quant(xh, xtype="bf16")
                codes += [c.reshape(workloads.KV_SHAPE), sc]
            qh = workloads.as_u16(workloads.attention_queries(B, hq, d, seed=200 + layer))
            if paged:   # the same rows in the paged placement (not timed)
                pk = np.zeros((nblk * PAGE_ROWS, hkv, d), np.uint8)
                pv = np.zeros((nblk * PAGE_ROWS, hkv, d), np.uint8)
                for b in range(B):
                    for j in range(-(-int(lens[b]) // PAGE_ROWS)):
                        r0 = int(starts[b]) + j * PAGE_ROWS
                        n = min(PAGE_ROWS, int(starts[b + 1]) - r0)
                        blk = int(tables[b, j])
                        pk[blk * PAGE_ROWS:blk * PAGE_ROWS + n] = codes[0][r0:r0 + n]
                        pv[blk * PAGE_ROWS:blk * PAGE_ROWS + n] = codes[2][r0:r0 + n]
            t0 = time.perf_counter()
            if paged:
                oracle.decode_attention_fp8kv_paged(qh, pk, pv, tables, lens, PAGE_ROWS, codes[1], codes[3])
            else:
                oracle.decode_attention_fp8kv(qh, codes[0], codes[2], starts, codes[1], codes[3])
            dt += time.perf_counter() - t0
            nbytes += 2 * codes[0].size + 4 * B * hq * d
            done += 1
            if dt > budget_s:
                break
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
                "kind": "oracle",
                "sample": f"attention over {done} of the step's {workloads.KV_LAYERS} layer caches "
                          f"({dt:.1f} s; the offline cache quantisation not timed)"}
    if spec.get("layers") is None:   # kv: quant + dequant of whole layer tensors
        n = 1
        for d in workloads.KV_SHAPE:
            n *= d
        dt, done = 0.0, 0
        for layer in range(workloads.KV_LAYERS):
            for which in ("k", "v"):
                xh = workloads.as_u16(workloads.kv_tensor(layer, which)).reshape(-1)
                t0 = time.perf_counter()
                q, s = oracle.kv_quant(xh, xtype="bf16")
                oracle.kv_dequant(q, s, "bf16")
                dt += time.perf_counter() - t0
                done += 1
                if dt > budget_s:
                    break
            if dt > budget_s:
                break
        return {"value": round(5 * n * done / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
                "kind": "oracle",
                "sample": f"KV quant+dequant of {done} of the step's 64 layer tensors "
                          f"[32768, 8, 128] ({dt:.1f} s; the step's per-token quant not sampled)"}
    frac = spec["cpu_n_frac"]
    flops, dt, done = 0, 0.0, 0
    for M in spec["Ms"]:
        for name, N, K in spec["layers"]:
            Ms = min(M, 64)
            Ns = max(16, N // frac)
            # inputs and the offline weight quantisation are not timed
            x = workloads.as_u16(workloads.activations(Ms, K, seed=7))
            w = workloads.as_u16(workloads.weights(Ns, K, seed=8))
            b, sb = oracle.quant_per_token(w, spec["qtype"], xtype="bf16")
            t0 = time.perf_counter()
            if spec["act"] == "azp":
                a, sa, z = oracle.quant_per_token_azp(x, "bf16")
                oracle.scaled_mm_azp(a, b, sa, z, sb, "bf16")
            else:
                if spec["act"] == "per_token":
                    a, sa = oracle.quant_per_token(x, spec["qtype"], xtype="bf16")
                else:
                    a, sa = oracle.quant_per_tensor(x, spec["qtype"], scale=np.float32(0.05),
                                                    xtype="bf16")
                    sa = np.array([sa], np.float32)
                oracle.scaled_mm(a, b, spec["qtype"], sa, sb, "bf16")
            dt += time.perf_counter() - t0
            flops += 2 * Ms * Ns * K
            done += 1
            if dt > budget_s:
                break
        if dt > budget_s:
            break
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{done} of the step's {len(spec['Ms']) * len(spec['layers'])} (M, layer) "
                      f"GEMMs with their activation quant, on "
                      + ("all" if frac == 1 else f"the first N/{frac}")
                      + f" weight rows and at most 64 rows of M ({flops / 1e9:.2f} GFLOP, "
                      f"{dt:.1f} s)"}


ROTATE_BYTES = 512 << 20   # twice the 256 MB last-level cache
MAX_COPIES = 16


def build(name, spec, dev, otype):
    if name == "kv":
        return build_kv_workload(dev)
    if name == "attn":
        return build_attn_workload(dev)
    if name == "attn_paged":
        return build_attn_workload(dev, paged=True)
    if name == "merge":
        return build_merge_workload(dev)
    return build_gemm_workload(spec["layers"], spec["Ms"], spec["qtype"], spec["act"], dev, otype)


def time_kernels(launches, stream, reps):
    """Per kernel configuration: the step's launches of that kernel captured
    alone and replayed `reps` times, timed with HIP events on the launch
    stream. Where those launches touch fewer than ROTATE_BYTES of distinct
    algorithmic bytes, copies of them on their own buffers are added (up to
    MAX_COPIES in all), so that the replay streams from HBM rather than from
    the last-level cache; per-token quantisations of decode batches (a few KB,
    latency-bound) are timed as they are."""
    kernels = {}
    for name in dict.fromkeys(L.kernel for L in launches):
        group = [L for L in launches if L.kernel == name]
        per_copy = sum(L.nbytes for L in group)
        copies = 1
        if group[0].kind != "quant" and per_copy > 0:
            copies = min(MAX_COPIES, max(1, -(-ROTATE_BYTES // per_copy)))
        timed = list(group)
        for _ in range(copies - 1):
            timed += [L.copy() for L in group]
        g = capture(timed, stream)
        g.replay()
        ms, _ = time_graph(g, stream, reps)
        kernels[name] = dict(launches=len(group), avg_s=ms / 1e3 / len(timed),
                             nbytes=per_copy / len(group),
                             flops=sum(L.flops for L in group) / len(group),
                             rotated_bytes=per_copy * copies, copies=copies, graph=g,
                             replay_s=ms / 1e3, buffers=timed)  # alive while the graph is
    return kernels


def measure(name, args, dev, stream, otype, detail=False):
    """Build one workload, time its step, every kernel configuration, and the
    clock under the dominant kernel; returns the figures and the launches."""
    spec = WORKLOADS[name]
    log(f"[bench] workload {name}: building inputs")
    launches, keep = build(name, spec, dev, otype)
    torch.cuda.synchronize()
    # eager warm-up of every launch (also validates arguments before capture)
    with torch.cuda.stream(stream):
        for L in launches:
            L.fn()
    torch.cuda.synchronize()
    graph = capture(launches, stream)
    with torch.cuda.stream(stream):
        log(f"[bench] {name}: warmup {args.warmup} steps")
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        log(f"[bench] {name}: timing {args.steps} steps")
        step_ms, wall = time_graph(graph, stream, args.steps)
        log(f"[bench] {name}: timing each kernel's launches")
        kernels = time_kernels(launches, stream, args.steps)
        # The roofline entry is for the scaled-product (or KV) kernel that takes
        # the most time per step; the small per-token quantizations of decode
        # batches are latency-bound (a few KB each) and are listed with their
        # latency only.
        kinds = {L.kernel: L.kind for L in launches}
        main_kind = {"kv": "kv_quant", "merge": "merge_requant", "attn": "attn",
                     "attn_paged": "attn"}.get(name, "gemm")
        dom = max((k for k in kernels if kinds[k] == main_kind),
                  key=lambda k: kernels[k]["avg_s"] * kernels[k]["launches"])
        roof = roofline(dom, kernels[dom], spec, name if otype == torch.bfloat16 else f"{name}_{OUT_NAMES[otype]}")
        # The clock the roofline kernel runs at: the matrix-core peak scales
        # with it (HBM bandwidth does not), so an MFMA-bound entry is also
        # given against the peak at the measured clock.
        clock = None
        if args.clock_seconds > 0:
            clock = clock_under_load(kernels[dom]["graph"], stream, kernels[dom]["replay_s"],
                                     seconds=args.clock_seconds)
        if clock is not None and roof["bound"] == "mfma":
            peak_clk = roof["peak"] * clock["gfx_mhz_mean"] / SPEC_GFX_MHZ
            roof.update(peak_at_clock=round(peak_clk, 1),
                        frac_at_clock=round(roof["achieved"] / peak_clk, 4))
        if detail:
            # per-launch times: each launch alone, graph of 10 back-to-back copies
            for L in launches:
                g3 = capture([L] * 10, stream)
                g3.replay()
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(5):
                    g3.replay()
                b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / 50
                log(f"[bench]   {L.label:40s} {us:9.2f} us  {L.nbytes / us / 1e3:8.1f} GB/s  "
                    f"{L.flops / us / 1e6:9.1f} TFLOP/s")
    per_step_flops = sum(L.flops for L in launches)
    per_step_bytes = sum(L.nbytes for L in launches)
    for k in kernels.values():
        del k["graph"], k["buffers"]
    del graph, keep
    return dict(spec=spec, step_ms=step_ms, wall=wall, kernels=kernels, roof=roof, clock=clock,
                flops=per_step_flops, nbytes=per_step_bytes, n_launches=len(launches),
                launches=launches)


def kernel_table(kernels, spec):
    return {n: {"launches_per_step": k["launches"],
                "avg_launch_us": round(k["avg_s"] * 1e6, 3),
                "hbm_frac": round(k["nbytes"] / k["avg_s"] / 1e9 / HBM_PEAK_GBS, 4),
                "mfma_frac": round(k["flops"] / k["avg_s"] / 1e12
                                   / MFMA_PEAK_TFLOPS.get(spec.get("qtype"), 5000.0), 4),
                "rotated_bytes": round(k["rotated_bytes"])}
            for n, k in kernels.items()}


OUT_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
OUT_NAMES = {v: k for k, v in OUT_DTYPES.items()}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode")
    ap.add_argument("--out-dtype", choices=sorted(OUT_DTYPES), default="bf16",
                    help="output type of the GEMM workloads (the prefill configuration has both)")
    ap.add_argument("--mfma-workload", choices=["prefill", "int8", "none"], default="prefill",
                    help="with --workload decode: the MFMA-bound workload whose roofline entry "
                         "is added to the line as roofline_mfma (none: skip)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for the CPU baseline (0: skip)")
    ap.add_argument("--detail", action="store_true", help="per-launch times on stderr")
    ap.add_argument("--clock-seconds", type=float, default=2.5,
                    help="seconds of back-to-back replays of the roofline kernel during which "
                         "the graphics clock is read (0: no clock reading)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 256 MiB on the device 4 times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: multi-GPU runs (collectives, sharding) are "
              "not implemented; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 4}), flush=True)
        return

    w8.load_library()
    stream = torch.cuda.Stream()
    otype = OUT_DTYPES[args.out_dtype]
    r = measure(args.workload, args, dev, stream, otype, detail=args.detail)
    spec = r["spec"]
    step_ms = r["step_ms"]
    if args.workload == "kv":
        value = r["nbytes"] / (step_ms / 1e3) / 1e9
        metric, unit = "scaled fp8 KV cache quant+dequant GB/s (algorithmic bytes)", "GB/s"
        dtype = "fp8e4m3"
    elif args.workload in ("attn", "attn_paged"):
        value = r["nbytes"] / (step_ms / 1e3) / 1e9
        metric, unit = "fp8 KV cache decode attention GB/s (algorithmic bytes)", "GB/s"
        dtype = "fp8e4m3 cache, f32 arithmetic"
    elif args.workload == "merge":
        value = r["nbytes"] / (step_ms / 1e3) / 1e9
        metric, unit = "merged-layer scale expansion + shared-scale requant GB/s (algorithmic bytes)", "GB/s"
        dtype = "u8 codes (fp8e4m3, int8), f32 arithmetic"
    else:
        value = r["flops"] / (step_ms / 1e3) / 1e12
        metric, unit = METRIC, "TFLOP/s"
        dtype = "fp8e4m3" if spec["qtype"] == "fp8" else "int8"

    desc = spec["desc"]
    if spec.get("layers") is not None and args.out_dtype != "bf16":
        desc = desc.replace("bf16 out", f"{args.out_dtype} out")
    result = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded; Llama-3 layer shapes, bf16 N(0,1) activations with 1% "
                "outlier channels x20, N(0,0.02) weights)" if args.workload not in ("kv", "merge", "attn", "attn_paged") else
                "synthetic (seeded; N(0,1) K/V with 0.1% outliers x10)" if args.workload == "kv" else
                "synthetic (seeded; N(0,1) K/V with 0.1% outliers x10 quantised to e4m3fn, "
                "N(0,1) bf16 queries, sequence lengths from seeded weights)" if args.workload in ("attn", "attn_paged") else
                "synthetic (seeded; uniformly random valid codes, shard scales U(2e-4, 4e-3))",
        "config": {"workload": desc, "mode": "hip-graph replay, inputs resident in HBM",
                   "step_bytes": r["nbytes"], "step_flops": r["flops"],
                   "launches_per_step": r["n_launches"], "parallelism": "single GPU"},
        "roofline": r["roof"],
        "clock": r["clock"],
        "kernels": kernel_table(r["kernels"], spec),
    }
    launches = r.pop("launches")
    if args.workload == "decode" and args.mfma_workload != "none":
        # The metric's other half: the MFMA-bound roofline of the prefill (or
        # int8) GEMMs, measured in the same run the same way.
        del launches
        torch.cuda.empty_cache()
        m = measure(args.mfma_workload, args, dev, stream, torch.bfloat16)
        m.pop("launches")
        mroof = dict(m["roof"])
        mroof.update(workload=m["spec"]["desc"], clock=m["clock"],
                     step_value=round(m["flops"] / (m["step_ms"] / 1e3) / 1e12, 3),
                     step_unit="TFLOP/s", step_ms=round(m["step_ms"], 4))
        result["roofline_mfma"] = mroof
        result["kernels_mfma"] = kernel_table(m["kernels"], m["spec"])
        torch.cuda.empty_cache()
    if args.cpu_budget > 0:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(spec, None, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    log(f"[bench] wall {r['wall']:.3f}s for the timed loop")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
