#!/usr/bin/env python
"""Benchmark of the fused-dequantize Q4_K GEMV on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c2|c1|c3|c4|n1|c5|...]

Default workload: Q4_K GEMV, input_dim 4096 x output_dim 4096, batch 1,
fp32 activations, 64 distinct weight copies (604 MB, more than twice the
256 MB Infinity Cache) used in rotation so that every call streams its
weights from HBM.  A step is one q4k_gemv call on the next copy.  Inputs
are generated (seeded, synthetic) and copied to HBM before timing.  The
timed region holds device work only: every rotating copy gets one untimed
call first (its pages touched, as for resident inputs), a delay kernel
keeps the GPU busy while the host submits the timed calls (one launch per
call for up to 512 steps, replays of a captured HIP graph with one node per
call above), and HIP events on the launch stream bracket exactly the timed
steps.

Prints one JSON line: mean us/call (value), achieved GB/s of algorithmic
bytes against the 8 TB/s HBM peak (roofline), and the CPU oracle timed on
a bounded sample on this host (cpu_baseline).

Other workloads (measurement of the sibling paths, same JSON shape):
  c1  Q4_K GEMV 1024 x 1024, batch 1 (911 rotating copies)
  c3  Q4_K FFN pair: up 4096->14336 then down 14336->4096, batch 1; a step
      is the pair (9 rotating pairs)
  c4  Q4_K prefill 64 tokens x 4096 -> 4096 (64 rotating weight copies)
  n1  Q4_K few-token product, 4 tokens x 4096 -> 4096 (64 rotating weight
      copies; the batched matrix-core GEMV, weights read once for all tokens)
  c5  ternary GEMV 4096 x 4096, batch 1 (128 rotating copies)
  q40 Q4_0 GEMV 4096 x 4096, batch 1 (64 rotating copies; the Q4_K page's
      follow-up format, the same 9.4 MB of weights per call as c2)
  q6k Q6_K GEMV 4096 x 4096, batch 1 (43 rotating copies of 13.8 MB; the
      page's other follow-up format)
  t64 ternary prefill 64 tokens x 4096 -> 4096 (128 rotating code copies)
  c2t c2 with the weights relayouted once (before timing) into the tiled
      block order and multiplied by q4k_gemv_tiled
  c3t c3 with both matrices in the tiled block order
  copy  plain 64 MiB device-to-device copy kernel (4 rotating buffer pairs):
      the kernel of known traffic used to scale hardware byte counters
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
ROTATION_BYTES = 2 * 256 * 2 ** 20


def kernel_hash(files):
    """Hash of a kernel's sources and of the build script that holds the
    compile flags (a committed profile is valid only for the same code)."""
    h = hashlib.sha256()
    for f in list(files) + ["q4_packed_weight_amd/build.py"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


GEMV_SRC = ["q4_packed_weight_amd/csrc/q4k_gemv.hip",
            "q4_packed_weight_amd/csrc/q4k_gemv_mfma.hip",
            "q4_packed_weight_amd/csrc/device_common.h"]
Q40_SRC = GEMV_SRC + ["q4_packed_weight_amd/csrc/q4_0_gemv_mfma.hip"]
PREFILL_SRC = ["q4_packed_weight_amd/csrc/q4k_prefill_splitk.hip",
               "q4_packed_weight_amd/csrc/device_common.h"]
TERNARY_SRC = ["q4_packed_weight_amd/csrc/ternary_gemv.hip",
               "q4_packed_weight_amd/csrc/device_common.h"]
TILED_SRC = ["q4_packed_weight_amd/csrc/q4k_tiled.hip",
             "q4_packed_weight_amd/csrc/device_common.h"]
BATCH_SRC = ["q4_packed_weight_amd/csrc/q4k_gemv_batch.hip",
             "q4_packed_weight_amd/csrc/device_common.h"]
TERNARY_MM_SRC = ["q4_packed_weight_amd/csrc/ternary_matmul.hip",
                  "q4_packed_weight_amd/csrc/device_common.h"]


class Workload:
    """Inputs resident on the GPU plus a `call(i)` that runs step i."""


MFMA_DTYPE = "f32 (x as exact fp16 hi+lo MFMA operands, fp32 accumulation)"


def row_slices(n_rows, n_chunks=64):
    """Contiguous output-row ranges covering [0, n_rows): the CPU oracle's
    work split for the multi-threaded baseline (rows are independent)."""
    b = [n_rows * i // n_chunks for i in range(n_chunks + 1)]
    return [(o0, o1) for o0, o1 in zip(b, b[1:]) if o1 > o0]


def make_workload(name, torch, binding, synth):
    import numpy as np
    dev = "cuda:0"
    wl = Workload()
    wl.name = name

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if name in ("c1", "c2"):
        K = N = 1024 if name == "c1" else 4096
        cfg = synth.C1_Q4K_1K if name == "c1" else synth.C2_Q4K_4K
        wbytes = N * K // 256 * 144
        copies = 64 if name == "c2" else -(-ROTATION_BYTES // wbytes)
        wl.W = [to_dev(synth.q4k_weights(N, K, config=cfg, copy=c)) for c in range(copies)]
        wl.x = to_dev(synth.activations(K, config=cfg))
        wl.y = torch.empty(N, dtype=torch.float32, device=dev)
        wl.call = lambda i: binding.q4k_gemv(wl.x, wl.W[i % copies], K, N, wl.y)
        wl.copies = copies
        wl.bytes = wbytes + 4 * K + 4 * N
        wl.flops = 2 * K * N
        # 4096 x 4096 runs the matrix-core form (256 workgroups of 16 rows)
        wl.kernel = "q4k_gemv_mfma_kernel<false>" if name == "c2" else "q4k_gemv_kernel"
        wl.src_files = GEMV_SRC
        wl.config = {"workload": f"q4k_gemv {K}x{N} batch 1", "input_dim": K,
                     "output_dim": N, "batch": 1, "rotating_copies": copies,
                     "weight_bytes_per_copy": wbytes}
        wl.metric = f"Q4_K GEMV us/call + achieved HBM GB/s (% peak) at {K}x{N}, batch 1"

        wl.dtype = MFMA_DTYPE if name == "c2" else "f32"

        def cpu(oracle):
            w0 = wl.W[0].cpu().numpy().reshape(-1)
            x0 = wl.x.cpu().numpy()
            rb = K // 256 * 144
            return [lambda a=a, b=b: oracle.q4k_gemv(x0, w0[a * rb:b * rb], K, b - a)
                    for a, b in row_slices(N)], 1.0, f"oracle q4k_gemv {K}x{N}, full call"
        wl.cpu = cpu
    elif name == "c3":
        K1, N1, K2, N2 = 4096, 14336, 14336, 4096
        b1, b2 = N1 * K1 // 256 * 144, N2 * K2 // 256 * 144
        copies = -(-ROTATION_BYTES // (b1 + b2))
        wl.Wu = [to_dev(synth.q4k_weights(N1, K1, config=synth.C3_FFN, copy=c)) for c in range(copies)]
        wl.Wd = [to_dev(synth.q4k_weights(N2, K2, config=synth.C3_FFN, copy=c, extra=1)) for c in range(copies)]
        wl.xu = to_dev(synth.activations(K1, config=synth.C3_FFN))
        wl.xd = to_dev(synth.activations(K2, config=synth.C3_FFN, extra=1))
        wl.yu = torch.empty(N1, dtype=torch.float32, device=dev)
        wl.yd = torch.empty(N2, dtype=torch.float32, device=dev)

        def call(i):
            binding.q4k_gemv(wl.xu, wl.Wu[i % copies], K1, N1, wl.yu)
            binding.q4k_gemv(wl.xd, wl.Wd[i % copies], K2, N2, wl.yd)
        wl.call = call
        wl.copies = copies
        wl.bytes = b1 + b2 + 4 * (K1 + N1 + K2 + N2)
        wl.flops = 2 * (K1 * N1 + K2 * N2)
        wl.kernel = "q4k_gemv_walk_kernel (up: 4 row groups per workgroup; down: 1, staged per wave)"
        wl.src_files = GEMV_SRC
        wl.config = {"workload": "q4k_gemv FFN pair 4096->14336 + 14336->4096 batch 1",
                     "rotating_pairs": copies}
        wl.metric = "Q4_K FFN GEMV pair us/pair + achieved HBM GB/s (% peak), batch 1"

        def cpu(oracle):
            wu, wd = wl.Wu[0].cpu().numpy().reshape(-1), wl.Wd[0].cpu().numpy().reshape(-1)
            xu, xd = wl.xu.cpu().numpy(), wl.xd.cpu().numpy()
            ru, rd = K1 // 256 * 144, K2 // 256 * 144
            return ([lambda a=a, b=b: oracle.q4k_gemv(xu, wu[a * ru:b * ru], K1, b - a)
                     for a, b in row_slices(N1)] +
                    [lambda a=a, b=b: oracle.q4k_gemv(xd, wd[a * rd:b * rd], K2, b - a)
                     for a, b in row_slices(N2)]), 1.0, "oracle q4k_gemv up+down pair, full call"
        wl.cpu = cpu
    elif name == "n1":
        # the few-token regime between the GEMV and the prefill tiles: 4
        # tokens x 4096 -> 4096 runs the batched matrix-core GEMV, every
        # weight byte read once for all four
        M, K, N = 4, 4096, 4096
        wbytes = N * K // 256 * 144
        copies = 64
        wl.W = [to_dev(synth.q4k_weights(N, K, config=synth.C2_Q4K_4K, copy=c)) for c in range(copies)]
        wl.X = to_dev(synth.activations(K, n_tokens=M, config=synth.C2_Q4K_4K))
        wl.Y = torch.empty(M, N, dtype=torch.float32, device=dev)
        wl.call = lambda i: binding.q4k_matmul(wl.X, wl.W[i % copies], M, K, N, wl.Y)
        wl.copies = copies
        wl.bytes = wbytes + 4 * M * K + 4 * M * N
        wl.flops = 2 * M * K * N
        wl.kernel = "q4k_gemv_batch_kernel<4, false, 16>"
        wl.src_files = BATCH_SRC
        wl.config = {"workload": "q4k_matmul 4 tokens x 4096 -> 4096", "tokens": M,
                     "input_dim": K, "output_dim": N, "rotating_copies": copies}
        wl.metric = "Q4_K few-token matmul us/call + achieved HBM GB/s (% peak), 4x4096x4096"

        wl.dtype = MFMA_DTYPE

        def cpu(oracle):
            w0, X0 = wl.W[0].cpu().numpy().reshape(-1), wl.X.cpu().numpy()
            rb = K // 256 * 144
            return [lambda a=a, b=b: oracle.q4k_matmul(X0[:1], w0[a * rb:b * rb], 1, K, b - a)
                    for a, b in row_slices(N)], M / 1, \
                "oracle q4k_matmul on 1 of 4 token rows, scaled x4 to a call"
        wl.cpu = cpu
    elif name == "c4":
        M, K, N = 64, 4096, 4096
        wbytes = N * K // 256 * 144
        copies = 64
        wl.W = [to_dev(synth.q4k_weights(N, K, config=synth.C4_PREFILL, copy=c)) for c in range(copies)]
        wl.X = to_dev(synth.activations(K, n_tokens=M, config=synth.C4_PREFILL))
        wl.Y = torch.empty(M, N, dtype=torch.float32, device=dev)
        form = PREFILL_FORM
        wl.call = (lambda i: binding.q4k_matmul(wl.X, wl.W[i % copies], M, K, N, wl.Y)) if form == 0 \
            else (lambda i: binding.q4k_matmul_shaped(wl.X, wl.W[i % copies], M, K, N, wl.Y, form))
        wl.copies = copies
        wl.bytes = wbytes + 4 * M * K + 4 * M * N
        wl.flops = 2 * M * K * N
        wl.kernel = "q4k_prefill_splitk_kernel"
        wl.src_files = PREFILL_SRC
        wl.config = {"workload": "q4k_matmul prefill 64 tokens x 4096 -> 4096",
                     "tokens": M, "input_dim": K, "output_dim": N, "rotating_copies": copies}
        if form:
            wl.config["form"] = form
        wl.metric = "Q4_K prefill matmul us/call + achieved TFLOP/s (% fp16 MFMA peak), 64x4096x4096"

        wl.dtype = MFMA_DTYPE

        def cpu(oracle):
            w0, X0 = wl.W[0].cpu().numpy().reshape(-1), wl.X.cpu().numpy()
            rb = K // 256 * 144
            return [lambda a=a, b=b: oracle.q4k_matmul(X0[:2], w0[a * rb:b * rb], 2, K, b - a)
                    for a, b in row_slices(N)], M / 2, \
                "oracle q4k_matmul on 2 of 64 token rows, scaled x32 to a call"
        wl.cpu = cpu
    elif name == "c5":
        K = N = 4096
        cbytes = N * K // 4
        copies = -(-ROTATION_BYTES // cbytes)
        wl.C = [to_dev(synth.ternary_codes(N, K, copy=c)[0]) for c in range(copies)]
        wl.x = to_dev(synth.activations(K, config=synth.C5_TERNARY))
        wl.scale = float(synth.ternary_scale())
        wl.y = torch.empty(N, dtype=torch.float32, device=dev)
        wl.call = lambda i: binding.ternary_gemv(wl.x, wl.C[i % copies], wl.scale, K, N, wl.y)
        wl.copies = copies
        wl.bytes = cbytes + 4 * K + 4 * N + 4
        wl.flops = 2 * K * N
        wl.kernel = "ternary_gemv_kernel"
        wl.data = "synthetic (seeded numpy generators; random ternary codes, N(0,1) activations)"
        wl.src_files = TERNARY_SRC
        wl.config = {"workload": "ternary_gemv 4096x4096 batch 1", "input_dim": K,
                     "output_dim": N, "rotating_copies": copies}
        wl.metric = "Ternary GEMV us/call + achieved HBM GB/s (% peak) at 4096x4096, batch 1"

        def cpu(oracle):
            c0, x0 = wl.C[0].cpu().numpy().reshape(-1), wl.x.cpu().numpy()
            rb = K // 4
            return [lambda a=a, b=b: oracle.ternary_gemv(x0, c0[a * rb:b * rb], wl.scale, K, b - a)
                    for a, b in row_slices(N)], 1.0, "oracle ternary_gemv 4096x4096, full call"
        wl.cpu = cpu
    elif name == "q40":
        K = N = 4096
        wbytes = N * K // 32 * 18
        copies = 64
        wl.W = [to_dev(synth.q4_0_weights(N, K, copy=c)) for c in range(copies)]
        wl.x = to_dev(synth.activations(K, config=synth.Q40_4K))
        wl.y = torch.empty(N, dtype=torch.float32, device=dev)
        wl.call = lambda i: binding.q4_0_gemv(wl.x, wl.W[i % copies], K, N, wl.y)
        wl.copies = copies
        wl.bytes = wbytes + 4 * K + 4 * N
        wl.flops = 2 * K * N
        wl.kernel = "q4_0_gemv_mfma_kernel"
        wl.src_files = Q40_SRC
        wl.data = "synthetic (seeded numpy generators; random Q4_0 blocks, N(0,1) activations)"
        wl.config = {"workload": f"q4_0_gemv {K}x{N} batch 1", "input_dim": K,
                     "output_dim": N, "batch": 1, "rotating_copies": copies,
                     "weight_bytes_per_copy": wbytes}
        wl.metric = f"Q4_0 GEMV us/call + achieved HBM GB/s (% peak) at {K}x{N}, batch 1"

        def cpu(oracle):
            w0 = wl.W[0].cpu().numpy().reshape(-1)
            x0 = wl.x.cpu().numpy()
            rb = K // 32 * 18
            return [lambda a=a, b=b: oracle.q4_0_gemv(x0, w0[a * rb:b * rb], K, b - a)
                    for a, b in row_slices(N)], 1.0, f"oracle q4_0_gemv {K}x{N}, full call"
        wl.cpu = cpu
    elif name == "q6k":
        K = N = 4096
        wbytes = N * K // 256 * 210
        copies = -(-ROTATION_BYTES // wbytes)
        wl.W = [to_dev(synth.q6k_weights(N, K, copy=c)) for c in range(copies)]
        wl.x = to_dev(synth.activations(K, config=synth.Q6K_4K))
        wl.y = torch.empty(N, dtype=torch.float32, device=dev)
        wl.call = lambda i: binding.q6k_gemv(wl.x, wl.W[i % copies], K, N, wl.y)
        wl.copies = copies
        wl.bytes = wbytes + 4 * K + 4 * N
        wl.flops = 2 * K * N
        wl.kernel = "q4k_gemv_kernel<Q6K, 64, 2, 1, 4>"
        wl.src_files = GEMV_SRC
        wl.data = "synthetic (seeded numpy generators; random Q6_K blocks, N(0,1) activations)"
        wl.config = {"workload": f"q6k_gemv {K}x{N} batch 1", "input_dim": K,
                     "output_dim": N, "batch": 1, "rotating_copies": copies,
                     "weight_bytes_per_copy": wbytes}
        wl.metric = f"Q6_K GEMV us/call + achieved HBM GB/s (% peak) at {K}x{N}, batch 1"

        def cpu(oracle):
            w0 = wl.W[0].cpu().numpy().reshape(-1)
            x0 = wl.x.cpu().numpy()
            rb = K // 256 * 210
            return [lambda a=a, b=b: oracle.q6k_gemv(x0, w0[a * rb:b * rb], K, b - a)
                    for a, b in row_slices(N)], 1.0, f"oracle q6k_gemv {K}x{N}, full call"
        wl.cpu = cpu
    elif name == "t64":
        M, K, N = 64, 4096, 4096
        cbytes = N * K // 4
        copies = -(-ROTATION_BYTES // cbytes)
        wl.C = [to_dev(synth.ternary_codes(N, K, copy=c)[0]) for c in range(copies)]
        wl.X = to_dev(synth.activations(K, n_tokens=M, config=synth.C5_TERNARY))
        wl.scale = float(synth.ternary_scale())
        wl.Y = torch.empty(M, N, dtype=torch.float32, device=dev)
        wl.call = lambda i: binding.ternary_matmul(wl.X, wl.C[i % copies], wl.scale, M, K, N, wl.Y)
        wl.copies = copies
        wl.bytes = cbytes + 4 * M * K + 4 * M * N
        wl.flops = 2 * M * K * N
        wl.kernel = "ternary_matmul_kernel"
        wl.src_files = TERNARY_MM_SRC
        wl.data = "synthetic (seeded numpy generators; random ternary codes, N(0,1) activations)"
        wl.config = {"workload": "ternary_matmul prefill 64 tokens x 4096 -> 4096",
                     "tokens": M, "input_dim": K, "output_dim": N, "rotating_copies": copies}
        wl.metric = "Ternary prefill matmul us/call + achieved TFLOP/s (% fp16 MFMA peak), 64x4096x4096"

        wl.dtype = MFMA_DTYPE

        def cpu(oracle):
            c0, X0 = wl.C[0].cpu().numpy().reshape(-1), wl.X.cpu().numpy()
            rb = K // 4
            return [lambda a=a, b=b: oracle.ternary_matmul(X0[:2], c0[a * rb:b * rb], wl.scale,
                                                           2, K, b - a)
                    for a, b in row_slices(N)], M / 2, \
                "oracle ternary_matmul on 2 of 64 token rows, scaled x32 to a call"
        wl.cpu = cpu
    elif name in ("c2t", "c3t"):
        # the canonical matrices of c2 / c3, each relayouted once into the
        # tiled block order (outside the timed region: a load-time step)
        mats = ([(4096, 4096, synth.C2_Q4K_4K, 0)] if name == "c2t" else
                [(4096, 14336, synth.C3_FFN, 0), (14336, 4096, synth.C3_FFN, 1)])
        per = sum(N * K // 256 * 144 for K, N, _, _ in mats)
        copies = 64 if name == "c2t" else -(-ROTATION_BYTES // per)
        wl.T = [[] for _ in mats]
        relayout_ms = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for m, (K, N, cfg, extra) in enumerate(mats):
            for c in range(copies):
                w = to_dev(synth.q4k_weights(N, K, config=cfg, copy=c, extra=extra))
                t = torch.empty(binding.q4k_tiled_size(K, N), dtype=torch.uint8, device=dev)
                e0.record()
                binding.q4k_relayout_tiled(w, K, N, t)
                e1.record()
                torch.cuda.synchronize()
                relayout_ms.append((m, e0.elapsed_time(e1)))
                wl.T[m].append(t)
                del w
        wl.xs = [to_dev(synth.activations(K, config=cfg, extra=extra)) for K, _, cfg, extra in mats]
        wl.ys = [torch.empty(N, dtype=torch.float32, device=dev) for _, N, _, _ in mats]

        def call(i):
            for m, (K, N, _, _) in enumerate(mats):
                binding.q4k_gemv_tiled(wl.xs[m], wl.T[m][i % copies], K, N, wl.ys[m])
        wl.call = call
        wl.copies = copies
        wl.W = wl.T[0] if name == "c2t" else None
        wl.bytes = sum(N * K // 256 * 144 + 4 * (K + N) for K, N, _, _ in mats)
        wl.flops = sum(2 * K * N for K, N, _, _ in mats)
        wl.kernel = "q4k_gemv_tiled_kernel"
        wl.src_files = TILED_SRC
        relayout_us = []
        for m in range(len(mats)):
            ts = sorted(t for mm, t in relayout_ms if mm == m)
            relayout_us.append(round(1000 * ts[len(ts) // 2], 1))  # median, one call each
        if name == "c2t":
            wl.config = {"workload": "q4k_gemv_tiled 4096x4096 batch 1 (tiled block order)",
                         "input_dim": 4096, "output_dim": 4096, "batch": 1,
                         "rotating_copies": copies, "weight_bytes_per_copy": per,
                         "relayout_us_once_per_matrix": relayout_us[0]}
            wl.metric = "Q4_K GEMV (tiled block order) us/call + achieved HBM GB/s (% peak) at 4096x4096, batch 1"
        else:
            wl.config = {"workload": "q4k_gemv_tiled FFN pair 4096->14336 + 14336->4096 batch 1 "
                                     "(tiled block order)", "rotating_pairs": copies,
                         "relayout_us_once_per_matrix": relayout_us}
            wl.metric = "Q4_K FFN GEMV pair (tiled block order) us/pair + achieved HBM GB/s (% peak), batch 1"
        wl.data = "synthetic (seeded numpy generators; random Q4_K blocks relayouted into the tiled order, N(0,1) activations)"

        wl.dtype = MFMA_DTYPE

        def cpu(oracle):
            # the oracle multiplies the canonical matrices (the same weights)
            ws = [synth.q4k_weights(N, K, config=cfg, copy=0, extra=extra).reshape(-1)
                  for K, N, cfg, extra in mats]
            xs = [x.cpu().numpy() for x in wl.xs]
            jobs = []
            for m, (K, N, _, _) in enumerate(mats):
                rb = K // 256 * 144
                jobs += [lambda m=m, K=K, rb=rb, a=a, b=b: oracle.q4k_gemv(xs[m], ws[m][a * rb:b * rb], K, b - a)
                         for a, b in row_slices(N)]
            return jobs, 1.0, "oracle q4k_gemv on the canonical matrices, full call"
        wl.cpu = cpu
    elif name == "copy":
        nbytes = 64 * 2 ** 20
        copies = 4
        wl.src = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(c + 1) for c in range(copies)]
        wl.dst = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for c in range(copies)]
        wl.call = lambda i: binding.bench_copy(wl.src[i % copies], wl.dst[i % copies])
        wl.copies = copies
        wl.bytes = 2 * nbytes
        wl.flops = 0
        wl.kernel = "copy_kernel"
        wl.data = "synthetic (constant-filled device buffers)"
        wl.src_files = ["q4_packed_weight_amd/csrc/bench_kernels.hip"]
        wl.config = {"workload": "device copy 64 MiB (read 64 MiB + write 64 MiB)",
                     "rotating_pairs": copies}
        wl.metric = "copy kernel us/call + GB/s (read + write bytes)"
        wl.cpu = None
    else:
        raise SystemExit(f"unknown workload {name}")
    return wl


def capture(torch, wl, start, count):
    """A HIP graph of `count` consecutive steps starting at step `start`."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(start, start + count):
                wl.call(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


DELAY_NS = 1_000_000
EAGER_DELAY_NS_PER_STEP = 20_000  # host time to enqueue one call, with margin
PREFILL_FORM = 0  # c4: 0 = q4k_matmul's own choice, else the q4k_matmul_shaped form


def time_steps(torch, binding, wl, steps, launch, graphs, first=0):
    """Mean ms per step over exactly `steps` steps, HIP events on the stream
    the kernels run on, and the host's submission time of those steps.

    After the synchronization a delay kernel (1 ms, or 20 us per step for
    individual launches) is enqueued ahead of the start event: while it
    runs, the host submits the timed calls, so the events time the device's
    execution of exactly the `steps` calls and not the host's submission."""
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    delay = DELAY_NS if launch != "eager" else max(DELAY_NS, EAGER_DELAY_NS_PER_STEP * steps)
    binding.bench_delay(min(delay, 100_000_000))
    start.record(stream)
    t0 = time.perf_counter()
    if launch == "eager":
        # continue the rotation after the warmup calls, so that no timed call
        # finds its weights left in the Infinity Cache by a recent one
        for i in range(first, first + steps):
            wl.call(i)
    else:
        full, rem = graphs
        G = wl.copies
        for _ in range(steps // G):
            full.replay()
        if rem is not None:
            rem.replay()
    host_s = time.perf_counter() - t0
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, host_s


def context_measurements(torch, binding, wl, launch_graph_len):
    """Launch floor (empty kernel) and a streaming read of the same rotating
    weight copies, each as graph replays like the main measurement."""
    out = {}
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
        for _ in range(launch_graph_len):
            binding.bench_empty()
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    out["empty_kernel_us"] = round(e0.elapsed_time(e1) * 1000 / (reps * launch_graph_len), 3)

    bufs = getattr(wl, "W", None) or getattr(wl, "C", None)
    if wl.name == "copy":
        bufs = None
    if bufs:
        sink = torch.zeros(65536, dtype=torch.int32, device="cuda:0")
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s), torch.cuda.graph(g2, stream=s):
            for b in bufs:
                binding.bench_stream_read(b, sink)
        torch.cuda.current_stream().wait_stream(s)
        for _ in range(3):
            g2.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g2.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000 / (reps * len(bufs))
        nbytes = bufs[0].numel()
        out["stream_read_same_bytes_us"] = round(us, 3)
        out["stream_read_GBps"] = round(nbytes / us / 1e3, 1)
        # the runtime's own device-to-device copy of each rotating buffer
        # (graph memcpy nodes): reads the same bytes and writes them once
        dst = torch.empty_like(bufs[0])
        g3 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s), torch.cuda.graph(g3, stream=s):
            for b in bufs:
                dst.copy_(b)
        torch.cuda.current_stream().wait_stream(s)
        for _ in range(3):
            g3.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g3.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000 / (reps * len(bufs))
        out["memcpy_d2d_same_bytes_us"] = round(us, 3)
        out["memcpy_d2d_GBps_read_plus_write"] = round(2 * nbytes / us / 1e3, 1)
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, seconds):
    """The oracle (plain scalar C, untouched) timed on the host: one thread,
    then all threads of the host's share (at most 16) each taking whole
    output-row ranges.  The oracle releases the interpreter lock inside its
    C calls, so the row ranges run in parallel."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    jobs, scale, sample = wl.cpu(oracle)

    def timed(fn, budget):
        fn()  # warm caches / page in
        times = []
        t_end = time.perf_counter() + budget
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        times.sort()
        return times[len(times) // 2] * scale, len(times)

    def serial():
        for j in jobs:
            j()
    threads = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(threads) as pool:
        def parallel():
            list(pool.map(lambda j: j(), jobs))
        t1, n1 = timed(serial, seconds / 2)
        tn, nn = timed(parallel, seconds / 2)
    return {"value": round(tn * 1e6, 1), "unit": "us/call", "cores": threads, "kind": "oracle",
            "sample": f"{sample}; output rows split into {len(jobs)} ranges over {threads} "
                      f"threads, median of {nn} calls (1 thread: median of {n1} calls)",
            "value_1_thread": round(t1 * 1e6, 1), "cpu_model": cpu_model(),
            "host_cpus_visible": os.cpu_count()}


TRAFFIC_FILES = {"c1": "q4k_gemv_1024x1024_b1.traffic.json",
                 "c2": "q4k_gemv_4096x4096_b1.traffic.json",
                 "c3": "q4k_gemv_ffn_4096x14336_pair.traffic.json",
                 "c4": "q4k_prefill_64x4096x4096.traffic.json",
                 "n1": "q4k_matmul_4x4096x4096.traffic.json",
                 "c5": "ternary_gemv_4096x4096_b1.traffic.json",
                 "q40": "q4_0_gemv_4096x4096_b1.traffic.json",
                 "q6k": "q6k_gemv_4096x4096_b1.traffic.json",
                 "t64": "ternary_matmul_64x4096x4096.traffic.json",
                 "c2t": "q4k_gemv_tiled_4096x4096_b1.traffic.json",
                 "c3t": "q4k_gemv_tiled_ffn_4096x14336_pair.traffic.json"}


def traffic_for(wl):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by the copy-kernel calibration), if
    it was taken on the current kernel source; else None."""
    name = TRAFFIC_FILES.get(wl.name)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash(wl.src_files):
        return None
    return t.get("traffic_bytes_per_launch")


def trace_for(wl, key="trace_avg_ns_per_step"):
    """Average (or, with key trace_median_ns_per_step, median) kernel-trace
    duration (us per step, rocprofv3 --kernel-trace) from the committed
    profile summary, if it was taken on the current kernel source; else
    None."""
    name = TRAFFIC_FILES.get(wl.name)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash(wl.src_files) or key not in t:
        return None
    return round(t[key] / 1000.0, 3)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64000)
    ap.add_argument("--warmup", type=int, default=6400)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "n1", "c5", "q40", "q6k", "t64", "c2t", "c3t", "copy"])
    ap.add_argument("--launch", default="auto", choices=["auto", "graph", "eager"],
                    help="auto: individual launches for up to 512 steps (queued while a "
                         "delay kernel keeps the GPU busy), graph replays above")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--prefill-form", type=int, default=0,
                    help="c4 only: force a q4k_matmul_shaped form (0 = q4k_matmul)")
    args = ap.parse_args()
    global PREFILL_FORM
    PREFILL_FORM = args.prefill_form

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the Q4_K GEMV path here has no multi-GPU form.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from q4_packed_weight_amd import binding, synth

    binding.lib()  # fail loudly now if the HIP library is missing
    wl = make_workload(args.workload, torch, binding, synth)
    steps, warmup = args.steps, args.warmup
    print(f"[bench] workload {wl.name}: {wl.config}", file=sys.stderr, flush=True)

    # A replay of a captured graph costs the device a few microseconds of its
    # own on top of its nodes, which a short run cannot amortize; up to 512
    # steps the calls are therefore launched one by one behind the delay
    # kernel (the host enqueues them while it runs), above that as graph
    # replays.
    if args.launch == "auto":
        args.launch = "eager" if steps <= 512 else "graph"
    # One untimed call on every rotating copy first, so that every input is
    # resident when the timed region starts: a copy's first call pays for the
    # first touch of its pages (measured at 4096x4096: 20 timed calls after 5
    # warm-up calls 4.90 us/call, after 64 or 200 4.71-4.74), and each call
    # of a short run would otherwise be a first touch.  This also lets the
    # library allocate its per-device workspace outside any graph capture.
    for i in range(wl.copies):
        wl.call(i)
    torch.cuda.synchronize()
    graphs = None
    if args.launch == "graph":
        full = capture(torch, wl, 0, wl.copies)
        rem = capture(torch, wl, 0, steps % wl.copies) if steps % wl.copies else None
        graphs = (full, rem)
        for _ in range(max(1, warmup // wl.copies)):
            full.replay()
    else:
        for i in range(warmup):
            wl.call(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {steps} steps", file=sys.stderr, flush=True)

    ms, host_s = time_steps(torch, binding, wl, steps, args.launch, graphs, first=warmup)
    us = ms * 1000.0
    torch.cuda.synchronize()
    print(f"[bench] {us:.3f} us/step", file=sys.stderr, flush=True)

    gbps = wl.bytes / us / 1e3
    if wl.name in ("c4", "t64"):
        tflops = wl.flops / us / 1e6
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": traffic_for(wl)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "traffic": traffic_for(wl)}

    line = {
        "metric": wl.metric,
        "value": round(us, 3),
        "unit": "us/pair" if wl.name in ("c3", "c3t") else "us/call",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": getattr(wl, "dtype", "f32"),
        "data": getattr(wl, "data", "synthetic (seeded numpy generators; random Q4_K blocks, "
                                       "N(0,1) activations)"),
        "config": dict(wl.config, launch="hipGraph replay, one node per call"
                       if args.launch == "graph" else
                       "one launch per call, enqueued while a delay kernel runs"),
        "achieved_GBps": round(gbps, 1),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "gflops": round(wl.flops / us / 1e3, 1) if wl.flops else None,
        "roofline": roof,
        "algorithmic_bytes_per_step": wl.bytes,
        "kernel_source_hash": kernel_hash(wl.src_files),
    }
    if not args.no_context:
        ctx = context_measurements(torch, binding, wl, min(wl.copies, 256))
        ctx["host_submit_ms_of_timed_steps"] = round(host_s * 1000, 3)
        ctx["delay_before_timed_region_ms"] = (DELAY_NS if args.launch != "eager" else
                                               min(max(DELAY_NS, EAGER_DELAY_NS_PER_STEP * steps),
                                                   100_000_000)) / 1e6
        ctx["kernel_trace_avg_us_per_step"] = trace_for(wl)
        ctx["kernel_trace_median_us_per_step"] = trace_for(wl, "trace_median_ns_per_step")
        line["context"] = ctx
    if not args.no_cpu_baseline and wl.cpu is not None:
        print(f"[bench] timing the CPU oracle (~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
