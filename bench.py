"""Benchmark of the product-key memory lookup on one MI355X.

One step = the whole hot path over one batch: forward (projection, BatchNorm,
per-half scores and top-k, k x k merge + softmax, value gather-sum) and
backward (value gradient into the touched rows, softmax backward, sub-key
gradients, BatchNorm backward, dWq, dx).  Workload: the paper-scale memory
layer (32,768 tokens of width 1600, h=4, dq=512, 1024 x 1024 = 1,048,576 slots,
k=32, bf16 storage, fp32 accumulation, BatchNorm), seeded synthetic inputs.  Beside
it, the fast-weight memorization (FwPKM) of one stream and of a batch of streams.

Prints one JSON line: tokens/s, the roofline of the step's dominant kernel and the
CPU oracle's rate on a bounded sample.  ``--gpus`` above 1 is
not supported: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# dense MFMA peaks of the MI355X by operand type
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}

# HBM bytes per launch measured with two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) at the named
# workload, scaled by the same counters for a plain 1 GiB copy (profiles/*_hbm_counters.md).  Each figure
# holds for the kernel sources whose combined sha256 prefix is given; any change to them voids it (traffic null).
KERNEL_TRAFFIC = {
    ("gather", "paper"): {"bytes": 13551980544, "sources": ["gather.hip", "common.h"], "sources_sha256_16": "1bbc293266b6964f"},
    ("value_grad", "paper"): {"bytes": 29789221888, "sources": ["value_grad.hip", "sparse_common.h", "common.h"], "sources_sha256_16": "c71e5fb32d3e118e"},
    ("value_adam", "paper"): {"bytes": 47242236928, "sources": ["value_grad.hip", "sparse_common.h", "common.h"], "sources_sha256_16": "c71e5fb32d3e118e"},
    ("gather_fp8", "paper"): {"bytes": 7666533376, "sources": ["gather.hip", "common.h"], "sources_sha256_16": "1bbc293266b6964f"},
    ("value_grad", "skewed"): {"bytes": 58854975488, "sources": ["value_grad.hip", "sparse_common.h", "common.h"], "sources_sha256_16": "c71e5fb32d3e118e"},
}


def sources_digest(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "product_key_memory_pkm_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(name, workload):
    ent = KERNEL_TRAFFIC.get((name, workload))
    if ent is None:
        return None
    return ent["bytes"] if sources_digest(ent["sources"]) == ent["sources_sha256_16"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="paper", choices=["paper", "skewed", "small"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=6144, help="tokens in the oracle's timed sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter calibration)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run this many steps and nothing else (for profilers)")
    ap.add_argument("--profile-stages", type=int, default=0,
                    help="run every stage entry point this many times alone, the GPU drained in between (for profilers)")
    ap.add_argument("--profile-diag", action="store_true",
                    help="after one step, five launches of the diagnostics on its selection and nothing else")
    ap.add_argument("--profile-adam", action="store_true",
                    help="after one step, one launch of the Adam-fused value kernel and nothing else (for profilers)")
    ap.add_argument("--profile-fwpkm", type=int, default=0,
                    help="run this many fast-weight memorization chunks and nothing else (for profilers)")
    ap.add_argument("--profile-fwpkm-batch", action="store_true",
                    help="run the batched fast-weight memorization calls once and nothing else (for profilers)")
    ap.add_argument("--profile-fwpkm-one-call", action="store_true",
                    help="memorize the fast-weight stream in one pkm_fwpkm_chunks call and nothing else (for profilers)")
    ap.add_argument("--profile-fwpkm-batch-one-call", action="store_true",
                    help="the batched fast-weight calls as one pkm_fwpkm_chunks call and nothing else (for profilers)")
    ap.add_argument("--no-fwpkm", action="store_true", help="skip the fast-weight memorization legs")
    ap.add_argument("--no-skewed", action="store_true",
                    help="skip the skewed 4,194,304-slot workload reported beside the paper-scale line")
    ap.add_argument("--sweep-keys", action="store_true",
                    help="only time the forward and forward + backward at |C| = |C'| = 256, 512, 1024 and 2048 "
                         "sub-keys, the other sizes those of the paper scale, and print one JSON line")
    return ap.parse_args()


# The fast-weight memory (FwPKM) leg: one token stream memorized in chunks of 512 tokens
# (the chunking of the fast-weight page) by a single-head memory with IDW scores that reads
# k = 8 of the 1024 x 1024 slots per token, over the value table of the main workload.
FWPKM_CHUNK = 512
FWPKM_CHUNKS = 64
FWPKM_TOPK = 8
FWPKM_LR = 0.1
# and a batch of independent streams, each with its own copy of the table, one chunk of each per call
FWPKM_STREAMS = 8
FWPKM_BATCH_CHUNKS = 16


def fwpkm_chunk_bytes(chunk, k, dv, e, touched):
    """Algorithmic HBM bytes of one memorization chunk (heads = 1).

    Read: every lookup's value row, index and weight (gather); y, the target and e for the
    residual; every touched row once more for its step and the token's e once per touched row
    group, with the sorted lookup id, weight and dw (4 bytes each).  Written: y, e, idx and w,
    and every touched row once.  The sub-key scoring reads the chunk's queries (counted) and
    the sub-keys (small, not counted)."""
    L = chunk * k
    gather = L * (dv * e + 8) + chunk * dv * e
    residual = 3 * chunk * dv * e
    update = touched * (2 * dv * e + 4) + chunk * dv * e + L * 12
    select = L * 8
    return gather + residual + update + select


def measured_peaks(torch, timed):
    """What this GPU sustains, measured in this run with libpkm_probe.so: a streaming read of 4 GiB
    (non-temporal 16-byte loads) and back-to-back bf16 16x16x32 MFMAs on register operands.  None if
    the probe library is absent (it is not part of the lookup)."""
    import ctypes
    path = os.path.join(ROOT, "product_key_memory_pkm_amd", "libpkm_probe.so")
    if not os.path.exists(path):
        return None
    P = ctypes.CDLL(path)
    P.pkm_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_uint32, ctypes.c_void_p]
    P.pkm_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                      ctypes.c_void_p]
    P.pkm_probe_stream_read.restype = P.pkm_probe_mfma_bf16.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    best = None
    for blocks in (2048, 4096, 8192):
        def rd():
            assert P.pkm_probe_stream_read(stream, ctypes.c_void_p(buf.data_ptr()), nbytes, blocks, 0xDEADBEEF,
                                           ctypes.c_void_p(out.data_ptr())) == 0
        rd()
        ms = timed(rd, 5)
        bw = nbytes / (ms * 1e-3) / 1e9
        best = bw if best is None or bw > best else best
    del buf
    blocks, iters = 2048, 4000
    tf = {}
    for shape, fl in ((0, 16384), (1, 32768)):
        def mf():
            assert P.pkm_probe_mfma_bf16(stream, blocks, iters, shape, 0xDEADBEEF,
                                         ctypes.c_void_p(out.data_ptr())) == 0
        mf()
        ms = timed(mf, 5)
        tf["16x16x32" if shape == 0 else "32x32x16"] = blocks * 4 * iters * 8 * fl / (ms * 1e-3) / 1e12
    return {"hbm_read_GBs": best, "mfma_bf16_TFLOPs": max(tf.values()), "mfma_bf16_TFLOPs_by_shape": tf,
            "method": "streaming read of 4 GiB (best of 2048/4096/8192 blocks), and 2048 blocks x 4 waves x "
                      "4000 x 8 independent bf16 MFMAs of each shape; 5 event-timed launches each"}


def alg_bytes(cfg, touched):
    """Algorithmic HBM bytes per launch of the forward gather and of the value-gradient kernel.

    gather: every lookup reads its value row, index and weight; y is written once.
    value gradient: every touched row of V is read once, its fp32 dV row read and
    written (accumulating), dY is needed once per token, and per lookup the sorted
    lookup id, its weight and its dw (4 bytes each) plus one row id per touched row.
    value_adam: as the value gradient, with the Adam step in place of dV.
    """
    e = 2 if cfg.dtype == "bf16" else 4
    L = cfg.T * cfg.heads * cfg.topk
    dv = cfg.d_value
    gather = L * (dv * e + 8) + cfg.T * dv * e
    value_grad = touched * (dv * e + 2 * dv * 4 + 4) + cfg.T * dv * e + L * 12
    # the same kernel with the Adam step of the touched rows instead of dV: the
    # value row read and written, both fp32 moment rows read and written
    value_adam = touched * (2 * dv * e + 4 * dv * 4 + 4) + cfg.T * dv * e + L * 12
    # monitoring signals: idx and w read once, entropy written, the per-head
    # slot byte maps cleared and read once by the count pass
    diagnostics = L * 8 + cfg.T * cfg.heads * 4 + cfg.heads * cfg.slots * 2
    # the gather over fp8 value rows (16-byte header + one byte per element)
    gather_fp8 = L * (dv + 16 + 8) + cfg.T * dv * e
    return {"gather": gather, "value_grad": value_grad, "value_adam": value_adam, "diagnostics": diagnostics,
            "gather_fp8": gather_fp8}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import pkm_inputs as pi
    from product_key_memory_pkm_amd import (PKM_WS_FWPKM_CHUNK, ProductKeyMemory, pkm_diagnostics, pkm_fwpkm_chunk,
                                            pkm_fwpkm_chunks,
                                            pkm_quantize_values, pkm_stage_gather, pkm_stage_merge_softmax,
                                            pkm_stage_query, pkm_stage_query_grad, pkm_stage_subkey_grad,
                                            pkm_stage_row_groups, pkm_stage_score_topk, pkm_stage_value_adam,
                                            pkm_stage_value_adam_grouped, pkm_stage_value_adam_rows,
                                            pkm_stage_value_grad_grouped)

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)
        return

    if args.sweep_keys:
        print(json.dumps(sweep_keys(args)), flush=True)
        return

    cfg = pi.CONFIGS[args.workload]
    t0 = time.time()
    inp = pi.make_inputs(cfg, with_dy=True)
    gen_s = time.time() - t0

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, Wq, C, Cp, V, dY = (dev(inp[k]) for k in ("x", "Wq", "C", "Cp", "V", "dY"))
    gamma, beta = dev(inp["gamma"]), dev(inp["beta"])
    m = ProductKeyMemory(cfg.d, cfg.heads, cfg.dq, cfg.n_keys, cfg.n_keys2, cfg.topk, cfg.d_value, dtype=cfg.dtype,
                         bn=cfg.bn, bn_eps=cfg.bn_eps, temperature=cfg.temperature, accumulate_dv=True)
    T = cfg.T
    saved = m.alloc_saved(T)
    y = torch.empty((T, cfg.d_value), dtype=m.storage, device="cuda")
    dV = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
    grads = None

    def step():
        nonlocal grads
        m.forward(x, Wq, gamma, beta, C, Cp, V, saved=saved, y=y)
        grads = m.backward(dY, x, Wq, gamma, C, Cp, V, saved, dV, want_dx=True, out=grads)

    def fwpkm_setup():
        """The fast-weight leg's memory, stream and buffers (allocated outside any timed region)."""
        mf = ProductKeyMemory(cfg.d, 1, cfg.dq, cfg.n_keys, cfg.n_keys2, FWPKM_TOPK, cfg.d_value, dtype=cfg.dtype,
                              bn=False, score="idw")
        n = FWPKM_CHUNK * FWPKM_CHUNKS
        qn, tn = pi.fwpkm_stream(cfg.seed + 100, n, cfg.dq, cfg.d_value, cfg.dtype)
        st = {"m": mf, "q": dev(qn), "target": dev(tn), "C": C[:1].contiguous(), "Cp": Cp[:1].contiguous(),
              "V": V.clone(), "y": torch.empty((n, cfg.d_value), dtype=m.storage, device="cuda"),
              "idx": torch.empty((FWPKM_CHUNK, 1, FWPKM_TOPK), dtype=torch.int32, device="cuda"),
              "w": torch.empty((FWPKM_CHUNK, 1, FWPKM_TOPK), dtype=torch.float32, device="cuda"),
              "ws": mf.workspace(FWPKM_CHUNK, PKM_WS_FWPKM_CHUNK)}
        return st

    def fwpkm_run(st, nchunks):
        c0 = FWPKM_CHUNK
        for c in range(nchunks):
            sl = slice(c * c0, (c + 1) * c0)
            pkm_fwpkm_chunk(st["m"].handle, c0, st["q"][sl], st["C"], st["Cp"], st["V"], st["target"][sl],
                            FWPKM_LR, st["y"][sl], st["idx"], st["w"], st["ws"])

    def fwpkm_batch_setup():
        """A batch of FWPKM_STREAMS streams: per call one chunk of each, stream-major (pkm_fwpkm_chunk)."""
        nb, c0, nc = FWPKM_STREAMS, FWPKM_CHUNK, FWPKM_BATCH_CHUNKS
        mf = ProductKeyMemory(cfg.d, 1, cfg.dq, cfg.n_keys, cfg.n_keys2, FWPKM_TOPK, cfg.d_value, dtype=cfg.dtype,
                              bn=False, score="idw")
        qs, ts = [], []
        for b in range(nb):
            qn, tn = pi.fwpkm_stream(cfg.seed + 200 + b, nc * c0, cfg.dq, cfg.d_value, cfg.dtype)
            qs.append(qn.reshape(nc, c0, -1))
            ts.append(tn.reshape(nc, c0, -1))
        # [chunk call, stream, token, feature]: the call's tokens stream-major
        qa = np.ascontiguousarray(np.stack(qs, axis=1)).reshape(nc, nb * c0, -1)
        ta = np.ascontiguousarray(np.stack(ts, axis=1)).reshape(nc, nb * c0, -1)
        Vb = torch.empty((nb * cfg.slots, cfg.d_value), dtype=m.storage, device="cuda")
        for b in range(nb):
            Vb[b * cfg.slots:(b + 1) * cfg.slots].copy_(V)
        return {"m": mf, "q": dev(qa), "target": dev(ta), "C": C[:1].contiguous(), "Cp": Cp[:1].contiguous(),
                "V": Vb, "y": torch.empty((nc, nb * c0, cfg.d_value), dtype=m.storage, device="cuda"),
                "idx": torch.empty((nb * c0, 1, FWPKM_TOPK), dtype=torch.int32, device="cuda"),
                "w": torch.empty((nb * c0, 1, FWPKM_TOPK), dtype=torch.float32, device="cuda"),
                "ws": mf.workspace(nb * c0, PKM_WS_FWPKM_CHUNK)}

    def fwpkm_batch_run(st, ncalls):
        for c in range(ncalls):
            pkm_fwpkm_chunk(st["m"].handle, FWPKM_STREAMS * FWPKM_CHUNK, st["q"][c], st["C"], st["Cp"], st["V"],
                            st["target"][c], FWPKM_LR, st["y"][c], st["idx"], st["w"], st["ws"],
                            streams=FWPKM_STREAMS)

    if args.profile_fwpkm_batch_one_call:
        st = fwpkm_batch_setup()
        nt_b = FWPKM_BATCH_CHUNKS * FWPKM_STREAMS * FWPKM_CHUNK
        pkm_fwpkm_chunks(st["m"].handle, nt_b, FWPKM_STREAMS * FWPKM_CHUNK, st["q"].view(nt_b, -1), st["C"], st["Cp"],
                         st["V"], st["target"].view(nt_b, -1), FWPKM_LR, st["y"].view(nt_b, -1),
                         torch.empty((nt_b, 1, FWPKM_TOPK), dtype=torch.int32, device="cuda"),
                         torch.empty((nt_b, 1, FWPKM_TOPK), dtype=torch.float32, device="cuda"),
                         st["m"].workspace(nt_b, PKM_WS_FWPKM_CHUNK), streams=FWPKM_STREAMS)
        torch.cuda.synchronize()
        print(json.dumps({"profile_fwpkm_batch_one_call": FWPKM_BATCH_CHUNKS}), flush=True)
        return
    if args.profile_fwpkm_batch:
        st = fwpkm_batch_setup()
        fwpkm_batch_run(st, FWPKM_BATCH_CHUNKS)
        torch.cuda.synchronize()
        print(json.dumps({"profile_fwpkm_batch": FWPKM_BATCH_CHUNKS}), flush=True)
        return
    if args.profile_fwpkm_one_call:
        st = fwpkm_setup()
        n_all = FWPKM_CHUNK * FWPKM_CHUNKS
        pkm_fwpkm_chunks(st["m"].handle, n_all, FWPKM_CHUNK, st["q"], st["C"], st["Cp"], st["V"], st["target"],
                         FWPKM_LR, st["y"], torch.empty((n_all, 1, FWPKM_TOPK), dtype=torch.int32, device="cuda"),
                         torch.empty((n_all, 1, FWPKM_TOPK), dtype=torch.float32, device="cuda"),
                         st["m"].workspace(n_all, PKM_WS_FWPKM_CHUNK))
        torch.cuda.synchronize()
        print(json.dumps({"profile_fwpkm_one_call": FWPKM_CHUNKS}), flush=True)
        return
    if args.profile_fwpkm:
        st = fwpkm_setup()
        fwpkm_run(st, min(args.profile_fwpkm, FWPKM_CHUNKS))
        torch.cuda.synchronize()
        print(json.dumps({"profile_fwpkm": min(args.profile_fwpkm, FWPKM_CHUNKS)}), flush=True)
        return

    # first call allocates the outputs and the workspace outside the timed region
    step()
    torch.cuda.synchronize()
    if args.profile_diag:
        hits_c = torch.empty((cfg.heads, cfg.n_keys), dtype=torch.int32, device="cuda")
        hits_cp = torch.empty((cfg.heads, cfg.n_keys2), dtype=torch.int32, device="cuda")
        used = torch.empty(1 + cfg.heads, dtype=torch.int64, device="cuda")
        ent = torch.empty((T, cfg.heads), dtype=torch.float32, device="cuda")
        ent_sum = torch.empty(1, dtype=torch.float64, device="cuda")
        for _ in range(5):
            pkm_diagnostics(m.handle, T, saved["idx"], saved["w"], hits_c, hits_cp, used, ent, ent_sum,
                            m.workspace(T, True))
        torch.cuda.synchronize()
        print(json.dumps({"profile_diag": 5, "slots_in_use": int(used[0].item())}), flush=True)
        return
    if args.profile_adam:
        # one launch of the Adam-fused value kernel on this step's grouping (for kernel counters)
        ws = m.workspace(T, True)
        touched = torch.empty(T * cfg.heads * cfg.topk, dtype=torch.int32, device="cuda")
        nt = torch.zeros(1, dtype=torch.int64, device="cuda")
        dw = torch.empty(T * cfg.heads * cfg.topk, dtype=torch.float32, device="cuda")
        pkm_stage_row_groups(m.handle, T, saved["idx"], touched, nt, ws)
        adam_m = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
        adam_v = torch.zeros_like(adam_m)
        hp = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "step": 1}
        pkm_stage_value_adam_grouped(m.handle, T, saved["w"], dY, V, adam_m, adam_v, hp, dw, nt, ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile_adam": 1, "touched_rows": int(nt.item())}), flush=True)
        return
    if args.profile_stages:
        # every step of the path alone through its stage entry point, K launches each with the GPU
        # drained in between, so a kernel trace shows each kernel without the backward's second stream
        ws = m.workspace(T, True)
        N = T * cfg.heads * cfg.topk
        touched = torch.empty(N, dtype=torch.int32, device="cuda")
        nt = torch.zeros(1, dtype=torch.int64, device="cuda")
        dw = torch.empty(N, dtype=torch.float32, device="cuda")
        F = cfg.heads * cfg.dq
        dq = torch.empty((T, F), dtype=torch.float32, device="cuda")
        sdC = torch.empty((cfg.heads, cfg.n_keys, cfg.dq // 2), dtype=torch.float32, device="cuda")
        sdCp = torch.empty((cfg.heads, cfg.n_keys2, cfg.dq // 2), dtype=torch.float32, device="cuda")
        sdWq = torch.empty((F, cfg.d), dtype=torch.float32, device="cuda")
        sdg = torch.empty(F, dtype=torch.float32, device="cuda") if cfg.bn else None
        sdb = torch.empty(F, dtype=torch.float32, device="cuda") if cfg.bn else None
        sdx = torch.empty((T, cfg.d), dtype=m.storage, device="cuda")
        sub_idx = torch.empty((T, cfg.heads, 2, cfg.topk), dtype=torch.int32, device="cuda")
        sub_score = torch.empty((T, cfg.heads, 2, cfg.topk), dtype=torch.float32, device="cuda")
        dV = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
        y_s = torch.empty((T, cfg.d_value), dtype=m.storage, device="cuda")
        stages = [
            lambda: pkm_stage_query(m.handle, T, x, Wq, gamma, beta, saved, ws),
            lambda: pkm_stage_score_topk(m.handle, T, saved["q"], C, Cp, sub_idx, sub_score, ws),
            lambda: pkm_stage_merge_softmax(m.handle, T, sub_idx, sub_score, saved["idx"], saved["w"]),
            lambda: pkm_stage_gather(m.handle, T, saved["idx"], saved["w"], V, y_s),
            lambda: pkm_stage_row_groups(m.handle, T, saved["idx"], touched, nt, ws),
            lambda: pkm_stage_value_grad_grouped(m.handle, T, saved["w"], dY, V, dV, dw, nt, ws),
            lambda: pkm_stage_subkey_grad(m.handle, T, saved["idx"], saved["w"], dw, saved["q"], C, Cp, dq, sdC,
                                          sdCp, ws),
            lambda: pkm_stage_query_grad(m.handle, T, dq, x, Wq, gamma, saved, sdWq, sdg, sdb, sdx, ws),
        ]
        for fn in stages:
            for _ in range(args.profile_stages):
                fn()
                torch.cuda.synchronize()
        print(json.dumps({"profile_stages": args.profile_stages}), flush=True)
        return
    if args.profile_steps:
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.time()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.time() - t_wall
    ms = start.elapsed_time(end) / args.steps

    # forward alone
    for _ in range(2):
        m.forward(x, Wq, gamma, beta, C, Cp, V, saved=saved, y=y)
    torch.cuda.synchronize()
    start.record()
    nf = max(3, args.steps)
    for _ in range(nf):
        m.forward(x, Wq, gamma, beta, C, Cp, V, saved=saved, y=y)
    end.record()
    torch.cuda.synchronize()
    ms_fwd = start.elapsed_time(end) / nf

    # The two HBM-bound kernels alone, each timed with events on the stream it runs on:
    # pkm_stage_gather launches exactly the forward's gather kernel, and
    # pkm_stage_value_grad_grouped exactly the backward's value-gradient kernel
    # (on a grouping made beforehand by pkm_stage_row_groups).
    def timed(fn, n):
        fn()  # one untimed launch: a kernel the step does not use is loaded on its first launch
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    gather_ms = timed(lambda: pkm_stage_gather(m.handle, T, saved["idx"], saved["w"], V, y), nf)
    ws = m.workspace(T, True)
    touched = torch.empty(T * cfg.heads * cfg.topk, dtype=torch.int32, device="cuda")
    nt = torch.zeros(1, dtype=torch.int64, device="cuda")
    dw = torch.empty(T * cfg.heads * cfg.topk, dtype=torch.float32, device="cuda")
    pkm_stage_row_groups(m.handle, T, saved["idx"], touched, nt, ws)
    torch.cuda.synchronize()
    vg_ms = timed(lambda: pkm_stage_value_grad_grouped(m.handle, T, saved["w"], dY, V, dV, dw, nt, ws), nf)
    n_touched = int(nt.item())
    # the same kernel with the fused Adam step of the touched value rows (on a copy of V)
    V_opt = V.clone()
    adam_m = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
    adam_v = torch.zeros_like(adam_m)
    hp = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "step": 1}
    va_ms = timed(lambda: pkm_stage_value_adam_grouped(m.handle, T, saved["w"], dY, V_opt, adam_m, adam_v, hp, dw, nt,
                                                       ws), nf)
    # the whole stage (grouping + kernel) with dense moments, and with the moments in a pool of slots handed
    # out on a row's first gradient (grouping, slot hand-out, kernel); the pool holds the touched rows, and
    # after the untimed first call every row has its slot
    touched_a = torch.empty(T * cfg.heads * cfg.topk, dtype=torch.int32, device="cuda")
    va_stage_ms = timed(lambda: pkm_stage_value_adam(m.handle, T, saved["idx"], saved["w"], dY, V_opt, adam_m, adam_v,
                                                     hp, touched_a, nt, dw, ws), nf)
    del adam_m, adam_v
    torch.cuda.empty_cache()
    pool = m.adam_row_state(n_touched)
    var_stage_ms = timed(lambda: pkm_stage_value_adam_rows(m.handle, T, saved["idx"], saved["w"], dY, V_opt, pool, hp,
                                                           touched_a, nt, dw, ws), nf)
    adam_rows = {"stage_ms_dense_moments": va_stage_ms, "stage_ms_row_slots": var_stage_ms,
                 "pool_rows": int(pool["n_used"].item()), "pool_bytes": 2 * n_touched * cfg.d_value * 4,
                 "dense_moment_bytes": 2 * cfg.slots * cfg.d_value * 4}
    del V_opt, pool, touched_a
    torch.cuda.empty_cache()
    # monitoring signals of the step's selection
    hits_c = torch.empty((cfg.heads, cfg.n_keys), dtype=torch.int32, device="cuda")
    hits_cp = torch.empty((cfg.heads, cfg.n_keys2), dtype=torch.int32, device="cuda")
    used = torch.empty(1 + cfg.heads, dtype=torch.int64, device="cuda")
    ent = torch.empty((T, cfg.heads), dtype=torch.float32, device="cuda")
    ent_sum = torch.empty(1, dtype=torch.float64, device="cuda")
    dg_ms = timed(lambda: pkm_diagnostics(m.handle, T, saved["idx"], saved["w"], hits_c, hits_cp, used, ent, ent_sum,
                                          ws), nf)
    diag = {"slots_in_use": int(used[0].item()), "slots_in_use_fraction": int(used[0].item()) / cfg.slots,
            "mean_softmax_entropy": float(ent_sum.item()) / (T * cfg.heads),
            "max_subkey_hits": int(max(hits_c.max().item(), hits_cp.max().item())),
            "mean_subkey_hits": T * cfg.topk / cfg.n_keys}
    # the forward with the value table stored as fp8 rows (a forward format)
    m8 = ProductKeyMemory(cfg.d, cfg.heads, cfg.dq, cfg.n_keys, cfg.n_keys2, cfg.topk, cfg.d_value, dtype=cfg.dtype,
                          bn=cfg.bn, bn_eps=cfg.bn_eps, temperature=cfg.temperature, values="fp8")
    V8 = torch.empty(cfg.slots * ((cfg.d_value + 16 + 127) // 128 * 128), dtype=torch.uint8, device="cuda")
    quant_ms = timed(lambda: pkm_quantize_values(m8.handle, V, V8), 3)
    saved8 = m8.alloc_saved(T)
    y8 = torch.empty_like(y)
    for _ in range(2):
        m8.forward(x, Wq, gamma, beta, C, Cp, V8, saved=saved8, y=y8)
    torch.cuda.synchronize()
    start.record()
    for _ in range(nf):
        m8.forward(x, Wq, gamma, beta, C, Cp, V8, saved=saved8, y=y8)
    end.record()
    torch.cuda.synchronize()
    ms_fwd8 = start.elapsed_time(end) / nf
    g8_ms = timed(lambda: pkm_stage_gather(m8.handle, T, saved8["idx"], saved8["w"], V8, y8), nf)
    y_rel = float(((y8.float() - y.float()).norm() / y.float().norm()).item())
    fp8 = {"fwd_tokens_per_s": T / (ms_fwd8 * 1e-3), "fwd_ms": ms_fwd8, "quantize_ms": quant_ms,
           "table_bytes": V8.numel(), "y_rel_diff_vs_storage_values": y_rel}
    del V8, y8, saved8, m8
    torch.cuda.empty_cache()
    fw = None
    if not args.no_fwpkm:
        # the fast-weight memorization of one stream, chunk after chunk (each chunk reads what the
        # chunks before it wrote); a second pass over the same stream is timed
        st = fwpkm_setup()
        fwpkm_run(st, FWPKM_CHUNKS)
        torch.cuda.synchronize()
        t_host = time.time()
        start.record()
        fwpkm_run(st, FWPKM_CHUNKS)
        end.record()
        host_s = time.time() - t_host
        torch.cuda.synchronize()
        ms_fw = start.elapsed_time(end)
        # the same 64 calls captured once in a HIP graph and replayed (no host enqueue per call)
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            fwpkm_run(st, 1)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fwpkm_run(st, FWPKM_CHUNKS)
        graph.replay()
        torch.cuda.synchronize()
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        ms_fw_graph = start.elapsed_time(end)
        del graph
        touched_c = int(torch.unique(st["idx"]).numel())   # the last chunk's distinct rows
        # the same 64 chunks in one pkm_fwpkm_chunks call: the selection of every chunk first (it does
        # not read V), then each chunk's gather and value step in order; timed on a second pass
        n_all = FWPKM_CHUNK * FWPKM_CHUNKS
        ws_all = st["m"].workspace(n_all, PKM_WS_FWPKM_CHUNK)
        idx_all = torch.empty((n_all, 1, FWPKM_TOPK), dtype=torch.int32, device="cuda")
        w_all = torch.empty((n_all, 1, FWPKM_TOPK), dtype=torch.float32, device="cuda")

        def fwpkm_one_call():
            pkm_fwpkm_chunks(st["m"].handle, n_all, FWPKM_CHUNK, st["q"], st["C"], st["Cp"], st["V"], st["target"],
                             FWPKM_LR, st["y"], idx_all, w_all, ws_all)

        fwpkm_one_call()
        torch.cuda.synchronize()
        start.record()
        fwpkm_one_call()
        end.record()
        torch.cuda.synchronize()
        ms_fw_one = start.elapsed_time(end)
        del ws_all, idx_all, w_all
        e_ = 2 if cfg.dtype == "bf16" else 4
        cb = fwpkm_chunk_bytes(FWPKM_CHUNK, FWPKM_TOPK, cfg.d_value, e_, touched_c)
        ms_chunk = ms_fw / FWPKM_CHUNKS
        fw = {"workload": (f"one stream of {FWPKM_CHUNKS} x {FWPKM_CHUNK} tokens, heads=1, dq={cfg.dq}, "
                           f"|C|=|C'|={cfg.n_keys} ({cfg.slots} slots), k={FWPKM_TOPK}, IDW scores, "
                           f"d_value={cfg.d_value}, {cfg.dtype} storage, lr={FWPKM_LR}"),
              "tokens_per_s": FWPKM_CHUNK * FWPKM_CHUNKS / (ms_fw * 1e-3), "ms_per_chunk": ms_chunk,
              "host_enqueue_ms_per_chunk": host_s * 1e3 / FWPKM_CHUNKS,
              "tokens_per_s_graph_replay": FWPKM_CHUNK * FWPKM_CHUNKS / (ms_fw_graph * 1e-3),
              "ms_per_chunk_graph_replay": ms_fw_graph / FWPKM_CHUNKS,
              "tokens_per_s_one_call": n_all / (ms_fw_one * 1e-3),
              "ms_per_chunk_one_call": ms_fw_one / FWPKM_CHUNKS,
              "touched_rows_last_chunk": touched_c, "alg_bytes_per_chunk": cb,
              "achieved_GBs_whole_chunk": cb / (ms_chunk * 1e-3) / 1e9}
        del st
        torch.cuda.empty_cache()
        # a batch of independent streams: one chunk of each per call
        st = fwpkm_batch_setup()
        fwpkm_batch_run(st, FWPKM_BATCH_CHUNKS)
        torch.cuda.synchronize()
        start.record()
        fwpkm_batch_run(st, FWPKM_BATCH_CHUNKS)
        end.record()
        torch.cuda.synchronize()
        ms_b = start.elapsed_time(end)
        ntok_b = FWPKM_STREAMS * FWPKM_CHUNK * FWPKM_BATCH_CHUNKS
        touched_b = int(torch.unique(st["idx"]).numel())
        cb_b = fwpkm_chunk_bytes(FWPKM_STREAMS * FWPKM_CHUNK, FWPKM_TOPK, cfg.d_value, e_, touched_b)
        ms_call = ms_b / FWPKM_BATCH_CHUNKS
        # the same 16 calls in one pkm_fwpkm_chunks call (the selection of all of them first; each call
        # still groups its own 8 streams' lookups); timed on a second pass
        nt_b = FWPKM_BATCH_CHUNKS * FWPKM_STREAMS * FWPKM_CHUNK
        ws_b = st["m"].workspace(nt_b, PKM_WS_FWPKM_CHUNK)
        idx_b = torch.empty((nt_b, 1, FWPKM_TOPK), dtype=torch.int32, device="cuda")
        w_b = torch.empty((nt_b, 1, FWPKM_TOPK), dtype=torch.float32, device="cuda")

        def fwpkm_batch_one_call():
            pkm_fwpkm_chunks(st["m"].handle, nt_b, FWPKM_STREAMS * FWPKM_CHUNK, st["q"].view(nt_b, -1), st["C"],
                             st["Cp"], st["V"], st["target"].view(nt_b, -1), FWPKM_LR, st["y"].view(nt_b, -1),
                             idx_b, w_b, ws_b, streams=FWPKM_STREAMS)

        fwpkm_batch_one_call()
        torch.cuda.synchronize()
        start.record()
        fwpkm_batch_one_call()
        end.record()
        torch.cuda.synchronize()
        ms_b_one = start.elapsed_time(end)
        del ws_b, idx_b, w_b
        fw["batch"] = {"workload": (f"{FWPKM_STREAMS} streams x {FWPKM_BATCH_CHUNKS} chunks of {FWPKM_CHUNK} tokens, "
                                    f"one chunk of each stream per call, each stream on its own table "
                                    f"({FWPKM_STREAMS} x {cfg.slots} slots); otherwise as above"),
                       "tokens_per_s": ntok_b / (ms_b * 1e-3), "ms_per_call": ms_call,
                       "tokens_per_s_one_call": ntok_b / (ms_b_one * 1e-3),
                       "touched_rows_last_call": touched_b, "alg_bytes_per_call": cb_b,
                       "achieved_GBs_whole_call": cb_b / (ms_call * 1e-3) / 1e9}
        del st
        torch.cuda.empty_cache()
    # the per-half scoring + top-k kernel alone (its MFMA roofline)
    sub_idx = torch.empty((T, cfg.heads, 2, cfg.topk), dtype=torch.int32, device="cuda")
    sub_score = torch.empty((T, cfg.heads, 2, cfg.topk), dtype=torch.float32, device="cuda")
    score_ms = timed(lambda: pkm_stage_score_topk(m.handle, T, saved["q"], C, Cp, sub_idx, sub_score, ws), nf)
    # every step alone, through the stage entry points (each launches exactly the kernels the full calls
    # launch for that step); inside pkm_backward the sub-key gradients overlap the query gradients
    F = cfg.heads * cfg.dq
    dq = torch.empty((T, F), dtype=torch.float32, device="cuda")
    sdC = torch.empty((cfg.heads, cfg.n_keys, cfg.dq // 2), dtype=torch.float32, device="cuda")
    sdCp = torch.empty((cfg.heads, cfg.n_keys2, cfg.dq // 2), dtype=torch.float32, device="cuda")
    sdWq = torch.empty((F, cfg.d), dtype=torch.float32, device="cuda")
    sdg = torch.empty(F, dtype=torch.float32, device="cuda") if cfg.bn else None
    sdb = torch.empty(F, dtype=torch.float32, device="cuda") if cfg.bn else None
    sdx = torch.empty((T, cfg.d), dtype=m.storage, device="cuda")
    stages = {
        "a1_a2_query": timed(lambda: pkm_stage_query(m.handle, T, x, Wq, gamma, beta, saved, ws), nf),
        "a3_a4_score_topk": score_ms,
        "a5_merge_softmax": timed(lambda: pkm_stage_merge_softmax(m.handle, T, sub_idx, sub_score, saved["idx"],
                                                                  saved["w"]), nf),
        "a6_gather": gather_ms,
        "a8_row_grouping": timed(lambda: pkm_stage_row_groups(m.handle, T, saved["idx"], touched, nt, ws), nf),
        "a7_a8_value_grad": vg_ms,
        "a7_a9_subkey_grad": timed(lambda: pkm_stage_subkey_grad(m.handle, T, saved["idx"], saved["w"], dw,
                                                                 saved["q"], C, Cp, dq, sdC, sdCp, ws), nf),
        "a10_query_grad": timed(lambda: pkm_stage_query_grad(m.handle, T, dq, x, Wq, gamma, saved, sdWq, sdg, sdb,
                                                             sdx, ws), nf),
    }
    del dq, sdC, sdCp, sdWq, sdg, sdb, sdx
    score_flops = 2.0 * T * cfg.heads * (cfg.n_keys + cfg.n_keys2) * (cfg.dq // 2)
    score_peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    score_tf = score_flops / (score_ms * 1e-3) / 1e12
    ab = alg_bytes(cfg, n_touched)
    peaks = measured_peaks(torch, timed)
    kern = {
        "gather": {"kernel": "gather_sum (a6)", "ms": gather_ms, "alg": ab["gather"]},
        "value_grad": {"kernel": "value_grad (a7 dw + a8 dV)", "ms": vg_ms, "alg": ab["value_grad"]},
    }
    dom = max(kern, key=lambda n: kern[n]["ms"])
    # not a step of the lookup itself: the optimizer step fused into a8 (reported beside it)
    kern["value_adam"] = {"kernel": "value_grad with the Adam step of the touched value rows (a7 dw + a8 + optimizer)",
                          "ms": va_ms, "alg": ab["value_adam"], "row_slot_state": adam_rows}
    kern["diagnostics"] = {"kernel": "diagnostics (hit counts, slots in use, softmax entropy)", "ms": dg_ms,
                           "alg": ab["diagnostics"]}
    kern["gather_fp8"] = {"kernel": "gather_sum over fp8 value rows (a6, value_format fp8)", "ms": g8_ms,
                          "alg": ab["gather_fp8"]}
    for k_ in kern.values():
        k_["achieved"] = k_["alg"] / (k_["ms"] * 1e-3) / 1e9

    def roof(name):
        k_ = kern[name]
        r = {"kernel": k_["kernel"], "bound": "hbm", "achieved": k_["achieved"], "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": k_["achieved"] / HBM_PEAK_GBS, "traffic": measured_traffic(name, args.workload),
             "alg_bytes_per_launch": k_["alg"], "avg_launch_ms": k_["ms"]}
        if "row_slot_state" in k_:
            r["row_slot_state"] = k_["row_slot_state"]
        if peaks:
            r["frac_of_measured_peak"] = k_["achieved"] / peaks["hbm_read_GBs"]
        return r

    out = {
        "metric": f"PKM lookup tokens/sec (fwd+bwd) at {cfg.n_keys}^2 slots h={cfg.heads} k={cfg.topk}",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": (f"{cfg.name}: T={T}, d={cfg.d}, heads={cfg.heads}, dq={cfg.dq}, "
                                f"|C|=|C'|={cfg.n_keys} ({cfg.slots} slots), k={cfg.topk}, d_value={cfg.d_value}, "
                                f"{cfg.dtype} storage, fp32 accumulation, BatchNorm, dV accumulated in fp32"),
                   "tokens_per_step": T, "step": "forward + backward (all steps a1-a10)"},
        "fwd_tokens_per_s": T / (ms_fwd * 1e-3),
        "fwd_ms": ms_fwd,
        "wall_s_timed_region": wall,
        "roofline": roof(dom),
        "roofline_other": dict({n: roof(n) for n in kern if n != dom},
                               score_topk={"kernel": "score_topk (a3 MFMA scores + a4 per-half top-k)", "bound": "mfma",
                                           "achieved": score_tf, "peak": score_peak, "unit": "TFLOP/s",
                                           "frac": score_tf / score_peak, "traffic": None,
                                           "alg_flops_per_launch": score_flops, "avg_launch_ms": score_ms,
                                           "frac_of_measured_peak": (score_tf / peaks["mfma_bf16_TFLOPs"]
                                                                     if peaks and cfg.dtype == "bf16" else None)}),
        "measured_peaks": peaks,
        "stages_ms": stages,
        "touched_rows": n_touched,
        "diagnostics": diag,
        "fp8_values": fp8,
        "fwpkm": fw,
        "memory_usage": n_touched / cfg.slots,
        "input_generation_s": gen_s,
    }

    if args.workload == "paper" and not args.no_skewed:
        del saved, y, dV, grads
        torch.cuda.empty_cache()
        out["skewed"] = skewed_leg(args, timed)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_tokens)
    print(json.dumps(out), flush=True)


def sweep_keys(args) -> dict:
    """Forward and forward + backward tokens/s of the paper-scale layer (T = 32,768, d = 1600, h = 4, k = 32,
    bf16, BatchNorm) at several codebook sizes: the speed side of the product-key summary's 512^2 -> 1024^2
    slot comparison ("关键结果"), for this layer alone.  Inputs from the same seeded generator per size."""
    import dataclasses
    import numpy as np
    import torch

    import pkm_inputs as pi
    from product_key_memory_pkm_amd import ProductKeyMemory

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    rows = []
    for nk in (256, 512, 1024, 2048):
        c = dataclasses.replace(pi.CONFIGS["paper"], name=f"paper_keys{nk}", n_keys=nk, n_keys2=nk)
        inp = pi.make_inputs(c, with_dy=True)
        x, Wq, C, Cp, V, dY = (dev(inp[k]) for k in ("x", "Wq", "C", "Cp", "V", "dY"))
        gamma, beta = dev(inp["gamma"]), dev(inp["beta"])
        del inp
        m = ProductKeyMemory(c.d, c.heads, c.dq, c.n_keys, c.n_keys2, c.topk, c.d_value, dtype=c.dtype, bn=c.bn,
                             bn_eps=c.bn_eps, temperature=c.temperature, accumulate_dv=True)
        saved = m.alloc_saved(c.T)
        y = torch.empty((c.T, c.d_value), dtype=m.storage, device="cuda")
        dV = torch.zeros((c.slots, c.d_value), dtype=torch.float32, device="cuda")
        grads = None

        def fwd():
            m.forward(x, Wq, gamma, beta, C, Cp, V, saved=saved, y=y)

        def step():
            nonlocal grads
            fwd()
            grads = m.backward(dY, x, Wq, gamma, C, Cp, V, saved, dV, want_dx=True, out=grads)

        res = {"n_keys": nk, "slots": c.slots}
        for name, fn in (("fwd", fwd), ("fwd_bwd", step)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / args.steps
            res[f"{name}_ms"] = ms
            res[f"{name}_tokens_per_s"] = c.T / (ms * 1e-3)
        res["touched_rows"] = int(grads["n_touched"].item())
        res["memory_usage"] = res["touched_rows"] / c.slots
        rows.append(res)
        print(json.dumps(res), file=sys.stderr, flush=True)
        del x, Wq, C, Cp, V, dY, gamma, beta, m, saved, y, dV, grads
        torch.cuda.empty_cache()
    return {"sweep": "codebook size |C| = |C'|", "workload": "paper scale otherwise: T=32768, d=1600, heads=4, "
            "dq=512, k=32, d_value=1600, bf16 storage, BatchNorm, dV accumulated in fp32", "data": "synthetic",
            "steps": args.steps, "warmup": args.warmup, "rows": rows}


def rank_frequency(idx, slots: int) -> dict:
    """Access skew of a selection idx [T, h, k] (device tensor): lookups per touched row, rows ranked by that
    count; the least-squares slope of log10(count) against log10(rank) over 64 log-spaced ranks of the most
    used 1% of touched rows and over all of them (Zipf(s) access has slope -s), and the share of lookups
    that the most used 1% of rows take."""
    import numpy as np
    import torch
    cnt = torch.bincount(idx.reshape(-1).long(), minlength=slots)
    cnt = torch.sort(cnt[cnt > 0], descending=True).values.double().cpu().numpy()
    U = cnt.size

    def slope(n):
        r = np.unique(np.round(np.logspace(0, np.log10(max(n, 2)), 64)).astype(np.int64))
        return float(np.polyfit(np.log10(r), np.log10(cnt[r - 1]), 1)[0])
    top = max(2, U // 100)
    return {"touched_rows": int(U), "max_lookups_per_row": int(cnt[0]), "mean_lookups_per_row": float(cnt.mean()),
            "slope_top_1pct": slope(top), "slope_all": slope(U), "top_1pct_share": float(cnt[:top].sum() / cnt.sum())}


def skewed_leg(args, timed):
    """The large skewed workload (65,536 tokens from a 256-centroid Gaussian mixture with Zipf(1) weights,
    h=8, 2048 x 2048 = 4,194,304 slots, k=32, d=1024, bf16): whole fwd + bwd steps, the forward alone, the
    value-gradient kernel alone, the slots in use and the access skew."""
    import numpy as np
    import torch

    import pkm_inputs as pi
    from product_key_memory_pkm_amd import ProductKeyMemory, pkm_stage_row_groups, pkm_stage_value_grad_grouped
    cfg = pi.CONFIGS["skewed"]
    inp = pi.make_inputs(cfg, with_dy=True)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    x, Wq, C, Cp, V, dY = (dev(inp[k]) for k in ("x", "Wq", "C", "Cp", "V", "dY"))
    gamma, beta = dev(inp["gamma"]), dev(inp["beta"])
    del inp
    m = ProductKeyMemory(cfg.d, cfg.heads, cfg.dq, cfg.n_keys, cfg.n_keys2, cfg.topk, cfg.d_value, dtype=cfg.dtype,
                         bn=cfg.bn, bn_eps=cfg.bn_eps, temperature=cfg.temperature, accumulate_dv=True)
    T = cfg.T
    saved = m.alloc_saved(T)
    y = torch.empty((T, cfg.d_value), dtype=m.storage, device="cuda")
    dV = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
    grads = None

    def step():
        nonlocal grads
        m.forward(x, Wq, gamma, beta, C, Cp, V, saved=saved, y=y)
        grads = m.backward(dY, x, Wq, gamma, C, Cp, V, saved, dV, want_dx=True, out=grads)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    n = max(3, args.steps)
    ms = timed(step, n)
    ms_fwd = timed(lambda: m.forward(x, Wq, gamma, beta, C, Cp, V, saved=saved, y=y), n)
    ws = m.workspace(T, True)
    touched = torch.empty(T * cfg.heads * cfg.topk, dtype=torch.int32, device="cuda")
    nt = torch.zeros(1, dtype=torch.int64, device="cuda")
    dw = torch.empty(T * cfg.heads * cfg.topk, dtype=torch.float32, device="cuda")
    pkm_stage_row_groups(m.handle, T, saved["idx"], touched, nt, ws)
    torch.cuda.synchronize()
    vg_ms = timed(lambda: pkm_stage_value_grad_grouped(m.handle, T, saved["w"], dY, V, dV, dw, nt, ws), n)
    U = int(nt.item())
    ab = alg_bytes(cfg, U)
    skew = rank_frequency(saved["idx"], cfg.slots)
    del x, Wq, C, Cp, V, dY, saved, y, dV, grads, ws, touched, dw, m
    torch.cuda.empty_cache()
    vg_gbs = ab["value_grad"] / (vg_ms * 1e-3) / 1e9
    return {"workload": (f"skewed: T={T}, d={cfg.d}, heads={cfg.heads}, dq={cfg.dq}, |C|=|C'|={cfg.n_keys} "
                         f"({cfg.slots} slots), k={cfg.topk}, d_value={cfg.d_value}, {cfg.dtype} storage, "
                         f"queries from a 256-centroid Gaussian mixture (Zipf(1) weights)"),
            "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms, "fwd_tokens_per_s": T / (ms_fwd * 1e-3),
            "fwd_ms": ms_fwd,
            "value_grad_roofline": {"kernel": "value_grad (a7 dw + a8 dV)", "bound": "hbm", "achieved": vg_gbs,
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": vg_gbs / HBM_PEAK_GBS,
                                    "traffic": measured_traffic("value_grad", "skewed"),
                                    "alg_bytes_per_launch": ab["value_grad"], "avg_launch_ms": vg_ms},
            "memory_usage": U / cfg.slots, "rank_frequency": skew}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, ntok):
    """The fp64 oracle, as it stands, on a bounded sample: the first ``ntok`` tokens as their own batch."""
    import numpy as np

    from oracle import pkm_oracle as O
    import pkm_inputs as pi
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    sub = pi.with_tokens(cfg, ntok)
    sinp = dict(inp)
    sinp["x"] = inp["x"][:ntok]
    sinp["dY"] = inp["dY"][:ntok]
    t0 = time.time()
    fwd = O.forward(sub, sinp)
    t1 = time.time()
    bwd = O.backward(sub, sinp, fwd, sinp["dY"], dv_rows=np.unique(fwd["rows"]))
    t2 = time.time()
    dt = t2 - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"first {ntok} tokens of the benchmark batch as one batch (BatchNorm over the sample), "
                       f"full forward + backward in fp64 numpy, {dt:.1f} s; the matrix products use the BLAS "
                       f"threads counted in cores, the sorts and the per-lookup loops one thread"),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "seconds": dt, "fwd_seconds": t1 - t0, "bwd_seconds": t2 - t1,
            "fwd_tokens_per_s": ntok / (t1 - t0), "bwd_tokens_per_s": ntok / (t2 - t1),
            "parity": sample_parity(sub, sinp, fwd, bwd)}


def sample_parity(sub, sinp, fwd, bwd):
    """The HIP path on the oracle's sample (same inputs, same batch) against the oracle's result.

    Selections are judged by the tests' rule with no slack, against the oracle's exact search run on the
    GPU's own bf16 query (the search input; the query itself equals the oracle's or is one bf16 ulp off):
    invalid selections, and sets differing from that search where the k-th and (k+1)-th full-key scores
    are more than 1e-4 relative apart, must both be 0.  Against the oracle's search on its own query the
    sets are counted too.  y is compared on the tokens whose sets all match, dV on the rows that no
    differing selection touches, the reductions by Frobenius norm ratio.
    """
    import numpy as np
    import torch

    from oracle import pkm_oracle as O
    from product_key_memory_pkm_amd import ProductKeyMemory
    from tests import parity as P

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    m = ProductKeyMemory(sub.d, sub.heads, sub.dq, sub.n_keys, sub.n_keys2, sub.topk, sub.d_value, dtype=sub.dtype,
                         bn=sub.bn, bn_eps=sub.bn_eps, temperature=sub.temperature, accumulate_dv=True)
    x, Wq, C, Cp, V, dY = (dev(sinp[k]) for k in ("x", "Wq", "C", "Cp", "V", "dY"))
    gamma, beta = dev(sinp["gamma"]), dev(sinp["beta"])
    y, saved = m.forward(x, Wq, gamma, beta, C, Cp, V)
    dV = torch.zeros((sub.slots, sub.d_value), dtype=torch.float32, device="cuda")
    g = m.backward(dY, x, Wq, gamma, C, Cp, V, saved, dV, want_dx=True)
    torch.cuda.synchronize()
    k = sub.topk
    G = saved["idx"].cpu().numpy().astype(np.int64)
    R = fwd["rows"].astype(np.int64)
    same = (np.sort(G, axis=-1) == np.sort(R, axis=-1)).all(-1)          # [T, h]
    s = fwd["scores_k1"]
    near = (s[..., k - 1] - s[..., k]) <= P.REL_GAP * np.maximum(np.abs(s[..., k - 1]), np.abs(s[..., k]))
    # the exact search on the GPU's own query
    qo, qg = fwd["q"], P.to_f64(saved["q"])
    Cd, Cpd = O.decode(sinp["C"], sub.dtype), O.decode(sinp["Cp"], sub.dtype)
    sel = P.lookup_chunks(sub, qg, Cd, Cpd)
    valid, exact_g, order_g = P.check_selection(
        G, sel["rows_k1"], sel["scores_k1"], lambda r: P.full_scores(r, sel["s1"], sel["s2"], sub.n_keys2),
        sub.slots, k)
    sg = sel["scores_k1"]
    near_g = (sg[..., k - 1] - sg[..., k]) <= P.REL_GAP * np.maximum(np.abs(sg[..., k - 1]), np.abs(sg[..., k]))
    q_ulp_frac = float((qg != qo).mean())
    q_ok = bool((np.abs(qg - qo) <= P.q_allowed(qg, qo)).all())
    tok_ok = same.all(-1)
    y_err = float(P.row_rel_err(P.to_f64(y)[tok_ok], fwd["y"][tok_ok]).max()) if tok_ok.any() else None
    bad_rows = np.union1d(G[~same].ravel(), R[~same].ravel())
    rows = np.unique(R)                       # the rows the oracle's dV_rows covers, in that order
    keep = ~np.isin(rows, bad_rows)
    dv_g = dV[torch.from_numpy(rows[keep]).cuda()].double().cpu().numpy()
    dv_o = bwd["dV_rows"][keep]
    dv_err = float(P.row_rel_err(dv_g, dv_o).max()) if keep.any() else None

    def fro(name, ref):
        return P.fro_rel_err(g[name].double().cpu().numpy().reshape(ref.shape), ref)

    return {"tolerance": P.TOL[sub.dtype],
            "query_within_one_bf16_ulp": q_ok, "query_elements_one_ulp_off_frac": q_ulp_frac,
            "gpu_query_search": {"invalid_selections": int((~valid).sum()),
                                 "exact_set_frac": float(exact_g.mean()),
                                 "exact_order_frac": float(order_g.mean()),
                                 "near_tie_frac": float(near_g.mean()),
                                 "differing_sets_outside_near_ties": int((~exact_g & ~near_g).sum())},
            "oracle_query_search": {"same_set_frac": float(same.mean()), "near_tie_frac": float(near.mean()),
                                    "differing_sets": int((~same).sum()),
                                    "differing_sets_outside_near_ties": int((~same & ~near).sum())},
            "y_max_row_rel_err": y_err,
            "dV_max_row_rel_err": dv_err,
            "dC_rel_err": fro("dC", bwd["dC"]), "dCp_rel_err": fro("dCp", bwd["dCp"]),
            "dWq_rel_err": fro("dWq", bwd["dWq"])}


if __name__ == "__main__":
    main()
