"""Benchmark of the quantised attention forward on one MI355X.

One step = the whole quantised path over one resident batch: the Q/K/V
quantisation (sage_quantize_qkv: INT8 Q and smoothed K, E4M3 V, in one call; the
pages' qk_quantize and v_quantize stages are also timed as separate calls) and
the fused INT8-QK / FP8-PV attention, on the
block-24 workload B=1, N=37810, H=56, D=128 (Q/K/V strided views of a packed
bf16 [N, 3*56*128] projection buffer, token-major [N, 7168] bf16 output).
Inputs are seeded synthetic stand-ins (N(0,1); K with a per-channel N(0,2)
offset) for the real activations the benchmark artefacts measured.

Prints ONE JSON line.  Besides the contract keys it carries:
  roofline      -- the attention kernel (dominant) against the INT8/FP8 MFMA peak;
                   its duration is measured with HIP events on its own stream.
  stages        -- per-stage ms and the quantisers' achieved HBM bandwidth.
  bf16_path     -- the unquantised BF16-MFMA path on the same inputs (output
                   digest; with the CPU leg, rel-L2 against the exact fp64 result
                   on 64 sampled rows per head, gate 5e-3).
  int8qk_path   -- INT8 Q K^T with the bf16 V unquantised (BF16 P.V) on the same inputs
                   (output digest; with the CPU leg, rel-L2 against its oracle,
                   gate 1e-3).
  rope_path     -- RMSNorm + RoPE of Q and K before quantisation: in place
                   (sage_qk_norm_rope) then sage_quantize_qkv, against the fused
                   sage_quantize_qkv_rope (Q and K never written); both sets of
                   codes and scales digested, byte_exact when they are equal.
  mx_path       -- the attention with its output written as OCP MX blocks (E4M3 and
                   E2M1) by the fused epilogue, against attention + the standalone
                   MX quantiser (sage_mx_quantize) on the bf16 output; both
                   digested, byte_exact when equal.
  cpu_baseline  -- the CPU oracle (quantisers in full + step-by-step quantised
                   attention on sampled rows, extrapolated), on the host cores.
  parity        -- the timed output at those sampled rows against the oracle's
                   result (rounded to bf16): whole-set rel-L2 and the largest
                   row error against the typical row norm (plus each row's
                   error against its own norm, and the worst rows).  The run
                   exits non-zero above any gate or when a byte-exact pair differs.
  output_sha256 -- digest of the timed output's bytes.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOPS (4·N²·d·H/t) + ms/call at N=37810,H=56,d=128; % MFMA peak"
PEAK_I8F8_TFLOPS = 5000.0      # MI355X dense INT8 (POP/s) and FP8 (FLOP/s)
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_INT8QK_TFLOPS = 1.0 / (0.5 / PEAK_I8F8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)   # INT8 QK^T + BF16 P.V
B, N, H, D = 1, 37810, 56, 128
PARITY_GATE = 1e-3        # timed output vs the quantised oracle, whole sampled set
PARITY_ROW_GATE = 3e-2    # ... and each sampled row's error against the typical (RMS) row norm: one wrong
                          # element of a row gives ~0.09; one E4M3 rounding of a large p at a midpoint,
                          # taken the other way in fp32 than in fp64, up to ~0.015



def attn_flops(b=B, n=N, h=H, d=D) -> float:
    return 4.0 * b * n * n * d * h


def quant_bytes(b=B, n=N, h=H, d=D) -> dict:
    """Algorithmic HBM bytes of the quantisers (each input read as the kernels
    must, each output written once)."""
    e = b * n * h * d
    npad = (n + 255) // 256 * 256
    codes = b * h * npad * d
    return {
        # K read for the mean, Q and K read for the codes, int8 codes written
        "qk_quantize": 2 * e + 2 * 2 * e + 2 * codes,
        # V read for the channel maxima, V read again for the codes, fp8 codes written
        "v_quantize": 2 * e + 2 * e + codes,
    }


def rope_bytes(b=B, n=N, h=H, d=D) -> dict:
    """Algorithmic HBM bytes of the RMSNorm + RoPE step: in place, Q and K read
    and written once plus the rotary table (fp32 cos/sin per token and channel
    pair); fused into the quantiser, its bytes are the quantiser's plus the
    table once per pass that reads Q or K (two)."""
    e = b * n * h * d
    table = n * d * 4
    qb = quant_bytes(b, n, h, d)
    return {"norm_rope": 4 * 2 * e + table,
            "qkv_rope": qb["qk_quantize"] + qb["v_quantize"] + 2 * table}


def attn_bytes(b=B, n=N, h=H, d=D) -> int:
    """Algorithmic HBM bytes of one attention launch: Q, K, V codes read once,
    the bf16 output written once (scales are negligible)."""
    npad = (n + 255) // 256 * 256
    return 3 * b * h * npad * d + 2 * b * n * h * d


def kv_restream_bytes(b=B, n=N, h=H, d=D, queries_per_workgroup=128) -> int:
    """On-chip secondary bound of the attention: every workgroup (one block of 128 queries of one head) stages
    its head's whole K and V codes (padded) from L2 into LDS."""
    npad = (n + 255) // 256 * 256
    return -(-n // queries_per_workgroup) * 2 * npad * d * h * b


CSRC = os.path.join(ROOT, "quantized_softmax_attention_amd", "csrc")
# the sources the fused attention kernel is compiled from
ATTN_SOURCES = [os.path.join(CSRC, f) for f in ("sage_attn.hip", "sage_attn_parts.h", "sage_common.h")]


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """Measured HBM traffic of the attention kernel from committed counter runs,
    only if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "attn_i8f8_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != source_hash(ATTN_SOURCES):
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, rows_per_head=512, heads=None):
    """Time the oracle: quantisers at full size (once on one core, then on all
    cores), then the step-by-step quantised attention on `rows_per_head` sampled rows (the last 64 plus
    seeded random rows) of `heads` heads (all by default) against all keys,
    extrapolated to the whole call."""
    import numpy as np

    import oracle
    from quantized_softmax_attention_amd import inputs
    from tests.helpers import oracle_view

    q, k, v = (oracle_view(t) for t in (case.q, case.k, case.v))
    cores = oracle.num_threads()

    def quantise():
        t0 = time.perf_counter()
        km = oracle.kmean(k)
        res = oracle.quant_q(q, 32), oracle.quant_k(k, km, 64), oracle.quant_v(v)
        return time.perf_counter() - t0, res

    oracle.set_num_threads(1)
    t_quant_1, _ = quantise()
    oracle.set_num_threads(cores)
    t_quant, ((qc, qs), (kc, ks), (vc, vs)) = quantise()
    heads = case.H if heads is None else heads
    rows = inputs.sample_rows(case.B, case.H, case.N, count=rows_per_head, tail=64)[:, :heads]
    sub = lambda a: np.ascontiguousarray(a[:, :heads])
    t0 = time.perf_counter()
    meth = oracle.attn_method(sub(qc), sub(qs), sub(kc), sub(ks), sub(vc), sub(vs), 1.0 / math.sqrt(D), rows)
    t_attn = time.perf_counter() - t0
    scale = (case.N * case.H) / (rows_per_head * heads)
    t_call = t_quant + t_attn * scale
    extras = {"rows": rows, "method": meth, "codes": (qc, qs, kc, ks), "heads": heads}
    return extras, {
        "value": attn_flops(case.B, case.N, case.H, case.D) / t_call / 1e12,
        "unit": "TFLOP/s",
        "ms_per_call_extrapolated": t_call * 1e3,
        "cores": cores,
        "kind": "oracle",
        "quantisers_s_all_cores": t_quant,
        "quantisers_s_one_core": t_quant_1,
        "host": {"nproc": os.cpu_count(), "cpu_model": cpu_model()},
        "sample": ("quantisers at full size (%.2f s measured) + step-by-step quantised attention on %d sampled "
                   "rows x %d heads against all %d keys (%.2f s measured), attention time extrapolated x%.1f "
                   "to %d rows x %d heads" % (t_quant, rows_per_head, heads, case.N, t_attn, scale, case.N,
                                              case.H)),
    }


def tensor_sha256(*ts) -> str:
    """sha256 of the raw bytes of the given tensors, in order."""
    import torch  # noqa: F401  (the tensors' own module; imported where the GPU work is)

    h = hashlib.sha256()
    for t in ts:
        h.update(t.detach().contiguous().view(-1).view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def out_rows(out, rows):
    """A token-major bf16 output [B, N, H*D] (on the GPU) at sampled rows [B, H', R] -> fp64 [B, H', R, D]."""
    import numpy as np
    import torch

    Bq, Hq, R = rows.shape
    o = out.view(out.shape[0], out.shape[1], -1, D)[:, :, :Hq]            # [B, N, H', D]
    idx = torch.from_numpy(np.ascontiguousarray(rows.transpose(0, 2, 1))).long().to(out.device)   # [B, R, H']
    got = torch.gather(o, 1, idx[..., None].expand(Bq, R, Hq, D)).float().cpu().numpy()
    return got.transpose(0, 2, 1, 3).astype(np.float64)                     # [B, H', R, D]


def row_errors(got, ref):
    """Whole-set rel-L2 and per-row errors of got against ref ([..., D] fp64): each row's L2 error over the
    RMS row norm of ref (the per-row bound) and over its own norm."""
    import numpy as np

    err = np.sqrt(((got - ref) ** 2).sum(-1))
    nrm = np.sqrt((ref ** 2).sum(-1))
    typical = float(np.sqrt((nrm ** 2).mean()))
    return {"rel_l2": float(np.sqrt((err ** 2).sum() / (nrm ** 2).sum())),
            "max_row_err_vs_typical_row": float(err.max() / typical),
            "max_row_rel_l2": float((err / np.maximum(nrm, 1e-300)).max())}


def parity_vs_method(out, rows, meth):
    """The timed bf16 output [B, N, H*D] (token-major, on the GPU) at the oracle's sampled rows [B, H', R]
    against the step-by-step quantised oracle's result there [B, H', R, D], rounded to bf16 as the kernel
    stores it: whole-set rel-L2 and the largest per-row rel-L2."""
    import numpy as np
    import torch

    Bq, Hq, R = rows.shape
    got = out_rows(out, rows)
    ref = torch.from_numpy(meth).float().to(torch.bfloat16).double().numpy()
    err = np.sqrt(((got - ref) ** 2).sum(-1))
    nrm = np.sqrt((ref ** 2).sum(-1))
    typical = float(np.sqrt((nrm ** 2).mean()))          # RMS row norm
    own = err / np.maximum(nrm, 1e-300)
    worst = np.argsort(own.ravel())[::-1][:5]
    return {"rel_l2_vs_method": float(np.sqrt((err ** 2).sum() / (nrm ** 2).sum())),
            "max_row_err_vs_typical_row": float(err.max() / typical),
            "max_row_rel_l2": float(own.max()),
            "worst_rows": [{"b": int(i // (Hq * R)), "h": int(i // R % Hq), "row": int(rows.ravel()[i]),
                            "rel_l2": float(own.ravel()[i]), "norm_vs_typical": float(nrm.ravel()[i] / typical)}
                           for i in worst],
            "rows": int(Bq * Hq * R), "reference": "step-by-step quantised oracle, rounded to bf16",
            "gate": {"rel_l2_vs_method": PARITY_GATE, "max_row_err_vs_typical_row": PARITY_ROW_GATE}}


SIDE_GATES = {"bf16_path": 5e-3, "int8qk_path": 1e-3}   # rel-L2, as the GPU tests; rows: PARITY_ROW_GATE


def side_parity(case, codes, rows, got16, gotq):
    """The bf16 path's output at the sampled rows against the exact fp64 result, and the INT8-QK / bf16-PV
    path's against the step-by-step oracle of the same precision split rounded to bf16 (the GPU tests'
    references and gates)."""
    import torch

    import oracle
    from tests.helpers import oracle_view

    q, k, v = (oracle_view(t) for t in (case.q, case.k, case.v))
    qc, qs, kc, ks = codes
    sm = 1.0 / math.sqrt(D)
    exact = oracle.attn_exact(q, k, v, sm, rows)
    meth = oracle.attn_int8qk(qc, qs, kc, ks, v, sm, rows)
    meth16 = torch.from_numpy(meth).float().to(torch.bfloat16).double().numpy()
    res = {"bf16_path": {**row_errors(got16, exact), "reference": "exact fp64 attention"},
           "int8qk_path": {**row_errors(gotq, meth16), "reference": "step-by-step INT8-QK / bf16-PV oracle, bf16"}}
    for name, r in res.items():
        r["rows"] = int(rows.size)
        r["gate"] = {"rel_l2": SIDE_GATES[name], "max_row_err_vs_typical_row": PARITY_ROW_GATE}
        r["ok"] = r["rel_l2"] <= SIDE_GATES[name] and r["max_row_err_vs_typical_row"] <= PARITY_ROW_GATE
    return res


def rescale_fraction(codes, N, H, waves_per_head=4, head_step=7):
    """Share of the attention kernel's tiles (after the first) in which some row maximum of a 32-query wave
    moves, so the wave rescales its 64 output accumulators: taken on the workload's own INT8 codes for a
    sample of waves (waves_per_head evenly spaced 32-query blocks of every head_step-th head), with the
    kernel's fp32 scale products."""
    import numpy as np

    qc, qs, kc, ks = codes
    cb = np.float32(1.0 / math.sqrt(D)) * np.float32(1.4426950408889634)
    T = -(-N // 64)
    fired = total = 0
    for h in range(0, H, head_step):
        K = kc[0, h, :N].astype(np.float64)
        for w in range(waves_per_head):
            q0 = (w * (N // waves_per_head)) // 32 * 32
            Q = qc[0, h, q0:q0 + 32].astype(np.float64)
            S = Q @ K.T                                              # exact integer scores [32, N]
            pad = T * 64 - N
            S = np.concatenate([S, np.full((S.shape[0], pad), -np.inf)], axis=1).reshape(S.shape[0], T, 64)
            amax = S.max(axis=2).astype(np.float32)                  # [32, T]
            cq = np.float32(qs[0, h, q0 // 32]) * cb
            c2 = (cq * ks[0, h, :T].astype(np.float32)).astype(np.float32)
            m = np.full(Q.shape[0], -np.inf, np.float32)
            for t in range(T):
                mn = np.maximum(m, c2[t] * amax[:, t])
                if t > 0:
                    fired += bool((mn != m).any())
                    total += 1
                m = mn
    return fired / max(total, 1)


def valu_floor(rescale_frac):
    """Issue floor of the attention's per-tile instruction stream at two waves per SIMD, from the committed
    tile-replay measurement (profiles/valu_rates.json): SIMD cycles per wave-tile."""
    path = os.path.join(ROOT, "profiles", "valu_rates.json")
    if not os.path.exists(path):
        return None
    rep = json.load(open(path))["rates"]["tile_replay"]
    t0, t64 = rep["rescale_0"]["2"]["cyc_per_tile"], rep["rescale_64"]["2"]["cyc_per_tile"]
    return t0 + rescale_frac * (t64 - t0)


def stats_ms(xs):
    xs = sorted(xs)
    pick = lambda p: xs[min(len(xs) - 1, int(round(p * (len(xs) - 1))))]
    return {"mean": statistics.fmean(xs), "p50": pick(0.5), "p90": pick(0.9), "p95": pick(0.95), "p99": pick(0.99),
            "min": xs[0], "max": xs[-1], "count": len(xs)}


class Sensors:
    """Graphics clock and hotspot temperature of the GPU torch uses, read through
    amdsmi (None where unavailable).  Matched to the device by PCI bus."""

    def __init__(self, torch):
        self.h, self.note = None, None
        try:
            import amdsmi
            self.smi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            prop = torch.cuda.get_device_properties(0)
            bus = getattr(prop, "pci_bus_id", None)
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "dddd:bb:dd.f"
                if bus is not None and int(bdf.split(":")[1], 16) == bus:
                    self.h = h
            if self.h is None and len(handles) == 1:
                self.h = handles[0]
            if self.h is None:
                self.note = "no amdsmi handle matched the device"
        except Exception as e:          # sensors are context, never a failure
            self.note = "amdsmi unavailable: %s" % type(e).__name__

    def close(self):
        if self.h is not None:
            try:
                self.smi.amdsmi_shut_down()
            except Exception:
                pass
            self.h = None

    def sample(self, stop, period, out):
        """Append (host time, reading) every `period` seconds until stop is set."""
        while not stop.is_set():
            out.append((time.perf_counter(), self.read()))
            stop.wait(period)

    def read(self):
        if self.h is None:
            return None
        out = {}
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and 0 < c < 10000]
            if clks:
                out["gfxclk_mhz"] = statistics.fmean(clks)
            elif isinstance(m.get("current_gfxclk"), int):
                out["gfxclk_mhz"] = m["current_gfxclk"]
            t = m.get("temperature_hotspot")
            if isinstance(t, int):
                out["hotspot_c"] = t
            p = m.get("current_socket_power")
            if isinstance(p, int):
                out["socket_power_w"] = p
        except Exception as e:
            out["error"] = type(e).__name__
        return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--bf16-calls", type=int, default=5,
                    help="timed calls of each comparison path (bf16, INT8-QK/bf16-PV)")
    ap.add_argument("--rope-calls", type=int, default=20,
                    help="timed rounds of the RMSNorm + RoPE comparison (about 2.5 ms each)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch one plain 1 GiB device copy (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the heads would shard across GPUs "
              "with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_softmax_attention_amd import inputs, sage

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sage.lib()                       # fail loudly if the HIP library is missing

    t0 = time.perf_counter()
    case = inputs.config("block24")
    gen_s = time.perf_counter() - t0
    g = case.to(dev)
    buf = sage.Buffers(B, N, H, device=dev)
    out = sage.token_major_out(B, N, H, device=dev)
    sm = 1.0 / math.sqrt(D)
    stream = torch.cuda.Stream(device=dev)    # default priority

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        with torch.cuda.stream(stream):
            bcopy.copy_(a)
        stream.synchronize()
        del a, bcopy

    def step(evs=None):
        # quantise Q, K (with smoothing) and V in the single three-pass call, then attend
        if evs is not None:
            evs[0].record(stream)
        sage.sage_quantize_qkv(g.q, g.k, g.v, buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.k_mean,
                               buf.v_codes, buf.v_scale, buf.ws_qkv, stream)
        if evs is not None:
            evs[1].record(stream)
        sage.sage_attn_fwd(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.v_codes, buf.v_scale, out, sm,
                           stream)
        if evs is not None:
            evs[2].record(stream)

    for _ in range(args.warmup):
        step()
    stream.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    out_sha = hashlib.sha256(out.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
    qkv_ms = [e[0].elapsed_time(e[1]) for e in evs]
    at_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    ms_per_step = wall * 1e3 / args.steps
    flops = attn_flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_mean = statistics.fmean(at_ms)
    achieved = flops / (attn_mean * 1e-3) / 1e12
    qb = quant_bytes()

    # the attention alone: 5 rounds x 10 launches; a host thread reads the graphics
    # clock, hotspot temperature and socket power every 50 ms meanwhile (the
    # driver's metrics table refreshes more slowly, so a reading can be stale)
    import threading

    sensors = Sensors(torch)
    samples, stop = [], threading.Event()
    sampler = threading.Thread(target=sensors.sample, args=(stop, 0.05, samples), daemon=True)
    sampler.start()
    for _ in range(40):            # about 1 s of load first, so the metrics table shows it
        sage.sage_attn_fwd(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.v_codes, buf.v_scale, out, sm,
                           stream)
    stream.synchronize()
    rounds, all_round_ms = [], []
    for _ in range(5):
        t_begin = time.perf_counter()
        er = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
        for e in er:
            e[0].record(stream)
            sage.sage_attn_fwd(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.v_codes, buf.v_scale, out, sm,
                               stream)
            e[1].record(stream)
        stream.synchronize()
        t_end = time.perf_counter()
        ms = [e[0].elapsed_time(e[1]) for e in er]
        all_round_ms += ms
        inside = [r for t, r in samples if t_begin <= t <= t_end and r and "gfxclk_mhz" in r]
        rounds.append({"ms": stats_ms(ms),
                       "gfxclk_mhz": statistics.fmean(r["gfxclk_mhz"] for r in inside) if inside else None,
                       "hotspot_c_max": max((r.get("hotspot_c", -1) for r in inside), default=None),
                       "socket_power_w_max": max((r.get("socket_power_w", -1) for r in inside), default=None),
                       "samples": len(inside)})
    stop.set()
    sampler.join(timeout=2.0)
    sensors.close()
    # readings under full load only: socket power within 80 % of the highest seen
    # (a stale reading from before the load shows far less power)
    loaded = [r for t, r in samples if r and "gfxclk_mhz" in r and "socket_power_w" in r]
    pmax = max((r["socket_power_w"] for r in loaded), default=0)
    clk = [r["gfxclk_mhz"] for r in loaded if r["socket_power_w"] >= 0.8 * pmax]
    sclk = statistics.fmean(clk) if clk else None

    # practical HBM ceiling for the quantisers: a plain 1 GiB device-to-device copy
    ca = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cb = torch.empty_like(ca)
    ec = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    with torch.cuda.stream(stream):
        cb.copy_(ca)
        for e in ec:
            e[0].record(stream)
            cb.copy_(ca)
            e[1].record(stream)
    stream.synchronize()
    copy_ms = statistics.median(e[0].elapsed_time(e[1]) for e in ec)
    del ca, cb

    # the pages' two quantisation stages as separate calls (same outputs)
    eqk = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in eqk:
        e[0].record(stream)
        sage.sage_quantize_qk(g.q, g.k, buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.k_mean,
                              buf.ws_qk, stream)
        e[1].record(stream)
        sage.sage_quantize_v(g.v, buf.v_codes, buf.v_scale, buf.ws_v, stream)
        e[2].record(stream)
    stream.synchronize()
    qk_ms = [e[0].elapsed_time(e[1]) for e in eqk]
    v_ms = [e[1].elapsed_time(e[2]) for e in eqk]

    # the bf16 comparison path on the same resident inputs
    out16 = sage.token_major_out(B, N, H, device=dev)
    e16 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.bf16_calls)]
    sage.sage_attn_fwd_bf16(g.q, g.k, g.v, out16, sm, stream)
    for e in e16:
        e[0].record(stream)
        sage.sage_attn_fwd_bf16(g.q, g.k, g.v, out16, sm, stream)
        e[1].record(stream)
    stream.synchronize()
    bf16_ms = [e[0].elapsed_time(e[1]) for e in e16]
    side_rows = inputs.sample_rows(B, H, N, count=64, tail=16)        # rows checked against the oracle
    bf16_sha, got16 = tensor_sha256(out16), out_rows(out16, side_rows)

    # INT8 Q K^T with the bf16 V unquantised (codes of the last step's quantise_qk)
    eq = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.bf16_calls)]
    sage.sage_attn_fwd_int8qk(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, g.v, out16, sm, stream)
    for e in eq:
        e[0].record(stream)
        sage.sage_attn_fwd_int8qk(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, g.v, out16, sm, stream)
        e[1].record(stream)
    stream.synchronize()
    int8qk_ms = [e[0].elapsed_time(e[1]) for e in eq]
    int8qk_sha, gotq = tensor_sha256(out16), out_rows(out16, side_rows)
    del out16

    # RMSNorm + RoPE of Q and K: in place then quantise, vs fused into the quantiser
    nr = inputs.norm_rope_params(N).to(dev)
    pk = g.packed.clone()                 # the in-place transform works on a copy
    HD = H * D
    pq, pk_k = (pk[:, :, i * HD:(i + 1) * HD].unflatten(2, (H, D)) for i in range(2))
    rbuf = sage.Buffers(B, N, H, device=dev)              # fused
    ubuf = sage.Buffers(B, N, H, device=dev)              # in place, then sage_quantize_qkv
    er = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.rope_calls)]
    sage.quantize_qkv_rope(g.q, g.k, g.v, nr, rbuf, stream)
    for e in er:
        # each in-place transform starts from the workload's own Q and K (transforming the same buffer again
        # and again would multiply channel d by gamma_d per call and drift far from the workload)
        with torch.cuda.stream(stream):
            pk.copy_(g.packed)
        e[0].record(stream)
        sage.sage_qk_norm_rope(pq, pk_k, nr.gamma_q, nr.gamma_k, nr.rope, nr.eps, stream)
        e[1].record(stream)
        sage.quantize_qkv(pq, pk_k, g.v, ubuf, stream)
        e[2].record(stream)
        sage.quantize_qkv_rope(g.q, g.k, g.v, nr, rbuf, stream)
        e[3].record(stream)
    stream.synchronize()
    codes_of = lambda bb: (bb.q_codes, bb.q_scale, bb.k_codes, bb.k_scale, bb.k_mean, bb.v_codes, bb.v_scale)
    rope_sha, unf_sha = tensor_sha256(*codes_of(rbuf)), tensor_sha256(*codes_of(ubuf))
    nr_ms = [e[0].elapsed_time(e[1]) for e in er]
    unf_ms = [e[0].elapsed_time(e[2]) for e in er]
    fused_ms = [e[2].elapsed_time(e[3]) for e in er]
    rb = rope_bytes()
    rope = {"norm_rope_ms": stats_ms(nr_ms),
            "norm_rope_GBps": rb["norm_rope"] / (statistics.fmean(nr_ms) * 1e-3) / 1e9,
            "unfused_norm_rope_plus_qkv_ms": stats_ms(unf_ms),
            "qkv_rope_fused_ms": stats_ms(fused_ms),
            "qkv_rope_fused_GBps": rb["qkv_rope"] / (statistics.fmean(fused_ms) * 1e-3) / 1e9,
            "codes_sha256": rope_sha, "unfused_codes_sha256": unf_sha, "byte_exact": rope_sha == unf_sha,
            "pages_context": {"gb10_block24_rms_rope_p50_ms": 12.535, "note": "NVIDIA GB10, whole rms_rope component"}}
    del pk, rbuf, ubuf

    # MX output: fused epilogue vs the standalone quantiser over the bf16 output
    mx = {}
    for fmt, name in ((sage.MX_E4M3, "e4m3"), (sage.MX_E2M1, "e2m1")):
        codes, scales = sage.mx_out(B, N, H, fmt, device=dev)       # fused epilogue
        codes_s, scales_s = sage.mx_out(B, N, H, fmt, device=dev)   # standalone quantiser over `out`
        ef = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.bf16_calls)]
        sage.sage_attn_fwd_mx(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.v_codes, buf.v_scale, fmt,
                              codes, scales, sm, stream)
        for e in ef:
            e[0].record(stream)
            sage.sage_attn_fwd_mx(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.v_codes, buf.v_scale, fmt,
                                  codes, scales, sm, stream)
            e[1].record(stream)
            sage.sage_mx_quantize(out, fmt, codes_s, scales_s, stream)
            e[2].record(stream)
        stream.synchronize()
        fused = [e[0].elapsed_time(e[1]) for e in ef]
        alone = [e[1].elapsed_time(e[2]) for e in ef]
        mx_bytes = B * N * H * D * 2 + codes.numel() + scales.numel()
        mx[name] = {"attn_fwd_mx_ms": stats_ms(fused),
                    "tflops": flops / (statistics.fmean(fused) * 1e-3) / 1e12,
                    "mx_quantize_ms": stats_ms(alone),
                    "mx_quantize_GBps": mx_bytes / (statistics.fmean(alone) * 1e-3) / 1e9,
                    "unfused_ms": attn_mean + statistics.fmean(alone)}
        mx[name]["output_sha256"] = tensor_sha256(codes, scales)
        mx[name]["unfused_sha256"] = tensor_sha256(codes_s, scales_s)
        mx[name]["byte_exact"] = mx[name]["output_sha256"] == mx[name]["unfused_sha256"]
        del codes, scales, codes_s, scales_s

    # one GPU's share of an 8-way head split: 7 heads of the same buffer (strided
    # views of their columns), writing their slice of the token-major output
    hs = slice(0, H // 8)
    sbuf = sage.Buffers(B, N, H // 8, device=dev)
    es = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.bf16_calls)]
    sage.forward(g.q[:, :, hs], g.k[:, :, hs], g.v[:, :, hs], out[:, :, hs], sbuf, sm, stream)
    for e in es:
        e[0].record(stream)
        sage.quantize_qkv(g.q[:, :, hs], g.k[:, :, hs], g.v[:, :, hs], sbuf, stream)
        e[1].record(stream)
        sage.sage_attn_fwd(sbuf.q_codes, sbuf.q_scale, sbuf.k_codes, sbuf.k_scale, sbuf.v_codes, sbuf.v_scale,
                           out[:, :, hs], sm, stream)
        e[2].record(stream)
    stream.synchronize()
    s_q = [e[0].elapsed_time(e[1]) for e in es]
    s_a = [e[1].elapsed_time(e[2]) for e in es]
    f7 = attn_flops(h=H // 8)
    n_wg = -(-N // 128) * (H // 8) * B
    shard = {"heads": H // 8, "qkv_quantize_ms": stats_ms(s_q), "attn_fwd_ms": stats_ms(s_a),
             "attn_tflops": f7 / (statistics.fmean(s_a) * 1e-3) / 1e12,
             "attn_workgroups": n_wg, "workgroup_rounds": n_wg / (2 * 256),
             "note": "per-GPU share of an 8-way head split, measured on one GPU; no multi-GPU run"}
    del sbuf

    # the two-sequence stress workload: B=2, x10 outlier channels in Q and K,
    # Student-t V (twice the block-24 work per call)
    t0 = time.perf_counter()
    sc = inputs.config("stress")
    st_gen = time.perf_counter() - t0
    sgc = sc.to(dev)
    del sc
    tbuf = sage.Buffers(2, N, H, device=dev)
    tout = sage.token_major_out(2, N, H, device=dev)
    et = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.bf16_calls)]
    sage.forward(sgc.q, sgc.k, sgc.v, tout, tbuf, sm, stream)
    for e in et:
        e[0].record(stream)
        sage.quantize_qkv(sgc.q, sgc.k, sgc.v, tbuf, stream)
        e[1].record(stream)
        sage.sage_attn_fwd(tbuf.q_codes, tbuf.q_scale, tbuf.k_codes, tbuf.k_scale, tbuf.v_codes, tbuf.v_scale,
                           tout, sm, stream)
        e[2].record(stream)
    stream.synchronize()
    t_q = [e[0].elapsed_time(e[1]) for e in et]
    t_a = [e[1].elapsed_time(e[2]) for e in et]
    f2, qb2 = attn_flops(b=2), quant_bytes(b=2)
    stress = {"B": 2, "qkv_quantize_ms": stats_ms(t_q),
              "qkv_quantize_GBps": (qb2["qk_quantize"] + qb2["v_quantize"]) / (statistics.fmean(t_q) * 1e-3) / 1e9,
              "attn_fwd_ms": stats_ms(t_a), "attn_tflops": f2 / (statistics.fmean(t_a) * 1e-3) / 1e12,
              "step_tflops": f2 / ((statistics.fmean(t_q) + statistics.fmean(t_a)) * 1e-3) / 1e12,
              "input_generation_s": st_gen}
    del sgc, tbuf, tout

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp8e4m3 (fp32 softmax/accumulate)",
        "data": "synthetic (seeded N(0,1) Q/K/V, K + per-channel N(0,2) offset; stand-in for block-24 activations)",
        "config": {"workload": "block24 quantised forward: B=1, N=37810, H=56, D=128, Q/K/V strided NHD views of "
                               "a packed bf16 [37810, 21504] QKV buffer, token-major bf16 [37810, 7168] output",
                   "B": B, "N": N, "H": H, "D": D, "layout": "strided_nhd", "non_causal": True},
        "roofline": {"bound": "mfma", "kernel": "attn_i8f8_kernel", "achieved": achieved,
                     "peak": PEAK_I8F8_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_I8F8_TFLOPS,
                     "traffic": load_traffic(), "algorithmic_bytes": attn_bytes(),
                     "flops_per_launch": flops, "ms_per_launch": attn_mean,
                     "sclk_mhz_measured": sclk,
                     "peak_at_measured_sclk": None if sclk is None else 256 * 8192 * sclk * 1e6 / 1e12,
                     "frac_at_measured_sclk": None if sclk is None else achieved / (256 * 8192 * sclk * 1e6 / 1e12),
                     "peak_note": "5000 = published dense INT8/FP8 figure; 256 CU x 8192 ops/clk x 2.4 GHz = 5033",
                     # on-chip: the K/V codes every workgroup stages from L2 into LDS, and that rate
                     "kv_restream_bytes_per_launch": kv_restream_bytes(),
                     "kv_restream_GBps": kv_restream_bytes() / (attn_mean * 1e-3) / 1e9},
        "attn_rounds": {"all": stats_ms(all_round_ms), "rounds": rounds, "sensor_note": sensors.note},
        "stages": {
            "qkv_quantize_ms": stats_ms(qkv_ms), "attn_fwd_ms": stats_ms(at_ms), "step_ms_events": stats_ms(step_ms),
            "qkv_quantize_GBps": (qb["qk_quantize"] + qb["v_quantize"]) / (statistics.fmean(qkv_ms) * 1e-3) / 1e9,
            "qk_quantize_ms": stats_ms(qk_ms), "v_quantize_ms": stats_ms(v_ms),
            # the pages' pipeline: the two quantiser calls then the attention (means of the separate timings)
            "pipeline_qk_v_attn_ms": statistics.fmean(qk_ms) + statistics.fmean(v_ms) + attn_mean,
            "qk_quantize_GBps": qb["qk_quantize"] / (statistics.fmean(qk_ms) * 1e-3) / 1e9,
            "v_quantize_GBps": qb["v_quantize"] / (statistics.fmean(v_ms) * 1e-3) / 1e9,
            "hbm_peak_GBps": PEAK_HBM_GBS,
            "copy_1GiB_GBps": 2 * (1 << 30) / (copy_ms * 1e-3) / 1e9,   # read + write of a plain device copy
            "attn_pct_of_i8f8_peak": 100.0 * achieved / PEAK_I8F8_TFLOPS,
            "step_pct_of_i8f8_peak": 100.0 * value / PEAK_I8F8_TFLOPS,
        },
        "bf16_path": {"ms_per_call": stats_ms(bf16_ms), "output_sha256": bf16_sha,
                      "tflops": flops / (statistics.fmean(bf16_ms) * 1e-3) / 1e12,
                      "frac_of_bf16_peak": flops / (statistics.fmean(bf16_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "int8qk_path": {"ms_per_call": stats_ms(int8qk_ms), "output_sha256": int8qk_sha,
                        "tflops": flops / (statistics.fmean(int8qk_ms) * 1e-3) / 1e12,
                        "frac_of_peak": flops / (statistics.fmean(int8qk_ms) * 1e-3) / 1e12 / PEAK_INT8QK_TFLOPS,
                        "peak_note": "half the ops at the INT8 peak, half at the BF16 peak: 1/(0.5/5000 + 0.5/2500)"},
        "rope_path": rope,
        "mx_path": mx,
        "head_shard": shard,
        "stress_path": stress,
        "pages_context": {"gb10_attention_forward_p50_ms": 238.995, "gb10_total_excluding_layout_ms": 258.613,
                          "note": "NVIDIA GB10 on real activations; context only"},
        "input_generation_s": gen_s,
    }
    line["output_sha256"] = out_sha
    # the byte-exact pairs: fused vs unfused RoPE quantiser, fused vs standalone MX quantiser
    ok = rope["byte_exact"] and all(m["byte_exact"] for m in mx.values())
    if not args.no_cpu:
        extras, line["cpu_baseline"] = cpu_baseline(case)
        par = parity_vs_method(out, extras["rows"], extras["method"])
        line["parity"] = par
        ok = ok and par["rel_l2_vs_method"] <= PARITY_GATE and par["max_row_err_vs_typical_row"] <= PARITY_ROW_GATE
        side = side_parity(case, extras["codes"], side_rows, got16, gotq)
        for name, r in side.items():
            line[name]["parity"] = r
            ok = ok and r["ok"]
        # VALU roofline of the attention kernel: the issue floor of its instruction stream (tile replay) at
        # the workload's share of rescaling tiles, over the measured kernel time at the measured clock
        frac = rescale_fraction(extras["codes"], N, H)
        floor = valu_floor(frac)
        wave_tiles_per_simd = (-(-N // 128)) * 4 * H * B * (-(-N // 64)) / 1024.0
        line["roofline"]["rescale_fraction"] = frac
        line["roofline"]["valu_floor_cycles_per_wave_tile"] = floor
        if floor is not None and sclk:
            t_floor = floor * wave_tiles_per_simd / (sclk * 1e6)
            line["roofline"]["valu_floor_ms_at_measured_sclk"] = t_floor * 1e3
            line["roofline"]["valu_frac"] = t_floor / (attn_mean * 1e-3)
        else:
            line["roofline"]["valu_frac"] = None
    else:
        line["parity"] = None
    print(json.dumps(line), flush=True)
    if not ok:
        print("bench.py: a timed output failed its check (parity gate of an oracle, or a byte-exact pair)",
              file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
