"""Throughput of the DiT denoising loop on one MI355X.

    python bench.py [--gpus 1] [--steps 40] [--warmup 3] [--workload 4]

Workload (default): the full 32-block DiT at 1024^2 -- hidden 4096, 32 heads x
128, SwiGLU 12288, L = 407 text tokens, N = 4096 image tokens (64 x 64),
bf16 random-init weights, seeded synthetic inputs.  One step is one pass of
the whole hot path: modulation rows, embed, 32 blocks, head and the fp32
Euler update.  The timed region is a denoising loop of --steps steps: step 1
is the joint pass that captures the text K/V, later steps run the image rows
only against the cache (exact text-K/V reuse), each followed by the Euler
update, with the FlowMatch schedule of the workload.  Inputs and weights are
resident in HBM before the timed region starts.

Printed: one JSON line with steps/s (whole job), the per-kernel durations of
the image-only steps measured with HIP events on the launch stream, the
roofline fraction of the dominant kernel, the CPU oracle's throughput on a
bounded sample (one image-only block, scaled to a step), and, as an extra,
true CFG on the same workload (a negative prompt of half the length in a
second K/V slot, both branches through every block at once), the
first-block cache (Fast mode), the 36-layer text encoder on the 1024^2
prompt, and the other workloads on the same weights: one full-width block
(L 22, N 256: HBM-bound, reported against the HBM peak), the 384^2 step
(L 494, N 576: where text is 46% of the joint sequence and reuse matters
most) and the 2048^2 step (L 512, N 16384: attention over 16896 tokens).
The CPU baseline is the oracle in fp32 numpy on a bounded sample of every
workload (block 0 of a joint and of an image-only step, scaled)."""
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

METRIC = "DiT steps/sec (32 blocks, bf16) at 1024² L=407; attn+GEMM MFMA util"
CFG_STEPS = 10
FBC_STEPS = 10
ENC_REPS = 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=40)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cfg", action="store_true", help="skip the true-CFG and first-block-cache extras")
    p.add_argument("--no-encoder", action="store_true", help="skip the text-encoder extra")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the other workloads (one full-width block, 384^2, 2048^2)")
    p.add_argument("--only-encoder", action="store_true",
                   help="run only the text-encoder measurement and print its JSON (for profiling)")
    p.add_argument("--threads", type=int, default=16, help="host threads for weight generation")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only copy 1 GiB device-to-device (10 times): the known-size reference for "
                        "scaling the HBM byte counters")
    p.add_argument("--calibrate", action="store_true",
                   help="only measure this GPU: register-only MFMA rates, copy bandwidth, vendor GEMM")
    return p.parse_args()


def calibrate_copy():
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": 4 * n, "bytes_written": 4 * n, "repeats": 10}))


def calibrate():
    """Sustained rates of the running part: the library's register-only MFMA
    loops, copy kernel, LDS / MFMA and VALU / MFMA instruction mixes (shader
    cycles per iteration of 8 waves per CU), and torch's (vendor library) bf16 GEMM on
    the four projection shapes of the 1024^2 step."""
    import ctypes

    import torch
    import torch.nn.functional as F

    from block_causal_attention_qi_amd import _lib
    lib = _lib.load_calib()
    res = {}
    for shape, name in ((0, "mfma_32x32x16_bf16_tflops"), (1, "mfma_16x16x32_bf16_tflops")):
        v = ctypes.c_double(0)
        _lib.check(lib.qi_calib_mfma_tflops(shape, 20000, ctypes.byref(v)), "qi_calib_mfma_tflops")
        res[name] = round(v.value, 1)
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    v = ctypes.c_double(0)
    _lib.check(lib.qi_calib_copy_gbs(a.data_ptr(), b.data_ptr(), n, 5, ctypes.byref(v)), "qi_calib_copy_gbs")
    res["copy_gbs_read_plus_write"] = round(v.value, 1)
    scratch = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    _lib.check(lib.qi_calib_read_gbs(a.data_ptr(), n, scratch.data_ptr(), 5, ctypes.byref(v)), "qi_calib_read_gbs")
    res["read_gbs"] = round(v.value, 1)
    del a, b, scratch
    lds = {}
    for mode, name in ((0, "8_ds_read_b128"), (1, "8_ds_write_b128"), (2, "8_mfma"),
                       (3, "8_mfma_6_reads_2_ds_writes"), (4, "8_mfma_6_reads_2_lds_copies")):
        v = ctypes.c_double(0)
        _lib.check(lib.qi_calib_lds_cycles(mode, 20000, ctypes.byref(v)), "qi_calib_lds_cycles")
        lds[name] = round(v.value, 1)
    res["lds_mix_cycles_per_iteration_per_cu"] = lds
    valu = {}
    for mode, name in ((0, "2w_32_exp"), (1, "2w_32_fma"), (2, "2w_8_mfma_32_exp_interleaved"),
                       (3, "2w_8_mfma_32_fma_interleaved"), (4, "2w_8_mfma"), (5, "mfma_wave_beside_exp_wave"),
                       (6, "mfma_wave_beside_fma_wave"), (7, "1w_8_mfma"), (8, "1w_32_exp"), (9, "1w_32_fma")):
        v = ctypes.c_double(0)
        _lib.check(lib.qi_calib_valu_ns(mode, 20000, ctypes.byref(v)), "qi_calib_valu_ns")
        valu[name] = round(v.value, 1)
    res["valu_mix_ns_per_iteration"] = valu
    gemm = {}
    for (M, N, K) in [(4096, 24576, 4096), (4096, 12288, 4096), (4096, 4096, 12288), (4096, 4096, 4096)]:
        A = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        W = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            F.linear(A, W)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            F.linear(A, W)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        gemm[f"{M}x{N}x{K}"] = round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)
    res["vendor_bf16_gemm_tflops"] = gemm
    print(json.dumps({"calibration": "MI355X", **res}))


def host_info():
    """CPU model, core count and the BLAS numpy uses (threads it runs)."""
    blas, cores = "unknown", os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        pass
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:  # pragma: no cover
        pass
    return {"cpu_model": cpu_model, "nproc": os.cpu_count(), "blas": blas, "cores": int(cores)}


def cpu_oracle_config(wl, joint_block=True):
    """The oracle as it stands, in fp32 numpy, on one workload: the shared
    part of a step (modulation rows, embed, head) and block 0 on the step's
    real input -- a joint pass over [text | image] and an image-only pass on
    the text K/V the joint pass captured -- each timed once with
    perf_counter; a step is the shared part plus n_blocks blocks (every block
    has the same shape and work).  joint_block=False skips the joint block
    (its time is then not reported)."""
    import qi_synth as qs
    from oracle import dit
    f32 = np.float32
    H, L, N = wl.hidden, wl.L, wl.N
    sw = qs.weights_as_f32(qs.shared_weights(wl, as_bf16=wl.bf16_weights, threads=8))
    bw = qs.weights_as_f32(qs.block_weights(wl, 0, as_bf16=wl.bf16_weights, threads=8))
    X, E = qs.img_tokens(wl), qs.txt_feats(wl)
    tc, ts, ic, is_ = dit.rope_rows(L, wl.h, wl.w)
    t = f32(0.7)
    t0 = time.perf_counter()
    m_txt, m_img = dit.modulation_rows(sw["w_mod"], sw["b_mod"], t, H, f32)
    x = dit.embed(sw, X, E, f32)
    dit.head(sw, x[L:])
    t_shared = time.perf_counter() - t0
    out = {"shared_s": round(t_shared, 3)}
    if joint_block:
        cos, sin = np.concatenate([tc, ic]), np.concatenate([ts, is_])
        t0 = time.perf_counter()
        _, kv = dit.dit_block(x, L, bw, m_txt, m_img, cos, sin, wl.heads)
        out["joint_block_s"] = round(time.perf_counter() - t0, 3)
    else:
        kv = tuple(qs.normal_array((wl.heads, L, 128), seed=33 + i) for i in range(2))
    t0 = time.perf_counter()
    dit.dit_block(x[L:], 0, bw, m_txt, m_img, ic, is_, wl.heads, kv_text=kv)
    out["image_only_block_s"] = round(time.perf_counter() - t0, 3)
    nb = wl.n_blocks
    out["image_only_step_s"] = round(t_shared + nb * out["image_only_block_s"], 2)
    if joint_block:
        out["joint_step_s"] = round(t_shared + nb * out["joint_block_s"], 2)
    return out


def cpu_baseline(wl4, extra_workloads=(2, 3, 5)):
    """The CPU oracle's throughput on the benchmark's workload (1024^2) as
    the same 40-step loop the GPU runs (1 joint + 39 image-only steps), from
    the bounded sample of cpu_oracle_config, plus the same figures for the
    other workloads (the 2048^2 one image-only only, which keeps the whole
    sample near half a minute of CPU time)."""
    import qi_synth as qs
    info = host_info()
    per = {}
    c4 = cpu_oracle_config(wl4)
    per[wl4.name] = c4
    for k in extra_workloads:
        wl = qs.workload(k)
        log(f"cpu oracle (fp32) on {wl.name}")
        per[wl.name] = cpu_oracle_config(wl, joint_block=(k != 5))
    loop_s = (c4["joint_step_s"] + 39 * c4["image_only_step_s"]) / 40
    log(f"cpu oracle (fp32): {loop_s:.1f} s per loop step at {wl4.name}")
    return {"value": 1.0 / loop_s, "unit": "steps/s", "cores": info["cores"], "kind": "oracle",
            "cpu_model": info["cpu_model"], "nproc": info["nproc"], "blas": info["blas"],
            "sample": f"oracle in fp32 numpy: the shared part and block 0 of a joint and of an image-only step of "
                      f"{wl4.name}, each timed once; step = shared + {wl4.n_blocks} blocks; value = 40 / (joint step "
                      f"+ 39 image-only steps)", "per_workload": per}


def measured_traffic(kind: str):
    """HBM bytes per image-only launch of `kind` from the committed rocprofv3
    counter summary (FETCH_SIZE / WRITE_SIZE scaled by a 1 GiB copy), or None
    when the kernel sources have changed since the counters were taken."""
    from block_causal_attention_qi_amd.profile_summary import kernel_source_sha256
    path = os.path.join(ROOT, "profiles", "dit32_1024px_hbm_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None, "no counter summary"
    if kernel_source_sha256() != rec.get("kernel_source_sha256"):
        return None, "kernels changed since the counters were taken"
    ent = rec.get("kernels", {}).get(kind, {}).get("image-only")
    if not ent:
        return None, "kernel not in the counter summary"
    return int(ent["hbm_bytes"]), "profiles/dit32_1024px_hbm_traffic.json"


def measure_workload(qi, qs, wl, model, loop_steps, n_img, n_joint=3):
    """One workload on the device model (a reported extra): a denoising loop
    of loop_steps steps (step 1 joint with capture, then image-only steps on
    the cache, each followed by the Euler update) timed with events; the
    first call; the median of n_joint warm joint steps and of n_img warm
    image-only steps, each timed alone; per-kernel durations over n_img
    image-only steps with the library's event timer; FLOP and byte rates from
    the FLOP model."""
    import torch

    from block_causal_attention_qi_amd import flops
    dev = "cuda"
    H, N, L, nb = wl.hidden, wl.N, wl.L, wl.n_blocks
    dims = model.dims
    x0 = torch.from_numpy(qs.img_tokens(wl)).to(dev)
    txt = torch.from_numpy(qs.txt_feats(wl)).to(dev)
    rope = [torch.from_numpy(a).to(dev) for a in qi.rope_tables(L, wl.h, wl.w)]
    sig, ts = qi.flow_sigmas(40, N)
    tin = [np.float32(ts[i]) / np.float32(1000) for i in range(40)]
    ws = qi.Workspace(dims, L, N, dev)
    cache = qi.KVCache(dims, L, dev)
    vel = torch.empty((N, 64), dtype=torch.float32, device=dev)
    x = torch.empty_like(x0)

    def step(i):
        k = i % 40
        if k == 0:
            qi.text_kv_capture(model, L, N, x, txt, tin[k], *rope, cache, vel, ws)
        else:
            qi.dit_step(model, L, N, x, None, tin[k], None, None, rope[2], rope[3], vel, ws, cache)
        qi.euler_update(x, vel, sig[k], sig[k + 1])

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    x.copy_(x0)
    torch.cuda.synchronize()
    first_ms = timed(lambda: step(0))

    def loop():
        x.copy_(x0)
        for i in range(loop_steps):
            step(i)
    loop()                                     # warm
    loop_ms = timed(loop)
    joint_ms = float(np.median([timed(lambda: (x.copy_(x0), step(0))) for _ in range(n_joint)]))
    img_ms = float(np.median([timed(lambda i=i: step(i)) for i in range(1, 1 + n_img)]))
    qi.timing_begin(4096 * 4)
    for i in range(1, 1 + n_img):
        step(i)
    timing = qi.timing_end()
    if not torch.isfinite(vel).all():
        raise RuntimeError(f"non-finite vel at {wl.name}")
    sh_img = flops.Shape(H, wl.ffn, L, N, nb, wl.txt_dim, joint=False)
    sh_joint = flops.Shape(H, wl.ffn, L, N, nb, wl.txt_dim, joint=True)
    work = flops.kernel_work(sh_img)
    kern = {}
    for kind, (ms, cnt) in timing.items():
        if cnt == 0 or kind not in work:
            continue
        ent = {"avg_us": round(ms / cnt * 1e3, 2)}
        f, b = work[kind]
        if f and kind.startswith(("gemm", "attention")):
            tf = f / (ms / cnt * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), frac_bf16_peak=round(tf / flops.PEAK_BF16_TFLOPS, 4))
        elif b:
            ent.update(gbs=round(b / (ms / cnt * 1e-3) / 1e9, 1))
        kern[kind] = ent
    gemm_ms = sum(timing[k][0] for k in timing if k.startswith("gemm")) / n_img
    gemm_f = sum(work[k][0] * timing[k][1] for k in work if k.startswith("gemm") and k in timing) / n_img
    attn_ms = timing["attention"][0] / n_img
    attn_f = work["attention"][0] * nb
    out = {"workload": wl.name, "blocks": nb, "L": L, "N": N,
           "loop": f"{loop_steps} steps: 1 joint + {loop_steps - 1} image-only, Euler update each",
           "loop_steps_per_s": round(loop_steps / (loop_ms * 1e-3), 3),
           "first_call_joint_step_ms": round(first_ms, 3),
           f"joint_step_ms_median_of_{n_joint}": round(joint_ms, 3),
           f"image_only_step_ms_median_of_{n_img}": round(img_ms, 3),
           "reuse_speedup_joint_over_image_only": round(joint_ms / img_ms, 3),
           "ms_per_block_image_only": round(img_ms / nb, 4),
           "step_tflops_image_only": round(flops.step_flops(sh_img) / (img_ms * 1e-3) / 1e12, 1),
           "step_tflops_joint": round(flops.step_flops(sh_joint) / (joint_ms * 1e-3) / 1e12, 1),
           "gemm_tflops_image_only": round(gemm_f / (gemm_ms * 1e-3) / 1e12, 1),
           "gemm_mfma_frac": round(gemm_f / (gemm_ms * 1e-3) / 1e12 / flops.PEAK_BF16_TFLOPS, 4),
           "attention_tflops_image_only": round(attn_f / (attn_ms * 1e-3) / 1e12, 1),
           "attention_mfma_frac": round(attn_f / (attn_ms * 1e-3) / 1e12 / flops.PEAK_BF16_TFLOPS, 4),
           "kernels_image_only": kern}
    # attention over the joint pass's L + N keys (text rows causal), one launch per block
    qi.timing_begin(4096)
    x.copy_(x0)
    step(0)
    tj = qi.timing_end()
    aj = flops.kernel_work(sh_joint)["attention"][0] * nb / (tj["attention"][0] * 1e-3) / 1e12
    out["attention_tflops_joint"] = round(aj, 1)
    out["attention_joint_tokens"] = L + N
    # the joint step's algorithmic bytes against the HBM peak (what bounds a
    # one-block step at small T)
    jb = flops.step_bytes(sh_joint)
    out["joint_step_bytes"] = jb
    out["joint_step_gbs"] = round(jb / (joint_ms * 1e-3) / 1e9, 1)
    out["joint_step_frac_hbm_peak"] = round(jb / (joint_ms * 1e-3) / 1e9 / flops.PEAK_HBM_GBS, 4)
    log(f"{wl.name}: {out['loop_steps_per_s']} steps/s over the loop, joint {joint_ms:.3f} ms, "
        f"image-only {img_ms:.3f} ms")
    return out


def profiled_duration(kind: str):
    """Average duration (us) of `kind`'s image-only launches in the committed
    rocprofv3 kernel trace (profiles/dit32_1024px_kernel_trace.json), or None
    when the kernel sources have changed since the trace was taken."""
    from block_causal_attention_qi_amd.profile_summary import kernel_source_sha256
    path = os.path.join(ROOT, "profiles", "dit32_1024px_kernel_trace.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None, "no kernel-trace summary"
    if kernel_source_sha256() != rec.get("kernel_source_sha256"):
        return None, "kernels changed since the trace was taken"
    ent = rec.get("kinds", {}).get(kind, {}).get("image-only")
    if not ent:
        return None, "kernel not in the trace summary"
    return float(ent["avg_us"]), "profiles/dit32_1024px_kernel_trace.json"


class ClockSampler:
    """Samples the GPU's current shader clock (the level marked '*' in the
    driver's pp_dpm_sclk file) from a host thread while running; the mean of
    the samples is the clock the timed region ran at.  Reports None where the
    file is not readable."""

    def __init__(self, period_s: float = 0.005):
        import glob
        self.period = period_s
        self.path = next((p for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
                          if self._read(p) is not None), None)
        self.samples = []
        self._stop = None
        self._thread = None

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                for ln in f:
                    if "*" in ln:
                        v = ln.split(":", 1)[1].strip().rstrip("*").strip().lower()
                        return float(v.replace("mhz", "").strip())
        except (OSError, ValueError, IndexError):
            return None
        return None

    def __enter__(self):
        import threading
        if self.path is None:
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                v = self._read(self.path)
                if v is not None:
                    self.samples.append(v)
                self._stop.wait(self.period)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        a = np.asarray(self.samples)
        return {"mean_mhz": round(float(a.mean()), 1), "median_mhz": round(float(np.median(a)), 1),
                "min_mhz": round(float(a.min()), 1), "max_mhz": round(float(a.max()), 1), "samples": int(a.size),
                "source": self.path}


def measure_cfg(qi, qs, wl, model, dims, x0, rope, sig, tin, img_step_ms):
    """True CFG on the same workload (a reported extra, not the headline): both
    prompts captured on step 1, then image-only CFG steps running both
    branches through every block at once, each followed by the fused CFG
    Euler update.  Timed over CFG_STEPS steps with events."""
    import torch
    N, L = wl.N, wl.L
    Ln = qs.neg_prompt_len(wl)
    dev = "cuda"
    txt = torch.from_numpy(qs.txt_feats(wl)).to(dev)
    txt_neg = torch.from_numpy(qs.neg_txt_feats(wl)).to(dev)
    rope_n = [torch.from_numpy(a).to(dev) for a in qi.rope_tables(Ln, wl.h, wl.w)]
    cos2 = torch.cat([rope[2], rope_n[2]]).contiguous()
    sin2 = torch.cat([rope[3], rope_n[3]]).contiguous()
    c_pos, c_neg = qi.KVCache(dims, L, dev), qi.KVCache(dims, Ln, dev)
    ws = qi.Workspace(dims, max(L, Ln), N, dev)
    cws = qi.CfgWorkspace(dims, N, dev)
    vel = torch.empty((N, 64), dtype=torch.float32, device=dev)
    vel2 = torch.empty((2, N, 64), dtype=torch.float32, device=dev)
    x = x0.clone()
    g = 2.5
    qi.text_kv_capture(model, L, N, x, txt, tin[0], *rope, c_pos, vel, ws)
    qi.text_kv_capture(model, Ln, N, x, txt_neg, tin[0], *rope_n, c_neg, vel, ws)
    qi.dit_step_cfg(model, N, x, tin[1], cos2, sin2, c_pos, c_neg, vel2, cws)   # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(1, 1 + CFG_STEPS):
        qi.dit_step_cfg(model, N, x, tin[k], cos2, sin2, c_pos, c_neg, vel2, cws)
        qi.euler_update_cfg(x, vel2, g, sig[k], sig[k + 1])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / CFG_STEPS
    if not torch.isfinite(x).all():
        raise RuntimeError("non-finite latents in the CFG loop")
    log(f"CFG: {ms:.2f} ms per image-only CFG step (two single steps: {2 * img_step_ms:.2f} ms)")
    return {"guidance": g, "L_pos": L, "L_neg": Ln, "steps": CFG_STEPS,
            "image_only_step_ms": round(ms, 3), "steps_per_s": round(1e3 / ms, 3),
            "vs_two_single_steps": round(2 * img_step_ms / ms, 3)}


def measure_fbc(qi, qs, wl, model, dims, x0, rope, sig, tin, img_step_ms):
    """First-block cache (Fast mode) on the same workload, a reported extra:
    FBC_STEPS image-only steps at the page's threshold 0.08 (on random-init
    weights block 0's residual changes far more than that, so nothing is
    skipped: the figure is the bookkeeping overhead), then the same steps with
    every step after the first skipped (an unbounded threshold): the cost of a
    skipped step."""
    import torch
    N, L = wl.N, wl.L
    dev = "cuda"
    txt = torch.from_numpy(qs.txt_feats(wl)).to(dev)
    cache = qi.KVCache(dims, L, dev)
    ws = qi.Workspace(dims, L, N, dev)
    fbc = qi.FirstBlockCache(dims, N, dev)
    vel = torch.empty((N, 64), dtype=torch.float32, device=dev)
    out = {}
    for name, thr in (("threshold_0.08", 0.08), ("always_skip", 3.0e38)):
        x = x0.clone()
        qi.text_kv_capture(model, L, N, x, txt, tin[0], *rope, cache, vel, ws)
        fbc.reset()
        qi.dit_step_fbc(model, L, N, x, tin[1], rope[2], rope[3], cache, thr, fbc, vel, ws)   # fills the cache
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(2, 2 + FBC_STEPS):
            qi.dit_step_fbc(model, L, N, x, tin[k], rope[2], rope[3], cache, thr, fbc, vel, ws)
            qi.euler_update(x, vel, sig[k], sig[k + 1])
        e1.record()
        st = fbc.stats()
        ms = e0.elapsed_time(e1) / FBC_STEPS
        out[name] = {"image_only_step_ms": round(ms, 3), "skipped": st["skipped"], "steps_incl_first": st["steps"],
                     "last_change": round(st["last_change"], 4)}
        log(f"FBC {name}: {ms:.2f} ms per step, {st['skipped']} of {st['steps']} skipped, "
            f"last change {st['last_change']:.3f}")
    out["exact_image_only_step_ms"] = round(img_step_ms, 3)
    return out


def measure_encoder(qi, qs, threads):
    """The 36-layer text encoder on the 1024^2 prompt (407 DiT tokens plus
    the 14-token system prefix, L = 421), a reported extra: ENC_REPS forwards
    timed with events, per-kernel durations from the library's launch timer,
    FLOPs of the plain definition.  Each fp32 GEMM product runs as three bf16
    MFMA passes over the exact 3-plane split of the activations, so the MFMA
    work issued is three times the GEMM FLOPs."""
    import concurrent.futures as cf

    import torch

    from block_causal_attention_qi_amd import flops
    ew = qs.enc_workload(3)
    L = ew.L_full
    dims = qi.make_enc_dims(ew.hidden, ew.heads, ew.kv_heads, ew.ffn, ew.n_layers, ew.vocab)
    t0 = time.time()
    with cf.ThreadPoolExecutor(threads) as ex:
        layers = ex.map(lambda i: qs.enc_layer_weights(ew, i, threads=1), range(ew.n_layers))
        model = qi.DeviceEncoder(dims, qs.enc_embed(ew), layers)
    log(f"encoder weights ({ew.n_layers} layers) on device in {time.time() - t0:.1f} s")
    ids = torch.from_numpy(qs.enc_input_ids(ew).astype(np.int32)).cuda()
    c, s = (torch.from_numpy(a).cuda() for a in qi.enc_rope_table(L, ew.rope_theta))
    out = torch.empty((L, ew.hidden), dtype=torch.float32, device="cuda")
    ws = qi.EncWorkspace(dims, L)
    qi.text_encoder_fwd(model, ids, L, c, s, out, ws)      # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(ENC_REPS):
        qi.text_encoder_fwd(model, ids, L, c, s, out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / ENC_REPS
    qi.timing_begin(4096)
    qi.text_encoder_fwd(model, ids, L, c, s, out, ws)
    timing = qi.timing_end()
    if not torch.isfinite(out).all():
        raise RuntimeError("non-finite encoder output")
    fl = flops.encoder_flops(ew.hidden, ew.heads, ew.kv_heads, ew.ffn, ew.n_layers, L)
    kern = {}
    for kind in ("enc_gemm", "enc_attention", "enc_misc"):
        t, n = timing[kind]
        kern[kind] = {"launches": n, "ms": round(t, 3)}
    g_ms, a_ms = timing["enc_gemm"][0], timing["enc_attention"][0]
    kern["enc_gemm"].update(fp32_tflops=round(fl["gemm"] / (g_ms * 1e-3) / 1e12, 1),
                            bf16_mfma_tflops_issued=round(3 * fl["gemm"] / (g_ms * 1e-3) / 1e12, 1))
    kern["enc_attention"].update(fp32_tflops=round(fl["attention"] / (a_ms * 1e-3) / 1e12, 1))
    log(f"encoder: {ms:.2f} ms per forward ({ew.n_layers} layers, L {L})")
    return {"workload": ew.name, "layers": ew.n_layers, "L": L, "hidden": ew.hidden, "reps": ENC_REPS,
            "ms_per_forward": round(ms, 3), "tflops_fp32_effective": round(fl["total"] / (ms * 1e-3) / 1e12, 1),
            "flops_per_forward": fl["total"], "kernels": kern}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate:
        calibrate()
        return
    if args.only_encoder:
        import block_causal_attention_qi_amd as qi
        import qi_synth as qs
        print(json.dumps({"text_encoder": measure_encoder(qi, qs, args.threads)}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the DiT step here is built and measured on one MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    import block_causal_attention_qi_amd as qi
    import qi_synth as qs
    from block_causal_attention_qi_amd import flops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    wl = qs.workload(args.workload)
    H, N, L, nb = wl.hidden, wl.N, wl.L, wl.n_blocks
    dims = qi.make_dims(H, wl.ffn, nb, wl.txt_dim)
    t0 = time.time()
    log(f"generating {nb} blocks of bf16 weights ({wl.name})")
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(args.threads) as ex:
        blocks = ex.map(lambda b: qs.block_weights(wl, b, as_bf16=True, threads=1), range(nb))
        model = qi.DeviceModel(dims, qs.shared_weights(wl, as_bf16=True), blocks, dev)
    log(f"weights on device in {time.time() - t0:.1f} s")

    x0 = torch.from_numpy(qs.img_tokens(wl)).to(dev)
    txt = torch.from_numpy(qs.txt_feats(wl)).to(dev)
    rope = [torch.from_numpy(a).to(dev) for a in qi.rope_tables(L, wl.h, wl.w)]
    sig, ts = qi.flow_sigmas(40, N)
    tin = [np.float32(ts[i]) / np.float32(1000) for i in range(40)]
    ws = qi.Workspace(dims, L, N, dev)
    cache = qi.KVCache(dims, L, dev)
    vel = torch.empty((N, 64), dtype=torch.float32, device=dev)
    x = torch.empty_like(x0)

    def step(i):
        k = i % 40
        if k == 0:
            qi.text_kv_capture(model, L, N, x, txt, tin[k], *rope, cache, vel, ws)
        else:
            qi.dit_step(model, L, N, x, None, tin[k], None, None, rope[2], rope[3], vel, ws, cache)
        qi.euler_update(x, vel, sig[k], sig[k + 1])

    def loop(K):
        x.copy_(x0)
        for i in range(K):
            step(i)

    # first call: the joint step on a fresh process (cold caches and code)
    x.copy_(x0)
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    step(0)
    f1.record()
    torch.cuda.synchronize()
    first_call_ms = f0.elapsed_time(f1)

    log(f"warmup {args.warmup} steps")
    loop(args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: K steps of the denoising loop
    K = args.steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    loop(K)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    value = K / elapsed
    log(f"timed {K} steps: {elapsed * 1e3:.1f} ms -> {value:.3f} steps/s")
    if not torch.isfinite(vel).all():
        raise RuntimeError("non-finite vel in the timed loop")

    # ---- per-kernel durations over image-only steps (events on the launch stream)
    x.copy_(x0)
    step(0)
    n_img = max(3, min(K - 1, 10))
    qi.timing_begin(4096 * 4)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clock:
        ev0.record()
        for i in range(1, 1 + n_img):
            step(i)
        ev1.record()
        timing = qi.timing_end()
    img_step_ms = ev0.elapsed_time(ev1) / n_img
    # warm calls, each timed on its own: 10 image-only steps and the joint step
    x.copy_(x0)
    step(0)
    torch.cuda.synchronize()
    per_step = []
    for i in range(1, 11):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step(i)
        e1.record()
        torch.cuda.synchronize()
        per_step.append(e0.elapsed_time(e1))
    img_step_median_ms = float(np.median(per_step))
    x.copy_(x0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    step(0)
    e1.record()
    torch.cuda.synchronize()
    joint_step_ms = e0.elapsed_time(e1)

    shape = flops.Shape(H, wl.ffn, L, N, nb, wl.txt_dim, joint=False)
    work = flops.kernel_work(shape)
    kernels = {}
    for kind, (ms, cnt) in timing.items():
        if cnt == 0:
            continue
        avg_ms = ms / cnt
        f, b = work.get(kind, (0, 0))
        ent = {"launches": cnt, "avg_us": round(avg_ms * 1e3, 2), "ms_per_step": round(ms / n_img, 3)}
        if f and kind.startswith(("gemm", "attention")):
            tf = f / (avg_ms * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), frac_bf16_peak=round(tf / flops.PEAK_BF16_TFLOPS, 4))
        elif b:
            gbs = b / (avg_ms * 1e-3) / 1e9
            ent.update(gbs=round(gbs, 1), frac_hbm_peak=round(gbs / flops.PEAK_HBM_GBS, 4))
        kernels[kind] = ent
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dms = timing[dom][0] / timing[dom][1]
    df, db = work[dom]
    if df and dom.startswith(("gemm", "attention")):
        ach = df / (dms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": flops.PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / flops.PEAK_BF16_TFLOPS, 4), "traffic": None,
                "flops_per_launch": df, "avg_launch_us": round(dms * 1e3, 2)}
    else:
        ach = db / (dms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": flops.PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / flops.PEAK_HBM_GBS, 4), "traffic": None,
                "bytes_per_launch": db, "avg_launch_us": round(dms * 1e3, 2)}
    roof["traffic"], roof["traffic_source"] = measured_traffic(dom)
    prof_us, roof["profile_source"] = profiled_duration(dom)
    roof["profile_avg_launch_us"] = prof_us
    if prof_us:
        pa = (df / (prof_us * 1e-6) / 1e12) if roof["bound"] == "mfma" else (db / (prof_us * 1e-6) / 1e9)
        roof["frac_from_profile"] = round(pa / roof["peak"], 4)
    else:
        roof["frac_from_profile"] = None
    roof["sclk_during_kernel_timing"] = clock.summary()
    gemm_ms = sum(timing[k][0] for k in timing if k.startswith("gemm")) / n_img
    gemm_f = sum(work[k][0] * timing[k][1] for k in work if k.startswith("gemm") and k in timing) / n_img
    attn_ms = timing["attention"][0] / n_img
    step_f = flops.step_flops(shape)
    cfg = None if args.no_cfg else measure_cfg(qi, qs, wl, model, dims, x0, rope, sig, tin, img_step_ms)
    fbc = None if args.no_cfg else measure_fbc(qi, qs, wl, model, dims, x0, rope, sig, tin, img_step_ms)
    enc = None if args.no_encoder else measure_encoder(qi, qs, args.threads)
    others = None
    if not args.no_workloads and args.workload == 4:
        others = {}
        for k, view, loop_steps, n_img, n_joint in ((2, model.prefix(1), 40, 10, 5), (3, model, 40, 10, 5),
                                                     (5, model, 6, 3, 2)):
            w2 = qs.workload(k)
            assert view.dims.n_blocks == w2.n_blocks and w2.hidden == H
            others[w2.name] = measure_workload(qi, qs, w2, view, loop_steps, n_img, n_joint)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, (2, 3, 5) if args.workload == 4 else ())

    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / K, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and inputs)",
        "config": {"workload": wl.name, "hidden": H, "heads": wl.heads, "ffn": wl.ffn, "blocks": nb,
                   "L": L, "N": N, "grid": f"{wl.h}x{wl.w}", "loop": "step 1 joint + capture, then image-only "
                   "steps on cached text K/V, fp32 Euler update each step", "parallelism": "single GPU"},
        "image_only_step_ms": round(img_step_ms, 3),
        "image_only_step_ms_median_of_10": round(img_step_median_ms, 3),
        "joint_step_ms": round(joint_step_ms, 3),
        "first_call_joint_step_ms": round(first_call_ms, 3),
        "ms_per_block_image_only": round(img_step_ms / nb, 4),
        "step_tflops_image_only": round(step_f / (img_step_ms * 1e-3) / 1e12, 1),
        "gemm_tflops": round(gemm_f / (gemm_ms * 1e-3) / 1e12, 1),
        "gemm_mfma_frac": round(gemm_f / (gemm_ms * 1e-3) / 1e12 / flops.PEAK_BF16_TFLOPS, 4),
        "attention_tflops": round(work["attention"][0] * nb / (attn_ms * 1e-3) / 1e12, 1),
        "attention_mfma_frac": round(work["attention"][0] * nb / (attn_ms * 1e-3) / 1e12 / flops.PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": cpu,
        "cfg": cfg,
        "first_block_cache": fbc,
        "text_encoder": enc,
        "workloads": others,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
