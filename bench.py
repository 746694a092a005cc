"""Decode-attention benchmark on one MI355X.

A step is one pass of the hot path over one batch: the step's new tokens
(the last q_len tokens of every request) are quantized and stored, and the
decode attends the cache they were written to.  The step is one
pa_decode_write call (after the indexer, for the config that draws its
block-sparse lists from it): the decode's main kernel writes the new
tokens with kv_quant_write's code and attends them, plus the log-sum-exp
merge kernel when the plan splits the context; calls the library cannot
fuse (a bf16 cache, long q_len) run its writer first.  --separate-write
runs kv_quant_write, then pa_decode_ex (main kernel and merge).
The default workload is the long-context shape: batch 32, q_len 1, one KV
head x 16 query heads, head_dim 128, 128-token pages, context 131072 each
(1024 pages per request), per-token e4m3 scales, block tables drawn from a
32768-page pool -- 1.1 GB of KV per step, so every step reads it from HBM.
Smaller shapes (--config c2: batch 4 at 8K contexts, ...) replicate their
cache over up to 64 layers (distinct cache tensors sharing one block table)
and steps rotate through them, as consecutive attention layers of one model
would, so every step reads its KV from HBM rather than from the 256 MB
Infinity Cache.

Timing: W untimed warmup steps, then exactly K steps replayed from captured
HIP graphs, bracketed by torch.cuda.synchronize().  The main decode kernel's
own duration is measured with HIP events recorded around it on the launch
stream.  One cold launch (idle GPU, caches evicted first) is reported beside
the steady state.  The CPU oracle is then timed on the host's cores (one
single-threaded process per core, at most 16) over requests of the same
workload, and checks the GPU's output on them.  Prints one JSON line.

Long query segments (--config p16k, and p16kb over a bf16 cache: a
16384-token prompt as one request) run the prefill kernel, whose roofline
is the bf16 MFMA one.  --issue-probe prints the probe library's
instruction rates, launch floor and workgroup start spread instead.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_paged_kv_pa_amd as pa  # noqa: E402
import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0

CONFIGS = {
    "c1": lambda: wl.c1_tiny(),
    "c2": lambda: wl.c2_dense_8k(),
    "c3": lambda: wl.c3_dense_128k(wl.PER_TOKEN),
    "c3s": lambda: wl.c3_dense_128k(wl.SCALAR),
    "c4": lambda: wl.c4_spec("uniform"),
    "c4r": lambda: wl.c4_spec("ragged"),
    "c4m": lambda: wl.c4_spec("mixed"),
    "c5": lambda: wl.c5_sparse(False),
    "c5t": lambda: wl.c5_sparse(True),
    # the same shapes over the unquantized bf16 cache (the FP8 cache's control)
    "c2b": lambda: wl.bf16_kv(wl.c2_dense_8k()),
    "c3b": lambda: wl.bf16_kv(wl.c3_dense_128k(wl.PER_TOKEN)),
    "c4b": lambda: wl.bf16_kv(wl.c4_spec("uniform")),
    "c5b": lambda: wl.bf16_kv(wl.c5_sparse(False)),
    # the sparse indexer in the step: write, index top-32, block-sparse decode
    "c5i": lambda: wl.index_workload("c5"),
    # per-token-as-decode prefill of a 16K prompt (one q_len-16384 request)
    "p16k": lambda: wl.prefill_16k(),
    "p16kb": lambda: wl.bf16_kv(wl.prefill_16k()),
}
# shapes whose main kernel is bound by the matrix cores, not HBM: their
# roofline is algorithmic flops against the dense bf16 MFMA peak
MFMA_BOUND = {"p16k", "p16kb"}
# query positions per workgroup of the prefill kernel (calls whose requests
# hold at least 128 rows run it; pa_plan_describe reports this row count)
PREFILL_POSITIONS = 8
BF16_MFMA_PEAK_TFLOPS = 2500.0
INDEX_TOPK = {"c5i": 32}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Layers:
    """The workload's cache replicated over `n` layers: one allocation,
    whose pages [l*NB, (l+1)*NB) are layer l's cache tensor.  Every layer
    uses the same block table and slot mapping, as a model's layers share a
    request's block table and each has its own cache."""

    def __init__(self, w, n, dev, index_topk=0):
        self.w, self.n, self.dev = w, n, dev
        self.index_topk = index_topk
        NB, Hkv = w.num_blocks, w.Hkv
        tot = NB * n
        bf = w.kv_dtype == "bf16"
        self.kc = torch.empty(tot, Hkv, 16384, dtype=torch.int16 if bf else torch.uint8, device=dev)
        self.vc = torch.empty_like(self.kc)
        self.ks = torch.empty(tot, Hkv, 128, dtype=torch.float32, device=dev)
        self.vs = torch.empty_like(self.ks)
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed)
        # unwritten slots hold random finite codes and large scales (bf16:
        # random bit patterns); no scales for a bf16 cache
        if bf:
            self.kc[:NB].random_(-32768, 32768, generator=g)
            self.vc[:NB].random_(-32768, 32768, generator=g)
            self.kc = self.kc.view(torch.bfloat16)
            self.vc = self.vc.view(torch.bfloat16)
        else:
            self.kc[:NB].random_(0, 0x7F, generator=g)
            self.vc[:NB].random_(0, 0x7F, generator=g)
        self.ks[:NB].fill_(1e3)
        self.vs[:NB].fill_(1e3)
        self.mode = w.mode
        if w.mode == wl.SCALAR:
            self.ks_arg = torch.tensor([w.k_scalar], dtype=torch.float32, device=dev)
            self.vs_arg = torch.tensor([w.v_scalar], dtype=torch.float32, device=dev)
        elif w.mode == wl.NONE:
            self.ks_arg = self.vs_arg = None
        else:
            self.ks_arg, self.vs_arg = self.ks, self.vs
        t0 = time.time()
        for b in range(w.B):
            pages = w.written[b]
            for i in range(0, len(pages), 256):
                k, v, s = w.request_kv(b, pages[i:i + 256])
                pa.kv_quant_write(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                                  torch.from_numpy(s).to(dev), self.kc, self.vc, self.ks_arg,
                                  self.vs_arg, self.mode)
        torch.cuda.synchronize()
        for l in range(1, n):
            self.kc[l * NB:(l + 1) * NB].copy_(self.kc[:NB])
            self.vc[l * NB:(l + 1) * NB].copy_(self.vc[:NB])
            self.ks[l * NB:(l + 1) * NB].copy_(self.ks[:NB])
            self.vs[l * NB:(l + 1) * NB].copy_(self.vs[:NB])
        torch.cuda.synchronize()
        log(f"cache for {w.name} x {n} layers written in {time.time() - t0:.1f}s")
        # per-layer cache views, one shared block table
        self.kcl = [self.kc[l * NB:(l + 1) * NB] for l in range(n)]
        self.vcl = [self.vc[l * NB:(l + 1) * NB] for l in range(n)]
        if w.mode == wl.PER_TOKEN:
            self.ksl = [self.ks[l * NB:(l + 1) * NB] for l in range(n)]
            self.vsl = [self.vs[l * NB:(l + 1) * NB] for l in range(n)]
        else:
            self.ksl, self.vsl = [self.ks_arg] * n, [self.vs_arg] * n
        bt = torch.from_numpy(w.block_table).to(dev)
        self.bt = [bt] * n
        self.ctx = torch.from_numpy(w.ctx).to(dev)
        self.cu = None if w.cu is None else torch.from_numpy(w.cu).to(dev)
        self.sp = None if w.sparse is None else torch.from_numpy(w.sparse).to(dev)
        q = torch.from_numpy(w.q).to(dev).to(torch.bfloat16)
        self.q = [q.clone() for _ in range(n)]
        self.out = [torch.empty(w.rows, w.Hq, 128, dtype=torch.bfloat16, device=dev) for _ in range(n)]
        k, v, s = w.step_tokens()
        self.step_k = torch.from_numpy(k).to(dev)
        self.step_v = torch.from_numpy(v).to(dev)
        self.step_slots = [torch.from_numpy(s).to(dev)] * n
        self.max_q_len = int(w.q_lens.max())
        if index_topk:
            # index cache over the same pages (layer l at pool pages l*NB ...),
            # index queries, and per-layer score and list buffers
            t1 = time.time()
            self.icache = torch.empty(tot, 128, 128, dtype=torch.uint8, device=dev)
            self.icache[:NB].copy_(torch.from_numpy(w.index_cache().reshape(NB, 128, 128)))
            for l in range(1, n):
                self.icache[l * NB:(l + 1) * NB].copy_(self.icache[:NB])
            self.icl = [self.icache[l * NB:(l + 1) * NB] for l in range(n)]
            self.q_idx = torch.from_numpy(w.index_queries()).to(dev).to(torch.bfloat16)
            self.scores = [torch.empty(w.rows, w.W, dtype=torch.float32, device=dev) for _ in range(n)]
            self.lists = [torch.empty(w.rows, index_topk, dtype=torch.int32, device=dev) for _ in range(n)]
            torch.cuda.synchronize()
            log(f"index cache x {n} layers ready in {time.time() - t1:.1f}s")

    force_parts = 0
    prefetch_depth = 0
    workgroup_waves = 0
    merge_mode = 0
    partition_mode = 0
    separate_write = False

    def step(self, l, ev=None, ev_index=None):
        mq = self.max_q_len if self.cu is not None else 0
        if self.separate_write:
            pa.kv_quant_write(self.step_k, self.step_v, self.step_slots[l], self.kcl[l], self.vcl[l],
                              self.ksl[l], self.vsl[l], self.mode)
        sp = self.sp
        if self.index_topk:
            if ev_index is not None:
                ev_index[0].record()
            pa.pa_index_topk(self.q_idx, self.icl[l], self.bt[l], self.ctx, self.cu, self.lists[l],
                             self.scores[l], max_q_len=mq)
            if ev_index is not None:
                ev_index[1].record()
            sp = self.lists[l]
        if not self.separate_write:
            # one decode step through pa_decode_write: the new tokens are
            # written inside the decode launch where the library can (the
            # indexer reads only the index cache, so it may run first)
            pa.pa_decode_write(self.q[l], self.step_k, self.step_v, self.step_slots[l], self.kcl[l],
                               self.vcl[l], self.ksl[l], self.vsl[l], self.bt[l], self.ctx, self.cu, self.mode,
                               self.out[l], max_q_len=mq, force_parts=self.force_parts,
                               prefetch_depth=self.prefetch_depth, workgroup_waves=self.workgroup_waves,
                               merge_mode=self.merge_mode, partition_mode=self.partition_mode,
                               sparse_page_idx=sp,
                               main_begin_event=None if ev is None else ev[0],
                               main_end_event=None if ev is None else ev[1])
            return
        pa.pa_decode_ex(self.q[l], self.kcl[l], self.vcl[l], self.ksl[l], self.vsl[l], self.bt[l], self.ctx,
                        self.cu, sp, self.mode, self.out[l],
                        max_q_len=self.max_q_len if self.cu is not None else 0,
                        force_parts=self.force_parts, prefetch_depth=self.prefetch_depth,
                        workgroup_waves=self.workgroup_waves, merge_mode=self.merge_mode,
                        partition_mode=self.partition_mode,
                        main_begin_event=None if ev is None else ev[0],
                        main_end_event=None if ev is None else ev[1])


def algorithmic_flops(w):
    """Flops one decode call must do: for every (query row, query head,
    attended token) a 128-wide dot product for the score and a 128-wide
    multiply-add of V (2 flops per multiply-add each)."""
    rs = w.row_start
    pairs = 0
    for b in range(w.B):
        L, c = int(w.q_lens[b]), min(int(w.ctx[b]), w.W * 128)
        for i in range(L):
            lim = max(0, min(int(w.ctx[b]) - L + i + 1, c))
            if w.sparse is None:
                pairs += lim
            else:
                sel = {int(x) for x in w.sparse[rs[b] + i] if 0 <= x < w.W}
                pairs += sum(max(0, min(128, lim - 128 * x)) for x in sel)
    return pairs * w.Hq * 128 * 4


def index_bytes(w, topk):
    """Bytes one pa_index_topk call must move: the index keys of every
    visible page once per request (the rows of a request share each read),
    the index queries, the score matrix written and read back, the lists
    written, and the block-table entries."""
    pages = sum(min((int(c) + 127) // 128, w.W) for c in w.ctx)
    return pages * 128 * 128 + w.rows * 128 * 2 + 2 * w.rows * w.W * 4 + w.rows * topk * 4 + 4 * pages


def algorithmic_bytes(w):
    """Bytes one decode call must move: attended KV (codes + per-token
    scales), q, out, the block-table entries and per-request metadata."""
    kv = w.kv_bytes_attended()
    qo = 2 * w.rows * w.Hq * 128 * 2
    pages = sum(int(math.ceil(min(int(c), w.W * 128) / 128)) for c in w.ctx) if w.sparse is None \
        else w.sparse.size
    meta = 4 * pages + 4 * w.B + (0 if w.cu is None else 4 * (w.B + 1)) + \
        (0 if w.sparse is None else 4 * w.sparse.size)
    return kv, kv + qo + meta


# the sources whose code a main kernel's traffic depends on (its kernel
# file, the shared device code, the argument block and the planner)
_SHARED_SOURCES = ("fp8_paged_kv_pa_amd/csrc/device_common.h", "fp8_paged_kv_pa_amd/csrc/launch.h",
                   "fp8_paged_kv_pa_amd/csrc/plan.cpp", "fp8_paged_kv_pa_amd/csrc/plan.h")
KERNEL_SOURCES = {
    "pa_decode_main": ("fp8_paged_kv_pa_amd/csrc/pa_decode.hip",
                       "fp8_paged_kv_pa_amd/csrc/writer_common.h") + _SHARED_SOURCES,
    "pa_prefill_main": ("fp8_paged_kv_pa_amd/csrc/pa_prefill.hip",) + _SHARED_SOURCES,
}


def sources_sha256(kernel):
    """SHA-256 over the sources of a main kernel (KERNEL_SOURCES)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def write_in_decode(w, separate_write, index_topk):
    """Whether a step's cache write runs inside the decode launch: calls
    through pa_decode_write with at most PA_FUSED_WRITE_MAX_Q_LEN rows per
    request (16), one row per request when block-sparse, and the default
    two-page ring."""
    sparse = w.sparse is not None or bool(index_topk)
    return (not separate_write and int(w.q_lens.max()) <= 16
            and (not sparse or int(w.q_lens.max()) == 1))


def recorded_traffic(workload):
    """HBM bytes per main-kernel launch from the committed counter record
    (profiles/pa_decode_main_traffic.json), or None when the workload has no
    record or its kernel's sources no longer hash to the recorded digest."""
    path = os.path.join(ROOT, "profiles", "pa_decode_main_traffic.json")
    if not os.path.exists(path):
        return None
    w = json.load(open(path)).get("workloads", {}).get(workload)
    if w is None or w.get("kernel") not in KERNEL_SOURCES or sources_sha256(w["kernel"]) != w.get("source_sha256"):
        return None
    return int(w["traffic_bytes_per_launch"])


def _events(n):
    """n pairs of timing events, each recorded once so that the underlying
    HIP events exist before a probe's dispatch records them."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    return evs


def hbm_probe(dev, gib=4, same_bytes=None):
    """Best streaming-read rate (GB/s) of a plain 16-byte-per-lane read
    kernel over a 4 GiB buffer, for a few grid sizes; with `same_bytes`, also
    the best rate for reads of that size (rotating through the buffer so
    they come from HBM), the floor a kernel moving that many bytes meets.
    Every launch is timed by dispatch-recorded events, as the main kernel."""
    import ctypes
    path = os.path.join(ROOT, "fp8_paged_kv_pa_amd", "libhbmprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    best = 0.0
    stream = torch.cuda.current_stream()
    for blocks in (256, 512, 1024, 2048, 4096):
        sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        for rep in range(4):
            e0, e1 = _events(1)[0]
            rc = lib.hbm_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, e0.cuda_event, e1.cuda_event,
                                    stream.cuda_stream)
            torch.cuda.synchronize()
            if rc != 0:
                return None
            if rep:
                best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    best_small = None
    if same_bytes:
        nb = (int(same_bytes) + 15) // 16 * 16
        slots = max(1, nbytes // nb)
        best_small = 0.0
        for blocks in (256, 512, 1024):
            sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
            evs = _events(24)
            torch.cuda._sleep(int(5e7))
            for i, (e0, e1) in enumerate(evs):
                if lib.hbm_read_probe(buf.data_ptr() + (i % slots) * nb, nb, sink.data_ptr(), blocks,
                                      e0.cuda_event, e1.cuda_event, stream.cuda_stream) != 0:
                    return None
            torch.cuda.synchronize()
            ts = sorted(a.elapsed_time(b) for a, b in evs[4:])
            best_small = max(best_small, nb / (ts[len(ts) // 2] * 1e-3) / 1e9)
        best_small = round(best_small, 1)
    del buf
    torch.cuda.empty_cache()
    return round(best, 1), best_small


def launch_floor(dev, grid=256, threads=256):
    """Median dispatch-recorded duration (us) of the probe library's empty
    kernel at the main kernel's usual grid: what any launch costs here,
    timed the way the main kernel is."""
    import ctypes
    path = os.path.join(ROOT, "fp8_paged_kv_pa_amd", "libhbmprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.launch_floor_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    sink = torch.zeros(grid, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    evs = _events(72)
    torch.cuda._sleep(int(2e7))
    for e0, e1 in evs:
        if lib.launch_floor_probe(flag.data_ptr(), sink.data_ptr(), grid, threads, e0.cuda_event, e1.cuda_event,
                                  stream.cuda_stream) != 0:
            return None
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs[8:])
    return round(ts[len(ts) // 2], 3)


def start_spread(dev, blocks, lds_bytes, reps=9):
    """Median over `reps` launches of the spread (us) of the workgroups'
    entry times (s_memrealtime, 100 MHz) in the probe library's start
    kernel: `blocks` workgroups of 256 threads, `lds_bytes` of LDS each."""
    import ctypes
    path = os.path.join(ROOT, "fp8_paged_kv_pa_amd", "libhbmprobe.so")
    lib = ctypes.CDLL(path)
    lib.start_spread_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    ticks = torch.zeros(blocks, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    spreads = []
    for rep in range(reps + 1):  # the first launch warms up
        if lib.start_spread_probe(ticks.data_ptr(), blocks, 256, lds_bytes, stream.cuda_stream):
            raise RuntimeError("start_spread_probe failed")
        torch.cuda.synchronize()
        t = ticks.cpu().numpy()
        if rep:
            spreads.append(float(t.max() - t.min()) * 0.01)
    return round(float(np.median(spreads)), 2)


ISSUE_KINDS = (("mfma_f32_16x16x32_bf16", 8), ("fmac_f32", 32), ("cvt_scalef32_pk_bf16_fp8", 16), ("exp_f32", 32))


def issue_probe(dev, iters=4096):
    """Per instruction kind the decode issues and for one and two waves per
    SIMD: shader-clock cycles (s_memtime) per wave64 instruction and SIMD,
    independent instructions -- the median over the waves of the probe
    library's instruction-rate kernel, divided by the waves per SIMD -- and
    the clock (GHz) they ran at, from the 100 MHz s_memrealtime count of the
    same interval.  Also whether every workgroup's waves sat evenly on its
    CU's four SIMDs."""
    import ctypes
    path = os.path.join(ROOT, "fp8_paged_kv_pa_amd", "libhbmprobe.so")
    lib = ctypes.CDLL(path)
    lib.issue_rate_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_void_p]
    blocks = 256
    stream = torch.cuda.current_stream()
    res = {}
    for wps in (1, 2):
        waves = 4 * wps
        rec = torch.zeros(blocks * waves * 3, dtype=torch.int64, device=dev)
        sink = torch.zeros(blocks * 64 * waves, dtype=torch.float32, device=dev)
        cyc, ghz, even = {}, {}, True
        for kind, (name, per_round) in enumerate(ISSUE_KINDS):
            for rep in range(2):  # the first run warms up
                if lib.issue_rate_probe(kind, iters, wps, rec.data_ptr(), sink.data_ptr(), blocks,
                                        stream.cuda_stream):
                    raise RuntimeError("issue_rate_probe failed")
                torch.cuda.synchronize()
            r = rec.view(blocks, waves, 3).cpu().numpy()
            c = np.sort(r[:, :, 0].reshape(-1))
            f = np.sort((r[:, :, 0] / np.maximum(r[:, :, 1], 1) * 0.1).reshape(-1))
            cyc[name] = round(float(c[len(c) // 2]) / (iters * per_round * wps), 2)
            ghz[name] = round(float(f[len(f) // 2]), 3)
            even = even and all(sorted(np.bincount(r[b, :, 2], minlength=4).tolist()) == [wps] * 4
                                for b in range(blocks))
        res[f"{wps}_wave_per_simd"] = {"cycles_per_instruction": cyc, "clock_ghz": ghz, "waves_even": bool(even)}
    # one MFMA wave and one fma wave (four times the rounds) on each SIMD: each
    # wave's cycles per own instruction; alone they would be the one-wave figures
    waves = 8
    rec = torch.zeros(blocks * waves * 3, dtype=torch.int64, device=dev)
    sink = torch.zeros(blocks * 64 * waves, dtype=torch.float32, device=dev)
    for rep in range(2):
        if lib.issue_rate_probe(4, iters, 2, rec.data_ptr(), sink.data_ptr(), blocks, stream.cuda_stream):
            raise RuntimeError("issue_rate_probe failed")
        torch.cuda.synchronize()
    r = rec.view(blocks, waves, 3).cpu().numpy()
    paired = bool(np.array_equal(np.sort(r[:, :4, 2], axis=1), np.tile(np.arange(4), (blocks, 1)))
                  and np.array_equal(np.sort(r[:, 4:, 2], axis=1), np.tile(np.arange(4), (blocks, 1))))
    mf = float(np.median(r[:, :4, 0])) / (iters * ISSUE_KINDS[0][1])
    fm = float(np.median(r[:, 4:, 0])) / (iters * 4 * ISSUE_KINDS[1][1])
    res["mfma_wave_beside_fmac_wave"] = {"mfma_cycles": round(mf, 2), "fmac_cycles": round(fm, 2),
                                         "one_of_each_per_simd": paired}
    return res


def block_probe(layers, w):
    """Best rate (GB/s) of the bench probe library's block-read kernel over
    exactly the (page, head) blocks one decode call reads -- every request's
    attended pages of layer l, K and V (and their scale pieces in per-token
    mode) -- with non-temporal 16-byte loads and no arithmetic, up to 256
    workgroups, rotating over the layers as the bench's steps do; and, in
    per-token mode, the same over the K/V blocks alone; each launch timed by
    dispatch-recorded events, as the main kernel.  FP8 caches only; None
    otherwise."""
    import ctypes
    path = os.path.join(ROOT, "fp8_paged_kv_pa_amd", "libhbmprobe.so")
    if not os.path.exists(path) or w.kv_dtype == "bf16":
        return None
    lib = ctypes.CDLL(path)
    lib.hbm_block_probe.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4
    ids = []
    for b in range(w.B):
        if w.sparse is None:
            pages = range(min((int(w.ctx[b]) + 127) // 128, w.W))
        else:
            start, L = int(w.row_start[b]), int(w.q_lens[b])
            pages = sorted({int(x) for r in range(start, start + L) for x in w.sparse[r] if 0 <= x < w.W})
        for n in pages:
            P = int(w.block_table[b, n])
            ids += [P * w.Hkv + h for h in range(w.Hkv)]
    nblk = w.num_blocks * w.Hkv
    assert ids and all(0 <= i < nblk for i in ids)
    # at most 256 workgroups, as few entries each as that allows, and only as
    # many workgroups as the entries fill (a small call must not be padded
    # with repeated blocks, which would count cache hits as traffic)
    per_wg = (len(ids) + 255) // 256
    wgs = (len(ids) + per_wg - 1) // per_wg
    tab = np.resize(np.asarray(ids, np.int32), per_wg * wgs)  # pads fewer than per_wg entries
    dev = layers.q[0].device
    table = torch.from_numpy(tab).to(dev)
    sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def rate(scales):
        nbytes = len(tab) * (2 * 16384 + (2 * 512 if scales else 0))
        best = 0.0
        for rnd in range(3):
            evs = _events(16)
            torch.cuda._sleep(int(5e7))
            for i, (e0, e1) in enumerate(evs):
                l = i % layers.n
                rc = lib.hbm_block_probe(layers.kcl[l].data_ptr(), layers.vcl[l].data_ptr(),
                                         layers.ksl[l].data_ptr() if scales else None,
                                         layers.vsl[l].data_ptr() if scales else None,
                                         table.data_ptr(), per_wg, wgs, sink.data_ptr(), e0.cuda_event,
                                         e1.cuda_event, stream.cuda_stream)
                if rc != 0:
                    return None
            torch.cuda.synchronize()
            ts = sorted(a.elapsed_time(b) for a, b in evs[2:])
            best = max(best, nbytes / (ts[len(ts) // 2] * 1e-3) / 1e9)
        return round(best, 1)

    # with the scale pieces when the call reads them, and the K/V blocks alone
    pt = w.mode == wl.PER_TOKEN
    return rate(pt), (rate(False) if pt else None)


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_workers():
    """Worker processes for the oracle leg: the CPUs this process may run
    on, at most 16 (one GPU's share of a shared 8-GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_worker(w, reqs, index_topk, budget_s, go, barrier, results, wid):
    """One worker of the oracle leg, in a process forked before the parent
    touched the GPU: build the oracle's cache of each of its requests
    (untimed: it is state, as the GPU cache is), wait until every worker is
    ready, then repeat request-steps -- write the request's new tokens,
    (with the indexer: score its visible pages and take the top-k,) attend
    its rows over its cache -- until about `budget_s` seconds of work.
    Single-threaded numpy (BLAS limited to one thread)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    from oracle import attention as oatt
    from oracle import indexer as oidx
    from oracle import writer as owr
    try:
        go.wait()
        sk, sv, _ = w.step_tokens()
        sc_k = np.array([w.k_scalar], np.float32)
        sc_v = np.array([w.v_scalar], np.float32)
        bf = w.kv_dtype == "bf16"

        def write(k, v, slots, kc, vc, ka, va):
            if bf:
                owr.write_bf16_ref(k, v, slots, kc, vc, w.Hkv)
            else:
                owr.quant_write_ref(k, v, slots, kc, vc, ka, va, w.mode, w.Hkv)

        def request_state(b):
            pages = [int(x) for x in w.written[b]]
            nb = len(pages) + 1
            kc = np.zeros(nb * w.Hkv * 16384, np.uint16 if bf else np.uint8)
            vc = np.zeros_like(kc)
            ks = np.zeros(nb * w.Hkv * 128, np.float32)
            vs = np.zeros_like(ks)
            ka, va = (sc_k, sc_v) if w.mode == wl.SCALAR else ((ks, vs) if w.mode == wl.PER_TOKEN else (None, None))
            bt = np.full((1, w.W), -1, np.int64)
            for ci, pg in enumerate(pages):
                bt[0, pg] = ci
                k, v = w.page_kv(b, pg)
                write(k, v, ci * 128 + np.arange(k.shape[0], dtype=np.int64), kc, vc, ka, va)
            L = int(w.q_lens[b])
            c = int(w.ctx[b])
            new_slots = np.array([bt[0, (c - L + i) // 128] * 128 + (c - L + i) % 128 for i in range(L)],
                                 dtype=np.int64)
            icache = None
            if index_topk:
                pm = {(b, pg): ci for ci, pg in enumerate(pages)}
                icache = w.index_cache(poison=False, num_blocks=nb, page_map=pm)
            return kc, vc, ka, va, bt, new_slots, icache

        state = {b: request_state(b) for b in reqs}
        q_idx = w.index_queries() if index_topk else None
        barrier.wait()
        done_bytes, t_used, n, checks = 0, 0.0, 0, []
        while (t_used < budget_s and n < 4096) or n < len(reqs):
            b = reqs[n % len(reqs)]
            kc, vc, ka, va, bt, new_slots, icache = state[b]
            start, L = int(w.row_start[b]), int(w.q_lens[b])
            rows = list(range(start, start + L))
            sp = None if w.sparse is None else w.sparse[start:start + L]
            cu = None if w.cu is None else np.array([0, L])
            t0 = time.perf_counter()
            write(sk[start:start + L], sv[start:start + L], new_slots, kc, vc, ka, va)
            if index_topk:
                sc = oidx.block_scores_ref(q_idx[start:start + L], icache, bt, w.ctx[b:b + 1], cu)
                sp = oidx.topk_ref(sc, index_topk)
            ref = oatt.attention_ref(w.q[start:start + L], kc, vc, ka, va, bt, w.ctx[b:b + 1], cu, sp,
                                     w.mode, w.Hkv, kv_dtype=w.kv_dtype)
            t_used += time.perf_counter() - t0
            if n < len(reqs):
                checks.append((b, rows, ref, sp))
            if w.sparse is None and not index_topk:
                toks = min(int(w.ctx[b]), w.W * 128)
            else:
                sel = {int(x) for r in range(L) for x in sp[r] if 0 <= x < w.W}
                toks = sum(min(128, int(w.ctx[b]) - 128 * x) for x in sel)
            done_bytes += toks * w.Hkv * (512 if bf else 256 + (8 if w.mode == wl.PER_TOKEN else 0))
            if index_topk:
                done_bytes += min((int(w.ctx[b]) + 127) // 128, w.W) * 128 * 128
            n += 1
        results.put((wid, done_bytes, t_used, n, checks, None))
    except BaseException as e:  # report, never hang the parent
        import traceback
        results.put((wid, 0, 0.0, 0, [], traceback.format_exc() + repr(e)))


class OracleLeg:
    """The oracle timed on the host's cores: one single-threaded worker
    process per core (at most 16), forked before the parent initialises the
    GPU, each holding one or more requests of the workload.  `run()` releases
    them once the GPU measurement is done."""

    def __init__(self, w, index_topk=0, budget_s=12.0):
        import multiprocessing as mp
        ctx = mp.get_context("fork")
        self.w, self.index_topk, self.budget_s = w, index_topk, budget_s
        self.n = cpu_workers()
        self.go = ctx.Event()
        self.barrier = ctx.Barrier(self.n)
        self.results = ctx.Queue()
        nreq = min(w.B, self.n)
        self.reqs = [[i % nreq] for i in range(self.n)]
        self.procs = [ctx.Process(target=_oracle_worker, daemon=True,
                                  args=(w, self.reqs[i], index_topk, budget_s, self.go, self.barrier,
                                        self.results, i))
                      for i in range(self.n)]
        for p in self.procs:
            p.start()

    def stop(self):
        for p in self.procs:
            if p.is_alive():
                p.kill()

    def run(self, layers):
        """Release the workers, collect their request-steps, check the GPU's
        layer-0 output (and, with the indexer, its page lists) on the rows
        the oracle computed, and return the cpu_baseline record."""
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from harness import compare
        w, index_topk = self.w, self.index_topk
        out0 = layers.out[0].float().cpu().numpy()
        gpu_lists = layers.lists[0].cpu().numpy() if index_topk else None
        t0 = time.perf_counter()
        self.go.set()
        got = []
        for _ in range(self.n):
            got.append(self.results.get(timeout=600))
        wall = time.perf_counter() - t0
        for p in self.procs:
            p.join(timeout=30)
        errs = [r[5] for r in got if r[5]]
        if errs:
            raise RuntimeError("oracle worker failed:\n" + errs[0])
        done_bytes = sum(r[1] for r in got)
        t_max = max(r[2] for r in got)
        steps = sum(r[3] for r in got)
        check, lists_equal, checked = None, True, set()
        for r in got:
            for b, rows, ref, sp in r[4]:
                if b in checked:
                    continue
                checked.add(b)
                if index_topk:
                    same = bool(np.array_equal(sp, gpu_lists[rows[0]:rows[-1] + 1]))
                    lists_equal &= same
                    if not same:
                        continue
                err, cos = compare(out0[rows], ref, what=f"bench check request {b}")
                check = (err, cos) if check is None else (max(err, check[0]), min(cos, check[1]))
        nreq = len({b for r in self.reqs for b in r})
        return {
            "value": round(done_bytes / t_max / 1e9, 5),
            "unit": "GB/s",
            "cores": self.n,
            "kind": "oracle",
            "sample": f"{steps} request-steps over the first {nreq} requests of {w.name} on {self.n} "
                      f"single-threaded worker processes running together (each: write the request's new "
                      f"tokens, "
                      + (f"score its visible pages on the index cache and take the top-{index_topk}, "
                         if index_topk else "")
                      + f"decode its attended pages, fp64 softmax attention for its rows), about "
                      f"{self.budget_s:.0f} s of work each; value = KV bytes of all steps / the longest "
                      f"worker's timed seconds ({t_max:.1f} s)",
            "cpu_model": cpu_model(),
            "host_cpus_visible": os.cpu_count(),
            "wall_s": round(wall, 1),
            "check_max_abs_err": None if check is None else round(check[0], 6),
            **({"check_index_lists_equal": lists_equal} if index_topk else {}),
            "check_min_cos": None if check is None else round(check[1], 8),
            "check_requests": sorted(checked),
        }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3200)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--config", default="c3", choices=sorted(CONFIGS))
    ap.add_argument("--layers", type=int, default=0, help="distinct cache copies to rotate (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--force-parts", type=int, default=0, help="split-K partitions (0: the plan's choice)")
    ap.add_argument("--prefetch-depth", type=int, default=0, help="pages in flight per wave (0: the plan's)")
    ap.add_argument("--workgroup-waves", type=int, default=0, help="4 or 8 waves per workgroup (0: the plan's)")
    ap.add_argument("--merge-mode", type=int, default=0,
                    help="split-K merge: 0 the plan's, 1 separate kernel, 2 in the main kernel")
    ap.add_argument("--partition-mode", type=int, default=0,
                    help="split-K partitions: 0 the plan's, 1 fixed, 2 length-balanced")
    ap.add_argument("--separate-write", action="store_true",
                    help="write the step's new tokens with kv_quant_write, then decode (two launches)")
    ap.add_argument("--issue-probe", action="store_true",
                    help="print the cycles per wave64 instruction of the kinds the decode issues and the empty-launch floor, then exit")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB copy kernel (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the library has no "
              f"multi-GPU path; the decode kernel's per-GPU share is what one GPU shows).", file=sys.stderr)
        sys.exit(2)
    if args.issue_probe:
        assert torch.cuda.is_available(), "the probe needs a GPU"
        dev = torch.device("cuda:0")
        print(json.dumps({"issue_probe": issue_probe(dev),
                          "launch_floor_us_by_grid": {g: launch_floor(dev, grid=g) for g in (1, 256, 1984)},
                          "start_spread_us": {f"{g}x{lds // 1024}KiB": start_spread(dev, g, lds)
                                              for g in (144, 1152) for lds in (0, 34 * 1024)},
                          "note": "s_memtime cycles per wave64 instruction and SIMD with one and two waves per "
                                  "SIMD, independent instructions, and the clock they ran at (probe library "
                                  "issue_rate_probe); "
                                  "median dispatch-recorded duration of an empty 256-thread kernel per grid "
                                  "size (launch_floor_probe); spread of workgroup entry times per grid and "
                                  "LDS size (start_spread_probe)"}))
        return
    w = CONFIGS[args.config]()
    index_topk = INDEX_TOPK.get(args.config, 0)
    idx_bytes = index_bytes(w, index_topk) if index_topk else 0
    if index_topk:
        # the decode attends the indexer's lists: size its bytes for full pages
        # now, recomputed from the lists the indexer produced after warmup
        w.sparse = np.zeros((w.rows, index_topk), np.int32)
    kv_bytes, alg_bytes = algorithmic_bytes(w)
    n_layers = args.layers or max(1, min(64, int(math.ceil(1.0e9 / max(alg_bytes + idx_bytes, 1)))))
    if index_topk:
        w.sparse = None
    # the oracle's workers are forked now, before this process touches the
    # GPU; they wait until the GPU measurement is over
    leg = None if args.no_cpu_baseline else OracleLeg(w, index_topk)

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = Layers(w, n_layers, dev, index_topk)

    stream = torch.cuda.Stream()
    cfg = pa.make_config(w.Hkv, w.rows, w.B, w.W,
                         topk=index_topk or (0 if w.sparse is None else w.sparse.shape[1]),
                         ragged=w.cu is not None, max_q_len=int(w.q_lens.max()) if w.cu is not None else 0,
                         scale_mode=w.mode, force_parts=args.force_parts,
                         kv_dtype=3 if w.kv_dtype == "bf16" else 1, merge_mode=args.merge_mode,
                         partition_mode=args.partition_mode)
    layers.force_parts = args.force_parts
    layers.prefetch_depth = args.prefetch_depth
    layers.workgroup_waves = args.workgroup_waves
    layers.merge_mode = args.merge_mode
    layers.partition_mode = args.partition_mode
    layers.separate_write = args.separate_write
    plan = pa.pa_plan_describe(cfg)
    pa.pa_reserve(cfg, stream)

    K, W = args.steps, args.warmup
    G = min(n_layers, max(1, K))
    with torch.cuda.stream(stream):
        for i in range(max(W, n_layers)):   # warm up eagerly (also first-touch)
            layers.step(i % n_layers)
    torch.cuda.synchronize()
    if index_topk:
        # the pages the decode attends are the ones the indexer chose
        w.sparse = layers.lists[0].cpu().numpy()
        kv_bytes, alg_bytes = algorithmic_bytes(w)

    # one graph per G consecutive steps (layers 0..G-1)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for l in range(G):
            layers.step(l)
    tail = K % G
    tail_graph = None
    if tail:
        tail_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(tail_graph, stream=stream):
            for l in range(tail):
                layers.step(l)
    torch.cuda.synchronize()
    for _ in range(max(1, W // G)):
        graph.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps --------------------------------
    reps = K // G
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    if tail_graph is not None:
        tail_graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    # ---- live duration of the main decode kernel --------------------------
    # Eager steps queued behind a spin kernel, so the stream runs them back to
    # back; the library records a HIP event pair around every main-kernel
    # launch on the launch stream.
    n_ev = min(max(K, 1), max(4 * n_layers, 32), 512)
    evs2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_ev)]
    evs_idx = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_ev)] if index_topk else [None] * n_ev
    with torch.cuda.stream(stream):
        for a, b in evs2:
            a.record()
            b.record()
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2e8))
        for i, ev in enumerate(evs2):
            layers.step(i % n_layers, ev, evs_idx[i])
    torch.cuda.synchronize()
    main_ms = [a.elapsed_time(b) for a, b in evs2]
    timing = (f"HIP events recorded around each main-kernel launch on the launch stream, {n_ev} "
              f"steps queued behind a spin kernel")
    main_avg_ms = float(np.mean(main_ms))
    achieved = alg_bytes / (main_avg_ms * 1e-3) / 1e9
    mfma_bound = args.config in MFMA_BOUND
    flops = algorithmic_flops(w) if mfma_bound else 0
    value = (kv_bytes + idx_bytes) / (ms_per_step * 1e-3) / 1e9
    index_avg_ms = float(np.mean([a.elapsed_time(b) for a, b in evs_idx])) if index_topk else None
    tokens_per_s = w.attended_tokens() * w.Hkv / (ms_per_step * 1e-3)

    # ---- one cold launch: an idle GPU, and caches evicted by a 1 GiB fill
    # first; the main kernel's own time from its dispatch events, and the
    # host's wall time for the whole step from submission to completion
    cev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    with torch.cuda.stream(stream):
        cev[0].record()
        cev[1].record()
    flush = torch.empty(256 << 20, dtype=torch.float32, device=dev)
    flush.fill_(1.0)
    torch.cuda.synchronize()
    del flush
    c0 = time.perf_counter()
    with torch.cuda.stream(stream):
        layers.step(0, cev)
    torch.cuda.synchronize()
    cold_wall_us = (time.perf_counter() - c0) * 1e6
    cold_main_us = cev[0].elapsed_time(cev[1]) * 1e3

    if args.calib_copy:
        x = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        for _ in range(5):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()

    probe, probe_same = hbm_probe(dev, same_bytes=idx_bytes if index_topk else alg_bytes) or (None, None)
    probe_blocks, probe_blocks_kv = (None, None) if index_topk else (block_probe(layers, w) or (None, None))
    floor_us = launch_floor(dev)
    try:
        cpu = None if leg is None else leg.run(layers)
    finally:
        if leg is not None:
            leg.stop()

    res = {
        "metric": "decode attention KV GB/s & % HBM roofline (attended tokens/s), 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if w.kv_dtype == "bf16" else "fp8e4m3") + "-kv/bf16-mfma/f32-acc",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.B, "q_len": int(w.q_lens.max()), "rows": w.rows, "kv_heads": w.Hkv,
            "q_heads_per_kv": 16, "head_dim": 128, "page": 128,
            "context": [int(w.ctx.min()), int(w.ctx.max())],
            "kv_dtype": w.kv_dtype,
            "scale_mode": ["none", "scalar", "per_token"][w.mode],
            "sparse_topk": 0 if w.sparse is None else int(w.sparse.shape[1]),
            "write": "in_decode" if write_in_decode(w, args.separate_write, index_topk) and args.prefetch_depth <= 2
                     else "separate",
            "layers_rotated": n_layers,
            "kv_bytes_per_step": int(kv_bytes),
            "plan": {k: int(v) for k, v in plan.items() if k in ("parts", "pages_per_part", "grid_x",
                                                                  "rows_per_group", "merge",
                                                                  "merge_in_kernel", "balanced")},
        },
        "attended_tokens_per_s": round(tokens_per_s, 1),
        "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_prefill_main" if plan["rows_per_group"] == PREFILL_POSITIONS else "pa_decode_main",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(w.name),
            "avg_launch_us": round(main_avg_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": int(alg_bytes),
            "timing": timing,
            "hbm_read_probe_gbs": probe,
            "frac_of_probe": None if not probe else round(achieved / probe, 4),
            "hbm_read_probe_same_bytes_gbs": probe_same,
            "frac_of_same_bytes_probe": None if not probe_same else round(achieved / probe_same, 4),
            "launch_floor_us": floor_us,
            "block_read_probe_gbs": probe_blocks,
            "block_read_probe_kv_only_gbs": probe_blocks_kv,
            "frac_of_block_probe": None if not probe_blocks else round(achieved / probe_blocks, 4),
        },
        "cpu_baseline": cpu,
        "cold_launch": {
            "main_kernel_us": round(cold_main_us, 3),
            "step_wall_us": round(cold_wall_us, 1),
            "note": "one eager step on an idle GPU after a 1 GiB fill evicted the caches: the main "
                    "kernel's dispatch-recorded events, and host wall time from submission to completion",
        },
    }
    if mfma_bound:
        # q_len 16384 over a 16384-token context: ~8000 flop per byte moved,
        # far above the bf16 ridge (~312 flop/B), so the roofline is the MFMA one
        tf = flops / (main_avg_ms * 1e-3) / 1e12
        res["decode_main_hbm"] = {k: res["roofline"][k] for k in ("achieved", "frac", "algorithmic_bytes_per_launch")}
        res["roofline"].update({
            "bound": "mfma",
            "achieved": round(tf, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_launch": int(flops),
            "dtype_note": "bf16 MFMA peak (dense); the kernel runs P.V as a bf16 hi + lo pair, "
                          "1.5x the algorithmic MFMA work",
        })
    if index_topk:
        # the indexer reads 16x the decode's bytes here: it is the dominant kernel
        ia = idx_bytes / (index_avg_ms * 1e-3) / 1e9
        res["config"]["index_topk"] = index_topk
        res["config"]["index_bytes_per_step"] = int(idx_bytes)
        res["decode_main"] = {k: res["roofline"][k] for k in ("achieved", "frac", "avg_launch_us",
                                                               "algorithmic_bytes_per_launch")}
        res["roofline"].update({
            "kernel": "pa_index_topk (index_score_kernel + index_topk_kernel)",
            "achieved": round(ia, 1),
            "frac": round(ia / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_launch_us": round(index_avg_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": int(idx_bytes),
            "timing": f"torch events on the launch stream around each pa_index_topk call, {n_ev} steps "
                      f"queued behind a spin kernel",
            "frac_of_probe": None if not probe else round(ia / probe, 4),
            "frac_of_same_bytes_probe": None if not probe_same else round(ia / probe_same, 4),
        })
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
