#!/usr/bin/env python3
"""Benchmark of the batched speculative-sampling verify step on one MI355X.

One step = the whole hot path over one batch resident in HBM: the counter-based
uniforms and the verify (pass 1 row streaming; pass 2 resolve and categorical draws), by
spec_verify_philox (the uniforms come from the first workgroups of pass 1; with
--separate-uniforms: sv_fill_uniforms, then spec_verify).  Default workload: B=256
sequences, K=8 drafted tokens, V=152064 bf16 logits, Zipf(1.1)-offset target logits,
T ~ U[0, 1.2] with a quarter of the sequences greedy (T = 0).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 100] [--warmup 40] [--min-warmup-ms 200]
                    [--workload 1-5] [--no-cpu-baseline]
                    [--path verify|greedy|ragged|sample|tree]

Warm-up: at least --warmup steps and at least --min-warmup-ms of back-to-back steps.
From idle, the first ~25 ms of sustained load on an MI355X run at shifting clocks (the
step time first dips, then rises by up to a quarter, then settles), so a short warm-up
measures the transient; the JSON line reports the warm-up actually run.

--path greedy: spec_verify_greedy on the same target rows, every sequence greedy (argmax
rule, no draft rows read); --path ragged: spec_verify_ragged on the same rows with K_b
uniform on 1..K per sequence (packed layout); --path sample: sv_sample on the B draft
rows of position 0 (one draw per row from softmax(z / T)); --path tree:
spec_verify_tree_greedy on 64 draft trees of 64 nodes (V=152064 bf16).  Each prints the
same JSON contract for its own workload.

The CPU leg (cpu_baseline) times the fp64 oracle on the timed batches and compares its
results with the GPU's (the parity object: draws, near-ties, hard mismatches).
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published peak
COPY_BYTES = 1 << 30    # size of the calibration copy (--copy-calibration)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pass1_kernel_traffic_workload4.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("sv_pass1.hip", "sv_device.h", "sv_common.h"):
        with open(os.path.join(ROOT, "speculative_decoding_verification_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per pass-1 launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    if workload != 4 or not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def needed_rows(temperature, accept_len, status, K):
    """Logit rows the verify rule needs for one batch: the positions up to each sequence's
    first rejection n (target and draft rows 0..n of a sampled sequence, K+1 target and K
    draft rows if all K drafts are accepted; target rows 0..n of a greedy one).  A sequence
    with a data error counts with every row."""
    import numpy as np
    T = np.asarray(temperature)
    n = np.asarray(accept_len).astype(np.int64)
    err = (np.asarray(status) & ~16) != 0
    sampled = T != 0
    full = K + 1 + np.where(sampled, K, 0)
    rows = np.where(sampled, np.where(n == K, 2 * K + 1, 2 * (n + 1)), n + 1)
    return int(np.where(err, full, rows).sum())


def drawn_rows(temperature, accept_len, status, K):
    """Rows pass 2 reads for one batch: the target and draft rows at the rejection of each
    sampled sequence that rejected a draft, the target row K of each that accepted all;
    none for greedy sequences or sequences with a data error."""
    import numpy as np
    T = np.asarray(temperature)
    n = np.asarray(accept_len)
    ok = (T != 0) & ((np.asarray(status) & ~16) == 0)
    return int(((ok & (n < K)) * 2 + (ok & (n == K)) * 1).sum())


def host_logits(x):
    import numpy as np
    import torch
    x = x.detach().cpu()
    return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()


def to_host(out):
    return {k: (None if v is None else v.detach().cpu().numpy()) for k, v in out.items()}


def host_info():
    """The host the CPU leg runs on: CPU model, counts, and the share of it this process
    may use (OMP_NUM_THREADS when set, else the smaller of the affinity mask and the
    cgroup's CPU quota)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    quota = None
    try:
        a, b = open("/sys/fs/cgroup/cpu.max").read().split()
        if a != "max":
            quota = int(a) / int(b)
    except (OSError, ValueError):
        pass
    try:
        omp = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        omp = 0
    share = omp if omp > 0 else min(affinity, math.ceil(quota) if quota else affinity)
    return dict(cpu_model=model, nproc=os.cpu_count(), affinity=affinity, cgroup_cpus=quota,
                omp_num_threads=omp or None, share=max(1, min(share, affinity)))


# --------------------------------------------------------------------------------------
# CPU leg: the oracle on the timed batches, and the parity of the GPU results with it
# --------------------------------------------------------------------------------------

def _orc_arrays(results, B, K):
    """verify_sequence results {b: dict} -> the arrays oracle.parity.compare reads."""
    import numpy as np
    o = dict(tokens=np.full((B, K + 1), -1, np.int32), accept_len=np.full(B, -1, np.int32),
             status=np.full(B, -1, np.int32), p=np.full((B, K), np.nan, np.float32),
             q=np.full((B, K), np.nan, np.float32), draws={})
    for b, r in results.items():
        o["tokens"][b] = r["tokens"]
        o["accept_len"][b] = r["n"]
        o["status"][b] = r["status"]
        if K:
            o["p"][b] = np.asarray(r["p"], np.float64).astype(np.float32)
            o["q"][b] = np.asarray(r["q"], np.float64).astype(np.float32)
        o["draws"][b] = r["draws"]
    return o


def cpu_legs_dense(hosts, records, seed, greedy, info, early_exit=False, budget_s=20.0):
    """The oracle on (record, sequence) tasks of the timed batches, in record order.

    hosts[k]: host inputs of input set k; records: (philox step, set k, host GPU outputs)
    of the steps whose outputs were kept.  Three legs: the C oracle on the host's CPU
    share (about half the budget; its results give the parity tally), the C oracle on one
    thread and the numpy oracle on one thread (a quarter each).  early_exit: the GPU
    reports p and q only up to each sequence's first rejection (NaN after it).
    """
    from concurrent.futures import ThreadPoolExecutor

    from oracle import c_oracle as Cor
    from oracle import parity, philox
    from oracle import spec_verify_oracle as O

    B, K = hosts[0]["B"], hosts[0]["K"]
    tasks = [(j, b) for j in range(len(records)) for b in range(B)]
    unis = [None if greedy else philox.uniforms_array(seed, 0, st, B, K) for st, _, _ in records]

    def args_of(task):
        j, b = task
        h = hosts[records[j][1]]
        T = float(h["T"][b])
        sampled = T != 0.0 and not greedy
        return (h["t"][b], h["d"][b] if sampled else None, h["x"][b],
                unis[j][b] if sampled else None, T if sampled else 0.0)

    def leg(fn, threads, budget):
        done, res = 0, {}
        with ThreadPoolExecutor(max_workers=threads) as ex:
            t0 = time.perf_counter()
            while done < len(tasks) and time.perf_counter() - t0 < budget:
                chunk = tasks[done:done + 8 * threads]
                for task, r in zip(chunk, ex.map(lambda t: fn(*args_of(t)), chunk)):
                    res[task] = r
                done += len(chunk)
            wall = time.perf_counter() - t0
        return done, wall, res

    n_all, w_all, res_all = leg(Cor.verify_sequence, info["share"], budget_s / 2)
    n_one, w_one, _ = leg(Cor.verify_sequence, 1, budget_s / 4)
    n_np, w_np, _ = leg(O.verify_sequence, 1, budget_s / 4)

    import numpy as np
    tally = parity.Tally()
    uni_ok = True
    for j, (st, k, gpu) in enumerate(records):
        mine = {b: res_all[(j, b)] for b in range(B) if (j, b) in res_all}
        if not mine:
            break
        T = hosts[k]["T"] if not greedy else None
        orc = _orc_arrays(mine, B, K)
        if early_exit:
            for b in mine:
                n = int(gpu["accept_len"][b])
                if T[b] != 0 and 0 <= n < K:
                    orc["p"][b, n + 1:] = np.nan
                    orc["q"][b, n + 1:] = np.nan
        if not greedy and "uniforms" in gpu:
            uni_ok = uni_ok and bool(np.array_equal(gpu["uniforms"], unis[j]))
        tally.merge(parity.compare(gpu, orc, sorted(mine), T, greedy_only=greedy))
    what = "greedy verify" if greedy else "verify"
    cpu = f"{info['cpu_model']}; nproc {info['nproc']}, affinity {info['affinity']}, " \
          f"cgroup CPUs {info['cgroup_cpus']}"
    main = dict(value=n_all * (K + 1) / w_all, unit="positions/s", cores=info["share"],
                kind="oracle",
                sample=f"{n_all} sequences of the timed steps ({n_all / B:.1f} batches), C fp64 "
                       f"oracle ({what}) on {info['share']} threads (the host's CPU share), "
                       f"{w_all:.1f} s of wall time; host: {cpu}",
                host=info)
    one = dict(value=n_one * (K + 1) / w_one, unit="positions/s", cores=1, kind="oracle",
               sample=f"{n_one} sequences, C fp64 oracle on one thread, {w_one:.1f} s")
    nump = dict(value=n_np * (K + 1) / w_np, unit="positions/s", cores=1, kind="oracle",
                sample=f"{n_np} sequences, numpy fp64 oracle on one thread, {w_np:.1f} s")
    par = dict(tally.as_dict(), oracle="C fp64 oracle, uniforms from the oracle's own "
               "counter generator", steps=len({j for j, _ in res_all}),
               ok=tally_ok(tally) and uni_ok)
    if not greedy:
        par["gpu_uniforms_equal_oracle_generator"] = uni_ok
    return main, one, nump, par


def tally_ok(t):
    from oracle import parity
    return (not t.hard and not t.prob_bad
            and t.near_ties <= parity.NEAR_TIE_BUDGET * max(t.draws, 1))


def cpu_leg_ragged(packs, records, seed, budget_s=15.0):
    """The numpy oracle on whole sequences of the ragged batches' last steps (one thread),
    compared with the GPU's results."""
    import numpy as np

    from oracle import parity, philox
    from oracle import spec_verify_oracle as O
    B = packs[0]["B"]
    hosts = []
    for P in packs:
        hosts.append(dict(t=host_logits(P["target"]), d=host_logits(P["draft"]),
                          cu=P["cu"].cpu().numpy(), x=P["tokens"].cpu().numpy(),
                          T=P["temperature"].cpu().numpy(), K=P["K_max"], total=P["total"]))
    tally = parity.Tally()
    done, pos, t_total = 0, 0, 0.0
    while t_total < budget_s and done < len(records) * B:
        st, k, gpu = records[done // B]
        h = hosts[k]
        b = done % B
        if b == 0:
            u = philox.uniforms_packed(seed, 0, st, h["cu"], h["total"])
        t0 = time.perf_counter()
        r = O.verify_ragged(h["t"], h["d"], h["cu"], h["x"], u, h["T"], h["K"], seqs=[b])
        t_total += time.perf_counter() - t0
        c0, c1 = int(h["cu"][b]), int(h["cu"][b + 1])
        g1 = dict(tokens=gpu["tokens"][None, c0 + b:c1 + b + 1], accept_len=gpu["accept_len"][b:b + 1],
                  status=gpu["status"][b:b + 1], p=gpu["p"][None, c0:c1], q=gpu["q"][None, c0:c1])
        o1 = dict(tokens=r["tokens"][None, c0 + b:c1 + b + 1], accept_len=r["accept_len"][b:b + 1],
                  status=r["status"][b:b + 1], p=r["p"][None, c0:c1], q=r["q"][None, c0:c1],
                  draws={0: r["draws"][b]})
        tally.merge(parity.compare(g1, o1, [0], np.asarray(h["T"][b:b + 1])))
        pos += int(r["K"][b]) + 1
        done += 1
    base = dict(value=pos / t_total, unit="positions/s", cores=1, kind="oracle",
                sample=f"{done} sequences ({pos} positions) of the ragged batches' last steps, "
                       f"fp64 numpy oracle, one thread, {t_total:.1f} s of CPU time")
    return base, dict(tally.as_dict(), oracle="numpy fp64 oracle", ok=tally_ok(tally))


def cpu_leg_sample(rows, Ts, records, seed, budget_s=15.0):
    """The numpy oracle's sampler on rows of the last steps, compared with the GPU's draws."""
    import numpy as np

    from oracle import parity, philox
    from oracle import spec_verify_oracle as O
    hosts = [(host_logits(z), T.cpu().numpy()) for z, T in zip(rows, Ts)]
    B = hosts[0][0].shape[0]
    tally = parity.Tally()
    done, t_total = 0, 0.0
    while t_total < budget_s and done < len(records) * B:
        st, k, gpu = records[done // B]
        z, T = hosts[k]
        b = done % B
        if b == 0:
            u = philox.uniforms_array(seed, 1, st, B, 0).reshape(B)
        t0 = time.perf_counter()
        r = O.sample(z[b:b + 1], u[b:b + 1], T[b:b + 1])
        t_total += time.perf_counter() - t0
        g1 = dict(tokens=gpu["tokens"][b:b + 1, None],
                  accept_len=np.where(gpu["status"][b:b + 1] & ~16, -1, 0),
                  status=gpu["status"][b:b + 1], p=np.zeros((1, 0)), q=np.zeros((1, 0)))
        o1 = dict(tokens=r["tokens"][:, None], accept_len=np.where(r["status"] & ~16, -1, 0),
                  status=r["status"], p=np.zeros((1, 0)), q=np.zeros((1, 0)),
                  draws={0: r["draws"][0]})
        tally.merge(parity.compare(g1, o1, [0], T[b:b + 1]))
        done += 1
    base = dict(value=done / t_total, unit="draws/s", cores=1, kind="oracle",
                sample=f"{done} rows of the last steps, fp64 numpy oracle, one thread, "
                       f"{t_total:.1f} s of CPU time")
    return base, dict(tally.as_dict(), oracle="numpy fp64 oracle", ok=tally_ok(tally))


def cpu_leg_tree(trees, records, budget_s=15.0):
    """The numpy oracle's tree verification on whole trees of the last steps (one thread),
    compared with the GPU's results (bit for bit)."""
    from oracle import spec_verify_oracle as O
    hosts = [(host_logits(t["target"]), t["parents"].cpu().numpy(), t["tokens"].cpu().numpy())
             for t in trees]
    B, N = hosts[0][1].shape
    done, t_total, mism = 0, 0.0, 0
    while t_total < budget_s and done < len(records) * B:
        st, k, gpu = records[done // B]
        z, par, tok = hosts[k]
        b = done % B
        t0 = time.perf_counter()
        r = O.verify_tree_sequence(z[b], par[b], tok[b])
        t_total += time.perf_counter() - t0
        if (list(gpu["tokens"][b]) != r["tokens"] or int(gpu["accept_len"][b]) != r["n"]
                or int(gpu["status"][b]) != r["status"]):
            mism += 1
        done += 1
    base = dict(value=done * N / t_total, unit="nodes/s", cores=1, kind="oracle",
                sample=f"{done} trees of {N} nodes of the last steps, fp64 numpy oracle, "
                       f"one thread, {t_total:.1f} s of CPU time")
    return base, dict(sequences=done, hard=mism, oracle="numpy fp64 oracle (greedy: bit for bit)",
                      ok=mism == 0)


def copy_gbps(dev):
    """Device-to-device copy of 1 GiB (read + write), as GB/s of traffic: the same
    box's streaming rate, beside the published peak."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--min-warmup-ms", type=float, default=200.0,
                    help="keep warming up until this many ms of back-to-back steps have run")
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="verify", choices=["verify", "greedy", "ragged", "sample", "tree"])
    ap.add_argument("--early-exit", action="store_true",
                    help="verify path: sv_fill_uniforms, then spec_verify_early_exit (rows read "
                         "only up to each sequence's first rejection; p, q past it not reported)")
    ap.add_argument("--separate-uniforms", action="store_true",
                    help="verify path: sv_fill_uniforms, then spec_verify (default: "
                         "spec_verify_philox, which generates them in the same launches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain device-to-device copy of COPY_BYTES, so that a "
                         "counter profile of this command holds a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the verify step "
              "shards by sequence with no communication, so there is no multi-GPU path to time.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import speculative_decoding_verification_03_amd as sv
    from speculative_decoding_verification_03_amd import workloads as W

    dev = torch.device("cuda:0")
    cfg = args.workload
    c = W.WORKLOADS[cfg]
    esize = 2 if c["dtype"] == torch.bfloat16 else 4
    log(f"bench: workload {cfg} ({W.describe(cfg)}), path {args.path}, generating inputs")
    nsets = 2
    sets = ([W.make_inputs(cfg, step=s, device=dev) for s in range(nsets)] if args.path != "tree"
            else [W.make_inputs(cfg, step=s, device=dev, B=1) for s in range(nsets)])
    B, K, V = sets[0]["B"], sets[0]["K"], sets[0]["V"]
    ws = sv.Workspace(dev)
    seed = 1000 + cfg
    temps = sets[0]["temperature"]
    positions = B * (K + 1)
    p1_bytes = W.logit_bytes(B, K, V, c["dtype"], temps)

    def new_out():
        return dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                    accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                    p=torch.empty((B, K), dtype=torch.float32, device=dev),
                    q=torch.empty((B, K), dtype=torch.float32, device=dev),
                    status=torch.empty((B,), dtype=torch.int32, device=dev),
                    uniforms=torch.empty((B, K + 1), dtype=torch.float32, device=dev))

    outs = [new_out() for _ in range(nsets)]
    keep_timed = args.path == "verify"  # every timed step writes outputs of its own

    def step(i, out=None):
        k = i % nsets
        x = sets[k]
        o = outs[k] if out is None else out
        if args.early_exit:
            sv.sv_fill_uniforms(seed, 0, i, B, K, out=o["uniforms"])
            sv.spec_verify_early_exit(x["target"], x["draft"], x["tokens"], o["uniforms"],
                                      x["temperature"], out=o, workspace=ws)
        elif args.separate_uniforms:
            sv.sv_fill_uniforms(seed, 0, i, B, K, out=o["uniforms"])
            sv.spec_verify(x["target"], x["draft"], x["tokens"], o["uniforms"], x["temperature"],
                           out=o, workspace=ws)
        else:
            sv.spec_verify_philox(x["target"], x["draft"], x["tokens"], x["temperature"], seed, 0,
                                  i, out=o, workspace=ws)

    if args.path == "tree":
        trees = [W.make_tree_inputs(device=dev, V=V, dtype=c["dtype"], step=s_)
                 for s_ in range(nsets)]
        B, N = trees[0]["B"], trees[0]["N"]
        outs = [dict(tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
                     nodes=torch.empty((B, N), dtype=torch.int32, device=dev),
                     accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                     status=torch.empty((B,), dtype=torch.int32, device=dev))
                for _ in range(nsets)]
        positions = B * N
        p1_bytes = B * N * V * esize

        def step(i, out=None):  # noqa: F811
            k = i % nsets
            t = trees[k]
            sv.spec_verify_tree_greedy(t["target"], t["parents"], t["tokens"], out=outs[k],
                                       workspace=ws)
    elif args.path == "ragged":
        packs = []
        for s_, x in enumerate(sets):
            packs.append(W.pack_ragged(x, W.draft_counts(B, K, 4000 + s_)))
        del sets[:]
        torch.cuda.empty_cache()
        u = [torch.empty((P["total"] + B,), dtype=torch.float32, device=dev) for P in packs]
        outs = [dict(tokens=torch.empty((P["total"] + B,), dtype=torch.int32, device=dev),
                     accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                     p=torch.empty((P["total"],), dtype=torch.float32, device=dev),
                     q=torch.empty((P["total"],), dtype=torch.float32, device=dev),
                     status=torch.empty((B,), dtype=torch.int32, device=dev)) for P in packs]
        positions = sum(P["total"] + B for P in packs) / nsets
        p1_bytes = sum(W.ragged_logit_bytes(P["kb"], V, c["dtype"], P["temperature"])
                       for P in packs) / nsets

        def step(i, out=None):  # noqa: F811
            k = i % nsets
            P = packs[k]
            sv.sv_fill_uniforms_ragged(seed, 0, i, P["cu"], P["total"], K, out=u[k])
            sv.spec_verify_ragged(P["target"], P["draft"], P["cu"], P["tokens"], u[k],
                                  P["temperature"], K, out=outs[k], workspace=ws)
    elif args.path == "greedy":
        for x in sets:
            x["draft"] = None
        torch.cuda.empty_cache()
        outs = [dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                     accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                     status=torch.empty((B,), dtype=torch.int32, device=dev))
                for _ in range(nsets)]
        p1_bytes = B * (K + 1) * V * esize

        def step(i, out=None):  # noqa: F811
            k = i % nsets
            x = sets[k]
            sv.spec_verify_greedy(x["target"], x["tokens"], out=outs[k], workspace=ws)
    elif args.path == "sample":
        rows = [x["draft"][:, 0].contiguous() for x in sets]
        Ts = [x["temperature"] for x in sets]
        del sets[:]
        torch.cuda.empty_cache()
        u = [torch.empty((B,), dtype=torch.float32, device=dev) for _ in range(nsets)]
        outs = [dict(tokens=torch.empty((B,), dtype=torch.int32, device=dev),
                     status=torch.empty((B,), dtype=torch.int32, device=dev))
                for _ in range(nsets)]
        positions = B
        p1_bytes = B * V * esize

        def step(i, out=None):  # noqa: F811
            k = i % nsets
            sv.sv_fill_uniforms(seed, 1, i, B, 0, out=u[k].view(B, 1))
            sv.sv_sample(rows[k], u[k], Ts[k], out=outs[k], workspace=ws)

    box_copy = copy_gbps(dev)
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copy calibration, 3 copies of {COPY_BYTES} bytes")
        del src, dst

    # warm-up: at least args.warmup steps and at least args.min_warmup_ms of back-to-back
    # steps (the clocks settle after ~25 ms of load)
    log(f"bench: warmup (at least {args.warmup} steps and {args.min_warmup_ms:.0f} ms)")
    n_warm = 0
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    while n_warm < args.warmup or (time.perf_counter() - tw0) * 1e3 < args.min_warmup_ms:
        for _ in range(10):
            step(n_warm)
            n_warm += 1
        torch.cuda.synchronize()
        if n_warm >= 1_000_000:
            break
    warm_ms = (time.perf_counter() - tw0) * 1e3

    # clean timed region
    log(f"bench: timing {args.steps} steps")
    touts = [new_out() for _ in range(args.steps)] if keep_timed else None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(n_warm + i, touts[i] if keep_timed else None)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # the same steps again with per-kernel HIP events recorded by the library on the
    # stream its kernels run on
    log("bench: per-kernel timing")
    torch.cuda.synchronize()
    sv.sv_profile_begin()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for i in range(args.steps):
        step(n_warm + args.steps + i)
    f1.record()
    torch.cuda.synchronize()
    calls, ms_p1, ms_p2 = sv.sv_profile_end()
    ms_step_profiled = f0.elapsed_time(f1) / args.steps
    ms_pass1 = ms_p1 / calls
    ms_pass2 = ms_p2 / calls

    # outputs whose inputs the CPU leg can rebuild: every timed step (verify path), else
    # each input set's last step
    if keep_timed:
        records = [(n_warm + i, (n_warm + i) % nsets, to_host(touts[i])) for i in range(args.steps)]
    else:
        last = n_warm + 2 * args.steps - 1
        records = sorted(((s_, s_ % nsets, to_host(outs[s_ % nsets]))
                          for s_ in (last - 1, last)), key=lambda r: r[1])
    acc_all = [r[2]["accept_len"] for r in records] if "accept_len" in records[0][2] else None
    bad = int(sum(int(((r[2]["status"] & ~16) != 0).sum()) for r in records))
    value = positions / (ms_step * 1e-3)
    if args.path == "verify" and args.early_exit:
        need = sum(needed_rows(sets[k]["temperature"].cpu().numpy(), o["accept_len"], o["status"], K)
                   for st, k, o in records)
        p1_bytes = need / len(records) * V * esize
    achieved = p1_bytes / (ms_pass1 * 1e-3) / 1e9
    traffic = measured_traffic(cfg)

    # bytes of the draws (pass 2): the drawn row pair of each residual draw, the one row of
    # each bonus draw, from the kept steps' accept lengths
    draw_bytes = 0.0
    if args.path == "verify":
        for st, k, o in records:
            draw_bytes += drawn_rows(sets[k]["temperature"].cpu().numpy(), o["accept_len"],
                                     o["status"], K) * V * esize
        draw_bytes /= len(records)
    call_bytes = p1_bytes + draw_bytes

    result = {
        "metric": "verified positions/sec and logit-read GB/s (% HBM peak) at B×(K+1)×V",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_ms": args.min_warmup_ms,
        "warmup_steps_run": n_warm,
        "warmup_ms": warm_ms,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{W.describe(cfg)}" + (
                ", Zipf(1.1)-offset N(0,3^2) target logits, draft noise sigma in {0.3,1,3}, "
                "T~U[0,1.2] with 25% greedy" if cfg == 4 else ""),
            "B": B, "K": K, "V": V,
            "logits": "bf16" if c["dtype"] == torch.bfloat16 else "fp32",
            "arithmetic": "pass 1 fp32 exp with fp64 sums; resolve and pass 2 fp64",
            "parallelism": "single GPU",
        },
        "logit_bytes_call": call_bytes,
        "logit_read_gbps_call": call_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_peak_frac_call": call_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "ms_pass1": ms_pass1,
        "ms_pass2": ms_pass2,
        "ms_per_step_profiled": ms_step_profiled,
        "mean_accept_len": None if acc_all is None else float(sum(a.mean() for a in acc_all) / len(acc_all)),
        "sequences_with_data_errors": bad,
        "box": {"device": torch.cuda.get_device_name(0), "copy_gbps": box_copy},
        "roofline": {
            "kernel": "pass1_kernel (logit row streaming)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": p1_bytes,
        },
    }
    if args.path == "verify" and args.early_exit:
        result["metric"] += " (early exit)"
        result["config"]["workload"] += "; rows read only up to each sequence's first rejection"
        result["roofline"]["kernel"] = ("pass1_kernel, both rounds (algorithmic bytes: the rows "
                                        "the rule needs, up to each sequence's first rejection)")
        result["roofline"]["traffic"] = None
    if args.path == "ragged":
        kbs = [k for P in packs for k in P["kb"]]
        result["metric"] = "verified positions/sec at ragged K_b (adaptive verification)"
        result["config"]["workload"] = (
            f"ragged: {W.describe(cfg)} rows packed with K_b uniform on 1..{K} "
            f"(mean {sum(kbs) / len(kbs):.2f}), workload-4 row recipe")
        result["config"]["K_max"] = K
        result["config"]["mean_positions"] = positions
        result["roofline"]["traffic"] = None
    elif args.path == "greedy":
        result["metric"] = "verified positions/sec, every sequence greedy (spec_verify_greedy)"
        result["config"]["workload"] = (f"greedy: the target rows of {W.describe(cfg)}, "
                                       "workload-4 row recipe, T = 0 for every sequence")
        result["config"]["arithmetic"] = "fp32 compares, int32 indices (argmax, lowest index on ties)"
        result["roofline"]["traffic"] = None
    elif args.path == "tree":
        result["metric"] = "verified tree nodes/sec (greedy tree verification)"
        result["unit"] = "nodes/s"
        result["config"] = {
            "workload": f"tree: B={B} trees of N={N} nodes (levels {list(W.TREE_LEVELS)}), "
                        f"V={V} {'bf16' if c['dtype'] == torch.bfloat16 else 'fp32'}, "
                        "workload-4 row recipe, node token = parent row argmax w.p. 0.75",
            "B": B, "N": N, "V": V, "parallelism": "single GPU"}
        result["roofline"]["traffic"] = None
    elif args.path == "sample":
        result["metric"] = "sampled tokens/sec (draft-side sampler)"
        result["unit"] = "draws/s"
        result["config"]["workload"] = (f"sampler: B={B} rows of V={V} "
                                       f"{'bf16' if c['dtype'] == torch.bfloat16 else 'fp32'} "
                                       "draft logits (workload-4 recipe), T~U[0,1.2], 25% greedy")
        result["config"]["K"] = 0
        result["config"]["arithmetic"] = "fp64 weights from an LDS table of the row's bf16 values"
        result["roofline"]["traffic"] = None
        result["roofline"]["kernel"] = ("sample_kernel (one workgroup per row; algorithmic bytes: "
                                        "each row read once)")
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle) and parity")
        info = host_info()
        if args.path == "tree":
            result["cpu_baseline"], result["parity"] = cpu_leg_tree(trees, records)
        elif args.path == "ragged":
            result["cpu_baseline"], result["parity"] = cpu_leg_ragged(packs, records, seed)
        elif args.path == "sample":
            result["cpu_baseline"], result["parity"] = cpu_leg_sample(rows, Ts, records, seed)
        else:
            hosts = [dict(t=host_logits(x["target"]),
                          d=None if x["draft"] is None else host_logits(x["draft"]),
                          x=x["tokens"].cpu().numpy(), T=x["temperature"].cpu().numpy(), B=B, K=K)
                     for x in sets]
            main_, one, nump, par = cpu_legs_dense(hosts, records, seed, args.path == "greedy", info,
                                                   early_exit=args.early_exit)
            result["cpu_baseline"] = main_
            result["cpu_baseline_single_thread"] = one
            result["cpu_baseline_numpy"] = nump
            result["parity"] = par
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
