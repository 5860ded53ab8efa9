"""Throughput of the sparse-KV self-speculative decoding hot path on one MI355X.

One step = one pass of every call of the path over one batch of the workload (default: the
Llama-3.1-8B-shaped layer, batch 64, 32000-token context, gamma 4):
  snapkv_select (SnapKV budget 512 from the prompt), kvss_streaming_set (sink 16 + window 496),
  verify_attn_full (gamma + 1 causal queries), draft_attn_sparse over the StreamingLLM set,
  spec_accept (rejection sampling, temperature 1), draft_attn_sparse over the SnapKV set.
Each draft follows a call that streams far more than the 256 MB last-level cache, so no draft
is served from rows an earlier call left there. Inputs are resident in HBM before the timed region; the timed
region allocates nothing.

value = algorithmic bytes of the whole step / step time (GB/s). Per call it also reports the
time (HIP events on the launching stream), GB/s, fraction of the 8 TB/s HBM peak and tokens/s.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "KV-attn HBM GB/s (% peak) + verify/draft tokens/s, B=64 S=32000, 1 GPU"
KERNEL_SOURCE = os.path.join(ROOT, "kv_sparse_speculative_amd", "csrc", "attn_mfma.hip")
COPY_BYTES = 1 << 30          # plain copy used to calibrate the HBM byte counters


def verify_kernel_name(wl):
    """The verify kernel instance a workload launches (one 16-row tile up to 16 query rows per
    KV head, else two; up to 8 rows the tile's spare rows carry the lo parts of P)."""
    rows = wl.group * (wl.gamma + 1)
    if wl.dtype != "bf16":
        return f"attn_simple_kernel<{wl.head_dim}, false>"
    fold = "true" if rows <= 8 else "false"
    return f"attn_mfma_kernel<{wl.head_dim}, false, {1 if rows <= 16 else 2}, {fold}>"


def verify_algorithmic_bytes(wl):
    """Algorithmic bytes of one verify call on a workload (the same definition as the timed
    run's: every K and V row once, Q, the fp32 output and LSE)."""
    from kv_sparse_speculative_amd.synth import prompt_lengths
    P = prompt_lengths(wl)
    return algorithmic_bytes(wl, P, wl.gamma + 1, 16, 496, wl.vocab)["verify"]


def _read_csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True):
        rows.extend(csv.DictReader(open(f)))
    return rows


def verify_dispatches(stats_dir, wl, warmup):
    """Durations (us) of the verify call's kernels in the timed steps, from the kernel trace: the
    verify kernel instance's dispatches that last at least half its longest one (a T = 1 decode
    over the compact draft cache can run the same instance), in launch order, less the first
    `warmup`; and the split-merge dispatches that follow each of them."""
    rows = _read_csv_rows(stats_dir, "kernel_trace.csv")
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    name = verify_kernel_name(wl)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    mine = [r for r in rows if name in r["Kernel_Name"]]
    if not mine:
        return [], []
    longest = max(dur(r) for r in mine)
    attn, merge = [], []
    for i, r in enumerate(rows):
        if name in r["Kernel_Name"] and dur(r) >= 0.5 * longest:
            nxt = rows[i + 1] if i + 1 < len(rows) else None
            attn.append(dur(r))
            merge.append(dur(nxt) if nxt is not None and "merge_kernel" in nxt["Kernel_Name"] else 0.0)
    return attn[warmup:], merge[warmup:]


def summarize_stats(stats_dir, out_path, title, command, wl=None, warmup=3):
    """rocprofv3 --stats kernel table (kvss kernels) -> profiles summary; with a workload, also
    the verify call's kernel times over the timed steps (the span bench.py's events measure)."""
    rows = _read_csv_rows(stats_dir, "kernel_stats.csv")
    lines = [f"# {title}", "", "Command:", "", *[f"    {c}" for c in command], "",
             "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        if "kvss" not in r["Name"]:
            continue
        name = r["Name"].replace("kvss::(anonymous namespace)::", "").replace("(kvss::", "(")
        lines.append(f"| `{name[:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    if wl is not None:
        attn, merge = verify_dispatches(stats_dir, wl, warmup)
        if attn:
            mean = lambda v: sum(v) / len(v)
            algo = verify_algorithmic_bytes(wl)
            total = mean(attn) + mean(merge)
            lines += ["", f"Verify calls in the timed steps ({len(attn)} calls after {warmup} warm-up "
                      f"calls; `{verify_kernel_name(wl)}` followed by `merge_kernel`):", "",
                      f"- attention kernel average: {mean(attn):.2f} us (min {min(attn):.2f}, max {max(attn):.2f})",
                      f"- split merge average: {mean(merge):.2f} us",
                      f"- call (attention + merge): {total:.2f} us, "
                      f"{algo / (total * 1e-6) / 1e9:.1f} GB/s of {algo} algorithmic bytes"]
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def library_digest():
    """Digest of everything that decides the library's kernels and launches: every source and
    header, the C ABI header and the compiler flags."""
    import glob
    import hashlib
    from kv_sparse_speculative_amd import build as kbuild
    h = hashlib.sha256()
    csrc = os.path.dirname(KERNEL_SOURCE)
    for path in sorted(glob.glob(os.path.join(csrc, "*"))) + [os.path.join(ROOT, "include", "kvss.h")]:
        if path.endswith((".hip", ".h")):
            h.update(os.path.basename(path).encode())
            h.update(open(path, "rb").read())
    h.update(" ".join(kbuild.HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


MARK_KERNEL = "philox_kernel"       # the marker launched before every call in --mark-calls runs


def _dispatches(directory):
    """Counter rows of one rocprofv3 run, grouped per dispatch in launch order:
    [(dispatch id, kernel name, {counter: value})]."""
    by_id = {}
    for r in _read_csv_rows(directory, "counter_collection.csv"):
        d = by_id.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], {}])
        d[1][r["Counter_Name"]] = d[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [(i, n, c) for i, (n, c) in sorted(by_id.items())]


def _short_kernel(name):
    return (name.replace("void ", "").replace("kvss::(anonymous namespace)::", "")
            .replace("kvss::", "").split("(")[0])


def split_calls(directory, calls):
    """Per marked call: the dispatches between its marker and the next one. Returns
    ({call: [segment, ...]}, [calibration-copy dispatches]); a segment is the list of
    (kernel name, {counter: value}) of one occurrence of the call."""
    segs, copies, cur = [], [], None
    for _, name, ctr in _dispatches(directory):
        if MARK_KERNEL in name:
            cur = []
            segs.append(cur)
        elif "copyBuffer" in name:
            copies.append(ctr)
        elif cur is not None and "kvss" in name:
            cur.append((name, ctr))
    if len(segs) != len(calls):
        raise ValueError(f"{directory}: {len(segs)} marked segments for {len(calls)} calls")
    out = {}
    for call, seg in zip(calls, segs):
        out.setdefault(call, []).append(seg)
    return out, copies


def summarize_calls(dirs, calls_path, out_path, command, wl, algo):
    """Counter summary per call of one marked bench run per directory (each directory one
    rocprofv3 --pmc pass). FETCH_SIZE and WRITE_SIZE become HBM bytes, each scaled by what the
    same counter reads for the run's plain 1 GiB copy; every other counter is reported as its
    mean per call (summed over the call's kernels) and per kernel."""
    import json as _json
    calls = _json.load(open(calls_path))
    mean = lambda v: sum(v) / len(v) if v else 0.0
    per_call, per_kernel, scale = {}, {}, {}
    for d in dirs:
        split, copies = split_calls(d, calls)
        for counter in sorted({c for segs in split.values() for seg in segs for _, ctr in seg for c in ctr}):
            if counter in ("FETCH_SIZE", "WRITE_SIZE"):
                big = max((c.get(counter, 0.0) for c in copies), default=0.0)
                scale[counter] = COPY_BYTES / (big * 1024) if big > 0 else None
            for call, segs in split.items():
                per_call.setdefault(call, {})[counter] = mean(
                    [sum(ctr.get(counter, 0.0) for _, ctr in seg) for seg in segs])
                for name, _ in segs[0]:
                    k = _short_kernel(name)
                    per_kernel.setdefault(call, {}).setdefault(k, {})[counter] = mean(
                        [sum(ctr.get(counter, 0.0) for n, ctr in seg if _short_kernel(n) == k)
                         for seg in segs])
    lines = [f"# HBM traffic and counters per call on `{wl.name}` (batch {wl.batch}, "
             f"{wl.num_q_heads} / {wl.num_kv_heads} heads, head_dim {wl.head_dim}, prompts "
             f"{wl.prompt[0]}-{wl.prompt[1]}, gamma {wl.gamma})", "",
             "Counter runs (one rocprofv3 --pmc pass each), then this summary:", "",
             *[f"    {c}" for c in command], "",
             f"- library sha256/16: `{library_digest()}`",
             f"- scale factors (bytes per counter byte, from a plain {COPY_BYTES}-byte copy): "
             f"fetch {scale.get('FETCH_SIZE')}, write {scale.get('WRITE_SIZE')}", ""]
    have_bytes = scale.get("FETCH_SIZE") and scale.get("WRITE_SIZE")
    if have_bytes:
        lines += ["| call | HBM read (B) | HBM write (B) | HBM bytes | algorithmic bytes | traffic / algorithmic |",
                  "|---|---|---|---|---|---|"]
        for call in dict.fromkeys(calls):
            if call == "setup":
                continue
            c = per_call[call]
            rd = int(c.get("FETCH_SIZE", 0.0) * 1024 * scale["FETCH_SIZE"])
            wr = int(c.get("WRITE_SIZE", 0.0) * 1024 * scale["WRITE_SIZE"])
            al = algo.get(call)
            ratio = f"{(rd + wr) / al:.4f}" if al else "-"
            lines.append(f"| {call} | {rd} | {wr} | {rd + wr} | {al if al else '-'} | {ratio} |")
        lines.append("")
    other = sorted({k for c in per_call.values() for k in c} - {"FETCH_SIZE", "WRITE_SIZE"})
    if other:
        lines += ["Other counters, mean per call:", "",
                  "| call | kernel | " + " | ".join(other) + " |", "|---|---|" + "---|" * len(other)]
        for call in dict.fromkeys(calls):
            if call == "setup":
                continue
            for k, ctr in per_kernel.get(call, {}).items():
                lines.append(f"| {call} | `{k}` | " + " | ".join(f"{ctr.get(o, 0.0):.4g}" for o in other) + " |")
        lines.append("")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def calls_summary_path(workload):
    """The committed per-call traffic summary of one workload."""
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.md")


def committed_call_traffic(workload):
    """{call: (HBM bytes, traffic / algorithmic)} from the committed per-call summary of this
    workload, if it was taken on the current library sources; else {}."""
    path = calls_summary_path(workload)
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    if f"library sha256/16: `{library_digest()}`" not in text:
        return {}
    out = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[3].isdigit():
            try:
                out[cells[0]] = (int(cells[3]), float(cells[5]))
            except ValueError:
                out[cells[0]] = (int(cells[3]), None)
    return out


def algorithmic_bytes(wl, P, T, sink, window, V):
    """Bytes each call must move (inputs read once, outputs written once); per the definitions:
    verify: all K and V rows of every sequence + Q + fp32 O and LSE; draft: the attended K and V
    rows + index list + Q + O; SnapKV: the K prompt read once + Q_obs + indices; accept: every
    logit row once."""
    eb = 2 if wl.dtype == "bf16" else 4
    Hq, Hkv, D, B = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, len(P)
    budget, w, _ = wl.snapkv
    L_verify = P + T
    L_draft = P + 1
    row = Hkv * D * 2 * eb                                      # one K row + one V row, all heads
    q_out = lambda rows: rows * Hq * D * (eb + 4) + rows * Hq * 4
    out = {}
    out["verify"] = int(L_verify.sum()) * row + q_out(B * T)
    stream_rows = sum(min(int(L), sink + window) for L in L_draft)
    out["draft_streaming"] = stream_rows * row + B * Hkv * sink * 4 + q_out(B)
    k = budget - w
    snap_rows = sum(min(k, max(int(p) - w, 0)) + (int(L) - max(int(p) - w, 0)) for p, L in zip(P, L_draft))
    out["draft_snapkv"] = snap_rows * row + B * Hkv * k * 4 + q_out(B)
    out["snapkv_select"] = int(P.sum()) * Hkv * D * eb + B * Hq * w * D * eb + B * Hkv * k * 4
    out["streaming_set"] = B * Hkv * sink * 4 + B * 12
    out["spec_accept"] = B * (2 * (T - 1) + 1) * V * 4 + B * T * 4
    return out


def measure_next_rows(wl, ns, kv_p, kv_d, sel, cnt, tail, reps, gather_detail, mark=None):
    """The calls around the hot path, each timed alone after a scrub read of the K cache (so
    the last-level cache holds none of its bytes):
      kv_append            the gamma + 1 verify rows of every sequence (rewritten in place
                           with the values already stored, so the cache is unchanged)
      draft_cache_build    the compact SnapKV draft cache, built once per prompt
      draft_snapkv_compact one draft step as a plain T = 1 decode over the compact cache,
                           next to the gathered SnapKV draft it replaces
      draft_topk_dynamic   one dynamic Top-K draft step (budget - 1 keys searched over the
                           whole prefix, plus the current token), next to the static draft
      draft_sample         the draft token of one draft step from the draft's logits
                           (temperature 1)
      decode_full          one decode token per sequence over the whole cache (verify_attn_full
                           with T = 1): the target's attention step T_T of the speedup model.
    With `mark` (a counter run), each call runs once after mark(name) and the algorithmic bytes
    per call are returned instead of timings."""
    import numpy as np
    import torch
    from kv_sparse_speculative_amd import kvss

    if mark is not None:
        mark("setup")                     # the set-up below is not one of the calls
    dev = ns.k_cache.device
    B, Hkv, D, T = ns.batch, wl.num_kv_heads, wl.head_dim, ns.T
    eb = ns.k_cache.element_size()
    P = ns.prompt_lens_np
    budget, w, _ = wl.snapkv
    k = budget - w
    stream = torch.cuda.current_stream()
    sink_buf = torch.zeros(1, dtype=torch.int32, device=dev)

    # the verify rows as they are stored (positions P .. P + T - 1)
    pos = torch.from_numpy(P.astype(np.int64))[:, None] + torch.arange(T)[None, :]
    bs = wl.block_size
    blk = torch.gather(ns.block_table.cpu().long(), 1, pos // bs)
    k_new = ns.k_cache[blk.to(dev), :, (pos % bs).to(dev)].permute(0, 2, 1, 3).contiguous()
    v_new = ns.v_cache[blk.to(dev), :, (pos % bs).to(dev)].permute(0, 2, 1, 3).contiguous()
    start = ns.prompt_lens.clone()

    cap = k + w + 1
    cb = (cap + bs - 1) // bs
    ck = torch.empty((B * cb, Hkv, bs, D), dtype=ns.k_cache.dtype, device=dev)
    cv = torch.empty_like(ck)
    ctab = torch.arange(B * cb, dtype=torch.int32, device=dev).view(B, cb)
    clens = torch.empty(B, dtype=torch.int32, device=dev)
    kv_c = kvss.PagedKV(ck, cv, ctab, clens, cap)
    q1 = ns.q_draft.unsqueeze(2).contiguous()
    o1 = torch.empty((B, wl.num_q_heads, 1, D), dtype=torch.float32, device=dev)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    kv_full = kv_p.with_lens(ns.kv_lens_draft, int(P.max()) + 1)
    o_full = torch.empty((B, wl.num_q_heads, 1, D), dtype=torch.float32, device=dev)
    q_logits = ns.draft_logits[:, 0].contiguous()                     # the draft's logits [B, V]
    d_tok = torch.empty(B, dtype=torch.int32, device=dev)
    ws_s = torch.empty(kvss.lib().kvss_sample_workspace_bytes(B, q_logits.shape[1]),
                       dtype=torch.uint8, device=dev)
    k_dyn = budget - 1
    o_t = torch.empty((B, wl.num_q_heads, D), dtype=torch.float32, device=dev)
    ws_t = torch.empty(max(kvss.lib().kvss_topk_workspace_bytes(
        __import__("ctypes").byref(kv_d.desc()), wl.num_q_heads, k_dyn), 1), dtype=torch.uint8,
        device=dev)
    calls = {
        "kv_append": lambda: kvss.kvss_kv_append(kv_p, k_new, v_new, start),
        "draft_cache_build": lambda: kvss.kvss_draft_cache_build(kv_d, sel, cnt, tail, w + 1, kv_c,
                                                                 dst_lens=clens),
        "draft_snapkv_compact": lambda: kvss.verify_attn_full(kv_c, q1, out=o1, want_lse=False,
                                                              workspace=ws),
        "draft_topk_dynamic": lambda: kvss.draft_attn_topk(kv_d, ns.q_draft, k_dyn, out=o_t,
                                                           want_lse=False, workspace=ws_t),
        "draft_sample": lambda: kvss.draft_sample(q_logits, 1.0, seed=99, offset=1, step=0,
                                                  tokens=d_tok, workspace=ws_s),
        "decode_full": lambda: kvss.verify_attn_full(kv_full, q1, out=o_full, want_lse=False,
                                                     workspace=ws),
    }
    calls["draft_cache_build"]()
    torch.cuda.synchronize()
    n_rows = int(clens.sum().item())
    row = Hkv * D * 2 * eb
    q_out = B * wl.num_q_heads * D * (eb + 4)
    L_d = P + 1
    prefix_k = int((L_d - 1).sum()) * Hkv * D * eb                 # the search reads K once
    dyn_rows = int(sum(min(k_dyn, int(x) - 1) + 1 for x in L_d))
    nbytes = {"kv_append": 2 * B * T * row,
              "draft_cache_build": 2 * n_rows * row + B * Hkv * k * 4,
              "draft_snapkv_compact": n_rows * row + q_out,
              "draft_topk_dynamic": prefix_k + dyn_rows * row + q_out,
              "draft_sample": q_logits.numel() * 4 + B * 4,
              "decode_full": int((P + 1).sum()) * row + q_out}
    if mark is not None:
        for name, fn in calls.items():
            mark(name)
            fn()
        return nbytes
    out = {}
    for name, fn in calls.items():
        times = []
        for _ in range(max(reps, 3) + 1):
            kvss.kvss_stream_read(ns.k_cache, sink_buf)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times = sorted(times[1:])
        ms = times[len(times) // 2]
        gbs = nbytes[name] / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "GB_per_s": round(gbs, 1),
                     "frac_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes[name]}
    out["draft_snapkv_compact"]["tokens_per_s"] = round(B / (out["draft_snapkv_compact"]["ms"] * 1e-3), 1)
    out["draft_snapkv_compact"]["speedup_vs_gather"] = round(
        gather_detail["ms"] / out["draft_snapkv_compact"]["ms"], 3)
    out["draft_round"] = draft_round_timing(wl, ns, kv_d, sel, cnt, tail, q_logits, d_tok, ws_s,
                                            max(reps, 3))
    out["draft_topk_dynamic"]["tokens_per_s"] = round(B / (out["draft_topk_dynamic"]["ms"] * 1e-3), 1)
    out["decode_full"]["tokens_per_s"] = round(B / (out["decode_full"]["ms"] * 1e-3), 1)
    out["draft_topk_dynamic"]["cost_vs_static_draft"] = round(
        out["draft_topk_dynamic"]["ms"] / gather_detail["ms"], 1)
    return out


def measure_config(name, reps, scrub):
    """One other workload, timed in the same run: the calls it names (verify, SnapKV selection,
    the SnapKV draft, acceptance with sampling at temperature 1, and the StreamingLLM set and
    draft where the workload has one), each after a scrub read of `scrub` (more than the 256 MB
    last-level cache), median of `reps` event-timed calls. Inputs are freed afterwards."""
    import torch
    from kv_sparse_speculative_amd import kvss
    from kv_sparse_speculative_amd.synth import generate
    from kv_sparse_speculative_amd.workloads import WORKLOADS

    wl = WORKLOADS[name]
    dev = scrub.device
    ns = generate(wl, device=dev)
    P = ns.prompt_lens_np
    B, T, D, Hq, Hkv = ns.batch, ns.T, wl.head_dim, wl.num_q_heads, wl.num_kv_heads
    budget, w, pool = wl.snapkv
    sink, window = wl.streaming or (0, 0)
    maxP = int(P.max())
    kv_p = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.prompt_lens, maxP)
    kv_d = kv_p.with_lens(ns.kv_lens_draft, maxP + 1)
    kv_v = kv_p.with_lens(ns.kv_lens_verify, maxP + T)
    tail = (ns.prompt_lens - w).contiguous()
    f32 = dict(dtype=torch.float32, device=dev)
    o_v = torch.empty((B, Hq, T, D), **f32)
    l_v = torch.empty((B, Hq, T), **f32)
    o_d = torch.empty((B, Hq, D), **f32)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sel, cnt, _ = kvss.snapkv_select(kv_p, ns.q_obs, w, pool, budget, workspace=ws)
    acc_tok = torch.empty((B, T), dtype=torch.int32, device=dev)
    acc_n = torch.empty(B, dtype=torch.int32, device=dev)
    calls = {
        "snapkv_select": lambda: kvss.snapkv_select(kv_p, ns.q_obs, w, pool, budget, sel_idx=sel,
                                                    sel_count=cnt, workspace=ws),
        "verify": lambda: kvss.verify_attn_full(kv_v, ns.q_verify, out=o_v, lse=l_v, workspace=ws),
        "draft_snapkv": lambda: kvss.draft_attn_sparse(kv_d, ns.q_draft, sel, cnt, tail, w + 1,
                                                       out=o_d, want_lse=False, workspace=ws),
        "spec_accept": lambda: kvss.spec_accept(ns.target_logits, ns.draft_logits,
                                                ns.draft_tokens, 1.0, seed=5, offset=2,
                                                out_tokens=acc_tok, num_accepted=acc_n,
                                                workspace=ws),
    }
    if wl.streaming:
        s_idx, s_cnt, s_tail = kvss.kvss_streaming_set(ns.kv_lens_draft, Hkv, sink, window)
        calls["draft_streaming"] = lambda: kvss.draft_attn_sparse(
            kv_d, ns.q_draft, s_idx, s_cnt, s_tail, window, out=o_d, want_lse=False, workspace=ws)
    nbytes = algorithmic_bytes(wl, P, T, max(sink, 1), window, ns.vocab)
    sink_buf = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    for c, fn in calls.items():
        fn()
        t = []
        for _ in range(reps):
            kvss.kvss_stream_read(scrub, sink_buf)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        t.sort()
        ms = t[len(t) // 2]
        gbs = nbytes[c] / (ms * 1e-3) / 1e9
        d = {"ms": round(ms, 4), "GB_per_s": round(gbs, 1), "frac_peak": round(gbs / HBM_PEAK_GBS, 4),
             "bytes": nbytes[c]}
        if c == "verify":
            d["tokens_per_s"] = round(B * T / (ms * 1e-3), 1)
        if c.startswith("draft"):
            d["tokens_per_s"] = round(B / (ms * 1e-3), 1)
        out[c] = d
    shape = {"batch": B, "context": [int(P.min()), maxP], "gamma": ns.gamma, "q_heads": Hq,
             "kv_heads": Hkv, "head_dim": D, "dtype": wl.dtype, "snapkv_budget": budget,
             "vocab": ns.vocab, "reps": reps}
    if wl.streaming:
        shape["streaming"] = [sink, window]
    del ns, kv_p, kv_d, kv_v, ws, calls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"shape": shape, "calls": out}


def draft_round_timing(wl, ns, kv_d, sel, cnt, tail, q_logits, tokens, ws_s, reps):
    """gamma back-to-back draft steps (gathered SnapKV draft + draft-token sampling), launched
    eagerly and as one captured HIP graph; per-step time. Within a round the draft set is read
    gamma times, so steps after the first may find it in the 256 MB last-level cache -- as in a
    real draft round; the per-call cold timings are reported separately."""
    import ctypes
    import torch
    from kv_sparse_speculative_amd import kvss

    B, Hq, D = ns.batch, wl.num_q_heads, wl.head_dim
    budget, w, _ = wl.snapkv
    gamma = ns.gamma
    o = torch.empty((B, Hq, D), dtype=torch.float32, device=ns.k_cache.device)
    ws = torch.empty(max(kvss.lib().kvss_draft_workspace_bytes(ctypes.byref(kv_d.desc()), Hq,
                                                               budget - w, w + 1), 1),
                     dtype=torch.uint8, device=ns.k_cache.device)

    def round_():
        for step in range(gamma):
            kvss.draft_attn_sparse(kv_d, ns.q_draft, sel, cnt, tail, w + 1, out=o, want_lse=False,
                                   workspace=ws)
            kvss.draft_sample(q_logits, 1.0, seed=7, offset=3, step=step, tokens=tokens,
                              workspace=ws_s)

    def timed(fn):
        sink = torch.zeros(1, dtype=torch.int32, device=ns.k_cache.device)
        t = []
        for _ in range(reps):
            kvss.kvss_stream_read(ns.k_cache, sink)        # the round starts cold
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        t.sort()
        return t[len(t) // 2] / gamma

    round_()
    torch.cuda.synchronize()
    eager = timed(round_)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        round_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            round_()
    torch.cuda.synchronize()
    graph = timed(g.replay)
    return {"gamma": gamma, "ms_per_step_eager": round(eager, 4), "ms_per_step_graph": round(graph, 4),
            "draft_tokens_per_s_graph": round(B / (graph * 1e-3), 1)}


def cpu_baseline(wl, ns, sink, window, budget_s=12.0):
    """The oracle, as written, timed on this host on a bounded sample of the same step:
    sequence 0 / KV head 0 for the attention and selection calls, sequence 0 for acceptance."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle.accept as oacc
    import oracle.attention as oatt
    import oracle.snapkv as osnap
    import oracle.streaming as ostream
    from kv_sparse_speculative_amd.synth import to_numpy

    cores = len(os.sched_getaffinity(0))
    budget, w, pool = wl.snapkv
    P = ns.prompt_lens_np
    T = ns.T
    Hkv = wl.num_kv_heads
    eb = 2 if wl.dtype == "bf16" else 4
    row = wl.head_dim * 2 * eb
    # host copies of sequence 0's blocks only
    blocks = ns.block_table_np[0][ns.block_table_np[0] >= 0]
    import torch
    idx = torch.as_tensor(blocks.astype(np.int64), device=ns.k_cache.device)
    kh = to_numpy(ns.k_cache.index_select(0, idx))
    vh = to_numpy(ns.v_cache.index_select(0, idx))
    table = np.full((1, ns.block_table_np.shape[1]), -1, dtype=np.int32)
    table[0, : len(blocks)] = np.arange(len(blocks))
    q_obs = to_numpy(ns.q_obs[:1])
    q_draft = to_numpy(ns.q_draft[:1])
    q_ver = to_numpy(ns.q_verify[:1])
    tl = to_numpy(ns.target_logits[:1])
    dl = to_numpy(ns.draft_logits[:1])
    tok = to_numpy(ns.draft_tokens[:1])
    p0 = P[:1]
    nbytes = 0
    steps = 0
    t0 = time.perf_counter()
    c0 = time.process_time()
    with threadpool_limits(limits=cores):
        while True:
            c = osnap.snapkv_scores(q_obs, kh, table, p0, w, 1 / math.sqrt(wl.head_dim), pairs=[(0, 0)])
            sel = np.full((1, Hkv, budget - w), -1, dtype=np.int32)
            n = max(int(p0[0]) - w, 0)
            sel[0, 0] = -1
            keep = osnap.top_k_positions(osnap.max_pool(c[0, 0, :n], pool), budget - w)
            sel[0, 0, : len(keep)] = keep
            cnt = np.array([len(keep)], dtype=np.int32)
            s_idx, s_cnt, s_tail = ostream.streaming_set(p0 + 1, Hkv, sink, window)
            scale = 1 / math.sqrt(wl.head_dim)
            oatt.draft_attention(q_draft, kh, vh, table, p0 + 1, s_idx, s_cnt, s_tail, scale, pairs=[(0, 0)])
            oatt.verify_attention(q_ver, kh, vh, table, p0 + T, scale, pairs=[(0, 0)])
            oatt.draft_attention(q_draft, kh, vh, table, p0 + 1, sel, cnt, p0 - w, scale, pairs=[(0, 0)])
            oacc.spec_accept(tl, dl, tok, 1.0, seed=1, offset=0)
            steps += 1
            nbytes += (int(p0[0]) + T) * row                           # verify, one KV head
            nbytes += (min(int(p0[0]) + 1, sink + window)) * row       # streaming draft
            nbytes += (len(keep) + w + 1) * row                        # SnapKV draft
            nbytes += int(p0[0]) * wl.head_dim * eb                    # SnapKV K read
            nbytes += (2 * (T - 1) + 1) * tl.shape[-1] * 4             # acceptance rows
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    busy = (time.process_time() - c0) / dt          # CPU seconds per wall second: cores in use
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "busy_cores": round(busy, 2),
            "sample": (f"{steps} step(s) of sequence 0 / KV head 0 (SnapKV select, StreamingLLM "
                       f"draft, verify, SnapKV draft) plus sequence 0's acceptance, "
                       f"{dt:.1f} s wall; numpy with a BLAS pool of {cores} threads, "
                       f"{busy:.2f} cores busy on average")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the timing of the other workloads (section 'configs')")
    ap.add_argument("--copy-reference", action="store_true",
                    help="after timing, run a plain 1 GiB copy (counter calibration)")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_DIR", "OUT"))
    ap.add_argument("--mark-calls", metavar="JSON",
                    help="counter-run mode: after warm-up, run the steps and the f-row calls once "
                         "each with a marker kernel before every call, write the call order and "
                         "algorithmic bytes to JSON, and print no benchmark line")
    ap.add_argument("--summarize-calls", nargs="+", metavar="ARG",
                    help="CALLS_JSON OUT DIR [DIR ...]: per-call summary of marked counter runs")
    ap.add_argument("--title", default="kvss kernels")
    ap.add_argument("--command", action="append", default=[])
    args = ap.parse_args()
    if args.summarize_calls:
        from kv_sparse_speculative_amd.workloads import HEADLINE, WORKLOADS
        calls_json, out, *dirs = args.summarize_calls
        import json as _json
        meta = _json.load(open(calls_json))
        tmp = calls_json + ".order"
        _json.dump(meta["calls"], open(tmp, "w"))
        summarize_calls(dirs, tmp, out, args.command, WORKLOADS[args.workload or HEADLINE],
                        meta["algorithmic"])
        os.remove(tmp)
        return
    if args.summarize_stats:
        from kv_sparse_speculative_amd.workloads import HEADLINE, WORKLOADS
        summarize_stats(*args.summarize_stats, args.title, args.command,
                        WORKLOADS[args.workload or HEADLINE], args.warmup)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path is not sharded across GPUs (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_sparse_speculative_amd import kvss
    from kv_sparse_speculative_amd.synth import generate
    from kv_sparse_speculative_amd.workloads import HEADLINE, WORKLOADS

    wl = WORKLOADS[args.workload or HEADLINE]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    ns = generate(wl, device=dev)
    B, T, D = ns.batch, ns.T, wl.head_dim
    P = ns.prompt_lens_np
    budget, w, pool = wl.snapkv
    sink, window = wl.streaming or (16, 496)
    maxP = int(P.max())
    kv_p = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.prompt_lens, maxP)
    kv_d = kv_p.with_lens(ns.kv_lens_draft, maxP + 1)
    kv_v = kv_p.with_lens(ns.kv_lens_verify, maxP + T)
    tail = (ns.prompt_lens - w).contiguous()

    # outputs and workspaces allocated once, outside the timed region
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    o_ver = torch.empty((B, wl.num_q_heads, T, D), **f32)
    l_ver = torch.empty((B, wl.num_q_heads, T), **f32)
    o_ds = torch.empty((B, wl.num_q_heads, D), **f32)
    o_dk = torch.empty((B, wl.num_q_heads, D), **f32)
    ws = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    snap_ws = torch.empty(kvss.lib().kvss_snapkv_workspace_bytes(
        __import__("ctypes").byref(kv_p.desc()), wl.num_q_heads, w, budget), dtype=torch.uint8, device=dev)
    sel = torch.empty((B, wl.num_kv_heads, budget - w), **i32)
    cnt = torch.empty(B, **i32)
    s_idx = torch.empty((B, wl.num_kv_heads, sink), **i32)
    s_cnt = torch.empty(B, **i32)
    s_tail = torch.empty(B, **i32)
    acc_tok = torch.empty((B, T), **i32)
    acc_n = torch.empty(B, **i32)
    stream = torch.cuda.current_stream()
    # Order: each draft follows a call that streams far more than the 256 MB last-level cache
    # (verify, acceptance), so neither draft is served from bytes an earlier call left there.
    calls = ["snapkv_select", "streaming_set", "verify", "draft_streaming", "spec_accept", "draft_snapkv"]
    state = {}

    def step(ev=None, marker=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
            if marker is not None and i < len(calls):
                marker(calls[i])
        mark(0)
        kvss.snapkv_select(kv_p, ns.q_obs, w, pool, budget, sel_idx=sel, sel_count=cnt,
                           workspace=snap_ws)
        mark(1)
        kvss.kvss_streaming_set(ns.kv_lens_draft, wl.num_kv_heads, sink, window, sel_idx=s_idx,
                                sel_count=s_cnt, tail_lo=s_tail)
        mark(2)
        kvss.verify_attn_full(kv_v, ns.q_verify, out=o_ver, lse=l_ver, workspace=ws)
        mark(3)
        kvss.draft_attn_sparse(kv_d, ns.q_draft, s_idx, s_cnt, s_tail, window, out=o_ds,
                               want_lse=False, workspace=ws)
        mark(4)
        out = kvss.spec_accept(ns.target_logits, ns.draft_logits, ns.draft_tokens, 1.0,
                               seed=1234, offset=state.setdefault("offset", 0), out_tokens=acc_tok,
                               num_accepted=acc_n, workspace=ws)
        state["offset"] += 1
        mark(5)
        kvss.draft_attn_sparse(kv_d, ns.q_draft, sel, cnt, tail, w + 1, out=o_dk, want_lse=False,
                               workspace=ws)
        mark(6)
        return out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.mark_calls:
        # Counter run: a one-counter Philox launch (a kernel the path never launches) before
        # every call splits the dispatch stream into calls.
        ctr = torch.zeros((1, 4), dtype=torch.int32, device=dev)
        ctr_out = torch.empty_like(ctr)
        order = []

        def marker(name):
            kvss.kvss_philox4x32_10(ctr, 0, out=ctr_out)
            order.append(name)
        for _ in range(args.steps):
            step(marker=marker)
        nb = algorithmic_bytes(wl, P, T, sink, window, ns.vocab)
        nb.update(measure_next_rows(wl, ns, kv_p, kv_d, sel, cnt, tail, 1, None, mark=marker))
        if args.copy_reference:
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(2):
                dst.copy_(src)
        torch.cuda.synchronize()
        json.dump({"calls": order, "algorithmic": nb}, open(args.mark_calls, "w"))
        print(f"marked {len(order)} calls -> {args.mark_calls}", flush=True)
        return
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = {c: 0.0 for c in calls}
    for ev in events:
        for i, c in enumerate(calls):
            per_call[c] += ev[i].elapsed_time(ev[i + 1]) / args.steps
    ms_step = wall * 1e3 / args.steps

    # measured read ceiling: a plain stream over the K cache (after the timed region)
    sink_buf = torch.zeros(1, dtype=torch.int32, device=dev)
    rd = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvss.kvss_stream_read(ns.k_cache, sink_buf)
        e1.record(stream)
        torch.cuda.synchronize()
        rd.append(e0.elapsed_time(e1))
    rd.sort()
    stream_gbs = ns.k_cache.numel() * ns.k_cache.element_size() / (rd[2] * 1e-3) / 1e9

    nbytes = algorithmic_bytes(wl, P, T, sink, window, ns.vocab)
    # The same read at a draft call's size (one launch over as many bytes as the StreamingLLM
    # draft moves, from rows no earlier read left in the last-level cache): the ceiling for a
    # launch that short, ramp-up and drain included.
    small = min(nbytes["draft_streaming"], ns.v_cache.numel() * ns.v_cache.element_size())
    v_bytes = ns.v_cache.view(-1).view(torch.uint8)[:small]
    rd = []
    for _ in range(5):
        kvss.kvss_stream_read(ns.k_cache, sink_buf)       # evicts the region read below
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvss.kvss_stream_read(v_bytes, sink_buf)
        e1.record(stream)
        torch.cuda.synchronize()
        rd.append(e0.elapsed_time(e1))
    rd.sort()
    small_gbs = small / (rd[2] * 1e-3) / 1e9

    total_bytes = sum(nbytes.values())
    traffic = committed_call_traffic(wl.name)
    detail = {}
    for c in calls:
        ms = per_call[c]
        gbs = nbytes[c] / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        d = {"ms": round(ms, 4), "GB_per_s": round(gbs, 1), "frac_peak": round(gbs / HBM_PEAK_GBS, 4),
             "frac_stream": round(gbs / stream_gbs, 4), "bytes": nbytes[c]}
        if c == "verify":
            d["tokens_per_s"] = round(B * T / (ms * 1e-3), 1)
        if c.startswith("draft"):
            d["tokens_per_s"] = round(B / (ms * 1e-3), 1)
            d["frac_stream_same_size"] = round(gbs / small_gbs, 4)
        if c in traffic:
            d["traffic_ratio"] = traffic[c][1]
        detail[c] = d
    v = detail["verify"]
    result = {
        "metric": METRIC,
        "value": round(total_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "context": maxP, "gamma": ns.gamma,
                   "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads, "head_dim": D,
                   "snapkv_budget": budget, "streaming": [sink, window], "vocab": ns.vocab},
        "roofline": {"bound": "hbm", "achieved": v["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": v["frac_peak"], "traffic": traffic.get("verify", (None,))[0],
                     "kernel": "verify_attn_full"},
        "calls": detail,
        "stream_read_GB_per_s": round(stream_gbs, 1),
        "stream_read_draft_size": {"bytes": small, "GB_per_s": round(small_gbs, 1)},
    }
    result["next"] = measure_next_rows(wl, ns, kv_p, kv_d, sel, cnt, tail, args.steps,
                                               detail["draft_snapkv"])
    for name, d in result["next"].items():
        if name in traffic:
            d["traffic_ratio"] = traffic[name][1]
    if wl.name.startswith("llama8b"):
        from kv_sparse_speculative_amd import speedup_model
        rates = speedup_model.rates_from_bench(detail, result["next"], stream_gbs, B, maxP,
                                               sink + window)
        result["model"] = speedup_model.summary(rates, B, maxP)
    if not args.no_other_configs:
        # every other workload, timed in the same run (its calls alone, cold, median of 5)
        result["configs"] = {n: measure_config(n, 5, ns.k_cache) for n in WORKLOADS
                             if n != wl.name}
    if args.copy_reference:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, ns, sink, window)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
