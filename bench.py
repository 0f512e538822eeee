"""Benchmark: CSA + HCA decode at 1M-token context on one MI355X.

One step = one decode query per sequence through
  * a CSA layer  (1M context, 4x pooling -> 262144 blocks, B = 4): the FP4
    lightning-indexer scan + top-2048 select, then attention over the
    selected blocks and the 128-token window, in one call
    (v4attn_csa_index_attend: the selector's ordering step runs inside the
    attention kernel; the same results as v4attn_index_topk followed by
    v4attn_csa_attend, which are timed beside it);
  * an HCA layer (1M context, 128x pooling -> 8192 entries, B = 16): dense
    attention over every entry plus the window (v4attn_hca_attend).
Headline `value` = decode queries per second through a CSA + HCA layer pair:
1 / (t_csa / 4 + t_hca / 16), each layer at its own batch.

Inputs are synthetic and seeded (long_context_attention_v4attn_amd.synth),
uploaded once and quantised to the cache formats on the GPU by the library
(v4attn_compress with m = 1).  `--replicas` address-distinct copies of every
cache are cycled so that no step re-reads data another recent step left in the
256 MB Infinity Cache.  Each layer is one HIP graph holding that layer's
calls for all replicas in turn (one graph launch per `--replicas` steps); the
timed loop replays K steps with a HIP event between the two layers of every
round (torch's current stream, which is the stream the library launches on).
After the timed loop, each call's graphs are replayed back to back for a
per-call breakdown, and the dominant kernel of each call is timed live with
HIP events that the library records immediately around that kernel
(v4attn_time_next_kernel); the roofline is reported for the slowest of them.

The `cpu_baseline` leg times the CPU oracle (test infrastructure) on a bounded
sample of the same workload: 4 CSA queries over one 1M-context cache row and
16 HCA queries over one cache row.
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0       # dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0       # dense MXFP4 MFMA

CSA_WID, HCA_WID = 4, 3


def algorithmic_bytes(c_csa, c_hca):
    """Bytes the method must move per query (cache reads at storage size,
    query / output / selection traffic)."""
    entry = c_csa["d_nope"] + 2 * c_csa["d_rope"] + 4                 # 580 B
    key = c_csa["d_I"] // 2 + c_csa["d_I"] // 32                       # 68 B
    D = c_csa["d_nope"] + c_csa["d_rope"]
    qo = c_csa["H"] * D * 2 * 2                                        # q in + out, bf16
    n_blocks = c_csa["ctx"] // c_csa["m"]
    idx = n_blocks * key + c_csa["H_I"] * c_csa["d_I"] * 2 + c_csa["H_I"] * 4 + c_csa["k"] * 4
    csa = (c_csa["k"] + c_csa["n_win"]) * entry + qo + c_csa["k"] * 4
    hca = (c_hca["ctx"] // c_hca["m"] + c_hca["n_win"]) * entry + qo
    return dict(index=idx, csa_attend=csa, hca_attend=hca)


def algorithmic_flops(c_csa, c_hca):
    D = c_csa["d_nope"] + c_csa["d_rope"]
    idx = (c_csa["ctx"] // c_csa["m"]) * c_csa["H_I"] * c_csa["d_I"] * 2
    csa = (c_csa["k"] + c_csa["n_win"]) * c_csa["H"] * D * 4
    hca = (c_hca["ctx"] // c_hca["m"] + c_hca["n_win"]) * c_hca["H"] * D * 4
    return dict(index=idx, csa_attend=csa, hca_attend=hca)


def kernel_bytes(c_csa, c_hca):
    """Algorithmic bytes per launch of each call's dominant kernel: the index
    scan reads every visible key (68 B per block), q^I and w; the attention
    kernel reads every entry it attends (580 B), q and (CSA) the top-k ids.
    The outputs are written by the split merge, not counted here."""
    entry = c_csa["d_nope"] + 2 * c_csa["d_rope"] + 4
    key = c_csa["d_I"] // 2 + c_csa["d_I"] // 32
    D = c_csa["d_nope"] + c_csa["d_rope"]
    q = c_csa["H"] * D * 2
    n_blocks = c_csa["ctx"] // c_csa["m"]
    return {
        "k_score_mx [index_topk]": c_csa["B"] * (n_blocks * key + c_csa["H_I"] * c_csa["d_I"] * 2
                                                  + c_csa["H_I"] * 4),
        "k_attend_fp8 [csa_attend]": c_csa["B"] * ((c_csa["k"] + c_csa["n_win"]) * entry + q
                                                    + c_csa["k"] * 4),
        "k_attend_fp8 [hca_attend]": c_hca["B"] * ((c_hca["ctx"] // c_hca["m"] + c_hca["n_win"])
                                                    * entry + q),
    }


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or
    None when the summary does not exist or was taken on a different kernel
    source (its recorded sha256 differs from the current file's)."""
    path = os.path.join(ROOT, "profiles", "attend_hca_decode_1m_counters.md")
    src = os.path.join(ROOT, "long_context_attention_v4attn_amd", "csrc", "attend.hip")
    if not kernel.startswith("k_attend_fp8") or not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    rec = {}
    for line in open(path):
        if line.startswith("traffic:"):
            for kv in line[len("traffic:"):].split():
                k_, _, v_ = kv.partition("=")
                rec[k_] = v_
    tag = "hca" if "hca" in kernel else "csa"
    if rec.get("source_sha256") != sha or f"{tag}_bytes" not in rec:
        return None
    return int(rec[f"{tag}_bytes"])


# ---------------------------------------------------------------- GPU setup

class Replica:
    pass


def copy_bandwidth(torch, nbytes=1 << 30, n=10):
    """Measured HBM streaming rate: a plain device-to-device copy of `nbytes`
    (read + written), n launches timed with events; GB/s of read + write."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / n
    del x, y
    torch.cuda.empty_cache()
    return 2 * nbytes / t / 1e9


def upload(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def quant_kv(v4, torch, x, d_nope=448, d_rope=64, fmt=None):
    """Rows x [B][n][D] (fp32, host) stored as a cache by the library
    (v4attn_compress with m = 1)."""
    B, n = x.shape[:2]
    kv = v4.KVCache.empty(B, n, d_nope, d_rope, v4.KV_FP8_BF16ROPE if fmt is None else fmt)
    xs = upload(torch, x)
    v4.v4attn_compress(xs, None, None, None, None, 1, 0, kv)
    del xs
    return kv


def quant_keys(v4, torch, x, fmt=None):
    B, n, d = x.shape
    ix = v4.IdxCache.empty(B, n, d, v4.IDX_MXFP4 if fmt is None else fmt)
    xs = upload(torch, x)
    v4.v4attn_compress(xs, None, None, None, None, 1, 0, ix)
    del xs
    return ix


def clone_kv(v4, kv):
    return v4.KVCache(kv.fmt, kv.d_nope, kv.d_rope, kv.nope.clone(), kv.rope.clone(),
                      None if kv.scale is None else kv.scale.clone())


def clone_keys(v4, ix):
    return v4.IdxCache(ix.fmt, ix.d, ix.codes.clone(), None if ix.scales is None else ix.scales.clone())


def build_inputs(v4, torch, replicas, log):
    from long_context_attention_v4attn_amd import synth
    dev = "cuda"
    cc, ch = synth.WORKLOADS[CSA_WID], synth.WORKLOADS[HCA_WID]
    t0 = time.time()
    gc = synth.decode_inputs(CSA_WID)
    gh = synth.decode_inputs(HCA_WID)
    log(f"synthetic inputs drawn in {time.time() - t0:.1f}s")

    up = lambda a: upload(torch, a)
    qkv = lambda x: quant_kv(v4, torch, x)
    qkeys = lambda x: quant_keys(v4, torch, x)

    t0 = time.time()
    base = Replica()
    base.c_comp = qkv(gc["comp"])
    base.c_keys = qkeys(gc["keys"])
    base.c_win = qkv(gc["win"])
    base.h_comp = qkv(gh["comp"])
    base.h_win = qkv(gh["win"])
    base.c_q = up(gc["q"]).to(torch.bfloat16)
    base.c_qi = up(gc["q_idx"]).to(torch.bfloat16)
    base.c_w = up(gc["w"])
    base.c_pos = up(gc["pos"])
    base.h_q = up(gh["q"]).to(torch.bfloat16)
    base.h_pos = up(gh["pos"])
    torch.cuda.synchronize()
    log(f"caches quantised on the GPU in {time.time() - t0:.1f}s")

    reps = [base]
    for _ in range(replicas - 1):
        r = Replica()
        r.c_comp, r.c_win, r.h_comp, r.h_win = (clone_kv(v4, base.c_comp), clone_kv(v4, base.c_win),
                                                clone_kv(v4, base.h_comp), clone_kv(v4, base.h_win))
        r.c_keys = clone_keys(v4, base.c_keys)
        for name in ("c_q", "c_qi", "c_w", "c_pos", "h_q", "h_pos"):
            setattr(r, name, getattr(base, name).clone())
        reps.append(r)
    for r in reps:
        r.c_topk = torch.empty(cc["B"], 1, cc["k"], dtype=torch.int32, device=dev)
        r.c_topk16 = torch.empty_like(r.c_topk)
        r.c_out = torch.empty_like(r.c_q)
        r.h_out = torch.empty_like(r.h_q)
    torch.cuda.synchronize()
    return reps, gc, gh


def make_calls(v4, torch, r, ws, cc, ch):
    """The C-ABI calls on replica r (fixed buffers): index top-k, CSA attend,
    HCA attend, the BF16-score selector variant, and the fused CSA layer
    (index top-k + CSA attend in one call).  A step is the fused CSA layer
    and the HCA attend; the separate CSA calls are timed beside it."""
    D = 512
    sc = D ** -0.5

    def idx():
        v4.v4attn_index_topk(r.c_qi, r.c_w, r.c_keys, r.c_pos, cc["m"], cc["k"], topk=r.c_topk,
                             ws=ws["index"])

    def csa():
        v4.v4attn_csa_attend(r.c_q, r.c_comp, r.c_topk, r.c_win, cc["n_win"], r.c_pos, None, sc,
                             out=r.c_out, ws=ws["csa"])

    def hca():
        v4.v4attn_hca_attend(r.h_q, r.h_comp, ch["m"], r.h_win, ch["n_win"], r.h_pos, None, sc,
                             out=r.h_out, ws=ws["hca"])

    def idx16():
        v4.v4attn_index_topk_bf16(r.c_qi, r.c_w, r.c_keys, r.c_pos, cc["m"], cc["k"],
                                  topk=r.c_topk16, ws=ws["index"])

    def csa_layer():
        v4.v4attn_csa_index_attend(r.c_qi, r.c_w, r.c_keys, cc["m"], cc["k"], r.c_q, r.c_comp,
                                   r.c_win, cc["n_win"], r.c_pos, None, sc, topk=r.c_topk,
                                   out=r.c_out, ws_index=ws["index_fused"], ws_attend=ws["csa"])

    return [idx, csa, hca, idx16, csa_layer]


# ---------------------------------------------------------------- production shapes

def graph_time(torch, fns, n):
    """Seconds per call: the calls `fns` (one per replica) captured in one
    graph, replayed n times."""
    cap_stream = torch.cuda.Stream()
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap_stream):
        for f in fns:
            f()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (n * len(fns)) * 1e-3


def bench_production(v4, torch, reps, ws, cc, ch, n=8):
    """The production shapes of the pages' hyper-parameter table on the CSA
    layer's caches: the indexer with 64 heads, top-512 and top-1024 with their
    CSA attention; and a window-only (compression-free) layer on the HCA
    layer's queries and window rings.  Each call over all replicas in one
    graph (as the step's calls), per-call times."""
    from long_context_attention_v4attn_amd import synth
    H_I, D, sc = synth.PRODUCTION["H_I"], 512, 512 ** -0.5
    B, cap = cc["B"], cc["ctx"] // cc["m"]
    q64, w64 = synth.index_queries(CSA_WID, B, H_I)
    qi = torch.from_numpy(q64).cuda().to(torch.bfloat16)
    w = torch.from_numpy(w64).cuda()
    wsi = torch.empty(v4.v4attn_workspace_bytes(v4.OP_INDEX_TOPK, B, 1, H_I, 128, cap, 4096, 0),
                      dtype=torch.uint8, device="cuda")
    res = {"indexer_heads": H_I}
    for k in synth.PRODUCTION["ks"]:
        topk = [torch.empty(B, 1, k, dtype=torch.int32, device="cuda") for _ in reps]
        wsa = torch.empty(max(1, v4.v4attn_workspace_bytes(v4.OP_CSA_ATTEND, B, 1, 64, D, 0, k, cc["n_win"])),
                          dtype=torch.uint8, device="cuda")
        f_i = [(lambda r=r, t=t: v4.v4attn_index_topk(qi, w, r.c_keys, r.c_pos, cc["m"], k, topk=t, ws=wsi))
               for r, t in zip(reps, topk)]
        f_a = [(lambda r=r, t=t: v4.v4attn_csa_attend(r.c_q, r.c_comp, t, r.c_win, cc["n_win"], r.c_pos, None,
                                                      sc, out=r.c_out, ws=wsa))
               for r, t in zip(reps, topk)]
        t_i, t_a = graph_time(torch, f_i, n), graph_time(torch, f_a, n)
        res[f"top{k}"] = {"index_topk_us": round(t_i * 1e6, 3), "csa_attend_us": round(t_a * 1e6, 3),
                          "csa_queries_per_s": round(B / (t_i + t_a), 1)}
    # window-only: a one-row compressed cache that no position reaches (the
    # split plan follows the cache size, so the list bound is the window)
    none = v4.KVCache.empty(ch["B"], 1, 448, 64, v4.KV_FP8_BF16ROPE)
    wsw = torch.empty(max(1, v4.v4attn_workspace_bytes(v4.OP_HCA_ATTEND, ch["B"], 1, 64, D, 1, 1 << 30,
                                                       ch["n_win"])), dtype=torch.uint8, device="cuda")
    f_w = [(lambda r=r: v4.v4attn_hca_attend(r.h_q, none, 1 << 30, r.h_win, ch["n_win"], r.h_pos, None,
                                             sc, out=r.h_out, ws=wsw)) for r in reps]
    t_w = graph_time(torch, f_w, n)
    res["window_only"] = {"B": ch["B"], "entries": ch["n_win"], "attend_us": round(t_w * 1e6, 3),
                          "queries_per_s": round(ch["B"] / t_w, 1)}
    return res


def bench_norm_rope(v4, torch, reps, ws, cc, ch, n=8):
    """The attend calls with the query RMSNorm + partial RoPE and the output's
    rotation back ([Notes §9], the _nr variants) beside the plain calls, on the
    benchmark's shapes (per-call times over all replicas)."""
    D, sc = 512, 512 ** -0.5
    g = torch.Generator(device="cuda").manual_seed(7)
    gamma = 0.5 + torch.rand(D, device="cuda", generator=g)
    inv = (10000.0 ** (-2.0 * torch.arange(32, dtype=torch.float64) / 64)).float().cuda()
    nr = v4.NormRope(gamma, inv, 1e-6)
    wsc = torch.empty(v4.v4attn_workspace_bytes(v4.OP_CSA_ATTEND_NR, cc["B"], 1, 64, D, 0, cc["k"],
                                                cc["n_win"]), dtype=torch.uint8, device="cuda")
    wsh = torch.empty(v4.v4attn_workspace_bytes(v4.OP_HCA_ATTEND_NR, ch["B"], 1, 64, D,
                                                ch["ctx"] // ch["m"], ch["m"], ch["n_win"]),
                      dtype=torch.uint8, device="cuda")
    f_c = [(lambda r=r: v4.v4attn_csa_attend_nr(r.c_q, r.c_comp, r.c_topk, r.c_win, cc["n_win"], r.c_pos,
                                                None, sc, nr, out=r.c_out, ws=wsc)) for r in reps]
    f_h = [(lambda r=r: v4.v4attn_hca_attend_nr(r.h_q, r.h_comp, ch["m"], r.h_win, ch["n_win"], r.h_pos,
                                                None, sc, nr, out=r.h_out, ws=wsh)) for r in reps]
    t_c, t_h = graph_time(torch, f_c, n), graph_time(torch, f_h, n)
    return {"csa_attend_nr_us": round(t_c * 1e6, 3), "hca_attend_nr_us": round(t_h * 1e6, 3)}


def bench_paged(v4, torch, reps, ws, cc, ch, n=8, page_tokens=8192):
    """The decode calls over paged caches ([Notes §11] classical cache in
    blocks of raw tokens): every replica's CSA entries, indexer keys and HCA
    entries copied into a pool whose pages are shuffled, called through the
    block table (per-call times over all replicas, as the plain calls); and
    one decode step of the compressor appends (CSA entries, indexer keys and
    window token at B = 4; HCA entry and window token at B = 16), at a
    position that completes a block of every layer."""
    dev = "cuda"
    gen = torch.Generator(device="cpu").manual_seed(5)

    def pool_of(t, P_, perm, n_pool):
        B, n_pg = perm.shape
        out = torch.empty((n_pool, P_) + tuple(t.shape[2:]), dtype=t.dtype, device=dev)
        out[perm.reshape(-1).to(dev)] = t.reshape((B * n_pg, P_) + tuple(t.shape[2:]))
        return out.reshape((1, n_pool * P_) + tuple(t.shape[2:]))

    def paged(kv, m):
        P_ = page_tokens // m
        B, n_pg = kv.nope.shape[0], kv.nope.shape[1] // P_
        n_pool = B * n_pg
        perm = torch.randperm(n_pool, generator=gen).reshape(B, n_pg)
        tab = v4.Pages(perm.to(torch.int32).to(dev).contiguous(), page_tokens)
        if isinstance(kv, v4.KVCache):
            return v4.KVCache(kv.fmt, kv.d_nope, kv.d_rope, pool_of(kv.nope, P_, perm, n_pool),
                              pool_of(kv.rope, P_, perm, n_pool),
                              pool_of(kv.scale, P_, perm, n_pool)), tab, perm, n_pool
        return v4.IdxCache(kv.fmt, kv.d, pool_of(kv.codes, P_, perm, n_pool),
                           pool_of(kv.scales, P_, perm, n_pool)), tab, perm, n_pool

    sc = 512 ** -0.5
    for r in reps:
        r.pc_comp, r.pc_tab, perm, n_pool = paged(r.c_comp, cc["m"])
        P_ = page_tokens // cc["m"]
        # the keys share the entries' table ([Notes §11]: one block layout)
        r.pc_keys = v4.IdxCache(r.c_keys.fmt, 128, pool_of(r.c_keys.codes, P_, perm, n_pool),
                                pool_of(r.c_keys.scales, P_, perm, n_pool))
        r.ph_comp, r.ph_tab, _, _ = paged(r.h_comp, ch["m"])
        r.pc_topk = torch.empty_like(r.c_topk)
    torch.cuda.synchronize()
    f_i = [(lambda r=r: v4.v4attn_index_topk_paged(r.c_qi, r.c_w, r.pc_keys, r.pc_tab, r.c_pos,
                                                   cc["m"], cc["k"], topk=r.pc_topk,
                                                   ws=ws["index"])) for r in reps]
    f_c = [(lambda r=r: v4.v4attn_csa_attend_paged(r.c_q, r.pc_comp, r.pc_tab, cc["m"], r.pc_topk,
                                                   r.c_win, cc["n_win"], r.c_pos, None, sc,
                                                   out=r.c_out, ws=ws["csa"])) for r in reps]
    f_h = [(lambda r=r: v4.v4attn_hca_attend_paged(r.h_q, r.ph_comp, r.ph_tab, ch["m"], r.h_win,
                                                   ch["n_win"], r.h_pos, None, sc,
                                                   out=r.h_out, ws=ws["hca"])) for r in reps]
    t_i, t_c, t_h = graph_time(torch, f_i, n), graph_time(torch, f_c, n), graph_time(torch, f_h, n)
    same = all(torch.equal(r.pc_topk, r.c_topk) for r in reps)
    # one decode step of the compressor appends, on replica 0's paged caches
    r = reps[0]
    g = torch.Generator(device=dev).manual_seed(9)
    rows = lambda B, d, s=1.0: (torch.randn(B, d, device=dev, generator=g) * s).to(torch.bfloat16)
    D, dI = 512, 128
    Bc, Bh = cc["B"], ch["B"]
    c_tok = [rows(Bc, D, D ** -0.5), rows(Bc, D), rows(Bc, D, D ** -0.5), rows(Bc, D)]
    k_tok = [rows(Bc, dI, dI ** -0.5), rows(Bc, dI), rows(Bc, dI, dI ** -0.5), rows(Bc, dI)]
    h_tok = [rows(Bh, D, D ** -0.5), rows(Bh, D)]
    c_state, k_state = v4.append_state(Bc, D), v4.append_state(Bc, dI)
    h_state = v4.append_state(Bh, D)
    c_bias = torch.randn(2 * cc["m"], D, device=dev, generator=g) * 0.5
    k_bias = torch.randn(2 * cc["m"], dI, device=dev, generator=g) * 0.5
    h_bias = torch.randn(ch["m"], D, device=dev, generator=g) * 0.5
    c_pos, h_pos = r.c_pos.reshape(-1).contiguous(), r.h_pos.reshape(-1).contiguous()
    f_a = [lambda: v4.v4attn_append(*c_tok, c_state, c_pos, c_bias, cc["m"], r.pc_comp, r.pc_tab),
           lambda: v4.v4attn_append(*k_tok, k_state, c_pos, k_bias, cc["m"], r.pc_keys, r.pc_tab),
           lambda: v4.v4attn_append(c_tok[0], None, None, None, None, c_pos, None, 1, r.c_win),
           lambda: v4.v4attn_append(*h_tok, None, None, h_state, h_pos, h_bias, ch["m"], r.ph_comp,
                                    r.ph_tab),
           lambda: v4.v4attn_append(h_tok[0], None, None, None, None, h_pos, None, 1, r.h_win)]
    # eight steps per graph, as the other legs (a one-node graph would time
    # the graph launch); repeated steps fold the same tokens again
    t_a = graph_time(torch, f_a * 8, n) * len(f_a)
    # the same five appends in one launch
    ent = dict(kv_cur=c_tok[0], gate_cur=c_tok[1], kv_prev=c_tok[2], gate_prev=c_tok[3],
               state=c_state, pos=c_pos, pos_bias=c_bias, m=cc["m"], out=r.pc_comp, pages=r.pc_tab)
    key = dict(kv_cur=k_tok[0], gate_cur=k_tok[1], kv_prev=k_tok[2], gate_prev=k_tok[3],
               state=k_state, pos=c_pos, pos_bias=k_bias, m=cc["m"], out=r.pc_keys, pages=r.pc_tab)
    hca = dict(kv_cur=h_tok[0], gate_cur=h_tok[1], state=h_state, pos=h_pos, pos_bias=h_bias,
               m=ch["m"], out=r.ph_comp, pages=r.ph_tab)
    batch = [ent, key, dict(kv_cur=c_tok[0], pos=c_pos, m=1, out=r.c_win), hca,
             dict(kv_cur=h_tok[0], pos=h_pos, m=1, out=r.h_win)]
    t_ab = graph_time(torch, [lambda: v4.v4attn_append_batch(batch)] * 8, n)
    for r in reps:
        del r.pc_comp, r.pc_keys, r.ph_comp
    torch.cuda.empty_cache()
    return {"page_tokens": page_tokens, "index_topk_us": round(t_i * 1e6, 3),
            "csa_attend_us": round(t_c * 1e6, 3), "hca_attend_us": round(t_h * 1e6, 3),
            "topk_equal_to_contiguous": bool(same),
            "append_step_us": round(t_ab * 1e6, 3),
            "append_step_separate_calls_us": round(t_a * 1e6, 3),
            "append_step": "CSA entry + indexer key + window token at B = 4, HCA entry + "
                           "window token at B = 16, every sequence completing a block: one "
                           "v4attn_append_batch launch (and as five v4attn_append calls)"}


def bench_append(v4, torch, r, cc, ch, n):
    """Seconds per launch of one decode step's cache appends per layer, each
    layer one v4attn_append_batch: CSA entry (overlapped pooling, m = 4),
    indexer key and window token at B = 4; HCA entry (m = 128) and window
    token at B = 16.  Position ctx - 1 completes a block of both layers, so
    every append pools its block and stores it.  Into copies of replica r's
    caches (the appended rows would otherwise change its last blocks)."""
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(11)
    rows = lambda B, d, s=1.0: (torch.randn(B, d, device=dev, generator=g) * s).to(torch.bfloat16)
    D, dI, Bc, Bh = 512, 128, cc["B"], ch["B"]
    c_tok = [rows(Bc, D, D ** -0.5), rows(Bc, D), rows(Bc, D, D ** -0.5), rows(Bc, D)]
    k_tok = [rows(Bc, dI, dI ** -0.5), rows(Bc, dI), rows(Bc, dI, dI ** -0.5), rows(Bc, dI)]
    h_tok = [rows(Bh, D, D ** -0.5), rows(Bh, D)]
    c_bias = torch.randn(2 * cc["m"], D, device=dev, generator=g) * 0.5
    k_bias = torch.randn(2 * cc["m"], dI, device=dev, generator=g) * 0.5
    h_bias = torch.randn(ch["m"], D, device=dev, generator=g) * 0.5
    c_pos, h_pos = r.c_pos.reshape(-1).contiguous(), r.h_pos.reshape(-1).contiguous()
    comp, keys, win = clone_kv(v4, r.c_comp), clone_keys(v4, r.c_keys), clone_kv(v4, r.c_win)
    hcomp, hwin = clone_kv(v4, r.h_comp), clone_kv(v4, r.h_win)
    csa_batch = [dict(kv_cur=c_tok[0], gate_cur=c_tok[1], kv_prev=c_tok[2], gate_prev=c_tok[3],
                      state=v4.append_state(Bc, D), pos=c_pos, pos_bias=c_bias, m=cc["m"], out=comp),
                 dict(kv_cur=k_tok[0], gate_cur=k_tok[1], kv_prev=k_tok[2], gate_prev=k_tok[3],
                      state=v4.append_state(Bc, dI), pos=c_pos, pos_bias=k_bias, m=cc["m"], out=keys),
                 dict(kv_cur=c_tok[0], pos=c_pos, m=1, out=win)]
    hca_batch = [dict(kv_cur=h_tok[0], gate_cur=h_tok[1], state=v4.append_state(Bh, D), pos=h_pos,
                      pos_bias=h_bias, m=ch["m"], out=hcomp),
                 dict(kv_cur=h_tok[0], pos=h_pos, m=1, out=hwin)]
    t_c = graph_time(torch, [lambda: v4.v4attn_append_batch(csa_batch)] * 8, n)
    t_h = graph_time(torch, [lambda: v4.v4attn_append_batch(hca_batch)] * 8, n)
    del comp, keys, win, hcomp, hwin
    torch.cuda.empty_cache()
    return t_c, t_h


# ---------------------------------------------------------------- the other decode configurations

def bench_csa_128k(v4, torch, log, replicas=8, n=25):
    """csa_decode_128k: B = 8 sequences of 131072 tokens (32768 blocks),
    top-1024, window 128, 64 heads x D = 512, indexer 16 x 128 MXFP4.  A step
    is v4attn_csa_index_attend for the batch (index top-k and CSA attention
    in one call; the two separate calls are timed beside it); `replicas`
    address-distinct cache copies (8 x 170 MB) cycled in one graph, as in the
    headline; the index scan kernel timed live."""
    from long_context_attention_v4attn_amd import synth
    wid = 2
    c = synth.WORKLOADS[wid]
    B, cap, k, nw = c["B"], c["ctx"] // c["m"], c["k"], c["n_win"]
    t0 = time.time()
    g = synth.decode_inputs(wid)
    base = Replica()
    base.comp, base.keys, base.win = (quant_kv(v4, torch, g["comp"]), quant_keys(v4, torch, g["keys"]),
                                      quant_kv(v4, torch, g["win"]))
    base.q = upload(torch, g["q"]).to(torch.bfloat16)
    base.qi = upload(torch, g["q_idx"]).to(torch.bfloat16)
    base.w, base.pos = upload(torch, g["w"]), upload(torch, g["pos"])
    del g
    reps = [base]
    for _ in range(replicas - 1):
        r = Replica()
        r.comp, r.keys, r.win = clone_kv(v4, base.comp), clone_keys(v4, base.keys), clone_kv(v4, base.win)
        r.q, r.qi, r.w, r.pos = base.q.clone(), base.qi.clone(), base.w.clone(), base.pos.clone()
        reps.append(r)
    for r in reps:
        r.topk = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
        r.out = torch.empty_like(r.q)
    wsi = torch.empty(v4.v4attn_workspace_bytes(v4.OP_CSA_INDEX, B, 1, c["H_I"], c["d_I"], cap, k, 0),
                      dtype=torch.uint8, device="cuda")
    wsa = torch.empty(max(1, v4.v4attn_workspace_bytes(v4.OP_CSA_ATTEND, B, 1, c["H"], 512, 0, k, nw)),
                      dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"csa_decode_128k inputs on the GPU in {time.time() - t0:.1f}s")
    sc = 512 ** -0.5
    f_i = [(lambda r=r: v4.v4attn_index_topk(r.qi, r.w, r.keys, r.pos, c["m"], k, topk=r.topk, ws=wsi))
           for r in reps]
    f_a = [(lambda r=r: v4.v4attn_csa_attend(r.q, r.comp, r.topk, r.win, nw, r.pos, None, sc,
                                             out=r.out, ws=wsa)) for r in reps]
    f_s = [(lambda r=r: v4.v4attn_csa_index_attend(r.qi, r.w, r.keys, c["m"], k, r.q, r.comp, r.win,
                                                   nw, r.pos, None, sc, topk=r.topk, out=r.out,
                                                   ws_index=wsi, ws_attend=wsa)) for r in reps]
    t_step = graph_time(torch, f_s, n)
    t_i, t_a = graph_time(torch, f_i, n), graph_time(torch, f_a, n)
    t_scan = kernel_time_of(v4, torch, f_i, 4 * replicas)
    ab = algorithmic_bytes(c, c)
    step_bytes = B * (ab["index"] + ab["csa_attend"])
    scan_bytes = B * (cap * (c["d_I"] // 2 + c["d_I"] // 32) + c["H_I"] * c["d_I"] * 2 + c["H_I"] * 4)
    for r in reps:
        del r.comp, r.keys, r.win
    del reps, wsi, wsa
    torch.cuda.empty_cache()
    return {
        "workload": "csa_decode_128k (B=8, 32768 blocks, top-1024, window 128; 64 heads x D=512; "
                    "indexer 16 x 128 MXFP4)",
        "queries_per_s": round(B / t_step, 1), "us_per_step": round(t_step * 1e6, 3),
        "calls_us": {"csa_index_attend": round(t_step * 1e6, 3), "index_topk": round(t_i * 1e6, 3),
                     "csa_attend": round(t_a * 1e6, 3)},
        "step_bytes": step_bytes,
        "step_GBps": round(step_bytes / t_step / 1e9, 1),
        "step_hbm_frac": round(step_bytes / t_step / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "k_score_mx [index_topk]", "t_us": round(t_scan * 1e6, 3),
                     "algorithmic_bytes": scan_bytes,
                     "achieved": round(scan_bytes / t_scan / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(scan_bytes / t_scan / 1e9 / HBM_PEAK_GBPS, 4)},
    }


def bench_csa_f32_4k(v4, torch, log, n=50):
    """csa_decode_f32_4k: the fp32 CSA pipeline of one sequence, a step being
    the full pipeline: pool 4096 raw tokens into 1024 entries (D = 128) and
    1024 indexer keys (d = 64), store the last 128 tokens in the window ring,
    then top-64 selection and attention for the decode query (8 heads).  A
    correctness configuration, launch-bound: 8 steps per graph on one set of
    buffers (about 13 MB, resident in the caches)."""
    from long_context_attention_v4attn_amd import synth
    m, T, D, dI, k, nw = 4, 4096, 128, 64, 64, 128
    g = synth.workload1_inputs()
    prev = lambda x: np.concatenate([np.zeros_like(x[:, :m]), x[:, :T - m]], axis=1)
    up = lambda a: upload(torch, a)
    kv_b, z_b, kv_a, z_a, bias = (up(g["kv_b"]), up(g["z_b"]), up(prev(g["kv_a"])), up(prev(g["z_a"])),
                                  up(g["bias"]))
    ki_b, zi_b, ki_a, zi_a, bias_i = (up(g["ki_b"]), up(g["zi_b"]), up(prev(g["ki_a"])),
                                      up(prev(g["zi_a"])), up(g["bias_i"]))
    tail = up(g["kv_b"][:, T - nw:])
    q, qi, w, pos = up(g["q"]), up(g["q_idx"]), up(g["w"]), up(g["pos"])
    comp = v4.KVCache.empty(1, T // m, 64, 64, v4.F32)
    keys = v4.IdxCache.empty(1, T // m, dI, v4.F32)
    win = v4.KVCache.empty(1, nw, 64, 64, v4.F32)
    topk = torch.empty(1, 1, k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    wsi = torch.empty(v4.v4attn_workspace_bytes(v4.OP_INDEX_TOPK, 1, 1, 4, dI, T // m, k, 0),
                      dtype=torch.uint8, device="cuda")
    wsa = torch.empty(max(1, v4.v4attn_workspace_bytes(v4.OP_CSA_ATTEND, 1, 1, 8, D, 0, k, nw)),
                      dtype=torch.uint8, device="cuda")

    def compress():
        v4.v4attn_compress(kv_b, z_b, kv_a, z_a, bias, m, 0, comp)
        v4.v4attn_compress(ki_b, zi_b, ki_a, zi_a, bias_i, m, 0, keys)
        v4.v4attn_compress(tail, None, None, None, None, 1, T - nw, win)

    def decode():
        v4.v4attn_index_topk(qi, w, keys, pos, m, k, topk=topk, ws=wsi)
        v4.v4attn_csa_attend(q, comp, topk, win, nw, pos, None, D ** -0.5, out=out, ws=wsa)

    step = lambda: (compress(), decode())
    t_step = graph_time(torch, [step] * 8, n)
    t_dec = graph_time(torch, [decode] * 8, n)
    f32b = 4
    comp_bytes = (4 * T * D + 4 * T * dI) * f32b + (T // m) * (D + dI) * f32b + 2 * nw * D * f32b
    dec_bytes = ((T // m) * dI + (k + nw) * D + 2 * 8 * D + 4 * dI + 4 + k) * f32b
    return {
        "workload": "csa_decode_f32_4k (B=1, 4096 raw tokens pooled to 1024 blocks, top-64, window 128; "
                    "8 heads x D=128, indexer 4 x 64; fp32)",
        "queries_per_s": round(1.0 / t_step, 1), "us_per_step": round(t_step * 1e6, 3),
        "decode_only_us": round(t_dec * 1e6, 3),
        "step_bytes": comp_bytes + dec_bytes, "decode_bytes": dec_bytes,
        "roofline": {"bound": "hbm", "what": "whole step (launch-bound: 5 launches of a few us)",
                     "achieved": round((comp_bytes + dec_bytes) / t_step / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round((comp_bytes + dec_bytes) / t_step / 1e9 / HBM_PEAK_GBPS, 4)},
    }


def kernel_time_of(v4, torch, fns, n):
    """Mean duration of the dominant kernel of the calls `fns` (cycled, n
    eager launches), from HIP events the library records around it."""
    hip = ctypes.CDLL("libamdhip64.so")
    evs = []
    for _ in range(2 * n):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs.append(e)
    torch.cuda.synchronize()
    for s in range(n):
        v4.v4attn_time_next_kernel(evs[2 * s].value, evs[2 * s + 1].value)
        fns[s % len(fns)]()
    torch.cuda.synchronize()
    tot, ms = 0.0, ctypes.c_float()
    for s in range(n):
        if hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * s], evs[2 * s + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        tot += ms.value
    for e in evs:
        hip.hipEventDestroy(e)
    return tot / n * 1e-3


# ---------------------------------------------------------------- prefill chunk

PREFILL_WID = 5


def bench_prefill(v4, torch, log, iters=8, warmup=2):
    """One chunk of 4096 new tokens after a 1M-token context (B = 1): pool the
    chunk into the CSA entries, indexer keys and HCA entries, then index top-k,
    CSA attend and HCA attend for every chunk query.  Inputs are random
    device tensors of the workload's shapes and distributions (the caches
    quantised by the library); eager launches (each call runs for
    milliseconds)."""
    from long_context_attention_v4attn_amd import synth
    c = synth.WORKLOADS[PREFILL_WID]
    dev = "cuda"
    ctx, T, H, HI, dI = c["ctx"], c["chunk"], c["H"], c["H_I"], c["d_I"]
    D = c["d_nope"] + c["d_rope"]
    n_csa, n_hca, n_win, k = ctx // c["m_csa"], ctx // c["m_hca"], c["n_win"], c["k"]
    g = torch.Generator(device=dev)
    g.manual_seed(5)

    def randn(*shape, std=1.0, dtype=torch.float32):
        return (torch.randn(*shape, device=dev, generator=g) * std).to(dtype)

    def quant_kv(n, rows_src):
        kv = v4.KVCache.empty(1, n, c["d_nope"], c["d_rope"], v4.KV_FP8_BF16ROPE)
        v4.v4attn_compress(rows_src, None, None, None, None, 1, 0, kv)
        return kv

    t0 = time.time()
    comp = v4.KVCache.empty(1, n_csa + T // 4, c["d_nope"], c["d_rope"], v4.KV_FP8_BF16ROPE)
    v4.v4attn_compress(randn(1, n_csa, D, std=D ** -0.5), None, None, None, None, 1, 0, comp)
    keys = v4.IdxCache.empty(1, n_csa + T // 4, dI, v4.IDX_MXFP4)
    v4.v4attn_compress(randn(1, n_csa, dI, std=dI ** -0.5), None, None, None, None, 1, 0, keys)
    hcomp = v4.KVCache.empty(1, n_hca + T // 128, c["d_nope"], c["d_rope"], v4.KV_FP8_BF16ROPE)
    v4.v4attn_compress(randn(1, n_hca, D, std=D ** -0.5), None, None, None, None, 1, 0, hcomp)
    R = T + n_win
    win = quant_kv(R, randn(1, R, D, std=D ** -0.5))
    hwin = quant_kv(R, randn(1, R, D, std=D ** -0.5))
    bf = torch.bfloat16
    s_csa = [randn(1, T, D, std=D ** -0.5, dtype=bf), randn(1, T, D, dtype=bf),
             randn(1, T, D, std=D ** -0.5, dtype=bf), randn(1, T, D, dtype=bf)]
    s_idx = [randn(1, T, dI, std=dI ** -0.5, dtype=bf), randn(1, T, dI, dtype=bf),
             randn(1, T, dI, std=dI ** -0.5, dtype=bf), randn(1, T, dI, dtype=bf)]
    s_hca = [randn(1, T, D, std=D ** -0.5, dtype=bf), randn(1, T, D, dtype=bf)]
    b_csa, b_idx, b_hca = randn(8, D, std=0.5), randn(8, dI, std=0.5), randn(128, D, std=0.5)
    q = randn(1, T, H, D, std=D ** -0.5, dtype=bf)
    qi = randn(1, T, HI, dI, std=dI ** -0.5, dtype=bf)
    w = torch.rand(1, T, HI, device=dev, generator=g)
    pos = (ctx + torch.arange(T, device=dev, dtype=torch.int64)).view(1, T)
    topk = torch.empty(1, T, k, dtype=torch.int32, device=dev)
    out, hout = torch.empty_like(q), torch.empty_like(q)
    ws = {
        "index": torch.empty(v4.v4attn_workspace_bytes(v4.OP_INDEX_TOPK, 1, T, HI, dI, n_csa + T // 4,
                                                       k, 0), dtype=torch.uint8, device=dev),
        "csa": torch.empty(max(1, v4.v4attn_workspace_bytes(v4.OP_CSA_ATTEND, 1, T, H, D, 0, k, n_win)),
                           dtype=torch.uint8, device=dev),
        "hca": torch.empty(max(1, v4.v4attn_workspace_bytes(v4.OP_HCA_ATTEND, 1, T, H, D,
                                                            n_hca + T // 128, 128, n_win)),
                           dtype=torch.uint8, device=dev),
    }
    torch.cuda.synchronize()
    log(f"prefill inputs on the GPU in {time.time() - t0:.1f}s")
    sc = D ** -0.5
    calls = [
        ("compress", lambda: (v4.v4attn_compress(*s_csa, b_csa, 4, ctx, comp),
                              v4.v4attn_compress(*s_idx, b_idx, 4, ctx, keys),
                              v4.v4attn_compress(s_hca[0], s_hca[1], None, None, b_hca, 128, ctx,
                                                 hcomp))),
        ("index_topk", lambda: v4.v4attn_index_topk(qi, w, keys, pos, 4, k, topk=topk, ws=ws["index"])),
        ("csa_attend", lambda: v4.v4attn_csa_attend(q, comp, topk, win, n_win, pos, None, sc, out=out,
                                                    ws=ws["csa"])),
        ("hca_attend", lambda: v4.v4attn_hca_attend(q, hcomp, 128, hwin, n_win, pos, None, sc,
                                                    out=hout, ws=ws["hca"])),
    ]
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
    tot = np.zeros(len(calls))
    for _ in range(iters):
        for i, (_, f) in enumerate(calls):
            ev[i].record(stream)
            f()
        ev[-1].record(stream)
        torch.cuda.synchronize()
        tot += [ev[i].elapsed_time(ev[i + 1]) for i in range(len(calls))]
    t_calls = tot / iters * 1e-3
    # the index scan kernel, timed live
    hip = ctypes.CDLL("libamdhip64.so")
    e0, e1, ms = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_float()
    hip.hipEventCreate(ctypes.byref(e0))
    hip.hipEventCreate(ctypes.byref(e1))
    t_scan = 0.0
    for _ in range(iters):
        v4.v4attn_time_next_kernel(e0.value, e1.value)
        calls[1][1]()
        torch.cuda.synchronize()
        hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1)
        t_scan += ms.value * 1e-3
    hip.hipEventDestroy(e0)
    hip.hipEventDestroy(e1)
    t_scan /= iters
    n_vis = (ctx + np.arange(T) + 1) // c["m_csa"]
    flops = 2.0 * HI * dI * float(n_vis.sum())
    t_chunk = float(t_calls.sum())
    return {
        "workload": "prefill_pair_1m (B=1, 4096-token chunk after 1048576 cached tokens; CSA top-2048 "
                    "+ HCA, window 128; 64 heads x D=512; indexer 16 x 128 MXFP4)",
        "tokens_per_s": round(T / t_chunk, 1),
        "ms_per_chunk": round(t_chunk * 1e3, 3),
        "calls_ms": {name: round(t * 1e3, 3) for (name, _), t in zip(calls, t_calls)},
        "index_scan": {"kernel": "k_score_mx_q", "t_us": round(t_scan * 1e6, 1),
                       "algorithmic_tflop": round(flops / 1e12, 4),
                       "achieved_tflops": round(flops / t_scan / 1e12, 1), "peak_tflops": FP4_PEAK_TFLOPS,
                       "mfma_frac": round(flops / t_scan / 1e12 / FP4_PEAK_TFLOPS, 4)},
    }


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(gc, gh, log):
    from oracle import codecs as C
    from oracle.attend import hca_attend
    from oracle.pipeline import csa_layer
    from long_context_attention_v4attn_amd import synth
    cc, ch = synth.WORKLOADS[CSA_WID], synth.WORKLOADS[HCA_WID]
    cores = len(os.sched_getaffinity(0))
    t0 = time.time()
    # one cache row of each layer, quantised by the oracle (setup, untimed)
    comp = C.kv_encode(gc["comp"][:1], "fp8", 448)
    keys = C.idx_encode(gc["keys"][:1], "mxfp4")
    win = C.kv_encode(gc["win"][:1], "fp8", 448)
    hcomp = C.kv_encode(gh["comp"][:1], "fp8", 448)
    hwin = C.kv_encode(gh["win"][:1], "fp8", 448)
    log(f"oracle setup (quantise one row of each cache) {time.time() - t0:.1f}s")
    sc = 512 ** -0.5
    # CSA: every query of the CSA batch against cache row 0
    t0 = time.time()
    for b in range(cc["B"]):
        qb = C.bf16_encode(gc["q"][b:b + 1])
        qi = C.bf16_decode(C.bf16_encode(gc["q_idx"][b:b + 1])).astype(np.float32)
        csa_layer(qb, "bf16", qi, gc["w"][b:b + 1], comp, keys, win, cc["n_win"],
                  gc["pos"][b:b + 1], cc["m"], cc["k"], sc)
    t_csa = (time.time() - t0) / cc["B"]
    t0 = time.time()
    for b in range(ch["B"]):
        qb = C.bf16_encode(gh["q"][b:b + 1])
        hca_attend(qb, "bf16", hcomp, ch["m"], hwin, ch["n_win"], gh["pos"][b:b + 1], None, sc, "bf16")
    t_hca = (time.time() - t0) / ch["B"]
    value = 1.0 / (t_csa + t_hca)
    # the prefill chunk (4096 tokens after 1048576 cached, one sequence): its
    # compress is run in full; each chunk query does a decode query's work
    # (index scores over 262145..263168 blocks, top-2048, CSA over 2176
    # entries; HCA over 8192..8224 entries + 128), so the query part is the
    # per-query times above x 4096: a fraction run, stated as such
    from oracle.compress import compress
    c5 = synth.WORKLOADS[PREFILL_WID]
    g5 = synth.prefill_inputs(n_csa=4, n_hca=1, H=1)
    ctx5, T5 = c5["ctx"], c5["chunk"]
    t0 = time.time()
    compress(g5["csa_kv_cur"], g5["csa_z_cur"], g5["csa_kv_prev"], g5["csa_z_prev"], g5["csa_bias"],
             c5["m_csa"], ctx5)
    compress(g5["idx_kv_cur"], g5["idx_z_cur"], g5["idx_kv_prev"], g5["idx_z_prev"], g5["idx_bias"],
             c5["m_csa"], ctx5)
    compress(g5["hca_kv"], g5["hca_z"], None, None, g5["hca_bias"], c5["m_hca"], ctx5)
    t_comp5 = time.time() - t0
    del g5
    est5 = t_comp5 + T5 * (t_csa + t_hca)
    prefill = {"workload": "prefill_pair_1m chunk (4096 tokens after 1048576 cached, B = 1)",
               "compress_s": round(t_comp5, 3), "compress_fraction_run": 1.0,
               "query_fraction_run": {"csa": round(cc["B"] / T5, 6), "hca": round(ch["B"] / T5, 6)},
               "est_chunk_s": round(est5, 1), "tokens_per_s": round(T5 / est5, 4),
               "how": "compress of the whole chunk timed; the query part = 4096 x the per-query "
                      "oracle times measured on the decode queries (the same work per query)"}
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": value, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": (f"{cc['B']} CSA queries over one 1M-context cache row (index scores over "
                       f"262144 blocks, top-2048, attend 2176 entries) + {ch['B']} HCA queries over "
                       f"one 8192-entry row; oracle s/query: csa {t_csa:.3f}, hca {t_hca:.3f}"),
            "cpu_model": cpu, "s_per_csa_query": t_csa, "s_per_hca_query": t_hca,
            "prefill_chunk": prefill}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk leg")
    ap.add_argument("--only", choices=["decode", "prefill"], default=None,
                    help="run one leg alone (for profiling): the decode step and its kernels, "
                         "or the prefill chunk")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    args = ap.parse_args()

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        x = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 10
        print(json.dumps({"calibration": "device copy", "bytes_read": x.numel() * 4,
                          "bytes_written": y.numel() * 4, "launches": 11,
                          "copy_GBps": round(2 * x.numel() * 4 / t / 1e9, 1),
                          "peak_GBps": HBM_PEAK_GBPS}))
        return
    import long_context_attention_v4attn_amd as v4
    from long_context_attention_v4attn_amd import synth
    v4.load()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    cc, ch = synth.WORKLOADS[CSA_WID], synth.WORKLOADS[HCA_WID]
    if args.only == "prefill":
        print(json.dumps({"prefill": bench_prefill(v4, torch, log)}))
        return

    reps, gc, gh = build_inputs(v4, torch, args.replicas, log)
    ws = {
        "index": torch.empty(v4.v4attn_workspace_bytes(v4.OP_INDEX_TOPK, cc["B"], 1, cc["H_I"], 128,
                                                       cc["ctx"] // cc["m"], cc["k"], 0),
                             dtype=torch.uint8, device="cuda"),
        "index_fused": torch.empty(v4.v4attn_workspace_bytes(v4.OP_CSA_INDEX, cc["B"], 1, cc["H_I"],
                                                             128, cc["ctx"] // cc["m"], cc["k"], 0),
                                   dtype=torch.uint8, device="cuda"),
        "csa": torch.empty(max(1, v4.v4attn_workspace_bytes(v4.OP_CSA_ATTEND, cc["B"], 1, cc["H"], 512,
                                                            0, cc["k"], cc["n_win"])),
                           dtype=torch.uint8, device="cuda"),
        "hca": torch.empty(max(1, v4.v4attn_workspace_bytes(v4.OP_HCA_ATTEND, ch["B"], 1, ch["H"], 512,
                                                            ch["ctx"] // ch["m"], ch["m"], ch["n_win"])),
                           dtype=torch.uint8, device="cuda"),
    }
    calls = [make_calls(v4, torch, r, ws, cc, ch) for r in reps]
    # eager run once per replica (also validates every call)
    for cs in calls:
        for f in cs:
            f()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    R = len(calls)
    # one graph per layer holding that layer's calls for every replica in
    # turn (R consecutive steps' worth, one graph launch per R steps, as a
    # serving loop would capture many layers at once); the same per call for
    # the breakdown
    if not args.no_graph:
        cap_stream = torch.cuda.Stream()

        def capture(fns):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_stream):
                for f in fns:
                    f()
            return g.replay

        csa_layer = capture([cs[4] for cs in calls])
        hca_layer = capture([cs[2] for cs in calls])
        per_call_g = [capture([cs[i] for cs in calls]) for i in range(5)]
        torch.cuda.synchronize()
    else:
        csa_layer = lambda: [cs[4]() for cs in calls]
        hca_layer = lambda: [cs[2]() for cs in calls]
        per_call_g = [(lambda i=i: [cs[i]() for cs in calls]) for i in range(5)]

    warm_rounds = max(1, -(-args.warmup // R))
    for _ in range(warm_rounds):
        csa_layer()
        hca_layer()
    torch.cuda.synchronize()

    # ---- the timed region: K steps = K / R rounds of (the CSA layer for the
    # R replicas, then the HCA layer for the R replicas), events between them
    K = -(-args.steps // R) * R
    rounds = K // R
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(rounds + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(rounds):
        ev[s][0].record(stream)
        csa_layer()
        ev[s][1].record(stream)
        hca_layer()
    ev[rounds][0].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_csa = sum(ev[s][0].elapsed_time(ev[s][1]) for s in range(rounds)) / K * 1e-3     # s per step
    t_hca = sum(ev[s][1].elapsed_time(ev[s + 1][0]) for s in range(rounds)) / K * 1e-3
    t_gpu = ev[0][0].elapsed_time(ev[rounds][0]) / K * 1e-3
    ms_per_step = max(wall / K, t_gpu) * 1e3
    pair_qps = 1.0 / (t_csa / cc["B"] + t_hca / ch["B"])
    # the same figure per round of R steps (the events between the rounds),
    # for its spread over the timed region
    round_qps = sorted(R / (ev[s][0].elapsed_time(ev[s][1]) * 1e-3 / cc["B"]
                            + ev[s][1].elapsed_time(ev[s + 1][0]) * 1e-3 / ch["B"])
                       for s in range(rounds))

    # ---- per-call breakdown (each call's graph replayed back to back)
    def per_call(i, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            per_call_g[i]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (n * R) * 1e-3

    n_call = max(4, rounds // 4)
    t_idx, t_csa_att, t_hca_call, t_idx16, t_fused = (per_call(i, n_call) for i in range(5))
    # recall of the fp32 selection by the BF16-score selector (every replica
    # ran both in the eager pass; same inputs)
    recalls = []
    for r in reps:
        a32, a16 = r.c_topk.cpu().numpy(), r.c_topk16.cpu().numpy()
        for b in range(cc["B"]):
            recalls.append(len(set(a32[b, 0].tolist()) & set(a16[b, 0].tolist())) / cc["k"])

    # ---- dominant kernels, timed live with HIP events recorded by the
    # library immediately around each kernel (eager launches)
    n_k = max(20, K // 8)
    kern = {
        "k_score_mx [index_topk]": kernel_time_of(v4, torch, [cs[0] for cs in calls], n_k),
        "k_attend_fp8 [csa_attend]": kernel_time_of(v4, torch, [cs[1] for cs in calls], n_k),
        "k_attend_fp8 [hca_attend]": kernel_time_of(v4, torch, [cs[2] for cs in calls], n_k),
    }

    # ---- the pair figure at a common B = 4: the HCA call on the first four
    # sequences of each replica, beside the CSA layer's B = 4
    def first4(kv):
        return v4.KVCache(kv.fmt, kv.d_nope, kv.d_rope, kv.nope[:4], kv.rope[:4], kv.scale[:4])

    sc = 512 ** -0.5
    f_h4 = [(lambda r=r, hc=first4(r.h_comp), hw=first4(r.h_win):
             v4.v4attn_hca_attend(r.h_q[:4], hc, ch["m"], hw, ch["n_win"], r.h_pos[:4], None, sc,
                                  out=r.h_out[:4], ws=ws["hca"])) for r in reps]
    t_hca4 = graph_time(torch, f_h4, n_call)

    # ---- the decode-time cache appends of one step (timed separately, not
    # in `value`): the CSA layer's entry, indexer key and window token at
    # B = 4, the HCA layer's entry and window token at B = 16, each layer one
    # v4attn_append_batch launch, on replica 0 at a position that completes
    # a block of every layer
    t_app_c, t_app_h = bench_append(v4, torch, reps[0], cc, ch, n_call)

    copy_gbps = copy_bandwidth(torch)
    ab = algorithmic_bytes(cc, ch)
    af = algorithmic_flops(cc, ch)
    kb = kernel_bytes(cc, ch)
    bytes_step = cc["B"] * (ab["index"] + ab["csa_attend"]) + ch["B"] * ab["hca_attend"]
    calls_meta = {
        "csa_index_attend": dict(t_us=t_fused * 1e6, bytes=cc["B"] * (ab["index"] + ab["csa_attend"]),
                                 flops=cc["B"] * (af["index"] + af["csa_attend"])),
        "index_topk": dict(t_us=t_idx * 1e6, bytes=cc["B"] * ab["index"], flops=cc["B"] * af["index"]),
        "csa_attend": dict(t_us=t_csa_att * 1e6, bytes=cc["B"] * ab["csa_attend"],
                           flops=cc["B"] * af["csa_attend"]),
        "hca_attend": dict(t_us=t_hca_call * 1e6, bytes=ch["B"] * ab["hca_attend"],
                           flops=ch["B"] * af["hca_attend"]),
    }
    for k_, m_ in calls_meta.items():
        m_["GBps"] = m_["bytes"] / (m_["t_us"] * 1e-6) / 1e9
        m_["hbm_frac"] = m_["GBps"] / HBM_PEAK_GBPS
    kernels_meta = {}
    for name, t in kern.items():
        b_ = kb[name]
        kernels_meta[name] = {"t_us": round(t * 1e6, 3), "bytes": b_,
                              "GBps": round(b_ / t / 1e9, 1)}
    dom = max(kern, key=lambda n_: kern[n_])
    dm = kernels_meta[dom]
    roofline = {"bound": "hbm", "achieved": dm["GBps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dm["GBps"] / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dom), "kernel": dom, "t_us": dm["t_us"],
                "algorithmic_bytes": dm["bytes"], "measured_copy_GBps": round(copy_gbps, 1)}

    result = {
        "metric": "CSA+HCA decode queries/sec at 1M ctx; achieved HBM GB/s vs peak",
        "value": round(pair_qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm_rounds * R,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "arith": "attention: bf16 MFMA on exactly widened FP8 entries, fp32 accumulate and softmax; "
                 "indexer: MXFP4 MFMA, fp32 scores",
        "data": "synthetic",
        "config": {"workload": "csa_decode_1m (B=4, 262144 blocks, top-2048, window 128) + "
                               "hca_decode_1m (B=16, 8192 entries, window 128); 64 heads x D=512",
                   "global_batch": cc["B"] + ch["B"], "seq_len": cc["ctx"], "parallelism": "none (1 GPU)"},
        "achieved_GBps_step": round(bytes_step / (t_csa + t_hca) / 1e9, 1),
        "hbm_frac_step": round(bytes_step / (t_csa + t_hca) / 1e9 / HBM_PEAK_GBPS, 4),
        "t_csa_layer_us": round(t_csa * 1e6, 3),
        "t_hca_layer_us": round(t_hca * 1e6, 3),
        "csa_qps": round(cc["B"] / t_csa, 1),
        "hca_qps": round(ch["B"] / t_hca, 1),
        "value_derivation": "value = 1 / (t_csa_layer / 4 + t_hca_layer / 16): the step time per "
                            "query of each layer at its own batch (CSA B = 4, HCA B = 16), summed",
        "value_over_rounds": {"what": "the value of each timed round of `replicas` steps",
                              "rounds": rounds, "median": round(float(np.median(round_qps)), 1),
                              "min": round(round_qps[0], 1), "max": round(round_qps[-1], 1)},
        "pair_common_b4": {"what": "both layers at B = 4: 4 / (t_csa_layer + t_hca_attend(B = 4))",
                           "queries_per_s": round(cc["B"] / (t_csa + t_hca4), 1),
                           "t_hca_attend_b4_us": round(t_hca4 * 1e6, 3)},
        "append": {"what": "the step's decode-time cache appends, not in value: one "
                           "v4attn_append_batch per layer (CSA entry + indexer key + window token "
                           "at B = 4; HCA entry + window token at B = 16)",
                   "csa_layer_us": round(t_app_c * 1e6, 3), "hca_layer_us": round(t_app_h * 1e6, 3),
                   "value_with_append": round(1.0 / ((t_csa + t_app_c) / cc["B"]
                                                     + (t_hca + t_app_h) / ch["B"]), 1)},
        "calls": {k_: {kk: round(vv, 3) for kk, vv in m_.items()} for k_, m_ in calls_meta.items()},
        "kernels": kernels_meta,
        "replicas": R,
        "graph": not args.no_graph,
        "roofline": roofline,
        "selector_bf16": {
            "what": "v4attn_index_topk_bf16 (index scores ranked in bf16) on the CSA decode call",
            "index_topk_us": round(t_idx16 * 1e6, 3), "index_topk_fp32_us": round(t_idx * 1e6, 3),
            "speedup": round(t_idx / t_idx16, 3),
            "recall_vs_fp32": round(float(np.mean(recalls)), 5),
            "recall_min": round(float(np.min(recalls)), 5)},
    }
    if args.only == "decode":
        print(json.dumps(result))
        return
    log("production shapes ...")
    result["production_shapes"] = bench_production(v4, torch, reps, ws, cc, ch)
    log("norm + RoPE variants ...")
    result["norm_rope"] = bench_norm_rope(v4, torch, reps, ws, cc, ch)
    result["norm_rope"]["csa_attend_us"] = round(t_csa_att * 1e6, 3)
    result["norm_rope"]["hca_attend_us"] = round(t_hca_call * 1e6, 3)
    log("paged caches ...")
    result["paged"] = bench_paged(v4, torch, reps, ws, cc, ch)
    result["paged"]["contiguous"] = {"index_topk_us": round(t_idx * 1e6, 3),
                                     "csa_attend_us": round(t_csa_att * 1e6, 3),
                                     "hca_attend_us": round(t_hca_call * 1e6, 3)}
    del csa_layer, hca_layer, per_call_g, calls, reps, ws, f_h4
    torch.cuda.empty_cache()
    log("csa_decode_128k ...")
    result["csa_decode_128k"] = bench_csa_128k(v4, torch, log)
    log("csa_decode_f32_4k ...")
    result["csa_decode_f32_4k"] = bench_csa_f32_4k(v4, torch, log)
    if not args.no_prefill:
        log("prefill chunk ...")
        result["prefill"] = bench_prefill(v4, torch, log)
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(gc, gh, log)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
