"""Seeded synthetic inputs for the CSA / HCA workloads.

Only random numbers and shapes live here -- no pooling, scoring, quantisation
or attention arithmetic -- so that the test-suite (which feeds the CPU oracle)
and the benchmark (which feeds the HIP library) can share it.

Every tensor is drawn from its own PCG64 stream keyed by (workload id, tensor
id, batch row), so a row's values do not depend on the batch size or on the
order of generation.  N(mu, sigma) takes sigma as the standard deviation.

Workloads (the pages run real agent traces at up to 1M tokens; no dataset is
used -- these i.i.d. inputs stand in for them, which makes the indexer's
selections random: a worst-case gather with no locality):

  1  CSA decode, fp32, B=1, 4096 raw tokens, m=4 -> 1024 blocks; 8 query heads,
     D=128 (64+64 RoPE); indexer 4 heads x 64; k=64; window 128.  Full
     pipeline from raw token streams.
  2  CSA decode, B=8, 131072 tokens -> 32768 blocks; 64 heads, D=512
     (448 FP8 + 64 BF16); indexer 16 x 128 MXFP4; k=1024; window 128.
  3  HCA decode, B=16, 1048576 tokens, m=128 -> 8192 entries + window 128.
  4  CSA decode, B=4, 1048576 tokens -> 262144 blocks; k=2048; window 128.
  5  chunked prefill, B=1: 4096 new tokens after 1048576 cached; CSA (m=4,
     k=2048) and HCA (m=128) layers; causal window 128.
Workloads 2-5 draw their cached compressed entries and index keys directly
(entries ~ N(0,1)/sqrt(512), keys ~ N(0,1)/sqrt(128)) because pooling a
1M-token raw stream on the host is impractical; pooling itself is exercised
on workload 1, on the workload-5 chunk and on the `compress_*` inputs.
"""

import numpy as np

# tensor ids (part of every stream's seed)
T_KV_A, T_KV_B, T_Z_A, T_Z_B, T_BIAS = 1, 2, 3, 4, 5
T_KI_A, T_KI_B, T_ZI_A, T_ZI_B, T_BIAS_I = 6, 7, 8, 9, 10
T_Q, T_QI, T_W, T_COMP, T_KEYS, T_WIN, T_SINK = 11, 12, 13, 14, 15, 16, 17
T_HCA_KV, T_HCA_Z, T_HCA_BIAS, T_HCA_COMP, T_HCA_WIN = 18, 19, 20, 21, 22
T_QI64, T_W64 = 23, 24

# Production shapes of the pages' hyper-parameter table (the indexer's 64
# heads, top-512 / top-1024) run on workload 4's caches with these queries.
PRODUCTION = dict(H_I=64, ks=(512, 1024))

WORKLOADS = {
    1: dict(name="csa_decode_f32_4k", kind="csa", B=1, ctx=4096, m=4, H=8,
            d_nope=64, d_rope=64, H_I=4, d_I=64, k=64, n_win=128, fmt="f32"),
    2: dict(name="csa_decode_128k", kind="csa", B=8, ctx=131072, m=4, H=64,
            d_nope=448, d_rope=64, H_I=16, d_I=128, k=1024, n_win=128, fmt="fp8"),
    3: dict(name="hca_decode_1m", kind="hca", B=16, ctx=1048576, m=128, H=64,
            d_nope=448, d_rope=64, n_win=128, fmt="fp8"),
    4: dict(name="csa_decode_1m", kind="csa", B=4, ctx=1048576, m=4, H=64,
            d_nope=448, d_rope=64, H_I=16, d_I=128, k=2048, n_win=128, fmt="fp8"),
    5: dict(name="prefill_pair_1m", kind="prefill", B=1, ctx=1048576, chunk=4096,
            m_csa=4, m_hca=128, H=64, d_nope=448, d_rope=64, H_I=16, d_I=128,
            k=2048, n_win=128, fmt="fp8"),
}


def rng(workload, tensor, b):
    return np.random.default_rng([int(workload), int(tensor), int(b)])


def normal(workload, tensor, b, shape, std=1.0):
    g = rng(workload, tensor, b)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def uniform(workload, tensor, b, shape):
    g = rng(workload, tensor, b)
    return g.random(size=shape, dtype=np.float32)


def batched(fn, B, *args, **kw):
    return np.stack([fn(b, *args, **kw) for b in range(B)])


# ---------------------------------------------------------------- workload 1

def workload1_inputs(B=1, ctx=4096, wid=1):
    """Raw token streams for the fp32 full CSA pipeline (one layer)."""
    c = WORKLOADS[1]
    D = c["d_nope"] + c["d_rope"]
    dI, m = c["d_I"], c["m"]
    g = {}
    g["kv_a"] = batched(lambda b: normal(wid, T_KV_A, b, (ctx, D), D ** -0.5), B)
    g["kv_b"] = batched(lambda b: normal(wid, T_KV_B, b, (ctx, D), D ** -0.5), B)
    g["z_a"] = batched(lambda b: normal(wid, T_Z_A, b, (ctx, D)), B)
    g["z_b"] = batched(lambda b: normal(wid, T_Z_B, b, (ctx, D)), B)
    g["bias"] = normal(wid, T_BIAS, 0, (2 * m, D), 0.5)
    g["ki_a"] = batched(lambda b: normal(wid, T_KI_A, b, (ctx, dI), dI ** -0.5), B)
    g["ki_b"] = batched(lambda b: normal(wid, T_KI_B, b, (ctx, dI), dI ** -0.5), B)
    g["zi_a"] = batched(lambda b: normal(wid, T_ZI_A, b, (ctx, dI)), B)
    g["zi_b"] = batched(lambda b: normal(wid, T_ZI_B, b, (ctx, dI)), B)
    g["bias_i"] = normal(wid, T_BIAS_I, 0, (2 * m, dI), 0.5)
    g["q"] = batched(lambda b: normal(wid, T_Q, b, (1, c["H"], D), D ** -0.5), B)
    g["q_idx"] = batched(lambda b: normal(wid, T_QI, b, (1, c["H_I"], dI), dI ** -0.5), B)
    g["w"] = batched(lambda b: uniform(wid, T_W, b, (1, c["H_I"])), B)
    g["pos"] = np.full((B, 1), ctx - 1, dtype=np.int64)
    return g


# ---------------------------------------------------------------- decode, cache-direct

def decode_inputs(wid, B=None, n_comp=None, ctx=None, with_index=None, ring=None, rows=None):
    """Cache-direct decode inputs for workloads 2-4 (fp32 values, unquantised).

    comp [B][n_comp][D], keys [B][n_comp][d_I] (CSA only), win [B][R][D] holding
    raw tokens ctx-R .. ctx-1 at ring rows t mod R, q [B][1][H][D],
    q_idx [B][1][H_I][d_I], w [B][1][H_I], pos [B][1] = ctx-1.
    Sizes may be overridden to build smaller cases with the same statistics.
    `rows` (optional) lists the batch rows to draw (default: all B); the arrays
    then hold those rows, in that order.
    """
    c = WORKLOADS[wid]
    B = c["B"] if B is None else B
    ctx = c["ctx"] if ctx is None else ctx
    m = c["m"]
    n_comp = ctx // m if n_comp is None else n_comp
    D = c["d_nope"] + c["d_rope"]
    R = c["n_win"] if ring is None else ring
    with_index = (c["kind"] == "csa") if with_index is None else with_index
    rows = list(range(B)) if rows is None else list(rows)
    batched_rows = lambda fn: np.stack([fn(b) for b in rows])
    g = {}
    g["comp"] = batched_rows(lambda b: normal(wid, T_COMP, b, (n_comp, D), D ** -0.5))
    win_tok = batched_rows(lambda b: normal(wid, T_WIN, b, (R, D), D ** -0.5))
    # token ctx-R+i lives at ring row (ctx-R+i) mod R
    ring_rows = np.arange(ctx - R, ctx) % R
    win = np.empty_like(win_tok)
    win[:, ring_rows] = win_tok
    g["win"] = win
    g["q"] = batched_rows(lambda b: normal(wid, T_Q, b, (1, c["H"], D), D ** -0.5))
    if with_index:
        dI = c["d_I"]
        g["keys"] = batched_rows(lambda b: normal(wid, T_KEYS, b, (n_comp, dI), dI ** -0.5))
        g["q_idx"] = batched_rows(lambda b: normal(wid, T_QI, b, (1, c["H_I"], dI), dI ** -0.5))
        g["w"] = batched_rows(lambda b: uniform(wid, T_W, b, (1, c["H_I"])))
    g["pos"] = np.full((len(rows), 1), ctx - 1, dtype=np.int64)
    return g


def index_queries(wid, B, H_I, rows=None):
    """Indexer queries with H_I heads for workload wid's decode rows:
    q_idx [B][1][H_I][d_I] ~ N(0,1)/sqrt(d_I), w [B][1][H_I] ~ U(0,1), drawn
    from their own streams (the 16-head draws are untouched)."""
    c = WORKLOADS[wid]
    dI = c["d_I"]
    rows = list(range(B)) if rows is None else list(rows)
    q = np.stack([normal(wid, T_QI64, b, (1, H_I, dI), dI ** -0.5) for b in rows])
    w = np.stack([uniform(wid, T_W64, b, (1, H_I)) for b in rows])
    return q, w


# ---------------------------------------------------------------- compress inputs

def compress_inputs(wid, B, T, d, m, overlap, t0=0):
    """Token streams for one compress call: kv/gate for the current role and,
    with overlap, the previous role (rows = tokens t0-m .. t0+T-m-1)."""
    g = {}
    g["kv_cur"] = batched(lambda b: normal(wid, T_KV_B, b, (T, d), d ** -0.5), B)
    g["gate_cur"] = batched(lambda b: normal(wid, T_Z_B, b, (T, d)), B)
    slots = 2 * m if overlap else m
    g["bias"] = normal(wid, T_BIAS, 0, (slots, d), 0.5)
    if overlap:
        g["kv_prev"] = batched(lambda b: normal(wid, T_KV_A, b, (T, d), d ** -0.5), B)
        g["gate_prev"] = batched(lambda b: normal(wid, T_Z_A, b, (T, d)), B)
    else:
        g["kv_prev"] = None
        g["gate_prev"] = None
    return g


# ---------------------------------------------------------------- prefill (workload 5)

def prefill_inputs(wid=5, ctx=None, chunk=None, n_csa=None, n_hca=None, H=None):
    """Workload-5 inputs (B=1).  Cached part cache-direct; the chunk as raw
    token streams.  Sizes may be overridden for smaller cases.

    csa_comp [1][n_csa][D], keys [1][n_csa][d_I], hca_comp [1][n_hca][D];
    chunk streams (fp32 values; the bench / tests cast them to bf16):
      csa_kv_cur/csa_z_cur [1][chunk][D], csa_kv_prev/csa_z_prev [1][chunk][D]
      (rows = tokens ctx-4 .. ctx+chunk-5), csa_bias [8][D];
      idx_kv_cur/idx_z_cur, idx_kv_prev/idx_z_prev [1][chunk][d_I], idx_bias [8][d_I];
      hca_kv/hca_z [1][chunk][D], hca_bias [128][D];
    window tokens before the chunk: csa_win_pre/hca_win_pre [1][n_win-1][D]
    (tokens ctx-n_win+1 .. ctx-1);
    q [1][chunk][H][D], q_idx [1][chunk][H_I][d_I], w [1][chunk][H_I],
    pos [1][chunk] = ctx .. ctx+chunk-1.
    """
    c = WORKLOADS[wid]
    ctx = c["ctx"] if ctx is None else ctx
    T = c["chunk"] if chunk is None else chunk
    H = c["H"] if H is None else H
    D = c["d_nope"] + c["d_rope"]
    dI, mc, mh, nw = c["d_I"], c["m_csa"], c["m_hca"], c["n_win"]
    n_csa = ctx // mc if n_csa is None else n_csa
    n_hca = ctx // mh if n_hca is None else n_hca
    s, sI = D ** -0.5, dI ** -0.5
    g = {}
    g["csa_comp"] = normal(wid, T_COMP, 0, (1, n_csa, D), s)
    g["keys"] = normal(wid, T_KEYS, 0, (1, n_csa, dI), sI)
    g["hca_comp"] = normal(wid, T_HCA_COMP, 0, (1, n_hca, D), s)
    g["csa_kv_cur"] = normal(wid, T_KV_B, 0, (1, T, D), s)
    g["csa_z_cur"] = normal(wid, T_Z_B, 0, (1, T, D))
    g["csa_kv_prev"] = normal(wid, T_KV_A, 0, (1, T, D), s)
    g["csa_z_prev"] = normal(wid, T_Z_A, 0, (1, T, D))
    g["csa_bias"] = normal(wid, T_BIAS, 0, (2 * mc, D), 0.5)
    g["idx_kv_cur"] = normal(wid, T_KI_B, 0, (1, T, dI), sI)
    g["idx_z_cur"] = normal(wid, T_ZI_B, 0, (1, T, dI))
    g["idx_kv_prev"] = normal(wid, T_KI_A, 0, (1, T, dI), sI)
    g["idx_z_prev"] = normal(wid, T_ZI_A, 0, (1, T, dI))
    g["idx_bias"] = normal(wid, T_BIAS_I, 0, (2 * mc, dI), 0.5)
    g["hca_kv"] = normal(wid, T_HCA_KV, 0, (1, T, D), s)
    g["hca_z"] = normal(wid, T_HCA_Z, 0, (1, T, D))
    g["hca_bias"] = normal(wid, T_HCA_BIAS, 0, (mh, D), 0.5)
    g["csa_win_pre"] = normal(wid, T_WIN, 0, (1, nw - 1, D), s)
    g["hca_win_pre"] = normal(wid, T_HCA_WIN, 0, (1, nw - 1, D), s)
    g["q"] = normal(wid, T_Q, 0, (1, T, H, D), s)
    g["q_idx"] = normal(wid, T_QI, 0, (1, T, c["H_I"], dI), sI)
    g["w"] = uniform(wid, T_W, 0, (1, T, c["H_I"]))
    g["pos"] = (ctx + np.arange(T, dtype=np.int64))[None, :]
    return g
