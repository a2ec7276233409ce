"""Seeded synthetic inputs for the KDA hot path.

This module only draws and rounds random numbers; it holds none of the
method's arithmetic.  It serves both the HIP path (through torch tensors built
by the caller) and the fp64 oracle, which receive the identical bits.

Recipe (every config):
  * numpy ``default_rng(seed)`` (PCG64), all draws in float32.
  * Draw order: sequence lengths -> q -> k -> v -> beta -> g -> S0, each
    tensor drawn whole in token order (in blocks of rows for very long T).
  * Streamed configs (``stream_rows`` > 0, one sequence, S0 = 0) instead draw
    the tokens in blocks of ``stream_rows`` rows, block b from its own
    generator ``default_rng([seed, b])`` in the same q -> k -> v -> beta -> g
    order, so that a million-token input can be produced block by block, in
    parallel, and fed to the GPU and to the oracle without holding it whole.
  * q and k ~ N(0, 1), each (token, head) vector L2-normalised in float32.
  * v ~ N(0, 1).
  * beta = sigmoid(N(0, 1)) per (token, head).
  * log-gate g = -softplus(N(mu, 1)) per (token, head, channel) or per
    (token, head) for a per-head gate; alpha = exp(g) lies in (0, 1).
  * S0 ~ N(0, sigma^2) with sigma = 0.1 (variance 0.01), or zeros.
  * Round once, round-to-nearest-even, to the config dtype.  bf16 tensors
    are returned as uint16 bit patterns; float32 as float32.  S0 is float32.
"""
from __future__ import annotations

import dataclasses

import numpy as np

BLOCK_ROWS = 8192  # tokens per draw block for long sequences


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class ChunkConfig:
    name: str
    H: int
    dk: int
    dv: int
    dtype: str            # "bf16" | "f32"
    gate: str             # "channel" | "head"
    gate_mu: float        # mean of the normal fed to -softplus
    s0_sigma: float       # 0 -> S0 = zeros
    seed: int
    T: int = 0            # equal-length sequences: total tokens (with N)
    N: int = 1
    lengths: tuple = ()   # varlen: (lo, hi) inclusive uniform, N draws
    stream_rows: int = 0  # > 0: tokens drawn per block of rows (see module doc)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: str
    gate: str
    gate_mu: float
    s_sigma: float
    seed: int


CONFIGS = {
    # tiny fp32 KDA forward: B=1, T=256, H=2, d=64, S0 = 0
    "kda_tiny_f32": ChunkConfig("kda_tiny_f32", H=2, dk=64, dv=64, dtype="f32", gate="channel",
                                gate_mu=0.0, s0_sigma=0.0, seed=101, T=256, N=1),
    # Gated DeltaNet special case: 8 packed sequences, lengths U{256..8192}, per-head gate
    "gdn_varlen_bf16": ChunkConfig("gdn_varlen_bf16", H=16, dk=128, dv=128, dtype="bf16",
                                   gate="head", gate_mu=0.0, s0_sigma=0.1, seed=202, N=8,
                                   lengths=(256, 8192)),
    # full KDA prefill: B=1, T=32768, H=32, d=128
    "kda_32k_bf16": ChunkConfig("kda_32k_bf16", H=32, dk=128, dv=128, dtype="bf16", gate="channel",
                                gate_mu=-1.0, s0_sigma=0.0, seed=303, T=32768, N=1),
    # long-context KDA prefill: B=1, T=1,048,576, H=16, d=128
    "kda_1m_bf16": ChunkConfig("kda_1m_bf16", H=16, dk=128, dv=128, dtype="bf16", gate="channel",
                               gate_mu=-1.0, s0_sigma=0.0, seed=404, T=1 << 20, N=1,
                               stream_rows=16384),
}

DECODE_CONFIGS = {
    # 256 independent sequences x 32 heads, d=128, fp32 state, 64 steps
    "decode_256x32": DecodeConfig("decode_256x32", N=256, H=32, dk=128, dv=128, steps=64,
                                  dtype="bf16", gate="channel", gate_mu=0.0, s_sigma=0.1, seed=505),
}


def _normal(rng, shape, mu=0.0):
    """N(mu, 1) float32, drawn in row blocks along axis 0."""
    out = np.empty(shape, dtype=np.float32)
    for s in range(0, shape[0], BLOCK_ROWS):
        e = min(s + BLOCK_ROWS, shape[0])
        out[s:e] = rng.standard_normal((e - s,) + tuple(shape[1:]), dtype=np.float32)
    if mu != 0.0:
        out += np.float32(mu)
    return out


def _l2norm_rows(x):
    for s in range(0, x.shape[0], BLOCK_ROWS):
        blk = x[s:s + BLOCK_ROWS]
        blk /= np.sqrt(np.sum(blk * blk, axis=-1, keepdims=True, dtype=np.float32))
    return x


def _round(x32, dtype):
    if dtype == "bf16":
        return bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(dtype)


def _neg_softplus(x32):
    return -np.logaddexp(np.float32(0.0), x32).astype(np.float32)


def _sigmoid(x32):
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x32))).astype(np.float32)


def draw_tokens(rng, T, H, dk, dv, dtype, gate, gate_mu):
    """q, k, v, beta, g for T tokens (in that draw order), rounded to dtype."""
    out = {}
    for name in ("q", "k"):
        out[name] = _round(_l2norm_rows(_normal(rng, (T, H, dk))), dtype)
    out["v"] = _round(_normal(rng, (T, H, dv)), dtype)
    out["beta"] = _round(_sigmoid(_normal(rng, (T, H))), dtype)
    gshape = (T, H, dk) if gate == "channel" else (T, H)
    g = _normal(rng, gshape, gate_mu)
    for s in range(0, T, BLOCK_ROWS):
        g[s:s + BLOCK_ROWS] = _neg_softplus(g[s:s + BLOCK_ROWS])
    out["g"] = _round(g, dtype)
    return out


def draw_raw_tokens(rng, T, H, dk, dv, dtype, gate, gate_mu):
    """Raw projections for T tokens, before the pre-path transforms: q, k ~ N(0,1)
    (not normalised), v ~ N(0,1), beta ~ N(0,1) (before the logistic), g ~ N(mu,1)
    (before -softplus); drawn in the order of draw_tokens and rounded to dtype."""
    out = {}
    for name in ("q", "k"):
        out[name] = _round(_normal(rng, (T, H, dk)), dtype)
    out["v"] = _round(_normal(rng, (T, H, dv)), dtype)
    out["beta"] = _round(_normal(rng, (T, H)), dtype)
    out["g"] = _round(_normal(rng, (T, H, dk) if gate == "channel" else (T, H), gate_mu), dtype)
    return out


def draw_cotangents(rng, T, N, H, dk, dv, dtype, sigma_state=1.0):
    """Cotangents for a backward pass: dO ~ N(0,1) [T, H, dv] rounded to dtype,
    and dS_T ~ N(0, sigma_state^2) fp32 [N, H, dk, dv] (drawn in that order)."""
    dO = _round(_normal(rng, (T, H, dv)), dtype)
    dST = (_normal(rng, (N, H, dk, dv)) * np.float32(sigma_state)).astype(np.float32)
    return dO, dST


def chunk_inputs(cfg, seed=None, lengths=None):
    """Inputs of a chunked-forward config.

    Returns a dict with q, k, v, g, beta (uint16 bf16 bits or float32),
    S0 (float32 [N,H,dk,dv] or None), cu_seqlens (int32 [N+1]) and the config.
    ``lengths`` overrides the sequence lengths (for small parity cases).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    if lengths is None:
        if cfg.lengths:
            lo, hi = cfg.lengths
            lengths = rng.integers(lo, hi, size=cfg.N, endpoint=True)
        else:
            lengths = [cfg.T // cfg.N] * cfg.N
    if cfg.stream_rows:
        if lengths is not None:
            raise ValueError("a streamed config has fixed lengths")
        out = {n: np.concatenate([blk[n] for _, _, blk in iter_token_blocks(cfg, workers=1)])
               for n in ("q", "k", "v", "beta", "g")}
        out["S0"] = None
        out["cu_seqlens"] = np.array([0, cfg.T], dtype=np.int32)
        out["cfg"] = cfg
        return out
    lengths = np.asarray(lengths, dtype=np.int64)
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    out = draw_tokens(rng, T, cfg.H, cfg.dk, cfg.dv, cfg.dtype, cfg.gate, cfg.gate_mu)
    if cfg.s0_sigma > 0:
        out["S0"] = (_normal(rng, (N, cfg.H, cfg.dk, cfg.dv)) * np.float32(cfg.s0_sigma)).astype(np.float32)
    else:
        out["S0"] = None
    out["cu_seqlens"] = cu
    out["cfg"] = cfg
    return out


def token_block(cfg, b):
    """Block b (rows b*R .. b*R+R-1, R = stream_rows) of a streamed config."""
    R = cfg.stream_rows
    if R <= 0 or cfg.N != 1 or cfg.s0_sigma > 0:
        raise ValueError("not a streamed config")
    start = b * R
    rows = min(R, cfg.T - start)
    if rows <= 0:
        raise IndexError(b)
    rng = np.random.default_rng([cfg.seed, b])
    return draw_tokens(rng, rows, cfg.H, cfg.dk, cfg.dv, cfg.dtype, cfg.gate, cfg.gate_mu)


def iter_token_blocks(cfg, workers=8):
    """Yield (b, start_row, block) in order for a streamed config, drawing up
    to ``workers`` blocks ahead on threads (numpy releases the GIL while it
    fills arrays, and every block has its own generator)."""
    import concurrent.futures as cf
    R = cfg.stream_rows
    nb = (cfg.T + R - 1) // R
    if workers <= 1:
        for b in range(nb):
            yield b, b * R, token_block(cfg, b)
        return
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        pending = {}
        for b in range(nb):
            while len(pending) < workers and b + len(pending) < nb:
                nxt = b + len(pending)
                pending[nxt] = ex.submit(token_block, cfg, nxt)
            yield b, b * R, pending.pop(b).result()


def small_chunk_config(H=2, dk=64, dv=64, dtype="bf16", gate="channel", gate_mu=0.0,
                       s0_sigma=0.1, seed=7):
    """A config of the same recipe at small, test-chosen shapes."""
    return ChunkConfig("custom", H=H, dk=dk, dv=dv, dtype=dtype, gate=gate, gate_mu=gate_mu,
                       s0_sigma=s0_sigma, seed=seed, T=0, N=1)


def decode_state(cfg, rng):
    """Initial fp32 state S ~ N(0, sigma^2) [N, H, dk, dv] (drawn first)."""
    return (_normal(rng, (cfg.N, cfg.H, cfg.dk, cfg.dv)) * np.float32(cfg.s_sigma)).astype(np.float32)


def decode_step_inputs(cfg, rng):
    """One decode step's tokens: q, k [N,H,dk], v [N,H,dv], beta [N,H], g [N,H,dk|]."""
    return draw_tokens(rng, cfg.N, cfg.H, cfg.dk, cfg.dv, cfg.dtype, cfg.gate, cfg.gate_mu)


def sample_positions(T, count, seed):
    """Seeded sample of token positions (without replacement, sorted)."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=min(count, T), replace=False)).astype(np.int64)
