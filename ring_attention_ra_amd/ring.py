"""Simulated ring: the sequence of K/V chunks one rank receives, on one GPU.

A real ring passes each K/V chunk from device i to device i+1 while every
device folds the chunk it holds into its running state (discosf.com article,
§3.1 环形通信拓扑; digipub.cc "大模型如何訓練百萬 Token 上下文", section "Zig
Zag Ring Attention"). Here all N chunks sit in HBM, rank-major, and the rank
under study meets them in ring order: its own chunk first, then the chunk of
rank r-1, r-2, ... . Every step runs in libra.so's kernels; this module only
sequences the calls and allocates the buffers.
"""

from __future__ import annotations

import torch

from . import _lib


def ring_schedule(n_ranks: int, rank: int) -> list[int]:
    """Chunk folded in at each hop: after j hops rank r holds rank (r-j)'s chunk."""
    if not 0 <= rank < n_ranks:
        raise ValueError("rank out of range")
    return [(rank - j) % n_ranks for j in range(n_ranks)]


def alibi_slopes(num_heads: int, device="cuda") -> torch.Tensor:
    """Head slopes 2^(-8 i / H), i = 1..H, as fp32 (intelliparadigm.com
    long-context survey, §2.1.2 ALiBi方案的创新设计)."""
    return torch.tensor([2.0 ** (-8.0 * i / num_heads) for i in range(1, num_heads + 1)],
                        dtype=torch.float32, device=device)


def positions(seq_len: int, n_ranks: int, layout: str, rank: int = -1, device="cuda") -> torch.Tensor:
    """Global positions per rank ([N, C], or [C] for one rank), int32."""
    c = seq_len // n_ranks
    out = torch.empty((n_ranks, c) if rank < 0 else (c,), dtype=torch.int32, device=device)
    _lib.ra_positions(seq_len, n_ranks, rank, layout, out)
    return out


def shard(q_g, k_g, v_g, n_ranks: int, layout: str, rank: int, stream=None):
    """Permute global-order Q/K/V [B,H,S,D] into this rank's query chunk
    [B,Hq,C,D], the rank-major K/V chunks [N,B,Hkv,C,D] and the positions
    [N,C] (int32)."""
    b, hq, s, d = q_g.shape
    hkv = k_g.shape[1]
    c = s // n_ranks
    q_loc = torch.empty((b, hq, c, d), dtype=q_g.dtype, device=q_g.device)
    k_ch = torch.empty((n_ranks, b, hkv, c, d), dtype=k_g.dtype, device=k_g.device)
    v_ch = torch.empty_like(k_ch)
    pos = torch.empty((n_ranks, c), dtype=torch.int32, device=q_g.device)
    _lib.ra_layout_permute(q_g, q_loc, None, b * hq, s, d, n_ranks, layout, rank=rank, stream=stream)
    _lib.ra_layout_permute(k_g, k_ch, pos, b * hkv, s, d, n_ranks, layout, rank=-1, stream=stream)
    _lib.ra_layout_permute(v_g, v_ch, None, b * hkv, s, d, n_ranks, layout, rank=-1, stream=stream)
    return q_loc, k_ch, v_ch, pos


class State:
    """Running accumulators of one rank: o_acc [B,Hq,C,D], m and l [B,Hq,C] (fp32)."""

    def __init__(self, dims, device, stream=None):
        rows = (dims.batch, dims.heads_q, dims.len_q)
        self.dims = dims
        self.o_acc = torch.empty(rows + (dims.head_dim,), dtype=torch.float32, device=device)
        self.m = torch.empty(rows, dtype=torch.float32, device=device)
        self.l = torch.empty(rows, dtype=torch.float32, device=device)
        _lib.ra_state_init(dims, self.o_acc, self.m, self.l, stream)


def fold(state: State, q_loc, k_blk, v_blk, q_pos, k_pos, causal, scale, slopes, stream=None):
    """One ring step: fold a K/V chunk into the state."""
    dims = _lib.dims_of(q_loc, k_blk)
    _lib.ra_step_fwd(dims, q_loc, k_blk, v_blk, q_pos, k_pos, causal, scale, slopes,
                     state.o_acc, state.m, state.l, stream)


def finalize(state: State, out_dtype, stream=None):
    dims = state.dims
    o = torch.empty(state.o_acc.shape, dtype=out_dtype, device=state.o_acc.device)
    lse = torch.empty(state.m.shape, dtype=torch.float32, device=state.m.device)
    _lib.ra_finalize(dims, state.o_acc, state.m, state.l, o, lse, stream)
    return o, lse


def forward(q_loc, k_ch, v_ch, pos, rank: int, causal: bool, scale: float, slopes=None,
            chunks=None, stream=None):
    """Run rank `rank`'s ring: fold the chunks in ring order (or the given
    chunk list) and normalise. Returns O [B,Hq,C,D] (input dtype) and LSE
    [B,Hq,C] (fp32)."""
    n = k_ch.shape[0]
    order = ring_schedule(n, rank) if chunks is None else list(chunks)
    # A chunk folded in twice, or one out of range, would be counted wrongly
    # without any error: every chunk is visited at most once.
    if len(set(order)) != len(order) or not all(0 <= s < n for s in order):
        raise ValueError(f"chunk order {order} must visit each of the {n} chunks at most once")
    state = State(_lib.dims_of(q_loc, k_ch[0]), q_loc.device, stream)
    for s in order:
        fold(state, q_loc, k_ch[s], v_ch[s], pos[rank], pos[s], causal, scale, slopes, stream)
    return finalize(state, q_loc.dtype, stream)


def backward(q_loc, k_ch, v_ch, pos, rank: int, causal: bool, scale: float, slopes, o, lse, d_o,
             stream=None):
    """Backward of rank `rank`'s share: dQ [B,Hq,C,D] and per-chunk dK, dV
    [N,B,Hkv,C,D] (fp32), one ra_step_bwd per chunk in ring order."""
    n = k_ch.shape[0]
    dims = _lib.dims_of(q_loc, k_ch[0])
    delta = torch.empty(lse.shape, dtype=torch.float32, device=q_loc.device)
    _lib.ra_bwd_delta(dims, o, d_o, delta, stream)
    dq = torch.zeros(q_loc.shape, dtype=torch.float32, device=q_loc.device)
    dk = torch.zeros(k_ch.shape, dtype=torch.float32, device=q_loc.device)
    dv = torch.zeros(k_ch.shape, dtype=torch.float32, device=q_loc.device)
    for s in ring_schedule(n, rank):
        _lib.ra_step_bwd(dims, q_loc, k_ch[s], v_ch[s], pos[rank], pos[s], causal, scale, slopes,
                         d_o, lse, delta, dq, dk[s], dv[s], stream)
    return dq, dk, dv
