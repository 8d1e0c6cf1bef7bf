"""Segment-wise HGA over a long sequence (truncated backpropagation through time).

Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
differently": the sequence is cut into segments (2,048 tokens there) that run
forward and backward one after another; the summaries of earlier chunks stay
resident, later segments still route to and attend the exact tokens of
earlier ones, and the earlier keys and values are detached, so no gradient
reaches them.

``SegmentRunner`` holds one attention layer's key/value history and its chunk
and group summaries in buffers sized once for the whole sequence (the shape's
``kv_capacity``).  For segment ``i`` (positions ``[i*S, (i+1)*S)``) it

1. appends the summaries of the segment's chunks (``hga_build_summaries``
   over chunks ``[i*S/64, (i+1)*S/64)``; the older ones are not rebuilt);
2. routes the segment's queries over everything up to the segment's end
   (``kv_len = (i+1)*S``);
3. runs the exact-token attention forward;
4. runs the backward: dQ of the segment's queries, and dK, dV of the
   segment's own keys only (``hga_attend_bwd_dkdv_range``): history rows of
   dK, dV are neither computed nor written.

Every step is a call of the C ABI; this module only sequences them and owns
the buffers.  The caller writes a segment's keys and values into
``k_history[:, :, i*S:(i+1)*S]`` (and the same for ``v_history``) before
calling ``step(i, ...)``.

With ``causal=True`` the routing is the strictly causal variant
(``hga_route_causal``): block j of a segment is routed with the mean of the 64
queries before it.  For a segment's first block those are the last 64 queries
of the previous segment, which the runner keeps from the previous ``forward``.

With ``kv_on_host=True`` the key/value history lives in pinned host memory
(the page's RAM tier, same section): the summaries stay in GPU memory, and the
kernels fetch only the rows they gather (the kept groups, the own chunk, the
segment's keys for its dK/dV) across the host link.

With ``stage=True`` each segment's routed working set is staged into device
memory once, after its routing (``hga_stage_routed_from``): the distinct
history groups its rows kept and the segment's own rows go into a compact
device buffer, the routing rows are rewritten against it, and the attention
and backward run there.  Two such buffers alternate: a group that the
previous segment's staging already holds (in its union or among its own
rows) is copied from there, in device memory, so only the groups no earlier
staging held cross the host link.  When ``step`` is given the segment's keys
and values in device memory (``K_seg``, ``V_seg``: the active segment, as a
projection produces it), the segment's summaries are built and its rows
staged from those.  Results
equal the unstaged ones bit for bit.
"""
from __future__ import annotations

import contextlib
from dataclasses import dataclass

from . import (CHUNK, hga_attend_bwd_dkdv_range, hga_attend_bwd_dq, hga_attend_bwd_workspace,
               hga_attend_fwd, hga_build_summaries, hga_build_summaries_rows, hga_route,
               hga_route_causal, hga_stage_min_groups, hga_stage_routed_from,
               hga_stage_workspace, make_shape)


@dataclass
class SegmentResult:
    O: object            # [B, Hq, S, D]
    lse: object          # [B, Hq, S]
    group_idx: object    # [B, Hq, S/64, top_g]
    dQ: object           # [B, Hq, S, D]
    dK: object           # view [B, Hkv, S, D] of the segment's rows
    dV: object           # view [B, Hkv, S, D] of the segment's rows


class SegmentRunner:
    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, seq_len: int,
                 seg_len: int, top_k: int, top_g: int, dtype: str = "bf16",
                 softmax_scale: float = 0.0, device="cuda:0", kv_on_host: bool = False,
                 causal: bool = False, stage: bool = False):
        import torch
        if seg_len % CHUNK or seq_len % seg_len:
            raise ValueError("seg_len must be a multiple of 64 dividing seq_len")
        self.B, self.Hq, self.Hkv, self.D = batch, n_q_heads, n_kv_heads, head_dim
        self.L, self.S, self.top_k, self.top_g = seq_len, seg_len, top_k, top_g
        self.dtype, self.scale = dtype, softmax_scale
        self.nseg = seq_len // seg_len
        self.causal = causal
        elt = torch.bfloat16 if dtype == "bf16" else torch.float32
        f32, i32 = torch.float32, torch.int32
        kv = (batch, n_kv_heads, seq_len, head_dim)
        q = (batch, n_q_heads, seg_len, head_dim)
        nblk = seg_len // 64
        if kv_on_host:
            self.k_history = torch.zeros(kv, dtype=elt, pin_memory=True)
            self.v_history = torch.zeros(kv, dtype=elt, pin_memory=True)
        else:
            self.k_history = torch.zeros(kv, dtype=elt, device=device)
            self.v_history = torch.zeros(kv, dtype=elt, device=device)
        self.chunk_mean = torch.zeros(batch, n_kv_heads, seq_len // 64, head_dim, dtype=f32,
                                      device=device)
        self.group_mean = torch.zeros(batch, n_kv_heads, seq_len // 8, head_dim, dtype=f32,
                                      device=device)
        self.chunk_idx = torch.empty(batch, n_q_heads, nblk, top_k, dtype=i32, device=device)
        self.group_idx = torch.empty(batch, n_q_heads, nblk, top_g, dtype=i32, device=device)
        self.O = torch.empty(q, dtype=elt, device=device)
        self.lse = torch.empty(batch, n_q_heads, seg_len, dtype=f32, device=device)
        self.dQ = torch.empty(q, dtype=elt, device=device)
        self.dK = torch.zeros(kv, dtype=elt, device=device)
        self.dV = torch.zeros(kv, dtype=elt, device=device)
        # strictly causal routing: the last 64 queries of the previous segment
        self.q_prev = torch.zeros(batch, n_q_heads, CHUNK, head_dim, dtype=elt, device=device) \
            if causal else None
        # the last segment needs the largest workspace (longest history)
        self.workspace = torch.empty(hga_attend_bwd_workspace(self.shape(self.nseg - 1)),
                                     dtype=torch.uint8, device=device)
        self.stage = stage
        self._cur = 0
        self._last_staged = -1   # segment staged last (a staging source only for the next one)
        if stage:
            # the staged history of the last segment is the largest the bound
            # allows: every history group, or every row's top_g
            sg_max = max(hga_stage_min_groups(self.shape(i)) for i in range(self.nseg))
            self.stage_cap = -(-(8 * sg_max + seg_len) // 64) * 64
            st = (batch, n_kv_heads, self.stage_cap, head_dim)
            # two staging buffers, segments alternate between them; each
            # segment's staging copies from the other what it already holds
            self.k_stages = [torch.empty(st, dtype=elt, device=device) for _ in range(2)]
            self.v_stages = [torch.empty(st, dtype=elt, device=device) for _ in range(2)]
            self.dk_stage = torch.empty(st, dtype=elt, device=device)
            self.dv_stage = torch.empty(st, dtype=elt, device=device)
            self.group_idx_staged = torch.empty_like(self.group_idx)
            self.stage_wss = [torch.empty(max(256, hga_stage_workspace(self.shape(self.nseg - 1),
                                                                       sg_max)),
                                          dtype=torch.uint8, device=device) for _ in range(2)]
            big = make_shape(batch, n_q_heads, n_kv_heads, head_dim, seg_len, self.stage_cap,
                             top_k, top_g, dtype=dtype, softmax_scale=softmax_scale)
            self.workspace = torch.empty(max(self.workspace.numel(),
                                             hga_attend_bwd_workspace(big)),
                                         dtype=torch.uint8, device=device)
            self.stage_groups = [hga_stage_min_groups(self.shape(i)) for i in range(self.nseg)]

    def shape(self, i: int):
        """Shape of segment i: q_len = S at the end of kv_len = (i+1) S."""
        return make_shape(self.B, self.Hq, self.Hkv, self.D, self.S, (i + 1) * self.S,
                          self.top_k, self.top_g, dtype=self.dtype,
                          softmax_scale=self.scale, kv_capacity=self.L)

    def staged_shape(self, i: int):
        """Shape of segment i over its staged working set."""
        return make_shape(self.B, self.Hq, self.Hkv, self.D, self.S,
                          8 * self.stage_groups[i] + self.S, self.top_k, self.top_g,
                          dtype=self.dtype, softmax_scale=self.scale,
                          kv_capacity=self.stage_cap)

    @property
    def k_stage(self):
        return self.k_stages[self._cur]

    @property
    def v_stage(self):
        return self.v_stages[self._cur]

    def forward(self, i: int, Q, stream=None, K_seg=None, V_seg=None):
        """Steps 1-3 for segment i (its keys/values already in the history;
        K_seg / V_seg optionally the same rows in device memory, from which the
        segment's summaries and, with ``stage``, its staged rows are taken)."""
        s = self.shape(i)
        c0, c1 = i * self.S // CHUNK, (i + 1) * self.S // CHUNK
        if K_seg is not None:
            # the segment's summaries from its rows in device memory
            hga_build_summaries_rows(s, K_seg, i * self.S, self.chunk_mean, self.group_mean,
                                     c0, c1, stream=stream)
        else:
            hga_build_summaries(s, self.k_history, self.chunk_mean, self.group_mean, c0, c1,
                                stream=stream)
        if self.causal:
            hga_route_causal(s, Q, self.q_prev if i > 0 else None, self.chunk_mean,
                             self.group_mean, self.chunk_idx, self.group_idx, stream=stream)
        else:
            hga_route(s, Q, self.chunk_mean, self.group_mean, self.chunk_idx, self.group_idx,
                      stream=stream)
        if self.stage:
            cur = i % 2
            prev = None
            if i > 0 and self._last_staged == i - 1:
                # the previous segment's staging, in the other buffer
                prev = dict(K_stage=self.k_stages[1 - cur], V_stage=self.v_stages[1 - cur],
                            workspace=self.stage_wss[1 - cur],
                            stage_groups=self.stage_groups[i - 1], q0=(i - 1) * self.S,
                            q_len=self.S)
            self._cur = cur
            hga_stage_routed_from(s, self.group_idx, self.k_history, self.v_history,
                                  self.stage_groups[i], self.k_stage, self.v_stage,
                                  self.group_idx_staged, self.stage_wss[cur], K_seg=K_seg,
                                  V_seg=V_seg, prev=prev, stream=stream)
            self._last_staged = i
            hga_attend_fwd(self.staged_shape(i), Q, self.k_stage, self.v_stage,
                           self.group_idx_staged, self.O, self.lse, stream=stream)
        else:
            hga_attend_fwd(s, Q, self.k_history, self.v_history, self.group_idx, self.O,
                           self.lse, stream=stream)
        if self.causal:
            # the next segment's first block routes with this segment's last 64 queries
            import torch
            with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
                self.q_prev.copy_(Q[:, :, -CHUNK:])

    def backward(self, i: int, Q, dO, stream=None):
        """Step 4 for segment i, after forward(i, Q): dQ, and dK, dV of the
        segment's own keys (history detached)."""
        if self.stage:
            import torch
            s = self.staged_shape(i)
            c0 = self.stage_groups[i] // 8
            c1 = c0 + self.S // CHUNK
            hga_attend_bwd_dq(s, Q, self.k_stage, self.v_stage, self.O, self.lse, dO,
                              self.group_idx_staged, self.dQ, self.workspace, stream=stream)
            hga_attend_bwd_dkdv_range(s, Q, self.k_stage, self.v_stage, self.lse, dO,
                                      self.group_idx_staged, c0, c1, self.dk_stage,
                                      self.dv_stage, self.workspace, stream=stream)
            rows = slice(i * self.S, (i + 1) * self.S)
            srows = slice(64 * c0, 64 * c1)
            with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
                self.dK[:, :, rows].copy_(self.dk_stage[:, :, srows])
                self.dV[:, :, rows].copy_(self.dv_stage[:, :, srows])
            return
        s = self.shape(i)
        c0, c1 = i * self.S // CHUNK, (i + 1) * self.S // CHUNK
        hga_attend_bwd_dq(s, Q, self.k_history, self.v_history, self.O, self.lse, dO,
                          self.group_idx, self.dQ, self.workspace, stream=stream)
        hga_attend_bwd_dkdv_range(s, Q, self.k_history, self.v_history, self.lse, dO,
                                  self.group_idx, c0, c1, self.dK, self.dV, self.workspace,
                                  stream=stream)

    def step(self, i: int, Q, dO, stream=None, K_seg=None, V_seg=None) -> SegmentResult:
        self.forward(i, Q, stream, K_seg=K_seg, V_seg=V_seg)
        self.backward(i, Q, dO, stream)
        rows = slice(i * self.S, (i + 1) * self.S)
        return SegmentResult(self.O, self.lse, self.group_idx, self.dQ,
                             self.dK[:, :, rows], self.dV[:, :, rows])
