"""Fixed-bucket graph replay of the padded forward (pack -> fused-QKV attention ->
unpack), for short batches whose cost is the host's kernel launches.

Source: packed-encoders README, "CUDA graphs": a bucketed runner over padded
(batch, length) shapes turns the forward into one replay; packed graphs take
explicit batch and sequence bounds; shapes outside every bucket run eagerly.

A bucket owns the static device buffers its captured graph reads and writes.
The caller writes a batch into ``bucket.lengths`` / ``bucket.qkv_grid`` (or lets
:meth:`ForwardBucket.run` copy it there), replays, and reads ``bucket.out_grid``.
All computation is the library's kernels; this module only holds buffers.
"""
from __future__ import annotations

import torch

from . import pe


def bucket_shape(num_seqs: int, max_seq_len: int, pad_to: int = 64) -> tuple[int, int]:
    """(slots, length bound) of the bucket serving a batch: slots rounded up to a
    power of two (at least 8), the length bound up to a multiple of pad_to."""
    slots = 8
    while slots < num_seqs:
        slots *= 2
    return slots, -(-max_seq_len // pad_to) * pad_to


class ForwardBucket:
    """Buffers and the captured forward of one (slots, max_seq_len) bucket."""

    def __init__(self, slots: int, max_seq_len: int, num_heads: int, head_dim: int, dtype: torch.dtype,
                 softmax_scale: float, window: int = -1, with_lse: bool = False, device="cuda"):
        self.slots, self.max_seq_len = slots, max_seq_len
        cap = slots * max_seq_len
        self.lengths = torch.ones(slots, dtype=torch.int32, device=device)
        self.qkv_grid = torch.zeros(slots, max_seq_len, 3, num_heads, head_dim, dtype=dtype, device=device)
        self.cu_seqlens = torch.zeros(slots + 1, dtype=torch.int32, device=device)
        self.qkv_packed = torch.empty(cap, 3, num_heads, head_dim, dtype=dtype, device=device)
        self.out_packed = torch.empty(cap, num_heads, head_dim, dtype=dtype, device=device)
        self.lse = torch.empty(num_heads, cap, dtype=torch.float32, device=device) if with_lse else None
        self.out_grid = torch.empty(slots, max_seq_len, num_heads, head_dim, dtype=dtype, device=device)
        self.status = torch.zeros(2, dtype=torch.int64, device=device)
        code = {torch.bfloat16: pe.PE_BF16, torch.float16: pe.PE_FP16}.get(dtype, pe.PE_FP32)
        self.workspace = pe.workspace(
            pe.pe_forward_graph_workspace_size(slots, max_seq_len, num_heads, head_dim, code), device)
        torch.cuda.synchronize(device)  # the buffers exist before the capture records their addresses
        self.graph = pe.pe_forward_graph_create(self.lengths, self.qkv_grid, softmax_scale, window,
                                                self.cu_seqlens, self.qkv_packed, self.out_packed, self.lse,
                                                self.out_grid, self.status, self.workspace)

    def replay(self) -> None:
        pe.pe_graph_launch(self.graph)

    def run(self, lengths: torch.Tensor, qkv_grid: torch.Tensor) -> torch.Tensor:
        """Copies a batch (B <= slots sequences, grid [B, S, 3, H, d] with S <= the
        bound) into the bucket, replays, and returns the view out_grid[:B, :S]."""
        B, S = qkv_grid.shape[:2]
        if B > self.slots or S > self.max_seq_len:
            raise ValueError(f"batch ({B}, {S}) does not fit bucket ({self.slots}, {self.max_seq_len})")
        self.lengths[:B].copy_(lengths)
        self.lengths[B:].fill_(1)       # unused slots: one-token sequences, independent of the real ones
        self.qkv_grid[:B, :S].copy_(qkv_grid)
        self.replay()
        return self.out_grid[:B, :S]

    def close(self) -> None:
        if self.graph:
            pe.pe_graph_destroy(self.graph)
            self.graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
