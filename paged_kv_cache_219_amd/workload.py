"""Run a seeded workload script (``synth``) on the GPU through libpa.

The script's allocator operations go to libpa's block allocator; every
append's K/V rows are copied to the device and written into the returned slots
with ``pa_reshape_and_cache``; a copy-on-write pair reported by the allocator
is applied with ``pa_copy_blocks`` after the writes queued before it.
"""

from __future__ import annotations

import numpy as np
import torch

from ._lib import BlockAllocator, check
from .kernels import new_kv_cache, pa_copy_blocks, pa_reshape_and_cache

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host values (float32, or bf16 bit patterns as uint16) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array of its raw stored values (uint16 bits for bf16)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


class DeviceWorkload:
    def __init__(self, script, device="cuda", poison=True, flush_tokens: int = 1 << 16):
        """``poison``: fill the pool before any write -- True: all-ones bits (NaN
        in fp32 and bf16); a float: that value (e.g. +-1e4); False: leave it."""
        self.script = script
        self.spec = s = script.spec
        self.device = torch.device(device)
        self.dtype = TORCH_DTYPE[s.dtype]
        self.alloc = BlockAllocator(script.num_blocks, s.block_size, script.free_order)
        self.k_cache, self.v_cache = new_kv_cache(script.num_blocks, s.num_kv_heads, s.head_dim,
                                                  self.dtype, self.device, s.block_size)
        if poison is True:  # all-ones bits: NaN in fp32 and bf16
            self.k_cache.view(torch.int16 if s.dtype == "bf16" else torch.int32).fill_(-1)
            self.v_cache.view(torch.int16 if s.dtype == "bf16" else torch.int32).fill_(-1)
        elif poison is not False:
            self.k_cache.fill_(float(poison))
            self.v_cache.fill_(float(poison))
        self.cow_pairs: list = []
        self._flush_tokens = flush_tokens
        self._pending: list = []
        self.run_ops(script.setup)

    # ------------------------------------------------------------- allocator
    def _flush(self):
        if not self._pending:
            return
        slots = np.concatenate([p[0] for p in self._pending]).astype(np.int64)
        k = np.concatenate([p[1] for p in self._pending])
        v = np.concatenate([p[2] for p in self._pending])
        self._pending = []
        dt = self.spec.dtype
        pa_reshape_and_cache(to_device(k, dt, self.device), to_device(v, dt, self.device),
                             self.k_cache, self.v_cache,
                             torch.from_numpy(slots).to(self.device), check_device_args=True)

    def run_ops(self, ops) -> list:
        """Apply allocator ops, write appended tokens; returns slots per append."""
        out = []
        queued = 0
        for op in ops:
            if op.kind == "new":
                check("pa_seq_new", self.alloc.new(op.seq))
            elif op.kind == "fork":
                check("pa_seq_fork", self.alloc.fork(op.parent, op.seq))
            else:
                rc, slots, pairs = self.alloc.append(op.seq, op.n)
                check("pa_seq_append", rc)
                if pairs:
                    self._flush()
                    queued = 0
                    pa_copy_blocks(self.k_cache, self.v_cache,
                                   torch.tensor(pairs, dtype=torch.int32, device=self.device))
                    self.cow_pairs.extend(pairs)
                k, v = self.script.kv(op)
                self._pending.append((np.asarray(slots, np.int64), k, v))
                queued += op.n
                out.append(slots)
                if queued >= self._flush_tokens:
                    self._flush()
                    queued = 0
        self._flush()
        return out

    def run_step(self) -> list:
        return self.run_ops(self.script.step)

    # ------------------------------------------------------------- batch
    def batch_tables(self):
        sc = self.script
        tables, lens = self.alloc.export_tables(sc.batch, sc.max_blocks_per_seq)
        return (torch.from_numpy(tables).to(self.device), torch.from_numpy(lens).to(self.device),
                tables, lens)

    def queries(self, step: int = 0) -> torch.Tensor:
        return to_device(self.script.q(step), self.spec.dtype, self.device)

    def query_start_loc(self) -> torch.Tensor:
        qsl = np.concatenate([[0], np.cumsum(self.script.query_lens)]).astype(np.int32)
        return torch.from_numpy(qsl).to(self.device)
