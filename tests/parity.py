"""Shared helpers of the GPU parity tests: run a workload on the GPU through
libpa and on the CPU through the oracle, and compare."""

from __future__ import annotations

import numpy as np
import torch

from oracle import run
from paged_kv_cache_219_amd.kernels import (pa_decode, pa_decode_shared_prefix, pa_prefill_chunk,
                                            pa_prefix_plan)
from paged_kv_cache_219_amd.workload import DeviceWorkload, to_host_bits

# Tolerances for the attention output: fp32 inputs max |err| <= 1e-5; bf16
# inputs (fp32 accumulation) max |err| <= 2e-2 and relative L2 <= 5e-3.
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def say(msg: str):
    print(msg, flush=True)


def assert_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, mask=None, what=""):
    g = gpu.float().cpu().numpy().astype(np.float64)
    if mask is not None:
        g, ref = g[mask], ref[mask]
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - ref)
    mx = float(err.max()) if err.size else 0.0
    if dtype == "f32":
        assert mx <= F32_MAX_ABS, f"{what}: max abs err {mx:.3e} > {F32_MAX_ABS}"
        return mx, None
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    assert mx <= BF16_MAX_ABS, f"{what}: max abs err {mx:.3e} > {BF16_MAX_ABS}"
    assert rel <= BF16_REL_L2, f"{what}: rel L2 err {rel:.3e} > {BF16_REL_L2}"
    return mx, rel


def raw_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_pool_equal(w: DeviceWorkload, st) -> None:
    gk, gv = to_host_bits(w.k_cache), to_host_bits(w.v_cache)
    assert gk.shape == st.k_cache.shape and gv.shape == st.v_cache.shape
    assert np.array_equal(raw_bits(gk), raw_bits(st.k_cache)), "k_cache differs from the oracle"
    assert np.array_equal(raw_bits(gv), raw_bits(st.v_cache)), "v_cache differs from the oracle"


def gpu_step(script, partition=None, scale=None, step=0, workload=None, shared_prefix=None,
             find_shared=False):
    """Run the script's setup and step on the GPU; return (workload, out,
    host tables, host lens).  ``shared_prefix`` = (max_members, min_prefix)
    runs decode through pa_decode_shared_prefix with the groups
    pa_prefix_plan finds (kept in ``w.prefix_plan``); ``find_shared`` runs it
    through pa_decode with PA_DECODE_FIND_SHARED."""
    w = workload or DeviceWorkload(script)
    w.run_step()
    bt, lens, bt_h, lens_h = w.batch_tables()
    q = w.queries(step)
    out = torch.empty_like(q)
    s = script.spec
    sc = s.scale if scale is None else scale
    if s.kind == "decode":
        part = s.partition if partition is None else partition
        if shared_prefix is None:
            pa_decode(out, q, w.k_cache, w.v_cache, bt, lens, sc, part, int(max(lens_h.max(), 0)),
                      check_device_args=True, find_shared=find_shared)
        else:
            groups, pre, mp = pa_prefix_plan(bt_h, lens_h, *shared_prefix)
            w.prefix_plan = (groups, pre, mp)
            pa_decode_shared_prefix(out, q, w.k_cache, w.v_cache, bt, lens, sc, part,
                                    int(max(lens_h.max(), 0)),
                                    torch.from_numpy(groups).to(q.device),
                                    torch.from_numpy(pre).to(q.device), mp,
                                    check_device_args=True)
    else:
        pa_prefill_chunk(out, q, w.k_cache, w.v_cache, bt, w.query_start_loc(), lens,
                         max(script.query_lens), sc, check_device_args=True)
    torch.cuda.synchronize()
    return w, out, bt_h, lens_h


def oracle_step(script, scale=None, select=None, only_seqs=None, step=0):
    st = run.build(script, only_seqs=only_seqs)
    q = script.q(step)
    if scale is not None:
        from oracle import attention
        s = script.spec
        tables, lens = run.batch_tables(st, script)
        if s.kind == "decode":
            ref = attention.decode(q, st.k_cache, st.v_cache, tables, lens, scale, s.dtype, select)
        else:
            qsl = np.concatenate([[0], np.cumsum(script.query_lens)]).astype(np.int32)
            ref = attention.prefill(q, st.k_cache, st.v_cache, tables, qsl, lens, scale, s.dtype, select)
        return st, ref
    return st, run.step_output(st, script, q, select)
