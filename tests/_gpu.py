"""Helpers for the GPU tests: move a seeded tick to the device, run it through
the C ABI (via the thin binding), bring results back, and compare with the
oracle at the stated tolerances."""

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_page_amd as pa
from paged_kv_cache_page_amd import workloads as W

DEV = "cuda:0"

# Tolerances (attention outputs against the unrounded float64 oracle):
#   fp32: max |gpu - oracle| / max |oracle| <= 1e-5 (norm-wise relative)
#   bf16 (bf16 inputs, fp32 accumulation, bf16 output): max abs <= 2e-2, mean abs <= 1e-2
F32_REL = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 1e-2


def say(*a):
    """Name the case before each GPU step, flushed, so a crash log shows it."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def storage_tensor(a, dtype):
    """Host storage array (float32, or bf16 bits as uint16) -> GPU tensor."""
    if dtype == W.F32:
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)
    t = torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16)


def host_storage(t, dtype):
    """GPU tensor -> host storage array (float32, or bf16 bits as uint16)."""
    t = t.detach().cpu()
    if dtype == W.F32:
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_f32(t):
    return t.detach().float().cpu().numpy()


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


class DevTick:
    """A tick's tensors on the device."""

    def __init__(self, tick):
        self.t = tick
        self.q = storage_tensor(tick.q, tick.dtype)
        self.k = storage_tensor(tick.k, tick.dtype) if tick.k is not None else None
        self.v = storage_tensor(tick.v, tick.dtype) if tick.v is not None else None
        self.k_pool = storage_tensor(tick.k_pool, tick.dtype)
        self.v_pool = storage_tensor(tick.v_pool, tick.dtype)
        self.block_tables = i32(tick.block_tables)
        self.seq_lens = i32(tick.seq_lens)
        self.qsl = i32(tick.qsl)
        self.positions = i32(tick.positions)
        self.table = None
        self.slots = None

    def oracle_table(self):
        """The oracle's cos/sin table on the device (None without RoPE): the
        call input both sides share, so that the rotated q/k and the stored K
        can be compared bit for bit. The library's own table builder is
        checked against this table separately."""
        t = self.t
        if t.theta is None:
            return None
        return torch.from_numpy(oracle.rope_table(t.max_pos, t.D, t.theta)).to(DEV)

    def write(self):
        """Table (the oracle's, if RoPE), slot mapping, RoPE + page write.
        Returns self."""
        t = self.t
        if t.theta is not None:
            self.table = self.oracle_table()
        self.slots = pa.pa_compute_slot_mapping(self.block_tables, self.qsl, self.positions,
                                                t.P, t.num_pages)
        if not t.new_in_pool:
            pa.pa_rope_and_cache_write(self.q, self.k, self.v, self.positions, self.slots,
                                       self.table, self.k_pool, self.v_pool)
        return self

    def attend(self, kv_split_tokens=0, max_query_len=None, max_seq_len=None):
        t = self.t
        return pa.pa_paged_attention_varlen(
            self.q, self.k_pool, self.v_pool, self.block_tables, self.seq_lens, self.qsl,
            max_query_len if max_query_len is not None else t.max_query_len,
            max_seq_len if max_seq_len is not None else t.max_seq_len, scale=t.scale,
            kv_split_tokens=kv_split_tokens)


def run_gpu_tick(tick, kv_split_tokens=0):
    d = DevTick(tick).write()
    out = d.attend(kv_split_tokens)
    torch.cuda.synchronize()
    return d, out


def fp32_errors(g, ref):
    """Relative errors of a float32 output against the float64 oracle:
    norm-wise (max |g - o| / max |o| over the config), per output row (the
    same ratio within each (token, head) row of D values, worst row), and
    elementwise where |o| > 1e-3 and where |o| >= 0.1."""
    err = np.abs(g - ref)
    rel = err.max() / max(np.abs(ref).max(), 1e-30)
    row_scale = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    row = (err.max(axis=-1) / row_scale).max()

    def elem_where(mask):
        return float((err[mask] / np.abs(ref[mask])).max()) if mask.any() else 0.0
    return (float(rel), float(row), elem_where(np.abs(ref) > 1e-3),
            elem_where(np.abs(ref) >= 0.1))


def check_attention(got, ref, dtype, where=""):
    """got: GPU output tensor; ref: float64 oracle output. Returns error stats.

    float32: the norm-wise and the per-row relative error, and the
    elementwise relative error where |o| >= 0.1, must each be at most 1e-5.
    The elementwise error where |o| > 1e-3 is reported: float32 sums over
    hundreds of keys leave an absolute error near 1e-7 of the row's scale, so
    an element of 1e-3 carries about 1e-4 relative error whatever the
    kernel."""
    g = host_f32(got).astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{where}: non-finite GPU output"
    err = np.abs(g - ref)
    if dtype == W.F32:
        rel, row, elem, elem_big = fp32_errors(g, ref)
        say(f"{where}: fp32 relative error norm-wise {rel:.3e}, worst row {row:.3e}, "
            f"elementwise (|o| > 1e-3) {elem:.3e}, elementwise (|o| >= 0.1) {elem_big:.3e}")
        assert rel <= F32_REL, f"{where}: fp32 norm-wise relative error {rel:.3e} > {F32_REL}"
        assert row <= F32_REL, f"{where}: fp32 per-row relative error {row:.3e} > {F32_REL}"
        assert elem_big <= F32_REL, (f"{where}: fp32 elementwise relative error (|o| >= 0.1) "
                                     f"{elem_big:.3e} > {F32_REL}")
        return {"rel": rel, "row_rel": row, "elem_rel": elem, "elem_rel_big": elem_big}
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= BF16_MAX_ABS, f"{where}: bf16 max abs error {mx:.4e} > {BF16_MAX_ABS}"
    assert mean <= BF16_MEAN_ABS, f"{where}: bf16 mean abs error {mean:.4e} > {BF16_MEAN_ABS}"
    return {"max_abs": mx, "mean_abs": mean}
