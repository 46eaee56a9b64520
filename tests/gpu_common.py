"""Helpers for the GPU parity tests: upload a seeded workload, run the HIP
path through the C ABI, and compare with the oracle."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as G
import oracle.reference as R

# Tolerances for the decode outputs against the fp64 oracle.
O_ATOL_BF16 = 2e-2
O_ATOL_FP8 = 6e-2
LSE_ATOL = 1e-3
# Stricter internal gates (bf16 output rounding plus bf16 softmax weights
# bound the error well below these).
O_REL_L2 = 1e-2
O_COSINE = 0.9999


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def i32(x, device="cuda"):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def f32(x, device="cuda"):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


class Uploaded:
    """A workload's inputs on the device plus the matching params."""

    def __init__(self, w: gi.Workload, *, kv_chunk=0, gate_mode=None, softmax_scale=None, math="auto",
                 device="cuda"):
        s = w.spec
        self.w = w
        fp8 = s.kv_dtype in (gi.KV_FP8, gi.KV_INT8)   # one-byte codes
        self.q = bf16_tensor(w.q, device)
        if fp8:
            self.k = torch.from_numpy(np.ascontiguousarray(w.k_cache)).to(device)
            self.v = torch.from_numpy(np.ascontiguousarray(w.v_cache)).to(device)
        else:
            self.k = bf16_tensor(w.k_cache, device)
            self.v = bf16_tensor(w.v_cache, device)
        self.seqlens = i32(w.seqlens, device) if s.layout != "ragged" else None
        self.cu = i32(w.cu_seqlens, device)
        self.bt = i32(w.block_table, device)
        self.topk = i32(w.topk_idx, device)
        self.ks = f32(w.k_scale, device)
        self.vs = f32(w.v_scale, device)
        self.gate_mode = gate_mode or ("elementwise" if w.gate is not None else "none")
        if w.gate is not None:
            g = w.gate if self.gate_mode == "elementwise" else np.ascontiguousarray(w.gate[..., 0])
            self.gate = bf16_tensor(g, device)
        else:
            self.gate = None
        B, Sq, Hq, d = s.batch, s.s_q, s.h_q, s.head_dim
        if s.layout == "contiguous":
            cap = w.k_cache.shape[1]
            kv_rows, mpp = B * cap, 0
        elif s.layout == "ragged":
            cap, kv_rows, mpp = 0, w.k_cache.shape[0], 0
        else:
            cap, mpp = 0, w.block_table.shape[1]
            kv_rows = w.k_cache.shape[0] * s.page_size
        self.params = G.make_params(
            batch=B, s_q=Sq, h_q=Hq, h_kv=s.h_kv, head_dim=d, layout=s.layout, kv_dtype=s.kv_dtype,
            causal=s.causal, max_seqlen_kv=w.max_seqlen, seq_capacity=cap, kv_rows=max(kv_rows, 1),
            page_size=s.page_size, max_pages_per_seq=max(mpp, 1) if s.layout == "paged" else 0,
            topk=s.topk, gate_mode=self.gate_mode, softmax_scale=softmax_scale, kv_chunk=kv_chunk, math=math)
        self.plan = G.gqa_decode_make_plan(self.params)
        ws = self.plan["workspace_bytes"]
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.o = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device)

    def run(self, stream=None):
        G.gqa_decode_run(self.params, self.q, self.k, self.v, self.seqlens, self.cu, self.bt, self.topk,
                         self.ks, self.vs, self.gate, self.o, self.lse, self.ws, self.ws.numel(), stream)
        return self.o, self.lse

    def result(self):
        torch.cuda.synchronize()
        return self.o.float().cpu().numpy().astype(np.float64), self.lse.cpu().numpy().astype(np.float64)


def oracle(w: gi.Workload, gate_mode="elementwise", softmax_scale=None, rows=None):
    arrays = w.arrays()
    gm = gate_mode
    if w.gate is not None and gate_mode == "headwise":
        arrays = dict(arrays)
        arrays["gate"] = np.ascontiguousarray(w.gate[..., 0])
    return R.reference_decode(**arrays, **w.params(), gate_mode=gm, softmax_scale=softmax_scale, rows=rows)


def compare(O, LSE, Oref, Lref, *, fp8=False, mask=None, label=""):
    """Assert the HIP outputs match the oracle; returns the error stats."""
    if mask is None:
        mask = np.isfinite(Lref) | np.isneginf(Lref)
    # fully masked rows: O = 0, LSE = -inf on both sides
    ninf = np.isneginf(Lref)
    assert np.array_equal(np.isneginf(LSE)[ninf], ninf[ninf]), f"{label}: LSE not -inf where nothing is visible"
    assert not np.isnan(O).any() and not np.isnan(LSE).any(), f"{label}: NaN in output"
    fin = np.isfinite(Lref)
    assert np.array_equal(np.isfinite(LSE), fin), f"{label}: LSE finiteness differs"
    lse_err = float(np.abs(LSE[fin] - Lref[fin]).max()) if fin.any() else 0.0
    # rows of O that the oracle computed
    orow = np.isfinite(Oref).all(axis=-1)
    d_o = O[orow] - Oref[orow]
    o_err = float(np.abs(d_o).max()) if d_o.size else 0.0
    nref = float(np.linalg.norm(Oref[orow]))
    rel = float(np.linalg.norm(d_o) / nref) if nref > 0 else float(np.linalg.norm(d_o))
    a = O[orow].ravel()
    b = Oref[orow].ravel()
    na, nb = float(np.linalg.norm(a)), float(np.linalg.norm(b))
    cos = float(a @ b / (na * nb)) if na > 0 and nb > 0 else (1.0 if na == nb else 0.0)
    stats = dict(o_max_abs=o_err, lse_max_abs=lse_err, o_rel_l2=rel, o_cosine=cos)
    log(f"  [{label}] {stats}")
    atol = O_ATOL_FP8 if fp8 else O_ATOL_BF16
    assert o_err <= atol, f"{label}: O max abs err {o_err} > {atol}"
    assert lse_err <= LSE_ATOL, f"{label}: LSE max abs err {lse_err} > {LSE_ATOL}"
    if nref > 1e-6:
        assert rel <= O_REL_L2, f"{label}: O relative L2 err {rel} > {O_REL_L2}"
        assert cos >= O_COSINE, f"{label}: O cosine {cos} < {O_COSINE}"
    return stats


def check_workload(w: gi.Workload, *, kv_chunk=0, gate_mode=None, softmax_scale=None, math="auto", label=""):
    up = Uploaded(w, kv_chunk=kv_chunk, gate_mode=gate_mode, softmax_scale=softmax_scale, math=math)
    up.run()
    O, LSE = up.result()
    Oref, Lref = oracle(w, gate_mode=up.gate_mode, softmax_scale=softmax_scale)
    return compare(O, LSE, Oref, Lref, fp8=w.spec.kv_dtype in (gi.KV_FP8, gi.KV_INT8), label=label or w.spec.name)
