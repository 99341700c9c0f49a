"""Shared glue for the GPU parity tests: workload -> library rows, workload -> oracle rows,
and the tolerance bars.  Holds no arithmetic of the method."""
import os
import sys

import numpy as np
import torch

import oracle
import sparse_attention_08_amd as dsa
import workloads

# Tolerances (max-abs-relative over one output tensor): indexer 1e-5 in fp32 and 2e-2
# in bf16/fp8, attention 1e-5 in fp32 and 2e-2 in bf16; top-k bit-exact.
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 2e-2}


def say(msg: str):
    """Name the case on stdout before a GPU step (a crash then still says what ran)."""
    sys.stdout.write(f"[case] {msg}\n")
    sys.stdout.flush()


def dev_rows(wl: workloads.Workload) -> dsa.Rows:
    return dsa.Rows(wl.row_seq, wl.row_len, wl.max_row_len, wl.num_seqs, seq_start=wl.seq_start,
                    page_table=wl.page_table)


def oracle_rows(wl: workloads.Workload) -> oracle.Rows:
    h = wl.host_rows()
    return oracle.Rows(h["row_seq"], h["row_len"], seq_start=h["seq_start"],
                       page_table=h["page_table"], page_size=h["page_size"])


def raw(t):
    return workloads.raw_numpy(t)


def gpu_indexer(wl, ld=None):
    rows = dev_rows(wl)
    ld = ld or wl.max_row_len
    logits = torch.full((wl.num_rows, ld), float("nan"), dtype=torch.float32, device=wl.q_idx.device)
    fn = dsa.indexer_logits_paged if wl.paged else dsa.indexer_logits
    fn(rows, wl.q_idx, wl.w, wl.k_idx, logits, q_scale=wl.q_scale, k_scale=wl.k_scale)
    return logits


def oracle_indexer(wl, which=None, ld=None):
    return oracle.indexer(wl.idx_dtype, raw(wl.q_idx), raw(wl.w), raw(wl.k_idx), oracle_rows(wl),
                          q_scale=raw(wl.q_scale), k_scale=raw(wl.k_scale), which=which,
                          ld=ld or wl.max_row_len)


def gpu_mla(wl, idx, lse=True):
    rows = dev_rows(wl)
    out = torch.empty((wl.num_rows, wl.H, wl.D_v), dtype=wl.q.dtype, device=wl.q.device)
    l = torch.empty((wl.num_rows, wl.H), dtype=torch.float32, device=wl.q.device) if lse else None
    if wl.mode == "prefill":
        fn = dsa.sparse_mla_prefill_paged if wl.paged else dsa.sparse_mla_prefill
        fn(rows, wl.q, wl.kv, idx, wl.scale, wl.D_v, out=out, lse=l)
    elif wl.paged:
        dsa.sparse_mla_decode_paged(rows, wl.q, wl.kv, idx, wl.scale, wl.D_v, out=out, lse=l)
    else:
        dsa.sparse_mla_decode(rows, wl.q, wl.kv, idx, wl.scale, wl.D_v, out=out, lse=l)
    return out, l


def oracle_mla(wl, idx_np, which=None):
    return oracle.sparse_mla(wl.mla_dtype, raw(wl.q), raw(wl.kv), idx_np, oracle_rows(wl), wl.scale,
                             wl.D_v, which=which)


def valid_logits(x: np.ndarray, lens, which):
    """Concatenate the valid prefix of each listed row (row i of x is row which[i])."""
    return np.concatenate([x[i, :lens[r]] for i, r in enumerate(which)])


def sorted_sets(idx: np.ndarray) -> np.ndarray:
    return np.sort(idx, axis=-1)

