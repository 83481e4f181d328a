"""Shared helpers of the GPU parity tests (device transfers, chunked oracle
logits, comparisons).  Not a test module."""
import sys

import numpy as np
import torch

from oracle import bf16 as obf16
from oracle import rules


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_bf16(bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def oracle_logits_bf16(h_bits, w_bits, chunk=16384):
    """float64 logits of bf16 hidden rows [R, d] against a bf16 table [V, d]:
    oracle.rules.lm_head_logits applied to column blocks of the table."""
    h = obf16.bf16_to_f64(h_bits.reshape(-1, h_bits.shape[-1]))
    V = w_bits.shape[0]
    out = np.empty((h.shape[0], V))
    for v0 in range(0, V, chunk):
        out[:, v0:v0 + chunk] = rules.lm_head_logits(h, obf16.bf16_to_f64(w_bits[v0:v0 + chunk]))
    return out.reshape(h_bits.shape[:-1] + (V,))


def row_rel_err(gpu, ref):
    """max_v |gpu - ref| / max_v |ref| per row."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return np.abs(g - r).max(axis=-1) / np.maximum(np.abs(r).max(axis=-1), 1e-30)


def compare_decisions(n_gpu, tok_gpu, n_ref, tok_ref, flagged, label=""):
    """Bit-exact n and tokens except on flagged sequences.  Returns (#mismatch, #flagged)."""
    n_gpu = np.asarray(n_gpu).astype(np.int64)
    tok_gpu = np.asarray(tok_gpu).astype(np.int64)
    same = (n_gpu == n_ref) & np.all(tok_gpu == tok_ref, axis=1)
    bad = ~same & ~flagged
    if np.any(bad):
        i = int(np.nonzero(bad)[0][0])
        raise AssertionError(f"{label}: {int(bad.sum())} unflagged mismatches; first b={i}: "
                             f"gpu n={n_gpu[i]} tok={tok_gpu[i].tolist()} ref n={n_ref[i]} tok={tok_ref[i].tolist()}")
    return int((~same).sum()), int(flagged.sum())


def check_token_structure(n, tok, gamma):
    n = np.asarray(n)
    tok = np.asarray(tok)
    for b in range(len(n)):
        k = int(n[b])
        assert 0 <= k <= gamma
        assert np.all(tok[b, :k + 1] >= 0)
        assert np.all(tok[b, k + 1:] == -1)
