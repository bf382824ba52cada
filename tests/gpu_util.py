"""Helpers shared by the GPU parity tests (host-side conversions and error
measures; no method arithmetic)."""
import sys

import numpy as np


def say(*a):
    """Progress line naming the case before a GPU step (flushed)."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def u16(t):
    """Device int16 tensor holding bf16 bits -> numpy uint16."""
    return t.detach().cpu().numpy().view(np.uint16)


def bf16_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rel_inf(got, ref):
    """max|got - ref| / max|ref| (the bf16/fp8 parity measure)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def decisions_agree(dec_gpu, dec_ref, margin_ref, tau):
    """Decisions must match wherever the oracle's |margin| exceeds tau."""
    dec_gpu = np.asarray(dec_gpu)
    dec_ref = np.asarray(dec_ref)
    sure = np.abs(np.asarray(margin_ref)) > tau
    return bool(np.all(dec_gpu[sure] == dec_ref[sure])), int(sure.sum())
