"""Thin ctypes binding of libquail.so (include/quail.h).

Argument marshalling only: torch tensors are passed as device pointers, host
arrays as ctypes buffers, torch streams as hipStream_t handles. Every step of
the prefill path runs inside the library's HIP kernels; this module computes
nothing. It fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libquail.so")
_lib = None

OK, E_INVAL, E_NOMEM, E_STALE, E_HIP, E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
GUARD_BYTES = 256          # QUAIL_GUARD_BYTES
PROF_KINDS = ("qkv", "o", "gate_up", "down", "attn", "norm", "other")
DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
NO_ANCHOR = -1

_STATUS = {E_INVAL: "E_INVAL", E_NOMEM: "E_NOMEM", E_STALE: "E_STALE", E_HIP: "E_HIP",
           E_UNSUPPORTED: "E_UNSUPPORTED"}


class QuailError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class ModelConfig(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("vocab", C.c_int32), ("rope_theta", C.c_float), ("rms_eps", C.c_float),
                ("kv_dtype", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float),
                ("max_anchor_len", C.c_int32), ("max_suffix_len", C.c_int32),
                ("act_dtype", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("mlp_norm", C.c_void_p),
                ("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("w_gate_up", C.c_void_p),
                ("w_down", C.c_void_p), ("s_qkv", C.c_void_p), ("s_o", C.c_void_p),
                ("s_gate_up", C.c_void_p), ("s_down", C.c_void_p)]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("layers", C.POINTER(LayerWeights)),
                ("final_norm", C.c_void_p), ("head8", C.c_void_p)]


_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_szp = C.POINTER(C.c_size_t)
_vp = C.c_void_p

class Table(C.Structure):
    _fields_ = [("rows", C.c_int32), ("field_tokens", C.c_float)]


class AIJoin(C.Structure):
    _fields_ = [("left", C.c_int32), ("right", C.c_int32), ("anchor_glue", C.c_float),
                ("suffix_glue", C.c_float), ("selectivity", C.c_float), ("symmetric", C.c_int32)]


_f64p = C.POINTER(C.c_double)

_SIGS = {
    "quail_version": ([], C.c_char_p),
    "quail_last_error": ([], C.c_char_p),
    "quail_anchor_bytes": ([C.POINTER(ModelConfig), C.c_int32, _szp], C.c_int32),
    "quail_workspace_bytes": ([C.POINTER(ModelConfig), C.c_int32, _szp], C.c_int32),
    "quail_plan_build": ([C.POINTER(ModelConfig), C.c_size_t, C.c_int32, C.c_int32, _i32p, C.c_int32,
                          _i32p, _i32p, _i32p, _i32p, _i32p, _szp], C.c_int32),
    "quail_multiplan_build": ([C.POINTER(ModelConfig), C.c_size_t, C.c_int32, C.c_int32, _i32p, C.c_int32,
                               _i32p, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p, _i64p], C.c_int32),
    "quail_ctx_create": ([C.POINTER(ModelConfig), C.POINTER(Weights), _vp, C.c_size_t, _vp, C.c_size_t,
                          C.c_int32, C.POINTER(_vp)], C.c_int32),
    "quail_ctx_destroy": ([_vp], C.c_int32),
    "quail_anchor_prefill": ([_vp, C.c_int32, _vp, _i32p, _i32p, _i64p, _i64p, _vp], C.c_int32),
    "quail_anchor_release": ([_vp, C.c_int64], C.c_int32),
    "quail_join_search": ([C.POINTER(ModelConfig), C.c_int32, C.POINTER(Table), C.c_int32, C.POINTER(AIJoin),
                           C.c_double, C.c_double, _i32p, _i32p, _f64p, _f64p, C.c_int32, _i32p], C.c_int32),
    "quail_prefix_groups": ([C.c_int32, _i32p, _i32p, _i32p, C.c_int32, _i32p, _i32p, _i32p, _i32p],
                            C.c_int32),
    "quail_prefix_tree": ([C.c_int32, _i32p, _i32p, _i32p, C.c_int32, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p],
                          C.c_int32),
    "quail_prefix_prefill": ([_vp, C.c_int32, _i64p, _vp, _i32p, _i32p, _i64p, _vp], C.c_int32),
    "quail_anchor_kv": ([_vp, C.c_int64, C.c_int32, C.POINTER(_vp), C.POINTER(_vp), _i32p, _i32p],
                        C.c_int32),
    "quail_join_prefill": ([_vp, C.c_int32, _i64p, _vp, _i32p, _vp, _vp, _vp], C.c_int32),
    "quail_head8": ([_vp, C.c_int32, _vp, C.c_uint8, _vp, _vp, _vp, _vp], C.c_int32),
    "quail_head8_f32": ([C.c_int32, C.c_int32, _vp, _vp, C.c_uint8, _vp, _vp, _vp, _vp], C.c_int32),
    "quail_join_run": ([_vp, C.c_int32, _vp, _i32p, C.c_int32, _i32p, _vp, _i32p, C.c_uint8, _vp, _vp,
                        _vp, _vp], C.c_int32),
    "quail_join_run_shared": ([_vp, C.c_int32, _vp, _i32p, C.c_int32, _i32p, _vp, _i32p, _i32p, C.c_int32,
                               C.c_int32, C.c_uint8, _vp, _vp, _vp, _vp], C.c_int32),
    "quail_multijoin_run": ([_vp, C.c_int32, _vp, _i32p, C.c_int32, _i32p, _i32p, _vp, _i32p, C.c_uint8,
                             _vp, _vp, _vp, _vp], C.c_int32),
    "quail_pool_stats": ([_vp, _szp, _szp, _i64p, _i64p, _i64p], C.c_int32),
    "quail_ctx_check": ([_vp, _vp, _i64p, _i64p], C.c_int32),
    "quail_ctx_profile": ([_vp, C.c_int32], C.c_int32),
    "quail_ctx_profile_read": ([_vp, _i64p, _f64p, _f64p], C.c_int32),
    "quail_cascade_workspace_bytes": ([C.c_int32, _i32p, C.c_int32, _i32p, _szp], C.c_int32),
    "quail_cascade_attn": ([C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_int32, _vp, _vp,
                            _i32p, C.c_int32, _i32p, _vp, _vp, _vp, _i32p, _vp, _vp, _vp, C.c_size_t,
                            _vp], C.c_int32),
    "quail_cascade_attn_noalloc": ([C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_int32, _vp,
                                    _vp, _i32p, C.c_int32, _i32p, _vp, _vp, _vp, _i32p, _vp, _vp, _vp],
                                   C.c_int32),
    "quail_gemm_w8a16": ([C.c_int32, C.c_int32, C.c_int32, _vp, _vp, _vp, _vp, _vp], C.c_int32),
    "quail_act_quant_e4m3": ([C.c_int32, C.c_int32, _vp, _vp, _vp, _vp], C.c_int32),
    "quail_gemm_w8a8": ([C.c_int32, C.c_int32, C.c_int32, _vp, _vp, _vp, _vp, _vp, _vp], C.c_int32),
    "quail_fp8_e4m3_encode": ([C.c_int64, _vp, C.c_float, _vp, _vp], C.c_int32),
    "quail_fp8_e4m3_decode": ([C.c_int64, _vp, C.c_float, _vp, _vp], C.c_int32),
}

EXPORTS = tuple(_SIGS)


def load(path: str = _LIB_PATH):
    """Load libquail.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m query_aware_prefill_amd.build` (there is no fallback)")
    lib = C.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(st):
    if st != OK:
        raise QuailError(st, load().quail_last_error().decode())


# ---- marshalling helpers ------------------------------------------------------
def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


def _i64(a):
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(_i64p)


def dptr(t):
    """Device pointer of a contiguous torch CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---- library calls (same names as the C ABI) -----------------------------------
def quail_version() -> str:
    return load().quail_version().decode()


def quail_anchor_bytes(cfg: ModelConfig, anchor_len: int) -> int:
    out = C.c_size_t()
    _check(load().quail_anchor_bytes(C.byref(cfg), anchor_len, C.byref(out)))
    return out.value


def quail_workspace_bytes(cfg: ModelConfig, max_batch_tokens: int) -> int:
    out = C.c_size_t()
    _check(load().quail_workspace_bytes(C.byref(cfg), max_batch_tokens, C.byref(out)))
    return out.value


def quail_plan_build(cfg: ModelConfig, pool_bytes: int, max_batch_tokens: int, anchor_len,
                     pair_anchor, pair_len):
    al, alp = _i32(anchor_len)
    pa, pap = _i32(pair_anchor)
    pl, plp = _i32(pair_len)
    n = len(pa)
    order, op = _i32(np.zeros(n, np.int32))
    bounds, bp = _i32(np.zeros(n + 1, np.int32))
    nsteps = C.c_int32()
    peak = C.c_size_t()
    _check(load().quail_plan_build(C.byref(cfg), pool_bytes, max_batch_tokens, len(al), alp, n, pap,
                                   plp, op, bp, C.byref(nsteps), C.byref(peak)))
    return order, bounds[: nsteps.value + 1].copy(), peak.value


def quail_multiplan_build(cfg: ModelConfig, pool_bytes: int, max_batch_tokens: int, anchor_len,
                          join_offsets, pair_anchor, pair_len) -> dict:
    """Plan of several joins over one anchor table (see include/quail.h).
    Returns pair_order, steps [(join, lo, hi, prefill, evict_before,
    evict_after)] and the totals."""
    al, alp = _i32(anchor_len)
    jo, jop = _i32(join_offsets)
    pa, pap = _i32(pair_anchor)
    pl, plp = _i32(pair_len)
    P = int(jo[-1]) if len(jo) else 0
    order, op = _i32(np.zeros(max(P, 1), np.int32))
    info, ip = _i32(np.zeros(3 * max(P, 1), np.int32))
    eoff, eop = _i32(np.zeros(3 * P + 1, np.int32))
    ean, eap = _i32(np.zeros(2 * max(P, 1), np.int32))
    tot = np.zeros(4, np.int64)
    nsteps = C.c_int32()
    _check(load().quail_multiplan_build(C.byref(cfg), pool_bytes, max_batch_tokens, len(al), alp, len(jo) - 1,
                                        jop, pap, plp, op, ip, C.byref(nsteps), eop, eap,
                                        tot.ctypes.data_as(_i64p)))
    steps = []
    for t in range(nsteps.value):
        lists = [ean[eoff[3 * t + q]:eoff[3 * t + q + 1]].tolist() for q in range(3)]
        steps.append((int(info[3 * t]), int(info[3 * t + 1]), int(info[3 * t + 2]), *lists))
    return dict(pair_order=order[:P].copy(), steps=steps, prefills=int(tot[0]), evictions=int(tot[1]),
                regret_tokens=int(tot[2]), peak=int(tot[3]))


class Context:
    """Owns a quail_ctx; device buffers (weights, pool, workspace) are torch
    tensors held by the caller and borrowed here."""

    def __init__(self, cfg: ModelConfig, weights: Weights, kv_pool, workspace, max_batch_tokens: int):
        self.cfg = cfg
        self._weights = weights       # keep the ctypes struct (and its layer array) alive
        self._pool = kv_pool
        self._ws = workspace
        h = C.c_void_p()
        _check(load().quail_ctx_create(C.byref(cfg), C.byref(weights), dptr(kv_pool),
                                       kv_pool.numel() * kv_pool.element_size() if kv_pool is not None else 0,
                                       dptr(workspace), workspace.numel() * workspace.element_size(),
                                       max_batch_tokens, C.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            load().quail_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def quail_anchor_prefill(ctx: Context, tokens, offsets, n_uses, anchor_ids=None, stream=None):
    off, offp = _i32(offsets)
    nu, nup = _i32(n_uses)
    n = len(off) - 1
    out, outp = _i64(np.zeros(n, np.int64))
    ids, idsp = (None, None) if anchor_ids is None else _i64(anchor_ids)
    _check(load().quail_anchor_prefill(ctx.handle, n, dptr(tokens), offp, nup, idsp, outp,
                                       stream_handle(stream)))
    return out


def quail_anchor_release(ctx: Context, handle: int):
    _check(load().quail_anchor_release(ctx.handle, int(handle)))


def quail_join_search(cfg: ModelConfig, tables, joins, peak_flops: float, peak_bytes_per_s: float,
                      cap: int = 256):
    """tables: [(rows, field_tokens)]; joins: [(left, right, anchor_glue,
    suffix_glue, selectivity, symmetric)]. Returns dict(order, anchor_right,
    metrics, frontier)."""
    nt, nj = len(tables), len(joins)
    ta = (Table * max(nt, 1))(*[Table(int(r), float(t)) for r, t in tables])
    ja = (AIJoin * max(nj, 1))(*[AIJoin(int(a), int(b), float(ga), float(gs), float(s), int(y))
                                 for a, b, ga, gs, s, y in joins])
    order, op = _i32(np.zeros(max(nt, 1), np.int32))
    ar, arp = _i32(np.zeros(max(nj, 1), np.int32))
    met = np.zeros(4, np.float64)
    fr = np.zeros((max(cap, 1), 4), np.float64)
    nf = C.c_int32()
    _check(load().quail_join_search(C.byref(cfg), nt, ta, nj, ja, peak_flops, peak_bytes_per_s, op, arp,
                                    met.ctypes.data_as(_f64p), fr.ctypes.data_as(_f64p), cap, C.byref(nf)))
    return dict(order=order[:nt].copy(), anchor_right=ar[:nj].copy(), metrics=met,
                frontier=fr[:min(cap, nf.value)].copy(), n_frontier=nf.value)


def quail_prefix_groups(tokens, offsets, keys, min_len: int):
    """Host radix grouping; returns (group_of, node_first, node_len) numpy int32."""
    tok, tokp = _i32(np.asarray(tokens).reshape(-1) if len(tokens) else np.zeros(1, np.int32))
    off, offp = _i32(offsets)
    n = len(off) - 1
    ks, ksp = (None, None) if keys is None else _i32(keys)
    g, gp = _i32(np.zeros(max(n, 1), np.int32))
    f, fp = _i32(np.zeros(max(n, 1), np.int32))
    ln, lnp = _i32(np.zeros(max(n, 1), np.int32))
    nn = C.c_int32()
    _check(load().quail_prefix_groups(n, tokp, offp, ksp, int(min_len), gp, fp, lnp, C.byref(nn)))
    return g[:n].copy(), f[:nn.value].copy(), ln[:nn.value].copy()


def quail_prefix_tree(tokens, offsets, keys, min_len: int):
    """Nested radix grouping; returns (group_of, nodes) with nodes a list of
    (parent, first, start, end) tuples."""
    tok, tokp = _i32(np.asarray(tokens).reshape(-1) if len(tokens) else np.zeros(1, np.int32))
    off, offp = _i32(offsets)
    n = len(off) - 1
    ks, ksp = (None, None) if keys is None else _i32(keys)
    arrs = [_i32(np.zeros(max(n, 1), np.int32)) for _ in range(5)]
    nn = C.c_int32()
    _check(load().quail_prefix_tree(n, tokp, offp, ksp, int(min_len), *[a[1] for a in arrs], C.byref(nn)))
    g, par, first, start, end = [a[0] for a in arrs]
    nodes = [(int(par[k]), int(first[k]), int(start[k]), int(end[k])) for k in range(nn.value)]
    return g[:n].copy(), nodes


def quail_prefix_prefill(ctx: Context, parent, tokens, offsets, n_uses, stream=None):
    pa, pap = _i64(parent)
    off, offp = _i32(offsets)
    nu, nup = _i32(n_uses)
    n = len(off) - 1
    out, outp = _i64(np.zeros(n, np.int64))
    _check(load().quail_prefix_prefill(ctx.handle, n, pap, dptr(tokens), offp, nup, outp,
                                       stream_handle(stream)))
    return out


def quail_anchor_kv(ctx: Context, handle: int, layer: int):
    k, v = C.c_void_p(), C.c_void_p()
    la, lp = C.c_int32(), C.c_int32()
    _check(load().quail_anchor_kv(ctx.handle, int(handle), layer, C.byref(k), C.byref(v),
                                  C.byref(la), C.byref(lp)))
    return k.value, v.value, la.value, lp.value


def quail_join_prefill(ctx: Context, pair_anchor, tokens, offsets, h_last, h_all=None, stream=None):
    pa, pap = _i64(pair_anchor)
    off, offp = _i32(offsets)
    _check(load().quail_join_prefill(ctx.handle, len(pa), pap, dptr(tokens), offp, dptr(h_last),
                                     dptr(h_all), stream_handle(stream)))


def quail_head8(ctx: Context, h_last, true_mask, logits, token, decision, stream=None):
    _check(load().quail_head8(ctx.handle, h_last.shape[0], dptr(h_last), true_mask, dptr(logits),
                              dptr(token), dptr(decision), stream_handle(stream)))


def quail_head8_f32(x, w8, true_mask, logits, token, decision, stream=None):
    _check(load().quail_head8_f32(x.shape[0], x.shape[1], dptr(x), dptr(w8), true_mask, dptr(logits),
                                  dptr(token), dptr(decision), stream_handle(stream)))


def quail_join_run(ctx: Context, a_tokens, a_offsets, pair_anchor, s_tokens, s_offsets, true_mask,
                   logits, token, decision, stream=None):
    ao, aop = _i32(a_offsets)
    pa, pap = _i32(pair_anchor)
    so, sop = _i32(s_offsets)
    _check(load().quail_join_run(ctx.handle, len(ao) - 1, dptr(a_tokens), aop, len(pa), pap,
                                 dptr(s_tokens), sop, true_mask, dptr(logits), dptr(token),
                                 dptr(decision), stream_handle(stream)))


def quail_join_run_shared(ctx: Context, a_tokens, a_offsets, pair_anchor, s_tokens, s_offsets, s_tokens_host,
                          min_shared, true_mask, logits, token, decision, stream=None, nested=False):
    ao, aop = _i32(a_offsets)
    pa, pap = _i32(pair_anchor)
    so, sop = _i32(s_offsets)
    sh, shp = _i32(s_tokens_host)
    _check(load().quail_join_run_shared(ctx.handle, len(ao) - 1, dptr(a_tokens), aop, len(pa), pap,
                                        dptr(s_tokens), sop, shp, int(min_shared), int(bool(nested)), true_mask,
                                        dptr(logits), dptr(token), dptr(decision), stream_handle(stream)))


def quail_multijoin_run(ctx: Context, a_tokens, a_offsets, join_offsets, pair_anchor, s_tokens, s_offsets,
                        true_mask, logits, token, decision, stream=None):
    ao, aop = _i32(a_offsets)
    jo, jop = _i32(join_offsets)
    pa, pap = _i32(pair_anchor)
    so, sop = _i32(s_offsets)
    _check(load().quail_multijoin_run(ctx.handle, len(ao) - 1, dptr(a_tokens), aop, len(jo) - 1, jop, pap,
                                      dptr(s_tokens), sop, true_mask, dptr(logits), dptr(token),
                                      dptr(decision), stream_handle(stream)))


def quail_pool_stats(ctx: Context) -> dict:
    r, p = C.c_size_t(), C.c_size_t()
    pf, ev, rg = C.c_int64(), C.c_int64(), C.c_int64()
    _check(load().quail_pool_stats(ctx.handle, C.byref(r), C.byref(p), C.byref(pf), C.byref(ev),
                                   C.byref(rg)))
    return dict(resident=r.value, peak=p.value, prefills=pf.value, evictions=ev.value,
                regret_tokens=rg.value)


def quail_ctx_check(ctx: Context, stream=None) -> dict:
    """Guard-region and token-range counters (waits for the stream)."""
    g, t = C.c_int64(), C.c_int64()
    _check(load().quail_ctx_check(ctx.handle, stream_handle(stream), C.byref(g), C.byref(t)))
    return dict(guard_errors=g.value, bad_tokens=t.value)


def quail_ctx_profile(ctx: Context, enable: bool) -> None:
    _check(load().quail_ctx_profile(ctx.handle, 1 if enable else 0))


def quail_ctx_profile_read(ctx: Context) -> dict:
    """Per kind (PROF_KINDS): launches, summed launch ms and algorithmic FLOP."""
    n = len(PROF_KINDS)
    la = (C.c_int64 * n)()
    ms = (C.c_double * n)()
    fl = (C.c_double * n)()
    _check(load().quail_ctx_profile_read(ctx.handle, la, ms, fl))
    return {k: dict(launches=la[i], ms=ms[i], flop=fl[i]) for i, k in enumerate(PROF_KINDS)}


def quail_cascade_workspace_bytes(a_off, s_off) -> int:
    ao, aop = _i32(a_off)
    so, sop = _i32(s_off)
    out = C.c_size_t()
    _check(load().quail_cascade_workspace_bytes(max(len(ao) - 1, 0), aop, len(so) - 1, sop,
                                                C.byref(out)))
    return out.value


def quail_cascade_attn(dtype, hq, hkv, d, sm_scale, ak, av, a_off, s_anchor, q, k, v, s_off, out,
                       lse=None, workspace=None, stream=None):
    ao, aop = _i32(a_off)
    sa, sap = _i32(s_anchor)
    so, sop = _i32(s_off)
    _check(load().quail_cascade_attn(dtype, hq, hkv, d, sm_scale, max(len(ao) - 1, 0), dptr(ak),
                                     dptr(av), aop, len(sa), sap, dptr(q), dptr(k), dptr(v), sop,
                                     dptr(out), dptr(lse), dptr(workspace),
                                     workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                     stream_handle(stream)))


def quail_cascade_attn_noalloc(dtype, hq, hkv, d, sm_scale, ak, av, a_off, s_anchor, q, k, v, s_off, out,
                               lse=None, stream=None):
    """quail_cascade_attn without a workspace (the library's static scratch)."""
    ao, aop = _i32(a_off)
    sa, sap = _i32(s_anchor)
    so, sop = _i32(s_off)
    _check(load().quail_cascade_attn_noalloc(dtype, hq, hkv, d, sm_scale, max(len(ao) - 1, 0), dptr(ak),
                                             dptr(av), aop, len(sa), sap, dptr(q), dptr(k), dptr(v), sop,
                                             dptr(out), dptr(lse), stream_handle(stream)))


def quail_gemm_w8a16(x, w, scale, y, stream=None):
    M, K = x.shape
    N = w.shape[0]
    _check(load().quail_gemm_w8a16(M, N, K, dptr(x), dptr(w), dptr(scale), dptr(y),
                                   stream_handle(stream)))


def quail_act_quant_e4m3(x, codes, scale, stream=None):
    M, K = x.shape
    _check(load().quail_act_quant_e4m3(M, K, dptr(x), dptr(codes), dptr(scale), stream_handle(stream)))


def quail_gemm_w8a8(xc, x_scale, wc, w_scale, y, stream=None):
    M, K = xc.shape
    N = wc.shape[0]
    _check(load().quail_gemm_w8a8(M, N, K, dptr(xc), dptr(x_scale), dptr(wc), dptr(w_scale), dptr(y),
                                  stream_handle(stream)))


def quail_fp8_e4m3_encode(x, scale, codes, stream=None):
    _check(load().quail_fp8_e4m3_encode(x.numel(), dptr(x), scale, dptr(codes), stream_handle(stream)))


def quail_fp8_e4m3_decode(codes, scale, x, stream=None):
    _check(load().quail_fp8_e4m3_decode(codes.numel(), dptr(codes), scale, dptr(x), stream_handle(stream)))
