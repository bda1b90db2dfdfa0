"""ctypes binding of libjolt (argument marshalling only).

Every step of compression and reconstruction runs inside libjolt.so on the GPU; this module
only converts Python/torch arguments into the C structs of include/jolt.h, allocates device
buffers with torch and passes the current HIP stream.  If the library is missing it raises;
there is no other code path.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjolt.so")

F16, BF16, F32 = 0, 1, 2
EXACT, FLASH = 0, 1
ALLOC_JOINT, ALLOC_GREEDY, ALLOC_KV_DECOUPLED, ALLOC_UNIFORM_RANKS = 0, 1, 2, 4
STATUS = {0: "JOLT_OK", -1: "JOLT_EINVAL", -2: "JOLT_EINFEASIBLE", -3: "JOLT_EWORKSPACE", -4: "JOLT_EHIP",
          -5: "JOLT_ENONFINITE", -6: "JOLT_EBUFFER"}
TORCH_DTYPE = {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}
DTYPE_OF = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
EXPORTS = ["jolt_workspace_bytes", "jolt_output_bytes", "jolt_allocate", "jolt_compress", "jolt_reconstruct",
           "jolt_spectra", "jolt_token_spectrum_len", "jolt_encode_residual",
           "jolt_encode_residual_workspace_bytes", "jolt_rotation", "jolt_eps2", "jolt_last_error", "jolt_profile",
           "jolt_profile_read", "jolt_sketch_matrix", "jolt_test_wait_policy", "jolt_allocate_static", "jolt_layer_groups",
           "jolt_layer_groups_workspace_bytes", "jolt_rope_table", "jolt_decode_attention_workspace_bytes",
           "jolt_decode_attention"]


class JoltError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_tokens", ctypes.c_int32), ("d_head", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("group_start", ctypes.POINTER(ctypes.c_int32))]


class Params(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("oversample", ctypes.c_int32), ("power_iters", ctypes.c_int32),
                ("qcap", ctypes.c_int32),
                ("rT_grid", ctypes.POINTER(ctypes.c_int32)), ("n_rT", ctypes.c_int32),
                ("rd_grid", ctypes.POINTER(ctypes.c_int32)), ("n_rd", ctypes.c_int32),
                ("bits", ctypes.POINTER(ctypes.c_int32)), ("n_bits", ctypes.c_int32),
                ("eps2", ctypes.POINTER(ctypes.c_double)), ("target_ratio", ctypes.c_double),
                ("rot_seed", ctypes.c_uint64), ("sketch_seed", ctypes.c_uint64), ("alloc_variant", ctypes.c_int32)]


class Pick(ctypes.Structure):
    _fields_ = [("rT", ctypes.c_int32), ("rd", ctypes.c_int32), ("bits", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("bytes", ctypes.c_int64), ("err_pred", ctypes.c_double), ("offset", ctypes.c_int64),
                ("section_bytes", ctypes.c_int64)]


_lib = None


def load():
    """Load libjolt.so (built by __graft_entry__.build()); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libjolt.so not built ({LIB_PATH}); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, dbl, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
    pd, pp = ctypes.POINTER(CacheDesc), ctypes.POINTER(Params)
    sig = {
        "jolt_workspace_bytes": (sz, [pd, pp]),
        "jolt_output_bytes": (sz, [pd, pp]),
        "jolt_token_spectrum_len": (i64, [pd, pp]),
        "jolt_allocate": (ctypes.c_int, [i32, ctypes.POINTER(i32), i32, P, ctypes.POINTER(i64), P,
                                         ctypes.POINTER(i64), P, pp, dbl, ctypes.POINTER(Pick),
                                         ctypes.POINTER(dbl), P, sz, P]),
        "jolt_allocate_static": (ctypes.c_int, [i32, ctypes.POINTER(i32), i32, P, ctypes.POINTER(i64), P,
                                                ctypes.POINTER(i64), P, pp, dbl, ctypes.POINTER(Pick),
                                                ctypes.POINTER(dbl), P]),
        "jolt_compress": (ctypes.c_int, [P, P, pd, pp, P, sz, P, sz, ctypes.POINTER(Pick), ctypes.POINTER(dbl), P]),
        "jolt_reconstruct": (ctypes.c_int, [P, pd, pp, ctypes.POINTER(Pick), P, P, P, sz, P]),
        "jolt_spectra": (ctypes.c_int, [P, P, pd, pp, P, P, P, P, i32, P, sz, P]),
        "jolt_encode_residual": (ctypes.c_int, [P, i32, i32, i32, i32, i32, P, P, P, i32, i32, i32,
                                                ctypes.c_uint64, P, P, P, sz, P]),
        "jolt_encode_residual_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
        "jolt_rotation": (ctypes.c_int, [i32, ctypes.c_uint64, ctypes.POINTER(dbl)]),
        "jolt_eps2": (ctypes.c_int, [i32, ctypes.POINTER(dbl)]),
        "jolt_last_error": (ctypes.c_char_p, []),
        "jolt_profile": (ctypes.c_int, [i32]),
        "jolt_sketch_matrix": (ctypes.c_int, [i32, i32, i32, ctypes.c_uint64, P, P]),
        "jolt_layer_groups_workspace_bytes": (sz, [pd]),
        "jolt_layer_groups": (ctypes.c_int, [P, pd, ctypes.c_uint64, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                             ctypes.POINTER(dbl), P, sz, P]),
        "jolt_test_wait_policy": (ctypes.c_int, [ctypes.c_uint32, i32]),
        "jolt_profile_read": (i32, [ctypes.c_char_p, i32, ctypes.POINTER(dbl), ctypes.POINTER(i32), i32]),
        "jolt_rope_table": (ctypes.c_int, [i32, dbl, i32, P, P]),
        "jolt_decode_attention_workspace_bytes": (sz, [pd, ctypes.POINTER(Pick), i32, i32, i32]),
        "jolt_decode_attention": (ctypes.c_int, [P, pd, pp, ctypes.POINTER(Pick), i32, i32, P, i32, P, P, i32, P, i32,
                                                 P, P, sz, i32, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        msg = load().jolt_last_error().decode()
        raise JoltError(status, msg)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _i32arr(vals):
    a = (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])
    return a


class Config:
    """Cache descriptor + parameters, holding the ctypes arrays alive."""

    def __init__(self, n_seq, n_layers, n_heads, n_tokens, d_head, dtype, group_start, mode, rT_grid, rd_grid,
                 bits, target_ratio, oversample=10, power_iters=1, qcap=0, eps2=None, rot_seed=0, sketch_seed=0,
                 alloc_variant=0):
        self._gs = _i32arr(group_start)
        self.desc = CacheDesc(n_seq, n_layers, n_heads, n_tokens, d_head, dtype, len(group_start) - 1, self._gs)
        self._rT, self._rd, self._bits = _i32arr(rT_grid), _i32arr(rd_grid), _i32arr(bits)
        self._eps = None
        if eps2 is not None:
            e = np.ones(9)
            for b, v in dict(eps2).items():
                e[int(b)] = float(v)
            self._eps = (ctypes.c_double * 9)(*e.tolist())
        self.params = Params(mode, oversample, power_iters, qcap, self._rT, len(rT_grid), self._rd, len(rd_grid),
                             self._bits, len(bits), self._eps, float(target_ratio), rot_seed, sketch_seed,
                             int(alloc_variant))
        self.n_cells = n_seq * (len(group_start) - 1) * 2

    def workspace_bytes(self):
        n = load().jolt_workspace_bytes(ctypes.byref(self.desc), ctypes.byref(self.params))
        if n == 0:
            _check(-1)
        return n

    def output_bytes(self):
        n = load().jolt_output_bytes(ctypes.byref(self.desc), ctypes.byref(self.params))
        if n == 0:
            _check(-1)
        return n

    def token_spectrum_len(self):
        n = load().jolt_token_spectrum_len(ctypes.byref(self.desc), ctypes.byref(self.params))
        if n <= 0:
            _check(int(n))
        return int(n)


def _device_of(t):
    return t.device if t is not None else torch.device("cuda")


def workspace(cfg, device="cuda"):
    return torch.empty(cfg.workspace_bytes(), dtype=torch.uint8, device=device)


def compress(K, V, cfg, out=None, ws=None):
    """Compress K and V (contiguous [n_seq][L][H][T][D] device tensors).

    Returns (blob uint8 tensor, list of pick dicts, lambda)."""
    lib = load()
    K, V = K.contiguous(), V.contiguous()
    if ws is None:
        ws = workspace(cfg, K.device)
    if out is None:
        out = torch.empty(cfg.output_bytes(), dtype=torch.uint8, device=K.device)
    picks = (Pick * cfg.n_cells)()
    lam = (ctypes.c_double * 2)(0.0, 0.0)  # K/V-decoupled allocations return two multipliers
    _check(lib.jolt_compress(_ptr(K), _ptr(V), ctypes.byref(cfg.desc), ctypes.byref(cfg.params), _ptr(out),
                             out.numel(), _ptr(ws), ws.numel(), picks, lam, _stream()))
    return out, [_pick_dict(p) for p in picks], _lam(lam, cfg.params.alloc_variant)


def _pick_dict(p):
    return {"rT": p.rT, "rd": p.rd, "bits": p.bits, "bytes": p.bytes, "err_pred": p.err_pred, "offset": p.offset,
            "section_bytes": p.section_bytes}


def _picks_array(picks):
    arr = (Pick * len(picks))()
    for a, p in zip(arr, picks):
        a.rT, a.rd, a.bits = int(p["rT"]), int(p["rd"]), int(p["bits"])
        a.bytes = int(p.get("bytes", 0))
        a.err_pred = float(p.get("err_pred", 0.0))
        a.offset = int(p["offset"])
        a.section_bytes = int(p.get("section_bytes", 0))
    return arr


def reconstruct(blob, cfg, picks, K_out, V_out, ws=None):
    lib = load()
    if ws is None:
        ws = workspace(cfg, blob.device)
    arr = _picks_array(picks)
    _check(lib.jolt_reconstruct(_ptr(blob), ctypes.byref(cfg.desc), ctypes.byref(cfg.params), arr, _ptr(K_out),
                                _ptr(V_out), _ptr(ws), ws.numel(), _stream()))


def rope_table(d_head, base, n_pos, device="cuda"):
    """[n_pos][d_head/2][2] float32 device tensor of RoPE cosines and sines (jolt_rope_table)."""
    lib = load()
    out = torch.empty(max(n_pos, 1), d_head // 2, 2, dtype=torch.float32, device=device)
    _check(lib.jolt_rope_table(int(d_head), float(base), int(n_pos), _ptr(out), _stream()))
    return out


def decode_attention(blob, cfg, picks, seq, layer, q, k_tail=None, v_tail=None, rope=None, rope_base=500000.0,
                     out=None, ws=None, reuse_prepared=False):
    """One decode step of one layer over the compressed cells (jolt_decode_attention).

    q: [n_q_heads][d_head] float32 (rotated at its position); k_tail / v_tail: [n_heads][n_tail][d_head]
    in the cache dtype or None; rope: a rope_table covering T + n_tail positions (built if None);
    reuse_prepared: ws holds the layer's state from an earlier call on the same layer."""
    lib = load()
    arr = _picks_array(picks)
    q = q.contiguous()
    n_q, D = q.shape
    T = cfg.desc.n_tokens
    n_tail = 0 if k_tail is None else int(k_tail.shape[1])
    if rope is None:
        rope = rope_table(D, rope_base, T + n_tail, q.device)
    if out is None:
        out = torch.empty(n_q, D, dtype=torch.float32, device=q.device)
    if ws is None:
        nb = lib.jolt_decode_attention_workspace_bytes(ctypes.byref(cfg.desc), arr, int(seq), int(layer), int(n_q))
        if nb == 0:
            raise JoltError(-1, "decode_attention: invalid arguments")
        ws = torch.empty(nb, dtype=torch.uint8, device=q.device)
    kt = k_tail.contiguous() if k_tail is not None else None
    vt = v_tail.contiguous() if v_tail is not None else None
    _check(lib.jolt_decode_attention(_ptr(blob), ctypes.byref(cfg.desc), ctypes.byref(cfg.params), arr, int(seq),
                                     int(layer), _ptr(q), int(n_q), _ptr(kt) if kt is not None else None,
                                     _ptr(vt) if vt is not None else None, n_tail, _ptr(rope), int(rope.shape[0]),
                                     _ptr(out), _ptr(ws), ws.numel(), int(bool(reuse_prepared)), _stream()))
    return out


def spectra(K, V, cfg, n_vec=0, ws=None):
    """Returns (specT [n_cells][nT], specD [n_cells][D], norm2 [n_cells], UT [n_cells][n_vec][T] or None)."""
    lib = load()
    dev = K.device
    nT = cfg.token_spectrum_len()
    nc, D, T = cfg.n_cells, cfg.desc.d_head, cfg.desc.n_tokens
    specT = torch.empty(nc, nT, dtype=torch.float64, device=dev)
    specD = torch.empty(nc, D, dtype=torch.float64, device=dev)
    norm2 = torch.empty(nc, dtype=torch.float64, device=dev)
    UT = torch.empty(nc, n_vec, T, dtype=torch.float32, device=dev) if n_vec > 0 else None
    if ws is None:
        extra = 0
        if n_vec > 0:
            extra = 4 * nc * (n_vec + 8) * (T + 8) * 3 + 8 * nc * (n_vec + 8) * (max(nT, T) + 8) * 6
        ws = torch.empty(cfg.workspace_bytes() + extra, dtype=torch.uint8, device=dev)
    _check(lib.jolt_spectra(_ptr(K.contiguous()), _ptr(V.contiguous()), ctypes.byref(cfg.desc),
                            ctypes.byref(cfg.params), _ptr(specT), _ptr(specD), _ptr(norm2), _ptr(UT), int(n_vec),
                            _ptr(ws), ws.numel(), _stream()))
    return specT, specD, norm2, UT


def _lam(lam, variant):
    return (lam[0], lam[1]) if variant & ALLOC_KV_DECOUPLED else lam[0]


def allocate(cell_shapes, elem_bytes, specT_list, specD_list, norm2, rT_grid, rd_grid, bits, budget, eps2=None,
             device="cuda", static_scratch=False, alloc_variant=0):
    """Lagrangian allocation on given spectra (lists of 1-D float64 arrays, one per cell).

    static_scratch=True calls jolt_allocate_static (no workspace: the library's fixed device scratch)."""
    lib = load()
    cfg = Config(1, 1, 1, 1, 64, F16, [0, 1], EXACT, rT_grid, rd_grid, bits, 2.0, eps2=eps2,
                 alloc_variant=alloc_variant)
    n = len(cell_shapes)
    shp = (ctypes.c_int32 * (4 * n))(*[int(v) for s in cell_shapes for v in s])
    offT = np.concatenate([[0], np.cumsum([len(s) for s in specT_list])]).astype(np.int64)
    offD = np.concatenate([[0], np.cumsum([len(s) for s in specD_list])]).astype(np.int64)
    dT = torch.from_numpy(np.concatenate(specT_list).astype(np.float64)).to(device)
    dD = torch.from_numpy(np.concatenate(specD_list).astype(np.float64)).to(device)
    dn = torch.from_numpy(np.asarray(norm2, dtype=np.float64)).to(device)
    picks = (Pick * n)()
    lam = (ctypes.c_double * 2)(0.0, 0.0)  # K/V-decoupled allocations return two multipliers
    if static_scratch:
        status = lib.jolt_allocate_static(n, shp, int(elem_bytes), _ptr(dT),
                                          offT.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr(dD),
                                          offD.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr(dn),
                                          ctypes.byref(cfg.params), float(budget), picks, lam,
                                          _stream())
        return status, [_pick_dict(p) for p in picks], _lam(lam, cfg.params.alloc_variant)
    per = (len(set(bits) | {0})) * len(rT_grid) * len(rd_grid)
    ws = torch.empty(n * per * 16 + n * (len(rT_grid) + len(rd_grid)) * 8 + n * 64 + (1 << 20), dtype=torch.uint8,
                     device=device)
    status = lib.jolt_allocate(n, shp, int(elem_bytes), _ptr(dT), offT.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                               _ptr(dD), offD.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr(dn),
                               ctypes.byref(cfg.params), float(budget), picks, lam, _ptr(ws),
                               ws.numel(), _stream())
    return status, [_pick_dict(p) for p in picks], _lam(lam, cfg.params.alloc_variant)


def encode_residual(X, UT, core, Ud, rT, rd, bits, rot_seed=0):
    """Residual stage of one cell with given factors (storage dtype = X dtype).

    X [G][H][T][D], UT [T][rT], core [G][H][rT][rd], Ud [D][rd].  Returns (scales, codes)."""
    lib = load()
    G, H, T, D = X.shape
    dtype = DTYPE_OF[X.dtype]
    scales = torch.empty(G * H * T, dtype=torch.float32, device=X.device)
    codes = torch.empty(G * H * T, D * bits // 8, dtype=torch.uint8, device=X.device)
    nws = lib.jolt_encode_residual_workspace_bytes(G, H, T, D, rT, rd)
    if nws == 0:
        _check(-1)
    ws = torch.empty(nws, dtype=torch.uint8, device=X.device)
    _check(lib.jolt_encode_residual(_ptr(X.contiguous()), G, H, T, D, dtype, _ptr(UT.contiguous()),
                                    _ptr(core.contiguous()), _ptr(Ud.contiguous()), rT, rd, bits, rot_seed,
                                    _ptr(scales), _ptr(codes), _ptr(ws), nws, _stream()))
    return scales, codes


def rotation(d_head, seed=0):
    out = np.zeros((d_head, d_head))
    _check(load().jolt_rotation(d_head, seed, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return out


def eps2(d_head):
    out = np.zeros(9)
    _check(load().jolt_eps2(d_head, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return out


def layer_groups(K, sketch_seed=0):
    """Layer groups of a key cache [n_seq][L][H][T][D] by token-subspace alignment.

    Returns (group_start list, scores array of the L-1 consecutive-layer pairs)."""
    lib = load()
    n_seq, L, H, T, D = K.shape
    cfg = Config(n_seq, L, H, T, D, DTYPE_OF[K.dtype], list(range(L + 1)), FLASH, [8], [8], [2], 2.0)
    nws = lib.jolt_layer_groups_workspace_bytes(ctypes.byref(cfg.desc))
    if nws == 0:
        _check(-1)
    ws = torch.empty(nws, dtype=torch.uint8, device=K.device)
    starts = (ctypes.c_int32 * (L + 1))()
    ng = ctypes.c_int32(0)
    sc = np.zeros(max(L - 1, 0))
    _check(lib.jolt_layer_groups(_ptr(K.contiguous()), ctypes.byref(cfg.desc), int(sketch_seed), starts,
                                 ctypes.byref(ng), sc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), _ptr(ws),
                                 nws, _stream()))
    return [int(starts[i]) for i in range(ng.value + 1)], sc


def sketch_matrix(M, ell, dtype, seed=0, device="cuda"):
    """Omega^T (ell x M) in the cache dtype, as jolt_compress draws it (bf16 returned as torch.bfloat16)."""
    out = torch.empty(ell, M, dtype=TORCH_DTYPE[dtype], device=device)
    _check(load().jolt_sketch_matrix(int(M), int(ell), int(dtype), int(seed), _ptr(out), _stream()))
    return out


def test_wait_policy(spin_limit=0, unreachable=False):
    """Testing hook: spin limit of the bounded cross-workgroup waits; unreachable=True makes every wait lapse."""
    _check(load().jolt_test_wait_policy(int(spin_limit), 1 if unreachable else 0))


def profile(enable=True):
    """Turn the library's per-stage HIP-event timing on or off."""
    _check(load().jolt_profile(1 if enable else 0))


def profile_read():
    """{stage: (total ms, occurrences)} since the last read (waits for the recorded events)."""
    n_max = 64
    names = ctypes.create_string_buffer(8192)
    ms = (ctypes.c_double * n_max)()
    cnt = (ctypes.c_int32 * n_max)()
    n = load().jolt_profile_read(names, 8192, ms, cnt, n_max)
    if n < 0:
        _check(n)
    keys = names.value.decode().split("\n")[:n]
    return {k: (ms[i], cnt[i]) for i, k in enumerate(keys)}
