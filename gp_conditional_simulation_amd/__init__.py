"""Python binding of libgpex, the gfx950 excursion-set simulation library.

Thin marshalling over the C ABI in ``include/gpex.h``: every step runs in the library's HIP
kernels; PyTorch only provides device memory and the stream.  The functions keep the C names
without the ``gpex_`` prefix.  There is no CPU fallback: when ``libgpex.so`` is missing the
import fails with instructions to build it.

The method is the one of "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial
Excursion Sets" (covariance tiles, adaptive mixed-precision tile Cholesky, FP16 TRMM simulation,
universal kriging, conditioning and calibration of inner/outer regions).
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpex.so")

FP64, FP32, FP16 = 0, 1, 2
OK, ERR_ARG, ERR_HIP, ERR_NOMEM, ERR_STATE = 0, -1, -2, -3, -4
ERR_NOT_SPD, ERR_MSPE_NONPOS, ERR_EMPTY_SAMPLE, WARN_CHECKS_FAILED, WARN_FP16_OVERFLOW = 1, 2, 3, 4, 5
STATUS_NAMES = {0: "OK", -1: "ERR_ARG", -2: "ERR_HIP", -3: "ERR_NOMEM", -4: "ERR_STATE", 1: "ERR_NOT_SPD",
                2: "ERR_MSPE_NONPOS", 3: "ERR_EMPTY_SAMPLE", 4: "WARN_CHECKS_FAILED", 5: "WARN_FP16_OVERFLOW"}
EXPORTS = ["gpex_version", "gpex_ctx_create", "gpex_ctx_destroy", "gpex_ctx_release_workspace", "gpex_ctx_set_serial",
           "gpex_last_error", "gpex_cov_gen",
           "gpex_tiled_info", "gpex_tiled_stats", "gpex_tiled_to_dense", "gpex_tiled_block", "gpex_tiled_block_raw",
           "gpex_tiled_destroy",
           "gpex_potrf_mp", "gpex_normals", "gpex_trmm_sim", "gpex_krige", "gpex_excursion_regions",
           "gpex_excursion_regions_below", "gpex_excursion_regions_noalloc",
           "gpex_plan", "gpex_ctx_set_timing", "gpex_ctx_timings"]


class CovParams(C.Structure):
    _fields_ = [("kind", C.c_int), ("sigma2", C.c_double), ("range", C.c_double), ("nu", C.c_double),
                ("nugget", C.c_double)]


class PrecOpts(C.Structure):
    _fields_ = [("amp", C.c_int), ("tol", C.c_double), ("allow_fp16", C.c_int), ("unscaled_rule", C.c_int),
                ("auto_tol", C.c_int), ("fp16_dest_emulation", C.c_int)]


class Diag(C.Structure):
    _fields_ = [("s", C.c_double), ("frob", C.c_double), ("l_bound", C.c_double), ("u_bound", C.c_double),
                ("l_bound_sub", C.c_double), ("r_hp", C.c_double), ("rho1", C.c_double), ("rho2", C.c_double),
                ("norm_B", C.c_double), ("eq10_pass", C.c_int), ("eq11_pass", C.c_int),
                ("lower_exceeds_upper", C.c_int), ("fp16_overflow", C.c_int), ("tiles", C.c_int64 * 3),
                ("tol", C.c_double), ("tol_reductions", C.c_int64), ("u_factor", C.c_double)]

    def to_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_ if k != "tiles"}
        d["tiles"] = list(self.tiles)
        return d


class RegionStats(C.Structure):
    _fields_ = [("q_in", C.c_double), ("q_out", C.c_double), ("n_psi", C.c_int64), ("n_phi", C.c_int64)]


# Device allocator callbacks handed to gpex_ctx_create: void* alloc(size_t, void*), void free(void*, void*).
_ALLOC_FN = C.CFUNCTYPE(C.c_void_p, C.c_size_t, C.c_void_p)
_FREE_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p)


class GpexError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib():
    """The loaded libgpex (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                              "g.build()'` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        P, I, I64, D, U64 = C.c_void_p, C.c_int, C.c_int64, C.c_double, C.c_uint64
        L.gpex_version.restype = C.c_char_p
        L.gpex_last_error.restype = C.c_char_p
        L.gpex_last_error.argtypes = [P]
        L.gpex_ctx_create.argtypes = [I, P, _ALLOC_FN, _FREE_FN, P, C.POINTER(P)]
        L.gpex_ctx_destroy.argtypes = [P]
        L.gpex_ctx_release_workspace.argtypes = [P]
        L.gpex_ctx_set_serial.argtypes = [P, I]
        L.gpex_cov_gen.argtypes = [P, P, I64, P, C.POINTER(CovParams), I, C.POINTER(PrecOpts), C.POINTER(P),
                                   C.POINTER(Diag)]
        L.gpex_tiled_info.argtypes = [P, C.POINTER(I64), C.POINTER(I), C.POINTER(I64), P, C.POINTER(D)]
        L.gpex_tiled_stats.argtypes = [P, P]
        L.gpex_tiled_to_dense.argtypes = [P, P, P, I64]
        L.gpex_tiled_block.argtypes = [P, P, I64, I64, I64, I64, P, I64]
        L.gpex_tiled_block_raw.argtypes = [P, P, I, I64, I64, I64, I64, P, I64]
        L.gpex_tiled_destroy.argtypes = [P]
        L.gpex_potrf_mp.argtypes = [P, P, C.POINTER(I64)]
        L.gpex_normals.argtypes = [P, U64, C.c_uint32, I64, I64, P, I64]
        L.gpex_trmm_sim.argtypes = [P, P, I64, U64, P, P, I64, C.POINTER(Diag)]
        L.gpex_krige.argtypes = [P, P, I64, P, I64, P, I, C.POINTER(CovParams), D, I, P, P, P, C.POINTER(I64)]
        L.gpex_excursion_regions.argtypes = [P, P, I64, I64, I64, I64, P, P, P, P, D, D, P, P, P, P, P, P, P,
                                             C.POINTER(RegionStats)]
        L.gpex_excursion_regions_noalloc.argtypes = L.gpex_excursion_regions.argtypes
        L.gpex_excursion_regions_below.argtypes = L.gpex_excursion_regions.argtypes
        L.gpex_plan.argtypes = [P, I64, C.POINTER(PrecOpts), P, C.POINTER(Diag)]
        L.gpex_ctx_set_timing.argtypes = [P, I]
        L.gpex_ctx_timings.argtypes = [P, P]
        _lib = L
    return _lib


def version() -> str:
    return lib().gpex_version().decode()


def _ptr(t) -> Optional[int]:
    """Raw device pointer of a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libgpex must be contiguous")
    return t.data_ptr()


def _cm(view) -> Optional[int]:
    """Pointer of a column-major matrix given as a 2-D view whose transpose is contiguous."""
    if view is None:
        return None
    if view.dim() != 2 or not view.T.is_contiguous():
        raise ValueError("matrices are passed column-major: a 2-D view whose .T is contiguous")
    return view.data_ptr()


def _dev_check(t, ctx, dtype=None):
    if t is None:
        return
    if t.device.type != "cuda" or t.device.index != ctx.device:
        raise ValueError(f"tensor on {t.device}, context on cuda:{ctx.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")


class Context:
    """A library context bound to one device and one torch stream (default: the current one).

    The library's device memory (tile storage, workspaces) comes from torch's caching allocator on
    that stream, so repeated runs reuse cached blocks instead of calling hipMalloc / hipFree."""

    def __init__(self, device: int = 0, stream=None, torch_alloc: bool = True):
        import torch
        self.device = device
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        sp = self.stream.cuda_stream

        def _alloc(nbytes, _user):
            try:
                return torch.cuda.caching_allocator_alloc(int(nbytes), device, sp)
            except Exception:   # out of memory: the library reports GPEX_ERR_NOMEM
                return None

        def _free(ptr, _user):
            torch.cuda.caching_allocator_delete(ptr)

        # the callbacks must live as long as anything allocated through them
        self._alloc = _ALLOC_FN(_alloc) if torch_alloc else _ALLOC_FN()
        self._free = _FREE_FN(_free) if torch_alloc else _FREE_FN()
        h = C.c_void_p()
        rc = lib().gpex_ctx_create(device, C.c_void_p(sp), self._alloc, self._free, None, C.byref(h))
        if rc != 0:
            raise GpexError(rc, "gpex_ctx_create failed")
        self.h = h

    def check(self, rc: int, allow=(0,)) -> int:
        if rc not in allow:
            raise GpexError(rc, lib().gpex_last_error(self.h).decode())
        return rc

    def close(self):
        if getattr(self, "h", None):
            lib().gpex_ctx_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_timing(self, on: bool):
        self.check(lib().gpex_ctx_set_timing(self.h, int(on)))

    def set_serial(self, on: bool):
        """Serial schedule: every launch on the context stream (bitwise the same results)."""
        self.check(lib().gpex_ctx_set_serial(self.h, int(on)))

    def release_workspace(self):
        self.check(lib().gpex_ctx_release_workspace(self.h))

    def timings(self) -> dict:
        out = (C.c_double * 32)()
        self.check(lib().gpex_ctx_timings(self.h, out))
        v = list(out)
        return {"potrf_ms": v[0],
                "update_ms": {"fp64": v[1], "fp32": v[4], "fp16": v[7]},
                "update_launches": {"fp64": int(v[2]), "fp32": int(v[5]), "fp16": int(v[8])},
                "update_flops": {"fp64": v[3], "fp32": v[6], "fp16": v[9]},
                "update_flops_exact": {"fp64": v[12], "fp32": v[13], "fp16": v[14]},
                "update_busy_ms": {"fp64": v[15], "fp32": v[16], "fp16": v[17]},
                "trmm_ms": v[10], "trmm_kernels_ms": v[11], "trmm_rows_ms": v[18],
                "trmm_rows_with_diagonal": bool(v[19])}


@dataclasses.dataclass
class Tiled:
    """Library-owned tiled symmetric matrix / factor (released with close())."""
    ctx: Context
    h: C.c_void_p
    diag: dict
    status: int
    potrf_status: int = 0

    def info(self) -> dict:
        n, nb, nt, s = C.c_int64(), C.c_int(), C.c_int64(), C.c_double()
        lib().gpex_tiled_info(self.h, C.byref(n), C.byref(nb), C.byref(nt), None, C.byref(s))
        pmap = np.zeros((nt.value, nt.value), dtype=np.uint8)
        lib().gpex_tiled_info(self.h, None, None, None, pmap.ctypes.data, None)
        return {"n": n.value, "nb": nb.value, "nt": nt.value, "s": s.value, "map": pmap}

    def stats(self) -> np.ndarray:
        nt = self.info()["nt"]
        st = np.zeros(3 * nt * (nt + 1) // 2)
        self.ctx.check(lib().gpex_tiled_stats(self.h, st.ctypes.data))
        return st.reshape(-1, 3)

    def to_dense(self, out=None):
        import torch
        n = self.info()["n"]
        if out is None:
            out = torch.empty((n, n), dtype=torch.float64, device=f"cuda:{self.ctx.device}")
        # column-major n x n == row-major transpose: out.T is the matrix
        self.ctx.check(lib().gpex_tiled_to_dense(self.ctx.h, self.h, _ptr(out), n))
        return out.T

    def block(self, r0: int, c0: int, rows: int, cols: int):
        """Unscaled sub-block [r0, r0+rows) x [c0, c0+cols) as a column-major rows x cols view."""
        out = colmajor(rows, cols, self.ctx)
        self.ctx.check(lib().gpex_tiled_block(self.ctx.h, self.h, r0, c0, rows, cols, _cm(out), rows))
        return out

    def block_raw(self, r0: int, c0: int, rows: int, cols: int, fp16_copy: bool = False, diag_parts: bool = False):
        """Stored values of a block, exactly, without unscaling; fp16_copy: the FP16 copy of the
        off-diagonal factor tiles; diag_parts: the diagonal tiles as the sum of their two FP16 parts."""
        which = 2 if diag_parts else int(fp16_copy)
        out = colmajor(rows, cols, self.ctx)
        self.ctx.check(lib().gpex_tiled_block_raw(self.ctx.h, self.h, which, r0, c0, rows, cols, _cm(out), rows))
        return out

    def close(self):
        if self.h:
            lib().gpex_tiled_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cov_gen(ctx: Context, loc, n: int, params: dict, nb: int, amp: int = 0, tol: float = 0.0,
            allow_fp16: bool = True, nt_rule: bool = True, diag_add=None, auto_tol: bool = False,
            fp16_dest: bool = False) -> Tiled:
    """gpex_cov_gen.  loc: float64 device tensor of 2n values (x then y)."""
    import torch
    _dev_check(loc, ctx, torch.float64)
    _dev_check(diag_add, ctx, torch.float64)
    cp = CovParams(int(params.get("kind", 0)), float(params["sigma2"]), float(params["range"]),
                   float(params.get("nu", 0.5)), float(params.get("nugget", 0.0)))
    po = PrecOpts(int(amp), float(tol), int(allow_fp16), int(not nt_rule), int(auto_tol), int(fp16_dest))
    h = C.c_void_p()
    d = Diag()
    rc = lib().gpex_cov_gen(ctx.h, _ptr(loc), n, _ptr(diag_add), C.byref(cp), nb, C.byref(po), C.byref(h),
                            C.byref(d))
    ctx.check(rc, allow=(OK, WARN_CHECKS_FAILED, WARN_FP16_OVERFLOW))
    return Tiled(ctx, h, d.to_dict(), rc)


def potrf_mp(ctx: Context, a: Tiled) -> int:
    """gpex_potrf_mp; returns info (0 or the failing column); raises on error.  The status
    (OK or WARN_FP16_OVERFLOW) is kept in a.potrf_status."""
    info = C.c_int64()
    rc = lib().gpex_potrf_mp(ctx.h, a.h, C.byref(info))
    a.potrf_status = rc
    if rc == ERR_NOT_SPD:
        return info.value
    ctx.check(rc, allow=(OK, WARN_FP16_OVERFLOW))
    if rc == WARN_FP16_OVERFLOW:
        a.diag["fp16_overflow"] = 1
    return info.value


def normals(ctx: Context, seed: int, stream: int, n: int, nsim: int, out=None):
    """gpex_normals -> column-major n x nsim view."""
    if out is None:
        out = colmajor(n, nsim, ctx)
    ctx.check(lib().gpex_normals(ctx.h, seed, stream, n, nsim, _cm(out), n))
    return out


def plan(stats, nt: int, amp: int = 1, tol: float = 0.0, allow_fp16: bool = True, nt_rule: bool = True,
         auto_tol: bool = False):
    """gpex_plan (host only): precision map and diagnostics from tile statistics."""
    st = np.ascontiguousarray(stats, dtype=np.float64).reshape(-1)
    if st.size != 3 * nt * (nt + 1) // 2:
        raise ValueError("stats must hold 3 values per lower tile")
    pmap = np.zeros((nt, nt), dtype=np.uint8)
    po = PrecOpts(int(amp), float(tol), int(allow_fp16), int(not nt_rule), int(auto_tol), 0)
    d = Diag()
    rc = lib().gpex_plan(st.ctypes.data, nt, C.byref(po), pmap.ctypes.data, C.byref(d))
    if rc != 0:
        raise GpexError(rc, "gpex_plan failed")
    return pmap, d.to_dict()


def colmajor(rows: int, cols: int, ctx: "Context", dtype=None):
    """An uninitialised column-major rows x cols device matrix (a view of a (cols, rows) tensor)."""
    import torch
    return torch.empty((cols, rows), dtype=dtype or torch.float64, device=f"cuda:{ctx.device}").T


def trmm_sim(ctx: Context, L: Tiled, nsim: int, seed: int = 0, Z=None, M=None, want_diag=True, status=False):
    """gpex_trmm_sim.  Z: explicit normals, column-major n x nsim view (or None: seeded normals).
    Returns (M as a column-major n x nsim view, diag dict or None), plus the status code (OK or
    WARN_FP16_OVERFLOW) when status=True."""
    import torch
    n = L.info()["n"]
    if M is None:
        M = colmajor(n, nsim, ctx)
    _dev_check(Z, ctx, torch.float64)
    _dev_check(M, ctx, torch.float64)
    d = Diag()
    rc = lib().gpex_trmm_sim(ctx.h, L.h, nsim, seed, _cm(Z), _cm(M), n, C.byref(d) if want_diag else None)
    ctx.check(rc, allow=(OK, WARN_FP16_OVERFLOW))
    out = (M, (d.to_dict() if want_diag else None))
    return out + (rc,) if status else out


def krige(ctx: Context, loc_o, n_o: int, loc_p, n_p: int, y_o, k_trend: int, params: dict, tau2: float,
          nb: int):
    """gpex_krige -> (W as n_o x n_p view, zhat, v, info)."""
    import torch
    dev = f"cuda:{ctx.device}"
    W = torch.empty((n_p, n_o), dtype=torch.float64, device=dev)
    zhat = torch.empty(n_p, dtype=torch.float64, device=dev)
    v = torch.empty(n_p, dtype=torch.float64, device=dev)
    cp = CovParams(int(params.get("kind", 0)), float(params["sigma2"]), float(params["range"]),
                   float(params.get("nu", 0.5)), 0.0)
    info = C.c_int64()
    rc = lib().gpex_krige(ctx.h, _ptr(loc_o), n_o, _ptr(loc_p), n_p, _ptr(y_o), k_trend, C.byref(cp), tau2, nb,
                          _ptr(W), _ptr(zhat), _ptr(v), C.byref(info))
    if rc == ERR_NOT_SPD:
        return None, None, None, info.value
    ctx.check(rc)
    return W.T, zhat, v, info.value


def excursion_regions(ctx: Context, M, n_p: int, n_o: int, nsim: int, u: float, level: float = 0.9, W=None,
                      y_o=None, zhat=None, v=None, want_S=False, noalloc=False, counts=None, sizes=None,
                      below=False):
    """gpex_excursion_regions (gpex_excursion_regions_noalloc with noalloc=True, which needs
    want_S when n_o > 0; gpex_excursion_regions_below, the negative excursion set, with below=True).  M: column-major (n_p + n_o) x nsim view; W: column-major n_o x n_p view.
    counts / sizes: optional int64 (n_p) / int32 (nsim) device outputs to reuse (the call writes
    every entry).  Returns dict with counts, sizes, and (with zhat) psi, phi, cin, cout, q_in,
    q_out, n_psi, n_phi, status."""
    import torch
    dev = f"cuda:{ctx.device}"
    ldm = n_p + n_o
    if counts is None:
        counts = torch.empty(n_p, dtype=torch.int64, device=dev)
    if sizes is None:
        sizes = torch.empty(nsim, dtype=torch.int32, device=dev)
    if counts.numel() != n_p or counts.dtype != torch.int64 or sizes.numel() != nsim or sizes.dtype != torch.int32:
        raise ValueError("counts must be int64 of n_p entries and sizes int32 of nsim entries")
    S = torch.empty((nsim, n_p), dtype=torch.float64, device=dev) if want_S else None
    out = {"counts": counts, "sizes": sizes}
    psi = phi = cin = cout = None
    st = RegionStats()
    if zhat is not None:
        psi = np.zeros(nsim)
        phi = np.zeros(nsim)
        cin = torch.zeros(n_p, dtype=torch.uint8, device=dev)
        cout = torch.zeros(n_p, dtype=torch.uint8, device=dev)
    if M.shape[0] != ldm or M.shape[1] != nsim:
        raise ValueError("M must be (n_p + n_o) x nsim")
    if noalloc and below:
        raise ValueError("the allocation-free entry point computes the positive excursion set only")
    fn = (lib().gpex_excursion_regions_noalloc if noalloc else
          lib().gpex_excursion_regions_below if below else lib().gpex_excursion_regions)
    rc = fn(
        ctx.h, _cm(M), ldm, n_p, n_o, nsim, _cm(W), _ptr(y_o), _ptr(zhat), _ptr(v), u, level,
        _ptr(counts), _ptr(sizes), psi.ctypes.data if psi is not None else None,
        phi.ctypes.data if phi is not None else None, _ptr(cin), _ptr(cout), _ptr(S), C.byref(st))
    if S is not None:
        S = S.T
    ctx.check(rc, allow=(OK, ERR_MSPE_NONPOS, ERR_EMPTY_SAMPLE))
    out["status"] = rc
    if S is not None:
        out["S"] = S
    if zhat is not None:
        out.update(psi=psi, phi=phi, cin=cin, cout=cout, q_in=st.q_in, q_out=st.q_out, n_psi=st.n_psi,
                   n_phi=st.n_phi)
    return out
