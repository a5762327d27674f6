"""Python binding of the JoLT codec C ABI (include/jolt.h).

Argument marshalling only: every step of the codec runs in libjolt.so's HIP
kernels and host code.  PyTorch provides device memory and the current HIP
stream.  Names follow the C entry points: ``allocate``, ``factors``,
``rotation``, ``encode``, ``decode``, ``quantize``, plus the host-only
``plan_from_spectra`` and ``rotation_host``.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from ._lib import AllocReq, Choice, Plan, Shape, check, lib

D_FEATURES = 128


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return _lib.JOLT_BF16
    if dt == torch.float32:
        return _lib.JOLT_F32
    raise TypeError(f"unsupported dtype {dt}")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == _lib.JOLT_BF16 else torch.float32


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_buf(t: torch.Tensor, device: torch.device, name: str, nbytes: int = 0) -> None:
    """A contiguous tensor on `device` holding at least `nbytes` bytes (cheap
    when it holds: this runs per record on the decode's host path)."""
    if (isinstance(t, torch.Tensor) and t.device == device and t.is_contiguous()
            and t.numel() * t.element_size() >= nbytes):
        return
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.device == device, f"{name} must be on {device}, not {t.device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _check_out(o: torch.Tensor, device: torch.device, H: int, T: int, dtype: torch.dtype, name: str) -> None:
    _check_buf(o, device, name)
    _need(o.shape == (H, T, D_FEATURES), f"{name} must have shape {(H, T, D_FEATURES)}, not {tuple(o.shape)}")
    _need(o.dtype == dtype, f"{name} must be {dtype}, not {o.dtype}")


def _blob_sizes(shape: Shape, choices) -> list:
    """jolt_blob_bytes per record (one library call per distinct choice)."""
    memo = {}
    out = []
    for c in choices:
        key = tuple(c)
        if key not in memo:
            memo[key] = lib().jolt_blob_bytes(C.byref(shape), Choice(*key))
        out.append(memo[key])
    return out


def _check_factor(f: torch.Tensor, device, rows: int, cols: int, name: str) -> None:
    _need(isinstance(f, torch.Tensor) and f.dtype == torch.float32 and f.dim() == 2 and f.stride(1) == 1,
          f"{name} must be fp32 [rows, ld] with unit column stride")
    _need(f.device == torch.device(device), f"{name} must be on {device}")
    _need(f.shape[0] >= rows and f.shape[1] >= cols and f.stride(0) >= cols,
          f"{name} {tuple(f.shape)} must have at least {rows} rows and {cols} columns")


def make_shape(H: int, T: int, D: int, dtype) -> Shape:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return Shape(H, T, D, code)


def make_req(H, T, D, dtype, n_layers, ratio, method="exact", bits=(1, 2, 3, 4), group_layers=4,
             seed=0, oversample=10, power_iters=1, r_T_cap=0, step_T=0, step_D=0) -> AllocReq:
    menu = (C.c_int32 * 4)(*(list(bits) + [0] * (4 - len(bits))))
    m = _lib.JOLT_FLASH if method == "flash" else _lib.JOLT_EXACT
    return AllocReq(make_shape(H, T, D, dtype), n_layers, group_layers, float(ratio), menu, len(bits), m,
                    oversample, power_iters, r_T_cap, step_T, step_D, seed)


# ----------------------------------------------------------------- sizes
def blob_bytes(H, T, D, choice, dtype=torch.bfloat16) -> int:
    return lib().jolt_blob_bytes(C.byref(make_shape(H, T, D, dtype)), Choice(*choice))


def workspace_bytes(req: AllocReq) -> int:
    return lib().jolt_workspace_bytes(C.byref(req))


def spectrum_len(req: AllocReq) -> int:
    return lib().jolt_spectrum_len(C.byref(req))


# -------------------------------------------------------------- rotation
def rotation(seed: int, D: int = D_FEATURES, device="cuda") -> torch.Tensor:
    """Prepared rotation buffer (fp32 Q, fp32 Q^T, bf16 Q^T) on the device."""
    n = lib().jolt_rotation_bytes(D)
    buf = torch.empty(n, dtype=torch.uint8, device=device)
    check(lib().jolt_rotation(seed, D, buf.data_ptr(), n, _stream(buf.device)), "jolt_rotation")
    return buf


def rotation_from(Q: np.ndarray, device="cuda") -> torch.Tensor:
    """Prepared rotation buffer from a host orthogonal matrix (identity: the
    unrotated quantizer)."""
    Qh = np.ascontiguousarray(Q, dtype=np.float64)
    D = Qh.shape[0]
    _need(Qh.shape == (D, D), "Q must be square")
    n = lib().jolt_rotation_bytes(D)
    buf = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    check(lib().jolt_rotation_from(Qh.ctypes.data_as(C.POINTER(C.c_double)), D, buf.data_ptr(), n,
                                   _stream(buf.device)), "jolt_rotation_from")
    return buf


def rotation_host(seed: int, D: int = D_FEATURES) -> np.ndarray:
    out = np.empty((D, D), dtype=np.float64)
    check(lib().jolt_rotation_host(seed, D, out.ctypes.data_as(C.POINTER(C.c_double))),
          "jolt_rotation_host")
    return out


def rng_normal(seed: int, tag: int, index: int) -> float:
    return lib().jolt_rng_normal(seed, tag, index)


# -------------------------------------------------------------- allocate
@dataclass
class Allocation:
    req: AllocReq
    workspace: torch.Tensor
    choice: dict           # (group, kind) -> (r_T, r_D, bits)
    tensor_bytes: list
    total_bytes: int
    budget_bytes: int
    objective: float
    r_T_cap: int
    spectra_T: np.ndarray | None
    spectra_D: np.ndarray | None
    frob2: np.ndarray | None

    def choice_of(self, layer: int, kind: int):
        return self.choice[(layer // self.req.group_layers, kind)]

    def factors(self, tensor: int):
        """(U_T [T, ld] fp32, U_D [D, D] fp32) views into the workspace."""
        ut, ldt, ud = C.c_void_p(), C.c_int32(), C.c_void_p()
        check(lib().jolt_factors(C.byref(self.req), self.workspace.data_ptr(), tensor, C.byref(ut),
                                 C.byref(ldt), C.byref(ud)), "jolt_factors")
        base = self.workspace.data_ptr()
        T, D = self.req.shape.T, self.req.shape.D
        w32 = self.workspace.view(torch.float32)
        o1 = (ut.value - base) // 4
        o2 = (ud.value - base) // 4
        return (w32[o1:o1 + T * ldt.value].view(T, ldt.value), w32[o2:o2 + D * D].view(D, D))


def _plan_arrays(req: AllocReq, spectra: bool):
    L = req.n_layers
    ng = (L + req.group_layers - 1) // req.group_layers
    choice = (Choice * (2 * ng))()
    tb = (C.c_uint64 * (2 * L))()
    plan = Plan(choice, tb, None, None, None, 0.0, 0, 0, 0)
    arrs = {}
    if spectra:
        lt = max(1, spectrum_len(req))
        arrs["T"] = np.zeros((2 * L, lt))
        arrs["D"] = np.zeros((2 * L, req.shape.D))
        arrs["f"] = np.zeros(2 * L)
        plan.spectra_T = arrs["T"].ctypes.data_as(C.POINTER(C.c_double))
        plan.spectra_D = arrs["D"].ctypes.data_as(C.POINTER(C.c_double))
        plan.frob2 = arrs["f"].ctypes.data_as(C.POINTER(C.c_double))
    return plan, choice, tb, ng, arrs


def _plan_dict(req, plan, choice, tb, ng):
    ch = {(g, k): choice[2 * g + k].tuple() for g in range(ng) for k in (0, 1)}
    return ch, [int(tb[i]) for i in range(2 * req.n_layers)]


def allocate(tensors, ratio: float, method: str = "exact", bits=(1, 2, 3, 4), group_layers: int = 4,
             seed: int = 0, oversample: int = 10, power_iters: int = 1, r_T_cap: int = 0,
             step_T: int = 0, step_D: int = 0, spectra: bool = True) -> Allocation:
    """Spectra, factors and the Lagrangian-dual plan of a cache.

    tensors[layer] = (K, V), each a contiguous [H, T, 128] bf16/fp32 CUDA tensor.
    """
    L = len(tensors)
    x0 = tensors[0][0]
    H, T, D = x0.shape
    req = make_req(H, T, D, x0.dtype, L, ratio, method, bits, group_layers, seed, oversample,
                   power_iters, r_T_cap, step_T, step_D)
    ptrs = (C.c_void_p * (2 * L))()
    for l in range(L):
        for k in (0, 1):
            t = tensors[l][k]
            if t.shape != x0.shape or t.dtype != x0.dtype or not t.is_contiguous():
                raise ValueError("all tensors must be contiguous with one shape and dtype")
            ptrs[2 * l + k] = t.data_ptr()
    nws = workspace_bytes(req)
    if nws == 0:
        check(_lib.JOLT_EINVAL, "jolt_workspace_bytes")
    ws = torch.empty(nws, dtype=torch.uint8, device=x0.device)
    plan, choice, tb, ng, arrs = _plan_arrays(req, spectra)
    check(lib().jolt_allocate(C.byref(req), ptrs, ws.data_ptr(), nws, _stream(x0.device), C.byref(plan)),
          "jolt_allocate")
    ch, tbl = _plan_dict(req, plan, choice, tb, ng)
    return Allocation(req, ws, ch, tbl, plan.total_bytes, plan.budget_bytes, plan.objective,
                      plan.r_T_cap, arrs.get("T"), arrs.get("D"), arrs.get("f"))


def plan_from_spectra(req: AllocReq, spectra_T: np.ndarray, spectra_D: np.ndarray, frob2: np.ndarray):
    """The Lagrangian dual alone on host spectra (no device)."""
    sT = np.ascontiguousarray(spectra_T, dtype=np.float64)
    sD = np.ascontiguousarray(spectra_D, dtype=np.float64)
    f2 = np.ascontiguousarray(frob2, dtype=np.float64)
    plan, choice, tb, ng, _ = _plan_arrays(req, False)
    P = C.POINTER(C.c_double)
    check(lib().jolt_plan_from_spectra(C.byref(req), sT.ctypes.data_as(P), sT.shape[1],
                                       sD.ctypes.data_as(P), f2.ctypes.data_as(P), C.byref(plan)),
          "jolt_plan_from_spectra")
    ch, tbl = _plan_dict(req, plan, choice, tb, ng)
    return dict(choice=ch, tensor_bytes=tbl, total_bytes=plan.total_bytes, budget=plan.budget_bytes,
                objective=plan.objective, r_T_cap=plan.r_T_cap)


# ------------------------------------------------------- encode / decode
def encode(x: torch.Tensor, choice, U_T: torch.Tensor | None, U_D: torch.Tensor | None,
           rot: torch.Tensor, seed: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """Compress one [H, T, 128] tensor into a device record (uint8 tensor)."""
    _need(x.dim() == 3 and x.shape[2] == D_FEATURES, f"x must be [H, T, {D_FEATURES}]")
    _check_buf(x, x.device, "x")
    H, T, D = x.shape
    shape = make_shape(H, T, D, x.dtype)
    ch = Choice(*choice)
    nb = lib().jolt_blob_bytes(C.byref(shape), ch)
    if nb == 0:
        check(_lib.JOLT_EINVAL, "jolt_blob_bytes")
    _check_buf(rot, x.device, "rot", lib().jolt_rotation_bytes(D))
    if out is not None:
        _check_buf(out, x.device, "out", nb)
    blob = out if out is not None else torch.empty(nb, dtype=torch.uint8, device=x.device)
    nws = lib().jolt_encode_workspace_bytes(C.byref(shape), ch)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device)
    if choice[0] > 0:
        _need(U_T is not None and U_D is not None, "a Tucker choice needs both factors")
        _check_factor(U_T, x.device, T, choice[0], "U_T")
        _check_factor(U_D, x.device, D, choice[1], "U_D")
    ut = U_T.data_ptr() if U_T is not None else None
    ud = U_D.data_ptr() if U_D is not None else None
    ldt = U_T.stride(0) if U_T is not None else 0
    ldd = U_D.stride(0) if U_D is not None else 0
    check(lib().jolt_encode(C.byref(shape), x.data_ptr(), ch, ut, ldt, ud, ldd, rot.data_ptr(), seed,
                            blob.data_ptr(), blob.numel(), ws.data_ptr(), ws.numel(),
                            _stream(x.device)), "jolt_encode")
    return blob


def encode_many(xs, choices, factors, rot: torch.Tensor, seed: int = 0, outs=None):
    """Compress several [H, T, 128] tensors of one shape and dtype into device
    records (the same bytes as encode() per tensor, in batched launches).
    factors[i] = (U_T, U_D) fp32 [rows, ld] with unit column stride (or
    (None, None) for a choice with r_T == 0); or the Allocation of the cache
    whose tensors xs are, in order (its factors are read in place)."""
    n = len(xs)
    if n == 0:
        return []
    x0 = xs[0]
    H, T, D = x0.shape
    shape = make_shape(H, T, D, x0.dtype)
    ch = (Choice * n)(*[Choice(*c) for c in choices])
    _need(x0.dim() == 3 and x0.shape[2] == D_FEATURES, f"tensors must be [H, T, {D_FEATURES}]")
    _need(len(choices) == n, "one choice per tensor")
    for x in xs:
        if x.shape != x0.shape or x.dtype != x0.dtype or not x.is_contiguous() or x.device != x0.device:
            raise ValueError("all tensors must be contiguous with one shape, dtype and device")
    _check_buf(rot, x0.device, "rot", lib().jolt_rotation_bytes(D))
    if outs is not None:
        _need(len(outs) == n, "one output record per tensor")
        for i, nb in enumerate(_blob_sizes(shape, choices)):
            _check_buf(outs[i], x0.device, f"outs[{i}]", nb)
        blobs = outs
    else:
        # one allocation cut into 256-aligned records
        sizes = _blob_sizes(shape, choices)
        offs, o = [], 0
        for nb in sizes:
            offs.append(o)
            o += (nb + 255) // 256 * 256
        buf = torch.empty(max(o, 1), dtype=torch.uint8, device=x0.device)
        blobs = [buf[a:a + nb] for a, nb in zip(offs, sizes)]
    xp = (C.c_void_p * n)(*[x.data_ptr() for x in xs])
    if isinstance(factors, Allocation):
        if n != 2 * factors.req.n_layers:
            raise ValueError("an Allocation supplies the factors of its whole cache")
        utp, udp = (C.c_void_p * n)(), (C.c_void_p * n)()
        ldt, ldd = (C.c_int32 * n)(), (C.c_int32 * n)(*([factors.req.shape.D] * n))
        check(lib().jolt_factors_many(C.byref(factors.req), factors.workspace.data_ptr(), 0, n, utp, ldt, udp),
              "jolt_factors_many")
    else:
        _need(len(factors) == n, "one factor pair per tensor")
        for i, (c, pair) in enumerate(zip(choices, factors)):
            if c[0] > 0:
                _need(pair[0] is not None and pair[1] is not None, "a Tucker choice needs both factors")
                _check_factor(pair[0], x0.device, T, c[0], f"factors[{i}][0]")
                _check_factor(pair[1], x0.device, D, c[1], f"factors[{i}][1]")
        utp = (C.c_void_p * n)(*[f[0].data_ptr() if f[0] is not None else None for f in factors])
        udp = (C.c_void_p * n)(*[f[1].data_ptr() if f[1] is not None else None for f in factors])
        ldt = (C.c_int32 * n)(*[f[0].stride(0) if f[0] is not None else 0 for f in factors])
        ldd = (C.c_int32 * n)(*[f[1].stride(0) if f[1] is not None else 0 for f in factors])
    bp = (C.c_void_p * n)(*[b.data_ptr() for b in blobs])
    bb = (C.c_size_t * n)(*[b.numel() for b in blobs])
    nws = lib().jolt_encode_many_workspace_bytes(n, C.byref(shape), ch)
    if nws == 0:
        check(_lib.JOLT_EINVAL, "jolt_encode_many_workspace_bytes")
    ws = torch.empty(nws, dtype=torch.uint8, device=x0.device)
    check(lib().jolt_encode_many(n, C.byref(shape), ch, xp, utp, ldt, udp, ldd, rot.data_ptr(), seed, bp, bb,
                                 ws.data_ptr(), ws.numel(), _stream(x0.device)), "jolt_encode_many")
    return blobs


def decode_workspace_bytes(H: int, T: int, choice, dtype=torch.bfloat16) -> int:
    return lib().jolt_decode_workspace_bytes(C.byref(make_shape(H, T, D_FEATURES, dtype)), Choice(*choice))


def decode(blob: torch.Tensor, H: int, T: int, choice, rot: torch.Tensor, dtype=torch.bfloat16,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Reconstruct [H, T, 128] from a record."""
    shape = make_shape(H, T, D_FEATURES, dtype)
    ch = Choice(*choice)
    nb = lib().jolt_blob_bytes(C.byref(shape), ch)
    if nb == 0:
        check(_lib.JOLT_EINVAL, "jolt_blob_bytes")
    _check_buf(blob, blob.device, "blob", nb)
    _check_buf(rot, blob.device, "rot", lib().jolt_rotation_bytes(D_FEATURES))
    if out is not None:
        _check_out(out, blob.device, H, T, dtype, "out")
    xh = out if out is not None else torch.empty((H, T, D_FEATURES), dtype=dtype, device=blob.device)
    nws = lib().jolt_decode_workspace_bytes(C.byref(shape), ch)
    if workspace is not None:
        _check_buf(workspace, blob.device, "workspace", nws)
    ws = workspace if workspace is not None else torch.empty(max(nws, 1), dtype=torch.uint8,
                                                              device=blob.device)
    check(lib().jolt_decode(C.byref(shape), ch, blob.data_ptr(), blob.numel(), rot.data_ptr(),
                            xh.data_ptr(), ws.data_ptr(), ws.numel(), _stream(blob.device)), "jolt_decode")
    return xh


def decode_many_workspace_bytes(H: int, T: int, choices, dtype=torch.bfloat16) -> int:
    arr = (Choice * len(choices))(*[Choice(*c) for c in choices])
    return lib().jolt_decode_many_workspace_bytes(len(choices), C.byref(make_shape(H, T, D_FEATURES, dtype)), arr)


def decode_many(blobs, H: int, T: int, choices, rot: torch.Tensor, outs, workspace: torch.Tensor,
                dtype=torch.bfloat16, validate: bool = True) -> None:
    """Reconstruct several records of one shape into the given output tensors.
    validate=False skips the per-buffer checks of this binding (for a caller
    repeating a call whose buffers it has already checked once); the C ABI
    still checks everything it can see."""
    n = len(blobs)
    _need(len(choices) == n and len(outs) == n, "one choice and one output per record")
    shape = make_shape(H, T, D_FEATURES, dtype)
    ch = (Choice * n)(*[Choice(*c) for c in choices])
    dev = workspace.device
    if validate:
        _check_buf(workspace, dev, "workspace", lib().jolt_decode_many_workspace_bytes(n, C.byref(shape), ch))
        _check_buf(rot, dev, "rot", lib().jolt_rotation_bytes(D_FEATURES))
        for i, nb in enumerate(_blob_sizes(shape, choices)):
            _check_buf(blobs[i], dev, f"blobs[{i}]", nb)
            _check_out(outs[i], dev, H, T, dtype, f"outs[{i}]")
    bp = (C.c_void_p * n)(*[b.data_ptr() for b in blobs])
    bb = (C.c_size_t * n)(*[b.numel() for b in blobs])
    op = (C.c_void_p * n)(*[o.data_ptr() for o in outs])
    check(lib().jolt_decode_many(n, C.byref(shape), ch, bp, bb, rot.data_ptr(), op, workspace.data_ptr(),
                                 workspace.numel(), _stream(workspace.device)), "jolt_decode_many")


def decode_many_static(blobs, H: int, T: int, choices, rot: torch.Tensor, outs, dtype=torch.bfloat16) -> None:
    """decode_many without a workspace: the library's per-GPU static scratch
    (no device allocation in the call; overlapping calls on one GPU race)."""
    n = len(blobs)
    _need(len(choices) == n and len(outs) == n, "one choice and one output per record")
    if n == 0:
        return
    shape = make_shape(H, T, D_FEATURES, dtype)
    ch = (Choice * n)(*[Choice(*c) for c in choices])
    dev = blobs[0].device
    _check_buf(rot, dev, "rot", lib().jolt_rotation_bytes(D_FEATURES))
    for i, nb in enumerate(_blob_sizes(shape, choices)):
        _check_buf(blobs[i], dev, f"blobs[{i}]", nb)
        _check_out(outs[i], dev, H, T, dtype, f"outs[{i}]")
    bp = (C.c_void_p * n)(*[b.data_ptr() for b in blobs])
    bb = (C.c_size_t * n)(*[b.numel() for b in blobs])
    op = (C.c_void_p * n)(*[o.data_ptr() for o in outs])
    check(lib().jolt_decode_many_static(n, C.byref(shape), ch, bp, bb, rot.data_ptr(), op, _stream(dev)),
          "jolt_decode_many_static")


def append_workspace_bytes(H: int, T: int, choice, n_new: int, dtype=torch.bfloat16) -> int:
    return lib().jolt_append_workspace_bytes(C.byref(make_shape(H, T, D_FEATURES, dtype)), Choice(*choice), n_new)


def append(base_blob: torch.Tensor, H: int, T: int, choice, x_new: torch.Tensor, rot: torch.Tensor, seed: int = 0,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Record of tokens appended to an encoded tensor (folding-in against the
    base record's stored factors); x_new [H, n_new, 128] in the base's dtype."""
    _need(x_new.dim() == 3 and x_new.shape[0] == H and x_new.shape[2] == D_FEATURES,
          f"x_new must be [{H}, n_new, {D_FEATURES}]")
    dev = x_new.device
    _check_buf(x_new, dev, "x_new")
    n_new = x_new.shape[1]
    base = make_shape(H, T, D_FEATURES, x_new.dtype)
    ch = Choice(*choice)
    _check_buf(base_blob, dev, "base_blob", lib().jolt_blob_bytes(C.byref(base), ch))
    _check_buf(rot, dev, "rot", lib().jolt_rotation_bytes(D_FEATURES))
    nb = lib().jolt_blob_bytes(C.byref(make_shape(H, n_new, D_FEATURES, x_new.dtype)), ch)
    nws = lib().jolt_append_workspace_bytes(C.byref(base), ch, n_new)
    if nb == 0 or nws == 0:
        check(_lib.JOLT_EINVAL, "jolt_append_workspace_bytes")
    if out is not None:
        _check_buf(out, dev, "out", nb)
    if workspace is not None:
        _check_buf(workspace, dev, "workspace", nws)
    blob = out if out is not None else torch.empty(nb, dtype=torch.uint8, device=dev)
    ws = workspace if workspace is not None else torch.empty(nws, dtype=torch.uint8, device=dev)
    check(lib().jolt_append(C.byref(base), ch, base_blob.data_ptr(), base_blob.numel(), x_new.data_ptr(), n_new,
                            rot.data_ptr(), seed, blob.data_ptr(), blob.numel(), ws.data_ptr(), ws.numel(),
                            _stream(dev)), "jolt_append")
    return blob


def attend_workspace_bytes(H: int, T: int, choice_k, choice_v, G: int, n_new: int,
                           dtype=torch.bfloat16) -> int:
    return lib().jolt_attend_workspace_bytes(C.byref(make_shape(H, T, D_FEATURES, dtype)), Choice(*choice_k),
                                             Choice(*choice_v), G, n_new)


def attend(blob_k, choice_k, blob_v, choice_v, H: int, T: int, q: torch.Tensor, G: int, rot: torch.Tensor,
           dtype=torch.bfloat16, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """softmax(q K^T / sqrt(D)) V over one layer's K and V records, decoded in
    registers.  q: fp32 [H * G, n_new, 128]; returns fp32 of q's shape."""
    _need(q.dim() == 3 and q.shape[0] == H * G and q.shape[2] == D_FEATURES and q.dtype == torch.float32,
          f"q must be fp32 [{H * G}, n_new, {D_FEATURES}]")
    dev = q.device
    _check_buf(q, dev, "q")
    n_new = q.shape[1]
    shape = make_shape(H, T, D_FEATURES, dtype)
    ck, cv = Choice(*choice_k), Choice(*choice_v)
    _check_buf(blob_k, dev, "blob_k", lib().jolt_blob_bytes(C.byref(shape), ck))
    _check_buf(blob_v, dev, "blob_v", lib().jolt_blob_bytes(C.byref(shape), cv))
    _check_buf(rot, dev, "rot", lib().jolt_rotation_bytes(D_FEATURES))
    nws = lib().jolt_attend_workspace_bytes(C.byref(shape), ck, cv, G, n_new)
    if nws == 0:
        check(_lib.JOLT_EINVAL, "jolt_attend_workspace_bytes")
    if workspace is not None:
        _check_buf(workspace, dev, "workspace", nws)
    ws = workspace if workspace is not None else torch.empty(nws, dtype=torch.uint8, device=dev)
    if out is not None:
        _need(out.shape == q.shape and out.dtype == torch.float32, "out must be fp32 of q's shape")
        _check_buf(out, dev, "out")
    o = out if out is not None else torch.empty_like(q)
    check(lib().jolt_attend(C.byref(shape), ck, blob_k.data_ptr(), blob_k.numel(), cv, blob_v.data_ptr(),
                            blob_v.numel(), rot.data_ptr(), q.data_ptr(), G, n_new, o.data_ptr(), ws.data_ptr(),
                            ws.numel(), _stream(dev)), "jolt_attend")
    return o


def xl_encode(xs, r: int):
    """Cross-layer SVD of tensors of one shape (one layer group's K or V):
    (basis bf16 [r, 128], coefficients [bf16 [H, T, r] per tensor], leading
    eigenvalues [r])."""
    n = len(xs)
    _need(n >= 1, "at least one tensor")
    x0 = xs[0]
    _need(x0.dim() == 3 and x0.shape[2] == D_FEATURES, f"tensors must be [H, T, {D_FEATURES}]")
    H, T, D = x0.shape
    for i, x in enumerate(xs):
        _need(x.shape == x0.shape and x.dtype == x0.dtype, "one shape and dtype")
        _check_buf(x, x0.device, f"xs[{i}]")
    shape = make_shape(H, T, D, x0.dtype)
    basis = torch.empty((r, D), dtype=torch.bfloat16, device=x0.device)
    coeffs = [torch.empty((H, T, r), dtype=torch.bfloat16, device=x0.device) for _ in range(n)]
    nws = lib().jolt_xl_workspace_bytes(n, C.byref(shape), r)
    if nws == 0:
        check(_lib.JOLT_EINVAL, "jolt_xl_workspace_bytes")
    ws = torch.empty(nws, dtype=torch.uint8, device=x0.device)
    lam = np.zeros(r)
    xp = (C.c_void_p * n)(*[x.data_ptr() for x in xs])
    cp = (C.c_void_p * n)(*[c.data_ptr() for c in coeffs])
    check(lib().jolt_xl_encode(n, C.byref(shape), xp, r, basis.data_ptr(), cp,
                               lam.ctypes.data_as(C.POINTER(C.c_double)), ws.data_ptr(), nws,
                               _stream(x0.device)), "jolt_xl_encode")
    return basis, coeffs, lam


def xl_decode(basis: torch.Tensor, coeffs, dtype=torch.bfloat16):
    """X^_i = C_i U~^T for every coefficient tensor, in `dtype`."""
    n = len(coeffs)
    r, D = basis.shape
    H, T, _ = coeffs[0].shape
    _check_buf(basis, basis.device, "basis", 2 * r * D)
    for i, c in enumerate(coeffs):
        _need(c.shape == (H, T, r) and c.dtype == torch.bfloat16, f"coeffs[{i}] must be bf16 {(H, T, r)}")
        _check_buf(c, basis.device, f"coeffs[{i}]")
    outs = [torch.empty((H, T, D), dtype=dtype, device=basis.device) for _ in range(n)]
    shape = make_shape(H, T, D, dtype)
    cp = (C.c_void_p * n)(*[c.data_ptr() for c in coeffs])
    op = (C.c_void_p * n)(*[o.data_ptr() for o in outs])
    check(lib().jolt_xl_decode(n, C.byref(shape), r, basis.data_ptr(), cp, op, _stream(basis.device)),
          "jolt_xl_decode")
    return outs


def quantize(y: torch.Tensor, bits: int):
    """Group quantizer alone: y [rows, 128] fp32 -> (scales [rows, 4, 2] bf16 bits as int16,
    codes [rows, 4, 4*bits] uint8)."""
    _need(y.dim() == 2 and y.shape[1] == D_FEATURES and y.dtype == torch.float32,
          f"y must be fp32 [rows, {D_FEATURES}]")
    _check_buf(y, y.device, "y")
    rows, D = y.shape
    sc = torch.empty((rows, D // 32, 2), dtype=torch.int16, device=y.device)
    cd = torch.empty((rows, D // 32, 4 * bits), dtype=torch.uint8, device=y.device)
    check(lib().jolt_quantize(y.data_ptr(), rows, D, bits, sc.data_ptr(), cd.data_ptr(),
                              _stream(y.device)), "jolt_quantize")
    return sc, cd


def header_parse(header: bytes):
    s, c, seed = Shape(), Choice(), C.c_uint64()
    buf = C.create_string_buffer(bytes(header), len(header))
    check(lib().jolt_header_parse(buf, len(header), C.byref(s), C.byref(c), C.byref(seed)),
          "jolt_header_parse")
    return (s.H, s.T, s.D, s.dtype), c.tuple(), seed.value


# -------------------------------------------------------------- profiling
def profile_enable(kernels: str | None = "*") -> None:
    """Profile the named kernels ("a,b", "*" for all); None or "" turns it off."""
    check(lib().jolt_profile_enable(kernels.encode() if kernels else None), "jolt_profile_enable")


def profile_query(kernel: str) -> dict:
    st = _lib.KernelStats()
    check(lib().jolt_profile_query(kernel.encode(), C.byref(st)), "jolt_profile_query")
    return dict(launches=st.launches, total_ms=st.total_ms, bytes=st.bytes, flops=st.flops)
