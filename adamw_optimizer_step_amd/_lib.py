"""ctypes declarations of the C ABI in ``include/muon_adamw.h``.

Loads ``libmuonadamw.so`` from this package directory.  There is no fallback:
if the library is missing the import fails with instructions to build it.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuonadamw.so")

MO_OK, MO_EINVAL, MO_ESHAPE, MO_ECONFLICT, MO_EEMPTY, MO_EDTYPE, MO_EWORKSPACE, MO_EHIP, \
    MO_EALIGN = range(9)
MO_F32, MO_BF16 = 0, 1
MO_NS_BF16, MO_NS_F32 = 0, 1
MO_ROLE_MATRIX, MO_ROLE_EMBEDDING, MO_ROLE_HEAD, MO_ROLE_NORM = range(4)
MO_ALG_SKIP, MO_ALG_ADAMW, MO_ALG_MUON = -1, 0, 1
MO_MAX_NDIM = 8
MO_MAX_SPLIT = 8
MO_NS_MAX_STEPS = 64
MO_MAX_GROUPS = 256

ROLE_CODES = {"matrix": MO_ROLE_MATRIX, "embedding": MO_ROLE_EMBEDDING, "head": MO_ROLE_HEAD,
              "norm": MO_ROLE_NORM}

vp = C.c_void_p
i32 = C.c_int32
i64 = C.c_int64
f32 = C.c_float


class MomentumItem(C.Structure):
    _fields_ = [("grad", vp), ("momentum", vp), ("dir", vp), ("numel", i64),
                ("grad_dtype", i32), ("dir_dtype", i32)]


class NsItem(C.Structure):
    _fields_ = [("inp", vp), ("out", vp), ("rows", i64), ("cols", i64), ("ld_in", i64),
                ("ld_out", i64), ("in_dtype", i32), ("out_dtype", i32)]


class AdamwItem(C.Structure):
    _fields_ = [("param", vp), ("grad", vp), ("exp_avg", vp), ("exp_avg_sq", vp),
                ("numel", i64), ("dtype", i32), ("step", i32), ("weight_decay", f32),
                ("reserved", f32)]


class ParamDesc(C.Structure):
    _fields_ = [("name", C.c_char_p), ("ident", i64), ("ndim", i32), ("role", i32),
                ("shape", i64 * MO_MAX_NDIM), ("no_decay", i32), ("requires_grad", i32),
                ("view_ndim", i32), ("nsplit", i32), ("view", i64 * MO_MAX_NDIM),
                ("split", i64 * MO_MAX_SPLIT), ("exclude_mask", C.c_uint32), ("reserved", i32)]


class RouteOut(C.Structure):
    _fields_ = [("algorithm", i32), ("decay", i32), ("group", i32), ("nslices", i32)]


class Param(C.Structure):
    _fields_ = [("desc", ParamDesc), ("param", vp), ("grad", vp), ("dtype", i32),
                ("reserved", i32), ("momentum", vp), ("normuon_v", vp), ("exp_avg", vp),
                ("exp_avg_sq", vp)]


class HParams(C.Structure):
    _fields_ = [("muon_lr", f32), ("muon_wd", f32), ("mu", f32), ("nesterov", i32),
                ("ns_steps", i32), ("ns_precision", i32),
                ("ns_coeffs", (f32 * 3) * MO_NS_MAX_STEPS), ("normuon", i32),
                ("normuon_beta2", f32), ("normuon_eps", f32), ("adamw_lr", f32),
                ("beta1", f32), ("beta2", f32), ("eps", f32), ("adamw_wd", f32),
                ("max_norm", f32), ("spectral_cap", f32), ("spectral_iters", i32)]


class SpectralItem(C.Structure):
    _fields_ = [("b", vp), ("rows", i64), ("cols", i64), ("ld", i64)]


class NsOptions(C.Structure):
    _fields_ = [("gram_space", i32), ("big_tile_min_work", i32), ("few_tile_max", i32),
                ("reserved", i32)]


class PlanOptions(C.Structure):
    _fields_ = [("ns", NsOptions), ("keep_ns_output", i32), ("reserved", i32)]


class StepArgs(C.Structure):
    _fields_ = [("muon_lr", f32), ("adamw_lr", f32), ("norm_out", vp), ("group_lr", C.POINTER(f32)),
                ("n_group_lr", i32), ("reserved", i32)]


class Group(C.Structure):
    _fields_ = [("algorithm", i32), ("nparams", i32), ("params", C.POINTER(Param)),
                ("hp", HParams)]


class LrSchedule(C.Structure):
    _fields_ = [("peak", C.c_double), ("warmup_tokens", C.c_double),
                ("stable_end_tokens", C.c_double), ("end_tokens", C.c_double),
                ("floor", C.c_double)]


#: (name, restype, argtypes) of every function the header declares.
SIGNATURES = [
    ("mo_status_str", C.c_char_p, [i32]),
    ("mo_last_error", C.c_char_p, []),
    ("mo_version", C.c_char_p, []),
    ("muon_momentum_workspace_bytes", C.c_size_t, [i32]),
    ("muon_momentum", i32, [C.POINTER(MomentumItem), i32, f32, i32, vp, C.c_size_t, vp]),
    ("mo_ns_options_default", None, [C.POINTER(NsOptions)]),
    ("ns_workspace_bytes", C.c_size_t, [C.POINTER(NsItem), i32, C.POINTER(f32), i32, i32,
                                        C.POINTER(NsOptions)]),
    ("ns_orthogonalize_batched", i32, [C.POINTER(NsItem), i32, C.POINTER(f32), i32, i32,
                                       C.POINTER(NsOptions), vp, C.c_size_t, vp]),
    ("muon_spectral_workspace_bytes", C.c_size_t, [C.POINTER(SpectralItem), i32]),
    ("muon_spectral_estimate", i32, [C.POINTER(SpectralItem), i32, i32, vp, vp, C.c_size_t,
                                     vp]),
    ("normuon_rownorm", i32, [vp, i32, i64, i64, i64, vp, f32, f32, vp]),
    ("muon_update", i32, [vp, i32, vp, i32, i64, i64, i64, i64, f32, f32, f32, vp]),
    ("adamw_workspace_bytes", C.c_size_t, [C.POINTER(AdamwItem), i32]),
    ("adamw_clip_step", i32, [C.POINTER(AdamwItem), i32, f32, f32, f32, f32, f32, vp, vp,
                              C.c_size_t, vp]),
    ("adamw_clip_step_noalloc", i32, [C.POINTER(AdamwItem), i32, f32, f32, f32, f32, f32, vp,
                                      vp]),
    ("mo_route", i32, [C.POINTER(ParamDesc), i32, C.POINTER(RouteOut), C.POINTER(i32)]),
    ("mo_expand_view", i32, [i64, i64, i32, C.POINTER(i64), i32, C.POINTER(i64),
                             C.POINTER(i64), i32, C.POINTER(i32)]),
    ("mo_plan_options_default", None, [C.POINTER(PlanOptions)]),
    ("mo_plan_create", i32, [C.POINTER(Param), i32, C.POINTER(HParams), C.POINTER(PlanOptions),
                             C.POINTER(vp)]),
    ("mo_plan_create_groups", i32, [C.POINTER(Group), i32, C.POINTER(PlanOptions),
                                    C.POINTER(vp)]),
    ("mo_plan_num_params", i32, [vp]),
    ("mo_plan_num_groups", i32, [vp]),
    ("mo_plan_destroy", None, [vp]),
    ("mo_plan_workspace_bytes", C.c_size_t, [vp]),
    ("mo_plan_route", i32, [vp, C.POINTER(RouteOut), i32]),
    ("mo_plan_num_slices", i32, [vp]),
    ("mo_plan_slices", i32, [vp, C.POINTER(i64), i32]),
    ("mo_plan_get_steps", i32, [vp, C.POINTER(i32), i32]),
    ("mo_plan_set_steps", i32, [vp, C.POINTER(i32), i32]),
    ("mo_grouped_step", i32, [vp, C.POINTER(StepArgs), vp, C.c_size_t, vp]),
    ("mo_diag_copy", i32, [vp, vp, i64, vp]),
    ("mo_plan_ns_output", i32, [vp, i32, vp, C.POINTER(vp), C.POINTER(i64), C.POINTER(i32)]),
    ("mo_plan_keep_ns_output", i32, [vp, i32]),
    ("mo_plan_fuses_update", i32, [vp]),
    ("mo_plan_gram_space", i32, [vp]),
    ("mo_plan_slice_algorithms", i32, [vp, C.POINTER(i32), i32]),
    ("mo_abi_struct_size", C.c_size_t, [i32]),
    ("mo_lr_at", i32, [C.POINTER(LrSchedule), C.c_double, C.POINTER(C.c_double)]),
    ("mo_timing_enable", i32, [i32]),
    ("mo_timing_read", i32, [i32, C.POINTER(C.c_double), C.POINTER(i64)]),
]

KERNEL_CLASSES = ["momentum", "ns_stats", "ns_scale", "ns_prep", "ns_gemm", "ns_final", "rows",
                  "adam_sumsq", "adam_norm", "adam_apply", "ns_small", "spectral"]

#: ctypes mirror of each struct, in the order of mo_abi_struct_size's index.
ABI_STRUCTS = [MomentumItem, NsItem, AdamwItem, ParamDesc, RouteOut, Param, HParams, StepArgs,
               LrSchedule, NsOptions, PlanOptions, Group, SpectralItem]


class LibraryError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {status_name(status)}: {msg}")
        self.status = status


_LIB = None


def lib() -> C.CDLL:
    """The loaded library (raises ImportError if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m adamw_optimizer_step_amd.build`"
                " (hipcc, gfx950). There is no CPU fallback.")
        L = C.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_name(s: int) -> str:
    return lib().mo_status_str(s).decode()


def check(fn: str, status: int) -> None:
    if status != MO_OK:
        raise LibraryError(fn, status, lib().mo_last_error().decode())
