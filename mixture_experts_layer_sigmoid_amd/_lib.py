"""ctypes binding of libmoe_mi355x.so (include/moe_mi355x.h).

Argument marshalling only: every function takes torch tensors (device
memory) or None, passes their data pointers and the current HIP stream to
the C entry point of the same name, and raises MoEError on a non-zero
status. Nothing here computes any part of the layer.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16, MOE_MXFP8_E4M3, MOE_MXFP4_E2M1, MOE_NVFP4_E2M1 = 0, 1, 2, 3, 4
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_ALIGNMENT", -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_HIP"}

# exported entry points and their ctypes signatures
_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "moe_abi_version": (_I, []),
    "moe_status_str": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_route": (_I, [_P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_workspace": (_SZ, [_I, _I, _I]),
    "moe_quantize_mx": (_I, [_P, _I, _I64, _I, _I, _I, _P, _P, _P]),
    "moe_permute_rows_bound": (_I64, [_I, _I, _I, _I]),
    "moe_permute_workspace": (_SZ, [_I, _I, _I]),
    "moe_permute": (_I, [_P, _I, _I, _I, _I, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_noalloc": (_I, [_P, _I, _I, _I, _I, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "moe_permute_noalloc_max_bytes": (_SZ, []),
    "moe_grouped_mlp_workspace": (_SZ, [_I, _I, _I, _I64, _I, _I]),
    "moe_grouped_mlp_fwd": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I64, _P, _P,
                                 _I, _P, _SZ, _P]),
    "moe_grouped_fc1_swiglu": (_I, [_P, _P, _I, _P, _P, _P, _I, _P, _I, _I, _I, _I64, _P, _P, _P, _P]),
    "moe_grouped_fc2": (_I, [_P, _P, _I, _P, _P, _I, _P, _I, _I, _I, _I64, _P, _I, _P]),
    "moe_grouped_fc1_swiglu_dense": (_I, [_P, _P, _I, _P, _P, _P, _I, _P, _I, _I, _I, _I64, _P, _P,
                                          _P, _P, _P, _I, _P]),
    "moe_grouped_fc2_dense": (_I, [_P, _P, _I, _P, _P, _I, _P, _I, _I, _I, _I64, _P, _I, _P, _P, _I,
                                   _P]),
    "moe_combine": (_I, [_P, _I, _P, _P, _P, _I, _I, _I, _P, _I, _P]),
    "moe_pack_weights": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_combine_bwd": (_I, [_P, _I, _P, _P, _P, _I, _I, _I, _I64, _P, _I, _P, _P, _P]),
    "moe_unpermute": (_I, [_P, _I, _P, _I, _I, _I, _P, _I, _P]),
    "moe_segments_kstride": (_I64, [_I64, _I]),
    "moe_quantize_mx_segments": (_I, [_P, _I, _I, _P, _P, _P, _I, _I64, _I, _I64, _I, _P, _P, _P, _P]),
    "moe_grouped_fc2_dgrad_dswiglu": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I64, _P, _P, _P, _P, _P]),
    "moe_grouped_fc1_dgrad": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I64, _P, _P]),
    "moe_grouped_wgrad": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I64, _P, _P]),
    "moe_route_bwd_workspace": (_SZ, [_I, _I, _I, _I]),
    "moe_route_bwd": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _F, _P, _P, _P,
                           _P, _P, _SZ, _P]),
    "moe_bias_update": (_I, [_P, _I, _F, _P, _P, _P]),
    "moe_nvfp4_tensor_scale": (_I, [_P, _I, _I, _I64, _P, _P]),
    "moe_quantize_nvfp4": (_I, [_P, _I, _I64, _I, _I64, _P, _P, _P, _P, _P]),
    "moe_grouped_fc1_swiglu_nvfp4": (_I, [_P, _P, _P, _P, _P, _F, _F, _P, _I, _I, _I, _I64, _P, _P]),
    "moe_grouped_fc2_nvfp4": (_I, [_P, _P, _P, _P, _F, _P, _I, _I, _I, _I64, _P, _P]),
    "moe_grouped_mlp_bwd_workspace": (_SZ, [_I, _I, _I, _I, _I, _I64, _I]),
    "moe_grouped_mlp_bwd": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                 _I, _I64, _P, _P, _P, _P, _SZ, _P]),
}

_lib = None


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m mixture_experts_layer_sigmoid_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(name: str, status: int):
    if status != 0:
        raise MoEError(name, status, load().moe_last_error().decode())


def fmt_of_dtype(t) -> int:
    import torch
    return {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}[t.dtype]


# -- thin wrappers, same names and argument order as the C ABI -------------
def moe_abi_version() -> int:
    return load().moe_abi_version()


def moe_route(x, x_fmt, w_router, bias, logits_in, T, H, E, n_group, topk_group, k,
              routed_scale, logits_out, topk_idx, topk_w, ws, stream=None):
    _check("moe_route", load().moe_route(
        _ptr(x), x_fmt, _ptr(w_router), _ptr(bias), _ptr(logits_in), T, H, E, n_group,
        topk_group, k, float(routed_scale), _ptr(logits_out), _ptr(topk_idx), _ptr(topk_w),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_route_workspace(T, H, E) -> int:
    return load().moe_route_workspace(T, H, E)


def moe_quantize_mx(inp, in_fmt, rows, K, axis, out_fmt, codes, scales, stream=None):
    _check("moe_quantize_mx", load().moe_quantize_mx(
        _ptr(inp), in_fmt, rows, K, axis, out_fmt, _ptr(codes), _ptr(scales), _stream(stream)))


def moe_permute_rows_bound(T, k, E, align) -> int:
    return load().moe_permute_rows_bound(T, k, E, align)


def moe_permute_workspace(T, k, E) -> int:
    return load().moe_permute_workspace(T, k, E)


def moe_permute(topk_idx, T, k, E, align, rows_in, row_bytes, scales_in, scale_bytes, counts,
                offsets, row_map, src_row, rows_out, scales_out, ws, stream=None):
    _check("moe_permute", load().moe_permute(
        _ptr(topk_idx), T, k, E, align, _ptr(rows_in), row_bytes, _ptr(scales_in), scale_bytes,
        _ptr(counts), _ptr(offsets), _ptr(row_map), _ptr(src_row), _ptr(rows_out),
        _ptr(scales_out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def moe_permute_noalloc(topk_idx, T, k, E, align, rows_in, row_bytes, scales_in, scale_bytes,
                        counts, offsets, row_map, src_row, rows_out, scales_out, stream=None):
    _check("moe_permute_noalloc", load().moe_permute_noalloc(
        _ptr(topk_idx), T, k, E, align, _ptr(rows_in), row_bytes, _ptr(scales_in), scale_bytes,
        _ptr(counts), _ptr(offsets), _ptr(row_map), _ptr(src_row), _ptr(rows_out),
        _ptr(scales_out), _stream(stream)))


def moe_permute_noalloc_max_bytes() -> int:
    return load().moe_permute_noalloc_max_bytes()


def moe_grouped_mlp_workspace(E, H, F, rows, a_fmt, w_fmt) -> int:
    return load().moe_grouped_mlp_workspace(E, H, F, rows, a_fmt, w_fmt)


def moe_grouped_mlp_fwd(a, a_scales, a_fmt, src_row, w1, w1_scales, w2, w2_scales, w_fmt,
                        offsets, E, H, F, rows, act_save, y, y_fmt, ws, stream=None):
    _check("moe_grouped_mlp_fwd", load().moe_grouped_mlp_fwd(
        _ptr(a), _ptr(a_scales), a_fmt, _ptr(src_row), _ptr(w1), _ptr(w1_scales), _ptr(w2),
        _ptr(w2_scales), w_fmt, _ptr(offsets), E, H, F, rows, _ptr(act_save), _ptr(y), y_fmt,
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_fc1_swiglu(a, a_scales, a_fmt, src_row, w1, w1_scales, w_fmt, offsets, E, H, F,
                           rows, act_save, h, h_scales, stream=None):
    _check("moe_grouped_fc1_swiglu", load().moe_grouped_fc1_swiglu(
        _ptr(a), _ptr(a_scales), a_fmt, _ptr(src_row), _ptr(w1), _ptr(w1_scales), w_fmt,
        _ptr(offsets), E, H, F, rows, _ptr(act_save), _ptr(h), _ptr(h_scales), _stream(stream)))


def moe_grouped_fc2(h, h_scales, h_fmt, w2, w2_scales, w_fmt, offsets, E, H, F, rows, y, y_fmt,
                    stream=None):
    _check("moe_grouped_fc2", load().moe_grouped_fc2(
        _ptr(h), _ptr(h_scales), h_fmt, _ptr(w2), _ptr(w2_scales), w_fmt, _ptr(offsets), E, H, F,
        rows, _ptr(y), y_fmt, _stream(stream)))


def moe_grouped_fc1_swiglu_dense(a, a_scales, a_fmt, src_row, w1, w1_scales, w_fmt, offsets, E, H,
                                 F, rows, act_save, h, h_scales, w1d, w1d_scales, T, stream=None):
    _check("moe_grouped_fc1_swiglu_dense", load().moe_grouped_fc1_swiglu_dense(
        _ptr(a), _ptr(a_scales), a_fmt, _ptr(src_row), _ptr(w1), _ptr(w1_scales), w_fmt,
        _ptr(offsets), E, H, F, rows, _ptr(act_save), _ptr(h), _ptr(h_scales), _ptr(w1d),
        _ptr(w1d_scales), T, _stream(stream)))


def moe_grouped_fc2_dense(h, h_scales, h_fmt, w2, w2_scales, w_fmt, offsets, E, H, F, rows, y,
                          y_fmt, w2d, w2d_scales, T, stream=None):
    _check("moe_grouped_fc2_dense", load().moe_grouped_fc2_dense(
        _ptr(h), _ptr(h_scales), h_fmt, _ptr(w2), _ptr(w2_scales), w_fmt, _ptr(offsets), E, H, F,
        rows, _ptr(y), y_fmt, _ptr(w2d), _ptr(w2d_scales), T, _stream(stream)))


def moe_combine(y, y_fmt, row_map, topk_w, shared, T, k, H, out, out_fmt, stream=None):
    _check("moe_combine", load().moe_combine(
        _ptr(y), y_fmt, _ptr(row_map), _ptr(topk_w), _ptr(shared), T, k, H, _ptr(out), out_fmt,
        _stream(stream)))


def moe_combine_bwd(dout, dout_fmt, row_map, src_row, topk_w, T, k, H, rows, dy, dy_fmt, dy_scales,
                    row_w, stream=None):
    _check("moe_combine_bwd", load().moe_combine_bwd(
        _ptr(dout), dout_fmt, _ptr(row_map), _ptr(src_row), _ptr(topk_w), T, k, H, rows, _ptr(dy),
        dy_fmt, _ptr(dy_scales), _ptr(row_w), _stream(stream)))


def moe_unpermute(dx_perm, fmt, row_map, T, k, H, dx, out_fmt, stream=None):
    _check("moe_unpermute", load().moe_unpermute(
        _ptr(dx_perm), fmt, _ptr(row_map), T, k, H, _ptr(dx), out_fmt, _stream(stream)))


def moe_segments_kstride(rows, E) -> int:
    return load().moe_segments_kstride(rows, E)


def moe_quantize_mx_segments(inp, in_fmt, mode, src_row, offsets, row_scale, E, rows, C, kstride,
                             out_fmt, codes, scales, kofs, stream=None):
    _check("moe_quantize_mx_segments", load().moe_quantize_mx_segments(
        _ptr(inp), in_fmt, mode, _ptr(src_row), _ptr(offsets), _ptr(row_scale), E, rows, C, kstride,
        out_fmt, _ptr(codes), _ptr(scales), _ptr(kofs), _stream(stream)))


def moe_grouped_fc2_dgrad_dswiglu(dy, dy_scales, fmt, w2t, w2t_scales, offsets, E, H, F, rows,
                                  act_save, da, da_scales, da_f32, stream=None):
    _check("moe_grouped_fc2_dgrad_dswiglu", load().moe_grouped_fc2_dgrad_dswiglu(
        _ptr(dy), _ptr(dy_scales), fmt, _ptr(w2t), _ptr(w2t_scales), _ptr(offsets), E, H, F, rows,
        _ptr(act_save), _ptr(da), _ptr(da_scales), _ptr(da_f32), _stream(stream)))


def moe_grouped_fc1_dgrad(da, da_scales, fmt, w1t, w1t_scales, offsets, E, H, F, rows, dx_perm,
                          stream=None):
    _check("moe_grouped_fc1_dgrad", load().moe_grouped_fc1_dgrad(
        _ptr(da), _ptr(da_scales), fmt, _ptr(w1t), _ptr(w1t_scales), _ptr(offsets), E, H, F, rows,
        _ptr(dx_perm), _stream(stream)))


def moe_grouped_wgrad(at, at_scales, bt, bt_scales, fmt, kofs, E, M, N, kstride, dw, stream=None):
    _check("moe_grouped_wgrad", load().moe_grouped_wgrad(
        _ptr(at), _ptr(at_scales), _ptr(bt), _ptr(bt_scales), fmt, _ptr(kofs), E, M, N, kstride,
        _ptr(dw), _stream(stream)))


def moe_pack_weights(w, w_scales, fmt, E, N, K, half, out, out_scales, stream=None):
    _check("moe_pack_weights", load().moe_pack_weights(
        _ptr(w), _ptr(w_scales), fmt, E, N, K, half, _ptr(out), _ptr(out_scales), _stream(stream)))


def moe_grouped_mlp_bwd_workspace(T, k, E, H, F, rows, fmt) -> int:
    return load().moe_grouped_mlp_bwd_workspace(T, k, E, H, F, rows, fmt)


def moe_grouped_mlp_bwd(dout, x, act_fmt, row_map, src_row, topk_w, offsets, act_save, w1t,
                        w1t_scales, w2t, w2t_scales, fmt, T, k, E, H, F, rows, dx, dw1, dw2, ws,
                        stream=None):
    _check("moe_grouped_mlp_bwd", load().moe_grouped_mlp_bwd(
        _ptr(dout), _ptr(x), act_fmt, _ptr(row_map), _ptr(src_row), _ptr(topk_w), _ptr(offsets),
        _ptr(act_save), _ptr(w1t), _ptr(w1t_scales), _ptr(w2t), _ptr(w2t_scales), fmt, T, k, E, H,
        F, rows, _ptr(dx), _ptr(dw1), _ptr(dw2), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_route_bwd_workspace(T, H, E, seq_len) -> int:
    return load().moe_route_bwd_workspace(T, H, E, seq_len)


def moe_route_bwd(dout, y, act_fmt, row_map, topk_idx, logits, x, w_router, T, k, E, H,
                  routed_scale, seq_len, aux_alpha, dlogits, aux_loss, dx_router, dw_router, ws,
                  stream=None):
    _check("moe_route_bwd", load().moe_route_bwd(
        _ptr(dout), _ptr(y), act_fmt, _ptr(row_map), _ptr(topk_idx), _ptr(logits), _ptr(x),
        _ptr(w_router), T, k, E, H, routed_scale, seq_len, aux_alpha, _ptr(dlogits),
        _ptr(aux_loss), _ptr(dx_router), _ptr(dw_router), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_bias_update(counts, E, gamma, bias, bias_out, stream=None):
    _check("moe_bias_update", load().moe_bias_update(
        _ptr(counts), E, gamma, _ptr(bias), _ptr(bias_out), _stream(stream)))


def moe_nvfp4_tensor_scale(inp, in_fmt, n_tensors, elems_per_tensor, g, stream=None):
    _check("moe_nvfp4_tensor_scale", load().moe_nvfp4_tensor_scale(
        _ptr(inp), in_fmt, n_tensors, elems_per_tensor, _ptr(g), _stream(stream)))


def moe_quantize_nvfp4(inp, in_fmt, rows, K, rows_per_tensor, g, codes, scales, vals, stream=None):
    _check("moe_quantize_nvfp4", load().moe_quantize_nvfp4(
        _ptr(inp), in_fmt, rows, K, rows_per_tensor, _ptr(g), _ptr(codes), _ptr(scales),
        _ptr(vals), _stream(stream)))


def moe_grouped_fc1_swiglu_nvfp4(a_vals, src_row, w1, w1_scales, w1_g, x_g, h_g, offsets, E, H, F,
                                 rows, h_vals, stream=None):
    _check("moe_grouped_fc1_swiglu_nvfp4", load().moe_grouped_fc1_swiglu_nvfp4(
        _ptr(a_vals), _ptr(src_row), _ptr(w1), _ptr(w1_scales), _ptr(w1_g), x_g, h_g,
        _ptr(offsets), E, H, F, rows, _ptr(h_vals), _stream(stream)))


def moe_grouped_fc2_nvfp4(h_vals, w2, w2_scales, w2_g, h_g, offsets, E, H, F, rows, y, stream=None):
    _check("moe_grouped_fc2_nvfp4", load().moe_grouped_fc2_nvfp4(
        _ptr(h_vals), _ptr(w2), _ptr(w2_scales), _ptr(w2_g), h_g, _ptr(offsets), E, H, F, rows,
        _ptr(y), _stream(stream)))
