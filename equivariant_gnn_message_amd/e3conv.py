"""ctypes binding of libe3conv.so (argument marshalling only).

The functions named ``e3conv_*`` mirror the C ABI in include/e3conv.h one to
one, taking torch tensors where the C function takes device pointers (the
tensor's device pointer, and the current HIP stream of torch unless a stream
is given).  All arithmetic runs in the library's HIP kernels; there is no
fallback: if the library is missing every call raises.

``Plan`` and ``E3ConvFunction`` are conveniences over the same calls.
"""

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libe3conv.so")

E3CONV_OK = 0
E3CONV_ERR_INVALID_ARGUMENT, E3CONV_ERR_PARSE, E3CONV_ERR_UNSUPPORTED = 1, 2, 3
E3CONV_ERR_NO_PATH, E3CONV_ERR_GRAPH = 4, 5
E3CONV_F32 = 0
E3CONV_BF16 = 1
E3CONV_RECEIVER = 0
E3CONV_SENDER = 1
E3CONV_ACCUMULATE_GRAD_X = 1
E3CONV_ACCUMULATE_GRAD_Y = 2
E3CONV_ACCUMULATE_GRAD_S = 4

STATUS_NAMES = {
    0: "E3CONV_OK", 1: "E3CONV_ERR_INVALID_ARGUMENT", 2: "E3CONV_ERR_PARSE",
    3: "E3CONV_ERR_UNSUPPORTED", 4: "E3CONV_ERR_NO_PATH", 5: "E3CONV_ERR_GRAPH",
    6: "E3CONV_ERR_WORKSPACE", 7: "E3CONV_ERR_HIP", 8: "E3CONV_ERR_INTERNAL",
}

# every symbol include/e3conv.h declares
EXPORTED = [
    "e3conv_plan", "e3conv_plan_ordered", "e3conv_plan_ordering", "e3conv_plan_destroy",
    "e3conv_plan_shape", "e3conv_plan_paths",
    "e3conv_plan_coefficients", "e3conv_plan_supported", "e3conv_forward", "e3conv_forward_masked",
    "e3conv_forward_radial", "e3conv_jvp", "e3conv_backward_workspace_size", "e3conv_backward", "e3conv_backward_ex",
    "e3conv_linear", "e3conv_linear_backward", "e3conv_csr_from_receivers",
    "e3conv_validate_graph", "e3conv_validate_graph_async", "e3conv_validate_graph_noalloc",
    "e3conv_receiver_order",
    "e3conv_relabel_nodes",
    "e3conv_stream_reference", "e3conv_second_derivatives", "e3conv_backward_pairs", "e3conv_pair_layout", "e3conv_forward_linear", "e3conv_forward_pairs",
    "e3conv_plan_set_variant",
    "e3conv_plan_num_variants",
    "e3conv_status_string", "e3conv_last_error_detail",
]


class E3ConvError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None

P = ctypes.c_void_p
I32P = ctypes.POINTER(ctypes.c_int)
I64 = ctypes.c_int64


def load_library(path=LIB_PATH):
    """Load libe3conv.so (once) and declare its signatures; raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: its HIP runtime is then the one the library's dependency
    # resolves to, so device pointers and streams from torch are valid for the
    # library (loading the library first binds it to a second runtime copy,
    # which then sees no device).
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m equivariant_gnn_message_amd.build` first")
    lib = ctypes.CDLL(path)
    sig = {
        "e3conv_plan": ([ctypes.c_char_p, ctypes.c_int, ctypes.c_char_p, ctypes.c_float,
                         ctypes.POINTER(P)], ctypes.c_int),
        "e3conv_plan_ordered": ([ctypes.c_char_p, ctypes.c_int, ctypes.c_char_p, ctypes.c_float,
                                 ctypes.c_int, ctypes.POINTER(P)], ctypes.c_int),
        "e3conv_plan_ordering": ([P, I32P], ctypes.c_int),
        "e3conv_plan_destroy": ([P], None),
        "e3conv_plan_shape": ([P, I32P, I32P, I32P, I32P, I32P], ctypes.c_int),
        "e3conv_plan_paths": ([P] + [I32P] * 8, ctypes.c_int),
        "e3conv_plan_coefficients": ([P, I32P, I32P, I32P, I32P, I32P,
                                      ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "e3conv_plan_supported": ([P, I32P, I32P, I32P], ctypes.c_int),
        "e3conv_forward": ([P, ctypes.c_int, P, P, P, P, P, P, I64, I64, P, P], ctypes.c_int),
        "e3conv_forward_masked": ([P, ctypes.c_int, P, P, P, P, P, P, I64, I64, I64, P, P],
                                  ctypes.c_int),
        "e3conv_forward_radial": ([P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                   ctypes.c_float, P, P, P, I64, I64, I64, P, P], ctypes.c_int),
        "e3conv_jvp": ([P, ctypes.c_int, P, P, P, P, P, P, P, P, P, I64, I64, I64, P, P, P],
                       ctypes.c_int),
        "e3conv_backward_workspace_size": ([P, I64, I64, ctypes.POINTER(ctypes.c_size_t)],
                                           ctypes.c_int),
        "e3conv_backward": ([P, ctypes.c_int, P, P, P, P, P, P, I64, I64, P, P, P, P, P,
                             ctypes.c_size_t, P], ctypes.c_int),
        "e3conv_backward_ex": ([P, ctypes.c_int, P, P, P, P, P, P, I64, I64, I64, P, P, P, P,
                                ctypes.c_uint, P, ctypes.c_size_t, P], ctypes.c_int),
        "e3conv_receiver_order": ([P, P, I64, I64, ctypes.c_int, P], ctypes.c_int),
        "e3conv_relabel_nodes": ([P, P, I64, I64, ctypes.c_int, P, P], ctypes.c_int),
        "e3conv_linear": ([P, ctypes.c_int, ctypes.c_float, P, P, I64, P, P], ctypes.c_int),
        "e3conv_linear_backward": ([P, ctypes.c_int, ctypes.c_float, P, P, I64, P, P, P, P],
                                   ctypes.c_int),
        "e3conv_stream_reference": ([P, P, ctypes.c_size_t, P], ctypes.c_int),
        "e3conv_csr_from_receivers": ([P, I64, I64, P, P], ctypes.c_int),
        "e3conv_validate_graph": ([P, P, I64, I64, ctypes.c_int], ctypes.c_int),
        "e3conv_validate_graph_async": ([P, P, I64, I64, P, P], ctypes.c_int),
        "e3conv_validate_graph_noalloc": ([P, P, I64, I64, P], ctypes.c_int),
        "e3conv_backward_pairs": ([P, P, P, P, P, P, I64, I64, P, P, P, P, P], ctypes.c_int),
        "e3conv_pair_layout": ([P, P, I64, I64, ctypes.c_int, P, P], ctypes.c_int),
        "e3conv_forward_pairs": ([P, P, P, P, P, P, P, P, I64, I64, I64, P, P], ctypes.c_int),
        "e3conv_forward_linear": ([P, ctypes.c_int, P, P, P, P, P, P, I64, I64, ctypes.c_float, P, P, P],
                                  ctypes.c_int),
        "e3conv_second_derivatives": ([P, ctypes.c_int, P, P, P, P, P, P, I64, I64, I64, P, P, P, P,
                                       P, P, P, P, P], ctypes.c_int),
        "e3conv_plan_set_variant": ([P, ctypes.c_int, ctypes.c_int], ctypes.c_int),
        "e3conv_plan_num_variants": ([P, ctypes.c_int, I32P, I32P], ctypes.c_int),
        "e3conv_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "e3conv_last_error_detail": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status):
    if status != E3CONV_OK:
        detail = load_library().e3conv_last_error_detail().decode()
        raise E3ConvError(status, detail)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    """hipStream_t: a raw handle (int), a torch stream object, or None for torch's current
    stream."""
    if stream is not None:
        return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return E3CONV_F32
    if t.dtype == torch.bfloat16:
        return E3CONV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, device=True):
    if t is None:
        raise ValueError(f"{name} is required")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


# ----------------------------------------------------- C-ABI mirrors ---

def e3conv_plan(irreps_in, sh_lmax, irreps_out, avg_num_neighbors=1.0):
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.e3conv_plan(irreps_in.encode(), int(sh_lmax), irreps_out.encode(),
                           float(avg_num_neighbors), ctypes.byref(h)))
    return h


def e3conv_plan_ordered(irreps_in, sh_lmax, irreps_out, avg_num_neighbors=1.0,
                        ordering=E3CONV_RECEIVER):
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.e3conv_plan_ordered(irreps_in.encode(), int(sh_lmax), irreps_out.encode(),
                                   float(avg_num_neighbors), int(ordering), ctypes.byref(h)))
    return h


def e3conv_plan_ordering(handle):
    v = ctypes.c_int()
    _check(load_library().e3conv_plan_ordering(handle, ctypes.byref(v)))
    return v.value


def e3conv_plan_destroy(handle):
    if handle:
        load_library().e3conv_plan_destroy(handle)


def e3conv_plan_shape(handle):
    vals = [ctypes.c_int() for _ in range(5)]
    _check(load_library().e3conv_plan_shape(handle, *[ctypes.byref(v) for v in vals]))
    return tuple(v.value for v in vals)   # channels, num_x, num_y, num_paths, num_out


def e3conv_plan_paths(handle):
    n = e3conv_plan_shape(handle)[3]
    arrs = [(ctypes.c_int * max(n, 1))() for _ in range(8)]
    _check(load_library().e3conv_plan_paths(handle, *arrs))
    keys = ("l1", "p1", "l2", "l3", "p3", "o1", "o2", "o3")
    return [dict(zip(keys, (a[i] for a in arrs))) for i in range(n)]


def e3conv_plan_coefficients(handle):
    lib = load_library()
    nnz = ctypes.c_int()
    _check(lib.e3conv_plan_coefficients(handle, ctypes.byref(nnz), None, None, None, None, None))
    n = nnz.value
    ix, iy, ip, io = [(ctypes.c_int * max(n, 1))() for _ in range(4)]
    val = (ctypes.c_double * max(n, 1))()
    _check(lib.e3conv_plan_coefficients(handle, ctypes.byref(nnz), ix, iy, ip, io, val))
    return [list(a)[:n] for a in (ix, iy, ip, io)] + [list(val)[:n]]


def e3conv_plan_supported(handle):
    v = [ctypes.c_int() for _ in range(3)]
    _check(load_library().e3conv_plan_supported(handle, *[ctypes.byref(a) for a in v]))
    return tuple(bool(a.value) for a in v)


def e3conv_plan_num_variants(handle, dtype=E3CONV_F32):
    f, b = ctypes.c_int(), ctypes.c_int()
    _check(load_library().e3conv_plan_num_variants(handle, int(dtype), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def e3conv_plan_set_variant(handle, forward_variant=0, backward_variant=0):
    _check(load_library().e3conv_plan_set_variant(handle, int(forward_variant), int(backward_variant)))


def _check_graph_args(src, row_ptr, order):
    import torch
    _need(src, "src", torch.int32)
    _need(row_ptr, "row_ptr", torch.int32)
    if order is not None:
        _need(order, "order", torch.int32)


def e3conv_forward(handle, x, y, s, src, row_ptr, num_nodes, num_edges, out, order=None, stream=None):
    import torch
    dt = _dtype_code(x)
    for t, n in ((x, "x"), (y, "y"), (s, "s")):
        _need(t, n, x.dtype)
    _check_graph_args(src, row_ptr, order)
    _need(out, "out", torch.float32)
    _check(load_library().e3conv_forward(handle, dt, _ptr(x), _ptr(y), _ptr(s), _ptr(src),
                                         _ptr(row_ptr), _ptr(order), int(num_nodes), int(num_edges),
                                         _ptr(out), _stream(stream)))
    return out


def e3conv_forward_masked(handle, x, y, s, src, row_ptr, num_nodes, num_edges, num_real_nodes, out,
                          order=None, stream=None):
    import torch
    dt = _dtype_code(x)
    for t, n in ((x, "x"), (y, "y"), (s, "s")):
        _need(t, n, x.dtype)
    _check_graph_args(src, row_ptr, order)
    _need(out, "out", torch.float32)
    _check(load_library().e3conv_forward_masked(handle, dt, _ptr(x), _ptr(y), _ptr(s), _ptr(src),
                                                _ptr(row_ptr), _ptr(order), int(num_nodes),
                                                int(num_edges), int(num_real_nodes), _ptr(out),
                                                _stream(stream)))
    return out


def e3conv_forward_radial(handle, x, y, r, w1, w2, r_max, sigma, src, row_ptr, num_nodes, num_edges,
                          num_real_nodes, out, order=None, stream=None):
    import torch
    for t, n in ((x, "x"), (y, "y"), (r, "r"), (w1, "w1"), (w2, "w2"), (out, "out")):
        _need(t, n, torch.float32)
    _check_graph_args(src, row_ptr, order)
    if w1.dim() != 2 or w2.dim() != 2 or w1.shape[1] != w2.shape[0]:
        raise ValueError(f"w1 (num_basis, hidden) and w2 (hidden, P*C) do not chain: "
                         f"{tuple(w1.shape)}, {tuple(w2.shape)}")
    _check(load_library().e3conv_forward_radial(handle, _ptr(x), _ptr(y), _ptr(r), _ptr(w1), _ptr(w2),
                                                int(w1.shape[0]), int(w1.shape[1]), float(r_max),
                                                float(sigma), _ptr(src), _ptr(row_ptr), _ptr(order),
                                                int(num_nodes), int(num_edges), int(num_real_nodes),
                                                _ptr(out), _stream(stream)))
    return out


def e3conv_jvp(handle, x, y, s, dx, dy, ds, src, row_ptr, num_nodes, num_edges, out, out_dot,
               order=None, stream=None, num_real_nodes=None):
    import torch
    dt = _dtype_code(x)
    for t, n in ((x, "x"), (y, "y"), (s, "s"), (dx, "dx"), (dy, "dy"), (ds, "ds")):
        _need(t, n, x.dtype)
    _check_graph_args(src, row_ptr, order)
    _need(out_dot, "out_dot", torch.float32)
    if out is not None:
        _need(out, "out", torch.float32)
    _check(load_library().e3conv_jvp(handle, dt, _ptr(x), _ptr(y), _ptr(s), _ptr(dx), _ptr(dy),
                                     _ptr(ds), _ptr(src), _ptr(row_ptr), _ptr(order), int(num_nodes),
                                     int(num_edges),
                                     int(num_nodes if num_real_nodes is None else num_real_nodes),
                                     _ptr(out), _ptr(out_dot), _stream(stream)))
    return out, out_dot


def e3conv_backward_workspace_size(handle, num_nodes, num_edges):
    n = ctypes.c_size_t()
    _check(load_library().e3conv_backward_workspace_size(handle, int(num_nodes), int(num_edges),
                                                         ctypes.byref(n)))
    return n.value


def e3conv_backward(handle, x, y, s, src, row_ptr, num_nodes, num_edges, grad_out, grad_x,
                    grad_y, grad_s, workspace=None, order=None, stream=None):
    import torch
    for t, n in ((x, "x"), (y, "y"), (s, "s"), (grad_out, "grad_out"), (grad_x, "grad_x"),
                 (grad_y, "grad_y"), (grad_s, "grad_s")):
        _need(t, n, torch.float32)
    _check_graph_args(src, row_ptr, order)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().e3conv_backward(handle, E3CONV_F32, _ptr(x), _ptr(y), _ptr(s), _ptr(src),
                                          _ptr(row_ptr), _ptr(order), int(num_nodes), int(num_edges),
                                          _ptr(grad_out), _ptr(grad_x), _ptr(grad_y), _ptr(grad_s),
                                          _ptr(workspace), wbytes, _stream(stream)))


def e3conv_backward_ex(handle, x, y, s, src, row_ptr, num_nodes, num_edges, num_real_nodes,
                       grad_out, grad_x, grad_y, grad_s, flags=0, workspace=None, order=None,
                       stream=None):
    """General reverse pass: grad_x / grad_y / grad_s may be None (not computed)."""
    import torch
    for t, n in ((x, "x"), (y, "y"), (s, "s"), (grad_out, "grad_out")):
        _need(t, n, torch.float32)
    for t, n in ((grad_x, "grad_x"), (grad_y, "grad_y"), (grad_s, "grad_s")):
        if t is not None:
            _need(t, n, torch.float32)
    _check_graph_args(src, row_ptr, order)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().e3conv_backward_ex(
        handle, E3CONV_F32, _ptr(x), _ptr(y), _ptr(s), _ptr(src), _ptr(row_ptr), _ptr(order),
        int(num_nodes), int(num_edges), int(num_real_nodes), _ptr(grad_out), _ptr(grad_x),
        _ptr(grad_y), _ptr(grad_s), int(flags), _ptr(workspace), wbytes, _stream(stream)))


def e3conv_forward_pairs(handle, x, y, s, src, row_ptr, pair_of, num_nodes, num_edges, num_pairs, out,
                         order=None, stream=None):
    """Forward over the directed receiver CSR with y and s read from pair-stored rows."""
    import torch
    for t, n in ((x, "x"), (y, "y"), (s, "s"), (out, "out")):
        _need(t, n, torch.float32)
    _need(pair_of, "pair_of", torch.int32)
    _check_graph_args(src, row_ptr, order)
    _check(load_library().e3conv_forward_pairs(handle, _ptr(x), _ptr(y), _ptr(s), _ptr(src),
                                               _ptr(row_ptr), _ptr(pair_of), _ptr(order), int(num_nodes),
                                               int(num_edges), int(num_pairs), _ptr(out),
                                               _stream(stream)))
    return out


def e3conv_backward_pairs(handle, x, y, s, src, dst, num_nodes, num_pairs, grad_out, grad_x,
                          grad_y, grad_s, stream=None):
    """Pair-stored reverse pass: each stored edge (src -> dst) stands for itself and its reverse."""
    import torch
    for t, n in ((x, "x"), (y, "y"), (s, "s"), (grad_out, "grad_out"), (grad_x, "grad_x"),
                 (grad_y, "grad_y"), (grad_s, "grad_s")):
        _need(t, n, torch.float32)
    _need(src, "src", torch.int32)
    _need(dst, "dst", torch.int32)
    _check(load_library().e3conv_backward_pairs(handle, _ptr(x), _ptr(y), _ptr(s), _ptr(src),
                                                _ptr(dst), int(num_nodes), int(num_pairs),
                                                _ptr(grad_out), _ptr(grad_x), _ptr(grad_y),
                                                _ptr(grad_s), _stream(stream)))


def e3conv_forward_linear(handle, x, y, s, src, row_ptr, num_nodes, num_edges, scale, weights, out,
                          order=None, stream=None):
    """The convolution with the output linear (C_out = C) fused into its epilogue."""
    import torch
    dt = _dtype_code(x)
    for t, n in ((x, "x"), (y, "y"), (s, "s")):
        _need(t, n, x.dtype)
    _need(weights, "weights", torch.float32)
    _need(out, "out", torch.float32)
    _check_graph_args(src, row_ptr, order)
    _check(load_library().e3conv_forward_linear(handle, dt, _ptr(x), _ptr(y), _ptr(s), _ptr(src),
                                                _ptr(row_ptr), _ptr(order), int(num_nodes),
                                                int(num_edges), float(scale), _ptr(weights), _ptr(out),
                                                _stream(stream)))
    return out


def e3conv_linear(handle, channels_out, scale, weights, inp, num_nodes, out, stream=None):
    import torch
    for t, n in ((weights, "weights"), (inp, "in"), (out, "out")):
        _need(t, n, torch.float32)
    _check(load_library().e3conv_linear(handle, int(channels_out), float(scale), _ptr(weights),
                                        _ptr(inp), int(num_nodes), _ptr(out), _stream(stream)))
    return out


def e3conv_linear_backward(handle, channels_out, scale, weights, inp, num_nodes, grad_out,
                           grad_in=None, grad_weights=None, stream=None):
    import torch
    for t, n in ((weights, "weights"), (inp, "in"), (grad_out, "grad_out")):
        _need(t, n, torch.float32)
    for t, n in ((grad_in, "grad_in"), (grad_weights, "grad_weights")):
        if t is not None:
            _need(t, n, torch.float32)
    _check(load_library().e3conv_linear_backward(handle, int(channels_out), float(scale),
                                                 _ptr(weights), _ptr(inp), int(num_nodes),
                                                 _ptr(grad_out), _ptr(grad_in), _ptr(grad_weights),
                                                 _stream(stream)))
    return grad_in, grad_weights


def e3conv_csr_from_receivers(receivers, num_nodes, row_ptr=None, stream=None):
    import torch
    _need(receivers, "receivers", torch.int32)
    if row_ptr is None:
        row_ptr = torch.empty(int(num_nodes) + 1, dtype=torch.int32, device=receivers.device)
    _need(row_ptr, "row_ptr", torch.int32)
    _check(load_library().e3conv_csr_from_receivers(_ptr(receivers), receivers.numel(),
                                                    int(num_nodes), _ptr(row_ptr), _stream(stream)))
    return row_ptr


def e3conv_receiver_order(row_ptr, src, num_nodes, num_edges, cluster=512):
    """Host-side receiver order (numpy int32 permutation) for gather locality."""
    import numpy as np
    r = np.ascontiguousarray(np.asarray(row_ptr), dtype=np.int32)
    s = np.ascontiguousarray(np.asarray(src), dtype=np.int32)
    order = np.empty(int(num_nodes), dtype=np.int32)
    _check(load_library().e3conv_receiver_order(r.ctypes.data_as(P), s.ctypes.data_as(P),
                                                int(num_nodes), int(num_edges), int(cluster),
                                                order.ctypes.data_as(P)))
    return order


def e3conv_relabel_nodes(row_ptr, src, num_nodes, num_edges, cluster=512):
    """Host-side node relabeling in receiver-cluster order: (node_new, edge_perm) as numpy
    int32 (new id of each old node; old index of each edge of the relabeled graph)."""
    import numpy as np
    r = np.ascontiguousarray(np.asarray(row_ptr), dtype=np.int32)
    s = np.ascontiguousarray(np.asarray(src), dtype=np.int32)
    node_new = np.empty(int(num_nodes), dtype=np.int32)
    edge_perm = np.empty(int(num_edges), dtype=np.int32)
    _check(load_library().e3conv_relabel_nodes(r.ctypes.data_as(P), s.ctypes.data_as(P),
                                               int(num_nodes), int(num_edges), int(cluster),
                                               node_new.ctypes.data_as(P), edge_perm.ctypes.data_as(P)))
    return node_new, edge_perm


def e3conv_pair_layout(row_ptr, src, num_nodes, num_edges, cluster=512):
    """Host-side pair storage of a symmetric graph: (stored, pair_of) as numpy int32; pair_of[e]
    is the pair of directed edge e, or ~pair when e is the reverse of the stored edge."""
    import numpy as np
    r = np.ascontiguousarray(np.asarray(row_ptr), dtype=np.int32)
    s = np.ascontiguousarray(np.asarray(src), dtype=np.int32)
    stored = np.empty(int(num_edges) // 2, dtype=np.int32)
    pair_of = np.empty(int(num_edges), dtype=np.int32)
    _check(load_library().e3conv_pair_layout(r.ctypes.data_as(P), s.ctypes.data_as(P),
                                             int(num_nodes), int(num_edges), int(cluster),
                                             stored.ctypes.data_as(P), pair_of.ctypes.data_as(P)))
    return stored, pair_of


def e3conv_validate_graph(src, row_ptr, num_nodes, num_edges):
    """Raises E3ConvError(E3CONV_ERR_GRAPH) on a bad graph; host or device tensors/arrays."""
    import numpy as np
    lib = load_library()
    if hasattr(src, "is_cuda") and src.is_cuda:
        _check(lib.e3conv_validate_graph(_ptr(src), _ptr(row_ptr), int(num_nodes), int(num_edges), 1))
        return
    s = np.ascontiguousarray(np.asarray(src), dtype=np.int32)
    r = np.ascontiguousarray(np.asarray(row_ptr), dtype=np.int32)
    _check(lib.e3conv_validate_graph(s.ctypes.data_as(P), r.ctypes.data_as(P), int(num_nodes),
                                     int(num_edges), 0))


def e3conv_validate_graph_async(src, row_ptr, num_nodes, num_edges, result=None, stream=None):
    """Enqueue the device graph check; returns the int32[4] device result tensor
    (violations, first bad row_ptr index, first bad edge, 0), read it after the stream."""
    import torch
    _need(src, "src", torch.int32)
    _need(row_ptr, "row_ptr", torch.int32)
    if result is None:
        result = torch.empty(4, dtype=torch.int32, device=row_ptr.device)
    _need(result, "result", torch.int32)
    if result.numel() != 4:
        raise ValueError("result must hold 4 int32")
    _check(load_library().e3conv_validate_graph_async(_ptr(src), _ptr(row_ptr), int(num_nodes),
                                                      int(num_edges), _ptr(result), _stream(stream)))
    return result


def e3conv_validate_graph_noalloc(src, row_ptr, num_nodes, num_edges, stream=None):
    """Device graph check without allocation (the library's static result array); raises
    E3ConvError(E3CONV_ERR_GRAPH) on a bad graph."""
    import torch
    _need(src, "src", torch.int32)
    _need(row_ptr, "row_ptr", torch.int32)
    _check(load_library().e3conv_validate_graph_noalloc(_ptr(src), _ptr(row_ptr), int(num_nodes),
                                                        int(num_edges), _stream(stream)))


def e3conv_second_derivatives(handle, x, y, s, src, row_ptr, num_nodes, num_edges, num_real_nodes,
                              grad_out, cot_x, cot_y, cot_s, d_x, d_y, d_s, d_grad_out, order=None,
                              stream=None):
    """Gradient of <cot_x, grad_x> + <cot_y, grad_y> + <cot_s, grad_s> (the reverse pass's
    outputs) with respect to x, y, s and grad_out, written to d_x, d_y, d_s, d_grad_out."""
    import torch
    for t, name in ((x, "x"), (y, "y"), (s, "s"), (grad_out, "grad_out"), (cot_x, "cot_x"),
                    (cot_y, "cot_y"), (cot_s, "cot_s"), (d_x, "d_x"), (d_y, "d_y"), (d_s, "d_s"),
                    (d_grad_out, "d_grad_out")):
        _need(t, name, torch.float32)
    _check_graph_args(src, row_ptr, order)
    _check(load_library().e3conv_second_derivatives(
        handle, E3CONV_F32, _ptr(x), _ptr(y), _ptr(s), _ptr(src), _ptr(row_ptr), _ptr(order),
        int(num_nodes), int(num_edges), int(num_real_nodes), _ptr(grad_out), _ptr(cot_x),
        _ptr(cot_y), _ptr(cot_s), _ptr(d_x), _ptr(d_y), _ptr(d_s), _ptr(d_grad_out),
        _stream(stream)))
    return d_x, d_y, d_s, d_grad_out


def e3conv_stream_reference(src, dst=None, stream=None):
    """Streaming reference: copy src into dst (same size), or read src only if dst is None."""
    nbytes = src.numel() * src.element_size()
    if dst is not None and dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _check(load_library().e3conv_stream_reference(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def e3conv_status_string(status):
    return load_library().e3conv_status_string(int(status)).decode()


def e3conv_last_error_detail():
    return load_library().e3conv_last_error_detail().decode()


# ------------------------------------------------------ convenience ---

class Plan:
    """Owns a plan handle; shapes, forward and backward on torch tensors."""

    def __init__(self, irreps_in, sh_lmax, irreps_out, avg_num_neighbors=1.0,
                 ordering=E3CONV_RECEIVER):
        self.handle = e3conv_plan_ordered(irreps_in, sh_lmax, irreps_out, avg_num_neighbors, ordering)
        self.ordering = e3conv_plan_ordering(self.handle)
        (self.channels, self.num_x, self.num_y, self.num_paths,
         self.num_out) = e3conv_plan_shape(self.handle)
        self.avg_num_neighbors = float(avg_num_neighbors)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.e3conv_plan_destroy(h)
            self.handle = None

    def paths(self):
        return e3conv_plan_paths(self.handle)

    def coefficients(self):
        return e3conv_plan_coefficients(self.handle)

    def supported(self):
        return e3conv_plan_supported(self.handle)

    def num_variants(self, dtype=E3CONV_F32):
        return e3conv_plan_num_variants(self.handle, dtype)

    def set_variant(self, forward=0, backward=0):
        e3conv_plan_set_variant(self.handle, forward, backward)

    def num_out_blocks(self):
        return len({(p["l3"], p["p3"]) for p in self.paths()})

    def kernels_fused_linear(self, dtype=E3CONV_F32):
        """True if this plan has the forward with the output linear in its epilogue
        (asked with an empty graph: num_nodes = 0 is a no-op where it is compiled)."""
        return load_library().e3conv_forward_linear(self.handle, dtype, None, None, None, None, None,
                                                    None, 0, 0, 1.0, None, None, None) == E3CONV_OK

    def linear(self, inp, weights, channels_out, scale=1.0, out=None, stream=None):
        """Output linear (channel mixing per output irrep block); in (N, num_out, C)."""
        import torch
        N = inp.shape[0]
        if tuple(inp.shape) != (N, self.num_out, self.channels):
            raise ValueError(f"in must be (N, {self.num_out}, {self.channels}), got {tuple(inp.shape)}")
        if tuple(weights.shape) != (self.num_out_blocks(), self.channels, int(channels_out)):
            raise ValueError("weights must be (num_out_blocks, C, channels_out)")
        if out is None:
            out = torch.empty((N, self.num_out, int(channels_out)), dtype=torch.float32, device=inp.device)
        return e3conv_linear(self.handle, channels_out, scale, weights, inp, N, out, stream)

    def linear_backward(self, inp, weights, channels_out, grad_out, scale=1.0, want_in=True,
                        want_weights=True, stream=None):
        import torch
        N = inp.shape[0]
        if tuple(grad_out.shape) != (N, self.num_out, int(channels_out)):
            raise ValueError("grad_out must be (N, num_out, channels_out)")
        gi = torch.empty_like(inp) if want_in else None
        gw = torch.empty_like(weights) if want_weights else None
        return e3conv_linear_backward(self.handle, channels_out, scale, weights, inp, N,
                                      grad_out.contiguous(), gi, gw, stream)

    def _check_shapes(self, x, y, s, src, row_ptr):
        N, E = x.shape[0], s.shape[0]
        if tuple(x.shape) != (N, self.num_x, self.channels):
            raise ValueError(f"x must be (N, {self.num_x}, {self.channels}), got {tuple(x.shape)}")
        if tuple(y.shape) != (E, self.num_y):
            raise ValueError(f"y must be (E, {self.num_y}), got {tuple(y.shape)}")
        if tuple(s.shape) != (E, self.num_paths, self.channels):
            raise ValueError(f"s must be (E, {self.num_paths}, {self.channels}), got {tuple(s.shape)}")
        if src.numel() != E or row_ptr.numel() != N + 1:
            raise ValueError("src must have E entries and row_ptr N+1")
        return N, E

    def forward(self, x, y, s, src, row_ptr, out=None, order=None, stream=None, num_real_nodes=None):
        """out (N, num_out, C) fp32.  num_real_nodes: nodes from there on are padding."""
        import torch
        N, E = self._check_shapes(x, y, s, src, row_ptr)
        if order is not None and order.numel() != N:
            raise ValueError("order must have N entries")
        if out is None:
            out = torch.empty((N, self.num_out, self.channels), dtype=torch.float32, device=x.device)
        nr = N if num_real_nodes is None else int(num_real_nodes)
        return e3conv_forward_masked(self.handle, x, y, s, src, row_ptr, N, E, nr, out, order, stream)

    def forward_radial(self, x, y, r, w1, w2, src, row_ptr, r_max, sigma=0.5, out=None, order=None,
                       stream=None, num_real_nodes=None):
        """out (N, num_out, C) fp32 with s[e] = silu(f(r[e]) w1) w2 formed in the kernel.

        r (E,) edge lengths; w1 (num_basis, hidden); w2 (hidden, num_paths * C); f the
        Gaussian basis (centers k r_max / (num_basis - 1), width sigma) times the
        cosine cutoff.
        """
        import torch
        N, E = x.shape[0], r.shape[0]
        if tuple(x.shape) != (N, self.num_x, self.channels):
            raise ValueError(f"x must be (N, {self.num_x}, {self.channels}), got {tuple(x.shape)}")
        if tuple(y.shape) != (E, self.num_y) or tuple(r.shape) != (E,):
            raise ValueError(f"y must be (E, {self.num_y}) and r (E,), got {tuple(y.shape)}, {tuple(r.shape)}")
        if w2.dim() != 2 or w2.shape[1] != self.num_paths * self.channels:
            raise ValueError(f"w2 must be (hidden, {self.num_paths * self.channels}), got {tuple(w2.shape)}")
        if src.numel() != E or row_ptr.numel() != N + 1:
            raise ValueError("src must have E entries and row_ptr N+1")
        if order is not None and order.numel() != N:
            raise ValueError("order must have N entries")
        if out is None:
            out = torch.empty((N, self.num_out, self.channels), dtype=torch.float32, device=x.device)
        nr = N if num_real_nodes is None else int(num_real_nodes)
        return e3conv_forward_radial(self.handle, x, y, r, w1, w2, r_max, sigma, src, row_ptr, N, E, nr,
                                     out, order, stream)

    def jvp(self, x, y, s, dx, dy, ds, src, row_ptr, out=None, out_dot=None, order=None,
            stream=None, want_out=True, num_real_nodes=None):
        """(out, out_dot): the convolution and its derivative along (dx, dy, ds)."""
        import torch
        N, E = self._check_shapes(x, y, s, src, row_ptr)
        for t, ref, name in ((dx, x, "dx"), (dy, y, "dy"), (ds, s, "ds")):
            if tuple(t.shape) != tuple(ref.shape):
                raise ValueError(f"{name} must have shape {tuple(ref.shape)}, got {tuple(t.shape)}")
        if order is not None and order.numel() != N:
            raise ValueError("order must have N entries")
        shape = (N, self.num_out, self.channels)
        if out_dot is None:
            out_dot = torch.empty(shape, dtype=torch.float32, device=x.device)
        if want_out and out is None:
            out = torch.empty(shape, dtype=torch.float32, device=x.device)
        return e3conv_jvp(self.handle, x, y, s, dx, dy, ds, src, row_ptr, N, E,
                          out if want_out else None, out_dot, order, stream, num_real_nodes)

    def backward(self, x, y, s, src, row_ptr, grad_out, stream=None, grads=None, order=None,
                 num_real_nodes=None, accumulate=(False, False, False)):
        """(grad_x, grad_y, grad_s) of <grad_out, out>.

        grads: output arrays; an entry may be None in a given tuple to skip that
        gradient (returned as None).  accumulate[i]: add into grads[i] instead
        of overwriting it.
        """
        import torch
        N, E = self._check_shapes(x, y, s, src, row_ptr)
        if tuple(grad_out.shape) != (N, self.num_out, self.channels):
            raise ValueError(f"grad_out must be (N, {self.num_out}, {self.channels}), got {tuple(grad_out.shape)}")
        if grads is None:
            grads = (torch.empty_like(x, dtype=torch.float32), torch.empty_like(y, dtype=torch.float32),
                     torch.empty_like(s, dtype=torch.float32))
        gx, gy, gs = grads
        for gt, ref, name in ((gx, x, "grad_x"), (gy, y, "grad_y"), (gs, s, "grad_s")):
            if gt is not None and tuple(gt.shape) != tuple(ref.shape):
                raise ValueError(f"{name} must have shape {tuple(ref.shape)}, got {tuple(gt.shape)}")
        if order is not None and order.numel() != N:
            raise ValueError("order must have N entries")
        nr = N if num_real_nodes is None else int(num_real_nodes)
        flags = sum(bit for bit, on in zip((E3CONV_ACCUMULATE_GRAD_X, E3CONV_ACCUMULATE_GRAD_Y,
                                            E3CONV_ACCUMULATE_GRAD_S), accumulate) if on)
        e3conv_backward_ex(self.handle, x, y, s, src, row_ptr, N, E, nr, grad_out.contiguous(),
                           gx, gy, gs, flags, None, order, stream)
        return gx, gy, gs


    def second_derivatives(self, x, y, s, src, row_ptr, grad_out, cot_x, cot_y, cot_s,
                           order=None, num_real_nodes=None, stream=None, out=None):
        """(d_x, d_y, d_s, d_grad_out): gradient of <cot_x, grad_x> + <cot_y, grad_y> +
        <cot_s, grad_s> for the reverse pass at (x, y, s) with cotangent grad_out."""
        import torch
        N, E = self._check_shapes(x, y, s, src, row_ptr)
        if tuple(grad_out.shape) != (N, self.num_out, self.channels):
            raise ValueError(f"grad_out must be (N, {self.num_out}, {self.channels})")
        cot = tuple(t.contiguous() for t in (cot_x, cot_y, cot_s))
        for t, ref, name in zip(cot, (x, y, s), ("cot_x", "cot_y", "cot_s")):
            if tuple(t.shape) != tuple(ref.shape):
                raise ValueError(f"{name} must have shape {tuple(ref.shape)}, got {tuple(t.shape)}")
        if order is not None and order.numel() != N:
            raise ValueError("order must have N entries")
        if out is None:
            out = (torch.empty_like(x), torch.empty_like(y), torch.empty_like(s),
                   torch.empty_like(grad_out))
        nr = N if num_real_nodes is None else int(num_real_nodes)
        return e3conv_second_derivatives(self.handle, x, y, s, src, row_ptr, N, E, nr,
                                         grad_out.contiguous(), *cot, *out, order=order, stream=stream)

def _autograd_function():
    import torch

    class _ConvBackward(torch.autograd.Function):
        """(gx, gy, gs) = reverse pass at (x, y, s) for cotangent g; itself differentiable.

        L2 = <Gx, gx> + <Gy, gy> + <Gs, gs> is <g, D conv(x, y, s)[Gx, Gy, Gs]>, so
          dL2/dg = jvp of conv along (Gx, Gy, Gs),
          dL2/dx = reverse(x, Gy, s).gx + reverse(x, y, Gs).gx,
          dL2/dy = reverse(Gx, y, s).gy + reverse(x, y, Gs).gy,
          dL2/ds = reverse(Gx, y, s).gs + reverse(x, Gy, s).gs,
        each sum accumulated in place by the library's reverse kernel.
        """

        @staticmethod
        def forward(ctx, plan, graph, x, y, s, g):
            src, row_ptr, order, num_real = graph
            ctx.plan, ctx.graph = plan, graph
            ctx.save_for_backward(x, y, s, g)
            return plan.backward(x, y, s, src, row_ptr, g, order=order, num_real_nodes=num_real)

        @staticmethod
        def backward(ctx, Gx, Gy, Gs):
            x, y, s, g = ctx.saved_tensors
            src, row_ptr, order, num_real = ctx.graph
            dx, dy, ds, dg = ctx.plan.second_derivatives(x, y, s, src, row_ptr, g, Gx, Gy, Gs,
                                                         order=order, num_real_nodes=num_real)
            return None, None, dx, dy, ds, dg

    class E3ConvFunction(torch.autograd.Function):
        """out = conv(x, y, s) on a fixed graph; first and second derivatives (fp32).

        apply(plan, x, y, s, src, row_ptr, order=None, num_real_nodes=None).
        """

        @staticmethod
        def forward(ctx, plan, x, y, s, src, row_ptr, order=None, num_real_nodes=None):
            ctx.plan = plan
            ctx.graph = (src, row_ptr, order, num_real_nodes)
            ctx.save_for_backward(x, y, s)
            return plan.forward(x, y, s, src, row_ptr, order=order, num_real_nodes=num_real_nodes)

        @staticmethod
        def backward(ctx, grad_out):
            x, y, s = ctx.saved_tensors
            gx, gy, gs = _ConvBackward.apply(ctx.plan, ctx.graph, x, y, s, grad_out.contiguous())
            return None, gx, gy, gs, None, None, None, None

    return E3ConvFunction


def __getattr__(name):
    if name == "E3ConvFunction":
        return _autograd_function()
    raise AttributeError(name)
