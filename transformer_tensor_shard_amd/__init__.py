"""transformer_tensor_shard_amd -- one tensor-parallel rank's share of a
Megatron-style Transformer block on one MI355X (gfx950).

Python face of libtp.so.  Each function has the name of the C entry point it
wraps (include/tp.h) and only marshals arguments: output and workspace tensors
are allocated with torch when the caller does not pass them, pointers and
dtype codes are handed to the library, and a non-zero status becomes an
exception (ValueError for unsupported shapes, the pages' convention for a
size that does not divide; TpError otherwise).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import TP_BF16, TP_EPI_GELU, TP_EPI_GELU_BWD, TP_EPI_GELU_SAVE, TP_EPI_NONE, TP_F32

__all__ = [
    "TpError", "tp_abi_version", "tp_mlp_shard", "tp_mlp_shard_workspace", "tp_attn_shard",
    "tp_attn_shard_workspace", "tp_partial_sum", "tp_block_shard", "tp_block_shard_workspace",
    "tp_linear", "tp_linear_batched", "tp_attention_core", "tp_layernorm", "tp_probe_mfma",
    "tp_matmul", "tp_matmul_grouped", "tp_gemm_tile_cols", "tp_mlp_shard_train_fwd", "tp_mlp_shard_backward",
    "tp_mlp_shard_backward_workspace", "tp_attention_core_train", "tp_attention_core_backward",
    "tp_attn_shard_train_fwd", "tp_attn_shard_backward", "tp_attn_shard_backward_workspace",
    "tp_vocab_embedding_shard", "tp_vocab_ce_shard", "tp_vocab_ce_shard_workspace",
    "tp_vocab_ce_combine", "tp_vocab_parallel_ce", "tp_vocab_parallel_ce_workspace",
    "tp_attention_kv_split", "tp_attention_kv_split_workspace", "tp_mlp_shard_noalloc", "lib",
]


class TpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.load().tp_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


def lib() -> ctypes.CDLL:
    """The loaded libtp.so (raw C ABI)."""
    return _lib.load()


def _check(status: int, where: str) -> None:
    if status == _lib.TP_OK:
        return
    if status == _lib.TP_ERR_SHAPE:
        raise ValueError(f"{where}: {_lib.load().tp_status_string(status).decode()}")
    raise TpError(status, where)


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return TP_F32
    if dtype == torch.bfloat16:
        return TP_BF16
    raise TypeError(f"unsupported dtype {dtype}: float32 or bfloat16")


def _dev(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dev_rows(t: torch.Tensor, name: str):
    """A 2-D GPU tensor whose rows are contiguous, at any row pitch (passed to
    the library as its leading dimension)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D GPU tensor with contiguous rows")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ws(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    if ws is None:
        ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    return ws


def _bytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def tp_abi_version() -> int:
    return int(_lib.load().tp_abi_version())


# ------------------------------------------------------------------ MLP
def tp_mlp_shard_workspace(M: int, f: int, in_dtype=torch.bfloat16) -> int:
    return int(_lib.load().tp_mlp_shard_workspace(M, f, _code(in_dtype)))


def tp_mlp_shard(X, A_i, B_i, a_i=None, *, out=None, out_dtype=torch.float32, ws=None,
                 stream=None):
    """Z_i = GeLU(X·A_i + a_i)·B_i for one rank; returns Z_i [M,h]."""
    M, h = X.shape
    f = A_i.shape[1]
    if out is None:
        out = torch.empty(M, h, dtype=out_dtype, device=X.device)
    ws = _ws(ws, tp_mlp_shard_workspace(M, f, X.dtype), X.device)
    st = _lib.load().tp_mlp_shard(_dev(X, "X"), _dev(A_i, "A_i"), _dev(a_i, "a_i"),
                                  _dev(B_i, "B_i"), _dev(out, "out"), _dev(ws, "ws"), _bytes(ws),
                                  M, h, f, _code(X.dtype), _code(out.dtype), _stream(stream))
    _check(st, "tp_mlp_shard")
    return out


def tp_mlp_shard_noalloc(X, A_i, B_i, a_i=None, *, out=None, out_dtype=torch.float32,
                         stream=None):
    """tp_mlp_shard without a workspace: Y'_i lives in the library's fixed
    device scratch (f·256·sizeof(X) <= 64 MiB); returns Z_i [M,h]."""
    M, h = X.shape
    f = A_i.shape[1]
    if out is None:
        out = torch.empty(M, h, dtype=out_dtype, device=X.device)
    st = _lib.load().tp_mlp_shard_noalloc(_dev(X, "X"), _dev(A_i, "A_i"), _dev(a_i, "a_i"),
                                          _dev(B_i, "B_i"), _dev(out, "out"), M, h, f,
                                          _code(X.dtype), _code(out.dtype), _stream(stream))
    _check(st, "tp_mlp_shard_noalloc")
    return out


def tp_mlp_shard_train_fwd(X, A_i, B_i, a_i=None, *, out=None, out_dtype=torch.float32,
                           Y_out=None, Yp_out=None, stream=None):
    """Z_i as tp_mlp_shard, also returning the saved activations:
    (Z_i [M,h], Y_i = X·A_i + a_i [M,f] bf16, Yp_i = GeLU(Y_i) [M,f] bf16)."""
    M, h = X.shape
    f = A_i.shape[1]
    if out is None:
        out = torch.empty(M, h, dtype=out_dtype, device=X.device)
    if Y_out is None:
        Y_out = torch.empty(M, f, dtype=torch.bfloat16, device=X.device)
    if Yp_out is None:
        Yp_out = torch.empty(M, f, dtype=torch.bfloat16, device=X.device)
    st = _lib.load().tp_mlp_shard_train_fwd(
        _dev(X, "X"), _dev(A_i, "A_i"), _dev(a_i, "a_i"), _dev(B_i, "B_i"), _dev(out, "out"),
        _dev(Y_out, "Y_out"), _dev(Yp_out, "Yp_out"), M, h, f, _code(out.dtype), _stream(stream))
    _check(st, "tp_mlp_shard_train_fwd")
    return out, Y_out, Yp_out


def tp_mlp_shard_backward_workspace(M: int, f: int) -> int:
    return int(_lib.load().tp_mlp_shard_backward_workspace(M, f))


def tp_mlp_shard_backward(X, A_i, B_i, Y_i, Yp_i, dZ, *, bias_grad=True, dx_dtype=torch.float32,
                          dX_out=None, dA_out=None, dB_out=None, da_out=None, ws=None,
                          stream=None):
    """One rank's MLP gradients from the saved activations: returns
    (dX_i [M,h] partial, dA_i [h,f] f32, dB_i [f,h] f32, da_i [f] f32 or None)."""
    M, h = X.shape
    f = A_i.shape[1]
    dev = X.device
    if dX_out is None:
        dX_out = torch.empty(M, h, dtype=dx_dtype, device=dev)
    if dA_out is None:
        dA_out = torch.empty(h, f, dtype=torch.float32, device=dev)
    if dB_out is None:
        dB_out = torch.empty(f, h, dtype=torch.float32, device=dev)
    if bias_grad and da_out is None:
        da_out = torch.empty(f, dtype=torch.float32, device=dev)
    ws = _ws(ws, tp_mlp_shard_backward_workspace(M, f), dev)
    st = _lib.load().tp_mlp_shard_backward(
        _dev(X, "X"), _dev(A_i, "A_i"), _dev(B_i, "B_i"), _dev(Y_i, "Y_i"), _dev(Yp_i, "Yp_i"),
        _dev(dZ, "dZ"), _dev(dX_out, "dX_out"), _dev(dA_out, "dA_out"), _dev(dB_out, "dB_out"),
        _dev(da_out if bias_grad else None, "da_out"), _dev(ws, "ws"), _bytes(ws), M, h, f,
        _code(dX_out.dtype), _stream(stream))
    _check(st, "tp_mlp_shard_backward")
    return dX_out, dA_out, dB_out, (da_out if bias_grad else None)


# ------------------------------------------------------------------ attention
def tp_attn_shard_workspace(b: int, s: int, H_l: int, d: int = 128) -> int:
    return int(_lib.load().tp_attn_shard_workspace(b, s, H_l, d))


def tp_attn_shard(X, W_qkv_i, W_o_i, b: int, s: int, H_l: int, d: int = 128, causal=True, *,
                  out=None, out_dtype=torch.float32, ws=None, stream=None):
    """Z_i = MHA over this rank's H_l heads, times its row block of W_o."""
    h = X.shape[1]
    if out is None:
        out = torch.empty(b * s, h, dtype=out_dtype, device=X.device)
    ws = _ws(ws, tp_attn_shard_workspace(b, s, H_l, d), X.device)
    st = _lib.load().tp_attn_shard(_dev(X, "X"), _dev(W_qkv_i, "W_qkv_i"), _dev(W_o_i, "W_o_i"),
                                   _dev(out, "out"), _dev(ws, "ws"), _bytes(ws), b, s, h, H_l, d,
                                   int(bool(causal)), _code(out.dtype), _stream(stream))
    _check(st, "tp_attn_shard")
    return out


# ------------------------------------------------------------------ partial sum
def tp_partial_sum(partials, bias=None, residual=None, *, out=None, out_dtype=torch.float32,
                   stream=None):
    """Z = sum_r partials[r] (+bias) (+residual); partials is [P, M, h]."""
    P, M, h = partials.shape
    if out is None:
        out = torch.empty(M, h, dtype=out_dtype, device=partials.device)
    res_code = _code(residual.dtype) if residual is not None else TP_F32
    st = _lib.load().tp_partial_sum(_dev(out, "out"), _code(out.dtype), _dev(partials, "partials"),
                                    _code(partials.dtype), P, M, h, _dev(bias, "bias"),
                                    _dev(residual, "residual"), res_code, _stream(stream))
    _check(st, "tp_partial_sum")
    return out


# ------------------------------------------------------------------ block
def tp_block_shard_workspace(b, s, h, H, d, F, P) -> int:
    return int(_lib.load().tp_block_shard_workspace(b, s, h, H, d, F, P))


def _ptr_array(ts: Sequence[torch.Tensor], name: str):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _dev(t, f"{name}[{i}]").value
    return arr


def tp_block_shard(x, W_qkv: Sequence, W_o: Sequence, A: Sequence, B: Sequence, b: int, s: int,
                   H: int, d: int = 128, *, ln1=(None, None), ln2=(None, None), eps=1e-5,
                   out=None, out_dtype=torch.float32, x1=None, ws=None, stream=None,
                   gelu_gemm_events=None):
    """Pre-LN block with every rank's share run in turn on this GPU.

    Returns out [b·s, h]; pass an f32 ``x1`` tensor to also receive the
    residual stream after attention.  ``gelu_gemm_events``, a pair of
    torch.cuda.Event(enable_timing=True), calls tp_block_shard_timed: the
    events are recorded around the MLP's grouped GeLU GEMM launch."""
    P = len(W_qkv)
    h = x.shape[1]
    F = A[0].shape[1] * P
    if out is None:
        out = torch.empty(b * s, h, dtype=out_dtype, device=x.device)
    ws = _ws(ws, tp_block_shard_workspace(b, s, h, H, d, F, P), x.device)
    args = (_dev(x, "x"), _dev(out, "out"), _code(out.dtype), _dev(x1, "x1"),
            _dev(ln1[0], "ln1_g"), _dev(ln1[1], "ln1_b"), _dev(ln2[0], "ln2_g"),
            _dev(ln2[1], "ln2_b"), float(eps), _ptr_array(W_qkv, "W_qkv"), _ptr_array(W_o, "W_o"),
            _ptr_array(A, "A"), _ptr_array(B, "B"), P, _dev(ws, "ws"), _bytes(ws), b, s, h, H, d,
            F, _stream(stream))
    if gelu_gemm_events is None:
        st = _lib.load().tp_block_shard(*args)
        _check(st, "tp_block_shard")
    else:
        ev = [_event(e) for e in gelu_gemm_events]
        st = _lib.load().tp_block_shard_timed(*args, ev[0], ev[1])
        _check(st, "tp_block_shard_timed")
    return out


def _event(e):
    """The raw hipEvent_t of a torch.cuda.Event (torch creates it lazily, on
    its first record, so an unused event is recorded once here)."""
    if not e.cuda_event:
        e.record()
    return ctypes.c_void_p(e.cuda_event)


# ------------------------------------------------------------------ components
def tp_linear(X, W, bias=None, *, gelu=False, out=None, out_dtype=torch.float32, stream=None):
    """C = epi(X·W + bias); X [M,K], W [K,N]."""
    M, K = X.shape
    N = W.shape[1]
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=X.device)
    st = _lib.load().tp_linear(_dev(X, "X"), K, _dev(W, "W"), N, _dev(bias, "bias"),
                               _dev(out, "out"), N, M, N, K, _code(X.dtype), _code(out.dtype),
                               TP_EPI_GELU if gelu else TP_EPI_NONE, _stream(stream))
    _check(st, "tp_linear")
    return out


def tp_linear_batched(Xs: Sequence, Ws: Sequence, biases=None, *, gelu=False, outs=None,
                      out_dtype=torch.float32, stream=None):
    """C[g] = epi(X[g]·W[g] + bias[g]) for every g in one grouped launch."""
    count = len(Xs)
    if len(Ws) != count or (outs is not None and len(outs) != count):
        raise ValueError("Xs, Ws and outs must have the same length")
    M, K = Xs[0].shape
    N = Ws[0].shape[1]
    for X, W in zip(Xs, Ws):
        if tuple(X.shape) != (M, K) or tuple(W.shape) != (K, N) or X.dtype != Xs[0].dtype:
            raise ValueError("all products must have the same shape and dtype")
    if outs is None:
        outs = [torch.empty(M, N, dtype=out_dtype, device=Xs[0].device) for _ in range(count)]
    bias_arr = None
    if biases is not None:
        bias_arr = (ctypes.c_void_p * count)(
            *[(_dev(bv, "bias").value if bv is not None else None) for bv in biases])
    st = _lib.load().tp_linear_batched(
        _ptr_array(Xs, "X"), K, _ptr_array(Ws, "W"), N, bias_arr, _ptr_array(outs, "out"), N,
        count, M, N, K, _code(Xs[0].dtype), _code(outs[0].dtype),
        TP_EPI_GELU if gelu else TP_EPI_NONE, _stream(stream))
    _check(st, "tp_linear_batched")
    return outs


_EPILOGUES = {"none": TP_EPI_NONE, "gelu": TP_EPI_GELU, "gelu_bwd": TP_EPI_GELU_BWD,
              "gelu_save": TP_EPI_GELU_SAVE}


def tp_matmul(A, B, bias=None, *, trans_a=False, trans_b=False, epilogue="none", aux=None,
              out=None, out_dtype=torch.float32, stream=None):
    """C = epi(op(A)·op(B) + bias) on bf16 operands: op(A) = A.T when trans_a
    (A stored [K,M]), op(B) = B.T when trans_b (B stored [N,K]).  epilogue:
    "none", "gelu", "gelu_bwd" (C ⊙ GeLU'(aux)) or "gelu_save" (aux receives
    the pre-activation).  Returns C [M,N]."""
    M, K = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    N = B.shape[0] if trans_b else B.shape[1]
    if (B.shape[1] if trans_b else B.shape[0]) != K:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} and {tuple(B.shape)}")
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=A.device)
    if epilogue == "gelu_save" and aux is None:
        aux = torch.empty(M, N, dtype=torch.bfloat16, device=A.device)
    st = _lib.load().tp_matmul(
        _dev(A, "A"), A.shape[1], int(bool(trans_a)), _dev(B, "B"), B.shape[1],
        int(bool(trans_b)), _dev(bias, "bias"), _dev(out, "out"), out.shape[1], _dev(aux, "aux"),
        aux.shape[1] if aux is not None else 0, M, N, K, _code(out.dtype), _EPILOGUES[epilogue],
        _stream(stream))
    _check(st, "tp_matmul")
    return (out, aux) if epilogue == "gelu_save" else out


def tp_gemm_tile_cols(shapes, K: int, *, trans_a=False, trans_b=False, epilogue="none") -> int:
    """Output-tile width (128, 192, 256 or 384 columns) the bf16 GEMM uses for one
    launch of the products `shapes` = [(M, N), ...] with inner size K on the
    current device (256 compute units when there is none).  Host logic only."""
    count = len(shapes)
    I64 = ctypes.c_int64 * max(count, 1)
    cols = _lib.load().tp_gemm_tile_cols(int(bool(trans_a)), int(bool(trans_b)),
                                         _EPILOGUES[epilogue], count,
                                         I64(*[m for m, _ in shapes]), I64(*[n for _, n in shapes]),
                                         int(K))
    if cols == 0:
        raise ValueError(f"tp_gemm_tile_cols: invalid launch {shapes}, K={K}")
    return cols


def tp_matmul_grouped(As, Bs, *, trans_a=False, trans_b=False, outs=None,
                      out_dtype=torch.float32, ws=None, stream=None):
    """C[g] = op(A[g])·op(B[g]) for every g in one launch; the products share
    layout and K but may differ in M and N.  ws: optional device memory the
    launch may use to split its last wave of workgroups over K (f32 output).
    Returns the list of C[g]."""
    count = len(As)
    if len(Bs) != count or (outs is not None and len(outs) != count):
        raise ValueError("As, Bs and outs must have the same length")
    Ms = [A.shape[1] if trans_a else A.shape[0] for A in As]
    Ks = {A.shape[0] if trans_a else A.shape[1] for A in As}
    Ks |= {B.shape[1] if trans_b else B.shape[0] for B in Bs}
    if len(Ks) != 1:
        raise ValueError("all products must share the inner size K")
    K = Ks.pop()
    Ns = [B.shape[0] if trans_b else B.shape[1] for B in Bs]
    if outs is None:
        outs = [torch.empty(m, n, dtype=out_dtype, device=As[0].device) for m, n in zip(Ms, Ns)]
    I64 = ctypes.c_int64 * count
    st = _lib.load().tp_matmul_grouped(
        _ptr_array(As, "A"), I64(*[A.shape[1] for A in As]), int(bool(trans_a)),
        _ptr_array(Bs, "B"), I64(*[B.shape[1] for B in Bs]), int(bool(trans_b)),
        _ptr_array(outs, "out"), I64(*[C.shape[1] for C in outs]), I64(*Ms), I64(*Ns), count, K,
        _code(outs[0].dtype), _dev(ws, "ws"), _bytes(ws) if ws is not None else 0,
        _stream(stream))
    _check(st, "tp_matmul_grouped")
    return outs


def tp_attention_kv_split_workspace(b: int, s: int, H: int, P: int, d: int = 128) -> int:
    return int(_lib.load().tp_attention_kv_split_workspace(b, s, H, d, P))


def tp_attention_kv_split(qkv, b: int, s: int, H: int, P: int, d: int = 128, causal=True, *,
                          out=None, ws=None, stream=None):
    """Attention with Q, K, V split along the feature dimension over P ranks:
    partial scores per rank, summed before the softmax, each rank its output
    feature slice.  qkv [b·s, ld] bf16 ([Q | K | V], H·d each); returns O
    [b·s, H·d] bf16."""
    dev = qkv.device
    if out is None:
        out = torch.empty(b * s, H * d, dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = torch.empty(tp_attention_kv_split_workspace(b, s, H, P, d), dtype=torch.uint8,
                         device=dev)
    st = _lib.load().tp_attention_kv_split(_dev_rows(qkv, "qkv"), qkv.stride(0),
                                           _dev_rows(out, "out"),
                                           out.stride(0), b, s, H, d, P, int(bool(causal)),
                                           _dev(ws, "ws"), ws.numel() * ws.element_size(),
                                           _stream(stream))
    _check(st, "tp_attention_kv_split")
    return out


def tp_attention_core(qkv, b: int, s: int, H_l: int, d: int = 128, causal=True, *, out=None,
                      stream=None):
    """O = softmax(QK^T/sqrt d)·V per (sequence, head); qkv [b·s, ld] bf16."""
    if out is None:
        out = torch.empty(b * s, H_l * d, dtype=torch.bfloat16, device=qkv.device)
    st = _lib.load().tp_attention_core(_dev(qkv, "qkv"), qkv.shape[1], _dev(out, "out"), b, s,
                                       H_l, d, int(bool(causal)), _stream(stream))
    _check(st, "tp_attention_core")
    return out


def tp_attention_core_train(qkv, b: int, s: int, H_l: int, d: int = 128, causal=True, *,
                            out=None, lse=None, stream=None):
    """tp_attention_core that also returns the per-query base-2 log of the
    softmax normaliser: (O [b·s, H_l·d] bf16, lse [b, H_l, s] f32)."""
    dev = qkv.device
    if out is None:
        out = torch.empty(b * s, H_l * d, dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty(b, H_l, s, dtype=torch.float32, device=dev)
    st = _lib.load().tp_attention_core_train(_dev(qkv, "qkv"), qkv.shape[1], _dev(out, "out"),
                                             _dev(lse, "lse"), b, s, H_l, d, int(bool(causal)),
                                             _stream(stream))
    _check(st, "tp_attention_core_train")
    return out, lse


def tp_attention_core_backward(qkv, O, dO, lse, b: int, s: int, H_l: int, d: int = 128,
                               causal=True, *, dqkv=None, D_ws=None, stream=None):
    """dQ, dK, dV of tp_attention_core in qkv's layout: dqkv [b·s, 3·H_l·d] bf16."""
    dev = qkv.device
    if dqkv is None:
        dqkv = torch.empty(b * s, 3 * H_l * d, dtype=torch.bfloat16, device=dev)
    if D_ws is None:
        D_ws = torch.empty(b * H_l * s, dtype=torch.float32, device=dev)
    st = _lib.load().tp_attention_core_backward(
        _dev(qkv, "qkv"), qkv.shape[1], _dev(O, "O"), _dev(dO, "dO"), _dev(lse, "lse"),
        _dev(dqkv, "dqkv"), _dev(D_ws, "D_ws"), b, s, H_l, d, int(bool(causal)), _stream(stream))
    _check(st, "tp_attention_core_backward")
    return dqkv


def tp_attn_shard_train_fwd(X, W_qkv_i, W_o_i, b: int, s: int, H_l: int, d: int = 128,
                            causal=True, *, out=None, out_dtype=torch.float32, qkv_out=None,
                            O_out=None, lse_out=None, stream=None):
    """Z_i as tp_attn_shard plus the saved activations: (Z_i, qkv, O, lse)."""
    M, h = X.shape
    dev = X.device
    HD = H_l * d
    if out is None:
        out = torch.empty(M, h, dtype=out_dtype, device=dev)
    if qkv_out is None:
        qkv_out = torch.empty(M, 3 * HD, dtype=torch.bfloat16, device=dev)
    if O_out is None:
        O_out = torch.empty(M, HD, dtype=torch.bfloat16, device=dev)
    if lse_out is None:
        lse_out = torch.empty(b, H_l, s, dtype=torch.float32, device=dev)
    st = _lib.load().tp_attn_shard_train_fwd(
        _dev(X, "X"), _dev(W_qkv_i, "W_qkv_i"), _dev(W_o_i, "W_o_i"), _dev(out, "out"),
        _dev(qkv_out, "qkv_out"), _dev(O_out, "O_out"), _dev(lse_out, "lse_out"), b, s, h, H_l,
        d, int(bool(causal)), _code(out.dtype), _stream(stream))
    _check(st, "tp_attn_shard_train_fwd")
    return out, qkv_out, O_out, lse_out


def tp_attn_shard_backward_workspace(b: int, s: int, H_l: int, d: int = 128) -> int:
    return int(_lib.load().tp_attn_shard_backward_workspace(b, s, H_l, d))


def tp_attn_shard_backward(X, W_qkv_i, W_o_i, qkv, O, lse, dZ, b: int, s: int, H_l: int,
                           d: int = 128, causal=True, *, dx_dtype=torch.float32, dX_out=None,
                           dWqkv_out=None, dWo_out=None, ws=None, stream=None):
    """One rank's attention gradients from the saved activations:
    (dX_i [b·s, h] partial, dW_qkv,i [h, 3·H_l·d] f32, dW_o,i [H_l·d, h] f32)."""
    M, h = X.shape
    dev = X.device
    HD = H_l * d
    if dX_out is None:
        dX_out = torch.empty(M, h, dtype=dx_dtype, device=dev)
    if dWqkv_out is None:
        dWqkv_out = torch.empty(h, 3 * HD, dtype=torch.float32, device=dev)
    if dWo_out is None:
        dWo_out = torch.empty(HD, h, dtype=torch.float32, device=dev)
    ws = _ws(ws, tp_attn_shard_backward_workspace(b, s, H_l, d), dev)
    st = _lib.load().tp_attn_shard_backward(
        _dev(X, "X"), _dev(W_qkv_i, "W_qkv_i"), _dev(W_o_i, "W_o_i"), _dev(qkv, "qkv"),
        _dev(O, "O"), _dev(lse, "lse"), _dev(dZ, "dZ"), _dev(dX_out, "dX_out"),
        _dev(dWqkv_out, "dWqkv_out"), _dev(dWo_out, "dWo_out"), _dev(ws, "ws"), _bytes(ws), b, s,
        h, H_l, d, int(bool(causal)), _code(dX_out.dtype), _stream(stream))
    _check(st, "tp_attn_shard_backward")
    return dX_out, dWqkv_out, dWo_out


# ------------------------------------------------------------------ vocabulary ends
def _tokens(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _dev(t, name)


def tp_vocab_embedding_shard(tokens, E_r, vocab_start: int, *, out=None,
                             out_dtype=torch.float32, stream=None):
    """One rank's embedding share: E_r[token - vocab_start] or a zero row."""
    M = tokens.numel()
    V_r, h = E_r.shape
    if out is None:
        out = torch.empty(M, h, dtype=out_dtype, device=E_r.device)
    st = _lib.load().tp_vocab_embedding_shard(_tokens(tokens, "tokens"), M, _dev(E_r, "E_r"), V_r,
                                              h, int(vocab_start), _dev(out, "out"),
                                              _code(out.dtype), _stream(stream))
    _check(st, "tp_vocab_embedding_shard")
    return out


def tp_vocab_ce_shard_workspace(M: int, V_r: int) -> int:
    return int(_lib.load().tp_vocab_ce_shard_workspace(M, V_r))


def tp_vocab_ce_shard(H, E_r, targets, vocab_start: int, *, stats=None, ws=None, stream=None):
    """One rank's cross-entropy statistics [3, M] f32: row max, exp-sum, target logit."""
    M, h = H.shape
    V_r = E_r.shape[0]
    if stats is None:
        stats = torch.empty(3, M, dtype=torch.float32, device=H.device)
    ws = _ws(ws, tp_vocab_ce_shard_workspace(M, V_r), H.device)
    st = _lib.load().tp_vocab_ce_shard(_dev(H, "H"), _dev(E_r, "E_r"), _tokens(targets, "targets"),
                                       M, h, V_r, int(vocab_start), _dev(stats, "stats"),
                                       _dev(ws, "ws"), _bytes(ws), _stream(stream))
    _check(st, "tp_vocab_ce_shard")
    return stats


def tp_vocab_ce_combine(stats, *, loss=None, loss_mean=None, stream=None):
    """Combine ranks' statistics [P, 3, M] into the loss [M] and its mean [1]."""
    P, three, M = stats.shape
    if loss is None:
        loss = torch.empty(M, dtype=torch.float32, device=stats.device)
    if loss_mean is None:
        loss_mean = torch.empty(1, dtype=torch.float32, device=stats.device)
    st = _lib.load().tp_vocab_ce_combine(_dev(stats, "stats"), P, M, _dev(loss, "loss"),
                                         _dev(loss_mean, "loss_mean"), _stream(stream))
    _check(st, "tp_vocab_ce_combine")
    return loss, loss_mean


def tp_vocab_parallel_ce_workspace(M: int, V_r: int, P: int) -> int:
    return int(_lib.load().tp_vocab_parallel_ce_workspace(M, V_r, P))


def tp_vocab_parallel_ce(H, Es: Sequence, targets, *, loss=None, loss_mean=None, ws=None,
                         stream=None):
    """All ranks of the vocab-parallel cross-entropy: rank r's table Es[r]
    covers rows [r·V_r, (r+1)·V_r).  Returns (loss [M], mean [1])."""
    M, h = H.shape
    P, V_r = len(Es), Es[0].shape[0]
    dev = H.device
    if loss is None:
        loss = torch.empty(M, dtype=torch.float32, device=dev)
    if loss_mean is None:
        loss_mean = torch.empty(1, dtype=torch.float32, device=dev)
    ws = _ws(ws, tp_vocab_parallel_ce_workspace(M, V_r, P), dev)
    st = _lib.load().tp_vocab_parallel_ce(_dev(H, "H"), _ptr_array(Es, "E"), P,
                                          _tokens(targets, "targets"), M, h, V_r,
                                          _dev(loss, "loss"), _dev(loss_mean, "loss_mean"),
                                          _dev(ws, "ws"), _bytes(ws), _stream(stream))
    _check(st, "tp_vocab_parallel_ce")
    return loss, loss_mean


def tp_layernorm(x, gamma=None, beta=None, eps=1e-5, *, out=None, stream=None):
    """bf16 LayerNorm of each row of x [M,h] (x in f32 or bf16)."""
    M, h = x.shape
    if out is None:
        out = torch.empty(M, h, dtype=torch.bfloat16, device=x.device)
    st = _lib.load().tp_layernorm(_dev(x, "x"), _code(x.dtype), _dev(out, "out"),
                                  _dev(gamma, "gamma"), _dev(beta, "beta"), float(eps), M, h,
                                  _stream(stream))
    _check(st, "tp_layernorm")
    return out


# ------------------------------------------------------------------ measurement support
def tp_probe_mfma(blocks: int = 256, iters: int = 2000, *, out=None, stream=None) -> int:
    """Launch the register-only MFMA loop; returns the FLOPs of the launch."""
    if out is None:
        out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    st = _lib.load().tp_probe_mfma(_dev(out, "out"), int(blocks), int(iters), _stream(stream))
    _check(st, "tp_probe_mfma")
    return blocks * 8 * 32 * iters * 16384
