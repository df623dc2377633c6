"""ctypes binding of libpeagle (include/peagle.h).

Argument marshalling only: every step of the draft forward runs in the library's HIP
kernels. torch provides device memory and the stream; tensors are passed by
``data_ptr()`` and work is enqueued on ``torch.cuda.current_stream()``.

bf16 tensors may be ``torch.bfloat16`` or ``torch.uint16``/``int16`` holding raw bits.
The library must be built (``python -m token_drafting_amd.build``); loading fails loudly
otherwise.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpeagle.so")
_lib = None

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, -1, -2, -3, -4
MAX_DEPTHS = 64

_i32, _i64, _u64, _f32, _f64, _p, _sz = (C.c_int32, C.c_int64, C.c_uint64, C.c_float,
                                         C.c_double, C.c_void_p, C.c_size_t)
_ATTN = [_i64, _i32, _i64, _p, _p, _p, _p, _i32, _p, _p, _p, _i32, _i32, _i32, _f32, _p, _p,
         _i32, _p, _p, _p, _sz, _p]
SIGNATURES = {
    "peagle_status_string": ([_i32], C.c_char_p),
    "peagle_version": ([], _i32),
    "peagle_cod_counts": ([_i64, _i32, _f64, _f64, _p, _p], _i32),
    "peagle_cod_workspace_bytes": ([_i64, _i32], _sz),
    "peagle_cod_select_noalloc": ([_i64, _i32, _f64, _f64, _u64, _p, _i32, _p, _p, _p, _p, _p],
                                  _i32),
    "peagle_cod_select": ([_i64, _i32, _f64, _f64, _u64, _p, _i32, _p, _p, _p, _p, _p, _sz, _p],
                          _i32),
    "peagle_fuse_inputs": ([_i64, _i32, _i64, _p, _p, _i32, _p, _p, _p, _p, _i32, _i32, _i32,
                            _p, _p, _p], _i32),
    "peagle_rope_table": ([_i32, _f64, _i32, _p, _p, _p], _i32),
    "peagle_draft_attn_workspace_bytes": ([_i64, _i64, _i32, _i32, _i32], _sz),
    "peagle_draft_attn_fwd": (_ATTN, _i32),
    "peagle_draft_attn_prepare": (_ATTN, _i32),
    "peagle_draft_attn_core": (_ATTN, _i32),
    "peagle_draft_attn_bwd_workspace_bytes": ([_i64, _i64, _i32, _i32, _i32], _sz),
    "peagle_draft_attn_bwd": ([_i64, _i32, _i64, _p, _p, _p, _p, _i32, _p, _p, _p, _i32, _i32,
                               _i32, _f32, _p, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _sz, _p],
                              _i32),
    "peagle_accept_prefix": ([_i32, _i32, _i32, _p, _p, _p, _p, _p, _p], _i32),
    "peagle_depth_ce_workspace_bytes": ([_i64, _i32], _sz),
    "peagle_depth_ce": ([_i64, _i32, _i32, _p, _p, _p, _f32, _p, _p, _p, _p, _sz, _p], _i32),
    "peagle_layer1_qkv_workspace_bytes": ([_i64, _i64, _i32], _sz),
    "peagle_layer1_qkv": ([_i64, _i32, _i64, _p, _p, _i32, _p, _p, _f32, _p, _i32, _i32, _i32, _p,
                           _p, _p, _p, _sz, _p], _i32),
    "peagle_layer1_post_workspace_bytes": ([_i64, _i64, _i32, _i32, _i32], _sz),
    "peagle_layer1_post": ([_i64, _i32, _i64, _p, _i32, _p, _i32, _p, _i32, _p, _p, _p, _p, _i32,
                            _p, _f32, _p, _p, _sz, _p], _i32),
    "peagle_layer_qkv_workspace_bytes": ([_i64, _i32], _sz),
    "peagle_layer_qkv": ([_i64, _p, _i32, _p, _f32, _p, _i32, _i32, _i32, _p, _p, _p, _p, _sz,
                          _p], _i32),
    "peagle_layer_post_workspace_bytes": ([_i64, _i32, _i32, _i32], _sz),
    "peagle_layer_post": ([_i64, _p, _i32, _p, _i32, _p, _p, _p, _p, _i32, _p, _f32, _p, _p, _sz,
                           _p], _i32),
    "peagle_draft_head_workspace_bytes": ([_i64, _i32, _i32], _sz),
    "peagle_draft_head": ([_i64, _p, _i32, _p, _p, _i32, _f32, _p, _p, _sz, _p], _i32),
    "peagle_fuse_inputs_fc_norm": ([_i64, _i32, _i64, _p, _p, _i32, _p, _p, _p, _p, _i32, _i32,
                                    _i32, _p, _f32, _p, _p, _p], _i32),
    "peagle_accept_prefix_d2t": ([_i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p], _i32),
    "peagle_accept_sampled": ([_i32, _i32, _i32, _p, _p, _p, _p, _p, _f32, _p, _p, _p], _i32),
    "peagle_accept_sampled_bonus": ([_i32, _i32, _i32, _p, _p, _p, _p, _p, _f32, _p, _p, _p],
                                    _i32),
    "peagle_decode_v_tiles_bytes": ([_i64, _i32, _i32, _i32], _sz),
    "peagle_decode_pack_v": ([_i32, _p, _i64, _i32, _p, _i32, _i32, _p, _sz, _p], _i32),
    "peagle_draft_decode_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i64, _i32], _sz),
    "peagle_draft_decode_attn": ([_i32, _i32, _p, _i64, _i32, _p, _p, _sz, _p, _p, _p, _i32,
                                  _i32, _i32, _f32, _p, _p, _i32, _p, _p, _p, _sz, _p], _i32),
    "peagle_draft_decode_attn_lens": ([_i32, _i32, _p, _p, _i64, _i32, _p, _p, _sz, _p, _p, _p,
                                       _i32, _i32, _i32, _f32, _p, _p, _i32, _p, _p, _p, _sz,
                                       _p], _i32),
    "peagle_decode_pack_v_lens": ([_i32, _p, _p, _i64, _i32, _p, _i32, _i32, _p, _sz, _p], _i32),
    "peagle_decode_append": ([_i32, _p, _p, _p, _i32, _i32, _p, _p, _i32, _i32, _p, _p, _i32,
                              _i64, _i32, _p, _p, _sz, _p, _p], _i32),
}


class PeagleError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({lib().peagle_status_string(status).decode()})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m token_drafting_amd.build`")
        h = C.CDLL(_LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(h, name)
            f.argtypes, f.restype = args, res
        _lib = h
    return _lib


def _check(fn: str, status: int):
    if status != OK:
        raise PeagleError(fn, status)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA tensor")
    return t


# ---------------------------------------------------------------- COD
def cod_counts(n: int, K: int, r: float, r_min: float) -> tuple[list, int]:
    m = (C.c_int64 * K)()
    T = C.c_int64()
    _check("peagle_cod_counts", lib().peagle_cod_counts(n, K, r, r_min, m, C.byref(T)))
    return list(m), T.value


def cod_workspace_bytes(n: int, K: int) -> int:
    return int(lib().peagle_cod_workspace_bytes(n, K))


def cod_select(n: int, K: int, r: float, r_min: float, seed: int, cu_seqlens: torch.Tensor):
    """Returns dict(m, T, idx, depth_off, cu_seqlens_d [K,S+1], row_of [K,n], workspace)."""
    _dev(cu_seqlens, "cu_seqlens")
    m, T = cod_counts(n, K, r, r_min)
    S = cu_seqlens.numel() - 1
    dev = cu_seqlens.device
    out = dict(m=m, T=T,
               idx=torch.empty(T, dtype=torch.int32, device=dev),
               depth_off=torch.empty(K + 1, dtype=torch.int32, device=dev),
               cu_seqlens_d=torch.empty((K, S + 1), dtype=torch.int32, device=dev),
               row_of=torch.empty((K, n), dtype=torch.int32, device=dev),
               workspace=torch.empty(cod_workspace_bytes(n, K), dtype=torch.uint8, device=dev))
    cod_select_into(n, K, r, r_min, seed, cu_seqlens, out)
    return out


def cod_select_into(n, K, r, r_min, seed, cu_seqlens, out):
    """Writes idx, depth_off, cu_seqlens_d and row_of of ``out`` (using its workspace)."""
    S = cu_seqlens.numel() - 1
    ws = out["workspace"]
    _check("peagle_cod_select", lib().peagle_cod_select(
        n, K, r, r_min, seed & ((1 << 64) - 1), _ptr(cu_seqlens), S, _ptr(out["idx"]),
        _ptr(out["depth_off"]), _ptr(out["cu_seqlens_d"]), _ptr(out["row_of"]), _ptr(ws),
        ws.numel(), _stream()))


COD_NOALLOC_SCRATCH_BYTES = 1 << 20   # PEAGLE_COD_NOALLOC_SCRATCH_BYTES


def cod_select_noalloc(n: int, K: int, r: float, r_min: float, seed: int, cu_seqlens, out):
    """peagle_cod_select_noalloc into the caller's tensors out[idx, depth_off, cu_seqlens_d,
    row_of] (no workspace: the library's static device scratch)."""
    _dev(cu_seqlens, "cu_seqlens")
    S = cu_seqlens.numel() - 1
    _check("peagle_cod_select_noalloc", lib().peagle_cod_select_noalloc(
        n, K, r, r_min, seed & ((1 << 64) - 1), _ptr(cu_seqlens), S, _ptr(out["idx"]),
        _ptr(out["depth_off"]), _ptr(out["cu_seqlens_d"]), _ptr(out["row_of"]), _stream()))
    return out


# ---------------------------------------------------------------- fuse
def fuse_inputs(n, K, T, idx, aux, fc_weight, mask_hidden, tokens, embed, ptd_token_id,
                hidden_out=None, embed_out=None, fc_norm_weight=None, eps=1e-6):
    H, A = fc_weight.shape
    vocab = embed.shape[0]
    for t, name in ((idx, "idx"), (aux, "aux"), (fc_weight, "fc_weight"),
                    (mask_hidden, "mask_hidden"), (tokens, "tokens"), (embed, "embed")):
        _dev(t, name)
    dev = aux.device
    if hidden_out is None:
        hidden_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if embed_out is None:
        embed_out = torch.empty((T, H), dtype=embed.dtype, device=dev)
    if fc_norm_weight is None:
        _check("peagle_fuse_inputs", lib().peagle_fuse_inputs(
            n, K, T, _ptr(idx), _ptr(aux), A, _ptr(fc_weight), _ptr(mask_hidden), _ptr(tokens),
            _ptr(embed), vocab, ptd_token_id, H, _ptr(hidden_out), _ptr(embed_out), _stream()))
    else:
        _dev(fc_norm_weight, "fc_norm_weight")
        _check("peagle_fuse_inputs_fc_norm", lib().peagle_fuse_inputs_fc_norm(
            n, K, T, _ptr(idx), _ptr(aux), A, _ptr(fc_weight), _ptr(mask_hidden), _ptr(tokens),
            _ptr(embed), vocab, ptd_token_id, H, _ptr(fc_norm_weight), float(eps),
            _ptr(hidden_out), _ptr(embed_out), _stream()))
    return hidden_out, embed_out


# ---------------------------------------------------------------- RoPE
def rope_table(head_dim: int, theta: float, max_pos: int, device="cuda"):
    cos = torch.empty((max_pos + 1, head_dim // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check("peagle_rope_table", lib().peagle_rope_table(head_dim, theta, max_pos, _ptr(cos),
                                                        _ptr(sin), _stream()))
    return cos, sin


def rope_max_pos(n: int, K: int) -> int:
    """Largest position any draft row can take: (n - 1) + (K - 1)."""
    return n + K - 2


# ---------------------------------------------------------------- attention
def attn_workspace_bytes(n, T, Hq, Hkv, D) -> int:
    return int(lib().peagle_draft_attn_workspace_bytes(n, T, Hq, Hkv, D))


def _attn_args(n, K, sel, cu_seqlens, q, k, v, cos, sin, out, lse, ws, scale):
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    S = cu_seqlens.numel() - 1
    return (n, K, T, _ptr(sel["idx"]), _ptr(sel["depth_off"]), _ptr(sel["row_of"]),
            _ptr(cu_seqlens), S, _ptr(q), _ptr(k), _ptr(v), Hq, Hkv, D,
            float(scale if scale is not None else 1.0 / math.sqrt(D)), _ptr(cos), _ptr(sin),
            cos.shape[0] - 1, _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream())


def draft_attn(n, K, sel, cu_seqlens, q, k, v, cos, sin, out=None, lse=None, workspace=None,
               scale=None, phase="fwd"):
    """phase: "fwd" (prepare + core), "prepare" or "core"."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (cos, "rope_cos"), (sin, "rope_sin")):
        _dev(t, name)
    T, Hq, D = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(attn_workspace_bytes(n, T, Hq, k.shape[1], D), dtype=torch.uint8,
                                device=dev)
    fn = {"fwd": "peagle_draft_attn_fwd", "prepare": "peagle_draft_attn_prepare",
          "core": "peagle_draft_attn_core"}[phase]
    _check(fn, getattr(lib(), fn)(*_attn_args(n, K, sel, cu_seqlens, q, k, v, cos, sin, out,
                                               lse, workspace, scale)))
    return out, lse, workspace


def draft_attn_bwd(n, K, sel, cu_seqlens, q, k, v, cos, sin, out, lse, dout, dq=None, dk=None,
                   dv=None, workspace=None, scale=None):
    """dq [T, Hq, D], dk and dv [T, Hkv, D] (fp32, with respect to the pre-RoPE inputs) of
    the draft attention, from the forward's out and lse on the same inputs and dout."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (cos, "rope_cos"), (sin, "rope_sin"),
                    (out, "out"), (lse, "lse"), (dout, "dout")):
        _dev(t, name)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if dq is None:
        dq = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((T, Hkv, D), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((T, Hkv, D), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(int(lib().peagle_draft_attn_bwd_workspace_bytes(n, T, Hq, Hkv, D)),
                                dtype=torch.uint8, device=dev)
    S = cu_seqlens.numel() - 1
    _check("peagle_draft_attn_bwd", lib().peagle_draft_attn_bwd(
        n, K, T, _ptr(sel["idx"]), _ptr(sel["depth_off"]), _ptr(sel["row_of"]), _ptr(cu_seqlens),
        S, _ptr(q), _ptr(k), _ptr(v), Hq, Hkv, D,
        float(scale if scale is not None else 1.0 / math.sqrt(D)), _ptr(cos), _ptr(sin),
        cos.shape[0] - 1, _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dv, workspace


def depth_ce(depth_off, logits, labels, decay=0.8, want_grad=True, loss=None, depth_loss=None,
             dlogits=None, workspace=None):
    """Depth-weighted cross-entropy: loss [1] (fp32), per-depth losses [K] and, with
    want_grad, d loss / d logits [T, V] (bf16 bits, int16)."""
    for t, name in ((depth_off, "depth_off"), (logits, "logits"), (labels, "labels")):
        _dev(t, name)
    T, V = logits.shape
    K = depth_off.numel() - 1
    dev = logits.device
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
    if depth_loss is None:
        depth_loss = torch.empty(K, dtype=torch.float32, device=dev)
    if want_grad and dlogits is None:
        dlogits = torch.empty((T, V), dtype=torch.int16, device=dev)
    if workspace is None:
        workspace = torch.empty(int(lib().peagle_depth_ce_workspace_bytes(T, K)),
                                dtype=torch.uint8, device=dev)
    _check("peagle_depth_ce", lib().peagle_depth_ce(
        T, K, V, _ptr(depth_off), _ptr(logits), _ptr(labels), float(decay), _ptr(loss),
        _ptr(depth_loss), _ptr(dlogits) if want_grad else None, _ptr(workspace),
        workspace.numel(), _stream()))
    return loss, depth_loss, dlogits


# ---------------------------------------------------------------- verify
def accept_prefix(draft_logits, target_logits, draft_tok=None, target_tok=None, accept_len=None):
    _dev(draft_logits, "draft_logits")
    _dev(target_logits, "target_logits")
    N, K, V = draft_logits.shape
    dev = draft_logits.device
    if draft_tok is None:
        draft_tok = torch.empty((N, K), dtype=torch.int32, device=dev)
    if target_tok is None:
        target_tok = torch.empty((N, K), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(N, dtype=torch.int32, device=dev)
    _check("peagle_accept_prefix", lib().peagle_accept_prefix(
        N, K, V, _ptr(draft_logits), _ptr(target_logits), _ptr(draft_tok), _ptr(target_tok),
        _ptr(accept_len), _stream()))
    return draft_tok, target_tok, accept_len


def accept_prefix_d2t(draft_logits, target_logits, d2t, draft_tok=None, target_tok=None,
                      accept_len=None):
    """Verification with a draft vocabulary of Vd ids mapped into the target's Vt by d2t."""
    for t, name in ((draft_logits, "draft_logits"), (target_logits, "target_logits"), (d2t, "d2t")):
        _dev(t, name)
    N, K, Vd = draft_logits.shape
    Vt = target_logits.shape[2]
    dev = draft_logits.device
    if draft_tok is None:
        draft_tok = torch.empty((N, K), dtype=torch.int32, device=dev)
    if target_tok is None:
        target_tok = torch.empty((N, K), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(N, dtype=torch.int32, device=dev)
    _check("peagle_accept_prefix_d2t", lib().peagle_accept_prefix_d2t(
        N, K, Vd, Vt, _ptr(draft_logits), _ptr(target_logits), _ptr(d2t), _ptr(draft_tok),
        _ptr(target_tok), _ptr(accept_len), _stream()))
    return draft_tok, target_tok, accept_len


def accept_sampled(draft_logits, target_logits, draft_tok, u, w, temperature=1.0,
                   accept_len=None, next_tok=None):
    """Speculative-sampling verification of sampled drafts: accept_len [N] and the token
    drawn from the residual at the first rejected depth (next_tok [N]). draft_tok int32
    [N, K]; u fp32 [N, K] and w fp32 [N] uniforms in [0, 1). target_logits [N, K, V]: all K
    accepted gives next_tok -1; [N, K + 1, V]: row K is the bonus distribution, drawn from
    when all K are accepted."""
    for t, name in ((draft_logits, "draft_logits"), (target_logits, "target_logits"),
                    (draft_tok, "draft_tok"), (u, "u"), (w, "w")):
        _dev(t, name)
    N, K, V = draft_logits.shape
    bonus = tuple(target_logits.shape) == (N, K + 1, V)
    if not (bonus or tuple(target_logits.shape) == (N, K, V)) or \
            tuple(draft_tok.shape) != (N, K) or tuple(u.shape) != (N, K) or tuple(w.shape) != (N,):
        raise ValueError("accept_sampled: shapes do not match [N, K, V] logits")
    dev = draft_logits.device
    if accept_len is None:
        accept_len = torch.empty(N, dtype=torch.int32, device=dev)
    if next_tok is None:
        next_tok = torch.empty(N, dtype=torch.int32, device=dev)
    fn = "peagle_accept_sampled_bonus" if bonus else "peagle_accept_sampled"
    _check(fn, getattr(lib(), fn)(
        N, K, V, _ptr(draft_logits), _ptr(target_logits), _ptr(draft_tok), _ptr(u), _ptr(w),
        float(temperature), _ptr(accept_len), _ptr(next_tok), _stream()))
    return accept_len, next_tok


# ---------------------------------------------------------------- first draft layer
def layer1_qkv_workspace_bytes(n: int, T: int, H: int) -> int:
    return int(lib().peagle_layer1_qkv_workspace_bytes(n, T, H))


def layer1_qkv(n, K, T, hidden, embed, w_norm_emb, w_norm_hidden, w_qkv, Hq, Hkv, D, eps=1e-6,
               q=None, k=None, v=None, workspace=None):
    """q [T, Hq, D], k and v [T, Hkv, D] (bf16, pre-RoPE) of the first draft layer from the
    fused stage's hidden_out [T, H] (fp32) and embed_out [T, H] (bf16)."""
    for t, name in ((hidden, "hidden"), (embed, "embed"), (w_norm_emb, "w_norm_emb"),
                    (w_norm_hidden, "w_norm_hidden"), (w_qkv, "w_qkv")):
        _dev(t, name)
    H = hidden.shape[1]
    dev = hidden.device
    if q is None:
        q = torch.empty((T, Hq, D), dtype=embed.dtype, device=dev)
    if k is None:
        k = torch.empty((T, Hkv, D), dtype=embed.dtype, device=dev)
    if v is None:
        v = torch.empty((T, Hkv, D), dtype=embed.dtype, device=dev)
    if workspace is None:
        workspace = torch.empty(layer1_qkv_workspace_bytes(n, T, H), dtype=torch.uint8, device=dev)
    _check("peagle_layer1_qkv", lib().peagle_layer1_qkv(
        n, K, T, _ptr(hidden), _ptr(embed), H, _ptr(w_norm_emb), _ptr(w_norm_hidden), float(eps),
        _ptr(w_qkv), Hq, Hkv, D, _ptr(q), _ptr(k), _ptr(v), _ptr(workspace), workspace.numel(),
        _stream()))
    return q, k, v


def layer1_post(n, K, T, attn_out, hidden, w_norm_hidden, w_o, w_post, w_gate, w_up, w_down,
                eps=1e-6, norm_before_residual=True, h2=None, workspace=None):
    """h2 [T, H] (fp32) of the first draft layer from the attention output [T, Hq, D] or
    [T, Hq*D] (fp32) and the fused stage's hidden_out [T, H]."""
    for t, name in ((attn_out, "attn_out"), (hidden, "hidden"), (w_o, "w_o"), (w_post, "w_post"),
                    (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _dev(t, name)
    H = hidden.shape[1]
    QW = attn_out.numel() // T
    I = w_gate.shape[0]
    dev = hidden.device
    if h2 is None:
        h2 = torch.empty((T, H), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(int(lib().peagle_layer1_post_workspace_bytes(n, T, H, QW, I)),
                                dtype=torch.uint8, device=dev)
    _check("peagle_layer1_post", lib().peagle_layer1_post(
        n, K, T, _ptr(attn_out), QW, _ptr(hidden), H, _ptr(w_norm_hidden),
        1 if norm_before_residual else 0, _ptr(w_o), _ptr(w_post), _ptr(w_gate), _ptr(w_up), I,
        _ptr(w_down), float(eps), _ptr(h2), _ptr(workspace), workspace.numel(), _stream()))
    return h2


def layer_qkv(h, w_norm, w_qkv, Hq, Hkv, D, eps=1e-6, q=None, k=None, v=None, workspace=None):
    """q [T, Hq, D], k and v [T, Hkv, D] (bf16, pre-RoPE) of a stacked draft layer (2nd and
    later) from the residual stream h [T, H] (fp32, the previous layer's output)."""
    for t, name in ((h, "h"), (w_norm, "w_norm"), (w_qkv, "w_qkv")):
        _dev(t, name)
    T, H = h.shape
    dev = h.device
    if q is None:
        q = torch.empty((T, Hq, D), dtype=w_qkv.dtype, device=dev)
    if k is None:
        k = torch.empty((T, Hkv, D), dtype=w_qkv.dtype, device=dev)
    if v is None:
        v = torch.empty((T, Hkv, D), dtype=w_qkv.dtype, device=dev)
    if workspace is None:
        workspace = torch.empty(int(lib().peagle_layer_qkv_workspace_bytes(T, H)),
                                dtype=torch.uint8, device=dev)
    _check("peagle_layer_qkv", lib().peagle_layer_qkv(
        T, _ptr(h), H, _ptr(w_norm), float(eps), _ptr(w_qkv), Hq, Hkv, D, _ptr(q), _ptr(k),
        _ptr(v), _ptr(workspace), workspace.numel(), _stream()))
    return q, k, v


def layer_post(attn_out, h, w_o, w_post, w_gate, w_up, w_down, eps=1e-6, h2=None,
               workspace=None):
    """h2 [T, H] (fp32) of a stacked draft layer from its attention output [T, Hq, D] or
    [T, Hq*D] (fp32) and its input residual stream h [T, H]; h2 may be h."""
    for t, name in ((attn_out, "attn_out"), (h, "h"), (w_o, "w_o"), (w_post, "w_post"),
                    (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _dev(t, name)
    T, H = h.shape
    QW = attn_out.numel() // T
    I = w_gate.shape[0]
    dev = h.device
    if h2 is None:
        h2 = torch.empty((T, H), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(int(lib().peagle_layer_post_workspace_bytes(T, H, QW, I)),
                                dtype=torch.uint8, device=dev)
    _check("peagle_layer_post", lib().peagle_layer_post(
        T, _ptr(attn_out), QW, _ptr(h), H, _ptr(w_o), _ptr(w_post), _ptr(w_gate), _ptr(w_up), I,
        _ptr(w_down), float(eps), _ptr(h2), _ptr(workspace), workspace.numel(), _stream()))
    return h2


def draft_head(h, w_final, w_head, eps=1e-6, tokens=None, workspace=None):
    """Argmax draft token [T] (int32) of rms(h) * w_final projected by w_head [V, H]."""
    for t, name in ((h, "h"), (w_final, "w_final"), (w_head, "w_head")):
        _dev(t, name)
    T, H = h.shape
    V = w_head.shape[0]
    dev = h.device
    if tokens is None:
        tokens = torch.empty(T, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(int(lib().peagle_draft_head_workspace_bytes(T, H, V)),
                                dtype=torch.uint8, device=dev)
    _check("peagle_draft_head", lib().peagle_draft_head(
        T, _ptr(h), H, _ptr(w_final), _ptr(w_head), V, float(eps), _ptr(tokens), _ptr(workspace),
        workspace.numel(), _stream()))
    return tokens


# ---------------------------------------------------------------- decode shape
def decode_v_tiles_bytes(total_ctx: int, B: int, Hkv: int, D: int) -> int:
    return int(lib().peagle_decode_v_tiles_bytes(total_ctx, B, Hkv, D))


def decode_pack_v(cu_ctx, max_ctx: int, v_cache, v_tiles=None):
    """V cache [Ltot, Hkv, D] (natural layout) -> the decode kernel's V tiles (flat bf16)."""
    _dev(cu_ctx, "cu_ctx")
    _dev(v_cache, "v_cache")
    Ltot, Hkv, D = v_cache.shape
    B = cu_ctx.numel() - 1
    nbytes = decode_v_tiles_bytes(Ltot, B, Hkv, D)
    if v_tiles is None:
        v_tiles = torch.zeros(max(nbytes // 2, 8), dtype=v_cache.dtype, device=v_cache.device)
    _check("peagle_decode_pack_v", lib().peagle_decode_pack_v(
        B, _ptr(cu_ctx), Ltot, max_ctx, _ptr(v_cache), Hkv, D, _ptr(v_tiles),
        v_tiles.numel() * v_tiles.element_size(), _stream()))
    return v_tiles


def decode_workspace_bytes(B, K, Hq, Hkv, D, total_ctx, max_ctx) -> int:
    return int(lib().peagle_draft_decode_workspace_bytes(B, K, Hq, Hkv, D, total_ctx, max_ctx))


def draft_decode_attn(cu_ctx, max_ctx: int, k_cache, v_tiles, q, k, v, cos, sin, out=None,
                      lse=None, workspace=None, scale=None):
    """K new rows per request over a KV cache: q [B, K, Hq, D], k/v [B, K, Hkv, D] (pre-RoPE
    q and k), k_cache [Ltot, Hkv, D] rotated, v_tiles from decode_pack_v.
    Returns out [B, K, Hq, D] fp32, lse [B, K, Hq] fp32 and the workspace."""
    for t, name in ((cu_ctx, "cu_ctx"), (k_cache, "k_cache"), (v_tiles, "v_tiles"), (q, "q"),
                    (k, "k"), (v, "v"), (cos, "rope_cos"), (sin, "rope_sin")):
        _dev(t, name)
    B, K, Hq, D = q.shape
    Hkv = k.shape[2]
    Ltot = k_cache.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((B, K, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, K, Hq), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(B, K, Hq, Hkv, D, Ltot, max_ctx),
                                dtype=torch.uint8, device=dev)
    _check("peagle_draft_decode_attn", lib().peagle_draft_decode_attn(
        B, K, _ptr(cu_ctx), Ltot, max_ctx, _ptr(k_cache), _ptr(v_tiles),
        v_tiles.numel() * v_tiles.element_size(), _ptr(q), _ptr(k), _ptr(v), Hq, Hkv, D,
        float(scale if scale is not None else 1.0 / math.sqrt(D)), _ptr(cos), _ptr(sin),
        cos.shape[0] - 1, _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse, workspace


# ---------------------------------------------------------------- decode loop
def decode_pack_v_lens(cu_cap, lens, max_cap: int, v_cache, v_tiles=None):
    """V tiles of a cache with per-request capacities (cu_cap) holding lens[b] rows each;
    zeros in the rest of every capacity."""
    for t, name in ((cu_cap, "cu_cap"), (lens, "lens"), (v_cache, "v_cache")):
        _dev(t, name)
    Ltot, Hkv, D = v_cache.shape
    B = cu_cap.numel() - 1
    nbytes = decode_v_tiles_bytes(Ltot, B, Hkv, D)
    if v_tiles is None:
        v_tiles = torch.zeros(max(nbytes // 2, 8), dtype=v_cache.dtype, device=v_cache.device)
    _check("peagle_decode_pack_v_lens", lib().peagle_decode_pack_v_lens(
        B, _ptr(cu_cap), _ptr(lens), Ltot, max_cap, _ptr(v_cache), Hkv, D, _ptr(v_tiles),
        v_tiles.numel() * v_tiles.element_size(), _stream()))
    return v_tiles


def draft_decode_attn_lens(cu_cap, lens, max_cap: int, k_cache, v_tiles, q, k, v, cos, sin,
                           out=None, lse=None, workspace=None, scale=None):
    """draft_decode_attn over a cache that grows in place: request b's context is the first
    lens[b] rows of its capacity [cu_cap[b], cu_cap[b+1])."""
    for t, name in ((cu_cap, "cu_cap"), (lens, "lens"), (k_cache, "k_cache"), (v_tiles, "v_tiles"),
                    (q, "q"), (k, "k"), (v, "v"), (cos, "rope_cos"), (sin, "rope_sin")):
        _dev(t, name)
    B, K, Hq, D = q.shape
    Hkv = k.shape[2]
    Ltot = k_cache.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((B, K, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, K, Hq), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(B, K, Hq, Hkv, D, Ltot, max_cap),
                                dtype=torch.uint8, device=dev)
    _check("peagle_draft_decode_attn_lens", lib().peagle_draft_decode_attn_lens(
        B, K, _ptr(cu_cap), _ptr(lens), Ltot, max_cap, _ptr(k_cache), _ptr(v_tiles),
        v_tiles.numel() * v_tiles.element_size(), _ptr(q), _ptr(k), _ptr(v), Hq, Hkv, D,
        float(scale if scale is not None else 1.0 / math.sqrt(D)), _ptr(cos), _ptr(sin),
        cos.shape[0] - 1, _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse, workspace


def decode_append(cu_cap, lens_in, n_new, n_add, max_cap: int, k_new, v_new, cos, sin, k_cache,
                  v_tiles, lens_out=None):
    """Append n_new[b] + n_add rows of k_new / v_new [B, max_new, Hkv, D] (pre-RoPE) to each
    request's context; returns the new lengths."""
    for t, name in ((cu_cap, "cu_cap"), (lens_in, "lens_in"), (n_new, "n_new"), (k_new, "k_new"),
                    (v_new, "v_new"), (cos, "rope_cos"), (sin, "rope_sin"), (k_cache, "k_cache"),
                    (v_tiles, "v_tiles")):
        _dev(t, name)
    B, max_new, Hkv, D = k_new.shape
    if lens_out is None:
        lens_out = torch.empty_like(lens_in)
    _check("peagle_decode_append", lib().peagle_decode_append(
        B, _ptr(cu_cap), _ptr(lens_in), _ptr(n_new), int(n_add), max_new, _ptr(k_new),
        _ptr(v_new), Hkv, D, _ptr(cos), _ptr(sin), cos.shape[0] - 1, k_cache.shape[0], max_cap,
        _ptr(k_cache), _ptr(v_tiles), v_tiles.numel() * v_tiles.element_size(), _ptr(lens_out),
        _stream()))
    return lens_out
