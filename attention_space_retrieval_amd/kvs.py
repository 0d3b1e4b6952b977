"""Python binding of libkvs (ctypes): argument marshalling only.

Each function carries the name of the C entry point it calls and takes torch
tensors that live on the GPU; every step of the computation runs in the HIP
library.  There is no CPU fallback: a missing library raises at import of the
first call, a tensor that is not on a GPU raises, and a non-zero status from
the library raises KvsError.  Work is enqueued on torch's current stream of
the tensors' device, without synchronising.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvs.so")

KVS_F32, KVS_BF16 = 0, 1
STATUS = {0: "KVS_OK", 1: "KVS_ERR_ARG", 2: "KVS_ERR_SHAPE", 3: "KVS_ERR_DTYPE",
          4: "KVS_ERR_UNSUPPORTED", 5: "KVS_ERR_WORKSPACE", 6: "KVS_ERR_HIP", 7: "KVS_ERR_LIMIT"}

# (name, restype, argtypes)
_P, _I32, _I64, _F32, _F64, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
_SIGNATURES = [
    ("kvs_status_string", ctypes.c_char_p, [_I32]),
    ("kvs_version", _I32, []),
    ("kvs_qmem_update", _I32, [_P, _I32, _I32, _I32, _I32, _I32, _F32, _I32, _P, _P]),
    ("kvs_rule_score_workspace", _SZ, [_I32, _I32, _I32, _I64]),
    ("kvs_rule_score", _I32, [_P, _I32, _P, _I32, _I32, _I32, _I32, _I64, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    ("kvs_rule_score_paged", _I32, [_P, _I32, _P, _I64, _P, _I32, _I32, _I32, _I32, _I64, _I64, _I64,
                                    _I64, _P, _P, _SZ, _P]),
    ("kvs_rule_score_wait_limit", _I64, [_I64]),
    ("kvs_window_score_workspace", _SZ, [_I32, _I32, _I32, _I64, _I64]),
    ("kvs_window_score", _I32, [_P, _P, _I32, _I32, _I32, _I32, _I64, _I64, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    ("kvs_topk_workspace", _SZ, [_I64]),
    ("kvs_topk_select", _I32, [_P, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    ("kvs_topk_select_redirect", _I32, [_P, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _I64, _P, _P,
                                        _SZ, _P]),
    ("kvs_topk_noalloc_max", _I64, []),
    ("kvs_topk_select_noalloc", _I32, [_P, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    ("kvs_slotmap_redirect", _I32, [_P, _P, _I64, _I64, _P, _P]),
    ("kvs_meank_build", _I32, [_P, _I32, _I32, _I32, _I64, _I32, _I32, _I64, _F64, _P, _P, _P]),
    ("kvs_meank_append", _I32, [_P, _I32, _I32, _I32, _I64, _I64, _I64, _F64, _P, _I64, _P, _P]),
    ("kvs_meank_score_workspace", _SZ, [_I32, _I32, _I32, _I64, _I64]),
    ("kvs_meank_score", _I32, [_P, _P, _I32, _I32, _I32, _I32, _I64, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    ("kvs_rerope_scatter", _I32, [_P, _P, _I64, _P, _P, _I64, _I32, _I32, _I32, _I32, _I64, _F64,
                                  _P, _P, _I64, _P, _P]),
    ("kvs_working_set_workspace", _SZ, [_I64]),
    ("kvs_working_set_update", _I32, [_P, _P, _I64, _P, _P, _I64, _P, _I64, _I32, _I32, _I32, _I32, _I64,
                                      _F64, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
]
ENTRY_POINTS = [s[0] for s in _SIGNATURES]


class KvsError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


_lib = None


def load():
    """Load libkvs.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m attention_space_retrieval_amd.build_lib`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGNATURES:
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib = lib
    return _lib


def _check(fn, status):
    if status != 0:
        raise KvsError(fn, status)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libkvs works on GPU tensors only")
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("libkvs needs contiguous tensors")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t):
    if t.dtype == torch.float32:
        return KVS_F32
    if t.dtype == torch.bfloat16:
        return KVS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(nbytes, device, ws):
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def kvs_version():
    return load().kvs_version()


def kvs_qmem_update(q_span, lam, M, first_turn):
    """QueryMemory step in place on M [L, H_q, D] float32; q_span [L, H_q, S, D]."""
    _dev(q_span, M)
    L, H_q, S, D = q_span.shape
    if M.dtype != torch.float32 or tuple(M.shape) != (L, H_q, D):
        raise ValueError("M must be float32 [L, H_q, D]")
    _check("kvs_qmem_update", load().kvs_qmem_update(
        _ptr(q_span), _dtype_code(q_span), L, H_q, S, D, float(lam), int(bool(first_turn)),
        _ptr(M), _stream(M)))
    return M


def kvs_rule_score_workspace(L, H_q, H_kv, N):
    return load().kvs_rule_score_workspace(L, H_q, H_kv, N)


def kvs_rule_score(K, M, pi, q_s, q_e, rule=None, ws=None):
    """rule [N] float32 from K [L, H_kv, N, D] and M [L, H_q, D]."""
    _dev(K, M, rule, ws)
    L, H_kv, N, D = K.shape
    H_q = M.shape[1]
    _need(M.dtype == torch.float32 and tuple(M.shape) == (L, H_q, D), "M must be float32 [L, H_q, D]")
    _need(rule is None or (rule.dtype == torch.float32 and rule.numel() == N), "rule must be float32 [N]")
    if rule is None:
        rule = torch.empty(N, dtype=torch.float32, device=K.device)
    need = kvs_rule_score_workspace(L, H_q, H_kv, N)
    ws = _workspace(need, K.device, ws)
    _check("kvs_rule_score", load().kvs_rule_score(
        _ptr(K), _dtype_code(K), _ptr(M), L, H_q, H_kv, D, N, pi, q_s, q_e, _ptr(rule),
        _ptr(ws), _nbytes(ws), _stream(K)))
    return rule


def kvs_rule_score_paged(K_pool, slots, M, pi, q_s, q_e, rule=None, ws=None):
    """rule [N] from the token-major pool K_pool [L, pool_size, H_kv, D] read through slots [N] (int64)."""
    _dev(K_pool, slots, M, rule, ws)
    L, pool_size, H_kv, D = K_pool.shape
    _need(M.dtype == torch.float32 and M.dim() == 3 and M.shape[0] == L and M.shape[2] == D,
          "M must be float32 [L, H_q, D]")
    if slots.dtype != torch.int64:
        raise TypeError("slots must be int64")
    H_q, N = M.shape[1], slots.numel()
    if rule is None:
        rule = torch.empty(N, dtype=torch.float32, device=K_pool.device)
    _need(rule.dtype == torch.float32 and rule.numel() == N, "rule must be float32 [N]")
    if ws is None:
        ws = torch.empty(max(1, kvs_rule_score_workspace(L, H_q, H_kv, N)), dtype=torch.uint8,
                         device=K_pool.device)
    _check("kvs_rule_score_paged", load().kvs_rule_score_paged(
        _ptr(K_pool), _dtype_code(K_pool), _ptr(slots), pool_size, _ptr(M), L, H_q, H_kv, D, N, int(pi),
        int(q_s), int(q_e), _ptr(rule), _ptr(ws), _nbytes(ws), _stream(K_pool)))
    return rule


def kvs_rule_score_wait_limit(polls):
    """Bounded wait of the rule scorer's fold in polls (< 0: every chunk takes the spill path);
    returns the previous setting.  Process-wide; a diagnostic and test setting."""
    return int(load().kvs_rule_score_wait_limit(int(polls)))


def kvs_window_score_workspace(L, H_q, H_kv, W, N):
    return load().kvs_window_score_workspace(L, H_q, H_kv, W, N)


def kvs_window_score(K, Qw, pi, q_s, q_e, score=None, ws=None):
    """score [N] float32 from bf16 K [L, H_kv, N, D] and bf16 window rows Qw [L, H_q, W, D]."""
    _dev(K, Qw, score, ws)
    if K.dtype != torch.bfloat16 or Qw.dtype != torch.bfloat16:
        raise TypeError("K and Qw must be bfloat16")
    L, H_kv, N, D = K.shape
    H_q, W = Qw.shape[1], Qw.shape[2]
    _need(Qw.shape[0] == L and Qw.shape[3] == D, "Qw must be [L, H_q, W, D] like K")
    if score is None:
        score = torch.empty(N, dtype=torch.float32, device=K.device)
    _need(score.dtype == torch.float32 and score.numel() == N, "score must be float32 [N]")
    if ws is None:
        ws = torch.empty(max(1, kvs_window_score_workspace(L, H_q, H_kv, W, N)), dtype=torch.uint8,
                         device=K.device)
    _check("kvs_window_score", load().kvs_window_score(
        _ptr(K), _ptr(Qw), L, H_q, H_kv, D, N, W, int(pi), int(q_s), int(q_e), _ptr(score), _ptr(ws),
        _nbytes(ws), _stream(K)))
    return score


def kvs_topk_workspace(n):
    return load().kvs_topk_workspace(n)


def kvs_topk_select(score, f0, f1, C, keep_mask=None, keep_idx=None, n_kept=None, ws=None,
                    single_workgroup=False):
    """Returns (keep_mask uint8 [n], keep_idx int32 [n], n_kept int64 [1]) on the device.

    Above 32768 scores the library selects with several workgroups through a
    small workspace; single_workgroup=True passes none (the slower path)."""
    _dev(score, keep_mask, keep_idx, n_kept, ws)
    if score.dtype != torch.float32:
        raise TypeError("score must be float32")
    n = score.numel()
    dev = score.device
    keep_mask = torch.empty(n, dtype=torch.uint8, device=dev) if keep_mask is None else keep_mask
    keep_idx = torch.empty(n, dtype=torch.int32, device=dev) if keep_idx is None else keep_idx
    n_kept = torch.empty(1, dtype=torch.int64, device=dev) if n_kept is None else n_kept
    _need(keep_mask.dtype == torch.uint8 and keep_mask.numel() == n, "keep_mask must be uint8 [n]")
    _need(keep_idx.dtype == torch.int32 and keep_idx.numel() >= n, "keep_idx must be int32 [n]")
    _need(n_kept.dtype == torch.int64 and n_kept.numel() >= 1, "n_kept must be int64 [1]")
    need = kvs_topk_workspace(n)
    if single_workgroup:
        ws = None
    elif need:
        ws = _workspace(need, dev, ws)
    _check("kvs_topk_select", load().kvs_topk_select(
        _ptr(score), n, f0[0], f0[1], f1[0], f1[1], C, _ptr(keep_mask), _ptr(keep_idx),
        _ptr(n_kept), _ptr(ws), _nbytes(ws), _stream(score)))
    return keep_mask, keep_idx, n_kept


def kvs_topk_select_redirect(score, f0, f1, C, slot_in, dead_slot, keep_mask=None, keep_idx=None, n_kept=None,
                             slot_out=None, ws=None, single_workgroup=False):
    """kvs_topk_select with the slot-map redirect written by the same launch: returns
    (keep_mask, keep_idx, n_kept, slot_out), slot_out[j] = slot_in[j] if kept else dead_slot
    (slot_out may be slot_in itself).  single_workgroup as in kvs_topk_select."""
    _dev(score, slot_in, keep_mask, keep_idx, n_kept, slot_out, ws)
    if score.dtype != torch.float32:
        raise TypeError("score must be float32")
    if slot_in.dtype != torch.int64:
        raise TypeError("slot_in must be int64")
    n = score.numel()
    dev = score.device
    keep_mask = torch.empty(n, dtype=torch.uint8, device=dev) if keep_mask is None else keep_mask
    keep_idx = torch.empty(n, dtype=torch.int32, device=dev) if keep_idx is None else keep_idx
    n_kept = torch.empty(1, dtype=torch.int64, device=dev) if n_kept is None else n_kept
    slot_out = torch.empty_like(slot_in) if slot_out is None else slot_out
    _need(keep_mask.dtype == torch.uint8 and keep_mask.numel() == n, "keep_mask must be uint8 [n]")
    _need(keep_idx.dtype == torch.int32 and keep_idx.numel() >= n, "keep_idx must be int32 [n]")
    _need(n_kept.dtype == torch.int64 and n_kept.numel() >= 1, "n_kept must be int64 [1]")
    _need(slot_in.numel() == n and slot_out.numel() == n and slot_out.dtype == torch.int64,
          "slot_in and slot_out must be int64 [n]")
    need = kvs_topk_workspace(n)
    if single_workgroup:
        ws = None
    elif need:
        ws = _workspace(need, dev, ws)
    _check("kvs_topk_select_redirect", load().kvs_topk_select_redirect(
        _ptr(score), n, f0[0], f0[1], f1[0], f1[1], C, _ptr(keep_mask), _ptr(keep_idx), _ptr(n_kept),
        _ptr(slot_in), int(dead_slot), _ptr(slot_out), _ptr(ws), _nbytes(ws), _stream(score)))
    return keep_mask, keep_idx, n_kept, slot_out


def kvs_topk_noalloc_max():
    return load().kvs_topk_noalloc_max()


def kvs_topk_select_noalloc(score, f0, f1, C, keep_mask, keep_idx, n_kept):
    """kvs_topk_select without a workspace: the library's own static device array holds the
    multi-workgroup state (n <= kvs_topk_noalloc_max(); calls overlapping on one device race).
    The caller passes every output; nothing is allocated."""
    _dev(score, keep_mask, keep_idx, n_kept)
    if score.dtype != torch.float32:
        raise TypeError("score must be float32")
    n = score.numel()
    _need(keep_mask.dtype == torch.uint8 and keep_mask.numel() == n, "keep_mask must be uint8 [n]")
    _need(keep_idx.dtype == torch.int32 and keep_idx.numel() >= n, "keep_idx must be int32 [n]")
    _need(n_kept.dtype == torch.int64 and n_kept.numel() >= 1, "n_kept must be int64 [1]")
    if n > kvs_topk_noalloc_max():
        raise ValueError(f"kvs_topk_select_noalloc takes at most {kvs_topk_noalloc_max()} scores, got {n}")
    _check("kvs_topk_select_noalloc", load().kvs_topk_select_noalloc(
        _ptr(score), n, f0[0], f0[1], f1[0], f1[1], C, _ptr(keep_mask), _ptr(keep_idx), _ptr(n_kept),
        _stream(score)))
    return keep_mask, keep_idx, n_kept


def kvs_slotmap_redirect(slot_in, keep_mask, dead_slot, slot_out=None):
    _dev(slot_in, keep_mask, slot_out)
    if slot_in.dtype != torch.int64 or keep_mask.dtype != torch.uint8:
        raise TypeError("slot_in must be int64 and keep_mask uint8")
    slot_out = torch.empty_like(slot_in) if slot_out is None else slot_out
    _need(keep_mask.numel() == slot_in.numel() and slot_out.numel() == slot_in.numel()
          and slot_out.dtype == torch.int64, "slot_in, keep_mask and slot_out must have N elements")
    _check("kvs_slotmap_redirect", load().kvs_slotmap_redirect(
        _ptr(slot_in), _ptr(keep_mask), slot_in.numel(), int(dead_slot), _ptr(slot_out),
        _stream(slot_in)))
    return slot_out


def kvs_meank_build(K, k_is_rope=False, pos0=0, theta=1e6, raw_k_out=None, index=None, block=32):
    """Mean-K index bf16 [L, H_kv, ceil(N/block), D] from bf16 K [L, H_kv, N, D]."""
    _dev(K, raw_k_out, index)
    if K.dtype != torch.bfloat16:
        raise TypeError("K must be bfloat16")
    L, H_kv, N, D = K.shape
    nB = -(-N // block)
    if index is None:
        index = torch.empty((L, H_kv, nB, D), dtype=torch.bfloat16, device=K.device)
    _need(index.dtype == torch.bfloat16 and tuple(index.shape) == (L, H_kv, nB, D),
          "index must be bf16 [L, H_kv, ceil(N/block), D]")
    _need(raw_k_out is None or (raw_k_out.dtype == torch.bfloat16 and raw_k_out.shape == K.shape),
          "raw_k_out must be bf16 shaped like K")
    _check("kvs_meank_build", load().kvs_meank_build(
        _ptr(K), L, H_kv, D, N, block, int(bool(k_is_rope)), int(pos0), float(theta),
        _ptr(raw_k_out), _ptr(index), _stream(K)))
    return index


def kvs_meank_append(k_chunk, t0, raw_stage, index, pos0=0, theta=1e6):
    """Append the post-RoPE keys k_chunk [L, H_kv, n, D] (bf16) of tokens t0..t0+n-1:
    their raw K goes to raw_stage [L, H_kv, cap, D], the blocks they touch to index
    [L, H_kv, ceil(cap/32), D].  Returns index."""
    _dev(k_chunk, raw_stage, index)
    for t, name in ((k_chunk, "k_chunk"), (raw_stage, "raw_stage"), (index, "index")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    L, H_kv, n, D = k_chunk.shape
    cap = raw_stage.shape[2]
    _need(tuple(raw_stage.shape) == (L, H_kv, cap, D), "raw_stage must be [L, H_kv, cap, D] like k_chunk")
    _need(tuple(index.shape) == (L, H_kv, -(-cap // 32), D), "index must be [L, H_kv, ceil(cap/32), D]")
    _check("kvs_meank_append", load().kvs_meank_append(
        _ptr(k_chunk), L, H_kv, D, int(t0), n, int(pos0), float(theta), _ptr(raw_stage), cap,
        _ptr(index), _stream(raw_stage)))
    return index


def kvs_meank_score_workspace(L, H_q, H_kv, Mq, nB):
    return load().kvs_meank_score_workspace(L, H_q, H_kv, Mq, nB)


def kvs_meank_score(Q, index, n_sink, n_recent, R=None, ws=None):
    """R [nB] float32 from Q [L, H_q, Mq, D] and index [L, H_kv, nB, D] (both bf16)."""
    _dev(Q, index, R, ws)
    if Q.dtype != torch.bfloat16 or index.dtype != torch.bfloat16:
        raise TypeError("Q and index must be bfloat16")
    L, H_q, Mq, D = Q.shape
    H_kv, nB = index.shape[1], index.shape[2]
    _need(index.shape[0] == L and index.shape[3] == D, "index must be [L, H_kv, nB, D] like Q")
    _need(R is None or (R.dtype == torch.float32 and R.numel() == nB), "R must be float32 [nB]")
    R = torch.empty(nB, dtype=torch.float32, device=Q.device) if R is None else R
    need = kvs_meank_score_workspace(L, H_q, H_kv, Mq, nB)
    ws = _workspace(need, Q.device, ws)
    _check("kvs_meank_score", load().kvs_meank_score(
        _ptr(Q), _ptr(index), L, H_q, H_kv, D, Mq, nB, n_sink, n_recent, _ptr(R), _ptr(ws),
        _nbytes(ws), _stream(Q)))
    return R


def kvs_rerope_scatter(k_src, v_src, src_block, page_table, n_sel, pos_base, theta, k_pool,
                       v_pool, err_flag=None, block=32):
    """Scatter n_sel selected raw-K/V blocks into the pools with RoPE at compact positions."""
    _dev(k_src, v_src, src_block, page_table, k_pool, v_pool, err_flag)
    L, H_kv, src_tokens, D = k_src.shape
    pool_pages = k_pool.shape[2] // block
    _need(k_src.dtype == torch.bfloat16 and k_pool.dtype == torch.bfloat16, "K tensors must be bf16")
    _need(k_pool.shape[0] == L and k_pool.shape[1] == H_kv and k_pool.shape[3] == D
          and k_pool.shape[2] % block == 0, "k_pool must be [L, H_kv, pages*block, D]")
    _need((v_src is None) == (v_pool is None), "v_src and v_pool go together")
    _need(v_src is None or (v_src.shape == k_src.shape and v_pool.shape == k_pool.shape
                            and v_src.dtype == torch.bfloat16 and v_pool.dtype == torch.bfloat16),
          "V tensors must be bf16 shaped like the K tensors")
    _need(src_block.numel() >= n_sel and (page_table is None or page_table.numel() >= n_sel),
          "src_block and page_table need n_sel entries")
    _need(err_flag is None or (err_flag.dtype == torch.int32 and err_flag.numel() >= 1),
          "err_flag must be int32 [1]")
    if src_block.dtype != torch.int32 or (page_table is not None and page_table.dtype != torch.int32):
        raise TypeError("src_block and page_table must be int32")
    _check("kvs_rerope_scatter", load().kvs_rerope_scatter(
        _ptr(k_src), _ptr(v_src), src_tokens, _ptr(src_block), _ptr(page_table), int(n_sel), L,
        H_kv, D, block, int(pos_base), float(theta), _ptr(k_pool), _ptr(v_pool), pool_pages,
        _ptr(err_flag), _stream(k_src)))
    return k_pool, v_pool



def kvs_working_set_workspace(pool_pages):
    return load().kvs_working_set_workspace(pool_pages)


def kvs_working_set_update(k_src, v_src, prev_blocks, prev_pages, new_blocks, pos_base, theta, k_pool,
                           v_pool, err_flag=None, ws=None, block=32):
    """Differential working-set update of the pools (in place).

    prev_blocks/prev_pages: int32 G_{t-1} (ascending) and their pages; new_blocks: int32 W_t
    (ascending).  Returns (pages [n_new], old_rank [n_new], outgoing_pages [n_prev], counts [3]);
    the first counts[2] entries of outgoing_pages are the released pages.
    """
    _dev(k_src, v_src, prev_blocks, prev_pages, new_blocks, k_pool, v_pool, err_flag, ws)
    L, H_kv, src_tokens, D = k_src.shape
    pool_pages = k_pool.shape[2] // block
    _need(k_src.dtype == torch.bfloat16 and k_pool.dtype == torch.bfloat16, "K tensors must be bf16")
    _need(k_pool.shape[0] == L and k_pool.shape[1] == H_kv and k_pool.shape[3] == D
          and k_pool.shape[2] % block == 0, "k_pool must be [L, H_kv, pages*block, D]")
    _need((v_src is None) == (v_pool is None), "v_src and v_pool go together")
    _need(v_src is None or (v_src.shape == k_src.shape and v_pool.shape == k_pool.shape
                            and v_src.dtype == torch.bfloat16 and v_pool.dtype == torch.bfloat16),
          "V tensors must be bf16 shaped like the K tensors")
    for t in (prev_blocks, prev_pages, new_blocks):
        if t.dtype != torch.int32:
            raise TypeError("block ids and pages must be int32")
    n_prev, n_new = prev_blocks.numel(), new_blocks.numel()
    _need(prev_pages.numel() == n_prev, "prev_pages needs one page per previous block")
    _need(err_flag is None or (err_flag.dtype == torch.int32 and err_flag.numel() >= 1),
          "err_flag must be int32 [1]")
    dev = k_src.device
    pages = torch.empty(n_new, dtype=torch.int32, device=dev)
    old_rank = torch.empty(n_new, dtype=torch.int32, device=dev)
    outgoing = torch.empty(max(n_prev, 1), dtype=torch.int32, device=dev)
    counts = torch.empty(3, dtype=torch.int64, device=dev)
    if ws is None:
        ws = torch.empty(max(1, kvs_working_set_workspace(pool_pages)), dtype=torch.uint8, device=dev)
    _check("kvs_working_set_update", load().kvs_working_set_update(
        _ptr(k_src), _ptr(v_src), src_tokens, _ptr(prev_blocks), _ptr(prev_pages), n_prev,
        _ptr(new_blocks), n_new, L, H_kv, D, block, int(pos_base), float(theta), _ptr(k_pool),
        _ptr(v_pool), pool_pages, _ptr(pages), _ptr(old_rank), _ptr(outgoing), _ptr(counts),
        _ptr(err_flag), _ptr(ws), _nbytes(ws), _stream(k_src)))
    return pages, old_rank, outgoing[:n_prev], counts
