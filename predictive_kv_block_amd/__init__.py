"""Python binding of libspin, the MI355X SPIN decode-round library.

Argument marshalling only: every function forwards torch tensors' device
pointers and the current HIP stream to the C ABI declared in include/spin.h,
under the same names.  All computation runs in the library's HIP kernels; if
libspin.so is missing, load() raises instead of falling back to anything.
"""
import ctypes
import os

__all__ = [
    "load", "SpinError", "SpinState", "make_config", "make_batch",
    "spin_state_bytes", "spin_state_layout_of", "spin_state_init", "spin_state_destroy",
    "spin_reset_slots", "spin_predict_blocks", "spin_quantize_q", "spin_indexer_scores",
    "spin_topk_scores", "spin_topk_workspace_bytes", "spin_indexer_topk", "spin_update",
    "spin_mtp_replay", "spin_topk_update", "spin_measure_miss", "spin_allocate_budgets",
    "spin_allocate_budgets_curve", "spin_status_string", "spin_slot_scores", "spin_estimate_miss",
    "spin_predictor_fidelity",
    "spin_attention_workspace_bytes", "spin_sparse_attention", "spin_topk_scores_noalloc",
    "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspin.so")

EXPORTS = [
    "spin_state_bytes", "spin_state_layout_of", "spin_state_init", "spin_state_destroy",
    "spin_reset_slots", "spin_predict_blocks", "spin_quantize_q", "spin_indexer_scores",
    "spin_topk_scores", "spin_topk_workspace_bytes", "spin_indexer_topk", "spin_update",
    "spin_mtp_replay", "spin_topk_update", "spin_measure_miss", "spin_allocate_budgets",
    "spin_allocate_budgets_curve", "spin_status_string", "spin_slot_scores", "spin_estimate_miss",
    "spin_predictor_fidelity",
    "spin_attention_workspace_bytes", "spin_sparse_attention", "spin_topk_scores_noalloc",
]

SPIN_OK, SPIN_EINVAL, SPIN_EUNSUPPORTED, SPIN_EHIP, SPIN_ESTATE, SPIN_ESCRATCH = 0, -1, -2, -3, -4, -5
ERR_QPOS, ERR_SLOT, ERR_KEPT, ERR_PAGE, ERR_ACCEPT = 1, 2, 4, 8, 16


class SpinConfig(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("max_slots", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("max_rows", ctypes.c_int32), ("warmup_steps", ctypes.c_int32),
        ("explore_bp", ctypes.c_int32), ("alpha", ctypes.c_float),
        ("policy", ctypes.c_uint32), ("seed", ctypes.c_uint64),
    ]


class SpinBatch(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("R", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("slot", ctypes.c_void_p), ("qpos", ctypes.c_void_p),
    ]


class SpinLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("V", "D", "VB", "step", "request_id", "error", "tail_gate", "q8", "wq",
                 "qexp", "bscore", "ukey", "page_qmax", "topk_ws", "total")] + [
        ("max_blocks", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SpinError(RuntimeError):
    def __init__(self, status, text):
        super().__init__(f"spin status {status}: {text}")
        self.status = status


_lib = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "spin_state_bytes": [ctypes.POINTER(SpinConfig), ctypes.POINTER(_sz)],
    "spin_state_layout_of": [ctypes.POINTER(SpinConfig), ctypes.POINTER(SpinLayout)],
    "spin_state_init": [ctypes.POINTER(SpinConfig), _vp, _sz, _vp, ctypes.POINTER(_vp)],
    "spin_state_destroy": [_vp],
    "spin_reset_slots": [_vp, _i32, _vp, _vp, _vp],
    "spin_predict_blocks": [_vp, _i32, ctypes.POINTER(SpinBatch), _i32, _vp, _vp, _vp, _vp],
    "spin_quantize_q": [_vp, ctypes.POINTER(SpinBatch), _vp, _vp, _vp],
    "spin_indexer_scores": [_vp, ctypes.POINTER(SpinBatch), _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                            _vp],
    "spin_topk_scores": [ctypes.POINTER(SpinBatch), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "spin_topk_workspace_bytes": [ctypes.POINTER(SpinBatch), _i32, ctypes.POINTER(_sz)],
    "spin_topk_scores_noalloc": [ctypes.POINTER(SpinBatch), _i32, _vp, _vp, _vp, _vp, _vp, _vp],
    "spin_indexer_topk": [_vp, ctypes.POINTER(SpinBatch), _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                          _vp, _vp, _vp],
    "spin_update": [_vp, _i32, ctypes.POINTER(SpinBatch), _vp, _vp, _vp, _vp],
    "spin_mtp_replay": [_vp, _i32, ctypes.POINTER(SpinBatch), _vp, _vp, _vp, _vp, _vp],
    "spin_topk_update": [_vp, _i32, ctypes.POINTER(SpinBatch), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _vp],
    "spin_measure_miss": [ctypes.POINTER(SpinBatch), _i32, _vp, _vp, _vp, _vp],
    "spin_allocate_budgets": [_i32, ctypes.POINTER(ctypes.c_double), _i32,
                              ctypes.POINTER(ctypes.c_int32)],
    "spin_allocate_budgets_curve": [_i32, _i32, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int32), _i32,
                                    ctypes.POINTER(ctypes.c_int32)],
    "spin_status_string": [_i32],
    "spin_slot_scores": [_vp, _i32, ctypes.POINTER(SpinBatch), _vp, _vp],
    "spin_estimate_miss": [ctypes.POINTER(SpinBatch), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "spin_predictor_fidelity": [ctypes.POINTER(SpinBatch), _i32, _vp, _vp, _vp, _vp, _vp, _vp],
    "spin_attention_workspace_bytes": [ctypes.POINTER(SpinBatch), _i32, ctypes.POINTER(_sz)],
    "spin_sparse_attention": [ctypes.POINTER(SpinBatch), _i32, _vp, _vp, _vp, _i64, _vp,
                              ctypes.c_float, _vp, _vp, _vp, _sz, _vp],
}


def load(path=None):
    """Load libspin.so (built by predictive_kv_block_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m predictive_kv_block_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "spin_status_string" else ctypes.c_int
    _lib = lib
    return lib


def spin_status_string(status):
    return load().spin_status_string(int(status)).decode()


def _check(rc):
    if rc != SPIN_OK:
        raise SpinError(rc, spin_status_string(rc))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


SPIN_POOL_MAX, SPIN_POOL_MEAN, SPIN_POOL_TOP4, SPIN_MASK_ROW0 = 0, 1, 2, 4


def make_config(num_layers, max_slots, max_ctx, topk, max_rows=1, heads=64, head_dim=128,
                warmup_steps=1, explore_bp=500, alpha=0.9, seed=0x5350494E, policy=0):
    """policy: SPIN_POOL_MAX / SPIN_POOL_MEAN / SPIN_POOL_TOP4, optionally | SPIN_MASK_ROW0."""
    return SpinConfig(num_layers, max_slots, max_ctx, 64, heads, head_dim, topk, max_rows,
                      warmup_steps, explore_bp, alpha, int(policy), seed)


def make_batch(slot, qpos, R, max_blocks):
    """A spin_batch over device int32 tensors slot [B] and qpos [B]."""
    b = SpinBatch(int(qpos.numel()), int(R), int(max_blocks), 0, _p(slot), _p(qpos))
    b._keep = (slot, qpos)
    return b


# ------------------------------------------------------------------ state
def spin_state_bytes(cfg):
    n = _sz()
    _check(load().spin_state_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def spin_state_layout_of(cfg):
    lay = SpinLayout()
    _check(load().spin_state_layout_of(ctypes.byref(cfg), ctypes.byref(lay)))
    return {f: getattr(lay, f) for f, _ in SpinLayout._fields_}


def spin_state_init(cfg, state_mem, stream=None):
    h = _vp()
    _check(load().spin_state_init(ctypes.byref(cfg), _p(state_mem),
                                  state_mem.numel() * state_mem.element_size(),
                                  _stream(stream), ctypes.byref(h)))
    return h


def spin_state_destroy(h):
    _check(load().spin_state_destroy(h))


def spin_reset_slots(h, slots, request_ids, stream=None):
    _check(load().spin_reset_slots(h, int(slots.numel()), _p(slots), _p(request_ids),
                                   _stream(stream)))


# --------------------------------------------------------------- decode round
def spin_predict_blocks(h, layer, batch, keep_bp, kept_blocks, kept_count, block_flags,
                        stream=None):
    _check(load().spin_predict_blocks(h, int(layer), ctypes.byref(batch), int(keep_bp),
                                      _p(kept_blocks), _p(kept_count), _p(block_flags),
                                      _stream(stream)))


def spin_quantize_q(h, batch, q_bf16, w, stream=None):
    _check(load().spin_quantize_q(h, ctypes.byref(batch), _p(q_bf16), _p(w), _stream(stream)))


def spin_indexer_scores(h, batch, k_pool, k_scale, block_table, kept_blocks, kept_count, scores,
                        page_qmax=None, stream=None):
    _check(load().spin_indexer_scores(h, ctypes.byref(batch), _p(k_pool), _p(k_scale),
                                      int(k_scale.numel()), _p(block_table), _p(kept_blocks),
                                      _p(kept_count), _p(scores), _p(page_qmax), _stream(stream)))


def spin_topk_workspace_bytes(batch, topk):
    n = _sz()
    _check(load().spin_topk_workspace_bytes(ctypes.byref(batch), int(topk), ctypes.byref(n)))
    return n.value


def spin_topk_scores(batch, topk, scores, kept_blocks, kept_count, topk_out, workspace=None,
                     page_qmax=None, stream=None):
    """workspace: a uint8 device tensor of >= spin_topk_workspace_bytes bytes;
    page_qmax: the optional per-page quarter maxima from spin_indexer_scores."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().spin_topk_scores(ctypes.byref(batch), int(topk), _p(scores), _p(page_qmax),
                                   _p(kept_blocks), _p(kept_count), _p(topk_out), _p(workspace),
                                   nbytes, _stream(stream)))


def spin_topk_scores_noalloc(batch, topk, scores, kept_blocks, kept_count, topk_out,
                             page_qmax=None, stream=None):
    """spin_topk_scores with the library's static device scratch (no workspace)."""
    _check(load().spin_topk_scores_noalloc(ctypes.byref(batch), int(topk), _p(scores),
                                           _p(page_qmax), _p(kept_blocks), _p(kept_count),
                                           _p(topk_out), _stream(stream)))


def spin_indexer_topk(h, batch, q_bf16, w, k_pool, k_scale, block_table, kept_blocks,
                      kept_count, scores, topk_out, stream=None):
    _check(load().spin_indexer_topk(h, ctypes.byref(batch), _p(q_bf16), _p(w), _p(k_pool),
                                    _p(k_scale), int(k_scale.numel()), _p(block_table),
                                    _p(kept_blocks), _p(kept_count), _p(scores), _p(topk_out),
                                    _stream(stream)))


def spin_update(h, layer, batch, scores, kept_blocks, kept_count, stream=None):
    _check(load().spin_update(h, int(layer), ctypes.byref(batch), _p(scores), _p(kept_blocks),
                              _p(kept_count), _stream(stream)))


def spin_mtp_replay(h, layer, batch, accepted, scores, kept_blocks, kept_count, stream=None):
    _check(load().spin_mtp_replay(h, int(layer), ctypes.byref(batch), _p(accepted), _p(scores),
                                  _p(kept_blocks), _p(kept_count), _stream(stream)))


def spin_topk_update(h, layer, batch, scores, page_qmax, kept_blocks, kept_count, topk_out,
                     accepted=None, stream=None, update_stream=None):
    """The round's tail: the top-k on `stream` and the EMA update (or the
    prefix-valid replay with `accepted`) behind it, or beside it on
    `update_stream`, ordered by the library's gate."""
    us = None if update_stream is None else ctypes.c_void_p(update_stream.cuda_stream)
    _check(load().spin_topk_update(h, int(layer), ctypes.byref(batch), _p(scores), _p(page_qmax),
                                   _p(kept_blocks), _p(kept_count), _p(topk_out), _p(accepted),
                                   _stream(stream), us))


def spin_measure_miss(batch, topk, full_topk, block_flags, miss, stream=None):
    _check(load().spin_measure_miss(ctypes.byref(batch), int(topk), _p(full_topk),
                                    _p(block_flags), _p(miss), _stream(stream)))


def spin_slot_scores(handle, layer, batch, z_out, stream=None):
    _check(load().spin_slot_scores(handle, int(layer), ctypes.byref(batch), _p(z_out),
                                   _stream(stream)))


def spin_estimate_miss(batch, topk, scores, kept_blocks, kept_count, topk_out, block_flags, est,
                       stream=None):
    _check(load().spin_estimate_miss(ctypes.byref(batch), int(topk), _p(scores), _p(kept_blocks),
                                     _p(kept_count), _p(topk_out), _p(block_flags), _p(est),
                                     _stream(stream)))


def spin_predictor_fidelity(batch, topk, pred, actual, pred_topk, actual_topk, out, stream=None):
    _check(load().spin_predictor_fidelity(ctypes.byref(batch), int(topk), _p(pred), _p(actual),
                                          _p(pred_topk), _p(actual_topk), _p(out),
                                          _stream(stream)))


def spin_attention_workspace_bytes(batch, topk):
    n = _sz()
    _check(load().spin_attention_workspace_bytes(ctypes.byref(batch), int(topk), ctypes.byref(n)))
    return n.value


def spin_sparse_attention(batch, topk, topk_idx, q_bf16, kv_bf16, block_table, scale, out_bf16,
                          lse, workspace=None, stream=None):
    """q_bf16 [B,R,128,576] and kv_bf16 [pages,64,576] bf16 tensors; out_bf16 [B,R,128,512]."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().spin_sparse_attention(ctypes.byref(batch), int(topk), _p(topk_idx), _p(q_bf16),
                                        _p(kv_bf16), int(kv_bf16.shape[0]), _p(block_table),
                                        float(scale), _p(out_bf16), _p(lse), _p(workspace),
                                        ws_bytes, _stream(stream)))


def spin_allocate_budgets(miss, mean_keep_bp):
    L = len(miss)
    arr = (ctypes.c_double * L)(*[float(m) for m in miss])
    out = (ctypes.c_int32 * L)()
    _check(load().spin_allocate_budgets(L, arr, int(mean_keep_bp), out))
    return [int(x) for x in out]


def spin_allocate_budgets_curve(miss_curve, grid_bp, mean_keep_bp):
    """miss_curve: L rows of G mean miss rates, one per keep of grid_bp."""
    L, G = len(miss_curve), len(grid_bp)
    flat = [float(m) for row in miss_curve for m in row]
    if len(flat) != L * G:
        raise SpinError(SPIN_EINVAL, "miss_curve rows must have one value per grid keep")
    arr = (ctypes.c_double * (L * G))(*flat)
    grid = (ctypes.c_int32 * G)(*[int(g) for g in grid_bp])
    out = (ctypes.c_int32 * L)()
    _check(load().spin_allocate_budgets_curve(L, G, arr, grid, int(mean_keep_bp), out))
    return [int(x) for x in out]


class SpinState:
    """A state buffer allocated with torch on `device` and bound to the library."""

    def __init__(self, cfg, device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.layout = spin_state_layout_of(cfg)
        self.mem = torch.empty(self.layout["total"], dtype=torch.uint8, device=device)
        self.handle = spin_state_init(cfg, self.mem, stream)

    def region(self, name, dtype, shape):
        """A torch view of one state region (see spin_state_layout in spin.h)."""
        import torch
        off = self.layout[name]
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty(0, dtype=dtype).element_size()
        return self.mem[off:off + nbytes].view(dtype).view(*shape)

    def V(self):
        c = self.cfg
        import torch
        return self.region("V", torch.float32, (c.num_layers, c.max_slots, c.max_ctx))

    def D(self):
        c = self.cfg
        import torch
        return self.region("D", torch.float32, (c.num_layers, c.max_slots, c.max_ctx))

    def VB(self):
        c = self.cfg
        import torch
        return self.region("VB", torch.float32, (c.num_layers, c.max_slots, self.layout["max_blocks"]))

    def step(self):
        c = self.cfg
        import torch
        return self.region("step", torch.int32, (c.num_layers, c.max_slots))

    def error(self):
        import torch
        return int(self.region("error", torch.int32, (1,)).item())

    def close(self):
        if self.handle is not None:
            spin_state_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
