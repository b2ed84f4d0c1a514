"""Thin Python binding over liboscar (argument marshalling only).

Every function turns torch tensors into pointers and sizes and calls the C
entry point of the same name; all computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import MAX_HEAD_ROTATIONS, LayerCacheC, RotationC, check, load

HEAD_DIM = 128
PAGE = 16
N_SINK = 16
N_RECENT = 128
BF16_PAGES_PER_REQ = 9


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtypes, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def hist_block_bytes(group: int, code_bits: int = 2) -> int:
    return int(load().oscar_hist_block_bytes_bits(group, code_bits))


def rotation_bytes() -> int:
    return int(load().oscar_rotation_bytes())


class Rotation:
    """Device forms of a fixed rotation and its clip threshold, built by
    oscar_prepare_rotation: one per-layer R (fp64 [128, 128], x_rot = x R)
    with a scalar clip, or one R per KV head ([Hkv, 128, 128], Hkv <= 32)
    with a clip per head (the optional per-head extension)."""

    def __init__(self, R, clip, device: torch.device | str = "cuda"):
        device = torch.device(device)
        R64 = torch.as_tensor(R, dtype=torch.float64)
        per_head = R64.dim() == 3
        if (R64.dim() not in (2, 3)) or tuple(R64.shape[-2:]) != (HEAD_DIM, HEAD_DIM):
            raise ValueError("R must be [128, 128] or [Hkv, 128, 128]")
        self.R64 = R64.to(device).contiguous()
        self.n_heads = int(R64.shape[0]) if per_head else 0
        if per_head:
            clips = [float(c) for c in clip]
            if len(clips) != self.n_heads or not 1 <= self.n_heads <= MAX_HEAD_ROTATIONS:
                raise ValueError("per-head rotations: one clip per head, at most 32 heads")
            self._clips = (ctypes.c_float * self.n_heads)(*clips)
            self.clip = max(clips)
        else:
            self._clips = None
            self.clip = float(clip)
        nb = rotation_bytes()
        self.forms = torch.empty(max(self.n_heads, 1) * nb, dtype=torch.uint8, device=device)
        lib = load()
        for h in range(max(self.n_heads, 1)):
            Rh = self.R64[h] if per_head else self.R64
            check(lib.oscar_prepare_rotation(_ptr(Rh), self.forms.data_ptr() + h * nb, _stream(device)))

    def c(self) -> RotationC:
        if self.n_heads:
            return RotationC(self.forms.data_ptr(), self.clip, self.n_heads,
                             ctypes.cast(self._clips, ctypes.POINTER(ctypes.c_float)))
        return RotationC(self.forms.data_ptr(), self.clip, 0, None)


class LayerCache:
    """One layer's paged cache in the formats of include/oscar.h.

    hist:   uint8 [n_hist_pages, Hkv, hist_block_bytes(group, code_bits)]
    bf16:   bfloat16 [n_bf16_pages, Hkv, 2, 16, 128]
    hist_pt int32 [B, stride], bf16_pt int32 [B, 9], status int32 [1].
    code_bits: 2 (INT2 history) or 4 (INT4).
    """

    def __init__(self, n_kv_heads: int, group: int, n_hist_pages: int, n_bf16_pages: int,
                 hist_pt: torch.Tensor, bf16_pt: torch.Tensor, device="cuda",
                 hist: torch.Tensor | None = None, bf16: torch.Tensor | None = None, code_bits: int = 2):
        device = torch.device(device)
        self.device = device
        self.n_kv_heads, self.group, self.code_bits = int(n_kv_heads), int(group), int(code_bits)
        blk = hist_block_bytes(group, code_bits)
        if blk == 0:
            raise ValueError(f"unsupported group {group} / code_bits {code_bits}")
        if hist is not None and (hist.dim() != 3 or hist.shape[2] != blk):
            raise ValueError(f"hist must be [pages, Hkv, {blk}]")
        self.hist = hist if hist is not None else torch.zeros(
            (max(n_hist_pages, 0), n_kv_heads, blk), dtype=torch.uint8, device=device)
        self.bf16 = bf16 if bf16 is not None else torch.zeros(
            (n_bf16_pages, n_kv_heads, 2, PAGE, HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.hist_pt = torch.as_tensor(hist_pt, dtype=torch.int32).to(device).contiguous()
        self.bf16_pt = torch.as_tensor(bf16_pt, dtype=torch.int32).to(device).contiguous()
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        _need(self.hist, "hist", (torch.uint8,), device)
        _need(self.bf16, "bf16", (torch.bfloat16, torch.int16), device)

    def c(self) -> LayerCacheC:
        return LayerCacheC(self.n_kv_heads, self.group, self.hist.data_ptr(), self.hist.shape[0],
                           self.bf16.data_ptr(), self.bf16.shape[0], self.hist_pt.data_ptr(),
                           self.hist_pt.shape[1], self.bf16_pt.data_ptr(), self.status.data_ptr(),
                           self.code_bits)


def write_kv(cache: LayerCache, rot_k: Rotation, rot_v: Rotation, k_new: torch.Tensor,
             v_new: torch.Tensor, cu_new: torch.Tensor, len_before: torch.Tensor, max_new: int) -> None:
    """oscar_write_kv: append rows cu_new[b]..cu_new[b+1]-1 of k_new / v_new
    (bf16 [T, Hkv, 128]) to request b at positions len_before[b]... ."""
    dev = cache.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, (torch.bfloat16,), dev)
    _need(cu_new, "cu_new", (torch.int32,), dev)
    _need(len_before, "len_before", (torch.int32,), dev)
    batch = len_before.shape[0]
    if cu_new.shape[0] != batch + 1:
        raise ValueError("cu_new must have batch + 1 entries")
    c = cache.c()
    rk, rv = rot_k.c(), rot_v.c()
    check(load().oscar_write_kv(ctypes.byref(c), ctypes.byref(rk), ctypes.byref(rv), _ptr(k_new),
                                _ptr(v_new), _ptr(cu_new), _ptr(len_before), batch, k_new.shape[0],
                                int(max_new), _stream(dev)))


def decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int) -> int:
    return int(load().oscar_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, max_seq_len))


def decode_attn(cache: LayerCache, rot_k: Rotation, rot_v: Rotation, q: torch.Tensor,
                seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float | None = None,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """oscar_decode_attn: q bf16 [B, Hq, 128] -> out fp32 [B, Hq, 128]."""
    dev = cache.device
    _need(q, "q", (torch.bfloat16,), dev)
    _need(seq_lens, "seq_lens", (torch.int32,), dev)
    batch, hq = q.shape[0], q.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((batch, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), dev)
    need = decode_workspace_bytes(batch, hq, cache.n_kv_heads, max_seq_len)
    if workspace is None:  # zero-filled: it holds the merge counters
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    c = cache.c()
    rk, rv = rot_k.c(), rot_v.c()
    check(load().oscar_decode_attn(ctypes.byref(c), ctypes.byref(rk), ctypes.byref(rv), _ptr(q), hq,
                                   _ptr(seq_lens), batch, int(max_seq_len), float(sm_scale), _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def decode_attn_noalloc(cache: LayerCache, rot_k: Rotation, rot_v: Rotation, q: torch.Tensor,
                        seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float | None = None,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """oscar_decode_attn_noalloc: oscar_decode_attn on the library's own
    per-GPU scratch (no workspace, no allocation in the call)."""
    dev = cache.device
    _need(q, "q", (torch.bfloat16,), dev)
    _need(seq_lens, "seq_lens", (torch.int32,), dev)
    batch, hq = q.shape[0], q.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((batch, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), dev)
    c = cache.c()
    rk, rv = rot_k.c(), rot_v.c()
    check(load().oscar_decode_attn_noalloc(ctypes.byref(c), ctypes.byref(rk), ctypes.byref(rv), _ptr(q), hq,
                                           _ptr(seq_lens), batch, int(max_seq_len), float(sm_scale), _ptr(out),
                                           _stream(dev)))
    return out


def decode_step(cache: LayerCache, rot_k: Rotation, rot_v: Rotation, k_new: torch.Tensor,
                v_new: torch.Tensor, len_before: torch.Tensor, q: torch.Tensor, max_seq_len: int,
                sm_scale: float | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """oscar_decode_step: append k_new / v_new (bf16 [B, Hkv, 128]) at positions
    len_before, then decode q (bf16 [B, Hq, 128]) over len_before + 1 tokens."""
    dev = cache.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (q, "q")):
        _need(t, n, (torch.bfloat16,), dev)
    _need(len_before, "len_before", (torch.int32,), dev)
    batch, hq = q.shape[0], q.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((batch, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), dev)
    need = decode_workspace_bytes(batch, hq, cache.n_kv_heads, max_seq_len)
    if workspace is None:  # zero-filled: it holds the merge counters
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    c = cache.c()
    rk, rv = rot_k.c(), rot_v.c()
    check(load().oscar_decode_step(ctypes.byref(c), ctypes.byref(rk), ctypes.byref(rv), _ptr(k_new), _ptr(v_new),
                                   _ptr(len_before), _ptr(q), hq, batch, int(max_seq_len), float(sm_scale),
                                   _ptr(out), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def extend_attn(cache: LayerCache, rot_k: Rotation, rot_v: Rotation, q: torch.Tensor, k_new: torch.Tensor,
                v_new: torch.Tensor, cu_new: torch.Tensor, len_before: torch.Tensor, max_new: int,
                max_prefix: int, sm_scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """oscar_extend_attn: new tokens (rows cu_new[b]..cu_new[b+1]-1 of q bf16
    [T, Hq, 128], k_new / v_new bf16 [T, Hkv, 128]) attend to request b's
    cached prefix of len_before[b] tokens and causally to each other; the
    chunk is not written.  Returns out fp32 [T, Hq, 128]."""
    dev = cache.device
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, (torch.bfloat16,), dev)
    _need(cu_new, "cu_new", (torch.int32,), dev)
    _need(len_before, "len_before", (torch.int32,), dev)
    batch, hq = len_before.shape[0], q.shape[1]
    if cu_new.shape[0] != batch + 1:
        raise ValueError("cu_new must have batch + 1 entries")
    T = q.shape[0]
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [T, Hq, {HEAD_DIM}]")
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        if tuple(t.shape) != (T, cache.n_kv_heads, HEAD_DIM):
            raise ValueError(f"{n} must be [{T}, {cache.n_kv_heads}, {HEAD_DIM}], got {tuple(t.shape)}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((T, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), dev)
    if tuple(out.shape) != (T, hq, HEAD_DIM):
        raise ValueError(f"out must be [{T}, {hq}, {HEAD_DIM}], got {tuple(out.shape)}")
    c = cache.c()
    rk, rv = rot_k.c(), rot_v.c()
    check(load().oscar_extend_attn(ctypes.byref(c), ctypes.byref(rk), ctypes.byref(rv), _ptr(q), hq, _ptr(k_new),
                                   _ptr(v_new), _ptr(cu_new), _ptr(len_before), batch, q.shape[0], int(max_new),
                                   int(max_prefix), float(sm_scale), _ptr(out), _stream(dev)))
    return out


def bf16_decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int) -> int:
    return int(load().oscar_bf16_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, max_seq_len))


def bf16_paged_decode(q: torch.Tensor, kv_pages: torch.Tensor, pt: torch.Tensor, seq_lens: torch.Tensor,
                      max_seq_len: int, sm_scale: float | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None,
                      status: torch.Tensor | None = None) -> torch.Tensor:
    """oscar_bf16_paged_decode over kv_pages bf16 [pages, Hkv, 2, 16, 128]."""
    dev = q.device
    _need(q, "q", (torch.bfloat16,), dev)
    _need(kv_pages, "kv_pages", (torch.bfloat16,), dev)
    _need(pt, "pt", (torch.int32,), dev)
    _need(seq_lens, "seq_lens", (torch.int32,), dev)
    batch, hq = q.shape[0], q.shape[1]
    hkv = kv_pages.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((batch, hq, HEAD_DIM), dtype=torch.float32, device=dev)
    need = bf16_decode_workspace_bytes(batch, hq, hkv, max_seq_len)
    if workspace is None:  # zero-filled: it holds the merge counters
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    check(load().oscar_bf16_paged_decode(_ptr(q), _ptr(kv_pages), kv_pages.shape[0], _ptr(pt), pt.shape[1],
                                         _ptr(seq_lens), batch, int(max_seq_len), hq, hkv, float(sm_scale),
                                         _ptr(out), _ptr(status), _ptr(workspace), workspace.numel(),
                                         _stream(dev)))
    return out


def profile_events(before: "torch.cuda.Event | None", after: "torch.cuda.Event | None") -> None:
    """The next decode call on this thread records `before` / `after` around
    its split-K attention kernel, the next write call around its history
    write kernel (oscar_profile_events).  Events must have
    been recorded once (torch creates them lazily)."""
    h0 = ctypes.c_void_p(before.cuda_event) if before is not None else ctypes.c_void_p(None)
    h1 = ctypes.c_void_p(after.cuda_event) if after is not None else ctypes.c_void_p(None)
    check(load().oscar_profile_events(h0, h1))


def read_probe(buf: torch.Tensor, n_blocks: int, block_bytes: int, ids: torch.Tensor | None = None,
               sink: torch.Tensor | None = None) -> torch.Tensor:
    """oscar_read_probe: reads n_blocks blocks of block_bytes bytes of buf
    (slot ids[i], or slot i without ids) and adds their 32-bit words mod 2^32
    into sink (int32 [1] on the device, returned)."""
    dev = buf.device
    _need(buf, "buf", (torch.uint8,), dev)
    if ids is not None:
        _need(ids, "ids", (torch.int32,), dev)
        if ids.numel() < n_blocks:
            raise ValueError("ids holds fewer than n_blocks entries")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(sink, "sink", (torch.int32,), dev)
    check(load().oscar_read_probe(_ptr(buf), buf.numel(), int(n_blocks), int(block_bytes), _ptr(ids), _ptr(sink),
                                  _stream(dev)))
    return sink


def calib_accumulate(q_cal: torch.Tensor, k_cal: torch.Tensor, v_cal: torch.Tensor, sums: torch.Tensor) -> int:
    """oscar_calib_accumulate: adds one calibration sequence's moment sums to
    sums (float64 [2, 128, 128] on the device); returns n_tokens * Hq, the
    caller's count increment."""
    dev = q_cal.device
    for t, n in ((q_cal, "q_cal"), (k_cal, "k_cal"), (v_cal, "v_cal")):
        _need(t, n, (torch.bfloat16,), dev)
    _need(sums, "sums", (torch.float64,), dev)
    if tuple(sums.shape) != (2, HEAD_DIM, HEAD_DIM):
        raise ValueError("sums must be [2, 128, 128]")
    n = int(load().oscar_calib_accumulate_workspace_bytes(q_cal.shape[0], q_cal.shape[1], k_cal.shape[1]))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    check(load().oscar_calib_accumulate(_ptr(q_cal), _ptr(k_cal), _ptr(v_cal), q_cal.shape[0], q_cal.shape[1],
                                        k_cal.shape[1], _ptr(sums), _ptr(ws), ws.numel(), _stream(dev)))
    return int(q_cal.shape[0] * q_cal.shape[1])


def calib_accumulate_heads(q_cal: torch.Tensor, k_cal: torch.Tensor, v_cal: torch.Tensor,
                           sums: torch.Tensor) -> int:
    """oscar_calib_accumulate_heads: adds one calibration sequence's per-KV-head
    moment sums to sums (float64 [Hkv, 2, 128, 128] on the device); returns
    n_tokens * Hq/Hkv, each head's count increment."""
    dev = q_cal.device
    for t, n in ((q_cal, "q_cal"), (k_cal, "k_cal"), (v_cal, "v_cal")):
        _need(t, n, (torch.bfloat16,), dev)
    _need(sums, "sums", (torch.float64,), dev)
    hkv = k_cal.shape[1]
    if tuple(sums.shape) != (hkv, 2, HEAD_DIM, HEAD_DIM):
        raise ValueError("sums must be [Hkv, 2, 128, 128]")
    n = int(load().oscar_calib_accumulate_workspace_bytes(q_cal.shape[0], q_cal.shape[1], hkv))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    check(load().oscar_calib_accumulate_heads(_ptr(q_cal), _ptr(k_cal), _ptr(v_cal), q_cal.shape[0],
                                              q_cal.shape[1], hkv, _ptr(sums), _ptr(ws), ws.numel(),
                                              _stream(dev)))
    return int(q_cal.shape[0] * (q_cal.shape[1] // hkv))


def calibrate_per_head(q_cal: torch.Tensor, k_cal: torch.Tensor, v_cal: torch.Tensor,
                       clip_quantile: float = 0.999):
    """Per-KV-head calibration of one sequence (the optional per-head
    extension): per-head moments, then each head's R_K, R_V
    (oscar_calib_rotations) and clips over its own K and V vectors
    (oscar_clip_threshold).  Returns R_K, R_V float64 CPU [Hkv, 128, 128] and
    clip lists [Hkv]."""
    hkv = k_cal.shape[1]
    sums = torch.zeros((hkv, 2, HEAD_DIM, HEAD_DIM), dtype=torch.float64, device=q_cal.device)
    count = calib_accumulate_heads(q_cal, k_cal, v_cal, sums)
    RK, RV, ck, cv = [], [], [], []
    for h in range(hkv):
        rk, rv = calib_rotations(sums[h], count)
        RK.append(rk)
        RV.append(rv)
        ck.append(clip_threshold(k_cal[:, h].contiguous(), rk, clip_quantile))
        cv.append(clip_threshold(v_cal[:, h].contiguous(), rv, clip_quantile))
    return torch.stack(RK), torch.stack(RV), ck, cv


def calib_rotations(sums: torch.Tensor, count: float):
    """oscar_calib_rotations: (R_K, R_V) float64 CPU tensors [128, 128] from
    accumulated moment sums and their count."""
    dev = sums.device
    _need(sums, "sums", (torch.float64,), dev)
    R_K = torch.empty((HEAD_DIM, HEAD_DIM), dtype=torch.float64)
    R_V = torch.empty((HEAD_DIM, HEAD_DIM), dtype=torch.float64)
    ws = torch.empty(int(load().oscar_calib_rotations_workspace_bytes()), dtype=torch.uint8, device=dev)
    check(load().oscar_calib_rotations(_ptr(sums), float(count), _ptr(R_K), _ptr(R_V), _ptr(ws), ws.numel(),
                                       _stream(dev)))
    return R_K, R_V


def clip_threshold(x_cal: torch.Tensor, R: torch.Tensor, clip_quantile: float = 0.999) -> float:
    """oscar_clip_threshold: the clip of a caller-chosen rotation R (float64
    CPU [128, 128]) from bf16 calibration vectors [..., 128] on the device."""
    dev = x_cal.device
    _need(x_cal, "x_cal", (torch.bfloat16,), dev)
    R = R.detach().to(torch.float64).contiguous().cpu()
    if R.shape != (HEAD_DIM, HEAD_DIM):
        raise ValueError("R must be [128, 128]")
    out = ctypes.c_float(0)
    n_vec = x_cal.numel() // HEAD_DIM
    ws = torch.empty(max(int(load().oscar_clip_threshold_workspace_bytes(n_vec)), 1), dtype=torch.uint8, device=dev)
    check(load().oscar_clip_threshold(_ptr(x_cal), n_vec, _ptr(R), float(clip_quantile),
                                      ctypes.byref(out), _ptr(ws), ws.numel(), _stream(dev)))
    return out.value


def calibrate_rotation(q_cal: torch.Tensor, k_cal: torch.Tensor, v_cal: torch.Tensor,
                       clip_quantile: float = 0.999):
    """oscar_calibrate_rotation: bf16 [N, Hq, 128], [N, Hkv, 128] x2 on the device ->
    (R_K, R_V) float64 CPU tensors [128, 128] and (clip_K, clip_V) floats."""
    dev = q_cal.device
    for t, n in ((q_cal, "q_cal"), (k_cal, "k_cal"), (v_cal, "v_cal")):
        _need(t, n, (torch.bfloat16,), dev)
    R_K = torch.empty((HEAD_DIM, HEAD_DIM), dtype=torch.float64)
    R_V = torch.empty((HEAD_DIM, HEAD_DIM), dtype=torch.float64)
    ck, cv = ctypes.c_float(0), ctypes.c_float(0)
    n = int(load().oscar_calibrate_workspace_bytes(q_cal.shape[0], q_cal.shape[1], k_cal.shape[1]))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    check(load().oscar_calibrate_rotation(_ptr(q_cal), _ptr(k_cal), _ptr(v_cal), q_cal.shape[0],
                                          q_cal.shape[1], k_cal.shape[1], float(clip_quantile),
                                          _ptr(R_K), _ptr(R_V), ctypes.byref(ck), ctypes.byref(cv),
                                          _ptr(ws), ws.numel(), _stream(dev)))
    return R_K, R_V, ck.value, cv.value
