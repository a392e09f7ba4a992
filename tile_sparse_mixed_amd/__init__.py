"""tile_sparse_mixed_amd: three-tier tile-sparse attention on MI355X (gfx950).

Thin Python binding over the C ABI of ``libtattn.so`` (``include/tattn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only marshals torch tensors (device memory) and the current HIP stream into
the C calls.  There is no fallback: if the library is missing, importing the
binding's entry points raises.

    plan = tattn.plan(q, k, v, block_q=128, block_k=64, tau_hi=0.01, tau_lo=0.001)
    out = tattn.forward(plan, q, k, v)
"""
import ctypes
import os

import numpy as np

__all__ = ["plan", "replan", "forward", "forward_dump", "list_bound", "attention_static", "Plan", "TattnError", "load_library",
           "Config", "Stats",
           "MODE_THRESHOLD", "MODE_ADAPTIVE", "MODE_ALL_FULL", "MODE_EXTERNAL", "MODE_PRICE",
           "SKIP", "LOW", "FULL", "SKIM"]

MODE_THRESHOLD, MODE_ADAPTIVE, MODE_ALL_FULL, MODE_EXTERNAL, MODE_PRICE = 0, 1, 2, 3, 4
SKIP, LOW, FULL, SKIM = 0, 1, 2, 3
_MODES = {"threshold": MODE_THRESHOLD, "adaptive": MODE_ADAPTIVE, "all_full": MODE_ALL_FULL,
          "external": MODE_EXTERNAL, "price": MODE_PRICE}
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtattn.so")
_lib = None


class TattnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"tattn error {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("tau_hi", ctypes.c_float), ("tau_lo", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("keep_min", ctypes.c_float), ("keep_max", ctypes.c_float),
                ("full_frac", ctypes.c_float), ("entropy_samples", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
                ("price", ctypes.c_float), ("tau_skim", ctypes.c_float), ("low_refine", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("n_full", ctypes.c_int64), ("n_low", ctypes.c_int64), ("n_skip", ctypes.c_int64),
                ("n_diag", ctypes.c_int64), ("flops_bf16", ctypes.c_double), ("flops_fp8", ctypes.c_double),
                ("flops_dense", ctypes.c_double), ("n_skim", ctypes.c_int64), ("flops_fp4", ctypes.c_double)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_VP = ctypes.c_void_p
_SIGS = {
    "tattn_validate": (ctypes.c_int, [ctypes.POINTER(Config)]),
    "tattn_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_size_t)]),
    "tattn_plan": (ctypes.c_int, [ctypes.POINTER(Config), _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP,
                                  ctypes.POINTER(_VP)]),
    "tattn_forward": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP]),
    "tattn_forward_dump": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int32, _VP, _VP]),
    "tattn_list_bound": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_int32)]),
    "tattn_attention_static": (ctypes.c_int, [ctypes.POINTER(Config), _VP, _VP, _VP, _VP, _VP]),
    "tattn_replan": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP]),
    "tattn_plan_set_tiers": (ctypes.c_int, [_VP, _VP, _VP]),
    "tattn_plan_get_tiers": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "tattn_plan_get_lists": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "tattn_plan_get_pool": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "tattn_plan_get_codes": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "tattn_plan_get_mx4": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "tattn_plan_get_mx4_residual": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "tattn_plan_stats": (ctypes.c_int, [_VP, ctypes.POINTER(Stats)]),
    "tattn_plan_get_kh": (ctypes.c_int, [_VP, _VP, _VP]),
    "tattn_plan_get_moments": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "tattn_plan_destroy": (None, [_VP]),
    "tattn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "tattn_last_error": (ctypes.c_char_p, []),
}


def load_library(path: str = _LIB_PATH):
    """Load libtattn.so (built in-tree by ``python -m tile_sparse_mixed_amd.build``)."""
    global _lib
    if _lib is not None and path == _LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m tile_sparse_mixed_amd.build` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _check(status):
    if status != 0:
        lib = load_library()
        raise TattnError(status, lib.tattn_last_error().decode() or lib.tattn_status_str(status).decode())


def make_config(batch, heads, seq_len, head_dim, block_q, block_k, tau_hi=0.0, tau_lo=0.0, top_k=0,
                mode="threshold", keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256,
                out_fp32=False, strides=None, price=0.0, tau_skim=0.0, low_refine=False):
    if strides is None:
        strides = (heads * seq_len * head_dim, seq_len * head_dim, head_dim)
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    return Config(batch, heads, seq_len, head_dim, block_q, block_k, float(tau_hi), float(tau_lo), int(top_k), m,
                  float(keep_min), float(keep_max), float(full_frac), int(entropy_samples), 0,
                  1 if out_fp32 else 0, *[int(s) for s in strides], float(price), float(tau_skim),
                  1 if low_refine else 0)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Plan:
    """A routed plan: owns the device workspace (a torch uint8 tensor) and the
    host handle; keeps references to the K and V tensors it was built from."""

    def __init__(self, cfg: Config, q, k, v, workspace=None):
        import torch
        lib = load_library()
        self.cfg = cfg
        nbytes = ctypes.c_size_t(0)
        _check(lib.tattn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(nbytes)))
        need = int(nbytes.value) + 256
        if workspace is not None and workspace.numel() >= need and workspace.dtype == torch.uint8:
            self.workspace = workspace          # reuse: a plan overwrites every region it reads
        else:
            self.workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        base = self.workspace.data_ptr()
        self._ws_ptr = (base + 255) // 256 * 256
        self._k, self._v = k, v
        self._handle = _VP()
        self.n_q = -(-cfg.seq_len // cfg.block_q)
        self.n_k = -(-cfg.seq_len // cfg.block_k)
        _check(lib.tattn_plan(ctypes.byref(cfg), q.data_ptr(), k.data_ptr(), v.data_ptr(), self._ws_ptr,
                              int(nbytes.value), _stream(), ctypes.byref(self._handle)))

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h and _lib is not None:
            _lib.tattn_plan_destroy(h)
            self._handle = None

    @property
    def handle(self):
        return self._handle

    def _shape(self, *tail):
        return (self.cfg.batch, self.cfg.heads) + tail

    def set_tiers(self, tiers: np.ndarray):
        t = np.ascontiguousarray(tiers, dtype=np.uint8).reshape(self._shape(self.n_q, self.n_k))
        _check(load_library().tattn_plan_set_tiers(self._handle, t.ctypes.data, _stream()))

    def tiers(self, with_p=False):
        t = np.empty(self._shape(self.n_q, self.n_k), np.uint8)
        p = np.empty(self._shape(self.n_q, self.n_k), np.float32) if with_p else None
        _check(load_library().tattn_plan_get_tiers(self._handle, t.ctypes.data,
                                                   p.ctypes.data if with_p else None, _stream()))
        return (t, p) if with_p else t

    def lists(self):
        li = np.empty(self._shape(self.n_q, self.n_k), np.int16)
        c = np.empty(self._shape(self.n_q, 3), np.int32)
        _check(load_library().tattn_plan_get_lists(self._handle, li.ctypes.data, c.ctypes.data, _stream()))
        return li, c

    def pool(self):
        d = self.cfg.head_dim
        out = dict(qbar=np.empty(self._shape(self.n_q, d), np.float32),
                   kbar=np.empty(self._shape(self.n_k, d), np.float32),
                   vbar=np.empty(self._shape(self.n_k, d), np.float32),
                   sq=np.empty(self._shape(self.n_q), np.float32),
                   sk=np.empty(self._shape(self.n_k), np.float32),
                   sv=np.empty(self._shape(self.n_k), np.float32))
        _check(load_library().tattn_plan_get_pool(self._handle, *[out[k].ctypes.data for k in
                                                                  ("qbar", "kbar", "vbar", "sq", "sk", "sv")],
                                                  _stream()))
        return out

    def codes(self):
        """E4M3 codes of K and of V as uint8, both [B, H, N, d]."""
        k8 = np.empty(self._shape(self.cfg.seq_len, self.cfg.head_dim), np.uint8)
        v8 = np.empty(k8.shape, np.uint8)
        _check(load_library().tattn_plan_get_codes(self._handle, k8.ctypes.data, v8.ctypes.data, _stream()))
        return k8, v8

    def mx4(self):
        """SKIM tier: the MXFP4 copy of K (codes, two per byte, [B, H, N,
        d/2] uint8; E8M0 scale bytes [B, H, N, d/32])."""
        n, d = self.cfg.seq_len, self.cfg.head_dim
        k4 = np.empty(self._shape(n, d // 2), np.uint8)
        k4s = np.empty(self._shape(n, d // 32), np.uint8)
        _check(load_library().tattn_plan_get_mx4(self._handle, k4.ctypes.data, k4s.ctypes.data, _stream()))
        return dict(k4=k4, k4s=k4s)

    def mx4_residual(self):
        """Refined low tier: the MXFP4 copy of K's rounding residual (layouts
        as mx4())."""
        n, d = self.cfg.seq_len, self.cfg.head_dim
        k4r = np.empty(self._shape(n, d // 2), np.uint8)
        k4rs = np.empty(self._shape(n, d // 32), np.uint8)
        _check(load_library().tattn_plan_get_mx4_residual(self._handle, k4r.ctypes.data, k4rs.ctypes.data,
                                                          _stream()))
        return dict(k4r=k4r, k4rs=k4rs)

    def stats(self) -> dict:
        st = Stats()
        _check(load_library().tattn_plan_stats(self._handle, ctypes.byref(st)))
        return st.as_dict()

    def moments(self):
        """Price mode: the block second moments the router used (float32)."""
        d = self.cfg.head_dim
        out = dict(q2=np.empty(self._shape(self.n_q, d), np.float32), m2q=np.empty(self._shape(self.n_q), np.float32),
                   kvar=np.empty(self._shape(self.n_k, d), np.float32), m2k=np.empty(self._shape(self.n_k), np.float32),
                   vvar=np.empty(self._shape(self.n_k), np.float32), m2v=np.empty(self._shape(self.n_k), np.float32),
                   vnorm=np.empty(self._shape(self.n_k), np.float32))
        _check(load_library().tattn_plan_get_moments(self._handle, *[out[k].ctypes.data for k in
                                                                     ("q2", "m2q", "kvar", "m2k", "vvar", "m2v",
                                                                      "vnorm")], _stream()))
        return out

    def kh(self):
        bh = self.cfg.batch * self.cfg.heads
        kh = np.empty(bh, np.int32)
        rh = np.empty(bh, np.float64)
        _check(load_library().tattn_plan_get_kh(self._handle, kh.ctypes.data, rh.ctypes.data))
        return kh, rh


def _check_tensors(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be [B, H, N, d] with d contiguous")
    if not (q.shape == k.shape == v.shape and q.stride() == k.stride() == v.stride()):
        raise ValueError("q, k, v must share shape and strides")


def plan(q, k, v, block_q=128, block_k=64, tau_hi=0.01, tau_lo=0.001, top_k=0, mode="threshold",
         keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256, out_fp32=False,
         workspace=None, price=0.0, tau_skim=0.0, low_refine=False) -> Plan:
    """Pool, quantise and route (K1, K2).  q, k, v: bf16 [B, H, N, d] on the GPU.
    ``tau_skim`` > 0 adds the MXFP4 SKIM tier (every mode but all-full, every
    key-block size).  ``low_refine`` scores LOW tiles on MXFP4 copies with
    residual correction instead of E4M3 (no SKIM tier).
    ``workspace`` (a uint8 GPU tensor, e.g. an earlier
    plan's) is reused when large enough; the earlier plan must not be used
    afterwards."""
    _check_tensors(q, k, v)
    B, H, N, d = q.shape
    cfg = make_config(B, H, N, d, block_q, block_k, tau_hi, tau_lo, top_k, mode, keep_min, keep_max,
                      full_frac, entropy_samples, out_fp32, strides=q.stride()[:3], price=price,
                      tau_skim=tau_skim, low_refine=low_refine)
    return Plan(cfg, q, k, v, workspace=workspace)


def replan(p: Plan, q, k, v) -> Plan:
    """Reuse ``p``'s tiers for the next diffusion step: recompute the block
    means and fp8 copies from q, k, v (same shape and strides) without
    re-routing.  Returns ``p``, now bound to these k and v."""
    _check_tensors(q, k, v)
    if tuple(q.shape) != p._shape(p.cfg.seq_len, p.cfg.head_dim) or \
            tuple(q.stride()[:3]) != (p.cfg.stride_b, p.cfg.stride_h, p.cfg.stride_n):
        raise ValueError("replan needs tensors of the plan's shape and strides")
    _check(load_library().tattn_replan(p.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), _stream()))
    p._k, p._v = k, v
    return p


def list_bound(cfg: Config) -> int:
    """The most kept tiles a query block can hold under cfg's tier rule
    (host only: no device needed)."""
    b = ctypes.c_int32(0)
    _check(load_library().tattn_list_bound(ctypes.byref(cfg), ctypes.byref(b)))
    return int(b.value)


def _out_like(p, q, out):
    import torch
    dt = torch.float32 if p.cfg.out_dtype == 1 else torch.bfloat16
    if out is None:
        return torch.empty_strided(q.shape, q.stride(), dtype=dt, device=q.device)
    if out.dtype != dt or out.stride() != q.stride() or out.shape != q.shape:
        raise ValueError("out must match q's shape and strides and the plan's output dtype")
    return out


def forward_dump(p: Plan, q, k, v, rows, steps, out=None):
    """The fused pass, also returning the probability codes of the LOW and
    SKIM steps of the query blocks ``rows`` (a list of (b, h, I)): a uint8
    array [len(rows), steps, block_q, 64] (byte layout as tattn_forward_dump
    documents; steps past a row's count are zero)."""
    import torch
    _check_tensors(q, k, v)
    out = _out_like(p, q, out)
    slot = torch.full((p.cfg.batch * p.cfg.heads * p.n_q,), -1, dtype=torch.int32)
    for i, (b, h, I) in enumerate(rows):
        slot[(b * p.cfg.heads + h) * p.n_q + I] = i
    slot = slot.to(q.device)
    dump = torch.zeros((max(1, len(rows)), int(steps), p.cfg.block_q, 64), dtype=torch.uint8, device=q.device)
    _check(load_library().tattn_forward_dump(p.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                             slot.data_ptr(), int(steps), dump.data_ptr(), _stream()))
    return out, dump.cpu().numpy()[:len(rows)]


def attention_static(q, k, v, block_q=128, block_k=64, tau_hi=0.01, tau_lo=0.001, top_k=0, mode="threshold",
                     keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256, out_fp32=False, price=0.0,
                     tau_skim=0.0, out=None, low_refine=False):
    """Plan and forward in one call with the library's static workspace (no
    device allocation inside the call; ``out`` may be preallocated).
    Problems whose workspace exceeds 64 MiB raise."""
    import torch
    _check_tensors(q, k, v)
    B, H, N, d = q.shape
    cfg = make_config(B, H, N, d, block_q, block_k, tau_hi, tau_lo, top_k, mode, keep_min, keep_max,
                      full_frac, entropy_samples, out_fp32, strides=q.stride()[:3], price=price, tau_skim=tau_skim,
                      low_refine=low_refine)
    dt = torch.float32 if out_fp32 else torch.bfloat16
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=dt, device=q.device)
    elif out.dtype != dt or out.stride() != q.stride() or out.shape != q.shape:
        raise ValueError("out must match q's shape and strides and the output dtype")
    _check(load_library().tattn_attention_static(ctypes.byref(cfg), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 out.data_ptr(), _stream()))
    return out


def forward(p: Plan, q, k, v, out=None):
    """The fused three-tier pass (K3).  Returns O [B, H, N, d] (bf16, or fp32
    if the plan was made with out_fp32=True)."""
    _check_tensors(q, k, v)
    out = _out_like(p, q, out)
    _check(load_library().tattn_forward(p.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        _stream()))
    return out
