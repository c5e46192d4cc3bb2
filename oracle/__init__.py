"""CPU oracle for group-wise (or per-channel) INT4 / INT8 weight quantization,
the W4A16 / W8A16 linear layer, the KV-cache codec, W8A8 with SmoothQuant,
and GPTQ / AWQ as producers of the packed weights.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library
never loads it and shares no code with it; the C source `q4_oracle.c` holds
the arithmetic, and this module only marshals numpy arrays into it.

Every function cites the passage it follows in `q4_oracle.c`.  Parity
status: the quantizer, dequantizer, fp16 converter, reference product, KV
codec, W8A8 path, GPTQ and AWQ are
pinned by the CPU tests (brute force, the worked example of the interview
guide's §3, closed forms and invariants); the packing order is this
library's own convention (the pages give none) and is pinned only by the
brute-force unpack — parity unpinned against the pages for that layout.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_p = ctypes.c_void_p


class Oracle:
    """ctypes view of one compiled copy of the oracle library."""

    def __init__(self, path):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.orc_f32_to_f16.restype = ctypes.c_uint16
        lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
        lib.orc_f16_to_f32.restype = ctypes.c_float
        lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_f32_to_f16_array.argtypes = [_p, _p, _c_i64]
        lib.orc_f32_bits_range_to_f16.argtypes = [ctypes.c_uint32, _c_i64, _p]
        lib.orc_f16_to_f32_array.argtypes = [_p, _p, _c_i64]
        lib.orc_quantize_group.argtypes = [_p, _c_i64, ctypes.c_int, ctypes.c_int,
                                           _p, _p, _p]
        lib.orc_quantize_pack.restype = ctypes.c_int
        lib.orc_quantize_pack.argtypes = [_p, _c_i64, _c_i64, _c_i32, _c_i32,
                                          _p, _p, _p, _p]
        lib.orc_dequant.argtypes = [_p, _p, _p, _c_i64, _c_i64, _c_i32, _p]
        lib.orc_quantize_pack_bits.restype = ctypes.c_int
        lib.orc_quantize_pack_bits.argtypes = [_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                               _p, _p, _p, _p]
        lib.orc_dequant_bits.argtypes = [_p, _p, _p, _c_i64, _c_i64, _c_i32, _c_i32, _p]
        lib.orc_linear_ref.argtypes = [_p, _p, _c_i64, _c_i64, _c_i64, _p, _p]
        lib.orc_kv_quant_tokens.restype = ctypes.c_int
        lib.orc_kv_quant_tokens.argtypes = [_p, _c_i64, _c_i32, _c_i32, _p, _p]
        lib.orc_kv_quant_channels.restype = ctypes.c_int
        lib.orc_kv_quant_channels.argtypes = [_p, _c_i64, _c_i32, _c_i32, _c_i32, _p, _p]
        lib.orc_kv_dequant_tokens.argtypes = [_p, _p, _c_i64, _c_i32, _p]
        lib.orc_kv_dequant_channels.argtypes = [_p, _p, _c_i64, _c_i32, _c_i32, _p]
        lib.orc_col_absmax_f16.argtypes = [_p, _c_i64, _c_i64, _p]
        lib.orc_col_absmax_f32.argtypes = [_p, _c_i64, _c_i64, _p]
        lib.orc_smooth_factors.argtypes = [_p, _p, _c_i64, ctypes.c_float, _p]
        lib.orc_w8a8_quant_weight.restype = ctypes.c_int
        lib.orc_w8a8_quant_weight.argtypes = [_p, _p, _c_i64, _c_i64, _p, _p]
        lib.orc_w8a8_quant_act.restype = ctypes.c_int
        lib.orc_w8a8_quant_act.argtypes = [_p, _p, _c_i64, _c_i64, _p, _p]
        lib.orc_w8a8_gemm.argtypes = [_p, _p, _p, _p, _c_i64, _c_i64, _c_i64, _p, _p]
        lib.orc_gptq_hessian.argtypes = [_p, _c_i64, _c_i64, _p]
        lib.orc_gptq_damp.argtypes = [_p, _c_i64, ctypes.c_double]
        lib.orc_gptq_hinv_chol.restype = ctypes.c_int
        lib.orc_gptq_hinv_chol.argtypes = [_p, _c_i64, _p]
        lib.orc_gptq_quantize.restype = ctypes.c_int
        lib.orc_gptq_quantize.argtypes = [_p, _p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _p, _p, _p]
        lib.orc_awq_act_mean.argtypes = [_p, _c_i64, _c_i64, _p]
        lib.orc_awq_scales.argtypes = [_p, _c_i64, ctypes.c_double, _p]
        lib.orc_awq_apply.restype = ctypes.c_int
        lib.orc_awq_apply.argtypes = [_p, _p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _p, _p, _p, _p]
        lib.orc_awq_loss.restype = ctypes.c_double
        lib.orc_awq_loss.argtypes = [_p, _c_i64, _p, _p, _c_i64, _c_i64]
        lib.orc_kv_cache_bytes.restype = ctypes.c_double
        lib.orc_kv_cache_bytes.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i32]
        lib.orc_set_num_threads.argtypes = [ctypes.c_int]
        lib.orc_max_threads.restype = ctypes.c_int
        self.lib = lib

    def set_threads(self, n):
        """Threads of the oracle's parallel loops (results do not depend on it)."""
        self.lib.orc_set_num_threads(int(n))

    def max_threads(self):
        return int(self.lib.orc_max_threads())

    # -- binary32 <-> binary16 ------------------------------------------------
    def f32_to_f16(self, a):
        a = np.ascontiguousarray(a, dtype=np.float32)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.orc_f32_to_f16_array(a.ctypes.data, out.ctypes.data, a.size)
        return out

    def f32_bits_range_to_f16(self, first, count):
        out = np.empty(count, dtype=np.uint16)
        self.lib.orc_f32_bits_range_to_f16(first, count, out.ctypes.data)
        return out

    def f16_to_f32(self, h):
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.float32)
        self.lib.orc_f16_to_f32_array(h.ctypes.data, out.ctypes.data, h.size)
        return out

    # -- quantization ----------------------------------------------------------
    def quantize_group(self, v, bits=4, symmetric=False):
        """One group -> (fp32 scale, integer zero-point, int32 codes)."""
        v = np.ascontiguousarray(v, dtype=np.float32).ravel()
        s = np.zeros(1, dtype=np.float32)
        z = np.zeros(1, dtype=np.int32)
        q = np.empty(v.size, dtype=np.int32)
        self.lib.orc_quantize_group(v.ctypes.data, v.size, bits, int(bool(symmetric)),
                                    s.ctypes.data, z.ctypes.data, q.ctypes.data)
        return s[0], int(z[0]), q

    def quantize_pack(self, w, group_size=128, symmetric=False, bits=4):
        """W fp32 [n_out][n_in] -> (packed u32 [n_out][n_in*bits/32], scales fp16
        bits, zeros fp16 bits [n_out][n_in/g], fp32 scales before storage).
        bits is 4 or 8; group_size == n_in is per-channel."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        n_out, n_in = w.shape
        g = n_in // group_size
        packed = np.empty((n_out, n_in * bits // 32), dtype=np.uint32)
        scales = np.empty((n_out, g), dtype=np.uint16)
        zeros = np.empty((n_out, g), dtype=np.uint16)
        s32 = np.empty((n_out, g), dtype=np.float32)
        if bits == 4:
            rc = self.lib.orc_quantize_pack(w.ctypes.data, n_out, n_in, group_size,
                                            int(bool(symmetric)), packed.ctypes.data,
                                            scales.ctypes.data, zeros.ctypes.data,
                                            s32.ctypes.data)
        else:
            rc = self.lib.orc_quantize_pack_bits(w.ctypes.data, n_out, n_in, group_size, bits,
                                                 int(bool(symmetric)), packed.ctypes.data,
                                                 scales.ctypes.data, zeros.ctypes.data,
                                                 s32.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected shape {w.shape} with group_size {group_size}, bits {bits}")
        return packed, scales, zeros, s32

    def dequant(self, packed, scales, zeros, group_size, bits=4):
        """-> w' fp32 [n_out][n_in], w' = s * (q - z)."""
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
        zeros = np.ascontiguousarray(zeros, dtype=np.uint16)
        n_out, words = packed.shape
        n_in = words * (32 // bits)
        out = np.empty((n_out, n_in), dtype=np.float32)
        if bits == 4:
            self.lib.orc_dequant(packed.ctypes.data, scales.ctypes.data, zeros.ctypes.data,
                                 n_out, n_in, group_size, out.ctypes.data)
        else:
            self.lib.orc_dequant_bits(packed.ctypes.data, scales.ctypes.data, zeros.ctypes.data,
                                      n_out, n_in, group_size, bits, out.ctypes.data)
        return out

    def linear_ref(self, x_f16_bits, w_deq):
        """x fp16 bits [m][n_in], w' fp32 [n_out][n_in] -> (y, a) float64 [m][n_out]
        with y = x w'^T and a = |x| |w'|^T, accumulated in binary64."""
        x = np.ascontiguousarray(x_f16_bits, dtype=np.uint16)
        w = np.ascontiguousarray(w_deq, dtype=np.float32)
        m, n_in = x.shape
        n_out = w.shape[0]
        assert w.shape[1] == n_in
        y = np.empty((m, n_out), dtype=np.float64)
        a = np.empty((m, n_out), dtype=np.float64)
        self.lib.orc_linear_ref(x.ctypes.data, w.ctypes.data, m, n_out, n_in,
                                y.ctypes.data, a.ctypes.data)
        return y, a

    def linear_from_packed(self, x_f16_bits, packed, scales, zeros, group_size, bits=4):
        """Dequantize, then take the reference product (two plain steps)."""
        return self.linear_ref(x_f16_bits, self.dequant(packed, scales, zeros, group_size, bits))


    # -- KV-cache codec (q4_oracle.c, "KV-cache codec") -------------------------
    def kv_quant_tokens(self, x_f16_bits, bits=8):
        """fp16 bits [..., d] -> (int8 codes [..., d], fp32 scale [...]): one
        symmetric scale per token row (the V side)."""
        x = np.ascontiguousarray(x_f16_bits, dtype=np.uint16)
        d = x.shape[-1]
        rows = x.size // d
        q = np.empty(x.shape, dtype=np.int8)
        s = np.empty(x.shape[:-1], dtype=np.float32)
        rc = self.lib.orc_kv_quant_tokens(x.ctypes.data, rows, d, bits, q.ctypes.data, s.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected kv_quant_tokens d={d} bits={bits}")
        return q, s

    def kv_quant_channels(self, x_f16_bits, bits=8):
        """fp16 bits [blocks, t, d] -> (int8 codes [blocks, t, d], fp32 scale
        [blocks, d]): one symmetric scale per channel of a block (the K side)."""
        x = np.ascontiguousarray(x_f16_bits, dtype=np.uint16)
        blocks, t, d = x.shape
        q = np.empty(x.shape, dtype=np.int8)
        s = np.empty((blocks, d), dtype=np.float32)
        rc = self.lib.orc_kv_quant_channels(x.ctypes.data, blocks, t, d, bits, q.ctypes.data,
                                            s.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected kv_quant_channels t={t} d={d} bits={bits}")
        return q, s

    def kv_dequant_tokens(self, q, s):
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s, dtype=np.float32)
        d = q.shape[-1]
        out = np.empty(q.shape, dtype=np.uint16)
        self.lib.orc_kv_dequant_tokens(q.ctypes.data, s.ctypes.data, q.size // d, d, out.ctypes.data)
        return out

    def kv_dequant_channels(self, q, s):
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s, dtype=np.float32)
        blocks, t, d = q.shape
        out = np.empty(q.shape, dtype=np.uint16)
        self.lib.orc_kv_dequant_channels(q.ctypes.data, s.ctypes.data, blocks, t, d, out.ctypes.data)
        return out

    def kv_flush(self, k_blocks, v_blocks, dst, pool_blocks, bits=8):
        """Quantize blocks of the FP16 window into a block pool: block p goes to
        pool slot dst[p] (K per channel, V per token); entries of dst outside
        [0, pool_blocks) are skipped.  Returns the pool arrays, untouched slots
        zero."""
        kq, ks = self.kv_quant_channels(k_blocks, bits)
        vq, vs = self.kv_quant_tokens(v_blocks, bits)
        _, t, d = kq.shape
        pool = dict(k=np.zeros((pool_blocks, t, d), np.int8), k_scale=np.zeros((pool_blocks, d), np.float32),
                    v=np.zeros((pool_blocks, t, d), np.int8), v_scale=np.zeros((pool_blocks, t), np.float32))
        for p, slot in enumerate(np.asarray(dst).tolist()):
            if 0 <= slot < pool_blocks:
                pool["k"][slot], pool["k_scale"][slot] = kq[p], ks[p]
                pool["v"][slot], pool["v_scale"][slot] = vq[p], vs[p]
        return pool

    def kv_cache_bytes(self, layers, kv_heads, head_dim, seq, batch, bits):
        return self.lib.orc_kv_cache_bytes(layers, kv_heads, head_dim, seq, batch, bits)

    # -- GPTQ and AWQ (q4_oracle.c, "GPTQ", "AWQ") ------------------------------
    def gptq_hessian(self, x_f16_bits):
        """H = 2 X^T X in binary64 from fp16 calibration tokens X [t][n]."""
        x = np.ascontiguousarray(x_f16_bits, dtype=np.uint16)
        t, n = x.shape
        h = np.empty((n, n), dtype=np.float64)
        self.lib.orc_gptq_hessian(x.ctypes.data, t, n, h.ctypes.data)
        return h

    def gptq_damp(self, h, lam=0.01):
        h = np.array(h, dtype=np.float64, order="C")
        self.lib.orc_gptq_damp(h.ctypes.data, h.shape[0], float(lam))
        return h

    def gptq_hinv_chol(self, h):
        """Upper U with U^T U = H^-1 (binary64)."""
        h = np.ascontiguousarray(h, dtype=np.float64)
        u = np.empty_like(h)
        rc = self.lib.orc_gptq_hinv_chol(h.ctypes.data, h.shape[0], u.ctypes.data)
        if rc != 0:
            raise ValueError("oracle gptq_hinv_chol: H not positive definite" if rc == 1 else "out of memory")
        return u

    def gptq_quantize(self, w, u_f32, group_size=128, bits=4, symmetric=False):
        """The column loop: -> (packed, scales, zeros, compensated fp32 W)."""
        w = np.array(w, dtype=np.float32, order="C")
        u = np.ascontiguousarray(u_f32, dtype=np.float32)
        n_out, n = w.shape
        g = n // group_size
        packed = np.empty((n_out, n * bits // 32), dtype=np.uint32)
        scales = np.empty((n_out, g), dtype=np.uint16)
        zeros = np.empty((n_out, g), dtype=np.uint16)
        rc = self.lib.orc_gptq_quantize(w.ctypes.data, u.ctypes.data, n_out, n, group_size, bits,
                                        int(bool(symmetric)), packed.ctypes.data, scales.ctypes.data,
                                        zeros.ctypes.data)
        if rc != 0:
            raise ValueError("oracle gptq_quantize rejected the shape")
        return packed, scales, zeros, w

    def gptq(self, w, x_f16_bits, group_size=128, bits=4, symmetric=False, lam=0.01):
        """The whole method: Hessian, damping, U, column loop."""
        h = self.gptq_damp(self.gptq_hessian(x_f16_bits), lam)
        u = self.gptq_hinv_chol(h).astype(np.float32)
        return self.gptq_quantize(w, u, group_size, bits, symmetric)[:3]

    def awq_act_mean(self, x_f16_bits):
        x = np.ascontiguousarray(x_f16_bits, dtype=np.uint16)
        mean = np.empty(x.shape[1], dtype=np.float64)
        self.lib.orc_awq_act_mean(x.ctypes.data, x.shape[0], x.shape[1], mean.ctypes.data)
        return mean

    def awq_scales(self, mean, alpha):
        mean = np.ascontiguousarray(mean, dtype=np.float64)
        s = np.empty(mean.size, dtype=np.float32)
        self.lib.orc_awq_scales(mean.ctypes.data, mean.size, float(alpha), s.ctypes.data)
        return s

    def awq_apply(self, w, s, group_size=128, bits=4, symmetric=False):
        """-> (packed, scales, zeros, effective weights dequant(Q(W diag s)) / s)."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        s = np.ascontiguousarray(s, dtype=np.float32)
        n_out, n = w.shape
        g = n // group_size
        packed = np.empty((n_out, n * bits // 32), dtype=np.uint32)
        scales = np.empty((n_out, g), dtype=np.uint16)
        zeros = np.empty((n_out, g), dtype=np.uint16)
        w_eff = np.empty_like(w)
        rc = self.lib.orc_awq_apply(w.ctypes.data, s.ctypes.data, n_out, n, group_size, bits,
                                    int(bool(symmetric)), packed.ctypes.data, scales.ctypes.data,
                                    zeros.ctypes.data, w_eff.ctypes.data)
        if rc != 0:
            raise ValueError("oracle awq_apply failed")
        return packed, scales, zeros, w_eff

    def awq_loss(self, x_f16_bits, w, w_eff):
        x = np.ascontiguousarray(x_f16_bits, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        w_eff = np.ascontiguousarray(w_eff, dtype=np.float32)
        return self.lib.orc_awq_loss(x.ctypes.data, x.shape[0], w.ctypes.data, w_eff.ctypes.data,
                                     w.shape[0], w.shape[1])

    def awq(self, w, x_f16_bits, group_size=128, bits=4, symmetric=False, n_grid=20):
        """The search: -> (best alpha index, losses, s, packed, scales, zeros)."""
        mean = self.awq_act_mean(x_f16_bits)
        losses, best = [], None
        for i in range(n_grid + 1):
            s = self.awq_scales(mean, i / n_grid)
            packed, scales, zeros, w_eff = self.awq_apply(w, s, group_size, bits, symmetric)
            loss = self.awq_loss(x_f16_bits, w, w_eff)
            losses.append(loss)
            if best is None or loss < best[1]:
                best = (i, loss, s, packed, scales, zeros)
        return best[0], losses, best[2], best[3], best[4], best[5]

    # -- W8A8 with SmoothQuant (q4_oracle.c, "W8A8 with SmoothQuant") ---------
    def col_absmax_f16(self, x_f16_bits):
        x = np.ascontiguousarray(x_f16_bits, dtype=np.uint16)
        out = np.empty(x.shape[1], dtype=np.float32)
        self.lib.orc_col_absmax_f16(x.ctypes.data, x.shape[0], x.shape[1], out.ctypes.data)
        return out

    def col_absmax_f32(self, w):
        w = np.ascontiguousarray(w, dtype=np.float32)
        out = np.empty(w.shape[1], dtype=np.float32)
        self.lib.orc_col_absmax_f32(w.ctypes.data, w.shape[0], w.shape[1], out.ctypes.data)
        return out

    def smooth_factors(self, act_max, w_max, alpha=0.5):
        """Per input channel s_j = max|X_j|^alpha / max|W_j|^(1-alpha), clamps at 1e-5."""
        a = np.ascontiguousarray(act_max, dtype=np.float32)
        w = np.ascontiguousarray(w_max, dtype=np.float32)
        s = np.empty(a.size, dtype=np.float32)
        self.lib.orc_smooth_factors(a.ctypes.data, w.ctypes.data, a.size, np.float32(alpha), s.ctypes.data)
        return s

    def w8a8_quant_weight(self, w, s=None):
        """W fp32 [n_out][n_in] (times diag(s) if given) -> (int8 [n_out][n_in], fp32 sw [n_out])."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        n_out, n_in = w.shape
        q = np.empty((n_out, n_in), dtype=np.int8)
        sw = np.empty(n_out, dtype=np.float32)
        sp = None if s is None else np.ascontiguousarray(s, dtype=np.float32)
        rc = self.lib.orc_w8a8_quant_weight(w.ctypes.data, None if sp is None else sp.ctypes.data,
                                            n_out, n_in, q.ctypes.data, sw.ctypes.data)
        if rc != 0:
            raise ValueError("oracle w8a8_quant_weight failed")
        return q, sw

    def w8a8_quant_act(self, x_f16_bits, s=None):
        """x fp16 bits [m][k] (divided by s if given) -> (int8 [m][k], fp32 sx [m])."""
        x = np.ascontiguousarray(x_f16_bits, dtype=np.uint16)
        m, k = x.shape
        q = np.empty((m, k), dtype=np.int8)
        sx = np.empty(m, dtype=np.float32)
        sp = None if s is None else np.ascontiguousarray(s, dtype=np.float32)
        rc = self.lib.orc_w8a8_quant_act(x.ctypes.data, None if sp is None else sp.ctypes.data, m, k,
                                         q.ctypes.data, sx.ctypes.data)
        if rc != 0:
            raise ValueError("oracle w8a8_quant_act failed")
        return q, sx

    def w8a8_gemm(self, qx, sx, qw, sw):
        """-> (y fp16 bits [m][n], int64 accumulators [m][n])."""
        qx = np.ascontiguousarray(qx, dtype=np.int8)
        qw = np.ascontiguousarray(qw, dtype=np.int8)
        sx = np.ascontiguousarray(sx, dtype=np.float32)
        sw = np.ascontiguousarray(sw, dtype=np.float32)
        m, k = qx.shape
        n = qw.shape[0]
        assert qw.shape[1] == k
        acc = np.empty((m, n), dtype=np.int64)
        y = np.empty((m, n), dtype=np.uint16)
        self.lib.orc_w8a8_gemm(qx.ctypes.data, sx.ctypes.data, qw.ctypes.data, sw.ctypes.data, m, n, k,
                               acc.ctypes.data, y.ctypes.data)
        return y, acc


_DEFAULT = None


def load():
    """The oracle built from oracle/q4_oracle.c (built with gcc if absent), or
    the build named by the ORACLE_LIB environment variable (the sanitizer
    check loads an ASan/UBSan build that way)."""
    global _DEFAULT
    if _DEFAULT is None:
        path = os.environ.get("ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        _DEFAULT = Oracle(path)
    return _DEFAULT
