"""RWKV-4 WKV time-mixing operator for AMD MI355X (gfx950), with the
receptance gate and the token-shift mix around it.

The compute path is the HIP library librwkv_wkv.so (C ABI in include/wkv.h);
``ops`` is a thin torch binding of it with the same names:

    from rwkv_wkv_mixing_amd import ops
    y = ops.wkv_forward(w, u, k, v)
    dk, dv, dw, du = ops.wkv_backward(w, u, k, v, gy)
    y = ops.wkv_step(w, u, k, v, a, b, p)
    xr_xk_xv = ops.token_shift(mu, x)          # the mixes feeding r, k, v

``workloads`` draws the seeded synthetic inputs used by tests and the bench.
"""

__version__ = "0.1.0"
