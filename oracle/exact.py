"""Exact rational evaluation of the WKV weighted sum, for tiny pinned cases.

TEST INFRASTRUCTURE ONLY (see oracle/wkv_ref.py).

Evaluates the definition of "RWKV（Receptance Weighted Key Value）概念",
section 3.2, term by term in exact ``fractions.Fraction`` arithmetic:

    wkv_t = (sum_{i<t} d^{t-1-i} E_i v_i + U E_t v_t) / (sum_{i<t} d^{t-1-i} E_i + U E_t)

where the caller passes the exponentials themselves as rationals:
E_i = e^{k_i}, U = e^{u}, d = e^{-w}.  Gradients of L = sum_t gy_t wkv_t are
exact forward-mode derivatives (dual numbers over Fraction), one directional
derivative per input, so they rest only on the definition and the chain rule
d/dk e^k = e^k, d/dw e^{-w} = -e^{-w}, d/du e^u = e^u.  Nothing here shares
code with the float64 recurrences it pins.
"""
from __future__ import annotations

from fractions import Fraction


class Dual:
    """a + b*eps with eps^2 = 0, over Fraction."""

    __slots__ = ("a", "b")

    def __init__(self, a, b=0):
        self.a = Fraction(a)
        self.b = Fraction(b)

    @staticmethod
    def lift(x):
        return x if isinstance(x, Dual) else Dual(x)

    def __add__(self, o):
        o = Dual.lift(o)
        return Dual(self.a + o.a, self.b + o.b)

    __radd__ = __add__

    def __mul__(self, o):
        o = Dual.lift(o)
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    __rmul__ = __mul__

    def __truediv__(self, o):
        o = Dual.lift(o)
        return Dual(self.a / o.a, (self.b * o.a - self.a * o.b) / (o.a * o.a))

    def __pow__(self, n: int):
        r = Dual(1)
        for _ in range(n):
            r = r * self
        return r


def wkv_exact(d, U, E, v):
    """wkv_1..wkv_T for one channel; every argument rational (or Dual)."""
    T = len(E)
    out = []
    for t in range(T):  # 0-based position of the current token
        num = Dual(0)
        den = Dual(0)
        for i in range(t):
            wgt = Dual.lift(d) ** (t - 1 - i) * E[i]
            num = num + wgt * v[i]
            den = den + wgt
        cur = Dual.lift(U) * E[t]
        out.append((num + cur * v[t]) / (den + cur))
    return out


def loss_grads_exact(d, U, E, v, gy):
    """Exact y and dL/dk_i, dL/dv_i, dL/dw, dL/du for L = sum gy_t y_t (one channel)."""
    T = len(E)
    E = [Fraction(x) for x in E]
    v = [Fraction(x) for x in v]
    gy = [Fraction(x) for x in gy]
    d = Fraction(d)
    U = Fraction(U)

    def L(dd, UU, EE, vv):
        ys = wkv_exact(dd, UU, EE, vv)
        tot = Dual(0)
        for t in range(T):
            tot = tot + ys[t] * gy[t]
        return tot, ys

    _, ys = L(d, U, E, v)
    y = [yy.a for yy in ys]
    dk = []
    dv = []
    for j in range(T):
        Ej = [Dual(E[i], E[i] if i == j else 0) for i in range(T)]
        dk.append(L(d, U, Ej, v)[0].b)
        vj = [Dual(v[i], 1 if i == j else 0) for i in range(T)]
        dv.append(L(d, U, E, vj)[0].b)
    dw = L(Dual(d, -d), U, E, v)[0].b
    du = L(d, Dual(U, U), E, v)[0].b
    return y, dk, dv, dw, du
