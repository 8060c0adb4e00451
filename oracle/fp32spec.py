"""The float32 sigmoid used as a routing selection key -- oracle side.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Why it exists.  DeepSeek-V3-style routing ranks experts by a sigmoid affinity
plus a per-expert selection bias ("Mixture of experts" lecture field map,
section "DeepSeek v1 -> V2 -> V3"; "Lab 18 -- Mixture of experts", section 2,
auxiliary-loss-free balancing).  The top-k of ``sigmoid(z) + b`` is not a
function of ``z`` alone, so for the routing to be reproducible bit for bit the
float32 sigmoid itself must be one fixed sequence of IEEE float32 operations.
This module is that sequence, written with numpy float32 arithmetic (every
operation rounds to nearest-even, no fused multiply-add):

    exp_spec(a):  Cody & Waite argument reduction followed by the degree-7
                  Taylor polynomial of exp on |r| <= ln2/2, evaluated by Horner:
        a > 88           -> +inf
        a < -87          -> 0
        n  = rint(a * INV_LN2)                 (round half to even)
        r  = (a - n*LN2_HI) - n*LN2_LO
        p  = (((((((c7 r + c6) r + c5) r + c4) r + c3) r + c2) r + c1) r + c0)
        exp_spec = p * 2^n                       (exact scaling)
    sigmoid_spec(z) = 1 / (1 + exp_spec(-z))     (IEEE division)

Constants: INV_LN2 = float32(1/ln 2); LN2_HI = ln 2 cut to its leading 16
significant bits (so ``n*LN2_HI`` is exact for |n| <= 256); LN2_LO =
float32(ln 2 - LN2_HI); c_i = float32(1/i!).  The accuracy of the whole
sequence is pinned against libm in the tests (within 2 ulp on [-87, 88]).
"""
import math

import numpy as np

F32 = np.float32
INV_LN2 = F32(1.0 / math.log(2.0))
LN2_HI = F32(0.693145751953125)          # 0x3F317200
LN2_LO = F32(math.log(2.0) - 0.693145751953125)
TAYLOR = [F32(1.0 / math.factorial(i)) for i in range(8)]
EXP_HI = F32(88.0)
EXP_LO = F32(-87.0)


def exp_spec(a):
    a = np.asarray(a, dtype=np.float32)
    over = a > EXP_HI
    under = a < EXP_LO
    ac = np.where(over | under, F32(0.0), a).astype(np.float32)
    n = np.rint(ac * INV_LN2).astype(np.float32)
    r = (ac - n * LN2_HI) - n * LN2_LO
    p = TAYLOR[7]
    for c in TAYLOR[6::-1]:
        p = p * r + c
    p = np.asarray(p, dtype=np.float32)
    out = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    out = np.where(over, F32(np.inf), out)
    out = np.where(under, F32(0.0), out)
    return out.astype(np.float32)


def sigmoid_spec(z):
    z = np.asarray(z, dtype=np.float32)
    with np.errstate(over='ignore'):
        e = exp_spec(-z)
        return (F32(1.0) / (F32(1.0) + e)).astype(np.float32)
