"""Pure-Python brute-force references for tiny shapes, written straight from the format
definition and the pages' formulas.  They share nothing with the C oracle (no table, no
encoder), so the two pin each other on small inputs.  Python floats are binary64; fp32
steps use numpy.float32 scalars, whose arithmetic is IEEE binary32."""
import numpy as np


def e4m3_values():
    """All non-negative finite E4M3 values, in code order 0x00..0x7E."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return vals


_VALS = e4m3_values()


def encode(v: float) -> int:
    """Nearest E4M3 by scanning all 127 magnitudes; ties to the even code; clip at 448."""
    sign = 0x80 if np.signbit(v) else 0
    a = abs(float(v))
    if a >= 448.0:
        return sign | 0x7E
    best = 0
    for c in range(1, 0x7F):
        da, db = abs(_VALS[c] - a), abs(_VALS[best] - a)
        if da < db or (da == db and c % 2 == 0):
            best = c
    return sign | best


def decode(code: int) -> float:
    if code & 0x7F == 0x7F:
        return float("nan")
    v = _VALS[code & 0x7F]
    return -v if code & 0x80 else v


def bf16(bits: int) -> np.float32:
    return np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]


def group_quant(x_bits):
    m, k = x_bits.shape
    q = np.zeros((m, k), dtype=np.uint8)
    s = np.zeros((m, k // 128), dtype=np.float32)
    for r in range(m):
        for g in range(k // 128):
            xs = [bf16(int(b)) for b in x_bits[r, 128 * g:128 * g + 128]]
            amax = max(abs(float(x)) for x in xs)
            sc = np.float32(max(np.float32(amax), np.float32(1e-10))) / np.float32(448.0)
            s[r, g] = sc
            for j, x in enumerate(xs):
                q[r, 128 * g + j] = encode(float(np.float32(x) / sc))
    return q, s


def kv_write(kx, vx, kc, vc, slots, H, D, bs, k_scale, v_scale, ks, vs, cs):
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), bs)
        for h in range(H):
            for d in range(D):
                dst = blk * cs + (off * H + h) * D + d
                kc[dst] = encode(float(bf16(int(kx[t * ks + h * D + d])) / np.float32(k_scale)))
                vc[dst] = encode(float(bf16(int(vx[t * vs + h * D + d])) / np.float32(v_scale)))
