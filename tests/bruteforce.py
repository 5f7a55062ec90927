"""Scalar-loop brute force of the decoder, for pinning the oracle on tiny shapes.

Pure Python floats (IEEE double) and the ``math`` module, one element at a
time, written from the model definition (not from the oracle's tensor code):
no matrices, no broadcasting, no library softmax.  Used only by the tests.
"""
import math
import struct


def _f(t):
    """Stored tensor -> nested Python float lists."""
    return t.detach().to("cpu").double().tolist()


def dot(a, b):
    s = 0.0
    for i in range(len(a)):
        s += a[i] * b[i]
    return s


def mv(W, x):
    return [dot(row, x) for row in W]


def rms(x, g, eps):
    ss = 0.0
    for v in x:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(x) + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def rot(vec, pos, base):
    hd = len(vec)
    half = hd // 2
    out = list(vec)
    for i in range(half):
        ang = pos * base ** (-2.0 * i / hd)
        c, s = math.cos(ang), math.sin(ang)
        a, b = vec[i], vec[i + half]
        out[i] = a * c - b * s
        out[i + half] = a * s + b * c
    return out


def round_store(x, fmt):
    """x rounded to a 16-bit storage format ("bf16" or "f16") and back: first to
    the nearest float32, then to the nearest 16-bit value, ties to even (the
    route a float64 -> float32 -> 16-bit conversion takes)."""
    f = struct.unpack("<f", struct.pack("<f", x))[0]
    if fmt == "f16":
        return struct.unpack("<e", struct.pack("<e", f))[0]
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def model_logits(w, shape, tokens, store=None):
    """Logits at every position of ``tokens`` (a full causal pass), as lists.

    store: None keeps cached keys and values exact; "bf16" / "f16" rounds each
    cached element (keys after rotation) to that format, and nothing else."""
    s = shape
    E = _f(w["tok_emb"])
    layers = [{k: _f(v) for k, v in lw.items()} for lw in w["layers"]]
    gf = _f(w["final_norm"])
    Wlm = _f(w["lm_head"])
    hd, hq, hkv = s.head_dim, s.n_heads, s.n_kv_heads
    group = hq // hkv
    Kc = [[[] for _ in range(hkv)] for _ in range(s.n_layers)]
    Vc = [[[] for _ in range(hkv)] for _ in range(s.n_layers)]
    out = []
    for pos, t in enumerate(tokens):
        x = list(E[t])
        for l, lw in enumerate(layers):
            xn = rms(x, lw["attn_norm"], s.rms_eps)
            q = mv(lw["wq"], xn)
            k = mv(lw["wk"], xn)
            v = mv(lw["wv"], xn)
            for g in range(hkv):
                kr = rot(k[g * hd:(g + 1) * hd], pos, s.rope_base)
                vr = v[g * hd:(g + 1) * hd]
                if store is not None:
                    kr = [round_store(e, store) for e in kr]
                    vr = [round_store(e, store) for e in vr]
                Kc[l][g].append(kr)
                Vc[l][g].append(vr)
            att = []
            for h in range(hq):
                g = h // group
                qh = rot(q[h * hd:(h + 1) * hd], pos, s.rope_base)
                sc = [dot(qh, Kc[l][g][j]) / math.sqrt(hd) for j in range(pos + 1)]
                m = max(sc)
                e = [math.exp(v_ - m) for v_ in sc]
                z = sum(e)
                o = [0.0] * hd
                for j in range(pos + 1):
                    for i in range(hd):
                        o[i] += e[j] / z * Vc[l][g][j][i]
                att.extend(o)
            ao = mv(lw["wo"], att)
            x = [x[i] + ao[i] for i in range(len(x))]
            xn = rms(x, lw["ffn_norm"], s.rms_eps)
            gt = mv(lw["w_gate"], xn)
            up = mv(lw["w_up"], xn)
            hh = [gt[i] / (1.0 + math.exp(-gt[i])) * up[i] for i in range(len(gt))]
            dn = mv(lw["w_down"], hh)
            x = [x[i] + dn[i] for i in range(len(x))]
        xf = rms(x, gf, s.rms_eps)
        out.append(mv(Wlm, xf))
    return out
