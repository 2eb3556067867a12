"""Seeded generators: AR(1) hidden states, router weights, packed expert blocks.

Packed expert block (one contiguous block per (layer, expert), in the spirit
of the repacked contiguous per-expert blocks on the NVMe-streaming page,
"Workflow" list): three matrices in the order gate, up, down.  Gate and up
are [inter x hidden] (reduction over hidden), down is [hidden x inter]
(reduction over inter).  For a matrix of R rows and C reduction columns:

* fp32:  R*C float32, row-major.
* int4, group 32 along C, fp16 scale: a nibble plane of R*C/2 bytes
  (row-major; element 2j in the low nibble of byte j, element 2j+1 in the
  high nibble), then a scale plane of R*C/32 float16 (little-endian,
  row-major).  Weight = (q - 8) * s.
* e2m1 codes, group 16 along C, OCP E4M3 scale: a nibble plane as above
  (each nibble sign | 2-bit exponent | 1-bit mantissa), then a scale plane
  of R*C/16 bytes.  Weight = e4m3(s) * e2m1(q).

The quantisers here only prepare inputs: the method under test decodes the
bytes, it never encodes them.
"""
import numpy as np

QUANT_F32 = 0
QUANT_INT4_G32 = 1
QUANT_E2M1_G16 = 2
QUANT_NAMES = {QUANT_F32: "f32", QUANT_INT4_G32: "int4_g32_f16", QUANT_E2M1_G16: "e2m1_g16_e4m3"}

EXPERT_STD = 0.02
# An always-on shared expert enters every layer with weight 1, and these synthetic stacks
# chain x_{l+1} = x_l + y_l with no normalisation between layers; the expert FFN is
# quadratic in x, so at EXPERT_STD a shared expert adds about 0.34 * rms(x)^2 per layer
# (H = 3072, I = 512) and the stream overflows within 20 layers.  Half the std scales the
# shared expert's output by 1/8, which keeps the stream O(1) over 48 layers.
SHARED_EXPERT_STD = 0.01


def _matrix_bytes(quant, rows, cols):
    n = rows * cols
    if quant == QUANT_F32:
        return 4 * n
    if quant == QUANT_INT4_G32:
        return n // 2 + (n // 32) * 2
    if quant == QUANT_E2M1_G16:
        return n // 2 + n // 16
    raise ValueError(f"unknown quant {quant}")


def expert_bytes(quant, hidden, inter):
    """Bytes of one packed expert block (gate + up + down)."""
    return 2 * _matrix_bytes(quant, inter, hidden) + _matrix_bytes(quant, hidden, inter)


def block_layout(quant, hidden, inter):
    """[(name, rows, cols, byte_offset)] for gate, up, down."""
    out, off = [], 0
    for name, r, c in (("gate", inter, hidden), ("up", inter, hidden), ("down", hidden, inter)):
        out.append((name, r, c, off))
        off += _matrix_bytes(quant, r, c)
    return out


def _rng(seed, *key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key))))


# ----------------------------------------------------------------------------- hidden states / router

def ar1_streams(seed, n_streams, n_steps, hidden, rho=0.9, sigma=0.436):
    """AR(1) hidden-state streams, float32 [n_steps, n_streams, hidden].

    Stream s uses its own generator (spawn key (1, s)), so stream s is the
    same whatever n_streams is.
    """
    out = np.empty((n_steps, n_streams, hidden), dtype=np.float32)
    for s in range(n_streams):
        g = _rng(seed, 1, s)
        x = g.standard_normal(hidden)
        out[0, s] = x
        for t in range(1, n_steps):
            x = rho * x + sigma * g.standard_normal(hidden)
            out[t, s] = x
    return out


def prefill_prompt(seed, n_tokens, hidden):
    """One AR(1) stream of n_tokens positions, float32 [n_tokens, hidden]."""
    return ar1_streams(seed, 1, n_tokens, hidden)[:, 0, :].copy()


def router_weights(seed, n_layers, n_experts, hidden):
    """Router weights ~N(0, 1/sqrt(hidden)), float32 [n_layers, n_experts, hidden]."""
    out = np.empty((n_layers, n_experts, hidden), dtype=np.float32)
    std = 1.0 / np.sqrt(hidden)
    for layer in range(n_layers):
        out[layer] = (_rng(seed, 2, layer).standard_normal((n_experts, hidden), dtype=np.float32) * np.float32(std))
    return out


# ----------------------------------------------------------------------------- quantisers (input preparation)

def _pack_nibbles(q):
    """q uint8 [..., C] with values 0..15 -> bytes [..., C/2] (low nibble = even element)."""
    q = q.astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def quantize_int4_g32(w):
    """w float32 [R, C] -> (nibble plane [R, C/2] uint8, scale plane [R, C/32] float16)."""
    r, c = w.shape
    g = w.reshape(r, c // 32, 32)
    amax = np.abs(g).max(axis=2)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1)), 0.0)
    q = (np.clip(q, -8, 7) + 8).astype(np.uint8).reshape(r, c)
    return _pack_nibbles(q), s16


def _e4m3_positive_table():
    """Finite non-negative OCP E4M3 values indexed by code 0..126 (the generator's own table)."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nearest_code(table, v):
    """Nearest entry of an increasing table, saturating (an exact midpoint goes to the lower entry)."""
    mids = ((table[1:] + table[:-1]) * 0.5).astype(v.dtype)
    return np.searchsorted(mids, np.minimum(v, table[-1]).astype(v.dtype), side="left")


def quantize_e2m1_g16(w):
    """w float32 [R, C] -> (nibble plane [R, C/2] uint8, scale plane [R, C/16] uint8 E4M3)."""
    r, c = w.shape
    g = w.reshape(r, c // 16, 16)
    amax = np.abs(g).max(axis=2).astype(np.float64)
    scode = _nearest_code(_E4M3_POS, amax / 6.0).astype(np.uint8)
    s = _E4M3_POS[scode].astype(np.float32)[..., None]
    inv = np.where(s > 0, np.float32(1.0) / np.where(s > 0, s, np.float32(1.0)), np.float32(0.0))
    ratio = np.abs(g) * inv
    mag = _nearest_code(_E2M1_POS.astype(np.float32), ratio).astype(np.uint8)
    sign = ((g < 0) & (mag > 0)).astype(np.uint8) << 3
    q = (mag | sign).reshape(r, c)
    return _pack_nibbles(q), scode


def _encode_matrix(quant, w):
    if quant == QUANT_F32:
        return w.astype(np.float32).tobytes()
    if quant == QUANT_INT4_G32:
        nib, sc = quantize_int4_g32(w)
        return nib.tobytes() + sc.astype("<f2").tobytes()
    nib, sc = quantize_e2m1_g16(w)
    return nib.tobytes() + sc.tobytes()


def expert_block(seed, layer, expert, quant, hidden, inter, std=EXPERT_STD):
    """Packed bytes (uint8 [expert_bytes]) of expert `expert` of layer `layer`.

    layer = -1 is used for a model's always-on shared expert.
    """
    g = _rng(seed, 3, layer + 1, expert)
    parts = []
    for _name, r, c, _off in block_layout(quant, hidden, inter):
        w = g.standard_normal((r, c), dtype=np.float32) * np.float32(std)
        parts.append(_encode_matrix(quant, w))
    out = np.frombuffer(b"".join(parts), dtype=np.uint8)
    assert out.size == expert_bytes(quant, hidden, inter)
    return out


def shared_expert_blocks(seed, n_layers, quant, hidden, inter):
    """Packed blocks (uint8 [n_layers, expert_bytes]) of each layer's shared expert."""
    return np.stack([expert_block(seed, -1, l, quant, hidden, inter, std=SHARED_EXPERT_STD)
                     for l in range(n_layers)])


def _block_worker(args):
    seed, layer, expert, quant, hidden, inter = args
    return expert_block(seed, layer, expert, quant, hidden, inter)


def fill_expert_store(store, seed, quant, hidden, inter, n_layers, n_experts, n_distinct=None, workers=None):
    """Fill `store` (uint8 [n_layers, n_experts, S]) with packed blocks.

    With n_distinct = M, only M distinct blocks are drawn and block
    (layer, expert) holds distinct block (layer*n_experts + expert) % M,
    whose bytes are those of expert_block(seed, 0, m).  Returns the map
    [n_layers, n_experts] -> (layer, expert) source key actually drawn.
    """
    s = expert_bytes(quant, hidden, inter)
    assert store.shape == (n_layers, n_experts, s) and store.dtype == np.uint8
    src = np.empty((n_layers, n_experts, 2), dtype=np.int64)
    if n_distinct is None:
        keys = [(l, e) for l in range(n_layers) for e in range(n_experts)]
    else:
        keys = [(0, m) for m in range(n_distinct)]
    jobs = [(seed, l, e, quant, hidden, inter) for (l, e) in keys]
    if workers is None:
        import os
        workers = min(16, len(os.sched_getaffinity(0)))
    if workers > 1 and len(jobs) > 4:
        # NumPy releases the GIL while filling and transforming large arrays
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            _place(store, ex.map(_block_worker, jobs), keys, n_layers, n_experts, n_distinct, src)
    else:
        _place(store, map(_block_worker, jobs), keys, n_layers, n_experts, n_distinct, src)
    return src


def _place(store, blocks, keys, n_layers, n_experts, n_distinct, src):
    if n_distinct is None:
        for (l, e), b in zip(keys, blocks):
            store[l, e] = b
            src[l, e] = (l, e)
        return None
    blist = list(blocks)
    for l in range(n_layers):
        for e in range(n_experts):
            m = (l * n_experts + e) % n_distinct
            store[l, e] = blist[m]
            src[l, e] = (0, m)
    return None


def fill_blocks(out, seed, quant, hidden, inter, keys, workers=None):
    """out uint8 [len(keys), S]: out[i] = expert_block(seed, *keys[i]) (threads)."""
    jobs = [(seed, l, e, quant, hidden, inter) for (l, e) in keys]
    if workers is None:
        import os
        workers = min(16, len(os.sched_getaffinity(0)))
    if workers > 1 and len(jobs) > 4:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            for i, b in enumerate(ex.map(_block_worker, jobs)):
                out[i] = b
    else:
        for i, j in enumerate(jobs):
            out[i] = _block_worker(j)
    return out


def alias_index(layer, expert, n_experts, n_distinct):
    """Distinct block that (layer, expert) uses when only n_distinct blocks are drawn."""
    return (layer * n_experts + expert) % n_distinct
