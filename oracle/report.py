"""Bus and sizing arithmetic printed on the pages.  (Oracle: test infrastructure only.)

* ``napkin``: explainer page, section "The bus problem: 1.3 GB of experts
  per token over PCIe" -- expert size from 3 * hidden * inter parameters at
  18 bytes per 32 weights, the all-experts total, the bytes touched per
  token, the PCIe time per token if every pick crossed the bus, and the
  miss traffic per token at a given hit rate.
* ``preflight``: SGLang page, section "A preflight script before you turn
  it on" -- GPU memory per slot over all layers, the single-wave batch cap
  K // top_k, the miss rate of uniform routing 1 - K/E, the highest miss
  rate a measured speed allows on a given link, and the verdict rule
  (reuse implied when that bound is below 0.8 times the uniform miss rate).

MiB = 2^20 bytes, GiB = 2^30; link speeds are in 10^9 bytes per second.
"""

MIB = 1 << 20
GIB = 1 << 30


def napkin(layers, experts, routed_per_token, hidden, inter, bytes_per_weight=18 / 32):
    params = 3 * hidden * inter
    expert_bytes = params * bytes_per_weight
    n_all = layers * experts
    touched = layers * routed_per_token
    return dict(params_per_expert=params, expert_bytes=expert_bytes, expert_mib=expert_bytes / MIB,
                n_experts_total=n_all, all_experts_gib=n_all * expert_bytes / GIB,
                touched_per_token=touched, touched_mib=touched * expert_bytes / MIB,
                touched_bytes=touched * expert_bytes)


def pcie_ms_per_token(bytes_per_token, link_gbs):
    ms = bytes_per_token / (link_gbs * 1e9) * 1e3
    return ms, 1e3 / ms


def cache_line(napkin_row, cache_gib, hit_rate, link_gbs):
    """Cache fraction of the experts, miss MiB per token and its PCIe ms."""
    frac = cache_gib / napkin_row["all_experts_gib"]
    miss_mib = (1.0 - hit_rate) * napkin_row["touched_mib"]
    ms = miss_mib * MIB / (link_gbs * 1e9) * 1e3
    return dict(fraction=frac, miss_mib=miss_mib, ms=ms)


def preflight(layers, experts, top_k, expert_mb, K, link_gbps, tok_s, kv_bytes_per_token):
    """Slot cost and the reuse test of the SGLang page's preflight, in this project's terms.

    With S the expert size in MB (10^6 bytes), L layers, E experts, k picks per token
    and K slots per layer: a slot costs L*S MB of GPU memory over all layers (the same
    bytes as that many tokens of KV cache); one wave holds at most floor(K/k) tokens;
    a token whose L*k picks all miss moves L*k*S MB over the link, so a measured speed of
    tok_s tokens/s on a link of link_gbps GB/s allows a miss fraction of at most
    link_gbps / (tok_s * L*k*S/1000); routing with no reuse misses 1 - K/E of its picks.
    Reuse is implied when the allowed miss fraction is below 0.8 of the no-reuse one.
    """
    mb_per_slot = layers * expert_mb
    gb_all_miss = layers * top_k * expert_mb / 1e3
    allowed = link_gbps / tok_s / gb_all_miss
    no_reuse = 1.0 - K / experts
    return dict(slot_mb=mb_per_slot, kv_tokens=mb_per_slot * 1e6 / kv_bytes_per_token, batch_cap=K // top_k,
                random_miss=no_reuse, max_miss=allowed, reuse_implied=bool(allowed < 0.8 * no_reuse))
