"""The five workloads (shapes and flags), named by what they are.

c = entry width (head dim), m = compression ratio, nh = query heads,
hI x cI = indexer heads x dim, k = top-k, n_win = window, r = RoPE dims.
Overlap: the pages' CSA (m = 4) overlaps its blocks; the 2k-token fp32 case
states plain pooling over 4 tokens, and HCA never overlaps.
"""

COMMON = dict(qk_norm=1, eps=1e-6, theta=10000.0, n_win=128)

WORKLOADS = {
    "csa_prefill_2k_f32": dict(
        COMMON, kind="csa_prefill", dtype="f32", n=2048, d=1024, c=128, m=4, overlap=0,
        hI=4, cI=64, k=64, nh=8, rope_dims=0),
    "hca_prefill_16k_bf16": dict(
        COMMON, kind="hca_prefill", dtype="bf16", n=16384, d=4096, c=128, m=128, overlap=0,
        hI=0, cI=0, k=0, nh=64, rope_dims=0),
    "csa_prefill_64k_bf16": dict(
        COMMON, kind="csa_prefill", dtype="bf16", n=65536, d=4096, c=512, m=4, overlap=1,
        hI=16, cI=64, k=512, nh=64, rope_dims=64,
        # the layer around the calls: query latent width, output groups and
        # their width (the pages' V4-Flash values)
        d_c=1024, groups=8, d_g=1024),
    "decode_b32_128k_bf16": dict(
        COMMON, kind="decode", dtype="bf16", batch=32, ctx=131072, d=4096, c=512, m=4,
        overlap=1, m_hca=128, hI=16, cI=64, k=512, nh=64, rope_dims=0),
    "decode_b4_1m_bf16": dict(
        COMMON, kind="decode", dtype="bf16", batch=4, ctx=1048576, d=4096, c=512, m=4,
        overlap=1, m_hca=128, hI=16, cI=64, k=1024, nh=64, rope_dims=64),
}

for _name, _cfg in WORKLOADS.items():
    _cfg["name"] = _name


def get(name, **over):
    cfg = dict(WORKLOADS[name])
    cfg.update(over)
    return cfg
