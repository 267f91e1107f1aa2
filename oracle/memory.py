"""Storage accounting for quantized weights (oracle side).

TEST INFRASTRUCTURE (see the package docstring).

[BAL] section 4: the raw weight storage follows exactly from the parameter
count and the bit width; scales, zero points, unquantized layers, workspace,
activations and the KV cache come on top. GB (10^9) and GiB (2^30) are kept
apart, as in that page's worked example.
"""


def raw_weight_bytes(n_params, bits):
    """Ideal packed size of ``n_params`` weights at ``bits`` bits each."""
    return n_params * bits / 8.0


def gb(nbytes):
    return nbytes / 1e9


def gib(nbytes):
    return nbytes / 2.0 ** 30


def bits_per_weight(bits, group, scale_bits=32, zero_bits=None):
    """Effective bits per weight of a grouped affine format: the code plus
    one scale and one zero point per group ([BAL] section 1: finer groups
    carry more metadata). The zero point defaults to ``bits`` wide."""
    zb = bits if zero_bits is None else zero_bits
    return bits + (scale_bits + zb) / group
