"""placeholder; replaced below"""


def attn_tflops(B, H, Sq, Skv, D, seconds, causal):
    f = 4.0 * B * H * Sq * Skv * D
    return (f / 2 if causal else f) / seconds / 1e12


def pages_gbps(B, Hq, Hkv, Sq, Skv, D, elt, seconds):
    n = B * Hq * Sq * D * 2 + B * Hkv * Skv * D * 2
    return n * elt / seconds / 1e9
