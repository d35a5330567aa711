"""Host-side inputs for the oracle: the seeded draws (synth) encoded to Q2 bytes
by the oracle's own quantizer.  Nothing here comes from the HIP library."""
import functools

import numpy as np

from oracle import q2, q4
from synth import workloads as W
from synth.gen import bf16_bits_to_f32


class HostLayer:
    """Lazily generated host copy of one layer of a workload."""

    def __init__(self, wl, layer=0):
        self.wl = wl
        self.layer = layer
        self.router_w = W.router_weights(wl, layer)
        self.router_b = W.router_bias(wl, layer)
        bits = W.shared_bf16_bits(wl, layer)
        self.shared_bits = bits
        self.shared = None if bits is None else tuple(bf16_bits_to_f32(b) for b in bits)
        self._cache = {}

    def expert_bytes(self, e):
        """(gate, up, down) block bytes of routed expert e (each matrix in its layer's
        format), quantized on the host by the oracle's encoders."""
        if e not in self._cache:
            wl = self.wl
            gu4, dn4 = wl.q4_at(self.layer)
            codecs = (q4 if gu4 else q2, q4 if gu4 else q2, q4 if dn4 else q2)
            self._cache[e] = tuple(codecs[m].encode_matrix(W.expert_f32(wl, self.layer, e, m))
                                   for m in range(3))
        return self._cache[e]

    def packed_expert(self, e):
        """Expert e in the library's tiled layout."""
        return q2.pack_expert(*self.expert_bytes(e), self.wl.hidden, self.wl.inter)

    def all_expert_bytes(self):
        """All experts back to back in the library's tiled layout."""
        return np.concatenate([self.packed_expert(e) for e in range(self.wl.n_experts)])

    def oracle_layer(self):
        return dict(router_w=self.router_w, router_b=self.router_b,
                    expert_bytes=self.expert_bytes, shared=self.shared)


@functools.lru_cache(maxsize=8)
def host_layer(name, layer=0):
    return HostLayer(W.WORKLOADS[name], layer)
