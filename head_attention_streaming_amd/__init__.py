"""MI355X-native streaming multi-head attention (forward pass) behind a C-ABI library.

``binding`` wraps the C entry points of libstreamattn.so (declared in include/streamattn.h)
with the same names; ``synthetic`` draws the seeded inputs used by tests and the benchmark.
The shared library is loaded on first use and a missing build raises an error: there is no
fallback implementation.
"""
