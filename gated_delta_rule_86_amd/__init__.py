"""gated_delta_rule_86_amd -- Kimi Delta Attention (KDA) chunked forward pass for MI355X (gfx950).

``workloads`` draws the seeded synthetic inputs shared by the tests and the benchmark.
"""
