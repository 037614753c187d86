"""Test-only HIP probes (built by ``tests.probe.build``; not part of libmoe)."""
