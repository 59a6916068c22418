"""Seeded synthetic inputs for MoE dispatch/combine (shared by the CPU oracle tests and the GPU tests)."""
