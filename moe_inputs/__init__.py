"""Seeded synthetic inputs for the MoE layer: shapes, value distributions and
routing patterns only. Nothing in this package computes any step of the layer;
both the CPU oracle and the GPU path consume what it produces."""

from .generators import WORKLOADS, Workload, make_inputs, workload  # noqa: F401
