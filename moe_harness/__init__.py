"""Harness around the fused MoE forward pass: workload shapes, seeded synthetic inputs and the
FLOP/byte model used for roofline reporting.  Holds none of the method's arithmetic."""
