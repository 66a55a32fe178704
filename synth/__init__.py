"""Seeded synthetic inputs for the MoE finalize path.

This package only draws random inputs. It holds none of the finalize arithmetic, so the oracle
(`oracle/`) and the HIP path (`moe_expert_output_amd/`) can both consume it without sharing code.
"""
from .moe_inputs import MoeInputs, make_inputs, make_inputs_on_device, workload_seed  # noqa: F401
