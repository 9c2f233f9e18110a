"""CPU oracle for the NVFP4 W4A4 MoE expert path (test infrastructure only)."""
