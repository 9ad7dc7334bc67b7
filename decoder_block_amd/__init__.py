"""MI355X-native LLaMA decoder layer: C-ABI library binding and synthetic workloads."""
